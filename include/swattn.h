/*
 * swattn.h — C ABI of libswattn.so: attention over packed variable-length (THD)
 * token streams on MI355X (gfx950).
 *
 * Operations:
 *
 *  varlen_attn_fwd  Causal or causal sliding-window GQA attention over documents
 *                   packed back to back and delimited by cu_seqlens, with a score
 *                   scale and an optional learned per-query-head sink logit.
 *                   Defined by MuseMagiPlan.attention (query/key/value/window/scale;
 *                   nemo_automodel.components.models.muse_spark.magi_cp page),
 *                   FlintMagiPlan.attention (sink; window counts the current token;
 *                   nemo_automodel.components.models.flint.magi page), the GQA head
 *                   grouping of MuseGlimmerAttention / repeat_kv
 *                   (nemo_automodel.components.models.muse_glimmer.model page) and
 *                   the causal document mask of SequenceLayout.allowed
 *                   (nemo_automodel.components.models.mistral_large4.attention page).
 *
 *  varlen_attn_bwd  Its backward: dq, dk, dv (and dsink) of a loss through out, from
 *                   the forward's output and log-sum-exp. The pages return only the
 *                   attention output and print no backward; they call sparse_mla's
 *                   value weight differentiable (mistral_large4.attention page). The
 *                   LSE export of varlen_attn_fwd and its use here to recompute the
 *                   probabilities are this library's own design choice.
 *
 *  sparse_mla_fwd   Sparse MLA forward: each query token attends to the top-k key
 *                   rows its index row names; a key is a shared 512-wide latent row
 *                   plus a 64-wide rotary row and the value is the latent row.
 *                   Defined by sparse_mla and MistralLarge4Attention._sparse_forward
 *                   (nemo_automodel.components.models.mistral_large4.attention page).
 *
 *  mla_value_proj   The per-head value up-projection (value_weight) that sparse_mla
 *                   applies to sparse_mla_fwd's latent-space output.
 *
 * Conventions common to every entry point
 *  - Tensors are described by swa_tensor: a device pointer plus shape and strides in
 *    elements. The innermost dimension must be contiguous (stride 1); the other
 *    strides are free but must keep every row 16-byte aligned (base pointer and
 *    row strides multiples of 16 bytes) — except sparse_mla_fwd's int32 indices,
 *    whose rows need only 4-byte alignment.
 *  - The caller allocates and owns every buffer. The library allocates no device
 *    memory, keeps no per-call state and performs no host<->device copy or
 *    synchronisation: a call validates its arguments on the host, enqueues its
 *    kernels on `stream` (a hipStream_t; NULL = the legacy default stream) and
 *    returns. Buffers must stay valid until that stream work completes. A call
 *    enqueues kernel launches only (no memset, copy or event), so it may be captured
 *    into a HIP graph; a replay reads the buffers captured, with their contents at
 *    replay time.
 *  - Outputs must not alias inputs.
 *  - Return value: SWA_OK (0) or a negative swa_status. On any error detected on the
 *    host nothing is enqueued and the outputs are untouched; swa_last_error() then
 *    names the offending argument. No C++ exception crosses this interface.
 *  - Contract violations that only the device can see (non-monotone cu_seqlens,
 *    out-of-range indices) never cause an out-of-bounds access: offsets are
 *    clamped to [0, T] and out-of-range indices act as empty slots. The values
 *    written for tokens of a malformed cu_seqlens are then unspecified.
 *  - Thread-safe and reentrant; calls on different streams may run concurrently.
 */
#ifndef SWATTN_H_
#define SWATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWA_ABI_VERSION 1

/* Element types of swa_tensor.dtype. */
enum swa_dtype {
  SWA_DTYPE_F32 = 0,  /* IEEE binary32 */
  SWA_DTYPE_BF16 = 1, /* bfloat16 */
  SWA_DTYPE_I32 = 2   /* int32 */
};

/* Status codes. */
enum swa_status {
  SWA_OK = 0,
  SWA_ERR_NULL = -1,        /* a required pointer is NULL */
  SWA_ERR_DTYPE = -2,       /* unsupported or mismatched element type */
  SWA_ERR_SHAPE = -3,       /* ranks or shapes disagree */
  SWA_ERR_ARG = -4,         /* a scalar argument is out of range */
  SWA_ERR_UNSUPPORTED = -5, /* well-formed but not implemented (e.g. head_dim) */
  SWA_ERR_LAYOUT = -6,      /* stride or alignment requirement violated */
  SWA_ERR_LAUNCH = -7       /* the HIP runtime rejected the launch */
};

/* Non-owning view of a device tensor of rank <= 3. */
typedef struct swa_tensor {
  void* data;        /* device pointer (may be NULL only when the tensor is empty) */
  int32_t dtype;     /* enum swa_dtype */
  int32_t ndim;      /* number of valid entries in shape[] and stride[] */
  int64_t shape[3];
  int64_t stride[3]; /* in elements; stride[ndim-1] must be 1 */
} swa_tensor;

/*
 * varlen_attn_fwd — packed varlen causal / sliding-window GQA attention forward.
 *
 * For every document d = [cu_seqlens[d], cu_seqlens[d+1]), every token i in it and
 * every query head h (KV head g = h / (Hq/Hkv)):
 *     allowed(i,j)  <=>  cu_seqlens[d] <= j <= i  and  (window == 0 or i - j < window)
 *     S_j = scale * <q[i,h,:], k[j,g,:]>
 *     Z   = sum_{allowed j} exp(S_j)  +  exp(sinks[h])        (sink term only if sinks)
 *     out[i,h,:] = sum_{allowed j} exp(S_j) * v[j,g,:] / Z ;  lse[i,h] = ln Z
 * The sink is a logit: it is not multiplied by scale and has no value vector.
 * Tokens outside every document (before cu_seqlens[0] or from cu_seqlens[n_docs]
 * to T) are padding: out = 0, lse = -inf.
 *
 *   q          [T, Hq, D]   bf16 or f32
 *   k, v       [T, Hkv, D]  same dtype as q; Hq must be a multiple of Hkv
 *   cu_seqlens device int32 [n_docs + 1], non-decreasing document offsets with
 *              cu_seqlens[n_docs] <= T (zero-length documents allowed); may be
 *              NULL when n_docs == 0 (every token is padding)
 *   n_docs     >= 0
 *   window     >= 0; 0 = full causal, else the key window length including the
 *              current token
 *   scale      finite and > 0
 *   sinks      device f32 [Hq] learned logits, or NULL for none (-inf = no sink)
 *   out        [T, Hq, D]  same dtype as q
 *   lse        device f32 [T, Hq] contiguous (natural log), or NULL
 *   stream     hipStream_t
 * Supported: D in {64, 128}, and 256 for bf16; token strides of k and v and the token and head
 * strides of out below 2^24 elements (SWA_ERR_UNSUPPORTED otherwise). Arithmetic: f32 accumulation; bf16 inputs use bf16
 * matrix products with the probabilities rounded to bf16 for the value product,
 * and the output is rounded once from f32.
 */
int32_t varlen_attn_fwd(const swa_tensor* q, const swa_tensor* k, const swa_tensor* v,
                        const int32_t* cu_seqlens, int32_t n_docs, int32_t window, float scale,
                        const float* sinks, swa_tensor* out, float* lse, void* stream);

/*
 * varlen_attn_bwd — backward of varlen_attn_fwd.
 *
 * With the forward's definitions (same q, k, v, cu_seqlens, n_docs, window, scale,
 * sinks), its output out and log-sum-exp lse, and dout = dL/dout, for every allowed
 * pair (i, j) of a document and query head h (KV head g):
 *     P_ij   = exp(scale <q[i,h,:], k[j,g,:]> - lse[i,h])
 *     delta  = <dout[i,h,:], out[i,h,:]>
 *     dS_ij  = P_ij (<dout[i,h,:], v[j,g,:]> - delta[i,h])
 *     dq[i,h,:] = scale sum_j dS_ij k[j,g,:]
 *     dk[j,g,:] = scale sum_{i, h of group g} dS_ij q[i,h,:]
 *     dv[j,g,:] = sum_{i, h of group g} P_ij dout[i,h,:]
 *     dsinks[h] = - sum_i exp(sinks[h] - lse[i,h]) delta[i,h]   (with sinks only)
 * These are the gradients of L through out (lse is treated as auxiliary). Padding
 * tokens get zero dq, dk and dv and add nothing to dsinks (their lse is -inf).
 *
 *   q, out, dout, dq   [T, Hq, D]   bf16
 *   k, v, dk, dv       [T, Hkv, D]  bf16
 *   lse                device f32 [T, Hq] contiguous, as written by varlen_attn_fwd
 *   cu_seqlens, n_docs, window, scale, sinks  as for varlen_attn_fwd
 *   dsinks             device f32 [Hq], required when sinks is given (written), else
 *                      ignored
 *   delta              device f32 [T, Hq] contiguous workspace the caller owns (the
 *                      library allocates nothing); its contents on return are unspecified
 *   stream             hipStream_t; the dq (which also computes delta), dk/dv and, with
 *                      sinks, two dsink reduction kernels are enqueued in that order
 * Supported: D in {64, 128}, T * Hq < 2^30, token strides of q, k, v and dout and the token and
 * head strides of dq below 2^24 elements. Errors: as varlen_attn_fwd; SWA_ERR_NULL when lse,
 * delta or (with sinks) dsinks is NULL; SWA_ERR_ARG when a gradient aliases an input or
 * another gradient. Arithmetic: bf16 matrix products (P and dS rounded to bf16 as
 * operands), f32 accumulation, one rounding of each gradient.
 */
int32_t varlen_attn_bwd(const swa_tensor* q, const swa_tensor* k, const swa_tensor* v, const swa_tensor* out,
                        const swa_tensor* dout, const float* lse, const int32_t* cu_seqlens, int32_t n_docs,
                        int32_t window, float scale, const float* sinks, swa_tensor* dq, swa_tensor* dk,
                        swa_tensor* dv, float* dsinks, float* delta, void* stream);

/*
 * varlen_attn_bwd_noalloc — varlen_attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, semantics, kernels and results as varlen_attn_bwd, without `delta`: the
 * per-row workspace lives in a library-owned device array of 2^22 floats (16 MiB) per device,
 * resolved once per device and held until the process ends; the call allocates nothing.
 * Limit: T * Hq <= 4,194,304 (SWA_ERR_UNSUPPORTED beyond, nothing enqueued). Every call on a
 * device shares that device's array, so calls that overlap on one device (different streams,
 * or concurrent host threads without ordering) race and must not be issued; calls ordered on
 * one stream are safe. The array is the current device's: `stream` must belong to it.
 */
int32_t varlen_attn_bwd_noalloc(const swa_tensor* q, const swa_tensor* k, const swa_tensor* v,
                                const swa_tensor* out, const swa_tensor* dout, const float* lse,
                                const int32_t* cu_seqlens, int32_t n_docs, int32_t window, float scale,
                                const float* sinks, swa_tensor* dq, swa_tensor* dk, swa_tensor* dv,
                                float* dsinks, void* stream);

/*
 * sparse_mla_fwd — sparse MLA forward over gathered top-k latent rows.
 *
 * For token t, head h and slot r of indices[t,:] (idx = indices[t,r]):
 *     valid(r)  <=>  0 <= idx < T  and  idx <= t  and  doc_ids[idx] == doc_ids[t] >= 0
 *     S_r = scale * (<q[t,h,:Dl], latent[idx,:]> + <q[t,h,Dl:], k_pe[idx,:]>)
 *     out[t,h,:] = sum_{valid r} softmax(S)_r * latent[idx,:] ;  lse[t,h] = ln sum exp(S_r)
 * -1 marks an empty slot; repeated indices count once per slot; a row with no
 * valid slot gives out = 0 and lse = -inf. The value is the latent row (the KV-B
 * value up-projection is not part of this call).
 *
 *   q        [T, H, Dl + Dr] bf16, latent coordinates first, rotary last
 *   latent   [T, Dl] bf16
 *   k_pe     [T, Dr] bf16
 *   indices  [T, topk] int32, topk >= 1
 *   doc_ids  device int32 [T] document id per token (< 0 = padding token)
 *   scale    finite and > 0
 *   out      [T, H, Dl] bf16
 *   lse      device f32 [T, H] contiguous, or NULL
 * Supported: Dl = 512, Dr = 64 or Dr = 0 (the NoPE variant: q is [T, H, 512] and k_pe has
 * no columns; its data pointer may be NULL), H a multiple of 16.
 */
int32_t sparse_mla_fwd(const swa_tensor* q, const swa_tensor* latent, const swa_tensor* k_pe,
                       const swa_tensor* indices, const int32_t* doc_ids, float scale,
                       swa_tensor* out, float* lse, void* stream);

/*
 * mla_value_proj — value up-projection that follows sparse MLA.
 *
 * For every token t and head h:  out[t,h,:] = value_weight[h] @ o_latent[t,h,:]
 * i.e. out[t,h,v] = sum_d value_weight[h,v,d] * o_latent[t,h,d], accumulated in f32 and
 * rounded to bf16 once. Defined by sparse_mla (value_weight [heads, value_dim, 512],
 * returns [tokens, heads, value_dim]) on the
 * nemo_automodel.components.models.mistral_large4.attention page; applied to the output of
 * sparse_mla_fwd it completes that operation (rows of zeros stay zero).
 *
 *   o_latent      [T, H, 512] bf16 (e.g. sparse_mla_fwd's out)
 *   value_weight  [H, Dv, 512] bf16
 *   out           [T, H, Dv] bf16
 * Supported: Dv in {64, 128}, H <= 65535, and o_latent's token stride below 128 MiB
 * (SWA_ERR_UNSUPPORTED otherwise). out must not alias an input (SWA_ERR_ARG). T = 0 is a
 * no-op. The grid is sized from the current device's compute-unit count (queried on the
 * host at each call).
 */
int32_t mla_value_proj(const swa_tensor* o_latent, const swa_tensor* value_weight, swa_tensor* out,
                       void* stream);

/* Static description of a status code. Never NULL. */
const char* swa_strerror(int32_t status);

/* Detail of the last failing call on the calling thread ("" if none). Never NULL. */
const char* swa_last_error(void);

/* SWA_ABI_VERSION of the loaded library. */
int32_t swa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_H_ */
