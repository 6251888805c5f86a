// C ABI of libswattn.so: argument validation on the host, then one asynchronous launch.
// Declarations and the full contract are in include/swattn.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/swattn.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int elem_size(int32_t dtype) {
  switch (dtype) {
    case SWA_DTYPE_F32: return 4;
    case SWA_DTYPE_BF16: return 2;
    case SWA_DTYPE_I32: return 4;
    default: return 0;
  }
}

// Shape/stride/alignment checks shared by every tensor argument.
// `row_align` is the byte alignment every row (and the base pointer) must keep: 16 for
// tensors the kernels read in 16-byte vectors, 4 for the index rows read element-wise.
int32_t check_tensor(const swa_tensor* t, const char* name, int ndim, int row_align = 16) {
  if (t == nullptr) return fail(SWA_ERR_NULL, "%s: descriptor is NULL", name);
  if (t->ndim != ndim) return fail(SWA_ERR_SHAPE, "%s: expected rank %d, got %d", name, ndim, t->ndim);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(SWA_ERR_SHAPE, "%s: negative extent in dim %d", name, i);
    numel *= t->shape[i];
  }
  const int es = elem_size(t->dtype);
  if (es == 0) return fail(SWA_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  if (numel == 0 && t->data == nullptr) return SWA_OK;
  if (t->data == nullptr) return fail(SWA_ERR_NULL, "%s: data pointer is NULL", name);
  if (t->stride[ndim - 1] != 1) return fail(SWA_ERR_LAYOUT, "%s: innermost stride must be 1", name);
  if ((reinterpret_cast<uintptr_t>(t->data) % row_align) != 0)
    return fail(SWA_ERR_LAYOUT, "%s: data pointer must be %d-byte aligned", name, row_align);
  for (int i = 0; i + 1 < ndim; ++i) {
    if (t->stride[i] < 0) return fail(SWA_ERR_LAYOUT, "%s: negative stride in dim %d", name, i);
    if ((t->stride[i] * es) % row_align != 0)
      return fail(SWA_ERR_LAYOUT, "%s: stride of dim %d must be a multiple of %d bytes", name, i, row_align);
  }
  return SWA_OK;
}

bool same_data(const swa_tensor* a, const swa_tensor* b) { return a->data != nullptr && a->data == b->data; }

}  // namespace

namespace swa {
// Sets the calling thread's swa_last_error() detail and returns `code` (for entry points
// defined outside this file).
int32_t abi_fail(int32_t code, const char* detail) { return fail(code, "%s", detail); }
}  // namespace swa

extern "C" {

int32_t swa_abi_version(void) { return SWA_ABI_VERSION; }

const char* swa_last_error(void) { return g_last_error.c_str(); }

const char* swa_strerror(int32_t status) {
  switch (status) {
    case SWA_OK: return "success";
    case SWA_ERR_NULL: return "a required pointer is NULL";
    case SWA_ERR_DTYPE: return "unsupported or mismatched element type";
    case SWA_ERR_SHAPE: return "ranks or shapes disagree";
    case SWA_ERR_ARG: return "a scalar argument is out of range";
    case SWA_ERR_UNSUPPORTED: return "configuration not implemented";
    case SWA_ERR_LAYOUT: return "stride or alignment requirement violated";
    case SWA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int32_t varlen_attn_fwd(const swa_tensor* q, const swa_tensor* k, const swa_tensor* v,
                        const int32_t* cu_seqlens, int32_t n_docs, int32_t window, float scale,
                        const float* sinks, swa_tensor* out, float* lse, void* stream) {
  g_last_error.clear();
  int32_t st;
  if ((st = check_tensor(q, "q", 3)) != SWA_OK) return st;
  if ((st = check_tensor(k, "k", 3)) != SWA_OK) return st;
  if ((st = check_tensor(v, "v", 3)) != SWA_OK) return st;
  if ((st = check_tensor(out, "out", 3)) != SWA_OK) return st;
  if (q->dtype != SWA_DTYPE_BF16 && q->dtype != SWA_DTYPE_F32)
    return fail(SWA_ERR_DTYPE, "q: dtype must be bf16 or f32");
  if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype)
    return fail(SWA_ERR_DTYPE, "q, k, v and out must share one dtype");
  const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t Hkv = k->shape[1];
  if (k->shape[0] != T || v->shape[0] != T || out->shape[0] != T)
    return fail(SWA_ERR_SHAPE, "q, k, v and out must have the same token count");
  if (v->shape[1] != Hkv || k->shape[2] != D || v->shape[2] != D)
    return fail(SWA_ERR_SHAPE, "k and v must both be [T, Hkv, D] with q's D");
  if (out->shape[1] != Hq || out->shape[2] != D) return fail(SWA_ERR_SHAPE, "out must be [T, Hq, D]");
  if (Hq <= 0 || Hkv <= 0) return fail(SWA_ERR_SHAPE, "head counts must be positive");
  if (Hq % Hkv != 0) return fail(SWA_ERR_SHAPE, "Hq (%lld) must be a multiple of Hkv (%lld)",
                                 (long long)Hq, (long long)Hkv);
  if (T > (int64_t)1 << 30 || Hq > 65536) return fail(SWA_ERR_UNSUPPORTED, "T or Hq too large");
  if (D != 64 && D != 128 && !(D == 256 && q->dtype == SWA_DTYPE_BF16))
    return fail(SWA_ERR_UNSUPPORTED, "head_dim %lld not supported (64 or 128; 256 for bf16)", (long long)D);
  // per-tile row offsets are computed in 32 bits: 64 rows x token stride must fit
  if (k->stride[0] >= (int64_t)1 << 24 || v->stride[0] >= (int64_t)1 << 24)
    return fail(SWA_ERR_UNSUPPORTED, "k/v token stride must be below 2^24 elements");
  // the output tile's store offsets are 32-bit byte offsets from the wave's first row
  if (out->stride[0] >= (int64_t)1 << 24 || out->stride[1] >= (int64_t)1 << 24)
    return fail(SWA_ERR_UNSUPPORTED, "out token and head strides must be below 2^24 elements");
  if (n_docs < 0) return fail(SWA_ERR_ARG, "n_docs must be >= 0");
  if (window < 0) return fail(SWA_ERR_ARG, "window must be >= 0");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(SWA_ERR_ARG, "scale must be finite and > 0");
  if (n_docs > 0 && cu_seqlens == nullptr) return fail(SWA_ERR_NULL, "cu_seqlens is NULL with n_docs > 0");
  if (T > 0 && (same_data(out, q) || same_data(out, k) || same_data(out, v)))
    return fail(SWA_ERR_ARG, "out must not alias q, k or v");
  if (T == 0) return SWA_OK;
  if (static_cast<int64_t>(n_docs) + 2 + T > INT32_MAX / 2) return fail(SWA_ERR_UNSUPPORTED, "too many documents");

  swa::DenseFwdParams p{};
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.out = out->data;
  p.q_st = q->stride[0];
  p.q_sh = q->stride[1];
  p.k_st = k->stride[0];
  p.k_sh = k->stride[1];
  p.v_st = v->stride[0];
  p.v_sh = v->stride[1];
  p.o_st = out->stride[0];
  p.o_sh = out->stride[1];
  p.cu_seqlens = n_docs > 0 ? cu_seqlens : nullptr;
  p.sinks = sinks;
  p.lse = lse;
  p.T = (int32_t)T;
  p.n_docs = n_docs;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.window = window;
  p.scale = scale;
  swa::dense_fwd_plan(p);
  if ((int64_t)p.Hkv * p.n_chunks * p.n_vtiles > INT32_MAX / 2)
    return fail(SWA_ERR_UNSUPPORTED, "problem too large for one launch");
  const swa::Dtype dt = q->dtype == SWA_DTYPE_BF16 ? swa::Dtype::BF16 : swa::Dtype::F32;
  const hipError_t e = swa::dense_fwd_launch(p, dt, (int)D, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SWA_ERR_LAUNCH, "varlen_attn_fwd launch: %s", hipGetErrorString(e));
  return SWA_OK;
}

int32_t varlen_attn_bwd(const swa_tensor* q, const swa_tensor* k, const swa_tensor* v, const swa_tensor* out,
                        const swa_tensor* dout, const float* lse, const int32_t* cu_seqlens, int32_t n_docs,
                        int32_t window, float scale, const float* sinks, swa_tensor* dq, swa_tensor* dk,
                        swa_tensor* dv, float* dsinks, float* delta, void* stream) {
  g_last_error.clear();
  int32_t st;
  const swa_tensor* ins[] = {q, k, v, out, dout};
  const char* in_names[] = {"q", "k", "v", "out", "dout"};
  for (int i = 0; i < 5; ++i)
    if ((st = check_tensor(ins[i], in_names[i], 3)) != SWA_OK) return st;
  swa_tensor* outs[] = {dq, dk, dv};
  const char* out_names[] = {"dq", "dk", "dv"};
  for (int i = 0; i < 3; ++i)
    if ((st = check_tensor(outs[i], out_names[i], 3)) != SWA_OK) return st;
  for (int i = 0; i < 5; ++i)
    if (ins[i]->dtype != SWA_DTYPE_BF16) return fail(SWA_ERR_DTYPE, "%s must be bf16", in_names[i]);
  for (int i = 0; i < 3; ++i)
    if (outs[i]->dtype != SWA_DTYPE_BF16) return fail(SWA_ERR_DTYPE, "%s must be bf16", out_names[i]);
  const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t Hkv = k->shape[1];
  for (const swa_tensor* t : {q, out, dout, (const swa_tensor*)dq})
    if (t->shape[0] != T || t->shape[1] != Hq || t->shape[2] != D)
      return fail(SWA_ERR_SHAPE, "q, out, dout and dq must all be [T, Hq, D]");
  for (const swa_tensor* t : {k, v, (const swa_tensor*)dk, (const swa_tensor*)dv})
    if (t->shape[0] != T || t->shape[1] != Hkv || t->shape[2] != D)
      return fail(SWA_ERR_SHAPE, "k, v, dk and dv must all be [T, Hkv, D]");
  if (Hq <= 0 || Hkv <= 0) return fail(SWA_ERR_SHAPE, "head counts must be positive");
  if (Hq % Hkv != 0) return fail(SWA_ERR_SHAPE, "Hq (%lld) must be a multiple of Hkv (%lld)",
                                 (long long)Hq, (long long)Hkv);
  if (D != 64 && D != 128)
    return fail(SWA_ERR_UNSUPPORTED, "backward head_dim %lld not supported (64 or 128)", (long long)D);
  if (T * Hq >= (int64_t)1 << 30) return fail(SWA_ERR_UNSUPPORTED, "T * Hq too large");
  for (const swa_tensor* t : {q, k, v, dout})
    if (t->stride[0] >= (int64_t)1 << 24) return fail(SWA_ERR_UNSUPPORTED, "token strides must be below 2^24 elements");
  // dq's store offsets are 32-bit byte offsets from the wave's first row
  if (dq->stride[0] >= (int64_t)1 << 24 || dq->stride[1] >= (int64_t)1 << 24)
    return fail(SWA_ERR_UNSUPPORTED, "dq token and head strides must be below 2^24 elements");
  if (n_docs < 0) return fail(SWA_ERR_ARG, "n_docs must be >= 0");
  if (window < 0) return fail(SWA_ERR_ARG, "window must be >= 0");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(SWA_ERR_ARG, "scale must be finite and > 0");
  if (n_docs > 0 && cu_seqlens == nullptr) return fail(SWA_ERR_NULL, "cu_seqlens is NULL with n_docs > 0");
  if (T > 0 && (lse == nullptr || delta == nullptr)) return fail(SWA_ERR_NULL, "lse and delta are required");
  if (T > 0 && sinks != nullptr && dsinks == nullptr) return fail(SWA_ERR_NULL, "dsinks is required with sinks");
  if (T > 0) {
    for (const swa_tensor* o : {(const swa_tensor*)dq, (const swa_tensor*)dk, (const swa_tensor*)dv})
      for (const swa_tensor* i : ins)
        if (same_data(o, i)) return fail(SWA_ERR_ARG, "gradients must not alias an input");
    if (same_data(dq, dk) || same_data(dq, dv) || same_data(dk, dv))
      return fail(SWA_ERR_ARG, "dq, dk and dv must be distinct");
  }
  if (T == 0) return SWA_OK;
  if (static_cast<int64_t>(n_docs) + 2 + T > INT32_MAX / 2) return fail(SWA_ERR_UNSUPPORTED, "too many documents");

  swa::DenseBwdParams p{};
  swa::DenseFwdParams& f = p.f;
  f.q = q->data;
  f.k = k->data;
  f.v = v->data;
  f.out = out->data;
  f.q_st = q->stride[0];
  f.q_sh = q->stride[1];
  f.k_st = k->stride[0];
  f.k_sh = k->stride[1];
  f.v_st = v->stride[0];
  f.v_sh = v->stride[1];
  f.o_st = out->stride[0];
  f.o_sh = out->stride[1];
  f.cu_seqlens = n_docs > 0 ? cu_seqlens : nullptr;
  f.sinks = sinks;
  f.lse = const_cast<float*>(lse);
  f.T = (int32_t)T;
  f.n_docs = n_docs;
  f.Hq = (int32_t)Hq;
  f.Hkv = (int32_t)Hkv;
  f.window = window;
  f.scale = scale;
  p.dout = dout->data;
  p.do_st = dout->stride[0];
  p.do_sh = dout->stride[1];
  p.delta = delta;
  p.dq = dq->data;
  p.dq_st = dq->stride[0];
  p.dq_sh = dq->stride[1];
  p.dk = dk->data;
  p.dk_st = dk->stride[0];
  p.dk_sh = dk->stride[1];
  p.dv = dv->data;
  p.dv_st = dv->stride[0];
  p.dv_sh = dv->stride[1];
  p.dsinks = sinks != nullptr ? dsinks : nullptr;
  swa::dense_bwd_plan(p, (int)D);
  if ((int64_t)f.Hkv * f.n_chunks * f.n_vtiles > INT32_MAX / 2 || (int64_t)f.Hkv * p.kv_n_vtiles > INT32_MAX / 2)
    return fail(SWA_ERR_UNSUPPORTED, "problem too large for one launch");
  const hipError_t e = swa::dense_bwd_launch(p, (int)D, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SWA_ERR_LAUNCH, "varlen_attn_bwd launch: %s", hipGetErrorString(e));
  return SWA_OK;
}

int32_t sparse_mla_fwd(const swa_tensor* q, const swa_tensor* latent, const swa_tensor* k_pe,
                       const swa_tensor* indices, const int32_t* doc_ids, float scale,
                       swa_tensor* out, float* lse, void* stream) {
  g_last_error.clear();
  int32_t st;
  if ((st = check_tensor(q, "q", 3)) != SWA_OK) return st;
  if ((st = check_tensor(latent, "latent", 2)) != SWA_OK) return st;
  if ((st = check_tensor(k_pe, "k_pe", 2)) != SWA_OK) return st;
  if ((st = check_tensor(indices, "indices", 2, 4)) != SWA_OK) return st;
  if ((st = check_tensor(out, "out", 3)) != SWA_OK) return st;
  if (q->dtype != SWA_DTYPE_BF16 || latent->dtype != SWA_DTYPE_BF16 || k_pe->dtype != SWA_DTYPE_BF16 ||
      out->dtype != SWA_DTYPE_BF16)
    return fail(SWA_ERR_DTYPE, "q, latent, k_pe and out must be bf16");
  if (indices->dtype != SWA_DTYPE_I32) return fail(SWA_ERR_DTYPE, "indices must be int32");
  const int64_t T = q->shape[0], H = q->shape[1], Dqk = q->shape[2];
  const int64_t Dl = latent->shape[1], Dr = k_pe->shape[1], topk = indices->shape[1];
  if (latent->shape[0] != T || k_pe->shape[0] != T || indices->shape[0] != T || out->shape[0] != T)
    return fail(SWA_ERR_SHAPE, "q, latent, k_pe, indices and out must have the same token count");
  if (Dqk != Dl + Dr) return fail(SWA_ERR_SHAPE, "q's last dim must equal latent dim + rotary dim");
  if (out->shape[1] != H || out->shape[2] != Dl) return fail(SWA_ERR_SHAPE, "out must be [T, H, latent dim]");
  if (Dl != 512 || (Dr != 64 && Dr != 0))
    return fail(SWA_ERR_UNSUPPORTED, "only latent 512 with rotary 64 or 0 (NoPE) is supported");
  if (H <= 0 || H % 16 != 0 || H > 4096) return fail(SWA_ERR_UNSUPPORTED, "H must be a positive multiple of 16");
  if (topk < 1) return fail(SWA_ERR_ARG, "topk must be >= 1");
  if (topk > (1 << 20)) return fail(SWA_ERR_UNSUPPORTED, "topk too large");
  if (T > (int64_t)1 << 30) return fail(SWA_ERR_UNSUPPORTED, "T too large");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(SWA_ERR_ARG, "scale must be finite and > 0");
  if (T > 0 && doc_ids == nullptr) return fail(SWA_ERR_NULL, "doc_ids is NULL");
  if (T > 0 && (same_data(out, q) || same_data(out, latent) || same_data(out, k_pe)))
    return fail(SWA_ERR_ARG, "out must not alias an input");
  if (T == 0) return SWA_OK;
  // the gathers address both tensors with 32-bit byte offsets from their bases
  if ((T - 1) * latent->stride[0] * 2 + 1024 > (int64_t)UINT32_MAX ||
      (Dr > 0 && (T - 1) * k_pe->stride[0] * 2 + 128 > (int64_t)UINT32_MAX))
    return fail(SWA_ERR_UNSUPPORTED, "latent or k_pe spans more than 4 GiB");

  swa::SparseMlaParams p{};
  p.q = q->data;
  p.latent = latent->data;
  p.k_pe = k_pe->data;
  p.indices = static_cast<const int32_t*>(indices->data);
  p.doc_ids = doc_ids;
  p.out = out->data;
  p.lse = lse;
  p.q_st = q->stride[0];
  p.q_sh = q->stride[1];
  p.lat_st = latent->stride[0];
  p.kpe_st = Dr > 0 ? k_pe->stride[0] : 0;
  p.idx_st = indices->stride[0];
  p.o_st = out->stride[0];
  p.o_sh = out->stride[1];
  p.T = (int32_t)T;
  p.H = (int32_t)H;
  p.topk = (int32_t)topk;
  p.Dr = (int32_t)Dr;
  p.scale = scale;
  p.c2 = scale * 1.4426950408889634f;
  const hipError_t e = swa::sparse_mla_fwd_launch(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SWA_ERR_LAUNCH, "sparse_mla_fwd launch: %s", hipGetErrorString(e));
  return SWA_OK;
}

int32_t mla_value_proj(const swa_tensor* o_latent, const swa_tensor* value_weight, swa_tensor* out,
                       void* stream) {
  g_last_error.clear();
  int32_t st;
  if ((st = check_tensor(o_latent, "o_latent", 3)) != SWA_OK) return st;
  if ((st = check_tensor(value_weight, "value_weight", 3)) != SWA_OK) return st;
  if ((st = check_tensor(out, "out", 3)) != SWA_OK) return st;
  if (o_latent->dtype != SWA_DTYPE_BF16 || value_weight->dtype != SWA_DTYPE_BF16 || out->dtype != SWA_DTYPE_BF16)
    return fail(SWA_ERR_DTYPE, "o_latent, value_weight and out must be bf16");
  const int64_t T = o_latent->shape[0], H = o_latent->shape[1], Dl = o_latent->shape[2];
  const int64_t Dv = value_weight->shape[1];
  if (value_weight->shape[0] != H || value_weight->shape[2] != Dl)
    return fail(SWA_ERR_SHAPE, "value_weight must be [H, value_dim, latent dim]");
  if (out->shape[0] != T || out->shape[1] != H || out->shape[2] != Dv)
    return fail(SWA_ERR_SHAPE, "out must be [T, H, value_dim]");
  if (Dl != 512) return fail(SWA_ERR_UNSUPPORTED, "only latent dim 512 is supported");
  if (Dv != 64 && Dv != 128) return fail(SWA_ERR_UNSUPPORTED, "value_dim must be 64 or 128");
  if (H <= 0 || H > 65535) return fail(SWA_ERR_UNSUPPORTED, "H out of range");
  if (T > (int64_t)1 << 30) return fail(SWA_ERR_UNSUPPORTED, "T too large");
  if (o_latent->stride[0] * 2 * 32 + 1024 > (int64_t)UINT32_MAX)
    return fail(SWA_ERR_UNSUPPORTED, "o_latent tokens too far apart");
  if (T > 0 && (same_data(out, o_latent) || same_data(out, value_weight)))
    return fail(SWA_ERR_ARG, "out must not alias an input");
  if (T == 0) return SWA_OK;

  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
    return fail(SWA_ERR_LAUNCH, "mla_value_proj: cannot query the device");
  swa::MlaValueProjParams p{};
  p.o = o_latent->data;
  p.w = value_weight->data;
  p.out = out->data;
  p.o_st = o_latent->stride[0];
  p.o_sh = o_latent->stride[1];
  p.w_sh = value_weight->stride[0];
  p.w_sv = value_weight->stride[1];
  p.out_st = out->stride[0];
  p.out_sh = out->stride[1];
  p.T = (int32_t)T;
  p.H = (int32_t)H;
  p.Dv = (int32_t)Dv;
  const hipError_t e = swa::mla_value_proj_launch(p, n_cu, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SWA_ERR_LAUNCH, "mla_value_proj launch: %s", hipGetErrorString(e));
  return SWA_OK;
}

}  // extern "C"
