// Internal interface between the C ABI layer (abi.cpp) and the kernel launchers.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace swa {

// Packed varlen GQA forward. All strides in elements.
struct DenseFwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;  // token / head strides
  const int32_t* cu_seqlens;                              // device [n_docs + 1] or null
  const float* sinks;                                     // device [Hq] or null
  float* lse;                                             // device [T, Hq] or null
  int32_t T, n_docs, Hq, Hkv, G;
  int32_t hb_shift;     // log2 of the query heads folded into one wave's 32 columns
  int32_t n_chunks;     // G >> hb_shift head chunks per KV head
  int32_t tile_tokens;  // tokens per workgroup = 128 >> hb_shift
  int32_t n_vtiles;     // virtual query tiles per (KV head, chunk)
  int32_t n_work;       // Hkv * n_chunks * n_vtiles
  uint32_t vt_magic;    // floor(L / n_vtiles) = (L * vt_magic) >> vt_shift for 0 <= L < 2^31
  int32_t vt_shift;
  int32_t window;
  float scale;
  float c2;             // scale * log2(e)
};

enum class Dtype : int32_t { F32 = 0, BF16 = 1 };

// Grid size (workgroups) the dense launcher will use; 0 when there is no work.
int64_t dense_fwd_grid(const DenseFwdParams& p);
// Fills the derived fields of p (hb_shift ... c2) from the user-facing ones.
void dense_fwd_plan(DenseFwdParams& p);
hipError_t dense_fwd_launch(const DenseFwdParams& p, Dtype dt, int D, hipStream_t stream);

// Packed varlen GQA backward (bf16, head_dim 64 or 128). `f` carries the forward's geometry and
// inputs (q, k, v, out = the forward output, lse = the forward LSE, read only); strides in
// elements.
struct DenseBwdParams {
  DenseFwdParams f;
  const void* dout;
  int64_t do_st, do_sh;
  float* delta;  // [T, Hq] contiguous: <dout, out> per row (written)
  void* dq;
  int64_t dq_st, dq_sh;
  void* dk;
  int64_t dk_st, dk_sh;
  void* dv;
  int64_t dv_st, dv_sh;
  float* dsinks;        // [Hq] or null (written when f.sinks is set)
  int32_t kv_tile;      // keys per dk/dv workgroup: 64 (head_dim 64) or 128 (head_dim 128)
  int32_t kv_n_vtiles;  // virtual key tiles per KV head
  int32_t kv_n_work;    // Hkv * kv_n_vtiles
  int32_t kv_heavy_first;  // key tiles in heavy-first order (set by dense_bwd_plan)
};

// Fills the key-tile plan for head_dim D (and, through dense_fwd_plan, the query-tile plan) of p.
void dense_bwd_plan(DenseBwdParams& p, int D);
hipError_t dense_bwd_launch(const DenseBwdParams& p, int D, hipStream_t stream);

// Sparse MLA forward (bf16). Strides in elements.
struct SparseMlaParams {
  const void* q;       // [T, H, 512 + Dr]
  const void* latent;  // [T, 512]
  const void* k_pe;    // [T, Dr] (unused when Dr = 0)
  const int32_t* indices;  // [T, topk]
  const int32_t* doc_ids;  // [T]
  void* out;           // [T, H, 512]
  float* lse;          // [T, H] or null
  int64_t q_st, q_sh, lat_st, kpe_st, idx_st, o_st, o_sh;
  int32_t T, H, topk;
  int32_t Dr;  // rotary width: 64, or 0 (NoPE)
  float scale;
  float c2;
};

hipError_t sparse_mla_fwd_launch(const SparseMlaParams& p, hipStream_t stream);

// Sparse MLA value up-projection (bf16): out[t, h, :] = w[h] o[t, h, :]. Strides in elements.
struct MlaValueProjParams {
  const void* o;  // [T, H, 512]
  const void* w;  // [H, Dv, 512]
  void* out;      // [T, H, Dv]
  int64_t o_st, o_sh, w_sh, w_sv, out_st, out_sh;
  int32_t T, H, Dv;
};

// `n_cu`: compute units of the device (sizes the grid for one resident workgroup per CU).
hipError_t mla_value_proj_launch(const MlaValueProjParams& p, int n_cu, hipStream_t stream);

}  // namespace swa
