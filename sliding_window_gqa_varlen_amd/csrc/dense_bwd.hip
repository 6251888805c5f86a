// Packed variable-length causal / sliding-window GQA attention backward for gfx950 (bf16,
// head_dim 128).
//
// Operation: the gradients of a loss through `out` of the forward in dense_fwd.hip
// (MuseMagiPlan.attention on the muse_spark magi_cp page, FlintMagiPlan.attention on the
// flint magi page, GQA of MuseGlimmerAttention on the muse_glimmer model page), with the
// forward's log-sum-exp `lse` (sink included) kept from the forward pass:
//   P_ij = exp(scale q_i.k_j - lse_i)     delta_i = <dout_i, out_i>
//   dS_ij = P_ij (<dout_i, v_j> - delta_i)
//   dq_i = scale sum_j dS_ij k_j ;  dk_j = scale sum_{i,h} dS_ij q_i ;  dv_j = sum_{i,h} P_ij dout_i
//   dsink_h = -sum_i exp(sink_h - lse_i) delta_i
//
// Design (MFMA 32x32x16 bf16, fp32 accumulation, no atomics, no scratch beyond `delta`):
//  * delta kernel: one fp32 dot product per (token, head) row.
//  * dsink kernel: one workgroup per head reduces over the tokens in a fixed order.
//  * dq kernel (query-parallel): the forward's workgroup decomposition (per document, 128
//    query columns = tokens x folded GQA heads, XCD-aware placement).  Per 64-key tile:
//    S^T = K Q^T and dP^T = V dO^T with q and dout of the lane's column in registers, so
//    P^T = exp2(S^T c2 - lse_col) and dS^T = P^T (dP^T - delta_col) are lane-local; then
//    dQ^T += K^T dS^T with the K^T operand read transposed from LDS (ds_read_b64_tr_b16).
//  * dk/dv kernel (key-parallel): a workgroup owns 128 keys of one KV head (32 per wave,
//    their K and V rows held in registers) and walks the 64-query tiles of every query head
//    of the group that can see them.  S = Q K^T and dP = dO V^T (queries = M, keys = N),
//    so the lane of a key column holds P and dS in the B-operand layout of
//    dV^T += dO^T P and dK^T += Q^T dS, whose A operands are transposed LDS reads of the
//    staged Q and dO tiles.  All heads of the group accumulate in registers: GQA needs no
//    reduction pass.
//  * K tiles (dq kernel) and Q / dO tiles (dk/dv kernel) are read both row-wise and
//    transposed, so their 16-byte units are swizzled with rt_key(r) (row bits 0-1 into unit
//    bits 2-3, row bits 2-3 into unit bits 0-1), which keeps both access patterns free of
//    bank conflicts.  V tiles (dq kernel) are only read row-wise (unit ^ (r & 15)).
//  * Tiles travel HBM -> LDS by buffer_load ... lds into two statically named buffers per
//    operand (loop unrolled by two): the next tile is in flight while this one is used.
#include "dense_common.h"

namespace swa {
namespace {

constexpr int kBD = 128;           // head_dim of this path
constexpr int kU = kBD / 8;        // 16-byte units per row
constexpr int kQF = kBD / 16;      // k-steps of 16 coordinates
constexpr int kDB = kBD / 32;      // 32-row output blocks
constexpr int kTileUnits = 64 * kU;
constexpr int kTK = 128;           // keys per dk/dv workgroup
#ifndef SWA_BWD_AHEAD
#define SWA_BWD_AHEAD 8
#endif

__device__ __forceinline__ int rt_key(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int row_key(int r) { return r & 15; }

// 64 rows (r0 .. r0 + 63, clamped to r_last >= r0) of 128 bf16 each into buf; logical unit u of
// row r lands at physical unit u ^ key(r).  Four transfers per wave.
template <bool RT>
__device__ __forceinline__ void dma_rows64(const __bf16* base, int64_t st, int r0, int r_last, u32x4* buf, int wave,
                                           int lane_in) {
  const int lane = opaque(lane_in);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)r0 * st), (short)0, -1, kBufferWord3);
  const uint32_t stb = (uint32_t)st * 2u;
  const int lim = r_last - r0;
  const int lr = lane >> 4, lp = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = i * 4 + wave;  // wave-uniform block of 4 rows
    const int r = blk * 4 + lr;
    const int cu = lp ^ (RT ? rt_key(r) : row_key(r));
    u32x4* dst = buf + __builtin_amdgcn_readfirstlane(blk * 64);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, (uint32_t)min(r, lim) * stb + (uint32_t)cu * 16u,
                                             0, 0, 0);
  }
}

// 64 fp32 values base[(r0 + l) * Hq + h] (rows clamped to r_last) into buf[0..63]: one transfer.
__device__ __forceinline__ void dma_rowvals(const float* base, int Hq, int h, int r0, int r_last, float* buf,
                                            int lane) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, kBufferWord3);
  const int r = min(r0 + lane, r_last);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)buf, 4, (uint32_t)(r * Hq + h) * 4u, 0, 0, 0);
}

// Byte offset of the A-operand fragment of rows 32 blk + n, k-step s, in a row-swizzled tile:
// unit (2 s + h2) ^ key(n) = (h2 ^ key(n)) ^ 2 s, i.e. raddr ^ 32 s.
__device__ __forceinline__ const bf16x8& row_frag(const u32x4* buf, int raddr, int blk, int s) {
  return *(const bf16x8*)((const char*)buf + ((raddr ^ (32 * s)) + blk * 32 * kU * 16));
}

// Transposed A-operand reads (ds_read_b64_tr_b16) of an rt_key tile: lane j of a 16-lane group
// reads rows r0 = 4 h2 + j / 4 (+ 16 ks) and r0 + 8, 8-byte half (j & 1) of logical unit
// 4 d + 2 dh + ((j & 3) >> 1).  key(r0 + 8) = key(r0) ^ 2.
struct TrOffsets {
  int lo[kDB], hi[kDB];
};
__device__ __forceinline__ TrOffsets tr_offsets(int lane) {
  const int j16 = lane & 15, dh = (lane >> 4) & 1, h2 = lane >> 5;
  const int r0 = 4 * h2 + (j16 >> 2);
  const int k0 = rt_key(r0);
  const int sub = (j16 & 3) >> 1;
  const int half = (j16 & 1) * 4;
  TrOffsets t;
#pragma unroll
  for (int d = 0; d < kDB; ++d) {
    const int u = 4 * d + 2 * dh + sub;
    t.lo[d] = ((r0 * kU + (u ^ k0)) * 8 + half) * 2;
    t.hi[d] = (((r0 + 8) * kU + (u ^ k0 ^ 2)) * 8 + half) * 2;
  }
  return t;
}
__device__ __forceinline__ bf16x8 tr_frag(const u32x4* buf, const TrOffsets& t, int ks, int d) {
  const char* p = (const char*)buf + ks * 16 * kU * 16;
  const bf16x4 lo4 = lds_read_tr4((const __bf16*)(p + t.lo[d]));
  const bf16x4 hi4 = lds_read_tr4((const __bf16*)(p + t.hi[d]));
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// bf16 B operand of k-step ks (16 rows) from a pair of C-layout accumulators
__device__ __forceinline__ bf16x8 pack_ks(const f32x16 (&x)[2], int ks) {
  f32x8 pf;
#pragma unroll
  for (int e = 0; e < 8; ++e) pf[e] = x[ks >> 1][8 * (ks & 1) + e];
  return cvt_bf16x8(pf);
}

// ======================================================================================
// delta = <dout, out> per (token, head) row, and dsink
// ======================================================================================
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(DenseBwdParams p) {
  constexpr int LPR = kBD / 8;   // lanes per row (16 bytes each)
  constexpr int RPW = 64 / LPR;  // rows per wave step
  const int n_rows = p.f.T * p.f.Hq;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, u = lane % LPR;
  const int stride = gridDim.x * (kThreads / 64) * RPW;
  for (int base = (blockIdx.x * (kThreads / 64) + (int)(threadIdx.x >> 6)) * RPW; base < n_rows; base += stride) {
    const int r = base + sub;
    float acc = 0.f;
    if (r < n_rows) {
      const int t = r / p.f.Hq, h = r - t * p.f.Hq;
      const bf16x8 o = *(const bf16x8*)((const __bf16*)p.f.out + (int64_t)t * p.f.o_st + (int64_t)h * p.f.o_sh + 8 * u);
      const bf16x8 g = *(const bf16x8*)((const __bf16*)p.dout + (int64_t)t * p.do_st + (int64_t)h * p.do_sh + 8 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (r < n_rows && u == 0) p.delta[r] = acc;
  }
}

// dsink_h = -sum_t exp(sink_h - lse[t, h]) delta[t, h]; rows with lse = -inf (padding) add 0.
__global__ __launch_bounds__(kThreads) void bwd_dsink_kernel(DenseBwdParams p) {
  __shared__ float part[kThreads / 64];
  const int h = blockIdx.x;
  const float s = p.f.sinks[h];
  float acc = 0.f;
  for (int t = threadIdx.x; t < p.f.T; t += kThreads) {
    const float l = p.f.lse[(int64_t)t * p.f.Hq + h];
    if (l != -INFINITY) acc += __expf(s - l) * p.delta[(int64_t)t * p.f.Hq + h];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) tot += part[w];
    p.dsinks[h] = -tot;
  }
}

// ======================================================================================
// dq: query-parallel, the forward's tiles
// ======================================================================================
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(DenseBwdParams p) {
  __shared__ u32x4 k0[kTileUnits];
  __shared__ u32x4 k1[kTileUnits];
  __shared__ u32x4 v0[kTileUnits];
  __shared__ u32x4 v1[kTileUnits];
  const DenseFwdParams& f = p.f;

  Tile w;
  if (!decode_tile(f, w)) return;
  if (w.padding) {  // tokens outside every document receive no gradient
    const int n_rows = (w.t_end - w.t0) * w.HB;
    for (int idx = threadIdx.x; idx < n_rows * kU; idx += kThreads) {
      const int row = idx / kU, cu = idx - row * kU;
      const int t = w.t0 + row / w.HB, h = w.h0 + row % w.HB;
      *(u32x4*)((__bf16*)p.dq + (int64_t)t * p.dq_st + (int64_t)h * p.dq_sh + cu * 8) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  const Cols c = make_cols(f, w);
  const int tq = min(c.tq, w.t_end - 1);
  bf16x8 qf[kQF], gf[kQF];
  {
    const __bf16* qb = (const __bf16*)f.q + (int64_t)tq * f.q_st + (int64_t)c.hq * f.q_sh + 8 * c.h2;
    const __bf16* gb = (const __bf16*)p.dout + (int64_t)tq * p.do_st + (int64_t)c.hq * p.do_sh + 8 * c.h2;
#pragma unroll
    for (int s = 0; s < kQF; ++s) {
      qf[s] = *(const bf16x8*)(qb + 16 * s);
      gf[s] = *(const bf16x8*)(gb + 16 * s);
    }
  }
  const float lse2 = f.lse[(int64_t)tq * f.Hq + c.hq] * kLog2e;
  const float dl = p.delta[(int64_t)tq * f.Hq + c.hq];
  const float c2 = f.c2;
  const __bf16* kbase = (const __bf16*)f.k + (int64_t)w.g * f.k_sh;
  const __bf16* vbase = (const __bf16*)f.v + (int64_t)w.g * f.v_sh;
  const int kraddr = c.n * kU * 16 + ((c.h2 ^ rt_key(c.n)) << 4);
  const int vraddr = c.n * kU * 16 + ((c.h2 ^ row_key(c.n)) << 4);
  const TrOffsets to = tr_offsets(c.lane);

  f32x16 acc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) acc[d] = f32x16{};
  const int nt = c.n_tiles;
  const int last = c.k_hi - 1;

  auto tile = [&](const u32x4* kb_, const u32x4* vb_, int kb) {
    if (!tile_active(c, kb)) return;  // none of this wave's tokens sees these keys
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sc[blk] = f32x16{};
      dp[blk] = f32x16{};
#pragma unroll
      for (int s = 0; s < kQF; ++s) sc[blk] = mfma_bf16_32x32x16(row_frag(kb_, kraddr, blk, s), qf[s], sc[blk]);
#pragma unroll
      for (int s = 0; s < kQF; ++s) dp[blk] = mfma_bf16_32x32x16(row_frag(vb_, vraddr, blk, s), gf[s], dp[blk]);
    }
    if (tile_needs_mask(c, kb)) mask_tile(sc, kb, c);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float pr = fast_exp2(__builtin_fmaf(sc[blk][a], c2, -lse2));
        sc[blk][a] = pr * (dp[blk][a] - dl);
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 sb = pack_ks(sc, ks);
#pragma unroll
      for (int d = 0; d < kDB; ++d) acc[d] = mfma_bf16_32x32x16(tr_frag(kb_, to, ks, d), sb, acc[d]);
    }
  };

  dma_rows64<true>(kbase, f.k_st, c.k_lo, last, k0, c.wave, c.lane);
  dma_rows64<false>(vbase, f.v_st, c.k_lo, last, v0, c.wave, c.lane);
  int j = 0;
  for (; j + 1 < nt; j += 2) {
    wait_vm0();
    barrier_keep_loads();  // tile j landed for every wave; tile j - 1 fully consumed
    dma_rows64<true>(kbase, f.k_st, c.k_lo + (j + 1) * kBN, last, k1, c.wave, c.lane);
    dma_rows64<false>(vbase, f.v_st, c.k_lo + (j + 1) * kBN, last, v1, c.wave, c.lane);
    tile(k0, v0, c.k_lo + j * kBN);
    wait_vm0();
    barrier_keep_loads();
    if (j + 2 < nt) {
      dma_rows64<true>(kbase, f.k_st, c.k_lo + (j + 2) * kBN, last, k0, c.wave, c.lane);
      dma_rows64<false>(vbase, f.v_st, c.k_lo + (j + 2) * kBN, last, v0, c.wave, c.lane);
    }
    tile(k1, v1, c.k_lo + (j + 1) * kBN);
  }
  if (j < nt) {
    wait_vm0();
    barrier_keep_loads();
    tile(k0, v0, c.k_lo + j * kBN);
  }

  if (c.tq < w.t_end) {
    __bf16* ob = (__bf16*)p.dq + (int64_t)c.tq * p.dq_st + (int64_t)c.hq * p.dq_sh + 4 * c.h2;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = acc[d][4 * i + e] * f.scale;
        *(bf16x4*)(ob + 32 * d + 8 * i) = cvt_bf16x4(r);
      }
  }
}

// ======================================================================================
// dk, dv: key-parallel
// ======================================================================================
struct KeyTile {
  int g, k0, k1, seg_start, seg_end;
  bool padding;
};

// blockIdx -> (KV head, 128-key tile of a segment); each KV head's tiles on one XCD, each
// document's tiles first-first (under a causal mask the first keys are seen by the most queries).
__device__ __forceinline__ bool decode_key_tile(const DenseBwdParams& p, KeyTile& w) {
  const DenseFwdParams& f = p.f;
  const int per_xcd = gridDim.x / kXcds;
  const int L = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (L >= p.kv_n_work) return false;
  const int VT = p.kv_n_vtiles;
  w.g = L / VT;
  const int v = L - w.g * VT;
  int lo = 0, hi = f.n_docs + 2;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_bound(f, mid) / kTK + mid <= v) lo = mid; else hi = mid;
  }
  w.seg_start = seg_bound(f, lo);
  w.seg_end = seg_bound(f, lo + 1);
  w.k0 = w.seg_start + (v - (w.seg_start / kTK + lo)) * kTK;
  if (w.k0 >= w.seg_end) return false;
  w.k1 = min(w.k0 + kTK, w.seg_end);
  w.padding = (lo == 0 || lo == f.n_docs + 1);
  return true;
}

// One 64-query x 32-key tile of the dk/dv kernel as two fenced instruction streams (the
// emitted order is the program order; operand fragments are read kAhead MFMAs ahead):
//  1. S = Q K^T and dP = dO V^T (32 MFMAs, the two query blocks alternating); the
//     probabilities P = exp2(S c2 - lse log2 e) of the tile run in the dP slots.
//  2. dV^T += dO^T P and dK^T += Q^T dS (32 MFMAs); dS = P (dP - delta) runs in the dV slots.
// Rows of the tile are queries; `qoff` = first query - this lane's key, `eoff` = document end -
// key (the mask of MASK tiles: 0 <= query - key, query < end, and query - key < W when W > 0).
template <bool MASK>
__device__ __forceinline__ void dkdv_tile(const u32x4* qb, const u32x4* ob, const float* lb, const float* db,
                                          const bf16x8 (&kf)[kQF], const bf16x8 (&vf)[kQF], int raddr,
                                          const TrOffsets& to, float c2, f32x16 (&dk)[kDB], f32x16 (&dv)[kDB],
                                          int qoff, int eoff, int W, int h2) {
  constexpr int kAhead = SWA_BWD_AHEAD;
  bf16x8 frag[64];
  auto read = [&](int f) {
    if (f < 32) {  // S (f < 16) or dP: query block f & 1, k-step (f >> 1) & 7
      frag[f] = row_frag(f < 16 ? qb : ob, raddr, f & 1, (f >> 1) & 7);
    } else {       // dV (f < 48) or dK: k-step (f >> 2) & 3, output block f & 3
      frag[f] = tr_frag(f < 48 ? ob : qb, to, (f >> 2) & 3, f & 3);
    }
  };
  f32x4 l4[8], d4[8];  // lse and delta of query rows 32 b + 8 j + 4 h2 + (0..3), index 4 b + j
  f32x16 sc[2], dp[2];
  bf16x8 pb[4], sb[4];
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): nothing older in flight, later waits count exactly
  // rows of group x: 32 (x >> 2) + 8 (x & 3) + 4 h2 .. + 3; lse now, delta late in stream 1
  auto rows = [&](int x) { return 32 * (x >> 2) + 8 * (x & 3) + 4 * h2; };
#pragma unroll
  for (int x = 0; x < 8; ++x) l4[x] = *(const f32x4*)(lb + rows(x));
#pragma unroll
  for (int f = 0; f < kAhead; ++f) read(f);
  __builtin_amdgcn_sched_barrier(0);
  sc[0] = sc[1] = dp[0] = dp[1] = f32x16{};
  // stream 1a: S (16 MFMAs)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sc[i & 1] = mfma_bf16_32x32x16(frag[i], kf[i >> 1], sc[i & 1]);
    read(i + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  // stream 1b: dP (16 MFMAs) with the probabilities of S, two per slot
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    dp[i & 1] = mfma_bf16_32x32x16(frag[16 + i], vf[i >> 1], dp[i & 1]);
    read(16 + i + kAhead);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int x = 2 * i + e;  // element x of the tile's 32: block x >> 4, accumulator x & 15
      const int bb = x >> 4, a = x & 15;
      float pr = fast_exp2(__builtin_fmaf(sc[bb][a], c2, l4[x >> 2][a & 3] * -kLog2e));
      if constexpr (MASK) {
        const int d = qoff + 32 * bb + 8 * (a >> 2) + 4 * h2 + (a & 3);  // query - key
        pr = (d >= 0 && d < eoff && (W == 0 || d < W)) ? pr : 0.f;
      }
      sc[bb][a] = pr;
      asm volatile("" : "+v"(sc[bb][a]));  // this slot's probabilities stay in this slot
      if ((x & 7) == 7) pb[x >> 3] = pack_ks(sc, x >> 3);
    }
    if (i >= 8) d4[i - 8] = *(const f32x4*)(db + rows(i - 8));
    __builtin_amdgcn_sched_barrier(0);
  }
  // stream 2a: dV^T += dO^T P (16 MFMAs) with dS, two elements per slot
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    dv[i & 3] = mfma_bf16_32x32x16(frag[32 + i], pb[i >> 2], dv[i & 3]);
    read(32 + i + kAhead);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int x = 2 * i + e;
      const int bb = x >> 4, a = x & 15;
      dp[bb][a] = sc[bb][a] * (dp[bb][a] - d4[x >> 2][a & 3]);
      asm volatile("" : "+v"(dp[bb][a]));
      if ((x & 7) == 7) sb[x >> 3] = pack_ks(dp, x >> 3);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // stream 2b: dK^T += Q^T dS (16 MFMAs)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    dk[i & 3] = mfma_bf16_32x32x16(frag[48 + i], sb[i >> 2], dk[i & 3]);
    if (48 + i + kAhead < 64) read(48 + i + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(DenseBwdParams p) {
  __shared__ u32x4 q0[kTileUnits];
  __shared__ u32x4 q1[kTileUnits];
  __shared__ u32x4 o0[kTileUnits];
  __shared__ u32x4 o1[kTileUnits];
  __shared__ f32x4 lsv[4][16];  // lse and delta rows of the two query-tile buffers (16-byte aligned)
  float* ls0 = (float*)lsv[0];
  float* ls1 = (float*)lsv[1];
  float* dl0 = (float*)lsv[2];
  float* dl1 = (float*)lsv[3];
  const DenseFwdParams& f = p.f;

  KeyTile w;
  if (!decode_key_tile(p, w)) return;
  if (w.padding) {  // keys outside every document receive no gradient
    const int n_rows = w.k1 - w.k0;
    for (int idx = threadIdx.x; idx < n_rows * kU; idx += kThreads) {
      const int row = idx / kU, cu = idx - row * kU;
      const int64_t t = w.k0 + row;
      *(u32x4*)((__bf16*)p.dk + t * p.dk_st + (int64_t)w.g * p.dk_sh + cu * 8) = u32x4{0, 0, 0, 0};
      *(u32x4*)((__bf16*)p.dv + t * p.dv_st + (int64_t)w.g * p.dv_sh + cu * 8) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, h2 = lane >> 5;
  const int W = f.window, e_doc = w.seg_end;
  const int kw0 = w.k0 + 32 * wave;  // this wave's keys kw0 .. kw0 + 31
  const bool has_keys = kw0 < w.k1;
  const int key = kw0 + n;           // this lane's key column

  // K and V rows of this lane's key as B operands: coordinates 16 s + 8 h2 .. + 7
  bf16x8 kf[kQF], vf[kQF];
  {
    const int kr = min(key, w.k1 - 1);
    const __bf16* kb = (const __bf16*)f.k + (int64_t)kr * f.k_st + (int64_t)w.g * f.k_sh + 8 * h2;
    const __bf16* vb = (const __bf16*)f.v + (int64_t)kr * f.v_st + (int64_t)w.g * f.v_sh + 8 * h2;
#pragma unroll
    for (int s = 0; s < kQF; ++s) {
      kf[s] = *(const bf16x8*)(kb + 16 * s);
      vf[s] = *(const bf16x8*)(vb + 16 * s);
    }
  }
  f32x16 dk[kDB], dv[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }
  // queries that see these keys: [k0, i_hi); 64-query tiles for every head of the group
  const int i_hi = W ? min(e_doc, w.k1 - 1 + W) : e_doc;
  const int n_qt = (i_hi - w.k0 + 63) / 64;
  const int n_it = f.G * n_qt;
  const int raddr = n * kU * 16 + ((h2 ^ rt_key(n)) << 4);
  const TrOffsets to = tr_offsets(lane);
  const float c2 = f.c2;

  auto issue = [&](int it, u32x4* qb, u32x4* ob, float* lb, float* db) {
    const int h = w.g * f.G + it / n_qt;
    const int i0 = w.k0 + 64 * (it % n_qt);
    dma_rows64<true>((const __bf16*)f.q + (int64_t)h * f.q_sh, f.q_st, i0, i_hi - 1, qb, wave, lane);
    dma_rows64<true>((const __bf16*)p.dout + (int64_t)h * p.do_sh, p.do_st, i0, i_hi - 1, ob, wave, lane);
    if (wave == 0) dma_rowvals(f.lse, f.Hq, h, i0, i_hi - 1, lb, lane);
    if (wave == 1) dma_rowvals(p.delta, f.Hq, h, i0, i_hi - 1, db, lane);
  };
  auto step = [&](int it, const u32x4* qb, const u32x4* ob, const float* lb, const float* db) {
    const int i0 = w.k0 + 64 * (it % n_qt);
    // wave-uniform: skip tiles none of whose queries sees this wave's keys
    if (!has_keys || i0 + 63 < kw0 || (W != 0 && i0 > kw0 + 31 + W - 1)) return;
    const bool need_mask = !(i0 >= kw0 + 31 && i0 + 63 < e_doc && (W == 0 || i0 + 63 - kw0 < W));
    if (need_mask)
      dkdv_tile<true>(qb, ob, lb, db, kf, vf, raddr, to, c2, dk, dv, i0 - key, e_doc - key, W, h2);
    else
      dkdv_tile<false>(qb, ob, lb, db, kf, vf, raddr, to, c2, dk, dv, i0 - key, e_doc - key, W, h2);
  };

  issue(0, q0, o0, ls0, dl0);
  int it = 0;
  for (; it + 1 < n_it; it += 2) {
    wait_vm0();
    barrier_keep_loads();  // tile it landed for every wave; tile it - 1 fully consumed
    issue(it + 1, q1, o1, ls1, dl1);
    step(it, q0, o0, ls0, dl0);
    wait_vm0();
    barrier_keep_loads();
    if (it + 2 < n_it) issue(it + 2, q0, o0, ls0, dl0);
    step(it + 1, q1, o1, ls1, dl1);
  }
  if (it < n_it) {
    wait_vm0();
    barrier_keep_loads();
    step(it, q0, o0, ls0, dl0);
  }

  if (has_keys && key < w.k1) {
    __bf16* kb = (__bf16*)p.dk + (int64_t)key * p.dk_st + (int64_t)w.g * p.dk_sh + 4 * h2;
    __bf16* vb = (__bf16*)p.dv + (int64_t)key * p.dv_st + (int64_t)w.g * p.dv_sh + 4 * h2;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 rk, rv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rk[e] = dk[d][4 * i + e] * f.scale;
          rv[e] = dv[d][4 * i + e];
        }
        *(bf16x4*)(kb + 32 * d + 8 * i) = cvt_bf16x4(rk);
        *(bf16x4*)(vb + 32 * d + 8 * i) = cvt_bf16x4(rv);
      }
  }
}

}  // namespace

void dense_bwd_plan(DenseBwdParams& p) {
  dense_fwd_plan(p.f);
  p.kv_n_vtiles = p.f.T / kTK + p.f.n_docs + 2;
  p.kv_n_work = p.f.Hkv * p.kv_n_vtiles;
}

hipError_t dense_bwd_launch(const DenseBwdParams& p, int D, hipStream_t stream) {
  if (D != kBD) return hipErrorInvalidValue;
  if (p.f.T <= 0) return hipSuccess;
  const int64_t rows = (int64_t)p.f.T * p.f.Hq;
  const int64_t rows_per_block = (kThreads / 64) * (64 / (kBD / 8));
  int64_t gd = (rows + rows_per_block - 1) / rows_per_block;
  gd = gd > 8192 ? 8192 : gd;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)gd), dim3(kThreads), 0, stream, p);
  if (p.f.sinks != nullptr && p.dsinks != nullptr)
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3((unsigned)p.f.Hq), dim3(kThreads), 0, stream, p);
  const int64_t gq = dense_fwd_grid(p.f);
  if (gq > 0) hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)gq), dim3(kThreads), 0, stream, p);
  const int64_t gk = ((int64_t)p.kv_n_work + kXcds - 1) / kXcds * kXcds;
  if (gk > 0) hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)gk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace swa
