// Packed variable-length causal / sliding-window GQA attention backward for gfx950 (bf16,
// head_dim 64 or 128).
//
// Operation: the gradients of a loss through `out` of the forward in dense_fwd.hip
// (MuseMagiPlan.attention on the muse_spark magi_cp page, FlintMagiPlan.attention on the
// flint magi page, GQA of MuseGlimmerAttention on the muse_glimmer model page).  The pages
// print no backward and return no log-sum-exp; recomputing the probabilities from the
// forward's exported `lse` (sink included) is this library's own design:
//   P_ij = exp(scale q_i.k_j - lse_i)     delta_i = <dout_i, out_i>
//   dS_ij = P_ij (<dout_i, v_j> - delta_i)
//   dq_i = scale sum_j dS_ij k_j ;  dk_j = scale sum_{i,h} dS_ij q_i ;  dv_j = sum_{i,h} P_ij dout_i
//   dsink_h = -sum_i exp(sink_h - lse_i) delta_i
//
// Design (MFMA 32x32x16 bf16, fp32 accumulation, no atomics, no scratch beyond `delta`):
//  * dsink: two deterministic reduction passes (per 256-token chunk across heads, then per head).
//  * dq kernel (query-parallel): the forward's workgroup decomposition (per document, 128
//    query columns = tokens x folded GQA heads, XCD-aware placement).  Per 64-key tile:
//    S^T = K Q^T and dP^T = V dO^T with q and dout of the lane's column in registers, so
//    P^T = exp2(S^T c2 - lse_col) and dS^T = P^T (dP^T - delta_col) are lane-local; then
//    dQ^T += K^T dS^T with the K^T operand read transposed from LDS (ds_read_b64_tr_b16).
//    Its prologue computes delta = <dout, out> of the lane's column (the two half-waves each
//    hold half the coordinates) and writes it for the dk/dv and dsink kernels, which run after;
//    its dq tile leaves through the idle LDS buffer pair so every store writes whole rows.
//  * dk/dv kernel (key-parallel): a workgroup owns the keys of one KV head (head_dim 64: 64 keys,
//    32 per wave of 2 waves with 32x32 MFMAs; head_dim 128: 128 keys, 16 per wave of 8 waves with
//    16x16x32 MFMAs;
//    their K and V rows held in registers) and walks the 64-query tiles of every query head
//    of the group that can see them.  S = Q K^T and dP = dO V^T (queries = M, keys = N),
//    so the lane of a key column holds P and dS in the B-operand layout of
//    dV^T += dO^T P and dK^T += Q^T dS, whose A operands are transposed LDS reads of the
//    staged Q and dO tiles.  All heads of the group accumulate in registers: GQA needs no
//    reduction pass.
//  * K tiles (dq kernel) and Q / dO tiles (dk/dv kernel) are read both row-wise and
//    transposed, so their 16-byte units are swizzled with rt_key(r), which keeps both access
//    patterns free of bank conflicts: for 256-byte rows (D = 128) row bits 0-1 go to unit bits
//    2-3 and row bits 2-3 to unit bits 0-1; for 128-byte rows (D = 64, two rows per bank line)
//    m = (r >> 1) & 7 goes to m ^ ((m & 1) << 2).  V tiles (dq kernel) are only read row-wise.
//  * Tiles travel HBM -> LDS by buffer_load ... lds into two statically named buffers per
//    operand (loop unrolled by two): the next tile is in flight while this one is used.
#include <climits>
#include <type_traits>

#include "dense_common.h"

namespace swa {
namespace {

constexpr int kDkdvWaves64 = 2;    // waves of a head_dim-64 dk/dv workgroup (32 keys each)
constexpr int kBwdAhead = 8;    // dk/dv operand fragments read this many MFMAs ahead (head_dim 128)
constexpr int kBwdAhead64 = 4;  // the same for head_dim 64
constexpr int kDqOcc64 = 3;     // head_dim 64 dq: 3 waves / SIMD (168 VGPRs, 2 dwords spilled outside the loop)

template <int D>
struct Bw {
  static constexpr int U = D / 8;              // 16-byte units per row
  static constexpr int QF = D / 16;            // k-steps of 16 coordinates
  static constexpr int DB = D / 32;            // 32-row output blocks
  static constexpr int TileUnits = 64 * U;     // a 64-row tile
  static constexpr int NS = 2 * QF;            // MFMAs of S (or dP) for two 32-row blocks
  static constexpr int NV = 4 * DB;            // MFMAs of dV^T (or dK^T) over 64 rows
  static constexpr int HiXor = D == 128 ? 2 : 4;  // rt_key(r + 8) = rt_key(r) ^ HiXor for r < 8
};
template <int D>
__device__ __forceinline__ int rt_key(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r >> 1) & 7) ^ (((r >> 1) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int row_key(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}

// The lane's byte offset inside a 64-unit block of a full 64-row tile.  Transfer i of wave w
// covers rows (4 i + w) R + lane / U; the swizzle key depends only on the low bits of the row
// that the wave and the lane fix (R = 64 / U rows per block), so the offset is the same for
// every transfer and every tile, and the block's row offset goes into soffset.
template <int D, bool RT>
__device__ __forceinline__ uint32_t rows64_lane_off(int64_t st, int lane, int wave) {
  constexpr int U = Bw<D>::U, R = 64 / U;
  const int lr = lane / U, lp = lane % U;
  const int cu = lp ^ (RT ? rt_key<D>(wave * R + lr) : row_key<D>(wave * R + lr));
  return (uint32_t)lr * ((uint32_t)st * 2u) + (uint32_t)cu * 16u;
}

// 64 rows (r0 .. r0 + 63, clamped to r_last >= r0) of D bf16 each into buf; logical unit u of
// row r lands at physical unit u ^ key(r).  U / NW transfers of 64 units per wave (NW waves
// share the tile).  A full tile takes the lane offset from rows64_lane_off and costs no VALU; a
// clamped (last) tile recomputes every row.
template <int D, bool RT, int NW = 4>
__device__ __forceinline__ void dma_rows64(const __bf16* base, int64_t st, int r0, int r_last, u32x4* buf, int wave,
                                           int lane_in, uint32_t lane_off) {
  constexpr int U = Bw<D>::U, R = 64 / U;  // rows per 64-unit block
  // the lane offset is the same for every transfer when the key's row bits stay within the
  // wave's block of rows: true for NW = 4, and for NW = 2 at head_dim 64 (checked on the host)
  static_assert(NW == 4 || (NW == 2 && D == 64), "lane offset not invariant");
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)r0 * st), (short)0, -1, kBufferWord3);
  const uint32_t stb = (uint32_t)st * 2u;
  const int lim = r_last - r0;
  if (lim >= 63) {
#pragma unroll
    for (int i = 0; i < U / NW; ++i) {
      const int blk = i * NW + wave;
      u32x4* dst = buf + __builtin_amdgcn_readfirstlane(blk * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, lane_off,
                                               __builtin_amdgcn_readfirstlane((uint32_t)(blk * R) * stb), 0, 0);
    }
    return;
  }
  const int lane = opaque(lane_in);
  const int lr = lane / U, lp = lane % U;
#pragma unroll
  for (int i = 0; i < U / NW; ++i) {
    const int blk = i * NW + wave;  // wave-uniform block of R rows
    const int r = blk * R + lr;
    const int cu = lp ^ (RT ? rt_key<D>(r) : row_key<D>(r));
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
// unit (2 s + h2) ^ key(n) = (h2 ^ key(n)) ^ 2 s, i.e. raddr ^ 32 s with
// raddr = n * U * 16 + ((h2 ^ key(n)) << 4).
template <int D>
__device__ __forceinline__ const bf16x8& row_frag(const u32x4* buf, int raddr, int blk, int s) {
  return *(const bf16x8*)((const char*)buf + ((raddr ^ (32 * s)) + blk * 32 * Bw<D>::U * 16));
}

// Transposed A-operand reads (ds_read_b64_tr_b16) of an rt_key tile: lane j of a 16-lane group
// reads rows r0 = 4 h2 + j / 4 (+ 16 ks) and r0 + 8, 8-byte half (j & 1) of logical unit
// 4 d + 2 dh + ((j & 3) >> 1).
template <int D>
struct TrOffsets {
  int lo[Bw<D>::DB], hi[Bw<D>::DB];
};
template <int D>
__device__ __forceinline__ TrOffsets<D> tr_offsets(int lane) {
  using B = Bw<D>;
  const int j16 = lane & 15, dh = (lane >> 4) & 1, h2 = lane >> 5;
  const int r0 = 4 * h2 + (j16 >> 2);
  const int k0 = rt_key<D>(r0);
  const int sub = (j16 & 3) >> 1;
  const int half = (j16 & 1) * 4;
  TrOffsets<D> t;
#pragma unroll
  for (int d = 0; d < B::DB; ++d) {
    const int u = 4 * d + 2 * dh + sub;
    t.lo[d] = ((r0 * B::U + (u ^ k0)) * 8 + half) * 2;
    t.hi[d] = (((r0 + 8) * B::U + (u ^ k0 ^ B::HiXor)) * 8 + half) * 2;
  }
  return t;
}
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const u32x4* buf, const TrOffsets<D>& t, int ks, int d) {
  const char* p = (const char*)buf + ks * 16 * Bw<D>::U * 16;
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
// dsink
// ======================================================================================
// dsink_h = -sum_t exp(sink_h - lse[t, h]) delta[t, h]; rows with lse = -inf (padding) add 0.
// Two deterministic passes after the dk/dv kernel (which is the last reader of delta):
// one workgroup per 256-token chunk reads the chunk's rows across the heads (coalesced) and
// leaves each head's partial sum in the chunk's first delta row; one workgroup per head then
// adds the chunk partials in a fixed order.
constexpr int kSinkChunk = 256;
__global__ __launch_bounds__(kThreads) void bwd_dsink_partial_kernel(DenseBwdParams p) {
  const int Hq = p.f.Hq, T = p.f.T;
  const int t0 = blockIdx.x * kSinkChunk, t1 = min(t0 + kSinkChunk, T);
  for (int h = threadIdx.x; h < Hq; h += kThreads) {
    const float s = p.f.sinks[h];
    float acc = 0.f;
    for (int t = t0; t < t1; t += 16) {
      float l[16], d[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const bool ok = t + u < t1;
        l[u] = ok ? p.f.lse[(int64_t)(t + u) * Hq + h] : -INFINITY;
        d[u] = ok ? p.delta[(int64_t)(t + u) * Hq + h] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += l[u] != -INFINITY ? __expf(s - l[u]) * d[u] : 0.f;
    }
    p.delta[(int64_t)t0 * Hq + h] = acc;  // this thread alone read column h of the chunk
  }
}

__global__ __launch_bounds__(kThreads) void bwd_dsink_reduce_kernel(DenseBwdParams p) {
  __shared__ float part[kThreads / 64];
  const int h = blockIdx.x;
  const int n_chunks = (p.f.T + kSinkChunk - 1) / kSinkChunk;
  float acc = 0.f;
  for (int c = threadIdx.x; c < n_chunks; c += kThreads) acc += p.delta[(int64_t)c * kSinkChunk * p.f.Hq + h];
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
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? kDqOcc64 : 2) void bwd_dq_kernel(DenseBwdParams p) {
  using B = Bw<D>;
  __shared__ u32x4 k0[B::TileUnits];
  __shared__ u32x4 k1[B::TileUnits];
  __shared__ u32x4 v0[B::TileUnits];
  __shared__ u32x4 v1[B::TileUnits];
  const DenseFwdParams& f = p.f;

  Tile w;
  if (!decode_tile<false>(f, w)) return;
  if (w.padding) {  // tokens outside every document receive no gradient
    const int n_rows = (w.t_end - w.t0) * w.HB;
    for (int idx = threadIdx.x; idx < n_rows * B::U; idx += kThreads) {
      const int row = idx / B::U, cu = idx - row * B::U;
      const int t = w.t0 + row / w.HB, h = w.h0 + row % w.HB;
      *(u32x4*)((__bf16*)p.dq + (int64_t)t * p.dq_st + (int64_t)h * p.dq_sh + cu * 8) = u32x4{0, 0, 0, 0};
      if (cu == 0) p.delta[(int64_t)t * f.Hq + h] = 0.f;
    }
    return;
  }
  const Cols c = make_cols(f, w);
  const int tq = min(c.tq, w.t_end - 1);
  bf16x8 qf[B::QF], gf[B::QF];
  {
    const __bf16* qb = (const __bf16*)f.q + (int64_t)tq * f.q_st + (int64_t)c.hq * f.q_sh + 8 * c.h2;
    const __bf16* gb = (const __bf16*)p.dout + (int64_t)tq * p.do_st + (int64_t)c.hq * p.do_sh + 8 * c.h2;
#pragma unroll
    for (int s = 0; s < B::QF; ++s) {
      qf[s] = *(const bf16x8*)(qb + 16 * s);
      gf[s] = *(const bf16x8*)(gb + 16 * s);
    }
  }
  float dl = 0.f;  // delta = <dout, out> of this column: half the coordinates per half-wave
  {
    const __bf16* ob = (const __bf16*)f.out + (int64_t)tq * f.o_st + (int64_t)c.hq * f.o_sh + 8 * c.h2;
#pragma unroll
    for (int s = 0; s < B::QF; ++s) {
      const bf16x8 o8 = *(const bf16x8*)(ob + 16 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = __builtin_fmaf((float)o8[e], (float)gf[s][e], dl);
    }
    dl = half_swap_sum(dl);
    if (c.tq < w.t_end && c.h2 == 0) p.delta[(int64_t)c.tq * f.Hq + c.hq] = dl;
  }
  const float lse2 = f.lse[(int64_t)tq * f.Hq + c.hq] * kLog2e;
  const float c2 = f.c2;
  const __bf16* kbase = (const __bf16*)f.k + (int64_t)w.g * f.k_sh;
  const __bf16* vbase = (const __bf16*)f.v + (int64_t)w.g * f.v_sh;
  const int kraddr = c.n * B::U * 16 + ((c.h2 ^ rt_key<D>(c.n)) << 4);
  const int vraddr = c.n * B::U * 16 + ((c.h2 ^ row_key<D>(c.n)) << 4);
  const TrOffsets<D> to = tr_offsets<D>(c.lane);

  f32x16 acc[B::DB];
#pragma unroll
  for (int d = 0; d < B::DB; ++d) acc[d] = f32x16{};
  const int nt = c.n_tiles;
  const int last = c.k_hi - 1;

  // NB = 1: the tile's second 32-key block starts after every token of the wave, so the mask
  // would make its probabilities and dS exactly zero: its S, dP and dQ k-steps are skipped.
  // head_dim 64 only (a sixth of the blocks of the window-128 workload; at head_dim 128 the
  // second copy of the tile spilled 26 dwords for about 3 % of the causal work)
  auto tile_blocks = [&](auto nb, const u32x4* kb_, const u32x4* vb_, int kb) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb)::value;
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      sc[blk] = f32x16{};
      dp[blk] = f32x16{};
#pragma unroll
      for (int s = 0; s < B::QF; ++s) sc[blk] = mfma_bf16_32x32x16(row_frag<D>(kb_, kraddr, blk, s), qf[s], sc[blk]);
#pragma unroll
      for (int s = 0; s < B::QF; ++s) dp[blk] = mfma_bf16_32x32x16(row_frag<D>(vb_, vraddr, blk, s), gf[s], dp[blk]);
    }
    if (tile_needs_mask(c, kb)) mask_tile<NB>(sc, kb, c);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float pr = fast_exp2(__builtin_fmaf(sc[blk][a], c2, -lse2));
        sc[blk][a] = pr * (dp[blk][a] - dl);
      }
#pragma unroll
    for (int ks = 0; ks < 2 * NB; ++ks) {
      const bf16x8 sb = pack_ks(sc, ks);
#pragma unroll
      for (int d = 0; d < B::DB; ++d) acc[d] = mfma_bf16_32x32x16(tr_frag<D>(kb_, to, ks, d), sb, acc[d]);
    }
  };
  auto tile = [&](const u32x4* kb_, const u32x4* vb_, int kb) __attribute__((always_inline)) {
    if (!tile_active(c, kb)) return;  // none of this wave's tokens sees these keys
    if (D == 64 && kb + 32 > c.tw1) tile_blocks(std::integral_constant<int, D == 64 ? 1 : 2>{}, kb_, vb_, kb);
    else tile_blocks(std::integral_constant<int, 2>{}, kb_, vb_, kb);
  };

  const uint32_t koff = rows64_lane_off<D, true>(f.k_st, c.lane, c.wave);
  const uint32_t voff = rows64_lane_off<D, false>(f.v_st, c.lane, c.wave);
  dma_rows64<D, true>(kbase, f.k_st, c.k_lo, last, k0, c.wave, c.lane, koff);
  dma_rows64<D, false>(vbase, f.v_st, c.k_lo, last, v0, c.wave, c.lane, voff);
  int j = 0;
  for (; j + 1 < nt; j += 2) {
    wait_vm0();
    barrier_keep_loads();  // tile j landed for every wave; tile j - 1 fully consumed
    dma_rows64<D, true>(kbase, f.k_st, c.k_lo + (j + 1) * kBN, last, k1, c.wave, c.lane, koff);
    dma_rows64<D, false>(vbase, f.v_st, c.k_lo + (j + 1) * kBN, last, v1, c.wave, c.lane, voff);
    tile(k0, v0, c.k_lo + j * kBN);
    wait_vm0();
    barrier_keep_loads();
    if (j + 2 < nt) {
      dma_rows64<D, true>(kbase, f.k_st, c.k_lo + (j + 2) * kBN, last, k0, c.wave, c.lane, koff);
      dma_rows64<D, false>(vbase, f.v_st, c.k_lo + (j + 2) * kBN, last, v0, c.wave, c.lane, voff);
    }
    tile(k1, v1, c.k_lo + (j + 1) * kBN);
  }
  if (j < nt) {
    wait_vm0();
    barrier_keep_loads();
    tile(k0, v0, c.k_lo + j * kBN);
  }

  // the last tile was read from buffer pair (nt - 1) & 1; every wave finished the other pair
  // before the last barrier and no transfer targets it: it holds the output images, two waves
  // per buffer
  char* img = (char*)(((nt - 1) & 1) ? (c.wave < 2 ? k0 : v0) : (c.wave < 2 ? k1 : v1)) + (c.wave & 1) * (64 * D);
  store_out_bf16<D>(p.dq, p.dq_st, p.dq_sh, w, c, f.hb_shift, f.scale, acc, img);
}

// ======================================================================================
// dk, dv: key-parallel
// ======================================================================================
struct KeyTile {
  int g, k0, k1, seg_start, seg_end;
  bool padding;
};

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Rank r of the head's key tiles, heaviest first, when the segments fit a wave's lanes
// (n_docs + 2 <= 64).  The query tiles a key tile of TK keys walks are
// ceil(min(R, TK - 1 + W) / 64) (R = keys from the tile to the document end; no cap without a
// window), non-increasing along a document, so the tiles of a document with at least x query
// tiles are its first min(n_tiles, ceil((len - 64 (x - 1)) / TK)).  A binary search on x over the
// lane-wise counts finds the weight of rank r; ties go in document order.  Padding segments come
// last.
__device__ __forceinline__ bool decode_heavy_first(const DenseFwdParams& f, int r, int TK, KeyTile& w) {
  const int lane = threadIdx.x & 63;
  const int nseg = f.n_docs + 2;
  const bool seg_ok = lane < nseg;
  const int st = seg_ok ? seg_bound(f, lane) : 0;
  const int en = seg_ok ? seg_bound(f, lane + 1) : 0;
  const int len = en - st;
  const int nt = (len + TK - 1) / TK;
  const bool real = seg_ok && lane >= 1 && lane <= f.n_docs;
  const int cap = f.window ? TK - 1 + f.window : INT_MAX;
  auto count_ge = [&](int x) -> int {
    const int need = 64 * (x - 1);
    if (!real || cap <= need || len <= need) return 0;
    return min(nt, (len - need + TK - 1) / TK);
  };
  const int n_real = __builtin_amdgcn_readfirstlane(wave_sum(real ? nt : 0));
  int seg, t;
  if (r < n_real) {
    int lo = 1, hi = f.T / 64 + 2;  // count_ge(lo) > r >= count_ge(hi) = 0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(wave_sum(count_ge(mid))) > r) lo = mid; else hi = mid;
    }
    const int above = count_ge(lo + 1);
    const int j = r - __builtin_amdgcn_readfirstlane(wave_sum(above));  // rank among tiles of weight lo
    const int eq = count_ge(lo) - above;
    int incl = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const bool mine = eq > 0 && j >= incl - eq && j < incl;
    const uint64_t owner = __builtin_amdgcn_ballot_w64(mine);
    if (owner == 0) return false;  // unreachable: rank r always has an owner
    seg = __builtin_amdgcn_readfirstlane(__builtin_ctzll(owner));
    t = __builtin_amdgcn_readlane(above, seg) + (j - (__builtin_amdgcn_readlane(incl, seg) -
                                                      __builtin_amdgcn_readlane(eq, seg)));
    w.padding = false;
  } else {
    const int rp = r - n_real;
    const int nt0 = __builtin_amdgcn_readlane(nt, 0), ntn = __builtin_amdgcn_readlane(nt, nseg - 1);
    if (rp < nt0) {
      seg = 0;
      t = rp;
    } else if (rp - nt0 < ntn) {
      seg = nseg - 1;
      t = rp - nt0;
    } else {
      return false;
    }
    w.padding = true;
  }
  w.seg_start = __builtin_amdgcn_readlane(st, seg);
  w.seg_end = __builtin_amdgcn_readlane(en, seg);
  w.k0 = w.seg_start + t * TK;
  w.k1 = min(w.k0 + TK, w.seg_end);
  return true;
}

// blockIdx -> (KV head, key tile of a segment); each KV head's tiles on one XCD, heaviest
// first (the tail of a launch is then made of light tiles).  With more than 62 documents: each
// document's tiles first-first (under a causal mask the first keys are seen by the most queries).
// Workgroups reach the XCDs round-robin (x = blockIdx % 8, j = blockIdx / 8 is the order within
// an XCD).  A KV head's tiles stay on the XCDs that hold its K/V in L2.  In heavy-first order
// (full causal): with Hkv a multiple of 8 each XCD owns whole heads; with Hkv dividing 8 the
// 8 / Hkv XCDs of a head deal its ranks round robin (so each gets the same mix of heavy and light
// tiles).  Otherwise contiguous ranges (consecutive tiles of a document share an L2, which is
// what windowed problems, whose tiles weigh about the same, gain most from).
__device__ __forceinline__ bool key_tile_slot(const DenseBwdParams& p, int& g, int& r) {
  const int Hkv = p.f.Hkv, VT = p.kv_n_vtiles;
  const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  if (p.kv_heavy_first && Hkv % kXcds == 0) {
    g = x + kXcds * (j / VT);
    r = j % VT;
    return g < Hkv;
  }
  if (p.kv_heavy_first && kXcds % Hkv == 0) {
    const int m = kXcds / Hkv;
    g = x % Hkv;
    r = j * m + x / Hkv;
    return r < VT;
  }
  const int L = x * (gridDim.x / kXcds) + j;
  g = L / VT;
  r = L - g * VT;
  return L < p.kv_n_work;
}

__device__ __forceinline__ bool decode_key_tile(const DenseBwdParams& p, KeyTile& w) {
  const DenseFwdParams& f = p.f;
  int v;
  if (!key_tile_slot(p, w.g, v)) return false;
  const int TK = p.kv_tile;
  if (p.kv_heavy_first) return decode_heavy_first(f, v, TK, w);
  int lo = 0, hi = f.n_docs + 2;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_bound(f, mid) / TK + mid <= v) lo = mid; else hi = mid;
  }
  w.seg_start = seg_bound(f, lo);
  w.seg_end = seg_bound(f, lo + 1);
  w.k0 = w.seg_start + (v - (w.seg_start / TK + lo)) * TK;
  if (w.k0 >= w.seg_end) return false;
  w.k1 = min(w.k0 + TK, w.seg_end);
  w.padding = (lo == 0 || lo == f.n_docs + 1);
  return true;
}

// Order in which a key tile walks its (query head, 64-query tile) pairs, chosen so that the
// workgroups running together on one XCD read the same Q / dO tiles at about the same time and
// find them in L2 (every order gives the same sums, accumulated in another order):
//  * key tiles whose queries run to the document end (every tile under a full causal mask, or
//    a window that does not cut the range): query tiles outer, from the document end down, heads
//    inner; the key tiles of a document all start at its last query tile and stop at their own
//    diagonal, so they walk the same tiles in step.  The choice depends on the tile alone, so a
//    window at least as long as the document gives bitwise the full causal result.
//  * otherwise (cut by the window): heads outer; within a head the walk is rotated so that at step
//    s every key tile reads the query tile whose index in the document is congruent to s modulo
//    the walk length; neighbouring key tiles, whose ranges overlap, then read their shared tiles
//    at the same step.
// Measured on the causal 8192-token backward: the dk/dv kernel fetched 845 MiB beyond L2 in
// document order, 340 MiB with this walk (its Q, dO, K, V, lse and delta come to 162 MiB); on the
// window-1024 one 2176 -> 1342 MiB (minimum 584).
// Step `it` of the walk visits head head(it) and query tile tile(it).  The kernels advance a
// WalkPos one step at a time (compares instead of the divisions, which cost about a hundred
// scalar instructions per step); the two forms agree at every step.
struct WalkPos {
  int head, tile, s;  // s: position in the inner loop of the rotated walk
};
struct QueryWalk {
  bool down;  // from the document end, heads inner
  int rot;    // rotation of the sliding-window walk
  __device__ __forceinline__ int head(int it, int G, int n_qt) const { return down ? it % G : it / n_qt; }
  __device__ __forceinline__ int tile(int it, int G, int n_qt) const {
    return down ? n_qt - 1 - it / G : (it % n_qt + rot) % n_qt;
  }
  __device__ __forceinline__ WalkPos first(int n_qt) const {
    return down ? WalkPos{0, n_qt - 1, 0} : WalkPos{0, rot >= n_qt ? rot - n_qt : rot, 0};
  }
  __device__ __forceinline__ WalkPos next(const WalkPos& p, int G, int n_qt) const {
    if (down) return p.head + 1 == G ? WalkPos{0, p.tile - 1, 0} : WalkPos{p.head + 1, p.tile, 0};
    const bool wrap = p.s + 1 == n_qt;
    const int s1 = wrap ? 0 : p.s + 1;
    return WalkPos{wrap ? p.head + 1 : p.head, s1 + rot >= n_qt ? s1 + rot - n_qt : s1 + rot, s1};
  }
};
__device__ __forceinline__ QueryWalk query_walk(const KeyTile& w, int i_hi, int n_qt) {
  QueryWalk q;
  q.down = i_hi == w.seg_end;
  q.rot = n_qt - ((w.k0 - w.seg_start) / 64) % n_qt;  // in [1, n_qt]: (s + rot) % n_qt is s - first tile mod n_qt
  return q;
}

// One 64-query x 32-key tile of the dk/dv kernel as two fenced instruction streams (the
// emitted order is the program order; operand fragments are read kAhead MFMAs ahead):
//  1. S = Q K^T and dP = dO V^T (32 MFMAs, the two query blocks alternating); the
//     probabilities P = exp2(S c2 - lse log2 e) of the tile run in the dP slots.
//  2. dV^T += dO^T P and dK^T += Q^T dS (32 MFMAs); dS = P (dP - delta) runs in the dV slots.
// Rows of the tile are queries; `qoff` = first query - this lane's key, `eoff` = document end -
// key (the mask of MASK tiles: 0 <= query - key, query < end, and query - key < W when W > 0).
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_tile(const u32x4* qb, const u32x4* ob, const float* lb, const float* db,
                                          const bf16x8 (&kf)[Bw<D>::QF], const bf16x8 (&vf)[Bw<D>::QF], int raddr,
                                          const TrOffsets<D>& to, float c2, f32x16 (&dk)[Bw<D>::DB],
                                          f32x16 (&dv)[Bw<D>::DB], int qoff, int eoff, int W, int h2) {
  using B = Bw<D>;
  constexpr int NS = B::NS, NV = B::NV, NF = 2 * NS + 2 * NV;
  constexpr int EPS = 32 / NS;  // probabilities per dP slot
  constexpr int DPS = 32 / NV;  // dS elements per dV slot
  constexpr int kAhead = D == 64 ? kBwdAhead64 : kBwdAhead;
  static_assert(32 % NS == 0 && 32 % NV == 0 && NS >= 8, "slot shares");
  // MASK: query - key = d is allowed iff 0 <= d < eoff and d < W (W > 0): one unsigned compare
  // against lim (negative d wraps above it); a lane with no valid key (eoff <= 0) allows nothing
  const unsigned lim = (unsigned)max(0, W ? min(eoff, W) : eoff);
  bf16x8 frag[NF];
  auto read = [&](int f) {
    if (f < 2 * NS) {  // S (f < NS) or dP: query block f & 1, k-step (f % NS) >> 1
      frag[f] = row_frag<D>(f < NS ? qb : ob, raddr, f & 1, (f % NS) >> 1);
    } else {           // dV (first NV) or dK: k-step (i / DB) of 4, output block i % DB
      const int i = f - 2 * NS;
      frag[f] = tr_frag<D>(i < NV ? ob : qb, to, (i % NV) / B::DB, i % B::DB);
    }
  };
  f32x4 l4[8], d4[8];  // lse and delta of query rows 32 b + 8 j + 4 h2 + (0..3), index 4 b + j
  f32x16 sc[2], dp[2];
  bf16x8 pb[4], sb[4];
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): nothing older in flight, later waits count exactly
  // rows of group j: 32 (j >> 2) + 8 (j & 3) + 4 h2 .. + 3.  Slots are numbered over the four
  // streams (S, dP, dV, dK); lse group j is used in dP slot 4 j / EPS, delta group j in dV slot
  // 4 j / DPS, and each is read two slots before its use.
  auto rows = [&](int j) { return 32 * (j >> 2) + 8 * (j & 3) + 4 * h2; };
  auto stage_rows = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (slot == NS + 4 * j / EPS - 2) l4[j] = *(const f32x4*)(lb + rows(j));
      if (slot == 2 * NS + 4 * j / DPS - 2) d4[j] = *(const f32x4*)(db + rows(j));
    }
  };
#pragma unroll
  for (int f = 0; f < kAhead; ++f) read(f);
  __builtin_amdgcn_sched_barrier(0);
  sc[0] = sc[1] = dp[0] = dp[1] = f32x16{};
  // stream 1a: S (NS MFMAs, the two query blocks alternating)
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    sc[i & 1] = mfma_bf16_32x32x16(frag[i], kf[i >> 1], sc[i & 1]);
    read(i + kAhead);
    stage_rows(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  // stream 1b: dP (NS MFMAs) with the probabilities of S, EPS per slot
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    dp[i & 1] = mfma_bf16_32x32x16(frag[NS + i], vf[i >> 1], dp[i & 1]);
    read(NS + i + kAhead);
#pragma unroll
    for (int e = 0; e < EPS; ++e) {
      const int x = EPS * i + e;  // element x of the tile's 32: block x >> 4, accumulator x & 15
      const int bb = x >> 4, a = x & 15;
      float pr = fast_exp2(__builtin_fmaf(sc[bb][a], c2, l4[x >> 2][a & 3] * -kLog2e));
      if constexpr (MASK) {
        const int d = qoff + 32 * bb + 8 * (a >> 2) + 4 * h2 + (a & 3);  // query - key
        pr = (unsigned)d < lim ? pr : 0.f;
      }
      sc[bb][a] = pr;
      asm volatile("" : "+v"(sc[bb][a]));  // this slot's probabilities stay in this slot
      if ((x & 7) == 7) pb[x >> 3] = pack_ks(sc, x >> 3);
    }
    stage_rows(NS + i);
    __builtin_amdgcn_sched_barrier(0);
  }
  // stream 2a: dV^T += dO^T P (NV MFMAs) with dS, DPS elements per slot
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    dv[i % B::DB] = mfma_bf16_32x32x16(frag[2 * NS + i], pb[i / B::DB], dv[i % B::DB]);
    read(2 * NS + i + kAhead);
#pragma unroll
    for (int e = 0; e < DPS; ++e) {
      const int x = DPS * i + e;
      const int bb = x >> 4, a = x & 15;
      dp[bb][a] = sc[bb][a] * (dp[bb][a] - d4[x >> 2][a & 3]);
      asm volatile("" : "+v"(dp[bb][a]));
      if ((x & 7) == 7) sb[x >> 3] = pack_ks(dp, x >> 3);
    }
    stage_rows(2 * NS + i);
    __builtin_amdgcn_sched_barrier(0);
  }
  // stream 2b: dK^T += Q^T dS (NV MFMAs)
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    dk[i % B::DB] = mfma_bf16_32x32x16(frag[2 * NS + NV + i], sb[i / B::DB], dk[i % B::DB]);
    if (2 * NS + NV + i + kAhead < NF) read(2 * NS + NV + i + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

template <int D>
__global__ __launch_bounds__(64 * kDkdvWaves64, 2) void bwd_dkdv_kernel(DenseBwdParams p) {
  static_assert(D == 64, "head_dim 128 uses bwd_dkdv16_kernel");
  constexpr int NW = kDkdvWaves64;
  using B = Bw<D>;
  __shared__ u32x4 q0[B::TileUnits];
  __shared__ u32x4 q1[B::TileUnits];
  __shared__ u32x4 o0[B::TileUnits];
  __shared__ u32x4 o1[B::TileUnits];
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
    for (int idx = threadIdx.x; idx < n_rows * B::U; idx += 64 * NW) {
      const int row = idx / B::U, cu = idx - row * B::U;
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
  bf16x8 kf[B::QF], vf[B::QF];
  {
    const int kr = min(key, w.k1 - 1);
    const __bf16* kb = (const __bf16*)f.k + (int64_t)kr * f.k_st + (int64_t)w.g * f.k_sh + 8 * h2;
    const __bf16* vb = (const __bf16*)f.v + (int64_t)kr * f.v_st + (int64_t)w.g * f.v_sh + 8 * h2;
#pragma unroll
    for (int s = 0; s < B::QF; ++s) {
      kf[s] = *(const bf16x8*)(kb + 16 * s);
      vf[s] = *(const bf16x8*)(vb + 16 * s);
    }
  }
  f32x16 dk[B::DB], dv[B::DB];
#pragma unroll
  for (int d = 0; d < B::DB; ++d) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }
  // queries that see these keys: [k0, i_hi); 64-query tiles for every head of the group
  const int i_hi = W ? min(e_doc, w.k1 - 1 + W) : e_doc;
  const int n_qt = (i_hi - w.k0 + 63) / 64;
  const int n_it = f.G * n_qt;
  const QueryWalk walk = query_walk(w, i_hi, n_qt);
  const int raddr = n * B::U * 16 + ((h2 ^ rt_key<D>(n)) << 4);
  const TrOffsets<D> to = tr_offsets<D>(lane);
  const float c2 = f.c2;

  const uint32_t qoff_l = rows64_lane_off<D, true>(f.q_st, lane, wave);
  const uint32_t ooff_l = rows64_lane_off<D, true>(p.do_st, lane, wave);
  auto issue = [&](const WalkPos& wp, u32x4* qb, u32x4* ob, float* lb, float* db) {
    const int h = w.g * f.G + wp.head;
    const int i0 = w.k0 + 64 * wp.tile;
    dma_rows64<D, true, NW>((const __bf16*)f.q + (int64_t)h * f.q_sh, f.q_st, i0, i_hi - 1, qb, wave, lane, qoff_l);
    dma_rows64<D, true, NW>((const __bf16*)p.dout + (int64_t)h * p.do_sh, p.do_st, i0, i_hi - 1, ob, wave, lane,
                            ooff_l);
    if (wave == 0) dma_rowvals(f.lse, f.Hq, h, i0, i_hi - 1, lb, lane);
    if (wave == 1) dma_rowvals(p.delta, f.Hq, h, i0, i_hi - 1, db, lane);
  };
  auto step = [&](const WalkPos& wp, const u32x4* qb, const u32x4* ob, const float* lb, const float* db) {
    const int i0 = w.k0 + 64 * wp.tile;
    // wave-uniform: skip tiles none of whose queries sees this wave's keys
    if (!has_keys || i0 + 63 < kw0 || (W != 0 && i0 > kw0 + 31 + W - 1)) return;
    const bool need_mask = !(i0 >= kw0 + 31 && i0 + 63 < e_doc && (W == 0 || i0 + 63 - kw0 < W));
    if (need_mask)
      dkdv_tile<D, true>(qb, ob, lb, db, kf, vf, raddr, to, c2, dk, dv, i0 - key, e_doc - key, W, h2);
    else
      dkdv_tile<D, false>(qb, ob, lb, db, kf, vf, raddr, to, c2, dk, dv, i0 - key, e_doc - key, W, h2);
  };

  WalkPos p0 = walk.first(n_qt);
  issue(p0, q0, o0, ls0, dl0);
  int it = 0;
  for (; it + 1 < n_it; it += 2) {
    const WalkPos p1 = walk.next(p0, f.G, n_qt);
    wait_vm0();
    barrier_keep_loads();  // tile it landed for every wave; tile it - 1 fully consumed
    issue(p1, q1, o1, ls1, dl1);
    step(p0, q0, o0, ls0, dl0);
    const WalkPos p2 = walk.next(p1, f.G, n_qt);
    wait_vm0();
    barrier_keep_loads();
    if (it + 2 < n_it) issue(p2, q0, o0, ls0, dl0);
    step(p1, q1, o1, ls1, dl1);
    p0 = p2;
  }
  if (it < n_it) {
    wait_vm0();
    barrier_keep_loads();
    step(p0, q0, o0, ls0, dl0);
  }

  if (has_keys && key < w.k1) {
    __bf16* kb = (__bf16*)p.dk + (int64_t)key * p.dk_st + (int64_t)w.g * p.dk_sh + 4 * h2;
    __bf16* vb = (__bf16*)p.dv + (int64_t)key * p.dv_st + (int64_t)w.g * p.dv_sh + 4 * h2;
#pragma unroll
    for (int d = 0; d < B::DB; ++d)
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

// --------------------------------------------------------------------------------------
// dk/dv for head_dim 128 with v_mfma_f32_16x16x32_bf16: 8 waves x 16 keys per workgroup.
// Per wave: 2 x 32 accumulators, 32 registers of K/V rows, 2 x 16 of S/dP, so two waves fit a
// SIMD (the 32-key variant above needs one SIMD per wave).  16x16x32 operands: A[l % 16][8 (l / 16)
// + e], B[8 (l / 16) + e][l % 16], C[4 (l / 16) + a][l % 16].  The lane of key column n = l % 16
// and group g = l / 16 holds S and dP for query rows 16 b + 4 g + a of the 64-query tile (b, a <
// 4); k-step s of the dV / dK products takes rows 32 s + 4 g + e (e < 4) and 32 s + 16 + 4 g + e - 4
// (e >= 4), which are exactly the lane's values of blocks 2 s and 2 s + 1, and the matching
// transposed A operand reads column 16 m + l % 16 of those rows (ds_read_b64_tr_b16: supplier lane
// j of a 16-lane group gives row R + j / 4, columns 16 m + 4 (j % 4) .. + 3).
constexpr int kT16 = 512;

// Swizzle of the Q / dO tiles of this kernel: row bits 0-2 to unit bits 1-3 and row bit 3 to unit
// bits 0 and 3.  A row read takes one unit of 16 consecutive rows, a transposed read pass units
// {2 m, 2 m + 1} of 8 consecutive rows.  Being a bijection of r & 15 is not enough for the row
// reads: ds_read_b128 serves 16 lanes per cycle taken from all four 16-lane groups, and without
// the bit-3 flip rows r and r + 8 of two groups met on one unit (measured on gfx950: 8 LDS cycles
// per row read instead of 4, and half of the kernel's LDS cycles lost to bank conflicts).  With
// it, both read kinds run conflict-free (4 cycles per ds_read_b128, 2 per ds_read_b64_tr_b16).
__device__ __forceinline__ int rt16_key(int r) { return (((r & 7) << 1) | ((r >> 3) & 1)) ^ (r & 8); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 64 rows x 128 bf16 (rt_key swizzle) into buf by 8 waves: two 4-row blocks per wave
__device__ __forceinline__ uint32_t rows64_w8_lane_off(int64_t st, int lane, int wave) {
  const int lr = lane >> 4, lp = lane & 15;
  return (uint32_t)lr * ((uint32_t)st * 2u) + (uint32_t)(lp ^ rt16_key(wave * 4 + lr)) * 16u;
}
__device__ __forceinline__ void dma_rows64_w8(const __bf16* base, int64_t st, int r0, int r_last, u32x4* buf,
                                              int wave, int lane_in, uint32_t lane_off) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)r0 * st), (short)0, -1, kBufferWord3);
  const uint32_t stb = (uint32_t)st * 2u;
  const int lim = r_last - r0;
  if (lim >= 63) {  // full tile: the lane offset of rows64_w8_lane_off, the block's rows in soffset
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = i * 8 + wave;
      u32x4* dst = buf + __builtin_amdgcn_readfirstlane(blk * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, lane_off,
                                               __builtin_amdgcn_readfirstlane((uint32_t)(blk * 4) * stb), 0, 0);
    }
    return;
  }
  const int lane = opaque(lane_in);
  const int lr = lane >> 4, lp = lane & 15;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = i * 8 + wave;
    const int r = blk * 4 + lr;
    const int cu = lp ^ rt16_key(r);
    u32x4* dst = buf + __builtin_amdgcn_readfirstlane(blk * 64);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, (uint32_t)min(r, lim) * stb + (uint32_t)cu * 16u,
                                             0, 0, 0);
  }
}

// One 64-query x 16-key tile as fenced streams (S, dP with the probabilities, dV with dS, dK).
template <bool MASK>
__device__ __forceinline__ void dkdv16_tile(const u32x4* qb, const u32x4* ob, const float* lb, const float* db,
                                            const bf16x8 (&kf)[4], const bf16x8 (&vf)[4], int raddr,
                                            const int (&toff)[8], float c2, f32x4 (&dk)[8], f32x4 (&dv)[8],
                                            int qoff, int eoff, int W, int g) {
  constexpr int kAhead = kBwdAhead;
  const unsigned lim = (unsigned)max(0, W ? min(eoff, W) : eoff);  // as in dkdv_tile
  bf16x8 frag[64];
  auto read = [&](int f) {
    if (f < 32) {  // S (f < 16) or dP: query block b = f & 3, k-step s = (f >> 2) & 3
      const char* t = (const char*)(f < 16 ? qb : ob);
      frag[f] = *(const bf16x8*)(t + ((raddr ^ (64 * ((f >> 2) & 3))) + 4096 * (f & 3)));
    } else {       // dV (f < 48) or dK: output block m = f & 7, k-step s = (f >> 3) & 1
      const char* t = (const char*)(f < 48 ? ob : qb) + toff[f & 7] + 8192 * ((f >> 3) & 1);
      const bf16x4 lo4 = lds_read_tr4((const __bf16*)t);
      const bf16x4 hi4 = lds_read_tr4((const __bf16*)(t + 4096));
      frag[f] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  f32x4 l4[4], d4[4];  // lse / delta of query rows 16 b + 4 g + (0..3)
  f32x4 sc[4], dp[4];
  bf16x8 pb[2], sb[2];
  // lse block b is used in dP slot 4 b, delta block b in dV slot 4 b; each read two slots before
  auto stage_rows = [&](int slot) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (slot == 16 + 4 * b - 2) l4[b] = *(const f32x4*)(lb + 16 * b + 4 * g);
      if (slot == 32 + 4 * b - 2) d4[b] = *(const f32x4*)(db + 16 * b + 4 * g);
    }
  };
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): nothing older in flight, later waits count exactly
#pragma unroll
  for (int f = 0; f < kAhead; ++f) read(f);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < 4; ++b) sc[b] = dp[b] = f32x4{};
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // S
    sc[i & 3] = mfma16(frag[i], kf[i >> 2], sc[i & 3]);
    read(i + kAhead);
    stage_rows(i);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // dP, with probability i of the lane's 16 in this slot
    dp[i & 3] = mfma16(frag[16 + i], vf[i >> 2], dp[i & 3]);
    read(16 + i + kAhead);
    const int b = i >> 2, a = i & 3;
    float pr = fast_exp2(__builtin_fmaf(sc[b][a], c2, l4[b][a] * -kLog2e));
    if constexpr (MASK) {
      const int d = qoff + 16 * b + 4 * g + a;  // query - key
      pr = (unsigned)d < lim ? pr : 0.f;
    }
    sc[b][a] = pr;
    asm volatile("" : "+v"(sc[b][a]));
    if (i == 7 || i == 15) {
      const int s = i >> 3;
      f32x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = sc[2 * s + (e >> 2)][e & 3];
      pb[s] = cvt_bf16x8(pf);
    }
    stage_rows(16 + i);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // dV, with dS element i in this slot
    dv[i & 7] = mfma16(frag[32 + i], pb[i >> 3], dv[i & 7]);
    read(32 + i + kAhead);
    const int b = i >> 2, a = i & 3;
    dp[b][a] = sc[b][a] * (dp[b][a] - d4[b][a]);
    asm volatile("" : "+v"(dp[b][a]));
    if (i == 7 || i == 15) {
      const int s = i >> 3;
      f32x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = dp[2 * s + (e >> 2)][e & 3];
      sb[s] = cvt_bf16x8(pf);
    }
    stage_rows(32 + i);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // dK
    dk[i & 7] = mfma16(frag[48 + i], sb[i >> 3], dk[i & 7]);
    if (48 + i + kAhead < 64) read(48 + i + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

__global__ __launch_bounds__(kT16, 1) void bwd_dkdv16_kernel(DenseBwdParams p) {
  constexpr int U = 16;
  __shared__ u32x4 q0[64 * U];
  __shared__ u32x4 q1[64 * U];
  __shared__ u32x4 o0[64 * U];
  __shared__ u32x4 o1[64 * U];
  __shared__ f32x4 lsv[4][16];
  float* ls0 = (float*)lsv[0];
  float* ls1 = (float*)lsv[1];
  float* dl0 = (float*)lsv[2];
  float* dl1 = (float*)lsv[3];
  const DenseFwdParams& f = p.f;

  KeyTile w;
  if (!decode_key_tile(p, w)) return;
  if (w.padding) {
    const int n_rows = w.k1 - w.k0;
    for (int idx = threadIdx.x; idx < n_rows * U; idx += kT16) {
      const int row = idx / U, cu = idx - row * U;
      const int64_t t = w.k0 + row;
      *(u32x4*)((__bf16*)p.dk + t * p.dk_st + (int64_t)w.g * p.dk_sh + cu * 8) = u32x4{0, 0, 0, 0};
      *(u32x4*)((__bf16*)p.dv + t * p.dv_st + (int64_t)w.g * p.dv_sh + cu * 8) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int W = f.window, e_doc = w.seg_end;
  const int kw0 = w.k0 + 16 * wave;  // this wave's keys kw0 .. kw0 + 15
  const bool has_keys = kw0 < w.k1;
  const int key = kw0 + n;

  bf16x8 kf[4], vf[4];  // B operands: K / V row of this lane's key, coordinates 32 s + 8 g .. + 7
  {
    const int kr = min(key, w.k1 - 1);
    const __bf16* kb = (const __bf16*)f.k + (int64_t)kr * f.k_st + (int64_t)w.g * f.k_sh + 8 * g;
    const __bf16* vb = (const __bf16*)f.v + (int64_t)kr * f.v_st + (int64_t)w.g * f.v_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[s] = *(const bf16x8*)(kb + 32 * s);
      vf[s] = *(const bf16x8*)(vb + 32 * s);
    }
  }
  f32x4 dk[8], dv[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) dk[m] = dv[m] = f32x4{};
  const int i_hi = W ? min(e_doc, w.k1 - 1 + W) : e_doc;
  const int n_qt = (i_hi - w.k0 + 63) / 64;
  const int n_it = f.G * n_qt;
  const QueryWalk walk = query_walk(w, i_hi, n_qt);
  // row reads: row 16 b + n, logical unit 4 s + g -> physical (4 s + g) ^ key(n) = (g ^ key(n)) ^ 4 s
  const int raddr = n * U * 16 + ((g ^ rt16_key(n)) << 4);
  int toff[8];  // transposed reads: supplier row 4 g + n / 4 (+ 32 s, + 16), columns 16 m + 4 (n % 4)
  {
    const int r = 4 * g + (n >> 2);
    const int key0 = rt16_key(r);  // the same for rows + 16 and + 32 s
#pragma unroll
    for (int m = 0; m < 8; ++m) toff[m] = ((r * U + ((2 * m + ((n & 3) >> 1)) ^ key0)) * 8 + (n & 1) * 4) * 2;
  }
  const float c2 = f.c2;

  const uint32_t qoff_l = rows64_w8_lane_off(f.q_st, lane, wave);
  const uint32_t ooff_l = rows64_w8_lane_off(p.do_st, lane, wave);
  auto issue = [&](const WalkPos& wp, u32x4* qb, u32x4* ob, float* lb, float* db) {
    const int h = w.g * f.G + wp.head;
    const int i0 = w.k0 + 64 * wp.tile;
    dma_rows64_w8((const __bf16*)f.q + (int64_t)h * f.q_sh, f.q_st, i0, i_hi - 1, qb, wave, lane, qoff_l);
    dma_rows64_w8((const __bf16*)p.dout + (int64_t)h * p.do_sh, p.do_st, i0, i_hi - 1, ob, wave, lane, ooff_l);
    if (wave == 0) dma_rowvals(f.lse, f.Hq, h, i0, i_hi - 1, lb, lane);
    if (wave == 1) dma_rowvals(p.delta, f.Hq, h, i0, i_hi - 1, db, lane);
  };
  auto step = [&](const WalkPos& wp, const u32x4* qb, const u32x4* ob, const float* lb, const float* db) {
    const int i0 = w.k0 + 64 * wp.tile;
    if (!has_keys || i0 + 63 < kw0 || (W != 0 && i0 > kw0 + 15 + W - 1)) return;
    const bool need_mask = !(i0 >= kw0 + 15 && i0 + 63 < e_doc && (W == 0 || i0 + 63 - kw0 < W));
    if (need_mask)
      dkdv16_tile<true>(qb, ob, lb, db, kf, vf, raddr, toff, c2, dk, dv, i0 - key, e_doc - key, W, g);
    else
      dkdv16_tile<false>(qb, ob, lb, db, kf, vf, raddr, toff, c2, dk, dv, i0 - key, e_doc - key, W, g);
  };

  WalkPos p0 = walk.first(n_qt);
  issue(p0, q0, o0, ls0, dl0);
  int it = 0;
  for (; it + 1 < n_it; it += 2) {
    const WalkPos p1 = walk.next(p0, f.G, n_qt);
    wait_vm0();
    barrier_keep_loads();
    issue(p1, q1, o1, ls1, dl1);
    step(p0, q0, o0, ls0, dl0);
    const WalkPos p2 = walk.next(p1, f.G, n_qt);
    wait_vm0();
    barrier_keep_loads();
    if (it + 2 < n_it) issue(p2, q0, o0, ls0, dl0);
    step(p1, q1, o1, ls1, dl1);
    p0 = p2;
  }
  if (it < n_it) {
    wait_vm0();
    barrier_keep_loads();
    step(p0, q0, o0, ls0, dl0);
  }

  if (has_keys && key < w.k1) {
    __bf16* kb = (__bf16*)p.dk + (int64_t)key * p.dk_st + (int64_t)w.g * p.dk_sh + 4 * g;
    __bf16* vb = (__bf16*)p.dv + (int64_t)key * p.dv_st + (int64_t)w.g * p.dv_sh + 4 * g;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      f32x4 rk = dk[m];
#pragma unroll
      for (int e = 0; e < 4; ++e) rk[e] *= f.scale;
      *(bf16x4*)(kb + 16 * m) = cvt_bf16x4(rk);
      *(bf16x4*)(vb + 16 * m) = cvt_bf16x4(dv[m]);
    }
  }
}

}  // namespace

void dense_bwd_plan(DenseBwdParams& p, int D) {
  dense_fwd_plan(p.f);
  p.kv_tile = D == 64 ? 32 * kDkdvWaves64 : 128;
  p.kv_n_vtiles = p.f.T / p.kv_tile + p.f.n_docs + 2;
  p.kv_n_work = p.f.Hkv * p.kv_n_vtiles;
  // heavy-first key tiles where the causal mask makes their weights uneven (segments must fit
  // the lanes of one wave)
  p.kv_heavy_first = p.f.window == 0 && p.f.n_docs + 2 <= 64 ? 1 : 0;
}

namespace {
template <int D>
hipError_t bwd_launch(const DenseBwdParams& p, hipStream_t stream) {
  // dq writes delta; the dk/dv kernel reads it, then the dsink passes reuse it (same stream)
  const int64_t gq = dense_fwd_grid(p.f);
  if (gq > 0) hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)gq), dim3(kThreads), 0, stream, p);
  // grid of key_tile_slot: 8 XCD columns of (Hkv / 8) VT, ceil(VT / (8 / Hkv)) or ceil(Hkv VT / 8) slots
  const int64_t Hkv = p.f.Hkv, VT = p.kv_n_vtiles;
  const int64_t per_xcd = p.kv_heavy_first && Hkv % kXcds == 0 ? Hkv / kXcds * VT
                          : p.kv_heavy_first && kXcds % Hkv == 0 ? (VT + kXcds / Hkv - 1) / (kXcds / Hkv)
                                                                 : (Hkv * VT + kXcds - 1) / kXcds;
  const int64_t gk = per_xcd * kXcds;
  if (gk > 0) {
    if constexpr (D == 128)
      hipLaunchKernelGGL(bwd_dkdv16_kernel, dim3((unsigned)gk), dim3(kT16), 0, stream, p);
    else
      hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)gk), dim3(64 * kDkdvWaves64), 0, stream, p);
  }
  if (p.f.sinks != nullptr && p.dsinks != nullptr) {
    const unsigned n_chunks = (unsigned)((p.f.T + kSinkChunk - 1) / kSinkChunk);
    hipLaunchKernelGGL(bwd_dsink_partial_kernel, dim3(n_chunks), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(bwd_dsink_reduce_kernel, dim3((unsigned)p.f.Hq), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t dense_bwd_launch(const DenseBwdParams& p, int D, hipStream_t stream) {
  if (p.f.T <= 0) return hipSuccess;
  if (D == 128) return bwd_launch<128>(p, stream);
  if (D == 64) return bwd_launch<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace swa
