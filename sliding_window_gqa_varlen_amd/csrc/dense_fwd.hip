// Packed variable-length causal / sliding-window GQA attention forward for gfx950.
//
// Operation (MuseMagiPlan.attention on the muse_spark magi_cp page, FlintMagiPlan.attention
// on the flint magi page, GQA grouping of MuseGlimmerAttention / repeat_kv on the
// muse_glimmer model page): for token i of document [s, e), query head h, KV head
// g = h / G, keys j with s <= j <= i and (window == 0 or i - j < window),
//   out[i,h] = sum_j exp(scale q.k_j) v_j / (sum_j exp(scale q.k_j) + exp(sink_h)).
//
// Design (one workgroup = 4 waves = 256 threads):
//  * Query columns.  Each wave owns 32 query "columns" = (32 / HB) consecutive tokens x
//    HB query heads of one KV group (HB = largest power of two dividing G, <= 32).  The
//    four waves stack along tokens, so a workgroup owns TQ = 128 / HB tokens x HB heads
//    and every key/value tile staged in LDS serves all 128 columns (GQA head-group reuse).
//  * Transposed scores.  S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys = M, query
//    columns = N): each lane holds one query column and 16 keys of every 32-key block, so
//    the softmax row statistics are lane-local except for one permlane32 swap with the
//    other half-wave, and the probabilities already sit in the B-operand layout of
//    O^T += V^T P^T.  V stays row-major in LDS; its transposed A operand comes from
//    ds_read_b64_tr_b16.
//  * Per-document tiling.  Query tiles start at document starts (virtual tile index
//    v -> segment by one ballot over cu_seqlens held one boundary per lane, or a binary
//    search beyond 61 documents; no host round trip), key tiles cover
//    only [max(doc start, first query - window + 1), last query]; masks are evaluated
//    only on tiles that straddle the diagonal or the window edge.
//  * Scheduling.  Blocks are remapped so that all tiles of one KV head land on the same
//    XCD (its L2 holds that head's K/V), and each document's tiles run last-first
//    (heaviest first for causal masks).  XCDs that share a head chunk under a causal mask
//    deal its tiles round robin.
//  * bf16 pipeline.  64-key K and V tiles arrive by buffer_load ... lds straight into
//    two LDS buffers each (no register staging); iteration j issues the MFMAs of
//    S(j) = K(j) Q^T, runs the online softmax of tile j-1 in their shadow, then
//    O += V(j-1) P(j-1), while K(j+1) and V(j) are in flight.  Buffers are separate
//    __shared__ arrays named statically (the loop is unrolled by two), so no LDS read
//    waits on a transfer into another buffer.  Rows are XOR-swizzled for the 64-bank
//    LDS: K for row reads of 16 rows at one unit, V for transposed reads of 4 rows x 4
//    units.  The output tile leaves through LDS so that every store writes whole rows.
//  * Online softmax with lazy rescaling: the reference maximum moves only when a score
//    exceeds it by more than 2^8 (probabilities stay <= 256), so most tiles skip the O
//    rescale; the final normalisation uses the same reference, so the result is exact.  The
//    bf16 kernel takes a tile's maximum only when a lane's partial row sum of the tile
//    exceeds 2^8 (the sum bounds every probability), which is rare once the first tile has
//    set the reference.
//  * fp32 inputs use v_mfma_f32_32x32x2_f32 with the same accumulator layout and a
//    register-staged, padded LDS layout (parity path, not tuned).
#include <type_traits>

#include "dense_common.h"

namespace swa {
namespace {

constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)
constexpr int kAhead128 = 6;  // operand fragments read this many MFMAs ahead (head_dim >= 128)
constexpr int kAhead64 = 2;   // the same for head_dim 64
constexpr int kOcc64 = 3;     // head_dim 64: three workgroups per CU

template <typename T, int D>
__device__ __forceinline__ void write_padding(const DenseFwdParams& p, const Tile& w) {
  // zero rows [t0, t_end) x heads [h0, h0 + HB); lse = -inf
  T* out = (T*)p.out;
  constexpr int kC = 16 / (int)sizeof(T);
  const int per_row = D / kC;
  const int n_rows = (w.t_end - w.t0) * w.HB;
  for (int idx = threadIdx.x; idx < n_rows * per_row; idx += kThreads) {
    const int row = idx / per_row, c = idx - row * per_row;
    const int t = w.t0 + row / w.HB, h = w.h0 + row % w.HB;
    *(u32x4*)(out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + c * kC) = u32x4{0, 0, 0, 0};
  }
  if (p.lse != nullptr)
    for (int idx = threadIdx.x; idx < n_rows; idx += kThreads)
      p.lse[(int64_t)(w.t0 + idx / w.HB) * p.Hq + w.h0 + idx % w.HB] = -INFINITY;
}

struct Softmax {
  float mref;  // reference max of the scores in log2 units (scale folded in)
  float l;     // running sum of exp2(s * c2 - mref) over this half-wave's keys
};

// Online-softmax statistics of one tile, from this lane's raw score maximum.  Lazy
// rescale: the reference max moves only when a score exceeds it by more than 2^8, so
// probabilities stay <= 256 and most tiles leave O alone (exact either way); lanes that
// keep their reference scale by exactly 1, also while it is -inf.  `alpha` is the factor
// O and l must be scaled by, `mu` the exponent offset of the probabilities (0 while
// nothing was visible).
struct TileStats {
  float alpha, mu;
  bool move;
};
__device__ __forceinline__ TileStats tile_stats(float lane_max, float c2, Softmax& st) {
  const float mx = half_swap_max(lane_max) * c2;
  TileStats t;
  t.move = mx > st.mref + kRescaleLog2;
  const float mnew = t.move ? mx : st.mref;
  t.alpha = t.move ? fast_exp2(st.mref - mnew) : 1.f;
  st.mref = mnew;
  t.mu = mnew == -INFINITY ? 0.f : mnew;
  return t;
}
__device__ __forceinline__ float lane_max(const f32x16 (&sc)[2]) {
  float mx = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sc[blk][a]);
  return mx;
}

// What the pipelined loop keeps of the statistics between tiles: the exponent offset of the
// probabilities, and the largest partial row sum that shows the reference may stay.  A lane's
// 32 probabilities of a tile that sum to at most 2^8 are each at most 2^8, so the maximum of its
// scores lies at most 8 (log2 units) above the reference and tile_stats would keep it (up to the
// rounding of that comparison, where either choice gives the exact result).  The maximum is then
// needed only when a sum exceeds the bound: rarely, once the first tile has set the reference.
// While the reference is -inf (nothing visible yet) the bound is -1, so every tile takes the
// exact path until something is visible.
constexpr float kLazyMax = 256.f;  // 2^kRescaleLog2
struct Lazy {
  float mu, thr;
};
__device__ __forceinline__ Lazy lazy_of(const Softmax& st, const TileStats& t) {
  return Lazy{t.mu, st.mref == -INFINITY ? -1.f : kLazyMax};
}

// Masks a diagonal / window-edge tile block by block (head_dim 256, whose one wave per SIMD has
// no other wave to hide the masking behind).  A block that needs no mask is left alone; a block
// that no query of the wave sees (all keys after the wave's last token, or all before its first
// token's window) is set to -inf without per-score tests; only a block that the cut crosses is
// masked score by score.
__device__ __forceinline__ void mask_tile_blocks(f32x16 (&sc)[2], int kb, const Cols& c) {
  const int tq4 = opaque(c.tq - 4 * c.h2);  // as in mask_tile
  const int lo = c.W ? tq4 - c.W + 1 - kb : -(1 << 30);
  const unsigned range = (unsigned)(tq4 - kb - lo);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int b0 = kb + 32 * blk;
    if (!(b0 + 31 > c.tw0 || (c.W != 0 && b0 <= c.tw1 - c.W))) continue;
    if (b0 > c.tw1 || (c.W != 0 && b0 + 31 <= c.tw0 - c.W)) {
#pragma unroll
      for (int a = 0; a < 16; ++a) sc[blk][a] = -INFINITY;
      continue;
    }
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int off = 32 * blk + 8 * (a >> 2) + (a & 3);
      sc[blk][a] = (unsigned)(off - lo) <= range ? sc[blk][a] : -INFINITY;
    }
  }
}

// Probabilities exp2(s c2 - mu) of the lane's scores as the four B operands of O^T += V^T P^T,
// and their sum, added in the order of the pipelined step.
__device__ __forceinline__ float tile_probs(const f32x16 (&sc)[2], float c2, float mu, bf16x8 (&pb)[4]) {
  float rs = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    f32x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = fast_exp2(__builtin_fmaf(sc[g >> 1][8 * (g & 1) + e], c2, -mu));
    pb[g] = cvt_bf16x8(pf);
#pragma unroll
    for (int e = 0; e < 8; ++e) rs += pf[e];
  }
  return rs;
}

// Scores -> unnormalised probabilities exp2(s * c2 - mu), in place; returns their sum.
// NB = 1: the first 32-key block only (the second is known to be fully masked)
template <int NB = 2>
__device__ __forceinline__ float tile_exp(f32x16 (&sc)[2], float c2, float mu) {
  float rs = 0.f;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const float e = fast_exp2(__builtin_fmaf(sc[blk][a], c2, -mu));
      sc[blk][a] = e;
      rs += e;
    }
  return rs;
}

template <int DB>
__device__ __forceinline__ void rescale_o(bool move, float alpha, f32x16 (&o)[DB]) {
  if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] *= alpha;
  }
}
// Full online-softmax step for one tile (used where nothing is interleaved with it).
template <int DB>
__device__ __forceinline__ void softmax_tile(f32x16 (&sc)[2], bool need_mask, int kb, const Cols& c, float c2,
                                             Softmax& st, f32x16 (&o)[DB]) {
  if (need_mask) mask_tile(sc, kb, c);
  const TileStats t = tile_stats(lane_max(sc), c2, st);
  rescale_o<DB>(t.move, t.alpha, o);
  st.l = st.l * t.alpha + tile_exp(sc, c2, t.mu);
}

// Half-wave sums combined, sink folded in; stores the LSE and returns the normaliser.
// `st.l` holds this half-wave's share of the row sum.  The normaliser comes from v_rcp_f32
// (within 1 ulp) rather than a correctly rounded division sequence: its error is far below the
// output's rounding.
// `sink` is the lane's sink logit (p.sinks[c.hq]) when there are sinks.
__device__ __forceinline__ float epilogue_scalars(const DenseFwdParams& p, const Tile& w, const Cols& c,
                                                  const Softmax& st, float sink) {
  const float lt = half_swap_sum(st.l);
  const float m2 = st.mref;  // reference max in log2 units (-inf if nothing was visible)
  float inv, lse_v;
  if (p.sinks != nullptr) {
    const float s2 = sink * kLog2e;
    const float mm = fmaxf(m2, s2);
    const float corr = fast_exp2(m2 - mm);
    const float lf = lt * corr + fast_exp2(s2 - mm);
    inv = corr * __builtin_amdgcn_rcpf(lf);
    lse_v = (mm + __builtin_amdgcn_logf(lf)) * kLn2;
  } else {
    inv = __builtin_amdgcn_rcpf(lt);
    lse_v = (m2 + __builtin_amdgcn_logf(lt)) * kLn2;
  }
  if (p.lse != nullptr && c.h2 == 0 && c.tq < w.t_end) p.lse[(int64_t)c.tq * p.Hq + c.hq] = lse_v;
  return inv;
}

// One normalisation, one rounding, stores straight from the accumulator layout.
template <typename T, int DB>
__device__ __forceinline__ void epilogue(const DenseFwdParams& p, const Tile& w, const Cols& c,
                                         const Softmax& st, const f32x16 (&o)[DB]) {
  const float inv = epilogue_scalars(p, w, c, st, p.sinks != nullptr ? p.sinks[c.hq] : 0.f);
  if (c.tq < w.t_end) {
    T* ob = (T*)p.out + (int64_t)c.tq * p.o_st + (int64_t)c.hq * p.o_sh;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = o[d][4 * i + e] * inv;
        T* dst = ob + 32 * d + 8 * i + 4 * c.h2;
        if constexpr (std::is_same<T, __bf16>::value) *(bf16x4*)dst = cvt_bf16x4(r);
        else *(f32x4*)dst = r;
      }
  }
}

// ======================================================================================
// bf16: DMA-staged, software-pipelined kernel
// ======================================================================================
template <int D>
struct Bf {
  static constexpr int U = D / 8;                   // 16-byte units per row
  static constexpr int kTileUnits = kBN * U;        // units per K (or V) tile
  static constexpr int kDmaPerWave = kTileUnits / 64 / 4;
  static constexpr int kQFrags = D / 16;
  static constexpr int kDBlocks = D / 32;
  static_assert(kTileUnits % 256 == 0, "tile must split evenly over the four waves");
};

// Physical 16-byte unit (within its row) of logical unit u is u ^ key(row).  K rows are
// read 16 rows at one unit (MFMA A operand); V rows by ds_read_b64_tr_b16, 4 consecutive
// rows x 4 consecutive units per half-wave.  With 64 banks of 4 bytes, a 256-byte bank line
// holds one D=128 row, two D=64 rows or half a D=256 row.
template <int D>
__device__ __forceinline__ int k_key(int r) {
  if constexpr (D >= 128) return r & 15;
  else return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int v_key(int r) {
  if constexpr (D >= 128) return (r & 3) << 2;
  else return ((r >> 1) & 1) << 2;
}

// Per-lane voffset of the full-tile transfers: lane row lr = lane / U, unit lp ^ key(row).
// The row of transfer i is (4 i + wave) R + lr, and every key depends on it only through its
// low four bits, which take at most two values over i (row steps of 4 R = 16 (D = 128),
// 32 (D = 64) or 8 (D = 256)): kClasses offsets per lane, computed once per workgroup.
// D = 256 has no register to spare: it recomputes them per tile (kKeep = false).
template <int D, bool IS_V>
struct DmaLane {
  static constexpr bool kKeep = D <= 128;
  static constexpr int kClasses = (D == 256 && !IS_V) ? 2 : 1;
  uint32_t off[kClasses];
};
template <int D, bool IS_V>
__device__ __forceinline__ DmaLane<D, IS_V> dma_lane(int64_t st, int lane, int wave) {
  using B = Bf<D>;
  constexpr int R = 64 / B::U;  // rows per 64-unit block
  const uint32_t stb = (uint32_t)st * 2u;
  const int lr = lane / B::U, lp = lane % B::U;
  DmaLane<D, IS_V> d;
#pragma unroll
  for (int i = 0; i < DmaLane<D, IS_V>::kClasses; ++i) {
    const int r = (i * 4 + wave) * R + lr;
    const int cu = lp ^ (IS_V ? v_key<D>(r) : k_key<D>(r));
    d.off[i] = (uint32_t)lr * stb + (uint32_t)cu * 16u;
  }
  return d;
}

// Gather one 64-key tile (rows kb.. clamped to k_hi - 1) of one tensor into `buf` with
// buffer_load ... lds (MUBUF LDS DMA: the tile base sits in the buffer descriptor, the
// 64-unit block's row offset in soffset and the lane's offset in a register kept across
// the loop, so a full-tile transfer costs no VALU).  Rows past the tile's last query are
// clamped to the last valid row (always in bounds); every such key lies after every valid
// query of the tile, so it is masked and contributes zero.
template <int D, bool IS_V>
__device__ __forceinline__ void dma_tile(const __bf16* base, int64_t st, int kb, int k_hi, u32x4* buf,
                                         int wave, int lane_in, const DmaLane<D, IS_V>& dl) {
  using B = Bf<D>;
  constexpr int R = 64 / B::U;  // rows per 64-unit block
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kb * st), (short)0, -1, kBufferWord3);
  const uint32_t stb = (uint32_t)st * 2u;  // row stride in bytes (< 2^25)
  const int lim = k_hi - 1 - kb;
  if (lim >= kBN - 1) {
    const DmaLane<D, IS_V> d = DmaLane<D, IS_V>::kKeep ? dl : dma_lane<D, IS_V>(st, opaque(lane_in), wave);
#pragma unroll
    for (int i = 0; i < B::kDmaPerWave; ++i) {
      const int blk = i * 4 + wave;  // wave-uniform 64-unit block
      u32x4* dst = buf + __builtin_amdgcn_readfirstlane(blk * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, d.off[i % DmaLane<D, IS_V>::kClasses],
                                               __builtin_amdgcn_readfirstlane((uint32_t)(blk * R) * stb), 0, 0);
    }
  } else {
    const int lane = opaque(lane_in);  // the last tile only: recomputed, nothing kept live
    const int lr = lane / B::U, lp = lane % B::U;
#pragma unroll
    for (int i = 0; i < B::kDmaPerWave; ++i) {
      const int blk = i * 4 + wave;
      const int r = blk * R + lr;
      const int cu = lp ^ (IS_V ? v_key<D>(r) : k_key<D>(r));
      u32x4* dst = buf + __builtin_amdgcn_readfirstlane(blk * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, (uint32_t)min(r, lim) * stb + (uint32_t)cu * 16u,
                                               0, 0, 0);
    }
  }
}

// S^T for the two 32-key blocks of the tile in `kbuf`.
template <int D>
__device__ __forceinline__ void qk_tile(const u32x4* kbuf, const bf16x8 (&qf)[Bf<D>::kQFrags], int n_in, int h2,
                                        f32x16 (&sc)[2]) {
  using B = Bf<D>;
  const int n = opaque(n_in);
  const int kk = k_key<D>(n);  // equal for rows n and 32 + n
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    sc[blk] = f32x16{};
    const int row = (32 * blk + n) * B::U;
#pragma unroll
    for (int s = 0; s < B::kQFrags; ++s) {
      const u32x4 a = kbuf[row + ((2 * s + h2) ^ kk)];
      sc[blk] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), qf[s], sc[blk]);
    }
  }
}

// Byte offsets, within a V tile, of this lane's ds_read_b64_tr_b16 for each output block
// (rows 4 h2 + (lane & 15) / 4, 16-byte units 4 d + 2 dh + sub, XOR-swizzled); the k-step
// rows and the +8-row half are immediate offsets on top.
template <int D>
struct VOffsets {
  int off[Bf<D>::kDBlocks];
};
template <int D>
__device__ __forceinline__ VOffsets<D> v_offsets(int lane) {
  using B = Bf<D>;
  const int j16 = lane & 15, dh = (lane >> 4) & 1, h2 = lane >> 5;
  const int vk = v_key<D>(j16 >> 2);  // rows 4*h2 + (j16 >> 2) (+16s, +32blk, +8): same key
  const int sub = (j16 & 3) >> 1;
  const int half = (j16 & 1) * 4;
  VOffsets<D> v;
#pragma unroll
  for (int d = 0; d < B::kDBlocks; ++d)
    v.off[d] = (((4 * h2 + (j16 >> 2)) * B::U + ((4 * d + 2 * dh + sub) ^ vk)) * 8 + half) * 2;
  return v;
}
template <int D>
__device__ __forceinline__ bf16x8 v_frag(const u32x4* vbuf, const VOffsets<D>& vo, int ks, int d) {
  using B = Bf<D>;
  const int row_off = (32 * (ks >> 1) + 16 * (ks & 1)) * B::U * 16;  // rows r0 and r0 + 8
  const char* p = (const char*)vbuf + vo.off[d] + row_off;
  const bf16x4 lo4 = lds_read_tr4((const __bf16*)p);
  const bf16x4 hi4 = lds_read_tr4((const __bf16*)(p + 8 * B::U * 16));
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// O^T += V^T P^T for the tile in `vbuf` (probabilities in sc).
// NKS = 2: k-steps 0 and 1 only (keys 0-31; the second block's probabilities are zero)
template <int D, int NKS = 4>
__device__ __forceinline__ void pv_tile(const u32x4* vbuf, const f32x16 (&sc)[2], const VOffsets<D>& vo,
                                        f32x16 (&o)[Bf<D>::kDBlocks]) {
  using B = Bf<D>;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    f32x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = sc[ks >> 1][8 * (ks & 1) + e];
    const bf16x8 pb = cvt_bf16x8(pf);
#pragma unroll
    for (int d = 0; d < B::kDBlocks; ++d) o[d] = mfma_bf16_32x32x16(v_frag<D>(vbuf, vo, ks, d), pb, o[d]);
  }
}

// One pipelined step in program order: S(j) = K(j) Q^T on the MFMA unit while the
// exponentials of tile j-1 run on the VALU (a wave64 VALU op issues in 4 cycles, an exponential
// in 8, and a 32x32x16 MFMA keeps the VALU from issuing for about half of its 32 cycles), then
// O += V(j-1) P(j-1).  Between the two halves one compare of the lane's partial row sum against
// lz.thr decides, for the whole wave, whether the rare exact path `move` runs: it takes the
// tile's maximum, moves the reference where tile_stats says so, rescales O and recomputes the
// probabilities (pb) and their sum, which it returns.  Operand fragments stream from LDS kAhead
// MFMAs ahead of their use (K fragments first, then the transposed V fragments), so each MFMA
// waits only for a read issued long before.  Every slot is fenced with sched_barrier: the
// emitted order is exactly this one.
template <int D, class Move>
__device__ __forceinline__ float qk_pv_step(const u32x4* kbuf, const u32x4* vbuf, const bf16x8 (&qf)[Bf<D>::kQFrags],
                                            int kaddr, const VOffsets<D>& vo, f32x16 (&sn)[2],
                                            const f32x16 (&sc)[2], float c2, const Lazy& lz,
                                            f32x16 (&o)[Bf<D>::kDBlocks], Move&& move) {
  using B = Bf<D>;
  constexpr int NQ = 2 * B::kQFrags;  // QK^T MFMAs (32 for D = 256, 16 for D = 128, 8 for D = 64)
  constexpr int NP = 4 * B::kDBlocks; // PV MFMAs
  constexpr int kAhead = (D >= 128) ? kAhead128 : kAhead64;
  u32x4 frag[NQ + NP];
  __builtin_amdgcn_s_setprio(1);  // the wave in its MFMA stream goes first
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): nothing older is in flight, later waits count exactly
  auto read = [&](int f) {
    if (f < NQ) {
      const int blk = f & 1, s = f >> 1;  // the two key blocks alternate: neighbours are independent
      frag[f] = *(const u32x4*)((const char*)kbuf + (kaddr ^ (32 * s)) + blk * 32 * B::U * 16);
    } else {
      const int i = f - NQ;
      frag[f] = __builtin_bit_cast(u32x4, v_frag<D>(vbuf, vo, i / B::kDBlocks, i % B::kDBlocks));
    }
  };
#pragma unroll
  for (int f = 0; f < kAhead; ++f) read(f);
  __builtin_amdgcn_sched_barrier(0);

  sn[0] = f32x16{};
  sn[1] = f32x16{};
  bf16x8 pb[4];
  f32x8 pf;
  float rs = 0.f;
  // exponential x of tile j-1 (block x / 16, accumulator x % 16); every 8 form a B operand
  auto exp_step = [&](int x) {
    pf[x & 7] = fast_exp2(__builtin_fmaf(sc[x >> 4][x & 15], c2, -lz.mu));
    asm volatile("" : "+v"(pf[x & 7]));  // this slot's exponentials stay in this slot
    if ((x & 7) == 7) {
      pb[x >> 3] = cvt_bf16x8(pf);
      // packed here: otherwise the conversion, common to both paths after the check, sinks
      // below it and keeps the 8 fp32 values live instead of 4 packed registers
      asm volatile("" : "+v"(pb[x >> 3]));
#pragma unroll
      for (int h = 0; h < 8; ++h) rs += pf[h];
    }
  };
  // head_dim 256 (one wave per SIMD, nothing to hide a stall behind) finishes its exponentials
  // two QK^T slots early, so the sum, the compare and the branch run under MFMAs already issued
  constexpr int QX = NQ - (D == 256 ? 2 : 0);  // QK^T slots that carry exponentials
#pragma unroll
  for (int i = 0; i < QX; ++i) {
    sn[i & 1] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, frag[i]), qf[i >> 1], sn[i & 1]);
    if (i + kAhead < NQ + NP) read(i + kAhead);
#pragma unroll
    for (int x = 32 * i / QX; x < 32 * (i + 1) / QX; ++x) exp_step(x);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (__builtin_amdgcn_ballot_w64(!(rs <= lz.thr)) != 0) rs = move(pb);
#pragma unroll
  for (int i = QX; i < NQ; ++i) {
    sn[i & 1] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, frag[i]), qf[i >> 1], sn[i & 1]);
    if (i + kAhead < NQ + NP) read(i + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int ks = i / B::kDBlocks, d = i % B::kDBlocks;
    o[d] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, frag[NQ + i]), pb[ks], o[d]);
    if (NQ + i + kAhead < NQ + NP) read(NQ + i + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  return rs;
}

template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? kOcc64 : D == 128 ? 2 : 1) void dense_fwd_bf16_kernel(
    DenseFwdParams p) {
  using B = Bf<D>;
  __shared__ u32x4 k0[B::kTileUnits];
  __shared__ u32x4 k1[B::kTileUnits];
  __shared__ u32x4 v0[B::kTileUnits];
  __shared__ u32x4 v1[B::kTileUnits];

  Tile w;
  if (!decode_tile<true>(p, w)) return;
  if (w.padding) {
    write_padding<__bf16, D>(p, w);
    return;
  }
  const Cols c = make_cols(p, w);

  // the lane's sink logit, loaded before the Q loads and the first transfers (loads complete in
  // order, so the transfer waits below cover it): read after the key loop, its latency would
  // otherwise sit at the end of every workgroup.  Without sinks the load reads q's first element
  // (always valid memory, never used), so it needs no branch that would make the compiler wait
  // for it at once.  head_dim 256 has no register to hold it across the loop: it reads the sink
  // at the end.
  const float sink = D == 256 ? 0.f : *(p.sinks != nullptr ? p.sinks + c.hq : (const float*)p.q);
  bf16x8 qf[B::kQFrags];
  {
    const __bf16* qb = (const __bf16*)p.q + (int64_t)min(c.tq, w.t_end - 1) * p.q_st + (int64_t)c.hq * p.q_sh;
#pragma unroll
    for (int s = 0; s < B::kQFrags; ++s) qf[s] = *(const bf16x8*)(qb + 16 * s + 8 * c.h2);
  }
  const __bf16* kbase = (const __bf16*)p.k + (int64_t)w.g * p.k_sh;
  const __bf16* vbase = (const __bf16*)p.v + (int64_t)w.g * p.v_sh;

  f32x16 o[B::kDBlocks];
#pragma unroll
  for (int d = 0; d < B::kDBlocks; ++d) o[d] = f32x16{};
  Softmax st{-INFINITY, 0.f};
  const float c2 = p.c2;
  const int nt = c.n_tiles;
  // loop-invariant LDS byte offsets of this lane's K and V fragments: K row n, unit
  // (2 s + h2) ^ key(n) = (h2 ^ key(n)) ^ 2 s, so the address is kaddr ^ (32 s)
  const int kaddr = c.n * B::U * 16 + ((c.h2 ^ k_key<D>(c.n)) << 4);
  const VOffsets<D> vo = v_offsets<D>(c.lane);

  // prologue: K(0) -> k0, V(0) -> v0, K(1) -> k1 all at once; wait for K(0) only (loads
  // complete in order) while V(0) and K(1) stay in flight through S(0)
  const DmaLane<D, false> kdl = dma_lane<D, false>(p.k_st, c.lane, c.wave);
  const DmaLane<D, true> vdl = dma_lane<D, true>(p.v_st, c.lane, c.wave);
  dma_tile<D, false>(kbase, p.k_st, c.k_lo, c.k_hi, k0, c.wave, c.lane, kdl);
  dma_tile<D, true>(vbase, p.v_st, c.k_lo, c.k_hi, v0, c.wave, c.lane, vdl);
  if (nt > 1) {
    dma_tile<D, false>(kbase, p.k_st, c.k_lo + kBN, c.k_hi, k1, c.wave, c.lane, kdl);
    wait_vmcnt<2 * B::kDmaPerWave>();
  } else {
    wait_vmcnt<B::kDmaPerWave>();
  }
  barrier_keep_loads();
  f32x16 sc[2];
  qk_tile<D>(k0, qf, c.n, c.h2, sc);
  if (tile_needs_mask(c, c.k_lo)) {
    if constexpr (D == 256) mask_tile_blocks(sc, c.k_lo, c);
    else mask_tile(sc, c.k_lo, c);
  }
  // the first tile sets the reference (O and l are still zero: nothing to rescale)
  Lazy lz;
  {
    const TileStats t0 = tile_stats(lane_max(sc), c2, st);
    lz = lazy_of(st, t0);
  }
  // the exact path of a tile whose probabilities may exceed 2^8 (scores of the tile in sc)
  auto exact = [&](float& alpha) {
    const TileStats t = tile_stats(lane_max(sc), c2, st);
    rescale_o<B::kDBlocks>(t.move, t.alpha, o);
    lz = lazy_of(st, t);
    alpha = t.alpha;
  };

  // iteration j: S(j) from K(j) ; softmax + PV of tile j-1 ; K(j+1), V(j) in flight.
  // On entry sc holds the masked scores of tile j-1 and lz the offset of their probabilities.
  // One fenced instruction stream runs the QK^T MFMAs of tile j with the exponentials of tile
  // j-1 between them, then (after the rare exact path) the PV MFMAs of tile j-1; tile j is then
  // masked if it straddles the diagonal or the window edge.  Tiles a wave does not see are
  // computed too: fully masked, they add nothing.
  auto step = [&](int j, const u32x4* kcur, u32x4* knext, u32x4* vcur_dst, const u32x4* vprev) {
    const int kb = c.k_lo + j * kBN;
    wait_vm0();
    barrier_keep_loads();  // K(j), V(j-1) landed for every wave; K(j-1), V(j-2) consumed
    if (j + 1 < nt) dma_tile<D, false>(kbase, p.k_st, kb + kBN, c.k_hi, knext, c.wave, c.lane, kdl);
    dma_tile<D, true>(vbase, p.v_st, kb, c.k_hi, vcur_dst, c.wave, c.lane, vdl);
    f32x16 sn[2];
    float alpha = 1.f;
    const float rs = qk_pv_step<D>(kcur, vprev, qf, kaddr, vo, sn, sc, c2, lz, o, [&](bf16x8 (&pb)[4]) {
      exact(alpha);
      return tile_probs(sc, c2, lz.mu, pb);
    });
    if (tile_needs_mask(c, kb)) {
      if constexpr (D == 256) mask_tile_blocks(sn, kb, c);
      else mask_tile(sn, kb, c);
    }
    st.l = st.l * alpha + rs;
    sc[0] = sn[0];
    sc[1] = sn[1];
  };
  int j = 1;
  for (; j + 1 < nt; j += 2) {
    step(j, k1, k0, v1, v0);
    step(j + 1, k0, k1, v0, v1);
  }
  if (j < nt) step(j, k1, k0, v1, v0);
  // last tile: its K and V are in buffers (nt - 1) & 1.  When its second 32-key block starts
  // after this wave's last token, the mask set all of that block's scores to -inf: their
  // probabilities are exactly zero, so its exponentials and PV k-steps 2 and 3 are skipped (a
  // uniform branch that leaves the result unchanged).  Not for D = 256, whose registers the
  // second copy of the tail would spill.  The probabilities replace the scores in place; if the
  // exact path is needed, the scores are computed again from the K tile, which no transfer
  // overwrites after the last step, and Q read again (the same MFMAs: the same scores).
  wait_vm0();
  barrier_keep_loads();
  const bool last_odd = (nt - 1) & 1;
  auto last_tile = [&](auto nb) {
    constexpr int NB = decltype(nb)::value;
    float rs = tile_exp<NB>(sc, c2, lz.mu);
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(!(rs <= lz.thr)) != 0) {
      const Cols cr = fresh_lane_cols(c, p.hb_shift, w);
      bf16x8 qr[B::kQFrags];
      const __bf16* qb = (const __bf16*)p.q + (int64_t)min(cr.tq, w.t_end - 1) * p.q_st + (int64_t)cr.hq * p.q_sh;
#pragma unroll
      for (int s = 0; s < B::kQFrags; ++s) qr[s] = *(const bf16x8*)(qb + 16 * s + 8 * cr.h2);
      qk_tile<D>(last_odd ? k1 : k0, qr, cr.n, cr.h2, sc);
      const int kb = c.k_lo + (nt - 1) * kBN;
      if (tile_needs_mask(cr, kb)) {
        if constexpr (D == 256) mask_tile_blocks(sc, kb, cr);
        else mask_tile(sc, kb, cr);
      }
      exact(alpha);
      rs = tile_exp<NB>(sc, c2, lz.mu);
    }
    st.l = st.l * alpha + rs;
    if (last_odd) pv_tile<D, 2 * NB>(v1, sc, vo, o);
    else pv_tile<D, 2 * NB>(v0, sc, vo, o);
  };
  const bool tail_half = D != 256 && c.k_lo + (nt - 1) * kBN + 32 > c.tw1;
  if (tail_half) last_tile(std::integral_constant<int, 1>{});
  else last_tile(std::integral_constant<int, 2>{});
  // the output images, two waves per buffer, go to the K and V buffers the last tile does not
  // use: every wave finished reading them before the barrier above and no transfer targets them,
  // while the last tile's K may still be read by a wave on its exact path and its V by the PV
  char* img = (char*)(c.wave < 2 ? (last_odd ? k0 : k1) : (last_odd ? v0 : v1)) + (c.wave & 1) * (64 * D);
  const Cols ce = fresh_lane_cols(c, p.hb_shift, w);
  const float inv =
      epilogue_scalars(p, w, ce, st, D == 256 ? (p.sinks != nullptr ? p.sinks[ce.hq] : 0.f) : sink);
  store_out_bf16<D>(p.out, p.o_st, p.o_sh, w, ce, p.hb_shift, inv, o, img);
}

// ======================================================================================
// fp32: register-staged kernel with padded LDS rows (parity path)
// ======================================================================================
template <int D>
struct F32Geo {
  static constexpr int kKPitch = D + 1;  // odd pitch: conflict-free scalar column reads
  static constexpr int kVPitch = D;
  static constexpr int kKElems = kBN * kKPitch;
  static constexpr int kStage = kKElems + kBN * kVPitch;
  static constexpr int kQFrags = D / 2;
  static constexpr int kDBlocks = D / 32;
  static constexpr int kChunksPerRow = D / 4;
  static constexpr int kLoads = kBN * kChunksPerRow / kThreads;
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dense_fwd_f32_kernel(DenseFwdParams p) {
  using G = F32Geo<D>;
  __shared__ __attribute__((aligned(16))) float smem[2 * G::kStage];
  Tile w;
  if (!decode_tile<true>(p, w)) return;
  if (w.padding) {
    write_padding<float, D>(p, w);
    return;
  }
  const Cols c = make_cols(p, w);
  float qf[G::kQFrags];
  {
    const float* qb = (const float*)p.q + (int64_t)min(c.tq, w.t_end - 1) * p.q_st + (int64_t)c.hq * p.q_sh;
#pragma unroll
    for (int s = 0; s < G::kQFrags; ++s) qf[s] = qb[2 * s + c.h2];
  }
  const float* kbase = (const float*)p.k + (int64_t)w.g * p.k_sh;
  const float* vbase = (const float*)p.v + (int64_t)w.g * p.v_sh;
  u32x4 kreg[G::kLoads], vreg[G::kLoads];
  // rows past the tile's last query are clamped to the last valid row; they are masked
  auto stage_load = [&](int kb) {
    const int lim = c.k_hi - 1 - kb;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int row = min(e / G::kChunksPerRow, lim);
      const int col = (e % G::kChunksPerRow) * 4;
      kreg[i] = *(const u32x4*)(kbase + (int64_t)(kb + row) * p.k_st + col);
      vreg[i] = *(const u32x4*)(vbase + (int64_t)(kb + row) * p.v_st + col);
    }
  };
  auto stage_store = [&](int buf) {
    float* Ks = smem + buf * G::kStage;
    float* Vs = Ks + G::kKElems;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int row = e / G::kChunksPerRow;
      const int col = (e % G::kChunksPerRow) * 4;
      float* kd = Ks + row * G::kKPitch + col;
      kd[0] = __uint_as_float(kreg[i][0]);
      kd[1] = __uint_as_float(kreg[i][1]);
      kd[2] = __uint_as_float(kreg[i][2]);
      kd[3] = __uint_as_float(kreg[i][3]);
      *(u32x4*)(Vs + row * G::kVPitch + col) = vreg[i];
    }
  };
  f32x16 o[G::kDBlocks];
#pragma unroll
  for (int d = 0; d < G::kDBlocks; ++d) o[d] = f32x16{};
  Softmax st{-INFINITY, 0.f};
  if (c.n_tiles > 0) {
    stage_load(c.k_lo);
    stage_store(0);
  }
  __syncthreads();
  for (int j = 0; j < c.n_tiles; ++j) {
    const int kb = c.k_lo + j * kBN;
    if (j + 1 < c.n_tiles) stage_load(kb + kBN);
    const float* Ks = smem + (j & 1) * G::kStage;
    const float* Vs = Ks + G::kKElems;
    if (tile_active(c, kb)) {
      f32x16 sc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        sc[blk] = f32x16{};
        const float* krow = Ks + (32 * blk + c.n) * G::kKPitch;
#pragma unroll
        for (int s = 0; s < G::kQFrags; ++s) sc[blk] = mfma_f32_32x32x2(krow[2 * s + c.h2], qf[s], sc[blk]);
      }
      softmax_tile<G::kDBlocks>(sc, tile_needs_mask(c, kb), kb, c, p.c2, st, o);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int key = 32 * blk + 8 * (u >> 2) + 4 * c.h2 + (u & 3);
          const float* vr = Vs + key * G::kVPitch + c.n;
#pragma unroll
          for (int d = 0; d < G::kDBlocks; ++d) o[d] = mfma_f32_32x32x2(vr[32 * d], sc[blk][u], o[d]);
        }
    }
    if (j + 1 < c.n_tiles) stage_store((j + 1) & 1);
    __syncthreads();
  }
  epilogue<float, G::kDBlocks>(p, w, c, st, o);
}

template <typename K>
hipError_t launch_kernel(K kernel, const DenseFwdParams& p, hipStream_t stream) {
  const int64_t grid = dense_fwd_grid(p);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

void dense_fwd_plan(DenseFwdParams& p) {
  p.G = p.Hq / p.Hkv;
  int hb = p.G & (-p.G);  // largest power of two dividing G
  if (hb > 32) hb = 32;
  int shift = 0;
  while ((1 << shift) < hb) ++shift;
  p.hb_shift = shift;
  p.n_chunks = p.G >> shift;
  p.tile_tokens = 128 >> shift;
  p.n_vtiles = p.T / p.tile_tokens + p.n_docs + 2;
  p.n_work = p.Hkv * p.n_chunks * p.n_vtiles;
  // division by n_vtiles on the device as a multiply and a shift (round-up method for 31-bit
  // numerators: with l = ceil(log2 d) and m = ceil(2^(31 + l) / d), m d - 2^(31 + l) < 2^l, so
  // floor(n / d) = floor(n m / 2^(31 + l)) for every 0 <= n < 2^31, and m < 2^32)
  {
    const uint64_t d = (uint64_t)(p.n_vtiles > 0 ? p.n_vtiles : 1);
    int l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    p.vt_shift = 31 + l;
    p.vt_magic = (uint32_t)((((uint64_t)1 << p.vt_shift) + d - 1) / d);
  }
  p.c2 = p.scale * 1.4426950408889634f;
}

int64_t dense_fwd_grid(const DenseFwdParams& p) {
  if (p.T <= 0) return 0;
  const int64_t w = (int64_t)p.n_work;
  return (w + kXcds - 1) / kXcds * kXcds;
}

hipError_t dense_fwd_launch(const DenseFwdParams& p, Dtype dt, int D, hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (D == 128) return launch_kernel(dense_fwd_bf16_kernel<128>, p, stream);
    if (D == 64) return launch_kernel(dense_fwd_bf16_kernel<64>, p, stream);
    if (D == 256) return launch_kernel(dense_fwd_bf16_kernel<256>, p, stream);
  } else {
    if (D == 128) return launch_kernel(dense_fwd_f32_kernel<128>, p, stream);
    if (D == 64) return launch_kernel(dense_fwd_f32_kernel<64>, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace swa
