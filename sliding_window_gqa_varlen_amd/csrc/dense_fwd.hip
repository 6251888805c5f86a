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
//    columns = N): each lane ends up holding one query column and 16 keys of every
//    32-key block, so the softmax row statistics are lane-local except for one
//    permlane32 swap with the other half-wave, and the probabilities already sit in the
//    B-operand layout of O^T += V^T P^T.  V stays row-major in LDS; its transposed
//    A operand comes from ds_read_b64_tr_b16.
//  * Per-document tiling.  Query tiles start at document starts (virtual tile index
//    v -> segment by binary search over cu_seqlens, no host round trip), key tiles cover
//    only [max(doc start, first query - window + 1), last query]; masks are evaluated
//    only on tiles that straddle the diagonal or the window edge.
//  * Scheduling.  Blocks are remapped so that all tiles of one KV head land on the same
//    XCD (its L2 holds that head's K/V), and each document's tiles run last-first
//    (heaviest first for causal masks).
//  * Double-buffered K/V tiles: the next tile's global loads are issued before the
//    current tile's math and written to the other LDS buffer after it.
//  * Online softmax with lazy rescaling: the reference maximum moves only when a score
//    exceeds it by more than 2^8 (probabilities stay <= 256), so most tiles skip the O
//    rescale; the final normalisation uses the same reference, so the result is exact.
//  * fp32 inputs use v_mfma_f32_32x32x2_f32 with the same accumulator layout.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;    // keys per tile
constexpr int kXcds = 8;   // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)

template <typename T, int D>
struct Geo {
  static constexpr bool kBf16 = std::is_same<T, __bf16>::value;
  static constexpr int kKPitch = kBf16 ? D + 8 : D + 1;  // LDS row pitch of K (elements)
  // LDS row pitch of V: the transposed reads of one half-wave touch 4 consecutive rows x
  // 64 bytes, conflict-free on the 64 4-byte banks when the pitch is 16 (mod 64) words
  static constexpr int kVPitch = kBf16 ? D + 32 : D;
  static constexpr int kKElems = kBN * kKPitch;
  static constexpr int kVElems = kBN * kVPitch;
  static constexpr int kStage = kKElems + kVElems;
  static constexpr int kQFrags = kBf16 ? D / 16 : D / 2;
  static constexpr int kDBlocks = D / 32;
  static constexpr int kChunk = 16 / (int)sizeof(T);      // elements per 16-byte chunk
  static constexpr int kChunksPerRow = D / kChunk;
  static constexpr int kLoads = kBN * kChunksPerRow / kThreads;  // chunks per thread per tensor
  static_assert(kBN * kChunksPerRow % kThreads == 0, "tile must split evenly over threads");
};

template <typename T>
using QFragT = typename std::conditional<std::is_same<T, __bf16>::value, bf16x8, float>::type;

// Segment boundaries: segment 0 = [0, cu[0]) and segment n+1 = [cu[n], T) are padding,
// segment s in 1..n is document s-1.  Entries are clamped to [0, T].
__device__ __forceinline__ int seg_bound(const DenseFwdParams& p, int s) {
  if (s <= 0) return 0;
  if (s > p.n_docs + 1 || p.cu_seqlens == nullptr) return s > p.n_docs + 1 ? p.T : 0;
  int x = p.cu_seqlens[s - 1];
  return x < 0 ? 0 : (x > p.T ? p.T : x);
}

template <typename T, int D>
__device__ __forceinline__ void write_padding(const DenseFwdParams& p, int t0, int t_end, int h0, int HB) {
  // zero rows [t0, t_end) x heads [h0, h0 + HB); lse = -inf
  T* out = (T*)p.out;
  constexpr int kC = 16 / (int)sizeof(T);
  const int per_row = D / kC;
  const int n_rows = (t_end - t0) * HB;
  for (int idx = threadIdx.x; idx < n_rows * per_row; idx += kThreads) {
    const int row = idx / per_row, c = idx - row * per_row;
    const int t = t0 + row / HB, h = h0 + row % HB;
    *(u32x4*)(out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + c * kC) = u32x4{0, 0, 0, 0};
  }
  if (p.lse != nullptr)
    for (int idx = threadIdx.x; idx < n_rows; idx += kThreads)
      p.lse[(int64_t)(t0 + idx / HB) * p.Hq + h0 + idx % HB] = -INFINITY;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void dense_fwd_kernel(DenseFwdParams p) {
  using G = Geo<T, D>;
  __shared__ __attribute__((aligned(16))) T smem[2 * G::kStage];

  // ---- work item: XCD-aware remap, then (KV head, head chunk, virtual tile)
  const int per_xcd = gridDim.x / kXcds;
  const int L = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (L >= p.n_work) return;
  const int VT = p.n_vtiles;
  const int hc = L / VT;
  const int v = VT - 1 - (L - hc * VT);
  const int g = hc / p.n_chunks;
  const int chunk = hc - g * p.n_chunks;
  const int TQ = p.tile_tokens;

  // segment s holding virtual tile v: A(s) = floor(bound(s) / TQ) + s, A(s) <= v < A(s+1)
  int lo = 0, hi = p.n_docs + 2;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_bound(p, mid) / TQ + mid <= v) lo = mid; else hi = mid;
  }
  const int seg_start = seg_bound(p, lo);
  const int seg_end = seg_bound(p, lo + 1);
  const int t0 = seg_start + (v - (seg_start / TQ + lo)) * TQ;
  if (t0 >= seg_end) return;
  const int t_end = min(t0 + TQ, seg_end);
  const int HB = 1 << p.hb_shift;
  const int h0 = g * p.G + chunk * HB;
  if (lo == 0 || lo == p.n_docs + 1) {
    write_padding<T, D>(p, t0, t_end, h0, HB);
    return;
  }

  // ---- lane geometry
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;   // query column of this lane
  const int h2 = lane >> 5;  // half-wave
  const int TW = 32 >> p.hb_shift;
  const int tw0 = t0 + wave * TW;
  const int tw1 = min(tw0 + TW, t_end) - 1;
  const int tq = tw0 + (n >> p.hb_shift);
  const int hq = h0 + (n & (HB - 1));
  const int W = p.window;
  const int s_d = seg_start;
  const int k_lo = W ? max(s_d, t0 - W + 1) : s_d;
  const int k_hi = t_end;
  const int n_tiles = (k_hi - k_lo + kBN - 1) / kBN;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers
  QFragT<T> qf[G::kQFrags];
  {
    const T* qb = (const T*)p.q + (int64_t)min(tq, t_end - 1) * p.q_st + (int64_t)hq * p.q_sh;
    if constexpr (G::kBf16) {
#pragma unroll
      for (int s = 0; s < G::kQFrags; ++s) qf[s] = *(const bf16x8*)(qb + 16 * s + 8 * h2);
    } else {
#pragma unroll
      for (int s = 0; s < G::kQFrags; ++s) qf[s] = qb[2 * s + h2];
    }
  }

  // ---- K/V staging through registers.  Rows past the tile's last query are clamped to the
  // last valid row (always in bounds); every such key lies after every valid query of the
  // tile, so it is masked to -inf and contributes exactly zero.
  const T* kbase = (const T*)p.k + (int64_t)g * p.k_sh;
  const T* vbase = (const T*)p.v + (int64_t)g * p.v_sh;
  u32x4 kreg[G::kLoads], vreg[G::kLoads];
  auto stage_load = [&](int kb) {
    const T* kt = kbase + (int64_t)kb * p.k_st;  // wave-uniform tile bases
    const T* vt = vbase + (int64_t)kb * p.v_st;
    const int lim = k_hi - 1 - kb;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int row = min(c / G::kChunksPerRow, lim);
      const int col = (c % G::kChunksPerRow) * G::kChunk;
      kreg[i] = *(const u32x4*)(kt + (int)(row * p.k_st) + col);
      vreg[i] = *(const u32x4*)(vt + (int)(row * p.v_st) + col);
    }
  };
  auto stage_store = [&](int buf) {
    T* Ks = smem + buf * G::kStage;
    T* Vs = Ks + G::kKElems;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int row = c / G::kChunksPerRow;
      const int col = (c % G::kChunksPerRow) * G::kChunk;
      if constexpr (G::kBf16) {
        *(u32x4*)(Ks + row * G::kKPitch + col) = kreg[i];
      } else {
        float* kd = (float*)(Ks + row * G::kKPitch + col);  // odd pitch: scalar stores
        kd[0] = __uint_as_float(kreg[i][0]);
        kd[1] = __uint_as_float(kreg[i][1]);
        kd[2] = __uint_as_float(kreg[i][2]);
        kd[3] = __uint_as_float(kreg[i][3]);
      }
      *(u32x4*)(Vs + row * G::kVPitch + col) = vreg[i];
    }
  };

  f32x16 o[G::kDBlocks];
#pragma unroll
  for (int d = 0; d < G::kDBlocks; ++d) o[d] = f32x16{};
  float mref = -INFINITY;  // reference max of the scores in log2 units (scale folded in)
  float l = 0.f;           // running sum of exp2(s * c2 - mref) over this half-wave's keys
  const float c2 = p.c2;

  if (n_tiles > 0) {
    stage_load(k_lo);
    stage_store(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int kb = k_lo + j * kBN;
    if (j + 1 < n_tiles) stage_load(kb + kBN);
    const T* Ks = smem + (j & 1) * G::kStage;
    const T* Vs = Ks + G::kKElems;
    const bool active = (tw0 <= tw1) && (kb <= tw1) && (W == 0 || kb + kBN - 1 > tw0 - W);
    if (active) {
      // S^T for two 32-key blocks
      f32x16 sc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        sc[blk] = f32x16{};
        const T* krow = Ks + (32 * blk + n) * G::kKPitch;
        if constexpr (G::kBf16) {
#pragma unroll
          for (int s = 0; s < G::kQFrags; ++s)
            sc[blk] = mfma_bf16_32x32x16(*(const bf16x8*)(krow + 16 * s + 8 * h2), qf[s], sc[blk]);
        } else {
#pragma unroll
          for (int s = 0; s < G::kQFrags; ++s)
            sc[blk] = mfma_f32_32x32x2(krow[2 * s + h2], qf[s], sc[blk]);
        }
      }
      // mask only tiles crossing the diagonal or the window edge of this wave's tokens
      const bool need_mask = (kb + kBN - 1 > tw0) || (W != 0 && kb <= tw1 - W);
      if (need_mask) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int key = kb + 32 * blk + 8 * (a >> 2) + 4 * h2 + (a & 3);
            const bool ok = key <= tq && (W == 0 || tq - key < W);
            sc[blk][a] = ok ? sc[blk][a] : -INFINITY;
          }
      }
      // online softmax (base 2, scale folded into c2)
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sc[blk][a]);
      mx = half_swap_max(mx) * c2;
      // lazy rescale: the reference moves only when a score exceeds it by more than 2^8, so
      // probabilities stay <= 256 and most tiles skip rescaling O (exact either way)
      const bool move = mx > mref + kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float mnew = move ? mx : mref;
        // lanes that keep their reference scale by exactly 1 (also when it is still -inf)
        const float alpha = move ? fast_exp2(mref - mnew) : 1.f;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < G::kDBlocks; ++d) o[d] *= alpha;
        mref = mnew;
      }
      const float mu = mref == -INFINITY ? 0.f : mref;
      float rs = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const float e = fast_exp2(__builtin_fmaf(sc[blk][a], c2, -mu));
          sc[blk][a] = e;
          rs += e;
        }
      l += rs;

      // O^T += V^T P^T
      if constexpr (G::kBf16) {
        const int j16 = lane & 15;
        const int dh = (lane >> 4) & 1;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            f32x8 pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = sc[blk][8 * s + e];
            const bf16x8 pb = cvt_bf16x8(pf);
            const int r0 = 32 * blk + 16 * s + 4 * h2 + (j16 >> 2);
            const __bf16* v0 = (const __bf16*)Vs + r0 * G::kVPitch + 16 * dh + 4 * (j16 & 3);
            const __bf16* v1 = v0 + 8 * G::kVPitch;
#pragma unroll
            for (int d = 0; d < G::kDBlocks; ++d) {
              const bf16x4 lo4 = lds_read_tr4(v0 + 32 * d);
              const bf16x4 hi4 = lds_read_tr4(v1 + 32 * d);
              const bf16x8 va = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
              o[d] = mfma_bf16_32x32x16(va, pb, o[d]);
            }
          }
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int key = 32 * blk + 8 * (u >> 2) + 4 * h2 + (u & 3);
            const float* vr = (const float*)Vs + key * G::kVPitch + n;
#pragma unroll
            for (int d = 0; d < G::kDBlocks; ++d) o[d] = mfma_f32_32x32x2(vr[32 * d], sc[blk][u], o[d]);
          }
      }
    }
    if (j + 1 < n_tiles) stage_store((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: combine half-wave sums, fold in the sink, normalise once, store
  const float lt = half_swap_sum(l);
  const float m2 = mref;  // reference max in log2 units (-inf if nothing was visible)
  float inv, lse_v;
  if (p.sinks != nullptr) {
    const float s2 = p.sinks[hq] * kLog2e;
    const float mm = fmaxf(m2, s2);
    const float corr = fast_exp2(m2 - mm);
    const float lf = lt * corr + fast_exp2(s2 - mm);
    inv = corr / lf;
    lse_v = (mm + __builtin_amdgcn_logf(lf)) * kLn2;
  } else {
    inv = 1.f / lt;
    lse_v = (m2 + __builtin_amdgcn_logf(lt)) * kLn2;
  }
  if (tq < t_end) {
    T* ob = (T*)p.out + (int64_t)tq * p.o_st + (int64_t)hq * p.o_sh;
#pragma unroll
    for (int d = 0; d < G::kDBlocks; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = o[d][4 * i + e] * inv;
        T* dst = ob + 32 * d + 8 * i + 4 * h2;
        if constexpr (G::kBf16) *(bf16x4*)dst = cvt_bf16x4(r);
        else *(f32x4*)dst = r;
      }
    if (p.lse != nullptr && h2 == 0) p.lse[(int64_t)tq * p.Hq + hq] = lse_v;
  }
}

template <typename T, int D>
hipError_t launch_one(const DenseFwdParams& p, hipStream_t stream) {
  const int64_t grid = dense_fwd_grid(p);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((dense_fwd_kernel<T, D>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
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
  p.c2 = p.scale * 1.4426950408889634f;
}

int64_t dense_fwd_grid(const DenseFwdParams& p) {
  if (p.T <= 0) return 0;
  const int64_t w = (int64_t)p.n_work;
  return (w + kXcds - 1) / kXcds * kXcds;
}

hipError_t dense_fwd_launch(const DenseFwdParams& p, Dtype dt, int D, hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (D == 128) return launch_one<__bf16, 128>(p, stream);
    if (D == 64) return launch_one<__bf16, 64>(p, stream);
  } else {
    if (D == 128) return launch_one<float, 128>(p, stream);
    if (D == 64) return launch_one<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace swa
