// Device helpers shared by the dense forward and backward kernels (gfx950): packed-document
// tile decoding (segment search over cu_seqlens, XCD-aware block placement), the per-lane
// query-column geometry of a 128-column workgroup, the causal / window mask of one 64-key
// tile in the transposed-score layout (lane = query column, rows = keys), and the
// LDS-staged bf16 store of a wave's 32 output columns.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;    // keys per tile
constexpr int kXcds = 8;   // MI355X: workgroups are dealt round-robin to 8 XCDs
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format, raw access
// s_waitcnt vmcnt(0) with expcnt / lgkmcnt unconstrained
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
// s_waitcnt vmcnt(N) with expcnt / lgkmcnt unconstrained (vector loads complete in order)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// workgroup barrier that does not drain outstanding vector-memory loads
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Segment boundaries: segment 0 = [0, cu[0]) and segment n+1 = [cu[n], T) are padding,
// segment s in 1..n is document s-1.  Entries are clamped to [0, T].
__device__ __forceinline__ int seg_bound(const DenseFwdParams& p, int s) {
  if (s <= 0) return 0;
  if (s > p.n_docs + 1 || p.cu_seqlens == nullptr) return s > p.n_docs + 1 ? p.T : 0;
  int x = p.cu_seqlens[s - 1];
  return x < 0 ? 0 : (x > p.T ? p.T : x);
}

// The workgroup's query tile: tokens [t0, t_end) of segment `seg`, heads [h0, h0 + HB).
struct Tile {
  int g, h0, HB, t0, t_end, seg_start, seg;
  bool padding;
};

// Decodes blockIdx into a tile; returns false for idle blocks.
__device__ __forceinline__ bool decode_tile(const DenseFwdParams& p, Tile& w) {
  // XCD-aware remap: workgroups reach the XCDs round-robin (x = blockIdx % 8, j = blockIdx / 8
  // is the order within an XCD) and a head chunk's tiles stay on the XCDs whose L2 holds its
  // K/V.  Under a full causal mask, when 8 / n_hc XCDs share a head chunk they deal its tiles
  // round robin, so each gets the same mix of heavy and light tiles; otherwise (and for
  // windows, whose tiles weigh about the same) each XCD takes a contiguous range.
  const int VT = p.n_vtiles;
  const int n_hc = p.Hkv * p.n_chunks;
  const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  int hc, r;
  if (p.window == 0 && n_hc < kXcds && kXcds % n_hc == 0) {
    const int m = kXcds / n_hc;
    hc = x % n_hc;
    r = j * m + x / n_hc;
    if (r >= VT) return false;
  } else {
    const int L = x * (gridDim.x / kXcds) + j;
    if (L >= p.n_work) return false;
    hc = L / VT;
    r = L - hc * VT;
  }
  const int v = VT - 1 - r;  // each document's tiles last-first
  w.g = hc / p.n_chunks;
  const int chunk = hc - w.g * p.n_chunks;
  const int TQ = p.tile_tokens;
  // segment s holding virtual tile v: A(s) = floor(bound(s) / TQ) + s, A(s) <= v < A(s+1).
  // A is increasing in s, so the segment is the number of s >= 1 with A(s) <= v: with at
  // most 64 boundaries lane s loads bound(s) and one ballot counts them (one memory round
  // trip); otherwise a binary search.
  int lo, seg_start, seg_end;
  if (p.n_docs + 3 <= 64) {  // lanes 0 .. n_docs + 2 hold every boundary
    const int s = threadIdx.x & 63;
    const int b = seg_bound(p, s);
    lo = __builtin_amdgcn_readfirstlane(
        __builtin_popcountll(__builtin_amdgcn_ballot_w64(s >= 1 && s <= p.n_docs + 1 && b < (v - s + 1) * TQ)));
    seg_start = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(b, lo));
    seg_end = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(b, lo + 1));
  } else {
    lo = 0;
    int hi = p.n_docs + 2;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seg_bound(p, mid) / TQ + mid <= v) lo = mid; else hi = mid;
    }
    seg_start = seg_bound(p, lo);
    seg_end = seg_bound(p, lo + 1);
  }
  w.seg = lo;
  w.seg_start = seg_start;
  if (seg_start / TQ + lo > v) return false;  // only with decreasing cu_seqlens: no tile
  w.t0 = w.seg_start + (v - (w.seg_start / TQ + lo)) * TQ;
  if (w.t0 >= seg_end) return false;
  w.t_end = min(w.t0 + TQ, seg_end);
  w.HB = 1 << p.hb_shift;
  w.h0 = w.g * p.G + chunk * w.HB;
  w.padding = (lo == 0 || lo == p.n_docs + 1);
  return true;
}

// Per-lane query geometry inside the tile.
struct Cols {
  int wave, lane, n, h2, tw0, tw1, tq, hq, k_lo, k_hi, n_tiles, W;
};

__device__ __forceinline__ Cols make_cols(const DenseFwdParams& p, const Tile& w) {
  Cols c;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.n = c.lane & 31;   // query column of this lane
  c.h2 = c.lane >> 5;  // half-wave
  const int TW = 32 >> p.hb_shift;
  c.tw0 = w.t0 + c.wave * TW;
  c.tw1 = min(c.tw0 + TW, w.t_end) - 1;  // last valid token of this wave (< tw0 if none)
  c.tq = c.tw0 + (c.n >> p.hb_shift);
  c.hq = w.h0 + (c.n & (w.HB - 1));
  c.W = p.window;
  c.k_lo = c.W ? max(w.seg_start, w.t0 - c.W + 1) : w.seg_start;
  c.k_hi = w.t_end;
  c.n_tiles = (c.k_hi - c.k_lo + kBN - 1) / kBN;
  return c;
}

// Does the wave see any key of the tile starting at kb?  Does the tile need masking?
__device__ __forceinline__ bool tile_active(const Cols& c, int kb) {
  return (c.tw0 <= c.tw1) && (kb <= c.tw1) && (c.W == 0 || kb + kBN - 1 > c.tw0 - c.W);
}
__device__ __forceinline__ bool tile_needs_mask(const Cols& c, int kb) {
  return (kb + kBN - 1 > c.tw0) || (c.W != 0 && kb <= c.tw1 - c.W);
}

// Masks keys outside [doc start, query] and outside the window (tiles that straddle the
// diagonal or the window edge only).
__device__ __forceinline__ void mask_tile(f32x16 (&sc)[2], int kb, const Cols& c) {
  // allowed keys of this lane's query: kb + off with lo <= off <= lo + range, where
  // off = 32 blk + 8 (a / 4) + 4 h2 + a % 4; the 4 h2 term is folded into lo so every
  // comparison is against an immediate: one subtract, one unsigned compare, one select
  const int tq4 = opaque(c.tq - 4 * c.h2);  // recomputed per use, nothing hoisted out of the loop
  const int lo = c.W ? tq4 - c.W + 1 - kb : -(1 << 30);
  const unsigned range = (unsigned)(tq4 - kb - lo);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int off = 32 * blk + 8 * (a >> 2) + (a & 3);
      sc[blk][a] = (unsigned)(off - lo) <= range ? sc[blk][a] : -INFINITY;
    }
}

// bf16 output of one wave through LDS, scaled by `mult`.  The wave's 32 query columns are
// 32 rows of D values; lane (n, h2) holds dims 32 d + 8 i + 4 h2 + (0..3) of column n.  Each
// lane writes its bf16 quads into a wave-private image of 64 D bytes (column n at n * 2D
// bytes, 16-byte unit u at u ^ key(n) so a half-wave's writes spread over the banks), then
// reads it back 16 bytes per lane: one store instruction writes 64 consecutive units = whole
// rows of 512 / D adjacent columns, and columns with adjacent heads of one token are adjacent
// in memory.  Direct stores from the accumulator layout would touch 32 rows with 8 bytes each
// per instruction.
template <int D>
__device__ __forceinline__ int out_key(int n) {
  if constexpr (D == 64) return (n >> 1) & 7;
  else return n & 15;
}
template <int D>
__device__ __forceinline__ void store_out_bf16(void* out, int64_t st, int64_t sh, const Tile& w, const Cols& c,
                                               int hb_shift, float mult, const f32x16 (&o)[D / 32], char* img) {
  constexpr int U = D / 8;           // 16-byte units per column
  constexpr int kCols = 512 / D;     // columns per store instruction
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = o[d][4 * i + e] * mult;
      *(bf16x4*)(img + c.n * (2 * D) + (((4 * d + i) ^ out_key<D>(c.n)) << 4) + 8 * c.h2) = cvt_bf16x4(r);
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own writes, in order
  const int u = c.lane % U;
#pragma unroll
  for (int k = 0; k < 32 / kCols; ++k) {
    const int n = k * kCols + c.lane / U;
    const u32x4 val = *(const u32x4*)(img + n * (2 * D) + ((u ^ out_key<D>(n)) << 4));
    const int t = c.tw0 + (n >> hb_shift);
    if (t <= c.tw1) *(u32x4*)((__bf16*)out + (int64_t)t * st + (int64_t)(w.h0 + (n & (w.HB - 1))) * sh + 8 * u) = val;
  }
}

}  // namespace
}  // namespace swa
