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

// Work item j of XCD x (the j-th item that XCD takes; per_xcd items each) -> head chunk hc and
// rank r of its query tiles (r = 0 is taken first).  Returns false past the end.  Workgroups reach
// the XCDs round-robin, and a head chunk's tiles stay on the XCDs whose L2 holds its K/V.  Under a
// full causal mask, when 8 / n_hc XCDs share a head chunk they deal its ranks round robin, so each
// gets the same mix of heavy and light tiles; otherwise (and for windows, whose tiles weigh about
// the same) each XCD takes a contiguous range.
__device__ __forceinline__ bool item_rank(const DenseFwdParams& p, int x, int j, int per_xcd, int& hc, int& r) {
  const int VT = p.n_vtiles;
  const int n_hc = p.Hkv * p.n_chunks;
  if (p.window == 0 && n_hc < kXcds && kXcds % n_hc == 0) {
    const int m = kXcds / n_hc;
    hc = x % n_hc;
    r = j * m + x / n_hc;
    return r < VT;
  }
  const int L = x * per_xcd + j;
  if (L >= p.n_work) return false;
  hc = (int)(((uint64_t)(uint32_t)L * p.vt_magic) >> p.vt_shift);  // L / VT
  r = L - hc * VT;
  return true;
}

// Virtual tile v of head chunk hc -> the workgroup's query tile; false for idle virtual tiles.
// `bnd` is this lane's segment boundary bound(lane) when n_docs + 3 <= 64 (else unused).
__device__ __forceinline__ bool vtile_to_tile(const DenseFwdParams& p, int hc, int v, int bnd, Tile& w) {
  w.g = p.n_chunks == 1 ? hc : hc / p.n_chunks;  // one chunk per KV head unless G has an odd factor
  const int chunk = hc - w.g * p.n_chunks;
  const int lg = 7 - p.hb_shift;  // TQ = 128 >> hb_shift tokens per tile: divisions by TQ are shifts
  const int TQ = 1 << lg;
  // segment s holding virtual tile v: A(s) = floor(bound(s) / TQ) + s, A(s) <= v < A(s+1).
  // A is increasing in s, so the segment is the number of s >= 1 with A(s) <= v: with at
  // most 64 boundaries lane s holds bound(s) and one ballot counts them; otherwise a binary
  // search.
  int lo, seg_start, seg_end;
  if (p.n_docs + 3 <= 64) {  // lanes 0 .. n_docs + 2 hold every boundary
    const int s = threadIdx.x & 63;
    lo = __builtin_amdgcn_readfirstlane(
        __builtin_popcountll(__builtin_amdgcn_ballot_w64(s >= 1 && s <= p.n_docs + 1 && bnd < (v - s + 1) * TQ)));
    seg_start = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(bnd, lo));
    seg_end = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(bnd, lo + 1));
  } else {
    lo = 0;
    int hi = p.n_docs + 2;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((seg_bound(p, mid) >> lg) + mid <= v) lo = mid; else hi = mid;
    }
    seg_start = seg_bound(p, lo);
    seg_end = seg_bound(p, lo + 1);
  }
  w.seg = lo;
  w.seg_start = seg_start;
  if ((seg_start >> lg) + lo > v) return false;  // only with decreasing cu_seqlens: no tile
  w.t0 = w.seg_start + (v - ((w.seg_start >> lg) + lo)) * TQ;
  if (w.t0 >= seg_end) return false;
  w.t_end = min(w.t0 + TQ, seg_end);
  w.HB = 1 << p.hb_shift;
  w.h0 = w.g * p.G + chunk * w.HB;
  w.padding = (lo == 0 || lo == p.n_docs + 1);
  return true;
}

// Heaviest-first ranks under a full causal mask.  A query tile's weight is its number of 64-key
// tiles, ceil((t_end - document start) / 64), non-decreasing along a document; rank r takes the
// tiles by weight, heaviest first, ties in document order and then along the document, so the
// tail of a launch is made of light tiles from every document.  With at most 32 documents of at
// most 64 * 64 tokens (at most 64 weight levels): lane x - 1 counts the tiles of weight >= x over
// all documents in one uniform pass over them, one ballot finds the level of rank r, and a prefix
// sum of the documents' counts at that level finds the document; no search, no memory beyond the
// boundaries already in `bnd` (bound(lane)).  Padding segments come after every document, idle
// ranks last.  Returns 1 with the tile in w, 0 for an idle rank, -1 when the documents do not fit
// (the caller then keeps document order).
__device__ __forceinline__ int heavy_first_tile(const DenseFwdParams& p, int hc, int r, int bnd, Tile& w) {
  const int lane = threadIdx.x & 63;
  const int nd = p.n_docs;
  const int lg = 7 - p.hb_shift;  // log2 of the tile tokens (128 >> hb_shift)
  const int TQ = 1 << lg;
  const int nxt = __shfl_down(bnd, 1);  // bound(lane + 1)
  const int len_v = nxt - bnd;          // segment `lane`: [bound(lane), bound(lane + 1))
  // lane x - 1 counts the tiles of weight >= x: a document of length L > 64 (x - 1) has its tiles
  // from index 64 (x - 1) / TQ on at that weight or above
  const int need = 64 * lane;
  int cnt = 0, maxlen = 0, minlen = 0;
  for (int s = 1; s <= nd; ++s) {
    const int L = __builtin_amdgcn_readlane(len_v, s);
    maxlen = max(maxlen, L);
    minlen = min(minlen, L);
    const int nt = (L + TQ - 1) >> lg;
    cnt += L > need ? nt - (need >> lg) : 0;
  }
  if (maxlen > 64 * 64 || minlen < 0) return -1;
  const int n_real = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(cnt, 0));
  int seg, i;
  if (r < n_real) {
    const int xs = __builtin_popcountll(__builtin_amdgcn_ballot_w64(cnt > r));  // weight level of rank r
    const int above = xs < 64 ? __builtin_amdgcn_readlane(cnt, xs) : 0;        // tiles of weight > xs
    const int j = r - above;                                                    // rank within the level
    // per document (lane s): its tiles of weight >= xs and >= xs + 1
    const bool real = lane >= 1 && lane <= nd;
    const int nt_l = (len_v + TQ - 1) >> lg;
    const int n1 = 64 * (xs - 1), n2 = 64 * xs;
    const int ge1 = real && len_v > n1 ? nt_l - (n1 >> lg) : 0;
    const int ge2 = real && len_v > n2 ? nt_l - (n2 >> lg) : 0;
    const int eq = ge1 - ge2;
    int incl = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const uint64_t owner = __builtin_amdgcn_ballot_w64(eq > 0 && j >= incl - eq && j < incl);
    if (owner == 0) return 0;  // unreachable: rank r < n_real always has an owner
    seg = __builtin_amdgcn_readfirstlane(__builtin_ctzll(owner));
    const int k = j - (__builtin_amdgcn_readlane(incl, seg) - __builtin_amdgcn_readlane(eq, seg));
    i = __builtin_amdgcn_readlane(nt_l, seg) - __builtin_amdgcn_readlane(ge1, seg) + k;
    w.padding = false;
  } else {
    const int rp = r - n_real;
    const int nt0 = (__builtin_amdgcn_readlane(len_v, 0) + TQ - 1) >> lg;
    const int ntn = (__builtin_amdgcn_readlane(len_v, nd + 1) + TQ - 1) >> lg;
    if (rp < nt0) {
      seg = 0;
      i = rp;
    } else if (rp - nt0 < ntn) {
      seg = nd + 1;
      i = rp - nt0;
    } else {
      return 0;
    }
    w.padding = true;
  }
  w.g = p.n_chunks == 1 ? hc : hc / p.n_chunks;
  const int chunk = hc - w.g * p.n_chunks;
  w.seg = seg;
  w.seg_start = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(bnd, seg));
  const int seg_end = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(nxt, seg));
  w.t0 = w.seg_start + i * TQ;
  w.t_end = min(w.t0 + TQ, seg_end);
  w.HB = 1 << p.hb_shift;
  w.h0 = w.g * p.G + chunk * w.HB;
  return 1;
}

// Decodes blockIdx into a tile (one tile per workgroup); returns false for idle blocks.  With
// HEAVY_FIRST (the forward), under a full causal mask with few documents and fewer head chunks
// than XCDs (several XCDs deal one head chunk's ranks round robin, so no XCD keeps a document's
// tiles together anyway), the ranks go heaviest first over all documents (heavy_first_tile):
// 2-3.5 % faster on the head_dim-256 forward.  Otherwise each document's tiles run last-first
// (heaviest first within it), documents from the last, which keeps an XCD's concurrent tiles on
// one or two documents' K/V: with one head chunk per XCD the heaviest-first order measured within
// 1 % either way on the head_dim-128 forward and 2 % slower in the dq kernel, which always keeps
// document order.
template <bool HEAVY_FIRST>
__device__ __forceinline__ bool decode_tile(const DenseFwdParams& p, Tile& w) {
  int hc, r;
  if (!item_rank(p, blockIdx.x % kXcds, blockIdx.x / kXcds, gridDim.x / kXcds, hc, r)) return false;
  const int bnd = p.n_docs + 3 <= 64 ? seg_bound(p, threadIdx.x & 63) : 0;
  if (HEAVY_FIRST && p.window == 0 && p.Hkv * p.n_chunks < kXcds && p.n_docs <= 32 && p.cu_seqlens != nullptr) {
    const int res = heavy_first_tile(p, hc, r, bnd, w);
    if (res >= 0) return res == 1;
  }
  return vtile_to_tile(p, hc, p.n_vtiles - 1 - r, bnd, w);
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

// The lane-dependent fields of `c` recomputed from an opaque lane id.  Code after the key loop
// uses this copy, so the loop does not hold those values in registers for it.
__device__ __forceinline__ Cols fresh_lane_cols(const Cols& c, int hb_shift, const Tile& w) {
  Cols r = c;
  r.lane = opaque((int)threadIdx.x & 63);
  r.n = r.lane & 31;
  r.h2 = r.lane >> 5;
  r.tq = c.tw0 + (r.n >> hb_shift);
  r.hq = w.h0 + (r.n & (w.HB - 1));
  return r;
}

// Does the wave see any key of the tile starting at kb?  Does the tile need masking?
__device__ __forceinline__ bool tile_active(const Cols& c, int kb) {
  return (c.tw0 <= c.tw1) && (kb <= c.tw1) && (c.W == 0 || kb + kBN - 1 > c.tw0 - c.W);
}
__device__ __forceinline__ bool tile_needs_mask(const Cols& c, int kb) {
  return (kb + kBN - 1 > c.tw0) || (c.W != 0 && kb <= c.tw1 - c.W);
}

// Masks keys outside [doc start, query] and outside the window (tiles that straddle the
// diagonal or the window edge only).  Each 32-key block is masked only when some key of it
// lies after the wave's first query or before its last query's window (a uniform test): in a
// window-edge or diagonal tile the other block is usually inside every query's range.
template <int NB = 2>  // NB = 1: block 0 only (block 1 is not computed)
__device__ __forceinline__ void mask_tile(f32x16 (&sc)[2], int kb, const Cols& c) {
  // allowed keys of this lane's query: kb + off with lo <= off <= lo + range, where
  // off = 32 blk + 8 (a / 4) + 4 h2 + a % 4; the 4 h2 term is folded into lo so every
  // comparison is against an immediate: one subtract, one unsigned compare, one select
  const int tq4 = opaque(c.tq - 4 * c.h2);  // recomputed per use, nothing hoisted out of the loop
  const int lo = c.W ? tq4 - c.W + 1 - kb : -(1 << 30);
  const unsigned range = (unsigned)(tq4 - kb - lo);
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int b0 = kb + 32 * blk;
    if (!(b0 + 31 > c.tw0 || (c.W != 0 && b0 <= c.tw1 - c.W))) continue;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int off = 32 * blk + 8 * (a >> 2) + (a & 3);
      sc[blk][a] = (unsigned)(off - lo) <= range ? sc[blk][a] : -INFINITY;
    }
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
  // Store k writes column n = k kCols + n0 (n0 = lane / U < kCols).  The bits of n0 and of
  // k kCols do not overlap, so the token (n >> hb_shift) and head (n & (HB - 1)) offsets of n
  // are sums of a lane part (from n0) and a uniform part (from k).  The stores are raw buffer
  // stores from the wave's first (token, head) row: the lane part is a 32-bit byte offset
  // formed once, the uniform part the scalar offset of each store, so no store needs a 64-bit
  // address (both parts stay below 2^31 bytes: token and head strides are below 2^24 elements).
  const int u = c.lane % U;
  const int n0 = opaque(c.lane / U);  // the columns n are not shared with the loop's addresses
  const int t_lane = n0 >> hb_shift;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((__bf16*)out + (int64_t)c.tw0 * st + (int64_t)w.h0 * sh), (short)0, -1, kBufferWord3);
  const int vlane = ((int)st * t_lane + (int)sh * (n0 & (w.HB - 1)) + 8 * u) * 2;
  const int t_last = c.tw1 - c.tw0 - t_lane;  // uniform token offsets beyond it are past the end
#pragma unroll
  for (int k = 0; k < 32 / kCols; ++k) {
    const int n = k * kCols + n0;
    const u32x4 val = *(const u32x4*)(img + n * (2 * D) + ((u ^ out_key<D>(n)) << 4));
    const int tk = (k * kCols) >> hb_shift, hk = (k * kCols) & (w.HB - 1);
    if (tk <= t_last)
      __builtin_amdgcn_raw_buffer_store_b128(val, rs, vlane, __builtin_amdgcn_readfirstlane(((int)st * tk + (int)sh * hk) * 2), 0);
  }
}

}  // namespace
}  // namespace swa
