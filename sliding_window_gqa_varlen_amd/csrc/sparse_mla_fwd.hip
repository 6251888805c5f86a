// Sparse MLA forward for gfx950: each query token attends to the key rows its top-k index
// row names; a key is latent[idx] (512) + k_pe[idx] (64) and the value is latent[idx].  The
// NoPE variant (no rotary part: q is 512 wide, k_pe has no columns) is the same kernel
// instantiated with DR = 0.
// Operation: sparse_mla / MistralLarge4Attention._sparse_forward on the
// nemo_automodel.components.models.mistral_large4.attention page (-1 = empty slot,
// empty query rows are zero).
//
// Design (one workgroup = 8 waves = one query token x 128 heads):
//  * Waves w and w+4 (same SIMD) own the same 32 heads (the N dimension of
//    v_mfma_f32_32x32x16_bf16).  Wave w contracts q.k over the even 16-coordinate
//    k-steps, wave w+4 over the odd ones; the two partial score tiles are swapped through LDS and summed
//    (a + b is commutative, so both waves hold bit-identical scores).  Each wave then
//    accumulates half of the 512 output coordinates.  Per wave: 72 Q registers and 128
//    fp32 accumulators, two waves per SIMD, equal MFMA work on every SIMD.
//  * The index row is first compacted in LDS to the slots that are valid (in range,
//    causal, same document), so invalid slots cost neither gather bytes nor MFMA work.
//  * Chunks of 32 compacted slots are gathered straight into LDS with
//    buffer_load ... lds (no register staging): 32 rows x 72 16-byte units
//    (64 latent + 8 rotary), unit index swizzled per row so the row reads of the QK^T
//    operand and the ds_read_b64_tr_b16 reads of the PV operand avoid bank conflicts.
//    Three buffers: the gather of chunk c+2 is issued right after the score exchange of
//    chunk c, and the loop is unrolled by three so every LDS read names its buffer
//    statically (no conservative wait on the gathers in flight).
//  * S^T = KV Q^T (slots = M, heads = N); online softmax with lazy rescaling (the
//    reference maximum moves only when a score exceeds it by more than 2^8, which keeps
//    probabilities <= 256 and the result exact); O^T += latent^T P^T.
#include "device_common.h"
#include "launch.h"


namespace swa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kHeadsPerBlock = 128;
constexpr int kSlots = 32;                          // slots per chunk
constexpr int kLatUnits = 64;                       // 16-byte latent units per row
constexpr int kRopeUnits = 8;                       // 16-byte rotary units per row
constexpr int kLatRegion = kSlots * kLatUnits;      // 2048 units: latent rows
constexpr int kLatDma = kLatRegion / 64 / kWaves;   // 4 x 16-byte gathers per lane
constexpr int kRopeDma = kSlots * kRopeUnits * 4 / 64 / kWaves;  // 2 x 4-byte gathers per lane
// per rotary width DR (64, or 0 for the NoPE variant): chunk size in 16-byte units (+ 256
// units of rotary rows), gathers per wave (identical on every wave), q k-steps per wave
constexpr int chunk_units(int dr) { return kLatRegion + (dr ? kSlots * kRopeUnits : 0); }
constexpr int dma_per_wave(int dr) { return kLatDma + (dr ? kRopeDma : 0); }
constexpr int q_frags(int dr) { return (512 + dr) / 32; }
constexpr int kSeg = 2048;                          // index slots compacted at a time
constexpr int kTokenRun = 64;                       // consecutive tokens per XCD turn
constexpr int kSlotsPerThread = kSeg / kThreads;    // 4
constexpr int kDBlocks = 8;                         // 256 output coordinates per wave / 32
constexpr float kRescaleLog2 = 8.f;                 // lazy-rescale threshold (log2 units)
constexpr float kLazyMax = 256.f;                   // 2^kRescaleLog2: the fast path's bound on a lane's sum
constexpr int kQAhead = 3;         // QK^T fragments read ahead of their MFMA
constexpr int kPvAhead = 2;       // PV fragments read ahead of their MFMA
static_assert(kLatRegion % (64 * kWaves) == 0 && (kSlots * kRopeUnits * 4) % (64 * kWaves) == 0,
              "every wave issues the same number of gathers");

// LDS swizzles (64 banks of 4 bytes; 16 lanes x 16 bytes per cycle).  Latent rows are 64
// 16-byte units; a row read of the QK operand touches one unit of 16 consecutive rows and a
// transposed read of the PV operand touches 4 consecutive units of 4 consecutive rows.  XOR-ing
// the low 4 unit bits with rot(r) = ((r & 3) << 2) | ((r >> 2) & 3) spreads both over all 16
// unit slots.  Rotary rows are 8 units; XOR with (r >> 1) & 7 spreads 16 rows of one unit.
__device__ __forceinline__ int lat_key(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int rope_key(int r) { return (r >> 1) & 7; }

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format, raw access

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt unconstrained
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) with vmcnt / expcnt unconstrained
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// workgroup barrier that does not drain outstanding vector-memory loads
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Lane {
  int wave, lane, n, h2, j16, dh, half, hg;
};

// Gather chunk `chunk` (32 compacted slots) into `buf`: latent unit u of row r at
// r * 64 + (u & 48) + ((u & 15) ^ lat_key(r)), rotary unit u of row r (as four 4-byte pieces)
// at 2048 + r * 8 + (u ^ rope_key(r)).
// Slots past the compacted count (and whole chunks past the end) read the token's own row.
template <int DR>
__device__ __forceinline__ void gather_chunk(const SparseMlaParams& p, const int32_t* s_idx, int nv, int chunk,
                                             int t, u32x4* buf, const Lane& L) {
  // MUBUF LDS DMA (buffer_load ... lds): byte offsets from the tensor bases (the host
  // checks that both tensors fit 32-bit offsets).  Unlike the FLAT form, pending buffer
  // transfers leave the LDS read counters exact, so LDS reads below wait only for
  // themselves.
  const __amdgpu_buffer_rsrc_t lat = __builtin_amdgcn_make_buffer_rsrc((void*)p.latent, (short)0, -1, kBufferWord3);
  const uint32_t lat_stb = (uint32_t)p.lat_st * 2u;
  // recompute the per-lane gather plan here instead of keeping it live across the loop
  int lane = L.lane;
  asm volatile("" : "+v"(lane));
  // lane l < 32 reads the index of slot row l once; each transfer takes its rows by readlane
  const int slot = chunk * kSlots + (lane & 31);
  const int my_idx = slot < nv ? s_idx[slot] : t;
  uint32_t lane16 = (uint32_t)lane * 16u;
  asm volatile("" : "+v"(lane16));  // kept as one value: each transfer's offset is then one XOR
#pragma unroll
  for (int i = 0; i < kLatDma; ++i) {
    const int r = i * kWaves + L.wave;  // wave-uniform: a 64-unit block is one latent row
    const uint32_t idx = (uint32_t)__builtin_amdgcn_readlane(my_idx, r);
    u32x4* dst = buf + __builtin_amdgcn_readfirstlane(r * 64);
    // physical unit `lane` of row r holds logical unit (lane & 48) | ((lane & 15) ^ key) = lane ^ key
    __builtin_amdgcn_raw_ptr_buffer_load_lds(lat, (lds_void*)dst, 16, lane16 ^ (uint32_t)(lat_key(r) * 16),
                                             idx * lat_stb, 0, 0);
  }
  if constexpr (DR == 0) return;
  const __amdgpu_buffer_rsrc_t kpe = __builtin_amdgcn_make_buffer_rsrc((void*)p.k_pe, (short)0, -1, kBufferWord3);
  const uint32_t kpe_stb = (uint32_t)p.kpe_st * 2u;
  // lane part of the rotary offsets: unit (lane >> 2) & 7, 4-byte piece lane & 3 (the unit's
  // swizzle key is uniform per transfer and enters by XOR)
  uint32_t rope_lane = (uint32_t)(((lane >> 2) & 7) * 16 + (lane & 3) * 4);
  asm volatile("" : "+v"(rope_lane));
#pragma unroll
  for (int i = 0; i < kRopeDma; ++i) {
    const int blk = i * kWaves + L.wave;  // wave-uniform 64-dword block: rows 2 blk and 2 blk + 1
    // both row offsets are uniform (scalar multiplies); each half-wave takes one
    uint32_t o0 = (uint32_t)__builtin_amdgcn_readlane(my_idx, 2 * blk) * kpe_stb;
    uint32_t o1 = (uint32_t)__builtin_amdgcn_readlane(my_idx, 2 * blk + 1) * kpe_stb;
    asm volatile("" : "+s"(o0), "+s"(o1));  // scalar products, not one vector multiply after the select
    const uint32_t row_off = lane < 32 ? o0 : o1;
    uint32_t* dst = (uint32_t*)(buf + kLatRegion) + __builtin_amdgcn_readfirstlane(blk * 64);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kpe, (lds_void*)dst, 4,
                                             row_off + (rope_lane ^ (uint32_t)(rope_key(2 * blk) * 16)), 0, 0, 0);
  }
}

struct SoftmaxState {
  float mref;  // reference max in log2 units (-inf before the first valid score)
  float l;     // this half-wave's sum of exp2(score - mref)
};

// Lane constants are rederived per chunk from an opaque lane id so that none of them stays
// live (or spilled) across the chunk loop.
__device__ __forceinline__ Lane opaque_lane(const Lane& Lw) {
  int lane_op = Lw.lane;
  asm volatile("" : "+v"(lane_op));
  Lane L = Lw;
  L.lane = lane_op;
  L.n = lane_op & 31;
  L.h2 = lane_op >> 5;
  L.j16 = lane_op & 15;
  L.dh = (lane_op >> 4) & 1;
  return L;
}

// Partial S^T[slot][head] over this wave's 18 (NoPE: 16) k-steps of 16 coordinates: global
// k-step 2 * s + half, i.e. 16-byte units 4 * s + 2 * half + h2 of each gathered row.
template <int DR>
__device__ __forceinline__ f32x16 qk_partial(const u32x4* buf, const bf16x8* qf, const Lane& Lw) {
  constexpr int kQFrags = q_frags(DR);
  const Lane L = opaque_lane(Lw);
  f32x16 sc = f32x16{};
  // k-step s covers latent units 4s + 2 half + h2 (s < 16), then rotary units 4(s-16) + 2 half + h2;
  // fragments are read kQAhead MFMAs ahead in a fenced order (the waits count exactly).
  // Byte offsets: latent unit (4 j + 2 half + h2) ^ lat_key(n) of row n, where lat_key(n) has bits
  // 2-3 = 4 (n & 3) and bits 0-1 = (n >> 2) & 3, is one base XOR 64 j (the unit sits in bits 4-7,
  // the row in bits 10 and up); rotary unit (4 j + 2 half + h2) ^ rope_key(n), j = 0, 1, is one
  // base XOR 64 j as well (unit in bits 4-6, row in bits 7 and up).
  const int xh = 2 * L.half + L.h2;
  const int lat_b = L.n * (kLatUnits * 16) + (L.n & 3) * 64 + ((xh ^ ((L.n >> 2) & 3)) << 4);
  const int rope_b = (kLatRegion + L.n * kRopeUnits) * 16 + ((xh ^ rope_key(L.n)) << 4);
  const char* bytes = (const char*)buf;
  u32x4 a[kQFrags];
  auto read = [&](int s) {
    const int off = s < 16 ? (lat_b ^ (64 * (s & 3))) + 256 * (s >> 2) : rope_b ^ (64 * (s - 16));
    a[s] = *(const u32x4*)&bytes[off];
  };
  __builtin_amdgcn_s_setprio(1);  // the wave in its MFMA stream goes first
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
  for (int s = 0; s < kQAhead; ++s) read(s);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < kQFrags; ++s) {
    sc = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a[s]), qf[s], sc);
    if (s + kQAhead < kQFrags) read(s + kQAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  return sc;
}

// Probabilities exp2(s c2 - mu) of the lane's 16 scores as the two B operands of the PV MFMAs,
// and their sum.
__device__ __forceinline__ float chunk_probs(const f32x16& sc, float c2, float mu, bf16x8 (&pb)[2]) {
  float rs = 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    f32x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = fast_exp2(__builtin_fmaf(sc[8 * s + e], c2, -mu));
    pb[s] = cvt_bf16x8(pf);
#pragma unroll
    for (int e = 0; e < 8; ++e) rs += pf[e];
  }
  return rs;
}

// Online softmax over the chunk's full scores, then O^T[d][head] += latent^T[d][slot] P^T[slot][head]
// over this wave's 256 output coordinates.
// The probabilities are first taken against the current reference without the chunk's maximum:
// a lane whose 16 probabilities sum to at most 2^8 has none above 2^8, so its scores lie at most
// 8 (log2 units) above the reference and the lazy rescale below would keep it (up to the
// rounding of that comparison, where either choice gives the exact result).  Only when some
// lane's sum exceeds the bound (or its reference is still -inf: the bound is then -1) does the
// wave take the exact path: the maximum, the move where it is due, the O rescale and the
// probabilities again.
__device__ __forceinline__ void finish_chunk(const u32x4* buf, f32x16 sc, int n_in_chunk, f32x16* o,
                                             SoftmaxState& st, float c2, const Lane& Lw) {
  const Lane L = opaque_lane(Lw);
  // raw scores; slots past the compacted count are masked
  if (n_in_chunk < kSlots) {
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int r = 8 * (a >> 2) + 4 * L.h2 + (a & 3);
      sc[a] = r < n_in_chunk ? sc[a] : -INFINITY;
    }
  }
  const bool none_yet = st.mref == -INFINITY;
  bf16x8 pb[2];
  float rs = chunk_probs(sc, c2, none_yet ? 0.f : st.mref, pb);
  if (__builtin_amdgcn_ballot_w64(!(rs <= (none_yet ? -1.f : kLazyMax))) != 0) {
    // the scale c2 > 0 is applied to the maximum (rounding is monotone: max(s) c2 = max(s c2))
    float mx = sc[0];
#pragma unroll
    for (int a = 1; a < 16; ++a) mx = fmaxf(mx, sc[a]);
    mx = half_swap_max(mx) * c2;
    // lazy rescale: move the reference only when a score exceeds it by > 2^8 (exact either way)
    const bool move = mx > st.mref + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float mnew = move ? mx : st.mref;
      // lanes that keep their reference scale by exactly 1 (also when it is still -inf)
      const float alpha = move ? fast_exp2(st.mref - mnew) : 1.f;
      st.l *= alpha;
#pragma unroll
      for (int d = 0; d < kDBlocks; ++d) o[d] *= alpha;
      st.mref = mnew;
    }
    rs = chunk_probs(sc, c2, st.mref == -INFINITY ? 0.f : st.mref, pb);
  }
  st.l += rs;
  // transposed reads: lane j of a 16-lane group reads row r0 + 16 s (+ 8) and the 8-byte half
  // (j & 1) of latent unit 32 half + 4 d + 2 dh + ((j & 3) >> 1); rows r0 and r0 + 8 differ
  // only in bit 3, which flips bit 1 of lat_key
  const int r0 = 4 * L.h2 + (L.j16 >> 2);
  const int xsub = (L.j16 & 3) >> 1;
  // byte offsets of this lane's two reads for output blocks d with d & 3 = e at k-step 0: row r0,
  // unit (4 e + 2 dh + xsub) ^ lat_key(r0), and row r0 + 8, that unit ^ 2.  lat_key(r0) has bits
  // 2-3 = j16 & 12 and bit 0 = h2; the unit sits in bits 4-7 of the offset and the row, half-row
  // and 8-byte-half parts in other bits, so the four blocks are one base XOR 64 e, and row r0 + 8
  // is that XOR 32 plus 8 rows.  k-step s and d >> 2 add the compile-time constant
  // (16 s kLatUnits + 16 (d >> 2)) * 16
  const int base_b = (r0 * kLatUnits + 32 * L.half) * 16 + (L.j16 & 1) * 8 + (((2 * L.dh + xsub) ^ L.h2) << 4) +
                     ((L.j16 & 12) << 4);
  int lo_b[4], hi_b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo_b[e] = base_b ^ (64 * e);
    hi_b[e] = (lo_b[e] ^ 32) + 8 * kLatUnits * 16;
  }
  // 16 MFMAs (k-step s = i / 8, output block d = i % 8), fragments read kPvAhead ahead
  const char* bytes = (const char*)buf;
  bf16x8 vf[2 * kDBlocks];
  auto read = [&](int i) {
    const int s = i / kDBlocks, d = i % kDBlocks;
    const int c = (16 * s * kLatUnits + 16 * (d >> 2)) * 16;
    // one integer index per read keeps the pointer a single GEP from the LDS buffer, so the
    // read keeps the buffer's alias scope (no wait on gathers into the other buffers)
    const bf16x4 lo4 = lds_read_tr4((const __bf16*)&bytes[lo_b[d & 3] + c]);
    const bf16x4 hi4 = lds_read_tr4((const __bf16*)&bytes[hi_b[d & 3] + c]);
    vf[i] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#pragma unroll
  for (int i = 0; i < kPvAhead; ++i) read(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 2 * kDBlocks; ++i) {
    o[i % kDBlocks] = mfma_bf16_32x32x16(vf[i], pb[i / kDBlocks], o[i % kDBlocks]);
    if (i + kPvAhead < 2 * kDBlocks) read(i + kPvAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

template <int DR>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_fwd_kernel(SparseMlaParams p) {
  constexpr int kChunkUnits = chunk_units(DR);
  constexpr int kDmaPerWave = dma_per_wave(DR);
  constexpr int kQFrags = q_frags(DR);
  __shared__ int32_t s_idx[kSeg];
  __shared__ int32_t s_wtot[kWaves];
  __shared__ f32x4 exch[kWaves * 4 * 64];
  __shared__ u32x4 buf0[kChunkUnits];
  __shared__ u32x4 buf1[kChunkUnits];
  __shared__ u32x4 buf2[kChunkUnits];

  // tokens dealt to the 8 XCDs in runs of kTokenRun, round-robin: neighbouring tokens (which
  // name mostly the same rows) share an L2, and every XCD gets an even share of each
  // document, so the cheap tokens at document starts do not leave whole XCDs idle at the end
  const int j = blockIdx.x / 8;  // blocks reach an XCD in this order
  const int t = ((j / kTokenRun) * 8 + blockIdx.x % 8) * kTokenRun + j % kTokenRun;
  if (t >= p.T) return;

  Lane L;
  L.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  L.lane = threadIdx.x & 63;
  L.n = L.lane & 31;
  L.h2 = L.lane >> 5;
  L.j16 = L.lane & 15;
  L.dh = (L.lane >> 4) & 1;
  L.half = L.wave >> 2;
  L.hg = L.wave & 3;
  const int head = blockIdx.y * kHeadsPerBlock + L.hg * 32 + L.n;
  const bool head_ok = head < p.H;
  const bool group_ok = blockIdx.y * kHeadsPerBlock + L.hg * 32 < p.H;

  bf16x8 qf[kQFrags];
  {
    const __bf16* qb = (const __bf16*)p.q + (int64_t)t * p.q_st + (int64_t)(head_ok ? head : p.H - 1) * p.q_sh;
#pragma unroll
    for (int s = 0; s < kQFrags; ++s) qf[s] = *(const bf16x8*)(qb + 16 * (2 * s + L.half) + 8 * L.h2);
  }
  f32x16 o[kDBlocks];
#pragma unroll
  for (int d = 0; d < kDBlocks; ++d) o[d] = f32x16{};
  SoftmaxState st{-INFINITY, 0.f};

  const int my_doc = p.doc_ids[t];
  const int32_t* irow = p.indices + (int64_t)t * p.idx_st;
  for (int seg = 0; seg < p.topk; seg += kSeg) {
    // ---- compact the valid slots of this segment into s_idx (order preserved)
    __syncthreads();  // previous segment's readers of s_idx and of the buffers are done
    const Lane Ls = opaque_lane(L);  // lane values rederived, not kept live across the chunk loop
    const int base = seg + (L.wave * 64 + Ls.lane) * kSlotsPerThread;
    int vals[kSlotsPerThread];
    uint32_t mask = 0;
    if (my_doc >= 0) {
#pragma unroll
      for (int k = 0; k < kSlotsPerThread; ++k) {
        const int slot = base + k;
        int idx = -1;
        if (slot < p.topk) idx = irow[slot];
        vals[k] = idx;
        if (idx >= 0 && idx < p.T && idx <= t && p.doc_ids[idx] == my_doc) mask |= 1u << k;
      }
    }
    const int cnt = __builtin_popcount(mask);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int yv = __shfl_up(incl, off);
      if (Ls.lane >= off) incl += yv;
    }
    if (Ls.lane == 63) s_wtot[L.wave] = incl;
    __syncthreads();
    int woff = 0, nv = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int v = s_wtot[w];
      woff += w < L.wave ? v : 0;
      nv += v;
    }
    int pos = woff + incl - cnt;
#pragma unroll
    for (int k = 0; k < kSlotsPerThread; ++k)
      if (mask & (1u << k)) s_idx[pos++] = vals[k];
    __syncthreads();

    // ---- gather + attend, 32 compacted slots per chunk, ring of three buffers.  Chunk cc is
    // consumed from buffer cc % 3; the gather of chunk cc + 2 is issued once the partial scores
    // of chunk cc have been exchanged, so it overlaps the rest of chunk cc and all of chunk
    // cc + 1.  Every wave issues exactly kDmaPerWave gathers per chunk (dummy ones past the
    // end), so "own gathers of chunk cc landed" is vmcnt <= kDmaPerWave.
    const int nc = (nv + kSlots - 1) / kSlots;
    if (nc > 0) {  // both prologue gathers unconditionally (chunk 1 may be a dummy)
      gather_chunk<DR>(p, s_idx, nv, 0, t, buf0, L);
      gather_chunk<DR>(p, s_idx, nv, 1, t, buf1, L);
    }
    auto phase = [&](int cc, const u32x4* cur, u32x4* ahead, bool steady) {
      if (steady) wait_vmcnt<kDmaPerWave>(); else wait_vmcnt<0>();
      barrier_keep_loads();  // chunk cc landed for every wave; chunk cc - 1 fully consumed
      // every wave computes its partial scores: the waves of a head group past H hold the
      // clamped head's Q rows and their scores are never read (no zero vector per chunk)
      f32x16 sc = qk_partial<DR>(cur, qf, L);
      const int xl = opaque_lane(L).lane;  // rederived, not kept live across the loop
      f32x4* mine = exch + L.wave * (4 * 64) + xl;
#pragma unroll
      for (int j = 0; j < 4; ++j) mine[j * 64] = f32x4{sc[4 * j], sc[4 * j + 1], sc[4 * j + 2], sc[4 * j + 3]};
      wait_lgkm0();
      barrier_keep_loads();
      const f32x4* theirs = exch + (L.wave ^ 4) * (4 * 64) + xl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = theirs[j * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[4 * j + e] += v[e];
      }
      if (steady) gather_chunk<DR>(p, s_idx, nv, cc + 2, t, ahead, L);
      if (group_ok) finish_chunk(cur, sc, min(kSlots, nv - cc * kSlots), o, st, p.c2, L);
    };
    int c = 0;
    for (; c + 2 < nc; c += 3) {  // full rounds: chunks c, c+1, c+2 all exist
      phase(c, buf0, buf2, true);
      phase(c + 1, buf1, buf0, true);
      phase(c + 2, buf2, buf1, true);
    }
    // the last one or two chunks were gathered by the rounds above (or the prologue)
    if (c < nc) phase(c, buf0, buf2, false);
    if (c + 1 < nc) phase(c + 1, buf1, buf0, false);
  }

  // ---- epilogue
  // the epilogue's lane values rederived as well
  const Lane Le = opaque_lane(L);
  const int head_e = blockIdx.y * kHeadsPerBlock + L.hg * 32 + Le.n;
  if (head_e >= p.H) return;
  const float lt = half_swap_sum(st.l);
  const bool empty = st.mref == -INFINITY;
  const float inv = empty ? 0.f : 1.f / lt;
  __bf16* ob = (__bf16*)p.out + (int64_t)t * p.o_st + (int64_t)head_e * p.o_sh + 256 * L.half;
#pragma unroll
  for (int d = 0; d < kDBlocks; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = o[d][4 * i + e] * inv;
      *(bf16x4*)(ob + 32 * d + 8 * i + 4 * Le.h2) = cvt_bf16x4(r);
    }
  if (p.lse != nullptr && Le.h2 == 0 && L.half == 0)
    p.lse[(int64_t)t * p.H + head_e] = empty ? -INFINITY : (st.mref + __builtin_amdgcn_logf(lt)) * kLn2;
}

}  // namespace

hipError_t sparse_mla_fwd_launch(const SparseMlaParams& p, hipStream_t stream) {
  if (p.T <= 0) return hipSuccess;
  const unsigned gx = (unsigned)((p.T + 8 * kTokenRun - 1) / (8 * kTokenRun) * (8 * kTokenRun));
  const unsigned gy = (unsigned)((p.H + kHeadsPerBlock - 1) / kHeadsPerBlock);
  if (p.Dr == 64)
    hipLaunchKernelGGL(sparse_mla_fwd_kernel<64>, dim3(gx, gy), dim3(kThreads), 0, stream, p);
  else if (p.Dr == 0)
    hipLaunchKernelGGL(sparse_mla_fwd_kernel<0>, dim3(gx, gy), dim3(kThreads), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace swa
