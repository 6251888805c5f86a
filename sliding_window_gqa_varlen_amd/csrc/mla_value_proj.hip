// Value up-projection of sparse MLA for gfx950: out[t, h, :] = W[h] o[t, h, :] with
// W = value_weight [H, Dv, 512] (the KV-B value weight of sparse_mla on the
// nemo_automodel.components.models.mistral_large4.attention page, applied to the attention
// output over latent rows).
//
// Design: per head a [T x 512] x [512 x Dv] product, bound by reading o once from HBM
// (1 KiB per token and head against Dv * 2 bytes written).
//  * A workgroup (4 waves, one per SIMD) owns one head and a strided set of token tiles.
//    Wave w keeps the 32 rows 32 (w % MB) .. + 31 of W[h] in registers for the whole kernel
//    (32 k-steps x 8 bf16 = 128 registers), so W is read from HBM once per workgroup.
//  * o rows travel HBM -> LDS with buffer_load ... lds, one whole 1 KiB row per wave
//    instruction (fully coalesced), into a ring of kSlots 32-token slots.  The 16-byte units
//    of row r are XOR-swizzled (unit u at u ^ (r & 15)) so the MFMA operand reads, one unit of
//    16 consecutive rows per 16 lanes, are bank-conflict free.
//  * C^T = W o^T with v_mfma_f32_32x32x16_bf16: Dv rows = M (A from registers), 32 tokens = N
//    (B from LDS), K = 512.  A slot feeds MB waves (one per 32-row block of W); with Dv = 64
//    two slots are consumed per iteration.  Loads run kAhead iterations ahead of the MFMAs.
#include "device_common.h"
#include "launch.h"


namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kDl = 512;                   // latent width (the contraction)
constexpr int kKSteps = kDl / 16;          // 32 k-steps of 16
constexpr int kTile = 32;                  // tokens per LDS slot (the MFMA N)
constexpr int kRowsPerWave = kTile / kWaves;  // row loads per wave and slot
constexpr int kSlotBytes = kTile * kDl * 2;

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format, raw access

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt unconstrained
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

template <int DV>
__global__ __launch_bounds__(kThreads, 1) void mla_value_proj_kernel(MlaValueProjParams p) {
  constexpr int MB = DV / 32;           // 32-row blocks of W
  constexpr int kSlots = 4;  // ring of 32 KiB slots
  constexpr int P = kWaves / MB;        // slots consumed per iteration
  constexpr int kAhead = kSlots / P - 1;  // iterations loaded ahead
  constexpr int kIterTokens = kTile * P;
  constexpr int kLoadsPerIter = kRowsPerWave * P;  // DMA instructions per wave and iteration
  __shared__ u32x4 olds[kSlots * kSlotBytes / 16];

  const int h = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, h2 = lane >> 5;
  const int m = wave % MB, pw = wave / MB;  // W block and slot of the iteration this wave multiplies
  const int T = p.T;
  const int n_iter_all = (T + kIterTokens - 1) / kIterTokens;
  const int g = blockIdx.x, split = gridDim.x;
  if (g >= n_iter_all) return;
  const int L = (n_iter_all - g + split - 1) / split;  // iterations of this workgroup: g + k split

  // ---- W rows of this wave: lane (n, h2) holds W[32 m + n][16 s + 8 h2 .. + 7] for every k-step s
  bf16x8 a[kKSteps];
  {
    const __bf16* wrow = (const __bf16*)p.w + (int64_t)h * p.w_sh + (int64_t)(32 * m + n) * p.w_sv + 8 * h2;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) a[s] = *(const bf16x8*)(wrow + 16 * s);
  }

  // ---- DMA of local iteration k: slot (k P + q) % kSlots gets tokens (g + k split) kIterTokens + q kTile + r
  const char* obase = (const char*)p.o + (int64_t)h * p.o_sh * 2;
  const uint32_t o_stb = (uint32_t)(p.o_st * 2);
  auto issue = [&](int k) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      // rows past the end re-read the last token (their results are never stored)
      const int t0 = min((g + k * split) * kIterTokens + q * kTile, T - 1);
      const int slot = (k * P + q) % kSlots;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(obase + (int64_t)t0 * o_stb), (short)0, -1, kBufferWord3);
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        const int r = i * kWaves + wave;
        const int tr = min(r, T - 1 - t0);
        u32x4* dst = olds + __builtin_amdgcn_readfirstlane(slot * (kSlotBytes / 16) + r * 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, (uint32_t)((lane ^ (r & 15)) * 16),
                                                 (uint32_t)tr * o_stb, 0, 0);
      }
    }
  };
#pragma unroll
  for (int k = 0; k < kAhead; ++k)
    if (k < L) issue(k);

  // operand of k-step s, token row n: unit 2 s + h2 of row n at (b0 ^ 32 (s & 7)) + 256 (s >> 3)
  const int b0 = n * (kDl * 2) + ((h2 ^ (n & 15)) << 4);
  const char* lbase = (const char*)olds;

  for (int k = 0; k < L; ++k) {
    if (k + kAhead - 1 < L) wait_vmcnt<kLoadsPerIter * (kAhead - 1)>();
    else wait_vmcnt<0>();
    barrier_keep_loads();  // every wave's rows of iteration k landed; iteration k - 1's slots are free
    if (k + kAhead < L) issue(k + kAhead);

    const char* sb = lbase + ((k * P + pw) % kSlots) * kSlotBytes;
    bf16x8 b[kKSteps];
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) b[s] = *(const bf16x8*)(sb + ((b0 ^ (32 * (s & 7))) + 256 * (s >> 3)));
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) acc = mfma_bf16_32x32x16(a[s], b[s], acc);

    // ---- store: lane holds rows 32 m + 8 j + 4 h2 + (0..3) of token column n
    const int t = (g + k * split) * kIterTokens + pw * kTile + n;
    if (t < T) {
      __bf16* ob = (__bf16*)p.out + (int64_t)t * p.out_st + (int64_t)h * p.out_sh + 32 * m + 4 * h2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = acc[4 * j + e];
        *(bf16x4*)(ob + 8 * j) = cvt_bf16x4(r);
      }
    }
  }
}

}  // namespace

hipError_t mla_value_proj_launch(const MlaValueProjParams& p, int n_cu, hipStream_t stream) {
  if (p.T <= 0 || p.H <= 0) return hipSuccess;
  const int iter_tokens = p.Dv == 128 ? kTile : 2 * kTile;
  const int n_iter = (p.T + iter_tokens - 1) / iter_tokens;
  // one resident workgroup per CU: split each head's iterations so that the grid fills the chip
  int split = (n_cu + p.H - 1) / p.H;
  split = split < 1 ? 1 : (split > n_iter ? n_iter : split);
  const dim3 grid((unsigned)split, (unsigned)p.H);
  if (p.Dv == 128)
    hipLaunchKernelGGL(mla_value_proj_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  else if (p.Dv == 64)
    hipLaunchKernelGGL(mla_value_proj_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace swa
