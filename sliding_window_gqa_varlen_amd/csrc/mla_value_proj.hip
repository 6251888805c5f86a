// Value up-projection of sparse MLA for gfx950: out[t, h, :] = W[h] o[t, h, :] with
// W = value_weight [H, Dv, 512] (the KV-B value weight of sparse_mla on the
// nemo_automodel.components.models.mistral_large4.attention page, applied to the attention
// output over latent rows).
//
// Design: per head a [T x 512] x [512 x Dv] product, bound by reading o once from HBM.
//  * A workgroup (4 waves, one per SIMD) owns one head and a strided set of 256-token
//    blocks; W[h] (Dv x 1 KB) is staged once into LDS with buffer_load ... lds, rows
//    XOR-swizzled (unit u of row r at u ^ (r & 15)) so the 32-row MFMA operand reads are
//    conflict free.
//  * C^T = W o^T with v_mfma_f32_32x32x16_bf16: Dv = M (W rows from LDS), tokens = N (o rows
//    straight from HBM into registers, 16 bytes per lane per k-step), K = 512.  Each wave
//    computes Dv x 64 tokens; o fragments are loaded kPrefetch k-steps ahead (across block
//    boundaries), so the loads stream while the MFMAs run.
//  * One wave per SIMD: 512 registers hold the accumulators and the prefetch ring.
#include "device_common.h"
#include "launch.h"

#ifndef SWA_VPROJ_PREFETCH
#define SWA_VPROJ_PREFETCH 8
#endif

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kDl = 512;                // latent width (the contraction)
constexpr int kKSteps = kDl / 16;       // 32 k-steps of 16
constexpr int kNB = 2;                  // 32-token MFMA blocks per wave
constexpr int kTokensPerWave = 32 * kNB;
constexpr int kBlockTokens = kWaves * kTokensPerWave;  // 256
constexpr int kPrefetch = SWA_VPROJ_PREFETCH;          // k-steps of o loaded ahead
static_assert(kKSteps % kPrefetch == 0, "the prefetch ring index must be a compile-time constant");

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format, raw access

template <int DV>
__global__ __launch_bounds__(kThreads, 1) void mla_value_proj_kernel(MlaValueProjParams p) {
  constexpr int MB = DV / 32;  // 32-row blocks of W
  __shared__ u32x4 wlds[DV * kDl / 8];

  const int h = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, h2 = lane >> 5;
  const int n_blocks = (p.T + kBlockTokens - 1) / kBlockTokens;
  if ((int)blockIdx.x >= n_blocks) return;

  // ---- stage W[h] into LDS: transfer i of a wave moves row r = 4 i + wave (64 units)
  {
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const __bf16*)p.w + (int64_t)h * p.w_sh), (short)0, -1, kBufferWord3);
    const uint32_t w_stb = (uint32_t)p.w_sv * 2u;
#pragma unroll
    for (int i = 0; i < DV / kWaves; ++i) {
      const int r = i * kWaves + wave;
      u32x4* dst = wlds + __builtin_amdgcn_readfirstlane(r * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)dst, 16, (uint32_t)((lane ^ (r & 15)) * 16),
                                               (uint32_t)r * w_stb, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
  }
  // W fragment of M-block m, k-step s: row 32 m + n, unit 2 s + h2 at
  // (wb[s & 7] + 32 KiB m) + 256 (s >> 3)
  int wb[8];
  {
    const int b0 = n * (kDl * 2) + ((h2 ^ (n & 15)) << 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) wb[j] = b0 ^ (32 * j);
  }
  const char* wbase = (const char*)wlds;

  // o rows of this lane: token t0 + 32 nb + n of each block, 16 coordinates 16 s + 8 h2
  const __bf16* obase = (const __bf16*)p.o + (int64_t)h * p.o_sh + 8 * h2;
  auto load_o = [&](int blk, int s, int nb) -> bf16x8 {
    const int t = min(blk * kBlockTokens + wave * kTokensPerWave + 32 * nb + n, p.T - 1);
    return *(const bf16x8*)(obase + (int64_t)t * p.o_st + 16 * s);
  };

  bf16x8 ring[kPrefetch][kNB];
  const int stride = gridDim.x;
  int blk = blockIdx.x;
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) ring[s][nb] = load_o(blk, s, nb);

  for (; blk < n_blocks; blk += stride) {
    const int nxt = blk + stride < n_blocks ? blk + stride : blk;  // tail prefetch re-reads a valid block
    f32x16 acc[MB][kNB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[m][nb] = f32x16{};
    // W fragments one k-step ahead of their MFMAs
    auto load_w = [&](int s, int m) -> bf16x8 {
      return *(const bf16x8*)(wbase + (wb[s & 7] + 32768 * m) + 256 * (s >> 3));
    };
    bf16x8 a[2][MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) a[0][m] = load_w(0, m);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      if (s + 1 < kKSteps) {
#pragma unroll
        for (int m = 0; m < MB; ++m) a[(s + 1) & 1][m] = load_w(s + 1, m);
      }
      bf16x8 b[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) b[nb] = ring[s % kPrefetch][nb];
      // refill this ring slot with the k-step kPrefetch ahead (next block past the end)
      const int s2 = s + kPrefetch;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        ring[s % kPrefetch][nb] = s2 < kKSteps ? load_o(blk, s2, nb) : load_o(nxt, s2 - kKSteps, nb);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[m][nb] = mfma_bf16_32x32x16(a[s & 1][m], b[nb], acc[m][nb]);
      __builtin_amdgcn_sched_barrier(0);  // k-step order as written: loads stay kPrefetch steps ahead
    }
    // ---- store: lane holds rows 32 m + 8 j + 4 h2 + (0..3) of token column n
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int t = blk * kBlockTokens + wave * kTokensPerWave + 32 * nb + n;
      if (t < p.T) {
        __bf16* ob = (__bf16*)p.out + (int64_t)t * p.out_st + (int64_t)h * p.out_sh + 4 * h2;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = acc[m][nb][4 * j + e];
            *(bf16x4*)(ob + 32 * m + 8 * j) = cvt_bf16x4(r);
          }
      }
    }
  }
}

}  // namespace

hipError_t mla_value_proj_launch(const MlaValueProjParams& p, int n_cu, hipStream_t stream) {
  if (p.T <= 0 || p.H <= 0) return hipSuccess;
  const int n_blocks = (p.T + kBlockTokens - 1) / kBlockTokens;
  // one resident workgroup per CU: split each head's blocks so that the grid fills the chip
  int split = (n_cu + p.H - 1) / p.H;
  split = split < 1 ? 1 : (split > n_blocks ? n_blocks : split);
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
