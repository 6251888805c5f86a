// Host-only stand-ins for the kernel launchers and the three HIP runtime calls abi.cpp makes,
// so the C ABI's argument validation can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven on a machine without a GPU.  Each launcher records
// that it was reached; nothing is launched.
#include <hip/hip_runtime_api.h>

#include "launch.h"

int g_launches = 0;

namespace swa {

void dense_fwd_plan(DenseFwdParams& p) {
  p.G = p.Hq / p.Hkv;
  p.hb_shift = 0;
  p.n_chunks = p.G;
  p.tile_tokens = 128;
  p.n_vtiles = p.T / 128 + p.n_docs + 2;
  p.n_work = p.Hkv * p.n_chunks * p.n_vtiles;
  p.c2 = p.scale * 1.4426950408889634f;
}
int64_t dense_fwd_grid(const DenseFwdParams& p) { return p.n_work; }
hipError_t dense_fwd_launch(const DenseFwdParams&, Dtype, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
void dense_bwd_plan(DenseBwdParams& p, int D) {
  dense_fwd_plan(p.f);
  p.kv_tile = D == 64 ? 64 : 128;  // the fields the size guard reads, as the device plan sets them
  p.kv_n_vtiles = p.f.T / p.kv_tile + p.f.n_docs + 2;
  p.kv_n_work = p.f.Hkv * p.kv_n_vtiles;
}
hipError_t dense_bwd_launch(const DenseBwdParams&, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t sparse_mla_fwd_launch(const SparseMlaParams&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t mla_value_proj_launch(const MlaValueProjParams&, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace swa

extern "C" {
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}
}
