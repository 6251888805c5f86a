// Drives every argument check of the C ABI (abi.cpp) with the kernel launchers stubbed out,
// under AddressSanitizer and UndefinedBehaviorSanitizer: each malformed call must return its
// status code, set swa_last_error() and reach no launcher; each well-formed call reaches
// exactly one.  Tensor data pointers point into a host arena (the checks only test them for
// NULL and alignment; nothing is read through them).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <limits>
#include <vector>

#include "swattn.h"

extern int g_launches;

namespace {

int g_failures = 0;
int g_cases = 0;
alignas(256) unsigned char g_arena[1 << 16];

void* at(int off) { return g_arena + off; }

swa_tensor tensor(int32_t dtype, std::vector<int64_t> shape, void* data) {
  swa_tensor t{};
  t.data = data;
  t.dtype = dtype;
  t.ndim = (int32_t)shape.size();
  int64_t st = 1;
  for (int i = t.ndim - 1; i >= 0; --i) {
    t.shape[i] = shape[i];
    t.stride[i] = st;
    st *= shape[i];
  }
  return t;
}

void expect(const char* what, int32_t got, int32_t want, int launches_before) {
  ++g_cases;
  const int launched = g_launches - launches_before;
  bool ok = got == want;
  if (want == SWA_OK) ok = ok && launched <= 1;
  else ok = ok && launched == 0 && std::strlen(swa_last_error()) > 0;
  if (!ok) {
    ++g_failures;
    std::printf("FAIL %s: status %d (want %d), launches %d, detail '%s'\n", what, got, want, launched, swa_last_error());
  }
}

#define CASE(what, want, call)                 \
  do {                                         \
    const int before__ = g_launches;           \
    const int32_t st__ = (call);               \
    expect(what, st__, want, before__);        \
  } while (0)

// ------------------------------------------------------------------------ dense forward
struct Dense {
  swa_tensor q, k, v, out;
  int32_t cu[3] = {0, 8, 16};
  int32_t n_docs = 2, window = 0;
  float scale = 0.125f;
  float sinks[4] = {0, 0, 0, 0};
  float lse[64];
  bool use_sinks = false;
  Dense(int32_t dt = SWA_DTYPE_BF16, int64_t D = 64) {
    q = tensor(dt, {16, 4, D}, at(0));
    k = tensor(dt, {16, 2, D}, at(16384));
    v = tensor(dt, {16, 2, D}, at(24576));
    out = tensor(dt, {16, 4, D}, at(32768));
  }
  int32_t call() {
    return varlen_attn_fwd(&q, &k, &v, cu, n_docs, window, scale, use_sinks ? sinks : nullptr, &out, lse, nullptr);
  }
};

void dense_cases() {
  { Dense d; CASE("dense ok", SWA_OK, d.call()); }
  { Dense d(SWA_DTYPE_F32, 64); CASE("dense f32 ok", SWA_OK, d.call()); }
  { Dense d; d.use_sinks = true; d.window = 5; CASE("dense sinks+window ok", SWA_OK, d.call()); }
  { Dense d; CASE("dense null q", SWA_ERR_NULL,
                  varlen_attn_fwd(nullptr, &d.k, &d.v, d.cu, 2, 0, 0.125f, nullptr, &d.out, nullptr, nullptr)); }
  { Dense d; d.out.data = nullptr; CASE("dense null out data", SWA_ERR_NULL, d.call()); }
  { Dense d; d.q.ndim = 2; CASE("dense rank", SWA_ERR_SHAPE, d.call()); }
  { Dense d; d.q.shape[0] = -1; CASE("dense negative extent", SWA_ERR_SHAPE, d.call()); }
  { Dense d; d.q.dtype = 7; CASE("dense unknown dtype", SWA_ERR_DTYPE, d.call()); }
  { Dense d; d.q.dtype = SWA_DTYPE_I32; d.k.dtype = d.v.dtype = d.out.dtype = SWA_DTYPE_I32;
    CASE("dense int dtype", SWA_ERR_DTYPE, d.call()); }
  { Dense d; d.k.dtype = SWA_DTYPE_F32; CASE("dense mixed dtype", SWA_ERR_DTYPE, d.call()); }
  { Dense d; d.k.shape[0] = 15; CASE("dense token mismatch", SWA_ERR_SHAPE, d.call()); }
  { Dense d; d.v.shape[1] = 1; CASE("dense kv head mismatch", SWA_ERR_SHAPE, d.call()); }
  { Dense d; d.out.shape[1] = 3; CASE("dense out shape", SWA_ERR_SHAPE, d.call()); }
  { Dense d; d.k = tensor(SWA_DTYPE_BF16, {16, 3, 64}, at(16384)); d.v = tensor(SWA_DTYPE_BF16, {16, 3, 64}, at(24576));
    CASE("dense Hq % Hkv", SWA_ERR_SHAPE, d.call()); }
  { Dense d(SWA_DTYPE_BF16, 96); CASE("dense head_dim 96", SWA_ERR_UNSUPPORTED, d.call()); }
  { Dense d(SWA_DTYPE_F32, 256); d.q.shape[0] = d.k.shape[0] = d.v.shape[0] = d.out.shape[0] = 1;
    CASE("dense f32 head_dim 256", SWA_ERR_UNSUPPORTED, d.call()); }
  { Dense d; d.q.stride[2] = 2; CASE("dense inner stride", SWA_ERR_LAYOUT, d.call()); }
  { Dense d; d.q.data = at(8); CASE("dense misaligned base", SWA_ERR_LAYOUT, d.call()); }
  { Dense d; d.q.stride[0] = 260; CASE("dense misaligned row", SWA_ERR_LAYOUT, d.call()); }
  { Dense d; d.q.stride[1] = -64; CASE("dense negative stride", SWA_ERR_LAYOUT, d.call()); }
  { Dense d; d.k.stride[0] = (int64_t)1 << 24; CASE("dense huge kv stride", SWA_ERR_UNSUPPORTED, d.call()); }
  { Dense d; d.n_docs = -1; CASE("dense n_docs < 0", SWA_ERR_ARG, d.call()); }
  { Dense d; d.window = -2; CASE("dense window < 0", SWA_ERR_ARG, d.call()); }
  { Dense d; d.scale = 0.f; CASE("dense scale 0", SWA_ERR_ARG, d.call()); }
  { Dense d; d.scale = std::numeric_limits<float>::quiet_NaN(); CASE("dense scale nan", SWA_ERR_ARG, d.call()); }
  { Dense d; d.scale = std::numeric_limits<float>::infinity(); CASE("dense scale inf", SWA_ERR_ARG, d.call()); }
  { Dense d; CASE("dense null cu_seqlens", SWA_ERR_NULL,
                  varlen_attn_fwd(&d.q, &d.k, &d.v, nullptr, 2, 0, 0.125f, nullptr, &d.out, nullptr, nullptr)); }
  { Dense d; d.out.data = d.q.data; CASE("dense out aliases q", SWA_ERR_ARG, d.call()); }
  { Dense d; d.q.shape[0] = d.k.shape[0] = d.v.shape[0] = d.out.shape[0] = 0;
    CASE("dense empty", SWA_OK, d.call()); }
  { Dense d; d.n_docs = 0; CASE("dense no documents", SWA_OK,
        varlen_attn_fwd(&d.q, &d.k, &d.v, nullptr, 0, 0, 0.125f, nullptr, &d.out, nullptr, nullptr)); }
}

// ------------------------------------------------------------------------ dense backward
struct Bwd {
  Dense f;
  swa_tensor dout, dq, dk, dv;
  float delta[64], dsinks[4];
  Bwd() : f(SWA_DTYPE_BF16, 128) {
    f.q = tensor(SWA_DTYPE_BF16, {16, 4, 128}, at(0));
    f.k = tensor(SWA_DTYPE_BF16, {16, 2, 128}, at(16384));
    f.v = tensor(SWA_DTYPE_BF16, {16, 2, 128}, at(24576));
    f.out = tensor(SWA_DTYPE_BF16, {16, 4, 128}, at(32768));
    dout = tensor(SWA_DTYPE_BF16, {16, 4, 128}, at(49152));
    dq = tensor(SWA_DTYPE_BF16, {16, 4, 128}, at(8192));
    dk = tensor(SWA_DTYPE_BF16, {16, 2, 128}, at(40960));
    dv = tensor(SWA_DTYPE_BF16, {16, 2, 128}, at(45056));
  }
  int32_t call(bool with_lse = true, bool with_delta = true, bool with_dsinks = true) {
    return varlen_attn_bwd(&f.q, &f.k, &f.v, &f.out, &dout, with_lse ? f.lse : nullptr, f.cu, f.n_docs, f.window,
                           f.scale, f.use_sinks ? f.sinks : nullptr, &dq, &dk, &dv,
                           with_dsinks ? dsinks : nullptr, with_delta ? delta : nullptr, nullptr);
  }
};

void bwd_cases() {
  { Bwd b; CASE("bwd ok", SWA_OK, b.call()); }
  { Bwd b; b.f.use_sinks = true; CASE("bwd sinks ok", SWA_OK, b.call()); }
  { Bwd b; CASE("bwd null lse", SWA_ERR_NULL, b.call(false)); }
  { Bwd b; CASE("bwd null delta", SWA_ERR_NULL, b.call(true, false)); }
  { Bwd b; b.f.use_sinks = true; CASE("bwd sinks without dsinks", SWA_ERR_NULL, b.call(true, true, false)); }
  { Bwd b; b.dq.dtype = SWA_DTYPE_F32; CASE("bwd f32 gradient", SWA_ERR_DTYPE, b.call()); }
  { Bwd b; b.f.q.dtype = SWA_DTYPE_F32; CASE("bwd f32 input", SWA_ERR_DTYPE, b.call()); }
  { Bwd b; b.dk.shape[1] = 4; CASE("bwd dk shape", SWA_ERR_SHAPE, b.call()); }
  { Bwd b; b.dout.shape[2] = 64; CASE("bwd dout shape", SWA_ERR_SHAPE, b.call()); }
  { Bwd b; b.dq.data = b.f.q.data; CASE("bwd dq aliases q", SWA_ERR_ARG, b.call()); }
  { Bwd b; b.dv.data = b.dk.data; CASE("bwd dk aliases dv", SWA_ERR_ARG, b.call()); }
  { Bwd b; b.f.window = -1; CASE("bwd window < 0", SWA_ERR_ARG, b.call()); }
  { Bwd b; b.f.n_docs = -3; CASE("bwd n_docs < 0", SWA_ERR_ARG, b.call()); }
  { Bwd b; b.f.scale = -1.f; CASE("bwd scale < 0", SWA_ERR_ARG, b.call()); }
  { Bwd b; b.f.q.stride[0] = (int64_t)1 << 24; CASE("bwd huge stride", SWA_ERR_UNSUPPORTED, b.call()); }
  { Bwd b; CASE("bwd null cu_seqlens", SWA_ERR_NULL,
                varlen_attn_bwd(&b.f.q, &b.f.k, &b.f.v, &b.f.out, &b.dout, b.f.lse, nullptr, 2, 0, 0.1f, nullptr,
                                &b.dq, &b.dk, &b.dv, nullptr, b.delta, nullptr)); }
  { Bwd b; CASE("bwd null dout", SWA_ERR_NULL,
                varlen_attn_bwd(&b.f.q, &b.f.k, &b.f.v, &b.f.out, nullptr, b.f.lse, b.f.cu, 2, 0, 0.1f, nullptr,
                                &b.dq, &b.dk, &b.dv, nullptr, b.delta, nullptr)); }
}

// ------------------------------------------------------------------------ sparse MLA
struct Sparse {
  swa_tensor q, latent, k_pe, idx, out;
  int32_t doc_ids[16];
  float lse[16 * 16];
  float scale = 0.04f;
  Sparse(int64_t Dr = 64) {
    q = tensor(SWA_DTYPE_BF16, {4, 16, 512 + Dr}, at(0));
    latent = tensor(SWA_DTYPE_BF16, {4, 512}, at(20480));
    k_pe = tensor(SWA_DTYPE_BF16, {4, Dr}, Dr ? at(24576) : nullptr);
    idx = tensor(SWA_DTYPE_I32, {4, 3}, at(25600));
    out = tensor(SWA_DTYPE_BF16, {4, 16, 512}, at(32768));
  }
  int32_t call(bool with_ids = true) {
    return sparse_mla_fwd(&q, &latent, &k_pe, &idx, with_ids ? doc_ids : nullptr, scale, &out, lse, nullptr);
  }
};

void sparse_cases() {
  { Sparse s; CASE("sparse ok", SWA_OK, s.call()); }
  { Sparse s(0); CASE("sparse NoPE ok", SWA_OK, s.call()); }
  { Sparse s; CASE("sparse null doc_ids", SWA_ERR_NULL, s.call(false)); }
  { Sparse s; s.idx.dtype = SWA_DTYPE_F32; CASE("sparse float indices", SWA_ERR_DTYPE, s.call()); }
  { Sparse s; s.latent.dtype = SWA_DTYPE_F32; CASE("sparse f32 latent", SWA_ERR_DTYPE, s.call()); }
  { Sparse s; s.q.shape[2] = 600; CASE("sparse q width", SWA_ERR_SHAPE, s.call()); }
  { Sparse s; s.latent.shape[0] = 3; CASE("sparse token mismatch", SWA_ERR_SHAPE, s.call()); }
  { Sparse s; s.out.shape[2] = 256; CASE("sparse out shape", SWA_ERR_SHAPE, s.call()); }
  { Sparse s; s.q = tensor(SWA_DTYPE_BF16, {4, 16, 544}, at(0)); s.k_pe = tensor(SWA_DTYPE_BF16, {4, 32}, at(24576));
    CASE("sparse rotary 32", SWA_ERR_UNSUPPORTED, s.call()); }
  { Sparse s; s.q.shape[1] = s.out.shape[1] = 12; CASE("sparse H % 16", SWA_ERR_UNSUPPORTED, s.call()); }
  { Sparse s; s.idx.shape[1] = 0; CASE("sparse topk 0", SWA_ERR_ARG, s.call()); }
  { Sparse s; s.scale = std::numeric_limits<float>::quiet_NaN(); CASE("sparse scale nan", SWA_ERR_ARG, s.call()); }
  { Sparse s; s.out.data = s.q.data; CASE("sparse out aliases q", SWA_ERR_ARG, s.call()); }
  { Sparse s; s.idx.data = at(25602); CASE("sparse misaligned indices", SWA_ERR_LAYOUT, s.call()); }
  { Sparse s; s.idx.data = at(25604); CASE("sparse 4-byte aligned indices ok", SWA_OK, s.call()); }
  { Sparse s; s.latent.stride[0] = (int64_t)1 << 30; CASE("sparse latent over 4 GiB", SWA_ERR_UNSUPPORTED, s.call()); }
  { Sparse s; s.q.shape[0] = s.latent.shape[0] = s.k_pe.shape[0] = s.idx.shape[0] = s.out.shape[0] = 0;
    CASE("sparse empty", SWA_OK, s.call(false)); }
}

// ------------------------------------------------------------------------ value projection
struct VProj {
  swa_tensor o, w, out;
  VProj(int64_t Dv = 128) {
    o = tensor(SWA_DTYPE_BF16, {4, 4, 512}, at(0));
    w = tensor(SWA_DTYPE_BF16, {4, Dv, 512}, at(16384));
    out = tensor(SWA_DTYPE_BF16, {4, 4, Dv}, at(49152));
  }
  int32_t call() { return mla_value_proj(&o, &w, &out, nullptr); }
};

void vproj_cases() {
  { VProj p; CASE("vproj ok", SWA_OK, p.call()); }
  { VProj p(64); CASE("vproj Dv 64 ok", SWA_OK, p.call()); }
  { VProj p(96); CASE("vproj Dv 96", SWA_ERR_UNSUPPORTED, p.call()); }
  { VProj p; p.w.dtype = SWA_DTYPE_F32; CASE("vproj f32 weight", SWA_ERR_DTYPE, p.call()); }
  { VProj p; p.w.shape[0] = 3; CASE("vproj head mismatch", SWA_ERR_SHAPE, p.call()); }
  { VProj p; p.out.shape[2] = 64; CASE("vproj out shape", SWA_ERR_SHAPE, p.call()); }
  { VProj p; p.o.shape[2] = p.w.shape[2] = 256; CASE("vproj latent 256", SWA_ERR_UNSUPPORTED, p.call()); }
  { VProj p; p.out.data = p.o.data; CASE("vproj out aliases input", SWA_ERR_ARG, p.call()); }
  { VProj p; p.o.stride[0] = (int64_t)1 << 26; CASE("vproj token stride", SWA_ERR_UNSUPPORTED, p.call()); }
  { VProj p; CASE("vproj null weight", SWA_ERR_NULL, mla_value_proj(&p.o, nullptr, &p.out, nullptr)); }
}

}  // namespace

int main() {
  if (swa_abi_version() != SWA_ABI_VERSION) {
    std::printf("FAIL version\n");
    return 1;
  }
  for (int code = -8; code <= 1; ++code) (void)std::strlen(swa_strerror(code));
  dense_cases();
  bwd_cases();
  sparse_cases();
  vproj_cases();
  std::printf("%d cases, %d failures\n", g_cases, g_failures);
  if (g_failures == 0) std::printf("ALL OK\n");
  return g_failures == 0 ? 0 : 1;
}
