"""Helpers for GPU parity tests: move seeded inputs to the device, compare with the oracle."""
import numpy as np
import torch

BF16_MAX_ABS = 2e-2      # out and lse, bf16 workloads
F32_NORMWISE_REL = 1e-5  # max|diff| / max|ref|, out and lse separately, f32 workloads


def dev(x, dtype, device="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device).to(dtype)


def tdtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def run_dense(inp, dtype, device="cuda:0", with_lse=True, window=None, sinks="inp"):
    from sliding_window_gqa_varlen_amd import varlen_attn_fwd
    td = tdtype(dtype)
    q, k, v = dev(inp["q"], td, device), dev(inp["k"], td, device), dev(inp["v"], td, device)
    cu = torch.from_numpy(inp["cu_seqlens"]).to(device)
    s = inp["sinks"] if isinstance(sinks, str) and sinks == "inp" else sinks
    s = None if s is None else torch.from_numpy(np.asarray(s, np.float32)).to(device)
    out, lse = varlen_attn_fwd(q, k, v, cu, inp["n_docs"], inp["window"] if window is None else window,
                               inp["scale"], s, return_lse=with_lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = None if lse is None else lse.cpu().numpy().astype(np.float64)
    return o, l


def assert_lse_match(got, ref, tol, what="lse"):
    """-inf entries must coincide exactly; finite entries within tol (absolute)."""
    ninf_g, ninf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf pattern differs at {np.argwhere(ninf_g != ninf_r)[:5]}"
    fin = ~ninf_r
    assert np.all(np.isfinite(got[fin])), f"{what}: non-finite values"
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def assert_dense_parity(dtype, out, lse, ref_out, ref_lse):
    assert np.all(np.isfinite(out)), "non-finite output"
    if dtype == "bf16":
        err = np.abs(out - ref_out).max() if out.size else 0.0
        assert err <= BF16_MAX_ABS, f"out: max abs error {err:.3e} > {BF16_MAX_ABS}"
        if lse is not None:
            assert_lse_match(lse, ref_lse, BF16_MAX_ABS)
    else:
        denom = max(np.abs(ref_out).max(), 1e-30)
        rel = np.abs(out - ref_out).max() / denom
        assert rel <= F32_NORMWISE_REL, f"out: normwise relative error {rel:.3e} > {F32_NORMWISE_REL}"
        if lse is not None:
            fin = np.isfinite(ref_lse)
            denom = max(np.abs(ref_lse[fin]).max() if fin.any() else 0.0, 1e-30)
            assert_lse_match(lse, ref_lse, F32_NORMWISE_REL * denom)
