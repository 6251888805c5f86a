"""GPU parity of the sparse MLA value up-projection (mla_value_proj, through the C ABI) and of
the composed sparse_mla (attention, then projection) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import mla_value_proj_ref, sparse_mla_ref_rows, sparse_mla_value_ref
from sliding_window_gqa_varlen_amd import mla_value_proj, sparse_mla, workloads as W
from tests.gpu_util import BF16_MAX_ABS, assert_lse_match, dev

pytestmark = pytest.mark.gpu

# bf16 output: one rounding (relative 2^-8) on top of a 512-term fp32 accumulation
REL_ROUNDING, ABS_ACCUM = 2.0 ** -8, 1e-3


def o_latent(seed, T, H):
    return W.round_to_bf16(W.normal(seed, W.STREAM_LATENT, (T, H, 512)))


def check_proj(got, ref):
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert err.max() <= BF16_MAX_ABS, f"max abs error {err.max():.3e}"
    bad = err > REL_ROUNDING * np.abs(ref) + ABS_ACCUM
    assert not bad.any(), f"{bad.sum()} elements beyond one bf16 rounding, first at {np.argwhere(bad)[0]}"


def run_proj(o, w, out=None):
    r = mla_value_proj(o, w, out=out)
    torch.cuda.synchronize()
    return r.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,H,Dv", [(1, 4, 128), (255, 16, 64), (300, 16, 128), (1000, 128, 128),
                                    (2000, 2, 64), (70000, 1, 64)])
def test_projection_elementwise(gpu, T, H, Dv):
    """T not a multiple of the 256-token block; H = 1 makes each workgroup walk many blocks."""
    o = o_latent(T + H, T, H)
    w = W.make_value_weight(Dv + H, H, Dv)
    got = run_proj(dev(o, torch.bfloat16), dev(w, torch.bfloat16))
    check_proj(got, mla_value_proj_ref(o, w))


def test_projection_strided_views(gpu):
    """o inside a [T, H, 576] buffer, every other row of a [H, 2 Dv, 512] weight, out inside a wider buffer."""
    T, H, Dv = 777, 8, 128
    o = o_latent(21, T, H)
    w = W.make_value_weight(22, H, Dv)
    o_big = torch.zeros(T, H, 576, dtype=torch.bfloat16, device="cuda:0")
    o_big[:, :, :512] = dev(o, torch.bfloat16)
    w_big = torch.zeros(H, 2 * Dv, 512, dtype=torch.bfloat16, device="cuda:0")
    w_big[:, ::2, :] = dev(w, torch.bfloat16)
    out_big = torch.full((T, H, 2 * Dv), 7.0, dtype=torch.bfloat16, device="cuda:0")
    out = out_big[:, :, Dv:]
    mla_value_proj(o_big[:, :, :512], w_big[:, ::2, :], out=out)
    torch.cuda.synchronize()
    check_proj(out.float().cpu().numpy().astype(np.float64), mla_value_proj_ref(o, w))
    assert torch.all(out_big[:, :, :Dv] == 7.0), "the projection wrote outside its output view"


def test_projection_zero_rows_and_identity_heads(gpu):
    """Zero latent rows (empty attention rows) project to exact zeros; W[h] = [I | 0] copies o."""
    T, H, Dv = 300, 4, 64
    o = o_latent(23, T, H)
    o[100:140] = 0.0
    w = W.make_value_weight(24, H, Dv)
    w[2] = 0.0
    w[2, np.arange(Dv), np.arange(Dv) + 64] = 1.0
    got = run_proj(dev(o, torch.bfloat16), dev(w, torch.bfloat16))
    check_proj(got, mla_value_proj_ref(o, w))
    assert np.all(got[100:140] == 0.0)
    np.testing.assert_array_equal(got[:, 2, :], o[:, 2, 64:64 + Dv])


def test_projection_full_size_sampled(gpu):
    """The bench shape (16384 tokens, 128 heads, value_dim 128), checked on sampled tokens."""
    T, H, Dv = 16384, 128, 128
    o = o_latent(25, T, H)
    w = W.make_value_weight(26, H, Dv)
    got = run_proj(dev(o, torch.bfloat16), dev(w, torch.bfloat16))
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([rng.integers(0, T, 200), [0, 255, 256, 8191, 8192, T - 257, T - 1]]))
    check_proj(got[toks], mla_value_proj_ref(o[toks], w))


def test_projection_full_size_every_element_against_a_pinned_gpu_fp32_reference(gpu):
    """Every element of the bench shape against a plain fp32 torch restatement on the GPU
    (per head [T, 512] x [512, Dv]), which is first pinned to the fp64 oracle on sampled tokens."""
    T, H, Dv = 16384, 128, 128
    o = o_latent(25, T, H)
    w = W.make_value_weight(26, H, Dv)
    got = run_proj(dev(o, torch.bfloat16), dev(w, torch.bfloat16))
    of = torch.from_numpy(o).to("cuda:0").float().permute(1, 0, 2).contiguous()       # [H, T, 512]
    wt = torch.from_numpy(w).to("cuda:0").float().transpose(1, 2).contiguous()        # [H, 512, Dv]
    ref = torch.bmm(of, wt).permute(1, 0, 2).contiguous().cpu().numpy().astype(np.float64)  # [T, H, Dv]
    toks = np.unique(np.random.default_rng(9).integers(0, T, 64))
    np.testing.assert_allclose(ref[toks], mla_value_proj_ref(o[toks], w), rtol=0, atol=1e-4)
    check_proj(got, ref)


def test_projection_repeat_runs_are_bitwise_identical(gpu):
    o = dev(o_latent(27, 600, 16), torch.bfloat16)
    w = dev(W.make_value_weight(28, 16, 128), torch.bfloat16)
    np.testing.assert_array_equal(run_proj(o, w), run_proj(o, w))


# ---------------------------------------------------------------- composed sparse_mla
def run_composed(inp, w):
    q, lat, kpe = (dev(inp[n], torch.bfloat16) for n in ("q", "latent", "k_pe"))
    idx = torch.from_numpy(inp["indices"]).to("cuda:0")
    ids = torch.from_numpy(inp["doc_ids"]).to("cuda:0")
    out, lse = sparse_mla(q, lat, kpe, idx, ids, dev(w, torch.bfloat16), inp["scale"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,topk,Dv", [(300, 64, 128), (700, 128, 64)])
def test_composed_small_elementwise(gpu, T, topk, Dv):
    w_ = W.SparseWorkload("sparse_small", T=T, H=128, d_latent=512, d_rope=64, topk=topk, scale=1.0 / 24.0,
                          seed=T, doc_dist=("uniform", 64, 600))
    inp = W.make_sparse(w_)
    w = W.make_value_weight(T, 128, Dv)
    out, lse = run_composed(inp, w)
    ref_o, ref_l = sparse_mla_value_ref(inp["q"], inp["latent"], inp["k_pe"], inp["indices"], inp["doc_ids"], w,
                                        inp["scale"])
    assert np.abs(out - ref_o).max() <= BF16_MAX_ABS
    assert_lse_match(lse, ref_l, BF16_MAX_ABS)


def test_composed_full_size_sampled(gpu):
    inp = W.make_sparse(W.WORKLOADS[4])
    w = W.make_value_weight(4, inp["q"].shape[1], 128)
    out, lse = run_composed(inp, w)
    assert np.all(np.isfinite(out))
    T = out.shape[0]
    cu = np.concatenate([[0], np.cumsum(inp["lengths"])])
    rng = np.random.default_rng(5)
    toks = list(rng.integers(0, T, 24)) + [int(s) for s in cu[:-1]] + [int(e) - 1 for e in cu[1:]]
    toks = np.array(sorted(set(toks)))
    ref_o, ref_l = sparse_mla_ref_rows(inp["q"], inp["latent"], inp["k_pe"], inp["indices"], inp["doc_ids"],
                                       inp["scale"], toks)
    assert np.abs(out[toks] - mla_value_proj_ref(ref_o, w)).max() <= BF16_MAX_ABS
    assert_lse_match(lse[toks], ref_l, BF16_MAX_ABS)
