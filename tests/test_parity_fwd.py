"""fa_fwd (through the C ABI) against the FP64 oracle on the GPU."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_flashattention_amd as fa
import oracle
import synth_inputs as si
from tests.parity import (compare, default_scale, log, make_inputs, oracle_on,
                          score_scaled_tolerance)

pytestmark = pytest.mark.gpu


def _run(B, H, N, Nk, d, dtype, causal, seed=0, std=1.0, scale=None, large_scores=False):
    q, k, v = make_inputs(B, H, N, Nk, d, d, dtype, seed, std)
    scale = default_scale(d) if scale is None else scale
    log(f"fa_fwd dtype={dtype} B={B} H={H} N={N} Nk={Nk} d={d} causal={causal} scale={scale:.4g} seed={seed}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_on(q, k, v, causal, scale)
    tol = score_scaled_tolerance(q, k, v, scale, dtype) if large_scores else None
    compare(o, lse, o_ref, l_ref, dtype, f"fwd {dtype} {B}x{H}x{N}x{Nk}x{d} c={int(causal)}", tol)
    return q, k, v, o, lse


def test_single_head_f32():
    w = si.WORKLOADS["single_head_f32"]
    s = w.shapes[0]
    _run(s.B, s.H, s.N, s.Nk, s.d, "f32", False, seed=w.seed)


@pytest.mark.parametrize("shape", si.WORKLOADS["ragged_f32"].shapes, ids=str)
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_f32(shape, causal):
    _run(shape.B, shape.H, shape.N, shape.Nk, shape.d, "f32", causal, seed=0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N,Nk", [(300, 300), (77, 513), (513, 77), (1, 1000), (256, 256),
                                  (129, 1), (1, 1), (64, 64), (100, 150)])
@pytest.mark.parametrize("causal", [False, True])
def test_small_multi_tile(dtype, d, N, Nk, causal):
    _run(2, 3, N, Nk, d, dtype, causal, seed=N * 7 + Nk + d)


# d = dv = 64 runs on the two-workgroup 32x32 kernel up to 3072 keys and on
# the ping-pong 16x16 kernel beyond; these shapes sit on both sides.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,Nk", [(300, 3072), (300, 3073), (3200, 3200), (1, 4100)])
@pytest.mark.parametrize("causal", [False, True])
def test_d64_key_range_dispatch(dtype, N, Nk, causal):
    _run(1, 2, N, Nk, 64, dtype, causal, seed=N + Nk)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scale_zero_is_mean_of_visible_values(dtype):
    _run(1, 2, 200, 333, 64, dtype, True, seed=9, scale=0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_large_scores_stay_finite(dtype):
    # scores of order hundreds: scale 4 on N(0, 2) inputs
    _run(1, 2, 130, 260, 64, dtype, True, seed=10, std=2.0, scale=4.0, large_scores=True)


def test_constant_values_give_constant_output():
    q, k, v = make_inputs(2, 2, 190, 190, 64, 64, "bf16", 11)
    v = torch.full_like(v, 0.75)
    o, _ = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0.75).item()


def test_deterministic():
    q, k, v = make_inputs(2, 4, 384, 384, 64, 64, "bf16", 12)
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_b64_h16_n1024_d64_sampled_heads():
    """The GPT-2-medium-shaped prefill at full size, launched as the bench
    launches it; the oracle checks four whole heads."""
    w = si.WORKLOADS["prefill_b64_h16_n1024_d64"]
    s = w.shapes[0]
    log(f"fa_fwd full-size {w.name}")
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    o, lse = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    heads = [(0, 0), (s.B - 1, s.H - 1), (17, 5), (40, 11)]
    o_ref, l_ref = oracle_on(q, k, v, True, default_scale(s.d), heads)
    o_s = torch.stack([o[b, h] for b, h in heads])
    l_s = torch.stack([lse[b, h] for b, h in heads])
    compare(o_s, l_s, o_ref, l_ref, w.dtype, w.name)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()


def test_prefill_b2_h32_n8192_d128_sampled_rows():
    """The long causal prefill at full size; the oracle checks row windows of
    two heads (a causal row i only needs keys 0..i, so each window is the
    oracle on that window's queries and the key prefix it sees)."""
    w = si.WORKLOADS["prefill_b2_h32_n8192_d128"]
    s = w.shapes[0]
    log(f"fa_fwd full-size {w.name}")
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    o, lse = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    scale = default_scale(s.d)
    for (b, h) in ((0, 0), (1, 31)):
        for (r0, nr) in ((0, 64), (4000, 96), (8192 - 64, 64)):
            qs = si.as_f64(q[b, h, r0:r0 + nr])
            ks = si.as_f64(k[b, h, :r0 + nr])
            vs = si.as_f64(v[b, h, :r0 + nr])
            o_ref, l_ref = oracle.attention(qs, ks, vs, causal=True, scale=scale)
            compare(o[b, h, r0:r0 + nr], lse[b, h, r0:r0 + nr], o_ref, l_ref, w.dtype,
                    f"{w.name} head ({b},{h}) rows {r0}..{r0 + nr - 1}")
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
