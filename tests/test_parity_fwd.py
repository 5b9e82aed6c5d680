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
    tol = score_scaled_tolerance(q, k, v, scale, dtype, causal) if large_scores else None
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


def _nan_outputs(B, H, N, dv, dtype):
    """Outputs prefilled with NaN: an element the kernels never write fails
    the comparison instead of passing with stale finite data."""
    o = torch.full((B, H, N, dv), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def _compare_all_heads(q, k, v, o, lse, causal, scale, dtype, what, batches_per_chunk):
    """Every element of every head against the oracle, a few batches at a
    time so that host memory stays bounded.  Returns the number of heads."""
    B, H = q.shape[:2]
    for b0 in range(0, B, batches_per_chunk):
        b1 = min(B, b0 + batches_per_chunk)
        o_ref, l_ref = oracle_on(q[b0:b1], k[b0:b1], v[b0:b1], causal, scale)
        compare(o[b0:b1], lse[b0:b1], o_ref, l_ref, dtype, f"{what} batches {b0}..{b1 - 1}")
    log(f"  {what}: {B * H}/{B * H} heads compared element by element")
    return B * H


def test_prefill_b64_h16_n1024_d64_all_heads():
    """The GPT-2-medium-shaped prefill at full size, launched as the bench
    launches it (persistent grid with the XCD-aware unit numbering); every
    element of all 1024 heads against the oracle."""
    w = si.WORKLOADS["prefill_b64_h16_n1024_d64"]
    s = w.shapes[0]
    log(f"fa_fwd full-size {w.name}")
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    o, lse = _nan_outputs(s.B, s.H, s.N, s.dv, q.dtype)
    fa.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    n = _compare_all_heads(q, k, v, o, lse, True, default_scale(s.d), w.dtype, w.name, 8)
    assert n == 1024


def test_prefill_b2_h32_n8192_d128_all_heads():
    """The long causal prefill at full size: every element of all 64 heads
    against the oracle (every 256-row query block, every causal tile skip)."""
    w = si.WORKLOADS["prefill_b2_h32_n8192_d128"]
    s = w.shapes[0]
    log(f"fa_fwd full-size {w.name}")
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    o, lse = _nan_outputs(s.B, s.H, s.N, s.dv, q.dtype)
    fa.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    scale = default_scale(s.d)
    for h0 in range(0, s.H, 8):
        sl = (slice(None), slice(h0, h0 + 8))
        o_ref, l_ref = oracle_on(q[sl], k[sl], v[sl], True, scale)
        compare(o[sl], lse[sl], o_ref, l_ref, w.dtype, f"{w.name} heads {h0}..{h0 + 7}")
    log(f"  {w.name}: {s.B * s.H}/{s.B * s.H} heads compared element by element")


# Small shapes whose grid and head counts are multiples of 8, so that the
# persistent kernels number their units XCD by XCD, checked in full.
@pytest.mark.parametrize("B,H,N,Nk,d,dv", [
    (1, 8, 1024, 1024, 64, 64),      # 32x32 kernel, two workgroups per CU
    (1, 16, 1000, 1000, 64, 64),     # ragged last block
    (1, 16, 1280, 1280, 64, 64),     # five query blocks: the odd middle one alone
    (1, 8, 2048, 2048, 128, 128),    # 32x32 kernel, one workgroup per CU
    (1, 8, 4096, 4096, 64, 64),      # ping-pong kernel (long key range)
    (1, 8, 2048, 2048, 128, 64),     # ping-pong kernel, dv = 64
])
@pytest.mark.parametrize("causal", [False, True])
def test_xcd_unit_numbering(B, H, N, Nk, d, dv, causal):
    q, k, v = make_inputs(B, H, N, Nk, d, dv, "bf16", seed=B + H + N + d + dv)
    scale = default_scale(d)
    log(f"fa_fwd xcd numbering B={B} H={H} N={N} Nk={Nk} d={d} dv={dv} causal={causal}")
    o, lse = _nan_outputs(B, H, N, dv, q.dtype)
    fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_on(q, k, v, causal, scale)
    compare(o, lse, o_ref, l_ref, "bf16", f"xcd {B}x{H}x{N}x{Nk}x{d}x{dv} c={int(causal)}")
