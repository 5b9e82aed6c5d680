"""fa_decode_splitkv (through the C ABI) against the FP64 oracle on the GPU."""
import pytest
import torch

import exact_tiled_attention_flashattention_amd as fa
import synth_inputs as si
from tests.parity import TOL, compare, default_scale, log, make_inputs, oracle_on

pytestmark = pytest.mark.gpu


def _run(B, H, N, Nk, d, dtype, causal, num_splits, seed=0, std=1.0, scale=None):
    q, k, v = make_inputs(B, H, N, Nk, d, d, dtype, seed, std)
    scale = default_scale(d) if scale is None else scale
    log(f"fa_decode_splitkv dtype={dtype} B={B} H={H} N={N} Nk={Nk} d={d} causal={causal} "
        f"splits={num_splits} seed={seed}")
    o, lse = fa.decode_splitkv(q, k, v, causal=causal, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_on(q, k, v, causal, scale)
    compare(o, lse, o_ref, l_ref, dtype, f"decode {dtype} {B}x{H}x{N}x{Nk}x{d} S={num_splits}")
    return q, k, v, o, lse


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("num_splits", [1, 3, 16, 64])
def test_single_query(dtype, d, num_splits):
    _run(2, 3, 1, 1000, d, dtype, False, num_splits, seed=d + num_splits)


@pytest.mark.parametrize("num_splits", [1, 7, 40, 999])
def test_more_splits_than_tiles(num_splits):
    # 130 keys: segments are 64 keys, so most of 40 or 999 segments are empty
    _run(1, 2, 1, 130, 128, "bf16", False, num_splits, seed=3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,Nk", [(4, 777), (5, 600), (9, 9), (12, 5), (1, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_several_rows(dtype, N, Nk, causal):
    _run(2, 2, N, Nk, 64, dtype, causal, 8, seed=N + Nk)


def test_decode_equals_fwd_within_tolerance():
    q, k, v = make_inputs(2, 4, 1, 4096, 128, 128, "bf16", 21)
    o1, l1 = fa.decode_splitkv(q, k, v, num_splits=32)
    o2, l2 = fa.fwd(q, k, v)
    torch.cuda.synchronize()
    tol_o, tol_l = TOL["bf16"]
    assert (o1.float() - o2.float()).abs().max().item() <= tol_o
    assert (l1 - l2).abs().max().item() <= tol_l


def test_deterministic():
    q, k, v = make_inputs(2, 4, 1, 5000, 128, 128, "bf16", 22)
    o1, l1 = fa.decode_splitkv(q, k, v, num_splits=16)
    o2, l2 = fa.decode_splitkv(q, k, v, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_b8_h32_nk32768_d128_sampled_heads():
    """The long-context decode at full size with 64 splits, launched as the
    bench launches it; the oracle checks eight whole heads."""
    w = si.WORKLOADS["decode_b8_h32_nk32768_d128"]
    s = w.shapes[0]
    log(f"fa_decode_splitkv full-size {w.name}")
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    o, lse = fa.decode_splitkv(q, k, v, num_splits=w.num_splits)
    torch.cuda.synchronize()
    heads = [(0, 0), (s.B - 1, s.H - 1), (3, 17), (5, 2), (1, 30), (6, 9), (2, 0), (7, 16)]
    o_ref, l_ref = oracle_on(q, k, v, False, default_scale(s.d), heads)
    o_s = torch.stack([o[b, h] for b, h in heads])
    l_s = torch.stack([lse[b, h] for b, h in heads])
    compare(o_s, l_s, o_ref, l_ref, w.dtype, w.name)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
