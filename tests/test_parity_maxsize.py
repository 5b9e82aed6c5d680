"""The largest per-head slices the library accepts, on the GPU against the
FP64 oracle.  Each per-head K and V slice is just under 2 GiB, the limit of
the 32-bit buffer offsets the kernels use within a head: the last key
tiles sit at the top of that range, and the second head starts past 2 GiB
(its base address comes from 64-bit arithmetic).  Key counts are ragged
(not a multiple of 64).  The oracle checks every head of a few query rows."""
import pytest
import torch

import exact_tiled_attention_flashattention_amd as fa
import oracle
import synth_inputs as si
from tests.parity import compare, default_scale, log, oracle_on

pytestmark = pytest.mark.gpu


def _largest_nk(d):
    # Nk * d * 2 bytes < 2^31, less a ragged tail.
    return (1 << 31) // (2 * d) - 61


def _check(o, lse, o_ref, l_ref, heads, name):
    o_s = torch.stack([o[b, h] for b, h in heads])
    l_s = torch.stack([lse[b, h] for b, h in heads])
    compare(o_s, l_s, o_ref, l_ref, "bf16", name)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_largest_head_slice(d):
    # d = 64 runs the 16x16 ping-pong kernel here, d = 128 the 32x32 kernel.
    s = si.Shape(1, 2, 8, _largest_nk(d), d, d)
    log(f"fa_fwd largest head slice B=1 H=2 N=8 Nk={s.Nk} d={d} causal")
    q, k, v = si.device_qkv(s, 21, "bf16", "cuda", 1.0)
    o, lse = fa.fwd(q, k, v, causal=True, scale=default_scale(d))
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 1)]
    o_ref, l_ref = oracle_on(q, k, v, True, default_scale(d), heads)
    _check(o, lse, o_ref, l_ref, heads, f"fwd Nk={s.Nk} d={d}")


@pytest.mark.parametrize("num_splits", [0, 64])
def test_decode_largest_head_slice(num_splits):
    d = 128
    s = si.Shape(1, 2, 1, _largest_nk(d), d, d)
    log(f"fa_decode_splitkv largest head slice B=1 H=2 N=1 Nk={s.Nk} d={d} splits={num_splits}")
    q, k, v = si.device_qkv(s, 22, "bf16", "cuda", 1.0)
    o, lse = fa.decode_splitkv(q, k, v, num_splits=num_splits)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 1)]
    o_ref, l_ref = oracle_on(q, k, v, False, default_scale(d), heads)
    _check(o, lse, o_ref, l_ref, heads, f"decode Nk={s.Nk} S={num_splits}")


def test_gqa_largest_head_slice():
    d, G = 128, 4
    nk = _largest_nk(d)
    sq = si.Shape(1, 2 * G, 2, 1, d, d)
    skv = si.Shape(1, 2, 1, nk, d, d)
    log(f"fa_decode_splitkv_gqa largest head slice B=1 Hq=8 Hkv=2 N=2 Nk={nk} d={d}")
    q, _, _ = si.device_qkv(sq, 23, "bf16", "cuda", 1.0)
    _, k, v = si.device_qkv(skv, 24, "bf16", "cuda", 1.0)
    o, lse = fa.decode_splitkv_gqa(q, k, v, num_splits=0)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 2 * G - 1)]
    os_, ls_ = [], []
    for b, h in heads:
        r = oracle.attention(si.as_f64(q[b, h]), si.as_f64(k[b, h // G]), si.as_f64(v[b, h // G]),
                             causal=False, scale=default_scale(d))
        os_.append(r[0])
        ls_.append(r[1])
    import numpy as np
    _check(o, lse, np.stack(os_), np.stack(ls_), heads, f"gqa Nk={nk}")


def test_bwd_largest_head_slice():
    # One head is checked (the second, past 2 GiB): the oracle's gradients of
    # a slice this long take tens of GB of host memory in fp64.
    from tests.parity import compare_grads, oracle_bwd_on
    d = 128
    s = si.Shape(1, 2, 8, _largest_nk(d), d, d)
    log(f"fa_bwd largest head slice B=1 H=2 N=8 Nk={s.Nk} d={d} causal")
    q, k, v = si.device_qkv(s, 25, "bf16", "cuda", 1.0)
    dout, _, _ = si.device_qkv(si.Shape(1, 2, 8, 1, d, d), 26, "bf16", "cuda", 1.0)
    scale = default_scale(d)
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dout, causal=True, scale=scale)
    torch.cuda.synchronize()
    heads = [(0, 1)]
    ref = oracle_bwd_on(q, k, v, dout, True, scale, heads=heads)
    got = tuple(torch.stack([g[b, h] for b, h in heads]) for g in (dq, dk, dv))
    compare_grads(got, ref, "bf16", f"bwd Nk={s.Nk}")


def test_bwd_largest_head_slice_d64_unmasked():
    # d = 64 without the mask runs the 32-key dK/dV kernel: one head of the
    # largest accepted slice (the second, past 2 GiB) against the oracle.
    from tests.parity import compare_grads, oracle_bwd_on
    d = 64
    s = si.Shape(1, 2, 8, _largest_nk(d), d, d)
    log(f"fa_bwd largest head slice B=1 H=2 N=8 Nk={s.Nk} d={d} non-causal")
    q, k, v = si.device_qkv(s, 27, "bf16", "cuda", 1.0)
    dout, _, _ = si.device_qkv(si.Shape(1, 2, 8, 1, d, d), 28, "bf16", "cuda", 1.0)
    scale = default_scale(d)
    o, lse = fa.fwd(q, k, v, causal=False, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dout, causal=False, scale=scale)
    torch.cuda.synchronize()
    heads = [(0, 1)]
    ref = oracle_bwd_on(q, k, v, dout, False, scale, heads=heads)
    got = tuple(torch.stack([g[b, h] for b, h in heads]) for g in (dq, dk, dv))
    compare_grads(got, ref, "bf16", f"bwd Nk={s.Nk} d={d}")
