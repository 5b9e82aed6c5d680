"""fa_bwd (through the C ABI) against the FP64 oracle's backward on the GPU.

The forward outputs o and lse that fa_bwd consumes come from fa_fwd on the
same inputs, as a training step would pass them."""
import pytest
import torch

import exact_tiled_attention_flashattention_amd as fa
import synth_inputs as si
from tests.parity import compare_grads, default_scale, log, make_inputs, oracle_bwd_on

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, Nk, d, dtype, seed, std=1.0):
    q, k, v = make_inputs(B, H, N, Nk, d, d, dtype, seed, std)
    dout, _, _ = make_inputs(B, H, N, 1, d, d, dtype, seed + 500)
    return q, k, v, dout


def _run(B, H, N, Nk, d, dtype, causal, seed=0, std=1.0, scale=None):
    q, k, v, dout = _inputs(B, H, N, Nk, d, dtype, seed, std)
    scale = default_scale(d) if scale is None else scale
    log(f"fa_bwd dtype={dtype} B={B} H={H} N={N} Nk={Nk} d={d} causal={causal} seed={seed}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    grads = fa.bwd(q, k, v, o, lse, dout, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle_bwd_on(q, k, v, dout, causal, scale)
    compare_grads(grads, ref, dtype, f"bwd {dtype} {B}x{H}x{N}x{Nk}x{d} causal={causal}")
    return grads


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N,Nk", [(77, 513), (300, 300), (129, 1), (1, 1000), (40, 17)])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged(dtype, d, N, Nk, causal):
    _run(1, 2, N, Nk, d, dtype, causal, seed=N + Nk + d)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,Nk", [(2048, 2048), (2100, 2300), (2300, 2100)])
def test_causal_long_rows_d64(dtype, N, Nk):
    # d = 64 causal with N >= 2048 takes the 32-key-per-wave dK/dV kernel:
    # several 256-key blocks and 64-row steps, ragged ends, N > Nk rows that
    # see no key and N < Nk
    _run(1, 2, N, Nk, 64, dtype, True, seed=N + Nk)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_several_blocks(dtype, d, causal):
    # several query and key blocks of every kernel, with ragged ends
    _run(2, 3, 700, 650, d, dtype, causal, seed=d + int(causal))


def test_scale_zero():
    # uniform weights: dq = dk = 0
    dq, dk, dv = _run(1, 2, 64, 96, 64, "bf16", True, seed=3, scale=0.0)
    assert torch.count_nonzero(dq).item() == 0 and torch.count_nonzero(dk).item() == 0


def test_deterministic():
    q, k, v, dout = _inputs(2, 2, 333, 444, 64, "bf16", 7)
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd(q, k, v, o, lse, dout, causal=True)
    g2 = fa.bwd(q, k, v, o, lse, dout, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_prefill_b64_h16_n1024_d64_all_heads():
    """The backward at the B64 x H16 x 1024 causal prefill size, in the launch
    configuration the benchmark times; every element of the gradients of all
    1024 heads against the oracle, into NaN-prefilled dq, dk, dv."""
    w = si.WORKLOADS["prefill_b64_h16_n1024_d64"]
    s = w.shapes[0]
    log(f"fa_bwd full-size {w.name}")
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    dout, _, _ = si.device_qkv(si.Shape(s.B, s.H, s.N, 1, s.dv, s.dv), w.seed + 100, w.dtype,
                               "cuda", 1.0)
    scale = default_scale(s.d)
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.bwd(q, k, v, o, lse, dout, causal=True, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for b0 in range(0, s.B, 8):
        sl = slice(b0, b0 + 8)
        ref = oracle_bwd_on(q[sl], k[sl], v[sl], dout[sl], True, scale)
        compare_grads((dq[sl], dk[sl], dv[sl]), ref, "bf16", f"bwd full-size batches {b0}..{b0 + 7}")
    log(f"  bwd full-size: {s.B * s.H}/{s.B * s.H} heads compared element by element")


@pytest.mark.parametrize("B,H,N,Nk,causal", [(8, 16, 1024, 1024, False), (5, 7, 1800, 1900, True),
                                              (8, 16, 2100, 1900, True)])
def test_several_blocks_per_workgroup_all_heads(B, H, N, Nk, causal):
    """Shapes with more 256-key (256-row) blocks than the GPU holds
    workgroups at once: under the mask one workgroup of the d = 64 dK/dV and
    dQ kernels walks several pairs of blocks (a head count that is not a
    multiple of 8 in the second case; rows that see no key in the third),
    without it each block has a workgroup of its own.  Every element of the
    gradients of every head against the oracle."""
    q, k, v, dout = _inputs(B, H, N, Nk, 64, "bf16", seed=N + Nk)
    scale = default_scale(64)
    log(f"fa_bwd several blocks per workgroup B={B} H={H} N={N} Nk={Nk} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.bwd(q, k, v, o, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle_bwd_on(q, k, v, dout, causal, scale)
    compare_grads((dq, dk, dv), ref, "bf16", f"bwd B={B} H={H} N={N} Nk={Nk}")


@pytest.mark.parametrize("N,Nk,causal", [(1100, 1200, True), (1024, 1000, False)])
def test_d128_row_blocks_all_heads(N, Nk, causal):
    """d = dv = 128 with more 256-row blocks than resident workgroups,
    N != Nk (ragged): the 32x32 dQ kernel with one 32-key sub-block per
    step (a persistent walk of pairs under the mask).  Every element of
    every head against the oracle."""
    B, H = 8, 16
    q, k, v, dout = _inputs(B, H, N, Nk, 128, "bf16", seed=N + Nk + 128)
    scale = default_scale(128)
    log(f"fa_bwd d=128 B={B} H={H} N={N} Nk={Nk} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.bwd(q, k, v, o, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle_bwd_on(q, k, v, dout, causal, scale)
    compare_grads((dq, dk, dv), ref, "bf16", f"bwd d=128 B={B} H={H} N={N} Nk={Nk} causal={causal}")


@pytest.mark.parametrize("N,Nk,causal", [(1100, 1200, True), (1024, 1000, False)])
def test_d64_dv128_row_blocks_all_heads(N, Nk, causal):
    """d = 64 with dv = 128, more 256-row blocks than resident workgroups,
    N != Nk: the 32x32 dQ kernel with V rows twice as long as K rows.  Every
    element of every head against the oracle."""
    B, H, d, dv = 8, 16, 64, 128
    q, k, v = make_inputs(B, H, N, Nk, d, dv, "bf16", 71)
    dout, _, _ = make_inputs(B, H, N, 1, dv, dv, "bf16", 72)
    scale = default_scale(d)
    log(f"fa_bwd d={d} dv={dv} B={B} H={H} N={N} Nk={Nk} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dvv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.bwd(q, k, v, o, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk, dv=dvv)
    torch.cuda.synchronize()
    ref = oracle_bwd_on(q, k, v, dout, causal, scale)
    compare_grads((dq, dk, dvv), ref, "bf16", f"bwd d={d} dv={dv} B={B} H={H} N={N} Nk={Nk}")
