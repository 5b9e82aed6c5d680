"""Head dimensions beyond d = dv in {32, 64, 128}: dv != d and d or dv = 256,
through fa_fwd, fa_decode_splitkv(_gqa) and fa_bwd, against the FP64 oracle
(whose V is [Nk, dv] like the pages' convention)."""
import pytest
import torch

import exact_tiled_attention_flashattention_amd as fa
from tests.parity import (compare, compare_grads, default_scale, log, make_inputs, oracle_bwd_on,
                          oracle_on)

pytestmark = pytest.mark.gpu

DIMS = [(64, 128), (128, 64), (32, 256), (256, 32), (256, 256), (128, 256)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d,dv", DIMS)
@pytest.mark.parametrize("N,Nk,causal", [(77, 513, True), (300, 300, False), (40, 17, True)])
def test_fwd(dtype, d, dv, N, Nk, causal):
    q, k, v = make_inputs(1, 2, N, Nk, d, dv, dtype, seed=d + dv + N)
    scale = default_scale(d)
    log(f"fa_fwd dtype={dtype} N={N} Nk={Nk} d={d} dv={dv} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_on(q, k, v, causal, scale)
    compare(o, lse, o_ref, l_ref, dtype, f"fwd {dtype} d={d} dv={dv} {N}x{Nk}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,dv", DIMS)
@pytest.mark.parametrize("G,N,splits", [(1, 1, 16), (4, 1, 7), (1, 3, 5), (8, 2, 0)])
def test_decode(dtype, d, dv, G, N, splits):
    B, Hkv, Nk = 2, 2, 1500
    q, _, _ = make_inputs(B, Hkv * G, N, 1, d, dv, dtype, seed=d + G)
    _, k, v = make_inputs(B, Hkv, 1, Nk, d, dv, dtype, seed=dv + 1000)
    scale = default_scale(d)
    log(f"fa_decode_splitkv_gqa dtype={dtype} d={d} dv={dv} G={G} N={N} splits={splits}")
    o, lse = fa.decode_splitkv_gqa(q, k, v, causal=True, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_on(q, k.repeat_interleave(G, dim=1).contiguous(),
                             v.repeat_interleave(G, dim=1).contiguous(), True, scale)
    compare(o, lse, o_ref, l_ref, dtype, f"decode {dtype} d={d} dv={dv} G={G} N={N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,dv", DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_bwd(dtype, d, dv, causal):
    N, Nk = 150, 230
    q, k, v = make_inputs(1, 2, N, Nk, d, dv, dtype, seed=d * 3 + dv)
    dout, _, _ = make_inputs(1, 2, N, 1, dv, dv, dtype, seed=d + dv + 7)
    scale = default_scale(d)
    log(f"fa_bwd dtype={dtype} d={d} dv={dv} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    grads = fa.bwd(q, k, v, o, lse, dout, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle_bwd_on(q, k, v, dout, causal, scale)
    compare_grads(grads, ref, dtype, f"bwd {dtype} d={d} dv={dv} causal={causal}")
