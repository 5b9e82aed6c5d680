"""fa_decode_splitkv_noalloc (through the C ABI) against fa_decode_splitkv
with a workspace, and against the oracle, on two calls in a row -- the
second one smaller, so that it runs over what the first left in the static
scratch."""
import pytest
import torch

import exact_tiled_attention_flashattention_amd as fa
import synth_inputs as si
from tests.parity import compare, default_scale, log, make_inputs, oracle_on

pytestmark = pytest.mark.gpu


def _both(q, k, v, causal, num_splits, what):
    scale = default_scale(q.shape[-1])
    nan_o = lambda: torch.full((*q.shape[:3], v.shape[3]), float("nan"), dtype=q.dtype,
                               device=q.device)
    nan_l = lambda: torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o1, l1 = fa.decode_splitkv_noalloc(q, k, v, causal=causal, scale=scale, num_splits=num_splits,
                                       out=nan_o(), lse=nan_l())
    o2, l2 = fa.decode_splitkv(q, k, v, causal=causal, scale=scale, num_splits=num_splits,
                               out=nan_o(), lse=nan_l())
    torch.cuda.synchronize()
    log(f"{what}: noalloc vs workspace bitwise equal: "
        f"{torch.equal(o1, o2) and torch.equal(l1, l2)}")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    return o1, l1, scale


def test_noalloc_two_calls_second_smaller():
    # call 1: the long-context decode workload, 64 splits (8,454,144 bytes of partials)
    w = si.WORKLOADS["decode_b8_h32_nk32768_d128"]
    s = w.shapes[0]
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    o, lse, scale = _both(q, k, v, False, w.num_splits, "call 1 " + w.name)
    for b in (0, s.B - 1):
        o_ref, l_ref = oracle_on(q[b:b + 1], k[b:b + 1], v[b:b + 1], False, scale)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, w.dtype, f"noalloc call 1 batch {b}")
    del q, k, v
    # call 2: smaller, several rows, causal, more splits than 64-key segments
    q, k, v = make_inputs(2, 3, 4, 700, 64, 64, "bf16", seed=77)
    o, lse, scale = _both(q, k, v, True, 20, "call 2 (2x3x4x700, d=64)")
    o_ref, l_ref = oracle_on(q, k, v, True, scale)
    compare(o, lse, o_ref, l_ref, "bf16", "noalloc call 2")


@pytest.mark.parametrize("dtype,d,num_splits", [("f32", 128, 16), ("f16", 32, 0), ("bf16", 256, 5)])
def test_noalloc_other_kernels(dtype, d, num_splits):
    """The VALU segment kernel at fp32 and d = 256, the automatic split count."""
    q, k, v = make_inputs(1, 4, 1, 3000, d, d, dtype, seed=d + num_splits)
    o, lse, scale = _both(q, k, v, False, num_splits, f"{dtype} d={d} splits={num_splits}")
    o_ref, l_ref = oracle_on(q, k, v, False, scale)
    compare(o, lse, o_ref, l_ref, dtype, f"noalloc {dtype} d={d}")
