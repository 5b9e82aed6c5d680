"""Race checks of the LDS staging of the wide matrix-core forward and of the
32-key dK/dV backward kernel (GPU).

``libfa_serial.so`` is the same library with those two kernels built with
FA_SERIAL_COPIES=1: every K/V tile and Q block (backward: every Q/dO step
and its (LSE, D) strip) is copied between two barriers and waited for
before it is read, so no copy is ever in flight while LDS is read and no
stage is refilled early.  The arithmetic and
its order are the same, so both builds must give bit-identical O and LSE;
a copy that landed late, or a stage overwritten while still being read, in
the pipelined build (three stages, copies two tiles ahead and across items)
would show up as a difference.  Shapes cover the three head-dimension pairs
the kernel serves, one and many items per workgroup, items of 0, 1, 2 and
more tiles, ragged ends, N > Nk causal rows, and both dtypes.
"""
import ctypes
import os

import pytest
import torch

import exact_tiled_attention_flashattention_amd as fa
from tests.parity import log, make_inputs

pytestmark = pytest.mark.gpu

SERIAL = os.path.join(os.path.dirname(fa.LIBRARY_PATH), "libfa_serial.so")


def _serial_lib():
    if not os.path.exists(SERIAL):
        raise FileNotFoundError(f"{SERIAL} is not built")
    lib = ctypes.CDLL(SERIAL)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, c_int,
                           ctypes.c_float, c_int, vp]
    lib.fa_fwd.restype = c_int
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, c_int,
                           ctypes.c_float, c_int, vp, ctypes.c_size_t, vp]
    lib.fa_bwd.restype = c_int
    return lib


CASES = [
    (64, 16, 1024, 1024, 64, 64, True),     # the GPT-2-medium-shaped prefill
    (2, 3, 1, 1, 64, 64, True),
    (2, 3, 64, 64, 64, 64, False),
    (1, 4, 300, 300, 64, 64, True),
    (3, 5, 77, 513, 64, 64, True),
    (3, 5, 513, 77, 64, 64, True),          # causal rows that see no key
    (2, 8, 1000, 3000, 64, 64, False),
    (4, 16, 2048, 2048, 64, 64, True),
    (2, 32, 4096, 4096, 128, 128, True),    # a long causal prefill at d = 128
    (2, 5, 700, 1300, 128, 128, False),
    (3, 4, 1100, 1100, 64, 128, True),
    (2, 3, 130, 70, 64, 128, False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,N,Nk,d,dv,causal", CASES)
def test_pipelined_equals_serial_bitwise(dtype, B, H, N, Nk, d, dv, causal):
    lib = _serial_lib()
    q, k, v = make_inputs(B, H, N, Nk, d, dv, dtype, seed=B * 7 + N + Nk + d)
    scale = d ** -0.5
    log(f"race check dtype={dtype} B={B} H={H} N={N} Nk={Nk} d={d} dv={dv} causal={causal}")
    o1, l1 = fa.fwd(q, k, v, causal=causal, scale=scale)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                    B, H, N, Nk, d, dv, int(causal), scale, 2 if dtype == "bf16" else 1,
                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), f"O differs: max {(o1.float() - o2.float()).abs().max().item()}"
    assert torch.equal(l1, l2) or torch.equal(torch.nan_to_num(l1), torch.nan_to_num(l2))


BWD_CASES = [
    (2, 3, 1000, 1000, False),      # d = 64 without the mask: several 256-key blocks, ragged
    (1, 2, 2048, 2048, True),       # causal, 64-row steps across the diagonal
    (1, 2, 2300, 2100, True),       # causal N > Nk: rows that see no key
    (2, 2, 130, 700, False),        # one 64-row step, ragged keys
    # causal with more 256-key blocks than resident workgroups: each
    # workgroup walks pairs of blocks and copies the next block's first steps
    # during the last steps of the one before
    (8, 16, 2048, 2048, True),      # two pairs per workgroup
    (5, 7, 1800, 1900, True),       # head count not a multiple of 8, ragged
    (8, 16, 2100, 1900, True),      # N > Nk: rows that see no key, several row blocks each
    (8, 16, 1024, 1024, False),     # unmasked: 512 blocks, one per workgroup
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,N,Nk,causal,d,dv", [c + (64, 64) for c in BWD_CASES] + [
    # the 32x32 dQ kernel at d = 128 (one 32-key sub-block per step) and at
    # d = 64 with dv = 128
    (8, 16, 1100, 1200, True, 128, 128),
    (8, 16, 1100, 1200, True, 64, 128),
])
def test_backward_pipelined_equals_serial_bitwise(dtype, B, H, N, Nk, causal, d, dv):
    lib = _serial_lib()
    q, k, v = make_inputs(B, H, N, Nk, d, dv, dtype, seed=B + N + Nk)
    dout, _, _ = make_inputs(B, H, N, 1, dv, dv, dtype, seed=N + 7)
    scale = 0.125
    log(f"bwd race check dtype={dtype} B={B} H={H} N={N} Nk={Nk} d={d} dv={dv} causal={causal}")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    g1 = fa.bwd(q, k, v, o, lse, dout, causal=causal, scale=scale)
    g2 = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    ws = torch.empty(fa.bwd_workspace_size(B, H, N), dtype=torch.uint8, device=q.device)
    st = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), g2[0].data_ptr(), g2[1].data_ptr(), g2[2].data_ptr(),
                    B, H, N, Nk, d, dv, int(causal), scale, 2 if dtype == "bf16" else 1,
                    ws.data_ptr(), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert torch.equal(a, b), f"{name} differs: max {(a.float() - b.float()).abs().max().item()}"
