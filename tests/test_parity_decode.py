"""fa_decode_splitkv (through the C ABI) against the FP64 oracle on the GPU."""
import math

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


def test_decode_b8_h32_nk32768_d128_all_heads():
    """The long-context decode at full size with 64 splits, launched as the
    bench launches it; every head against the oracle, one batch at a time,
    into NaN-prefilled outputs."""
    w = si.WORKLOADS["decode_b8_h32_nk32768_d128"]
    s = w.shapes[0]
    log(f"fa_decode_splitkv full-size {w.name}")
    q, k, v = si.device_qkv(s, w.seed, w.dtype, "cuda", w.std)
    o = torch.full((s.B, s.H, s.N, s.dv), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((s.B, s.H, s.N), float("nan"), dtype=torch.float32, device="cuda")
    fa.decode_splitkv(q, k, v, num_splits=w.num_splits, out=o, lse=lse)
    torch.cuda.synchronize()
    for b in range(s.B):
        o_ref, l_ref = oracle_on(q[b:b + 1], k[b:b + 1], v[b:b + 1], False, default_scale(s.d))
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, w.dtype, f"{w.name} batch {b}")
    log(f"  {w.name}: {s.B * s.H}/{s.B * s.H} heads compared element by element")


# ---- grouped-query decode (fa_decode_splitkv_gqa) ---------------------------
# The definition: query head h attends with key/value head h // G, i.e.
# standard attention on K and V with each key/value head repeated G times.

def _run_gqa(B, Hkv, G, N, Nk, d, dtype, causal, num_splits, seed=0, std=1.0, dv=None):
    """`std` scales Q and K; V keeps unit scale (dividing by a power of two is
    exact), so the tolerance on O keeps its meaning."""
    Hq = Hkv * G
    dv = d if dv is None else dv
    q, _, _ = make_inputs(B, Hq, N, 1, d, dv, dtype, seed, std)
    _, k, v = make_inputs(B, Hkv, 1, Nk, d, dv, dtype, seed + 1000, std)
    if std != 1.0:
        assert std == 2.0 ** round(math.log2(std))
        v = v / std
    scale = default_scale(d)
    log(f"fa_decode_splitkv_gqa dtype={dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} Nk={Nk} d={d} "
        f"causal={causal} splits={num_splits} seed={seed}")
    o, lse = fa.decode_splitkv_gqa(q, k, v, causal=causal, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    k_rep = k.repeat_interleave(G, dim=1).contiguous()
    v_rep = v.repeat_interleave(G, dim=1).contiguous()
    o_ref, l_ref = oracle_on(q, k_rep, v_rep, causal, scale)
    compare(o, lse, o_ref, l_ref, dtype,
            f"gqa {dtype} {B}x{Hq}/{Hkv}x{N}x{Nk}x{d}/{dv} S={num_splits}")
    return q, k, v, o, lse


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G", [2, 3, 4, 8])
@pytest.mark.parametrize("N", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa(dtype, G, N, causal):
    _run_gqa(2, 2, G, N, 700, 128 if dtype == "bf16" else 64, dtype, causal, 8, seed=G * 10 + N)


@pytest.mark.parametrize("d", [32, 64])
def test_gqa_many_rows_per_group(d):
    # 16 query heads per key/value head and 5 rows each: 80 rows, 10 row groups of 8
    _run_gqa(1, 2, 16, 5, 333, d, "bf16", True, 3, seed=d)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("G,N,Nk,splits,causal", [
    (4, 1, 1000, 16, False),    # one 16-row tile, 4 rows used
    (16, 1, 95, 7, True),       # a full tile; ragged last block of 32 keys
    (2, 8, 70, 40, True),       # most segments empty
    (5, 4, 3, 2, True),         # N > Nk: row 0 of every head sees no key
    (6, 3, 515, 5, False),      # 18 rows: two tiles, the second nearly empty
])
def test_gqa_matrix_core_shapes(dtype, d, G, N, Nk, splits, causal):
    _run_gqa(1, 2, G, N, Nk, d, dtype, causal, splits, seed=G + N + d)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d,dv", [(32, 64), (32, 128), (64, 32), (64, 128), (128, 32), (128, 64)])
@pytest.mark.parametrize("G,N,Nk,splits,causal", [
    (16, 1, 95, 7, True),       # a full tile; ragged last block of 32 keys
    (5, 4, 3, 2, True),         # N > Nk: row 0 of every head sees no key
    (6, 3, 515, 5, False),      # 18 rows: two tiles, the second nearly empty
])
def test_gqa_matrix_core_unequal_dims(dtype, d, dv, G, N, Nk, splits, causal):
    # K rows of d and V rows of dv elements on the matrix-core segment kernel
    _run_gqa(1, 2, G, N, Nk, d, dtype, causal, splits, seed=G + N + d + dv, dv=dv)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("splits", [64, 0])
def test_gqa_d256_several_units_per_workgroup(dtype, splits):
    # d = dv = 256 with 64 splits: 2048 (segment, head, tile) units for at
    # most 256 resident workgroups, so each walks several units in a row
    _run_gqa(4, 8, 4, 1, 6000, 256, dtype, True, splits, seed=31)


def test_gqa_large_scores():
    # scores with standard deviation ~16: the running maximum moves often
    _run_gqa(2, 2, 4, 1, 2000, 128, "bf16", False, 8, seed=5, std=4.0)


def test_gqa_with_one_group_is_plain_decode():
    q, k, v = make_inputs(2, 4, 1, 3000, 128, 128, "bf16", 23)
    o1, l1 = fa.decode_splitkv(q, k, v, num_splits=16)
    o2, l2 = fa.decode_splitkv_gqa(q, k, v, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_b8_hq32_hkv8_nk32768_d128_all_heads():
    """Grouped-query decode at the long-context size (4 query heads per
    key/value head, 64 splits); every query head against the oracle, one
    batch at a time, into NaN-prefilled outputs."""
    B, Hq, Hkv, Nk, d = 8, 32, 8, 32768, 128
    G = Hq // Hkv
    log(f"fa_decode_splitkv_gqa full-size B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} d={d}")
    q, _, _ = si.device_qkv(si.Shape(B, Hq, 1, 1, d, d), 31, "bf16", "cuda", 1.0)
    _, k, v = si.device_qkv(si.Shape(B, Hkv, 1, Nk, d, d), 32, "bf16", "cuda", 1.0)
    o = torch.full((B, Hq, 1, d), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, Hq, 1), float("nan"), dtype=torch.float32, device="cuda")
    fa.decode_splitkv_gqa(q, k, v, num_splits=64, out=o, lse=lse)
    torch.cuda.synchronize()
    for b in range(B):
        k_rep = k[b:b + 1].repeat_interleave(G, dim=1)
        v_rep = v[b:b + 1].repeat_interleave(G, dim=1)
        o_ref, l_ref = oracle_on(q[b:b + 1], k_rep, v_rep, False, default_scale(d))
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, "bf16", f"gqa full-size batch {b}")
    log(f"  gqa full-size: {B * Hq}/{B * Hq} query heads compared element by element")


# ---- automatic split count (num_splits = 0) ---------------------------------

@pytest.mark.parametrize("B,Hkv,G,N,Nk,d,dtype,causal", [
    (2, 8, 1, 1, 5000, 128, "bf16", False),
    (2, 4, 4, 1, 3000, 64, "f16", True),
    (1, 4, 1, 2, 2000, 64, "f32", True),
    (1, 2, 3, 3, 700, 32, "bf16", False),
])
def test_auto_splits_equals_explicit_count(B, Hkv, G, N, Nk, d, dtype, causal):
    """num_splits = 0 runs exactly the split count the rule reports, and the
    result is the oracle's."""
    q, k, v, o, lse = _run_gqa(B, Hkv, G, N, Nk, d, dtype, causal, 0, seed=B + G + N)
    S = fa.decode_splitkv_auto_splits(B, Hkv * G, Hkv, N, Nk, d, d, q.dtype)
    assert S >= 1
    o2, l2 = fa.decode_splitkv_gqa(q, k, v, causal=causal, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_auto_splits_plain_entry_point():
    q, k, v = make_inputs(2, 4, 1, 6000, 128, 128, "bf16", 9)
    o1, l1 = fa.decode_splitkv(q, k, v, num_splits=0)
    S = fa.decode_splitkv_auto_splits(2, 4, 4, 1, 6000, 128, 128, q.dtype)
    o2, l2 = fa.decode_splitkv(q, k, v, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = oracle_on(q, k, v, False, default_scale(128))
    compare(o1, l1, o_ref, l_ref, "bf16", "decode auto splits")
