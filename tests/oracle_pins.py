"""Pins for the FP64 oracle: facts fixed by the lecture pages and by mathematics.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
``AssertionError`` when the oracle disagrees with something *other than
itself*: hand-derived golden values, closed forms, invariants, brute force in
50-digit decimal arithmetic, or torch's float64 softmax/logsumexp.  The same
battery is run against deliberately broken builds of the oracle (see
``test_oracle_mutants.py``) to show that plausible mistakes are caught.

Run as ``python -m tests.oracle_pins <liboracle.so>`` to print the names of the
failing pins as JSON (used by the mutant test, one subprocess per build).

Citations name the page and section: [FL] = CS349E Lecture 11 shared module
flash_lab.py (section 2 holds the backward of standard attention); [XS] = xserv design doc
"04-transformer-kernels", test plan.
"""
from __future__ import annotations

import json
import math
import os
import sys
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "hand_derived.json")


# --------------------------------------------------------------------------
# helpers (no attention arithmetic here beyond what each pin states)
# --------------------------------------------------------------------------
def _value(x):
    """Evaluate a golden-file number expression to float."""
    if isinstance(x, (int, float)):
        return float(x)
    if isinstance(x, str):
        if x == "-inf":
            return -math.inf
        return float(Fraction(x))
    if isinstance(x, dict):
        (key, arg), = x.items()
        if key == "log":
            return math.log(_value(arg))
        if key == "sum":
            return sum(_value(a) for a in arg)
        if key == "e_over_1pe":
            return _value(arg) * math.e / (1 + math.e)
        if key == "one_over_1pe":
            return _value(arg) / (1 + math.e)
        if key == "log1pe":
            return _value(arg) * math.log(1 + math.e)
    raise ValueError(f"bad golden value {x!r}")


def _arr(rows):
    return np.array([[_value(x) for x in r] for r in rows], dtype=np.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _visible_count(N, Nk, causal):
    """Number of keys query i sees: all, or those at positions <= Nk-N+i."""
    i = np.arange(N)
    if not causal:
        return np.full(N, Nk)
    return np.clip(Nk - N + i + 1, 0, Nk)


def _brute_decimal(q, k, v, causal, scale, prec=50):
    """Attention by brute force in `prec`-digit decimal: weights exp(score)
    taken directly (no maximum subtracted), normalised by their total."""
    getcontext().prec = prec
    N, d = q.shape
    Nk, dv = v.shape
    sc = Decimal(float(scale))
    o = np.zeros((N, dv))
    lse = np.zeros(N)
    for i in range(N):
        weights = []
        for j in range(Nk):
            if causal and j > Nk - N + i:
                continue
            s = sum(Decimal(float(q[i, c])) * Decimal(float(k[j, c])) for c in range(d)) * sc
            weights.append((j, s.exp()))
        if not weights:
            o[i] = 0.0
            lse[i] = -math.inf
            continue
        z = sum(w for _, w in weights)
        for c in range(dv):
            o[i, c] = float(sum(w * Decimal(float(v[j, c])) for j, w in weights) / z)
        lse[i] = float(z.ln())
    return o, lse


def _torch_attention(q, k, v, causal, scale):
    """torch float64 softmax/logsumexp with an explicit bottom-right boolean mask."""
    import torch
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    s = (qt @ kt.transpose(-1, -2).contiguous()) * scale
    N, Nk = s.shape[-2:]
    if causal:
        allowed = torch.arange(Nk)[None, :] <= (Nk - N + torch.arange(N))[:, None]
        s = s.masked_fill(~allowed, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    o = p @ vt
    return o.numpy(), lse.numpy()


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb), f"{what}: finiteness differs"
    assert np.array_equal(a[~fa], b[~fb]), f"{what}: non-finite values differ"
    err = float(np.max(np.abs(a[fa] - b[fb]))) if fa.any() else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# pins of standard attention (the definition both GPU entry points reach)
# --------------------------------------------------------------------------
def pin_golden_hand_derived(orc):
    """Hand-derived values of [FL] section 2's definition (tests/golden)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = _arr(c["q"]), _arr(c["k"]), _arr(c["v"])
        o, lse = orc.attention(q, k, v, causal=c["causal"], scale=_value(c["scale"]))
        _close(o, _arr(c["o"]), 1e-14, c["name"] + " O")
        _close(lse, np.array([_value(x) for x in c["lse"]]), 1e-14, c["name"] + " LSE")


def pin_single_key(orc):
    """Nk = 1: the only key gets weight 1, so O = v0 and LSE = scale*q.k0.
    Under causal masking with N > 1 only the last query sees it."""
    rng = _rng(11)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 6))
    o, lse = orc.attention(q, k, v, causal=False, scale=0.3)
    _close(o, np.repeat(v, 5, axis=0), 1e-15, "Nk=1 O")
    _close(lse, 0.3 * (q @ k[0]), 1e-14, "Nk=1 LSE")
    o, lse = orc.attention(q, k, v, causal=True, scale=0.3)
    _close(o[:4], np.zeros((4, 6)), 0.0, "Nk=1 causal hidden rows O")
    assert np.all(lse[:4] == -np.inf), "Nk=1 causal hidden rows LSE"
    _close(o[4], v[0], 1e-15, "Nk=1 causal last row O")


def pin_scale_zero(orc):
    """scale = 0: every visible key has weight 1/#visible, so O_i is the mean
    of the visible V rows and LSE_i = ln(#visible)."""
    rng = _rng(12)
    for (N, Nk, causal) in ((6, 6, False), (6, 6, True), (4, 9, True), (9, 4, True)):
        q = rng.standard_normal((N, 5))
        k = rng.standard_normal((Nk, 5))
        v = rng.standard_normal((Nk, 3))
        o, lse = orc.attention(q, k, v, causal=causal, scale=0.0)
        cnt = _visible_count(N, Nk, causal)
        for i in range(N):
            if cnt[i] == 0:
                assert lse[i] == -np.inf and np.all(o[i] == 0.0), f"empty row {i}"
                continue
            _close(o[i], v[:cnt[i]].mean(axis=0), 1e-14, f"scale0 O row {i}")
            _close(lse[i], math.log(cnt[i]), 1e-14, f"scale0 LSE row {i}")


def pin_causal_first_row(orc):
    """Causal with N = Nk: query 0 sees key 0 only, so O_0 = v_0."""
    rng = _rng(13)
    q, k, v = rng.standard_normal((7, 4)), rng.standard_normal((7, 4)), rng.standard_normal((7, 5))
    o, lse = orc.attention(q, k, v, causal=True, scale=0.5)
    _close(o[0], v[0], 1e-15, "causal row 0 O")
    _close(lse[0], 0.5 * float(q[0] @ k[0]), 1e-14, "causal row 0 LSE")


def pin_probabilities(orc):
    """Rows of P are non-negative and sum to 1 ([XS] test plan); P_ij is
    exactly 0 iff key j is hidden from query i (j > Nk-N+i), else positive."""
    rng = _rng(14)
    for (N, Nk, causal) in ((5, 9, True), (9, 9, True), (9, 5, True), (6, 7, False)):
        q, k, v = rng.standard_normal((N, 4)), rng.standard_normal((Nk, 4)), rng.standard_normal((Nk, 3))
        _, _, p = orc.attention(q, k, v, causal=causal, scale=0.7, want_p=True)
        assert np.all(p >= 0.0)
        for i in range(N):
            hidden = np.arange(Nk) > (Nk - N + i) if causal else np.zeros(Nk, bool)
            assert np.all(p[i, hidden] == 0.0), f"hidden keys get weight, row {i}"
            assert np.all(p[i, ~hidden] > 0.0), f"visible keys get no weight, row {i}"
            if (~hidden).any():
                assert abs(p[i].sum() - 1.0) < 1e-14, f"row {i} sums to {p[i].sum()}"


def pin_constant_v(orc):
    """Constant V rows give a constant O (weights sum to one)."""
    rng = _rng(15)
    q, k = rng.standard_normal((8, 6)), rng.standard_normal((11, 6))
    row = rng.standard_normal(4)
    v = np.tile(row, (11, 1))
    for causal in (False, True):
        o, _ = orc.attention(q, k, v, causal=causal)
        _close(o, np.tile(row, (8, 1)), 1e-14, f"constant V (causal={causal})")


def pin_shift_invariance(orc):
    """Adding c to every score of a row (append c/scale to q and 1 to k)
    leaves O unchanged and adds c to LSE."""
    rng = _rng(16)
    N, Nk, d = 6, 10, 5
    q, k, v = rng.standard_normal((N, d)), rng.standard_normal((Nk, d)), rng.standard_normal((Nk, 3))
    scale = 0.4
    c = rng.uniform(-30, 30, size=N)
    q2 = np.concatenate([q, (c / scale)[:, None]], axis=1)
    k2 = np.concatenate([k, np.ones((Nk, 1))], axis=1)
    for causal in (False, True):
        o1, l1 = orc.attention(q, k, v, causal=causal, scale=scale)
        o2, l2 = orc.attention(q2, k2, v, causal=causal, scale=scale)
        _close(o2, o1, 1e-12, "shift O")
        _close(l2, l1 + c, 1e-12, "shift LSE")


def pin_key_permutation(orc):
    """Without a mask, permuting keys jointly in K and V changes nothing."""
    rng = _rng(17)
    q, k, v = rng.standard_normal((5, 6)), rng.standard_normal((13, 6)), rng.standard_normal((13, 4))
    perm = rng.permutation(13)
    o1, l1 = orc.attention(q, k, v)
    o2, l2 = orc.attention(q, k[perm], v[perm])
    _close(o2, o1, 1e-14, "perm O")
    _close(l2, l1, 1e-14, "perm LSE")


def pin_single_query_causal(orc):
    """N = 1: the query sits at the last position, so causal == non-causal."""
    rng = _rng(18)
    q, k, v = rng.standard_normal((1, 8)), rng.standard_normal((20, 8)), rng.standard_normal((20, 8))
    o1, l1 = orc.attention(q, k, v, causal=False)
    o2, l2 = orc.attention(q, k, v, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_large_scores(orc):
    """Scores in the thousands stay finite ([XS] test plan: stable for large
    values); a key ahead by 60 takes all the weight to within e^-60."""
    rng = _rng(19)
    Nk, d = 12, 4
    k = rng.standard_normal((Nk, d))
    v = rng.standard_normal((Nk, 3))
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k[:, 0] = 1000.0 + rng.uniform(0, 1, Nk)
    k[5, 0] = 1061.0
    o, lse = orc.attention(q, k, v, scale=1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    _close(o[0], v[5], 1e-20 + 1e-24 + float(np.abs(v).max()) * 12 * math.exp(-59), "dominant key O")
    _close(lse[0], 1061.0, 12 * math.exp(-59) + 1e-12, "dominant key LSE")


def pin_brute_force_decimal(orc):
    """Tiny shapes against 50-digit decimal brute force (no max subtraction)."""
    rng = _rng(20)
    for (N, Nk, d, dv) in ((3, 3, 2, 2), (2, 5, 3, 1), (5, 2, 2, 3), (4, 6, 4, 2), (1, 6, 3, 3)):
        q, k, v = rng.standard_normal((N, d)), rng.standard_normal((Nk, d)), rng.standard_normal((Nk, dv))
        for causal in (False, True):
            o, lse = orc.attention(q, k, v, causal=causal, scale=0.9)
            ob, lb = _brute_decimal(q, k, v, causal, 0.9)
            _close(o, ob, 2e-15, f"brute O {N,Nk,causal}")
            _close(lse, lb, 2e-15, f"brute LSE {N,Nk,causal}")


def pin_torch_crosscheck(orc):
    """torch float64 softmax/logsumexp with an explicit bottom-right mask,
    on the single-head and ragged shapes of the fp32 workloads."""
    rng = _rng(21)
    for (N, Nk, d) in ((256, 256, 64), (300, 300, 64), (77, 513, 32), (1, 1000, 64), (40, 17, 16)):
        q, k, v = rng.standard_normal((N, d)), rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d))
        for causal in (False, True):
            o, lse = orc.attention(q, k, v, causal=causal, scale=1 / math.sqrt(d))
            ot, lt = _torch_attention(q, k, v, causal, 1 / math.sqrt(d))
            hidden = ~np.isfinite(lt)
            ot[hidden] = 0.0                       # torch gives NaN for empty rows
            _close(o, ot, 1e-12, f"torch O {N,Nk,causal}")
            _close(lse, lt, 1e-12, f"torch LSE {N,Nk,causal}")


def pin_lse_reconstructs_p(orc):
    """exp(S_ij - LSE_i) recovers P_ij ([FL] section 3 backward recomputes P
    from L this way), with S = scale*Q K^T taken from numpy."""
    rng = _rng(22)
    q, k, v = rng.standard_normal((7, 5)), rng.standard_normal((9, 5)), rng.standard_normal((9, 2))
    _, lse, p = orc.attention(q, k, v, causal=True, scale=0.6, want_p=True)
    s = (q @ k.T) * 0.6
    mask = np.arange(9)[None, :] <= (9 - 7 + np.arange(7))[:, None]
    rec = np.where(mask, np.exp(np.where(mask, s, 0.0) - lse[:, None]), 0.0)
    _close(rec, p, 1e-14, "exp(S - LSE)")


# --------------------------------------------------------------------------
# pins of the online-softmax and merge machinery ([FL] section 1, section 4)
# --------------------------------------------------------------------------
def pin_softmax_online_equals_3pass(orc):
    """[FL] self-test: x = 4*N(0,1) of shape (5, 300), block 37, |diff| < 1e-15;
    also other blocks (1, 300, 1000) and torch's softmax."""
    import torch
    x = _rng(0).standard_normal((5, 300)) * 4
    y3 = orc.softmax_3pass(x)
    for b in (37, 1, 300, 1000):
        yo = orc.softmax_online(x, block=b)
        assert np.abs(y3 - yo).max() < 1e-15, f"online vs 3-pass, block {b}"
    yt = torch.softmax(torch.from_numpy(x), dim=-1).numpy()
    assert np.abs(y3 - yt).max() < 1e-15, "3-pass vs torch.softmax"


def pin_merge_halves(orc):
    """[FL] self-test: merging the states of x[:, :100] and x[:, 100:] gives
    the state of the whole row (rtol 1e-14), here with values too."""
    rng = _rng(23)
    x = rng.standard_normal((5, 300)) * 4
    v = rng.standard_normal((300, 3))
    a = orc.partial_state(x[:, :100], v[:100])
    b = orc.partial_state(x[:, 100:], v[100:])
    m, l, o = orc.merge_states(a, b)
    mf, lf, of = orc.partial_state(x, v)
    assert np.array_equal(m, mf)
    assert np.allclose(l, lf, rtol=1e-14, atol=0)
    assert np.allclose(o, of, rtol=1e-13, atol=1e-13)


def _identity(rows, dv):
    return np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, dv))


def pin_merge_identity_and_masked(orc):
    """The state of an empty or fully masked segment is (m=-inf, l=0, o=0)
    and merging it changes nothing, bitwise ([FL] section 1 boundary rule)."""
    rng = _rng(24)
    x = rng.standard_normal((4, 20))
    v = rng.standard_normal((20, 3))
    a = orc.partial_state(x, v)
    masked = orc.partial_state(np.full((4, 7), -np.inf), v[:7])
    assert np.all(masked[0] == -np.inf) and np.all(masked[1] == 0) and np.all(masked[2] == 0)
    empty = orc.partial_state(np.zeros((4, 0)), np.zeros((0, 3)))
    assert np.all(empty[0] == -np.inf) and np.all(empty[1] == 0) and np.all(empty[2] == 0)
    for e in (masked, empty, _identity(4, 3)):
        for r in (orc.merge_states(a, e), orc.merge_states(e, a)):
            assert np.array_equal(r[0], a[0]) and np.array_equal(r[1], a[1]) and np.array_equal(r[2], a[2])
    r = orc.merge_states(_identity(4, 3), _identity(4, 3))
    assert np.all(r[0] == -np.inf) and np.all(r[1] == 0) and np.all(r[2] == 0), "identity+identity"


def pin_merge_assoc_comm(orc):
    """merge_states is commutative (bitwise) and associative: any split of a
    row (empty segments included) merged in any order or tree gives the state
    of the whole row ([FL] section 1)."""
    rng = _rng(25)
    n = 64
    x = rng.standard_normal((3, n)) * 3
    v = rng.standard_normal((n, 4))
    whole = orc.partial_state(x, v)
    for trial in range(20):
        cuts = np.sort(rng.integers(0, n + 1, size=rng.integers(1, 8)))
        bounds = [0, *cuts.tolist(), n]
        parts = [orc.partial_state(x[:, a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        for a, b in zip(parts[:-1], parts[1:]):
            ab, ba = orc.merge_states(a, b), orc.merge_states(b, a)
            assert all(np.array_equal(s, t) for s, t in zip(ab, ba)), "not commutative"
        orders = [list(range(len(parts))), list(range(len(parts)))[::-1],
                  rng.permutation(len(parts)).tolist()]
        for order in orders:
            acc = parts[order[0]]
            for idx in order[1:]:
                acc = orc.merge_states(acc, parts[idx])
            # and a balanced tree over the same order
            level = [parts[i] for i in order]
            while len(level) > 1:
                level = [orc.merge_states(level[i], level[i + 1]) if i + 1 < len(level) else level[i]
                         for i in range(0, len(level), 2)]
            for got in (acc, level[0]):
                assert np.array_equal(got[0], whole[0])
                assert np.allclose(got[1], whole[1], rtol=1e-13, atol=0)
                assert np.allclose(got[2], whole[2], rtol=1e-12, atol=1e-12)


def pin_split_kv_decode(orc):
    """[FL] self-test: split-KV decode of q [4,32] against K, V [1000,32]
    equals standard attention within 1e-13 for n_splits 1, 3, 16, 999; here
    also for n_splits > S (empty segments), checked against torch; and the
    grid of rounded bounds leaves min(n_splits, S) non-empty segments."""
    rng = _rng(0)
    q = rng.standard_normal((4, 32))
    K, V = rng.standard_normal((1000, 32)), rng.standard_normal((1000, 32))
    ot, lt = _torch_attention(q, K, V, False, 1 / math.sqrt(32))
    for ns in (1, 3, 16, 64, 999, 1000, 1001, 2000):
        o, lse, used = orc.split_kv_decode(q, K, V, ns)
        assert used == min(ns, 1000), (ns, used)
        assert np.abs(o - ot).max() < 1e-13, f"split {ns} O"
        assert np.abs(lse - lt).max() < 1e-13, f"split {ns} LSE"


# --------------------------------------------------------------------------
# pins of the backward ([FL] section 2, standard_attention_bwd)
# --------------------------------------------------------------------------
def _loss(orc, q, k, v, dout, causal, scale):
    """sum(dout * O): the scalar whose gradient the backward returns."""
    o, _ = orc.attention(q, k, v, causal=causal, scale=scale)
    return float(np.sum(dout * o))


def pin_bwd_finite_differences(orc):
    """Every entry of dq, dk, dv against a central difference of
    sum(dout * O) through the (separately pinned) forward, as the pages'
    self-test does for one entry (step 1e-6, agreement to 1e-7)."""
    rng = _rng(41)
    eps = 1e-6
    for (N, Nk, d, dv, causal) in ((5, 7, 3, 2, False), (4, 4, 3, 3, True), (6, 4, 2, 3, True)):
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((Nk, d))
        v = rng.standard_normal((Nk, dv))
        dout = rng.standard_normal((N, dv))
        grads = orc.attention_bwd(q, k, v, dout, causal=causal, scale=0.7)
        for which, x in enumerate((q, k, v)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                args = [q, k, v]
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args[which] = xp
                fp = _loss(orc, *args, dout, causal, 0.7)
                args[which] = xm
                fm = _loss(orc, *args, dout, causal, 0.7)
                num[idx] = (fp - fm) / (2 * eps)
            _close(grads[which], num, 1e-7, f"finite differences d{'qkv'[which]} {N}x{Nk} causal={causal}")


def pin_bwd_single_key(orc):
    """Nk = 1: O_i = v0 whatever q and k are, so dq = dk = 0 and
    dv0 = sum_i dout_i."""
    rng = _rng(42)
    q = rng.standard_normal((5, 4))
    k = rng.standard_normal((1, 4))
    v = rng.standard_normal((1, 3))
    dout = rng.standard_normal((5, 3))
    dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal=False, scale=0.5)
    _close(dq, np.zeros_like(q), 1e-15, "Nk=1 dq")
    _close(dk, np.zeros_like(k), 1e-15, "Nk=1 dk")
    _close(dv, dout.sum(axis=0, keepdims=True), 1e-14, "Nk=1 dv")


def pin_bwd_scale_zero(orc):
    """scale = 0: the weights are 1/#visible whatever q and k are, so
    dq = dk = 0 and dv_j = sum over the rows i that see key j of
    dout_i / #visible_i."""
    rng = _rng(43)
    for (N, Nk, causal) in ((5, 5, False), (5, 5, True), (3, 6, True), (6, 3, True)):
        q = rng.standard_normal((N, 4))
        k = rng.standard_normal((Nk, 4))
        v = rng.standard_normal((Nk, 2))
        dout = rng.standard_normal((N, 2))
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal=causal, scale=0.0)
        _close(dq, np.zeros_like(q), 0.0, "scale=0 dq")
        _close(dk, np.zeros_like(k), 0.0, "scale=0 dk")
        cnt = _visible_count(N, Nk, causal)
        want = np.zeros((Nk, 2))
        for i in range(N):
            for j in range(Nk):
                if (not causal or j <= Nk - N + i) and cnt[i] > 0:
                    want[j] += dout[i] / cnt[i]
        _close(dv, want, 1e-14, f"scale=0 dv {N}x{Nk} causal={causal}")


def pin_bwd_invariants(orc):
    """Facts of the gradient that hold at any size:
    * each row of dS sums to 0 (softmax is invariant to a shift of a row's
      scores), so sum_j dk_j = 0;
    * each row of P sums to 1 (0 for a row that sees no key), so
      sum_j dv_j = sum of dout over the rows that see some key;
    * scaling q by t scales the scores like scaling k by t, so
      sum(q * dq) = sum(k * dk)."""
    rng = _rng(44)
    for (N, Nk, causal) in ((9, 13, False), (9, 13, True), (12, 7, True)):
        q = rng.standard_normal((N, 6))
        k = rng.standard_normal((Nk, 6))
        v = rng.standard_normal((Nk, 5))
        dout = rng.standard_normal((N, 5))
        dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal=causal, scale=0.4)
        _close(dk.sum(axis=0), np.zeros(6), 1e-13, "sum of dk")
        seen = _visible_count(N, Nk, causal) > 0
        _close(dv.sum(axis=0), dout[seen].sum(axis=0), 1e-13, "sum of dv")
        _close(np.sum(q * dq), np.sum(k * dk), 1e-12, "q.dq = k.dk")


def pin_bwd_torch_autograd(orc):
    """torch float64 autograd through softmax with an explicit bottom-right
    mask (a different code base), on shapes where every row sees a key."""
    import torch
    rng = _rng(45)
    for (N, Nk, d, dv, causal) in ((17, 23, 8, 5, False), (17, 23, 8, 5, True), (16, 16, 4, 4, True)):
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((Nk, d))
        v = rng.standard_normal((Nk, dv))
        dout = rng.standard_normal((N, dv))
        qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        s = (qt @ kt.transpose(0, 1)) * 0.35
        if causal:
            allowed = torch.arange(Nk)[None, :] <= (Nk - N + torch.arange(N))[:, None]
            s = s.masked_fill(~allowed, float("-inf"))
        o = torch.softmax(s, dim=-1) @ vt
        o.backward(torch.from_numpy(dout))
        dq, dk, dvv = orc.attention_bwd(q, k, v, dout, causal=causal, scale=0.35)
        _close(dq, qt.grad.numpy(), 1e-12, "autograd dq")
        _close(dk, kt.grad.numpy(), 1e-12, "autograd dk")
        _close(dvv, vt.grad.numpy(), 1e-12, "autograd dv")


def pin_bwd_heads_independent(orc):
    """Batched heads give the per-head results (the head strides are right)."""
    rng = _rng(46)
    q = rng.standard_normal((2, 3, 5, 4))
    k = rng.standard_normal((2, 3, 6, 4))
    v = rng.standard_normal((2, 3, 6, 3))
    dout = rng.standard_normal((2, 3, 5, 3))
    dq, dk, dv = orc.attention_bwd(q, k, v, dout, causal=True, scale=0.5)
    for b in range(2):
        for h in range(3):
            g = orc.attention_bwd(q[b, h], k[b, h], v[b, h], dout[b, h], causal=True, scale=0.5)
            _close(dq[b, h], g[0], 0.0, "head dq")
            _close(dk[b, h], g[1], 0.0, "head dk")
            _close(dv[b, h], g[2], 0.0, "head dv")


PINS = [v for k, v in list(globals().items()) if k.startswith("pin_") and callable(v)]


def run_battery(orc):
    """Names of the pins that fail (any exception counts as a failure)."""
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(orc)
            except Exception:  # noqa: BLE001 -- every failure mode counts
                failed.append(pin.__name__)
    return failed


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    import oracle as _oracle

    print(json.dumps(run_battery(_oracle.Oracle(sys.argv[1]))))
