"""Helpers of the GPU parity tests: run the oracle on the same (dtype-rounded)
inputs the GPU saw and compare element by element.

Tolerances (max absolute error against the FP64 oracle):
  fp32 inputs:       O <= 2e-5, LSE <= 2e-5
  bf16/fp16 inputs:  O <= 2e-2, LSE <= 1e-2
LSE = -inf (a row that sees no key) must match exactly, with O = 0 there.

Gradients (dq, dk, dv of the backward) use the same per-dtype bars on O,
relative to the gradient's own scale: max|g - g_ref| <= tol * max(1,
max|g_ref|).  O is a convex combination of V rows (unit scale); a gradient
is a sum over up to N rows or Nk keys and grows with them, and its bf16
rounding error (and that of the rounded P and dS the matrix cores use)
grows in proportion.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth_inputs as si

TOL = {"f32": (2e-5, 2e-5), "bf16": (2e-2, 1e-2), "f16": (2e-2, 1e-2)}
DTYPE_NAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def make_inputs(B, H, N, Nk, d, dv, dtype="bf16", seed=0, std=1.0, device="cuda"):
    """Seeded host draw (numpy), rounded to dtype, placed on the GPU."""
    q, k, v = si.host_qkv(si.Shape(B, H, N, Nk, d, dv), seed, std)
    return tuple(si.to_storage(x, dtype, device) for x in (q, k, v))


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what: str, tol=None):
    """Assert the GPU result matches the oracle; returns (err_o, err_lse).
    ``tol`` = (tol_o, tol_lse) overrides the per-dtype bar."""
    tol_o, tol_l = TOL[dtype] if tol is None else tol
    o = si.as_f64(o_gpu)
    l = si.as_f64(lse_gpu)
    assert o.shape == o_ref.shape, (what, o.shape, o_ref.shape)
    assert l.shape == lse_ref.shape, (what, l.shape, lse_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    ref_empty = np.isneginf(lse_ref)
    got_empty = np.isneginf(l)
    assert np.array_equal(ref_empty, got_empty), f"{what}: -inf LSE pattern differs"
    assert np.all(np.isfinite(l[~got_empty])), f"{what}: non-finite LSE"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(l[~got_empty] - lse_ref[~ref_empty]))) if (~got_empty).any() else 0.0
    log(f"  {what}: max|dO|={err_o:.3e} (tol {tol_o:.0e})  max|dLSE|={err_l:.3e} (tol {tol_l:.0e})")
    assert err_o <= tol_o, f"{what}: O error {err_o:.3e} > {tol_o:.0e}"
    assert err_l <= tol_l, f"{what}: LSE error {err_l:.3e} > {tol_l:.0e}"
    return err_o, err_l


GRAD_TOL = {"f32": 2e-5, "bf16": 2e-2, "f16": 2e-2}


def compare_grads(got, ref, dtype: str, what: str):
    """Assert (dq, dk, dv) match the oracle's within GRAD_TOL (relative to
    max(1, max|ref|) per tensor); returns the three errors."""
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = si.as_f64(g)
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        err = float(np.max(np.abs(g - r))) if g.size else 0.0
        bound = GRAD_TOL[dtype] * max(1.0, float(np.max(np.abs(r))) if r.size else 0.0)
        log(f"  {what}: max|d{name}|={err:.3e} (bar {bound:.2e})")
        assert err <= bound, f"{what}: {name} error {err:.3e} > {bound:.2e}"
        errs.append(err)
    return errs


def oracle_bwd_on(q, k, v, dout, causal, scale, heads=None):
    """Oracle gradients on the GPU tensors' values; ``heads`` = list of (b, h)."""
    f = lambda t: si.as_f64(t)
    if heads is None:
        return oracle.attention_bwd(f(q), f(k), f(v), f(dout), causal=causal, scale=scale)
    parts = [oracle.attention_bwd(f(q[b, h]), f(k[b, h]), f(v[b, h]), f(dout[b, h]),
                                  causal=causal, scale=scale) for (b, h) in heads]
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))


def oracle_on(q, k, v, causal, scale, heads=None):
    """Oracle result on the GPU tensors' values; ``heads`` = list of (b, h)."""
    if heads is None:
        return oracle.attention(si.as_f64(q), si.as_f64(k), si.as_f64(v), causal=causal, scale=scale)
    os_, ls_ = [], []
    for (b, h) in heads:
        o, l = oracle.attention(si.as_f64(q[b, h]), si.as_f64(k[b, h]), si.as_f64(v[b, h]),
                                causal=causal, scale=scale)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def default_scale(d):
    return 1.0 / math.sqrt(d)


def score_scaled_tolerance(q, k, v, scale, dtype: str, causal: bool):
    """Tolerance for inputs whose scores are far larger than the workloads'.

    First-order perturbation bound.  If every score s_ij carries an error
    e_ij, the softmax weights move to p_ij (1 + e_ij - sum_k p_ik e_ik), so
        |dO_ic|  <= sum_j p_ij |e_ij| |v_jc - O_ic|,
        |dLSE_i| <= sum_j p_ij |e_ij|.
    A float32 score is a length-d inner product; its rounding error is
    bounded, in the probabilistic sense of Higham and Mary's analysis, by
    sqrt(d) * 2^-24 * |scale| * sum_c |q_ic k_jc|.  The bar is the dtype's
    bar plus that bound, evaluated with the oracle's P on these inputs: weights
    of keys that hardly count, and keys whose value rows equal the output,
    add nothing, unlike the worst case over all keys."""
    qf, kf, vf = si.as_f64(q), si.as_f64(k), si.as_f64(v)
    d = qf.shape[-1]
    o_ref, _, p = oracle.attention(qf, kf, vf, causal=causal, scale=scale, want_p=True)
    eps = math.sqrt(d) * 2.0 ** -24 * abs(scale) * (np.abs(qf) @ np.swapaxes(np.abs(kf), -1, -2))
    w = p * eps                                              # [..., N, Nk]
    dev = np.abs(vf[..., None, :, :] - o_ref[..., :, None, :])   # [..., N, Nk, dv]
    bound_o = float(np.max(np.einsum("...ij,...ijc->...ic", w, dev)))
    bound_l = float(np.max(w.sum(-1)))
    base_o, base_l = TOL[dtype]
    return base_o + bound_o, base_l + bound_l
