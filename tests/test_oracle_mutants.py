"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pin battery catches every one of them.

Each mutant is a single textual edit of ``oracle/oracle.c`` -- a dropped term,
a wrong sign, index or stride, a transposed operand, a mask off by one -- built
with gcc into a temporary library and run through ``tests/oracle_pins.py`` in
a subprocess.  A mutant passes this test when at least one pin fails on it.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "scale_dropped": ("srow[j] = scale * acc;", "srow[j] = acc;"),
    "mask_top_left": ("last = Nk - N + i;", "last = i;"),
    "mask_off_by_one": ("if (j > last) {", "if (j >= last) {"),
    "mask_always_on": ("        if (causal)\n            last", "        if (1)\n            last"),
    "masked_score_zero": ("srow[j] = -INFINITY;\n                continue;",
                          "srow[j] = 0.0;\n                continue;"),
    "lse_without_max": ("lse[i] = m + log(l);", "lse[i] = log(l);"),
    "lse_log2": ("lse[i] = m + log(l);", "lse[i] = m + log2(l);"),
    "no_normalisation": ("double pij = srow[j] / l;", "double pij = srow[j];"),
    "exp_sign": ("srow[j] = exp(srow[j] - m);", "srow[j] = exp(m - srow[j]);"),
    "k_transposed": ("acc += qi[c] * kj[c];", "acc += qi[c] * k[c * Nk + j];"),
    "v_wrong_stride": ("const double *vj = v + j * dv;\n            for (long c = 0; c < dv; ++c)\n                oi[c]",
                       "const double *vj = v + j;\n            for (long c = 0; c < dv; ++c)\n                oi[c]"),
    "empty_row_nan": ("if (m == -INFINITY) {                    /* R1",
                      "if (0) {                    /* R1"),
    "online_no_carry": ("l = l * carry + add;", "l = l + add;"),
    "online_stale_max": ("double m_new = m > mb ? m : mb;", "double m_new = mb;"),
    "merge_factor_sign": ("double fa = (a == -INFINITY) ? 0.0 : exp(a - mm);",
                          "double fa = (a == -INFINITY) ? 0.0 : exp(mm - a);"),
    "merge_identity_unguarded": ("double fb = (b == -INFINITY) ? 0.0 : exp(b - mm);",
                                 "double fb = exp(b - mm);"),
    "merge_l_dropped_term": ("double lr = la[r] * fa + lb[r] * fb;", "double lr = la[r] * fa + lb[r];"),
    "partial_unnormalised_max": ("double e = exp(xr[j] - mr);", "double e = exp(xr[j]);"),
    "split_weights_about_max": ("acc += exp(seg_lse[u * R + r] - lse[r])",
                                "acc += exp(seg_lse[u * R + r] - big)"),
    "split_segment_unnormalised": ("os[c] /= lr;", "os[c] /= 1.0;"),
    "split_last_bound": ("long b = (sp + 1 == n_splits) ? S :", "long b = (sp + 1 == n_splits) ? S - 1 :"),
    "bwd_D_dropped": ("double dsij = pij * (dpij - Di);", "double dsij = pij * dpij;"),
    "bwd_dS_sign": ("double dsij = pij * (dpij - Di);", "double dsij = pij * (Di - dpij);"),
    "bwd_D_from_v": ("Di += doi[c] * oi[c];", "Di += doi[c] * v[c];"),
    "bwd_dP_from_o": ("dpij += doi[c] * vj[c];", "dpij += doi[c] * oi[c];"),
    "bwd_dq_unscaled": ("dqi[c] += scale * dsij * kj[c];", "dqi[c] += dsij * kj[c];"),
    "bwd_dk_from_k": ("dkj[c] += scale * dsij * qi[c];", "dkj[c] += scale * dsij * kj[c];"),
    "bwd_dv_row_index": ("double *dvj = dvv + j * dv;", "double *dvj = dvv + (i % Nk) * dv;"),
    "bwd_dv_from_v": ("dvj[c] += pij * doi[c];", "dvj[c] += pij * vj[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / "liboracle_mutant.so"))
    proc = subprocess.run([sys.executable, "-m", "tests.oracle_pins", lib], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)
    if proc.returncode != 0:
        return  # the broken build crashed the battery: caught
    failed = json.loads(proc.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_source_passes_battery(tmp_path):
    lib = oracle.build(oracle.SOURCE, str(tmp_path / "liboracle_copy.so"))
    proc = subprocess.run([sys.executable, "-m", "tests.oracle_pins", lib], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stderr
    assert json.loads(proc.stdout.strip().splitlines()[-1]) == []
