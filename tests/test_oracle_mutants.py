"""Planted mistakes in the oracle must fail its pins.

Each mutant is a one-line edit of a copy of ``oracle/linattn_oracle.c``
(a dropped term, a wrong sign, a wrong operand or index, a transposed state),
compiled to a temporary library; ``tests/test_oracle.py`` is then run against it
in a subprocess and must fail.  The real oracle source is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "linattn_oracle.c")

MUTANTS = {
    "phi_drops_plus_one": ("return (x >= 0.0) ? x + 1.0 : exp(x);", "return (x >= 0.0) ? x : exp(x);"),
    "phi_wrong_sign": ("return (x >= 0.0) ? x + 1.0 : exp(x);", "return (x >= 0.0) ? x + 1.0 : exp(-x);"),
    "read_with_key": ("num[j] += fq[i] * s[(int64_t)i * Dv + j];", "num[j] += fk[i] * s[(int64_t)i * Dv + j];"),
    "state_transposed": ("s[(int64_t)i * Dv + j] += fk[i] * vt[j];", "s[(int64_t)j * Dk + i] += fk[i] * vt[j];"),
    "z_not_decayed": ("z[i] *= a;", ";"),
    "z_adds_query": ("z[i] += fk[i];", "z[i] += fq[i];"),
    "den_counts_tokens": ("den += fq[i] * z[i];", "den += z[i];"),
    "eps_dropped": ("ot[j] = num[j] / (den + eps);", "ot[j] = num[j] / den;"),
    "gate_index_shifted": ("double a = alpha[t];", "double a = alpha[t > 0 ? t - 1 : 0];"),
    "value_scaled_by_query": ("s[(int64_t)i * Dv + j] += fk[i] * vt[j];", "s[(int64_t)i * Dv + j] += fq[i] * vt[j];"),
}
# Mistakes in the backward (the adjoint), caught by its own pins.
BACKWARD_MUTANTS = {
    "bwd_dd_sign": ("dd[t] = -go_dot_o / den;", "dd[t] = go_dot_o / den;"),
    "bwd_dphi_is_one": ("return (x >= 0.0) ? 1.0 : exp(x);", "return 1.0;"),
    "bwd_g_not_decayed": ("z[i] = a_next * z[i] + dd[t] * fq[i];", "z[i] = z[i] + dd[t] * fq[i];"),
    "bwd_dv_uses_query": ("acc += s[(int64_t)i * Dv + j] * fk[i];", "acc += s[(int64_t)i * Dv + j] * fq[i];"),
    "bwd_dq_drops_den_term": ("double acc = dd[t] * z[i];", "double acc = 0.0;"),
    "bwd_dk_drops_den_term": ("double acc = z[i];", "double acc = 0.0;"),
    "bwd_init_grad_undecayed": ("ds_init[e] = a_next * s[e];", "ds_init[e] = s[e];"),
}


DELTA_MUTANTS = {
    "delta_key_not_unit": ("kh[i] = nrm > 0.0 ? kh[i] / nrm : 0.0;", "kh[i] = kh[i];"),
    "delta_writes_value": ("b * kh[i] * (vt[j] - u[j]);", "b * kh[i] * vt[j];"),
    "delta_beta_ignored": ("const double b = beta ? beta[t] : 1.0;", "const double b = 1.0;"),
    "delta_gate_ignored": ("s[e] *= alpha[t];", "s[e] *= 1.0;"),
    "delta_read_with_query": ("acc += s[(int64_t)i * Dv + j] * kh[i];", "acc += s[(int64_t)i * Dv + j] * phi(q[t * Dk + i], mode);"),
    # normalize the raw key first, then apply the feature map
    "delta_normalize_then_phi": ("kh[i] = phi(kt[i], mode);\n            nrm += kh[i] * kh[i];\n        }\n        nrm = sqrt(nrm);\n"
                                 "        for (int i = 0; i < Dk; ++i)\n            kh[i] = nrm > 0.0 ? kh[i] / nrm : 0.0;",
                                 "kh[i] = kt[i];\n            nrm += kh[i] * kh[i];\n        }\n        nrm = sqrt(nrm);\n"
                                 "        for (int i = 0; i < Dk; ++i)\n            kh[i] = phi(nrm > 0.0 ? kh[i] / nrm : 0.0, mode);"),
}
LOWP_MUTANTS = {
    "lowp_truncates": ("return nearbyint(x / q) * q;", "return trunc(x / q) * q;"),
    "lowp_fp8_saturates": ("return fabs(r) > 448.0 ? NAN : r;", "return fabs(r) > 448.0 ? copysign(448.0, r) : r;"),
    "lowp_denominator_shifted": ("den += phi(qt[i], mode) * zb[i];", "den += phi(qt[i], mode) * (zb[i] + 0.5);"),
}
PINS = {**{n: "test_oracle.py" for n in MUTANTS}, **{n: "test_oracle_backward.py" for n in BACKWARD_MUTANTS},
        **{n: "test_oracle_delta.py" for n in DELTA_MUTANTS}, **{n: "test_oracle_lowp.py" for n in LOWP_MUTANTS}}


@pytest.mark.parametrize("name", sorted(PINS))
def test_mutant_is_caught(name, tmp_path):
    old, new = {**MUTANTS, **BACKWARD_MUTANTS, **DELTA_MUTANTS, **LOWP_MUTANTS}[name]
    pins = PINS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(csrc), "-lm"], check=True)
    env = dict(os.environ, LINATTN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
