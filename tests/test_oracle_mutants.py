"""The oracle's pins must reject plausible mistakes.

Each case plants one mistake in a copy of ``oracle/engram_oracle.c`` (on the
CPU, in a temporary directory), builds it, and runs the pin suite against
that build in a subprocess: the suite must fail.  This shows that a dropped
term, a wrong sign, a transposed operand or a misplaced index anywhere in the
oracle is caught by something other than the oracle itself.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "engram_oracle.c")

MUTANTS = [
    ("dx drops the dot term", "dxs[j] = Gs[j] + tx1 - tx2;", "dxs[j] = Gs[j] + tx1;"),
    ("dk wrong sign", "dks[j] = tk1 - tk2;", "dks[j] = tk1 + tk2;"),
    ("dk transposed operand", "tk1 = delta * rk * ws[j] * xh", "tk1 = delta * rk * ws[j] * kh"),
    ("dx missing 1/d", "tx2 = delta * rx * dot * xh / (double)d", "tx2 = delta * rx * dot * xh"),
    ("dw uses x^ twice", "dws[j] += delta * xh * kh;", "dws[j] += delta * xh * xh;"),
    ("dz drops (1 - gate)", "dg * gate * (1.0 - gate)", "dg * gate"),
    ("clamp derivative not blocked", "(fabs(dot) >= c) ? dz / (2.0 * sqrt(fabs(dot))) : 0.0",
     "dz / (2.0 * sqrt(fabs(dot) > c ? fabs(dot) : c))"),
    ("eps outside the sqrt", "1.0 / sqrt(sxx / (double)d + eps)", "1.0 / (sqrt(sxx / (double)d) + eps)"),
    ("rstd without the mean", "1.0 / sqrt(sxx / (double)d + eps)", "1.0 / sqrt(sxx + eps)"),
    ("sgn(0) taken as +1", "  return 0.0;\n}\n\nstatic double sigmoid", "  return sqrt(c);\n}\n\nstatic double sigmoid"),
    ("saved rstd fields swapped", "sv[4 * s + 2] = rx;\n    sv[4 * s + 3] = rk;",
     "sv[4 * s + 2] = rk;\n    sv[4 * s + 3] = rx;"),
    ("masked token saves the raw gate", "sv[4 * s + 0] = m ? g : 0.0;", "sv[4 * s + 0] = g;"),
    ("mask ignored in the output", "os[j] = m ? xs[j] + g * v[j] : xs[j];", "os[j] = xs[j] + g * v[j];"),
    ("value gradient reads stream 0 only", "dv[j] += gate * Gs[j];", "dv[j] += gate * G[j];"),
    ("value taken from the last key block", "fwd_token(d, x, kv, kv + NS * d, w, m, out, sv, aux);",
     "fwd_token(d, x, kv, kv + 3 * d, w, m, out, sv, aux);"),
    ("bf16 rounding half-up instead of ties-to-even", "u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    ("dot over raw (unnormalised) key", "(xs[j] * rx) * ws[j] * (ks[j] * rk)", "(xs[j] * rx) * ws[j] * ks[j]"),
    ("product rule uses the wrong factor", "grad_wh[q] = dw[q] * bf16_bits_to_double(we[q]);",
     "grad_wh[q] = dw[q] * bf16_bits_to_double(wh[q]);"),
    ("fused weight drops a factor", "weight[q] = (float)(bf16_bits_to_double(wh[q]) * bf16_bits_to_double(we[q]));",
     "weight[q] = (float)(bf16_bits_to_double(wh[q]));"),
    # GateConv
    ("gateconv taps reversed", "c += cw[(int64_t)i * d + j] * u_scr[tau * d + j];",
     "c += cw[(int64_t)(GC_TAPS - 1 - i) * d + j] * u_scr[tau * d + j];"),
    ("gateconv gate without 1/sqrt(d)", "s /= sd; /* G2 */", "/* G2 */"),
    ("gateconv key normalised with w_v", "const double term = (Ht[j] * rh * wh[j]) * (kt[j] * rk * wh[j]);",
     "const double term = (Ht[j] * rh * wh[j]) * (kt[j] * rk * wv[j]);"),
    ("gateconv SiLU derivative wrong", "return s * (1.0 + c * (1.0 - s));", "return s;"),
    ("gateconv residual dropped", "Y[t * d + j] = silu(c) + vhat[t * d + j]; /* G6 */", "Y[t * d + j] = silu(c); /* G6 */"),
    ("gateconv backward conv runs causally", "const int64_t tau = t + (GC_TAPS - 1) - i;",
     "const int64_t tau = t - (GC_TAPS - 1) + i;"),
    ("gateconv rms_v backward sign", "- vh[j] * rv * rv * s1 / (double)d);", "+ vh[j] * rv * rv * s1 / (double)d);"),
    ("gateconv dv misses alpha", "      dv[t * d + j] *= a;\n", "\n"),
    ("gateconv dwh drops the key path", "dwh[j] += dhh * Ht[j] * rh + dkh * kt[j] * rk;", "dwh[j] += dhh * Ht[j] * rh;"),
    ("gateconv dcw pairs the wrong token", "dcw[(int64_t)i * d + j] += dc[t * d + j] * u[tau * d + j];",
     "dcw[(int64_t)i * d + j] += dc[t * d + j] * u[t * d + j];"),
    # tolerance scales (the magnitudes that set the parity bars)
    ("dot conditioning x1000", "absdot += fabs(term);", "absdot += 1000.0 * fabs(term);"),
    ("mag_dx x1000", "mdx[(int64_t)s * d + j] = fabs(Gs[j]) + dmag",
     "mdx[(int64_t)s * d + j] = 1000.0 * fabs(Gs[j]) + 1000.0 * dmag"),
    ("mag_dw x1000", "mdw[(int64_t)s * d + j] += dmag * fabs(xh * kh);",
     "mdw[(int64_t)s * d + j] += 1000.0 * dmag * fabs(xh * kh);"),
    ("mag_dx drops |G|", "mdx[(int64_t)s * d + j] = fabs(Gs[j]) + dmag", "mdx[(int64_t)s * d + j] = dmag"),
    ("mag_dx drops the dot term", "(fabs(ws[j] * kh) + fabs(dot * xh) / (double)d)", "fabs(ws[j] * kh)"),
    ("mag_dk drops the dot term", "dmag * rk * (fabs(ws[j] * xh) + fabs(dot * kh) / (double)d)",
     "dmag * rk * fabs(ws[j] * xh)"),
    ("mag_dv drops the gate", "if (mdv) mdv[j] += fabs(gate * Gs[j]);", "if (mdv) mdv[j] += fabs(Gs[j]);"),
    ("delta magnitude from |dg| instead of sum |G v|", "dgabs * gate * (1.0 - gate) / (2.0 * sqrt(fabs(dot)))",
     "fabs(dg) * gate * (1.0 - gate) / (2.0 * sqrt(fabs(dot)))"),
    ("gate slope drops the 2", "if (fabs(dot) >= c) return g * (1.0 - g) / (2.0 * sqrt(fabs(dot)));",
     "if (fabs(dot) >= c) return g * (1.0 - g) / sqrt(fabs(dot));"),
    ("gate slope kept for masked tokens", "aux[2 * s + 1] = m ? gate_slope(dot, g) : 0.0;",
     "aux[2 * s + 1] = gate_slope(dot, g);"),
    ("gateconv magY drops the residual", "fabs(silu_grad(c)) * cm + fabs(vhat[t * d + j]) +",
     "fabs(silu_grad(c)) * cm +"),
    ("gateconv m(u) ignores alpha", "um_scr[t * d + j] = fabs(u_scr[t * d + j]) * (1.0 + (a > 0.0 ? 2.0 * da_scr[t] / a : 0.0));",
     "um_scr[t * d + j] = fabs(u_scr[t * d + j]);"),
    ("gateconv m(alpha) drops the logit magnitude", "da_scr[t] = a * (1.0 - a) * smag;", "da_scr[t] = a * (1.0 - a);"),
    ("gateconv m(dc) drops the SiLU'' term", "dcm[t * d + j] = fabs(dY[t * d + j]) * (fabs(g) + 0.5 * cm);",
     "dcm[t * d + j] = fabs(dY[t * d + j]) * fabs(g);"),
    ("gateconv magH x1000", "if (magH) magH[t * d + j] = rh * (", "if (magH) magH[t * d + j] = 1000.0 * rh * ("),
    ("gateconv mag_dconv_w x1000", "if (mdcw) mdcw[(int64_t)i * d + j] += dcm[t * d + j] * fabs(u[tau * d + j]);",
     "if (mdcw) mdcw[(int64_t)i * d + j] += 1000.0 * dcm[t * d + j] * fabs(u[tau * d + j]);"),
    ("gateconv mag_drms_w_v drops rrms_v", "if (mdwv) mdwv[j] += dum * fabs(vh[j] * rv);",
     "if (mdwv) mdwv[j] += dum * fabs(vh[j]);"),
    ("gateconv magv misses alpha", "if (magv) magv[t * d + j] *= a;", "if (magv) magv[t * d + j] *= 1.0;"),
    ("gateconv mag_drms_w_h drops the key path",
     "if (mdwh) mdwh[j] += dsm * (fabs(kh * Ht[j] * rh) + fabs(hh * kt[j] * rk)) / sd;",
     "if (mdwh) mdwh[j] += dsm * fabs(kh * Ht[j] * rh) / sd;"),
    ("gateconv row-sum magnitudes swapped", "const double s2m = dsm / sd * rk * pm, s3m = dsm / sd * rh * pm;",
     "const double s2m = dsm / sd * rh * pm, s3m = dsm / sd * rk * pm;"),
]


PIN_FILES = ("test_oracle_pins.py", "test_oracle_gateconv_pins.py", "test_oracle_tolerance_scales.py")
WORKERS = max(1, min(8, os.cpu_count() or 1))


def _missed(descs, files_for, tmp_path):
    """Build each named mutant of the oracle and run `files_for(desc)` against
    it in a child pytest (isolated: a mutant may read out of bounds); up to
    WORKERS children at a time.  Returns the mutants whose pins all passed."""
    src = open(SRC).read()
    table = {m[0]: m for m in MUTANTS}

    def one(i, desc):
        _, old, new = table[desc]
        assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
        mutant, lib = tmp_path / f"mutant{i}.c", tmp_path / f"libmutant{i}.so"
        mutant.write_text(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-o",
                               str(lib), str(mutant), "-lm", "-lpthread"])
        env = dict(os.environ, ENGRAM_ORACLE_LIB=str(lib), PYTEST_DISABLE_PLUGIN_AUTOLOAD="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            *[os.path.join(ROOT, "tests", f) for f in files_for(desc)]],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        return desc if r.returncode == 0 else None

    with ThreadPoolExecutor(max_workers=WORKERS) as pool:
        return [d for d in pool.map(one, range(len(descs)), descs) if d is not None]


def test_pins_reject_every_mutant(tmp_path):
    missed = _missed([m[0] for m in MUTANTS], lambda desc: PIN_FILES, tmp_path)
    assert not missed, f"the pins did not catch: {missed}"


# The mistakes in the method's own arithmetic (forward and backward of the gate
# and of GateConv), each of which the autograd pins must catch on their own
# (they run the fp64 entry points; mistakes only in the storage-type path are
# left to the other pins).
AUTOGRAD_CAUGHT = [
    "dx drops the dot term", "dk wrong sign", "dk transposed operand", "dx missing 1/d", "dw uses x^ twice",
    "dz drops (1 - gate)", "clamp derivative not blocked", "eps outside the sqrt", "rstd without the mean",
    "sgn(0) taken as +1", "saved rstd fields swapped", "masked token saves the raw gate",
    "mask ignored in the output", "value gradient reads stream 0 only", "dot over raw (unnormalised) key", "gateconv taps reversed", "gateconv gate without 1/sqrt(d)",
    "gateconv key normalised with w_v", "gateconv SiLU derivative wrong", "gateconv residual dropped",
    "gateconv backward conv runs causally", "gateconv rms_v backward sign", "gateconv dv misses alpha",
    "gateconv dwh drops the key path", "gateconv dcw pairs the wrong token",
]


def test_autograd_pins_alone_reject_mutants(tmp_path):
    missed = _missed(AUTOGRAD_CAUGHT, lambda desc: ("test_oracle_autograd_pins.py",), tmp_path)
    assert not missed, f"the autograd pins alone did not catch: {missed}"


# The mistakes that the invariance properties catch on their own, with no
# expected value at all: for the gate, masking, power-of-two scales, key
# negation, stream order and Euler's orthogonality (the special cases -- the
# clamp, sgn(0), eps --, the rounding mode and the weight's product rule are
# left to the fixed pins); for GateConv, row scales of H, k and v, the H-k
# exchange, the sign of rms_w_h, the rms_w_v-conv_w trade and Euler's
# relations (the conv's tap order, the 1/sqrt(d) scale, the SiLU derivative
# and the two identical halves of drms_w_h are left to the fixed pins).
PROPERTY_CAUGHT = [
    "dx drops the dot term", "dk wrong sign", "dk transposed operand", "dx missing 1/d", "dw uses x^ twice",
    "dz drops (1 - gate)", "rstd without the mean", "saved rstd fields swapped", "masked token saves the raw gate",
    "mask ignored in the output", "value gradient reads stream 0 only", "value taken from the last key block",
    "dot over raw (unnormalised) key",
    "gateconv key normalised with w_v", "gateconv residual dropped", "gateconv backward conv runs causally",
    "gateconv rms_v backward sign", "gateconv dv misses alpha", "gateconv dcw pairs the wrong token",
]


def test_property_pins_alone_reject_mutants(tmp_path):
    pytest.importorskip("hypothesis")
    missed = _missed(PROPERTY_CAUGHT, lambda desc: ("test_oracle_gateconv_property_cpu.py" if desc.startswith("gateconv")
                                                    else "test_oracle_property_cpu.py",), tmp_path)
    assert not missed, f"the property pins alone did not catch: {missed}"
