"""The fp64 oracle against its pins, and planted mistakes against the pins.

A planted mistake is a textual change to a copy of the oracle's C source,
compiled on the CPU into a throwaway library; the pin suite must reject every
one of them.  Nothing here needs a GPU.
"""
import os
import subprocess

import pytest

import oracle_pins as P
from oracle import oracle as O

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attn_oracle.c")


@pytest.fixture(scope="module")
def lib():
    return O.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(lib, pin):
    pin(lib)


# (name, original text, planted text): each original occurs exactly once.
MUTANTS = [
    ("window_off_by_one", "a - b > P->window - 1", "a - b > P->window"),
    ("causal_leak", "if (b > a) return 0;", "if (b > a + 1) return 0;"),
    ("agent_rule_inverted", "if (is_agent(P, b) && !is_agent(P, a)) return 0;",
     "if (is_agent(P, a) && !is_agent(P, b)) return 0;"),
    ("no_isolation", "if (is_agent(P, b) && !is_agent(P, a)) return 0;", ""),
    ("gqa_interleaved", "int u = (int)(job / Hq), h = (int)(job % Hq), g = h / G;",
     "int u = (int)(job / Hq), h = (int)(job % Hq), g = h % Hkv;"),
    ("scale_dropped", "z[b] = scale * dot(qa, kbase + (long)b * P->kpos_stride, D);",
     "z[b] = dot(qa, kbase + (long)b * P->kpos_stride, D);"),
    ("lse_without_max", "return m + log(l);", "return log(l);"),
    ("ds_sign", "double ds = p[b] * (dot(da, vbb, D) - delta);",
     "double ds = p[b] * (delta - dot(da, vbb, D));"),
    ("delta_from_q", "double delta = dot(da, oa, D);", "double delta = dot(da, qa, D);"),
    ("dq_reads_v", "dqa[d] += scale * ds * kbb[d];", "dqa[d] += scale * ds * vbb[d];"),
    ("dk_unscaled", "dkb[(long)b * P.kpos_stride + d] += scale * ds * qa[d];",
     "dkb[(long)b * P.kpos_stride + d] += ds * qa[d];"),
    ("dv_uses_ds", "dvb[(long)b * P.kpos_stride + d] += p[b] * da[d];",
     "dvb[(long)b * P.kpos_stride + d] += ds * da[d];"),
    ("time_kv_stride", "P.kpos_stride = (long)N * Hkv * D;", "P.kpos_stride = (long)Hkv * D;"),
    ("space_unit_base", "*kv0 = (long)u * N * Hkv * D;", "*kv0 = (long)(u % 2) * N * Hkv * D;"),
    ("fwd_p_unnormalised", "for (int b = 0; b < P->L; ++b) p[b] /= l;",
     "for (int b = 0; b < P->L; ++b) p[b] /= (l + 1e-3);"),
    ("decode_ring_key", "const long ko = (((long)b * C + f % C) * N + n) * Hkv * D + (long)g * D;",
     "const long ko = (((long)b * C + (f + 1) % C) * N + n) * Hkv * D + (long)g * D;"),
    ("decode_ring_value", "const long vo = (((long)b * C + f % C) * N + n) * Hkv * D + (long)g * D;",
     "const long vo = (((long)b * C + f / C) * N + n) * Hkv * D + (long)g * D;"),
    ("decode_query_frame", "const int a = q_frame0 + t;", "const int a = q_frame0 + t + 1;"),
    ("decode_lse", "lse[(((long)b * Tq + t) * N + n) * Hq + h] = m + log(l);",
     "lse[(((long)b * Tq + t) * N + n) * Hq + h] = log(l);"),
    ("rms_without_mean", "const double r = 1.0 / sqrt(ss / dm + eps);",
     "const double r = 1.0 / sqrt(ss + eps);"),
    ("norm_rounded", "for (int c = 0; c < dm; ++c) y[c] = xm[c] * r * gamma[c];",
     "for (int c = 0; c < dm; ++c) y[c] = (float)(xm[c] * r * gamma[c]);"),
    ("gain_dropped", "for (int c = 0; c < dm; ++c) y[c] = xm[c] * r * gamma[c];",
     "for (int c = 0; c < dm; ++c) y[c] = xm[c] * r;"),
    ("qkv_split", "else if (n < nq + nkv) k[m * nkv + (n - nq)] = acc;",
     "else if (n <= nq + nkv) k[m * nkv + (n - nq) % nkv] = acc;"),
    ("residual_dropped", "y[m * dm + n] = (residual ? residual[m * dm + n] : 0.0) + dot(",
     "y[m * dm + n] = 0.0 + dot("),
    ("out_weight_row", "dot(o + m * din, w + (long)n * din, din);",
     "dot(o + m * din, w + (long)(n % 2) * din, din);"),
]


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(tmp_path, name, orig, planted):
    src = open(ORACLE_SRC).read()
    assert src.count(orig) == 1, "mutation anchor for %s must occur once" % name
    mutated = tmp_path / ("oracle_%s.c" % name)
    mutated.write_text(src.replace(orig, planted))
    so = tmp_path / ("lib_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so),
                    str(mutated), "-lm"], check=True)
    bad = O.load(str(so))
    failures = []
    for pin in P.ALL_PINS:
        try:
            pin(bad)
        except (AssertionError, ValueError) as e:
            failures.append((pin.__name__, str(e)[:80]))
    assert failures, "planted mistake %s passed every pin" % name
