"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/sfa_oracle.c (a dropped or
misplaced term, a wrong sign, an off-by-one index, a swapped weight, a wrong
order of operations), builds that copy with gcc in a temporary directory, and
runs tests/test_oracle_pins.py against it.  The pin suite must fail for every
mutant and pass for the unmodified source.  Everything here runs on the CPU.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sfa_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

DECODE_EVICT_THEN_WRITE = """                    } else if (p >= W) {
                        for (int e = 0; e < d; ++e) S[e] = g * S[e] + (1.0 - g) * rk[(size_t)s * d + e];
                    }
                }
"""
DECODE_WRITE_THEN_EVICT = """                    } else if (p >= W) {
                        for (int e = 0; e < d; ++e) {
                            rk[(size_t)s * d + e] = kn[e];
                            rv[(size_t)s * d + e] = vn[e];
                        }
                        for (int e = 0; e < d; ++e) S[e] = g * S[e] + (1.0 - g) * rk[(size_t)s * d + e];
                    }
                }
"""

MUTANTS = {
    "per_query_gamma_of_kv_head": ("const double g = gamma[hs];", "const double g = gamma[G];"),
    "per_query_state_of_first_head_only": ("if (s_per_query || h % group == 0)", "if (h % group == 0)"),
    "per_query_decode_one_gamma": ("gamma[(size_t)l * Hq + (size_t)G * group + i]",
                                   "gamma[(size_t)l * Hq + (size_t)G * group]"),
    "running_mean_count_off_by_one": ("const double m = (double)(p - W + 1); /* keys left so far */",
                                      "const double m = (double)(p - W + 2); /* keys left so far */"),
    "running_mean_ignored_in_s": ("S[e] = g * S[e] + (1.0 - g) * (C[e] / m);",
                                  "S[e] = g * S[e] + (1.0 - g) * ke[e];"),
    "running_mean_decode_count": ("const double m = (double)(p - W + 1); /* keys left, this one included */",
                                  "const double m = (double)(p - W + 2); /* keys left, this one included */"),
    "running_mean_continuation_count": ("const int m_in = (p0 - W > 0) ? p0 - W : 0;",
                                        "const int m_in = (p0 - W + 1 > 0) ? p0 - W + 1 : 0;"),
    "decode_negative_position_processed": ("if (p < 0) continue;", "if (p < -1000000) continue;"),
    "window_one_too_wide": ("const int lo = (p - W + 1 > 0) ? p - W + 1 : 0;",
                            "const int lo = (p - W > 0) ? p - W : 0;"),
    "evicts_wrong_key": ("kv_row(k, ring_k, b, G, p - W, p0", "kv_row(k, ring_k, b, G, p - W + 1, p0"),
    "eviction_starts_late": ("if (p >= W) {\n                    const double *ke",
                             "if (p > W) {\n                    const double *ke"),
    "ewma_weights_swapped": ("S[e] = g * S[e] + (1.0 - g) * ke[e];",
                             "S[e] = (1.0 - g) * S[e] + g * ke[e];"),
    "fusion_sign": ("dst[e] = o[e] + alpha[h] * S[e];", "dst[e] = o[e] - alpha[h] * S[e];"),
    "fusion_dropped": ("dst[e] = o[e] + alpha[h] * S[e];", "dst[e] = o[e];"),
    "gqa_interleaved": ("const int G = h / group;", "const int G = h % Hkv;"),
    "scale_one_over_d": ("if (scale <= 0.0) scale = 1.0 / sqrt((double)d);",
                         "if (scale <= 0.0) scale = 1.0 / (double)d;"),
    "prefill_ring_slot": ("double *rk = ring_k + IDX4(b, G, p % W",
                          "double *rk = ring_k + IDX4(b, G, (p + 1) % W"),
    "continuation_ring_slot": ("return ring + IDX4(b, G, qpos % W", "return ring + IDX4(b, G, (qpos + 1) % W"),
    "decode_partial_ring_ignored": ("(p >= W - 1) ? W : p + 1", "(p >= W - 1) ? W : W"),
    "decode_wrong_slot": ("const int s = p % W;", "const int s = (p + 1) % W;"),
    "decode_write_before_evict": (DECODE_EVICT_THEN_WRITE, DECODE_WRITE_THEN_EVICT),
    "decode_alpha_index": ("const double a = alpha[(size_t)l * Hq + h];",
                           "const double a = alpha[(size_t)l * Hq + hh];"),
    "ring_mean_partial_divisor": ("const double rm = rs / ring_size;",
                                  "const double rm = rs / ((t + 1 < ring_size) ? t + 1 : ring_size);"),
    "ring_slot_ignores_t0": ("(((long)t0 + t) % ring_size)", "(((long)t) % ring_size)"),
    "field_weights_swapped": ("F[x] = ema_gamma * F[x] + (1.0 - ema_gamma) * a[x];",
                              "F[x] = (1.0 - ema_gamma) * F[x] + ema_gamma * a[x];"),
    "temperature_multiplies": ("c[i] = dot / (na * pn[i]) / temperature;",
                               "c[i] = dot / (na * pn[i]) * temperature;"),
    "cosine_without_query_norm": ("c[i] = dot / (na * pn[i]) / temperature;",
                                  "c[i] = dot / pn[i] / temperature;"),
    "semantic_weight_one": ("double e = rm + 0.5 * F[x] + 0.5 * sem;",
                            "double e = rm + 0.5 * F[x] + sem;"),
    "scale_then_clip": ("if (e > clip) e = clip;\n                if (e < -clip) e = -clip;\n"
                        "                const double enh = al * e;",
                        "e = al * e;\n                if (e > clip) e = clip;\n"
                        "                if (e < -clip) e = -clip;\n                const double enh = e;"),
    "layer_ratio_over_L": ("(double)layer / (double)(n_layers - 1)", "(double)layer / (double)n_layers"),
    "decay_exponent_shifted": ("pow(cross_decay, (double)layer)", "pow(cross_decay, (double)(layer + 1))"),
    "prefill_softmax_unnormalized": ("const double pj = sc[j - lo] / den;", "const double pj = sc[j - lo];"),
    "prefill_pv_reads_keys": ("const double *vr = kv_row(v, ring_v, b, G, j, p0, n, Hkv, d, W, tv);",
                              "const double *vr = kv_row(k, ring_k, b, G, j, p0, n, Hkv, d, W, tv);"),
    "decode_softmax_unnormalized": ("o += (sc[j] / den) * rv[(size_t)j * d + e];",
                                    "o += sc[j] * rv[(size_t)j * d + e];"),
    "decode_pv_reads_keys": ("o += (sc[j] / den) * rv[(size_t)j * d + e];",
                             "o += (sc[j] / den) * rk[(size_t)j * d + e];"),
    "decode_query_of_group_head": ("const float *qr = q + (((size_t)l * B + b) * Hq + h) * d;",
                                   "const float *qr = q + (((size_t)l * B + b) * Hq + G * group) * d;"),
    "ring_never_written": ("for (int x = 0; x < H; ++x) R[(size_t)slot * H + x] = a[x];", "(void)slot;"),
    "field_read_before_update": ("double e = rm + 0.5 * F[x] + 0.5 * sem;",
                                 "double e = rm + 0.5 * (F[x] - (1.0 - ema_gamma) * a[x]) / ema_gamma + 0.5 * sem;"),
    "semantic_unit_slots": ("sem += (c[i] / den) * (double)P[(size_t)i * H + x];",
                            "sem += (c[i] / den) * (double)P[(size_t)i * H + x] / pn[i];"),
    "cosine_without_slot_norm": ("c[i] = dot / (na * pn[i]) / temperature;", "c[i] = dot / na / temperature;"),
    "slot_softmax_unnormalized": ("sem += (c[i] / den) * (double)P[(size_t)i * H + x];",
                                  "sem += c[i] * (double)P[(size_t)i * H + x];"),
    "enhancement_subtracted": ("out[((size_t)l * T + t) * H + x] = a[x] + enh;",
                               "out[((size_t)l * T + t) * H + x] = a[x] - enh;"),
    "clip_upper_only": ("                if (e < -clip) e = -clip;\n", ""),
}


def _run_pins(src_text, tmpdir, name):
    c_path = os.path.join(tmpdir, f"{name}.c")
    so_path = os.path.join(tmpdir, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", c_path, "-o",
                    so_path, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, SFA_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def test_pins_catch_every_planted_mistake():
    base = open(SRC).read()
    jobs = {"unmodified": base}
    for name, (old, new) in MUTANTS.items():
        assert base.count(old) >= 1, f"mutation site for {name} not found"
        jobs[name] = base.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 2)) as ex:
            futs = {name: ex.submit(_run_pins, text, tmp, name) for name, text in jobs.items()}
            results = {name: f.result() for name, f in futs.items()}
    rc, log = results.pop("unmodified")
    assert rc == 0, f"pins fail on the unmodified oracle:\n{log}"
    survivors = [name for name, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"planted mistakes the pins did not catch: {survivors}"
