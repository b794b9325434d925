"""Each plausible mistake planted in a copy of the oracle (dropped term, wrong
sign, wrong index, wrong operand) must make at least one pin fail: forward
mistakes against the forward pins, backward mistakes against the backward
pins.

The mutants are compiled on the CPU from text substitutions of oracle.c into a
temporary directory; the pins run against them in a subprocess through the
SINKATTN_ORACLE_LIB override.  The oracle itself is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "eps_dropped": ("ss / (double)d + eps", "ss / (double)d"),
    "sum_not_mean": ("sqrt(ss / (double)d + eps)", "sqrt(ss + eps)"),
    "norm_weight_dropped": ("y[i] = w[i] * x[i] * inv;", "y[i] = x[i] * inv;"),
    "rope_sign": ("y[i] = a * c - b * s;", "y[i] = a * c + b * s;"),
    "rope_interleaved_halves": ("int half = d / 2;", "int half = d / 4;"),
    "rope_exponent": ("-2.0 * (double)i / (double)d", "-1.0 * (double)i / (double)d"),
    "global_positions": ("pos_of[t] = t - cu[n];", "pos_of[t] = t;"),
    "window_off_by_one": ("dp >= window", "dp > window"),
    "anti_causal": ("if (dp < 0) return 0;", "if (dp > 0) return 0;"),
    "cross_document": ("if (doc_of[u] != doc_of[t]) return 0;", ""),
    "gqa_modulo": ("h / group, d, qh", "h % Hkv, d, qh"),
    "score_scale_dropped": ("scores[u] = scale * dot;", "scores[u] = dot;"),
    "sink_term_dropped": ("double Z = exp(sink - M);", "double Z = 0.0;"),
    "sink_scaled": ("double Z = exp(sink - M);", "double Z = exp(sink * scale - M);"),
    "sink_in_max_dropped": ("double M = sink;", "double M = -INFINITY;"),
    "lse_shift_dropped": ("*lse_out = M + log(Z);", "*lse_out = log(Z);"),
    "value_of_query_token": ("v + ((size_t)u * Hkv + g) * d", "v + ((size_t)t * Hkv + g) * d"),
    "key_head_zero": ("kh + ((size_t)u * Hkv + g) * d", "kh + ((size_t)u * Hkv) * d"),
}


# A mutant is one substitution, or a list of them when the mistake concerns a
# quantity the oracle's two backward passes both form (the softmax gradient's
# D term is used by the row pass for dq and by the key pass for dk).
BWD_MUTANTS = {
    "bwd_D_term_dropped": [("const double dS = P * (dP - D);", "const double dS = P * dP;"),
                           ("const double dS = P * (dP - row_D[r]);",
                            "const double dS = P * dP;")],
    "bwd_sink_sign": ("part -= row_sink[(size_t)t * Hq + h];",
                      "part += row_sink[(size_t)t * Hq + h];"),
    "bwd_sink_not_normalised": ("exp(sinks[h] - lse) * D", "exp(sinks[h]) * D"),
    "bwd_dq_scale_dropped": ("dqrow[i] += scale * dS * ku[i];", "dqrow[i] += dS * ku[i];"),
    "bwd_dk_from_key": ("dku[i] += scale * dS * qrow[i];", "dku[i] += scale * dS * ku[i];"),
    "bwd_dv_weight": ("dvu[i] += P * dorow[i];", "dvu[i] += dS * dorow[i];"),
    "bwd_dP_against_key": ("dP += dorow[i] * vu[i];", "dP += dorow[i] * ku[i];"),
    "bwd_rope_not_transposed": ("y[i] = a * c + b * s;", "y[i] = a * c - b * s;"),
    "bwd_norm_second_term": ("dx[i] = w[i] * dy[i] * r - x[i] * r * r * r * dot / (double)d;",
                             "dx[i] = w[i] * dy[i] * r;"),
    "bwd_norm_weight_grad_unnormalised": ("dw[i] += dy[i] * x[i] * r;", "dw[i] += dy[i] * x[i];"),
}


def _run_mutant(name, subs, pins, tmp_path):
    import oracle.oracle as O
    mutated = open(SRC).read()
    for old, new in (subs if isinstance(subs, list) else [subs]):
        assert mutated.count(old) >= 1, f"mutation site for {name} not found: {old}"
        mutated = mutated.replace(old, new)
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(mutated)
    lib = O.build(force=True, src=str(csrc), out=str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, SINKATTN_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    _run_mutant(name, MUTANTS[name], "test_oracle_pins.py", tmp_path)


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    _run_mutant(name, BWD_MUTANTS[name], "test_oracle_bwd_pins.py", tmp_path)
