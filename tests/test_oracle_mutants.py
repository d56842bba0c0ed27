"""CPU: plausible mistakes planted in a copy of the oracle source must each
trip at least one pin.  This shows the pins are strong enough to catch a
dropped term, a wrong sign, index, order or operand in the oracle.

Mistakes are planted in a temporary copy only; the real oracle is untouched.
Each mutant runs in its own process so a bad mutant cannot take pytest down.
"""
import os
import subprocess
import sys

import pytest

import oracle

# (name, original text, planted text): the first occurrence is replaced.
MUTANTS = [
    ("delta_sign", "c = (v[j] - dot(m, 1, k, dk)) * beta;", "c = (dot(m, 1, k, dk) - v[j]) * beta;"),
    ("beta_dropped", "c = (v[j] - dot(m, 1, k, dk)) * beta;", "c = (v[j] - dot(m, 1, k, dk));"),
    ("rank1_update_dropped", "m[i] = m[i] + c * k[i];", "m[i] = m[i] + 0.0f * c * k[i];"),
    ("decay_dropped", "m[i] = m[i] * e;", "m[i] = m[i];"),
    ("decay_squared", "const float e = expf(gate);", "const float e = expf(2.0f * gate);"),
    ("sk_transposed_operand", "c = (v[j] - dot(m, 1, k, dk)) * beta;",
     "c = (v[j] - dot(M + j, (size_t)dk, k, dk)) * beta;"),
    ("sk_before_decay", "for (i = 0; i < dk; ++i)\n            m[i] = m[i] * e;\n        c = (v[j] - dot(m, 1, k, dk)) * beta;",
     "c = (v[j] - dot(m, 1, k, dk)) * beta;\n        for (i = 0; i < dk; ++i)\n            m[i] = m[i] * e;"),
    ("out_uses_k", "out[j] = dot(m, 1, q, dk) / rs;", "out[j] = dot(m, 1, k, dk) / rs;"),
    ("out_unscaled", "out[j] = dot(m, 1, q, dk) / rs;", "out[j] = dot(m, 1, q, dk);"),
    ("out_scale_dv", "const float rs = sqrtf((float)dk);", "const float rs = sqrtf((float)(dk + 1));"),
    ("head_map_interleaved", "static int32_t key_head_of(int32_t h, int32_t Hk) { return h % Hk; }",
     "static int32_t key_head_of(int32_t h, int32_t Hk) { return (h / 2) % Hk; }"),
    ("seq_wrong_token_stride", "q + (bt * Hk + kh) * dk,", "q + ((size_t)b * Hk + kh) * dk,"),
    ("f64_decay_dropped", "m[i] = m[i] * e;\n        c = ((double)v[j]", "m[i] = m[i];\n        c = ((double)v[j]"),
    ("f64_beta_dropped", "c = ((double)v[j] - dot64(m, k, dk)) * (double)beta;",
     "c = ((double)v[j] - dot64(m, k, dk));"),
    ("f64_out_unscaled", "out[j] = dot64(m, q, dk) / rs;", "out[j] = dot64(m, q, dk);"),
    ("seq_f64_token_stride", "v + (bt * Hv + h) * dv,\n                               beta",
     "v + ((size_t)b * Hv + h) * dv,\n                               beta"),
    ("pair_tentative_from_old_state", "if (p == 1)", "if (p == 0)"),
    ("pair_positions_swapped", "const size_t bp = (size_t)b * 2 + p;", "const size_t bp = (size_t)b * 2 + (1 - p);"),
    ("tail_pair_tentative_from_old", "for (p = 0; p < 2; ++p) {\n            const size_t bp = 2 * (size_t)b + p;",
     "for (p = 1; p >= 0; --p) {\n            const size_t bp = 2 * (size_t)b + p;"),
    ("tail_pair_positions_swapped", "const size_t bp = 2 * (size_t)b + p;", "const size_t bp = 2 * (size_t)b + (1 - p);"),
    ("tail_pair_state_not_carried", "memcpy(Mb, M + (size_t)b * st, st * sizeof(float));",
     "memset(Mb, 0, st * sizeof(float));"),
    ("conv_taps_reversed", "acc = acc + conv_w[(size_t)c * K + t] * win[t];",
     "acc = acc + conv_w[(size_t)c * K + (K - 1 - t)] * win[t];"),
    ("conv_cache_not_shifted", "cs[(size_t)t * C + c] = win[t + 1];", "cs[(size_t)t * C + c] = win[t];"),
    ("silu_sign", "return x / (1.0f + expf(-x));", "return x / (1.0f + expf(x));"),
    ("l2_without_sqrt", "nrm = sqrtf(ss);", "nrm = ss;"),
    ("rms_weight_index", "* w[i] *", "* w[0] *"),
    ("rms_eps_outside_sqrt", "rms = sqrtf(ss / (float)group + eps);", "rms = sqrtf(ss / (float)group) + eps;"),
    ("rms_mean_over_wrong_n", "rms = sqrtf(ss / (float)group + eps);", "rms = sqrtf(ss / (float)n + eps);"),
    ("tail_split_q_from_k", "memcpy(q + (size_t)b * nq, act + (size_t)b * C, ",
     "memcpy(q + (size_t)b * nq, act + (size_t)b * C + nq, "),
    ("tail_k_not_normalized", "oracle_l2norm_rows(B * Hk, dk, k);", ";"),
    ("gate_tf_halves_swapped", "const float bl = row[h];", "const float bl = row[Hv + h];"),
    ("gate_tf_sigmoid_sign", "1.0f / (1.0f + expf(-bl));", "1.0f / (1.0f + expf(bl));"),
    ("gate_tf_gate_sign", "= -expf(a_log[h]) *", "= expf(a_log[h]) *"),
    ("gate_tf_dt_bias_dropped", "softplus(al + dt_bias[h])", "softplus(al)"),
    ("gate_tf_a_log_not_exponentiated", "= -expf(a_log[h]) *", "= -a_log[h] *"),
    ("gate_tf_softplus_branch", "x + log1pf(expf(-x))", "log1pf(expf(-x))"),
    ("gate_tf_head_index", "softplus(al + dt_bias[h])", "softplus(al + dt_bias[0])"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, source, name, old, new):
    assert old in source, f"mutation site for {name} not found"
    src = tmp_path / "gdn_oracle.c"
    src.write_text(source.replace(old, new, 1))
    hdr = os.path.join(os.path.dirname(oracle.SOURCE), "gdn_oracle.h")
    (tmp_path / "gdn_oracle.h").write_text(open(hdr).read())
    lib = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", str(src), "-o", lib, "-lm"], check=True)
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, os.path.join(here, "pins.py"), lib],
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": os.pathsep.join(
                           [os.path.dirname(here), here, os.environ.get("PYTHONPATH", "")])})
    assert r.returncode == 1 and "FAIL" in r.stdout, \
        f"planted mistake {name} not caught (rc={r.returncode}):\n{r.stdout}\n{r.stderr}"


def test_unmodified_copy_passes(tmp_path, source):
    """Control: the same harness on an unmodified copy reports no failure."""
    src = tmp_path / "gdn_oracle.c"
    src.write_text(source)
    hdr = os.path.join(os.path.dirname(oracle.SOURCE), "gdn_oracle.h")
    (tmp_path / "gdn_oracle.h").write_text(open(hdr).read())
    lib = str(tmp_path / "liboracle_copy.so")
    subprocess.run(["gcc", *oracle.CFLAGS, str(src), "-o", lib, "-lm"], check=True)
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, os.path.join(here, "pins.py"), lib],
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": os.pathsep.join(
                           [os.path.dirname(here), here, os.environ.get("PYTHONPATH", "")])})
    assert r.returncode == 0, r.stdout + r.stderr
