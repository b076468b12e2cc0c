"""Plant plausible mistakes in copies of the oracle (on the CPU) and check a pin catches each.

Every mutant is an edit of the oracle's C source: a dropped term, a flipped sign, a wrong or
transposed index, a wrong padding rule, a missing validity check, a wrong rounding rule. For
each, at least one of the pins in oracle_pins.py must fail.
"""

import os
import subprocess
import sys
from pathlib import Path

import pytest

import oracle

# (name, old text, new text): the first occurrence of `old` is replaced.
MUTANTS = [
    ("tap_order_reversed", "xval(x, h0, T, D, W, b, t - (W - 1) + j, d);\n    return z;", "xval(x, h0, T, D, W, b, t - j, d);\n    return z;"),
    ("bias_dropped", "real z = bias ? (real)bias[d] : (real)0;\n    for (int j = 0; j < W; ++j)", "real z = 0;\n    for (int j = 0; j < W; ++j)"),
    ("sigmoid_sign", "r_exp(-z)", "r_exp(z)"),
    ("dsilu_sign", "s * ((real)1 + z * ((real)1 - s))", "s * ((real)1 - z * ((real)1 - s))"),
    ("dsilu_dy_dropped", "return (real)dy[(b * T + t) * D + d] * s *", "return s *"),
    ("dx_index", "g_at(x, h0, dy, T, D, w, W, bias, b, u + (W - 1) - j, d,", "g_at(x, h0, dy, T, D, w, W, bias, b, u + j, d,"),
    ("dx_tap_transposed", "acc = acc + (real)w[d * W + j] * g_at", "acc = acc + (real)w[d * W + (W - 1 - j)] * g_at"),
    ("dw_index", "* xval(x, h0, T, D, W, b, t - (W - 1) + j, d);\n    return acc;", "* xval(x, h0, T, D, W, b, t - j, d);\n    return acc;"),
    ("dbias_skips_head", "for (int64_t t = 0; t < T; ++t) acc = acc + g_at", "for (int64_t t = W - 1; t < T; ++t) acc = acc + g_at"),
    ("replicate_left_pad", "    return 0;\n}\n\n/* z[b, t, d]", "    return (real)x[(b * T + 0) * D + d];\n}\n\n/* z[b, t, d]"),
    ("g_not_zero_past_T", "if (t < 0 || t >= T) return 0;\n    real z", "if (t < 0) return 0;\n    if (t >= T) t = T - 1;\n    real z"),
    ("decode_taps_reversed", "(real)w[d * W + j] * (real)st[j]", "(real)w[d * W + (L - 1 - j)] * (real)st[j]"),
    ("decode_new_token_tap", "(real)w[d * W + (W - 1)] * (real)x[n * D + d]", "(real)w[d * W + 0] * (real)x[n * D + d]"),
    ("decode_shift_direction", "for (int64_t j = 0; j + 1 < L; ++j) st[j] = st[j + 1];\n            if (L > 0) st[L - 1] = x[n * D + d];", "for (int64_t j = L - 1; j > 0; --j) st[j] = st[j - 1];\n            if (L > 0) st[0] = x[n * D + d];"),
    ("slot_no_duplicate_check", "if (idx[n] >= 0 && idx[n] == idx[m]) return 0;", "(void)m;"),
    ("slot_range_off_by_one", "idx[n] >= S) return 0;", "idx[n] > S) return 0;"),
    ("pool_ignores_has_init", "if (idx[b] >= 0 && has_init && has_init[b])", "if (idx[b] >= 0)"),
    ("pool_final_state_dropped", "if (idx[b] >= 0) memcpy(state + (int64_t)idx[b] * D * L", "if (0) memcpy(state + (int64_t)idx[b] * D * L"),
    ("pool_slot_by_batch_row", "memcpy(state + (int64_t)idx[b] * D * L, hT", "memcpy(state + b * D * L, hT"),
    ("decode_padding_output", "y_out[n * D + d] = 0;", "y_out[n * D + d] = (real)x[n * D + d];"),
    ("history_reversed", "h0[(b * D + d) * (W - 1) + (t + W - 1)]", "h0[(b * D + d) * (W - 1) + (-1 - t)]"),
    ("history_ignored", "if (h0 && t >= -(int64_t)(W - 1))", "if (0)"),
    ("final_state_off_by_one", "xval(x, h0, T, D, W, b, T - (W - 1) + j, d)", "xval(x, h0, T, D, W, b, T - W + j, d)"),
    ("history_grad_shifted", "b, -(int64_t)(W - 1) + j, d, 1)", "b, -(int64_t)(W - 1) + j + 1, d, 1)"),
    ("varlen_end_unchecked", "if (cu[0] != 0 || (int64_t)cu[n] != total) return 0;", "if (cu[0] != 0) return 0;"),
    ("varlen_history_of_next", "oracle_fwd_state(x + a * D, h0 ? h0 + i * D * L : NULL", "oracle_fwd_state(x + a * D, h0 ? h0 + ((i + 1) % n) * D * L : NULL"),
    ("varlen_rows_shifted", "oracle_fwd_state(x + a * D,", "oracle_fwd_state(x + (a > 0 ? a - 1 : 0) * D,"),
    ("varlen_dw_last_only", "dw_out[e] = dw_out[e] + dwi[e];", "dw_out[e] = dwi[e];"),
    ("ring_write_off_by_one", "st[c % L] = x[n * D + d];", "st[(c + 1) % L] = x[n * D + d];"),
    ("ring_read_reversed", "((c - k) % L + L) % L", "((c + k) % L + L) % L"),
    ("ex_shift_reads_oldest", "cache_seqlens ? ((c - k) % L + L) % L : L - k;", "cache_seqlens ? ((c - k) % L + L) % L : (L - k) % (W - 1);"),
    ("ex_negative_seqlen_accepted", "if (cache_seqlens[n] < 0) return 1;", "(void)n;"),
    ("linear_keeps_silu", "real y = act ? z * sigmoid(z) : z;", "real y = z * sigmoid(z);"),
    ("linear_grad_dsilu", "if (!act) return (real)dy[(b * T + t) * D + d];", "(void)act;"),
    ("residual_before_activation", "real y = act ? z * sigmoid(z) : z;\n            if (r) y = y + (real)r[q * D + d];", "if (r) z = z + (real)r[q * D + d];\n            real y = act ? z * sigmoid(z) : z;"),
    ("round_half_away", "nearbyint(a / q)", "floor(a / q + 0.5)"),
    ("round_truncate", "nearbyint(a / q)", "trunc(a / q)"),
]


_CHILD = r"""
import sys
from pathlib import Path
import oracle
from oracle_pins import ALL_CHECKS
name, workdir = sys.argv[1], Path(sys.argv[2])
src = Path(workdir / "mutant.c").read_text()
mutant = oracle.build_variant(src, workdir)
for check in ALL_CHECKS:
    try:
        check(mutant)
    except AssertionError as e:
        print("CAUGHT", check.__name__, str(e)[:120], flush=True)
        sys.exit(0)
print("MISSED", name, flush=True)
sys.exit(1)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    """Each mutant runs in a child process: a planted indexing mistake may write out of bounds
    and must not take the test process down with it."""
    src = oracle.source_text()
    assert old in src, f"mutant {name}: pattern not found in the oracle source"
    (tmp_path / "mutant.c").write_text(src.replace(old, new, 1))
    here = Path(__file__).resolve().parent
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(here.parent), str(here)]), OMP_NUM_THREADS="2")
    r = subprocess.run(
        [sys.executable, "-c", _CHILD, name, str(tmp_path)], capture_output=True, text=True, env=env, timeout=600
    )
    assert "CAUGHT" in r.stdout, f"no pin caught the planted mistake {name}: rc={r.returncode} {r.stdout[-400:]} {r.stderr[-400:]}"
