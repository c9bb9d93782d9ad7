"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/oracle.c with one plausible mistake (a dropped
term, a wrong sign, index or operand), built with gcc on the CPU into a
temporary directory.  The pin battery of tests/pins_oracle.py runs against it
and must fail at least once; the pristine source must pass every pin.
"""
import os
import tempfile

import pytest

import oracle
from pins_oracle import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement, occurrence to change)
MUTANTS = [
    ("no_max_shift", "s[j] = exp(s[j] - m); l += s[j];", "s[j] = exp(s[j]); l += s[j];", 0),
    ("top_left_causal", "i64 lim = i + (J->Nk - J->Nq) + 1;", "i64 lim = i + 1;", 0),
    ("causal_off_by_one", "i64 lim = i + (J->Nk - J->Nq) + 1;", "i64 lim = i + (J->Nk - J->Nq);", 0),
    ("gqa_modulo", "hk = h / g;", "hk = h % J->Hkv;", 0),
    ("lse_sign", "*lse_out = m + log(l);", "*lse_out = m - log(l);", 0),
    ("scale_dropped", "s[j] = J->scale * dot(qi, kb + j * d, d);", "s[j] = dot(qi, kb + j * d, d);", 0),
    ("no_normalise", "const double p = s[j] / l;", "const double p = s[j];", 0),
    ("batch_head_swap", "J->q + ((b * J->H + h) * J->Nq + i) * d;", "J->q + ((h * J->B + b) * J->Nq + i) * d;", 0),
    ("v_uses_key", "o_row[c] += p * (double)vj[c];", "o_row[c] += p * (double)(kb + j * d)[c];", 0),
    ("pcast_no_rescale", "for (i64 c = 0; c < d; ++c) o_row[c] *= a;", "", 0),
    ("pcast_reverse_ignored", "J->reverse ? (ntiles - 1 - tt) : tt", "tt", 0),
    ("pcast_sum_of_cast", "l += (double)p * beta;",
     "l += (double)orc_e4m3_decode(orc_e4m3_encode(p * J->p_scale)) / J->p_scale * beta;", 0),
    ("pcast_tile_local_weight_dropped", "const double beta = J->tile_local ? exp((double)mt - (double)mn) : 1.0;",
     "const double beta = 1.0;", 0),
    ("pcast_tile_local_uses_running_max", "const float pref = J->tile_local ? mt : mn;",
     "const float pref = mn;", 0),
    ("pcast_tile_local_max", "float mn = m;", "float mn = -INFINITY;", 0),
    ("pcast_scale_not_divided", "const double den = (double)J->p_scale * l;", "const double den = l;", 0),
    ("e4m3_subnormal_step", "nearbyint(a * 512.0)", "nearbyint(a * 1024.0)", 0),
    ("e4m3_ties_away", "nearbyint(ldexp(a, 3 - E))", "round(ldexp(a, 3 - E))", 0),
    ("F_sign_of_delta_k", "delta + delta_k - 10.0 * log(2.0) - log(S)", "delta - delta_k - 10.0 * log(2.0) - log(S)", 0),
    ("dp_exponent", "ldexp(1.0, (int)k - 4) / S", "ldexp(1.0, (int)k - 3) / S", 0),
    ("bwd_no_D", "const double ds = p[j] * (dp[j] - D);", "const double ds = p[j] * dp[j];", 0),
    ("bwd_dk_unscaled", "dkb[j * d + c] += J->scale * ds * (double)qi[c];",
     "dkb[j * d + c] += ds * (double)qi[c];", 0),
    ("bwd_dv_uses_dp", "dvb[j * d + c] += p[j] * (double)doi[c];",
     "dvb[j * d + c] += dp[j] * (double)doi[c];", 0),
    ("bwd_dq_uses_v", "dqi[c] += J->scale * ds * (double)kj[c];",
     "dqi[c] += J->scale * ds * (double)(vb + j * d)[c];", 0),
    ("fwht_difference_sign", "y[j + h] = a - b;", "y[j + h] = b - a;", 0),
    ("fwht_last_stage_dropped", "for (i64 h = 1; h < d; h *= 2)", "for (i64 h = 1; h < d / 2; h *= 2)", 0),
    ("rotation_signs_ignored", "signs ? signs[c] * x[r * d + c] : x[r * d + c]", "x[r * d + c]", 0),
    ("scale_exponent_one_low", "(f <= 0.875) ? E2 - 9 : E2 - 8", "(f <= 0.875) ? E2 - 9 : E2 - 9", 0),
    ("row_block_of_31", "bh * nblk + i / 32 : bh * d + c;", "bh * nblk + i / 31 : bh * d + c;", 0),
    ("whole_tensor_ignored", "if (whole) {", "if (0) {", 0),
    ("bwd_gqa_one_head", "for (i64 h = hk * g; h < (hk + 1) * g; ++h) {",
     "for (i64 h = hk * g; h < hk * g + 1; ++h) {", 0),
]


def _mutate(src, old, new, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = src.index(old, idx + 1)
    return src[:idx] + new + src[idx + len(old):]


def _first_failure():
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            return f"{pin.__name__}: {type(e).__name__}"
    return None


def test_pristine_passes_all_pins():
    assert _first_failure() is None


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, occ, tmp_path):
    src = open(SRC).read()
    assert old in src, f"mutation target for {name} not found"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(_mutate(src, old, new, occ))
    lib = oracle.compile_library(str(mut), str(tmp_path / "liboracle_mut.so"))
    with oracle.use_library(lib):
        failure = _first_failure()
    assert failure is not None, f"mutant {name} passed every pin"
