"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin is a plain function that raises AssertionError on failure, so the same
battery runs on the real oracle (tests/test_oracle_pins.py) and on copies of it
with a planted mistake (tests/test_oracle_mutants.py), where at least one pin
must fail.

What pins what:
  * brute force in 50-digit arithmetic (mpmath), with the softmax written
    without the max shift -- the exact definition of [MM] "Por que la atencion
    esta ligada a la memoria" / [SA] "Problematica dell'attention standard";
  * torch's fp64 CPU scaled_dot_product_attention and logsumexp (library);
  * closed forms (Q = 0, a single visible key, a very large scale);
  * invariants: probability rows sum to 1, convex hull, permutation
    equivariance, GQA == MHA with repeated KV, decode == last causal row,
    split-KV log-sum-exp merge == whole;
  * the online recurrence of [MM] "El algoritmo de atencion flash" and "La
    recurrencia de softmax en linea" (running max, running sum, accumulator
    rescaled by e^(m_old - m_new)), both with the tile-local max and
    per-step normalisation and with the deferred normalisation of [MM] "FA2:
    paralelismo", which must equal the two-pass definition;
  * E4M3 facts printed on the P-cast summary ([PC]) and torch's float8_e4m3fn;
  * the closed form F(Delta,S) and its printed constants ([PC] "Marco Teorico",
    "Optimizacion 1", "Optimizacion 2", "Contribuciones Clave").

Page keys: [MM] marketmaker.cc flash-attention blog post; [SA] systems-analysis
"FlashAttention (IT)"; [PC] gist.science "Precision de P-Cast en la Atencion
FP8"; [FV] gist.science "FlashAttention for Scalable Vector Architectures".
"""
from __future__ import annotations

import math
import os

import mpmath
import numpy as np
import torch

import oracle

RNG = np.random.default_rng(1234)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(fname: str) -> dict:
    """name -> float from a cited fixture in tests/golden (2^k allowed)."""
    out = {}
    for line in open(os.path.join(GOLDEN, fname)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        name, rest = line.split("=", 1)
        val = rest.split("|", 1)[0].strip()
        out[name.strip()] = 2.0 ** float(val[2:]) if val.startswith("2^") else float(val)
    return out


def _rand(*shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float32)


def _inputs(B, H, Hkv, Nq, Nk, d, seed=0, sc=1.0):
    g = np.random.default_rng(seed)
    q = (g.standard_normal((B, H, Nq, d)) * sc).astype(np.float32)
    k = (g.standard_normal((B, Hkv, Nk, d)) * sc).astype(np.float32)
    v = g.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    return q, k, v


def _visible(i, Nq, Nk, causal):
    if not causal:
        return Nk
    return max(0, min(Nk, i + (Nk - Nq) + 1))


# --------------------------------------------------------------------------
# brute force, 50 digits, no max shift
# --------------------------------------------------------------------------

def _brute(q, k, v, causal, scale):
    mpmath.mp.dps = 50
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = H // Hkv
    o = np.zeros((B, H, Nq, d))
    lse = np.zeros((B, H, Nq))
    sc = mpmath.mpf(float(scale))
    for b in range(B):
        for h in range(H):
            hk = h // g
            for i in range(Nq):
                lim = _visible(i, Nq, Nk, causal)
                if lim == 0:
                    lse[b, h, i] = -math.inf
                    continue
                w = []
                for j in range(lim):
                    s = mpmath.fsum(mpmath.mpf(float(q[b, h, i, c])) * mpmath.mpf(float(k[b, hk, j, c]))
                                    for c in range(d))
                    w.append(mpmath.exp(sc * s))
                z = mpmath.fsum(w)
                for c in range(d):
                    o[b, h, i, c] = float(mpmath.fsum(w[j] * mpmath.mpf(float(v[b, hk, j, c]))
                                                      for j in range(lim)) / z)
                lse[b, h, i] = float(mpmath.log(z))
    return o, lse


def pin_bruteforce_50_digits():
    cases = [
        (1, 2, 1, 5, 7, 3, False, 0.7),
        (2, 2, 2, 6, 6, 4, True, 0.5),
        (1, 4, 2, 4, 9, 3, True, 1.3),   # Nq < Nk, bottom-right causal, GQA
        (1, 1, 1, 7, 4, 2, True, 0.9),   # Nq > Nk: rows 0..2 see no key
    ]
    for n, (B, H, Hkv, Nq, Nk, d, causal, scale) in enumerate(cases):
        q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed=10 + n, sc=1.5)
        o, lse = oracle.attention(q, k, v, causal, scale)
        ob, lb = _brute(q, k, v, causal, scale)
        assert np.allclose(o, ob, rtol=1e-13, atol=1e-13), f"O mismatch case {n}"
        fin = np.isfinite(lb)
        assert np.array_equal(fin, np.isfinite(lse)), f"empty-row pattern case {n}"
        assert np.allclose(lse[fin], lb[fin], rtol=1e-13, atol=1e-13), f"LSE case {n}"
        assert np.all(o[~fin] == 0.0), f"empty rows must be zero, case {n}"


# --------------------------------------------------------------------------
# torch fp64 library routines
# --------------------------------------------------------------------------

def _torch_ref(q, k, v, causal, scale):
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = H // Hkv
    tq = torch.from_numpy(q).double()
    tk = torch.from_numpy(k).double().repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).double().repeat_interleave(g, dim=1)
    mask = None
    if causal:
        mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    s = (tq @ tk.transpose(-1, -2)) * scale
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def pin_torch_sdpa_fp64():
    cases = [
        (2, 4, 2, 37, 37, 16, False, 0.25),
        (2, 4, 2, 37, 37, 16, True, 0.25),
        (1, 6, 3, 21, 50, 8, True, 0.4),   # bottom-right mask, explicit in torch
        (3, 2, 1, 1, 65, 16, False, 0.25),  # decode shape
    ]
    for n, (B, H, Hkv, Nq, Nk, d, causal, scale) in enumerate(cases):
        q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed=20 + n)
        o, lse = oracle.attention(q, k, v, causal, scale)
        ot, lt = _torch_ref(q, k, v, causal, scale)
        assert np.allclose(o, ot, rtol=1e-12, atol=1e-12), f"O vs torch case {n}"
        assert np.allclose(lse, lt, rtol=1e-12, atol=1e-12), f"LSE vs torch case {n}"


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def pin_closed_form_zero_query():
    """Q = 0: every visible score is 0, so O_i is the mean of the visible V rows
    and LSE_i = ln(number of visible keys)."""
    B, H, Hkv, Nq, Nk, d = 1, 2, 1, 9, 13, 4
    _, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed=31)
    q = np.zeros((B, H, Nq, d), np.float32)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.5)
        for i in range(Nq):
            n = _visible(i, Nq, Nk, causal)
            exp_o = v[0, 0, :n].astype(np.float64).mean(axis=0)
            assert np.allclose(o[0, :, i], exp_o, atol=1e-14), (causal, i)
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-14, (causal, i)


def pin_closed_form_single_key():
    """Causal row 0 with Nq == Nk sees only key 0: O_0 = V_0, LSE_0 = s_00."""
    q, k, v = _inputs(2, 3, 3, 6, 6, 5, seed=32)
    o, lse = oracle.attention(q, k, v, True, 0.3)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(o[b, h, 0], v[b, h, 0].astype(np.float64))
            s00 = 0.3 * float(np.dot(q[b, h, 0].astype(np.float64), k[b, h, 0].astype(np.float64)))
            assert abs(lse[b, h, 0] - s00) < 1e-13


def pin_closed_form_large_scale():
    """As the scale grows the softmax becomes the indicator of the arg-max."""
    q, k, v = _inputs(1, 1, 1, 5, 11, 6, seed=33)
    s = q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T
    srt = np.sort(s, axis=1)
    scale = 80.0 / float((srt[:, -1] - srt[:, -2]).min())   # every runner-up below e^-80
    o, _ = oracle.attention(q, k, v, False, scale)
    for i in range(5):
        j = int(np.argmax(s[i]))
        assert np.allclose(o[0, 0, i], v[0, 0, j], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def pin_probability_rows():
    q, k, v = _inputs(2, 4, 2, 10, 14, 8, seed=41)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal, 0.35)
        for (b, h, i) in [(0, 0, 0), (1, 3, 9), (0, 2, 5), (1, 1, 3)]:
            p = oracle.attention_probs(q, k, causal, 0.35, b, h, i)
            n = _visible(i, 10, 14, causal)
            assert abs(p.sum() - 1.0) < 1e-13
            assert np.all(p[:n] > 0) and np.all(p[n:] == 0)
            assert np.allclose(p @ v[b, h // 2].astype(np.float64), o[b, h, i], atol=1e-13)


def pin_convex_hull():
    q, k, v = _inputs(1, 3, 3, 16, 16, 8, seed=42, sc=2.0)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal, 0.6)
        for i in range(16):
            n = _visible(i, 16, 16, causal)
            lo = v[0, :, :n].min(axis=1)
            hi = v[0, :, :n].max(axis=1)
            assert np.all(o[0, :, i] >= lo - 1e-14) and np.all(o[0, :, i] <= hi + 1e-14)


def pin_permutation_equivariance():
    q, k, v = _inputs(2, 2, 2, 12, 15, 6, seed=43)
    o, lse = oracle.attention(q, k, v, False, 0.4)
    pq = RNG.permutation(12)
    pk = RNG.permutation(15)
    o2, l2 = oracle.attention(q[:, :, pq], k, v, False, 0.4)
    assert np.allclose(o2, o[:, :, pq], atol=1e-14) and np.allclose(l2, lse[:, :, pq], atol=1e-14)
    o3, l3 = oracle.attention(q, k[:, :, pk], v[:, :, pk], False, 0.4)
    assert np.allclose(o3, o, atol=1e-13) and np.allclose(l3, lse, atol=1e-13)


def pin_gqa_equals_repeated_mha():
    q, k, v = _inputs(2, 8, 2, 9, 9, 4, seed=44)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.5)
        kr = np.repeat(k, 4, axis=1)
        vr = np.repeat(v, 4, axis=1)
        o2, l2 = oracle.attention(q, kr, vr, causal, 0.5)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def pin_decode_is_last_causal_row():
    q, k, v = _inputs(3, 4, 2, 17, 17, 8, seed=45)
    o, lse = oracle.attention(q, k, v, True, 0.35)
    od, ld = oracle.attention(q[:, :, -1:], k, v, True, 0.35)
    assert np.array_equal(od[:, :, 0], o[:, :, -1]) and np.array_equal(ld[:, :, 0], lse[:, :, -1])
    od2, ld2 = oracle.attention(q[:, :, -1:], k, v, False, 0.35)
    assert np.array_equal(od, od2) and np.array_equal(ld, ld2)


def pin_split_merge():
    """Attention over any partition of the keys merges to the whole with
    LSE = ln sum_s e^lse_s and O = sum_s e^(lse_s - LSE) O_s."""
    q, k, v = _inputs(1, 2, 1, 3, 40, 8, seed=46)
    o, lse = oracle.attention(q, k, v, False, 0.3)
    cuts = [0, 7, 8, 23, 40]
    parts = [oracle.attention(q, k[:, :, a:b], v[:, :, a:b], False, 0.3)
             for a, b in zip(cuts[:-1], cuts[1:])]
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[0] for p in parts])
    L = np.logaddexp.reduce(ls, axis=0)
    O = (np.exp(ls - L)[..., None] * os_).sum(axis=0)
    assert np.allclose(L, lse, atol=1e-13) and np.allclose(O, o, atol=1e-13)


def _online(q, k, v, causal, scale, Bc, deferred):
    """Tile-by-tile softmax for one (b,h) slice in fp64, in two forms that the
    recurrence of [MM] "La recurrencia de softmax en linea" makes equal to the
    two-pass definition:
      deferred=True:  running max m, unnormalised sum l and accumulator, one
                      division at the end (the form of "FA2: paralelismo");
      deferred=False: every tile is reduced to its own normalised state
                      (O_t, lse_t) -- a softmax-weighted mean of its V rows
                      and the log-sum-exp of its logits -- and folded into the
                      running normalised state with the log-sum-exp identity
                      lse' = log(e^lse + e^lse_t),
                      O' = e^(lse - lse') O + e^(lse_t - lse') O_t,
                      the same associativity the split-KV merge relies on."""
    Nq, d = q.shape
    Nk = k.shape[0]
    O = np.zeros((Nq, d))
    LSE = np.zeros(Nq)
    for i in range(Nq):
        lim = _visible(i, Nq, Nk, causal)
        m, l, acc = -math.inf, 0.0, np.zeros(d)     # deferred state
        lse, o = -math.inf, np.zeros(d)              # normalised state
        for j0 in range(0, lim, Bc):
            j1 = min(lim, j0 + Bc)
            s = scale * (k[j0:j1].astype(np.float64) @ q[i].astype(np.float64))
            vj = v[j0:j1].astype(np.float64)
            if deferred:
                mn = max(m, s.max())
                a = math.exp(m - mn) if m > -math.inf else 0.0
                p = np.exp(s - mn)
                l = a * l + p.sum()
                acc = a * acc + p @ vj
                m = mn
            else:
                lse_t = float(np.logaddexp.reduce(s))
                o_t = np.exp(s - lse_t) @ vj
                lse_n = float(np.logaddexp(lse, lse_t))
                o = math.exp(lse - lse_n) * o + math.exp(lse_t - lse_n) * o_t
                lse = lse_n
        if lim == 0:
            LSE[i] = -math.inf
            continue
        O[i] = acc / l if deferred else o
        LSE[i] = m + math.log(l) if deferred else lse
    return O, LSE


def pin_online_recurrence():
    q, k, v = _inputs(1, 1, 1, 70, 70, 8, seed=47)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.35)
        for Bc in (1, 3, 64, 70):
            for deferred in (False, True):
                O, L = _online(q[0, 0], k[0, 0], v[0, 0], causal, 0.35, Bc, deferred)
                assert np.allclose(O, o[0, 0], rtol=1e-13, atol=1e-13), (causal, Bc, deferred)
                assert np.allclose(L, lse[0, 0], rtol=1e-13, atol=1e-13), (causal, Bc, deferred)


def pin_row_subset_and_threads():
    q, k, v = _inputs(2, 2, 1, 33, 33, 8, seed=48)
    o, lse = oracle.attention(q, k, v, True, 0.35, nthreads=1)
    o8, l8 = oracle.attention(q, k, v, True, 0.35, nthreads=8)
    assert np.array_equal(o, o8) and np.array_equal(lse, l8)
    rows = np.array([[0, 5, 32], [1, 2, 3], [31, 30, 0], [7, 7, 8]])
    orow, lrow = oracle.attention(q, k, v, True, 0.35, rows=rows)
    for bh in range(4):
        b, h = divmod(bh, 2)
        assert np.array_equal(orow[b, h], o[b, h, rows[bh]])
        assert np.array_equal(lrow[b, h], lse[b, h, rows[bh]])


# --------------------------------------------------------------------------
# E4M3 codec
# --------------------------------------------------------------------------

def pin_e4m3_page_constants():
    """[PC]: 3-bit mantissa; round-to-zero threshold 2^-10 ("Marco Teorico");
    normal range from 2^-6, largest value 448 ("Optimizacion 2")."""
    g = golden("pcast_page_values.txt")
    dec = oracle.e4m3_decode(np.arange(256))
    fin = dec[np.isfinite(dec)]
    assert fin.max() == g["max_finite"] and dec[0x7E] == g["max_finite"]
    assert np.min(fin[fin >= g["min_normal"]]) == g["min_normal"] == dec[0x08]
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    # everything at or below the round-to-zero threshold encodes to 0 (the
    # tie goes to the even code 0), anything above it to a nonzero code
    t = np.float32(g["round_to_zero"])
    assert oracle.e4m3_encode(t) == 0
    assert oracle.e4m3_encode(np.nextafter(t, np.float32(1))) != 0
    assert np.min(fin[fin > 0]) == 2 * g["round_to_zero"]  # smallest subnormal
    # mantissa bits: one step between 1 and 2 is 2^-(bits)
    assert dec[0x39] - dec[0x38] == 2.0 ** -g["e4m3_mantissa_bits"] and dec[0x38] == 1.0


def pin_e4m3_vs_torch():
    dec = oracle.e4m3_decode(np.arange(256))
    td = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    same = (dec == td) | (np.isnan(dec) & np.isnan(td))
    assert same.all()
    # encode: every fp32 magnitude on a dense grid below 464, plus all midpoints
    grid = np.concatenate([
        np.float32(2.0) ** np.linspace(-14, 8.85, 40000).astype(np.float32),
        (fin := np.unique(dec[np.isfinite(dec) & (dec >= 0)])),
        ((fin[1:] + fin[:-1]) / 2).astype(np.float32),
        np.nextafter(((fin[1:] + fin[:-1]) / 2).astype(np.float32), np.float32(0)),
        np.nextafter(((fin[1:] + fin[:-1]) / 2).astype(np.float32), np.float32(1e9)),
    ]).astype(np.float32)
    grid = np.concatenate([grid, -grid])
    ours = oracle.e4m3_encode(grid)
    theirs = torch.from_numpy(grid).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


# --------------------------------------------------------------------------
# closed forms of the P-cast summary
# --------------------------------------------------------------------------

def pin_expected_max_gauss():
    assert abs(oracle.expected_max_gauss(1)) < 1e-12
    assert abs(oracle.expected_max_gauss(2) - 1 / math.sqrt(math.pi)) < 1e-10
    assert abs(oracle.expected_max_gauss(3) - 1.5 / math.sqrt(math.pi)) < 1e-10
    d4 = oracle.expected_max_gauss(4)
    mc = np.random.default_rng(5).standard_normal((2_000_000, 4)).max(axis=1).mean()
    assert abs(d4 - mc) < 3e-3
    # [PC] "Marco Teorico" prints "roughly 1.0" for k = 4 (exact value 1.0294)
    assert abs(d4 - golden("pcast_page_values.txt")["delta_k4"]) < 0.05


def pin_F_closed_form():
    g = golden("pcast_page_values.txt")
    d4 = oracle.expected_max_gauss(4)
    # 6.93 is -ln of the 2^-10 round-to-zero threshold
    assert abs(-math.log(g["round_to_zero"]) - g["ln_round_to_zero"]) < 5e-3
    for S in (1.0, 256.0, 448.0):
        dc = oracle.delta_c(S, d4)
        assert abs(dc - (g["ln_round_to_zero"] + math.log(S) - d4)) < 5e-3  # "Contribuciones Clave"
        assert abs(oracle.F_closed_form(dc, S, d4) - 0.5) < 1e-12
    # threshold effect near Delta 6-7 for S = 1 ("Marco Teorico")
    lo, hi = g["collapse_delta_lo"], g["collapse_delta_hi"]
    assert oracle.F_closed_form(lo - 2, 1, d4) < 0.05 < 0.5 < oracle.F_closed_form(hi, 1, d4)
    assert lo - 0.2 < oracle.delta_c(1.0, d4) < hi
    # monotone in Delta, decreasing in S
    fs = [oracle.F_closed_form(x, 1, d4) for x in np.linspace(0, 14, 29)]
    assert all(a < b for a, b in zip(fs, fs[1:]))
    assert oracle.F_closed_form(8, 256, d4) < oracle.F_closed_form(8, 1, d4)
    # Monte Carlo of the model behind F: non-sink logit z ~ N(0,1) is flushed
    # when S * e^(z - m) <= 2^-10 with m = Delta + delta_k
    z = np.random.default_rng(6).standard_normal(4_000_000)
    for delta, S in ((6.0, 1.0), (8.0, 1.0), (10.0, 256.0)):
        m = delta + d4
        frac = np.mean(S * np.exp(z - m) <= 2.0 ** -10)
        assert abs(frac - oracle.F_closed_form(delta, S, d4)) < 2e-3
    # "Optimizacion 1": reverse order, S = 256, N <= 1e6: the pre-sink max is a
    # max of N standard normals, and the flush probability stays below 1e-12
    n_max = g["reverse256_max_n"]
    m_pre = 4.9  # E[max of 1e6 N(0,1)] is about 4.86
    assert n_max == 1e6
    assert oracle.Phi(m_pre - g["ln_round_to_zero"] - math.log(256.0)) < g["reverse256_bound"]


def pin_dp():
    """[PC] "Optimizacion 2": d_p(S) is a sawtooth whose lower envelope is at
    powers of two with value 2^-4; S = 448 sits 14% above it; 2^-6/256 = 2^-14."""
    g = golden("pcast_page_values.txt")
    for kexp in range(0, 9):
        assert oracle.dp(2.0 ** kexp) == g["dp_envelope"]
    assert abs(oracle.dp(448.0) / g["dp_envelope"] - (1 + g["dp_448_excess"])) < 0.01
    # brute force over the code table for representable S: (S - pred(S)) / S
    dec = oracle.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    for S in (1.0, 2.0, 16.0, 240.0, 256.0, 320.0, 416.0, 448.0):
        pred = dec[dec < S].max()
        assert abs(oracle.dp(S) - (S - pred) / S) < 1e-15, S
    assert g["min_normal"] / 256 == g["coverage_256"]


def pin_trading_day_workload():
    """[MM] opening paragraphs: a day of 23,400 one-second steps, 12 heads,
    an fp16 score matrix of about 12.9 GB -- the full-size prefill shape."""
    import fagen
    g = golden("trading_day.txt")
    c3 = fagen.WORKLOADS["trading_day_prefill_bf16"]
    assert c3["Nq"] == c3["Nk"] == g["steps_per_day"] == 6.5 * 3600 and c3["H"] == g["heads"]
    gb = g["steps_per_day"] ** 2 * g["heads"] * 2 / 1e9
    assert abs(gb - g["score_matrix_gb_printed"]) / g["score_matrix_gb_printed"] < 0.10


# --------------------------------------------------------------------------
# backward ([MM] "Pase hacia atras": P recomputed from the stored statistics)
# --------------------------------------------------------------------------

def _torch_grads(q, k, v, dout, causal, scale):
    """fp64 autograd of torch SDPA with an explicit bottom-right mask."""
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = H // Hkv
    tq = torch.from_numpy(q).double().requires_grad_()
    tk = torch.from_numpy(k).double().requires_grad_()
    tv = torch.from_numpy(v).double().requires_grad_()
    mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq) if causal else None
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=mask,
        scale=scale)
    o.backward(torch.from_numpy(dout).double())
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_bwd_torch_autograd():
    cases = [
        (2, 4, 2, 37, 37, 16, True, 0.25),
        (1, 3, 3, 20, 20, 8, False, 0.5),
        (1, 6, 3, 21, 50, 8, True, 0.4),    # bottom-right mask, Nq < Nk
        (1, 4, 1, 45, 45, 32, True, 0.177),  # MQA
    ]
    for n, (B, H, Hkv, Nq, Nk, d, causal, scale) in enumerate(cases):
        q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed=70 + n)
        dout = np.random.default_rng(80 + n).standard_normal((B, H, Nq, d)).astype(np.float32)
        ours = oracle.attention_bwd(q, k, v, dout, causal, scale)
        ref = _torch_grads(q, k, v, dout, causal, scale)
        for name, a, b in zip(("dq", "dk", "dv"), ours, ref):
            assert np.allclose(a, b, rtol=1e-11, atol=1e-11), f"{name} vs torch case {n}"


def pin_bwd_finite_differences():
    """Central differences of L = sum(O * dO) through the forward oracle, on a
    causal case with Nq > Nk (rows without keys contribute nothing)."""
    B, H, Hkv, Nq, Nk, d, scale = 1, 2, 1, 7, 5, 4, 0.6
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed=91)
    dout = np.random.default_rng(92).standard_normal((B, H, Nq, d)).astype(np.float32)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, True, scale)
    h = 2.0 ** -10   # exact in fp32 for these magnitudes

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, True, scale)
        return float(np.sum(o * dout))

    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(arr.shape):
            x0 = arr[idx]
            arr[idx] = x0 + np.float32(h)
            lp = loss(q, k, v)
            arr[idx] = x0 - np.float32(h)
            lm = loss(q, k, v)
            arr[idx] = x0
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-5 * (1 + abs(grad[idx])), (idx, fd, grad[idx])


def pin_bwd_sum_rules():
    """Adding one vector to every key leaves each softmax row unchanged, so
    sum_j dK_j = 0; adding one vector to every value adds it to every O row
    with a visible key, so sum_j dV_j = sum of those dO_i (per KV head)."""
    B, H, Hkv, Nq, Nk, d = 2, 6, 2, 40, 64, 16
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed=93)
    dout = np.random.default_rng(94).standard_normal((B, H, Nq, d)).astype(np.float32)
    for causal in (False, True):
        dq, dk, dv, adq, adk, adv = oracle.attention_bwd(q, k, v, dout, causal, 0.3, abs_sums=True)
        assert np.abs(dk.sum(axis=2)).max() < 1e-10
        g = H // Hkv
        want = dout.astype(np.float64).reshape(B, Hkv, g, Nq, d).sum(axis=(2, 3))
        assert np.abs(dv.sum(axis=2) - want).max() < 1e-10
        # the absolute sums bound the gradients (triangle inequality)
        for a, b in ((dq, adq), (dk, adk), (dv, adv)):
            assert np.all(np.abs(a) <= b * (1 + 1e-12) + 1e-300)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


# --------------------------------------------------------------------------
# P-cast emulation ([PC] "Planteamiento del Problema", "Optimizacion 1/2")
# --------------------------------------------------------------------------

def _pcast_python(q, k, v, scale, Bc, S, reverse, n_sink, tile_local=False):
    """Independent tiny implementation; the E4M3 cast is torch's float8_e4m3fn.
    tile_local: P relative to each tile's own max, weight exp(mt - m_new)."""
    Nq, d = q.shape
    Nk = k.shape[0]
    O = np.zeros((Nq, d))
    L = np.zeros(Nq)
    cnt = [0, 0, 0, 0]
    sink_end = -(-n_sink // Bc) * Bc
    for i in range(Nq):
        lim = _visible(i, Nq, Nk, True)
        tiles = list(range(-(-lim // Bc)))
        if reverse:
            tiles = tiles[::-1]
        m, l, acc = np.float32(-np.inf), 0.0, np.zeros(d)
        for t in tiles:
            js = range(t * Bc, min(lim, (t + 1) * Bc))
            s = [np.float32(float(np.float32(scale)) * float(np.dot(q[i].astype(np.float64),
                                                                    k[j].astype(np.float64))))
                 for j in js]
            mn = max([m] + s)
            mt = max(s)
            ref = mt if tile_local else mn
            w = math.exp(float(mt) - float(mn)) if tile_local else 1.0
            a = 0.0 if m == -np.inf else math.exp(float(m) - float(mn))
            l *= a
            acc *= a
            for j, sj in zip(js, s):
                p = np.float32(math.exp(float(sj) - float(ref)))
                l += float(p) * w
                x = np.float32(p * np.float32(S))
                pt = float(torch.tensor([float(x)], dtype=torch.float32)
                           .to(torch.float8_e4m3fn).float()[0])
                fl = int(pt == 0.0 and p > 0)
                if j >= n_sink:
                    cnt[0] += 1
                    cnt[1] += fl
                if j >= sink_end:
                    cnt[2] += 1
                    cnt[3] += fl
                acc += w * pt * v[j].astype(np.float64)
            m = mn
        O[i] = acc / (S * l)
        L[i] = float(m) + math.log(l)
    return O, L, cnt


def pin_pcast_bruteforce_tiny():
    g = np.random.default_rng(61)
    N, d = 19, 4
    q = g.standard_normal((1, 1, N, d)).astype(np.float32) * 2.5
    k = g.standard_normal((1, 1, N, d)).astype(np.float32) * 2.5
    v = g.standard_normal((1, 1, N, d)).astype(np.float32)
    k[0, 0, :2, 0] += 6.0   # two sink keys
    q[0, 0, :, 0] = 1.0
    for (Bc, S, rev) in ((4, 1.0, False), (4, 256.0, True), (3, 448.0, False), (5, 256.0, False)):
        for tl in (False, True):
            o, lse, cnt = oracle.pcast_emulate(q, k, v, True, 0.5, Bc, S, rev, n_sink=2, tile_local=tl)
            O, L, c2 = _pcast_python(q[0, 0], k[0, 0], v[0, 0], 0.5, Bc, S, rev, 2, tile_local=tl)
            assert np.allclose(o[0, 0], O, rtol=1e-12, atol=1e-12), (Bc, S, rev, tl)
            assert np.allclose(lse[0, 0], L, rtol=1e-12, atol=1e-12), (Bc, S, rev, tl)
            assert cnt == c2, (Bc, S, rev, tl, cnt, c2)


def pin_pcast_tile_local_ablation():
    """The tile-local ablation: with one tile covering every key it is the
    running-max emulation exactly; with many tiles on a strong sink (forward,
    S = 1) it flushes far fewer non-sink values, since every tile's largest P
    casts from exactly S instead of from a value shrunk by the sink."""
    q, k, v = _inputs(1, 2, 2, 200, 200, 16, seed=64)
    q[..., 0] = 1.0
    k[:, :, :4, 0] += 8.0 * 4.0
    a = oracle.pcast_emulate(q, k, v, True, 0.25, 256, 1.0, False, 4)
    b = oracle.pcast_emulate(q, k, v, True, 0.25, 256, 1.0, False, 4, tile_local=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]
    run = oracle.pcast_emulate(q, k, v, True, 0.25, 16, 1.0, False, 4)
    loc = oracle.pcast_emulate(q, k, v, True, 0.25, 16, 1.0, False, 4, tile_local=True)
    assert run[2][1] > 0.5 * run[2][0], run[2]           # P-collapse under the running max
    assert loc[2][3] < 0.1 * max(run[2][3], 1), (run[2], loc[2])


def pin_pcast_single_key():
    """Causal row 0 sees key 0 only: p = 1, S*p = S is exact in E4M3 for
    S = 1, 256, 448, so O_0 = V_0 and LSE_0 is the fp32 logit s_00."""
    q, k, v = _inputs(1, 2, 2, 5, 5, 8, seed=62)
    for S in (1.0, 256.0, 448.0):
        for rev in (False, True):
            o, lse, _ = oracle.pcast_emulate(q, k, v, True, 0.35, 64, S, rev)
            for h in range(2):
                assert np.array_equal(o[0, h, 0], v[0, h, 0].astype(np.float64))
                s00 = np.float32(float(np.float32(0.35)) * float(
                    np.dot(q[0, h, 0].astype(np.float64), k[0, h, 0].astype(np.float64))))
                assert lse[0, h, 0] == float(s00)


def pin_pcast_error_bound():
    """The emulation stays within the per-element bound of oracle.pcast_bound
    around exact attention, for both orders and several S."""
    pcast_bound = oracle.pcast_bound
    q, k, v = _inputs(1, 2, 2, 150, 150, 16, seed=63, sc=1.7)
    q[..., 0] = 1.0
    k[:, :, :4, 0] += 9.0 * 4.0   # strong sink: many flushes at S = 1 forward
    o_ex, _ = oracle.attention(q, k, v, True, 0.25)
    for S, rev, Bc in ((1.0, False, 32), (256.0, True, 32), (448.0, False, 64), (256.0, False, 7)):
        o, _, _ = oracle.pcast_emulate(q, k, v, True, 0.25, Bc, S, rev, n_sink=4)
        for h in range(2):
            a = np.stack([oracle.attention_probs(q, k, True, 0.25, 0, h, i) for i in range(150)])
            bnd = pcast_bound(a, v[0, h], S)
            err = np.abs(o[0, h] - o_ex[0, h])
            assert np.all(err <= bnd), (S, rev, Bc, float((err - bnd).max()))


def _model_flush(delta, S, n=200_000):
    """Monte Carlo of the model behind F: a query's sink logits are Delta plus
    4 iid N(0,1); a non-sink logit z ~ N(0,1) flushes when S e^(z-M) <= 2^-10."""
    g = np.random.default_rng(7)
    M = delta + g.standard_normal((n, 4)).max(axis=1)
    z = g.standard_normal(n)
    return float(np.mean(S * np.exp(z - M) <= 2.0 ** -10))


def pin_pcast_underflow_claims():
    """On the sink workload (reduced to N = 2048, 2 heads, d = 64):
      * forward order: the non-sink flush fraction follows the page's closed
        form F(Delta,S) within 0.05 where 0.01 <= F <= 0.99, and the Monte
        Carlo of its model within 0.01 everywhere;
      * reverse order with S = 256: no flush among values cast before the
        sink block ([PC] "Optimizacion 1");
      * orderings of [PC] "Resultados Experimentales": MSE of (forward, S=1)
        exceeds (reverse, S=256) at moderate Delta; forward S=448 is worse
        than forward S=256; reverse+256 and forward+256 agree closely.  The
        page's 3-10x magnitude (N = 4096, its own V) is not pinned here."""
    import fagen
    d4 = oracle.expected_max_gauss(4)
    N, d = 2048, 64
    scale = float(np.float32(1 / math.sqrt(d)))
    for delta in (4.0, 6.0, 8.0, 10.0):
        q, k, v = fagen.sink_inputs(0, 1, 2, N, d, delta)
        rows = np.arange(0, N, 4)
        o_ex, _ = oracle.attention(q, k, v, True, scale, rows=rows)
        o_f, _, cf = oracle.pcast_emulate(q, k, v, True, scale, 64, 1.0, False, 4, rows=rows)
        o_r, _, cr = oracle.pcast_emulate(q, k, v, True, scale, 64, 256.0, True, 4, rows=rows)
        o_f256, _, _ = oracle.pcast_emulate(q, k, v, True, scale, 64, 256.0, False, 4, rows=rows)
        o_f448, _, _ = oracle.pcast_emulate(q, k, v, True, scale, 64, 448.0, False, 4, rows=rows)
        frac = cf[1] / cf[0]
        F = oracle.F_closed_form(delta, 1.0, d4)
        if 0.01 <= F <= 0.99:
            assert abs(frac - F) <= 0.05, (delta, frac, F)
        assert abs(frac - _model_flush(delta, 1.0)) <= 0.01, (delta, frac)
        assert cr[3] == 0, (delta, cr)
        mse = {n: np.mean((x - o_ex) ** 2) for n, x in
               (("f1", o_f), ("r256", o_r), ("f256", o_f256), ("f448", o_f448))}
        if delta in (6.0, 8.0):
            assert mse["f1"] > 1.2 * mse["r256"], (delta, mse)
        assert mse["f448"] > mse["f256"], (delta, mse)
        assert abs(mse["r256"] - mse["f256"]) < 0.05 * mse["f256"], (delta, mse)



# ---------------------------------------------------------------------------
# FP8 quantisation with incoherent processing ([MM] "FA3: Mecanica de la
# tolva", item 3): random-sign Hadamard rotation, power-of-two group scales,
# E4M3 codes.
# ---------------------------------------------------------------------------

def _sylvester(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h


def _min_exponent(amax):
    """Brute force: the smallest e >= -126 with amax <= 448 * 2^e (exact in fp64)."""
    if amax == 0:
        return -126
    e = -126
    while float(amax) > 448.0 * 2.0 ** e:
        e += 1
    return e


def pin_quant_hadamard_matrix():
    """Sparse small-integer rows: every rotated entry is an integer of size <= 16,
    which E4M3 holds exactly at any power-of-two scale, so the dequantised
    codes must equal H_d (s o x) computed with the explicit Sylvester matrix."""
    g = np.random.default_rng(21)
    for d in (64, 128):
        Hm = _sylvester(d)
        x = np.zeros((1, 2, 40, d), np.float32)
        for r in range(80):
            idx = g.choice(d, size=3, replace=False)
            x.reshape(80, d)[r, idx] = g.choice([-2.0, -1.0, 1.0, 2.0, 3.0], size=3)
        s = np.where(g.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
        codes, sc = oracle.quant_e4m3(x, signs=s)
        got = oracle.dequant_e4m3(codes, sc).astype(np.float64)
        want = (x.astype(np.float64) * s) @ Hm.T
        assert np.abs(want).max() <= 16
        assert np.array_equal(got, want), d
        # H^T H = d I: dot products scale by exactly d
        assert np.allclose(got[0, 0] @ got[0, 1].T, d * (x[0, 0].astype(np.float64) @ x[0, 1].T))


def pin_quant_scale_minimal():
    """Each 32-row block's scale is 2^e with e the brute-force minimal exponent."""
    g = np.random.default_rng(22)
    N, d = 32 * 12 + 7, 64
    x = g.standard_normal((1, 1, N, d)).astype(np.float32)
    mags = [0.0, 2.0 ** -140, 2.0 ** -118, 1e-9, 0.5, 1.0, 1.75, 1.7500001, 448.0, 449.0,
            3.0e5, 2.0 ** 100, 7.0 * 2.0 ** 40]
    for t, m in enumerate(mags):
        blk = x[0, 0, 32 * t:32 * t + 32]
        if m == 0.0:
            blk[:] = 0.0
        else:
            blk *= np.float32(m) / np.abs(blk).max()
            blk[0, 0] = np.float32(m)          # amax exactly m (as float32)
    codes, sc = oracle.quant_e4m3(x)
    for t in range(sc.shape[2]):
        amax = float(np.abs(x[0, 0, 32 * t:32 * t + 32]).max())
        assert sc[0, 0, t] == np.float32(2.0 ** _min_exponent(amax)), (t, amax, sc[0, 0, t])
        assert amax <= 448.0 * float(sc[0, 0, t])


def pin_quant_codes_vs_torch():
    """Codes equal torch's float8_e4m3fn conversion of x / scale, and the round
    trip stays within half an E4M3 step."""
    g = np.random.default_rng(23)
    x = (g.standard_normal((2, 3, 100, 64)) * np.exp(g.normal(0, 3, (2, 3, 100, 1)))).astype(np.float32)
    codes, sc = oracle.quant_e4m3(x)
    srow = np.repeat(sc, 32, axis=2)[:, :, :100, None]
    ref = torch.from_numpy((x / srow).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    deq = oracle.dequant_e4m3(codes, sc).astype(np.float64)
    y = x.astype(np.float64) / srow
    bound = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** -4 * np.abs(y), 2.0 ** -10) * srow
    assert np.all(np.abs(deq - x) <= bound + 0.0)


def pin_quant_group_layouts():
    """Channel groups, whole-tensor groups and a ragged last row block."""
    g = np.random.default_rng(24)
    B, H, N, d = 2, 2, 70, 64
    x = g.standard_normal((B, H, N, d)).astype(np.float32)
    x[1, 0, :, 5] *= 1000.0
    x[0, 1, 64:, :] *= 1e-3
    _, sc = oracle.quant_e4m3(x, layout="channels")
    assert sc.shape == (B, H, d)
    for b in range(B):
        for h in range(H):
            for c in range(d):
                assert sc[b, h, c] == np.float32(2.0 ** _min_exponent(float(np.abs(x[b, h, :, c]).max())))
    _, sc = oracle.quant_e4m3(x, layout="rows32")
    assert sc.shape == (B, H, 3)
    assert sc[0, 1, 2] == np.float32(2.0 ** _min_exponent(float(np.abs(x[0, 1, 64:]).max())))
    for lay in ("rows32", "channels"):
        _, sc = oracle.quant_e4m3(x, layout=lay, whole=True)
        assert np.all(sc == np.float32(2.0 ** _min_exponent(float(np.abs(x).max())))), lay


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
