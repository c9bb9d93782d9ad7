"""Seeded random configurations of prefill, decode and backward against the
fp64 oracle, through the C ABI.

The other GPU tests vary one or two factors at a time; here each seed draws a
whole configuration (dtype, head dim, GQA ratio, batch, query and key lengths,
causal flag, decode split count) from its own generator, so that factors meet
in combinations no hand-picked case names.  Sizes stay where the oracle checks
every output in well under a second, and the same tolerances apply
(tests/gpu_util.py; the backward's elementwise bound, tests/test_gpu_bwd.py).
"""
import numpy as np
import pytest

import math

import torch

import exact_io_aware_08_amd as fa
import oracle
from gpu_util import announce, compare, need_gpu, to_dev, widen
from test_gpu_bwd import run_bwd
from test_gpu_decode import _paged_case, run_decode
from test_gpu_fwd import run_case


def _lengths(rng, lo, hi, pairs_cap, BH):
    """Query and key lengths in [lo, hi); equal in about 40% of draws; the
    longer one halved until B*H*Nq*Nk fits the oracle budget."""
    nq = int(rng.integers(lo, hi))
    nk = nq if rng.random() < 0.4 else int(rng.integers(lo, hi))
    while BH * nq * nk > pairs_cap:
        if nq >= nk:
            nq = max(1, nq // 2)
        else:
            nk = max(1, nk // 2)
    return nq, nk


def _fwd_config(seed):
    rng = np.random.default_rng(71_000 + seed)
    dt = str(rng.choice(["bf16", "f16", "f32"]))
    d = int(rng.choice([64, 128] if dt == "f32" else [64, 128, 256]))
    Hkv = int(rng.integers(1, 4))
    H = Hkv * int(rng.choice([1, 2, 4, 5]))
    B = int(rng.integers(1, 3))
    Nq, Nk = _lengths(rng, 1, 900, 2_500_000, B * H)
    causal = bool(rng.random() < 0.6)
    return B, H, Hkv, Nq, Nk, d, dt, causal


def _bwd_config(seed):
    """Backward draws keep G*Nq <= 8*Nk (G = H/Hkv).  A dK or dV element sums
    G*Nq terms; the elementwise bound grows with the sum of their magnitudes,
    the gradient only with its square root, and the backward tests require the
    bound to stay under 5% of the largest gradient so that it can catch a
    wrong term.  At G*Nq/Nk = 13.8 (381 queries, 83 keys, G = 3) the dV bound
    reaches 6.4%; the hand-picked cases go up to 6.7."""
    rng = np.random.default_rng(72_000 + seed)
    dt = str(rng.choice(["bf16", "f16"]))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 3]))
    H = Hkv * G
    B = int(rng.integers(1, 3))
    Nq, Nk = _lengths(rng, 1, 420, 400_000, B * H)
    while G * Nq > 8 * Nk:
        Nq = max(1, Nq // 2)
    causal = bool(rng.random() < 0.6)
    return B, H, Hkv, Nq, Nk, d, dt, causal


def _decode_config(seed):
    rng = np.random.default_rng(73_000 + seed)
    dt = str(rng.choice(["bf16", "f16"]))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 5))
    H = Hkv * int(rng.choice([1, 3, 8, 16, 20]))   # 20: two query groups per KV head
    B = int(rng.integers(1, 5))
    Nk = int(rng.integers(1, 6000))
    splits = int(rng.choice([0, 1, 2, 5, 13]))
    return B, H, Hkv, Nk, d, dt, splits


def _paged_config(seed):
    rng = np.random.default_rng(74_000 + seed)
    dt = str(rng.choice(["bf16", "f16"]))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    H = Hkv * int(rng.choice([1, 4, 8, 20]))
    B = int(rng.integers(1, 7))
    page_size = int(rng.choice([32, 64, 96, 128, 256]))
    lens = [0 if rng.random() < 0.15 else int(rng.integers(1, 3000)) for _ in range(B)]
    splits = int(rng.choice([0, 3, 8]))
    return B, H, Hkv, d, dt, page_size, lens, splits


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(16))
def test_random_prefill(seed):
    B, H, Hkv, Nq, Nk, d, dt, causal = _fwd_config(seed)
    run_case(B, H, Hkv, Nq, Nk, d, dt, causal, seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(8))
def test_random_backward(seed):
    B, H, Hkv, Nq, Nk, d, dt, causal = _bwd_config(seed)
    run_bwd(B, H, Hkv, Nq, Nk, d, dt, causal, seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    B, H, Hkv, Nk, d, dt, splits = _decode_config(seed)
    run_decode(B, H, Hkv, Nk, d, dt, splits=splits, seed=seed, poison_ws=True)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(8))
def test_random_paged_decode(seed):
    """Paged cache over a random page permutation; table entries past each
    sequence are invalid (-7); the workspace starts as NaN."""
    need_gpu()
    B, H, Hkv, d, dt, ps, lens, splits = _paged_config(seed)
    announce(f"fa_decode_paged random seed={seed} B={B} H={H} Hkv={Hkv} d={d} {dt} "
             f"page={ps} lens={lens} splits={splits}")
    q, k, v, kp, vp, table, max_pages, _ = _paged_case(B, H, Hkv, lens, ps, d, dt, seed=seed)
    scale = float(np.float32(1 / math.sqrt(d)))
    ws = fa.decode_paged_workspace(B, H, Hkv, max_pages, ps, d, splits)
    if ws is not None:
        ws.fill_(255)
    o, lse = fa.decode_paged(to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=scale,
                             num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))
            continue
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], dt), widen(k[b:b + 1, :, :L], dt),
                                        widen(v[b:b + 1, :, :L], dt), False, scale)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, dt, f"paged b={b} L={L}")


def test_configs_span_the_factors():
    """The drawn configurations cover every dtype, head dim and mask mode,
    GQA and MHA, Nq < Nk and Nq > Nk, forced and automatic splits (host-only
    check of the draws above)."""
    f = [_fwd_config(s) for s in range(16)]
    assert {c[6] for c in f} == {"bf16", "f16", "f32"}
    assert {c[5] for c in f} == {64, 128, 256}
    assert {c[7] for c in f} == {True, False}
    assert any(c[1] > c[2] for c in f) and any(c[1] == c[2] for c in f)
    assert any(c[3] < c[4] for c in f) and any(c[3] > c[4] for c in f)
    b = [_bwd_config(s) for s in range(8)]
    assert {c[5] for c in b} == {64, 128} and {c[7] for c in b} == {True, False}
    assert all((c[1] // c[2]) * c[3] <= 8 * c[4] for c in b)
    dc = [_decode_config(s) for s in range(12)]
    assert {c[4] for c in dc} == {64, 128}
    assert 0 in {c[6] for c in dc} and len({c[6] for c in dc}) >= 3
    assert any(c[1] // c[2] > 16 for c in dc)
    pg = [_paged_config(s) for s in range(8)]
    assert {c[5] for c in pg} >= {32, 96} and any(0 in c[6] for c in pg)
    assert {c[7] for c in pg} == {0, 3, 8} and {c[3] for c in pg} == {64, 128}
