"""GPU parity of fa_fwd (prefill) against the fp64 oracle, through the C ABI.

Full-size workloads are checked on seeded sampled rows (the oracle computes
them one by one); smaller shapes that still span several tiles and ragged
tails are checked on every output.  Tolerances: tests/gpu_util.py.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_08_amd as fa
import fagen
import oracle
from gpu_util import TORCH_DT, announce, compare, need_gpu, to_dev, widen

pytestmark = pytest.mark.gpu


def _scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))


def run_case(B, H, Hkv, Nq, Nk, d, dt, causal, seed=0, kind="iid", rows=None, scale=None):
    need_gpu()
    scale = _scale(d) if scale is None else scale
    announce(f"fa_fwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} causal={causal} "
             f"kind={kind} seed={seed}")
    cfg = dict(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dt, kind=kind)
    q, k, v = fagen.make_inputs(cfg, seed)
    o, lse = fa.fwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(widen(q, dt), widen(k, dt), widen(v, dt), causal, scale,
                                      rows=rows)
    if rows is not None:
        r = np.asarray(rows).reshape(B * H, -1)
        og = o.reshape(B * H, Nq, d)[torch.arange(B * H)[:, None], torch.from_numpy(r)]
        lg = lse.reshape(B * H, Nq)[torch.arange(B * H)[:, None], torch.from_numpy(r)]
        return compare(og.reshape(B, H, -1, d), lg.reshape(B, H, -1), o_ref, lse_ref, dt,
                       "sampled rows")
    return compare(o, lse, o_ref, lse_ref, dt, "all rows")


def test_tiny_exact_f32():
    """256 x 64 fp32, full attention, seed 0."""
    c = fagen.WORKLOADS["tiny_exact_f32"]
    m = run_case(1, 1, 1, 256, 256, 64, "f32", False, scale=c["scale"])
    assert m["max_abs"] <= 1e-5


def _sampled_rows(B, H, N, n, seed=0):
    rows = [np.unique(np.concatenate([[0, N - 1], fagen.sample_rows(seed, bh, N, n)]))
            for bh in range(B * H)]
    width = min(len(r) for r in rows)
    return np.stack([r[:width] for r in rows])


def test_gpt2_small_prefill_bf16_sampled():
    """B=4, H=12, N=2048, d=64, bf16, causal: 128 sampled rows per head plus
    the first and last row."""
    rows = _sampled_rows(4, 12, 2048, 128)
    run_case(4, 12, 12, 2048, 2048, 64, "bf16", True, rows=rows)


def test_trading_day_prefill_bf16_sampled():
    """B=1, H=12, N=23,400, d=64, bf16, causal, AR(1)+noise inputs: 512 seeded
    sampled rows per head plus rows 0 and N-1."""
    N = 23400
    rows = np.stack([np.unique(np.concatenate([[0, N - 1], fagen.sample_rows(0, h, N, 512)]))
                     for h in range(12)])
    run_case(1, 12, 12, N, N, 64, "bf16", True, kind="ar1", rows=rows)


@pytest.mark.parametrize("N", [1, 63, 65, 127, 129, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths_bf16(N, causal):
    run_case(1, 2, 2, N, N, 64, "bf16", causal, seed=N)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_dtypes_and_head_dims(dt, d):
    run_case(2, 3, 3, 300, 300, d, dt, True, seed=7)
    run_case(1, 2, 2, 257, 257, d, dt, False, seed=8)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_head_dim_256(dt):
    """d = 256 (16-bit types only): causal and full, ragged query and key
    tails, GQA, Nq != Nk."""
    run_case(2, 4, 2, 300, 300, 256, dt, True, seed=11)
    run_case(1, 2, 1, 257, 257, 256, dt, False, seed=12)
    run_case(1, 2, 2, 100, 333, 256, dt, True, seed=13)
    run_case(1, 2, 2, 1, 65, 256, dt, False, seed=14)


def test_head_dim_256_long_sampled():
    """B=1, H=8, Hkv=2, N=4,096, d=256, bf16, causal, AR(1) inputs: 96 sampled
    rows per head plus the first and last row."""
    rows = _sampled_rows(1, 8, 4096, 96, seed=3)
    run_case(1, 8, 2, 4096, 4096, 256, "bf16", True, kind="ar1", rows=rows)


@pytest.mark.parametrize("Nq,Nk", [(100, 333), (333, 100), (300, 130), (1, 700), (129, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_nq_ne_nk(Nq, Nk, causal):
    """Bottom-right causal alignment; Nq > Nk leaves the first rows empty."""
    run_case(1, 2, 2, Nq, Nk, 64, "bf16", causal, seed=Nq + Nk)


@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (6, 3)])
def test_gqa(H, Hkv):
    run_case(2, H, Hkv, 200, 200, 64, "bf16", True, seed=H * 10 + Hkv)
    run_case(1, H, Hkv, 150, 150, 128, "f32", False, seed=H * 10 + Hkv)


def test_non_default_scale():
    run_case(1, 2, 2, 190, 190, 64, "bf16", True, seed=3, scale=0.31)
    run_case(1, 2, 2, 190, 190, 64, "f32", False, seed=4, scale=0.02)


def test_empty_kv_and_empty_batch():
    need_gpu()
    announce("fa_fwd Nk=0 / B=0")
    q = torch.randn(1, 2, 5, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, float("nan"))
    o, lse = fa.fwd(q, k, k, causal=False, out=o)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    qe = torch.empty(0, 2, 5, 64, device="cuda", dtype=torch.bfloat16)
    oe, _ = fa.fwd(qe, qe, qe, causal=True)
    assert oe.shape == qe.shape


def test_determinism_and_poisoned_outputs():
    need_gpu()
    announce("fa_fwd determinism B=2 H=4 N=1500 bf16 causal")
    g = torch.Generator(device="cuda").manual_seed(0)
    q, k, v = (torch.randn(2, 4, 1500, 64, device="cuda", generator=g).to(torch.bfloat16)
               for _ in range(3))
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((2, 4, 1500), float("nan"), device="cuda")
    fa.fwd(q, k, v, causal=True, out=o1, lse=l1)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lse_optional_and_stream():
    need_gpu()
    announce("fa_fwd on a side stream without lse")
    cfg = dict(B=1, H=2, Hkv=2, Nq=300, Nk=300, d=64, dtype="bf16", kind="iid")
    q, k, v = fagen.make_inputs(cfg, 5)
    dq, dk, dv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.fwd(dq, dk, dv, causal=True, return_lse=False)
    s.synchronize()
    assert lse is None
    o_ref, _ = oracle.attention(widen(q, "bf16"), widen(k, "bf16"), widen(v, "bf16"), True,
                                _scale(64))
    compare(o, None, o_ref, None, "bf16", "side stream")


@pytest.mark.parametrize("causal", [True, False])
def test_large_grid_uses_256_row_tiles(causal):
    """ceil(N/256)*B*H >= 1024 selects the 256-row workgroups (32-key tiles);
    smaller grids use 128-row workgroups.  Ragged N, GQA, sampled rows that
    include the last row of every head."""
    B, H, Hkv, N = 8, 16, 4, 2000
    assert fa.kv_tile(torch.bfloat16, 64) == 32
    rows = _sampled_rows(B, H, N, 24)
    m = run_case(B, H, Hkv, N, N, 64, "bf16", causal, seed=21, rows=rows)
    assert m["max_abs"] <= 2e-2
