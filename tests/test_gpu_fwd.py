"""GPU parity of fa_fwd (prefill) against the fp64 oracle, through the C ABI.

Every output row is compared for the GPT-2-small-shaped workload, for the
256-row-workgroup kernel the trading day runs (bf16 and fp16), and for the
smaller shapes that span several tiles and ragged tails; the trading day
itself is compared on seeded sampled rows (its whole-row comparison is the
bench's parity leg).  Tolerances: tests/gpu_util.py.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_08_amd as fa
import fagen
import oracle
from gpu_util import TOL, TORCH_DT, announce, compare, need_gpu, to_dev, widen

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


def test_gpt2_small_prefill_bf16_all_rows():
    """B=4, H=12, N=2048, d=64, bf16, causal, seed 0: every row of every head
    (98,304 rows) against the oracle."""
    c = fagen.WORKLOADS["gpt2s_prefill_bf16"]
    m = run_case(c["B"], c["H"], c["Hkv"], c["Nq"], c["Nk"], c["d"], "bf16", True, scale=c["scale"])
    announce(f"  gpt2-small all rows: {m}")


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


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", [(2, 4, 2, 1500, 1500), (1, 3, 1, 640, 1000),
                                           (1, 2, 2, 1000, 640), (3, 2, 1, 64, 64),
                                           (1, 2, 1, 130, 130)])
def test_small_causal_grid_all_rows(dt, B, H, Hkv, Nq, Nk):
    """Small causal grids (fewer than 1,024 workgroups of 256 rows) run
    128-row workgroups with 64-key tiles.  Shapes give odd and even tile
    counts per workgroup, rows that see no key (Nq > Nk), GQA and ragged last
    tiles; every row of every head is compared, bf16 and fp16."""
    assert -(-Nq // 256) * B * H < 1024
    m = run_case(B, H, Hkv, Nq, Nk, 64, dt, True, seed=Nq + 3 * Nk + B + (dt == "f16"))
    announce(f"  small causal grid {dt} {B}x{H}/{Hkv} {Nq}x{Nk}: {m}")


@pytest.mark.parametrize("dt,causal", [("bf16", True), ("bf16", False), ("f16", True),
                                       ("f16", False)])
def test_large_grid_uses_256_row_tiles(dt, causal):
    """ceil(N/256)*B*H >= 1024 selects the 256-row workgroups (two 32-row
    query blocks per wave, 32-key tiles) -- the kernel instance the trading
    day runs; smaller grids use 128-row workgroups.  B=8, H=16, Hkv=4,
    N=2000 gives exactly 1,024 such workgroups with a ragged last query tile
    (2000 = 7*256 + 208) and a ragged last key tile; every row of every head
    is compared."""
    B, H, Hkv, N = 8, 16, 4, 2000
    assert -(-N // 256) * B * H == 1024
    assert fa.kv_tile(torch.bfloat16, 64) == 32
    m = run_case(B, H, Hkv, N, N, 64, dt, causal, seed=21 + int(causal) + 2 * (dt == "f16"))
    announce(f"  256-row workgroups {dt} causal={causal}: {m}")


def test_caller_outputs_are_checked():
    """Outputs passed in by the caller must match exactly (shape, dtype,
    device, contiguity); a mismatch raises before any launch and leaves the
    buffer untouched."""
    need_gpu()
    announce("fa_fwd / fa_fwd_pcast / fa_decode output checks")
    q = torch.randn(1, 2, 70, 64, device="cuda").to(torch.bfloat16)
    for kw in (dict(out=torch.empty(1, 2, 69, 64, device="cuda", dtype=torch.bfloat16)),
               dict(out=torch.empty(1, 2, 70, 64, device="cuda", dtype=torch.float16)),
               dict(lse=torch.empty(1, 2, 69, device="cuda")),
               dict(lse=torch.empty(1, 2, 70, device="cuda", dtype=torch.float16))):
        with pytest.raises(ValueError):
            fa.fwd(q, q, q, causal=True, **kw)
    x = torch.randn(1, 2, 70, 64, device="cuda")
    cnt = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd_pcast(x, x, x, counts=cnt)
    torch.cuda.synchronize()
    assert torch.all(cnt == 7)
    qd = torch.randn(2, 8, 1, 64, device="cuda").to(torch.bfloat16)
    kv = torch.randn(2, 2, 300, 64, device="cuda").to(torch.bfloat16)
    with pytest.raises(ValueError):
        fa.decode(qd, kv, kv, out=torch.empty(2, 8, 64, device="cuda", dtype=torch.bfloat16))


def _moving_max_inputs(B, H, Hkv, N, d, dt, pattern, seed):
    """Q, K, V storage arrays whose scores move far across the key axis.

    growing: q_i = 1 + noise, k_j = g(j)(1 + noise) with g(j) = 1 + j/64, so
      at d = 64 a row's scores rise by about 1 (raw) per key, 4 nats per
      32-key tile at scale 1/8: its exponentials leave any fixed
      reference's 2^64 range within about a dozen tiles (and pass the fp16
      maximum within three), while the scores stay small enough (a few
      thousand) for fp32 accumulation to keep them to about 1e-3;
    falling: the same with g reversed, so the first keys hold every row's
      maximum and later exponentials underflow;
    spike: iid keys, plus one key at N/2 aligned with every query (score
      about 768 raw against order-1 scores elsewhere).
    Values stay in the normal range of bf16 and fp16; the noise is the
    seeded normal stream."""
    nq = fagen.normal(fagen.stream_key(seed, 71), B * H * N * d).reshape(B, H, N, d)
    nk = fagen.normal(fagen.stream_key(seed, 72), B * Hkv * N * d).reshape(B, Hkv, N, d)
    nv = fagen.normal(fagen.stream_key(seed, 73), B * Hkv * N * d).reshape(B, Hkv, N, d)
    j = np.arange(N, dtype=np.float64)
    q = 1.0 + 0.25 * nq
    if pattern == "growing":
        k = (1.0 + j / 64.0)[None, None, :, None] * (1.0 + 0.25 * nk)
    elif pattern == "falling":
        k = (1.0 + (N - 1 - j) / 64.0)[None, None, :, None] * (1.0 + 0.25 * nk)
    elif pattern == "spike":
        k = 0.25 * nk
        k[:, :, N // 2, :] = 12.0
    else:
        raise ValueError(pattern)
    return (fagen.to_storage(q, dt), fagen.to_storage(k, dt), fagen.to_storage(nv, dt))


def _check_peaked(o, lse, o_ref, lse_ref, v, dt, what):
    """Peaked rows have outputs as large as the largest |v| (about 5 for
    these inputs), where the stored 16-bit output alone is off by up to
    u|O| (unit roundoff u = 2^-8 for bf16, 2^-11 for fp16), beyond the
    2e-2 absolute bound sized for averaged outputs.  The bound used here
    follows the arithmetic: P rounded to the input type before P V adds at
    most u max|v| (the weights are normalised by the unrounded sum), the
    output rounding u|O|, and 1e-3 covers the fp32 scores (about 1e-3 raw
    at a few thousand), exp2 and accumulation.  The mean-abs and LSE bounds
    are the usual ones."""
    u = 2.0 ** -8 if dt == "bf16" else 2.0 ** -11
    og = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)), what
    B, H = og.shape[:2]
    vw = np.abs(widen(v, dt)).max(axis=(2, 3))                 # [B, Hkv]
    vmax = np.repeat(vw, H // vw.shape[1], axis=1)[:, :, None, None]
    err = np.abs(og - o_ref)
    bound = u * (np.abs(o_ref) + vmax) + 1e-3
    worst = float((err / bound).max())
    assert worst <= 1.0, (what, worst, float(err.max()))
    assert float(err.mean()) <= TOL[dt]["mean_abs"], (what, float(err.mean()))
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin), what
    lse_err = float(np.abs(lg[fin] - lse_ref[fin]).max())
    assert lse_err <= TOL[dt]["lse"], (what, lse_err)
    return dict(max_abs=float(err.max()), worst_over_bound=worst, lse=lse_err)


def _reference_moves(q, k, dt, row, tile, scale):
    """How often the kernel's lazy reference max must move for one causal
    row of head 0 (a host-side restatement of its rule, to show that these
    inputs reach that path): the reference starts as the first tile's max
    and moves to a tile's max when that tile's exponentials, taken against
    it, sum to 2^64 or more.  (With fp16 inputs the kernel also moves it
    when a converted probability overflows, so this count is a lower
    bound there.)"""
    qf = widen(q, dt)[0, 0, row].astype(np.float64)
    kf = widen(k, dt)[0, 0, : row + 1].astype(np.float64)
    s = kf @ qf
    c = scale * math.log2(math.e)
    ref, moves = s[:tile].max(), 0
    for t0 in range(tile, len(s), tile):
        st = s[t0:t0 + tile]
        with np.errstate(over="ignore"):
            if np.exp2((st - ref) * c).sum() >= 2.0 ** 64:
                ref, moves = max(ref, st.max()), moves + 1
    return moves


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("pattern", ["growing", "spike"])
def test_moving_max_large_grid_all_rows(dt, pattern):
    """The 256-row instance (B=8, H=16, Hkv=4, N=2000: 1,024 workgroups of
    256 rows), causal, with scores that force the reference max to move
    during the sweep (the out-of-range rebase and its redone tile; for fp16
    also the overflow of a converted probability); every row of every
    head against the oracle, to the bound of _check_peaked."""
    need_gpu()
    B, H, Hkv, N, d = 8, 16, 4, 2000, 64
    assert -(-N // 256) * B * H == 1024
    announce(f"fa_fwd moving max ({pattern}) B={B} H={H}/{Hkv} N={N} {dt} causal")
    q, k, v = _moving_max_inputs(B, H, Hkv, N, d, dt, pattern, seed=5)
    assert fa.kv_tile(TORCH_DT[dt], d) == 32
    assert _reference_moves(q, k, dt, N - 1, 32, 0.125) >= (3 if pattern == "growing" else 1)
    o, lse = fa.fwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), causal=True, scale=0.125)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(widen(q, dt), widen(k, dt), widen(v, dt), True, 0.125)
    m = _check_peaked(o, lse, o_ref, lse_ref, v, dt, f"moving max {pattern}")
    announce(f"  {m}")


@pytest.mark.parametrize("pattern", ["growing", "falling", "spike"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_moving_max_small_shapes_all_rows(pattern, causal, d):
    """The same score patterns on the 128-row instance (d = 64), the
    32-key-tile instance (d = 128) and the split-d instance (d = 256),
    bf16, full and causal, every row, to the bound of _check_peaked."""
    need_gpu()
    B, H, Hkv, N = 1, 4, 2, 1000
    dt = "bf16"
    announce(f"fa_fwd moving max ({pattern}) B={B} H={H}/{Hkv} N={N} d={d} causal={causal}")
    q, k, v = _moving_max_inputs(B, H, Hkv, N, d, dt, pattern, seed=6 + d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.fwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(widen(q, dt), widen(k, dt), widen(v, dt), causal, scale)
    m = _check_peaked(o, lse, o_ref, lse_ref, v, dt, f"moving max {pattern} d={d}")
    announce(f"  {m}")
