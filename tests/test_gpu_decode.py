"""GPU parity of fa_decode (split-KV GQA decode + LSE merge) against the fp64
oracle (the definition with one query row and every key visible)."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_08_amd as fa
import fagen
import oracle
from gpu_util import announce, compare, need_gpu, to_dev, widen

pytestmark = pytest.mark.gpu


def run_decode(B, H, Hkv, Nk, d, dt, splits=0, seed=0, poison_ws=False):
    need_gpu()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"fa_decode B={B} H={H} Hkv={Hkv} Nk={Nk} d={d} {dt} splits={splits} seed={seed}")
    cfg = dict(B=B, H=H, Hkv=Hkv, Nq=1, Nk=Nk, d=d, dtype=dt, kind="iid")
    q, k, v = fagen.make_inputs(cfg, seed)
    ws = None
    if poison_ws:
        # every partial slot poisoned (NaN): each must be written before the merge
        ws = fa.decode_workspace(B, H, Hkv, Nk, d, splits)
        if ws is not None:
            ws.fill_(255)
    o, lse = fa.decode(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), scale=scale,
                       num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(widen(q, dt), widen(k, dt), widen(v, dt), False, scale)
    return compare(o, lse, o_ref, lse_ref, dt, "decode")


def test_tinyllama_gqa_decode_bf16():
    """B=16, 32 query heads / 4 KV heads, Nk=8192, d=64, bf16 (automatic split)."""
    assert fa.decode_splits(16, 32, 4, 8192) == 4
    run_decode(16, 32, 4, 8192, 64, "bf16")


def test_single_sequence_gqa_decode():
    """B=1, 32 query heads / 4 KV heads, 65,536 keys, d=64, bf16: B*Hkv = 4,
    so the automatic policy cuts each KV head into 64 splits and the merge
    takes its many-split path (one round of loads per 64 partials)."""
    assert fa.decode_splits(1, 32, 4, 65536) == 64
    run_decode(1, 32, 4, 65536, 64, "bf16", seed=5, poison_ws=True)


@pytest.mark.parametrize("splits", [17, 100, 257])
def test_many_split_merge(splits):
    """Split counts above 16 take the many-split merge, including more than
    one round of 64 partials (100, 257) and empty trailing splits."""
    run_decode(1, 8, 2, 30000, 64, "bf16", splits=splits, seed=splits, poison_ws=True)
    run_decode(1, 4, 1, 20000, 128, "f16", splits=splits, seed=splits + 1, poison_ws=True)


@pytest.mark.parametrize("splits", [1, 3, 16, 64])
def test_split_counts(splits):
    run_decode(2, 8, 2, 3000, 64, "bf16", splits=splits, seed=splits, poison_ws=True)


@pytest.mark.parametrize("Nk", [1, 100, 129, 1000, 8191])
def test_ragged_cache_lengths(Nk):
    run_decode(3, 8, 2, Nk, 64, "bf16", seed=Nk)


@pytest.mark.parametrize("H,Hkv", [(8, 8), (8, 1), (40, 2), (32, 1)])
def test_group_sizes(H, Hkv):
    """MHA, MQA, and groups wider than 16 heads (two query groups per KV head)."""
    run_decode(2, H, Hkv, 777, 64, "bf16", seed=H + Hkv)


@pytest.mark.parametrize("dt,d", [("f16", 64), ("bf16", 128), ("f16", 128)])
def test_dtypes_and_head_dims(dt, d):
    run_decode(4, 16, 4, 2048, d, dt, seed=d)


def test_empty_cache():
    need_gpu()
    announce("fa_decode Nk=0")
    q = torch.randn(2, 4, 1, 64, device="cuda").to(torch.bfloat16)
    kv = torch.empty(2, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = fa.decode(q, kv, kv)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_decode_equals_last_causal_prefill_row():
    need_gpu()
    announce("fa_decode vs fa_fwd last causal row, N=1500")
    cfg = dict(B=2, H=8, Hkv=2, Nq=1500, Nk=1500, d=64, dtype="bf16", kind="iid")
    q, k, v = fagen.make_inputs(cfg, 11)
    dq, dk, dv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o_full, l_full = fa.fwd(dq, dk, dv, causal=True)
    o_dec, l_dec = fa.decode(dq[:, :, -1:].contiguous(), dk, dv)
    torch.cuda.synchronize()
    diff = (o_full[:, :, -1:].float() - o_dec.float()).abs().max().item()
    assert diff <= 2e-2
    assert (l_full[:, :, -1:] - l_dec).abs().max().item() <= 1e-3


def test_determinism():
    need_gpu()
    announce("fa_decode determinism")
    g = torch.Generator(device="cuda").manual_seed(1)
    q = torch.randn(4, 16, 1, 64, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(4, 2, 5000, 64, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(4, 2, 5000, 64, device="cuda", generator=g).to(torch.bfloat16)
    o1, l1 = fa.decode(q, k, v)
    o2, l2 = fa.decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_workspace_reuse_across_shapes():
    """One workspace serves consecutive calls of different sizes and split
    counts; stale partials of an earlier call never leak into a later one."""
    need_gpu()
    cases = [(4, 16, 2, 5000, 16), (3, 40, 2, 2100, 5), (2, 8, 8, 1300, 3), (4, 16, 2, 5000, 16)]
    nb = max(fa.decode_workspace_bytes(B, H, Hkv, Nk, 64, s) for B, H, Hkv, Nk, s in cases)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    for i, (B, H, Hkv, Nk, s) in enumerate(cases):
        announce(f"fa_decode reuse B={B} H={H} Hkv={Hkv} Nk={Nk} splits={s}")
        cfg = dict(B=B, H=H, Hkv=Hkv, Nq=1, Nk=Nk, d=64, dtype="bf16", kind="iid")
        q, k, v = fagen.make_inputs(cfg, 10 + i)
        o, lse = fa.decode(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), scale=0.125,
                           num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention(widen(q, "bf16"), widen(k, "bf16"), widen(v, "bf16"),
                                          False, 0.125)
        compare(o, lse, o_ref, lse_ref, "bf16", "decode reuse")


def _paged_case(B, H, Hkv, lens, page_size, d, dt, seed, extra_pages=3):
    """Seeded contiguous K/V per sequence, scattered over randomly permuted
    pages.  Returns device tensors and the per-sequence host arrays."""
    max_len = max(max(lens), 1)
    max_pages = (max_len + page_size - 1) // page_size
    need = sum((L + page_size - 1) // page_size for L in lens)
    num_pages = need + extra_pages
    cfg = dict(B=B, H=H, Hkv=Hkv, Nq=1, Nk=max_pages * page_size, d=d, dtype=dt, kind="iid")
    q, k, v = fagen.make_inputs(cfg, seed)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_pages)
    table = np.full((B, max_pages), -7, np.int32)   # entries past a sequence stay invalid
    kp = np.zeros((num_pages, Hkv, page_size, d), k.dtype)
    vp = np.zeros_like(kp)
    nxt = 0
    for b, L in enumerate(lens):
        for pg in range((L + page_size - 1) // page_size):
            phys = int(perm[nxt]); nxt += 1
            table[b, pg] = phys
            rows = slice(pg * page_size, (pg + 1) * page_size)
            kp[phys] = k[b, :, rows]
            vp[phys] = v[b, :, rows]
    return q, k, v, kp, vp, table, max_pages, num_pages


@pytest.mark.parametrize("page_size", [32, 128, 256])
def test_paged_varlen_matches_oracle(page_size):
    need_gpu()
    B, H, Hkv, d, dt = 6, 8, 2, 64, "bf16"
    lens = [0, 1, 33, 700, 1024, 1500]
    announce(f"fa_decode_paged page_size={page_size} lens={lens}")
    q, k, v, kp, vp, table, max_pages, num_pages = _paged_case(B, H, Hkv, lens, page_size, d, dt,
                                                                 seed=page_size)
    scale = 0.125
    o, lse = fa.decode_paged(to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=scale)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        o_b = o[b:b + 1]
        if L == 0:
            assert torch.all(o_b == 0) and torch.all(torch.isneginf(lse[b]))
            continue
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], dt), widen(k[b:b + 1, :, :L], dt),
                                        widen(v[b:b + 1, :, :L], dt), False, scale)
        compare(o_b, lse[b:b + 1], o_ref, l_ref, dt, f"paged b={b} L={L}")


@pytest.mark.parametrize("splits", [1, 2, 3])
def test_paged_block_table_window_refresh(splits):
    """32-key pages and splits that span more than 64 pages: the sweep holds a
    64-entry window of the block table per wave and refreshes it as it walks;
    lengths end on, just past and well inside a window boundary."""
    need_gpu()
    B, H, Hkv, d, dt = 4, 8, 2, 64, "bf16"
    lens = [2048, 2049, 6000, 4097]
    announce(f"fa_decode_paged page_size=32 lens={lens} splits={splits}")
    q, k, v, kp, vp, table, _, _ = _paged_case(B, H, Hkv, lens, 32, d, dt, seed=31 + splits)
    o, lse = fa.decode_paged(to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=0.125,
                             num_splits=splits)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], dt), widen(k[b:b + 1, :, :L], dt),
                                        widen(v[b:b + 1, :, :L], dt), False, 0.125)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, dt, f"paged window b={b} L={L}")


@pytest.mark.parametrize("dt,d", [("f16", 64), ("bf16", 128)])
def test_paged_dtypes_and_head_dims(dt, d):
    need_gpu()
    B, H, Hkv = 3, 16, 4
    lens = [257, 64, 999]
    announce(f"fa_decode_paged {dt} d={d}")
    q, k, v, kp, vp, table, _, _ = _paged_case(B, H, Hkv, lens, 64, d, dt, seed=d + 1)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.decode_paged(to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=scale)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], dt), widen(k[b:b + 1, :, :L], dt),
                                        widen(v[b:b + 1, :, :L], dt), False, scale)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, dt, f"paged {dt} d={d} b={b}")


def test_paged_full_length_equals_contiguous_and_clamps():
    """Every sequence at the full length: the paged path reads the same keys
    in the same order as fa_decode on the contiguous cache (identical bits);
    a length above max_pages * page_size is clamped to it."""
    need_gpu()
    B, H, Hkv, d, ps = 4, 8, 2, 64, 128
    L = 1024
    announce("fa_decode_paged vs fa_decode, full length")
    q, k, v, kp, vp, table, max_pages, _ = _paged_case(B, H, Hkv, [L] * B, ps, d, "bf16", seed=4)
    dq, dk, dv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    splits = fa.decode_splits(B, H, Hkv, L)
    o1, l1 = fa.decode(dq, dk, dv, scale=0.125, num_splits=splits)
    lens = torch.tensor([L, L + 5, L, 1 << 30], dtype=torch.int32, device="cuda")
    o2, l2 = fa.decode_paged(dq, to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                             torch.from_numpy(table).cuda(), lens, scale=0.125, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B", [129, 256])
def test_paged_auto_many_sequences(B):
    """Automatic splits over more than two 64-lane blocks of sequences: the
    device-side length scan (sum and prefix sum across the blocks) must give
    every (sequence, split) pair exactly once; seeded lengths with some
    empty sequences, 64-key pages."""
    need_gpu()
    H, Hkv, d, dt, ps = 8, 2, 64, "bf16", 64
    rng = np.random.default_rng(B)
    lens = [0 if rng.random() < 0.1 else int(rng.integers(1, 400)) for _ in range(B)]
    announce(f"fa_decode_paged automatic splits, B={B}")
    q, k, v, kp, vp, table, _, _ = _paged_case(B, H, Hkv, lens, ps, d, dt, seed=B)
    o, lse = fa.decode_paged(to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=0.125)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))
            continue
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], dt), widen(k[b:b + 1, :, :L], dt),
                                        widen(v[b:b + 1, :, :L], dt), False, 0.125)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, dt, f"paged B={B} b={b} L={L}")


def test_paged_large_batch_streamed_equals_contiguous():
    """A paged batch whose K and V exceed the streaming threshold (the
    TinyLlama shape at full length: 134 MB) takes the non-temporal loads,
    chosen on the device from the lengths, and automatic splits; it must give
    the bits of fa_decode on the contiguous cache (also streamed, same
    four-split partition)."""
    need_gpu()
    B, H, Hkv, d, ps, L = 16, 32, 4, 64, 128, 8192
    assert 2 * B * Hkv * L * d * 2 >= 96 << 20
    announce("fa_decode_paged, 134 MB batch (non-temporal loads) vs fa_decode")
    q, k, v, kp, vp, table, _, _ = _paged_case(B, H, Hkv, [L] * B, ps, d, "bf16", seed=5)
    dq = to_dev(q, "bf16")
    o1, l1 = fa.decode(dq, to_dev(k, "bf16"), to_dev(v, "bf16"), scale=0.125)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o2, l2 = fa.decode_paged(dq, to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                             torch.from_numpy(table).cuda(), lens, scale=0.125)
    torch.cuda.synchronize()
    assert fa.decode_splits(B, H, Hkv, L) == 4
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_ragged_poisoned_workspace_many_splits():
    """Splits past a sequence's end write nothing and the merge must not read
    them: the whole workspace starts as NaN, lengths are ragged (one empty),
    eight splits are forced."""
    need_gpu()
    B, H, Hkv, d, ps = 4, 8, 2, 64, 64
    lens = [0, 1, 200, 1500]
    announce(f"fa_decode_paged poisoned workspace, 8 splits, lens={lens}")
    q, k, v, kp, vp, table, max_pages, _ = _paged_case(B, H, Hkv, lens, ps, d, "bf16", seed=8)
    ws = fa.decode_workspace(B, H, Hkv, max_pages * ps, d, 8)
    ws.fill_(255)
    o, lse = fa.decode_paged(to_dev(q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=0.125,
                             num_splits=8, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    for b in range(1, B):
        L = lens[b]
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], "bf16"), widen(k[b:b + 1, :, :L], "bf16"),
                                        widen(v[b:b + 1, :, :L], "bf16"), False, 0.125)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, "bf16", f"paged poisoned b={b}")


def test_paged_auto_full_length_equals_forced_splits():
    """Automatic splits at full length: 4 sequences of 2,048 keys, 2 KV
    heads -> a chunk of 512 keys, i.e. the partition of 4 forced splits, so
    the bits are the same (only the workgroup order differs)."""
    need_gpu()
    B, H, Hkv, d, ps, L = 4, 8, 2, 64, 64, 2048
    announce("fa_decode_paged automatic vs 4 forced splits, full length")
    q, k, v, kp, vp, table, max_pages, _ = _paged_case(B, H, Hkv, [L] * B, ps, d, "bf16", seed=11)
    args = (to_dev(q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"), torch.from_numpy(table).cuda(),
            torch.full((B,), L, dtype=torch.int32, device="cuda"))
    o1, l1 = fa.decode_paged(*args, scale=0.125, num_splits=4)
    o2, l2 = fa.decode_paged(*args, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
def test_paged_auto_skewed_lengths_poisoned_workspace(d):
    """Automatic splits on a skewed batch of 70 sequences (more than one
    64-lane block of the device-side scan): one long sequence, the rest
    empty or a few keys; the workspace starts as NaN."""
    need_gpu()
    B, H, Hkv, ps, dt = 70, 4, 2, 32, "f16" if d == 128 else "bf16"
    rng = np.random.default_rng(d)
    lens = [int(x) for x in rng.choice([0, 1, 5, 31, 40], B)]
    lens[37] = 3000
    announce(f"fa_decode_paged automatic, skewed lengths, B={B} d={d}")
    q, k, v, kp, vp, table, max_pages, _ = _paged_case(B, H, Hkv, lens, ps, d, dt, seed=d + 3)
    ws = fa.decode_paged_workspace(B, H, Hkv, max_pages, ps, d)
    ws.fill_(255)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.decode_paged(to_dev(q, dt), to_dev(kp, dt), to_dev(vp, dt),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=scale,
                             workspace=ws)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b])), b
            continue
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], dt), widen(k[b:b + 1, :, :L], dt),
                                        widen(v[b:b + 1, :, :L], dt), False, scale)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, dt, f"paged auto b={b} L={L}")


def test_paged_auto_all_empty():
    need_gpu()
    B, H, Hkv, d, ps = 5, 8, 2, 64, 128
    announce("fa_decode_paged automatic, every sequence empty")
    q, k, v, kp, vp, table, max_pages, _ = _paged_case(B, H, Hkv, [0] * B, ps, d, "bf16", seed=2,
                                                        extra_pages=2)
    o, lse = fa.decode_paged(to_dev(q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                             torch.from_numpy(table).cuda(),
                             torch.zeros(B, dtype=torch.int32, device="cuda"), scale=0.125)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_paged_large_batch_uses_uniform_split():
    """Past 256 sequences the automatic mode takes the uniform split; 260
    short ragged sequences (some empty) against the oracle."""
    need_gpu()
    B, H, Hkv, d, ps = 260, 4, 1, 64, 32
    rng = np.random.default_rng(260)
    lens = [int(x) for x in rng.integers(0, 90, B)]
    announce(f"fa_decode_paged B={B}, automatic mode past 256 sequences")
    q, k, v, kp, vp, table, max_pages, _ = _paged_case(B, H, Hkv, lens, ps, d, "bf16", seed=260)
    o, lse = fa.decode_paged(to_dev(q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                             torch.from_numpy(table).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=0.125)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b])), b
            continue
        o_ref, l_ref = oracle.attention(widen(q[b:b + 1], "bf16"), widen(k[b:b + 1, :, :L], "bf16"),
                                        widen(v[b:b + 1, :, :L], "bf16"), False, 0.125)
        compare(o[b:b + 1], lse[b:b + 1], o_ref, l_ref, "bf16", f"paged B=260 b={b} L={L}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 0])
@pytest.mark.parametrize("pattern", ["growing", "falling"])
def test_moving_max_every_step(pattern, splits, d):
    """Scores that rise (or fall) steadily along the cache: with growing
    keys every 128-key step raises each row's running max, so the rescale
    of the accumulator runs at every step; with falling keys the first step
    holds the max and later exponentials underflow.  One split (one
    workgroup sweeps the whole cache) and the automatic split.  Outputs of
    peaked rows are as large as the largest |v|, so the check is the
    arithmetic bound u(|O| + max|v|) + 1e-3 (u = 2^-8 for bf16: P and O
    rounded to bf16), and LSE within 1e-3."""
    need_gpu()
    B, H, Hkv, Nk, dt = 2, 16, 4, 3000, "bf16"
    announce(f"fa_decode moving max ({pattern}) B={B} H={H}/{Hkv} Nk={Nk} d={d} splits={splits}")
    nq = fagen.normal(fagen.stream_key(11, 81), B * H * d).reshape(B, H, 1, d)
    nk = fagen.normal(fagen.stream_key(11, 82), B * Hkv * Nk * d).reshape(B, Hkv, Nk, d)
    nv = fagen.normal(fagen.stream_key(11, 83), B * Hkv * Nk * d).reshape(B, Hkv, Nk, d)
    j = np.arange(Nk, dtype=np.float64)
    g = 1.0 + (j if pattern == "growing" else Nk - 1 - j) / 128.0
    q = fagen.to_storage(1.0 + 0.25 * nq, dt)
    k = fagen.to_storage(g[None, None, :, None] * (1.0 + 0.25 * nk), dt)
    v = fagen.to_storage(nv, dt)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.decode(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(widen(q, dt), widen(k, dt), widen(v, dt), False, scale)
    # peaked rows: the bound of the prefill's peaked-row test (u = 2^-8)
    og = o.float().cpu().numpy().astype(np.float64)
    vmax = np.repeat(np.abs(widen(v, dt)).max(axis=(2, 3)), H // Hkv, axis=1)[:, :, None, None]
    err = np.abs(og - o_ref)
    assert np.all(err <= 2.0 ** -8 * (np.abs(o_ref) + vmax) + 1e-3), float(err.max())
    lg = lse.cpu().numpy().astype(np.float64)
    assert float(np.abs(lg - lse_ref).max()) <= 1e-3
