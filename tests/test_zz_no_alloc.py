"""GPU test of fa_decode_noalloc (decode with the split partials in the
library's static device scratch) against fa_decode (partials in a caller
workspace), through the C ABI.

Two calls in a row -- the TinyLlama-shaped decode, then a smaller one with a
different split count -- each compared bit for bit with fa_decode on the
same inputs and against the fp64 oracle at the bf16/fp16 bars; the second
call reuses the scratch the first one left behind.  A fp16, d = 128 call
follows, then an oversized one that must be refused with FA_ERR_SCRATCH
before anything is launched.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_08_amd as fa
import fagen
import oracle
from gpu_util import announce, compare, need_gpu, to_dev, widen

pytestmark = pytest.mark.gpu


def _run(B, H, Hkv, Nk, d, dt, seed, splits):
    announce(f"fa_decode_noalloc vs fa_decode B={B} H={H} Hkv={Hkv} Nk={Nk} d={d} {dt} "
             f"splits={splits} seed={seed}")
    cfg = dict(B=B, H=H, Hkv=Hkv, Nq=1, Nk=Nk, d=d, dtype=dt, kind="iid")
    q, k, v = fagen.make_inputs(cfg, seed)
    dq, dk, dv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o_ws, l_ws = fa.decode(dq, dk, dv, scale=scale, num_splits=splits)
    o_na = torch.full_like(dq, float("nan"))
    l_na = torch.full((B, H, 1), float("nan"), device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa.decode_noalloc(dq, dk, dv, scale=scale, num_splits=splits, out=o_na, lse=l_na)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before   # nothing allocated through torch
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
    o_ref, l_ref = oracle.attention(widen(q, dt), widen(k, dt), widen(v, dt), False, scale)
    return compare(o_na, l_na, o_ref, l_ref, dt, "decode_noalloc")


def test_noalloc_decode_two_calls_then_limit():
    need_gpu()
    c = fagen.WORKLOADS["gqa_decode_bf16"]
    assert fa.decode_splits(c["B"], c["H"], c["Hkv"], c["Nk"]) == 4
    # 1: the TinyLlama-shaped decode (4 splits, 0.53 MB of partials)
    _run(c["B"], c["H"], c["Hkv"], c["Nk"], c["d"], "bf16", 0, 0)
    # 2: smaller, three splits, a ragged cache and two query-head groups per KV head
    _run(2, 40, 2, 1000, 64, "bf16", 1, 3)
    # 3: fp16, d = 128
    _run(3, 16, 4, 2100, 128, "f16", 2, 0)
    # refused above the scratch size, nothing launched: 4,096 forced splits of
    # 8 heads at d = 128 need 16.9 MB of partials
    B, H, Hkv, Nk, d, splits = 1, 8, 8, 64, 128, 4096
    assert fa.decode_workspace_bytes(B, H, Hkv, Nk, d, splits) > 8 << 20
    q = torch.zeros(B, H, 1, d, device="cuda", dtype=torch.bfloat16)
    kv = torch.zeros(B, Hkv, Nk, d, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 7.0)
    with pytest.raises(fa.FaError) as e:
        fa.decode_noalloc(q, kv, kv, num_splits=splits, out=o)
    assert e.value.status == 12
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
