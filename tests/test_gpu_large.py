"""Slices of more than 2 GiB, against the fp64 oracle through the C ABI.

A KV slice of 2^24 + 1,000 bf16 keys at d = 64 (2.15 GB per tensor) goes
through a single-split decode (one workgroup streams the whole slice), and
2^24 + 100 keys stand behind 64 prefill queries (full attention).  The byte
ranges of the buffer descriptors passed to the kernels exceed the 31-bit
range there, so these cases check that they are formed without overflow.
Inputs are seeded normals drawn on the device; the oracle sees the exact
bf16 values, widened.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_08_amd as fa
import oracle
from gpu_util import announce, compare, need_gpu

pytestmark = pytest.mark.gpu


def _randn(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)


def _host(x):
    return x.float().cpu().numpy()


def test_decode_single_split_over_2gib_slice():
    need_gpu()
    B, H, Hkv, Nk, d = 1, 8, 1, (1 << 24) + 1000, 64
    announce(f"fa_decode B={B} H={H} Hkv={Hkv} Nk={Nk} d={d} bf16 splits=1 (2.15 GB per tensor)")
    q, k, v = _randn((B, H, 1, d), 1), _randn((B, Hkv, Nk, d), 2), _randn((B, Hkv, Nk, d), 3)
    assert k.numel() * k.element_size() > (1 << 31)
    o, lse = fa.decode(q, k, v, scale=0.125, num_splits=1,
                       workspace=fa.decode_workspace(B, H, Hkv, Nk, d, 1))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(_host(q), _host(k), _host(v), False, 0.125)
    compare(o, lse, o_ref, lse_ref, "bf16", "decode over a >2 GiB slice")


def test_prefill_over_2gib_key_slice_sampled():
    need_gpu()
    B, H, Hkv, Nq, Nk, d = 1, 2, 1, 64, (1 << 24) + 100, 64
    announce(f"fa_fwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} bf16 full (2.15 GB per tensor)")
    q, k, v = _randn((B, H, Nq, d), 4), _randn((B, Hkv, Nk, d), 5), _randn((B, Hkv, Nk, d), 6)
    o, lse = fa.fwd(q, k, v, causal=False, scale=0.125)
    torch.cuda.synchronize()
    rows = np.array([0, 17, 40, 63])
    o_ref, lse_ref = oracle.attention(_host(q), _host(k), _host(v), False, 0.125, rows=rows)
    compare(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, "bf16", "prefill over a >2 GiB key slice")
