"""GPU parity of fa_bwd (attention backward by recomputation) against the
fp64 oracle gradient, through the C ABI.

Tolerance, derived from the arithmetic of the kernels (bf16/fp16 inputs,
fp32 scores, dP and accumulators).  Every gradient element is a sum of terms
(scale dS_ij k_j, scale dS_ij q_i, P_ij dO_i).  P and dS are rounded to the
input type as MFMA operands (relative 2^-9 each), and the fp32 sums add at
most N 2^-24 <= 2^-9 for N <= 32K.  The bound therefore allows 2^-6 times the
sum of |terms| (the oracle returns it).

D_i = dO_i . O_i is formed from the O the kernel is given, not from the
exact O.  Its error dD_i <= sum_c |dO_ic| |O_ic - O_exact,ic| + 2^-12
sum_c |dO_ic O_ic| enters as P_ij dD_i, which adds:
  * to dQ_ic: scale dD_i sum_j P_ij |k_jc|, the forward oracle with V := |K|;
  * to dK_jc: scale sum_i P_ij dD_i |q_ic|, the oracle's dV for dO := dD |Q|.
The final rounding of the gradient to the input type adds 2^-9 |g|.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_08_amd as fa
import fagen
import oracle
from gpu_util import announce, need_gpu, to_dev, widen

pytestmark = pytest.mark.gpu


def _dout(B, H, N, d, dt, seed):
    x = fagen.normal(fagen.stream_key(seed, 9, 0), B * H * N * d).reshape(B, H, N, d)
    return fagen.to_storage(x, dt)


def _bounds(q, k, v, dout, o_given, o_exact, causal, scale, ad, ref):
    """Elementwise error bounds for (dq, dk, dv); all arrays float64."""
    adq, adk, adv = ad
    dq, dk, dv = ref
    dd = (np.abs(dout) * np.abs(o_given - o_exact)).sum(-1) \
        + 2.0 ** -12 * (np.abs(dout) * np.abs(o_given)).sum(-1)          # [B,H,Nq]
    pk = oracle.attention(q, k, np.abs(k).astype(np.float32), causal, scale)[0]  # sum_j P_ij |k_jc|
    bq = 2.0 ** -6 * adq + scale * dd[..., None] * pk * (1 + 1e-6) \
        + 2.0 ** -9 * np.abs(dq) + 1e-6
    wq = (dd[..., None] * np.abs(q)).astype(np.float32)
    pq = oracle.attention_bwd(q, k, v, wq, causal, scale)[2]              # sum_i P_ij dD_i |q_ic|
    bk = 2.0 ** -6 * adk + scale * pq * (1 + 1e-6) + 2.0 ** -9 * np.abs(dk) + 1e-6
    bv = 2.0 ** -6 * adv + 2.0 ** -9 * np.abs(dv) + 1e-6
    return bq, bk, bv


def run_bwd(B, H, Hkv, Nq, Nk, d, dt, causal, seed=0, gpu_forward=False, inputs=None):
    need_gpu()
    announce(f"fa_bwd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} causal={causal} "
             f"seed={seed} gpu_forward={gpu_forward}" + (" (given inputs)" if inputs else ""))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    cfg = dict(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dt, kind="iid")
    qs, ks, vs = fagen.make_inputs(cfg, seed) if inputs is None else inputs
    gs = _dout(B, H, Nq, d, dt, seed)
    q, k, v, gout = (widen(x, dt) for x in (qs, ks, vs, gs))
    o_ex, lse_ex = oracle.attention(q, k, v, causal, scale)
    dq_d, dk_d, dv_d = to_dev(qs, dt), to_dev(ks, dt), to_dev(vs, dt)
    if gpu_forward:
        o_t, lse_t = fa.fwd(dq_d, dk_d, dv_d, causal=causal, scale=scale)
    else:
        o_t = to_dev(fagen.to_storage(o_ex, dt), dt)
        lse_t = torch.from_numpy(lse_ex.astype(np.float32)).cuda()
    grads = fa.bwd(dq_d, dk_d, dv_d, o_t, to_dev(gs, dt), lse_t, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_given = o_t.float().cpu().numpy().astype(np.float64)
    ref = oracle.attention_bwd(q, k, v, gout, causal, scale, abs_sums=True)
    bounds = _bounds(q, k, v, gout, o_given, o_ex, causal, scale, ref[3:], ref[:3])
    worst = {}
    for name, gt, r, bnd in zip(("dq", "dk", "dv"), grads, ref[:3], bounds):
        got = gt.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), f"{name}: non-finite"
        err = np.abs(got - r)
        ratio = err / bnd
        i = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
        assert np.all(err <= bnd), (name, i, float(got[i]), float(r[i]), float(bnd[i]))
        worst[name] = float(ratio.max()) if ratio.size else 0.0
        # the bound must stay a real constraint: well below the gradient's size
        if r.size and np.abs(r).max() > 1e-3:
            assert np.median(bnd) < 0.05 * np.abs(r).max(), (name, np.median(bnd), np.abs(r).max())
    announce("  worst err/bound: " + ", ".join(f"{k} {x:.3f}" for k, x in worst.items()))
    return worst


@pytest.mark.parametrize("N", [1, 65, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths_bf16(N, causal):
    run_bwd(2, 4, 2, N, N, 64, "bf16", causal, seed=N)


@pytest.mark.parametrize("Nq,Nk", [(100, 333), (333, 100), (1, 257)])
@pytest.mark.parametrize("causal", [False, True])
def test_nq_ne_nk(Nq, Nk, causal):
    run_bwd(2, 4, 2, Nq, Nk, 64, "bf16", causal, seed=Nq + Nk)


@pytest.mark.parametrize("H,Hkv", [(8, 8), (8, 1), (6, 3)])
def test_gqa(H, Hkv):
    run_bwd(2, H, Hkv, 200, 200, 64, "bf16", True, seed=H * 10 + Hkv)


@pytest.mark.parametrize("dt,d", [("f16", 64), ("bf16", 128), ("f16", 128)])
def test_dtypes_and_head_dims(dt, d):
    run_bwd(2, 4, 2, 250, 250, d, dt, True, seed=d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv,N", [(2, 2, 129), (3, 1, 161), (6, 2, 97)])
def test_pipeline_iteration_counts(d, H, Hkv, N):
    """The dK/dV sweep is software-pipelined over (query head, query tile)
    iterations: odd and even counts, a single iteration (causal N = 129 with
    one query head per KV head: the last key block sees one query tile) and
    GQA groups of 1, 2 and 3, causal and full."""
    run_bwd(1, H, Hkv, N, N, d, "bf16", True, seed=N + d)
    run_bwd(1, H, Hkv, N, N, d, "f16", False, seed=N + d + 1)


def test_gpt2_shape_heads_causal():
    """GPT-2-small-shaped heads (d = 64) at N = 2048, causal, bf16."""
    run_bwd(2, 4, 2, 2048, 2048, 64, "bf16", True, seed=5)


def test_end_to_end_with_gpu_forward():
    """O and LSE from fa_fwd itself; the bound accounts for the forward's error in O."""
    run_bwd(2, 4, 2, 700, 700, 64, "bf16", True, seed=7, gpu_forward=True)


def test_empty_sides():
    need_gpu()
    announce("fa_bwd empty sides")
    q = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    kv0 = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.full((1, 2, 5), float("-inf"), device="cuda")
    dq, dk, dv = fa.bwd(q, kv0, kv0, o, torch.randn_like(q), lse, causal=False)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
    # no queries: dK = dV = 0
    q0 = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(1, 2, 7, 64, device="cuda").to(torch.bfloat16)
    dq, dk, dv = fa.bwd(q0, k, k, q0, q0, torch.empty(1, 2, 0, device="cuda"), causal=True)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_determinism():
    need_gpu()
    announce("fa_bwd determinism")
    g = torch.Generator(device="cuda").manual_seed(3)
    q = torch.randn(2, 8, 600, 64, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(2, 2, 600, 64, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(2, 2, 600, 64, device="cuda", generator=g).to(torch.bfloat16)
    o, lse = fa.fwd(q, k, v, causal=True)
    do = torch.randn(2, 8, 600, 64, device="cuda", generator=g).to(torch.bfloat16)
    a = fa.bwd(q, k, v, o, do, lse, causal=True)
    b = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _growing_keys(B, H, Hkv, N, d, dt, seed):
    """q_i = 1 + noise, k_j = (1 + j/64)(1 + noise), v iid (storage arrays):
    scores rise along the key axis, so each row's softmax is peaked on its
    last visible keys and the recomputed P spans many orders of magnitude."""
    nq = fagen.normal(fagen.stream_key(seed, 61), B * H * N * d).reshape(B, H, N, d)
    nk = fagen.normal(fagen.stream_key(seed, 62), B * Hkv * N * d).reshape(B, Hkv, N, d)
    nv = fagen.normal(fagen.stream_key(seed, 63), B * Hkv * N * d).reshape(B, Hkv, N, d)
    g = 1.0 + np.arange(N, dtype=np.float64) / 64.0
    return (fagen.to_storage(1.0 + 0.25 * nq, dt),
            fagen.to_storage(g[None, None, :, None] * (1.0 + 0.25 * nk), dt),
            fagen.to_storage(nv, dt))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_growing_scores(causal, d):
    """Peaked rows (scores rising along the key axis) through the same
    bound as the other cases."""
    B, H, Hkv, N = 1, 4, 2, 600
    run_bwd(B, H, Hkv, N, N, d, "bf16", causal, seed=d,
            inputs=_growing_keys(B, H, Hkv, N, d, "bf16", seed=d))
