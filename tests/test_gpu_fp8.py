"""GPU checks of the FP8 path: fa_quant_e4m3 and fa_fwd_fp8, through the C ABI.

* Quantisation (codes and scales) equals the oracle bit for bit: the random-
  sign Hadamard rotation, the group maxima and the E4M3 rounding are all
  integer decisions taken in fp32 on both sides in the same order.
* The FP8 forward matches the oracle's step-by-step P-cast emulation
  (oracle.pcast_emulate) run on the dequantised operands with the kernel's
  KV tile: scores, running max and P in fp32 on the GPU against fp64 in the
  emulation.  The FP8 matrix cores sum their products with less than fp32
  accuracy (measured, see EPS_MMA), so scores differ by up to EPS_MMA times
  the sum of |products|; the LSE must stay within that bound, every output
  element within twice the P-cast error bound around exact attention on the
  same dequantised operands plus the accumulation error, and the MSE against
  exact attention within 5% of the emulation's.
* The incoherent-processing claim (marketmaker.cc blog, "FA3: Mecanica de la
  tolva", item 3): on inputs with rare large coordinates the rotation lowers
  the error against exact attention well below that of naive (per-tensor,
  unrotated) quantisation.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_08_amd as fa
import fagen
import oracle
from gpu_util import announce, need_gpu, to_dev, widen
from oracle import pcast_bound

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("dt,d,layout,whole,rot", [
    ("bf16", 64, "rows32", False, True), ("bf16", 64, "rows32", False, False),
    ("bf16", 128, "rows32", False, True), ("f16", 64, "rows32", False, True),
    ("f32", 128, "rows32", False, False), ("f32", 64, "rows32", False, True),
    ("bf16", 64, "channels", False, False), ("f16", 128, "channels", False, True),
    ("bf16", 64, "rows32", True, False), ("f32", 64, "channels", True, True),
    ("bf16", 128, "channels", True, False),
])
def test_quant_matches_oracle(dt, d, layout, whole, rot):
    need_gpu()
    B, H, N = 2, 3, 1000
    announce(f"fa_quant_e4m3 {dt} d={d} layout={layout} whole={whole} rot={rot} N={N}")
    xf = widen(fagen.outlier_normal(d + N, 1, (B, H, N, d), dt, 1e-2, 30.0), dt)
    xf[0, 1, 40:72] *= np.float32(1e-30)   # a near-zero block
    xf[1, 2, :, 3] = 0                     # an all-zero column
    x = fagen.to_storage(xf.astype(np.float64), dt)
    sg = fagen.random_signs(7, d) if rot else None
    codes, scales = fa.quant_e4m3(to_dev(x, dt), None if sg is None else _f32(sg), layout, whole)
    torch.cuda.synchronize()
    rc, rs = oracle.quant_e4m3(widen(x, dt), sg, layout, whole)
    got_c = codes.cpu().numpy()
    bad = np.argwhere(got_c != rc)
    assert bad.size == 0, (len(bad), bad[:5].tolist())
    assert np.array_equal(scales.cpu().numpy(), rs)


def test_quant_ragged_and_tiny_rows():
    need_gpu()
    for N in (1, 31, 33, 65):
        announce(f"fa_quant_e4m3 N={N}")
        x = fagen.outlier_normal(N, 2, (1, 2, N, 64), "bf16")
        codes, scales = fa.quant_e4m3(to_dev(x, "bf16"))
        torch.cuda.synchronize()
        rc, rs = oracle.quant_e4m3(widen(x, "bf16"))
        assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


def _operands(B, H, Hkv, Nq, Nk, d, seed, rot, whole=False, frac=1e-3, mag=10.0):
    """bf16 inputs with outliers, quantised by the oracle (codes, scales, dequantised values)."""
    q = widen(fagen.outlier_normal(seed, 1, (B, H, Nq, d), "bf16", frac, mag), "bf16")
    k = widen(fagen.outlier_normal(seed, 2, (B, Hkv, Nk, d), "bf16", frac, mag), "bf16")
    v = widen(fagen.outlier_normal(seed, 3, (B, Hkv, Nk, d), "bf16", frac, mag), "bf16")
    sg = fagen.random_signs(seed, d) if rot else None
    qc, qs = oracle.quant_e4m3(q, sg, "rows32", whole)
    kc, ks = oracle.quant_e4m3(k, sg, "rows32", whole)
    vc, vs = oracle.quant_e4m3(v, None, "channels", whole)
    deq = (oracle.dequant_e4m3(qc, qs), oracle.dequant_e4m3(kc, ks),
           oracle.dequant_e4m3(vc, vs, "channels"))
    scale = np.float32(1.0 / math.sqrt(d))
    sc = float(np.float32(scale / d)) if rot else float(scale)
    return (q, k, v), (qc, qs, kc, ks, vc, vs), deq, sc


def _gpu_fp8(codes, causal, sc, S, rev, out_dtype=torch.float32):
    qc, qs, kc, ks, vc, vs = codes
    o, lse = fa.fwd_fp8(_u8(qc), _u8(kc), _u8(vc), _f32(qs), _f32(ks), _f32(vs), causal=causal,
                        scale=sc, p_scale=S, kv_reverse=rev, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse


# The gfx950 FP8 MFMA does not return the fp32-rounded exact sum of its 64
# products: an in-bounds probe over 786,432 outputs of random finite E4M3
# operands found |error| <= 2^-11.3 * sum|a_i b_i| (mean 2^-15.4).  The bound
# below uses EPS_MMA = 2^-10.
EPS_MMA = 2.0 ** -10


def _score_err(qh, kh, causal, sc, b, h, rows):
    """Per row: EPS_MMA * scale * max over visible keys of sum_i |q_i k_ji|, a bound
    on every score's deviation and so on the LSE's (softmax is 1-Lipschitz)."""
    G = qh.shape[1] // kh.shape[1]
    Nq, Nk = qh.shape[2], kh.shape[2]
    rows = np.asarray(rows)
    m = np.abs(qh[b, h, rows].astype(np.float64)) @ np.abs(kh[b, h // G].astype(np.float64)).T
    if causal:
        m = np.where(np.arange(Nk)[None, :] <= rows[:, None] + (Nk - Nq), m, 0.0)
    return EPS_MMA * sc * (m.max(axis=1) if Nk else np.zeros(len(rows)))


def _check_vs_emulation(o, lse, deq, causal, sc, S, rev, what, rows=None, bound_heads=()):
    """Kernel vs the oracle's P-cast emulation on the dequantised operands:
    LSE within the score-error bound; on bound_heads every element within twice
    the P-cast bound around exact attention plus the matrix cores' accumulation
    error, (2 ds + 2 EPS_MMA) sum_j a_j |v_j|; the MSE against exact attention
    within 5% of the emulation's."""
    qh, kh, vh = deq
    B, H, Nq = o.shape[:3]
    G = H // kh.shape[1]
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    rr = np.tile(np.arange(Nq), (H, 1)) if rows is None else np.asarray(rows)
    og = np.stack([og[:, h, rr[h]] for h in range(H)], axis=1)
    lg = np.stack([lg[:, h, rr[h]] for h in range(H)], axis=1)
    ridx = np.tile(rr, (B, 1))
    oe, le, _ = oracle.pcast_emulate(qh, kh, vh, causal, sc, fa.fp8_kv_tile(), S, rev, rows=ridx)
    ox, _ = oracle.attention(qh, kh, vh, causal, sc, rows=ridx)
    assert np.all(np.isfinite(og)), what
    fin = np.isfinite(le)
    assert np.array_equal(np.isfinite(lg), fin), what
    for b in range(B):
        for h in range(H):
            ds = _score_err(qh, kh, causal, sc, b, h, rr[h])
            f = fin[b, h]
            dl = np.abs(lg[b, h][f] - le[b, h][f])
            assert np.all(dl <= ds[f] + 2e-6 * (1 + np.abs(le[b, h][f]))), (what, b, h, dl.max(), ds[f].max())
            if h in bound_heads:
                a = np.stack([oracle.attention_probs(qh, kh, causal, sc, b, h, int(i)) for i in rr[h]])
                av = a @ np.abs(vh[b, h // G].astype(np.float64))
                bnd = 2 * pcast_bound(a, vh[b, h // G], S) + (2 * ds[:, None] + 2 * EPS_MMA) * av
                assert np.all(np.abs(og[b, h] - oe[b, h]) <= bnd), (what, b, h)
    mse_g = np.mean((og - ox) ** 2)
    mse_e = np.mean((oe - ox) ** 2)
    assert abs(mse_g - mse_e) <= 0.05 * mse_e + 1e-12, (what, mse_g, mse_e)
    return og, oe


@pytest.mark.parametrize("d,causal,Nq,Nk,S,rev,rot", [
    (64, True, 300, 300, 256.0, False, True),
    (64, True, 300, 300, 1.0, False, False),
    (64, False, 257, 130, 256.0, True, True),
    (64, True, 100, 333, 256.0, True, False),
    (64, True, 333, 100, 128.0, False, True),
    (128, True, 300, 300, 256.0, False, True),
    (128, False, 65, 1000, 256.0, True, False),
    (128, True, 1, 70, 256.0, False, True),
])
def test_fp8_matches_emulation(d, causal, Nq, Nk, S, rev, rot):
    need_gpu()
    B, H, Hkv = 2, 4, 2
    announce(f"fa_fwd_fp8 d={d} causal={causal} Nq={Nq} Nk={Nk} S={S} rev={rev} rot={rot}")
    _, codes, deq, sc = _operands(B, H, Hkv, Nq, Nk, d, Nq + Nk + d, rot)
    o, lse = _gpu_fp8(codes, causal, sc, S, rev)
    _check_vs_emulation(o, lse, deq, causal, sc, S, rev, "fp8", bound_heads=(0, 3))


def test_bf16_output_is_rounded_fp32_output():
    need_gpu()
    announce("fa_fwd_fp8 bf16 vs fp32 output")
    _, codes, _, sc = _operands(1, 4, 4, 500, 500, 64, 5, True)
    o32, l32 = _gpu_fp8(codes, True, sc, 256.0, False, torch.float32)
    o16, l16 = _gpu_fp8(codes, True, sc, 256.0, False, torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(l16, l32)


def test_fp8_edge_cases():
    need_gpu()
    announce("fa_fwd_fp8 edge cases")
    # no keys at all
    q = torch.zeros(1, 2, 5, 64, dtype=torch.uint8, device="cuda")
    kv = torch.zeros(1, 2, 0, 64, dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd_fp8(q, kv, kv, torch.ones(1, 2, 1, device="cuda"), torch.ones(1, 2, 0, device="cuda"),
                        torch.ones(1, 2, 64, device="cuda"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # causal with Nq > Nk: the first Nq - Nk rows see nothing
    _, codes, deq, sc = _operands(1, 2, 1, 90, 20, 64, 9, False)
    o, lse = _gpu_fp8(codes, True, sc, 256.0, False)
    _check_vs_emulation(o, lse, deq, True, sc, 256.0, False, "Nq>Nk")
    assert torch.all(o[:, :, :70] == 0) and torch.all(torch.isneginf(lse[:, :, :70]))


def test_fp8_trading_day_shape_sampled_rows():
    """B=1, H=12, N=23,400, d=64, causal, rotated operands; sampled rows of
    every head against the emulation, codes of the GPU quantiser against the
    oracle's on the whole tensors."""
    need_gpu()
    c = fagen.WORKLOADS["trading_day_prefill_bf16"]
    B, H, N, d = c["B"], c["H"], c["Nq"], c["d"]
    announce(f"fa_fwd_fp8 trading-day shape B={B} H={H} N={N}")
    q, k, v = (widen(x, "bf16") for x in fagen.make_inputs(c, 0))
    sg = fagen.random_signs(0, d)
    qd, kd, vd = (to_dev(fagen.to_storage(x, "bf16"), "bf16") for x in (q, k, v))
    sgd = _f32(sg)
    gq, gqs = fa.quant_e4m3(qd, sgd)
    gk, gks = fa.quant_e4m3(kd, sgd)
    gv, gvs = fa.quant_e4m3(vd, None, "channels")
    torch.cuda.synchronize()
    qc, qs = oracle.quant_e4m3(q, sg)
    kc, ks = oracle.quant_e4m3(k, sg)
    vc, vs = oracle.quant_e4m3(v, None, "channels")
    for g_, r_ in ((gq, qc), (gqs, qs), (gk, kc), (gks, ks), (gv, vc), (gvs, vs)):
        assert np.array_equal(g_.cpu().numpy(), r_)
    sc = float(np.float32(np.float32(1 / math.sqrt(d)) / d))
    o, lse = fa.fwd_fp8(gq, gk, gv, gqs, gks, gvs, causal=True, scale=sc, p_scale=256.0,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.stack([np.unique(np.concatenate([[0, 1, 63, 64, N - 1], fagen.sample_rows(1, h, N, 10)]))
                     for h in range(H)])
    deq = (oracle.dequant_e4m3(qc, qs), oracle.dequant_e4m3(kc, ks), oracle.dequant_e4m3(vc, vs, "channels"))
    _check_vs_emulation(o, lse, deq, True, sc, 256.0, False, "trading day", rows=rows)


def _rmse_vs_exact(B, H, N, d, frac, mag, seed=3):
    (q, k, v), _, _, _ = _operands(B, H, H, N, N, d, seed, False, frac=frac, mag=mag)
    scale = float(np.float32(1 / math.sqrt(d)))
    o_ex, _ = oracle.attention(q, k, v, True, scale)
    out = {}
    for name, (rot, whole) in (("naive", (False, True)), ("rotated", (True, False))):
        _, codes, deq, sc = _operands(B, H, H, N, N, d, seed, rot, whole=whole, frac=frac, mag=mag)
        o, lse = _gpu_fp8(codes, True, sc, 256.0, False)
        og, _ = _check_vs_emulation(o, lse, deq, True, sc, 256.0, False, name)
        out[name] = float(np.sqrt(np.mean((og - o_ex) ** 2)))
    announce(f"  fp8 RMSE vs exact (frac={frac}, mag={mag}): {out}")
    return out


def test_incoherent_processing_lowers_error():
    need_gpu()
    announce("fa_fwd_fp8 incoherent processing error study")
    e = _rmse_vs_exact(1, 4, 1024, 64, 1e-3, 10.0)
    assert e["naive"] > 1.3 * e["rotated"], e
    e = _rmse_vs_exact(1, 4, 1024, 64, 1e-2, 10.0)
    assert e["naive"] > 1.5 * e["rotated"], e
    # without outliers the rotation neither helps nor hurts much
    e = _rmse_vs_exact(1, 4, 1024, 64, 0.0, 1.0)
    assert 0.9 < e["naive"] / e["rotated"] < 1.1, e


@pytest.mark.parametrize("rev,rot", [(False, False), (True, False), (False, True)])
def test_fp8_moving_max_matches_emulation(rev, rot):
    """Keys whose scores rise along the key axis (k_j = (1 + j/64)(1 + noise),
    q_i = 1 + noise, bf16 before quantisation): in forward order every tile
    raises each row's running max, so the rescale of O runs on every tile;
    in reverse order the first tile holds the max and later tiles' P
    underflow in E4M3.  Against the oracle's emulation on the dequantised
    operands, as in test_fp8_matches_emulation."""
    need_gpu()
    B, H, Hkv, N, d = 1, 4, 2, 700, 64
    announce(f"fa_fwd_fp8 moving max rev={rev} rot={rot}")
    nq = fagen.normal(fagen.stream_key(21, 91), B * H * N * d).reshape(B, H, N, d)
    nk = fagen.normal(fagen.stream_key(21, 92), B * Hkv * N * d).reshape(B, Hkv, N, d)
    nv = fagen.normal(fagen.stream_key(21, 93), B * Hkv * N * d).reshape(B, Hkv, N, d)
    g = 1.0 + np.arange(N, dtype=np.float64) / 64.0
    q = widen(fagen.to_storage(1.0 + 0.25 * nq, "bf16"), "bf16")
    k = widen(fagen.to_storage(g[None, None, :, None] * (1.0 + 0.25 * nk), "bf16"), "bf16")
    v = widen(fagen.to_storage(nv, "bf16"), "bf16")
    sg = fagen.random_signs(21, d) if rot else None
    qc, qs = oracle.quant_e4m3(q, sg, "rows32", False)
    kc, ks = oracle.quant_e4m3(k, sg, "rows32", False)
    vc, vs = oracle.quant_e4m3(v, None, "channels", False)
    deq = (oracle.dequant_e4m3(qc, qs), oracle.dequant_e4m3(kc, ks),
           oracle.dequant_e4m3(vc, vs, "channels"))
    scale = np.float32(1.0 / math.sqrt(d))
    sc = float(np.float32(scale / d)) if rot else float(scale)
    o, lse = _gpu_fp8((qc, qs, kc, ks, vc, vs), True, sc, 256.0, rev)
    _check_vs_emulation(o, lse, deq, True, sc, 256.0, rev, "fp8 moving max", bound_heads=(0, 3))
