"""Seeded synthetic inputs for the attention workloads.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests. It holds no attention arithmetic: only random numbers, the workload
shapes and the input constructions (iid Gaussian, AR(1) series, attention-sink
shift), and one rounding of fp64 draws to the storage dtype.

Random numbers: a counter-based SplitMix64 stream (Steele, Lea & Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; the 64-bit
finaliser constants are the published ones).  The value at element index i of
a stream depends only on (seed, stream tags, i), so any subset can be
regenerated and results do not depend on thread counts or chunking.
Gaussians: Box-Muller on pairs of uniforms (index 2p, 2p+1 -> outputs 2p, 2p+1).

Workloads (sizes and distributions) follow the pages' settings:
  * tiny exact check, GPT-2-small-shaped prefill (GPT-2 is named in the
    "FlashAttention (IT)" entry, section "Risultati empirici");
  * a full trading day at one row per second, 6.5 h x 3600 = 23,400 steps
    (marketmaker.cc blog "Atención flash y la pregunta sobre la longitud de la
    secuencia", opening paragraphs) built as AR(1) series plus noise;
  * a TinyLlama-shaped GQA decode (FlashAttention-V summary, "Configuração
    Experimental");
  * the attention-sink construction of the P-cast summary ("Precisión de
    P-Cast en la Atención FP8", section "Marco Teórico"): non-sink logits
    ~N(0,1), the first k=4 keys' logits shifted up by Delta.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "WORKLOADS", "stream_key", "uniform", "normal", "to_storage", "iid_normal",
    "ar1_series", "sink_inputs", "make_inputs", "sample_rows", "outlier_normal", "random_signs",
]

_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB

# Tensor ids used as stream tags.
T_Q, T_K, T_V = 1, 2, 3
_KIND_MAIN, _KIND_AR, _KIND_NOISE, _KIND_ROWS, _KIND_OUTLIER, _KIND_SIGNS = 0, 1, 2, 3, 4, 5

_CHUNK = 1 << 22  # elements generated per vectorised step (bounds temporaries)


def _mix64_scalar(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * _C1) & _M64
    z = ((z ^ (z >> 27)) * _C2) & _M64
    return z ^ (z >> 31)


def _mix64(z: np.ndarray) -> np.ndarray:
    # uint64 arithmetic wraps modulo 2**64, which is what the finaliser needs.
    z = (z ^ (z >> np.uint64(30))) * np.uint64(_C1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(_C2)
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, *tags: int) -> int:
    """64-bit key of the stream named by (seed, tags...)."""
    k = _mix64_scalar((int(seed) + _GAMMA) & _M64)
    for t in tags:
        k = _mix64_scalar(k ^ (((int(t) + 1) * _GAMMA) & _M64))
    return k


def _bits(key: int, counter: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (counter.astype(np.uint64) + np.uint64(1)) * np.uint64(_GAMMA)
        return _mix64(z)


def uniform(key: int, counter: np.ndarray) -> np.ndarray:
    """Uniform doubles in the open interval (0, 1) at the given counters."""
    b = _bits(key, counter) >> np.uint64(11)
    return (b.astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(key: int, n: int, start: int = 0) -> np.ndarray:
    """Standard normal doubles for element indices [start, start+n)."""
    out = np.empty(n, dtype=np.float64)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        idx = np.arange(start + c0, start + c1, dtype=np.int64)
        pair = idx >> 1
        u1 = uniform(key, 2 * pair)
        u2 = uniform(key, 2 * pair + 1)
        r = np.sqrt(-2.0 * np.log(u1))
        ang = 2.0 * math.pi * u2
        out[c0:c1] = np.where((idx & 1) == 0, r * np.cos(ang), r * np.sin(ang))
    return out


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype: fp64 -> fp32 (RNE), then, for
    the 16-bit types, fp32 -> target (RNE).  'bf16' returns uint16 arrays
    holding bfloat16 bit patterns."""
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float32).astype(np.float16)
    if dtype == "bf16":
        u = x.astype(np.float32).view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a storage array to float32."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


def iid_normal(seed: int, tensor: int, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    return to_storage(normal(stream_key(seed, tensor, _KIND_MAIN), n), dtype).reshape(shape)


def ar1_series(seed: int, tensor: int, shape, dtype: str, phi: float = 0.9,
               noise_var: float = 0.1) -> np.ndarray:
    """AR(1) series along the sequence axis of a [B, H, N, d] tensor.

    One independent series per (b, h, channel): x_0 ~ N(0,1) (stationary start),
    x_t = phi*x_{t-1} + sqrt(1-phi^2)*z_t (unit marginal variance), and the
    stored value is x_t + sqrt(noise_var)*eta_t with z, eta iid N(0,1).
    """
    B, H, N, d = shape
    z = normal(stream_key(seed, tensor, _KIND_AR), B * H * N * d).reshape(B, H, N, d)
    eta = normal(stream_key(seed, tensor, _KIND_NOISE), B * H * N * d).reshape(B, H, N, d)
    c = math.sqrt(1.0 - phi * phi)
    x = np.empty((B, H, N, d), dtype=np.float64)
    x[:, :, 0, :] = z[:, :, 0, :]
    for t in range(1, N):
        x[:, :, t, :] = phi * x[:, :, t - 1, :] + c * z[:, :, t, :]
    x += math.sqrt(noise_var) * eta
    return to_storage(x, dtype)


def sink_inputs(seed: int, B: int, H: int, N: int, d: int, delta: float,
                n_sink: int = 4):
    """fp32 Q, K, V with an attention sink on keys [0, n_sink).

    Q, K, V iid N(0,1); then Q[..., 0] := 1 for every query and
    K[:, :, j, 0] += delta*sqrt(d) for j < n_sink.  With scale 1/sqrt(d), every
    query's logit to a sink key rises by exactly delta (up to fp32 rounding) and
    non-sink logits stay ~N(0,1).
    """
    q = normal(stream_key(seed, T_Q, _KIND_MAIN), B * H * N * d).reshape(B, H, N, d)
    k = normal(stream_key(seed, T_K, _KIND_MAIN), B * H * N * d).reshape(B, H, N, d)
    v = normal(stream_key(seed, T_V, _KIND_MAIN), B * H * N * d).reshape(B, H, N, d)
    q[..., 0] = 1.0
    k[:, :, :n_sink, 0] += delta * math.sqrt(d)
    return to_storage(q, "f32"), to_storage(k, "f32"), to_storage(v, "f32")


def outlier_normal(seed: int, tensor: int, shape, dtype: str, frac: float = 1e-3,
                   mag: float = 10.0) -> np.ndarray:
    """iid N(0,1) entries, each independently (probability frac) multiplied by
    mag: rare large coordinates, the outliers that spoil naive FP8 attention
    (marketmaker.cc blog, "FA3: Mecanica de la tolva", item 3)."""
    n = int(np.prod(shape))
    x = normal(stream_key(seed, tensor, _KIND_MAIN), n)
    u = uniform(stream_key(seed, tensor, _KIND_OUTLIER), np.arange(n, dtype=np.int64))
    x = np.where(u < frac, mag * x, x)
    return to_storage(x, dtype).reshape(shape)


def random_signs(seed: int, d: int) -> np.ndarray:
    """d random signs (+1.0 / -1.0, fp32) for the random rotation."""
    u = uniform(stream_key(seed, 0, _KIND_SIGNS), np.arange(d, dtype=np.int64))
    return np.where(u < 0.5, -1.0, 1.0).astype(np.float32)


# Workload table.  'scale' is the fp32 value of 1/sqrt(d).
WORKLOADS = {
    "tiny_exact_f32": dict(name="tiny_exact_f32", B=1, H=1, Hkv=1, Nq=256, Nk=256, d=64,
            dtype="f32", causal=False, kind="iid"),
    "gpt2s_prefill_bf16": dict(name="gpt2s_prefill_bf16", B=4, H=12, Hkv=12, Nq=2048, Nk=2048, d=64,
            dtype="bf16", causal=True, kind="iid"),
    "trading_day_prefill_bf16": dict(name="trading_day_prefill_bf16", B=1, H=12, Hkv=12, Nq=23400, Nk=23400,
            d=64, dtype="bf16", causal=True, kind="ar1", sample_rows=512),
    "gqa_decode_bf16": dict(name="gqa_decode_bf16", B=16, H=32, Hkv=4, Nq=1, Nk=8192, d=64,
            dtype="bf16", causal=False, kind="iid", decode=True),
    "pcast_sink_f32": dict(name="pcast_sink_f32", B=1, H=32, Hkv=32, Nq=8192, Nk=8192, d=128,
            dtype="f32", causal=True, kind="sink", deltas=(4.0, 6.0, 8.0, 10.0),
            n_sink=4),
}
for _c in WORKLOADS.values():
    _c["scale"] = float(np.float32(1.0 / math.sqrt(_c["d"])))


def make_inputs(cfg: dict, seed: int = 0, delta: float | None = None):
    """Q, K, V storage arrays for a workload dict (see WORKLOADS)."""
    B, H, Hkv, Nq, Nk, d = (cfg[k] for k in ("B", "H", "Hkv", "Nq", "Nk", "d"))
    dt = cfg["dtype"]
    kind = cfg.get("kind", "iid")
    if kind == "iid":
        q = iid_normal(seed, T_Q, (B, H, Nq, d), dt)
        k = iid_normal(seed, T_K, (B, Hkv, Nk, d), dt)
        v = iid_normal(seed, T_V, (B, Hkv, Nk, d), dt)
    elif kind == "ar1":
        q = ar1_series(seed, T_Q, (B, H, Nq, d), dt)
        k = ar1_series(seed, T_K, (B, Hkv, Nk, d), dt)
        v = ar1_series(seed, T_V, (B, Hkv, Nk, d), dt)
    elif kind == "sink":
        assert Nq == Nk and H == Hkv and dt == "f32"
        q, k, v = sink_inputs(seed, B, H, Nq, d, float(delta), cfg.get("n_sink", 4))
    else:
        raise ValueError(kind)
    return q, k, v


def sample_rows(seed: int, head: int, N: int, n: int) -> np.ndarray:
    """n distinct query rows of one head, uniform without replacement, sorted."""
    u = uniform(stream_key(seed, _KIND_ROWS, head), np.arange(N, dtype=np.int64))
    return np.sort(np.argsort(u, kind="stable")[: min(n, N)]).astype(np.int64)
