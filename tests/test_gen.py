"""The seeded input generator: determinism, counter-based slicing, moments,
the storage rounding and the workload constructions."""
import math

import numpy as np
import torch

import fagen


def test_counter_based_slices():
    key = fagen.stream_key(0, 1, 2)
    full = fagen.normal(key, 1000)
    assert np.array_equal(fagen.normal(key, 10, start=5), full[5:15])
    assert np.array_equal(fagen.normal(key, 11, start=500), full[500:511])
    assert not np.array_equal(full, fagen.normal(fagen.stream_key(1, 1, 2), 1000))
    assert np.array_equal(full, fagen.normal(fagen.stream_key(0, 1, 2), 1000))


def test_uniform_open_interval_and_moments():
    key = fagen.stream_key(3, 9)
    u = fagen.uniform(key, np.arange(1 << 20))
    assert u.min() > 0 and u.max() < 1
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / u.size)
    z = fagen.normal(key, 1 << 20)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    assert abs(np.mean(z ** 4) - 3) < 0.05
    assert abs(np.corrcoef(z[:-1], z[1:])[0, 1]) < 5 / math.sqrt(n)


def test_storage_rounding_matches_torch():
    x = fagen.normal(fagen.stream_key(0, 7), 100000) * 3
    bf = fagen.to_storage(x, "bf16")
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bf.view(np.int16), ref)
    back = fagen.storage_to_f32(bf, "bf16")
    assert np.array_equal(back, torch.from_numpy(ref).view(torch.bfloat16).float().numpy())
    h = fagen.to_storage(x, "f16")
    assert np.array_equal(h, torch.from_numpy(x).float().to(torch.float16).numpy())


def test_ar1_statistics():
    x = fagen.ar1_series(0, 1, (1, 2, 20000, 4), "f32").astype(np.float64)
    s = x.reshape(2, 20000, 4).transpose(0, 2, 1).reshape(8, 20000)
    var = s.var(axis=1).mean()
    assert abs(var - 1.1) < 0.06           # unit AR(1) variance + 0.1 noise
    r1 = np.mean([np.corrcoef(r[:-1], r[1:])[0, 1] for r in s])
    assert abs(r1 - 0.9 / 1.1) < 0.02


def test_sink_construction():
    q, k, v = fagen.sink_inputs(0, 1, 2, 64, 16, 8.0)
    q0, k0, v0 = fagen.sink_inputs(0, 1, 2, 64, 16, 0.0)
    assert np.all(q[..., 0] == 1.0)
    shift = k.astype(np.float64) - k0.astype(np.float64)
    assert np.allclose(shift[:, :, :4, 0], 8.0 * 4.0, atol=1e-5)
    assert np.all(shift[:, :, 4:] == 0) and np.all(shift[..., 1:] == 0)
    assert np.array_equal(v, v0)


def test_sample_rows():
    r = fagen.sample_rows(0, 3, 23400, 512)
    assert r.size == 512 and np.all(np.diff(r) > 0) and r[0] >= 0 and r[-1] < 23400
    assert np.array_equal(r, fagen.sample_rows(0, 3, 23400, 512))
    assert not np.array_equal(r, fagen.sample_rows(0, 4, 23400, 512))
    assert np.array_equal(fagen.sample_rows(0, 0, 10, 512), np.arange(10))


def test_workload_table():
    c = fagen.WORKLOADS
    td, dec, tiny = c["trading_day_prefill_bf16"], c["gqa_decode_bf16"], c["tiny_exact_f32"]
    assert (td["Nq"], td["H"], td["d"], td["dtype"]) == (23400, 12, 64, "bf16")
    assert (dec["B"], dec["H"], dec["Hkv"], dec["Nk"]) == (16, 32, 4, 8192)
    assert tiny["scale"] == 0.125
    assert c["pcast_sink_f32"]["scale"] == float(np.float32(1 / math.sqrt(128)))
    assert all(name == w["name"] for name, w in c.items())
    q, k, v = fagen.make_inputs(tiny, 0)
    assert q.dtype == np.float32 and q.shape == (1, 1, 256, 64)
    q2, _, _ = fagen.make_inputs(tiny, 0)
    assert np.array_equal(q, q2)
