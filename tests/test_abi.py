"""The C ABI on the CPU: libfa.so loads, exports every function include/fa.h
declares, and rejects bad arguments on the host before anything is launched.

No test here launches a kernel: every call either fails validation (so no
pointer is touched) or is an empty problem that returns before any HIP call.
"""
import ctypes
import os
import re

import pytest

import exact_io_aware_08_amd as fa
from exact_io_aware_08_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = 0x10000       # a 16-byte aligned fake address, never dereferenced
PM = 0x10008      # misaligned fake address
F32, F16, BF16 = 0, 1, 2
S = {n: v for v, n in _lib.STATUS_NAMES.items()}


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), (names, sorted(_lib.SIGNATURES))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings_and_version():
    lib = fa.load()
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.fa_status_str(code).decode().startswith(name)
    assert lib.fa_status_str(99).decode() == "unknown fa_status"
    assert fa.version() == 100


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Hkv=1, Nq=8, Nk=8, d=64, causal=1,
             scale=0.125, dtype=BF16, stream=None)
    a.update(kw)
    return fa.load().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                            a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"],
                            a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), "FA_ERR_NULL"), (dict(o=None), "FA_ERR_NULL"), (dict(v=None), "FA_ERR_NULL"),
    (dict(k=PM), "FA_ERR_ALIGN"), (dict(lse=PM), "FA_ERR_ALIGN"),
    (dict(B=-1), "FA_ERR_SHAPE"), (dict(H=0), "FA_ERR_SHAPE"), (dict(Hkv=0), "FA_ERR_SHAPE"),
    (dict(Nq=-3), "FA_ERR_SHAPE"), (dict(Nk=-1), "FA_ERR_SHAPE"),
    (dict(Nq=(1 << 31) // 64), "FA_ERR_SHAPE"),
    (dict(d=96), "FA_ERR_HEADDIM"), (dict(d=512), "FA_ERR_HEADDIM"),
    (dict(d=256, dtype=F32), "FA_ERR_HEADDIM"), (dict(d=256, B=0), "FA_OK"),
    (dict(d=256, dtype=F16, Nq=0), "FA_OK"),
    (dict(H=3, Hkv=2), "FA_ERR_GQA"),
    (dict(dtype=7), "FA_ERR_DTYPE"),
    (dict(scale=0.0), "FA_ERR_SCALE"), (dict(scale=-1.0), "FA_ERR_SCALE"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"), (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(causal=2), "FA_ERR_ARG"),
    (dict(B=0), "FA_OK"), (dict(Nq=0), "FA_OK"),
])
def test_fwd_validation(kw, expect):
    assert _fwd(**kw) == S[expect]


def _pcast(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Hkv=2, Nq=8, Nk=8, d=128, causal=1,
             scale=0.088, dtype=F32, p_scale=256.0, rev=1, n_sink=4, counts=P)
    a.update(kw)
    return fa.load().fa_fwd_pcast(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                  a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                                  a["dtype"], a["p_scale"], a["rev"], a["n_sink"], a["counts"],
                                  None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), "FA_ERR_NULL"), (dict(counts=0x10004), "FA_ERR_ALIGN"),
    (dict(dtype=F16), "FA_ERR_DTYPE"),
    (dict(p_scale=0.0), "FA_ERR_SCALE"), (dict(p_scale=512.0), "FA_ERR_SCALE"),
    (dict(rev=4), "FA_ERR_ARG"), (dict(rev=-1), "FA_ERR_ARG"), (dict(n_sink=-1), "FA_ERR_ARG"),
    (dict(d=32), "FA_ERR_HEADDIM"), (dict(d=256), "FA_ERR_HEADDIM"),
    (dict(d=256, dtype=BF16), "FA_ERR_HEADDIM"), (dict(B=0), "FA_OK"),
])
def test_pcast_validation(kw, expect):
    assert _pcast(**kw) == S[expect]


def _decode(ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=8, Hkv=2, Nk=100, d=64, scale=0.125,
             dtype=BF16, splits=3, ws=P)
    a.update(kw)
    need = fa.decode_workspace_bytes(a["B"], a["H"], a["Hkv"], a["Nk"], a["d"], a["splits"])
    return fa.load().fa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                               a["Hkv"], a["Nk"], a["d"], a["scale"], a["dtype"], a["splits"],
                               a["ws"], need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(k=None), "FA_ERR_NULL"), (dict(ws=None), "FA_ERR_WORKSPACE"),
    (dict(ws_bytes=16), "FA_ERR_WORKSPACE"), (dict(ws=PM), "FA_ERR_ALIGN"),
    (dict(dtype=F32), "FA_ERR_DTYPE"), (dict(splits=-1), "FA_ERR_ARG"),
    (dict(splits=5000), "FA_ERR_ARG"), (dict(H=6, Hkv=4), "FA_ERR_GQA"),
    (dict(d=80), "FA_ERR_HEADDIM"), (dict(d=256), "FA_ERR_HEADDIM"), (dict(B=0), "FA_OK"),
])
def test_decode_validation(kw, expect):
    assert _decode(**kw) == S[expect]


def test_decode_split_policy_and_workspace():
    # automatic split count: about 256 workgroups, no split under 512 keys
    assert fa.decode_splits(16, 32, 4, 8192) == 4
    assert fa.decode_splits(1, 8, 8, 100) == 1
    assert fa.decode_splits(1, 8, 1, 1 << 20) == 256
    assert fa.decode_splits(1, 32, 2, 1 << 20) == 128
    assert fa.decode_splits(2, 8, 2, 100, num_splits=7) == 7
    assert fa.decode_splits(2, 8, 3, 100) == -1
    # layout: [per-split LSE | per-split O on a 256-byte boundary]
    ws = fa.decode_workspace_bytes(16, 32, 4, 8192, 64)
    rows = 16 * 32 * 4
    assert ws == rows * 4 + rows * 64 * 4
    assert fa.decode_workspace_bytes(1, 1, 1, 10, 96) == 0
    # one split needs no workspace (the GPU tests pass none then)
    assert fa.decode_workspace_bytes(2, 8, 2, 100, 64, 1) == 0


def test_decode_noalloc_validation_and_limit():
    """fa_decode_noalloc validates like fa_decode, then rejects partials larger
    than its 8 MiB static scratch with FA_ERR_SCRATCH (before any launch);
    sizes within it reach the device check."""
    lib = fa.load()

    def call(B, H, Hkv, Nk, d, splits=0, dtype=BF16, q=P):
        return lib.fa_decode_noalloc(q, P, P, P, P, B, H, Hkv, Nk, d, 0.125, dtype, splits, None)

    assert fa.decode_workspace_bytes(16, 32, 4, 8192, 64) <= 8 << 20
    assert call(16, 32, 4, 8192, 64) == S["FA_ERR_DEVICE"]
    big = (64, 64, 8, 1 << 20, 128, 64)
    assert fa.decode_workspace_bytes(*big) > 8 << 20
    assert call(*big) == S["FA_ERR_SCRATCH"]
    # just over and just under the limit: rows * (4 + 4d) bytes plus alignment
    assert call(8, 16, 16, 1 << 20, 128, 2) == S["FA_ERR_DEVICE"]          # 132 KB of partials
    assert call(1, 8, 8, 1 << 22, 128, 2048) == S["FA_ERR_SCRATCH"]        # 8.5 MB
    assert call(2, 8, 3, 100, 64) == S["FA_ERR_GQA"]
    assert call(2, 8, 2, 100, 64, q=None) == S["FA_ERR_NULL"]
    assert call(2, 8, 2, 100, 64, dtype=F32) == S["FA_ERR_DTYPE"]
    assert call(2, 8, 2, 100, 64, splits=5000) == S["FA_ERR_ARG"]
    assert call(0, 8, 2, 100, 64) == S["FA_OK"]
    assert "static" in lib.fa_status_str(12).decode()


def test_kv_tile_and_cast_validation():
    assert fa.kv_tile(__import__("torch").bfloat16, 64) in (32, 64)
    lib = fa.load()
    assert lib.fa_kv_tile(F32, 128, 1) in (32, 64)
    assert lib.fa_kv_tile(BF16, 64, 1) == lib.fa_kv_tile(F32, 64, 1)
    assert lib.fa_kv_tile(F16, 64, 1) == -1
    assert lib.fa_kv_tile(F32, 48, 0) == -1
    # d = 256: the 16-bit forward only (32-key tiles)
    assert lib.fa_kv_tile(BF16, 256, 0) == 32 and lib.fa_kv_tile(F16, 256, 0) == 32
    assert lib.fa_kv_tile(F32, 256, 0) == -1 and lib.fa_kv_tile(BF16, 256, 1) == -1
    assert lib.fa_cast_e4m3(None, None, None, 4, None) == S["FA_ERR_NULL"]
    assert lib.fa_cast_e4m3(None, None, None, 0, None) == S["FA_OK"]


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)


def test_binding_output_checks():
    """Caller-supplied outputs are checked for exact shape, dtype, device and
    contiguity before any launch (the C ABI cannot size-check raw pointers):
    the helper every entry point uses, exercised on CPU tensors."""
    import torch
    dev = torch.device("cpu")
    good = torch.zeros(2, 3, 5, 64, dtype=torch.bfloat16)
    fa._check_out("out", good, (2, 3, 5, 64), torch.bfloat16, dev)
    bad = [
        (torch.zeros(2, 3, 4, 64, dtype=torch.bfloat16), (2, 3, 5, 64), torch.bfloat16),  # short
        (torch.zeros(2, 3, 5, 64, dtype=torch.float16), (2, 3, 5, 64), torch.bfloat16),   # dtype
        (torch.zeros(2, 3, 64, 5, dtype=torch.bfloat16).transpose(-1, -2), (2, 3, 5, 64),
         torch.bfloat16),                                                                   # strided
        (torch.zeros(4, dtype=torch.int32), (4,), torch.int64),                             # counts
        (torch.zeros(3, dtype=torch.int64), (4,), torch.int64),
        (torch.zeros(2, 3, 5), (2, 3, 6), torch.float32),                                   # lse
    ]
    for t, shape, dt in bad:
        with pytest.raises(ValueError):
            fa._check_out("x", t, shape, dt, dev)
    with pytest.raises(ValueError):
        fa._check_out("x", good, (2, 3, 5, 64), torch.bfloat16, torch.device("meta"))
    with pytest.raises(TypeError):
        fa._check_out("x", None, (1,), torch.float32, dev)
    fa._check_workspace(torch.zeros(100, dtype=torch.uint8), dev)
    with pytest.raises(ValueError):
        fa._check_workspace(torch.zeros(10, 10, dtype=torch.uint8).t(), dev)


def _bwd(ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, H=4, Hkv=2, Nq=64, Nk=64,
             d=64, causal=1, scale=0.125, dtype=BF16, ws=P)
    a.update(kw)
    need = fa.bwd_workspace_bytes(a["B"], a["H"], a["Nq"])
    return fa.load().fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                            a["dv"], a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                            a["causal"], a["scale"], a["dtype"], a["ws"],
                            need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), "FA_ERR_NULL"), (dict(do=None), "FA_ERR_NULL"), (dict(lse=None), "FA_ERR_NULL"),
    (dict(o=None), "FA_ERR_NULL"), (dict(dk=None), "FA_ERR_NULL"), (dict(dv=None), "FA_ERR_NULL"),
    (dict(dq=None), "FA_ERR_NULL"), (dict(do=PM), "FA_ERR_ALIGN"), (dict(dv=PM), "FA_ERR_ALIGN"),
    (dict(ws=None), "FA_ERR_WORKSPACE"), (dict(ws_bytes=8), "FA_ERR_WORKSPACE"),
    (dict(ws=PM), "FA_ERR_ALIGN"), (dict(dtype=F32), "FA_ERR_DTYPE"), (dict(d=32), "FA_ERR_HEADDIM"), (dict(d=256), "FA_ERR_HEADDIM"),
    (dict(H=6, Hkv=4), "FA_ERR_GQA"), (dict(scale=0.0), "FA_ERR_SCALE"), (dict(causal=3), "FA_ERR_ARG"),
    (dict(B=-1), "FA_ERR_SHAPE"), (dict(B=0), "FA_OK"), (dict(Nq=0, Nk=0), "FA_OK"),
])
def test_bwd_validation(kw, expect):
    assert _bwd(**kw) == S[expect]


def test_bwd_workspace_size():
    assert fa.bwd_workspace_bytes(2, 3, 100) == 2560   # 600 floats, rounded up to 256 bytes
    assert fa.bwd_workspace_bytes(0, 3, 100) == 0
    assert fa.bwd_workspace_bytes(-1, 3, 100) == 0


def _paged(**kw):
    a = dict(q=P, kp=P, vp=P, bt=P, sl=P, o=P, lse=P, B=2, H=8, Hkv=2, num_pages=10, page_size=64,
             max_pages=4, d=64, scale=0.125, dtype=BF16, splits=0, ws=P, ws_bytes=1 << 20)
    a.update(kw)
    return fa.load().fa_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["o"], a["lse"],
                                     a["B"], a["H"], a["Hkv"], a["num_pages"], a["page_size"],
                                     a["max_pages"], a["d"], a["scale"], a["dtype"], a["splits"],
                                     a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(page_size=48), "FA_ERR_ARG"), (dict(page_size=16), "FA_ERR_ARG"),
    (dict(max_pages=0), "FA_ERR_ARG"), (dict(num_pages=-1), "FA_ERR_ARG"),
    (dict(bt=None), "FA_ERR_NULL"), (dict(sl=None), "FA_ERR_NULL"), (dict(kp=None), "FA_ERR_NULL"),
    (dict(bt=0x10002), "FA_ERR_ALIGN"), (dict(o=PM), "FA_ERR_ALIGN"),
    (dict(dtype=F32), "FA_ERR_DTYPE"), (dict(H=6, Hkv=4), "FA_ERR_GQA"), (dict(d=96), "FA_ERR_HEADDIM"),
    (dict(splits=2, ws=None, ws_bytes=0), "FA_ERR_WORKSPACE"), (dict(B=-2), "FA_ERR_SHAPE"),
    (dict(max_pages=64, ws_bytes=1000), "FA_ERR_WORKSPACE"),   # automatic splits: 33,288 bytes needed
    (dict(B=0), "FA_OK"),
])
def test_decode_paged_validation(kw, expect):
    assert _paged(**kw) == S[expect]


def test_paged_workspace_sizes():
    """Forced splits: the contiguous decode's layout at Nk = max_pages * page_size.
    Automatic: room for min(ceil(max_seq / 512), ceil(256 / hq)) splits per
    sequence, hq = Hkv * ceil((H / Hkv) / 16) workgroups per (sequence, split),
    then one int per sequence (its split count) on a 256-byte boundary."""
    assert fa.decode_paged_workspace_bytes(16, 32, 4, 64, 128, 64, 4) == \
        fa.decode_workspace_bytes(16, 32, 4, 8192, 64, 4)
    rows = 16 * 32 * 16                      # max_seq 8192 -> 16 splits (hq = 4 allows 64)
    assert fa.decode_paged_workspace_bytes(16, 32, 4, 64, 128, 64) == rows * 4 + rows * 64 * 4 + 16 * 4
    rows = 1 * 8 * 32                        # hq = 8 -> at most 32 splits
    assert fa.decode_paged_workspace_bytes(1, 8, 8, 4096, 256, 128) == rows * 4 + rows * 128 * 4 + 4
    rows = 2 * 8 * 8                         # max_seq 4096 -> 8 splits
    assert fa.decode_paged_workspace_bytes(2, 8, 2, 64, 64, 64) == 33288 == 512 + rows * 64 * 4 + 8
    assert fa.decode_paged_workspace_bytes(3, 8, 2, 1, 32, 64) == 0      # 32 keys: one split
    # more than 256 sequences: the uniform split (no per-sequence counts)
    assert fa.decode_paged_workspace_bytes(257, 8, 2, 64, 128, 64) == \
        fa.decode_workspace_bytes(257, 8, 2, 8192, 64)
    assert fa.decode_paged_workspace_bytes(256, 8, 2, 64, 128, 64) != \
        fa.decode_workspace_bytes(256, 8, 2, 8192, 64)
    assert fa.decode_paged_workspace_bytes(2, 8, 2, 4, 48, 64) == 0      # bad page size
    assert fa.decode_paged_workspace_bytes(2, 8, 2, 4, 64, 96) == 0      # bad head dim
    assert fa.decode_paged_workspace_bytes(2, 8, 3, 4, 64, 64) == 0      # H % Hkv != 0


def _quant(**kw):
    a = dict(x=P, codes=P, scales=P, signs=None, B=1, H=2, N=64, d=64, dtype=BF16, layout=0, whole=0)
    a.update(kw)
    return fa.load().fa_quant_e4m3(a["x"], a["codes"], a["scales"], a["signs"], a["B"], a["H"],
                                   a["N"], a["d"], a["dtype"], a["layout"], a["whole"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(d=96), "FA_ERR_HEADDIM"), (dict(dtype=7), "FA_ERR_DTYPE"), (dict(layout=2), "FA_ERR_ARG"),
    (dict(whole=2), "FA_ERR_ARG"), (dict(B=-1), "FA_ERR_SHAPE"), (dict(H=0), "FA_ERR_SHAPE"),
    (dict(B=70000), "FA_ERR_SHAPE"), (dict(x=None), "FA_ERR_NULL"), (dict(scales=None), "FA_ERR_NULL"),
    (dict(codes=PM), "FA_ERR_ALIGN"), (dict(scales=0x10002), "FA_ERR_ALIGN"),
    (dict(signs=0x10001), "FA_ERR_ALIGN"), (dict(B=0), "FA_OK"), (dict(N=0, x=None), "FA_OK"),
])
def test_quant_validation(kw, expect):
    assert _quant(**kw) == S[expect]


def _fp8(**kw):
    a = dict(q=P, k=P, v=P, qs=P, ks=P, vs=P, o=P, lse=P, B=1, H=4, Hkv=2, Nq=64, Nk=64, d=64,
             causal=1, scale=0.125, p_scale=256.0, rev=0, odt=BF16)
    a.update(kw)
    return fa.load().fa_fwd_fp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"],
                                a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"],
                                a["scale"], a["p_scale"], a["rev"], a["odt"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(p_scale=448.0), "FA_ERR_SCALE"), (dict(p_scale=0.5), "FA_ERR_SCALE"),
    (dict(p_scale=3.0), "FA_ERR_SCALE"), (dict(p_scale=float("nan")), "FA_ERR_SCALE"),
    (dict(scale=0.0), "FA_ERR_SCALE"), (dict(odt=F16), "FA_ERR_DTYPE"), (dict(causal=2), "FA_ERR_ARG"),
    (dict(rev=2), "FA_ERR_ARG"), (dict(d=96), "FA_ERR_HEADDIM"), (dict(H=3), "FA_ERR_GQA"),
    (dict(q=None), "FA_ERR_NULL"), (dict(qs=None), "FA_ERR_NULL"), (dict(vs=None), "FA_ERR_NULL"),
    (dict(vs=0x10004), "FA_ERR_ALIGN"), (dict(ks=0x10002), "FA_ERR_ALIGN"), (dict(o=PM), "FA_ERR_ALIGN"),
    (dict(B=0), "FA_OK"), (dict(Nq=0, q=None, o=None, qs=None), "FA_OK"),
])
def test_fwd_fp8_validation(kw, expect):
    assert _fp8(**kw) == S[expect]


def test_fp8_kv_tile():
    assert fa.fp8_kv_tile() == 64
