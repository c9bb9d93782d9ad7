"""libfa -- exact IO-aware attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of include/fa.h: it checks tensor
placement, dtype, shape and layout -- of the inputs and of every output or
workspace the caller passes in, because the C ABI receives raw pointers and
cannot size-check them -- allocates outputs with torch and passes raw device
pointers plus torch's current HIP stream.  Every step of the
computation runs in the HIP kernels of libfa.so; there is no Python or CPU
path.

    o, lse = fwd(q, k, v, causal=True)                       # prefill
    o, lse, counts = fwd_pcast(q, k, v, causal=True, p_scale=256.0, kv_reverse=True)
    o, lse = decode(q, k_cache, v_cache)                     # split-KV GQA decode
"""
from __future__ import annotations

import math

import torch

from ._lib import FA_BF16, FA_F16, FA_F32, FaError, check, load

__all__ = ["fwd", "fwd_pcast", "decode", "decode_noalloc", "cast_e4m3", "kv_tile", "decode_splits",
           "decode_workspace_bytes", "decode_paged_workspace_bytes", "version", "FaError", "load"]

_DT = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}


def _stream_ptr(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check_tensor(name, t, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims [B, heads, seq, d], got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in _DT:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output: exact shape and dtype, on `device`,
    contiguous.  Raises before anything is launched (an undersized or
    mistyped buffer would otherwise be written out of bounds)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(t, device):
    """A caller-supplied workspace: any dtype, on `device`, contiguous (its
    byte size is checked by the C ABI against what the call needs)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _qkv_shapes(q, k, v):
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(n, t, 4)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and k disagree on batch or head_dim")
    return B, H, Hkv, Nq, Nk, d


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
        return_lse: bool = True, stream=None):
    """Forward attention.  q: [B,H,Nq,d]; k, v: [B,Hkv,Nk,d]; returns (o, lse)."""
    B, H, Hkv, Nq, Nk, d = _qkv_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _check_out("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H, Nq), torch.float32, q.device)
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr() if lse is not None else None, B, H, Hkv, Nq, Nk, d,
                       int(bool(causal)), float(scale), _DT[q.dtype], _stream_ptr(stream))
    check(st, "fa_fwd")
    return o, lse


def fwd_pcast(q, k, v, causal: bool = True, scale: float | None = None, p_scale: float = 256.0,
              kv_reverse: bool = True, n_sink: int = 0, counts=None, out=None, lse=None,
              stream=None, tile_local_max: bool = False):
    """E4M3 P-cast forward (fp32 or bf16 q, k, v; bf16 is widened exactly on
    load).  Returns (o, lse, counts) where
    counts (int64 device tensor of 4) holds [non-sink casts, non-sink flushes,
    casts outside the sink tiles, flushes outside the sink tiles]."""
    B, H, Hkv, Nq, Nk, d = _qkv_shapes(q, k, v)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is not None:
        _check_out("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H, Nq), torch.float32, q.device)
    if counts is not None:  # the kernel adds four uint64 values into it
        _check_out("counts", counts, (4,), torch.int64, q.device)
    o = out if out is not None else torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if counts is None:
        counts = torch.zeros(4, dtype=torch.int64, device=q.device)
    st = load().fa_fwd_pcast(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, H, Hkv, Nq, Nk, d, int(bool(causal)),
                             float(scale), _DT[q.dtype], float(p_scale),
                             int(bool(kv_reverse)) | (int(bool(tile_local_max)) << 1),
                             int(n_sink), counts.data_ptr(), _stream_ptr(stream))
    check(st, "fa_fwd_pcast")
    return o, lse, counts


def decode_splits(B: int, H: int, Hkv: int, Nk: int, num_splits: int = 0) -> int:
    return load().fa_decode_splits(B, H, Hkv, Nk, num_splits)


def decode_workspace_bytes(B: int, H: int, Hkv: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, Hkv, Nk, d, num_splits))


def decode_paged_workspace_bytes(B: int, H: int, Hkv: int, max_pages: int, page_size: int, d: int,
                                 num_splits: int = 0) -> int:
    return int(load().fa_decode_paged_workspace_bytes(B, H, Hkv, max_pages, page_size, d, num_splits))


def decode_paged_workspace(B: int, H: int, Hkv: int, max_pages: int, page_size: int, d: int,
                           num_splits: int = 0, device="cuda"):
    """A paged-decode workspace (uint8 tensor), or None when the call needs none."""
    need = decode_paged_workspace_bytes(B, H, Hkv, max_pages, page_size, d, num_splits)
    return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None


def decode_workspace(B: int, H: int, Hkv: int, Nk: int, d: int, num_splits: int = 0,
                     device="cuda"):
    """A decode workspace (uint8 tensor) for these sizes, or None when the
    call needs none.  Any later call it is large enough for may reuse it."""
    need = decode_workspace_bytes(B, H, Hkv, Nk, d, num_splits)
    return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None


def decode(q, k_cache, v_cache, scale: float | None = None, num_splits: int = 0,
           workspace=None, out=None, lse=None, return_lse: bool = True, stream=None):
    """Split-KV decode.  q: [B,H,1,d]; k_cache, v_cache: [B,Hkv,Nk,d].
    workspace: from decode_workspace(); allocated here when not given."""
    B, H, Hkv, Nq, Nk, d = _qkv_shapes(q, k_cache, v_cache)
    if Nq != 1:
        raise ValueError("decode takes one query token per (batch, head)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _check_out("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H, 1), torch.float32, q.device)
    if workspace is None:
        workspace = decode_workspace(B, H, Hkv, Nk, d, num_splits, q.device)
    else:
        _check_workspace(workspace, q.device)
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
    st = load().fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                          lse.data_ptr() if lse is not None else None, B, H, Hkv, Nk, d,
                          float(scale), _DT[q.dtype], int(num_splits),
                          workspace.data_ptr() if workspace is not None else None,
                          workspace.numel() * workspace.element_size() if workspace is not None
                          else 0, _stream_ptr(stream))
    check(st, "fa_decode")
    return o, lse


def decode_noalloc(q, k_cache, v_cache, scale: float | None = None, num_splits: int = 0,
                   out=None, lse=None, return_lse: bool = True, stream=None):
    """decode() without a workspace: the split partials live in the library's
    static 8 MiB device scratch (fa_decode_noalloc), so the C call allocates
    nothing.  Outputs are allocated here unless passed in.  Calls that overlap
    on one GPU race on the shared scratch."""
    B, H, Hkv, Nq, Nk, d = _qkv_shapes(q, k_cache, v_cache)
    if Nq != 1:
        raise ValueError("decode takes one query token per (batch, head)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _check_out("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H, 1), torch.float32, q.device)
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
    st = load().fa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, B, H, Hkv, Nk, d,
                                  float(scale), _DT[q.dtype], int(num_splits), _stream_ptr(stream))
    check(st, "fa_decode_noalloc")
    return o, lse


def bwd_workspace_bytes(B: int, H: int, Nq: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, Nq))


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
        workspace=None, dq=None, dk=None, dv=None, stream=None):
    """Backward of fwd: (dq, dk, dv) from the forward's o and lse and dout = dL/dO."""
    B, H, Hkv, Nq, Nk, d = _qkv_shapes(q, k, v)
    for name, t, shape in (("o", o, q.shape), ("dout", dout, q.shape)):
        if t.device != q.device or t.dtype != q.dtype or not t.is_contiguous() or t.shape != shape:
            raise ValueError(f"{name} must match q (device, dtype, shape, contiguous)")
    if lse.device != q.device or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("lse must be a contiguous fp32 [B, H, Nq] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _check_out(name, t, ref.shape, ref.dtype, q.device)
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    if workspace is None:
        n = bwd_workspace_bytes(B, H, Nq)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    st = load().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, Nq,
                       Nk, d, int(bool(causal)), float(scale), _DT[q.dtype], workspace.data_ptr(),
                       workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    check(st, "fa_bwd")
    return dq, dk, dv


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float | None = None,
                 num_splits: int = 0, workspace=None, out=None, lse=None, stream=None):
    """Decode against a paged cache.  q: [B,H,1,d]; k_pages, v_pages:
    [num_pages,Hkv,page_size,d]; block_table: int32 [B,max_pages];
    seq_lens: int32 [B]."""
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        _check_tensor(n, t, 4)
    if not (q.dtype == k_pages.dtype == v_pages.dtype) or k_pages.shape != v_pages.shape:
        raise ValueError("q, k_pages, v_pages: one dtype; k_pages and v_pages one shape")
    B, H, Nq, d = q.shape
    num_pages, Hkv, page_size, dk = k_pages.shape
    if Nq != 1 or dk != d:
        raise ValueError("decode takes one query token per (batch, head) with the cache's d")
    for n, t, shape in (("block_table", block_table, None), ("seq_lens", seq_lens, (B,))):
        if t.device != q.device or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 tensor on q's device")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _check_out("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H, 1), torch.float32, q.device)
    if workspace is None:
        workspace = decode_paged_workspace(B, H, Hkv, max_pages, page_size, d, num_splits, q.device)
    else:
        _check_workspace(workspace, q.device)
    o = out if out is not None else torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
    st = load().fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                block_table.data_ptr(), seq_lens.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, H, Hkv, num_pages, page_size, max_pages, d,
                                float(scale), _DT[q.dtype], int(num_splits),
                                workspace.data_ptr() if workspace is not None else None,
                                workspace.numel() * workspace.element_size()
                                if workspace is not None else 0, _stream_ptr(stream))
    check(st, "fa_decode_paged")
    return o, lse


def cast_e4m3(x, stream=None):
    """Device E4M3 round trip used by the P-cast kernel: (codes uint8, values fp32)."""
    if x.device.type != "cuda" or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 GPU tensor")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    back = torch.empty_like(x)
    st = load().fa_cast_e4m3(x.data_ptr(), codes.data_ptr(), back.data_ptr(), x.numel(),
                             _stream_ptr(stream))
    check(st, "fa_cast_e4m3")
    return codes, back


def quant_e4m3(x, signs=None, layout: str = "rows32", whole: bool = False, codes=None,
               scales=None, stream=None):
    """E4M3 codes of x [B,H,N,d] and their power-of-two scales.

    signs: None or a GPU fp32 tensor [d] of +-1 (random-sign Hadamard rotation).
    layout "rows32": scales [B,H,ceil(N/32)]; "channels": scales [B,H,d].
    whole=True: one scale for the whole tensor, repeated in that layout."""
    _check_tensor("x", x, 4)
    B, H, N, d = x.shape
    lay = {"rows32": 0, "channels": 1}[layout]
    sshape = (B, H, (N + 31) // 32 if lay == 0 else d)
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    else:
        _check_out("codes", codes, x.shape, torch.uint8, x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    else:
        _check_out("scales", scales, sshape, torch.float32, x.device)
    if signs is not None and (signs.device != x.device or signs.dtype != torch.float32
                              or signs.numel() != d or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous fp32 tensor of d values on x's device")
    st = load().fa_quant_e4m3(x.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                              signs.data_ptr() if signs is not None else None, B, H, N, d,
                              _DT[x.dtype], lay, int(bool(whole)), _stream_ptr(stream))
    check(st, "fa_quant_e4m3")
    return codes, scales


def fp8_kv_tile() -> int:
    return load().fa_fp8_kv_tile()


def fwd_fp8(q, k, v, q_scales, k_scales, v_scales, causal: bool = False,
            scale: float | None = None, p_scale: float = 256.0, kv_reverse: bool = False,
            out_dtype=torch.bfloat16, out=None, lse=None, stream=None):
    """FP8 forward over E4M3 codes (uint8 tensors [B,H,Nq,d], [B,Hkv,Nk,d]) with
    the scales of quant_e4m3 (q, k: "rows32"; v: "channels").  scale defaults
    to 1/sqrt(d); divide it by d when q and k were rotated."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 4 \
                or t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous uint8 GPU tensor [B, heads, seq, d]")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("q, k, v shapes disagree")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    want = {"q_scales": (q_scales, (B, H, (Nq + 31) // 32)),
            "k_scales": (k_scales, (B, Hkv, (Nk + 31) // 32)),
            "v_scales": (v_scales, (B, Hkv, d))}
    for n, (t, shp) in want.items():
        if t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError(f"{n} must be a contiguous fp32 tensor of shape {shp} on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _check_out("out", out, (B, H, Nq, d), out_dtype, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H, Nq), torch.float32, q.device)
    o = out if out is not None else torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = load().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scales.data_ptr(),
                           k_scales.data_ptr(), v_scales.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           B, H, Hkv, Nq, Nk, d, int(bool(causal)), float(scale), float(p_scale),
                           int(bool(kv_reverse)), _DT[o.dtype], _stream_ptr(stream))
    check(st, "fa_fwd_fp8")
    return o, lse


def kv_tile(dtype: torch.dtype, d: int, pcast: bool = False) -> int:
    return load().fa_kv_tile(_DT[dtype], d, int(bool(pcast)))


def version() -> int:
    return load().fa_version()
