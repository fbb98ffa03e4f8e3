"""Python binding of libmla, the gfx950 paged MLA decode library.

Argument marshalling only: every step of the decode runs in the library's
HIP kernels; torch supplies device memory (``data_ptr()``) and the current
stream.  The function names are those of the C ABI in ``include/libmla.h``.
If ``libmla.so`` has not been built, every call raises ``RuntimeError``:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "libmla.h")

MLA_OK = 0
MLA_ERR_INVALID_VALUE = 1
MLA_ERR_NOT_SUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3FN = 1

ROW_DIM = 576
LATENT_DIM = 512
ROPE_DIM = 64
ROWS_PER_BLOCK = 64     # query rows per workgroup
TILE = 32               # tokens per KV tile
PIECE_COST = 8          # balanced plan: start-up cost of a piece, in tiles


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_name(status)} ({status})")
        self.status = status


class mla_decode_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "num_heads", "kv_lora_rank", "qk_rope_head_dim", "page_size", "num_pages",
        "block_table_stride", "max_seq_len", "kv_dtype")] + [
        ("softmax_scale", ctypes.c_float), ("k_scale", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("num_splits", "min_work_units", "num_cus", "quantize_q_fp8")]


class mla_query_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("nope_token_stride", "nope_head_stride", "rope_token_stride",
                                             "rope_head_stride")]


class mla_rope(ctypes.Structure):
    _fields_ = [("positions", ctypes.c_void_p), ("cos_sin_cache", ctypes.c_void_p), ("max_position", ctypes.c_int32),
                ("is_neox", ctypes.c_int32)]


class mla_kv_append_params(ctypes.Structure):
    _fields_ = [("nope_stride", ctypes.c_int64), ("rope_stride", ctypes.c_int64)] + [
        (n, ctypes.c_int32) for n in ("num_tokens", "kv_lora_rank", "qk_rope_head_dim", "page_size", "num_pages",
                                      "kv_dtype")] + [("k_scale", ctypes.c_float)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libmla.so; raises RuntimeError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmla.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                               "python -m paged_mla_decode_06_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(mla_decode_params)
        vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
        L.mla_abi_version.restype = ctypes.c_int32
        L.mla_abi_version.argtypes = []
        L.mla_status_str.restype = ctypes.c_char_p
        L.mla_status_str.argtypes = [ctypes.c_int32]
        L.mla_decode_workspace_size.restype = ctypes.c_int
        L.mla_decode_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.mla_decode.restype = ctypes.c_int
        L.mla_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.mla_decode_timed.restype = ctypes.c_int
        L.mla_decode_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp, vp]
        L.mla_gather_kv.restype = ctypes.c_int
        L.mla_gather_kv.argtypes = [P, vp, vp, vp, ctypes.c_int32, vp, vp]
        L.mla_plan_host.restype = ctypes.c_int
        L.mla_plan_host.argtypes = [P, vp, vp, ctypes.c_int32, i32p, i32p]
        L.mla_plan_host_ragged.restype = ctypes.c_int
        L.mla_plan_host_ragged.argtypes = [P, vp, vp, ctypes.c_int32, vp, ctypes.c_int32, i32p, i32p, i32p]
        L.mla_plan_device.restype = ctypes.c_int
        L.mla_plan_device.argtypes = [P, vp, vp, ctypes.c_int32, vp, ctypes.c_int32, vp]
        L.mla_check_inputs_host.restype = ctypes.c_int
        L.mla_check_inputs_host.argtypes = [P, vp, vp]
        L.mla_decode_qparts.restype = ctypes.c_int
        L.mla_decode_qparts.argtypes = [P, vp, vp, ctypes.POINTER(mla_query_layout), vp, vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
        L.mla_decode_ragged.restype = ctypes.c_int
        L.mla_decode_ragged.argtypes = [P, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.mla_check_qo_indptr_host.restype = ctypes.c_int
        L.mla_check_qo_indptr_host.argtypes = [P, vp, ctypes.c_int32]
        L.mla_decode_qparts_rope.restype = ctypes.c_int
        L.mla_decode_qparts_rope.argtypes = [P, vp, vp, ctypes.POINTER(mla_query_layout), ctypes.POINTER(mla_rope),
                                             vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.mla_kv_append_rope.restype = ctypes.c_int
        L.mla_kv_append_rope.argtypes = [ctypes.POINTER(mla_kv_append_params), vp, vp, vp, ctypes.POINTER(mla_rope),
                                         vp, vp]
        L.mla_decode_noalloc.restype = ctypes.c_int
        L.mla_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.mla_kv_append.restype = ctypes.c_int
        L.mla_kv_append.argtypes = [ctypes.POINTER(mla_kv_append_params), vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/libmla.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(mla_\w+)\s*\(", text, re.M)))


def mla_abi_version() -> int:
    return int(lib().mla_abi_version())


def status_name(status: int) -> str:
    try:
        return lib().mla_status_str(int(status)).decode()
    except RuntimeError:
        return str(status)


mla_status_str = status_name


def _check(status: int, what: str) -> None:
    if status != MLA_OK:
        raise MlaError(status, what)


def make_params(batch: int, q_len: int, num_heads: int, page_size: int, num_pages: int, block_table_stride: int,
                max_seq_len: int, kv_dtype: int = MLA_KV_BF16, softmax_scale: float = 1.0, k_scale: float = 1.0,
                num_splits: int = 0, min_work_units: int = 0, num_cus: int = 0,
                kv_lora_rank: int = LATENT_DIM, qk_rope_head_dim: int = ROPE_DIM,
                quantize_q_fp8: int = 0) -> mla_decode_params:
    return mla_decode_params(int(batch), int(q_len), int(num_heads), int(kv_lora_rank), int(qk_rope_head_dim),
                             int(page_size), int(num_pages), int(block_table_stride), int(max_seq_len),
                             int(kv_dtype), float(softmax_scale), float(k_scale), int(num_splits),
                             int(min_work_units), int(num_cus), int(quantize_q_fp8))


def params_for(q, kv_pool, block_table, max_seq_len: int, softmax_scale: float, k_scale: float = 1.0,
               num_splits: int = 0, min_work_units: int = 0, num_cus: int = 0,
               quantize_q_fp8: bool = False) -> mla_decode_params:
    """Parameters read off the tensor shapes of a decode call."""
    import torch
    B, ql, H, D = q.shape
    assert D == ROW_DIM, "query rows must be 576 wide"
    N, P, Dk = kv_pool.shape
    assert Dk == ROW_DIM, "pool rows must be 576 wide"
    fp8 = kv_pool.dtype in (torch.float8_e4m3fn, torch.uint8)
    return make_params(B, ql, H, P, N, block_table.stride(0) if block_table.dim() == 2 else 1, max_seq_len,
                       MLA_KV_FP8_E4M3FN if fp8 else MLA_KV_BF16, softmax_scale, k_scale, num_splits,
                       min_work_units, num_cus, quantize_q_fp8=int(bool(quantize_q_fp8)))


def mla_decode_workspace_size(p: mla_decode_params) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)), "mla_decode_workspace_size")
    return int(n.value)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else int(t.data_ptr()))


def alloc_workspace(p: mla_decode_params, device="cuda"):
    """A workspace tensor of the size mla_decode needs (torch allocates it)."""
    import torch
    n = mla_decode_workspace_size(p)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _check_decode_shapes(B: int, q_len: int, H: int, kv_pool, block_table, seq_lens, out, lse, max_seq_len: int,
                         out_shape, lse_shape):
    """Shape checks of a decode call, before any device work: the library
    takes plain pointers, so a tensor smaller than the sizes the parameters
    imply would be read or written past its end."""
    import torch
    if kv_pool.dim() != 3 or kv_pool.shape[-1] != ROW_DIM:
        raise ValueError("kv_pool must be [num_pages, page_size, 576]")
    if kv_pool.dtype not in (torch.bfloat16, torch.float8_e4m3fn, torch.uint8):
        raise ValueError("kv_pool must be bfloat16, or float8_e4m3fn (or uint8 holding e4m3fn codes)")
    if tuple(out.shape) != tuple(out_shape):
        raise ValueError(f"out must be {list(out_shape)}, got {list(out.shape)}")
    if lse is not None and tuple(lse.shape) != tuple(lse_shape):
        raise ValueError(f"lse must be {list(lse_shape)}, got {list(lse.shape)}")
    if seq_lens.numel() != B:
        raise ValueError(f"seq_lens must hold {B} lengths, got {seq_lens.numel()}")
    P = kv_pool.shape[1]
    need = -(-int(max_seq_len) // P) if P > 0 else 0
    if block_table.dim() != 2 or block_table.shape[0] < B or block_table.shape[1] < need:
        raise ValueError(f"block_table must be [B, W] with at least {B} rows and W >= ceil(max_seq_len / "
                         f"page_size) = {need}, got {list(block_table.shape)}")


def mla_decode(q, kv_pool, block_table, seq_lens, out, lse=None, workspace=None, *, max_seq_len: int,
               softmax_scale: float, k_scale: float = 1.0, num_splits: int = 0, min_work_units: int = 0,
               stream=None, params: Optional[mla_decode_params] = None, quantize_q_fp8: bool = False):
    """Enqueue the decode on ``stream`` (default: torch's current stream).

    q [B, q_len, H, 576] bf16; kv_pool [N, P, 576] bf16 or float8_e4m3fn;
    block_table int32 [B, W]; seq_lens int32 [B]; out [B, q_len, H, 512]
    bf16; lse fp32 [B, q_len, H] or None; workspace uint8 (allocated here when
    None).  All on the GPU, contiguous.  Returns (out, lse)."""
    import torch
    if q.dim() != 4 or q.shape[-1] != ROW_DIM:
        raise ValueError("q must be [B, q_len, H, 576]")
    B, ql, H, _ = q.shape
    _check_decode_shapes(B, ql, H, kv_pool, block_table, seq_lens, out, lse, max_seq_len, (B, ql, H, LATENT_DIM),
                         (B, ql, H))
    for name, t in (("q", q), ("kv_pool", kv_pool), ("block_table", block_table), ("seq_lens", seq_lens),
                    ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if not (q.is_contiguous() and kv_pool.is_contiguous() and out.is_contiguous() and seq_lens.is_contiguous()):
        raise ValueError("q, kv_pool, seq_lens and out must be contiguous")
    if block_table.stride(-1) != 1:
        raise ValueError("block_table rows must be contiguous")
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32")
    p = params if params is not None else params_for(q, kv_pool, block_table, max_seq_len, softmax_scale, k_scale,
                                                     num_splits, min_work_units, quantize_q_fp8=quantize_q_fp8)
    if workspace is None:
        workspace = alloc_workspace(p, q.device)
    st = lib().mla_decode(ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens), _ptr(out),
                          _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                          _stream_handle(stream))
    _check(st, "mla_decode")
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20   # MLA_NOALLOC_SCRATCH_BYTES


def mla_decode_noalloc(q, kv_pool, block_table, seq_lens, out, lse=None, *, max_seq_len: int,
                       softmax_scale: float, k_scale: float = 1.0, num_splits: int = 0, min_work_units: int = 0,
                       stream=None, params: Optional[mla_decode_params] = None, quantize_q_fp8: bool = False):
    """mla_decode with the library's own per-device workspace array: nothing
    is allocated, here or in the library (for graph capture and loops that
    cannot allocate).  Calls that overlap on one device race on that array.
    Same tensors and checks as mla_decode.  Returns (out, lse)."""
    import torch
    if q.dim() != 4 or q.shape[-1] != ROW_DIM:
        raise ValueError("q must be [B, q_len, H, 576]")
    B, ql, H, _ = q.shape
    _check_decode_shapes(B, ql, H, kv_pool, block_table, seq_lens, out, lse, max_seq_len, (B, ql, H, LATENT_DIM),
                         (B, ql, H))
    for name, t in (("q", q), ("kv_pool", kv_pool), ("block_table", block_table), ("seq_lens", seq_lens),
                    ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if not (q.is_contiguous() and kv_pool.is_contiguous() and out.is_contiguous() and seq_lens.is_contiguous()):
        raise ValueError("q, kv_pool, seq_lens and out must be contiguous")
    if block_table.stride(-1) != 1:
        raise ValueError("block_table rows must be contiguous")
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32")
    p = params if params is not None else params_for(q, kv_pool, block_table, max_seq_len, softmax_scale, k_scale,
                                                     num_splits, min_work_units, quantize_q_fp8=quantize_q_fp8)
    st = lib().mla_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens),
                                  _ptr(out), _ptr(lse), _stream_handle(stream))
    _check(st, "mla_decode_noalloc")
    return out, lse


def _token_head_strides(t, B: int, q_len: int, H: int, width: int, name: str):
    """(token stride, head stride) of a query part given as [B, q_len, H, width]
    or [B*q_len, H, width] with contiguous elements."""
    if t.stride(-1) != 1 or t.shape[-1] != width:
        raise ValueError(f"{name}: last dimension must be {width} contiguous elements")
    if t.dim() == 4:
        if tuple(t.shape[:3]) != (B, q_len, H) or (B > 1 and t.stride(0) != q_len * t.stride(1)):
            raise ValueError(f"{name}: [B, q_len, H, {width}] with token rows b*q_len + j evenly strided")
        return t.stride(1), t.stride(2)
    if t.dim() == 3 and tuple(t.shape[:2]) == (B * q_len, H):
        return t.stride(0), t.stride(1)
    raise ValueError(f"{name}: expected [B, q_len, H, {width}] or [B*q_len, H, {width}]")


def _rope_struct(positions, cos_sin_cache, is_neox: bool):
    """mla_rope for GPU tensors positions (int64 [tokens]) and cos_sin_cache
    (float32 [max_position, 64], contiguous)."""
    import torch
    if positions.dtype != torch.int64 or not positions.is_contiguous() or not positions.is_cuda:
        raise ValueError("positions must be a contiguous int64 GPU tensor")
    if (cos_sin_cache.dtype != torch.float32 or not cos_sin_cache.is_contiguous() or not cos_sin_cache.is_cuda
            or cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != 64):
        raise ValueError("cos_sin_cache must be a contiguous float32 [max_position, 64] GPU tensor")
    return mla_rope(int(positions.data_ptr()), int(cos_sin_cache.data_ptr()), int(cos_sin_cache.shape[0]),
                    1 if is_neox else 0)


def mla_decode_qparts(q_nope, q_rope, kv_pool, block_table, seq_lens, out, lse=None, workspace=None, *,
                      max_seq_len: int, softmax_scale: float, k_scale: float = 1.0, num_splits: int = 0,
                      min_work_units: int = 0, stream=None, positions=None, cos_sin_cache=None,
                      is_neox: bool = True, quantize_q_fp8: bool = False):
    """mla_decode with the query as its latent part q_nope (512 wide) and rope
    part q_rope (64 wide), each [B, q_len, H, w] or [B*q_len, H, w] with any
    token and head strides (multiples of 8 elements): read in place, no
    concatenation.  out [B, q_len, H, 512] fixes B, q_len and H.  With
    positions (int64 [B*q_len]) and cos_sin_cache (float32 [max_pos, 64]) the
    rope part is first turned by the rotary embedding (mla_decode_qparts_rope)."""
    import torch
    if out.dim() != 4 or out.shape[-1] != LATENT_DIM:
        raise ValueError("out must be [B, q_len, H, 512]")
    B, ql, H, _ = out.shape
    _check_decode_shapes(B, ql, H, kv_pool, block_table, seq_lens, out, lse, max_seq_len, (B, ql, H, LATENT_DIM),
                         (B, ql, H))
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("kv_pool", kv_pool), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if q_nope.dtype != torch.bfloat16 or q_rope.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q_nope, q_rope and out must be bfloat16")
    if not (kv_pool.is_contiguous() and out.is_contiguous() and seq_lens.is_contiguous()):
        raise ValueError("kv_pool, seq_lens and out must be contiguous")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or block_table.stride(-1) != 1:
        raise ValueError("block_table and seq_lens must be int32 with contiguous rows")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32")
    B, ql, H, Dv = out.shape
    if Dv != LATENT_DIM:
        raise ValueError("out must be [B, q_len, H, 512]")
    nt, nh = _token_head_strides(q_nope, B, ql, H, LATENT_DIM, "q_nope")
    rt, rh = _token_head_strides(q_rope, B, ql, H, ROPE_DIM, "q_rope")
    N, P, Dk = kv_pool.shape
    fp8 = kv_pool.dtype in (torch.float8_e4m3fn, torch.uint8)
    p = make_params(B, ql, H, P, N, block_table.stride(0) if block_table.dim() == 2 else 1, max_seq_len,
                    MLA_KV_FP8_E4M3FN if fp8 else MLA_KV_BF16, softmax_scale, k_scale, num_splits, min_work_units,
                    quantize_q_fp8=int(bool(quantize_q_fp8)))
    if workspace is None:
        workspace = alloc_workspace(p, out.device)
    lay = mla_query_layout(int(nt), int(nh), int(rt), int(rh))
    wsb = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    if cos_sin_cache is not None:
        if positions is None or positions.numel() != B * ql:
            raise ValueError("positions must hold one position per query token (B * q_len)")
        r = _rope_struct(positions, cos_sin_cache, is_neox)
        st = lib().mla_decode_qparts_rope(ctypes.byref(p), _ptr(q_nope), _ptr(q_rope), ctypes.byref(lay),
                                          ctypes.byref(r), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens),
                                          _ptr(out), _ptr(lse), _ptr(workspace), wsb, _stream_handle(stream))
        _check(st, "mla_decode_qparts_rope")
        return out, lse
    st = lib().mla_decode_qparts(ctypes.byref(p), _ptr(q_nope), _ptr(q_rope), ctypes.byref(lay), _ptr(kv_pool),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
                                 _stream_handle(stream))
    _check(st, "mla_decode_qparts")
    return out, lse


def mla_decode_ragged(q, qo_indptr, kv_pool, block_table, seq_lens, out, lse=None, workspace=None, *,
                      max_q_len: int, max_seq_len: int, softmax_scale: float, k_scale: float = 1.0,
                      num_splits: int = 0, min_work_units: int = 0, stream=None,
                      params: Optional[mla_decode_params] = None, validate: bool = False,
                      quantize_q_fp8: bool = False):
    """Ragged multi-token decode: request b's query tokens are rows
    qo_indptr[b] .. qo_indptr[b+1]-1 of the packed q [T, H, 576] bf16
    (qo_indptr int32 [B+1] on the GPU, at most max_q_len per request); out
    [T, H, 512] bf16, lse [T, H] fp32 or None.  Returns (out, lse).

    The library trusts the offsets on the device: a request whose offsets
    fall outside [0, T] or run backwards gets no query token, and a request
    with more than max_q_len tokens only its first max_q_len; the out/lse
    rows of the tokens left out are not written.  validate=True copies the
    offsets to the host first (a synchronisation) and raises MlaError
    (MLA_ERR_INVALID_VALUE) unless they pass mla_check_qo_indptr_host."""
    import torch
    if q.dim() != 3 or q.shape[-1] != ROW_DIM:
        raise ValueError("q must be [T, H, 576]")
    T, H, _ = q.shape
    _check_decode_shapes(seq_lens.numel(), max_q_len, H, kv_pool, block_table, seq_lens, out, lse, max_seq_len,
                         (T, H, LATENT_DIM), (T, H))
    if qo_indptr.numel() != seq_lens.numel() + 1:
        raise ValueError("qo_indptr must hold B+1 offsets")
    for name, t in (("q", q), ("qo_indptr", qo_indptr), ("kv_pool", kv_pool), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if not (q.is_contiguous() and kv_pool.is_contiguous() and out.is_contiguous() and seq_lens.is_contiguous()
            and qo_indptr.is_contiguous()):
        raise ValueError("q, qo_indptr, kv_pool, seq_lens and out must be contiguous")
    if q.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16")
    if qo_indptr.dtype != torch.int32 or block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("qo_indptr, block_table and seq_lens must be int32")
    if block_table.stride(-1) != 1:
        raise ValueError("block_table rows must be contiguous")
    T, H, D = q.shape
    if D != ROW_DIM or tuple(out.shape) != (T, H, LATENT_DIM):
        raise ValueError("q must be [T, H, 576] and out [T, H, 512]")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (T, H)):
        raise ValueError("lse must be contiguous float32 [T, H]")
    B = seq_lens.numel()
    if qo_indptr.numel() != B + 1:
        raise ValueError("qo_indptr must hold B+1 offsets")
    N, P, Dk = kv_pool.shape
    fp8 = kv_pool.dtype in (torch.float8_e4m3fn, torch.uint8)
    p = params if params is not None else make_params(
        B, max_q_len, H, P, N, block_table.stride(0) if block_table.dim() == 2 else 1, max_seq_len,
        MLA_KV_FP8_E4M3FN if fp8 else MLA_KV_BF16, softmax_scale, k_scale, num_splits, min_work_units,
        quantize_q_fp8=int(bool(quantize_q_fp8)))
    if validate:
        ind_host = qo_indptr.cpu().numpy()
        _check(mla_check_qo_indptr_host(p, ind_host, T), "mla_decode_ragged: qo_indptr")
    if workspace is None:
        workspace = alloc_workspace(p, q.device)
    st = lib().mla_decode_ragged(ctypes.byref(p), _ptr(q), _ptr(qo_indptr), int(T), _ptr(kv_pool),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                                 ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                 _stream_handle(stream))
    _check(st, "mla_decode_ragged")
    return out, lse


def mla_check_qo_indptr_host(p: mla_decode_params, qo_indptr_host: np.ndarray, total_q_tokens: int) -> int:
    a = np.ascontiguousarray(qo_indptr_host, dtype=np.int32)
    return int(lib().mla_check_qo_indptr_host(ctypes.byref(p), a.ctypes.data_as(ctypes.c_void_p),
                                              int(total_q_tokens)))


def mla_decode_timed(p: mla_decode_params, q, kv_pool, block_table, seq_lens, out, lse, workspace, stream,
                     ev_start, ev_split_done, ev_end):
    """mla_decode with raw hipEvent_t handles (ints, or None) recorded around the two kernels."""
    st = lib().mla_decode_timed(ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens),
                                _ptr(out), _ptr(lse), _ptr(workspace),
                                ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                _stream_handle(stream), ctypes.c_void_p(ev_start), ctypes.c_void_p(ev_split_done),
                                ctypes.c_void_p(ev_end))
    _check(st, "mla_decode_timed")


def mla_gather_kv(p: mla_decode_params, kv_pool, block_table, seq_lens, b: int, dst, stream=None):
    _check(lib().mla_gather_kv(ctypes.byref(p), _ptr(kv_pool), _ptr(block_table), _ptr(seq_lens), int(b),
                               _ptr(dst), _stream_handle(stream)), "mla_gather_kv")
    return dst


def mla_plan_host(p: mla_decode_params, seq_lens_host: np.ndarray) -> Tuple[np.ndarray, int]:
    """The work plan as int32 rows (g, b, row_block, tile_begin, tile_end, slot), and the grid size."""
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    n = ctypes.c_int32(0)
    grid = ctypes.c_int32(0)
    st = lib().mla_plan_host(ctypes.byref(p), sl.ctypes.data_as(ctypes.c_void_p), None, 0, ctypes.byref(n),
                             ctypes.byref(grid))
    if st not in (MLA_OK, MLA_ERR_INVALID_VALUE) or (st == MLA_ERR_INVALID_VALUE and n.value == 0 and p.batch > 0):
        _check(st, "mla_plan_host")
    cap = max(n.value, 1)
    pieces = np.zeros((cap, 6), dtype=np.int32)
    _check(lib().mla_plan_host(ctypes.byref(p), sl.ctypes.data_as(ctypes.c_void_p),
                               pieces.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n), ctypes.byref(grid)),
           "mla_plan_host")
    return pieces[:n.value], int(grid.value)


def mla_plan_host_ragged(p: mla_decode_params, seq_lens_host: np.ndarray, qo_indptr_host: np.ndarray,
                         total_q_tokens: int) -> Tuple[np.ndarray, int, bool]:
    """The plan of a ragged batch: int32 rows (g, b, row_block, tile_begin, tile_end, slot), the
    grid size, and whether the row-block class plan was used."""
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    qi = np.ascontiguousarray(qo_indptr_host, dtype=np.int32)
    n, grid, used = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    args = (ctypes.byref(p), sl.ctypes.data_as(ctypes.c_void_p), qi.ctypes.data_as(ctypes.c_void_p),
            int(total_q_tokens))
    st = lib().mla_plan_host_ragged(*args, None, 0, ctypes.byref(n), ctypes.byref(grid), ctypes.byref(used))
    if st not in (MLA_OK, MLA_ERR_INVALID_VALUE) or (st == MLA_ERR_INVALID_VALUE and n.value == 0 and p.batch > 0):
        _check(st, "mla_plan_host_ragged")
    cap = max(n.value, 1)
    pieces = np.zeros((cap, 6), dtype=np.int32)
    _check(lib().mla_plan_host_ragged(*args, pieces.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n),
                                      ctypes.byref(grid), ctypes.byref(used)), "mla_plan_host_ragged")
    return pieces[:n.value], int(grid.value), bool(used.value)


def mla_plan_device(p: mla_decode_params, seq_lens_dev, grid: int, max_per_wg: int, stream=None):
    """The plan as the decode kernel computes it: (pieces [grid, max_per_wg, 6], counts [grid]) on the GPU."""
    import torch
    pieces = torch.full((grid, max_per_wg, 6), -7, dtype=torch.int32, device=seq_lens_dev.device)
    counts = torch.zeros(grid, dtype=torch.int32, device=seq_lens_dev.device)
    _check(lib().mla_plan_device(ctypes.byref(p), _ptr(seq_lens_dev), _ptr(pieces), int(max_per_wg), _ptr(counts),
                                 int(grid), _stream_handle(stream)), "mla_plan_device")
    return pieces, counts


def mla_check_inputs_host(p: mla_decode_params, block_table_host: np.ndarray, seq_lens_host: np.ndarray) -> int:
    bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    return int(lib().mla_check_inputs_host(ctypes.byref(p), bt.ctypes.data_as(ctypes.c_void_p),
                                           sl.ctypes.data_as(ctypes.c_void_p)))


def make_append_params(num_tokens: int, page_size: int, num_pages: int, kv_dtype: int = MLA_KV_BF16,
                       k_scale: float = 1.0, nope_stride: int = LATENT_DIM, rope_stride: int = ROPE_DIM,
                       kv_lora_rank: int = LATENT_DIM, qk_rope_head_dim: int = ROPE_DIM) -> mla_kv_append_params:
    return mla_kv_append_params(int(nope_stride), int(rope_stride), int(num_tokens), int(kv_lora_rank),
                                int(qk_rope_head_dim), int(page_size), int(num_pages), int(kv_dtype), float(k_scale))


def mla_kv_append(k_nope, k_rope, out_cache_loc, kv_pool, *, k_scale: float = 1.0, stream=None,
                  params: Optional[mla_kv_append_params] = None, positions=None, cos_sin_cache=None,
                  is_neox: bool = True):
    """Enqueue the cache write of T new rows on ``stream`` (default: torch's current stream).

    k_nope [T, 512] and k_rope [T, 64] bf16 (rows may be strided, e.g. the two
    slices of one [T, 576] tensor; elements contiguous); out_cache_loc int64
    [T] flat slots page * page_size + slot; kv_pool [N, P, 576] bf16 or
    float8_e4m3fn (written).  All on the GPU.  Returns kv_pool."""
    import torch
    for name, t in (("k_nope", k_nope), ("k_rope", k_rope), ("out_cache_loc", out_cache_loc), ("kv_pool", kv_pool)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if k_nope.dtype != torch.bfloat16 or k_rope.dtype != torch.bfloat16:
        raise ValueError("k_nope and k_rope must be bfloat16")
    if out_cache_loc.dtype != torch.int64 or not out_cache_loc.is_contiguous():
        raise ValueError("out_cache_loc must be contiguous int64")
    if k_nope.dim() != 2 or k_rope.dim() != 2 or k_nope.shape[1] != LATENT_DIM or k_rope.shape[1] != ROPE_DIM:
        raise ValueError("k_nope must be [T, 512] and k_rope [T, 64]")
    if k_nope.stride(1) != 1 or k_rope.stride(1) != 1 or not kv_pool.is_contiguous():
        raise ValueError("row elements must be contiguous, and the pool contiguous")
    T = k_nope.shape[0]
    if k_rope.shape[0] != T or out_cache_loc.numel() != T:
        raise ValueError("k_nope, k_rope and out_cache_loc must have the same number of rows")
    N, P, D = kv_pool.shape
    if D != ROW_DIM:
        raise ValueError("pool rows must be 576 wide")
    fp8 = kv_pool.dtype in (torch.float8_e4m3fn, torch.uint8)
    p = params if params is not None else make_append_params(
        T, P, N, MLA_KV_FP8_E4M3FN if fp8 else MLA_KV_BF16, k_scale,
        k_nope.stride(0) if T > 1 else LATENT_DIM, k_rope.stride(0) if T > 1 else ROPE_DIM)
    if cos_sin_cache is not None:
        if positions is None or positions.numel() != T:
            raise ValueError("positions must hold one position per row")
        r = _rope_struct(positions, cos_sin_cache, is_neox)
        _check(lib().mla_kv_append_rope(ctypes.byref(p), _ptr(k_nope), _ptr(k_rope), _ptr(out_cache_loc),
                                        ctypes.byref(r), _ptr(kv_pool), _stream_handle(stream)), "mla_kv_append_rope")
        return kv_pool
    _check(lib().mla_kv_append(ctypes.byref(p), _ptr(k_nope), _ptr(k_rope), _ptr(out_cache_loc), _ptr(kv_pool),
                               _stream_handle(stream)), "mla_kv_append")
    return kv_pool


def append_work(num_tokens: int, kv_bytes: int) -> int:
    """Bytes a KV append must move: each row's 576 bf16 inputs read, its 576
    pool elements written, and its 8-byte location read."""
    return int(num_tokens) * (ROW_DIM * 2 + ROW_DIM * kv_bytes + 8)


def algorithmic_work_ragged(seq_lens: np.ndarray, q_lens: np.ndarray, heads: int, page_size: int, kv_bytes: int):
    """(bytes, flops) of a ragged decode: as algorithmic_work, with request b's
    own q_b query tokens (vis(j) = L_b - q_b + 1 + j)."""
    L = np.maximum(np.asarray(seq_lens, dtype=np.int64), 0)
    qb = np.asarray(q_lens, dtype=np.int64)
    n_pages = (L + page_size - 1) // page_size
    rows = int(qb.sum()) * heads
    nbytes = int(L.sum()) * ROW_DIM * kv_bytes + rows * (ROW_DIM * 2 + LATENT_DIM * 2 + 4) \
        + 4 * int(n_pages.sum()) + 4 * L.shape[0] + 4 * (L.shape[0] + 1)
    vis = sum(int(np.maximum(L[b] - qb[b] + 1 + np.arange(qb[b]), 0).sum()) for b in range(L.shape[0]))
    return nbytes, 2 * heads * (ROW_DIM + LATENT_DIM) * vis


def algorithmic_work(seq_lens: np.ndarray, q_len: int, heads: int, page_size: int, kv_bytes: int):
    """(bytes, flops) a decode call must move / compute: every visible KV row
    once, Q in, O and LSE out, the block-table entries read and seq_lens;
    QK^T over 576 dims plus P.V over 512 dims for each unmasked (row, token)."""
    L = np.maximum(np.asarray(seq_lens, dtype=np.int64), 0)
    B = L.shape[0]
    n_pages = (L + page_size - 1) // page_size
    nbytes = int(L.sum()) * ROW_DIM * kv_bytes + B * q_len * heads * (ROW_DIM * 2 + LATENT_DIM * 2 + 4) \
        + 4 * int(n_pages.sum()) + 4 * B
    vis = np.maximum(L[:, None] - q_len + 1 + np.arange(q_len)[None, :], 0)
    flops = 2 * heads * (ROW_DIM + LATENT_DIM) * int(vis.sum())
    return nbytes, flops
