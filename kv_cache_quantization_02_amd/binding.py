"""ctypes binding of libtq.so (include/tq.h), with the same entry-point names.

Only argument marshalling happens here: torch supplies device memory and the
current HIP stream; every step of the codec runs in the library's kernels.
There is no fallback: if libtq.so cannot be loaded the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_OK = 0
PLANES = ("k_q", "k_scale", "k_zero", "v_q", "v_scale")


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class Scheme(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32)]


class Planes(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in PLANES]


class Rows(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("n_seq", "n_tok", "n_head", "seq_stride", "tok_stride", "head_stride")]


class DenseScheme(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32), ("qjl", ctypes.c_int32)]


DENSE_PLANES = ("idx", "norm", "qjl", "gamma")


class DensePlanes(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in DENSE_PLANES]


_lib = None
# the same sources built with every kernel's bounds tests (TQ_CHECK)
CHECKED_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq_check.so")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load(_LIB_PATH)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """The library at `path` (libtq.so or libtq_check.so) with every entry
    point's argument types set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m kv_cache_quantization_02_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    L.tq_check_scheme.argtypes = [P(Scheme)]
    L.tq_check_scheme.restype = ctypes.c_int32
    L.tq_plane_row_bytes.argtypes = [P(Scheme), ctypes.c_int32]
    L.tq_plane_row_bytes.restype = ctypes.c_int64
    L.tq_row_bytes.argtypes = [P(Scheme)]
    L.tq_row_bytes.restype = ctypes.c_int64
    L.tq_codebook.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.tq_codebook.restype = ctypes.c_int32
    L.tq_quantize_kv.argtypes = [P(Scheme), ctypes.c_void_p, ctypes.c_void_p, P(Rows),
                                 ctypes.c_void_p, P(Planes), P(Rows), ctypes.c_void_p]
    L.tq_quantize_kv.restype = ctypes.c_int32
    L.tq_dequantize_kv.argtypes = [P(Scheme), P(Planes), P(Rows), ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, P(Rows), ctypes.c_void_p]
    L.tq_dequantize_kv.restype = ctypes.c_int32
    L.tq_append_kv.argtypes = [P(Scheme), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_void_p, P(Planes), ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.tq_append_kv.restype = ctypes.c_int32
    L.tq_fetch_kv.argtypes = [P(Scheme), P(Planes), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                              ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                              ctypes.c_void_p]
    L.tq_fetch_kv.restype = ctypes.c_int32
    L.tq_grown_capacity.argtypes = [ctypes.c_int64]
    L.tq_grown_capacity.restype = ctypes.c_int64
    L.tq_grow_kv.argtypes = [P(Scheme), ctypes.c_int32, ctypes.c_int32, P(Planes), ctypes.c_int64,
                             ctypes.c_int64, ctypes.c_int32, P(Planes), ctypes.c_int64, ctypes.c_int64,
                             ctypes.c_int32, ctypes.c_void_p]
    L.tq_grow_kv.restype = ctypes.c_int32
    L.tq_unrotate_rows.argtypes = [ctypes.c_int32, ctypes.c_void_p, P(Rows), ctypes.c_void_p, ctypes.c_void_p,
                                   P(Rows), ctypes.c_void_p]
    L.tq_unrotate_rows.restype = ctypes.c_int32
    L.tq_decode_attn_workspace_bytes.argtypes = [P(Scheme), ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_int32]
    L.tq_decode_attn_workspace_bytes.restype = ctypes.c_size_t
    L.tq_decode_attn_quant.argtypes = [
        P(Scheme), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(Planes),
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.tq_decode_attn_quant.restype = ctypes.c_int32
    L.tq_attn_quant_workspace_bytes.argtypes = [P(Scheme), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32]
    L.tq_attn_quant_workspace_bytes.restype = ctypes.c_size_t
    L.tq_attn_quant.argtypes = [
        P(Scheme), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(Planes),
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.tq_attn_quant.restype = ctypes.c_int32
    L.tq_attn_quant_noalloc.argtypes = [
        P(Scheme), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(Planes),
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.tq_attn_quant_noalloc.restype = ctypes.c_int32
    L.tq_dense_check_scheme.argtypes = [P(DenseScheme)]
    L.tq_dense_check_scheme.restype = ctypes.c_int32
    L.tq_dense_plane_row_bytes.argtypes = [P(DenseScheme), ctypes.c_int32]
    L.tq_dense_plane_row_bytes.restype = ctypes.c_int64
    L.tq_dense_quantize.argtypes = [P(DenseScheme), ctypes.c_void_p, P(Rows), ctypes.c_void_p, ctypes.c_void_p,
                                    P(DensePlanes), P(Rows), ctypes.c_void_p]
    L.tq_dense_quantize.restype = ctypes.c_int32
    L.tq_dense_dequantize.argtypes = [P(DenseScheme), P(DensePlanes), P(Rows), ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, P(Rows), ctypes.c_void_p]
    L.tq_dense_dequantize.restype = ctypes.c_int32
    L.tq_status_string.argtypes = [ctypes.c_int32]
    L.tq_status_string.restype = ctypes.c_char_p
    L.tq_check_flags.argtypes = []
    L.tq_check_flags.restype = ctypes.c_int64
    L.tq_check_set_margin.argtypes = [ctypes.c_int64]
    L.tq_check_set_margin.restype = ctypes.c_int64
    return L


class checked_library:
    """Context manager: within it every call of this module goes to
    libtq_check.so (the bounds-checked build); the library in use before
    comes back on exit."""

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = load(CHECKED_LIB_PATH)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def tq_check_flags() -> int:
    """Bounds-test flag bits set since the last call (checked build; -1 otherwise)."""
    return lib().tq_check_flags()


def tq_check_set_margin(margin: int) -> int:
    return lib().tq_check_set_margin(margin)


def status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream
    if torch.cuda.is_available() and torch.cuda.is_initialized():
        return torch.cuda.current_stream().cuda_stream
    return None


# ----------------------------------------------------------------- raw C ABI
def tq_check_scheme(scheme: Scheme) -> int:
    return lib().tq_check_scheme(ctypes.byref(scheme))


def tq_plane_row_bytes(scheme: Scheme, plane: int) -> int:
    return lib().tq_plane_row_bytes(ctypes.byref(scheme), plane)


def tq_row_bytes(scheme: Scheme) -> int:
    return lib().tq_row_bytes(ctypes.byref(scheme))


def tq_codebook(bits: int):
    import numpy as np
    c = np.zeros(1 << bits, np.float32)
    b = np.zeros((1 << bits) - 1, np.float32)
    _check(lib().tq_codebook(bits, c.ctypes.data, b.ctypes.data), "tq_codebook")
    return c, b


def tq_quantize_kv(scheme, k, v, in_rows, signs, out, out_rows, stream=None) -> int:
    return lib().tq_quantize_kv(ctypes.byref(scheme), _ptr(k), _ptr(v), ctypes.byref(in_rows),
                                _ptr(signs), ctypes.byref(out), ctypes.byref(out_rows), _stream(stream))


def tq_append_kv(scheme, k, v, batch, n_new, n_kv_heads, signs, cache, seq_stride_rows, head_stride_rows,
                 positions, capacity, stream=None) -> int:
    return lib().tq_append_kv(ctypes.byref(scheme), _ptr(k), _ptr(v), batch, n_new, n_kv_heads, _ptr(signs),
                              ctypes.byref(cache), seq_stride_rows, head_stride_rows, _ptr(positions),
                              capacity, _stream(stream))


def tq_fetch_kv(scheme, cache, batch, n_kv_heads, seq_stride_rows, head_stride_rows, capacity, lens, window,
                signs, values_rotated, k_out, v_out, stream=None) -> int:
    return lib().tq_fetch_kv(ctypes.byref(scheme), ctypes.byref(cache), batch, n_kv_heads, seq_stride_rows,
                             head_stride_rows, capacity, _ptr(lens), window, _ptr(signs), int(values_rotated),
                             _ptr(k_out), _ptr(v_out), _stream(stream))


def tq_grown_capacity(tokens: int) -> int:
    return lib().tq_grown_capacity(tokens)


def tq_grow_kv(scheme, batch, n_kv_heads, src, src_seq_stride_rows, src_head_stride_rows, src_capacity, dst,
               dst_seq_stride_rows, dst_head_stride_rows, dst_capacity, stream=None) -> int:
    return lib().tq_grow_kv(ctypes.byref(scheme), batch, n_kv_heads, ctypes.byref(src), src_seq_stride_rows,
                            src_head_stride_rows, src_capacity, ctypes.byref(dst), dst_seq_stride_rows,
                            dst_head_stride_rows, dst_capacity, _stream(stream))


def tq_unrotate_rows(head_dim, x, in_rows, signs, out, out_rows, stream=None) -> int:
    return lib().tq_unrotate_rows(head_dim, _ptr(x), ctypes.byref(in_rows), _ptr(signs), _ptr(out),
                                  ctypes.byref(out_rows), _stream(stream))


def tq_dequantize_kv(scheme, planes, in_rows, signs, k_out, v_out, out_rows, stream=None) -> int:
    return lib().tq_dequantize_kv(ctypes.byref(scheme), ctypes.byref(planes), ctypes.byref(in_rows),
                                  _ptr(signs), _ptr(k_out), _ptr(v_out), ctypes.byref(out_rows),
                                  _stream(stream))


def tq_decode_attn_workspace_bytes(scheme, batch, n_q_heads, n_kv_heads, max_ctx) -> int:
    return lib().tq_decode_attn_workspace_bytes(ctypes.byref(scheme), batch, n_q_heads, n_kv_heads, max_ctx)


def tq_decode_attn_quant(scheme, q, batch, n_q_heads, n_kv_heads, cache, seq_stride_rows,
                         head_stride_rows, ctx_lens, max_ctx, softmax_scale, signs, out,
                         workspace, workspace_bytes, stream=None) -> int:
    return lib().tq_decode_attn_quant(
        ctypes.byref(scheme), _ptr(q), batch, n_q_heads, n_kv_heads, ctypes.byref(cache),
        seq_stride_rows, head_stride_rows, _ptr(ctx_lens), max_ctx, softmax_scale, _ptr(signs),
        _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream))


# ------------------------------------------------------- torch conveniences
def scheme(head_dim: int, k_bits: int, v_bits: int) -> Scheme:
    return Scheme(head_dim, k_bits, v_bits)


def rows(n_seq, n_tok, n_head, seq_stride, tok_stride, head_stride) -> Rows:
    return Rows(n_seq, n_tok, n_head, seq_stride, tok_stride, head_stride)


def contiguous_rows(shape) -> Rows:
    """Rows of a contiguous [L, T, H, ...] tensor."""
    L, T, H = shape[:3]
    return Rows(L, T, H, T * H, H, 1)


def alloc_planes(sch: Scheme, lead_shape, device) -> dict:
    """Empty planes of shape lead_shape + [row bytes] (fp16 planes as float16)."""
    out = {}
    for i, name in enumerate(PLANES):
        nbytes = tq_plane_row_bytes(sch, i)
        if nbytes < 0:
            raise TQError(nbytes, "tq_plane_row_bytes")
        if name in ("k_q", "v_q"):
            out[name] = torch.empty(tuple(lead_shape) + (nbytes,), dtype=torch.uint8, device=device)
        else:
            out[name] = torch.empty(tuple(lead_shape) + (nbytes // 2,), dtype=torch.float16, device=device)
    return out


def planes_struct(planes: dict) -> Planes:
    return Planes(*[planes[n].data_ptr() for n in PLANES])


def quantize_kv(k: torch.Tensor, v: torch.Tensor, signs: torch.Tensor, k_bits: int, v_bits: int,
                out: dict | None = None) -> dict:
    """Quantize contiguous bf16 [L, T, H, d] K and V into planes [L, T, H, bytes]."""
    assert k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16 and k.shape == v.shape
    assert k.is_contiguous() and v.is_contiguous() and k.dim() == 4
    sch = scheme(k.shape[-1], k_bits, v_bits)
    if out is None:
        out = alloc_planes(sch, k.shape[:3], k.device)
    r = contiguous_rows(k.shape)
    _check(tq_quantize_kv(sch, k, v, r, signs, planes_struct(out), r), "tq_quantize_kv")
    return out


def dequantize_kv(planes: dict, signs: torch.Tensor, head_dim: int, k_bits: int, v_bits: int,
                  k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None,
                  keys: bool = True, values: bool = True):
    """bf16 [L, T, H, d] K and V from contiguous planes [L, T, H, bytes]."""
    sch = scheme(head_dim, k_bits, v_bits)
    lead = planes["k_q"].shape[:3]
    dev = planes["k_q"].device
    if keys and k_out is None:
        k_out = torch.empty(tuple(lead) + (head_dim,), dtype=torch.bfloat16, device=dev)
    if values and v_out is None:
        v_out = torch.empty(tuple(lead) + (head_dim,), dtype=torch.bfloat16, device=dev)
    r = contiguous_rows(tuple(lead))
    _check(tq_dequantize_kv(sch, planes_struct(planes), r, signs, k_out if keys else None,
                            v_out if values else None, r), "tq_dequantize_kv")
    return (k_out if keys else None), (v_out if values else None)


def quantize_into_cache(k: torch.Tensor, v: torch.Tensor, signs: torch.Tensor, k_bits: int,
                        v_bits: int, cache: dict | None = None) -> dict:
    """Quantize bf16 [B, N, Hkv, d] K and V into a cache laid out [B, Hkv, N, bytes]."""
    B, N, H, d = k.shape
    sch = scheme(d, k_bits, v_bits)
    if cache is None:
        cache = alloc_planes(sch, (B, H, N), k.device)
    rin = Rows(B, N, H, N * H, H, 1)
    rout = Rows(B, N, H, H * N, 1, N)
    _check(tq_quantize_kv(sch, k, v, rin, signs, planes_struct(cache), rout), "tq_quantize_kv")
    return cache


def decode_attn(q: torch.Tensor, cache: dict, ctx_lens: torch.Tensor, signs: torch.Tensor,
                k_bits: int, v_bits: int, n_kv_heads: int, softmax_scale: float | None = None,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Fused decode attention; q [B, Hq, d] bf16, cache planes [B, Hkv, N, bytes]."""
    B, Hq, d = q.shape
    N = cache["k_q"].shape[2]
    sch = scheme(d, k_bits, v_bits)
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    ws = tq_decode_attn_workspace_bytes(sch, B, Hq, n_kv_heads, N)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    _check(tq_decode_attn_quant(sch, q, B, Hq, n_kv_heads, planes_struct(cache), n_kv_heads * N, N,
                                ctx_lens, N, float(softmax_scale), signs, out, workspace,
                                workspace.numel()), "tq_decode_attn_quant")
    return out


def append_kv(k: torch.Tensor, v: torch.Tensor, cache: dict, positions: torch.Tensor, signs: torch.Tensor,
              k_bits: int, v_bits: int) -> dict:
    """Append bf16 [B, n_new, Hkv, d] tokens into a cache laid out [B, Hkv, capacity, bytes]
    at device int32 positions [B]; tokens at or past the capacity are dropped."""
    B, n_new, H, d = k.shape
    cap = cache["k_q"].shape[2]
    _check(tq_append_kv(scheme(d, k_bits, v_bits), k, v, B, n_new, H, signs, planes_struct(cache), H * cap, cap,
                        positions, cap), "tq_append_kv")
    return cache


def grow_kv(cache: dict, new_capacity: int, head_dim: int, k_bits: int, v_bits: int) -> dict:
    """A new [B, Hkv, new_capacity, bytes] cache holding the old rows below both
    capacities and zero bytes after them (new planes; the old ones are kept)."""
    B, H, cap = cache["k_q"].shape[:3]
    sch = scheme(head_dim, k_bits, v_bits)
    out = alloc_planes(sch, (B, H, new_capacity), cache["k_q"].device)
    _check(tq_grow_kv(sch, B, H, planes_struct(cache), H * cap, cap, cap, planes_struct(out),
                      H * new_capacity, new_capacity, new_capacity), "tq_grow_kv")
    return out


def fetch_kv(cache: dict, lens: torch.Tensor, window: int, signs: torch.Tensor | None, head_dim: int,
             k_bits: int, v_bits: int, values_rotated: bool = False, keys: bool = True, values: bool = True):
    """bf16 [B, Hkv, window, d] K and V of a [B, Hkv, capacity, bytes] cache; rows t >= min(lens[b],
    capacity) are +0 (the window may be longer than the capacity).
    With values_rotated the V rows stay in the rotated domain (centroid * scale)."""
    B, H, cap = cache["k_q"].shape[:3]
    dev = cache["k_q"].device
    k_out = torch.empty((B, H, window, head_dim), dtype=torch.bfloat16, device=dev) if keys else None
    v_out = torch.empty((B, H, window, head_dim), dtype=torch.bfloat16, device=dev) if values else None
    _check(tq_fetch_kv(scheme(head_dim, k_bits, v_bits), planes_struct(cache), B, H, H * cap, cap, cap, lens,
                       window, signs, values_rotated, k_out, v_out), "tq_fetch_kv")
    return k_out, v_out


def unrotate_rows(x: torch.Tensor, signs: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [..., d] rows in the rotated domain -> signs * FWHT(x) / sqrt(d) (bf16); out may be x."""
    d = x.shape[-1]
    n = x.numel() // d
    if out is None:
        out = torch.empty_like(x)
    r = contiguous_rows((n, 1, 1))
    _check(tq_unrotate_rows(d, x, r, signs, out, r), "tq_unrotate_rows")
    return out


def tq_attn_quant_workspace_bytes(scheme, batch, n_queries, n_q_heads, n_kv_heads, max_ctx) -> int:
    return lib().tq_attn_quant_workspace_bytes(ctypes.byref(scheme), batch, n_queries, n_q_heads, n_kv_heads,
                                               max_ctx)


def tq_attn_quant(scheme, q, batch, n_queries, n_q_heads, n_kv_heads, cache, seq_stride_rows, head_stride_rows,
                  ctx_lens, max_ctx, softmax_scale, signs, out, workspace, workspace_bytes, stream=None) -> int:
    return lib().tq_attn_quant(ctypes.byref(scheme), _ptr(q), batch, n_queries, n_q_heads, n_kv_heads,
                               ctypes.byref(cache), seq_stride_rows, head_stride_rows, _ptr(ctx_lens), max_ctx,
                               softmax_scale, _ptr(signs), _ptr(out), _ptr(workspace), workspace_bytes,
                               _stream(stream))


# Size of the library's device scratch behind tq_attn_quant_noalloc (include/tq.h).
NOALLOC_SCRATCH_BYTES = 16 << 20


def tq_attn_quant_noalloc(scheme, q, batch, n_queries, n_q_heads, n_kv_heads, cache, seq_stride_rows,
                          head_stride_rows, ctx_lens, max_ctx, softmax_scale, signs, out, stream=None) -> int:
    return lib().tq_attn_quant_noalloc(ctypes.byref(scheme), _ptr(q), batch, n_queries, n_q_heads, n_kv_heads,
                                       ctypes.byref(cache), seq_stride_rows, head_stride_rows, _ptr(ctx_lens),
                                       max_ctx, softmax_scale, _ptr(signs), _ptr(out), _stream(stream))


def attn_quant(q: torch.Tensor, cache: dict, ctx_lens: torch.Tensor, signs: torch.Tensor, k_bits: int,
               v_bits: int, n_kv_heads: int, softmax_scale: float | None = None,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Multi-query fused attention; q [B, M, Hq, d] bf16 (query m of sequence b is cached token
    ctx_lens[b] - M + m, causal), cache planes [B, Hkv, N, bytes]; returns [B, M, Hq, d]."""
    B, M, Hq, d = q.shape
    N = cache["k_q"].shape[2]
    sch = scheme(d, k_bits, v_bits)
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    if out is None:
        out = torch.empty((B, M, Hq, d), dtype=torch.bfloat16, device=q.device)
    ws = tq_attn_quant_workspace_bytes(sch, B, M, Hq, n_kv_heads, N)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    _check(tq_attn_quant(sch, q, B, M, Hq, n_kv_heads, planes_struct(cache), n_kv_heads * N, N, ctx_lens, N,
                         float(softmax_scale), signs, out, workspace, workspace.numel()), "tq_attn_quant")
    return out


# -------------------------------------------------------------- paper variant
def tq_dense_check_scheme(scheme: DenseScheme) -> int:
    return lib().tq_dense_check_scheme(ctypes.byref(scheme))


def tq_dense_plane_row_bytes(scheme: DenseScheme, plane: int) -> int:
    return lib().tq_dense_plane_row_bytes(ctypes.byref(scheme), plane)


def tq_dense_quantize(scheme, x, in_rows, rot, proj, out, out_rows, stream=None) -> int:
    return lib().tq_dense_quantize(ctypes.byref(scheme), _ptr(x), ctypes.byref(in_rows), _ptr(rot), _ptr(proj),
                                   ctypes.byref(out), ctypes.byref(out_rows), _stream(stream))


def tq_dense_dequantize(scheme, planes, in_rows, rot, proj, x, out_rows, stream=None) -> int:
    return lib().tq_dense_dequantize(ctypes.byref(scheme), ctypes.byref(planes), ctypes.byref(in_rows), _ptr(rot),
                                     _ptr(proj), _ptr(x), ctypes.byref(out_rows), _stream(stream))


def dense_scheme(head_dim: int, bits: int, qjl: bool = False) -> DenseScheme:
    return DenseScheme(head_dim, bits, 1 if qjl else 0)


def alloc_dense_planes(sch: DenseScheme, lead_shape, device) -> dict:
    """Empty paper-variant planes of shape lead_shape + [row bytes] (norm, gamma as float32 [...])."""
    out = {}
    for i, name in enumerate(DENSE_PLANES):
        nbytes = tq_dense_plane_row_bytes(sch, i)
        if nbytes < 0:
            raise TQError(nbytes, "tq_dense_plane_row_bytes")
        if nbytes == 0:
            continue
        if name in ("idx", "qjl"):
            out[name] = torch.empty(tuple(lead_shape) + (nbytes,), dtype=torch.uint8, device=device)
        else:
            out[name] = torch.empty(tuple(lead_shape), dtype=torch.float32, device=device)
    return out


def dense_planes_struct(planes: dict) -> DensePlanes:
    return DensePlanes(*[_ptr(planes.get(n)) for n in DENSE_PLANES])


def _lead_rows(lead) -> Rows:
    lead = tuple(lead)
    while len(lead) < 3:
        lead = (1,) + lead
    if len(lead) != 3:
        raise ValueError("rows must be given as at most three leading dims")
    return contiguous_rows(lead)


def dense_quantize(x: torch.Tensor, rot: torch.Tensor, bits: int, proj: torch.Tensor | None = None,
                   out: dict | None = None) -> dict:
    """Paper-variant codec of contiguous bf16 rows [..., d] (at most three leading dims):
    rot (and proj for the QJL stage) are bf16 [d, d]."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    sch = dense_scheme(x.shape[-1], bits, proj is not None)
    lead = x.shape[:-1]
    if out is None:
        out = alloc_dense_planes(sch, lead, x.device)
    r = _lead_rows(lead)
    _check(tq_dense_quantize(sch, x, r, rot, proj, dense_planes_struct(out), r), "tq_dense_quantize")
    return out


def dense_dequantize(planes: dict, rot: torch.Tensor, bits: int, proj: torch.Tensor | None = None,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 rows [..., d] rebuilt from contiguous paper-variant planes."""
    d = rot.shape[-1]
    sch = dense_scheme(d, bits, proj is not None)
    lead = planes["norm"].shape
    if out is None:
        out = torch.empty(tuple(lead) + (d,), dtype=torch.bfloat16, device=planes["norm"].device)
    r = _lead_rows(lead)
    _check(tq_dense_dequantize(sch, dense_planes_struct(planes), r, rot, proj, out, r), "tq_dense_dequantize")
    return out
