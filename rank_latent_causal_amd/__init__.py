"""Python binding of the MI355X absorbed Gated MLA library (libmla_absorb.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in include/mla_absorb.h.  Tensors are PyTorch
tensors on the GPU (PyTorch provides device memory and streams); the binding
checks shapes, dtypes and contiguity, allocates the output and workspace when
the caller does not pass them, and calls the C entry point on the current
stream.  There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes as ct
import os

__all__ = [
    "LIB_PATH", "MLA_OK", "MLA_ERR_INVALID_ARG", "MLA_ERR_UNSUPPORTED", "MLA_ERR_WORKSPACE",
    "MLA_ERR_HIP", "DTYPE_F32", "DTYPE_BF16", "MLAError", "lib", "status_string",
    "prefill_workspace_size", "workspace_size", "decode_workspace_size", "decode_paged_workspace_size", "forward_workspace_size",
    "mla_absorb_prefill", "mla_absorb_extend", "mla_absorb_extend_paged", "mla_absorb_decode",
    "mla_absorb_decode_noalloc",
    "mla_absorb_decode_paged", "mla_cache_append_paged", "mla_gated_forward", "mla_absorb_prefill_train",
    "backward_workspace_size", "mla_absorb_prefill_backward", "varlen_workspace_size",
    "mla_absorb_extend_varlen_paged", "train_state_size", "mla_gated_forward_train",
    "layer_backward_workspace_size", "mla_gated_backward", "LAYER_GRAD_KEYS", "kda_workspace_size",
    "kda_chunk_forward",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_absorb.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
DTYPE_F32, DTYPE_BF16 = 0, 1

EXPORTS = (
    "mla_status_string",
    "mla_absorb_prefill_workspace_size",
    "mla_absorb_workspace_size",
    "mla_absorb_prefill",
    "mla_absorb_extend",
    "mla_absorb_decode_workspace_size",
    "mla_absorb_decode",
    "mla_absorb_decode_noalloc",
    "mla_absorb_extend_paged",
    "mla_absorb_extend_varlen_workspace_size",
    "mla_absorb_extend_varlen_paged",
    "mla_absorb_decode_paged_workspace_size",
    "mla_absorb_decode_paged",
    "mla_cache_append_paged",
    "mla_absorb_prefill_train",
    "mla_absorb_prefill_backward_workspace_size",
    "mla_absorb_prefill_backward",
    "mla_gated_forward_workspace_size",
    "mla_gated_forward",
    "mla_gated_train_state_size",
    "mla_gated_forward_train",
    "mla_gated_backward_workspace_size",
    "mla_gated_backward",
    "kda_chunk_workspace_size",
    "kda_chunk_forward",
)

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def lib() -> ct.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with rank_latent_causal_amd.build.build()")
        L = ct.CDLL(LIB_PATH)
        vp, sz, I, I64, F = ct.c_void_p, ct.c_size_t, ct.c_int, ct.c_int64, ct.c_float
        L.mla_status_string.argtypes = [I]
        L.mla_status_string.restype = ct.c_char_p
        L.mla_absorb_prefill_workspace_size.argtypes = [I, I, I, I, I, I]
        L.mla_absorb_prefill_workspace_size.restype = sz
        L.mla_absorb_workspace_size.argtypes = [I, I, I, I, I, I]
        L.mla_absorb_workspace_size.restype = sz
        L.mla_absorb_prefill.argtypes = [vp, vp, vp, vp, vp, vp, I, I, I, I, I, I, F, I, vp, sz, vp]
        L.mla_absorb_prefill.restype = I
        L.mla_absorb_extend.argtypes = [vp, vp, vp, vp, vp, vp, I, I, I, I, I, I, I, F, I, vp, sz, vp]
        L.mla_absorb_extend.restype = I
        L.mla_absorb_decode_workspace_size.argtypes = [I, I, I, I, I, I]
        L.mla_absorb_decode_workspace_size.restype = sz
        L.mla_absorb_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, I64, F, I, I, vp, sz, vp]
        L.mla_absorb_decode.restype = I
        L.mla_absorb_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, I64, F, I, I, vp]
        L.mla_absorb_decode_noalloc.restype = I
        L.mla_absorb_extend_paged.argtypes = [vp] * 7 + [I] * 7 + [I64, I, I, F, I, vp, sz, vp]
        L.mla_absorb_extend_paged.restype = I
        L.mla_absorb_extend_varlen_workspace_size.argtypes = [I] * 6
        L.mla_absorb_extend_varlen_workspace_size.restype = sz
        L.mla_absorb_extend_varlen_paged.argtypes = [vp] * 9 + [I] * 6 + [I64, I, I, F, I, vp, sz, vp]
        L.mla_absorb_extend_varlen_paged.restype = I
        L.mla_absorb_decode_paged_workspace_size.argtypes = [I, I, I, I, I, I]
        L.mla_absorb_decode_paged_workspace_size.restype = sz
        L.mla_absorb_decode_paged.argtypes = [vp] * 8 + [I] * 5 + [I64, I, I, F, I, I, vp, sz, vp]
        L.mla_absorb_decode_paged.restype = I
        L.mla_cache_append_paged.argtypes = [vp] * 4 + [I, I, I64, I, I, I, vp]
        L.mla_cache_append_paged.restype = I
        L.mla_absorb_prefill_train.argtypes = [vp] * 7 + [I] * 6 + [F, I, vp, sz, vp]
        L.mla_absorb_prefill_train.restype = I
        L.mla_absorb_prefill_backward_workspace_size.argtypes = [I] * 7
        L.mla_absorb_prefill_backward_workspace_size.restype = sz
        L.mla_absorb_prefill_backward.argtypes = [vp] * 13 + [I] * 6 + [F, I, vp, sz, vp]
        L.mla_absorb_prefill_backward.restype = I
        L.mla_gated_forward_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
        L.mla_gated_forward_workspace_size.restype = sz
        L.mla_gated_forward.argtypes = [vp] * 11 + [I] * 8 + [F, F, I, vp, sz, vp]
        L.mla_gated_forward.restype = I
        L.mla_gated_train_state_size.argtypes = [I] * 8
        L.mla_gated_train_state_size.restype = sz
        L.mla_gated_forward_train.argtypes = [vp] * 11 + [I] * 8 + [F, F, I, vp, sz, vp]
        L.mla_gated_forward_train.restype = I
        L.mla_gated_backward_workspace_size.argtypes = [I] * 9
        L.mla_gated_backward_workspace_size.restype = sz
        L.mla_gated_backward.argtypes = [vp] * 12 + [sz] + [vp] * 10 + [I] * 8 + [F, I, vp, sz, vp]
        L.mla_gated_backward.restype = I
        L.kda_chunk_workspace_size.argtypes = [I] * 7
        L.kda_chunk_workspace_size.restype = sz
        L.kda_chunk_forward.argtypes = [vp] * 8 + [I] * 6 + [I, vp, sz, vp]
        L.kda_chunk_forward.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


_BAD = ct.c_size_t(-1).value


def prefill_workspace_size(B: int, T: int, H: int, d_q: int, r: int, dtype: int) -> int:
    n = lib().mla_absorb_prefill_workspace_size(B, T, H, d_q, r, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_absorb_prefill_workspace_size")
    return n


def workspace_size(is_decode: bool, B: int, T_or_max_len: int, H: int, r: int, dtype: int) -> int:
    """Workspace bytes of a prefill (T) or a default-split decode call."""
    n = lib().mla_absorb_workspace_size(int(bool(is_decode)), B, T_or_max_len, H, r, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_absorb_workspace_size")
    return n


def decode_workspace_size(B: int, H: int, d_q: int, r: int, num_splits: int, dtype: int) -> int:
    n = lib().mla_absorb_decode_workspace_size(B, H, d_q, r, num_splits, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_absorb_decode_workspace_size")
    return n


def varlen_workspace_size(B: int, Nq: int, H: int, d_q: int, r: int, dtype: int) -> int:
    n = lib().mla_absorb_extend_varlen_workspace_size(B, Nq, H, d_q, r, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_absorb_extend_varlen_workspace_size")
    return n


def decode_paged_workspace_size(B: int, H: int, d_q: int, r: int, num_splits: int, dtype: int) -> int:
    n = lib().mla_absorb_decode_paged_workspace_size(B, H, d_q, r, num_splits, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_absorb_decode_paged_workspace_size")
    return n


def backward_workspace_size(B: int, T: int, H: int, d_q: int, d_v: int, r: int, dtype: int) -> int:
    n = lib().mla_absorb_prefill_backward_workspace_size(B, T, H, d_q, d_v, r, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_absorb_prefill_backward_workspace_size")
    return n


def forward_workspace_size(B: int, T: int, q_rank: int, H: int, d_q: int, d_v: int, r: int, dtype: int) -> int:
    n = lib().mla_gated_forward_workspace_size(B, T, q_rank, H, d_q, d_v, r, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_gated_forward_workspace_size")
    return n


def train_state_size(B: int, T: int, q_rank: int, H: int, d_q: int, d_v: int, r: int, dtype: int) -> int:
    n = lib().mla_gated_train_state_size(B, T, q_rank, H, d_q, d_v, r, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_gated_train_state_size")
    return n


def layer_backward_workspace_size(B: int, T: int, D: int, q_rank: int, H: int, d_q: int, d_v: int, r: int,
                                  dtype: int) -> int:
    n = lib().mla_gated_backward_workspace_size(B, T, D, q_rank, H, d_q, d_v, r, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "mla_gated_backward_workspace_size")
    return n


def kda_workspace_size(B: int, T: int, H: int, G: int, K: int, V: int, dtype: int = DTYPE_BF16) -> int:
    n = lib().kda_chunk_workspace_size(B, T, H, G, K, V, dtype)
    if n == _BAD:
        raise MLAError(MLA_ERR_INVALID_ARG, "kda_chunk_workspace_size")
    return n


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: must be a contiguous GPU tensor")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ct.c_void_p(stream.cuda_stream)


def mla_absorb_prefill(q, c, w_uk, w_uv, gate, scale: float, out=None, workspace=None, stream=None):
    """Prefill of the absorbed Gated MLA layer.  q [B,T,H,d_q], c [B,T,r],
    w_uk [H,d_q,r], w_uv [H,d_v,r], gate [B,T,H*d_v] -> out [B,T,H*d_v]."""
    torch = _torch()
    B, T, H, dq = q.shape
    r = c.shape[-1]
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, T, H, dq), "q"), (c, (B, T, r), "c"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, T, H * dv), "gate")):
        _check(t, shp, dt, n)
    if out is None:
        out = torch.empty((B, T, H * dv), dtype=dt, device=q.device)
    _check(out, (B, T, H * dv), dt, "out")
    need = prefill_workspace_size(B, T, H, dq, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_prefill(q.data_ptr(), c.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                  gate.data_ptr(), out.data_ptr(), B, T, H, dq, dv, r, float(scale),
                                  code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_prefill")
    return out


def mla_absorb_extend(q, c, w_uk, w_uv, gate, scale: float, out=None, workspace=None, stream=None):
    """Chunked prefill against a cached prefix.  q [B,T,H,d_q] are positions
    S-T .. S-1 of sequences whose latent is c [B,S,r] (S >= T), w_uk
    [H,d_q,r], w_uv [H,d_v,r], gate [B,T,H*d_v] -> out [B,T,H*d_v]."""
    torch = _torch()
    B, T, H, dq = q.shape
    S, r = c.shape[1], c.shape[2]
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, T, H, dq), "q"), (c, (B, S, r), "c"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, T, H * dv), "gate")):
        _check(t, shp, dt, n)
    if out is None:
        out = torch.empty((B, T, H * dv), dtype=dt, device=q.device)
    _check(out, (B, T, H * dv), dt, "out")
    need = prefill_workspace_size(B, T, H, dq, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_extend(q.data_ptr(), c.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                 gate.data_ptr(), out.data_ptr(), B, T, S, H, dq, dv, r, float(scale),
                                 code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_extend")
    return out


def mla_absorb_decode(q, c_cache, cu_seqlens, w_uk, w_uv, gate, scale: float, num_splits: int = 0,
                      out=None, workspace=None, stream=None):
    """Decode against a packed latent cache.  q [B,H,d_q], c_cache [N,r],
    cu_seqlens [B+1] int32 (device), w_uk [H,d_q,r], w_uv [H,d_v,r],
    gate [B,H*d_v] -> out [B,H*d_v]."""
    torch = _torch()
    B, H, dq = q.shape
    N, r = c_cache.shape
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, H, dq), "q"), (c_cache, (N, r), "c_cache"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, H * dv), "gate")):
        _check(t, shp, dt, n)
    _check(cu_seqlens, (B + 1,), torch.int32, "cu_seqlens")
    if out is None:
        out = torch.empty((B, H * dv), dtype=dt, device=q.device)
    _check(out, (B, H * dv), dt, "out")
    need = decode_workspace_size(B, H, dq, r, num_splits, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_decode(q.data_ptr(), c_cache.data_ptr(), cu_seqlens.data_ptr(), w_uk.data_ptr(),
                                 w_uv.data_ptr(), gate.data_ptr(), out.data_ptr(), B, H, dq, dv, r, N,
                                 float(scale), int(num_splits), code, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_decode")
    return out


def mla_absorb_decode_noalloc(q, c_cache, cu_seqlens, w_uk, w_uv, gate, scale: float, num_splits: int = 0,
                              out=None, stream=None):
    """mla_absorb_decode with its scratch in the library's static per-GPU
    buffer (no workspace argument; the C call allocates nothing).  Passing
    `out` keeps this wrapper allocation-free as well."""
    torch = _torch()
    B, H, dq = q.shape
    N, r = c_cache.shape
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, H, dq), "q"), (c_cache, (N, r), "c_cache"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, H * dv), "gate")):
        _check(t, shp, dt, n)
    _check(cu_seqlens, (B + 1,), torch.int32, "cu_seqlens")
    if out is None:
        out = torch.empty((B, H * dv), dtype=dt, device=q.device)
    _check(out, (B, H * dv), dt, "out")
    st = lib().mla_absorb_decode_noalloc(q.data_ptr(), c_cache.data_ptr(), cu_seqlens.data_ptr(), w_uk.data_ptr(),
                                         w_uv.data_ptr(), gate.data_ptr(), out.data_ptr(), B, H, dq, dv, r, N,
                                         float(scale), int(num_splits), code, _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_decode_noalloc")
    return out


def mla_absorb_extend_paged(q, c_pages, block_table, S: int, w_uk, w_uv, gate, scale: float, out=None,
                            workspace=None, stream=None):
    """Chunked prefill against a paged latent cache: c_pages
    [num_pages, page_size, r], block_table [B, max_pages] int32 (device);
    each sequence holds S rows, the T queries q [B,T,H,d_q] are its last
    positions.  gate, out [B,T,H*d_v]."""
    torch = _torch()
    B, T, H, dq = q.shape
    npg, ps, r = c_pages.shape
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, T, H, dq), "q"), (c_pages, (npg, ps, r), "c_pages"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, T, H * dv), "gate")):
        _check(t, shp, dt, n)
    _check(block_table, (B, block_table.shape[1]), torch.int32, "block_table")
    if out is None:
        out = torch.empty((B, T, H * dv), dtype=dt, device=q.device)
    _check(out, (B, T, H * dv), dt, "out")
    need = prefill_workspace_size(B, T, H, dq, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_extend_paged(q.data_ptr(), c_pages.data_ptr(), block_table.data_ptr(), w_uk.data_ptr(),
                                       w_uv.data_ptr(), gate.data_ptr(), out.data_ptr(), B, T, int(S), H, dq, dv, r,
                                       npg, ps, block_table.shape[1], float(scale), code, workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_extend_paged")
    return out


def mla_absorb_extend_varlen_paged(q, c_pages, block_table, cu_q, seq_lens, w_uk, w_uv, gate, scale: float,
                                   out=None, workspace=None, stream=None):
    """Varlen chunked prefill over a paged cache (a mixed prefill / chunk /
    decode batch in one call): q [Nq,H,d_q] packed by cu_q [B+1] (int32,
    device), seq_lens [B] (int32, device) cache rows per sequence; gate and
    out [Nq,H*d_v]."""
    torch = _torch()
    Nq, H, dq = q.shape
    npg, ps, r = c_pages.shape
    dv = w_uv.shape[1]
    B = seq_lens.shape[0]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (Nq, H, dq), "q"), (c_pages, (npg, ps, r), "c_pages"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (Nq, H * dv), "gate")):
        _check(t, shp, dt, n)
    _check(block_table, (B, block_table.shape[1]), torch.int32, "block_table")
    _check(cu_q, (B + 1,), torch.int32, "cu_q")
    _check(seq_lens, (B,), torch.int32, "seq_lens")
    if out is None:
        out = torch.empty((Nq, H * dv), dtype=dt, device=q.device)
    _check(out, (Nq, H * dv), dt, "out")
    need = varlen_workspace_size(B, Nq, H, dq, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_extend_varlen_paged(
        q.data_ptr(), c_pages.data_ptr(), block_table.data_ptr(), cu_q.data_ptr(), seq_lens.data_ptr(),
        w_uk.data_ptr(), w_uv.data_ptr(), gate.data_ptr(), out.data_ptr(), B, Nq, H, dq, dv, r, npg, ps,
        block_table.shape[1], float(scale), code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_extend_varlen_paged")
    return out


def mla_absorb_decode_paged(q, c_pages, block_table, seq_lens, w_uk, w_uv, gate, scale: float,
                            num_splits: int = 0, out=None, workspace=None, stream=None):
    """Decode against a paged latent cache: c_pages [num_pages, page_size, r],
    block_table [B, max_pages] int32, seq_lens [B] int32 (device, the new
    token's own row included).  q [B,H,d_q], gate [B,H*d_v] -> [B,H*d_v]."""
    torch = _torch()
    B, H, dq = q.shape
    npg, ps, r = c_pages.shape
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, H, dq), "q"), (c_pages, (npg, ps, r), "c_pages"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, H * dv), "gate")):
        _check(t, shp, dt, n)
    _check(block_table, (B, block_table.shape[1]), torch.int32, "block_table")
    _check(seq_lens, (B,), torch.int32, "seq_lens")
    if out is None:
        out = torch.empty((B, H * dv), dtype=dt, device=q.device)
    _check(out, (B, H * dv), dt, "out")
    need = decode_paged_workspace_size(B, H, dq, r, num_splits, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_decode_paged(q.data_ptr(), c_pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
                                       w_uk.data_ptr(), w_uv.data_ptr(), gate.data_ptr(), out.data_ptr(), B, H, dq,
                                       dv, r, npg, ps, block_table.shape[1], float(scale), int(num_splits), code,
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_decode_paged")
    return out


def mla_cache_append_paged(c_new, c_pages, block_table, positions, stream=None):
    """Writes row c_new[i] ([B, r]) at position positions[i] (int32, device)
    of sequence i of the paged cache c_pages (in place)."""
    torch = _torch()
    B, r = c_new.shape
    npg, ps, _ = c_pages.shape
    dt = c_new.dtype
    _check(c_new, (B, r), dt, "c_new")
    _check(c_pages, (npg, ps, r), dt, "c_pages")
    _check(block_table, (B, block_table.shape[1]), torch.int32, "block_table")
    _check(positions, (B,), torch.int32, "positions")
    st = lib().mla_cache_append_paged(c_new.data_ptr(), c_pages.data_ptr(), block_table.data_ptr(),
                                      positions.data_ptr(), B, r, npg, ps, block_table.shape[1], _dtype_code(c_new),
                                      _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_cache_append_paged")
    return c_pages


def mla_absorb_prefill_train(q, c, w_uk, w_uv, gate, scale: float, out=None, lse=None, workspace=None,
                             stream=None):
    """Prefill that also returns the log-sum-exp [B,H,T] (float32) the
    backward needs.  Returns (out, lse)."""
    torch = _torch()
    B, T, H, dq = q.shape
    r = c.shape[-1]
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, T, H, dq), "q"), (c, (B, T, r), "c"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, T, H * dv), "gate")):
        _check(t, shp, dt, n)
    if out is None:
        out = torch.empty((B, T, H * dv), dtype=dt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    _check(out, (B, T, H * dv), dt, "out")
    _check(lse, (B, H, T), torch.float32, "lse")
    need = prefill_workspace_size(B, T, H, dq, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_prefill_train(q.data_ptr(), c.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(), gate.data_ptr(),
                                        out.data_ptr(), lse.data_ptr(), B, T, H, dq, dv, r, float(scale), code,
                                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                        _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_prefill_train")
    return out, lse


def mla_absorb_prefill_backward(q, c, w_uk, w_uv, gate, out, lse, dout, scale: float, workspace=None, stream=None):
    """Gradients of the prefill core given dout [B,T,H*d_v]: returns a dict
    with dq [B,T,H,d_q], dc [B,T,r], dgate [B,T,H*d_v] (input dtype) and
    dw_uk [H,d_q,r], dw_uv [H,d_v,r] (float32)."""
    torch = _torch()
    B, T, H, dq = q.shape
    r = c.shape[-1]
    dv = w_uv.shape[1]
    dt = q.dtype
    code = _dtype_code(q)
    for t, shp, n in ((q, (B, T, H, dq), "q"), (c, (B, T, r), "c"), (w_uk, (H, dq, r), "w_uk"),
                      (w_uv, (H, dv, r), "w_uv"), (gate, (B, T, H * dv), "gate"), (out, (B, T, H * dv), "out"),
                      (dout, (B, T, H * dv), "dout")):
        _check(t, shp, dt, n)
    _check(lse, (B, H, T), torch.float32, "lse")
    g = dict(dq=torch.empty((B, T, H, dq), dtype=dt, device=q.device),
             dc=torch.empty((B, T, r), dtype=dt, device=q.device),
             dgate=torch.empty((B, T, H * dv), dtype=dt, device=q.device),
             dw_uk=torch.empty((H, dq, r), dtype=torch.float32, device=q.device),
             dw_uv=torch.empty((H, dv, r), dtype=torch.float32, device=q.device))
    need = backward_workspace_size(B, T, H, dq, dv, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().mla_absorb_prefill_backward(
        q.data_ptr(), c.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(), gate.data_ptr(), out.data_ptr(), lse.data_ptr(),
        dout.data_ptr(), g["dq"].data_ptr(), g["dc"].data_ptr(), g["dw_uk"].data_ptr(), g["dw_uv"].data_ptr(),
        g["dgate"].data_ptr(), B, T, H, dq, dv, r, float(scale), code, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_absorb_prefill_backward")
    return g


def mla_gated_forward(x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o,
                      eps: float, scale: float, out=None, workspace=None, stream=None):
    """Full Gated MLA forward (bf16): x [B,T,D] -> y [B,T,D].  Weights as
    linear layers: w_kv_down [r,D], kv_norm [r], w_q_down [q_rank,D],
    q_norm [q_rank], w_q_up [H*d_q,q_rank], w_uk [H,d_q,r], w_uv [H,d_v,r],
    w_gate [H*d_v,D], w_o [D,H*d_v]."""
    torch = _torch()
    B, T, D = x.shape
    r = w_kv_down.shape[0]
    q_rank = w_q_down.shape[0]
    H, dq, _ = w_uk.shape
    dv = w_uv.shape[1]
    dt = x.dtype
    code = _dtype_code(x)
    for t, shp, n in ((x, (B, T, D), "x"), (w_kv_down, (r, D), "w_kv_down"), (kv_norm, (r,), "kv_norm"),
                      (w_q_down, (q_rank, D), "w_q_down"), (q_norm, (q_rank,), "q_norm"),
                      (w_q_up, (H * dq, q_rank), "w_q_up"), (w_uk, (H, dq, r), "w_uk"), (w_uv, (H, dv, r), "w_uv"),
                      (w_gate, (H * dv, D), "w_gate"), (w_o, (D, H * dv), "w_o")):
        _check(t, shp, dt, n)
    if out is None:
        out = torch.empty((B, T, D), dtype=dt, device=x.device)
    _check(out, (B, T, D), dt, "out")
    need = forward_workspace_size(B, T, q_rank, H, dq, dv, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib().mla_gated_forward(x.data_ptr(), w_kv_down.data_ptr(), kv_norm.data_ptr(), w_q_down.data_ptr(),
                                 q_norm.data_ptr(), w_q_up.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                 w_gate.data_ptr(), w_o.data_ptr(), out.data_ptr(), B, T, D, q_rank, H, dq, dv,
                                 r, float(eps), float(scale), code, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_gated_forward")
    return out


def _layer_dims(x, w_kv_down, w_q_down, w_uk, w_uv):
    B, T, D = x.shape
    return B, T, D, w_q_down.shape[0], w_uk.shape[0], w_uk.shape[1], w_uv.shape[1], w_kv_down.shape[0]


def _check_layer_weights(x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o):
    B, T, D, q_rank, H, dq, dv, r = _layer_dims(x, w_kv_down, w_q_down, w_uk, w_uv)
    dt = x.dtype
    for t, shp, n in ((x, (B, T, D), "x"), (w_kv_down, (r, D), "w_kv_down"), (kv_norm, (r,), "kv_norm"),
                      (w_q_down, (q_rank, D), "w_q_down"), (q_norm, (q_rank,), "q_norm"),
                      (w_q_up, (H * dq, q_rank), "w_q_up"), (w_uk, (H, dq, r), "w_uk"), (w_uv, (H, dv, r), "w_uv"),
                      (w_gate, (H * dv, D), "w_gate"), (w_o, (D, H * dv), "w_o")):
        _check(t, shp, dt, n)


def mla_gated_forward_train(x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o,
                            eps: float, scale: float, out=None, state=None, stream=None):
    """Training form of mla_gated_forward: returns (y, state), state a uint8
    device buffer that mla_gated_backward reads."""
    torch = _torch()
    _check_layer_weights(x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o)
    B, T, D, q_rank, H, dq, dv, r = _layer_dims(x, w_kv_down, w_q_down, w_uk, w_uv)
    code = _dtype_code(x)
    if out is None:
        out = torch.empty((B, T, D), dtype=x.dtype, device=x.device)
    _check(out, (B, T, D), x.dtype, "out")
    need = train_state_size(B, T, q_rank, H, dq, dv, r, code)
    if state is None:
        state = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib().mla_gated_forward_train(x.data_ptr(), w_kv_down.data_ptr(), kv_norm.data_ptr(), w_q_down.data_ptr(),
                                       q_norm.data_ptr(), w_q_up.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                       w_gate.data_ptr(), w_o.data_ptr(), out.data_ptr(), B, T, D, q_rank, H, dq, dv,
                                       r, float(eps), float(scale), code, state.data_ptr(),
                                       state.numel() * state.element_size(), _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_gated_forward_train")
    return out, state


LAYER_GRAD_KEYS = ("dx", "dw_kv_down", "dkv_norm", "dw_q_down", "dq_norm", "dw_q_up", "dw_uk", "dw_uv", "dw_gate",
                   "dw_o")


def mla_gated_backward(x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o, dy, state,
                       scale: float, grads=None, workspace=None, stream=None) -> dict:
    """Backward of the full layer: dict keyed by LAYER_GRAD_KEYS (dx bf16
    like x, every parameter gradient float32 in its parameter's shape)."""
    torch = _torch()
    _check_layer_weights(x, w_kv_down, kv_norm, w_q_down, q_norm, w_q_up, w_uk, w_uv, w_gate, w_o)
    B, T, D, q_rank, H, dq, dv, r = _layer_dims(x, w_kv_down, w_q_down, w_uk, w_uv)
    _check(dy, (B, T, D), x.dtype, "dy")
    code = _dtype_code(x)
    shapes = dict(dx=(B, T, D), dw_kv_down=(r, D), dkv_norm=(r,), dw_q_down=(q_rank, D), dq_norm=(q_rank,),
                  dw_q_up=(H * dq, q_rank), dw_uk=(H, dq, r), dw_uv=(H, dv, r), dw_gate=(H * dv, D), dw_o=(D, H * dv))
    if grads is None:
        grads = {k: torch.empty(shapes[k], dtype=x.dtype if k == "dx" else torch.float32, device=x.device)
                 for k in LAYER_GRAD_KEYS}
    for k in LAYER_GRAD_KEYS:
        _check(grads[k], shapes[k], x.dtype if k == "dx" else torch.float32, k)
    need = layer_backward_workspace_size(B, T, D, q_rank, H, dq, dv, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib().mla_gated_backward(x.data_ptr(), w_kv_down.data_ptr(), kv_norm.data_ptr(), w_q_down.data_ptr(),
                                  q_norm.data_ptr(), w_q_up.data_ptr(), w_uk.data_ptr(), w_uv.data_ptr(),
                                  w_gate.data_ptr(), w_o.data_ptr(), dy.data_ptr(), state.data_ptr(),
                                  state.numel() * state.element_size(),
                                  *[grads[k].data_ptr() for k in LAYER_GRAD_KEYS], B, T, D, q_rank, H, dq, dv, r,
                                  float(scale), code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    if st != MLA_OK:
        raise MLAError(st, "mla_gated_backward")
    return grads


def kda_chunk_forward(q, k, v, g, beta, G: int = 1, initial_state=None, final_state: bool = False, out=None,
                      workspace=None, stream=None):
    """chunk_kda (bf16): q, k [B,T,H,K], v [B,T,G*H,V] bf16; g [B,T,G*H,K] and
    beta [B,T,G*H] float32; initial_state [B,G*H,K,V] float32 or None.
    Returns (o [B,T,G*H,V] bf16, final state float32 or None)."""
    torch = _torch()
    B, T, H, K = q.shape
    HV = G * H
    V = v.shape[3]
    _check(q, (B, T, H, K), torch.bfloat16, "q")
    _check(k, (B, T, H, K), torch.bfloat16, "k")
    _check(v, (B, T, HV, V), torch.bfloat16, "v")
    _check(g, (B, T, HV, K), torch.float32, "g")
    _check(beta, (B, T, HV), torch.float32, "beta")
    if initial_state is not None:
        _check(initial_state, (B, HV, K, V), torch.float32, "initial_state")
    if out is None:
        out = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=q.device)
    _check(out, (B, T, HV, V), torch.bfloat16, "out")
    st = torch.empty((B, HV, K, V), dtype=torch.float32, device=q.device) if final_state else None
    need = kda_workspace_size(B, T, H, G, K, V, DTYPE_BF16)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = lib().kda_chunk_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                 initial_state.data_ptr() if initial_state is not None else None, out.data_ptr(),
                                 st.data_ptr() if st is not None else None, B, T, H, G, K, V, DTYPE_BF16,
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != MLA_OK:
        raise MLAError(rc, "kda_chunk_forward")
    return out, st
