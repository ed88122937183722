"""Python binding of libfd_decode_attn.so (split-KV decode attention, gfx950).

The functions carry the names of the C entry points in
include/fd_decode_attn.h and only marshal arguments: they check that every
tensor is a contiguous device tensor of the dtype and size the descriptor
implies (so no kernel is handed a short buffer), then pass raw pointers and
torch's current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no other code path.  If the shared library is missing and
cannot be built, importing the binding's loader raises.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path
from typing import Optional

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libfd_decode_attn.so"

FD_OK, FD_ERR_INVALID_ARG, FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE_TOO_SMALL, FD_ERR_HIP = range(5)
FD_F32, FD_F16, FD_BF16, FD_FP8_E4M3 = 0, 1, 2, 3
FD_SOFTMAX_SYNC, FD_SOFTMAX_UNIFIED_MAX = 0, 1
FD_KERNEL_AUTO, FD_KERNEL_VALU, FD_KERNEL_MFMA = 0, 1, 2
FD_MERGE_AUTO, FD_MERGE_SEPARATE, FD_MERGE_FUSED = 0, 1, 2
FD_FALLBACK_SPLIT, FD_FALLBACK_ROW = 0, 1
TICKET_BYTES = 65536 * 4          # FD_TICKET_BYTES: merge counters at the start of a workspace
MAX_Q_LEN = 65536                 # FD_MAX_Q_LEN: query tokens per request

DTYPES = {"f32": FD_F32, "f16": FD_F16, "bf16": FD_BF16, "fp8": FD_FP8_E4M3}
MODES = {"sync": FD_SOFTMAX_SYNC, "unified": FD_SOFTMAX_UNIFIED_MAX}
KERNELS = {"auto": FD_KERNEL_AUTO, "valu": FD_KERNEL_VALU, "mfma": FD_KERNEL_MFMA}
MERGES = {"auto": FD_MERGE_AUTO, "separate": FD_MERGE_SEPARATE, "fused": FD_MERGE_FUSED}
FALLBACKS = {"split": FD_FALLBACK_SPLIT, "row": FD_FALLBACK_ROW}


class FdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {fd_status_string(status)} ({status})")
        self.status = status


class fd_decode_desc(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32),
                ("kv_dtype", C.c_int32), ("out_dtype", C.c_int32), ("split_size", C.c_int32),
                ("max_splits", C.c_int32), ("scale", C.c_float), ("mode", C.c_int32),
                ("phi", C.c_float), ("lo", C.c_float), ("hi", C.c_float), ("kernel", C.c_int32),
                ("q_dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float), ("q_len", C.c_int32),
                ("k_scales", C.c_void_p), ("v_scales", C.c_void_p), ("merge", C.c_int32),
                ("fallback", C.c_int32)]


def make_desc(B, Hq, Hkv, d, kv_dtype="bf16", out_dtype=None, split_size=256, max_splits=None,
              max_seq_len=None, scale=0.0, mode="sync", phi=0.0, lo=0.0, hi=0.0, kernel="auto", q_dtype=None,
              k_scale=0.0, v_scale=0.0, q_len=1, k_scales=None, v_scales=None, merge="auto",
              fallback="split"):
    """Descriptor with names instead of enum codes.  max_splits defaults to
    ceil(max_seq_len / split_size); q_dtype (8-bit caches only) defaults to
    bf16, and out_dtype to the type of q.  q_len: causal query tokens per request.
    k_scales / v_scales: float32 device tensors [Hkv] of per-KV-head scales of
    an 8-bit cache (kept referenced by the descriptor).  merge: "auto",
    "separate" or "fused" (fd_decode_attn and fd_decode_attn_paged).
    fallback: "split" or "row" (what unified max recomputes)."""
    if max_splits is None:
        if max_seq_len is None:
            raise ValueError("give max_splits or max_seq_len")
        max_splits = max(1, -(-int(max_seq_len) // int(split_size)))
    if q_dtype is None:
        q_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    desc = fd_decode_desc(int(B), int(Hq), int(Hkv), int(d), DTYPES[kv_dtype],
                          DTYPES[out_dtype or q_dtype], int(split_size), int(max_splits), float(scale),
                          MODES[mode], float(phi), float(lo), float(hi), KERNELS[kernel], DTYPES[q_dtype],
                          float(k_scale), float(v_scale), int(q_len), None, None, MERGES[merge],
                          FALLBACKS[fallback])
    keep = []
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        if t is not None:
            ptr = _ptr(t, name, _torch().float32, int(Hkv), align=4)
            keep.append(t)
            setattr(desc, name, ptr.value)
    desc._keep = keep        # the scale tensors live as long as the descriptor
    return desc


_lib = None


def lib():
    """The loaded shared library (built in-tree first if it is not there)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            from . import build as _build
            _build.build()
        L = C.CDLL(str(LIB_PATH))
        dp = C.POINTER(fd_decode_desc)
        vp, i32 = C.c_void_p, C.c_int32
        L.fd_decode_attn_partial.argtypes = [dp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
        L.fd_decode_attn_combine.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp]
        L.fd_decode_attn_paged.argtypes = [dp, vp, vp, vp, i32, i32, vp, i32, vp, vp, C.c_size_t, vp, vp, vp,
                                           vp, vp]
        L.fd_decode_attn.argtypes = [dp, vp, vp, vp, i32, vp, vp, C.c_size_t, vp, vp, vp, vp, vp]
        L.fd_decode_attn_paged_noalloc.argtypes = [dp, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp]
        L.fd_workspace_bytes.argtypes = [dp]
        L.fd_workspace_bytes.restype = C.c_size_t
        L.fd_split_heuristic.argtypes = [i32, i32, i32, i32, i32, i32, C.POINTER(i32), C.POINTER(i32)]
        L.fd_status_string.argtypes = [C.c_int]
        L.fd_status_string.restype = C.c_char_p
        for f in ("fd_decode_attn_partial", "fd_decode_attn_combine", "fd_decode_attn", "fd_decode_attn_paged",
                  "fd_decode_attn_paged_noalloc", "fd_split_heuristic"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def fd_status_string(status: int) -> str:
    return lib().fd_status_string(int(status)).decode()


def fd_workspace_bytes(desc: fd_decode_desc) -> int:
    return int(lib().fd_workspace_bytes(C.byref(desc)))


def fd_split_heuristic(B, Hq, Hkv, max_seq_len, page_size, num_cus):
    """Returns (split_size, num_splits); raises FdError on a bad argument."""
    split, S = C.c_int32(), C.c_int32()
    st = lib().fd_split_heuristic(int(B), int(Hq), int(Hkv), int(max_seq_len), int(page_size), int(num_cus),
                                  C.byref(split), C.byref(S))
    if st != FD_OK:
        raise FdError("fd_split_heuristic", st)
    return split.value, S.value


# ----------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _tdtype(code):
    """torch dtype(s) a tensor of this storage type may have (8-bit: E4M3 or raw bytes)."""
    torch = _torch()
    return {FD_F32: torch.float32, FD_F16: torch.float16, FD_BF16: torch.bfloat16,
            FD_FP8_E4M3: (torch.float8_e4m3fn, torch.uint8)}[code]


def _qdtype(desc):
    return _tdtype(desc.q_dtype if desc.kv_dtype == FD_FP8_E4M3 else desc.kv_dtype)


def _ptr(t, name, dtype=None, numel=None, optional=False, align=16):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    if t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn, st):
    if st != FD_OK:
        raise FdError(fn, st)


def query_rows(desc):
    """Query rows per request: q_len * Hq."""
    return max(1, desc.q_len) * desc.Hq


def partial_shapes(desc):
    """Shapes of (part_o, part_m, part_l, flags) for a descriptor."""
    rows = (desc.B, query_rows(desc), desc.max_splits)
    return rows + (desc.d,), rows, rows, rows


def fd_decode_attn_partial(desc, q, k, v, kv_capacity, seq_lens, part_o, part_m, part_l, flags=None,
                           fallback_count=None, stream=None):
    """Split partials over a contiguous cache k, v [B, kv_capacity, Hkv, d]."""
    torch = _torch()
    kvt = _tdtype(desc.kv_dtype)
    nrow = desc.B * query_rows(desc) * desc.max_splits
    args = [
        _ptr(q, "q", _qdtype(desc), desc.B * query_rows(desc) * desc.d),
        _ptr(k, "k", kvt, desc.B * kv_capacity * desc.Hkv * desc.d),
        _ptr(v, "v", kvt, desc.B * kv_capacity * desc.Hkv * desc.d),
        C.c_int32(int(kv_capacity)),
        _ptr(seq_lens, "seq_lens", torch.int32, desc.B, optional=True, align=4),
        _ptr(part_o, "part_o", torch.float32, nrow * desc.d),
        _ptr(part_m, "part_m", torch.float32, nrow, align=4),
        _ptr(part_l, "part_l", torch.float32, nrow, align=4),
        _ptr(flags, "flags", torch.uint8, nrow, optional=True, align=1),
        _ptr(fallback_count, "fallback_count", torch.int32, 1, optional=True, align=4),
        _stream(stream),
    ]
    _check("fd_decode_attn_partial", lib().fd_decode_attn_partial(C.byref(desc), *args))


def fd_decode_attn_combine(desc, part_o, part_m, part_l, seq_lens, out, lse=None, stream=None):
    torch = _torch()
    nrow = desc.B * query_rows(desc) * desc.max_splits
    args = [
        _ptr(part_o, "part_o", torch.float32, nrow * desc.d),
        _ptr(part_m, "part_m", torch.float32, nrow, align=4),
        _ptr(part_l, "part_l", torch.float32, nrow, align=4),
        _ptr(seq_lens, "seq_lens", torch.int32, desc.B, optional=True, align=4),
        _ptr(out, "out", _tdtype(desc.out_dtype), desc.B * query_rows(desc) * desc.d),
        _ptr(lse, "lse", torch.float32, desc.B * query_rows(desc), optional=True, align=4),
        _stream(stream),
    ]
    _check("fd_decode_attn_combine", lib().fd_decode_attn_combine(C.byref(desc), *args))


def fd_decode_attn(desc, q, k, v, kv_capacity, seq_lens, workspace, out, lse=None, flags=None, fallback_count=None,
                   stream=None):
    """Partial + merge over a contiguous cache k, v [B, kv_capacity, Hkv, d]
    (the merge as desc.merge says), partials in `workspace`."""
    torch = _torch()
    kvt = _tdtype(desc.kv_dtype)
    nrow = desc.B * query_rows(desc) * desc.max_splits
    ws_bytes = fd_workspace_bytes(desc)
    if workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace needs {ws_bytes} bytes")
    args = [
        _ptr(q, "q", _qdtype(desc), desc.B * query_rows(desc) * desc.d),
        _ptr(k, "k", kvt, desc.B * kv_capacity * desc.Hkv * desc.d),
        _ptr(v, "v", kvt, desc.B * kv_capacity * desc.Hkv * desc.d),
        C.c_int32(int(kv_capacity)),
        _ptr(seq_lens, "seq_lens", torch.int32, desc.B, optional=True, align=4),
        _ptr(workspace, "workspace", align=256),
        C.c_size_t(workspace.numel() * workspace.element_size()),
        _ptr(out, "out", _tdtype(desc.out_dtype), desc.B * query_rows(desc) * desc.d),
        _ptr(lse, "lse", torch.float32, desc.B * query_rows(desc), optional=True, align=4),
        _ptr(flags, "flags", torch.uint8, nrow, optional=True, align=1),
        _ptr(fallback_count, "fallback_count", torch.int32, 1, optional=True, align=4),
        _stream(stream),
    ]
    _check("fd_decode_attn", lib().fd_decode_attn(C.byref(desc), *args))


def fd_decode_attn_paged(desc, q, k_cache, v_cache, page_size, block_table, seq_lens, workspace, out,
                         lse=None, flags=None, fallback_count=None, stream=None):
    """Partial + combine over a paged cache [num_pages, page_size, Hkv, d]."""
    torch = _torch()
    kvt = _tdtype(desc.kv_dtype)
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (page_size, desc.Hkv, desc.d):
        raise ValueError(f"k_cache must be [num_pages, {page_size}, {desc.Hkv}, {desc.d}]")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must match k_cache")
    if block_table.dim() != 2 or block_table.shape[0] != desc.B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    num_pages = int(k_cache.shape[0])
    nrow = desc.B * query_rows(desc) * desc.max_splits
    ws_bytes = fd_workspace_bytes(desc)
    if workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace needs {ws_bytes} bytes")
    args = [
        _ptr(q, "q", _qdtype(desc), desc.B * query_rows(desc) * desc.d),
        _ptr(k_cache, "k_cache", kvt),
        _ptr(v_cache, "v_cache", kvt),
        C.c_int32(num_pages), C.c_int32(int(page_size)),
        _ptr(block_table, "block_table", torch.int32, align=4),
        C.c_int32(int(block_table.shape[1])),
        _ptr(seq_lens, "seq_lens", torch.int32, desc.B, align=4),
        _ptr(workspace, "workspace", align=256),
        C.c_size_t(workspace.numel() * workspace.element_size()),
        _ptr(out, "out", _tdtype(desc.out_dtype), desc.B * query_rows(desc) * desc.d),
        _ptr(lse, "lse", torch.float32, desc.B * query_rows(desc), optional=True, align=4),
        _ptr(flags, "flags", torch.uint8, nrow, optional=True, align=1),
        _ptr(fallback_count, "fallback_count", torch.int32, 1, optional=True, align=4),
        _stream(stream),
    ]
    _check("fd_decode_attn_paged", lib().fd_decode_attn_paged(C.byref(desc), *args))


NOALLOC_SCRATCH_BYTES = 64 << 20   # FD_NOALLOC_SCRATCH_BYTES


def fd_decode_attn_paged_noalloc(desc, q, k_cache, v_cache, page_size, block_table, seq_lens, out, lse=None,
                                 flags=None, fallback_count=None, stream=None):
    """fd_decode_attn_paged without a workspace: the partials live in the
    library's per-GPU scratch array (no allocation in the call)."""
    torch = _torch()
    kvt = _tdtype(desc.kv_dtype)
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (page_size, desc.Hkv, desc.d):
        raise ValueError(f"k_cache must be [num_pages, {page_size}, {desc.Hkv}, {desc.d}]")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must match k_cache")
    if block_table.dim() != 2 or block_table.shape[0] != desc.B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    nrow = desc.B * query_rows(desc) * desc.max_splits
    args = [
        _ptr(q, "q", _qdtype(desc), desc.B * query_rows(desc) * desc.d),
        _ptr(k_cache, "k_cache", kvt),
        _ptr(v_cache, "v_cache", kvt),
        C.c_int32(int(k_cache.shape[0])), C.c_int32(int(page_size)),
        _ptr(block_table, "block_table", torch.int32, align=4),
        C.c_int32(int(block_table.shape[1])),
        _ptr(seq_lens, "seq_lens", torch.int32, desc.B, align=4),
        _ptr(out, "out", _tdtype(desc.out_dtype), desc.B * query_rows(desc) * desc.d),
        _ptr(lse, "lse", torch.float32, desc.B * query_rows(desc), optional=True, align=4),
        _ptr(flags, "flags", torch.uint8, nrow, optional=True, align=1),
        _ptr(fallback_count, "fallback_count", torch.int32, 1, optional=True, align=4),
        _stream(stream),
    ]
    _check("fd_decode_attn_paged_noalloc", lib().fd_decode_attn_paged_noalloc(C.byref(desc), *args))


def alloc_partials(desc, device="cuda"):
    """Device buffers (part_o, part_m, part_l, flags) for a descriptor."""
    torch = _torch()
    so, sm, sl, sf = partial_shapes(desc)
    return (torch.empty(so, dtype=torch.float32, device=device),
            torch.empty(sm, dtype=torch.float32, device=device),
            torch.empty(sl, dtype=torch.float32, device=device),
            torch.zeros(sf, dtype=torch.uint8, device=device))


def alloc_workspace(desc, device="cuda"):
    """A workspace for fd_decode_attn / fd_decode_attn_paged, zeroed (the
    single-launch merge needs its counters zero before the first call)."""
    torch = _torch()
    return torch.zeros(fd_workspace_bytes(desc), dtype=torch.uint8, device=device)


def workspace_partials(desc, workspace):
    """Views (part_o, part_m, part_l) of a workspace at the layout the header
    states: FD_TICKET_BYTES of counters, then part_o, part_m and part_l, each
    on a 256-byte boundary.  With the single-launch merge they hold the
    workgroup partials (slots 0 .. of each row), not per-split ones."""
    torch = _torch()
    so, sm, sl, _ = partial_shapes(desc)
    n = desc.B * query_rows(desc) * desc.max_splits
    r256 = lambda x: (x + 255) // 256 * 256
    o_off = TICKET_BYTES
    m_off = o_off + r256(n * desc.d * 4)
    l_off = m_off + r256(n * 4)
    fw = workspace.view(torch.float32)
    return (fw[o_off // 4:o_off // 4 + n * desc.d].view(so), fw[m_off // 4:m_off // 4 + n].view(sm),
            fw[l_off // 4:l_off // 4 + n].view(sl))
