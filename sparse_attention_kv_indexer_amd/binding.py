"""Thin Python binding of the C ABI in ``include/dsa_indexer.h``.

Argument marshalling only: checks dtypes, shapes, devices and contiguity of
torch tensors, passes their device pointers and the current HIP stream to the
library, and raises ``DsaError`` on a negative status. Every step of the
decode path runs in the library's HIP kernels; there is no fallback, and a
missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

HEADS, DIM, PAGE = 32, 64, 64
HIST_BINS = 2048  # first-digit histogram of score_hist / topk_hist
ATT_HEADS, ATT_KD, ATT_VD = 32, 576, 512

_STATUS = {0: "DSA_OK", -1: "DSA_ERR_NULL", -2: "DSA_ERR_SHAPE", -3: "DSA_ERR_ALIGN",
           -4: "DSA_ERR_K", -5: "DSA_ERR_WORKSPACE", -6: "DSA_ERR_HIP", -7: "DSA_ERR_SCRATCH"}


class DsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def library_path() -> str:
    return _build.LIB_PATH


def load() -> ctypes.CDLL:
    """Load libdsa_indexer.so (building it first only if none is built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.dsa_indexer_abi_version.restype = ctypes.c_int
    lib.dsa_indexer_abi_version.argtypes = []
    lib.dsa_indexer_status_string.restype = ctypes.c_char_p
    lib.dsa_indexer_status_string.argtypes = [ctypes.c_int]
    lib.dsa_indexer_last_hip_error.restype = ctypes.c_int
    lib.dsa_indexer_last_hip_error.argtypes = []
    lib.dsa_indexer_score.restype = ctypes.c_int
    lib.dsa_indexer_score.argtypes = [vp, vp, vp, i64, vp, vp, i32, i32, vp, vp, vp]
    lib.dsa_indexer_score_hist.restype = ctypes.c_int
    lib.dsa_indexer_score_hist.argtypes = [vp, vp, vp, i64, vp, vp, i32, i32, vp, vp, vp, vp]
    lib.dsa_indexer_topk_hist.restype = ctypes.c_int
    lib.dsa_indexer_topk_hist.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.dsa_indexer_score_fp8.restype = ctypes.c_int
    lib.dsa_indexer_score_fp8.argtypes = [vp, vp, vp, vp, i64, vp, vp, i32, i32, vp, vp, vp]
    lib.dsa_indexer_score_mtp.restype = ctypes.c_int
    lib.dsa_indexer_score_mtp.argtypes = [vp, vp, vp, i64, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.dsa_indexer_topk_workspace_bytes.restype = sz
    lib.dsa_indexer_topk_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dsa_indexer_topk.restype = ctypes.c_int
    lib.dsa_indexer_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.dsa_indexer_topk_noalloc.restype = ctypes.c_int
    lib.dsa_indexer_topk_noalloc.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.dsa_indexer_sparse_attention_workspace_bytes.restype = sz
    lib.dsa_indexer_sparse_attention_workspace_bytes.argtypes = [i32, i32]
    lib.dsa_indexer_sparse_attention.restype = ctypes.c_int
    lib.dsa_indexer_sparse_attention.argtypes = [vp, vp, i64, vp, i32, i32, vp, i32, ctypes.c_float, vp, vp,
                                                 vp, sz, vp]
    _lib = lib
    return lib


def abi_version() -> int:
    return load().dsa_indexer_abi_version()


def status_string(status: int) -> str:
    return load().dsa_indexer_status_string(status).decode()


def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtypes, shape=None, device=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def score(q, w, k_pool, page_table, seq_lens, out=None, row_hwm=None, stream=None):
    """Logits [B, max_pages*64] (float32) of one decode step.

    q bf16 [B,32,64]; w float32 [B,32]; k_pool bf16 [num_pages,64,64];
    page_table int32 [B,max_pages]; seq_lens int32 [B]; ``out`` float32
    [B, max_pages*64] is allocated when not given; ``row_hwm`` int32 [B]
    selects the incremental -inf tail (see the header).
    """
    import torch

    B, S = page_table.shape
    dev = q.device
    bf16 = (torch.bfloat16, torch.int16)
    _check(q, "q", bf16, (B, HEADS, DIM))
    _check(w, "w", (torch.float32,), (B, HEADS), dev)
    _check(k_pool, "k_pool", bf16, None, dev)
    if k_pool.dim() != 3 or tuple(k_pool.shape[1:]) != (PAGE, DIM):
        raise ValueError(f"k_pool has shape {tuple(k_pool.shape)}, expected [num_pages, {PAGE}, {DIM}]")
    _check(page_table, "page_table", (torch.int32,), None, dev)
    _check(seq_lens, "seq_lens", (torch.int32,), (B,), dev)
    if out is None:
        out = torch.empty((B, S * PAGE), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (B, S * PAGE), dev)
    if row_hwm is not None:
        _check(row_hwm, "row_hwm", (torch.int32,), (B,), dev)
    st = load().dsa_indexer_score(
        q.data_ptr(), w.data_ptr(), k_pool.data_ptr(), k_pool.shape[0], page_table.data_ptr(),
        seq_lens.data_ptr(), B, S, out.data_ptr(), row_hwm.data_ptr() if row_hwm is not None else None,
        _stream_ptr(stream))
    if st != 0:
        raise DsaError(st, "dsa_indexer_score")
    return out


def hist_buffer(batch: int, device="cuda"):
    """A zeroed first-digit histogram [batch, 2048] for score_hist / topk_hist
    (int32 storage of the header's uint32 counts; topk_hist leaves it zero)."""
    import torch

    return torch.zeros((batch, HIST_BINS), dtype=torch.int32, device=device)


def score_hist(q, w, k_pool, page_table, seq_lens, hist, out=None, row_hwm=None, stream=None):
    """``score`` that also adds each request's first-digit key histogram to
    ``hist`` (int32 [B, 2048], zero on entry; see the header)."""
    import torch

    B, S = page_table.shape
    dev = q.device
    bf16 = (torch.bfloat16, torch.int16)
    _check(q, "q", bf16, (B, HEADS, DIM))
    _check(w, "w", (torch.float32,), (B, HEADS), dev)
    _check(k_pool, "k_pool", bf16, None, dev)
    if k_pool.dim() != 3 or tuple(k_pool.shape[1:]) != (PAGE, DIM):
        raise ValueError(f"k_pool has shape {tuple(k_pool.shape)}, expected [num_pages, {PAGE}, {DIM}]")
    _check(page_table, "page_table", (torch.int32,), None, dev)
    _check(seq_lens, "seq_lens", (torch.int32,), (B,), dev)
    _check(hist, "hist", (torch.int32,), (B, HIST_BINS), dev)
    if out is None:
        out = torch.empty((B, S * PAGE), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (B, S * PAGE), dev)
    if row_hwm is not None:
        _check(row_hwm, "row_hwm", (torch.int32,), (B,), dev)
    st = load().dsa_indexer_score_hist(
        q.data_ptr(), w.data_ptr(), k_pool.data_ptr(), k_pool.shape[0], page_table.data_ptr(),
        seq_lens.data_ptr(), B, S, out.data_ptr(), row_hwm.data_ptr() if row_hwm is not None else None,
        hist.data_ptr(), _stream_ptr(stream))
    if st != 0:
        raise DsaError(st, "dsa_indexer_score_hist")
    return out


def score_fp8(q, w, k8, k_scale, page_table, seq_lens, out=None, row_hwm=None, stream=None):
    """``score`` with fp8 keys: k8 uint8 [num_pages,64,64] e4m3fn codes and
    k_scale float32 [num_pages,64], one scale per key (see the header)."""
    import torch

    B, S = page_table.shape
    dev = q.device
    _check(q, "q", (torch.bfloat16, torch.int16), (B, HEADS, DIM))
    _check(w, "w", (torch.float32,), (B, HEADS), dev)
    _check(k8, "k8", (torch.uint8, torch.int8), None, dev)
    if k8.dim() != 3 or tuple(k8.shape[1:]) != (PAGE, DIM):
        raise ValueError(f"k8 has shape {tuple(k8.shape)}, expected [num_pages, {PAGE}, {DIM}]")
    _check(k_scale, "k_scale", (torch.float32,), (k8.shape[0], PAGE), dev)
    _check(page_table, "page_table", (torch.int32,), None, dev)
    _check(seq_lens, "seq_lens", (torch.int32,), (B,), dev)
    if out is None:
        out = torch.empty((B, S * PAGE), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (B, S * PAGE), dev)
    if row_hwm is not None:
        _check(row_hwm, "row_hwm", (torch.int32,), (B,), dev)
    st = load().dsa_indexer_score_fp8(
        q.data_ptr(), w.data_ptr(), k8.data_ptr(), k_scale.data_ptr(), k8.shape[0], page_table.data_ptr(),
        seq_lens.data_ptr(), B, S, out.data_ptr(), row_hwm.data_ptr() if row_hwm is not None else None,
        _stream_ptr(stream))
    if st != 0:
        raise DsaError(st, "dsa_indexer_score_fp8")
    return out


def score_mtp(q, w, k_pool, page_table, seq_lens, out=None, row_hwm=None, stream=None):
    """Logits [B, T, max_pages*64] (float32) for T query tokens per request.

    q bf16 [B,T,32,64]; w float32 [B,T,32]; k_pool bf16 [num_pages,64,64];
    page_table int32 [B,max_pages]; seq_lens int32 [B,T] (each token's
    length); ``out`` float32 [B,T,max_pages*64] is allocated when not given.
    ``row_hwm`` int32 [B] (one mark per request) selects the incremental tail
    (the caller keeps ``out`` and ``row_hwm`` across calls).
    """
    import torch

    B, S = page_table.shape
    if q.dim() != 4:
        raise ValueError(f"q has shape {tuple(q.shape)}, expected [B, T, {HEADS}, {DIM}]")
    T = q.shape[1]
    dev = q.device
    bf16 = (torch.bfloat16, torch.int16)
    _check(q, "q", bf16, (B, T, HEADS, DIM))
    _check(w, "w", (torch.float32,), (B, T, HEADS), dev)
    _check(k_pool, "k_pool", bf16, None, dev)
    if k_pool.dim() != 3 or tuple(k_pool.shape[1:]) != (PAGE, DIM):
        raise ValueError(f"k_pool has shape {tuple(k_pool.shape)}, expected [num_pages, {PAGE}, {DIM}]")
    _check(page_table, "page_table", (torch.int32,), None, dev)
    _check(seq_lens, "seq_lens", (torch.int32,), (B, T), dev)
    if out is None:
        out = torch.empty((B, T, S * PAGE), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (B, T, S * PAGE), dev)
    if row_hwm is not None:
        _check(row_hwm, "row_hwm", (torch.int32,), (B,), dev)
    st = load().dsa_indexer_score_mtp(
        q.data_ptr(), w.data_ptr(), k_pool.data_ptr(), k_pool.shape[0], page_table.data_ptr(), seq_lens.data_ptr(),
        B, T, S, out.data_ptr(), row_hwm.data_ptr() if row_hwm is not None else None, _stream_ptr(stream))
    if st != 0:
        raise DsaError(st, "dsa_indexer_score_mtp")
    return out


def topk_workspace_bytes(batch: int, max_c4: int, k: int) -> int:
    return int(load().dsa_indexer_topk_workspace_bytes(batch, max_c4, k))


def topk_workspace(batch: int, max_c4: int, k: int, device="cuda"):
    """A top-k workspace for these sizes (a uint8 tensor; None if none is needed)."""
    import torch

    need = topk_workspace_bytes(batch, max_c4, k)
    if need == 0:
        return None
    return torch.empty(need, dtype=torch.uint8, device=device)


_workspaces = {}  # (device, bytes) -> workspace reused by topk() calls that pass none


def topk(logits, seq_lens, k, out_idx=None, out_vals=None, with_values=False, workspace=None,
         stream=None, hist=None):
    """Top-k positions [B, k] (int32, ascending, -1 padded) of each row, and
    their scores [B, k] when ``with_values`` or ``out_vals`` is given. With
    ``hist`` (the histogram score_hist filled for these logits) the call is
    dsa_indexer_topk_hist, which also sets ``hist`` back to zero."""
    import torch

    B, N = logits.shape
    dev = logits.device
    _check(logits, "logits", (torch.float32,), None)
    _check(seq_lens, "seq_lens", (torch.int32,), (B,), dev)
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    _check(out_idx, "out_idx", (torch.int32,), (B, k), dev)
    if out_vals is None and with_values:
        out_vals = torch.empty((B, k), dtype=torch.float32, device=dev)
    if out_vals is not None:
        _check(out_vals, "out_vals", (torch.float32,), (B, k), dev)
    need = topk_workspace_bytes(B, N, k)
    if workspace is None:
        # one cached workspace per device and size: calls in stream order can share
        # it (overlapping calls on other streams need their own)
        key = (str(dev), need)
        if key not in _workspaces:
            _workspaces[key] = topk_workspace(B, N, k, device=dev)
        workspace = _workspaces[key]
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    vals_ptr = out_vals.data_ptr() if out_vals is not None else None
    if hist is not None:
        _check(hist, "hist", (torch.int32,), (B, HIST_BINS), dev)
        st = load().dsa_indexer_topk_hist(logits.data_ptr(), seq_lens.data_ptr(), B, N, k, out_idx.data_ptr(),
                                          vals_ptr, hist.data_ptr(), ws_ptr, ws_bytes, _stream_ptr(stream))
        if st != 0:
            raise DsaError(st, "dsa_indexer_topk_hist")
        return out_idx, out_vals
    st = load().dsa_indexer_topk(
        logits.data_ptr(), seq_lens.data_ptr(), B, N, k, out_idx.data_ptr(), vals_ptr, ws_ptr, ws_bytes,
        _stream_ptr(stream))
    if st != 0:
        raise DsaError(st, "dsa_indexer_topk")
    return out_idx, out_vals


def topk_noalloc(logits, seq_lens, k, out_idx=None, out_vals=None, with_values=False, stream=None):
    """``topk`` through dsa_indexer_topk_noalloc: the workspace is the
    library's fixed device array (for callers that cannot allocate; pass
    ``out_idx`` and ``out_vals`` to allocate nothing here either)."""
    import torch

    B, N = logits.shape
    dev = logits.device
    _check(logits, "logits", (torch.float32,), None)
    _check(seq_lens, "seq_lens", (torch.int32,), (B,), dev)
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    _check(out_idx, "out_idx", (torch.int32,), (B, k), dev)
    if out_vals is None and with_values:
        out_vals = torch.empty((B, k), dtype=torch.float32, device=dev)
    if out_vals is not None:
        _check(out_vals, "out_vals", (torch.float32,), (B, k), dev)
    st = load().dsa_indexer_topk_noalloc(logits.data_ptr(), seq_lens.data_ptr(), B, N, k, out_idx.data_ptr(),
                                         out_vals.data_ptr() if out_vals is not None else None, _stream_ptr(stream))
    if st != 0:
        raise DsaError(st, "dsa_indexer_topk_noalloc")
    return out_idx, out_vals


def sparse_attention_workspace_bytes(batch: int, k: int) -> int:
    return int(load().dsa_indexer_sparse_attention_workspace_bytes(batch, k))


def sparse_attention(q, kv_pool, page_table, idx, scale, out=None, lse=None, workspace=None, stream=None):
    """Attention of 32 heads over each request's selected positions.

    q bf16 [B,32,576]; kv_pool bf16 [num_pages,64,576] (latents, the first
    512 dims the value); page_table int32 [B,max_pages]; idx int32 [B,k]
    (negative entries skipped); returns out float32 [B,32,512] and the
    natural-log lse float32 [B,32] (see the header).
    """
    import torch

    B, k = idx.shape
    dev = q.device
    bf16 = (torch.bfloat16, torch.int16)
    _check(q, "q", bf16, (B, ATT_HEADS, ATT_KD))
    _check(kv_pool, "kv_pool", bf16, None, dev)
    if kv_pool.dim() != 3 or tuple(kv_pool.shape[1:]) != (PAGE, ATT_KD):
        raise ValueError(f"kv_pool has shape {tuple(kv_pool.shape)}, expected [num_pages, {PAGE}, {ATT_KD}]")
    _check(page_table, "page_table", (torch.int32,), None, dev)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError(f"page_table has shape {tuple(page_table.shape)}, expected [{B}, max_pages]")
    _check(idx, "idx", (torch.int32,), None, dev)
    if out is None:
        out = torch.empty((B, ATT_HEADS, ATT_VD), dtype=torch.float32, device=dev)
    _check(out, "out", (torch.float32,), (B, ATT_HEADS, ATT_VD), dev)
    if lse is None:
        lse = torch.empty((B, ATT_HEADS), dtype=torch.float32, device=dev)
    _check(lse, "lse", (torch.float32,), (B, ATT_HEADS), dev)
    need = sparse_attention_workspace_bytes(B, k)
    if workspace is None and need > 0:
        key = (str(dev), need)
        if key not in _workspaces:
            _workspaces[key] = torch.empty(need, dtype=torch.uint8, device=dev)
        workspace = _workspaces[key]
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().dsa_indexer_sparse_attention(
        q.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0], page_table.data_ptr(), B, page_table.shape[1],
        idx.data_ptr(), k, float(scale), out.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes, _stream_ptr(stream))
    if st != 0:
        raise DsaError(st, "dsa_indexer_sparse_attention")
    return out, lse


def attention_to_device(att, device="cuda"):
    """Upload a ``workloads.AttentionInputs`` (queries and latents) to the GPU."""
    import torch

    return {
        "q": torch.from_numpy(att.q_bits.view("int16")).to(device).view(torch.bfloat16),
        "kv_pool": torch.from_numpy(att.kv_bits.view("int16")).to(device).view(torch.bfloat16),
    }


def to_device(inp, device="cuda"):
    """Upload a ``workloads.Inputs`` to the GPU as the tensors ``score`` takes."""
    import torch

    t = {
        "q": torch.from_numpy(inp.q_bits.view("int16")).to(device).view(torch.bfloat16),
        "w": torch.from_numpy(inp.w).to(device),
        "page_table": torch.from_numpy(inp.page_table).to(device),
        "seq_lens": torch.from_numpy(inp.seq_lens).to(device),
    }
    if inp.k_bits is not None:
        t["k_pool"] = torch.from_numpy(inp.k_bits.view("int16")).to(device).view(torch.bfloat16)
    if inp.k8 is not None:
        t["k8"] = torch.from_numpy(inp.k8).to(device)
        t["k_scale"] = torch.from_numpy(inp.k_scale).to(device)
    return t
