"""ctypes binding of libdsa_sparse_mla.so: argument marshalling only.

Every step of the forward runs in the HIP kernels behind the C ABI
(include/dsa_sparse_mla.h). torch supplies device memory and the current
stream, nothing else. If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

# DSA_SPARSE_MLA_LIB names another build of the same library (for example a
# host-sanitizer build); by default the one built next to this file.
LIB_PATH = os.environ.get("DSA_SPARSE_MLA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                                "libdsa_sparse_mla.so")
DQK = 576
DV = 512

_lock = threading.Lock()
_lib = None

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP error", 4: "workspace too small"}


class DsaError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().dsa_status_string(status).decode()} (status {status})")


def lib() -> ctypes.CDLL:
    """Load the library once. torch is imported first, so the library binds to
    the HIP runtime torch already mapped (both carry soname libamdhip64.so.7)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python dsa_sparse_mla_amd/build.py` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        L.dsa_sparse_mla_fwd.restype = ctypes.c_int
        L.dsa_sparse_mla_fwd.argtypes = [
            vp, i64, i64,            # q
            vp, i64, i64,            # kv, row stride, num_kv
            vp, i64,                 # indices
            i64, i32, i32, f32,      # T, H, topk, sm_scale
            vp, i64, i64,            # out
            vp, i64,                 # lse
            i32, vp, i64,            # num_splits, workspace, bytes
            vp]                      # stream
        L.dsa_sparse_mla_fwd_paged.restype = ctypes.c_int
        L.dsa_sparse_mla_fwd_paged.argtypes = [
            vp, i64, i64,            # q
            vp, i64, i64, i64, i32,  # kv_pages, page stride, row stride, num_pages, page_size
            vp, i64, i32, vp,        # page_table, stride, max_pages, seq_lens
            vp, i64,                 # indices
            i32, i32, i32, i32, f32,  # num_seqs, q_per_seq, H, topk, sm_scale
            vp, i64, i64,            # out
            vp, i64,                 # lse
            i32, vp, i64,            # num_splits, workspace, bytes
            vp]                      # stream
        L.dsa_sparse_mla_fwd_paged_fp8.restype = ctypes.c_int
        L.dsa_sparse_mla_fwd_paged_fp8.argtypes = L.dsa_sparse_mla_fwd_paged.argtypes
        L.dsa_sparse_mla_fwd_paged_noalloc.restype = ctypes.c_int
        # the paged arguments up to num_splits, without workspace/bytes
        L.dsa_sparse_mla_fwd_paged_noalloc.argtypes = L.dsa_sparse_mla_fwd_paged.argtypes[:-3] + [
            vp]                      # stream
        L.dsa_sparse_mla_bwd.restype = ctypes.c_int
        L.dsa_sparse_mla_bwd.argtypes = [
            vp, i64, i64,            # q
            vp, i64, i64,            # kv, row stride, num_kv
            vp, i64,                 # indices
            i64, i32, i32, f32,      # T, H, topk, sm_scale
            vp, i64, i64,            # out (forward output)
            vp, i64,                 # lse (forward LSE)
            vp, i64, i64,            # dout
            vp, i64, i64,            # dq
            vp, i64,                 # dkv, row stride
            vp, i64,                 # workspace, bytes
            vp]                      # stream
        L.dsa_sparse_mla_bwd_workspace_size.restype = ctypes.c_int
        L.dsa_sparse_mla_bwd_workspace_size.argtypes = [i64, i32, i64, i32,
                                                        ctypes.POINTER(i32), ctypes.POINTER(i64)]
        L.dsa_sparse_mla_workspace_size.restype = ctypes.c_int
        L.dsa_sparse_mla_workspace_size.argtypes = [i64, i32, i32, i32,
                                                    ctypes.POINTER(i32), ctypes.POINTER(i64)]
        L.dsa_topk_indices.restype = ctypes.c_int
        L.dsa_topk_indices.argtypes = [
            vp, i64, i64,            # scores, row stride, num_cols
            vp, vp,                  # key_start, key_end
            i64, i32,                # num_tokens, topk
            vp, i64,                 # indices, row stride
            vp]                      # stream
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_status_string.argtypes = [ctypes.c_int]
        L.dsa_device_supported.restype = ctypes.c_int
        L.dsa_device_supported.argtypes = [ctypes.c_int]
        L.dsa_version.restype = ctypes.c_int
        L.dsa_version.argtypes = []
        _lib = L
        return _lib


def workspace_size(num_tokens: int, num_heads: int, topk: int, num_splits: int = 0):
    """(splits, bytes) that a forward call with these sizes uses on the current device."""
    s = ctypes.c_int32(0)
    b = ctypes.c_int64(0)
    st = lib().dsa_sparse_mla_workspace_size(num_tokens, num_heads, topk, num_splits,
                                             ctypes.byref(s), ctypes.byref(b))
    if st != 0:
        raise DsaError(st, "dsa_sparse_mla_workspace_size")
    return s.value, b.value


BWD_SCHEDULES = {0: "token-major", 1: "kv-major", 2: "split"}


def bwd_workspace_size(num_tokens: int, num_heads: int, num_kv: int, topk: int):
    """(schedule name, bytes) that a backward call with these sizes uses."""
    s = ctypes.c_int32(0)
    b = ctypes.c_int64(0)
    st = lib().dsa_sparse_mla_bwd_workspace_size(num_tokens, num_heads, num_kv, topk,
                                                 ctypes.byref(s), ctypes.byref(b))
    if st != 0:
        raise DsaError(st, "dsa_sparse_mla_bwd_workspace_size")
    return BWD_SCHEDULES[s.value], b.value


def _check(t: torch.Tensor, name: str, dtype, ndim: int, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() and t.stride(-1) != 1:
        raise ValueError(f"{name} needs a contiguous last dimension")


def _outputs(q, T, H, out, lse):
    if out is None:
        out = torch.empty((T, H, DV), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _check(out, "out", torch.bfloat16, 3, q.device)
    _check(lse, "lse", torch.float32, 2, q.device)
    if tuple(out.shape) != (T, H, DV) or tuple(lse.shape) != (T, H):
        raise ValueError("out must be [T, H, 512] and lse [T, H]")
    return out, lse


def _workspace(q, T, H, topk, num_splits, workspace):
    _, need = workspace_size(T, H, topk, num_splits)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    return workspace, workspace.numel() * workspace.element_size()


def sparse_mla_fwd(q, kv, indices, sm_scale, out=None, lse=None, num_splits=0, workspace=None):
    """Sparse MLA forward over flat KV (packed/varlen prefill).

    q [T,H,576] bf16, kv [N,576] bf16, indices [T,topk] int32 (row ids; -1 or
    any out-of-range value is padding). Returns (out [T,H,512] bf16, lse [T,H] fp32).
    Runs on torch's current stream of q's device.
    """
    dev = q.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(kv, "kv", torch.bfloat16, 2, dev)
    _check(indices, "indices", torch.int32, 2, dev)
    T, H, D = q.shape
    if D != DQK or kv.shape[1] != DQK:
        raise ValueError("q and kv rows must be 576 wide")
    if indices.shape[0] != T:
        raise ValueError("indices must have one row per token")
    topk = indices.shape[1]
    out, lse = _outputs(q, T, H, out, lse)
    ws, ws_bytes = _workspace(q, T, H, topk, num_splits, workspace)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib().dsa_sparse_mla_fwd(
            q.data_ptr(), q.stride(0), q.stride(1),
            kv.data_ptr(), kv.stride(0), kv.shape[0],
            indices.data_ptr(), indices.stride(0),
            T, H, topk, float(sm_scale),
            out.data_ptr(), out.stride(0), out.stride(1),
            lse.data_ptr(), lse.stride(0),
            int(num_splits), ws.data_ptr() if ws is not None else None, ws_bytes,
            stream)
    if st != 0:
        raise DsaError(st, "dsa_sparse_mla_fwd")
    return out, lse


def sparse_mla_fwd_paged(q, kv_pages, page_table, seq_lens, indices, sm_scale, q_per_seq,
                         out=None, lse=None, num_splits=0, workspace=None):
    """Sparse MLA forward over a paged bf16 cache (decode), no gather copy.

    q [S*q_per_seq, H, 576] bf16; kv_pages [P, page_size, 576] bf16;
    page_table [S, max_pages] int32; seq_lens [S] int32; indices
    [S*q_per_seq, topk] int32 logical positions. Returns (out, lse).
    """
    dev = q.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(kv_pages, "kv_pages", torch.bfloat16, 3, dev)
    _check(page_table, "page_table", torch.int32, 2, dev)
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check(indices, "indices", torch.int32, 2, dev)
    T, H, D = q.shape
    S = page_table.shape[0]
    if D != DQK or kv_pages.shape[2] != DQK:
        raise ValueError("q and kv rows must be 576 wide")
    if seq_lens.shape[0] != S or T != S * q_per_seq or indices.shape[0] != T:
        raise ValueError("need num_seqs * q_per_seq query tokens and one seq_len per sequence")
    topk = indices.shape[1]
    out, lse = _outputs(q, T, H, out, lse)
    ws, ws_bytes = _workspace(q, T, H, topk, num_splits, workspace)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib().dsa_sparse_mla_fwd_paged(
            q.data_ptr(), q.stride(0), q.stride(1),
            kv_pages.data_ptr(), kv_pages.stride(0), kv_pages.stride(1),
            kv_pages.shape[0], kv_pages.shape[1],
            page_table.data_ptr(), page_table.stride(0), page_table.shape[1], seq_lens.data_ptr(),
            indices.data_ptr(), indices.stride(0),
            S, int(q_per_seq), H, topk, float(sm_scale),
            out.data_ptr(), out.stride(0), out.stride(1),
            lse.data_ptr(), lse.stride(0),
            int(num_splits), ws.data_ptr() if ws is not None else None, ws_bytes,
            stream)
    if st != 0:
        raise DsaError(st, "dsa_sparse_mla_fwd_paged")
    return out, lse


FP8_ROW_BYTES = 656


def sparse_mla_fwd_paged_fp8(q, kv_pages, page_table, seq_lens, indices, sm_scale, q_per_seq,
                             out=None, lse=None, num_splits=0, workspace=None):
    """Sparse MLA forward over a paged FP8 MLA cache (decode), no gather copy.

    kv_pages: uint8 [P, page_size, >= 656] FP8 MLA rows (512 e4m3 latent values
    in 4 groups of 128, 4 fp32 scales, 64 bf16 rope values); the other
    arguments as in sparse_mla_fwd_paged (at most 32 heads).
    """
    dev = q.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(kv_pages, "kv_pages", torch.uint8, 3, dev)
    _check(page_table, "page_table", torch.int32, 2, dev)
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check(indices, "indices", torch.int32, 2, dev)
    T, H, D = q.shape
    S = page_table.shape[0]
    if D != DQK or kv_pages.shape[2] < FP8_ROW_BYTES:
        raise ValueError("q rows must be 576 wide and FP8 cache rows at least 656 bytes")
    if seq_lens.shape[0] != S or T != S * q_per_seq or indices.shape[0] != T:
        raise ValueError("need num_seqs * q_per_seq query tokens and one seq_len per sequence")
    topk = indices.shape[1]
    out, lse = _outputs(q, T, H, out, lse)
    ws, ws_bytes = _workspace(q, T, H, topk, num_splits, workspace)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib().dsa_sparse_mla_fwd_paged_fp8(
            q.data_ptr(), q.stride(0), q.stride(1),
            kv_pages.data_ptr(), kv_pages.stride(0), kv_pages.stride(1),
            kv_pages.shape[0], kv_pages.shape[1],
            page_table.data_ptr(), page_table.stride(0), page_table.shape[1], seq_lens.data_ptr(),
            indices.data_ptr(), indices.stride(0),
            S, int(q_per_seq), H, topk, float(sm_scale),
            out.data_ptr(), out.stride(0), out.stride(1),
            lse.data_ptr(), lse.stride(0),
            int(num_splits), ws.data_ptr() if ws is not None else None, ws_bytes,
            stream)
    if st != 0:
        raise DsaError(st, "dsa_sparse_mla_fwd_paged_fp8")
    return out, lse


def sparse_mla_fwd_paged_noalloc(q, kv_pages, page_table, seq_lens, indices, sm_scale, q_per_seq,
                                 out, lse, num_splits=0):
    """sparse_mla_fwd_paged for callers that cannot allocate: out and lse are
    required, and the split partials go to the library's own fixed-size
    device scratch (DSA_NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace.
    Calls on one GPU that may overlap in time race on that scratch."""
    dev = q.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(kv_pages, "kv_pages", torch.bfloat16, 3, dev)
    _check(page_table, "page_table", torch.int32, 2, dev)
    _check(seq_lens, "seq_lens", torch.int32, 1, dev)
    _check(indices, "indices", torch.int32, 2, dev)
    T, H, D = q.shape
    S = page_table.shape[0]
    if D != DQK or kv_pages.shape[2] != DQK:
        raise ValueError("q and kv rows must be 576 wide")
    if seq_lens.shape[0] != S or T != S * q_per_seq or indices.shape[0] != T:
        raise ValueError("need num_seqs * q_per_seq query tokens and one seq_len per sequence")
    if out is None or lse is None:
        raise ValueError("out and lse must be given (this entry point allocates nothing)")
    out, lse = _outputs(q, T, H, out, lse)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib().dsa_sparse_mla_fwd_paged_noalloc(
            q.data_ptr(), q.stride(0), q.stride(1),
            kv_pages.data_ptr(), kv_pages.stride(0), kv_pages.stride(1),
            kv_pages.shape[0], kv_pages.shape[1],
            page_table.data_ptr(), page_table.stride(0), page_table.shape[1], seq_lens.data_ptr(),
            indices.data_ptr(), indices.stride(0),
            S, int(q_per_seq), H, indices.shape[1], float(sm_scale),
            out.data_ptr(), out.stride(0), out.stride(1),
            lse.data_ptr(), lse.stride(0),
            int(num_splits), stream)
    if st != 0:
        raise DsaError(st, "dsa_sparse_mla_fwd_paged_noalloc")
    return out, lse


def topk_indices(scores, key_start, key_end, topk, indices=None, num_cols=None):
    """Top-k index rows from indexer scores (dsa_topk_indices).

    scores [T, num_cols] fp32 (or None when no row has more than topk
    candidates); key_start, key_end [T] int32: token t's candidates are the
    columns key_start[t] <= j < key_end[t]. Returns indices [T, topk] int32:
    the selected columns ascending, then -1. Rows with at most topk
    candidates select all of them without reading scores.
    """
    dev = key_start.device
    _check(key_start, "key_start", torch.int32, 1, dev)
    _check(key_end, "key_end", torch.int32, 1, dev)
    T = key_start.shape[0]
    if key_end.shape[0] != T:
        raise ValueError("key_start and key_end need one entry per token")
    if scores is not None:
        _check(scores, "scores", torch.float32, 2, dev)
        if scores.shape[0] != T:
            raise ValueError("scores need one row per token")
        if num_cols is None:
            num_cols = scores.shape[1]
        elif num_cols != scores.shape[1]:
            raise ValueError("num_cols differs from the score rows")
    elif num_cols is None:
        raise ValueError("num_cols is needed without scores")
    if indices is None:
        indices = torch.empty((T, topk), dtype=torch.int32, device=dev)
    _check(indices, "indices", torch.int32, 2, dev)
    if tuple(indices.shape) != (T, topk):
        raise ValueError("indices must be [T, topk]")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib().dsa_topk_indices(
            scores.data_ptr() if scores is not None else None,
            scores.stride(0) if scores is not None else 0, int(num_cols),
            key_start.data_ptr(), key_end.data_ptr(), T, int(topk),
            indices.data_ptr(), indices.stride(0), stream)
    if st != 0:
        raise DsaError(st, "dsa_topk_indices")
    return indices


def sparse_mla_bwd(q, kv, indices, sm_scale, out, lse, dout, dq=None, dkv=None, workspace=None):
    """Sparse MLA backward over flat KV: gradients of the forward output.

    q [T,H,576] bf16, kv [N,576] bf16, indices [T,topk] int32 as in the
    forward; out [T,H,512] bf16 and lse [T,H] fp32 from the forward on these
    inputs; dout [T,H,512] bf16. Returns (dq [T,H,576] fp32, dkv [N,576] fp32);
    dkv is written in full (rows no index names are 0). The workspace (a
    uint8 device tensor of at least bwd_workspace_size() bytes) is allocated
    here with torch when the schedule needs one and none is given.
    """
    dev = q.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(kv, "kv", torch.bfloat16, 2, dev)
    _check(indices, "indices", torch.int32, 2, dev)
    _check(dout, "dout", torch.bfloat16, 3, dev)
    T, H, D = q.shape
    N = kv.shape[0]
    if D != DQK or kv.shape[1] != DQK:
        raise ValueError("q and kv rows must be 576 wide")
    if indices.shape[0] != T or tuple(dout.shape) != (T, H, DV):
        raise ValueError("indices need one row per token and dout the shape of out")
    _check(out, "out", torch.bfloat16, 3, dev)
    _check(lse, "lse", torch.float32, 2, dev)
    if tuple(out.shape) != (T, H, DV) or tuple(lse.shape) != (T, H):
        raise ValueError("out must be [T, H, 512] and lse [T, H]")
    if dq is None:
        dq = torch.empty((T, H, DQK), dtype=torch.float32, device=dev)
    if dkv is None:
        dkv = torch.empty((N, DQK), dtype=torch.float32, device=dev)
    _check(dq, "dq", torch.float32, 3, dev)
    _check(dkv, "dkv", torch.float32, 2, dev)
    if tuple(dq.shape) != (T, H, DQK) or tuple(dkv.shape) != (N, DQK):
        raise ValueError("dq must be [T, H, 576] and dkv [N, 576]")
    _, need = bwd_workspace_size(T, H, N, indices.shape[1])
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib().dsa_sparse_mla_bwd(
            q.data_ptr(), q.stride(0), q.stride(1),
            kv.data_ptr(), kv.stride(0), N,
            indices.data_ptr(), indices.stride(0),
            T, H, indices.shape[1], float(sm_scale),
            out.data_ptr(), out.stride(0), out.stride(1),
            lse.data_ptr(), lse.stride(0),
            dout.data_ptr(), dout.stride(0), dout.stride(1),
            dq.data_ptr(), dq.stride(0), dq.stride(1),
            dkv.data_ptr(), dkv.stride(0),
            ws_ptr, ws_bytes,
            stream)
    if st != 0:
        raise DsaError(st, "dsa_sparse_mla_bwd")
    return dq, dkv
