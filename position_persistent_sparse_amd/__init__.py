"""Python binding of libppsa.so, the PPSA decode-step library for MI355X.

Argument marshalling only: every function checks tensor shapes, dtypes and
devices, then calls the C entry point of the same name (include/ppsa.h) with
raw device pointers and torch's current HIP stream. All arithmetic happens in
the library's HIP kernels; if the library is missing, import fails loudly.

Tensors: q/out [B, Hq, d]; k_cache/v_cache [B, Hkv, Nmax, d] (bfloat16 or
float32, contiguous, on the GPU); seq_lens [B] int32; idx [B, Hkv, topk]
int32; scores [B, Hkv, Nmax] float32. decode_step takes the same tensors
with a leading layer axis.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libppsa.so")

PPSA_OK, PPSA_ERR_INVALID_ARG, PPSA_ERR_UNSUPPORTED = 0, -1, -2
PPSA_ERR_WORKSPACE, PPSA_ERR_SCHEDULE, PPSA_ERR_HIP, PPSA_ERR_SCRATCH = -3, -4, -5, -6
PPSA_F32, PPSA_BF16 = 0, 1
PPSA_FULL, PPSA_FULL_SELECT, PPSA_SPARSE = 0, 1, 2
KIND_CODES = {"F": PPSA_FULL, "X": PPSA_FULL_SELECT, "S": PPSA_SPARSE}
PPSA_SELECT_PER_KV_HEAD, PPSA_SELECT_SHARED, PPSA_SELECT_SOFTMAX, PPSA_SELECT_COVERAGE = 0, 1, 2, 3
SELECT_MODES = {"kv_head": PPSA_SELECT_PER_KV_HEAD, "shared": PPSA_SELECT_SHARED, "softmax": PPSA_SELECT_SOFTMAX,
                "coverage": PPSA_SELECT_COVERAGE}
PPSA_KERNEL_KINDS = 8
KERNEL_KEYS = ("attn_full", "attn_full_scores", "attn_sparse", "combine", "select", "append",
               "softmax_scores", "coverage")  # ppsa_kernel_kind order


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class PPSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dp = ctypes.POINTER(Dims)
    lib.ppsa_abi_version.restype = ctypes.c_int
    lib.ppsa_status_string.argtypes = [ctypes.c_int]
    lib.ppsa_status_string.restype = ctypes.c_char_p
    lib.ppsa_workspace_bytes.argtypes = [dp, i32]
    lib.ppsa_workspace_bytes.restype = sz
    lib.ppsa_full_attn.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ppsa_full_attn_select.argtypes = [dp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.ppsa_select_topk.argtypes = [dp, vp, vp, i32, vp, vp, sz, vp]
    lib.ppsa_select_topk_ex.argtypes = [dp, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.ppsa_decode_step_ex.argtypes = [dp, i32, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp, vp, vp, sz,
                                        vp]
    lib.ppsa_sparse_attn.argtypes = [dp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
    lib.ppsa_sparse_attn_phases.argtypes = [dp, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.ppsa_decode_step.argtypes = [dp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.ppsa_append_kv.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.ppsa_decode_step_static.argtypes = [dp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    lib.ppsa_set_split_rows.argtypes = [i32, i32]
    lib.ppsa_probe_read.argtypes = [vp, sz, i32, vp, vp]
    lib.ppsa_probe_empty.argtypes = [i32, i32, vp, vp]
    lib.ppsa_probe_gather.argtypes = [dp, vp, vp, vp, vp, i32, i32, vp, vp]
    lib.ppsa_timing_enable.argtypes = [i32]
    lib.ppsa_timing_read.argtypes = [vp, vp, i32, vp]
    lib.ppsa_timing_kernel_name.argtypes = [i32]
    lib.ppsa_timing_kernel_name.restype = ctypes.c_char_p
    for name in ("ppsa_full_attn", "ppsa_full_attn_select", "ppsa_select_topk", "ppsa_sparse_attn",
                 "ppsa_sparse_attn_phases",
                 "ppsa_decode_step", "ppsa_append_kv", "ppsa_timing_enable", "ppsa_timing_read",
                 "ppsa_select_topk_ex", "ppsa_decode_step_ex", "ppsa_decode_step_static", "ppsa_set_split_rows",
                 "ppsa_probe_read",
                 "ppsa_probe_empty", "ppsa_probe_gather"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load()


def abi_version() -> int:
    return _lib.ppsa_abi_version()


def status_string(status: int) -> str:
    return _lib.ppsa_status_string(int(status)).decode()


def make_dims(batch, q_heads, kv_heads, head_dim, max_seq_len, dtype, scale: float = 0.0) -> Dims:
    code = {torch.float32: PPSA_F32, torch.bfloat16: PPSA_BF16}.get(dtype, dtype)
    return Dims(int(batch), int(q_heads), int(kv_heads), int(head_dim), int(max_seq_len), int(code), float(scale))


def workspace_bytes(dims: Dims, topk: int = 0) -> int:
    return int(_lib.ppsa_workspace_bytes(ctypes.byref(dims), int(topk)))


def alloc_workspace(dims: Dims, topk: int = 0, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(dims, topk), 16), dtype=torch.uint8, device=device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, where: str):
    if status != PPSA_OK:
        raise PPSAError(status, where)


def _dims_of(q, k_cache, scale, layered=False):
    if layered:
        _, B, Hq, d = q.shape
        _, _, Hkv, N, _ = k_cache.shape
    else:
        B, Hq, d = q.shape
        _, Hkv, N, _ = k_cache.shape
    return make_dims(B, Hq, Hkv, d, N, q.dtype, scale)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_buffer(t, shape, dtype, device, name):
    """A caller-provided output or state buffer: the library writes it by shape, so it must match."""
    _require(tuple(t.shape) == tuple(int(x) for x in shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous() and t.device == device, f"{name} must be contiguous on {device}")


def _workspace_nbytes(ws, device):
    _require(ws.is_contiguous() and ws.device == device, "workspace must be contiguous on the tensors' device")
    return ws.numel() * ws.element_size()


def _check_tensors(q, k_cache, v_cache, seq_lens, layered=False):
    nd = 4 if layered else 3
    _require(q.dim() == nd and k_cache.dim() == nd + 1, "q must be [(L,) B, Hq, d] and K [(L,) B, Hkv, N, d]")
    _require(k_cache.shape == v_cache.shape, "K and V shapes differ")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q, K and V must share a dtype")
    _require(q.shape[-1] == k_cache.shape[-1], "head_dim mismatch")
    _require(q.shape[-3] == k_cache.shape[-4], "batch mismatch")
    if layered:
        _require(q.shape[0] == k_cache.shape[0], "layer count mismatch")
    for t in (q, k_cache, v_cache, seq_lens):
        _require(t.is_cuda and t.is_contiguous(), "tensors must be contiguous GPU tensors")
    _require(seq_lens.dtype == torch.int32 and seq_lens.shape == (q.shape[-3],), "seq_lens must be int32 [B]")
    _require(q.device == k_cache.device == v_cache.device == seq_lens.device, "tensors must share one device")


def full_attn(q, k_cache, v_cache, seq_lens, out=None, workspace=None, scale: float = 0.0):
    _check_tensors(q, k_cache, v_cache, seq_lens)
    dims = _dims_of(q, k_cache, scale)
    out = torch.empty_like(q) if out is None else out
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    ws = alloc_workspace(dims, 0, q.device) if workspace is None else workspace
    _check(_lib.ppsa_full_attn(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                               _ptr(out), _ptr(ws), _workspace_nbytes(ws, q.device), _stream(q.device)),
           "ppsa_full_attn")
    return out


def full_attn_select(q, k_cache, v_cache, seq_lens, topk: int, out=None, scores=None, idx=None, workspace=None,
                     scale: float = 0.0):
    _check_tensors(q, k_cache, v_cache, seq_lens)
    dims = _dims_of(q, k_cache, scale)
    out = torch.empty_like(q) if out is None else out
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    if idx is None:
        idx = torch.empty((dims.batch, dims.num_kv_heads, int(topk)), dtype=torch.int32, device=q.device)
    _check_buffer(idx, (dims.batch, dims.num_kv_heads, int(topk)), torch.int32, q.device, "idx")
    if scores is not None:
        _check_buffer(scores, (dims.batch, dims.num_kv_heads, dims.max_seq_len), torch.float32, q.device, "scores")
    ws = alloc_workspace(dims, topk, q.device) if workspace is None else workspace
    _check(_lib.ppsa_full_attn_select(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                      int(topk), _ptr(out), _ptr(scores), _ptr(idx), _ptr(ws),
                                      _workspace_nbytes(ws, q.device), _stream(q.device)), "ppsa_full_attn_select")
    return out, idx


def select_topk(scores, seq_lens, topk: int, idx=None, num_q_heads=None, mode: str = "kv_head",
                workspace=None, two_stage: bool = True):
    """Top-k per (batch row, KV head), or per batch row over the KV heads' summed scores (mode "shared").
    With `two_stage` (default) a workspace is passed (allocated when not given), so that long rows are
    selected in two launches; two_stage=False passes none (one launch)."""
    _require(scores.dim() == 3 and scores.dtype == torch.float32 and scores.is_contiguous() and scores.is_cuda,
             "scores must be contiguous float32 [B, Hkv, N] on the GPU")
    B, Hkv, N = scores.shape
    _check_buffer(seq_lens, (B,), torch.int32, scores.device, "seq_lens")
    dims = make_dims(B, num_q_heads or Hkv, Hkv, 128, N, PPSA_F32)
    if idx is None:
        idx = torch.empty((B, Hkv, int(topk)), dtype=torch.int32, device=scores.device)
    _check_buffer(idx, (B, Hkv, int(topk)), torch.int32, scores.device, "idx")
    ws = None
    if two_stage:
        ws = alloc_workspace(dims, topk, scores.device) if workspace is None else workspace
    _check(_lib.ppsa_select_topk_ex(ctypes.byref(dims), _ptr(scores), _ptr(seq_lens), int(topk), SELECT_MODES[mode],
                                    _ptr(idx), _ptr(ws), 0 if ws is None else _workspace_nbytes(ws, scores.device),
                                    _stream(scores.device)), "ppsa_select_topk_ex")
    return idx


PHASE_ATTN = 1
PHASE_MERGE = 2


def sparse_attn(q, k_cache, v_cache, seq_lens, idx, out=None, workspace=None, scale: float = 0.0,
                phases: int = PHASE_ATTN | PHASE_MERGE):
    """Sparse attention over idx [B, Hkv, topk]. `phases` picks the attention launch, the merge launch or both
    (ppsa_sparse_attn_phases); a merge-only call completes an attention-only call on the same workspace."""
    _require(phases in (1, 2, 3), "phases must be PHASE_ATTN, PHASE_MERGE or both")
    _check_tensors(q, k_cache, v_cache, seq_lens)
    dims = _dims_of(q, k_cache, scale)
    _require(idx.dtype == torch.int32 and idx.is_contiguous() and idx.dim() == 3
             and tuple(idx.shape[:2]) == (dims.batch, dims.num_kv_heads), "idx must be int32 [B, Hkv, topk]")
    _require(idx.device == q.device, "idx must be on the tensors' device")
    topk = idx.shape[2]
    out = torch.empty_like(q) if out is None else out
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    ws = alloc_workspace(dims, topk, q.device) if workspace is None else workspace
    _check(_lib.ppsa_sparse_attn_phases(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                        _ptr(idx), int(topk), int(phases), _ptr(out), _ptr(ws),
                                        _workspace_nbytes(ws, q.device), _stream(q.device)),
           "ppsa_sparse_attn_phases")
    return out


def schedule_codes(schedule) -> ctypes.Array:
    codes = [KIND_CODES[k] if isinstance(k, str) else int(k) for k in schedule]
    return (ctypes.c_int32 * max(len(codes), 1))(*codes)


def decode_step(schedule, q, k_cache, v_cache, seq_lens, topk: int, out=None, idx=None, scores=None,
                workspace=None, scale: float = 0.0, sched_codes=None, select_mode: str = "kv_head",
                coverage_tau: float = 0.0):
    """One decode step; returns (out [L,B,Hq,d], idx [S,B,Hkv,topk]) with S = selection layers."""
    _check_tensors(q, k_cache, v_cache, seq_lens, layered=True)
    dims = _dims_of(q, k_cache, scale, layered=True)
    L = q.shape[0]
    _require(len(schedule) == L, "schedule length must equal the layer count")
    n_sel = sum(1 for k in schedule if k in ("X", PPSA_FULL_SELECT))
    out = torch.empty_like(q) if out is None else out
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    if idx is None and n_sel:
        idx = torch.empty((n_sel, dims.batch, dims.num_kv_heads, int(topk)), dtype=torch.int32, device=q.device)
    if n_sel:
        _check_buffer(idx, (n_sel, dims.batch, dims.num_kv_heads, int(topk)), torch.int32, q.device, "idx")
    if scores is not None:
        _check_buffer(scores, (n_sel, dims.batch, dims.num_kv_heads, dims.max_seq_len), torch.float32, q.device,
                      "scores")
    ws = alloc_workspace(dims, topk if n_sel else 0, q.device) if workspace is None else workspace
    codes = schedule_codes(schedule) if sched_codes is None else sched_codes
    _check(_lib.ppsa_decode_step_ex(ctypes.byref(dims), L, codes, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(seq_lens), int(topk), SELECT_MODES[select_mode], float(coverage_tau),
                                    _ptr(out), _ptr(idx),
                                    _ptr(scores), _ptr(ws), _workspace_nbytes(ws, q.device), _stream(q.device)),
           "ppsa_decode_step_ex")
    return out, idx


def decode_step_static(schedule, q, k_cache, v_cache, seq_lens, topk: int, out=None, idx=None, scores=None,
                       scale: float = 0.0, sched_codes=None):
    """decode_step (default selection) on the library's static device scratch: no workspace. Output
    tensors are still the caller's (allocated here when not given)."""
    _check_tensors(q, k_cache, v_cache, seq_lens, layered=True)
    dims = _dims_of(q, k_cache, scale, layered=True)
    L = q.shape[0]
    _require(len(schedule) == L, "schedule length must equal the layer count")
    n_sel = sum(1 for k in schedule if k in ("X", PPSA_FULL_SELECT))
    out = torch.empty_like(q) if out is None else out
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    if idx is None and n_sel:
        idx = torch.empty((n_sel, dims.batch, dims.num_kv_heads, int(topk)), dtype=torch.int32, device=q.device)
    if n_sel:
        _check_buffer(idx, (n_sel, dims.batch, dims.num_kv_heads, int(topk)), torch.int32, q.device, "idx")
    if scores is not None:
        _check_buffer(scores, (n_sel, dims.batch, dims.num_kv_heads, dims.max_seq_len), torch.float32, q.device,
                      "scores")
    codes = schedule_codes(schedule) if sched_codes is None else sched_codes
    _check(_lib.ppsa_decode_step_static(ctypes.byref(dims), L, codes, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(seq_lens), int(topk), _ptr(out), _ptr(idx), _ptr(scores),
                                        _stream(q.device)), "ppsa_decode_step_static")
    return out, idx


def append_kv(k_new, v_new, k_cache, v_cache, seq_lens, overflow=None):
    """Append one token: k_new/v_new [L,B,Hkv,d] go to row seq_lens[b] of the caches [L,B,Hkv,Nmax,d];
    seq_lens (device int32) grows by one per batch row with room. A full row (seq_lens[b] == Nmax) drops
    its token: the caller must keep within capacity, and can pass `overflow` (a device int32 [1] tensor)
    to which the number of dropped tokens is added."""
    _require(k_cache.dim() == 5 and v_cache.shape == k_cache.shape, "k_cache/v_cache must be [L,B,Hkv,Nmax,d]")
    L, B, Hkv, n_max, d = k_cache.shape
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _require(tuple(t.shape) == (L, B, Hkv, d), f"{name} must be [L,B,Hkv,d] = {(L, B, Hkv, d)}")
        _require(t.dtype == k_cache.dtype and t.is_contiguous() and t.device == k_cache.device,
                 f"{name}: dtype/device/layout must match the cache")
    _require(v_cache.dtype == k_cache.dtype and k_cache.is_contiguous() and v_cache.is_contiguous(),
             "caches must be contiguous with one dtype")
    _require(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,) and seq_lens.device == k_cache.device,
             "seq_lens must be int32 [B] on the cache's device")
    if overflow is not None:
        _require(overflow.dtype == torch.int32 and overflow.numel() >= 1 and overflow.device == k_cache.device,
                 "overflow must be a device int32 tensor")
    dims = make_dims(B, Hkv, Hkv, d, n_max, k_cache.dtype)
    _check(_lib.ppsa_append_kv(ctypes.byref(dims), L, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                               _ptr(seq_lens), _ptr(overflow), _stream(k_cache.device)), "ppsa_append_kv")


def timing_enable(capacity: int):
    """Switch launch timing on with an event pool for `capacity` launches (0 switches it off)."""
    _check(_lib.ppsa_timing_enable(int(capacity)), "ppsa_timing_enable")


def timing_read() -> dict:
    """{kernel key: (launches, total ms)} since the previous read, plus "dropped" (untimed launches)."""
    counts = (ctypes.c_int32 * PPSA_KERNEL_KINDS)()
    ms = (ctypes.c_double * PPSA_KERNEL_KINDS)()
    dropped = ctypes.c_int64()
    _check(_lib.ppsa_timing_read(counts, ms, PPSA_KERNEL_KINDS, ctypes.byref(dropped)), "ppsa_timing_read")
    res = {key: (int(counts[i]), float(ms[i])) for i, key in enumerate(KERNEL_KEYS)}
    res["dropped"] = int(dropped.value)
    return res


def timing_kernel_name(kind: int) -> str:
    return _lib.ppsa_timing_kernel_name(int(kind)).decode()


def set_split_rows(full_rows: int = 0, sparse_rows: int = 0):
    """Planner override (process-wide): rows per split of full and sparse layers; 0 = automatic."""
    _check(_lib.ppsa_set_split_rows(int(full_rows), int(sparse_rows)), "ppsa_set_split_rows")


def probe_read(buf, nontemporal: bool, sink):
    """Measurement probe: one read of the whole byte buffer `buf` (a multiple of 32 KiB)."""
    _check(_lib.ppsa_probe_read(_ptr(buf), buf.numel() * buf.element_size(), int(bool(nontemporal)), _ptr(sink),
                                _stream(buf.device)), "ppsa_probe_read")


def probe_empty(groups: int, threads: int, sink):
    """Measurement probe: one empty kernel launch."""
    _check(_lib.ppsa_probe_empty(int(groups), int(threads), _ptr(sink), _stream(sink.device)), "ppsa_probe_empty")


def probe_gather(k_cache, v_cache, seq_lens, idx, q_heads: int, sink, repeats: int = 1, scale: float = 0.0):
    """Measurement probe: `repeats` back-to-back launches of the load-only twin of sparse_attn's kernel over
    K/V [B,Hkv,N,d] and idx [B,Hkv,k]."""
    B, Hkv, N, d = k_cache.shape
    dims = make_dims(B, q_heads, Hkv, d, N, k_cache.dtype, scale)
    _check(_lib.ppsa_probe_gather(ctypes.byref(dims), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(idx),
                                  int(idx.shape[-1]), int(repeats), _ptr(sink), _stream(k_cache.device)),
           "ppsa_probe_gather")


def raw_library():
    """The ctypes handle itself, for callers that manage pointers directly."""
    return _lib
