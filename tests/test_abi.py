"""C ABI checks that need no GPU: exports, status text, workspace sizing and
every argument-validation path (validation runs before any HIP call)."""
import ctypes
import os
import re

import pytest

import position_persistent_sparse_amd as ppsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = ppsa.raw_library()
FAKE = ctypes.c_void_p(0x100000)      # 16-byte aligned, never dereferenced on failing paths
ODD = ctypes.c_void_p(0x100004)       # misaligned for 16-byte operands


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ppsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ppsa_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(LIB, name), name


def test_abi_version_and_status_strings():
    assert ppsa.abi_version() == 2
    assert ppsa.status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5, -6):
        assert ppsa.status_string(code) not in ("ok", "unknown status")
    assert ppsa.status_string(99) == "unknown status"


def dims(**kw):
    base = dict(batch=2, q_heads=8, kv_heads=2, head_dim=128, max_seq_len=1000, dtype=ppsa.PPSA_BF16, scale=0.0)
    base.update(kw)
    return ppsa.make_dims(base["batch"], base["q_heads"], base["kv_heads"], base["head_dim"],
                          base["max_seq_len"], base["dtype"], base["scale"])


def full(d, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, ws=FAKE, ws_bytes=None):
    wsb = ppsa.workspace_bytes(d, 0) if ws_bytes is None else ws_bytes
    return LIB.ppsa_full_attn(ctypes.byref(d), q, k, v, lens, out, ws, wsb, None)


def sparse(d, topk=16, idx=FAKE, ws_bytes=None, q=FAKE):
    wsb = ppsa.workspace_bytes(d, topk) if ws_bytes is None else ws_bytes
    return LIB.ppsa_sparse_attn(ctypes.byref(d), q, FAKE, FAKE, FAKE, idx, topk, FAKE, FAKE, wsb, None)


def select(d, topk=16, idx=FAKE, scores=FAKE):
    return LIB.ppsa_full_attn_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, topk, FAKE, scores, idx, FAKE,
                                     ppsa.workspace_bytes(d, topk), None)


def step(d, schedule, topk=16, idx=FAKE):
    codes = ppsa.schedule_codes(schedule)
    return LIB.ppsa_decode_step(ctypes.byref(d), len(schedule), codes, FAKE, FAKE, FAKE, FAKE, topk, FAKE, idx,
                                None, FAKE, ppsa.workspace_bytes(d, topk), None)


def test_workspace_bytes():
    d = dims()
    assert ppsa.workspace_bytes(d, 0) > 0
    assert ppsa.workspace_bytes(d, 64) >= ppsa.workspace_bytes(d, 0)
    assert ppsa.workspace_bytes(d, 64) % 256 == 0
    assert ppsa.workspace_bytes(dims(head_dim=96), 0) == 0
    assert ppsa.workspace_bytes(d, -1) == 0
    # The workspace always holds a scores buffer for full+select without caller scores.
    assert ppsa.workspace_bytes(d, 0) >= 2 * 2 * 1000 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), ppsa.PPSA_ERR_UNSUPPORTED),
    (dict(head_dim=0), ppsa.PPSA_ERR_INVALID_ARG),
    (dict(dtype=7), ppsa.PPSA_ERR_UNSUPPORTED),
    (dict(q_heads=7), ppsa.PPSA_ERR_INVALID_ARG),
    (dict(q_heads=34, kv_heads=2), ppsa.PPSA_ERR_UNSUPPORTED),
    (dict(kv_heads=0), ppsa.PPSA_ERR_INVALID_ARG),
    (dict(batch=-1), ppsa.PPSA_ERR_INVALID_ARG),
    (dict(max_seq_len=0), ppsa.PPSA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), ppsa.PPSA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), ppsa.PPSA_ERR_INVALID_ARG),
])
def test_bad_dims(kw, code):
    d = dims(**kw)
    assert full(d, ws_bytes=1 << 30) == code
    assert sparse(d, ws_bytes=1 << 30) == code


def test_null_and_misaligned_pointers():
    d = dims()
    for name in ("q", "k", "v", "lens", "out", "ws"):
        assert full(d, **{name: None}) == ppsa.PPSA_ERR_INVALID_ARG, name
    for name in ("q", "k", "v", "out", "ws"):
        assert full(d, **{name: ODD}) == ppsa.PPSA_ERR_INVALID_ARG, name
    assert sparse(d, idx=None) == ppsa.PPSA_ERR_INVALID_ARG
    assert select(d, idx=None) == ppsa.PPSA_ERR_INVALID_ARG
    assert select(d, scores=ctypes.c_void_p(0x100002)) == ppsa.PPSA_ERR_INVALID_ARG


def test_topk_range():
    d = dims()
    assert sparse(d, topk=0) == ppsa.PPSA_ERR_INVALID_ARG
    assert sparse(d, topk=1001) == ppsa.PPSA_ERR_INVALID_ARG
    assert select(d, topk=0) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_select_topk(ctypes.byref(d), FAKE, FAKE, 1001, FAKE, None, 0, None) == ppsa.PPSA_ERR_INVALID_ARG


def test_sparse_phases_validation():
    d = dims()
    wsb = ppsa.workspace_bytes(d, 16)

    def phases(ph, idx=FAKE, ws_bytes=wsb):
        return LIB.ppsa_sparse_attn_phases(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, idx, 16, ph, FAKE, FAKE,
                                           ws_bytes, None)

    for bad in (0, 4, -1):
        assert phases(bad) == ppsa.PPSA_ERR_INVALID_ARG, bad
    for ph in (1, 2, 3):
        assert phases(ph, idx=None) == ppsa.PPSA_ERR_INVALID_ARG, ph
        assert phases(ph, ws_bytes=wsb - 256) == ppsa.PPSA_ERR_WORKSPACE, ph


def test_workspace_too_small():
    d = dims()
    assert full(d, ws_bytes=ppsa.workspace_bytes(d, 0) - 1) == ppsa.PPSA_ERR_WORKSPACE
    assert sparse(d, ws_bytes=ppsa.workspace_bytes(d, 16) - 256) == ppsa.PPSA_ERR_WORKSPACE


def test_schedule_errors():
    d = dims()
    assert step(d, "FFS") == ppsa.PPSA_ERR_SCHEDULE
    assert step(d, "S") == ppsa.PPSA_ERR_SCHEDULE
    assert step(d, [0, 1, 7]) == ppsa.PPSA_ERR_SCHEDULE
    assert step(d, "FFXS", topk=0) == ppsa.PPSA_ERR_INVALID_ARG
    assert step(d, "FFXS", idx=None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_decode_step(ctypes.byref(d), 3, None, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, None, FAKE,
                                1 << 30, None) == ppsa.PPSA_ERR_INVALID_ARG


def test_empty_batch_and_empty_schedule_are_noops():
    d = dims(batch=0)
    assert full(d, q=None, k=None, v=None, lens=None, out=None, ws=None, ws_bytes=0) == ppsa.PPSA_OK
    assert LIB.ppsa_decode_step(ctypes.byref(dims()), 0, None, None, None, None, None, 0, None, None, None, None,
                                0, None) == ppsa.PPSA_OK


def test_timing_api_without_gpu_work():
    # Switching off (no pool) and reading with nothing recorded make no HIP call.
    assert LIB.ppsa_timing_enable(0) == ppsa.PPSA_OK
    assert LIB.ppsa_timing_enable(-1) == ppsa.PPSA_ERR_INVALID_ARG
    res = ppsa.timing_read()
    assert res["dropped"] == 0
    assert all(res[k] == (0, 0.0) for k in ppsa.KERNEL_KEYS)
    nk = ppsa.PPSA_KERNEL_KINDS
    assert nk == len(ppsa.KERNEL_KEYS) == 8
    counts = (ctypes.c_int32 * nk)()
    ms = (ctypes.c_double * nk)()
    assert LIB.ppsa_timing_read(counts, ms, nk - 1, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_timing_read(None, ms, nk, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_timing_read(counts, None, nk, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_timing_read(counts, ms, nk, None) == ppsa.PPSA_OK
    names = [ppsa.timing_kernel_name(i) for i in range(ppsa.PPSA_KERNEL_KINDS)]
    assert len(set(names)) == ppsa.PPSA_KERNEL_KINDS and "unknown" not in names
    assert ppsa.timing_kernel_name(ppsa.PPSA_KERNEL_KINDS) == "unknown"
    assert ppsa.timing_kernel_name(-1) == "unknown"


def append(d, layers=2, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, overflow=None):
    return LIB.ppsa_append_kv(ctypes.byref(d), layers, kn, vn, kc, vc, lens, overflow, None)


def test_append_kv_validation():
    d = dims()
    assert append(d, layers=-1) == ppsa.PPSA_ERR_INVALID_ARG
    assert append(d, layers=0) == ppsa.PPSA_OK                       # nothing to do, nothing launched
    assert append(dims(batch=0)) == ppsa.PPSA_OK
    for kw in ("kn", "vn", "kc", "vc", "lens"):
        assert append(d, **{kw: None}) == ppsa.PPSA_ERR_INVALID_ARG, kw
    for kw in ("kn", "vn", "kc", "vc"):
        assert append(d, **{kw: ODD}) == ppsa.PPSA_ERR_INVALID_ARG, kw
    assert append(d, lens=ctypes.c_void_p(0x100002)) == ppsa.PPSA_ERR_INVALID_ARG
    assert append(d, overflow=ctypes.c_void_p(0x100002)) == ppsa.PPSA_ERR_INVALID_ARG
    assert append(dims(head_dim=96)) == ppsa.PPSA_ERR_UNSUPPORTED
    assert append(dims(batch=-1)) == ppsa.PPSA_ERR_INVALID_ARG


def test_select_mode_validation():
    d = dims()
    codes = ppsa.schedule_codes("FFX")
    for mode, tau in ((-1, 0.0), (4, 0.0), (7, 0.0), (ppsa.PPSA_SELECT_COVERAGE, -0.1),
                      (ppsa.PPSA_SELECT_COVERAGE, 1.0), (ppsa.PPSA_SELECT_COVERAGE, float("nan"))):
        assert LIB.ppsa_decode_step_ex(ctypes.byref(d), 3, codes, FAKE, FAKE, FAKE, FAKE, 16, mode, tau, FAKE, FAKE,
                                       None, FAKE, 1 << 30, None) == ppsa.PPSA_ERR_INVALID_ARG, (mode, tau)
    for mode in (-1, ppsa.PPSA_SELECT_SOFTMAX, ppsa.PPSA_SELECT_COVERAGE, 7):  # need head logits: steps only
        assert LIB.ppsa_select_topk_ex(ctypes.byref(d), FAKE, FAKE, 16, mode, FAKE, None, 0, None) == \
            ppsa.PPSA_ERR_INVALID_ARG
    # A valid mode reaches the usual checks (idx misaligned for int32 here, so nothing is launched).
    assert LIB.ppsa_select_topk_ex(ctypes.byref(d), FAKE, FAKE, 16, ppsa.PPSA_SELECT_SHARED,
                                   ctypes.c_void_p(0x100002), None, 0, None) == ppsa.PPSA_ERR_INVALID_ARG
    # The optional workspace: a size without a pointer, or a pointer not 16-byte aligned.
    for ws, nbytes in ((None, 4096), (ctypes.c_void_p(0x100004), 1 << 30)):
        assert LIB.ppsa_select_topk_ex(ctypes.byref(d), FAKE, FAKE, 16, ppsa.PPSA_SELECT_PER_KV_HEAD, FAKE, ws,
                                       nbytes, None) == ppsa.PPSA_ERR_INVALID_ARG, (ws, nbytes)


def test_binding_rejects_mismatched_buffers():
    """Caller-provided buffers are written by shape on the device, so the binding checks them first."""
    import torch

    dev = torch.device("cpu")
    good = torch.empty((2, 3, 4), dtype=torch.int32)
    ppsa._check_buffer(good, (2, 3, 4), torch.int32, dev, "idx")
    for bad in (torch.empty((2, 3, 5), dtype=torch.int32), torch.empty((2, 3, 4), dtype=torch.int64),
                torch.empty((2, 4, 3), dtype=torch.int32).transpose(1, 2)):
        with pytest.raises(ValueError):
            ppsa._check_buffer(bad, (2, 3, 4), torch.int32, dev, "idx")
    assert ppsa._workspace_nbytes(torch.empty(10, dtype=torch.float32), dev) == 40


def static_step(d, schedule, topk=16, idx=FAKE, scores=None, q=FAKE):
    codes = ppsa.schedule_codes(schedule)
    return LIB.ppsa_decode_step_static(ctypes.byref(d), len(schedule), codes, q, FAKE, FAKE, FAKE, topk, FAKE, idx,
                                       scores, None)


def test_static_scratch_step_validation():
    """The no-workspace decode step checks its arguments, and its fit in the static scratch, before any
    HIP call."""
    d = dims()
    assert static_step(d, "FFS") == ppsa.PPSA_ERR_SCHEDULE
    assert static_step(d, "FFXS", topk=0) == ppsa.PPSA_ERR_INVALID_ARG
    assert static_step(d, "FFXS", idx=None) == ppsa.PPSA_ERR_INVALID_ARG
    assert static_step(d, "FFXS", q=ODD) == ppsa.PPSA_ERR_INVALID_ARG
    assert static_step(dims(batch=0), "FFXS") == ppsa.PPSA_OK
    # 8 x 8 units x 300000 rows: the score array alone (76.8 MB) is past the 16 MiB scratch; with the
    # caller's own score array the partials fit, and the call gets as far as the missing GPU.
    big = dims(batch=8, q_heads=64, kv_heads=8, max_seq_len=300000)
    assert static_step(big, "FFXS") == ppsa.PPSA_ERR_SCRATCH
    assert ppsa.status_string(ppsa.PPSA_ERR_SCRATCH) != "unknown status"


def test_probe_validation():
    """The measurement probes check their arguments before any HIP call."""
    assert LIB.ppsa_probe_read(None, 1 << 20, 1, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_probe_read(FAKE, (1 << 20) + 16, 1, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG  # not 32 KiB units
    assert LIB.ppsa_probe_read(ODD, 1 << 20, 1, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_probe_read(FAKE, 0, 1, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_probe_empty(0, 64, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_probe_empty(4, 2048, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_probe_empty(4, 64, None, None) == ppsa.PPSA_ERR_INVALID_ARG
    d = dims()
    assert LIB.ppsa_probe_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, 0, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_probe_gather(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, 1, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    assert LIB.ppsa_probe_gather(ctypes.byref(d), None, FAKE, FAKE, FAKE, 16, 1, FAKE, None) == ppsa.PPSA_ERR_INVALID_ARG
    f32 = dims(dtype=ppsa.PPSA_F32, head_dim=64)
    assert LIB.ppsa_probe_gather(ctypes.byref(f32), FAKE, FAKE, FAKE, FAKE, 16, 1, FAKE, None) == ppsa.PPSA_ERR_UNSUPPORTED


def test_split_rows_override_changes_the_plan():
    d = dims(batch=4, q_heads=32, kv_heads=8, max_seq_len=32768)
    auto = ppsa.workspace_bytes(d, 4096)
    try:
        assert LIB.ppsa_set_split_rows(-1, 0) == ppsa.PPSA_ERR_INVALID_ARG
        ppsa.set_split_rows(128, 128)  # many more splits: larger partial regions
        assert ppsa.workspace_bytes(d, 4096) > auto
    finally:
        ppsa.set_split_rows(0, 0)
    assert ppsa.workspace_bytes(d, 4096) == auto
