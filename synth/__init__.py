"""Seeded synthetic inputs for PPSA decode steps (shared by oracle and GPU legs).

Holds no attention or selection arithmetic. bf16 tensors are returned as
numpy uint16 arrays of raw bf16 bit patterns; f32 tensors as float32 arrays.
The C core (synth.c) is built by build() with gcc and OpenMP.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .workloads import (FULL, FULL_SELECT, SPARSE, WORKLOADS, BENCH_WORKLOAD, Workload, kv_cache_bytes,
                        layer_kv_bytes, schedule_for, step_kv_bytes)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libppsa_synth.so")

PAD_ZERO, PAD_NAN, PAD_RANDOM = 0, 1, 2

_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        raise RuntimeError(f"{_LIB} is missing: run __graft_entry__.build() (or synth.build()) first")
    lib = ctypes.CDLL(_LIB)
    u64, i32, i64, f32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.synth_abi_version.restype = i32
    lib.synth_seq_lens.argtypes = [u64, i32, i32, i32, vp]
    lib.synth_unit_vectors.argtypes = [u64, i32, i32, vp]
    lib.synth_heavy_positions.argtypes = [u64, i32, i32, vp, i32, vp, vp, i32]
    lib.synth_heavy_positions.restype = i32
    lib.synth_fill_q.argtypes = [u64, i32, i32, i32, i32, i32, vp, f32, i32, vp]
    lib.synth_fill_kv.argtypes = [u64, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, f32, i32, i32, vp, vp]
    lib.synth_round_bf16.argtypes = [vp, i64, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def round_bf16(x) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


class Generator:
    """Per-layer inputs of one workload; every call regenerates from the seed."""

    def __init__(self, wl: Workload, seed: int | None = None, seq_lens=None, pad_mode: int = PAD_ZERO):
        self.wl = wl
        self.seed = int(wl.seed if seed is None else seed)
        self.pad_mode = pad_mode
        lib = _load()
        if seq_lens is None:
            lens = np.empty(wl.batch, dtype=np.int32)
            lo = wl.min_len if wl.ragged else wl.max_len
            lib.synth_seq_lens(self.seed, wl.batch, lo, wl.max_len, _ptr(lens))
        else:
            lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
            assert lens.shape == (wl.batch,)
        self.seq_lens = lens
        self.u = np.empty((wl.kv_heads, wl.head_dim), dtype=np.float32)
        lib.synth_unit_vectors(self.seed, wl.kv_heads, wl.head_dim, _ptr(self.u))
        self.heavy_stride = wl.sinks + max(wl.heavy_random, 0)
        self.heavy = np.full((wl.batch, wl.kv_heads, self.heavy_stride), -1, dtype=np.int32)
        self.heavy_count = np.zeros((wl.batch, wl.kv_heads), dtype=np.int32)
        rc = lib.synth_heavy_positions(self.seed, wl.batch, wl.kv_heads, _ptr(self.lens_arr), wl.heavy_random,
                                       _ptr(self.heavy), _ptr(self.heavy_count), self.heavy_stride)
        if rc != 0:
            raise RuntimeError(f"synth_heavy_positions failed: {rc}")

    @property
    def lens_arr(self) -> np.ndarray:
        return self.seq_lens

    @property
    def storage_dtype(self):
        return np.float32 if self.wl.dtype == "f32" else np.uint16

    def q(self, layer: int) -> np.ndarray:
        wl = self.wl
        out = np.empty((wl.batch, wl.q_heads, wl.head_dim), dtype=self.storage_dtype)
        _load().synth_fill_q(self.seed, layer, wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, _ptr(self.u),
                             wl.q_bias, int(wl.dtype == "bf16"), _ptr(out))
        return out

    def kv(self, layer: int, out_k: np.ndarray | None = None, out_v: np.ndarray | None = None):
        wl = self.wl
        shape = (wl.batch, wl.kv_heads, wl.max_len, wl.head_dim)
        k = np.empty(shape, dtype=self.storage_dtype) if out_k is None else out_k
        v = np.empty(shape, dtype=self.storage_dtype) if out_v is None else out_v
        assert k.shape == shape and v.shape == shape and k.dtype == self.storage_dtype
        _load().synth_fill_kv(self.seed, layer, wl.batch, wl.kv_heads, wl.max_len, wl.head_dim,
                              _ptr(self.seq_lens), _ptr(self.heavy), _ptr(self.heavy_count), self.heavy_stride,
                              _ptr(self.u), wl.key_bias, int(wl.dtype == "bf16"), self.pad_mode, _ptr(k), _ptr(v))
        return k, v

    def heavy_set(self, b: int, h: int) -> np.ndarray:
        return self.heavy[b, h, : self.heavy_count[b, h]].copy()


__all__ = ["Generator", "Workload", "WORKLOADS", "BENCH_WORKLOAD", "FULL", "FULL_SELECT", "SPARSE",
           "schedule_for", "kv_cache_bytes", "layer_kv_bytes", "step_kv_bytes", "round_bf16", "build",
           "PAD_ZERO", "PAD_NAN", "PAD_RANDOM"]
