"""Seeded synthetic inputs, produced identically on the host and on the GPU.

This package is shared by the tests (which feed the oracle from the host
twin) and by the benchmark (which fills HBM from the device twin). It holds
none of the attention method's arithmetic; ``gen_host.c`` documents the
generator's definition and ``gen_device.hip`` implements the same definition
for the GPU. A GPU test checks that the two agree bit for bit.

Host arrays are numpy ``float32`` or ``uint16`` (bf16 bit patterns). Device
fills write into caller-allocated torch tensors on the current HIP stream.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SRC = os.path.join(_HERE, "gen_host.c")
_HOST_LIB = os.path.join(_HERE, "libdsagen_host.so")
_DEV_SRC = os.path.join(_HERE, "gen_device.hip")
_DEV_LIB = os.path.join(_HERE, "libdsagen_device.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# tensor ids of the stream keys
TID_Q, TID_K, TID_V, TID_QIDX, TID_KIDX, TID_W, TID_GATE, TID_INDICES, TID_SCORES = range(1, 10)
TID_SINK_K, TID_SINK_V = 10, 11  # attention-sink rows [n_sink, H, D]
SWA_TID_STRIDE = 16  # SWA layer j (1, 2) uses id + 16*j


def build_host(force: bool = True) -> str:
    if force or not os.path.exists(_HOST_LIB) or os.path.getmtime(_HOST_LIB) < os.path.getmtime(_HOST_SRC):
        tmp = _HOST_LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-ffp-contract=off", "-o", tmp, _HOST_SRC, "-lm"])
        os.replace(tmp, _HOST_LIB)
    return _HOST_LIB


def build_device(force: bool = True) -> str:
    if force or not os.path.exists(_DEV_LIB) or os.path.getmtime(_DEV_LIB) < os.path.getmtime(_DEV_SRC):
        tmp = _DEV_LIB + ".tmp"
        subprocess.check_call(["/opt/rocm/bin/hipcc", *HIP_FLAGS, "-o", tmp, _DEV_SRC])
        os.replace(tmp, _DEV_LIB)
    return _DEV_LIB


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(_HOST_LIB):
            build_host()
        lib = ctypes.CDLL(_HOST_LIB)
        vp, i32, i64, u64, f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_float)
        lib.dsagen_normal_host.argtypes = [vp, i32, i64, u64, i32, f32, i64]
        lib.dsagen_normal_host.restype = None
        lib.dsagen_indices_host.argtypes = [vp, i64, i64, i32, i32, i32, u64, i32]
        lib.dsagen_indices_host.restype = None
        lib.dsagen_scores_host.argtypes = [vp, i64, i64, i32, i32, i32, u64, i32, i32, f32]
        lib.dsagen_scores_host.restype = None
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_LIB):
            raise RuntimeError(f"{_DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_DEV_LIB)
        vp, i32, i64, u64, f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_float)
        lib.dsagen_normal_device.argtypes = [vp, i32, i64, u64, i32, f32, i64, vp]
        lib.dsagen_normal_device.restype = i32
        lib.dsagen_indices_device.argtypes = [vp, i64, i64, i32, i32, i32, u64, i32, vp]
        lib.dsagen_indices_device.restype = i32
        lib.dsagen_scores_device.argtypes = [vp, i64, i64, i32, i32, i32, u64, i32, i32, f32, vp]
        lib.dsagen_scores_device.restype = i32
        _dev = lib
    return _dev


def cscale(scale: float) -> float:
    """fp32 multiplier that turns the Irwin-Hall integer into N(0, scale^2)."""
    return float(np.float32(scale / math.sqrt(65536.0 * 65536.0 - 1.0)))


# ---------------------------------------------------------------- host twin
def normal_host(shape, dtype: str, seed: int, tensor_id: int, scale: float = 1.0,
                start: int = 0) -> np.ndarray:
    """Elements start .. start+prod(shape)-1 of a stream; dtype 'f32' or 'bf16' (uint16 bits)."""
    n = int(np.prod(shape)) if len(shape) else 1
    arr = np.empty(shape, np.float32 if dtype == "f32" else np.uint16)
    _host_lib().dsagen_normal_host(arr.ctypes.data_as(ctypes.c_void_p), 0 if dtype == "f32" else 1,
                                   n, seed, tensor_id, cscale(scale), start)
    return arr


def indices_host(row0: int, nrows: int, S: int, past_len: int, k: int, seed: int,
                 tensor_id: int = TID_INDICES) -> np.ndarray:
    out = np.empty((nrows, k), np.int32)
    _host_lib().dsagen_indices_host(out.ctypes.data_as(ctypes.c_void_p), row0, nrows, S, past_len,
                                    k, seed, tensor_id)
    return out


def scores_host(row0: int, nrows: int, S: int, T: int, past_len: int, seed: int, mode: int = 0,
                tensor_id: int = TID_SCORES, scale: float = 1.0) -> np.ndarray:
    out = np.empty((nrows, T), np.float32)
    _host_lib().dsagen_scores_host(out.ctypes.data_as(ctypes.c_void_p), row0, nrows, S, T, past_len,
                                   seed, tensor_id, mode, cscale(scale))
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


# -------------------------------------------------------------- device twin
def _stream_ptr(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def normal_device(t, seed: int, tensor_id: int, scale: float = 1.0, start: int = 0):
    """Fill torch tensor t (float32 or bfloat16, on the GPU, contiguous) in place."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    if t.dtype == torch.float32:
        dt = 0
    elif t.dtype == torch.bfloat16:
        dt = 1
    else:
        raise TypeError(t.dtype)
    _check(_dev_lib().dsagen_normal_device(ctypes.c_void_p(t.data_ptr()), dt, t.numel(), seed,
                                           tensor_id, cscale(scale), start, _stream_ptr(torch)),
           "dsagen_normal_device")
    return t


def indices_device(t, row0: int, S: int, past_len: int, seed: int,
                   tensor_id: int = TID_INDICES):
    """t: int32 [nrows, k] on the GPU."""
    import torch
    assert t.is_cuda and t.dtype == torch.int32 and t.is_contiguous()
    k = t.shape[-1]
    nrows = t.numel() // k
    _check(_dev_lib().dsagen_indices_device(ctypes.c_void_p(t.data_ptr()), row0, nrows, S,
                                            past_len, k, seed, tensor_id, _stream_ptr(torch)),
           "dsagen_indices_device")
    return t


def scores_device(t, row0: int, S: int, past_len: int, seed: int, mode: int = 0,
                  tensor_id: int = TID_SCORES, scale: float = 1.0):
    """t: float32 [nrows, T] on the GPU."""
    import torch
    assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()
    T = t.shape[-1]
    nrows = t.numel() // T
    _check(_dev_lib().dsagen_scores_device(ctypes.c_void_p(t.data_ptr()), row0, nrows, S, T,
                                           past_len, seed, tensor_id, mode, cscale(scale),
                                           _stream_ptr(torch)),
           "dsagen_scores_device")
    return t
