"""Python binding of libdsa.so: one DeepSeek-Sparse-Attention layer on MI355X.

Every function here has the name of a C entry point in ``include/dsa.h`` and
does argument marshalling only: it checks that tensors are contiguous, on the
GPU and of the expected dtype, turns them into raw pointers plus the current
HIP stream, calls the library, and raises ``DsaError`` on a non-zero status.
All computation happens in the HIP kernels behind the C ABI; there is no
fallback of any kind. If the library is not built, importing works but every
call raises.

Tensors (torch, device ``cuda``) follow the layouts of ``include/dsa.h``:
q [B,S,H,Dqk], k_cache [B,T,H,Dqk], v_cache [B,T,H,Dv], q_idx [B,S,HI,DI],
k_idx [B,T,DI], w [B,S,HI], scores [B,S,T] float32, indices [B,S,topk] int32,
gate [B,S,H] or [B,S,H,Dv].
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP, DSA_ERR_CHECK = range(6)
DSA_F32, DSA_BF16 = 0, 1
RELU_PER_HEAD, RELU_NONE, RELU_POST_SUM = 0, 1, 2
MAX_TOPK = 2048

_EXPORTS = [
    "dsa_index_scores", "dsa_topk_workspace_size", "dsa_topk", "dsa_topk_unsorted",
    "dsa_sparse_attn_prefill_workspace_size", "dsa_sparse_attn_prefill",
    "dsa_sparse_attn_decode_workspace_size", "dsa_sparse_attn_decode",
    "swa_attn_workspace_size", "swa_attn", "dsa_status_string", "dsa_last_error",
    "dsa_sparse_attn_prefill_pas_workspace_size", "dsa_sparse_attn_prefill_pas",
    "dsa_sparse_attn_decode_pas_workspace_size", "dsa_sparse_attn_decode_pas",
    "swa_attn_pas_workspace_size", "swa_attn_pas",
    "swa_attn_gqa_workspace_size", "swa_attn_gqa",
    "dsa_index_quant_fp8", "dsa_index_scores_fp8",
    "dsa_indexer_prologue_workspace_size", "dsa_indexer_prologue",
    "dsa_prefill_work_plan", "dsa_sparse_attn_decode_noalloc",
    "dsa_mla_prologue_workspace_size", "dsa_mla_prologue", "dsa_debug_build",
    "dsa_index_topk_workspace_size", "dsa_index_topk",
]
MAX_SINKS = 256


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {status}: {msg}")
        self.status = status


_lib = None

# The same library compiled with -DDSA_DEBUG (device-side checks; include/dsa.h).
DEBUG_LIB_PATH = os.path.join(_PKG, "libdsa_debug.so")


def use_library(path: str) -> str:
    """Make later calls go to the library at `path` (for example
    DEBUG_LIB_PATH); returns the path in use before."""
    global LIB_PATH, _lib
    prev = LIB_PATH
    LIB_PATH, _lib = path, None
    return prev


def lib():
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                               "python sparse_attention_11_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.dsa_index_scores.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                       i32, vp]
        L.dsa_topk_workspace_size.argtypes = [i32, i32, i32, i32]
        L.dsa_topk_workspace_size.restype = sz
        L.dsa_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, sz, vp]
        L.dsa_topk_unsorted.argtypes = [vp, vp, i32, i32, i32, i32, vp, sz, vp]
        L.dsa_sparse_attn_prefill_workspace_size.argtypes = [i32] * 8
        L.dsa_sparse_attn_prefill_workspace_size.restype = sz
        L.dsa_sparse_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                              i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
        L.dsa_sparse_attn_decode_workspace_size.argtypes = [i32] * 4
        L.dsa_sparse_attn_decode_workspace_size.restype = sz
        L.dsa_sparse_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                             i32, f32, i32, i32, vp, sz, vp]
        L.swa_attn_workspace_size.argtypes = [i32] * 7
        L.swa_attn_workspace_size.restype = sz
        L.swa_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                               i32, f32, i32, i32, vp, sz, vp]
        L.dsa_sparse_attn_prefill_pas_workspace_size.argtypes = [i32] * 9
        L.dsa_sparse_attn_prefill_pas_workspace_size.restype = sz
        L.dsa_sparse_attn_prefill_pas.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, i32,
                                                  i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                                  i32, vp, sz, vp]
        L.dsa_sparse_attn_decode_pas_workspace_size.argtypes = [i32] * 5
        L.dsa_sparse_attn_decode_pas_workspace_size.restype = sz
        L.dsa_sparse_attn_decode_pas.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, i32,
                                                 i32, i32, i32, i32, i32, f32, i32, i32, vp, sz,
                                                 vp]
        L.swa_attn_pas_workspace_size.argtypes = [i32] * 8
        L.swa_attn_pas_workspace_size.restype = sz
        L.swa_attn_pas.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                   i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
        L.dsa_index_quant_fp8.argtypes = [vp, vp, vp, ctypes.c_longlong, i32, i32, vp]
        L.dsa_index_scores_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           f32, i32, i32, vp]
        L.dsa_indexer_prologue_workspace_size.argtypes = [i32] * 3
        L.dsa_indexer_prologue_workspace_size.restype = sz
        L.dsa_indexer_prologue.argtypes = [vp] * 12 + [i32] * 9 + [f32, i32, vp, sz, vp]
        L.swa_attn_gqa_workspace_size.argtypes = [i32] * 7
        L.swa_attn_gqa_workspace_size.restype = sz
        L.swa_attn_gqa.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                   i32, i32, i32, f32, i32, i32, vp, sz, vp]
        L.dsa_prefill_work_plan.argtypes = [i32] * 7 + [vp] * 4 + [i32]
        L.dsa_mla_prologue_workspace_size.argtypes = [i32] * 3
        L.dsa_mla_prologue_workspace_size.restype = sz
        L.dsa_mla_prologue.argtypes = [vp] * 12 + [i32] * 13 + [vp, sz, vp]
        L.dsa_sparse_attn_decode_noalloc.argtypes = [vp] * 6 + [i32] * 7 + [f32, i32, i32, vp]
        for fn in ("dsa_prefill_work_plan", "dsa_sparse_attn_decode_noalloc", "dsa_mla_prologue", "dsa_index_scores", "dsa_topk", "dsa_topk_unsorted", "dsa_sparse_attn_prefill",
                   "dsa_sparse_attn_decode", "swa_attn", "dsa_sparse_attn_prefill_pas",
                   "dsa_sparse_attn_decode_pas", "swa_attn_pas", "swa_attn_gqa",
                   "dsa_index_quant_fp8", "dsa_index_scores_fp8", "dsa_indexer_prologue"):
            getattr(L, fn).restype = i32
        L.dsa_status_string.argtypes = [i32]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_index_topk_workspace_size.argtypes = [i32] * 4
        L.dsa_index_topk_workspace_size.restype = sz
        L.dsa_index_topk.argtypes = [vp] * 4 + [i32] * 6 + [f32] + [i32] * 4 + [vp, sz, vp]
        L.dsa_index_topk.restype = i32
        L.dsa_debug_build.argtypes = []
        L.dsa_debug_build.restype = i32
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn: str, st: int):
    if st != DSA_OK:
        L = lib()
        raise DsaError(fn, st, f"{L.dsa_status_string(st).decode()}: {L.dsa_last_error().decode()}")


def _workspace(nbytes: int, like):
    import torch
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


# ------------------------------------------------------------- entry points
def dsa_index_scores(q_idx, k_idx, w, scores, past_len: int, scale: float | None = None,
                     relu_mode: int = RELU_PER_HEAD, stream=None):
    B, S, HI, DI = q_idx.shape
    T = k_idx.shape[1]
    if scale is None:
        scale = DI ** -0.5
    _check("dsa_index_scores", lib().dsa_index_scores(
        _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(scores), B, S, T, past_len, HI, DI, scale,
        relu_mode, _dtype(q_idx), _stream(stream)))
    return scores


def dsa_index_topk_workspace_size(B: int, S: int, T: int, topk: int) -> int:
    return int(lib().dsa_index_topk_workspace_size(B, S, T, topk))


def dsa_index_topk(q_idx, k_idx, w, indices, past_len: int, scale: float | None = None,
                   relu_mode: int = RELU_PER_HEAD, sorted: bool = True, workspace=None,
                   stream=None):
    """dsa_index_scores + dsa_topk (or dsa_topk_unsorted) in one call; the
    scores stay in the workspace. indices [B,S,topk] int32."""
    B, S, HI, DI = q_idx.shape
    T = k_idx.shape[1]
    topk = indices.shape[-1]
    if scale is None:
        scale = DI ** -0.5
    if workspace is None:
        workspace = _workspace(dsa_index_topk_workspace_size(B, S, T, topk), q_idx)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_index_topk", lib().dsa_index_topk(
        _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(indices), B, S, T, past_len, HI, DI, scale,
        relu_mode, _dtype(q_idx), topk, 1 if sorted else 0, _ptr(workspace), nbytes,
        _stream(stream)))
    return indices


def dsa_topk_workspace_size(B: int, S: int, T: int, topk: int) -> int:
    return int(lib().dsa_topk_workspace_size(B, S, T, topk))


def dsa_prefill_work_plan(B: int, S: int, T: int, past_len: int, H: int, kv_offset: int = 0,
                          window: int = 0):
    """The MFMA prefill path's launch plan (host arithmetic only): returns
    (n_tiles, n_items, max_blocks, item_start) with item_start[o] the first
    work item of the o-th longest 128-query tile and item_start[n_tiles] =
    n_items."""
    import numpy as np
    nqt = (S + 127) // 128
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    start = np.zeros(nqt + 1, np.int32)
    _check("dsa_prefill_work_plan",
           lib().dsa_prefill_work_plan(B, S, T, past_len, H, kv_offset, window, ctypes.byref(a),
                                       ctypes.byref(b), ctypes.byref(c),
                                       start.ctypes.data_as(ctypes.c_void_p), nqt + 1))
    return a.value, b.value, c.value, start


def _topk_call(name, scores, indices, workspace, stream):
    B, S, T = scores.shape
    topk = indices.shape[-1]
    need = dsa_topk_workspace_size(B, S, T, topk)
    if workspace is None:
        workspace = _workspace(need, scores)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(name, getattr(lib(), name)(_ptr(scores), _ptr(indices), B, S, T, topk,
                                      _ptr(workspace), nbytes, _stream(stream)))
    return indices


def dsa_topk(scores, indices, workspace=None, stream=None):
    return _topk_call("dsa_topk", scores, indices, workspace, stream)


def dsa_topk_unsorted(scores, indices, workspace=None, stream=None):
    return _topk_call("dsa_topk_unsorted", scores, indices, workspace, stream)


def dsa_sparse_attn_prefill_workspace_size(B, S, T, H, qk_dim, v_dim, topk, dtype) -> int:
    return int(lib().dsa_sparse_attn_prefill_workspace_size(B, S, T, H, qk_dim, v_dim, topk, dtype))


def _gate_dim(gate, Dv):
    if gate is None:
        return 0
    return 1 if gate.dim() == 3 else Dv


def dsa_sparse_attn_prefill(q, k_cache, v_cache, indices, gate, out, past_len: int,
                            qk_nope_dim: int, qk_rope_dim: int, sm_scale: float | None = None,
                            workspace=None, stream=None):
    B, S, H, Dqk = q.shape
    T, Dv = k_cache.shape[1], v_cache.shape[3]
    topk = indices.shape[-1]
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    dt = _dtype(q)
    if workspace is None:
        workspace = _workspace(dsa_sparse_attn_prefill_workspace_size(B, S, T, H, Dqk, Dv, topk, dt), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_attn_prefill", lib().dsa_sparse_attn_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(indices), _ptr(gate), _ptr(out), B, S, T,
        past_len, H, qk_nope_dim, qk_rope_dim, Dv, topk, sm_scale, _gate_dim(gate, Dv), dt,
        _ptr(workspace), nbytes, _stream(stream)))
    return out


def dsa_sparse_attn_decode_workspace_size(B, H, v_dim, topk) -> int:
    return int(lib().dsa_sparse_attn_decode_workspace_size(B, H, v_dim, topk))


def dsa_sparse_attn_decode(q, k_cache, v_cache, indices, gate, out, qk_nope_dim: int,
                           qk_rope_dim: int, sm_scale: float | None = None, workspace=None,
                           stream=None):
    B, _, H, Dqk = q.shape
    T, Dv = k_cache.shape[1], v_cache.shape[3]
    topk = indices.shape[-1]
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    if workspace is None:
        workspace = _workspace(dsa_sparse_attn_decode_workspace_size(B, H, Dv, topk), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_attn_decode", lib().dsa_sparse_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(indices), _ptr(gate), _ptr(out), B, T, H,
        qk_nope_dim, qk_rope_dim, Dv, topk, sm_scale, _gate_dim(gate, Dv), _dtype(q),
        _ptr(workspace), nbytes, _stream(stream)))
    return out


STATIC_SCRATCH_BYTES = 32 << 20


def dsa_sparse_attn_decode_noalloc(q, k_cache, v_cache, indices, gate, out, qk_nope_dim: int,
                                   qk_rope_dim: int, sm_scale: float | None = None, stream=None):
    """dsa_sparse_attn_decode with its partial states in the library's static
    device scratch: no workspace, no allocation."""
    B, _, H, Dqk = q.shape
    T, Dv = k_cache.shape[1], v_cache.shape[3]
    topk = indices.shape[-1]
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    _check("dsa_sparse_attn_decode_noalloc", lib().dsa_sparse_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(indices), _ptr(gate), _ptr(out), B, T, H,
        qk_nope_dim, qk_rope_dim, Dv, topk, sm_scale, _gate_dim(gate, Dv), _dtype(q),
        _stream(stream)))
    return out


def swa_attn_workspace_size(B, S, H, qk_dim, v_dim, window, dtype) -> int:
    return int(lib().swa_attn_workspace_size(B, S, H, qk_dim, v_dim, window, dtype))


def swa_attn(q, k_buf, v_buf, gate, out, past_len: int, kv_offset: int, window: int,
             qk_nope_dim: int, qk_rope_dim: int, sm_scale: float | None = None, workspace=None,
             stream=None):
    B, S, H, Dqk = q.shape
    T_buf, Dv = k_buf.shape[1], v_buf.shape[3]
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    dt = _dtype(q)
    if workspace is None:
        workspace = _workspace(swa_attn_workspace_size(B, S, H, Dqk, Dv, window, dt), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("swa_attn", lib().swa_attn(
        _ptr(q), _ptr(k_buf), _ptr(v_buf), _ptr(gate), _ptr(out), B, S, T_buf, past_len,
        kv_offset, H, qk_nope_dim, qk_rope_dim, Dv, window, sm_scale, _gate_dim(gate, Dv), dt,
        _ptr(workspace), nbytes, _stream(stream)))
    return out


def _n_sink(sink_k, sink_v, H, Dqk, Dv) -> int:
    """Sink rows [n,H,Dqk] / [n,H,Dv] on the GPU, same dtype as q."""
    n = sink_k.shape[0]
    if tuple(sink_k.shape) != (n, H, Dqk) or tuple(sink_v.shape) != (n, H, Dv):
        raise ValueError(f"sink_k {tuple(sink_k.shape)} / sink_v {tuple(sink_v.shape)} do not "
                         f"match [n,{H},{Dqk}] / [n,{H},{Dv}]")
    return n


def dsa_sparse_attn_prefill_pas_workspace_size(B, S, T, H, qk_dim, v_dim, topk, n_sink,
                                               dtype) -> int:
    return int(lib().dsa_sparse_attn_prefill_pas_workspace_size(B, S, T, H, qk_dim, v_dim, topk,
                                                                n_sink, dtype))


def dsa_sparse_attn_prefill_pas(q, k_cache, v_cache, sink_k, sink_v, indices, gate, out,
                                past_len: int, qk_nope_dim: int, qk_rope_dim: int,
                                sm_scale: float | None = None, workspace=None, stream=None):
    B, S, H, Dqk = q.shape
    T, Dv = k_cache.shape[1], v_cache.shape[3]
    topk = indices.shape[-1]
    ns = _n_sink(sink_k, sink_v, H, Dqk, Dv)
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    dt = _dtype(q)
    if workspace is None:
        workspace = _workspace(
            dsa_sparse_attn_prefill_pas_workspace_size(B, S, T, H, Dqk, Dv, topk, ns, dt), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_attn_prefill_pas", lib().dsa_sparse_attn_prefill_pas(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sink_k), _ptr(sink_v), ns, _ptr(indices),
        _ptr(gate), _ptr(out), B, S, T, past_len, H, qk_nope_dim, qk_rope_dim, Dv, topk, sm_scale,
        _gate_dim(gate, Dv), dt, _ptr(workspace), nbytes, _stream(stream)))
    return out


def dsa_sparse_attn_decode_pas_workspace_size(B, H, v_dim, topk, n_sink) -> int:
    return int(lib().dsa_sparse_attn_decode_pas_workspace_size(B, H, v_dim, topk, n_sink))


def dsa_sparse_attn_decode_pas(q, k_cache, v_cache, sink_k, sink_v, indices, gate, out,
                               qk_nope_dim: int, qk_rope_dim: int, sm_scale: float | None = None,
                               workspace=None, stream=None):
    B, _, H, Dqk = q.shape
    T, Dv = k_cache.shape[1], v_cache.shape[3]
    topk = indices.shape[-1]
    ns = _n_sink(sink_k, sink_v, H, Dqk, Dv)
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    if workspace is None:
        workspace = _workspace(dsa_sparse_attn_decode_pas_workspace_size(B, H, Dv, topk, ns), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_attn_decode_pas", lib().dsa_sparse_attn_decode_pas(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sink_k), _ptr(sink_v), ns, _ptr(indices),
        _ptr(gate), _ptr(out), B, T, H, qk_nope_dim, qk_rope_dim, Dv, topk, sm_scale,
        _gate_dim(gate, Dv), _dtype(q), _ptr(workspace), nbytes, _stream(stream)))
    return out


def swa_attn_pas_workspace_size(B, S, H, qk_dim, v_dim, window, n_sink, dtype) -> int:
    return int(lib().swa_attn_pas_workspace_size(B, S, H, qk_dim, v_dim, window, n_sink, dtype))


def swa_attn_pas(q, k_buf, v_buf, sink_k, sink_v, gate, out, past_len: int, kv_offset: int,
                 window: int, qk_nope_dim: int, qk_rope_dim: int, sm_scale: float | None = None,
                 workspace=None, stream=None):
    B, S, H, Dqk = q.shape
    T_buf, Dv = k_buf.shape[1], v_buf.shape[3]
    ns = _n_sink(sink_k, sink_v, H, Dqk, Dv)
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    dt = _dtype(q)
    if workspace is None:
        workspace = _workspace(swa_attn_pas_workspace_size(B, S, H, Dqk, Dv, window, ns, dt), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("swa_attn_pas", lib().swa_attn_pas(
        _ptr(q), _ptr(k_buf), _ptr(v_buf), _ptr(sink_k), _ptr(sink_v), ns, _ptr(gate), _ptr(out),
        B, S, T_buf, past_len, kv_offset, H, qk_nope_dim, qk_rope_dim, Dv, window, sm_scale,
        _gate_dim(gate, Dv), dt, _ptr(workspace), nbytes, _stream(stream)))
    return out


def swa_attn_gqa_workspace_size(B, S, H, qk_dim, v_dim, window, dtype) -> int:
    return int(lib().swa_attn_gqa_workspace_size(B, S, H, qk_dim, v_dim, window, dtype))


def swa_attn_gqa(q, k_buf, v_buf, gate, out, past_len: int, kv_offset: int, window: int,
                 qk_nope_dim: int, qk_rope_dim: int, sm_scale: float | None = None,
                 workspace=None, stream=None):
    """swa_attn with grouped KV heads: k_buf [B,T_buf,H_kv,Dqk], v_buf [B,T_buf,H_kv,Dv]."""
    B, S, H, Dqk = q.shape
    T_buf, H_kv, Dv = k_buf.shape[1], k_buf.shape[2], v_buf.shape[3]
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    dt = _dtype(q)
    if workspace is None:
        workspace = _workspace(swa_attn_gqa_workspace_size(B, S, H, Dqk, Dv, window, dt), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("swa_attn_gqa", lib().swa_attn_gqa(
        _ptr(q), _ptr(k_buf), _ptr(v_buf), _ptr(gate), _ptr(out), B, S, T_buf, past_len,
        kv_offset, H, H_kv, qk_nope_dim, qk_rope_dim, Dv, window, sm_scale, _gate_dim(gate, Dv),
        dt, _ptr(workspace), nbytes, _stream(stream)))
    return out


def dsa_index_quant_fp8(x, codes, scales, stream=None):
    """x [..., D] bf16 -> codes [..., D] uint8 (FP8 E4M3 of the Hadamard-rotated rows),
    scales [...] float32 (one power of two per row)."""
    D = x.shape[-1]
    rows = x.numel() // D
    if tuple(codes.shape) != tuple(x.shape) or tuple(scales.shape) != tuple(x.shape[:-1]):
        raise ValueError("codes must match x and scales x.shape[:-1]")
    _check("dsa_index_quant_fp8", lib().dsa_index_quant_fp8(
        _ptr(x), _ptr(codes), _ptr(scales), rows, D, _dtype(x), _stream(stream)))
    return codes, scales


def dsa_index_scores_fp8(q_codes, q_scales, k_codes, k_scales, w, scores, past_len: int,
                         scale: float | None = None, relu_mode: int = RELU_PER_HEAD,
                         stream=None):
    """q_codes [B,S,HI,D] / q_scales [B,S,HI], k_codes [B,T,D] / k_scales [B,T] (from
    dsa_index_quant_fp8), w [B,S,HI] bf16 -> scores [B,S,T] float32."""
    B, S, HI, D = q_codes.shape
    T = k_codes.shape[1]
    if scale is None:
        scale = D ** -0.5
    _check("dsa_index_scores_fp8", lib().dsa_index_scores_fp8(
        _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(w), _ptr(scores),
        B, S, T, past_len, HI, D, scale, relu_mode, _dtype(w), _stream(stream)))
    return scores


def dsa_indexer_prologue_workspace_size(B, S, idx_dim) -> int:
    return int(lib().dsa_indexer_prologue_workspace_size(B, S, idx_dim))


def dsa_indexer_prologue(q_lora, hidden, wq_b, wk, k_norm_weight, k_norm_bias, weights_proj,
                         rope_cos, rope_sin, q_idx, k_idx_cache, w, past_len: int,
                         ln_eps: float = 1e-6, workspace=None, stream=None):
    """Indexer projections: q_lora [B,S,Q], hidden [B,S,Hd] -> q_idx [B,S,HI,D] (RoPE'd),
    k_idx_cache rows past_len.. (LayerNorm + RoPE), w [B,S,HI]; weights [out, in];
    rope_cos / rope_sin fp32 [T, rope_dim / 2] (None for no RoPE)."""
    B, S, Q = q_lora.shape
    Hd = hidden.shape[2]
    HI, D = q_idx.shape[2], q_idx.shape[3]
    T = k_idx_cache.shape[1]
    R = 0 if rope_cos is None else 2 * rope_cos.shape[1]
    if workspace is None:
        workspace = _workspace(dsa_indexer_prologue_workspace_size(B, S, D), q_lora)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_indexer_prologue", lib().dsa_indexer_prologue(
        _ptr(q_lora), _ptr(hidden), _ptr(wq_b), _ptr(wk), _ptr(k_norm_weight), _ptr(k_norm_bias),
        _ptr(weights_proj), _ptr(rope_cos), _ptr(rope_sin), _ptr(q_idx), _ptr(k_idx_cache),
        _ptr(w), B, S, T, past_len, Q, Hd, HI, D, R, ln_eps, _dtype(q_lora), _ptr(workspace),
        nbytes, _stream(stream)))
    return q_idx, k_idx_cache, w


def dsa_status_string(status: int) -> str:
    return lib().dsa_status_string(status).decode()


def dsa_last_error() -> str:
    return lib().dsa_last_error().decode()


def dsa_debug_build() -> bool:
    return bool(lib().dsa_debug_build())


def dsa_mla_prologue_workspace_size(B: int, S: int, kv_lora_rank: int) -> int:
    return int(lib().dsa_mla_prologue_workspace_size(B, S, kv_lora_rank))


def dsa_mla_prologue(q_resid, q_compressed, hidden, wq_gate, wkv_a, wkv_b, rope_cos, rope_sin,
                     q, gate, k_cache, v_cache, past_len: int, workspace=None, stream=None):
    """The main attention's projections (q_gate_proj split, kv_a_proj_with_mqa,
    expand_kv, interleaved RoPE); sizes are read from the tensors:
    q [B,S,H,Dqk], gate [B,S,H,Dv], rope tables [T, R/2] (None: R = 0)."""
    B, S, Qr = q_resid.shape
    Qc, Hd = q_compressed.shape[2], hidden.shape[2]
    H, Dqk = q.shape[2], q.shape[3]
    Dv = gate.shape[3]
    R = 0 if rope_cos is None else 2 * rope_cos.shape[1]
    L = wkv_a.shape[0] - R
    T = k_cache.shape[1]
    if workspace is None:
        workspace = _workspace(dsa_mla_prologue_workspace_size(B, S, L), q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_mla_prologue", lib().dsa_mla_prologue(
        _ptr(q_resid), _ptr(q_compressed), _ptr(hidden), _ptr(wq_gate), _ptr(wkv_a), _ptr(wkv_b),
        _ptr(rope_cos), _ptr(rope_sin), _ptr(q), _ptr(gate), _ptr(k_cache), _ptr(v_cache), B, S, T,
        past_len, Qr, Qc, Hd, L, H, Dqk - R, R, Dv, _dtype(q), _ptr(workspace), nbytes,
        _stream(stream)))
    return q, gate, k_cache, v_cache
