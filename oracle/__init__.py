"""fp64 CPU oracle for the DSA layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP product path never does, and
shares no code with it. The arithmetic lives in ``dsa_oracle.c`` (plain C,
double precision, OpenMP over independent outputs); this module only builds
that file with gcc and marshals numpy arrays into it.

Inputs are numpy arrays in their storage type: ``float32`` for fp32 data or
``uint16`` holding bf16 bit patterns. Outputs are float64 (scores, attention)
or int32 (top-k indices).

Parity status of each function (what pins it, in ``tests/test_oracle_pins.py``):
  index_scores  pinned: einsum/matmul closed forms, |u| and identity
                constructions for the per-head ReLU, causal -inf triangle.
  topk          pinned: brute-force subset enumeration, numpy lexsort,
                constant rows, signed-zero and -inf handling.
  sparse_attn   pinned: full selection equals torch's dense causal SDPA
                (float64), top-1 closed form, set semantics, convexity, gate
                limits.
  swa_attn      pinned: window >= context equals dense causal SDPA, window 1
                closed form, buffer-offset equivalence.
  swa_attn_gqa  pinned: torch SDPA with grouped KV heads (enable_gqa) under the
                band mask; equals swa_attn on explicitly repeated KV heads.
  index_quant_fp8
                pinned: closed forms (a unit vector rotates to all ones),
                torch's float8_e4m3fn conversion of the same scaled values,
                scipy's Hadamard matrix within FP8 rounding, the scale rule;
                against E4M3 of the exact fp64 rotation: equal on Gaussian
                rows, elsewhere different only at rounding midpoints within
                the fp32 rotation's error bound.
  index_scores_fp8
                pinned: index_scores on the dequantised rows with scale / D;
                Hadamard invariance of index_scores (H q . H k = D q . k).
  indexer_prologue
                pinned: torch's linear and layer_norm, RoPE closed forms
                (position 0 is the identity, pair norms are kept, rotating by
                a and then by -a restores the input, the angle-sum identity),
                the direction by a quarter turn and the textbook
                x cos + rotate_half(x) sin form.
  mla_prologue  pinned: torch's linear compositions (q_gate_proj on the
                concatenation, kv_a_proj, kv_b_proj of the latent) without
                RoPE, the interleaved RoPE as complex multiplication (a
                quarter turn maps (x_2j, x_2j+1) to (-x_2j+1, x_2j)), equal to
                the half-split rotation on de-interleaved dims, relative-
                position invariance of q.k, the rope key shared by all heads.
Parity unpinned by the pages (fixed by convention, tested in every mode):
ReLU placement (per head by default), the two scale constants, and the
inclusive window boundary.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "libdsa_oracle.so")

F32 = 0
BF16 = 1
RELU_PER_HEAD = 0
RELU_NONE = 1
RELU_POST_SUM = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile dsa_oracle.c into libdsa_oracle.so with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_mla_prologue.argtypes = [vp] * 8 + [i32] * 12 + [vp] * 4
        lib.oracle_mla_prologue.restype = None
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_index_scores.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            dbl, i32, vp]
        lib.oracle_index_scores.restype = None
        lib.oracle_topk.argtypes = [vp, i64, i64, i32, vp]
        lib.oracle_topk.restype = None
        lib.oracle_sparse_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           i32, i32, i32, dbl, i32, vp]
        lib.oracle_sparse_attn.restype = None
        lib.oracle_swa_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                        i32, i32, i32, dbl, i32, vp]
        lib.oracle_swa_attn.restype = None
        lib.oracle_sparse_attn_pas.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                               i32, i32, i32, i32, i32, i32, dbl, i32, vp]
        lib.oracle_sparse_attn_pas.restype = None
        lib.oracle_swa_attn_pas.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                            i32, i32, i32, i32, i32, i32, dbl, i32, vp]
        lib.oracle_swa_attn_pas.restype = None
        lib.oracle_swa_attn_gqa.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            i32, i32, i32, i32, dbl, i32, vp]
        lib.oracle_swa_attn_gqa.restype = None
        lib.oracle_e4m3_codes.argtypes = [vp, i64, vp]
        lib.oracle_e4m3_codes.restype = None
        lib.oracle_indexer_prologue.argtypes = [vp] * 9 + [i32] * 9 + [dbl, vp, vp, vp]
        lib.oracle_indexer_prologue.restype = None
        lib.oracle_index_quant_fp8.argtypes = [vp, i64, i32, vp, vp]
        lib.oracle_index_quant_fp8.restype = None
        lib.oracle_index_scores_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                i32, i32, dbl, i32, vp]
        lib.oracle_index_scores_fp8.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i32
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def _dtype_of(*arrs) -> int:
    kinds = {a.dtype for a in arrs if a is not None}
    if kinds == {np.dtype(np.float32)}:
        return F32
    if kinds == {np.dtype(np.uint16)}:
        return BF16
    raise TypeError(f"oracle inputs must all be float32 or all uint16 (bf16 bits), got {kinds}")


def _c(a):
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def index_scores(q_idx, k_idx, w, past_len: int, scale: float | None = None,
                 relu_mode: int = RELU_PER_HEAD) -> np.ndarray:
    """q_idx [B,S,HI,DI], k_idx [B,T,DI], w [B,S,HI] -> scores [B,S,T] float64."""
    q_idx, k_idx, w = _c(q_idx), _c(k_idx), _c(w)
    B, S, HI, DI = q_idx.shape
    T = k_idx.shape[1]
    assert k_idx.shape == (B, T, DI) and w.shape == (B, S, HI)
    if scale is None:
        scale = DI ** -0.5
    out = np.empty((B, S, T), np.float64)
    _load().oracle_index_scores(_ptr(q_idx), _ptr(k_idx), _ptr(w), _dtype_of(q_idx, k_idx, w),
                                B, S, T, past_len, HI, DI, float(scale), relu_mode, _ptr(out))
    return out


def topk(scores, k: int) -> np.ndarray:
    """scores [..., T] float32 -> indices [..., k] int32 (score desc, t asc; -1 pads)."""
    scores = _c(np.asarray(scores, dtype=np.float32))
    lead, T = scores.shape[:-1], scores.shape[-1]
    R = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (k,), np.int32)
    _load().oracle_topk(_ptr(scores), R, T, k, _ptr(out))
    return out


def _gate_dim(gate, Dv, gate_dim):
    if gate is None:
        return 0
    if gate_dim is None:
        return 1 if gate.ndim == 3 else Dv
    return gate_dim


def _sinks(sink_k, sink_v, H, Dqk, Dv):
    """Sink rows [n_sink,H,Dqk] / [n_sink,H,Dv] (or None for none) -> (sk, sv, n)."""
    if sink_k is None:
        assert sink_v is None
        return None, None, 0
    sink_k, sink_v = _c(sink_k), _c(sink_v)
    n = sink_k.shape[0]
    assert sink_k.shape == (n, H, Dqk) and sink_v.shape == (n, H, Dv)
    return sink_k, sink_v, n


def sparse_attn(q, k_cache, v_cache, indices, gate, past_len: int, qk_nope_dim: int,
                qk_rope_dim: int, sm_scale: float | None = None,
                gate_dim: int | None = None, sink_k=None, sink_v=None) -> np.ndarray:
    """q [B,S,H,Dqk], caches [B,T,H,D], indices [B,S,k] int32, gate [B,S,H] (one logit
    per head) or [B,S,H,Dv] (one per element) or None, optional attention sinks
    sink_k [n,H,Dqk] / sink_v [n,H,Dv] -> out [B,S,H,Dv] float64."""
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    indices = _c(np.asarray(indices, dtype=np.int32))
    B, S, H, Dqk = q.shape
    assert Dqk == qk_nope_dim + qk_rope_dim
    T = k_cache.shape[1]
    Dv = v_cache.shape[3]
    topk_ = indices.shape[2]
    gate_dim = _gate_dim(gate, Dv, gate_dim)
    if gate is not None:
        gate = _c(gate)
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    out = np.empty((B, S, H, Dv), np.float64)
    sk, sv, ns = _sinks(sink_k, sink_v, H, Dqk, Dv)
    _load().oracle_sparse_attn_pas(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sk), _ptr(sv), ns,
                                   _ptr(indices), _ptr(gate),
                                   _dtype_of(q, k_cache, v_cache, gate, sk, sv), B, S, T,
                                   past_len, H, Dqk, Dv, topk_, float(sm_scale), gate_dim,
                                   _ptr(out))
    return out


def swa_attn(q, k_buf, v_buf, gate, past_len: int, kv_offset: int, window: int,
             qk_nope_dim: int, qk_rope_dim: int, sm_scale: float | None = None,
             gate_dim: int | None = None, sink_k=None, sink_v=None) -> np.ndarray:
    """q [B,S,H,Dqk], buffers [B,T_buf,H,D] (row j = position kv_offset + j), optional
    attention sinks as in sparse_attn -> out [B,S,H,Dv] float64."""
    q, k_buf, v_buf = _c(q), _c(k_buf), _c(v_buf)
    B, S, H, Dqk = q.shape
    assert Dqk == qk_nope_dim + qk_rope_dim
    T_buf = k_buf.shape[1]
    Dv = v_buf.shape[3]
    gate_dim = _gate_dim(gate, Dv, gate_dim)
    if gate is not None:
        gate = _c(gate)
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    out = np.empty((B, S, H, Dv), np.float64)
    sk, sv, ns = _sinks(sink_k, sink_v, H, Dqk, Dv)
    _load().oracle_swa_attn_pas(_ptr(q), _ptr(k_buf), _ptr(v_buf), _ptr(sk), _ptr(sv), ns,
                                _ptr(gate), _dtype_of(q, k_buf, v_buf, gate, sk, sv), B, S,
                                T_buf, past_len, kv_offset, H, Dqk, Dv, window, float(sm_scale),
                                gate_dim, _ptr(out))
    return out


def swa_attn_gqa(q, k_buf, v_buf, gate, past_len: int, kv_offset: int, window: int,
                 qk_nope_dim: int, qk_rope_dim: int, sm_scale: float | None = None,
                 gate_dim: int | None = None) -> np.ndarray:
    """swa_attn with grouped KV heads: q [B,S,H,Dqk], buffers [B,T_buf,H_kv,D] with H_kv
    dividing H; query head h reads KV head h // (H // H_kv) -> out [B,S,H,Dv] float64."""
    q, k_buf, v_buf = _c(q), _c(k_buf), _c(v_buf)
    B, S, H, Dqk = q.shape
    assert Dqk == qk_nope_dim + qk_rope_dim
    T_buf, H_kv = k_buf.shape[1], k_buf.shape[2]
    assert H % H_kv == 0 and v_buf.shape[2] == H_kv
    Dv = v_buf.shape[3]
    gate_dim = _gate_dim(gate, Dv, gate_dim)
    if gate is not None:
        gate = _c(gate)
    if sm_scale is None:
        sm_scale = Dqk ** -0.5
    out = np.empty((B, S, H, Dv), np.float64)
    _load().oracle_swa_attn_gqa(_ptr(q), _ptr(k_buf), _ptr(v_buf), _ptr(gate),
                                _dtype_of(q, k_buf, v_buf, gate), B, S, T_buf, past_len,
                                kv_offset, H, H_kv, Dqk, Dv, window, float(sm_scale), gate_dim,
                                _ptr(out))
    return out


def e4m3_codes(v) -> np.ndarray:
    """float32 values with |v| <= 448 -> FP8 E4M3 codes (round to nearest, ties to even)."""
    v = _c(np.asarray(v, np.float32))
    assert np.all(np.abs(v) <= 448)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_codes(_ptr(v), v.size, _ptr(out))
    return out


def index_quant_fp8(x):
    """x [..., D] uint16 bf16 bits (D a power of two) -> (codes [..., D] uint8 FP8 E4M3,
    scales [...] float32): Hadamard-rotated rows, value = code * scale."""
    x = _c(x)
    assert x.dtype == np.uint16
    D = x.shape[-1]
    rows = int(np.prod(x.shape[:-1]))
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1], np.float32)
    _load().oracle_index_quant_fp8(_ptr(x), rows, D, _ptr(codes), _ptr(scales))
    return codes, scales


def index_scores_fp8(q_codes, q_scales, k_codes, k_scales, w, past_len: int,
                     scale: float | None = None, relu_mode: int = RELU_PER_HEAD) -> np.ndarray:
    """q_codes [B,S,HI,DI] / q_scales [B,S,HI], k_codes [B,T,DI] / k_scales [B,T] (from
    index_quant_fp8), w [B,S,HI] -> scores [B,S,T] float64."""
    q_codes, k_codes, w = _c(q_codes), _c(k_codes), _c(w)
    q_scales = _c(np.asarray(q_scales, np.float32))
    k_scales = _c(np.asarray(k_scales, np.float32))
    B, S, HI, DI = q_codes.shape
    T = k_codes.shape[1]
    assert k_codes.shape == (B, T, DI) and w.shape == (B, S, HI)
    assert q_scales.shape == (B, S, HI) and k_scales.shape == (B, T)
    if scale is None:
        scale = DI ** -0.5
    out = np.empty((B, S, T), np.float64)
    _load().oracle_index_scores_fp8(_ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales),
                                    _ptr(w), _dtype_of(w), B, S, T, past_len, HI, DI,
                                    float(scale), relu_mode, _ptr(out))
    return out


def indexer_prologue(q_lora, hidden, wq_b, wk, k_norm_w, k_norm_b, weights_proj, rope_cos,
                     rope_sin, past_len: int, n_idx_heads: int, eps: float = 1e-6):
    """q_lora [B,S,Q], hidden [B,S,Hd], weights [out, in], k_norm [D], rope tables fp32
    [T, R/2] or None -> (q_idx [B,S,HI,D], k [B,S,D], w [B,S,HI]) float64."""
    q_lora, hidden, wq_b, wk = _c(q_lora), _c(hidden), _c(wq_b), _c(wk)
    k_norm_w, k_norm_b, weights_proj = _c(k_norm_w), _c(k_norm_b), _c(weights_proj)
    B, S, Q = q_lora.shape
    Hd = hidden.shape[2]
    HI = n_idx_heads
    D = wk.shape[0]
    assert wq_b.shape == (HI * D, Q) and wk.shape == (D, Hd) and weights_proj.shape == (HI, Hd)
    R = 0
    if rope_cos is not None:
        rope_cos = _c(np.asarray(rope_cos, np.float32))
        rope_sin = _c(np.asarray(rope_sin, np.float32))
        R = 2 * rope_cos.shape[1]
    oq = np.empty((B, S, HI, D), np.float64)
    ok = np.empty((B, S, D), np.float64)
    ow = np.empty((B, S, HI), np.float64)
    _load().oracle_indexer_prologue(
        _ptr(q_lora), _ptr(hidden), _ptr(wq_b), _ptr(wk), _ptr(k_norm_w), _ptr(k_norm_b),
        _ptr(weights_proj), _ptr(rope_cos), _ptr(rope_sin),
        _dtype_of(q_lora, hidden, wq_b, wk, k_norm_w, k_norm_b, weights_proj), B, S, past_len,
        Q, Hd, HI, D, R, float(eps), _ptr(oq), _ptr(ok), _ptr(ow))
    return oq, ok, ow


def mla_prologue(q_resid, q_comp, hidden, wq_gate, wkv_a, wkv_b, rope_cos, rope_sin,
                 past_len: int, H: int, nope: int, rope: int, v_dim: int):
    """The main attention's projections (q_gate_proj split, kv_a_proj_with_mqa,
    expand_kv, interleaved RoPE). q_resid [B,S,Qr], q_comp [B,S,Qc], hidden
    [B,S,Hd], wq_gate [H*(nope+rope+v), Qr+Qc], wkv_a [L+rope, Hd], wkv_b
    [H*(nope+v), L], rope tables [T, rope/2] fp32 or None (rope 0) ->
    (q [B,S,H,nope+rope], gate [B,S,H,v], k_rows [B,S,H,nope+rope],
    v_rows [B,S,H,v]) float64."""
    q_resid, q_comp, hidden = _c(q_resid), _c(q_comp), _c(hidden)
    wq_gate, wkv_a, wkv_b = _c(wq_gate), _c(wkv_a), _c(wkv_b)
    B, S, Qr = q_resid.shape
    Qc, Hd = q_comp.shape[2], hidden.shape[2]
    Dqk = nope + rope
    L = wkv_a.shape[0] - rope
    assert wq_gate.shape == (H * (Dqk + v_dim), Qr + Qc)
    assert wkv_a.shape == (L + rope, Hd) and wkv_b.shape == (H * (nope + v_dim), L)
    if rope > 0:
        rope_cos = _c(np.asarray(rope_cos, np.float32))
        rope_sin = _c(np.asarray(rope_sin, np.float32))
        assert rope_cos.shape[1] == rope // 2 and rope_cos.shape[0] >= past_len + S
    else:
        rope_cos = rope_sin = None
    outs = (np.empty((B, S, H, Dqk)), np.empty((B, S, H, v_dim)), np.empty((B, S, H, Dqk)),
            np.empty((B, S, H, v_dim)))
    _load().oracle_mla_prologue(_ptr(q_resid), _ptr(q_comp), _ptr(hidden), _ptr(wq_gate),
                                _ptr(wkv_a), _ptr(wkv_b), _ptr(rope_cos), _ptr(rope_sin),
                                _dtype_of(q_resid, q_comp, hidden, wq_gate, wkv_a, wkv_b), B, S,
                                past_len, Qr, Qc, Hd, L, H, nope, rope, v_dim, *[_ptr(o) for o in outs])
    return outs
