"""Shared test helpers: seeded inputs on host and device, and the comparison rule.

Comparison rule for floating outputs (scores and attention outputs):
    |x - r| <= rtol * (|r| + rms(r))   elementwise,
rms over the finite entries of the compared row, -inf positions equal.
rtol = 2e-2 for bf16 paths and 1e-5 for fp32 paths.
"""
from __future__ import annotations

import numpy as np

import datagen
from datagen.configs import F32, Workload

RTOL = {F32: 1e-5, 1: 2e-2}


def assert_rows_close(got, ref, rtol, axis_rows=-1, what=""):
    """Compare row by row along the last axis with the rms-scaled rule."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g2 = got.reshape(-1, got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    fin = np.isfinite(r2)
    gfin = np.isfinite(g2)
    bad_pattern = np.nonzero((fin != gfin).any(axis=1))[0]
    assert len(bad_pattern) == 0, f"{what}: -inf pattern differs in rows {bad_pattern[:10]}"
    assert np.all(g2[~fin] == r2[~fin]), f"{what}: non-finite values differ"
    r0 = np.where(fin, r2, 0.0)
    cnt = np.maximum(fin.sum(axis=1, keepdims=True), 1)
    rms = np.sqrt((r0 ** 2).sum(axis=1, keepdims=True) / cnt)
    excess = np.where(fin, np.abs(np.where(fin, g2, 0.0) - r0) - rtol * (np.abs(r0) + rms), -1.0)
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max(initial=-1.0) <= 0.0, (
        f"{what}: row {worst[0]} col {worst[1]}: got {g2[worst]} ref {r2[worst]} "
        f"(excess {excess[worst]:.3g}, rms {rms[worst[0], 0]:.3g})")


def host_inputs(wl: Workload, S: int | None = None, past_len: int | None = None,
                T: int | None = None, with_attn=True, with_index=True, B: int | None = None,
                q_row0: int = 0):
    """Host arrays for a workload, optionally with overridden sizes.

    Query-side tensors start at row q_row0 of their streams (row = b*S_total + s
    with S_total = S), cache tensors cover T rows. Returns dict of numpy arrays.
    """
    B = wl.B if B is None else B
    S = wl.S if S is None else S
    P = wl.past_len if past_len is None else past_len
    T = P + S if T is None else T
    dt = wl.dtype_name
    g = lambda shape, tid, sc, start=0: datagen.normal_host(shape, dt, wl.seed, tid, sc, start)
    out = {}
    if with_index:
        out["q_idx"] = g((B, S, wl.HI, wl.DI), datagen.TID_QIDX, wl.scale_qidx, q_row0 * wl.HI * wl.DI)
        out["k_idx"] = g((B, T, wl.DI), datagen.TID_KIDX, wl.scale_kidx)
        out["w"] = g((B, S, wl.HI), datagen.TID_W, wl.scale_w, q_row0 * wl.HI)
    if with_attn:
        out["q"] = g((B, S, wl.H, wl.Dqk), datagen.TID_Q, wl.scale_q, q_row0 * wl.H * wl.Dqk)
        out["k"] = g((B, T, wl.H, wl.Dqk), datagen.TID_K, wl.scale_k)
        out["v"] = g((B, T, wl.H, wl.v), datagen.TID_V, wl.scale_v)
        out["gate"] = g((B, S, wl.H), datagen.TID_GATE, wl.scale_gate, q_row0 * wl.H)
    return out


def to_dev(a, device="cuda"):
    """numpy (float32 / uint16 bf16 bits / int32) -> torch tensor on the GPU."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_dev(t):
    """torch tensor -> numpy with bf16 widened exactly to float32."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def widen(a):
    return datagen.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
