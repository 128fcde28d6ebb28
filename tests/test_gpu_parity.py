"""Parity of every C-ABI entry point against the fp64 oracle (GPU).

Inputs come from the seeded generator (host twin for the oracle, identical
bytes uploaded for the GPU). Top-k is compared bit-exactly on the same fp32
score tensor (the oracle's own scores rounded to fp32); attention is compared
on the same index tensor (the oracle's top-k or a generated index set).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import sparse_attention_11_amd as dsa
from datagen.configs import WORKLOADS, F32
from tests._helpers import assert_rows_close, host_inputs, to_dev, from_dev, widen, RTOL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------- generator
def test_device_generator_matches_host():
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        t = torch.empty(1 << 20, dtype=tdt, device=DEV)
        datagen.normal_device(t, 3, 2, 0.7, start=12345)
        h = datagen.normal_host((1 << 20,), dt, 3, 2, 0.7, start=12345)
        _sync()
        got = t.cpu().view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.cpu().numpy()
        assert np.array_equal(got.view(np.uint8), h.view(np.uint8))
    ti = torch.empty(300, 64, dtype=torch.int32, device=DEV)
    datagen.indices_device(ti, 100, 400, 50, seed=2)
    _sync()
    assert np.array_equal(ti.cpu().numpy(), datagen.indices_host(100, 300, 400, 50, 64, seed=2))
    for mode in (0, 1, 2):
        ts = torch.empty(70, 333, dtype=torch.float32, device=DEV)
        datagen.scores_device(ts, 5, 80, 200, seed=4, mode=mode)
        _sync()
        ref = datagen.scores_host(5, 70, 80, 333, 200, seed=4, mode=mode)
        assert np.array_equal(ts.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------- indexer
def _run_index(hi, past_len, mode=dsa.RELU_PER_HEAD, scale=None):
    B, S, HI, DI = hi["q_idx"].shape
    T = hi["k_idx"].shape[1]
    sc = torch.empty(B, S, T, dtype=torch.float32, device=DEV)
    sc.fill_(float("nan"))
    dsa.dsa_index_scores(to_dev(hi["q_idx"]), to_dev(hi["k_idx"]), to_dev(hi["w"]), sc, past_len,
                         scale=scale, relu_mode=mode)
    _sync()
    return sc.cpu().numpy()


def test_index_scores_tiny_fp32():
    wl = WORKLOADS["tiny-fp32"]
    hi = host_inputs(wl, with_attn=False)
    got = _run_index(hi, 0)
    ref = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], 0)
    assert_rows_close(got, ref, RTOL[F32], what="tiny-fp32 scores")


def test_index_scores_mla_s4k():
    wl = WORKLOADS["mla-s4k"]
    hi = host_inputs(wl, with_attn=False)
    got = _run_index(hi, 0)
    ref = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], 0)
    assert_rows_close(got, ref, 2e-2, what="mla-s4k scores")


# (B, S, P, HI, DI, mode): tile path (S >= 32) and head-major rows path (S < 32)
INDEX_CASES = [
    (1, 200, 0, 3, 32, 0), (1, 200, 0, 3, 32, 1), (1, 200, 0, 3, 32, 2),
    (2, 130, 73, 5, 128, 0), (1, 257, 0, 64, 128, 0), (1, 64, 1000, 16, 64, 2),
    (2, 1, 999, 64, 128, 0), (3, 5, 300, 40, 64, 0), (1, 3, 40, 130, 32, 0),
    (1, 7, 0, 32, 128, 1), (2, 1, 4095, 4, 64, 2),
    # several 512-key tiles, head counts that leave a partial last LDS stage
    (1, 600, 0, 9, 64, 0), (1, 1000, 500, 13, 128, 2), (2, 333, 1200, 17, 32, 1),
    # heads x dim <= 512: 32-query tiles (two query groups share the key registers)
    (1, 700, 100, 4, 64, 0), (2, 150, 600, 8, 32, 2), (1, 1100, 0, 8, 64, 1),
    # few heads at dim 128 (one query group)
    (2, 150, 600, 4, 128, 2),
    # T >= 8 S: one workgroup multiplies a key tile with both query tiles of its pair
    (1, 100, 3000, 8, 128, 0), (2, 37, 700, 3, 64, 1), (1, 50, 900, 70, 128, 2),
    # per-head ReLU with 16+ heads at every dim, with partial last LDS stages,
    # ragged query and key tiles, and the key-stationary form (T >= 8 S)
    (1, 600, 0, 16, 32, 0), (1, 300, 0, 33, 32, 0), (2, 333, 1200, 20, 64, 0),
    (1, 1000, 500, 64, 128, 0), (1, 100, 3000, 18, 128, 0), (2, 70, 900, 17, 64, 0),
    # few-query rows through the LDS-streamed form: waves whose keys are all
    # visible and the wave holding each row's bound, ragged T, dims 64 and 32
    (2, 31, 577, 64, 64, 0), (1, 17, 1300, 48, 32, 2),
]


@pytest.mark.parametrize("B,S,P,HI,DI,mode", INDEX_CASES)
def test_index_scores_bf16_cases(B, S, P, HI, DI, mode):
    T = P + S
    seed = 100 + S + HI
    g = lambda shape, tid, sc: datagen.normal_host(shape, "bf16", seed, tid, sc)
    hi = {"q_idx": g((B, S, HI, DI), 4, DI ** -0.5), "k_idx": g((B, T, DI), 5, 1.0),
          "w": g((B, S, HI), 6, HI ** -0.5)}
    got = _run_index(hi, P, mode=mode)
    ref = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], P, relu_mode=mode)
    assert_rows_close(got, ref, 2e-2, what=f"scores {B, S, P, HI, DI, mode}")


def test_index_scores_custom_scale_and_longer_cache():
    # T larger than past_len + S (keys beyond the last position are masked)
    B, S, P, HI, DI = 1, 40, 10, 4, 64
    T = 100
    g = lambda shape, tid: datagen.normal_host(shape, "bf16", 9, tid, 0.5)
    hi = {"q_idx": g((B, S, HI, DI), 4), "k_idx": g((B, T, DI), 5), "w": g((B, S, HI), 6)}
    got = _run_index(hi, P, scale=0.3)
    ref = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], P, scale=0.3)
    assert_rows_close(got, ref, 2e-2, what="scores T > P+S")


# ----------------------------------------------------------------- top-k
def _run_topk(scores32: np.ndarray, k: int, order: int = 0) -> np.ndarray:
    B, S, T = scores32.shape
    idx = torch.full((B, S, k), -7, dtype=torch.int32, device=DEV)
    (dsa.dsa_topk_unsorted if order else dsa.dsa_topk)(to_dev(scores32), idx)
    _sync()
    return idx.cpu().numpy()


def as_set(x: np.ndarray) -> np.ndarray:
    """Index lists in canonical form: the selected positions ascending, then
    the -1 slots. Unsorted results must also hold their -1 slots last."""
    out = np.full_like(x, -1)
    for r in np.ndindex(x.shape[:-1]):
        valid = x[r] >= 0
        assert not np.any(valid[1:] & ~valid[:-1]), f"row {r}: a -1 slot before a selected one"
        sel = np.sort(x[r][valid])
        out[r][:len(sel)] = sel
    return out


def test_topk_on_oracle_scores_tiny_and_mla():
    for name in ("tiny-fp32", "mla-s4k"):
        wl = WORKLOADS[name]
        hi = host_inputs(wl, with_attn=False)
        sc = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], 0).astype(np.float32)
        got = _run_topk(sc, wl.topk)
        np.testing.assert_array_equal(got, oracle.topk(sc, wl.topk), err_msg=name)


@pytest.mark.parametrize("T,P,k,mode", [
    (100, 60, 1, 0), (100, 60, 17, 1), (256, 0, 64, 2), (5000, 4000, 2048, 1),
    (5000, 4500, 512, 2), (2048, 2000, 2048, 0), (33000, 32900, 2048, 1), (40000, 39990, 300, 2),
    (8192, 8100, 8, 1),
    # one-wave-per-row path (T <= 4096, k <= 512)
    (4096, 4000, 512, 1), (4096, 3990, 256, 2), (3000, 2900, 300, 1), (1000, 976, 512, 0),
    (4096, 4072, 129, 0),
])
@pytest.mark.parametrize("order", [0, 1])
def test_topk_synthetic_rows(T, P, k, mode, order):
    S = T - P
    rows = min(S, 24)
    sc = datagen.scores_host(0, rows, S, T, P, seed=T + k, mode=mode)
    got = _run_topk(sc[None], k, order)[0]
    ref = oracle.topk(sc, k)
    np.testing.assert_array_equal(as_set(got) if order else got, as_set(ref) if order else ref)


# Enough rows that every stage runs 256-thread workgroups (few-row calls use
# 1024-thread ones): a mid-length single-stage row and a two-stage row.
@pytest.mark.parametrize("rows,T,k,mode", [(300, 6000, 1024, 1), (96, 33000, 2048, 0)])
@pytest.mark.parametrize("order", [0, 1])
def test_topk_many_rows(rows, T, k, mode, order):
    P = T - rows
    sc = datagen.scores_host(0, rows, rows, T, P, seed=rows + T, mode=mode)
    got = _run_topk(sc[None], k, order)[0]
    ref = oracle.topk(sc, k)
    np.testing.assert_array_equal(as_set(got) if order else got, as_set(ref) if order else ref)


@pytest.mark.parametrize("T,k", [(3000, 2048), (2000, 500), (4096, 512)])
@pytest.mark.parametrize("order", [0, 1])
def test_topk_constant_and_all_masked_tail(T, k, order):
    sc = np.zeros((2, T), np.float32)
    sc[1, 5:] = -np.inf
    sc[0, ::2] = -0.0
    got = _run_topk(sc[None], k, order)[0]
    ref = oracle.topk(sc, k)
    np.testing.assert_array_equal(as_set(got) if order else got, as_set(ref) if order else ref)
    assert got[1, 5:].tolist() == [-1] * (k - 5)


# Few rows longer than one segment take the histogram-threshold path
# (threshold bin from the row's top-11-bit histogram, candidates in and above
# it, exact selection among them): constant rows (every key in the tie bin,
# the candidates are the whole row), +-0 ties, -inf tails, rows with fewer
# valid keys than k, chunk-boundary lengths.
@pytest.mark.parametrize("R,T,k", [(3, 40000, 2048), (1, 16385, 700), (2, 8192 * 5, 2048),
                                   (5, 70001, 129)])
@pytest.mark.parametrize("order", [0, 1])
def test_topk_row_path_edge_rows(R, T, k, order):
    rng = np.random.default_rng(T + k)
    sc = rng.standard_normal((R, T)).astype(np.float32)
    sc[0, :] = 0.25                      # constant row
    if R > 1:
        sc[1, ::3] = -0.0                # signed zeros among positives and negatives
        sc[1, ::2] = 0.0
    if R > 2:
        sc[2, 100:] = -np.inf            # 100 valid keys (fewer than k when k > 100)
    if R > 3:
        sc[3, :] = np.round(sc[3, :] * 4) / 4  # many exact ties
    got = _run_topk(sc[None], k, order)[0]
    ref = oracle.topk(sc, k)
    np.testing.assert_array_equal(as_set(got) if order else got, as_set(ref) if order else ref)


# Run-to-run determinism: both top-k calls must return the same array twice,
# order and -1 slots included (the unsorted call's order is its compaction
# order, which depends only on the scores). Shapes: single-stage rows
# (T <= 16384), two-segment rows and one 528 385-key row (two reduction passes).
@pytest.mark.parametrize("R,T,k,mode", [(64, 12000, 2048, 1), (48, 30000, 2048, 2),
                                        (1, 528385, 2048, 1), (1, 528385, 2048, 0)])
@pytest.mark.parametrize("order", [0, 1])
def test_topk_deterministic_run_to_run(R, T, k, mode, order):
    P = T - R
    sc = torch.empty(R, T, dtype=torch.float32, device=DEV)
    datagen.scores_device(sc, 0, R, P, seed=T + R, mode=mode)
    fn = dsa.dsa_topk_unsorted if order else dsa.dsa_topk
    a = torch.full((1, R, k), -7, dtype=torch.int32, device=DEV)
    b = torch.full((1, R, k), -9, dtype=torch.int32, device=DEV)
    fn(sc.view(1, R, T), a)
    fn(sc.view(1, R, T), b)
    _sync()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    # and the selection is the oracle's
    ref = oracle.topk(datagen.scores_host(0, R, R, T, P, seed=T + R, mode=mode), k)
    got = a.cpu().numpy()[0]
    np.testing.assert_array_equal(as_set(got) if order else got, as_set(ref) if order else ref)


# ------------------------------------------------ fused indexer + top-k
# dsa_index_topk against dsa_index_scores + dsa_topk / dsa_topk_unsorted on
# the same inputs: bit-identical indices. Its workspace is filled with 0x7F
# bytes (3.4e38 as fp32) first, so a read of any score above a row's causal
# bound (which the fused call never writes) would be selected and show up.
INDEX_TOPK_CASES = [  # B, S, T, P, HI, DI, k, dtype
    (1, 600, 600, 0, 4, 64, 64, 1),          # tile indexer, one top-k stage, rows with < k visible
    (2, 300, 20300, 20000, 8, 128, 512, 1),  # chunk after a long past: segmented top-k
    (4, 1, 70001, 70000, 16, 128, 2048, 1),  # decode: rows indexer, long-row top-k
    (1, 8, 9000, 8992, 4, 32, 100, 1),       # few queries: rows indexer with causal rows
    (1, 3, 50000, 10000, 8, 64, 2048, 1),    # rows end long before T (long-row path, empty chunks)
    (1, 100, 100, 0, 2, 32, 16, 0),          # fp32
    (1, 700, 700, 0, 32, 128, 256, 1),       # tile indexer with the weighted-query pass
]


@pytest.mark.parametrize("B,S,T,P,HI,DI,k,dt", INDEX_TOPK_CASES)
@pytest.mark.parametrize("srt", [True, False])
def test_index_topk_matches_two_calls(B, S, T, P, HI, DI, k, dt, srt):
    print(f"index_topk B {B} S {S} T {T} P {P} HI {HI} DI {DI} k {k} dtype {dt} sorted {srt}",
          flush=True)
    tdt = torch.bfloat16 if dt == 1 else torch.float32
    g = lambda shape, tid, sc=1.0: datagen.normal_device(torch.empty(*shape, dtype=tdt, device=DEV),
                                                         17 + S, tid, sc)
    qi, ki, w = g((B, S, HI, DI), 1), g((B, T, DI), 2), g((B, S, HI), 3, HI ** -0.5)
    sc = torch.empty(B, S, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(qi, ki, w, sc, P)
    ref = torch.full((B, S, k), -7, dtype=torch.int32, device=DEV)
    (dsa.dsa_topk if srt else dsa.dsa_topk_unsorted)(sc, ref)
    ws = torch.full((dsa.dsa_index_topk_workspace_size(B, S, T, k),), 0x7F, dtype=torch.uint8,
                    device=DEV)
    got = torch.full((B, S, k), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_index_topk(qi, ki, w, got, P, sorted=srt, workspace=ws)
    _sync()
    assert torch.equal(got, ref), f"{int((got != ref).sum())} of {got.numel()} slots differ"


# ----------------------------------------------------- sparse attention
def _attn_dev(hi):
    return {k_: to_dev(v_) for k_, v_ in hi.items()}


def _run_prefill(hi, idx, past_len, nope, rope, gate=None, gate_dim=1):
    B, S, H, Dqk = hi["q"].shape
    Dv = hi["v"].shape[3]
    dt = torch.bfloat16 if hi["q"].dtype == np.uint16 else torch.float32
    out = torch.full((B, S, H, Dv), float("nan"), dtype=dt, device=DEV)
    g = None if gate is None else to_dev(gate)
    dsa.dsa_sparse_attn_prefill(to_dev(hi["q"]), to_dev(hi["k"]), to_dev(hi["v"]), to_dev(idx), g,
                                out, past_len, nope, rope)
    _sync()
    return from_dev(out)


def _cmp_attn(got, ref, rtol, what):
    Dv = ref.shape[-1]
    assert_rows_close(got.reshape(-1, Dv), ref.reshape(-1, Dv), rtol, what=what)


def test_prefill_tiny_fp32_chain_indices():
    wl = WORKLOADS["tiny-fp32"]
    hi = host_inputs(wl)
    sc = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], 0).astype(np.float32)
    idx = oracle.topk(sc, wl.topk)
    got = _run_prefill(hi, idx, 0, wl.nope, wl.rope, hi["gate"])
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], 0, wl.nope, wl.rope)
    _cmp_attn(got, ref, RTOL[F32], "tiny-fp32 prefill")


def test_prefill_mla_s4k_chain_indices():
    wl = WORKLOADS["mla-s4k"]
    hi = host_inputs(wl)
    sc = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], 0).astype(np.float32)
    idx = oracle.topk(sc, wl.topk)
    got = _run_prefill(hi, idx, 0, wl.nope, wl.rope, hi["gate"])
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], 0, wl.nope, wl.rope)
    _cmp_attn(got, ref, 2e-2, "mla-s4k prefill")


def _attn_case(B, S, P, H, nope, rope, Dv, seed, dt="bf16"):
    T = P + S
    Dqk = nope + rope
    g = lambda shape, tid, sc: datagen.normal_host(shape, dt, seed, tid, sc)
    return {"q": g((B, S, H, Dqk), 1, Dqk ** -0.25), "k": g((B, T, H, Dqk), 2, Dqk ** -0.25),
            "v": g((B, T, H, Dv), 3, 1.0), "gate": g((B, S, H), 7, 1.0)}


# (B, S, P, H, nope, rope, Dv, topk): MFMA path for bf16 S >= 16, gather otherwise
PREFILL_CASES = [
    (1, 200, 50, 3, 128, 64, 128, 64), (2, 130, 100, 2, 64, 64, 128, 200), (1, 77, 300, 4, 32, 32, 64, 33),
    (1, 64, 0, 2, 128, 128, 128, 64), (1, 96, 10, 2, 64, 64, 64, 16), (2, 8, 500, 5, 128, 64, 128, 128),
    (1, 1, 40, 3, 64, 64, 128, 41), (1, 300, 1800, 1, 128, 64, 128, 2048),
    # head dims 256 / 256 (one workgroup per CU, long tiles split and merged)
    (1, 150, 100, 2, 128, 128, 256, 64),
    # bf16 chunks whose visible keys per query exceed 128 x topk take the row
    # gather: more than 32 heads (two head groups), ragged heads, small topk
    (1, 64, 20000, 2, 128, 64, 128, 64), (2, 40, 9000, 3, 64, 64, 128, 32),
    (1, 20, 12000, 40, 64, 32, 64, 48), (1, 17, 70000, 1, 128, 64, 128, 500),
    # qk 96 (A.X-K2-Light: nope 64 + rope 32) on the MFMA path, v 64 and 128
    (1, 150, 40, 3, 64, 32, 64, 48), (2, 90, 0, 2, 64, 32, 128, 64), (1, 300, 200, 1, 64, 32, 64, 300),
]


@pytest.mark.parametrize("B,S,P,H,nope,rope,Dv,k", PREFILL_CASES)
def test_prefill_bf16_cases(B, S, P, H, nope, rope, Dv, k):
    hi = _attn_case(B, S, P, H, nope, rope, Dv, seed=S + H)
    idx = datagen.indices_host(0, B * S, S, P, k, seed=S + k).reshape(B, S, k)
    got = _run_prefill(hi, idx, P, nope, rope, hi["gate"])
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], P, nope, rope)
    _cmp_attn(got, ref, 2e-2, f"prefill {B, S, P, H, nope, rope, Dv, k}")


# (B, S, P, H, nope, rope, Dv, k, gate): grids of at least 1024 workgroups of 256
# queries (selection mask, no sinks, no split) take the ping-pong prefill kernel,
# one case per head-dim pair it is built for; ragged last tiles, past context,
# the elementwise gate. Checked rows: both 128-query groups of the first, a
# middle and the last tile (their first, last and inner rows) plus random rows.
PINGPONG_CASES = [
    (1, 2085, 37, 128, 128, 64, 128, 256, "head"), (2, 1024, 0, 128, 64, 64, 128, 300, "head"),
    (1, 2048, 100, 128, 64, 64, 64, 128, "elem"), (1, 2048, 0, 128, 32, 32, 64, 64, "head"),
    (1, 1800, 5, 160, 64, 32, 64, 96, "head"), (1, 1800, 5, 160, 64, 32, 128, 96, "none"),
]


def _pp_rows(S, seed):
    nt = (S + 255) // 256
    rows = set()
    for t in (0, nt // 2, nt - 1):
        for r in (0, 31, 100, 127, 128, 159, 254, 255):
            rows.add(min(t * 256 + r, S - 1))
    rows |= set(np.random.default_rng(seed).integers(0, S, 16).tolist())
    return sorted(rows)


@pytest.mark.parametrize("B,S,P,H,nope,rope,Dv,k,gk", PINGPONG_CASES)
def test_prefill_pingpong_cases(B, S, P, H, nope, rope, Dv, k, gk):
    assert B * H * ((S + 255) // 256) >= 1024  # the grid that selects the ping-pong kernel
    hi = _attn_case(B, S, P, H, nope, rope, Dv, seed=S + H + Dv)
    idx = datagen.indices_host(0, B * S, S, P, k, seed=S + k).reshape(B, S, k)
    gate = {"none": None, "head": hi["gate"],
            "elem": datagen.normal_host((B, S, H, Dv), "bf16", 5, 8, 1.0)}[gk]
    got = _run_prefill(hi, idx, P, nope, rope, gate)
    for b in range(B):
        for s in _pp_rows(S, seed=S + b):
            g = None if gate is None else gate[b:b + 1, s:s + 1]
            ref = oracle.sparse_attn(hi["q"][b:b + 1, s:s + 1], hi["k"][b:b + 1], hi["v"][b:b + 1],
                                     idx[b:b + 1, s:s + 1], g, P + s, nope, rope)
            _cmp_attn(got[b:b + 1, s:s + 1], ref, 2e-2, f"ping-pong {B, S, P, H, nope, rope, Dv, k} b{b} s{s}")


@pytest.mark.parametrize("gate_kind", ["none", "elementwise", "limits"])
def test_prefill_gate_modes(gate_kind):
    B, S, P, H, nope, rope, Dv, k = 1, 150, 20, 3, 128, 64, 128, 48
    hi = _attn_case(B, S, P, H, nope, rope, Dv, seed=5)
    idx = datagen.indices_host(0, S, S, P, k, seed=6).reshape(B, S, k)
    if gate_kind == "none":
        gate = None
    elif gate_kind == "elementwise":
        gate = datagen.normal_host((B, S, H, Dv), "bf16", 5, 8, 1.0)
    else:
        gf = np.zeros((B, S, H), np.float32)
        gf[..., 0], gf[..., 1], gf[..., 2] = -np.inf, np.inf, 0.0
        gate = torch.from_numpy(gf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = _run_prefill(hi, idx, P, nope, rope, gate)
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, gate, P, nope, rope)
    _cmp_attn(got, ref, 2e-2, f"gate {gate_kind}")
    if gate_kind == "limits":
        assert np.all(got[:, :, 0] == 0.0)
        ung = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, None, P, nope, rope)
        _cmp_attn(got[:, :, 1], ung[:, :, 1], 2e-2, "gate +inf")


def test_prefill_set_semantics_on_gpu():
    # -1 padding, future and out-of-range entries are ignored by the GPU too
    B, S, P, H, nope, rope, Dv, k = 1, 100, 0, 2, 64, 64, 128, 24
    hi = _attn_case(B, S, P, H, nope, rope, Dv, seed=8)
    base = datagen.indices_host(0, S, S, P, k, seed=9).reshape(B, S, k)
    junk = base.copy()
    junk[:, :, -4] = -1
    junk[:, :, -3] = np.arange(S)[None, :] + 1  # future position (ignored)
    junk[:, :, -2] = S + 1000                     # beyond T (ignored)
    got = _run_prefill(hi, junk, P, nope, rope, hi["gate"])
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], junk, hi["gate"], P, nope, rope)
    _cmp_attn(got, ref, 2e-2, "junk indices")


def test_prefill_fp32_gather_path():
    hi = _attn_case(2, 40, 30, 3, 32, 16, 32, seed=12, dt="f32")
    idx = datagen.indices_host(0, 80, 40, 30, 20, seed=13).reshape(2, 40, 20)
    got = _run_prefill(hi, idx, 30, 32, 16, hi["gate"])
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], 30, 32, 16)
    _cmp_attn(got, ref, 1e-5, "fp32 prefill")


# ---------------------------------------------------------------- decode
# bf16 calls with rows x heads >= 256 take the whole-row decode kernel, the
# others the split form and its merge
@pytest.mark.parametrize("B,T,H,nope,rope,Dv,k,dt", [
    (3, 3000, 16, 128, 64, 128, 256, "bf16"), (2, 700, 4, 64, 64, 128, 700, "bf16"),
    (1, 5000, 8, 128, 64, 128, 2048, "bf16"), (2, 300, 4, 32, 16, 32, 64, "f32"),
    (2, 4000, 160, 64, 32, 64, 1000, "bf16"),
])
def test_decode_cases(B, T, H, nope, rope, Dv, k, dt):
    P = T - 1
    hi = _attn_case(B, 1, P, H, nope, rope, Dv, seed=T + k, dt=dt)
    idx = np.stack([datagen.indices_host(0, 1, 1, P, k, seed=T + b) for b in range(B)])
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((B, 1, H, Dv), float("nan"), dtype=tdt, device=DEV)
    dsa.dsa_sparse_attn_decode(to_dev(hi["q"]), to_dev(hi["k"]), to_dev(hi["v"]), to_dev(idx),
                               to_dev(hi["gate"]), out, nope, rope)
    _sync()
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], P, nope, rope)
    _cmp_attn(from_dev(out), ref, RTOL[F32] if dt == "f32" else 2e-2, f"decode {B, T, k, dt}")


# ------------------------------------------------------------------- SWA
@pytest.mark.parametrize("B,S,P,W,H,nope,rope,Dv,dt,offset", [
    (1, 300, 700, 128, 2, 128, 64, 128, "bf16", True), (2, 200, 0, 64, 3, 64, 64, 128, "bf16", False),
    (1, 150, 40, 512, 2, 128, 64, 128, "bf16", True), (1, 1, 900, 512, 4, 128, 64, 128, "bf16", True),
    (2, 6, 100, 32, 3, 64, 64, 64, "bf16", True), (1, 50, 20, 16, 2, 32, 16, 32, "f32", True),
    (1, 200, 300, 64, 2, 64, 32, 64, "bf16", True), (1, 130, 0, 40, 3, 64, 32, 128, "bf16", False),
])
def test_swa_cases(B, S, P, W, H, nope, rope, Dv, dt, offset):
    kv_off = max(0, P - W + 1) if offset else 0
    T = P + S
    full = _attn_case(B, S, P, H, nope, rope, Dv, seed=W + S, dt=dt)
    kb, vb = full["k"][:, kv_off:].copy(), full["v"][:, kv_off:].copy()
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((B, S, H, Dv), float("nan"), dtype=tdt, device=DEV)
    dsa.swa_attn(to_dev(full["q"]), to_dev(kb), to_dev(vb), to_dev(full["gate"]), out, P, kv_off, W,
                 nope, rope)
    _sync()
    ref = oracle.swa_attn(full["q"], kb, vb, full["gate"], P, kv_off, W, nope, rope)
    _cmp_attn(from_dev(out), ref, RTOL[F32] if dt == "f32" else 2e-2, f"swa {B, S, P, W}")


# ------------------------------------------------- SWA, grouped KV heads
@pytest.mark.parametrize("B,S,P,W,H,H_kv,nope,rope,Dv,dt,offset", [
    (1, 300, 700, 512, 8, 2, 128, 128, 256, "bf16", True),   # Spark heads, MFMA path
    (2, 200, 0, 64, 8, 2, 128, 64, 128, "bf16", False),
    (1, 130, 5, 512, 6, 3, 64, 64, 64, "bf16", False),
    (2, 100, 50, 32, 8, 8, 128, 128, 256, "bf16", True),     # H_kv = H at dims 256
    (1, 1, 900, 512, 8, 2, 128, 128, 256, "bf16", True),     # decode (gather path)
    (2, 5, 60, 16, 4, 1, 32, 16, 32, "f32", True),
    (1, 20, 10, 8, 8, 2, 128, 128, 256, "f32", False),
])
def test_swa_gqa_cases(B, S, P, W, H, H_kv, nope, rope, Dv, dt, offset):
    kv_off = max(0, P - W + 1) if offset else 0
    T = P + S
    Dqk = nope + rope
    g = lambda shape, tid, sc: datagen.normal_host(shape, dt, W + S + H_kv, tid, sc)
    q, gate = g((B, S, H, Dqk), 1, Dqk ** -0.25), g((B, S, H), 7, 1.0)
    kb = g((B, T, H_kv, Dqk), 2, Dqk ** -0.25)[:, kv_off:].copy()
    vb = g((B, T, H_kv, Dv), 3, 1.0)[:, kv_off:].copy()
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((B, S, H, Dv), float("nan"), dtype=tdt, device=DEV)
    dsa.swa_attn_gqa(to_dev(q), to_dev(kb), to_dev(vb), to_dev(gate), out, P, kv_off, W, nope,
                     rope)
    _sync()
    ref = oracle.swa_attn_gqa(q, kb, vb, gate, P, kv_off, W, nope, rope)
    _cmp_attn(from_dev(out), ref, RTOL[F32] if dt == "f32" else 2e-2,
              f"swa gqa {B, S, P, W, H, H_kv, Dv, dt}")


# ------------------------------------------------------------ full chain
def test_chain_mla_s4k_end_to_end():
    """GPU indexer -> GPU top-k -> GPU attention vs the oracle's own chain.

    Index sets may differ only at near-ties of the k-th score; rows whose
    sets agree must match the oracle's attention output."""
    wl = WORKLOADS["mla-s4k"]
    hi = host_inputs(wl)
    d = _attn_dev(hi)
    S, T, k = wl.S, wl.T, wl.topk
    sc = torch.empty(1, S, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(d["q_idx"], d["k_idx"], d["w"], sc, 0)
    idx = torch.empty(1, S, k, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(sc, idx)
    out = torch.empty(1, S, wl.H, wl.v, dtype=torch.bfloat16, device=DEV)
    dsa.dsa_sparse_attn_prefill(d["q"], d["k"], d["v"], idx, d["gate"], out, 0, wl.nope, wl.rope)
    _sync()
    g_idx = idx.cpu().numpy()[0]
    ref_sc = oracle.index_scores(hi["q_idx"], hi["k_idx"], hi["w"], 0)[0]
    o_idx = oracle.topk(ref_sc.astype(np.float32), k)
    same = np.array([set(g_idx[s]) == set(o_idx[s]) for s in range(S)])
    for s in np.nonzero(~same)[0]:
        kth = np.sort(ref_sc[s][np.isfinite(ref_sc[s])])[::-1][min(k, s + 1) - 1]
        fin = ref_sc[s][np.isfinite(ref_sc[s])]
        rms = math.sqrt(float(np.mean(fin ** 2)))
        for t in set(g_idx[s]) ^ set(o_idx[s]):
            assert abs(ref_sc[s, t] - kth) <= 2e-2 * (abs(kth) + rms), (s, t)
    assert same.mean() > 0.95
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], o_idx[None], hi["gate"], 0, wl.nope, wl.rope)
    got = from_dev(out)
    rows = np.nonzero(same)[0]
    _cmp_attn(got[0, rows], ref[0, rows], 2e-2, "chain mla-s4k")


# ------------------------------------------------ attention sinks (PAS)
def _sinks(H, nope, rope, Dv, n, seed, dt="bf16"):
    Dqk = nope + rope
    g = lambda shape, tid, sc: datagen.normal_host(shape, dt, seed, tid, sc)
    return g((n, H, Dqk), 11, Dqk ** -0.25), g((n, H, Dv), 12, 1.0)


# (B, S, P, H, nope, rope, Dv, topk, n_sink): sink counts that fill, half-fill and
# overrun a 64-key block; the MFMA path (bf16, S >= 16) and the gather path
PAS_PREFILL_CASES = [
    (1, 200, 50, 3, 128, 64, 128, 64, 128), (2, 130, 100, 2, 64, 64, 128, 200, 1),
    (1, 77, 300, 4, 32, 32, 64, 33, 100), (1, 300, 1800, 1, 128, 64, 128, 2048, 256),
    (2, 8, 500, 5, 128, 64, 128, 128, 65), (1, 40, 30, 3, 32, 16, 32, 20, 7),
    # the row-gather path of long bf16 chunks, with sinks
    (1, 50, 20000, 2, 128, 64, 128, 100, 7),
    # qk 96 with sinks on the MFMA path
    (1, 100, 60, 2, 64, 32, 64, 40, 33),
]


@pytest.mark.parametrize("B,S,P,H,nope,rope,Dv,k,n_sink", PAS_PREFILL_CASES)
def test_prefill_with_sinks(B, S, P, H, nope, rope, Dv, k, n_sink):
    dt = "f32" if (B, S) == (1, 40) else "bf16"
    hi = _attn_case(B, S, P, H, nope, rope, Dv, seed=S + n_sink, dt=dt)
    sk, sv = _sinks(H, nope, rope, Dv, n_sink, seed=n_sink, dt=dt)
    idx = datagen.indices_host(0, B * S, S, P, k, seed=S + k).reshape(B, S, k)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((B, S, H, Dv), float("nan"), dtype=tdt, device=DEV)
    dsa.dsa_sparse_attn_prefill_pas(to_dev(hi["q"]), to_dev(hi["k"]), to_dev(hi["v"]), to_dev(sk),
                                    to_dev(sv), to_dev(idx), to_dev(hi["gate"]), out, P, nope, rope)
    _sync()
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], P, nope, rope,
                             sink_k=sk, sink_v=sv)
    _cmp_attn(from_dev(out), ref, RTOL[F32] if dt == "f32" else 2e-2,
              f"prefill+sinks {B, S, P, H, nope, rope, Dv, k, n_sink}")


def test_prefill_sinks_only_when_selection_is_empty():
    B, S, P, H, nope, rope, Dv, n_sink = 1, 130, 0, 2, 64, 64, 128, 70
    hi = _attn_case(B, S, P, H, nope, rope, Dv, seed=5)
    sk, sv = _sinks(H, nope, rope, Dv, n_sink, seed=6)
    idx = np.full((B, S, 8), -1, np.int32)
    out = torch.full((B, S, H, Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    dsa.dsa_sparse_attn_prefill_pas(to_dev(hi["q"]), to_dev(hi["k"]), to_dev(hi["v"]), to_dev(sk),
                                    to_dev(sv), to_dev(idx), to_dev(hi["gate"]), out, P, nope, rope)
    _sync()
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], P, nope, rope,
                             sink_k=sk, sink_v=sv)
    _cmp_attn(from_dev(out), ref, 2e-2, "sinks only")


@pytest.mark.parametrize("B,T,H,nope,rope,Dv,k,n_sink,dt", [
    (3, 3000, 16, 128, 64, 128, 256, 128, "bf16"), (1, 5000, 8, 128, 64, 128, 2048, 200, "bf16"),
    (2, 300, 4, 32, 16, 32, 64, 3, "f32"),
    (2, 3000, 128, 128, 64, 128, 300, 64, "bf16"),  # whole-row kernel (2 x 128 pairs)
])
def test_decode_with_sinks(B, T, H, nope, rope, Dv, k, n_sink, dt):
    P = T - 1
    hi = _attn_case(B, 1, P, H, nope, rope, Dv, seed=T + n_sink, dt=dt)
    sk, sv = _sinks(H, nope, rope, Dv, n_sink, seed=k, dt=dt)
    idx = np.stack([datagen.indices_host(0, 1, 1, P, k, seed=T + b) for b in range(B)])
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((B, 1, H, Dv), float("nan"), dtype=tdt, device=DEV)
    dsa.dsa_sparse_attn_decode_pas(to_dev(hi["q"]), to_dev(hi["k"]), to_dev(hi["v"]), to_dev(sk),
                                   to_dev(sv), to_dev(idx), to_dev(hi["gate"]), out, nope, rope)
    _sync()
    ref = oracle.sparse_attn(hi["q"], hi["k"], hi["v"], idx, hi["gate"], P, nope, rope,
                             sink_k=sk, sink_v=sv)
    _cmp_attn(from_dev(out), ref, RTOL[F32] if dt == "f32" else 2e-2, f"decode+sinks {B, T, k, n_sink}")


@pytest.mark.parametrize("B,S,P,W,H,nope,rope,Dv,n_sink,dt", [
    (1, 300, 700, 128, 2, 128, 64, 128, 128, "bf16"), (2, 200, 0, 64, 3, 64, 64, 128, 30, "bf16"),
    (1, 1, 900, 512, 4, 128, 64, 128, 128, "bf16"), (1, 50, 20, 16, 2, 32, 16, 32, 5, "f32"),
])
def test_swa_with_sinks(B, S, P, W, H, nope, rope, Dv, n_sink, dt):
    kv_off = max(0, P - W + 1)
    full = _attn_case(B, S, P, H, nope, rope, Dv, seed=W + n_sink, dt=dt)
    sk, sv = _sinks(H, nope, rope, Dv, n_sink, seed=W, dt=dt)
    kb, vb = full["k"][:, kv_off:].copy(), full["v"][:, kv_off:].copy()
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((B, S, H, Dv), float("nan"), dtype=tdt, device=DEV)
    dsa.swa_attn_pas(to_dev(full["q"]), to_dev(kb), to_dev(vb), to_dev(sk), to_dev(sv),
                     to_dev(full["gate"]), out, P, kv_off, W, nope, rope)
    _sync()
    ref = oracle.swa_attn(full["q"], kb, vb, full["gate"], P, kv_off, W, nope, rope,
                          sink_k=sk, sink_v=sv)
    _cmp_attn(from_dev(out), ref, RTOL[F32] if dt == "f32" else 2e-2, f"swa+sinks {B, S, P, W, n_sink}")


# ------------------------------------------------------------ FP8 indexer
def _fp8_rows(R, D, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((R, D)) * 2.0 ** rng.integers(-20, 20, (R, 1))).astype(np.float32)
    if R >= 4:
        x[0] = 0.0                   # all-zero row: scale 1, codes 0
        x[1] = 0.0
        x[1, 3] = -3.0               # one spike: every rotated value is +-3
        x[2] = 1e-30                 # tiny rows stay normal in fp32 after the rotation
        x[3, : D // 2] = 448.0       # large values
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("R,D", [(1, 32), (37, 32), (300, 64), (1000, 128), (4097, 128)])
def test_quant_fp8_bit_exact(R, D):
    xh = _fp8_rows(R, D, seed=R + D)
    codes = torch.empty(R, D, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, dtype=torch.float32, device=DEV)
    dsa.dsa_index_quant_fp8(to_dev(xh), codes, scales)
    _sync()
    rc, rs = oracle.index_quant_fp8(xh)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


FP8_CASES = [  # (B, S, P, HI, mode): idx_dim 128
    (1, 200, 0, 64, 0), (2, 130, 73, 5, 0), (1, 257, 600, 9, 1), (1, 1000, 500, 13, 2),
    (2, 1, 999, 64, 0), (1, 3, 40, 130, 0), (1, 600, 0, 17, 0),
    (2, 333, 700, 24, 0),  # ReLU split (16+ heads): batched, ragged tiles, a past context
]


@pytest.mark.parametrize("B,S,P,HI,mode", FP8_CASES)
def test_index_scores_fp8_cases(B, S, P, HI, mode):
    T, D = P + S, 128
    seed = 300 + S + HI
    g = lambda shape, tid, sc: datagen.normal_host(shape, "bf16", seed, tid, sc)
    q, k, w = g((B, S, HI, D), 4, D ** -0.5), g((B, T, D), 5, 1.0), g((B, S, HI), 6, HI ** -0.5)
    qc = torch.empty(B, S, HI, D, dtype=torch.uint8, device=DEV)
    qs = torch.empty(B, S, HI, dtype=torch.float32, device=DEV)
    kc = torch.empty(B, T, D, dtype=torch.uint8, device=DEV)
    ks = torch.empty(B, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_quant_fp8(to_dev(q), qc, qs)
    dsa.dsa_index_quant_fp8(to_dev(k), kc, ks)
    sc = torch.full((B, S, T), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores_fp8(qc, qs, kc, ks, to_dev(w), sc, P, relu_mode=mode)
    _sync()
    rqc, rqs = oracle.index_quant_fp8(q)
    rkc, rks = oracle.index_quant_fp8(k)
    np.testing.assert_array_equal(qc.cpu().numpy(), rqc)
    np.testing.assert_array_equal(kc.cpu().numpy(), rkc)
    np.testing.assert_array_equal(ks.cpu().numpy(), rks)
    ref = oracle.index_scores_fp8(rqc, rqs, rkc, rks, w, P, relu_mode=mode)
    # same codes on both sides; the FP8 MFMA sums its products with a few bits
    # less than fp32 (measured about 1e-4 of the sum of |products|)
    assert_rows_close(sc.cpu().numpy(), ref, 1e-3, what=f"fp8 scores {B, S, P, HI, mode}")


def test_index_fp8_top_k_recall_against_bf16():
    # the approximation keeps most of the exact indexer's top-k (a property of
    # FP8 scoring, measured here; not a parity bound)
    B, S, P, HI, D, K = 1, 64, 2000, 16, 128, 256
    T = P + S
    g = lambda shape, tid, sc: datagen.normal_host(shape, "bf16", 77, tid, sc)
    q, k, w = g((B, S, HI, D), 4, D ** -0.5), g((B, T, D), 5, 1.0), g((B, S, HI), 6, HI ** -0.5)
    qc = torch.empty(B, S, HI, D, dtype=torch.uint8, device=DEV)
    qs = torch.empty(B, S, HI, dtype=torch.float32, device=DEV)
    kc = torch.empty(B, T, D, dtype=torch.uint8, device=DEV)
    ks = torch.empty(B, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_quant_fp8(to_dev(q), qc, qs)
    dsa.dsa_index_quant_fp8(to_dev(k), kc, ks)
    sc = torch.empty(B, S, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores_fp8(qc, qs, kc, ks, to_dev(w), sc, P)
    idx = torch.empty(B, S, K, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(sc, idx)
    _sync()
    exact = oracle.topk(oracle.index_scores(q, k, w, P).astype(np.float32), K)
    got = idx.cpu().numpy()
    recall = np.mean([len(set(got[0, s]) & set(exact[0, s])) / K for s in range(S)])
    assert recall > 0.85, recall


# ------------------------------------------------------ indexer prologue
def _prologue_case(B, S, Q, Hd, HI, D, seed):
    g = lambda shape, tid, sc: datagen.normal_host(shape, "bf16", seed, tid, sc)
    return dict(q_lora=g((B, S, Q), 20, 1.0), hidden=g((B, S, Hd), 21, 1.0),
                wq_b=g((HI * D, Q), 22, Q ** -0.5), wk=g((D, Hd), 23, Hd ** -0.5),
                k_norm_w=g((D,), 24, 1.0), k_norm_b=g((D,), 25, 0.1),
                weights_proj=g((HI, Hd), 26, Hd ** -0.5))


PROLOGUE_CASES = [  # (B, S, P, Q, Hd, HI, D, R)
    (1, 200, 0, 64, 96, 4, 64, 32), (2, 130, 70, 96, 160, 5, 128, 64), (1, 1, 999, 32, 64, 3, 128, 0),
    (1, 300, 17, 128, 256, 64, 128, 64), (3, 7, 5, 64, 32, 2, 64, 64),
    # rope_dim 128 and 16: the separate RoPE pass instead of the GEMM epilogue
    (1, 50, 3, 64, 64, 3, 128, 128), (1, 40, 0, 32, 64, 2, 64, 16),
]


@pytest.mark.parametrize("B,S,P,Q,Hd,HI,D,R", PROLOGUE_CASES)
def test_indexer_prologue_cases(B, S, P, Q, Hd, HI, D, R):
    T = P + S + 3  # rows past the call's must stay untouched
    x = _prologue_case(B, S, Q, Hd, HI, D, seed=S + HI)
    rng = np.random.default_rng(S)
    ang = rng.uniform(-np.pi, np.pi, (T, R // 2))
    cos, sin = (np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)) if R else (None, None)
    qd = torch.full((B, S, HI, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    kd = torch.full((B, T, D), 7.0, dtype=torch.bfloat16, device=DEV)
    wd = torch.full((B, S, HI), float("nan"), dtype=torch.bfloat16, device=DEV)
    dsa.dsa_indexer_prologue(*[to_dev(x[n]) for n in ("q_lora", "hidden", "wq_b", "wk", "k_norm_w",
                                                      "k_norm_b", "weights_proj")],
                             None if cos is None else to_dev(cos), None if sin is None else to_dev(sin),
                             qd, kd, wd, P, ln_eps=1e-6)
    _sync()
    rq, rk, rw = oracle.indexer_prologue(x["q_lora"], x["hidden"], x["wq_b"], x["wk"], x["k_norm_w"],
                                         x["k_norm_b"], x["weights_proj"], cos, sin, P, HI, 1e-6)
    what = f"prologue {B, S, P, Q, Hd, HI, D, R}"
    assert_rows_close(from_dev(qd), rq, 2e-2, what=what + " q_idx")
    got_k = from_dev(kd)
    assert_rows_close(got_k[:, P:P + S], rk, 2e-2, what=what + " k")
    assert np.all(got_k[:, :P] == 7.0) and np.all(got_k[:, P + S:] == 7.0), "rows outside the call changed"
    assert_rows_close(from_dev(wd), rw, 2e-2, what=what + " w")


# ------------------------------------------------------- MLA prologue
MLA_PROLOGUE_CASES = [
    # B, S, P, Qr, Qc, Hd, L, H, N, R, Dv
    (1, 200, 0, 64, 32, 96, 64, 4, 64, 32, 64),
    (2, 130, 70, 96, 64, 160, 128, 5, 128, 64, 128),   # ragged row tiles, odd head count
    (1, 1, 999, 32, 32, 64, 32, 3, 128, 64, 128),      # one decode token
    (1, 300, 17, 128, 128, 256, 512, 8, 128, 64, 128),  # latent rank 512
    (3, 7, 5, 64, 64, 32, 64, 2, 64, 0, 64),           # no RoPE
    (1, 50, 3, 64, 64, 64, 96, 3, 32, 16, 48),         # small dims
]


@pytest.mark.parametrize("B,S,P,Qr,Qc,Hd,L,H,N,R,Dv", MLA_PROLOGUE_CASES)
def test_mla_prologue_cases(B, S, P, Qr, Qc, Hd, L, H, N, R, Dv):
    seed = S + H
    Dqk, T = N + R, P + S + 3  # three cache rows past the call stay untouched
    g = lambda shape, tid, sc: datagen.normal_host(shape, "bf16", seed, tid, sc)
    qr, qc, hd = g((B, S, Qr), 30, 1.0), g((B, S, Qc), 31, 1.0), g((B, S, Hd), 32, 1.0)
    wq = g((H * (Dqk + Dv), Qr + Qc), 33, (Qr + Qc) ** -0.5)
    wa = g((L + R, Hd), 34, Hd ** -0.5)
    wb = g((H * (N + Dv), L), 35, L ** -0.5)
    cos = sin = None
    if R:
        ang = np.random.default_rng(seed).uniform(-np.pi, np.pi, (T, R // 2))
        cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    q = torch.full((B, S, H, Dqk), float("nan"), dtype=torch.bfloat16, device=DEV)
    gate = torch.full((B, S, H, Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    kc = torch.full((B, T, H, Dqk), 7.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full((B, T, H, Dv), 7.0, dtype=torch.bfloat16, device=DEV)
    dsa.dsa_mla_prologue(to_dev(qr), to_dev(qc), to_dev(hd), to_dev(wq), to_dev(wa), to_dev(wb),
                         None if cos is None else to_dev(cos), None if sin is None else to_dev(sin),
                         q, gate, kc, vc, P)
    _sync()
    rq, rg, rk, rv = oracle.mla_prologue(qr, qc, hd, wq, wa, wb, cos, sin, P, H, N, R, Dv)
    what = f"mla prologue {B, S, P, Qr, Qc, Hd, L, H, N, R, Dv}"
    assert_rows_close(from_dev(q), rq, 2e-2, what=what + " q")
    assert_rows_close(from_dev(gate), rg, 2e-2, what=what + " gate")
    kh, vh = from_dev(kc), from_dev(vc)
    assert_rows_close(kh[:, P:P + S], rk, 2e-2, what=what + " k rows")
    assert_rows_close(vh[:, P:P + S], rv, 2e-2, what=what + " v rows")
    outside = np.ones(T, bool)
    outside[P:P + S] = False
    assert (kh[:, outside] == 7.0).all() and (vh[:, outside] == 7.0).all(), "rows outside the call"
