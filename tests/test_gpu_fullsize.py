"""Parity at the full workload sizes, in the launch configuration the
benchmark times, on sampled outputs the oracle computes one by one (GPU).

Inputs are generated in HBM by the device twin of the seeded generator; the
oracle gets the same values from the host twin. For sampled attention rows
the oracle receives only the selected cache rows (a compact cache whose
position j holds the j-th selected key, with index list 0..n-1): attention
is a function of the selected set, so this is the same result.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import datagen
import oracle
import sparse_attention_11_amd as dsa
from datagen.configs import WORKLOADS
from tests._helpers import assert_rows_close, from_dev, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample_rows(S, k, n=12, seed=0):
    rng = np.random.default_rng(seed)
    base = {0, min(k - 1, S - 1), min(k, S - 1), S - 1}
    extra = rng.choice(S, size=min(n, S), replace=False).tolist()
    return sorted(base | set(extra))


def strat_rows(S, k, block, seed):
    """One seeded row in every block of `block` consecutive query rows (so every
    query tile of that size, and every pair of tiles the indexer schedules
    together, holds a sampled row), plus s = 0, k - 1, k and S - 1."""
    rng = np.random.default_rng(seed)
    rows = {min(b * block + int(rng.integers(0, block)), S - 1) for b in range((S + block - 1) // block)}
    return sorted(rows | {0, min(k - 1, S - 1), min(k, S - 1), S - 1})


def host_stream(wl, shape, tid, scale, start=0):
    """A whole bf16 stream (e.g. a K or V cache) generated once on the host."""
    return datagen.normal_host(shape, "bf16", wl.seed, tid, scale, start)


def check_attn_rows_full(wl, out, idx, rows, kh, vh, b=0, qtid=datagen.TID_Q,
                         gtid=datagen.TID_GATE, S_stream=None, P=0):
    """Compare out[s] (s in rows, query row b*S_stream + s at position P + s)
    against the oracle over the whole host caches kh / vh [B, T, H, D] with the
    row's own index list."""
    S_stream = wl.S if S_stream is None else S_stream
    H, Dqk, Dv = wl.H, wl.Dqk, wl.v
    for s in rows:
        r = b * S_stream + s
        q = host_row(wl, qtid, wl.scale_q, r, H * Dqk).reshape(1, 1, H, Dqk)
        g = host_row(wl, gtid, wl.scale_gate, r, H).reshape(1, 1, H)
        ir = np.ascontiguousarray(idx[s].reshape(1, 1, -1))
        ref = oracle.sparse_attn(q, kh[b:b + 1], vh[b:b + 1], ir, g, P + s, wl.nope, wl.rope)[0, 0]
        assert_rows_close(out[s].reshape(H, Dv), ref, 2e-2, what=f"{wl.name} attn row {s}")


def dev_normal(shape, wl, tid, scale, start=0):
    t = torch.empty(*shape, dtype=torch.bfloat16, device=DEV)
    return datagen.normal_device(t, wl.seed, tid, scale, start)


def host_row(wl, tid, scale, row, width):
    """Row `row` (elements row*width ... +width) of a bf16 stream."""
    return datagen.normal_host((width,), "bf16", wl.seed, tid, scale, start=row * width)


def compact_cache(wl, positions, b, T_alloc, H, D, tid, scale):
    """[1, n, H, D] rows of cache b at the given absolute positions."""
    rows = [host_row(wl, tid, scale, b * T_alloc + int(t), H * D) for t in positions]
    return np.stack(rows).reshape(1, len(positions), H, D)


def check_attn_rows(wl, out, idx, rows, b, T_alloc, qtid=datagen.TID_Q, gtid=datagen.TID_GATE,
                    S_stream=None, ktid=datagen.TID_K, vtid=datagen.TID_V, sinks=(None, None)):
    """Compare out[b, s] for s in rows against the oracle on compact caches
    (plus the layer's attention sinks, if any)."""
    S_stream = wl.S if S_stream is None else S_stream
    H, Dqk, Dv = wl.H, wl.Dqk, wl.v
    for s in rows:
        sel = [int(t) for t in idx[s] if t >= 0]
        kc = compact_cache(wl, sel, b, T_alloc, H, Dqk, ktid, wl.scale_k)
        vc = compact_cache(wl, sel, b, T_alloc, H, Dv, vtid, wl.scale_v)
        r = b * S_stream + s
        q = host_row(wl, qtid, wl.scale_q, r, H * Dqk).reshape(1, 1, H, Dqk)
        g = host_row(wl, gtid, wl.scale_gate, r, H).reshape(1, 1, H)
        n = len(sel)
        ci = np.arange(n, dtype=np.int32).reshape(1, 1, n)
        ref = oracle.sparse_attn(q, kc, vc, ci, g, n - 1, wl.nope, wl.rope,
                                 sink_k=sinks[0], sink_v=sinks[1])[0, 0]
        assert_rows_close(out[s].reshape(H, Dv), ref, 2e-2, what=f"{wl.name} attn row {s}")


# ------------------------------------------------------------ dsa-s32k
def test_dsa_s32k_indexer_sampled_rows():
    wl = WORKLOADS["dsa-s32k"]
    S, T = wl.S, wl.T
    q_idx = dev_normal((1, S, wl.HI, wl.DI), wl, datagen.TID_QIDX, wl.scale_qidx)
    k_idx = dev_normal((1, T, wl.DI), wl, datagen.TID_KIDX, wl.scale_kidx)
    w = dev_normal((1, S, wl.HI), wl, datagen.TID_W, wl.scale_w)
    sc = torch.empty(1, S, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(q_idx, k_idx, w, sc, 0)
    rows = strat_rows(S, wl.topk, 128, seed=1)  # every 128-query tile
    got = sc[0, rows].cpu().numpy()
    del sc, q_idx, w
    _free()
    kh = datagen.normal_host((1, T, wl.DI), "bf16", wl.seed, datagen.TID_KIDX, wl.scale_kidx)
    for i, s in enumerate(rows):
        qh = host_row(wl, datagen.TID_QIDX, wl.scale_qidx, s, wl.HI * wl.DI).reshape(1, 1, wl.HI, wl.DI)
        wh = host_row(wl, datagen.TID_W, wl.scale_w, s, wl.HI).reshape(1, 1, wl.HI)
        ref = oracle.index_scores(qh, kh, wh, s)[0, 0]
        assert_rows_close(got[i], ref, 2e-2, what=f"dsa-s32k scores row {s}")


def test_dsa_s32k_fp8_indexer_sampled_rows():
    """FP8 indexer at full size: every k_idx code and the sampled rows' q codes
    bit-exact, sampled score rows against the oracle's FP8 scores."""
    wl = WORKLOADS["dsa-s32k-fp8"]
    S, T, HI, DI = wl.S, wl.T, wl.HI, wl.DI
    q_idx = dev_normal((1, S, HI, DI), wl, datagen.TID_QIDX, wl.scale_qidx)
    k_idx = dev_normal((1, T, DI), wl, datagen.TID_KIDX, wl.scale_kidx)
    w = dev_normal((1, S, HI), wl, datagen.TID_W, wl.scale_w)
    qc = torch.empty(1, S, HI, DI, dtype=torch.uint8, device=DEV)
    qs = torch.empty(1, S, HI, dtype=torch.float32, device=DEV)
    kc = torch.empty(1, T, DI, dtype=torch.uint8, device=DEV)
    ks = torch.empty(1, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_quant_fp8(q_idx, qc, qs)
    dsa.dsa_index_quant_fp8(k_idx, kc, ks)
    sc = torch.empty(1, S, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores_fp8(qc, qs, kc, ks, w, sc, 0)
    rows = strat_rows(S, wl.topk, 512, seed=2)
    got = sc[0, rows].cpu().numpy()
    got_qc, got_qs = qc[0, rows].cpu().numpy(), qs[0, rows].cpu().numpy()
    got_kc, got_ks = kc.cpu().numpy(), ks.cpu().numpy()
    del sc, q_idx, k_idx, w, qc, qs, kc, ks
    _free()
    kh = datagen.normal_host((1, T, DI), "bf16", wl.seed, datagen.TID_KIDX, wl.scale_kidx)
    rkc, rks = oracle.index_quant_fp8(kh)
    np.testing.assert_array_equal(got_kc, rkc)
    np.testing.assert_array_equal(got_ks, rks)
    for i, s in enumerate(rows):
        qh = host_row(wl, datagen.TID_QIDX, wl.scale_qidx, s, HI * DI).reshape(1, 1, HI, DI)
        wh = host_row(wl, datagen.TID_W, wl.scale_w, s, HI).reshape(1, 1, HI)
        rqc, rqs = oracle.index_quant_fp8(qh)
        np.testing.assert_array_equal(got_qc[i], rqc[0, 0])
        np.testing.assert_array_equal(got_qs[i], rqs[0, 0])
        ref = oracle.index_scores_fp8(rqc, rqs, rkc, rks, wh, s)[0, 0]
        assert_rows_close(got[i], ref, 1e-3, what=f"dsa-s32k fp8 scores row {s}")


def _topk_full(wl, S, T, P, k, mode, rows, seed_off=0, order=0):
    sc = torch.empty(1, S, T, dtype=torch.float32, device=DEV)
    datagen.scores_device(sc.view(S, T), 0, S, P, wl.seed + seed_off, mode=mode)
    idx = torch.empty(1, S, k, dtype=torch.int32, device=DEV)
    (dsa.dsa_topk_unsorted if order else dsa.dsa_topk)(sc, idx)
    got = idx[0, rows].cpu().numpy()
    del sc, idx
    _free()
    for i, s in enumerate(rows):
        ref_sc = datagen.scores_host(s, 1, S, T, P, wl.seed + seed_off, mode=mode)
        ref = oracle.topk(ref_sc, k)[0]
        g = got[i]
        if order:  # unsorted: the same set, -1 slots last
            nv = int((ref >= 0).sum())
            assert (g[nv:] == -1).all(), f"row {s}: -1 slots not last"
            g, ref = np.sort(g[:nv]), np.sort(ref[:nv])
        np.testing.assert_array_equal(g, ref, err_msg=f"row {s}")


@pytest.mark.parametrize("mode,order", [(0, 0), (2, 0), (0, 1)])
def test_dsa_s32k_topk_full_tensor(mode, order):
    wl = WORKLOADS["dsa-s32k"]
    _topk_full(wl, wl.S, wl.T, 0, wl.topk, mode, strat_rows(wl.S, wl.topk, 128, seed=2),
               order=order)


@pytest.mark.parametrize("srt", [False, True])
def test_dsa_s32k_index_topk_full_tensor(srt):
    """The fused indexer + top-k call on the whole dsa-s32k prefill: every
    row's indices equal those of dsa_index_scores + dsa_topk(_unsorted)."""
    wl = WORKLOADS["dsa-s32k"]
    S, T = wl.S, wl.T
    print(f"dsa-s32k index_topk sorted {srt}", flush=True)
    qi = dev_normal((1, S, wl.HI, wl.DI), wl, datagen.TID_QIDX, wl.scale_qidx)
    ki = dev_normal((1, T, wl.DI), wl, datagen.TID_KIDX, wl.scale_kidx)
    w = dev_normal((1, S, wl.HI), wl, datagen.TID_W, wl.scale_w)
    sc = torch.empty(1, S, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(qi, ki, w, sc, 0)
    ref = torch.empty(1, S, wl.topk, dtype=torch.int32, device=DEV)
    (dsa.dsa_topk if srt else dsa.dsa_topk_unsorted)(sc, ref)
    del sc
    got = torch.full((1, S, wl.topk), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_index_topk(qi, ki, w, got, 0, sorted=srt)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), f"{int((got != ref).sum())} slots differ"


def test_dsa_s32k_prefill_sampled_rows():
    wl = WORKLOADS["dsa-s32k"]
    S, T, H = wl.S, wl.T, wl.H
    q = dev_normal((1, S, H, wl.Dqk), wl, datagen.TID_Q, wl.scale_q)
    k = dev_normal((1, T, H, wl.Dqk), wl, datagen.TID_K, wl.scale_k)
    v = dev_normal((1, T, H, wl.v), wl, datagen.TID_V, wl.scale_v)
    g = dev_normal((1, S, H), wl, datagen.TID_GATE, wl.scale_gate)
    idx = torch.empty(1, S, wl.topk, dtype=torch.int32, device=DEV)
    datagen.indices_device(idx.view(S, wl.topk), 0, S, 0, seed=wl.seed)
    out = torch.empty(1, S, H, wl.v, dtype=torch.bfloat16, device=DEV)
    dsa.dsa_sparse_attn_prefill(q, k, v, idx, g, out, 0, wl.nope, wl.rope)
    rows = strat_rows(S, wl.topk, 128, seed=3)  # one row in every 128-query tile
    got = from_dev(out[0, rows])
    idx_h = datagen.indices_host(0, S, S, 0, wl.topk, seed=wl.seed)
    del q, k, v, g, idx, out
    _free()
    kh = host_stream(wl, (1, T, H, wl.Dqk), datagen.TID_K, wl.scale_k)
    vh = host_stream(wl, (1, T, H, wl.v), datagen.TID_V, wl.scale_v)
    check_attn_rows_full(wl, dict(zip(rows, got)), idx_h, rows, kh, vh)


# ------------------------------------------------- mla-s4k with sinks
def test_mla_s4k_pas_prefill_sampled_rows():
    wl = WORKLOADS["mla-s4k-pas"]
    S, T, H, ns = wl.S, wl.T, wl.H, wl.n_sink
    q = dev_normal((1, S, H, wl.Dqk), wl, datagen.TID_Q, wl.scale_q)
    k = dev_normal((1, T, H, wl.Dqk), wl, datagen.TID_K, wl.scale_k)
    v = dev_normal((1, T, H, wl.v), wl, datagen.TID_V, wl.scale_v)
    g = dev_normal((1, S, H), wl, datagen.TID_GATE, wl.scale_gate)
    sk = dev_normal((ns, H, wl.Dqk), wl, datagen.TID_SINK_K, wl.scale_k)
    sv = dev_normal((ns, H, wl.v), wl, datagen.TID_SINK_V, wl.scale_v)
    idx = torch.empty(1, S, wl.topk, dtype=torch.int32, device=DEV)
    datagen.indices_device(idx.view(S, wl.topk), 0, S, 0, seed=wl.seed)
    out = torch.empty(1, S, H, wl.v, dtype=torch.bfloat16, device=DEV)
    dsa.dsa_sparse_attn_prefill_pas(q, k, v, sk, sv, idx, g, out, 0, wl.nope, wl.rope)
    rows = sample_rows(S, wl.topk, n=8, seed=5)
    got = from_dev(out[0, rows])
    idx_h = datagen.indices_host(0, S, S, 0, wl.topk, seed=wl.seed)
    del q, k, v, g, idx, out, sk, sv
    _free()
    skh = datagen.normal_host((ns, H, wl.Dqk), "bf16", wl.seed, datagen.TID_SINK_K, wl.scale_k)
    svh = datagen.normal_host((ns, H, wl.v), "bf16", wl.seed, datagen.TID_SINK_V, wl.scale_v)
    check_attn_rows(wl, dict(zip(rows, got)), idx_h, rows, 0, T, sinks=(skh, svh))


# ----------------------------------------------------------- decode-b8
def test_decode_b8_full_layer():
    wl = WORKLOADS["decode-b8"]
    B, T, H, P = wl.B, wl.T, wl.H, wl.past_len
    q_idx = dev_normal((B, 1, wl.HI, wl.DI), wl, datagen.TID_QIDX, wl.scale_qidx)
    k_idx = dev_normal((B, T, wl.DI), wl, datagen.TID_KIDX, wl.scale_kidx)
    w = dev_normal((B, 1, wl.HI), wl, datagen.TID_W, wl.scale_w)
    sc = torch.empty(B, 1, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(q_idx, k_idx, w, sc, P)
    got_sc = sc.cpu().numpy()
    del q_idx, k_idx, w, sc
    _free()
    kh = datagen.normal_host((B, T, wl.DI), "bf16", wl.seed, datagen.TID_KIDX, wl.scale_kidx)
    qh = datagen.normal_host((B, 1, wl.HI, wl.DI), "bf16", wl.seed, datagen.TID_QIDX, wl.scale_qidx)
    wh = datagen.normal_host((B, 1, wl.HI), "bf16", wl.seed, datagen.TID_W, wl.scale_w)
    ref = oracle.index_scores(qh, kh, wh, P)
    assert_rows_close(got_sc, ref, 2e-2, what="decode-b8 scores")
    del kh

    # top-k on a synthetic full-size score tensor
    scs = torch.empty(B, 1, T, dtype=torch.float32, device=DEV)
    datagen.scores_device(scs.view(B, T), 0, 1, P, wl.seed, mode=1)
    idx = torch.empty(B, 1, wl.topk, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(scs, idx)
    got_i = idx.cpu().numpy()[:, 0]
    ref_i = oracle.topk(datagen.scores_host(0, B, 1, T, P, wl.seed, mode=1), wl.topk)
    np.testing.assert_array_equal(got_i, ref_i)
    del scs, idx
    _free()

    # decode attention over 8 x 131072 expanded rows with generated selections
    k = dev_normal((B, T, H, wl.Dqk), wl, datagen.TID_K, wl.scale_k)
    v = dev_normal((B, T, H, wl.v), wl, datagen.TID_V, wl.scale_v)
    q = dev_normal((B, 1, H, wl.Dqk), wl, datagen.TID_Q, wl.scale_q)
    g = dev_normal((B, 1, H), wl, datagen.TID_GATE, wl.scale_gate)
    idx = torch.empty(B, 1, wl.topk, dtype=torch.int32, device=DEV)
    datagen.indices_device(idx.view(B, wl.topk), 0, 1, P, seed=wl.seed)
    out = torch.empty(B, 1, H, wl.v, dtype=torch.bfloat16, device=DEV)
    dsa.dsa_sparse_attn_decode(q, k, v, idx, g, out, wl.nope, wl.rope)
    got = from_dev(out)
    del k, v, q, g, idx, out
    _free()
    idx_h = datagen.indices_host(0, B, 1, P, wl.topk, seed=wl.seed)
    for b in range(B):
        check_attn_rows(wl, {0: got[b, 0]}, idx_h[b:b + 1], [0], b, T, S_stream=1)


# --------------------------------------------------------- hybrid-512k
def _hybrid_rows(wl):
    return strat_rows(wl.S, wl.topk, 16, seed=7)  # one row in every 16-query indexer tile


@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_hybrid_512k_indexer_sampled_rows(part):
    """Chunk scores (4096 queries after 524 288 cached keys: the key-stationary
    schedule that pairs query tiles) on a quarter of the 256+ sampled rows per
    part (the oracle's 2.2 G multiply-adds per row are the cost), and the
    decode token's row in part 0."""
    wl = WORKLOADS["hybrid-512k"]
    S, P, T = wl.S, wl.past_len, wl.T
    Ta = T + 1
    rows = _hybrid_rows(wl)[part::4]
    k_idx = dev_normal((1, Ta, wl.DI), wl, datagen.TID_KIDX, wl.scale_kidx)
    q_idx = dev_normal((1, S + 1, wl.HI, wl.DI), wl, datagen.TID_QIDX, wl.scale_qidx)
    w = dev_normal((1, S + 1, wl.HI), wl, datagen.TID_W, wl.scale_w)
    sc = torch.empty(1, S, T, dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(q_idx[:, :S], k_idx[:, :T].contiguous(), w[:, :S], sc, P)
    got = sc[0, rows].cpu().numpy()
    del sc
    got_d = None
    if part == 0:
        scd = torch.empty(1, 1, Ta, dtype=torch.float32, device=DEV)
        dsa.dsa_index_scores(q_idx[:, S:].contiguous(), k_idx, w[:, S:].contiguous(), scd, T)
        got_d = scd[0, 0].cpu().numpy()
        del scd
    del q_idx, k_idx, w
    _free()
    kh = host_stream(wl, (1, Ta, wl.DI), datagen.TID_KIDX, wl.scale_kidx)
    for i, s in enumerate(rows + ([S] if part == 0 else [])):
        qh = host_row(wl, datagen.TID_QIDX, wl.scale_qidx, s, wl.HI * wl.DI).reshape(1, 1, wl.HI, wl.DI)
        wh = host_row(wl, datagen.TID_W, wl.scale_w, s, wl.HI).reshape(1, 1, wl.HI)
        if s < S:
            ref = oracle.index_scores(qh, kh[:, :T], wh, P + s)[0, 0]
            assert_rows_close(got[i], ref, 2e-2, what=f"hybrid chunk scores row {s}")
        else:
            ref = oracle.index_scores(qh, kh, wh, T)[0, 0]
            assert_rows_close(got_d, ref, 2e-2, what="hybrid decode scores")


def test_hybrid_512k_topk():
    """Top-k on synthetic chunk-shaped (4096 rows of up to 528 384 keys) and
    decode-shaped (one row of 528 385 keys) score tensors, sorted and unsorted."""
    wl = WORKLOADS["hybrid-512k"]
    S, P, T = wl.S, wl.past_len, wl.T
    rows = _hybrid_rows(wl)
    _topk_full(wl, S, T, P, wl.topk, 1, rows, seed_off=50)
    _topk_full(wl, 1, T + 1, T, wl.topk, 2, [0], seed_off=51)
    _topk_full(wl, S, T, P, wl.topk, 1, rows[1::4], seed_off=50, order=1)
    _topk_full(wl, 1, T + 1, T, wl.topk, 2, [0], seed_off=51, order=1)


def test_hybrid_512k_chunk_and_decode_attention():
    """DSA attention of the 4096-token chunk (the bench's launch configuration)
    on 256+ sampled rows (every 16-query tile) and of the decode token, against
    the oracle over the whole 528 385-row caches."""
    wl = WORKLOADS["hybrid-512k"]
    S, P, T, H = wl.S, wl.past_len, wl.T, wl.H
    Ta = T + 1
    rows = _hybrid_rows(wl)
    k = dev_normal((1, Ta, H, wl.Dqk), wl, datagen.TID_K, wl.scale_k)
    v = dev_normal((1, Ta, H, wl.v), wl, datagen.TID_V, wl.scale_v)
    q = dev_normal((1, S + 1, H, wl.Dqk), wl, datagen.TID_Q, wl.scale_q)
    g = dev_normal((1, S + 1, H), wl, datagen.TID_GATE, wl.scale_gate)
    idx = torch.empty(1, S + 1, wl.topk, dtype=torch.int32, device=DEV)
    datagen.indices_device(idx.view(S + 1, wl.topk), 0, S + 1, P, seed=wl.seed)
    out = torch.empty(1, S, H, wl.v, dtype=torch.bfloat16, device=DEV)
    dsa.dsa_sparse_attn_prefill(q[:, :S], k[:, :T], v[:, :T], idx[:, :S], g[:, :S], out, P,
                                wl.nope, wl.rope)
    od = torch.empty(1, 1, H, wl.v, dtype=torch.bfloat16, device=DEV)
    dsa.dsa_sparse_attn_decode(q[:, S:].contiguous(), k, v, idx[:, S:].contiguous(),
                               g[:, S:].contiguous(), od, wl.nope, wl.rope)
    got = from_dev(out[0, rows])
    got_d = from_dev(od[0, 0])
    del k, v, q, g, idx, out, od
    _free()
    idx_h = datagen.indices_host(0, S + 1, S + 1, P, wl.topk, seed=wl.seed)
    kh = host_stream(wl, (1, Ta, H, wl.Dqk), datagen.TID_K, wl.scale_k)
    vh = host_stream(wl, (1, Ta, H, wl.v), datagen.TID_V, wl.scale_v)
    check_attn_rows_full(wl, dict(zip(rows, got)), idx_h, rows, kh, vh, S_stream=0, P=P)
    check_attn_rows_full(wl, {S: got_d}, idx_h, [S], kh, vh, S_stream=0, P=P)


def test_hybrid_512k_swa_layers():
    """Both SWA layers: the chunk through the MFMA path on 256+ sampled rows
    and the decode token through the gather path, against the oracle on the
    window buffers."""
    wl = WORKLOADS["hybrid-512k"]
    S, P, H, W = wl.S, wl.past_len, wl.H, wl.window
    rows = _hybrid_rows(wl)
    for j in (1, 2):
        tid = lambda base: base + datagen.SWA_TID_STRIDE * j
        off = P - W + 1
        Tb = P + S - off
        # buffer row r = absolute position off + r; one extra row for the decode token
        kb = dev_normal((1, Tb + 1, H, wl.Dqk), wl, tid(datagen.TID_K), wl.scale_k, off * H * wl.Dqk)
        vb = dev_normal((1, Tb + 1, H, wl.v), wl, tid(datagen.TID_V), wl.scale_v, off * H * wl.v)
        q = dev_normal((1, S + 1, H, wl.Dqk), wl, tid(datagen.TID_Q), wl.scale_q)
        g = dev_normal((1, S + 1, H), wl, tid(datagen.TID_GATE), wl.scale_gate)
        out = torch.empty(1, S, H, wl.v, dtype=torch.bfloat16, device=DEV)
        dsa.swa_attn(q[:, :S], kb[:, :Tb], vb[:, :Tb], g[:, :S], out, P, off, W, wl.nope, wl.rope)
        offd = P + S - W + 1
        od = torch.empty(1, 1, H, wl.v, dtype=torch.bfloat16, device=DEV)
        dsa.swa_attn(q[:, S:].contiguous(), kb[:, offd - off:].contiguous(),
                     vb[:, offd - off:].contiguous(), g[:, S:].contiguous(), od, P + S, offd, W,
                     wl.nope, wl.rope)
        got = from_dev(out[0, rows])
        got_d = from_dev(od[0, 0])
        del kb, vb, q, g, out, od
        _free()
        kh = host_stream(wl, (1, Tb + 1, H, wl.Dqk), tid(datagen.TID_K), wl.scale_k, off * H * wl.Dqk)
        vh = host_stream(wl, (1, Tb + 1, H, wl.v), tid(datagen.TID_V), wl.scale_v, off * H * wl.v)
        for s, o in list(zip(rows, got)) + [(S, got_d)]:
            p = P + s
            qh = host_row(wl, tid(datagen.TID_Q), wl.scale_q, s, H * wl.Dqk).reshape(1, 1, H, wl.Dqk)
            gh = host_row(wl, tid(datagen.TID_GATE), wl.scale_gate, s, H).reshape(1, 1, H)
            nb = p + 1 - off  # the buffer rows up to this query's position
            ref = oracle.swa_attn(qh, kh[:, :nb], vh[:, :nb], gh, p, off, W, wl.nope, wl.rope)[0, 0]
            assert_rows_close(o.reshape(H, wl.v), ref, 2e-2, what=f"swa layer {j} row {s}")


# ----------------------------------------------------------- spark-swa
def test_spark_swa_chunk_and_decode():
    """One grouped-KV SWA layer (8 query heads over 2 KV heads, dims 256):
    the 4096-token chunk through the MFMA path and the decode token through
    the gather path, sampled rows against the oracle on the window rows."""
    wl = WORKLOADS["spark-swa"]
    S, P, H, Hkv, W = wl.S, wl.past_len, wl.H, wl.H_kv, wl.window
    Dqk, Dv = wl.Dqk, wl.v
    off = P - W + 1
    Tb = P + S - off
    kb = dev_normal((1, Tb + 1, Hkv, Dqk), wl, datagen.TID_K, wl.scale_k, off * Hkv * Dqk)
    vb = dev_normal((1, Tb + 1, Hkv, Dv), wl, datagen.TID_V, wl.scale_v, off * Hkv * Dv)
    q = dev_normal((1, S + 1, H, Dqk), wl, datagen.TID_Q, wl.scale_q)
    g = dev_normal((1, S + 1, H), wl, datagen.TID_GATE, wl.scale_gate)
    out = torch.empty(1, S, H, Dv, dtype=torch.bfloat16, device=DEV)
    dsa.swa_attn_gqa(q[:, :S], kb[:, :Tb], vb[:, :Tb], g[:, :S], out, P, off, W, wl.nope, wl.rope)
    offd = P + S - W + 1
    od = torch.empty(1, 1, H, Dv, dtype=torch.bfloat16, device=DEV)
    dsa.swa_attn_gqa(q[:, S:].contiguous(), kb[:, offd - off:].contiguous(),
                     vb[:, offd - off:].contiguous(), g[:, S:].contiguous(), od, P + S, offd, W,
                     wl.nope, wl.rope)
    rows = [0, 1, 511, 2047, S - 1]
    got = from_dev(out[0, rows])
    got_d = from_dev(od[0, 0])
    del kb, vb, q, g, out, od
    _free()
    for s, o in list(zip(rows, got)) + [(S, got_d)]:
        p = P + s
        pos = list(range(p - W + 1, p + 1))
        kc = compact_cache(wl, pos, 0, 0, Hkv, Dqk, datagen.TID_K, wl.scale_k)
        vc = compact_cache(wl, pos, 0, 0, Hkv, Dv, datagen.TID_V, wl.scale_v)
        qh = host_row(wl, datagen.TID_Q, wl.scale_q, s, H * Dqk).reshape(1, 1, H, Dqk)
        gh = host_row(wl, datagen.TID_GATE, wl.scale_gate, s, H).reshape(1, 1, H)
        ref = oracle.swa_attn_gqa(qh, kc, vc, gh, p, p - W + 1, W, wl.nope, wl.rope)[0, 0]
        assert_rows_close(o.reshape(H, Dv), ref, 2e-2, what=f"spark-swa row {s}")


# -------------------------------------------------------- prologue-s32k
@pytest.mark.parametrize("S", [32768, 8100])
def test_prologue_s32k_sampled_rows(S):
    """The indexer's projections at full size (three GEMMs + LayerNorm / RoPE in
    the benchmark's launch configuration), sampled tokens against the oracle.
    S = 8100 still takes the 256-row tiles of the wide q projection (32 row
    tiles x 64 column tiles) and ends in a ragged row tile of 164 rows."""
    wl = WORKLOADS["prologue-s32k"]
    HI, D, Q, Hd, R = wl.HI, wl.DI, wl.q_lora, wl.hidden, wl.rope_idx
    E = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=DEV)
    gen = lambda t, tid, sc: datagen.normal_device(t, wl.seed, tid, sc)
    q_lora, hidden = gen(E(1, S, Q), 20, 1.0), gen(E(1, S, Hd), 21, 1.0)
    host = lambda shape, tid, sc: datagen.normal_host(shape, "bf16", wl.seed, tid, sc)
    wts = dict(wq_b=host((HI * D, Q), 22, Q ** -0.5), wk=host((D, Hd), 23, Hd ** -0.5),
               k_norm_w=host((D,), 24, 1.0), k_norm_b=host((D,), 25, 0.1),
               weights_proj=host((HI, Hd), 26, Hd ** -0.5))
    pos = np.arange(S, dtype=np.float64)[:, None]
    ang = pos * 10000.0 ** (-2.0 * np.arange(R // 2) / R)
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    q_idx, k_cache, w = E(1, S, HI, D), E(1, S, D), E(1, S, HI)
    dsa.dsa_indexer_prologue(q_lora, hidden, *[to_dev(wts[n]) for n in (
        "wq_b", "wk", "k_norm_w", "k_norm_b", "weights_proj")], to_dev(cos), to_dev(sin),
        q_idx, k_cache, w, 0)
    rows = sample_rows(S, 2048, n=8, seed=3)
    if S % 256:
        rows = sorted(set(rows) | {S // 256 * 256, S - 2})  # first and late rows of the ragged tile
    got_q, got_k, got_w = from_dev(q_idx[0, rows]), from_dev(k_cache[0, rows]), from_dev(w[0, rows])
    del q_lora, hidden, q_idx, k_cache, w
    _free()
    for i, s in enumerate(rows):
        ql = host_row(wl, 20, 1.0, s, Q).reshape(1, 1, Q)
        hd = host_row(wl, 21, 1.0, s, Hd).reshape(1, 1, Hd)
        # one-token call at position s: the tables' row s
        rq, rk, rw = oracle.indexer_prologue(ql, hd, wts["wq_b"], wts["wk"], wts["k_norm_w"],
                                             wts["k_norm_b"], wts["weights_proj"], cos, sin, s, HI)
        assert_rows_close(got_q[i], rq[0, 0], 2e-2, what=f"prologue q_idx row {s}")
        assert_rows_close(got_k[i], rk[0, 0], 2e-2, what=f"prologue k row {s}")
        assert_rows_close(got_w[i], rw[0, 0], 2e-2, what=f"prologue w row {s}")


# ---------------------------------------------------- mla-prologue-s32k
@pytest.mark.parametrize("S", [32768, 8100])
def test_mla_prologue_s32k_sampled_rows(S):
    """The main attention's projections at full size (three GEMMs with the
    query/gate split, the latent, the rope key broadcast and expand_kv in
    their epilogues), sampled tokens against the oracle. S = 8100 ends in a
    ragged row tile."""
    wl = WORKLOADS["mla-prologue-s32k"]
    H, N, R, Dv = wl.H, wl.nope, wl.rope, wl.v
    Qr, Qc, Hd, L = wl.q_lora, wl.q_comp, wl.hidden, wl.kv_lora
    E = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=DEV)
    gen = lambda t, tid, sc: datagen.normal_device(t, wl.seed, tid, sc)
    qr, qc, hd = gen(E(1, S, Qr), 40, 1.0), gen(E(1, S, Qc), 41, 1.0), gen(E(1, S, Hd), 42, 1.0)
    host = lambda shape, tid, sc: datagen.normal_host(shape, "bf16", wl.seed, tid, sc)
    wq = host((H * (N + R + Dv), Qr + Qc), 43, (Qr + Qc) ** -0.5)
    wa = host((L + R, Hd), 44, Hd ** -0.5)
    wb = host((H * (N + Dv), L), 45, L ** -0.5)
    pos = np.arange(S, dtype=np.float64)[:, None]
    ang = pos * 10000.0 ** (-2.0 * np.arange(R // 2) / R)
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    q, g, kc, vc = E(1, S, H, N + R), E(1, S, H, Dv), E(1, S, H, N + R), E(1, S, H, Dv)
    dsa.dsa_mla_prologue(qr, qc, hd, to_dev(wq), to_dev(wa), to_dev(wb), to_dev(cos), to_dev(sin),
                         q, g, kc, vc, 0)
    rows = strat_rows(S, 2048, 512, seed=4)
    if S % 256:
        rows = sorted(set(rows) | {S // 256 * 256, S - 2})
    got = [from_dev(t[0, rows]) for t in (q, g, kc, vc)]
    del qr, qc, hd, q, g, kc, vc
    _free()
    for i, s in enumerate(rows):
        args = [host_row(wl, tid, 1.0, s, w).reshape(1, 1, w) for tid, w in ((40, Qr), (41, Qc), (42, Hd))]
        ref = oracle.mla_prologue(*args, wq, wa, wb, cos, sin, s, H, N, R, Dv)
        for name, a, r in zip(("q", "gate", "k", "v"), got, ref):
            assert_rows_close(a[i], r[0, 0], 2e-2, what=f"mla prologue {name} row {s}")
