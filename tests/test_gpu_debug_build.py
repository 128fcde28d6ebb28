"""The debug build (libdsa_debug.so: the same sources with -DDSA_DEBUG, whose
kernels also check the invariants they rely on) against the release build.

Every entry point runs once per library on the same inputs, at shapes that
reach each kernel path: the indexer's tile and rows kernels (alone and fused
with the top-k), the FP8 indexer,
the top-k's single-stage, segmented and long-row paths (sorted and
unsorted), the MFMA prefill with and without split tiles and its ping-pong
form for large grids, the row gather for
short and long-context prefill, decode with and without sinks and through the
no-alloc entry, window attention (MFMA, gather, grouped heads, sinks) and both
prologues. A failed device check makes the debug call return DSA_ERR_CHECK
(raised by the binding); outputs must be bit-identical to the release
build's."""
import numpy as np
import pytest
import torch

import datagen
import sparse_attention_11_amd as dsa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bf(shape, tid, sc=1.0, seed=11):
    return datagen.normal_device(torch.empty(*shape, dtype=torch.bfloat16, device=DEV), seed, tid, sc)


def sel(B, S, P, k, seed):
    t = torch.empty(B, S, k, dtype=torch.int32, device=DEV)
    datagen.indices_device(t.view(B * S, k), 0, S, P, seed=seed)
    return t


def nan_like(*shape, dtype=torch.bfloat16):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def both(run):
    """Outputs of run() on the release library, then on the debug library."""
    assert not dsa.dsa_debug_build()
    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    prev = dsa.use_library(dsa.DEBUG_LIB_PATH)
    try:
        assert dsa.dsa_debug_build()
        got = [t.clone() for t in run()]
        torch.cuda.synchronize()
    finally:
        dsa.use_library(prev)
    return ref, got


def same(ref, got, what):
    assert len(ref) == len(got)
    for i, (r, g) in enumerate(zip(ref, got)):
        assert torch.equal(r.view(torch.uint8) if r.dtype != torch.int32 else r,
                           g.view(torch.uint8) if g.dtype != torch.int32 else g), f"{what}: output {i}"


def test_debug_build_indexer_and_topk():
    print("indexer tile + rows paths, FP8 indexer, top-k paths", flush=True)
    qi, ki, w = bf((1, 300, 4, 64), 1), bf((1, 300, 64), 2), bf((1, 300, 4), 3, 0.5)
    qd, kd, wd = bf((2, 1, 4, 128), 4), bf((2, 5000, 128), 5), bf((2, 1, 4), 6, 0.5)
    q8, k8 = bf((1, 300, 4, 128), 7), bf((1, 300, 128), 8)  # (the FP8 indexer takes idx_dim 128)
    rows_short = torch.randn(4, 3000, generator=torch.Generator().manual_seed(1)).to(DEV)
    rows_seg = torch.randn(300, 40000, generator=torch.Generator().manual_seed(2)).to(DEV)
    rows_long = torch.randn(2, 100000, generator=torch.Generator().manual_seed(3)).to(DEV)
    rows_long[1, 500:] = float("-inf")

    def run():
        outs = []
        s1 = torch.empty(1, 300, 300, dtype=torch.float32, device=DEV)
        dsa.dsa_index_scores(qi, ki, w, s1, 0)
        s2 = torch.empty(2, 1, 5000, dtype=torch.float32, device=DEV)
        dsa.dsa_index_scores(qd, kd, wd, s2, 4999)
        outs += [s1, s2]
        qc = torch.empty(1, 300, 4, 128, dtype=torch.uint8, device=DEV)
        qs = torch.empty(1, 300, 4, dtype=torch.float32, device=DEV)
        kc = torch.empty(1, 300, 128, dtype=torch.uint8, device=DEV)
        ks = torch.empty(1, 300, dtype=torch.float32, device=DEV)
        dsa.dsa_index_quant_fp8(q8, qc, qs)
        dsa.dsa_index_quant_fp8(k8, kc, ks)
        s3 = torch.empty(1, 300, 300, dtype=torch.float32, device=DEV)
        dsa.dsa_index_scores_fp8(qc, qs, kc, ks, w, s3, 0)
        outs += [qc, qs, kc, ks, s3]
        for srt in (True, False):  # fused indexer + top-k: tile rows and decode rows
            f1 = torch.empty(1, 300, 64, dtype=torch.int32, device=DEV)
            dsa.dsa_index_topk(qi, ki, w, f1, 0, sorted=srt)
            f2 = torch.empty(2, 1, 2048, dtype=torch.int32, device=DEV)
            dsa.dsa_index_topk(qd, kd, wd, f2, 4999, sorted=srt)
            outs += [f1, f2]
        for sc, k in ((rows_short, 256), (rows_seg, 512), (rows_long, 2048)):
            for fn in (dsa.dsa_topk, dsa.dsa_topk_unsorted):
                ix = torch.empty(1, sc.shape[0], k, dtype=torch.int32, device=DEV)
                fn(sc[None], ix)
                outs.append(ix)
        return outs

    ref, got = both(run)
    same(ref, got, "indexer / top-k")


def test_debug_build_attention():
    print("prefill (MFMA, split, gather), decode (+sinks, no-alloc), window paths", flush=True)
    H, N, R, Dv = 4, 128, 64, 128
    Dqk = N + R
    q, kc, vc, g = bf((1, 300, H, Dqk), 10, Dqk ** -0.5), bf((1, 300, H, Dqk), 11), bf((1, 300, H, Dv), 12), bf((1, 300, H), 13)
    ix = sel(1, 300, 0, 64, 14)
    qs8, ix8 = bf((1, 8, H, Dqk), 15, Dqk ** -0.5), sel(1, 8, 292, 64, 16)       # S < 16: gather
    kL, vL = bf((1, 20000, 2, Dqk), 17), bf((1, 20000, 2, Dv), 18)               # long context: gather
    qL, gL, ixL = bf((1, 64, 2, Dqk), 19, Dqk ** -0.5), bf((1, 64, 2), 20), sel(1, 64, 19936, 128, 21)
    sk, sv = bf((40, H, Dqk), 22), bf((40, H, Dv), 23)
    qd, gd = bf((3, 1, H, Dqk), 24, Dqk ** -0.5), bf((3, 1, H), 25)
    kd, vd = bf((3, 6000, H, Dqk), 26), bf((3, 6000, H, Dv), 27)
    ixd = sel(3, 1, 5999, 512, 28)
    kw, vw = bf((1, 400, 2, 256), 29), bf((1, 400, 2, 256), 30)                  # grouped KV, dims 256
    # 128 heads x 8 tiles of 256 queries: the ping-pong prefill kernel, ragged
    qP, kP, vP = bf((1, 2000, 128, Dqk), 33, Dqk ** -0.5), bf((1, 2000, 128, Dqk), 34), bf((1, 2000, 128, Dv), 35)
    gP, ixP = bf((1, 2000, 128), 36), sel(1, 2000, 0, 128, 37)
    qw, gw = bf((1, 200, 8, 256), 31, 1 / 16), bf((1, 200, 8), 32)

    def run():
        outs = []
        o = nan_like(1, 300, H, Dv)
        dsa.dsa_sparse_attn_prefill(q, kc, vc, ix, g, o, 0, N, R)       # MFMA, split tiles
        o2 = nan_like(1, 8, H, Dv)
        dsa.dsa_sparse_attn_prefill(qs8, kc, vc, ix8, g[:, :8].contiguous(), o2, 292, N, R)
        o3 = nan_like(1, 64, 2, Dv)
        dsa.dsa_sparse_attn_prefill(qL, kL, vL, ixL, gL, o3, 19936, N, R)
        o4 = nan_like(1, 300, H, Dv)
        dsa.dsa_sparse_attn_prefill_pas(q, kc, vc, sk, sv, ix, g, o4, 0, N, R)
        o5 = nan_like(3, 1, H, Dv)
        dsa.dsa_sparse_attn_decode(qd, kd, vd, ixd, gd, o5, N, R)
        o6 = nan_like(3, 1, H, Dv)
        dsa.dsa_sparse_attn_decode_pas(qd, kd, vd, sk, sv, ixd, gd, o6, N, R)
        o7 = nan_like(3, 1, H, Dv)
        dsa.dsa_sparse_attn_decode_noalloc(qd, kd, vd, ixd, gd, o7, N, R)
        o8 = nan_like(1, 300, H, Dv)
        dsa.swa_attn(q, kc, vc, g, o8, 0, 0, 64, N, R)                     # window, MFMA
        o9 = nan_like(3, 1, H, Dv)
        dsa.swa_attn(qd, kd, vd, gd, o9, 5999, 0, 512, N, R)               # window decode, gather
        o10 = nan_like(1, 200, 8, 256)
        dsa.swa_attn_gqa(qw, kw, vw, gw, o10, 200, 0, 128, 192, 64)       # grouped KV heads
        o11 = nan_like(1, 300, H, Dv)
        dsa.swa_attn_pas(q, kc, vc, sk, sv, g, o11, 0, 0, 64, N, R)
        o12 = nan_like(1, 2000, 128, Dv)
        dsa.dsa_sparse_attn_prefill(qP, kP, vP, ixP, gP, o12, 0, N, R)     # ping-pong kernel
        return [o, o2, o3, o4, o5, o6, o7, o8, o9, o10, o11, o12]

    ref, got = both(run)
    same(ref, got, "attention")


def test_debug_build_prologues():
    print("indexer and MLA prologues", flush=True)
    B, S, P, T = 2, 130, 70, 203
    Q, Hd, HI, D, R = 96, 160, 5, 128, 64
    ql, hd = bf((B, S, Q), 40), bf((B, S, Hd), 41)
    wqb, wk = bf((HI * D, Q), 42, Q ** -0.5), bf((D, Hd), 43, Hd ** -0.5)
    lnw, lnb, wp = bf((D,), 44), bf((D,), 45, 0.1), bf((HI, Hd), 46, Hd ** -0.5)
    ang = np.random.default_rng(5).uniform(-np.pi, np.pi, (T, R // 2))
    cos = torch.tensor(np.cos(ang), dtype=torch.float32, device=DEV)
    sin = torch.tensor(np.sin(ang), dtype=torch.float32, device=DEV)
    Qr, Qc, L, H, N, Dv = 96, 64, 128, 5, 128, 128
    qr, qcp = bf((B, S, Qr), 47), bf((B, S, Qc), 48)
    wq = bf((H * (N + R + Dv), Qr + Qc), 49, (Qr + Qc) ** -0.5)
    wa, wb = bf((L + R, Hd), 50, Hd ** -0.5), bf((H * (N + Dv), L), 51, L ** -0.5)

    def run():
        qo, ko, wo = nan_like(B, S, HI, D), torch.full((B, T, D), 7.0, dtype=torch.bfloat16, device=DEV), nan_like(B, S, HI)
        dsa.dsa_indexer_prologue(ql, hd, wqb, wk, lnw, lnb, wp, cos, sin, qo, ko, wo, P, ln_eps=1e-6)
        q, gt = nan_like(B, S, H, N + R), nan_like(B, S, H, Dv)
        kc = torch.full((B, T, H, N + R), 7.0, dtype=torch.bfloat16, device=DEV)
        vc = torch.full((B, T, H, Dv), 7.0, dtype=torch.bfloat16, device=DEV)
        dsa.dsa_mla_prologue(qr, qcp, hd, wq, wa, wb, cos, sin, q, gt, kc, vc, P)
        return [qo, ko, wo, q, gt, kc, vc]

    ref, got = both(run)
    same(ref, got, "prologues")
