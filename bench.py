"""Benchmark of the DSA layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
inputs already resident in HBM:
  prefill workloads  indexer scores -> top-k -> sparse attention (+ gate)
  decode workloads   indexer scores (S = 1) -> top-k -> split-K decode
  hybrid-512k        DSA chunk (indexer, top-k, attention) + 2 SWA chunk
                     layers, then one decode token through the DSA layer and
                     both SWA layers
  *-pas              the same with 128 attention sinks per layer
Every stage is a C-ABI call of libdsa.so; stage times come from HIP events
recorded on the same stream the library launches on. The top-k stage is
dsa_topk_unsorted: the same selection as dsa_topk without the final sort by
score, since the attention calls take the selection as a set.

Prints ONE JSON line. `value` is prefill tokens/s of the named workload
(default dsa-s32k: a 32768-token causal prefill with 128 heads, indexer 64 x
128, top-k 2048) over whole timed steps; `decode_us_per_step` is the decode
step of the decode workload (default decode-b8: 8 sequences x 131072 cached
tokens), and `decode` holds its roofline and CPU baseline. The other
workloads are measured in the same run and reported under "also".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA layer prefill tokens/s + decode µs/step; % MFMA / HBM roofline"
PEAK_BF16 = 2.5e15
PEAK_FP8 = 5.0e15
PEAK_HBM = 8.0e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsa-s32k",
                    help="the prefill workload whose tokens/s is `value`")
    ap.add_argument("--decode-workload", default="decode-b8",
                    help="decode workload whose us/step goes in the same line ('' for none)")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--also", default="hybrid-512k,mla-s4k,mla-s4k-pas,hybrid-512k-pas,spark-swa,dsa-s32k-fp8,prologue-s32k,mla-prologue-s32k",
                    help="comma-separated extra workloads ('' for none)")
    ap.add_argument("--also-steps", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------- workloads
class Layer:
    """Device buffers and the stage list of one workload."""

    def __init__(self, wl, torch, dsa, datagen):
        self.wl, self.torch, self.dsa = wl, torch, dsa
        dev = torch.device("cuda")
        tdt = torch.bfloat16 if wl.dtype == 1 else torch.float32
        B, S, P, T = wl.B, wl.S, wl.past_len, wl.T
        H, Dqk, Dv, HI, DI, k = wl.H, wl.Dqk, wl.v, wl.HI, wl.DI, wl.topk
        self.T_alloc = T + (1 if wl.decode_after else 0)
        Ta = self.T_alloc
        E = lambda *shape: torch.empty(*shape, dtype=tdt, device=dev)
        gen = lambda t, tid, sc, start=0: datagen.normal_device(t, wl.seed, tid, sc, start)
        # caches (B rows of T_alloc tokens) and query-side tensors
        self.k = gen(E(B, Ta, H, Dqk), datagen.TID_K, wl.scale_k)
        self.v = gen(E(B, Ta, H, Dv), datagen.TID_V, wl.scale_v)
        self.k_idx = gen(E(B, Ta, DI), datagen.TID_KIDX, wl.scale_kidx)
        self.q = gen(E(B, S, H, Dqk), datagen.TID_Q, wl.scale_q)
        self.q_idx = gen(E(B, S, HI, DI), datagen.TID_QIDX, wl.scale_qidx)
        self.w = gen(E(B, S, HI), datagen.TID_W, wl.scale_w)
        self.gate = gen(E(B, S, H), datagen.TID_GATE, wl.scale_gate)
        self.scores = torch.empty(B, S, T, dtype=torch.float32, device=dev)
        if wl.idx_fp8:  # FP8 codes and row scales of q_idx and k_idx
            u8 = lambda *shape: torch.empty(*shape, dtype=torch.uint8, device=dev)
            f32 = lambda *shape: torch.empty(*shape, dtype=torch.float32, device=dev)
            self.qc, self.qs = u8(B, S, HI, DI), f32(B, S, HI)
            self.kc, self.ks = u8(B, self.T_alloc, DI), f32(B, self.T_alloc)
        self.idx = torch.empty(B, S, k, dtype=torch.int32, device=dev)
        self.out = E(B, S, H, Dv)
        ns = wl.n_sink
        if ns:  # attention sinks (one set per layer)
            self.sk = gen(E(ns, H, Dqk), datagen.TID_SINK_K, wl.scale_k)
            self.sv = gen(E(ns, H, Dv), datagen.TID_SINK_V, wl.scale_v)
        if S > 1:
            nb = dsa.dsa_sparse_attn_prefill_pas_workspace_size(B, S, T, H, Dqk, Dv, k, ns, wl.dtype)
        else:
            nb = dsa.dsa_sparse_attn_decode_pas_workspace_size(B, H, Dv, k, ns)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        self.tk_ws = torch.empty(max(dsa.dsa_topk_workspace_size(B, S, T, k), 1), dtype=torch.uint8,
                                 device=dev)
        # hybrid: decode token + SWA layers
        self.swa = []
        if wl.decode_after:
            st = S  # the decode query is row S of the query streams
            self.qd = gen(E(B, 1, H, Dqk), datagen.TID_Q, wl.scale_q, st * H * Dqk)
            self.qd_idx = gen(E(B, 1, HI, DI), datagen.TID_QIDX, wl.scale_qidx, st * HI * DI)
            self.wd = gen(E(B, 1, HI), datagen.TID_W, wl.scale_w, st * HI)
            self.gd = gen(E(B, 1, H), datagen.TID_GATE, wl.scale_gate, st * H)
            self.sd = torch.empty(B, 1, T + 1, dtype=torch.float32, device=dev)
            self.idd = torch.empty(B, 1, k, dtype=torch.int32, device=dev)
            self.od = E(B, 1, H, Dv)
            self.wsd = torch.empty(dsa.dsa_sparse_attn_decode_pas_workspace_size(B, H, Dv, k, ns),
                                   dtype=torch.uint8, device=dev)
            self.tk_wsd = torch.empty(max(dsa.dsa_topk_workspace_size(B, 1, T + 1, k), 1),
                                      dtype=torch.uint8, device=dev)
            W = wl.window
            for j in range(1, wl.n_swa + 1):
                off = max(0, P - W + 1)
                Tb = P + S - off
                offd = max(0, P + S - W + 1)
                Tbd = P + S + 1 - offd
                tid = lambda base: base + datagen.SWA_TID_STRIDE * j
                lay = {
                    # buffer row r = absolute position off + r (B = 1 in this workload)
                    "k": gen(E(B, Tb + 1, H, Dqk), tid(datagen.TID_K), wl.scale_k, off * H * Dqk),
                    "v": gen(E(B, Tb + 1, H, Dv), tid(datagen.TID_V), wl.scale_v, off * H * Dv),
                    "q": gen(E(B, S, H, Dqk), tid(datagen.TID_Q), wl.scale_q),
                    "g": gen(E(B, S, H), tid(datagen.TID_GATE), wl.scale_gate),
                    "qd": gen(E(B, 1, H, Dqk), tid(datagen.TID_Q), wl.scale_q, S * H * Dqk),
                    "gd": gen(E(B, 1, H), tid(datagen.TID_GATE), wl.scale_gate, S * H),
                    "o": E(B, S, H, Dv), "od": E(B, 1, H, Dv),
                    "off": off, "Tb": Tb, "offd": offd, "Tbd": Tbd,
                }
                if ns:
                    lay["sk"] = gen(E(ns, H, Dqk), tid(datagen.TID_SINK_K), wl.scale_k)
                    lay["sv"] = gen(E(ns, H, Dv), tid(datagen.TID_SINK_V), wl.scale_v)
                nbw = dsa.swa_attn_pas_workspace_size(B, S, H, Dqk, Dv, W, ns, wl.dtype)
                lay["ws"] = torch.empty(max(nbw, 1), dtype=torch.uint8, device=dev)
                lay["wsd"] = torch.empty(
                    max(dsa.swa_attn_pas_workspace_size(B, 1, H, Dqk, Dv, W, ns, wl.dtype), 1),
                    dtype=torch.uint8, device=dev)
                self.swa.append(lay)
        torch.cuda.synchronize()

    # attention calls with or without the layer's sinks
    def _prefill(self, q, k, v, idx, g, o, P, ws):
        if self.wl.n_sink:
            return self.dsa.dsa_sparse_attn_prefill_pas(q, k, v, self.sk, self.sv, idx, g, o, P,
                                                        self.wl.nope, self.wl.rope, workspace=ws)
        return self.dsa.dsa_sparse_attn_prefill(q, k, v, idx, g, o, P, self.wl.nope, self.wl.rope,
                                                workspace=ws)

    def _decode(self, q, k, v, idx, g, o, ws):
        if self.wl.n_sink:
            return self.dsa.dsa_sparse_attn_decode_pas(q, k, v, self.sk, self.sv, idx, g, o,
                                                       self.wl.nope, self.wl.rope, workspace=ws)
        return self.dsa.dsa_sparse_attn_decode(q, k, v, idx, g, o, self.wl.nope, self.wl.rope,
                                               workspace=ws)

    def _swa(self, L, q, k, v, g, o, P, off, ws):
        wl = self.wl
        if wl.n_sink:
            return self.dsa.swa_attn_pas(q, k, v, L["sk"], L["sv"], g, o, P, off, wl.window,
                                         wl.nope, wl.rope, workspace=ws)
        return self.dsa.swa_attn(q, k, v, g, o, P, off, wl.window, wl.nope, wl.rope, workspace=ws)

    # each stage: (name, callable)
    def stages(self):
        wl, dsa = self.wl, self.dsa
        P, S = wl.past_len, wl.S
        if wl.idx_fp8:
            # the step quantises q_idx and the k_idx rows this chunk appended
            # (all of them in a prefill from position 0)
            kn = lambda t: t[:, P: wl.T]
            st = [
                ("K1q quant_fp8 q_idx", lambda: dsa.dsa_index_quant_fp8(self.q_idx, self.qc, self.qs)),
                ("K1k quant_fp8 k_idx", lambda: dsa.dsa_index_quant_fp8(
                    kn(self.k_idx), kn(self.kc), kn(self.ks))),
                ("K1 index_scores", lambda: dsa.dsa_index_scores_fp8(
                    self.qc, self.qs, self.kc[:, : wl.T], self.ks[:, : wl.T], self.w, self.scores, P)),
            ]
        else:
            st = [("K1 index_scores", lambda: dsa.dsa_index_scores(
                self.q_idx, self.k_idx[:, : wl.T] if wl.B == 1 else self.k_idx, self.w, self.scores, P))]
        st.append(("K2 topk", lambda: dsa.dsa_topk_unsorted(self.scores, self.idx, self.tk_ws)))
        kc = self.k if self.T_alloc == wl.T else self.k[:, : wl.T]
        vc = self.v if self.T_alloc == wl.T else self.v[:, : wl.T]
        if S > 1:
            st.append(("K3 sparse_attn_prefill", lambda: self._prefill(
                self.q, kc, vc, self.idx, self.gate, self.out, P, self.ws)))
        else:
            st.append(("K4 sparse_attn_decode", lambda: self._decode(
                self.q, kc, vc, self.idx, self.gate, self.out, self.ws)))
        for j, L in enumerate(self.swa):
            st.append((f"K5 swa_attn chunk L{j + 1}", lambda L=L: self._swa(
                L, L["q"], L["k"][:, : L["Tb"]], L["v"][:, : L["Tb"]], L["g"], L["o"], P, L["off"],
                L["ws"])))
        if wl.decode_after:
            Td = wl.T + 1
            st += [
                ("D K1 index_scores", lambda: dsa.dsa_index_scores(self.qd_idx, self.k_idx, self.wd, self.sd, Td - 1)),
                ("D K2 topk", lambda: dsa.dsa_topk_unsorted(self.sd, self.idd, self.tk_wsd)),
                ("D K4 sparse_attn_decode", lambda: self._decode(
                    self.qd, self.k, self.v, self.idd, self.gd, self.od, self.wsd)),
            ]
            for j, L in enumerate(self.swa):
                st.append((f"D K5 swa_attn L{j + 1}", lambda L=L: self._swa(
                    L, L["qd"], L["k"][:, L["offd"] - L["off"]:L["offd"] - L["off"] + L["Tbd"]],
                    L["v"][:, L["offd"] - L["off"]:L["offd"] - L["off"] + L["Tbd"]], L["gd"],
                    L["od"], Td - 1, L["offd"], L["wsd"])))
        return st


class SwaLayer:
    """One sliding-window layer with grouped KV heads: a chunk of S tokens
    after past_len cached ones, then one decode token. The K/V buffers hold
    the window suffix only (row r = absolute position off + r)."""

    def __init__(self, wl, torch, dsa, datagen):
        self.wl, self.dsa = wl, dsa
        dev = torch.device("cuda")
        B, S, P, W = wl.B, wl.S, wl.past_len, wl.window
        H, Hkv, Dqk, Dv = wl.H, wl.H_kv or wl.H, wl.Dqk, wl.v
        E = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=dev)
        gen = lambda t, tid, sc, start=0: datagen.normal_device(t, wl.seed, tid, sc, start)
        self.off = max(0, P - W + 1)
        self.Tb = P + S - self.off
        self.offd = max(0, P + S - W + 1)
        self.Tbd = P + S + 1 - self.offd
        self.k = gen(E(B, self.Tb + 1, Hkv, Dqk), datagen.TID_K, wl.scale_k, self.off * Hkv * Dqk)
        self.v = gen(E(B, self.Tb + 1, Hkv, Dv), datagen.TID_V, wl.scale_v, self.off * Hkv * Dv)
        self.q = gen(E(B, S + 1, H, Dqk), datagen.TID_Q, wl.scale_q)
        self.g = gen(E(B, S + 1, H), datagen.TID_GATE, wl.scale_gate)
        self.qc, self.gc = self.q[:, :S], self.g[:, :S]
        self.qd, self.gd = self.q[:, S:].contiguous(), self.g[:, S:].contiguous()
        self.kc, self.vc = self.k[:, : self.Tb], self.v[:, : self.Tb]
        d0 = self.offd - self.off
        self.kd = self.k[:, d0:d0 + self.Tbd].contiguous()
        self.vd = self.v[:, d0:d0 + self.Tbd].contiguous()
        self.o, self.od = E(B, S, H, Dv), E(B, 1, H, Dv)
        ws = lambda s_: torch.empty(max(dsa.swa_attn_gqa_workspace_size(B, s_, H, Dqk, Dv, W, 1), 1),
                                    dtype=torch.uint8, device=dev)
        self.ws, self.wsd = ws(S), ws(1)
        torch.cuda.synchronize()

    def stages(self):
        wl, dsa = self.wl, self.dsa
        P, S, W = wl.past_len, wl.S, wl.window
        return [
            ("K5 swa_attn chunk", lambda: dsa.swa_attn_gqa(
                self.qc, self.kc, self.vc, self.gc, self.o, P, self.off, W, wl.nope, wl.rope,
                workspace=self.ws)),
            ("D K5 swa_attn", lambda: dsa.swa_attn_gqa(
                self.qd, self.kd, self.vd, self.gd, self.od, P + S, self.offd, W, wl.nope,
                wl.rope, workspace=self.wsd)),
        ]


class PrologueLayer:
    """The indexer's projections for S tokens (one stage)."""

    def __init__(self, wl, torch, dsa, datagen):
        self.wl, self.dsa = wl, dsa
        dev = torch.device("cuda")
        B, S, P, HI, D, Q, Hd, R = wl.B, wl.S, wl.past_len, wl.HI, wl.DI, wl.q_lora, wl.hidden, wl.rope_idx
        E = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=dev)
        gen = lambda t, tid, sc: datagen.normal_device(t, wl.seed, tid, sc)
        self.q_lora, self.hidden = gen(E(B, S, Q), 20, 1.0), gen(E(B, S, Hd), 21, 1.0)
        self.wq_b, self.wk = gen(E(HI * D, Q), 22, Q ** -0.5), gen(E(D, Hd), 23, Hd ** -0.5)
        self.knw, self.knb = gen(E(D), 24, 1.0), gen(E(D), 25, 0.1)
        self.wp = gen(E(HI, Hd), 26, Hd ** -0.5)
        pos = torch.arange(P + S, device=dev, dtype=torch.float64)[:, None]
        freq = 10000.0 ** (-2.0 * torch.arange(R // 2, device=dev, dtype=torch.float64) / R)
        self.cos, self.sin = torch.cos(pos * freq).float(), torch.sin(pos * freq).float()
        self.q_idx, self.k_cache, self.w = E(B, S, HI, D), E(B, P + S, D), E(B, S, HI)
        self.ws = torch.empty(dsa.dsa_indexer_prologue_workspace_size(B, S, D), dtype=torch.uint8,
                              device=dev)
        torch.cuda.synchronize()

    def stages(self):
        return [("K0 indexer_prologue", lambda: self.dsa.dsa_indexer_prologue(
            self.q_lora, self.hidden, self.wq_b, self.wk, self.knw, self.knb, self.wp, self.cos,
            self.sin, self.q_idx, self.k_cache, self.w, self.wl.past_len, workspace=self.ws))]


class MlaPrologueLayer:
    """The main attention's projections for S tokens (one stage)."""

    def __init__(self, wl, torch, dsa, datagen):
        self.wl, self.dsa = wl, dsa
        dev = torch.device("cuda")
        B, S, P, H = wl.B, wl.S, wl.past_len, wl.H
        Qr, Qc, Hd, L, N, R, Dv = wl.q_lora, wl.q_comp, wl.hidden, wl.kv_lora, wl.nope, wl.rope, wl.v
        E = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=dev)
        gen = lambda t, tid, sc: datagen.normal_device(t, wl.seed, tid, sc)
        self.qr, self.qc, self.hd = gen(E(B, S, Qr), 40, 1.0), gen(E(B, S, Qc), 41, 1.0), gen(E(B, S, Hd), 42, 1.0)
        self.wq = gen(E(H * (N + R + Dv), Qr + Qc), 43, (Qr + Qc) ** -0.5)
        self.wa = gen(E(L + R, Hd), 44, Hd ** -0.5)
        self.wb = gen(E(H * (N + Dv), L), 45, L ** -0.5)
        pos = torch.arange(P + S, device=dev, dtype=torch.float64)[:, None]
        freq = 10000.0 ** (-2.0 * torch.arange(R // 2, device=dev, dtype=torch.float64) / R)
        self.cos, self.sin = torch.cos(pos * freq).float(), torch.sin(pos * freq).float()
        self.q, self.g = E(B, S, H, N + R), E(B, S, H, Dv)
        self.kc, self.vc = E(B, P + S, H, N + R), E(B, P + S, H, Dv)
        self.ws = torch.empty(dsa.dsa_mla_prologue_workspace_size(B, S, L), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def stages(self):
        return [("K0m mla_prologue", lambda: self.dsa.dsa_mla_prologue(
            self.qr, self.qc, self.hd, self.wq, self.wa, self.wb, self.cos, self.sin, self.q,
            self.g, self.kc, self.vc, self.wl.past_len, workspace=self.ws))]


def mla_prologue_flops(wl):
    M, H, N, R, Dv = wl.B * wl.S, wl.H, wl.nope, wl.rope, wl.v
    return 2.0 * M * ((wl.q_lora + wl.q_comp) * H * (N + R + Dv) + wl.hidden * (wl.kv_lora + R)
                      + wl.kv_lora * H * (N + Dv))


def make_layer(wl, torch, dsa, datagen):
    if wl.mla_prologue_only:
        return MlaPrologueLayer(wl, torch, dsa, datagen)
    if wl.prologue_only:
        return PrologueLayer(wl, torch, dsa, datagen)
    return (SwaLayer if wl.swa_only else Layer)(wl, torch, dsa, datagen)


def contiguous_view(t):
    return t if t.is_contiguous() else t.contiguous()


def time_layer(layer, steps, warmup, torch):
    """Whole steps are timed with one pair of HIP events around `steps` back-to-
    back steps (nothing else in the stream); the per-stage breakdown comes from
    a second pass with events around every call, which adds its own small
    event overhead and is reported separately."""
    stages = layer.stages()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for s in range(steps):
        for _, fn in stages:
            fn()
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_all0.elapsed_time(t_all1) / steps
    # per-stage pass
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in stages] for _ in range(steps)]
    for s in range(steps):
        for (name, fn), (a, b) in zip(stages, ev[s]):
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    per_stage = {}
    for i, (name, _) in enumerate(stages):
        ts = [ev[s][i][0].elapsed_time(ev[s][i][1]) * 1e3 for s in range(steps)]
        per_stage[name] = {"mean_us": float(np.mean(ts)), "min_us": float(np.min(ts)),
                           "median_us": float(np.median(ts))}
    return per_stage, total_ms, wall


def time_sorted_topk(layer, reps, torch):
    """Mean time of the sorted top-k (dsa_topk) on the layer's own indexer
    scores. The pipeline's K2 stage is dsa_topk_unsorted (the attention takes
    index lists as sets); this reports the sorted call beside it, outside the
    step."""
    fn = lambda: layer.dsa.dsa_topk(layer.scores, layer.idx, layer.tk_ws)
    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def time_graph(stages, steps, torch):
    """Mean time of one replay of the stages captured in a HIP graph (kernels
    only: the library's calls enqueue kernels and nothing else)."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for _, fn in stages:
            fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for _, fn in stages:
                fn()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


# ------------------------------------------------------ algorithmic work
def work(wl):
    """Algorithmic flops / bytes per stage (the dense work DSA avoids is not counted)."""
    B, S, P, T, k = wl.B, wl.S, wl.past_len, wl.T, wl.topk
    esz = 2 if wl.dtype == 1 else 4
    pos = P + np.arange(S, dtype=np.float64)
    vis = float(B * np.sum(pos + 1))                 # visible (s, t) pairs
    sel = float(B * np.sum(np.minimum(k, pos + 1)))  # selected pairs
    sink = float(B * S * wl.n_sink)                  # (query, sink) pairs
    out = {
        "K1": {"flops": 2.0 * wl.HI * wl.DI * vis,
               "bytes": esz * (B * S * wl.HI * wl.DI + B * T * wl.DI + B * S * wl.HI) + 4.0 * B * S * T},
        "K2": {"bytes": 4.0 * B * S * T + 4.0 * B * S * k},
        "attn": {"flops": 2.0 * wl.H * (wl.Dqk + wl.v) * (sel + sink),
                 "dense_flops": 2.0 * wl.H * (wl.Dqk + wl.v) * (vis + sink),
                 "bytes_once": esz * (B * T * wl.H * (wl.Dqk + wl.v) + B * S * wl.H * (wl.Dqk + 2 * wl.v)),
                 "bytes_gather": esz * (sel + sink) * wl.H * (wl.Dqk + wl.v)},
    }
    if wl.decode_after:
        Td = T + 1
        out["D"] = {"K1_bytes": esz * (B * Td * wl.DI) + 4.0 * B * Td,
                    "K4_bytes": esz * B * (k + wl.n_sink) * wl.H * (wl.Dqk + wl.v),
                    "K4_flops": 2.0 * wl.H * (wl.Dqk + wl.v) * B * (k + wl.n_sink)}
    if wl.n_swa:
        W = wl.window
        win = float(B * np.sum(np.minimum(W, pos + 1)))
        hkv = wl.H_kv or wl.H
        out["K5"] = {"flops": 2.0 * wl.H * (wl.Dqk + wl.v) * (win + sink),
                     # decode token: its window's K/V rows once, plus q and out
                     "decode_bytes": esz * B * (min(W, T + 1) * hkv * (wl.Dqk + wl.v)
                                                + wl.H * (wl.Dqk + wl.v))}
    return out


def summarize(wl, per_stage, total_ms):
    w = work(wl)
    g = lambda name: per_stage[name]["mean_us"] * 1e-6
    r = {"workload": wl.name, "ms_per_step": total_ms,
         "stages_us": {k: round(v["mean_us"], 2) for k, v in per_stage.items()}}
    if wl.mla_prologue_only:  # the main attention's projections: three GEMMs, fused epilogues
        t0 = g("K0m mla_prologue")
        fl = mla_prologue_flops(wl)
        r["prefill_tokens_per_s"] = wl.B * wl.S / t0
        r["K0m_mfma_frac"] = fl / t0 / PEAK_BF16
        r["K0m_tflops"] = fl / t0 / 1e12
        return r
    if wl.prologue_only:  # the indexer's projections: three GEMMs + LayerNorm / RoPE
        t0 = g("K0 indexer_prologue")
        M = wl.B * wl.S
        fl = 2.0 * M * (wl.q_lora * wl.HI * wl.DI + wl.hidden * wl.DI + wl.hidden * wl.HI)
        r["prefill_tokens_per_s"] = M / t0
        r["K0_mfma_frac"] = fl / t0 / PEAK_BF16
        r["K0_tflops"] = fl / t0 / 1e12
        return r
    if wl.swa_only:  # one grouped-KV SWA layer: chunk and decode token
        t5, t5d = g("K5 swa_attn chunk"), g("D K5 swa_attn")
        r["prefill_tokens_per_s"] = wl.B * wl.S / t5
        r["K5_mfma_frac"] = w["K5"]["flops"] / t5 / PEAK_BF16
        r["decode_us_per_step"] = t5d * 1e6
        r["D_K5_hbm_frac"] = w["K5"]["decode_bytes"] / t5d / PEAK_HBM
        return r
    t1, t2 = g("K1 index_scores"), g("K2 topk")
    r["K1_mfma_frac"] = w["K1"]["flops"] / t1 / (PEAK_FP8 if wl.idx_fp8 else PEAK_BF16)
    if wl.idx_fp8:
        r["K1_peak"] = "fp8 5.0 PFLOP/s"
        r["K1_with_quant_us"] = (t1 + g("K1q quant_fp8 q_idx") + g("K1k quant_fp8 k_idx")) * 1e6
    r["K1_tflops"] = w["K1"]["flops"] / t1 / 1e12
    r["K2_hbm_frac"] = w["K2"]["bytes"] / t2 / PEAK_HBM
    if wl.S > 1:
        t3 = g("K3 sparse_attn_prefill")
        r["K3_useful_mfma_frac"] = w["attn"]["flops"] / t3 / PEAK_BF16
        r["K3_issued_mfma_frac"] = w["attn"]["dense_flops"] / t3 / PEAK_BF16
        pre = sum(v["mean_us"] for k_, v in per_stage.items() if not k_.startswith("D ")) * 1e-6
        r["prefill_tokens_per_s"] = wl.B * wl.S / pre  # sum of the prefill stages' times
        r["prefill_us"] = pre * 1e6
        if not wl.decode_after:  # whole timed step, launch gaps included
            r["step_tokens_per_s"] = wl.B * wl.S / (total_ms * 1e-3)
    else:
        t4 = g("K4 sparse_attn_decode")
        r["decode_us_per_step"] = total_ms * 1e3
        r["K4_hbm_frac"] = w["attn"]["bytes_gather"] / t4 / PEAK_HBM
        r["K4_GBps"] = w["attn"]["bytes_gather"] / t4 / 1e9
        r["K1_hbm_frac"] = w["K1"]["bytes"] / t1 / PEAK_HBM
    if wl.decode_after:
        dec = sum(v["mean_us"] for k_, v in per_stage.items() if k_.startswith("D ")) * 1e-6
        r["decode_us_per_step"] = dec * 1e6
        r["D_K4_hbm_frac"] = w["D"]["K4_bytes"] / g("D K4 sparse_attn_decode") / PEAK_HBM
    return r


# --------------------------------------------------- counted HBM traffic
def counted_traffic(wl_name):
    """HBM bytes per launch of the dominant stage from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (copy-calibrated), or None when
    there is none or the kernel source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm-bytes_{wl_name}.json")
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    rec = json.load(open(path))
    src = os.path.join(ROOT, rec["kernel_source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest() if os.path.exists(src) else ""
    if sha != rec["kernel_source_sha256"]:
        return None, f"counters in {os.path.relpath(path, ROOT)} predate the current {rec['kernel_source']}"
    return rec["traffic_bytes_per_launch"], os.path.relpath(path, ROOT)


# ------------------------------------------------------------ CPU baseline
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _bitrev_order(n):
    bits = max(1, int(math.log2(n)))
    return [int(format(i, f"0{bits}b")[::-1], 2) for i in range(n)]


def cpu_prefill_baseline(wl, budget_s, threads=0, nblk=64, block=8):
    """The fp64 oracle (as it stands) on a bounded sample of the workload's
    query rows, on this host's cores: indexer -> top-k -> sparse attention +
    gate for blocks of `block` consecutive query rows, the blocks taken from an
    `nblk`-block grid over the sequence in bit-reversed order (any prefix mixes
    short and long causal contexts). Every input is generated before the timed
    region; blocks run until the time budget is spent."""
    import datagen
    import oracle

    oracle.build(force=False)
    S, P, T = wl.S, wl.past_len, wl.T
    dt = wl.dtype_name
    g = lambda shape, tid, sc, start=0: datagen.normal_host(shape, dt, wl.seed, tid, sc, start)
    k_idx = g((1, T, wl.DI), datagen.TID_KIDX, wl.scale_kidx)
    kc = g((1, T, wl.H, wl.Dqk), datagen.TID_K, wl.scale_k)
    vc = g((1, T, wl.H, wl.v), datagen.TID_V, wl.scale_v)
    whole = S <= nblk * block // 2  # short prefills: the whole layer per pass, repeated
    if whole:
        starts = [0]
        block = S
    else:
        grid = np.linspace(0, S - block, nblk).astype(int)
        starts = [int(grid[o]) for o in _bitrev_order(nblk)]
    inp = []
    for s0 in starts:
        n = min(block, S - s0)
        inp.append((s0, n,
                    g((1, n, wl.HI, wl.DI), datagen.TID_QIDX, wl.scale_qidx, s0 * wl.HI * wl.DI),
                    g((1, n, wl.HI), datagen.TID_W, wl.scale_w, s0 * wl.HI),
                    g((1, n, wl.H, wl.Dqk), datagen.TID_Q, wl.scale_q, s0 * wl.H * wl.Dqk),
                    g((1, n, wl.H), datagen.TID_GATE, wl.scale_gate, s0 * wl.H)))
    full = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    used = oracle.num_threads()
    rows, done = 0, 0
    t0 = time.perf_counter()
    while True:
        for s0, n, q_idx, w, q, gate in inp:
            Tn = P + s0 + n
            sc = oracle.index_scores(q_idx, k_idx[:, :Tn], w, P + s0)
            idx = oracle.topk(sc.astype(np.float32), wl.topk)
            oracle.sparse_attn(q, kc[:, :Tn], vc[:, :Tn], idx, gate, P + s0, wl.nope, wl.rope)
            rows += n
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if not whole or time.perf_counter() - t0 > min(budget_s, 2.0):
            break
    el = time.perf_counter() - t0
    oracle.set_num_threads(full)
    what = (f"the whole {S}-token prefill, {done} passes" if whole else
            f"{done} blocks of {block} consecutive rows spread over the {S}-token prefill")
    return {"value": rows / el, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{rows} query rows of {wl.name} ({what}, B=1): indexer + top-k + sparse "
                      f"attention + gate in fp64, {el:.1f} s; inputs generated before timing"}


def cpu_decode_baseline(wl, reps=3):
    """The oracle's decode step for one of the B sequences (indexer over its
    T cached keys -> top-k -> sparse attention + gate), times B: the B
    sequences are independent and alike, and their expanded caches (tens of
    GB) need not be generated on the host. Attention runs on the sequence's
    selected cache rows (the rows of its top-k, generated before timing;
    attention depends only on the selected set, so this is the same result)."""
    import datagen
    import oracle

    oracle.build(force=False)
    T, P, k = wl.T, wl.past_len, wl.topk
    dt = wl.dtype_name
    b = 0
    g = lambda shape, tid, sc, start=0: datagen.normal_host(shape, dt, wl.seed, tid, sc, start)
    k_idx = g((1, T, wl.DI), datagen.TID_KIDX, wl.scale_kidx, b * T * wl.DI)
    q_idx = g((1, 1, wl.HI, wl.DI), datagen.TID_QIDX, wl.scale_qidx, b * wl.HI * wl.DI)
    w = g((1, 1, wl.HI), datagen.TID_W, wl.scale_w, b * wl.HI)
    q = g((1, 1, wl.H, wl.Dqk), datagen.TID_Q, wl.scale_q, b * wl.H * wl.Dqk)
    gate = g((1, 1, wl.H), datagen.TID_GATE, wl.scale_gate, b * wl.H)
    idx = oracle.topk(oracle.index_scores(q_idx, k_idx, w, P).astype(np.float32), k)[0, 0]
    sel = [int(t) for t in idx if t >= 0]
    row = lambda tid, sc, t, D: g((wl.H * D,), tid, sc, (b * T + t) * wl.H * D)
    kc = np.stack([row(datagen.TID_K, wl.scale_k, t, wl.Dqk) for t in sel]).reshape(1, len(sel), wl.H, wl.Dqk)
    vc = np.stack([row(datagen.TID_V, wl.scale_v, t, wl.v) for t in sel]).reshape(1, len(sel), wl.H, wl.v)
    ci = np.arange(len(sel), dtype=np.int32).reshape(1, 1, -1)
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        sc = oracle.index_scores(q_idx, k_idx, w, P)
        got = oracle.topk(sc.astype(np.float32), k)
        oracle.sparse_attn(q, kc, vc, ci, gate, len(sel) - 1, wl.nope, wl.rope)
        ts.append(time.perf_counter() - t0)
        assert np.array_equal(got[0, 0], idx)
    one = float(np.median(ts))
    return {"value": one * wl.B * 1e6, "unit": "us/step", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"sequence 0 of {wl.B} ({T} cached keys, top-{k}): indexer + top-k + sparse "
                      f"attention + gate in fp64, median of {reps} runs {one * 1e3:.1f} ms, times "
                      f"{wl.B} sequences; its selected cache rows generated before timing"}


def headline_roofline(wl, per_stage):
    """The roofline object of the main workload's dominant stage (K3, or the
    stage a single-stage workload runs) from its mean stage time."""
    w = work(wl)
    t3 = (per_stage["K3 sparse_attn_prefill"]["mean_us"] * 1e-6
          if wl.S > 1 and not (wl.swa_only or wl.prologue_only or wl.mla_prologue_only) else None)
    if wl.mla_prologue_only:
        t0 = per_stage["K0m mla_prologue"]["mean_us"] * 1e-6
        fl = mla_prologue_flops(wl)
        roof = {"kernel": "K0m mla_prologue (three bf16 GEMMs with scattering epilogues)",
                "bound": "mfma", "achieved": fl / t0 / 1e12, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": fl / t0 / PEAK_BF16, "traffic": None,
                "algorithmic_flops_per_launch": fl, "mean_launch_us": t0 * 1e6}
    elif wl.prologue_only:
        t0 = per_stage["K0 indexer_prologue"]["mean_us"] * 1e-6
        M = wl.B * wl.S
        fl = 2.0 * M * (wl.q_lora * wl.HI * wl.DI + wl.hidden * wl.DI + wl.hidden * wl.HI)
        roof = {"kernel": "K0 indexer_prologue (bf16 GEMMs + LayerNorm / RoPE)", "bound": "mfma",
                "achieved": fl / t0 / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": fl / t0 / PEAK_BF16, "traffic": None, "algorithmic_flops_per_launch": fl,
                "mean_launch_us": t0 * 1e6}
    elif wl.swa_only:
        t5 = per_stage["K5 swa_attn chunk"]["mean_us"] * 1e-6
        ach = w["K5"]["flops"] / t5 / 1e12
        roof = {"kernel": "K5 swa_attn_gqa chunk (MFMA flash, window mask)", "bound": "mfma",
                "achieved": ach, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": ach * 1e12 / PEAK_BF16, "traffic": None,
                "algorithmic_flops_per_launch": w["K5"]["flops"], "mean_launch_us": t5 * 1e6}
    elif t3 is not None:
        ach = w["attn"]["flops"] / t3 / 1e12
        roof = {"kernel": "K3 sparse_attn_prefill (selection bitmap + dense-masked MFMA flash)",
                "bound": "mfma", "achieved": ach, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": ach * 1e12 / PEAK_BF16, "traffic": None,
                "algorithmic_flops_per_launch": w["attn"]["flops"],
                "issued_dense_flops_per_launch": w["attn"]["dense_flops"],
                "issued_frac": w["attn"]["dense_flops"] / t3 / PEAK_BF16,
                "mean_launch_us": t3 * 1e6}
    else:
        t4 = per_stage["K4 sparse_attn_decode"]["mean_us"] * 1e-6
        ach = w["attn"]["bytes_gather"] / t4 / 1e9
        roof = {"kernel": "K4 sparse_attn_decode", "bound": "hbm", "achieved": ach,
                "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": ach * 1e9 / PEAK_HBM,
                "traffic": None, "mean_launch_us": t4 * 1e6}
    roof["traffic"], roof["traffic_source"] = counted_traffic(wl.name)
    return roof


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by query rows / key ranges, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import datagen
    import sparse_attention_11_amd as dsa
    from datagen.configs import WORKLOADS

    dsa.lib()
    torch.cuda.init()
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log = lambda msg: print(f"# {msg}", file=sys.stderr, flush=True)

    # ---- prefill headline
    wl = WORKLOADS[args.workload]
    layer = make_layer(wl, torch, dsa, datagen)
    per_stage, total_ms, wall = time_layer(layer, args.steps, args.warmup, torch)
    main_r = summarize(wl, per_stage, total_ms)
    if "K2 topk" in per_stage:  # the sorted call, after the timed steps
        main_r["K2_sorted_topk_us"] = time_sorted_topk(layer, 5, torch)
    del layer
    torch.cuda.empty_cache()
    log(f"{wl.name}: {total_ms:.3f} ms/step")

    # ---- decode in the same line
    dec = None
    if args.decode_workload:
        dwl = WORKLOADS[args.decode_workload]
        dlay = make_layer(dwl, torch, dsa, datagen)
        dps, dtm, _ = time_layer(dlay, args.decode_steps, args.warmup, torch)
        dec_r = summarize(dwl, dps, dtm)
        dec_r["K2_sorted_topk_us"] = time_sorted_topk(dlay, 20, torch)
        dgraph = time_graph(dlay.stages(), args.decode_steps, torch)
        del dlay
        torch.cuda.empty_cache()
        log(f"{dwl.name}: {dtm * 1e3:.1f} us/step")
        dw = work(dwl)
        t4 = dps["K4 sparse_attn_decode"]["mean_us"] * 1e-6
        ach = dw["attn"]["bytes_gather"] / t4 / 1e9
        droof = {"kernel": "K4 sparse_attn_decode (split-K row gather + merge)", "bound": "hbm",
                 "achieved": ach, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                 "frac": ach * 1e9 / PEAK_HBM, "traffic": None,
                 "algorithmic_bytes_per_launch": dw["attn"]["bytes_gather"],
                 "mean_launch_us": t4 * 1e6}
        droof["traffic"], droof["traffic_source"] = counted_traffic(dwl.name)
        dec = {"workload": dwl.name, "us_per_step": dtm * 1e3, "steps": args.decode_steps,
               "us_per_step_graph": dgraph * 1e3,
               "config": {"B": dwl.B, "T": dwl.T, "heads": dwl.H, "qk": dwl.Dqk, "v": dwl.v,
                          "index_heads": dwl.HI, "index_dim": dwl.DI, "topk": dwl.topk},
               "stages": dec_r, "roofline": droof, "cpu_baseline": None}

    also = {}
    for name in [s for s in args.also.split(",") if s]:
        if name in (wl.name, args.decode_workload):
            continue
        lay = make_layer(WORKLOADS[name], torch, dsa, datagen)
        ps, tm, _ = time_layer(lay, args.also_steps, 2, torch)
        also[name] = summarize(WORKLOADS[name], ps, tm)
        dst = [st for st in lay.stages() if st[0].startswith("D ")]
        if dst:  # the decode token's stages replayed from a HIP graph
            also[name]["decode_us_per_step_graph"] = time_graph(dst, 20, torch) * 1e3
        del lay
        torch.cuda.empty_cache()
        log(f"{name}: {tm:.3f} ms/step")

    roof = headline_roofline(wl, per_stage)

    # ---- the oracle on this host's cores (after every GPU measurement)
    cpu = None
    if not args.no_cpu and not (wl.swa_only or wl.prologue_only or wl.mla_prologue_only):
        log("cpu baseline (oracle)")
        cpu = cpu_prefill_baseline(wl, args.cpu_seconds)
        cpu["cpu_model"] = cpu_model()
        cpu["one_thread"] = {
            name: cpu_prefill_baseline(WORKLOADS[name], args.cpu_seconds / 3, threads=1)
            for name in ("tiny-fp32", "mla-s4k")}
        if dec is not None:
            dec["cpu_baseline"] = cpu_decode_baseline(WORKLOADS[args.decode_workload])
            dec["cpu_baseline"]["cpu_model"] = cpu["cpu_model"]
    line = {
        "metric": METRIC,
        "value": main_r.get("step_tokens_per_s", main_r.get("prefill_tokens_per_s",
                                                            1e6 / main_r.get("decode_us_per_step", 1.0))),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype_name, "data": "synthetic (seeded Irwin-Hall normal inputs in HBM)",
        "config": {"workload": wl.name, "B": wl.B, "S": wl.S, "past_len": wl.past_len,
                   "heads": wl.H, "qk_nope": wl.nope, "qk_rope": wl.rope, "v": wl.v,
                   "index_heads": wl.HI, "index_dim": wl.DI, "topk": wl.topk,
                   "parallelism": "single GPU"},
        "decode_us_per_step": dec["us_per_step"] if dec else main_r.get("decode_us_per_step"),
        "stages": main_r,
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": dec,
        "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
