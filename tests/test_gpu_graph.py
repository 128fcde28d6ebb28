"""The decode step captured in a HIP graph (the library's calls only enqueue
kernels on the caller's stream: no allocation, memset or synchronisation), replayed
several times with other eager work and synchronisations between the replays;
every replay must give exactly the eager result. Shapes: a hybrid-like decode
token (one long row: indexer, the multi-stage top-k, split-K attention with
its merge) and a window (SWA) decode."""
import numpy as np
import pytest
import torch

import datagen
import sparse_attention_11_amd as dsa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gen(shape, seed, tid, scale=1.0):
    return datagen.normal_device(torch.empty(*shape, dtype=torch.bfloat16, device=DEV), seed, tid, scale)


def test_graph_replay_matches_eager_decode_step():
    B, T, H, nope, rope, Dv, HI, DI, k, W = 1, 70001, 8, 128, 64, 128, 16, 128, 2048, 512
    Dqk = nope + rope
    P = T - 1
    print(f"graph decode step: T {T} H {H} topk {k}", flush=True)
    kc, vc = _gen((B, T, H, Dqk), 21, 2), _gen((B, T, H, Dv), 21, 3)
    kidx = _gen((B, T, DI), 21, 5, DI ** -0.5)
    # two sets of query-side inputs: the graph reads set 0; eager work between
    # replays uses set 1 on the same buffers' neighbours
    qs = [_gen((B, 1, H, Dqk), 21 + j, 1, Dqk ** -0.5) for j in range(2)]
    qis = [_gen((B, 1, HI, DI), 21 + j, 4, DI ** -0.5) for j in range(2)]
    ws_ = [_gen((B, 1, HI), 21 + j, 6, HI ** -0.5) for j in range(2)]
    gs = [_gen((B, 1, H), 21 + j, 7) for j in range(2)]
    sc = torch.empty(B, 1, T, dtype=torch.float32, device=DEV)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device=DEV)
    out = torch.empty(B, 1, H, Dv, dtype=torch.bfloat16, device=DEV)
    outw = torch.empty(B, 1, H, Dv, dtype=torch.bfloat16, device=DEV)
    tk_ws = torch.empty(max(dsa.dsa_topk_workspace_size(B, 1, T, k), 1), dtype=torch.uint8, device=DEV)
    at_ws = torch.empty(dsa.dsa_sparse_attn_decode_workspace_size(B, H, Dv, k), dtype=torch.uint8, device=DEV)
    sw_ws = torch.empty(max(dsa.swa_attn_workspace_size(B, 1, H, Dqk, Dv, W, 1), 1), dtype=torch.uint8,
                        device=DEV)
    off = T - W
    kw, vw = kc[:, off:].contiguous(), vc[:, off:].contiguous()

    def step(j):
        dsa.dsa_index_scores(qis[j], kidx, ws_[j], sc, P)
        dsa.dsa_topk_unsorted(sc, idx, tk_ws)
        dsa.dsa_sparse_attn_decode(qs[j], kc, vc, idx, gs[j], out, nope, rope, workspace=at_ws)
        dsa.swa_attn(qs[j], kw, vw, gs[j], outw, P, off, W, nope, rope, workspace=sw_ws)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (sc, idx, out, outw)]

    step(0)
    ref0 = snapshot()
    step(1)
    ref1 = snapshot()
    assert not torch.equal(ref0[2], ref1[2])  # the two input sets differ

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        step(0)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            step(0)
    torch.cuda.current_stream().wait_stream(stream)
    for rep in range(4):
        step(1)  # eager work on the same buffers between replays
        got1 = snapshot()
        for a, b in zip(got1, ref1):
            assert torch.equal(a, b), f"eager step after replay {rep}"
        g.replay()
        got = snapshot()
        for name, a, b in zip(("scores", "indices", "decode out", "window out"), got, ref0):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
