"""dsa_sparse_attn_decode_noalloc (no workspace, static device scratch)
against dsa_sparse_attn_decode on the same inputs, through the C ABI: two
calls in a row, the second with smaller sizes (fewer rows, heads and
selected keys), so the second call runs over scratch the first one filled.
The two entry points share their kernels, so outputs must be bit-identical;
a few rows are also checked against the oracle."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import sparse_attention_11_amd as dsa
from tests._helpers import assert_rows_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, T, H, nope, rope, Dv, k, seed):
    Dqk = nope + rope
    g = lambda shape, tid, sc=1.0: datagen.normal_device(
        torch.empty(*shape, dtype=torch.bfloat16, device=DEV), seed, tid, sc)
    q, kc, vc = g((B, 1, H, Dqk), 1, Dqk ** -0.5), g((B, T, H, Dqk), 2), g((B, T, H, Dv), 3)
    gate = g((B, 1, H), 7)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device=DEV)
    datagen.indices_device(idx.view(B, k), 0, 1, T - 1, seed=seed)
    return q, kc, vc, gate, idx


@pytest.mark.parametrize("first,second", [
    ((4, 20000, 64, 128, 64, 128, 2048), (2, 5000, 16, 128, 64, 128, 512)),
    ((8, 9000, 128, 128, 64, 128, 2048), (1, 3000, 8, 64, 64, 64, 100)),
])
def test_noalloc_decode_matches_workspace_decode(first, second):
    for n, (B, T, H, nope, rope, Dv, k) in enumerate((first, second)):
        print(f"noalloc call {n}: B {B} T {T} H {H} dims {nope}+{rope}/{Dv} topk {k}", flush=True)
        q, kc, vc, gate, idx = _case(B, T, H, nope, rope, Dv, k, seed=40 + n)
        ref = torch.full((B, 1, H, Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
        got = torch.full((B, 1, H, Dv), float("nan"), dtype=torch.bfloat16, device=DEV)
        dsa.dsa_sparse_attn_decode(q, kc, vc, idx, gate, ref, nope, rope)
        dsa.dsa_sparse_attn_decode_noalloc(q, kc, vc, idx, gate, got, nope, rope)
        torch.cuda.synchronize()
        a = got.view(torch.int16).cpu().numpy()
        b = ref.view(torch.int16).cpu().numpy()
        np.testing.assert_array_equal(a, b)
        # and the oracle on the first and last sequence
        qh, kh, vh = (t.view(torch.int16).cpu().numpy().view(np.uint16) for t in (q, kc, vc))
        gh = gate.view(torch.int16).cpu().numpy().view(np.uint16)
        ih = idx.cpu().numpy()
        for bb in sorted({0, B - 1}):
            r = oracle.sparse_attn(qh[bb:bb + 1], kh[bb:bb + 1], vh[bb:bb + 1], ih[bb:bb + 1],
                                   gh[bb:bb + 1], T - 1, nope, rope)
            assert_rows_close(got[bb].float().cpu().numpy(), r[0], 2e-2, what=f"noalloc b {bb}")
