"""The MFMA prefill path's work plan, checked on the CPU (no GPU call).

The plan decides which 64-key blocks each workgroup of the flash kernel
multiplies and where split work items put their partial states. A wrong plan
is a wrong answer or an out-of-bounds write on the GPU, so its invariants are
checked here for many call shapes, by emulating the kernel's own item ->
(tile, split) -> key-range arithmetic on the plan the library reports:
  * every item of a tile covers a distinct, contiguous run of at most
    max_blocks blocks, and together they cover the tile's visible range;
  * sliding-window calls and calls with many tiles never split;
  * the partial-state buffer, sized from the plan of past_len = T - S, holds
    every item any call with the same sizes launches.
"""
import pytest

import sparse_attention_11_amd as dsa

BQ, BN = 128, 64
INT_MAX = 0x7FFFFFFF


def tile_range(qt, S, P, Tbuf, kv_offset, window):
    """Buffer rows [jlo, jhi] (jlo 64-aligned) a 128-query tile can see."""
    q0 = qt * BQ
    pmax = P + min(q0 + BQ - 1, S - 1)
    tlo = max(kv_offset, P + q0 - window + 1) if window > 0 else 0
    jlo = ((tlo - kv_offset) // BN) * BN
    jhi = min(pmax - kv_offset, Tbuf - 1)
    return jlo, jhi


def item_ranges(B, S, T, P, H, kv_offset=0, window=0):
    nqt, items, M, start = dsa.dsa_prefill_work_plan(B, S, T, P, H, kv_offset, window)
    assert nqt == (S + BQ - 1) // BQ
    assert start[0] == 0 and start[nqt] == items
    per_tile = {}
    for item in range(items):
        if M == INT_MAX:
            qt, split, nsplit = nqt - 1 - item, 0, 1
        else:
            o = max(i for i in range(nqt) if start[i] <= item)
            qt, split, nsplit = nqt - 1 - o, item - start[o], start[o + 1] - start[o]
        tjlo, tjhi = tile_range(qt, S, P, T, kv_offset, window)
        jlo = tjlo + split * M * BN
        jhi = min(tjhi, jlo + M * BN - 1)
        per_tile.setdefault(qt, []).append((split, nsplit, jlo, jhi))
    return nqt, items, M, per_tile


SHAPES = [
    # (B, S, T, P, H): the mla-s4k prefill, short and ragged chunks after long
    # caches, small S, many heads (no split), several batch rows
    (1, 4096, 4096, 0, 20), (1, 4096, 8192, 4096, 20), (1, 4000, 9000, 5000, 4),
    (1, 16, 50000, 49984, 8), (1, 300, 70000, 69700, 2), (2, 1000, 1000, 0, 3),
    (1, 32768, 32768, 0, 128), (1, 4096, 528384, 524288, 32), (3, 129, 129, 0, 1),
    (1, 4096, 6000, 100, 20),
]


@pytest.mark.parametrize("B,S,T,P,H", SHAPES)
def test_items_cover_each_tile_once(B, S, T, P, H):
    nqt, items, M, per_tile = item_ranges(B, S, T, P, H)
    assert sorted(per_tile) == list(range(nqt))
    for qt, its in per_tile.items():
        tjlo, tjhi = tile_range(qt, S, P, T, 0, 0)
        its.sort()
        assert [s for s, _, _, _ in its] == list(range(len(its)))
        assert all(n == len(its) for _, n, _, _ in its)
        nb = (tjhi - tjlo) // BN + 1
        if M != INT_MAX:
            assert len(its) == max(1, -(-nb // M))
        else:
            assert len(its) == 1
        # contiguous, non-overlapping, each at most M blocks, union = the tile's range
        nxt = tjlo
        for _, _, jlo, jhi in its:
            assert jlo == nxt and jhi >= jlo
            assert (jhi - jlo) // BN + 1 <= min(M, nb)
            nxt = jhi + 1
        assert nxt == tjhi + 1
        assert tjhi <= T - 1 and tjhi == P + min(qt * BQ + BQ - 1, S - 1)


@pytest.mark.parametrize("B,S,T,P,H", SHAPES)
def test_partial_buffer_from_the_bound_plan_holds_every_call(B, S, T, P, H):
    # the workspace holds B * H * items_bound partial tiles; every call with the
    # same (B, S, T, H) and any past_len <= T - S launches at most that many
    _, items_bound, _, _ = dsa.dsa_prefill_work_plan(B, S, T, T - S, H, 0, 0)
    for p in sorted({0, P, (T - S) // 2, T - S}):
        _, items, _, _ = dsa.dsa_prefill_work_plan(B, S, T, p, H, 0, 0)
        assert items <= items_bound, (p, items, items_bound)


@pytest.mark.parametrize("B,S,P,W,off,H", [
    (1, 300, 700, 128, 0, 2),        # the shape of the case that once faulted
    (1, 4096, 524288, 512, 524288 - 511, 32), (1, 4096, 131072, 512, 131072 - 511, 8),
    (2, 1000, 0, 64, 0, 4), (1, 16, 5000, 4096, 904, 1), (1, 200, 50, 1000, 0, 3),
])
def test_window_calls_never_split(B, S, P, W, off, H):
    Tbuf = P + S - off
    nqt, items, M, per_tile = item_ranges(B, S, Tbuf, P, H, off, W)
    assert M == INT_MAX and items == nqt
    for qt, [(split, nsplit, jlo, jhi)] in per_tile.items():
        assert split == 0 and nsplit == 1
        assert 0 <= jlo and jhi <= Tbuf - 1
        # the tile's window rows are inside [jlo, jhi]
        q0 = qt * BQ
        first = max(off, P + q0 - W + 1) - off
        last = P + min(q0 + BQ - 1, S - 1) - off
        assert jlo <= first and jhi == last


def test_many_tiles_never_split():
    nqt, items, M, _ = item_ranges(1, 300 * 128, 300 * 128, 0, 1)
    assert M == INT_MAX and items == nqt == 300


def test_work_plan_rejects_bad_sizes():
    with pytest.raises(dsa.DsaError):
        dsa.dsa_prefill_work_plan(1, 10, 5, 0, 4)  # past_len + S > T
    with pytest.raises(dsa.DsaError):
        dsa.dsa_prefill_work_plan(0, 10, 10, 0, 4)
