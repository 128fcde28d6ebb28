"""The host generator against its written definition (CPU only)."""
import numpy as np
import torch

import datagen

M64 = (1 << 64) - 1


def mix64(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def normal_ref(seed, tid, i, scale):
    key = mix64(((seed << 20) + tid) & M64)
    s = 0
    for j in (1, 2, 3):
        r = mix64((key + (3 * i + j) * 0x9E3779B97F4A7C15) & M64)
        s += sum((r >> sh) & 0xFFFF for sh in (0, 16, 32, 48))
    return np.float32(s - 393210) * np.float32(datagen.cscale(scale))


def test_splitmix_normal_matches_definition():
    idx = [0, 1, 2, 17, 12345, 10**9 + 7]
    for seed, tid in [(0, 1), (3, 5), (4, 2 + 16)]:
        for i in idx:
            got = datagen.normal_host((1,), "f32", seed, tid, 0.7, start=i)[0]
            assert got == normal_ref(seed, tid, i, 0.7)


def test_bf16_is_round_nearest_even_of_fp32():
    f = datagen.normal_host((4096,), "f32", 1, 3, 2.0)
    b = datagen.normal_host((4096,), "bf16", 1, 3, 2.0)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_start_offset_is_a_window_of_the_stream():
    a = datagen.normal_host((1000,), "bf16", 2, 2, 1.0)
    b = datagen.normal_host((300,), "bf16", 2, 2, 1.0, start=500)
    np.testing.assert_array_equal(a[500:800], b)


def test_normal_moments():
    a = datagen.normal_host((1 << 20,), "f32", 0, 1, 3.0).astype(np.float64)
    assert abs(a.mean()) < 0.02 and abs(a.std() - 3.0) < 0.02
    assert np.abs(a).max() <= 6 * 3.0 + 1e-3  # Irwin-Hall(12) support is +-6 sigma


def test_index_rows_distinct_and_visible():
    S, P, k = 50, 7, 16
    idx = datagen.indices_host(0, S, S, P, k, seed=3)
    for s in range(S):
        n = P + s + 1
        row = idx[s]
        valid = row[row >= 0]
        assert len(valid) == min(n, k) and len(set(valid.tolist())) == len(valid)
        assert valid.max() <= P + s
        assert np.all(row[len(valid):] == -1)


def test_score_rows_structure():
    S, T, P = 6, 20, 10
    for mode in (0, 1, 2):
        sc = datagen.scores_host(0, S, S, T, P, seed=1, mode=mode)
        for s in range(S):
            assert np.all(np.isneginf(sc[s, P + s + 1:]))
            assert np.all(np.isfinite(sc[s, : P + s + 1]))
    q = datagen.scores_host(0, S, S, T, P, seed=1, mode=1)
    fin = q[np.isfinite(q)]
    np.testing.assert_array_equal(fin * 8, np.rint(fin * 8))
    z = datagen.scores_host(0, 64, 64, 64, 63, seed=1, mode=2)
    zeros = z[z == 0]
    assert np.any(np.signbit(zeros)) and np.any(~np.signbit(zeros))
