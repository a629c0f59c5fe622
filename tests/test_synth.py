"""Seeded input generators: determinism, distributions, rounding."""
import numpy as np
import torch

import synth
from synth import configs


def test_tokens_deterministic_and_distinct_batches():
    wl = configs.workload(1)
    a, b = synth.tokens(wl), synth.tokens(wl)
    assert a.dtype == np.int32 and a.shape == (8, 2048)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.tokens(wl, batch=1))


def test_zipf_frequencies():
    wl = configs.with_tokens(configs.workload(1), 64, 4096)
    t = synth.tokens(wl).reshape(-1)
    V = wl["vocab"]
    p = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    freq = np.bincount(t, minlength=V) / t.size
    for i in range(5):
        se = np.sqrt(p[i] * (1 - p[i]) / t.size)
        assert abs(freq[i] - p[i]) < 5 * se
    assert t.min() >= 0 and t.max() < V


def test_uniform_tokens_in_range():
    t = synth.tokens(configs.workload(0))
    assert t.shape == (1, 256) and t.min() >= 0 and t.max() < 1024


def test_words_are_splitmix64_outputs():
    base = synth.stream_base(9, 3)
    w = synth.words(9, 3, np.arange(3))
    M = 2**64
    for i in range(3):
        z = (base + (i + 1) * synth.GOLDEN) % M
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) % M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) % M
        z ^= z >> 31
        assert int(w[i]) == z


def test_normal_generator_moments_and_bounds():
    v = synth.normal_f32(3, configs.STREAM_TABLE, np.arange(2_000_000), 0.02)
    assert v.dtype == np.float32
    assert abs(v.mean()) < 1e-4 and abs(v.std() - 0.02) < 2e-4
    assert np.abs(v).max() <= 0.02 * np.sqrt(3) * 2 + 1e-6


def test_bf16_rounding_matches_torch():
    v = synth.normal_f32(4, 1, np.arange(100_000), 0.02)
    v = np.concatenate([v, np.float32([1.0 + 2**-8, 1.0 + 3 * 2**-8, -0.0])])
    ours = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours, ref.view(np.uint16))


def test_nf4_rows():
    wl = configs.workload(3)
    codes, scales = synth.table_rows(wl, [0, 1, 312_499_967])
    assert codes.shape == (3, 32) and codes.dtype == np.uint8
    assert scales.dtype == np.float16
    s = scales.astype(np.float64)
    assert (s >= 0.0375 - 1e-4).all() and (s < 0.0875 + 1e-4).all()
    nib = np.concatenate([synth.table_rows(wl, np.arange(2000))[0] & 15,
                          synth.table_rows(wl, np.arange(2000))[0] >> 4])
    cnt = np.bincount(nib.reshape(-1), minlength=16)
    assert cnt.min() > 0.9 * cnt.mean()


def test_engram_params():
    wl = configs.workload(4)
    gh, gk, gu, cw = synth.engram_params(wl)
    assert (gh == 1).all() and cw.shape == (2560, 4)
    assert abs(cw.std() - 0.5) < 0.02
    wl2 = dict(wl, gamma="random")
    gh2, _, _, _ = synth.engram_params(wl2)
    assert gh2.dtype == np.float32 and abs(gh2.mean() - 1) < 0.02
