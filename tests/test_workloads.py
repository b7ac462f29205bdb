"""Seeded synthetic inputs: determinism, bf16 rounding, and the workload rules."""

import os

import numpy as np
import torch

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = [float(x) for x in v.split()]
    return out


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  65504.0, 1e-38, 0.0, -0.0], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(np.float32([1.0 + 2 ** -8])))[0] == 1.0


def test_same_seed_same_bits():
    a = wl.tiny_batch()
    b = wl.tiny_batch()
    for f in ("hidden", "weight", "targets", "keep", "g_logp", "g_entropy"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = wl.tiny_batch(seed=11)
    assert not np.array_equal(a.hidden, c.hidden)


def test_tiny_batch_shape_and_distribution():
    w = wl.tiny_batch()
    assert (w.N, w.H, w.V) == (128, 512, 8192)
    X = wl.bf16_bits_to_f32(w.hidden)
    W = wl.bf16_bits_to_f32(w.weight)
    assert abs(X.std() - 1.0) < 0.02
    assert abs(W.std() * np.sqrt(512) - 1.0) < 0.02
    assert w.targets.min() >= 0 and w.targets.max() < 8192
    assert 0.55 < w.keep.mean() < 0.85
    assert w.return_entropy and w.entropy_requires_grad


def test_keep_sweep_is_the_pages_table():
    g = _golden()
    assert tuple(g["skyrl_active_fractions"]) == wl.KEEP_SWEEP


def test_dense_rl_masks_nested_and_fractions():
    # reduced sizes, same rules as the full config
    ms = [wl.dense_rl(f, N=20000, H=64, V=256).keep for f in wl.KEEP_SWEEP]
    for f, m in zip(wl.KEEP_SWEEP, ms):
        assert abs(m.mean() - f) < 0.015
    for hi, lo in zip(ms, ms[1:]):
        assert np.all(lo <= hi)  # lower fraction is a subset
    assert wl.dense_rl(1.0, N=64, H=64, V=256, mask=False).keep is None


def test_dense_rl_masks_helper_matches_dense_rl():
    masks = wl.dense_rl_masks(wl.KEEP_SWEEP, N=5000)
    for f in wl.KEEP_SWEEP:
        assert np.array_equal(masks[f], wl.dense_rl(f, N=5000, H=64, V=256).keep)


def test_packed_grpo_layout_rules():
    rng = np.random.default_rng(1)
    N, V = 4096, 1000
    tok, t, keep, starts = wl.packed_grpo_layout(N, V, 16, rng)
    ends = np.append(starts[1:], N)
    assert len(starts) == 16 and starts[0] == 0 and np.all(np.diff(starts) > 0)
    for s, e in zip(starts, ends):
        # next-token targets inside each sequence, last position target 0 keep 0
        np.testing.assert_array_equal(t[s:e - 1], tok[s + 1:e])
        assert t[e - 1] == 0 and keep[e - 1] == 0
        k = keep[s:e]
        # prompt (keep 0) then completion (keep 1): one 0 -> 1 switch at most
        assert np.all(np.diff(k.astype(int)[:-1]) >= 0)
        L = e - s
        n_keep = int(k.sum())
        if L > 5:
            assert 0.4 * L - 2 <= n_keep <= 0.8 * L + 1


def test_packed_grpo_bias_makes_target_logits_peaked():
    w = wl.packed_grpo(N=2048, H=256, V=4096)
    X = wl.bf16_bits_to_f32(w.hidden).astype(np.float64)
    W = wl.bf16_bits_to_f32(w.weight).astype(np.float64)
    kept = np.flatnonzero(w.keep)
    sigma = np.sqrt(256) * 0.02
    # first kept row of each target gets z_t ~ N(0, sigma) + 3 sigma
    _, first = np.unique(w.targets[kept], return_index=True)
    rows = kept[first]
    zt = np.einsum("ij,ij->i", X[rows], W[w.targets[rows]])
    assert abs(zt.mean() - 3 * sigma) < 0.2
    assert not w.entropy_requires_grad and w.return_entropy


def test_fp32_stress_row_scales():
    w = wl.fp32_stress(N=4096, H=128, V=512)
    s = w.meta["row_scale"]
    assert s.min() >= 0.5 - 1e-6 and s.max() <= 8.0 + 1e-5
    X = wl.bf16_bits_to_f32(w.hidden)
    ratio = X.std(axis=1) / s
    assert abs(np.median(ratio) - 1.0) < 0.05
    assert w.keep.all()


def test_scoring_spans():
    rng = np.random.default_rng(2)
    keep = wl.span_keep(262144, rng)
    assert 0.35 < keep.mean() < 0.65
    # runs of equal values are made of spans of 64..2048 tokens
    edges = np.flatnonzero(np.diff(keep.astype(int))) + 1
    runs = np.diff(np.concatenate([[0], edges, [keep.size]]))
    assert runs[:-1].min() >= 64


def test_sample_rows_is_seeded_and_sorted():
    rows = np.arange(0, 10000, 3)
    a = wl.sample_rows(rows, 512, 1)
    b = wl.sample_rows(rows, 512, 1)
    np.testing.assert_array_equal(a, b)
    assert np.all(np.diff(a) > 0) and np.isin(a, rows).all()
    assert wl.sample_rows(rows[:10], 512, 1).size == 10
