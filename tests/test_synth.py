"""Host-side checks of the seeded workload generators (no GPU)."""
import numpy as np
import torch

from token_sparse_attention_amd import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 37.0
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]     # exact halfway cases
    ours = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_shapes_and_determinism():
    a = synth.generate("tiny")
    b = synth.generate("tiny")
    for t in "qkv":
        assert a[t].shape == (1, 2, 1024, 64) and a[t].dtype == np.uint16
        np.testing.assert_array_equal(a[t], b[t])
    assert not np.array_equal(a["q"][0, 0], a["q"][0, 1])


def test_head_subset_matches_full_generation():
    full = synth.generate("tiny")
    sub = synth.generate("tiny", heads=[(0, 1)])
    np.testing.assert_array_equal(sub["k"][0, 0], full["k"][0, 1])


def test_drift_is_small_and_seeded():
    a = synth.generate("tiny")
    b = synth.drift("tiny", a, step=1)
    c = synth.drift("tiny", a, step=1)
    d = synth.drift("tiny", a, step=2)
    np.testing.assert_array_equal(b["v"], c["v"])
    assert not np.array_equal(b["v"], d["v"])
    diff = synth.to_f64(b["q"]) - synth.to_f64(a["q"])
    assert 0.03 < diff.std() < 0.08


def test_video_generator_is_spatially_local():
    w = synth.WORKLOADS["small"]
    x = synth.generate("small", heads=[(0, 0)])
    q = synth.to_f64(x["q"][0, 0])
    k = synth.to_f64(x["k"][0, 0])
    s = q[:64] @ k.T / np.sqrt(w.D)
    # the strongest key of each early query lies near it in the grid
    near = np.abs(np.argmax(s, axis=1) - np.arange(64))
    assert np.median(near) < 3 * w.grid[2]


def test_index_set_and_perm_helpers():
    p = synth.random_perm(1, 3, 100, seed=1)
    assert p.dtype == np.int32 and all(sorted(r.tolist()) == list(range(100)) for r in p[0])
    ix = synth.random_index_sets(1, 2, 5, 17, 100, seed=2)
    assert ix.shape == (1, 2, 5, 17)
    for row in ix.reshape(-1, 17):
        assert (np.diff(row) > 0).all() and row.min() >= 0 and row.max() < 100
    full = synth.random_index_sets(1, 1, 2, 9, 9, seed=3)
    np.testing.assert_array_equal(full[0, 0, 1], np.arange(9))
    m = synth.mass_rows(3, 500, seed=4)
    assert m.dtype == np.float32 and (m >= 0).all()
    assert len(np.unique(m[0])) < 500
