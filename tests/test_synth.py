"""The seeded input generators: determinism, structure and bf16 rounding."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_bits(x), ref)
    back = synth.bf16_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_tiny_workload_is_deterministic_and_well_formed():
    wl = synth.WORKLOADS["c1"]
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    for f in ("h", "W", "idx", "tl"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.h.shape == (512, 256) and a.W.shape == (4096, 256) and a.idx.shape == (512, 10)
    assert a.idx.min() >= 0 and a.idx.max() < 4096
    assert all(len(set(r)) == 10 for r in a.idx.tolist())
    assert (np.diff(a.tl, axis=1) <= 0).all()
    # the GPU-facing copies are bf16 values; the raw fp32 draws are kept
    np.testing.assert_array_equal(synth.round_bf16(a.h_raw), a.h)
    assert abs(float(a.h_raw.std()) - 1.0) < 0.02 and abs(float(a.W_raw.std()) - 0.02) < 0.001


def test_perturbed_head_teacher_is_topk():
    from dataclasses import replace
    wl = replace(synth.WORKLOADS["c2"], N=40, H=32, V=300, K=12, batch=1, seq=40)
    x = synth.make_inputs(wl)
    Wp = synth.round_bf16(x.W + synth.normal(wl.seed(synth.S_WNOISE), x.W.shape, 0.01))
    z = x.h.astype(np.float64) @ Wp.astype(np.float64).T
    for i in range(wl.N):
        top = np.argsort(-z[i], kind="stable")[:wl.K]
        assert set(top.tolist()) == set(x.idx[i].tolist())
    assert (np.diff(x.tl, axis=1) <= 0).all()


def test_scaled_rows_and_samples():
    from dataclasses import replace
    wl = replace(synth.WORKLOADS["c5"], N=1000, H=16, V=500)
    x = synth.make_inputs(wl)
    rows = synth.scaled_rows(wl)
    assert rows.size == 10
    norms = np.linalg.norm(x.h, axis=1)
    assert norms[rows].min() > 5 * np.median(norms)
    s = synth.sample_rows(wl, 64, must_include=rows[:3])
    assert np.all(np.diff(s) > 0) and set(rows[:3]).issubset(set(s.tolist()))


def test_distinct_indices_full_range():
    idx = synth.distinct_indices(5, 200, 30, 40)
    assert all(len(set(r)) == 30 for r in idx.tolist())
    assert idx.min() >= 0 and idx.max() < 40
