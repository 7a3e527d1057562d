"""The seeded input generator: determinism, shapes, casts and the frozen calibration."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def test_configs_match_the_workload_shapes():
    c = W.CONFIGS
    assert (c["tiny"].tokens, c["tiny"].nblocks, c["tiny"].dtype) == (256, 4, "fp32")
    assert (c["wan13b_480p"].tokens, c["wan13b_480p"].nblocks) == (32760, 512)
    assert (c["wan14b_720p"].tokens, c["wan14b_720p"].nblocks) == (75600, 591)
    assert (c["hunyuan_720p"].tokens, c["hunyuan_720p"].nblocks) == (118800, 929)
    assert c["reuse_720p"].steps == 50 and c["reuse_720p"].drift_threshold == 0.05
    np.testing.assert_array_equal(c["wan13b_480p"].top_p_array()[:6],
                                  np.float32([0.8, 0.9, 0.95, 0.8, 0.9, 0.95]))


def test_generator_is_deterministic_and_head_local():
    wl = W.CONFIGS["wan13b_480p"].scaled(heads=3, grid=(3, 6, 10))
    a = W.make_inputs(wl)
    b = W.make_inputs(wl, heads=[2])
    assert torch.equal(a.q[2], b.q[0]) and torch.equal(a.v[2], b.v[0])
    c = W.make_inputs(wl)
    assert torch.equal(a.k, c.k)
    assert a.q.dtype == torch.bfloat16 and a.q.shape == (3, 180, 128)
    assert not torch.equal(a.q[0], a.q[1])


def test_bf16_cast_is_round_to_nearest_even():
    x = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8)], np.float32)
    got = W._cast(x, "bf16").float().numpy()
    np.testing.assert_array_equal(got, np.float32([1.0, 1.0 + 4 * 2**-8, -1.0]))


def test_tiny_config_stays_fp32():
    inp = W.make_inputs(W.CONFIGS["tiny"])
    assert inp.q.dtype == torch.float32 and inp.q.shape == (1, 256, 64)


def test_trajectory_drift_step_is_a_random_walk():
    wl = W.CONFIGS["reuse_720p"].scaled(heads=2, grid=(2, 4, 16))
    inp = W.make_inputs(wl, keep_masters=True)
    q0 = inp.q_master.copy()
    W.drift_step(inp, 1)
    d = inp.q_master - q0
    assert abs(d.std() - W.DRIFT_STD) < 0.1 * W.DRIFT_STD
    assert torch.equal(inp.q, torch.from_numpy(inp.q_master).to(torch.bfloat16))


def test_alpha_calibration_density_in_range():
    """Frozen ALPHA keeps the 720p Wan2.1-14B shape at 15-30 % mean density (p=0.9)."""
    wl = W.CONFIGS["wan14b_720p"]
    heads = list(range(0, wl.heads, 2))
    inp = W.make_inputs(wl, heads=heads)
    rng = np.random.default_rng(0)
    dens = []
    for i, h in enumerate(heads):
        qb = sorted(rng.choice(wl.nblocks, 6, replace=False))
        s = O.score_head(W.to_f64(inp.q[i]), W.to_f64(inp.k[i]), wl.block,
                         1 / np.sqrt(wl.head_dim), query_blocks=qb)
        dens.append(np.mean([O.select_row(r, 0.9)[1] for r in s]) / wl.nblocks)
    assert 0.15 <= float(np.mean(dens)) <= 0.30
