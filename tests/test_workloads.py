"""Host-side checks of the seeded input generator (shapes, determinism, value
ranges, bf16 rounding, step-speed tables)."""

import numpy as np
import pytest

from semi_ar_draft_round_amd import workloads as W


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -2.5, 1e-40], dtype=np.float32)
    bits = W.bf16_bits(x)
    back = W.bf16_to_f32(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                       # halfway: ties to even
    assert back[2] == np.float32(1.0 + 2.0 ** -7)
    assert back[3] == -2.5
    np.testing.assert_allclose(back, x, rtol=2.0 ** -8, atol=1e-38)


def test_uniforms_exact_and_open_interval():
    rng = np.random.default_rng(0)
    u = W.odd_uniform(rng, 100000)
    assert u.dtype == np.float32
    assert u.min() > 0.0 and u.max() < 1.0
    k = u.astype(np.float64) * 2.0 ** 24
    np.testing.assert_array_equal(k, np.round(k))
    assert np.all(np.round(k) % 2 == 1)
    g = W.gumbel_from_uniform(u)
    assert abs(float(g.mean()) - 0.5772156649) < 0.02


def test_small_workload_shapes_and_determinism():
    w = W.BY_NAME["tiny_r1_g4_v1024_f32"]
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for f in ("U", "E", "W2t", "w_conf", "h", "x0", "target", "G", "g", "u_acc", "u_res"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.U.shape == (1, 4, 1024) and a.U.dtype == np.float32
    assert a.target.shape == (1, 5, 1024)
    assert a.G.shape == (4, 64, 1) and a.g.shape == (1, 4, 16)
    assert a.E.shape == (1024, 32) and a.W2t.shape == (1024, 32)
    assert a.w_conf.shape == (96,) and a.h.shape == (1, 4, 64)
    assert a.sps.shape == (8,) and np.all(np.diff(a.sps) <= 0)
    assert a.T is None
    c = W.make_inputs(w, round_index=1)
    assert not np.array_equal(a.U, c.U)
    np.testing.assert_array_equal(a.E, c.E)      # weights do not change between rounds


def test_bf16_custom_workload_distributions():
    w = W.custom("t", R=4, gamma=3, V=300, r=32, d=48, seed=5, temperatures=True)
    a = W.make_inputs(w)
    assert a.U.dtype == np.uint16
    U = W.bf16_to_f32(a.U)
    # half of the positions carry a spike on top of N(0, 4)
    assert abs(float(np.std(U)) - 2.0) < 0.3
    assert a.G.shape == (3, 19, 4)
    np.testing.assert_allclose(a.T, [1.0, 1.5, 2.0])
    assert a.sps.shape[0] == w.R * (1 + w.gamma)


@pytest.mark.parametrize("name,n,first,last", [
    ("batch_r32_g16_v151936", 4096, 1000.0, 56.0),
    ("heavy_r128_g16_v129280", 4096, 1999.0, 666.0),
    ("full_r256_g16_v129280_sts", 4352, 1999.0, 640.0),
    ("latency_r1_g16_v151936", 17, 1000.0, 1000.0),
])
def test_step_speed_tables(name, n, first, last):
    s = W.make_sps(W.BY_NAME[name])
    assert s.shape == (n,)
    assert s[0] == first and s[-1] == last
    assert np.all(np.diff(s) <= 0)
    w = W.BY_NAME[name]
    assert s.shape[0] >= w.R * (1 + w.gamma)
