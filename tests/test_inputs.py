"""Seeded input generator: determinism, rounding and RoPE properties (CPU)."""

import numpy as np

from static_pattern_sparse_amd import inputs as I


def test_deterministic_and_distinct_streams():
    a = I.make_inputs(1, 2, 64, 16, "bf16", 2, 3)
    b = I.make_inputs(1, 2, 64, 16, "bf16", 2, 3)
    c = I.make_inputs(1, 2, 64, 16, "bf16", 2, 4)
    for n in a:
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert not np.array_equal(a["q"], a["k"])


def test_bf16_values_are_exact_and_nearest():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    r = I.round_to_bf16(x)
    assert (r.view(np.uint32) & 0xFFFF == 0).all()
    # nearest: no other bf16 neighbour is closer
    up = ((r.view(np.uint32) + 0x10000).view(np.float32))
    dn = ((r.view(np.uint32) - 0x10000).view(np.float32))
    e = np.abs(r.astype(np.float64) - x)
    assert (e <= np.abs(up.astype(np.float64) - x)).all()
    assert (e <= np.abs(dn.astype(np.float64) - x)).all()


def test_rope_is_a_rotation_of_each_pair():
    T, D = 50, 16
    raw = I.make_tensor(1, 1, T, D, "f32", 9, 0, "q", rope_base=None)[0, 0]
    rot = I.make_tensor(1, 1, T, D, "f32", 9, 0, "q", rope_base=10000.0)[0, 0]
    h = D // 2
    n_raw = raw[:, :h] ** 2 + raw[:, h:] ** 2
    n_rot = rot[:, :h] ** 2 + rot[:, h:] ** 2
    np.testing.assert_allclose(n_rot, n_raw, rtol=1e-5)
    assert np.array_equal(raw[0], rot[0])          # position 0 is not rotated


def test_workload_table_shapes():
    w = I.WORKLOADS["linear16_bf16_b1h16t65536d128_w12"]
    assert (w.B, w.H, w.T, w.D, w.rope_base) == (1, 16, 65536, 128, 500000.0)
    assert len({x.workload_id for x in I.WORKLOADS.values()}) == len(I.WORKLOADS)


def test_decode_inputs_share_the_sequence_generator():
    """A decoding step's caches are the sequence workload's k and v for the
    same seeds; the query is a rotated N(0,1) row (rotation keeps its norm)."""
    pos = I.decode_positions(3, 200)
    assert list(pos) == [199, 138, 77]
    x = I.make_decode_inputs(3, 2, 200, 64, "f32", 9, 1, pos)
    seq = I.make_inputs(3, 2, 200, 64, "f32", 9, 1, with_dout=False)
    assert np.array_equal(x["k"], seq["k"]) and np.array_equal(x["v"], seq["v"])
    assert x["q"].shape == (3, 2, 64) and x["pos"].dtype == np.int32
    raw = I._rng(9, 1, "q").standard_normal((2, 64))      # entry 0's draw
    np.testing.assert_allclose(np.linalg.norm(x["q"][0], axis=1),
                               np.linalg.norm(raw, axis=1), rtol=1e-6)
    xb = I.make_decode_inputs(2, 1, 50, 64, "bf16", 9, 1, [49, 0])
    for t in (xb["q"], xb["k"], xb["v"]):
        assert np.array_equal(t, I.round_to_bf16(t))       # bf16-exact


def test_seed_root_gives_another_draw_and_defaults_to_the_recipe():
    """The default seed root is the recipe's; another root is another draw of
    the same shapes and rounding."""
    a = I.make_inputs(1, 2, 64, 16, "bf16", 2, 3)
    b = I.make_inputs(1, 2, 64, 16, "bf16", 2, 3, seed_root=I.SEED_ROOT)
    c = I.make_inputs(1, 2, 64, 16, "bf16", 2, 3, seed_root=I.SEED_ROOT + 1)
    for n in ("q", "k", "v", "dout"):
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
        assert np.array_equal(c[n], I.round_to_bf16(c[n]))
