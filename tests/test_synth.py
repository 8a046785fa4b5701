"""The seeded input generator (CPU only): determinism and the recipes."""
import numpy as np

import synth


def test_counter_based_rows_are_independent_of_range():
    spec = synth.CONFIGS["C3"].with_(capacity=4, T=2, V=3000, V_pad=3000)
    full = np.empty((8, 3000), np.uint16)
    synth.fill_logits(spec, full, None, nthreads=3)
    part = np.empty((3, 3000), np.uint16)
    synth.fill_logits(spec, part, None, row_begin=4, nthreads=1)
    assert np.array_equal(full[4:7], part)
    again = np.empty_like(full)
    synth.fill_logits(spec, again, None, nthreads=5)
    assert np.array_equal(full, again)


def test_splitmix_reference_value():
    """The finalizer is SplitMix64's: seeded with 0, that generator's first two
    outputs are mix(GAMMA) = 0xE220A8397B1DCDAF and mix(2 GAMMA) =
    0x6E789E6AA1B965F4."""
    import ctypes
    lib = synth.lib()
    lib.synth_mix64.restype = ctypes.c_uint64
    lib.synth_mix64.argtypes = [ctypes.c_uint64]
    g = 0x9E3779B97F4A7C15
    assert lib.synth_mix64(g) == 0xE220A8397B1DCDAF
    assert lib.synth_mix64((2 * g) & (2**64 - 1)) == 0x6E789E6AA1B965F4


def test_normal_recipe_moments():
    spec = synth.CONFIGS["C1"]
    w = synth.make(spec)
    x = w.logits.astype(np.float64)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 3.0) < 0.05
    assert w.active_rows() == 8 and np.all(w.tokens < spec.V) and np.all(w.tokens >= 0)


def test_c2_padding_spike_and_half_requesting():
    spec = synth.CONFIGS["C2"].with_(capacity=16)
    w = synth.make(spec)
    assert int(w.requested.sum()) == 8
    g = synth.garbage_rows(spec, w.requested, w.emitted)
    for r in range(16):
        if g[r]:
            assert np.isnan(w.logits[r, 0]) and np.isinf(w.logits[r, 1])
        else:
            assert np.all(np.isposinf(w.logits[r, spec.V:]))
            assert w.logits[r, :spec.V].max() > 14.0


def test_c3_gumbel_and_garbage_rows():
    spec = synth.CONFIGS["C3"].with_(capacity=16)
    w = synth.make(spec)
    assert np.all((w.emitted >= 1) & (w.emitted <= 8))
    act = w.active_mask().reshape(-1)
    x = synth.bf16_to_f32(w.logits[act]).astype(np.float64)
    assert abs(np.median(x) - (-np.log(np.log(2)))) < 0.01  # Gumbel median
    assert np.all(x.max(axis=1) > 9.0)
    bad = w.logits[~act]
    assert np.all(bad[:, 0::2] == 0x7FC0) and np.all(bad[:, 1::2] == 0x7F80)


def test_c4_grid_one_hot_and_selected():
    spec = synth.CONFIGS["C4"].with_(V=5000, V_pad=5000)
    w = synth.make(spec)
    act = w.active_mask().reshape(-1)
    x = synth.bf16_to_f32(w.logits[act])
    finite = np.isfinite(x)
    one_hot = finite.sum(axis=1) == 1
    assert 0.05 < one_hot.mean() < 0.25
    grid = x[~one_hot]
    assert np.all(grid * 8 == np.round(grid * 8)) and grid.min() >= -8 and grid.max() <= 8
    sel = w.id_counts > 0
    assert sel.sum() == 51 and np.all(w.id_counts[sel] == 128)
    for s in np.nonzero(sel)[0]:
        ids = w.ids[s * 128:(s + 1) * 128]
        assert len(set(ids.tolist())) == 128 and ids.min() >= 0 and ids.max() < spec.V


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.01171875, 1.0 + 2**-9, -2.5, 3.0e38], np.float32)
    b = synth.bf16_bits(vals)
    back = synth.bf16_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.015625
    assert back[3] == 1.0 and back[4] == -2.5
    assert np.isfinite(back[5]) or back[5] == np.inf


def test_algorithmic_bytes_formula():
    spec = synth.CONFIGS["C3"].with_(capacity=4)
    w = synth.make(spec)
    rows = w.active_rows()
    assert w.algorithmic_bytes() == rows * (spec.V * 2 + 4 + 4 * 42) + 12 * 4
