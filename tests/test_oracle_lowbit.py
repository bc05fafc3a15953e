"""Pins of the oracle's E4M3 cache format (oracle/lowbit.py) against the OCP
8-bit floating point definition: hand-decoded codes, monotonicity and the
finite-value count, round trips, ties to even, saturation, the relative error
bound of a 3-bit mantissa, and nearest-value search by brute force; and the
low-bit layer step against the plain one."""
import numpy as np
import pytest

import oracle as O
from io_aware_kv_amd import workloads as W


def test_hand_decoded_codes():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x50: 8.0, 0x77: 240.0, 0x78: 256.0,
             0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, val in cases.items():
        assert O.e4m3_decode([code])[0] == val, hex(code)
    assert np.isnan(O.e4m3_decode([0x7F])[0]) and np.isnan(O.e4m3_decode([0xFF])[0])
    z = O.e4m3_decode([0x80])[0]
    assert z == 0.0 and np.signbit(z)


def test_finite_values_increase_with_the_code():
    v = O.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(v) > 0) and len(v) == 127 and v[-1] == O.E4M3_MAX
    assert np.array_equal(O.e4m3_decode(np.arange(0x80, 0xFF)), -v)


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


def test_ties_go_to_the_even_code():
    pairs = {1.0625: 0x38, 1.1875: 0x3A, 0.5 * 2.0 ** -9: 0x00, 1.5 * 2.0 ** -9: 0x02, 2.5 * 2.0 ** -9: 0x02,
             3.5 * 2.0 ** -9: 0x04, 2.125: 0x40, 400.0: 0x7C, 432.0: 0x7E, -1.0625: 0xB8}
    for x, code in pairs.items():
        assert O.e4m3_encode([x])[0] == code, x
    # just off a tie goes to the nearer neighbour
    assert O.e4m3_encode([1.0625 + 1e-12])[0] == 0x39
    assert O.e4m3_encode([1.0625 - 1e-12])[0] == 0x38


def test_saturation_and_signed_zero():
    assert list(O.e4m3_encode([448.0, 460.0, 1e6, -1e6, -449.0])) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert list(O.e4m3_encode([0.0, -0.0, -1e-9, 1e-9])) == [0x00, 0x80, 0x80, 0x00]
    with pytest.raises(ValueError):
        O.e4m3_encode([np.nan])


def test_relative_error_bound_and_nearest_by_brute_force():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 50, 5000), rng.uniform(-2e-3, 2e-3, 5000)])
    r = O.e4m3_round(x)
    normal = (np.abs(x) >= 2.0 ** -6) & (np.abs(x) <= O.E4M3_MAX)
    assert np.all(np.abs(r - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    assert np.all(np.abs(r - x)[np.abs(x) < 2.0 ** -6] <= 2.0 ** -10)
    table = np.concatenate([O.e4m3_decode(np.arange(0x7F)), -O.e4m3_decode(np.arange(1, 0x7F))])
    for xi, ri in zip(x[:3000], r[:3000]):
        d = np.abs(table - xi)
        assert abs(ri - xi) == d.min()


def test_low_bit_layer_step_stores_rounded_rows():
    """The e4m3 layer step writes exactly the rounded rows of the plain step
    (same projection and rotation), its attention reads them, and its output
    stays close to the plain one (the stored values move by at most 1/16)."""
    wl = W.make_workload("tiny_f32")
    sh = wl.shape
    table = O.build_block_table(wl.seq_pages, wl.pool_perm, wl.pool_pages, wl.max_pages)
    rows = W.full_refresh_rows(wl)
    x = W.as_f64(wl, W.activations(wl, rows, 0))
    w = W.as_f64(wl, W.weights(wl, 0))
    n = sh.n_heads * sh.head_dim
    zero = np.zeros((wl.pool_pages * W.PAGE, n))
    args = (x, w, rows.pos, rows.logical, rows.cu_q, rows.kv_len, rows.mass_count, zero, zero.copy(), table,
            sh.n_heads, sh.head_dim, sh.rope_base, W.PAGE)
    plain = O.layer_step(*args)
    low = O.layer_step(*args, kv_format="e4m3")
    np.testing.assert_array_equal(low["k"], O.e4m3_round(plain["k"]))
    np.testing.assert_array_equal(low["v"], O.e4m3_round(plain["v"]))
    np.testing.assert_array_equal(low["q"], plain["q"])
    np.testing.assert_array_equal(low["k_cache"][low["slots"]], low["k"])
    # attention over the stored values: recompute it from the low-bit cache
    o2, _ = O.attention(low["q"], low["k_cache"], low["v_cache"], table, rows.cu_q, rows.kv_len, sh.n_heads,
                        sh.head_dim, W.PAGE)
    np.testing.assert_allclose(low["o"], o2, rtol=1e-12, atol=1e-14)
    assert 0 < np.abs(low["o"] - plain["o"]).max() < 0.1
    with pytest.raises(O.OracleError):
        O.layer_step(*args, kv_format="int4")
