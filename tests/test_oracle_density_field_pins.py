"""Pins of the density-field codec oracle (oracle/density_field.py) that do not come
from the oracle itself (CPU only).

  * closed forms: a row of +s gives all cells 1 and reads back +s; -s gives all 0 and
    -s; an all-zero row has density 1/2, so the modulator alternates 1, 0, 1, 0 (two
    cells per value) and reads back 0; density 1/4 gives one 1 per value;
  * the exact form of a first-order sigma-delta: with the running sum S_c of the
    densities of cells 0 .. c - 1, the number of ones among those cells is
    floor(S_c + 1/2), so cell c is floor(S_{c+1} + 1/2) - floor(S_c + 1/2).  For
    densities that are multiples of 1/64 every fp32 step is exact, and the oracle's
    cells must equal that formula computed here with integers;
  * the error bound on random rows: every prefix of cells holds floor-or-ceil of its
    density sum (|ones - S_c| <= 1/2 up to fp32 rounding), so each value reads back
    within s / 2 of the input, and any run of consecutive values within s / 2 in total;
  * scaling a row by 2^j scales s by 2^j and leaves the cells unchanged;
  * the bit layout: cell c is bit c % 32 of word c // 32 (numpy's little-endian bit
    order), so value n is nibble n % 8 of word n // 8.
"""
import numpy as np
import pytest

from oracle import density_field as dfc


def test_field_side():
    assert dfc.field_side(128) == 23 and 23 * 23 >= 512 > 22 * 22
    assert dfc.field_side(64) == 16 and dfc.field_side(256) == 32


def test_constant_and_zero_rows():
    d = 128
    rows = np.stack([np.full(d, 3.5, np.float32), np.full(d, -0.25, np.float32), np.zeros(d, np.float32)])
    f, s = dfc.encode(rows)
    assert s.tolist() == [3.5, 0.25, 0.0]
    assert (f[0] == 0xFFFFFFFF).all() and (f[1] == 0).all()
    assert (f[2] == 0x55555555).all()            # 1, 0, 1, 0, ... : bit 0 set in each pair
    v = dfc.decode(f, s, d)
    np.testing.assert_array_equal(v[0], 3.5)
    np.testing.assert_array_equal(v[1], -0.25)
    np.testing.assert_array_equal(v[2], 0.0)


def test_quarter_density_gives_one_cell_per_value():
    # u = 1/4 for every value: v = s (2 u - 1) = -s / 2, one row element at +s sets the scale
    d = 64
    row = np.full(d, -1.0, np.float32)
    row[0] = 2.0                                  # s = 2, u = 1/4 elsewhere, 1 at value 0
    f, s = dfc.encode(row[None])
    cells = np.unpackbits(f.view(np.uint8), bitorder="little").reshape(d, 4)
    assert cells[0].sum() == 4
    assert (cells[1:].sum(axis=1) == 1).all()
    np.testing.assert_array_equal(dfc.decode(f, s, d)[0, 1:], -1.0)


def _prefix_form(k, d):
    """Cells from the closed form, densities u = k / 64 (integers k in [0, 64])."""
    u64 = np.repeat(k.astype(np.int64), 4)                  # density x 64 per cell
    S = np.concatenate([[0], np.cumsum(u64)])               # 64 x running sums
    ones = (2 * S + 64) // 128                              # floor(S / 64 + 1/2)
    return np.diff(ones).astype(np.uint8)


@pytest.mark.parametrize("seed", range(6))
def test_dyadic_densities_match_the_prefix_form(seed):
    rng = np.random.default_rng(seed)
    d = 128
    k = rng.integers(0, 65, d)
    k[rng.integers(0, d)] = 64 if seed % 2 else 0     # the absmax element: density 1 or 0
    v = ((2 * k - 64) / 64.0).astype(np.float32)      # s = 1 exactly, u = k / 64 exactly
    if np.abs(v).max() != 1.0:
        v[0] = 1.0
        k[0] = 64
    f, s = dfc.encode(v[None])
    assert s[0] == 1.0
    cells = np.unpackbits(f.view(np.uint8), bitorder="little")
    np.testing.assert_array_equal(cells, _prefix_form(k, d))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_error_bound_on_random_rows(d):
    rng = np.random.default_rng(d)
    x = (rng.standard_normal((200, d)) * rng.uniform(1e-3, 1e3, (200, 1))).astype(np.float32)
    f, s = dfc.encode(x)
    cells = np.unpackbits(f.view(np.uint8), axis=1, bitorder="little")[:, :4 * d].astype(np.int64)
    u = (x.astype(np.float64) / s[:, None] + 1) / 2
    S = np.concatenate([np.zeros((200, 1)), np.cumsum(np.repeat(u, 4, axis=1), axis=1)], axis=1)
    ones = np.concatenate([np.zeros((200, 1)), np.cumsum(cells, axis=1)], axis=1)
    assert (np.abs(ones - S) <= 0.5 + 1e-4).all()
    v = dfc.decode(f, s, d).astype(np.float64)
    err = v - x
    assert (np.abs(err) <= s[:, None] * (0.5 + 1e-4)).all()
    run = np.cumsum(err, axis=1)                              # any prefix of values
    assert (np.abs(run) <= s[:, None] * (0.5 + 1e-3)).all()


def test_power_of_two_scaling():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((20, 128)).astype(np.float32)
    f0, s0 = dfc.encode(x)
    for j in (-3, 5):
        f1, s1 = dfc.encode(x * np.float32(2.0 ** j))
        np.testing.assert_array_equal(f0, f1)
        np.testing.assert_array_equal(s1, s0 * np.float32(2.0 ** j))


def test_bit_layout():
    d = 16
    row = np.full(d, -1.0, np.float32)
    row[5] = 1.0                                  # value 5: all four cells 1, others 0
    f, s = dfc.encode(row[None])
    assert f.shape == (1, 2)
    assert f[0, 0] == 0x00F00000 and f[0, 1] == 0   # nibble 5 of word 0
