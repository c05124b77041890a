"""CPU oracle of the density-field state codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product path never imports it, and it
never imports the product path.

DF-SSM technical summary (gist.science), section 2D "Density Field State
Representation": the SSM hidden state is compressed into a K x K binary field per
state element, with K^2 about 4 d_state; the cycle is normalization, sigma-delta
injection (error feedback), binarization, and a popcount readout that recovers
continuous values, applied at chunk boundaries.  The page gives no formulas; the
readings taken (the plainest ones the passage supports):

  * "state element" is one row of the state, its d_state values (one channel of one
    head): a field per scalar would hold ~4 d_state bits for one value and compress
    nothing.  K = ceil(sqrt(4 d_state)) (23 for d_state 128: 529 cells); value n owns
    the 4 consecutive cells 4 n .. 4 n + 3 in row-major order, and the K^2 - 4 d_state
    cells left over are 0 (they carry nothing and are not stored).
  * normalization: s = max_n |v_n| (the row's absmax, kept in fp32); the density of
    value n is u_n = (v_n / s + 1) / 2 in [0, 1] (fp32: an IEEE division, an add, and
    an exact halving); an all-zero row has s = 0 and u_n = 1/2.
  * sigma-delta injection and binarization: a first-order modulator runs over the
    cells in order with one fp32 error e (0 at the row's start): for each cell of
    value n, w = u_n + e, the cell is 1 if w >= 1/2 else 0, and e = w - cell (the
    residual injected into the next cell; exact, by Sterbenz's lemma).
  * popcount readout: v_n = s (2 popcount(cells of n) / 4 - 1), i.e. s times one of
    -1, -1/2, 0, 1/2, 1 (exact in fp32).
  * "at chunk boundaries": the codec maps a state to its field and back; how many
    tokens a chunk spans is the caller's choice, not the codec's.

Storage: the 4 d_state cells of a row, 32 per uint32 word (cell c in bit c % 32 of word
c // 32, so value n is nibble n % 8 of word n // 8), and s as fp32.

Parity status: pinned by ``tests/test_oracle_density_field_pins.py`` -- closed forms
(constant rows, an all-zero row), the exact prefix-sum form of a first-order
sigma-delta on inputs whose densities are dyadic (computed there with integers), the
modulator's error bound on random rows, power-of-two scale invariance, and the bit
layout against numpy's bit unpacking.
"""
from __future__ import annotations

import math

import numpy as np

CELLS = 4  # cells per state value


def field_side(d_state: int) -> int:
    """K: the smallest side with K^2 >= 4 d_state."""
    return math.isqrt(CELLS * d_state - 1) + 1


def encode(state):
    """state fp32 [R, d] -> (field uint32 [R, d / 8], scale fp32 [R]).  Rows are
    independent; the modulator runs over each row's cells in order."""
    v = np.ascontiguousarray(state, dtype=np.float32)
    R, d = v.shape
    assert d % 8 == 0
    s = np.abs(v).max(axis=1).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        a = np.where(s[:, None] > 0, v / np.where(s > 0, s, np.float32(1))[:, None], np.float32(0))
    a = a.astype(np.float32)
    u = ((a + np.float32(1)) * np.float32(0.5)).astype(np.float32)        # density in [0, 1]
    cells = np.zeros((R, CELLS * d), np.uint8)
    e = np.zeros(R, np.float32)
    half = np.float32(0.5)
    for c in range(CELLS * d):
        w = (u[:, c // CELLS] + e).astype(np.float32)                       # inject the residual
        bit = w >= half                                                     # binarize
        cells[:, c] = bit
        e = (w - bit.astype(np.float32)).astype(np.float32)                 # carry the error
    field = np.packbits(cells, axis=1, bitorder="little").view(np.uint32).reshape(R, d // 8)
    return field, s


def decode(field, scale, d: int):
    """(field uint32 [R, d / 8], scale fp32 [R]) -> state fp32 [R, d]: popcount readout."""
    field = np.ascontiguousarray(field, dtype=np.uint32)
    R = field.shape[0]
    cells = np.unpackbits(field.view(np.uint8).reshape(R, -1), axis=1, bitorder="little")[:, :CELLS * d]
    pc = cells.reshape(R, d, CELLS).sum(axis=2).astype(np.float32)           # popcount per value
    level = (pc * np.float32(2.0 / CELLS) - np.float32(1)).astype(np.float32)
    return (np.asarray(scale, np.float32)[:, None] * level).astype(np.float32)


def requantize(state):
    """The round trip a chunk boundary applies: (state', field, scale)."""
    field, s = encode(state)
    return decode(field, s, np.asarray(state).shape[1]), field, s
