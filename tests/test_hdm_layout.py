"""Head-dim-major tiles (the forward's V copy), on the compiled layout
functions (csrc/cowa_layout.h built for the host by tests/host_shim.cpp).

The copy holds one row per head dim; inside each group of 16 keys, position q
holds key tr16_position(q).  A lane's P.V operand is one 16-byte read of
8 positions, and the MFMA sums over k = 8 * (lane / 32) + m, m = 0..7.  The
B operand (P) that the same lane supplies comes from the first product's
accumulator, whose layout is the documented 32x32 MFMA one: register i of a
lane holds row 8 * (i / 4) + 4 * (lane / 32) + i % 4 (rows = keys here, in
blocks of 32), converted to bf16 in pairs, 8 registers per 16-key step.  The
two must agree key for key, or P.V sums the wrong products."""

import numpy as np
import pytest

from tests import host_shim
from tests.test_lds_swizzle import conflicts


def mfma_acc_row(lane, i):
    """Row of accumulator register i (0..15) of a 32x32 MFMA for a lane."""
    return 8 * (i // 4) + 4 * (lane // 32) + i % 4


def p_operand_key(st, lane, m):
    """Key (0..63 in the tile) of element m of a lane's P operand at 16-key
    step st: register 8 * (st % 2) + m of accumulator block st // 2."""
    return 32 * (st // 2) + mfma_acc_row(lane, 8 * (st % 2) + m)


def test_tr16_position_is_an_involution_of_each_group():
    lib = host_shim.load()
    pos = [lib.shim_tr16_position(q) for q in range(16)]
    assert sorted(pos) == list(range(16))
    assert all(lib.shim_tr16_position(pos[q]) == q for q in range(16))


@pytest.mark.parametrize("d", [64, 128])
def test_operand_reads_hold_the_keys_of_the_p_operand(d):
    """Simulate a tile: direct loads place the copy's chunks in LDS, each
    lane reads its 8 positions; every element must be V[key][dim] with key
    the one the lane's P operand holds at the same k index."""
    lib = host_shim.load()
    rng = np.random.default_rng(3)
    V = rng.integers(1, 1 << 15, size=(64, d))  # V[key][dim], distinct-ish values
    copy = np.zeros((d, 64), np.int64)  # copy[dim][position]
    for q in range(64):
        copy[:, q] = V[16 * (q // 16) + lib.shim_tr16_position(q % 16), :]
    lds = np.full(d * 64, -1, np.int64)
    for P in range(d * 8):
        row, chunk = lib.shim_hdm_load_row(P), lib.shim_hdm_load_chunk(P)
        lds[8 * P: 8 * P + 8] = copy[row, 8 * chunk: 8 * chunk + 8]
    assert (lds >= 0).all()
    for lane in range(64):
        off = host_shim.int_array(4 * (d // 32))
        lib.shim_hdm_read_offsets(d, lane, off)
        for db in range(d // 32):
            dim = 32 * db + lane % 32
            for st in range(4):
                got = lds[off[4 * db + st]: off[4 * db + st] + 8]
                want = [V[p_operand_key(st, lane, m), dim] for m in range(8)]
                assert list(got) == want, (d, lane, db, st)


@pytest.mark.parametrize("d", [64, 128])
def test_operand_reads_are_conflict_free(d):
    lib = host_shim.load()
    offs = []
    for lane in range(64):
        a = host_shim.int_array(4 * (d // 32))
        lib.shim_hdm_read_offsets(d, lane, a)
        offs.append(list(a))
    for B in (128, 256):
        for i in range(4 * (d // 32)):
            assert conflicts([2 * offs[l][i] for l in range(64)], 16, B) == 0
    # the model is not vacuous: without the swizzle these reads conflict
    plain = [2 * ((l % 32) * 64 + 8 * (l // 32)) for l in range(64)]
    assert conflicts(plain, 16, 128) > 0


def test_loads_fill_every_position_once():
    lib = host_shim.load()
    for d in (64, 128):
        seen = set()
        for P in range(d * 8):
            seen.add((lib.shim_hdm_load_row(P), lib.shim_hdm_load_chunk(P)))
        assert seen == {(r, c) for r in range(d) for c in range(8)}
