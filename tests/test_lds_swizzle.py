"""Bank-conflict model of the kernels' LDS tiles, on the compiled layout
functions (csrc/cowa_layout.h built for the host by tests/host_shim.cpp).

Tiles are row-major [rows x d] bf16 with the 16-byte chunks of each row
XOR-swizzled by swz_both(row).  They are read two ways: 16-byte reads of one
chunk column by 32 consecutive rows (plain_offsets, the plain A operand) and
8-byte transposing reads of 4 consecutive rows x 2 adjacent chunks
(tr_offsets, the transposed A operand).  A read instruction is modelled as
served in groups of consecutive lanes moving B bytes per cycle (B = 128 or
256); a conflict is two lanes of one group touching the same 4-byte bank slot
at different addresses."""

import pytest

from tests import host_shim


def conflicts(addrs, width, B):
    n = 0
    per = B // width
    for g in range(0, 64, per):
        seen = {}
        for lane in range(g, g + per):
            for w in range(width // 4):
                word = addrs[lane] // 4 + w
                bank = word % (B // 4)
                if bank in seen and seen[bank] != word:
                    n += 1
                seen[bank] = word
    return n


def lane_offsets(fn, d, n):
    lib = host_shim.load()
    out = []
    for lane in range(64):
        a = host_shim.int_array(n)
        getattr(lib, fn)(d, lane, a)
        out.append(list(a))
    return out


def read_patterns(d):
    """(width in bytes, 64 byte addresses) of every read instruction of a tile
    step: the plain reads (row blocks x k steps) and the transposing reads
    (4 k steps of 16 rows x halves x head-dim blocks)."""
    nk, nd = d // 16, d // 32
    plain = lane_offsets("shim_plain_offsets", d, 2 * nk)
    for i in range(2 * nk):
        yield 16, [2 * plain[l][i] for l in range(64)]
    tr = lane_offsets("shim_tr_offsets", d, 2 * nd)
    for st in range(4):
        for i in range(2 * nd):
            yield 8, [2 * (tr[l][i] + 16 * d * st) for l in range(64)]


@pytest.mark.parametrize("d", [64, 128])
def test_swizzle_is_a_permutation_and_reads_are_conflict_free(d):
    lib = host_shim.load()
    cpr = d // 8
    for row in range(64):
        assert sorted(c ^ lib.shim_swz_both(d, row) for c in range(cpr)) == list(range(cpr))
    for B in (128, 256):
        for width, addrs in read_patterns(d):
            assert conflicts(addrs, width, B) == 0


@pytest.mark.parametrize("d", [64, 128])
def test_loads_place_what_the_reads_expect(d):
    """Direct global->LDS loads put global chunk load_col(P) / 8 of row
    load_row(P) at 16-byte position P; a plain read of that row and chunk
    (plain_offsets' formula, row block 0, k step chunk / 2) lands on P."""
    lib = host_shim.load()
    cpr = d // 8
    plain = lane_offsets("shim_plain_offsets", d, d // 8)
    for P in range(64 * cpr):
        row, chunk = lib.shim_load_row(d, P), lib.shim_load_col(d, P) // 8
        if row >= 32:
            continue
        hl, ks = chunk % 2, chunk // 2
        lane = row + 32 * hl
        assert plain[lane][ks] == 8 * P, (P, row, chunk)


def test_unswizzled_tiles_would_conflict():
    # the model is not vacuous: without the swizzle the plain reads conflict
    for d in (64, 128):
        addrs = [2 * ((l & 31) * d + (l >> 5) * 8) for l in range(64)]
        assert conflicts(addrs, 16, 128) > 0
