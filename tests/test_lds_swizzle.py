"""Bank-conflict model of the backward kernels' LDS tiles (host only).

The dQ and dK/dV kernels keep row-major [rows x d] bf16 tiles in LDS with the
16-byte chunks of each row XOR-swizzled by swz(row), and read them two ways:
16-byte reads of one chunk column by 32 consecutive rows (the plain A operand)
and 8-byte transposing reads of 4 consecutive rows x 2 adjacent chunks (the
transposed A operand).  The swizzles below mirror swz_both_d128 and
swz_both<64> of csrc/kernel_util.h, and the lane patterns mirror plain_offsets
and tr_offsets of csrc/bwd.hip.  A read instruction is modelled as served in
groups of consecutive lanes moving B bytes per cycle (B = 128 or 256); a
conflict is two lanes of one group touching the same 4-byte bank slot at
different addresses."""

import pytest


def swz128(row):
    a = row & 3
    return (((a << 2) ^ (a << 1)) & 14) ^ ((row >> 2) & 3)


def swz(d):
    return swz128 if d == 128 else (lambda row: swz128(row) & 7)


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


def read_patterns(d, sw):
    nk, nd = d // 16, d // 32
    for blk in range(2):  # plain: row 32 blk + lane % 32, chunk 2 ks + lane / 32
        for ks in range(nk):
            yield 16, [((32 * blk + (l & 31)) * d + ((2 * ks + (l >> 5)) ^ sw(l & 31)) * 8) * 2
                       for l in range(64)]
    for st in range(4):  # transposing: 4 rows x 2 chunks per 16 lanes
        for ri in range(2):
            for db in range(nd):
                addrs = []
                for l in range(64):
                    row = 16 * st + 8 * ri + 4 * (l >> 5) + ((l & 15) >> 2)
                    dd = 32 * db + 16 * ((l >> 4) & 1) + 4 * (l & 3)
                    addrs.append((row * d + ((dd >> 3) ^ sw(row)) * 8 + (dd & 7)) * 2)
                yield 8, addrs


@pytest.mark.parametrize("d", [64, 128])
def test_backward_swizzle_is_a_permutation_and_conflict_free(d):
    sw = swz(d)
    cpr = d // 8
    for row in range(64):
        assert sorted(c ^ sw(row) for c in range(cpr)) == list(range(cpr))
    for B in (128, 256):
        for width, addrs in read_patterns(d, sw):
            assert conflicts(addrs, width, B) == 0


def test_unswizzled_tiles_would_conflict():
    # the model is not vacuous: without the swizzle both patterns conflict
    for d in (64, 128):
        total = sum(conflicts(a, w, 128) for w, a in read_patterns(d, lambda row: 0))
        assert total > 0
