"""Host check of the chunked XCD workgroup order (mirrors xcd_chunk and
xcd_grid of csrc/cowa_internal.h and xcd_logical of csrc/kernel_util.h):
over the padded grid every logical workgroup runs exactly once, padding
workgroups are the only ones dropped, and each chunk of consecutive logical
workgroups runs on a single XCD, the rounds of eight chunks alternating their
direction over the XCDs."""

import numpy as np
import pytest

XCDS = 8


def xcd_chunk(per_unit, units, max_units):
    fill = (32 + per_unit - 1) // per_unit
    spread = units // (16 * XCDS)
    k = min(spread, max_units)
    k = max(k, fill)
    k = min(k, max_units)
    return per_unit * max(k, 1)


def xcd_grid(total, chunk):
    span = XCDS * chunk
    return (total + span - 1) // span * span


def xcd_logical(i, chunk, total):
    xcd = i % XCDS
    r = i // XCDS
    j = r // chunk
    c = np.where(j & 1, XCDS - 1 - xcd, xcd)
    lg = (j * XCDS + c) * chunk + (r - j * chunk)
    return np.where(lg < total, lg, -1)


SHAPES = [(5, 512, 8), (40, 128, 8), (64, 32, 8), (1, 1028, 8), (8, 258, 8), (320, 123, 8),
          (1, 1, 8), (3, 7, 8), (7, 1000, 8), (2, 4097, 8)]


@pytest.mark.parametrize("per_unit,units,max_units", SHAPES)
def test_xcd_order_is_a_bijection_with_one_xcd_per_chunk(per_unit, units, max_units):
    total = per_unit * units
    chunk = xcd_chunk(per_unit, units, max_units)
    assert per_unit <= chunk <= max_units * per_unit and chunk % per_unit == 0
    grid = xcd_grid(total, chunk)
    i = np.arange(grid)
    lg = xcd_logical(i, chunk, total)
    assert np.array_equal(np.sort(lg[lg >= 0]), np.arange(total))
    c = lg[lg >= 0] // chunk
    want = np.where((c // XCDS) % 2 == 0, c % XCDS, XCDS - 1 - c % XCDS)
    assert np.array_equal(i[lg >= 0] % XCDS, want)


def test_xcd_chunk_sizes_of_the_workloads():
    # prefill at the 128K rank (5 heads, 512 tiles of 256 rows): 7 query tiles
    # per chunk fill one XCD's 32 compute units; at 32K (40 heads) one tile does
    assert xcd_chunk(5, 512, 8) == 35
    assert xcd_chunk(40, 128, 8) == 40
    # long sequences with few heads get more units per chunk, up to the cap
    assert xcd_chunk(1, 1 << 16, 8) == 8


@pytest.mark.parametrize("total", [1, 255, 256, 2560, 5120, 2049, 10007])
def test_xcd_order_any_chunk_size(total):
    # the host may pick any chunk from 32 to 64 workgroups (balanced against
    # the plan's row lengths): the order stays a bijection for every size
    for chunk in range(32, 65):
        grid = xcd_grid(total, chunk)
        i = np.arange(grid)
        lg = xcd_logical(i, chunk, total)
        assert np.array_equal(np.sort(lg[lg >= 0]), np.arange(total))
