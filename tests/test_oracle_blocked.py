"""Pins of the oracle's 128x4 blocked scale layout (an index permutation) to the pages.

The oracle writes the offset as one closed formula.  These tests derive it a second way,
with a generic evaluator of hierarchical (shape, stride) layouts applied to the scale atom
of the page "kernelindex submission 402102" (shape ((32, 4), (16, 4)), stride ((16, 4),
(0, 1)): rows split as r % 32 + 32 * ((r / 32) % 4), K as kk % 16 + 16 * ((kk / 16) % 4),
the 16 K values of one scale sharing a byte), and placing the atoms as the producer of the
page "kernelindex submission 498317" addresses its 512-byte scale blocks: (row / 128)
times the K / 64 blocks of a row block, plus kk / 64.  They also check that the map is a
permutation of the padded buffer, spot values that follow from the two definitions, and
the padding fill.
"""
import numpy as np
import pytest

import oracle


def layout_eval(shape, stride, coord):
    """Offset of a hierarchical layout: shape/stride/coord are nested tuples of equal
    structure; leaves contribute coord * stride."""
    if isinstance(shape, tuple):
        return sum(layout_eval(s, d, c) for s, d, c in zip(shape, stride, coord))
    assert 0 <= coord < shape
    return coord * stride


def split(x, shape):
    """Colexicographic split of a flat index x over a (possibly nested) shape tuple."""
    if not isinstance(shape, tuple):
        return x
    out = []
    for s in shape:
        size = int(np.prod(flat(s)))
        out.append(split(x % size, s))
        x //= size
    return tuple(out)


def flat(s):
    return [s] if not isinstance(s, tuple) else [v for e in s for v in flat(e)]


ATOM_SHAPE = ((32, 4), (16, 4))
ATOM_STRIDE = ((16, 4), (0, 1))


def offset_from_pages(r, kk, k):
    in_atom = layout_eval(ATOM_SHAPE, ATOM_STRIDE, (split(r % 128, (32, 4)), split(kk % 64, (16, 4))))
    atom = (r // 128) * (k // 16 // 4) + kk // 64
    return atom * 512 + in_atom


@pytest.mark.parametrize("rows,k", [(1, 256), (127, 256), (128, 512), (129, 256), (300, 512), (64, 1536)])
def test_offsets_match_the_layout_algebra(rows, k):
    for r in range(rows):
        for kk in range(0, k, 4):
            assert oracle.blocked_offset(r, kk // 16, k) == offset_from_pages(r, kk, k), (r, kk)


@pytest.mark.parametrize("rows,k", [(128, 256), (256, 512), (384, 1024)])
def test_permutation_of_the_padded_buffer(rows, k):
    offs = [oracle.blocked_offset(r, c, k) for r in range(rows) for c in range(k // 16)]
    assert sorted(offs) == list(range(oracle.blocked_bytes(rows, k)))


def test_spot_values():
    k = 512                      # 8 atoms per 128-row block
    assert oracle.blocked_offset(0, 0, k) == 0
    assert oracle.blocked_offset(1, 0, k) == 16       # next row: stride 16
    assert oracle.blocked_offset(31, 0, k) == 496
    assert oracle.blocked_offset(32, 0, k) == 4       # row 32 starts the second group of 4
    assert oracle.blocked_offset(96, 0, k) == 12
    assert oracle.blocked_offset(0, 1, k) == 1        # next K block: stride 1
    assert oracle.blocked_offset(0, 3, k) == 3
    assert oracle.blocked_offset(0, 4, k) == 512      # fifth K block: next atom
    assert oracle.blocked_offset(127, 31, k) == 7 * 512 + 16 * 31 + 4 * 3 + 3
    assert oracle.blocked_offset(128, 0, k) == 8 * 512
    assert oracle.blocked_bytes(1, k) == 8 * 512
    assert oracle.blocked_bytes(128, k) == 8 * 512
    assert oracle.blocked_bytes(129, k) == 16 * 512
    assert oracle.blocked_bytes(0, k) == 0


@pytest.mark.parametrize("rows,k", [(1, 256), (200, 512), (129, 768)])
def test_conversion_round_trip_and_padding(rows, k):
    rng = np.random.default_rng(rows * 7 + k)
    src = rng.integers(0, 256, size=(rows, k // 16), dtype=np.uint8)
    dst = oracle.scales_to_blocked(src, k, pad=0xA5)
    assert dst.size == oracle.blocked_bytes(rows, k)
    got = np.empty_like(src)
    used = np.zeros(dst.size, dtype=bool)
    for r in range(rows):
        for c in range(k // 16):
            o = offset_from_pages(r, 16 * c, k)
            got[r, c] = dst[o]
            used[o] = True
    assert np.array_equal(got, src)
    assert np.all(dst[~used] == 0xA5)


def test_conversion_of_zero_rows():
    assert oracle.scales_to_blocked(np.zeros((0, 16), dtype=np.uint8), 256).size == 0


def test_conversion_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.scales_to_blocked(np.zeros((4, 3), dtype=np.uint8), 256)
