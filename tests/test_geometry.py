"""Host-side checks of the tile enumeration the kernels use (no GPU).

The library exports its geometry (the same header the kernels compile) as
plain C functions; these tests compare it with the oracle's explicit mask
by brute force.  Properties (Fast Diffusion Attention, "Visit only the
visible tiles"): every visible pair lies in a visited tile, visited tiles
never straddle the halves, "unmasked" tiles are entirely visible, "masked"
tiles hold both visible and invisible pairs, and the backward enumeration
is exactly the transpose of the forward one.
"""
import itertools

import numpy as np
import pytest

import oracle
import block_diffusion_lm_amd as bd

DIFF, CAUSAL = bd.MODE_DIFFUSION, bd.MODE_CAUSAL


def _mask(mode, n, b):
    if mode == DIFF:
        return oracle.block_diffusion_mask(n, b)
    return oracle.causal_mask(n)


def _halves(mode):
    return (bd.NOISY, bd.CLEAN) if mode == DIFF else (bd.CLEAN,)


def _off(mode, n, half):
    return n if (mode == DIFF and half == bd.CLEAN) else 0


def _check(mode, n, b, tm, tn):
    M = _mask(mode, n, b)
    fwd_pairs = set()
    for qh in _halves(mode):
        for qt in range(-(-n // tm)):
            r0, r1 = qt * tm, min(qt * tm + tm, n)
            rows = slice(_off(mode, n, qh) + r0, _off(mode, n, qh) + r1)
            tiles = bd.bdattn_fwd_tiles(mode, n, b, tm, tn, qh, qt)
            covered = np.zeros(M.shape[1], dtype=bool)
            seen = set()
            for kh, kt, masked in tiles:
                assert kh in _halves(mode)
                assert (kh, kt) not in seen
                seen.add((kh, kt))
                c0, c1 = kt * tn, min(kt * tn + tn, n)
                assert 0 <= c0 < n
                cols = slice(_off(mode, n, kh) + c0, _off(mode, n, kh) + c1)
                block = M[rows, cols]
                assert block.any(), "visited tile with no visible pair"
                assert bool(masked) == (not block.all()), (qh, qt, kh, kt, masked)
                covered[cols] = True
                fwd_pairs.add((qh, qt, kh, kt, masked))
            # every visible key of these rows lies in a visited tile
            assert not (M[rows] & ~covered[None, :]).any()
    bwd_pairs = set()
    for kh in _halves(mode):
        for kt in range(-(-n // tn)):
            for qh, qt, masked in bd.bdattn_bwd_tiles(mode, n, b, tm, tn, kh, kt):
                bwd_pairs.add((qh, qt, kh, kt, masked))
    assert fwd_pairs == bwd_pairs


SIZES = [1, 2, 7, 33, 100, 129, 300]
BLOCKS = [1, 2, 3, 5, 16, 48, 64, 127, 128, 200]


@pytest.mark.parametrize("n", SIZES)
def test_diffusion_tiles_bruteforce(n):
    for b in sorted(set(BLOCKS + [n, n + 5])):
        for tm, tn in ((128, 64), (64, 128), (32, 32), (128, 128)):
            _check(DIFF, n, b, tm, tn)


@pytest.mark.parametrize("n", SIZES)
def test_causal_tiles_bruteforce(n):
    for tm, tn in ((128, 64), (64, 128), (32, 32)):
        _check(CAUSAL, n, 1, tm, tn)


@pytest.mark.parametrize("n,b", list(itertools.product([5, 12, 37], [1, 3, 4, 12, 40])))
def test_row_intervals_match_mask(n, b):
    M = oracle.block_diffusion_mask(n, b)
    for qh in (bd.NOISY, bd.CLEAN):
        for p in range(n):
            row = M[_off(DIFF, n, qh) + p]
            for kh in (bd.NOISY, bd.CLEAN):
                lo, hi = bd.bdattn_row_interval(DIFF, n, b, qh, p, kh)
                seg = row[_off(DIFF, n, kh):_off(DIFF, n, kh) + n]
                want = np.zeros(n, dtype=bool)
                want[lo:hi] = True
                assert np.array_equal(seg, want), (qh, p, kh, lo, hi)


def test_visible_pairs_against_mask_and_closed_form():
    for n in (1, 4, 9, 64, 130):
        for b in (1, 2, 3, 8, 64, 200):
            assert bd.bdattn_visible_pairs(DIFF, n, b) == int(oracle.block_diffusion_mask(n, b).sum())
            if n % b == 0:
                assert bd.bdattn_visible_pairs(DIFF, n, b) == n * n + n * b
        assert bd.bdattn_visible_pairs(CAUSAL, n, 1) == n * (n + 1) // 2
    # the full-size workloads, against the page's closed form
    assert bd.bdattn_visible_pairs(DIFF, 8192, 32) == 8192 ** 2 + 8192 * 32


def test_noisy_diagonal_extra_work_is_small():
    """Fast Diffusion Attention, "Visit only the visible tiles": beyond causal
    attention on the halves, a noisy query tile visits one extra key tile,
    about 5% more tiles with halves of 2K tokens and about 1% at 16K
    (128x128 tiles; "tokens" read as the half length n)."""
    def tiles(mode, n, b):
        return sum(len(bd.bdattn_fwd_tiles(mode, n, b, 128, 128, qh, qt))
                   for qh in _halves(mode) for qt in range(-(-n // 128)))
    for n, b, bound in ((2048, 16, 0.065), (16384, 32, 0.01)):
        qtiles = -(-n // 128)
        assert tiles(DIFF, n, b) == 2 * tiles(CAUSAL, n, 1) + qtiles
        extra = tiles(DIFF, n, b) / (2 * tiles(CAUSAL, n, 1)) - 1
        assert 0 < extra < bound, (n, extra)


def test_geometry_rejects_bad_arguments():
    with pytest.raises(ValueError):
        bd.bdattn_fwd_tiles(DIFF, 0, 1, 128, 64, 0, 0)
    with pytest.raises(ValueError):
        bd.bdattn_fwd_tiles(DIFF, 100, 0, 128, 64, 0, 0)
    with pytest.raises(ValueError):
        bd.bdattn_fwd_tiles(DIFF, 100, 4, 128, 64, 0, 1)   # past the last tile
    with pytest.raises(ValueError):
        bd.bdattn_fwd_tiles(CAUSAL, 100, 1, 128, 64, bd.NOISY, 0)
    with pytest.raises(ValueError):
        bd.bdattn_row_interval(DIFF, 10, 2, 0, 10, 0)
    with pytest.raises(ValueError):
        bd.bdattn_visible_pairs(3, 10, 2)
