"""Pins of the OTIL selective-transmit oracle (CPU only).

Each check ties the oracle to something other than itself: closed forms of the
cosine, scipy's cosine distance, a reshape-based block decomposition, numpy's
lexsort, and the rules the pages state for the method ("OTIL for SDXL on 4x
L40S", "What is implemented where" and "Self-tests").
"""
from __future__ import annotations

import math

import numpy as np
import pytest
from scipy.spatial.distance import cosine as scipy_cosine

from oracle import otil


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_cosine_closed_forms():
    a = rnd(0, 37)
    assert abs(otil.cosine_dissimilarity(a, a)) < 1e-14
    assert abs(otil.cosine_dissimilarity(a, 3.5 * a)) < 1e-14
    assert abs(otil.cosine_dissimilarity(a, -a) - 2.0) < 1e-14
    e = np.zeros(8)
    f = np.zeros(8)
    e[2], f[5] = 1.0, -4.0
    assert otil.cosine_dissimilarity(e, f) == 1.0
    # a zero block has cosine 0 under the 1e-8 floor, so dissimilarity 1
    assert otil.cosine_dissimilarity(np.zeros(5), rnd(1, 5)) == 1.0


def test_cosine_matches_scipy_and_is_bounded():
    for s in range(20):
        a, b = rnd(10 + s, 64), rnd(50 + s, 64) + (s % 3) * rnd(10 + s, 64)
        d = otil.cosine_dissimilarity(a, b)
        assert abs(d - scipy_cosine(a, b)) < 1e-12
        assert 0.0 <= d <= 2.0


@pytest.mark.parametrize("B,h,W,C,bh,bw", [(2, 8, 16, 4, 4, 8), (1, 6, 6, 3, 2, 3), (2, 4, 4, 1, 4, 4)])
def test_blocks_partition_the_band(B, h, W, C, bh, bw):
    x = rnd(3, B, h, W, C)
    nby, nbx = otil.block_grid(h, W, bh, bw)
    K = nby * nbx
    # independent decomposition: reshape into the block grid
    ref = x.reshape(B, nby, bh, nbx, bw, C).transpose(1, 3, 0, 2, 4, 5).reshape(K, B, bh, bw, C)
    assert np.array_equal(otil.pack(x, np.arange(K), bh, bw), ref)


def test_block_grid_rejects_ragged_bands():
    with pytest.raises(ValueError):
        otil.block_grid(10, 16, 4, 8)


def test_topk_matches_lexsort_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(30):
        K = int(rng.integers(1, 40))
        k = int(rng.integers(0, K + 1))
        s = rng.integers(0, 5, K).astype(float)  # many ties
        want = np.lexsort((np.arange(K), -s))[:k]
        assert np.array_equal(otil.topk_blocks(s, k), want)


def test_scores_add_the_bonus_to_unvisited_blocks_only():
    x, ref = rnd(4, 1, 4, 4, 2), rnd(5, 1, 4, 4, 2)
    vis = np.array([1, 0, 1, 0])
    s = otil.block_scores(x, ref, vis, 2, 2)
    for j in range(4):
        d = scipy_cosine(otil.block_view(x, j, 2, 2).ravel(), otil.block_view(ref, j, 2, 2).ravel())
        assert abs(s[j] - d - (0.0 if vis[j] else 10.0)) < 1e-12


def test_the_most_changed_block_is_sent_first_once_all_are_visited():
    x = rnd(6, 2, 8, 16, 3)  # a 2 x 4 grid of 4 x 4 blocks
    ref = x.copy()
    blk = otil.block_view(ref, 5, 4, 4)
    blk *= -1.0  # block 5 of the last-sent state is the negation: dissimilarity 2
    otil.block_view(ref, 2, 4, 4)[...] += 0.1 * rnd(8, 2, 4, 4, 3)
    _, idx, packed, new_ref, new_vis = otil.send_step(x, ref, np.ones(8, np.int64), 4, 4, 2)
    assert list(idx) == [5, 2]
    assert np.array_equal(packed[0], otil.block_view(x, 5, 4, 4))
    assert np.array_equal(new_ref, x)  # the two changed blocks were re-sent


@pytest.mark.parametrize("K_grid,k", [((2, 4), 3), ((4, 16), 32), ((3, 5), 1), ((2, 2), 4)])
def test_every_block_is_covered_within_ceil_K_over_k_steps(K_grid, k):
    nby, nbx = K_grid
    bh, bw = 2, 2
    K = nby * nbx
    x = rnd(9, 1, nby * bh, nbx * bw, 2)
    ref = np.zeros_like(x)
    vis = np.zeros(K, np.int64)
    sent = set()
    rng = np.random.default_rng(11)
    for step in range(math.ceil(K / k)):
        _, idx, _, ref, new_vis = otil.send_step(x, ref, vis, bh, bw, k)
        assert len(idx) == min(k, K) and len(set(idx.tolist())) == len(idx)
        # unvisited blocks always come before visited ones
        unv = [j for j in idx if not vis[j]]
        assert list(idx[:len(unv)]) == unv
        assert len(unv) == min(len(idx), int((vis == 0).sum()))
        sent |= set(idx.tolist())
        vis = new_vis
        x = x + 0.3 * rng.standard_normal(x.shape)
    assert sent == set(range(K)) and vis.all()


def test_multi_rank_reconstruction_rules():
    """N ranks each own a band of one latent; every step each sends k blocks
    and every other rank copies them into its copy.  The pages' rules: the
    local band is exactly fresh, a remote position is a received block or the
    previous copy (never a blend), exactly k blocks arrive per peer, and the
    final gather of the local bands is exact."""
    N, B, C, bh, bw, k = 3, 2, 2, 2, 4, 3
    h, W = 4, 8
    H = N * h
    K = (h // bh) * (W // bw)
    rng = np.random.default_rng(12)
    latent = rng.standard_normal((B, H, W, C))
    copies = [latent.copy() for _ in range(N)]  # every rank starts from the exact latent
    last = [latent[:, p * h:(p + 1) * h].copy() for p in range(N)]
    vis = [np.zeros(K, np.int64) for _ in range(N)]
    for step in range(4):
        latent = latent + 0.2 * rng.standard_normal(latent.shape)
        sends = []
        for p in range(N):
            band = latent[:, p * h:(p + 1) * h]
            _, idx, packed, last[p], vis[p] = otil.send_step(band, last[p], vis[p], bh, bw, k)
            sends.append((idx, packed))
        for r in range(N):
            before = copies[r].copy()
            copies[r][:, r * h:(r + 1) * h] = latent[:, r * h:(r + 1) * h]  # local: fresh
            for p in range(N):
                if p == r:
                    continue
                idx, packed = sends[p]
                assert len(idx) == k
                copies[r] = otil.unpack(copies[r], packed, idx, p * h, h, bh, bw)
                band_new = copies[r][:, p * h:(p + 1) * h]
                band_old = before[:, p * h:(p + 1) * h]
                band_true = latent[:, p * h:(p + 1) * h]
                for j in range(K):
                    got = otil.block_view(band_new, j, bh, bw)
                    if j in set(idx.tolist()):
                        assert np.array_equal(got, otil.block_view(band_true, j, bh, bw))
                    else:
                        assert np.array_equal(got, otil.block_view(band_old, j, bh, bw))
            assert np.array_equal(copies[r][:, r * h:(r + 1) * h], latent[:, r * h:(r + 1) * h])
    # The pre-decode gather takes each rank's own band from that rank's copy:
    # it is exact, although every rank's copy is stale somewhere remote.
    gathered = np.concatenate([copies[p][:, p * h:(p + 1) * h] for p in range(N)], axis=1)
    assert np.array_equal(gathered, latent)
    for r in range(N):
        remote = np.r_[0:r * h, (r + 1) * h:H]
        assert not np.array_equal(copies[r][:, remote], latent[:, remote])
