"""OTIL selective block transmit, CPU oracle (float64 numpy, plain loops).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the product path
never imports it.

Source: "OTIL for SDXL on 4x L40S", "What is implemented where" (selection is
one topk over the dissimilarity plus ten times an unvisited flag, packing is an
index select, reconstruction is one index copy per remote device; cosine
dissimilarity lies in [0, 2], so unvisited blocks always come first) and
"Self-tests" (the local slice stays exactly fresh, every remote position is a
received sub-block or stale memory and never a blend, exactly k blocks arrive
from each peer, every sub-block is covered within ceil(K/k) steps, and a final
exact gather recovers the latent).

Readings where the pages are silent (each one is listed with its reason in the
design notes):
  - the transmitted tensor is a rank's row band of the latent, stored like
    every activation here, token-major [B, h, W, C];
  - a sub-block is a bh x bw spatial block of that band, with all batch items
    and channels; blocks are numbered row-major over the block grid, and h, W
    must be multiples of bh, bw;
  - the dissimilarity of a block is 1 - cos(x_block, ref_block) with
    cos = <a, b> / max(|a| |b|, 1e-8), where ref is the block as the receivers
    last got it (the per-block last-sent state);
  - "unvisited" means never selected since the caller last cleared the mask;
    selecting a block marks it visited and makes it the new last-sent state;
  - topk ties go to the lower block id (a total order, so the selection is
    unique).
"""
from __future__ import annotations

import math

import numpy as np

COS_EPS = 1e-8
UNVISITED_BONUS = 10.0


def block_grid(h: int, W: int, bh: int, bw: int) -> tuple[int, int]:
    """(blocks per column, blocks per row) of a band of h x W pixels."""
    if h % bh or W % bw:
        raise ValueError("band sizes must be multiples of the block sizes")
    return h // bh, W // bw


def block_view(x: np.ndarray, j: int, bh: int, bw: int) -> np.ndarray:
    """The values of block j of x [B, h, W, C] as [B, bh, bw, C]."""
    _, h, W, _ = x.shape
    _, nbx = block_grid(h, W, bh, bw)
    by, bx = divmod(j, nbx)
    return x[:, by * bh:(by + 1) * bh, bx * bw:(bx + 1) * bw, :]


def cosine_dissimilarity(a: np.ndarray, b: np.ndarray) -> float:
    """1 - cos(a, b) of two flattened value sets, in [0, 2]."""
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    dot = 0.0
    na = 0.0
    nb = 0.0
    for u, v in zip(a, b):
        dot += u * v
        na += u * u
        nb += v * v
    return 1.0 - dot / max(math.sqrt(na) * math.sqrt(nb), COS_EPS)


def block_scores(x, ref, visited, bh: int, bw: int, bonus: float = UNVISITED_BONUS) -> np.ndarray:
    """Selection score of every block: dissimilarity to the last-sent state,
    plus `bonus` when the block is unvisited."""
    _, h, W, _ = x.shape
    nby, nbx = block_grid(h, W, bh, bw)
    K = nby * nbx
    s = np.empty(K)
    for j in range(K):
        d = cosine_dissimilarity(block_view(x, j, bh, bw), block_view(ref, j, bh, bw))
        s[j] = d + (0.0 if visited[j] else bonus)
    return s


def topk_blocks(scores, k: int) -> np.ndarray:
    """Ids of the k highest scores, highest first; equal scores in id order."""
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    return np.array(order[:k], dtype=np.int64)


def pack(x, idx, bh: int, bw: int) -> np.ndarray:
    """The selected blocks, in selection order: [k, B, bh, bw, C]."""
    return np.stack([block_view(x, int(j), bh, bw) for j in idx]) if len(idx) else \
        np.zeros((0, x.shape[0], bh, bw, x.shape[3]))


def send_step(x, last_sent, visited, bh: int, bw: int, k: int, bonus: float = UNVISITED_BONUS):
    """One sender step: scores, selection, packed blocks, and the updated
    last-sent state and visited mask (inputs are not modified)."""
    scores = block_scores(x, last_sent, visited, bh, bw, bonus)
    idx = topk_blocks(scores, k)
    packed = pack(x, idx, bh, bw)
    new_ref = np.array(last_sent, np.float64, copy=True)
    new_vis = np.array(visited, copy=True)
    for j in idx:
        block_view(new_ref, int(j), bh, bw)[...] = block_view(x, int(j), bh, bw)
        new_vis[int(j)] = 1
    return scores, idx, packed, new_ref, new_vis


def unpack(dst, packed, idx, r0: int, h: int, bh: int, bw: int) -> np.ndarray:
    """Receiver side: copies block p of `packed` into block idx[p] of the peer's
    band, rows [r0, r0 + h) of dst [B, H, W, C]; returns the updated copy."""
    out = np.array(dst, np.float64, copy=True)
    band = out[:, r0:r0 + h]
    for p, j in enumerate(idx):
        block_view(band, int(j), bh, bw)[...] = packed[p]
    return out
