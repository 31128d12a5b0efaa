"""The attention forward O = softmax(scale * Q K^T + mask) V, three ways.

Test infrastructure only (see the package docstring).

Sources (page titles and sections):
  * handbook page "算子加速：注意力、编译与融合", section
    "注意力：从 O(N²) 显存到分块": the materialised-score formula (its
    ``naive``), the blocked form with a running row max m, running
    denominator l and rescaled accumulator (its ``blocked`` and the
    FlashAttention figure), scale 1/sqrt(D);
  * essay page "FlashAttention原理与工业实战", section 2.1: boolean masks
    where 0 marks a dropped key; section 2.2: the exact softmax done as a max
    pass, a sum pass and an output pass; section 2.3: the Triton kernel also
    emits the row log-sum-exp;
  * case-study page, section 2.3: the order scale first, then add the mask.

Readings where the pages are silent (each listed in the design notes):
  * the mask is added after scaling and is not itself scaled;
  * a row whose every key is masked yields O = 0 and lse = -inf;
  * lse is the natural log of sum_j exp(scale * q.k_j + mask_j);
  * key_len[b] masks keys j >= key_len[b] of batch entry b.

Shapes: q [B, H, Nq, D], k and v [B, H, Nk, D]; mask broadcastable to
[B, H, Nq, Nk]; key_len [B] ints.  Inputs are any float arrays (bf16/fp16
values are passed already decoded); arithmetic runs in ``dtype``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _key_mask(B: int, Nk: int, key_len) -> Optional[np.ndarray]:
    if key_len is None:
        return None
    kl = np.asarray(key_len).reshape(B)
    return np.arange(Nk)[None, :] >= kl[:, None]          # True = dropped, [B, Nk]


def scores(q, k, scale, mask=None, key_len=None, dtype=np.float64) -> np.ndarray:
    """S = scale * Q K^T (+ mask), dropped keys at -inf.  Shape [B, H, Nq, Nk]."""
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * dtype(scale)
    if mask is not None:
        s = s + np.asarray(mask, dtype=dtype)
    km = _key_mask(q.shape[0], k.shape[2], key_len)
    if km is not None:
        s = np.where(km[:, None, None, :], -np.inf, s)
    return s


def naive(q, k, v, scale, mask=None, key_len=None, dtype=np.float64):
    """Materialise S, softmax over keys, multiply by V.  Returns (O, lse)."""
    s = scores(q, k, scale, mask, key_len, dtype)
    m = s.max(axis=-1, keepdims=True)
    dead = ~np.isfinite(m)                               # every key masked
    m_safe = np.where(dead, 0.0, m).astype(dtype)
    p = np.exp(s - m_safe)
    l = p.sum(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.matmul(p, np.asarray(v, dtype=dtype)) / l
        lse = (m_safe + np.log(l))[..., 0]
    o = np.where(dead, 0.0, o).astype(dtype)
    lse = np.where(dead[..., 0], -np.inf, lse).astype(dtype)
    return o, lse


def blocked(q, k, v, scale, block=64, mask=None, key_len=None, dtype=np.float64,
            q_block=None, return_peak=False):
    """Tile Q and K/V into blocks; keep a running max m, denominator l and
    accumulator per query row, rescaling l and the accumulator by
    exp(m_old - m_new) whenever a K/V block raises the max.  The score tile
    is at most q_block x block, never N x N.  Returns (O, lse[, peak bytes])."""
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    qb = block if q_block is None else q_block
    km = _key_mask(B, Nk, key_len)
    mfull = None if mask is None else np.broadcast_to(np.asarray(mask, dtype=dtype), (B, H, Nq, Nk))
    out = np.zeros((B, H, Nq, v.shape[3]), dtype=dtype)
    lse = np.zeros((B, H, Nq), dtype=dtype)
    peak = 0
    for i in range(0, Nq, qb):
        qi = q[:, :, i:i + qb]
        rows = qi.shape[2]
        m = np.full((B, H, rows, 1), -np.inf, dtype=dtype)
        l = np.zeros((B, H, rows, 1), dtype=dtype)
        acc = np.zeros((B, H, rows, v.shape[3]), dtype=dtype)
        for j in range(0, Nk, block):
            s = np.matmul(qi, np.swapaxes(k[:, :, j:j + block], -1, -2)) * dtype(scale)
            if mfull is not None:
                s = s + mfull[:, :, i:i + qb, j:j + block]
            if km is not None:
                s = np.where(km[:, None, None, j:j + block], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=-1, keepdims=True))
            # while every key seen so far is masked, m_new = -inf: hold the
            # reference point at 0 so exp() sees -inf - 0 rather than NaN
            ref = np.where(np.isfinite(m_new), m_new, 0.0).astype(dtype)
            p = np.exp(s - ref)
            alpha = np.exp(m - ref)
            l = l * alpha + p.sum(axis=-1, keepdims=True)
            acc = acc * alpha + np.matmul(p, v[:, :, j:j + block])
            m = m_new
            peak = max(peak, s.size * 4)
        dead = l == 0
        with np.errstate(invalid="ignore", divide="ignore"):
            out[:, :, i:i + qb] = np.where(dead, 0.0, acc / l)
            lse[:, :, i:i + qb] = np.where(dead, -np.inf, m + np.log(l))[..., 0]
    return (out, lse, peak) if return_peak else (out, lse)


def two_pass(q, k, v, scale, mask=None, key_len=None, dtype=np.float64, block=64):
    """Exact softmax in separate passes over the key blocks: pass 1 finds the
    row max, pass 2 the denominator against that max, pass 3 the normalised
    weighted sum.  No rescaling ever happens."""
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    km = _key_mask(B, Nk, key_len)
    mfull = None if mask is None else np.broadcast_to(np.asarray(mask, dtype=dtype), (B, H, Nq, Nk))

    def tile(j):
        s = np.matmul(q, np.swapaxes(k[:, :, j:j + block], -1, -2)) * dtype(scale)
        if mfull is not None:
            s = s + mfull[..., j:j + block]
        if km is not None:
            s = np.where(km[:, None, None, j:j + block], -np.inf, s)
        return s

    m = np.full((B, H, Nq, 1), -np.inf, dtype=dtype)
    for j in range(0, Nk, block):
        m = np.maximum(m, tile(j).max(axis=-1, keepdims=True))
    dead = ~np.isfinite(m)
    ref = np.where(dead, 0.0, m).astype(dtype)
    l = np.zeros_like(m)
    for j in range(0, Nk, block):
        l += np.exp(tile(j) - ref).sum(axis=-1, keepdims=True)
    o = np.zeros((B, H, Nq, v.shape[3]), dtype=dtype)
    with np.errstate(invalid="ignore", divide="ignore"):
        for j in range(0, Nk, block):
            o += np.matmul(np.exp(tile(j) - ref) / l, v[:, :, j:j + block])
        lse = (ref + np.log(l))[..., 0]
    o = np.where(dead, 0.0, o)
    lse = np.where(dead[..., 0], -np.inf, lse)
    return o, lse


def rows(q_rows, k_head, v_head, scale, key_len=None, mask_rows=None, dtype=np.float64):
    """The naive formula for selected query rows of one head.

    q_rows [R, D]; k_head, v_head [Nk, D]; key_len an int or None;
    mask_rows [R, Nk] or None.  Returns (O [R, D], lse [R])."""
    q4 = np.asarray(q_rows, dtype=dtype)[None, None]
    k4 = np.asarray(k_head, dtype=dtype)[None, None]
    v4 = np.asarray(v_head, dtype=dtype)[None, None]
    m4 = None if mask_rows is None else np.asarray(mask_rows)[None, None]
    kl = None if key_len is None else np.array([key_len])
    o, lse = naive(q4, k4, v4, scale, m4, kl, dtype)
    return o[0, 0], lse[0, 0]


def merge(o_a, lse_a, o_b, lse_b, dtype=np.float64):
    """Combine two attention results over disjoint key sets of the same queries.

    With lse_x the row log-sum-exp over key set x, the result over the union
    has lse = log(exp(lse_a) + exp(lse_b)) and O = O_a exp(lse_a - lse) +
    O_b exp(lse_b - lse): each part's softmax weights are rescaled to the
    union's denominator, the same rescale the blocked recurrence applies per
    tile.  Rows empty on both sides give O = 0, lse = -inf.  Shapes
    O [..., N, D], lse [..., N]."""
    o_a = np.asarray(o_a, dtype=dtype)
    o_b = np.asarray(o_b, dtype=dtype)
    la = np.asarray(lse_a, dtype=dtype)
    lb = np.asarray(lse_b, dtype=dtype)
    m = np.maximum(la, lb)
    dead = ~np.isfinite(m)
    ref = np.where(dead, 0.0, m)
    wa, wb = np.exp(la - ref), np.exp(lb - ref)
    z = wa + wb
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = np.where(dead, -np.inf, ref + np.log(z))
        o = (o_a * wa[..., None] + o_b * wb[..., None]) / z[..., None]
    o = np.where(dead[..., None], 0.0, o)
    return o, lse
