"""Exact emulation of the INT8-QK / FP8-PV attention variant (SageAttention style).

Test infrastructure only (see the package docstring).

Source: handbook page "算子加速：注意力、编译与融合", section "SageAttention":
K is smoothed by subtracting a mean (removing its outlier channels), Q and K
are quantised to INT8 so that Q K^T runs on integer matrix cores, and P and V
go through FP8 with wide accumulation.  The pages print no quantised result,
so the numerical choices below are this project's readings, applied the same
way on both sides:

  * K smoothing: kmean[b,h,:] = mean of K over all N tokens, summed in float64
    and rounded once to float32; Ks = fp32(K - kmean).  Softmax ignores a
    per-row constant, and q . kmean is one, so O is unchanged by smoothing.
  * INT8 Q and Ks: one scale per (b, h, block of 64 tokens from token 0; the
    last block may be partial) over all D channels: a = max |X|,
    inv = fp32(127 / a), x8 = clamp(rint(fp32(X * inv)), -127, 127),
    s = fp32(a / 127); an all-zero block gives x8 = 0, s = 0.
  * FP8 V: one scale per (b, h, channel): av = max_t |V|,
    v8 = e4m3(fp32(V * fp32(448 / av))), sv = fp32(av / 448).
  * Scores s = (sum_d q8 k8) * sq * sk * scale (the integer dot product is
    exact), then the mask as in the unquantised formula: an additive mask is
    added to the dequantised, scaled scores (scale first, then the mask, as
    the case-study page's attention code does in its section 2.3), before
    the running max; a key-length mask drops the keys at and past the length.
  * P is quantised against the running max of the blocked recurrence: for the
    key tiles of ``kv_block`` keys in ascending order, m_j = max(m_{j-1},
    tile max), P = exp(s - m_j) <= 1, l = l * exp(m_{j-1} - m_j) + sum P (the
    unquantised P), acc = acc * exp(m_{j-1} - m_j) + sum_t e4m3(448 P_t) v8_t.
  * O = acc * sv / (448 l); a row with every key masked gives O = 0.

Q smoothing (``smooth_q=True``, the handbook's "Q and K minus their block
means"): for each (b, h, 64-token block g) qbar_g = mean of the block's rows
of Q that exist (rows < N), summed in float64, divided by their count and
rounded once to float32; Qs = fp32(Q - qbar_g) on those rows (rows past N
stay zero), quantised per block as above; the score gets the compensation
back exactly, s = (sum_d q8 k8) sq sk scale + scale * (qbar_g . Ks_j), the
dot product taken in float64 over the float32 operands, before the mask.
Without quantisation error this is scale * Q . Ks, the same as without
smoothing; with it, only the within-block deviation of Q is quantised.

A second P V mode (``pv="bf16"`` or ``"f16"``) keeps the INT8 Q K^T steps and
runs P V in 16 bits: V is used as given (the 16-bit input values, not
quantised), P is rounded to the 16-bit type (round to nearest even) against
the same running max, acc = acc * exp(m_{j-1} - m_j) + sum_t round16(P_t) V_t,
O = acc / l (l again from the unrounded P).  This is the INT8-QK / FP16-PV
form of the method; the readings above apply unchanged.

The score, exp and accumulation steps run in float64; the quantisers use the
float32 steps written above, reproduced with numpy float32 (IEEE, correctly
rounded per operation).
"""
from __future__ import annotations

import numpy as np

from .rounding import round_bf16, round_e4m3, round_f16

QBLOCK = 64          # tokens per INT8 scale block
E4M3_MAX = 448.0


def k_mean(k_head) -> np.ndarray:
    """Token mean of one head's K [N, D], rounded once to float32."""
    k = np.asarray(k_head, dtype=np.float64)
    return (k.sum(axis=0) / k.shape[0]).astype(np.float32)


def quantise_int8_blocks(x_head, block=QBLOCK):
    """x_head [N, D] (float32 values) -> (x8 int8 [N, D], scale float32 [ceil(N/block)])."""
    x = np.asarray(x_head, dtype=np.float32)
    n, d = x.shape
    nb = -(-n // block)
    xp = np.zeros((nb * block, d), dtype=np.float32)
    xp[:n] = x
    xb = xp.reshape(nb, block * d)
    a = np.abs(xb).max(axis=1).astype(np.float32)               # per-block absmax
    live = a > 0
    safe = np.where(live, a, np.float32(1)).astype(np.float32)
    inv = np.where(live, (np.float32(127.0) / safe).astype(np.float32), np.float32(0)).astype(np.float32)
    y = (xb * inv[:, None]).astype(np.float32)
    x8 = np.clip(np.rint(y), -127, 127).astype(np.int8).reshape(nb * block, d)[:n]
    sc = np.where(live, (a / np.float32(127.0)).astype(np.float32), np.float32(0)).astype(np.float32)
    return x8, sc


def quantise_fp8_channels(v_head):
    """v_head [N, D] -> (v8 e4m3 values as float64 [N, D], per-channel scale float32 [D])."""
    v = np.asarray(v_head, dtype=np.float32)
    av = np.abs(v).max(axis=0).astype(np.float32)
    safe = np.where(av == 0, np.float32(1), av).astype(np.float32)
    mul = np.where(av == 0, np.float32(0), (np.float32(E4M3_MAX) / safe).astype(np.float32)).astype(np.float32)
    y = (v * mul[None, :]).astype(np.float32)
    v8 = round_e4m3(y.astype(np.float64))
    sv = np.where(av == 0, np.float32(0), (av / np.float32(E4M3_MAX)).astype(np.float32)).astype(np.float32)
    return v8, sv


def q_block_means(q_head, block=QBLOCK) -> np.ndarray:
    """qbar [ceil(N/block), D]: the mean of each block's existing rows of Q,
    summed in float64, divided by the row count, rounded once to float32."""
    q = np.asarray(q_head, dtype=np.float64)
    n, d = q.shape
    nb = -(-n // block)
    out = np.zeros((nb, d), dtype=np.float32)
    for g in range(nb):
        rows = q[g * block:min(n, (g + 1) * block)]
        out[g] = (rows.sum(axis=0) / rows.shape[0]).astype(np.float32)
    return out


def quantise_head(q_head, k_head, v_head, smooth_q=False):
    """All quantised operands of one (b, h) head; with smooth_q also the block
    means of Q and the compensation qbar_g . Ks_j [blocks, N] (float64)."""
    km = k_mean(k_head)
    ks = (np.asarray(k_head, dtype=np.float32) - km[None, :]).astype(np.float32)
    extra = {}
    if smooth_q:
        qf = np.asarray(q_head, dtype=np.float32)
        qbar = q_block_means(qf)
        rows_g = np.arange(qf.shape[0]) // QBLOCK
        qs = (qf - qbar[rows_g]).astype(np.float32)
        q8, sq = quantise_int8_blocks(qs)
        extra = dict(qbar=qbar, comp=qbar.astype(np.float64) @ ks.astype(np.float64).T)
    else:
        q8, sq = quantise_int8_blocks(q_head)
    k8, sk = quantise_int8_blocks(ks)
    v8, sv = quantise_fp8_channels(v_head)
    return dict(kmean=km, ks=ks, q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv,
                v16=np.asarray(v_head, dtype=np.float64), **extra)


def _quantised_attention_rows(row_ids, qz, scale, kv_block, key_len=None, quantise_p=True,
                              return_lse=False, pv="fp8", mask=None):
    """Blocked recurrence over key tiles with P quantised against the running max.
    The lse is that of the quantised, smoothed scores (natural log).  pv selects
    the P V arithmetic: "fp8" (448 P and V in e4m3) or "bf16" / "f16" (P rounded
    to that type, V unquantised).  mask: additive values [len(row_ids), N] for
    the selected rows (-inf drops a key), added after scaling."""
    if pv == "fp8":
        vmat, pmul, pround = qz["v8"], E4M3_MAX, round_e4m3
    elif pv in ("bf16", "f16"):
        vmat, pmul, pround = qz["v16"], 1.0, (round_bf16 if pv == "bf16" else round_f16)
    else:
        raise ValueError(f"unknown P V mode {pv!r}")
    row_ids = np.asarray(row_ids, dtype=np.int64)
    q8 = qz["q8"][row_ids].astype(np.float64)
    k8 = qz["k8"].astype(np.float64)
    n = k8.shape[0]
    s = q8 @ k8.T                                           # exact integers
    s = s * qz["sq"][row_ids // QBLOCK].astype(np.float64)[:, None]
    s = s * qz["sk"][np.arange(n) // QBLOCK].astype(np.float64)[None, :]
    s = s * float(scale)
    if "comp" in qz:                                        # Q smoothing: compensation back
        s = s + float(scale) * qz["comp"][row_ids // QBLOCK]
    if mask is not None:
        s = s + np.broadcast_to(np.asarray(mask, dtype=np.float64), s.shape)
    if key_len is not None:
        s[:, int(key_len):] = -np.inf
    R = len(row_ids)
    D = vmat.shape[1]
    m = np.full((R, 1), -np.inf)
    l = np.zeros((R, 1))
    acc = np.zeros((R, D))
    for j in range(0, n, kv_block):
        st = s[:, j:j + kv_block]
        m_new = np.maximum(m, st.max(axis=1, keepdims=True))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        p = np.exp(st - ref)
        alpha = np.exp(m - ref)
        l = l * alpha + p.sum(axis=1, keepdims=True)
        pq = pround(p * pmul) if quantise_p else p * pmul
        acc = acc * alpha + pq @ vmat[j:j + kv_block]
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        if pv == "fp8":
            o = acc * qz["sv"].astype(np.float64)[None, :] / (E4M3_MAX * l)
        else:
            o = acc / l
        lse = np.where(l[:, 0] == 0, -np.inf, m[:, 0] + np.log(l[:, 0]))
    o = np.where(l == 0, 0.0, o)
    return (o, lse) if return_lse else o


def emulate_rows(q_head, k_head, v_head, row_ids, scale, kv_block, key_len=None, qz=None,
                 return_lse=False, pv="fp8", mask=None, smooth_q=False):
    """Quantised-variant output for selected query rows of one head (float64, before
    the output rounding); with return_lse also the rows' log-sum-exp of the
    smoothed quantised scores.  mask: additive values for the selected rows,
    broadcastable to [len(row_ids), N].  smooth_q: Q smoothing with the
    compensation (ignored when qz is given: qz says whether it holds one)."""
    if qz is None:
        qz = quantise_head(q_head, k_head, v_head, smooth_q=smooth_q)
    return _quantised_attention_rows(row_ids, qz, scale, kv_block, key_len, return_lse=return_lse, pv=pv,
                                     mask=mask)


def emulate(q, k, v, scale, kv_block, key_len=None, return_lse=False, pv="fp8", mask=None, smooth_q=False):
    """Full [B, H, N, D] emulation (small shapes); mask broadcastable to
    [B, H, N, N] (additive); smooth_q: Q smoothing with compensation."""
    q = np.asarray(q)
    B, H, N, D = q.shape
    out = np.zeros((B, H, N, np.asarray(v).shape[3]))
    lse = np.zeros((B, H, N))
    mfull = None if mask is None else np.broadcast_to(np.asarray(mask, dtype=np.float64), (B, H, N, N))
    for b in range(B):
        for h in range(H):
            kl = None if key_len is None else int(np.asarray(key_len)[b])
            out[b, h], lse[b, h] = emulate_rows(q[b, h], k[b, h], v[b, h], np.arange(N), scale, kv_block,
                                                kl, return_lse=True, pv=pv,
                                                mask=None if mfull is None else mfull[b, h], smooth_q=smooth_q)
    return (out, lse) if return_lse else out
