"""Pins for the INT8-QK / FP8-PV emulation.

The pages print no quantised result, so the pins are: the quantisers against
their error bounds and a brute-force search; a lossless construction where
every quantiser is exact and the emulation must equal the unquantised formula;
the reduction to the blocked oracle when the quantisers are the identity; and
the accuracy criterion (cosine >= 0.99 against unquantised attention) on the
Wan-shaped recipe at a reduced size.
"""
import math

import numpy as np
import pytest

from oracle import attention, rounding, sage


def test_int8_block_quantiser_bound_and_extremes():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((200, 32)) * rng.uniform(0.1, 10, (200, 1))).astype(np.float32)
    x8, s = sage.quantise_int8_blocks(x)
    assert s.shape == (4,)                                   # 200 = 3*64 + 8: partial last block
    assert x8.dtype == np.int8 and np.abs(x8.astype(int)).max() <= 127
    for g in range(4):
        blk = slice(64 * g, 64 * g + 64)
        a = np.abs(x[blk]).max()
        assert s[g] == np.float32(a / np.float32(127))
        err = np.abs(x[blk].astype(np.float64) - x8[blk].astype(np.float64) * s[g])
        assert err.max() <= s[g] * (0.5 + 1e-5)
        # the absmax element lands on +-127
        i, j = np.unravel_index(np.abs(x[blk]).argmax(), x[blk].shape)
        assert abs(int(x8[blk][i, j])) == 127


def test_int8_quantiser_brute_force():
    """Each code is the integer nearest to fp32(x * fp32(127/a)), ties to even."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 8)).astype(np.float32)
    x[3, 3] = np.float32(0.5) * np.abs(x).max()             # something in the middle
    x8, s = sage.quantise_int8_blocks(x)
    inv = np.float32(np.float32(127) / np.float32(np.abs(x).max()))
    for val, code in zip(x.ravel(), x8.ravel()):
        y = float(np.float32(val * inv))
        cands = range(-127, 128)
        best = min(cands, key=lambda c: (abs(y - c), c % 2))
        assert code == best


def test_partial_block_has_its_own_scale():
    x = np.ones((130, 4), dtype=np.float32)
    x[129, 0] = 50.0                                        # outlier in the 2-token last block
    _, s = sage.quantise_int8_blocks(x)
    assert s[0] == s[1] == np.float32(1 / np.float32(127)) and s[2] == np.float32(50 / np.float32(127))


def test_zero_block_gives_zero_scale():
    x = np.zeros((70, 4), dtype=np.float32)
    x[65:] = 1.0
    x8, s = sage.quantise_int8_blocks(x)
    assert s[0] == 0 and not x8[:64].any() and s[1] > 0


def test_fp8_channel_quantiser():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((300, 16)) * rng.uniform(0.01, 5, 16)).astype(np.float32)
    v8, sv = sage.quantise_fp8_channels(v)
    assert np.all(np.abs(v8).max(axis=0) == 448.0)
    rel = np.abs(v8 * sv[None, :] - v) / np.maximum(np.abs(v), 1e-30)
    big = np.abs(v) * (448.0 / np.abs(v).max(axis=0)) >= 2.0 ** -6   # normal range of e4m3
    assert rel[big].max() <= 2.0 ** -4 + 1e-6                # 3 mantissa bits
    assert np.array_equal(rounding.round_e4m3(v8), v8)       # codes are e4m3 values


def _lossless_head(seed, d=8, n=256, step_q=2.0 ** -6, step_k=2.0 ** -5):
    """Q and K on integer grids with power-of-two steps, every 64-token block
    holding one code of magnitude 127 (so each block's scale is exactly the
    step); the 127s sit in channels the other operand leaves at zero, so scores
    stay small integers.  K's second half mirrors its first, making the token
    mean exactly zero.  V per channel takes {0, +-av/4, +-av/2, +-av} with
    av = 1.75 * 2^k (so 448/av and av/448 are exact) and av present."""
    rng = np.random.default_rng(seed)
    half = n // 2
    qc = rng.integers(-1, 2, (n, d))
    kc = rng.integers(-1, 2, (half, d))
    qc[:, :2] = 0
    kc[:, :2] = 0
    qc[::64, 0] = 127
    kc[::64, 1] = 127
    kc = np.concatenate([kc, -kc])
    av = 1.75 * 2.0 ** rng.integers(-2, 3, d)
    v = rng.choice([0, 0.25, 0.5, 1.0, -0.25, -0.5, -1.0], (n, d)) * av
    v[0] = av
    return qc * step_q, kc * step_k, v, step_q, step_k


@pytest.mark.parametrize("pv", ["fp8", "bf16", "f16"])
@pytest.mark.parametrize("kv_block", [64, 128])
def test_lossless_case_equals_unquantised_formula(kv_block, pv):
    q, k, v, step_q, step_k = _lossless_head(5)
    n = len(q)
    qz = sage.quantise_head(q, k, v)
    assert np.all(qz["kmean"] == 0)
    assert np.all(qz["sq"] == step_q) and np.all(qz["sk"] == step_k)
    assert np.array_equal(qz["q8"] * step_q, q) and np.array_equal(qz["k8"] * step_k, k)
    # every score is an integer multiple of ln 2 within 6 ln 2 of zero, so each
    # P relative to any running max is 2^-j with j <= 12: 448 P is an e4m3 value
    scale = math.log(2) / (step_q * step_k)
    # (P = 2^-j and V in {0, +-av/4, +-av/2, +-av} are exact in bf16 and fp16 too)
    o_emu = sage.emulate_rows(q, k, v, np.arange(n), scale, kv_block=kv_block, pv=pv)
    o_ref, _ = attention.naive(q[None, None], k[None, None], v[None, None], scale)
    assert np.abs(o_emu - o_ref[0, 0]).max() <= 1e-12 * np.abs(v).max()


def test_identity_quantisers_reduce_to_blocked_oracle_16bit_pv():
    rng = np.random.default_rng(16)
    n, d = 130, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    qz = dict(q8=q, sq=np.ones(3), k8=k - k.mean(axis=0), sk=np.ones(3), v16=v)
    for pv in ("bf16", "f16"):
        o_id = sage._quantised_attention_rows(np.arange(n), qz, 0.25, 64, quantise_p=False, pv=pv)
        o_bl, _ = attention.blocked(q[None, None], k[None, None], v[None, None], 0.25, block=64)
        assert np.abs(o_id - o_bl[0, 0]).max() < 1e-12


@pytest.mark.parametrize("pv,ulp", [("bf16", 2.0 ** -8), ("f16", 2.0 ** -11)])
def test_16bit_pv_constant_v_bound(pv, ulp):
    """With V constant per channel, O = c * (sum of rounded P) / (sum of P):
    within one half-ulp of the P type of c (P rounded to nearest), and not
    exactly c once P needs rounding."""
    rng = np.random.default_rng(21)
    n, d = 300, 8
    q, k = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(2))
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (n, d)).copy()
    o = sage.emulate_rows(q, k, v, np.arange(n), 0.5, 64, pv=pv)
    rel = np.abs(o / c[None, :] - 1.0)
    assert rel.max() <= ulp / 2 * 1.0000001
    assert rel.max() > ulp / 100            # P really was rounded (fp64 noise is ~1e-16)


def test_16bit_pv_is_closer_than_fp8_on_wan_recipe():
    from attention_fa_fwd_04_amd.workloads import WORKLOADS, head
    w = WORKLOADS[5].with_shape(N=1200)
    q, k, v = (head(w, t, 0, 0).double().numpy() for t in range(3))
    rows = np.arange(0, 1200, 7)
    ref = attention.rows(q[rows], k, v, w.scale)[0]
    def cos(o):
        return float((o * ref).sum() / np.sqrt((o * o).sum() * (ref * ref).sum()))
    c8 = cos(sage.emulate_rows(q, k, v, rows, w.scale, 64, pv="fp8"))
    c16 = cos(sage.emulate_rows(q, k, v, rows, w.scale, 64, pv="bf16"))
    assert c16 >= 0.999 and c16 >= c8


def test_identity_quantisers_reduce_to_blocked_oracle():
    rng = np.random.default_rng(6)
    n, d = 130, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    ks = k - k.mean(axis=0)
    av = np.abs(v).max(axis=0)
    qz = dict(q8=q, sq=np.ones(3), k8=ks, sk=np.ones(3), v8=v * 448.0 / av, sv=av / 448.0)
    o_id = sage._quantised_attention_rows(np.arange(n), qz, 0.25, 64, quantise_p=False)
    o_bl, _ = attention.blocked(q[None, None], k[None, None], v[None, None], 0.25, block=64)
    assert np.abs(o_id - o_bl[0, 0]).max() < 1e-12


def test_emulated_lse_is_that_of_smoothed_scores():
    """In the lossless construction the emulated lse equals the unquantised lse
    of (Q, K - kmean); with K's mean nonzero it equals the unquantised lse of
    (Q, K) minus scale * q . kmean (softmax's shift invariance)."""
    q, k, v, step_q, step_k = _lossless_head(5)
    scale = math.log(2) / (step_q * step_k)
    n = len(q)
    _, lse = sage.emulate_rows(q, k, v, np.arange(n), scale, 64, return_lse=True)
    _, ref = attention.naive(q[None, None], k[None, None], v[None, None], scale)
    assert np.abs(lse - ref[0, 0]).max() < 1e-9
    rng = np.random.default_rng(9)
    q2, k2, v2 = (rng.standard_normal((150, 16)) for _ in range(3))
    k2 += 3.0
    _, lse2 = sage.emulate_rows(q2, k2, v2, np.arange(150), 0.25, 64, return_lse=True)
    _, ref2 = attention.naive(q2[None, None], k2[None, None], v2[None, None], 0.25)
    shift = 0.25 * q2 @ sage.k_mean(k2).astype(np.float64)
    assert np.abs(lse2 + shift - ref2[0, 0]).max() < 0.05


def test_key_length_in_emulation():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((100, 16)).astype(np.float32) for _ in range(3))
    full = sage.emulate_rows(q, k, v, np.arange(100), 0.25, 64, key_len=70)
    assert np.all(np.isfinite(full))
    zero = sage.emulate_rows(q, k, v, np.arange(3), 0.25, 64, key_len=0)
    assert np.all(zero == 0)


@pytest.mark.parametrize("kv_block", [64, 128])
def test_cosine_against_unquantised_on_wan_recipe(kv_block):
    """Wan-shaped recipe at reduced N: N(0,1) Q/K/V plus a per-channel K offset of
    variance 2; the quantised output keeps cosine >= 0.99 with unquantised attention."""
    from attention_fa_fwd_04_amd.workloads import WORKLOADS, head
    w = WORKLOADS[5].with_shape(N=1000, H=2)
    cos = []
    for h in range(2):
        q, k, v = (head(w, t, 0, h).double().numpy() for t in range(3))
        ids = np.arange(0, 1000, 7)
        o = sage.emulate_rows(q, k, v, ids, w.scale, kv_block)
        ref, _ = attention.rows(q[ids], k, v, w.scale)
        cos.append((o * ref).sum() / np.linalg.norm(o) / np.linalg.norm(ref))
        assert np.abs(o - ref).max() < 5e-2          # loose: the bound that binds is the cosine
    print("cosines", cos)
    assert min(cos) >= 0.99


# ---- P rounding against the running max (reading R14), hand-derived values ----

def _three_key_row():
    """One query, three keys, D = 1, every scale 1: integer scores 0, -1, +1
    times c = -ln 0.3, so exp(s) = 1, 0.3 and 1 / 0.3.  V codes 1, 2, 0 with
    a channel scale of 1."""
    qz = dict(q8=np.array([[1]], dtype=np.int8), sq=np.float32([1.0]),
              k8=np.array([[0], [-1], [1]], dtype=np.int8), sk=np.float32([1.0]),
              v8=np.array([[1.0], [2.0], [0.0]]), sv=np.float32([1.0]))
    return qz, -math.log(0.3)


def test_p_rounded_against_running_max_hand_derived():
    """Key tiles of 2: tile 0 = keys 0, 1; tile 1 = key 2.

    Tile 0 (running max 0): P = 1, 0.3; 448 P = 448 (an e4m3 value) and 134.4,
    which rounds to 128 (e4m3 spacing 16 in [128, 256)); acc = 448*1 + 128*2
    = 704, l = 1.3.  Tile 1 raises the max to c: both are rescaled by
    exp(-c) = 0.3 (acc 211.2, l 0.39), key 2 adds P = 1 (448 * 0 to acc):
    l = 1.39, O = 211.2 / (448 * 1.39).

    Rounding against the final max instead would give 448*0.3 = 134.4 -> 128
    and 448*0.09 = 40.32 -> 40 (spacing 4 in [32, 64)): O = 208 / (448 * 1.39),
    which is what a single tile holding all three keys gives."""
    qz, c = _three_key_row()
    o, lse = sage._quantised_attention_rows(np.array([0]), qz, c, kv_block=2, return_lse=True)
    running = 0.3 * (448.0 * 1 + 128.0 * 2) / (448.0 * 1.39)
    final = (128.0 * 1 + 40.0 * 2) / (448.0 * 1.39)
    assert abs(running - final) > 1e-3                      # the readings really differ here
    assert abs(o[0, 0] - running) < 1e-12
    o1 = sage._quantised_attention_rows(np.array([0]), qz, c, kv_block=3)
    assert abs(o1[0, 0] - final) < 1e-12
    # l sums the unrounded P: lse is the exact log-sum-exp of the three scores
    assert abs(lse[0] - math.log(1 + 0.3 + 1 / 0.3)) < 1e-12


def test_p_rounding_16bit_pv_hand_derived():
    """The same scores with P V in bf16 and V = 1, 3, 0 (unquantised): tile 0
    rounds P = 0.3 to bf16 (0.30078125, the nearest value with 8 significant
    bits), then rescales by 0.3; against the final max P = 0.3 and 0.09 would
    round to 0.30078125 and 0.08984375."""
    qz, c = _three_key_row()
    qz["v16"] = np.array([[1.0], [3.0], [0.0]])
    o = sage._quantised_attention_rows(np.array([0]), qz, c, kv_block=2, pv="bf16")
    running = 0.3 * (1.0 + 0.30078125 * 3) / 1.39
    final = (0.30078125 + 0.08984375 * 3) / 1.39
    assert abs(running - final) > 1e-4
    assert abs(o[0, 0] - running) < 1e-12


# ---- additive mask in the emulation ----

@pytest.mark.parametrize("pv", ["fp8", "bf16"])
def test_lossless_case_with_additive_mask_equals_unquantised_formula(pv):
    """Mask values on the ln 2 grid ({-ln 2, 0, ln 2}) and -inf keep every P a
    power of two within the exact e4m3 range, so the emulation must equal the
    unquantised formula with the mask added after scaling.  Rows with every
    key masked give O = 0 and lse = -inf."""
    q, k, v, step_q, step_k = _lossless_head(5)
    n = len(q)
    scale = math.log(2) / (step_q * step_k)
    rng = np.random.default_rng(31)
    mask = rng.choice([-math.log(2), 0.0, math.log(2)], (n, n))
    mask[rng.random((n, n)) < 0.3] = -np.inf
    mask[7] = -np.inf                                        # a fully masked row
    mask[:, 64:128] = np.where(np.arange(n)[:, None] % 3 == 0, -np.inf, mask[:, 64:128])   # dead tiles
    o_emu, lse_emu = sage.emulate_rows(q, k, v, np.arange(n), scale, 64, pv=pv, mask=mask, return_lse=True)
    o_ref, lse_ref = attention.naive(q[None, None], k[None, None], v[None, None], scale, mask=mask[None, None])
    assert np.abs(o_emu - o_ref[0, 0]).max() <= 1e-12 * np.abs(v).max()
    assert np.all(o_emu[7] == 0) and np.isneginf(lse_emu[7])
    fin = np.isfinite(lse_ref[0, 0])
    assert np.array_equal(fin, np.isfinite(lse_emu))
    assert np.abs(lse_emu[fin] - lse_ref[0, 0][fin]).max() < 1e-9


def test_constant_additive_mask_shifts_lse_only():
    """A constant mask c moves every score and every running max by c: O is
    unchanged and lse moves by c (softmax's shift invariance, with P taken
    against the shifted running max)."""
    from attention_fa_fwd_04_amd.workloads import WORKLOADS, head
    w = WORKLOADS[5].with_shape(N=300)
    q, k, v = (head(w, t, 0, 0).double().numpy() for t in range(3))
    rows = np.arange(0, 300, 3)
    o0, l0 = sage.emulate_rows(q, k, v, rows, w.scale, 64, return_lse=True)
    o1, l1 = sage.emulate_rows(q, k, v, rows, w.scale, 64, return_lse=True, mask=-3.25)
    assert np.abs(o1 - o0).max() < 1e-12 and np.abs(l1 - (l0 - 3.25)).max() < 1e-12


def test_additive_mask_matches_key_length():
    """A 0 / -inf mask dropping keys >= L is the key-length mask L."""
    rng = np.random.default_rng(32)
    q, k, v = (rng.standard_normal((150, 16)).astype(np.float32) for _ in range(3))
    mask = np.where(np.arange(150)[None, :] < 97, 0.0, -np.inf)
    a = sage.emulate_rows(q, k, v, np.arange(150), 0.25, 64, mask=mask)
    b = sage.emulate_rows(q, k, v, np.arange(150), 0.25, 64, key_len=97)
    assert np.array_equal(a, b)


# ---- Q smoothing with compensation (handbook, section "SageAttention") ----

def test_q_block_means_brute_force():
    """Each 64-row block's mean over the rows that exist (the last block is
    partial), by pure-Python loops in float64 rounded once to float32."""
    rng = np.random.default_rng(21)
    n, d = 150, 5
    q = (rng.standard_normal((n, d)) * 3 + 1).astype(np.float32)
    got = sage.q_block_means(q)
    assert got.shape == (3, d) and got.dtype == np.float32
    for g in range(3):
        rows = range(64 * g, min(n, 64 * (g + 1)))
        for c in range(d):
            tot = 0.0
            for r in rows:
                tot += float(q[r, c])
            assert got[g, c] == np.float32(tot / len(rows))


def _lossless_smoothed_head(seed, d=8, n=256, step_q=2.0 ** -6, step_k=2.0 ** -5):
    """A head where Q smoothing is lossless and plain Q quantisation is not.
    Qs has codes in {-1,0,1} on channels 2-4 and +127 / -127 on channel 0 in
    rows 0 / 32 of each block, mirrored about the block middle so every block
    mean is zero; each block adds its own offset qbar_g (codes in {-1,0,1} on
    channels 5-7, and 50 on channel 0, times step_q), so Q's block means are
    exactly qbar_g and Q - qbar_g is exactly Qs, while Q itself reaches 177
    steps in a block (plain INT8 Q is then lossy).  K as in the lossless head (channel 0 zero, mean
    zero), so every score is an integer times step_q * step_k within 6 of 0."""
    rng = np.random.default_rng(seed)
    nb = n // 64
    qs = np.zeros((n, d))
    for g in range(nb):
        half = rng.integers(-1, 2, (32, 3))
        blk = np.zeros((64, d))
        blk[:32, 2:5] = half
        blk[32:, 2:5] = -half
        blk[0, 0], blk[32, 0] = 127, -127
        qs[64 * g:64 * (g + 1)] = blk
    qbar = np.zeros((nb, d))
    qbar[:, 5:8] = rng.integers(-1, 2, (nb, 3))
    qbar[:, 5] = np.where(qbar[:, 5] == 0, 1, qbar[:, 5])     # every block offset nonzero
    qbar[:, 0] = 50        # K's channel 0 is zero: no score change, but Q's block max becomes 177
    q = (qs + np.repeat(qbar, 64, axis=0)) * step_q
    _, k, v, _, _ = _lossless_head(seed + 1, d=d, n=n, step_q=step_q, step_k=step_k)
    return q, k, v, qs * step_q, qbar * step_q, step_q, step_k


@pytest.mark.parametrize("pv", ["fp8", "bf16"])
def test_smoothing_lossless_equals_unquantised_formula(pv):
    """The compensation restores qbar_g . Ks_j exactly: with lossless operands
    the smoothed emulation equals unquantised attention (a dropped, mis-signed
    or mis-indexed compensation would not), while plain quantisation of the
    same Q is lossy."""
    q, k, v, qs, qbar, step_q, step_k = _lossless_smoothed_head(31)
    n = len(q)
    qz = sage.quantise_head(q, k, v, smooth_q=True)
    assert np.array_equal(qz["qbar"].astype(np.float64), qbar)
    assert np.all(qz["sq"] == step_q) and np.array_equal(qz["q8"] * step_q, qs)
    scale = math.log(2) / (step_q * step_k)
    o_s, lse_s = sage.emulate_rows(q, k, v, np.arange(n), scale, 64, return_lse=True, pv=pv, smooth_q=True)
    o_ref, lse_ref = attention.naive(q[None, None], k[None, None], v[None, None], scale)
    assert np.abs(o_s - o_ref[0, 0]).max() <= 1e-12 * np.abs(v).max()
    assert np.abs(lse_s - lse_ref[0, 0]).max() < 1e-9
    o_plain = sage.emulate_rows(q, k, v, np.arange(n), scale, 64, pv=pv)
    assert np.abs(o_plain - o_ref[0, 0]).max() > 1e-6


def test_smoothing_helps_with_block_offsets():
    """Queries with a large common offset per 64-token block: smoothing
    quantises only the deviation, so the output (16-bit P V, leaving the Q K^T
    quantisation as the main error) is closer to unquantised attention than
    with plain INT8 Q; on offset-free queries it is no worse than a small
    factor."""
    rng = np.random.default_rng(41)
    n, d = 320, 32
    off = np.repeat(rng.choice([-20.0, 20.0], (n // 64, d)), 64, axis=0)
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    for q, must_gain in ((rng.standard_normal((n, d)) + off, True), (rng.standard_normal((n, d)), False)):
        q = q.astype(np.float32)
        ref, _ = attention.naive(q[None, None].astype(np.float64), k[None, None], v[None, None], d ** -0.5)
        e = {}
        for sm in (False, True):
            o = sage.emulate_rows(q, k, v, np.arange(n), d ** -0.5, 64, smooth_q=sm, pv="bf16")
            e[sm] = np.sqrt(((o - ref[0, 0]) ** 2).mean())
        print("rms error plain / smoothed", e[False], e[True])
        if must_gain:
            assert e[True] < 0.5 * e[False]
        else:
            assert e[True] < 2.0 * e[False]


def test_smoothing_partial_block_and_key_length():
    """A partial last block takes the mean of its existing rows only, and
    smoothing composes with a key-length mask and the 16-bit P V form."""
    rng = np.random.default_rng(43)
    n, d = 100, 16
    q = (rng.standard_normal((n, d)) + 2.0).astype(np.float32)
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    qz = sage.quantise_head(q, k, v, smooth_q=True)
    assert np.array_equal(qz["qbar"][1], sage.q_block_means(q[64:]).reshape(-1))
    for pv in ("fp8", "f16"):
        o = sage.emulate_rows(q, k, v, np.arange(n), 0.25, 64, key_len=70, pv=pv, smooth_q=True)
        ref, _ = attention.naive(q[None, None].astype(np.float64), k[None, None], v[None, None], 0.25,
                                 key_len=np.array([70]))
        cos = (o * ref[0, 0]).sum() / np.linalg.norm(o) / np.linalg.norm(ref[0, 0])
        assert cos > 0.999
