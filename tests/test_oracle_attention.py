"""Pins for the unquantised oracle: the handbook's worked example and printed
tables, closed forms, invariants, brute force and a library routine.

None of these compares the oracle with a retyped copy of itself: each check
would fail for a dropped term, a sign or index slip, or a transposed operand.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import accounting, attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- worked example

def _worked_inputs():
    torch.manual_seed(0)
    B, H, N, D = 1, 4, 256, 32
    return [torch.randn(B, H, N, D) for _ in range(3)]


def test_worked_example_naive_blocked_library_agree():
    g = _golden("worked_example.json")
    q, k, v = _worked_inputs()
    scale = 1.0 / math.sqrt(32)
    for dt in (np.float32, np.float64):
        o1, _ = attention.naive(q.numpy(), k.numpy(), v.numpy(), scale, dtype=dt)
        o2, _, peak = attention.blocked(q.numpy(), k.numpy(), v.numpy(), scale, block=64,
                                        dtype=dt, return_peak=True)
        assert np.allclose(o1, o2, atol=g["naive_vs_blocked_allclose_atol"], rtol=0) == g["naive_vs_blocked"]
        o3 = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
        assert np.allclose(o1, o3, atol=1e-5, rtol=0) == g["naive_vs_library_sdpa"]
        assert peak == g["blocked_peak_score_kib"] * 1024
    s = attention.scores(q.numpy(), k.numpy(), scale)
    assert s.size * 4 == g["naive_score_kib"] * 1024
    assert (s.size * 4) // peak == g["ratio"]


def test_library_sdpa_agrees_in_fp64_with_mask():
    """A library routine with an additive mask, in float64 (pins the mask order:
    scale the product, then add the mask)."""
    B, H, N, D = 2, 3, 37, 16
    q, k, v = (_rand((B, H, N, D), s) for s in (1, 2, 3))
    mask = _rand((B, 1, N, N), 4, 3.0)
    scale = 0.3
    o, _ = attention.naive(q, k, v, scale, mask=mask)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()
    assert np.abs(o - ref).max() < 1e-12


# ---------------------------------------------------------------- brute force

def _brute(q, k, v, scale, mask=None):
    """Pure-Python loops over scalars: softmax row by row with math.exp."""
    Nq, D = len(q), len(q[0])
    Nk = len(k)
    out, lse = [], []
    for i in range(Nq):
        s = []
        for j in range(Nk):
            t = sum(q[i][d] * k[j][d] for d in range(D)) * scale
            if mask is not None:
                t += mask[i][j]
            s.append(t)
        mx = max(s)
        w = [math.exp(t - mx) for t in s]
        z = sum(w)
        out.append([sum(w[j] * v[j][d] for j in range(Nk)) / z for d in range(len(v[0]))])
        lse.append(mx + math.log(z))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("nq,nk,d", [(1, 1, 1), (3, 5, 2), (7, 4, 3), (5, 9, 8)])
def test_brute_force_tiny(nq, nk, d):
    q = _rand((nq, d), 10 + nq)
    k = _rand((nk, d), 20 + nk)
    v = _rand((nk, d), 30 + d)
    mask = _rand((nq, nk), 40, 2.0)
    scale = 0.7
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), scale, mask.tolist())
    for fn in (attention.naive, attention.blocked, attention.two_pass):
        kw = {"block": 2} if fn is not attention.naive else {}
        o, lse = fn(q[None, None], k[None, None], v[None, None], scale, mask=mask[None, None], **kw)
        assert np.abs(o[0, 0] - ob).max() < 1e-12
        assert np.abs(lse[0, 0] - lb).max() < 1e-12


# ---------------------------------------------------------------- tiling claims

def test_block_size_independence_and_peak_scaling():
    """The handbook's exercise: block 16 / 64 / 256 give the same O; the peak
    score tile scales with the block size (1/4 and 4x of block 64)."""
    q, k, v = (_rand((1, 2, 256, 32), s) for s in (5, 6, 7))
    scale = 1 / math.sqrt(32)
    o_ref, l_ref = attention.naive(q, k, v, scale)
    peaks = {}
    for b in (16, 64, 256):
        o, lse, peaks[b] = attention.blocked(q, k, v, scale, block=b, q_block=64, return_peak=True)
        assert np.abs(o - o_ref).max() < 1e-13
        assert np.abs(lse - l_ref).max() < 1e-12
    assert peaks[16] * 4 == peaks[64] and peaks[256] == 4 * peaks[64]


def test_two_pass_matches_naive_with_ragged_blocks():
    q, k, v = (_rand((2, 2, 67, 24), s) for s in (8, 9, 10))
    o1, l1 = attention.naive(q, k, v, 0.2)
    o2, l2 = attention.two_pass(q, k, v, 0.2, block=16)
    o3, l3 = attention.blocked(q, k, v, 0.2, block=16, q_block=20)
    for o, l in ((o2, l2), (o3, l3)):
        assert np.abs(o - o1).max() < 1e-13 and np.abs(l - l1).max() < 1e-12


# ---------------------------------------------------------------- printed tables

def test_byte_table_matches_printed_digits():
    g = _golden("attn_bytes_table.json")
    GB = 1024 ** 3
    fmt = g["format"]
    for row in g["rows"]:
        s, nv, fl = accounting.attn_bytes(row["n"], row["d_head"], row["heads"])
        assert format(s / GB, fmt["scores"]) == row["scores"]
        assert format(nv / GB, fmt["naive"]) == row["naive"]
        assert format(fl / GB, fmt["flash"]) == row["flash"]


def test_hundred_k_token_head_is_20_gb():
    """The handbook's quick-check answer: one head's N x N bf16 scores at 100k tokens ~ 20 GB."""
    s, _, _ = accounting.attn_bytes(100_000, 128, 1)
    assert round(s / 1e9) == 20


def test_attention_row_of_block_profile():
    g = _golden("block_profile_attention.json")
    flops, byts = accounting.attention_block_row(g["n"], g["d_model"])
    assert format(flops / 1e9, ".1f") == g["gflop"]
    assert format(byts / 2 ** 20, ".0f") == g["mib"]
    assert format(flops / byts, ".0f") == g["intensity"]
    t = max(flops / g["h100_peak_flops"], byts / g["h100_bw"]) * 1e6
    assert format(t, ".0f") == g["time_us"]
    assert flops / g["h100_peak_flops"] > byts / g["h100_bw"]       # compute bound
    # the same FLOPs as the headline metric 4*B*H*N^2*D with H*D = d_model
    assert accounting.attention_flops(1, 24, 4608, 128) == flops


# ---------------------------------------------------------------- invariants

@pytest.fixture(scope="module")
def qkv():
    return tuple(_rand((2, 3, 50, 16), s) for s in (11, 12, 13))


def test_rows_of_p_sum_to_one(qkv):
    q, k, v = qkv
    mask = _rand((2, 3, 50, 50), 14)
    _, lse = attention.naive(q, k, v, 0.25, mask=mask)
    s = attention.scores(q, k, 0.25, mask=mask)
    assert np.abs(np.exp(s - lse[..., None]).sum(-1) - 1).max() < 1e-13


def test_constant_v_gives_that_constant(qkv):
    q, k, _ = qkv
    v = np.full(k.shape, -2.5)
    o, _ = attention.blocked(q, k, v, 0.25, block=16)
    assert np.abs(o + 2.5).max() < 1e-13


def test_constant_score_shift(qkv):
    q, k, v = qkv
    o1, l1 = attention.naive(q, k, v, 0.25)
    o2, l2 = attention.naive(q, k, v, 0.25, mask=np.full((1, 1, 1, 1), 3.75))
    assert np.abs(o1 - o2).max() < 1e-13
    assert np.abs(l2 - l1 - 3.75).max() < 1e-12


def test_joint_kv_permutation(qkv):
    q, k, v = qkv
    perm = np.random.default_rng(15).permutation(k.shape[2])
    o1, l1 = attention.blocked(q, k, v, 0.25, block=16)
    o2, l2 = attention.blocked(q, k[:, :, perm], v[:, :, perm], 0.25, block=16)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-12


def test_single_key_returns_v():
    q, k, v = (_rand((1, 2, 5, 8), s) for s in (16, 17, 18))
    o, lse = attention.naive(q, k[:, :, :1], v[:, :, :1], 0.5)
    assert np.abs(o - v[:, :, :1]).max() < 1e-15
    assert np.abs(lse - 0.5 * (q @ np.swapaxes(k[:, :, :1], -1, -2))[..., 0]).max() < 1e-14


def test_zero_scale_gives_mean_of_v(qkv):
    q, k, v = qkv
    o, lse = attention.two_pass(q, k, v, 0.0)
    assert np.abs(o - v.mean(axis=2, keepdims=True)).max() < 1e-13
    assert np.abs(lse - math.log(k.shape[2])).max() < 1e-13


def test_key_length_equals_truncated_keys(qkv):
    q, k, v = qkv
    kl = np.array([17, 50])
    o, lse = attention.naive(q, k, v, 0.25, key_len=kl)
    ob, lb = attention.blocked(q, k, v, 0.25, key_len=kl, block=16)
    for b, L in enumerate(kl):
        ot, lt = attention.naive(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], 0.25)
        assert np.abs(o[b] - ot[0]).max() < 1e-13 and np.abs(lse[b] - lt[0]).max() < 1e-12
        assert np.abs(ob[b] - ot[0]).max() < 1e-13


def test_boolean_mask_convention_zero_drops(qkv):
    """A boolean mask with 0 marking dropped keys equals additive 0/-inf."""
    q, k, v = qkv
    keep = np.random.default_rng(19).random((2, 3, 50, 50)) > 0.3
    keep[..., 0] = True
    add = np.where(keep, 0.0, -np.inf)
    o1, _ = attention.naive(q, k, v, 0.25, mask=add)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(keep), scale=0.25).numpy()
    assert np.abs(o1 - ref).max() < 1e-12


def test_v_linearity(qkv):
    q, k, v = qkv
    o1, _ = attention.naive(q, k, v, 0.25)
    o2, _ = attention.naive(q, k, -3.0 * v, 0.25)
    assert np.abs(o2 + 3.0 * o1).max() < 1e-13


def test_k_smoothing_is_exact(qkv):
    """Subtracting any per-head constant vector from K leaves O unchanged and
    shifts lse by scale * q . c (softmax ignores a per-row constant)."""
    q, k, v = qkv
    c = k.mean(axis=2, keepdims=True) + 0.3
    o1, l1 = attention.naive(q, k, v, 0.25)
    o2, l2 = attention.naive(q, k - c, v, 0.25)
    assert np.abs(o1 - o2).max() < 1e-13
    shift = 0.25 * (q @ np.swapaxes(c, -1, -2))[..., 0]
    assert np.abs(l1 - l2 - shift).max() < 1e-12


def test_fully_masked_rows_give_zero_and_minus_inf():
    q, k, v = (_rand((1, 1, 6, 4), s) for s in (21, 22, 23))
    mask = np.zeros((1, 1, 6, 6))
    mask[0, 0, 2, :] = -np.inf
    for fn, kw in ((attention.naive, {}), (attention.blocked, {"block": 4}), (attention.two_pass, {"block": 4})):
        o, lse = fn(q, k, v, 0.5, mask=mask, **kw)
        assert np.all(o[0, 0, 2] == 0) and lse[0, 0, 2] == -np.inf
        assert np.all(np.isfinite(o)) and np.isfinite(lse[0, 0, [0, 1, 3, 4, 5]]).all()
    o, lse = attention.naive(q, k, v, 0.5, key_len=np.array([0]))
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_rows_helper_matches_full(qkv):
    q, k, v = qkv
    kl = np.array([30, 50])
    o, lse = attention.naive(q, k, v, 0.25, key_len=kl)
    ids = np.array([0, 7, 49])
    orow, lrow = attention.rows(q[1, 2, ids], k[1, 2], v[1, 2], 0.25, key_len=30)
    ofull, _ = attention.naive(q[1:2], k[1:2], v[1:2], 0.25, key_len=np.array([30]))
    assert np.abs(orow - ofull[0, 2, ids]).max() < 1e-14


# ---------------------------------------------------------------- merge of key shards

@pytest.mark.parametrize("split", [1, 17, 25, 49])
def test_merge_of_key_split_equals_full(split):
    """Attention over keys [0, s) and [s, N) merged by lse equals attention over
    all keys (sequence sharding of K/V, the essay's ring-attention section)."""
    q, k, v = (_rand((2, 3, 30, 8), s) for s in (31, 32, 33))
    k, v = np.concatenate([k, k[:, :, :20]], axis=2), np.concatenate([v, v[:, :, :20]], axis=2)
    o_full, l_full = attention.naive(q, k, v, 0.4)
    oa, la = attention.naive(q, k[:, :, :split], v[:, :, :split], 0.4)
    ob, lb = attention.naive(q, k[:, :, split:], v[:, :, split:], 0.4)
    o, lse = attention.merge(oa, la, ob, lb)
    assert np.abs(o - o_full).max() < 1e-13 and np.abs(lse - l_full).max() < 1e-12


def test_merge_handles_empty_sides():
    q, k, v = (_rand((1, 1, 4, 8), s) for s in (34, 35, 36))
    o1, l1 = attention.naive(q, k, v, 0.3)
    dead_o, dead_l = np.zeros_like(o1), np.full_like(l1, -np.inf)
    for o, lse in (attention.merge(o1, l1, dead_o, dead_l), attention.merge(dead_o, dead_l, o1, l1)):
        assert np.abs(o - o1).max() < 1e-15 and np.abs(lse - l1).max() < 1e-15
    o, lse = attention.merge(dead_o, dead_l, dead_o, dead_l)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_cross_attention_shapes_in_oracle():
    """Nq != Nk: the definition against a library routine."""
    q = _rand((2, 2, 13, 16), 37)
    k, v = _rand((2, 2, 40, 16), 38), _rand((2, 2, 40, 16), 39)
    o, _ = attention.naive(q, k, v, 0.25, key_len=np.array([40, 9]))
    keep = np.arange(40)[None, :] < np.array([40, 9])[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(keep[:, None, None, :]), scale=0.25).numpy()
    assert np.abs(o - ref).max() < 1e-12
