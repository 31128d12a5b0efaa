"""The largest key lengths the 32-bit row addressing allows.

One head's rows are addressed with 32-bit byte offsets, so the library
accepts (N + 256) * D * sizeof(dtype) < 2^32 and rejects anything longer
(include/fa.h).  These tests run cross-attention at the largest accepted key
length for the long-sequence kernels, so the last rows sit just under 4 GiB
from the head's base: 400 query rows (more than the 384 the short-sequence
workgroups take, with a ragged last query tile) reach the phase-alternating
LDS-DMA kernel for bf16 D = 128 (no mask, key length), the in-step LDS-DMA
kernel for bf16 D = 128 with an additive mask, and the register-staged
kernel for fp16 D = 40.

Exact reference without a 4 GiB oracle: K and V repeat P distinct rows
(row j is row j mod P).  Attention over the repeated keys equals attention
over the P distinct keys with an additive mask of log(multiplicity) (each
copy contributes the same exp(score) and value), which the oracle's naive
formula computes directly; a key-length mask shortens the repeated sequence
first, which changes only the multiplicities.  An additive mask whose value
at key j depends only on j mod P adds that value to the distinct key's
log-multiplicity.
"""
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_04_amd as fa
from oracle import attention

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 32 - 1


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    fa.lib()
    return torch.device("cuda", 0)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def max_keys(D, elt):
    return LIMIT // (D * elt) - 256


def reduced_reference(q, k_small, v_small, nk, scale, key_len=None, mask_small=None):
    """Attention of q over k_small/v_small repeated to nk rows (row j = row j mod P),
    with an optional additive mask value mask_small[j mod P] on key j."""
    P = k_small.shape[0]
    n = nk if key_len is None else key_len
    counts = np.full(P, n // P, dtype=np.float64)
    counts[: n % P] += 1
    mask = np.where(counts > 0, np.log(np.maximum(counts, 1)), -np.inf)
    if mask_small is not None:
        mask = mask + mask_small
    mask = mask[None, None, None, :]
    o, lse = attention.naive(q[None, None], k_small[None, None], v_small[None, None], scale, mask=mask)
    return o[0, 0], lse[0, 0]


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 40)])
def test_largest_key_length(dev, dt, D):
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    elt = 2
    nk = max_keys(D, elt)
    assert (nk + 256) * D * elt <= LIMIT < (nk + 257) * D * elt
    P, nq = 997, 400
    say(f"case dt={dt} D={D} Nk={nk} ({nk * D * elt / 2 ** 30:.3f} GiB per K/V head)")
    g = torch.Generator().manual_seed(D)
    q = torch.randn(1, 1, nq, D, generator=g).to(tdt)
    ks = torch.randn(P, D, generator=g).to(tdt)
    vs = torch.randn(P, D, generator=g).to(tdt)
    reps = -(-nk // P)
    k = ks.to(dev).repeat(reps, 1)[:nk].reshape(1, 1, nk, D)
    v = vs.to(dev).repeat(reps, 1)[:nk].reshape(1, 1, nk, D)
    qd = q.to(dev)
    scale = 1.0 / np.sqrt(D)
    qn, kn, vn = (t.double().numpy().reshape(-1, D) for t in (q, ks, vs))
    for key_len in (None, nk - 3, 12345):
        kl = None if key_len is None else torch.tensor([key_len], dtype=torch.int32, device=dev)
        o, lse = fa.fwd(qd, k, v, key_len=kl, return_lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = reduced_reference(qn, kn, vn, nk, scale, key_len)
        got = o[0, 0].cpu().double().numpy()
        err = np.abs(got - ref)
        say(f"  key_len={key_len}: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
        half_ulp = 2.0 ** -8 if dt == "bf16" else 2.0 ** -11
        assert np.all(err <= 1e-2 + half_ulp * np.abs(ref)) and err.mean() <= 1e-3
        assert np.abs(lse[0, 0].cpu().double().numpy() - ref_lse).max() <= 1e-3
    if dt == "bf16":
        # a broadcast additive mask [1, 1, 1, Nk] (about 64 MB): value at key j
        # depends on j mod P; some distinct keys are dropped everywhere
        ms = np.random.default_rng(5).standard_normal(P).astype(np.float32)
        ms[::7] = -np.inf
        mfull = torch.from_numpy(ms).to(dev).repeat(reps)[:nk].reshape(1, 1, 1, nk)
        o, lse = fa.fwd(qd, k, v, attn_mask=mfull, return_lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = reduced_reference(qn, kn, vn, nk, scale, mask_small=ms.astype(np.float64))
        got = o[0, 0].cpu().double().numpy()
        err = np.abs(got - ref)
        say(f"  additive mask [1,1,1,Nk]: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
        assert np.all(err <= 1e-2 + 2.0 ** -8 * np.abs(ref)) and err.mean() <= 1e-3
        assert np.abs(lse[0, 0].cpu().double().numpy() - ref_lse).max() <= 1e-3
        del mfull
    # one key more is refused before anything is launched
    big = nk + 1
    rc = fa.fa_fwd_cross(qd.data_ptr(), k.data_ptr(), v.data_ptr(), torch.empty_like(qd).data_ptr(), None, None,
                         1, 1, nq, big, D, scale, fa.FA_BF16 if dt == "bf16" else fa.FA_F16, None)
    assert rc == fa.FA_ERR_SHAPE
    del k, v
    torch.cuda.empty_cache()
