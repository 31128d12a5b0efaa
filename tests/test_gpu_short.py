"""Short query sequences (Nq <= 384): batched window attention.

The case-study page (section 3.2) cuts the latent into non-overlapping 8x8
windows and runs attention inside each, batched over windows; such calls
take workgroups of one, two or four waves (32, 64 or 128 query rows).  Parity with the
CPU oracle element by element, for every head dimension, 16-bit dtype and
mask kind, window sizes on both sides of 32 rows, cross-attention with a
short query side, strided views, and the full SD1.5 window workload.
"""
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_04_amd as fa
from attention_fa_fwd_04_amd.workloads import WORKLOADS, Workload, make_inputs
from oracle import attention

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}
HALF_ULP = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    fa.lib()
    return torch.device("cuda", 0)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check(o, lse, ref_o, ref_l, dtype, what):
    o = o.detach().cpu().double().numpy()
    l = lse.detach().cpu().double().numpy()
    err = np.abs(o - ref_o)
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
    assert np.isfinite(o).all(), what
    assert np.all(err <= 1e-2 + HALF_ULP[dtype] * np.abs(ref_o)), what
    assert err.mean() <= 1e-3, what
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l)), what
    fin = np.isfinite(ref_l)
    if fin.any():
        assert np.abs(l[fin] - ref_l[fin]).max() <= 1e-4, what


def oracle(inp, scale, mask=None, key_len=None):
    return attention.naive(inp["q"].double().numpy(), inp["k"].double().numpy(), inp["v"].double().numpy(),
                           scale, mask=mask, key_len=key_len)


@pytest.mark.parametrize("mask_kind", ["none", "keylen", "additive"])
@pytest.mark.parametrize("D", [32, 40, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_windows(dev, dt, D, mask_kind):
    for B, H, N in [(40, 2, 16), (24, 3, 32), (12, 4, 49), (20, 3, 64), (6, 3, 100), (5, 2, 128), (3, 2, 300)]:
        w = Workload(120 + D, f"window-{dt}", dt, B, H, N, D)
        inp = make_inputs(w)
        kl = mask = None
        if mask_kind == "keylen":
            kl = torch.tensor([(7 * b) % (N + 1) for b in range(B)], dtype=torch.int32)   # includes 0 and N
        elif mask_kind == "additive":
            g = np.random.default_rng(N * 11 + D)
            mv = g.standard_normal((B, 1, N, N)) * 2.0
            mv[g.random((B, 1, N, N)) < 0.2] = -np.inf
            mask = torch.from_numpy(mv.astype(np.float32))
        say(f"case window dt={dt} D={D} B={B} H={H} N={N} mask={mask_kind}")
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o, lse = fa.fwd(q, k, v, attn_mask=None if mask is None else mask.to(dev),
                        key_len=None if kl is None else kl.to(dev), return_lse=True)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle(inp, w.scale, None if mask is None else mask.double().numpy(),
                              None if kl is None else kl.numpy())
        check(o, lse, ref_o, ref_l, DT[dt], f"B={B} H={H} N={N}")


@pytest.mark.parametrize("D", [40, 128])
def test_short_queries_long_keys(dev, D):
    """Cross-attention with a short query side: Nq <= 64 rows, many key tiles."""
    for Nq, Nk in [(1, 77), (30, 300), (64, 1000), (120, 700)]:
        w = Workload(130 + D, "short-cross", "f16", 3, 2, Nq, D, Nk=Nk)
        inp = make_inputs(w)
        say(f"case short-cross D={D} Nq={Nq} Nk={Nk}")
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o, lse = fa.fwd(q, k, v, return_lse=True)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle(inp, w.scale)
        check(o, lse, ref_o, ref_l, torch.float16, f"Nq={Nq} Nk={Nk}")


def test_short_strided_matches_contiguous(dev):
    """[B, N, H, D] window views through fa_fwd_strided equal the contiguous call bitwise."""
    w = Workload(140, "short-strided", "bf16", 16, 4, 64, 40)
    inp = make_inputs(w)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = fa.fwd(q, k, v)
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    os_ = fa.fwd(qs, ks, vs)
    torch.cuda.synchronize()
    assert not qs.is_contiguous()
    assert torch.equal(o.view(torch.int16), os_.contiguous().view(torch.int16))


def test_window_workload_full(dev):
    """The SD1.5 768^2 window workload (576 windows of 8x8 latents, 8 heads,
    D = 40, fp16) at full size, every element."""
    w = WORKLOADS[9]
    say(f"case {w}")
    inp = make_inputs(w)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle(inp, w.scale)
    check(o, lse, ref_o, ref_l, torch.float16, w.name)
