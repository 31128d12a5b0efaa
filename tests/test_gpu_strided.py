"""Strided inputs (fa_fwd_strided): attention on [B, N, H, D] projection
outputs viewed as [B, H, N, D] without a copy.

Each case is checked two ways: (a) bit for bit against the contiguous entry
points on the same values (the kernels are the same; only the addressing
differs), and (b) element-wise against the oracle's fp64 definition with the
self-attention tolerances (1e-2 + the output type's half ulp max, 1e-3 mean
for fp16/bf16; 1e-5 for fp32).  Covers every kernel configuration (16-bit
D = 128 with LDS DMA, the register-staged kernel for D = 32 / 40 and fp32),
the three mask kinds, cross-attention lengths, ragged tails and an output in
a different layout from the inputs.
"""
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_04_amd as fa
from attention_fa_fwd_04_amd.workloads import Workload, make_inputs
from oracle import attention

pytestmark = pytest.mark.gpu

O_TOL = {torch.float32: (1e-5, None), torch.float16: (1e-2, 1e-3), torch.bfloat16: (1e-2, 1e-3)}
HALF_ULP = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    fa.lib()
    return torch.device("cuda", 0)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bnhd_inputs(dt, B, H, Nq, Nk, D, seed):
    """Seeded q [B, Nq, H, D] and k, v [B, Nk, H, D] (projection layout)."""
    wq = Workload(150 + seed, "strided-q", dt, B, H, Nq, D)
    wk = Workload(170 + seed, "strided-kv", dt, B, H, Nk, D)
    q = make_inputs(wq)["q"].transpose(1, 2).contiguous()
    kv = make_inputs(wk)
    return q, kv["k"].transpose(1, 2).contiguous(), kv["v"].transpose(1, 2).contiguous(), wq.scale


def check(o, ref, dtype, what):
    got = o.detach().cpu().double().numpy()
    err = np.abs(got - ref)
    mx, mean_tol = O_TOL[dtype]
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
    assert np.isfinite(got).all()
    assert np.all(err <= mx + HALF_ULP[dtype] * np.abs(ref)), what
    if mean_tol is not None:
        assert err.mean() <= mean_tol, what


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 128), ("f16", 40), ("bf16", 32), ("f32", 32), ("f32", 128)])
def test_strided_matches_contiguous_and_oracle(dev, dt, D):
    for (Nq, Nk) in ((333, 333), (129, 1000), (1000, 77)):
        for mask_kind in ("none", "keylen", "additive"):
            say(f"case dt={dt} D={D} Nq={Nq} Nk={Nk} mask={mask_kind}")
            B, H = 2, 3
            qb, kb, vb, scale = bnhd_inputs(dt, B, H, Nq, Nk, D, D % 5)
            kl = mask = None
            if mask_kind == "keylen":
                kl = torch.tensor([max(1, Nk // 2 + 3), Nk], dtype=torch.int32, device=dev)
            elif mask_kind == "additive":
                g = np.random.default_rng(Nq * 7 + Nk + D)
                mv = g.standard_normal((B, 1, Nq, Nk)) * 2.0
                mv[g.random((B, 1, Nq, Nk)) < 0.2] = -np.inf
                mask = torch.from_numpy(mv.astype(np.float32)).to(dev)
            q, k, v = (t.to(dev).transpose(1, 2) for t in (qb, kb, vb))      # [B, H, N, D] views
            assert not q.is_contiguous() and q.stride(3) == 1
            o, lse = fa.fwd(q, k, v, attn_mask=mask, key_len=kl, return_lse=True)
            oc, lsec = fa.fwd(q.contiguous(), k.contiguous(), v.contiguous(), attn_mask=mask, key_len=kl,
                              return_lse=True)
            torch.cuda.synchronize()
            assert o.stride() == q.stride()                                   # O keeps q's layout
            assert torch.equal(o.contiguous(), oc), "strided != contiguous"
            assert torch.equal(lse, lsec)
            ref, ref_l = attention.naive(q.cpu().double().numpy(), k.cpu().double().numpy(),
                                         v.cpu().double().numpy(), scale,
                                         mask=None if mask is None else mask.cpu().double().numpy(),
                                         key_len=None if kl is None else kl.cpu().numpy())
            check(o, ref, q.dtype, "O")
            fin = np.isfinite(ref_l)
            assert np.array_equal(np.isfinite(lse.cpu().numpy()), fin)
            assert np.abs(lse.cpu().double().numpy()[fin] - ref_l[fin]).max() <= 1e-4


def test_strided_output_layout_differs_from_inputs(dev):
    B, H, N, D = 1, 4, 700, 128
    qb, kb, vb, scale = bnhd_inputs("bf16", B, H, N, N, D, 9)
    q, k, v = (t.to(dev).transpose(1, 2) for t in (qb, kb, vb))
    out = torch.empty((B, H, N, D), dtype=q.dtype, device=dev)                # contiguous output
    o = fa.fwd(q, k, v, out=out)
    out2 = torch.empty((B, N, H, D), dtype=q.dtype, device=dev).transpose(1, 2)   # [B, N, H, D] output
    o2 = fa.fwd(q.contiguous(), k.contiguous(), v.contiguous(), out=out2)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and o2.data_ptr() == out2.data_ptr()
    assert torch.equal(o, o2.contiguous())
    ref, _ = attention.naive(q.cpu().double().numpy(), k.cpu().double().numpy(), v.cpu().double().numpy(), scale)
    check(o, ref, q.dtype, "O")


def test_strided_head_slices(dev):
    """Heads taken from a packed [B, N, 3, H, D] qkv projection (every q, k, v
    stride differs from a plain [B, N, H, D] tensor)."""
    B, N, H, D = 2, 515, 3, 40
    g = torch.Generator().manual_seed(5)
    qkv = torch.randn(B, N, 3, H, D, generator=g).to(torch.float16).to(dev)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    o = fa.fwd(q, k, v)
    oc = fa.fwd(q.contiguous(), k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous(), oc)
    ref, _ = attention.naive(q.cpu().double().numpy(), k.cpu().double().numpy(), v.cpu().double().numpy(),
                             1.0 / np.sqrt(D))
    check(o, ref, q.dtype, "O")
