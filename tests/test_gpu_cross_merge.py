"""Cross-attention (Nq != Nk) and the merge of results over split key sets,
against the oracle.

Cross-attention: element-wise against the fp64 definition, same tolerances as
the self-attention parity tests (1e-2 + the output type's half ulp max, 1e-3
mean for fp16/bf16; 1e-5 for fp32), including the SD1.5 text
cross-attention shape (4096 latents x 77 text tokens, D = 40).
Merge: (a) the GPU merge of two GPU partials equals the oracle's merge of the
same partials up to fp32 arithmetic and the output rounding (one ulp of the
output type); (b) attention over keys [0, s) and [s, Nk) merged on the GPU
matches attention over all keys within the self-attention tolerances.
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
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    fa.lib()
    return torch.device("cuda", 0)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cross_inputs(dt, B, H, Nq, Nk, D, seed):
    wq = Workload(110 + seed, "cross-q", dt, B, H, Nq, D)
    wk = Workload(130 + seed, "cross-kv", dt, B, H, Nk, D)
    q = make_inputs(wq)["q"]
    kv = make_inputs(wk)
    return q, kv["k"], kv["v"], wq.scale


def check(o, ref, dtype, what):
    got = o.detach().cpu().double().numpy()
    err = np.abs(got - ref)
    mx, mean_tol = O_TOL[dtype]
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
    assert np.isfinite(got).all()
    assert np.all(err <= mx + HALF_ULP[dtype] * np.abs(ref)), what
    if mean_tol is not None:
        assert err.mean() <= mean_tol, what


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [32, 40, 128])
def test_cross_attention(dev, dt, D):
    for (Nq, Nk) in ((4096, 77), (200, 1000), (1000, 65), (1, 300), (300, 1)):
        for mask_kind in ("none", "keylen", "additive"):
            say(f"case dt={dt} D={D} Nq={Nq} Nk={Nk} mask={mask_kind}")
            q, k, v = cross_inputs(dt, 2, 2, Nq, Nk, D, D % 7)[:3]
            scale = 1.0 / np.sqrt(D)
            kl = mask = None
            if mask_kind == "keylen":
                kl = torch.tensor([max(1, Nk // 3), Nk], dtype=torch.int32)
            elif mask_kind == "additive":
                g = np.random.default_rng(Nq + Nk + D)
                mv = g.standard_normal((2, 1, Nq, Nk)) * 2.0
                mv[g.random((2, 1, Nq, Nk)) < 0.2] = -np.inf
                mask = torch.from_numpy(mv.astype(np.float32))
            o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), attn_mask=None if mask is None else mask.to(dev),
                            key_len=None if kl is None else kl.to(dev), return_lse=True)
            torch.cuda.synchronize()
            ref, ref_l = attention.naive(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                                         mask=None if mask is None else mask.double().numpy(),
                                         key_len=None if kl is None else kl.numpy())
            check(o, ref, DT[dt], f"{Nq}x{Nk}")
            lg = lse.cpu().double().numpy()
            assert np.array_equal(np.isneginf(lg), np.isneginf(ref_l))
            fin = np.isfinite(ref_l)
            assert np.abs(lg[fin] - ref_l[fin]).max() <= (1e-5 if dt == "f32" else 1e-4)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_merge_matches_oracle_merge(dev, dt):
    """The merge itself: GPU partials in, compared with the oracle's merge of the
    very same partials (only fp32 arithmetic and the output rounding differ)."""
    D = 128 if dt != "f16" else 40
    q, k, v, scale = cross_inputs(dt, 1, 3, 700, 900, D, 3)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    s = 333
    oa, la = fa.fwd(qd, kd[:, :, :s].contiguous(), vd[:, :, :s].contiguous(), return_lse=True)
    ob, lb = fa.fwd(qd, kd[:, :, s:].contiguous(), vd[:, :, s:].contiguous(), return_lse=True)
    la[0, 1, 5] = float("-inf")            # one row empty on one side
    la[0, 2, 7] = float("-inf")
    lb[0, 2, 7] = float("-inf")            # and one row empty on both
    oa[0, 2, 7] = 0
    ob[0, 2, 7] = 0
    o, lse = fa.merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    ref, ref_l = attention.merge(oa.cpu().double().numpy(), la.cpu().double().numpy(),
                                 ob.cpu().double().numpy(), lb.cpu().double().numpy())
    got = o.cpu().double().numpy()
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dt]
    assert np.all(np.abs(got - ref) <= ulp * np.abs(ref) + 1e-6)
    lg = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(lg[fin] - ref_l[fin]).max() < 1e-5
    assert torch.all(o[0, 2, 7] == 0)
    # in place into the first part
    o2, l2 = fa.merge(oa, la, ob, lb, out=oa, out_lse=la)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(l2, lse)


@pytest.mark.parametrize("parts", [2, 4])
def test_key_split_merged_equals_full_attention(dev, parts):
    """Sequence-sharded K/V on one GPU: attention over each key shard, merged
    in order, equals attention over all keys."""
    q, k, v, scale = cross_inputs("bf16", 1, 4, 1111, 2345, 128, 5)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    cuts = np.linspace(0, 2345, parts + 1).astype(int)
    o = lse = None
    for a, b in zip(cuts[:-1], cuts[1:]):
        op, lp = fa.fwd(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), return_lse=True)
        if o is None:
            o, lse = op, lp
        else:
            o, lse = fa.merge(o, lse, op, lp, out=o, out_lse=lse)
    torch.cuda.synchronize()
    ref, ref_l = attention.naive(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale)
    check(o, ref, torch.bfloat16, f"{parts} shards")
    assert np.abs(lse.cpu().double().numpy() - ref_l).max() < 1e-4
