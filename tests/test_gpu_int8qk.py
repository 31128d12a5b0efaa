"""Parity of the INT8-QK entry points (fa_fwd_int8qk: FP8 P V;
fa_fwd_int8qk_pv16: 16-bit P V) with the oracle's exact emulation, and of
their quantised operands with the oracle's quantisers.

The quantised codes and scales are decided in float32 by the same steps on
both sides (the K mean is summed in float64 on both sides and rounded once),
so they are compared bit for bit.  The output is compared with the
emulation to 1e-2 max (+ the output type's half ulp) and 1e-3 mean, and
with unquantised attention by cosine >= 0.99 (the stated tolerances).

Those absolute bounds are loose where |O| is small (|O| ~ 0.006 at the
76112-token shape), so every case also bounds the error relative to the
emulation, row by row and over the case.  A correct kernel differs from the
float64 emulation by the rounding of O to the output type (per-row relative
RMS 1.64-1.68e-3 for bf16 and 2.06-2.31e-4 for fp16, measured over every
case here: the rounding noise of those formats) and by rare e4m3 codes of
448 P that round the other way because the kernel decides them from an fp32
exp2 and the emulation from an fp64 exp.  Such a flip moves one row (at small
N by up to ~1e-2 of |O|, visible above the fp16 noise); a wrong scale,
dropped tile or misplaced key moves every row.  So: the median per-row
relative RMS error sits within about 20 % of the rounding noise (ROW_MEDIAN),
at most 1 % of rows exceed five times that, and the relative RMS error over
the whole case and the cosine leave room for the flips (REL_RMS, COS_EMU).
"""
import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_04_amd as fa
from attention_fa_fwd_04_amd.workloads import WORKLOADS, Workload, make_inputs, sample_rows
from oracle import attention, rounding, sage

from gpu_masks import mask_layouts

pytestmark = pytest.mark.gpu

HALF_ULP = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
ROW_MEDIAN = {torch.float16: 2.6e-4, torch.bfloat16: 2.0e-3}
REL_RMS = {torch.float16: 8e-4, torch.bfloat16: 2.5e-3}
COS_EMU = 0.999996


def check_vs_emulation(got, ref, tdt, what):
    """Per-row and whole-case relative RMS error and cosine of the GPU output
    against the float64 emulation (rows with every key masked are exactly 0
    on both sides and are left out of the per-row statistics)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, 128)
    r = np.asarray(ref, dtype=np.float64).reshape(-1, 128)
    rn = np.sqrt((r * r).sum(axis=1))
    live = rn > 0
    assert np.all(g[~live] == 0), what
    row = np.sqrt(((g - r) ** 2).sum(axis=1))[live] / rn[live]
    med = float(np.median(row)) if row.size else 0.0
    bad = float((row > 5 * ROW_MEDIAN[tdt]).mean()) if row.size else 0.0
    rel = np.sqrt(((g - r) ** 2).sum() / max((r * r).sum(), 1e-300))
    cos = (g.ravel() @ r.ravel()) / max(np.linalg.norm(g) * np.linalg.norm(r), 1e-300)
    say(f"  {what}: per-row relRMS median {med:.3e} (rows > 5x bound: {bad:.2%}), relRMS {rel:.3e}, "
        f"cosine vs emulation {cos:.7f}")
    assert med <= ROW_MEDIAN[tdt], what
    assert bad <= 0.01, what
    assert rel <= REL_RMS[tdt], what
    assert cos >= COS_EMU, what


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    fa.lib()
    return torch.device("cuda", 0)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _a256(x):
    return (x + 255) // 256 * 256


def layout(B, H, N, D, vbytes=1):
    """Region offsets of the workspace as documented in include/fa.h."""
    bh, npad = B * H, (N + 63) // 64 * 64
    g = npad // 64
    off, out = 0, {}
    for name, nbytes in (("q8", bh * npad * D), ("k8", bh * npad * D), ("v8t", bh * D * npad * vbytes),
                         ("sq", bh * g * 4), ("sk", bh * g * 4), ("sv", bh * D * 4),
                         ("vmul", bh * D * 4), ("kmean", bh * D * 4)):
        out[name] = (off, nbytes)
        off = _a256(off + nbytes)
    return out, npad


def v8_pos(k):
    return 32 * ((k >> 2) & 1) + 16 * (k >> 5) + 4 * ((k >> 3) & 3) + (k & 3)


def v16_pos(k):
    return 32 * (k >> 5) + 16 * ((k >> 2) & 1) + 4 * ((k >> 3) & 3) + (k & 3)


def run(dev, inp, key_len=None, ws=None, pv="fp8"):
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    kl = None if key_len is None else key_len.to(dev)
    o, lse = fa.fwd_int8qk(q, k, v, key_len=kl, return_lse=True, workspace=ws, pv=pv)
    torch.cuda.synchronize()
    return o, lse


def test_kv_block_matches_oracle_block():
    assert fa.fa_int8qk_kv_block() == 64 and sage.QBLOCK == 64


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_quantised_operands_bit_exact(dev, dt):
    w = WORKLOADS[5].with_shape(H=3, N=1000, dtype=dt)
    inp = make_inputs(w)
    B, H, N, D = w.B, w.H, w.N, w.D
    ws = torch.empty(fa.fa_fwd_int8qk_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=dev)
    run(dev, inp, ws=ws)
    buf = ws.cpu().numpy()
    lay, npad = layout(B, H, N, D)

    def region(name, dtype, shape):
        off, nbytes = lay[name]
        return buf[off:off + nbytes].view(dtype).reshape(shape)

    q8 = region("q8", np.int8, (B * H, npad, D))
    k8 = region("k8", np.int8, (B * H, npad, D))
    v8t = region("v8t", np.uint8, (B * H, D, npad))
    sq = region("sq", np.float32, (B * H, npad // 64))
    sk = region("sk", np.float32, (B * H, npad // 64))
    sv = region("sv", np.float32, (B * H, D))
    km = region("kmean", np.float32, (B * H, D))
    perm = np.array([v8_pos(k) for k in range(64)])
    for h in range(H):
        qz = sage.quantise_head(inp["q"][0, h].double().numpy(), inp["k"][0, h].double().numpy(),
                                inp["v"][0, h].double().numpy())
        assert np.array_equal(km[h], qz["kmean"]), "kmean"
        assert np.array_equal(q8[h, :N], qz["q8"]) and not q8[h, N:].any(), "q8"
        assert np.array_equal(k8[h, :N], qz["k8"]), "k8"
        assert np.array_equal(sq[h], qz["sq"]) and np.array_equal(sk[h], qz["sk"]), "scales"
        assert np.array_equal(sv[h], qz["sv"]), "sv"
        vt = v8t[h].reshape(D, npad // 64, 64)[:, :, perm].reshape(D, npad)   # undo the key order
        vals = rounding.e4m3_bits_to_f64(vt[:, :N].T)
        assert np.array_equal(vals, qz["v8"]), "v8"


@pytest.mark.parametrize("keylen", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_int8qk_parity_small(dev, dt, keylen):
    for N in (1, 63, 64, 65, 127, 128, 129, 200, 1000):
        w = Workload(95, f"int8-{dt}", dt, 2, 2, N, 128, k_offset_var=2.0)
        inp = make_inputs(w)
        kl = torch.tensor([max(1, N // 3), N], dtype=torch.int32) if keylen else None
        say(f"case dt={dt} N={N} keylen={keylen}")
        o, lse = run(dev, inp, key_len=kl)
        qn, kn, vn = (inp[n].double().numpy() for n in ("q", "k", "v"))
        ref, ref_lse = sage.emulate(qn, kn, vn, w.scale, fa.fa_int8qk_kv_block(),
                                    key_len=None if kl is None else kl.numpy(), return_lse=True)
        got = o.cpu().double().numpy()
        err = np.abs(got - ref)
        say(f"  max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
        assert np.all(err <= 1e-2 + HALF_ULP[w.torch_dtype] * np.abs(ref))
        assert err.mean() <= 1e-3
        check_vs_emulation(got, ref, w.torch_dtype, f"N={N}")
        un, ul = attention.naive(qn, kn, vn, w.scale, key_len=None if kl is None else kl.numpy())
        cos = (got * un).sum() / np.linalg.norm(got) / np.linalg.norm(un)
        say(f"  cosine vs unquantised {cos:.5f}")
        assert cos >= 0.99
        # lse is that of the smoothed quantised scores
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 1e-4


@pytest.mark.parametrize("pv", ["fp8", "16"])
def test_int8qk_deterministic_and_in_bounds(dev, pv):
    """Through the C ABI: bitwise identical reruns (the phase-alternating
    loops read LDS tiles that other waves' DMA fills, so a missing wait would
    show as run-to-run differences) and guard bands around o and lse left
    untouched; N = 1111 leaves a ragged last tile and a partial query block."""
    w = Workload(97, f"int8-det-{pv}", "bf16", 1, 3, 1111, 128, k_offset_var=2.0)
    inp = make_inputs(w)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    B, H, N, D = q.shape
    G = 4096
    guard = torch.full((G + q.numel() + G,), 7.0, dtype=q.dtype, device=dev)
    lguard = torch.full((G + B * H * N + G,), 7.0, dtype=torch.float32, device=dev)
    o = guard[G:G + q.numel()].view(q.shape)
    lse = lguard[G:G + B * H * N].view(B, H, N)
    size, entry = ((fa.fa_fwd_int8qk_workspace_bytes, fa.fa_fwd_int8qk) if pv == "fp8" else
                   (fa.fa_fwd_int8qk_pv16_workspace_bytes, fa.fa_fwd_int8qk_pv16))
    ws = torch.empty(size(B, H, N, D), dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(3):
        rc = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), None, B, H, N, D,
                   w.scale, fa.FA_BF16, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    for oo, ll in outs[1:]:
        assert torch.equal(oo.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(ll.view(torch.int32), outs[0][1].view(torch.int32))
    assert torch.all(guard[:G] == 7) and torch.all(guard[-G:] == 7)
    assert torch.all(lguard[:G] == 7) and torch.all(lguard[-G:] == 7)
    assert torch.isfinite(o).all()


@pytest.mark.parametrize("pv", ["fp8", "16"])
def test_degenerate_quantisation_blocks(dev, pv):
    """Blocks whose quantisation scale is zero.  Head 0: an all-zero 64-token
    Q block (sq = 0, so those queries see equal scores); head 1: every key the
    same (K - kmean = 0, every sk = 0, so every query sees equal scores); head
    2: an all-zero V channel (its FP8 scale is 0).  Outputs against the
    emulation; the equal-score rows take the plain average of V, so they are
    identical, and the zero channel is exactly zero."""
    N, dt = 300, "bf16"
    w = Workload(99, "int8-degenerate", dt, 1, 3, N, 128, k_offset_var=2.0)
    inp = dict(make_inputs(w))
    q, k, v = (inp[n].clone() for n in ("q", "k", "v"))
    q[0, 0, 64:128] = 0
    k[0, 1] = k[0, 1, :1].expand(N, -1)
    v[0, 2, :, 5] = 0
    inp.update(q=q, k=k, v=v)
    say(f"case degenerate blocks pv={pv}")
    o, lse = run(dev, inp, pv=pv)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    ref, ref_lse = sage.emulate(qn, kn, vn, w.scale, fa.fa_int8qk_kv_block(), return_lse=True,
                                pv="fp8" if pv == "fp8" else EMU_PV[dt])
    got = o.cpu().double().numpy()
    err = np.abs(got - ref)
    say(f"  max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
    assert np.all(err <= 1e-2 + HALF_ULP[w.torch_dtype] * np.abs(ref))
    check_vs_emulation(got, ref, w.torch_dtype, f"degenerate pv={pv}")
    oc = o.cpu()
    assert torch.equal(oc[0, 0, 64:128], oc[0, 0, 64:65].expand(64, -1)), "zero Q block: equal rows"
    assert torch.equal(oc[0, 1], oc[0, 1, :1].expand(N, -1)), "equal keys: equal rows"
    assert torch.all(oc[0, 2, :, 5] == 0), "zero V channel"
    lg = lse.cpu().double().numpy()
    assert np.abs(lg - ref_lse).max() < 1e-4
    assert np.allclose(lg[0, 1], math.log(N), atol=1e-5), "equal scores: lse = ln N"


def test_int8qk_fully_masked_batch(dev):
    w = Workload(96, "int8-mask", "bf16", 2, 2, 100, 128)
    inp = make_inputs(w)
    o, lse = run(dev, inp, key_len=torch.tensor([0, 100], dtype=torch.int32))
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.isfinite(o[1]).all()


def test_int8qk_wan_full(dev):
    w = WORKLOADS[5]
    say(f"case {w}")
    inp = make_inputs(w)
    o, _ = run(dev, inp)
    rows = sample_rows(w, w.sampled_rows)
    o_c = o.cpu()
    errs, got_all, ref_all, un_all = [], [], [], []
    for h in sorted({int(r[1]) for r in rows}):
        ids = rows[rows[:, 1] == h][:, 2]
        qh, kh, vh = (inp[n][0, h].double().numpy() for n in ("q", "k", "v"))
        ref = sage.emulate_rows(qh, kh, vh, ids, w.scale, fa.fa_int8qk_kv_block())
        un, _ = attention.rows(qh[ids], kh, vh, w.scale)
        got = o_c[0, h, ids].double().numpy()
        errs.append(np.abs(got - ref))
        got_all.append(got)
        ref_all.append(ref)
        un_all.append(un)
    err = np.concatenate([e.ravel() for e in errs])
    g = np.concatenate(got_all).ravel()
    u = np.concatenate(un_all).ravel()
    cos = g @ u / np.linalg.norm(g) / np.linalg.norm(u)
    say(f"  {len(rows)} rows max|err|={err.max():.3e} mean|err|={err.mean():.3e} cosine={cos:.5f}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
    assert cos >= 0.99
    check_vs_emulation(g, np.concatenate(ref_all).ravel(), w.torch_dtype, f"{len(rows)} rows")


# ---- INT8-QK / 16-bit-PV (fa_fwd_int8qk_pv16) ----

EMU_PV = {"bf16": "bf16", "f16": "f16"}


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_pv16_operands_bit_exact(dev, dt):
    w = WORKLOADS[5].with_shape(H=2, N=1000, dtype=dt)
    inp = make_inputs(w)
    B, H, N, D = w.B, w.H, w.N, w.D
    ws = torch.empty(fa.fa_fwd_int8qk_pv16_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=dev)
    run(dev, inp, ws=ws, pv="16")
    buf = ws.cpu().numpy()
    lay, npad = layout(B, H, N, D, vbytes=2)

    def region(name, dtype, shape):
        off, nbytes = lay[name]
        return buf[off:off + nbytes].view(dtype).reshape(shape)

    q8 = region("q8", np.int8, (B * H, npad, D))
    k8 = region("k8", np.int8, (B * H, npad, D))
    vt = region("v8t", np.uint16, (B * H, D, npad))
    sq = region("sq", np.float32, (B * H, npad // 64))
    sk = region("sk", np.float32, (B * H, npad // 64))
    perm = np.array([v16_pos(k) for k in range(64)])
    vbits = inp["v"].view(torch.int16).numpy().astype(np.uint16)
    for h in range(H):
        qz = sage.quantise_head(inp["q"][0, h].double().numpy(), inp["k"][0, h].double().numpy(),
                                inp["v"][0, h].double().numpy())
        assert np.array_equal(q8[h, :N], qz["q8"]) and np.array_equal(k8[h, :N], qz["k8"]), "q8/k8"
        assert np.array_equal(sq[h], qz["sq"]) and np.array_equal(sk[h], qz["sk"]), "scales"
        got = vt[h].reshape(D, npad // 64, 64)[:, :, perm].reshape(D, npad)     # undo the key order
        assert np.array_equal(got[:, :N].T, vbits[0, h]), "V^T"
        assert not got[:, N:].any(), "padding keys"


@pytest.mark.parametrize("keylen", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_pv16_parity_small(dev, dt, keylen):
    for N in (1, 63, 64, 65, 200, 1000):
        w = Workload(97, f"int8pv16-{dt}", dt, 2, 2, N, 128, k_offset_var=2.0)
        inp = make_inputs(w)
        kl = torch.tensor([max(1, N // 3), N], dtype=torch.int32) if keylen else None
        say(f"case pv16 dt={dt} N={N} keylen={keylen}")
        o, lse = run(dev, inp, key_len=kl, pv="16")
        qn, kn, vn = (inp[n].double().numpy() for n in ("q", "k", "v"))
        ref, ref_lse = sage.emulate(qn, kn, vn, w.scale, fa.fa_int8qk_kv_block(),
                                    key_len=None if kl is None else kl.numpy(), return_lse=True, pv=EMU_PV[dt])
        got = o.cpu().double().numpy()
        err = np.abs(got - ref)
        say(f"  max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
        assert np.all(err <= 1e-2 + HALF_ULP[w.torch_dtype] * np.abs(ref))
        assert err.mean() <= 1e-3
        check_vs_emulation(got, ref, w.torch_dtype, f"N={N}")
        un, _ = attention.naive(qn, kn, vn, w.scale, key_len=None if kl is None else kl.numpy())
        cos = (got * un).sum() / np.linalg.norm(got) / np.linalg.norm(un)
        say(f"  cosine vs unquantised {cos:.5f}")
        assert cos >= 0.99
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 1e-4


def test_pv16_fully_masked_batch(dev):
    w = Workload(98, "int8pv16-mask", "f16", 2, 2, 100, 128)
    inp = make_inputs(w)
    o, lse = run(dev, inp, key_len=torch.tensor([0, 100], dtype=torch.int32), pv="16")
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.isfinite(o[1]).all()


def test_pv16_wan_full(dev):
    w = WORKLOADS[5]
    say(f"case pv16 {w}")
    inp = make_inputs(w)
    o, _ = run(dev, inp, pv="16")
    rows = sample_rows(w, w.sampled_rows)
    o_c = o.cpu()
    errs, got_all, ref_all, un_all = [], [], [], []
    for h in sorted({int(r[1]) for r in rows}):
        ids = rows[rows[:, 1] == h][:, 2]
        qh, kh, vh = (inp[n][0, h].double().numpy() for n in ("q", "k", "v"))
        ref = sage.emulate_rows(qh, kh, vh, ids, w.scale, fa.fa_int8qk_kv_block(), pv="bf16")
        un, _ = attention.rows(qh[ids], kh, vh, w.scale)
        got = o_c[0, h, ids].double().numpy()
        errs.append(np.abs(got - ref))
        got_all.append(got)
        ref_all.append(ref)
        un_all.append(un)
    err = np.concatenate([e.ravel() for e in errs])
    g = np.concatenate(got_all).ravel()
    u = np.concatenate(un_all).ravel()
    cos = g @ u / np.linalg.norm(g) / np.linalg.norm(u)
    say(f"  {len(rows)} rows max|err|={err.max():.3e} mean|err|={err.mean():.3e} cosine={cos:.5f}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
    assert cos >= 0.99
    check_vs_emulation(g, np.concatenate(ref_all).ravel(), w.torch_dtype, f"pv16 {len(rows)} rows")


# ---- additive masks (both P V forms) ----

def additive_mask(N, seed, B=2):
    """[B, 1, N, N] float32 (broadcast over heads): N(0, 4) values, 20 % of
    entries -inf, row 5 of batch 0 fully masked, and for every third row
    of batch 1 the keys 64..127 masked (a dead key tile)."""
    g = np.random.default_rng(seed)
    mv = g.standard_normal((B, 1, N, N)) * 2.0
    mv[g.random((B, 1, N, N)) < 0.2] = -np.inf
    if N > 5:
        mv[0, 0, 5] = -np.inf
    if N > 64:
        mv[1, 0, ::3, 64:128] = -np.inf
    return mv.astype(np.float32)


@pytest.mark.parametrize("pv", ["fp8", "16"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_additive_mask_parity(dev, dt, pv):
    for N in (1, 63, 64, 65, 129, 200, 1000):
        w = Workload(99, f"int8-add-{dt}", dt, 2, 2, N, 128, k_offset_var=2.0)
        inp = make_inputs(w)
        mv = additive_mask(N, 1000 + N)
        say(f"case additive mask pv={pv} dt={dt} N={N}")
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o, lse = fa.fwd_int8qk(q, k, v, attn_mask=torch.from_numpy(mv).to(dev), return_lse=True, pv=pv)
        torch.cuda.synchronize()
        qn, kn, vn = (inp[n].double().numpy() for n in ("q", "k", "v"))
        emu_pv = "fp8" if pv == "fp8" else dt
        ref, ref_lse = sage.emulate(qn, kn, vn, w.scale, fa.fa_int8qk_kv_block(), return_lse=True, pv=emu_pv,
                                    mask=mv.astype(np.float64))
        got = o.cpu().double().numpy()
        assert np.isfinite(got).all()
        err = np.abs(got - ref)
        say(f"  max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
        assert np.all(err <= 1e-2 + HALF_ULP[w.torch_dtype] * np.abs(ref))
        assert err.mean() <= 1e-3
        check_vs_emulation(got, ref, w.torch_dtype, f"N={N}")
        un, _ = attention.naive(qn, kn, vn, w.scale, mask=mv.astype(np.float64))
        cos = (got * un).sum() / np.linalg.norm(got) / np.linalg.norm(un)
        say(f"  cosine vs unquantised {cos:.5f}")
        assert cos >= 0.99
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 1e-4
        if N > 5:
            assert np.all(got[0, :, 5] == 0) and np.all(np.isneginf(lg[0, :, 5]))


def test_additive_mask_full_strides(dev):
    """A per-head [B, H, N, N] mask (no broadcast) through the FP8 form."""
    w = Workload(99, "int8-add-full", "bf16", 1, 3, 300, 128, k_offset_var=2.0)
    inp = make_inputs(w)
    g = np.random.default_rng(77)
    mv = (g.standard_normal((1, 3, 300, 300)) * 3.0).astype(np.float32)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = fa.fwd_int8qk(q, k, v, attn_mask=torch.from_numpy(mv).to(dev))
    torch.cuda.synchronize()
    qn, kn, vn = (inp[n].double().numpy() for n in ("q", "k", "v"))
    ref = sage.emulate(qn, kn, vn, w.scale, fa.fa_int8qk_kv_block(), mask=mv.astype(np.float64))
    got = o.cpu().double().numpy()
    assert np.abs(got - ref).max() <= 1e-2
    check_vs_emulation(got, ref, torch.bfloat16, "per-head mask")


@pytest.mark.parametrize("pv", ["fp8", "16"])
def test_additive_mask_layouts_int8(dev, pv):
    """The quantised kernels read every additive-mask layout (aligned rows,
    unaligned, transposed, broadcast over queries or over keys) to the
    emulation's result."""
    N = 200
    w = Workload(94, "int8-masklayout", "bf16", 2, 2, N, 128, k_offset_var=2.0)
    inp = make_inputs(w)
    qn, kn, vn = (inp[n].double().numpy() for n in ("q", "k", "v"))
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    for name, md in mask_layouts(dev, 2, 2, N, 12).items():
        say(f"case pv={pv} N={N} mask={name} strides={tuple(md.stride())}")
        o, lse = fa.fwd_int8qk(q, k, v, attn_mask=md, return_lse=True, pv=pv)
        torch.cuda.synchronize()
        mref = np.ascontiguousarray(np.broadcast_to(md.cpu().double().numpy(), (2, 2, N, N)))
        ref, ref_lse = sage.emulate(qn, kn, vn, w.scale, fa.fa_int8qk_kv_block(), return_lse=True,
                                    pv="fp8" if pv == "fp8" else "bf16", mask=mref)
        got = o.cpu().double().numpy()
        err = np.abs(got - ref)
        say(f"  max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
        assert np.all(err <= 1e-2 + HALF_ULP[w.torch_dtype] * np.abs(ref))
        assert err.mean() <= 1e-3
        check_vs_emulation(got, ref, w.torch_dtype, name)
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 1e-4


# ---- Q smoothing (fa_fwd_int8qk_smooth) ----

def offset_queries(inp, amp, seed):
    """Q plus a common offset per (b, h, 64-token block, channel) of +-amp, in
    Q's own dtype: the structure Q smoothing is for."""
    q = inp["q"]
    B, H, N, D = q.shape
    g = torch.Generator().manual_seed(seed)
    nb = (N + 63) // 64
    off = (torch.randint(0, 2, (B, H, nb, D), generator=g).float() * 2 - 1) * amp
    off = off.repeat_interleave(64, dim=2)[:, :, :N]
    out = dict(inp)
    out["q"] = (q.float() + off).to(q.dtype)
    return out


@pytest.mark.parametrize("pv", ["fp8", "16"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_smooth_operands_bit_exact(dev, dt, pv):
    """The smoothed Q codes and scales and the block means bit-exact against
    the oracle; the compensation table within float32 rounding of the
    oracle's float64 value times scale * log2(e)."""
    w = WORKLOADS[5].with_shape(H=2, N=200, dtype=dt)
    inp = offset_queries(make_inputs(w), 4.0, 1)
    B, H, N, D = w.B, w.H, w.N, w.D
    pv16 = 0 if pv == "fp8" else 1
    ws = torch.empty(fa.fa_fwd_int8qk_smooth_workspace_bytes(B, H, N, D, pv16), dtype=torch.uint8, device=dev)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    fa.fwd_int8qk(q, k, v, workspace=ws, pv=pv, smooth_q=True)
    torch.cuda.synchronize()
    buf = ws.cpu().numpy()
    lay, npad = layout(B, H, N, D, 1 if pv == "fp8" else 2)
    g = npad // 64
    base = (fa.fa_fwd_int8qk_workspace_bytes if pv == "fp8" else fa.fa_fwd_int8qk_pv16_workspace_bytes)(B, H, N, D)
    qbar_off = base
    comp_off = _a256(qbar_off + B * H * g * D * 4)

    def region(off, nbytes, dtype, shape):
        return buf[off:off + nbytes].view(dtype).reshape(shape)

    q8 = region(*lay["q8"], np.int8, (B * H, npad, D))
    sq = region(*lay["sq"], np.float32, (B * H, g))
    qbar = region(qbar_off, B * H * g * D * 4, np.float32, (B * H, g, D))
    comp = region(comp_off, B * H * g * npad * 4, np.float32, (B * H, g, npad))
    for h in range(H):
        qz = sage.quantise_head(inp["q"][0, h].double().numpy(), inp["k"][0, h].double().numpy(),
                                inp["v"][0, h].double().numpy(), smooth_q=True)
        assert np.array_equal(qbar[h], qz["qbar"]), "qbar"
        assert np.array_equal(q8[h, :N], qz["q8"]) and not q8[h, N:].any(), "q8"
        assert np.array_equal(sq[h], qz["sq"]), "sq"
        want = (qz["comp"] * (w.scale * math.log2(math.e))).astype(np.float32)
        got = comp[h, :, :N]
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        say(f"  head {h}: comp max|err| {err.max():.3e} (|comp| max {np.abs(want).max():.3e})")
        assert np.all(err <= 2.0 ** -22 * np.abs(want.astype(np.float64)) + 1e-30), "comp"


@pytest.mark.parametrize("keylen", [False, True])
@pytest.mark.parametrize("pv", ["fp8", "16"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_smooth_parity_small(dev, dt, pv, keylen):
    for N in (1, 63, 64, 65, 129, 200, 1000):
        w = Workload(92, f"int8-smooth-{dt}", dt, 2, 2, N, 128, k_offset_var=2.0)
        inp = offset_queries(make_inputs(w), 4.0, N)
        kl = torch.tensor([max(1, N // 3), N], dtype=torch.int32) if keylen else None
        say(f"case smooth pv={pv} dt={dt} N={N} keylen={keylen}")
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o, lse = fa.fwd_int8qk(q, k, v, key_len=None if kl is None else kl.to(dev), return_lse=True, pv=pv,
                               smooth_q=True)
        torch.cuda.synchronize()
        qn, kn, vn = (inp[n].double().numpy() for n in ("q", "k", "v"))
        ref, ref_lse = sage.emulate(qn, kn, vn, w.scale, fa.fa_int8qk_kv_block(), return_lse=True,
                                    key_len=None if kl is None else kl.numpy(),
                                    pv="fp8" if pv == "fp8" else dt, smooth_q=True)
        got = o.cpu().double().numpy()
        err = np.abs(got - ref)
        say(f"  max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
        assert np.all(err <= 1e-2 + HALF_ULP[w.torch_dtype] * np.abs(ref))
        assert err.mean() <= 1e-3
        check_vs_emulation(got, ref, w.torch_dtype, f"N={N}")
        un, _ = attention.naive(qn, kn, vn, w.scale, key_len=None if kl is None else kl.numpy())
        cos = (got * un).sum() / np.linalg.norm(got) / np.linalg.norm(un)
        say(f"  cosine vs unquantised {cos:.5f}")
        assert cos >= 0.99
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 1e-4


def test_smooth_gain_on_offset_queries(dev):
    """On queries with large per-block offsets the smoothed call is closer to
    unquantised attention than the plain INT8 one (16-bit P V, so that Q K^T
    quantisation is the main error); N = 5000 takes two 64-block tiles of the
    compensation table and many key tiles."""
    w = Workload(91, "int8-smooth-gain", "bf16", 1, 2, 5000, 128)
    inp = offset_queries(make_inputs(w), 20.0, 7)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o_s = fa.fwd_int8qk(q, k, v, pv="16", smooth_q=True)
    o_p = fa.fwd_int8qk(q, k, v, pv="16")
    torch.cuda.synchronize()
    rows = np.arange(0, 5000, 37)
    e = {}
    for name, o in (("smoothed", o_s), ("plain", o_p)):
        tot = 0.0
        for h in range(2):
            qh, kh, vh = (inp[n][0, h].double().numpy() for n in ("q", "k", "v"))
            un, _ = attention.rows(qh[rows], kh, vh, w.scale)
            tot += ((o[0, h, rows].cpu().double().numpy() - un) ** 2).sum()
        e[name] = np.sqrt(tot / (2 * len(rows) * 128))
    say(f"  rms error vs unquantised: smoothed {e['smoothed']:.3e}, plain {e['plain']:.3e}")
    assert e["smoothed"] < 0.5 * e["plain"]


def test_smooth_fully_masked_and_additive_refused(dev):
    w = Workload(90, "int8-smooth-mask", "bf16", 2, 2, 100, 128)
    inp = make_inputs(w)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd_int8qk(q, k, v, key_len=torch.tensor([0, 100], dtype=torch.int32, device=dev),
                           return_lse=True, smooth_q=True)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.isfinite(o[1]).all()
    with pytest.raises(fa.FAError):
        fa.fwd_int8qk(q, k, v, attn_mask=torch.zeros(1, 1, 100, 100, device=dev), smooth_q=True)
