"""The kernels' narrowing conversions, bit for bit against the format
definitions in oracle.rounding.

fa_cvt_probe runs the same device helpers the kernels use: e4m3x4 (448 P and
V of the quantised kernels: hardware v_cvt_pk_fp8_f32, OCP e4m3fn, round to
nearest even) and pack2<bf16 / fp16> (P of the 16-bit P V paths, and every
16-bit output).  The sweeps hold every representable value, every midpoint
between neighbours (where round-to-nearest-even decides), the fp32
neighbours of each midpoint, and log-uniform random values over the range
the kernels feed.  Ranges: e4m3 within +-448 (1 + 2^-22), which bounds every
input the kernels convert; bf16 and fp16 over normal fp32 values (fp32
subnormals excluded) and, for fp16, its own subnormal range, which small P
values reach.  Zero's sign is not compared (both zeros feed the matrix
cores as zero).
"""
import numpy as np
import pytest
import torch

import attention_fa_fwd_04_amd as fa
from oracle import rounding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    fa.lib()
    return torch.device("cuda", 0)


def probe(dev, kind, x):
    x = np.asarray(x, dtype=np.float32)
    n = len(x)
    xp = np.concatenate([x, np.zeros((-n) % 4, dtype=np.float32)])
    t = torch.from_numpy(xp).to(dev)
    out = torch.zeros(len(xp) * (1 if kind == 0 else 2), dtype=torch.uint8, device=dev)
    rc = fa.fa_cvt_probe(kind, t.data_ptr(), out.data_ptr(), len(xp), torch.cuda.current_stream(dev).cuda_stream)
    assert rc == fa.FA_OK
    torch.cuda.synchronize()
    b = out.cpu().numpy()
    return b[:n] if kind == 0 else b.view(np.uint16)[:n]


def with_midpoints(vals):
    """Sorted distinct values, their midpoints and the fp32 neighbours of each midpoint."""
    v = np.unique(np.asarray(vals, dtype=np.float64))
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (v[:-1] + v[1:]) / 2)   # midpoints exact in fp32
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    return np.concatenate([v.astype(np.float32), mid, up, dn])


def log_uniform(rng, lo, hi, n):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), n)).astype(np.float32)


def test_e4m3_rounding_bits(dev):
    pos = rounding.e4m3_bits_to_f64(np.arange(0, 0x7F, dtype=np.uint8))      # 0 .. 448
    rng = np.random.default_rng(11)
    x = np.concatenate([with_midpoints(pos), log_uniform(rng, 2.0 ** -12, 448.0, 200_000),
                        np.float32([448.0 * (1 + 2.0 ** -23), 448.0 * (1 + 2.0 ** -22)])])
    x = np.concatenate([x, -x])
    got = probe(dev, 0, x)
    want = rounding.f64_to_e4m3_bits(x.astype(np.float64))
    canon = lambda b: np.where((b & 0x7F) == 0, 0, b)           # noqa: E731  (+0 and -0)
    bad = np.flatnonzero(canon(got) != canon(want))
    print(f"e4m3: {len(x)} values, {len(bad)} mismatches", flush=True)
    assert len(bad) == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_bf16_rounding_bits(dev):
    # every bf16 value in [2^-126, 2^16), their midpoints and neighbours
    bits = np.arange(0x0080, 0x4780, dtype=np.uint32) << 16
    vals = bits.view(np.float32).astype(np.float64)
    rng = np.random.default_rng(12)
    x = np.concatenate([with_midpoints(vals), log_uniform(rng, 2.0 ** -126, 2.0 ** 100, 200_000)])
    x = np.concatenate([x, -x, np.float32([0.0])])
    got = probe(dev, 1, x)
    want = rounding.f32_to_bf16_bits(x)
    canon = lambda b: np.where((b & 0x7FFF) == 0, 0, b)         # noqa: E731
    bad = np.flatnonzero(canon(got) != canon(want))
    print(f"bf16: {len(x)} values, {len(bad)} mismatches", flush=True)
    assert len(bad) == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_f16_rounding_bits(dev):
    # every finite fp16 value (subnormals included), midpoints and neighbours
    bits = np.arange(0x0000, 0x7C00, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    rng = np.random.default_rng(13)
    x = np.concatenate([with_midpoints(vals), log_uniform(rng, 2.0 ** -30, 65504.0, 200_000)])
    x = x[np.abs(x) <= 65504.0]
    x = np.concatenate([x, -x])
    got = probe(dev, 2, x)
    want = rounding.f32_to_f16_bits(x)
    canon = lambda b: np.where((b & 0x7FFF) == 0, 0, b)         # noqa: E731
    bad = np.flatnonzero(canon(got) != canon(want))
    print(f"f16: {len(x)} values, {len(bad)} mismatches", flush=True)
    assert len(bad) == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]
