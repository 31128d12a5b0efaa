"""The C ABI library loads and exports what include/fa.h declares, and its
host-side validation rejects bad arguments before touching the GPU (these
calls return before any HIP runtime call, so they run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import attention_fa_fwd_04_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# a fake but 256-byte aligned, never dereferenced, device address
P = 1 << 20


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"FA_API\s+[\w\s\*]*?\b(fa_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.lib()


def test_header_declares_the_python_names():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing but the C ABI is exported (templates and helpers stay hidden)
    assert {e for e in exported if not e.startswith("_")} == set(declared_functions())


def test_static_queries(lib):
    assert fa.fa_abi_version() == 4
    assert fa.fa_int8qk_kv_block() % 64 == 0
    assert fa.fa_status_string(0) == "ok"
    for code in range(-7, 0):
        assert fa.fa_status_string(code) not in ("ok", "unknown status")
    assert fa.fa_status_string(-99) == "unknown status"
    assert fa.fa_last_hip_error() == ""


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, mask=None, B=1, H=2, N=64, D=128, scale=0.1, dtype=fa.FA_BF16,
             hip_stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["mask"], a["B"], a["H"], a["N"], a["D"],
                     a["scale"], a["dtype"], a["hip_stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(N=-3), fa.FA_ERR_SHAPE), (dict(D=0), fa.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 10, N=1 << 20), fa.FA_ERR_SHAPE),
    (dict(D=64), fa.FA_ERR_UNSUPPORTED), (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_ARG), (dict(scale=-1.0), fa.FA_ERR_ARG), (dict(scale=float("nan")), fa.FA_ERR_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_ARG),
    (dict(k=P + 8), fa.FA_ERR_ALIGN), (dict(lse=P + 2), fa.FA_ERR_ALIGN),
])
def test_fwd_validation(lib, kw, code):
    assert _fwd(**kw) == code


def test_mask_validation(lib):
    bad_kind = fa.fa_mask_t(9, P, 0, 0, 0, 0)
    assert _fwd(mask=ctypes.byref(bad_kind)) == fa.FA_ERR_ARG
    null_ptr = fa.fa_mask_t(fa.FA_MASK_KEYLEN, None, 0, 0, 0, 0)
    assert _fwd(mask=ctypes.byref(null_ptr)) == fa.FA_ERR_NULL
    misaligned = fa.fa_mask_t(fa.FA_MASK_ADDITIVE, P + 1, 0, 0, 64, 1)
    assert _fwd(mask=ctypes.byref(misaligned)) == fa.FA_ERR_ALIGN
    neg = fa.fa_mask_t(fa.FA_MASK_ADDITIVE, P, 0, 0, -64, 1)
    assert _fwd(mask=ctypes.byref(neg)) == fa.FA_ERR_ARG


def test_int8qk_validation(lib):
    ws = fa.fa_fwd_int8qk_workspace_bytes(1, 2, 1000, 128)
    assert ws > 3 * 2 * 1000 * 128
    assert fa.fa_fwd_int8qk_workspace_bytes(0, 2, 1000, 128) == 0

    def call(**kw):
        a = dict(dtype=fa.FA_BF16, D=128, ws=P, wsb=ws, mask=None)
        a.update(kw)
        return fa.fa_fwd_int8qk(P, P, P, P, None, a["mask"], 1, 2, 1000, a["D"], 0.1, a["dtype"],
                                a["ws"], a["wsb"], None)

    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert call(D=40) == fa.FA_ERR_UNSUPPORTED
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(wsb=ws - 1) == fa.FA_ERR_WORKSPACE
    assert call(ws=P + 16) == fa.FA_ERR_ALIGN
    # additive masks are taken; a malformed descriptor is refused before any launch
    for m, code in ((fa.fa_mask_t(fa.FA_MASK_ADDITIVE, None, 0, 0, 0, 1), fa.FA_ERR_NULL),
                    (fa.fa_mask_t(fa.FA_MASK_ADDITIVE, P + 2, 0, 0, 0, 1), fa.FA_ERR_ALIGN),
                    (fa.fa_mask_t(fa.FA_MASK_ADDITIVE, P, 0, 0, -1, 1), fa.FA_ERR_ARG)):
        assert call(mask=ctypes.byref(m)) == code


def test_cvt_probe_validation(lib):
    assert fa.fa_cvt_probe(0, None, P, 16, None) == fa.FA_ERR_NULL
    assert fa.fa_cvt_probe(0, P, None, 16, None) == fa.FA_ERR_NULL
    assert fa.fa_cvt_probe(1, P, P, 0, None) == fa.FA_ERR_SHAPE
    assert fa.fa_cvt_probe(1, P, P, 6, None) == fa.FA_ERR_SHAPE
    assert fa.fa_cvt_probe(2, P + 4, P, 16, None) == fa.FA_ERR_ALIGN
    assert fa.fa_cvt_probe(2, P, P + 4, 16, None) == fa.FA_ERR_ALIGN
    assert fa.fa_cvt_probe(3, P, P, 16, None) == fa.FA_ERR_ARG


def test_wrapper_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)


def test_cross_validation(lib):
    def call(**kw):
        a = dict(q=P, k=P, v=P, o=P, Nq=100, Nk=77, D=40, dtype=fa.FA_F16, scale=0.1)
        a.update(kw)
        return fa.fa_fwd_cross(a["q"], a["k"], a["v"], a["o"], None, None, 2, 8, a["Nq"], a["Nk"], a["D"],
                               a["scale"], a["dtype"], None)
    assert call(Nk=0) == fa.FA_ERR_SHAPE
    assert call(Nq=0) == fa.FA_ERR_SHAPE
    assert call(v=None) == fa.FA_ERR_NULL
    assert call(D=64) == fa.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == fa.FA_ERR_ARG


def test_merge_validation(lib):
    def call(**kw):
        a = dict(oa=P, la=P, ob=P, lb=P, o=P, lse=None, N=10, D=128, dtype=fa.FA_BF16)
        a.update(kw)
        return fa.fa_merge(a["oa"], a["la"], a["ob"], a["lb"], a["o"], a["lse"], 1, 2, a["N"], a["D"],
                           a["dtype"], None)
    assert call(oa=None) == fa.FA_ERR_NULL
    assert call(lb=None) == fa.FA_ERR_NULL
    assert call(N=0) == fa.FA_ERR_SHAPE
    assert call(D=36) == fa.FA_ERR_UNSUPPORTED          # 72 bytes: not whole 16-byte chunks
    assert call(D=1024) == fa.FA_ERR_UNSUPPORTED        # rows over 1 KB
    assert call(dtype=9) == fa.FA_ERR_UNSUPPORTED
    assert call(o=P + 8) == fa.FA_ERR_ALIGN
    assert call(lse=P + 2) == fa.FA_ERR_ALIGN


def test_strided_validation(lib):
    ok = fa.fa_stride_t(4 * 100 * 8 * 128, 128, 8 * 128)     # [B, N, H, D] view, H = 8, D = 128

    def call(q=ok, k=ok, v=ok, o=ok, **kw):
        a = dict(ptr=P, Nq=100, Nk=100, D=128, dtype=fa.FA_BF16)
        a.update(kw)
        ref = [None if s is None else ctypes.byref(s) for s in (q, k, v, o)]
        return fa.fa_fwd_strided(a["ptr"], P, P, P, None, None, 4, 8, a["Nq"], a["Nk"], a["D"], *ref,
                                 0.1, a["dtype"], None)
    assert call(q=None) == fa.FA_ERR_NULL
    assert call(o=None) == fa.FA_ERR_NULL
    assert call(k=fa.fa_stride_t(-1, 128, 1024)) == fa.FA_ERR_ARG
    assert call(v=fa.fa_stride_t(0, 0, 0)) == fa.FA_ERR_ARG
    assert call(o=fa.fa_stride_t(0, 128, 64)) == fa.FA_ERR_ARG          # output rows overlap
    assert call(q=fa.fa_stride_t(0, 128, 1028)) == fa.FA_ERR_ALIGN       # rows not 16-byte aligned
    assert call(k=fa.fa_stride_t(4, 128, 1024)) == fa.FA_ERR_ALIGN       # batch base not aligned
    assert call(Nk=1 << 21, k=fa.fa_stride_t(0, 0, 1 << 10)) == fa.FA_ERR_SHAPE   # 4 GiB range
    assert call(Nq=0) == fa.FA_ERR_SHAPE
    assert call(D=64) == fa.FA_ERR_UNSUPPORTED
    assert call(dtype=5) == fa.FA_ERR_UNSUPPORTED
    assert call(ptr=None) == fa.FA_ERR_NULL


def test_contiguous_range_limit(lib):
    # rows * D * 2 bytes beyond the 32-bit buffer range of one (b, h) head
    assert _fwd(N=1 << 24, D=128) == fa.FA_ERR_SHAPE


def test_int8qk_pv16_validation(lib):
    ws = fa.fa_fwd_int8qk_pv16_workspace_bytes(1, 2, 1000, 128)
    assert ws > fa.fa_fwd_int8qk_workspace_bytes(1, 2, 1000, 128)     # 16-bit V^T region
    assert fa.fa_fwd_int8qk_pv16_workspace_bytes(1, 0, 1000, 128) == 0

    def call(**kw):
        a = dict(dtype=fa.FA_BF16, D=128, ws=P, wsb=ws, mask=None, N=1000)
        a.update(kw)
        return fa.fa_fwd_int8qk_pv16(P, P, P, P, None, a["mask"], 1, 2, a["N"], a["D"], 0.1, a["dtype"],
                                     a["ws"], a["wsb"], None)
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert call(D=40) == fa.FA_ERR_UNSUPPORTED
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(wsb=fa.fa_fwd_int8qk_workspace_bytes(1, 2, 1000, 128)) == fa.FA_ERR_WORKSPACE
    assert call(ws=P + 16) == fa.FA_ERR_ALIGN
    assert call(N=1 << 24) == fa.FA_ERR_SHAPE
    neg = fa.fa_mask_t(fa.FA_MASK_ADDITIVE, P, -1, 0, 0, 1)
    assert call(mask=ctypes.byref(neg)) == fa.FA_ERR_ARG


def test_fwd_ws_outside_split_domain(lib):
    """Shapes the key-tile split does not take (decided before any device
    query): the workspace size is 0 and fa_fwd_ws validates like fa_fwd."""
    for B, H, N, D, dt in [(1, 24, 4608, 40, fa.FA_F16), (1, 24, 4608, 128, fa.FA_F32),
                           (1, 24, 4600, 128, fa.FA_BF16), (0, 24, 4608, 128, fa.FA_BF16)]:
        assert fa.fa_fwd_workspace_bytes(B, H, N, D, dt) == 0

    def call(**kw):
        a = dict(q=P, B=1, H=2, N=100, D=40, dtype=fa.FA_F16, scale=0.1, mask=None)
        a.update(kw)
        return fa.fa_fwd_ws(a["q"], P, P, P, None, a["mask"], a["B"], a["H"], a["N"], a["D"], a["scale"],
                            a["dtype"], None, 0, None)
    assert call(q=None) == fa.FA_ERR_NULL
    assert call(D=64) == fa.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == fa.FA_ERR_ARG
    assert call(B=0) == fa.FA_ERR_SHAPE
    assert call(q=P + 8) == fa.FA_ERR_ALIGN


def test_fwd_ws_static_outside_split_domain(lib):
    """Shapes the split does not take run fa_fwd, with its validation
    (decided before any device query, so no GPU is touched)."""
    def call(**kw):
        a = dict(q=P, B=1, H=2, N=100, D=40, dtype=fa.FA_F16, scale=0.1, mask=None)
        a.update(kw)
        return fa.fa_fwd_ws_static(a["q"], P, P, P, None, a["mask"], a["B"], a["H"], a["N"], a["D"], a["scale"],
                                   a["dtype"], None)
    assert call(q=None) == fa.FA_ERR_NULL
    assert call(D=64) == fa.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == fa.FA_ERR_ARG
    assert call(B=0) == fa.FA_ERR_SHAPE
    assert call(q=P + 8) == fa.FA_ERR_ALIGN


def test_int8qk_smooth_validation(lib):
    """Q smoothing's entry point: the workspace adds the block means and the
    [B*H, Np/64, Np] float32 compensation table to the chosen P V form's."""
    for pv16, base in ((0, fa.fa_fwd_int8qk_workspace_bytes), (1, fa.fa_fwd_int8qk_pv16_workspace_bytes)):
        ws = fa.fa_fwd_int8qk_smooth_workspace_bytes(1, 2, 1000, 128, pv16)
        groups, npad = 16, 1024
        assert ws >= base(1, 2, 1000, 128) + 2 * groups * 128 * 4 + 2 * groups * npad * 4
        assert ws <= base(1, 2, 1000, 128) + 2 * groups * 128 * 4 + 2 * groups * npad * 4 + 512
    assert fa.fa_fwd_int8qk_smooth_workspace_bytes(1, 2, 1000, 128, 2) == 0
    assert fa.fa_fwd_int8qk_smooth_workspace_bytes(0, 2, 1000, 128, 0) == 0
    ws = fa.fa_fwd_int8qk_smooth_workspace_bytes(1, 2, 1000, 128, 0)

    def call(**kw):
        a = dict(dtype=fa.FA_BF16, D=128, ws=P, wsb=ws, mask=None, N=1000, pv16=0)
        a.update(kw)
        return fa.fa_fwd_int8qk_smooth(P, P, P, P, None, a["mask"], 1, 2, a["N"], a["D"], 0.1, a["dtype"],
                                       a["pv16"], a["ws"], a["wsb"], None)
    assert call(pv16=2) == fa.FA_ERR_ARG
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert call(D=40) == fa.FA_ERR_UNSUPPORTED
    add = fa.fa_mask_t(fa.FA_MASK_ADDITIVE, P, 0, 0, 0, 1)
    assert call(mask=ctypes.byref(add)) == fa.FA_ERR_UNSUPPORTED
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(wsb=fa.fa_fwd_int8qk_workspace_bytes(1, 2, 1000, 128)) == fa.FA_ERR_WORKSPACE
    assert call(pv16=1) == fa.FA_ERR_WORKSPACE          # the 16-bit form's workspace is larger
    assert call(ws=P + 16) == fa.FA_ERR_ALIGN
    assert call(N=1 << 24) == fa.FA_ERR_SHAPE


def test_int8qk_smooth_table_limit(lib):
    """One head's compensation table stays under 2^31 bytes: N = 185,344 is
    accepted as far as the workspace check, one 64-token block more is not."""
    def call(N):
        return fa.fa_fwd_int8qk_smooth(P, P, P, P, None, None, 1, 1, N, 128, 0.1, fa.FA_BF16, 0, P, 0, None)
    assert call(185344) == fa.FA_ERR_WORKSPACE
    assert call(185345) == fa.FA_ERR_SHAPE


def test_int8qk_batch_head_limit(lib):
    """B*H above 65535 is refused before any launch, by every quantised entry point."""
    ws = fa.fa_fwd_int8qk_workspace_bytes(1, 1, 64, 128)
    assert fa.fa_fwd_int8qk(P, P, P, P, None, None, 2, 32768, 64, 128, 0.1, fa.FA_BF16, P, ws, None) == fa.FA_ERR_SHAPE
    assert fa.fa_fwd_int8qk_pv16(P, P, P, P, None, None, 65536, 1, 64, 128, 0.1, fa.FA_BF16, P, ws,
                                 None) == fa.FA_ERR_SHAPE
    assert fa.fa_fwd_int8qk_smooth(P, P, P, P, None, None, 256, 257, 64, 128, 0.1, fa.FA_BF16, 0, P, ws,
                                   None) == fa.FA_ERR_SHAPE
    # 65535 itself passes the shape checks (and fails on the tiny workspace)
    assert fa.fa_fwd_int8qk(P, P, P, P, None, None, 5, 13107, 64, 128, 0.1, fa.FA_BF16, P, ws, None) == fa.FA_ERR_WORKSPACE
