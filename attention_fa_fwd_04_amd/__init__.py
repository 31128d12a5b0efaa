"""MI355X (gfx950) attention forward: Python binding of libfa.so.

The C ABI is declared in include/fa.h.  This module only marshals arguments:
the raw entry points ``fa_fwd`` / ``fa_fwd_int8qk`` / ... take the same
arguments as their C counterparts (device pointers as ints), and the tensor
wrappers ``fwd`` / ``fwd_int8qk`` take torch tensors that already live on the
GPU, allocate the outputs with torch and pass torch's current stream.  Every
step of the computation runs in the HIP kernels; there is no fallback: if
libfa.so is missing or cannot be loaded, calls raise ``FAUnavailable``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_MASK_NONE, FA_MASK_ADDITIVE, FA_MASK_KEYLEN = 0, 1, 2
FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED = 0, -1, -2, -3
FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_ARG, FA_ERR_HIP = -4, -5, -6, -7

EXPORTED = ("fa_fwd", "fa_fwd_workspace_bytes", "fa_fwd_ws", "fa_fwd_ws_static", "fa_fwd_cross", "fa_fwd_strided",
            "fa_fwd_int8qk_workspace_bytes", "fa_fwd_int8qk",
            "fa_fwd_int8qk_pv16_workspace_bytes", "fa_fwd_int8qk_pv16",
            "fa_fwd_int8qk_smooth_workspace_bytes", "fa_fwd_int8qk_smooth",
            "fa_merge", "fa_mfma_probe", "fa_cvt_probe", "fa_int8qk_kv_block", "fa_status_string", "fa_last_hip_error", "fa_abi_version")


class FAUnavailable(RuntimeError):
    """libfa.so is not built or cannot be loaded."""


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where} failed: {status} ({status_string(status)})"
        if status == FA_ERR_HIP:
            msg += f": {last_hip_error()}"
        super().__init__(msg)
        self.status = status


class fa_mask_t(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("ptr", ctypes.c_void_p),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64)]


class fa_stride_t(ctypes.Structure):
    _fields_ = [("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libfa.so once and declare the C signatures."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise FAUnavailable(f"{LIB_PATH} is not built; run attention_fa_fwd_04_amd.build")
    try:
        h = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise FAUnavailable(f"cannot load {LIB_PATH}: {e}") from e
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    mp = ctypes.POINTER(fa_mask_t)
    h.fa_fwd.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, f32, i32, vp]
    h.fa_fwd.restype = i32
    h.fa_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    h.fa_fwd_workspace_bytes.restype = sz
    h.fa_fwd_ws.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    h.fa_fwd_ws.restype = i32
    h.fa_fwd_ws_static.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, f32, i32, vp]
    h.fa_fwd_ws_static.restype = i32
    h.fa_fwd_cross.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, i32, f32, i32, vp]
    h.fa_fwd_cross.restype = i32
    sp = ctypes.POINTER(fa_stride_t)
    h.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, i32, sp, sp, sp, sp, f32, i32, vp]
    h.fa_fwd_strided.restype = i32
    h.fa_fwd_int8qk_workspace_bytes.argtypes = [i32, i32, i32, i32]
    h.fa_fwd_int8qk_workspace_bytes.restype = sz
    h.fa_fwd_int8qk.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    h.fa_fwd_int8qk.restype = i32
    h.fa_fwd_int8qk_pv16_workspace_bytes.argtypes = [i32, i32, i32, i32]
    h.fa_fwd_int8qk_pv16_workspace_bytes.restype = sz
    h.fa_fwd_int8qk_pv16.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    h.fa_fwd_int8qk_pv16.restype = i32
    h.fa_fwd_int8qk_smooth_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    h.fa_fwd_int8qk_smooth_workspace_bytes.restype = sz
    h.fa_fwd_int8qk_smooth.argtypes = [vp, vp, vp, vp, vp, mp, i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
    h.fa_fwd_int8qk_smooth.restype = i32
    h.fa_merge.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    h.fa_merge.restype = i32
    h.fa_mfma_probe.argtypes = [i32, i32, i32, vp, vp]
    h.fa_mfma_probe.restype = i32
    h.fa_cvt_probe.argtypes = [i32, vp, vp, ctypes.c_int64, vp]
    h.fa_cvt_probe.restype = i32
    h.fa_int8qk_kv_block.argtypes = []
    h.fa_int8qk_kv_block.restype = i32
    h.fa_status_string.argtypes = [i32]
    h.fa_status_string.restype = ctypes.c_char_p
    h.fa_last_hip_error.argtypes = []
    h.fa_last_hip_error.restype = ctypes.c_char_p
    h.fa_abi_version.argtypes = []
    h.fa_abi_version.restype = i32
    _lib_handle = h
    return h


# ---- raw entry points (same names and arguments as the C ABI) -------------

def fa_fwd(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, hip_stream) -> int:
    return lib().fa_fwd(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, hip_stream)


def fa_fwd_workspace_bytes(B, H, N, D, dtype) -> int:
    return lib().fa_fwd_workspace_bytes(B, H, N, D, dtype)


def fa_fwd_ws(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, workspace, workspace_bytes,
              hip_stream) -> int:
    return lib().fa_fwd_ws(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, workspace,
                           workspace_bytes, hip_stream)


def fa_fwd_ws_static(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, hip_stream) -> int:
    return lib().fa_fwd_ws_static(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, hip_stream)


def fa_fwd_cross(q, k, v, o, lse, mask, B, H, Nq, Nk, D, scale, dtype, hip_stream) -> int:
    return lib().fa_fwd_cross(q, k, v, o, lse, mask, B, H, Nq, Nk, D, scale, dtype, hip_stream)


def fa_fwd_strided(q, k, v, o, lse, mask, B, H, Nq, Nk, D, q_strides, k_strides, v_strides,
                   o_strides, scale, dtype, hip_stream) -> int:
    return lib().fa_fwd_strided(q, k, v, o, lse, mask, B, H, Nq, Nk, D, q_strides, k_strides,
                                v_strides, o_strides, scale, dtype, hip_stream)


def fa_fwd_int8qk_workspace_bytes(B, H, N, D) -> int:
    return lib().fa_fwd_int8qk_workspace_bytes(B, H, N, D)


def fa_fwd_int8qk(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, workspace,
                  workspace_bytes, hip_stream) -> int:
    return lib().fa_fwd_int8qk(q, k, v, o, lse, mask, B, H, N, D, scale, dtype,
                               workspace, workspace_bytes, hip_stream)


def fa_fwd_int8qk_pv16_workspace_bytes(B, H, N, D) -> int:
    return lib().fa_fwd_int8qk_pv16_workspace_bytes(B, H, N, D)


def fa_fwd_int8qk_pv16(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, workspace,
                       workspace_bytes, hip_stream) -> int:
    return lib().fa_fwd_int8qk_pv16(q, k, v, o, lse, mask, B, H, N, D, scale, dtype,
                                    workspace, workspace_bytes, hip_stream)


def fa_merge(o_a, lse_a, o_b, lse_b, o, lse, B, H, N, D, dtype, hip_stream) -> int:
    return lib().fa_merge(o_a, lse_a, o_b, lse_b, o, lse, B, H, N, D, dtype, hip_stream)


def fa_mfma_probe(kind, workgroups, iters, out, hip_stream) -> int:
    return lib().fa_mfma_probe(kind, workgroups, iters, out, hip_stream)


def fa_cvt_probe(kind, inp, out, n, hip_stream) -> int:
    return lib().fa_cvt_probe(kind, inp, out, n, hip_stream)


PROBE_FLOPS = {0: 2.0 * 32 * 32 * 16, 1: 2.0 * 32 * 32 * 64, 2: 2.0 * 32 * 32 * 32}


def mfma_peak(kind: int, ms_target: float = 40.0, device=None, warmup_ms: float = 150.0) -> float:
    """Sustained dense MFMA rate (TFLOP/s or TOP/s) of one shape on the
    current GPU from fa_mfma_probe: kind 0 bf16, 1 fp8 e4m3, 2 int8.  After
    about warmup_ms of the probe (the clock ramps up from idle), the median
    of three runs of about ms_target milliseconds: the rate the part holds
    under load."""
    import torch
    dev = device or torch.device("cuda", torch.cuda.current_device())
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(4 * wgs, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev)

    def run(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        rc = fa_mfma_probe(kind, wgs, iters, out.data_ptr(), st.cuda_stream)
        e1.record(st)
        if rc != FA_OK:
            raise FAError(rc, "fa_mfma_probe")
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1)

    iters = 2000
    t = run(iters)
    iters = max(iters, int(iters * ms_target / max(t, 1e-3)))
    spent = 0.0
    while spent < warmup_ms:
        spent += run(iters)
    ts = sorted(run(iters) for _ in range(3))
    return wgs * 16 * iters * PROBE_FLOPS[kind] / (ts[1] * 1e-3) / 1e12


def fa_fwd_int8qk_smooth_workspace_bytes(B, H, N, D, pv16) -> int:
    return lib().fa_fwd_int8qk_smooth_workspace_bytes(B, H, N, D, pv16)


def fa_fwd_int8qk_smooth(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, pv16, workspace,
                         workspace_bytes, hip_stream) -> int:
    return lib().fa_fwd_int8qk_smooth(q, k, v, o, lse, mask, B, H, N, D, scale, dtype, pv16, workspace,
                                      workspace_bytes, hip_stream)


def fa_int8qk_kv_block() -> int:
    return lib().fa_int8qk_kv_block()


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


def fa_last_hip_error() -> str:
    return lib().fa_last_hip_error().decode()


def fa_abi_version() -> int:
    return lib().fa_abi_version()


status_string = fa_status_string
last_hip_error = fa_last_hip_error


# ---- torch tensor wrappers ------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_qkv(q, k, v, same_length=True, strided=False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, D], got {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if strided:
            if t.stride(3) != 1:
                raise ValueError(f"{name} must have contiguous D (stride(3) == 1)")
        elif not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, D]")
    if k.shape != v.shape:
        raise ValueError(f"k, v shapes differ: {tuple(k.shape)} {tuple(v.shape)}")
    if q.shape[0] != k.shape[0] or q.shape[1] != k.shape[1] or q.shape[3] != k.shape[3]:
        raise ValueError(f"q and k must share B, H, D: {tuple(q.shape)} {tuple(k.shape)}")
    if same_length and q.shape != k.shape:
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v dtypes differ")


def _mask_struct(q, attn_mask, key_len, keep, nk=None):
    """Build fa_mask_t from a torch mask.  Boolean masks follow the convention
    that False / 0 drops a key and become additive 0 / -inf float32."""
    import torch
    B, H, N, _ = q.shape
    Nk = N if nk is None else nk
    if attn_mask is not None and key_len is not None:
        raise ValueError("give either attn_mask or key_len, not both")
    if key_len is not None:
        kl = key_len.to(device=q.device, dtype=torch.int32).contiguous()
        if kl.shape != (B,):
            raise ValueError(f"key_len must have shape [{B}]")
        keep.append(kl)
        return fa_mask_t(FA_MASK_KEYLEN, kl.data_ptr(), 0, 0, 0, 0)
    if attn_mask is not None:
        m = attn_mask
        if m.dtype == torch.bool:
            m = torch.zeros(m.shape, dtype=torch.float32, device=m.device).masked_fill_(~m, float("-inf"))
        m = m.to(device=q.device, dtype=torch.float32)
        while m.dim() < 4:
            m = m.unsqueeze(0)
        m = m.expand(B, H, N, Nk)
        strides = [s if sz > 1 else 0 for s, sz in zip(m.stride(), m.shape)]
        keep.append(m)
        return fa_mask_t(FA_MASK_ADDITIVE, m.data_ptr(), *strides)
    return None


# Zero-filled workspaces of fa_fwd_ws, one per (device, stream): the arrival
# counters at their start return to zero after every completed call, so each
# is zero-filled once and reused by the calls queued on its stream.
_split_ws = {}


def split_workspace(device, stream, nbytes: int):
    """The cached fa_fwd_ws workspace for (device, stream), at least nbytes."""
    import torch
    key = (device.index, stream)
    ws = _split_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("fa_fwd_ws needs its workspace before graph capture: run the call "
                               "once eagerly on the capture stream first")
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _split_ws[key] = ws
    return ws


def fwd(q, k, v, *, attn_mask=None, key_len=None, scale: Optional[float] = None,
        return_lse: bool = False, out=None, split: bool = True):
    """O = softmax(scale * q k^T + mask) v for GPU tensors q [B, H, Nq, D] and
    k, v [B, H, Nk, D] (self-attention when Nq == Nk, else cross-attention).
    The tensors may be strided views with contiguous D (e.g. [B, N, H, D]
    projections viewed through .transpose(1, 2)); those go through
    fa_fwd_strided without a copy.  O has q's layout unless `out` is given.
    Contiguous unmasked self-attention goes through fa_fwd_ws (the even
    key-tile split) when the shape takes it, unless split=False."""
    import torch
    _check_qkv(q, k, v, same_length=False, strided=True)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or o.stride(3) != 1:
        raise ValueError("out must match q in shape and dtype, with contiguous D")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if return_lse else None
    keep = []
    m = _mask_struct(q, attn_mask, key_len, keep, nk=Nk)
    st = torch.cuda.current_stream(q.device).cuda_stream
    mp = ctypes.byref(m) if m is not None else None
    lp = lse.data_ptr() if lse is not None else None
    if not all(t.is_contiguous() for t in (q, k, v, o)):
        sd = [fa_stride_t(t.stride(0), t.stride(1), t.stride(2)) for t in (q, k, v, o)]
        rc = fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lp, mp,
                            B, H, Nq, Nk, D, *[ctypes.byref(x) for x in sd], scale, _dtype_code(q), st)
        where = "fa_fwd_strided"
    elif Nq == Nk:
        need = fa_fwd_workspace_bytes(B, H, Nq, D, _dtype_code(q)) if split and m is None else 0
        if need > 0:
            ws = split_workspace(q.device, st, need)
            rc = fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lp, mp,
                           B, H, Nq, D, scale, _dtype_code(q), ws.data_ptr(), ws.numel(), st)
            where = "fa_fwd_ws"
        else:
            rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lp, mp,
                        B, H, Nq, D, scale, _dtype_code(q), st)
            where = "fa_fwd"
    else:
        rc = fa_fwd_cross(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lp, mp,
                          B, H, Nq, Nk, D, scale, _dtype_code(q), st)
        where = "fa_fwd_cross"
    if rc != FA_OK:
        raise FAError(rc, where)
    return (o, lse) if return_lse else o


def fwd_int8qk(q, k, v, *, attn_mask=None, key_len=None, scale: Optional[float] = None,
               return_lse: bool = False, workspace=None, out=None, pv: str = "fp8", smooth_q: bool = False):
    """The INT8-QK variant for GPU tensors [B, H, N, 128] (bf16 / fp16): P V
    in FP8 (pv="fp8", fa_fwd_int8qk) or in the input's 16-bit type
    (pv="16", fa_fwd_int8qk_pv16).  Masks as for fwd (additive or boolean
    attn_mask broadcastable to [B, H, N, N], or key_len [B]).  smooth_q:
    Q smoothing with compensation as well (fa_fwd_int8qk_smooth; no
    additive mask; its workspace holds a [B*H, N/64, N] float32 table)."""
    import torch
    if pv not in ("fp8", "16"):
        raise ValueError('pv must be "fp8" or "16"')
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    pv16 = 0 if pv == "fp8" else 1
    if smooth_q:
        need = fa_fwd_int8qk_smooth_workspace_bytes(B, H, N, D, pv16)
        where = "fa_fwd_int8qk_smooth"
        entry = lambda *a: fa_fwd_int8qk_smooth(*a[:12], pv16, *a[12:])  # noqa: E731
    else:
        size_fn, entry, where = ((fa_fwd_int8qk_workspace_bytes, fa_fwd_int8qk, "fa_fwd_int8qk") if pv == "fp8" else
                                 (fa_fwd_int8qk_pv16_workspace_bytes, fa_fwd_int8qk_pv16, "fa_fwd_int8qk_pv16"))
        need = size_fn(B, H, N, D)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=q.device)
    keep = []
    m = _mask_struct(q, attn_mask, key_len, keep)
    st = torch.cuda.current_stream(q.device).cuda_stream
    rc = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
               lse.data_ptr() if lse is not None else None,
               ctypes.byref(m) if m is not None else None,
               B, H, N, D, scale, _dtype_code(q), ws.data_ptr(), ws.numel(), st)
    if rc != FA_OK:
        raise FAError(rc, where)
    return (o, lse) if return_lse else o


def merge(o_a, lse_a, o_b, lse_b, *, out=None, out_lse=None):
    """Combine two results over disjoint key sets of the same queries:
    O [B, H, N, D] and lse [B, H, N] per part; returns (O, lse).  out / out_lse
    may be o_a / lse_a to accumulate in place."""
    import torch
    for t in (o_a, o_b):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("partial outputs must be contiguous 4-D GPU tensors")
    if o_a.shape != o_b.shape or o_a.dtype != o_b.dtype:
        raise ValueError("partial outputs differ in shape or dtype")
    B, H, N, D = o_a.shape
    for t in (lse_a, lse_b):
        if t.shape != (B, H, N) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("lse must be contiguous float32 [B, H, N]")
    o = torch.empty_like(o_a) if out is None else out
    lse = torch.empty_like(lse_a) if out_lse is None else out_lse
    st = torch.cuda.current_stream(o_a.device).cuda_stream
    rc = fa_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(), o.data_ptr(),
                  lse.data_ptr(), B, H, N, D, _dtype_code(o_a), st)
    if rc != FA_OK:
        raise FAError(rc, "fa_merge")
    return o, lse
