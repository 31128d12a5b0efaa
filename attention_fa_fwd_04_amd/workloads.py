"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random tensors and rounds them to the storage dtype.
It holds none of the attention arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it without sharing any computation.

Workloads (shapes follow the handbook page "算子加速：注意力、编译与融合",
section "注意力：从 O(N²) 显存到分块", its byte table and worked example, and
the case-study page's resolution / batching discussion, section 2.2):

  1  tiny fp32    B=1 H=4  N=256    D=32   the handbook's worked example
  2  FLUX 1024²   B=1 H=24 N=4608   D=128  bf16, no mask
  3  SD1.5 768²   B=4 H=8  N=9216   D=40   fp16, per-sample key length
  4  video 720p   B=1 H=24 N=119056 D=128  bf16, 4 K outlier channels x8
  5  Wan 2.1 720p B=1 H=40 N=76112  D=128  bf16, per-(b,h) K channel offset

Recipe: workload 1 reproduces the worked example exactly (torch CPU RNG,
manual_seed(0), then q, k, v drawn with randn in that order).  Workloads 2-5
draw each (tensor, b, h) head from its own numpy Generator seeded with
SeedSequence([workload, tensor_id, b, h]) as float32 N(0, 1), then round to
the storage dtype; the rounded values are the ground truth for both sides.
Per-head streams let the oracle rebuild one head without the others.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

# tensor ids inside a workload's seed tree
T_Q, T_K, T_V, T_LEN, T_CHAN, T_KOFF, T_ROWS = 0, 1, 2, 3, 4, 5, 6

_TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    dtype: str          # storage dtype of q, k, v, o: "f32" | "f16" | "bf16"
    B: int
    H: int
    N: int
    D: int
    key_len: bool = False        # per-sample valid key length in [N/2, N]
    outlier_channels: int = 0    # K channels scaled by outlier_scale
    outlier_scale: float = 8.0
    k_offset_var: float = 0.0    # per-(b,h,channel) K offset ~ N(0, var)
    quantised: bool = False      # run through the INT8-QK / FP8-PV entry point
    pv16: bool = False           # with quantised: the INT8-QK / 16-bit-PV form instead
    sampled_rows: int = 0        # rows the oracle checks at full size (0 = all)
    Nk: int = 0                  # key / value length when it differs from N (cross-attention)
    merge: bool = False          # time the merge of two partial results of this shape

    @property
    def n_keys(self) -> int:
        return self.Nk if self.Nk else self.N

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    def with_shape(self, **kw) -> "Workload":
        """Same recipe at another size (parity cases that span tiles and tails)."""
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny-fp32", "f32", 1, 4, 256, 32),
    2: Workload(2, "flux-1024", "bf16", 1, 24, 4608, 128),
    3: Workload(3, "sd15-768-keylen", "f16", 4, 8, 9216, 40, key_len=True),
    4: Workload(4, "video-720p", "bf16", 1, 24, 119056, 128,
                outlier_channels=4, sampled_rows=512),
    5: Workload(5, "wan-720p-int8qk", "bf16", 1, 40, 76112, 128,
                k_offset_var=2.0, quantised=True, sampled_rows=512),
    # cross-attention of an SD1.5 768^2 UNet block (4096 latents x 77 text tokens)
    6: Workload(6, "sd15-text-cross", "f16", 2, 8, 4096, 40, Nk=77),
    # merge of two partial results of the FLUX-1024^2 layer (key split)
    7: Workload(7, "flux-1024-merge", "bf16", 1, 24, 4608, 128, merge=True),
    # the Wan 2.1 inputs of workload 5 through the INT8-QK / 16-bit-PV form
    8: Workload(5, "wan-720p-int8qk-pv16", "bf16", 1, 40, 76112, 128,
                k_offset_var=2.0, quantised=True, pv16=True, sampled_rows=512),
    # window attention of an SD1.5 768^2 UNet block: the 96x96 latent cut into
    # 8x8 windows (144 per image, 4 images) batched as 576 sequences of 64
    9: Workload(9, "sd15-768-window8x8", "f16", 576, 8, 64, 40),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _normal_head(wid: int, tid: int, b: int, h: int, n: int, d: int) -> np.ndarray:
    return _rng(wid, tid, b, h).standard_normal((n, d), dtype=np.float32)


def outlier_channel_ids(w: Workload) -> np.ndarray:
    """Distinct K channels scaled for the outlier workload, shared by all heads."""
    if w.outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(w.wid, T_CHAN).choice(w.D, size=w.outlier_channels, replace=False))


def key_lengths(w: Workload) -> Optional[np.ndarray]:
    """Per-sample valid key count, uniform over the integers [N/2, N]."""
    if not w.key_len:
        return None
    return _rng(w.wid, T_LEN).integers(w.N // 2, w.N, size=w.B, endpoint=True).astype(np.int32)


def head_f32(w: Workload, tid: int, b: int, h: int) -> np.ndarray:
    """One (b, h) head of q (tid 0), k (1) or v (2) as float32 before rounding."""
    x = _normal_head(w.wid, tid, b, h, w.N if tid == T_Q else w.n_keys, w.D)
    if tid == T_K:
        if w.outlier_channels:
            x[:, outlier_channel_ids(w)] *= np.float32(w.outlier_scale)
        if w.k_offset_var > 0.0:
            off = _rng(w.wid, T_KOFF, b, h).standard_normal(w.D, dtype=np.float32)
            x += off * np.float32(np.sqrt(w.k_offset_var))
    return x


def head(w: Workload, tid: int, b: int, h: int) -> torch.Tensor:
    """One head rounded to the storage dtype, as a CPU tensor [N, D]."""
    return torch.from_numpy(head_f32(w, tid, b, h)).to(w.torch_dtype)


def make_inputs(w: Workload, threads: int = 8) -> dict:
    """CPU tensors q, k, v [B, H, N, D] in the storage dtype (+ key_len).

    Heads are drawn on a thread pool (numpy's generators release the GIL);
    the per-head streams make the result independent of the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    if w.wid == 1 and (w.B, w.H, w.N, w.D) == (1, 4, 256, 32):
        torch.manual_seed(0)
        q, k, v = (torch.randn(w.B, w.H, w.N, w.D) for _ in range(3))
        return {"q": q, "k": k, "v": v, "key_len": None}
    out = {}
    for name, tid in (("q", T_Q), ("k", T_K), ("v", T_V)):
        x = np.empty((w.B, w.H, w.N if tid == T_Q else w.n_keys, w.D), dtype=np.float32)

        def fill(bh, x=x, tid=tid):
            b, h = divmod(bh, w.H)
            x[b, h] = head_f32(w, tid, b, h)

        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(fill, range(w.B * w.H)))
        out[name] = torch.from_numpy(x).to(w.torch_dtype)
        del x
    kl = key_lengths(w)
    out["key_len"] = None if kl is None else torch.from_numpy(kl)
    return out


def sample_rows(w: Workload, count: int, tile_rows: int = 128) -> np.ndarray:
    """Query rows (b, h, i) to verify at full size: stratified over heads,
    always holding the first and last rows, the first row of the last
    partial tile and the last row of the last full tile."""
    rng = _rng(w.wid, T_ROWS)
    n = w.N
    special = sorted({0, n - 1, (n // tile_rows) * tile_rows if n % tile_rows else n - tile_rows,
                      (n // tile_rows) * tile_rows - 1})
    special = [i for i in special if 0 <= i < n]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rows = []
    for idx in range(count):
        b, h = heads[idx % len(heads)]
        if idx < len(special) * len(heads) and idx // len(heads) < len(special):
            i = special[idx // len(heads)]
        else:
            i = int(rng.integers(0, n))
        rows.append((b, h, i))
    return np.array(sorted(set(rows)), dtype=np.int64)
