"""Additive masks in the memory layouts the attention kernels read
differently, for the GPU parity tests (no test of its own)."""
import numpy as np
import torch


def mask_layouts(dev, B, H, N, seed):
    """Additive masks in the layouts the kernels read differently, as device
    tensors: key-contiguous 16-byte-aligned rows (16-byte loads on whole
    tiles), the same values one float past alignment (one load per key), the
    transpose of a contiguous tensor (key stride N), and masks broadcast
    over queries ([B,1,1,N]) and over keys ([B,H,N,1], a per-row constant)."""
    g = np.random.default_rng(seed)
    full = (g.standard_normal((B, H, N, N)) * 2.0).astype(np.float32)
    full[g.random((B, H, N, N)) < 0.2] = -np.inf
    t = torch.from_numpy(full).to(dev)
    base = torch.zeros(t.numel() + 1, device=dev)
    base[1:] = t.reshape(-1)
    out = {"aligned": t,
           "unaligned": base[1:].view(t.shape),
           "transposed": t.transpose(-1, -2).contiguous().transpose(-1, -2),
           "key_broadcast": torch.from_numpy((g.standard_normal((B, 1, 1, N)) * 2.0).astype(np.float32)).to(dev),
           "query_constant": torch.from_numpy((g.standard_normal((B, H, N, 1)) * 2.0).astype(np.float32)).to(dev)}
    assert out["unaligned"].data_ptr() % 16 != 0 and out["transposed"].stride(-1) == N
    return out

