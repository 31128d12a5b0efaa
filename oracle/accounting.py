"""FLOP and HBM-byte models of one attention layer.

Test infrastructure only (see the package docstring).

Source: handbook page "算子加速：注意力、编译与融合".
  * Section "注意力：从 O(N²) 显存到分块", the byte model and its printed table:
    the score matrix holds n*n*heads elements; the materialising form writes
    the scores, reads them back for the softmax and writes P (two score
    matrices of traffic) on top of reading Q, K, V and writing O; the tiled
    form moves only Q, K, V and O.
  * Section "访存受限的小算子", the per-op model of a DiT block: attention
    costs 4 n^2 d FLOP (two n x n x d products) and moves four activations
    (Q, K, V in, O out) of n*d elements each.
"""
from __future__ import annotations


def attn_bytes(n: int, d_head: int, heads: int, elt: int = 2):
    """(score-matrix bytes, materialising-form traffic, tiled-form traffic) of one layer."""
    scores = n * n * heads * elt
    act = n * heads * d_head * elt
    naive = 2 * scores + 3 * act + act
    flash = 3 * act + act
    return scores, naive, flash


def attention_flops(B: int, H: int, N: int, D: int, Nk: int | None = None) -> int:
    """4 * N * Nk * D per head: Q K^T and P V, each N*Nk*D multiply-adds."""
    nk = N if Nk is None else Nk
    return 4 * B * H * N * nk * D


def attention_block_row(n: int, d_model: int, elt: int = 2):
    """Attention row of the per-op DiT block model: (flops, bytes)."""
    act = n * d_model * elt
    return 4 * n * n * d_model, 4 * act
