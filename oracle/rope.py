"""Rotary position embedding and relocation of cached keys (plain fp64).

Test infrastructure (see the package docstring): never imported by the product.

Sources:
  * RedKnot product profile (tokenfly.club), section 3, second building block:
    reusable segments' KV is stored offline and, at serving time, rotary
    position encoding is used to re-align the cached keys to where the segment
    now sits.
  * The is96.com commentary on the RedKnot paper, the two RoPE paragraphs: a
    cached key carries the rotation angle of its offline position; RedKnot
    rotates it backwards by that angle and forwards by the angle of its online
    position, a purely arithmetic step that removes the position error.

Rotary embedding itself is the RoFormer construction (Su et al.), in the
half-split pairing used by the Llama/Qwen model families the pages name:
coordinate i is paired with i + D/2, frequency w_i = theta^(-2i/D), and the pair
is rotated by the angle pos * w_i.  The pages do not fix the pairing; it is one
constant for both sides, so parity does not depend on it.
"""
from __future__ import annotations

import numpy as np


def freqs(head_dim: int, theta: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope(x, pos, theta: float):
    """Rotate each vector of ``x`` [..., D] to position ``pos`` (broadcast over x[..., 0])."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    h = D // 2
    ang = np.asarray(pos, np.float64)[..., None] * freqs(D, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def relocate(x, old_pos, new_pos, theta: float):
    """Move keys cached at ``old_pos`` to ``new_pos``: undo the old rotation
    (rotate to -old_pos), then apply the new one - two rotations, literally."""
    back = rope(x, -np.asarray(old_pos, np.float64), theta)
    return rope(back, new_pos, theta)
