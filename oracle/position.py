"""Oracle: query / KV normalisation and partial rotary positions around the
core attention (test infrastructure only; plain float64 NumPy).

"DeepSeek-V4" book:
* ch. 2 "Normalization and position": RMSNorm rescales a vector by its root
  mean square with a learned scale g and a small epsilon, without
  subtracting the mean; RoPE rotates pairs of coordinates by an angle
  proportional to the position, so that the product of a rotated query and
  a rotated key depends only on their relative position.
* ch. 7 "Query and KV normalization": RMSNorm on every query head and on the
  shared compressed KV head, before the core attention.
* ch. 7 "Partial rotary position embeddings": RoPE on the last 64
  coordinates of queries and KV entries; the other 448 of a 512-dimensional
  vector are not rotated.
* ch. 7 "Why the output is de-rotated": the stored vector is key and value,
  so the attention output's rotary coordinates carry the sources' absolute
  rotations; the output is rotated back by the inverse of the query
  position's rotation.

Readings where the pages leave a step open (each listed in the design
notes): the pairs rotated together are coordinates (2i, 2i+1) of the rotary
part, rotated by the angle pos * inv_freq[i]; the frequency table is an
input (the pages leave frequency scaling to the implementation; the
workloads use 10000^(-2i/64)); epsilon is an input (1e-6 in the
workloads); a query head and a KV vector each have their own scale vector
(one for all query heads, one for the KV head); a compressed entry takes
the position of the first token of its block; window rows (uncompressed KV
vectors) are normalised and rotated like entries, at their own positions.
"""

import numpy as np


def rms_norm(x, g, eps):
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(g, np.float64) * x / np.sqrt(ms + eps)


def rope(x, pos, inv_freq):
    """Rotate the last 2 * len(inv_freq) coordinates of x (pairs (2i, 2i+1))
    by the angles pos * inv_freq[i]; pos broadcasts against x's leading
    axes.  The other coordinates are returned unchanged."""
    x = np.array(x, dtype=np.float64)
    f = np.asarray(inv_freq, np.float64)
    R = 2 * f.size
    ang = np.asarray(pos, np.float64)[..., None] * f  # [..., R/2]
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., -R::2].copy()
    b = x[..., -R + 1::2].copy()
    x[..., -R::2] = a * c - b * s
    x[..., -R + 1::2] = a * s + b * c
    return x


def derotate(o, pos, inv_freq):
    """The inverse rotation of rope at pos (applied to attention outputs)."""
    return rope(o, -np.asarray(pos, np.float64), inv_freq)


def prepare(x, g, eps, pos, inv_freq):
    """A query head or KV vector as the core attention sees it: RMSNorm,
    then RoPE on its rotary part at position pos."""
    return rope(rms_norm(x, g, eps), pos, inv_freq)


def entry_position(i, m):
    """Rotary position of compressed entry i (block of m tokens): its first
    token, m * i."""
    return m * np.asarray(i, np.int64)
