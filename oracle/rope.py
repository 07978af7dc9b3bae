"""CPU oracle for rotary position embeddings fused with store_kv -- TEST
INFRASTRUCTURE (imported only by the tests; the product library never uses
it and shares no code with it).

The pages list rotary position embeddings (RoPE) among the model layers
("Code Structure", section Model Layers, the get_rope / set_rope_device
entry; section Model Definitions, RotaryConfig among the model configuration
classes) without
stating the formula.  The reading taken is the standard rotary embedding:
channel i < d/2 of a head is paired with channel i + d/2 (the half-split
pairing of the Llama family the pages' model list names), and the pair at
position p is rotated by the angle p * base^(-2i/d):

    y_i       = x_i cos(a) - x_{i+d/2} sin(a)
    y_{i+d/2} = x_{i+d/2} cos(a) + x_i sin(a)

The caller supplies the cos/sin values as a table (one fp32 row of d values
per position: the d/2 cosines, then the d/2 sines); ``rope`` reads that
table, so the oracle and the kernel rotate with the same numbers and differ
only in arithmetic precision (here fp64, rounded once to bf16).
"""

from __future__ import annotations

import numpy as np

from .paged_kv import bf16_bits_to_float, float_to_bf16_bits, store_kv

__all__ = ["rope_table", "rope_f64", "rope", "rope_store_kv", "f64_to_bf16_bits"]


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) in one step.

    Rounding to binary32 first would round twice.  Instead the value is
    first rounded to binary32 *to odd* (truncate toward zero, then set the
    last bit when anything was dropped), which keeps enough information for
    the following round-to-nearest-even to bf16 to equal the direct
    rounding (binary32 carries 16 more significand bits than bf16).
    """
    x = np.asarray(x, dtype=np.float64)
    t = x.astype(np.float32)
    over = np.abs(t.astype(np.float64)) > np.abs(x)
    t = np.where(over, np.nextafter(t, np.float32(0)), t)
    inexact = t.astype(np.float64) != x
    u = t.view(np.uint32) | inexact.astype(np.uint32)
    return float_to_bf16_bits(u.view(np.float32))


def rope_table(max_position: int, head_dim: int, base: float) -> np.ndarray:
    """(max_position, head_dim) float64: cos then sin of p * base^(-2i/d)."""
    assert head_dim % 2 == 0
    half = head_dim // 2
    inv_freq = float(base) ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.outer(np.arange(max_position, dtype=np.float64), inv_freq)
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def rope_f64(x: np.ndarray, positions: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rotate float rows x (T, H, d) at positions (T,) with the table rows."""
    x = np.asarray(x, dtype=np.float64)
    T, H, d = x.shape
    half = d // 2
    rows = np.asarray(table, dtype=np.float64)[np.asarray(positions, dtype=np.int64)]
    cos = rows[:, None, :half]
    sin = rows[:, None, half:]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def rope(x_bits: np.ndarray, positions: np.ndarray, table: np.ndarray) -> np.ndarray:
    """bf16 rows in, bf16 rows out: exact rotation, one rounding to bf16."""
    x = bf16_bits_to_float(x_bits, np.float64)
    return f64_to_bf16_bits(rope_f64(x, positions, table))


def rope_store_kv(pool: np.ndarray, layer: int, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                  out_loc: np.ndarray, positions: np.ndarray, table: np.ndarray):
    """(rotated q, pool after storing rotated k and v at out_loc)."""
    q_rot = rope(q, positions, table)
    k_rot = rope(k, positions, table)
    return q_rot, store_kv(pool, layer, k_rot, v, out_loc)
