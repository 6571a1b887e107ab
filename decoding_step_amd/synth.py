"""Seeded synthetic inputs for the decode step.

This module holds no arithmetic of the decode step itself: it only draws
vocabulary-head weights and block hidden states from a fixed recipe, so that
the HIP path and the CPU oracle can be fed the very same bits.  The oracle
never imports it; the tests, the smoke check and the benchmark call it and
hand the arrays to both sides.

Recipe (stand-in for the model forward the pages describe: the dInfer
explainer page, the "model component" and "diffusion-iteration manager"
paragraphs, says a pluggable dLLM produces the block's hidden states and the
manager walks fixed-size blocks in turn):

* every random stream is ``PCG64(SeedSequence(seed, spawn_key=key))``;
* ``W`` (V x H): stream ``(0, 0)``, standard normals times 0.02 in float32,
  rounded to bfloat16 (round to nearest, ties to even) unless the workload
  is float32;
* block ``j`` of a sequence with seed ``s``: planted tokens
  ``t = stream(s, 1, j).integers(0, V, L)``, kept across the block;
* iteration ``i`` of block ``j``: stream ``g = (s, 2, j, i)``.  With a
  re-draw probability ``p > 0`` the planted tokens first change in place:
  ``r = g.random(L) < p; t[r] = g.integers(0, V, r.sum())`` (the change
  persists into later iterations of the block).  Then amplitudes
  ``a = g.uniform(0, a_max, L)``, noise ``n = g.standard_normal((L, H))`` and
  ``h = a * W[t] / ||W[t]|| + n`` in float32, rounded like ``W``.

Inputs therefore depend only on (seed, block, iteration), never on what the
step commits, so they can be drawn ahead of time and kept resident.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "stream",
    "bf16_bits",
    "bf16_to_f32",
    "make_weights",
    "BlockStream",
    "hidden_block",
]


def stream(seed: int, *key: int) -> np.random.Generator:
    """Independent PCG64 stream addressed by ``(seed, *key)``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).reshape(-1)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 22
    for i in range(0, u.size, step):          # chunked, in place: keeps temporaries small
        c = u[i:i + step] >> np.uint32(16)
        c &= np.uint32(1)
        c += u[i:i + step]
        c += np.uint32(0x7FFF)
        c >>= np.uint32(16)
        out[i:i + step] = c
    return out.reshape(np.shape(x))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_weights(V: int, H: int, dtype: str = "bf16", seed: int = 0) -> np.ndarray:
    """Vocabulary head ``W[V][H]``: uint16 bf16 bits for ``"bf16"``, float32 for ``"f32"``."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    g = stream(seed, 0)
    out = np.empty((V, H), dtype=np.uint16 if dtype == "bf16" else np.float32)
    rows = max(1, (1 << 23) // max(H, 1))
    for r in range(0, V, rows):      # row chunks draw the same sequence as one (V, H) call
        w = g.standard_normal((min(rows, V - r), H), dtype=np.float32)
        w *= np.float32(0.02)
        out[r:r + w.shape[0]] = bf16_bits(w) if dtype == "bf16" else w
    return out


def _rows_f32(W: np.ndarray, rows: np.ndarray) -> np.ndarray:
    r = W[rows]
    return bf16_to_f32(r) if r.dtype == np.uint16 else r.astype(np.float32)


class BlockStream:
    """Hidden states of one sequence, block by block, iteration by iteration."""

    def __init__(self, W: np.ndarray, L: int, seed: int, a_max: float, redraw_p: float = 0.0):
        self.W = W
        self.V, self.H = W.shape
        self.L = L
        self.seed = seed
        self.a_max = float(a_max)
        self.redraw_p = float(redraw_p)
        self.bf16 = W.dtype == np.uint16
        self._block = None
        self._iter = -1
        self._t = None

    def planted(self, block: int, iteration: int) -> np.ndarray:
        """Planted tokens in force at (block, iteration)."""
        self._advance(block, iteration)
        return self._t.copy()

    def _advance(self, block: int, iteration: int) -> None:
        if self._block != block or iteration < self._iter:
            self._block = block
            self._iter = -1
            self._t = stream(self.seed, 1, block).integers(0, self.V, self.L)
        while self._iter < iteration:
            self._iter += 1
            if self.redraw_p > 0.0:
                g = stream(self.seed, 2, block, self._iter)
                r = g.random(self.L) < self.redraw_p
                self._t[r] = g.integers(0, self.V, int(r.sum()))

    def hidden(self, block: int, iteration: int) -> np.ndarray:
        """``h[L][H]`` for (block, iteration): uint16 bf16 bits or float32, like ``W``."""
        self._advance(block, iteration)
        g = stream(self.seed, 2, block, iteration)
        if self.redraw_p > 0.0:  # replay the re-draw so the stream position matches
            r = g.random(self.L) < self.redraw_p
            g.integers(0, self.V, int(r.sum()))
        a = g.uniform(0.0, self.a_max, self.L).astype(np.float32)
        n = g.standard_normal((self.L, self.H), dtype=np.float32)
        w = _rows_f32(self.W, self._t)
        norm = np.sqrt(np.sum(w.astype(np.float64) ** 2, axis=1)).astype(np.float32)
        norm[norm == 0] = np.float32(1)
        h = (a[:, None] * (w / norm[:, None]) + n).astype(np.float32)
        return bf16_bits(h) if self.bf16 else h


def hidden_block(W: np.ndarray, L: int, seed: int, block: int, iteration: int,
                 a_max: float, redraw_p: float = 0.0) -> np.ndarray:
    """One-shot convenience wrapper around :class:`BlockStream`."""
    return BlockStream(W, L, seed, a_max, redraw_p).hidden(block, iteration)
