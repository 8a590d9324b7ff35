"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module holds shapes and random draws only: no step of the forward pass is
computed here. Both sides receive exactly the same numbers from it:

* weight matrices are N(0, 1) draws whose rows are scaled to unit L2 length
  (the normalized-Transformer convention that weights live on the unit sphere
  along the embedding dimension) and then rounded to bfloat16 with
  round-to-nearest-even; the GPU receives the bf16 bit patterns and the oracle
  receives the same values widened to float64, so a parity comparison measures
  kernel error only;
* per-channel scale vectors are U(lo, hi) draws rounded to float32;
* token ids are uniform over the vocabulary.

Every tensor has its own generator, seeded from (base seed, tensor name) with
CRC-32, so the draw of one tensor never depends on which others were drawn.
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Optional, Tuple

import numpy as np

KIND_SWA = "swa"
KIND_FULL = "full"
KIND_MLP = "mlp"


@dataclasses.dataclass(frozen=True)
class Shape:
    """Model shape. Sublayer counts count attention-only and MLP-only layers
    separately (the paper's 72 "physical layers" are 36 of each)."""

    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    n_input: int
    n_recurrent: int
    n_output: int
    window: int
    full_every: int = 4
    rope_base_swa: float = 1.0e4
    rope_base_full: float = 1.0e7
    layer_kinds: Optional[Tuple[str, ...]] = None
    has_lm_head: bool = True
    # arithmetic of the GPU build the shape is run with: "bf16", or "fp32"
    # (debug build; the weights are the same bf16-rounded draws, held in fp32)
    precision: str = "bf16"

    @property
    def n_sublayers(self) -> int:
        return self.n_input + self.n_recurrent + self.n_output

    @property
    def d_q(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def d_kv(self) -> int:
        return self.n_kv_heads * self.head_dim


# Tiny model used for oracle pins and exhaustive parity (all k, both cache modes).
TINY = Shape(d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32, d_ff=512,
             vocab=256, n_input=2, n_recurrent=4, n_output=2, window=16)
# The same tiny model with a full-attention layer inside the recurrent block
# (the default 3:1 rule puts none there at this depth).
TINY_REC_FULL = dataclasses.replace(
    TINY, layer_kinds=(KIND_SWA, KIND_MLP,
                       KIND_SWA, KIND_MLP, KIND_FULL, KIND_MLP,
                       KIND_FULL, KIND_MLP))
# The tiny models in the fp32 debug build.
TINY_F32 = dataclasses.replace(TINY, precision="fp32")
TINY_REC_FULL_F32 = dataclasses.replace(TINY_REC_FULL, precision="fp32")
# Mid-size model whose projections take the large-M GEMM path with ragged
# tiles: d=192 (3 K steps of 64), q/k/v/gate width 384, SwiGLU 320.
MID = Shape(d_model=192, n_q_heads=4, n_kv_heads=2, head_dim=32, d_ff=320,
            vocab=300, n_input=2, n_recurrent=4, n_output=2, window=64,
            layer_kinds=(KIND_SWA, KIND_MLP, KIND_SWA, KIND_MLP, KIND_FULL, KIND_MLP,
                         KIND_FULL, KIND_MLP))
# Mid-size model with 128-wide heads: its prefill projections take the fused
# q/k/v/gate GEMM epilogue (one head per 128 output columns).
MID128 = Shape(d_model=256, n_q_heads=2, n_kv_heads=1, head_dim=128, d_ff=512,
               vocab=300, n_input=2, n_recurrent=4, n_output=2, window=64,
               layer_kinds=(KIND_SWA, KIND_MLP, KIND_SWA, KIND_MLP, KIND_FULL, KIND_MLP,
                            KIND_FULL, KIND_MLP))
# Full-size shape: d=2304, 16 query / 4 KV heads of 128, SwiGLU 6144,
# vocab 131072, 16 input + 40 recurrent + 16 output sublayers, window 1024.
FULL = Shape(d_model=2304, n_q_heads=16, n_kv_heads=4, head_dim=128, d_ff=6144,
             vocab=131072, n_input=16, n_recurrent=40, n_output=16, window=1024)
# One recurrent pair at full size: [SWA attention, MLP, full attention, MLP],
# no input/output blocks and no LM head; the loop input is the embedding.
PAIR = dataclasses.replace(
    FULL, n_input=0, n_recurrent=4, n_output=0,
    layer_kinds=(KIND_SWA, KIND_MLP, KIND_FULL, KIND_MLP), has_lm_head=False)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([seed & 0xFFFFFFFF, zlib.crc32(name.encode())])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even);
    returns the 16-bit patterns. Inputs must be finite (no overflow of the
    32-bit sum is then possible)."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = (u >> 16) & 1
    u += 0x7FFF
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unit_rows(seed: int, name: str, rows: int, cols: int) -> np.ndarray:
    """bf16 bit patterns of an N(0,1) [rows, cols] matrix with unit-L2 rows."""
    g = _rng(seed, name)
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, (1 << 22) // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        w = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        w /= np.sqrt(np.einsum("ij,ij->i", w, w, dtype=np.float64)).astype(np.float32)[:, None]
        out[r0:r1] = bf16_bits_from_f32(w)
    return out


def uniform_vec(seed: int, name: str, n: int, lo: float, hi: float,
                mult: float = 1.0) -> np.ndarray:
    g = _rng(seed, name)
    return (mult * g.uniform(lo, hi, size=n)).astype(np.float32)


def tokens(seed: int, batch: int, length: int, vocab: int, name: str = "tokens") -> np.ndarray:
    g = _rng(seed, name)
    return g.integers(0, vocab, size=(batch, length), dtype=np.int64).astype(np.int32)


def kv_context(seed: int, sublayer: int, slot: int, row: int, n_kv: int, n_pos: int,
               dh: int):
    """Synthetic cached keys and values of `n_pos` positions for one
    (sublayer, cache slot, sequence), as bf16 bits [n_kv, n_pos, dh]: keys
    N(0, 1/dh) per entry (rows of about unit length, the scale of normalized
    keys), values N(0, 0.02^2) (the scale of a unit row projected on unit
    rows at d = 2304)."""
    g = np.random.default_rng([seed & 0xFFFFFFFF, sublayer, slot, row, 0x4B56])
    k = g.standard_normal((n_kv, n_pos, dh), dtype=np.float32)
    k *= np.float32(1.0 / np.sqrt(dh))
    v = g.standard_normal((n_kv, n_pos, dh), dtype=np.float32)
    v *= np.float32(0.02)
    return bf16_bits_from_f32(k), bf16_bits_from_f32(v)


def layer_kind_list(shape: Shape):
    """Kinds as data: the explicit tuple if given, else None (each side derives
    the default interleave itself)."""
    return None if shape.layer_kinds is None else list(shape.layer_kinds)


class Weights:
    """Lazily drawn weights of one model. `bits(name)` gives bf16 patterns
    (uint16) for matrices; `vec(name)` gives float32 vectors. Names:

      embed [V, d]; lm_head [V, d]; s_z [V]
      sub{i}.w_qkvg [2*d_q + 2*d_kv, d]   rows: q | k | v | gate
      sub{i}.w_o [d, d_q]; sub{i}.s_qk [head_dim]; sub{i}.alpha [d]
      sub{i}.w_upgate [2*F, d]            rows: up | gate
      sub{i}.w_down [d, F]; sub{i}.s_u [F]; sub{i}.s_v [F]

    `kinds` must be the per-sublayer kind list (attention or MLP) so that
    only the right tensors exist for each sublayer.
    """

    # float64 copies kept per object, up to this many bytes (first come);
    # larger models convert the rest on every access
    F64_CACHE_BYTES = 4 << 30

    def __init__(self, shape: Shape, kinds, seed: int = 0):
        self.shape = shape
        self.kinds = list(kinds)
        self.seed = seed
        self._cache = {}
        self._f64 = {}
        self._f64_bytes = 0

    def names(self):
        s = self.shape
        out = ["embed"]
        if s.has_lm_head:
            out += ["lm_head", "s_z"]
        for i, k in enumerate(self.kinds):
            if k == KIND_MLP:
                out += [f"sub{i}.w_upgate", f"sub{i}.w_down", f"sub{i}.s_u",
                        f"sub{i}.s_v", f"sub{i}.alpha"]
            else:
                out += [f"sub{i}.w_qkvg", f"sub{i}.w_o", f"sub{i}.s_qk", f"sub{i}.alpha"]
        return out

    def _draw(self, name: str):
        s = self.shape
        base = name.split(".")[-1]
        sd = math.sqrt(s.d_model)
        if base == "embed":
            return unit_rows(self.seed, name, s.vocab, s.d_model)
        if base == "lm_head":
            return unit_rows(self.seed, name, s.vocab, s.d_model)
        if base == "s_z":
            return uniform_vec(self.seed, name, s.vocab, 0.5, 1.5, sd)
        if base == "w_qkvg":
            return unit_rows(self.seed, name, 2 * s.d_q + 2 * s.d_kv, s.d_model)
        if base == "w_o":
            return unit_rows(self.seed, name, s.d_model, s.d_q)
        if base == "s_qk":
            return uniform_vec(self.seed, name, s.head_dim, 0.5, 1.5)
        if base == "alpha":
            return uniform_vec(self.seed, name, s.d_model, 0.5, 1.5, 0.05)
        if base == "w_upgate":
            return unit_rows(self.seed, name, 2 * s.d_ff, s.d_model)
        if base == "w_down":
            return unit_rows(self.seed, name, s.d_model, s.d_ff)
        if base == "s_u":
            return uniform_vec(self.seed, name, s.d_ff, 0.5, 1.5)
        if base == "s_v":
            return uniform_vec(self.seed, name, s.d_ff, 0.5, 1.5, sd)
        raise KeyError(name)

    def raw(self, name: str) -> np.ndarray:
        """bf16 bits (uint16) for matrices, float32 for vectors."""
        if name not in self._cache:
            self._cache[name] = self._draw(name)
        return self._cache[name]

    def f64(self, name: str) -> np.ndarray:
        """float64 values of a tensor (read-only when kept in the cache)."""
        if name in self._f64:
            return self._f64[name]
        r = self.raw(name)
        out = f64_from_bf16_bits(r) if r.dtype == np.uint16 else r.astype(np.float64)
        if self._f64_bytes + out.nbytes <= self.F64_CACHE_BYTES:
            out.flags.writeable = False
            self._f64[name] = out
            self._f64_bytes += out.nbytes
        return out

    def _forget_f64(self, name: str) -> None:
        old = self._f64.pop(name, None)
        if old is not None:
            self._f64_bytes -= old.nbytes

    def set_raw(self, name: str, value: np.ndarray) -> None:
        """Override one tensor (bf16 bits for matrices, float32 for vectors),
        used to build special cases such as zero gates."""
        self._forget_f64(name)
        self._cache[name] = value

    def drop(self, name: str) -> None:
        self._forget_f64(name)
        self._cache.pop(name, None)
