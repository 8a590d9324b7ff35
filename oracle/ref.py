"""float64 reference of the looped normalized-GPT forward pass (prefill and
decode, both KV-cache policies). TEST INFRASTRUCTURE ONLY: imported by the
tests, the smoke check and the benchmark's CPU-baseline leg, never by the GPU
library.

What the pages fix (paper "Dory1.0-4B: A Looped Normalized-GPT"):
  * Architecture: normalized-Transformer residual rule; the concatenated gated
    attention output and the SwiGLU activation are L2-normalized before their
    output projections; input-dependent sigmoid gates on the attention output;
    grouped-query attention with 16 query heads and 4 KV groups; 36 MLP-only
    layers interleaved with 27 sliding-window and 9 full-attention layers
    (a 3:1 pattern).
  * Training with Loops: 16-layer input block, 40-layer recurrent block with
    every parameter shared across invocations, 16-layer output block; the
    state starts as a copy of the input block's output x, x is added before
    every invocation, the state is replaced by the block's output, and
    per-token L2 normalization sits at both boundaries; no adapters and no
    outer residual; the final state goes to the output block and the LM head.
    Effective depth 32 + 40k.
  * Long-Context Extension: RoPE base 1e7 for full attention, 1e4 for
    sliding-window attention, window 1024.
  * Last-Loop KV Caching: per-loop caches give every recurrent attention
    layer one cache per loop (a loop-i query reads loop-i entries); last-loop
    caching keeps one cache per recurrent attention layer, overwritten at each
    loop, so that queries read final-loop entries for tokens cached by earlier
    steps and current-loop entries for the tokens of the current step. Input
    and output blocks keep one cache each. At k = 1 the two coincide.

Readings where the pages are silent, garbled or disagree (each applied below):
  R1  The loop equation is missing from the extracted text. Reading:
      s_0 = x; s_i = N(F(N(s_{i-1} + x))) for i = 1..k; s_k feeds the output
      block. F ends in a normalization, so the exit N is idempotent.
  R2  A "layer" is one sublayer (attention-only or MLP-only). Sublayers
      alternate attention, MLP, ... starting with attention; attention
      sublayer j (0-based over the whole stack) is full attention iff
      j mod 4 == 3, else sliding-window.
  R3  Sliding window: a query at position p sees keys u with p - u < W
      (W keys including itself); full attention sees u <= p.
  R4  RoPE: rotate-half over the whole head, inverse frequencies
      base^(-2i/head_dim), absolute 0-based positions.
  R5  Query-key normalization: after RoPE, each head of q and k is L2
      normalized and multiplied by the per-channel vector s_qk (shared by all
      heads and by q and k); logits are scaled by sqrt(head_dim).
  R6  Gate: elementwise sigmoid of h @ W_g^T (no bias), one gate per query
      channel, applied to each head's output before the concatenation norm.
  R7  SwiGLU: a = SiLU(s_v * (h @ W_gate^T)) * (s_u * (h @ W_up^T)); the
      sqrt(d) factor of the normalized Transformer is folded into s_v.
  R8  Residual update after every sublayer: h <- N(h + alpha * (N(y) - h))
      with per-channel effective rates alpha.
  R9  LM head: logits = s_z * (h @ W_lm^T), untied from the embedding; no
      scaling of the embedding rows.
  R10 No epsilon inside N; a zero vector is an error.
  R11 Last-loop write timing: overwriting at every loop equals writing once
      at the last loop while reading the step's own keys from the current
      loop; both forms are implemented and must agree.
  R12 Per-loop caches with a loop count different from earlier steps on the
      same cache have no defined meaning; this is an error.
  R13 Greedy selection: argmax, lowest index on ties.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

KIND_SWA = "swa"
KIND_FULL = "full"
KIND_MLP = "mlp"
MODE_LAST = "last_loop"
MODE_PER = "per_loop"


# ---------------------------------------------------------------------------
# elementary operations
# ---------------------------------------------------------------------------

def l2_normalize(v: np.ndarray) -> np.ndarray:
    """N(v): per-token L2 normalization over the last axis (Architecture,
    normalized-Transformer backbone; Training with Loops, normalization of
    each token vector at the loop boundaries). Reading R10: no epsilon."""
    n = np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    if np.any(n == 0.0):
        raise ValueError("N() of a zero vector")
    return v / n


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-x), evaluated as e^x / (1 + e^x) for negative x so that
    neither form overflows and small results keep their relative accuracy."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(x: np.ndarray) -> np.ndarray:
    return x * sigmoid(x)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis with the row maximum subtracted first;
    -inf entries get probability 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """Reading R4: theta_i = base^(-2i/head_dim), i = 0 .. head_dim/2 - 1."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary embedding, rotate-half layout (reading R4).

    x: [..., T, head_dim]; pos: [T] absolute positions. Channel i and channel
    i + head_dim/2 form one pair rotated by the angle pos * theta_i.
    Bases come from Long-Context Extension (1e4 sliding window, 1e7 full)."""
    dh = x.shape[-1]
    half = dh // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(dh, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def ngpt_update(h: np.ndarray, y: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """Residual rule kept from the normalized Transformer (Architecture;
    reading R8): h <- N(h + alpha * (N(y) - h))."""
    return l2_normalize(h + alpha * (l2_normalize(y) - h))


def swiglu(u: np.ndarray, gt: np.ndarray, s_u: np.ndarray, s_v: np.ndarray) -> np.ndarray:
    """Reading R7: SiLU on the scaled gate branch times the scaled up branch."""
    return silu(s_v * gt) * (s_u * u)


def greedy(logits: np.ndarray) -> np.ndarray:
    """Reading R13: argmax over the last axis; numpy returns the first
    (lowest) index among equal maxima."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def softmax_t(logits: np.ndarray, temperature: float) -> np.ndarray:
    """Sampling distribution softmax(logits / temperature) over the last axis
    (max subtracted first)."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - np.max(z, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def sample_inverse_cdf(probs: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Sampling by inversion: for each row, the smallest index i whose
    cumulative weight exceeds u * (total), u in [0, 1) (so an entry of zero
    weight is never chosen). probs [..., V] (unnormalized weights are fine),
    u [...]."""
    probs = np.asarray(probs, dtype=np.float64)
    c = np.cumsum(probs, axis=-1)
    target = np.asarray(u, dtype=np.float64)[..., None] * c[..., -1:]
    idx = np.sum(c <= target, axis=-1)
    # u * total can exceed the last cumulative sum only by rounding
    return np.minimum(idx, probs.shape[-1] - 1).astype(np.int32)


def speculative_sample(draft_logits: np.ndarray, verify_logits: np.ndarray, drafts: np.ndarray,
                       u: np.ndarray, temperature: float):
    """Rejection rule of self-speculative decoding (Self-Speculative
    Decoding: the drafter proposes gamma tokens, the verifier scores them in
    one pass, and rejection sampling with both models' probabilities accepts
    proposals and corrects the first rejection so that the verifier's
    sampling distribution is preserved). Written from the standard rule:

      q_j = softmax(draft_logits_j / T), p_j = softmax(verify_logits_j / T);
      draft x_j (sampled from q_j) is accepted while u_j < p_j(x_j) / q_j(x_j)
      (always when p_j(x_j) >= q_j(x_j));
      at the first rejection j the next token is drawn from the residual
      max(0, p_j - q_j) (normalized) with the uniform u_gamma; if all gamma
      drafts pass, the next token is drawn from p_{gamma+1} with u_gamma.

    draft_logits [gamma, B, V], verify_logits [gamma + 1, B, V], drafts
    [gamma, B], u [gamma + 1, B] uniforms in [0, 1). Returns (n_accepted [B],
    next [B]): the tokens emitted for sequence b are drafts[:n_b, b] then
    next[b]."""
    draft_logits = np.asarray(draft_logits, dtype=np.float64)
    verify_logits = np.asarray(verify_logits, dtype=np.float64)
    gamma, B, V = draft_logits.shape
    q = softmax_t(draft_logits, temperature)
    p = softmax_t(verify_logits, temperature)
    n = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        j = 0
        while j < gamma:
            x = int(drafts[j, b])
            if not (u[j, b] < p[j, b, x] / q[j, b, x]):
                break
            j += 1
        n[b] = j
        if j < gamma:
            resid = np.maximum(p[j, b] - q[j, b], 0.0)
            nxt[b] = sample_inverse_cdf(resid, u[gamma, b])
        else:
            nxt[b] = sample_inverse_cdf(p[gamma, b], u[gamma, b])
    return n, nxt


def visible(qpos: np.ndarray, kpos: np.ndarray, window: Optional[int]) -> np.ndarray:
    """[T, L] boolean: key position u is visible to the query at position p iff
    u <= p and, for a sliding-window layer, p - u < window (reading R3)."""
    qpos = np.asarray(qpos)[:, None]
    kpos = np.asarray(kpos)[None, :]
    ok = kpos <= qpos
    if window is not None:
        ok &= (qpos - kpos) < window
    return ok


def attention_core(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                   qpos: np.ndarray, kpos: np.ndarray,
                   window: Optional[int], tau: float,
                   q_chunk: int = 512) -> np.ndarray:
    """Masked grouped-query softmax attention.

    q [B, n_q, T, dh]; k, v [B, n_kv, L, dh]; qpos [T], kpos [L] absolute
    positions. Query head j reads KV head j // (n_q / n_kv) (Architecture,
    grouped-query attention). A query at p sees key u iff u <= p and, for a
    sliding-window layer, p - u < window (reading R3). Scores are tau * q.k.
    Returns o [B, n_q, T, dh]."""
    B, nq, T, dh = q.shape
    nkv = k.shape[1]
    if nq % nkv:
        raise ValueError("n_q must be a multiple of n_kv")
    grp = nq // nkv
    qpos = np.asarray(qpos)
    kpos = np.asarray(kpos)
    out = np.empty_like(q)
    for t0 in range(0, T, q_chunk):
        t1 = min(T, t0 + q_chunk)
        qp = qpos[t0:t1]
        lo_pos = -np.inf if window is None else qp.min() - window + 1
        sel = np.nonzero((kpos <= qp.max()) & (kpos >= lo_pos))[0]
        if sel.size == 0:
            raise ValueError("query without keys")
        ks, ke = sel[0], sel[-1] + 1
        allowed = visible(qp, kpos[ks:ke], window)
        for g in range(nkv):
            qq = q[:, g * grp:(g + 1) * grp, t0:t1, :]            # [B, grp, Tc, dh]
            kk = k[:, g, ks:ke, :]                                  # [B, Lc, dh]
            vv = v[:, g, ks:ke, :]
            sc = tau * np.einsum("bjtd,bud->bjtu", qq, kk, optimize=True)
            sc = np.where(allowed[None, None], sc, -np.inf)
            p = softmax_rows(sc)
            out[:, g * grp:(g + 1) * grp, t0:t1, :] = np.einsum(
                "bjtu,bud->bjtd", p, vv, optimize=True)
    return out


# ---------------------------------------------------------------------------
# schedule and cache sizes
# ---------------------------------------------------------------------------

def layer_kinds(shape) -> List[str]:
    """Reading R2 (Architecture: 27 sliding-window + 9 full attention + 36 MLP
    layers in a 3:1 pattern). An explicit `shape.layer_kinds` wins."""
    total = shape.n_input + shape.n_recurrent + shape.n_output
    if getattr(shape, "layer_kinds", None) is not None:
        kinds = list(shape.layer_kinds)
        if len(kinds) != total:
            raise ValueError("layer_kinds length")
        return kinds
    kinds, j = [], 0
    for s in range(total):
        if s % 2 == 0:
            kinds.append(KIND_FULL if j % shape.full_every == shape.full_every - 1 else KIND_SWA)
            j += 1
        else:
            kinds.append(KIND_MLP)
    return kinds


def block_of(shape, s: int) -> str:
    if s < shape.n_input:
        return "input"
    if s < shape.n_input + shape.n_recurrent:
        return "recurrent"
    return "output"


def kv_bytes(shape, mode: str, k: int, batch: int, length: int,
             elem_bytes: int = 2, ring: bool = True, extra: int = 0) -> int:
    """Cache bytes for `length` tokens per sequence (Last-Loop KV Caching):
    each attention sublayer of the recurrent block holds k slots under
    per-loop caching and one under last-loop caching; input and output
    attention sublayers hold one. A slot stores K and V for n_kv heads of
    head_dim; a sliding-window slot stored as a ring holds min(length, W)
    tokens, or min(length, W + extra) when the ring also keeps `extra`
    older tokens (so that a cache can be shortened by that many positions,
    as speculative decoding does when it drops rejected drafts)."""
    per_tok = 2 * shape.n_kv_heads * shape.head_dim * elem_bytes
    total = 0
    for s, kind in enumerate(layer_kinds(shape)):
        if kind == KIND_MLP:
            continue
        slots = k if (mode == MODE_PER and block_of(shape, s) == "recurrent") else 1
        toks = min(length, shape.window + extra) if (kind == KIND_SWA and ring) else length
        total += slots * batch * per_tok * toks
    return total


# ---------------------------------------------------------------------------
# cache
# ---------------------------------------------------------------------------

class Cache:
    """Linear (never ring) K/V storage per (attention sublayer, slot), in
    float64: K[s, slot] has shape [B, n_kv, L, dh]."""

    def __init__(self, shape, mode: str, batch: int):
        if mode not in (MODE_LAST, MODE_PER):
            raise ValueError(mode)
        self.shape = shape
        self.mode = mode
        self.batch = batch
        self.length = 0
        self.k_used: Optional[int] = None
        self.K: Dict[Tuple[int, int], np.ndarray] = {}
        self.V: Dict[Tuple[int, int], np.ndarray] = {}

    def read(self, s: int, slot: int, length: int) -> Tuple[np.ndarray, np.ndarray]:
        sh = self.shape
        if length == 0:
            z = np.zeros((self.batch, sh.n_kv_heads, 0, sh.head_dim))
            return z, z
        key = (s, slot)
        if key not in self.K or self.K[key].shape[2] < length:
            raise ValueError(f"cache slot {key} lacks entries below {length}")
        return self.K[key][:, :, :length], self.V[key][:, :, :length]

    def write(self, s: int, slot: int, p0: int, kk: np.ndarray, vv: np.ndarray) -> None:
        key = (s, slot)
        C = kk.shape[2]
        if key not in self.K:
            if p0 != 0:
                raise ValueError(f"cache slot {key} lacks entries below {p0}")
            self.K[key] = kk.copy()
            self.V[key] = vv.copy()
            return
        L = self.K[key].shape[2]
        if L < p0:
            raise ValueError(f"cache slot {key} lacks entries below {p0}")
        if L < p0 + C:
            pad = p0 + C - L
            z = np.zeros(kk.shape[:2] + (pad, kk.shape[3]))
            self.K[key] = np.concatenate([self.K[key], z], axis=2)
            self.V[key] = np.concatenate([self.V[key], z], axis=2)
        self.K[key][:, :, p0:p0 + C] = kk
        self.V[key][:, :, p0:p0 + C] = vv


# ---------------------------------------------------------------------------
# model
# ---------------------------------------------------------------------------

class OracleModel:
    """The forward step. `weight(name)` returns float64 arrays:

      embed [V, d]; lm_head [V, d]; s_z [V]
      sub{i}.w_qkvg [2*d_q + 2*d_kv, d] (rows q | k | v | gate); sub{i}.w_o [d, d_q];
      sub{i}.s_qk [dh]; sub{i}.alpha [d]
      sub{i}.w_upgate [2F, d] (rows up | gate); sub{i}.w_down [d, F];
      sub{i}.s_u [F]; sub{i}.s_v [F]
    """

    def __init__(self, shape, weight: Callable[[str], np.ndarray]):
        self.shape = shape
        self.weight = weight
        self.kinds = layer_kinds(shape)
        self.tau = math.sqrt(shape.head_dim)          # reading R5

    # -- sublayers ---------------------------------------------------------
    def qkvg(self, s: int, h: np.ndarray, pos: np.ndarray):
        """Projections plus the query-key transform of attention sublayer s.
        h [B, C, d] -> q_hat [B, n_q, C, dh], k_hat, v [B, n_kv, C, dh], g [B, C, d_q]."""
        sh = self.shape
        kind = self.kinds[s]
        base = sh.rope_base_full if kind == KIND_FULL else sh.rope_base_swa
        B, C, _ = h.shape
        dq, dkv, dh = sh.d_q, sh.d_kv, sh.head_dim
        w = self.weight(f"sub{s}.w_qkvg")
        proj = h @ w.T
        q = proj[..., :dq].reshape(B, C, sh.n_q_heads, dh).transpose(0, 2, 1, 3)
        k = proj[..., dq:dq + dkv].reshape(B, C, sh.n_kv_heads, dh).transpose(0, 2, 1, 3)
        v = proj[..., dq + dkv:dq + 2 * dkv].reshape(B, C, sh.n_kv_heads, dh).transpose(0, 2, 1, 3)
        g = proj[..., dq + 2 * dkv:]
        s_qk = self.weight(f"sub{s}.s_qk")
        q_hat = s_qk * l2_normalize(rope(q, pos, base))
        k_hat = s_qk * l2_normalize(rope(k, pos, base))
        return q_hat, k_hat, v, g

    def attention_out(self, s: int, h: np.ndarray, o: np.ndarray, g: np.ndarray) -> np.ndarray:
        """Gate, concatenation norm, output projection and residual update."""
        B, nq, C, dh = o.shape
        cat = o.transpose(0, 2, 1, 3).reshape(B, C, nq * dh)
        z = l2_normalize(cat * sigmoid(g))                      # Architecture
        y = z @ self.weight(f"sub{s}.w_o").T
        return ngpt_update(h, y, self.weight(f"sub{s}.alpha"))

    def attention(self, s: int, h: np.ndarray, p0: int, cache: Cache, slot: int,
                  write: bool, literal: bool) -> np.ndarray:
        sh = self.shape
        C = h.shape[1]
        pos = p0 + np.arange(C)
        q_hat, k_hat, v, g = self.qkvg(s, h, pos)
        if literal:
            # overwrite the cache entries of this step, then read everything
            # from the cache (last-loop rule taken word for word)
            cache.write(s, slot, p0, k_hat, v)
            K, V = cache.read(s, slot, p0 + C)
        else:
            Kp, Vp = cache.read(s, slot, p0)
            K = np.concatenate([Kp, k_hat], axis=2)
            V = np.concatenate([Vp, v], axis=2)
            if write:
                cache.write(s, slot, p0, k_hat, v)
        window = sh.window if self.kinds[s] == KIND_SWA else None
        o = attention_core(q_hat, K, V, pos, np.arange(p0 + C), window, self.tau)
        return self.attention_out(s, h, o, g)

    def mlp(self, s: int, h: np.ndarray) -> np.ndarray:
        F = self.shape.d_ff
        w = self.weight(f"sub{s}.w_upgate")
        u = h @ w[:F].T
        gt = h @ w[F:].T
        a = swiglu(u, gt, self.weight(f"sub{s}.s_u"), self.weight(f"sub{s}.s_v"))
        y = l2_normalize(a) @ self.weight(f"sub{s}.w_down").T   # Architecture
        return ngpt_update(h, y, self.weight(f"sub{s}.alpha"))

    def sublayer(self, s: int, h: np.ndarray, p0: int, cache: Cache, slot: int,
                 write: bool, literal: bool) -> np.ndarray:
        if self.kinds[s] == KIND_MLP:
            return self.mlp(s, h)
        return self.attention(s, h, p0, cache, slot, write, literal)

    # -- one forward step ----------------------------------------------------
    def step(self, cache: Cache, tokens: np.ndarray, k: int, *,
             literal_overwrite: bool = False, logits: Optional[str] = "last",
             trace: Optional[list] = None):
        """Process C new tokens per sequence at positions cache.length ..
        cache.length + C - 1. Returns dict with 'hidden' [B, C, d] (output of
        the last sublayer), 'states' [k x [B, C, d]] (s_1 .. s_k), 'x' (input
        block output) and 'logits' ([B, V] for 'last', [B, C, V] for 'all').
        `trace`, if a list, receives every sublayer output in order."""
        sh = self.shape
        if k < 1:
            raise ValueError("k >= 1")
        if cache.mode == MODE_PER and cache.k_used is not None and cache.k_used != k:
            raise ValueError("per-loop cache used with a different loop count")  # R12
        tokens = np.asarray(tokens)
        B, C = tokens.shape
        if B != cache.batch:
            raise ValueError("batch")
        p0 = cache.length
        nin, nrec = sh.n_input, sh.n_recurrent
        h = self.weight("embed")[tokens]                                      # R9
        for s in range(nin):
            h = self.sublayer(s, h, p0, cache, 0, True, False)
            if trace is not None:
                trace.append(h)
        x = h
        state = x
        states = []
        for i in range(k):                                                    # R1
            u = l2_normalize(state + x)
            for s in range(nin, nin + nrec):
                if cache.mode == MODE_PER:
                    slot, write, lit = i, True, False
                else:
                    slot, write, lit = 0, (i == k - 1), literal_overwrite
                u = self.sublayer(s, u, p0, cache, slot, write, lit)
                if trace is not None:
                    trace.append(u)
            state = l2_normalize(u)
            states.append(state)
        h = state
        for s in range(nin + nrec, sh.n_sublayers):
            h = self.sublayer(s, h, p0, cache, 0, True, False)
            if trace is not None:
                trace.append(h)
        cache.length += C
        if cache.mode == MODE_PER:
            cache.k_used = k
        out = {"hidden": h, "states": states, "x": x}
        if logits is not None and sh.has_lm_head:
            sel = h[:, -1] if logits == "last" else h
            out["logits"] = self.weight("s_z") * (sel @ self.weight("lm_head").T)
        return out
