"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test grounds the oracle in something other than itself: numbers the pages
print (golden fixtures under tests/golden, each with its citation), closed
forms, invariants, brute force over tiny inputs, and library routines that
compute the same textbook operation by another route.
"""
import dataclasses
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def tiny_model(shape=synth.TINY, seed=0, overrides=None):
    kinds = ref.layer_kinds(shape)
    w = synth.Weights(shape, kinds, seed)
    for name, val in (overrides or {}).items():
        w.set_raw(name, val)
    return ref.OracleModel(shape, w.f64), w


# Shape with the full model's layer counts and tiny widths, so that the loop
# structure of the real model runs in milliseconds.
COUNTS = synth.Shape(d_model=32, n_q_heads=2, n_kv_heads=1, head_dim=16, d_ff=64,
                     vocab=32, n_input=16, n_recurrent=40, n_output=16, window=4)


# ---------------------------------------------------------------- structure

def test_schedule_counts_match_pages():
    g = {k: int(v) for k, v in read_golden("schedule_counts.txt")}
    kinds = ref.layer_kinds(synth.FULL)
    assert len(kinds) == g["total"]
    assert kinds.count(ref.KIND_SWA) == g["swa"]
    assert kinds.count(ref.KIND_FULL) == g["full"]
    assert kinds.count(ref.KIND_MLP) == g["mlp"]
    assert (synth.FULL.n_input, synth.FULL.n_recurrent, synth.FULL.n_output) == \
        (g["input"], g["recurrent"], g["output"])
    # 3:1 pattern: every run of four consecutive attention layers has one full
    att = [k for k in kinds if k != ref.KIND_MLP]
    for i in range(0, len(att), 4):
        assert att[i:i + 4].count(ref.KIND_FULL) == 1


def test_heads_and_rope_constants_match_pages():
    h = {k: int(v) for k, v in read_golden("heads.txt")}
    assert (synth.FULL.n_q_heads, synth.FULL.n_kv_heads) == (h["n_q_heads"], h["n_kv_heads"])
    r = {k: float(v) for k, v in read_golden("rope_window.txt")}
    assert synth.FULL.rope_base_full == r["rope_base_full"]
    assert synth.FULL.rope_base_swa == r["rope_base_swa"]
    assert synth.FULL.window == r["window"]


@pytest.mark.parametrize("k", [1, 2, 4])
def test_effective_depth_counts_sublayer_applications(k):
    depth = {int(a): int(b) for a, b in read_golden("effective_depth.txt")}
    m, _ = tiny_model(COUNTS)
    trace = []
    toks = synth.tokens(1, 1, 3, COUNTS.vocab)
    m.step(ref.Cache(COUNTS, ref.MODE_LAST, 1), toks, k, trace=trace)
    assert len(trace) == depth[k]


# ---------------------------------------------------------------- P1 unit norm

@pytest.mark.parametrize("mode", [ref.MODE_LAST, ref.MODE_PER])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_unit_norm_after_every_sublayer_and_boundary(mode, k):
    m, _ = tiny_model(synth.TINY_REC_FULL)
    toks = synth.tokens(0, 2, 24, synth.TINY.vocab)
    cache = ref.Cache(synth.TINY_REC_FULL, mode, 2)
    trace = []
    out = m.step(cache, toks, k, trace=trace)
    out2 = m.step(cache, toks[:, :1], k, trace=trace)
    for t in trace + out["states"] + out2["states"]:
        assert np.max(np.abs(np.linalg.norm(t, axis=-1) - 1.0)) < 1e-12


# ---------------------------------------------------------------- P2 k=1

def test_k1_equals_plain_non_looped_stack():
    sh = synth.TINY_REC_FULL
    m, w = tiny_model(sh)
    flat = dataclasses.replace(sh, n_input=sh.n_sublayers, n_recurrent=0, n_output=0)
    mf = ref.OracleModel(flat, w.f64)
    toks = synth.tokens(3, 2, 40, sh.vocab)
    a = m.step(ref.Cache(sh, ref.MODE_LAST, 2), toks, 1, logits="all")
    b = mf.step(ref.Cache(flat, ref.MODE_LAST, 2), toks, 1, logits="all")
    np.testing.assert_allclose(a["hidden"], b["hidden"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(a["logits"], b["logits"], atol=1e-10, rtol=0)


# ---------------------------------------------------------------- P3 unrolled

def _unrolled(sh, w, k):
    kinds = ref.layer_kinds(sh)
    nin, nrec = sh.n_input, sh.n_recurrent
    order = list(range(nin)) + [nin + j for _ in range(k) for j in range(nrec)] + \
        list(range(nin + nrec, sh.n_sublayers))
    ush = dataclasses.replace(sh, n_input=len(order), n_recurrent=0, n_output=0,
                              layer_kinds=tuple(kinds[o] for o in order))

    def weight(name):
        if name.startswith("sub"):
            i, rest = name[3:].split(".", 1)
            return w.f64(f"sub{order[int(i)]}.{rest}")
        return w.f64(name)
    return ref.OracleModel(ush, weight), ush


def _unrolled_step(um, ush, sh, cache, toks, k):
    """Independent driver over an unrolled stack of k weight copies, each with
    its own cache, with the loop-boundary transforms written out."""
    nin, nrec = sh.n_input, sh.n_recurrent
    p0 = cache.length
    h = um.weight("embed")[toks]
    idx = 0
    for _ in range(nin):
        h = um.sublayer(idx, h, p0, cache, 0, True, False)
        idx += 1
    x = h
    s = x.copy()
    for _ in range(k):
        u = (s + x) / np.linalg.norm(s + x, axis=-1, keepdims=True)
        for _ in range(nrec):
            u = um.sublayer(idx, u, p0, cache, 0, True, False)
            idx += 1
        s = u / np.linalg.norm(u, axis=-1, keepdims=True)
    h = s
    while idx < ush.n_sublayers:
        h = um.sublayer(idx, h, p0, cache, 0, True, False)
        idx += 1
    cache.length += toks.shape[1]
    return h


@pytest.mark.parametrize("k", [2, 3])
def test_loops_equal_unrolled_weight_copies_per_loop(k):
    sh = synth.TINY_REC_FULL
    m, w = tiny_model(sh)
    um, ush = _unrolled(sh, w, k)
    toks = synth.tokens(5, 2, 40, sh.vocab)
    ca = ref.Cache(sh, ref.MODE_PER, 2)
    cb = ref.Cache(ush, ref.MODE_LAST, 2)
    # prefill 20, chunk 12, then 8 single-token decode steps
    for a, b in [(0, 20), (20, 32)] + [(t, t + 1) for t in range(32, 40)]:
        ha = m.step(ca, toks[:, a:b], k)["hidden"]
        hb = _unrolled_step(um, ush, sh, cb, toks[:, a:b], k)
        np.testing.assert_allclose(ha, hb, atol=1e-12, rtol=0)


def test_loops_equal_unrolled_one_shot_last_loop():
    sh = synth.TINY_REC_FULL
    k = 4
    m, w = tiny_model(sh)
    um, ush = _unrolled(sh, w, k)
    toks = synth.tokens(6, 2, 48, sh.vocab)
    ha = m.step(ref.Cache(sh, ref.MODE_LAST, 2), toks, k)["hidden"]
    hb = _unrolled_step(um, ush, sh, ref.Cache(ush, ref.MODE_LAST, 2), toks, k)
    np.testing.assert_allclose(ha, hb, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- P4/P5 attention

def _brute_attention(q, k, v, qpos, kpos, band, tau):
    """Pure-Python loops: explicit band mask, textbook softmax."""
    B, nq, T, dh = q.shape
    nkv = k.shape[1]
    grp = nq // nkv
    o = np.zeros_like(q)
    for b in range(B):
        for j in range(nq):
            g = j // grp
            for t in range(T):
                sc = []
                for u in range(len(kpos)):
                    ok = kpos[u] <= qpos[t]
                    if band is not None:
                        ok = ok and (qpos[t] - kpos[u]) <= band - 1
                    if ok:
                        sc.append((u, tau * sum(q[b, j, t, d] * k[b, g, u, d] for d in range(dh))))
                mx = max(s for _, s in sc)
                den = sum(math.exp(s - mx) for _, s in sc)
                for u, s in sc:
                    o[b, j, t] += math.exp(s - mx) / den * v[b, g, u]
    return o


def _rand_qkv(seed, B=1, nq=4, nkv=2, T=9, L=None, dh=4):
    g = np.random.default_rng(seed)
    L = T if L is None else L
    return (g.standard_normal((B, nq, T, dh)), g.standard_normal((B, nkv, L, dh)),
            g.standard_normal((B, nkv, L, dh)))


@pytest.mark.parametrize("window", [1, 3, 5])
def test_sliding_window_equals_brute_force_band_mask(window):
    q, k, v = _rand_qkv(11, B=2, T=7, L=11)
    qpos = np.arange(4, 11)
    kpos = np.arange(11)
    a = ref.attention_core(q, k, v, qpos, kpos, window, 1.3)
    b = _brute_attention(q, k, v, qpos, kpos, window, 1.3)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_full_attention_equals_brute_force_causal():
    q, k, v = _rand_qkv(12, B=2, T=6, L=10)
    qpos = np.arange(4, 10)
    a = ref.attention_core(q, k, v, qpos, np.arange(10), None, 0.7, q_chunk=4)
    b = _brute_attention(q, k, v, qpos, np.arange(10), None, 0.7)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_window_at_least_sequence_equals_full():
    q, k, v = _rand_qkv(13, T=12)
    p = np.arange(12)
    np.testing.assert_allclose(ref.attention_core(q, k, v, p, p, 12, 2.0),
                               ref.attention_core(q, k, v, p, p, None, 2.0), atol=1e-14)


def test_attention_matches_torch_sdpa_with_gqa_repeat():
    q, k, v = _rand_qkv(14, B=2, nq=8, nkv=2, T=10, dh=8)
    p = np.arange(10)
    tau = 1.7
    for window in (None, 4):
        a = ref.attention_core(q, k, v, p, p, window, tau)
        mask = p[None, :] <= p[:, None]
        if window is not None:
            mask &= (p[:, None] - p[None, :]) < window
        kt = torch.from_numpy(k).repeat_interleave(4, dim=1)
        vt = torch.from_numpy(v).repeat_interleave(4, dim=1)
        b = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), kt, vt, attn_mask=torch.from_numpy(mask), scale=tau)
        np.testing.assert_allclose(a, b.numpy(), atol=1e-12, rtol=0)


def test_first_position_attends_only_to_itself():
    q, k, v = _rand_qkv(15, T=5)
    p = np.arange(5)
    o = ref.attention_core(q, k, v, p, p, None, 3.0)
    np.testing.assert_array_equal(o[:, 0::2, 0], v[:, :, 0])
    np.testing.assert_array_equal(o[:, 1::2, 0], v[:, :, 0])


# ---------------------------------------------------------------- P6 RoPE

def test_rope_matches_complex_rotation_and_pages_bases():
    g = np.random.default_rng(21)
    dh = 16
    x = g.standard_normal((3, 5, dh))
    pos = np.array([0, 1, 7, 1000, 262143])
    for base in (1.0e4, 1.0e7):
        y = ref.rope(x, pos, base)
        z = x[..., :dh // 2] + 1j * x[..., dh // 2:]
        theta = np.array([base ** (-(2.0 * i) / dh) for i in range(dh // 2)])
        zr = z * np.exp(1j * np.outer(pos, theta))
        np.testing.assert_allclose(y[..., :dh // 2], zr.real, atol=1e-12)
        np.testing.assert_allclose(y[..., dh // 2:], zr.imag, atol=1e-12)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
        np.testing.assert_array_equal(y[:, 0], x[:, 0])       # position 0: identity


def test_attention_scores_invariant_to_position_shift():
    g = np.random.default_rng(22)
    q = g.standard_normal((6, 32))
    k = g.standard_normal((6, 32))
    p = np.arange(6)
    s0 = ref.rope(q, p, 1e4) @ ref.rope(k, p, 1e4).T
    s1 = ref.rope(q, p + 777, 1e4) @ ref.rope(k, p + 777, 1e4).T
    np.testing.assert_allclose(s0, s1, atol=1e-10)


def test_attention_sublayer_invariant_to_position_shift():
    """RoPE makes attention depend on relative positions only: the same tokens
    evaluated at positions 0..7 and 50..57 (no cached prefix) give the same
    attention output when s_qk is uniform across channels."""
    sh = synth.TINY
    # per-channel s_qk applied after the rotation weighs paired channels
    # differently, which breaks the invariance; a uniform s_qk keeps it
    m, _ = tiny_model(sh, overrides={"sub0.s_qk": np.full(sh.head_dim, 1.3, np.float32)})
    h = m.weight("embed")[synth.tokens(23, 1, 8, sh.vocab)]
    p = np.arange(8)
    q0, k0, v0, _ = m.qkvg(0, h, p)
    q1, k1, v1, _ = m.qkvg(0, h, p + 50)
    o0 = ref.attention_core(q0, k0, v0, p, p, 8, m.tau)
    o1 = ref.attention_core(q1, k1, v1, p + 50, p + 50, 8, m.tau)
    np.testing.assert_allclose(o0, o1, atol=1e-12)
    assert np.max(np.abs(q0 - q1)) > 1e-3


# ---------------------------------------------------------------- R5 query-key transform

def _head_norms(x):
    return np.linalg.norm(x, axis=-1)


def test_qkvg_uniform_scale_gives_per_head_norm_c():
    """Reading R5 (section Architecture, query-key scale): with s_qk = c on
    every channel, each head of q_hat and of k_hat has length c at every
    token. A normalization over all heads jointly (or none) fails this."""
    sh = synth.TINY
    c = float(np.float32(1.3))         # the vector is stored in float32
    m, _ = tiny_model(sh, overrides={"sub0.s_qk": np.full(sh.head_dim, c, np.float32)})
    h = m.weight("embed")[synth.tokens(41, 2, 9, sh.vocab)]
    pos = np.arange(9) + 5
    q, k, v, g = m.qkvg(0, h, pos)
    assert q.shape == (2, sh.n_q_heads, 9, sh.head_dim)
    assert k.shape == (2, sh.n_kv_heads, 9, sh.head_dim)
    np.testing.assert_allclose(_head_norms(q), c, rtol=1e-13)
    np.testing.assert_allclose(_head_norms(k), c, rtol=1e-13)
    # the pin is sensitive: a joint normalization of all heads (head norms
    # c * |q_j| / |q|) departs from c by far more than rounding
    raw = h @ m.weight("sub0.w_qkvg").T
    qr = raw[..., :sh.d_q]
    joint = c * qr / np.linalg.norm(qr, axis=-1, keepdims=True)
    jn = np.linalg.norm(joint.reshape(2, 9, sh.n_q_heads, sh.head_dim), axis=-1)
    assert np.max(np.abs(jn - c)) > 0.1


def test_qkvg_scale_applied_after_rotation_and_norm():
    """With a per-channel s_qk, q_hat / s_qk and k_hat / s_qk are unit vectors
    per head: the scale multiplies the rotated, normalized head. Applying it
    before the norm, or before the rotation (which mixes channel i with
    channel i + dh/2), would leave these lengths away from 1."""
    sh = synth.TINY
    m, w = tiny_model(sh)
    s_qk = m.weight("sub0.s_qk")
    assert np.ptp(s_qk) > 0.3                     # a genuinely non-uniform scale
    h = m.weight("embed")[synth.tokens(42, 1, 7, sh.vocab)]
    pos = np.array([0, 1, 2, 50, 300, 1023, 4000])
    q, k, _, _ = m.qkvg(0, h, pos)
    np.testing.assert_allclose(_head_norms(q / s_qk), 1.0, rtol=1e-13)
    np.testing.assert_allclose(_head_norms(k / s_qk), 1.0, rtol=1e-13)
    # scale before the norm: N(s * rope(q)) / s is not unit length
    raw = (h @ m.weight("sub0.w_qkvg").T)[..., :sh.d_q]
    qr = raw.reshape(1, 7, sh.n_q_heads, sh.head_dim).transpose(0, 2, 1, 3)
    alt = ref.l2_normalize(s_qk * ref.rope(qr, pos, sh.rope_base_swa))
    assert np.max(np.abs(_head_norms(alt / s_qk) - 1.0)) > 1e-2
    # scale before the rotation: rope(s * N(q)) / s is not unit length
    alt2 = ref.rope(s_qk * ref.l2_normalize(qr), pos, sh.rope_base_swa)
    assert np.max(np.abs(_head_norms(alt2 / s_qk) - 1.0)) > 1e-2


def test_qkvg_hand_built_weights_closed_form():
    """Hand-built projection rows: with h = e_0 the projections are column 0
    of w_qkvg. Each q and k head gets one nonzero channel pair (i, i + dh/2)
    holding (a, b), so after the rotate-half RoPE (reading R4) the head is the
    2-D rotation of (a, b) by p * base^(-2i/dh) in that pair, and after the
    per-head norm and s_qk (reading R5) q_hat = s_qk * rotated / |(a, b)|.
    v and g are column 0 of their row blocks unchanged. Distinct pairs and
    values per head pin the row order q | k | v | gate, the head order, the
    pair layout and the RoPE base of the sublayer's kind."""
    sh = synth.TINY_REC_FULL        # sublayer 0 sliding-window, sublayer 4 full attention
    d, dh, nq, nkv = sh.d_model, sh.head_dim, sh.n_q_heads, sh.n_kv_heads
    half = dh // 2
    nrows = 2 * sh.d_q + 2 * sh.d_kv
    g_ = np.random.default_rng(43)
    col = np.zeros(nrows)
    pairs = {}
    for j in range(nq + nkv):
        i = (3 * j + 1) % half
        a, b = g_.uniform(0.5, 2.0), g_.uniform(-2.0, 2.0)
        r0 = j * dh                      # q heads first, then k heads (rows d_q ..)
        col[r0 + i], col[r0 + i + half] = a, b
        pairs[j] = (i, a, b)
    vg = g_.standard_normal(sh.d_kv + sh.d_q)
    col[sh.d_q + sh.d_kv:] = vg
    wmat = np.zeros((nrows, d))
    wmat[:, 0] = col
    s_qk = g_.uniform(0.5, 1.5, dh)
    for sub, base in ((0, sh.rope_base_swa), (4, sh.rope_base_full)):
        m = ref.OracleModel(sh, lambda n, sub=sub: {f"sub{sub}.w_qkvg": wmat,
                                                     f"sub{sub}.s_qk": s_qk}[n])
        h = np.zeros((1, 3, d))
        h[..., 0] = 1.0
        pos = np.array([0, 3, 777])
        q, k, v, gt = m.qkvg(sub, h, pos)
        for j in range(nq + nkv):
            i, a, b = pairs[j]
            out = q[0, j] if j < nq else k[0, j - nq]
            for t, p in enumerate(pos):
                ang = p * base ** (-2.0 * i / dh)
                want = np.zeros(dh)
                want[i] = a * math.cos(ang) - b * math.sin(ang)
                want[i + half] = b * math.cos(ang) + a * math.sin(ang)
                want *= s_qk / math.hypot(a, b)
                np.testing.assert_allclose(out[t], want, atol=1e-14)
        for t in range(3):
            np.testing.assert_array_equal(v[0, :, t].reshape(-1), vg[:sh.d_kv])
            np.testing.assert_array_equal(gt[0, t], vg[sh.d_kv:])


# ---------------------------------------------------------------- P7 scale cancellation

def test_output_projection_scale_cancels():
    sh = synth.TINY
    m, w = tiny_model(sh)
    h = m.weight("embed")[synth.tokens(31, 1, 10, sh.vocab)]
    base = m.sublayer(0, h, 0, ref.Cache(sh, ref.MODE_LAST, 1), 0, True, False)
    base_mlp = m.mlp(1, h)
    wo = w.f64("sub0.w_o")
    wd = w.f64("sub1.w_down")

    def scaled(name):
        if name == "sub0.w_o":
            return 3.5 * wo
        if name == "sub1.w_down":
            return 0.25 * wd
        return w.f64(name)
    ms = ref.OracleModel(sh, scaled)
    np.testing.assert_allclose(ms.sublayer(0, h, 0, ref.Cache(sh, ref.MODE_LAST, 1), 0, True, False),
                               base, atol=1e-14)
    np.testing.assert_allclose(ms.mlp(1, h), base_mlp, atol=1e-14)
    assert np.linalg.norm(ref.l2_normalize(3.0 * h) - ref.l2_normalize(h)) < 1e-14


def test_zero_gate_weights_equal_constant_gate_and_gate_matters():
    sh = synth.TINY
    m, w = tiny_model(sh)
    h = m.weight("embed")[synth.tokens(32, 1, 10, sh.vocab)]
    dq, dkv = sh.d_q, sh.d_kv
    wq = w.f64("sub0.w_qkvg").copy()
    wq0 = wq.copy()
    wq0[dq + 2 * dkv:] = 0.0
    m0 = ref.OracleModel(sh, lambda n: wq0 if n == "sub0.w_qkvg" else w.f64(n))
    out0 = m0.sublayer(0, h, 0, ref.Cache(sh, ref.MODE_LAST, 1), 0, True, False)
    # with zero gate weights every gate is 1/2, which the concatenation norm
    # removes: equal to the ungated attention output pushed through W_o
    pos = np.arange(10)
    q_hat, k_hat, v, _ = m0.qkvg(0, h, pos)
    o = ref.attention_core(q_hat, k_hat, v, pos, pos, sh.window, m0.tau)
    cat = o.transpose(0, 2, 1, 3).reshape(1, 10, dq)
    y = cat @ w.f64("sub0.w_o").T
    np.testing.assert_allclose(out0, ref.ngpt_update(h, y, w.f64("sub0.alpha")), atol=1e-13)
    out = m.sublayer(0, h, 0, ref.Cache(sh, ref.MODE_LAST, 1), 0, True, False)
    assert np.max(np.abs(out - out0)) > 1e-6


# ---------------------------------------------------------------- P8 update rule

def test_update_special_cases():
    g = np.random.default_rng(41)
    h = ref.l2_normalize(g.standard_normal((4, 7, 16)))
    y = g.standard_normal((4, 7, 16))
    np.testing.assert_allclose(ref.ngpt_update(h, y, np.zeros(16)), h, atol=1e-15)
    np.testing.assert_allclose(ref.ngpt_update(h, y, np.ones(16)), ref.l2_normalize(y), atol=1e-15)
    np.testing.assert_allclose(ref.ngpt_update(h, 5.0 * h, g.uniform(0, 1, 16)), h, atol=1e-15)
    # scalar alpha: the result lies on the great circle between h and N(y)
    a = 0.3
    r = ref.ngpt_update(h, y, np.full(16, a))
    lin = (1 - a) * h + a * ref.l2_normalize(y)
    np.testing.assert_allclose(r, lin / np.linalg.norm(lin, axis=-1, keepdims=True), atol=1e-15)


def test_swiglu_and_sigmoid_match_library():
    g = np.random.default_rng(42)
    x = g.standard_normal(1000) * 20
    np.testing.assert_allclose(ref.sigmoid(x), scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    u, v = g.standard_normal(50), g.standard_normal(50) * 8
    su, sv = g.uniform(0.5, 1.5, 50), g.uniform(0.5, 1.5, 50)
    t = torch.nn.functional.silu(torch.from_numpy(sv * v)) * torch.from_numpy(su * u)
    np.testing.assert_allclose(ref.swiglu(u, v, su, sv), t.numpy(), rtol=1e-13, atol=1e-15)
    sm = ref.softmax_rows(x.reshape(10, 100))
    np.testing.assert_allclose(sm, scipy.special.softmax(x.reshape(10, 100), axis=-1), rtol=1e-12)


# ---------------------------------------------------------------- P9 cache modes

def _run(m, sh, mode, toks, k, splits, literal=False):
    c = ref.Cache(sh, mode, toks.shape[0])
    hs, lg = [], []
    for a, b in splits:
        o = m.step(c, toks[:, a:b], k, literal_overwrite=literal)
        hs.append(o["hidden"])
        lg.append(o["logits"])
    return np.concatenate(hs, axis=1), lg, c


SPLIT_PD = [(0, 32)] + [(t, t + 1) for t in range(32, 40)]


def test_modes_identical_at_k1():
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(51, 2, 40, sh.vocab)
    a, _, _ = _run(m, sh, ref.MODE_LAST, toks, 1, SPLIT_PD)
    b, _, _ = _run(m, sh, ref.MODE_PER, toks, 1, SPLIT_PD)
    np.testing.assert_array_equal(a, b)


def test_one_shot_prefill_identical_in_both_modes():
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(52, 2, 48, sh.vocab)
    a, _, _ = _run(m, sh, ref.MODE_LAST, toks, 4, [(0, 48)])
    b, _, _ = _run(m, sh, ref.MODE_PER, toks, 4, [(0, 48)])
    np.testing.assert_allclose(a, b, atol=1e-13)


@pytest.mark.parametrize("k", [2, 4])
def test_decode_differs_between_modes_when_looping(k):
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(53, 2, 40, sh.vocab)
    a, _, _ = _run(m, sh, ref.MODE_LAST, toks, k, SPLIT_PD)
    b, _, _ = _run(m, sh, ref.MODE_PER, toks, k, SPLIT_PD)
    np.testing.assert_allclose(a[:, :32], b[:, :32], atol=1e-13)
    assert np.max(np.abs(a[:, 32:] - b[:, 32:])) > 1e-4


def test_per_loop_chunked_and_decode_equal_one_shot():
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(54, 2, 64, sh.vocab)
    one, _, _ = _run(m, sh, ref.MODE_PER, toks, 3, [(0, 64)])
    chunked, _, _ = _run(m, sh, ref.MODE_PER, toks, 3, [(0, 16), (16, 32), (32, 48), (48, 64)])
    dec, _, _ = _run(m, sh, ref.MODE_PER, toks, 3, [(0, 50)] + [(t, t + 1) for t in range(50, 64)])
    np.testing.assert_allclose(chunked, one, atol=1e-13)
    np.testing.assert_allclose(dec, one, atol=1e-13)


def test_last_loop_chunked_differs_from_one_shot_when_looping():
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(55, 2, 64, sh.vocab)
    one, _, _ = _run(m, sh, ref.MODE_LAST, toks, 3, [(0, 64)])
    chunked, _, _ = _run(m, sh, ref.MODE_LAST, toks, 3, [(0, 32), (32, 64)])
    np.testing.assert_allclose(chunked[:, :32], one[:, :32], atol=1e-13)
    assert np.max(np.abs(chunked[:, 32:] - one[:, 32:])) > 1e-4


@pytest.mark.parametrize("k", [1, 3])
def test_literal_overwrite_equals_last_loop_write(k):
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(56, 2, 44, sh.vocab)
    sp = [(0, 20), (20, 36)] + [(t, t + 1) for t in range(36, 44)]
    a, la, ca = _run(m, sh, ref.MODE_LAST, toks, k, sp, literal=False)
    b, lb, cb = _run(m, sh, ref.MODE_LAST, toks, k, sp, literal=True)
    np.testing.assert_allclose(a, b, atol=1e-13)
    for key in ca.K:
        np.testing.assert_allclose(ca.K[key], cb.K[key], atol=1e-13)


def test_per_loop_rejects_changed_loop_count():
    sh = synth.TINY
    m, _ = tiny_model(sh)
    c = ref.Cache(sh, ref.MODE_PER, 1)
    toks = synth.tokens(57, 1, 8, sh.vocab)
    m.step(c, toks[:, :4], 2)
    with pytest.raises(ValueError):
        m.step(c, toks[:, 4:5], 3)


# ---------------------------------------------------------------- P10 KV bytes

def test_kv_bytes_closed_form_matches_worked_values():
    for mode, k, val in read_golden("kv_bytes_tiny.txt"):
        assert ref.kv_bytes(synth.TINY, mode, int(k), 2, 64) == int(val)


@pytest.mark.parametrize("mode", [ref.MODE_LAST, ref.MODE_PER])
def test_kv_bytes_equals_what_the_cache_holds(mode):
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(58, 2, 40, sh.vocab)
    for k in (1, 2, 4):
        _, _, c = _run(m, sh, mode, toks, k, [(0, 30), (30, 40)])
        held = 0
        kinds = ref.layer_kinds(sh)
        for (s, _slot), arr in c.K.items():
            L = arr.shape[2]
            toks_kept = min(L, sh.window) if kinds[s] == ref.KIND_SWA else L
            held += 2 * arr.shape[0] * arr.shape[1] * toks_kept * arr.shape[3] * 2
        assert held == ref.kv_bytes(sh, mode, k, 2, 40)


def test_kv_bytes_constant_in_k_for_last_loop_linear_for_per_loop():
    sh = synth.FULL
    last = [ref.kv_bytes(sh, ref.MODE_LAST, k, 64, 33024) for k in (1, 2, 3, 4)]
    per = [ref.kv_bytes(sh, ref.MODE_PER, k, 64, 33024) for k in (1, 2, 3, 4)]
    assert len(set(last)) == 1
    steps = np.diff(per)
    assert per[0] == last[0] and np.all(steps == steps[0]) and steps[0] > 0
    # bf16 full shape, 2 KV-bytes x 4 heads x 128 x 2 = 2048 B per token per slot
    assert last[0] == 64 * 2048 * (9 * 33024 + 27 * 1024)


# ---------------------------------------------------------------- P12/P13

def test_causality():
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(61, 1, 30, sh.vocab)
    t2 = toks.copy()
    t2[0, 17] = (t2[0, 17] + 1) % sh.vocab
    a = m.step(ref.Cache(sh, ref.MODE_LAST, 1), toks, 2)["hidden"]
    b = m.step(ref.Cache(sh, ref.MODE_LAST, 1), t2, 2)["hidden"]
    np.testing.assert_array_equal(a[:, :17], b[:, :17])
    assert np.all(np.max(np.abs(a[:, 17:] - b[:, 17:]), axis=-1) > 0)


def test_batch_rows_independent():
    sh = synth.TINY_REC_FULL
    m, _ = tiny_model(sh)
    toks = synth.tokens(62, 3, 20, sh.vocab)
    full = m.step(ref.Cache(sh, ref.MODE_LAST, 3), toks, 2)
    one = m.step(ref.Cache(sh, ref.MODE_LAST, 1), toks[1:2], 2)
    np.testing.assert_allclose(full["hidden"][1:2], one["hidden"], atol=1e-14)
    np.testing.assert_allclose(full["logits"][1:2], one["logits"], atol=1e-12)


def test_greedy_lowest_index_on_ties():
    lg = np.array([[0.0, 2.0, 2.0, 1.0], [5.0, 5.0, 5.0, 5.0]])
    np.testing.assert_array_equal(ref.greedy(lg), [1, 0])


# ---------------------------------------------------------------- speculative sampling

def _rand_dists(seed, V, B=1, spread=2.0):
    g = np.random.default_rng(seed)
    return spread * g.standard_normal((B, V)), spread * g.standard_normal((B, V))


def test_speculative_rule_output_law_equals_verifier_distribution():
    """Closed form of the rule (Self-Speculative Decoding: the verifier's
    sampling distribution is preserved): with one draft x ~ q accepted with
    probability a(x) = min(1, p(x) / q(x)) and the residual
    r = max(0, p - q) / sum otherwise, P(first token = y) = q(y) a(y) +
    (1 - sum_x q(x) a(x)) r(y) must equal p(y). The acceptance probability and
    residual are read off the oracle's rule itself by integrating over u:
    draft x is accepted exactly for u below the threshold the rule uses."""
    for seed, T in ((1, 1.0), (2, 0.7), (3, 1.6)):
        dl, vl = _rand_dists(seed, 23)
        q = ref.softmax_t(dl[0], T)
        p = ref.softmax_t(vl[0], T)
        acc = np.zeros(23)
        for x in range(23):
            # the largest u the rule accepts for draft x, by bisection on u
            lo, hi = 0.0, 1.0
            n, _ = ref.speculative_sample(dl[None], np.stack([vl, vl]), np.array([[x]]),
                                          np.array([[1.0 - 1e-15], [0.5]]), T)
            if n[0] == 1:
                acc[x] = 1.0
                continue
            for _ in range(60):
                mid = 0.5 * (lo + hi)
                n, _ = ref.speculative_sample(dl[None], np.stack([vl, vl]), np.array([[x]]),
                                              np.array([[mid], [0.5]]), T)
                lo, hi = (mid, hi) if n[0] == 1 else (lo, mid)
            acc[x] = lo
        # residual: the rule's correction token as a function of the second uniform
        grid = (np.arange(200000) + 0.5) / 200000
        _, corr = ref.speculative_sample(np.repeat(dl[None], 1, 0), np.stack([vl, vl]),
                                         np.array([[int(np.argmax(q - p))]]),
                                         np.array([[1.0 - 1e-15], [0.5]]), T)
        resid_cdf = np.cumsum(np.maximum(p - q, 0))
        resid_cdf /= resid_cdf[-1]
        r = np.diff(np.concatenate([[0.0], resid_cdf]))
        law = q * acc + (1.0 - np.sum(q * acc)) * r
        np.testing.assert_allclose(acc, np.minimum(1.0, p / q), atol=1e-12)
        np.testing.assert_allclose(law, p, atol=1e-12)
        assert 0 <= corr[0] < 23


def test_speculative_rule_monte_carlo_matches_verifier():
    """Seeded uniforms through the oracle's rule (gamma = 2, drafts sampled
    from q by inversion): the empirical law of the first emitted token is the
    verifier's p_1 within 5 binomial standard deviations, and that of the
    second emitted token (conditioned on the first being an accepted draft) is
    p_2."""
    V, N, T = 12, 60000, 1.0
    g = np.random.default_rng(7)
    dl = 1.5 * g.standard_normal((2, 1, V))
    vl = 1.5 * g.standard_normal((3, 1, V))
    q = ref.softmax_t(dl, T)
    p = ref.softmax_t(vl, T)
    u = g.random((N, 5))
    first = np.zeros(V)
    for i in range(N):
        d1 = ref.sample_inverse_cdf(q[0, 0], u[i, 0])
        d2 = ref.sample_inverse_cdf(q[1, 0], u[i, 1])
        n, nxt = ref.speculative_sample(dl, vl, np.array([[d1], [d2]]),
                                        u[i, 2:5].reshape(3, 1), T)
        first[d1 if n[0] >= 1 else nxt[0]] += 1
    sd = np.sqrt(N * p[0, 0] * (1 - p[0, 0]))
    assert np.all(np.abs(first - N * p[0, 0]) <= 5 * sd + 1)


def test_speculative_rule_special_cases():
    """p = q: every draft is accepted and the extra token is drawn from the
    verifier's last distribution; a draft the verifier gives probability 0 is
    always rejected and corrected from the residual; inversion sampling at
    u = 0 gives the first index with mass."""
    g = np.random.default_rng(9)
    dl = g.standard_normal((3, 4, 10))
    vl = np.concatenate([dl, g.standard_normal((1, 4, 10))])
    drafts = g.integers(0, 10, (3, 4))
    u = g.random((4, 4)) * 0.999
    n, nxt = ref.speculative_sample(dl, vl, drafts, u, 1.0)
    assert np.all(n == 3)
    np.testing.assert_array_equal(nxt, ref.sample_inverse_cdf(ref.softmax_t(vl[3], 1.0), u[3]))
    vl2 = vl.copy()
    vl2[0, :, 4] = -np.inf                         # the verifier never emits token 4
    drafts2 = drafts.copy()
    drafts2[0] = 4
    n2, nxt2 = ref.speculative_sample(dl, vl2, drafts2, np.zeros((4, 4)), 1.0)
    assert np.all(n2 == 0) and np.all(nxt2 != 4)
    assert ref.sample_inverse_cdf(np.array([0.0, 0.0, 0.3, 0.7]), np.array(0.0)) == 2
