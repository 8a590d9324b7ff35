"""GPU checks of the full 72-sublayer model (d=2304, 16/4 heads of 128,
SwiGLU 6144, window 1024, vocab 131072, 16 input + 40 recurrent x k + 16
output sublayers) at the sizes and launch configurations of the benchmark.

* Prefill B=4 x T=8192, k = 1, 2, 4: attention is causal, so the first S
  positions of a sequence depend on its first S tokens only; at k = 1 and 4
  the first 1,100 positions of sequence 0 (beyond the 1,024-key window, over
  several key and query tiles), at k = 2 the first 48 of sequences 0 and 3,
  are compared with the float64 oracle run on those tokens (hidden state and
  every loop state). At every position: hidden rows have
  unit length, the logits are s_z times the inner products of the last hidden
  row with the LM-head rows, and the greedy token is their argmax (lowest
  index on ties, bit-exact). Prefill from an empty cache does not depend on
  the cache policy: per-loop caching gives bit-identical hidden states.
* Decode B=64 at position 32768: sequences 0 and 63 get cached keys and
  values drawn on the host (the input generator), written into both the
  device cache slots and the oracle's cache; the rest of the cache is random.
  One decode step per (k, policy) against the oracle: loop states, hidden
  state and logits of both sequences.
* Long context, one sequence of 262144 positions at k=4: with 262120
  cached positions drawn on the host, a 16-token prefill chunk and two
  decode steps under last-loop caching against the oracle; and, under
  per-loop caching, chunked prefill of 262144 real tokens in 8192-token
  chunks, where decode steps over the whole prefix give the loop states,
  hidden states and logits that a prefill chunk computes at the same
  positions.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log, per_token_check, upload

pytestmark = pytest.mark.gpu

SHAPE = synth.FULL
UNIT_TOL = 1e-4


class _RowGather:
    """Embedding rows widened to float64 on demand."""

    def __init__(self, bits):
        self.bits = bits

    def __getitem__(self, idx):
        return synth.f64_from_bf16_bits(self.bits[idx])


@pytest.fixture(scope="module")
def full():
    from looped_ngpt_transformer_fwd_amd import model as M
    kinds = ref.layer_kinds(SHAPE)
    log("full model: drawing weights")
    W = synth.Weights(SHAPE, kinds, 0)
    gm = M.Model(SHAPE, upload(W))
    cache = {"embed": _RowGather(W.raw("embed"))}

    def weight(name):
        if name not in cache:
            cache[name] = W.f64(name)
        return cache[name]
    om = ref.OracleModel(SHAPE, weight)
    yield weight, gm, om
    del gm
    torch.cuda.empty_cache()


def _check_unit_rows(h, what):
    n = torch.linalg.vector_norm(h.reshape(-1, h.shape[-1]).double(), dim=1)
    assert bool(torch.isfinite(n).all()), f"{what}: non-finite rows"
    err = float((n - 1.0).abs().max())
    assert err <= UNIT_TOL, f"{what}: row norm off by {err:.2e}"


def _check_lm_head(weight, hidden_last, logits, nxt, what):
    """logits = s_z * (h W_lm^T) per row (float64 on the host) and next is
    the first maximum of the device logits."""
    h = hidden_last.cpu().numpy().astype(np.float64)
    lg = logits.cpu().numpy()
    want = weight("s_z")[None, :] * (h @ weight("lm_head").T)
    per_token_check(lg, want, f"{what} logits")
    np.testing.assert_array_equal(nxt.cpu().numpy(), np.argmax(lg, axis=1).astype(np.int32))


@pytest.mark.parametrize("k", [1, 2, 4])
def test_prefill_benchmark_config(full, k):
    """At k = 1 and 4 the first 1,100 positions of sequence 0 (past the
    1,024-key window of the sliding-window layers, over 17 causal key tiles
    and 5 query tiles of the attention kernel), at k = 2 the first 48 of
    sequences 0 and 3, against the oracle run on those tokens (causality
    makes the prefix exact)."""
    weight, gm, om = full
    B, T = 4, 8192
    S, rows = (48, [0, 3]) if k == 2 else (1100, [0])
    log(f"full prefill B={B} T={T} k={k}")
    toks = synth.tokens(0, B, T, SHAPE.vocab)
    kv = gm.kv_cache("last_loop", k, B, T)
    out = gm.prefill(kv, torch.from_numpy(toks).cuda(), k, logits=True, next_token=True,
                     hidden=True, states=True)
    torch.cuda.synchronize()
    _check_unit_rows(out["hidden"], "hidden")
    for i in range(k):
        _check_unit_rows(out["states"][i], f"s_{i + 1}")
    _check_lm_head(weight, out["hidden"][:, -1], out["logits"], out["next"], "last position")

    o = om.step(ref.Cache(SHAPE, "last_loop", len(rows)), toks[rows, :S], k, logits=None)
    per_token_check(out["hidden"][rows, :S].cpu().numpy(), o["hidden"], f"hidden[:{S}]")
    for i in range(k):
        per_token_check(out["states"][i][rows, :S].cpu().numpy(), o["states"][i],
                        f"s_{i + 1}[:{S}]")

    if k == 2:
        hid = out["hidden"].clone()
        del out, kv
        kvp = gm.kv_cache("per_loop", k, B, T)
        outp = gm.prefill(kvp, torch.from_numpy(toks).cuda(), k, logits=False, hidden=True)
        torch.cuda.synchronize()
        assert torch.equal(outp["hidden"], hid), "per-loop prefill differs from last-loop"


def _fill_context(gm, kv, oc, mode, k, rows, ctx, seed, cap=None):
    """Writes host-drawn K/V of positions [0, ctx) for the sampled rows into
    the device slots (K rows at the position or at position mod ring, V^T
    columns likewise) and into the oracle cache (float64, linear, `cap`
    positions, ctx + 1 by default, so that later entries are stored in
    place)."""
    cap = ctx + 1 if cap is None else cap
    kinds = ref.layer_kinds(SHAPE)
    nkv, dh, win = SHAPE.n_kv_heads, SHAPE.head_dim, SHAPE.window
    base = kv.buffer.data_ptr()
    for s, kind in enumerate(kinds):
        if kind == ref.KIND_MLP:
            continue
        slots = k if (mode == "per_loop" and ref.block_of(SHAPE, s) == "recurrent") else 1
        lo = 0 if kind == ref.KIND_FULL else ctx - (win - 1)
        for slot in range(slots):
            info = kv.slot(s, slot)
            R = info.rows
            K = np.zeros((len(rows), nkv, cap, dh))
            V = np.zeros((len(rows), nkv, cap, dh))
            pos = np.arange(lo, ctx)
            dev_rows = torch.from_numpy(pos % info.ring if info.ring > 0 else pos).cuda()
            for j, b in enumerate(rows):
                kb, vb = synth.kv_context(seed, s, slot, b, nkv, ctx - lo, dh)
                K[j, :, lo:ctx] = synth.f64_from_bf16_bits(kb)
                V[j, :, lo:ctx] = synth.f64_from_bf16_bits(vb)
                n = nkv * R * dh * 2
                ko = info.k - base + b * n
                vo = info.v - base + b * n
                kd = kv.buffer[ko:ko + n].view(torch.int16).view(nkv, R, dh)
                vd = kv.buffer[vo:vo + n].view(torch.int16).view(nkv, dh, R)
                kd[:, dev_rows] = torch.from_numpy(kb.view(np.int16)).cuda()
                vd[:, :, dev_rows] = torch.from_numpy(vb.view(np.int16)).cuda().transpose(1, 2)
            oc.K[(s, slot)] = K
            oc.V[(s, slot)] = V
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_decode_benchmark_config(full, mode, k):
    weight, gm, om = full
    B, ctx = 64, 32768
    rows = [0, 63]
    log(f"full decode B={B} ctx={ctx} k={k} {mode}")
    kv = gm.kv_cache(mode, k, B, ctx + 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    buf = kv.buffer.view(torch.bfloat16)
    chunk = 1 << 28
    for o in range(0, buf.numel(), chunk):
        n = min(chunk, buf.numel() - o)
        buf[o:o + n] = (0.02 * torch.randn(n, device="cuda", generator=g)).to(torch.bfloat16)
    oc = ref.Cache(SHAPE, mode, len(rows))
    _fill_context(gm, kv, oc, mode, k, rows, ctx, seed=11)
    oc.length = ctx
    kv.set_length(ctx)
    toks = synth.tokens(12, B, 1, SHAPE.vocab)
    out = gm.decode_step(kv, torch.from_numpy(toks[:, 0].copy()).cuda(), k, logits=True,
                         next_token=True, hidden=True, states=True)
    torch.cuda.synchronize()
    assert kv.length == ctx + 1
    _check_unit_rows(out["hidden"], "hidden")
    _check_lm_head(weight, out["hidden"].reshape(B, -1), out["logits"], out["next"], "decode")
    o = om.step(oc, toks[rows], k, logits="last")
    per_token_check(out["hidden"].reshape(B, 1, -1)[rows].cpu().numpy(), o["hidden"], "hidden")
    for i in range(k):
        per_token_check(out["states"][i].reshape(B, 1, -1)[rows].cpu().numpy(), o["states"][i],
                        f"s_{i + 1}")
    per_token_check(out["logits"][rows].cpu().numpy(), o["logits"], "logits")
    del out, kv, buf
    torch.cuda.empty_cache()


def test_long_context_against_oracle(full):
    """One sequence at the long-context shape, k=4, last-loop caching:
    262120 cached positions drawn on the host (full-attention slots hold all
    of them, sliding-window slots the last 1023), then a 16-token prefill
    chunk and two decode steps, each against the oracle on the same cache.
    The oracle overwrites its cache entries at every loop and reads them
    back (the literal form of last-loop caching, pinned equal to the
    reading-before-writing form), which keeps its cache arrays in place."""
    weight, gm, om = full
    L, k, C, n_dec = 262144, 4, 16, 2
    ctx = L - 24
    log(f"long context against the oracle: ctx={ctx} k={k}")
    kv = gm.kv_cache("last_loop", k, 1, L)
    kv.buffer.zero_()
    oc = ref.Cache(SHAPE, "last_loop", 1)
    _fill_context(gm, kv, oc, "last_loop", k, [0], ctx, seed=31, cap=L)
    oc.length = ctx
    kv.set_length(ctx)
    toks = synth.tokens(32, 1, C + n_dec, SHAPE.vocab)
    out = gm.prefill(kv, torch.from_numpy(toks[:, :C].copy()).cuda(), k, logits=True,
                     next_token=True, hidden=True, states=True)
    torch.cuda.synchronize()
    o = om.step(oc, toks[:, :C], k, literal_overwrite=True, logits="last")
    per_token_check(out["hidden"].cpu().numpy(), o["hidden"], "prefill hidden")
    for i in range(k):
        per_token_check(out["states"][i].cpu().numpy(), o["states"][i], f"prefill s_{i + 1}")
    per_token_check(out["logits"].cpu().numpy(), o["logits"], "prefill logits")
    for j in range(C, C + n_dec):
        out = gm.decode_step(kv, torch.from_numpy(toks[:, j].copy()).cuda(), k, logits=True,
                             next_token=True, hidden=True, states=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, j:j + 1], k, literal_overwrite=True, logits="last")
        per_token_check(out["hidden"].reshape(1, 1, -1).cpu().numpy(), o["hidden"],
                        f"decode {ctx + j} hidden")
        for i in range(k):
            per_token_check(out["states"][i].reshape(1, 1, -1).cpu().numpy(), o["states"][i],
                            f"decode {ctx + j} s_{i + 1}")
        per_token_check(out["logits"].cpu().numpy(), o["logits"], f"decode {ctx + j} logits")
    assert kv.length == ctx + C + n_dec
    del kv
    torch.cuda.empty_cache()


def test_long_context_per_loop_decode_matches_prefill(full):
    """Under per-loop caching every loop reads keys of its own loop, so a
    token's result does not depend on how the sequence was split into steps.
    One sequence of 262144 tokens at k=4: chunked prefill in 8192-token
    chunks, then the last 8 positions once as part of a prefill chunk and
    once as decode steps over the whole prefix. (Under last-loop caching the
    two legitimately differ: inside a chunk, earlier positions of the same
    chunk are read at the current loop, cached positions at the last loop.)"""
    weight, gm, om = full
    L, CH, k, n_dec = 262144, 8192, 4, 8
    log(f"long context per_loop L={L} chunks of {CH} k={k}")
    toks = synth.tokens(21, 1, L, SHAPE.vocab)
    dtoks = torch.from_numpy(toks).cuda()
    kv = gm.kv_cache("per_loop", k, 1, L)
    ws = gm.workspace(1, CH)
    for c in range(0, L - CH, CH):
        out = gm.prefill(kv, dtoks[:, c:c + CH], k, ws=ws, logits=False, hidden=True)
        _check_unit_rows(out["hidden"], f"chunk at {c}")
    torch.cuda.synchronize()
    log("  prefix done")
    snap = kv.buffer.clone()
    ref_out = gm.prefill(kv, dtoks[:, L - CH:], k, ws=ws, logits=True, next_token=True,
                         hidden=True, states=True)
    torch.cuda.synchronize()
    kv.buffer.copy_(snap)
    del snap
    # the device memory is restored: declare its positions valid again (a
    # plain roll-back by a whole chunk is refused once the rings wrapped)
    kv.reset()
    kv.set_length(L - CH)
    gm.prefill(kv, dtoks[:, L - CH:L - n_dec], k, ws=ws, logits=False)
    for j in range(n_dec):
        p = L - n_dec + j
        out = gm.decode_step(kv, dtoks[:, p], k, logits=True, next_token=True, hidden=True,
                             states=True)
        torch.cuda.synchronize()
        at = CH - n_dec + j
        for i in range(k):
            per_token_check(out["states"][i].reshape(1, -1).cpu().numpy(),
                            ref_out["states"][i][:, at].cpu().numpy(), f"decode at {p} s_{i + 1}")
        per_token_check(out["hidden"].reshape(1, -1).cpu().numpy(),
                        ref_out["hidden"][:, at].cpu().numpy(), f"decode at {p}")
    per_token_check(out["logits"].cpu().numpy(), ref_out["logits"].cpu().numpy(),
                    "logits at the last position")
    assert kv.length == L
    del kv
    torch.cuda.empty_cache()


def _top2_gap(logits):
    srt = np.sort(logits, axis=1)
    return srt[:, -1] - srt[:, -2]


def test_selfspec_full_shape_matches_plain_decode(full):
    """Self-speculative rounds at full shape (per-loop cache, 4 sequences,
    40-token prompts, gamma 4, verify at k = 4, drafts at k = 1 and 4) emit
    the tokens of plain greedy decoding at k = 4, up to the first position
    whose top-2 logit gap in the plain run is below 0.05 (rounding of the
    different launch shapes may pick the other token there)."""
    _, gm, _ = full
    B, T0, k, gamma, n = 4, 40, 4, 4, 8
    toks = torch.from_numpy(synth.tokens(71, B, T0, SHAPE.vocab)).cuda()
    kv = gm.kv_cache("per_loop", k, B, T0 + 16)
    out = gm.prefill(kv, toks, k, logits=True, next_token=True)
    t = out["next"]
    plain, gaps = [t.cpu().numpy()], [_top2_gap(out["logits"].cpu().numpy())]
    for _ in range(n - 1):
        out = gm.decode_step(kv, t, k, logits=True, next_token=True)
        t = out["next"]
        plain.append(t.cpu().numpy())
        gaps.append(_top2_gap(out["logits"].cpu().numpy()))
    torch.cuda.synchronize()
    plain, gaps = np.stack(plain, axis=1), np.stack(gaps, axis=1)
    del kv
    for kd in (1, k):
        log(f"full-shape selfspec k_draft={kd}")
        kv = gm.kv_cache("per_loop", k, B, T0 + 16)
        last = gm.prefill(kv, toks, k, logits=False, next_token=True)["next"]
        got, accepted = [last.cpu().numpy()[:, None]], 0
        while sum(x.shape[1] for x in got) < n:
            na, tk = gm.selfspec_step(kv, last, gamma, kd, k)
            got.append(tk.cpu().numpy())
            last = tk[:, -1].contiguous()
            accepted += na
        torch.cuda.synchronize()
        spec = np.concatenate(got, axis=1)[:, :n]
        compared = 0
        for r in range(B):
            for i in range(n):
                if spec[r, i] != plain[r, i]:
                    assert gaps[r, i] < 0.05, f"row {r} token {i}: {spec[r, i]} vs {plain[r, i]}"
                    break
                compared += 1
                if gaps[r, i] < 0.05:
                    break
        log(f"  accepted drafts {accepted}, tokens compared {compared}")
        assert compared >= B
        if kd == k:
            assert accepted > 0
        del kv


def test_prefix_copy_full_shape_continuation(full):
    """Prefix caching at full shape: an 1100-token prefix (the sliding-window
    rings of 1,024 + 64 rows have wrapped) prefilled once for one sequence and
    copied into two, then a 40-token suffix and one decode step, matches
    prefilling the whole prompt for both sequences, bit for bit: the prefix
    runs the large-M kernels either way (1,100 or 2,200 rows), which compute
    every row the same way whatever the row count (no split-K), so the
    copied entries equal the ones computed in place."""
    _, gm, _ = full
    B, n, T, k = 2, 1100, 40, 2
    prefix = synth.tokens(72, 1, n, SHAPE.vocab)
    rest = torch.from_numpy(synth.tokens(73, B, T + 1, SHAPE.vocab)).cuda()
    ref_kv = gm.kv_cache("last_loop", k, B, n + T + 1)
    gm.prefill(ref_kv, torch.from_numpy(np.repeat(prefix, B, axis=0)).cuda(), k, logits=False)
    want = gm.prefill(ref_kv, rest[:, :T].contiguous(), k, logits=True, hidden=True)
    want_d = gm.decode_step(ref_kv, rest[:, T].contiguous(), k, logits=True, next_token=False,
                            hidden=True)
    src = gm.kv_cache("last_loop", k, 1, n)
    gm.prefill(src, torch.from_numpy(prefix).cuda(), k, logits=False)
    dst = gm.kv_cache("last_loop", k, B, n + T + 1)
    for b in range(B):
        dst.copy_prefix_from(src, 0, b, n)
    got = gm.prefill(dst, rest[:, :T].contiguous(), k, logits=True, hidden=True)
    got_d = gm.decode_step(dst, rest[:, T].contiguous(), k, logits=True, next_token=False, hidden=True)
    torch.cuda.synchronize()
    for what, a, b in [("suffix hidden", got["hidden"], want["hidden"]),
                       ("suffix logits", got["logits"], want["logits"]),
                       ("decode hidden", got_d["hidden"], want_d["hidden"]),
                       ("decode logits", got_d["logits"], want_d["logits"])]:
        a, b = a.cpu().numpy(), b.cpu().numpy()
        per_token_check(a, b.astype(np.float64), what)
        np.testing.assert_array_equal(a, b, err_msg=what)
