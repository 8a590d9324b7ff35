"""GPU tests of the decode attention forms chosen by batch size: with at
least 256 (sequence, KV head) pairs every pair is one workgroup over all its
keys, writing the gated output directly; smaller batches split the keys and
merge the splits in a second kernel (one group of head-dim threads per
head up to 8 splits, 1024 threads per head up to 64, 32-dim chunks of a
head per workgroup beyond). Both are compared with the oracle (decode steps
on the tiny model with 128 sequences, and the split form with 131 splits on
a synthesized context; the full-shape long-context tests cover the chunked
merge at head_dim 128), and the direct form's graph replays with the direct
launches."""
import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log, oracle_model, per_token_check, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from looped_ngpt_transformer_fwd_amd import model
    return model


@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_direct_form_decode_matches_oracle(M, mode):
    """Tiny model (2 KV heads), 128 sequences: 256 pairs take the direct
    form. Prefill of 40 tokens (rings of 80 rows) then 45 decode steps
    (the sliding-window ring wraps), k = 3, every step against the
    oracle."""
    shape = synth.TINY_REC_FULL
    log(f"direct decode B=128 {mode}")
    W = synth.Weights(shape, ref.layer_kinds(shape), 17)
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    B, P, S, k = 128, 40, 45, 3
    toks = synth.tokens(18, B, P + S, shape.vocab)
    kv = gm.kv_cache(mode, k, B, P + S)
    oc = ref.Cache(shape, mode, B)
    gm.prefill(kv, torch.from_numpy(toks[:, :P].copy()).cuda(), k, logits=False)
    om.step(oc, toks[:, :P], k, logits=None)
    for t in range(P, P + S):
        out = gm.decode_step(kv, torch.from_numpy(toks[:, t].copy()).cuda(), k, hidden=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, t:t + 1], k)
        per_token_check(out["hidden"].cpu().numpy().reshape(B, 1, -1), o["hidden"], f"hidden {t}")
        per_token_check(out["logits"].cpu().numpy(), o["logits"], f"logits {t}")
    assert kv.length == P + S


def test_direct_form_graph_replays(M):
    """The direct form under captured graphs: bit-identical to direct
    launches, step after step."""
    shape = synth.TINY_REC_FULL
    log("direct decode graphs")
    W = synth.Weights(shape, ref.layer_kinds(shape), 19)
    dev = upload(W)
    g, e = M.Model(shape, dev), M.Model(shape, dev)
    e.set_decode_graphs(False)
    B, P, k = 128, 20, 2
    toks = torch.from_numpy(synth.tokens(20, B, P + 12, shape.vocab)).cuda()
    kvg, kve = g.kv_cache("last_loop", k, B, 64), e.kv_cache("last_loop", k, B, 64)
    g.prefill(kvg, toks[:, :P].contiguous(), k, logits=False)
    e.prefill(kve, toks[:, :P].contiguous(), k, logits=False)
    lg = torch.empty(B, shape.vocab, dtype=torch.float32, device="cuda")
    nx = torch.empty(B, dtype=torch.int32, device="cuda")
    tk = torch.empty(B, dtype=torch.int32, device="cuda")
    for step in range(12):
        tk.copy_(toks[:, P + step])
        a = g.decode_step(kvg, tk, k, hidden=True, into={"logits": lg, "next": nx})
        b = e.decode_step(kve, tk, k, hidden=True)
        torch.cuda.synchronize()
        assert torch.equal(a["hidden"], b["hidden"]) and torch.equal(lg, b["logits"]), f"step {step}"


def test_split_form_with_many_splits_matches_oracle(M):
    """One sequence at 33,300 cached positions of a full-attention layer:
    131 splits of 256 keys, merged by 32 groups. The cache holds
    host-drawn K/V; the next decode step's hidden state and logits are
    compared with the oracle on the same cache."""
    shape = synth.TINY_REC_FULL
    log("split form, 131 splits")
    W = synth.Weights(shape, ref.layer_kinds(shape), 23)
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    B, L, k = 1, 33300, 2
    kv = gm.kv_cache("last_loop", k, B, L + 2)
    oc = ref.Cache(shape, "last_loop", B)
    rng = np.random.default_rng(24)
    nkv, dh = shape.n_kv_heads, shape.head_dim
    base = kv.buffer.data_ptr()
    for s, kind in enumerate(ref.layer_kinds(shape)):
        if kind == ref.KIND_MLP:
            continue
        info = kv.slot(s, 0)
        lo = 0 if kind == ref.KIND_FULL else L - shape.window
        K = np.zeros((B, nkv, L + 2, dh))
        V = np.zeros((B, nkv, L + 2, dh))
        kk = (rng.standard_normal((nkv, L - lo, dh)) * 0.3).astype(np.float32)
        vv = (rng.standard_normal((nkv, L - lo, dh)) * 0.3).astype(np.float32)
        kb, vb = synth.bf16_bits_from_f32(kk), synth.bf16_bits_from_f32(vv)
        K[0, :, lo:L] = synth.f64_from_bf16_bits(kb)
        V[0, :, lo:L] = synth.f64_from_bf16_bits(vb)
        pos = np.arange(lo, L)
        rows = torch.from_numpy(pos % info.ring if info.ring > 0 else pos).cuda()
        n = nkv * info.rows * dh * 2
        kd = kv.buffer[info.k - base:info.k - base + n].view(torch.int16).view(nkv, info.rows, dh)
        vd = kv.buffer[info.v - base:info.v - base + n].view(torch.int16).view(nkv, dh, info.rows)
        kd[:, rows] = torch.from_numpy(kb.view(np.int16)).cuda()
        vd[:, :, rows] = torch.from_numpy(vb.view(np.int16)).cuda().transpose(1, 2)
        oc.K[(s, 0)], oc.V[(s, 0)] = K, V
    oc.length = L
    kv.set_length(L)
    tok = synth.tokens(25, B, 2, shape.vocab)
    for j in range(2):
        out = gm.decode_step(kv, torch.from_numpy(tok[:, j].copy()).cuda(), k, hidden=True)
        torch.cuda.synchronize()
        o = om.step(oc, tok[:, j:j + 1], k, literal_overwrite=True)
        per_token_check(out["hidden"].cpu().numpy().reshape(B, 1, -1), o["hidden"], f"hidden {L + j}")
        per_token_check(out["logits"].cpu().numpy(), o["logits"], f"logits {L + j}")
