"""GPU parity where the projections run the large-M GEMM path.

* mid-size model, 1100 tokens: ragged M and N tiles, an odd number of K
  steps, two chunks (the second with a cached prefix) under both policies;
* the full-width recurrent pair [SWA, MLP, full, MLP] at d=2304, 16/4 heads
  of 128, SwiGLU 6144, window 1024, B=1 x T=4096, k = 1..4, compared with the
  float64 oracle on every loop state and the final hidden states.
"""
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


@pytest.mark.parametrize("shape_name", ["mid", "mid128"])
@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_mid_model_large_gemm_path(M, mode, shape_name):
    shape = {"mid": synth.MID, "mid128": synth.MID128}[shape_name]
    k = 2
    log(f"{shape_name} {mode}")
    W = synth.Weights(shape, ref.layer_kinds(shape), 3)
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    B = 1
    toks = synth.tokens(9, B, 2213, shape.vocab)
    kv = gm.kv_cache(mode, k, B, 2300)
    oc = ref.Cache(shape, mode, B)
    for a, b in [(0, 1100), (1100, 2213)]:
        out = gm.prefill(kv, torch.from_numpy(toks[:, a:b].copy()).cuda(), k, hidden=True,
                         states=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, a:b], k)
        per_token_check(out["hidden"].cpu().numpy(), o["hidden"], f"hidden[{a}:{b}]")
        st = out["states"].cpu().numpy()
        for i in range(k):
            per_token_check(st[i], o["states"][i], f"s_{i + 1}[{a}:{b}]")
        per_token_check(out["logits"].cpu().numpy(), o["logits"], f"logits[{a}:{b}]")


@pytest.fixture(scope="module")
def pair(M):
    shape = synth.PAIR
    W = synth.Weights(shape, ref.layer_kinds(shape), 0)
    log("pair: drawing weights")
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    return shape, W, gm, om


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_recurrent_pair_full_width(pair, k):
    shape, W, gm, om = pair
    log(f"pair k={k}")
    B, T = 1, 4096
    toks = synth.tokens(2, B, T, shape.vocab)
    kv = gm.kv_cache("last_loop", k, B, T)
    out = gm.prefill(kv, torch.from_numpy(toks).cuda(), k, logits=False, hidden=True, states=True)
    torch.cuda.synchronize()
    o = om.step(ref.Cache(shape, "last_loop", B), toks, k, logits=None)
    st = out["states"].cpu().numpy()
    for i in range(k):
        c, m = per_token_check(st[i], o["states"][i], f"s_{i + 1}")
        log(f"  s_{i + 1}: min cos {c:.6f} max abs {m:.2e}")
    per_token_check(out["hidden"].cpu().numpy(), o["hidden"], "hidden")


@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_recurrent_pair_decode_full_width(pair, mode):
    """Decode at full width after a 1100-token prefill: the sliding-window
    ring has wrapped and the full-attention keys span several 128-key decode
    blocks; k=2 under both cache policies."""
    shape, W, gm, om = pair
    log(f"pair decode {mode}")
    B, k, T0, steps = 2, 2, 1100, 3
    toks = synth.tokens(4, B, T0 + steps, shape.vocab)
    kv = gm.kv_cache(mode, k, B, T0 + steps)
    oc = ref.Cache(shape, mode, B)
    gm.prefill(kv, torch.from_numpy(toks[:, :T0].copy()).cuda(), k, logits=False)
    om.step(oc, toks[:, :T0], k, logits=None)
    for t in range(T0, T0 + steps):
        out = gm.decode_step(kv, torch.from_numpy(toks[:, t].copy()).cuda(), k, logits=False,
                             next_token=False, hidden=True, states=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, t:t + 1], k, logits=None)
        st = out["states"].cpu().numpy()
        for i in range(k):
            per_token_check(st[i].reshape(B, 1, -1), o["states"][i], f"decode {t} s_{i + 1}")
        per_token_check(out["hidden"].cpu().numpy().reshape(B, 1, -1), o["hidden"], f"decode {t} hidden")


def test_recurrent_pair_rows_between_64_and_1024(pair):
    """Projections with 64 < M < 1024 rows at full width: the skinny GEMM's
    XCD-grouped 64-row blocks with K = 2304 and 6144 and N up to 12288, last
    block ragged. Chunked prefill of 3 sequences (600 and 990 rows) under the
    per-loop cache, then decode of 100 sequences (100 rows) after a 12-token
    prefill (1200 rows, large-M path)."""
    shape, W, gm, om = pair
    k = 2
    log("pair 3 x (200 + 330) per_loop")
    B = 3
    toks = synth.tokens(5, B, 530, shape.vocab)
    kv = gm.kv_cache("per_loop", k, B, 530)
    oc = ref.Cache(shape, "per_loop", B)
    for a, b in [(0, 200), (200, 530)]:
        out = gm.prefill(kv, torch.from_numpy(toks[:, a:b].copy()).cuda(), k, logits=False,
                         hidden=True, states=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, a:b], k, logits=None)
        st = out["states"].cpu().numpy()
        for i in range(k):
            per_token_check(st[i], o["states"][i], f"[{a},{b}) s_{i + 1}")
        per_token_check(out["hidden"].cpu().numpy(), o["hidden"], f"[{a},{b}) hidden")
    log("pair decode B=100")
    B, T0 = 100, 12
    toks = synth.tokens(6, B, T0 + 2, shape.vocab)
    kv = gm.kv_cache("last_loop", k, B, T0 + 2)
    oc = ref.Cache(shape, "last_loop", B)
    gm.prefill(kv, torch.from_numpy(toks[:, :T0].copy()).cuda(), k, logits=False)
    om.step(oc, toks[:, :T0], k, logits=None)
    for t in range(T0, T0 + 2):
        out = gm.decode_step(kv, torch.from_numpy(toks[:, t].copy()).cuda(), k, logits=False,
                             next_token=False, hidden=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, t:t + 1], k, logits=None)
        per_token_check(out["hidden"].cpu().numpy().reshape(B, 1, -1), o["hidden"], f"decode {t} hidden")
