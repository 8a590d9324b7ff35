"""GPU parity of steps whose sequences run different loop counts
(dory_prefill_rows / dory_decode_step_rows, last-loop cache).

The reference for a mixed batch is each sequence run alone through the
float64 oracle at its own loop count, with its own cache: sequences never
attend to each other, so a mixed step must reproduce every one of them.
Covered: the tiny model (small-M path, ring caches, chunked prefill, decode),
a head-dim-128 model whose prefill takes the large-M fused q/k/v epilogue and
the per-sequence KV store at each sequence's own last loop, and the
full-width recurrent pair at T = 1,100 (sliding-window ring wrapped) with
decode steps after it.
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


def _run(M, shape, k_rows, chunks, n_dec, seed, logits=True):
    B = len(k_rows)
    log(f"mixed k {k_rows} on d={shape.d_model} chunks={chunks} decode={n_dec}")
    W = synth.Weights(shape, ref.layer_kinds(shape), seed)
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    L = chunks[-1][1] + n_dec
    toks = synth.tokens(seed + 1, B, L, shape.vocab)
    kv = gm.kv_cache("last_loop", max(k_rows), B, L)
    ocs = [ref.Cache(shape, "last_loop", 1) for _ in range(B)]
    want = "last" if (logits and shape.has_lm_head) else None

    def check(out, a, b, what):
        for r in range(B):
            o = om.step(ocs[r], toks[r:r + 1, a:b], k_rows[r], logits=want)
            hid = out["hidden"].reshape(B, b - a, -1)[r:r + 1].cpu().numpy()
            per_token_check(hid, o["hidden"], f"{what} row {r} hidden")
            st = out["states"]
            for i in range(k_rows[r]):
                per_token_check(st[i].reshape(B, b - a, -1)[r:r + 1].cpu().numpy(), o["states"][i],
                                f"{what} row {r} s_{i + 1}")
            if want:
                per_token_check(out["logits"][r:r + 1].cpu().numpy(), o["logits"],
                                f"{what} row {r} logits")

    for a, b in chunks:
        out = gm.prefill(kv, torch.from_numpy(toks[:, a:b].copy()).cuda(), list(k_rows),
                         logits=bool(want), hidden=True, states=True)
        torch.cuda.synchronize()
        check(out, a, b, f"prefill [{a},{b})")
    for t in range(chunks[-1][1], L):
        out = gm.decode_step(kv, torch.from_numpy(toks[:, t].copy()).cuda(), list(k_rows),
                             logits=bool(want), next_token=bool(want), hidden=True, states=True)
        torch.cuda.synchronize()
        check(out, t, t + 1, f"decode {t}")
        if want:
            lg = out["logits"].cpu().numpy()
            np.testing.assert_array_equal(out["next"].cpu().numpy(),
                                          np.argmax(lg, axis=1).astype(np.int32))
    assert kv.length == L


@pytest.mark.parametrize("k_rows", [(1, 3, 2), (4, 1, 4), (2, 2, 2)])
def test_mixed_k_tiny(M, k_rows):
    _run(M, synth.TINY_REC_FULL, k_rows, [(0, 21), (21, 40)], 4, seed=5)


def test_mixed_k_large_m_fused_path(M):
    _run(M, synth.MID128, (1, 3), [(0, 600), (600, 1100)], 2, seed=6)


def test_mixed_k_full_width_pair(M):
    _run(M, synth.PAIR, (4, 2), [(0, 1100)], 2, seed=7, logits=False)
