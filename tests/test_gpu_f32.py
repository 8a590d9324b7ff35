"""The fp32 debug build (precision DORY_PRECISION_FP32) on the tiny model of
the parity configuration, through the C ABI, against the float64 oracle on the
same seeded inputs (the same bf16-rounded weight draws, held in fp32): every
k in {1, 2, 4}, both cache policies, one-shot, chunked, ragged-chunk and
prefill + teacher-forced decode patterns, and a batch with per-sequence loop
counts. Bar: max-abs error <= 1e-4 on every loop state, the final hidden
states and the logits (per-token cosine >= 0.999999), greedy tokens equal to
the argmax of the returned logits."""
import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log, oracle_model, per_token_check, upload

pytestmark = pytest.mark.gpu

ABS_F32 = 1e-4
COS_F32 = 0.999999
SHAPES = {"tiny": synth.TINY_F32, "tiny_rec_full": synth.TINY_REC_FULL_F32}
PATTERNS = {
    "one_shot": [(0, 64)],
    "chunked": [(0, 16), (16, 32), (32, 48), (48, 64)],
    "ragged": [(0, 13), (13, 30), (30, 31), (31, 53), (53, 64)],
    "decode": [(0, 32)] + [(t, t + 1) for t in range(32, 64)],
}


def _check(g, o, what):
    per_token_check(g, o, what, cos_min=COS_F32, abs_max=ABS_F32)


@pytest.mark.parametrize("pattern", list(PATTERNS))
@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("shape_name", list(SHAPES))
def test_f32_parity(shape_name, k, mode, pattern):
    from looped_ngpt_transformer_fwd_amd import model as M
    shape = SHAPES[shape_name]
    log(f"fp32 {shape_name} k={k} {mode} {pattern}")
    W = synth.Weights(shape, ref.layer_kinds(shape), 0)
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    B = 2
    toks = synth.tokens(0, B, 64, shape.vocab)
    kv = gm.kv_cache(mode, 4, B, 64)
    oc = ref.Cache(shape, mode, B)
    cur = toks.copy()
    for a, b in PATTERNS[pattern]:
        T = b - a
        tt = torch.from_numpy(cur[:, a:b].copy()).cuda()
        if T == 1 and pattern == "decode":
            out = gm.decode_step(kv, tt[:, 0].contiguous(), k, hidden=True, states=True)
        else:
            out = gm.prefill(kv, tt, k, hidden=True, states=True, next_token=True)
        torch.cuda.synchronize()
        o = om.step(oc, cur[:, a:b], k)
        _check(out["hidden"].cpu().numpy().reshape(B, T, -1), o["hidden"], f"hidden[{a}:{b}]")
        sts = out["states"].cpu().numpy().reshape(k, B, T, -1)
        for i in range(k):
            _check(sts[i], o["states"][i], f"state s_{i + 1}[{a}:{b}]")
        lg = out["logits"].cpu().numpy()
        _check(lg, o["logits"], f"logits[{a}:{b}]")
        nx = out["next"].cpu().numpy()
        np.testing.assert_array_equal(nx, np.argmax(lg, axis=-1))
        if pattern == "decode" and b < 64:
            cur[:, b] = nx
    assert kv.length == 64


def test_f32_mixed_loop_counts():
    """Per-sequence loop counts 1 / 3 / 2 in one batch (last-loop cache),
    prefill then decode, each sequence against its own oracle run."""
    from looped_ngpt_transformer_fwd_amd import model as M
    shape = synth.TINY_REC_FULL_F32
    log("fp32 mixed k")
    W = synth.Weights(shape, ref.layer_kinds(shape), 0)
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    ks = [1, 3, 2]
    B = len(ks)
    toks = synth.tokens(2, B, 40, shape.vocab)
    kv = gm.kv_cache("last_loop", 3, B, 64)
    caches = [ref.Cache(shape, "last_loop", 1) for _ in range(B)]
    for a, b in [(0, 30), (30, 31), (31, 32), (32, 40)]:
        tt = torch.from_numpy(toks[:, a:b].copy()).cuda()
        out = gm.prefill(kv, tt, ks, hidden=True) if b - a > 1 else \
            gm.decode_step(kv, tt[:, 0].contiguous(), ks, hidden=True)
        torch.cuda.synchronize()
        hid = out["hidden"].cpu().numpy().reshape(B, b - a, -1)
        for i in range(B):
            o = om.step(caches[i], toks[i:i + 1, a:b], ks[i])
            _check(hid[i:i + 1], o["hidden"], f"seq {i} hidden[{a}:{b}]")
            _check(out["logits"].cpu().numpy()[i:i + 1], o["logits"], f"seq {i} logits[{a}:{b}]")
