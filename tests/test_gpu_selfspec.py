"""GPU tests of self-speculative decoding (dory_selfspec_step) and of the
per-loop cache rule it relies on.

With greedy selection, drafting at k_draft and verifying at k_verify must
emit exactly the tokens of plain greedy decoding at k_verify: the rounds are
compared with plain decoding on the GPU and with the float64 oracle's greedy
decoding (tokens whose top-2 logit gap in the oracle is below the GPU's
logit error are not required to agree, nor is anything after them)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log, oracle_model, upload

pytestmark = pytest.mark.gpu

GAP = 0.05   # logit gap below which a greedy choice may legitimately differ


@pytest.fixture(scope="module")
def M():
    from looped_ngpt_transformer_fwd_amd import model
    return model


@pytest.fixture(scope="module")
def tiny(M):
    shape = synth.TINY_REC_FULL
    W = synth.Weights(shape, ref.layer_kinds(shape), 21)
    return shape, W, M.Model(shape, upload(W))


def test_per_loop_fill_rule(M, tiny):
    from looped_ngpt_transformer_fwd_amd import _lib as C
    shape, W, gm = tiny
    toks = torch.from_numpy(synth.tokens(3, 2, 12, shape.vocab)).cuda()
    kv = gm.kv_cache("per_loop", 4, 2, 32)
    gm.prefill(kv, toks[:, :8], 4, logits=False)
    gm.decode_step(kv, toks[:, 8], 1, logits=False, next_token=False)   # fewer loops: allowed
    with pytest.raises(C.DoryError) as e:                               # position 8 lacks loops 2-4
        gm.decode_step(kv, toks[:, 9], 4, logits=False, next_token=False)
    assert e.value.status == C.DORY_ERR_MODE
    gm.decode_step(kv, toks[:, 9], 1, logits=False, next_token=False)   # k = 1 still fine
    kv.set_length(8)                                                    # roll back: allowed again
    gm.decode_step(kv, toks[:, 8], 4, logits=False, next_token=False)
    torch.cuda.synchronize()
    assert kv.length == 9


def _plain(gm, kv, prompt, k, n):
    out = gm.prefill(kv, prompt, k, logits=False, next_token=True)
    t = out["next"]
    toks = [t.cpu().numpy()]
    for _ in range(n - 1):
        t = gm.decode_step(kv, t, k, logits=False, next_token=True)["next"]
        toks.append(t.cpu().numpy())
    torch.cuda.synchronize()
    return np.stack(toks, axis=1)            # [B, n]


def _oracle_greedy(shape, W, prompt, k, n):
    """Oracle greedy tokens and the top-2 logit gap of each choice."""
    om = oracle_model(shape, W)
    B = prompt.shape[0]
    oc = ref.Cache(shape, "per_loop", B)
    o = om.step(oc, prompt, k, logits="last")
    toks, gaps = [], []
    for i in range(n):
        lg = o["logits"]
        srt = np.sort(lg, axis=1)
        gaps.append(srt[:, -1] - srt[:, -2])
        t = np.argmax(lg, axis=1).astype(np.int32)
        toks.append(t)
        if i < n - 1:
            o = om.step(oc, t[:, None], k, logits="last")
    return np.stack(toks, axis=1), np.stack(gaps, axis=1)


def _agree_until_close_call(a, b, gaps):
    for r in range(a.shape[0]):
        for i in range(a.shape[1]):
            if a[r, i] != b[r, i]:
                assert gaps[r, i] < GAP, f"row {r} token {i}: {a[r, i]} vs {b[r, i]}, gap {gaps[r, i]:.3g}"
                break
            if gaps[r, i] < GAP:
                break


@pytest.mark.parametrize("mode", ["per_loop"])
@pytest.mark.parametrize("k_draft", [1, 2, 4])
@pytest.mark.parametrize("B", [2, 16])
def test_selfspec_equals_plain_greedy(M, tiny, mode, k_draft, B):
    shape, W, gm = tiny
    k, gamma, n = 4, 4, 14
    log(f"selfspec B={B} {mode} k_draft={k_draft}")
    prompt = synth.tokens(31 + B, B, 10, shape.vocab)
    tp = torch.from_numpy(prompt).cuda()
    plain = _plain(gm, gm.kv_cache(mode, k, B, 64), tp, k, n)

    kv = gm.kv_cache(mode, k, B, 64)
    last = gm.prefill(kv, tp, k, logits=False, next_token=True)["next"]
    got = [last.cpu().numpy()[:, None]]
    accepted, rounds = 0, 0
    while sum(g.shape[1] for g in got) < n:
        L = kv.length
        na, toks = gm.selfspec_step(kv, last, gamma, k_draft, k)
        torch.cuda.synchronize()
        assert 0 <= na <= gamma and toks.shape == (B, na + 1)
        assert kv.length == L + na + 1
        got.append(toks.cpu().numpy())
        last = toks[:, -1].contiguous()
        accepted += na
        rounds += 1
    spec = np.concatenate(got, axis=1)[:, :n]
    ora, gaps = _oracle_greedy(shape, W, prompt, k, n)
    _agree_until_close_call(plain, ora, gaps)
    _agree_until_close_call(spec, ora, gaps)
    # GPU against GPU: the same tokens up to the first oracle close call
    _agree_until_close_call(spec, plain, gaps)
    log(f"  rounds {rounds}, accepted drafts {accepted}")
    if k_draft == k:
        # drafting at the verifier's own depth, drafts are the verifier's own
        # greedy tokens up to near-ties that the two GEMM paths round
        # differently (common with this tiny random vocabulary, and the batch
        # keeps the shortest accepted prefix): some drafts must be accepted
        assert accepted > 0


def test_selfspec_validation(M, tiny):
    from looped_ngpt_transformer_fwd_amd import _lib as C
    shape, W, gm = tiny
    kv = gm.kv_cache("per_loop", 2, 2, 16)
    last = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = gm.workspace(2, 5)
    scratch = torch.empty(2 * 2 * 5, dtype=torch.int32, device="cuda")
    out = torch.empty(5, 2, dtype=torch.int32, device="cuda")
    n = ctypes.c_int32(-1)

    def call(gamma=4, kd=1, kvf=2, wsb=None):
        return C.dory_selfspec_step(gm.handle, kv.handle, ctypes.c_void_p(last.data_ptr()), 2, gamma,
                                    kd, kvf, kv.mode_code, ctypes.c_void_p(ws.data_ptr()),
                                    ws.numel() if wsb is None else wsb,
                                    ctypes.c_void_p(scratch.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()), n, None)
    assert call(gamma=0) == C.DORY_ERR_ARG
    assert call(kd=3, kvf=2) == C.DORY_ERR_ARG
    assert call(kvf=3) == C.DORY_ERR_MODE            # above k_max
    assert call(wsb=16) == C.DORY_ERR_WORKSPACE
    kv.set_length(12)
    assert call() == C.DORY_ERR_CAPACITY             # 12 + 4 + 1 > 16
    assert kv.length == 12 and n.value == -1
    kv2 = gm.kv_cache("last_loop", 2, 2, 16)
    assert C.dory_selfspec_step(gm.handle, kv2.handle, ctypes.c_void_p(last.data_ptr()), 2, 4, 1, 2,
                                kv2.mode_code, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                ctypes.c_void_p(scratch.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                n, None) == C.DORY_ERR_MODE
