"""GPU tests of prefix caching (dory_kv_copy_prefix): a prompt prefix is
prefilled once for one sequence, its cached K/V is copied into the
sequences of another cache, and each sequence then continues with its own
suffix and decode steps. Every continued sequence must match the float64
oracle run on the whole prompt (prefix and suffix as two chunks), under
both cache policies, with sliding-window rings that have wrapped, and on
the large-M path with a cached prefix."""
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


def _check_continuation(M, shape, mode, k, n, T, n_dec, B, seed, dst_max=None, same_cache=False):
    log(f"prefix copy d={shape.d_model} {mode} k={k} n={n} T={T} B={B} same={same_cache}")
    W = synth.Weights(shape, ref.layer_kinds(shape), seed)
    gm = M.Model(shape, upload(W))
    prefix = synth.tokens(seed + 1, 1, n, shape.vocab)
    rest = synth.tokens(seed + 2, B, T + n_dec, shape.vocab)
    full = np.concatenate([np.repeat(prefix, B, axis=0), rest], axis=1)
    L = n + T + n_dec
    lm = "last" if shape.has_lm_head else None

    if same_cache:
        # one cache: sequence 0 runs the prefix, the others get junk there
        # and then receive sequence 0's entries
        dst = gm.kv_cache(mode, k, B, dst_max or L)
        junk = synth.tokens(seed + 3, B, n, shape.vocab)
        junk[0] = prefix[0]
        gm.prefill(dst, torch.from_numpy(junk).cuda(), k, logits=False)
        for b in range(1, B):
            dst.copy_prefix_from(dst, 0, b, n)
    else:
        src = gm.kv_cache(mode, k, 1, n + 8)
        gm.prefill(src, torch.from_numpy(prefix).cuda(), k, logits=False)
        dst = gm.kv_cache(mode, k, B, dst_max or L)
        for b in range(B):
            dst.copy_prefix_from(src, 0, b, n)
    assert dst.length == n

    om = oracle_model(shape, W)
    oc = ref.Cache(shape, mode, B)
    om.step(oc, full[:, :n], k, logits=None)
    out = gm.prefill(dst, torch.from_numpy(rest[:, :T].copy()).cuda(), k, logits=bool(lm), hidden=True)
    torch.cuda.synchronize()
    o = om.step(oc, full[:, n:n + T], k, logits=lm)
    per_token_check(out["hidden"].cpu().numpy(), o["hidden"], "suffix hidden")
    if lm:
        per_token_check(out["logits"].cpu().numpy(), o["logits"], "suffix logits")
    for t in range(n_dec):
        tok = torch.from_numpy(rest[:, T + t].copy()).cuda()
        out = gm.decode_step(dst, tok, k, logits=bool(lm), next_token=False, hidden=True)
        torch.cuda.synchronize()
        o = om.step(oc, full[:, n + T + t:n + T + t + 1], k, logits=lm)
        per_token_check(out["hidden"].cpu().numpy(), o["hidden"], f"decode {t} hidden")
        if lm:
            per_token_check(out["logits"].cpu().numpy(), o["logits"], f"decode {t} logits")
    return gm, dst


@pytest.mark.parametrize("k", [1, 3])
@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_tiny_prefix_copy(M, mode, k):
    # 101-token prefix: the sliding-window rings (window 16 + 64 rows) have
    # wrapped in the source
    _check_continuation(M, synth.TINY_REC_FULL, mode, k, n=101, T=7, n_dec=2, B=3, seed=41)


@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_tiny_prefix_copy_within_one_cache(M, mode):
    _check_continuation(M, synth.TINY_REC_FULL, mode, 2, n=19, T=5, n_dec=1, B=3, seed=43,
                        same_cache=True)


def test_tiny_prefix_copy_into_smaller_ring(M):
    # destination max_seq 8: its sliding-window rings hold 8 rows, the source's 16
    # (max_seq 13 rounded up to 8 rows)
    _check_continuation(M, synth.TINY_REC_FULL, "last_loop", 2, n=5, T=2, n_dec=1, B=2, seed=44,
                        dst_max=8)


def test_mid128_prefix_copy_large_m(M):
    # 300-token prefix (window-64 rings wrapped), 2 x 280-token suffixes take
    # the large-M GEMM path with the fused q/k/v epilogue over a cached prefix
    _check_continuation(M, synth.MID128, "last_loop", 2, n=300, T=280, n_dec=1, B=2, seed=45)


def test_per_loop_copy_carries_the_source_loops(M):
    """A source prefilled with 2 loops gives the destination loops 1-2 only:
    a 4-loop step is a mode error, a 2-loop step matches the oracle."""
    from looped_ngpt_transformer_fwd_amd import _lib as C
    shape = synth.TINY_REC_FULL
    W = synth.Weights(shape, ref.layer_kinds(shape), 46)
    gm = M.Model(shape, upload(W))
    prefix = synth.tokens(47, 1, 11, shape.vocab)
    src = gm.kv_cache("per_loop", 4, 1, 16)
    gm.prefill(src, torch.from_numpy(prefix).cuda(), 2, logits=False)
    dst = gm.kv_cache("per_loop", 4, 2, 16)
    dst.copy_prefix_from(src, 0, 0, 11)
    dst.copy_prefix_from(src, 0, 1, 11)
    rest = synth.tokens(48, 2, 3, shape.vocab)
    with pytest.raises(C.DoryError) as e:
        gm.prefill(dst, torch.from_numpy(rest).cuda(), 4, logits=False)
    assert e.value.status == C.DORY_ERR_MODE and dst.length == 11
    out = gm.prefill(dst, torch.from_numpy(rest).cuda(), 2, logits=True, hidden=True)
    torch.cuda.synchronize()
    om = oracle_model(shape, W)
    oc = ref.Cache(shape, "per_loop", 2)
    om.step(oc, np.repeat(prefix, 2, axis=0), 2, logits=None)
    o = om.step(oc, rest, 2, logits="last")
    per_token_check(out["hidden"].cpu().numpy(), o["hidden"], "hidden")
    per_token_check(out["logits"].cpu().numpy(), o["logits"], "logits")
