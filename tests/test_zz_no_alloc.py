"""The allocation-free decode step (dory_decode_step_noalloc, for callers that
cannot allocate: graph capture, tight serving loops) against dory_decode_step
through the C ABI: identical caches, identical inputs, two calls in a row with
the second on a smaller batch (the static scratch keeps the first call's
contents). The two entry points run the same kernels with the same split
choices, so every output is bit-identical, which is within the parity bar of
the oracle comparisons."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log, upload

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("shape_name,B1,B2,ctx,k,mode", [
    ("tiny_rec_full", 3, 1, 40, 3, "last_loop"),
    ("tiny_rec_full", 4, 2, 30, 2, "per_loop"),
    ("mid128", 8, 3, 1100, 2, "last_loop"),
])
def test_noalloc_decode_matches_decode_step(shape_name, B1, B2, ctx, k, mode):
    from looped_ngpt_transformer_fwd_amd import _lib as C
    from looped_ngpt_transformer_fwd_amd import model as M
    shape = {"tiny_rec_full": synth.TINY_REC_FULL, "mid128": synth.MID128}[shape_name]
    log(f"noalloc {shape_name} B {B1} then {B2} ctx {ctx} k {k} {mode}")
    W = synth.Weights(shape, ref.layer_kinds(shape), 0)
    gm = M.Model(shape, upload(W))
    d, V = shape.d_model, shape.vocab
    for B in (B1, B2):
        toks = torch.from_numpy(synth.tokens(11 + B, B, ctx + 1, V)).cuda()
        kva = gm.kv_cache(mode, k, B, ctx + 8)
        kvb = gm.kv_cache(mode, k, B, ctx + 8)
        gm.prefill(kva, toks[:, :ctx].contiguous(), k, logits=False)
        gm.prefill(kvb, toks[:, :ctx].contiguous(), k, logits=False)
        cur = toks[:, ctx].contiguous()
        outs = []
        for which, kv in (("decode_step", kva), ("noalloc", kvb)):
            lg = torch.empty(B, V, dtype=torch.float32, device="cuda")
            nx = torch.empty(B, dtype=torch.int32, device="cuda")
            hd = torch.empty(B, d, dtype=torch.float32, device="cuda")
            stt = torch.empty(k, B, d, dtype=torch.float32, device="cuda")
            if which == "decode_step":
                ws = gm.workspace(B, 1)
                st = C.dory_decode_step(gm.handle, kv.handle, _ptr(cur), B, k, kv.mode_code, _ptr(ws),
                                        ws.numel(), _ptr(lg), _ptr(nx), _ptr(hd), _ptr(stt), _stream())
            else:
                st = C.dory_decode_step_noalloc(gm.handle, kv.handle, _ptr(cur), B, k, kv.mode_code,
                                                _ptr(lg), _ptr(nx), _ptr(hd), _ptr(stt), _stream())
            C.check(st, which)
            outs.append((lg, nx, hd, stt))
        torch.cuda.synchronize()
        assert kva.length == kvb.length == ctx + 1
        for a, b, what in zip(outs[0], outs[1], ("logits", "next", "hidden", "states")):
            assert torch.equal(a, b), f"B={B}: {what} differs"
        # the next token of every sequence is the argmax of its logits
        np.testing.assert_array_equal(outs[1][1].cpu().numpy(),
                                      np.argmax(outs[1][0].cpu().numpy(), axis=1))


def test_noalloc_refuses_oversized_step():
    from looped_ngpt_transformer_fwd_amd import _lib as C
    from looped_ngpt_transformer_fwd_amd import model as M
    shape = synth.MID128
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda")
    names = synth.Weights(shape, ref.layer_kinds(shape)).names()
    gm = M.Model(shape, {n: dummy for n in names})
    # 256 MiB of scratch do not hold the split-K partials of 40,000 sequences
    B = 40000
    kv = gm.kv_cache("last_loop", 1, B, 8)
    st = C.dory_decode_step_noalloc(gm.handle, kv.handle, _ptr(dummy), B, 1, kv.mode_code, None, None,
                                    None, None, _stream())
    assert st == C.DORY_ERR_WORKSPACE
    assert kv.length == 0
