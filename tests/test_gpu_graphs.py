"""Decode steps replayed from captured HIP graphs (dory_model_set_decode_graphs)
against the same steps launched kernel by kernel, through the C ABI.

The graph path runs the same kernels with the step position read from
device memory (written by the graph's first node) and the decode attention
launched for the highest position the graph serves (its extra splits exit),
so every output must be bit-identical to the direct path, at every replay:
several replays in a row with other work on the stream in between (a
prefill of another cache), new output buffers (a second capture), both cache
policies, and a context that crosses 65,536 cached keys (where the decode
attention's split size changes and a second graph is captured). The direct
path itself is checked against the oracle by the other decode tests."""
import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log, upload

pytestmark = pytest.mark.gpu


def _models(shape):
    from looped_ngpt_transformer_fwd_amd import model as M
    W = synth.Weights(shape, ref.layer_kinds(shape), 0)
    dev = upload(W)
    g = M.Model(shape, dev)            # graphs on (the default)
    e = M.Model(shape, dev)
    e.set_decode_graphs(False)
    return g, e


def _same(a, b, what):
    for key in ("logits", "next", "hidden", "states"):
        assert torch.equal(a[key], b[key]), f"{what}: {key} differs between graph and direct"


@pytest.mark.parametrize("mode,k", [("last_loop", 1), ("last_loop", 3), ("per_loop", 2)])
def test_graph_replays_equal_direct_launches(mode, k):
    shape = synth.TINY_REC_FULL
    log(f"graphs tiny {mode} k={k}")
    gm, em = _models(shape)
    B, P, S = 2, 20, 12
    toks = torch.from_numpy(synth.tokens(3, B, P + S + 1, shape.vocab)).cuda()
    kvg = gm.kv_cache(mode, 4, B, 64)
    kve = em.kv_cache(mode, 4, B, 64)
    gm.prefill(kvg, toks[:, :P].contiguous(), k, logits=False)
    em.prefill(kve, toks[:, :P].contiguous(), k, logits=False)
    other = em.kv_cache(mode, 4, B, 64)
    ws_g = gm.workspace(B, 1)
    ws_e = em.workspace(B, 1)
    d, V = shape.d_model, shape.vocab

    def bufs():
        return {"logits": torch.empty(B, V, dtype=torch.float32, device="cuda"),
                "next": torch.empty(B, dtype=torch.int32, device="cuda"),
                "hidden": torch.empty(B, 1, d, dtype=torch.float32, device="cuda"),
                "states": torch.empty(k, B, 1, d, dtype=torch.float32, device="cuda")}
    from looped_ngpt_transformer_fwd_amd import _lib as C
    from looped_ngpt_transformer_fwd_amd.model import _ptr, _stream
    outs_g, outs_e = bufs(), bufs()
    tok_g = torch.empty(B, dtype=torch.int32, device="cuda")
    tok_e = torch.empty(B, dtype=torch.int32, device="cuda")
    for step in range(S):
        if step == 7:
            outs_g = bufs()                # new buffers: a second capture
        tok_g.copy_(toks[:, P + step])
        tok_e.copy_(toks[:, P + step])
        for m, kv, ws, o, t in ((gm, kvg, ws_g, outs_g, tok_g), (em, kve, ws_e, outs_e, tok_e)):
            C.check(C.dory_decode_step(m.handle, kv.handle, _ptr(t), B, k, kv.mode_code, _ptr(ws),
                                       ws.numel(), _ptr(o["logits"]), _ptr(o["next"]),
                                       _ptr(o["hidden"]), _ptr(o["states"]), _stream()),
                    "decode")
        # other work on the stream between replays
        if step % 3 == 1:
            other.reset()
            em.prefill(other, toks[:, :9].contiguous(), k, logits=False)
        torch.cuda.synchronize()
        _same(outs_g, outs_e, f"step {step}")
        np.testing.assert_array_equal(outs_g["next"].cpu().numpy(),
                                      np.argmax(outs_g["logits"].cpu().numpy(), axis=1))
    assert kvg.length == kve.length == P + S


def test_graph_across_split_size_change():
    """Decode from 65,530 to 65,542 cached keys (full-attention splits of 256
    keys, then 512): both graphs equal the direct launches bit for bit. The
    cached entries are the same random values in both caches."""
    shape = synth.TINY_REC_FULL
    log("graphs across 65,536 keys")
    gm, em = _models(shape)
    B, L0, k = 1, 65530, 2
    kvg = gm.kv_cache("last_loop", 2, B, 65600)
    kve = em.kv_cache("last_loop", 2, B, 65600)
    g = torch.Generator(device="cuda").manual_seed(5)
    fill = (torch.randn(kvg.buffer.numel() // 2, generator=g, device="cuda") * 0.2).to(torch.bfloat16)
    kvg.buffer.copy_(fill.view(torch.uint8))
    kve.buffer.copy_(fill.view(torch.uint8))
    kvg.set_length(L0)
    kve.set_length(L0)
    toks = torch.from_numpy(synth.tokens(9, B, 12, shape.vocab)).cuda()
    for step in range(12):
        t = toks[:, step].contiguous()
        a = gm.decode_step(kvg, t, k, hidden=True, states=True)
        b = em.decode_step(kve, t, k, hidden=True, states=True)
        torch.cuda.synchronize()
        _same(a, b, f"position {L0 + step}")
    assert kvg.length == L0 + 12


def test_graph_list_bounded_with_new_buffers_each_step():
    """Forty decode steps, each with new output buffers (a new capture every
    step, more than the 32 graphs a model keeps, so the oldest are dropped
    while decoding continues): every step equals the direct launches."""
    shape = synth.TINY_REC_FULL
    log("graphs: new buffers every step")
    gm, em = _models(shape)
    B, P, S, k = 2, 8, 40, 2
    toks = torch.from_numpy(synth.tokens(8, B, P + S, shape.vocab)).cuda()
    kvg = gm.kv_cache("last_loop", k, B, 64)
    kve = em.kv_cache("last_loop", k, B, 64)
    gm.prefill(kvg, toks[:, :P].contiguous(), k, logits=False)
    em.prefill(kve, toks[:, :P].contiguous(), k, logits=False)
    for step in range(S):
        t = toks[:, P + step].contiguous()
        a = gm.decode_step(kvg, t, k, hidden=True, states=True)
        b = em.decode_step(kve, t, k, hidden=True, states=True)
        torch.cuda.synchronize()
        _same(a, b, f"step {step}")
    assert kvg.length == P + S
