"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every declared symbol, the schedule and byte formulas agree with the
oracle, and every validation path returns its status without touching the
device (fake device pointers are never dereferenced on the host)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import synth
from looped_ngpt_transformer_fwd_amd import _lib as C
from looped_ngpt_transformer_fwd_amd import model as M
from oracle import ref

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dory.h")

# These checks hand fake device addresses to the compute calls and rely on the
# host refusing them; with a visible device a regressed check would enqueue
# kernels on those addresses, so the module runs on hosts without a GPU only.
# (Counting devices does not initialise the runtime.)
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="host-validation checks with fake device pointers run "
                                       "on GPU-less hosts only")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dory_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = C.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
        assert n in C.SIGNATURES, n


@pytest.mark.parametrize("shape", [synth.FULL, synth.TINY, synth.TINY_REC_FULL, synth.PAIR])
def test_schedule_matches_oracle(shape):
    assert M.schedule(shape) == ref.layer_kinds(shape)


def test_kv_bytes_matches_oracle_closed_form():
    """The cache size is the closed form with sliding-window rings of
    W + DORY_KV_ROLLBACK tokens (lengths and windows multiples of 8, so the
    runtime's rows equal the formula's tokens)."""
    ex = C.DORY_KV_ROLLBACK
    for sh in (synth.TINY, synth.TINY_REC_FULL):
        for mode in ("last_loop", "per_loop"):
            for k in (1, 2, 4):
                for L in (64, 200):
                    assert M.kv_bytes(sh, mode, k, 2, L) == ref.kv_bytes(sh, mode, k, 2, L, extra=ex)
    for mode in ("last_loop", "per_loop"):
        for k in (1, 2, 4):
            assert M.kv_bytes(synth.FULL, mode, k, 64, 33024) == \
                ref.kv_bytes(synth.FULL, mode, k, 64, 33024, extra=ex)
    # the slack is small next to the window at the full shape
    assert ref.kv_bytes(synth.FULL, "last_loop", 1, 64, 33024, extra=ex) < \
        1.01 * ref.kv_bytes(synth.FULL, "last_loop", 1, 64, 33024)


def test_kv_bytes_constant_in_k_for_last_loop():
    v = [M.kv_bytes(synth.FULL, "last_loop", k, 4, 8192) for k in (1, 2, 3, 4, 8)]
    assert len(set(v)) == 1
    p = [M.kv_bytes(synth.FULL, "per_loop", k, 4, 8192) for k in (1, 2, 3, 4)]
    assert np.all(np.diff(p) == p[1] - p[0]) and p[1] > p[0]


def test_workspace_bytes_monotone():
    a = M.workspace_bytes(synth.TINY, 2, 16)
    b = M.workspace_bytes(synth.TINY, 2, 64)
    assert 0 < a < b


def _fake_tensor_map(shape):
    """Fake device addresses: the validation paths never dereference them."""
    kinds = ref.layer_kinds(shape)
    names = synth.Weights(shape, kinds).names()

    class Fake:
        def __init__(self, addr):
            self.addr = addr

        def data_ptr(self):
            return self.addr
    return {n: Fake(0x10000 + 0x1000 * i) for i, n in enumerate(names)}


class _FakeT:
    def __init__(self, addr, n=0):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n


def _model_and_kv(shape=synth.TINY, mode="last_loop", k_max=4, batch=2, max_seq=64):
    m = M.Model(shape, _fake_tensor_map(shape))
    kvb = M.kv_bytes(shape, mode, k_max, batch, max_seq)
    h = ctypes.c_void_p()
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), kvb, M.MODE_CODE[mode], k_max,
                           batch, max_seq, h), "bind")
    return m, h


def _prefill(m, kv, B=2, T=8, k=1, mode=C.DORY_CACHE_LAST_LOOP, ws_bytes=None, tokens=0x500000,
             ws=0x700000, logits=None):
    if ws_bytes is None:
        ws_bytes = M.workspace_bytes(m.shape, B, T)
    return C.dory_prefill(m.handle, kv, ctypes.c_void_p(tokens) if tokens else None, B, T, k, mode,
                          ctypes.c_void_p(ws) if ws else None, ws_bytes, logits, None, None, None,
                          None)


def test_validation_errors_enqueue_nothing():
    m, kv = _model_and_kv()
    assert _prefill(m, kv, k=0) == C.DORY_ERR_ARG
    assert _prefill(m, kv, T=0) == C.DORY_ERR_ARG
    assert _prefill(m, kv, B=0) == C.DORY_ERR_ARG
    assert _prefill(m, kv, tokens=0) == C.DORY_ERR_ARG
    assert _prefill(m, kv, ws=0) == C.DORY_ERR_ARG
    assert _prefill(m, kv, mode=C.DORY_CACHE_PER_LOOP) == C.DORY_ERR_MODE
    assert _prefill(m, kv, B=3) == C.DORY_ERR_CAPACITY
    assert _prefill(m, kv, T=65) == C.DORY_ERR_CAPACITY
    assert _prefill(m, kv, ws_bytes=16) == C.DORY_ERR_WORKSPACE
    assert "workspace" in C.dory_last_error()
    assert C.dory_kv_length(kv) == 0
    C.dory_kv_destroy(kv)


def _prefill_rows(m, kv, k_rows, B=2, T=8, mode=C.DORY_CACHE_LAST_LOOP, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = M.workspace_bytes(m.shape, B, T)
    rows = (ctypes.c_int32 * len(k_rows))(*k_rows) if k_rows is not None else None
    return C.dory_prefill_rows(m.handle, kv, ctypes.c_void_p(0x500000), B, T, rows, mode,
                               ctypes.c_void_p(0x700000), ws_bytes, None, None, None, None, None)


def test_mixed_loop_counts_validated_before_enqueue():
    """Per-sequence loop counts: NULL or a count below 1 is an argument error,
    a per-loop cache is a mode error (each sequence's cache comes from its own
    last loop), and every rejection leaves the cache length unchanged."""
    m, kv = _model_and_kv()
    assert _prefill_rows(m, kv, None) == C.DORY_ERR_ARG
    assert _prefill_rows(m, kv, [1, 0]) == C.DORY_ERR_ARG
    assert _prefill_rows(m, kv, [2, 3], ws_bytes=16) == C.DORY_ERR_WORKSPACE
    assert _prefill_rows(m, kv, [2, 3], mode=C.DORY_CACHE_PER_LOOP) == C.DORY_ERR_MODE
    assert C.dory_kv_length(kv) == 0
    C.dory_kv_destroy(kv)
    m2, kv2 = _model_and_kv(mode="per_loop")
    assert _prefill_rows(m2, kv2, [1, 2], mode=C.DORY_CACHE_PER_LOOP) == C.DORY_ERR_MODE
    C.dory_kv_destroy(kv2)


def test_per_loop_k_above_k_max_rejected():
    m, kv = _model_and_kv(mode="per_loop", k_max=2)
    assert _prefill(m, kv, k=3, mode=C.DORY_CACHE_PER_LOOP) == C.DORY_ERR_MODE
    assert C.dory_kv_length(kv) == 0
    C.dory_kv_destroy(kv)


def test_bind_rejects_small_buffer_and_bad_mode():
    m = M.Model(synth.TINY, _fake_tensor_map(synth.TINY))
    h = ctypes.c_void_p()
    n = M.kv_bytes(synth.TINY, "last_loop", 1, 2, 64)
    assert C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), n - 1, 0, 1, 2, 64, h) == \
        C.DORY_ERR_CAPACITY
    assert C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), n, 7, 1, 2, 64, h) == C.DORY_ERR_MODE
    # the attention kernels take positions in 31 bits (at most 2^24) and
    # address a slab of rows x head_dim x 2 bytes with 32-bit offsets
    big = 1 << 24
    assert M.kv_bytes(synth.TINY, "last_loop", 1, 1, big) > 0
    assert M.kv_bytes(synth.TINY, "last_loop", 1, 1, big + 1) == 0
    assert C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), 1 << 40, 0, 1, 1, big + 1, h) == \
        C.DORY_ERR_ARG


def test_bind_refuses_a_slab_of_2_pow_32_bytes():
    """At head_dim 128 a full-attention slab of 2^24 rows is exactly 2^32
    bytes, which 32-bit offsets cannot span: binding it is refused before
    anything is enqueued, and 2^24 - 8 rows (the last multiple of 8 below)
    are accepted."""
    m = M.Model(synth.PAIR, _fake_tensor_map(synth.PAIR))
    h = ctypes.c_void_p()
    big = 1 << 24
    assert M.kv_bytes(synth.PAIR, "last_loop", 1, 1, big) == 0
    assert M.kv_bytes(synth.PAIR, "last_loop", 1, 1, big - 7) == 0   # rounds up to 2^24 rows
    n = M.kv_bytes(synth.PAIR, "last_loop", 1, 1, big - 8)
    assert n == ref.kv_bytes(synth.PAIR, "last_loop", 1, 1, big - 8, extra=C.DORY_KV_ROLLBACK)
    assert C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), 1 << 40, 0, 1, 1, big, h) == \
        C.DORY_ERR_ARG
    assert "2^32" in C.dory_last_error()
    assert not h.value
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), n, 0, 1, 1, big - 8, h), "bind")
    C.dory_kv_destroy(h)


def test_model_create_rejects_bad_configs():
    bad = [
        dict(n_q_heads=3),           # not a multiple of n_kv
        dict(head_dim=48),           # no kernel
        dict(d_model=100),           # not a multiple of 64
        dict(window=0),
    ]
    for kw in bad:
        import dataclasses
        sh = dataclasses.replace(synth.TINY, **kw)
        with pytest.raises(C.DoryError):
            M.Model(sh, _fake_tensor_map(synth.TINY))


def test_model_create_rejects_missing_weights():
    t = _fake_tensor_map(synth.TINY)

    class Null:
        def data_ptr(self):
            return 0
    t["sub1.w_down"] = Null()
    with pytest.raises(C.DoryError) as e:
        M.Model(synth.TINY, t)
    assert e.value.status == C.DORY_ERR_ARG


def test_no_lm_head_rejects_logits_request():
    m = M.Model(synth.PAIR, _fake_tensor_map(synth.PAIR))
    kvb = M.kv_bytes(synth.PAIR, "last_loop", 1, 1, 64)
    h = ctypes.c_void_p()
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), kvb, 0, 1, 1, 64, h), "bind")
    st = C.dory_prefill(m.handle, h, ctypes.c_void_p(0x500000), 1, 8, 1, 0, ctypes.c_void_p(0x700000),
                        M.workspace_bytes(synth.PAIR, 1, 8), ctypes.c_void_p(0x800000), None, None,
                        None, None)
    assert st == C.DORY_ERR_ARG


def test_status_strings():
    for s in range(8):
        assert C.dory_status_string(s)


def _mx_region(rows, cols):
    a = lambda x: (x + 255) // 256 * 256
    n = rows * cols
    return a(n) + a(n // 32) + a(2 * n)


@pytest.mark.parametrize("shape", [synth.TINY, synth.MID128, synth.FULL])
def test_mxfp8_bytes_closed_form(shape):
    # per projection matrix: E4M3 codes (1 B per weight), scale codes (1 B per
    # 32 weights) and the bf16 dequantized copy, each padded to 256 bytes
    want = 0
    for kind in ref.layer_kinds(shape):
        if kind == "mlp":
            want += _mx_region(2 * shape.d_ff, shape.d_model) + _mx_region(shape.d_model, shape.d_ff)
        else:
            nqkvg = 2 * shape.d_q + 2 * shape.d_kv
            want += _mx_region(nqkvg, shape.d_model) + _mx_region(shape.d_model, shape.d_q)
    assert M.mxfp8_bytes(shape) == want


def test_mxfp8_argument_validation_enqueues_nothing():
    m = M.Model(synth.TINY, _fake_tensor_map(synth.TINY))
    P = ctypes.c_void_p
    assert C.dory_mxfp8_quantize(P(0x10000), 4, 48, P(0x20000), P(0x30000), None, None) == \
        C.DORY_ERR_ARG                                    # cols not a multiple of 32
    assert C.dory_mxfp8_quantize(P(0x10008), 4, 64, P(0x20000), P(0x30000), None, None) == \
        C.DORY_ERR_ARG                                    # misaligned matrix
    assert C.dory_mxfp8_quantize(None, 4, 64, P(0x20000), P(0x30000), None, None) == C.DORY_ERR_ARG
    assert C.dory_model_use_mxfp8(m.handle, 1) == C.DORY_ERR_ARG   # nothing quantized yet
    assert C.dory_model_use_mxfp8(m.handle, 0) == C.DORY_OK
    n = M.mxfp8_bytes(synth.TINY)
    assert C.dory_model_quantize_mxfp8(m.handle, P(0x100000), n - 1, None) == C.DORY_ERR_CAPACITY
    assert C.dory_model_quantize_mxfp8(m.handle, P(0x100010), n, None) == C.DORY_ERR_ARG
    assert C.dory_model_use_mxfp8(m.handle, 1) == C.DORY_ERR_ARG


def test_copy_prefix_validated_before_enqueue():
    """Prefix copy: every rejection happens on the host, before anything is
    enqueued, and leaves both caches' lengths as they were."""
    m, src = _model_and_kv(batch=1, max_seq=64)
    kvb = M.kv_bytes(synth.TINY, "last_loop", 4, 3, 32)
    dst = ctypes.c_void_p()
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0xA00000), kvb, C.DORY_CACHE_LAST_LOOP, 4, 3,
                           32, dst), "bind")
    C.check(C.dory_kv_set_length(src, 40), "set_length")
    assert C.dory_kv_copy_prefix(None, 0, dst, 0, 8, None) == C.DORY_ERR_ARG
    assert C.dory_kv_copy_prefix(src, 1, dst, 0, 8, None) == C.DORY_ERR_ARG     # src batch is 1
    assert C.dory_kv_copy_prefix(src, 0, dst, 3, 8, None) == C.DORY_ERR_ARG     # dst batch is 3
    assert C.dory_kv_copy_prefix(src, 0, dst, -1, 8, None) == C.DORY_ERR_ARG
    assert C.dory_kv_copy_prefix(src, 0, dst, 0, 0, None) == C.DORY_ERR_ARG
    assert C.dory_kv_copy_prefix(src, 0, dst, 0, 41, None) == C.DORY_ERR_ARG    # beyond src length
    assert C.dory_kv_copy_prefix(src, 0, dst, 0, 33, None) == C.DORY_ERR_CAPACITY
    C.check(C.dory_kv_set_length(dst, 5), "set_length")
    assert C.dory_kv_copy_prefix(src, 0, dst, 0, 8, None) == C.DORY_ERR_STATE   # dst length not 0 / n
    assert C.dory_kv_length(src) == 40 and C.dory_kv_length(dst) == 5
    m2, other = _model_and_kv(mode="per_loop", batch=1, max_seq=64)
    C.check(C.dory_kv_set_length(other, 40), "set_length")
    assert C.dory_kv_copy_prefix(other, 0, dst, 0, 8, None) == C.DORY_ERR_ARG   # another model
    kvp = M.kv_bytes(synth.TINY, "per_loop", 4, 3, 32)
    dst2 = ctypes.c_void_p()
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0xA00000), kvp, C.DORY_CACHE_PER_LOOP, 4, 3, 32,
                           dst2), "bind")
    assert C.dory_kv_copy_prefix(src, 0, dst2, 0, 8, None) == C.DORY_ERR_MODE   # policies differ
    for h in (src, dst, other, dst2):
        C.dory_kv_destroy(h)


def test_selfspec_validated_before_enqueue():
    """Self-speculative round: argument, mode, workspace and capacity errors
    are found on the host before anything is enqueued; the cache length and
    the accepted count are left as they were."""
    m = M.Model(synth.TINY, _fake_tensor_map(synth.TINY))
    h = ctypes.c_void_p()
    kvb = M.kv_bytes(synth.TINY, "per_loop", 2, 2, 16)
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), kvb, C.DORY_CACHE_PER_LOOP, 2, 2, 16, h),
            "bind")
    ws_bytes = M.workspace_bytes(synth.TINY, 2, 5)
    n = ctypes.c_int32(-1)

    def call(B=2, gamma=4, kd=1, kv_=2, mode=C.DORY_CACHE_PER_LOOP, wsb=ws_bytes, last=0x500000,
             handle=h):
        return C.dory_selfspec_step(m.handle, handle, ctypes.c_void_p(last) if last else None, B, gamma,
                                    kd, kv_, mode, ctypes.c_void_p(0x700000), wsb,
                                    ctypes.c_void_p(0x600000), ctypes.c_void_p(0x680000), n, None)
    assert call(gamma=0) == C.DORY_ERR_ARG
    assert call(kd=0) == C.DORY_ERR_ARG
    assert call(kd=3, kv_=2) == C.DORY_ERR_ARG                 # k_draft above k_verify
    assert call(last=0) == C.DORY_ERR_ARG
    assert call(B=1) == C.DORY_ERR_ARG                         # B must equal the bound batch
    assert call(kv_=3) == C.DORY_ERR_MODE                      # above k_max
    assert call(mode=C.DORY_CACHE_LAST_LOOP) == C.DORY_ERR_MODE
    assert call(wsb=16) == C.DORY_ERR_WORKSPACE
    C.check(C.dory_kv_set_length(h, 12), "set_length")
    assert call() == C.DORY_ERR_CAPACITY                       # 12 + 4 + 1 > 16
    assert C.dory_kv_length(h) == 12 and n.value == -1
    hl = ctypes.c_void_p()
    kvl = M.kv_bytes(synth.TINY, "last_loop", 2, 2, 16)
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), kvl, C.DORY_CACHE_LAST_LOOP, 2, 2, 16,
                           hl), "bind")
    assert call(mode=C.DORY_CACHE_LAST_LOOP, handle=hl) == C.DORY_ERR_MODE   # per-loop caches only
    for x in (h, hl):
        C.dory_kv_destroy(x)


def test_sampled_entries_validated_before_enqueue():
    """dory_sample, dory_speculative_accept and dory_selfspec_step_sampled
    reject bad arguments on the host, before anything is enqueued (the
    pointers below are never dereferenced)."""
    P = ctypes.c_void_p
    a, b, c, d, e, f = (P(0x100000 * i) for i in range(1, 7))
    assert C.dory_sample(None, 4, 10, 1.0, b, c, None) == C.DORY_ERR_ARG
    assert C.dory_sample(a, 0, 10, 1.0, b, c, None) == C.DORY_ERR_ARG
    assert C.dory_sample(a, 4, 0, 1.0, b, c, None) == C.DORY_ERR_ARG
    assert C.dory_sample(a, 4, 10, 0.0, b, c, None) == C.DORY_ERR_ARG
    assert C.dory_sample(a, 4, 10, float("nan"), b, c, None) == C.DORY_ERR_ARG
    acc = C.dory_speculative_accept
    assert acc(a, b, c, None, 2, 10, 3, 1.0, e, f, None) == C.DORY_ERR_ARG
    assert acc(a, b, c, d, 2, 10, 0, 1.0, e, f, None) == C.DORY_ERR_ARG
    assert acc(a, b, c, d, 2, 10, 1001, 1.0, e, f, None) == C.DORY_ERR_ARG
    assert acc(a, b, c, d, 0, 10, 3, 1.0, e, f, None) == C.DORY_ERR_ARG
    assert acc(a, b, c, d, 2, 10, 3, -1.0, e, f, None) == C.DORY_ERR_ARG

    m = M.Model(synth.TINY, _fake_tensor_map(synth.TINY))
    h = ctypes.c_void_p()
    kvb = M.kv_bytes(synth.TINY, "per_loop", 2, 2, 16)
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), kvb, C.DORY_CACHE_PER_LOOP, 2, 2, 16, h),
            "bind")
    ws_bytes = M.workspace_bytes(synth.TINY, 2, 5)
    n = ctypes.c_int32(-1)

    def call(B=2, gamma=4, kd=1, kv_=2, T=0.7, u=0x880000, wsb=ws_bytes, lbuf=0x800000):
        return C.dory_selfspec_step_sampled(m.handle, h, P(0x500000), B, gamma, kd, kv_,
                                            C.DORY_CACHE_PER_LOOP, T, P(u) if u else None, P(0x700000),
                                            wsb, P(0x600000), P(lbuf) if lbuf else None, P(0x680000),
                                            n, None)
    assert call(T=0.0) == C.DORY_ERR_ARG
    assert call(u=0) == C.DORY_ERR_ARG
    assert call(lbuf=0) == C.DORY_ERR_ARG
    assert call(gamma=0) == C.DORY_ERR_ARG
    assert call(kd=3) == C.DORY_ERR_ARG
    assert call(B=1) == C.DORY_ERR_ARG
    assert call(kv_=3) == C.DORY_ERR_MODE
    assert call(wsb=16) == C.DORY_ERR_WORKSPACE
    C.check(C.dory_kv_set_length(h, 12), "set_length")
    assert call() == C.DORY_ERR_CAPACITY
    assert C.dory_kv_length(h) == 12 and n.value == -1
    C.dory_kv_destroy(h)


def test_decode_context_limit_rejected_before_enqueue():
    """Decode attention covers at most 1,048,576 keys (2,048 splits of 512 at
    long contexts): a decode step at position 1,048,576 is refused on the
    host."""
    m = M.Model(synth.TINY, _fake_tensor_map(synth.TINY))
    h = ctypes.c_void_p()
    kvb = M.kv_bytes(synth.TINY, "last_loop", 1, 1, 1100000)
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), kvb, C.DORY_CACHE_LAST_LOOP, 1, 1,
                           1100000, h), "bind")
    C.check(C.dory_kv_set_length(h, 1048576), "set_length")
    ws_bytes = M.workspace_bytes(synth.TINY, 1, 1)
    assert C.dory_decode_step(m.handle, h, ctypes.c_void_p(0x500000), 1, 1, C.DORY_CACHE_LAST_LOOP,
                              ctypes.c_void_p(0x700000), ws_bytes, None, None, None, None,
                              None) == C.DORY_ERR_UNSUPPORTED
    assert C.dory_kv_length(h) == 1048576
    C.dory_kv_destroy(h)


def test_debug_probes_validated_before_enqueue():
    """The attention probes, the slot dump and greedy selection refuse bad
    arguments on the host (fake device pointers are never touched)."""
    m, kv = _model_and_kv(synth.TINY_REC_FULL, batch=1, max_seq=64)
    P = ctypes.c_void_p
    wsb = M.workspace_bytes(synth.TINY_REC_FULL, 1, 8)

    def mask(sub=0, loop=0, p0=0, T=8, ws=0x700000, wsn=wsb, out=0x800000):
        return C.dory_debug_mask(m.handle, kv, sub, loop, p0, T, P(ws) if ws else None, wsn,
                                 P(out) if out else None, None)

    def attn(sub=0, p0=0, T=8, q=0x510000):
        return C.dory_debug_attention(m.handle, kv, sub, 0, p0, T, P(q) if q else None, P(0x520000),
                                      P(0x530000), P(0x540000), P(0x550000), P(0x700000), wsb, None)
    assert mask(sub=1) == C.DORY_ERR_ARG          # an MLP sublayer
    assert mask(sub=99) == C.DORY_ERR_ARG
    assert mask(T=0) == C.DORY_ERR_ARG
    assert mask(p0=-1) == C.DORY_ERR_ARG
    assert mask(p0=60, T=8) == C.DORY_ERR_CAPACITY
    assert mask(wsn=16) == C.DORY_ERR_WORKSPACE
    assert mask(ws=0) == C.DORY_ERR_ARG
    assert mask(out=0) == C.DORY_ERR_ARG
    assert attn(q=0) == C.DORY_ERR_ARG
    assert attn(sub=3) == C.DORY_ERR_ARG
    rows = P(0x600000)
    assert C.dory_debug_kv_slots(kv, 1, 0, 4, rows, None) == C.DORY_ERR_ARG
    assert C.dory_debug_kv_slots(kv, 0, 60, 8, rows, None) == C.DORY_ERR_ARG
    assert C.dory_debug_kv_slots(kv, 0, 0, 0, rows, None) == C.DORY_ERR_ARG
    assert C.dory_debug_kv_slots(kv, 0, 0, 4, None, None) == C.DORY_ERR_ARG
    assert C.dory_greedy(P(0x600000), 0, 10, P(0x610000), None) == C.DORY_ERR_ARG
    assert C.dory_greedy(P(0x600000), 2, 0, P(0x610000), None) == C.DORY_ERR_ARG
    assert C.dory_greedy(None, 2, 10, P(0x610000), None) == C.DORY_ERR_ARG
    assert C.dory_kv_length(kv) == 0
    C.dory_kv_destroy(kv)


def test_noalloc_decode_size_checked_before_any_hip_call():
    """The allocation-free decode step refuses a step whose exact scratch
    exceeds the static array (here 1,024 sequences at full width) before any
    HIP call, and validates its arguments like dory_decode_step."""
    m = M.Model(synth.FULL, _fake_tensor_map(synth.FULL))
    h = ctypes.c_void_p()
    kvb = M.kv_bytes(synth.FULL, "last_loop", 1, 1024, 64)
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), kvb, C.DORY_CACHE_LAST_LOOP, 1, 1024,
                           64, h), "bind")
    st = C.dory_decode_step_noalloc(m.handle, h, ctypes.c_void_p(0x500000), 1024, 1,
                                    C.DORY_CACHE_LAST_LOOP, None, None, None, None, None)
    assert st == C.DORY_ERR_WORKSPACE
    assert "static array" in C.dory_last_error()
    assert C.dory_decode_step_noalloc(None, h, ctypes.c_void_p(0x500000), 1024, 1, 0, None, None,
                                      None, None, None) == C.DORY_ERR_ARG
    assert C.dory_decode_step_noalloc(m.handle, h, ctypes.c_void_p(0x500000), 0, 1, 0, None, None,
                                      None, None, None) == C.DORY_ERR_ARG
    assert C.dory_kv_length(h) == 0
    C.dory_kv_destroy(h)


def test_f32_build_sizes_and_refusals():
    """fp32 debug build: the cache holds 4-byte entries (the closed form with
    4-byte elements), the workspace grows, and the bf16-only features refuse."""
    for sh, shf in ((synth.TINY, synth.TINY_F32), (synth.TINY_REC_FULL, synth.TINY_REC_FULL_F32)):
        for mode in ("last_loop", "per_loop"):
            for k in (1, 2, 4):
                assert M.kv_bytes(shf, mode, k, 2, 64) == ref.kv_bytes(sh, mode, k, 2, 64, elem_bytes=4,
                                                                             extra=C.DORY_KV_ROLLBACK)
                assert M.kv_bytes(shf, mode, k, 2, 64) == 2 * M.kv_bytes(sh, mode, k, 2, 64)
        assert M.workspace_bytes(shf, 2, 16) > M.workspace_bytes(sh, 2, 16)
    assert M.mxfp8_bytes(synth.TINY_F32) == 0
    m = M.Model(synth.TINY_F32, _fake_tensor_map(synth.TINY_F32))
    assert C.dory_model_quantize_mxfp8(m.handle, ctypes.c_void_p(0x1000000), 1 << 30, None) == \
        C.DORY_ERR_UNSUPPORTED
    cfg = M.make_config(synth.TINY)
    cfg.precision = 7
    assert C.dory_kv_bytes(cfg, 0, 1, 1, 64) == 0


def test_rollback_depth_bounded_on_wrapping_rings():
    """A sliding-window ring holds W + DORY_KV_ROLLBACK positions: where it
    is shorter than max_seq, shortening below (longest length written) -
    DORY_KV_ROLLBACK is refused and the length stays; a cache whose rings
    never wrap can be shortened to any length; reset clears the record."""
    m = M.Model(synth.TINY, _fake_tensor_map(synth.TINY))
    R = C.DORY_KV_ROLLBACK
    h = ctypes.c_void_p()
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), M.kv_bytes(synth.TINY, "last_loop", 1, 2, 400),
                           C.DORY_CACHE_LAST_LOOP, 1, 2, 400, h), "bind")
    C.check(C.dory_kv_set_length(h, 300), "extend")
    assert C.dory_kv_set_length(h, 300 - R - 1) == C.DORY_ERR_ARG
    assert C.dory_kv_length(h) == 300
    C.check(C.dory_kv_set_length(h, 300 - R), "shorten by DORY_KV_ROLLBACK")
    C.check(C.dory_kv_set_length(h, 290), "lengthen again")
    # measured from the longest length written (300), not the current one
    assert C.dory_kv_set_length(h, 300 - R - 1) == C.DORY_ERR_ARG
    C.check(C.dory_kv_reset(h), "reset")
    C.check(C.dory_kv_set_length(h, 100), "extend")
    C.check(C.dory_kv_set_length(h, 100 - R), "shorten")
    C.dory_kv_destroy(h)
    # rings of W + DORY_KV_ROLLBACK rows never wrap below that length
    n = synth.TINY.window + R
    C.check(C.dory_kv_bind(m.handle, ctypes.c_void_p(0x900000), M.kv_bytes(synth.TINY, "last_loop", 1, 2, n),
                           C.DORY_CACHE_LAST_LOOP, 1, 2, n, h), "bind")
    C.check(C.dory_kv_set_length(h, n), "extend")
    C.check(C.dory_kv_set_length(h, 0), "shorten to 0")
    C.dory_kv_destroy(h)
