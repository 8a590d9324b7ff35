"""GPU parity of the MXFP8 weight path (dory_mxfp8_quantize,
dory_model_quantize_mxfp8): the quantizer's codes and scales bit-exact
against the oracle's (integer results), its bf16 dequantized copy equal to
the oracle's dequantization, and whole-model steps with the quantized
weights against the float64 oracle run on the dequantized weights (W8A16),
covering the small-M kernel that streams the codes (decode and short
prefills, up to 64 rows), the large-M path on the dequantized copy, both
cache policies and k = 1..4."""
import numpy as np
import pytest
import torch

import synth
from oracle import mx, ref
from tests.gpu_util import log, per_token_check, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from looped_ngpt_transformer_fwd_amd import model
    return model


def _bits_to_f64(b):
    return synth.f64_from_bf16_bits(np.asarray(b, dtype=np.uint16))


def _crafted_rows(cols, rng):
    """Rows whose blocks hit the rule's edge cases: zero blocks, a block
    maximum that saturates (1.99 * 2^e), exact E4M3 ties, values far below
    the block maximum (subnormal codes and zeros, signed), mixed magnitudes."""
    rows = []
    z = np.zeros(cols)
    rows.append(z.copy())
    r = z.copy(); r[::32] = 1.99; r[1::32] = -1.0; rows.append(r)
    pos = mx.e4m3_value(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2                         # exact ties at scale 2^0
    r = np.resize(np.concatenate([[256.0], mids[:31]]), cols) * 2.0 ** -8
    r[::32] = 1.0                                           # block maximum 1.0: scale 2^-8
    rows.append(r)
    r = np.resize([1.0, -3e-6, 2e-7, -0.0, 5e-5, -1e-9, 0.5, 7.5e-3], cols); rows.append(r)
    rows.append(rng.standard_normal(cols) * np.exp(rng.uniform(-12, 4, cols)))
    return np.array(rows)


@pytest.mark.parametrize("rows,cols", [(7, 32), (64, 2304), (300, 6144), (5, 96)])
def test_quantizer_bit_exact(M, rows, cols):
    log(f"mxfp8 quantizer {rows}x{cols}")
    rng = np.random.default_rng(rows * 131 + cols)
    w = rng.standard_normal((rows, cols)) / np.sqrt(cols)
    w = np.concatenate([w, _crafted_rows(cols, rng)])
    bits = synth.bf16_bits_from_f32(w.astype(np.float32))
    wt = torch.from_numpy(bits.view(np.int16)).cuda()
    codes, scales, deq = M.mxfp8_quantize(wt)
    torch.cuda.synchronize()
    want_c, want_s = mx.quantize(_bits_to_f64(bits))
    np.testing.assert_array_equal(scales.cpu().numpy(), want_s)
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)
    got_deq = deq.float().cpu().numpy().astype(np.float64)
    want_deq = mx.dequantize(want_c, want_s)
    np.testing.assert_array_equal(got_deq, want_deq)
    assert np.array_equal(np.signbit(got_deq), np.signbit(want_deq))


def _run(M, shape, B, T, n_dec, k, mode, seed, chunks=None):
    log(f"mxfp8 model d={shape.d_model} B={B} T={T} k={k} {mode}")
    W = synth.Weights(shape, ref.layer_kinds(shape), seed)
    gm = M.Model(shape, upload(W))
    gm.quantize_mxfp8()
    om = ref.OracleModel(shape, mx.quantized_weight_fn(W.f64))
    L = T + n_dec
    toks = synth.tokens(seed + 1, B, L, shape.vocab)
    kv = gm.kv_cache(mode, k, B, L)
    oc = ref.Cache(shape, mode, B)
    want = "last" if shape.has_lm_head else None
    for a, b in chunks or [(0, T)]:
        out = gm.prefill(kv, torch.from_numpy(toks[:, a:b].copy()).cuda(), k, logits=bool(want),
                         hidden=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, a:b], k, logits=want)
        per_token_check(out["hidden"].cpu().numpy(), o["hidden"], f"prefill [{a},{b}) hidden")
        if want:
            per_token_check(out["logits"].cpu().numpy(), o["logits"], f"prefill [{a},{b}) logits")
    for t in range(T, L):
        out = gm.decode_step(kv, torch.from_numpy(toks[:, t].copy()).cuda(), k,
                             logits=bool(want), next_token=bool(want), hidden=True)
        torch.cuda.synchronize()
        o = om.step(oc, toks[:, t:t + 1], k, logits=want)
        per_token_check(out["hidden"].cpu().numpy(), o["hidden"], f"decode {t} hidden")
        if want:
            lg = out["logits"].cpu().numpy()
            per_token_check(lg, o["logits"], f"decode {t} logits")
            np.testing.assert_array_equal(out["next"].cpu().numpy(),
                                          np.argmax(lg, axis=1).astype(np.int32))
    return gm


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_tiny_model_mxfp8(M, k, mode):
    # B x T = 48 rows: the prefill also streams the codes
    _run(M, synth.TINY_REC_FULL, 2, 24, 3, k, mode, seed=11)


def test_tiny_model_mxfp8_64_rows(M):
    # 64 sequences: decode at the small-M kernel's largest row count
    _run(M, synth.TINY_REC_FULL, 64, 5, 2, 3, "last_loop", seed=12)


def test_mid128_mxfp8_large_m_prefill_then_decode(M):
    # 2 x 600 rows: the prefill takes the large-M GEMM (with the fused q/k/v
    # epilogue) on the dequantized copy; decode streams the codes
    _run(M, synth.MID128, 2, 600, 2, 2, "last_loop", seed=13, chunks=[(0, 600)])


def test_full_width_pair_mxfp8(M):
    _run(M, synth.PAIR, 2, 40, 2, 2, "per_loop", seed=14)


def test_switch_back_to_bf16_matches_bf16_model(M):
    shape = synth.TINY_REC_FULL
    W = synth.Weights(shape, ref.layer_kinds(shape), 15)
    gm = M.Model(shape, upload(W))
    toks = torch.from_numpy(synth.tokens(16, 2, 12, shape.vocab)).cuda()

    def run():
        kv = gm.kv_cache("last_loop", 2, 2, 12)
        return gm.prefill(kv, toks, 2, hidden=True)["hidden"].cpu().numpy()
    ref_bf16 = run()
    gm.quantize_mxfp8()
    q = run()
    gm.use_mxfp8(False)
    back = run()
    np.testing.assert_array_equal(back, ref_bf16)
    assert not np.array_equal(q, ref_bf16)
