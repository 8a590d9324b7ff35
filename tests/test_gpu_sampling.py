"""GPU tests of sampled decoding: dory_sample (inversion from
softmax(logits / T)), dory_speculative_accept (the rejection rule of
self-speculative decoding) and dory_selfspec_step_sampled, through the C ABI.

The uniforms are inputs, so every decision is compared with the float64
oracle on the same logits and uniforms: a token or an accept/reject decision
must agree wherever the oracle's decision is clear of fp32 rounding (the
uniform more than MARGIN away from the cumulative boundary or from p/q); at
a near-boundary case the GPU's choice must still be one of the two
neighbours. Beyond element parity, a 100,000-trial run checks that the rule's
output follows the verifier's distribution (binomial 5-sigma per token)."""
import copy

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log, oracle_model, per_token_check, upload

pytestmark = pytest.mark.gpu

MARGIN = 2e-5


@pytest.fixture(scope="module")
def M():
    from looped_ngpt_transformer_fwd_amd import model
    return model


def _check_inversion(got, probs, u, what):
    """got [R] against inversion of probs [R, V] (float64) at u [R]."""
    probs = np.asarray(probs, dtype=np.float64)
    probs = probs / probs.sum(axis=-1, keepdims=True)
    c = np.cumsum(probs, axis=-1)
    want = ref.sample_inverse_cdf(probs, u)
    for r in range(len(got)):
        g, w = int(got[r]), int(want[r])
        assert 0 <= g < probs.shape[1], f"{what} row {r}: index {g} out of range"
        assert probs[r, g] > 0, f"{what} row {r}: token {g} has zero probability"
        if g == w:
            continue
        # only a rounding-close call may differ: the boundary between the two
        # choices lies within MARGIN of u
        lo, hi = min(g, w), max(g, w)
        assert abs(c[r, lo] - u[r]) < MARGIN or abs(c[r, hi - 1] - u[r]) < MARGIN, \
            f"{what} row {r}: GPU {g}, oracle {w}, u {u[r]:.7f}"
    return want


@pytest.mark.parametrize("V,T", [(37, 1.0), (1000, 0.7), (4099, 1.3), (151936, 1.0)])
def test_sample_matches_oracle_inversion(M, V, T):
    log(f"sample V={V} T={T}")
    rng = np.random.default_rng(V)
    R = 64 if V < 100000 else 8
    logits = (rng.standard_normal((R, V)) * 3).astype(np.float32)
    u = rng.random(R).astype(np.float32)
    u[0], u[1] = 0.0, np.float32(1 - 2 ** -24)          # both ends of [0, 1)
    got = M.sample(torch.from_numpy(logits).cuda(), T, torch.from_numpy(u).cuda()).cpu().numpy()
    _check_inversion(got, ref.softmax_t(logits.astype(np.float64), T), u.astype(np.float64), "sample")


def test_sample_never_picks_zero_probability(M):
    """-inf logits have probability zero: never chosen at any u, u = 0 gives
    the first allowed token and u -> 1 the last."""
    log("sample with -inf logits")
    rng = np.random.default_rng(3)
    R, V = 48, 3000
    logits = rng.standard_normal((R, V)).astype(np.float32)
    allowed = rng.random((R, V)) < 0.05
    allowed[:, 7] = True
    logits[~allowed] = -np.inf
    u = rng.random(R).astype(np.float32)
    u[:16] = 0.0
    u[16:32] = np.float32(1 - 2 ** -24)
    got = M.sample(torch.from_numpy(logits).cuda(), 1.0, torch.from_numpy(u).cuda()).cpu().numpy()
    assert np.all(allowed[np.arange(R), got])
    first = np.argmax(allowed, axis=1)
    last = V - 1 - np.argmax(allowed[:, ::-1], axis=1)
    np.testing.assert_array_equal(got[:16], first[:16])
    np.testing.assert_array_equal(got[16:32], last[16:32])
    # a row with a single allowed token always picks it
    one = np.full((4, V), -np.inf, dtype=np.float32)
    one[np.arange(4), [0, 5, V - 1, 1234]] = 0.0
    got1 = M.sample(torch.from_numpy(one).cuda(), 0.5,
                    torch.tensor([0.0, 0.5, 0.999, 0.3], device="cuda")).cpu().numpy()
    np.testing.assert_array_equal(got1, [0, 5, V - 1, 1234])
    # a row without a finite logit has no distribution: token 0 (documented)
    none = np.full((2, V), -np.inf, dtype=np.float32)
    got2 = M.sample(torch.from_numpy(none).cuda(), 1.0, torch.tensor([0.0, 0.7], device="cuda")).cpu().numpy()
    np.testing.assert_array_equal(got2, [0, 0])


def _spec_inputs(rng, gamma, B, V, spread):
    dl = (rng.standard_normal((gamma, B, V)) * 2).astype(np.float32)
    vl = (dl[np.r_[0:gamma, gamma - 1]] + spread * rng.standard_normal((gamma + 1, B, V))).astype(np.float32)
    q = ref.softmax_t(dl.astype(np.float64), 1.0)
    ud = rng.random((gamma, B))
    drafts = ref.sample_inverse_cdf(q, ud).astype(np.int32)
    u = rng.random((gamma + 1, B)).astype(np.float32)
    return dl, vl, drafts, u


@pytest.mark.parametrize("gamma,B,V,T", [(1, 64, 37, 1.0), (3, 256, 1000, 0.8), (5, 32, 4099, 1.0)])
def test_speculative_accept_matches_oracle(M, gamma, B, V, T):
    log(f"accept gamma={gamma} B={B} V={V}")
    rng = np.random.default_rng(100 + gamma)
    dl, vl, drafts, u = _spec_inputs(rng, gamma, B, V, 0.7)
    u[0, :4] = 0.0                                          # always accepted
    n, out = M.speculative_accept(torch.from_numpy(dl).cuda(), torch.from_numpy(vl).cuda(),
                                  torch.from_numpy(drafts).cuda(), torch.from_numpy(u).cuda(), T)
    n, out = n.cpu().numpy(), out.cpu().numpy()
    dl64, vl64, u64 = dl.astype(np.float64), vl.astype(np.float64), u.astype(np.float64)
    on, onx = ref.speculative_sample(dl64, vl64, drafts, u64, T)
    q = ref.softmax_t(dl64, T)
    p = ref.softmax_t(vl64, T)
    assert np.all(n[:4] >= 1)
    checked = 0
    for b in range(B):
        # the accept decisions are compared up to the first close call
        j = 0
        close = False
        while j < gamma:
            x = drafts[j, b]
            ratio = p[j, b, x] / q[j, b, x]
            if abs(u64[j, b] - ratio) < MARGIN * max(1.0, ratio):
                close = True
                break
            if not u64[j, b] < ratio:
                break
            j += 1
        if close:
            continue
        assert n[b] == on[b] == j, f"seq {b}: GPU accepted {n[b]}, oracle {on[b]}"
        np.testing.assert_array_equal(out[:j, b], drafts[:j, b])
        assert np.all(out[j + 1:, b] == -1)
        w = np.maximum(p[j, b] - q[j, b], 0.0) if j < gamma else p[gamma, b]
        _check_inversion(out[j:j + 1, b], w[None], u64[gamma:gamma + 1, b], f"seq {b} next")
        checked += 1
    assert checked >= B * 0.9


def test_speculative_rule_preserves_verifier_distribution(M):
    """100,000 trials of one gamma = 2 round with fixed drafter and verifier
    distributions (V = 40), drafts sampled on the GPU with dory_sample: the
    first emitted token follows p_1, the second (when emitted) follows p_2,
    and draft 1 is accepted with probability sum_x min(p_1(x), q_1(x)), each
    within 5 binomial standard deviations."""
    log("speculative rule, 100k trials")
    rng = np.random.default_rng(77)
    gamma, V, N, T = 2, 40, 100000, 1.0
    base_d = (rng.standard_normal((gamma, V)) * 1.5).astype(np.float32)
    base_v = (rng.standard_normal((gamma + 1, V)) * 1.5).astype(np.float32)
    dl = torch.from_numpy(np.repeat(base_d[:, None], N, axis=1)).cuda().contiguous()
    vl = torch.from_numpy(np.repeat(base_v[:, None], N, axis=1)).cuda().contiguous()
    g = torch.Generator(device="cuda").manual_seed(5)
    ud = torch.rand(gamma, N, generator=g, device="cuda")
    drafts = torch.stack([M.sample(dl[j], T, ud[j]) for j in range(gamma)]).contiguous()
    ua = torch.rand(gamma + 1, N, generator=g, device="cuda")
    n, out = M.speculative_accept(dl, vl, drafts, ua, T)
    n, out = n.cpu().numpy(), out.cpu().numpy()
    q = ref.softmax_t(base_d.astype(np.float64), T)
    p = ref.softmax_t(base_v.astype(np.float64), T)
    # drafts follow q_1
    d0 = np.bincount(drafts[0].cpu().numpy(), minlength=V) / N
    assert np.all(np.abs(d0 - q[0]) <= 5 * np.sqrt(q[0] * (1 - q[0]) / N) + 1e-12)
    # first emitted token ~ p_1
    f0 = np.bincount(out[0], minlength=V) / N
    assert np.all(np.abs(f0 - p[0]) <= 5 * np.sqrt(p[0] * (1 - p[0]) / N) + 1e-12), \
        f"first token law off: max dev {np.max(np.abs(f0 - p[0])):.4g}"
    # second emitted token (sequences with n >= 1) ~ p_2
    sel = n >= 1
    N2 = int(sel.sum())
    f1 = np.bincount(out[1][sel], minlength=V) / N2
    assert np.all(np.abs(f1 - p[1]) <= 5 * np.sqrt(p[1] * (1 - p[1]) / N2) + 1e-12)
    acc = float(np.minimum(p[0], q[0]).sum())
    assert abs(sel.mean() - acc) <= 5 * np.sqrt(acc * (1 - acc) / N)
    # tokens the verifier rules out never appear
    assert np.all(out[0] >= 0) and np.all(out[1][sel] >= 0)


def test_selfspec_sampled_round_against_oracle(M):
    """Two sampled rounds on the tiny model (per-loop cache, k_draft 1,
    k_verify 4, gamma 3): the drafts' logits and the verification's logits
    equal the oracle's on the same tokens, each draft is the inversion of its
    own logits at its uniform, the accept decisions equal the oracle rule on
    the GPU's logits, and the cache kept the batch-minimum accepted prefix
    (the second round's verification, run on that cache, matches the
    oracle's)."""
    shape = synth.TINY_REC_FULL
    W = synth.Weights(shape, ref.layer_kinds(shape), 21)
    gm = M.Model(shape, upload(W))
    om = oracle_model(shape, W)
    B, k, kd, gamma, T = 3, 4, 1, 3, 0.8
    log("sampled selfspec rounds")
    prompt = synth.tokens(55, B, 10, shape.vocab)
    kv = gm.kv_cache("per_loop", k, B, 64)
    oc = ref.Cache(shape, "per_loop", B)
    last = gm.prefill(kv, torch.from_numpy(prompt).cuda(), k, logits=False, next_token=True)["next"]
    om.step(oc, prompt, k, logits="last")
    rng = np.random.default_rng(9)
    for rnd in range(2):
        L0 = kv.length
        u = rng.random((2 * gamma + 1, B)).astype(np.float32)
        n, out, lbuf, drafts = gm.selfspec_step_sampled(kv, last, gamma, kd, k, T, torch.from_numpy(u).cuda())
        torch.cuda.synchronize()
        out, lbuf, drafts = out.cpu().numpy(), lbuf.cpu().numpy(), drafts.cpu().numpy()
        lastn = last.cpu().numpy()
        # drafts: inversion of their own logits
        for j in range(gamma):
            _check_inversion(drafts[j], ref.softmax_t(lbuf[j].astype(np.float64), T),
                             u[j].astype(np.float64), f"round {rnd} draft {j}")
        # draft logits against the oracle at k_draft on the same tokens (the
        # per-loop cache's first k_draft loop slots hold the verifier's entries)
        od = copy.deepcopy(oc)
        od.k_used = None
        seq = np.concatenate([lastn[:, None], drafts.T], axis=1)
        for j in range(gamma):
            o = om.step(od, seq[:, j:j + 1], kd, logits="last")
            per_token_check(lbuf[j], o["logits"], f"round {rnd} draft logits {j}")
        # verification logits at k over last + drafts
        ov = copy.deepcopy(oc)
        o = om.step(ov, seq, k, logits="all")
        for j in range(gamma + 1):
            per_token_check(lbuf[gamma + j], o["logits"][:, j], f"round {rnd} verify logits {j}")
        on, onx = ref.speculative_sample(lbuf[:gamma].astype(np.float64), lbuf[gamma:].astype(np.float64),
                                         drafts, u[gamma:].astype(np.float64), T)
        nb = np.array([int(np.sum(out[:, b] >= 0)) - 1 for b in range(B)])
        for b in range(B):
            np.testing.assert_array_equal(out[:nb[b], b], drafts[:nb[b], b])
            if nb[b] != on[b]:
                # only a decision within rounding of u = p/q may differ
                j = min(nb[b], on[b])
                x = drafts[j, b]
                pq = ref.softmax_t(lbuf[gamma + j, b].astype(np.float64), T)[x] / \
                    ref.softmax_t(lbuf[j, b].astype(np.float64), T)[x]
                assert abs(u[j, b] - pq) < MARGIN * max(1.0, pq), f"round {rnd} seq {b}"
                continue
            j = nb[b]
            pv = ref.softmax_t(lbuf[gamma + j, b].astype(np.float64), T)
            w = np.maximum(pv - ref.softmax_t(lbuf[j, b].astype(np.float64), T), 0.0) if j < gamma else pv
            _check_inversion(out[j:j + 1, b], w[None], u[2 * gamma:, b].astype(np.float64),
                             f"round {rnd} seq {b} next")
        assert n == nb.min()
        assert kv.length == L0 + n + 1
        log(f"  round {rnd}: accepted {nb.tolist()}, kept {n}")
        # advance the oracle by the kept tokens: last, then drafts 1 .. n
        om.step(oc, seq[:, :n + 1], k, logits="last")
        last = torch.from_numpy(out[n].copy()).cuda()
