"""Bit-exact GPU checks of index and mask construction, read off the
production kernels (through the C ABI's debug probes, which run the same
attention launches as a step):

* the visibility every query head of the attention kernels applies, dumped by
  dory_debug_mask and compared with the oracle's mask (reading R3: key u is
  visible to the query at p iff u <= p and, for a sliding-window layer,
  p - u < W), together with the exact weight under equal scores
  (1 / number of visible keys, so a key counted twice also fails), for
  prefill and decode, sliding-window rings that have wrapped,
  chunks that start past 0 and do not start at a multiple of 8, several key
  tiles, and a full-attention decode past 65,536 keys (where the decode
  kernel's split size changes);
* window edges with real scores: for one query, the key just outside the
  window and the key just inside it get a large score and distinct one-hot
  values; the output must carry the inside key only (the keys are written
  into the cache slot by the test itself, in the documented layout);
* cache rows of positions, evaluated on the device by the function the
  cache-writing kernels use, equal position mod ring (sliding window) or the
  position (full attention);
* greedy selection on rows with repeated maxima: the lowest index wins.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    from looped_ngpt_transformer_fwd_amd import model as M
    return M


def _probe_model(M, shape):
    """A model whose weight pointers all name one small device buffer: the
    probes run attention only and read no weight."""
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda")
    names = synth.Weights(shape, ref.layer_kinds(shape)).names()
    return M.Model(shape, {n: dummy for n in names}), dummy


def _oracle_mask(p0, T, window):
    return ref.visible(np.arange(p0, p0 + T), np.arange(p0 + T), window)


MASK_CASES = [
    # shape, sublayer, p0, T, max_seq, batch
    ("tiny", 0, 0, 64, 64, 1),        # sliding window 16, one shot
    ("tiny", 0, 117, 29, 256, 2),     # ring of 80 rows wrapped, chunk start not a multiple of 8
    ("tiny", 4, 0, 64, 64, 1),        # full attention (recurrent full layer)
    ("tiny", 4, 100, 1, 128, 2),      # full-attention decode
    ("tiny", 0, 330, 1, 400, 1),      # sliding-window decode, ring wrapped 4 times
    ("pair", 0, 1500, 600, 2100, 1),  # window 1024, ring wrapped, 600-query chunk
    ("pair", 0, 0, 1100, 1100, 1),    # window 1024 inside one chunk (fresh keys only)
    ("pair", 2, 0, 1100, 1100, 1),    # causal over 18 key tiles
    ("pair", 2, 700, 333, 1040, 1),   # causal with a cached prefix, ragged chunk
    ("pair", 0, 3000, 1, 4096, 1),    # sliding-window decode, ring wrapped
    ("pair", 2, 70000, 1, 70016, 1),  # full-attention decode past 65,536 keys
]


@pytest.mark.parametrize("case", MASK_CASES, ids=[f"{c[0]}-sub{c[1]}-p{c[2]}-T{c[3]}-B{c[5]}"
                                                  for c in MASK_CASES])
def test_mask_from_kernels_bit_exact(M, case):
    name, sub, p0, T, max_seq, B = case
    shape = {"tiny": synth.TINY_REC_FULL, "pair": synth.PAIR}[name]
    log(f"mask {name} sublayer {sub} p0={p0} T={T} B={B}")
    m, _ = _probe_model(M, shape)
    kv = m.kv_cache("last_loop", 1, B, max_seq)
    got = M.debug_mask(kv, sub, p0, T).cpu().numpy().view(np.uint16)
    torch.cuda.synchronize()
    kind = ref.layer_kinds(shape)[sub]
    want = _oracle_mask(p0, T, shape.window if kind == ref.KIND_SWA else None)
    # equal scores: every visible key weighs 1 / (visible keys), rounded
    # to bf16 from the float32 quotient; a masked key weighs exactly 0
    cnt = want.sum(axis=1).astype(np.float32)
    wbits = synth.bf16_bits_from_f32(np.float32(1.0) / cnt)
    want_w = np.where(want, wbits[:, None], np.uint16(0))
    assert got.shape == (B, shape.n_q_heads, T, p0 + T)
    for b in range(B):
        for h in range(shape.n_q_heads):
            np.testing.assert_array_equal(got[b, h] != 0, want, err_msg=f"mask, sequence {b} head {h}")
            np.testing.assert_array_equal(got[b, h], want_w, err_msg=f"weights, sequence {b} head {h}")
    assert kv.length == 0


def _bf16(x):
    return torch.from_numpy(synth.bf16_bits_from_f32(np.asarray(x, np.float32)).view(np.int16)).cuda()


EDGE_CASES = [
    # sublayer, p0, T, query offset, hot keys, expected winner, max_seq
    (0, 1500, 300, 100, (576, 577), 577, 2100),     # cached keys in the wrapped ring, window edge
    (0, 1500, 300, 0, (476, 477), 477, 2100),       # first query of the chunk
    (0, 1500, 300, 299, (775, 776), 776, 2100),     # last query of the chunk
    (0, 0, 1100, 1090, (66, 67), 67, 1100),         # fresh keys of the same chunk
    (0, 3000, 1, 0, (1976, 1977), 1977, 4096),      # decode, ring wrapped
    (2, 70000, 1, 0, (0, 70001), 0, 70016),         # full decode: the first key; a stale row past the query
    (2, 70000, 1, 0, (65536, 70000), None, 70016),  # full decode: two visible keys share the weight
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[f"sub{c[0]}-p{c[1]}-T{c[2]}-q{c[3]}" for c in EDGE_CASES])
def test_window_edges_with_hot_keys(M, case):
    """Two keys get a score of 4 sqrt(dh) (about e^45 times the others) and
    one-hot values at dims (u mod 128); every other key has score 0. The
    query's output is then the one-hot of the visible hot key (or the mean
    of both when both are visible): a key read from the wrong cache row, or
    an off-by-one window edge, moves the weight elsewhere."""
    sub, p0, T, qoff, hot, winner, max_seq = case
    shape = synth.PAIR
    nq, nkv, dh = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    log(f"edge sublayer {sub} p0={p0} T={T} query {p0 + qoff} hot {hot}")
    m, _ = _probe_model(M, shape)
    kv = m.kv_cache("last_loop", 1, 1, max_seq)
    info = kv.slot(sub)
    rows, ring = info.rows, info.ring
    L = p0 + T

    def kvec(u):
        v = np.zeros(dh, np.float32)
        if u in hot:
            v[0] = 4.0
        return v

    def vvec(u):
        v = np.zeros(dh, np.float32)
        v[u % dh] = 1.0
        return v

    # cached positions below p0, written where the documented layout puts
    # them: row u mod ring (sliding window) or u (full attention)
    lo = max(0, p0 - ring) if ring > 0 else 0
    Kc = np.zeros((nkv, rows, dh), np.float32)
    Vt = np.zeros((nkv, dh, rows), np.float32)
    for u in range(lo, p0):
        r = u % ring if ring > 0 else u
        Kc[:, r] = kvec(u)
        Vt[:, :, r] = vvec(u)
    if ring == 0:
        # rows past the step hold stale entries that must never be read
        for u in range(L, rows):
            Kc[:, u] = kvec(u)
            Vt[:, :, u] = vvec(u)
    base = kv.buffer.data_ptr()
    nb = nkv * rows * dh * 2
    kv.buffer[info.k - base: info.k - base + nb].copy_(_bf16(Kc).view(torch.uint8).reshape(-1))
    kv.buffer[info.v - base: info.v - base + nb].copy_(_bf16(Vt).view(torch.uint8).reshape(-1))
    kn = np.stack([kvec(u) for u in range(p0, L)])[None, None].repeat(nkv, 1)
    vn = np.stack([vvec(u) for u in range(p0, L)])[None, None].repeat(nkv, 1)
    q = np.zeros((1, nq, T, dh), np.float32)
    q[..., 0] = 1.0
    gate = np.ones((T, nq * dh), np.float32)
    z = M.debug_attention(kv, sub, p0, _bf16(q), _bf16(kn), _bf16(vn), _bf16(gate))
    torch.cuda.synchronize()
    zb = z.cpu().numpy().view(np.uint16)
    zf = synth.f64_from_bf16_bits(zb).reshape(T, nq, dh)[qoff]
    p = p0 + qoff
    window = shape.window if ref.layer_kinds(shape)[sub] == ref.KIND_SWA else None
    vis = [u for u in hot if ref.visible(np.array([p]), np.array([u]), window)[0, 0]]
    if winner is not None:
        assert vis == [winner]
    want = np.zeros(dh)
    for u in vis:
        want[u % dh] += 1.0 / len(vis)
    for h in range(nq):
        np.testing.assert_allclose(zf[h], want, atol=4e-3, err_msg=f"head {h}")


def test_cache_rows_of_positions(M):
    shape = synth.TINY_REC_FULL
    m, _ = _probe_model(M, shape)
    kv = m.kv_cache("per_loop", 2, 2, 200)
    for sub, kind in enumerate(ref.layer_kinds(shape)):
        if kind == ref.KIND_MLP:
            continue
        info = kv.slot(sub)
        for pos_a, n in ((0, 200), (37, 100), (199, 1)):
            got = M.debug_kv_slots(kv, sub, pos_a, n).cpu().numpy()
            pos = np.arange(pos_a, pos_a + n)
            # a ring holds the window and DORY_KV_ROLLBACK (64) more positions
            ring = shape.window + 64
            want = pos % ring if kind == ref.KIND_SWA else pos
            assert info.ring == (ring if kind == ref.KIND_SWA else 0)
            np.testing.assert_array_equal(got, want)
    # a full-shape window of 1,024 positions: 1,088 rows
    mp, _ = _probe_model(M, synth.PAIR)
    kvp = mp.kv_cache("last_loop", 1, 1, 5000)
    got = M.debug_kv_slots(kvp, 0, 1000, 4000).cpu().numpy()
    np.testing.assert_array_equal(got, np.arange(1000, 5000) % 1088)
    got = M.debug_kv_slots(kvp, 2, 1000, 4000).cpu().numpy()
    np.testing.assert_array_equal(got, np.arange(1000, 5000))


def test_greedy_lowest_index_on_repeated_maxima(M):
    """Rows of the LM-head width with repeated maxima placed in the same
    thread's stride, in different waves, at the ends of the row and next to
    each other; the first maximum (numpy's argmax) must win, bit for bit.
    NaN entries never win."""
    V = 131072
    g = np.random.default_rng(5)
    rows = []
    expect = []

    def row_with(idx, val=5.0, base=None):
        r = g.standard_normal(V).astype(np.float32) if base is None else base.copy()
        for i in idx:
            r[i] = val
        return r

    cases = [
        (np.zeros(V, np.float32), 0),
        (row_with([7, 1031]), 7),              # the same thread's strided elements
        (row_with([1029, 5]), 5),              # different threads and waves
        (row_with([131071, 64]), 64),          # the last element ties
        (row_with([131071]), 131071),
        (row_with([1000, 999]), 999),          # neighbours in one wave
        (row_with([64, 63]), 63),              # neighbours in two waves
        (row_with([70000, 3000, 90000]), 3000),
        (np.full(V, -np.inf, np.float32), 0),  # nothing above -inf
    ]
    r = row_with([100], 2.0, np.full(V, -np.inf, np.float32))
    r[3] = np.nan
    cases.append((r, 100))                     # NaN never wins
    for i in range(6):
        r = g.standard_normal(V).astype(np.float32)
        idx = np.sort(g.choice(V, 4, replace=False))
        r[idx] = r.max() + 1.0
        cases.append((r, int(idx[0])))
    for r, e in cases:
        rows.append(r)
        expect.append(e)
    x = torch.from_numpy(np.stack(rows)).cuda()
    got = M.greedy(x).cpu().numpy()
    np.testing.assert_array_equal(got, np.array(expect, np.int32))
    finite = [i for i, r in enumerate(rows) if not np.isnan(r).any()]
    np.testing.assert_array_equal(got[finite], np.argmax(np.stack(rows)[finite], axis=1))
