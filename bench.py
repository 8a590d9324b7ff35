"""Benchmark of the looped normalized-GPT forward pass on one MI355X.

Step = one prefill of the full 72-sublayer model (16 input + 40 recurrent x k
+ 16 output sublayers, d=2304, 16/4 heads of 128, SwiGLU 6144, window 1024,
vocab 131072) over B=4 sequences of 8192 synthetic tokens with last-loop KV
caching: embedding, every sublayer, the last-loop KV writes, the LM head for
the last position and greedy selection. Weights are random row-normalized
bf16 matrices drawn on the GPU from a seeded generator; inputs are resident
in HBM before timing starts.

Prints one JSON line: `value` is prefill tokens/s at the chosen k (default
4); extra fields give prefill tokens/s at k = 1, 2, 4, decode tokens/s at
B=64 with 32768 tokens of synthesized cached context for k = 1, 2, 4 under
both cache policies, per-kernel-class timings measured with HIP events on the
call's stream over the timed region, the roofline entry of the dominant
kernel and the CPU oracle baseline.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def gpu_weights(shape, kinds, seed=0, device="cuda"):
    """Random N(0,1) rows scaled to unit length, rounded to bf16 on the GPU;
    per-channel vectors as in the parity tests (alpha 0.05 U(.5,1.5), s_qk
    U(.5,1.5), s_u U(.5,1.5), s_v and s_z sqrt(d) U(.5,1.5))."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def mat(r, c):
        out = torch.empty(r, c, dtype=torch.bfloat16, device=device)
        step = max(1, (1 << 26) // c)
        for r0 in range(0, r, step):
            w = torch.randn(min(step, r - r0), c, device=device, generator=g)
            w /= w.norm(dim=1, keepdim=True)
            out[r0:r0 + w.shape[0]] = w.to(torch.bfloat16)
        return out.view(torch.int16)

    def vec(n, mult=1.0):
        return (mult * (0.5 + torch.rand(n, device=device, generator=g))).float()

    s = shape
    sd = s.d_model ** 0.5
    t = {"embed": mat(s.vocab, s.d_model), "lm_head": mat(s.vocab, s.d_model), "s_z": vec(s.vocab, sd)}
    for i, k in enumerate(kinds):
        t[f"sub{i}.alpha"] = vec(s.d_model, 0.05)
        if k == "mlp":
            t[f"sub{i}.w_upgate"] = mat(2 * s.d_ff, s.d_model)
            t[f"sub{i}.w_down"] = mat(s.d_model, s.d_ff)
            t[f"sub{i}.s_u"] = vec(s.d_ff)
            t[f"sub{i}.s_v"] = vec(s.d_ff, sd)
        else:
            t[f"sub{i}.w_qkvg"] = mat(2 * s.d_q + 2 * s.d_kv, s.d_model)
            t[f"sub{i}.w_o"] = mat(s.d_model, s.d_q)
            t[f"sub{i}.s_qk"] = vec(s.head_dim)
    return t


def attention_flops(shape, kinds, B, T, k):
    """Algorithmic attention FLOPs of one prefill from position 0: per query
    4 * n_q * head_dim per visible key (QK^T and PV)."""
    p = np.arange(T, dtype=np.float64)
    full = np.sum(p + 1)
    swa = np.sum(np.minimum(p + 1, shape.window))
    per = 4.0 * shape.n_q_heads * shape.head_dim * B
    tot = 0.0
    for i, kind in enumerate(kinds):
        if kind == "mlp":
            continue
        rep = k if shape.n_input <= i < shape.n_input + shape.n_recurrent else 1
        tot += rep * per * (full if kind == "full" else swa)
    return tot


def class_work(shape, M):
    """Algorithmic work per launch of each kernel class at M token rows:
    (amount, unit, bound)."""
    s = shape
    d, F, dq, dkv = s.d_model, s.d_ff, s.d_q, s.d_kv
    return {
        "gemm_qkvg": (2.0 * M * (2 * dq + 2 * dkv) * d, "flop", "mfma"),
        "gemm_o": (2.0 * M * d * dq, "flop", "mfma"),
        "gemm_upgate": (2.0 * M * 2 * F * d, "flop", "mfma"),
        "gemm_down": (2.0 * M * d * F, "flop", "mfma"),
        # read h (fp32) and y (bf16: the large-M projections write their
        # output once in bf16), write h (fp32) and its bf16 copy
        "update": (float(M) * d * (4 + 2 + 4 + 2), "byte", "hbm"),
    }


# Source files whose kernels make up each timed class; a counter record is
# valid only for the sources it was taken on.
CLASS_SOURCES = {
    "gemm_qkvg": ("gemm.hip", "common.h"), "gemm_o": ("gemm.hip", "common.h"),
    "gemm_upgate": ("gemm.hip", "common.h"), "gemm_down": ("gemm.hip", "common.h"),
    "update": ("rowops.hip", "common.h"), "attn": ("attention.hip", "common.h"),
}


def source_digest(cls):
    import hashlib
    h = hashlib.sha256()
    for f in CLASS_SOURCES[cls]:
        with open(os.path.join(ROOT, "looped_ngpt_transformer_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(cls):
    """HBM bytes per launch of the class from the hardware counter record in
    profiles/ (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads
    for a copy of known size), or None if none was taken on the current
    kernel sources."""
    import glob
    import re
    want = source_digest(cls)
    pat = re.compile(r"traffic-record: class=(\S+) sources=(\S+) bytes_per_launch=(\S+)")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                m = pat.search(line)
                if m and m.group(1) == cls and m.group(2) == want:
                    return float(m.group(3))
    return None


def run_prefill(gm, kv, toks, k, ws):
    kv.reset()
    return gm.prefill(kv, toks, k, ws=ws, logits=True, next_token=True)


def time_steps(fn, steps):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def fill_random(kv, g):
    """Synthesized cache contents: N(0, 0.02^2) bf16 in every slot."""
    buf = kv.buffer.view(torch.bfloat16)
    chunk = 1 << 28
    for o in range(0, buf.numel(), chunk):
        n = min(chunk, buf.numel() - o)
        buf[o:o + n] = (0.02 * torch.randn(n, device="cuda", generator=g)).to(torch.bfloat16)


def greedy_decode(gm, kv, first, k, ws, ctx, warmup, steps):
    """Greedy decoding from position ctx, each step's input token being the
    previous step's greedy choice (fixed token and logits buffers, so the
    steps replay captured graphs). The cache is declared to hold ctx valid
    positions (its K/V synthesized beforehand). Returns the seconds of the
    `steps` timed steps, which follow `warmup` untimed ones."""
    B = first.shape[0]
    toks = [first.clone(), torch.empty_like(first)]
    lg = torch.empty(B, gm.shape.vocab, dtype=torch.float32, device="cuda")
    kv.reset()
    kv.set_length(ctx)
    i = [0]

    def step():
        gm.decode_step(kv, toks[i[0] % 2], k, ws=ws, into={"logits": lg, "next": toks[(i[0] + 1) % 2]})
        i[0] += 1
    for _ in range(warmup):
        step()
    dt = time_steps(step, steps)
    assert kv.length == ctx + warmup + steps
    return dt


def decode_mxfp8(gm, shape, B=64, steps=256):
    """Decode tokens/s with MXFP8 weights (W8A16) against bf16: at the same
    32768-token context (last-loop, k = 1, 2, 4) and at a 2048-token context
    (k = 4), where the weight stream is a larger share of a step. The model
    is switched back to bf16 afterwards."""
    out = {}
    short = decode_table(gm, shape, (4,), ("last_loop",), B=B, ctx=2048, steps=steps)
    out["bf16_ctx2048_last_loop_k4"] = short["last_loop_k4"]
    gm.quantize_mxfp8()
    try:
        t = decode_table(gm, shape, (1, 2, 4), ("last_loop",), B=B, steps=steps, mixed=False)
        for k in (1, 2, 4):
            out[f"mxfp8_last_loop_k{k}"] = t[f"last_loop_k{k}"]
        short = decode_table(gm, shape, (4,), ("last_loop",), B=B, ctx=2048, steps=steps)
        out["mxfp8_ctx2048_last_loop_k4"] = short["last_loop_k4"]
    finally:
        gm.use_mxfp8(False)
        del gm.mx_buffer
        torch.cuda.empty_cache()
    return out


def decode_table(gm, shape, ks, modes, B=64, ctx=32768, steps=256, warmup=2, mixed=True):
    """Decode tokens/s: `steps` greedy steps (token fed back) after `ctx`
    cached tokens whose K/V are synthesized at random (the cost of a step
    depends on the context length, not on the cached values), per (mode, k),
    with the cache size of each."""
    out = {}
    ws = gm.workspace(B, 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    toks = torch.randint(0, shape.vocab, (B,), dtype=torch.int32, device="cuda", generator=g)
    n_seq = ctx + warmup + steps
    for mode in modes:
        for k in ks:
            kv = gm.kv_cache(mode, k, B, n_seq)
            fill_random(kv, g)
            dt = greedy_decode(gm, kv, toks, k, ws, ctx, warmup, steps)
            out[f"{mode}_k{k}"] = round(B * steps / dt, 1)
            out[f"{mode}_k{k}_kv_gb"] = round(kv.buffer.numel() / 1e9, 2)
            progress(f"decode B={B} ctx={ctx} {mode} k={k}: {out[f'{mode}_k{k}']} tokens/s")
            del kv
            torch.cuda.empty_cache()
    if mixed and "last_loop" in modes and max(ks) >= 4:
        # one batch whose sequences run different loop counts, 4:1:1:1 over
        # k = 1, 2, 3, 4 (36 / 9 / 9 / 10 of 64 sequences)
        k_rows = [1] * 36 + [2] * 9 + [3] * 9 + [4] * 10
        kv = gm.kv_cache("last_loop", 4, B, n_seq)
        fill_random(kv, g)
        dt = greedy_decode(gm, kv, toks, k_rows, ws, ctx, warmup, steps)
        out["last_loop_mixed_k1k2k3k4_4111"] = round(B * steps / dt, 1)
        del kv
        torch.cuda.empty_cache()
    return out


def decode_selfspec(gm, shape, B=64, ctx=32768, gamma=4, k_draft=1, k_verify=4, steps=4):
    """Self-speculative rounds (per-loop caches): gamma greedy drafts at
    k_draft, then one verification pass over gamma + 1 positions at k_verify.
    With random weights the acceptance rate carries no information, so the
    round time is reported against the k_verify decode step: a round pays
    off when the batch accepts more than (round / step - 1) drafts. The
    sampled round (temperature 1) drafts by sampling and applies the
    rejection rule per sequence."""
    ws = gm.workspace(B, gamma + 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    toks = torch.randint(0, shape.vocab, (B,), dtype=torch.int32, device="cuda", generator=g)
    kv = gm.kv_cache("per_loop", k_verify, B, ctx + gamma + 1)
    fill_random(kv, g)
    acc = []

    def rnd():
        kv.set_length(ctx)
        acc.append(gm.selfspec_step(kv, toks, gamma, k_draft, k_verify, ws=ws)[0])

    def plain():
        kv.set_length(ctx)
        gm.decode_step(kv, toks, k_verify, ws=ws, logits=True, next_token=True)
    u = torch.rand(2 * gamma + 1, B, generator=g, device="cuda")

    def rnd_sampled():
        kv.set_length(ctx)
        gm.selfspec_step_sampled(kv, toks, gamma, k_draft, k_verify, 1.0, u, ws=ws)
    rnd()
    plain()
    rnd_sampled()
    t_round = time_steps(rnd, steps) / steps
    t_step = time_steps(plain, steps) / steps
    t_sampled = time_steps(rnd_sampled, steps) / steps
    del kv
    torch.cuda.empty_cache()
    return {"round_ms": round(t_round * 1e3, 3), "decode_step_ms": round(t_step * 1e3, 3),
            "round_sampled_ms": round(t_sampled * 1e3, 3),
            "break_even_accepted": round(t_round / t_step - 1, 2),
            "tok_s_all_accepted": round(B * (gamma + 1) / t_round, 1),
            "tok_s_none_accepted": round(B / t_round, 1),
            "decode_tok_s": round(B / t_step, 1),
            "accepted_random_weights": acc[1:],
            "config": f"B={B}, {ctx} cached tokens, per_loop, gamma={gamma}, "
                      f"draft k={k_draft}, verify k={k_verify}"}


def prefix_copy(gm, shape, n=32768, B=8, steps=4):
    """Prefix caching: the cached K/V of one sequence's n-token prefix
    (synthesized at random) copied into B sequences of another cache.
    Algorithmic bytes: what the source holds for the prefix (every full
    attention sublayer's n positions, every sliding-window ring), read once
    and written once per destination sequence."""
    src = gm.kv_cache("last_loop", 1, 1, n)
    buf = src.buffer.view(torch.bfloat16)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    buf.copy_((0.02 * torch.randn(buf.numel(), device="cuda", generator=g)).to(torch.bfloat16))
    src.set_length(n)
    dst = gm.kv_cache("last_loop", 1, B, n)

    def one():
        dst.reset()
        for b in range(B):
            dst.copy_prefix_from(src, 0, b, n)
    one()
    dt = time_steps(one, steps) / steps
    moved = 2 * src.buffer.numel() * B
    del src, dst, buf
    torch.cuda.empty_cache()
    return {"prefix_tokens": n, "sequences": B, "ms": round(dt * 1e3, 3),
            "GB_s": round(moved / dt / 1e9, 1), "frac_hbm": round(moved / dt / 1e9 / HBM_PEAK_GBS, 3)}


def long_context(gm, shape, k=4, total=262144, chunk=8192, n_dec=128):
    """One 262,144-token sequence: chunked prefill in chunks of 8,192 at k
    (last-loop cache; the later chunks attend over up to 262,143 earlier
    positions), then greedy decode steps at the full context."""
    kv = gm.kv_cache("last_loop", k, 1, total + n_dec)
    ws = gm.workspace(1, chunk)
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    toks = torch.randint(0, shape.vocab, (1, total), dtype=torch.int32, device="cuda", generator=g)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = None
    for a in range(0, total, chunk):
        last = a + chunk == total
        out = gm.prefill(kv, toks[:, a:a + chunk], k, ws=ws, logits=last, next_token=last)
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t0
    t = out["next"]
    t0 = time.perf_counter()
    for _ in range(n_dec):
        t = gm.decode_step(kv, t, k, ws=ws, logits=True, next_token=True)["next"]
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t0
    del kv, ws
    torch.cuda.empty_cache()
    return {"prefill_tok_s": round(total / t_pre, 1), "prefill_s": round(t_pre, 3),
            "decode_tok_s": round(n_dec / t_dec, 1), "decode_ms_per_step": round(t_dec / n_dec * 1e3, 3),
            "config": f"B=1, {total} tokens in chunks of {chunk}, k={k}, last_loop, "
                      f"then {n_dec} greedy decode steps"}


def pair_kernels(M, steps=3):
    """One recurrent pair at full width ([SWA attention, MLP, full attention,
    MLP], no input / output blocks, no LM head), B=1 x T=4096 prefill at
    k = 1..4, last-loop cache: tokens/s and per-kernel-class time and rate
    (the kernel classes without the rest of the model)."""
    shape = synth.PAIR
    kinds = M.schedule(shape)
    gp = M.Model(shape, gpu_weights(shape, kinds, seed=5))
    B, T = 1, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    toks = torch.randint(0, shape.vocab, (B, T), dtype=torch.int32, device="cuda", generator=g)
    ws = gp.workspace(B, T)
    work = class_work(shape, B * T)
    out = {}
    for k in (1, 2, 3, 4):
        kv = gp.kv_cache("last_loop", k, B, T)

        def one():
            kv.reset()
            gp.prefill(kv, toks, k, ws=ws, logits=False, next_token=False)
        one()
        torch.cuda.synchronize()
        gp.profile_begin(max_launches=64 * k * steps + 64)
        dt = time_steps(one, steps)
        prof = gp.profile_end()
        attn_flop = attention_flops(shape, kinds, B, T, k)
        kern = {}
        for cls, (n, ms) in prof.items():
            if n == 0:
                continue
            e = {"launches": n, "ms_avg": round(ms / n, 4)}
            if cls in work:
                amt, unit, bound = work[cls]
                e["rate"] = round(amt / (ms / n * 1e-3) / (1e12 if unit == "flop" else 1e9), 1)
                e["rate_unit"] = "TFLOP/s" if unit == "flop" else "GB/s"
            if cls == "attn":
                e["rate"] = round(attn_flop * steps / (ms * 1e-3) / 1e12, 1)
                e["rate_unit"] = "TFLOP/s"
            kern[cls] = e
        out[f"k{k}"] = {"tok_s": round(B * T * steps / dt, 1), "ms_per_step": round(dt / steps * 1e3, 3),
                        "kernels": kern}
        del kv
    del gp, ws
    torch.cuda.empty_cache()
    out["config"] = "recurrent pair [SWA, MLP, full, MLP] at d=2304, B=1 x T=4096, last_loop, k=1..4"
    return out


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class _RowGather:
    """Embedding rows widened to float64 on demand."""

    def __init__(self, bits):
        self.bits = bits

    def __getitem__(self, idx):
        return synth.f64_from_bf16_bits(self.bits[idx])


def _oracle_full_model():
    """The float64 oracle at the full model shape. Every attention sublayer
    is given one drawn weight set and every MLP sublayer another (identical
    shapes and arithmetic, a fraction of the host memory)."""
    from oracle import ref
    sh = synth.FULL
    kinds = ref.layer_kinds(sh)
    W = synth.Weights(sh, kinds, 0)
    cache = {"embed": _RowGather(W.raw("embed"))}

    def weight(name):
        if name.startswith("sub"):
            i, rest = name[3:].split(".", 1)
            name = ("sub1." if kinds[int(i)] == "mlp" else "sub0.") + rest
        if name not in cache:
            cache[name] = W.f64(name)
        return cache[name]
    for n in ("lm_head", "s_z", "sub0.w_qkvg", "sub0.w_o", "sub0.s_qk", "sub0.alpha",
              "sub1.w_upgate", "sub1.w_down", "sub1.s_u", "sub1.s_v", "sub1.alpha"):
        weight(n)
    return ref.OracleModel(sh, weight)


def _oracle_context(ctx, cap, seed):
    """A last-loop oracle cache (B=1) holding `ctx` positions of synthesized
    K/V, `cap` positions long. Full-attention slots get a random block of
    4096 positions repeated over the context; sliding-window slots get random
    values in the last window only (the oracle reads no older key of them;
    the rest of the array stays untouched zero pages)."""
    from oracle import ref
    sh = synth.FULL
    rng = np.random.default_rng(seed)
    c = ref.Cache(sh, ref.MODE_LAST, 1)
    shp = (1, sh.n_kv_heads, cap, sh.head_dim)
    for s, kind in enumerate(ref.layer_kinds(sh)):
        if kind == ref.KIND_MLP:
            continue
        K, V = np.zeros(shp), np.zeros(shp)
        if kind == ref.KIND_FULL:
            blk = rng.standard_normal((2, 1, sh.n_kv_heads, 4096, sh.head_dim)) * 0.3
            for a in range(0, ctx, 4096):
                n = min(4096, ctx - a)
                K[:, :, a:a + n] = blk[0, :, :, :n]
                V[:, :, a:a + n] = blk[1, :, :, :n]
        else:
            lo = max(0, ctx - sh.window)
            K[:, :, lo:ctx] = rng.standard_normal((1, sh.n_kv_heads, ctx - lo, sh.head_dim)) * 0.3
            V[:, :, lo:ctx] = rng.standard_normal((1, sh.n_kv_heads, ctx - lo, sh.head_dim)) * 0.3
        c.K[(s, 0)], c.V[(s, 0)] = K, V
    c.length = ctx
    return c


def cpu_baseline(k, n_tokens=512, slices=True):
    """The float64 oracle, unchanged, timed on this host's cores over bounded
    samples of the workloads. Main figure: the first n_tokens tokens of
    sequence 0 of the prefill at loop count k, full model shape. Slices:
    one decode step of one sequence after 32,768 cached tokens (k = 1 and 4,
    last-loop; per-loop caching computes the same), and one decode step at
    the end of a 262,144-token context (k = 4, last-loop), with synthesized
    cached K/V (the oracle's attention contracts over the whole prefix per
    query in one thread, so a slice of 16 such queries already takes
    minutes). Both slices run the oracle's literal
    last-loop form (write the step's entries, then read the cache), which
    leaves its cache arrays in place."""
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    sh = synth.FULL
    om = _oracle_full_model()
    toks = synth.tokens(0, 1, n_tokens, sh.vocab)
    t0 = time.perf_counter()
    om.step(ref.Cache(sh, ref.MODE_LAST, 1), toks, k)
    dt = time.perf_counter() - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    out = {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"float64 oracle, full 72-sublayer shape, k={k}, sequence 0 tokens "
                     f"0..{n_tokens - 1} (of 4 x 8192), one prefill step, {dt:.1f} s",
           "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
           "precision": "float64"}
    if not slices:
        return out
    sl = {}
    progress(f"oracle prefill sample: {n_tokens / dt:.2f} tokens/s")
    # the recurrent pair (C2 shape) over its first 512 tokens
    kp = ref.layer_kinds(synth.PAIR)
    Wp = synth.Weights(synth.PAIR, kp, 5)
    wcache = {"embed": _RowGather(Wp.raw("embed"))}

    def wpair(name):
        if name not in wcache:
            wcache[name] = Wp.f64(name)
        return wcache[name]
    op = ref.OracleModel(synth.PAIR, wpair)
    tp = synth.tokens(5, 1, 512, synth.PAIR.vocab)
    for kk in (1, 4):
        t0 = time.perf_counter()
        op.step(ref.Cache(synth.PAIR, ref.MODE_LAST, 1), tp, kk, logits=None)
        d = time.perf_counter() - t0
        sl[f"pair_t512_k{kk}"] = {"tokens_s": round(512 / d, 2), "s": round(d, 2),
                                  "sample": "recurrent pair at d=2304, B=1, tokens 0..511 (of 4096), one prefill step"}
    del op, Wp, wcache
    ctx = 32768
    cache = _oracle_context(ctx, ctx + 1, seed=11)
    tok = synth.tokens(1, 1, 1, sh.vocab)
    for kk in (1, 4):
        cache.length = ctx
        t0 = time.perf_counter()
        om.step(cache, tok, kk, literal_overwrite=True, logits="last")
        d = time.perf_counter() - t0
        sl[f"decode_ctx32768_k{kk}"] = {"tokens_s": round(1 / d, 4), "s": round(d, 2),
                                        "sample": "B=1, one decode step at position 32,768, last-loop"}
    del cache
    progress("oracle decode slices done")
    total, nq = 262144, 1
    cache = _oracle_context(total - nq, total, seed=12)
    toks = synth.tokens(2, 1, nq, sh.vocab)
    t0 = time.perf_counter()
    om.step(cache, toks, 4, literal_overwrite=True, logits="last")
    d = time.perf_counter() - t0
    sl["long_context_k4"] = {"tokens_s": round(nq / d, 4), "s": round(d, 2),
                             "sample": f"B=1, the last {nq} position(s) of a {total}-token sequence "
                                       f"in one step over {total - nq} cached positions, k=4, last-loop"}
    del cache
    out["slices"] = sl
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--k", type=int, default=4)
    ap.add_argument("--no-extra", action="store_true", help="skip k-sweep and decode table")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode table (B=64, 32768 cached tokens), for profiling")
    ap.add_argument("--decode-b1", action="store_true",
                    help="only one-sequence decode (2048 cached tokens, k = 1 and 4, 64 "
                         "steps each), for profiling the launch-bound case")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 4 GiB device-to-device copy first (reference for "
                         "hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences are independent; see the sharding notes).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    from looped_ngpt_transformer_fwd_amd import model as M
    if args.calibrate_copy:
        # 2^30 fp32 = 4 GiB read and 4 GiB written by one copy kernel
        src = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    shape = synth.FULL
    B, T, k = 4, 8192, args.k
    kinds = M.schedule(shape)
    weights = gpu_weights(shape, kinds)
    gm = M.Model(shape, weights)
    if args.decode_b1:
        # one sequence: the step is bound by its chain of launches and the
        # weight stream
        d = decode_table(gm, shape, (1, 4), ("last_loop",), B=1, ctx=2048, steps=64, mixed=False)
        print(json.dumps({"decode_b1_ctx2048_tok_s": d}), flush=True)
        return
    if args.decode_only:
        d = decode_table(gm, shape, (1, 2, 4), ("last_loop", "per_loop"))
        d.update(decode_mxfp8(gm, shape))
        print(json.dumps({"decode_tok_s": d, "selfspec": decode_selfspec(gm, shape),
                          "selfspec_b8_ctx4096": decode_selfspec(gm, shape, B=8, ctx=4096),
                          "prefix_copy": prefix_copy(gm, shape)}), flush=True)
        return
    ws = gm.workspace(B, T)
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    toks = torch.randint(0, shape.vocab, (B, T), dtype=torch.int32, device="cuda", generator=g)
    kv = gm.kv_cache("last_loop", k, B, T)

    for _ in range(args.warmup):
        run_prefill(gm, kv, toks, k, ws)
    torch.cuda.synchronize()
    gm.profile_begin(max_launches=2000 * max(1, args.steps))
    dt = time_steps(lambda: run_prefill(gm, kv, toks, k, ws), args.steps)
    prof = gm.profile_end()
    value = B * T * args.steps / dt
    ms_per_step = dt / args.steps * 1e3

    M_rows = B * T
    work = class_work(shape, M_rows)
    attn_flop = attention_flops(shape, kinds, B, T, k)
    kernels = {}
    for cls, (n, ms) in prof.items():
        if n == 0:
            continue
        e = {"launches": n, "ms_total": round(ms, 3), "ms_avg": round(ms / n, 4),
             "share": round(ms / max(1e-9, sum(v[1] for v in prof.values())), 4)}
        if cls in work:
            amt, unit, bound = work[cls]
            rate = amt / (ms / n * 1e-3)
            e["rate"] = round(rate / (1e12 if unit == "flop" else 1e9), 2)
            e["rate_unit"] = "TFLOP/s" if unit == "flop" else "GB/s"
        if cls == "attn":
            e["rate"] = round(attn_flop * args.steps / (ms * 1e-3) / 1e12, 2)
            e["rate_unit"] = "TFLOP/s"
        kernels[cls] = e
    dom = max((c for c in kernels if c in work), key=lambda c: kernels[c]["ms_total"])
    amt, unit, bound = work[dom]
    achieved = kernels[dom]["rate"]
    peak = MFMA_BF16_PEAK_TFLOPS if bound == "mfma" else HBM_PEAK_GBS
    roofline = {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_record(dom),
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "work_per_launch": amt, "work_unit": unit}

    result = {
        "metric": "prefill & decode tokens/sec at k=1/2/4 on 1 GPU; % of MFMA/HBM roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"prefill, full 72-sublayer looped nGPT (16+40k+16), k={k}, "
                               f"last_loop KV, B={B} x T={T}",
                   "global_batch": B, "seq_len": T, "loops": k, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kernels": kernels,
    }
    progress(f"prefill k={k}: {value:.0f} tokens/s")
    if not args.no_extra:
        pre = {f"k{k}": round(value, 1)}
        for kk in (1, 2, 4):
            if kk == k:
                continue
            kv2 = gm.kv_cache("last_loop", kk, B, T)
            run_prefill(gm, kv2, toks, kk, ws)
            d2 = time_steps(lambda: run_prefill(gm, kv2, toks, kk, ws), 2)
            pre[f"k{kk}"] = round(B * T * 2 / d2, 1)
            del kv2
        result["prefill_tok_s"] = dict(sorted(pre.items()))
        # cache size of the prefill configuration per policy and loop count
        result["prefill_kv_gb"] = {f"{md}_k{kk}": round(M.kv_bytes(shape, md, kk, B, T) / 1e9, 3)
                                   for md in ("last_loop", "per_loop") for kk in (1, 2, 4)}
        del kv, ws
        torch.cuda.empty_cache()
        progress("prefill k-sweep done")
        result["decode_tok_s"] = decode_table(gm, shape, (1, 2, 4), ("last_loop", "per_loop"))
        progress("decode table done")
        result["decode_tok_s"].update(decode_mxfp8(gm, shape))
        progress("mxfp8 decode done")
        result["selfspec"] = decode_selfspec(gm, shape)
        result["selfspec_b8_ctx4096"] = decode_selfspec(gm, shape, B=8, ctx=4096)
        progress("self-speculative rounds done")
        result["prefix_copy"] = prefix_copy(gm, shape)
        result["pair_c2"] = pair_kernels(M)
        progress("recurrent pair done")
        result["long_context"] = long_context(gm, shape)
        progress("long context done")
        result["decode_config"] = ("B=64, 32768 cached tokens (K/V synthesized), then 256 greedy "
                                   "steps with each step's token fed back (2 untimed first); "
                                   "mixed: per-sequence loop counts 1/2/3/4 for 36/9/9/10 sequences; "
                                   "mxfp8: projection weights in MXFP8 (W8A16), embedding and LM head "
                                   "bf16; ctx2048: 2048 cached tokens")
    if not args.no_cpu:
        progress("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(k)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
