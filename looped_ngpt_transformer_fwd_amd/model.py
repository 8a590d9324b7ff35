"""Python handles over the C ABI. PyTorch supplies device memory and the
stream; every step of the forward pass runs in libdory.so."""
import ctypes

import torch

from . import _lib as C

KIND_CODE = {"swa": C.DORY_LAYER_ATTN_SWA, "full": C.DORY_LAYER_ATTN_FULL, "mlp": C.DORY_LAYER_MLP}
MODE_CODE = {"last_loop": C.DORY_CACHE_LAST_LOOP, "per_loop": C.DORY_CACHE_PER_LOOP}


def make_config(shape):
    """dory_config from any object with the Shape attributes (d_model,
    n_q_heads, ..., layer_kinds as a tuple of 'swa'/'full'/'mlp' or None)."""
    cfg = C.dory_config()
    cfg.d_model = shape.d_model
    cfg.n_q_heads = shape.n_q_heads
    cfg.n_kv_heads = shape.n_kv_heads
    cfg.head_dim = shape.head_dim
    cfg.d_ff = shape.d_ff
    cfg.vocab = shape.vocab
    cfg.n_input = shape.n_input
    cfg.n_recurrent = shape.n_recurrent
    cfg.n_output = shape.n_output
    cfg.window = shape.window
    cfg.full_every = getattr(shape, "full_every", 4)
    cfg.has_lm_head = 1 if getattr(shape, "has_lm_head", True) else 0
    cfg.rope_base_swa = shape.rope_base_swa
    cfg.rope_base_full = shape.rope_base_full
    cfg.softmax_scale = 0.0
    cfg.precision = (C.DORY_PRECISION_FP32 if getattr(shape, "precision", "bf16") == "fp32"
                     else C.DORY_PRECISION_BF16)
    kinds = getattr(shape, "layer_kinds", None)
    cfg._kinds_keepalive = None
    if kinds is not None:
        arr = (ctypes.c_int32 * len(kinds))(*[KIND_CODE[k] for k in kinds])
        cfg._kinds_keepalive = arr
        cfg.layer_kinds = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return cfg


def schedule(shape):
    cfg = make_config(shape)
    n = shape.n_input + shape.n_recurrent + shape.n_output
    out = (ctypes.c_int32 * n)()
    C.check(C.dory_schedule(cfg, out, n), "dory_schedule")
    inv = {v: k for k, v in KIND_CODE.items()}
    return [inv[x] for x in out]


def kv_bytes(shape, mode, k_max, batch, max_seq):
    return C.dory_kv_bytes(make_config(shape), MODE_CODE[mode], k_max, batch, max_seq)


def workspace_bytes(shape, batch, tokens):
    return C.dory_workspace_bytes(make_config(shape), batch, tokens)


def mxfp8_bytes(shape):
    return C.dory_mxfp8_bytes(make_config(shape))


def mxfp8_quantize(w):
    """MXFP8 quantization of a bf16 device matrix [rows, cols]: (codes uint8
    [rows, cols], scale codes uint8 [rows, cols / 32], dequantized bf16)."""
    rows, cols = w.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=w.device)
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device=w.device)
    deq = torch.empty(rows, cols, dtype=torch.bfloat16, device=w.device)
    C.check(C.dory_mxfp8_quantize(_ptr(w), rows, cols, _ptr(codes), _ptr(scales), _ptr(deq),
                                  _stream()), "dory_mxfp8_quantize")
    return codes, scales, deq


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Model:
    """Wraps dory_model. `tensors` maps weight names to device tensors:
    embed, lm_head, s_z, sub{i}.w_qkvg, sub{i}.w_o, sub{i}.s_qk,
    sub{i}.w_upgate, sub{i}.w_down, sub{i}.s_u, sub{i}.s_v, sub{i}.alpha
    (bf16 matrices in [out, in] layout, fp32 vectors)."""

    def __init__(self, shape, tensors):
        self.shape = shape
        self.cfg = make_config(shape)
        self.tensors = tensors
        self.kinds = schedule(shape)
        n = len(self.kinds)
        subs = (C.dory_sublayer_weights * n)()
        for i, kind in enumerate(self.kinds):
            s = subs[i]
            s.alpha = _ptr(tensors[f"sub{i}.alpha"])
            if kind == "mlp":
                s.w_upgate = _ptr(tensors[f"sub{i}.w_upgate"])
                s.w_down = _ptr(tensors[f"sub{i}.w_down"])
                s.s_u = _ptr(tensors[f"sub{i}.s_u"])
                s.s_v = _ptr(tensors[f"sub{i}.s_v"])
            else:
                s.w_qkvg = _ptr(tensors[f"sub{i}.w_qkvg"])
                s.w_o = _ptr(tensors[f"sub{i}.w_o"])
                s.s_qk = _ptr(tensors[f"sub{i}.s_qk"])
        w = C.dory_weights()
        w.embed = _ptr(tensors["embed"])
        if getattr(shape, "has_lm_head", True):
            w.lm_head = _ptr(tensors["lm_head"])
            w.s_z = _ptr(tensors["s_z"])
        w.sublayers = subs
        self._subs = subs
        self.handle = ctypes.c_void_p()
        C.check(C.dory_model_create(self.cfg, w, self.handle), "dory_model_create")

    def __del__(self):
        h = getattr(self, "handle", None)
        try:
            if h is not None and h.value:
                C.dory_model_destroy(h)
        except Exception:  # interpreter shutdown
            pass
        self.handle = None

    def selfspec_step(self, kv, last, gamma, k_draft, k_verify, ws=None):
        """One self-speculative round (greedy): returns (n accepted, tokens
        [B, n + 1]) -- the next n + 1 tokens of every sequence."""
        B = kv.batch
        if ws is None:
            ws = self.workspace(B, gamma + 1)
        scratch = torch.empty(2 * B * (gamma + 1), dtype=torch.int32, device=last.device)
        out = torch.empty(gamma + 1, B, dtype=torch.int32, device=last.device)
        n = ctypes.c_int32()
        C.check(C.dory_selfspec_step(self.handle, kv.handle, _ptr(last), B, gamma, k_draft, k_verify,
                                     kv.mode_code, _ptr(ws), ws.numel(), _ptr(scratch), _ptr(out), n,
                                     _stream()), "dory_selfspec_step")
        return n.value, out[:n.value + 1].t().contiguous()

    def selfspec_step_sampled(self, kv, last, gamma, k_draft, k_verify, temperature, u, ws=None):
        """One sampled self-speculative round; u: device fp32 [2 gamma + 1, B]
        uniforms. Returns (n accepted by the batch, out [gamma + 1, B] device
        int32 per-sequence tokens, logits buffer [2 gamma + 1, B, V], the
        drafted tokens [gamma, B])."""
        B = kv.batch
        dev = last.device
        if ws is None:
            ws = self.workspace(B, gamma + 1)
        scratch = torch.empty(2 * B * (gamma + 1), dtype=torch.int32, device=dev)
        lbuf = torch.empty(2 * gamma + 1, B, self.shape.vocab, dtype=torch.float32, device=dev)
        out = torch.empty(gamma + 1, B, dtype=torch.int32, device=dev)
        n = ctypes.c_int32()
        C.check(C.dory_selfspec_step_sampled(self.handle, kv.handle, _ptr(last), B, gamma, k_draft,
                                             k_verify, kv.mode_code, float(temperature), _ptr(u),
                                             _ptr(ws), ws.numel(), _ptr(scratch), _ptr(lbuf),
                                             _ptr(out), n, _stream()), "dory_selfspec_step_sampled")
        return n.value, out, lbuf, scratch[B:(gamma + 1) * B].view(gamma, B)

    def quantize_mxfp8(self, device="cuda"):
        """Quantizes the projection matrices to MXFP8 (weight-only) into a
        buffer owned by this object and switches the model to them."""
        n = mxfp8_bytes(self.shape)
        self.mx_buffer = torch.empty(n, dtype=torch.uint8, device=device)
        C.check(C.dory_model_quantize_mxfp8(self.handle, _ptr(self.mx_buffer), n, _stream()),
                "dory_model_quantize_mxfp8")

    def set_decode_graphs(self, on):
        """Decode steps replayed from captured HIP graphs (default) or launched
        kernel by kernel."""
        C.check(C.dory_model_set_decode_graphs(self.handle, 1 if on else 0),
                "dory_model_set_decode_graphs")

    def use_mxfp8(self, on):
        C.check(C.dory_model_use_mxfp8(self.handle, 1 if on else 0), "dory_model_use_mxfp8")

    def profile_begin(self, max_launches=100000):
        C.check(C.dory_profile_begin(self.handle, max_launches), "dory_profile_begin")

    def profile_end(self):
        """{class: (launches, total ms)} of the launches timed since profile_begin."""
        counts = (ctypes.c_int64 * C.DORY_K_NUM_CLASSES)()
        ms = (ctypes.c_double * C.DORY_K_NUM_CLASSES)()
        C.check(C.dory_profile_end(self.handle, counts, ms), "dory_profile_end")
        return {C.KERNEL_CLASSES[i]: (int(counts[i]), float(ms[i]))
                for i in range(C.DORY_K_NUM_CLASSES)}

    def workspace(self, batch, tokens, device="cuda"):
        n = workspace_bytes(self.shape, batch, tokens)
        return torch.empty(n, dtype=torch.uint8, device=device)

    def kv_cache(self, mode, k_max, batch, max_seq, device="cuda"):
        return KVCache(self, mode, k_max, batch, max_seq, device)

    def prefill(self, kv, tokens, k, ws=None, logits=True, next_token=False, hidden=False,
                states=False):
        """tokens: int32 device tensor [B, T]; k: loop count, or one loop count
        per sequence (list) for a mixed step. Returns a dict of the requested
        outputs (logits [B, V], next [B], hidden [B, T, d], states [max k, B,
        T, d])."""
        B, T = tokens.shape
        return self._step(kv, tokens, B, T, k, ws, logits, next_token, hidden, states, decode=False)

    def decode_step(self, kv, tokens, k, ws=None, logits=True, next_token=True, hidden=False,
                    states=False, into=None):
        """tokens: int32 device tensor [B]. `into` (optional dict) supplies the
        "logits" [B, V] fp32 and/or "next" [B] int32 tensors to write into
        (fixed buffers let repeated steps replay one captured graph)."""
        B = tokens.shape[0]
        return self._step(kv, tokens, B, 1, k, ws, logits, next_token, hidden, states, decode=True,
                          into=into)

    def _step(self, kv, tokens, B, T, k, ws, logits, next_token, hidden, states, decode, into=None):
        dev = tokens.device
        sh = self.shape
        if ws is None:
            ws = self.workspace(B, T, dev)
        out = {}
        into = into or {}
        lg = (into.get("logits") if "logits" in into else
              torch.empty(B, sh.vocab, dtype=torch.float32, device=dev)) if logits else None
        nx = (into.get("next") if "next" in into else
              torch.empty(B, dtype=torch.int32, device=dev)) if next_token else None
        hd = torch.empty(B, T, sh.d_model, dtype=torch.float32, device=dev) if hidden else None
        rows = None
        if isinstance(k, (list, tuple)):
            # per-sequence loop counts (host int32 array handed to the library)
            if len(k) != B:
                raise ValueError("one loop count per sequence")
            rows = (ctypes.c_int32 * B)(*[int(x) for x in k])
            k = max(int(x) for x in k)
        stt = torch.empty(k, B, T, sh.d_model, dtype=torch.float32, device=dev) if states else None
        mode = kv.mode_code
        if rows is not None:
            if decode:
                st = C.dory_decode_step_rows(self.handle, kv.handle, _ptr(tokens), B, rows, mode,
                                             _ptr(ws), ws.numel(), _ptr(lg), _ptr(nx), _ptr(hd),
                                             _ptr(stt), _stream())
                where = "dory_decode_step_rows"
            else:
                st = C.dory_prefill_rows(self.handle, kv.handle, _ptr(tokens), B, T, rows, mode,
                                         _ptr(ws), ws.numel(), _ptr(lg), _ptr(nx), _ptr(hd),
                                         _ptr(stt), _stream())
                where = "dory_prefill_rows"
        elif decode:
            st = C.dory_decode_step(self.handle, kv.handle, _ptr(tokens), B, k, mode, _ptr(ws),
                                    ws.numel(), _ptr(lg), _ptr(nx), _ptr(hd), _ptr(stt), _stream())
            where = "dory_decode_step"
        else:
            st = C.dory_prefill(self.handle, kv.handle, _ptr(tokens), B, T, k, mode, _ptr(ws),
                                ws.numel(), _ptr(lg), _ptr(nx), _ptr(hd), _ptr(stt), _stream())
            where = "dory_prefill"
        C.check(st, where)
        if lg is not None:
            out["logits"] = lg
        if nx is not None:
            out["next"] = nx
        if hd is not None:
            out["hidden"] = hd
        if stt is not None:
            out["states"] = stt
        return out


class KVCache:
    def __init__(self, model, mode, k_max, batch, max_seq, device="cuda"):
        self.model = model
        self.mode = mode
        self.mode_code = MODE_CODE[mode]
        self.batch = batch
        n = kv_bytes(model.shape, mode, k_max, batch, max_seq)
        if n == 0:
            raise ValueError("invalid cache parameters")
        self.buffer = torch.empty(n, dtype=torch.uint8, device=device)
        self.handle = ctypes.c_void_p()
        C.check(C.dory_kv_bind(model.handle, _ptr(self.buffer), n, self.mode_code, k_max, batch,
                               max_seq, self.handle), "dory_kv_bind")

    @property
    def length(self):
        return C.dory_kv_length(self.handle)

    def reset(self):
        C.check(C.dory_kv_reset(self.handle), "dory_kv_reset")

    def set_length(self, length):
        C.check(C.dory_kv_set_length(self.handle, length), "dory_kv_set_length")

    def copy_prefix_from(self, src, src_seq, dst_seq, n):
        """Reuses the first n cached positions of sequence src_seq of cache
        `src` as those of sequence dst_seq of this cache (prefix caching);
        this cache's length becomes n."""
        C.check(C.dory_kv_copy_prefix(src.handle, src_seq, self.handle, dst_seq, n, _stream()),
                "dory_kv_copy_prefix")

    def slot(self, sublayer, loop=0):
        info = C.dory_kv_slot_info()
        C.check(C.dory_kv_slot(self.handle, sublayer, loop, info), "dory_kv_slot")
        return info

    def __del__(self):
        h = getattr(self, "handle", None)
        try:
            if h is not None and h.value:
                C.dory_kv_destroy(h)
        except Exception:  # interpreter shutdown
            pass
        self.handle = None


def sample(logits, temperature, u):
    """Sampling by inversion from softmax(logits / temperature), one uniform
    per row (device fp32 [rows]): device int32 [rows]."""
    rows, n = logits.shape
    out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    C.check(C.dory_sample(_ptr(logits), rows, n, float(temperature), _ptr(u), _ptr(out), _stream()),
            "dory_sample")
    return out


def speculative_accept(draft_logits, verify_logits, drafts, u, temperature):
    """draft_logits [gamma, B, V], verify_logits [gamma + 1, B, V], drafts
    [gamma, B], u [gamma + 1, B] (device): (n_accepted [B], out [gamma + 1, B])."""
    gamma, B, V = draft_logits.shape
    n = torch.empty(B, dtype=torch.int32, device=draft_logits.device)
    out = torch.empty(gamma + 1, B, dtype=torch.int32, device=draft_logits.device)
    C.check(C.dory_speculative_accept(_ptr(draft_logits), _ptr(verify_logits), _ptr(drafts), _ptr(u),
                                      B, V, gamma, float(temperature), _ptr(n), _ptr(out), _stream()),
            "dory_speculative_accept")
    return n, out


def greedy(logits):
    """Argmax of each row of a device fp32 [rows, n] tensor (lowest index on
    ties): device int32 [rows]."""
    rows, n = logits.shape
    out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    C.check(C.dory_greedy(_ptr(logits), rows, n, _ptr(out), _stream()), "dory_greedy")
    return out


def debug_kv_slots(kv, sublayer, pos_a, n):
    """Device-evaluated cache rows of positions pos_a .. pos_a + n - 1."""
    out = torch.empty(n, dtype=torch.int64, device=kv.buffer.device)
    C.check(C.dory_debug_kv_slots(kv.handle, sublayer, pos_a, n, _ptr(out), _stream()),
            "dory_debug_kv_slots")
    return out


def debug_attention(kv, sublayer, p0, q_hat, k_new, v_new, gate, loop=0, ws=None):
    """Attention kernels of `sublayer` on caller inputs (see
    dory_debug_attention): q_hat [B, n_q, T, dh], k_new / v_new
    [B, n_kv, T, dh], gate [B * T, n_q * dh] (bf16 device tensors); returns z."""
    m = kv.model
    T = q_hat.shape[2]
    if ws is None:
        ws = m.workspace(kv.batch, T, q_hat.device)
    z = torch.empty_like(gate)
    C.check(C.dory_debug_attention(m.handle, kv.handle, sublayer, loop, p0, T, _ptr(q_hat),
                                   _ptr(k_new), _ptr(v_new), _ptr(gate), _ptr(z), _ptr(ws),
                                   ws.numel(), _stream()), "dory_debug_attention")
    return z


def debug_mask(kv, sublayer, p0, T, loop=0, ws=None):
    """Key weights under equal scores, read off the attention kernels of
    `sublayer` (see dory_debug_mask): bf16 bit patterns as int16
    [B, n_q, T, p0 + T]; nonzero exactly at the visible keys."""
    m = kv.model
    dev = kv.buffer.device
    if ws is None:
        ws = m.workspace(kv.batch, T, dev)
    out = torch.empty(kv.batch, m.shape.n_q_heads, T, p0 + T, dtype=torch.int16, device=dev)
    C.check(C.dory_debug_mask(m.handle, kv.handle, sublayer, loop, p0, T, _ptr(ws), ws.numel(),
                              _ptr(out), _stream()), "dory_debug_mask")
    return out
