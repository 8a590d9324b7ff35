"""ctypes view of include/dory.h: the same names, argument marshalling only.

Loading fails loudly when libdory.so has not been built; there is no other
implementation to fall back to.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdory.so")

DORY_OK = 0
DORY_ERR_ARG = 1
DORY_ERR_MODE = 2
DORY_ERR_CAPACITY = 3
DORY_ERR_WORKSPACE = 4
DORY_ERR_UNSUPPORTED = 5
DORY_ERR_HIP = 6
DORY_ERR_STATE = 7

DORY_CACHE_LAST_LOOP = 0
DORY_CACHE_PER_LOOP = 1

DORY_PRECISION_BF16 = 0
DORY_PRECISION_FP32 = 1

DORY_LAYER_ATTN_SWA = 0
DORY_LAYER_ATTN_FULL = 1
DORY_LAYER_MLP = 2


class dory_config(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("n_input", ctypes.c_int32), ("n_recurrent", ctypes.c_int32),
        ("n_output", ctypes.c_int32), ("window", ctypes.c_int32),
        ("full_every", ctypes.c_int32), ("has_lm_head", ctypes.c_int32),
        ("rope_base_swa", ctypes.c_double), ("rope_base_full", ctypes.c_double),
        ("softmax_scale", ctypes.c_double),
        ("layer_kinds", ctypes.POINTER(ctypes.c_int32)),
        ("precision", ctypes.c_int32),
    ]


class dory_sublayer_weights(ctypes.Structure):
    _fields_ = [
        ("w_qkvg", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("s_qk", ctypes.c_void_p),
        ("w_upgate", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("s_u", ctypes.c_void_p), ("s_v", ctypes.c_void_p), ("alpha", ctypes.c_void_p),
    ]


class dory_weights(ctypes.Structure):
    _fields_ = [
        ("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("s_z", ctypes.c_void_p),
        ("sublayers", ctypes.POINTER(dory_sublayer_weights)),
    ]


class dory_kv_slot_info(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("ring", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "dory_model_create": (_I32, [ctypes.POINTER(dory_config), ctypes.POINTER(dory_weights),
                                 ctypes.POINTER(_P)]),
    "dory_model_destroy": (None, [_P]),
    "dory_schedule": (_I32, [ctypes.POINTER(dory_config), ctypes.POINTER(_I32), _I32]),
    "dory_kv_bytes": (_SZ, [ctypes.POINTER(dory_config), _I32, _I32, _I32, _I64]),
    "dory_workspace_bytes": (_SZ, [ctypes.POINTER(dory_config), _I32, _I32]),
    "dory_kv_bind": (_I32, [_P, _P, _SZ, _I32, _I32, _I32, _I64, ctypes.POINTER(_P)]),
    "dory_kv_destroy": (None, [_P]),
    "dory_kv_reset": (_I32, [_P]),
    "dory_kv_length": (_I64, [_P]),
    "dory_kv_slot": (_I32, [_P, _I32, _I32, ctypes.POINTER(dory_kv_slot_info)]),
    "dory_prefill": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _SZ, _P, _P, _P, _P, _P]),
    "dory_decode_step": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _SZ, _P, _P, _P, _P, _P]),
    "dory_decode_step_noalloc": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "dory_prefill_rows": (_I32, [_P, _P, _P, _I32, _I32, _P, _I32, _P, _SZ, _P, _P, _P, _P, _P]),
    "dory_decode_step_rows": (_I32, [_P, _P, _P, _I32, _P, _I32, _P, _SZ, _P, _P, _P, _P, _P]),
    "dory_greedy": (_I32, [_P, _I32, _I32, _P, _P]),
    "dory_debug_kv_slots": (_I32, [_P, _I32, _I64, _I64, _P, _P]),
    "dory_debug_attention": (_I32, [_P, _P, _I32, _I32, _I64, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dory_debug_mask": (_I32, [_P, _P, _I32, _I32, _I64, _I32, _P, _SZ, _P, _P]),
    "dory_kv_set_length": (_I32, [_P, _I64]),
    "dory_kv_copy_prefix": (_I32, [_P, _I32, _P, _I32, _I64, _P]),
    "dory_profile_begin": (_I32, [_P, _I32]),
    "dory_profile_end": (_I32, [_P, ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double)]),
    "dory_selfspec_step": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _SZ, _P, _P,
                                  ctypes.POINTER(_I32), _P]),
    "dory_sample": (_I32, [_P, _I32, _I32, ctypes.c_float, _P, _P, _P]),
    "dory_speculative_accept": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, ctypes.c_float, _P, _P, _P]),
    "dory_selfspec_step_sampled": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                                          _P, _P, _SZ, _P, _P, _P, ctypes.POINTER(_I32), _P]),
    "dory_mxfp8_quantize": (_I32, [_P, _I64, _I32, _P, _P, _P, _P]),
    "dory_mxfp8_bytes": (_SZ, [ctypes.POINTER(dory_config)]),
    "dory_model_quantize_mxfp8": (_I32, [_P, _P, _SZ, _P]),
    "dory_model_use_mxfp8": (_I32, [_P, _I32]),
    "dory_model_set_decode_graphs": (_I32, [_P, _I32]),
    "dory_status_string": (ctypes.c_char_p, [_I32]),
    "dory_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libdory.so not found at %s: build it with "
                "`python -m looped_ngpt_transformer_fwd_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class DoryError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        L = lib()
        msg = "%s: %s (%s)" % (where, L.dory_status_string(status).decode(),
                               L.dory_last_error().decode())
        super().__init__(msg)


def check(status, where):
    if status != DORY_OK:
        raise DoryError(status, where)
    return status


# Thin wrappers with the C names (status returned, not raised).
def dory_model_create(cfg, w, out):
    return lib().dory_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(out))


def dory_model_destroy(m):
    lib().dory_model_destroy(m)


def dory_schedule(cfg, kinds_out, capacity):
    return lib().dory_schedule(ctypes.byref(cfg), kinds_out, capacity)


def dory_kv_bytes(cfg, mode, k_max, batch, max_seq):
    return lib().dory_kv_bytes(ctypes.byref(cfg), mode, k_max, batch, max_seq)


def dory_workspace_bytes(cfg, batch, tokens):
    return lib().dory_workspace_bytes(ctypes.byref(cfg), batch, tokens)


def dory_kv_bind(m, buf, nbytes, mode, k_max, batch, max_seq, out):
    return lib().dory_kv_bind(m, buf, nbytes, mode, k_max, batch, max_seq, ctypes.byref(out))


def dory_kv_destroy(kv):
    lib().dory_kv_destroy(kv)


def dory_kv_reset(kv):
    return lib().dory_kv_reset(kv)


def dory_kv_length(kv):
    return lib().dory_kv_length(kv)


def dory_kv_slot(kv, sublayer, loop, out):
    return lib().dory_kv_slot(kv, sublayer, loop, ctypes.byref(out))


def dory_prefill(m, kv, tokens, B, T, k, mode, ws, ws_bytes, logits, nxt, hidden, states, stream):
    return lib().dory_prefill(m, kv, tokens, B, T, k, mode, ws, ws_bytes, logits, nxt, hidden,
                              states, stream)


def dory_decode_step(m, kv, tokens, B, k, mode, ws, ws_bytes, logits, nxt, hidden, states, stream):
    return lib().dory_decode_step(m, kv, tokens, B, k, mode, ws, ws_bytes, logits, nxt, hidden,
                                  states, stream)


def dory_decode_step_noalloc(m, kv, tokens, B, k, mode, logits, nxt, hidden, states, stream):
    return lib().dory_decode_step_noalloc(m, kv, tokens, B, k, mode, logits, nxt, hidden, states,
                                          stream)


NOALLOC_SCRATCH_BYTES = 256 << 20
DORY_KV_ROLLBACK = 64        # positions a cache can be shortened by (sliding-window rings)


def dory_prefill_rows(m, kv, tokens, B, T, k_rows, mode, ws, ws_bytes, logits, nxt, hidden, states,
                      stream):
    return lib().dory_prefill_rows(m, kv, tokens, B, T, k_rows, mode, ws, ws_bytes, logits, nxt,
                                   hidden, states, stream)


def dory_decode_step_rows(m, kv, tokens, B, k_rows, mode, ws, ws_bytes, logits, nxt, hidden,
                          states, stream):
    return lib().dory_decode_step_rows(m, kv, tokens, B, k_rows, mode, ws, ws_bytes, logits, nxt,
                                       hidden, states, stream)


def dory_greedy(logits, rows, n, out, stream):
    return lib().dory_greedy(logits, rows, n, out, stream)


def dory_debug_kv_slots(kv, sublayer, pos_a, n, rows_out, stream):
    return lib().dory_debug_kv_slots(kv, sublayer, pos_a, n, rows_out, stream)


def dory_debug_attention(m, kv, sublayer, loop, p0, T, q_hat, k_new, v_new, gate, z, ws, ws_bytes,
                         stream):
    return lib().dory_debug_attention(m, kv, sublayer, loop, p0, T, q_hat, k_new, v_new, gate, z, ws,
                                      ws_bytes, stream)


def dory_debug_mask(m, kv, sublayer, loop, p0, T, ws, ws_bytes, out, stream):
    return lib().dory_debug_mask(m, kv, sublayer, loop, p0, T, ws, ws_bytes, out, stream)


def dory_kv_set_length(kv, length):
    return lib().dory_kv_set_length(kv, length)


def dory_kv_copy_prefix(src, src_seq, dst, dst_seq, n, stream):
    return lib().dory_kv_copy_prefix(src, src_seq, dst, dst_seq, n, stream)


def dory_selfspec_step(m, kv, last, B, gamma, k_draft, k_verify, mode, ws, ws_bytes, scratch, out,
                       n_accepted, stream):
    return lib().dory_selfspec_step(m, kv, last, B, gamma, k_draft, k_verify, mode, ws, ws_bytes,
                                    scratch, out, ctypes.byref(n_accepted), stream)


def dory_sample(logits, rows, V, temperature, u, out, stream):
    return lib().dory_sample(logits, rows, V, temperature, u, out, stream)


def dory_speculative_accept(draft_logits, verify_logits, drafts, u, B, V, gamma, temperature,
                            n_accepted, out, stream):
    return lib().dory_speculative_accept(draft_logits, verify_logits, drafts, u, B, V, gamma,
                                         temperature, n_accepted, out, stream)


def dory_selfspec_step_sampled(m, kv, last, B, gamma, k_draft, k_verify, mode, temperature, u, ws,
                               ws_bytes, scratch, logits_buf, out, n_accepted, stream):
    return lib().dory_selfspec_step_sampled(m, kv, last, B, gamma, k_draft, k_verify, mode,
                                            temperature, u, ws, ws_bytes, scratch, logits_buf, out,
                                            ctypes.byref(n_accepted), stream)


def dory_mxfp8_quantize(w, rows, cols, codes, scales, deq, stream):
    return lib().dory_mxfp8_quantize(w, rows, cols, codes, scales, deq, stream)


def dory_mxfp8_bytes(cfg):
    return lib().dory_mxfp8_bytes(ctypes.byref(cfg))


def dory_model_quantize_mxfp8(m, buf, nbytes, stream):
    return lib().dory_model_quantize_mxfp8(m, buf, nbytes, stream)


def dory_model_use_mxfp8(m, on):
    return lib().dory_model_use_mxfp8(m, on)


def dory_model_set_decode_graphs(m, on):
    return lib().dory_model_set_decode_graphs(m, on)


DORY_K_NUM_CLASSES = 10
KERNEL_CLASSES = ["gemm_qkvg", "gemm_o", "gemm_upgate", "gemm_down", "gemm_lm", "attn", "qk",
                  "update", "kv_write", "other"]


def dory_profile_begin(m, max_launches):
    return lib().dory_profile_begin(m, max_launches)


def dory_profile_end(m, counts, ms):
    return lib().dory_profile_end(m, counts, ms)


def dory_status_string(s):
    return lib().dory_status_string(s).decode()


def dory_last_error():
    return lib().dory_last_error().decode()
