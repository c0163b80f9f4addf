"""ctypes binding of the C ABI in include/dualflow.h (argument marshalling only).

Every function here has the name and argument order of its C counterpart;
device pointers are passed as Python ints, `stream` as a hipStream_t value
(int, 0 = default stream). The library is loaded from the package directory;
if it is missing the import fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdualflow.so")

DF_OK = 0
DF_ERR_NULL = -1
DF_ERR_SHAPE = -2
DF_ERR_DTYPE = -3
DF_ERR_ALIGN = -4
DF_ERR_WORKSPACE = -5
DF_ERR_KV_FULL = -6
DF_ERR_HIP = -7
DF_ERR_ARG = -8
DF_F32 = 0
DF_BF16 = 1
DF_VARIANT_NO_COUPLING = 1
DF_VARIANT_AUX_OUTPUT = 2
DF_VARIANT_ALPHA_HALF = 4
DF_MIX_PRIMARY, DF_MIX_COLLISION, DF_MIX_AUX, DF_MIX_HALF = 0, 1, 2, 3

EXPORTS = ["df_workspace_bytes", "df_prefill_workspace_bytes", "df_forward_workspace_bytes", "df_forward_dual",
           "df_decode_step", "df_prefill_primary", "df_kv_append", "df_mix_head",
           "df_attention_dual", "df_attention_workspace_bytes", "df_device_status", "df_status_str",
           "df_timing_enable", "df_timing_read", "df_stacked_gemv", "df_stacked_gemv_workspace_bytes",
           "df_pack_weights", "df_attention_dual_noalloc", "df_stream_read"]
DF_ATTENTION_NOALLOC_SCRATCH_BYTES = 17040384
DF_STREAM_READ_OUT_WORDS = 4096


class df_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("expert_ffn", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("variant", ctypes.c_int32), ("top_k_aux", ctypes.c_int32),
                ("prefill_rows", ctypes.c_int32)]


class df_weights(ctypes.Structure):
    _fields_ = [("tok_emb", ctypes.c_void_p * 2), ("pos_emb", ctypes.c_void_p), ("ln1", ctypes.c_void_p),
                ("ln2", ctypes.c_void_p), ("lnf", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("w_router", ctypes.c_void_p), ("w_exp_up", ctypes.c_void_p), ("w_exp_down", ctypes.c_void_p),
                ("cpl_a", ctypes.c_void_p), ("cpl_b", ctypes.c_void_p), ("cpl_c", ctypes.c_void_p),
                ("w_out", ctypes.c_void_p)]


class df_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m dual_flow_transformer_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.df_workspace_bytes.restype = sz
        L.df_workspace_bytes.argtypes = [P(df_config)]
        L.df_prefill_workspace_bytes.restype = sz
        L.df_prefill_workspace_bytes.argtypes = [P(df_config)]
        L.df_forward_workspace_bytes.restype = sz
        L.df_forward_workspace_bytes.argtypes = [P(df_config)]
        L.df_forward_dual.restype = ctypes.c_int
        L.df_forward_dual.argtypes = [P(df_config), P(df_weights), P(df_kv), vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.df_decode_step.restype = ctypes.c_int
        L.df_decode_step.argtypes = [P(df_config), P(df_weights), P(df_kv), vp, i32, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]
        L.df_prefill_primary.restype = ctypes.c_int
        L.df_prefill_primary.argtypes = [P(df_config), P(df_weights), P(df_kv), vp, i32, vp, sz, vp]
        L.df_kv_append.restype = ctypes.c_int
        L.df_kv_append.argtypes = [P(df_config), P(df_kv), i32, vp, vp, vp, vp, vp]
        L.df_mix_head.restype = ctypes.c_int
        L.df_mix_head.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.df_attention_dual.restype = ctypes.c_int
        L.df_attention_dual.argtypes = [i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.df_attention_dual_noalloc.restype = ctypes.c_int
        L.df_attention_dual_noalloc.argtypes = [i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.df_attention_workspace_bytes.restype = sz
        L.df_attention_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.df_device_status.restype = ctypes.c_int
        L.df_device_status.argtypes = [vp, vp, P(i32)]
        L.df_status_str.restype = ctypes.c_char_p
        L.df_status_str.argtypes = [ctypes.c_int]
        L.df_stacked_gemv.restype = ctypes.c_int
        L.df_stacked_gemv.argtypes = [i32, vp, vp, i32, i32, i32, vp, vp, sz, vp]
        L.df_stacked_gemv_workspace_bytes.restype = sz
        L.df_stacked_gemv_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.df_pack_weights.restype = ctypes.c_int
        L.df_pack_weights.argtypes = [i32, vp, vp, ctypes.c_int64, i32, i32, vp]
        L.df_stream_read.restype = ctypes.c_int
        L.df_stream_read.argtypes = [vp, sz, vp, vp]
        L.df_timing_enable.restype = ctypes.c_int
        L.df_timing_enable.argtypes = [i32, i32]
        L.df_timing_read.restype = ctypes.c_int
        L.df_timing_read.argtypes = [P(ctypes.c_double), P(ctypes.c_int64)]
        _lib = L
    return _lib


class DFError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {df_status_str(code)} ({code})")
        self.code = code


def check(code: int, where: str) -> int:
    if code != DF_OK:
        raise DFError(code, where)
    return code


def df_workspace_bytes(cfg: df_config) -> int:
    return int(lib().df_workspace_bytes(ctypes.byref(cfg)))


def df_prefill_workspace_bytes(cfg: df_config) -> int:
    return int(lib().df_prefill_workspace_bytes(ctypes.byref(cfg)))


def df_forward_workspace_bytes(cfg: df_config) -> int:
    return int(lib().df_forward_workspace_bytes(ctypes.byref(cfg)))


def df_forward_dual(cfg, w, kv, d_tokens, T, d_logits, d_p_mix, d_alpha, d_next_tok, d_ws, ws_bytes, stream=0) -> int:
    return lib().df_forward_dual(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), d_tokens, int(T), d_logits,
                                 d_p_mix, d_alpha, d_next_tok, d_ws, ws_bytes, stream)


def df_decode_step(cfg, w, kv, d_tokens, aux_on, d_router_logits, d_logits, d_p_mix, d_alpha, d_next_tok,
                   d_expert_ids, d_ws, ws_bytes, stream=0) -> int:
    return lib().df_decode_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), d_tokens, int(aux_on),
                                d_router_logits, d_logits, d_p_mix, d_alpha, d_next_tok, d_expert_ids, d_ws,
                                ws_bytes, stream)


def df_prefill_primary(cfg, w, kv, d_tokens, T, d_ws, ws_bytes, stream=0) -> int:
    return lib().df_prefill_primary(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), d_tokens, int(T), d_ws,
                                    ws_bytes, stream)


def df_kv_append(cfg, kv, layer, d_pos, d_k, d_v, d_status=None, stream=0) -> int:
    return lib().df_kv_append(ctypes.byref(cfg), ctypes.byref(kv), int(layer), d_pos, d_k, d_v, d_status, stream)


def df_mix_head(d_logits, batch, vocab, mode, d_p_mix, d_alpha, d_next_tok=None, stream=0) -> int:
    return lib().df_mix_head(d_logits, int(batch), int(vocab), int(mode), d_p_mix, d_alpha, d_next_tok, stream)


def df_attention_dual(dtype, d_k, d_v, batch, n_heads, max_seq, head_dim, d_len, d_q, d_a, d_o, d_lse, d_ws,
                      ws_bytes, stream=0) -> int:
    return lib().df_attention_dual(int(dtype), d_k, d_v, int(batch), int(n_heads), int(max_seq), int(head_dim),
                                   d_len, d_q, d_a, d_o, d_lse, d_ws, ws_bytes, stream)


def df_attention_dual_noalloc(dtype, d_k, d_v, batch, n_heads, max_seq, head_dim, d_len, d_q, d_a, d_o, d_lse,
                              stream=0) -> int:
    return lib().df_attention_dual_noalloc(int(dtype), d_k, d_v, int(batch), int(n_heads), int(max_seq),
                                           int(head_dim), d_len, d_q, d_a, d_o, d_lse, stream)


def df_attention_workspace_bytes(batch, n_heads, max_seq, head_dim) -> int:
    return int(lib().df_attention_workspace_bytes(int(batch), int(n_heads), int(max_seq), int(head_dim)))


def df_device_status(d_ws, stream=0):
    out = ctypes.c_int32(0)
    rc = lib().df_device_status(d_ws, stream, ctypes.byref(out))
    return rc, int(out.value)


def df_status_str(code: int) -> str:
    return lib().df_status_str(int(code)).decode()


def df_stacked_gemv(dtype, d_x, d_w, rows, N, K, d_y, d_ws, ws_bytes, stream=0) -> int:
    return lib().df_stacked_gemv(int(dtype), d_x, d_w, int(rows), int(N), int(K), d_y, d_ws, ws_bytes, stream)


def df_stacked_gemv_workspace_bytes(dtype, rows, N, K) -> int:
    return int(lib().df_stacked_gemv_workspace_bytes(int(dtype), int(rows), int(N), int(K)))


def df_pack_weights(dtype, d_src, d_dst, n_mats, rows, cols, stream=0) -> int:
    return lib().df_pack_weights(int(dtype), d_src, d_dst, int(n_mats), int(rows), int(cols), stream)


def df_stream_read(d_src, nbytes, d_out, stream=0) -> int:
    return lib().df_stream_read(d_src, nbytes, d_out, stream)


def df_timing_enable(kclass: int = 0, stride: int = 1) -> int:
    return lib().df_timing_enable(int(kclass), int(stride))


def df_timing_read():
    t = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    rc = lib().df_timing_read(ctypes.byref(t), ctypes.byref(n))
    return rc, float(t.value), int(n.value)
