"""Thin ctypes binding over libmla.so (include/mla.h).  Argument marshalling only.

Device memory and streams come from PyTorch (torch tensors on a HIP device and
torch.cuda.current_stream()).  Every step of the computation runs in libmla's HIP kernels;
if the library is missing this module raises instead of computing anything itself.
"""
import ctypes
import os

import torch

from .configs import PAGE_SIZE

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
TORCH_ACT = {"f32": torch.float32, "bf16": torch.bfloat16}
TORCH_CACHE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_WORKSPACE", 4: "MLA_ERR_HIP"}

# Every function include/mla.h declares, with (restype, argtypes).
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


class MlaConfig(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("q_lora_rank", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_nope_head_dim", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("rope_factor", ctypes.c_float), ("rope_original_max_position", ctypes.c_int32),
                ("rope_beta_fast", ctypes.c_float), ("rope_beta_slow", ctypes.c_float),
                ("rope_mscale", ctypes.c_float), ("prefill_key_block", ctypes.c_int32)]


class MlaWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q_a_proj", "q_a_norm", "q_b_proj", "kv_a_proj", "kv_a_norm", "kv_b_proj", "o_proj")]


class MlaCache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("num_blocks", ctypes.c_int32)]


_P = ctypes.POINTER
SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_compress_append_workspace_size": (_sz, [_P(MlaConfig), _i32]),
    "mla_compress_append": (ctypes.c_int, [_P(MlaConfig), _P(MlaWeights), _vp, _vp, _vp, _P(MlaCache), _i32,
                                           _vp, _sz, _vp]),
    "mla_decode_num_splits": (_i32, [_P(MlaConfig), _i32, _i32]),
    "mla_decode_workspace_size": (_sz, [_P(MlaConfig), _i32, _i32, _i32]),
    "mla_decode": (ctypes.c_int, [_P(MlaConfig), _P(MlaWeights), _vp, _vp, _vp, _i32, _P(MlaCache), _i32, _i32,
                                  _vp, _sz, _vp, _vp]),
    "mla_decode_timed": (ctypes.c_int, [_P(MlaConfig), _P(MlaWeights), _vp, _vp, _vp, _i32, _P(MlaCache), _i32,
                                        _i32, _vp, _sz, _vp, _vp, _vp, _vp]),
    "mla_fp8_e4m3_encode": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, _vp]),
    "mla_fp8_e4m3_decode": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, _vp]),
    "mla_decode_noalloc": (ctypes.c_int, [_P(MlaConfig), _P(MlaWeights), _vp, _vp, _vp, _i32, _P(MlaCache), _i32,
                                          _i32, _vp, _vp]),
    "mla_stream_read": (ctypes.c_int, [_vp, _sz, _vp, ctypes.c_int, _vp]),
    "mla_prefill_workspace_size": (_sz, [_P(MlaConfig), _i32, _i32, _i32, _i32]),
    "mla_prefill": (ctypes.c_int, [_P(MlaConfig), _P(MlaWeights), _vp, _vp, _vp, _vp, _i32, _P(MlaCache), _i32,
                                   _i32, _i32, _i32, _vp, _sz, _vp, _vp]),
}

_lib = None


def lib():
    """Load libmla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mla_latent_kv_compress_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _lib = h
    return _lib


class MLAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({lib().mla_status_string(status).decode()})")


def _check(status, where):
    if status != 0:
        raise MLAError(status, where)


def make_config(shape, act_dtype, cache_dtype, out_dtype="f32"):
    return MlaConfig(shape.hidden_size, shape.num_heads, shape.q_lora_rank, shape.kv_lora_rank,
                     shape.qk_nope_head_dim, shape.qk_rope_head_dim, shape.v_head_dim, PAGE_SIZE,
                     shape.rope_theta, shape.rms_eps, shape.softmax_scale,
                     DTYPE_CODES[act_dtype], DTYPE_CODES[cache_dtype], DTYPE_CODES[out_dtype],
                     shape.rope_factor, shape.rope_original_max_position, shape.rope_beta_fast,
                     shape.rope_beta_slow, shape.rope_mscale)


TORCH_OUT = {0: torch.float32, 1: torch.bfloat16}


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libmla must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmla must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def make_weights(w):
    """MlaWeights from a dict of device tensors (q_proj may stand in for q_b_proj)."""
    q_b = w.get("q_b_proj", w.get("q_proj"))
    return MlaWeights(*[_ptr(x) for x in (w.get("q_a_proj"), w.get("q_a_norm"), q_b,
                                         w["kv_a_proj"], w["kv_a_norm"], w["kv_b_proj"], w.get("o_proj"))])


def out_shape(cfg, weights, tokens):
    """Shape of decode / prefill output: [tokens, hidden] with o_proj, else [tokens, H, v_head_dim]."""
    has_o = (weights.o_proj is not None) if isinstance(weights, MlaWeights) else weights.get("o_proj") is not None
    return (tokens, cfg.hidden_size) if has_o else (tokens, cfg.num_heads, cfg.v_head_dim)


class Cache:
    """A paged latent cache: data [num_blocks, 64, kv_lora_rank + rope] (+ fp32 scales for fp8)."""

    def __init__(self, shape, cache_dtype, num_blocks, device="cuda", fill=None):
        self.dtype = cache_dtype
        W = shape.row_width
        self.data = torch.empty((num_blocks, PAGE_SIZE, W), dtype=TORCH_CACHE[cache_dtype], device=device)
        if fill is not None:
            self.data.view(torch.uint8).fill_(fill)
        self.scale = (torch.zeros((num_blocks, PAGE_SIZE), dtype=torch.float32, device=device)
                      if cache_dtype == "fp8" else None)
        self.num_blocks = num_blocks

    def struct(self):
        return MlaCache(_ptr(self.data), _ptr(self.scale) if self.scale is not None else None, self.num_blocks)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def compress_append(cfg, weights, hidden, positions, slot_mapping, cache, workspace=None, stream=None):
    L = lib()
    T = hidden.shape[0]
    nbytes = L.mla_compress_append_workspace_size(ctypes.byref(cfg), T)
    ws = _workspace(nbytes, hidden.device, workspace)
    W = make_weights(weights)
    cs = cache.struct()
    _check(L.mla_compress_append(ctypes.byref(cfg), ctypes.byref(W), _ptr(hidden), _ptr(positions),
                                 _ptr(slot_mapping), ctypes.byref(cs), T, _ptr(ws), nbytes, _stream(stream)),
           "mla_compress_append")
    return ws


def decode_num_splits(cfg, batch, max_blocks):
    return lib().mla_decode_num_splits(ctypes.byref(cfg), batch, max_blocks)


def decode_workspace_size(cfg, batch, max_blocks, num_splits=0):
    return lib().mla_decode_workspace_size(ctypes.byref(cfg), batch, max_blocks, num_splits)


def decode(cfg, weights, hidden, context_lens, block_table, cache, num_splits=0, out=None, workspace=None,
           stream=None, weights_struct=None, attn_events=None):
    """attn_events: optional (begin, end) hipEvent_t handles recorded around the attention kernel."""
    L = lib()
    B, max_blocks = block_table.shape
    nbytes = L.mla_decode_workspace_size(ctypes.byref(cfg), B, max_blocks, num_splits)
    ws = _workspace(nbytes, hidden.device, workspace)
    W = weights_struct if weights_struct is not None else make_weights(weights)
    if out is None:
        out = torch.empty(out_shape(cfg, W, B), dtype=TORCH_OUT[cfg.out_dtype], device=hidden.device)
    cs = cache.struct()
    if attn_events is None:
        _check(L.mla_decode(ctypes.byref(cfg), ctypes.byref(W), _ptr(hidden), _ptr(context_lens),
                            _ptr(block_table), max_blocks, ctypes.byref(cs), B, num_splits, _ptr(ws), nbytes,
                            _ptr(out), _stream(stream)), "mla_decode")
    else:
        _check(L.mla_decode_timed(ctypes.byref(cfg), ctypes.byref(W), _ptr(hidden), _ptr(context_lens),
                                  _ptr(block_table), max_blocks, ctypes.byref(cs), B, num_splits, _ptr(ws), nbytes,
                                  _ptr(out), _stream(stream), ctypes.c_void_p(attn_events[0]),
                                  ctypes.c_void_p(attn_events[1])), "mla_decode_timed")
    return out


def decode_noalloc(cfg, weights, hidden, context_lens, block_table, cache, num_splits=0, out=None, stream=None):
    """mla_decode_noalloc: the decode step on the library's static per-GPU workspace."""
    L = lib()
    B, max_blocks = block_table.shape
    W = make_weights(weights)
    if out is None:
        out = torch.empty(out_shape(cfg, W, B), dtype=TORCH_OUT[cfg.out_dtype], device=hidden.device)
    cs = cache.struct()
    _check(L.mla_decode_noalloc(ctypes.byref(cfg), ctypes.byref(W), _ptr(hidden), _ptr(context_lens),
                                _ptr(block_table), max_blocks, ctypes.byref(cs), B, num_splits, _ptr(out),
                                _stream(stream)), "mla_decode_noalloc")
    return out


def prefill_workspace_size(cfg, num_seqs, total_tokens, max_q_len, max_ctx):
    return lib().mla_prefill_workspace_size(ctypes.byref(cfg), num_seqs, total_tokens, max_q_len, max_ctx)


def prefill(cfg, weights, hidden, cu_seqlens, start_pos, block_table, cache, max_q_len, max_ctx, out=None,
            workspace=None, stream=None):
    L = lib()
    T = hidden.shape[0]
    S, max_blocks = block_table.shape
    nbytes = L.mla_prefill_workspace_size(ctypes.byref(cfg), S, T, max_q_len, max_ctx)
    ws = _workspace(nbytes, hidden.device, workspace)
    W = make_weights(weights)
    if out is None:
        out = torch.empty(out_shape(cfg, W, T), dtype=TORCH_OUT[cfg.out_dtype], device=hidden.device)
    cs = cache.struct()
    _check(L.mla_prefill(ctypes.byref(cfg), ctypes.byref(W), _ptr(hidden), _ptr(cu_seqlens), _ptr(start_pos),
                         _ptr(block_table), max_blocks, ctypes.byref(cs), S, T, max_q_len, max_ctx, _ptr(ws),
                         nbytes, _ptr(out), _stream(stream)),
           "mla_prefill")
    return out


def stream_read(src, sink, mode=0, stream=None):
    """mla_stream_read: read all of `src` (a contiguous device tensor) once and discard it; mode 0
    plain cached loads (a cache sweep), mode 1 the non-temporal direct-to-LDS read (the bandwidth
    reference)."""
    _check(lib().mla_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), int(mode),
                                 _stream(stream)), "mla_stream_read")
