"""Thin ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels; this module only
turns torch device tensors into pointers, picks torch's current HIP stream and
maps status codes to exceptions.  It raises ImportError if the built library
is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_ENOMEM, KVQ_ECAPACITY, KVQ_ESTATE, KVQ_EHIP = range(6)
KVQ_F16, KVQ_F32 = 0, 1
CODEC_BGTQ, CODEC_UNIFORM, CODEC_NF16_B256, CODEC_UNIFORM_ROT, CODEC_KIVI, CODEC_BGTQ_ROT = 0, 1, 2, 3, 4, 5
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
PART_K_CODES, PART_V_CODES, PART_K_SCALES, PART_V_SCALES, PART_K_RECENT, PART_V_RECENT = range(6)

EXPORTED = (
    "kvq_cache_create", "kvq_cache_destroy", "kvq_alloc_bits", "kvq_get_plan",
    "kvq_quantize_append", "kvq_decode_attn", "kvq_decode_attn_splits", "kvq_key_fidelity", "kvq_set_rotation", "kvq_seq_len",
    "kvq_layer_info_get", "kvq_read_cache", "kvq_codebook", "kvq_delta",
    "kvq_nf16_codebook", "kvq_status_str", "kvq_last_error", "kvq_cache_status", "kvq_cache_view",
    "kvq_decode_attn_noalloc", "kvq_probe_stream_read", "kvq_decode_step",
)

PLAN_BYTES, PLAN_OFF_GAIN, PLAN_OFF_FIELD_DIM, PLAN_OFF_FIELD_WIDTH = 2256, 0, 1280, 1408
PLAN_OFF_BLOCK_WIDTH, PLAN_OFF_N_FIELDS = 1664, 2240


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__(f"{what}: {_status_name(status)}" + (f" ({detail})" if detail else ""))


class kvq_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("batch", ctypes.c_int32), ("max_tokens", ctypes.c_int64),
        ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("b_min", ctypes.c_int32),
        ("b_max", ctypes.c_int32), ("codec", ctypes.c_int32), ("pairing", ctypes.c_int32),
        ("recent_window", ctypes.c_int32), ("per_sequence_plans", ctypes.c_int32),
    ]


class kvq_layer_info(ctypes.Structure):
    _fields_ = [
        ("capacity", ctypes.c_int64), ("len", ctypes.c_int64), ("k_row_words", ctypes.c_int32),
        ("v_dim_words", ctypes.c_int32), ("k_codes_bytes", ctypes.c_int64),
        ("v_codes_bytes", ctypes.c_int64), ("k_scales_bytes", ctypes.c_int64),
        ("v_scales_bytes", ctypes.c_int64), ("plan_ready", ctypes.c_int32),
        ("recent_window", ctypes.c_int32), ("packed_len", ctypes.c_int64), ("recent_bytes", ctypes.c_int64),
        ("ring_slots", ctypes.c_int32),
    ]


class kvq_view(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p), ("k_codes_strides", ctypes.c_int64 * 3),
        ("v_codes", ctypes.c_void_p), ("v_codes_strides", ctypes.c_int64 * 3),
        ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p), ("scale_strides", ctypes.c_int64 * 3),
        ("k_recent", ctypes.c_void_p), ("v_recent", ctypes.c_void_p), ("plans", ctypes.c_void_p),
        ("n_plans", ctypes.c_int32), ("plan_bytes", ctypes.c_int32), ("capacity", ctypes.c_int64),
        ("len", ctypes.c_int64), ("packed_len", ctypes.c_int64),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libkvq.so not built at {_LIB_PATH}; run __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "kvq_cache_create": (I32, [ctypes.POINTER(kvq_config), ctypes.POINTER(P)]),
        "kvq_cache_destroy": (None, [P]),
        "kvq_alloc_bits": (I32, [P, I32, P, I32, I64, P, P]),
        "kvq_get_plan": (I32, [P, I32, P, P]),
        "kvq_quantize_append": (I32, [P, I32, P, P, I32, I64, P]),
        "kvq_decode_attn": (I32, [P, I32, P, I32, F32, P, P]),
        "kvq_decode_attn_splits": (I32, [P, I32, P, I32, F32, P, I32, P]),
        "kvq_key_fidelity": (I32, [P, I32, P, P, I32, F32, P, P, P]),
        "kvq_set_rotation": (I32, [P, I32, P]),
        "kvq_seq_len": (I32, [P, I32, ctypes.POINTER(I64)]),
        "kvq_layer_info_get": (I32, [P, I32, ctypes.POINTER(kvq_layer_info)]),
        "kvq_read_cache": (I32, [P, I32, I32, I64, I64, P]),
        "kvq_codebook": (I32, [I32, P, P]),
        "kvq_delta": (I32, [P]),
        "kvq_nf16_codebook": (I32, [P, P]),
        "kvq_status_str": (ctypes.c_char_p, [I32]),
        "kvq_last_error": (ctypes.c_char_p, []),
        "kvq_cache_status": (I32, [P]),
        "kvq_cache_view": (I32, [P, I32, ctypes.POINTER(kvq_view)]),
        "kvq_decode_attn_noalloc": (I32, [P, I32, P, I32, F32, P, P]),
        "kvq_probe_stream_read": (I32, [P, I64, I32, P, P]),
        "kvq_decode_step": (I32, [P, I32, P, P, P, I32, F32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _status_name(s: int) -> str:
    return lib.kvq_status_str(s).decode()


def _check(status: int, what: str):
    if status != KVQ_OK:
        detail = lib.kvq_last_error().decode() if status == KVQ_EHIP else ""
        raise KvqError(status, what, detail)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int:
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ---- host-only constant tables --------------------------------------------------------------

def codebook(bits: int):
    """(fp16 centroids as np.float16[2^bits], fp32 boundaries[2^bits - 1]) from the library."""
    cb = np.zeros(1 << bits, dtype=np.uint16)
    bd = np.zeros((1 << bits) - 1, dtype=np.float32)
    _check(lib.kvq_codebook(bits, cb.ctypes.data, bd.ctypes.data), "kvq_codebook")
    return cb.view(np.float16), bd


def delta():
    d = np.zeros(8, dtype=np.float32)
    _check(lib.kvq_delta(d.ctypes.data), "kvq_delta")
    return d


def nf16_codebook():
    lv = np.zeros(16, dtype=np.uint16)
    bd = np.zeros(15, dtype=np.float32)
    _check(lib.kvq_nf16_codebook(lv.ctypes.data, bd.ctypes.data), "kvq_nf16_codebook")
    return lv.view(np.float16), bd


def probe_stream_read(src, n_blocks: int, sink, stream=None):
    """One streaming-read launch over the bytes of the GPU tensor `src` (a measurement aid)."""
    _check(lib.kvq_probe_stream_read(_ptr(src), src.numel() * src.element_size(), int(n_blocks), _ptr(sink),
                                     _stream(stream)), "kvq_probe_stream_read")


# ---- cache -----------------------------------------------------------------------------------

@dataclass
class Config:
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    batch: int
    max_tokens: int
    k_bits: int
    v_bits: int
    head_dim: int = 128
    b_min: int = 0
    b_max: int = 8
    codec: int = CODEC_BGTQ
    pairing: int = ROPE_HALF
    recent_window: int = 0
    per_sequence_plans: int = 0

    def to_c(self) -> kvq_config:
        return kvq_config(self.n_layers, self.n_kv_heads, self.n_q_heads, self.head_dim, self.batch,
                          self.max_tokens, self.k_bits, self.v_bits, self.b_min, self.b_max,
                          self.codec, self.pairing, self.recent_window, self.per_sequence_plans)


def create_status(cfg: Config) -> int:
    """Raw status of kvq_cache_create (the cache is destroyed right away on success)."""
    h = ctypes.c_void_p()
    c = cfg.to_c()
    st = lib.kvq_cache_create(ctypes.byref(c), ctypes.byref(h))
    if st == KVQ_OK:
        lib.kvq_cache_destroy(h)
    return st


class Cache:
    """Owns one kvq_cache; all tensor arguments are torch GPU tensors."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self._h = ctypes.c_void_p()
        c = cfg.to_c()
        _check(lib.kvq_cache_create(ctypes.byref(c), ctypes.byref(self._h)), "kvq_cache_create")

    def close(self):
        if self._h:
            lib.kvq_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def alloc_bits(self, layer: int, keys=None, block_weight=None, stream=None):
        """keys: [n_tok, n_kv_heads, head_dim], or [batch, n_tok, n_kv_heads, head_dim] with
        per-sequence plans; block_weight: fp64 [(batch,) n_kv_heads, 64] or None."""
        per_seq = bool(self.cfg.per_sequence_plans)
        if keys is not None:
            lead = (self.cfg.batch,) if per_seq else ()
            if keys.dim() != len(lead) + 3 or tuple(keys.shape[:len(lead)]) != lead \
                    or tuple(keys.shape[-2:]) != (self.cfg.n_kv_heads, self.cfg.head_dim):
                raise ValueError(f"keys must be [{'batch, ' if per_seq else ''}n_tok, n_kv_heads, head_dim], "
                                 f"got {tuple(keys.shape)}")
        kp = _ptr(keys) if keys is not None else None
        dt = _dtype_code(keys) if keys is not None else KVQ_F16
        n = keys.shape[-3] if keys is not None else 0
        wp = None
        if block_weight is not None:
            import torch
            want = lead + (self.cfg.n_kv_heads, 64) if keys is not None else \
                ((self.cfg.batch,) if per_seq else ()) + (self.cfg.n_kv_heads, 64)
            if block_weight.dtype != torch.float64 or tuple(block_weight.shape) != want:
                raise ValueError(f"block_weight must be float64 of shape {want}, got "
                                 f"{block_weight.dtype} {tuple(block_weight.shape)}")
            wp = _ptr(block_weight)
        _check(lib.kvq_alloc_bits(self._h, layer, kp, dt, n, wp, _stream(stream)), "kvq_alloc_bits")

    def set_rotation(self, layer: int, signs):
        """Key-rotation signs of `layer` (codecs CODEC_UNIFORM_ROT, CODEC_BGTQ_ROT): int8
        [n_kv_heads, 128] of +-1, indexed by dim."""
        sg = np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
        if sg.shape != (self.cfg.n_kv_heads, self.cfg.head_dim):
            raise ValueError(f"signs must be [n_kv_heads, head_dim], got {sg.shape}")
        _check(lib.kvq_set_rotation(self._h, layer, sg.ctypes.data), "kvq_set_rotation")

    def get_plan(self, layer: int):
        shape = ((self.cfg.batch,) if self.cfg.per_sequence_plans else ()) + (self.cfg.n_kv_heads, 64)
        bits = np.zeros(shape, dtype=np.int8)
        gains = np.zeros(shape, dtype=np.float32)
        _check(lib.kvq_get_plan(self._h, layer, bits.ctypes.data, gains.ctypes.data), "kvq_get_plan")
        return bits.astype(np.int64), gains

    def quantize_append(self, layer: int, k, v, stream=None):
        if k.shape != v.shape or k.dtype != v.dtype:
            raise ValueError("k and v must have the same shape and dtype")
        if k.dim() != 4 or k.shape[0] != self.cfg.batch or k.shape[2] != self.cfg.n_kv_heads \
                or k.shape[3] != self.cfg.head_dim:
            raise ValueError(f"k must be [batch, n_new, n_kv_heads, head_dim], got {tuple(k.shape)}")
        _check(lib.kvq_quantize_append(self._h, layer, _ptr(k), _ptr(v), _dtype_code(k), k.shape[1],
                                       _stream(stream)), "kvq_quantize_append")

    def decode_attn(self, layer: int, q, out=None, scale: float = 0.0, n_splits: int = 0, stream=None):
        import torch
        if q.dim() != 3 or tuple(q.shape) != (self.cfg.batch, self.cfg.n_q_heads, self.cfg.head_dim):
            raise ValueError(f"q must be [batch, n_q_heads, head_dim], got {tuple(q.shape)}")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must be fp32 with q's shape")
        _check(lib.kvq_decode_attn_splits(self._h, layer, _ptr(q), _dtype_code(q), float(scale),
                                          _ptr(out), int(n_splits), _stream(stream)), "kvq_decode_attn")
        return out

    def decode_step(self, layer: int, k_new, v_new, q, out=None, scale: float = 0.0, stream=None):
        """kvq_decode_step: append one position (k_new, v_new [batch, n_kv_heads, head_dim]) to
        every sequence of `layer`, then attend with q over all positions (one launch where the
        codec allows it)."""
        import torch
        B, H, d = self.cfg.batch, self.cfg.n_kv_heads, self.cfg.head_dim
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t.dim() != 3 or tuple(t.shape) != (B, H, d) or t.dtype != q.dtype or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous [batch, n_kv_heads, head_dim] in q's dtype, "
                                 f"got {tuple(t.shape)} {t.dtype}")
        if q.dim() != 3 or tuple(q.shape) != (B, self.cfg.n_q_heads, d):
            raise ValueError(f"q must be [batch, n_q_heads, head_dim], got {tuple(q.shape)}")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must be fp32 with q's shape")
        _check(lib.kvq_decode_step(self._h, layer, _ptr(k_new), _ptr(v_new), _ptr(q), _dtype_code(q),
                                   float(scale), _ptr(out), _stream(stream)), "kvq_decode_step")
        return out

    def decode_attn_noalloc(self, layer: int, q, out, scale: float = 0.0, stream=None):
        """kvq_decode_attn_noalloc: as decode_attn (automatic splits) into the caller's `out`,
        with no allocation anywhere (split scratch in the library's fixed device array)."""
        import torch
        if q.dim() != 3 or tuple(q.shape) != (self.cfg.batch, self.cfg.n_q_heads, self.cfg.head_dim):
            raise ValueError(f"q must be [batch, n_q_heads, head_dim], got {tuple(q.shape)}")
        if out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must be fp32 with q's shape")
        st = lib.kvq_decode_attn_noalloc(self._h, layer, _ptr(q), _dtype_code(q), float(scale), _ptr(out),
                                         _stream(stream))
        if st != KVQ_OK:
            raise KvqError(st, "kvq_decode_attn_noalloc", lib.kvq_last_error().decode())
        return out

    def key_fidelity(self, layer: int, q, keys, scale: float = 0.0, stream=None):
        """(mae, kl) fp64 [batch, n_q_heads] of the stored keys of `layer` against `keys`
        [batch, len, n_kv_heads, head_dim] (the keys appended to it), for queries q."""
        import torch
        B, Hq, d = self.cfg.batch, self.cfg.n_q_heads, self.cfg.head_dim
        if q.dim() != 3 or tuple(q.shape) != (B, Hq, d):
            raise ValueError(f"q must be [batch, n_q_heads, head_dim], got {tuple(q.shape)}")
        if keys.dim() != 4 or keys.shape[0] != B or keys.shape[2] != self.cfg.n_kv_heads or keys.shape[3] != d:
            raise ValueError(f"keys must be [batch, len, n_kv_heads, head_dim], got {tuple(keys.shape)}")
        if keys.shape[1] != self.seq_len(layer):
            raise ValueError("keys must hold exactly the positions appended to the layer")
        if keys.dtype != q.dtype:
            raise ValueError("q and keys must have the same dtype")
        mae = torch.empty((B, Hq), dtype=torch.float64, device=q.device)
        kl = torch.empty((B, Hq), dtype=torch.float64, device=q.device)
        _check(lib.kvq_key_fidelity(self._h, layer, _ptr(q), _ptr(keys), _dtype_code(q), float(scale),
                                    _ptr(mae), _ptr(kl), _stream(stream)), "kvq_key_fidelity")
        return mae, kl

    def status(self):
        """Raise KvqError if a decode split merge of this cache gave up since the last check
        (kvq_cache_status; synchronizes the device and clears the error)."""
        _check(lib.kvq_cache_status(self._h), "kvq_cache_status")

    def view(self, layer: int) -> kvq_view:
        """Read-only device pointers and strides of one layer's storage and plans (no copy)."""
        v = kvq_view()
        _check(lib.kvq_cache_view(self._h, layer, ctypes.byref(v)), "kvq_cache_view")
        return v

    def seq_len(self, layer: int) -> int:
        n = ctypes.c_int64()
        _check(lib.kvq_seq_len(self._h, layer, ctypes.byref(n)), "kvq_seq_len")
        return n.value

    def layer_info(self, layer: int) -> kvq_layer_info:
        info = kvq_layer_info()
        _check(lib.kvq_layer_info_get(self._h, layer, ctypes.byref(info)), "kvq_layer_info_get")
        return info

    def read(self, layer: int, part: int, dtype, offset: int = 0, nbytes: Optional[int] = None) -> np.ndarray:
        info = self.layer_info(layer)
        size = {PART_K_CODES: info.k_codes_bytes, PART_V_CODES: info.v_codes_bytes,
                PART_K_SCALES: info.k_scales_bytes, PART_V_SCALES: info.v_scales_bytes,
                PART_K_RECENT: info.recent_bytes, PART_V_RECENT: info.recent_bytes}[part]
        n = size - offset if nbytes is None else nbytes
        buf = np.empty(n, dtype=np.uint8)
        _check(lib.kvq_read_cache(self._h, layer, part, offset, n, buf.ctypes.data), "kvq_read_cache")
        return buf.view(dtype)
