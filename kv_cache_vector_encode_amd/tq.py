"""ctypes binding of libtq (include/tq.h): the same entry points, argument
marshalling only.

Device buffers are torch tensors on a ROCm device (torch supplies memory and
streams; every step of the codec runs in libtq's HIP kernels).  Status codes
other than TQ_OK raise ``TQError``.  The library is loaded from this package
directory; if it is missing the import fails loudly (there is no fallback).
"""

from __future__ import annotations

import ctypes
import math
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "tq.h")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_BITS_MISMATCH = 0, -1, -2, -3
TQ_ERR_OOM, TQ_ERR_NO_DEVICE, TQ_ERR_HIP, TQ_ERR_WORKSPACE = -4, -5, -6, -7
TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2
LAYOUT_VERSION = 1
BLOCK = 16


class TQError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_string(status)} ({status}): {detail}")
        self.status = status


class CacheConfig(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("bits_k", ctypes.c_int32), ("bits_v", ctypes.c_int32),
        ("qjl", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("rot", ctypes.c_void_p), ("rot_qjl", ctypes.c_void_p),
        ("layout_version", ctypes.c_int32),
    ]


class CacheLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "block_bytes", "k_rec_bytes", "v_rec_bytes", "off_k", "off_v", "off_gamma_k",
        "off_gamma_v", "off_rho", "off_sign", "pool_bytes")]


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libtq.so not built ({LIB_PATH}); run python -m kv_cache_vector_encode_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "tq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "tq_last_error": (ctypes.c_char_p, []),
            "tq_layout_version": (ctypes.c_int, []),
            "tq_make_rotation": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_int32, ctypes.POINTER(_P)]),
            "tq_rotation_signs": (ctypes.c_int, [_P, _P]),
            "tq_rotation_dim": (ctypes.c_int32, [_P]),
            "tq_rotation_destroy": (None, [_P]),
            "tq_codebook": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P]),
            "tq_cache_bytes": (ctypes.c_int64, [ctypes.POINTER(CacheConfig)]),
            "tq_cache_layout_query": (ctypes.c_int, [ctypes.POINTER(CacheConfig), ctypes.POINTER(CacheLayout)]),
            "tq_cache_create": (ctypes.c_int, [ctypes.POINTER(CacheConfig), _P, ctypes.POINTER(_P)]),
            "tq_cache_destroy": (None, [_P]),
            "tq_encode_kv": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int64, _P, ctypes.c_int32, _P, _P]),
            "tq_decode_workspace_bytes": (ctypes.c_int64, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
            "tq_decode_attend": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_float, _P, _P, _P, ctypes.c_int64, _P]),
            "tq_decode_attend_noalloc": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, _P, ctypes.c_int32,
                                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P, _P]),
            "tq_decode_logits": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_float, _P, _P]),
            "tq_reconstruct": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P]),
            "tq_decompress_kv": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
            "tq_minmax_encode": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]),
            "tq_stream_read": (ctypes.c_int, [_P, ctypes.c_int64, _P, _P]),
            "tq_octo_record_bytes": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32]),
            "tq_octo_table_bytes": (ctypes.c_int64, [ctypes.c_int32]),
            "tq_octo_codebook": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P]),
            "tq_octo_tables": (ctypes.c_int, [ctypes.c_int32, _P, _P]),
            "tq_octo_encode": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P,
                                              ctypes.c_int64, _P, _P, _P]),
            "tq_octo_logits": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                              ctypes.c_int32, _P, _P, ctypes.c_int64, ctypes.c_float, _P, _P]),
            "tq_octo_attend_workspace_bytes": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]),
            "tq_octo_attend": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                              ctypes.c_int32, _P, _P, ctypes.c_int64, ctypes.c_float, _P, _P,
                                              ctypes.c_int64, _P]),
            "tq_octo_encode_qjl": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P, _P,
                                                  ctypes.c_int64, _P, _P, _P, _P, _P]),
            "tq_octo_logits_qjl": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                                  ctypes.c_int32, _P, _P, _P, ctypes.c_int64, ctypes.c_float, _P,
                                                  _P]),
            "tq_minmax_decode": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_int32, _P, _P]),
            "tq_decode_step": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, ctypes.c_int32, _P, _P, _P, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P, _P,
                                              ctypes.c_int64, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/tq.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def _check(status: int, where: str):
    if status != TQ_OK:
        raise TQError(status, where, lib().tq_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: TQ_F32, torch.float16: TQ_F16, torch.bfloat16: TQ_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


# ------------------------------------------------------- argument checks --
# The C ABI takes raw device pointers and trusts the sizes it is given, so
# every wrapper checks its tensors here first: a wrong index dtype (int64 is
# torch's default), a non-contiguous view, a wrong shape or a host tensor
# would otherwise be read out of bounds by the kernels.

_FLOATS = ("float32", "float16", "bfloat16")


def _need(t, name: str, dtypes=None, shape=None):
    """t must be a contiguous torch tensor of one of `dtypes` (torch dtype
    names) with `shape` (None entries match any size).  Returns t.  Where it
    lives is checked by _on_gpu once every argument has passed these checks."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if dtypes is not None and str(t.dtype).replace("torch.", "") not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {', '.join(dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w) for g, w in zip(t.shape, shape)):
            want = "[" + "][".join("*" if w is None else str(w) for w in shape) + "]"
            raise ValueError(f"{name}: shape {list(t.shape)}, expected {want}")
    return t


def _need_bytes(t, name: str, nbytes: int):
    """A contiguous tensor of at least nbytes bytes (any dtype)."""
    _need(t, name)
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, needs {nbytes}")
    return t


def _int32(t, name: str, shape):
    return _need(t, name, ("int32",), shape)


def _on_gpu(device=None, **tensors):
    """Every given tensor (None entries are skipped) is on one GPU device:
    `device` if given (the cache pool's), else the first one's."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name}: must be on a GPU device, is on {t.device}")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name}: on {t.device}, expected {device}")


def _pool_device(cache):
    import torch
    pool = getattr(cache, "pool", None)
    return pool.device if isinstance(pool, torch.Tensor) and pool.device.type == "cuda" else None


# ----------------------------------------------------------------- rotation --

class Rotation:
    """Owns a tq_rotation* (freed on garbage collection)."""

    def __init__(self, handle: int, seed: int, d: int):
        self.handle, self.seed, self.d = handle, seed, d

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tq_rotation_destroy(self.handle)
            self.handle = None


def tq_make_rotation(seed: int, d: int) -> Rotation:
    h = _P()
    _check(lib().tq_make_rotation(ctypes.c_uint64(seed & (2 ** 64 - 1)), d, ctypes.byref(h)), "tq_make_rotation")
    return Rotation(h.value, seed, d)


def tq_rotation_signs(rot: Rotation) -> np.ndarray:
    out = np.empty(rot.d, dtype=np.int8)
    _check(lib().tq_rotation_signs(rot.handle, out.ctypes.data), "tq_rotation_signs")
    return out


def tq_codebook(d: int, bits: int):
    c = np.empty(1 << bits, dtype=np.float32)
    t = np.empty((1 << bits) - 1, dtype=np.float32)
    _check(lib().tq_codebook(d, bits, c.ctypes.data, t.ctypes.data), "tq_codebook")
    return c, t


# -------------------------------------------------------------------- cache --

def make_config(num_kv_heads: int, num_blocks: int, bits_k: int, bits_v: int, rot: Rotation,
                qjl: bool = False, rot_qjl: Rotation | None = None, d: int = 128) -> CacheConfig:
    return CacheConfig(d, num_kv_heads, bits_k, bits_v, int(qjl), BLOCK, num_blocks,
                       rot.handle if rot else None, rot_qjl.handle if rot_qjl else None,
                       LAYOUT_VERSION)


def tq_cache_bytes(cfg: CacheConfig) -> int:
    n = lib().tq_cache_bytes(ctypes.byref(cfg))
    if n < 0:
        _check(int(n), "tq_cache_bytes")
    return int(n)


def tq_cache_layout_query(cfg: CacheConfig) -> CacheLayout:
    lay = CacheLayout()
    _check(lib().tq_cache_layout_query(ctypes.byref(cfg), ctypes.byref(lay)), "tq_cache_layout_query")
    return lay


class Cache:
    """Owns a tq_cache* descriptor bound to a caller pool (kept alive here)."""

    def __init__(self, handle: int, cfg: CacheConfig, pool, rots):
        self.handle, self.cfg, self.pool, self._rots = handle, cfg, pool, rots
        self.layout = tq_cache_layout_query(cfg)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tq_cache_destroy(self.handle)
            self.handle = None


def tq_cache_create(cfg: CacheConfig, pool) -> Cache:
    h = _P()
    _check(lib().tq_cache_create(ctypes.byref(cfg), _ptr(pool), ctypes.byref(h)), "tq_cache_create")
    return Cache(h.value, cfg, pool, None)


# ------------------------------------------------------------------- encode --

def tq_encode_kv(K, V, slot_mapping, bits: int, cache: Cache, stream=None):
    """K, V: device tensors [tokens][kv_heads][128] (V None for keys-only)."""
    dev, H = _pool_device(cache), cache.cfg.num_kv_heads
    _need(K, "K", _FLOATS, (None, H, 128))
    if V is not None:
        _need(V, "V", (str(K.dtype).replace("torch.", ""),), tuple(K.shape))
    _int32(slot_mapping, "slot_mapping", (K.shape[0],))
    _on_gpu(dev, K=K, V=V, slot_mapping=slot_mapping)
    _check(lib().tq_encode_kv(_ptr(K), _ptr(V), _dtype_code(K), K.shape[0], _ptr(slot_mapping), bits,
                              cache.handle, _stream(stream)), "tq_encode_kv")


# ------------------------------------------------------------------- decode --

def tq_decode_workspace_bytes(cache: Cache, num_seqs: int, num_q_heads: int, max_blocks_per_seq: int) -> int:
    n = lib().tq_decode_workspace_bytes(cache.handle, num_seqs, num_q_heads, max_blocks_per_seq)
    if n < 0:
        _check(int(n), "tq_decode_workspace_bytes")
    return int(n)


def tq_decode_attend(q, cache: Cache, block_tables, seq_lens, out, workspace, logits_out=None,
                     scale: float = 0.0, stream=None):
    """q [seqs][q_heads][128]; block_tables int32 [seqs][max_blocks]; out f32
    [seqs][q_heads][128]; workspace: uint8 tensor of tq_decode_workspace_bytes() bytes."""
    ns, hq, mb = _check_decode_args(q, cache, block_tables, seq_lens, logits_out)
    _need(out, "out", ("float32",), (ns, hq, 128))
    _need_bytes(workspace, "workspace", tq_decode_workspace_bytes(cache, ns, hq, mb))
    _on_gpu(_pool_device(cache), q=q, block_tables=block_tables, seq_lens=seq_lens, out=out, workspace=workspace,
            logits_out=logits_out)
    _check(lib().tq_decode_attend(_ptr(q), _dtype_code(q), cache.handle, _ptr(block_tables), _ptr(seq_lens),
                                  ns, hq, block_tables.shape[1], scale, _ptr(out), _ptr(logits_out),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)), "tq_decode_attend")


NOALLOC_SCRATCH_BYTES = 16 << 20


def tq_decode_attend_noalloc(q, cache: Cache, block_tables, seq_lens, out, logits_out=None, scale: float = 0.0,
                             stream=None):
    """tq_decode_attend with the split partials in the library's fixed
    per-GPU scratch (NOALLOC_SCRATCH_BYTES) instead of a workspace; the call
    allocates nothing.  Calls that overlap in time on one GPU race."""
    ns, hq, mb = _check_decode_args(q, cache, block_tables, seq_lens, logits_out)
    _need(out, "out", ("float32",), (ns, hq, 128))
    _on_gpu(_pool_device(cache), q=q, block_tables=block_tables, seq_lens=seq_lens, out=out, logits_out=logits_out)
    _check(lib().tq_decode_attend_noalloc(_ptr(q), _dtype_code(q), cache.handle, _ptr(block_tables), _ptr(seq_lens),
                                          ns, hq, mb, scale, _ptr(out), _ptr(logits_out), _stream(stream)),
           "tq_decode_attend_noalloc")


def _check_decode_args(q, cache: Cache, block_tables, seq_lens, logits_out):
    dev = _pool_device(cache)
    _need(q, "q", _FLOATS, (None, None, 128))
    ns, hq, _ = q.shape
    _int32(block_tables, "block_tables", (ns, None))
    _int32(seq_lens, "seq_lens", (ns,))
    mb = block_tables.shape[1]
    if logits_out is not None:
        _need(logits_out, "logits_out", ("float32",), (ns, hq, mb * BLOCK))
    return ns, hq, mb


def tq_decode_logits(q, cache: Cache, block_tables, seq_lens, logits_out, scale: float = 0.0, stream=None):
    ns, hq, _ = _check_decode_args(q, cache, block_tables, seq_lens, logits_out)
    _on_gpu(_pool_device(cache), q=q, block_tables=block_tables, seq_lens=seq_lens, logits_out=logits_out)
    _check(lib().tq_decode_logits(_ptr(q), _dtype_code(q), cache.handle, _ptr(block_tables), _ptr(seq_lens),
                                  ns, hq, block_tables.shape[1], scale, _ptr(logits_out), _stream(stream)),
           "tq_decode_logits")


def tq_reconstruct(cache: Cache, slots, which: int, out, stream=None):
    dev = _pool_device(cache)
    _int32(slots, "slots", (None,))
    _need(out, "out", ("float32",), (slots.shape[0], cache.cfg.num_kv_heads, 128))
    _on_gpu(dev, slots=slots, out=out)
    _check(lib().tq_reconstruct(cache.handle, _ptr(slots), slots.shape[0], which, _ptr(out), _stream(stream)),
           "tq_reconstruct")


def tq_decode_step(q, K_new, V_new, cache: Cache, block_tables, seq_lens, out, workspace, logits_out=None,
                   scale: float = 0.0, stream=None):
    """Append every sequence's new token (K_new, V_new [seqs][kv_heads][128],
    at position seq_len - 1) and attend over the whole sequence; arguments
    otherwise as tq_decode_attend."""
    ns, hq, mb = _check_decode_args(q, cache, block_tables, seq_lens, logits_out)
    dev, H = _pool_device(cache), cache.cfg.num_kv_heads
    _need(K_new, "K_new", _FLOATS, (ns, H, 128))
    _need(V_new, "V_new", (str(K_new.dtype).replace("torch.", ""),), (ns, H, 128))
    _need(out, "out", ("float32",), (ns, hq, 128))
    _need_bytes(workspace, "workspace", tq_decode_workspace_bytes(cache, ns, hq, mb))
    _on_gpu(dev, q=q, K_new=K_new, V_new=V_new, block_tables=block_tables, seq_lens=seq_lens, out=out,
            workspace=workspace, logits_out=logits_out)
    _check(lib().tq_decode_step(_ptr(q), _dtype_code(q), _ptr(K_new), _ptr(V_new), _dtype_code(K_new), cache.handle,
                                _ptr(block_tables), _ptr(seq_lens), ns, hq, block_tables.shape[1], scale, _ptr(out),
                                _ptr(logits_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "tq_decode_step")


def tq_minmax_encode(X, bits: int, rot, codes, params, stream=None):
    """X: device [n][128] (f32/f16/bf16); codes: uint8 [n][16*bits]; params:
    [n][2] 16-bit words (fp16 scale, fp16 zero point)."""
    _need(X, "X", _FLOATS, (None, 128))
    n = X.shape[0]
    _need(codes, "codes", ("uint8",), (n, 16 * bits))
    _need(params, "params", ("int16", "float16", "bfloat16"), (n, 2))
    _on_gpu(None, X=X, codes=codes, params=params)
    _check(lib().tq_minmax_encode(_ptr(X), _dtype_code(X), X.shape[0], bits, rot.handle, _ptr(codes),
                                  _ptr(params), _stream(stream)), "tq_minmax_encode")


def tq_minmax_decode(codes, params, bits: int, rot, out, stream=None):
    """out: device [n][128] of f32/f16/bf16."""
    _need(codes, "codes", ("uint8",), (None, 16 * bits))
    n = codes.shape[0]
    _need(params, "params", ("int16", "float16", "bfloat16"), (n, 2))
    _need(out, "out", _FLOATS, (n, 128))
    _on_gpu(None, codes=codes, params=params, out=out)
    _check(lib().tq_minmax_decode(_ptr(codes), _ptr(params), codes.shape[0], bits, rot.handle,
                                  _dtype_code(out), _ptr(out), _stream(stream)), "tq_minmax_decode")


def tq_stream_read(src, sink, stream=None):
    """Measurement aid: stream-read the device tensor src (its whole storage)."""
    _need(src, "src")
    _need_bytes(sink, "sink", 4)
    _on_gpu(None, src=src, sink=sink)
    _check(lib().tq_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "tq_stream_read")


def tq_octo_record_bytes(d: int, bits: int) -> int:
    n = lib().tq_octo_record_bytes(d, bits)
    _check(int(n) if n < 0 else 0, "tq_octo_record_bytes")
    return int(n)


def tq_octo_table_bytes(bits: int) -> int:
    n = lib().tq_octo_table_bytes(bits)
    _check(int(n) if n < 0 else 0, "tq_octo_table_bytes")
    return int(n)


def tq_octo_codebook(d: int, bits: int):
    """Host tables: (dirs float32 [4^(bits+1)][4], rho centroids float32 [2^(bits-1)])."""
    dirs = np.zeros((1 << (2 * (bits + 1)), 4), np.float32)
    rho = np.zeros(1 << (bits - 1), np.float32)
    _check(lib().tq_octo_codebook(d, bits, dirs.ctypes.data, rho.ctypes.data), "tq_octo_codebook")
    return dirs, rho


def tq_octo_tables(bits: int, dev_tables, stream=None):
    """dev_tables: device uint8 tensor of tq_octo_table_bytes(bits) bytes."""
    _need_bytes(dev_tables, "dev_tables", tq_octo_table_bytes(bits))
    _on_gpu(None, dev_tables=dev_tables)
    _check(lib().tq_octo_tables(bits, _ptr(dev_tables), _stream(stream)), "tq_octo_tables")


def tq_octo_encode(X, bits: int, rot, dev_tables, codes, gamma, stream=None):
    """X: device [n][128] (f32/f16/bf16); codes: uint8 [n][record bytes]; gamma: [n] 16-bit."""
    _need(X, "X", _FLOATS, (None, 128))
    n = X.shape[0]
    _need_bytes(dev_tables, "dev_tables", tq_octo_table_bytes(bits))
    _need(codes, "codes", ("uint8",), (n, tq_octo_record_bytes(128, bits)))
    _need(gamma, "gamma", ("int16", "float16"), (n,))
    _on_gpu(None, X=X, dev_tables=dev_tables, codes=codes, gamma=gamma)
    _check(lib().tq_octo_encode(_ptr(X), _dtype_code(X), X.shape[0], bits, rot.handle, _ptr(dev_tables),
                                dev_tables.numel() * dev_tables.element_size(), _ptr(codes), _ptr(gamma),
                                _stream(stream)), "tq_octo_encode")


def tq_octo_logits(q, codes, gamma, bits: int, rot, dev_tables, out, scale=None, stream=None):
    """q: fp32 [heads][group][128]; codes: uint8 [heads][n][record bytes];
    gamma: [heads][n] 16-bit; out: fp32 [heads][group][n]."""
    _need(q, "q", ("float32",), (None, None, 128))
    heads, group, _ = q.shape
    _need(codes, "codes", ("uint8",), (heads, None, tq_octo_record_bytes(128, bits)))
    n = codes.shape[1]
    _need(gamma, "gamma", ("int16", "float16"), (heads, n))
    _need(out, "out", ("float32",), (heads, group, n))
    _need_bytes(dev_tables, "dev_tables", tq_octo_table_bytes(bits))
    _on_gpu(None, q=q, codes=codes, gamma=gamma, out=out, dev_tables=dev_tables)
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    _check(lib().tq_octo_logits(_ptr(q), _ptr(codes), _ptr(gamma), heads, group, codes.shape[1], bits, rot.handle,
                                _ptr(dev_tables), dev_tables.numel() * dev_tables.element_size(), scale, _ptr(out),
                                _stream(stream)), "tq_octo_logits")


def tq_octo_encode_qjl(X, bits: int, rot, rot_qjl, dev_tables, codes, gamma, signs, rho, stream=None):
    """tq_octo_encode plus the residual sketch: signs uint8 [n][16] (16-byte
    aligned), rho [n] 16-bit."""
    _need(X, "X", _FLOATS, (None, 128))
    n = X.shape[0]
    _need_bytes(dev_tables, "dev_tables", tq_octo_table_bytes(bits))
    _need(codes, "codes", ("uint8",), (n, tq_octo_record_bytes(128, bits)))
    _need(gamma, "gamma", ("int16", "float16"), (n,))
    _need(signs, "signs", ("uint8",), (n, 16))
    _need(rho, "rho", ("int16", "float16"), (n,))
    _on_gpu(None, X=X, dev_tables=dev_tables, codes=codes, gamma=gamma, signs=signs, rho=rho)
    _check(lib().tq_octo_encode_qjl(_ptr(X), _dtype_code(X), n, bits, rot.handle, rot_qjl.handle, _ptr(dev_tables),
                                    dev_tables.numel() * dev_tables.element_size(), _ptr(codes), _ptr(gamma),
                                    _ptr(signs), _ptr(rho), _stream(stream)), "tq_octo_encode_qjl")


def tq_octo_logits_qjl(q, codes, gamma, signs, rho, bits: int, rot, rot_qjl, dev_tables, out, scale=None,
                       stream=None):
    """tq_octo_logits plus the residual sketch's estimate: signs uint8
    [heads][n][16], rho [heads][n] 16-bit, as tq_octo_encode_qjl wrote them."""
    _need(q, "q", ("float32",), (None, None, 128))
    heads, group, _ = q.shape
    _need(codes, "codes", ("uint8",), (heads, None, tq_octo_record_bytes(128, bits)))
    n = codes.shape[1]
    _need(gamma, "gamma", ("int16", "float16"), (heads, n))
    _need(signs, "signs", ("uint8",), (heads, n, 16))
    _need(rho, "rho", ("int16", "float16"), (heads, n))
    _need(out, "out", ("float32",), (heads, group, n))
    _need_bytes(dev_tables, "dev_tables", tq_octo_table_bytes(bits))
    _on_gpu(None, q=q, codes=codes, gamma=gamma, signs=signs, rho=rho, out=out, dev_tables=dev_tables)
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    _check(lib().tq_octo_logits_qjl(_ptr(q), _ptr(codes), _ptr(gamma), _ptr(signs), _ptr(rho), heads, group, n, bits,
                                    rot.handle, rot_qjl.handle, _ptr(dev_tables),
                                    dev_tables.numel() * dev_tables.element_size(), scale, _ptr(out),
                                    _stream(stream)), "tq_octo_logits_qjl")


def tq_octo_attend_workspace_bytes(heads: int, group: int, n: int) -> int:
    v = lib().tq_octo_attend_workspace_bytes(heads, group, n)
    _check(int(v) if v < 0 else 0, "tq_octo_attend_workspace_bytes")
    return int(v)


def tq_octo_attend(q, k_codes, k_gamma, v_codes, v_gamma, bits: int, rot, dev_tables, out, workspace, scale=None,
                   stream=None):
    """q: fp32 [heads][group][128]; k_codes / v_codes: uint8 [heads][n][record
    bytes]; k_gamma / v_gamma: [heads][n] 16-bit; out: fp32 [heads][group][128];
    workspace: device uint8 of tq_octo_attend_workspace_bytes(heads, group, n)."""
    _need(q, "q", ("float32",), (None, None, 128))
    heads, group, _ = q.shape
    rb = tq_octo_record_bytes(128, bits)
    _need(k_codes, "k_codes", ("uint8",), (heads, None, rb))
    n = k_codes.shape[1]
    _need(v_codes, "v_codes", ("uint8",), (heads, n, rb))
    _need(k_gamma, "k_gamma", ("int16", "float16"), (heads, n))
    _need(v_gamma, "v_gamma", ("int16", "float16"), (heads, n))
    _need(out, "out", ("float32",), (heads, group, 128))
    _need_bytes(dev_tables, "dev_tables", tq_octo_table_bytes(bits))
    _need_bytes(workspace, "workspace", tq_octo_attend_workspace_bytes(heads, group, n))
    _on_gpu(None, q=q, k_codes=k_codes, k_gamma=k_gamma, v_codes=v_codes, v_gamma=v_gamma, out=out,
            dev_tables=dev_tables, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    _check(lib().tq_octo_attend(_ptr(q), _ptr(k_codes), _ptr(k_gamma), _ptr(v_codes), _ptr(v_gamma), heads, group, n,
                                bits, rot.handle, _ptr(dev_tables), dev_tables.numel() * dev_tables.element_size(),
                                scale, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "tq_octo_attend")


def tq_decompress_kv(cache: Cache, slots, K_out, V_out=None, stream=None):
    """K_out / V_out: device tensors [n][kv_heads][128] of bfloat16 or float16
    (the same dtype); either may be None."""
    dev, H = _pool_device(cache), cache.cfg.num_kv_heads
    if K_out is not None and V_out is not None and getattr(K_out, "dtype", None) != getattr(V_out, "dtype", None):
        raise TypeError("K_out and V_out must have one dtype")
    _int32(slots, "slots", (None,))
    ref = K_out if K_out is not None else V_out
    for t, name in ((K_out, "K_out"), (V_out, "V_out")):
        if t is not None:
            _need(t, name, ("bfloat16", "float16"), (slots.shape[0], H, 128))
    _on_gpu(dev, slots=slots, K_out=K_out, V_out=V_out)
    _check(lib().tq_decompress_kv(cache.handle, _ptr(slots), slots.shape[0], _dtype_code(ref) if ref is not None else 2,
                                  _ptr(K_out), _ptr(V_out), _stream(stream)), "tq_decompress_kv")


# ------------------------------------------------------------------ helpers --

def new_cache(num_kv_heads: int, num_blocks: int, bits_k: int, bits_v: int, seed: int = 42,
              qjl: bool = False, qjl_seed: int = 43, device="cuda"):
    """Allocate a zeroed pool with torch and bind a descriptor to it."""
    import torch
    rot = tq_make_rotation(seed, 128)
    rq = tq_make_rotation(qjl_seed, 128) if qjl else None
    cfg = make_config(num_kv_heads, num_blocks, bits_k, bits_v, rot, qjl, rq)
    pool = torch.zeros(tq_cache_bytes(cfg), dtype=torch.uint8, device=device)
    c = tq_cache_create(cfg, pool)
    c._rots = (rot, rq)
    return c


def new_workspace(cache: Cache, num_seqs: int, num_q_heads: int, max_blocks: int, device="cuda"):
    import torch
    return torch.zeros(tq_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_blocks),
                       dtype=torch.uint8, device=device)
