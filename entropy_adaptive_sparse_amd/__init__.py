"""Token Radius Attention (TRA) hot path for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libtra.so`` (declared in include/tra.h).
It only marshals arguments: it checks tensor shapes/dtypes/devices, allocates
outputs with torch when the caller passes none, and forwards raw device pointers
and the current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no fallback of any kind -- if the library is missing, every
call raises.

Functions (names as in the C ABI, without the ``tra_`` prefix):
    tile_major_permute / tile_major_unpermute
    dense_attn_entropy
    dense_attn_entropy_mask (the warm-up pass with the mask builder fused in)
    build_block_mask, mask_prepare, natural_prepare
    build_block_mask_1d, mask_prepare_1d (the 1D-distance variant of the mask)
    block_sparse_attn
    block_sparse_attn_fp8 (fp8 E4M3 q and k, bf16 v and o)
    sparse_schedule, block_sparse_attn_scheduled (the order the sparse workgroups take the rows in)
    dense_attn_entropy_natural, dense_attn_entropy_mask_natural, block_sparse_attn_natural
        (natural-order q, k, v, o; the tile-major map applied inside the kernels' loads and stores)
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "TraError", "library_path", "load", "tile_major_permute", "tile_major_unpermute", "dense_attn_entropy",
    "dense_attn_entropy_mask", "build_block_mask", "mask_prepare", "natural_prepare", "build_block_mask_1d",
    "mask_prepare_1d", "block_sparse_attn",
    "block_sparse_attn_fp8", "sparse_schedule", "block_sparse_attn_scheduled", "dense_attn_entropy_natural", "dense_attn_entropy_mask_natural", "block_sparse_attn_natural",
    "exported_symbols",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "libtra.so")
_lock = threading.Lock()
_lib = None

TRA_F32, TRA_BF16 = 0, 1
_STATUS = {0: "TRA_OK", 1: "TRA_ERR_INVALID_ARG", 2: "TRA_ERR_UNSUPPORTED", 3: "TRA_ERR_HIP", 4: "TRA_ERR_CAPACITY"}


class TraError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s failed: %s (%d)" % (fn, _STATUS.get(code, "?"), code))
        self.code = code


def library_path() -> str:
    return _LIBPATH


def load():
    """Load libtra.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # torch ships its own HIP runtime (same soname as ROCm's libamdhip64.so.7).  Loading
        # torch first makes libtra.so bind to that runtime, so the process holds one HIP/HSA
        # runtime; the other order would load a second runtime that sees no device.
        try:
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover - a plain C caller needs no torch
            pass
        if not os.path.exists(_LIBPATH):
            raise RuntimeError("libtra.so is not built (%s); run `python -m entropy_adaptive_sparse_amd.build`"
                               % _LIBPATH)
        lib = ctypes.CDLL(_LIBPATH)
        P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.tra_status_string.argtypes = [i32]
        lib.tra_status_string.restype = ctypes.c_char_p
        perm_args = [P, P, i32, i32, i32, i32, i32, i32, i32, i32, P]
        lib.tra_tile_major_permute.argtypes = perm_args
        lib.tra_tile_major_unpermute.argtypes = perm_args
        lib.tra_dense_attn_entropy.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, P]
        lib.tra_build_block_mask.argtypes = [P, i32, i32, i32, i32, f32, f32, i32, i32, i32, i32, i32, P, P, i64,
                                             P, P]
        lib.tra_mask_prepare.argtypes = [i32, i32, i32, f32, f32, i32, i32, i32, i32]
        lib.tra_natural_prepare.argtypes = [i32, i32, i32, i32, i32]
        lib.tra_build_block_mask_1d.argtypes = [P, i32, i32, i32, i32, f32, i32, i32, i32, i32, i32, P, P, i64, P, P]
        lib.tra_mask_prepare_1d.argtypes = [i32, i32, i32, f32, i32, i32, i32, i32]
        lib.tra_block_sparse_attn.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, f32, i32, i32, P]
        lib.tra_block_sparse_attn_fp8.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, f32, i32, i32, P]
        lib.tra_sparse_schedule.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, i32, P, i64, P]
        lib.tra_block_sparse_attn_scheduled.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, f32, i32, i32, P]
        lib.tra_dense_attn_entropy_mask.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f32, f32, f32,
                                                    i32, i32, i32, i32, i32, P, P, i64, P, P]
        lib.tra_dense_attn_entropy_mask_natural.argtypes = lib.tra_dense_attn_entropy_mask.argtypes
        lib.tra_dense_attn_entropy_natural.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f32, i32,
                                                       i32, P]
        lib.tra_block_sparse_attn_natural.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f32, i32,
                                                      i32, i32, i32, P]
        for name in ("tra_tile_major_permute", "tra_tile_major_unpermute", "tra_dense_attn_entropy",
                     "tra_build_block_mask", "tra_mask_prepare", "tra_natural_prepare", "tra_block_sparse_attn",
                     "tra_block_sparse_attn_fp8", "tra_sparse_schedule", "tra_block_sparse_attn_scheduled",
                     "tra_build_block_mask_1d", "tra_mask_prepare_1d",
                     "tra_dense_attn_entropy_mask", "tra_dense_attn_entropy_natural",
                     "tra_block_sparse_attn_natural", "tra_dense_attn_entropy_mask_natural"):
            getattr(lib, name).restype = i32
        _lib = lib
        return lib


def exported_symbols():
    return ["tra_status_string", "tra_tile_major_permute", "tra_tile_major_unpermute", "tra_dense_attn_entropy",
            "tra_build_block_mask", "tra_mask_prepare", "tra_natural_prepare", "tra_block_sparse_attn",
            "tra_block_sparse_attn_fp8", "tra_sparse_schedule", "tra_block_sparse_attn_scheduled",
            "tra_build_block_mask_1d", "tra_mask_prepare_1d", "tra_dense_attn_entropy_mask",
            "tra_dense_attn_entropy_natural", "tra_block_sparse_attn_natural", "tra_dense_attn_entropy_mask_natural"]


# ------------------------------------------------------------------------------------------------
# marshalling helpers (torch is used only for device memory and the current stream)
# ------------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TRA_F32
    if t.dtype == torch.bfloat16:
        return TRA_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _rows(x):
    """(row_elems, dtype code) under which the permutation moves x's token rows as bytes: fp32 and
    bf16 as themselves, one-byte types (fp8) as bf16 pairs."""
    per_row = 1 if x.dim() == 2 else int(x[0, 0].numel())
    if x.element_size() == 1:
        if per_row % 2:
            raise ValueError("one-byte rows must hold an even number of elements")
        return per_row // 2, TRA_BF16
    return per_row, _dt(x)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _buf(t, name, shape, dtype, like):
    """A caller-supplied buffer (input list or output), or a new one when t is None: on like's GPU,
    contiguous, of exactly this shape and dtype, so that the kernels stay inside it."""
    torch = _torch()
    if t is None:
        return torch.empty(tuple(shape), dtype=dtype, device=like.device)
    _dev(t, name)
    if t.device != like.device:
        raise ValueError("%s is on %s, the inputs on %s" % (name, t.device, like.device))
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError("%s must be %s %s, got %s %s" % (name, dtype, tuple(shape), t.dtype, tuple(t.shape)))
    return t


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.device).cuda_stream


def _call(fn: str, *args) -> None:
    rc = getattr(load(), fn)(*args)
    if rc != 0:
        raise TraError(fn, rc)


# ------------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------------
def tile_major_permute(x, F: int, H: int, W: int, tile_h: int = 8, tile_w: int = 8, out=None):
    """x [outer][N][row] (natural order) -> y in tile-major order.  Also accepts [outer][N]."""
    _dev(x, "x")
    y = _buf(out, "out", x.shape, x.dtype, x)
    outer, N = x.shape[0], x.shape[1]
    row, dt = _rows(x)
    if N != F * H * W:
        raise ValueError("x has %d tokens, F*H*W = %d" % (N, F * H * W))
    _call("tra_tile_major_permute", _ptr(x), _ptr(y), outer, F, H, W, row, dt, tile_h, tile_w, _stream(x))
    return y


def tile_major_unpermute(y, F: int, H: int, W: int, tile_h: int = 8, tile_w: int = 8, out=None):
    """y [outer][N][row] (tile-major) -> x in natural order."""
    _dev(y, "y")
    x = _buf(out, "out", y.shape, y.dtype, y)
    outer, N = y.shape[0], y.shape[1]
    row, dt = _rows(y)
    if N != F * H * W:
        raise ValueError("y has %d tokens, F*H*W = %d" % (N, F * H * W))
    _call("tra_tile_major_unpermute", _ptr(y), _ptr(x), outer, F, H, W, row, dt, tile_h, tile_w, _stream(y))
    return x


def _check_qkv(q, k, v):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
        if t.dim() != 3:
            raise ValueError("%s must be [outer][N][D]" % n)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    return q.shape


def dense_attn_entropy(q, k, v, sm_scale: float | None = None, entropy: bool = True, lse: bool = False,
                       out=None, ent_out=None, lse_out=None):
    """Dense attention over all N keys with the per-query entropy (nats).  Returns (o, H, lse)."""
    torch = _torch()
    outer, N, D = _check_qkv(q, k, v)
    o = _buf(out, "out", q.shape, q.dtype, q)
    H = _buf(ent_out, "ent_out", (outer, N), torch.float32, q) if entropy else None
    L = _buf(lse_out, "lse_out", (outer, N), torch.float32, q) if lse else None
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    _call("tra_dense_attn_entropy", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(H), _ptr(L), outer, N, D, _dt(q),
          scale, _stream(q))
    return o, H, L


def _dense_mask(fn, q, k, v, F, H, W, tau, gamma, sm_scale, block_q, block_k, vote_threshold, tile_h, tile_w,
                entropy, lse, want_mask, out, ent_out, lse_out, kv_count, kv_index, block_mask):
    torch = _torch()
    outer, N, D = _check_qkv(q, k, v)
    if N != F * H * W:
        raise ValueError("N must equal F*H*W")
    o = _buf(out, "out", q.shape, q.dtype, q)
    Hh = _buf(ent_out, "ent_out", (outer, N), torch.float32, q) if entropy else None
    L = _buf(lse_out, "lse_out", (outer, N), torch.float32, q) if lse else None
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    cnt = _buf(kv_count, "kv_count", (outer, nqb), torch.int32, q)
    idx = _buf(kv_index, "kv_index", (outer, nqb, nkb), torch.int32, q)
    msk = _buf(block_mask, "block_mask", (outer, nqb, nkb), torch.uint8, q) if (want_mask or block_mask is not None) \
        else None
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    _call(fn, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(Hh), _ptr(L), outer, F, H, W, D,
          _dt(q), scale, float(tau), float(gamma), block_q, block_k, int(vote_threshold), tile_h, tile_w, _ptr(cnt),
          _ptr(idx), idx.numel(), _ptr(msk), _stream(q))
    return o, Hh, L, cnt, idx, msk


def dense_attn_entropy_mask(q, k, v, F: int, H: int, W: int, tau: float, gamma: float, sm_scale: float | None = None,
                            block_q: int = 128, block_k: int = 64, vote_threshold: int = 1, tile_h: int = 8,
                            tile_w: int = 8, entropy: bool = True, lse: bool = False, want_mask: bool = False,
                            out=None, ent_out=None, lse_out=None, kv_count=None, kv_index=None, block_mask=None):
    """Warm-up pass with the mask fused in.  Returns (o, H, lse, kv_count, kv_index, mask); H, lse and
    mask are None unless requested (the mask is built from the entropies either way)."""
    return _dense_mask("tra_dense_attn_entropy_mask", q, k, v, F, H, W, tau, gamma, sm_scale, block_q, block_k,
                       vote_threshold, tile_h, tile_w, entropy, lse, want_mask, out, ent_out, lse_out, kv_count,
                       kv_index, block_mask)


def dense_attn_entropy_mask_natural(q, k, v, F: int, H: int, W: int, tau: float, gamma: float,
                                    sm_scale: float | None = None, block_q: int = 128, block_k: int = 64,
                                    vote_threshold: int = 1, tile_h: int = 8, tile_w: int = 8, entropy: bool = True,
                                    lse: bool = False, want_mask: bool = False, out=None, ent_out=None, lse_out=None,
                                    kv_count=None, kv_index=None, block_mask=None):
    """dense_attn_entropy_mask on natural-order q, k, v (o natural; H, lse and the lists tile-major)."""
    return _dense_mask("tra_dense_attn_entropy_mask_natural", q, k, v, F, H, W, tau, gamma, sm_scale, block_q,
                       block_k, vote_threshold, tile_h, tile_w, entropy, lse, want_mask, out, ent_out, lse_out,
                       kv_count, kv_index, block_mask)


def mask_prepare(F, H, W, tau, gamma, block_q=128, block_k=64, tile_h=8, tile_w=8) -> None:
    _call("tra_mask_prepare", F, H, W, float(tau), float(gamma), block_q, block_k, tile_h, tile_w)


def natural_prepare(F, H, W, tile_h=8, tile_w=8) -> None:
    """Build and upload the tile-major map of the natural-order calls ahead of a timed region."""
    _call("tra_natural_prepare", F, H, W, tile_h, tile_w)


def build_block_mask(entropy, F: int, H: int, W: int, tau: float, gamma: float, block_q: int = 128,
                     block_k: int = 64, vote_threshold: int = 1, tile_h: int = 8, tile_w: int = 8,
                     want_mask: bool = False, kv_count=None, kv_index=None, block_mask=None):
    """entropy fp32 [outer][N] (tile-major) -> (kv_count [outer][nqb], kv_index [outer][nqb][nkb], mask|None)."""
    torch = _torch()
    _dev(entropy, "entropy")
    if entropy.dtype != torch.float32 or entropy.dim() != 2:
        raise ValueError("entropy must be float32 [outer][N]")
    outer, N = entropy.shape
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    cnt = _buf(kv_count, "kv_count", (outer, nqb), torch.int32, entropy)
    idx = _buf(kv_index, "kv_index", (outer, nqb, nkb), torch.int32, entropy)
    msk = _buf(block_mask, "block_mask", (outer, nqb, nkb), torch.uint8, entropy) \
        if (want_mask or block_mask is not None) else None
    _call("tra_build_block_mask", _ptr(entropy), outer, F, H, W, float(tau), float(gamma), block_q, block_k,
          int(vote_threshold), tile_h, tile_w, _ptr(cnt), _ptr(idx), idx.numel(), _ptr(msk), _stream(entropy))
    return cnt, idx, msk


def mask_prepare_1d(F, H, W, tau, block_q=128, block_k=64, tile_h=8, tile_w=8) -> None:
    _call("tra_mask_prepare_1d", F, H, W, float(tau), block_q, block_k, tile_h, tile_w)


def build_block_mask_1d(entropy, F: int, H: int, W: int, tau: float, block_q: int = 128, block_k: int = 64,
                        vote_threshold: int = 1, tile_h: int = 8, tile_w: int = 8, want_mask: bool = False,
                        kv_count=None, kv_index=None, block_mask=None):
    """The 1D-distance variant: query i keeps the keys within tau*exp(H_i)/2 of it in the natural raster
    sequence.  entropy fp32 [outer][N] (tile-major) -> (kv_count, kv_index, mask|None) as build_block_mask."""
    torch = _torch()
    _dev(entropy, "entropy")
    if entropy.dtype != torch.float32 or entropy.dim() != 2:
        raise ValueError("entropy must be float32 [outer][N]")
    outer, N = entropy.shape
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    cnt = _buf(kv_count, "kv_count", (outer, nqb), torch.int32, entropy)
    idx = _buf(kv_index, "kv_index", (outer, nqb, nkb), torch.int32, entropy)
    msk = _buf(block_mask, "block_mask", (outer, nqb, nkb), torch.uint8, entropy) \
        if (want_mask or block_mask is not None) else None
    _call("tra_build_block_mask_1d", _ptr(entropy), outer, F, H, W, float(tau), block_q, block_k, int(vote_threshold),
          tile_h, tile_w, _ptr(cnt), _ptr(idx), idx.numel(), _ptr(msk), _stream(entropy))
    return cnt, idx, msk


def block_sparse_attn(q, k, v, kv_count, kv_index, block_q: int = 128, block_k: int = 64,
                      sm_scale: float | None = None, lse: bool = False, out=None, lse_out=None):
    """Attention of each query over the tokens of its q-block's retained k-blocks.  Returns (o, lse)."""
    torch = _torch()
    outer, N, D = _check_qkv(q, k, v)
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    if kv_count is None or kv_index is None:
        raise ValueError("kv_count and kv_index are required")
    _buf(kv_count, "kv_count", (outer, nqb), torch.int32, q)
    _buf(kv_index, "kv_index", (outer, nqb, nkb), torch.int32, q)
    o = _buf(out, "out", q.shape, q.dtype, q)
    L = _buf(lse_out, "lse_out", (outer, N), torch.float32, q) if lse else None
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    _call("tra_block_sparse_attn", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(kv_count), _ptr(kv_index),
          outer, N, D, _dt(q), scale, block_q, block_k, _stream(q))
    return o, L


def block_sparse_attn_fp8(q, k, v, kv_count, kv_index, block_q: int = 128, block_k: int = 64,
                          sm_scale: float | None = None, lse: bool = False, out=None, lse_out=None, order=None):
    """block_sparse_attn with fp8 (OCP E4M3, torch.float8_e4m3fn) q and k and bf16 v; o is bf16.
    order: None, or a schedule from sparse_schedule.  Returns (o, lse)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
        if t.dim() != 3:
            raise ValueError("%s must be [outer][N][D]" % n)
    if q.dtype != torch.float8_e4m3fn or k.dtype != torch.float8_e4m3fn or v.dtype != torch.bfloat16:
        raise ValueError("q and k must be float8_e4m3fn, v bfloat16")
    if not (q.shape == k.shape == v.shape) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must share shape and device")
    outer, N, D = q.shape
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    if kv_count is None or kv_index is None:
        raise ValueError("kv_count and kv_index are required")
    _buf(kv_count, "kv_count", (outer, nqb), torch.int32, q)
    _buf(kv_index, "kv_index", (outer, nqb, nkb), torch.int32, q)
    if order is not None:
        _buf(order, "order", (outer * nqb,), torch.int32, q)
    o = _buf(out, "out", v.shape, torch.bfloat16, q)
    L = _buf(lse_out, "lse_out", (outer, N), torch.float32, q) if lse else None
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    _call("tra_block_sparse_attn_fp8", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(kv_count), _ptr(kv_index),
          _ptr(order), outer, N, D, scale, block_q, block_k, _stream(q))
    return o, L


def sparse_schedule(kv_count, F: int, H: int, W: int, block_q: int = 128, block_k: int = 64, tile_h: int = 8,
                    tile_w: int = 8, out=None):
    """The order the block-sparse calls take the (head, q-block) rows in: int32 [outer * nqb]
    (longest first for short grids, the spatial band order otherwise)."""
    torch = _torch()
    _dev(kv_count, "kv_count")
    if kv_count.dtype != torch.int32 or kv_count.dim() != 2:
        raise ValueError("kv_count must be int32 [outer][nqb]")
    outer, nqb = kv_count.shape
    if nqb != -(-(F * H * W) // block_q):
        raise ValueError("kv_count has %d q-blocks, the grid %d" % (nqb, -(-(F * H * W) // block_q)))
    order = _buf(out, "out", (outer * nqb,), torch.int32, kv_count)
    _call("tra_sparse_schedule", _ptr(kv_count), outer, F, H, W, block_q, block_k, tile_h, tile_w, _ptr(order),
          order.numel(), _stream(kv_count))
    return order


def block_sparse_attn_scheduled(q, k, v, kv_count, kv_index, order, block_q: int = 128, block_k: int = 64,
                                sm_scale: float | None = None, lse: bool = False, out=None, lse_out=None):
    """block_sparse_attn with the workgroups taking the rows in `order` (from sparse_schedule);
    the same results bit for bit.  Returns (o, lse)."""
    torch = _torch()
    outer, N, D = _check_qkv(q, k, v)
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    if kv_count is None or kv_index is None or order is None:
        raise ValueError("kv_count, kv_index and order are required")
    _buf(kv_count, "kv_count", (outer, nqb), torch.int32, q)
    _buf(kv_index, "kv_index", (outer, nqb, nkb), torch.int32, q)
    _buf(order, "order", (outer * nqb,), torch.int32, q)
    o = _buf(out, "out", q.shape, q.dtype, q)
    L = _buf(lse_out, "lse_out", (outer, N), torch.float32, q) if lse else None
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    _call("tra_block_sparse_attn_scheduled", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(kv_count),
          _ptr(kv_index), _ptr(order), outer, N, D, _dt(q), scale, block_q, block_k, _stream(q))
    return o, L


def dense_attn_entropy_natural(q, k, v, F: int, H: int, W: int, sm_scale: float | None = None, entropy: bool = True,
                               lse: bool = False, tile_h: int = 8, tile_w: int = 8, out=None, ent_out=None,
                               lse_out=None):
    """dense_attn_entropy on natural-order q, k, v (the sums over keys taken in natural order); o in
    natural order, H and lse indexed by tile-major position.  Returns (o, H, lse)."""
    torch = _torch()
    outer, N, D = _check_qkv(q, k, v)
    if N != F * H * W:
        raise ValueError("N must equal F*H*W")
    o = _buf(out, "out", q.shape, q.dtype, q)
    Hh = _buf(ent_out, "ent_out", (outer, N), torch.float32, q) if entropy else None
    L = _buf(lse_out, "lse_out", (outer, N), torch.float32, q) if lse else None
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    _call("tra_dense_attn_entropy_natural", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(Hh), _ptr(L), outer, F, H, W,
          D, _dt(q), scale, tile_h, tile_w, _stream(q))
    return o, Hh, L


def block_sparse_attn_natural(q, k, v, kv_count, kv_index, F: int, H: int, W: int, block_q: int = 128,
                              block_k: int = 64, sm_scale: float | None = None, lse: bool = False, tile_h: int = 8,
                              tile_w: int = 8, out=None, lse_out=None):
    """block_sparse_attn on natural-order q, k, v (kv_count / kv_index: the tile-major block lists);
    o in natural order, lse indexed by tile-major position.  Returns (o, lse)."""
    torch = _torch()
    outer, N, D = _check_qkv(q, k, v)
    if N != F * H * W:
        raise ValueError("N must equal F*H*W")
    nqb, nkb = -(-N // block_q), -(-N // block_k)
    if kv_count is None or kv_index is None:
        raise ValueError("kv_count and kv_index are required")
    _buf(kv_count, "kv_count", (outer, nqb), torch.int32, q)
    _buf(kv_index, "kv_index", (outer, nqb, nkb), torch.int32, q)
    o = _buf(out, "out", q.shape, q.dtype, q)
    L = _buf(lse_out, "lse_out", (outer, N), torch.float32, q) if lse else None
    scale = (1.0 / D ** 0.5) if sm_scale is None else float(sm_scale)
    _call("tra_block_sparse_attn_natural", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(kv_count),
          _ptr(kv_index), outer, F, H, W, D, _dt(q), scale, block_q, block_k, tile_h, tile_w, _stream(q))
    return o, L
