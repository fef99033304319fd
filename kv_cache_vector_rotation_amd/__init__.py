"""Python binding of libturboquant (TurboQuant KV-cache path on MI355X).

A thin ctypes layer over the C ABI declared in include/turboquant.h. It only
marshals arguments: torch tensors supply device memory and the stream, and
every step of quantization and attention runs in the library's HIP kernels.
The functions carry the C names (tq_build_codebook, tq_quantize,
tq_attn_decode, ...). If the shared library has not been built, loading it
raises immediately; there is no fallback path.

Helpers:
  Quantizer  -- device copies of a quantizer instance (rotation, sketch,
                folded sketch, float32 codebook) assembled from its parts.
  Cache      -- caller-owned compressed-cache tensors for one record format.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libturboquant.so")

TQ_OK = 0
TQ_ERR_INVALID = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_NOCONVERGE = -3
TQ_ERR_WORKSPACE = -4
TQ_ERR_DEVICE = -5
TQ_F32 = 0
TQ_BF16 = 1
TQ_TOKEN_MAJOR = 0
TQ_BLOCK32 = 1

TQ_PHASE_PREP = 1
TQ_PHASE_SPLIT = 2
TQ_PHASE_COMBINE = 4
TQ_PHASE_ALL = 7

SYMBOLS = ("tq_abi_version", "tq_status_string", "tq_build_codebook", "tq_record_layout",
           "tq_fold_sketch", "tq_quantize", "tq_attn_decode_workspace_bytes", "tq_attn_decode",
           "tq_attn_decode_phases", "tq_attn_decode_append", "tq_attn_decode_bf16_workspace_bytes",
           "tq_attn_decode_bf16", "tq_search_workspace_bytes", "tq_search", "tq_attn_decode_paged",
           "tq_attn_decode_scratch")


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {tq_status_string(status)} ({status})")
        self.status = status


class tq_layout(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_groups", C.c_int32), ("group_dim", C.c_int32 * 2),
                ("mse_bits", C.c_int32 * 2), ("mse_only", C.c_int32),
                ("norm_f16", C.c_int32)]


class tq_quantizer(C.Structure):
    _fields_ = [("layout", tq_layout), ("rot", C.c_void_p), ("sketch", C.c_void_p),
                ("sketch_rot", C.c_void_p), ("centroids", C.c_void_p), ("boundaries", C.c_void_p)]


class tq_cache(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("signs", C.c_void_p), ("norms", C.c_void_p),
                ("n_rows", C.c_int64)]


class tq_record_info(C.Structure):
    _fields_ = [("code_words", C.c_int32), ("sign_words", C.c_int32), ("norm_floats", C.c_int32),
                ("block_code_words", C.c_int32), ("block_sign_words", C.c_int32),
                ("record_bits", C.c_int32)]


class tq_rows(C.Structure):
    _fields_ = [("dst_rows", C.c_void_p), ("seg_len", C.c_int64), ("seg_stride", C.c_int64),
                ("seg_offset", C.c_int64)]


class tq_append(C.Structure):
    _fields_ = [("x", C.c_void_p), ("dtype", C.c_int), ("n_vec", C.c_int64), ("x_row_stride", C.c_int64),
                ("rows", tq_rows)]


class tq_decode_shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("n_split", C.c_int32), ("n_ctx", C.c_int64), ("cache_capacity", C.c_int64),
                ("scale", C.c_float), ("n_q_tokens", C.c_int32)]


class tq_paging(C.Structure):
    _fields_ = [("block_table", C.c_void_p), ("seq_lens", C.c_void_p), ("max_blocks", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """The loaded shared library (loads it on first use; raises if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libturboquant is not built ({LIB_PATH} missing); run "
                              "python -m kv_cache_vector_rotation_amd.build")
        try:
            import torch
            if torch.cuda.is_available():
                # let torch bring up the HIP runtime before the library's
                # kernels are registered with it
                torch.cuda.init()
        except ImportError:
            pass
        L = C.CDLL(LIB_PATH)
        L.tq_abi_version.restype = C.c_int
        L.tq_status_string.restype = C.c_char_p
        L.tq_status_string.argtypes = [C.c_int]
        L.tq_build_codebook.restype = C.c_int
        L.tq_build_codebook.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_double,
                                        C.POINTER(C.c_double), C.POINTER(C.c_double),
                                        C.POINTER(C.c_double)]
        L.tq_record_layout.restype = C.c_int
        L.tq_record_layout.argtypes = [C.POINTER(tq_layout), C.POINTER(tq_record_info)]
        L.tq_fold_sketch.restype = C.c_int
        L.tq_fold_sketch.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
        L.tq_quantize.restype = C.c_int
        L.tq_quantize.argtypes = [C.POINTER(tq_quantizer), C.c_int, C.c_void_p, C.c_int, C.c_int64,
                                  C.c_int64, C.POINTER(tq_rows), C.POINTER(tq_cache), C.c_void_p]
        L.tq_attn_decode_workspace_bytes.restype = C.c_int
        L.tq_attn_decode_workspace_bytes.argtypes = [C.POINTER(tq_quantizer), C.POINTER(tq_quantizer),
                                                     C.POINTER(tq_decode_shape), C.POINTER(C.c_size_t)]
        L.tq_attn_decode.restype = C.c_int
        L.tq_attn_decode.argtypes = [C.POINTER(tq_quantizer), C.POINTER(tq_quantizer),
                                     C.POINTER(tq_decode_shape), C.c_void_p, C.c_int,
                                     C.POINTER(tq_cache), C.POINTER(tq_cache), C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_size_t, C.c_void_p]
        L.tq_attn_decode_phases.restype = C.c_int
        L.tq_attn_decode_phases.argtypes = [C.c_uint] + L.tq_attn_decode.argtypes
        L.tq_attn_decode_append.restype = C.c_int
        L.tq_attn_decode_append.argtypes = (L.tq_attn_decode.argtypes[:3] +
                                            [C.POINTER(tq_append), C.POINTER(tq_append)] +
                                            L.tq_attn_decode.argtypes[3:])
        L.tq_attn_decode_bf16_workspace_bytes.restype = C.c_int
        L.tq_attn_decode_bf16_workspace_bytes.argtypes = [C.POINTER(tq_decode_shape), C.c_int,
                                                          C.POINTER(C.c_size_t)]
        L.tq_attn_decode_bf16.restype = C.c_int
        L.tq_attn_decode_bf16.argtypes = [C.POINTER(tq_decode_shape), C.c_int, C.c_void_p, C.c_int, C.c_void_p,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                          C.c_void_p]
        L.tq_attn_decode_paged.restype = C.c_int
        L.tq_attn_decode_paged.argtypes = (L.tq_attn_decode.argtypes[:3] + [C.POINTER(tq_paging)] +
                                           L.tq_attn_decode.argtypes[3:])
        L.tq_attn_decode_scratch.restype = C.c_int
        L.tq_attn_decode_scratch.argtypes = (L.tq_attn_decode.argtypes[:9] + [C.c_void_p])
        L.tq_search_workspace_bytes.restype = C.c_int
        L.tq_search_workspace_bytes.argtypes = [C.POINTER(tq_quantizer), C.c_int64, C.c_int64, C.c_int,
                                                C.POINTER(C.c_size_t)]
        L.tq_search.restype = C.c_int
        L.tq_search.argtypes = [C.POINTER(tq_quantizer), C.POINTER(tq_cache), C.c_int64, C.c_void_p, C.c_int,
                                C.c_int64, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where)


def make_layout(dims: Sequence[int], mse_bits: Sequence[int], mse_only: bool = False,
                norm_f16: bool = False) -> tq_layout:
    l = tq_layout()
    l.d = int(sum(dims))
    l.n_groups = len(dims)
    l.mse_only = int(bool(mse_only))
    l.norm_f16 = int(bool(norm_f16))
    for g, (d, m) in enumerate(zip(dims, mse_bits)):
        l.group_dim[g] = int(d)
        l.mse_bits[g] = int(m)
    return l


# ---------------------------------------------------------------------------
# Host-only entry points
# ---------------------------------------------------------------------------

def tq_abi_version() -> int:
    return int(lib().tq_abi_version())


def tq_status_string(status: int) -> str:
    return lib().tq_status_string(int(status)).decode()


def tq_build_codebook(d: int, mse_bits: int, max_iter: int = 0, tol: float = 0.0):
    """(centroids [2^m] float64, boundaries [2^m - 1] float64, mse_per_coord)."""
    L = 1 << mse_bits if 1 <= mse_bits <= 4 else 1
    c = (C.c_double * L)()
    t = (C.c_double * max(L - 1, 1))()
    mse = C.c_double()
    _check(lib().tq_build_codebook(d, mse_bits, max_iter, tol, c, t, C.byref(mse)),
           "tq_build_codebook")
    return np.array(c[:L]), np.array(t[:L - 1]), float(mse.value)


def tq_record_layout(layout: tq_layout) -> tq_record_info:
    info = tq_record_info()
    _check(lib().tq_record_layout(C.byref(layout), C.byref(info)), "tq_record_layout")
    return info


def tq_fold_sketch(rot: np.ndarray, sketch: np.ndarray) -> np.ndarray:
    rot = np.ascontiguousarray(rot, dtype=np.float32)
    sketch = np.ascontiguousarray(sketch, dtype=np.float32)
    d = rot.shape[0]
    out = np.empty((d, d), dtype=np.float32)
    _check(lib().tq_fold_sketch(d, rot.ctypes.data, sketch.ctypes.data, out.ctypes.data),
           "tq_fold_sketch")
    return out


# ---------------------------------------------------------------------------
# Device objects
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _dev(t, name: str, dtypes, device=None, numel: Optional[int] = None,
         min_numel: Optional[int] = None, optional: bool = False) -> Optional[int]:
    """Device address of tensor ``t`` after checking what the C ABI cannot:
    its dtype, contiguity and size, that it lives on the GPU, and that it is
    on ``device`` (the call's device). Raises ValueError otherwise."""
    torch = _torch()
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    dts = dtypes if isinstance(dtypes, (tuple, list)) else (dtypes,)
    if t.dtype not in dts:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dts)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's tensors are on {device}")
    return int(t.data_ptr())


def _call_device(t, name: str):
    """The device of the call's leading tensor, which must be the current
    device (kernels are launched there)."""
    torch = _torch()
    if t is None or not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return t.device


def _qdtype(t, name: str) -> int:
    torch = _torch()
    dt = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}.get(getattr(t, "dtype", None))
    if dt is None:
        raise ValueError(f"{name} must be float32 or bfloat16")
    return dt


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


@dataclass
class Quantizer:
    """Device copies of one quantizer instance plus its ABI struct."""
    layout: tq_layout
    dims: tuple
    mse_bits: tuple
    rot: "object"
    sketch: "object"
    sketch_rot: "object"
    centroids: "object"
    boundaries: "object"

    @staticmethod
    def from_parts(rotations: Sequence[np.ndarray], sketches: Sequence[np.ndarray],
                   mse_bits: Sequence[int], perm: Optional[np.ndarray] = None,
                   device: str = "cuda", mse_only: bool = False, norm_f16: bool = False) -> "Quantizer":
        """Assemble rot = blockdiag(Pi_g) P and sketch = blockdiag(S_g) P (P the
        channel permutation x -> x[perm]), fold sketch rot^T on the host, and
        build the float32 codebooks with tq_build_codebook."""
        torch = _torch()
        dims = [int(r.shape[0]) for r in rotations]
        d = sum(dims)
        perm = np.arange(d) if perm is None else np.asarray(perm, dtype=np.int64)
        bd_r = np.zeros((d, d), dtype=np.float64)
        bd_s = np.zeros((d, d), dtype=np.float64)
        o = 0
        for r, s in zip(rotations, sketches):
            g = r.shape[0]
            bd_r[o:o + g, o:o + g] = r
            bd_s[o:o + g, o:o + g] = s
            o += g
        rot = np.zeros((d, d), dtype=np.float32)
        sk = np.zeros((d, d), dtype=np.float32)
        rot[:, perm] = bd_r.astype(np.float32)
        sk[:, perm] = bd_s.astype(np.float32)
        skr = tq_fold_sketch(rot, sk)
        cents, bnds = [], []
        for g, m in zip(dims, mse_bits):
            c, t, _ = tq_build_codebook(g, int(m))
            cents.append(c.astype(np.float32))
            bnds.append(t.astype(np.float32))
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return Quantizer(layout=make_layout(dims, mse_bits, mse_only, norm_f16), dims=tuple(dims),
                         mse_bits=tuple(int(m) for m in mse_bits), rot=to(rot), sketch=to(sk),
                         sketch_rot=to(skr), centroids=to(np.concatenate(cents)),
                         boundaries=to(np.concatenate(bnds)))

    def struct(self, device=None) -> tq_quantizer:
        """The ABI struct; with ``device`` the tensors are checked first
        (float32, contiguous, sizes of the layout, on that device)."""
        q = tq_quantizer()
        q.layout = self.layout
        if device is None:
            q.rot, q.sketch, q.sketch_rot = _ptr(self.rot), _ptr(self.sketch), _ptr(self.sketch_rot)
            q.centroids, q.boundaries = _ptr(self.centroids), _ptr(self.boundaries)
            return q
        torch = _torch()
        d = int(self.layout.d)
        nc = sum(1 << m for m in self.mse_bits)
        q.rot = _dev(self.rot, "quantizer.rot", torch.float32, device, numel=d * d)
        q.sketch = _dev(self.sketch, "quantizer.sketch", torch.float32, device, numel=d * d)
        q.sketch_rot = _dev(self.sketch_rot, "quantizer.sketch_rot", torch.float32, device, numel=d * d)
        q.centroids = _dev(self.centroids, "quantizer.centroids", torch.float32, device, numel=nc)
        q.boundaries = _dev(self.boundaries, "quantizer.boundaries", torch.float32, device,
                            numel=nc - len(self.mse_bits))
        return q


@dataclass
class Cache:
    """Compressed-cache tensors (caller-owned device memory)."""
    fmt: int
    n_rows: int
    codes: "object"
    signs: "object"
    norms: "object"

    @staticmethod
    def empty(quantizer: Quantizer, n_rows: int, fmt: int, device: str = "cuda") -> "Cache":
        torch = _torch()
        info = tq_record_layout(quantizer.layout)
        if fmt == TQ_BLOCK32:
            if n_rows % 32:
                raise ValueError("TQ_BLOCK32 needs a multiple of 32 rows")
            nb = n_rows // 32
            codes = torch.zeros(nb * info.block_code_words, dtype=torch.int32, device=device)
            signs = torch.zeros(nb * info.block_sign_words, dtype=torch.int32, device=device)
        else:
            codes = torch.zeros(n_rows * info.code_words, dtype=torch.int32, device=device)
            signs = torch.zeros(n_rows * info.sign_words, dtype=torch.int32, device=device)
        ndt = torch.float16 if quantizer.layout.norm_f16 else torch.float32
        norms = torch.zeros(n_rows * info.norm_floats, dtype=ndt, device=device)
        return Cache(fmt=fmt, n_rows=n_rows, codes=codes, signs=signs, norms=norms)

    def struct(self, quantizer: Optional["Quantizer"] = None, device=None) -> tq_cache:
        """The ABI struct; with ``quantizer`` and ``device`` the tensors are
        checked first (int32 words and float32 / float16 norms as the layout
        says, large enough for n_rows records, on that device)."""
        c = tq_cache()
        c.n_rows = int(self.n_rows)
        if quantizer is None:
            c.codes, c.signs, c.norms = _ptr(self.codes), _ptr(self.signs), _ptr(self.norms)
            return c
        torch = _torch()
        info = tq_record_layout(quantizer.layout)
        if self.fmt == TQ_BLOCK32:
            if self.n_rows % 32:
                raise ValueError("a TQ_BLOCK32 cache needs a multiple of 32 rows")
            nw_c, nw_s = self.n_rows // 32 * info.block_code_words, self.n_rows // 32 * info.block_sign_words
        else:
            nw_c, nw_s = self.n_rows * info.code_words, self.n_rows * info.sign_words
        ndt = torch.float16 if quantizer.layout.norm_f16 else torch.float32
        c.codes = _dev(self.codes, "cache.codes", torch.int32, device, min_numel=nw_c)
        c.signs = (_dev(self.signs, "cache.signs", torch.int32, device, min_numel=nw_s) if nw_s
                   else (None if self.signs is None or self.signs.numel() == 0 else _ptr(self.signs)))
        c.norms = _dev(self.norms, "cache.norms", ndt, device, min_numel=self.n_rows * info.norm_floats)
        return c

    def clone(self) -> "Cache":
        return Cache(self.fmt, self.n_rows, self.codes.clone(), self.signs.clone(), self.norms.clone())


def decode_shape(batch: int, n_q_heads: int, n_kv_heads: int, n_ctx: int, capacity: int,
                 scale: float, n_split: int = 0, n_q_tokens: int = 1) -> tq_decode_shape:
    s = tq_decode_shape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.n_split = batch, n_q_heads, n_kv_heads, n_split
    s.n_ctx, s.cache_capacity, s.scale, s.n_q_tokens = n_ctx, capacity, scale, n_q_tokens
    return s


# ---------------------------------------------------------------------------
# Device entry points
# ---------------------------------------------------------------------------

def _x_rows(x, name: str, d: int, device=None):
    """(address, dtype code, n_vec, row stride) of a [n_vec, >= d] input."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit stride along the channels")
    dt = _qdtype(x, name)
    if x.shape[1] < d or (x.shape[0] > 1 and x.stride(0) < d):
        raise ValueError(f"{name} rows must hold at least d = {d} channels")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, the call's tensors are on {device}")
    return int(x.data_ptr()), dt, int(x.shape[0]), int(x.stride(0))


def _rows_ptr(dst_rows, n_vec: int, device):
    torch = _torch()
    return _dev(dst_rows, "dst_rows", torch.int64, device, numel=n_vec, optional=True)


def tq_quantize(quantizer: Quantizer, fmt: int, x, cache: Cache, dst_rows=None, seg_len: int = 1,
                seg_stride: int = 1, seg_offset: int = 0, stream=None) -> None:
    """Quantize the rows of x ([n_vec, >= d], float32 or bfloat16, on the GPU)
    into ``cache``. Rows: dst_rows (int64 device tensor [n_vec]) if given, else
    (i // seg_len) * seg_stride + seg_offset + i % seg_len."""
    dev = _call_device(x, "x")
    xp, dt, n_vec, stride = _x_rows(x, "x", int(quantizer.layout.d), dev)
    if cache.fmt != fmt:
        raise ValueError("cache.fmt differs from fmt")
    rows = tq_rows()
    rows.dst_rows = _rows_ptr(dst_rows, n_vec, dev)
    rows.seg_len, rows.seg_stride, rows.seg_offset = seg_len, seg_stride, seg_offset
    q = quantizer.struct(dev)
    c = cache.struct(quantizer, dev)
    _check(lib().tq_quantize(C.byref(q), fmt, xp, dt, n_vec, stride, C.byref(rows), C.byref(c),
                             _stream(stream)), "tq_quantize")


def tq_attn_decode_workspace_bytes(kq: Quantizer, vq: Optional[Quantizer], shape: tq_decode_shape) -> int:
    n = C.c_size_t()
    kqs = kq.struct()
    vqs = vq.struct() if vq is not None else None
    _check(lib().tq_attn_decode_workspace_bytes(C.byref(kqs), C.byref(vqs) if vqs is not None else None,
                                                C.byref(shape), C.byref(n)),
           "tq_attn_decode_workspace_bytes")
    return int(n.value)


def _decode_args(kq: Quantizer, vq: Optional[Quantizer], shape: tq_decode_shape, q, k_cache: Cache,
                 v_cache: Optional[Cache], logits, out):
    """Checked ABI arguments shared by the decode wrappers: (device, q address,
    q dtype, kq struct, vq struct or None, K cache struct, V cache struct or
    None, logits address, out address)."""
    torch = _torch()
    dev = _call_device(q, "q")
    T = max(1, int(shape.n_q_tokens))
    B, HQ, d = int(shape.batch), int(shape.n_q_heads), int(kq.layout.d)
    dt = _qdtype(q, "q")
    qp = _dev(q, "q", (torch.float32, torch.bfloat16), dev, numel=B * T * HQ * d)
    if k_cache.fmt != TQ_TOKEN_MAJOR:
        raise ValueError("k_cache must be a TQ_TOKEN_MAJOR cache")
    kqs, kc = kq.struct(dev), k_cache.struct(kq, dev)
    vqs = vc = None
    if vq is not None:
        if v_cache is None or v_cache.fmt != TQ_BLOCK32:
            raise ValueError("v_cache must be a TQ_BLOCK32 cache when vq is given")
        vqs, vc = vq.struct(dev), v_cache.struct(vq, dev)
    lp = _dev(logits, "logits", torch.float32, dev, numel=B * HQ * T * int(shape.n_ctx), optional=True)
    op = _dev(out, "out", torch.float32, dev, numel=B * T * HQ * d, optional=True)
    return dev, qp, dt, kqs, vqs, kc, vc, lp, op


def _workspace(workspace, kq, vq, shape, dev):
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(tq_attn_decode_workspace_bytes(kq, vq, shape), dtype=torch.uint8, device=dev)
    return _dev(workspace, "workspace", torch.uint8, dev), workspace.numel()


def _ref(x):
    return C.byref(x) if x is not None else None


def tq_attn_decode(kq: Quantizer, vq: Optional[Quantizer], shape: tq_decode_shape, q,
                   k_cache: Cache, v_cache: Optional[Cache], logits=None, out=None, workspace=None,
                   stream=None) -> None:
    """One decode step (see include/turboquant.h). q: [batch, n_q_heads, d]
    float32/bfloat16 contiguous on the GPU; logits / out: float32 device
    tensors or None; workspace: uint8 device tensor (allocated here if None)."""
    tq_attn_decode_phases(TQ_PHASE_ALL, kq, vq, shape, q, k_cache, v_cache, logits, out, workspace,
                          stream)


def tq_attn_decode_phases(phases: int, kq: Quantizer, vq: Optional[Quantizer], shape: tq_decode_shape,
                          q, k_cache: Cache, v_cache: Optional[Cache], logits=None, out=None,
                          workspace=None, stream=None) -> None:
    """The stages of tq_attn_decode selected by ``phases`` (TQ_PHASE_* bits);
    stages share state through ``workspace``, which must then be given."""
    dev, qp, dt, kqs, vqs, kc, vc, lp, op = _decode_args(kq, vq, shape, q, k_cache, v_cache, logits, out)
    wp, wn = _workspace(workspace, kq, vq, shape, dev)
    _check(lib().tq_attn_decode_phases(phases, C.byref(kqs), _ref(vqs), C.byref(shape), qp, dt, C.byref(kc),
                                       _ref(vc), lp, op, wp, wn, _stream(stream)),
           "tq_attn_decode")


def tq_attn_decode_scratch(kq: Quantizer, vq: Optional[Quantizer], shape: tq_decode_shape, q,
                           k_cache: Cache, v_cache: Optional[Cache], logits=None, out=None,
                           stream=None) -> None:
    """tq_attn_decode with the library's static device workspace (no workspace
    argument, nothing allocated; see include/turboquant.h). Calls that overlap
    in time on one GPU race."""
    dev, qp, dt, kqs, vqs, kc, vc, lp, op = _decode_args(kq, vq, shape, q, k_cache, v_cache, logits, out)
    _check(lib().tq_attn_decode_scratch(C.byref(kqs), _ref(vqs), C.byref(shape), qp, dt, C.byref(kc),
                                        _ref(vc), lp, op, _stream(stream)),
           "tq_attn_decode_scratch")


def append_spec(x, dst_rows=None, seg_len: int = 1, seg_stride: int = 1, seg_offset: int = 0) -> tq_append:
    """Vectors to append within tq_attn_decode_append: the rows of x ([n_vec,
    >= d] float32/bfloat16 on the GPU) go to dst_rows (int64 [n_vec]), or by
    segments as in tq_quantize. The returned struct keeps a reference to its
    tensors; tq_attn_decode_append checks them against its quantizers."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit stride along the channels")
    a = tq_append()
    a.x = _ptr(x)
    a.dtype = _qdtype(x, "x")
    a.n_vec = x.shape[0]
    a.x_row_stride = x.stride(0)
    a.rows.dst_rows = _ptr(dst_rows)
    a.rows.seg_len, a.rows.seg_stride, a.rows.seg_offset = seg_len, seg_stride, seg_offset
    a._keep = (x, dst_rows)
    return a


def _check_append(a: Optional[tq_append], name: str, qz: Optional[Quantizer], dev) -> None:
    if a is None:
        return
    if qz is None:
        raise ValueError(f"{name} needs its quantizer")
    x, dst_rows = getattr(a, "_keep", (None, None))
    if x is None:
        raise ValueError(f"{name} must come from append_spec")
    _x_rows(x, f"{name}.x", int(qz.layout.d), dev)
    _rows_ptr(dst_rows, int(x.shape[0]), dev)


def tq_attn_decode_append(kq: Quantizer, vq: Optional[Quantizer], shape: tq_decode_shape, q,
                          k_cache: Cache, v_cache: Optional[Cache], k_new: Optional[tq_append] = None,
                          v_new: Optional[tq_append] = None, logits=None, out=None, workspace=None,
                          stream=None) -> None:
    """Appends k_new / v_new (append_spec structs, or None) to the caches and
    runs the decode step over them, as one launch for the appends and the
    query preparation followed by the split-K pass and the combine."""
    dev, qp, dt, kqs, vqs, kc, vc, lp, op = _decode_args(kq, vq, shape, q, k_cache, v_cache, logits, out)
    _check_append(k_new, "k_new", kq, dev)
    _check_append(v_new, "v_new", vq, dev)
    wp, wn = _workspace(workspace, kq, vq, shape, dev)
    _check(lib().tq_attn_decode_append(C.byref(kqs), _ref(vqs), C.byref(shape), _ref(k_new), _ref(v_new), qp, dt,
                                       C.byref(kc), _ref(vc), lp, op, wp, wn, _stream(stream)),
           "tq_attn_decode_append")


def tq_attn_decode_bf16_workspace_bytes(shape: tq_decode_shape, d: int = 128) -> int:
    n = C.c_size_t()
    _check(lib().tq_attn_decode_bf16_workspace_bytes(C.byref(shape), d, C.byref(n)),
           "tq_attn_decode_bf16_workspace_bytes")
    return int(n.value)


def tq_attn_decode_bf16(shape: tq_decode_shape, q, k, v, out, logits=None, workspace=None, stream=None) -> None:
    """Uncompressed baseline decode (see include/turboquant.h): q [batch,
    n_q_heads, d] float32/bfloat16; k bf16 [batch*n_kv_heads*capacity, d];
    v bf16 [batch*n_kv_heads*capacity/32, d, 32]; out / logits float32 device
    tensors; workspace: uint8 device tensor (allocated here if None)."""
    torch = _torch()
    dev = _call_device(q, "q")
    d = int(q.shape[-1])
    B, HQ, H, cap = int(shape.batch), int(shape.n_q_heads), int(shape.n_kv_heads), int(shape.cache_capacity)
    dt = _qdtype(q, "q")
    qp = _dev(q, "q", (torch.float32, torch.bfloat16), dev, numel=B * HQ * d)
    kp = _dev(k, "k", torch.bfloat16, dev, min_numel=B * H * cap * d)
    vp = _dev(v, "v", torch.bfloat16, dev, min_numel=B * H * cap * d)
    op = _dev(out, "out", torch.float32, dev, numel=B * HQ * d)
    lp = _dev(logits, "logits", torch.float32, dev, numel=B * HQ * int(shape.n_ctx), optional=True)
    if workspace is None:
        workspace = torch.empty(tq_attn_decode_bf16_workspace_bytes(shape, d), dtype=torch.uint8, device=dev)
    wp = _dev(workspace, "workspace", torch.uint8, dev)
    _check(lib().tq_attn_decode_bf16(C.byref(shape), d, qp, dt, kp, vp, lp, op, wp, workspace.numel(),
                                     _stream(stream)),
           "tq_attn_decode_bf16")


def tq_attn_decode_paged(kq: Quantizer, vq: Optional[Quantizer], shape: tq_decode_shape, block_table, q,
                         k_cache: Cache, v_cache: Optional[Cache], seq_lens=None, logits=None, out=None,
                         workspace=None, stream=None) -> None:
    """tq_attn_decode over a paged cache (see include/turboquant.h):
    block_table int32 device tensor [batch, max_blocks]; seq_lens int32
    device tensor [batch] or None."""
    torch = _torch()
    dev, qp, dt, kqs, vqs, kc, vc, lp, op = _decode_args(kq, vq, shape, q, k_cache, v_cache, logits, out)
    B = int(shape.batch)
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be an int32 tensor [batch, max_blocks]")
    bp = _dev(block_table, "block_table", torch.int32, dev)
    sp = _dev(seq_lens, "seq_lens", torch.int32, dev, numel=B, optional=True)
    wp, wn = _workspace(workspace, kq, vq, shape, dev)
    pg = tq_paging()
    pg.block_table = bp
    pg.seq_lens = sp
    pg.max_blocks = int(block_table.shape[-1])
    _check(lib().tq_attn_decode_paged(C.byref(kqs), _ref(vqs), C.byref(shape), C.byref(pg), qp, dt, C.byref(kc),
                                      _ref(vc), lp, op, wp, wn, _stream(stream)),
           "tq_attn_decode_paged")


def tq_search_workspace_bytes(quantizer: Quantizer, n_db: int, n_q: int, k: int) -> int:
    n = C.c_size_t()
    q = quantizer.struct()
    _check(lib().tq_search_workspace_bytes(C.byref(q), n_db, n_q, k, C.byref(n)), "tq_search_workspace_bytes")
    return int(n.value)


def tq_search(quantizer: Quantizer, db: Cache, n_db: int, q, k: int, out_idx=None, out_score=None,
              workspace=None, stream=None):
    """k best database rows per query (see include/turboquant.h): q [n_q, d]
    float32/bfloat16 device tensor; db a token-major Cache; returns
    (out_idx int64 [n_q, k], out_score float32 [n_q, k]) device tensors."""
    torch = _torch()
    dev = _call_device(q, "q")
    if q.dim() != 2 or q.shape[1] != quantizer.layout.d:
        raise ValueError("q must be a contiguous [n_q, d] tensor")
    dt = _qdtype(q, "q")
    n_q = int(q.shape[0])
    qp = _dev(q, "q", (torch.float32, torch.bfloat16), dev)
    if db.fmt != TQ_TOKEN_MAJOR:
        raise ValueError("db must be a TQ_TOKEN_MAJOR cache")
    if out_idx is None:
        out_idx = torch.empty((n_q, k), dtype=torch.int64, device=dev)
    if out_score is None:
        out_score = torch.empty((n_q, k), dtype=torch.float32, device=dev)
    ip = _dev(out_idx, "out_idx", torch.int64, dev, numel=n_q * k)
    scp = _dev(out_score, "out_score", torch.float32, dev, numel=n_q * k)
    if workspace is None:
        workspace = torch.empty(tq_search_workspace_bytes(quantizer, n_db, n_q, k), dtype=torch.uint8, device=dev)
    wp = _dev(workspace, "workspace", torch.uint8, dev)
    qs = quantizer.struct(dev)
    c = db.struct(quantizer, dev)
    _check(lib().tq_search(C.byref(qs), C.byref(c), n_db, qp, dt, n_q, k, ip, scp, wp, workspace.numel(),
                           _stream(stream)), "tq_search")
    return out_idx, out_score


__all__ = [
    "LIB_PATH", "SYMBOLS", "lib", "TQError", "Quantizer", "Cache", "make_layout", "decode_shape",
    "tq_abi_version", "tq_status_string", "tq_build_codebook", "tq_record_layout", "tq_fold_sketch",
    "tq_quantize", "tq_attn_decode_workspace_bytes", "tq_attn_decode", "tq_attn_decode_phases",
    "tq_attn_decode_append", "append_spec", "tq_append", "tq_attn_decode_bf16_workspace_bytes",
    "tq_attn_decode_bf16", "tq_search_workspace_bytes", "tq_search", "tq_attn_decode_paged", "tq_paging",
    "tq_attn_decode_scratch",
    "TQ_PHASE_PREP", "TQ_PHASE_SPLIT", "TQ_PHASE_COMBINE", "TQ_PHASE_ALL",
    "TQ_OK", "TQ_ERR_INVALID", "TQ_ERR_UNSUPPORTED", "TQ_ERR_NOCONVERGE", "TQ_ERR_WORKSPACE",
    "TQ_ERR_DEVICE", "TQ_F32", "TQ_BF16", "TQ_TOKEN_MAJOR", "TQ_BLOCK32",
]
