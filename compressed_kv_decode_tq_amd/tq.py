"""Thin Python binding of libtq (include/tq.h).

Argument marshalling only: every step of encode and decode runs in the HIP
kernels of libtq.so.  PyTorch provides device memory and the current stream.
Functions keep the C names without the ``tq_`` prefix.  A missing or unloadable
libtq.so raises at first use; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_OK, TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP = 0, -1, -2, -3, -4, -5
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_V_MINMAX, TQ_V_MSE = 0, 1
TQ_BYTES_DATA, TQ_BYTES_PARAMS, TQ_BYTES_RING = 0, 1, 2
MAX_LEVELS = 16

#: Every symbol include/tq.h declares.
EXPORTS = ("tq_make_codebook", "tq_memory_bytes", "tq_params_derived_bytes", "tq_prepare_params",
           "tq_encode_kv", "tq_ring_append", "tq_decode_workspace_bytes", "tq_decode_attn",
           "tq_decode_workspace_bytes_multi", "tq_decode_attn_multi", "tq_decode_attn_append",
           "tq_decode_attn_noalloc", "tq_time_next_launch", "tq_last_error", "tq_version")
TQ_KERNEL_DECODE_SCAN, TQ_KERNEL_ENCODE_KEYS, TQ_KERNEL_ENCODE_VALUES = 0, 1, 2


class TqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libtq error {code}: {msg}")
        self.code = code


class _Layout(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("key_mse_bits", ctypes.c_int32),
                ("key_qjl", ctypes.c_int32), ("value_kind", ctypes.c_int32),
                ("value_bits", ctypes.c_int32), ("value_group", ctypes.c_int32),
                ("scalar_dtype", ctypes.c_int32), ("key_half", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [("pi", ctypes.c_void_p), ("s", ctypes.c_void_p), ("derived", ctypes.c_void_p),
                ("k_centroids", ctypes.c_float * MAX_LEVELS),
                ("k_thresholds", ctypes.c_float * (MAX_LEVELS - 1)),
                ("v_centroids", ctypes.c_float * MAX_LEVELS),
                ("v_thresholds", ctypes.c_float * (MAX_LEVELS - 1)),
                ("k_centroids_hi", ctypes.c_float * MAX_LEVELS),
                ("k_thresholds_hi", ctypes.c_float * (MAX_LEVELS - 1))]


class _Cache(ctypes.Structure):
    _fields_ = [("k_planes", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
                ("k_rnorm", ctypes.c_void_p), ("v_planes", ctypes.c_void_p),
                ("v_meta", ctypes.c_void_p), ("v_norm", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("capacity", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtq.so (built in-tree by compressed_kv_decode_tq_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run python -m compressed_kv_decode_tq_amd.build")
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER
        L.tq_make_codebook.argtypes = [i32, i32, P(ctypes.c_float), P(ctypes.c_float)]
        L.tq_make_codebook.restype = ctypes.c_int
        L.tq_memory_bytes.argtypes = [P(_Layout), i32, i32, i64, i32, i32]
        L.tq_memory_bytes.restype = i64
        L.tq_params_derived_bytes.argtypes = [i32]
        L.tq_params_derived_bytes.restype = sz
        L.tq_prepare_params.argtypes = [i32, vp, vp, vp, sz, vp]
        L.tq_prepare_params.restype = ctypes.c_int
        L.tq_encode_kv.argtypes = [P(_Layout), P(_Params), vp, vp, i32, i64, P(i64), P(_Cache), vp]
        L.tq_encode_kv.restype = ctypes.c_int
        L.tq_ring_append.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, i32, P(i32), vp]
        L.tq_ring_append.restype = ctypes.c_int
        L.tq_decode_workspace_bytes.argtypes = [P(_Layout), i32, i32, i32, i64]
        L.tq_decode_workspace_bytes.restype = sz
        L.tq_decode_attn.argtypes = [P(_Layout), P(_Params), vp, i32, i32, P(_Cache), P(i64), vp, vp,
                                     i32, P(i32), ctypes.c_float, vp, vp, sz, vp]
        L.tq_decode_attn.restype = ctypes.c_int
        L.tq_decode_workspace_bytes_multi.argtypes = [P(_Layout), i32, i32, i32, i64, i32]
        L.tq_decode_workspace_bytes_multi.restype = sz
        L.tq_decode_attn_multi.argtypes = [P(_Layout), P(_Params), vp, i32, i32, i32, P(_Cache), P(i64), vp,
                                           vp, i32, P(i32), ctypes.c_float, vp, vp, sz, vp]
        L.tq_decode_attn_multi.restype = ctypes.c_int
        L.tq_decode_attn_append.argtypes = [P(_Layout), P(_Params), vp, i32, i32, P(_Cache), P(i64), vp, vp, i32,
                                            vp, vp, i32, P(i32), ctypes.c_float, vp, vp, sz, vp]
        L.tq_decode_attn_append.restype = ctypes.c_int
        L.tq_decode_attn_noalloc.argtypes = [P(_Layout), P(_Params), vp, i32, i32, P(_Cache), P(i64), vp, vp,
                                             i32, P(i32), ctypes.c_float, vp, vp]
        L.tq_decode_attn_noalloc.restype = ctypes.c_int
        L.tq_time_next_launch.argtypes = [i32, vp, vp]
        L.tq_time_next_launch.restype = ctypes.c_int
        L.tq_last_error.argtypes = []
        L.tq_last_error.restype = ctypes.c_char_p
        L.tq_version.argtypes = []
        L.tq_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != TQ_OK:
        raise TqError(rc, lib().tq_last_error().decode())


_LAYOUT_C: dict = {}  # Layout -> its C struct (a Layout is immutable)


@dataclasses.dataclass(frozen=True)
class Layout:
    head_dim: int = 128
    key_mse_bits: int = 2
    key_qjl: int = 1
    value_kind: int = TQ_V_MINMAX
    value_bits: int = 2
    value_group: int = 32
    scalar_dtype: int = TQ_F32
    key_half: int = 0  # 1: half of the rotated coordinates get key_mse_bits + 1 bits

    def c(self) -> _Layout:
        st = _LAYOUT_C.get(self)
        if st is None:
            st = _LAYOUT_C[self] = _Layout(self.head_dim, self.key_mse_bits, self.key_qjl, self.value_kind,
                                           self.value_bits, self.value_group, self.scalar_dtype, self.key_half)
        return st

    @property
    def key_planes(self) -> int:
        return self.key_mse_bits + self.key_qjl

    @property
    def scalar_torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.scalar_dtype == TQ_F32 else torch.float16


def make_codebook(d: int, bits: int):
    """Lloyd-Max centroids (2^bits) and thresholds (2^bits - 1) as float32 arrays."""
    c = (ctypes.c_float * (1 << bits))()
    t = (ctypes.c_float * max(1, (1 << bits) - 1))()
    _check(lib().tq_make_codebook(d, bits, c, t))
    return np.frombuffer(c, dtype=np.float32).copy(), np.frombuffer(t, dtype=np.float32)[: (1 << bits) - 1].copy()


def memory_bytes(layout: Layout, batch: int, num_kv_heads: int, n_tokens: int, ring_cap: int, what: int) -> int:
    lay = layout.c()
    r = lib().tq_memory_bytes(ctypes.byref(lay), batch, num_kv_heads, n_tokens, ring_cap, what)
    if r < 0:
        _check(int(r))
    return int(r)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


_F32, _BF16, _U8 = torch.float32, torch.bfloat16, torch.uint8


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_seq_list(name: str, xs, batch: int):
    _require(xs is not None and len(xs) == batch, f"{name} must hold one entry per sequence ({batch})")


def _check_device(cache: "Cache", **tensors):
    dev = cache.k_planes.device
    for name, t in tensors.items():
        if t is not None:
            _require(t.device == dev, f"{name} is on {t.device}, the cache on {dev}")


def _check_ring(cache: "Cache", ring_k, ring_v, n_ring, d: int):
    """Rings: both or neither; contiguous bf16 [B, R, H_kv, d] of one shape."""
    if ring_k is None and ring_v is None:
        return 0
    if (ring_k is not None and ring_v is not None and ring_k.dtype is _BF16 and ring_v.dtype is _BF16
            and ring_k.dim() == 4 and ring_k.shape == ring_v.shape and ring_k.shape[0] == cache.batch
            and ring_k.shape[2] == cache.num_kv_heads and ring_k.shape[3] == d and ring_k.shape[1] > 0
            and ring_k.is_contiguous() and ring_v.is_contiguous() and n_ring is not None
            and len(n_ring) == cache.batch):
        return int(ring_k.shape[1])
    _require(ring_k is not None and ring_v is not None, "ring_k and ring_v must be given together")
    for name, r in (("ring_k", ring_k), ("ring_v", ring_v)):
        _require(r.dtype == torch.bfloat16, f"{name} must be bf16")
        _require(r.is_contiguous(), f"{name} must be contiguous (a slice of a ring has the wrong row stride)")
        _require(r.dim() == 4 and r.shape[0] == cache.batch and r.shape[2] == cache.num_kv_heads
                 and r.shape[3] == d and r.shape[1] > 0,
                 f"{name} must be [{cache.batch}, R, {cache.num_kv_heads}, {d}], got {tuple(r.shape)}")
    _require(ring_k.shape == ring_v.shape, "ring_k and ring_v must have the same shape")
    _check_seq_list("n_ring", n_ring, cache.batch)
    return int(ring_k.shape[1])


def _check_decode(layout: Layout, q: torch.Tensor, cache: "Cache", n_compressed, out, workspace):
    """Shapes, dtypes, contiguity and devices of a decode call, checked before
    anything reaches the library (which trusts sizes it is given).  The common
    case is one expression; anything off goes through the detailed checks,
    which name the problem."""
    sh = q.shape
    dev = cache.k_planes.device
    if (len(sh) in (3, 4) and sh[0] == cache.batch and sh[-1] == layout.head_dim and sh[-2] > 0
            and sh[-2] % cache.num_kv_heads == 0 and (q.dtype is _F32 or q.dtype is _BF16) and q.device == dev
            and q.is_contiguous() and len(n_compressed) == cache.batch
            and (out is None or (out.dtype is _F32 and out.shape == sh and out.device == dev and out.is_contiguous()))
            and (workspace is None or (workspace.dtype is _U8 and workspace.device == dev
                                       and workspace.is_contiguous()))):
        return
    _check_decode_detail(layout, q, cache, n_compressed, out, workspace)


def _check_decode_detail(layout: Layout, q: torch.Tensor, cache: "Cache", n_compressed, out, workspace):
    d = layout.head_dim
    _require(q.dim() in (3, 4), "q must be [B, H_q, d] or [B, T, H_q, d]")
    _require(q.dtype in (torch.float32, torch.bfloat16), "q must be fp32 or bf16")
    _require(q.is_contiguous(), "q must be contiguous")
    _require(q.shape[0] == cache.batch, f"q holds {q.shape[0]} sequences, the cache {cache.batch}")
    _require(q.shape[-1] == d, f"q's last dimension {q.shape[-1]} is not head_dim {d}")
    h_q = q.shape[-2]
    _require(h_q > 0 and h_q % cache.num_kv_heads == 0,
             f"h_q = {h_q} must be a positive multiple of num_kv_heads = {cache.num_kv_heads}")
    _check_seq_list("n_compressed", n_compressed, cache.batch)
    if out is not None:
        _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == tuple(q.shape),
                 f"out must be contiguous fp32 of q's shape {tuple(q.shape)}")
    if workspace is not None:
        _require(workspace.dtype == torch.uint8 and workspace.is_contiguous(), "workspace must be contiguous uint8")
    _check_device(cache, q=q, out=out, workspace=workspace)


class Params:
    """Per-layer parameters on one device: Pi and S (fp32), the operands
    tq_prepare_params derives from them, and the codebook tables."""

    def __init__(self, layout: Layout, pi, s, device="cuda", stream=None,
                 k_codebook=None, v_codebook=None):
        d = layout.head_dim
        self.layout = layout
        self.pi = torch.as_tensor(np.asarray(pi, dtype=np.float32)).to(device).contiguous()
        self.s = torch.as_tensor(np.asarray(s, dtype=np.float32)).to(device).contiguous()
        nbytes = lib().tq_params_derived_bytes(d)
        if nbytes == 0:
            raise TqError(TQ_ERR_UNSUPPORTED, f"head_dim {d} is not built")
        self.derived = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _check(lib().tq_prepare_params(d, _ptr(self.pi), _ptr(self.s), _ptr(self.derived), nbytes, _stream(stream)))
        self.k_centroids, self.k_thresholds = k_codebook or make_codebook(d, layout.key_mse_bits)
        if layout.key_half:
            self.k_centroids_hi, self.k_thresholds_hi = make_codebook(d, layout.key_mse_bits + 1)
        else:
            self.k_centroids_hi = self.k_thresholds_hi = np.zeros(0, dtype=np.float32)
        if layout.value_kind == TQ_V_MSE:
            self.v_centroids, self.v_thresholds = v_codebook or make_codebook(d, layout.value_bits)
        else:
            self.v_centroids = self.v_thresholds = np.zeros(0, dtype=np.float32)

    def c(self) -> _Params:
        """The C struct; built on first use (a Params is not changed after
        construction)."""
        p = self.__dict__.get("_cstruct")
        if p is not None:
            return p
        p = _Params()
        p.pi, p.s, p.derived = _ptr(self.pi), _ptr(self.s), _ptr(self.derived)
        for i, x in enumerate(self.k_centroids):
            p.k_centroids[i] = float(x)
        for i, x in enumerate(self.k_thresholds):
            p.k_thresholds[i] = float(x)
        for i, x in enumerate(self.v_centroids):
            p.v_centroids[i] = float(x)
        for i, x in enumerate(self.v_thresholds):
            p.v_thresholds[i] = float(x)
        for i, x in enumerate(self.k_centroids_hi):
            p.k_centroids_hi[i] = float(x)
        for i, x in enumerate(self.k_thresholds_hi):
            p.k_thresholds_hi[i] = float(x)
        self._cstruct = p
        return p


class Cache:
    """Device tensors of a compressed cache (layout as in include/tq.h)."""

    def __init__(self, layout: Layout, batch: int, num_kv_heads: int, capacity: int, device="cuda"):
        if capacity % 32:
            raise ValueError("capacity must be a multiple of 32")
        d = layout.head_dim
        self.layout, self.batch, self.num_kv_heads, self.capacity = layout, batch, num_kv_heads, capacity
        sd = layout.scalar_torch_dtype
        shp = (batch, num_kv_heads, capacity)
        rec = layout.key_planes * d // 8 + layout.key_half * d // 16
        self.k_planes = torch.zeros(batch, num_kv_heads, (capacity + 63) // 64, 64 * rec,
                                    dtype=torch.uint8, device=device)
        self.k_norm = torch.zeros(shp, dtype=sd, device=device)
        self.k_rnorm = torch.zeros(shp, dtype=sd, device=device) if layout.key_qjl else None
        self.v_planes = torch.zeros(batch, num_kv_heads, capacity // 32, layout.value_bits, d,
                                    dtype=torch.int32, device=device)
        if layout.value_kind == TQ_V_MINMAX:
            self.v_meta = torch.zeros(*shp, d // layout.value_group, 2, dtype=torch.float16, device=device)
            self.v_norm = None
        else:
            self.v_meta = None
            self.v_norm = torch.zeros(shp, dtype=sd, device=device)

    def c(self) -> _Cache:
        """The C struct; built on first use (the tensors are fixed at construction)."""
        st = self.__dict__.get("_cstruct")
        if st is None:
            st = self._cstruct = _Cache(_ptr(self.k_planes), _ptr(self.k_norm), _ptr(self.k_rnorm),
                                        _ptr(self.v_planes), _ptr(self.v_meta), _ptr(self.v_norm), self.batch,
                                        self.num_kv_heads, self.capacity)
        return st


def encode_kv(params: Params, k: torch.Tensor, v: torch.Tensor, dst_pos, cache: Cache, stream=None):
    """Encode k, v ([B, n_new, H_kv, d], fp32 or bf16, contiguous, on device)
    into cache positions dst_pos[b] ... dst_pos[b] + n_new - 1."""
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
        raise ValueError("k and v must be [B, n_new, H_kv, d] with the same dtype")
    if not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k and v must be contiguous")
    if k.shape[0] != cache.batch or k.shape[2] != cache.num_kv_heads:
        raise ValueError("k/v batch or head count does not match the cache")
    _require(k.shape[3] == params.layout.head_dim, f"k's last dimension {k.shape[3]} is not head_dim "
             f"{params.layout.head_dim}")
    _require(k.dtype in (torch.float32, torch.bfloat16), "k and v must be fp32 or bf16")
    _check_seq_list("dst_pos", dst_pos, cache.batch)
    _check_device(cache, k=k, v=v)
    pos = (ctypes.c_int64 * cache.batch)(*[int(x) for x in dst_pos])
    lay, prm, cc = params.layout.c(), params.c(), cache.c()
    _check(lib().tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), _ptr(k), _ptr(v), _dtype_code(k),
                              k.shape[1], pos, ctypes.byref(cc), _stream(stream)))


def ring_append(k_new: torch.Tensor, v_new: torch.Tensor, ring_k: torch.Tensor, ring_v: torch.Tensor,
                n_ring, stream=None):
    """Write one token per sequence (k_new, v_new: [B, 1, H_kv, d]) into the
    bf16 rings ([B, R, H_kv, d]) at positions n_ring[b]."""
    _require(ring_k.dim() == 4, "rings must be [B, R, H_kv, d]")
    b, r, h, d = ring_k.shape
    if ring_k.dtype != torch.bfloat16 or ring_v.dtype != torch.bfloat16:
        raise ValueError("rings are bf16")
    _require(ring_v.shape == ring_k.shape and ring_k.is_contiguous() and ring_v.is_contiguous(),
             "ring_k and ring_v must be contiguous and of one shape")
    if tuple(k_new.shape) != (b, 1, h, d) or not k_new.is_contiguous() or not v_new.is_contiguous():
        raise ValueError("k_new/v_new must be contiguous [B, 1, H_kv, d]")
    _require(v_new.shape == k_new.shape and v_new.dtype == k_new.dtype, "k_new and v_new must match")
    _require(k_new.dtype in (torch.float32, torch.bfloat16), "k_new must be fp32 or bf16")
    _check_seq_list("n_ring", n_ring, b)
    for name, t in (("v_new", v_new), ("ring_k", ring_k), ("ring_v", ring_v)):
        _require(t.device == k_new.device, f"{name} is not on k_new's device")
    nr = (ctypes.c_int32 * b)(*[int(x) for x in n_ring])
    _check(lib().tq_ring_append(_ptr(k_new), _ptr(v_new), _dtype_code(k_new), b, h, d,
                                _ptr(ring_k), _ptr(ring_v), r, nr, _stream(stream)))


def decode_workspace_bytes(layout: Layout, batch: int, num_q_heads: int, num_kv_heads: int, max_tokens: int,
                           num_queries: int = 1) -> int:
    lay = layout.c()
    if num_queries == 1:
        return int(lib().tq_decode_workspace_bytes(ctypes.byref(lay), batch, num_q_heads, num_kv_heads, max_tokens))
    return int(lib().tq_decode_workspace_bytes_multi(ctypes.byref(lay), batch, num_q_heads, num_kv_heads,
                                                     max_tokens, num_queries))


def decode_attn(params: Params, q: torch.Tensor, cache: Cache, n_compressed, ring_k=None, ring_v=None,
                n_ring=None, scale: float | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step: q [B, H_q, d] (fp32 or bf16) -> out [B, H_q, d] fp32; or
    several causal queries per sequence: q [B, T, H_q, d] -> out [B, T, H_q, d]
    (tq_decode_attn_multi)."""
    lay_py = params.layout
    _check_decode(lay_py, q, cache, n_compressed, out, workspace)
    ring_cap = _check_ring(cache, ring_k, ring_v, n_ring, lay_py.head_dim)
    if ring_cap == 0 and n_ring is not None:
        _check_seq_list("n_ring", n_ring, cache.batch)
        _require(all(int(x) == 0 for x in n_ring), "n_ring must be 0 without ring buffers")
    multi = q.dim() == 4
    if multi:
        b, nq, h_q, d = q.shape
    else:
        b, h_q, d = q.shape
        nq = 1
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    nc = (ctypes.c_int64 * b)(*n_compressed)
    if workspace is None:  # (a given workspace is checked against the need by the library)
        need = decode_workspace_bytes(lay_py, b, h_q, cache.num_kv_heads, max(n_compressed), nq)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nr = (ctypes.c_int32 * b)(*(n_ring if n_ring is not None else [0] * b))
    lay, prm, cc = lay_py.c(), params.c(), cache.c()
    if multi:
        _check(lib().tq_decode_attn_multi(ctypes.byref(lay), ctypes.byref(prm), _ptr(q), _dtype_code(q), h_q, nq,
                                          ctypes.byref(cc), nc, _ptr(ring_k), _ptr(ring_v), ring_cap, nr,
                                          float(scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    else:
        _check(lib().tq_decode_attn(ctypes.byref(lay), ctypes.byref(prm), _ptr(q), _dtype_code(q), h_q,
                                    ctypes.byref(cc), nc, _ptr(ring_k), _ptr(ring_v), ring_cap, nr,
                                    float(scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    return out


def decode_attn_append(params: Params, q: torch.Tensor, cache: Cache, n_compressed, k_new: torch.Tensor,
                       v_new: torch.Tensor, ring_k: torch.Tensor, ring_v: torch.Tensor, n_ring,
                       scale: float | None = None, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step with the ring append fused in (tq_decode_attn_append):
    k_new, v_new [B, 1, H_kv, d] (fp32 or bf16) go to ring positions n_ring[b],
    then q [B, H_q, d] attends over the compressed tokens and n_ring[b] + 1
    ring tokens.  n_ring holds the lengths before the append."""
    lay_py = params.layout
    _require(q.dim() == 3, "q must be [B, H_q, d] (one query per sequence)")
    _check_decode(lay_py, q, cache, n_compressed, out, workspace)
    _require(ring_k is not None and ring_v is not None, "the fused append needs the ring buffers")
    _check_ring(cache, ring_k, ring_v, n_ring, lay_py.head_dim)
    b, h_q, d = q.shape
    for t in (q, k_new, v_new, ring_k, ring_v):
        if not t.is_contiguous():
            raise ValueError("q, k_new, v_new and the ring buffers must be contiguous")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    _require(tuple(k_new.shape) == (b, 1, cache.num_kv_heads, d) and tuple(v_new.shape) == tuple(k_new.shape),
             f"k_new and v_new must be [{b}, 1, {cache.num_kv_heads}, {d}]")
    _require(k_new.dtype in (torch.float32, torch.bfloat16), "k_new and v_new must be fp32 or bf16")
    _check_device(cache, k_new=k_new, v_new=v_new, ring_k=ring_k, ring_v=ring_v)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    nc = (ctypes.c_int64 * b)(*n_compressed)
    if workspace is None:  # (a given workspace is checked against the need by the library)
        need = decode_workspace_bytes(lay_py, b, h_q, cache.num_kv_heads, max(n_compressed))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nr = (ctypes.c_int32 * b)(*n_ring)
    lay, prm, cc = lay_py.c(), params.c(), cache.c()
    _check(lib().tq_decode_attn_append(ctypes.byref(lay), ctypes.byref(prm), _ptr(q), _dtype_code(q), h_q,
                                       ctypes.byref(cc), nc, _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                       _ptr(ring_k), _ptr(ring_v), ring_k.shape[1], nr, float(scale), _ptr(out),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def time_next_launch(kernel: int, ev_begin, ev_end):
    """Record the caller's hipEvent_t handles around the next launch of
    `kernel` (TQ_KERNEL_*) on this thread."""
    _check(lib().tq_time_next_launch(kernel, ev_begin, ev_end))


def version() -> str:
    return lib().tq_version().decode()
