"""ctypes binding of libmhla (names and arguments mirror include/mhla.h).

Tensors are torch tensors already on the GPU; the binding passes their
device pointers and the current HIP stream.  Nothing here computes: when the
library is missing the calls raise instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

MHLA_PHI_RELU, MHLA_PHI_ELU1 = 0, 1
MHLA_DTYPE_F32, MHLA_DTYPE_BF16 = 0, 1
(MHLA_OK, MHLA_ERR_INVALID_ARG, MHLA_ERR_SHAPE, MHLA_ERR_UNSUPPORTED, MHLA_ERR_HIP,
 MHLA_ERR_ALIAS) = range(6)
(MHLA_PATH_AUTO, MHLA_PATH_GENERIC, MHLA_PATH_FUSED, MHLA_PATH_PAIRS, MHLA_PATH_BLOCKED,
 MHLA_PATH_COLUMNS) = range(6)
MHLA_FLAG_NO_NORM, MHLA_FLAG_CAUSAL = 1, 2
MHLA_MAX_LAUNCHES = 8

EXPORTED_SYMBOLS = (
    "mhla_forward", "mhla_forward_path", "mhla_forward_ex", "mhla_backward",
    "mhla_decode_state_bytes", "mhla_decode_step", "mhla_decode_steps", "mhla_decode_prefill",
    "mhla_validate",
    "mhla_plan",
    "mhla_plan_ex", "mhla_lb_init", "mhla_num_blocks", "mhla_workspace_bytes",
    "mhla_workspace_bytes_ex", "mhla_forward_profiled", "mhla_forward_noalloc",
    "mhla_error_string", "mhla_last_error", "mhla_release",
)
MHLA_NOALLOC_SCRATCH_BYTES = 256 << 20

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmhla.so")
_lib = None


class MhlaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("mhla error %d (%s): %s" % (code, mhla_error_string(code), message))
        self.code = code


class BlockShape(ctypes.Structure):
    """mhla_block_shape: grid (T, Hg, Wg) and block (bt, bh, bw)."""
    _fields_ = [("ndim", ctypes.c_int), ("grid", ctypes.c_int * 3), ("block", ctypes.c_int * 3)]

    @classmethod
    def make(cls, grid: Sequence[int], block: Sequence[int], ndim: Optional[int] = None):
        g = tuple(int(x) for x in grid)
        b = tuple(int(x) for x in block)
        if len(g) != len(b):
            raise ValueError("grid and block need the same number of axes")
        if ndim is None:
            ndim = len(g)
        g = (1,) * (3 - len(g)) + g
        b = (1,) * (3 - len(b)) + b
        return cls(int(ndim), (ctypes.c_int * 3)(*g), (ctypes.c_int * 3)(*b))


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmhla.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libmhla.so is not built: run `python -m token_level_head_mhla_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ip = ctypes.c_void_p, ctypes.c_int
    bsp = ctypes.POINTER(BlockShape)
    lib.mhla_forward.argtypes = [vp, vp, vp, vp, vp, ip, ip, ip, ip, bsp, ip, ip, vp]
    lib.mhla_forward.restype = ip
    lib.mhla_forward_path.argtypes = [vp, vp, vp, vp, vp, ip, ip, ip, ip, bsp, ip, ip, ip, vp]
    lib.mhla_forward_path.restype = ip
    lib.mhla_forward_ex.argtypes = [vp, vp, vp, vp, vp, ip, ip, ip, ip, bsp, ip, ip, ip, ip, vp]
    lib.mhla_forward_ex.restype = ip
    lib.mhla_forward_profiled.argtypes = [vp, vp, vp, vp, vp, ip, ip, ip, ip, bsp, ip, ip, ip, ip,
                                          ctypes.POINTER(vp), ip, ctypes.POINTER(ip),
                                          ctypes.POINTER(ctypes.c_char_p), vp]
    lib.mhla_forward_profiled.restype = ip
    lib.mhla_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, ip, ip, ip, ip, bsp, ip, ip, ip, ip,
                                         vp]
    lib.mhla_forward_noalloc.restype = ip
    lib.mhla_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, bsp, ip, ip,
                                  ip, vp]
    lib.mhla_backward.restype = ip
    lib.mhla_decode_state_bytes.argtypes = [ip, ip, ip, ip]
    lib.mhla_decode_state_bytes.restype = ctypes.c_size_t
    lib.mhla_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, ip, ip, ip, ip,
                                     vp]
    lib.mhla_decode_step.restype = ip
    lib.mhla_decode_steps.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, ip, ip, ip, ip,
                                      ip, vp]
    lib.mhla_decode_steps.restype = ip
    lib.mhla_decode_prefill.argtypes = [vp, vp, vp, vp, ip, ip, ip, ip, ip, ip, ip, ip, ip, vp]
    lib.mhla_decode_prefill.restype = ip
    lib.mhla_plan_ex.argtypes = [ip, ip, ip, ip, bsp, ip, ip, ip]
    lib.mhla_plan_ex.restype = ip
    lib.mhla_lb_init.argtypes = [bsp, ctypes.POINTER(ctypes.c_float), ctypes.c_size_t]
    lib.mhla_lb_init.restype = ip
    lib.mhla_validate.argtypes = [ip, ip, ip, ip, bsp, ip, ip]
    lib.mhla_validate.restype = ip
    lib.mhla_plan.argtypes = [ip, ip, ip, ip, bsp, ip, ip]
    lib.mhla_plan.restype = ip
    lib.mhla_num_blocks.argtypes = [ip, bsp]
    lib.mhla_num_blocks.restype = ip
    lib.mhla_workspace_bytes.argtypes = [ip, ip, ip, ip, bsp, ip]
    lib.mhla_workspace_bytes.restype = ctypes.c_size_t
    lib.mhla_workspace_bytes_ex.argtypes = [ip, ip, ip, ip, bsp, ip, ip, ip]
    lib.mhla_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.mhla_error_string.argtypes = [ip]
    lib.mhla_error_string.restype = ctypes.c_char_p
    lib.mhla_last_error.argtypes = []
    lib.mhla_last_error.restype = ctypes.c_char_p
    lib.mhla_release.argtypes = []
    lib.mhla_release.restype = None
    _lib = lib
    return lib


def mhla_error_string(code: int) -> str:
    return load_library().mhla_error_string(int(code)).decode()


def mhla_last_error() -> str:
    return load_library().mhla_last_error().decode()


def _shape(block_shape) -> BlockShape:
    if isinstance(block_shape, BlockShape):
        return block_shape
    grid, block = block_shape
    return BlockShape.make(grid, block)


def mhla_validate(B, H, N, d, block_shape, phi_kind, dtype) -> int:
    return int(load_library().mhla_validate(B, H, N, d, ctypes.byref(_shape(block_shape)),
                                            phi_kind, dtype))


def mhla_plan(B, H, N, d, block_shape, phi_kind, dtype) -> int:
    return int(load_library().mhla_plan(B, H, N, d, ctypes.byref(_shape(block_shape)), phi_kind,
                                        dtype))


def mhla_plan_ex(B, H, N, d, block_shape, phi_kind, dtype, flags) -> int:
    return int(load_library().mhla_plan_ex(B, H, N, d, ctypes.byref(_shape(block_shape)),
                                           phi_kind, dtype, flags))


def mhla_lb_init(block_shape):
    """The locality-biased initial mixing matrix [M, M] as a float32 numpy array
    (host-only call; replicate it per head for Wmix)."""
    import numpy as np
    bs = _shape(block_shape)
    M = mhla_num_blocks(int(np.prod(list(bs.grid))), bs)
    if M < 0:
        raise MhlaError(-M, mhla_last_error())
    out = np.empty((M, M), dtype=np.float32)
    rc = load_library().mhla_lb_init(ctypes.byref(bs),
                                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), M * M)
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return out


def mhla_num_blocks(N, block_shape) -> int:
    return int(load_library().mhla_num_blocks(N, ctypes.byref(_shape(block_shape))))


def mhla_workspace_bytes(B, H, N, d, block_shape, dtype) -> int:
    return int(load_library().mhla_workspace_bytes(B, H, N, d, ctypes.byref(_shape(block_shape)),
                                                   dtype))


def mhla_workspace_bytes_ex(B, H, N, d, block_shape, dtype, flags=0, path=MHLA_PATH_AUTO) -> int:
    return int(load_library().mhla_workspace_bytes_ex(
        B, H, N, d, ctypes.byref(_shape(block_shape)), dtype, int(flags), int(path)))


def mhla_release() -> None:
    load_library().mhla_release()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MHLA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MHLA_DTYPE_BF16
    raise TypeError("Q/K/V must be float32 or bfloat16, got %s" % t.dtype)


def _check_tensors(Q, K, V, W, out, block_shape):
    """Types, devices, shapes and dtypes; Wmix must hold exactly H*M*M floats,
    since the library reads (and the backward writes) that many and cannot see
    a buffer's size.  Returns the block shape structure."""
    import torch
    for name, t in (("Q", Q), ("K", K), ("V", V), ("Wmix", W), ("out", out)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape or out.shape != Q.shape:
        raise ValueError("Q, K, V, out must share one [B,H,N,d] shape")
    if K.dtype != Q.dtype or V.dtype != Q.dtype or out.dtype != Q.dtype:
        raise ValueError("Q, K, V, out must share one dtype")
    if W.dtype != torch.float32:
        raise ValueError("Wmix must be float32")
    bs = _shape(block_shape)
    B, H, N, d = Q.shape
    M = mhla_num_blocks(N, bs)
    if M < 0:
        raise MhlaError(-M, mhla_last_error())
    if W.numel() != H * M * M:
        raise ValueError("Wmix has %d elements; H*M*M = %d*%d*%d = %d are needed"
                         % (W.numel(), H, M, M, H * M * M))
    return bs


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def mhla_forward_path(Q, K, V, Wmix, out, block_shape, phi_kind, path, stream=None):
    """Enqueue the forward on `stream` (default: torch's current stream)."""
    bs = _check_tensors(Q, K, V, Wmix, out, block_shape)
    B, H, N, d = Q.shape
    rc = load_library().mhla_forward_path(
        Q.data_ptr(), K.data_ptr(), V.data_ptr(), Wmix.data_ptr(), out.data_ptr(), B, H, N, d,
        ctypes.byref(bs), int(phi_kind), _dtype_code(Q), int(path), _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return out


def mhla_forward_ex(Q, K, V, Wmix, out, block_shape, phi_kind, flags=0, path=MHLA_PATH_AUTO,
                    stream=None):
    """Enqueue the forward with option bits (MHLA_FLAG_NO_NORM, MHLA_FLAG_CAUSAL)."""
    bs = _check_tensors(Q, K, V, Wmix, out, block_shape)
    B, H, N, d = Q.shape
    rc = load_library().mhla_forward_ex(
        Q.data_ptr(), K.data_ptr(), V.data_ptr(), Wmix.data_ptr(), out.data_ptr(), B, H, N, d,
        ctypes.byref(bs), int(phi_kind), _dtype_code(Q), int(flags), int(path),
        _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return out


def mhla_forward_noalloc(Q, K, V, Wmix, out, block_shape, phi_kind, flags=0,
                         path=MHLA_PATH_AUTO, stream=None):
    """mhla_forward_ex on the library's fixed scratch (no device allocation;
    calls that overlap on one device race)."""
    bs = _check_tensors(Q, K, V, Wmix, out, block_shape)
    B, H, N, d = Q.shape
    rc = load_library().mhla_forward_noalloc(
        Q.data_ptr(), K.data_ptr(), V.data_ptr(), Wmix.data_ptr(), out.data_ptr(), B, H, N, d,
        ctypes.byref(bs), int(phi_kind), _dtype_code(Q), int(flags), int(path),
        _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return out


def mhla_backward(Q, K, V, Wmix, dY, dQ, dK, dV, dWmix, block_shape, phi_kind, flags=0,
                  stream=None):
    """Enqueue the backward pass: writes dQ, dK, dV (like Q) and dWmix (like Wmix)."""
    bs = _check_tensors(Q, K, V, Wmix, dY, block_shape)
    _check_tensors(dQ, dK, dV, dWmix, dY, block_shape)
    B, H, N, d = Q.shape
    rc = load_library().mhla_backward(
        Q.data_ptr(), K.data_ptr(), V.data_ptr(), Wmix.data_ptr(), dY.data_ptr(), dQ.data_ptr(),
        dK.data_ptr(), dV.data_ptr(), dWmix.data_ptr(), B, H, N, d, ctypes.byref(bs),
        int(phi_kind), _dtype_code(Q), int(flags), _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return dQ, dK, dV, dWmix


def mhla_decode_state_bytes(B, H, d, M) -> int:
    return int(load_library().mhla_decode_state_bytes(B, H, d, M))


def mhla_decode_step(q, k, v, Wmix, y, state, M, nb, t, phi_kind, flags=0, stream=None):
    """One streaming step: q, k, v, y are [B, H, d] GPU tensors (the token at
    position t of every slice); state is a GPU buffer of
    mhla_decode_state_bytes(B, H, d, M) bytes."""
    import torch
    for name, t_ in (("q", q), ("k", k), ("v", v), ("Wmix", Wmix), ("y", y)):
        if not (isinstance(t_, torch.Tensor) and t_.is_cuda and t_.is_contiguous()):
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape or y.shape != q.shape:
        raise ValueError("q, k, v, y must share one [B, H, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype or y.dtype != q.dtype:
        raise ValueError("q, k, v, y must share one dtype")
    if Wmix.dtype != torch.float32:
        raise ValueError("Wmix must be float32")
    if not (isinstance(state, torch.Tensor) and state.is_cuda and state.is_contiguous()):
        raise ValueError("state must be a contiguous GPU tensor")
    B, H, d = q.shape
    if Wmix.numel() != H * int(M) * int(M):
        raise ValueError("Wmix has %d elements; H*M*M = %d are needed"
                         % (Wmix.numel(), H * int(M) * int(M)))
    if state.numel() * state.element_size() < mhla_decode_state_bytes(B, H, d, M):
        raise ValueError("state is smaller than mhla_decode_state_bytes")
    rc = load_library().mhla_decode_step(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), Wmix.data_ptr(), y.data_ptr(), state.data_ptr(),
        B, H, d, int(M), int(nb), int(t), int(phi_kind), _dtype_code(q), int(flags),
        _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return y


def mhla_decode_steps(q, k, v, Wmix, y, state, M, nb, t0, phi_kind, flags=0, stream=None):
    """n streaming steps in one call: q, k, v, y are [B, H, n, d] GPU tensors
    (tokens t0 .. t0+n-1 of every slice); state is a GPU buffer of
    mhla_decode_state_bytes(B, H, d, M) bytes.  Same results as n calls of
    mhla_decode_step."""
    import torch
    for name, t_ in (("q", q), ("k", k), ("v", v), ("Wmix", Wmix), ("y", y)):
        if not (isinstance(t_, torch.Tensor) and t_.is_cuda and t_.is_contiguous()):
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or y.shape != q.shape:
        raise ValueError("q, k, v, y must share one [B, H, n, d] shape")
    if k.dtype != q.dtype or v.dtype != q.dtype or y.dtype != q.dtype:
        raise ValueError("q, k, v, y must share one dtype")
    if Wmix.dtype != torch.float32:
        raise ValueError("Wmix must be float32")
    if not (isinstance(state, torch.Tensor) and state.is_cuda and state.is_contiguous()):
        raise ValueError("state must be a contiguous GPU tensor")
    B, H, n, d = q.shape
    if Wmix.numel() != H * int(M) * int(M):
        raise ValueError("Wmix has %d elements; H*M*M = %d are needed"
                         % (Wmix.numel(), H * int(M) * int(M)))
    if state.numel() * state.element_size() < mhla_decode_state_bytes(B, H, d, M):
        raise ValueError("state is smaller than mhla_decode_state_bytes")
    rc = load_library().mhla_decode_steps(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), Wmix.data_ptr(), y.data_ptr(), state.data_ptr(),
        B, H, d, int(M), int(nb), int(t0), n, int(phi_kind), _dtype_code(q), int(flags),
        _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return y


def mhla_decode_prefill(k, v, Wmix, state, M, nb, phi_kind, flags=0, stream=None):
    """Decode state from a prompt: k, v are [B, H, T, d] GPU tensors (its first
    T tokens); state is a GPU buffer of mhla_decode_state_bytes(B, H, d, M)
    bytes.  mhla_decode_step continues at t = T."""
    import torch
    for name, t_ in (("k", k), ("v", v), ("Wmix", Wmix), ("state", state)):
        if not (isinstance(t_, torch.Tensor) and t_.is_cuda and t_.is_contiguous()):
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if k.dim() != 4 or v.shape != k.shape:
        raise ValueError("k, v must share one [B, H, T, d] shape")
    if v.dtype != k.dtype:
        raise ValueError("k, v must share one dtype")
    if Wmix.dtype != torch.float32:
        raise ValueError("Wmix must be float32")
    B, H, T, d = k.shape
    if Wmix.numel() != H * int(M) * int(M):
        raise ValueError("Wmix has %d elements; H*M*M = %d are needed"
                         % (Wmix.numel(), H * int(M) * int(M)))
    if state.numel() * state.element_size() < mhla_decode_state_bytes(B, H, d, M):
        raise ValueError("state is smaller than mhla_decode_state_bytes")
    rc = load_library().mhla_decode_prefill(
        k.data_ptr(), v.data_ptr(), Wmix.data_ptr(), state.data_ptr(), B, H, d, int(M), int(nb),
        T, int(phi_kind), _dtype_code(k), int(flags), _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return state


def mhla_forward(Q, K, V, Wmix, out, block_shape, phi_kind, stream=None):
    """Enqueue the forward with the library's path choice."""
    bs = _check_tensors(Q, K, V, Wmix, out, block_shape)
    B, H, N, d = Q.shape
    rc = load_library().mhla_forward(
        Q.data_ptr(), K.data_ptr(), V.data_ptr(), Wmix.data_ptr(), out.data_ptr(), B, H, N, d,
        ctypes.byref(bs), int(phi_kind), _dtype_code(Q), _stream_ptr(stream))
    if rc != MHLA_OK:
        raise MhlaError(rc, mhla_last_error())
    return out


class PreparedForward:
    """A forward call with its arguments marshalled once, for timing loops.
    call() enqueues mhla_forward_ex; profiled(events) enqueues
    mhla_forward_profiled with `events` (at least MHLA_MAX_LAUNCHES + 1
    hipEvent_t handles as ints) and returns the names of the launched
    kernels."""

    def __init__(self, Q, K, V, Wmix, out, block_shape, phi_kind, flags=0, path=MHLA_PATH_AUTO,
                 stream=None):
        bs = _check_tensors(Q, K, V, Wmix, out, block_shape)
        B, H, N, d = Q.shape
        self._bs = bs
        self._args = (Q.data_ptr(), K.data_ptr(), V.data_ptr(), Wmix.data_ptr(), out.data_ptr(),
                      B, H, N, d, ctypes.byref(bs), int(phi_kind), _dtype_code(Q), int(flags),
                      int(path))
        self._stream = _stream_ptr(stream)
        self._names = (ctypes.c_char_p * MHLA_MAX_LAUNCHES)()
        self._n = ctypes.c_int(0)
        lib = load_library()
        self._fwd, self._prof = lib.mhla_forward_ex, lib.mhla_forward_profiled
        self._keep = (Q, K, V, Wmix, out)

    def call(self):
        rc = self._fwd(*self._args, self._stream)
        if rc != MHLA_OK:
            raise MhlaError(rc, mhla_last_error())

    def profiled(self, events):
        ev = (ctypes.c_void_p * len(events))(*events)
        rc = self._prof(*self._args, ev, len(events), ctypes.byref(self._n), self._names,
                        self._stream)
        if rc != MHLA_OK:
            raise MhlaError(rc, mhla_last_error())
        return [self._names[i].decode() for i in range(min(self._n.value, MHLA_MAX_LAUNCHES))]


def mhla_forward_profiled(Q, K, V, Wmix, out, block_shape, phi_kind, flags, path, events,
                          stream=None):
    """mhla_forward_ex recording events[0] before and events[k] after launch k;
    returns the launched kernels' names."""
    return PreparedForward(Q, K, V, Wmix, out, block_shape, phi_kind, flags, path,
                           stream).profiled(events)
