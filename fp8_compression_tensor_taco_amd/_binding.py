"""ctypes binding over libtaco's C ABI (include/taco.h).

Argument marshalling only: every step of compress / decompress / decompress-sum
runs in the HIP kernels of libtaco.so.  torch provides device memory and the
current stream.  There is no CPU fallback: without the built library, or with
tensors that are not on a GPU, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

from .build import LIB_PATH

TACO_MAX_PARTS = 8
TACO_AMAX_SLOTS = 64
TACO_AMAX_FLOATS = 4096
_STATUS = {
    0: "TACO_OK", 1: "TACO_ERR_NULL", 2: "TACO_ERR_ALIGN", 3: "TACO_ERR_SHAPE",
    4: "TACO_ERR_UNSUPPORTED_BLOCK", 5: "TACO_ERR_BAD_ENERGY", 6: "TACO_ERR_WORKSPACE",
    7: "TACO_ERR_BAD_NPARTS", 8: "TACO_ERR_HIP", 9: "TACO_ERR_FLAGS", 10: "TACO_ERR_ALIAS",
}
TACO_FLAG_TWO_PASS = 1
TACO_DEFAULT_BARRIER_POLLS = 1 << 16


class TacoError(RuntimeError):
    """A libtaco call returned a nonzero status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.name = _STATUS.get(status, "TACO_ERR_UNKNOWN")


_lib = None
_lock = threading.Lock()
_workspaces: dict[tuple[int, str, int], torch.Tensor] = {}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32


def library_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load libtaco.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libtaco.so not found at {LIB_PATH}; build it first with "
                "`python -m fp8_compression_tensor_taco_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.taco_status_string.restype = ctypes.c_char_p
        lib.taco_status_string.argtypes = [ctypes.c_int]
        lib.taco_version.restype = ctypes.c_char_p
        lib.taco_version.argtypes = []
        lib.taco_compress_is_single_pass.restype = ctypes.c_int
        lib.taco_compress_is_single_pass.argtypes = [_i64, _i64, _i32]
        lib.taco_workspace_timed_out.restype = ctypes.c_int
        lib.taco_workspace_timed_out.argtypes = [_vp, _vp, ctypes.POINTER(ctypes.c_int)]
        lib.taco_num_scales.restype = _i64
        lib.taco_num_scales.argtypes = [_i64, _i64, _i32]
        lib.taco_compress_workspace_bytes.restype = ctypes.c_size_t
        lib.taco_compress_workspace_bytes.argtypes = [_i64, _i64, _i32]
        lib.taco_compress.restype = ctypes.c_int
        lib.taco_compress.argtypes = [_vp, _i64, _i64, _i32, ctypes.c_float, _vp, _vp, _vp,
                                      _vp, ctypes.c_size_t, _vp]
        lib.taco_compress_ex.restype = ctypes.c_int
        lib.taco_compress_ex.argtypes = [_vp, _i64, _i64, _i32, ctypes.c_float, _vp, _vp, _vp,
                                         _vp, ctypes.c_size_t, _u32, _u32, _vp]
        lib.taco_compress_noalloc.restype = ctypes.c_int
        lib.taco_compress_noalloc.argtypes = [_vp, _i64, _i64, _i32, ctypes.c_float, _vp, _vp, _vp,
                                              _u32, _u32, _vp]
        lib.taco_decompress.restype = ctypes.c_int
        lib.taco_decompress.argtypes = [_vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
        lib.taco_decompress_sum_compress_workspace_bytes.restype = ctypes.c_size_t
        lib.taco_decompress_sum_compress_workspace_bytes.argtypes = [_i64, _i64, _i32]
        lib.taco_decompress_sum_compress.restype = ctypes.c_int
        lib.taco_decompress_sum_compress.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                     ctypes.POINTER(_vp), _i32, _i64, _i64, _i32,
                                                     ctypes.c_float, _vp, _vp, _vp, _vp,
                                                     ctypes.c_size_t, _vp]
        lib.taco_decompress_sum_compress_ex.restype = ctypes.c_int
        lib.taco_decompress_sum_compress_ex.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                        ctypes.POINTER(_vp), _i32, _i64, _i64, _i32,
                                                        ctypes.c_float, _vp, _vp, _vp, _vp,
                                                        ctypes.c_size_t, _u32, _u32, _vp]
        lib.taco_compress_blockscale.restype = ctypes.c_int
        lib.taco_compress_blockscale.argtypes = [_vp, _i64, _i64, _i32, ctypes.c_float, _vp, _vp, _vp, _vp]
        lib.taco_decompress_blockscale.restype = ctypes.c_int
        lib.taco_decompress_blockscale.argtypes = [_vp, _vp, _vp, _i64, _i64, _i32, _vp, _vp]
        lib.taco_compress_delayed.restype = ctypes.c_int
        lib.taco_compress_delayed.argtypes = [_vp, _i64, _i64, _i32, ctypes.c_float, _vp, _vp, _vp, _vp,
                                              _vp, _vp]
        lib.taco_compress_int8_workspace_bytes.restype = ctypes.c_size_t
        lib.taco_compress_int8_workspace_bytes.argtypes = [_i64, _i64, _i32]
        lib.taco_compress_int8.restype = ctypes.c_int
        lib.taco_compress_int8.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        lib.taco_decompress_int8.restype = ctypes.c_int
        lib.taco_decompress_int8.argtypes = [_vp, _vp, _i64, _i64, _i32, _vp, _vp]
        lib.taco_decompress_sum.restype = ctypes.c_int
        lib.taco_decompress_sum.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                            ctypes.POINTER(_vp), _i32, _i64, _i64, _i32, _vp, _vp]
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().taco_status_string(status).decode()
        raise TacoError(status, msg)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on(stream):
    """Allocations (outputs and .contiguous() copies) on the stream the call
    runs on, so that torch's caching allocator does not hand their memory to
    another stream while the call's kernels still use it."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _require_buffer(t: torch.Tensor, name: str, dtype, numel: int, shape=None) -> None:
    """Output / input buffers must be contiguous, of the right dtype and size:
    the kernels index them by the shape alone."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {t.numel()}")


def _require_gpu(*tensors: torch.Tensor) -> torch.device:
    dev = tensors[0].device
    for t in tensors:
        if t.device.type != "cuda":
            raise ValueError("libtaco works on GPU tensors only (no CPU fallback)")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def version() -> str:
    return load().taco_version().decode()


def is_single_pass(tokens: int, hidden: int, block: int) -> bool:
    """Whether compress of this shape runs as the single fused kernel here."""
    r = int(load().taco_compress_is_single_pass(tokens, hidden, block))
    if r < 0:
        raise ValueError("invalid shape or no usable GPU")
    return bool(r)


def _pass_args(single_pass: bool, barrier_polls: int):
    if not 0 <= int(barrier_polls) < 2 ** 32:
        raise ValueError("barrier_polls must fit in 32 bits")
    return (0 if single_pass else TACO_FLAG_TWO_PASS), int(barrier_polls)


def _timed_out_and_clear(lib, workspace: torch.Tensor, handle: int) -> bool:
    flag = ctypes.c_int(0)
    _check(lib.taco_workspace_timed_out(_ptr(workspace), handle, ctypes.byref(flag)))
    if flag.value:
        workspace.zero_()
    return bool(flag.value)


def workspace_timed_out(workspace: torch.Tensor | None = None, stream=None) -> bool:
    """Whether a single-pass call on `workspace` has given up at its grid
    barrier since the workspace was zero-filled (waits for the stream).  With
    no argument, checks every workspace the binding has allocated, each after
    waiting for the stream it serves."""
    lib = load()
    if workspace is not None:
        checks = [(workspace, _stream(_require_gpu(workspace), stream))]
    else:
        checks = [(ws, key[2]) for key, ws in _workspaces.items()]   # each on its own stream
    for ws, handle in checks:
        flag = ctypes.c_int(0)
        _check(lib.taco_workspace_timed_out(_ptr(ws), handle, ctypes.byref(flag)))
        if flag.value:
            return True
    return False


def num_scales(tokens: int, hidden: int, block: int) -> int:
    return int(load().taco_num_scales(tokens, hidden, block))


def workspace_bytes(tokens: int, hidden: int, block: int) -> int:
    return int(load().taco_compress_workspace_bytes(tokens, hidden, block))


def _workspace(device: torch.device, nbytes: int, kind: str, stream_handle: int) -> torch.Tensor:
    """A zero-filled workspace per device, kind and stream, grown when too
    small (a new one starts zeroed, as the library requires).  Calls on one
    stream are ordered, so they may share it; calls on different streams get
    different workspaces, since concurrent calls on one workspace race."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    key = (idx, kind, int(stream_handle or 0))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        current = torch.cuda.current_stream(device)
        if int(current.cuda_stream) != key[2]:
            current.synchronize()       # the zero-fill ran on another stream than the call's
        _workspaces[key] = ws
    return ws


def compress(x: torch.Tensor, block: int, target_energy: float = 1.0, *,
             q: torch.Tensor | None = None, alpha: torch.Tensor | None = None,
             scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
             stream=None, single_pass: bool = True, barrier_polls: int = 0,
             check_barrier: bool = False):
    """Compress a bf16 [tokens, hidden] GPU tensor.

    Returns (q uint8 [tokens, hidden], alpha float32 [tokens, hidden/block],
    scale float32 [1]).  Output tensors may be passed in to avoid allocation.
    single_pass=False takes the two kernels that need no co-residency (for
    callers whose compute units are shared with other kernels; the same
    result bitwise).  barrier_polls bounds the single-pass barrier's wait (0:
    the library's default).  check_barrier=True waits for the call and, if a
    workgroup gave up at the barrier, clears the workspace's flag and
    compresses again with the two kernels (the fallback include/taco.h
    documents); it synchronises the stream.
    """
    with _on(stream):
        return _compress(x, block, target_energy, q, alpha, scale, workspace, stream, single_pass,
                         barrier_polls, check_barrier)


def _compress(x, block, target_energy, q, alpha, scale, workspace, stream, single_pass, barrier_polls,
              check_barrier):
    lib = load()
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    dev = _require_gpu(x)
    flags, polls = _pass_args(single_pass, barrier_polls)
    x = x.contiguous()
    T, H = x.shape
    n = lib.taco_num_scales(T, H, block)
    if n < 0:
        _check(4 if block not in (64, 128, 256) else 3)
    if q is None:
        q = torch.empty((T, H), dtype=torch.uint8, device=dev)
    if alpha is None:
        alpha = torch.empty((T, H // block), dtype=torch.float32, device=dev)
    if scale is None:
        scale = torch.empty((1,), dtype=torch.float32, device=dev)
    need = lib.taco_compress_workspace_bytes(T, H, block)
    if workspace is None:
        workspace = _workspace(dev, need, "compress", _stream(dev, stream))
    _require_gpu(x, q, alpha, scale, workspace)
    _require_buffer(q, "q", torch.uint8, T * H, (T, H))
    _require_buffer(alpha, "alpha", torch.float32, n)
    _require_buffer(scale, "scale", torch.float32, 1)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    args = (_ptr(x), T, H, block, float(target_energy), _ptr(q), _ptr(alpha), _ptr(scale), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    handle = _stream(dev, stream)
    _check(lib.taco_compress_ex(*args, flags, polls, handle))
    if check_barrier and flags == 0 and _timed_out_and_clear(lib, workspace, handle):
        _check(lib.taco_compress_ex(*args, TACO_FLAG_TWO_PASS, polls, handle))
    return q, alpha, scale


def compress_noalloc(x: torch.Tensor, block: int, target_energy: float = 1.0, *, q: torch.Tensor,
                     alpha: torch.Tensor, scale: torch.Tensor, stream=None, single_pass: bool = True,
                     barrier_polls: int = 0):
    """compress() with the workspace in the library's own device scratch
    (taco_compress_noalloc): neither the library nor this function allocates,
    so the outputs must be passed in.  Calls on one GPU share the scratch and
    must be ordered."""
    lib = load()
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 tensor")
    dev = _require_gpu(x, q, alpha, scale)
    T, H = x.shape
    n = lib.taco_num_scales(T, H, block)
    if n < 0:
        _check(4 if block not in (64, 128, 256) else 3)
    _require_buffer(q, "q", torch.uint8, T * H, (T, H))
    _require_buffer(alpha, "alpha", torch.float32, n)
    _require_buffer(scale, "scale", torch.float32, 1)
    flags, polls = _pass_args(single_pass, barrier_polls)
    _check(lib.taco_compress_noalloc(_ptr(x), T, H, block, float(target_energy), _ptr(q), _ptr(alpha),
                                     _ptr(scale), flags, polls, _stream(dev, stream)))
    return q, alpha, scale


def decompress(q: torch.Tensor, alpha: torch.Tensor, scale: torch.Tensor, block: int, *,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decompress (q, alpha, scale) into a bf16 [tokens, hidden] GPU tensor."""
    with _on(stream):
        return _decompress(q, alpha, scale, block, out, stream)


def _decompress(q, alpha, scale, block, out, stream):
    lib = load()
    if q.dim() != 2 or q.dtype != torch.uint8:
        raise ValueError("q must be a 2-D uint8 tensor")
    if alpha.dtype != torch.float32 or scale.dtype != torch.float32:
        raise ValueError("alpha and scale must be float32")
    dev = _require_gpu(q, alpha, scale)
    T, H = q.shape
    if alpha.numel() != max(lib.taco_num_scales(T, H, block), 0):
        raise ValueError("alpha has the wrong number of elements for this shape and block")
    if scale.numel() < 1:
        raise ValueError("scale must hold one float32")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _require_gpu(q, out)
    _require_buffer(out, "out", torch.bfloat16, T * H, (T, H))
    _check(lib.taco_decompress(_ptr(q.contiguous()), _ptr(alpha.contiguous()), _ptr(scale), T, H,
                               block, _ptr(out), _stream(dev, stream)))
    return out


def _check_parts(lib, parts):
    parts = [(q.contiguous(), a.contiguous(), s) for q, a, s in parts]
    if not 1 <= len(parts) <= TACO_MAX_PARTS:
        _check(7)
    dev = _require_gpu(*[t for p in parts for t in p])
    return parts, dev


def decompress_sum_compress(parts, block: int, target_energy: float = 1.0, *,
                            q: torch.Tensor | None = None, alpha: torch.Tensor | None = None,
                            scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            stream=None, single_pass: bool = True, barrier_polls: int = 0,
                            check_barrier: bool = False):
    """compress(decompress_sum(parts)) in one call: returns (q, alpha, scale) of
    the bf16 sum of the parts' reconstructions.  single_pass, barrier_polls
    and check_barrier as in compress()."""
    with _on(stream):
        return _decompress_sum_compress(parts, block, target_energy, q, alpha, scale, workspace, stream,
                                        single_pass, barrier_polls, check_barrier)


def _decompress_sum_compress(parts, block, target_energy, q, alpha, scale, workspace, stream, single_pass,
                             barrier_polls, check_barrier):
    lib = load()
    flags, polls = _pass_args(single_pass, barrier_polls)
    parts, dev = _check_parts(lib, parts)
    T, H = parts[0][0].shape
    for pq, pa, ps in parts:
        if pq.shape != (T, H) or pq.dtype != torch.uint8:
            raise ValueError("every part's q must be uint8 with the same shape")
        if pa.dtype != torch.float32 or ps.dtype != torch.float32:
            raise ValueError("alpha and scale must be float32")
        if pa.numel() != max(lib.taco_num_scales(T, H, block), 0):
            raise ValueError("alpha has the wrong number of elements for this shape and block")
        if ps.numel() < 1:
            raise ValueError("scale must hold one float32")
    n = lib.taco_num_scales(T, H, block)
    if n < 0:
        _check(4 if block not in (64, 128, 256) else 3)
    if q is None:
        q = torch.empty((T, H), dtype=torch.uint8, device=dev)
    if alpha is None:
        alpha = torch.empty((T, H // block), dtype=torch.float32, device=dev)
    if scale is None:
        scale = torch.empty((1,), dtype=torch.float32, device=dev)
    need = lib.taco_decompress_sum_compress_workspace_bytes(T, H, block)
    if workspace is None:
        workspace = _workspace(dev, need, "decompress_sum_compress", _stream(dev, stream))
    _require_gpu(parts[0][0], q, alpha, scale, workspace)
    _require_buffer(q, "q", torch.uint8, T * H, (T, H))
    _require_buffer(alpha, "alpha", torch.float32, n)
    _require_buffer(scale, "scale", torch.float32, 1)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    P = len(parts)
    qa = (_vp * P)(*[p[0].data_ptr() for p in parts])
    aa = (_vp * P)(*[p[1].data_ptr() for p in parts])
    sa = (_vp * P)(*[p[2].data_ptr() for p in parts])
    args = (qa, aa, sa, P, T, H, block, float(target_energy), _ptr(q), _ptr(alpha), _ptr(scale),
            _ptr(workspace), workspace.numel() * workspace.element_size())
    handle = _stream(dev, stream)
    _check(lib.taco_decompress_sum_compress_ex(*args, flags, polls, handle))
    if check_barrier and flags == 0 and _timed_out_and_clear(lib, workspace, handle):
        _check(lib.taco_decompress_sum_compress_ex(*args, TACO_FLAG_TWO_PASS, polls, handle))
    return q, alpha, scale


def decompress_sum(parts, block: int, *, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """Sum of the decompressions of ``parts`` (a list of (q, alpha, scale)), rounded once to bf16."""
    with _on(stream):
        return _decompress_sum(parts, block, out, stream)


def _decompress_sum(parts, block, out, stream):
    lib = load()
    parts = [(q.contiguous(), a.contiguous(), s) for q, a, s in parts]
    if not 1 <= len(parts) <= TACO_MAX_PARTS:
        _check(7)
    dev = _require_gpu(*[t for p in parts for t in p])
    T, H = parts[0][0].shape
    for q, a, s in parts:
        if q.shape != (T, H) or q.dtype != torch.uint8:
            raise ValueError("every part's q must be uint8 with the same shape")
        if a.dtype != torch.float32 or s.dtype != torch.float32:
            raise ValueError("alpha and scale must be float32")
        if a.numel() != max(lib.taco_num_scales(T, H, block), 0):
            raise ValueError("alpha has the wrong number of elements for this shape and block")
        if s.numel() < 1:
            raise ValueError("scale must hold one float32")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _require_gpu(parts[0][0], out)
    _require_buffer(out, "out", torch.bfloat16, T * H, (T, H))
    P = len(parts)
    qa = (_vp * P)(*[q.data_ptr() for q, _, _ in parts])
    aa = (_vp * P)(*[a.data_ptr() for _, a, _ in parts])
    sa = (_vp * P)(*[s.data_ptr() for _, _, s in parts])
    _check(lib.taco_decompress_sum(qa, aa, sa, P, T, H, block, _ptr(out), _stream(dev, stream)))
    return out


def _compress_outputs(x, block, q, alpha, scale, per_block_scale):
    lib = load()
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    dev = _require_gpu(x)
    T, H = x.shape
    n = lib.taco_num_scales(T, H, block)
    if n < 0:
        _check(4 if block not in (64, 128, 256) else 3)
    if q is None:
        q = torch.empty((T, H), dtype=torch.uint8, device=dev)
    if alpha is None:
        alpha = torch.empty((T, H // block), dtype=torch.float32, device=dev)
    if scale is None:
        scale = torch.empty((T, H // block) if per_block_scale else (1,), dtype=torch.float32, device=dev)
    _require_gpu(x, q, alpha, scale)
    _require_buffer(q, "q", torch.uint8, T * H, (T, H))
    _require_buffer(alpha, "alpha", torch.float32, n)
    _require_buffer(scale, "scale", torch.float32, n if per_block_scale else 1)
    return lib, dev, T, H, q, alpha, scale


def compress_blockscale(x: torch.Tensor, block: int, target_energy: float = 1.0, *,
                        q: torch.Tensor | None = None, alpha: torch.Tensor | None = None,
                        scale: torch.Tensor | None = None, stream=None):
    """Dual-Scale variant with a per-block overflow guard: returns (q, alpha,
    scale [tokens, hidden/block]); one streaming kernel."""
    with _on(stream):
        x = x.contiguous()
        lib, dev, T, H, q, alpha, scale = _compress_outputs(x, block, q, alpha, scale, True)
        _check(lib.taco_compress_blockscale(_ptr(x), T, H, block, float(target_energy), _ptr(q), _ptr(alpha),
                                            _ptr(scale), _stream(dev, stream)))
        return q, alpha, scale


def decompress_blockscale(q: torch.Tensor, alpha: torch.Tensor, scale: torch.Tensor, block: int, *,
                          out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Inverse of compress_blockscale (one post-rotation scale per block)."""
    with _on(stream):
        return _decompress_blockscale(q, alpha, scale, block, out, stream)


def _decompress_blockscale(q, alpha, scale, block, out, stream):
    lib = load()
    if q.dim() != 2 or q.dtype != torch.uint8:
        raise ValueError("q must be a 2-D uint8 tensor")
    if alpha.dtype != torch.float32 or scale.dtype != torch.float32:
        raise ValueError("alpha and scale must be float32")
    dev = _require_gpu(q, alpha, scale)
    T, H = q.shape
    n = max(lib.taco_num_scales(T, H, block), 0)
    if alpha.numel() != n or scale.numel() != n:
        raise ValueError("alpha and scale need one element per block")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _require_gpu(q, out)
    _require_buffer(out, "out", torch.bfloat16, T * H, (T, H))
    _check(lib.taco_decompress_blockscale(_ptr(q.contiguous()), _ptr(alpha.contiguous()),
                                          _ptr(scale.contiguous()), T, H, block, _ptr(out),
                                          _stream(dev, stream)))
    return out


def _int8_scales(T: int, H: int, block: int) -> int:
    if block == 0:
        return 1
    if block not in (64, 128, 256) or H % block:
        _check(4 if block not in (64, 128, 256) else 3)
    return T * (H // block)


def compress_int8(x: torch.Tensor, block: int = 0, *, q: torch.Tensor | None = None,
                  scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  stream=None):
    """INT8 degrade path: symmetric absmax INT8 of a bf16 [tokens, hidden] GPU
    tensor, one scale per tensor (block 0) or per block of `block` elements.
    Returns (q int8 [tokens, hidden], scale float32 [1] or [tokens, hidden/block])."""
    with _on(stream):
        return _compress_int8(x, block, q, scale, workspace, stream)


def _compress_int8(x, block, q, scale, workspace, stream):
    lib = load()
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    dev = _require_gpu(x)
    x = x.contiguous()
    T, H = x.shape
    n = _int8_scales(T, H, block)
    if q is None:
        q = torch.empty((T, H), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty((1,) if block == 0 else (T, H // block), dtype=torch.float32, device=dev)
    _require_gpu(x, q, scale)
    _require_buffer(q, "q", torch.int8, T * H, (T, H))
    _require_buffer(scale, "scale", torch.float32, n)
    nbytes = 0
    if block == 0:
        need = lib.taco_compress_int8_workspace_bytes(T, H, 0)
        if workspace is None:
            workspace = _workspace(dev, need, "compress", _stream(dev, stream))
        _require_gpu(workspace)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        nbytes = workspace.numel() * workspace.element_size()
    _check(lib.taco_compress_int8(_ptr(x), T, H, block, _ptr(q), _ptr(scale), _ptr(workspace), nbytes,
                                  _stream(dev, stream)))
    return q, scale


def decompress_int8(q: torch.Tensor, scale: torch.Tensor, block: int = 0, *,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Inverse of compress_int8 with the same block: bf16 [tokens, hidden]."""
    with _on(stream):
        return _decompress_int8(q, scale, block, out, stream)


def _decompress_int8(q, scale, block, out, stream):
    lib = load()
    if q.dim() != 2 or q.dtype != torch.int8:
        raise ValueError("q must be a 2-D int8 tensor")
    if scale.dtype != torch.float32:
        raise ValueError("scale must be float32")
    dev = _require_gpu(q, scale)
    T, H = q.shape
    if scale.numel() != _int8_scales(T, H, block):
        raise ValueError("scale needs one element per tensor (block 0) or per block")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _require_gpu(q, out)
    _require_buffer(out, "out", torch.bfloat16, T * H, (T, H))
    _check(lib.taco_decompress_int8(_ptr(q.contiguous()), _ptr(scale.contiguous()), T, H, block, _ptr(out),
                                    _stream(dev, stream)))
    return out


def compress_delayed(x: torch.Tensor, block: int, amax_prev: torch.Tensor | None = None,
                     target_energy: float = 1.0, *, q: torch.Tensor | None = None,
                     alpha: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                     amax_out: torch.Tensor | None = None, stream=None):
    """Dual-Scale variant with the per-tensor scale of an earlier tensor:
    s = 448 / max(amax_prev) (1 if zero).  Returns (q, alpha, scale, amax_out),
    where amax_out (zero-filled when not passed) holds
    this tensor's largest |y| as its maximum (TACO_AMAX_FLOATS fp32; see
    include/taco.h), to pass as amax_prev next time.
    Decompress with decompress()."""
    with _on(stream):
        return _compress_delayed(x, block, amax_prev, target_energy, q, alpha, scale, amax_out, stream)


def _compress_delayed(x, block, amax_prev, target_energy, q, alpha, scale, amax_out, stream):
    x = x.contiguous()
    lib, dev, T, H, q, alpha, scale = _compress_outputs(x, block, q, alpha, scale, False)
    if amax_prev is None:
        amax_prev = torch.zeros(TACO_AMAX_FLOATS, dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.zeros(TACO_AMAX_FLOATS, dtype=torch.float32, device=dev)
    for t, name in ((amax_prev, "amax_prev"), (amax_out, "amax_out")):
        _require_gpu(x, t)
        _require_buffer(t, name, torch.float32, TACO_AMAX_FLOATS)
    _check(lib.taco_compress_delayed(_ptr(x), T, H, block, float(target_energy), _ptr(amax_prev), _ptr(q),
                                     _ptr(alpha), _ptr(scale), _ptr(amax_out), _stream(dev, stream)))
    return q, alpha, scale, amax_out


def two_shot_allreduce(xs, block: int, target_energy: float = 1.0, stream=None,
                       single_pass: bool = True) -> torch.Tensor:
    """The compressed two-shot all-reduce of P bf16 [T, H] tensors as P ranks
    would run it, emulated on one GPU with the library's calls: each rank's
    compress; per row shard j (T/P whole rows), decompress_sum_compress over
    the ranks' rows of that shard (the reduce-scatter step, FP8 out for the
    all-gather); decompress of every reduced shard.  Returns the bf16 result.
    single_pass as in compress()."""
    with _on(stream):
        xs = [x.contiguous() for x in xs]
        P = len(xs)
        if P < 1 or P > TACO_MAX_PARTS:
            _check(7)
        T, H = xs[0].shape
        if T % P != 0 or any(x.shape != (T, H) for x in xs):
            raise ValueError("P tensors of one shape whose rows split into P equal shards")
        rows = T // P
        comp = [compress(x, block, target_energy, stream=stream, single_pass=single_pass) for x in xs]
        out = torch.empty((T, H), dtype=torch.bfloat16, device=xs[0].device)
        for j in range(P):
            sl = slice(j * rows, (j + 1) * rows)
            red = decompress_sum_compress([(q[sl], a[sl], s) for q, a, s in comp], block, target_energy,
                                          stream=stream, single_pass=single_pass)
            decompress(*red, block, out=out[sl], stream=stream)
        return out
