"""Python binding of libfgq.so: fine-grained FP8 quantisation and the
block-scaled FP8 GEMM on MI355X (gfx950).

Argument marshalling only.  PyTorch supplies device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing, every call raises.

Functions (same names as the C ABI in include/fgq.h, without the prefix):

    quant_act_1x128(x)                     -> (q uint8 [M,K], s float32 [M,K/128])
    quant_w_128x128(w)                     -> (q uint8 [N,K] or [B,N,K], s float32 [.., N/128, K/128])
    fused_rmsnorm_quant(x, gamma, eps)     -> (q, s) as quant_act_1x128
    gemm_fp8_blockscaled(qa, sa, qw, sw)   -> c bfloat16 [M, N]
    grouped_gemm_fp8_blockscaled(qa, sa, qw, sw, offsets) -> c bfloat16 [R, N]
    gemm_bf16a_fp8_blockscaled(a, qw, sw)  -> c: the activation quantisation fused into the GEMM's A-load
    quant_dispatch_1x128(x, ids, E)        -> (q, s, offsets, row_src, dest): FP8 rows grouped by expert

Power-of-two (E8M0) scale variants, scales as uint8 exponent bytes
(value = 2^(byte - 127)) that the FP8 matrix core applies itself:

    quant_act_1x128_e8m0(x), quant_w_128x128_e8m0(w), fused_rmsnorm_quant_e8m0(x, gamma, eps)
    quant_dispatch_1x128_e8m0(x, ids, E)
    gemm_fp8_e8m0(qa, sa, qw, sw, accumulate=E8M0_PROMOTE)
    grouped_gemm_fp8_e8m0(qa, sa, qw, sw, offsets, accumulate=E8M0_PROMOTE)

Codes are returned as ``torch.uint8`` (``.view(torch.float8_e4m3fn)`` gives
the FP8 dtype).  Scales may be any strided float32 view; the strides are
passed to the kernels as they are.  Activation scales are allocated
K-block-major by default (storage [K/128, M], returned as the [M, K/128]
view): a GEMM tile then loads the scales of one K chunk from consecutive
addresses.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "FgqError", "load_library", "library_path", "lib",
    "quant_act_1x128", "quant_w_128x128", "fused_rmsnorm_quant", "act_scales",
    "gemm_fp8_blockscaled", "grouped_gemm_fp8_blockscaled", "gemm_workspace_bytes",
    "quant_dispatch_1x128", "quant_dispatch_workspace_bytes",
    "debug_encode_e4m3", "debug_copy", "debug_mfma_16x16x128", "STATUS", "GEMM_EXACT", "GEMM_FP8_CORE",
    "quant_act_1x128_e8m0", "quant_w_128x128_e8m0", "fused_rmsnorm_quant_e8m0", "act_scales_e8m0",
    "gemm_fp8_e8m0", "grouped_gemm_fp8_e8m0", "debug_mfma_e8m0_16x16x128", "E8M0_PROMOTE", "E8M0_IN_CORE",
    "quant_dispatch_1x128_e8m0", "gemm_bf16a_fp8_blockscaled", "debug_mfma_loop", "MFMA_LOOP_FLOPS",
    "gemm_fp8_blockscaled_noalloc",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))

GEMM_EXACT = 0       # exact FP8 products on the FP16 matrix cores (default)
GEMM_FP8_CORE = 1    # FP8 matrix cores: 2x rate, ~13-bit in-group accumulation window

E8M0_PROMOTE = 0     # E8M0 GEMMs: per-chunk sum promoted into an FP32 accumulator (default)
E8M0_IN_CORE = 1     # E8M0 GEMMs: running sum kept in the matrix core (no promotion)

STATUS = {
    0: "FGQ_OK", 1: "FGQ_ERR_NULL", 2: "FGQ_ERR_SHAPE", 3: "FGQ_ERR_ALIGN",
    4: "FGQ_ERR_STRIDE", 5: "FGQ_ERR_UNSUPPORTED", 6: "FGQ_ERR_HIP", 7: "FGQ_ERR_SCRATCH",
}


class FgqError(RuntimeError):
    """A nonzero status from libfgq, or the library could not be loaded."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


def library_path() -> str:
    return os.environ.get("FGQ_LIB", os.path.join(_PKG_DIR, "libfgq.so"))


_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_st = ctypes.c_int32

_SIGNATURES = {
    "fgq_quant_act_1x128": [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp],
    "fgq_quant_w_128x128": [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _vp],
    "fgq_fused_rmsnorm_quant": [_vp, _i64, _vp, _f32, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp],
    "fgq_gemm_fp8_blockscaled": [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64,
                                 _i64, _i64, _i64, _st, _vp, ctypes.c_size_t, _vp],
    "fgq_grouped_gemm_fp8_blockscaled": [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                         _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _st, _vp],
    "fgq_gemm_workspace_bytes": [_i64, _i64, _i64],
    "fgq_quant_dispatch_1x128": [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                                 _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "fgq_quant_dispatch_workspace_bytes": [_i64, _i64, _i64, _i64],
    "fgq_status_string": [_st],
    "fgq_last_hip_error": [],
    "fgq_abi_version": [],
    "fgq_debug_encode_e4m3": [ctypes.c_uint32, _i64, _vp, _vp],
    "fgq_debug_copy": [_vp, _vp, _i64, _vp],
    "fgq_debug_mfma_16x16x128": [_vp, _vp, _vp, _vp, _vp],
    "fgq_quant_act_1x128_e8m0": [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp],
    "fgq_quant_w_128x128_e8m0": [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _vp],
    "fgq_fused_rmsnorm_quant_e8m0": [_vp, _i64, _vp, _f32, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp],
    "fgq_gemm_fp8_e8m0": [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64,
                          _i64, _i64, _i64, _st, _vp, ctypes.c_size_t, _vp],
    "fgq_grouped_gemm_fp8_e8m0": [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                  _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _st, _vp],
    "fgq_debug_mfma_e8m0_16x16x128": [_vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "fgq_debug_mfma_loop": [_st, _i64, _i64, _vp, _vp, _vp],
    "fgq_gemm_fp8_blockscaled_noalloc": [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64,
                                         _i64, _i64, _i64, _st, _vp],
    "fgq_gemm_bf16a_fp8_blockscaled": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _st,
                                       _vp, _i64, _vp, _i64, _i64, _vp, ctypes.c_size_t, _vp],
    "fgq_quant_dispatch_1x128_e8m0": [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                                      _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
}
_RESTYPES = {
    "fgq_gemm_workspace_bytes": ctypes.c_size_t,
    "fgq_quant_dispatch_workspace_bytes": ctypes.c_size_t,
    "fgq_status_string": ctypes.c_char_p,
}

lib = None


def load_library(path: str | None = None):
    """Load libfgq.so (once) and declare its C signatures.  Raises FgqError if absent."""
    global lib
    if lib is not None:
        return lib
    # torch first: it brings its own HIP runtime, and libfgq must bind to that
    # same runtime (same soname).  Loaded before torch, the library would pull
    # in the system ROCm runtime and its launches would go to a second runtime
    # that fails with "no device" once torch has set up its own.
    _torch()
    path = path or library_path()
    if not os.path.exists(path):
        raise FgqError(-1, f"libfgq.so not found at {path}; build it with "
                           f"`python -m fine_grained_fp8_quant_amd.build`")
    handle = ctypes.CDLL(path)
    for name, args in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, _st)
    lib = handle
    return lib


def _check(status: int):
    if status != 0:
        msg = lib.fgq_status_string(status).decode()
        if status == 6:
            msg += f" (hipError {lib.fgq_last_hip_error()})"
        raise FgqError(status, msg)


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _scoped(fn):
    """Run a call helper (its last positional argument is the caller's stream,
    or None) with that stream current, so the outputs and scratch buffers it
    allocates come from that stream's pool and are not handed to another
    stream while the call's kernels still use them."""
    import functools

    @functools.wraps(fn)
    def run(*args):
        stream = args[-1]
        if stream is None:
            return fn(*args)
        with _torch().cuda.stream(stream):
            return fn(*args)
    return run


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _need(t, dtype, what):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected dtype {dtype}, got {t.dtype}")
    if t.numel() > 0 and not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")
    if t.dim() >= 1 and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{what}: the last dimension must be contiguous")


def _need_scales(t, what, dtype=None):
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype} scales, got {t.dtype}")
    if t.numel() > 0 and not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")


def _codes(t):
    """Accept uint8 or float8_e4m3fn code tensors; return a uint8 view."""
    torch = _torch()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t


def act_scales(M: int, K: int, device, dtype=None):
    """Uninitialised activation-scale buffer for an [M, K] operand: a
    [M, K/128] view of K-block-major storage (strides (1, M)); float32 unless
    ``dtype`` says otherwise."""
    torch = _torch()
    return torch.empty((K // 128, M), dtype=dtype or torch.float32, device=device).t()


def act_scales_e8m0(M: int, K: int, device):
    """As act_scales, for E8M0 exponent bytes (uint8)."""
    return act_scales(M, K, device, _torch().uint8)


@_scoped
def _quant_act(fn, sdtype, x, q, s, stream):
    torch = _torch()
    load_library()
    _need(x, torch.bfloat16, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = act_scales(M, K, x.device, sdtype)
    _need_scales(s, "s", sdtype)
    _check(fn(_ptr(x), x.stride(0), M, K, _ptr(q), q.stride(0), _ptr(s), s.stride(0), s.stride(1), _stream(stream)))
    return q, s


def quant_act_1x128(x, q=None, s=None, stream=None):
    """1x128 tile quantisation of BF16 ``x [M, K]``.  Optional preallocated
    outputs ``q`` (uint8 [M, K]) and ``s`` (float32 view of shape [M, K/128],
    any strides)."""
    load_library()
    return _quant_act(lib.fgq_quant_act_1x128, _torch().float32, x, q, s, stream)


def quant_act_1x128_e8m0(x, q=None, s=None, stream=None):
    """quant_act_1x128 with power-of-two scales: ``s`` holds uint8 E8M0 bytes."""
    load_library()
    return _quant_act(lib.fgq_quant_act_1x128_e8m0, _torch().uint8, x, q, s, stream)


@_scoped
def _quant_w(fn, sdtype, w, q, s, stream):
    torch = _torch()
    load_library()
    _need(w, torch.bfloat16, "w")
    batched = w.dim() == 3
    w3 = w if batched else w.unsqueeze(0)
    B, N, K = w3.shape
    if q is None:
        q = torch.empty((B, N, K), dtype=torch.uint8, device=w.device)
    elif not batched:
        q = q.unsqueeze(0)
    if s is None:
        s = torch.empty((B, N // 128, K // 128), dtype=sdtype, device=w.device)
    elif not batched:
        s = s.unsqueeze(0)
    _need_scales(s, "s", sdtype)
    _check(fn(_ptr(w3), w3.stride(1), w3.stride(0), B, N, K, _ptr(q), q.stride(1), q.stride(0), _ptr(s),
              s.stride(1), s.stride(2), s.stride(0), _stream(stream)))
    return (q, s) if batched else (q[0], s[0])


def quant_w_128x128(w, q=None, s=None, stream=None):
    """128x128 block quantisation of BF16 ``w [N, K]`` or ``[B, N, K]``."""
    load_library()
    return _quant_w(lib.fgq_quant_w_128x128, _torch().float32, w, q, s, stream)


def quant_w_128x128_e8m0(w, q=None, s=None, stream=None):
    """quant_w_128x128 with power-of-two scales: ``s`` holds uint8 E8M0 bytes."""
    load_library()
    return _quant_w(lib.fgq_quant_w_128x128_e8m0, _torch().uint8, w, q, s, stream)


@_scoped
def _fused(fn, sdtype, x, gamma, eps, q, s, stream):
    torch = _torch()
    load_library()
    _need(x, torch.bfloat16, "x")
    _need(gamma, torch.bfloat16, "gamma")
    M, K = x.shape
    if gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous [K] tensor")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = act_scales(M, K, x.device, sdtype)
    _need_scales(s, "s", sdtype)
    _check(fn(_ptr(x), x.stride(0), _ptr(gamma), float(eps), M, K, _ptr(q), q.stride(0), _ptr(s), s.stride(0),
              s.stride(1), _stream(stream)))
    return q, s


def fused_rmsnorm_quant(x, gamma, eps: float, q=None, s=None, stream=None):
    """RMSNorm(x; gamma, eps) in binary32 fused with 1x128 quantisation."""
    load_library()
    return _fused(lib.fgq_fused_rmsnorm_quant, _torch().float32, x, gamma, eps, q, s, stream)


def fused_rmsnorm_quant_e8m0(x, gamma, eps: float, q=None, s=None, stream=None):
    """fused_rmsnorm_quant with power-of-two scales (uint8 E8M0 bytes)."""
    load_library()
    return _fused(lib.fgq_fused_rmsnorm_quant_e8m0, _torch().uint8, x, gamma, eps, q, s, stream)


def quant_dispatch_workspace_bytes(T: int, topk: int, E: int, K: int) -> int:
    load_library()
    return int(lib.fgq_quant_dispatch_workspace_bytes(T, topk, E, K))


def quant_dispatch_1x128(x, ids, n_experts: int, q=None, s=None, offsets=None, row_src=None, dest=None,
                         workspace=None, stream=None):
    """Quantise-then-dispatch of BF16 tokens ``x [T, K]`` routed by ``ids``
    (int32 ``[T, topk]``, device) to ``n_experts`` experts.  Returns
    ``(q, s, offsets, row_src, dest)``: ``q`` uint8 and ``s`` float32 with
    room for ``T * topk`` rows (rows of expert e are
    ``offsets[e] .. offsets[e+1] - 1``), ``offsets`` int32 ``[E + 1]``,
    ``row_src`` and ``dest`` int32 ``[T * topk]`` (see include/fgq.h)."""
    load_library()
    return _dispatch(lib.fgq_quant_dispatch_1x128, _torch().float32, x, ids, n_experts, q, s, offsets, row_src,
                     dest, workspace, stream)


def quant_dispatch_1x128_e8m0(x, ids, n_experts: int, q=None, s=None, offsets=None, row_src=None, dest=None,
                              workspace=None, stream=None):
    """quant_dispatch_1x128 with power-of-two scales (``s`` uint8 E8M0 bytes)."""
    load_library()
    return _dispatch(lib.fgq_quant_dispatch_1x128_e8m0, _torch().uint8, x, ids, n_experts, q, s, offsets, row_src,
                     dest, workspace, stream)


@_scoped
def _dispatch(fn, sdtype, x, ids, n_experts, q, s, offsets, row_src, dest, workspace, stream):
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    _need(ids, torch.int32, "ids")
    T, K = x.shape
    if ids.dim() != 2 or ids.shape[0] != T or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 [T, topk] tensor")
    topk = ids.shape[1]
    R = T * topk
    dev = x.device
    if q is None:
        q = torch.empty((R, K), dtype=torch.uint8, device=dev)
    if s is None:
        s = act_scales(R, K, dev, sdtype)
    _need_scales(s, "s", sdtype)
    if offsets is None:
        offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    if row_src is None:
        row_src = torch.empty(R, dtype=torch.int32, device=dev)
    if dest is None:
        dest = torch.empty(R, dtype=torch.int32, device=dev)
    need = quant_dispatch_workspace_bytes(T, topk, n_experts, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = _nbytes(workspace)
    _check(fn(_ptr(x), x.stride(0), T, K, _ptr(ids), topk, n_experts, _ptr(q), q.stride(0), _ptr(s), s.stride(0),
              s.stride(1), _ptr(offsets), _ptr(row_src), _ptr(dest), _ptr(workspace), ws_bytes, _stream(stream)))
    return q, s, offsets, row_src, dest


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    load_library()
    return int(lib.fgq_gemm_workspace_bytes(M, N, K))


def gemm_fp8_blockscaled(qa, sa, qw, sw, out=None, workspace=None, mode=GEMM_EXACT, stream=None):
    """``C = (dec(qa) * sa) @ (dec(qw) * sw).T`` with per-chunk FP32 promotion, BF16 out.
    ``mode``: GEMM_EXACT (default) or GEMM_FP8_CORE."""
    load_library()
    return _gemm(lib.fgq_gemm_fp8_blockscaled, _torch().float32, qa, sa, qw, sw, out, workspace, mode, stream)


def gemm_fp8_blockscaled_noalloc(qa, sa, qw, sw, out, mode=GEMM_EXACT, stream=None):
    """gemm_fp8_blockscaled through the library's no-allocation entry point:
    the call uses the library's own device scratch and allocates nothing, so
    ``out`` (bfloat16 [M, N]) must be given.  Calls that can overlap on one GPU
    share that scratch and must be serialised by the caller."""
    torch = _torch()
    load_library()
    qa, qw = _codes(qa), _codes(qw)
    _need(qa, torch.uint8, "qa")
    _need(qw, torch.uint8, "qw")
    _need_scales(sa, "sa")
    _need_scales(sw, "sw")
    _need(out, torch.bfloat16, "out")
    M, K = qa.shape
    N = qw.shape[0]
    if qw.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("qa, qw and out disagree on M, N or K")
    _check(lib.fgq_gemm_fp8_blockscaled_noalloc(
        _ptr(qa), qa.stride(0), _ptr(sa), sa.stride(0), sa.stride(1), _ptr(qw), qw.stride(0), _ptr(sw),
        sw.stride(0), sw.stride(1), _ptr(out), out.stride(0), M, N, K, int(mode), _stream(stream)))
    return out


def gemm_fp8_e8m0(qa, sa, qw, sw, out=None, workspace=None, accumulate=E8M0_PROMOTE, stream=None):
    """The block-scaled GEMM with E8M0 scale bytes ``sa`` [M, K/128] and ``sw``
    [N/128, K/128] (uint8), applied by the matrix core.  ``accumulate``:
    E8M0_PROMOTE (default) or E8M0_IN_CORE."""
    load_library()
    return _gemm(lib.fgq_gemm_fp8_e8m0, _torch().uint8, qa, sa, qw, sw, out, workspace, accumulate, stream)


@_scoped
def _gemm(fn, sdtype, qa, sa, qw, sw, out, workspace, mode, stream):
    torch = _torch()
    qa, qw = _codes(qa), _codes(qw)
    _need(qa, torch.uint8, "qa")
    _need(qw, torch.uint8, "qw")
    _need_scales(sa, "sa", sdtype)
    _need_scales(sw, "sw", sdtype)
    M, K = qa.shape
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError("qa and qw disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
    need = gemm_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=qa.device)
    ws_bytes = _nbytes(workspace)
    _check(fn(_ptr(qa), qa.stride(0), _ptr(sa), sa.stride(0), sa.stride(1), _ptr(qw), qw.stride(0), _ptr(sw),
              sw.stride(0), sw.stride(1), _ptr(out), out.stride(0), M, N, K, int(mode), _ptr(workspace), ws_bytes,
              _stream(stream)))
    return out


def gemm_bf16a_fp8_blockscaled(a, qw, sw, out=None, workspace=None, mode=GEMM_EXACT, qa_out=None, sa_out=None,
                               stream=None):
    """GEMM of BF16 ``a [M, K]`` with quantised weights, the 1x128 quantisation of
    ``a`` done inside the GEMM's A-load.  Optional ``qa_out`` (uint8 [M, K]) and
    ``sa_out`` (float32 [M, K/128] view) receive the codes and scales."""
    return _gemm_bf16a(a, qw, sw, out, workspace, mode, qa_out, sa_out, stream)


@_scoped
def _gemm_bf16a(a, qw, sw, out, workspace, mode, qa_out, sa_out, stream):
    torch = _torch()
    load_library()
    qw = _codes(qw)
    _need(a, torch.bfloat16, "a")
    _need(qw, torch.uint8, "qw")
    _need_scales(sw, "sw")
    M, K = a.shape
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError("a and qw disagree on K")
    if (qa_out is None) != (sa_out is None):
        raise ValueError("give both qa_out and sa_out, or neither")
    if sa_out is not None:
        _need_scales(sa_out, "sa_out")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    need = gemm_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
    ws_bytes = _nbytes(workspace)
    _check(lib.fgq_gemm_bf16a_fp8_blockscaled(
        _ptr(a), a.stride(0), _ptr(qw), qw.stride(0), _ptr(sw), sw.stride(0), sw.stride(1), _ptr(out), out.stride(0),
        M, N, K, int(mode), _ptr(qa_out), qa_out.stride(0) if qa_out is not None else 0, _ptr(sa_out),
        sa_out.stride(0) if sa_out is not None else 0, sa_out.stride(1) if sa_out is not None else 0,
        _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def grouped_gemm_fp8_blockscaled(qa, sa, qw, sw, offsets, out=None, mode=GEMM_EXACT, stream=None):
    """Ragged grouped GEMM: rows ``offsets[e]..offsets[e+1]`` of ``qa`` times expert
    ``e``'s ``qw[e]``.  ``offsets`` is a device int32 tensor of E+1 entries."""
    load_library()
    return _grouped(lib.fgq_grouped_gemm_fp8_blockscaled, _torch().float32, qa, sa, qw, sw, offsets, out, mode,
                    stream)


def grouped_gemm_fp8_e8m0(qa, sa, qw, sw, offsets, out=None, accumulate=E8M0_PROMOTE, stream=None):
    """grouped_gemm_fp8_blockscaled with E8M0 scale bytes (uint8) and the
    accumulation choice of gemm_fp8_e8m0."""
    load_library()
    return _grouped(lib.fgq_grouped_gemm_fp8_e8m0, _torch().uint8, qa, sa, qw, sw, offsets, out, accumulate,
                    stream)


@_scoped
def _grouped(fn, sdtype, qa, sa, qw, sw, offsets, out, mode, stream):
    torch = _torch()
    qa, qw = _codes(qa), _codes(qw)
    _need(qa, torch.uint8, "qa")
    _need(qw, torch.uint8, "qw")
    _need(offsets, torch.int32, "offsets")
    _need_scales(sa, "sa", sdtype)
    _need_scales(sw, "sw", sdtype)
    R, K = qa.shape
    E, N, K2 = qw.shape
    if K2 != K:
        raise ValueError("qa and qw disagree on K")
    if offsets.numel() != E + 1:
        raise ValueError("offsets must have E + 1 entries")
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=qa.device)
    _check(fn(_ptr(qa), qa.stride(0), _ptr(sa), sa.stride(0), sa.stride(1), _ptr(qw), qw.stride(1), qw.stride(0),
              _ptr(sw), sw.stride(1), sw.stride(2), sw.stride(0), _ptr(offsets), E, R, _ptr(out), out.stride(0), N, K,
              int(mode), _stream(stream)))
    return out


def debug_encode_e4m3(start: int, n: int, out=None, stream=None):
    """Device E4M3 codes of clamp(float(bits), +-448) for bits = start .. start+n-1."""
    torch = _torch()
    load_library()
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device="cuda")
    _check(lib.fgq_debug_encode_e4m3(start & 0xFFFFFFFF, n, _ptr(out), _stream(stream)))
    return out


def debug_mfma_16x16x128(a, b, cin=None, stream=None):
    """One matrix-core op: a, b uint8 E4M3 [16,128] device tensors; returns float32 [16,16]."""
    torch = _torch()
    load_library()
    if cin is None:
        cin = torch.zeros((16, 16), dtype=torch.float32, device=a.device)
    d = torch.empty((16, 16), dtype=torch.float32, device=a.device)
    _check(lib.fgq_debug_mfma_16x16x128(_ptr(a.contiguous()), _ptr(b.contiguous()), _ptr(cin.contiguous()),
                                        _ptr(d), _stream(stream)))
    return d


def debug_mfma_e8m0_16x16x128(a, b, sa, sb, cin=None, stream=None):
    """One scaled matrix-core op: a, b uint8 E4M3 [16,128]; sa, sb uint8 [16] E8M0
    row / column scales; returns float32 [16,16] = diag(2^(sa-127)) a b^T diag(2^(sb-127)) + cin."""
    torch = _torch()
    load_library()
    if cin is None:
        cin = torch.zeros((16, 16), dtype=torch.float32, device=a.device)
    d = torch.empty((16, 16), dtype=torch.float32, device=a.device)
    _check(lib.fgq_debug_mfma_e8m0_16x16x128(_ptr(a.contiguous()), _ptr(b.contiguous()), _ptr(sa.contiguous()),
                                             _ptr(sb.contiguous()), _ptr(cin.contiguous()), _ptr(d), _stream(stream)))
    return d


MFMA_LOOP_FLOPS = {0: 65536, 1: 16384, 2: 32768}   # per operation of each fgq_debug_mfma_loop kind
_MFMA_LOOP_OPS = {0: 8, 1: 8, 2: 8}                # operations per wave per round


def debug_mfma_loop(kind: int, iters: int, waves: int = 2048, stream=None):
    """Run fgq_debug_mfma_loop once; returns a dict with the elapsed time
    (HIP events, ms), the matrix-core rate (TFLOP/s) over the whole launch,
    and the shader clock (GHz) the waves measured while they ran."""
    torch = _torch()
    load_library()
    with (torch.cuda.stream(stream) if stream is not None else __import__("contextlib").nullcontext()):
        out = torch.zeros(4 * waves, dtype=torch.int64, device="cuda")
        sink = torch.empty(64 * waves, dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        _check(lib.fgq_debug_mfma_loop(int(kind), int(iters), int(waves), _ptr(out), _ptr(sink), _stream(stream)))
        e1.record(st)
        e1.synchronize()
    ms = e0.elapsed_time(e1)
    t = out.view(waves, 4).cpu().numpy().astype(float)
    clk = (t[:, 1] - t[:, 0]).sum()
    real = (t[:, 3] - t[:, 2]).sum()
    flops = float(waves) * iters * _MFMA_LOOP_OPS[kind] * MFMA_LOOP_FLOPS[kind]
    return {"kind": int(kind), "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "sclk_ghz": clk / real * 0.1 if real > 0 else float("nan"), "waves": int(waves), "iters": int(iters)}


def debug_copy(src, dst, stream=None):
    load_library()
    _check(lib.fgq_debug_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(), _stream(stream)))
    return dst
