"""GPTQ per-layer quantization solver on AMD gfx950 (MI355X).

A thin ctypes binding of ``libgptq.so`` (C ABI in ``include/gptq.h``).  The
functions keep the C names; PyTorch only provides device memory and the HIP
stream.  Every step of the solver runs in the library's HIP kernels; there is
no Python or CPU fallback, and loading fails loudly if the library is missing.

    H = torch.zeros(d, d, device="cuda")
    gptq_hessian_accumulate(H, X_chunk)            # once per calibration chunk
    U, lam, info = gptq_prepare_hinv(H, 0.01)
    codes, scales, zeros, err = gptq_quantize_layer(W, U, lam, bits=4, group_size=128)

``quantize_layer`` chains the three calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional

__all__ = [
    "GPTQ_F32", "GPTQ_F16", "GPTQError", "NotPositiveDefinite", "library", "lib_path",
    "gptq_hessian_accumulate", "gptq_hessian_accumulate_workspace_size",
    "gptq_prepare_hinv", "gptq_prepare_hinv_workspace_size",
    "gptq_quantize_layer", "gptq_quantize_layer_workspace_size", "gptq_quantize_layer_noalloc",
    "GPTQ_NOALLOC_SCRATCH_BYTES",
    "gptq_act_order_perm", "gptq_prepare_hinv_perm", "gptq_quantize_layer_perm",
    "gptq_packed_words_per_row", "gptq_pack_codes", "gptq_dequant_matmul", "gptq_dequantize",
    "gptq2d_quantize", "gptq2d_quantize_workspace_size",
    "gptq_launch_timing", "gptq_launch_timing_read", "TIMING_PANEL", "TIMING_PRODUCT",
    "gptq_status_string", "gptq_version", "quantize_layer",
]

GPTQ_F32 = 0
GPTQ_F16 = 1
GPTQ_NOALLOC_SCRATCH_BYTES = 96 << 20   # include/gptq.h
TIMING_PANEL, TIMING_PRODUCT = 0, 1     # kinds of gptq_launch_timing_read

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    """The in-tree libgptq.so, or the library named by GPTQ_LIBRARY (the
    sanitizer build of the host code is tested that way)."""
    return os.environ.get("GPTQ_LIBRARY") or os.path.join(_HERE, "_lib", "libgptq.so")


class GPTQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status}: {gptq_status_string(status)}")
        self.status = status


class NotPositiveDefinite(GPTQError):
    def __init__(self, info: int):
        RuntimeError.__init__(self, f"damped Hessian is not positive definite (info={info})")
        self.status = -1
        self.info = info


def library() -> ctypes.CDLL:
    """Load libgptq.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(python -m post_weight_quantization_02_amd._build)")
    lib = ctypes.CDLL(path)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.gptq_hessian_accumulate.argtypes = [vp, i64, vp, i32, i64, i64, vp, sz, vp]
    lib.gptq_hessian_accumulate.restype = i32
    lib.gptq_hessian_accumulate_workspace_size.argtypes = [i64, i64, i32]
    lib.gptq_hessian_accumulate_workspace_size.restype = sz
    lib.gptq_prepare_hinv.argtypes = [vp, i64, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.gptq_prepare_hinv.restype = i32
    lib.gptq_prepare_hinv_workspace_size.argtypes = [i64]
    lib.gptq_prepare_hinv_workspace_size.restype = sz
    lib.gptq_quantize_layer.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, i64, i64, vp, vp, vp,
                                        vp, vp, sz, vp]
    lib.gptq_quantize_layer.restype = i32
    lib.gptq_quantize_layer_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, i64, i64, vp, vp,
                                                vp, vp, vp]
    lib.gptq_quantize_layer_noalloc.restype = i32
    lib.gptq_quantize_layer_workspace_size.argtypes = [i64, i64, i64]
    lib.gptq_quantize_layer_workspace_size.restype = sz
    lib.gptq_act_order_perm.argtypes = [vp, i64, vp, vp]
    lib.gptq_act_order_perm.restype = i32
    lib.gptq_prepare_hinv_perm.argtypes = [vp, i64, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.gptq_prepare_hinv_perm.restype = i32
    lib.gptq_quantize_layer_perm.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, i64, i64, vp,
                                             vp, vp, vp, vp, vp, sz, vp]
    lib.gptq_quantize_layer_perm.restype = i32
    lib.gptq_packed_words_per_row.argtypes = [i64, i32]
    lib.gptq_packed_words_per_row.restype = i64
    lib.gptq_pack_codes.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, vp]
    lib.gptq_pack_codes.restype = i32
    lib.gptq_dequant_matmul.argtypes = [vp, i64, i32, vp, vp, i64, vp, i64, i64, vp, i32, i64, i64, vp,
                                        i64, vp]
    lib.gptq_dequant_matmul.restype = i32
    lib.gptq2d_quantize_workspace_size.argtypes = [i64, i64]
    lib.gptq2d_quantize_workspace_size.restype = sz
    lib.gptq2d_quantize.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.gptq2d_quantize.restype = i32
    lib.gptq_dequantize.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp, i32, i64, vp]
    lib.gptq_dequantize.restype = i32
    lib.gptq_launch_timing.argtypes = [i32]
    lib.gptq_launch_timing.restype = i32
    lib.gptq_launch_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64),
                                            ctypes.POINTER(ctypes.c_double)]
    lib.gptq_launch_timing_read.restype = i32
    lib.gptq_status_string.argtypes = [i32]
    lib.gptq_status_string.restype = ctypes.c_char_p
    lib.gptq_version.argtypes = []
    lib.gptq_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def gptq_status_string(status: int) -> str:
    return library().gptq_status_string(int(status)).decode()


def gptq_version() -> str:
    return library().gptq_version().decode()


# --------------------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, *tensors) -> Optional[int]:
    """The HIP stream handle to launch on.

    With no stream, or torch's current stream, nothing else happens.  With any
    other stream, that stream first waits for the work already queued on the
    current stream (the producer of the inputs, in torch's usual stream
    semantics), and every tensor the call touches (inputs, outputs and the
    workspace) is recorded as in use on that stream, so the caching allocator
    does not hand its memory out again before the launched kernels are done."""
    torch = _torch()
    cur = torch.cuda.current_stream()
    if stream is None or stream == cur:
        return cur.cuda_stream
    stream.wait_stream(cur)
    for t in tensors:
        if t is not None:
            t.record_stream(stream)
    return stream.cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return GPTQ_F16
    if t.dtype == torch.float32:
        return GPTQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _workspace(nbytes: int, device, ws=None):
    torch = _torch()
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _check(status: int, where: str):
    if status != 0:
        raise GPTQError(status, where)


# --------------------------------------------------------------------------- C names
def gptq_hessian_accumulate_workspace_size(d_col: int, n_rows: int, x_dtype: int) -> int:
    return int(library().gptq_hessian_accumulate_workspace_size(d_col, n_rows, x_dtype))


def gptq_prepare_hinv_workspace_size(d_col: int) -> int:
    return int(library().gptq_prepare_hinv_workspace_size(d_col))


def gptq_quantize_layer_workspace_size(d_row: int, d_col: int, block_size: int) -> int:
    return int(library().gptq_quantize_layer_workspace_size(d_row, d_col, block_size))


def gptq_hessian_accumulate(H, X, ws=None, stream=None):
    """H += 2 X^T X on the device (H [d x d] fp32, X [n x d] fp16/fp32 row-major)."""
    _rowmajor(X, "X")
    d = H.shape[0]
    n = X.shape[0]
    code = _dtype_code(X)
    need = gptq_hessian_accumulate_workspace_size(d, n, code)
    ws = _workspace(need, X.device, ws)
    st = library().gptq_hessian_accumulate(H.data_ptr(), d, X.data_ptr(), code, n, X.stride(0),
                                           ws.data_ptr(), ws.numel(), _stream(stream, H, X, ws))
    _check(st, "gptq_hessian_accumulate")
    return H


def gptq_prepare_hinv(H, percdamp: float = 0.01, U=None, lam=None, info=None, ws=None,
                      stream=None):
    """Damping and U (upper, U^T U = (H + lambda I)^-1).  Returns (U, lambda, info) as
    device tensors; ``info`` is nonzero if the damped H was not positive definite."""
    torch = _torch()
    d = H.shape[0]
    dev = H.device
    U = U if U is not None else torch.empty(d, d, dtype=torch.float32, device=dev)
    lam = lam if lam is not None else torch.empty(1, dtype=torch.float32, device=dev)
    info = info if info is not None else torch.empty(1, dtype=torch.int32, device=dev)
    ws = _workspace(gptq_prepare_hinv_workspace_size(d), dev, ws)
    st = library().gptq_prepare_hinv(H.data_ptr(), d, float(percdamp), U.data_ptr(),
                                     lam.data_ptr(), info.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream(stream, H, U, lam, info, ws))
    _check(st, "gptq_prepare_hinv")
    return U, lam, info


def gptq_quantize_layer(W0, U, lam=None, bits: int = 4, group_size: int = 0,
                        block_size: int = 128, codes=None, scales=None, zeros=None,
                        out_err=None, ws=None, stream=None):
    """The lazy-batch loop.  Returns (codes uint8, scales fp32, zeros int32, err fp64)."""
    torch = _torch()
    _rowmajor(W0, "W0")
    d_row, d_col = W0.shape
    dev = W0.device
    ng = -(-d_col // group_size) if group_size else 1
    codes = codes if codes is not None else torch.empty(d_row, d_col, dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty(d_row, ng, dtype=torch.float32, device=dev)
    zeros = zeros if zeros is not None else torch.empty(d_row, ng, dtype=torch.int32, device=dev)
    out_err = out_err if out_err is not None else torch.empty(1, dtype=torch.float64, device=dev)
    ws = _workspace(gptq_quantize_layer_workspace_size(d_row, d_col, block_size), dev, ws)
    st = library().gptq_quantize_layer(W0.data_ptr(), _dtype_code(W0), d_row, d_col, W0.stride(0),
                                       U.data_ptr(), _ptr(lam), int(bits), int(group_size),
                                       int(block_size), codes.data_ptr(), scales.data_ptr(),
                                       zeros.data_ptr(), out_err.data_ptr(), ws.data_ptr(),
                                       ws.numel(), _stream(stream, W0, U, lam, codes, scales, zeros,
                                                           out_err, ws))
    _check(st, "gptq_quantize_layer")
    return codes, scales, zeros, out_err


def gptq_quantize_layer_noalloc(W0, U, lam=None, bits: int = 4, group_size: int = 0,
                                block_size: int = 128, codes=None, scales=None, zeros=None,
                                out_err=None, stream=None):
    """gptq_quantize_layer without a workspace: the library's fixed per-device
    array (GPTQ_NOALLOC_SCRATCH_BYTES) serves as one.  Pass every output to keep
    the call free of allocations (e.g. under graph capture).  Calls that may
    overlap on one device race on that array."""
    torch = _torch()
    _rowmajor(W0, "W0")
    d_row, d_col = W0.shape
    dev = W0.device
    ng = -(-d_col // group_size) if group_size else 1
    codes = codes if codes is not None else torch.empty(d_row, d_col, dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty(d_row, ng, dtype=torch.float32, device=dev)
    zeros = zeros if zeros is not None else torch.empty(d_row, ng, dtype=torch.int32, device=dev)
    out_err = out_err if out_err is not None else torch.empty(1, dtype=torch.float64, device=dev)
    st = library().gptq_quantize_layer_noalloc(W0.data_ptr(), _dtype_code(W0), d_row, d_col, W0.stride(0),
                                               U.data_ptr(), _ptr(lam), int(bits), int(group_size),
                                               int(block_size), codes.data_ptr(), scales.data_ptr(),
                                               zeros.data_ptr(), out_err.data_ptr(),
                                               _stream(stream, W0, U, lam, codes, scales, zeros, out_err))
    _check(st, "gptq_quantize_layer_noalloc")
    return codes, scales, zeros, out_err


def gptq_act_order_perm(H, perm=None, stream=None):
    """Act-order quantization order: int32 [d] with perm[i] the column quantized at
    position i (descending diag(H), equal diagonals in ascending index order)."""
    torch = _torch()
    d = H.shape[0]
    perm = perm if perm is not None else torch.empty(d, dtype=torch.int32, device=H.device)
    st = library().gptq_act_order_perm(H.data_ptr(), d, perm.data_ptr(), _stream(stream, H, perm))
    _check(st, "gptq_act_order_perm")
    return perm


def gptq_prepare_hinv_perm(H, perm, percdamp: float = 0.01, U=None, lam=None, info=None,
                           ws=None, stream=None):
    """gptq_prepare_hinv for H with rows and columns in the order ``perm``; U is in
    that order.  Returns (U, lambda, info)."""
    torch = _torch()
    d = H.shape[0]
    dev = H.device
    U = U if U is not None else torch.empty(d, d, dtype=torch.float32, device=dev)
    lam = lam if lam is not None else torch.empty(1, dtype=torch.float32, device=dev)
    info = info if info is not None else torch.empty(1, dtype=torch.int32, device=dev)
    ws = _workspace(gptq_prepare_hinv_workspace_size(d), dev, ws)
    st = library().gptq_prepare_hinv_perm(H.data_ptr(), d, perm.data_ptr(), float(percdamp),
                                          U.data_ptr(), lam.data_ptr(), info.data_ptr(),
                                          ws.data_ptr(), ws.numel(),
                                          _stream(stream, H, perm, U, lam, info, ws))
    _check(st, "gptq_prepare_hinv_perm")
    return U, lam, info


def gptq_quantize_layer_perm(W0, U, lam, perm, bits: int = 4, group_size: int = 0,
                             block_size: int = 128, codes=None, scales=None, zeros=None,
                             g_idx=None, out_err=None, ws=None, stream=None):
    """The loop over the columns in the order ``perm`` (U from gptq_prepare_hinv_perm).
    Returns (codes in the original column order, scales, zeros, g_idx, err)."""
    torch = _torch()
    _rowmajor(W0, "W0")
    d_row, d_col = W0.shape
    dev = W0.device
    ng = -(-d_col // group_size) if group_size else 1
    codes = codes if codes is not None else torch.empty(d_row, d_col, dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty(d_row, ng, dtype=torch.float32, device=dev)
    zeros = zeros if zeros is not None else torch.empty(d_row, ng, dtype=torch.int32, device=dev)
    g_idx = g_idx if g_idx is not None else torch.empty(d_col, dtype=torch.int32, device=dev)
    out_err = out_err if out_err is not None else torch.empty(1, dtype=torch.float64, device=dev)
    ws = _workspace(gptq_quantize_layer_workspace_size(d_row, d_col, block_size), dev, ws)
    st = library().gptq_quantize_layer_perm(W0.data_ptr(), _dtype_code(W0), d_row, d_col,
                                            W0.stride(0), U.data_ptr(), _ptr(lam), perm.data_ptr(),
                                            int(bits), int(group_size), int(block_size),
                                            codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                            g_idx.data_ptr(), out_err.data_ptr(), ws.data_ptr(),
                                            ws.numel(), _stream(stream, W0, U, lam, perm, codes, scales,
                                                                zeros, g_idx, out_err, ws))
    _check(st, "gptq_quantize_layer_perm")
    return codes, scales, zeros, g_idx, out_err


def gptq_packed_words_per_row(d_col: int, bits: int) -> int:
    return int(library().gptq_packed_words_per_row(d_col, bits))


def gptq_pack_codes(codes, bits: int, perm=None, packed=None, stream=None):
    """Pack uint8 codes [d_row x d_col] into 32-bit words (position i holds column
    perm[i] when perm is given).  Returns the packed int32 tensor (bit patterns)."""
    torch = _torch()
    _rowmajor(codes, "codes")
    d_row, d_col = codes.shape
    words = gptq_packed_words_per_row(d_col, bits)
    packed = packed if packed is not None else torch.empty(d_row, words, dtype=torch.int32,
                                                             device=codes.device)
    st = library().gptq_pack_codes(codes.data_ptr(), d_row, d_col, codes.stride(0), int(bits),
                                   _ptr(perm), packed.data_ptr(), packed.stride(0),
                                   _stream(stream, codes, perm, packed))
    _check(st, "gptq_pack_codes")
    return packed


def gptq2d_quantize_workspace_size(m: int, n: int) -> int:
    return int(library().gptq2d_quantize_workspace_size(m, n))


def gptq2d_quantize(X, U_Q, U_P, bits: int, codes=None, scale=None, zero=None, out_err=None, ws=None,
                    stream=None):
    """Two-sided adaptive rounding of X [m x n] (fp16/fp32) with the upper factors
    U_Q [m x m] and U_P [n x n].  Returns (codes uint8, scale fp32 [1], zero int32 [1],
    err fp64 [1])."""
    torch = _torch()
    _rowmajor(X, "X")
    m, n = X.shape
    dev = X.device
    codes = codes if codes is not None else torch.empty(m, n, dtype=torch.uint8, device=dev)
    scale = scale if scale is not None else torch.empty(1, dtype=torch.float32, device=dev)
    zero = zero if zero is not None else torch.empty(1, dtype=torch.int32, device=dev)
    out_err = out_err if out_err is not None else torch.empty(1, dtype=torch.float64, device=dev)
    ws = _workspace(gptq2d_quantize_workspace_size(m, n), dev, ws)
    st = library().gptq2d_quantize(X.data_ptr(), _dtype_code(X), m, n, X.stride(0), U_Q.data_ptr(),
                                   U_P.data_ptr(), int(bits), codes.data_ptr(), codes.stride(0), scale.data_ptr(),
                                   zero.data_ptr(), out_err.data_ptr(), ws.data_ptr(), ws.numel(),
                                   _stream(stream, X, U_Q, U_P, codes, scale, zero, out_err, ws))
    _check(st, "gptq2d_quantize")
    return codes, scale, zero, out_err


def gptq_dequantize(codes, scales, zeros, group_size: int, g_idx=None, out=None, out_dtype=None,
                    stream=None):
    """What [d_row x d_col] = scales * (codes - zeros) per group (through g_idx if
    given), fp32 unless out / out_dtype say fp16."""
    torch = _torch()
    _rowmajor(codes, "codes")
    d_row, d_col = codes.shape
    if out is None:
        out = torch.empty(d_row, d_col, dtype=out_dtype or torch.float32, device=codes.device)
    _rowmajor(out, "out")
    st = library().gptq_dequantize(codes.data_ptr(), d_row, d_col, codes.stride(0), scales.data_ptr(),
                                   zeros.data_ptr(), int(group_size), _ptr(g_idx), out.data_ptr(),
                                   _dtype_code(out), out.stride(0),
                                   _stream(stream, codes, scales, zeros, g_idx, out))
    _check(st, "gptq_dequantize")
    return out


def gptq_dequant_matmul(packed, bits: int, scales, zeros, group_size: int, X, d_col: int,
                        perm=None, Y=None, stream=None):
    """Y [m x d_row] fp32 = X What^T from packed codes (1 <= m <= 8)."""
    torch = _torch()
    _rowmajor(X, "X")
    d_row = packed.shape[0]
    m = X.shape[0]
    Y = Y if Y is not None else torch.empty(m, d_row, dtype=torch.float32, device=X.device)
    st = library().gptq_dequant_matmul(packed.data_ptr(), packed.stride(0), int(bits), scales.data_ptr(),
                                       zeros.data_ptr(), int(group_size), _ptr(perm), d_row, d_col,
                                       X.data_ptr(), _dtype_code(X), m, X.stride(0), Y.data_ptr(),
                                       Y.stride(0), _stream(stream, packed, scales, zeros, perm, X, Y))
    _check(st, "gptq_dequant_matmul")
    return Y


def gptq_launch_timing(enable: bool) -> None:
    """Switch per-launch timing of the loop's panel and product launches on or
    off for the calling thread (a measurement aid)."""
    _check(library().gptq_launch_timing(1 if enable else 0), "gptq_launch_timing")


def gptq_launch_timing_read(kind: int):
    """(milliseconds, launches, work) summed over the recorded launches of
    ``kind`` (TIMING_PANEL: work in bytes; TIMING_PRODUCT: work in flop), which
    are then forgotten.  Waits for the recorded events."""
    ms, n, work = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double()
    _check(library().gptq_launch_timing_read(int(kind), ctypes.byref(ms), ctypes.byref(n), ctypes.byref(work)),
           "gptq_launch_timing_read")
    return ms.value, n.value, work.value


def quantize_layer(W0, x_chunks: Iterable, bits: int = 4, group_size: int = 0,
                   block_size: int = 128, percdamp: float = 0.01, act_order: bool = False,
                   stream=None):
    """All three calls for one layer (natural order, or act-order with
    ``act_order=True``); raises NotPositiveDefinite after synchronising if the
    damped Hessian could not be factored.  Returns a dict of device tensors."""
    torch = _torch()
    d_col = W0.shape[1]
    H = torch.zeros(d_col, d_col, dtype=torch.float32, device=W0.device)
    for xc in x_chunks:
        gptq_hessian_accumulate(H, xc, stream=stream)
    out = {"H": H}
    if act_order:
        perm = gptq_act_order_perm(H, stream=stream)
        U, lam, info = gptq_prepare_hinv_perm(H, perm, percdamp, stream=stream)
        codes, scales, zeros, g_idx, err = gptq_quantize_layer_perm(
            W0, U, lam, perm, bits, group_size, block_size, stream=stream)
        out.update(perm=perm, g_idx=g_idx)
    else:
        U, lam, info = gptq_prepare_hinv(H, percdamp, stream=stream)
        codes, scales, zeros, err = gptq_quantize_layer(W0, U, lam, bits, group_size, block_size,
                                                        stream=stream)
    (stream or torch.cuda.current_stream()).synchronize()
    if int(info.item()) != 0:
        raise NotPositiveDefinite(int(info.item()))
    out.update(U=U, codes=codes, scales=scales, zeros=zeros, err=err)
    out["lambda"] = lam
    return out
