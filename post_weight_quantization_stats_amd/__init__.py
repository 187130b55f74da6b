"""AWQ per-layer scale search on AMD Instinct MI355X (gfx950).

Thin ctypes binding over libawq_mi355x.so (C ABI in include/awq_mi355x.h).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, allocates outputs with torch on the tensors' device and
passes raw device pointers plus the current HIP stream.  There is no CPU
fallback: if the library cannot be loaded the calls raise.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

__all__ = ["AwqError", "lib", "library_path", "act_stats", "candidate_scales", "quantize_pack",
           "reference_gemm", "w4a16_gemm", "search_scale", "search_scale_gram", "decode_gemm",
           "dequant_operand", "diff_operand", "candidate_sse", "quantize_pack3", "decode_gemm3",
           "decode_tiles", "decode_tiles_size", "decode_gemm_tiled", "decode_gemm_tiled_noalloc", "LAYOUT_NIBBLE", "LAYOUT_INT3_DENSE",
           "quantize_pack16", "expand_meta16", "decode_gemm_tiled16", "decode_meta_size",
           "decode_meta", "decode_gemm_tiled_meta", "ceiling_mfma", "ceiling_stream",
           "CEILING_COPY", "CEILING_READ", "CEILING_WRITE",
           "rmsnorm", "silu_mul", "divide_rows", "residual_add", "workspace_size",
           "OP_ACT_STATS", "OP_W4A16_GEMM", "OP_SEARCH_SCALE", "OP_CANDIDATE_SCALES",
           "OP_DECODE_GEMM", "OP_CANDIDATE_SSE", "OP_SEARCH_SCALE_GRAM", "OP_W4A16_GEMM_STAGED"]

(OP_ACT_STATS, OP_W4A16_GEMM, OP_SEARCH_SCALE, OP_CANDIDATE_SCALES, OP_DECODE_GEMM,
 OP_CANDIDATE_SSE, OP_SEARCH_SCALE_GRAM, OP_W4A16_GEMM_STAGED) = 0, 1, 2, 3, 4, 5, 6, 7

CEILING_COPY, CEILING_READ, CEILING_WRITE = 0, 1, 2

_c_void_p, _i64, _i32, _size_t = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t

# name -> argtypes (restype is int32 status unless noted)
_SIGNATURES = {
    "awq_abi_version": ([], _i32),
    "awq_status_string": ([_i32], ctypes.c_char_p),
    "awq_last_error": ([], ctypes.c_char_p),
    "awq_workspace_size": ([_i32, _i64, _i64, _i64, _i32, _i32, _i32, ctypes.POINTER(_size_t)], _i32),
    "awq_act_stats": ([_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
    "awq_candidate_scales": ([_c_void_p, _i64, _i32, _c_void_p, _c_void_p, _c_void_p, _size_t,
                              _c_void_p], _i32),
    "awq_quantize_pack": ([_c_void_p, _i64, _i64, _c_void_p, _i32, _i32, _c_void_p, _c_void_p,
                           _c_void_p, _c_void_p], _i32),
    "awq_dequant_operand": ([_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i32, _i32, _c_void_p,
                             _c_void_p], _i32),
    "awq_quantize_pack3": ([_c_void_p, _i64, _i64, _c_void_p, _i32, _c_void_p, _c_void_p,
                            _c_void_p, _c_void_p], _i32),
    "awq_w3a16_decode_gemm": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _i32,
                               _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
    "awq_decode_tiles_size": ([_i64, _i64, _i32, _i32, _c_void_p], _i32),
    "awq_decode_tiles": ([_c_void_p, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p], _i32),
    "awq_decode_gemm_tiled": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _i32,
                               _i32, _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
    "awq_decode_gemm_tiled_noalloc": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                       _c_void_p, _i32, _i32, _c_void_p, _c_void_p], _i32),
    "awq_quantize_pack16": ([_c_void_p, _i64, _i64, _c_void_p, _i32, _i32, _i32, _c_void_p,
                             _c_void_p, _c_void_p, _c_void_p], _i32),
    "awq_expand_meta16": ([_c_void_p, _c_void_p, _i64, _i64, _i32, _c_void_p, _c_void_p,
                           _c_void_p], _i32),
    "awq_decode_gemm_tiled16": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                 _i32, _i32, _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
    "awq_decode_meta_size": ([_i64, _i64, _i32, _c_void_p], _i32),
    "awq_decode_meta": ([_c_void_p, _c_void_p, _i64, _i64, _i32, _c_void_p, _c_void_p], _i32),
    "awq_decode_gemm_tiled_meta": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _i32, _i32,
                                    _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
    "awq_ceiling_mfma": ([_i32, _i32, _i32, _c_void_p, ctypes.POINTER(_i64), _c_void_p], _i32),
    "awq_ceiling_stream": ([_i32, _c_void_p, _c_void_p, _size_t, _i32, _c_void_p], _i32),
    "awq_rmsnorm": ([_c_void_p, _i64, _i64, _c_void_p, ctypes.c_double, _c_void_p, _c_void_p,
                     _c_void_p], _i32),
    "awq_silu_mul": ([_c_void_p, _i64, _i64, _c_void_p, _c_void_p], _i32),
    "awq_divide_rows": ([_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p], _i32),
    "awq_residual_add": ([_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p], _i32),
    "awq_diff_operand": ([_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i32, _i32, _c_void_p,
                          _c_void_p], _i32),
    "awq_candidate_sse": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _size_t, _c_void_p], _i32),
    "awq_reference_gemm": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p], _i32),
    "awq_w4a16_gemm": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                        _c_void_p], _i32),
    "awq_w3a16_gemm": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _i32,
                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                        _c_void_p], _i32),
    "awq_w4a16_gemm_staged": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _i32,
                               _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _size_t, _c_void_p], _i32),
    "awq_w4a16_decode_gemm": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _i32,
                               _i32, _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
    "awq_search_scale_gram": ([_c_void_p, _i64, _i64, _c_void_p, _i64, _i32, _i32, _i32,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
    "awq_search_scale": ([_c_void_p, _i64, _i64, _c_void_p, _i64, _i32, _i32, _i32, _c_void_p,
                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                          _c_void_p, _size_t, _c_void_p], _i32),
}

_LIB = None


class AwqError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        self.status = status
        super().__init__(f"{func}: {lib().awq_status_string(status).decode()} ({message})")


def library_path() -> str:
    return _build.LIB_PATH


def lib() -> ctypes.CDLL:
    """Load the HIP library (building it first only if no build exists)."""
    global _LIB
    if _LIB is None:
        path = _build.LIB_PATH
        if not os.path.exists(path):
            _build.build()
        handle = ctypes.CDLL(path)
        for name, (argtypes, restype) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _LIB = handle
    return _LIB


def _check(status: int, func: str) -> None:
    if status != 0:
        raise AwqError(status, func, lib().awq_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _tensor(t, name: str, dtypes, shape=None) -> torch.Tensor:
    """Validate a tensor argument before any pointer reaches the library:
    its dtype, exact shape and contiguity.  The kernels size their accesses
    from the shape arguments, not from the allocations, so a mismatch here
    would read or write past a buffer on the device.  Where the tensors live
    is checked afterwards, once for all of a call's tensors (_gpu), so every
    shape error is reported the same way on any machine."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} must have shape {tuple(int(v) for v in shape)} "
                         f"(got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _gpu(**tensors) -> torch.device:
    """Every given tensor (None skipped) is on the same GPU; returns it."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")
    return dev


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_WORDS = (torch.int32, torch.uint32)


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if isinstance(t, torch.Tensor) and t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return _tensor(t, name, _BF16)


def _f32(t: torch.Tensor, name: str, shape=None) -> torch.Tensor:
    return _tensor(t, name, torch.float32, shape)


def _vec_f32(t: torch.Tensor | None, name: str, n: int) -> torch.Tensor | None:
    """Optional float32 vector of n elements (s, inv_s): 1-D or any shape of n."""
    if t is None:
        return None
    _tensor(t, name, torch.float32)
    if t.numel() != n:
        raise ValueError(f"{name} must have {n} elements (got {t.numel()})")
    return t


def _meta(scales, zeros, N: int, K: int, group: int):
    """fp32 steps and u8 zeros, [N][K/group] each."""
    if group <= 0 or K % group:
        raise ValueError(f"K={K} must be a multiple of the group size {group}")
    _tensor(scales, "scales", torch.float32, (N, K // group))
    _tensor(zeros, "zeros", torch.uint8, (N, K // group))


def _out(out, M: int, N: int):
    return None if out is None else _tensor(out, "out", torch.float32, (M, N))


def _rows_of(t, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return t.shape[0]


def workspace_size(op: int, M: int = 0, N: int = 0, K: int = 0, bits: int = 4, group: int = 128,
                   n_grid: int = 20) -> int:
    out = _size_t(0)
    _check(lib().awq_workspace_size(op, M, N, K, bits, group, n_grid, ctypes.byref(out)),
           "awq_workspace_size")
    return int(out.value)


def _workspace(nbytes: int, device, workspace: torch.Tensor | None = None) -> torch.Tensor:
    if workspace is not None:
        _tensor(workspace, "workspace", torch.uint8)
        _gpu(workspace=workspace)
        if workspace.device == device and workspace.numel() >= nbytes:
            return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def act_stats(x: torch.Tensor) -> torch.Tensor:
    """mean |x| per input channel, float32 [K]."""
    x = _bf16(x, "x")
    M, K = x.shape
    dev = _gpu(x=x)
    out = torch.empty(K, dtype=torch.float32, device=dev)
    ws = _workspace(workspace_size(OP_ACT_STATS, M, 0, K), dev)
    _check(lib().awq_act_stats(_ptr(x), M, K, _ptr(out), _ptr(ws), ws.numel(), _stream(dev)),
           "awq_act_stats")
    return out


def candidate_scales(mean_abs: torch.Tensor, n_grid: int = 20):
    """(s, inv_s), each float32 [n_grid][K]."""
    mean_abs = _f32(mean_abs, "mean_abs")
    K = mean_abs.numel()
    dev = _gpu(mean_abs=mean_abs)
    s = torch.empty((n_grid, K), dtype=torch.float32, device=dev)
    inv = torch.empty_like(s)
    ws = _workspace(workspace_size(OP_CANDIDATE_SCALES, 0, 0, K, n_grid=n_grid), dev)
    _check(lib().awq_candidate_scales(_ptr(mean_abs), K, n_grid, _ptr(s), _ptr(inv), _ptr(ws),
                                      ws.numel(), _stream(dev)), "awq_candidate_scales")
    return s, inv


def quantize_pack(w: torch.Tensor, s: torch.Tensor | None = None, bits: int = 4, group: int = 128):
    """(qweight int32 [N][K/8] holding u32 words, scales float32 [N][K/g], zeros uint8 [N][K/g])."""
    w = _bf16(w, "w")
    N, K = w.shape
    s = _vec_f32(s, "s", K)
    dev = _gpu(w=w, s=s)
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    scales = torch.empty((N, K // group), dtype=torch.float32, device=dev)
    zeros = torch.empty((N, K // group), dtype=torch.uint8, device=dev)
    _check(lib().awq_quantize_pack(_ptr(w), N, K, _ptr(s), bits, group, _ptr(qweight), _ptr(scales),
                                   _ptr(zeros), _stream(dev)), "awq_quantize_pack")
    return qweight, scales, zeros


def reference_gemm(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """Y = X . W^T in fp32 [M][N] (bf16 operands, fp32 accumulation)."""
    x, w = _bf16(x, "x"), _bf16(w, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w disagree on K")
    dev = _gpu(x=x, w=w)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _check(lib().awq_reference_gemm(_ptr(x), M, N, K, _ptr(w), _ptr(y), _stream(dev)),
           "awq_reference_gemm")
    return y


LAYOUT_NIBBLE, LAYOUT_INT3_DENSE = 0, 1


def _packed_words(qweight, N: int, K: int, layout: int, name: str = "qweight"):
    """Row-major packed codes: [N][K/8] 4-bit containers or [N][3K/32] dense INT3."""
    if layout not in (LAYOUT_NIBBLE, LAYOUT_INT3_DENSE):
        raise ValueError(f"unknown layout {layout}")
    words = 3 * K // 32 if layout == LAYOUT_INT3_DENSE else K // 8
    return _tensor(qweight, name, _WORDS, (N, words))


def w4a16_gemm(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
               bits: int = 4, group: int = 128, inv_s: torch.Tensor | None = None,
               y_ref: torch.Tensor | None = None, return_y: bool = True,
               workspace: torch.Tensor | None = None, layout: int | None = None,
               staged: bool = False):
    """Y = X . dequant(Q)^T (fp32).  With y_ref also returns sse = sum (Y - y_ref)^2
    as a float64 [1] device tensor: returns (y or None, sse).

    layout LAYOUT_NIBBLE (default; qweight [N][K/8]) or LAYOUT_INT3_DENSE
    (bits 3, qweight [N][3K/32]).  staged=True runs awq_w4a16_gemm_staged
    (the operand dequantized once into the workspace, then the bf16
    matrix-core contraction: the same operand, Y equal to the fused kernel's
    up to fp32 rounding of the sums); otherwise the fused product,
    dequantized in LDS per tile: awq_w4a16_gemm, or awq_w3a16_gemm for the
    dense INT3 layout.  Either way dense INT3 gives the product of the same
    codes in 4-bit containers bit for bit."""
    x = _bf16(x, "x")
    M, K = x.shape
    layout = LAYOUT_NIBBLE if layout is None else layout
    N = _rows_of(qweight, "qweight")
    _packed_words(qweight, N, K, layout)
    if layout == LAYOUT_INT3_DENSE and bits != 3:
        raise ValueError("the dense INT3 layout holds 3-bit codes (bits=3)")
    _meta(scales, zeros, N, K, group)
    inv_s = _vec_f32(inv_s, "inv_s", K)
    if y_ref is not None:
        y_ref = _f32(y_ref, "y_ref", (M, N))
    elif not return_y:
        raise ValueError("return_y=False needs y_ref (nothing to compute)")
    dev = _gpu(x=x, qweight=qweight, scales=scales, zeros=zeros, inv_s=inv_s, y_ref=y_ref)
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if return_y else None
    sse = torch.empty(1, dtype=torch.float64, device=dev) if y_ref is not None else None
    if staged:
        ws = _workspace(workspace_size(OP_W4A16_GEMM_STAGED, M, N, K, bits, group), dev, workspace)
        _check(lib().awq_w4a16_gemm_staged(_ptr(x), M, N, K, _ptr(qweight), _ptr(scales),
                                           _ptr(zeros), bits, group, layout, _ptr(inv_s),
                                           _ptr(y_ref), _ptr(y), _ptr(sse), _ptr(ws), ws.numel(),
                                           _stream(dev)), "awq_w4a16_gemm_staged")
    else:
        ws = None
        if y_ref is not None:
            ws = _workspace(workspace_size(OP_W4A16_GEMM, M, N, K), dev, workspace)
        nws = 0 if ws is None else ws.numel()
        if layout == LAYOUT_INT3_DENSE:
            _check(lib().awq_w3a16_gemm(_ptr(x), M, N, K, _ptr(qweight), _ptr(scales),
                                        _ptr(zeros), group, _ptr(inv_s), _ptr(y_ref), _ptr(y),
                                        _ptr(sse), _ptr(ws), nws, _stream(dev)), "awq_w3a16_gemm")
        else:
            _check(lib().awq_w4a16_gemm(_ptr(x), M, N, K, _ptr(qweight), _ptr(scales),
                                        _ptr(zeros), bits, group, _ptr(inv_s), _ptr(y_ref),
                                        _ptr(y), _ptr(sse), _ptr(ws), nws, _stream(dev)),
                   "awq_w4a16_gemm")
    if y_ref is None:
        return y
    return y, sse


def dequant_operand(w: torch.Tensor, s: torch.Tensor | None, inv_s: torch.Tensor | None,
                    bits: int = 4, group: int = 128) -> torch.Tensor:
    """One candidate's bf16 weight operand bf16(f32(f32((q - z) * step) * inv_s[k]))."""
    w = _bf16(w, "w")
    N, K = w.shape
    s, inv_s = _vec_f32(s, "s", K), _vec_f32(inv_s, "inv_s", K)
    dev = _gpu(w=w, s=s, inv_s=inv_s)
    b = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    _check(lib().awq_dequant_operand(_ptr(w), N, K, _ptr(s), _ptr(inv_s), bits, group, _ptr(b),
                                     _stream(dev)), "awq_dequant_operand")
    return b


def diff_operand(w: torch.Tensor, s: torch.Tensor | None, inv_s: torch.Tensor | None,
                 bits: int = 4, group: int = 128) -> torch.Tensor:
    """One candidate's bf16 difference operand bf16(B - W) (B as dequant_operand writes it)."""
    w = _bf16(w, "w")
    N, K = w.shape
    s, inv_s = _vec_f32(s, "s", K), _vec_f32(inv_s, "inv_s", K)
    dev = _gpu(w=w, s=s, inv_s=inv_s)
    d = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    _check(lib().awq_diff_operand(_ptr(w), N, K, _ptr(s), _ptr(inv_s), bits, group, _ptr(d),
                                  _stream(dev)), "awq_diff_operand")
    return d


def candidate_sse(x: torch.Tensor, b: torch.Tensor, y_ref: torch.Tensor | None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """sum (X . B^T - y_ref)^2 (y_ref None: sum (X . B^T)^2) as a float64 [1]
    device tensor; the product is never stored."""
    x, b = _bf16(x, "x"), _bf16(b, "b")
    M, K = x.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("x and b disagree on K")
    if y_ref is not None:
        y_ref = _f32(y_ref, "y_ref", (M, N))
    dev = _gpu(x=x, b=b, y_ref=y_ref)
    sse = torch.empty(1, dtype=torch.float64, device=dev)
    ws = _workspace(workspace_size(OP_CANDIDATE_SSE, M, N, K), dev, workspace)
    _check(lib().awq_candidate_sse(_ptr(x), M, N, K, _ptr(b), _ptr(y_ref), _ptr(sse), _ptr(ws),
                                   ws.numel(), _stream(dev)), "awq_candidate_sse")
    return sse


def _decode_ws(M: int, N: int, K: int, bits: int, group: int, dev, workspace):
    need = workspace_size(OP_DECODE_GEMM, M, N, K, bits, group)
    return _workspace(need, dev, workspace) if need > 0 else None


def decode_gemm(a: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                bits: int = 4, group: int = 128, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = A . ((q - z) * step)^T for 1 <= M <= 64 tokens (fp32 [M][N])."""
    a = _bf16(a, "a")
    M, K = a.shape
    N = _rows_of(qweight, "qweight")
    _packed_words(qweight, N, K, LAYOUT_NIBBLE)
    _meta(scales, zeros, N, K, group)
    y = _out(out, M, N)
    dev = _gpu(a=a, qweight=qweight, scales=scales, zeros=zeros, out=y)
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else y
    ws = _decode_ws(M, N, K, bits, group, dev, workspace)
    _check(lib().awq_w4a16_decode_gemm(_ptr(a), M, N, K, _ptr(qweight), _ptr(scales), _ptr(zeros),
                                       bits, group, _ptr(y), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(dev)),
           "awq_w4a16_decode_gemm")
    return y


def quantize_pack3(w: torch.Tensor, s: torch.Tensor | None, group: int = 128):
    """Dense INT3 codes of W . diag(s): (qweight3 int32 [N][3K/32], scales f32, zeros u8)."""
    w = _bf16(w, "w")
    N, K = w.shape
    s = _vec_f32(s, "s", K)
    dev = _gpu(w=w, s=s)
    qw = torch.empty((N, 3 * K // 32), dtype=torch.int32, device=dev)
    sc = torch.empty((N, K // group), dtype=torch.float32, device=dev)
    ze = torch.empty((N, K // group), dtype=torch.uint8, device=dev)
    _check(lib().awq_quantize_pack3(_ptr(w), N, K, _ptr(s), group, _ptr(qw), _ptr(sc), _ptr(ze),
                                    _stream(dev)), "awq_quantize_pack3")
    return qw, sc, ze


def decode_gemm3(a: torch.Tensor, qweight3: torch.Tensor, scales: torch.Tensor,
                 zeros: torch.Tensor, group: int = 128, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = A . ((q - z) * step)^T from dense INT3 weights, 1 <= M <= 64 (fp32 [M][N])."""
    a = _bf16(a, "a")
    M, K = a.shape
    N = _rows_of(qweight3, "qweight3")
    _packed_words(qweight3, N, K, LAYOUT_INT3_DENSE, "qweight3")
    _meta(scales, zeros, N, K, group)
    y = _out(out, M, N)
    dev = _gpu(a=a, qweight3=qweight3, scales=scales, zeros=zeros, out=y)
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else y
    ws = _decode_ws(M, N, K, 3, group, dev, workspace)
    _check(lib().awq_w3a16_decode_gemm(_ptr(a), M, N, K, _ptr(qweight3), _ptr(scales), _ptr(zeros),
                                       group, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(dev)), "awq_w3a16_decode_gemm")
    return y


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5, return_r: bool = False):
    """u = bf16(f32(f32(x * r) * gamma)), r = f32(1/sqrt(mean x^2 + eps)) per token."""
    x = _bf16(x, "x")
    M, K = x.shape
    gamma = _f32(gamma, "gamma", (K,))
    dev = _gpu(x=x, gamma=gamma)
    u = torch.empty_like(x)
    r = torch.empty(M, dtype=torch.float32, device=dev) if return_r else None
    _check(lib().awq_rmsnorm(_ptr(x), M, K, _ptr(gamma), float(eps), _ptr(u), _ptr(r),
                             _stream(dev)), "awq_rmsnorm")
    return (u, r) if return_r else u


def silu_mul(y: torch.Tensor) -> torch.Tensor:
    """H = bf16(f32(silu(g) * v)) for y = [g | v] fp32 [M][2F]."""
    y = _f32(y, "y")
    if y.dim() != 2 or y.shape[1] % 2:
        raise ValueError("y must be [M][2F]")
    M, F2 = y.shape
    dev = _gpu(y=y)
    h = torch.empty((M, F2 // 2), dtype=torch.bfloat16, device=dev)
    _check(lib().awq_silu_mul(_ptr(y), M, F2 // 2, _ptr(h), _stream(dev)), "awq_silu_mul")
    return h


def divide_rows(v: torch.Tensor, s: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out[r][...] = f32(v[r][...] / s[r])."""
    v = _f32(v, "v")
    if v.dim() < 1:
        raise ValueError("v must have at least one dimension")
    R = v.shape[0]
    C = v.numel() // max(R, 1)
    s = _vec_f32(s, "s", R)
    if out is not None:
        _f32(out, "out", tuple(v.shape))
    dev = _gpu(v=v, s=s, out=out)
    out = torch.empty_like(v) if out is None else out
    _check(lib().awq_divide_rows(_ptr(v), R, C, _ptr(s), _ptr(out), _stream(dev)),
           "awq_divide_rows")
    return out


def residual_add(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """bf16(f32(x + y)) for bf16 x and fp32 y of the same shape [M][K]."""
    x = _bf16(x, "x")
    M, K = x.shape
    y = _f32(y, "y", (M, K))
    dev = _gpu(x=x, y=y)
    out = torch.empty_like(x)
    _check(lib().awq_residual_add(_ptr(x), _ptr(y), M, K, _ptr(out), _stream(dev)),
           "awq_residual_add")
    return out


def decode_tiles_size(N: int, K: int, layout: int = LAYOUT_NIBBLE, group: int = 128) -> int:
    """Bytes of the decode tiles of an N x K layer."""
    nbytes = _size_t(0)
    _check(lib().awq_decode_tiles_size(N, K, layout, group, ctypes.byref(nbytes)),
           "awq_decode_tiles_size")
    return int(nbytes.value)


def decode_tiles(qweight: torch.Tensor, K: int, layout: int = LAYOUT_NIBBLE,
                 group: int = 128) -> torch.Tensor:
    """The packed words as decode tiles (int32, flat), for decode_gemm_tiled."""
    N = _rows_of(qweight, "qweight")
    _packed_words(qweight, N, K, layout)
    nbytes = decode_tiles_size(N, K, layout, group)
    dev = _gpu(qweight=qweight)
    tiles = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    _check(lib().awq_decode_tiles(_ptr(qweight), N, K, layout, group, _ptr(tiles), _stream(dev)),
           "awq_decode_tiles")
    return tiles


def _tiles(tiles, N: int, K: int, layout: int, group: int):
    _tensor(tiles, "tiles", _WORDS)
    nbytes = decode_tiles_size(N, K, layout, group)
    if tiles.numel() * tiles.element_size() != nbytes:
        raise ValueError(f"tiles must hold {nbytes} bytes for an {N} x {K} layer in layout "
                         f"{layout} (got {tiles.numel() * tiles.element_size()})")
    return tiles


def decode_gemm_tiled(a: torch.Tensor, tiles: torch.Tensor, scales: torch.Tensor,
                      zeros: torch.Tensor, layout: int = LAYOUT_NIBBLE, group: int = 128,
                      out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode_gemm / decode_gemm3 reading decode tiles (fp32 [M][N])."""
    a = _bf16(a, "a")
    M, K = a.shape
    N = _rows_of(scales, "scales")
    _meta(scales, zeros, N, K, group)
    _tiles(tiles, N, K, layout, group)
    y = _out(out, M, N)
    dev = _gpu(a=a, tiles=tiles, scales=scales, zeros=zeros, out=y)
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else y
    ws = _decode_ws(M, N, K, 3 if layout == LAYOUT_INT3_DENSE else 4, group, dev, workspace)
    _check(lib().awq_decode_gemm_tiled(_ptr(a), M, N, K, _ptr(tiles), _ptr(scales), _ptr(zeros),
                                       layout, group, _ptr(y), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(dev)),
           "awq_decode_gemm_tiled")
    return y


def decode_gemm_tiled_noalloc(a: torch.Tensor, tiles: torch.Tensor, scales: torch.Tensor,
                              zeros: torch.Tensor, layout: int = LAYOUT_NIBBLE, group: int = 128,
                              out: torch.Tensor | None = None) -> torch.Tensor:
    """decode_gemm_tiled without a workspace: the K-split partials go to the
    library's static 16 MiB scratch (awq_decode_gemm_tiled_noalloc), so a
    call with `out` given allocates nothing.  Calls that overlap on one GPU
    race on that scratch."""
    a = _bf16(a, "a")
    M, K = a.shape
    N = _rows_of(scales, "scales")
    _meta(scales, zeros, N, K, group)
    _tiles(tiles, N, K, layout, group)
    y = _out(out, M, N)
    dev = _gpu(a=a, tiles=tiles, scales=scales, zeros=zeros, out=y)
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else y
    _check(lib().awq_decode_gemm_tiled_noalloc(_ptr(a), M, N, K, _ptr(tiles), _ptr(scales),
                                               _ptr(zeros), layout, group, _ptr(y), _stream(dev)),
           "awq_decode_gemm_tiled_noalloc")
    return y


def quantize_pack16(w: torch.Tensor, s: torch.Tensor | None, bits: int = 4, group: int = 128,
                    layout: int = LAYOUT_NIBBLE):
    """The compact deployment format of W . diag(s): (qweight int32, steps16
    float16 [N][K/group], zeros4 uint8 [N][ceil(G/2)], two zeros per byte).
    qweight is [N][K/8] (LAYOUT_NIBBLE) or [N][3K/32] (LAYOUT_INT3_DENSE, bits 3)."""
    w = _bf16(w, "w")
    N, K = w.shape
    s = _vec_f32(s, "s", K)
    dev = _gpu(w=w, s=s)
    G = K // group
    words = 3 * K // 32 if layout == LAYOUT_INT3_DENSE else K // 8
    qw = torch.empty((N, words), dtype=torch.int32, device=dev)
    st = torch.empty((N, G), dtype=torch.float16, device=dev)
    ze = torch.empty((N, (G + 1) // 2), dtype=torch.uint8, device=dev)
    _check(lib().awq_quantize_pack16(_ptr(w), N, K, _ptr(s), bits, group, layout, _ptr(qw),
                                     _ptr(st), _ptr(ze), _stream(dev)), "awq_quantize_pack16")
    return qw, st, ze


def _meta16(steps16, zeros4, N: int, G: int):
    _tensor(steps16, "steps16", torch.float16, (N, G))
    _tensor(zeros4, "zeros4", torch.uint8, (N, (G + 1) // 2))


def expand_meta16(steps16: torch.Tensor, zeros4: torch.Tensor, group: int = 128):
    """(scales f32 [N][G], zeros u8 [N][G]) from the compact metadata (exact)."""
    N = _rows_of(steps16, "steps16")
    G = steps16.shape[1]
    _meta16(steps16, zeros4, N, G)
    dev = _gpu(steps16=steps16, zeros4=zeros4)
    sc = torch.empty((N, G), dtype=torch.float32, device=dev)
    ze = torch.empty((N, G), dtype=torch.uint8, device=dev)
    _check(lib().awq_expand_meta16(_ptr(steps16), _ptr(zeros4), N, G * group, group,
                                   _ptr(sc), _ptr(ze), _stream(dev)), "awq_expand_meta16")
    return sc, ze


def decode_gemm_tiled16(a: torch.Tensor, tiles: torch.Tensor, steps16: torch.Tensor,
                        zeros4: torch.Tensor, layout: int = LAYOUT_NIBBLE, group: int = 128,
                        out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode_gemm_tiled with the compact metadata (fp32 [M][N])."""
    a = _bf16(a, "a")
    M, K = a.shape
    if group <= 0 or K % group:
        raise ValueError(f"K={K} must be a multiple of the group size {group}")
    N = _rows_of(steps16, "steps16")
    _meta16(steps16, zeros4, N, K // group)
    _tiles(tiles, N, K, layout, group)
    y = _out(out, M, N)
    dev = _gpu(a=a, tiles=tiles, steps16=steps16, zeros4=zeros4, out=y)
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else y
    ws = _decode_ws(M, N, K, 3 if layout == LAYOUT_INT3_DENSE else 4, group, dev, workspace)
    _check(lib().awq_decode_gemm_tiled16(_ptr(a), M, N, K, _ptr(tiles), _ptr(steps16),
                                         _ptr(zeros4), layout, group, _ptr(y),
                                         _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)),
           "awq_decode_gemm_tiled16")
    return y


def decode_meta_size(N: int, K: int, group: int = 128) -> int:
    """Bytes of the metadata tiles of an N x K layer."""
    nbytes = _size_t(0)
    _check(lib().awq_decode_meta_size(N, K, group, ctypes.byref(nbytes)), "awq_decode_meta_size")
    return int(nbytes.value)


def decode_meta(steps16: torch.Tensor, zeros4: torch.Tensor, group: int = 128) -> torch.Tensor:
    """The compact metadata as metadata tiles (int32, flat), for
    decode_gemm_tiled_meta."""
    N = _rows_of(steps16, "steps16")
    G = steps16.shape[1]
    _meta16(steps16, zeros4, N, G)
    dev = _gpu(steps16=steps16, zeros4=zeros4)
    meta = torch.empty(decode_meta_size(N, G * group, group) // 4, dtype=torch.int32, device=dev)
    _check(lib().awq_decode_meta(_ptr(steps16), _ptr(zeros4), N, G * group, group, _ptr(meta),
                                 _stream(dev)), "awq_decode_meta")
    return meta


def decode_gemm_tiled_meta(a: torch.Tensor, tiles: torch.Tensor, meta: torch.Tensor, N: int,
                           layout: int = LAYOUT_NIBBLE, group: int = 128,
                           out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode_gemm_tiled16 reading metadata tiles (fp32 [M][N]); N is the
    layer's output width (the tiles round it up to 16)."""
    a = _bf16(a, "a")
    M, K = a.shape
    if group <= 0 or K % group:
        raise ValueError(f"K={K} must be a multiple of the group size {group}")
    _tiles(tiles, N, K, layout, group)
    _tensor(meta, "meta", _WORDS, (decode_meta_size(N, K, group) // 4,))
    y = _out(out, M, N)
    dev = _gpu(a=a, tiles=tiles, meta=meta, out=y)
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if y is None else y
    ws = _decode_ws(M, N, K, 3 if layout == LAYOUT_INT3_DENSE else 4, group, dev, workspace)
    _check(lib().awq_decode_gemm_tiled_meta(_ptr(a), M, N, K, _ptr(tiles), _ptr(meta), layout,
                                            group, _ptr(y), _ptr(ws),
                                            0 if ws is None else ws.numel(), _stream(dev)),
           "awq_decode_gemm_tiled_meta")
    return y


def ceiling_mfma(sink: torch.Tensor, blocks: int, iters: int, zero: bool = False) -> int:
    """Launch the matrix-core ceiling kernel (awq_ceiling_mfma) on the
    current stream; returns the launch's flops.  sink: one float on the GPU."""
    _tensor(sink, "sink", torch.float32)
    if sink.numel() < 1:
        raise ValueError("sink must hold at least one float")
    dev = _gpu(sink=sink)
    flops = ctypes.c_int64(0)
    _check(lib().awq_ceiling_mfma(blocks, iters, int(bool(zero)), _ptr(sink), ctypes.byref(flops),
                                  _stream(dev)), "awq_ceiling_mfma")
    return int(flops.value)


def ceiling_stream(mode: int, src: torch.Tensor | None, dst: torch.Tensor, nbytes: int,
                   blocks: int = 4096) -> None:
    """Launch a streaming ceiling kernel (awq_ceiling_stream) over nbytes on
    the current stream with `blocks` workgroups: CEILING_COPY src -> dst,
    CEILING_READ src (dst a sink), CEILING_WRITE dst."""
    need_dst = 4 if mode == CEILING_READ else nbytes
    if dst.numel() * dst.element_size() < need_dst or not dst.is_contiguous():
        raise ValueError(f"dst must be a contiguous buffer of at least {need_dst} bytes")
    if mode != CEILING_WRITE and (src is None or src.numel() * src.element_size() < nbytes
                                  or not src.is_contiguous()):
        raise ValueError(f"src must be a contiguous buffer of at least {nbytes} bytes")
    dev = _gpu(src=src, dst=dst)
    _check(lib().awq_ceiling_stream(mode, _ptr(src), _ptr(dst), nbytes, blocks, _stream(dev)),
           "awq_ceiling_stream")


def _search_outputs(K: int, N: int, n_grid: int, group: int, dev) -> dict:
    return dict(
        mean_abs=torch.empty(K, dtype=torch.float32, device=dev),
        losses=torch.empty(n_grid, dtype=torch.float64, device=dev),
        best_idx=torch.empty(1, dtype=torch.int32, device=dev),
        best_s=torch.empty(K, dtype=torch.float32, device=dev),
        qweight=torch.empty((N, K // 8), dtype=torch.int32, device=dev),
        scales=torch.empty((N, K // group), dtype=torch.float32, device=dev),
        zeros=torch.empty((N, K // group), dtype=torch.uint8, device=dev),
    )


def _search_args(x, w):
    x, w = _bf16(x, "x"), _bf16(w, "w")
    if w.shape[1] != x.shape[1]:
        raise ValueError("x and w disagree on K")
    return x, w, _gpu(x=x, w=w)


def search_scale(x: torch.Tensor, w: torch.Tensor, bits: int = 4, group: int = 128,
                 n_grid: int = 20, workspace: torch.Tensor | None = None) -> dict:
    """The whole per-layer AWQ search; every output stays on the GPU."""
    x, w, dev = _search_args(x, w)
    M, K = x.shape
    N = w.shape[0]
    out = _search_outputs(K, N, n_grid, group, dev)
    ws = _workspace(workspace_size(OP_SEARCH_SCALE, M, N, K, bits, group, n_grid), dev, workspace)
    _check(lib().awq_search_scale(_ptr(x), M, K, _ptr(w), N, bits, group, n_grid,
                                  _ptr(out["mean_abs"]), _ptr(out["losses"]), _ptr(out["best_idx"]),
                                  _ptr(out["best_s"]), _ptr(out["qweight"]), _ptr(out["scales"]),
                                  _ptr(out["zeros"]), _ptr(ws), ws.numel(), _stream(dev)),
           "awq_search_scale")
    return out


def search_scale_gram(x: torch.Tensor, w: torch.Tensor, bits: int = 4, group: int = 128,
                      n_grid: int = 20, workspace: torch.Tensor | None = None) -> dict:
    """The per-layer search with Gram-form losses (pays when 2K < M); outputs as search_scale."""
    x, w, dev = _search_args(x, w)
    M, K = x.shape
    N = w.shape[0]
    out = _search_outputs(K, N, n_grid, group, dev)
    ws = _workspace(workspace_size(OP_SEARCH_SCALE_GRAM, M, N, K, bits, group, n_grid), dev,
                    workspace)
    _check(lib().awq_search_scale_gram(_ptr(x), M, K, _ptr(w), N, bits, group, n_grid,
                                       _ptr(out["mean_abs"]), _ptr(out["losses"]),
                                       _ptr(out["best_idx"]), _ptr(out["best_s"]),
                                       _ptr(out["qweight"]), _ptr(out["scales"]),
                                       _ptr(out["zeros"]), _ptr(ws), ws.numel(), _stream(dev)),
           "awq_search_scale_gram")
    return out


from .linear import W4A16Linear, fold_inverse_scale  # noqa: E402  (needs the names above)

__all__ += ["W4A16Linear", "fold_inverse_scale"]

from .pipeline import quantize_mlp_block, quantize_mlp_blocks  # noqa: E402

__all__ += ["quantize_mlp_block", "quantize_mlp_blocks"]
