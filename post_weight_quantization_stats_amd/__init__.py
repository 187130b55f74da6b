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
           "decode_tiles", "decode_gemm_tiled", "LAYOUT_NIBBLE", "LAYOUT_INT3_DENSE",
           "quantize_pack16", "expand_meta16", "decode_gemm_tiled16",
           "rmsnorm", "silu_mul", "divide_rows", "residual_add", "workspace_size",
           "OP_ACT_STATS", "OP_W4A16_GEMM", "OP_SEARCH_SCALE", "OP_CANDIDATE_SCALES",
           "OP_DECODE_GEMM", "OP_CANDIDATE_SSE", "OP_SEARCH_SCALE_GRAM"]

(OP_ACT_STATS, OP_W4A16_GEMM, OP_SEARCH_SCALE, OP_CANDIDATE_SCALES, OP_DECODE_GEMM,
 OP_CANDIDATE_SSE, OP_SEARCH_SCALE_GRAM) = 0, 1, 2, 3, 4, 5, 6

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
    "awq_quantize_pack16": ([_c_void_p, _i64, _i64, _c_void_p, _i32, _i32, _i32, _c_void_p,
                             _c_void_p, _c_void_p, _c_void_p], _i32),
    "awq_expand_meta16": ([_c_void_p, _c_void_p, _i64, _i64, _i32, _c_void_p, _c_void_p,
                           _c_void_p], _i32),
    "awq_decode_gemm_tiled16": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                 _i32, _i32, _c_void_p, _c_void_p, _size_t, _c_void_p], _i32),
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


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values (got {t.dtype})")
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")
    return t


def _f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 GPU tensor")
    return t


def workspace_size(op: int, M: int = 0, N: int = 0, K: int = 0, bits: int = 4, group: int = 128,
                   n_grid: int = 20) -> int:
    out = _size_t(0)
    _check(lib().awq_workspace_size(op, M, N, K, bits, group, n_grid, ctypes.byref(out)),
           "awq_workspace_size")
    return int(out.value)


def _workspace(nbytes: int, device, workspace: torch.Tensor | None = None) -> torch.Tensor:
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def act_stats(x: torch.Tensor) -> torch.Tensor:
    """mean |x| per input channel, float32 [K]."""
    x = _bf16(x, "x")
    M, K = x.shape
    out = torch.empty(K, dtype=torch.float32, device=x.device)
    ws = _workspace(workspace_size(OP_ACT_STATS, M, 0, K), x.device)
    _check(lib().awq_act_stats(_ptr(x), M, K, _ptr(out), _ptr(ws), ws.numel(), _stream(x.device)),
           "awq_act_stats")
    return out


def candidate_scales(mean_abs: torch.Tensor, n_grid: int = 20):
    """(s, inv_s), each float32 [n_grid][K]."""
    mean_abs = _f32(mean_abs, "mean_abs")
    K = mean_abs.numel()
    s = torch.empty((n_grid, K), dtype=torch.float32, device=mean_abs.device)
    inv = torch.empty_like(s)
    ws = _workspace(workspace_size(OP_CANDIDATE_SCALES, 0, 0, K, n_grid=n_grid), mean_abs.device)
    _check(lib().awq_candidate_scales(_ptr(mean_abs), K, n_grid, _ptr(s), _ptr(inv), _ptr(ws),
                                      ws.numel(), _stream(mean_abs.device)), "awq_candidate_scales")
    return s, inv


def quantize_pack(w: torch.Tensor, s: torch.Tensor | None = None, bits: int = 4, group: int = 128):
    """(qweight int32 [N][K/8] holding u32 words, scales float32 [N][K/g], zeros uint8 [N][K/g])."""
    w = _bf16(w, "w")
    N, K = w.shape
    if s is not None:
        s = _f32(s, "s")
        if s.numel() != K:
            raise ValueError("s must have K elements")
    dev = w.device
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
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().awq_reference_gemm(_ptr(x), M, N, K, _ptr(w), _ptr(y), _stream(x.device)),
           "awq_reference_gemm")
    return y


def w4a16_gemm(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
               bits: int = 4, group: int = 128, inv_s: torch.Tensor | None = None,
               y_ref: torch.Tensor | None = None, return_y: bool = True,
               workspace: torch.Tensor | None = None):
    """Y = X . dequant(Q)^T (fp32).  With y_ref also returns sse = sum (Y - y_ref)^2
    as a float64 [1] device tensor: returns (y or None, sse)."""
    x = _bf16(x, "x")
    M, K = x.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 8 != K:
        raise ValueError("qweight must be [N][K/8]")
    dev = x.device
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if return_y else None
    sse = None
    ws = None
    if y_ref is not None:
        y_ref = _f32(y_ref, "y_ref")
        sse = torch.empty(1, dtype=torch.float64, device=dev)
        ws = _workspace(workspace_size(OP_W4A16_GEMM, M, N, K), dev, workspace)
    if inv_s is not None:
        inv_s = _f32(inv_s, "inv_s")
    _check(lib().awq_w4a16_gemm(_ptr(x), M, N, K, _ptr(qweight), _ptr(scales), _ptr(zeros), bits,
                                group, _ptr(inv_s), _ptr(y_ref), _ptr(y), _ptr(sse), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(dev)), "awq_w4a16_gemm")
    if y_ref is None:
        return y
    return y, sse


def dequant_operand(w: torch.Tensor, s: torch.Tensor | None, inv_s: torch.Tensor | None,
                    bits: int = 4, group: int = 128) -> torch.Tensor:
    """One candidate's bf16 weight operand bf16(f32(f32((q - z) * step) * inv_s[k]))."""
    w = _bf16(w, "w")
    N, K = w.shape
    if s is not None:
        s = _f32(s, "s")
    if inv_s is not None:
        inv_s = _f32(inv_s, "inv_s")
    b = torch.empty((N, K), dtype=torch.bfloat16, device=w.device)
    _check(lib().awq_dequant_operand(_ptr(w), N, K, _ptr(s), _ptr(inv_s), bits, group, _ptr(b),
                                     _stream(w.device)), "awq_dequant_operand")
    return b


def diff_operand(w: torch.Tensor, s: torch.Tensor | None, inv_s: torch.Tensor | None,
                 bits: int = 4, group: int = 128) -> torch.Tensor:
    """One candidate's bf16 difference operand bf16(B - W) (B as dequant_operand writes it)."""
    w = _bf16(w, "w")
    N, K = w.shape
    if s is not None:
        s = _f32(s, "s")
    if inv_s is not None:
        inv_s = _f32(inv_s, "inv_s")
    d = torch.empty((N, K), dtype=torch.bfloat16, device=w.device)
    _check(lib().awq_diff_operand(_ptr(w), N, K, _ptr(s), _ptr(inv_s), bits, group, _ptr(d),
                                  _stream(w.device)), "awq_diff_operand")
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
        y_ref = _f32(y_ref, "y_ref")
        if tuple(y_ref.shape) != (M, N):
            raise ValueError("y_ref must be [M][N]")
    sse = torch.empty(1, dtype=torch.float64, device=x.device)
    ws = _workspace(workspace_size(OP_CANDIDATE_SSE, M, N, K), x.device, workspace)
    _check(lib().awq_candidate_sse(_ptr(x), M, N, K, _ptr(b), _ptr(y_ref), _ptr(sse), _ptr(ws),
                                   ws.numel(), _stream(x.device)), "awq_candidate_sse")
    return sse


def decode_gemm(a: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                bits: int = 4, group: int = 128, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = A . ((q - z) * step)^T for 1 <= M <= 64 tokens (fp32 [M][N])."""
    a = _bf16(a, "a")
    M, K = a.shape
    N = qweight.shape[0]
    if qweight.shape[1] * 8 != K:
        raise ValueError("qweight must be [N][K/8]")
    dev = a.device
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if out is None else _f32(out, "out")
    need = workspace_size(OP_DECODE_GEMM, M, N, K, bits, group)
    ws = _workspace(need, dev, workspace) if need > 0 else None
    _check(lib().awq_w4a16_decode_gemm(_ptr(a), M, N, K, _ptr(qweight), _ptr(scales), _ptr(zeros),
                                       bits, group, _ptr(y), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(dev)),
           "awq_w4a16_decode_gemm")
    return y


def quantize_pack3(w: torch.Tensor, s: torch.Tensor | None, group: int = 128):
    """Dense INT3 codes of W . diag(s): (qweight3 int32 [N][3K/32], scales f32, zeros u8)."""
    w = _bf16(w, "w")
    N, K = w.shape
    if s is not None:
        s = _f32(s, "s")
    dev = w.device
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
    N = qweight3.shape[0]
    if qweight3.shape[1] * 32 != 3 * K:
        raise ValueError("qweight3 must be [N][3K/32]")
    dev = a.device
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if out is None else _f32(out, "out")
    need = workspace_size(OP_DECODE_GEMM, M, N, K, 3, group)
    ws = _workspace(need, dev, workspace) if need > 0 else None
    _check(lib().awq_w3a16_decode_gemm(_ptr(a), M, N, K, _ptr(qweight3), _ptr(scales), _ptr(zeros),
                                       group, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(dev)), "awq_w3a16_decode_gemm")
    return y


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5, return_r: bool = False):
    """u = bf16(f32(f32(x * r) * gamma)), r = f32(1/sqrt(mean x^2 + eps)) per token."""
    x, gamma = _bf16(x, "x"), _f32(gamma, "gamma")
    M, K = x.shape
    u = torch.empty_like(x)
    r = torch.empty(M, dtype=torch.float32, device=x.device) if return_r else None
    _check(lib().awq_rmsnorm(_ptr(x), M, K, _ptr(gamma), float(eps), _ptr(u), _ptr(r),
                             _stream(x.device)), "awq_rmsnorm")
    return (u, r) if return_r else u


def silu_mul(y: torch.Tensor) -> torch.Tensor:
    """H = bf16(f32(silu(g) * v)) for y = [g | v] fp32 [M][2F]."""
    y = _f32(y, "y")
    M, F2 = y.shape
    h = torch.empty((M, F2 // 2), dtype=torch.bfloat16, device=y.device)
    _check(lib().awq_silu_mul(_ptr(y), M, F2 // 2, _ptr(h), _stream(y.device)), "awq_silu_mul")
    return h


def divide_rows(v: torch.Tensor, s: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out[r][...] = f32(v[r][...] / s[r])."""
    v, s = _f32(v, "v"), _f32(s, "s")
    R = v.shape[0]
    C = v.numel() // max(R, 1)
    out = torch.empty_like(v) if out is None else _f32(out, "out")
    _check(lib().awq_divide_rows(_ptr(v), R, C, _ptr(s), _ptr(out), _stream(v.device)),
           "awq_divide_rows")
    return out


def residual_add(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """bf16(f32(x + y)) for bf16 x and fp32 y of the same shape [M][K]."""
    x, y = _bf16(x, "x"), _f32(y, "y")
    M, K = x.shape
    out = torch.empty_like(x)
    _check(lib().awq_residual_add(_ptr(x), _ptr(y), M, K, _ptr(out), _stream(x.device)),
           "awq_residual_add")
    return out


LAYOUT_NIBBLE, LAYOUT_INT3_DENSE = 0, 1


def decode_tiles(qweight: torch.Tensor, K: int, layout: int = LAYOUT_NIBBLE,
                 group: int = 128) -> torch.Tensor:
    """The packed words as decode tiles (int32, flat), for decode_gemm_tiled."""
    N = qweight.shape[0]
    nbytes = _size_t(0)
    _check(lib().awq_decode_tiles_size(N, K, layout, group, ctypes.byref(nbytes)),
           "awq_decode_tiles_size")
    tiles = torch.empty(nbytes.value // 4, dtype=torch.int32, device=qweight.device)
    _check(lib().awq_decode_tiles(_ptr(qweight.contiguous()), N, K, layout, group, _ptr(tiles),
                                  _stream(qweight.device)), "awq_decode_tiles")
    return tiles


def decode_gemm_tiled(a: torch.Tensor, tiles: torch.Tensor, scales: torch.Tensor,
                      zeros: torch.Tensor, layout: int = LAYOUT_NIBBLE, group: int = 128,
                      out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode_gemm / decode_gemm3 reading decode tiles (fp32 [M][N])."""
    a = _bf16(a, "a")
    M, K = a.shape
    N = scales.shape[0]
    dev = a.device
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if out is None else _f32(out, "out")
    need = workspace_size(OP_DECODE_GEMM, M, N, K, 3 if layout == LAYOUT_INT3_DENSE else 4, group)
    ws = _workspace(need, dev, workspace) if need > 0 else None
    _check(lib().awq_decode_gemm_tiled(_ptr(a), M, N, K, _ptr(tiles), _ptr(scales), _ptr(zeros),
                                       layout, group, _ptr(y), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(dev)),
           "awq_decode_gemm_tiled")
    return y


def quantize_pack16(w: torch.Tensor, s: torch.Tensor | None, bits: int = 4, group: int = 128,
                    layout: int = LAYOUT_NIBBLE):
    """The compact deployment format of W . diag(s): (qweight int32, steps16
    float16 [N][K/group], zeros4 uint8 [N][ceil(G/2)], two zeros per byte).
    qweight is [N][K/8] (LAYOUT_NIBBLE) or [N][3K/32] (LAYOUT_INT3_DENSE, bits 3)."""
    w = _bf16(w, "w")
    N, K = w.shape
    if s is not None:
        s = _f32(s, "s")
    dev = w.device
    G = K // group
    words = 3 * K // 32 if layout == LAYOUT_INT3_DENSE else K // 8
    qw = torch.empty((N, words), dtype=torch.int32, device=dev)
    st = torch.empty((N, G), dtype=torch.float16, device=dev)
    ze = torch.empty((N, (G + 1) // 2), dtype=torch.uint8, device=dev)
    _check(lib().awq_quantize_pack16(_ptr(w), N, K, _ptr(s), bits, group, layout, _ptr(qw),
                                     _ptr(st), _ptr(ze), _stream(dev)), "awq_quantize_pack16")
    return qw, st, ze


def _f16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.float16:
        raise ValueError(f"{name} must be float16 (binary16 steps)")
    return t.contiguous()


def expand_meta16(steps16: torch.Tensor, zeros4: torch.Tensor, group: int = 128):
    """(scales f32 [N][G], zeros u8 [N][G]) from the compact metadata (exact)."""
    steps16 = _f16(steps16, "steps16")
    N, G = steps16.shape
    if zeros4.dtype != torch.uint8 or tuple(zeros4.shape) != (N, (G + 1) // 2):
        raise ValueError("zeros4 must be uint8 [N][ceil(G/2)]")
    dev = steps16.device
    sc = torch.empty((N, G), dtype=torch.float32, device=dev)
    ze = torch.empty((N, G), dtype=torch.uint8, device=dev)
    _check(lib().awq_expand_meta16(_ptr(steps16), _ptr(zeros4.contiguous()), N, G * group, group,
                                   _ptr(sc), _ptr(ze), _stream(dev)), "awq_expand_meta16")
    return sc, ze


def decode_gemm_tiled16(a: torch.Tensor, tiles: torch.Tensor, steps16: torch.Tensor,
                        zeros4: torch.Tensor, layout: int = LAYOUT_NIBBLE, group: int = 128,
                        out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode_gemm_tiled with the compact metadata (fp32 [M][N])."""
    a = _bf16(a, "a")
    M, K = a.shape
    steps16 = _f16(steps16, "steps16")
    N, G = steps16.shape
    if G * group != K:
        raise ValueError("steps16 must be [N][K/group]")
    if zeros4.dtype != torch.uint8 or tuple(zeros4.shape) != (N, (G + 1) // 2):
        raise ValueError("zeros4 must be uint8 [N][ceil(G/2)]")
    dev = a.device
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if out is None else _f32(out, "out")
    need = workspace_size(OP_DECODE_GEMM, M, N, K, 3 if layout == LAYOUT_INT3_DENSE else 4, group)
    ws = _workspace(need, dev, workspace) if need > 0 else None
    _check(lib().awq_decode_gemm_tiled16(_ptr(a), M, N, K, _ptr(tiles), _ptr(steps16),
                                         _ptr(zeros4.contiguous()), layout, group, _ptr(y),
                                         _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)),
           "awq_decode_gemm_tiled16")
    return y


def search_scale(x: torch.Tensor, w: torch.Tensor, bits: int = 4, group: int = 128,
                 n_grid: int = 20, workspace: torch.Tensor | None = None) -> dict:
    """The whole per-layer AWQ search; every output stays on the GPU."""
    x, w = _bf16(x, "x"), _bf16(w, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w disagree on K")
    dev = x.device
    out = dict(
        mean_abs=torch.empty(K, dtype=torch.float32, device=dev),
        losses=torch.empty(n_grid, dtype=torch.float64, device=dev),
        best_idx=torch.empty(1, dtype=torch.int32, device=dev),
        best_s=torch.empty(K, dtype=torch.float32, device=dev),
        qweight=torch.empty((N, K // 8), dtype=torch.int32, device=dev),
        scales=torch.empty((N, K // group), dtype=torch.float32, device=dev),
        zeros=torch.empty((N, K // group), dtype=torch.uint8, device=dev),
    )
    ws = _workspace(workspace_size(OP_SEARCH_SCALE, M, N, K, bits, group, n_grid), dev, workspace)
    _check(lib().awq_search_scale(_ptr(x), M, K, _ptr(w), N, bits, group, n_grid,
                                  _ptr(out["mean_abs"]), _ptr(out["losses"]), _ptr(out["best_idx"]),
                                  _ptr(out["best_s"]), _ptr(out["qweight"]), _ptr(out["scales"]),
                                  _ptr(out["zeros"]), _ptr(ws), ws.numel(), _stream(dev)),
           "awq_search_scale")
    return out


def search_scale_gram(x: torch.Tensor, w: torch.Tensor, bits: int = 4, group: int = 128,
                      n_grid: int = 20, workspace: torch.Tensor | None = None) -> dict:
    """The per-layer search with Gram-form losses (pays when 3K < M); outputs as search_scale."""
    x, w = _bf16(x, "x"), _bf16(w, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w disagree on K")
    dev = x.device
    out = dict(
        mean_abs=torch.empty(K, dtype=torch.float32, device=dev),
        losses=torch.empty(n_grid, dtype=torch.float64, device=dev),
        best_idx=torch.empty(1, dtype=torch.int32, device=dev),
        best_s=torch.empty(K, dtype=torch.float32, device=dev),
        qweight=torch.empty((N, K // 8), dtype=torch.int32, device=dev),
        scales=torch.empty((N, K // group), dtype=torch.float32, device=dev),
        zeros=torch.empty((N, K // group), dtype=torch.uint8, device=dev),
    )
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
