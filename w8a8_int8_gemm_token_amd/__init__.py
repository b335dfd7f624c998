"""W8A8 INT8 linear layer for AMD MI355X (gfx950): Python binding of libq8.

A thin ctypes layer over the C ABI in ``include/q8.h``.  Every function takes
torch tensors that already live on the GPU, checks dtypes/shapes, and passes
raw device pointers and the current HIP stream to the library; all arithmetic
runs in the HIP kernels.  There is no CPU fallback: if ``libq8.so`` is not
built, importing works but the first call raises ``RuntimeError``.

Functions mirror the C entry points:
  q8_quant_per_token(x) -> (xq, scale_tok)
  q8_scaled_mm(xq, wq, scale_tok, scale_ch) -> y
  q8_scaled_mm_group128(xq, wq, scale_tok, scale_grp) -> y
  w8a16_mm(x, wq, scale_ch) -> y
  q8_quant_scaled_mm(x, wq, scale_ch) -> (y, xq, scale_tok)
  q8_mm_i32(a, b) -> int32 acc
  q8_quant_weight(w, group=None) -> (wq, scale)
  q8_smooth_fold(x, w, cap=16.0) -> (x', w', s)
  q8_rmsnorm_quant(x, gamma, eps, residual=None) -> (xq, scale_tok)
  q8_quant_per_group128(x) -> (xq, scale_grp)
  q8_scaled_mm_group128_act(xq, wq, scale_x, scale_w) -> y
  q8_quant_fp8_per_group128(x) -> (xq float8_e4m3fn, scale_grp)
  q8_quant_weight_fp8_block128(w) -> (wq float8_e4m3fn, scale_blk)
  q8_fp8_block_scaled_mm(xq, wq, scale_x, scale_w) -> y
  q8_workspace_bytes(M, N, K) -> bytes; q8_scaled_mm_ws, q8_quant_scaled_mm_ws,
  w8a16_mm_ws: the same with K split over a workspace (workspace=);
  q8_quant_scaled_mm_noalloc: the layer with the library's own workspace
  ..._f16 variants of the per-token and per-group quantizers, q8_scaled_mm,
  q8_quant_scaled_mm, q8_scaled_mm_group128_act and w8a16_mm (fp16 in / out)
Each also accepts preallocated outputs (``out=`` ...) so callers control
allocation; the library itself never allocates.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Q8Error", "lib_path", "load", "q8_quant_per_token", "q8_scaled_mm",
    "q8_scaled_mm_group128", "w8a16_mm", "q8_quant_scaled_mm", "q8_mm_i32",
    "q8_quant_weight", "q8_smooth_fold", "q8_rmsnorm_quant", "q8_quant_per_group128",
    "q8_scaled_mm_group128_act", "q8_quant_fp8_per_group128", "q8_quant_weight_fp8_block128",
    "q8_fp8_block_scaled_mm", "q8_quant_per_token_f16", "q8_scaled_mm_f16",
    "q8_quant_scaled_mm_f16", "q8_quant_per_group128_f16", "q8_scaled_mm_group128_act_f16",
    "w8a16_mm_f16", "q8_workspace_bytes", "q8_scaled_mm_ws", "q8_quant_scaled_mm_ws", "w8a16_mm_ws",
    "q8_quant_scaled_mm_noalloc", "q8_wait_timeouts", "NOALLOC_MAX_WORKSPACE", "EXPORTS", "MAX_K",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
MAX_K = 130944
NOALLOC_MAX_WORKSPACE = 32 << 20  # bytes of the allocation-free variant's own workspace
EXPORTS = (
    "q8_status_str", "q8_quant_per_token", "q8_scaled_mm",
    "q8_scaled_mm_group128", "w8a16_mm", "q8_quant_scaled_mm", "q8_mm_i32",
    "q8_quant_weight", "q8_smooth_fold", "q8_rmsnorm_quant", "q8_quant_per_group128",
    "q8_scaled_mm_group128_act", "q8_quant_fp8_per_group128", "q8_quant_weight_fp8_block128",
    "q8_fp8_block_scaled_mm", "q8_quant_per_token_f16", "q8_scaled_mm_f16",
    "q8_quant_scaled_mm_f16", "q8_quant_per_group128_f16", "q8_scaled_mm_group128_act_f16",
    "w8a16_mm_f16", "q8_workspace_bytes", "q8_scaled_mm_ws", "q8_quant_scaled_mm_ws", "w8a16_mm_ws",
    "q8_quant_scaled_mm_noalloc", "q8_wait_timeouts",
)
_STATUS = {0: "Q8_OK", 1: "Q8_EINVAL", 2: "Q8_EUNSUPPORTED", 3: "Q8_EHIP"}


class Q8Error(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn}: {_STATUS.get(code, code)} ({text})")
        self.code = code


def lib_path() -> str:
    return os.path.join(_HERE, "libq8.so")


_lib = None


def load():
    """Load libq8.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"libq8.so not found at {path}: build it first "
            "(python -m w8a8_int8_gemm_token_amd.build)")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    S = ctypes.c_int
    sig = {
        "q8_status_str": ([S], ctypes.c_char_p),
        "q8_quant_per_token": ([P, I, P, I, P, I, I, P], S),
        "q8_scaled_mm": ([P, I, P, I, P, P, P, I, I, I, I, P], S),
        "q8_scaled_mm_group128": ([P, I, P, I, P, P, P, I, I, I, I, P], S),
        "w8a16_mm": ([P, I, P, I, P, P, I, I, I, I, P], S),
        "q8_quant_scaled_mm": ([P, I, P, I, P, P, I, P, P, I, I, I, P], S),
        "q8_mm_i32": ([P, I, P, I, P, I, I, I, I, P], S),
        "q8_quant_weight": ([P, I, P, I, P, I, I, I, P], S),
        "q8_smooth_fold": ([P, I, P, I, P, P, I, P, I, I, I, I, F, P], S),
        "q8_rmsnorm_quant": ([P, I, P, I, P, F, P, I, P, I, I, P], S),
        "q8_quant_per_group128": ([P, I, P, I, P, I, I, P], S),
        "q8_scaled_mm_group128_act": ([P, I, P, I, P, P, P, I, I, I, I, P], S),
        "q8_quant_fp8_per_group128": ([P, I, P, I, P, I, I, P], S),
        "q8_quant_weight_fp8_block128": ([P, I, P, I, P, I, I, P], S),
        "q8_fp8_block_scaled_mm": ([P, I, P, I, P, P, P, I, I, I, I, P], S),
        "q8_quant_per_token_f16": ([P, I, P, I, P, I, I, P], S),
        "q8_scaled_mm_f16": ([P, I, P, I, P, P, P, I, I, I, I, P], S),
        "q8_quant_scaled_mm_f16": ([P, I, P, I, P, P, I, P, P, I, I, I, P], S),
        "q8_quant_per_group128_f16": ([P, I, P, I, P, I, I, P], S),
        "q8_scaled_mm_group128_act_f16": ([P, I, P, I, P, P, P, I, I, I, I, P], S),
        "w8a16_mm_f16": ([P, I, P, I, P, P, I, I, I, I, P], S),
        "q8_workspace_bytes": ([I, I, I], I),
        "q8_scaled_mm_ws": ([P, I, P, I, P, P, P, I, I, I, I, P, I, P], S),
        "q8_quant_scaled_mm_ws": ([P, I, P, I, P, P, I, P, P, I, I, I, P, I, P], S),
        "w8a16_mm_ws": ([P, I, P, I, P, P, I, I, I, I, P, I, P], S),
        "q8_quant_scaled_mm_noalloc": ([P, I, P, I, P, P, I, P, P, I, I, I, P], S),
        "q8_wait_timeouts": ([P, S], S),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(fn: str, code: int):
    if code != 0:
        raise Q8Error(fn, code, load().q8_status_str(code).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim}-D, got shape {tuple(t.shape)}")
    if ndim == 2 and t.stride(1) != 1:
        raise ValueError(f"{name}: rows must be contiguous (stride(1) == 1)")
    if ndim == 1 and t.numel() > 0 and t.stride(0) != 1:
        raise ValueError(f"{name}: must be contiguous")
    return t


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _quant_per_token(name, dtype, x, out, scale_out):
    _dev(x, dtype, "x", 2)
    M, K = x.shape
    xq = out if out is not None else torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = scale_out if scale_out is not None else torch.empty((M,), dtype=torch.float32, device=x.device)
    _dev(xq, torch.int8, "out", 2)
    _dev(s, torch.float32, "scale_out", 1)
    _check(name, getattr(load(), name)(
        _ptr(x), _ld(x), _ptr(xq), _ld(xq), _ptr(s), M, K, _stream(x.device)))
    return xq, s


def q8_quant_per_token(x: torch.Tensor, out=None, scale_out=None):
    """Per-token symmetric INT8: x bf16 [M,K] -> (xq int8 [M,K], scale fp32 [M])."""
    return _quant_per_token("q8_quant_per_token", torch.bfloat16, x, out, scale_out)


def q8_quant_per_token_f16(x: torch.Tensor, out=None, scale_out=None):
    """As q8_quant_per_token, on fp16 activations."""
    return _quant_per_token("q8_quant_per_token_f16", torch.float16, x, out, scale_out)


def _gemm_out(M, N, device, out, dtype=torch.bfloat16):
    c = out if out is not None else torch.empty((M, N), dtype=dtype, device=device)
    _dev(c, dtype, "out", 2)
    if tuple(c.shape) != (M, N):
        raise ValueError(f"out: expected shape {(M, N)}, got {tuple(c.shape)}")
    return c


def _mk(a, b, a_dtype=torch.int8, b_dtype=torch.int8):
    _dev(a, a_dtype, "a", 2)
    _dev(b, b_dtype, "b", 2)
    if a.shape[1] != b.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)} vs b {tuple(b.shape)}")
    return a.shape[0], b.shape[0], a.shape[1]


def _scaled_mm(name, out_dtype, a, b, scale_tok, scale_ch, out):
    M, N, K = _mk(a, b)
    _dev(scale_tok, torch.float32, "scale_tok", 1)
    _dev(scale_ch, torch.float32, "scale_ch", 1)
    if scale_tok.numel() != M or scale_ch.numel() != N:
        raise ValueError("scale sizes do not match M / N")
    c = _gemm_out(M, N, a.device, out, out_dtype)
    _check(name, getattr(load(), name)(
        _ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(scale_tok), _ptr(scale_ch),
        _ptr(c), _ld(c), M, N, K, _stream(a.device)))
    return c


def q8_scaled_mm(a, b, scale_tok, scale_ch, out=None):
    """bf16 [M,N] = ((float)(a @ b^T) * scale_tok[m]) * scale_ch[n]."""
    return _scaled_mm("q8_scaled_mm", torch.bfloat16, a, b, scale_tok, scale_ch, out)


def q8_scaled_mm_f16(a, b, scale_tok, scale_ch, out=None):
    """As q8_scaled_mm, with fp16 outputs."""
    return _scaled_mm("q8_scaled_mm_f16", torch.float16, a, b, scale_tok, scale_ch, out)


def q8_scaled_mm_group128(a, b, scale_tok, scale_grp, out=None):
    """Group-128 weight scales: scale_grp fp32 [N, K/128] (contiguous)."""
    M, N, K = _mk(a, b)
    _dev(scale_tok, torch.float32, "scale_tok", 1)
    _dev(scale_grp, torch.float32, "scale_grp", 2)
    if scale_tok.numel() != M or tuple(scale_grp.shape) != (N, K // 128) \
            or not scale_grp.is_contiguous():
        raise ValueError("scale_grp must be a contiguous [N, K/128] tensor")
    c = _gemm_out(M, N, a.device, out)
    _check("q8_scaled_mm_group128", load().q8_scaled_mm_group128(
        _ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(scale_tok), _ptr(scale_grp),
        _ptr(c), _ld(c), M, N, K, _stream(a.device)))
    return c


def _w8a16_mm(name, dtype, x, w, scale_ch, out):
    M, N, K = _mk(x, w, dtype)
    _dev(scale_ch, torch.float32, "scale_ch", 1)
    if scale_ch.numel() != N:
        raise ValueError("scale_ch size does not match N")
    c = _gemm_out(M, N, x.device, out, dtype)
    _check(name, getattr(load(), name)(
        _ptr(x), _ld(x), _ptr(w), _ld(w), _ptr(scale_ch), _ptr(c), _ld(c),
        M, N, K, _stream(x.device)))
    return c


def w8a16_mm(x, w, scale_ch, out=None):
    """bf16 [M,N] = scale_ch[n] * (x @ bf16(w)^T), fp32 accumulation."""
    return _w8a16_mm("w8a16_mm", torch.bfloat16, x, w, scale_ch, out)


def w8a16_mm_f16(x, w, scale_ch, out=None):
    """fp16 [M,N] = scale_ch[n] * (x @ fp16(w)^T), fp16 x, fp32 accumulation."""
    return _w8a16_mm("w8a16_mm_f16", torch.float16, x, w, scale_ch, out)


def q8_quant_scaled_mm(x, b, scale_ch, out=None, xq_out=None, scale_tok_out=None):
    """The whole W8A8 layer: per-token quant of x, then the scaled INT8 GEMM.
    Returns (y bf16 [M,N], xq int8 [M,K], scale_tok fp32 [M])."""
    return _quant_scaled_mm("q8_quant_scaled_mm", torch.bfloat16, x, b, scale_ch, out, xq_out,
                            scale_tok_out)


def q8_quant_scaled_mm_noalloc(x, b, scale_ch, out, xq_out, scale_tok_out):
    """As q8_quant_scaled_mm_ws with the library's own workspace: for callers
    that cannot allocate (all outputs are the caller's tensors; nothing is
    allocated here or in the library).  Returns (y, xq, scale_tok)."""
    return _quant_scaled_mm("q8_quant_scaled_mm_noalloc", torch.bfloat16, x, b, scale_ch, out, xq_out,
                            scale_tok_out)


def q8_quant_scaled_mm_f16(x, b, scale_ch, out=None, xq_out=None, scale_tok_out=None):
    """As q8_quant_scaled_mm, fp16 in and out."""
    return _quant_scaled_mm("q8_quant_scaled_mm_f16", torch.float16, x, b, scale_ch, out, xq_out,
                            scale_tok_out)


def _quant_scaled_mm(name, dtype, x, b, scale_ch, out, xq_out, scale_tok_out):
    M, N, K = _mk(x, b, dtype)
    _dev(scale_ch, torch.float32, "scale_ch", 1)
    if scale_ch.numel() != N:
        raise ValueError("scale_ch size does not match N")
    c = _gemm_out(M, N, x.device, out, dtype)
    xq = xq_out if xq_out is not None else torch.empty((M, K), dtype=torch.int8, device=x.device)
    st = scale_tok_out if scale_tok_out is not None else torch.empty((M,), dtype=torch.float32, device=x.device)
    _dev(xq, torch.int8, "xq_out", 2)
    if not xq.is_contiguous() or tuple(xq.shape) != (M, K):
        raise ValueError("xq_out must be a contiguous [M, K] tensor")
    _dev(st, torch.float32, "scale_tok_out", 1)
    _check(name, getattr(load(), name)(
        _ptr(x), _ld(x), _ptr(b), _ld(b), _ptr(scale_ch), _ptr(c), _ld(c),
        _ptr(xq), _ptr(st), M, N, K, _stream(x.device)))
    return c, xq, st


def q8_wait_timeouts(reset: bool = False) -> int:
    """Waits of the weight-streaming kernel that gave up on the current
    device since the library was loaded (0 in correct operation).
    Synchronizes the device."""
    n = ctypes.c_uint32(0)
    _check("q8_wait_timeouts", load().q8_wait_timeouts(ctypes.byref(n), int(bool(reset))))
    return int(n.value)


def q8_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes the _ws entry points need for an (M, N, K) problem
    (0 when they do not split K)."""
    return int(load().q8_workspace_bytes(int(M), int(N), int(K)))


def _workspace(M, N, K, device, workspace):
    """The caller's workspace (any contiguous GPU tensor) and its size in
    bytes, or one allocated with torch when the caller passes none."""
    need = q8_workspace_bytes(M, N, K)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty((need,), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous GPU tensor")
    return workspace, workspace.numel() * workspace.element_size()


def q8_scaled_mm_ws(a, b, scale_tok, scale_ch, out=None, workspace=None):
    """As q8_scaled_mm, splitting K over a workspace where that is faster
    (same bits as q8_scaled_mm)."""
    M, N, K = _mk(a, b)
    _dev(scale_tok, torch.float32, "scale_tok", 1)
    _dev(scale_ch, torch.float32, "scale_ch", 1)
    if scale_tok.numel() != M or scale_ch.numel() != N:
        raise ValueError("scale sizes do not match M / N")
    c = _gemm_out(M, N, a.device, out)
    ws, nb = _workspace(M, N, K, a.device, workspace)
    _check("q8_scaled_mm_ws", load().q8_scaled_mm_ws(
        _ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(scale_tok), _ptr(scale_ch),
        _ptr(c), _ld(c), M, N, K, _ptr(ws), nb, _stream(a.device)))
    return c


def q8_quant_scaled_mm_ws(x, b, scale_ch, out=None, xq_out=None, scale_tok_out=None, workspace=None):
    """As q8_quant_scaled_mm, splitting K over a workspace where that is
    faster.  Returns (y, xq, scale_tok)."""
    M, N, K = _mk(x, b, torch.bfloat16)
    _dev(scale_ch, torch.float32, "scale_ch", 1)
    if scale_ch.numel() != N:
        raise ValueError("scale_ch size does not match N")
    c = _gemm_out(M, N, x.device, out)
    xq = xq_out if xq_out is not None else torch.empty((M, K), dtype=torch.int8, device=x.device)
    st = scale_tok_out if scale_tok_out is not None else torch.empty((M,), dtype=torch.float32, device=x.device)
    _dev(xq, torch.int8, "xq_out", 2)
    if not xq.is_contiguous() or tuple(xq.shape) != (M, K):
        raise ValueError("xq_out must be a contiguous [M, K] tensor")
    _dev(st, torch.float32, "scale_tok_out", 1)
    ws, nb = _workspace(M, N, K, x.device, workspace)
    _check("q8_quant_scaled_mm_ws", load().q8_quant_scaled_mm_ws(
        _ptr(x), _ld(x), _ptr(b), _ld(b), _ptr(scale_ch), _ptr(c), _ld(c),
        _ptr(xq), _ptr(st), M, N, K, _ptr(ws), nb, _stream(x.device)))
    return c, xq, st


def w8a16_mm_ws(x, w, scale_ch, out=None, workspace=None):
    """As w8a16_mm, splitting K over a workspace where that is faster."""
    M, N, K = _mk(x, w, torch.bfloat16)
    _dev(scale_ch, torch.float32, "scale_ch", 1)
    if scale_ch.numel() != N:
        raise ValueError("scale_ch size does not match N")
    c = _gemm_out(M, N, x.device, out)
    ws, nb = _workspace(M, N, K, x.device, workspace)
    _check("w8a16_mm_ws", load().w8a16_mm_ws(
        _ptr(x), _ld(x), _ptr(w), _ld(w), _ptr(scale_ch), _ptr(c), _ld(c),
        M, N, K, _ptr(ws), nb, _stream(x.device)))
    return c


def q8_mm_i32(a, b, out=None):
    """Raw exact int32 [M,N] = a @ b^T (test hook for the INT8 mainloop)."""
    M, N, K = _mk(a, b)
    c = _gemm_out(M, N, a.device, out, torch.int32)
    _check("q8_mm_i32", load().q8_mm_i32(
        _ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(c), _ld(c), M, N, K,
        _stream(a.device)))
    return c


def q8_quant_weight(w, group=None, out=None, scale_out=None):
    """Symmetric INT8 weights: per channel (group=None) or per 128-group."""
    _dev(w, torch.float32, "w", 2)
    N, K = w.shape
    g = K if group is None else int(group)
    wq = out if out is not None else torch.empty((N, K), dtype=torch.int8, device=w.device)
    if scale_out is not None:
        s = scale_out
    elif group is None:
        s = torch.empty((N,), dtype=torch.float32, device=w.device)
    else:
        s = torch.empty((N, K // g if g else 0), dtype=torch.float32, device=w.device)
    _dev(wq, torch.int8, "out", 2)
    _check("q8_quant_weight", load().q8_quant_weight(
        _ptr(w), _ld(w), _ptr(wq), _ld(wq), _ptr(s), N, K, g, _stream(w.device)))
    return wq, s


def q8_smooth_fold(x, w, cap: float = 16.0, x_out=None, w_out=None, s_out=None):
    """Smoothing fold: s = min(cap, sqrt(colmax|x|)), x' = x/s, w' = w*s."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(w, torch.float32, "w", 2)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("K mismatch")
    xo = x_out if x_out is not None else torch.empty_like(x)
    wo = w_out if w_out is not None else torch.empty_like(w)
    s = s_out if s_out is not None else torch.empty((K,), dtype=torch.float32, device=x.device)
    _check("q8_smooth_fold", load().q8_smooth_fold(
        _ptr(x), _ld(x), _ptr(w), _ld(w), _ptr(s), _ptr(xo), _ld(xo), _ptr(wo),
        _ld(wo), M, N, K, ctypes.c_float(cap), _stream(x.device)))
    return xo, wo, s


def q8_rmsnorm_quant(x, gamma, eps: float, residual=None, out=None, scale_out=None):
    """Residual add (optional, in place on `residual`) + RMSNorm + per-token
    INT8 quant: returns (xq int8 [M,K], scale_tok fp32 [M])."""
    _dev(x, torch.bfloat16, "x", 2)
    _dev(gamma, torch.bfloat16, "gamma", 1)
    M, K = x.shape
    if gamma.numel() != K:
        raise ValueError("gamma must have K entries")
    if residual is not None:
        _dev(residual, torch.bfloat16, "residual", 2)
        if tuple(residual.shape) != (M, K):
            raise ValueError("residual shape must match x")
    xq = out if out is not None else torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = scale_out if scale_out is not None else torch.empty((M,), dtype=torch.float32, device=x.device)
    _dev(xq, torch.int8, "out", 2)
    _dev(s, torch.float32, "scale_out", 1)
    _check("q8_rmsnorm_quant", load().q8_rmsnorm_quant(
        _ptr(x), _ld(x), None if residual is None else _ptr(residual),
        0 if residual is None else _ld(residual), _ptr(gamma), ctypes.c_float(eps),
        _ptr(xq), _ld(xq), _ptr(s), M, K, _stream(x.device)))
    return xq, s


def q8_quant_per_group128(x, out=None, scale_out=None):
    """Per-token-per-128-group INT8: x bf16 [M,K] -> (xq int8 [M,K],
    scale fp32 [M, K/128])."""
    return _quant_per_group128("q8_quant_per_group128", torch.bfloat16, x, out, scale_out)


def q8_quant_per_group128_f16(x, out=None, scale_out=None):
    """As q8_quant_per_group128, on fp16 activations."""
    return _quant_per_group128("q8_quant_per_group128_f16", torch.float16, x, out, scale_out)


def _quant_per_group128(name, dtype, x, out, scale_out):
    _dev(x, dtype, "x", 2)
    M, K = x.shape
    xq = out if out is not None else torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = scale_out if scale_out is not None else torch.empty((M, K // 128), dtype=torch.float32,
                                                           device=x.device)
    _dev(xq, torch.int8, "out", 2)
    _dev(s, torch.float32, "scale_out", 2)
    if not s.is_contiguous():
        raise ValueError("scale_out must be contiguous")
    _check(name, getattr(load(), name)(
        _ptr(x), _ld(x), _ptr(xq), _ld(xq), _ptr(s), M, K, _stream(x.device)))
    return xq, s


def q8_scaled_mm_group128_act(a, b, scale_x, scale_w, out=None):
    """bf16 [M,N]: per 128-block fmaf((float)p_g, fl(s_x[m,g]*s_w[n,g]), acc)."""
    return _scaled_mm_group128_act("q8_scaled_mm_group128_act", torch.bfloat16, a, b, scale_x,
                                   scale_w, out)


def q8_scaled_mm_group128_act_f16(a, b, scale_x, scale_w, out=None):
    """As q8_scaled_mm_group128_act, with fp16 outputs."""
    return _scaled_mm_group128_act("q8_scaled_mm_group128_act_f16", torch.float16, a, b, scale_x,
                                   scale_w, out)


def _scaled_mm_group128_act(name, out_dtype, a, b, scale_x, scale_w, out):
    M, N, K = _mk(a, b)
    _dev(scale_x, torch.float32, "scale_x", 2)
    _dev(scale_w, torch.float32, "scale_w", 2)
    if tuple(scale_x.shape) != (M, K // 128) or tuple(scale_w.shape) != (N, K // 128):
        raise ValueError("block scale shapes must be [M, K/128] and [N, K/128]")
    if not scale_x.is_contiguous() or not scale_w.is_contiguous():
        raise ValueError("block scales must be contiguous")
    c = _gemm_out(M, N, a.device, out, out_dtype)
    _check(name, getattr(load(), name)(
        _ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(scale_x), _ptr(scale_w), _ptr(c), _ld(c),
        M, N, K, _stream(a.device)))
    return c


FP8 = torch.float8_e4m3fn


def q8_quant_fp8_per_group128(x, out=None, scale_out=None):
    """Per-token-per-128-group FP8: x bf16 [M,K] -> (xq float8_e4m3fn [M,K],
    scale fp32 [M, K/128]), scale = absmax/448."""
    _dev(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    xq = out if out is not None else torch.empty((M, K), dtype=FP8, device=x.device)
    s = scale_out if scale_out is not None else torch.empty((M, K // 128), dtype=torch.float32,
                                                           device=x.device)
    _dev(xq, FP8, "out", 2)
    _dev(s, torch.float32, "scale_out", 2)
    if not s.is_contiguous():
        raise ValueError("scale_out must be contiguous")
    _check("q8_quant_fp8_per_group128", load().q8_quant_fp8_per_group128(
        _ptr(x), _ld(x), _ptr(xq), _ld(xq), _ptr(s), M, K, _stream(x.device)))
    return xq, s


def q8_quant_weight_fp8_block128(w, out=None, scale_out=None):
    """FP8 [128,128] block weights: w fp32 [N,K] -> (wq float8_e4m3fn [N,K],
    scale fp32 [N/128, K/128])."""
    _dev(w, torch.float32, "w", 2)
    N, K = w.shape
    wq = out if out is not None else torch.empty((N, K), dtype=FP8, device=w.device)
    s = scale_out if scale_out is not None else torch.empty((N // 128, K // 128), dtype=torch.float32,
                                                           device=w.device)
    _dev(wq, FP8, "out", 2)
    _dev(s, torch.float32, "scale_out", 2)
    if not s.is_contiguous():
        raise ValueError("scale_out must be contiguous")
    _check("q8_quant_weight_fp8_block128", load().q8_quant_weight_fp8_block128(
        _ptr(w), _ld(w), _ptr(wq), _ld(wq), _ptr(s), N, K, _stream(w.device)))
    return wq, s


def q8_fp8_block_scaled_mm(a, b, scale_x, scale_w, out=None):
    """bf16 [M,N] = sum_g scale_x[m,g] * scale_w[n/128,g] * (a_g @ b_g^T) on
    FP8 matrix cores (fp32 block sums folded in ascending g)."""
    M, N, K = _mk(a, b, a_dtype=FP8, b_dtype=FP8)
    _dev(scale_x, torch.float32, "scale_x", 2)
    _dev(scale_w, torch.float32, "scale_w", 2)
    if tuple(scale_x.shape) != (M, K // 128) or tuple(scale_w.shape) != (N // 128, K // 128):
        raise ValueError("block scale shapes must be [M, K/128] and [N/128, K/128]")
    if not scale_x.is_contiguous() or not scale_w.is_contiguous():
        raise ValueError("block scales must be contiguous")
    c = _gemm_out(M, N, a.device, out)
    _check("q8_fp8_block_scaled_mm", load().q8_fp8_block_scaled_mm(
        _ptr(a), _ld(a), _ptr(b), _ld(b), _ptr(scale_x), _ptr(scale_w), _ptr(c), _ld(c),
        M, N, K, _stream(a.device)))
    return c
