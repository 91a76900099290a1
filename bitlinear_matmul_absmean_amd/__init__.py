"""Python binding of the MI355X BitNet b1.58 BitLinear library (W1.58A8).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libbitlinear.so`` behind the C ABI of ``include/bitlinear.h``.  PyTorch provides device
memory (tensors) and the current HIP stream; nothing here computes on the host.  If the
library has not been built, importing this package raises -- there is no fallback.

The functions carry the C names.  ``lib`` exposes the raw C entry points (ctypes) for
callers that manage pointers themselves.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbitlinear.so")

BITLINEAR_OK = 0
BITLINEAR_ERR_INVALID_ARG = -1
BITLINEAR_ERR_SHAPE = -2
BITLINEAR_ERR_ALIGNMENT = -3
BITLINEAR_ERR_WORKSPACE = -4
BITLINEAR_ERR_HIP = -5
BITLINEAR_ERR_SCRATCH = -6
BITLINEAR_MAX_K = 16909320

# Every symbol the header declares, with (restype, argtypes).
_P, _I64, _SZ, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "bitlinear_abi_version": (_INT, []),
    "bitlinear_status_string": (ctypes.c_char_p, [_INT]),
    "bitlinear_last_hip_error": (_INT, []),
    "bitlinear_quantize_weights_workspace_size": (_SZ, [_I64, _I64]),
    "bitlinear_quantize_weights": (_INT, [_P, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "bitlinear_quantize_weights_noalloc": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "bitlinear_quantize_weights_noalloc_max_rows": (_SZ, []),
    "bitlinear_quantize_weights_rows": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "bitlinear_quantize_act": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "bitlinear_forward": (_INT, [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P]),
    "bitlinear_forward_rows": (_INT, [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P]),
    "bitlinear_forward_kernel": (ctypes.c_char_p, [_I64, _I64, _I64, _P, _P]),
    "bitlinear_forward_fused": (_INT, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _P, _P]),
    "bitlinear_forward_fused_rows": (_INT, [_P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _P, _P]),
    "bitlinear_forward_fused_kernel": (ctypes.c_char_p, [_I64, _I64, _I64, _P, _P, _P]),
    "bitlinear_t5_row_bytes": (_SZ, [_I64]),
    "bitlinear_quantize_weights_t5": (_INT, [_P, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "bitlinear_forward_t5": (_INT, [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P]),
    "bitlinear_repack_t5": (_INT, [_P, _I64, _I64, _P, _P]),
    "bitlinear_quantize_weights_blocks": (_INT, [_P, _I64, _I64, _P, _P, _P]),
    "bitlinear_forward_blocks": (_INT, [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P]),
    "bitlinear_mlp_forward": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bitlinear_hadamard_rows": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "bitlinear_quantize_act_hadamard": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "bitlinear_forward_fused_hadamard": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _P, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m bitlinear_matmul_absmean_amd.build` "
            "(hipcc --offload-arch=gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class BitLinearError(RuntimeError):
    def __init__(self, what: str, status: int):
        msg = lib.bitlinear_status_string(status).decode()
        if status == BITLINEAR_ERR_HIP:
            msg += f" (hipError {lib.bitlinear_last_hip_error()})"
        super().__init__(f"{what}: {msg} [status {status}]")
        self.status = status


def _check(what: str, status: int):
    if status != BITLINEAR_OK:
        raise BitLinearError(what, status)


def abi_version() -> int:
    return lib.bitlinear_abi_version()


# ------------------------------------------------------------------ torch marshalling
def _torch():
    import torch  # imported lazily: the C entry points above need no torch
    return torch


def _dev(t, dtype, name, numel=None):
    """Device pointer of t after checking device, dtype, layout and (numel) the minimum number of
    elements the library reads or writes through it."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _stream(stream):
    """Raw HIP stream handle: `stream`, else torch's current stream on the current device (the
    capture stream inside torch.cuda.graph).  The raw accessor skips building a Stream object,
    a few microseconds of host time per call."""
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def bitlinear_quantize_weights(W, W_packed=None, alpha=None, workspace=None, stream=None):
    """W [N, K] fp32 -> (W_packed uint8 [N, K/4], alpha fp32 [1]) on the device."""
    torch = _torch()
    N, K = W.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=W.device)
    need = lib.bitlinear_quantize_weights_workspace_size(N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=W.device)
    _check("bitlinear_quantize_weights", lib.bitlinear_quantize_weights(
        _dev(W, torch.float32, "W", N * K), N, K, _dev(W_packed, torch.uint8, "W_packed", N * (K // 4)),
        _dev(alpha, torch.float32, "alpha", 1), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream)))
    return W_packed, alpha


def bitlinear_quantize_weights_noalloc(W, W_packed, alpha, stream=None):
    """bitlinear_quantize_weights into caller buffers W_packed uint8 [N, K/4] and alpha fp32 [1],
    without a workspace: the library uses its fixed per-device scratch and allocates nothing
    (neither does this wrapper).  Calls that overlap on one device race."""
    torch = _torch()
    N, K = W.shape
    _check("bitlinear_quantize_weights_noalloc", lib.bitlinear_quantize_weights_noalloc(
        _dev(W, torch.float32, "W", N * K), N, K, _dev(W_packed, torch.uint8, "W_packed", N * (K // 4)),
        _dev(alpha, torch.float32, "alpha", 1), _stream(stream)))
    return W_packed, alpha


def bitlinear_quantize_weights_rows(W, W_packed=None, alpha_rows=None, stream=None):
    """W [N, K] fp32 -> (W_packed uint8 [N, K/4], alpha_rows fp32 [N])."""
    torch = _torch()
    N, K = W.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if alpha_rows is None:
        alpha_rows = torch.empty(N, dtype=torch.float32, device=W.device)
    _check("bitlinear_quantize_weights_rows", lib.bitlinear_quantize_weights_rows(
        _dev(W, torch.float32, "W", N * K), N, K, _dev(W_packed, torch.uint8, "W_packed", N * (K // 4)),
        _dev(alpha_rows, torch.float32, "alpha_rows", N), _stream(stream)))
    return W_packed, alpha_rows


def bitlinear_quantize_act(x, x_q=None, beta=None, stream=None):
    """x [M, K] fp32 -> (x_q int8 [M, K], beta fp32 [M])."""
    torch = _torch()
    M, K = x.shape
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if beta is None:
        beta = torch.empty(M, dtype=torch.float32, device=x.device)
    _check("bitlinear_quantize_act", lib.bitlinear_quantize_act(
        _dev(x, torch.float32, "x", M * K), M, K, _dev(x_q, torch.int8, "x_q", M * K),
        _dev(beta, torch.float32, "beta", M), _stream(stream)))
    return x_q, beta


def bitlinear_quantize_weights_t5(W, W_t5=None, alpha=None, workspace=None, stream=None):
    """W [N, K] fp32 -> (W_t5 uint8 [N, 16 ceil(K/80)], alpha fp32 [1]): five codes per byte."""
    torch = _torch()
    N, K = W.shape
    rb = lib.bitlinear_t5_row_bytes(K)
    if W_t5 is None:
        W_t5 = torch.empty((N, rb), dtype=torch.uint8, device=W.device)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=W.device)
    need = lib.bitlinear_quantize_weights_workspace_size(N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=W.device)
    _check("bitlinear_quantize_weights_t5", lib.bitlinear_quantize_weights_t5(
        _dev(W, torch.float32, "W", N * K), N, K, _dev(W_t5, torch.uint8, "W_t5", N * rb),
        _dev(alpha, torch.float32, "alpha", 1),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return W_t5, alpha


def bitlinear_repack_t5(W_packed, K, W_t5=None, stream=None):
    """2-bit packed [N, K/4] -> five codes per byte [N, 16 ceil(K/80)] (same codes)."""
    torch = _torch()
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    if W_t5 is None:
        W_t5 = torch.empty((N, lib.bitlinear_t5_row_bytes(K)), dtype=torch.uint8, device=W_packed.device)
    _check("bitlinear_repack_t5", lib.bitlinear_repack_t5(
        _dev(W_packed, torch.uint8, "W_packed"), N, K,
        _dev(W_t5, torch.uint8, "W_t5", N * lib.bitlinear_t5_row_bytes(K)), _stream(stream)))
    return W_t5


def bitlinear_forward_t5(x_q, beta, W_t5, alpha, bias=None, y=None, stream=None):
    """y [M, N] from x_q, beta and 5-trit packed weights."""
    torch = _torch()
    M, K = x_q.shape
    N = W_t5.shape[0]
    if W_t5.shape[1] != lib.bitlinear_t5_row_bytes(K):
        raise ValueError("W_t5 must be [N, bitlinear_t5_row_bytes(K)]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x_q.device)
    _check("bitlinear_forward_t5", lib.bitlinear_forward_t5(
        _dev(x_q, torch.int8, "x_q"), _dev(beta, torch.float32, "beta", M), M, K, _dev(W_t5, torch.uint8, "W_t5"),
        _dev(alpha, torch.float32, "alpha", 1), N,
        _dev(bias, torch.float32, "bias", N) if bias is not None else None,
        _dev(y, torch.float32, "y", M * N), _stream(stream)))
    return y


def bitlinear_quantize_weights_blocks(W, W_packed=None, alpha_blocks=None, stream=None):
    """W [N, K] fp32 -> (W_packed uint8 [N, K/4], alpha_blocks fp32 [N, K/128])."""
    torch = _torch()
    N, K = W.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if alpha_blocks is None:
        alpha_blocks = torch.empty((N, K // 128), dtype=torch.float32, device=W.device)
    _check("bitlinear_quantize_weights_blocks", lib.bitlinear_quantize_weights_blocks(
        _dev(W, torch.float32, "W", N * K), N, K, _dev(W_packed, torch.uint8, "W_packed", N * (K // 4)),
        _dev(alpha_blocks, torch.float32, "alpha_blocks", N * (K // 128)), _stream(stream)))
    return W_packed, alpha_blocks


def bitlinear_forward_blocks(x_q, beta, W_packed, alpha_blocks, bias=None, y=None, stream=None):
    """y [M, N] from x_q, beta and block-scaled packed weights."""
    torch = _torch()
    M, K = x_q.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x_q.device)
    _check("bitlinear_forward_blocks", lib.bitlinear_forward_blocks(
        _dev(x_q, torch.int8, "x_q"), _dev(beta, torch.float32, "beta", M), M, K,
        _dev(W_packed, torch.uint8, "W_packed"), _dev(alpha_blocks, torch.float32, "alpha_blocks", N * (K // 128)),
        N, _dev(bias, torch.float32, "bias", N) if bias is not None else None, _dev(y, torch.float32, "y", M * N),
        _stream(stream)))
    return y


def bitlinear_mlp_forward(x, W1_packed, alpha1, W2_packed, alpha2, bias1=None, bias2=None, y=None, g=None,
                          x_q1=None, beta1=None, x_q2=None, beta2=None, stream=None):
    """BitMLP y = fc2(GELU(fc1(x))); returns (y, g).  x_q1/beta1/x_q2/beta2 are allocated
    when M > 1 and not given (the two-call path needs them beyond four tokens and is the
    faster one for most several-token shapes)."""
    torch = _torch()
    M, d_model = x.shape
    d_ff = W1_packed.shape[0]
    if W1_packed.shape[1] * 4 != d_model or W2_packed.shape != (d_model, d_ff // 4):
        raise ValueError("W1_packed must be [d_ff, d_model/4] and W2_packed [d_model, d_ff/4]")
    if y is None:
        y = torch.empty((M, d_model), dtype=torch.float32, device=x.device)
    if g is None:
        g = torch.empty((M, d_ff), dtype=torch.float32, device=x.device)
    if M > 1:
        if x_q1 is None:
            x_q1 = torch.empty((M, d_model), dtype=torch.int8, device=x.device)
        if beta1 is None:
            beta1 = torch.empty(M, dtype=torch.float32, device=x.device)
        if x_q2 is None:
            x_q2 = torch.empty((M, d_ff), dtype=torch.int8, device=x.device)
        if beta2 is None:
            beta2 = torch.empty(M, dtype=torch.float32, device=x.device)
    opt = lambda t, dt, n, k: _dev(t, dt, n, k) if t is not None else None
    _check("bitlinear_mlp_forward", lib.bitlinear_mlp_forward(
        _dev(x, torch.float32, "x", M * d_model), M, d_model, d_ff, _dev(W1_packed, torch.uint8, "W1_packed"),
        _dev(alpha1, torch.float32, "alpha1", 1), opt(bias1, torch.float32, "bias1", d_ff),
        _dev(W2_packed, torch.uint8, "W2_packed"), _dev(alpha2, torch.float32, "alpha2", 1),
        opt(bias2, torch.float32, "bias2", d_model), _dev(y, torch.float32, "y", M * d_model),
        _dev(g, torch.float32, "g", M * d_ff), opt(x_q1, torch.int8, "x_q1", M * d_model),
        opt(beta1, torch.float32, "beta1", M), opt(x_q2, torch.int8, "x_q2", M * d_ff),
        opt(beta2, torch.float32, "beta2", M), _stream(stream)))
    return y, g


def bitlinear_hadamard_rows(x, block, signs=None, out=None, stream=None):
    """x [M, K] fp32 -> rows rotated by diag(d) . blockdiag(H_block) / sqrt(block); out may be x."""
    torch = _torch()
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=x.device)
    _check("bitlinear_hadamard_rows", lib.bitlinear_hadamard_rows(
        _dev(x, torch.float32, "x", M * K), M, K, int(block),
        _dev(signs, torch.int8, "signs", K) if signs is not None else None,
        _dev(out, torch.float32, "out", M * K), _stream(stream)))
    return out


def bitlinear_quantize_act_hadamard(x, block, signs=None, x_q=None, beta=None, stream=None):
    """x [M, K] fp32 -> (x_q int8 [M, K], beta fp32 [M]) of the rotated rows."""
    torch = _torch()
    M, K = x.shape
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if beta is None:
        beta = torch.empty(M, dtype=torch.float32, device=x.device)
    _check("bitlinear_quantize_act_hadamard", lib.bitlinear_quantize_act_hadamard(
        _dev(x, torch.float32, "x", M * K), M, K, int(block),
        _dev(signs, torch.int8, "signs", K) if signs is not None else None,
        _dev(x_q, torch.int8, "x_q", M * K), _dev(beta, torch.float32, "beta", M), _stream(stream)))
    return x_q, beta


def bitlinear_forward_fused_hadamard(x, block, signs, W_packed, alpha, bias=None, y=None, x_q=None, beta=None,
                                     stream=None):
    """y [M, N] from fp32 x: rotation (block, signs), absmax int8 and the forward in one call."""
    torch = _torch()
    M, K = x.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    opt = lambda t, dt, n, k: _dev(t, dt, n, k) if t is not None else None
    _check("bitlinear_forward_fused_hadamard", lib.bitlinear_forward_fused_hadamard(
        _dev(x, torch.float32, "x", M * K), M, K, int(block), opt(signs, torch.int8, "signs", K),
        _dev(W_packed, torch.uint8, "W_packed"), _dev(alpha, torch.float32, "alpha", 1), N,
        opt(bias, torch.float32, "bias", N), _dev(y, torch.float32, "y", M * N), opt(x_q, torch.int8, "x_q", M * K),
        opt(beta, torch.float32, "beta", M), _stream(stream)))
    return y


def _forward(fn, what, x_q, beta, W_packed, alpha, bias, y, acc, stream, alpha_n=1):
    torch = _torch()
    M, K = x_q.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x_q.device)
    if acc is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=x_q.device)
    acc_ptr = _dev(acc, torch.int32, "acc", M * N) if acc is not None and acc is not False else None
    bias_ptr = _dev(bias, torch.float32, "bias", N) if bias is not None else None
    _check(what, fn(
        _dev(x_q, torch.int8, "x_q"), _dev(beta, torch.float32, "beta", M), M, K,
        _dev(W_packed, torch.uint8, "W_packed"), _dev(alpha, torch.float32, "alpha", alpha_n), N,
        bias_ptr, _dev(y, torch.float32, "y", M * N), acc_ptr, _stream(stream)))
    return (y, acc) if acc_ptr is not None else y


def bitlinear_forward(x_q, beta, W_packed, alpha, bias=None, y=None, acc=None, stream=None):
    """y [M, N] = (x_q . W_hat^T) * alpha*beta/127 (+ bias).  acc=True (or an int32 [M, N]
    tensor) also returns the exact integer sums: (y, acc)."""
    return _forward(lib.bitlinear_forward, "bitlinear_forward", x_q, beta, W_packed, alpha,
                    bias, y, acc, stream)


def bitlinear_forward_rows(x_q, beta, W_packed, alpha_rows, bias=None, y=None, acc=None, stream=None):
    """bitlinear_forward with one alpha per output row."""
    return _forward(lib.bitlinear_forward_rows, "bitlinear_forward_rows", x_q, beta, W_packed,
                    alpha_rows, bias, y, acc, stream, alpha_n=W_packed.shape[0])


def _forward_fused(name, x, W_packed, alpha, bias, y, x_q, beta, acc, stream):
    torch = _torch()
    M, K = x.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if acc is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=x.device)
    acc_ptr = _dev(acc, torch.int32, "acc", M * N) if acc is not None and acc is not False else None
    _check(name, getattr(lib, name)(
        _dev(x, torch.float32, "x", M * K), M, K, _dev(W_packed, torch.uint8, "W_packed"),
        _dev(alpha, torch.float32, "alpha", N if name.endswith("_rows") else 1), N,
        _dev(bias, torch.float32, "bias", N) if bias is not None else None, _dev(y, torch.float32, "y", M * N),
        _dev(x_q, torch.int8, "x_q", M * K) if x_q is not None else None,
        _dev(beta, torch.float32, "beta", M) if beta is not None else None, acc_ptr, _stream(stream)))
    return (y, acc) if acc_ptr is not None else y


def bitlinear_forward_fused(x, W_packed, alpha, bias=None, y=None, x_q=None, beta=None, acc=None,
                            stream=None):
    """y [M, N] from fp32 x [M, K] in one call (activation quantization + forward).
    x_q / beta (tensors) receive the quantized activations if given; acc as bitlinear_forward.
    Returns y, or (y, acc) when acc is requested."""
    return _forward_fused("bitlinear_forward_fused", x, W_packed, alpha, bias, y, x_q, beta, acc, stream)


def bitlinear_forward_fused_rows(x, W_packed, alpha_rows, bias=None, y=None, x_q=None, beta=None, acc=None,
                                 stream=None):
    """bitlinear_forward_fused with alpha_rows [N] fp32 (one alpha per output row); also the
    call for grouped projections (stacked packed rows, each projection's alpha repeated)."""
    return _forward_fused("bitlinear_forward_fused_rows", x, W_packed, alpha_rows, bias, y, x_q, beta, acc, stream)


def bitlinear_forward_fused_kernel(M, K, N, x=None, W_packed=None, x_q=None) -> str:
    xp = x.data_ptr() if x is not None else 256
    wp = W_packed.data_ptr() if W_packed is not None else 256
    qp = x_q.data_ptr() if x_q is not None else None
    return lib.bitlinear_forward_fused_kernel(M, K, N, xp, wp, qp).decode()


def bitlinear_forward_kernel(M, K, N, x_q=None, W_packed=None) -> str:
    """Name of the kernel bitlinear_forward selects (pointers decide alignment; None
    stands for a 256-byte aligned allocation)."""
    xp = x_q.data_ptr() if x_q is not None else 256
    wp = W_packed.data_ptr() if W_packed is not None else 256
    return lib.bitlinear_forward_kernel(M, K, N, xp, wp).decode()
