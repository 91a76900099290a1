"""CPU oracle for the BitNet b1.58 BitLinear path (W1.58A8) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The GPU library never imports, links or calls it, and this
package imports nothing from the GPU library.

The arithmetic lives in ``oracle.c`` (plain scalar C, built with ``-ffp-contract=off``);
this module only marshals NumPy arrays through ctypes.  Page keys used in citations:

* [P1] 2kiu.com, article on 1.58-bit quantization and hardware co-optimization (§2.3 and
  §4.2: one scale per block of 128 weights, shape [C_out, C_in/128]).
* [P2] nxmr.cn tutorial "1.58 位大模型" (per-row absmean, add/sub derivation, memory estimate,
  §1.1 and §6.1: more compact encodings than 2 bits).
* [P3] chenxutan.com, "1.58-bit 大模型极限量化实战：从 BitNet 三值权重到单颗 CPU 跑起 100B 模型"
  (absmean / absmax formulas, worked example, BitLinear forward, 2-bit packing, §6.1 the
  BitMLP, §6.2 the rotation before absmax).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]

_lib = None


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (plain C, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    p, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    sig = {
        "oracle_absmean": (f32, [p, i64]),
        "oracle_absmean_rows": (ctypes.c_int, [p, i64, i64, p]),
        "oracle_ternarize": (ctypes.c_int, [p, i64, f32, p]),
        "oracle_ternarize_rows": (ctypes.c_int, [p, i64, i64, p, p]),
        "oracle_pack": (ctypes.c_int, [p, i64, i64, p]),
        "oracle_unpack": (ctypes.c_int, [p, i64, i64, p]),
        "oracle_quantize_weights": (ctypes.c_int, [p, i64, i64, p, p, p]),
        "oracle_quantize_act": (ctypes.c_int, [p, i64, i64, p, p]),
        "oracle_ternary_matmul": (ctypes.c_int, [p, i64, i64, p, i64, p, i64, i64]),
        "oracle_dequant_scale": (f32, [f32, f32]),
        "oracle_dequant": (ctypes.c_int, [p, p, f32, p, i64, i64, p, p, i64, i64]),
        "oracle_hadamard_rows": (ctypes.c_int, [p, i64, i64, i64, p, p]),
        "oracle_absmean_blocks": (ctypes.c_int, [p, i64, i64, p]),
        "oracle_ternarize_blocks": (ctypes.c_int, [p, i64, i64, p, p]),
        "oracle_ternary_matmul_blocks": (ctypes.c_int, [p, i64, i64, p, i64, p]),
        "oracle_dequant_blocks": (ctypes.c_int, [p, p, p, i64, i64, i64, p, p]),
        "oracle_gelu": (ctypes.c_int, [p, i64, p]),
        "oracle_t5_row_bytes": (i64, [i64]),
        "oracle_pack_t5": (ctypes.c_int, [p, i64, i64, p]),
        "oracle_unpack_t5": (ctypes.c_int, [p, i64, i64, p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what} failed with oracle status {rc}")


def absmean(w: np.ndarray) -> np.float32:
    """[P3 §2.3] alpha = mean|W| over the whole tensor (fp64 sum, one fp32 rounding)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    return np.float32(_load().oracle_absmean(_ptr(w), w.size))


def absmean_rows(w: np.ndarray) -> np.ndarray:
    """[P2 §3.1, §4.2] per-output-row alpha[n] = mean_k |W[n, k]|."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    out = np.empty(n, np.float32)
    _check(_load().oracle_absmean_rows(_ptr(w), n, k, _ptr(out)), "absmean_rows")
    return out


def ternarize(w: np.ndarray, alpha) -> np.ndarray:
    """[P3 §2.3] clip(round(W / alpha), -1, 1) as int8 codes."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    out = np.empty(w.shape, np.int8)
    _check(_load().oracle_ternarize(_ptr(w), w.size, float(np.float32(alpha)), _ptr(out)),
           "ternarize")
    return out


def ternarize_rows(w: np.ndarray, alpha_rows: np.ndarray) -> np.ndarray:
    """Per-row variant of :func:`ternarize`: row n is divided by alpha_rows[n]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    a = np.ascontiguousarray(alpha_rows, dtype=np.float32)
    n, k = w.shape
    out = np.empty(w.shape, np.int8)
    _check(_load().oracle_ternarize_rows(_ptr(w), n, k, _ptr(a), _ptr(out)), "ternarize_rows")
    return out


def pack(codes: np.ndarray) -> np.ndarray:
    """[P3 §5.3] 2-bit packing, code w+1, 4 per byte, weight k=4b+i at bits 2i..2i+1."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n, k = codes.shape
    out = np.empty((n, k // 4), np.uint8)
    _check(_load().oracle_pack(_ptr(codes), n, k, _ptr(out)), "pack")
    return out


def unpack(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of :func:`pack`; raises on the never-written pattern 11."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    assert packed.size == n * (k // 4)
    out = np.empty((n, k), np.int8)
    _check(_load().oracle_unpack(_ptr(packed), n, k, _ptr(out)), "unpack")
    return out


def quantize_weights(w: np.ndarray):
    """[P3 §2.3, §4.1, §5.3] returns (codes int8 [N,K], packed uint8 [N,K/4], alpha fp32)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    codes = np.empty((n, k), np.int8)
    packed = np.empty((n, k // 4), np.uint8)
    alpha = np.zeros(1, np.float32)
    _check(_load().oracle_quantize_weights(_ptr(w), n, k, _ptr(codes), _ptr(packed), _ptr(alpha)),
           "quantize_weights")
    return codes, packed, alpha[0]


def quantize_act(x: np.ndarray):
    """[P3 §2.4, §4.1] per-token absmax int8: returns (x_q int8 [M,K], beta fp32 [M])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    beta = np.empty(m, np.float32)
    _check(_load().oracle_quantize_act(_ptr(x), m, k, _ptr(xq), _ptr(beta)), "quantize_act")
    return xq, beta


def ternary_matmul(xq: np.ndarray, codes: np.ndarray, n0: int = 0, n1: int | None = None,
                   out: np.ndarray | None = None) -> np.ndarray:
    """[P2 §3.3] acc[m,n] = sum_{W=+1} x_q - sum_{W=-1} x_q (int32), rows n0..n1 of W."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    m, k = xq.shape
    n = codes.shape[0]
    assert codes.shape[1] == k
    n1 = n if n1 is None else n1
    if out is None:
        out = np.zeros((m, n), np.int32)
    _check(_load().oracle_ternary_matmul(_ptr(xq), m, k, _ptr(codes), n, _ptr(out), n0, n1),
           "ternary_matmul")
    return out


def dequant_scale(alpha, beta) -> np.float32:
    """[P3 §2.4] fp32((double)alpha * (double)beta / 127)."""
    return np.float32(_load().oracle_dequant_scale(float(np.float32(alpha)), float(np.float32(beta))))


def dequant(acc: np.ndarray, beta: np.ndarray, alpha=0.0, alpha_rows: np.ndarray | None = None,
            bias: np.ndarray | None = None, n0: int = 0, n1: int | None = None,
            out: np.ndarray | None = None) -> np.ndarray:
    """[P3 §2.4, §3.2] y = acc * alpha*beta/127 (+ bias), fp32."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    m, n = acc.shape
    ar = None if alpha_rows is None else np.ascontiguousarray(alpha_rows, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    n1 = n if n1 is None else n1
    if out is None:
        out = np.zeros((m, n), np.float32)
    _check(_load().oracle_dequant(_ptr(acc), _ptr(beta), float(np.float32(alpha)), _ptr(ar), m, n,
                                  _ptr(b), _ptr(out), n0, n1), "dequant")
    return out


def forward(xq: np.ndarray, beta: np.ndarray, packed: np.ndarray, k: int, alpha,
            bias: np.ndarray | None = None, alpha_rows: np.ndarray | None = None):
    """[P3 §3.2] integer matmul on the unpacked codes, then the dequant epilogue.

    Returns (acc int32 [M,N], y fp32 [M,N])."""
    codes = unpack(packed, k)
    acc = ternary_matmul(xq, codes)
    y = dequant(acc, beta, alpha, alpha_rows=alpha_rows, bias=bias)
    return acc, y


def bitlinear(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None = None):
    """[P3 §3.2, §4.2] whole BitLinear inference forward from float x and W.

    Returns a dict with every intermediate: codes, packed, alpha, xq, beta, acc, y."""
    codes, packed, alpha = quantize_weights(w)
    xq, beta = quantize_act(x)
    acc = ternary_matmul(xq, codes)
    y = dequant(acc, beta, alpha, bias=bias)
    return dict(codes=codes, packed=packed, alpha=alpha, xq=xq, beta=beta, acc=acc, y=y)


def hadamard_rows(x: np.ndarray, block: int, signs: np.ndarray | None = None) -> np.ndarray:
    """[P3 §6.2] randomized Hadamard rotation along K in blocks of ``block`` (readings R10,
    R11 of ``oracle.c``): sign flip by ``signs`` (int8, negative = flip), Sylvester
    butterflies with stride 1, 2, ..., block/2 in fp32, then a multiply by fp32(1/sqrt(block))."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    d = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    if d is not None:
        assert d.shape == (k,)
    out = np.empty((m, k), np.float32)
    _check(_load().oracle_hadamard_rows(_ptr(x), m, k, int(block), _ptr(d), _ptr(out)), "hadamard_rows")
    return out


def quantize_act_hadamard(x: np.ndarray, block: int, signs: np.ndarray | None = None):
    """[P3 §6.2 then §2.4] rotate each token (:func:`hadamard_rows`), then per-token absmax
    int8 of the rotated row.  Returns (x_q int8 [M,K], beta fp32 [M])."""
    return quantize_act(hadamard_rows(x, block, signs))


def bitlinear_hadamard(x: np.ndarray, w: np.ndarray, block: int, signs: np.ndarray | None = None,
                       bias: np.ndarray | None = None):
    """BitLinear forward with the rotation of [P3 §6.2] on both operands: W and x are rotated
    by the same R, then quantized and multiplied as in :func:`bitlinear`."""
    return bitlinear(hadamard_rows(x, block, signs), hadamard_rows(w, block, signs), bias=bias)


# ------------------------------------------------------------------ block scales (R12)
BLOCK = 128


def absmean_blocks(w: np.ndarray) -> np.ndarray:
    """[P1 §2.3, §4.2] alpha [N, K/128]: mean |W| over each block of 128 weights of a row."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    out = np.empty((n, k // BLOCK), np.float32)
    _check(_load().oracle_absmean_blocks(_ptr(w), n, k, _ptr(out)), "absmean_blocks")
    return out


def ternarize_blocks(w: np.ndarray, alpha_blocks: np.ndarray) -> np.ndarray:
    """[P3 §2.3] codes with every weight divided by its block's alpha."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    a = np.ascontiguousarray(alpha_blocks, dtype=np.float32)
    n, k = w.shape
    assert a.shape == (n, k // BLOCK)
    out = np.empty((n, k), np.int8)
    _check(_load().oracle_ternarize_blocks(_ptr(w), n, k, _ptr(a), _ptr(out)), "ternarize_blocks")
    return out


def quantize_weights_blocks(w: np.ndarray):
    """Block-scaled weight quantization: returns (codes int8 [N,K], packed uint8 [N,K/4],
    alpha_blocks fp32 [N,K/128]); the packing is the 2-bit layout of :func:`pack`."""
    a = absmean_blocks(w)
    codes = ternarize_blocks(w, a)
    return codes, pack(codes), a


def ternary_matmul_blocks(xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """[P2 §3.3] per-block integer sums acc [M, N, K/128] (int32)."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    m, k = xq.shape
    n = codes.shape[0]
    out = np.zeros((m, n, k // BLOCK), np.int32)
    _check(_load().oracle_ternary_matmul_blocks(_ptr(xq), m, k, _ptr(codes), n, _ptr(out)), "ternary_matmul_blocks")
    return out


def dequant_blocks(acc: np.ndarray, beta: np.ndarray, alpha_blocks: np.ndarray,
                   bias: np.ndarray | None = None) -> np.ndarray:
    """[P1 §2.3; P3 §2.4] y = fp32(sum_b alpha[n,b] acc[m,n,b] * beta[m]/127) in fp64 (+ bias)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    a = np.ascontiguousarray(alpha_blocks, dtype=np.float32)
    m, n, kb = acc.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((m, n), np.float32)
    _check(_load().oracle_dequant_blocks(_ptr(acc), _ptr(beta), _ptr(a), m, n, kb, _ptr(b), _ptr(out)),
           "dequant_blocks")
    return out


def forward_blocks(xq: np.ndarray, beta: np.ndarray, packed: np.ndarray, k: int, alpha_blocks: np.ndarray,
                   bias: np.ndarray | None = None):
    """Block-scaled forward on packed codes: returns (acc_blocks [M,N,K/128], y [M,N])."""
    acc = ternary_matmul_blocks(xq, unpack(packed, k))
    return acc, dequant_blocks(acc, beta, alpha_blocks, bias)


def bitlinear_blocks(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None = None):
    """Whole BitLinear forward with block scales; returns every intermediate."""
    codes, packed, a = quantize_weights_blocks(w)
    xq, beta = quantize_act(x)
    acc = ternary_matmul_blocks(xq, codes)
    y = dequant_blocks(acc, beta, a, bias)
    return dict(codes=codes, packed=packed, alpha_blocks=a, xq=xq, beta=beta, acc_blocks=acc, y=y)


# ------------------------------------------------------------------ BitMLP (R13)
def gelu(h: np.ndarray) -> np.ndarray:
    """[P3 §6.1] torch.nn.GELU (erf form) in fp64, one fp32 rounding (reading R13)."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    out = np.empty(h.shape, np.float32)
    _check(_load().oracle_gelu(_ptr(h), h.size, _ptr(out)), "gelu")
    return out


def bitmlp(x: np.ndarray, w1: np.ndarray, w2: np.ndarray, b1: np.ndarray | None = None,
           b2: np.ndarray | None = None):
    """[P3 §6.1] BitMLP forward fc2(GELU(fc1(x))), both layers BitLinear (per-tensor alpha).
    Returns a dict with fc1's and fc2's intermediates (``fc1``, ``fc2``), ``g`` and ``y``."""
    r1 = bitlinear(x, w1, bias=b1)
    g = gelu(r1["y"])
    r2 = bitlinear(g, w2, bias=b2)
    return dict(fc1=r1, g=g, fc2=r2, y=r2["y"])


# ------------------------------------------------------------------ 5 trits per byte (R14)
def t5_row_bytes(k: int) -> int:
    """Bytes per row of the 5-trit packing: 16 * ceil(K / 80)."""
    return int(_load().oracle_t5_row_bytes(int(k)))


def pack_t5(codes: np.ndarray) -> np.ndarray:
    """[P2 §1.1, §6.1] five codes per byte, sum_i (W_hat[5b+i] + 1) 3^i (reading R14)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n, k = codes.shape
    out = np.empty((n, t5_row_bytes(k)), np.uint8)
    _check(_load().oracle_pack_t5(_ptr(codes), n, k, _ptr(out)), "pack_t5")
    return out


def unpack_t5(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of :func:`pack_t5` (first K weights of each row)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    assert packed.shape[1] == t5_row_bytes(k)
    out = np.empty((n, k), np.int8)
    _check(_load().oracle_unpack_t5(_ptr(packed), n, k, _ptr(out)), "unpack_t5")
    return out


def forward_t5(xq: np.ndarray, beta: np.ndarray, packed_t5: np.ndarray, k: int, alpha,
               bias: np.ndarray | None = None):
    """Forward on 5-trit packed codes: unpack, then the integer matmul and dequant of
    :func:`forward`.  Returns (acc, y)."""
    acc = ternary_matmul(xq, unpack_t5(packed_t5, k))
    return acc, dequant(acc, beta, alpha, bias=bias)
