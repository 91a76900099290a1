"""Host-side checks of the C ABI that need no GPU: the library loads, exports every symbol
include/bitlinear.h declares, and rejects invalid arguments before any HIP call.

Every call below is invalid on purpose, so nothing is ever enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


@pytest.fixture(scope="module")
def bl():
    pkg = os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "libbitlinear.so")
    if not os.path.exists(pkg):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "bitlinear_hip_build", os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    import bitlinear_matmul_absmean_amd as m
    return m


def _declared(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_are_exported(bl):
    names = _declared()
    assert "bitlinear_forward" in names and "bitlinear_quantize_act" in names
    lib = ctypes.CDLL(bl.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in bitlinear.h but not exported"
    # and the binding knows each of them
    assert set(names) <= set(bl.SIGNATURES)


def test_ceiling_library_exports_its_header(bl):
    """The measurement kernels live in their own library, declared by bitlinear_ceiling.h."""
    names = _declared(os.path.join(ROOT, "include", "bitlinear_ceiling.h"))
    assert names == ["bitlinear_ceiling_mfma", "bitlinear_ceiling_read"]
    lib = ctypes.CDLL(os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "libbitlinear_ceiling.so"))
    for n in names:
        assert hasattr(lib, n), f"{n} declared in bitlinear_ceiling.h but not exported"
    # invalid arguments are rejected before any HIP call
    lib.bitlinear_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.bitlinear_ceiling_read(None, 16, None, None) == -1
    assert lib.bitlinear_ceiling_read(ctypes.c_void_p(16), 15, ctypes.c_void_p(16), None) == -1
    lib.bitlinear_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    assert lib.bitlinear_ceiling_mfma(0, 1, ctypes.c_void_p(16), ctypes.c_void_p(16), None, None) == -1


def test_abi_version_and_status_strings(bl):
    assert bl.abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5, -6):
        s = bl.lib.bitlinear_status_string(st).decode()
        assert s and s != "unknown status"
    assert bl.lib.bitlinear_status_string(-99).decode() == "unknown status"
    assert bl.lib.bitlinear_last_hip_error() == 0


def test_workspace_size(bl):
    assert bl.lib.bitlinear_quantize_weights_workspace_size(4096, 11008) == 4096 * 8
    assert bl.lib.bitlinear_quantize_weights_workspace_size(0, 16) == 0
    assert bl.lib.bitlinear_quantize_weights_workspace_size(4, -1) == 0


A = 4096  # a fake, 4096-aligned "device address"; never dereferenced (calls are invalid)


def test_quantize_weights_noalloc_validation(bl):
    """The allocation-free call validates like bitlinear_quantize_weights and rejects N beyond
    its fixed scratch before any HIP call."""
    f = bl.lib.bitlinear_quantize_weights_noalloc
    rows = bl.lib.bitlinear_quantize_weights_noalloc_max_rows()
    assert rows == 262144
    assert f(None, 4, 16, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 16, None, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 16, A, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 0, 16, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 18, A, A, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(A, rows + 1, 16, A, A, None) == bl.BITLINEAR_ERR_SCRATCH
    assert f(A + 4, 4, 16, A, A, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, 4, 16, A + 1, A, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert bl.lib.bitlinear_last_hip_error() == 0


def test_quantize_weights_validation(bl):
    f = bl.lib.bitlinear_quantize_weights
    ws = 1 << 20
    assert f(None, 4, 8, A, A, A, ws, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 8, None, A, A, ws, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 8, A, None, A, ws, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 0, 8, A, A, A, ws, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, -8, A, A, A, ws, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 6, A, A, A, ws, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(A, 4, bl.BITLINEAR_MAX_K + 4, A, A, A, ws, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(A, 1 << 62, 1 << 20, A, A, A, ws, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(A + 4, 4, 8, A, A, A, ws, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, 4, 8, A + 2, A, A, ws, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, 4, 8, A, A, None, ws, None) == bl.BITLINEAR_ERR_WORKSPACE
    assert f(A, 4, 8, A, A, A, 31, None) == bl.BITLINEAR_ERR_WORKSPACE
    assert f(A, 4, 8, A, A, A + 4, ws, None) == bl.BITLINEAR_ERR_ALIGNMENT


def test_quantize_weights_rows_validation(bl):
    f = bl.lib.bitlinear_quantize_weights_rows
    assert f(None, 4, 8, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 8, A, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 4, 10, A, A, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(A + 8, 4, 8, A, A, None) == bl.BITLINEAR_ERR_ALIGNMENT


def test_quantize_act_validation(bl):
    f = bl.lib.bitlinear_quantize_act
    assert f(None, 1, 8, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1, 8, None, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1, 8, A, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 0, 8, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1, 0, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1 << 40, 1 << 30, A, A, None) == bl.BITLINEAR_ERR_SHAPE


@pytest.mark.parametrize("name", ["bitlinear_forward", "bitlinear_forward_rows"])
def test_forward_validation(bl, name):
    f = getattr(bl.lib, name)
    ok = dict(xq=A, beta=A, M=1, K=64, wp=A, alpha=A, N=8, bias=None, y=A, acc=None, s=None)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return f(d["xq"], d["beta"], d["M"], d["K"], d["wp"], d["alpha"], d["N"], d["bias"], d["y"],
                 d["acc"], d["s"])

    for k in ("xq", "beta", "wp", "alpha", "y"):
        assert call(**{k: None}) == bl.BITLINEAR_ERR_INVALID_ARG
    for k in ("M", "K", "N"):
        assert call(**{k: 0}) == bl.BITLINEAR_ERR_INVALID_ARG
        assert call(**{k: -4}) == bl.BITLINEAR_ERR_INVALID_ARG
    assert call(K=66) == bl.BITLINEAR_ERR_SHAPE
    assert call(K=bl.BITLINEAR_MAX_K + 4) == bl.BITLINEAR_ERR_SHAPE
    assert call(M=1 << 40, K=1 << 24 - 4) == bl.BITLINEAR_ERR_SHAPE
    assert call(N=1 << 33) == bl.BITLINEAR_ERR_SHAPE


def test_forward_fused_rows_validation(bl):
    """The per-row (grouped) fused call validates like the per-tensor one, before any HIP call."""
    f = bl.lib.bitlinear_forward_fused_rows
    good = 4096
    # null x, null alpha_rows, null y
    assert f(None, 1, 64, good, good, 8, None, good, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(good, 1, 64, good, None, 8, None, good, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(good, 1, 64, good, good, 8, None, None, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    # K % 4, sizes
    assert f(good, 1, 66, good, good, 8, None, good, None, None, None, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(good, 0, 64, good, good, 8, None, good, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    # the two-call path (M > 4) needs x_q and beta
    assert f(good, 8, 64, good, good, 8, None, good, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG


def test_forward_fused_validation(bl):
    f = bl.lib.bitlinear_forward_fused
    assert f(None, 1, 64, A, A, 8, None, A, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1, 64, None, A, 8, None, A, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1, 64, A, None, 8, None, A, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1, 64, A, A, 8, None, None, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 0, 64, A, A, 8, None, A, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 1, 66, A, A, 8, None, A, None, None, None, None) == bl.BITLINEAR_ERR_SHAPE
    # two-call path without x_q / beta buffers
    assert f(A, 5, 64, A, A, 8, None, A, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A + 4, 1, 64, A, A, 8, None, A, None, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG


def test_kernel_selection(bl):
    sel = bl.lib.bitlinear_forward_kernel
    assert sel(1, 4096, 4096, A, A).decode() == "gemv_dot4"
    assert sel(2, 4096, 4096, A, A).decode() == "decode_mfma_i8"   # two tokens, < 2^26 weights, K < 8192
    assert sel(2, 8192, 1000, A, A).decode() == "gemv_dot4"         # two tokens with K >= 8192
    assert sel(2, 4096, 16384, A, A).decode() == "gemv_dot4"        # two tokens, >= 2^26 weights
    assert sel(3, 8192, 1000, A, A).decode() == "decode_mfma_i8"
    assert sel(4, 8192, 8191, A, A).decode() == "decode_mfma_i8"
    assert sel(2, 8192, 8192, A, A).decode() == "gemv_dot4"
    assert sel(4, 16384, 4096, A, A).decode() == "decode_mfma_i8"   # three and four tokens: decode kernel
    assert sel(3, 8192, 28672, A, A).decode() == "decode_mfma_i8"
    assert sel(5, 4096, 4096, A, A).decode() == "decode_mfma_i8"
    assert sel(64, 11008, 4096, A, A).decode() == "decode_mfma_i8"
    assert sel(65, 4096, 4096, A, A).decode() == "gemm_mfma_i8"
    assert sel(65, 4160, 4096, A, A).decode() == "gemm_mfma_i8"
    assert sel(2048, 4096, 11008, A, A).decode() == "gemm_mfma_i8"
    assert sel(1, 4100, 4096, A, A).decode() == "generic"        # K % 64 != 0
    assert sel(1, 4096, 4096, A + 4, A).decode() == "generic"    # unaligned x_q
    assert sel(64, 4096, 4096, A, A + 8).decode() == "generic"   # unaligned W_packed
    assert sel(1, 32768, 64, A, A).decode() == "gemv_dot4"
    assert sel(1, 32832, 64, A, A).decode() == "decode_mfma_i8"   # K beyond the GEMV's registers
    assert sel(2, 16384, 4096, A, A).decode() == "gemv_dot4"
    assert sel(2, 16448, 4096, A, A).decode() == "decode_mfma_i8"   # K beyond the several-token GEMV
    fsel = bl.lib.bitlinear_forward_fused_kernel
    assert fsel(1, 4096, 4096, A, A, None).decode() == "gemv_fused"
    assert fsel(1, 4096, 4096, A, A, A + 4).decode() == "quantize_act+forward"  # x_q export unaligned
    assert fsel(5, 4096, 4096, A, A, A).decode() == "quantize_act+forward"
    assert fsel(3, 4096, 4096, A, A, None).decode() == "gemv_fused"            # no buffers: one launch
    assert fsel(3, 4096, 4096, A, A, A).decode() == "quantize_act+forward"     # buffers: the faster route
    assert fsel(2, 4096, 4096, A, A, A).decode() == "gemv_fused"
    assert fsel(2, 4160, 4096, A, A, A).decode() == "quantize_act+forward"
    assert fsel(1, 32768, 4096, A, A, None).decode() == "gemv_fused"
    assert fsel(1, 32832, 4096, A, A, None).decode() == "quantize_act+forward"   # K beyond the GEMV


def test_binding_has_no_host_fallback():
    src = open(os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "__init__.py")).read()
    assert "import oracle" not in src and "from oracle" not in src
    csrc = os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        path = os.path.join(csrc, f)
        if not os.path.isfile(path):
            continue
        text = open(path).read()
        assert "oracle" not in text.lower(), f


def test_hadamard_validation(bl):
    """Rotation calls reject bad blocks, shapes and alignments before any HIP call."""
    h, q = bl.lib.bitlinear_hadamard_rows, bl.lib.bitlinear_quantize_act_hadamard
    for block in (0, 3, 6, 8192):
        assert h(A, 1, 8192, block, None, A, None) in (bl.BITLINEAR_ERR_SHAPE, bl.BITLINEAR_ERR_INVALID_ARG)
        assert q(A, 1, 8192, block, None, A, A, None) in (bl.BITLINEAR_ERR_SHAPE, bl.BITLINEAR_ERR_INVALID_ARG)
    assert h(A, 1, 96, 64, None, A, None) == bl.BITLINEAR_ERR_SHAPE          # K % block
    assert h(A, 1, 6, 2, None, A, None) == bl.BITLINEAR_ERR_SHAPE            # K % 4
    assert h(None, 1, 64, 64, None, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert h(A, 1, 64, 64, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert h(A, 0, 64, 64, None, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert h(A + 4, 1, 64, 64, None, A, None) == bl.BITLINEAR_ERR_ALIGNMENT   # x 16-byte
    assert h(A, 1, 64, 64, None, A + 8, None) == bl.BITLINEAR_ERR_ALIGNMENT   # out 16-byte
    assert h(A, 1, 64, 64, A + 2, A, None) == bl.BITLINEAR_ERR_ALIGNMENT      # signs 4-byte
    assert q(A, 1, 64, 64, None, None, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert q(A, 1, 64, 64, None, A, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert q(A, 1, 64, 64, None, A + 2, A, None) == bl.BITLINEAR_ERR_ALIGNMENT  # x_q 4-byte
    assert q(A, 1, 64, 64, A + 1, A, A, None) == bl.BITLINEAR_ERR_ALIGNMENT


def test_blocks_validation(bl):
    q, f = bl.lib.bitlinear_quantize_weights_blocks, bl.lib.bitlinear_forward_blocks
    assert q(None, 4, 128, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert q(A, 4, 192, A, A, None) == bl.BITLINEAR_ERR_SHAPE                 # K % 128
    assert q(A + 4, 4, 128, A, A, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert q(A, 4, 128, A, A + 2, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, A, 1, 192, A, A, 8, None, A, None) == bl.BITLINEAR_ERR_SHAPE   # K % 128
    assert f(A, A, 1, 65536, A, A, 8, None, A, None) == bl.BITLINEAR_ERR_SHAPE # K > 32768
    assert f(A + 4, A, 1, 128, A, A, 8, None, A, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, A, 1, 128, A + 8, A, 8, None, A, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, A, 1, 128, A, None, 8, None, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, A, 0, 128, A, A, 8, None, A, None) == bl.BITLINEAR_ERR_INVALID_ARG


def test_mlp_validation_checks_both_layers_first(bl):
    """A bad second layer is reported before the first is enqueued (nothing runs)."""
    f = bl.lib.bitlinear_mlp_forward
    ok = (A, 1, 64, 128, A, A, None, A, A, None, A, A, None, None, None, None, None)
    assert f(*ok[:11], None, *ok[12:]) == bl.BITLINEAR_ERR_INVALID_ARG        # g missing
    assert f(A, 1, 64, 130, A, A, None, A, A, None, A, A, None, None, None, None, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(A, 1, 66, 128, A, A, None, A, A, None, A, A, None, None, None, None, None) == bl.BITLINEAR_ERR_SHAPE
    # M > 4 needs each layer's x_q / beta: missing for the second layer only
    assert f(A, 8, 64, 128, A, A, None, A, A, None, A, A, A, A, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert f(A, 8, 64, 128, A, None, None, A, A, None, A, A, A, A, A, A, None) == bl.BITLINEAR_ERR_INVALID_ARG


def test_t5_validation(bl):
    assert bl.lib.bitlinear_t5_row_bytes(4096) == 832 and bl.lib.bitlinear_t5_row_bytes(0) == 0
    q, f, r = bl.lib.bitlinear_quantize_weights_t5, bl.lib.bitlinear_forward_t5, bl.lib.bitlinear_repack_t5
    assert q(None, 4, 64, A, A, A, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert q(A, 4, 66, A, A, A, 1 << 20, None) == bl.BITLINEAR_ERR_SHAPE
    assert q(A, 4, 1 << 17, A, A, A, 1 << 20, None) == bl.BITLINEAR_ERR_SHAPE
    assert q(A, 4, 64, A, A, A, 8, None) == bl.BITLINEAR_ERR_WORKSPACE
    assert f(A, A, 1, 64, A + 4, A, 8, None, A, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, A, 1, 1 << 17, A, A, 8, None, A, None) == bl.BITLINEAR_ERR_SHAPE
    assert f(A, A, 70000, 64, A, A, 8, None, A, None) == bl.BITLINEAR_ERR_SHAPE
    assert r(None, 4, 64, A, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert r(A, 4, 66, A, None) == bl.BITLINEAR_ERR_SHAPE


def test_forward_fused_hadamard_validation(bl):
    f = bl.lib.bitlinear_forward_fused_hadamard
    assert f(A, 1, 4096, 3, None, A, A, 8, None, A, None, None, None) == bl.BITLINEAR_ERR_SHAPE        # block
    assert f(A, 1, 4096, 8192, None, A, A, 8, None, A, None, None, None) == bl.BITLINEAR_ERR_SHAPE     # block > 4096
    assert f(A, 1, 96, 64, None, A, A, 8, None, A, None, None, None) == bl.BITLINEAR_ERR_SHAPE         # K % block
    assert f(A + 4, 1, 4096, 4096, None, A, A, 8, None, A, None, None, None) == bl.BITLINEAR_ERR_ALIGNMENT
    assert f(A, 1, 4096, 4096, None, A, None, 8, None, A, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
    # the two-step path (M > 1) needs x_q and beta
    assert f(A, 2, 4096, 4096, None, A, A, 8, None, A, None, None, None) == bl.BITLINEAR_ERR_INVALID_ARG
