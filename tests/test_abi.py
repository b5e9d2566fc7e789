"""C-ABI checks that need no GPU: the library loads, exports every function
include/bfp8.h declares, and rejects bad arguments with status codes before
any HIP call (so these run on a host without a device)."""
import ctypes
import os
import re

import pytest

import blockwise_fp8_gemm_bfp8_amd as bfp8
from blockwise_fp8_gemm_bfp8_amd import build as bfp8_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bfp8.h")

OK, NULL, SHAPE, ALIGN, DTYPE, LAYOUT, SMODE, WS = range(8)
P = 0x10000  # a 16-byte aligned fake address; never dereferenced on error paths


@pytest.fixture(scope="session")
def L():
    if not os.path.exists(bfp8_build.LIB_PATH):
        bfp8_build.build()
    return bfp8.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:bfp8_status|size_t|const char\*|int)\s+(bfp8_\w+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["bfp8_quantize_act", "bfp8_quantize_act_transposed",
                            "bfp8_quantize_act_dual",
                            "bfp8_quantize_weight", "bfp8_quantize_weight_batch",
                            "bfp8_gemm", "bfp8_gemm_workspace_bytes",
                            "bfp8_quantize_mx_act", "bfp8_quantize_mx_act_transposed",
                            "bfp8_quantize_mx_act_dual", "bfp8_quantize_mx_weight",
                            "bfp8_quantize_mx_weight_batch",
                            "bfp8_gemm_mx", "bfp8_gemm_static_scratch",
                            "bfp8_quantize_act_kmajor", "bfp8_quantize_act_transposed_kmajor",
                            "bfp8_quantize_act_dual_kmajor", "bfp8_quantize_mx_act_dual_kmajor",
                            "bfp8_status_str", "bfp8_abi_version"])


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.bfp8_abi_version() == 5
    for code in range(10):
        assert len(L.bfp8_status_str(code)) > 0
    assert b"Inf or NaN" in L.bfp8_status_str(9)
    src = open(HEADER).read()
    assert "BFP8_ERR_NONFINITE = 9" in src and bfp8.STATUS[9] == "BFP8_ERR_NONFINITE"
    assert L.bfp8_status_str(99) == b"unknown status"


def test_weight_job_struct_matches_header():
    # bfp8_weight_job: w, rows, cols, ldw, q, ldq, s (pointers and int64s, no padding)
    assert ctypes.sizeof(bfp8.WeightJob) == 56
    assert [f[0] for f in bfp8.WeightJob._fields_] == ["w", "rows", "cols", "ldw", "q", "ldq", "s"]
    src = open(HEADER).read()
    assert "#define BFP8_MAX_WEIGHT_JOBS %d" % bfp8.MAX_WEIGHT_JOBS in src


def test_quantize_weight_batch_errors(L):
    def batch(*jobs, n=None, dt=0):
        arr = (bfp8.WeightJob * max(len(jobs), 1))(*jobs)
        return L.bfp8_quantize_weight_batch(ctypes.cast(arr, ctypes.c_void_p),
                                            len(jobs) if n is None else n, dt, None)
    good = dict(w=P, rows=384, cols=256, ldw=256, q=P, ldq=256, s=P)
    J = lambda **k: bfp8.WeightJob(**{**good, **k})
    assert L.bfp8_quantize_weight_batch(None, 0, 0, None) == OK   # nothing to do
    assert L.bfp8_quantize_weight_batch(None, 1, 0, None) == NULL
    assert batch(J(), n=-1) == SHAPE
    assert batch(J(), n=bfp8.MAX_WEIGHT_JOBS + 1) == SHAPE
    assert batch(J(), J(w=None)) == NULL                           # second job checked too
    assert batch(J(s=None)) == NULL
    assert batch(J(q=P + 4)) == ALIGN
    assert batch(J(ldw=260)) == ALIGN                              # bf16 row not 16-byte aligned
    assert batch(J(ldq=128)) == SHAPE                              # ldq < cols
    assert batch(J(rows=-1)) == SHAPE
    assert batch(J(), dt=5) == DTYPE
    # empty jobs are skipped; a batch of only empty jobs launches nothing
    assert batch(J(w=None, q=None, s=None, rows=0), J(w=None, q=None, s=None, cols=0)) == OK


def test_quantize_mx_weight_batch_errors(L):
    def batch(*jobs, n=None, dt=0):
        arr = (bfp8.WeightJob * max(len(jobs), 1))(*jobs)
        return L.bfp8_quantize_mx_weight_batch(ctypes.cast(arr, ctypes.c_void_p),
                                               len(jobs) if n is None else n, dt, None)
    good = dict(w=P, rows=384, cols=256, ldw=256, q=P, ldq=256, s=P)
    J = lambda **k: bfp8.WeightJob(**{**good, **k})
    assert L.bfp8_quantize_mx_weight_batch(None, 0, 0, None) == OK
    assert L.bfp8_quantize_mx_weight_batch(None, 2, 0, None) == NULL
    assert batch(J(), n=bfp8.MAX_WEIGHT_JOBS + 1) == SHAPE
    assert batch(J(), J(q=None)) == NULL
    assert batch(J(w=P + 8)) == ALIGN
    assert batch(J(ldq=128)) == SHAPE                              # ldq < cols
    assert batch(J(), dt=3) == DTYPE


def qa(L, x=P, dt=0, rows=256, cols=512, ldx=512, q=P, ldq=512, s=P):
    return L.bfp8_quantize_act(x, dt, rows, cols, ldx, q, ldq, s, None)


def test_quantize_act_errors(L):
    assert qa(L, x=None) == NULL
    assert qa(L, q=None) == NULL
    assert qa(L, s=None) == NULL
    assert qa(L, cols=500, ldx=512) == SHAPE      # grouped axis not a multiple of 128
    assert qa(L, rows=-1) == SHAPE
    assert qa(L, ldx=256) == SHAPE                # ldx < cols
    assert qa(L, ldq=256) == SHAPE
    assert qa(L, x=P + 8) == ALIGN
    assert qa(L, q=P + 4) == ALIGN
    assert qa(L, ldx=516) == ALIGN                # bf16 row not 16-byte aligned
    assert qa(L, ldq=520) == ALIGN
    assert qa(L, dt=7) == DTYPE
    # empty problems are valid and touch nothing, even with null pointers
    assert qa(L, x=None, q=None, s=None, rows=0) == OK
    assert qa(L, x=None, q=None, s=None, cols=0) == OK


def test_quantize_transposed_errors(L):
    f = lambda **k: L.bfp8_quantize_act_transposed(
        k.get("x", P), k.get("dt", 0), k.get("rows", 256), k.get("cols", 384),
        k.get("ldx", 384), k.get("q", P), k.get("ldq", 256), k.get("s", P), None)
    assert f(rows=200) == SHAPE                   # token axis must be a multiple of 128
    assert f(ldq=128) == SHAPE
    assert f(x=None) == NULL
    assert f(dt=1, ldx=385) == ALIGN
    assert f(rows=0, x=None, q=None, s=None) == OK
    assert f(cols=0, x=None, q=None, s=None) == OK


def test_quantize_dual_errors(L):
    f = lambda **k: L.bfp8_quantize_act_dual(
        k.get("x", P), k.get("dt", 0), k.get("rows", 256), k.get("cols", 384), k.get("ldx", 384),
        k.get("q", P), k.get("ldq", 384), k.get("s", P), k.get("qt", P), k.get("ldqt", 256),
        k.get("st", P), None)
    assert f(rows=200) == SHAPE                   # both axes are grouped
    assert f(cols=200, ldx=208, ldq=208) == SHAPE
    assert f(qt=None) == NULL
    assert f(st=None) == NULL
    assert f(qt=P + 8) == ALIGN
    assert f(ldqt=200) == SHAPE
    assert f(ldqt=264) == ALIGN
    assert f(dt=3) == DTYPE
    assert f(rows=0, x=None, q=None, s=None, qt=None, st=None) == OK


def test_quantize_weight_errors(L):
    f = lambda **k: L.bfp8_quantize_weight(
        k.get("x", P), k.get("dt", 0), k.get("rows", 384), k.get("cols", 512),
        k.get("ldx", 512), k.get("q", P), k.get("ldq", 512), k.get("s", P), None)
    assert f(s=None) == NULL
    assert f(ldx=500) == SHAPE
    assert f(q=P + 1) == ALIGN
    assert f(dt=-1) == DTYPE
    assert f(rows=0, x=None, q=None, s=None) == OK


def gemm(L, layout=1, M=256, N=384, K=512, A=P, lda=512, sA=P, ma=0, B=P, ldb=512, sB=P,
         mb=1, C=P, ldc=384, ws=None, wsb=0):
    return L.bfp8_gemm(layout, M, N, K, A, lda, sA, ma, B, ldb, sB, mb, C, ldc, ws, wsb, None)


def test_gemm_errors(L):
    assert gemm(L, layout=3) == LAYOUT
    assert gemm(L, ma=2) == SMODE                 # 1x32 needs E8M0 scales (bfp8_gemm_mx)
    assert gemm(L, ma=4) == SMODE
    assert gemm(L, mb=-1) == SMODE
    assert gemm(L, K=500) == SHAPE
    assert gemm(L, M=-1) == SHAPE
    assert gemm(L, A=None) == NULL
    assert gemm(L, sB=None) == NULL
    assert gemm(L, C=None) == NULL
    assert gemm(L, A=P + 4) == ALIGN
    assert gemm(L, C=P + 2) == ALIGN
    assert gemm(L, ldc=388) == ALIGN
    assert gemm(L, ldc=256) == SHAPE
    assert gemm(L, lda=256) == SHAPE              # NT: A row is K long
    assert gemm(L, lda=520) == ALIGN
    # NN: B stored [K][N], read in place (no workspace)
    assert L.bfp8_gemm_workspace_bytes(0, 0, 1, 256, 384, 512) == 0
    assert gemm(L, layout=0, ldb=256) == SHAPE    # NN: B row is N long
    assert gemm(L, layout=2, lda=128) == SHAPE    # TN: A row is M long
    assert gemm(L, lda=1 << 23) == SHAPE          # beyond 32-bit tile offsets
    # empty problems
    assert gemm(L, M=0, A=None, B=None, C=None) == OK
    assert gemm(L, N=0, A=None, B=None, C=None) == OK


def test_workspace_query(L):
    for layout in (0, 1, 2):
        assert L.bfp8_gemm_workspace_bytes(layout, 0, 1, 8192, 4096, 2048) == 0
    # few output tiles and a long K: fp32 split-K partials are requested
    ws = L.bfp8_gemm_workspace_bytes(1, 0, 0, 2048, 2048, 16384)
    assert ws > 0 and ws % (2048 * 2048 * 4) == 0
    # 48 x 8 tiles: one whole wave of 256 tiles runs unsplit, and only the
    # remaining 16 rows of tiles (4096 output rows) are split (in 2 along K);
    # the partials cover those rows only, for both GEMM entry points (1x32
    # modes exist only for the E8M0 one, which also keeps room to copy the
    # split rows' K-block-major scale bytes: 128 K blocks x 4096 rows)
    assert L.bfp8_gemm_workspace_bytes(1, 2, 2, 12288, 2048, 16384) == 2 * 4096 * 2048 * 4 + 128 * 4096 + 256
    assert L.bfp8_gemm_workspace_bytes(1, 0, 0, 12288, 2048, 16384) == 2 * 4096 * 2048 * 4 + 128 * 4096 + 256
    # 8 x 24 tiles under-fill the GPU but splitting costs more: unsplit
    assert L.bfp8_gemm_workspace_bytes(1, 0, 0, 2048, 6144, 16384) == 0
    assert L.bfp8_gemm_workspace_bytes(1, 2, 2, 2048, 2048, 16384) == 4 * 2048 * 2048 * 4
    assert L.bfp8_gemm_workspace_bytes(3, 0, 1, 1, 1, 128) == ctypes.c_size_t(-1).value
    assert L.bfp8_gemm_workspace_bytes(1, 0, 1, 1, 1, 100) == ctypes.c_size_t(-1).value
    assert L.bfp8_gemm_workspace_bytes(1, 5, 1, 1, 1, 128) == ctypes.c_size_t(-1).value


def test_gemm_rejects_misaligned_workspace(L):
    assert gemm(L, ws=P + 4, wsb=1 << 20) == ALIGN


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        bfp8.lib(str(tmp_path / "missing.so"))


# ---- power-of-two (E8M0) entry points ---------------------------------------

def test_quantize_mx_errors(L):
    f = lambda **k: L.bfp8_quantize_mx_act(
        k.get("x", P), k.get("dt", 0), k.get("rows", 256), k.get("cols", 512),
        k.get("ldx", 512), k.get("group", 32), k.get("q", P), k.get("ldq", 512), k.get("s", P), None)
    assert f(group=64) == SMODE
    assert f(group=0) == SMODE
    assert f(cols=500, ldx=512) == SHAPE
    assert f(s=None) == NULL
    assert f(x=P + 8) == ALIGN
    assert f(dt=5) == DTYPE
    assert f(rows=0, x=None, q=None, s=None) == OK
    t = lambda **k: L.bfp8_quantize_mx_act_transposed(
        k.get("x", P), 0, k.get("rows", 256), 384, 384, k.get("group", 128), P, 256, P, None)
    assert t(group=16) == SMODE
    assert t(rows=100) == SHAPE
    d = lambda **k: L.bfp8_quantize_mx_act_dual(
        P, 0, k.get("rows", 256), 384, 384, k.get("group", 32), P, 384, P, k.get("qt", P), 256,
        P, None)
    assert d(group=256) == SMODE
    assert d(qt=None) == NULL
    w = lambda **k: L.bfp8_quantize_mx_weight(P, k.get("dt", 0), 300, 200, 208, P, 208,
                                              k.get("s", P), None)
    assert w(s=None) == NULL
    assert w(dt=9) == DTYPE


def gemm_mx(L, layout=1, M=256, N=384, K=512, A=P, lda=512, sA=P, ma=0, B=P, ldb=512, sB=P,
            mb=1, C=P, ldc=384, ws=None, wsb=0):
    return L.bfp8_gemm_mx(layout, M, N, K, A, lda, sA, ma, B, ldb, sB, mb, C, ldc, ws, wsb, None)


def test_gemm_mx_errors(L):
    assert gemm_mx(L, layout=4) == LAYOUT
    assert gemm_mx(L, ma=4) == SMODE
    assert gemm_mx(L, layout=2, ma=2, lda=256) == SMODE   # 1x32 A must be K-contiguous
    assert gemm_mx(L, layout=0, mb=2, ldb=384) == SMODE   # 1x32 B must be K-contiguous
    assert gemm_mx(L, K=200) == SHAPE
    assert gemm_mx(L, sA=None) == NULL
    assert gemm_mx(L, sB=P + 1) == ALIGN
    assert gemm_mx(L, M=0, A=None, B=None, C=None) == OK
    assert L.bfp8_gemm_workspace_bytes(1, 2, 2, 8192, 4096, 2048) == 0


def test_static_scratch_gemm_rejects_before_any_launch(L):
    """bfp8_gemm_static_scratch validates like bfp8_gemm and refuses, on the
    host, a problem whose split-K partials exceed the static array."""
    def call(layout=1, M=3072, N=4096, K=65536, A=P, sA=P, ma=0, B=P, sB=P, mb=0, C=P, ldc=4096):
        return L.bfp8_gemm_static_scratch(layout, M, N, K, A, K, sA, ma, B, K, sB, mb, C, ldc,
                                          None)
    assert call(layout=7) == LAYOUT
    assert call(ma=2) == SMODE
    assert call(C=None) == NULL
    assert call(K=100) == SHAPE
    assert bfp8.gemm_workspace_bytes("NT", "act", "act", 3072, 4096, 65536) > bfp8.STATIC_SCRATCH_BYTES
    assert call() == WS
    assert "BFP8_STATIC_SCRATCH_BYTES (64u << 20)" in open(HEADER).read()
    assert bfp8.STATIC_SCRATCH_BYTES == 64 << 20


def test_kmajor_scale_mode_and_quantisers_validate(L):
    """BFP8_SCALE_1x128_KMAJOR (3) is a float32 and an E8M0 mode; the
    K-block-major quantisers reject what the default ones reject."""
    assert "BFP8_SCALE_1x128_KMAJOR = 3" in open(HEADER).read() and bfp8.MODES["act_km"] == 3
    assert bfp8.gemm_workspace_bytes("NT", "act_km", "act_km", 2048, 2048, 16384) == \
        bfp8.gemm_workspace_bytes("NT", "act", "act", 2048, 2048, 16384)
    assert L.bfp8_gemm_workspace_bytes(1, 4, 0, 256, 256, 256) == ctypes.c_size_t(-1).value
    # bfp8_gemm / bfp8_gemm_mx: mode 4 unknown
    args = (1, 256, 256, 256, P, 256, P, 4, P, 256, P, 0, P, 256, None, 0, None)
    assert L.bfp8_gemm(*args) == SMODE and L.bfp8_gemm_mx(*args) == SMODE
    for fn in (L.bfp8_quantize_act_kmajor, L.bfp8_quantize_act_transposed_kmajor):
        assert fn(P, 0, 256, 256, 256, P, 256, None, None) == NULL
        assert fn(P, 7, 256, 256, 256, P, 256, P, None) == DTYPE
    assert L.bfp8_quantize_act_kmajor(P, 0, 256, 100, 256, P, 256, P, None) == SHAPE
    assert L.bfp8_quantize_act_transposed_kmajor(P, 0, 100, 256, 256, P, 256, P, None) == SHAPE
    for fn in (L.bfp8_quantize_act_dual_kmajor, L.bfp8_quantize_mx_act_dual_kmajor):
        assert fn(P, 0, 256, 256, 256, P, 256, P, None, 256, P, None) == NULL
        assert fn(P, 0, 256, 100, 256, P, 256, P, P, 256, P, None) == SHAPE
