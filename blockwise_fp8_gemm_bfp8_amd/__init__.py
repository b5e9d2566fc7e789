"""Python binding of libbfp8: blockwise FP8 (E4M3) linear layers on MI355X.

Argument marshalling only: every step runs in the HIP kernels of libbfp8.so
(built in-tree by ``blockwise_fp8_gemm_bfp8_amd.build``).  PyTorch supplies
device memory and the current stream; nothing here computes.  If the
library is missing the first call raises -- there is no fallback path.

Functions (same names as the C ABI in include/bfp8.h, without the prefix):
  quantize_act(x)               -> (q uint8 [R][C], s f32 [R][C/128])
  quantize_act_transposed(x)    -> (qt uint8 [C][M], st f32 [C][M/128])
  quantize_act_dual(x)          -> (q, s, qt, st): both of the above from one read
  quantize_weight(w)            -> (q uint8 [R][C], s f32 [ceil(R/128)][ceil(C/128)])
  quantize_weight_batch(ws)     -> [(q, s), ...]: several weights in one launch
  gemm(layout, qa, sa, qb, sb, mode_a, mode_b) -> bf16 [M][N]
Power-of-two (E8M0) scales, group 32 or 128 (scales are uint8 tensors):
  quantize_mx_act(x, group)            -> (q, s u8 [R][C/group])
  quantize_mx_act_transposed(x, group) -> (qt, st u8 [C][M/group])
  quantize_mx_act_dual(x, group)       -> (q, s, qt, st)
  quantize_mx_weight(w)                -> (q, s u8 [ceil(R/128)][ceil(C/128)])
  quantize_mx_weight_batch(ws)         -> [(q, s), ...]: several weights in one launch
  gemm_mx(layout, qa, sa, qb, sb, mode_a, mode_b) -> bf16 [M][N]
    (modes 'act' = 1x128, 'block' = 128x128, 'mx32' = 1x32, 'act_km' = 1x128 with the
    scale tensor stored K-block major, [K/128][rows])
K-block-major scale variants (the layout of mode 'act_km'):
  quantize_act_kmajor, quantize_act_transposed_kmajor, quantize_act_dual_kmajor,
  quantize_mx_act_dual_kmajor
"""

import ctypes
import os

import torch

from .build import LIB_PATH

__all__ = [
    "quantize_act",
    "quantize_act_dual",
    "quantize_act_transposed",
    "quantize_act_kmajor",
    "quantize_act_transposed_kmajor",
    "quantize_act_dual_kmajor",
    "quantize_mx_act_dual_kmajor",
    "quantize_weight",
    "quantize_weight_batch",
    "gemm",
    "gemm_workspace_bytes",
    "gemm_static_scratch",
    "STATIC_SCRATCH_BYTES",
    "quantize_mx_act",
    "quantize_mx_act_transposed",
    "quantize_mx_act_dual",
    "quantize_mx_weight",
    "quantize_mx_weight_batch",
    "gemm_mx",
    "lib",
    "BFP8Error",
    "STATUS",
    "LAYOUTS",
    "MODES",
]

STATUS = {
    0: "BFP8_OK",
    1: "BFP8_ERR_NULL",
    2: "BFP8_ERR_SHAPE",
    3: "BFP8_ERR_ALIGN",
    4: "BFP8_ERR_DTYPE",
    5: "BFP8_ERR_LAYOUT",
    6: "BFP8_ERR_SCALE_MODE",
    7: "BFP8_ERR_WORKSPACE",
    8: "BFP8_ERR_HIP",
    9: "BFP8_ERR_NONFINITE",
}
LAYOUTS = {"NN": 0, "NT": 1, "TN": 2}
MODES = {"act": 0, "block": 1, "mx32": 2, "act_km": 3}
DTYPES = {torch.bfloat16: 0, torch.float32: 1}

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int

_SIGNATURES = {
    "bfp8_quantize_act": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
    "bfp8_quantize_act_transposed": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
    "bfp8_quantize_weight": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
    "bfp8_quantize_weight_batch": [_vp, _int, _int, _vp],
    "bfp8_quantize_act_dual": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp],
    "bfp8_quantize_act_kmajor": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
    "bfp8_quantize_act_transposed_kmajor": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
    "bfp8_quantize_act_dual_kmajor": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64,
                                      _vp, _vp],
    "bfp8_quantize_mx_act_dual_kmajor": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64,
                                         _vp, _vp],
    "bfp8_gemm": [_int, _i64, _i64, _i64, _vp, _i64, _vp, _int, _vp, _i64, _vp, _int, _vp,
                  _i64, _vp, ctypes.c_size_t, _vp],
    "bfp8_gemm_workspace_bytes": [_int, _int, _int, _i64, _i64, _i64],
    "bfp8_quantize_mx_act": [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _vp],
    "bfp8_quantize_mx_act_transposed": [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _vp],
    "bfp8_quantize_mx_act_dual": [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _vp, _i64,
                                  _vp, _vp],
    "bfp8_quantize_mx_weight": [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
    "bfp8_quantize_mx_weight_batch": [_vp, _int, _int, _vp],
    "bfp8_gemm_mx": [_int, _i64, _i64, _i64, _vp, _i64, _vp, _int, _vp, _i64, _vp, _int, _vp,
                     _i64, _vp, ctypes.c_size_t, _vp],
    "bfp8_gemm_static_scratch": [_int, _i64, _i64, _i64, _vp, _i64, _vp, _int, _vp, _i64, _vp,
                                 _int, _vp, _i64, _vp],
    "bfp8_status_str": [_int],
    "bfp8_abi_version": [],
}
_RESTYPES = {
    "bfp8_gemm_workspace_bytes": ctypes.c_size_t,
    "bfp8_status_str": ctypes.c_char_p,
}

MAX_WEIGHT_JOBS = 16  # BFP8_MAX_WEIGHT_JOBS
STATIC_SCRATCH_BYTES = 64 << 20  # BFP8_STATIC_SCRATCH_BYTES


class WeightJob(ctypes.Structure):
    """bfp8_weight_job, and bfp8_mx_weight_job (the same layout; s points at
    E8M0 bytes there)."""
    _fields_ = [("w", _vp), ("rows", _i64), ("cols", _i64), ("ldw", _i64), ("q", _vp),
                ("ldq", _i64), ("s", _vp)]


_lib = None


class BFP8Error(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = lib().bfp8_status_str(code).decode()
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({msg})")


def lib(path: str = None):
    """Load libbfp8.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"libbfp8 not built ({p} missing); run `python -m blockwise_fp8_gemm_bfp8_amd.build`")
    handle = ctypes.CDLL(p)
    for name, args in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, ctypes.c_int)
    if path is None:
        _lib = handle
    return handle


def _padded_empty(rows: int, cols: int, dtype, device, align_elems: int):
    """[rows][cols] view of a buffer whose rows start 16-byte aligned."""
    ld = max(-(-cols // align_elems) * align_elems, align_elems)
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :cols]


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn, code):
    if code != 0:
        raise BFP8Error(fn, code)


def _check_input(x: torch.Tensor, name: str):
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if x.dtype not in DTYPES:
        raise ValueError(f"{name} must be bfloat16 or float32, got {x.dtype}")
    if x.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last axis")


def quantize_act(x: torch.Tensor, q: torch.Tensor = None, s: torch.Tensor = None):
    """1x128 groups along rows; see bfp8_quantize_act."""
    _check_input(x, "x")
    R, C = x.shape
    if q is None:
        q = _padded_empty(R, C, torch.uint8, x.device, 16)
    if s is None:
        s = torch.empty((R, max(C // 128, 0)), dtype=torch.float32, device=x.device)
    _check("bfp8_quantize_act", lib().bfp8_quantize_act(
        x.data_ptr(), DTYPES[x.dtype], R, C, x.stride(0), q.data_ptr(), q.stride(0),
        s.data_ptr(), _stream(x)))
    return q, s


def quantize_act_transposed(x: torch.Tensor, qt: torch.Tensor = None, st: torch.Tensor = None):
    """Token-axis 1x128 groups written transposed; see bfp8_quantize_act_transposed."""
    _check_input(x, "x")
    M, C = x.shape
    if qt is None:
        qt = _padded_empty(C, M, torch.uint8, x.device, 16)
    if st is None:
        st = torch.empty((C, max(M // 128, 0)), dtype=torch.float32, device=x.device)
    _check("bfp8_quantize_act_transposed", lib().bfp8_quantize_act_transposed(
        x.data_ptr(), DTYPES[x.dtype], M, C, x.stride(0), qt.data_ptr(), qt.stride(0),
        st.data_ptr(), _stream(x)))
    return qt, st


def quantize_act_dual(x: torch.Tensor, q=None, s=None, qt=None, st=None):
    """Row-grouped and token-grouped (transposed) codes from one read; see
    bfp8_quantize_act_dual.  Returns (q, s, qt, st)."""
    _check_input(x, "x")
    M, C = x.shape
    if q is None:
        q = _padded_empty(M, C, torch.uint8, x.device, 16)
    if s is None:
        s = torch.empty((M, max(C // 128, 0)), dtype=torch.float32, device=x.device)
    if qt is None:
        qt = _padded_empty(C, M, torch.uint8, x.device, 16)
    if st is None:
        st = torch.empty((C, max(M // 128, 0)), dtype=torch.float32, device=x.device)
    _check("bfp8_quantize_act_dual", lib().bfp8_quantize_act_dual(
        x.data_ptr(), DTYPES[x.dtype], M, C, x.stride(0), q.data_ptr(), q.stride(0),
        s.data_ptr(), qt.data_ptr(), qt.stride(0), st.data_ptr(), _stream(x)))
    return q, s, qt, st


def quantize_act_kmajor(x: torch.Tensor, q=None, s=None):
    """1x128 groups along rows, scales stored [C/128][R]; see bfp8_quantize_act_kmajor."""
    _check_input(x, "x")
    R, C = x.shape
    if q is None:
        q = _padded_empty(R, C, torch.uint8, x.device, 16)
    if s is None:
        s = torch.empty((max(C // 128, 0), R), dtype=torch.float32, device=x.device)
    _check("bfp8_quantize_act_kmajor", lib().bfp8_quantize_act_kmajor(
        x.data_ptr(), DTYPES[x.dtype], R, C, x.stride(0), q.data_ptr(), q.stride(0),
        s.data_ptr(), _stream(x)))
    return q, s


def quantize_act_transposed_kmajor(x: torch.Tensor, qt=None, st=None):
    """Token-axis groups written transposed, scales stored [M/128][C]; see
    bfp8_quantize_act_transposed_kmajor."""
    _check_input(x, "x")
    M, C = x.shape
    if qt is None:
        qt = _padded_empty(C, M, torch.uint8, x.device, 16)
    if st is None:
        st = torch.empty((max(M // 128, 0), C), dtype=torch.float32, device=x.device)
    _check("bfp8_quantize_act_transposed_kmajor", lib().bfp8_quantize_act_transposed_kmajor(
        x.data_ptr(), DTYPES[x.dtype], M, C, x.stride(0), qt.data_ptr(), qt.stride(0),
        st.data_ptr(), _stream(x)))
    return qt, st


def quantize_act_dual_kmajor(x: torch.Tensor, q=None, s=None, qt=None, st=None):
    """Both layouts from one read, scales K-block major (s [C/128][M],
    st [M/128][C]); see bfp8_quantize_act_dual_kmajor.  Returns (q, s, qt, st)."""
    _check_input(x, "x")
    M, C = x.shape
    if q is None:
        q = _padded_empty(M, C, torch.uint8, x.device, 16)
    if s is None:
        s = torch.empty((max(C // 128, 0), M), dtype=torch.float32, device=x.device)
    if qt is None:
        qt = _padded_empty(C, M, torch.uint8, x.device, 16)
    if st is None:
        st = torch.empty((max(M // 128, 0), C), dtype=torch.float32, device=x.device)
    _check("bfp8_quantize_act_dual_kmajor", lib().bfp8_quantize_act_dual_kmajor(
        x.data_ptr(), DTYPES[x.dtype], M, C, x.stride(0), q.data_ptr(), q.stride(0),
        s.data_ptr(), qt.data_ptr(), qt.stride(0), st.data_ptr(), _stream(x)))
    return q, s, qt, st


def _weight_batch(fn, ws, qs, ss, scale_dtype):
    ws = list(ws)
    if len(ws) > MAX_WEIGHT_JOBS:
        raise ValueError(f"at most {MAX_WEIGHT_JOBS} weights per batch")
    if not ws:
        return []
    qs = list(qs) if qs is not None else [None] * len(ws)
    ss = list(ss) if ss is not None else [None] * len(ws)
    if len(qs) != len(ws) or len(ss) != len(ws):
        raise ValueError("qs and ss must match ws in length")
    dt = ws[0].dtype
    jobs = (WeightJob * len(ws))()
    out = []
    for i, w in enumerate(ws):
        _check_input(w, f"ws[{i}]")
        if w.dtype != dt or w.device != ws[0].device:
            raise ValueError("all weights of a batch share dtype and device")
        R, C = w.shape
        q = qs[i] if qs[i] is not None else _padded_empty(R, C, torch.uint8, w.device, 16)
        s = ss[i] if ss[i] is not None else torch.empty(((R + 127) // 128, (C + 127) // 128),
                                                         dtype=scale_dtype, device=w.device)
        jobs[i] = WeightJob(w.data_ptr(), R, C, w.stride(0), q.data_ptr(), q.stride(0),
                            s.data_ptr())
        out.append((q, s))
    _check(fn, getattr(lib(), fn)(ctypes.cast(jobs, _vp), len(ws), DTYPES[dt], _stream(ws[0])))
    return out


def quantize_weight_batch(ws, qs=None, ss=None):
    """128x128 blocks of several weights (same dtype, same device) in one
    launch; see bfp8_quantize_weight_batch.  Returns [(q, s), ...]."""
    return _weight_batch("bfp8_quantize_weight_batch", ws, qs, ss, torch.float32)


def quantize_weight(w: torch.Tensor, q: torch.Tensor = None, s: torch.Tensor = None):
    """128x128 blocks; see bfp8_quantize_weight."""
    _check_input(w, "w")
    R, C = w.shape
    if q is None:
        q = _padded_empty(R, C, torch.uint8, w.device, 16)
    if s is None:
        s = torch.empty(((R + 127) // 128, (C + 127) // 128), dtype=torch.float32,
                        device=w.device)
    _check("bfp8_quantize_weight", lib().bfp8_quantize_weight(
        w.data_ptr(), DTYPES[w.dtype], R, C, w.stride(0), q.data_ptr(), q.stride(0),
        s.data_ptr(), _stream(w)))
    return q, s


def gemm_dims(layout: str, qa: torch.Tensor, qb: torch.Tensor):
    """(M, N, K) from the stored operand shapes and the layout letters."""
    if layout[0] == "N":
        M, K = qa.shape
    else:
        K, M = qa.shape
    if layout[1] == "T":
        N, Kb = qb.shape
    else:
        Kb, N = qb.shape
    if Kb != K:
        raise ValueError(f"K mismatch: A gives {K}, B gives {Kb}")
    return M, N, K


def gemm_workspace_bytes(layout: str, mode_a: str, mode_b: str, M: int, N: int, K: int) -> int:
    return int(lib().bfp8_gemm_workspace_bytes(LAYOUTS[layout], MODES[mode_a], MODES[mode_b],
                                               M, N, K))


def gemm(layout: str, qa, sa, qb, sb, mode_a: str = "act", mode_b: str = "block",
         out: torch.Tensor = None, workspace: torch.Tensor = None, split_k: bool = True):
    """Blockwise FP8 GEMM -> bf16 [M][N]; see bfp8_gemm for layouts and scales.

    A split-K workspace is allocated when the library asks for one and none
    (or too small a one) is passed; ``split_k=False`` passes no workspace,
    which makes the library run the GEMM unsplit."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    M, N, K = gemm_dims(layout, qa, qb)
    for name, sc in (("sa", sa), ("sb", sb)):
        if not sc.is_contiguous() or sc.dtype != torch.float32:
            raise ValueError(f"{name} must be a dense float32 tensor")
    if out is None:
        out = _padded_empty(M, N, torch.bfloat16, qa.device, 8)
    ws_bytes = gemm_workspace_bytes(layout, mode_a, mode_b, M, N, K) if split_k else 0
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=qa.device)
    _check("bfp8_gemm", lib().bfp8_gemm(
        LAYOUTS[layout], M, N, K, qa.data_ptr(), qa.stride(0), sa.data_ptr(), MODES[mode_a],
        qb.data_ptr(), qb.stride(0), sb.data_ptr(), MODES[mode_b], out.data_ptr(),
        out.stride(0), workspace.data_ptr() if ws_bytes else None, ws_bytes, _stream(qa)))
    return out


def gemm_static_scratch(layout: str, qa, sa, qb, sb, mode_a: str = "act",
                        mode_b: str = "block", out: torch.Tensor = None):
    """bfp8_gemm with its split-K partials in the library's static device
    array (no workspace, no allocation inside the library); see
    bfp8_gemm_static_scratch.  Raises BFP8Error (BFP8_ERR_WORKSPACE) when the
    problem's partials exceed STATIC_SCRATCH_BYTES."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    M, N, K = gemm_dims(layout, qa, qb)
    for name, sc in (("sa", sa), ("sb", sb)):
        if not sc.is_contiguous() or sc.dtype != torch.float32:
            raise ValueError(f"{name} must be a dense float32 tensor")
    if out is None:
        out = _padded_empty(M, N, torch.bfloat16, qa.device, 8)
    _check("bfp8_gemm_static_scratch", lib().bfp8_gemm_static_scratch(
        LAYOUTS[layout], M, N, K, qa.data_ptr(), qa.stride(0), sa.data_ptr(), MODES[mode_a],
        qb.data_ptr(), qb.stride(0), sb.data_ptr(), MODES[mode_b], out.data_ptr(),
        out.stride(0), _stream(qa)))
    return out


# ---- power-of-two (E8M0) scales --------------------------------------------

def _scale_bytes(rows: int, cols: int, device):
    """Dense uint8 [rows][cols] scale tensor with 4 readable bytes of slack
    past its end (the GEMM fetches scales as aligned 32-bit words)."""
    n = rows * cols
    return torch.empty((n + 4,), dtype=torch.uint8, device=device)[:n].view(rows, cols)


def quantize_mx_act(x: torch.Tensor, group: int = 128, q=None, s=None):
    """Power-of-two scales, groups of `group` along rows; see bfp8_quantize_mx_act."""
    _check_input(x, "x")
    R, C = x.shape
    if q is None:
        q = _padded_empty(R, C, torch.uint8, x.device, 16)
    if s is None:
        s = _scale_bytes(R, max(C // group, 0), x.device)
    _check("bfp8_quantize_mx_act", lib().bfp8_quantize_mx_act(
        x.data_ptr(), DTYPES[x.dtype], R, C, x.stride(0), group, q.data_ptr(), q.stride(0),
        s.data_ptr(), _stream(x)))
    return q, s


def quantize_mx_act_transposed(x: torch.Tensor, group: int = 128, qt=None, st=None):
    """Power-of-two scales, token groups written transposed; see
    bfp8_quantize_mx_act_transposed."""
    _check_input(x, "x")
    M, C = x.shape
    if qt is None:
        qt = _padded_empty(C, M, torch.uint8, x.device, 16)
    if st is None:
        st = _scale_bytes(C, max(M // group, 0), x.device)
    _check("bfp8_quantize_mx_act_transposed", lib().bfp8_quantize_mx_act_transposed(
        x.data_ptr(), DTYPES[x.dtype], M, C, x.stride(0), group, qt.data_ptr(), qt.stride(0),
        st.data_ptr(), _stream(x)))
    return qt, st


def quantize_mx_act_dual(x: torch.Tensor, group: int = 128, q=None, s=None, qt=None, st=None):
    """Both power-of-two layouts from one read; returns (q, s, qt, st)."""
    _check_input(x, "x")
    M, C = x.shape
    if q is None:
        q = _padded_empty(M, C, torch.uint8, x.device, 16)
    if s is None:
        s = _scale_bytes(M, max(C // group, 0), x.device)
    if qt is None:
        qt = _padded_empty(C, M, torch.uint8, x.device, 16)
    if st is None:
        st = _scale_bytes(C, max(M // group, 0), x.device)
    _check("bfp8_quantize_mx_act_dual", lib().bfp8_quantize_mx_act_dual(
        x.data_ptr(), DTYPES[x.dtype], M, C, x.stride(0), group, q.data_ptr(), q.stride(0),
        s.data_ptr(), qt.data_ptr(), qt.stride(0), st.data_ptr(), _stream(x)))
    return q, s, qt, st


def quantize_mx_act_dual_kmajor(x: torch.Tensor, q=None, s=None, qt=None, st=None):
    """Power-of-two scales, group 128, both layouts from one read with the
    scale bytes K-block major (s [C/128][M], st [M/128][C]); see
    bfp8_quantize_mx_act_dual_kmajor.  Returns (q, s, qt, st)."""
    _check_input(x, "x")
    M, C = x.shape
    if q is None:
        q = _padded_empty(M, C, torch.uint8, x.device, 16)
    if s is None:
        s = _scale_bytes(max(C // 128, 0), M, x.device)
    if qt is None:
        qt = _padded_empty(C, M, torch.uint8, x.device, 16)
    if st is None:
        st = _scale_bytes(max(M // 128, 0), C, x.device)
    _check("bfp8_quantize_mx_act_dual_kmajor", lib().bfp8_quantize_mx_act_dual_kmajor(
        x.data_ptr(), DTYPES[x.dtype], M, C, x.stride(0), q.data_ptr(), q.stride(0),
        s.data_ptr(), qt.data_ptr(), qt.stride(0), st.data_ptr(), _stream(x)))
    return q, s, qt, st


def quantize_mx_weight(w: torch.Tensor, q=None, s=None):
    """128x128 blocks with power-of-two scales; see bfp8_quantize_mx_weight."""
    _check_input(w, "w")
    R, C = w.shape
    if q is None:
        q = _padded_empty(R, C, torch.uint8, w.device, 16)
    if s is None:
        s = _scale_bytes((R + 127) // 128, (C + 127) // 128, w.device)
    _check("bfp8_quantize_mx_weight", lib().bfp8_quantize_mx_weight(
        w.data_ptr(), DTYPES[w.dtype], R, C, w.stride(0), q.data_ptr(), q.stride(0),
        s.data_ptr(), _stream(w)))
    return q, s



def quantize_mx_weight_batch(ws, qs=None, ss=None):
    """Power-of-two 128x128 blocks of several weights in one launch; see
    bfp8_quantize_mx_weight_batch.  Returns [(q, s u8), ...]."""
    return _weight_batch("bfp8_quantize_mx_weight_batch", ws, qs, ss, torch.uint8)

def gemm_mx(layout: str, qa, sa, qb, sb, mode_a: str = "act", mode_b: str = "block",
            out: torch.Tensor = None, workspace: torch.Tensor = None, split_k: bool = True):
    """GEMM on E8M0-scaled operands -> bf16 [M][N]; see bfp8_gemm_mx."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    M, N, K = gemm_dims(layout, qa, qb)
    for name, sc in (("sa", sa), ("sb", sb)):
        if not sc.is_contiguous() or sc.dtype != torch.uint8:
            raise ValueError(f"{name} must be a dense uint8 (E8M0) tensor")
    if out is None:
        out = _padded_empty(M, N, torch.bfloat16, qa.device, 8)
    ws_bytes = gemm_workspace_bytes(layout, mode_a, mode_b, M, N, K) if split_k else 0
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=qa.device)
    _check("bfp8_gemm_mx", lib().bfp8_gemm_mx(
        LAYOUTS[layout], M, N, K, qa.data_ptr(), qa.stride(0), sa.data_ptr(), MODES[mode_a],
        qb.data_ptr(), qb.stride(0), sb.data_ptr(), MODES[mode_b], out.data_ptr(),
        out.stride(0), workspace.data_ptr() if ws_bytes else None, ws_bytes, _stream(qa)))
    return out
