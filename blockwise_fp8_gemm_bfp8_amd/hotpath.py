"""One training pass of the blockwise-FP8 linear layers, on preallocated buffers.

For each Transformer linear y = x W^T (W stored [out][in]) the pass runs, per
the Puro-2B paper translation (papers.lianghsun.dev), section 3.2:
  fprop:  quantize_act(x), quantize_weight(W), gemm NT     -> y  [M][out]
  dgrad:  quantize_act(dy), gemm NN with W's codes as stored -> dx [M][in]
  wgrad:  quantize_act_transposed(dy), quantize_act_transposed(x),
          gemm NT on the two token-grouped operands          -> dW [out][in]
where a tensor needed in both layouts is read once (quantize_act_dual), all
the weights are quantised in one launch (quantize_weight_batch), and the
activation / gradient scales are kept K-block major (the _kmajor quantisers,
GEMM scale mode 'act_km'; the 1x32 groups keep their one layout).
All buffers (codes, scales, outputs, split-K workspaces) are allocated once, so a
pass only enqueues kernels on the current stream.  The pass is kept as a list of
kernel calls with the work each does (flops, algorithmic bytes), which is what
the benchmark times call by call.  This module only calls the binding; every
step runs in libbfp8's kernels.

`scales` selects the scale format:
  "fp32"  float32 amax/448 scales, per-128-K promotion on the VALU (the above);
  "mx128" the same groups with power-of-two E8M0 scales (the translation,
          section 3.2: the SM120 runs constrained block scales to powers of
          two), applied by the scaled MFMA;
  "mx32"  MXFP8: 1x32 power-of-two groups along K for every operand (the
          tutorial's MXFP figure); the weight is quantised along both axes
          (its in-features groups feed fprop, its out-features groups dgrad),
          so all three GEMMs are NT.
"""

import ctypes
import sys
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Tuple

import torch

from . import (MAX_WEIGHT_JOBS, _scale_bytes, gemm, gemm_mx, gemm_workspace_bytes,
               quantize_act_dual_kmajor, quantize_act_kmajor, quantize_act_transposed_kmajor,
               quantize_mx_act_dual, quantize_mx_act_dual_kmajor, quantize_mx_weight_batch,
               quantize_weight_batch)

SCALE_FORMATS = ("fp32", "mx128", "mx32")

_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hip_rt = None


def _hip():
    """The HIP runtime torch has loaded (its SONAME is libamdhip64.so.7, so this
    dlopen returns that same instance and its streams are torch's)."""
    global _hip_rt
    if _hip_rt is None:
        torch.cuda.init()
        h = ctypes.CDLL("libamdhip64.so.7")
        vp = ctypes.c_void_p
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        h.hipEventRecord.argtypes = [vp, vp]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        h.hipEventDestroy.argtypes = [vp]
        _hip_rt = h
    return _hip_rt


class TimingEvent:
    """A HIP event used only to time kernels, created with
    hipEventDisableSystemFence.  torch.cuda.Event records with a system-scope
    fence, whose cache writeback and invalidation leave the GPU idle for about
    6 us per record between two kernels; a pass timed GEMM by GEMM records 24
    of them.  Same interface as torch.cuda.Event for record/elapsed_time."""

    def __init__(self):
        self._h = _hip()
        self.ev = ctypes.c_void_p()
        rc = self._h.hipEventCreateWithFlags(ctypes.byref(self.ev), _HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        rc = self._h.hipEventRecord(self.ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = ctypes.c_float()
        rc = self._h.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self, _finalizing=sys.is_finalizing):
        # at interpreter exit the HIP runtime (and this module's globals) may
        # already be torn down
        if self.ev and not _finalizing():
            self._h.hipEventDestroy(self.ev)
        self.ev = ctypes.c_void_p()


@dataclass
class LinearState:
    name: str
    x: torch.Tensor                      # [M][in]
    w: torch.Tensor                      # [out][in]
    dy: Optional[torch.Tensor] = None    # [M][out]
    buf: Dict[str, torch.Tensor] = field(default_factory=dict)


@dataclass
class Op:
    """One kernel call of the pass, with the work it does.

    kind: 'gemm', 'quant' (activation / gradient quantiser) or 'weight_quant'.
    flops: 2MNK for a GEMM (0 otherwise).  bytes: the algorithmic HBM bytes
    -- inputs read once, codes and scales written once (for a GEMM: both code
    operands, their scales and the bf16 output).  feeds: for a quantiser, the
    GEMMs whose operands it writes, with the share of its time charged to
    each (a dual quantiser serves two GEMMs, half each).  codes: for a GEMM,
    its two code operands as passed (A, B), for comparisons on the same
    bytes.  src: for a quantiser, the tensors it reads."""

    label: str
    kind: str
    fn: Callable[[], None]
    flops: int = 0
    bytes: int = 0
    layout: str = ""
    mnk: Tuple[int, int, int] = (0, 0, 0)
    feeds: List[Tuple[str, float]] = field(default_factory=list)
    codes: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
    src: Tuple[torch.Tensor, ...] = ()


def _esize(t: torch.Tensor) -> int:
    return t.element_size()


class HotPath:
    """Preallocated fprop/dgrad/wgrad pass over a list of linear layers.

    The pass is a fixed list of kernel calls (`ops`) on preallocated buffers;
    run() enqueues them in order on the current stream."""

    def __init__(self, tensors: Dict[str, torch.Tensor], names: List[str], roles: List[str],
                 scales: str = "fp32"):
        if scales not in SCALE_FORMATS:
            raise ValueError(f"scales must be one of {SCALE_FORMATS}")
        self.scales = scales
        self.roles = list(roles)
        if scales != "fp32" and set(self.roles) != {"fprop", "dgrad", "wgrad"}:
            raise ValueError("the power-of-two passes run the full fprop + dgrad + wgrad step")
        self.layers: List[LinearState] = []
        for n in names:
            L = LinearState(n, tensors["x." + n], tensors["w." + n], tensors.get("dy." + n))
            self._alloc(L)
            self.layers.append(L)
        self.ops: List[Op] = self._build_ops() if scales == "fp32" else self._build_ops_mx()

    def run(self, events: Optional[list] = None):
        """Enqueue one full pass on the current stream.  With `events` (a
        list), each kernel call is bracketed by a pair of TimingEvents and
        (op index, start, end) is appended."""
        if events is None:
            for op in self.ops:
                op.fn()
            return
        for i, op in enumerate(self.ops):
            s, e = TimingEvent(), TimingEvent()
            s.record()
            op.fn()
            e.record()
            events.append((i, s, e))

    def _alloc(self, L: LinearState):
        if self.scales != "fp32":
            return self._alloc_mx(L)
        dev = L.x.device
        M, din = L.x.shape
        dout = L.w.shape[0]
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
        b = L.buf
        b["wq"] = torch.empty((dout, din), dtype=u8, device=dev)
        b["ws"] = torch.empty(((dout + 127) // 128, din // 128), dtype=f32, device=dev)
        # activation / gradient scales K-block major ([K/128][rows]): each
        # quantiser tile writes its scales as one run, each GEMM K block
        # reads them as a few cache lines
        if "fprop" in self.roles:
            b["xq"] = torch.empty((M, din), dtype=u8, device=dev)
            b["xs"] = torch.empty((din // 128, M), dtype=f32, device=dev)
            b["y"] = torch.empty((M, dout), dtype=bf, device=dev)
        if "dgrad" in self.roles:
            b["dyq"] = torch.empty((M, dout), dtype=u8, device=dev)
            b["dys"] = torch.empty((dout // 128, M), dtype=f32, device=dev)
            b["dx"] = torch.empty((M, din), dtype=bf, device=dev)
        if "wgrad" in self.roles:
            b["dyqt"] = torch.empty((dout, M), dtype=u8, device=dev)
            b["dyst"] = torch.empty((M // 128, dout), dtype=f32, device=dev)
            b["xqt"] = torch.empty((din, M), dtype=u8, device=dev)
            b["xst"] = torch.empty((M // 128, din), dtype=f32, device=dev)
            b["dw"] = torch.empty((dout, din), dtype=bf, device=dev)
            nb = gemm_workspace_bytes("NT", "act_km", "act_km", dout, din, M)
            b["ws_wgrad"] = torch.empty((max(nb, 16),), dtype=u8, device=dev)

    def _alloc_mx(self, L: LinearState):
        """Buffers of the power-of-two passes (E8M0 scale bytes)."""
        dev = L.x.device
        M, din = L.x.shape
        dout = L.w.shape[0]
        u8, bf = torch.uint8, torch.bfloat16
        grp = 32 if self.scales == "mx32" else 128
        b = L.buf
        b["wq"] = torch.empty((dout, din), dtype=u8, device=dev)
        if grp == 32:
            b["ws"] = _scale_bytes(dout, din // 32, dev)
            b["wqt"] = torch.empty((din, dout), dtype=u8, device=dev)
            b["wst"] = _scale_bytes(din, dout // 32, dev)
        else:
            b["ws"] = _scale_bytes((dout + 127) // 128, (din + 127) // 128, dev)
        # group 128: scale bytes K-block major ([K/128][rows]); group 32 keeps
        # [rows][K/32] (the only layout of mode mx32)
        km = grp == 128
        b["xq"] = torch.empty((M, din), dtype=u8, device=dev)
        b["xs"] = _scale_bytes(din // grp, M, dev) if km else _scale_bytes(M, din // grp, dev)
        b["xqt"] = torch.empty((din, M), dtype=u8, device=dev)
        b["xst"] = _scale_bytes(M // grp, din, dev) if km else _scale_bytes(din, M // grp, dev)
        b["y"] = torch.empty((M, dout), dtype=bf, device=dev)
        b["dyq"] = torch.empty((M, dout), dtype=u8, device=dev)
        b["dys"] = _scale_bytes(dout // grp, M, dev) if km else _scale_bytes(M, dout // grp, dev)
        b["dyqt"] = torch.empty((dout, M), dtype=u8, device=dev)
        b["dyst"] = _scale_bytes(M // grp, dout, dev) if km else _scale_bytes(dout, M // grp, dev)
        b["dx"] = torch.empty((M, din), dtype=bf, device=dev)
        b["dw"] = torch.empty((dout, din), dtype=bf, device=dev)
        mode = "mx32" if grp == 32 else "act_km"
        nb = gemm_workspace_bytes("NT", mode, mode, dout, din, M)
        b["ws_wgrad"] = torch.empty((max(nb, 16),), dtype=u8, device=dev)

    # ---- the pass as a list of kernel calls ---------------------------------

    def _build_ops(self) -> List[Op]:
        """float32 scales.  When a pass has both fprop and wgrad, X is
        quantised once into both layouts (the token-grouped codes are kept
        for wgrad, FP8 being the activation storage format); likewise dY
        serves dgrad and wgrad from one read.  Every weight's 128x128 blocks
        are quantised in one launch (the weights are independent of the rest
        of the pass)."""
        ops: List[Op] = []
        roles = self.roles
        both_x = "fprop" in roles and "wgrad" in roles
        both_dy = "dgrad" in roles and "wgrad" in roles
        for i in range(0, len(self.layers), MAX_WEIGHT_JOBS):
            group = self.layers[i:i + MAX_WEIGHT_JOBS]
            nbytes = sum(L.w.numel() * (_esize(L.w) + 1) + L.buf["ws"].numel() * 4 for L in group)
            ops.append(Op("weights", "weight_quant",
                          lambda g=group: quantize_weight_batch(
                              [L.w for L in g], [L.buf["wq"] for L in g],
                              [L.buf["ws"] for L in g]), bytes=nbytes,
                          src=tuple(L.w for L in group)))

        def gemm_op(L, role, layout, a, sa, b, sb, ma, mb, out, M, N, K, ws=None):
            nbytes = a.numel() + b.numel() + 4 * (sa.numel() + sb.numel()) + 2 * M * N
            fn = (lambda: gemm(layout, a, sa, b, sb, ma, mb, out=out, workspace=ws)) if ws is not None \
                else (lambda: gemm(layout, a, sa, b, sb, ma, mb, out=out))
            return Op(f"{L.name}.{role}", "gemm", fn, flops=2 * M * N * K, bytes=nbytes,
                      layout=layout, mnk=(M, N, K), codes=(a, b))

        for L in self.layers:
            b = L.buf
            M, din = L.x.shape
            dout = L.w.shape[0]
            e = _esize(L.x)
            if "fprop" in roles:
                if both_x:
                    ops.append(Op(f"{L.name}.x dual", "quant",
                                  lambda L=L, b=b: quantize_act_dual_kmajor(
                                      L.x, b["xq"], b["xs"], b["xqt"], b["xst"]),
                                  bytes=M * din * (e + 2) + 4 * (b["xs"].numel() + b["xst"].numel()),
                                  feeds=[(f"{L.name}.fprop", 0.5), (f"{L.name}.wgrad", 0.5)],
                                  src=(L.x,)))
                else:
                    ops.append(Op(f"{L.name}.x act", "quant",
                                  lambda L=L, b=b: quantize_act_kmajor(L.x, b["xq"], b["xs"]),
                                  bytes=M * din * (e + 1) + 4 * b["xs"].numel(),
                                  feeds=[(f"{L.name}.fprop", 1.0)], src=(L.x,)))
                ops.append(gemm_op(L, "fprop", "NT", b["xq"], b["xs"], b["wq"], b["ws"], "act_km",
                                   "block", b["y"], M, dout, din))
        for L in self.layers:
            b = L.buf
            M, din = L.x.shape
            dout = L.w.shape[0]
            e = _esize(L.x)
            if both_dy:
                ops.append(Op(f"{L.name}.dy dual", "quant",
                              lambda L=L, b=b: quantize_act_dual_kmajor(
                                  L.dy, b["dyq"], b["dys"], b["dyqt"], b["dyst"]),
                              bytes=M * dout * (e + 2) + 4 * (b["dys"].numel() + b["dyst"].numel()),
                              feeds=[(f"{L.name}.dgrad", 0.5), (f"{L.name}.wgrad", 0.5)],
                              src=(L.dy,)))
            elif "dgrad" in roles:
                ops.append(Op(f"{L.name}.dy act", "quant",
                              lambda L=L, b=b: quantize_act_kmajor(L.dy, b["dyq"], b["dys"]),
                              bytes=M * dout * (e + 1) + 4 * b["dys"].numel(),
                              feeds=[(f"{L.name}.dgrad", 1.0)], src=(L.dy,)))
            elif "wgrad" in roles:
                ops.append(Op(f"{L.name}.dy transposed", "quant",
                              lambda L=L, b=b: quantize_act_transposed_kmajor(
                                  L.dy, b["dyqt"], b["dyst"]),
                              bytes=M * dout * (e + 1) + 4 * b["dyst"].numel(),
                              feeds=[(f"{L.name}.wgrad", 1.0)], src=(L.dy,)))
            if "dgrad" in roles:
                ops.append(gemm_op(L, "dgrad", "NN", b["dyq"], b["dys"], b["wq"], b["ws"],
                                   "act_km", "block", b["dx"], M, din, dout))
            if "wgrad" in roles:
                if not both_x:
                    ops.append(Op(f"{L.name}.x transposed", "quant",
                                  lambda L=L, b=b: quantize_act_transposed_kmajor(
                                      L.x, b["xqt"], b["xst"]),
                                  bytes=M * din * (e + 1) + 4 * b["xst"].numel(),
                                  feeds=[(f"{L.name}.wgrad", 1.0)], src=(L.x,)))
                ops.append(gemm_op(L, "wgrad", "NT", b["dyqt"], b["dyst"], b["xqt"], b["xst"],
                                   "act_km", "act_km", b["dw"], dout, din, M,
                                   ws=b["ws_wgrad"]))
        return ops

    def _build_ops_mx(self) -> List[Op]:
        """One fprop + dgrad + wgrad pass with power-of-two scales.  Every
        activation / gradient is quantised once into both layouts; with 1x32
        groups the weight is too (in-features groups for fprop, out-features
        groups for dgrad), otherwise its 128x128 blocks serve both GEMMs."""
        grp = 32 if self.scales == "mx32" else 128
        mode = "mx32" if grp == 32 else "act_km"
        ops: List[Op] = []

        def gemm_op(L, role, layout, a, sa, b, sb, ma, mb, out, M, N, K, ws=None):
            nbytes = a.numel() + b.numel() + sa.numel() + sb.numel() + 2 * M * N
            fn = (lambda: gemm_mx(layout, a, sa, b, sb, ma, mb, out=out, workspace=ws)) \
                if ws is not None else (lambda: gemm_mx(layout, a, sa, b, sb, ma, mb, out=out))
            return Op(f"{L.name}.{role}", "gemm", fn, flops=2 * M * N * K, bytes=nbytes,
                      layout=layout, mnk=(M, N, K), codes=(a, b))

        if grp == 128:
            for i in range(0, len(self.layers), MAX_WEIGHT_JOBS):
                group = self.layers[i:i + MAX_WEIGHT_JOBS]
                nbytes = sum(L.w.numel() * (_esize(L.w) + 1) + L.buf["ws"].numel() for L in group)
                ops.append(Op("weights", "weight_quant",
                              lambda g=group: quantize_mx_weight_batch(
                                  [L.w for L in g], [L.buf["wq"] for L in g],
                                  [L.buf["ws"] for L in g]), bytes=nbytes,
                          src=tuple(L.w for L in group)))
        for L in self.layers:
            b = L.buf
            M, din = L.x.shape
            dout = L.w.shape[0]
            e = _esize(L.x)
            if grp == 32:
                ops.append(Op(f"{L.name}.w dual", "weight_quant",
                              lambda L=L, b=b: quantize_mx_act_dual(L.w, 32, b["wq"], b["ws"],
                                                                    b["wqt"], b["wst"]),
                              bytes=L.w.numel() * (e + 2) + b["ws"].numel() + b["wst"].numel(),
                              src=(L.w,)))
                wmode = "mx32"
            else:
                wmode = "block"
            ops.append(Op(f"{L.name}.x dual", "quant",
                          (lambda L=L, b=b: quantize_mx_act_dual_kmajor(
                              L.x, b["xq"], b["xs"], b["xqt"], b["xst"])) if grp == 128 else
                          (lambda L=L, b=b: quantize_mx_act_dual(L.x, grp, b["xq"], b["xs"],
                                                                 b["xqt"], b["xst"])),
                          bytes=M * din * (e + 2) + b["xs"].numel() + b["xst"].numel(),
                          feeds=[(f"{L.name}.fprop", 0.5), (f"{L.name}.wgrad", 0.5)], src=(L.x,)))
            ops.append(gemm_op(L, "fprop", "NT", b["xq"], b["xs"], b["wq"], b["ws"], mode, wmode,
                               b["y"], M, dout, din))
        for L in self.layers:
            b = L.buf
            M, din = L.x.shape
            dout = L.w.shape[0]
            e = _esize(L.x)
            ops.append(Op(f"{L.name}.dy dual", "quant",
                          (lambda L=L, b=b: quantize_mx_act_dual_kmajor(
                              L.dy, b["dyq"], b["dys"], b["dyqt"], b["dyst"])) if grp == 128 else
                          (lambda L=L, b=b: quantize_mx_act_dual(L.dy, grp, b["dyq"], b["dys"],
                                                                 b["dyqt"], b["dyst"])),
                          bytes=M * dout * (e + 2) + b["dys"].numel() + b["dyst"].numel(),
                          feeds=[(f"{L.name}.dgrad", 0.5), (f"{L.name}.wgrad", 0.5)], src=(L.dy,)))
            if grp == 32:
                ops.append(gemm_op(L, "dgrad", "NT", b["dyq"], b["dys"], b["wqt"], b["wst"], mode,
                                   "mx32", b["dx"], M, din, dout))
            else:
                ops.append(gemm_op(L, "dgrad", "NN", b["dyq"], b["dys"], b["wq"], b["ws"], mode,
                                   "block", b["dx"], M, din, dout))
            ops.append(gemm_op(L, "wgrad", "NT", b["dyqt"], b["dyst"], b["xqt"], b["xst"], mode,
                               mode, b["dw"], dout, din, M, ws=b["ws_wgrad"]))
        return ops
