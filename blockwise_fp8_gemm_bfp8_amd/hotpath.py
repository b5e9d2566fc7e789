"""One training pass of the blockwise-FP8 linear layers, on preallocated buffers.

For each Transformer linear y = x W^T (W stored [out][in]) the pass runs, per
the Puro-2B paper translation (papers.lianghsun.dev), section 3.2:
  fprop:  quantize_act(x), quantize_weight(W), gemm NT     -> y  [M][out]
  dgrad:  quantize_act(dy), gemm NN with W's codes as stored -> dx [M][in]
  wgrad:  quantize_act_transposed(dy), quantize_act_transposed(x),
          gemm NT on the two token-grouped operands          -> dW [out][in]
where a tensor needed in both layouts is read once (quantize_act_dual), and
all the weights are quantised in one launch (quantize_weight_batch).
All buffers (codes, scales, outputs, split-K workspaces) are allocated once, so a
pass only enqueues kernels on the current stream.  This module only calls
the binding; every step runs in libbfp8's kernels.

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
from typing import Dict, List, Optional

import torch

from . import (MAX_WEIGHT_JOBS, _scale_bytes, gemm, gemm_mx, gemm_workspace_bytes, quantize_act,
               quantize_act_dual, quantize_act_transposed, quantize_mx_act_dual,
               quantize_mx_weight_batch, quantize_weight_batch)

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

    def __del__(self):
        # at interpreter exit the HIP runtime may already be torn down
        if self.ev and not sys.is_finalizing():
            self._h.hipEventDestroy(self.ev)
        self.ev = ctypes.c_void_p()


@dataclass
class LinearState:
    name: str
    x: torch.Tensor                      # [M][in]
    w: torch.Tensor                      # [out][in]
    dy: Optional[torch.Tensor] = None    # [M][out]
    buf: Dict[str, torch.Tensor] = field(default_factory=dict)


class HotPath:
    """Preallocated fprop/dgrad/wgrad pass over a list of linear layers."""

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
        self.gemm_events = None

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
        if "fprop" in self.roles:
            b["xq"] = torch.empty((M, din), dtype=u8, device=dev)
            b["xs"] = torch.empty((M, din // 128), dtype=f32, device=dev)
            b["y"] = torch.empty((M, dout), dtype=bf, device=dev)
        if "dgrad" in self.roles:
            b["dyq"] = torch.empty((M, dout), dtype=u8, device=dev)
            b["dys"] = torch.empty((M, dout // 128), dtype=f32, device=dev)
            b["dx"] = torch.empty((M, din), dtype=bf, device=dev)
        if "wgrad" in self.roles:
            b["dyqt"] = torch.empty((dout, M), dtype=u8, device=dev)
            b["dyst"] = torch.empty((dout, M // 128), dtype=f32, device=dev)
            b["xqt"] = torch.empty((din, M), dtype=u8, device=dev)
            b["xst"] = torch.empty((din, M // 128), dtype=f32, device=dev)
            b["dw"] = torch.empty((dout, din), dtype=bf, device=dev)
            nb = gemm_workspace_bytes("NT", "act", "act", dout, din, M)
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
        b["xq"] = torch.empty((M, din), dtype=u8, device=dev)
        b["xs"] = _scale_bytes(M, din // grp, dev)
        b["xqt"] = torch.empty((din, M), dtype=u8, device=dev)
        b["xst"] = _scale_bytes(din, M // grp, dev)
        b["y"] = torch.empty((M, dout), dtype=bf, device=dev)
        b["dyq"] = torch.empty((M, dout), dtype=u8, device=dev)
        b["dys"] = _scale_bytes(M, dout // grp, dev)
        b["dyqt"] = torch.empty((dout, M), dtype=u8, device=dev)
        b["dyst"] = _scale_bytes(dout, M // grp, dev)
        b["dx"] = torch.empty((M, din), dtype=bf, device=dev)
        b["dw"] = torch.empty((dout, din), dtype=bf, device=dev)
        mode = "mx32" if grp == 32 else "act"
        nb = gemm_workspace_bytes("NT", mode, mode, dout, din, M)
        b["ws_wgrad"] = torch.empty((max(nb, 16),), dtype=u8, device=dev)

    def _gemm(self, *args, **kw):
        fn = gemm if self.scales == "fp32" else gemm_mx
        ev = self.gemm_events
        if ev is not None:
            s = TimingEvent()
            e = TimingEvent()
            s.record()
            out = fn(*args, **kw)
            e.record()
            ev.append((s, e))
            return out
        return fn(*args, **kw)

    def run(self):
        """Enqueue one full pass (every quantiser and GEMM) on the current stream.

        When a pass has both fprop and wgrad, X is quantised once into both
        layouts (the token-grouped codes are kept for wgrad, FP8 being the
        activation storage format); likewise dY serves dgrad and wgrad from
        one read."""
        if self.scales != "fp32":
            return self._run_mx()
        both_x = "fprop" in self.roles and "wgrad" in self.roles
        both_dy = "dgrad" in self.roles and "wgrad" in self.roles
        # every weight's 128x128 blocks in one launch (the weights are
        # independent of the rest of the pass)
        for i in range(0, len(self.layers), MAX_WEIGHT_JOBS):
            group = self.layers[i:i + MAX_WEIGHT_JOBS]
            quantize_weight_batch([L.w for L in group], [L.buf["wq"] for L in group],
                                  [L.buf["ws"] for L in group])
        for L in self.layers:
            b = L.buf
            if "fprop" in self.roles:
                if both_x:
                    quantize_act_dual(L.x, b["xq"], b["xs"], b["xqt"], b["xst"])
                else:
                    quantize_act(L.x, b["xq"], b["xs"])
                self._gemm("NT", b["xq"], b["xs"], b["wq"], b["ws"], "act", "block", out=b["y"])
        for L in self.layers:
            b = L.buf
            if both_dy:
                quantize_act_dual(L.dy, b["dyq"], b["dys"], b["dyqt"], b["dyst"])
            elif "dgrad" in self.roles:
                quantize_act(L.dy, b["dyq"], b["dys"])
            elif "wgrad" in self.roles:
                quantize_act_transposed(L.dy, b["dyqt"], b["dyst"])
            if "dgrad" in self.roles:
                self._gemm("NN", b["dyq"], b["dys"], b["wq"], b["ws"], "act", "block",
                           out=b["dx"])
            if "wgrad" in self.roles:
                if not both_x:
                    quantize_act_transposed(L.x, b["xqt"], b["xst"])
                self._gemm("NT", b["dyqt"], b["dyst"], b["xqt"], b["xst"], "act", "act",
                           out=b["dw"], workspace=b["ws_wgrad"])

    def _run_mx(self):
        """One fprop + dgrad + wgrad pass with power-of-two scales.  Every
        activation / gradient is quantised once into both layouts; with 1x32
        groups the weight is too (in-features groups for fprop, out-features
        groups for dgrad), otherwise its 128x128 blocks serve both GEMMs."""
        grp = 32 if self.scales == "mx32" else 128
        mode = "mx32" if grp == 32 else "act"
        if grp == 128:
            for i in range(0, len(self.layers), MAX_WEIGHT_JOBS):
                group = self.layers[i:i + MAX_WEIGHT_JOBS]
                quantize_mx_weight_batch([L.w for L in group], [L.buf["wq"] for L in group],
                                         [L.buf["ws"] for L in group])
        for L in self.layers:
            b = L.buf
            if grp == 32:
                quantize_mx_act_dual(L.w, 32, b["wq"], b["ws"], b["wqt"], b["wst"])
                wmode = "mx32"
            else:
                wmode = "block"
            quantize_mx_act_dual(L.x, grp, b["xq"], b["xs"], b["xqt"], b["xst"])
            self._gemm("NT", b["xq"], b["xs"], b["wq"], b["ws"], mode, wmode, out=b["y"])
        for L in self.layers:
            b = L.buf
            quantize_mx_act_dual(L.dy, grp, b["dyq"], b["dys"], b["dyqt"], b["dyst"])
            if grp == 32:
                self._gemm("NT", b["dyq"], b["dys"], b["wqt"], b["wst"], mode, "mx32", out=b["dx"])
            else:
                self._gemm("NN", b["dyq"], b["dys"], b["wq"], b["ws"], mode, "block", out=b["dx"])
            self._gemm("NT", b["dyqt"], b["dyst"], b["xqt"], b["xst"], mode, mode, out=b["dw"],
                       workspace=b["ws_wgrad"])
