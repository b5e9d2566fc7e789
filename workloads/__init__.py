"""Seeded synthetic inputs for the blockwise-FP8 linear-layer workloads.

This module only draws random tensors and describes shapes; it holds none of
the quantisation or GEMM arithmetic.  Both the CPU oracle and the HIP path
receive the tensors produced here (the HIP side after a copy to the device),
so both see identical bytes.

Shapes follow the model and batch geometry on the pages:
  * Puro-2B tutorial (bloombook.cn), hardware/architecture section: hidden
    size 2048, 16 query + 8 KV heads (head dim 128, derived), FFN 6144;
  * Puro-2B paper translation (papers.lianghsun.dev), section 2 and
    section 3.1.3: sequence length 4096, micro-batch size 2, so one
    micro-batch holds M = 8192 tokens.
Distributions (readings; the pages do not fix them): activations N(0,1) with a
seeded 0.5% of feature columns multiplied by 50 (the pages only say that
outliers exist, section 3.2); weights N(0, 0.02); activation gradients
N(0, 1e-3); the full-layer workload uses unscaled Student-t(3) activations.
Everything is drawn on the CPU with torch.Generator and cast to bfloat16
(float32 for the tiny workload).
"""

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import torch

HIDDEN = 2048
FFN = 6144
QKV_OUT = 2048 + 1024 + 1024  # 16 q heads + 8 k heads + 8 v heads, x128
TOKENS_PER_MICROBATCH = 2 * 4096


@dataclass(frozen=True)
class Linear:
    """One Transformer linear layer y = x W^T with W stored [out][in]."""

    name: str
    in_features: int
    out_features: int


@dataclass(frozen=True)
class GemmSpec:
    """One GEMM of the hot path.

    role: 'fprop' (Y = X W^T, layout NT), 'dgrad' (dX = dY W, layout NN) or
    'wgrad' (dW = dY^T X, layout NT on token-axis-quantised operands).
    """

    linear: Linear
    role: str
    tokens: int

    @property
    def layout(self) -> str:
        return "NN" if self.role == "dgrad" else "NT"

    @property
    def mnk(self) -> Tuple[int, int, int]:
        L, M = self.linear, self.tokens
        if self.role == "fprop":
            return (M, L.out_features, L.in_features)
        if self.role == "dgrad":
            return (M, L.in_features, L.out_features)
        return (L.out_features, L.in_features, M)

    @property
    def flops(self) -> int:
        m, n, k = self.mnk
        return 2 * m * n * k


@dataclass
class Workload:
    name: str
    description: str
    tokens: int
    seed: int
    dtype: torch.dtype
    linears: List[Linear]
    roles: List[str]
    act_dist: str  # 'normal_outliers' | 'student_t3' | 'normal'
    gemms: List[GemmSpec] = field(default_factory=list)

    def __post_init__(self):
        self.gemms = [GemmSpec(l, r, self.tokens) for r in ("fprop", "dgrad", "wgrad")
                      if r in self.roles for l in self.linears]

    @property
    def flops(self) -> int:
        return sum(g.flops for g in self.gemms)


QKV = Linear("qkv", HIDDEN, QKV_OUT)
O_PROJ = Linear("o_proj", HIDDEN, HIDDEN)
GATE_UP = Linear("gate_up", HIDDEN, 2 * FFN)
DOWN = Linear("down", FFN, HIDDEN)

WORKLOADS: Dict[str, Workload] = {
    "tiny_256x512x384": Workload(
        "tiny_256x512x384",
        "X 256x512 fp32 N(0,1), W [384][512] fp32 N(0,0.02), seed 0; fprop NT",
        256, 0, torch.float32, [Linear("tiny", 512, 384)], ["fprop"], "normal"),
    "qkv_fprop_m8192": Workload(
        "qkv_fprop_m8192",
        "Puro-2B fused QKV fprop, X [8192][2048] bf16 with outlier channels",
        TOKENS_PER_MICROBATCH, 1, torch.bfloat16, [QKV], ["fprop"], "normal_outliers"),
    "mlp_fprop_m8192": Workload(
        "mlp_fprop_m8192",
        "Puro-2B MLP fprop: gate/up 2048->12288 and down 6144->2048 at M=8192",
        TOKENS_PER_MICROBATCH, 2, torch.bfloat16, [GATE_UP, DOWN], ["fprop"],
        "normal_outliers"),
    "down_backward_m8192": Workload(
        "down_backward_m8192",
        "Puro-2B down-proj dgrad (NN) and wgrad (NT, token-axis groups) at M=8192",
        TOKENS_PER_MICROBATCH, 3, torch.bfloat16, [DOWN], ["dgrad", "wgrad"],
        "normal_outliers"),
    "layer_fwd_bwd_m16384": Workload(
        "layer_fwd_bwd_m16384",
        "One Puro-2B decoder layer's four linears, fprop+dgrad+wgrad at M=16384, "
        "Student-t(3) activations",
        16384, 4, torch.bfloat16, [QKV, O_PROJ, GATE_UP, DOWN],
        ["fprop", "dgrad", "wgrad"], "student_t3"),
}

# The order the workloads are listed in the task's configuration table.
WORKLOAD_ORDER = list(WORKLOADS)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal(shape, std, gen, dtype=torch.bfloat16):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(dtype)


def normal_with_outliers(shape, gen, dtype=torch.bfloat16, frac=0.005, factor=50.0):
    """N(0,1) with round(frac*C) seeded feature columns scaled by ``factor``."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    c = shape[-1]
    n_out = int(round(frac * c))
    cols = torch.randperm(c, generator=gen)[:n_out]
    x[:, cols] *= factor
    return x.to(dtype)


def student_t3(shape, gen, dtype=torch.bfloat16):
    """Standard Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3)."""
    z = torch.randn(shape, generator=gen, dtype=torch.float32)
    v = torch.zeros(shape, dtype=torch.float32)
    for _ in range(3):
        e = torch.randn(shape, generator=gen, dtype=torch.float32)
        v.addcmul_(e, e)
    return (z / torch.sqrt(v / 3.0)).to(dtype)


def _activation(w: Workload, shape, gen):
    if w.act_dist == "normal":
        return normal(shape, 1.0, gen, w.dtype)
    if w.act_dist == "normal_outliers":
        return normal_with_outliers(shape, gen, w.dtype)
    if w.act_dist == "student_t3":
        return student_t3(shape, gen, w.dtype)
    raise ValueError(w.act_dist)


def make_inputs(name: str, seed: int = None) -> Dict[str, torch.Tensor]:
    """Draw every tensor a workload needs, in a fixed order, on the CPU.

    Keys: 'x.<linear>' [M][in], 'w.<linear>' [out][in], and for backward
    workloads 'dy.<linear>' [M][out].  Draw order: activations of every
    linear, then weights, then gradients, linears in listed order.
    """
    w = WORKLOADS[name]
    gen = _gen(w.seed if seed is None else seed)
    out: Dict[str, torch.Tensor] = {}
    M = w.tokens
    for L in w.linears:
        out["x." + L.name] = _activation(w, (M, L.in_features), gen)
    for L in w.linears:
        out["w." + L.name] = normal((L.out_features, L.in_features), 0.02, gen, w.dtype)
    if "dgrad" in w.roles or "wgrad" in w.roles:
        for L in w.linears:
            out["dy." + L.name] = normal((M, L.out_features), 1e-3, gen, w.dtype)
    return out


def bf16_bits(t: torch.Tensor):
    """Raw bfloat16 bit patterns of a CPU tensor as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def to_numpy_input(t: torch.Tensor):
    """CPU tensor -> numpy array the oracle accepts (float32, or bf16 bits)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.contiguous().numpy()
