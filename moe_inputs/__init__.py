"""Seeded synthetic inputs for the MoE expert layer.

This module draws random arrays of the layer's shapes and, for bf16 workloads,
rounds them to bf16 (round-to-nearest-even).  It holds none of the layer's
arithmetic: both the CPU oracle tests and the HIP path tests/bench read their
inputs from here and nowhere else.

The pages benchmark on random dummy tokens with a balanced routing gate,
sequence length 4,096 and local batch 1 (page "Accelerating Transformers
fine-tuning with NVIDIA NeMo AutoModel", section 单节点30B MoE基准测试, method
table and the note on the routing gate).  The workloads below are synthetic in
the same way; none of them stands in for a dataset.

Stream layout (one numpy ``SeedSequence`` per workload seed):
``SeedSequence(seed).spawn(7)`` -> streams for ``[x, Wr, b, Wg, Wu, Wd, dY]``;
each expert-weight stream is spawned once more into ``E`` children, one per
global expert id, so any subset of experts can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "round_bf16", "bf16_bits", "generate",
           "expert_weights", "small_workload"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    d: int                 # model width
    E: int                 # global expert count
    k: int                 # experts per token
    I: int                 # expert FFN width
    dtype: str             # "f32" or "bf16"
    gate: str              # "softmax_topk" or "balanced"
    seed: int
    x_sigma: float
    w_sigma: float = 0.02
    bias_sigma: Optional[float] = None   # per-expert router bias ~N(0, bias_sigma), fp32
    dy_sigma: float = 1.0
    e_lo: int = 0          # local experts are [e_lo, e_hi)
    e_hi: Optional[int] = None
    backward: bool = False

    @property
    def e_end(self) -> int:
        return self.E if self.e_hi is None else self.e_hi

    @property
    def E_loc(self) -> int:
        return self.e_end - self.e_lo


# The five measured / parity workloads.  Shapes follow the Qwen3-30B-A3B and
# DeepSeek-V3 (one expert-parallel rank of eight) expert layers.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_f32_T64_d128_E8_k2_I256", T=64, d=128, E=8, k=2, I=256,
             dtype="f32", gate="softmax_topk", seed=1, x_sigma=0.02),
    Workload("qwen3_balanced_fwd_T4096_d2048_E128_k8_I768", T=4096, d=2048, E=128,
             k=8, I=768, dtype="bf16", gate="balanced", seed=2, x_sigma=1.0),
    Workload("qwen3_natural_fwd_T4096_d2048_E128_k8_I768", T=4096, d=2048, E=128,
             k=8, I=768, dtype="bf16", gate="softmax_topk", seed=3, x_sigma=1.0,
             bias_sigma=1.5),
    Workload("qwen3_balanced_fwdbwd_T4096_d2048_E128_k8_I768", T=4096, d=2048,
             E=128, k=8, I=768, dtype="bf16", gate="balanced", seed=4, x_sigma=1.0,
             backward=True),
    Workload("dsv3_ep8_rank_fwdbwd_T32768_d7168_E256_loc32_k8_I2048", T=32768,
             d=7168, E=256, k=8, I=2048, dtype="bf16", gate="balanced", seed=5,
             x_sigma=1.0, e_lo=0, e_hi=32, backward=True),
]}


def small_workload(name: str, T: int, d: int, E: int, k: int, I: int, *, dtype="bf16",
                   gate="softmax_topk", seed=11, x_sigma=1.0, w_sigma=0.02,
                   bias_sigma: Optional[float] = None, e_lo=0, e_hi=None,
                   backward=True) -> Workload:
    """A parity-test workload of arbitrary (small) shape."""
    return Workload(name, T=T, d=d, E=E, k=k, I=I, dtype=dtype, gate=gate, seed=seed,
                    x_sigma=x_sigma, w_sigma=w_sigma, bias_sigma=bias_sigma,
                    e_lo=e_lo, e_hi=e_hi, backward=backward)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); float32 out."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns (uint16) of float32 values that are already bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable; call round_bf16 first")
    return (u >> 16).astype(np.uint16).reshape(a.shape)


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(7)


def _normal(ss: np.random.SeedSequence, shape, sigma: float, dtype: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return round_bf16(a) if dtype == "bf16" else a


def expert_weights(w: Workload, which: str, experts: Iterable[int]) -> np.ndarray:
    """Weights of the given GLOBAL expert ids: which in {"Wg", "Wu", "Wd"}.

    Wg, Wu have shape [n, d, I]; Wd has shape [n, I, d]."""
    slot = {"Wg": 3, "Wu": 4, "Wd": 5}[which]
    children = _streams(w.seed)[slot].spawn(w.E)
    shape = (w.d, w.I) if which != "Wd" else (w.I, w.d)
    experts = list(experts)
    out = np.empty((len(experts),) + shape, dtype=np.float32)
    for i, e in enumerate(experts):
        out[i] = _normal(children[e], shape, w.w_sigma, w.dtype)
    return out


def generate(w: Workload, parts: Iterable[str] = ("x", "Wr", "b", "Wg", "Wu", "Wd", "dY")
             ) -> Dict[str, np.ndarray]:
    """Draw the requested arrays (float32 numpy; bf16-valued for bf16 workloads).

    x [T,d]; Wr [d,E]; b [E] (fp32, only when the workload has a router bias);
    Wg, Wu [E_loc,d,I] and Wd [E_loc,I,d] for local experts [e_lo, e_hi);
    dY [T,d] (only for workloads with a backward pass)."""
    s = _streams(w.seed)
    out: Dict[str, np.ndarray] = {}
    parts = set(parts)
    if "x" in parts:
        out["x"] = _normal(s[0], (w.T, w.d), w.x_sigma, w.dtype)
    if "Wr" in parts:
        out["Wr"] = _normal(s[1], (w.d, w.E), w.w_sigma, w.dtype)
    if "b" in parts and w.bias_sigma is not None:
        out["b"] = _normal(s[2], (w.E,), w.bias_sigma, "f32")
    loc = range(w.e_lo, w.e_end)
    for name in ("Wg", "Wu", "Wd"):
        if name in parts:
            out[name] = expert_weights(w, name, loc)
    if "dY" in parts and w.backward:
        out["dY"] = _normal(s[6], (w.T, w.d), w.dy_sigma, w.dtype)
    return out
