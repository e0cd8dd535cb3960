"""Seeded synthetic inputs for the owner-rank step: the five workload shapes,
the initial fp32 shard states and each step's R gradient contributions.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no reduce, no Adam, no overflow logic), so the oracle and
the GPU path can both be fed from it.  Everything is generated with torch on
the requested device from a seeded torch.Generator; the oracle side receives
the same values by copying them to the host.

Workloads follow the pages' model sizes (GPT-2 1.5B, 7.5B, 13B, 128B; the
"AI论文陪读·ZeRO" section 01 and the blog.vllbc.top ZeRO/DeepSpeed worked
examples and Table 1; the fp32 SGD cases of that page's extension group C),
with synthetic values in place of real gradients:
gradients N(0, 1e-3) per contribution times the loss scale, master weights
N(0, 0.02).  N(0, s) means standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    psi: int
    nd: int
    rank: int
    R: int
    bucket_elems: int
    lp: str                   # "fp16", "bf16" or "fp32" (4-byte storage)
    scale: float
    dynamic: int
    lr: float
    weight_decay: float
    steps: int
    grad_std: float = 1e-3
    master_std: float = 0.02
    m_std: float = 0.0
    v_std: float = 0.0
    inject_step: Optional[int] = None     # 0-based step with a +inf in contribution 0
    layout: Optional[str] = None          # tensor layout of the flat buffer, if any
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    opt: str = "adam"                     # "adam" or "sgd"
    momentum: float = 0.0                 # SGD: > 0 keeps a momentum buffer

    @property
    def shard(self) -> int:
        return -(-self.psi // self.nd)

    @property
    def begin(self) -> int:
        return self.rank * self.shard

    @property
    def torch_lp(self):
        return {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}[self.lp]

    @property
    def has_m(self) -> bool:
        """Whether the shard keeps a first-moment / momentum array."""
        return self.opt == "adam" or self.momentum > 0.0

    @property
    def has_v(self) -> bool:
        return self.opt == "adam"


WORKLOADS = {
    "tiny": Workload("tiny: Psi=1,048,576, Nd=4, shard 262,144, R=4, fp16, scale 1024",
                     psi=1_048_576, nd=4, rank=0, R=4, bucket_elems=50_000_000, lp="fp16",
                     scale=1024.0, dynamic=1, lr=1e-3, weight_decay=0.0, steps=3),
    "gpt2_1.5b": Workload("GPT-2 1.5B, Nd=8, shard 187.5M, R=8, C_B 50M, fp16, scale 65536",
                          psi=1_500_000_000, nd=8, rank=0, R=8, bucket_elems=50_000_000,
                          lp="fp16", scale=65536.0, dynamic=1, lr=1e-3, weight_decay=0.01,
                          steps=10),
    "7.5b_bf16": Workload("7.5B, Nd=64, shard 117,187,500, R=8, C_B 50M, bf16, static scale 1",
                          psi=7_500_000_000, nd=64, rank=0, R=8, bucket_elems=50_000_000,
                          lp="bf16", scale=1.0, dynamic=0, lr=1e-4, weight_decay=0.0, steps=10,
                          m_std=1e-4, v_std=1e-8),
    "13b_inf": Workload("13B (40 layers, h=5120, 4x MLP), Nd=16, rank 1, shard 812.5M, R=16, "
                        "C_B 50M, fp16, scale 32768, +inf at step 3",
                        psi=13_000_000_000, nd=16, rank=1, R=16, bucket_elems=50_000_000,
                        lp="fp16", scale=32768.0, dynamic=1, lr=1e-3, weight_decay=0.0,
                        steps=8, inject_step=2, layout="13b"),
    "128b": Workload("128B, Nd=64, shard 2.0e9, R=4, C_B 200M, fp16, scale 4096",
                     psi=128_000_000_000, nd=64, rank=0, R=4, bucket_elems=200_000_000,
                     lp="fp16", scale=4096.0, dynamic=1, lr=6e-5, weight_decay=0.1, steps=5),
    # extension group C of the blog.vllbc.top page: fp32 storage (b = 4)
    "c1_7.5b_sgdm": Workload("C1: 7.5B, Nd=64, shard 117,187,500, R=8, C_B 50M, fp32 SGD with "
                             "momentum 0.9, static scale 1",
                             psi=7_500_000_000, nd=64, rank=0, R=8, bucket_elems=50_000_000,
                             lp="fp32", scale=1.0, dynamic=0, lr=1e-2, weight_decay=1e-4,
                             steps=10, opt="sgd", momentum=0.9),
    "c2_1.5b_sgd": Workload("C2: GPT-2 1.5B, Nd=8, shard 187.5M, R=8, C_B 50M, fp32 plain SGD, "
                            "static scale 1",
                            psi=1_500_000_000, nd=8, rank=0, R=8, bucket_elems=50_000_000,
                            lp="fp32", scale=1.0, dynamic=0, lr=1e-2, weight_decay=0.0,
                            steps=10, opt="sgd"),
}


# ------------------------------------------------------------------ 13B layout

def layout_13b(hidden: int = 5120, layers: int = 40, psi: int = 13_000_000_000
               ) -> List[Tuple[str, int, int]]:
    """(name, start, size) of every tensor of the flattened 13B transformer:
    a 1-D embedding that brings the total to exactly psi, then per layer
    ln1.w, ln1.b, qkv.w, qkv.b, proj.w, proj.b, ln2.w, ln2.b, fc1.w, fc1.b,
    fc2.w, fc2.b (12 h^2 + 13 h parameters per layer)."""
    h = hidden
    per_layer = [("ln1.w", h), ("ln1.b", h), ("qkv.w", 3 * h * h), ("qkv.b", 3 * h),
                 ("proj.w", h * h), ("proj.b", h), ("ln2.w", h), ("ln2.b", h),
                 ("fc1.w", 4 * h * h), ("fc1.b", 4 * h), ("fc2.w", 4 * h * h), ("fc2.b", h)]
    body = layers * sum(s for _, s in per_layer)
    emb = psi - body
    out = [("embed", 0, emb)]
    pos = emb
    for li in range(layers):
        for name, s in per_layer:
            out.append((f"layer{li}.{name}", pos, s))
            pos += s
    assert pos == psi
    return out


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


CHUNK = 1 << 27


def _fill_normal(out: torch.Tensor, std: float, seed: int, absolute: bool = False) -> None:
    """out[:] = N(0, std) (|N(0, std)| if absolute), drawn in fp32 chunks."""
    g = _gen(out.device, seed)
    n = out.numel()
    for off in range(0, n, CHUNK):
        ln = min(CHUNK, n - off)
        x = torch.randn(ln, generator=g, device=out.device, dtype=torch.float32)
        x.mul_(std)
        if absolute:
            x.abs_()
        out[off:off + ln].copy_(x)


def init_state(w: Workload, device, seed: int = 0, elems: Optional[int] = None):
    """fp32 master, m, v of the owner's shard (first `elems` elements)."""
    n = w.shard if elems is None else elems
    master = torch.empty(n, dtype=torch.float32, device=device)
    m = torch.zeros(n, dtype=torch.float32, device=device)
    v = torch.zeros(n, dtype=torch.float32, device=device)
    if w.layout == "13b":
        # per-tensor init: norm weights 1, biases 0, matrices N(0, master_std)
        lo, hi = w.begin, w.begin + n
        for k, (name, start, size) in enumerate(layout_13b(psi=w.psi)):
            a, b = max(lo, start), min(hi, start + size)
            if a >= b:
                continue
            seg = master[a - lo:b - lo]
            kind = name.rsplit(".", 1)[-1]
            if name.endswith("ln1.w") or name.endswith("ln2.w"):
                seg.fill_(1.0)
            elif kind == "b":
                seg.zero_()
            else:
                _fill_normal(seg, w.master_std, seed * 7919 + 17 * k + 1)
    else:
        _fill_normal(master, w.master_std, seed * 7919 + 1)
    if w.m_std:
        _fill_normal(m, w.m_std, seed * 7919 + 2)
    if w.v_std:
        _fill_normal(v, w.v_std, seed * 7919 + 3, absolute=True)
    return master, m, v


def contribution_seed(seed: int, step: int, r: int) -> int:
    return ((seed * 1_000_003 + step) * 131 + r) * 2 + 1


def fill_contribs(w: Workload, bufs: List[torch.Tensor], step: int, scale: float,
                  seed: int = 0) -> None:
    """Fill the R contribution buffers of `step` (0-based) with
    N(0, grad_std) * scale rounded to the buffers' dtype; at the workload's
    inject step,
    contribution 0 gets +inf at element n/2 + 1 of its n elements."""
    for r, b in enumerate(bufs):
        _fill_normal(b, w.grad_std * scale, contribution_seed(seed, step, r))
    if w.inject_step is not None and step == w.inject_step:
        i = inject_index(bufs[0].numel())
        if i < bufs[0].numel():
            bufs[0][i] = float("inf")


def inject_index(n: int) -> int:
    return n // 2 + 1


def alloc_contribs(w: Workload, device, elems: Optional[int] = None,
                   phase_step: int = 16) -> List[torch.Tensor]:
    """R contribution buffers of `elems` (default: shard) elements.  With
    phase_step p < 16, contribution r starts (r * p) mod 16 bytes past a
    16-byte boundary, as contributions carved back to back from one buffer do
    when the shard size is not a multiple of 8 elements (p = 8, 4 or 2; fp32
    data takes 8 or 4)."""
    n = w.shard if elems is None else elems
    if phase_step == 16:
        return [torch.empty(n, dtype=w.torch_lp, device=device) for _ in range(w.R)]
    esz = torch.empty(0, dtype=w.torch_lp).element_size()
    if phase_step not in (8, 4, 2) or phase_step % esz:
        raise ValueError(f"phase_step {phase_step} for {esz}-byte elements")
    out = []
    for r in range(w.R):
        base = torch.empty(n + 16 // esz, dtype=w.torch_lp, device=device)
        k = (r * phase_step) % 16 // esz
        out.append(base[k:k + n])
    return out
