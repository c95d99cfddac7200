"""Seeded synthetic inputs shaped like the pages' attention workloads.

The pages measure on random-normal Q/K/V tensors in the (B, T, N, H) layout
(codelab "Speed up attention on GPU with cuDNN and TransformerEngine",
sections 3, 8, 9 and 10); no dataset is involved.  This module only draws and
casts numbers: it holds none of the attention arithmetic, and both the tests
(for the oracle and the HIP path) and the benchmark use it.

Draw rule: numpy PCG64 generator seeded with 1000 * config + case; Q, K, V, dO
are float32 N(0, 1) drawn in that order, then the per-head sink logits alpha
(float32 N(0, 1)), then the per-batch lengths.  Casting to bf16 is torch's
round-to-nearest-even; the oracle receives the cast values upcast exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Problem:
    """One attention problem: shapes, mask, softmax variant and dtype."""
    B: int
    S: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    dtype: str = "bf16"             # "bf16" or "f32"
    causal: bool = True
    window: tuple = (-1, -1)        # (left, right); -1 = unbounded
    softmax_type: str = "vanilla"   # "vanilla" | "off_by_one" | "learnable"
    scale_factor: float = 0.0       # 0 => 1/sqrt(d_qk)
    seqlen_range: tuple | None = None  # (lo, hi) inclusive => padded batches
    name: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return self.scale_factor if self.scale_factor else 1.0 / math.sqrt(self.d_qk)

    def with_(self, **kw) -> "Problem":
        return replace(self, **kw)


def workload_configs() -> dict:
    """The five workloads: tiny fp32 causal GQA; GQA+SWA S=4096; the MHA/GQA/MQA
    sweep; MLA-style head dims 192/128; sink attention with padding."""
    cfg = {
        1: [Problem(1, 128, 4, 2, 64, 64, "f32", True, (-1, -1), "vanilla", 0.125,
                    name="tiny causal GQA fp32")],
        2: [Problem(4, 4096, 32, 8, 128, 128, "bf16", True, (1024, 0), "vanilla",
                    name="GQA+SWA S=4096")],
        3: [],
        4: [Problem(2, 4096, 128, 128, 192, 128, "bf16", True, (-1, -1), "vanilla",
                    1.0 / math.sqrt(192), name="MLA head dims 192/128")],
        5: [Problem(4, 8192, 32, 8, 128, 128, "bf16", True, (4096, 0), st,
                    seqlen_range=(4096, 8192), name=f"sink {st} + padding")
            for st in ("off_by_one", "learnable")],
    }
    for hkv in (16, 4, 1):
        for b, s in ((32, 512), (16, 1024), (8, 2048), (4, 4096), (2, 8192), (1, 16384)):
            cfg[3].append(Problem(b, s, 16, hkv, 64, 64, "bf16", True, (-1, -1), "vanilla",
                                  name=f"sweep Hkv={hkv} B={b} S={s}"))
    return cfg


def draw(p: Problem, seed: int) -> dict:
    """Float32 draws for problem p: q, k, v, do, alpha [Hq], seqlens [B] or None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((p.B, p.S, p.Hq, p.d_qk), dtype=np.float32)
    k = rng.standard_normal((p.B, p.S, p.Hkv, p.d_qk), dtype=np.float32)
    v = rng.standard_normal((p.B, p.S, p.Hkv, p.d_v), dtype=np.float32)
    do = rng.standard_normal((p.B, p.S, p.Hq, p.d_v), dtype=np.float32)
    alpha = rng.standard_normal((p.Hq,), dtype=np.float32)
    seqlens = None
    if p.seqlen_range is not None:
        lo, hi = p.seqlen_range
        seqlens = rng.integers(lo, hi, size=(p.B,), endpoint=True).astype(np.int32)
    return {"q": q, "k": k, "v": v, "do": do, "alpha": alpha, "seqlens": seqlens}


def to_torch(arrays: dict, dtype: str, device="cpu") -> dict:
    """Cast the float32 draws to the problem dtype (bf16 round-to-nearest-even)."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    out = {}
    for name in ("q", "k", "v", "do"):
        out[name] = torch.from_numpy(arrays[name]).to(tdt).to(device).contiguous()
    out["alpha"] = torch.from_numpy(arrays["alpha"]).to(device)
    s = arrays["seqlens"]
    out["seqlens"] = None if s is None else torch.from_numpy(s).to(device)
    return out


def exact_f64(t) -> np.ndarray:
    """Exact float64 copy of a (bf16 or f32) torch tensor's values."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def pack(arrays: dict, seg_sizes) -> dict:
    """Packed (THD) copy of BSHD draws: segment b is the first seg_sizes[b]
    token rows of batch b; segments lie back to back along one token axis,
    followed by `tail` extra rows (zeros) that belong to no segment when
    arrays holds a "tail" entry.  Adds seq_offsets [B+1] (int32).  Pure data
    movement: no attention arithmetic."""
    sizes = [int(n) for n in seg_sizes]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    tail = int(arrays.get("tail", 0))
    out = dict(arrays)
    for name in ("q", "k", "v", "do"):
        x = arrays[name]
        parts = [x[b, :n] for b, n in enumerate(sizes)]
        parts.append(np.zeros((tail,) + x.shape[2:], dtype=x.dtype))
        out[name] = np.concatenate(parts, axis=0)
    out["seq_offsets"] = off
    return out


def to_torch_packed(arrays: dict, dtype: str, device="cpu") -> dict:
    """to_torch for packed arrays (adds seq_offsets)."""
    import torch
    out = to_torch(arrays, dtype, device)
    out["seq_offsets"] = torch.from_numpy(arrays["seq_offsets"]).to(device)
    return out
