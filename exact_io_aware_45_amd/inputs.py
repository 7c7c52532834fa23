"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: it only draws random tensors and
builds tile masks.  Both the HIP path and the CPU oracle are fed from it.

Recipe (the pages measure on no public dataset for this path; every input is
synthetic):
  * Q, K, V (and dO for the backward) are drawn i.i.d. N(0, 1) in float32 from
    one CPU ``torch.Generator`` seeded with ``seed``, in the order Q, K, V, dO,
    each shaped [B, H, N, d], then rounded to the working dtype (bf16 by
    round-to-nearest-even, or kept float32).
  * fp8 inputs: the same fp32 draws stored as OCP e4m3 codes with one
    per-tensor descale amax / 448 (``qkv_fp8``).
  * The block-sparse tile mask is the symmetric diagonal band |qb - kb| <= band
    plus off-band tiles drawn uniformly without replacement (a CPU generator
    seeded ``seed + 1000``) until ``round(density * nb * nb)`` tiles are set.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype and mask structure."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "bf16" or "f32"
    causal: bool
    backward: bool = False
    sparse: bool = False
    band: int = 1
    density: float = 0.125
    mask_block: int = 128
    Hkv: int = 0  # K/V heads (grouped-head runs); 0: one per query head

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


# The five problem shapes the method is checked and measured on.
WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 128, 64, "f32", False),
    "batched_d64": Workload("batched_d64", 8, 16, 1024, 64, "bf16", False),
    "batched_d64_causal": Workload("batched_d64_causal", 8, 16, 1024, 64, "bf16", True),
    "long_d128_causal": Workload("long_d128_causal", 1, 32, 8192, 128, "bf16", True),
    "bwd_d128_causal": Workload("bwd_d128_causal", 4, 16, 4096, 128, "bf16", True, backward=True),
    "blocksparse_d64": Workload("blocksparse_d64", 1, 16, 16384, 64, "bf16", False, sparse=True),
}


def qkv(B: int, H: int, N: int, d: int, dtype=torch.bfloat16, seed: int = 0,
        with_dout: bool = False, device="cpu"):
    """Q, K, V (and dO) i.i.d. N(0,1), drawn in fp32 on the CPU, then cast.

    Returns a tuple of contiguous tensors on ``device``.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    names = 4 if with_dout else 3
    out = []
    for _ in range(names):
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(t.to(dtype).contiguous().to(device))
    return tuple(out)


FP8_MAX = 448.0  # largest finite OCP e4m3 value


def qkv_fp8(B: int, H: int, N: int, d: int, seed: int = 0, device="cpu"):
    """Q, K, V drawn exactly as ``qkv`` draws them (fp32), then stored as OCP
    e4m3 codes (torch.float8_e4m3fn) with one fp32 descale per tensor,
    descale = amax / 448, so that code * descale approximates the draw.

    Returns [(q_codes, q_descale), (k_codes, k_descale), (v_codes, v_descale)].
    """
    out = []
    for t in qkv(B, H, N, d, torch.float32, seed):
        amax = float(t.abs().max())
        descale = float(torch.tensor(amax / FP8_MAX if amax > 0 else 1.0, dtype=torch.float32))
        codes = (t / descale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
        out.append((codes.contiguous().to(device), descale))
    return out


def block_mask(N: int, mask_block: int = 128, band: int = 1, density: float = 0.125,
               seed: int = 0, device="cpu") -> torch.Tensor:
    """uint8 tile mask [nb][nb]: a diagonal band plus seeded random off-band tiles."""
    nb = -(-N // mask_block)
    idx = torch.arange(nb)
    m = ((idx[:, None] - idx[None, :]).abs() <= band)
    target = int(round(density * nb * nb))
    off = (~m).flatten().nonzero().flatten()
    extra = max(0, min(target - int(m.sum()), off.numel()))
    if extra:
        g = torch.Generator(device="cpu").manual_seed(int(seed) + 1000)
        pick = off[torch.randperm(off.numel(), generator=g)[:extra]]
        flat = m.flatten().clone()
        flat[pick] = True
        m = flat.view(nb, nb)
    return m.to(torch.uint8).contiguous().to(device)


def workload_inputs(w: Workload, seed: int = 0, device="cpu"):
    """Inputs of one workload: dict with q, k, v (dout if backward, mask if sparse)."""
    t = qkv(w.B, w.H, w.N, w.d, w.torch_dtype, seed, with_dout=w.backward, device=device)
    out = {"q": t[0], "k": t[1], "v": t[2]}
    if w.backward:
        out["dout"] = t[3]
    if w.sparse:
        out["mask"] = block_mask(w.N, w.mask_block, w.band, w.density, seed, device=device)
    return out
