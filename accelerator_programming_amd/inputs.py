"""Seeded synthetic attention workloads.

This module only draws random numbers and names shapes; it holds none of the
attention arithmetic. Both the HIP path's callers and the oracle's callers
take their inputs from here, so both sides see identical bits.

Recipe (the pages fix no random generator, so this is the reading used):
torch CPU ``Generator(seed)`` -> ``randn`` in fp32, drawing Q, then K, then V,
each [B, H, N, d] contiguous; bf16 workloads round that fp32 draw to bf16
(round-to-nearest-even, torch's ``.to(torch.bfloat16)``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    dqk: int
    dv: int
    causal: bool
    dtype: torch.dtype
    seed: int
    k_mult: float = 1.0          # K scaled after the draw (exact in bf16 for 2.0)
    v_from_k: bool = False       # V is the first dv columns of K (a strided view)
    scale: float = field(default=0.0)
    decode: bool = False         # run through the split-KV path (few query rows)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.dqk)

    def flops(self) -> float:
        """Algorithmic FLOPs: 2·B·H_q·N_q·N_kv·(d_qk + d_v), halved when causal."""
        f = 2.0 * self.B * self.Hq * self.Nq * self.Nkv * (self.dqk + self.dv)
        return f / 2.0 if self.causal else f

    def io_bytes(self) -> int:
        """Each tensor counted once: Q, K, V (unless aliased into K), O, lse."""
        es = 4 if self.dtype == torch.float32 else 2
        q = self.B * self.Hq * self.Nq * self.dqk * es
        k = self.B * self.Hkv * self.Nkv * self.dqk * es
        v = 0 if self.v_from_k else self.B * self.Hkv * self.Nkv * self.dv * es
        o = self.B * self.Hq * self.Nq * self.dv * es
        lse = self.B * self.Hq * self.Nq * 4
        return q + k + v + o + lse

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads of the attention-forward study (seeds 1001-1005).
C1 = Workload("C1_B1_H1_N128_d64_fp32", 1, 1, 1, 128, 128, 64, 64, False, torch.float32, 1001)
C2 = Workload("C2_B4_H16_N2048_d64_causal", 4, 16, 16, 2048, 2048, 64, 64, True, torch.bfloat16, 1002)
C3 = Workload("C3_B2_Hq32_Hkv8_N4096_d128_causal", 2, 32, 8, 4096, 4096, 128, 128, True,
              torch.bfloat16, 1003)
C4 = Workload("C4_B1_Hq32_Hkv8_N16384_d128_causal_K2", 1, 32, 8, 16384, 16384, 128, 128, True,
              torch.bfloat16, 1004, k_mult=2.0)
C5 = Workload("C5_B1_Hq128_Hkv1_Nq64_Nkv8192_dqk576_dv512", 1, 128, 1, 64, 8192, 576, 512, False,
              torch.bfloat16, 1005, v_from_k=True)

# Decode-shaped workloads for the split-KV path (seeds 2001-2002): Llama-3.1-8B
# attention heads (H_q 32, H_kv 8, d 128) at one new token per sequence over a
# 32K-key cache (batch 4), and 4 new tokens over a 128K-key cache.
D1 = Workload("D1_B4_Hq32_Hkv8_Nq1_Nkv32768_d128_decode", 4, 32, 8, 1, 32768, 128, 128, False,
              torch.bfloat16, 2001, decode=True)
D2 = Workload("D2_B1_Hq32_Hkv8_Nq4_Nkv131072_d128_decode", 1, 32, 8, 4, 131072, 128, 128, False,
              torch.bfloat16, 2002, decode=True)

WORKLOADS = {w.name.split("_")[0]: w for w in (C1, C2, C3, C4, C5, D1, D2)}


def make_inputs(w: Workload, device: str | torch.device = "cpu"):
    """Return (q, k, v) for workload ``w``; v may be a strided view of k."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.Nq, w.dqk), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hkv, w.Nkv, w.dqk), generator=g, dtype=torch.float32)
    if w.k_mult != 1.0:
        k = k * w.k_mult
    if not w.v_from_k:
        v = torch.randn((w.B, w.Hkv, w.Nkv, w.dv), generator=g, dtype=torch.float32)
    q = q.to(w.dtype).to(device)
    k = k.to(w.dtype).to(device)
    if w.v_from_k:
        v = k[..., : w.dv]
    else:
        v = v.to(w.dtype).to(device)
    return q, k, v


def sample_rows(w: Workload, n: int, seed: int = 7) -> torch.Tensor:
    """n (b, h, i) triples: both ends of the sequence plus a seeded spread."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    fixed = []
    for i in (0, 1, w.Nq - 1, w.Nq // 2):
        if i >= w.Nq:
            continue  # one query row: 0 only
        fixed.append((0, 0, i))
        fixed.append((w.B - 1, w.Hq - 1, i))
    m = max(n - len(fixed), 0)
    b = torch.randint(0, w.B, (m,), generator=g)
    h = torch.randint(0, w.Hq, (m,), generator=g)
    i = torch.randint(0, w.Nq, (m,), generator=g)
    rnd = torch.stack([b, h, i], dim=1)
    rows = torch.cat([torch.tensor(fixed, dtype=torch.int64), rnd], dim=0)[:n]
    return rows


@dataclass(frozen=True)
class GemmWorkload:
    """C = A·Bᵀ with A [M, K] and B [N, K] bf16, drawn i.i.d. N(0, 1)."""
    name: str
    M: int
    N: int
    K: int
    seed: int

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def io_bytes(self) -> int:
        return 2 * (self.M * self.K + self.N * self.K + self.M * self.N)


# The projections on either side of the Llama-3.1-8B-shaped attention (C3:
# batch 2 x 4096 tokens, d_model 4096, 32 query and 8 kv heads of 128): the
# fused Q/K/V projection (N = (32 + 8 + 8) * 128) and the O projection.
G1 = GemmWorkload("G1_M8192_N6144_K4096_qkv_proj", 8192, 6144, 4096, 3001)
G2 = GemmWorkload("G2_M8192_N4096_K4096_o_proj", 8192, 4096, 4096, 3002)
GEMM_WORKLOADS = {w.name.split("_")[0]: w for w in (G1, G2)}


def make_gemm_inputs(w: GemmWorkload, device: str | torch.device = "cpu"):
    """Return (a, b): A [M, K] then B [N, K], fp32 N(0, 1) draws rounded to bf16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    a = torch.randn((w.M, w.K), generator=g, dtype=torch.float32)
    b = torch.randn((w.N, w.K), generator=g, dtype=torch.float32)
    return a.to(torch.bfloat16).to(device), b.to(torch.bfloat16).to(device)
