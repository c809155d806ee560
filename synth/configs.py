"""The five attention-forward workloads and their seeded input recipes.

Each workload names its shape, mask, dtype and the distribution of Q, K, V.
Seeds are fixed per workload: q = 1000*i + 1, k = 1000*i + 2, v = 1000*i + 3
for workload number i (1-based).
"""

import math
from dataclasses import dataclass

import numpy as np

from .gen import normal_bf16, normal_f32


@dataclass(frozen=True)
class Workload:
    index: int          # 1-based workload number
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    fmt: str            # "bf16", "mxfp4" or "mxfp8"
    sigma_qk: float = 1.0
    sigma_v: float = 1.0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self):
        """4*B*Hq*N^2*d, halved for the causal mask (the metric's convention)."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def seeds(self):
        base = 1000 * self.index
        return base + 1, base + 2, base + 3

    def shapes(self):
        return ((self.B, self.Hq, self.N, self.d),
                (self.B, self.Hkv, self.N, self.d),
                (self.B, self.Hkv, self.N, self.d))

    def describe(self):
        return {"workload": self.name, "B": self.B, "Hq": self.Hq, "Hkv": self.Hkv,
                "N": self.N, "d": self.d, "causal": self.causal, "format": self.fmt}

    def make(self):
        """Returns (q, k, v): uint16 bf16 bits for bf16 workloads, fp32 for the block-scaled
        formats (quantised by the consumer)."""
        sq, sk, sv = self.seeds()
        shq, shk, shv = self.shapes()
        if self.fmt == "bf16":
            return (normal_bf16(shq, sq, self.sigma_qk),
                    normal_bf16(shk, sk, self.sigma_qk),
                    normal_bf16(shv, sv, self.sigma_v))
        return (normal_f32(shq, sq, self.sigma_qk),
                normal_f32(shk, sk, self.sigma_qk),
                normal_f32(shv, sv, self.sigma_v))


CONFIGS = {
    1: Workload(1, "noncausal_B1_H2_N256_d64", 1, 2, 2, 256, 64, False, "bf16"),
    2: Workload(2, "causal_B4_H16_N2048_d128", 4, 16, 16, 2048, 128, True, "bf16"),
    3: Workload(3, "causal_gqa_B1_Hq32_Hkv8_N8192_d128", 1, 32, 8, 8192, 128, True, "bf16"),
    4: Workload(4, "noncausal_B2_H16_N16384_d128_qk_sigma3", 2, 16, 16, 16384, 128, False,
                "bf16", sigma_qk=3.0),
    5: Workload(5, "noncausal_mxfp4_directp_B1_H24_N16384_d128", 1, 24, 24, 16384, 128, False,
                "mxfp4"),
    # MXFP8 forward on the shapes of workloads 5 and 3 (FP8 path; not one of the five above)
    6: Workload(6, "noncausal_mxfp8_B1_H24_N16384_d128", 1, 24, 24, 16384, 128, False, "mxfp8"),
    7: Workload(7, "causal_gqa_mxfp8_B1_Hq32_Hkv8_N8192_d128", 1, 32, 8, 8192, 128, True,
                "mxfp8"),
}


def workload(i):
    return CONFIGS[int(i)]


def random_case(seed, B, Hq, Hkv, N, d, sigma=1.0):
    """A small ad-hoc bf16 case for ragged / edge-case tests."""
    shq = (B, Hq, N, d)
    shk = (B, Hkv, N, d)
    return (normal_bf16(shq, seed * 3 + 1, sigma),
            normal_bf16(shk, seed * 3 + 2, sigma),
            normal_bf16(shk, seed * 3 + 3, 1.0))


__all__ = ["Workload", "CONFIGS", "workload", "random_case", "np"]
