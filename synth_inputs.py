"""Seeded synthetic inputs for the weight-only quantized matmul.

Shared by the tests, the benchmark and the smoke check; it holds random
draws only, none of the method's arithmetic.  Packed low-bit weights are
drawn directly as uniformly random 32-bit words: every w_bit-wide field of a
uniform word is itself uniform on [0, 2^w_bit), which is exactly "codes
uniform 0..2^w_bit-1, packed"; no packing step is needed here.

Every case is drawn on the CPU from torch.Generator().manual_seed(seed) in
the fixed order x, Q, scales, zeros, so the GPU path and the oracle see the
same bytes.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

F16, BF16 = 0, 1
_TORCH_DT = {F16: torch.float16, BF16: torch.bfloat16}


@dataclass
class Case:
    name: str
    M: int
    N: int
    K: int
    w_bit: int
    group_size: int          # 0 for int8 (per-row scale); -1 per column (one group)
    x_dtype: int             # F16 or BF16
    x: torch.Tensor          # (M, K) fp16/bf16
    Q: torch.Tensor          # int4/int2: (K/pack, N) int32; int8: (N, K) int8
    scales: torch.Tensor     # low-bit: (G, N) fp16; int8: (N,) fp32
    zeros: Optional[torch.Tensor]  # (ceil(G/pack), N) int32 or None

    # numpy views for the oracle (16-bit floats as bit patterns)
    def np_x(self):
        return self.x.contiguous().view(torch.int16).numpy().view(np.uint16)

    def np_Q(self):
        return self.Q.contiguous().numpy()

    def np_scales(self):
        if self.w_bit == 8:
            return self.scales.contiguous().numpy()
        return self.scales.contiguous().view(torch.int16).numpy().view(np.uint16)

    def np_zeros(self):
        return None if self.zeros is None else self.zeros.contiguous().numpy()

    def oracle_args(self):
        return (self.np_x(), self.x_dtype, self.np_Q(), self.np_scales(), self.np_zeros(),
                self.M, self.N, self.K, self.w_bit, self.group_size)

    def to(self, device):
        return Case(self.name, self.M, self.N, self.K, self.w_bit, self.group_size,
                    self.x_dtype, self.x.to(device), self.Q.to(device),
                    self.scales.to(device),
                    None if self.zeros is None else self.zeros.to(device))


def _words(rows, cols, g):
    return torch.randint(-2**31, 2**31, (rows, cols), dtype=torch.int64,
                         generator=g).to(torch.int32)


def _uniform(shape, lo, hi, g):
    return lo + (hi - lo) * torch.rand(shape, generator=g, dtype=torch.float32)


def lowbit_case(M, N, K, w_bit, group_size, x_dtype=F16, symmetric=False, seed=0,
                x_std=1.0, s_lo=1e-3, s_hi=2e-2, name="lowbit"):
    """int4/int2 grouped weights: x ~ x_std*N(0,1); codes and zeros uniform;
    fp16 scales uniform [s_lo, s_hi].  group_size -1: per-column (G = 1)."""
    pack = 32 // w_bit
    G = 1 if group_size == -1 else (K // group_size if group_size else 0)
    g = torch.Generator().manual_seed(seed)
    x = (x_std * torch.randn((M, K), generator=g)).to(_TORCH_DT[x_dtype])
    Q = _words(K // pack, N, g)
    scales = _uniform((G, N), s_lo, s_hi, g).to(torch.float16)
    zeros = None if symmetric else _words(-(-G // pack), N, g)
    return Case(name, M, N, K, w_bit, group_size, x_dtype, x, Q, scales, zeros)


def int8_case(M, N, K, x_dtype=BF16, seed=0, s_lo=1e-3, s_hi=1e-2, name="int8"):
    """int8 per-row weights: x ~ N(0,1); Q uniform in [-127, 127];
    fp32 row scales uniform [s_lo, s_hi]."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g).to(_TORCH_DT[x_dtype])
    Q = torch.randint(-127, 128, (N, K), dtype=torch.int64, generator=g).to(torch.int8)
    scales = _uniform((N,), s_lo, s_hi, g)
    return Case(name, M, N, K, 8, 0, x_dtype, x, Q, scales, None)


def exact_lowbit_case(M, N, K, w_bit, group_size, x_dtype=F16, symmetric=False, seed=0,
                      name="exact_lowbit"):
    """Inputs on which every summation order is exact in fp32: x integer in
    [-3, 3]; scales 2^-(6 + (g + n) % 5), varying per group and column."""
    pack = 32 // w_bit
    G = 1 if group_size == -1 else K // group_size
    g = torch.Generator().manual_seed(seed)
    x = torch.randint(-3, 4, (M, K), generator=g).to(_TORCH_DT[x_dtype])
    Q = _words(K // pack, N, g)
    gi = torch.arange(G).view(G, 1)
    ni = torch.arange(N).view(1, N)
    scales = torch.pow(2.0, -(6 + (gi + ni) % 5).to(torch.float32)).to(torch.float16)
    zeros = None if symmetric else _words(-(-G // pack), N, g)
    return Case(name, M, N, K, w_bit, group_size, x_dtype, x, Q, scales, zeros)


def exact_int8_case(M, N, K, x_dtype=BF16, seed=0, name="exact_int8"):
    """x integer in [-3, 3], Q uniform int8, scales 2^-(6 + n % 5)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randint(-3, 4, (M, K), generator=g).to(_TORCH_DT[x_dtype])
    Q = torch.randint(-128, 128, (N, K), dtype=torch.int64, generator=g).to(torch.int8)
    scales = torch.pow(2.0, -(6 + torch.arange(N) % 5).to(torch.float32))
    return Case(name, M, N, K, 8, 0, x_dtype, x, Q, scales, None)


@dataclass
class T2Case:
    """int8 activations x ternary weights (the liger-kernel int8 x int2 product)."""
    name: str
    M: int
    N: int
    K: int
    A: torch.Tensor    # (M, K) int8
    Wp: torch.Tensor   # (K/4, N) uint8: four 2-bit codes per byte

    def to(self, device):
        return T2Case(self.name, self.M, self.N, self.K, self.A.to(device), self.Wp.to(device))


def t2_case(M, N, K, seed=0, codes=3, name="t2"):
    """A uniform over all int8 values; every 2-bit field of the packed weight
    uniform over {0, .., codes-1} (3: the ternary codes; 4 also draws code 3)."""
    g = torch.Generator().manual_seed(seed)
    A = torch.randint(-128, 128, (M, K), dtype=torch.int64, generator=g).to(torch.int8)
    f = torch.randint(0, codes, (K // 4, N, 4), dtype=torch.int64, generator=g)
    Wp = (f[..., 0] | (f[..., 1] << 2) | (f[..., 2] << 4) | (f[..., 3] << 6)).to(torch.uint8)
    return T2Case(name, M, N, K, A, Wp)


def one_hot(case: Case, ks):
    """Copy of `case` whose x row m is the unit vector e_{ks[m]}."""
    x = torch.zeros_like(case.x)
    for m, k in enumerate(ks):
        x[m, k] = 1
    return Case(case.name + "_onehot", case.M, case.N, case.K, case.w_bit, case.group_size,
                case.x_dtype, x, case.Q, case.scales, case.zeros)


# The synthetic workloads: name -> builder, each with a fixed seed.
def workload(name):
    if name == "int8_gemv_m1_k1024_n1024":
        return int8_case(1, 1024, 1024, BF16, seed=1000, name=name)
    if name == "int4_g128_asym_gemv_m1_k4096_n4096":
        return lowbit_case(1, 4096, 4096, 4, 128, F16, False, seed=2000, name=name)
    for M in (16, 32, 64):
        if name == f"int8_skinny_m{M}_k4096_n14336":
            return int8_case(M, 14336, 4096, BF16, seed=3000 + M, name=name)
    if name == "int4_pc_sym_gemv_m1_k4096_n4096":  # per-column, Marlin-style symmetric
        return lowbit_case(1, 4096, 4096, 4, -1, F16, True, seed=7000, name=name)
    if name == "int4_g128_sym_m16_k8192_n8192":
        return lowbit_case(16, 8192, 8192, 4, 128, F16, True, seed=4000, x_std=0.5, name=name)
    if name == "int4_g128_asym_smalln_m16_k14336_n1024":
        return lowbit_case(16, 1024, 14336, 4, 128, BF16, False, seed=6000, name=name)
    if name == "int4_g128_asym_prefill_m4096_k4096_n11008":
        return lowbit_case(4096, 11008, 4096, 4, 128, BF16, False, seed=5004, name=name)
    if name == "int2_g64_asym_prefill_m4096_k4096_n11008":
        return lowbit_case(4096, 11008, 4096, 2, 64, BF16, False, seed=5002, name=name)
    if name == "i8t2_m4096_k4096_n11008":
        return t2_case(4096, 11008, 4096, seed=8000, name=name)
    if name == "i8t2_m16_k4096_n4096":
        return t2_case(16, 4096, 4096, seed=8016, name=name)
    raise KeyError(name)


WORKLOADS = [
    "int8_gemv_m1_k1024_n1024",
    "int4_g128_asym_gemv_m1_k4096_n4096",
    "int4_pc_sym_gemv_m1_k4096_n4096",
    "int8_skinny_m16_k4096_n14336",
    "int8_skinny_m32_k4096_n14336",
    "int8_skinny_m64_k4096_n14336",
    "int4_g128_sym_m16_k8192_n8192",
    "int4_g128_asym_smalln_m16_k14336_n1024",
    "int4_g128_asym_prefill_m4096_k4096_n11008",
    "int2_g64_asym_prefill_m4096_k4096_n11008",
]
T2_WORKLOADS = ["i8t2_m16_k4096_n4096", "i8t2_m4096_k4096_n11008"]
