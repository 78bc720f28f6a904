"""Seeded synthetic inputs for the attention workloads.

This module is shared by the GPU tests, the oracle tests and the benchmark.
It only draws random numbers and arranges them in memory: it holds none of
the attention arithmetic, and imports neither the GPU library nor the oracle.

Recipe (the same bytes go to the GPU and, upcast to float64, to the oracle):
  * a ``torch.Generator`` on the CPU seeded with the case's seed;
  * Q, K, V (and dO for the backward) drawn in that order as float32
    ``torch.randn`` in the PHYSICAL layout (B,H,S,D for BHSD, B,S,H,D for
    BSHD, T,H,D for packed THD), then cast to the io dtype with
    round-to-nearest-even;
  * packed sequence lengths drawn with ``torch.randint(lo, hi + 1, (n,))``
    from the same generator BEFORE the tensors, and turned into int32
    prefix sums with cu[0] = 0.

The workloads mirror the pages: the causal bf16 demo at b4 h16 s1024 d64 with
scale 1/sqrt(d) ("Inside NVIDIA's cuDNN Graph API ...", section 5), BSHD
allocations viewed as logical BHSD (cudnn-frontend PR #554 merge log, the
benchmark entry that allocates BSHD), and packed THD batches indexed by
cu_seqlens (same pull request).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class DenseCase:
    name: str
    dtype: str
    b: int
    h: int
    s_q: int
    s_kv: int
    d: int
    causal: bool
    layout: str  # "bhsd" or "bshd" (physical order; logical order is always b,h,s,d)
    seed: int
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class VarlenCase:
    name: str
    dtype: str
    n_seqs: int
    len_lo: int
    len_hi: int
    h: int
    d: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads, by what they are.
FWD_FP32_B1H2S128D64 = DenseCase("fwd fp32 causal b1 h2 s128 d64 BHSD", "fp32",
                                 1, 2, 128, 128, 64, True, "bhsd", 1001)
FWD_BF16_B4H16S1024D64 = DenseCase("fwd bf16 causal b4 h16 s1024 d64 BHSD", "bf16",
                                   4, 16, 1024, 1024, 64, True, "bhsd", 1002)
FWD_BF16_B2H16S4096D128 = DenseCase("fwd bf16 non-causal b2 h16 s4096 d128 BSHD", "bf16",
                                    2, 16, 4096, 4096, 128, False, "bshd", 1003)
FWD_FP16_B2H16S4096D128 = DenseCase("fwd fp16 non-causal b2 h16 s4096 d128 BSHD", "fp16",
                                    2, 16, 4096, 4096, 128, False, "bshd", 1003)
VARLEN_BF16_32SEQ_H16D128 = VarlenCase("fwd varlen bf16 causal 32 seqs L~U[64,2048] h16 d128",
                                       "bf16", 32, 64, 2048, 16, 128, True, 1004)
BWD_BF16_B4H16S2048D128 = DenseCase("bwd bf16 causal b4 h16 s2048 d128 BHSD", "bf16",
                                    4, 16, 2048, 2048, 128, True, "bhsd", 1005, backward=True)


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _draw(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def device_normal(shape, dtype: str, seed: int, device) -> torch.Tensor:
    """iid N(0,1) drawn on the device by its own seeded generator (fp32, cast to
    the io dtype): for inputs of several GiB, which the host would take long to
    draw. Checks copy the parts they need back to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device).to(DTYPES[dtype])


def dense_inputs(b: int, h: int, s_q: int, s_kv: int, d: int, dtype: str, layout: str,
                 seed: int, with_dout: bool = False) -> List[torch.Tensor]:
    """CPU tensors [q, k, v(, dout)] as logical (b, h, s, d) views of the physical layout."""
    dt = DTYPES[dtype]
    g = generator(seed)
    out = []
    for i, s in enumerate([s_q, s_kv, s_kv] + ([s_q] if with_dout else [])):
        if layout == "bhsd":
            t = _draw(g, (b, h, s, d), dt)
        elif layout == "bshd":
            t = _draw(g, (b, s, h, d), dt).transpose(1, 2)
        else:
            raise ValueError(f"unknown layout {layout!r}")
        out.append(t)
    return out


def case_inputs(case: DenseCase) -> List[torch.Tensor]:
    return dense_inputs(case.b, case.h, case.s_q, case.s_kv, case.d, case.dtype, case.layout,
                        case.seed, with_dout=case.backward)


def lengths(n: int, lo: int, hi: int, g: torch.Generator) -> torch.Tensor:
    """n integer lengths, uniform on [lo, hi] inclusive."""
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64)


def cu_seqlens(lens) -> torch.Tensor:
    """int32 prefix sums [n+1] with cu[0] = 0."""
    lens = torch.as_tensor(lens, dtype=torch.int64)
    cu = torch.zeros(lens.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    return cu.to(torch.int32)


def capacity(total: int) -> int:
    """Rows allocated for a packed buffer: the next multiple of 64 strictly above
    `total`, plus one more block of 64, so a tail of live capacity always exists."""
    return (total // 64 + 1) * 64 + 64


@dataclass
class VarlenInputs:
    q: torch.Tensor  # [cap_q, h, d]; rows >= total_q are NaN poison
    k: torch.Tensor
    v: torch.Tensor
    cu_q: torch.Tensor  # int32 [n+1]
    cu_kv: torch.Tensor
    lens_q: torch.Tensor
    lens_kv: torch.Tensor
    total_q: int
    total_kv: int
    dout: Optional[torch.Tensor] = None


def varlen_inputs(lens_q, lens_kv, h: int, d: int, dtype: str, seed: int,
                  poison_tail: bool = True, with_dout: bool = False,
                  h_kv: Optional[int] = None) -> VarlenInputs:
    """Packed THD tensors with a NaN-filled capacity tail (when poison_tail);
    k and v carry h_kv heads (default h)."""
    dt = DTYPES[dtype]
    h_kv = h if h_kv is None else h_kv
    lens_q = torch.as_tensor(lens_q, dtype=torch.int64)
    lens_kv = torch.as_tensor(lens_kv, dtype=torch.int64)
    cu_q, cu_kv = cu_seqlens(lens_q), cu_seqlens(lens_kv)
    tq, tkv = int(cu_q[-1]), int(cu_kv[-1])
    g = generator(seed)
    bufs = []
    for tot, nh in ((tq, h), (tkv, h_kv), (tkv, h_kv)) + (((tq, h),) if with_dout else ()):
        cap = capacity(tot) if poison_tail else tot
        t = torch.full((cap, nh, d), float("nan"), dtype=dt)
        t[:tot] = _draw(g, (tot, nh, d), dt)
        bufs.append(t)
    return VarlenInputs(bufs[0], bufs[1], bufs[2], cu_q, cu_kv, lens_q, lens_kv, tq, tkv,
                        bufs[3] if with_dout else None)


def varlen_case_inputs(case: VarlenCase, poison_tail: bool = True) -> VarlenInputs:
    g = generator(case.seed)
    lens = lengths(case.n_seqs, case.len_lo, case.len_hi, g)
    return varlen_inputs(lens, lens, case.h, case.d, case.dtype, case.seed + 100_000,
                         poison_tail=poison_tail)


def causal_fwd_flops(b: int, h: int, s: int, d: int, causal: bool) -> float:
    """The pages' FLOP count for the forward: 4*b*h*s*s*d, halved when causal."""
    f = 4.0 * b * h * s * s * d
    return f * 0.5 if causal else f
