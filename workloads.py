"""Seeded synthetic attention workloads: shapes, dtypes and input tensors.

This module only draws random inputs; it holds none of the attention
arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP library
(``exact_attention_66_amd``) take their inputs from here, and nothing else is
shared between the two.

Recipe (one fixed reading of "i.i.d. N(0,1) from seed"):

* a CPU ``torch.Generator`` seeded with the workload's seed;
* fp32 ``randn`` tensors of shape ``[B, H, N, d]`` drawn in the order
  Q, K, V, dO (dO only for workloads that run the backward pass);
* the ``peaky`` workload multiplies Q and K by 2 in fp32 (exact);
* each tensor is rounded to the I/O dtype (bf16 or fp16) with
  round-to-nearest-even, and those rounded values are what both sides see.

The sizes are those of the attention workloads the pages discuss: causal
GPT/Llama-style training shapes (d = 64 and 128, N from 2K to 32K) plus two
small forward-only cases.  No dataset is involved: Gaussian activations stand
in for the unnamed training data.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "fp16"
    causal: bool
    backward: bool      # whether the workload runs fwd+bwd or fwd only
    seed: int
    qk_gain: float = 1.0  # Q and K multiplied by this in fp32 before rounding
    description: str = ""

    @property
    def scale(self) -> float:
        """Softmax scale as the fp32 value handed to the kernel: fp32(1/sqrt(d))."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]

    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def fwd_flops(self) -> float:
        """Counted forward flops: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Counted backward flops: 2.5 x forward."""
        return 2.5 * self.fwd_flops() if self.backward else 0.0

    def with_size(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("fwd_b1h4n256d64", 1, 4, 256, 64, "bf16", False, False, 1001,
                 description="forward only, non-causal, small"),
        Workload("causal_b8h16n2048d64", 8, 16, 2048, 64, "bf16", True, True, 1002,
                 description="causal fwd+bwd, d=64"),
        Workload("causal_b4h32n4096d128", 4, 32, 4096, 128, "bf16", True, True, 1003,
                 description="causal fwd+bwd, Llama-7B-shaped attention (headline)"),
        Workload("causal_peaky_b1h32n16384d128", 1, 32, 16384, 128, "bf16", True, True, 1004,
                 qk_gain=2.0,
                 description="long sequence, small batch, Q and K x2 (peaky rows)"),
        Workload("causal_fp16_b1h16n32768d128", 1, 16, 32768, 128, "fp16", True, True, 1005,
                 description="very long context, fp16"),
        Workload("fwd_fp16_b2h16n8192d128", 2, 16, 8192, 128, "fp16", False, False, 1006,
                 description="non-causal forward, fp16, for comparison"),
    ]
}

HEADLINE = "causal_b4h32n4096d128"


def make_inputs(w: Workload, *, with_grad: Optional[bool] = None):
    """Return dict of CPU tensors (I/O dtype): q, k, v and, for backward workloads, do.

    Follows the recipe in the module docstring exactly; ``with_grad`` overrides
    whether dO is drawn (it is always drawn after Q, K, V).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    shape = w.shape()
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.qk_gain != 1.0:
        q.mul_(w.qk_gain)
        k.mul_(w.qk_gain)
    out = {"q": q.to(w.torch_dtype), "k": k.to(w.torch_dtype), "v": v.to(w.torch_dtype)}
    want_do = w.backward if with_grad is None else with_grad
    if want_do:
        do = torch.randn(shape, generator=g, dtype=torch.float32)
        out["do"] = do.to(w.torch_dtype)
    return out


@dataclasses.dataclass(frozen=True)
class KvWorkload:
    """Decoding against a KV cache: Nq new queries per head, Nk cached keys and values."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool        # the queries are the last Nq positions (query i sees keys <= i + Nk - Nq)
    seed: int
    qk_gain: float = 1.0
    description: str = ""
    Hkv: int = 0        # KV heads (grouped heads: query head h uses KV head h // (H // Hkv)); 0 = H

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]

    def kv_bytes(self) -> int:
        """K and V bytes: the one pass over the cache that bounds the call."""
        return 2 * self.B * self.kv_heads * self.Nk * self.d * 2

    def io_bytes(self) -> int:
        """All algorithmic HBM bytes: K, V and Q read, O written (16-bit), lse written (fp32)."""
        return self.kv_bytes() + 2 * self.B * self.H * self.Nq * self.d * 2 + 4 * self.B * self.H * self.Nq

    def with_size(self, **kw) -> "KvWorkload":
        return dataclasses.replace(self, **kw)


# The head shapes of the training workloads above, one or a few new tokens
# against the cache of their context length.
KV_WORKLOADS: Dict[str, KvWorkload] = {
    w.name: w
    for w in [
        KvWorkload("decode_b4h32q1k4096d128", 4, 32, 1, 4096, 128, "bf16", True, 2001,
                   description="one new token per sequence, Llama-7B-shaped heads, 4K cache"),
        KvWorkload("decode_fp16_b1h16q1k32768d128", 1, 16, 1, 32768, 128, "fp16", True, 2002,
                   description="one new token, 32K fp16 cache"),
        KvWorkload("spec_b4h32q8k4096d128", 4, 32, 8, 4096, 128, "bf16", True, 2003,
                   description="eight speculative tokens, causal within the block, 4K cache"),
        KvWorkload("decode_gqa_b8h32kv8q1k8192d128", 8, 32, 1, 8192, 128, "bf16", True, 2004, Hkv=8,
                   description="one new token, 32 query heads on 8 KV heads (grouped-query), 8K cache"),
    ]
}


def make_kv_inputs(w: KvWorkload):
    """CPU tensors q [B,H,Nq,d], k and v [B,Hkv,Nk,d] (I/O dtype): fp32 randn drawn
    in the order Q, K, V from the workload's seed, Q and K times qk_gain,
    rounded to nearest-even."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    q = torch.randn((w.B, w.H, w.Nq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.kv_heads, w.Nk, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.kv_heads, w.Nk, w.d), generator=g, dtype=torch.float32)
    if w.qk_gain != 1.0:
        q.mul_(w.qk_gain)
        k.mul_(w.qk_gain)
    return {"q": q.to(w.torch_dtype), "k": k.to(w.torch_dtype), "v": v.to(w.torch_dtype)}


def to_f64_numpy(t: torch.Tensor):
    """Upcast a rounded I/O tensor to an fp64 numpy array (exact)."""
    return t.to(torch.float64).numpy()
