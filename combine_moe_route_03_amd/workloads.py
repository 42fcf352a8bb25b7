"""Seeded synthetic workloads for MoE routing, dispatch and combine.

This module only draws random inputs and describes their shapes. It holds none of the routing,
dispatch or combine arithmetic, so both the HIP path and the CPU oracle can be fed from it.

The shapes follow the evaluation setting of Perplexity, "Enabling trillion-parameter models on AWS
EFA", section "Evaluatie / Dispatch/Combine-latentie" (DeepSeek-V3 / Kimi-K2: hidden size 7168,
block-scaled fp8 dispatch, bf16 combine, 128 decode tokens and 4096 prefill tokens).

Recipe (same for every workload): ``numpy.random.default_rng(seed)``; draw the activations
``x = standard_normal((T, H), float32)`` first, then the router logits
``standard_normal((T, E), float32)``. bf16 activations are the round-to-nearest-even bf16 of the
fp32 draw (torch's CPU conversion). The skewed workload adds to every logit of expert ``e`` the
fp32 value of ``2 * ln(p_e)``, with ``p_e`` the Zipf(s=1.2) popularity ``(e+1)^-1.2 / sum``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens on this GPU
    H: int            # hidden size
    E: int            # experts
    k: int            # experts per token
    N: int            # destination ranks; rank r hosts experts [r*E/N, (r+1)*E/N)
    x_dtype: str      # "f32" or "bf16"
    payload: str      # dispatched row format: "f32", "bf16" or "fp8_e4m3"
    y_dtype: str      # expert-output format read by combine
    out_dtype: str    # combine output format
    experts: str      # "identity" or "scale": emulated expert e maps a row v to v*(e+1)/256
    zipf_bias: bool = False
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.T * self.k


WORKLOADS = {
    # 16 tokens, hidden 256, fp32, 8 experts top-2, 2 ranks of 4 experts, identity experts.
    "tiny": Workload("tiny", 16, 256, 8, 2, 2, "f32", "f32", "f32", "f32", "identity"),
    # Decode batch: 128 tokens, hidden 7168 bf16, 256 experts top-8, 32 ranks of 8 experts.
    "decode": Workload("decode", 128, 7168, 256, 8, 32, "bf16", "bf16", "bf16", "bf16", "scale"),
    # Decode batch with block-scaled fp8-e4m3 dispatch (one fp32 scale per 128 elements).
    "decode_fp8": Workload("decode_fp8", 128, 7168, 256, 8, 32, "bf16", "fp8_e4m3", "bf16", "bf16",
                           "scale"),
    # Prefill batch: 4096 tokens, hidden 7168 bf16, 384 experts top-8, 48 ranks of 8 experts.
    "prefill": Workload("prefill", 4096, 7168, 384, 8, 48, "bf16", "bf16", "bf16", "bf16", "scale"),
    # The prefill batch with block-scaled fp8-e4m3 dispatch and bf16 combine: the evaluation
    # setting of the pages at 4096 tokens (same draws as "prefill").
    "prefill_fp8": Workload("prefill_fp8", 4096, 7168, 384, 8, 48, "bf16", "fp8_e4m3", "bf16",
                            "bf16", "scale"),
    # Skewed load: 8192 tokens, hidden 4096, 128 experts top-4, 16 ranks, Zipf(1.2) logit bias.
    "skewed": Workload("skewed", 8192, 4096, 128, 4, 16, "bf16", "bf16", "bf16", "bf16", "scale",
                       zipf_bias=True),
}

ORDER = ["tiny", "decode", "decode_fp8", "prefill", "skewed"]
# Also checked at full size on the GPU: the pages' own prefill setting (fp8 dispatch).
GPU_ORDER = ORDER + ["prefill_fp8"]


@dataclass(frozen=True)
class EpWorkload:
    """Expert parallelism over S source devices and N destination ranks, emulated on one GPU."""
    name: str
    S: int            # source devices, T tokens each
    T: int
    H: int
    E: int
    k: int
    N: int            # destination ranks; rank r hosts experts [r*E/N, (r+1)*E/N)
    dtype: str        # x, payload, expert output and combine output format
    seed: int = 0

    @property
    def L(self) -> int:
        return self.E // self.N

    @property
    def cap(self) -> int:
        """Rows of one (rank, source) region: the most one source can send to one rank."""
        return self.T * min(self.k, self.L)

    def as_workload(self) -> Workload:
        """The whole batch (all sources' tokens, source s owning tokens [s*T, (s+1)*T))."""
        return Workload(self.name, self.S * self.T, self.H, self.E, self.k, self.N, self.dtype,
                        self.dtype, self.dtype, self.dtype, "identity", seed=self.seed)


EP_WORKLOADS = {
    # 3 sources of 10 tokens, hidden 256 fp32, 8 experts top-2 over 4 ranks of 2 experts.
    "ep_tiny": EpWorkload("ep_tiny", 3, 10, 256, 8, 2, 4, "f32"),
    # A decode batch of 128 tokens spread over 8 devices: 16 tokens each, 256 experts top-8 over 8
    # ranks of 32 experts.
    "ep_decode": EpWorkload("ep_decode", 8, 16, 7168, 256, 8, 8, "bf16"),
    # The 4096-token prefill batch spread over 8 devices: 512 tokens each, 384 experts top-8 over
    # 8 ranks of 48 experts.
    "ep_prefill": EpWorkload("ep_prefill", 8, 512, 7168, 384, 8, 8, "bf16"),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns of an fp32 array (torch's CPU conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def zipf_logit_bias(E: int, s: float = 1.2) -> np.ndarray:
    """fp32(2*ln p_e) with p_e = (e+1)^-s / sum_i (i+1)^-s; expert 0 is the most popular."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    return (2.0 * np.log(p)).astype(np.float32)


def make_inputs(w: Workload, seed: int | None = None, T: int | None = None) -> dict:
    """Draw (x, logits) for a workload. ``T`` overrides the token count (same recipe).

    Returns numpy arrays: ``x`` is float32 [T,H] for f32 workloads and uint16 bf16 bits [T,H]
    for bf16 workloads; ``logits`` is float32 [T,E].
    """
    seed = w.seed if seed is None else seed
    T = w.T if T is None else T
    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((T, w.H), dtype=np.float32)
    logits = rng.standard_normal((T, w.E), dtype=np.float32)
    if w.zipf_bias:
        logits = (logits + zipf_logit_bias(w.E)[None, :]).astype(np.float32)
    x = x32 if w.x_dtype == "f32" else bf16_bits_from_f32(x32)
    return {"x": x, "logits": np.ascontiguousarray(logits)}


def random_topk(T: int, E: int, k: int, seed: int) -> np.ndarray:
    """k distinct expert ids per token, uniformly at random, int32 [T,k] (for layout-only cases)."""
    rng = np.random.default_rng(seed)
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)
