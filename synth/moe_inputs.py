"""Seeded synthetic inputs for the routed FP4 expert FFN workloads.

Shared by the tests, the bench and the smoke check: both the HIP path and the oracle are fed
from here. This module holds none of the method's arithmetic (no decoding, no routing, no
FFN): it only draws random numbers and lays them out in the canonical input formats.

Every tensor has its own stream, seeded by
``SeedSequence([root, workload_id, layer, index, tensor_id])``, so any one expert (or any one
token's activations) can be regenerated on its own, in any order.

Canonical formats (the inputs the library's pack and FFN calls consume):
* expert codes: uint8 [3 * H * I / 2] per expert = gate [I x H/2] | up [I x H/2] |
  down [H x I/2], row-major, two E2M1 codes per byte (low nibble = even K index);
* expert scales: uint8 [3 * H * I / 32] per expert, same matrix order, one byte per 32 K;
* activations and router weights: bfloat16 bit patterns (uint16), row-major.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

T_CODES, T_SCALES, T_X, T_ROUTER, T_LOGITS, T_PERM = range(6)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes and value distributions."""
    name: str
    wid: int                 # workload id, part of every seed
    hidden: int
    inter: int
    n_experts: int
    k: int
    tokens: int              # tokens per step
    layers: int = 1
    routing: str = "router"  # "router" (x -> W_r GEMV), "zipf", "uniform", "correlated", "fixed"
    zipf_s: float = 1.1
    corr: float = 0.9        # "correlated": logit correlation between the tokens of a step
    scale_lo: int = 120      # ue8m0 scale bytes drawn uniformly from [scale_lo, scale_hi]
    scale_hi: int = 130
    router_std: float = 0.02
    steps: int = 1           # sequential steps (tokens for decode)
    note: str = field(default="", compare=False)

    @property
    def expert_code_bytes(self) -> int:
        return 3 * self.hidden * self.inter // 2

    @property
    def expert_scale_bytes(self) -> int:
        return 3 * self.hidden * self.inter // 32


WORKLOADS = {
    # One SwiGLU expert, batch 1, every code uniform over 16 values, scales in [120, 130].
    "expert_h256_i128": Workload("expert_h256_i128", 1, 256, 128, 1, 1, 1, routing="fixed",
                                 note="single expert, hidden 256, intermediate 128, batch 1"),
    # One 384-expert MoE layer, batch-1 decode, router N(0, 0.02), top-6.
    "layer_decode_h4096_i2880_e384": Workload(
        "layer_decode_h4096_i2880_e384", 2, 4096, 2880, 384, 6, 1, steps=1000,
        note="one MoE layer decode, batch 1, 384 experts, top-6, fresh x per token"),
    # 16 chained layers, batch 1.
    "stack16_decode": Workload("stack16_decode", 3, 4096, 2880, 384, 6, 1, layers=16, steps=1000,
                               note="16 MoE layers, residual + RMSNorm between layers"),
    # 64 tokens per step, Zipf(1.1)-skewed router logits.
    "batched64_zipf": Workload("batched64_zipf", 4, 4096, 2880, 384, 6, 64, routing="zipf",
                               note="64 tokens per step, Zipf(1.1) logits"),
    # 8192 tokens, uniform router logits.
    "prefill8192_uniform": Workload("prefill8192_uniform", 5, 4096, 2880, 384, 6, 8192,
                                    routing="uniform", note="8192 tokens, U(0,1) logits"),
    # Several draft tokens of one sequence per step (multi-token prediction with three
    # draft tokens): the tokens' logits share a per-step component, correlation 0.9
    # (two tokens share about 2.4 of their 6 experts; about 14 distinct experts per step).
    "mtp4_correlated": Workload("mtp4_correlated", 7, 4096, 2880, 384, 6, 4, routing="correlated",
                                note="4 tokens per step, logits correlated 0.9 across the step"),
    # Eight independent streams decoded together.
    "streams8_uniform": Workload("streams8_uniform", 8, 4096, 2880, 384, 6, 8, routing="uniform",
                                 note="8 tokens per step, U(0,1) logits"),
    # Supplementary compute-bound shape.
    "prefill32768_uniform": Workload("prefill32768_uniform", 6, 4096, 2880, 384, 6, 32768,
                                     routing="uniform", note="32768 tokens, U(0,1) logits"),
}


def rng_for(root: int, wid: int, layer: int, index: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([root, wid, layer, index, tensor]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def expert_blob(wl: Workload, layer: int, expert: int, root: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Canonical (codes, scales) of one expert: code bytes uniform over 0..255 (so both
    nibbles are uniform over the 16 codes), scale bytes uniform over [scale_lo, scale_hi]."""
    codes = np.frombuffer(rng_for(root, wl.wid, layer, expert, T_CODES).bytes(wl.expert_code_bytes),
                          dtype=np.uint8).copy()
    scales = rng_for(root, wl.wid, layer, expert, T_SCALES).integers(
        wl.scale_lo, wl.scale_hi + 1, size=wl.expert_scale_bytes, dtype=np.uint8)
    return codes, scales


def expert_source(wl: Workload, layer: int = 0, root: int = 0):
    """Callable e -> canonical (codes, scales), regenerating expert e from its seed."""
    def src(e: int):
        return expert_blob(wl, layer, e, root)
    return src


def activations(wl: Workload, layer: int, step: int, tokens: Optional[int] = None,
                root: int = 0) -> np.ndarray:
    """bf16 bits [T, H] with values bf16(N(0, 1))."""
    t = wl.tokens if tokens is None else tokens
    z = rng_for(root, wl.wid, layer, step, T_X).standard_normal((t, wl.hidden), dtype=np.float32)
    return f32_to_bf16_bits(z)


def router_weights(wl: Workload, layer: int, root: int = 0) -> np.ndarray:
    """bf16 bits [E, H] with values bf16(router_std * N(0, 1))."""
    z = rng_for(root, wl.wid, layer, 0, T_ROUTER).standard_normal((wl.n_experts, wl.hidden),
                                                                   dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(wl.router_std))


def router_logits(wl: Workload, layer: int, step: int, tokens: Optional[int] = None,
                  root: int = 0) -> np.ndarray:
    """Synthetic router logits fp32 [T, E] for workloads that draw them directly.

    zipf:    logits[t, e] = ln p_{pi(e)} + Gumbel(0, 1), p_r proportional to r**-s for rank
             r = 1..E and pi a seeded permutation fixed per layer; the top-k of these is a
             draw of k experts without replacement with probabilities p.
    uniform: logits i.i.d. U(0, 1), so the top-k is a uniform k-subset.
    correlated: logits[t, e] = c g[e] + sqrt(1 - c^2) z[t, e] with g (one draw per step) and
             z i.i.d. N(0, 1), c = corr: each token's top-k is uniform over the experts, and
             the tokens of a step share experts more often the larger c is.
    """
    t = wl.tokens if tokens is None else tokens
    rng = rng_for(root, wl.wid, layer, step, T_LOGITS)
    if wl.routing == "uniform":
        return rng.random((t, wl.n_experts), dtype=np.float32)
    if wl.routing == "correlated":
        g = rng.standard_normal(wl.n_experts)
        z = rng.standard_normal((t, wl.n_experts))
        return (wl.corr * g[None, :] + np.sqrt(1.0 - wl.corr * wl.corr) * z).astype(np.float32)
    if wl.routing == "zipf":
        perm = rng_for(root, wl.wid, layer, 0, T_PERM).permutation(wl.n_experts)
        ranks = np.arange(1, wl.n_experts + 1, dtype=np.float64)
        logp = -wl.zipf_s * np.log(ranks)
        logp -= np.log(np.exp(logp).sum())
        base = logp[perm]  # expert e gets rank perm[e] + 1
        gumbel = -np.log(-np.log(rng.random((t, wl.n_experts))))
        return (base[None, :] + gumbel).astype(np.float32)
    raise ValueError(f"workload {wl.name} does not draw logits directly")


def random_codes(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """Uniform code bytes [rows, k/2] for ad-hoc small matrices in tests."""
    return rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)


#: Experts per device-generator call when a stack's experts are drawn on the device: the
#: draw of expert e depends on its chunk [e0, e0 + STACK_CHUNK) (the seed is the chunk's
#: first expert), so the bench and the tests that regenerate an expert use this one size.
STACK_CHUNK = 32


def device_expert_blobs(wl: Workload, layer: int, e0: int, e1: int, device, root: int = 0):
    """Codes [e1 - e0, 3 H I / 2] and scales [e1 - e0, 3 H I / 32] (uint8, canonical layout)
    of experts e0 .. e1 - 1 drawn on the device with torch's counter-based Philox
    generator, seeded by (root, workload, layer, e0): the distributions of expert_blob
    (uniform code bytes, scale bytes uniform in [scale_lo, scale_hi]) for stacks too large
    to generate on the host. A different generator than expert_blob, so the values differ."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([root, wl.wid, layer, e0, 99]).generate_state(1)[0]))
    n = e1 - e0
    codes = torch.randint(0, 256, (n, wl.expert_code_bytes), dtype=torch.uint8, device=device,
                          generator=g)
    scales = torch.randint(wl.scale_lo, wl.scale_hi + 1, (n, wl.expert_scale_bytes),
                           dtype=torch.uint8, device=device, generator=g)
    return codes, scales


def fp8_matrix(rows: int, cols: int, seed: int, root: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """A dense FP8 matrix: E4M3 codes [rows x cols] uniform over the 254 finite codes, and
    one fp32 multiplier per 128 x 128 block, 2^u * (1 + v) with u uniform on the integers
    -12 .. -6 and v uniform on [0, 1) (arbitrary fp32 values, not powers of two)."""
    rng = np.random.default_rng(np.random.SeedSequence([root, 7000 + seed, rows, cols]))
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = finite[rng.integers(0, finite.size, size=(rows, cols))]
    nb = ((rows + 127) // 128, (cols + 127) // 128)
    scales = (np.exp2(rng.integers(-12, -5, size=nb)) * (1.0 + rng.random(nb))).astype(np.float32)
    return codes, scales


def small_workload(hidden: int, inter: int, n_experts: int, k: int, tokens: int,
                   wid: int = 100, **kw) -> Workload:
    """A reduced-size workload with the same value distributions, for parity tests."""
    return Workload(f"small_h{hidden}_i{inter}_e{n_experts}_k{k}_t{tokens}", wid, hidden, inter,
                    n_experts, k, tokens, **kw)
