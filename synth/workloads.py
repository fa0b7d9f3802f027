"""Shapes and seeded generators of the synthetic FP8 linear-layer workloads.

The shapes mimic the models the recipe's page names (Llama 3.1 8B, Moonlight
16B, Qwen3-30B-A3B); no model weights or datasets are involved.  Every tensor
is drawn in fp32 from a seeded torch generator on the requested device and
rounded to bf16 (round to nearest even, torch's conversion).  The same bits
then feed both the GPU path and the CPU oracle.

Nothing here quantizes or multiplies; it only draws inputs.
"""
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "TINY", "LLAMA_TOKENS", "LLAMA_LAYERS", "LLAMA_NUM_LAYERS", "QWEN3", "MOONLIGHT",
    "MoEShape", "seed_of", "normal_bf16", "bf16_bits", "outlier_channels",
    "tiny_inputs", "llama_layer_inputs", "llama_weight", "moe_routing",
    "moe_token_matrix", "moe_down_input", "moe_weights",
]

# Tiny linear layer: X 256x512 ~ N(0,1), W 256x512 ~ N(0, 0.02).
TINY = dict(M=256, N=256, K=512)

# Llama-3.1-8B-shaped dense linear layers at 4096 tokens: (name, N, K) for
# Y[M,N] = X[M,K] * W[N,K]^T.  Hidden 4096, 32 query + 8 key/value heads of
# dimension 128 (QKV width 6144), FFN 14336 (gate and up fused: 28672).
LLAMA_TOKENS = 4096
LLAMA_LAYERS = (("qkv", 6144, 4096), ("o", 4096, 4096),
                ("gate_up", 28672, 4096), ("down", 4096, 14336))
LLAMA_NUM_LAYERS = 32


@dataclass(frozen=True)
class MoEShape:
    name: str
    tokens: int
    hidden: int
    routed_experts: int
    top_k: int
    shared_experts: int
    ffn: int
    zipf_alpha: float  # 0.0 = uniform routing

    @property
    def groups(self):
        return self.routed_experts + self.shared_experts

    @property
    def rows(self):
        return self.tokens * (self.top_k + self.shared_experts)

    def layers(self):
        """(name, N, K) of the two expert linear layers."""
        return (("gate_up", 2 * self.ffn, self.hidden), ("down", self.hidden, self.ffn))


QWEN3 = MoEShape("qwen3_30b_a3b", tokens=8192, hidden=2048, routed_experts=128, top_k=8,
                 shared_experts=0, ffn=768, zipf_alpha=1.1)
MOONLIGHT = MoEShape("moonlight_16b", tokens=16384, hidden=2048, routed_experts=64, top_k=6,
                     shared_experts=2, ffn=1408, zipf_alpha=0.0)


def seed_of(*parts):
    """A 63-bit seed from small integers (workload id, layer, tensor id)."""
    ss = np.random.SeedSequence([int(p) for p in parts])
    return int(ss.generate_state(2, dtype=np.uint32).astype(np.uint64).dot([1, 1 << 31])) & ((1 << 63) - 1)


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def outlier_channels(K, frac, seed):
    """Sorted indices of round(frac*K) channels (seeded, host)."""
    n = int(round(frac * K))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(K, size=n, replace=False))


def normal_bf16(shape, std, seed, device="cpu", outlier_frac=0.0, outlier_mult=20.0):
    """bf16 tensor ~ N(0, std^2); optionally a fraction of the last-axis
    channels multiplied by outlier_mult before the bf16 rounding."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if outlier_frac > 0.0:
        ch = outlier_channels(shape[-1], outlier_frac, seed ^ 0x5A5A)
        idx = torch.from_numpy(ch).to(device)
        x[..., idx] *= outlier_mult
    return x.to(torch.bfloat16)


def bf16_bits(t):
    """Raw uint16 bit patterns (numpy, host) of a bf16 tensor."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def tiny_inputs(device="cpu"):
    """(X bf16 [256,512] ~ N(0,1), W bf16 [256,512] ~ N(0,0.02)): literally
    seed 0 -- numpy's default_rng(0) draws X, then W, in fp32 on the host,
    rounded to bf16 (RNE)."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((TINY["M"], TINY["K"]), dtype=np.float32)
    w = rng.standard_normal((TINY["N"], TINY["K"]), dtype=np.float32) * np.float32(0.02)
    return (torch.from_numpy(x).to(torch.bfloat16).to(device),
            torch.from_numpy(w).to(torch.bfloat16).to(device))


def llama_layer_inputs(layer_idx, device="cpu", tokens=LLAMA_TOKENS):
    """(X [tokens, K] with 1% outlier channels x20, W [N, K] ~ N(0,0.02)) of
    one of the four Llama-shaped linear layers."""
    _, N, K = LLAMA_LAYERS[layer_idx]
    x = normal_bf16((tokens, K), 1.0, seed_of(2, layer_idx, 0), device, outlier_frac=0.01)
    w = normal_bf16((N, K), 0.02, seed_of(2, layer_idx, 1), device)
    return x, w


def llama_weight(layer, kind, device="cpu"):
    """bf16 weight ~ N(0,0.02) of matrix `kind` (0..3) of decoder layer
    `layer` (0..31) of the Llama-shaped model, for the recalibration pass."""
    _, N, K = LLAMA_LAYERS[kind]
    return normal_bf16((N, K), 0.02, seed_of(3, layer, kind), device)


def moe_routing(shape: MoEShape, seed_parts=None):
    """Expert choice per token: int32 [tokens, top_k], distinct experts per row.

    Gumbel-top-k sampling without replacement.  Zipf load (alpha > 0): a
    seeded permutation lists the experts in rank order (the expert it puts
    first has rank 1) and p(e) ~ rank(e)^-alpha; the permutation is drawn
    before the Gumbel noise.  Uniform load (alpha = 0): the Gumbel noise
    alone, with no permutation drawn.  With the default seeds the expert
    loads come out as Qwen3: max 7397 / median 196 / min 79 rows per expert;
    Moonlight: 1477..1662.
    """
    wid = 4 if shape.zipf_alpha > 0 else 5
    rng = np.random.default_rng(np.random.SeedSequence(seed_parts or [wid, 0, 3]))
    E = shape.routed_experts
    if shape.zipf_alpha > 0:
        by_rank = rng.permutation(E)
        ranks = np.empty(E, dtype=np.float64)
        ranks[by_rank] = np.arange(1, E + 1)
        logp = -shape.zipf_alpha * np.log(ranks)
    else:
        logp = np.zeros(E)
    g = rng.gumbel(size=(shape.tokens, E))
    keys = logp[None, :] + g
    choice = np.argsort(-keys, axis=1, kind="stable")[:, : shape.top_k]
    return choice.astype(np.int32)


def moe_token_matrix(shape: MoEShape, device="cpu"):
    """The tokens' hidden states before dispatch, bf16 [tokens, hidden] ~ N(0,1)
    (Moonlight: 1% outlier channels x20): the expert gate+up layer's input,
    whose row r after dispatch is the state of the token the dispatch order
    assigns to row r."""
    wid = 4 if shape.zipf_alpha > 0 else 5
    outl = 0.01 if shape.zipf_alpha == 0 else 0.0
    return normal_bf16((shape.tokens, shape.hidden), 1.0, seed_of(wid, 0, 0), device, outlier_frac=outl)


def moe_down_input(shape: MoEShape, device="cpu"):
    """The expert down layer's input, an independent bf16 [rows, ffn] ~ N(0,1)
    (Moonlight: 1% outlier channels x20)."""
    wid = 4 if shape.zipf_alpha > 0 else 5
    outl = 0.01 if shape.zipf_alpha == 0 else 0.0
    return normal_bf16((shape.rows, shape.ffn), 1.0, seed_of(wid, 1, 0), device, outlier_frac=outl)


def moe_weights(shape: MoEShape, layer, device="cpu"):
    """Expert weights of one layer ("gate_up" or "down"), bf16 [G, N, K] ~ N(0, 0.02)."""
    wid = 4 if shape.zipf_alpha > 0 else 5
    names = [l[0] for l in shape.layers()]
    li = names.index(layer)
    _, N, K = shape.layers()[li]
    return normal_bf16((shape.groups, N, K), 0.02, seed_of(wid, li, 1), device)
