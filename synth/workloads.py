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
    "moe_group_offsets", "moe_inputs", "moe_dispatch_inputs",
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
    """(X bf16 [256,512] ~ N(0,1), W bf16 [256,512] ~ N(0,0.02)), seed 0."""
    x = normal_bf16((TINY["M"], TINY["K"]), 1.0, seed_of(1, 0, 0), device)
    w = normal_bf16((TINY["N"], TINY["K"]), 0.02, seed_of(1, 0, 1), device)
    return x, w


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
    """Expert choice per token: int64 [tokens, top_k], distinct experts per row.

    Gumbel-top-k sampling without replacement from p(e) ~ rank(e)^-alpha,
    with ranks a seeded permutation of the expert ids (alpha = 0: uniform).
    """
    wid = 4 if shape.zipf_alpha > 0 else 5
    rng = np.random.default_rng(np.random.SeedSequence(seed_parts or [wid, 0, 3]))
    E = shape.routed_experts
    ranks = rng.permutation(E) + 1
    logp = -shape.zipf_alpha * np.log(ranks.astype(np.float64))
    g = rng.gumbel(size=(shape.tokens, E))
    keys = logp[None, :] + g
    choice = np.argsort(-keys, axis=1, kind="stable")[:, : shape.top_k]
    return choice


def moe_group_offsets(shape: MoEShape, choice):
    """Rows sorted by expert (stable in token order); shared experts follow as
    groups of all tokens.  Returns (offsets int32 [G+1], row_token int64 [rows])."""
    E = shape.routed_experts
    tok = np.repeat(np.arange(shape.tokens), shape.top_k)
    exp = choice.reshape(-1)
    order = np.argsort(exp, kind="stable")
    row_token = tok[order]
    counts = np.bincount(exp, minlength=E)
    counts = np.concatenate([counts, np.full(shape.shared_experts, shape.tokens)])
    row_token = np.concatenate([row_token] + [np.arange(shape.tokens)] * shape.shared_experts)
    offsets = np.zeros(len(counts) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return offsets, row_token


def moe_inputs(shape: MoEShape, layer, device="cpu"):
    """Inputs of one expert layer ("gate_up" or "down").

    gate_up: the routed rows are copies of the tokens' hidden states
    (~N(0,1); Moonlight with 1% outlier channels x20); down: an independent
    N(0,1) matrix of the FFN width.  Weights [G, N, K] ~ N(0,0.02).
    Returns (X bf16 [rows, K], W bf16 [G, N, K], offsets int32 [G+1]).
    """
    wid = 4 if shape.zipf_alpha > 0 else 5
    choice = moe_routing(shape)
    offsets, row_token = moe_group_offsets(shape, choice)
    outl = 0.01 if shape.zipf_alpha == 0 else 0.0
    names = [l[0] for l in shape.layers()]
    li = names.index(layer)
    _, N, K = shape.layers()[li]
    if layer == "gate_up":
        xt = normal_bf16((shape.tokens, K), 1.0, seed_of(wid, li, 0), device, outlier_frac=outl)
        x = xt[torch.from_numpy(row_token).to(device)]
    else:
        x = normal_bf16((shape.rows, K), 1.0, seed_of(wid, li, 0), device, outlier_frac=outl)
    w = normal_bf16((shape.groups, N, K), 0.02, seed_of(wid, li, 1), device)
    return x.contiguous(), w, offsets


def moe_dispatch_inputs(shape: MoEShape, device="cpu"):
    """The expert gate_up layer before dispatch: the token matrix and the
    routed row -> token map instead of the gathered rows.

    Returns (XT bf16 [tokens, hidden], row_token int64 [rows], W bf16
    [G, N, K], offsets int32 [G+1]); XT[row_token] is exactly the X that
    moe_inputs(shape, "gate_up") returns, and W and offsets are its own.
    """
    wid = 4 if shape.zipf_alpha > 0 else 5
    offsets, row_token = moe_group_offsets(shape, moe_routing(shape))
    outl = 0.01 if shape.zipf_alpha == 0 else 0.0
    _, N, K = shape.layers()[0]
    xt = normal_bf16((shape.tokens, K), 1.0, seed_of(wid, 0, 0), device, outlier_frac=outl)
    w = normal_bf16((shape.groups, N, K), 0.02, seed_of(wid, 0, 1), device)
    return xt, row_token, w, offsets
