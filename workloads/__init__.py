"""Seeded synthetic inputs for the NF4 path: shapes of the measured layer sets and
generators of weights and activations.

This module holds none of the method's arithmetic.  It only draws numbers:
weights W = sigma * z (fp32) and activations x = bf16(z), z ~ N(0, 1), from
torch's seeded Philox generator on the requested device.  The GPU library and
the CPU oracle both consume what it produces (the oracle through host copies),
so the two sides never derive inputs from each other.

Shapes follow the model families the Trapetum and deep-fold pages run
(Llama-2-7B/13B/70B and Llama-3.1-8B linear layers, out x in).
"""
from dataclasses import dataclass

import torch

BASE_SEED = 0x4E463400

# per layer: (projection name, N = out features, K = in features)
LLAMA2_7B = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
             ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
LLAMA2_13B = [("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
              ("gate", 13824, 5120), ("up", 13824, 5120), ("down", 5120, 13824)]
LLAMA2_70B = [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
              ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]
LLAMA31_8B = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
              ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]


@dataclass(frozen=True)
class LayerSet:
    name: str
    projections: tuple      # ((name, N, K), ...)
    layers: int
    sigma: float
    ms: tuple = (1,)        # activation batch sizes measured


# one 4096x4096 GEMV; 64 distinct copies are rotated (572 MB > the 256 MB
# infinity cache) so that every launch reads its weights from HBM
SINGLE_4096 = LayerSet("single-4096x4096", (("w", 4096, 4096),), 64, 0.02)
SET_7B = LayerSet("llama2-7b", tuple(LLAMA2_7B), 32, 0.02)
SET_13B = LayerSet("llama2-13b", tuple(LLAMA2_13B), 40, 0.02)
SET_70B = LayerSet("llama2-70b", tuple(LLAMA2_70B), 80, 0.015)
SET_8B_SMALLM = LayerSet("llama3.1-8b-smallm", tuple(LLAMA31_8B), 32, 0.02, (4, 8, 32))
SET_8B_PREFILL = LayerSet("llama3.1-8b-prefill", tuple(LLAMA31_8B), 32, 0.02, (64, 128, 256, 512))

ALL_SETS = {s.name: s for s in (SINGLE_4096, SET_7B, SET_13B, SET_70B, SET_8B_SMALLM,
                                SET_8B_PREFILL)}


# Projections of one decoder layer that read the same activation vector: q, k and v
# all take the attention input, gate and up both take the MLP input.  In the
# row-major packed layout such a group is one matrix concatenated along N.
SAME_X_GROUPS = (("q", "k", "v"), ("gate", "up"))


def launch_groups(set_: "LayerSet", fused: bool):
    """One layer's products in order, as (name, ((proj, N, K), ...)): with
    `fused`, the same-x projections form one product over their concatenated rows."""
    projs = list(set_.projections)
    if not fused:
        return [(p, ((p, N, K),)) for p, N, K in projs]
    out = []
    i = 0
    while i < len(projs):
        for grp in SAME_X_GROUPS:
            names = tuple(p for p, _, _ in projs[i:i + len(grp)])
            if names == grp and len({K for _, _, K in projs[i:i + len(grp)]}) == 1:
                out.append(("|".join(grp), tuple(projs[i:i + len(grp)])))
                i += len(grp)
                break
        else:
            p, N, K = projs[i]
            out.append((p, ((p, N, K),)))
            i += 1
    return out


def _mix(*parts) -> int:
    """SplitMix64-style mixing of integers into a 63-bit seed."""
    h = BASE_SEED
    for p in parts:
        h = (h + 0x9E3779B97F4A7C15 + (int(p) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 30
        h = (h * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 27
        h = (h * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
    return h & 0x7FFFFFFFFFFFFFFF


def seed_for(set_name: str, layer: int, proj: str, kind: str) -> int:
    return _mix(sum(set_name.encode()) * 131 + len(set_name), layer,
                sum(proj.encode()) * 7 + len(proj), {"W": 1, "x": 2}[kind])


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def weights(N: int, K: int, sigma: float, seed: int, device="cpu") -> torch.Tensor:
    """fp32 [N][K], sigma * N(0,1) (the product rounded to fp32)."""
    z = torch.randn((N, K), generator=_gen(seed, device), device=device, dtype=torch.float32)
    return z.mul_(sigma)


def activations(M: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    """bf16 [M][K], N(0,1) drawn in fp32 and rounded to bf16 (nearest even)."""
    z = torch.randn((M, K), generator=_gen(seed, device), device=device, dtype=torch.float32)
    return z.to(torch.bfloat16)


def algorithmic_bytes(N: int, K: int, M: int = 1) -> int:
    """Bytes one product must move at least: codes + scales + bf16 X + fp32 Y."""
    return N * K // 2 + N * (K // 64) * 2 + 2 * M * K + 4 * M * N


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor (bit patterns, for the oracle)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
