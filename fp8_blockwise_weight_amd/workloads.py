"""Seeded synthetic BF16 weight sets for the quantizer's tests and benchmark.

This module holds shapes and random distributions only; none of the
quantizer's arithmetic lives here.  The tests feed the same generated tensor
to the GPU library and to the CPU oracle.

The shapes stand in for the weights the rollout stack re-quantizes every RL
step (the abstract of "FP8-RL: A Practical and Stable Low-Precision Stack for
LLM Reinforcement Learning"; the dense run in "[rollout, sglang] feat:
support blockwise fp8 rollout", Experiments section, uses Qwen3-8B-Base).  No
checkpoint is loaded: every value is drawn from a seeded generator.

Workloads (the five weight sets the quantizer is tested and measured on):

* ``C1``  one 256x256 matrix, block [128,128]: N(0, 0.02); tile (0,0) holds
  8 planted +-5.0 outliers at distinct seeded positions with seeded signs;
  tile (1,1) is all +0.
* ``C2``  one Qwen3-8B-shaped decoder layer ([out, in] linear weights):
  q_proj 4096x4096, k_proj 1024x4096, v_proj 1024x4096, o_proj 4096x4096,
  gate_proj 12288x4096, up_proj 12288x4096, down_proj 4096x12288.
  N(0, 0.02) with round(1e-4 * numel) distinct seeded positions replaced by
  0.5 * Student-t(3) draws.
* ``C3``  36 independently seeded C2 layers (252 tensors, 6.95e9 values).
* ``C4``  48 MoE layers x 128 experts: w13 1536x2048 and down 2048x768.
  Each expert draws sigma ~ U(0.01, 0.04) (shared by its two matrices);
  values N(0, sigma^2).
* ``C5``  ragged shapes 1000x3000, 4097x11008, 151937x4096, 77x128, each
  used with blocks [128,128], [64,64] and [1,128]: per element 90% N(0,0.02)
  and 10% Laplace(0, 0.2); row 0, the last row and 1% of the rows (seeded)
  are all zero.

Seeds: ``(config << 32) | (layer << 16) | index``.
"""

from dataclasses import dataclass
from typing import List, Tuple

import torch

QWEN3_8B_LAYER: Tuple[Tuple[str, int, int], ...] = (
    ("q_proj", 4096, 4096),
    ("k_proj", 1024, 4096),
    ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 12288, 4096),
    ("up_proj", 12288, 4096),
    ("down_proj", 4096, 12288),
)
DENSE_LAYERS = 36
MOE_LAYERS = 48
MOE_EXPERTS = 128
MOE_W13 = (1536, 2048)
MOE_DOWN = (2048, 768)
RAGGED_SHAPES = ((1000, 3000), (4097, 11008), (151937, 4096), (77, 128))
RAGGED_BLOCKS = ((128, 128), (64, 64), (1, 128))
DEFAULT_BLOCK = (128, 128)


def seed_of(config: int, layer: int, index: int) -> int:
    return (config << 32) | (layer << 16) | index


@dataclass(frozen=True)
class TensorSpec:
    name: str
    M: int
    N: int
    seed: int
    recipe: str            # "c1", "dense", "moe", "ragged"
    sigma: float = 0.02

    @property
    def numel(self) -> int:
        return self.M * self.N


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _c1(spec: TensorSpec, device) -> torch.Tensor:
    g = _gen(spec.seed, device)
    x = torch.randn((spec.M, spec.N), generator=g, device=device) * spec.sigma
    pos = torch.randperm(128 * 128, generator=g, device=device)[:8]
    sign = torch.randint(0, 2, (8,), generator=g, device=device).float() * 2 - 1
    tile = x[:128, :128].reshape(-1)
    tile[pos] = 5.0 * sign
    x[:128, :128] = tile.reshape(128, 128)
    x[128:256, 128:256] = 0.0
    return x.to(torch.bfloat16)


def _dense(spec: TensorSpec, device) -> torch.Tensor:
    g = _gen(spec.seed, device)
    n = spec.numel
    x = torch.randn(n, generator=g, device=device) * spec.sigma
    k = round(1e-4 * n)
    if k:
        pos = torch.randperm(n, generator=g, device=device)[:k]
        z = torch.randn(k, generator=g, device=device)
        chi2 = torch.randn((k, 3), generator=g, device=device).square().sum(dim=1)
        x[pos] = 0.5 * z / torch.sqrt(chi2 / 3.0)
    return x.reshape(spec.M, spec.N).to(torch.bfloat16)


def _moe(spec: TensorSpec, device) -> torch.Tensor:
    g = _gen(spec.seed, device)
    return (torch.randn((spec.M, spec.N), generator=g, device=device) * spec.sigma).to(torch.bfloat16)


def _ragged(spec: TensorSpec, device) -> torch.Tensor:
    g = _gen(spec.seed, device)
    shape = (spec.M, spec.N)
    normal = torch.randn(shape, generator=g, device=device) * 0.02
    # Laplace(0, b) as b times the difference of two unit exponentials.
    e1 = torch.empty(shape, device=device).exponential_(1.0, generator=g)
    e2 = torch.empty(shape, device=device).exponential_(1.0, generator=g)
    laplace = 0.2 * (e1 - e2)
    pick = torch.rand(shape, generator=g, device=device) < 0.1
    x = torch.where(pick, laplace, normal)
    x[0] = 0.0
    x[-1] = 0.0
    n_zero = round(0.01 * spec.M)
    if n_zero:
        rows = torch.randperm(spec.M, generator=g, device=device)[:n_zero]
        x[rows] = 0.0
    return x.to(torch.bfloat16)


_RECIPES = {"c1": _c1, "dense": _dense, "moe": _moe, "ragged": _ragged}


def materialize(spec: TensorSpec, device="cpu") -> torch.Tensor:
    """Draw the BF16 [M, N] tensor a spec describes, on ``device``."""
    return _RECIPES[spec.recipe](spec, device)


def c1() -> List[TensorSpec]:
    return [TensorSpec("c1", 256, 256, seed_of(1, 0, 0), "c1")]


def dense_layer(layer: int, config: int = 3) -> List[TensorSpec]:
    return [TensorSpec(f"layers.{layer}.{name}", M, N, seed_of(config, layer, i), "dense")
            for i, (name, M, N) in enumerate(QWEN3_8B_LAYER)]


def c2() -> List[TensorSpec]:
    return dense_layer(0, config=2)


def c3() -> List[TensorSpec]:
    return [s for layer in range(DENSE_LAYERS) for s in dense_layer(layer, config=3)]


def moe_sigmas(layer: int) -> List[float]:
    """Per-expert standard deviations of one MoE layer, U(0.01, 0.04), drawn on the CPU."""
    g = _gen(seed_of(4, layer, 0xFFFF), "cpu")
    u = torch.rand(MOE_EXPERTS, generator=g, dtype=torch.float64)
    return [0.01 + 0.03 * float(v) for v in u]


def c4_layer(layer: int) -> List[TensorSpec]:
    sig = moe_sigmas(layer)
    out = []
    for e in range(MOE_EXPERTS):
        out.append(TensorSpec(f"layers.{layer}.experts.{e}.w13", *MOE_W13,
                              seed_of(4, layer, 2 * e), "moe", sig[e]))
        out.append(TensorSpec(f"layers.{layer}.experts.{e}.down", *MOE_DOWN,
                              seed_of(4, layer, 2 * e + 1), "moe", sig[e]))
    return out


def c5() -> List[TensorSpec]:
    return [TensorSpec(f"ragged.{M}x{N}", M, N, seed_of(5, 0, i), "ragged")
            for i, (M, N) in enumerate(RAGGED_SHAPES)]


def algorithmic_bytes(M: int, N: int, bm: int, bn: int) -> int:
    """Bytes a quantizer must move for one tensor: BF16 in, FP8 out, fp32 scales out."""
    TM, TN = -(-M // bm), -(-N // bn)
    return 2 * M * N + M * N + 4 * TM * TN
