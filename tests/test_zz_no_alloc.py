"""fp8bq_quantize_many_noalloc, the grouped call that allocates nothing,
against fp8bq_quantize_many with a caller workspace: equal bytes and scales
on two calls in a row, the second with a smaller list, for lists whose
descriptor table goes through the library's per-device block (more than 512
tensors) and lists that carry it in the kernel arguments."""

import numpy as np
import pytest
import torch

import fp8_blockwise_weight_amd as fq
from gpu_helpers import assert_matches_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SHAPES = [(1, 8), (77, 128), (300, 520), (256, 1024), (129, 264), (1000, 512), (64, 7)]


def _tensors(seed, count):
    g = torch.Generator(device=DEV).manual_seed(seed)
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(count):
        M, N = SHAPES[int(rng.integers(len(SHAPES)))]
        xs.append((torch.randn((M, N), generator=g, device=DEV) * float(rng.uniform(0.01, 0.1)))
                  .to(torch.bfloat16))
    return xs


def _outputs(xs, block):
    """Outputs filled with bytes the call must overwrite everywhere."""
    return [(torch.full(x.shape, 0x5A, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn),
             torch.full(fq.scale_shape(*x.shape, *block), float("nan"), device=DEV)) for x in xs]


@pytest.mark.parametrize("block", [(128, 128), (64, 64), (1, 128), (5, 3)])
def test_noalloc_equals_workspace_call(gpu_lib, block):
    for seed, count in ((1, 700), (2, 530), (3, 40)):   # the second and third smaller
        print("noalloc", block, count, flush=True)
        xs = _tensors(seed, count)
        want = fq.quantize_many(xs, block)                # the workspace entry point
        got = fq.quantize_many_noalloc(xs, _outputs(xs, block), block)
        torch.cuda.synchronize()
        for i, ((q, s), (q1, s1)) in enumerate(zip(got, want)):
            assert torch.equal(q.view(torch.uint8), q1.view(torch.uint8)), (block, count, i)
            assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), (block, count, i)
        for i in (0, count // 2, count - 1):
            assert_matches_oracle(xs[i], *got[i], *block, f"noalloc {block} {count} [{i}]")
        del xs, want, got
