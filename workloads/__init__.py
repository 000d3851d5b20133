"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module only draws random inputs and names shapes.  It holds none of the
attention arithmetic, and it imports neither the oracle nor the HIP library,
so both sides of every parity check get the same inputs from a third place.

Shapes follow the workloads the pages measure:
  * BERT-large self-attention at sequence 512 and GPT-2 small at sequence 1K
    (FlashAttention reading notes, section "experimental setup"), with the
    standard 16 and 12 heads of head size 64;
  * patch self-attention of a vision mask decoder with 16 heads of size 64,
    where the patch count is about pixels/256 (16x16 patches) (Qiita page,
    section 2), at the page's measured patch counts 1,944 / 3,952 / 7,776 /
    11,616 (section 1's table) and at 3840x2560 = 8 MP, i.e. 38,400 patches.
The pages train or run real models on datasets and images; none of that is
needed here because the kernel's work depends only on shapes and value
distributions.  Values are i.i.d. normal from a fixed seed.

Recipe: numpy.random.default_rng(seed); draw Q, then K, then V as
standard_normal(shape, float32) * sigma; bf16 workloads round each value to
bf16 with round-to-nearest-even (torch's conversion).  Every consumer sees
the rounded values, so input quantisation is never counted as error.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "fp32": the I/O type of Q, K, V and O
    sigma: float        # standard deviation of the i.i.d. normal inputs
    scale: float        # multiplies Q K^T
    causal: bool
    seed: int
    what: str

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def flops(self):
        """4*B*H*N^2*d (QK^T plus PV), halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def with_n(self, n):
        return replace(self, N=n, name=f"{self.name.split('@')[0]}@N={n}")


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 64, "fp32", 1.0, 0.125, False, 0,
                     "tiny exact attention, fp32 I/O"),
    "bert_large": Workload("bert_large", 8, 16, 512, 64, "bf16", 1.0, 0.125, False, 1,
                           "BERT-large-shaped self-attention, sequence 512"),
    "gpt2_small_causal": Workload("gpt2_small_causal", 8, 12, 1024, 64, "bf16", 1.0, 0.125,
                                  True, 2, "GPT-2-small-shaped causal attention, sequence 1K"),
    "patch_3mp": Workload("patch_3mp", 1, 16, 11616, 64, "bf16", 0.5, 0.125, False, 3,
                          "vision-decoder patch self-attention at 3 MP (11,616 patches)"),
    "patch_8mp": Workload("patch_8mp", 1, 16, 38400, 64, "bf16", 0.5, 0.125, False, 4,
                          "patch self-attention at 8 MP, 3840x2560 (38,400 patches)"),
}

# The page's other measured patch counts; drawn with the 3 MP workload's seed.
PATCH_SWEEP = (1944, 3952, 7776)

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def make_inputs(w: Workload):
    """(q, k, v) as contiguous CPU torch tensors [B, H, N, d] in w.dtype."""
    rng = np.random.default_rng(w.seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal(w.shape, dtype=np.float32)
        if w.sigma != 1.0:
            x *= np.float32(w.sigma)
        out.append(torch.from_numpy(x).to(TORCH_DTYPE[w.dtype]).contiguous())
    return tuple(out)


def to_f64(t):
    """Exact float64 numpy copy of a CPU or device tensor (bf16/fp32 -> f64)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def sample_rows(n, count, seed=12345):
    """Sorted query indices for sampled checks: both ends, the ragged tail
    past the last multiple of 64, and random rows in between."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, n - 1, n - 2, n // 2}
    tail0 = (n // 64) * 64
    fixed |= set(range(tail0, n))
    fixed |= {max(tail0 - 1, 0)}
    rest = max(count - len(fixed), 0)
    fixed |= set(rng.integers(0, n, size=rest).tolist())
    return np.array(sorted(i for i in fixed if 0 <= i < n), dtype=np.int64)


def block_rows(n, blocks, seed, rows_per_block=256):
    """Sorted query indices of `blocks` distinct random aligned blocks of
    `rows_per_block` rows (every row offset 0 .. rows_per_block-1 of a
    workgroup's row block), plus the last, possibly ragged, block."""
    rng = np.random.default_rng(seed)
    nb = -(-n // rows_per_block)
    pick = set(rng.choice(nb, size=min(blocks, nb), replace=False).tolist()) | {nb - 1}
    rows = [np.arange(b * rows_per_block, min(n, (b + 1) * rows_per_block)) for b in sorted(pick)]
    return np.concatenate(rows).astype(np.int64)


def make_device_normal(shape, seed, device, dtype="bf16", sigma=1.0):
    """A seeded i.i.d. normal tensor drawn on `device` itself, for tensors too
    large to draw on the host and copy (several GiB).  Recipe:
    torch.Generator(device).manual_seed(seed), torch.randn(shape) in float32
    one slice of dim 1 at a time (bounded temporary memory), times sigma,
    rounded to dtype (round-to-nearest-even for bf16).  Checks copy the
    slices they compare back to the host, so both sides see the same values."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
    step = max(1, (1 << 26) // max(1, int(np.prod(shape[2:])) * shape[0]))
    for h0 in range(0, shape[1], step):
        h1 = min(shape[1], h0 + step)
        x = torch.randn((shape[0], h1 - h0) + tuple(shape[2:]), generator=g, device=device,
                        dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out[:, h0:h1].copy_(x)
    return out
