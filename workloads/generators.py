"""Seeded input generators (numpy PCG64 via default_rng).

Distributions follow the workloads the NVFP4 pages discuss: heavy-tailed
activations (Student-t, nu = 3), small Gaussian weights, Gaussian gradients
with rare large spikes, and MoE routing with Zipf-skewed expert loads.
Nothing here implements any step of the NVFP4 method.
"""
import numpy as np


def rng(seed):
    return np.random.default_rng(seed)


def normal(shape, std=1.0, seed=0):
    return (rng(seed).standard_normal(shape) * std).astype(np.float32)


def student_t(shape, nu=3.0, seed=0):
    return rng(seed).standard_t(nu, size=shape).astype(np.float32)


def uniform(shape, lo=-1.0, hi=1.0, seed=0):
    return rng(seed).uniform(lo, hi, size=shape).astype(np.float32)


def with_spikes(x, frac, factor, seed=0):
    """Multiply exactly round(frac * x.size) distinct positions by `factor`."""
    x = np.array(x, dtype=np.float32, copy=True)
    n = int(round(frac * x.size))
    if n:
        pos = rng(seed).choice(x.size, size=n, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= np.float32(factor)
    return x


def f32_to_bf16_bits(x):
    """Storage conversion float32 -> bfloat16 bit patterns, nearest-even
    (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_expert_counts(n_experts=32, n_tokens=16384, top_k=4, s=1.1):
    """Rows per expert for top-k routing with Zipf(s) popularity.

    Weights (e+1)^-s are water-filled under the cap n_tokens (a token cannot
    pick one expert twice), floored, and the remainder goes to the largest
    fractional parts (earlier expert first on ties)."""
    total = n_tokens * top_k
    w = (np.arange(n_experts, dtype=np.float64) + 1.0) ** (-s)
    target = np.zeros(n_experts)
    capped = np.zeros(n_experts, dtype=bool)
    while True:
        remaining = total - n_tokens * capped.sum()
        free_w = w[~capped].sum()
        target[~capped] = remaining * w[~capped] / free_w
        target[capped] = n_tokens
        over = (~capped) & (target > n_tokens)
        if not over.any():
            break
        capped |= over
    counts = np.floor(target).astype(np.int64)
    rem = int(total - counts.sum())
    frac = target - counts
    order = sorted(range(n_experts), key=lambda e: (-frac[e], e))
    for e in order[:rem]:
        counts[e] += 1
    return counts


def moe_routing(counts, n_tokens):
    """Expert-sorted slot list: slot i (of sum(counts)) reads token i mod
    n_tokens.  With every count <= n_tokens each token lands on distinct
    experts.  Returns (group offsets [G+1], token index per slot)."""
    counts = np.asarray(counts, dtype=np.int64)
    offsets = np.zeros(counts.size + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    token = np.arange(offsets[-1], dtype=np.int64) % n_tokens
    return offsets, token
