"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module only draws random numbers and builds arrays of the right shape
and dtype; it contains none of the method's arithmetic.  bf16 arrays are
returned as raw ``np.uint16`` bit patterns; narrowing from the float32 draw
uses torch's CPU cast (round to nearest even).

Workloads (sizes and distributions of the quantization pages' experiments;
no public dataset is involved):

* ``round_trip_fp32``   65,536 fp32 values from N(0,1)            (seed 42)
* ``k_sweep_bf16``      2^24 + 17 bf16 values from N(0,1); exactly
                        round(0.001 n) distinct positions multiplied by 20 in
                        fp32 before the bf16 cast                  (seed 123)
* ``weight``            an R x C weight from N(0, 0.02) cast to the element
                        type, optionally with ``extra`` trailing values
                        (the 64 x 3 = 192 values that force an odd tail group)
* ``activations_bf16``  T x d bf16 rows from N(0,1), each row scaled by
                        10^U(-1, 1) (log-uniform in [0.1, 10]), plus a shared
                        random sign mask of d bits                 (seed 5)
"""

import numpy as np
import torch

SEED_ROUND_TRIP = 42
SEED_K_SWEEP = 123
SEED_WEIGHT_SQUARE = 7
SEED_WEIGHT_SHAPES = 11
SEED_ACT = 5

WEIGHT_SHAPES = {
    "square4096": (4096, 4096),
    "wide11008": (11008, 4096),
    "tall11008": (4096, 11008),
    "square8192": (8192, 8192),
}
TAIL_EXTRA = 64 * 3


def to_dtype(x32, dtype):
    """Cast a float32 draw to the storage dtype (bf16 as raw uint16 bits)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "fp32":
        return x32
    if dtype == "fp16":
        return torch.from_numpy(x32).to(torch.float16).numpy()
    if dtype == "bf16":
        t = torch.from_numpy(x32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def normal(n, seed, dtype="fp32", sigma=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x = (x * np.float32(sigma)).astype(np.float32)
    return to_dtype(x, dtype)


def round_trip_fp32(n=65536, seed=SEED_ROUND_TRIP):
    return normal(n, seed, "fp32")


def k_sweep_bf16(n=(1 << 24) + 17, seed=SEED_K_SWEEP, outlier_frac=0.001, outlier_mult=20.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    m = int(round(outlier_frac * n))
    pos = rng.choice(n, size=m, replace=False)
    x[pos] = (x[pos] * np.float32(outlier_mult)).astype(np.float32)
    return to_dtype(x, "bf16")


def weight(rows, cols, dtype, seed, extra=0, sigma=0.02):
    return normal(rows * cols + extra, seed, dtype, sigma)


def activations_bf16(tokens=4096, d=4096, seed=SEED_ACT):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, d), dtype=np.float32)
    scale = np.power(10.0, rng.uniform(-1.0, 1.0, size=tokens)).astype(np.float32)
    x = (x * scale[:, None]).astype(np.float32)
    signs = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    return to_dtype(x, "bf16").reshape(tokens, d), signs


def uniform_indices(n, K, seed):
    """Random K-bit indices (uint8) for layout-only tests."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << K, size=n, dtype=np.uint8)


def nested_state_synthetic(nb, seed, qmap_size=256, group=256):
    """Random nested-state inputs of the right shape (codes, absmax2, offset).

    Only for workloads whose cost is independent of the values; parity
    cases encode real states instead.
    """
    rng = np.random.default_rng(seed)
    code = rng.integers(0, qmap_size, size=nb, dtype=np.uint8)
    ng = -(-nb // group)
    absmax2 = rng.uniform(0.01, 0.05, size=ng).astype(np.float32)
    offset = np.float32(0.05)
    return code, absmax2, offset
