"""Seeded synthetic inputs for the block-quantized product.

Only random draws live here: no quantization, packing or product arithmetic.
Both the oracle-side checks and the HIP path are fed from these functions.

Seeds follow one rule: seed = 1000 * workload_id + tensor_index, the
activation vector of a workload uses tensor_index 99 (and 98, 97, ... for
further activation vectors).

Distributions (workload recipes):
  * dense weights: N(0, 0.02^2)
  * weights with outliers: N(0, 0.02^2), then round(0.001 * N * K) positions
    chosen uniformly without replacement are replaced by +-10 * 0.02 with a
    random sign
  * heavy-tailed weights: Student-t with 5 degrees of freedom scaled to a
    standard deviation of 0.02, i.e. t * 0.02 / sqrt(5 / 3)
  * activations: N(0, 1)
"""

import math

import numpy as np

STD = 0.02


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def normal(seed, rows, cols, std=1.0):
    """float32 [rows, cols] drawn N(0, std^2) with NumPy's PCG64."""
    return (_rng(seed).standard_normal((rows, cols)) * std).astype(np.float32)


def weights_normal(seed, n, k, std=STD):
    return normal(seed, n, k, std)


def weights_outliers(seed, n, k, std=STD, frac=0.001, sigma=10.0):
    rng = _rng(seed)
    w = rng.standard_normal((n, k)) * std
    cnt = int(round(frac * n * k))
    if cnt:
        idx = rng.choice(n * k, size=cnt, replace=False)
        sign = np.where(rng.random(cnt) < 0.5, -1.0, 1.0)
        w.reshape(-1)[idx] = sign * sigma * std
    return w.astype(np.float32)


def weights_student_t(seed, n, k, nu=5, std=STD):
    t = _rng(seed).standard_t(nu, size=(n, k))
    return (t * (std / math.sqrt(nu / (nu - 2)))).astype(np.float32)


def activations(seed, m, k):
    return normal(seed, m, k, 1.0)


# ---------------------------------------------------------------- device draws
# Large workloads are drawn directly in device memory with torch's seeded
# Philox generator (same distributions as above, different stream of numbers).

def torch_weights(kind, seed, n, k, device="cuda", std=STD, out=None):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if kind == "normal":
        w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32, out=out)
        return w.mul_(std)
    if kind == "outliers":
        w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32, out=out)
        w.mul_(std)
        cnt = int(round(0.001 * n * k))
        if cnt:
            idx = torch.randperm(n * k, generator=g, device=device)[:cnt]
            sign = torch.where(torch.rand(cnt, generator=g, device=device) < 0.5, -1.0, 1.0)
            w.view(-1)[idx] = sign * (10.0 * std)
        return w
    if kind == "student_t":
        # t = Z / sqrt(V / nu) with V a chi-square(nu) variable, the sum of nu
        # squared standard normals (nu = 5)
        nu = 5
        w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32, out=out)
        v = torch.zeros((n, k), device=device, dtype=torch.float32)
        for _ in range(nu):
            z = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
            v.addcmul_(z, z)
            del z
        w.div_(v.div_(nu).sqrt_())
        del v
        return w.mul_(std / math.sqrt(nu / (nu - 2)))
    raise ValueError(kind)


def torch_activations(seed, m, k, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((m, k), generator=g, device=device, dtype=torch.float32)


# ---------------------------------------------------------------- workloads

LAYER_7B = [  # (name, N, K): one 7B-shaped decoder layer
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336),
]

LAYER_70B = [  # one 70B-shaped decoder layer
    ("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
    ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672),
]

LAYER_70B_TP8 = [  # one GPU's share of a 70B-shaped layer split over 8 GPUs (Megatron style):
    # q, k, v, gate and up split by output rows; o and down split along K (whole super-blocks)
    ("q", 1024, 8192), ("k", 128, 8192), ("v", 128, 8192), ("o", 8192, 1024),
    ("gate", 3584, 8192), ("up", 3584, 8192), ("down", 8192, 3584),
]

WORKLOADS = {
    1: dict(name="q4_0_gemv_4096x4096", type="Q4_0", dist="normal",
            shapes=[("w", 4096, 4096)], m=[1]),
    2: dict(name="q8_0_gemv_14336x4096", type="Q8_0", dist="normal",
            shapes=[("w", 14336, 4096)], m=[1]),
    3: dict(name="q4_k_gemv_7b_layer", type="Q4_K", dist="outliers",
            shapes=LAYER_7B, m=[1]),
    4: dict(name="q4_k_gemm_512x14336x4096", type="Q4_K", dist="outliers",
            shapes=[("gate", 14336, 4096)], m=[512, 1, 8, 64]),
    5: dict(name="q4_k_gemv_70b_80_layers", type="Q4_K", dist="student_t",
            shapes=LAYER_70B, m=[1, 4], layers=80),
}


def weights(workload, tensor_index, n, k):
    """float32 weights of a workload tensor, drawn on the host."""
    dist = WORKLOADS[workload]["dist"]
    seed = 1000 * workload + tensor_index
    if dist == "normal":
        return weights_normal(seed, n, k)
    if dist == "outliers":
        return weights_outliers(seed, n, k)
    if dist == "student_t":
        return weights_student_t(seed, n, k)
    raise ValueError(dist)


def act(workload, m, k, index=99):
    return activations(1000 * workload + index, m, k)
