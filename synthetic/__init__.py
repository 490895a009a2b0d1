"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's
callers.  This module holds no arithmetic of the quantization method: it only
draws weights and activations with the shapes and distributions of the
Llama-shaped workloads (fp16 weights ~ N(0, sigma), activations ~ N(0, 1) with
a seeded fraction of input channels scaled up as outliers).

Random numbers: numpy ``Generator(PCG64(seed))``; normals are drawn in float64
and rounded once to fp16.  Seeds: ``seed_of(cfg, layer, slot, tensor)``.
"""
from __future__ import annotations

import numpy as np

# (name, N out, K in) of one Llama-3-8B-shaped decoder layer
LLAMA3_8B_LINEARS = (
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336),
)
# (name, N out, K in) of the Llama-3-70B-shaped single-GPU linears
LLAMA3_70B_LINEARS = (
    ("qo", 8192, 8192), ("kv", 1024, 8192), ("gate_up", 28672, 8192), ("down", 8192, 28672),
)
SLOTS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6,
         "attn_in": 7, "mlp_in": 8, "down_in": 9,
         "qo": 0, "kv": 1, "gate_up": 4}
# which distinct input feeds each linear (q/k/v share the attention input,
# gate/up share the MLP input; o and down have their own)
INPUT_OF = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o",
            "gate": "mlp_in", "up": "mlp_in", "down": "down_in",
            "qo": "qo", "kv": "kv", "gate_up": "gate_up"}
TENSOR_W, TENSOR_XCAL, TENSOR_XRUN, TENSOR_PERM = 0, 1, 2, 3


def seed_of(cfg: int, layer: int, slot: int, tensor: int) -> int:
    return 1_000_000 * cfg + 1_000 * layer + 10 * slot + tensor


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def weights(n: int, k: int, sigma: float, seed: int) -> np.ndarray:
    """fp16 [n, k], iid N(0, sigma) drawn in float64 then rounded to fp16."""
    return (rng(seed).standard_normal((n, k)) * sigma).astype(np.float16)


def outlier_channels(k: int, frac: float, seed: int) -> np.ndarray:
    """round(frac * k) distinct channels chosen by a seeded permutation."""
    count = int(round(frac * k))
    return np.sort(rng(seed).permutation(k)[:count])


def activations(m: int, k: int, seed: int, channels: np.ndarray | None = None,
                mult: float = 1.0) -> np.ndarray:
    """fp16 [m, k]: iid N(0, 1), the given channels multiplied by ``mult`` in
    float64 before the single fp16 rounding."""
    x = rng(seed).standard_normal((m, k))
    if channels is not None and len(channels):
        x[:, channels] *= mult
    return x.astype(np.float16)


def activations_bf16(m: int, k: int, seed: int, channels: np.ndarray | None = None,
                     mult: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) [m, k] of the same draws as ``activations``:
    float64 values rounded to float32, then to the nearest bf16 (ties to even
    on the float32 bits)."""
    x = rng(seed).standard_normal((m, k))
    if channels is not None and len(channels):
        x[:, channels] *= mult
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def config_layer(cfg: int, name: str, n: int, k: int, m_cal: int, m_run: int,
                 sigma: float, frac: float, mult: float, layer: int = 0):
    """Weights, calibration tokens and run-time tokens of one linear."""
    slot = SLOTS[name]
    inp = INPUT_OF[name]
    islot = SLOTS.get(inp, slot)
    w = weights(n, k, sigma, seed_of(cfg, layer, slot, TENSOR_W))
    ch = outlier_channels(k, frac, seed_of(cfg, layer, islot, TENSOR_PERM))
    x_cal = activations(m_cal, k, seed_of(cfg, layer, islot, TENSOR_XCAL), ch, mult)
    x_run = activations(m_run, k, seed_of(cfg, layer, islot, TENSOR_XRUN), ch, mult) if m_run else None
    return w, x_cal, x_run, ch


# Workload descriptions (sizes and distributions of the five configurations).
CONFIGS = {
    1: dict(linears=(("q", 4096, 4096),), sigma=0.02, frac=0.01, mult=20.0, m_cal=128, m_run=(1,), g=(128,)),
    2: dict(linears=LLAMA3_8B_LINEARS, sigma=0.02, frac=0.01, mult=20.0, m_cal=128, m_run=(1, 8), g=(128,)),
    3: dict(linears=LLAMA3_8B_LINEARS, sigma=0.02, frac=0.01, mult=20.0, m_cal=512, m_run=(2048,), g=(128,)),
    4: dict(linears=LLAMA3_70B_LINEARS, sigma=0.015, frac=0.005, mult=30.0, m_cal=128, m_run=(1, 16), g=(128,)),
    5: dict(linears=LLAMA3_8B_LINEARS, sigma=0.02, frac=0.01, mult=20.0, m_cal=128, m_run=(1, 32), g=(64, 128), layers=32),
}


def torch_weights(n: int, k: int, sigma: float, seed: int, device):
    """Large-size variant drawn on the device with torch's seeded generator
    (used where numpy generation of hundreds of millions of values would
    dominate set-up time).  Same distribution, different stream of numbers."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return (torch.randn((n, k), generator=gen, device=device, dtype=torch.float32) * sigma).half()


def torch_activations(m: int, k: int, seed: int, channels, mult: float, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn((m, k), generator=gen, device=device, dtype=torch.float32)
    if channels is not None and len(channels):
        idx = torch.as_tensor(np.asarray(channels), device=device, dtype=torch.long)
        x[:, idx] *= mult
    return x.half()
