"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module draws random numbers and casts them; it holds none of the scan's arithmetic.
Shapes, distributions and structure follow the workloads the selective-scan pages and the
shipped configurations describe (Mamba-style layers with d_state = 16; the per-channel
elementwise form of "15. Selective (Data-Dependent) SSM Scan", whose example uses
A = sigmoid(randn), h0 = 0).  There is no dataset or trained weight anywhere: the
"Mamba-130M/2.8B-shaped" configurations only borrow layer shapes (d_inner 1536 / 5120).

Layouts (row-major): x, delta, z, y: (batch, seqlen, dim); B, C: (batch, seqlen, dstate);
A: (dim, dstate); D: (dim,); h0, h_last: (batch, dim, dstate).  Elementwise form: x, A, B, C,
y: (batch, seqlen, dim); h0, h_last: (batch, dim).

bf16 tensors are uint16 arrays of raw bf16 bits, rounded from fp32 to nearest-even; both
sides consume the identical bits.
"""
from __future__ import annotations

import math

import numpy as np

# log(e^0.01 - 1): shifts softplus so that the median step is 0.01.
DELTA_SHIFT = math.log(math.expm1(0.01))

CONFIGS = [
    dict(name="elementwise_fp32_b2_L64_d4", api="elementwise", batch=2, seqlen=64, dim=4,
         h0=False, h0_std=None),
    dict(name="selective_fp32_b2_D64_N16_L512", api="selective", batch=2, dim=64, dstate=16, seqlen=512,
         io="f32", with_D=True, with_z=False, h0=False, h0_std=None, h_last=True),
    dict(name="selective_bf16_b8_D1536_N16_L2048", api="selective", batch=8, dim=1536, dstate=16, seqlen=2048,
         io="bf16", with_D=True, with_z=True, h0=False, h0_std=None, h_last=True),
    dict(name="selective_bf16_b1_D5120_N16_L65536", api="selective", batch=1, dim=5120, dstate=16,
         seqlen=65536, io="bf16", with_D=True, with_z=True, h0=True, h0_std=0.1, h_last=True),
    dict(name="elementwise_fp32_b8_L32768_d4096", api="elementwise", batch=8, seqlen=32768, dim=4096,
         h0=True, h0_std=1.0),
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return the raw 16-bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def _sigmoid(v: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * v))


def selective_inputs(batch, seqlen, dim, dstate, *, io="f32", with_D=True, with_z=False, h0=False,
                     h0_std=0.1, seed=0, large=False):
    """Mamba-form inputs.  Draw order: A_u, delta noise, B, C, x, D, z, h0.

    A[d, n] = -exp(U(0, ln 16)); delta = softplus(0.5 * N(0,1) + log(e^0.01 - 1)) per
    (b, t, d); B, C ~ N(0,1) per (b, t, n), shared by every channel; x, D, z ~ N(0,1);
    h0 ~ N(0, h0_std^2) when requested.  ``large`` draws float32 directly (same
    distributions) to bound host memory on the big shapes.
    """
    rng = np.random.default_rng(seed)
    fdt = np.float32 if large else np.float64
    A_u = rng.random((dim, dstate), dtype=fdt)
    A = (-np.exp(A_u * math.log(16.0))).astype(np.float32)
    dn = rng.standard_normal((batch, seqlen, dim), dtype=fdt)
    delta = _softplus(dn * fdt(0.5) + fdt(DELTA_SHIFT)).astype(np.float32)
    del dn
    B = rng.standard_normal((batch, seqlen, dstate), dtype=fdt).astype(np.float32)
    C = rng.standard_normal((batch, seqlen, dstate), dtype=fdt).astype(np.float32)
    x = rng.standard_normal((batch, seqlen, dim), dtype=fdt).astype(np.float32)
    D = rng.standard_normal((dim,), dtype=fdt).astype(np.float32) if with_D else None
    z = rng.standard_normal((batch, seqlen, dim), dtype=fdt).astype(np.float32) if with_z else None
    h0a = (rng.standard_normal((batch, dim, dstate), dtype=fdt) * h0_std).astype(np.float32) if h0 else None
    if io == "bf16":
        x = f32_to_bf16_bits(x)
        delta = f32_to_bf16_bits(delta)
        z = f32_to_bf16_bits(z) if z is not None else None
    elif io != "f32":
        raise ValueError(io)
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h0a, io=io)


def elementwise_inputs(batch, seqlen, dim, *, h0=False, h0_std=1.0, seed=0, large=False):
    """Elementwise-form inputs.  Draw order: x, A noise, B, C, h0.

    x, B, C ~ N(0,1); A = sigmoid(N(0,1)) per (b, t, d), in (0, 1); h0 ~ N(0, h0_std^2).
    """
    rng = np.random.default_rng(seed)
    fdt = np.float32 if large else np.float64
    x = rng.standard_normal((batch, seqlen, dim), dtype=fdt).astype(np.float32)
    an = rng.standard_normal((batch, seqlen, dim), dtype=fdt)
    A = _sigmoid(an).astype(np.float32)
    del an
    B = rng.standard_normal((batch, seqlen, dim), dtype=fdt).astype(np.float32)
    C = rng.standard_normal((batch, seqlen, dim), dtype=fdt).astype(np.float32)
    h0a = (rng.standard_normal((batch, dim), dtype=fdt) * h0_std).astype(np.float32) if h0 else None
    return dict(x=x, A=A, B=B, C=C, h0=h0a)


def config_inputs(i: int):
    """Inputs of configuration ``i`` (seed 1000 + i).  Large ones draw float32 directly."""
    cfg = CONFIGS[i]
    large = cfg["batch"] * cfg["seqlen"] * cfg["dim"] > (1 << 26)
    if cfg["api"] == "selective":
        inp = selective_inputs(cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"], io=cfg["io"],
                               with_D=cfg["with_D"], with_z=cfg["with_z"], h0=cfg["h0"],
                               h0_std=cfg["h0_std"] or 0.1, seed=1000 + i, large=large)
    else:
        inp = elementwise_inputs(cfg["batch"], cfg["seqlen"], cfg["dim"], h0=cfg["h0"],
                                 h0_std=cfg["h0_std"] or 1.0, seed=1000 + i, large=large)
    return cfg, inp
