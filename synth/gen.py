"""Seeded Gaussian draws (numpy PCG64) stored as bf16 bit patterns or fp32."""

import numpy as np


def normal_f32(shape, seed, sigma=1.0):
    """i.i.d. N(0, sigma^2) draws, generated and scaled in fp32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return x


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Works on the fp32 bit pattern: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits.  NaN inputs are kept quiet NaNs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns to float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def normal_bf16(shape, seed, sigma=1.0):
    """N(0, sigma^2) drawn in fp32 then rounded to bf16; returns uint16 bits."""
    return f32_to_bf16_bits(normal_f32(shape, seed, sigma))
