"""Distances between BF16 bit patterns for the cache checks.

bf16_steps(a, b): how many representable BF16 values apart two patterns are,
sign-aware (+0 and -0 are the same point; the smallest positive and negative
subnormals are two steps apart, with zero between them)."""
import numpy as np


def bf16_ord(bits):
    """Map BF16 bit patterns (uint16) to integers in the order of their values,
    consecutive representable values to consecutive integers."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_steps(a, b):
    return np.abs(bf16_ord(a) - bf16_ord(b))
