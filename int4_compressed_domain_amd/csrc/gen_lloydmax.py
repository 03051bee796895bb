"""Derive the 16-entry key codebook compiled into the kernels (TQ_LUT16_BITS in tq_device.h).

The codebook is the 16-level Lloyd-Max quantizer of a standard normal variable
("TurboQuant on AMD GPUs", section 2: keys use rotation + LUT quantization), divided by
sqrt(32) because a coordinate of a unit-norm group of 32 rotated values has variance 1/32,
and rounded to fp16 (round to nearest even). Run as a script to print the table.

Lloyd's fixed point: every level is the mean of N(0,1) over its cell, and cell edges are
midpoints of neighbouring levels. Pure Python (math.erf), no third-party code.
"""
import math
import struct


def _pdf(x):
    return 0.0 if math.isinf(x) else math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cdf(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def levels(n=16, tol=1e-15, max_iter=200000):
    c = [-2.5 + 5.0 * (i + 0.5) / n for i in range(n)]
    for _ in range(max_iter):
        edges = [-math.inf] + [0.5 * (c[i] + c[i + 1]) for i in range(n - 1)] + [math.inf]
        new = [(_pdf(edges[i]) - _pdf(edges[i + 1])) / (_cdf(edges[i + 1]) - _cdf(edges[i]))
               for i in range(n)]
        delta = max(abs(a - b) for a, b in zip(new, c))
        c = new
        if delta < tol:
            break
    half = [0.5 * (c[n - 1 - i] - c[i]) for i in range(n // 2)]  # symmetric refinement
    return [-v for v in half] + half[::-1]


def fp16_bits(x):
    return struct.unpack("<H", struct.pack("<e", x))[0]


def lut_bits():
    return [fp16_bits(m / math.sqrt(32.0)) for m in levels()]


if __name__ == "__main__":
    print(", ".join("0x%04xu" % b for b in lut_bits()))
