"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the reduce itself: it only draws random
partials with the shapes and value distributions of the decode and prefill
activations the pages talk about (one hidden vector for token generation,
``tokens x hidden`` for prompt processing) and hands them out as numpy arrays.
Both the CPU oracle and the HIP library consume exactly these bytes.

Every draw uses ``numpy.random.default_rng(SeedSequence([case, set, rank]))`` so
any single rank of any call or rotation set can be regenerated on its own.

Wire-typed sources (buffers a peer has already narrowed) are produced here by a
generator choice that is *not* the method's rounding: bfloat16 partials keep the
upper 16 bits of a float32 draw (truncation), float16 partials come from
numpy's ``astype(float16)``.  The reduce treats such buffers as given bits.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity configuration."""

    case: int            # seed namespace
    name: str
    R: int               # simulated ranks
    shape: tuple         # activation shape; n = prod(shape)
    wire: int            # wire type
    dist: str            # value distribution of the partials
    mode: str            # schedule the configuration exercises
    calls: int = 1       # sequential calls with fresh data (decode)

    @property
    def n(self) -> int:
        return int(np.prod(self.shape))


# The five configurations: decode vector (fp32 wire / bf16 wire), prefill
# 2048 tokens x 4096 hidden, a 4-rank slice + broadcast schedule over
# 2048 x 8192, and an 8-rank 8192 x 8192 reduce staged from host memory.
WORKLOADS = {
    "decode_f32": Workload(1, "decode_f32", 2, (4096,), F32, "normal", "single_shot"),
    "decode_bf16": Workload(2, "decode_bf16", 2, (4096,), BF16, "normal*0.05", "single_shot",
                            calls=10_000),
    "prefill_bf16": Workload(3, "prefill_bf16", 2, (2048, 4096), BF16, "normal+outliers",
                             "chunked"),
    "slice_bcast_f16": Workload(4, "slice_bcast_f16", 4, (2048, 8192), F16, "normal(0,0.5)",
                                "rs_bcast"),
    "host_staged_bf16": Workload(5, "host_staged_bf16", 8, (8192, 8192), BF16, "uniform(-1,1)",
                                 "host_staged"),
}


def rng_for(case: int, set_idx: int, rank: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([case, set_idx, rank]))


def draw(dist: str, n: int, rng: np.random.Generator) -> np.ndarray:
    """float32 partial of length n from the named distribution."""
    if dist == "normal":
        return rng.standard_normal(n, dtype=np.float32)
    if dist == "normal*0.05":
        return rng.standard_normal(n, dtype=np.float32) * np.float32(0.05)
    if dist == "normal+outliers":
        # N(0,1) with an iid 0.1% of elements scaled by 100 (activation outliers)
        x = rng.standard_normal(n, dtype=np.float32)
        mask = rng.random(n, dtype=np.float32) < np.float32(0.001)
        x[mask] *= np.float32(100.0)
        return x
    if dist == "normal(0,0.5)":
        return rng.standard_normal(n, dtype=np.float32) * np.float32(0.5)
    if dist == "uniform(-1,1)":
        return rng.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    if dist == "wide":
        # magnitudes spread over many binades, both signs: exercises rounding
        # at every exponent and the fp16 overflow / underflow edges
        mant = rng.random(n, dtype=np.float32) + np.float32(1.0)
        expo = rng.integers(-30, 20, n).astype(np.float32)
        sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
        return (sign * mant * np.exp2(expo)).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def partials(w: Workload, set_idx: int = 0, n: int | None = None) -> list[np.ndarray]:
    """The R float32 partials of one call / rotation set of workload ``w``."""
    n = w.n if n is None else n
    return [draw(w.dist, n, rng_for(w.case, set_idx, r)) for r in range(w.R)]


def random_partials(case: int, set_idx: int, R: int, n: int, dist: str = "normal") -> list[np.ndarray]:
    """R float32 partials of length n for ad-hoc parity cases."""
    return [draw(dist, n, rng_for(case, set_idx, r)) for r in range(R)]


def as_wire_typed(x: np.ndarray, wire: int) -> np.ndarray:
    """Synthetic wire-typed buffer (uint16 bit patterns) derived from a float32 draw.

    bf16: the upper half of each float32 (truncation -- a generator choice);
    f16: numpy's float16 conversion.  float32 wire returns the array itself.
    """
    if wire == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if wire == BF16:
        return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if wire == F16:
        with np.errstate(over="ignore"):
            return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    raise ValueError(wire)


def special_values() -> np.ndarray:
    """float32 values at the edges of every wire type (bit-exact constants)."""
    bits = [
        0x00000000, 0x80000000,              # +0, -0
        0x00000001, 0x80000001,              # min subnormal
        0x007FFFFF, 0x807FFFFF,              # max subnormal
        0x00008000, 0x00018000,              # bf16 subnormal ties
        0x00800000,                          # min normal
        0x3F800000, 0xBF800000,              # +-1
        0x3F808000, 0x3F818000, 0x3F808008,  # bf16 ties / above tie
        0x3F801000, 0x3F803000,              # f16 ties
        0x33000000, 0x33C00000,              # f16 subnormal ties (2^-25, 3*2^-25)
        0x387FC000, 0x387FE000, 0x38800000,  # around f16 min normal
        0x477FE000, 0x477FF000, 0xC77FF000,  # 65504, 65520, -65520
        0x477FEFFF,                          # just below the f16 overflow tie
        0x7F7FFFFF, 0xFF7FFFFF,              # +-FLT_MAX
        0x7F7F8000, 0x7F7F7FFF,              # bf16 overflow tie / just below
        0x7F800000, 0xFF800000,              # +-inf
        0x4B800000, 0x4B800001,              # 2^24, 2^24 + 2
        0x3B800000, 0xBB800000,              # +-2^-8
        0x3F7FFFFF, 0x3FFFFFFF,              # just below 1, just below 2
        0x1E3CE508, 0x9E3CE508,              # small normals
        0x5F000000, 0xDF000000,              # +-2^63
    ]
    return np.array(bits, dtype=np.uint32).view(np.float32)


def nan_values() -> np.ndarray:
    """A few NaN encodings (quiet, signalling, negative)."""
    return np.array([0x7FC00000, 0x7F800001, 0xFFC00001, 0x7FBFFFFF], dtype=np.uint32).view(np.float32)


def special_values16(wire: int) -> np.ndarray:
    """16-bit edge patterns of a wire / destination type (uint16 bit constants):
    signed zeros, smallest / largest subnormals, smallest normal, +-1 and its
    neighbours, the largest finite values, infinities and a few small powers
    of two that tie when added to 1."""
    if wire == F16:
        bits = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x8400,
                0x3C00, 0xBC00, 0x3C01, 0x3BFF, 0x1000, 0x9000, 0x1400, 0x0C00,
                0x7BFF, 0xFBFF, 0x7BFE, 0x7C00, 0xFC00, 0x5BFF, 0x4000, 0xC000]
    elif wire == BF16:
        bits = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080,
                0x3F80, 0xBF80, 0x3F81, 0x3F7F, 0x3B80, 0xBB80, 0x3C00, 0x3B00,
                0x7F7F, 0xFF7F, 0x7F7E, 0x7F80, 0xFF80, 0x4B80, 0x4000, 0xC000]
    else:
        raise ValueError(wire)
    return np.array(bits, dtype=np.uint16)


def nan_values16(wire: int) -> np.ndarray:
    """Two NaN encodings of a 16-bit type."""
    return np.array([0x7E00, 0xFD01] if wire == F16 else [0x7FC0, 0xFF81], dtype=np.uint16)


def random_narrow(case: int, set_idx: int, R: int, n: int, dtype: int, dist: str = "normal") -> list[np.ndarray]:
    """R partials already held in a 16-bit type (uint16 bit patterns), made from
    float32 draws by the same generator choice as ``as_wire_typed``."""
    return [as_wire_typed(x, dtype) for x in random_partials(case, set_idx, R, n, dist)]


def residual(case: int, set_idx: int, length: int, dtype: int = F32, dist: str = "normal") -> np.ndarray:
    """A residual stream of the destination type: float32, or uint16 bit patterns."""
    x = draw(dist, length, rng_for(case, set_idx, 1000))
    return x if dtype == F32 else as_wire_typed(x, dtype)
