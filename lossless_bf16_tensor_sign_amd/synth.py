"""Seeded synthetic bf16 workloads (numpy only; no codec arithmetic here).

These stand in for the communication buffers the ZipCCL pages measure on
(parameters in an FSDP all-gather, gradients in a reduce-scatter, MoE
activations in an all-to-all, and a uniform-random stress case the pith page
proposes as the test that would break a Gaussian-tuned code).  No real
training tensors are available, so each buffer is drawn from a stated
distribution with a fixed seed.

Every chunk is generated from its own seeded stream, so one chunk can be
rebuilt alone (CPU tests use this to check a few chunks of a 512 MiB buffer).
Values are drawn in float32 and rounded to bf16 with round-to-nearest-even on
the bit pattern; buffers are uint16 bit patterns.

Workloads (sizes are the full ones):
  1  one chunk of 2^20 values, N(0, 0.02^2)
  2  64 chunks x 2^22 values; chunk c is N(0, s_c^2), s_c log-uniform in
     [0.005, 0.05]
  3  64 chunks x 2^22 values of N(0, 1e-4^2); each value independently is
     replaced by +0.0 with probability 1 %, or by 100 * 1e-4 * t with t drawn
     from Student-t(3) with probability 0.1 %
  4  16384 tokens x 7168 channels, value = s_h * z with s_h ~ LogNormal(0, 0.5)
     per channel and z ~ N(0, 1); token counts of 64 experts drawn
     multinomially with p_e proportional to (e + 1)^-1.1; rows grouped by
     expert (the all-to-all send layout), so chunk e holds count_e rows
  5  64 chunks x 2^22 uniformly random 16-bit patterns (NaN, Inf,
     subnormals and both zeros included)
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20260000

NAMES = {
    1: "gauss_2^20_single_chunk",
    2: "fsdp_allgather_64x4Mi_sigma_loguniform",
    3: "grad_reducescatter_64x4Mi_zeros_t3_outliers",
    4: "moe_alltoall_16384x7168_zipf64",
    5: "uniform_random_bits_64x4Mi",
}

TOKENS, HIDDEN, EXPERTS = 16384, 7168, 64
CHUNK_4MI = 1 << 22


def default_seed(cfg: int) -> int:
    return SEED_BASE + cfg


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b >> 16) & 1
    r += 0x7FFF
    r += b
    r >>= 16
    return r.astype(np.uint16)


def counts(cfg: int, seed: int | None = None) -> np.ndarray:
    """Values per chunk, in chunk order."""
    seed = default_seed(cfg) if seed is None else seed
    if cfg == 1:
        return np.array([1 << 20], np.int64)
    if cfg in (2, 3, 5):
        return np.full(64, CHUNK_4MI, np.int64)
    if cfg == 4:
        rng = np.random.default_rng([seed, 1_000_001])
        p = (np.arange(EXPERTS) + 1.0) ** -1.1
        p /= p.sum()
        tok = rng.multinomial(TOKENS, p)
        return tok.astype(np.int64) * HIDDEN
    raise ValueError("unknown workload %r" % cfg)


def _sigmas_cfg2(seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 1_000_000])
    return np.exp(rng.uniform(np.log(0.005), np.log(0.05), 64))


def _scales_cfg4(seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 1_000_002])
    return rng.lognormal(0.0, 0.5, HIDDEN).astype(np.float32)


def chunk(cfg: int, c: int, seed: int | None = None) -> np.ndarray:
    """Chunk c of workload cfg, as uint16 bf16 bit patterns."""
    seed = default_seed(cfg) if seed is None else seed
    n = int(counts(cfg, seed)[c])
    rng = np.random.default_rng([seed, c])
    if cfg == 1:
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.float32(0.02)
        return to_bf16_bits(x)
    if cfg == 2:
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.float32(_sigmas_cfg2(seed)[c])
        return to_bf16_bits(x)
    if cfg == 3:
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.float32(1e-4)
        u = rng.random(n, dtype=np.float32)
        zero = u < np.float32(0.01)
        outl = (u >= np.float32(0.01)) & (u < np.float32(0.011))
        x[zero] = np.float32(0.0)
        k = int(outl.sum())
        x[outl] = (100.0 * 1e-4 * rng.standard_t(3, size=k)).astype(np.float32)
        return to_bf16_bits(x)
    if cfg == 4:
        rows = n // HIDDEN
        z = rng.standard_normal((rows, HIDDEN), dtype=np.float32)
        z *= _scales_cfg4(seed)[None, :]
        return to_bf16_bits(z.reshape(-1))
    if cfg == 5:
        return rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    raise ValueError("unknown workload %r" % cfg)


def make(cfg: int, seed: int | None = None, workers: int = 1):
    """Whole buffer (chunks back to back) and the counts array."""
    seed = default_seed(cfg) if seed is None else seed
    cnt = counts(cfg, seed)
    out = np.empty(int(cnt.sum()), np.uint16)
    offs = np.concatenate([[0], np.cumsum(cnt)])

    def fill(c):
        out[offs[c]:offs[c + 1]] = chunk(cfg, c, seed)

    if workers > 1 and len(cnt) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(len(cnt))))
    else:
        for c in range(len(cnt)):
            fill(c)
    return out, cnt


def gaussian_bits(n: int, sigma: float, seed: int) -> np.ndarray:
    """n i.i.d. N(0, sigma^2) values as bf16 bit patterns (test helper)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    return to_bf16_bits(x)
