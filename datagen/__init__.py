"""Seeded synthetic inputs for the device-scan workloads.

This module is shared by the tests, the benchmark and the smoke check, and
feeds both the oracle and the HIP library identical bytes. It holds no scan,
reduction or compaction arithmetic: only a counter-based random generator and
the value distributions the workloads are stated in.

Generator: Vigna's SplitMix64. Output i of a generator seeded with `seed` is
the SplitMix64 finaliser applied to ``seed + (i + 1) * 0x9E3779B97F4A7C15``
(mod 2**64), so any slice of the stream can be made without the ones before.

Workloads (n, dtype, values), one documented seed each:
  one_tile      int32, n = 4,096,        uniform integers in [0, 9],       seed 1
  mid           int32, n = 1,048,576,    uniform integers in [0, 100],     seed 2
  fp32_10m      fp32,  n = 10,000,000,   uniform in [0, 1),                seed 3
  int32_100m    int32, n = 100,000,007,  uniform integers in [-1000,1000], seed 4
  fp32_100m     fp32,  n = 100,000,007,  standard normal (Box-Muller),     seed 4
  compact_256m  uint32, n = 268,435,456, uniform over [0, 2**32),          seed 5
                (also the keys of the counting-sort pass)
  moe_64k       int32 router choices: 65,536 tokens x top-8 of 256 experts,
                Zipf(1) expert popularity, distinct experts per token,  seed 6

Router choices (moe_topk_ids): expert e gets popularity weight
1 / rank(e)^skew, rank a seeded permutation of the experts; each token draws
top_k distinct experts with probability in proportion to those weights
(Gumbel top-k: the k largest log-weight + Gumbel-noise scores), listed
highest score first.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 20

# workload name -> (n, dtype, seed)
WORKLOADS = {
    "one_tile": (4096, "int32", 1),
    "mid": (1_048_576, "int32", 2),
    "fp32_10m": (10_000_000, "float32", 3),
    "int32_100m": (100_000_007, "int32", 4),
    "fp32_100m": (100_000_007, "float32", 4),
    "compact_256m": (268_435_456, "uint32", 5),
}

# MoE routing workloads: name -> (num_tokens, top_k, num_experts, block, skew, seed)
MOE_WORKLOADS = {
    "moe_64k": (65_536, 8, 256, 64, 1.0, 6),
    "moe_decode": (256, 8, 256, 64, 1.0, 7),
}


def splitmix64(seed: int, start: int, count: int, out: np.ndarray | None = None) -> np.ndarray:
    """Outputs start .. start+count-1 of SplitMix64 seeded with `seed` (uint64)."""
    z = np.arange(start + 1, start + count + 1, dtype=np.uint64) if out is None else out
    if out is not None:
        z[:] = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    t = np.empty_like(z)
    with np.errstate(over="ignore"):
        np.multiply(z, GAMMA, out=z)
        np.add(z, np.uint64(seed % (1 << 64)), out=z)
        np.right_shift(z, np.uint64(30), out=t)
        np.bitwise_xor(z, t, out=z)
        np.multiply(z, _M1, out=z)
        np.right_shift(z, np.uint64(27), out=t)
        np.bitwise_xor(z, t, out=z)
        np.multiply(z, _M2, out=z)
        np.right_shift(z, np.uint64(31), out=t)
        np.bitwise_xor(z, t, out=z)
    return z


def _chunked(n: int, out_dtype, fn) -> np.ndarray:
    out = np.empty(n, dtype=out_dtype)
    for s in range(0, n, _CHUNK):
        c = min(_CHUNK, n - s)
        out[s:s + c] = fn(s, c)
    return out


def uniform_int(seed: int, n: int, lo: int, hi: int, dtype=np.int32) -> np.ndarray:
    """Integers uniform in [lo, hi]: lo + floor(top32(u) * (hi - lo + 1) / 2**32)."""
    span = np.uint64(hi - lo + 1)
    assert 0 < int(span) <= (1 << 32)

    def f(s, c):
        u = splitmix64(seed, s, c) >> np.uint64(32)
        return (np.int64(lo) + ((u * span) >> np.uint64(32)).astype(np.int64)).astype(dtype)

    return _chunked(n, dtype, f)


def uniform01_f32(seed: int, n: int) -> np.ndarray:
    """fp32 uniform in [0, 1): top 24 bits of u times 2**-24 (exact in fp32)."""
    def f(s, c):
        u = splitmix64(seed, s, c) >> np.uint64(40)
        return u.astype(np.float32) * np.float32(2.0 ** -24)

    return _chunked(n, np.float32, f)


def normal_f32(seed: int, n: int) -> np.ndarray:
    """fp32 standard normal by Box-Muller in float64, from draws 2i and 2i+1."""
    def f(s, c):
        u = splitmix64(seed, 2 * s, 2 * c)
        a = ((u[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53  # (0, 1]
        b = (u[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53          # [0, 1)
        return (np.sqrt(-2.0 * np.log(a)) * np.cos(2.0 * np.pi * b)).astype(np.float32)

    return _chunked(n, np.float32, f)


def keys_u32(seed: int, n: int) -> np.ndarray:
    """uint32 keys uniform over [0, 2**32): the low 32 bits of each draw."""
    def f(s, c):
        return (splitmix64(seed, s, c) & np.uint64(0xFFFFFFFF)).astype(np.uint32)

    return _chunked(n, np.uint32, f)


def uniform_i64(seed: int, n: int, bits: int) -> np.ndarray:
    """int64 uniform in [-2**bits, 2**bits) from the top bits+1 bits of each draw."""
    def f(s, c):
        u = splitmix64(seed, s, c) >> np.uint64(63 - bits)
        return u.astype(np.int64) - np.int64(1 << bits)

    return _chunked(n, np.int64, f)


def raw_u64(seed: int, n: int) -> np.ndarray:
    """Raw 64-bit draws (uint64): inputs that wrap a 64-bit sum at once."""
    return _chunked(n, np.uint64, lambda s, c: splitmix64(seed, s, c))


def quarter_twos_f32(n: int) -> np.ndarray:
    """1.0 everywhere except 2.0 at every index i with i % 4 == 3.

    Every prefix of this input is an integer below 2**24 for n < 1.3e7, so it
    is exact in fp32 whatever order the additions take.
    """
    x = np.ones(n, dtype=np.float32)
    x[3::4] = 2.0
    return x


def mod8_plus1(n: int, dtype=np.float32) -> np.ndarray:
    """x_i = (i % 8) + 1."""
    return ((np.arange(n, dtype=np.int64) % 8) + 1).astype(dtype)


def moe_topk_ids(seed: int, num_tokens: int, top_k: int, num_experts: int, skew: float = 1.0) -> np.ndarray:
    """int32 [num_tokens, top_k]: distinct experts per token, Zipf(skew) popularity."""
    assert 1 <= top_k <= num_experts
    rank = np.empty(num_experts, dtype=np.int64)
    rank[np.argsort(splitmix64(seed, 0, num_experts), kind="stable")] = np.arange(num_experts)
    logw = -skew * np.log((rank + 1).astype(np.float64))
    out = np.empty((num_tokens, top_k), dtype=np.int32)
    step = max(1, _CHUNK // num_experts)
    for t0 in range(0, num_tokens, step):
        c = min(step, num_tokens - t0)
        u = ((splitmix64(seed + 1, t0 * num_experts, c * num_experts) >> np.uint64(11)).astype(np.float64) + 0.5) \
            * 2.0 ** -53
        score = logw[None, :] - np.log(-np.log(u.reshape(c, num_experts)))
        top = np.argpartition(-score, top_k - 1, axis=1)[:, :top_k]
        order = np.argsort(-np.take_along_axis(score, top, axis=1), axis=1, kind="stable")
        out[t0:t0 + c] = np.take_along_axis(top, order, axis=1)
    return out


def moe_workload(name: str) -> np.ndarray:
    t, k, e, _, skew, seed = MOE_WORKLOADS[name]
    return moe_topk_ids(seed, t, k, e, skew)


def workload(name: str, n: int | None = None) -> np.ndarray:
    """The named workload's input (optionally truncated or extended to n)."""
    wn, dt, seed = WORKLOADS[name]
    n = wn if n is None else n
    if name == "one_tile":
        return uniform_int(seed, n, 0, 9)
    if name == "mid":
        return uniform_int(seed, n, 0, 100)
    if name == "fp32_10m":
        return uniform01_f32(seed, n)
    if name == "int32_100m":
        return uniform_int(seed, n, -1000, 1000)
    if name == "fp32_100m":
        return normal_f32(seed, n)
    if name == "compact_256m":
        return keys_u32(seed, n)
    raise KeyError(name)
