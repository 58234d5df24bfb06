"""Seeded synthetic inputs for the Echo rank pipeline.

Both the HIP path and the CPU oracle consume the bytes this module makes;
it holds none of the method's arithmetic (no correction, quantizer, sum or
average): it only draws numbers.

Generator: counter-based.  Draw i of a stream is SplitMix64 (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
finalizer constants as published by Vigna) applied to key + i, where the
key is itself SplitMix64 of the stream's tags folded in order.  Normals come
from the Box-Muller transform in float64, Student-t(3) from z / sqrt(chi2_3/3),
and bf16 values from torch's round-to-nearest-even float32 -> bfloat16 cast.

Workload recipes follow the shapes and distributions of the pages' settings
(TP=8 serving of Llama-3-8B-shaped hidden states, Qwen3-0.6B-shaped
pretraining activations and gradients, a 1 GB message): synthetic stand-ins,
since no weights, datasets or benchmark suites are used.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output for state values x (uint64 array, wrapping)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _tag(t) -> int:
    if isinstance(t, str):
        return int.from_bytes(hashlib.blake2b(t.encode(), digest_size=8).digest(), "little")
    return int(t) & ((1 << 64) - 1)


def stream_key(*tags) -> int:
    """Fold tags (ints or strings) into one 64-bit stream key."""
    h = np.uint64(0)
    for t in tags:
        h = splitmix64(np.array([h ^ np.uint64(_tag(t))], dtype=np.uint64))[0]
    return int(h)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, fill, dtype) -> np.ndarray:
    """Run fill(lo, hi, out_slice) over chunks of [0, n) on a thread pool."""
    out = np.empty(n, dtype=dtype)
    spans = [(lo, min(n, lo + _CHUNK)) for lo in range(0, n, _CHUNK)]
    if len(spans) <= 1:
        for lo, hi in spans:
            fill(lo, hi, out[lo:hi])
        return out
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda s: fill(s[0], s[1], out[s[0]:s[1]]), spans))
    return out


def _bits(key: int, lo: int, hi: int, lane: int = 0, lanes: int = 1) -> np.ndarray:
    idx = np.arange(lo, hi, dtype=np.uint64) * np.uint64(lanes) + np.uint64(lane)
    with np.errstate(over="ignore"):
        return splitmix64(idx + np.uint64(key))


def _u01_open0(h: np.ndarray) -> np.ndarray:
    """(0, 1]"""
    return ((h >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)


def _u01(h: np.ndarray) -> np.ndarray:
    """[0, 1)"""
    return (h >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def _normal_span(key: int, lo: int, hi: int) -> np.ndarray:
    u1 = _u01_open0(_bits(key, lo, hi, 0, 2))
    u2 = _u01(_bits(key, lo, hi, 1, 2))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def normal(n: int, key: int) -> np.ndarray:
    """n standard normals (float64); draw i depends only on (key, i)."""
    def fill(lo, hi, out):
        out[:] = _normal_span(key, lo, hi)
    return _chunked(n, fill, np.float64)


def uniform(n: int, key: int) -> np.ndarray:
    def fill(lo, hi, out):
        out[:] = _u01(_bits(key, lo, hi))
    return _chunked(n, fill, np.float64)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32/float64 values -> bf16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def outlier_channels(hidden: int, frac: float, key: int) -> np.ndarray:
    """The round(frac*hidden) channels (at least one) with the smallest
    seeded hash: a fixed seeded subset."""
    k = max(1, int(round(frac * hidden)))
    h = splitmix64(np.arange(hidden, dtype=np.uint64) + np.uint64(key))
    return np.sort(np.argsort(h, kind="stable")[:k])


# ---- workload recipes ------------------------------------------------------------

def gaussian_outlier_channels(tokens: int, hidden: int, key: int, sigma: float = 1.0,
                              outlier_mult: float = 20.0, outlier_frac: float = 0.001,
                              channel_key: int | None = None) -> np.ndarray:
    """[tokens x hidden] bf16 bits: N(0, sigma), a fixed 0.1% of channels x mult."""
    z = normal(tokens * hidden, key).reshape(tokens, hidden) * sigma
    ck = key if channel_key is None else channel_key
    z[:, outlier_channels(hidden, outlier_frac, stream_key(ck, "outliers"))] *= outlier_mult
    return to_bf16_bits(z.ravel())


def lognormal_channel_activations(tokens: int, hidden: int, key: int, channel_key: int,
                                  sigma: float = 0.5, channel_sigma: float = 1.0,
                                  outlier_mult: float = 30.0,
                                  outlier_frac: float = 0.001) -> np.ndarray:
    """[tokens x hidden] bf16 bits: sigma * z * lambda_c with lambda_c =
    exp(N(0, channel_sigma)) per channel and a 0.1% outlier subset x mult;
    lambda and the outlier subset depend on channel_key only."""
    lam = np.exp(channel_sigma * normal(hidden, stream_key(channel_key, "lambda")))
    lam[outlier_channels(hidden, outlier_frac, stream_key(channel_key, "outliers"))] *= outlier_mult
    z = normal(tokens * hidden, key).reshape(tokens, hidden)
    return to_bf16_bits((sigma * z * lam[None, :]).ravel())


def student_t3(n: int, key: int, scale: float = 1e-3) -> np.ndarray:
    """n bf16 bits: scale * z / sqrt((z1^2 + z2^2 + z3^2) / 3) (Student-t, nu=3)."""
    z = normal(n, stream_key(key, "z"))
    chi = np.zeros(n)
    for j in range(3):
        chi += normal(n, stream_key(key, "chi", j)) ** 2
    return to_bf16_bits(scale * z / np.sqrt(chi / 3.0))


def vector_with_outliers(n: int, key: int, outlier_mult: float = 20.0,
                         outlier_frac: float = 0.001) -> np.ndarray:
    """n bf16 bits: N(0, 1), elements whose hash falls below frac * 2^64 x mult."""
    thr = np.uint64(int(outlier_frac * 2.0 ** 64))
    okey = stream_key(key, "outliers")

    def fill(lo, hi, out):
        z = _normal_span(key, lo, hi)
        z[_bits(okey, lo, hi) < thr] *= outlier_mult
        out[:] = z
    return to_bf16_bits(_chunked(n, fill, np.float32))


# ---- packed int4 messages (incoming shards, gathered chunks) --------------------

def _valid_code_bytes() -> np.ndarray:
    """All byte values whose two 4-bit fields both differ from 0x8 (the code
    -8, which the quantizer never emits): 225 of the 256 bytes."""
    b = np.arange(256)
    ok = ((b & 0xF) != 8) & ((b >> 4) != 8)
    return b[ok].astype(np.uint8)


def int4_message(n: int, key: int, scale_lo: float = 0.05, scale_hi: float = 0.55,
                 zero_group_frac: float = 0.0, any_byte: bool = False,
                 group: int = 128, bits: int = 4):
    """A seeded message of n codes: (codes u8[n/2] for 4-bit or u8[n] for 8-bit
    codes, scales f32[n/group]).  4-bit: bytes drawn uniformly from the 225
    bytes without a -8 field; 8-bit: from the 255 bytes other than 0x80 (-128);
    all 256 when any_byte.  Scales uniform in [scale_lo, scale_hi); a seeded
    fraction of groups is all-zero (codes 0, scale 0)."""
    if any_byte:
        alphabet = np.arange(256, dtype=np.uint8)
    elif bits == 8:
        alphabet = np.array([b for b in range(256) if b != 0x80], dtype=np.uint8)
    else:
        alphabet = _valid_code_bytes()
    ckey = stream_key(key, "codes")
    nbytes = n if bits == 8 else n // 2

    def fill(lo, hi, out):
        out[:] = alphabet[(_bits(ckey, lo, hi) % np.uint64(alphabet.size)).astype(np.int64)]
    codes = _chunked(nbytes, fill, np.uint8)
    g = n // group
    scales = (scale_lo + (scale_hi - scale_lo) * uniform(g, stream_key(key, "scales"))).astype(np.float32)
    if zero_group_frac > 0.0:
        zg = uniform(g, stream_key(key, "zero")) < zero_group_frac
        scales[zg] = 0.0
        cv = codes.reshape(g, nbytes // g)
        cv[zg] = 0
    return codes, scales


# ---- device-side recipes (torch's seeded Philox generator on the GPU) ------------
# For call sequences too long to draw on the host (the training workload's 112
# calls of 32M elements).  Deterministic for a given seed, shape and device;
# both sides of a comparison read the same device bytes.

def _device_gen(seed: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    return g


def device_lognormal_channel_activations(tokens: int, hidden: int, seed: int, lam, device,
                                         sigma: float = 0.5):
    """bf16 bits (int16 tensor) of sigma * z * lam[c]; lam is the per-channel
    scale (outliers included) from channel_scales()."""
    import torch

    g = _device_gen(seed, device)
    z = torch.randn(tokens, hidden, generator=g, device=device)
    lam_t = torch.as_tensor(lam, dtype=torch.float32, device=device)
    return (sigma * z * lam_t[None, :]).to(torch.bfloat16).view(torch.int16).reshape(-1)


def device_student_t3(n: int, seed: int, device, scale: float = 1e-3):
    """bf16 bits (int16 tensor) of scale * z / sqrt((z1^2 + z2^2 + z3^2) / 3)."""
    import torch

    g = _device_gen(seed, device)
    z = torch.randn(4, n, generator=g, device=device)
    t = z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0)
    return (scale * t).to(torch.bfloat16).view(torch.int16)


def device_message(n: int, seed: int, device, scale_lo: float = 0.05, scale_hi: float = 0.55,
                   bits: int = 4):
    """A seeded message of n codes drawn on the device, with int4_message's
    distribution: (codes u8 tensor, scales f32 tensor [n/128]); 4-bit bytes
    uniform over the 225 without a -8 field, 8-bit bytes over the 255 other
    than 0x80, scales uniform in [scale_lo, scale_hi)."""
    import torch

    g = _device_gen(seed, device)
    if bits == 8:
        alphabet = np.array([b for b in range(256) if b != 0x80], dtype=np.uint8)
        nbytes = n
    else:
        alphabet = _valid_code_bytes()
        nbytes = n // 2
    table = torch.as_tensor(alphabet, device=device)
    codes = table[torch.randint(0, alphabet.size, (nbytes,), generator=g, device=device)]
    scales = scale_lo + (scale_hi - scale_lo) * torch.rand(n // 128, generator=g, device=device)
    return codes.contiguous(), scales.contiguous()


def channel_scales(hidden: int, channel_key: int, channel_sigma: float = 1.0,
                   outlier_mult: float = 30.0, outlier_frac: float = 0.001) -> np.ndarray:
    """Per-channel scale exp(N(0, channel_sigma)), a fixed 0.1% subset x mult
    (the same lambda as lognormal_channel_activations)."""
    lam = np.exp(channel_sigma * normal(hidden, stream_key(channel_key, "lambda")))
    lam[outlier_channels(hidden, outlier_frac, stream_key(channel_key, "outliers"))] *= outlier_mult
    return lam.astype(np.float32)
