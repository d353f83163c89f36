"""Counter-based random inputs (splitmix64, Vigna 2014) usable on CPU or GPU.

Every value is a pure function of (seed, stream, flat index), so any slice of
any tensor (one expert's weight matrix, a subset of tokens) can be generated on
its own and on either device with the same integer results. Uniforms have 53
random bits; normals use the Box-Muller transform in float64 on the pair of
uniforms (2i, 2i+1).

Integer arithmetic runs in torch.int64, whose multiplication wraps modulo 2^64
on both CPU and GPU; logical right shifts are written as an arithmetic shift
followed by a mask.

Streams: 0 = x, 1 = router logits, 2 = per-expert logit bias, 3 = W1, 4 = W2.
"""
from __future__ import annotations

import math

import torch

_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB

STREAM_X, STREAM_LOGITS, STREAM_BIAS, STREAM_W1, STREAM_W2 = 0, 1, 2, 3, 4


def _s64(v: int) -> int:
    """Reinterpret an unsigned 64-bit constant as a signed int64."""
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


def _mix_py(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * _MIX1) & _M64
    z = ((z ^ (z >> 27)) * _MIX2) & _M64
    return z ^ (z >> 31)


def splitmix64_ref(seed: int, stream: int, index: int) -> int:
    """Plain-Python definition of one generator output (used to pin the torch
    version): key = mix(mix(seed) ^ stream*golden); out = mix(key + (index+1)*golden)."""
    key = _mix_py(_mix_py(seed) ^ ((stream * _GOLDEN) & _M64))
    return _mix_py((key + (index + 1) * _GOLDEN) & _M64)


def _key(seed: int, stream: int) -> int:
    return _mix_py(_mix_py(seed) ^ ((stream * _GOLDEN) & _M64))


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix_t(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_MIX1)
    z = (z ^ _lsr(z, 27)) * _s64(_MIX2)
    return z ^ _lsr(z, 31)


def _raw(seed: int, stream: int, start: int, n: int, device) -> torch.Tensor:
    idx = torch.arange(start + 1, start + 1 + n, dtype=torch.int64, device=device)
    z = idx * _s64(_GOLDEN) + _s64(_key(seed, stream))
    return _mix_t(z)


def uniform(seed: int, stream: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """n float64 uniforms in [0, 1) for counters start .. start+n-1."""
    z = _raw(seed, stream, start, n, device)
    return _lsr(z, 11).to(torch.float64) * (1.0 / (1 << 53))


def normal(seed: int, stream: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """n float64 N(0,1) values; value i uses uniforms 2(start+i) and 2(start+i)+1."""
    u = uniform(seed, stream, 2 * start, 2 * n, device).view(n, 2)
    r = torch.sqrt(-2.0 * torch.log1p(-u[:, 0]))
    return r * torch.cos((2.0 * math.pi) * u[:, 1])


def make_x(seed: int, T: int, H: int, device="cpu", token0: int = 0) -> torch.Tensor:
    """Activations x ~ N(0,1), rounded to bf16 (round-to-nearest-even). Rows
    token0 .. token0+T-1 of the full [T_total, H] tensor."""
    v = normal(seed, STREAM_X, token0 * H, T * H, device)
    return v.to(torch.float32).to(torch.bfloat16).view(T, H)


def make_logits(seed: int, T: int, E: int, kind: str, device="cpu", bias_sigma: float = 0.5,
                zipf_s: float = 1.1) -> torch.Tensor:
    """Router logits [T, E] fp32.

    kind: "normal"   N(0,1)
          "normal_bias" N(0,1) + b_e with b_e ~ N(0, bias_sigma^2) per expert
          "uniform"  U[0,1)
          "zipf"     N(0,1) - zipf_s * ln(e+1): expert popularity falls off as
                     a Zipf(s) law in the expert index (expert 0 hottest)
    """
    if kind == "uniform":
        v = uniform(seed, STREAM_LOGITS, 0, T * E, device).view(T, E)
    else:
        v = normal(seed, STREAM_LOGITS, 0, T * E, device).view(T, E)
        if kind == "normal_bias":
            v = v + bias_sigma * normal(seed, STREAM_BIAS, 0, E, device).view(1, E)
        elif kind == "zipf":
            e = torch.arange(E, dtype=torch.float64, device=device)
            v = v - zipf_s * torch.log(e + 1.0).view(1, E)
        elif kind != "normal":
            raise ValueError(f"unknown logits kind {kind!r}")
    return v.to(torch.float32).contiguous()


def make_weight(seed: int, stream: int, e: int, N: int, K: int, device="cpu") -> torch.Tensor:
    """One expert's [N, K] fp32 weight matrix ~ N(0, 1/K) (variance 1/fan_in)."""
    v = normal(seed, stream, e * N * K, N * K, device)
    return (v * (1.0 / math.sqrt(K))).to(torch.float32).view(N, K)


def make_expert_weights(seed: int, E: int, N1: int, H: int, I: int, device="cpu",
                        experts=None):
    """W1 [E, N1, H] and W2 [E, H, I] fp32 (or only the listed experts, stacked
    in the order given)."""
    ex = list(range(E)) if experts is None else list(experts)
    w1 = torch.empty((len(ex), N1, H), dtype=torch.float32, device=device)
    w2 = torch.empty((len(ex), H, I), dtype=torch.float32, device=device)
    for i, e in enumerate(ex):
        w1[i] = make_weight(seed, STREAM_W1, e, N1, H, device)
        w2[i] = make_weight(seed, STREAM_W2, e, H, I, device)
    return w1, w2
