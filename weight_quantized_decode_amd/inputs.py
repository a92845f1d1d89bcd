"""Seeded synthetic inputs, shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and lays them out as the canonical
(interchange) byte format of each packed weight type.  It holds none of the
decoding or multiply arithmetic: it never turns a code back into a weight.

Canonical byte layouts (little-endian, fp16 = IEEE binary16 bit patterns):

* Q4_0  -- per row, K/32 blocks of 18 bytes: fp16 scale ``d`` then 16 code bytes
  (the ggml "oldest 4-bit format": 32 weights per block with one fp16 scale,
  4.5 bits per weight; blog.localai.hex7.com, "The ladder, with corrected
  numbers" table and "Anatomy of a block").
* CB4   -- 16 fp16 centroids (32 bytes), then codes [N][K/2], two 4-bit indices
  per byte (trapetum benchmarks page, "Kernel microbenchmarks", 4-bit K = 16).
* CB8   -- 256 fp16 centroids (512 bytes), then codes [N][K], one index per byte
  (trapetum benchmarks page, 8-bit LM head).
* TQ2   -- per row, K/128 blocks of 34 bytes: fp16 scale then 32 bytes holding
  four 2-bit codes each (the ternary PQ2_0 block; "Anatomy of a PQ2_0 block").
* AQ2x8 -- codebooks C[2][256][8] fp16 (8192 bytes), per-row scales s[N] fp16,
  then codes [N][K/8][2] uint8, codebook 0 first (trapetum benchmarks page,
  "Additive vector-quantization GEMV (AQLM-style, 2-bit)").
* AQ1x16 -- one codebook C[65536][8] fp16 (1 MiB), per-row scales s[N] fp16, then
  codes [N][K/8] uint16 (trapetum benchmarks page, the November update's 70B
  PV-tuned model in AQLM's 1x16 layout).

Seeds: every tensor is drawn from ``PCG64(SeedSequence([0, *key]))`` where the
key names the config, layer, projection and tensor, so any piece can be
regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

Q4_0, CB4, CB8, TQ2, AQ2X8, AQ1X16 = 1, 2, 3, 4, 5, 6
FORMAT_NAMES = {Q4_0: "q4_0", CB4: "cb4", CB8: "cb8", TQ2: "tq2", AQ2X8: "aq2x8", AQ1X16: "aq1x16"}
# K must be a multiple of this (whole blocks / whole groups / whole bytes).
K_MULTIPLE = {Q4_0: 32, CB4: 2, CB8: 1, TQ2: 128, AQ2X8: 8, AQ1X16: 8}


def rng(*key: int) -> np.random.Generator:
    """Counter-free seeded generator for one tensor, base seed 0."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, *[int(k) for k in key]])))


def f16_bits(values: np.ndarray) -> np.ndarray:
    """Round float64 values to fp16 (round-to-nearest-even) and return the uint16 bit patterns."""
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def canonical_bytes(fmt: int, N: int, K: int) -> int:
    if fmt == Q4_0:
        return N * (K // 32) * 18
    if fmt == CB4:
        return 32 + N * (K // 2)
    if fmt == CB8:
        return 512 + N * K
    if fmt == TQ2:
        return N * (K // 128) * 34
    if fmt == AQ2X8:
        return 8192 + 2 * N + N * (K // 8) * 2
    if fmt == AQ1X16:
        return 65536 * 8 * 2 + 2 * N + N * (K // 8) * 2
    raise ValueError(f"unknown format {fmt}")


def _check(fmt: int, N: int, K: int) -> None:
    if N < 1 or K < 1 or K % K_MULTIPLE[fmt]:
        raise ValueError(f"bad shape for {FORMAT_NAMES[fmt]}: N={N} K={K}")


def gen_weight(fmt: int, N: int, K: int, key: Sequence[int], *, cb_sigma: float = 0.02,
               scale_sigma: float | None = None, tq2_code3: float = 0.0) -> np.ndarray:
    """Canonical bytes (uint8 array) of one random packed weight matrix.

    Distributions follow the workloads: Q4_0 codes uniform over 16 values and
    d = fp16(|N(0,1)|*0.01); CB4/CB8 centroids sorted fp16(N(0, cb_sigma)) with
    uniform codes; TQ2 codes 0/1/2 with probabilities .25/.5/.25 (code 3 never
    drawn, unless tq2_code3 > 0: then code 3 takes that share of the code-2 draws) and
    d = fp16(|N(0,1)|*0.02); AQ2x8 codebooks fp16(N(0,0.01)),
    uniform 8-bit codes and row scales fp16(U(0.5,1.5)); AQ1x16 one codebook
    fp16(N(0,0.014)) (about the spread of a sum of two AQ2x8 entries), uniform
    16-bit codes and row scales fp16(U(0.5,1.5)).
    """
    _check(fmt, N, K)
    key = tuple(int(k) for k in key)
    if fmt == Q4_0:
        sig = 0.01 if scale_sigma is None else scale_sigma
        nb = K // 32
        d = f16_bits(np.abs(rng(*key, 0).standard_normal((N, nb))) * sig)
        qs = rng(*key, 1).integers(0, 256, size=(N, nb, 16), dtype=np.uint8)
        blk = np.empty((N, nb, 18), dtype=np.uint8)
        blk[:, :, 0:2] = d.astype("<u2").view(np.uint8).reshape(N, nb, 2)
        blk[:, :, 2:] = qs
        return blk.reshape(-1)
    if fmt in (CB4, CB8):
        ncb = 16 if fmt == CB4 else 256
        cb = np.sort(rng(*key, 0).standard_normal(ncb) * cb_sigma).astype(np.float16)
        cb = np.sort(cb)  # sorted after rounding as well
        nbytes = N * (K // 2) if fmt == CB4 else N * K
        codes = rng(*key, 1).integers(0, 256, size=nbytes, dtype=np.uint8)
        return np.concatenate([cb.view(np.uint16).astype("<u2").view(np.uint8), codes])
    if fmt == TQ2:
        sig = 0.02 if scale_sigma is None else scale_sigma
        nb = K // 128
        d = f16_bits(np.abs(rng(*key, 0).standard_normal((N, nb))) * sig)
        if tq2_code3 > 0:
            crumbs = rng(*key, 1).choice(np.array([0, 1, 2, 3], dtype=np.uint8), size=(N, nb, 32, 4),
                                         p=[0.25, 0.5, 0.25 - tq2_code3, tq2_code3])
        else:
            crumbs = rng(*key, 1).choice(np.array([0, 1, 2], dtype=np.uint8), size=(N, nb, 32, 4),
                                         p=[0.25, 0.5, 0.25])
        qs = (crumbs[..., 0] | (crumbs[..., 1] << 2) | (crumbs[..., 2] << 4) | (crumbs[..., 3] << 6)).astype(np.uint8)
        blk = np.empty((N, nb, 34), dtype=np.uint8)
        blk[:, :, 0:2] = d.astype("<u2").view(np.uint8).reshape(N, nb, 2)
        blk[:, :, 2:] = qs
        return blk.reshape(-1)
    if fmt == AQ2X8:
        C = f16_bits(rng(*key, 0).standard_normal((2, 256, 8)) * 0.01)
        s = f16_bits(rng(*key, 2).uniform(0.5, 1.5, size=N))
        codes = rng(*key, 1).integers(0, 256, size=N * (K // 8) * 2, dtype=np.uint8)
        return np.concatenate([C.astype("<u2").view(np.uint8).reshape(-1),
                               s.astype("<u2").view(np.uint8).reshape(-1), codes])
    if fmt == AQ1X16:
        C = f16_bits(rng(*key, 0).standard_normal((65536, 8)) * 0.014)
        s = f16_bits(rng(*key, 2).uniform(0.5, 1.5, size=N))
        codes = rng(*key, 1).integers(0, 65536, size=N * (K // 8), dtype=np.uint16)
        return np.concatenate([C.astype("<u2").view(np.uint8).reshape(-1),
                               s.astype("<u2").view(np.uint8).reshape(-1),
                               codes.astype("<u2").view(np.uint8)])
    raise ValueError(fmt)


def gen_x(M: int, K: int, key: Sequence[int]) -> np.ndarray:
    """Activations: fp16(N(0,1)) of shape (M, K), returned as uint16 bit patterns."""
    return f16_bits(rng(*[int(k) for k in key], 7).standard_normal((M, K)))


# --------------------------------------------------------------------------------------------
# Workload configurations (one entry per projection).
# --------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Proj:
    name: str
    fmt: int
    N: int
    K: int
    wkey: Tuple[int, ...]  # seed key of the weight
    xkey: Tuple[int, ...]  # seed key of the activation row(s); projections sharing it share x


LLAMA7B_LAYER = (  # (name, N, K, x role) ; roles: 0 = layer input, 1 = attention output, 2 = MLP hidden
    ("q", 4096, 4096, 0), ("k", 4096, 4096, 0), ("v", 4096, 4096, 0), ("o", 4096, 4096, 1),
    ("gate", 11008, 4096, 0), ("up", 11008, 4096, 0), ("down", 4096, 11008, 2),
)

CONFIG_NAMES = {
    1: "q4_0_gemv_4096x4096",
    2: "cb4_llama7b_layer",
    3: "cb4_llama7b_stack_cb8_head",
    4: "tq2_mlp_17408x5120",
    5: "aq2x8_llama70b_mlp",
    6: "aq1x16_llama70b_mlp",
}


def config_projections(cfg: int, layers: int | None = None) -> List[Proj]:
    """The projections of one workload config, in execution order."""
    out: List[Proj] = []
    if cfg == 1:
        out.append(Proj("q4_0", Q4_0, 4096, 4096, (1, 0, 0), (1, 0, 0)))
    elif cfg in (2, 3):
        nl = 1 if cfg == 2 else (32 if layers is None else layers)
        for layer in range(nl):
            for pi, (name, N, K, role) in enumerate(LLAMA7B_LAYER):
                out.append(Proj(f"L{layer}.{name}", CB4, N, K, (cfg, layer, pi), (cfg, layer, 100 + role)))
        if cfg == 3:
            out.append(Proj("lm_head", CB8, 32000, 4096, (cfg, 999, 0), (cfg, 999, 100)))
    elif cfg == 4:
        out.append(Proj("gate", TQ2, 17408, 5120, (4, 0, 0), (4, 0, 100)))
        out.append(Proj("up", TQ2, 17408, 5120, (4, 0, 1), (4, 0, 100)))
        out.append(Proj("down", TQ2, 5120, 17408, (4, 0, 2), (4, 0, 102)))
    elif cfg == 5:
        out.append(Proj("gate", AQ2X8, 28672, 8192, (5, 0, 0), (5, 0, 100)))
        out.append(Proj("up", AQ2X8, 28672, 8192, (5, 0, 1), (5, 0, 100)))
        out.append(Proj("down", AQ2X8, 8192, 28672, (5, 0, 2), (5, 0, 102)))
    elif cfg == 6:
        # the 70B MLP in AQLM's 1x16 layout (the PV-tuned 70B of the trapetum November update)
        out.append(Proj("gate", AQ1X16, 28672, 8192, (6, 0, 0), (6, 0, 100)))
        out.append(Proj("up", AQ1X16, 28672, 8192, (6, 0, 1), (6, 0, 100)))
        out.append(Proj("down", AQ1X16, 8192, 28672, (6, 0, 2), (6, 0, 102)))
    else:
        raise ValueError(cfg)
    return out


def gen_proj_weight(p: Proj) -> np.ndarray:
    return gen_weight(p.fmt, p.N, p.K, p.wkey)


def gen_proj_x(p: Proj, M: int) -> np.ndarray:
    return gen_x(M, p.K, p.xkey)
