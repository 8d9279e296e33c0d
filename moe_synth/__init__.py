"""Seeded synthetic inputs for the MoE layer hot path.

This module is shared by the CPU oracle and the GPU path and therefore holds
none of the method's arithmetic: it only draws random numbers, encodes them in
the storage dtypes (fp32, bf16 bit patterns in uint16, int8) and builds the
per-expert logit offsets that skew routing.  Everything a method step computes
(gate, softmax, top-k, quantisation, grouping, FFN, combine) lives elsewhere.

Recipe (one NumPy PCG64 stream per tensor chunk, so large tensors are drawn in
parallel and every chunk is reproducible on its own):

* seed of a chunk = ``SeedSequence([seed_base + tensor_id, chunk])`` where
  ``seed_base = 1000 * cfg`` for the named workloads, tensor ids x=0, Wg=1,
  W13=2, W2=3, expert permutation=4, W13 scales=5, W2 scales=6;
* x ~ N(0, 1), row chunks of 1024 tokens;
* Wg, W13, W2 ~ N(0, 0.02), W13/W2 one chunk per expert;
* values are drawn in fp32, then rounded to nearest-even bf16 where bf16 is
  the storage type; bf16 tensors are returned as uint16 bit patterns;
* int8 expert weights (the W8A8 workload) are drawn directly as integers
  ``clip(rint(N(0, 1) * 32), -127, 127)`` with per-output-channel fp32 scales
  ``0.02 / 32 * (0.75 + 0.5 * U(0, 1))``, i.e. weights of std ~0.02 already in
  their quantised storage form;
* int4 expert weights (W4A16 and W4A8) are drawn the same way with
  ``clip(rint(N(0, 1) * 2.5), -8, 7)`` codes (stored one per int8, unpacked)
  and scales ``0.02 / 2.5 * (0.75 + 0.5 * U(0, 1))``;
* the skewed workload adds per-expert logit offsets ``-s * ln(rank_e)`` with
  ``rank_e = perm(e) + 1`` for a seeded permutation ``perm`` of the experts and
  s = 1.1, which gives the softmax a Zipf(s) prior over experts.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TENSOR_X, TENSOR_WG, TENSOR_W13, TENSOR_W2, TENSOR_PERM, TENSOR_S13, TENSOR_S2 = range(7)

INT8_WEIGHT_STD = 32.0
INT4_WEIGHT_STD = 2.5
X_ROW_CHUNK = 1024


@dataclass(frozen=True)
class Spec:
    """Shape and storage dtypes of one MoE layer workload."""

    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    x_dtype: str = "bf16"      # "f32" | "bf16"
    wg_dtype: str = "bf16"     # "f32" | "bf16"
    w_dtype: str = "bf16"      # "f32" | "bf16" | "i8" | "i4", "i4a8" (int4 codes in int8 storage)
    out_dtype: str = "bf16"    # "f32" | "bf16"
    capacity_factor: float = 0.0   # <= 0: no capacity limit
    zipf_s: float = 0.0            # > 0: per-expert Zipf(s) logit offsets
    w_std: float = 0.02
    x_std: float = 1.0

    def replace(self, **kw) -> "Spec":
        d = dict(self.__dict__)
        d.update(kw)
        return Spec(**d)


# The five workloads: tiny fp32, Mixtral-8x7B-shaped prefill, 256-expert top-8
# with capacity, decode, and skewed W8A8.
CONFIGS = {
    1: Spec("tiny_fp32_T64_H128_E8_k2_I256", 64, 128, 8, 2, 256,
            x_dtype="f32", wg_dtype="f32", w_dtype="f32", out_dtype="f32"),
    2: Spec("mixtral_prefill_T4096_H4096_E8_k2_I14336", 4096, 4096, 8, 2, 14336,
            x_dtype="bf16", wg_dtype="f32", w_dtype="bf16", out_dtype="bf16"),
    3: Spec("finegrained_T4096_H4096_E256_k8_I1024_cap1.25", 4096, 4096, 256, 8, 1024,
            capacity_factor=1.25),
    4: Spec("decode_T16_H4096_E256_k8_I1024", 16, 4096, 256, 8, 1024),
    5: Spec("skewed_w8a8_T16384_H2048_E64_k6_I1408_cap1.25", 16384, 2048, 64, 6, 1408,
            w_dtype="i8", capacity_factor=1.25, zipf_s=1.1),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode finite fp32 values as bf16 bit patterns, rounding to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _rng(seed_base: int, tensor_id: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed_base + tensor_id, chunk])))


def _normal_into(out: np.ndarray, dtype: str, rng: np.random.Generator, std: float) -> None:
    v = rng.standard_normal(out.shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if dtype == "bf16":
        out[...] = f32_to_bf16_bits(v)
    else:
        out[...] = v


def _int8_into(q_out: np.ndarray, s_out: np.ndarray, rng_q, rng_s, std: float, bits: int = 8) -> None:
    qstd, lo, hi = (INT8_WEIGHT_STD, -127, 127) if bits == 8 else (INT4_WEIGHT_STD, -8, 7)
    v = rng_q.standard_normal(q_out.shape, dtype=np.float32) * np.float32(qstd)
    q_out[...] = np.clip(np.rint(v), lo, hi).astype(np.int8)
    u = rng_s.random(s_out.shape, dtype=np.float32)
    s_out[...] = np.float32(std / qstd) * (np.float32(0.75) + np.float32(0.5) * u)


def _storage(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "i8": np.int8, "i4": np.int8, "i4a8": np.int8}[dtype]


@dataclass
class Inputs:
    """One workload's tensors, in their storage dtypes (bf16 = uint16 bits)."""

    spec: Spec
    seed_base: int
    x: np.ndarray                # [T, H]
    wg: np.ndarray               # [E, H]
    bias: np.ndarray | None      # [E] fp32 or None
    w13: np.ndarray              # [E, 2I, H]: rows 0..I-1 are W1, rows I..2I-1 are W3
    w2: np.ndarray               # [E, H, I]
    s13: np.ndarray | None = None    # [E, 2I] fp32 (int8 / int4 weights only)
    s2: np.ndarray | None = None     # [E, H] fp32 (int8 / int4 weights only)
    extra: dict = field(default_factory=dict)


def make_inputs(spec: Spec, seed_base: int, threads: int | None = None,
                with_experts: bool = True) -> Inputs:
    """Draw every tensor of ``spec``; deterministic in (spec, seed_base)."""
    T, H, E, k, I = spec.T, spec.H, spec.E, spec.k, spec.I
    nthr = threads or _threads()
    x = np.empty((T, H), dtype=_storage(spec.x_dtype))
    wg = np.empty((E, H), dtype=_storage(spec.wg_dtype))
    jobs = []
    for c in range(0, max(T, 1), X_ROW_CHUNK):
        if c >= T:
            break
        jobs.append((x[c:c + X_ROW_CHUNK], spec.x_dtype, TENSOR_X, c // X_ROW_CHUNK, spec.x_std))
    jobs.append((wg, spec.wg_dtype, TENSOR_WG, 0, spec.w_std))
    w13 = w2 = s13 = s2 = None
    if with_experts:
        w13 = np.empty((E, 2 * I, H), dtype=_storage(spec.w_dtype))
        w2 = np.empty((E, H, I), dtype=_storage(spec.w_dtype))
        if spec.w_dtype in ("i8", "i4", "i4a8"):
            s13 = np.empty((E, 2 * I), dtype=np.float32)
            s2 = np.empty((E, H), dtype=np.float32)

    def run_normal(job):
        out, dt, tid, chunk, std = job
        _normal_into(out, dt, _rng(seed_base, tid, chunk), std)

    def run_expert(e):
        if spec.w_dtype in ("i8", "i4", "i4a8"):
            b = 8 if spec.w_dtype == "i8" else 4
            _int8_into(w13[e], s13[e], _rng(seed_base, TENSOR_W13, e), _rng(seed_base, TENSOR_S13, e), spec.w_std, b)
            _int8_into(w2[e], s2[e], _rng(seed_base, TENSOR_W2, e), _rng(seed_base, TENSOR_S2, e), spec.w_std, b)
        else:
            _normal_into(w13[e], spec.w_dtype, _rng(seed_base, TENSOR_W13, e), spec.w_std)
            _normal_into(w2[e], spec.w_dtype, _rng(seed_base, TENSOR_W2, e), spec.w_std)

    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(run_normal, jobs))
        if with_experts:
            list(ex.map(run_expert, range(E)))

    bias = None
    if spec.zipf_s > 0:
        perm = _rng(seed_base, TENSOR_PERM, 0).permutation(E)
        bias = (-spec.zipf_s * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)
    return Inputs(spec, seed_base, x, wg, bias, w13, w2, s13, s2)


def config_inputs(cfg: int, threads: int | None = None, with_experts: bool = True) -> Inputs:
    """Inputs of named workload ``cfg`` (1..5) with its canonical seed base."""
    return make_inputs(CONFIGS[cfg], 1000 * cfg, threads, with_experts)


def bf16_bits_as_f32(u16: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns to fp32 (exact); used to build test inputs."""
    return (np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
