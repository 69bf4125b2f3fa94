"""Seeded synthetic inputs for the W4 verify projection and the greedy verify.

This module only draws random inputs. It holds none of the method's
arithmetic: no dequantisation, no matmul, no argmax, no accept walk. Both the
CPU oracle (``oracle/``) and the HIP path (``w4_gemm_vqv_amd``) consume what it
returns; neither shares any other code with the other.

Shapes and distributions follow the workloads the pages measure:

* K=5120, N=17408 and K=5120, N=1024 projections at M=8 versus M=4
  ("perf: tune DFlash2 M=8 verification for M1 and M2", Performance).
* An eight-token verify block ("perf: tune DFlash2 ...", What/Why) and a
  batched run of B=4 sequences with block 16 ("perf(speculative): commit
  per-row accepts in batched DFlash", commit message).
* W4A32 draft/vocabulary projections with seven zero-padded rows
  ("perf: tune DFlash2 ...", PR description).
* An M=16 gate/up projection ("perf: tune DFlash2 ...", Validation).

The trained models and prompts behind those measurements are not available;
these tensors stand in for them with the same shapes.

Array conventions (all numpy, C-contiguous):

* ``wq``      uint8  [N, K/2]  packed 4-bit codes; byte j of row n holds
                               k=2j in bits 0-3 and k=2j+1 in bits 4-7.
* ``scales``  uint16 [N, K/group] IEEE fp16 bit patterns (group 64 unless
                               asked for 128).
* ``biases``  uint16 [N, K/group] IEEE fp16 bit patterns.
* ``x``       uint16 [M, K] bf16 or fp16 bit patterns, or float32 [M, K].
* ``draft``   int32  [B, T-1].
"""

from __future__ import annotations

import numpy as np

GROUP = 64

# name -> shape/dtype/seed recipe. "real_rows" < M means rows >= real_rows are
# zero padding (the W4A32 draft projection pads one real row to eight).
CONFIGS = {
    "tiny": dict(M=8, K=512, N=1024, act="bf16", sigma=1.0, seed=1, B=1, T=8,
                 drafts="force_first_3"),
    "target": dict(M=8, K=5120, N=17408, act="bf16", sigma=1.0, seed=2, B=1, T=8,
                   drafts="uniform_accept"),
    "draft_w4a32": dict(M=8, K=5120, N=1024, act="fp32", sigma=1.0, seed=3,
                        real_rows=1),
    "vocab_verify": dict(M=8, K=2560, N=151936, act="fp16", sigma=0.5, seed=4, B=1,
                         T=8, drafts="uniform_accept"),
    "batched_vocab": dict(M=64, K=2560, N=151936, act="bf16", sigma=1.0, seed=5, B=4,
                          T=16, drafts="uniform_accept"),
    "gate_up": dict(M=16, K=2560, N=18432, act="bf16", sigma=1.0, seed=6),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def make_weights(rng: np.random.Generator, N: int, K: int, group: int = GROUP):
    """Packed codes uniform in 0..15, fp16 scales ~U(0.005, 0.02) and fp16
    biases = -8*scale + N(0, 0.001), rounded to fp16 after the sum.

    Draw order: codes, scales, bias noise. Two independent uniform nibbles
    make one uniform byte, so the codes are drawn as bytes.
    """
    if K % 2 or K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s16 = rng.uniform(0.005, 0.02, size=(N, G)).astype(np.float16)
    noise = rng.normal(0.0, 0.001, size=(N, G))
    b16 = (-8.0 * s16.astype(np.float64) + noise).astype(np.float16)
    return wq, s16.view(np.uint16).copy(), b16.view(np.uint16).copy()


def make_x(rng: np.random.Generator, M: int, K: int, act: str, sigma: float = 1.0,
           real_rows: int | None = None) -> np.ndarray:
    """Activations ~N(0, sigma) (sigma is the standard deviation), cast to
    the activation dtype. Rows >= real_rows are exact zeros."""
    v = rng.standard_normal(size=(M, K), dtype=np.float32) * np.float32(sigma)
    if real_rows is not None:
        v[real_rows:] = 0.0
    if act == "bf16":
        return f32_to_bf16_bits(v)
    if act == "fp16":
        return v.astype(np.float16).view(np.uint16).copy()
    if act == "fp32":
        return v
    raise ValueError(f"unknown activation dtype {act!r}")


def make_config(name: str, seed: int | None = None, **overrides) -> dict:
    """Inputs of one named workload. ``overrides`` may change M, K, N, the
    seed (for scaled-down parity cases that keep the recipe) or the group
    size (64 or 128 k per scale and bias)."""
    spec = dict(CONFIGS[name])
    spec.update(overrides)
    if seed is not None:
        spec["seed"] = seed
    rng = np.random.default_rng(spec["seed"])
    M, K, N = spec["M"], spec["K"], spec["N"]
    group = spec.get("group", GROUP)
    wq, scales, biases = make_weights(rng, N, K, group)
    x = make_x(rng, M, K, spec["act"], spec.get("sigma", 1.0), spec.get("real_rows"))
    out = dict(spec, name=name, group=group, wq=wq, scales=scales, biases=biases, x=x)
    return out


def accept_lengths(seed: int, B: int, T: int) -> np.ndarray:
    """Target accept lengths, independent and uniform in 0..T-1."""
    rng = np.random.default_rng((seed, 7))
    return rng.integers(0, T, size=B).astype(np.int32)


def make_drafts(argmax_rows: np.ndarray, B: int, T: int, N: int, seed: int,
                accept: np.ndarray | None = None, force_first: int | None = None
                ) -> np.ndarray:
    """Draft tokens [B, T-1] built around a given per-row argmax [B*T].

    * ``force_first=f``: all drafts uniform in [0, N), then the first f of
      each sequence are overwritten with that row's argmax.
    * ``accept=L[b]``: draft[b, i] = argmax[b*T+i] for i < L[b]; if L[b] < T-1
      then draft[b, L] = (argmax[b*T+L] + 1 + u) mod N with u uniform in
      0..N-2 (so it always misses); later drafts are uniform in [0, N).

    The argmax is an input here; this function never computes one.
    """
    rng = np.random.default_rng((seed, 11))
    a = np.asarray(argmax_rows, dtype=np.int64).reshape(B, T)
    d = rng.integers(0, N, size=(B, max(T - 1, 0))).astype(np.int64)
    if force_first is not None:
        f = min(force_first, T - 1)
        d[:, :f] = a[:, :f]
    if accept is not None:
        for b in range(B):
            L = int(accept[b])
            d[b, :L] = a[b, :L]
            if L < T - 1:
                if N > 1:
                    u = int(rng.integers(0, N - 1))
                    d[b, L] = (a[b, L] + 1 + u) % N
                else:
                    d[b, L] = N  # out of range: never equal to an index in [0, N)
    return d.astype(np.int32)
