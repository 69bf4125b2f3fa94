"""Plain CPU oracle for the W4 verify projection and the greedy verify.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library never does, and shares no code, table or helper with it.

What it computes, step by step, is the plain definition of the operation:

1. ``decode_act``: activations to float64 (exact for bf16, fp16 and fp32).
2. ``unpack_codes`` and ``dequantize``: w[n,k] = s[n,g]*q[n,k] + b[n,g],
   g = k // 64, evaluated exactly in float64.
3. ``qgemm_ref``: y[m,n] = sum_k x[m,k]*w[n,k] in float64 (y = x @ W.T).
4. ``argmax_ref``: per row, the lowest index holding the maximum; -0 and +0
   are equal; any NaN wins and the first NaN is taken.
5. ``accept_walk_ref`` and ``verify_ref``: per sequence, the number of
   leading drafts equal to the target's argmax of the row before them,
   optionally capped by the sequence's count of valid drafts.
6. ``margin_ref``: per row, top-1 minus top-2 in fp32.
7. ``silu_ref``, ``swiglu_ref`` and ``qgemm_swiglu_ref``: the gated
   activation over a gate/up projection, h = silu(gate) * up in float64.

Sources on the pages:

* The projection is a quantized matmul over the M rows of a verify block,
  with 4-bit weights and BF16, FP16 or FP32 activations ("perf: tune DFlash2
  M=8 verification for M1 and M2", PR description: the scalar K-major and
  FP16-matrix QMM kernels, the W4A32 draft and vocabulary projection).
* Row 0 of a verify block is the committed token and the following rows are
  the drafts ("dspark: fold first-token forward into verify + bit-exact M5
  Metal decode wins", first commit and the PR body's fold section).
* Each row commits its own accepted count from the walk ("perf(speculative):
  commit per-row accepts in batched DFlash", commit message).

Where the pages are silent the readings are: little-endian nibbles (even k
in the low nibble), W stored as [N, K] with K contiguous ("K-major"), an
affine w = s*q + b with fp16 scale and bias per group of 64 contiguous k
(32 and 128 taken as the other group sizes, with the same layout),
NaN-first argmax with a lowest-index tie break, and accept_len counting the
accepted drafts only (0..T-1). Every function here is pinned by tests that do
not reuse its code (brute force, closed forms, library argmax, hand walks).
"""

from __future__ import annotations

import numpy as np

GROUP = 64


def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE fp16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_act(x: np.ndarray, act: str) -> np.ndarray:
    """Activations -> float64. bf16 is the upper half of an fp32 word."""
    if act == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    if act == "fp16":
        return decode_f16(x)
    if act == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown activation dtype {act!r}")


def unpack_codes(wq: np.ndarray) -> np.ndarray:
    """[N, K/2] packed bytes -> [N, K] codes in 0..15 (even k = low nibble)."""
    wq = np.asarray(wq, dtype=np.uint8)
    N, half = wq.shape
    q = np.empty((N, 2 * half), dtype=np.uint8)
    q[:, 0::2] = wq & 0x0F
    q[:, 1::2] = wq >> 4
    return q


def dequantize(wq: np.ndarray, scales: np.ndarray, biases: np.ndarray,
               group: int = GROUP) -> np.ndarray:
    """[N, K] float64 weights w[n,k] = s[n, k//group] * q[n,k] + b[n, k//group]."""
    q = unpack_codes(wq).astype(np.float64)
    K = q.shape[1]
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    if scales.shape[-1] != K // group or biases.shape[-1] != K // group:
        raise ValueError("scales and biases must hold K/group entries per row")
    g = np.arange(K) // group
    s = decode_f16(scales)
    b = decode_f16(biases)
    return s[:, g] * q + b[:, g]


def qgemm_ref(x: np.ndarray, act: str, wq: np.ndarray, scales: np.ndarray,
              biases: np.ndarray, group: int = GROUP, cols=None,
              chunk: int = 2048) -> np.ndarray:
    """y = x @ W.T in float64, with W dequantized exactly.

    ``cols`` restricts the output to the given column indices (for sampled
    checks of very large N). Columns are processed ``chunk`` at a time so that
    the float64 weight slab stays small; chunking does not change the result
    beyond float64 rounding.
    """
    xd = decode_act(x, act)
    N = wq.shape[0]
    idx = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    y = np.empty((xd.shape[0], idx.size), dtype=np.float64)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        w = dequantize(wq[sel], scales[sel], biases[sel], group)
        y[:, c0:c0 + sel.size] = xd @ w.T
    return y


def argmax_ref(v: np.ndarray) -> int:
    """Lowest index of the maximum of one row.

    IEEE comparison, so -0.0 == +0.0 tie. If the row holds a NaN, the index of
    the first NaN. An all -inf row gives 0.
    """
    v = np.asarray(v)
    nan = np.isnan(v)
    if nan.any():
        return int(np.flatnonzero(nan)[0])
    top = v.max()
    return int(np.flatnonzero(v == top)[0])


def margin_ref(v: np.ndarray) -> np.float32:
    """Top-1 minus top-2 of one fp32 row, in fp32.

    The margin the verifier's gate compares with a bar ("dspark: fold
    first-token forward into verify + bit-exact M5 Metal decode wins", first
    commit: the target's top-1 minus top-2 logit margin gate). Top-2 is the
    largest value at any index other than the argmax, so a tied maximum gives
    0 (-0 and +0 tie; so do two +inf or two -inf). A row holding a NaN gives
    NaN; a row of one value gives +inf (no competitor). Otherwise the
    difference is rounded to fp32, as the GPU computes it.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        return np.float32(np.nan)
    if v.size == 1:
        return np.float32(np.inf)
    i = argmax_ref(v)
    top = v[i]
    second = np.delete(v, i).max()
    if second == top:
        return np.float32(0.0)
    return np.float32(top) - np.float32(second)


def accept_walk_ref(row_argmax: np.ndarray, draft: np.ndarray, T: int,
                    draft_len: int | None = None) -> int:
    """Accepted drafts of one sequence: leading i < T-1 with
    argmax[i] == draft[i]. Row i's prediction checks the token fed at row i+1.

    With draft_len, only drafts i < draft_len are walked; it is clamped to
    0..T-1. A sequence's block may hold fewer valid drafts than T-1: the
    batched loop's rows have different live lengths ("perf(speculative):
    commit per-row accepts in batched DFlash", commit message), and a block
    can end in a partial tail ("perf: tune DFlash2 M=8 verification for M1
    and M2", Validation).
    """
    limit = T - 1 if draft_len is None else min(max(int(draft_len), 0), T - 1)
    L = 0
    while L < limit and int(row_argmax[L]) == int(draft[L]):
        L += 1
    return L


def verify_ref(logits: np.ndarray, draft, B: int, T: int, draft_len=None, margin=False):
    """logits [B*T, N] -> (argmax [B*T] int32, accept_len [B] int32), and the
    margins [B*T] fp32 when margin=True. draft_len [B] limits each walk."""
    logits = np.asarray(logits)
    if logits.shape[0] != B * T:
        raise ValueError("logits must have B*T rows")
    a = np.array([argmax_ref(logits[r]) for r in range(B * T)], dtype=np.int32)
    if T > 1:
        d = np.asarray(draft).reshape(B, T - 1)
    else:
        d = np.zeros((B, 0), dtype=np.int32)
    lens = [None] * B if draft_len is None else [int(v) for v in np.asarray(draft_len)]
    acc = np.array([accept_walk_ref(a[b * T:(b + 1) * T], d[b], T, lens[b]) for b in range(B)],
                   dtype=np.int32)
    if margin:
        m = np.array([margin_ref(logits[r]) for r in range(B * T)], dtype=np.float32)
        return a, acc, m
    return a, acc


def silu_ref(g):
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), elementwise in float64.

    For g below about -709 exp(-g) overflows to inf and the quotient is -0,
    the float64 limit of the exact value.
    """
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ref(y):
    """Gated activation of a fused gate/up projection output.

    ``y`` is [M, 2*Nh]: columns 0..Nh-1 are the gate, columns Nh..2*Nh-1 the
    up projection, one matmul over the two weight blocks stacked along N (the
    M=16 gate/up block of "perf: tune DFlash2 M=8 verification for M1 and
    M2", Validation; the pages name no activation, and silu-gating is the
    plainest reading for the Qwen 3.5 targets of "perf(speculative): commit
    per-row accepts in batched DFlash"). Returns h [M, Nh] = silu(gate) * up
    in float64.
    """
    y = np.asarray(y, dtype=np.float64)
    if y.shape[-1] % 2:
        raise ValueError("a gate/up output has an even number of columns")
    nh = y.shape[-1] // 2
    return silu_ref(y[..., :nh]) * y[..., nh:]


def qgemm_swiglu_ref(x: np.ndarray, act: str, wq: np.ndarray, scales: np.ndarray,
                     biases: np.ndarray, group: int = GROUP, cols=None) -> np.ndarray:
    """h = silu(x @ Wg.T) * (x @ Wu.T) in float64, with W = [Wg; Wu] stacked
    along N (rows 0..Nh-1 gate, Nh..2*Nh-1 up). ``cols`` restricts h to the
    given columns j, each computed from weight rows j and Nh + j."""
    N = wq.shape[0]
    if N % 2:
        raise ValueError("a gate/up weight has an even number of rows")
    nh = N // 2
    idx = np.arange(nh) if cols is None else np.asarray(cols, dtype=np.int64)
    gate = qgemm_ref(x, act, wq, scales, biases, group, cols=idx)
    up = qgemm_ref(x, act, wq, scales, biases, group, cols=nh + idx)
    return swiglu_ref(np.concatenate([gate, up], axis=1))
