"""Helpers shared by the GPU tests: move generated numpy inputs to the device
as the dtypes the binding expects, and compare against the oracle."""

from __future__ import annotations

import hashlib

import numpy as np
import torch

TOL = {"bf16": 1e-3, "fp16": 1e-3, "fp32": 1e-4}


def to_device(c: dict, device: str = "cuda") -> dict:
    """x, wq, scales, biases of a generated config as device tensors."""
    act = c["act"]
    if act == "bf16":
        x = torch.from_numpy(c["x"].view(np.int16)).view(torch.bfloat16)
    elif act == "fp16":
        x = torch.from_numpy(c["x"].view(np.int16)).view(torch.float16)
    else:
        x = torch.from_numpy(c["x"])
    return dict(
        x=x.to(device),
        wq=torch.from_numpy(c["wq"]).to(device),
        scales=torch.from_numpy(c["scales"].view(np.int16)).view(torch.float16).to(device),
        biases=torch.from_numpy(c["biases"].view(np.int16)).view(torch.float16).to(device),
    )


def assert_close(y_gpu: np.ndarray, y_ref: np.ndarray, act: str, what: str = "") -> float:
    """|y_gpu - y_ref| <= tol * (1 + |y_ref|) elementwise; returns the worst
    ratio of error to allowance."""
    tol = TOL[act]
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    allow = tol * (1.0 + np.abs(y_ref))
    ratio = err / allow
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    bad = ~(err <= allow)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside {tol}*(1+|y|); first "
            + ", ".join(f"{tuple(i)} gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r}" for i in idx))
    return worst


def sha(t: torch.Tensor) -> str:
    return hashlib.sha256(t.detach().cpu().contiguous().numpy().tobytes()).hexdigest()


def top2_gap(row: np.ndarray) -> float:
    """Top-1 minus top-2 of a float64 row (inf if the row has one element)."""
    if row.size < 2:
        return np.inf
    part = np.partition(row, -2)
    return float(part[-1] - part[-2])
