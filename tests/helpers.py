"""Shared helpers for the GPU parity tests."""

from __future__ import annotations

import os

import numpy as np
import torch

import gdn_inputs as gi


def ensure_built() -> None:
    """Build libgdn.so only when nothing is built yet."""
    from linear_attention_recurrence_net_amd import _binding, build
    if not os.path.exists(_binding.library_path()):
        build.build()


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda").contiguous()


def upload(case: gi.Case):
    """q, k, v, g, beta, state on the GPU in the case's storage types."""
    qdt = torch.bfloat16 if case.qkv_dtype == "bf16" else torch.float32
    return dict(
        q=dev(case.q, qdt),  # bf16 cast is exact: values are bf16-representable
        k=dev(case.k, qdt),
        v=dev(case.v, qdt),
        g=dev(case.g),
        beta=dev(case.beta),
        state=dev(case.state),
    )


def oracle_args(case: gi.Case):
    return [case.f64(n) for n in ("q", "k", "v", "g", "beta")]


def rel_err(gpu, ref, name: str = "") -> float:
    """max|gpu - ref| / max|ref| over one output tensor.

    When the environment variable GDN_PARITY_LOG names a file, every
    comparison is appended to it as one tab-separated line: the running
    test, the tensor's name (or its shape) and the error, so that a GPU run
    leaves a record of the headroom under each bar.
    """
    if isinstance(gpu, torch.Tensor):
        gpu = gpu.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    num = np.abs(np.asarray(gpu, dtype=np.float64) - ref).max()
    err = float(num) if den == 0 else float(num / den)
    log = os.environ.get("GDN_PARITY_LOG")
    if log:
        test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        label = name or "x".join(str(n) for n in ref.shape)
        with open(log, "a") as f:
            f.write(f"{test}\t{label}\t{err:.3e}\n")
    return err


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy().copy()
