"""Helpers shared by the GPU parity tests."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.paged_attention as orc
from oracle import run as orun


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from paged_kv_cache_87_amd import binding
    binding.load_library()          # raises if libpa.so is missing: no silent fallback


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def assert_pools_equal(gpu_step, k_ref, v_ref):
    kg, vg = gpu_step.pools_stored()
    assert kg.shape == k_ref.shape
    assert kg.tobytes() == k_ref.tobytes(), "K pool differs from the oracle's"
    assert vg.tobytes() == v_ref.tobytes(), "V pool differs from the oracle's"


# (case, dtype, max abs error, tolerance) of every comparison with the oracle
# in this session, printed at the end of the run by tests/conftest.py
ERRORS = []


def assert_close(gpu_f64, ref_f64, dtype, what=""):
    tol = orc.tolerance(dtype)
    assert np.all(np.isfinite(gpu_f64)), f"{what}: non-finite output"
    err = orc.max_abs_err(gpu_f64, ref_f64)
    ERRORS.append((what, dtype, err, tol))
    print(f"[gpu-case] {what}: max abs error {err:.3e} (tolerance {tol:.0e})", flush=True)
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.0e}"
    return err


def oracle_step(w):
    return orun.run_step(w)
