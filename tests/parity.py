"""Shared helpers for the GPU parity tests (not collected by pytest).

Tolerances (written here once, used by every GPU test):
  O   : max|O - O_ref| <= 2e-2 * max|O_ref| for fp16/bf16 io, <= 1e-4 absolute for fp32 io
  LSE : max|LSE - LSE_ref| <= 5e-3 (natural log units), -inf exactly where the oracle has -inf
  dQ, dK, dV : max|G - G_ref| <= 5e-2 * max|G_ref| per tensor, with an absolute
               floor of 1e-5 for references that are identically zero (one visible
               key: dS = dP - D vanishes exactly, the GPU leaves ~1e-7 of rounding)
FP8 forward (e4m3 Q, K, V; P rounded to e4m3 before P.V; O in bf16/fp16):
  every P value is within a relative 2^-4 of its exact value (round to
  nearest with 3 mantissa bits; the largest P of a row lies in [2^4, 2^8], so
  values down to 2^-10 of it are in the normal range; smaller ones round with
  an absolute step of 2^-10 of the row max), and l sums those rounded values, so
  LSE : |LSE - LSE_ref| <= -ln(1 - 2^-4) < 0.065, -inf exactly where the oracle has -inf
  O   : a weighted mean with each weight off by at most that factor; no sharp
        elementwise bound exists, so the test takes max|O - O_ref| <= 2^-3 max|O_ref|
        and rms(O - O_ref) <= 2^-5 rms(O_ref) (a wrong index or operand gives errors
        of the order of O itself); rows whose P is exact (one visible key, or V
        constant over the keys) are checked to the output rounding in their own tests
  amax: |amax - amax_ref| <= 2^-3 amax_ref
The reference is always the fp64 oracle run on the very same input bytes.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

O_REL_TOL = {"bf16": 2e-2, "fp16": 2e-2}
O_ABS_TOL_FP32 = 1e-4
LSE_ABS_TOL = 5e-3
GRAD_REL_TOL = 5e-2
GRAD_ABS_FLOOR = 1e-5
FP8_LSE_ABS_TOL = 0.065
FP8_O_MAX_REL = 2.0 ** -3
FP8_O_RMS_REL = 2.0 ** -5

DT_NAME = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}


def announce(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (bypasses capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).contiguous().numpy()


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = "O") -> float:
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite values"
    err = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    if dtype == "fp32":
        tol = O_ABS_TOL_FP32
    else:
        tol = O_REL_TOL[dtype] * float(np.max(np.abs(o_ref))) if o_ref.size else 0.0
    assert err <= tol, f"{what}: max|diff| {err:.3e} > tol {tol:.3e} ({dtype})"
    return err


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray, what: str = "LSE") -> float:
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), dead), f"{what}: -inf pattern differs"
    live = ~dead
    if not live.any():
        return 0.0
    assert np.all(np.isfinite(lse_gpu[live])), f"{what}: non-finite live values"
    err = float(np.max(np.abs(lse_gpu[live] - lse_ref[live])))
    assert err <= LSE_ABS_TOL, f"{what}: max|diff| {err:.3e} > {LSE_ABS_TOL}"
    return err


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, what: str) -> float:
    assert np.all(np.isfinite(g_gpu)), f"{what}: non-finite values"
    ref_max = float(np.max(np.abs(g_ref))) if g_ref.size else 0.0
    err = float(np.max(np.abs(g_gpu - g_ref))) if g_ref.size else 0.0
    tol = max(GRAD_REL_TOL * ref_max, GRAD_ABS_FLOOR)
    assert err <= tol, f"{what}: max|diff| {err:.3e} > tol {tol:.3e}"
    return err


def check_o_fp8(o_gpu: np.ndarray, o_ref: np.ndarray, what: str = "O") -> float:
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite values"
    if not o_ref.size:
        return 0.0
    diff = o_gpu - o_ref
    err = float(np.max(np.abs(diff)))
    tol = FP8_O_MAX_REL * float(np.max(np.abs(o_ref)))
    assert err <= tol, f"{what}: max|diff| {err:.3e} > tol {tol:.3e} (fp8)"
    rms, rms_ref = float(np.sqrt(np.mean(diff ** 2))), float(np.sqrt(np.mean(o_ref ** 2)))
    assert rms <= FP8_O_RMS_REL * rms_ref, f"{what}: rms diff {rms:.3e} > {FP8_O_RMS_REL} x {rms_ref:.3e}"
    return err


def check_lse_fp8(lse_gpu: np.ndarray, lse_ref: np.ndarray, what: str = "LSE") -> float:
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), dead), f"{what}: -inf pattern differs"
    live = ~dead
    if not live.any():
        return 0.0
    err = float(np.max(np.abs(lse_gpu[live] - lse_ref[live])))
    assert err <= FP8_LSE_ABS_TOL, f"{what}: max|diff| {err:.3e} > {FP8_LSE_ABS_TOL} (fp8)"
    return err
