"""Comparison helpers and oracle adapters for the GPU parity tests.

Tolerances:
  * the output of the path, o = z . W_UV:
      float32 inputs:             max |gpu - oracle| <= 1e-4 * RMS(oracle)
      bfloat16 inputs, fp32 acc:  max |gpu - oracle| <= 2e-2 * RMS(oracle)
  * intermediates (the weighted latent z, split partials): the same bf16 bound on the largest
    error, max |err| <= 2e-2 * RMS, and RMS(err) <= 5e-3 * RMS; float32: 1e-4 and 1e-5.  The bf16
    path scores in IEEE binary16 (binary16 absorbed query times the exactly converted cache
    values) and rounds the probabilities to binary16, 2^-11 relative each: a CPU simulation of
    those roundings over short, peaked and long rows gives max/RMS of at most ~4e-3 on o and z
    for every head of a row, against ~2.7e-2 when the query and the probabilities are rounded to
    bf16.
  * lse (a log quantity) is compared in absolute terms: 2e-2 (bf16), 1e-4 (float32)
  * split-K indexing and length masking: exact (integer counts, bitwise re-runs)
"""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle.mla_oracle as O
from mla_workloads import gen

TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_MID = {"f32": 1e-4, "bf16": 2e-2}
TOL_MID_RMS = {"f32": 1e-5, "bf16": 5e-3}


def note(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def assert_rms_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite pattern differs"
    if not fin.all():
        assert np.array_equal(got[~fin], ref[~fin]), f"{what}: non-finite values differ"
    if fin.any():
        rms = math.sqrt(float(np.mean(ref[fin] ** 2)))
        err = float(np.max(np.abs(got[fin] - ref[fin])))
        assert err <= tol * max(rms, 1e-30), f"{what}: max err {err:.3e} > {tol:.0e} * rms {rms:.3e}"
        return err / max(rms, 1e-30)
    return 0.0


def assert_mid_close(got, ref, dtype, what):
    """Intermediate outputs (z, split partials): max-abs and RMS-of-error bounds."""
    assert_rms_close(got, ref, TOL_MID[dtype], what)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    if fin.any():
        rms = math.sqrt(float(np.mean(ref[fin] ** 2)))
        rerr = math.sqrt(float(np.mean((got[fin] - ref[fin]) ** 2)))
        assert rerr <= TOL_MID_RMS[dtype] * max(rms, 1e-30), f"{what}: rms err {rerr:.3e} > {TOL_MID_RMS[dtype]:.0e} * rms {rms:.3e}"


def assert_abs_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite pattern differs"
    if not fin.all():
        assert np.array_equal(got[~fin], ref[~fin]), f"{what}: non-finite values differ"
    if fin.any():
        err = float(np.max(np.abs(got[fin] - ref[fin])))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.0e}"


class OracleView:
    """fp64 views of one workload's stored inputs, widened once, for oracle calls."""

    def __init__(self, inp: dict):
        self.inp = inp
        self.w = inp["workload"]
        dt = inp["dtype"]
        self.w_uk = gen.as_f64(inp["w_uk"], dt)
        self.w_uv = gen.as_f64(inp["w_uv"], dt)
        self.dt = dt

    def cache(self, b: int, length: int | None = None) -> np.ndarray:
        L = int(self.inp["lens"][b]) if length is None else length
        return gen.as_f64(O.gather_rows(self.inp["pool"], self.inp["page_table"], b, L), self.dt)

    def decode(self, b: int, heads=None, key_range=None) -> dict:
        L = int(self.inp["lens"][b])
        return O.attention(gen.as_f64(self.inp["q_c"][b], self.dt), gen.as_f64(self.inp["q_r"][b], self.dt),
                           L - 1, self.cache(b), self.w_uk, self.w_uv, self.w.d_c, base=self.w.rope_base,
                           heads=heads, key_range=key_range)

    def q_hat(self, b: int) -> np.ndarray:
        L = int(self.inp["lens"][b])
        return O.absorbed_query(gen.as_f64(self.inp["q_c"][b], self.dt), gen.as_f64(self.inp["q_r"][b], self.dt),
                                L - 1, self.w_uk, self.w.rope_base)

    def prefill_row(self, b: int, i: int, heads=None) -> dict:
        q0 = int(self.inp["q_start"][b])
        cache = self.cache(b, q0 + i + 1)
        return O.attention(gen.as_f64(self.inp["q_c"][b, i], self.dt), gen.as_f64(self.inp["q_r"][b, i], self.dt),
                           q0 + i, cache, self.w_uk, self.w_uv, self.w.d_c, base=self.w.rope_base, heads=heads)
