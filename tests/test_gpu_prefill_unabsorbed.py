"""GPU parity of the unabsorbed chunked prefill (mla_decompress_kv + mla_prefill_unabsorbed)
against the fp64 oracle, which evaluates the plain definition (decompressed keys and values,
[molayo] formal definition; [ase] Fig. 2) and so is the natural reference for this path.

Tolerances are those of the bf16 inputs' final output o (max |err| <= 2e-2 * RMS over every head
of a row) and of lse (2e-2 absolute).  The path multiplies the bf16 cache and weights exactly and
rounds the decompressed keys and values, the rotated query part and the softmax probabilities to
binary16 once each (2^-11 relative), all with fp32 accumulation.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_31_amd as M
from mla_latent_kv_31_amd import runner
from mla_workloads import gen
from parity import TOL, OracleView, assert_abs_close, assert_rms_close, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def test_unabsorbed_small_ragged_starts_all_rows():
    """Three sequences with different chunk starts (q_start 0 puts the first row on a single key),
    every row on every head, o and lse against the oracle; a fourth sequence starts at -3, so its
    first three rows see no key (o = 0, lse = -inf)."""
    w = gen.Workload(name="prefill_small_u", seed=9, kind="prefill", batch=4, ctx=70, q_len=40, random_pages=True)
    inp = gen.make_prefill_inputs(w)
    inp["q_start"] = np.array([70, 0, 33, -3], np.int32)
    note("unabsorbed prefill small ragged starts")
    st = runner.PrefillUnabsorbedStep(inp, DEV)
    assert st.supported()
    st.run()
    torch.cuda.synchronize()
    view = OracleView(inp)
    heads = list(range(128))
    tol = TOL["bf16"]
    out, lse = _np(st.out), _np(st.lse)
    for b in range(4):
        for i in range(40):
            if int(inp["q_start"][b]) + i < 0:
                assert np.all(out[b, i] == 0.0) and np.all(np.isneginf(lse[b, i])), f"row ({b},{i}) sees no key"
                continue
            ref = view.prefill_row(b, i, heads)
            assert_abs_close(lse[b, i, heads], ref["lse"][heads], tol, f"lse ({b},{i})")
            assert_rms_close(out[b, i, heads], ref["o"][heads], tol, f"o ({b},{i})")


@pytest.fixture(scope="module")
def inp_prefill():
    return gen.make_prefill_inputs(gen.WORKLOADS["v3_prefill_b2"])


def test_unabsorbed_v3_prefill_sampled(inp_prefill):
    """The benchmark chunk (2 x 512 queries over 2,560 keys): sampled rows against the oracle, and
    every output against the absorbed path (same inputs; both are the same attention up to
    rounding)."""
    note("unabsorbed prefill v3_prefill_b2")
    st = runner.PrefillUnabsorbedStep(inp_prefill, DEV)
    st.run()
    ab = runner.PrefillStep(inp_prefill, DEV)
    ab.run()
    torch.cuda.synchronize()
    view = OracleView(inp_prefill)
    tol = TOL["bf16"]
    heads = list(range(128))
    out, lse = _np(st.out), _np(st.lse)
    for b in (0, 1):
        for i in (0, 1, 63, 64, 127, 128, 255, 510, 511):
            ref = view.prefill_row(b, i, heads)
            assert_abs_close(lse[b, i, heads], ref["lse"][heads], tol, f"lse ({b},{i})")
            assert_rms_close(out[b, i, heads], ref["o"][heads], tol, f"o ({b},{i})")
    # every output against the absorbed path.  That path carries bf16 rounding noise of RMS about
    # 2e-3 of the output RMS (measured), this one several times less, so their difference has an
    # RMS below 5e-3; a lost tile or a wrong mask moves whole rows by O(1).  lse: each within tol
    # of the oracle.
    ao = _np(ab.out).astype(np.float64)
    diff = out.astype(np.float64) - ao
    rms = float(np.sqrt(np.mean(ao ** 2)))
    d_rms, d_max = float(np.sqrt(np.mean(diff ** 2))), float(np.max(np.abs(diff)))
    assert d_rms <= 5e-3 * rms, f"unabsorbed vs absorbed: rms diff {d_rms:.3e} > 5e-3 * rms {rms:.3e}"
    assert d_max <= 1e-1 * rms, f"unabsorbed vs absorbed: max diff {d_max:.3e} > 1e-1 * rms {rms:.3e}"
    assert np.all(np.abs(lse - _np(ab.lse)) <= 2 * tol)


def test_unabsorbed_rejects_other_shapes():
    w = gen.Workload(name="u_small_h", seed=3, kind="prefill", batch=1, n_heads=4, ctx=8, q_len=4)
    d = runner.dims_for(w)
    assert not M.mla_prefill_unabsorbed_supported(d)
