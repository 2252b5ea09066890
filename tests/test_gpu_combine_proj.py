"""GPU parity of the fused split-K merge + value projection (mla_combine_out_proj*): against the
fp64 oracle on every head of the checked sequences, and against the two calls it replaces
(mla_combine* then mla_out_proj) on the same partials, through the C ABI."""

import numpy as np
import pytest
import torch

import mla_latent_kv_31_amd as M
from mla_latent_kv_31_amd import runner
from mla_workloads import gen
from parity import TOL, OracleView, assert_abs_close, assert_rms_close, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# Same partials, same product: the two sides differ only in the order the merge weights are summed
# (float32), far below the bf16 tolerance of the path.
TOL_SAME = 1e-5


def _np(t):
    return t.cpu().numpy()


def _small(lens, seed=41, H=128, dtype="bf16"):
    w = gen.Workload(name="small", seed=seed, kind="decode", batch=len(lens), n_heads=H, dtype=dtype,
                     random_pages=True)
    return gen.make_decode_inputs(w, lens=np.array(lens, np.int32))


def _both(st):
    """Run the step unfused, keep (out, lse), then run the fused call on the same partials."""
    st.absorb()
    st.attend()
    st.combine()
    st.out_proj()
    torch.cuda.synchronize()
    out_u, lse_u = _np(st.out).copy(), _np(st.lse).copy()
    st.out.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    st.combine_out_proj()
    torch.cuda.synchronize()
    return out_u, lse_u, _np(st.out), _np(st.lse)


def _compare_same(out_u, lse_u, out_f, lse_f, what):
    assert np.isfinite(out_f).all(), f"{what}: non-finite output"
    assert_rms_close(out_f, out_u, TOL_SAME, f"{what}: fused o vs combine + out_proj")
    assert_abs_close(lse_f, lse_u, 1e-5, f"{what}: fused lse vs combine")


@pytest.fixture(scope="module")
def inp_ragged():
    return gen.make_decode_inputs(gen.WORKLOADS["v3_b64_ragged_paged"])


def test_v3_b64_ragged_paged_balanced(inp_ragged):
    """The benchmark configuration: 64 ragged sequences, the balanced split over every compute unit."""
    n = runner.balanced_units(inp_ragged["lens"], runner.compute_units(DEV))
    note(f"v3_b64_ragged_paged fused merge+projection units={n}")
    st = runner.DecodeStep(inp_ragged, 0, DEV, n_units=n, fused=True)
    assert st.fused
    out_u, lse_u, out_f, lse_f = _both(st)
    _compare_same(out_u, lse_u, out_f, lse_f, "v3_b64_ragged_paged")
    view = OracleView(inp_ragged)
    lens = inp_ragged["lens"]
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17}):  # every head of three sequences
        ref = view.decode(b)
        assert_abs_close(lse_f[b], ref["lse"], TOL["bf16"], f"lse seq {b}")
        assert_rms_close(out_f[b], ref["o"], TOL["bf16"], f"o seq {b}")


@pytest.mark.parametrize("split", [64, 192, "units=1", "units=7", "units=256"])
def test_small_ragged_every_sequence(split):
    """Short, page-boundary and longer rows, an empty row, and a batch that is not a multiple of
    the 32 rows of a workgroup (37 rows: a ragged last row slice)."""
    rng = np.random.default_rng(5)
    lens = [0, 1, 63, 64, 65, 300, 1000] + [int(x) for x in rng.integers(1, 700, size=30)]
    note(f"small ragged fused split={split} rows={len(lens)}")
    inp = _small(lens)
    if isinstance(split, str):
        st = runner.DecodeStep(inp, 0, DEV, n_units=int(split.split("=")[1]), fused=True)
    else:
        st = runner.DecodeStep(inp, split, DEV, fused=True)
    out_u, lse_u, out_f, lse_f = _both(st)
    _compare_same(out_u, lse_u, out_f, lse_f, f"split={split}")
    assert np.all(out_f[0] == 0) and np.all(lse_f[0] == -np.inf)  # no key: o = 0, lse = -inf
    view = OracleView(inp)
    for b in range(1, 8):
        ref = view.decode(b)
        assert_abs_close(lse_f[b], ref["lse"], TOL["bf16"], f"lse seq {b}")
        assert_rms_close(out_f[b], ref["o"], TOL["bf16"], f"o seq {b}")


def test_unwritten_slots_never_reach_the_output():
    """Spare chunks of a fixed split (max_len far above every length) are never written by the
    decode; NaN, Inf or zero in them leaves the fused output bitwise unchanged."""
    lens = [0, 130, 5, 64]
    note("fused merge with poisoned spare chunks")
    inp = _small(lens, seed=42)
    st = runner.DecodeStep(inp, 64, DEV, max_len=inp["page_table"].shape[1] * 64, fused=True)
    results = []
    for fill in (0.0, float("nan"), float("inf")):
        st.ws.view(torch.float32).fill_(fill)
        st.absorb()
        st.attend()
        st.combine_out_proj()
        torch.cuda.synchronize()
        results.append((_np(st.out).copy(), _np(st.lse).copy()))
    for out, lse in results[1:]:
        assert np.array_equal(out, results[0][0]) and np.array_equal(lse, results[0][1])
    assert np.isfinite(results[0][0]).all()


def test_verify_row_groups():
    """The draft rows of a multi-token verify step as row groups (mla_combine_out_proj_grouped)."""
    w = gen.WORKLOADS["v3_verify_b64_sq4"]
    inp = gen.make_prefill_inputs(w)
    note("verify row groups fused merge+projection")
    st = runner.VerifyStep(inp, DEV, n_units=256, fused=True)
    assert st.fused and st.group == 4
    st.rows()
    st.absorb()
    st.attend()
    st.combine()
    st.out_proj()
    torch.cuda.synchronize()
    out_u, lse_u = _np(st.out).copy(), _np(st.lse).copy()
    st.out.fill_(float("nan"))
    st.combine_out_proj()
    torch.cuda.synchronize()
    _compare_same(out_u, lse_u, _np(st.out), _np(st.lse), "verify groups")
    view = OracleView(inp)
    for b, i in ((0, 0), (0, 3), (37, 2)):
        ref = view.prefill_row(b, i)
        assert_rms_close(_np(st.out)[b, i], ref["o"], TOL["bf16"], f"o ({b},{i})")


@pytest.mark.parametrize("H", [12, 130])
def test_head_counts_off_the_xcd_grid(H):
    """Head counts that are not a multiple of the eight XCDs (the grid rounds them up and the spare
    workgroups leave at once): the partials come from the generic decode, the fused call must
    still match combine + out_proj and the oracle."""
    lens = [5, 300, 64, 1]
    note(f"fused merge+projection H={H}")
    inp = _small(lens, seed=43, H=H)
    st = runner.DecodeStep(inp, 0, DEV, n_units=7, fused=True)
    assert st.fused
    out_u, lse_u, out_f, lse_f = _both(st)
    _compare_same(out_u, lse_u, out_f, lse_f, f"H={H}")
    view = OracleView(inp)
    for b in range(len(lens)):
        ref = view.decode(b)
        assert_rms_close(out_f[b], ref["o"], TOL["bf16"], f"o seq {b}")
