"""GPU parity of multi-token verify through the decode path (mla_verify_rows, then the balanced
split-K decode, combine and out-projection over batch * q_len rows) against the fp64 oracle.

Query i of sequence b sits at position q_start[b] + i and reads keys t <= q_start[b] + i,
t < seq_lens[b] ([ase] causal-mask remark after Fig. 2), exactly as a chunked-prefill row, so the
oracle reference is the prefill row.  The rows' page table, lengths and positions are integers and
are checked bit for bit; o and lse use the bf16 tolerances on every head of the checked rows (o:
max |err| <= 2e-2 * RMS of the row, lse: 2e-2 absolute).  Every output is also compared with mla_prefill_chunk on the
same inputs: both round the same q_hat bits, so they differ only by the rounding of P and the
order of the sums.
"""

import numpy as np
import pytest
import torch

from mla_latent_kv_31_amd import runner
from mla_workloads import gen
from parity import TOL, OracleView, assert_abs_close, assert_rms_close, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _check_rows(inp, st):
    B, Sq = st.B, st.Sq
    qs = inp["q_start"].astype(np.int64)
    pos = (qs[:, None] + np.arange(Sq)[None, :]).reshape(-1)
    lens = np.minimum(np.maximum(pos + 1, 0), np.repeat(inp["lens"].astype(np.int64), Sq))
    assert np.array_equal(st.row_lens.cpu().numpy(), lens.astype(np.int32)), "row lengths"
    assert np.array_equal(st.row_pos.cpu().numpy(), pos.astype(np.int32)), "row positions"
    assert np.array_equal(st.row_table.cpu().numpy(), np.repeat(inp["page_table"], Sq, axis=0)), "row page table"


def _check_against_prefill(inp, st):
    pf = runner.PrefillStep(inp, DEV)
    pf.run()
    torch.cuda.synchronize()
    a, b = _np(st.out).astype(np.float64), _np(pf.out).astype(np.float64)
    rms = float(np.sqrt(np.mean(b ** 2)))
    diff = a - b
    assert float(np.sqrt(np.mean(diff ** 2))) <= 5e-3 * rms, "verify vs prefill: rms diff"
    assert float(np.max(np.abs(diff))) <= 5e-2 * rms, "verify vs prefill: max diff"
    la, lb = _np(st.lse), _np(pf.lse)
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(la), fin) and np.array_equal(la[~fin], lb[~fin])
    assert np.all(np.abs(la[fin] - lb[fin]) <= 2 * TOL["bf16"])


@pytest.mark.parametrize("grouped", [True, False])
def test_verify_small_ragged(grouped):
    """Five sequences with prior lengths 1..300 and four draft tokens; one verify window starts
    at -2 (its first two rows see no key: o = 0, lse = -inf), one at 0.  Every head of every row
    against the oracle, every output against mla_prefill_chunk; with the draft rows of a sequence
    as one row group (mla_decode_partial_grouped) and with the plain balanced split."""
    w = gen.Workload(name="verify_small", seed=21, kind="prefill", batch=5, ctx_range=(1, 300), q_len=4,
                     random_pages=True)
    inp = gen.make_prefill_inputs(w)
    inp["q_start"] = inp["q_start"].copy()
    inp["q_start"][1] = -2
    inp["q_start"][3] = 0
    note(f"verify small ragged grouped={grouped} lens={inp['lens'].tolist()} q_start={inp['q_start'].tolist()}")
    st = runner.VerifyStep(inp, DEV, n_units=16, grouped=grouped)
    assert st.group == (4 if grouped else 1)
    st.run()
    torch.cuda.synchronize()
    _check_rows(inp, st)
    view = OracleView(inp)
    out, lse = _np(st.out), _np(st.lse)
    for b in range(w.batch):
        for i in range(w.q_len):
            if int(inp["q_start"][b]) + i < 0:
                assert np.all(out[b, i] == 0.0) and np.all(np.isneginf(lse[b, i])), f"row ({b},{i}) sees no key"
                continue
            ref = view.prefill_row(b, i)
            assert_abs_close(lse[b, i], ref["lse"], TOL["bf16"], f"lse ({b},{i})")
            assert_rms_close(out[b, i], ref["o"], TOL["bf16"], f"o ({b},{i})")
    _check_against_prefill(inp, st)


def test_verify_v3_b64_sq4():
    """The benchmark verify batch (64 ragged sequences of 1k-32k prior tokens, 4 draft tokens
    each, 256 units): integer row data exactly, every head of sampled rows against the oracle,
    every output against mla_prefill_chunk."""
    inp = gen.make_prefill_inputs(gen.WORKLOADS["v3_verify_b64_sq4"])
    note("verify v3_verify_b64_sq4")
    st = runner.VerifyStep(inp, DEV, n_units=256)
    assert st.group == 4
    st.run()
    torch.cuda.synchronize()
    _check_rows(inp, st)
    view = OracleView(inp)
    out, lse = _np(st.out), _np(st.lse)
    longest = int(np.argmax(inp["lens"]))
    for b, i in [(0, 0), (0, 3), (longest, 3), (63, 1), (17, 2)]:
        ref = view.prefill_row(b, i)
        assert_abs_close(lse[b, i], ref["lse"], TOL["bf16"], f"lse ({b},{i})")
        assert_rms_close(out[b, i], ref["o"], TOL["bf16"], f"o ({b},{i})")
    _check_against_prefill(inp, st)
