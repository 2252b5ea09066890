"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Every workload of the table runs at its full size in the launch configuration the benchmark
times; outputs the oracle can afford are compared in full (toy, batch-1 4k, small V3 shapes),
the large workloads on sampled (sequence, head) or (query row, head) outputs.
"""

import math

import numpy as np
import pytest
import torch

import mla_latent_kv_31_amd as M
import oracle.mla_oracle as O
from mla_latent_kv_31_amd import runner
from mla_workloads import gen
from balanced_ref import segments
from parity import TOL, OracleView, assert_abs_close, assert_mid_close, assert_rms_close, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LOG2E = 1.0 / math.log(2.0)


def _np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


# ------------------------------------------------------------------------------------------ toy
@pytest.mark.parametrize("page_size,split", [(4, 4), (1, 1), (2, 2), (1, 3)])
def test_toy_single_step_end_to_end(page_size, split):
    """Toy fp32 step from hidden states: cache write, query projections, absorb, split-K decode,
    combine and value projection all on the GPU; the oracle decompresses from the same h."""
    note(f"toy page_size={page_size} split={split}")
    t = gen.make_toy_inputs()
    w = t["workload"]
    d = runner.dims_for(w)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    h = dev(t["h"])
    Lc = w.ctx
    npages = -(-Lc // page_size)
    pool = torch.full((npages + 1, page_size, w.d_c + w.d_r), float("nan"), device=DEV)
    table = dev(np.arange(npages, dtype=np.int32)[None])
    lens = dev(np.array([Lc], np.int32))
    c = M.cache(pool, table, lens)
    M.mla_kv_append(d, c, w.d_model, h, dev(t["w_dkv"]), dev(t["w_kr"]), dev(np.zeros(Lc, np.int32)),
                    dev(np.arange(Lc, dtype=np.int32)), Lc, 0.0, None, 0)
    q_c = torch.empty((1, w.n_heads, w.d_k), device=DEV)
    q_r = torch.empty((1, w.n_heads, w.d_r), device=DEV)
    M.mla_project_query(d, w.d_model, w.d_cq, h[Lc - 1:Lc], dev(t["w_dq"]), dev(t["w_uq"]), dev(t["w_qr"]), 1, q_c, q_r)
    q_hat = torch.empty((1, w.n_heads, w.d_c + w.d_r), device=DEV)
    M.mla_absorb_query(d, q_c, q_r, dev(t["w_uk"]), dev(np.array([Lc - 1], np.int32)), 1, q_hat)
    S = M.mla_decode_num_splits(Lc, split)
    assert M.mla_decode_workspace_bytes(d, c, Lc, split) == M.mla_partials_bytes(d, S)
    ws, ws_bytes, o_part, lse_part = runner.partials_workspace(d, S, DEV)
    o_part, lse_part = o_part.view(1, S, w.n_heads, w.d_c), lse_part.view(1, S, w.n_heads)
    M.mla_decode_partial(d, c, q_hat, Lc, split, ws, ws_bytes)
    z = torch.empty((1, w.n_heads, w.d_c), device=DEV)
    lse = torch.empty((1, w.n_heads), device=DEV)
    M.mla_combine(d, 1, S, ws, ws_bytes, z, lse)
    out = torch.empty((1, w.n_heads, w.d_v), device=DEV)
    M.mla_out_proj(d, z, dev(t["w_uv"]), 1, out)
    torch.cuda.synchronize()

    hh = t["h"].astype(np.float64)
    rows = O.cache_rows(O.kv_latent(hh, t["w_dkv"]), O.rope_key(hh, t["w_kr"], np.arange(Lc), w.rope_base))
    _, qc, qr = O.query_parts(hh[Lc - 1], t["w_dq"], t["w_uq"], t["w_qr"])
    ref = O.attention(qc, qr, Lc - 1, rows, t["w_uk"], t["w_uv"], w.d_c, base=w.rope_base)
    tol = TOL["f32"]
    got_rows = _np(pool)[np.arange(npages)].reshape(-1, w.d_c + w.d_r)[:Lc]
    assert_rms_close(got_rows, rows, tol, "cache rows")
    assert_rms_close(_np(q_c)[0], qc, tol, "q_c")
    assert_rms_close(_np(q_r)[0], qr, tol, "q_r")
    qh = O.absorbed_query(qc, qr, Lc - 1, t["w_uk"], w.rope_base) * (w.sm_scale * LOG2E)
    assert_rms_close(_np(q_hat)[0], qh, tol, "q_hat")
    zp, lp = O.chunk_partials(qc, qr, Lc - 1, rows, t["w_uk"], t["w_uv"], w.d_c, split, base=w.rope_base)
    assert_rms_close(_np(o_part)[0], zp, tol, "o_part")
    assert_abs_close(_np(lse_part)[0], lp, tol, "lse_part")
    assert_rms_close(_np(z)[0], ref["z"], tol, "z")
    assert_abs_close(_np(lse)[0], ref["lse"], tol, "lse")
    assert_rms_close(_np(out)[0], ref["o"], tol, "o")


# ------------------------------------------------------------------------------------------ V3 decode
@pytest.fixture(scope="module")
def inp_b1():
    return gen.make_decode_inputs(gen.WORKLOADS["v3_b1_ctx4k"])


def _check_full_sequence(step, view, b, tol, flags_note="", dtype="bf16"):
    ref = view.decode(b)
    assert_mid_close(_np(step.z)[b], ref["z"], dtype, f"z seq {b} {flags_note}")
    assert_abs_close(_np(step.lse)[b], ref["lse"], tol, f"lse seq {b} {flags_note}")
    assert_rms_close(_np(step.out)[b], ref["o"], tol, f"o seq {b} {flags_note}")


@pytest.mark.parametrize("flags", [0, M.MLA_FLAG_FORCE_GENERIC])
def test_v3_b1_ctx4k_all_heads(inp_b1, flags):
    w = inp_b1["workload"]
    note(f"v3_b1_ctx4k flags={flags} split={w.split_tokens}")
    st = runner.DecodeStep(inp_b1, w.split_tokens, DEV, flags=flags)
    st.run()
    torch.cuda.synchronize()
    view = OracleView(inp_b1)
    tol = TOL["bf16"]
    assert_rms_close(_np(st.q_hat)[0], view.q_hat(0) * (w.sm_scale * LOG2E), tol, "q_hat")
    _check_full_sequence(st, view, 0, tol, f"flags={flags}")
    # split partials of the first, a middle and the last chunk
    for i in (0, st.S // 2, st.S - 1):
        r = view.decode(0, key_range=(i * st.split_tokens, (i + 1) * st.split_tokens))
        assert_mid_close(_np(st.o_part)[0, i], r["z"], "bf16", f"o_part chunk {i}")
        assert_abs_close(_np(st.lse_part)[0, i], r["lse"], tol, f"lse_part chunk {i}")


@pytest.fixture(scope="module")
def inp_ragged():
    return gen.make_decode_inputs(gen.WORKLOADS["v3_b64_ragged_paged"])


def _decode_step(inp, mode, flags=0):
    """The fixed split at the workload's chunk length, or the balanced split over the device's
    compute units (the configuration the benchmark times)."""
    w = inp["workload"]
    if mode == "balanced":
        n = runner.balanced_units(inp["lens"], runner.compute_units(DEV))
        return runner.DecodeStep(inp, 0, DEV, flags=flags, n_units=n)
    split = w.split_tokens if mode == "fixed" else int(mode)
    return runner.DecodeStep(inp, split, DEV, flags=flags)


def _check_balanced_slots(st, view, picks):
    """Compare the partials of a few balanced segments, every head, with the oracle over their
    token ranges."""
    segs = segments(_lens_of(st), st.n_units)
    for k in picks:
        w_, b, t0, t1, slot = segs[k % len(segs)]
        r = view.decode(b, key_range=(t0, t1))
        assert_mid_close(_np(st.o_part)[slot], r["z"], "bf16", f"o_part slot {slot} seq {b} [{t0},{t1})")
        assert_abs_close(_np(st.lse_part)[slot], r["lse"], TOL["bf16"], f"lse_part slot {slot}")


def _lens_of(st):
    return st.lens.cpu().numpy()


@pytest.mark.parametrize("mode", ["fixed", "balanced"])
def test_v3_b64_ragged_paged_sampled(inp_ragged, mode):
    w = inp_ragged["workload"]
    st = _decode_step(inp_ragged, mode)
    note(f"v3_b64_ragged_paged mode={mode} split={st.split_tokens} units={st.n_units} "
         f"total_tokens={int(inp_ragged['lens'].sum())}")
    assert st.uses_mfma()
    st.run()
    torch.cuda.synchronize()
    view = OracleView(inp_ragged)
    lens = inp_ragged["lens"]
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17})
    tol = TOL["bf16"]
    for b in seqs:  # every head of the shortest, the longest and one other sequence
        ref = view.decode(b)
        assert_mid_close(_np(st.z)[b], ref["z"], "bf16", f"z seq {b}")
        assert_abs_close(_np(st.lse)[b], ref["lse"], tol, f"lse seq {b}")
        assert_rms_close(_np(st.out)[b], ref["o"], tol, f"o seq {b}")
    if mode == "balanced":
        _check_balanced_slots(st, view, (0, 1, 150, -1))
    # any-size properties on every output: finite, and z inside the convex hull bound of |c|
    assert np.isfinite(_np(st.out)).all() and np.isfinite(_np(st.lse)).all()


@pytest.fixture(scope="module")
def inp_long():
    return gen.make_decode_inputs(gen.WORKLOADS["v3_b4_ctx128k"])


@pytest.mark.parametrize("mode", ["fixed", "512", "balanced"])
def test_v3_b4_ctx128k_sampled(inp_long, mode):
    st = _decode_step(inp_long, mode)
    note(f"v3_b4_ctx128k mode={mode} split={st.split_tokens} units={st.n_units}")
    if st.n_units is None:
        assert st.B * st.S >= 256  # at least 256 split-K chunks over the batch
    else:
        assert len(segments(_lens_of(st), st.n_units)) >= 256
    assert st.uses_mfma()
    st.run()
    torch.cuda.synchronize()
    view = OracleView(inp_long)
    tol = TOL["bf16"]
    b = {"fixed": 0, "512": 3, "balanced": 1}[mode]  # every head of one 131,072-token sequence
    ref = view.decode(b)
    assert_mid_close(_np(st.z)[b], ref["z"], "bf16", f"z seq {b}")
    assert_abs_close(_np(st.lse)[b], ref["lse"], tol, f"lse seq {b}")
    assert_rms_close(_np(st.out)[b], ref["o"], tol, f"o seq {b}")
    if st.n_units is not None:
        _check_balanced_slots(st, view, (0, 1, 128, -1))
        return
    for i in (0, 1, st.S // 2, st.S - 1):
        r = view.decode(1, key_range=(i * st.split_tokens, (i + 1) * st.split_tokens))
        assert_mid_close(_np(st.o_part)[1, i], r["z"], "bf16", f"o_part chunk {i}")
        assert_abs_close(_np(st.lse_part)[1, i], r["lse"], tol, f"lse_part chunk {i}")


# ------------------------------------------------------------------------------------------ prefill
@pytest.fixture(scope="module")
def inp_prefill():
    return gen.make_prefill_inputs(gen.WORKLOADS["v3_prefill_b2"])


@pytest.mark.parametrize("flags", [0, M.MLA_FLAG_FORCE_GENERIC])
def test_v3_prefill_sampled(inp_prefill, flags):
    note(f"v3_prefill_b2 flags={flags}")
    st = runner.PrefillStep(inp_prefill, DEV, flags=flags)
    assert st.uses_mfma() == (flags == 0)
    st.run()
    torch.cuda.synchronize()
    view = OracleView(inp_prefill)
    tol = TOL["bf16"]
    for b in (0, 1):  # every head of sampled rows
        for i in (0, 1, 63, 64, 255, 510, 511):
            ref = view.prefill_row(b, i)
            assert_mid_close(_np(st.z)[b, i], ref["z"], "bf16", f"z ({b},{i})")
            assert_abs_close(_np(st.lse)[b, i], ref["lse"], tol, f"lse ({b},{i})")
            assert_rms_close(_np(st.out)[b, i], ref["o"], tol, f"o ({b},{i})")


@pytest.mark.parametrize("flags", [0, M.MLA_FLAG_FORCE_GENERIC])
def test_prefill_small_ragged_start_all_rows(flags):
    """Small chunks with different starts per sequence (q_start 0 puts the first row on a single
    key); every head of every row of every sequence, z / lse / o against the oracle."""
    w = gen.Workload(name="prefill_small", seed=9, kind="prefill", batch=3, ctx=70, q_len=40, random_pages=True)
    inp = gen.make_prefill_inputs(w)
    inp["q_start"] = np.array([70, 0, 33], np.int32)  # rows past q_start+i stay invisible
    note(f"prefill small flags={flags}")
    st = runner.PrefillStep(inp, DEV, flags=flags)
    assert st.uses_mfma() == (flags == 0)
    st.run()
    torch.cuda.synchronize()
    view = OracleView(inp)
    tol = TOL["bf16"]
    for b in range(3):
        for i in range(40):
            if int(inp["q_start"][b]) + i < 0:
                continue
            ref = view.prefill_row(b, i)
            assert_mid_close(_np(st.z)[b, i], ref["z"], "bf16", f"z ({b},{i})")
            assert_abs_close(_np(st.lse)[b, i], ref["lse"], tol, f"lse ({b},{i})")
            assert_rms_close(_np(st.out)[b, i], ref["o"], tol, f"o ({b},{i})")


# ------------------------------------------------------------------------------------------ small V3 shapes
def _small(dtype, lens, seed=11, random_pages=True, H=128):
    w = gen.Workload(name="small", seed=seed, kind="decode", batch=len(lens), n_heads=H, dtype=dtype,
                     random_pages=random_pages)
    return gen.make_decode_inputs(w, lens=np.array(lens, np.int32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("split", [64, 192, 4096, "units=1", "units=7", "units=256"])
def test_v3_small_ragged_all_heads(dtype, split):
    lens = [1, 63, 64, 65, 300, 1000]
    note(f"small ragged dtype={dtype} split={split}")
    inp = _small(dtype, lens)
    if isinstance(split, str):
        st = runner.DecodeStep(inp, 0, DEV, n_units=int(split.split("=")[1]))
    else:
        st = runner.DecodeStep(inp, split, DEV)
    st.run()
    torch.cuda.synchronize()
    view = OracleView(inp)
    for b in range(len(lens)):
        _check_full_sequence(st, view, b, TOL[dtype], f"{dtype} split={split}", dtype)


def test_empty_sequence_and_spare_chunks():
    """A zero-length sequence yields z = 0, o = 0, lse = -inf; a max_len well above every length
    adds empty chunks that must not change the others."""
    lens = [0, 130, 5]
    note("empty sequence + spare chunks")
    inp = _small("bf16", lens, seed=12)
    inp["lens"] = np.array(lens, np.int32)
    st = runner.DecodeStep(inp, 64, DEV, max_len=inp["page_table"].shape[1] * 64)
    st.run()
    torch.cuda.synchronize()
    z, lse, out = _np(st.z), _np(st.lse), _np(st.out)
    assert np.all(z[0] == 0) and np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(_np(st.lse_part)[0] == -np.inf)
    view = OracleView(inp)
    for b in (1, 2):
        _check_full_sequence(st, view, b, TOL["bf16"], "spare chunks")
