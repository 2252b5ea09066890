"""Exactness of split-K indexing and length masking on the GPU.

* count test: with a zero query every score is 0, so each chunk's softmax sum is exactly its
  number of valid tokens; exp(lse_part) must round to that integer, empty chunks give -inf/0.
* spike test: one token scores 2^128 above the rest, so z must equal that token's latent; a
  chunk or length boundary off by one gives an O(1) error instead of a 1/len-sized one.
* poison test: NaN / Inf / zero in every slot a correct reader never touches must give
  bitwise-identical outputs.
* permutation test: two physical page layouts of one logical cache give bitwise-identical outputs.
* re-runs are bitwise deterministic; split sizes agree to fp32 rounding.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_31_amd as M
from mla_latent_kv_31_amd import runner
from mla_workloads import gen
from parity import note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
V3 = dict(n_heads=128, d_c=512, d_r=64, d_k=128, d_v=128)


def _w(batch, seed=21, random_pages=True):
    return gen.Workload(name="exact", seed=seed, kind="decode", batch=batch, random_pages=random_pages, **V3)


def _np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _run_partial(inp, split, q_hat_np=None, flags=0, max_len=None):
    st = runner.DecodeStep(inp, split, DEV, flags=flags, max_len=max_len)
    if q_hat_np is None:
        st.absorb()
    else:
        st.q_hat.copy_(runner.to_device(q_hat_np, DEV))
    st.attend()
    st.combine()
    torch.cuda.synchronize()
    return st


PATHS = [0, M.MLA_FLAG_FORCE_GENERIC]


def _masked_parts(st):
    """Split partials of the non-empty chunks (an empty chunk's o_part row is left untouched)."""
    o = _np(st.o_part).copy()
    o[~np.isfinite(_np(st.lse_part))] = 0.0
    return o


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("split", [64, 128, 512])
def test_count(split, flags):
    lens = [1, 2, 63, 64, 65, 127, 128, 129, 500, 1000, 1024, 1025]
    note(f"count split={split} flags={flags}")
    inp = gen.make_decode_inputs(_w(len(lens)), lens=np.array(lens, np.int32), fill="nan")
    q0 = np.zeros((len(lens), 128, 576), np.uint16)
    st = _run_partial(inp, split, q0, flags=flags)
    lse_p, o_p = _np(st.lse_part), _np(st.o_part)
    for b, L in enumerate(lens):
        for i in range(st.S):
            cnt = max(0, min(L, (i + 1) * split) - i * split)
            if cnt == 0:  # empty chunk: lse = -inf (its o_part is never read)
                assert np.all(lse_p[b, i] == -np.inf), (b, i)
                continue
            e = np.exp(lse_p[b, i].astype(np.float64))
            assert np.all(np.rint(e) == cnt), (b, i, cnt, e[:4])
            assert np.max(np.abs(e - cnt)) <= 1e-4 * cnt, (b, i)
    # whole-sequence count through the combine
    assert np.all(np.rint(np.exp(_np(st.lse).astype(np.float64))) == np.array(lens)[:, None])


def _spike_inputs(cases, seed=31):
    """cases: list of (length, spike position).  Column 0 of every latent is 0 except the spike
    token's (8.0); the query is 16 on that column only (base-2 logit 128 for the spike)."""
    rng = np.random.default_rng(seed)
    rows = []
    for L, t in cases:
        c = rng.standard_normal((L, 576)).astype(np.float32)
        c[:, 0] = 0.0
        c[t, 0] = 8.0
        rows.append(gen.bf16_bits(c))
    w = _w(len(cases), seed=seed)
    lens = np.array([L for L, _ in cases], np.int32)
    inp = gen.make_decode_inputs(w, lens=lens, latent_rows=rows, fill="nan")
    q = np.zeros((len(cases), 128, 576), np.float32)
    q[:, :, 0] = 16.0
    return inp, gen.bf16_bits(q), rows


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("split", [64, 128, 256])
def test_spike_at_every_boundary(split, flags):
    cases = []
    for L in (1, 64, 65, 200, 1000, 1025):
        ts = {0, L - 1}
        for i in range(0, -(-L // split)):
            ts |= {i * split, i * split + split - 1, i * split + 63, i * split + 64}
        cases += [(L, t) for t in sorted(ts) if 0 <= t < L]
    note(f"spike split={split} flags={flags} cases={len(cases)}")
    inp, q, rows = _spike_inputs(cases)
    st = _run_partial(inp, split, q, flags=flags)
    z, lse = _np(st.z), _np(st.lse)
    for b, (L, t) in enumerate(cases):
        want = gen.bf16_from_bits(rows[b][t, :512]).astype(np.float64)
        err = np.max(np.abs(z[b] - want[None]))
        assert err <= 1e-5, f"len {L} spike {t}: z off by {err}"
        assert np.allclose(lse[b], 128.0 * np.log(2.0), atol=1e-4), (L, t, lse[b, :2])


@pytest.mark.parametrize("flags", PATHS)
def test_poison_bitwise(flags):
    lens = np.array([1, 63, 64, 65, 700, 1234, 4000], np.int32)
    note(f"poison flags={flags}")
    outs = []
    for fill in ("zero", "nan", "inf"):
        inp = gen.make_decode_inputs(_w(len(lens)), lens=lens, fill=fill, spare_pages=16)
        st = _run_partial(inp, 128, flags=flags)
        st.out_proj()
        torch.cuda.synchronize()
        outs.append([_masked_parts(st)] + [_np(x).copy() for x in (st.lse_part, st.z, st.lse, st.out)])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("flags", PATHS)
def test_page_permutation_bitwise_and_determinism(flags):
    lens = np.array([5, 640, 1999, 3000], np.int32)
    note(f"permutation flags={flags}")
    res = []
    for rp in (False, True):
        inp = gen.make_decode_inputs(_w(len(lens), random_pages=rp), lens=lens, fill="zero", random_pages=rp)
        st = _run_partial(inp, 256, flags=flags)
        res.append([_masked_parts(st)] + [_np(x).copy() for x in (st.lse_part, st.z, st.lse)])
        st.attend()
        st.combine()
        torch.cuda.synchronize()
        again = [_masked_parts(st)] + [_np(x) for x in (st.lse_part, st.z, st.lse)]
        for a, b in zip(res[-1], again):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "re-run differs"
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "page layout changes the result"


def test_split_invariance():
    """Different chunkings agree to rounding: each chunk rounds its probabilities to binary16
    relative to its own reference maximum (2^-11 relative), and each result is within ~2e-3 of the
    RMS of z of the exact one on short peaked rows (CPU simulation of those roundings), so two
    splits differ by at most 4e-3 of it (measured: 1.7e-3 between 64-token chunks and whole
    sequences).  An indexing slip across chunk boundaries would be O(RMS)."""
    lens = np.array([3000, 70, 4096], np.int32)
    note("split invariance")
    inp = gen.make_decode_inputs(_w(len(lens), seed=41), lens=lens)
    zs = []
    for split in (64, 128, 512, 4096):
        st = _run_partial(inp, split)
        zs.append((_np(st.z).copy(), _np(st.lse).copy()))
    for z, lse in zs[1:]:
        d = np.max(np.abs(z - zs[0][0])) / np.sqrt(np.mean(zs[0][0] ** 2))
        note(f"split invariance: max |dz| / RMS(z) = {d:.2e}")
        assert d <= 4e-3
        assert np.max(np.abs(lse - zs[0][1])) <= 1e-3


# ------------------------------------------------------------------------------ balanced split
from balanced_ref import segments  # noqa: E402


def _run_balanced(inp, n_units, q_hat_np=None, flags=0):
    st = runner.DecodeStep(inp, 0, DEV, flags=flags, n_units=n_units)
    if q_hat_np is None:
        st.absorb()
    else:
        st.q_hat.copy_(runner.to_device(q_hat_np, DEV))
    st.attend()
    st.combine()
    torch.cuda.synchronize()
    return st


def _segment_parts(st, lens):
    """Partials of the non-empty segments only (other slots are never written)."""
    segs = segments(lens, st.n_units)
    idx = [s[4] for s in segs]
    return _np(st.o_part)[idx].copy(), _np(st.lse_part)[idx].copy()


BAL_LENS = [0, 1, 2, 63, 64, 65, 127, 128, 129, 500, 1000, 1024, 1025, 0, 3000, 31, 33]


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("n_units", [1, 3, 16, 64, 256, 2048])
def test_count_balanced(n_units, flags):
    lens = BAL_LENS
    note(f"count balanced n_units={n_units} flags={flags}")
    inp = gen.make_decode_inputs(_w(len(lens)), lens=np.array(lens, np.int32), fill="nan")
    q0 = np.zeros((len(lens), 128, 576), np.uint16)
    st = _run_balanced(inp, n_units, q0, flags=flags)
    lse_p = _np(st.lse_part)
    segs = segments(lens, n_units)
    assert segs and len({s[4] for s in segs}) == len(segs)
    for w, b, t0, t1, slot in segs:
        e = np.exp(lse_p[slot].astype(np.float64))
        assert np.all(np.rint(e) == t1 - t0), (w, b, t0, t1, e[:4])
    lse = _np(st.lse).astype(np.float64)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(lse[b] == -np.inf) and np.all(_np(st.z)[b] == 0)
        else:
            assert np.all(np.rint(np.exp(lse[b])) == L), b


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("n_units", [1, 5, 256])
def test_spike_balanced(n_units, flags):
    cases = []
    for L in (1, 65, 1000, 1025):
        cases += [(L, t) for t in sorted({0, 31, 32, L // 2, L - 1}) if t < L]
    note(f"spike balanced n_units={n_units} flags={flags} cases={len(cases)}")
    inp, q, rows = _spike_inputs(cases)
    st = _run_balanced(inp, n_units, q, flags=flags)
    z, lse = _np(st.z), _np(st.lse)
    for b, (L, t) in enumerate(cases):
        want = gen.bf16_from_bits(rows[b][t, :512]).astype(np.float64)
        err = np.max(np.abs(z[b] - want[None]))
        assert err <= 1e-5, f"len {L} spike {t}: z off by {err}"
        assert np.allclose(lse[b], 128.0 * np.log(2.0), atol=1e-4), (L, t, lse[b, :2])


# ------------------------------------------------------------------------------ row groups
def _run_grouped(inp, n_units, group, q_hat_np, flags=0):
    """The balanced split with row groups (mla_decode_partial_grouped / mla_combine_grouped) on
    a DecodeStep's buffers; the plain split's workspace size suffices."""
    st = runner.DecodeStep(inp, 0, DEV, flags=flags, n_units=n_units)
    st.q_hat.copy_(runner.to_device(q_hat_np, DEV))
    M.mla_decode_partial_grouped(st.d, st.c, st.q_hat, n_units, group, st.ws, st.ws_bytes)
    M.mla_combine_grouped(st.d, st.c, n_units, group, st.ws, st.ws_bytes, st.z, st.lse)
    torch.cuda.synchronize()
    return st


# verify-style groups (lengths base+1 .. base+G) and unrelated lengths, empty rows included
GROUP_LENS = {2: [0, 1, 63, 64, 64, 65, 1000, 1025, 0, 0, 3000, 31, 500, 501, 32, 1],
              4: [62, 63, 64, 65, 0, 1, 2, 3, 1022, 1023, 1024, 1025, 0, 0, 0, 0, 3000, 31, 33, 129]}
GROUP_LENS[20] = GROUP_LENS[4]  # the whole batch as one group


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("group,n_units", [(2, 2), (2, 16), (4, 4), (4, 16), (4, 256), (20, 20), (20, 60)])
def test_count_grouped(group, n_units, flags):
    """Zero query: every segment slot of the grouped split holds its exact token count, and each
    row's merged lse its length."""
    lens = GROUP_LENS[group]
    note(f"count grouped group={group} n_units={n_units} flags={flags}")
    inp = gen.make_decode_inputs(_w(len(lens)), lens=np.array(lens, np.int32), fill="nan")
    st = _run_grouped(inp, n_units, group, np.zeros((len(lens), 128, 576), np.uint16), flags=flags)
    lse_p = _np(st.lse_part)
    segs = segments(lens, n_units, group=group)
    assert segs and len({s[4] for s in segs}) == len(segs)
    for u, r, t0, t1, slot in segs:
        e = np.exp(lse_p[slot].astype(np.float64))
        assert np.all(np.rint(e) == t1 - t0), (u, r, t0, t1, e[:4])
    lse = _np(st.lse).astype(np.float64)
    for r, L in enumerate(lens):
        if L == 0:
            assert np.all(lse[r] == -np.inf) and np.all(_np(st.z)[r] == 0)
        else:
            assert np.all(np.rint(np.exp(lse[r])) == L), r


@pytest.mark.parametrize("flags", PATHS)
@pytest.mark.parametrize("n_units", [4, 8, 256])
def test_spike_grouped(n_units, flags):
    """A 2^128-weight token at segment and length boundaries of rows in groups of 4."""
    cases = []
    for L in (1, 65, 1000, 1025):
        cases += [(L, t) for t in sorted({0, 31, 32, L // 2, L - 1}) if t < L]
    while len(cases) % 4:
        cases.append((33, 32))
    note(f"spike grouped n_units={n_units} flags={flags} cases={len(cases)}")
    inp, q, rows = _spike_inputs(cases)
    st = _run_grouped(inp, n_units, 4, q, flags=flags)
    z, lse = _np(st.z), _np(st.lse)
    for b, (L, t) in enumerate(cases):
        want = gen.bf16_from_bits(rows[b][t, :512]).astype(np.float64)
        err = np.max(np.abs(z[b] - want[None]))
        assert err <= 1e-5, f"len {L} spike {t}: z off by {err}"
        assert np.allclose(lse[b], 128.0 * np.log(2.0), atol=1e-4), (L, t, lse[b, :2])


@pytest.mark.parametrize("flags", PATHS)
def test_poison_bitwise_grouped(flags):
    """NaN / Inf / zero in every cache slot past the rows' ends and in the spare pages give
    bitwise-identical grouped partials, merges and outputs (row groups of 4, verify-style and
    unrelated lengths)."""
    lens = np.array([62, 63, 64, 65, 1, 2, 3, 4, 1200, 31, 4000, 0], np.int32)
    note(f"poison grouped flags={flags}")
    outs = []
    for fill in ("zero", "nan", "inf"):
        inp = gen.make_decode_inputs(_w(len(lens)), lens=lens, fill=fill, spare_pages=16)
        st = runner.DecodeStep(inp, 0, DEV, flags=flags, n_units=8)
        st.absorb()
        M.mla_decode_partial_grouped(st.d, st.c, st.q_hat, 8, 4, st.ws, st.ws_bytes)
        M.mla_combine_grouped(st.d, st.c, 8, 4, st.ws, st.ws_bytes, st.z, st.lse)
        st.out_proj()
        torch.cuda.synchronize()
        idx = [sg[4] for sg in segments(lens, 8, group=4)]
        outs.append([_np(st.o_part)[idx].copy(), _np(st.lse_part)[idx].copy()] +
                    [_np(x).copy() for x in (st.z, st.lse, st.out)])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_long_segment_page_windows():
    """Segments longer than 64 pages move the page-id window inside the tile loop; with a spike
    near the end the rerun pass restarts from the first window.  Page size 32 (one tile per
    page) makes 64 pages only 2,048 tokens."""
    L = 5000
    cases = [(L, L - 1), (L, 2100), (L, 2047), (L, 2048)]
    note("long segment windows")
    rng = np.random.default_rng(5)
    rows = []
    for _, t in cases:
        c = rng.standard_normal((L, 576)).astype(np.float32)
        c[:, 0] = 0.0
        c[t, 0] = 8.0
        rows.append(gen.bf16_bits(c))
    w = gen.Workload(name="exact", seed=5, kind="decode", batch=len(cases), random_pages=True, page_size=32, **V3)
    inp = gen.make_decode_inputs(w, lens=np.full(len(cases), L, np.int32), latent_rows=rows, fill="nan")
    q = np.zeros((len(cases), 128, 576), np.float32)
    q[:, :, 0] = 16.0
    qb = gen.bf16_bits(q)
    for mode in ("balanced", "fixed"):
        if mode == "balanced":
            st = _run_balanced(inp, 1, qb)
        else:
            st = _run_partial(inp, 8192, qb)
        assert st.uses_mfma()
        z = _np(st.z)
        for b, (_, t) in enumerate(cases):
            want = gen.bf16_from_bits(rows[b][t, :512]).astype(np.float64)
            assert np.max(np.abs(z[b] - want[None])) <= 1e-5, (mode, t)
    # counts over the same long segments with a zero query
    st = _run_balanced(inp, 1, np.zeros_like(qb))
    assert np.all(np.rint(np.exp(_np(st.lse).astype(np.float64))) == L)


@pytest.mark.parametrize("flags", PATHS)
def test_poison_bitwise_balanced(flags):
    lens = np.array([1, 63, 64, 65, 700, 1234, 4000, 0], np.int32)
    note(f"poison balanced flags={flags}")
    outs = []
    for fill in ("zero", "nan", "inf"):
        inp = gen.make_decode_inputs(_w(len(lens)), lens=lens, fill=fill, spare_pages=16)
        st = _run_balanced(inp, 7, flags=flags)
        st.out_proj()
        torch.cuda.synchronize()
        outs.append(list(_segment_parts(st, lens)) + [_np(x).copy() for x in (st.z, st.lse, st.out)])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_balanced_matches_fixed_and_is_deterministic():
    lens = np.array([3000, 70, 4096, 1, 999], np.int32)
    note("balanced vs fixed")
    inp = gen.make_decode_inputs(_w(len(lens), seed=43), lens=lens)
    ref = _run_partial(inp, 4096)
    z0 = _np(ref.z).copy()
    for n_units in (1, 4, 33, 256):
        st = _run_balanced(inp, n_units)
        z, lse = _np(st.z).copy(), _np(st.lse).copy()
        d = np.max(np.abs(z - z0)) / np.sqrt(np.mean(z0 ** 2))
        note(f"balanced vs fixed: n_units {n_units}, max |dz| / RMS(z) = {d:.2e}")
        assert d <= 1e-3, n_units
        assert np.max(np.abs(lse - _np(ref.lse))) <= 1e-3
        st.attend()
        st.combine()
        torch.cuda.synchronize()
        assert np.array_equal(_np(st.z).view(np.uint32), z.view(np.uint32)), "re-run differs"


# ------------------------------------------------------------------------------ prefill causal mask
def _prefill_direct(inp, q_hat_np, q_start, flags=0):
    """mla_prefill_chunk on a given q_hat [B, q_len, H, 576] (given as bf16 bits, stored as the
    binary16 q_hat of the bf16 path: every test value is exact in both) and q_start [B]."""
    w = inp["workload"]
    d = runner.dims_for(w, flags)
    pool = runner.to_device(inp["pool"], DEV)
    table = runner.to_device(inp["page_table"], DEV)
    lens = runner.to_device(inp["lens"].astype(np.int32), DEV)
    c = M.cache(pool, table, lens)
    qh = runner.to_device(q_hat_np, DEV).to(runner.q_hat_dtype(w.dtype))
    B, Sq = q_hat_np.shape[:2]
    z = torch.empty((B, Sq, 128, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Sq, 128), dtype=torch.float32, device=DEV)
    M.mla_prefill_chunk(d, c, qh, Sq, runner.to_device(np.asarray(q_start, np.int32), DEV), z, lse)
    torch.cuda.synchronize()
    return _np(z), _np(lse), M.mla_prefill_uses_mfma(d, c)


@pytest.mark.parametrize("flags", PATHS)
def test_prefill_count_and_causal_spike(flags):
    """Zero query: lse = ln(visible keys) for every row.  Spike at token T (logit 128): rows at
    positions >= T return exactly that latent, rows before it never see it."""
    lens = np.array([300, 97], np.int32)
    T = 150
    Sq = 40
    q_start = np.array([130, 57], np.int32)  # seq 0 rows 130..169 straddle T; seq 1 rows 57..96
    rng = np.random.default_rng(7)
    rows = []
    for L in lens:
        cr = rng.standard_normal((L, 576)).astype(np.float32)
        cr[:, 0] = 0.0
        rows.append(cr)
    rows[0][T, 0] = 8.0
    rows = [gen.bf16_bits(r) for r in rows]
    inp = gen.make_decode_inputs(_w(2, seed=8), lens=lens, latent_rows=rows, fill="nan")
    note(f"prefill count/spike flags={flags}")
    # count
    z, lse, mf = _prefill_direct(inp, np.zeros((2, Sq, 128, 576), np.uint16), q_start, flags)
    assert mf == (flags == 0)
    for b in range(2):
        for i in range(Sq):
            vis = min(int(lens[b]), int(q_start[b]) + i + 1)
            assert np.all(np.rint(np.exp(lse[b, i].astype(np.float64))) == vis), (b, i, vis)
    # spike
    q = np.zeros((2, Sq, 128, 576), np.float32)
    q[..., 0] = 16.0
    z, lse, _ = _prefill_direct(inp, gen.bf16_bits(q), q_start, flags)
    spike = gen.bf16_from_bits(rows[0][T, :512]).astype(np.float64)
    for i in range(Sq):
        p = int(q_start[0]) + i
        if p >= T:
            assert np.max(np.abs(z[0, i] - spike[None])) <= 1e-5, i
            assert np.allclose(lse[0, i], 128.0 * np.log(2.0), atol=1e-4), i
        else:
            assert np.all(np.rint(np.exp(lse[0, i].astype(np.float64))) == p + 1), i
    for i in range(Sq):
        assert np.all(np.rint(np.exp(lse[1, i].astype(np.float64))) == min(97, 57 + i + 1))
