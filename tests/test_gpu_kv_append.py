"""GPU parity of the cache write (mla_kv_append) against the fp64 oracle.

The oracle composes its own steps: c = RMSNorm(h . W_DKV) with unit gain and eps 1e-6, and
k^R = RoPE_pos(h . W_KR) on interleaved pairs ([molayo] formal definition and implementation
code; [huny] section 2, decoupled RoPE; [ase] Fig. 1 note on the norm after the latent).  The
library rounds the finished row to bf16 once, so every stored value must satisfy

    |gpu - oracle| <= 2^-8 |oracle| + 1e-4 * RMS(oracle)

(half a bf16 ulp relative, plus slack for fp32 accumulation over d_model products).  Rows that
are not written must keep their bits.  The MFMA path (bf16, d_c 512, d_r 64, d_model % 256 == 0)
and the generic kernel are both checked on the same inputs.
"""

import math

import numpy as np
import pytest
import torch

import mla_latent_kv_31_amd as M
import oracle.mla_oracle as O
from mla_latent_kv_31_amd import runner
from mla_workloads import gen
from parity import note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 1e-6


def _oracle_rows(t, w, rms_eps):
    h = gen.as_f64(t["h"], t["dtype"])
    c = O.kv_latent(h, gen.as_f64(t["w_dkv"], t["dtype"]))
    if rms_eps > 0:
        c = O.rms_normalize(c, rms_eps)
    kr = O.rope_key(h, gen.as_f64(t["w_kr"], t["dtype"]), t["positions"], w.rope_base)
    return O.cache_rows(c, kr)


def _run(t, w, rms_eps, generic=False):
    d = runner.dims_for(w, M.MLA_FLAG_FORCE_GENERIC if generic else 0)
    dev = lambda a: runner.to_device(a, DEV)  # noqa: E731  (uint16 arrays are bf16 bit patterns)
    pool = dev(t["pool"])
    table = dev(t["page_table"])
    lens = dev(np.zeros(w.batch, np.int32))  # the cache write reads no length
    c = M.cache(pool, table, lens)
    R = t["h"].shape[0]
    ws_bytes = M.mla_kv_append_workspace_bytes(d, w.d_model, R)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=DEV)
    M.mla_kv_append(d, c, w.d_model, dev(t["h"]), dev(t["w_dkv"]), dev(t["w_kr"]), dev(t["seq_ids"]),
                    dev(t["positions"]), R, rms_eps, ws, ws_bytes)
    torch.cuda.synchronize()
    host = pool.view(torch.int16).cpu().numpy().view(np.uint16) if pool.dtype == torch.bfloat16 else pool.cpu().numpy()
    return host, ws_bytes


def _check(t, w, pool_after, rms_eps, what):
    ps = w.page_size
    pages = t["page_table"][t["seq_ids"], t["positions"] // ps]
    slots = t["positions"] % ps
    got = gen.as_f64(pool_after[pages, slots], t["dtype"])
    ref = _oracle_rows(t, w, rms_eps)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * rms
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} values out of bound; worst excess "
                           f"{float(np.max(np.abs(got - ref) - bound)):.3e} (rms {rms:.3e})")
    untouched = np.ones(pool_after.shape[:2], dtype=bool)
    untouched[pages, slots] = False
    assert np.array_equal(pool_after[untouched].view(np.uint16), t["pool"][untouched].view(np.uint16)), \
        f"{what}: rows that were not written changed"


@pytest.mark.parametrize("name", ["v3_kv_append_b64", "v3_kv_append_prefill_b2"])
def test_kv_append_v3(name):
    w = gen.WORKLOADS[name]
    t = gen.make_kv_append_inputs(w)
    note(f"kv_append {name} rows={t['h'].shape[0]} d_model={w.d_model}")
    pool, ws = _run(t, w, EPS)
    assert ws > 0, "the V3 shape must take the MFMA path"
    _check(t, w, pool, EPS, name)


@pytest.mark.parametrize("rows,d_model", [(1, 256), (37, 768), (65, 4096), (130, 1024), (513, 256), (600, 768),
                                          (1000, 4096)])
def test_kv_append_edges(rows, d_model):
    """Row counts off the 64-row tile, single-chunk and odd-chunk-count hidden widths; from 512 rows
    on the tiled product (64 x 64 tiles, 64-k chunks), with ragged last tiles."""
    base = gen.WORKLOADS["v3_kv_append_b64"]
    w = gen.Workload(name="kv_edge", seed=11 + rows, kind="kv_append", batch=base.batch, ctx_range=base.ctx_range,
                     q_len=max(3, -(-rows // base.batch)), random_pages=True, d_model=d_model)
    t = gen.make_kv_append_inputs(w, rows=rows)
    note(f"kv_append edge rows={rows} d_model={d_model}")
    pool, _ = _run(t, w, EPS)
    _check(t, w, pool, EPS, f"rows {rows} d_model {d_model}")


def test_kv_append_generic_and_unnormalised():
    """The generic kernel on the V3 inputs, and both paths without the norm (rms_eps = 0)."""
    w = gen.WORKLOADS["v3_kv_append_b64"]
    t = gen.make_kv_append_inputs(w, rows=24)
    note("kv_append generic path, rms_eps 1e-6 and 0; MFMA path rms_eps 0")
    pool, ws = _run(t, w, EPS, generic=True)
    assert ws == 0
    _check(t, w, pool, EPS, "generic")
    pool, _ = _run(t, w, 0.0, generic=True)
    _check(t, w, pool, 0.0, "generic, no norm")
    pool, _ = _run(t, w, 0.0)
    _check(t, w, pool, 0.0, "mfma, no norm")
