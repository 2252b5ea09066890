"""GPU parity of the precomposed-weight path (row N2) against the fp64 oracle.

* mla_precompose_query / mla_precompose_out: each stored weight is one bf16 rounding of a float32
  sum of d_k (d_v) products, so every value must satisfy |gpu - oracle| <= 2^-8 |oracle| +
  1e-4 * RMS(oracle) (half a bf16 ulp, plus slack for the float32 sum); the copied W_QR columns
  must be bit-identical.  Checked on sampled heads of the V3-size weights.
* mla_absorb_query_precomposed: the precomposed weight is an input here, made by the oracle and
  stored in bf16 like every other weight; q_hat is rounded to IEEE binary16 once, so every value
  must satisfy |gpu - oracle| <= 2^-11 |oracle| + 1e-4 * RMS(oracle) (half a binary16 ulp, plus
  slack for the float32 sum and the binary16 subnormal range).
* mla_out_proj_fused and mla_output_projection: float32 outputs from float32 z (o) carried as bf16
  hi + lo parts; max |gpu - oracle| <= 1e-4 * RMS(oracle).
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
W = gen.WORKLOADS["v3_precomposed_b64"]


def _dims():
    return runner.dims_for(W)


def _dev(a):
    return runner.to_device(a, DEV)


def _bf16_bound(got, ref, what):
    rms = math.sqrt(float(np.mean(ref ** 2)))
    excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-4 * rms)
    assert excess.max() <= 0, f"{what}: worst excess {excess.max():.3e} (rms {rms:.3e})"


def _f16_bound(got, ref, what):
    rms = math.sqrt(float(np.mean(ref ** 2)))
    excess = np.abs(got - ref) - (2.0 ** -11 * np.abs(ref) + 1e-4 * rms)
    assert excess.max() <= 0, f"{what}: worst excess {excess.max():.3e} (rms {rms:.3e})"


@pytest.fixture(scope="module")
def inp():
    return gen.make_precomposed_inputs(W, rows=100)


def test_precompose_query(inp):
    note("precompose query weight")
    H, dq, dc, dr = W.n_heads, W.d_cq, W.d_c, W.d_r
    w_qcat = torch.empty((dq, H, dc + dr), dtype=torch.bfloat16, device=DEV)
    M.mla_precompose_query(_dims(), dq, _dev(inp["w_uq"]), _dev(inp["w_uk"]), _dev(inp["w_qr"]), w_qcat)
    torch.cuda.synchronize()
    got = w_qcat.view(torch.int16).cpu().numpy().view(np.uint16)
    for h in (0, 45, 127):
        ref = O.precompose_query_weights(gen.as_f64(inp["w_uq"][h:h + 1], "bf16"),
                                         gen.as_f64(inp["w_uk"][h:h + 1], "bf16"))[0]
        _bf16_bound(gen.as_f64(got[:, h, :dc], "bf16"), ref, f"head {h} absorbed weight")
        assert np.array_equal(got[:, h, dc:], inp["w_qr"][h]), f"head {h}: rotary columns"


def test_precompose_out(inp):
    note("precompose output weight")
    H, dc, dm, dv = W.n_heads, W.d_c, W.d_model, W.d_v
    w_uvo = torch.empty((H, dc, dm), dtype=torch.bfloat16, device=DEV)
    M.mla_precompose_out(_dims(), dm, _dev(inp["w_uv"]), _dev(inp["w_o"]), w_uvo)
    torch.cuda.synchronize()
    got = w_uvo.view(torch.int16).cpu().numpy().view(np.uint16)
    for h in (0, 77, 127):
        ref = O.precompose_out_weights(gen.as_f64(inp["w_uv"][h:h + 1], "bf16"),
                                       gen.as_f64(inp["w_o"][h * dv:(h + 1) * dv], "bf16"))[0]
        _bf16_bound(gen.as_f64(got[h], "bf16"), ref, f"head {h} fused output weight")


@pytest.fixture(scope="module")
def oracle_weights(inp):
    """The precomposed weights as the oracle forms them, stored in bf16 (inputs of the products)."""
    wa = O.precompose_query_weights(gen.as_f64(inp["w_uq"], "bf16"), gen.as_f64(inp["w_uk"], "bf16"))
    w_qcat = np.concatenate([gen.bf16_bits(wa.astype(np.float32)), inp["w_qr"]], axis=2).transpose(1, 0, 2)
    w_uvo = gen.bf16_bits(O.precompose_out_weights(gen.as_f64(inp["w_uv"], "bf16"),
                                                   gen.as_f64(inp["w_o"], "bf16")).astype(np.float32))
    return np.ascontiguousarray(w_qcat), w_uvo


@pytest.mark.parametrize("rows", [1, 64, 100])
def test_absorb_query_precomposed(inp, oracle_weights, rows):
    w_qcat, _ = oracle_weights
    H, dq, dc, dr = W.n_heads, W.d_cq, W.d_c, W.d_r
    note(f"absorb precomposed rows={rows}")
    d = _dims()
    ws_bytes = M.mla_absorb_query_precomposed_workspace_bytes(d, dq, rows)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=DEV)
    q_hat = torch.empty((rows, H, dc + dr), dtype=torch.float16, device=DEV)
    c_q, pos = _dev(inp["c_q"][:rows]), _dev(inp["pos"][:rows])
    wq = _dev(w_qcat)
    M.mla_absorb_query_precomposed(d, dq, c_q, wq, pos, rows, q_hat, ws, ws_bytes)
    torch.cuda.synchronize()
    got = q_hat.float().cpu().numpy().astype(np.float64)
    wa = gen.as_f64(w_qcat[:, :, :dc], "bf16").transpose(1, 0, 2)    # [H, d_cq, d_c]
    wr = gen.as_f64(w_qcat[:, :, dc:], "bf16").transpose(1, 0, 2)    # [H, d_cq, d_r]
    scale = 1.0 / math.sqrt(W.d_k + dr) / math.log(2.0)
    sample = range(rows) if rows <= 64 else sorted({0, 31, 64, 65, rows - 1})
    for r in sample:
        ref = O.absorbed_query_precomposed(gen.as_f64(inp["c_q"][r], "bf16"), wa, wr, int(inp["pos"][r])) * scale
        _f16_bound(got[r], ref, f"q_hat row {r}")


@pytest.mark.parametrize("rows", [1, 64, 100])
def test_out_proj_fused(inp, oracle_weights, rows):
    _, w_uvo = oracle_weights
    note(f"out_proj fused rows={rows}")
    d = _dims()
    ws_bytes = M.mla_out_proj_fused_workspace_bytes(d, W.d_model, rows)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=DEV)
    out = torch.full((rows, W.d_model), float("nan"), device=DEV)
    z, wo = _dev(inp["z"][:rows]), _dev(w_uvo)
    M.mla_out_proj_fused(d, W.d_model, z, wo, rows, out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = O.out_proj_fused(inp["z"][:rows].astype(np.float64), gen.as_f64(w_uvo, "bf16"))
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    assert err <= 1e-4 * rms, f"fused output rows {rows}: max err {err:.3e} > 1e-4 * rms {rms:.3e}"


@pytest.mark.parametrize("rows", [1, 100])
def test_output_projection(inp, rows):
    note(f"output projection rows={rows}")
    d = _dims()
    ws_bytes = M.mla_output_projection_workspace_bytes(d, W.d_model, rows)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=DEV)
    out = torch.full((rows, W.d_model), float("nan"), device=DEV)
    o, wo = _dev(inp["o"][:rows]), _dev(inp["w_o"])
    M.mla_output_projection(d, W.d_model, o, wo, rows, out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = O.output_projection(inp["o"][:rows].astype(np.float64), gen.as_f64(inp["w_o"], "bf16"))
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    assert err <= 1e-4 * rms, f"output projection rows {rows}: max err {err:.3e} > 1e-4 * rms {rms:.3e}"
