"""GPU parity of the two per-head projections on their own, at the row counts the decode and
prefill steps use and at ragged counts around the 32- and 64-row workgroup tiles.

  * mla_absorb_query ([ase] Fig. 3 equation): q_hat = [q_C . W_UK[h]^T | RoPE_pos(q_R)] times
    sm_scale * log2(e), rounded to IEEE binary16 once, so every value must satisfy
        |gpu - oracle| <= 2^-11 |oracle| + 2^-24 + 1e-5 * RMS(oracle)
    (half a binary16 ulp, the binary16 subnormal spacing, and slack for the fp32 accumulation over
    128 products).
  * mla_out_proj ([ase] Fig. 4 equation): out = z . W_UV[h] with float32 z and output, against
    oracle.absorbed_output.  z enters the MFMAs as a bf16 hi + lo pair (about 16 significant
    bits), so the float32 bound applies:
        max |gpu - oracle| <= 1e-4 * RMS(oracle).
Inputs: q_C, q_R, z ~ N(0,1); W_UK, W_UV ~ N(0,1)/sqrt(512), stored bf16; positions uniform on
[0, 131072).
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
H, DC, DR, DK, DV = 128, 512, 64, 128, 128


def _dims():
    return M.dims(n_heads=H, d_c=DC, d_r=DR, d_k=DK, d_v=DV, dtype=M.MLA_BF16)


@pytest.mark.parametrize("rows", [1, 33, 64, 128, 129, 1024])
def test_absorb_query_rows(rows):
    rng = np.random.Generator(np.random.PCG64(100 + rows))
    q_c = gen.bf16_bits(rng.standard_normal((rows, H, DK), dtype=np.float32))
    q_r = gen.bf16_bits(rng.standard_normal((rows, H, DR), dtype=np.float32))
    w_uk = gen.bf16_bits(rng.standard_normal((H, DC, DK), dtype=np.float32) / np.float32(math.sqrt(DC)))
    pos = rng.integers(0, 131072, size=rows, dtype=np.int64).astype(np.int32)
    note(f"absorb rows={rows}")
    d = _dims()
    q_hat = torch.empty((rows, H, DC + DR), dtype=torch.float16, device=DEV)
    M.mla_absorb_query(d, runner.to_device(q_c, DEV), runner.to_device(q_r, DEV), runner.to_device(w_uk, DEV),
                       runner.to_device(pos, DEV), rows, q_hat)
    torch.cuda.synchronize()
    # every row up to 129; a seeded sample of 96 (first and last included) of the 1,024
    sample = np.arange(rows) if rows <= 129 else np.unique(np.concatenate(
        [[0, rows - 1], rng.choice(rows, 94, replace=False)]))
    got = q_hat.float().cpu().numpy().astype(np.float64)[sample]
    scale = 1.0 / math.sqrt(DK + DR) / math.log(2.0)
    wk = gen.as_f64(w_uk, "bf16")
    ref = np.stack([O.absorbed_query(gen.as_f64(q_c[r], "bf16"), gen.as_f64(q_r[r], "bf16"), int(pos[r]), wk)
                    for r in sample]) * scale
    rms = math.sqrt(float(np.mean(ref ** 2)))
    excess = np.abs(got - ref) - (2.0 ** -11 * np.abs(ref) + 2.0 ** -24 + 1e-5 * rms)
    assert excess.max() <= 0, f"absorb rows {rows}: worst excess {excess.max():.3e} (rms {rms:.3e})"


@pytest.mark.parametrize("rows", [1, 31, 64, 100, 128, 129, 1024])
def test_out_proj_rows(rows):
    rng = np.random.Generator(np.random.PCG64(200 + rows))
    z = rng.standard_normal((rows, H, DC), dtype=np.float32)
    w_uv = gen.bf16_bits(rng.standard_normal((H, DC, DV), dtype=np.float32) / np.float32(math.sqrt(DC)))
    note(f"out_proj rows={rows}")
    out = torch.full((rows, H, DV), float("nan"), device=DEV)
    M.mla_out_proj(_dims(), runner.to_device(z, DEV), runner.to_device(w_uv, DEV), rows, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = O.absorbed_output(z.astype(np.float64), gen.as_f64(w_uv, "bf16"))
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    assert err <= 1e-4 * rms, f"out_proj rows {rows}: max err {err:.3e} > 1e-4 * rms {rms:.3e}"
