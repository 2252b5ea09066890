"""HIP graph capture of whole steps (runner.CapturedStep) on the GPU.

A captured step replays the same kernels on the same buffers, so every replay must give results
bitwise identical to an eager run on the same inputs. Each graph is replayed several times.
Between replays the program does its own eager work on other buffers and synchronises, and the
query tensors are rewritten in place (A, then B, then A). A replay must read its inputs again,
never reuse an earlier result. The outputs are filled with NaN before every replay, so each one
must write them in full.

Covered: the balanced, fixed-split and FP8-cache decode steps (and the balanced and fixed steps
with the merge and value projection fused), the absorbed and unabsorbed prefill calls, and the
multi-token verify step.
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
REPLAYS = ("A", "B", "A", "B")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def _check_replays(make, inp_a, inp_b, outs):
    """make(inp) -> step object; outs: names of the step's output tensors."""
    ref = {}
    for tag, inp in (("A", inp_a), ("B", inp_b)):
        st = make(inp)
        st.run()
        torch.cuda.synchronize()
        ref[tag] = [_bits(getattr(st, n)) for n in outs]
        del st
    st = make(inp_a)
    g = runner.CapturedStep(st)
    other = make(inp_b)  # eager work of the program between replays
    q = {tag: (runner.to_device(i["q_c"], DEV), runner.to_device(i["q_r"], DEV))
         for tag, i in (("A", inp_a), ("B", inp_b))}
    for k, tag in enumerate(REPLAYS):
        st.q_c.copy_(q[tag][0])
        st.q_r.copy_(q[tag][1])
        for n in outs:
            getattr(st, n).fill_(float("nan"))
        g.run()
        torch.cuda.synchronize()
        for n, want in zip(outs, ref[tag]):
            assert np.array_equal(_bits(getattr(st, n)), want), f"replay {k} (inputs {tag}): {n} differs from eager"
        other.run()
        torch.cuda.synchronize()


def _decode_inputs(seed):
    lens = np.array([700, 2000, 65, 3000, 1], np.int32)
    w = gen.Workload(name="graph", seed=seed, kind="decode", batch=len(lens), random_pages=True, **V3)
    return gen.make_decode_inputs(w, lens=lens, random_pages=True)


@pytest.mark.parametrize("mode", ["balanced", "fixed", "fp8"])
def test_decode_step_graph(mode):
    inp_a = _decode_inputs(61)
    q_b = _decode_inputs(62)
    flags = 0
    if mode == "fp8":
        src = runner.to_device(inp_a["pool"], DEV)
        P, ps, _ = src.shape
        pool8 = torch.empty((P, ps, M.MLA_FP8_ROW_BYTES), dtype=torch.uint8, device=DEV)
        M.mla_quantize_rows_fp8(runner.dims_for(inp_a["workload"]), src, P * ps, pool8)
        torch.cuda.synchronize()
        inp_a = dict(inp_a, pool=pool8)
        flags = M.MLA_FLAG_CACHE_FP8
    inp_b = dict(inp_a, q_c=q_b["q_c"], q_r=q_b["q_r"])
    note(f"graph replays, decode {mode}")
    if mode == "fixed":
        make = lambda i: runner.DecodeStep(i, 512, DEV, flags=flags)  # noqa: E731
    else:
        make = lambda i: runner.DecodeStep(i, 0, DEV, flags=flags, n_units=256)  # noqa: E731
    _check_replays(make, inp_a, inp_b, ("out", "z", "lse"))


@pytest.mark.parametrize("mode", ["balanced", "fixed"])
def test_decode_step_graph_fused(mode):
    """The step whose merge and value projection are one call (mla_combine_out_proj*); z is not
    written on this path, so out and lse are compared."""
    inp_a = _decode_inputs(65)
    q_b = _decode_inputs(66)
    inp_b = dict(inp_a, q_c=q_b["q_c"], q_r=q_b["q_r"])
    note(f"graph replays, fused decode {mode}")
    if mode == "fixed":
        make = lambda i: runner.DecodeStep(i, 512, DEV, fused=True)  # noqa: E731
    else:
        make = lambda i: runner.DecodeStep(i, 0, DEV, n_units=256, fused=True)  # noqa: E731
    assert make(inp_a).fused
    _check_replays(make, inp_a, inp_b, ("out", "lse"))


@pytest.mark.parametrize("kind", ["prefill", "prefill_unabsorbed", "verify"])
def test_prefill_and_verify_graph(kind):
    def inputs(seed):
        w = gen.Workload(name="graph_prefill", seed=seed, kind="prefill", batch=3, ctx_range=(1, 300), q_len=24,
                         random_pages=True)
        return gen.make_prefill_inputs(w)

    inp_a = inputs(63)
    q_b = inputs(64)
    inp_b = dict(inp_a, q_c=q_b["q_c"], q_r=q_b["q_r"])
    note(f"graph replays, {kind}")
    make = {"prefill": lambda i: runner.PrefillStep(i, DEV),
            "prefill_unabsorbed": lambda i: runner.PrefillUnabsorbedStep(i, DEV),
            "verify": lambda i: runner.VerifyStep(i, DEV, n_units=16)}[kind]
    _check_replays(make, inp_a, inp_b, ("out", "lse"))
