"""Cache pools past 4 GiB on the GPU.

The pages put the latent cache in pages reached through a page table ([molayo] serving notes)
and bound neither the pool nor a page id. One MI355X holds 288 GB, so a serving pool easily
passes 2^31 and 2^32 bytes, and every kernel forms row addresses in 64 bits. Each test places
one logical cache in two physical pools: a compact one, and one where the even page ids sit
across the 2^31-byte mark and the odd ones across the 2^32-byte mark. Every other page of the
large pool holds NaN. The outputs must be bitwise identical, which is the page-permutation rule
of the exactness tests carried past the 32-bit offsets. A read of a wrong page, or a wrapped
offset, would bring in NaN or other rows.
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
BF16_NAN = 0x7FC0  # the quiet NaN torch.full writes in bf16
F8_NAN = 0xFF   # E4M3 NaN code; as a scale byte pattern it is NaN too


def _placement(n_pages: int, page_bytes: int) -> np.ndarray:
    """New physical id of each compact page: even ids straddle 2^31 bytes, odd ids 2^32."""
    lo = (1 << 31) // page_bytes - 2
    hi = (1 << 32) // page_bytes - 2
    assert lo + n_pages < hi
    ids = np.arange(n_pages)
    new = np.where(ids % 2 == 0, lo + ids, hi + ids)
    assert int(new.max() + 1) * page_bytes > (1 << 32) + page_bytes, "the pool must pass 4 GiB"
    return new.astype(np.int64)


def _remap_table(table: np.ndarray, new: np.ndarray) -> np.ndarray:
    out = table.copy()
    m = table >= 0
    out[m] = new[table[m]].astype(np.int32)
    return out


def _large_pool(compact: torch.Tensor, new: np.ndarray, fill) -> torch.Tensor:
    big = torch.full((int(new.max()) + 1,) + tuple(compact.shape[1:]), fill, dtype=compact.dtype, device=DEV)
    big[torch.from_numpy(new).to(DEV)] = compact
    return big


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().view(np.uint32) if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _decode_outputs(inp, split, n_units, flags=0):
    st = runner.DecodeStep(inp, split, DEV, flags=flags, n_units=n_units)
    st.run()
    torch.cuda.synchronize()
    lse_part = st.lse_part.cpu().numpy()
    o_part = st.o_part.cpu().numpy().copy()
    o_part[~np.isfinite(lse_part)] = 0.0  # an empty chunk's partial row is left untouched
    res = [_bits(st.z), _bits(st.lse), _bits(st.out), lse_part.view(np.uint32), o_part.view(np.uint32)]
    del st
    return res


def _decode_inputs():
    lens = np.array([700, 2000, 65, 3000, 1], np.int32)
    w = gen.Workload(name="large_pool", seed=57, kind="decode", batch=len(lens), random_pages=True, **V3)
    return gen.make_decode_inputs(w, lens=lens, random_pages=True)


@pytest.mark.parametrize("split,n_units", [(512, None), (0, 256)], ids=["fixed_512", "balanced_256"])
def test_decode_pool_past_4gib(split, n_units):
    inp = _decode_inputs()
    compact = runner.to_device(inp["pool"], DEV)
    new = _placement(compact.shape[0], compact[0].numel() * 2)
    note(f"decode pool past 4 GiB split={split} units={n_units} pages={compact.shape[0]} -> {int(new.max()) + 1}")
    ref = _decode_outputs(inp, split, n_units)
    big = _large_pool(compact, new, float("nan"))
    got = _decode_outputs(dict(inp, pool=big, page_table=_remap_table(inp["page_table"], new)), split, n_units)
    for name, a, b in zip(("z", "lse", "out", "lse_part", "o_part"), ref, got):
        assert np.array_equal(a, b), f"{name} differs when the pool passes 4 GiB"
    del big, compact
    _free()


def test_fp8_decode_pool_past_4gib():
    inp = _decode_inputs()
    d = runner.dims_for(inp["workload"])
    src = runner.to_device(inp["pool"], DEV)
    P, ps, _ = src.shape
    compact = torch.empty((P, ps, M.MLA_FP8_ROW_BYTES), dtype=torch.uint8, device=DEV)
    M.mla_quantize_rows_fp8(d, src, P * ps, compact)
    torch.cuda.synchronize()
    del src
    new = _placement(P, ps * M.MLA_FP8_ROW_BYTES)
    note(f"fp8 decode pool past 4 GiB pages={P} -> {int(new.max()) + 1}")
    F8 = M.MLA_FLAG_CACHE_FP8
    ref = _decode_outputs(dict(inp, pool=compact), 0, 256, flags=F8)
    big = _large_pool(compact, new, F8_NAN)
    got = _decode_outputs(dict(inp, pool=big, page_table=_remap_table(inp["page_table"], new)), 0, 256, flags=F8)
    for name, a, b in zip(("z", "lse", "out", "lse_part", "o_part"), ref, got):
        assert np.array_equal(a, b), f"FP8 {name} differs when the pool passes 4 GiB"
    del big, compact
    _free()


def test_prefill_pool_past_4gib():
    """Absorbed (mla_prefill_chunk) and unabsorbed (mla_decompress_kv, mla_prefill_unabsorbed)."""
    w = gen.Workload(name="large_pool_prefill", seed=58, kind="prefill", batch=3, ctx_range=(1, 300), q_len=40,
                     random_pages=True)
    inp = gen.make_prefill_inputs(w)
    compact = runner.to_device(inp["pool"], DEV)
    new = _placement(compact.shape[0], compact[0].numel() * 2)
    note(f"prefill pool past 4 GiB lens={inp['lens'].tolist()} pages={compact.shape[0]} -> {int(new.max()) + 1}")
    big = _large_pool(compact, new, float("nan"))
    moved = dict(inp, pool=big, page_table=_remap_table(inp["page_table"], new))
    for cls in (runner.PrefillStep, runner.PrefillUnabsorbedStep):
        outs = []
        for src in (inp, moved):
            st = cls(src, DEV)
            st.run()
            torch.cuda.synchronize()
            outs.append((_bits(st.out), _bits(st.lse)))
            del st
        assert np.array_equal(outs[0][0], outs[1][0]), f"{cls.__name__}: out differs when the pool passes 4 GiB"
        assert np.array_equal(outs[0][1], outs[1][1]), f"{cls.__name__}: lse differs when the pool passes 4 GiB"
    del big, compact, moved
    _free()


def test_kv_append_pool_past_4gib():
    """The cache write lands in the same rows of the moved pages and leaves every other bit alone."""
    base = gen.WORKLOADS["v3_kv_append_b64"]
    w = gen.Workload(name="large_pool_kv", seed=59, kind="kv_append", batch=base.batch, ctx_range=base.ctx_range,
                     q_len=3, random_pages=True, d_model=base.d_model)
    t = gen.make_kv_append_inputs(w, rows=37)
    d = runner.dims_for(w)
    dev = lambda a: runner.to_device(a, DEV)  # noqa: E731
    compact = dev(t["pool"])
    new = _placement(compact.shape[0], compact[0].numel() * 2)
    note(f"kv_append pool past 4 GiB pages={compact.shape[0]} -> {int(new.max()) + 1}")
    big = _large_pool(compact, new, float("nan"))
    R = t["h"].shape[0]
    ws_bytes = M.mla_kv_append_workspace_bytes(d, w.d_model, R)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=DEV)
    lens = dev(np.zeros(w.batch, np.int32))  # the cache write reads no length; kept alive with the descriptor
    for pool, table in ((compact, t["page_table"]), (big, _remap_table(t["page_table"], new))):
        tbl = dev(table)
        c = M.cache(pool, tbl, lens)
        M.mla_kv_append(d, c, w.d_model, dev(t["h"]), dev(t["w_dkv"]), dev(t["w_kr"]), dev(t["seq_ids"]),
                        dev(t["positions"]), R, 1e-6, ws, ws_bytes)
        torch.cuda.synchronize()
    moved_back = big[torch.from_numpy(new).to(DEV)]
    assert torch.equal(moved_back.view(torch.int16), compact.view(torch.int16)), \
        "cache write differs when the pool passes 4 GiB"
    big[torch.from_numpy(new).to(DEV)] = float("nan")  # what is left must be the untouched fill
    assert bool(torch.all(big.view(torch.int16) == BF16_NAN)), "the cache write touched a page it does not own"
    del big, compact, moved_back
    _free()
