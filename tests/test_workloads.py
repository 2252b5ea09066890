"""Seeded input generators: storage-format rounding, lengths and paged layout (CPU only)."""

import numpy as np
import torch

from mla_workloads import gen


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0 ** r.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.3895314e38, 1e-40], np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = gen.bf16_bits(x)
    assert np.array_equal(got, ref)
    assert np.array_equal(gen.bf16_from_bits(got), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert np.isnan(gen.bf16_from_bits(gen.bf16_bits(np.array([np.nan], np.float32)))).all()


def test_decode_inputs_layout_and_determinism():
    w = gen.WORKLOADS["v3_b1_ctx4k"]
    a = gen.make_decode_inputs(w)
    b = gen.make_decode_inputs(w)
    for k in ("q_c", "q_r", "w_uk", "w_uv", "pool", "page_table", "lens"):
        assert np.array_equal(a[k], b[k]), k
    assert a["pool"].dtype == np.uint16 and a["pool"].shape[1:] == (64, 576)
    assert np.array_equal(a["page_table"][0], np.arange(64))
    assert a["lens"].tolist() == [4096] and a["pos"].tolist() == [4095]
    lat = gen.bf16_from_bits(a["pool"][:64].reshape(-1, 576)[:, :512]).astype(np.float64)
    rms = np.sqrt(np.mean(lat ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) < 1e-2)


def test_ragged_lengths_and_random_pages():
    w = gen.WORKLOADS["v3_b64_ragged_paged"]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lens = gen.draw_lengths(w, rng)
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 32768
    small = gen.Workload(name="t", seed=9, kind="decode", batch=5, n_heads=4, d_c=8, d_r=2, d_k=4, d_v=4,
                         ctx_range=(1, 200), random_pages=True)
    x = gen.make_decode_inputs(small, fill="nan")
    used = x["page_table"][x["page_table"] >= 0]
    assert len(set(used.tolist())) == used.size  # no page is shared
    for b, L in enumerate(x["lens"]):
        npg = -(-int(L) // 64)
        assert np.all(x["page_table"][b, :npg] >= 0) and np.all(x["page_table"][b, npg:] == -1)
        tail = x["pool"][x["page_table"][b, npg - 1], int(L) - (npg - 1) * 64:]
        assert np.all(np.isnan(gen.bf16_from_bits(tail)))


def test_prefill_and_toy_shapes():
    p = gen.make_prefill_inputs(gen.Workload(name="p", seed=5, kind="prefill", batch=2, n_heads=4, d_c=8, d_r=2,
                                             d_k=4, d_v=4, ctx=70, q_len=9))
    assert p["q_c"].shape == (2, 9, 4, 4) and p["lens"].tolist() == [79, 79] and p["q_start"].tolist() == [70, 70]
    t = gen.make_toy_inputs()
    assert t["h"].shape == (4, 8) and t["w_uk"].shape == (2, 3, 2) and t["w_kr"].shape == (8, 2)
    assert t["h"].dtype == np.float32
