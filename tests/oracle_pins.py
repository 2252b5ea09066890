"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each pin raises AssertionError on failure.  They are run directly by
test_oracle_pins.py and, against deliberately broken copies of oracle
functions, by test_oracle_mutations.py (every planted mistake must trip at
least one pin).  None of them re-types the oracle's own formula: they use
values printed on the pages (tests/golden), closed forms, textbook special
cases, a library routine (torch's scaled_dot_product_attention on the CPU in
float64), a complex-number form of the rotation, and brute-force identities.
"""

from __future__ import annotations

import cmath
import json
import math
import os

import numpy as np
import torch

import oracle.mla_oracle as O
from mla_workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.all(np.isfinite(a) == np.isfinite(b)), f"{what}: finiteness differs"
    fin = np.isfinite(b)
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
    neg = ~fin
    if neg.any():
        assert np.array_equal(a[neg], b[neg]), f"{what}: non-finite entries differ"


def _rng(seed):
    return np.random.default_rng(seed)


def _rope_complex(x, pos, base):
    """Rotation written as complex multiplication: pair (x[2i], x[2i+1]) is x[2i] + i x[2i+1],
    multiplied by exp(i * pos * base^(-2i/d))."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    out = np.empty_like(x)
    flat = x.reshape(-1, d)
    of = out.reshape(-1, d)
    for r in range(flat.shape[0]):
        for i in range(d // 2):
            theta = pos * base ** (-(2.0 * i) / d)
            v = complex(flat[r, 2 * i], flat[r, 2 * i + 1]) * cmath.exp(1j * theta)
            of[r, 2 * i], of[r, 2 * i + 1] = v.real, v.imag
    return out


def _sdpa(q, k, v, scale, mask=None):
    """torch CPU float64 scaled-dot-product attention; q [n,d], k [L,d], v [L,dv]."""
    q = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))[None, None]
    k = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


def _random_case(seed, H=3, d_c=5, d_r=4, d_k=2, d_v=3, L=7):
    r = _rng(seed)
    return dict(q_c=r.standard_normal((H, d_k)), q_r=r.standard_normal((H, d_r)),
                cache=r.standard_normal((L, d_c + d_r)), w_uk=r.standard_normal((H, d_c, d_k)),
                w_uv=r.standard_normal((H, d_c, d_v)), d_c=d_c)


# ---------------------------------------------------------------- page values
def pin_score_example():
    """Worked score: content 4 + position 0.6 = 4.6, divided by sqrt(2+2) = 2."""
    g = _golden("ase_worked_examples.json")["score_example"]
    row = np.array([g["k_content"] + g["k_position"]], dtype=np.float64)
    eye = np.eye(2)[None]
    q_c = np.array([g["q_content"]], dtype=np.float64)
    q_r = np.array([g["q_position_rotated"]], dtype=np.float64)  # position 0: rotation is the identity
    r = O.attention(q_c, q_r, 0, row, eye, eye, d_c=2)
    expect = g["total"] / g["scale_divisor"]
    _close(r["s"][0, 0], expect, 1e-15, "scaled score")
    _close(r["lse"][0], expect, 1e-15, "lse of a single key")
    rc = O.attention(q_c, 0 * q_r, 0, row, eye, eye, d_c=2)
    _close(rc["s"][0, 0], g["content_dot"] / g["scale_divisor"], 1e-15, "content-only score")
    rp = O.attention(0 * q_c, q_r, 0, row, eye, eye, d_c=2)
    _close(rp["s"][0, 0], g["position_dot"] / g["scale_divisor"], 1e-15, "position-only score")


def pin_key_absorption():
    """c3 = [1,2,3], U_K keeps the first two entries: key [1,2], q [2,1] -> 4; q~ = [2,1,0].
    The scale stays 1/sqrt(d_k + d_r) = 1/2 even though the latent is 3 wide."""
    g = _golden("ase_worked_examples.json")["key_absorption"]
    w_uk = np.array([g["U_K"]], dtype=np.float64)
    q_c = np.array([g["q"]], dtype=np.float64)
    q_r = np.zeros((1, 2))
    qh = O.absorbed_query(q_c, q_r, 0, w_uk)
    _close(qh[0, :3], g["q_tilde"], 0.0, "absorbed query")
    row = np.array([g["c3"] + [0.0, 0.0]], dtype=np.float64)
    K, _ = O.decompress(row[:, :3], w_uk[0], w_uk[0])
    _close(K[0], g["content_key"], 0.0, "decompressed content key")
    r = O.attention(q_c, q_r, 0, row, w_uk, w_uk, d_c=3)
    _close(r["s"][0, 0], g["content_dot"] / g["scale_divisor_kept"], 1e-15, "score with 3-wide latent")
    ra = O.attention_absorbed(q_c, q_r, 0, row, w_uk, w_uk, d_c=3)
    _close(ra["s"][0, 0], g["content_dot"] / g["scale_divisor_kept"], 1e-15, "absorbed score")


def pin_value_absorption():
    """Latents and weights of the Fig. 4 table: a.V = [2.3, 1.3], z = [0.8, 1.3, 1.5], z.U_V = [2.3, 1.3].

    The weights are produced through the position path: with d_r = 2 the first (only) rotary pair
    turns at one radian per position, so the query [1, 0] at position 3 points along
    (cos 3, sin 3); giving key j the rotary key (ln w_j / scale) (cos 3, sin 3) makes its scaled
    score ln w_j, and the softmax returns w itself (the weights sum to one)."""
    g = _golden("ase_worked_examples.json")["value_absorption"]
    lat = np.array(g["latents"], dtype=np.float64)
    w = np.array(g["weights"], dtype=np.float64)
    u_v = np.array([g["U_V"]], dtype=np.float64)
    scale = 0.5
    direction = np.array([math.cos(3.0), math.sin(3.0)])
    kr = (np.log(w) / scale)[:, None] * direction[None]
    cache = np.concatenate([lat, kr], axis=1)
    q_c = np.zeros((1, 2))
    q_r = np.array([[1.0, 0.0]])
    r = O.attention(q_c, q_r, 3, cache, np.zeros((1, 3, 2)), u_v, d_c=3)
    _close(r["a"][0], w, 1e-15, "attention weights")
    _close(r["z"][0], g["z"], 1e-15, "weighted latent z")
    _close(r["o"][0], g["output"], 1e-15, "output a.V")
    _close(lat @ u_v[0], g["values"], 0.0, "decompressed values")
    ra = O.attention_absorbed(q_c, q_r, 3, cache, np.zeros((1, 3, 2)), u_v, d_c=3)
    _close(ra["o"][0], g["output"], 1e-15, "absorbed output z.U_V")


def pin_cache_accounting():
    g = _golden("cache_accounting.json")
    h = g["huny"]
    mla = O.mla_bytes_per_token(h["d_c"], h["d_r"], h["bytes_per_value"])
    mha = O.mha_bytes_per_token(h["n_heads"], h["d_k"], h["bytes_per_value"])
    gqa = O.gqa_bytes_per_token(h["gqa_kv_heads"], h["d_k"], h["bytes_per_value"])
    assert O.mla_values_per_token(h["d_c"], h["d_r"]) == h["mla_values_per_token"]
    assert (mla, mha, gqa) == (h["mla_bytes_per_token"], h["mha_bytes_per_token"], h["gqa_bytes_per_token"])
    s_mha, s_gqa = O.saving(mla, mha), O.saving(mla, gqa)
    assert s_mha == 0.982421875 and s_gqa == 0.71875
    # the table truncates to two decimals, the summary rounds to one
    assert math.floor(s_mha * 1e4) / 100 == h["table_saving_pct"]["vs_mha"]
    assert math.floor(s_gqa * 1e4) / 100 == h["table_saving_pct"]["vs_gqa"]
    assert round(s_mha * 100, 1) == h["summary_saving_pct"]["vs_mha"]
    assert round(s_gqa * 100, 1) == h["summary_saving_pct"]["vs_gqa"]
    for k, b in (("mha", mha), ("gqa", gqa), ("mla", mla)):
        assert round(O.whole_cache_gib(b, h["ctx_tokens"], h["layers"]), 2) == h["whole_cache_printed"][k]
    m = g["molayo"]
    assert O.compression_ratio(m["n_heads"], m["d_k"], m["d_c"]) == m["compression_ratio"]


# ---------------------------------------------------------------- rotation
def pin_rope_closed_forms():
    # position 0 is the identity; d_r = 2 turns by exactly pos radians (inverse frequency 1)
    x = _rng(1).standard_normal((5, 64))
    _close(O.rope(x, 0, 10000.0), x, 0.0, "rope at position 0")
    for p in (1, 3, 17, 4095):
        _close(O.rope(np.array([1.0, 0.0]), p, 10000.0), [math.cos(p), math.sin(p)], 1e-15, "d_r=2 rotation")
        _close(O.rope(np.array([0.0, 1.0]), p, 10000.0), [-math.sin(p), math.cos(p)], 1e-15, "d_r=2 rotation")


def pin_rope_complex_form():
    r = _rng(2)
    for d, base in ((64, 10000.0), (8, 10000.0), (6, 500.0)):
        x = r.standard_normal((3, d))
        for p in (0, 1, 7, 2047, 131071):
            _close(O.rope(x, p, base), _rope_complex(x, p, base), 1e-9 * max(1, p / 1000), f"rope d={d} p={p}")
    # per-row positions broadcast
    x = r.standard_normal((4, 64))
    pos = np.array([0, 5, 100, 4095])
    got = O.rope(x, pos, 10000.0)
    for i in range(4):
        _close(got[i], _rope_complex(x[i:i + 1], int(pos[i]), 10000.0)[0], 1e-10, "rope broadcast")


def pin_rope_relative():
    """RoPE_m(q) . RoPE_n(k) depends only on m - n, and the norm is preserved."""
    r = _rng(3)
    q, k = r.standard_normal(64), r.standard_normal(64)
    ref = O.rope(q, 10, 1e4) @ O.rope(k, 3, 1e4)
    for m in (7, 50, 1000):
        _close(O.rope(q, m + 7, 1e4) @ O.rope(k, m, 1e4), ref, 1e-9, "relative-distance property")
    _close(np.linalg.norm(O.rope(q, 12345, 1e4)), np.linalg.norm(q), 1e-12, "norm")


# ---------------------------------------------------------------- attention
def pin_sdpa_textbook():
    """d_c = d_k = d_v with identity up-projections and no position part -> plain scaled-dot-product
    attention over the latent rows with scale 1/sqrt(d_k + d_r)."""
    r = _rng(4)
    H, d, d_r, L = 3, 6, 4, 9
    q_c = r.standard_normal((H, d))
    C = r.standard_normal((L, d))
    cache = np.concatenate([C, np.zeros((L, d_r))], axis=1)
    eye = np.repeat(np.eye(d)[None], H, axis=0)
    res = O.attention(q_c, np.zeros((H, d_r)), L - 1, cache, eye, eye, d_c=d)
    ref = _sdpa(q_c, C, C, 1.0 / math.sqrt(d + d_r))
    _close(res["o"], ref, 1e-12, "o vs sdpa")
    _close(res["z"], ref, 1e-12, "z vs sdpa")


def pin_sdpa_general():
    """Full MLA head-by-head against the library routine: Q = [q_C | rotated q_R] (rotation in
    complex form), K = [C.W_UK[h] | k^R], V = C.W_UV[h]."""
    for seed, dims in ((5, dict()), (6, dict(H=2, d_c=8, d_r=2, d_k=3, d_v=5, L=4)),
                       (7, dict(H=4, d_c=16, d_r=6, d_k=8, d_v=8, L=33))):
        c = _random_case(seed, **dims)
        d_c = c["d_c"]
        L = c["cache"].shape[0]
        res = O.attention(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], d_c)
        d_k, d_r = c["q_c"].shape[1], c["q_r"].shape[1]
        C, kr = c["cache"][:, :d_c], c["cache"][:, d_c:]
        qr = _rope_complex(c["q_r"], L - 1, 10000.0)
        for h in range(c["q_c"].shape[0]):
            Q = np.concatenate([c["q_c"][h], qr[h]])[None]
            K = np.concatenate([C @ c["w_uk"][h], kr], axis=1)
            ref = _sdpa(Q, K, C @ c["w_uv"][h], 1.0 / math.sqrt(d_k + d_r))[0]
            _close(res["o"][h], ref, 1e-12, f"o head {h} seed {seed}")


def pin_prefill_causal():
    """Query i at q_start + i reads keys 0..q_start+i: library routine with an explicit mask, and
    the decode definition on a truncated cache."""
    c = _random_case(8, H=2, d_c=6, d_r=4, d_k=3, d_v=2, L=12)
    r = _rng(9)
    Sq, q_start, d_c = 5, 7, 6
    q_c = r.standard_normal((Sq, 2, 3))
    q_r = r.standard_normal((Sq, 2, 4))
    res = O.prefill(q_c, q_r, q_start, c["cache"], c["w_uk"], c["w_uv"], d_c)
    C, kr = c["cache"][:, :d_c], c["cache"][:, d_c:]
    L = C.shape[0]
    for h in range(2):
        Q = np.concatenate([q_c[:, h], np.stack([_rope_complex(q_r[i, h:h + 1], q_start + i, 1e4)[0]
                                                 for i in range(Sq)])], axis=1)
        K = np.concatenate([C @ c["w_uk"][h], kr], axis=1)
        mask = np.arange(L)[None, :] <= (q_start + np.arange(Sq))[:, None]
        ref = _sdpa(Q, K, C @ c["w_uv"][h], 1.0 / math.sqrt(3 + 4), mask=mask)
        _close(res["o"][:, h], ref, 1e-12, f"prefill head {h}")
    for i in range(Sq):
        d = O.attention(q_c[i], q_r[i], q_start + i, c["cache"][:q_start + i + 1], c["w_uk"], c["w_uv"], d_c)
        _close(res["z"][i], d["z"], 1e-13, f"prefill row {i} vs truncated decode")


def pin_loops_twin():
    for seed, dims in ((10, dict()), (11, dict(H=2, d_c=3, d_r=2, d_k=2, d_v=2, L=4)),
                       (12, dict(H=1, d_c=4, d_r=0, d_k=4, d_v=1, L=1)), (13, dict(H=2, d_c=7, d_r=6, d_k=3, d_v=4, L=11))):
        c = _random_case(seed, **dims)
        L = c["cache"].shape[0]
        for q_pos in (L - 1, L // 2):
            a = O.attention(c["q_c"], c["q_r"], q_pos, c["cache"], c["w_uk"], c["w_uv"], c["d_c"])
            b = O.attention_loops(c["q_c"], c["q_r"], q_pos, c["cache"], c["w_uk"], c["w_uv"], c["d_c"])
            for k in ("o", "z", "lse"):
                _close(a[k], b[k], 1e-12, f"loops twin {k} seed {seed}")


def pin_absorbed_equals_decompressed():
    for seed in range(14, 20):
        r = _rng(seed)
        dims = dict(H=int(r.integers(1, 5)), d_c=int(r.integers(2, 20)), d_r=2 * int(r.integers(0, 5)),
                    d_k=int(r.integers(1, 9)), d_v=int(r.integers(1, 9)), L=int(r.integers(1, 40)))
        c = _random_case(seed, **dims)
        L = c["cache"].shape[0]
        a = O.attention(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"])
        b = O.attention_absorbed(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"])
        for k in ("o", "z", "lse"):
            scale = max(1.0, float(np.max(np.abs(a[k]))))
            _close(b[k] / scale, a[k] / scale, 1e-12, f"absorbed {k} seed {seed}")


def pin_softmax_and_special_cases():
    c = _random_case(20, L=13)
    L = 13
    r = O.attention(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"])
    _close(r["a"].sum(axis=1), np.ones(3), 1e-14, "softmax sums to one")
    # one cached token: o = c_0 . W_UV exactly, z = c_0
    r1 = O.attention(c["q_c"], c["q_r"], 0, c["cache"][:1], c["w_uk"], c["w_uv"], c["d_c"])
    _close(r1["z"], np.repeat(c["cache"][:1, :5], 3, axis=0), 0.0, "len 1 z")
    _close(r1["o"], np.stack([c["cache"][0, :5] @ c["w_uv"][h] for h in range(3)]), 1e-15, "len 1 o")
    # all scores equal -> z is the mean row and lse = ln L
    r0 = O.attention(0 * c["q_c"], 0 * c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"])
    _close(r0["z"], np.repeat(c["cache"][:, :5].mean(axis=0)[None], 3, axis=0), 1e-14, "uniform z")
    _close(r0["lse"], np.full(3, math.log(L)), 1e-14, "uniform lse")
    # permuting the cached rows changes nothing when every row is visible
    perm = _rng(21).permutation(L)
    rp = O.attention(c["q_c"], c["q_r"], L - 1, c["cache"][perm], c["w_uk"], c["w_uv"], c["d_c"])
    for k in ("o", "z", "lse"):
        _close(rp[k], r[k], 1e-13, f"permutation {k}")
    # empty key set
    re = O.attention(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"], key_range=(20, 30))
    assert np.all(re["z"] == 0) and np.all(re["o"] == 0) and np.all(re["lse"] == -math.inf)


def pin_merge_partials():
    c = _random_case(22, L=23)
    L = 23
    full = O.attention(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"])
    for T in (1, 4, 7, 23, 64):
        zs, ls = O.chunk_partials(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"], T)
        z, lse = O.merge_partials(zs, ls)
        _close(z, full["z"], 1e-13, f"merge T={T}")
        _close(lse, full["lse"], 1e-13, f"merge lse T={T}")
    # extra empty chunks change nothing
    zs, ls = O.chunk_partials(c["q_c"], c["q_r"], L - 1, c["cache"], c["w_uk"], c["w_uv"], c["d_c"], 8, n_chunks=6)
    assert np.all(ls[3:] == -math.inf)
    z, lse = O.merge_partials(zs, ls)
    _close(z, full["z"], 1e-13, "merge with empty chunks")
    # closed forms: one part is returned unchanged; two parts with equal lse average, lse + ln 2
    p = _rng(23).standard_normal((1, 3, 4))
    l1 = np.array([[0.3, -1.0, 2.0]])
    z1, lse1 = O.merge_partials(p, l1)
    _close(z1, p[0], 1e-15, "single part")
    _close(lse1, l1[0], 1e-15, "single lse")
    p2 = _rng(24).standard_normal((2, 3, 4))
    z2, lse2 = O.merge_partials(p2, np.stack([l1[0], l1[0]]))
    _close(z2, 0.5 * (p2[0] + p2[1]), 1e-15, "equal-lse average")
    _close(lse2, l1[0] + math.log(2.0), 1e-15, "equal-lse lse")
    zE, lE = O.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -math.inf))
    assert np.all(zE == 0) and np.all(lE == -math.inf)


def pin_gather_rows():
    """Page-table gather inverts the generator's scatter, for random and identity page orders."""
    r = _rng(25)
    rows = [r.standard_normal((n, 6)).astype(np.float32) for n in (5, 64, 65, 1, 130)]
    for rp in (True, False):
        pool, table = gen.paginate(rows, 8, rng=r, random_pages=rp, spare_pages=3, fill="nan", dtype="f32")
        for b, x in enumerate(rows):
            got = O.gather_rows(pool, table, b, x.shape[0])
            assert np.array_equal(got, x), f"gather seq {b}"


def pin_projections():
    """Upstream projections on selector weights (closed form) and the toy step end to end against
    the library routine."""
    h = np.arange(1.0, 9.0)[None]               # [1, 8]
    sel = np.zeros((8, 3))
    sel[[0, 2, 5], [0, 1, 2]] = 1.0                 # picks h[0], h[2], h[5]
    _close(O.kv_latent(h, sel), [[1.0, 3.0, 6.0]], 0.0, "latent projection")
    w_u = np.stack([np.eye(3)[:, :2], np.eye(3)[:, 1:]])   # head 0 keeps (0,1), head 1 keeps (1,2)
    cq, q_c, q_r = O.query_parts(h, sel, w_u, w_u[::-1])
    _close(cq, [[1.0, 3.0, 6.0]], 0.0, "query latent")
    _close(q_c, [[[1.0, 3.0], [3.0, 6.0]]], 0.0, "content query")
    _close(q_r, [[[3.0, 6.0], [1.0, 3.0]]], 0.0, "position query (unrotated)")
    kr = O.rope_key(h, sel[:, :2], 2, 1e4)
    _close(kr, _rope_complex(np.array([[1.0, 3.0]]), 2, 1e4), 1e-15, "rotated position key")
    # toy step: decompress-by-hand + library attention
    t = gen.make_toy_inputs()
    hh = t["h"].astype(np.float64)
    L = hh.shape[0]
    C = O.kv_latent(hh, t["w_dkv"])
    KR = np.stack([_rope_complex(hh[j:j + 1] @ t["w_kr"].astype(np.float64), j, 1e4)[0] for j in range(L)])
    _, qc, qr = O.query_parts(hh[L - 1], t["w_dq"], t["w_uq"], t["w_qr"])
    res = O.attention(qc, qr, L - 1, O.cache_rows(C, O.rope_key(hh, t["w_kr"], np.arange(L), 1e4)),
                      t["w_uk"], t["w_uv"], 3)
    qrr = _rope_complex(qr, L - 1, 1e4)
    for hd in range(2):
        Q = np.concatenate([qc[hd], qrr[hd]])[None]
        K = np.concatenate([C @ t["w_uk"][hd], KR], axis=1)
        ref = _sdpa(Q, K, C @ t["w_uv"][hd].astype(np.float64), 0.5)[0]
        _close(res["o"][hd], ref, 1e-12, f"toy head {hd}")


def pin_fp8_e4m3():
    """E4M3 against what the format and a library routine fix: the values of characteristic codes
    (OCP 8-bit floating point, E4M3: bias 7, subnormals m * 2^-9, S.1111.111 NaN, largest 448),
    every code's value against torch's float8_e4m3fn, the nearest-even encoding of random values,
    of every code value and of every midpoint against torch's cast, and the round trip."""
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, val in fixed.items():
        got = float(O.e4m3_decode(np.array([code], np.uint8))[0])
        assert got == val and math.copysign(1, got) == math.copysign(1, val), f"code {code:#04x}: {got} != {val}"
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all(), "NaN codes"
    codes = np.arange(256, dtype=np.uint8)
    val = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(val), nan) and np.array_equal(val[~nan], ref[~nan]), "decode vs torch"
    fin = np.sort(val[~nan])
    r = _rng(41)
    x = np.concatenate([r.uniform(-448, 448, 4000), r.standard_normal(4000) * np.exp2(r.integers(-12, 8, 4000)),
                        fin, (fin[:-1] + fin[1:]) / 2]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = O.e4m3_encode(x.astype(np.float64))
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want), f"encode vs torch: {int(np.sum(got != want))} codes differ"
    ok = codes[~nan]
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(ok)), ok), "round trip"


def pin_fp8_scale_and_rows():
    """The per-token scale rule by brute force (smallest e with amax <= 448 * 2^e), quantisation
    error within half a code step, the scaled maximum inside the range, and the row byte image."""
    for amax in (448.0, 448.0 * (1 + 2.0 ** -20), 224.0, 1.0, 0.875, 3.0e-5, 1.0e4, 0.0):
        e = int(O.fp8_scale_exponent(np.array([amax]))[0])
        if amax == 0.0:
            assert e == 0
            continue
        best = next(k for k in range(-200, 200) if amax <= 448.0 * 2.0 ** k)
        assert e == best, f"scale exponent of {amax}: {e} != {best}"
    r = _rng(42)
    c = r.standard_normal((9, 512)) * np.exp2(r.integers(-8, 8, (9, 1)))
    c[3] = 0.0
    codes, scale = O.quantize_latents_fp8(c)
    deq = O.dequantize_latents_fp8(codes, scale)
    assert np.all(np.abs(c / scale[:, None]) <= 448.0)
    assert np.all(np.max(np.abs(c), axis=1)[[0, 1, 2, 4]] > 224.0 * scale[[0, 1, 2, 4]]), "scale is the smallest"
    # each value within half the spacing of its binade: 2^-4 relative (normal), 2^-10 * scale (subnormal)
    half_step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(c), 1e-300))) - 4), 2.0 ** -10 * scale[:, None])
    assert np.all(np.abs(deq - c) <= half_step), "quantisation error beyond half a step"
    assert np.all(deq[3] == 0.0) and scale[3] == 1.0
    kr = gen.bf16_bits(r.standard_normal((9, 64)).astype(np.float32))
    rows = O.fp8_rows_pack(codes, kr, scale)
    assert rows.shape == (9, 656) and np.all(rows[:, 644:] == 0)
    assert np.array_equal(rows[0, :512], codes[0]) and rows[0, 512:514].view(np.uint16)[0] == kr[0, 0]
    assert rows[1, 640:644].view(np.float32)[0] == np.float32(scale[1])
    c2, k2, s2 = O.fp8_rows_unpack(rows)
    assert np.array_equal(c2, codes) and np.array_equal(k2, kr) and np.array_equal(s2, scale)


def pin_precomposed_weights():
    """Precomposition is associativity: the precomposed query row equals the absorbed row of the
    separately projected query (absorbed_query and query_parts are pinned on their own), and the
    fused output equals W_O applied to the per-head outputs z . W_UV[h], including a case where a
    selector W_O picks single head components by hand."""
    r = _rng(51)
    H, d_cq, d_c, d_r, d_k, d_v, d_m = 3, 5, 4, 2, 3, 2, 6
    w_uq = r.standard_normal((H, d_cq, d_k))
    w_uk = r.standard_normal((H, d_c, d_k))
    w_qr = r.standard_normal((H, d_cq, d_r))
    c_q = r.standard_normal(d_cq)
    wa = O.precompose_query_weights(w_uq, w_uk)
    assert wa.shape == (H, d_cq, d_c)
    q_c = np.einsum("q,hqk->hk", c_q, w_uq)
    q_r = np.einsum("q,hqr->hr", c_q, w_qr)
    _close(O.absorbed_query_precomposed(c_q, wa, w_qr, 7, 1e4), O.absorbed_query(q_c, q_r, 7, w_uk, 1e4), 1e-12,
           "precomposed query row")
    w_uv = r.standard_normal((H, d_c, d_v))
    w_o = r.standard_normal((H * d_v, d_m))
    z = r.standard_normal((4, H, d_c))
    per_head = np.einsum("rhc,hcv->rhv", z, w_uv)
    _close(O.out_proj_fused(z, O.precompose_out_weights(w_uv, w_o)), O.output_projection(per_head, w_o), 1e-12,
           "fused output")
    sel = np.zeros((H * d_v, d_m))
    sel[1 * d_v + 0, 0] = 1.0   # head 1, component 0 -> model column 0
    sel[2 * d_v + 1, 5] = -2.0  # head 2, component 1 -> model column 5, times -2
    fused = O.out_proj_fused(z, O.precompose_out_weights(w_uv, sel))
    _close(fused[:, 0], per_head[:, 1, 0], 1e-12, "selector head 1")
    _close(fused[:, 5], -2.0 * per_head[:, 2, 1], 1e-12, "selector head 2")
    _close(fused[:, 1:5], np.zeros((4, 4)), 0.0, "selector zeros")


def pin_rms_normalize():
    """RMSNorm with unit gain ([ase] Fig. 1 note: a norm follows the latent; eps and gain are not on
    the pages, the reading is eps = 1e-6 and gain 1) against the library routine (torch's rms_norm on
    the CPU in float64) and closed forms: a constant row a gives a / sqrt(a^2 + eps) everywhere; with
    eps = 0 every row has mean square exactly 1 and the result does not change when a row is scaled
    by a positive factor; the norm acts on each row alone."""
    r = _rng(41)
    x = r.standard_normal((6, 512)) * r.uniform(0.01, 30.0, size=(6, 1))
    for eps in (1e-6, 0.3):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), weight=None, eps=eps).numpy()
        _close(O.rms_normalize(x, eps), ref, 1e-12, f"library rms_norm eps={eps}")
    for a in (2.0, -0.5, 1e-3):
        for eps in (1e-6, 0.25):
            _close(O.rms_normalize(np.full((1, 7), a), eps), np.full((1, 7), a / math.sqrt(a * a + eps)), 1e-15,
                   f"constant row {a} eps={eps}")
    y = O.rms_normalize(x, 0.0)
    _close(np.mean(y * y, axis=-1), np.ones(6), 1e-12, "unit mean square at eps 0")
    _close(O.rms_normalize(x * np.array([[3.0], [0.01], [7.5], [1.0], [250.0], [0.5]]), 0.0), y, 1e-12,
           "positive row scaling")
    _close(O.rms_normalize(x[2:3], 1e-6), O.rms_normalize(x, 1e-6)[2:3], 0.0, "rows are independent")
    # eps decides rows of tiny magnitude: x = +-1e-3 has mean square 1e-6, so the result is x / sqrt(2e-6)
    t = np.array([[1e-3, -1e-3, 1e-3, -1e-3]])
    _close(O.rms_normalize(t, 1e-6), t / math.sqrt(2e-6), 1e-12, "eps on a tiny row")


ALL_PINS = {f.__name__: f for f in (
    pin_score_example, pin_key_absorption, pin_value_absorption, pin_cache_accounting,
    pin_rope_closed_forms, pin_rope_complex_form, pin_rope_relative,
    pin_sdpa_textbook, pin_sdpa_general, pin_prefill_causal, pin_loops_twin,
    pin_absorbed_equals_decompressed, pin_softmax_and_special_cases, pin_merge_partials,
    pin_gather_rows, pin_projections, pin_fp8_e4m3, pin_fp8_scale_and_rows, pin_precomposed_weights, pin_rms_normalize,
)}
