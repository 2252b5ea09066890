"""Workload table and seeded input generators.

Everything here is input preparation: random draws from a fixed-order PCG64
stream, round-to-nearest-even conversion to bfloat16 bit patterns, and the
paged cache layout (page permutation, page table, poison fills).  No attention
arithmetic lives here.

Value distributions (the pages fix none; these are the stated readings):
  * weights W_UK, W_UV ~ N(0, 1) / sqrt(d_c)   (d_c is their fan-in in C.W)
  * latent rows c ~ N(0, 1), then scaled to unit RMS over the d_c entries
  * k^R ~ N(0, 1) (stored as already rotated), q_C, q_R ~ N(0, 1)
  * toy workload: every value N(0, 1), fp32
With these, the scaled score of a V3-shaped head has a standard deviation of
about one, which keeps the bf16 logit error far inside the 2e-2 budget.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

RMS_EPS = 1e-6


# --------------------------------------------------------------------------
# bfloat16 storage format
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if is_nan.any():
        r[is_nan] = ((u[is_nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


# --------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    kind: str                       # "toy" | "decode" | "prefill" | "kv_append" | "verify" (prefill inputs)
    #                                 | "precomposed"
    batch: int
    n_heads: int = 128
    d_c: int = 512
    d_r: int = 64
    d_k: int = 128
    d_v: int = 128
    dtype: str = "bf16"             # storage / operand type of cache, queries, weights
    page_size: int = 64
    ctx: int = 0                    # cached tokens per sequence (fixed-length workloads)
    ctx_range: tuple | None = None  # inclusive [lo, hi] for ragged lengths
    random_pages: bool = False      # seeded random physical page order
    split_tokens: int = 0           # split-K chunk length used when this workload is timed
    q_len: int = 1                  # query tokens per sequence (prefill chunk length)
    rope_base: float = 10000.0
    d_model: int = 0                # hidden width (toy and cache-write workloads)
    d_cq: int = 0                   # toy only: query-latent width
    notes: str = field(default="", compare=False)

    @property
    def row_width(self) -> int:
        return self.d_c + self.d_r

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_k + self.d_r)


WORKLOADS: dict[str, Workload] = {
    "toy_fp32": Workload(
        name="toy_fp32", seed=1, kind="toy", batch=1, n_heads=2, d_c=3, d_r=2, d_k=2, d_v=2,
        dtype="f32", page_size=4, ctx=4, d_model=8, d_cq=3,
        notes="single decode step at p3 over p0..p3; every value N(0,1)"),
    "v3_b1_ctx4k": Workload(
        name="v3_b1_ctx4k", seed=2, kind="decode", batch=1, ctx=4096, split_tokens=256,
        notes="batch 1, 4,096 cached tokens, contiguous cache"),
    "v3_b64_ragged_paged": Workload(
        name="v3_b64_ragged_paged", seed=3, kind="decode", batch=64, ctx_range=(1024, 32768),
        random_pages=True, split_tokens=2048,
        notes="batch 64, lengths uniform on [1024, 32768], 64-token pages, random page table"),
    "v3_b4_ctx128k": Workload(
        name="v3_b4_ctx128k", seed=4, kind="decode", batch=4, ctx=131072, split_tokens=2048,
        notes="batch 4, 131,072 tokens each, split-K into 256 chunks over the batch (64 per sequence)"),
    "v3_prefill_b2": Workload(
        name="v3_prefill_b2", seed=5, kind="prefill", batch=2, ctx=2048, q_len=512,
        notes="2,048 prior tokens + a 512-token causal chunk already appended to the cache"),
    # cache-write workloads: d_model 4096 is the hidden width of the [molayo] implementation code
    "v3_kv_append_b64": Workload(
        name="v3_kv_append_b64", seed=6, kind="kv_append", batch=64, ctx_range=(1024, 32768), q_len=1,
        random_pages=True, d_model=4096,
        notes="one new token per sequence of the ragged decode batch, written at position len-1"),
    "v3_kv_append_prefill_b2": Workload(
        name="v3_kv_append_prefill_b2", seed=7, kind="kv_append", batch=2, ctx=2048, q_len=512,
        random_pages=True, d_model=4096,
        notes="the 512-token chunk of each of 2 sequences, written at positions 2048..2559"),
    # precomposed weights: the query side from the query latent and the fused output projection,
    # d_cq 1536 and d_model 4096 as in the [molayo] implementation code
    "v3_precomposed_b64": Workload(
        name="v3_precomposed_b64", seed=9, kind="precomposed", batch=64, q_len=1, d_model=4096, d_cq=1536,
        notes="64 query rows (one decode step of the ragged batch): c^Q [64, 1536], z [64, 128, 512]"),
    # multi-token verify (speculative decoding): 4 draft tokens per sequence of the ragged batch
    "v3_verify_b64_sq4": Workload(
        name="v3_verify_b64_sq4", seed=8, kind="verify", batch=64, ctx_range=(1024, 32768), q_len=4,
        random_pages=True,
        notes="64 sequences with prior lengths uniform on [1024, 32768] plus 4 draft tokens each, "
              "already appended; 64-token pages, random page table"),
}

WORKLOAD_ORDER = ["toy_fp32", "v3_b1_ctx4k", "v3_b64_ragged_paged", "v3_b4_ctx128k", "v3_prefill_b2",
                  "v3_kv_append_b64", "v3_kv_append_prefill_b2", "v3_verify_b64_sq4", "v3_precomposed_b64"]


# --------------------------------------------------------------------------
# Paged layout
# --------------------------------------------------------------------------
def _fill_values(rng: np.random.Generator | None, shape, fill: str, dtype: str) -> np.ndarray:
    if fill == "zero":
        v = np.zeros(shape, np.float32)
    elif fill == "nan":
        v = np.full(shape, np.nan, np.float32)
    elif fill == "inf":
        v = np.full(shape, np.inf, np.float32)
        v.reshape(-1)[1::2] = -np.inf
    elif fill == "random":
        v = (rng.standard_normal(shape, dtype=np.float32) * 3.0).astype(np.float32)
    else:
        raise ValueError(f"unknown fill {fill!r}")
    return bf16_bits(v) if dtype == "bf16" else v


def paginate(rows: list[np.ndarray], page_size: int, *, rng: np.random.Generator | None,
             random_pages: bool, spare_pages: int = 0, fill: str = "random",
             dtype: str = "bf16") -> tuple[np.ndarray, np.ndarray]:
    """Scatter per-sequence logical rows into a page pool.

    rows[b] is [len_b, W].  Returns (pool [P, page_size, W], page_table [B, max_pages] int32).
    Logical token t of sequence b lives at pool[page_table[b, t // page_size], t % page_size].
    Table entries past a sequence's last page are -1.  Slots past len_b in the last page and
    all spare pages hold ``fill`` values, which a correct reader never uses.
    """
    B = len(rows)
    W = rows[0].shape[1]
    npages = [-(-r.shape[0] // page_size) for r in rows]
    max_pages = max(1, max(npages))
    total = sum(npages) + spare_pages
    order = rng.permutation(total) if random_pages else np.arange(total)
    store_dtype = np.uint16 if dtype == "bf16" else np.float32
    pool = np.empty((total, page_size, W), dtype=store_dtype)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    nxt = 0
    for b, r in enumerate(rows):
        for i in range(npages[b]):
            pid = int(order[nxt])
            nxt += 1
            table[b, i] = pid
            seg = r[i * page_size:(i + 1) * page_size]
            pool[pid, :seg.shape[0]] = seg
            if seg.shape[0] < page_size:
                pool[pid, seg.shape[0]:] = _fill_values(rng, (page_size - seg.shape[0], W), fill, dtype)
    for k in range(nxt, total):
        pool[int(order[k])] = _fill_values(rng, (page_size, W), fill, dtype)
    return pool, table


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------
def _normal(rng, shape, scale=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _unit_rms_rows(x: np.ndarray) -> np.ndarray:
    """Scale each row to unit root-mean-square (the latent distribution of the V3 workloads)."""
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(RMS_EPS))).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.ctx_range is not None:
        lo, hi = w.ctx_range
        return rng.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)
    return np.full(w.batch, w.ctx + (w.q_len if w.kind == "prefill" else 0), dtype=np.int32)


def make_decode_inputs(w: Workload, *, seed: int | None = None, lens: np.ndarray | None = None,
                       fill: str = "random", spare_pages: int = 8, random_pages: bool | None = None,
                       latent_rows: np.ndarray | None = None) -> dict:
    """Inputs for one decode step of every sequence in the batch.

    Draw order: lengths, W_UK, W_UV, latent rows, k^R rows, q_C, q_R, page permutation, fills.
    Stored arrays are bf16 bit patterns (uint16) for dtype "bf16", float32 otherwise.
    Returns a dict with q_c [B,H,d_k], q_r [B,H,d_r], w_uk [H,d_c,d_k], w_uv [H,d_c,d_v],
    pool [P,page,d_c+d_r], page_table [B,max_pages], lens [B], pos [B] (= lens-1).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    if lens is None:
        lens = draw_lengths(w, rng)
    lens = np.asarray(lens, dtype=np.int32)
    H, dc, dr, dk, dv = w.n_heads, w.d_c, w.d_r, w.d_k, w.d_v
    w_uk = _normal(rng, (H, dc, dk), 1.0 / math.sqrt(dc))
    w_uv = _normal(rng, (H, dc, dv), 1.0 / math.sqrt(dc))
    rows = []
    for b in range(w.batch):
        L = int(lens[b])
        c = _unit_rms_rows(_normal(rng, (L, dc)))
        kr = _normal(rng, (L, dr))
        rows.append(_store(np.concatenate([c, kr], axis=1), w.dtype))
    if latent_rows is not None:
        rows = latent_rows
    q_c = _normal(rng, (w.batch, H, dk))
    q_r = _normal(rng, (w.batch, H, dr))
    pool, table = paginate(rows, w.page_size, rng=rng,
                           random_pages=w.random_pages if random_pages is None else random_pages,
                           spare_pages=spare_pages, fill=fill, dtype=w.dtype)
    return dict(workload=w, dtype=w.dtype, lens=lens, pos=(lens - 1).astype(np.int32),
                q_c=_store(q_c, w.dtype), q_r=_store(q_r, w.dtype),
                w_uk=_store(w_uk, w.dtype), w_uv=_store(w_uv, w.dtype),
                pool=pool, page_table=table)


def make_prefill_inputs(w: Workload, *, seed: int | None = None, fill: str = "random",
                        spare_pages: int = 8) -> dict:
    """Inputs for one chunked-prefill call: prior ctx tokens plus q_len new tokens.

    The new chunk's own rows are already in the cache (cache length ctx + q_len per sequence).
    Query i of sequence b sits at absolute position q_start[b] + i with q_start = the prior length
    (ctx, or drawn uniformly from ctx_range per sequence when the workload gives one).
    Draw order: [prior lengths], W_UK, W_UV, latent rows, k^R rows, q_C, q_R, page permutation, fills.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    H, dc, dr, dk, dv = w.n_heads, w.d_c, w.d_r, w.d_k, w.d_v
    if w.ctx_range is not None:
        lo, hi = w.ctx_range
        prior = rng.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)
    else:
        prior = np.full(w.batch, w.ctx, dtype=np.int32)
    lens = (prior + w.q_len).astype(np.int32)
    w_uk = _normal(rng, (H, dc, dk), 1.0 / math.sqrt(dc))
    w_uv = _normal(rng, (H, dc, dv), 1.0 / math.sqrt(dc))
    rows = []
    for b in range(w.batch):
        L = int(lens[b])
        c = _unit_rms_rows(_normal(rng, (L, dc)))
        kr = _normal(rng, (L, dr))
        rows.append(_store(np.concatenate([c, kr], axis=1), w.dtype))
    q_c = _normal(rng, (w.batch, w.q_len, H, dk))
    q_r = _normal(rng, (w.batch, w.q_len, H, dr))
    pool, table = paginate(rows, w.page_size, rng=rng, random_pages=w.random_pages,
                           spare_pages=spare_pages, fill=fill, dtype=w.dtype)
    return dict(workload=w, dtype=w.dtype, lens=lens,
                q_start=prior.copy(),
                q_c=_store(q_c, w.dtype), q_r=_store(q_r, w.dtype),
                w_uk=_store(w_uk, w.dtype), w_uv=_store(w_uv, w.dtype),
                pool=pool, page_table=table)


def make_precomposed_inputs(w: Workload, *, rows: int | None = None, seed: int | None = None) -> dict:
    """Inputs of the precomposed-weight products for `rows` query rows.

    Draw order: W_UQ, W_QR, W_UK, W_UV, W_O, c^Q, z, o, positions.  Weights are N(0,1)/sqrt(fan-in)
    (d_cq for W_UQ and W_QR, d_c for W_UK and W_UV, H * d_v for W_O) stored bf16; c^Q is N(0,1)
    bf16; the weighted latents z and the per-head outputs o are N(0,1) float32; positions are
    uniform on [0, 131072).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    R = w.batch if rows is None else rows
    H, dc, dr, dk, dv, dq, dm = w.n_heads, w.d_c, w.d_r, w.d_k, w.d_v, w.d_cq, w.d_model
    out = dict(workload=w, dtype=w.dtype, rows=R)
    out["w_uq"] = _store(_normal(rng, (H, dq, dk), 1.0 / math.sqrt(dq)), w.dtype)
    out["w_qr"] = _store(_normal(rng, (H, dq, dr), 1.0 / math.sqrt(dq)), w.dtype)
    out["w_uk"] = _store(_normal(rng, (H, dc, dk), 1.0 / math.sqrt(dc)), w.dtype)
    out["w_uv"] = _store(_normal(rng, (H, dc, dv), 1.0 / math.sqrt(dc)), w.dtype)
    out["w_o"] = _store(_normal(rng, (H * dv, dm), 1.0 / math.sqrt(H * dv)), w.dtype)
    out["c_q"] = _store(_normal(rng, (R, dq)), w.dtype)
    out["z"] = _normal(rng, (R, H, dc)).astype(np.float32)
    out["o"] = _normal(rng, (R, H, dv)).astype(np.float32)
    out["pos"] = rng.integers(0, 131072, size=R, dtype=np.int64).astype(np.int32)
    return out


def make_toy_inputs(w: Workload | None = None, *, seed: int | None = None) -> dict:
    """The toy single-step workload: hidden states of p0..p3 and every projection, N(0,1) fp32.

    Draw order: h [L, d_model], W_DQ [d_model, d_cq], W_UQ [H, d_cq, d_k], W_QR [H, d_cq, d_r],
    W_DKV [d_model, d_c], W_UK [H, d_c, d_k], W_UV [H, d_c, d_v], W_KR [d_model, d_r].
    The query is the last position (p3).
    """
    w = w or WORKLOADS["toy_fp32"]
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    L, d, H = w.ctx, w.d_model, w.n_heads
    out = dict(workload=w, dtype="f32")
    out["h"] = _normal(rng, (L, d))
    out["w_dq"] = _normal(rng, (d, w.d_cq))
    out["w_uq"] = _normal(rng, (H, w.d_cq, w.d_k))
    out["w_qr"] = _normal(rng, (H, w.d_cq, w.d_r))
    out["w_dkv"] = _normal(rng, (d, w.d_c))
    out["w_uk"] = _normal(rng, (H, w.d_c, w.d_k))
    out["w_uv"] = _normal(rng, (H, w.d_c, w.d_v))
    out["w_kr"] = _normal(rng, (d, w.d_r))
    out["pos"] = np.arange(L, dtype=np.int32)
    return out


def make_kv_append_inputs(w: Workload, *, seed: int | None = None, rows: int | None = None,
                          fill: str = "random", spare_pages: int = 4) -> dict:
    """Inputs for one cache write of new tokens.

    Sequence b receives q_len new tokens at positions p0_b .. p0_b + q_len - 1, where p0_b =
    len_b - 1 for ragged decode workloads (len_b drawn like the decode batch) and ctx otherwise.
    Only the pages that hold new tokens exist: distinct physical pages in seeded random order,
    every other table entry -1.  The pool starts filled with `fill` values.
    Draw order: lengths, W_DKV, W_KR (both N(0,1)/sqrt(d_model), d_model their fan-in), h
    (N(0,1)), page permutation, fills.  `rows` truncates the token list (edge cases).
    Returns h [R, d_model], w_dkv [d_model, d_c], w_kr [d_model, d_r], seq_ids [R], positions [R],
    pool [P, page, d_c+d_r], page_table [B, max_pages].
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    if w.ctx_range is not None:
        p0 = draw_lengths(w, rng) - 1
    else:
        p0 = np.full(w.batch, w.ctx, dtype=np.int32)
    d = w.d_model
    w_dkv = _normal(rng, (d, w.d_c), 1.0 / math.sqrt(d))
    w_kr = _normal(rng, (d, w.d_r), 1.0 / math.sqrt(d))
    seq_ids = np.repeat(np.arange(w.batch, dtype=np.int32), w.q_len)
    positions = (p0[:, None] + np.arange(w.q_len, dtype=np.int32)[None]).reshape(-1).astype(np.int32)
    if rows is not None:
        seq_ids, positions = seq_ids[:rows], positions[:rows]
    R = seq_ids.shape[0]
    h = _normal(rng, (R, d))
    ps = w.page_size
    need = sorted({(int(b), int(t) // ps) for b, t in zip(seq_ids, positions)})
    total = len(need) + spare_pages
    order = rng.permutation(total) if w.random_pages else np.arange(total)
    max_pages = max(int(t) // ps for t in positions) + 1
    table = np.full((w.batch, max_pages), -1, dtype=np.int32)
    for k, (b, lp) in enumerate(need):
        table[b, lp] = int(order[k])
    pool = _fill_values(rng, (total, ps, w.row_width), fill, w.dtype)
    return dict(workload=w, dtype=w.dtype, h=_store(h, w.dtype), w_dkv=_store(w_dkv, w.dtype),
                w_kr=_store(w_kr, w.dtype), seq_ids=seq_ids, positions=positions, pool=pool,
                page_table=table)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values (bf16 bits or float32) to float64."""
    if dtype == "bf16":
        return bf16_from_bits(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)
