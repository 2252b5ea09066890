"""fp64 CPU oracle for Multi-Head Latent Attention over a latent cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the test suite, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library and the library
never reads anything it produces.

What it computes is the plain definition of MLA attention, evaluated the
*unabsorbed* way: every cached latent is decompressed into a per-head content
key and value, scores are content dot plus position dot, one scale, one softmax
over every visible position, then the weighted sum of values.  Because key and
value absorption are exact rewrites by associativity, this definition is what
the absorbed GPU path must reproduce up to rounding.  An absorbed fp64 twin and
a scalar-loop twin (pure Python) are included to check the main routine.

Pages cited (title, site):
  [molayo] "Multi-Head Latent Attention (MLA)", molayo1419.me
  [ase]    "MLA의 계산: KV를 펼치지 않고 Attention하기", ai-systems-engineering.com
  [huny]   "DeepSeek Multi-Head Latent Attention(MLA) 아키텍처 해부 ...", blog.huny.dev
  [pcxr]   "Multi-Head Latent Attention", process-cxr.github.io

Conventions (readings where the pages differ or are silent):
  * row vectors: K_h = C . W_UK[h], with W_UK stored [H, d_c, d_k]   ([molayo] formal definition;
    [ase] Fig. 3 equation)
  * one scale 1/sqrt(d_k + d_r) on the summed score, unchanged by absorption ([ase] sections
    "Content 점수와 위치 점수 합치기" and "RoPE 경로를 분리한 이유")
  * k^R is one 64-wide key per token shared by all heads, cached already rotated
    ([ase] Fig. 1 caption and Fig. 2; [huny] section 2, decoupled-RoPE principle)
  * RoPE on interleaved pairs with inverse frequency base^(-2i/d_r) ([molayo] implementation code)
  * 0-based absolute positions; a query at position p sees keys j <= p ([ase] causal-mask remark
    after Fig. 2)
  * an empty key set gives z = 0, o = 0, lse = -inf
  * FP8 latent cache ([huny] section 5, FP8 item): E4M3 as the OCP 8-bit floating-point format
    defines it, one scale per token over its 512 latent values, taken as the smallest power of
    two that brings the largest magnitude within 448 (the page names per-tensor or per-token
    scales and fixes no rule; a power of two keeps code value x scale exact); the rotary key
    stays bf16

Parity pins for every function live in tests/ (oracle pins, invariants and planted-mistake
tests); none of the functions below is parity unpinned.
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# Rotary position embedding
# --------------------------------------------------------------------------
def rope_inv_freq(d_r: int, base: float) -> np.ndarray:
    """Inverse frequencies base^(-2i/d_r), i = 0 .. d_r/2-1.

    [molayo] implementation code: the frequency buffer built from the even indices 0, 2, 4, ...
    divided by the rotary width.
    """
    if d_r % 2:
        raise ValueError("rotary width must be even")
    i = np.arange(d_r // 2, dtype=F64)
    return np.power(F64(base), -(2.0 * i) / d_r)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate interleaved pairs (x[2i], x[2i+1]) by the angle pos * base^(-2i/d_r).

    [molayo] implementation code (the rotary helper of the MLA module): pairs are taken from
    the even and odd slots, rotated to (x1 cos - x2 sin, x1 sin + x2 cos) and interleaved back.
    ``pos`` broadcasts against x.shape[:-1]; positions are absolute.
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=F64)[..., None] * rope_inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=F64)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x1 * s + x2 * c
    return out


# --------------------------------------------------------------------------
# Projections upstream of the cache (the cache-write side)
# --------------------------------------------------------------------------
def kv_latent(h: np.ndarray, w_dkv: np.ndarray) -> np.ndarray:
    """c^KV = h . W_DKV  ([molayo] formal definition, compression; [pcxr] joint K/V compression)."""
    return np.asarray(h, F64) @ np.asarray(w_dkv, F64)


def rms_normalize(c: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm with unit gain over the latent width ([ase] Fig. 1 note: a norm follows the latent)."""
    c = np.asarray(c, F64)
    return c / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)


def rope_key(h: np.ndarray, w_kr: np.ndarray, pos, base: float) -> np.ndarray:
    """k^R_t = RoPE_t(h_t . W_KR): one position key per token, shared by every head.

    [huny] section 2, decoupled-RoPE principle; [ase] Fig. 1 caption (position key shared).
    """
    return rope(np.asarray(h, F64) @ np.asarray(w_kr, F64), pos, base)


def query_parts(h: np.ndarray, w_dq: np.ndarray, w_uq: np.ndarray, w_qr: np.ndarray):
    """c^Q = h . W_DQ; per head q^C_h = c^Q . W_UQ[h] and unrotated q^R_h = c^Q . W_QR[h].

    [ase] "현재 토큰의 Query 만들기", Fig. 1; [molayo] formal definition, query compression.
    Returns (c_q [..., d_cq], q_c [..., H, d_k], q_r_unrotated [..., H, d_r]).
    """
    cq = np.asarray(h, F64) @ np.asarray(w_dq, F64)
    q_c = np.einsum("...c,hck->...hk", cq, np.asarray(w_uq, F64))
    q_r = np.einsum("...c,hcr->...hr", cq, np.asarray(w_qr, F64))
    return cq, q_c, q_r


def cache_rows(c: np.ndarray, k_r: np.ndarray) -> np.ndarray:
    """One cached row per token: [c^KV | k^R] ([huny] section 1 table, 512 + 64 values per token)."""
    return np.concatenate([np.asarray(c, F64), np.asarray(k_r, F64)], axis=-1)


def gather_rows(pool: np.ndarray, page_table: np.ndarray, b: int, length: int) -> np.ndarray:
    """Logical rows 0..length-1 of sequence b from a paged pool (dtype preserved).

    [molayo] key concept 5: a page table whose entries hold latent rows instead of K/V pairs.
    Row t lives at pool[page_table[b, t // page], t % page].
    """
    page = pool.shape[1]
    out = np.empty((length, pool.shape[2]), dtype=pool.dtype)
    for t0 in range(0, length, page):
        n = min(page, length - t0)
        out[t0:t0 + n] = pool[int(page_table[b, t0 // page]), :n]
    return out


# --------------------------------------------------------------------------
# Attention, unabsorbed (the definition)
# --------------------------------------------------------------------------
def decompress(C: np.ndarray, w_uk_h: np.ndarray, w_uv_h: np.ndarray):
    """K_h = C . W_UK[h], V_h = C . W_UV[h]  ([molayo] formal definition, decompression;
    [ase] Fig. 2 left half)."""
    return C @ w_uk_h, C @ w_uv_h


def score_row(q_c_h, q_r_rot_h, K_h, k_r, scale):
    """s_j = (q^C_h . k^C_{j,h} + q^R_h . k^R_j) * scale: content dot plus position dot, no cross
    terms, one scale ([ase] Fig. 2 score equation and the scale remark that follows it)."""
    return (K_h @ q_c_h + k_r @ q_r_rot_h) * scale


def softmax_lse(s: np.ndarray):
    """Softmax over every visible position with max subtraction; also ln(sum exp(s)).

    [ase] Fig. 2: one softmax across all positions, not one per position.
    """
    if s.size == 0:
        return s.copy(), -math.inf
    m = np.max(s)
    e = np.exp(s - m)
    tot = np.sum(e)
    return e / tot, float(m + math.log(tot))


def visible_keys(L: int, q_pos: int, key_range=None) -> np.ndarray:
    """Key positions a query at q_pos reads: 0 <= j < L, j <= q_pos, intersected with key_range."""
    hi = min(L, q_pos + 1)
    lo = 0
    if key_range is not None:
        lo = max(lo, key_range[0])
        hi = min(hi, key_range[1])
    return np.arange(lo, max(lo, hi))


def attention(q_c, q_r, q_pos: int, cache, w_uk, w_uv, d_c: int, scale=None, base=10000.0,
              key_range=None, heads=None) -> dict:
    """One query token of every head against the logical cache rows of its sequence.

    q_c [H, d_k]; q_r [H, d_r] unrotated; cache [L, d_c + d_r], row j = [c_j | k^R_j] at
    position j; w_uk [H, d_c, d_k]; w_uv [H, d_c, d_v].
    Returns o [H, d_v], z [H, d_c] (= a . C, the weighted latent), lse [H] (natural log of the
    sum of exp(scaled score)), a [H, n] and s [H, n] over the visible keys, keys [n].
    ``heads`` restricts the computation to a subset of heads (other rows stay NaN), so single
    outputs of full-size workloads can be computed one by one.
    """
    q_c = np.asarray(q_c, F64)
    q_r = np.asarray(q_r, F64)
    cache = np.asarray(cache, F64)
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    H, d_k = q_c.shape
    d_r = q_r.shape[1]
    d_v = w_uv.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d_k + d_r)
    keys = visible_keys(cache.shape[0], q_pos, key_range)
    C = cache[keys, :d_c]
    k_r = cache[keys, d_c:d_c + d_r]
    q_r_rot = rope(q_r, q_pos, base)
    o = np.full((H, d_v), np.nan)
    z = np.full((H, d_c), np.nan)
    lse = np.full(H, np.nan)
    a_all = np.full((H, keys.size), np.nan)
    s_all = np.full((H, keys.size), np.nan)
    for h in (range(H) if heads is None else heads):
        K_h, V_h = decompress(C, w_uk[h], w_uv[h])
        s = score_row(q_c[h], q_r_rot[h], K_h, k_r, scale)
        a, lse[h] = softmax_lse(s)
        o[h] = a @ V_h if keys.size else 0.0
        z[h] = a @ C if keys.size else 0.0
        a_all[h] = a
        s_all[h] = s
    return dict(o=o, z=z, lse=lse, a=a_all, s=s_all, keys=keys)


def chunk_partials(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c, split_tokens, n_chunks=None,
                   scale=None, base=10000.0):
    """Per-chunk results over key ranges [i*T, (i+1)*T): z_i [S, H, d_c] and lse_i [S, H].

    The chunking itself is not on the pages; each chunk is the plain definition restricted to
    its key range (an empty range gives z_i = 0, lse_i = -inf).
    """
    L = np.asarray(cache).shape[0]
    S = n_chunks if n_chunks is not None else max(1, -(-L // split_tokens))
    zs, ls = [], []
    for i in range(S):
        r = attention(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c, scale, base,
                      key_range=(i * split_tokens, (i + 1) * split_tokens))
        zs.append(r["z"])
        ls.append(r["lse"])
    return np.stack(zs), np.stack(ls)


def merge_partials(parts: np.ndarray, lses: np.ndarray):
    """Merge normalised partial results by log-sum-exp: LSE = ln sum_i exp(lse_i) and
    out = sum_i exp(lse_i - LSE) parts_i.  Over any partition of the keys this equals the
    single-pass softmax result.  All-empty -> zeros and -inf.
    parts [S, H, d], lses [S, H] -> (out [H, d], lse [H]).
    """
    parts = np.asarray(parts, F64)
    lses = np.asarray(lses, F64)
    m = np.max(lses, axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - msafe[None]), 0.0)
    tot = np.sum(w, axis=0)
    lse = np.where(finite, msafe + np.log(np.where(finite, tot, 1.0)), -math.inf)
    wn = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)
    out = np.einsum("sh,shd->hd", wn, parts)
    return out, lse


def prefill(q_c, q_r, q_start: int, cache, w_uk, w_uv, d_c, scale=None, base=10000.0,
            rows=None) -> dict:
    """Chunked prefill: query i sits at absolute position q_start + i and reads keys j <= q_start + i
    ([ase] causal-mask remark after Fig. 2).  The chunk's own rows are already in the cache.

    q_c [Sq, H, d_k], q_r [Sq, H, d_r]; ``rows`` optionally restricts which query rows are computed.
    Returns o [n, H, d_v], z [n, H, d_c], lse [n, H] for the computed rows.
    """
    q_c = np.asarray(q_c, F64)
    idx = range(q_c.shape[0]) if rows is None else rows
    os_, zs, ls = [], [], []
    for i in idx:
        r = attention(q_c[i], q_r[i], q_start + i, cache, w_uk, w_uv, d_c, scale, base)
        os_.append(r["o"])
        zs.append(r["z"])
        ls.append(r["lse"])
    return dict(o=np.stack(os_), z=np.stack(zs), lse=np.stack(ls))


# --------------------------------------------------------------------------
# Absorbed twin (fp64) -- used to check absorbed == decompressed
# --------------------------------------------------------------------------
def absorbed_query(q_c, q_r, q_pos, w_uk, base=10000.0):
    """q_hat_h = [q^C_h . W_UK[h]^T | RoPE_pos(q^R_h)], width d_c + d_r.

    [ase] "Key 투영을 Query 쪽으로 옮기기", Fig. 3 equation: the key projection moves onto the query
    once, and the result is dotted with the raw latent rows.
    """
    q_c = np.asarray(q_c, F64)
    w_uk = np.asarray(w_uk, F64)
    q_lat = np.einsum("hk,hck->hc", q_c, w_uk)
    return np.concatenate([q_lat, rope(q_r, q_pos, base)], axis=-1)


def attention_absorbed(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c, scale=None, base=10000.0,
                       key_range=None) -> dict:
    """Same result as ``attention`` computed the absorbed way: scores q_hat . row_j over the
    concatenated row, z = a . C, and o = z . W_UV[h] applied once after the weighted sum
    ([ase] Fig. 3 and Fig. 4 equations; [huny] section 2, key and value absorption)."""
    q_c = np.asarray(q_c, F64)
    cache = np.asarray(cache, F64)
    w_uv = np.asarray(w_uv, F64)
    H, d_k = q_c.shape
    d_r = np.asarray(q_r).shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d_k + d_r)
    keys = visible_keys(cache.shape[0], q_pos, key_range)
    rows = cache[keys, :d_c + d_r]
    qh = absorbed_query(q_c, q_r, q_pos, w_uk, base)
    s = (qh @ rows.T) * scale
    z = np.zeros((H, d_c))
    lse = np.full(H, -math.inf)
    for h in range(H):
        a, lse[h] = softmax_lse(s[h])
        if keys.size:
            z[h] = a @ rows[:, :d_c]
    o = absorbed_output(z, w_uv)
    return dict(o=o, z=z, lse=lse, s=s, keys=keys)


def absorbed_output(z: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o_h = z_h . W_UV[h] for every head: the value up-projection applied once to the weighted
    latent instead of to every cached row ([ase] Fig. 4 equation; [huny] section 2, value
    absorption).  z [..., H, d_c], w_uv [H, d_c, d_v] -> [..., H, d_v]."""
    z = np.asarray(z, F64)
    w_uv = np.asarray(w_uv, F64)
    return np.einsum("...hc,hcv->...hv", z, w_uv)


# --------------------------------------------------------------------------
# Scalar-loop twin (pure Python, tiny sizes) -- checks the NumPy routine
# --------------------------------------------------------------------------
def attention_loops(q_c, q_r, q_pos, cache, w_uk, w_uv, d_c, scale=None, base=10000.0) -> dict:
    """Plain-loop evaluation of ``attention`` with math.cos/sin/exp/log only."""
    q_c = [[float(v) for v in row] for row in np.asarray(q_c)]
    q_r = [[float(v) for v in row] for row in np.asarray(q_r)]
    cache = [[float(v) for v in row] for row in np.asarray(cache)]
    w_uk = np.asarray(w_uk, F64).tolist()
    w_uv = np.asarray(w_uv, F64).tolist()
    H, d_k, d_r = len(q_c), len(q_c[0]), len(q_r[0])
    d_v = len(w_uv[0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d_k + d_r)
    n = min(len(cache), q_pos + 1)
    o = [[0.0] * d_v for _ in range(H)]
    z = [[0.0] * d_c for _ in range(H)]
    lse = [-math.inf] * H
    for h in range(H):
        qr = [0.0] * d_r
        for i in range(d_r // 2):
            ang = q_pos * base ** (-(2.0 * i) / d_r)
            x1, x2 = q_r[h][2 * i], q_r[h][2 * i + 1]
            qr[2 * i] = x1 * math.cos(ang) - x2 * math.sin(ang)
            qr[2 * i + 1] = x1 * math.sin(ang) + x2 * math.cos(ang)
        s = []
        for j in range(n):
            acc = 0.0
            for k in range(d_k):
                key = 0.0
                for c in range(d_c):
                    key += cache[j][c] * w_uk[h][c][k]
                acc += q_c[h][k] * key
            for r in range(d_r):
                acc += qr[r] * cache[j][d_c + r]
            s.append(acc * scale)
        if n == 0:
            continue
        m = max(s)
        e = [math.exp(v - m) for v in s]
        tot = sum(e)
        lse[h] = m + math.log(tot)
        for j in range(n):
            a = e[j] / tot
            for c in range(d_c):
                z[h][c] += a * cache[j][c]
            for v in range(d_v):
                val = 0.0
                for c in range(d_c):
                    val += cache[j][c] * w_uv[h][c][v]
                o[h][v] += a * val
    return dict(o=np.array(o), z=np.array(z), lse=np.array(lse))


# --------------------------------------------------------------------------
# Precomposed weights (offline products of consecutive projections)
# --------------------------------------------------------------------------
def precompose_query_weights(w_uq: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """W_absorbed[h] = W_UQ[h] . W_UK[h]^T, [H, d_cq, d_c]: the content query in latent space comes
    straight from c^Q ([molayo] formal definition, absorbed weight; [ase] section on multiplying
    consecutive projections ahead of time, query side)."""
    return np.matmul(np.asarray(w_uq, F64), np.swapaxes(np.asarray(w_uk, F64), 1, 2))


def absorbed_query_precomposed(c_q, w_absorbed, w_qr, q_pos, base=10000.0) -> np.ndarray:
    """q_hat_h = [c^Q . W_absorbed[h] | RoPE_pos(c^Q . W_QR[h])] for one query row c^Q [d_cq];
    the same row as absorbed_query on q^C_h = c^Q . W_UQ[h], q^R_h = c^Q . W_QR[h]."""
    c_q = np.asarray(c_q, F64)
    q_lat = np.tensordot(c_q, np.asarray(w_absorbed, F64), axes=([0], [1]))   # [H, d_c]
    q_r = np.tensordot(c_q, np.asarray(w_qr, F64), axes=([0], [1]))           # [H, d_r]
    return np.concatenate([q_lat, rope(q_r, q_pos, base)], axis=-1)


def output_projection(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """The layer output o_concat . W_O, heads concatenated: o [..., H, d_v], W_O [H * d_v, d_model]."""
    o = np.asarray(o, F64)
    return o.reshape(o.shape[:-2] + (-1,)) @ np.asarray(w_o, F64)


def precompose_out_weights(w_uv: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """W~_O[h] = W_UV[h] . W_O[h], [H, d_c, d_model], with W_O[h] the d_v rows of W_O that head h's
    output meets ([ase] section on multiplying consecutive projections ahead of time, value side;
    [huny] section 2, value absorption and output-projection fusion)."""
    w_uv = np.asarray(w_uv, F64)
    H, _, d_v = w_uv.shape
    return np.matmul(w_uv, np.asarray(w_o, F64).reshape(H, d_v, -1))


def out_proj_fused(z: np.ndarray, w_uvo: np.ndarray) -> np.ndarray:
    """Layer output straight from the weighted latents: sum_h z_h . W~_O[h]; z [..., H, d_c]."""
    z = np.asarray(z, F64)
    w_uvo = np.asarray(w_uvo, F64)
    return z.reshape(z.shape[:-2] + (-1,)) @ w_uvo.reshape(-1, w_uvo.shape[-1])


# --------------------------------------------------------------------------
# FP8 latent cache ([huny] section 5, FP8 mixed-precision item: E4M3 on the 512-wide latent with
# a per-token scale factor)
# --------------------------------------------------------------------------
# E4M3 as the OCP 8-bit floating-point format defines it (the "FN" variant): sign, 4 exponent
# bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; no infinities;
# S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
E4M3_MAX = 448.0
FP8_ROW_BYTES = 656  # 512 codes | 64 bf16 rotary values | fp32 scale | 12 zero bytes


def e4m3_decode(codes) -> np.ndarray:
    """Value of every E4M3 code (uint8 array) as float64; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(F64)))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def _half_even(x: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, ties to even (x >= 0)."""
    f = np.floor(x)
    d = x - f
    up = (d > 0.5) | ((d == 0.5) & (np.fmod(f, 2.0) == 1.0))
    return f + up


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code to each value, ties to the even code; |x| must not exceed 448 (the
    quantiser's scale guarantees it).  Zero keeps its sign; NaN gives 0x7F."""
    x = np.asarray(x, dtype=F64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("value beyond the E4M3 range")
    a = np.abs(np.nan_to_num(x, nan=0.0))
    code = np.zeros(x.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9 (a result of 8 steps is the smallest normal, code 0x08)
    code = np.where(sub, _half_even(a / 2.0 ** -9).astype(np.int64), code)
    # normal range: a = (1 + k/8) * 2^E, E = floor(log2 a); k = 8 carries into the exponent
    E = np.floor(np.log2(np.where(sub, 1.0, a)))
    # guard the floor of log2 against its own rounding at exact powers of two
    E = np.where(np.exp2(E) > a, E - 1, E)
    E = np.where(np.exp2(E + 1) <= a, E + 1, E)
    k = _half_even((a / np.exp2(E) - 1.0) * 8.0).astype(np.int64)
    norm_code = (((E + 7).astype(np.int64)) << 3) + k  # k = 8 rolls into the next exponent
    code = np.where(sub, code, norm_code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def fp8_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Per-token scale 2^e with the smallest integer e such that amax <= 448 * 2^e, so the scaled
    latent fills the E4M3 range; an all-zero latent takes e = 0.  A power of two keeps
    code value * scale exact in any binary format that holds it."""
    amax = np.asarray(amax, dtype=F64)
    e = np.zeros(amax.shape, dtype=np.int64)
    pos = amax > 0
    est = np.ceil(np.log2(np.where(pos, amax, 1.0) / E4M3_MAX)).astype(np.int64)
    # settle the estimate exactly: smallest e with amax <= 448 * 2^e
    est = np.where(amax > E4M3_MAX * np.exp2(est.astype(F64)), est + 1, est)
    est = np.where(amax <= E4M3_MAX * np.exp2((est - 1).astype(F64)), est - 1, est)
    return np.where(pos, est, e)


def quantize_latents_fp8(c: np.ndarray):
    """Per-token E4M3 quantisation of latent rows c [N, d_c]: returns (codes uint8 [N, d_c],
    scale float64 [N]) with codes = E4M3(c / scale) and scale = 2^e (fp8_scale_exponent of the
    row's largest magnitude).  Division by a power of two is exact."""
    c = np.asarray(c, dtype=F64)
    e = fp8_scale_exponent(np.max(np.abs(c), axis=-1))
    scale = np.exp2(e.astype(F64))
    return e4m3_encode(c / scale[..., None]), scale


def dequantize_latents_fp8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Latent values the FP8 cache holds: code value times the token's scale (exact in fp64)."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=F64)[..., None]


def fp8_rows_pack(codes: np.ndarray, kr_bf16_bits: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Byte image of FP8 cache rows [N, 656]: the d_c codes, the rotary key's bf16 bit patterns
    (unchanged), the scale as a little-endian float32, zero padding to a 16-byte multiple."""
    n = codes.shape[0]
    out = np.zeros((n, FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :512] = codes
    out[:, 512:640] = np.ascontiguousarray(kr_bf16_bits, dtype=np.uint16).view(np.uint8).reshape(n, 128)
    out[:, 640:644] = np.asarray(scale, dtype=np.float32).reshape(n, 1).view(np.uint8)
    return out


def fp8_rows_unpack(rows: np.ndarray):
    """Inverse of fp8_rows_pack: (codes [N, 512], rotary bf16 bits [N, 64], scale float64 [N])."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    codes = rows[:, :512].copy()
    kr = rows[:, 512:640].copy().view(np.uint16).reshape(n, 64)
    scale = rows[:, 640:644].copy().view(np.float32).reshape(n).astype(F64)
    return codes, kr, scale


# --------------------------------------------------------------------------
# Cache-size accounting (closed forms)
# --------------------------------------------------------------------------
def mla_values_per_token(d_c: int, d_r: int) -> int:
    """Cached values per token per layer: latent plus shared rotary key ([huny] section 1 table)."""
    return d_c + d_r


def mla_bytes_per_token(d_c: int, d_r: int, bytes_per_value: int = 2) -> int:
    return mla_values_per_token(d_c, d_r) * bytes_per_value


def mha_bytes_per_token(n_heads: int, d_k: int, bytes_per_value: int = 2) -> int:
    """Standard MHA caches a key and a value per head: 2 * n_h * d_k values
    ([molayo] formal definition; [huny] section 1 table)."""
    return 2 * n_heads * d_k * bytes_per_value


def gqa_bytes_per_token(n_kv_heads: int, d_k: int, bytes_per_value: int = 2) -> int:
    """GQA caches a key and a value per KV group ([molayo] comparison table; [huny] section 1)."""
    return 2 * n_kv_heads * d_k * bytes_per_value


def saving(new_bytes: float, old_bytes: float) -> float:
    return 1.0 - new_bytes / old_bytes


def whole_cache_gib(bytes_per_token: float, ctx: int, layers: int) -> float:
    """Total cache over ctx tokens and ``layers`` layers, in GiB (2^30 bytes)."""
    return bytes_per_token * ctx * layers / float(1 << 30)


def compression_ratio(n_heads: int, d_k: int, d_c: int) -> float:
    """Latent-only compression 2 * n_h * d_k / d_c ([molayo] formal definition, compression ratio)."""
    return 2.0 * n_heads * d_k / d_c
