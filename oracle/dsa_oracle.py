"""fp64 CPU oracle of the DSA decode path.  TEST INFRASTRUCTURE ONLY: imported
by the tests, the package smoke check and the bench's CPU-baseline leg, never
by the product path.  It shares no code with the HIP library.

Sources, cited by page title and section:

* [Atlas DSA page] -- the ``spark_model/layers/glm5next_dsa/mod.rs`` page of
  the Atlas docs: sections "Shape of the pipeline", "Traps carried from Slice
  8", the ``MASKED_ATTN_MAX_KEYS`` note, and the ``Glm5NextDsaConfig`` methods
  ``select_k``, ``out_width``, ``kv_cache_dim``, ``validate``.
* [PR 227 page] -- stkernel pull request #227, "indexer fp32 head-gate
  split-K": the head-gate is ``hidden.float() @ W_fp32``, [M,4096]x[4096,16].

Readings of points the pages leave open (each repeated where it is used):

* ape is an additive per-slot, per-channel bias on the gate logits, applied
  before the slot softmax.
* pooling and the LayerNorm are done without an intermediate rounding; the
  LayerNorm output is rounded once to bf16 (round to nearest even).
* pool "indices" are the request-local position of each pool's first row.
* a pool with any invalid slot keeps its position and is flagged invalid.
* the index score of pool p for query q is  sum_h w[q,h] * relu(<qi[q,h], key[p]>)
  with no scale and no bias; w is the raw head-gate output.
* pool p is a candidate for query q iff it is a full pool of q's request, it is
  valid, and its last row is at or before the query position.
* the pool top-k keeps the min(select_k, #candidates) best candidates, ties to
  the lower pool id, and lists them by ascending pool id; the rest is -1.
* an empty selection row gives O = 0 and lse = -inf.
* fp8 latent rows are OCP E4M3FN codes times one f32 scale per row.
* a paged latent cache is a pool of equal pages; a [B, max_blocks] block
  table names the page of each request's block of page_rows logical rows.
* a request's region may hold more rows than its live length; only the live
  rows exist for the step.  A decode step's query sits at the newest live row,
  and the step writes that row (its indexer row stored at a device-side
  position and marked valid).
* k_norm may instead be applied to each row when it is stored (the per-token
  k_normed buffer); the pooled row then gets no LayerNorm.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (any 16-bit integer dtype) -> float64, exactly."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 to bf16 (8 significant bits) to nearest, ties to even, in a
    single rounding step; returns the uint16 bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(x)                       # |x| = m * 2**e, 0.5 <= m < 1
        q = np.maximum(e - 8, -133)              # quantum; 2**-133 is bf16's smallest step
        r = np.rint(np.ldexp(x, -q))             # exact power-of-two scaling, RNE
        y = np.ldexp(r, q).astype(np.float32)    # representable, or +-inf on overflow
    bits = (y.view(np.uint32) >> 16).astype(np.uint16)
    out[...] = bits
    out[nan] = 0x7FC0
    return out


def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """OCP FP8 E4M3FN codes -> float64: 1 sign, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# ---------------------------------------------------------------------------
# configuration helpers  [Atlas DSA page, Glm5NextDsaConfig methods]
# ---------------------------------------------------------------------------


def select_k(index_topk: int, kpool: int, n_pools: int) -> int:
    """Pools selected per query: the pool budget index_topk / kpool, capped by
    the number of pools."""
    return min(index_topk // kpool, n_pools)


def out_width(index_topk: int, kpool: int, always_select_tail: bool) -> int:
    """Width of one emitted token-id row; the optional tail adds kpool-1 slots."""
    return index_topk + (kpool - 1 if always_select_tail else 0)


# ---------------------------------------------------------------------------
# a1: head gate  [PR 227 page]
# ---------------------------------------------------------------------------


def head_gate(hidden: np.ndarray, W: np.ndarray) -> np.ndarray:
    """w = hidden @ W for fp32 operands [M,K] x [K,N]; exact products and sums
    in float64, one rounding to float32 at the end."""
    return (hidden.astype(np.float64) @ W.astype(np.float64)).astype(np.float32)


# ---------------------------------------------------------------------------
# a2: pool geometry and gated pool compression  [Atlas DSA page, Traps]
# ---------------------------------------------------------------------------


def request_rows(tok_off, r: int, seq_len=None) -> tuple:
    """The cache rows of request r: [tok_off[r], tok_off[r] + T_r) with T_r the
    live length seq_len[r] when given (a request's region may hold more rows
    than it has written), else the whole region up to tok_off[r+1]."""
    lo = int(tok_off[r])
    hi = int(tok_off[r + 1])
    if seq_len is not None:
        assert 0 <= int(seq_len[r]) <= hi - lo, "live length outside the request's region"
        hi = lo + int(seq_len[r])
    return lo, hi


def kpool_geometry(valid: np.ndarray, tok_off: np.ndarray, kpool: int, seq_len=None):
    """Per request r: the first valid row f_r (request-local; -1 if none) and the
    number of full pools P_r = floor((T_r - f_r) / kpool).  Pooling starts at the
    first valid row, so left padding is skipped; the rows after the last full
    pool (a trailing partial pool) form no pool."""
    B = len(tok_off) - 1
    first = np.full(B, -1, dtype=np.int64)
    n_pools = np.zeros(B, dtype=np.int64)
    for r in range(B):
        lo, hi = request_rows(tok_off, r, seq_len)
        v = valid[lo:hi]
        nz = np.flatnonzero(v)
        if len(nz):
            first[r] = nz[0]
            n_pools[r] = (len(v) - nz[0]) // kpool
    return first, n_pools


def slot_weights(gate_rows: np.ndarray, ape: np.ndarray) -> np.ndarray:
    """Slot weights of pools: gate_rows [P, kpool, D] and ape [kpool, D] (both
    float64) -> alpha [P, kpool, D], a softmax over the slot axis taken
    separately for every channel (not over channels, not over pools)."""
    g = gate_rows + ape[None, :, :]
    g = g - g.max(axis=1, keepdims=True)
    e = np.exp(g)
    return e / e.sum(axis=1, keepdims=True)


def kpool_compress(k, gate, ape, valid, tok_off, pool_off, ln_w, ln_b, eps, kpool,
                   new_from: Optional[np.ndarray] = None, prev: Optional[dict] = None,
                   requests: Optional[Iterable[int]] = None, seq_len=None) -> dict:
    """Gated pool compression followed by k_norm.

    For request r with first valid row f and P full pools, pool p covers the
    rows f + p*kpool ... f + p*kpool + kpool - 1.  Per channel c:
    x_c = sum_s alpha[s,c] * k[row_s, c] with alpha the slot softmax of
    gate + ape; key = LayerNorm(x) * ln_w + ln_b (mean subtracted, biased
    variance, with bias -- an nn.LayerNorm, not an RMSNorm), rounded once to
    bf16.  pool_start = f + p*kpool (request-local); pool_valid = every slot
    valid.  Slots [P, cap) of the request's pool range are written as
    start -1, valid 0, key 0.

    new_from [B] (optional, the incremental form used by a decode step that
    appended rows): only the pools holding a row at position >= new_from[r],
    p in [floor((new_from[r] - f)/kpool), P), are recomputed; every other slot
    (sentinels included) is copied from ``prev``.  ``requests`` limits the
    work to some requests (the others are left as they are), for sampled
    checks at full size.  ``seq_len`` [B] (optional) is each request's live
    length (request_rows).

    ln_w = ln_b = None is the per-token k_normed reading: the rows were
    normalised when they were stored (indexer_store with a LayerNorm), so the
    pooled value is rounded to bf16 with no LayerNorm after it."""
    k = np.asarray(k)
    gate = np.asarray(gate)
    D = k.shape[1]
    B = len(tok_off) - 1
    ncap = int(pool_off[-1])
    if prev is not None:
        keys = prev["keys"].copy()
        start = prev["pool_start"].copy()
        pvalid = prev["pool_valid"].copy()
    else:
        keys = np.zeros((ncap, D), dtype=np.uint16)
        start = np.full(ncap, -1, dtype=np.int32)
        pvalid = np.zeros(ncap, dtype=np.uint8)
    first, n_pools = kpool_geometry(valid, tok_off, kpool, seq_len)
    ape64 = bf16_bits_to_f64(ape)
    post_ln = ln_w is not None
    if post_ln:
        lw = np.asarray(ln_w, dtype=np.float64)
        lb = np.asarray(ln_b, dtype=np.float64)
    reqs = range(B) if requests is None else requests
    for r in reqs:
        cap = int(pool_off[r + 1] - pool_off[r])
        P = int(n_pools[r])
        f = int(first[r])
        assert P <= cap, "pool capacity below the number of full pools"
        base = int(pool_off[r])
        p_from = 0
        if new_from is None:
            keys[base + P:base + cap] = 0          # sentinel slots past the full pools
            start[base + P:base + cap] = -1
            pvalid[base + P:base + cap] = 0
        elif P > 0 and new_from[r] >= f:
            p_from = min(P, (int(new_from[r]) - f) // kpool)
        if P <= p_from:
            continue
        p = np.arange(p_from, P)
        rows = int(tok_off[r]) + f + p[:, None] * kpool + np.arange(kpool)[None, :]
        alpha = slot_weights(bf16_bits_to_f64(gate[rows]), ape64)       # [n, kpool, D]
        x = (alpha * bf16_bits_to_f64(k[rows])).sum(axis=1)           # [n, D]
        if post_ln:
            mu = x.mean(axis=1, keepdims=True)
            var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
            y = (x - mu) / np.sqrt(var + eps) * lw[None, :] + lb[None, :]
        else:
            y = x
        keys[base + p_from:base + P] = f64_to_bf16_bits(y)
        start[base + p_from:base + P] = f + p * kpool
        pvalid[base + p_from:base + P] = np.asarray(valid)[rows].astype(bool).all(axis=1)
    return {"keys": keys, "pool_start": start, "pool_valid": pvalid,
            "n_pools": n_pools.astype(np.int32)}


# ---------------------------------------------------------------------------
# the cache-write side  [Atlas DSA page, Glm5NextDsaKernels: indexer_store and
# write_geom]
# ---------------------------------------------------------------------------


def layer_norm_rows(x, ln_w, ln_b, eps: float) -> np.ndarray:
    """k_norm of rows (float64): an nn.LayerNorm with a bias, biased variance."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(ln_w, np.float64) + np.asarray(ln_b, np.float64)


def indexer_store(k, gate, valid, tok_off, pos, k_new, gate_new, ln_w=None, ln_b=None,
                  eps: float = 1e-5) -> dict:
    """Place each request's staged indexer row at its device-side position:
    row tok_off[r] + pos[r] of k and gate receives k_new[r] and gate_new[r],
    and that row is marked valid.  With ln_w / ln_b (the per-token k_normed
    reading of the page's k_normed buffer) the stored k row is k_norm of the
    staged row, rounded once to bf16.  A position outside the request's region
    (negative, or at or past tok_off[r+1]) stores nothing.  Returns new
    arrays; the inputs are not modified."""
    k = np.array(k, copy=True)
    gate = np.array(gate, copy=True)
    valid = np.array(valid, copy=True)
    for r in range(len(tok_off) - 1):
        p = int(pos[r])
        if p < 0 or int(tok_off[r]) + p >= int(tok_off[r + 1]):
            continue
        row = int(tok_off[r]) + p
        if ln_w is None:
            k[row] = k_new[r]
        else:
            k[row] = f64_to_bf16_bits(layer_norm_rows(bf16_bits_to_f64(k_new[r]), ln_w, ln_b, eps))
        gate[row] = gate_new[r]
        valid[row] = 1
    return {"k": k, "gate": gate, "valid": valid}


def write_geom(seq_len, block_table=None, page_rows: Optional[int] = None) -> dict:
    """The decode step's geometry from the live lengths, one query per
    request: q_req[r] = r; q_pos[r] = seq_len[r] - 1 (the newest row; -1 for an
    empty request, which then has no candidate and no tail); new_from[r] = the
    row this step writes (max(seq_len[r] - 1, 0)), from which the incremental
    compression recomputes; slot[r] = the physical latent row of position
    seq_len[r] - 1 under the block table (paged_rows), -1 for an empty request."""
    n = np.asarray(seq_len, dtype=np.int64)
    B = len(n)
    out = {"q_req": np.arange(B, dtype=np.int32), "q_pos": (n - 1).astype(np.int32),
           "new_from": np.maximum(n - 1, 0).astype(np.int32)}
    if block_table is not None:
        slot = np.full(B, -1, dtype=np.int64)
        for r in range(B):
            if n[r] > 0:
                slot[r] = paged_rows(block_table, page_rows, r, n[r] - 1)
        out["slot"] = slot
    return out


# ---------------------------------------------------------------------------
# a3: index scores  [Atlas DSA page, Shape of the pipeline]
# ---------------------------------------------------------------------------


def index_scores(qi, w, keys, pool_start, pool_valid, pool_off, n_pools, q_req, q_pos,
                 kpool: int, pstride: int, queries: Optional[Iterable[int]] = None):
    """[Q, pstride] scores plus candidate validity.

    score[q,p] = sum_h w[q,h] * relu(<qi[q,h,:], key[p,:]>) over the request's
    pools, computed in float64 and rounded once to float32 (a -0 result is
    stored as +0).  Pool p is a candidate iff p < n_pools[r], pool_valid, and
    pool_start + kpool - 1 <= q_pos[q]; a non-candidate scores -inf with
    cand = 0, and so does every slot past the request's pools."""
    Q = len(q_req)
    scores = np.full((Q, pstride), -np.inf, dtype=np.float32)
    cand = np.zeros((Q, pstride), dtype=np.uint8)
    qs = range(Q) if queries is None else queries
    for q in qs:
        r = int(q_req[q])
        P = int(n_pools[r])
        if P == 0:
            continue
        base = int(pool_off[r])
        K = bf16_bits_to_f64(keys[base:base + P])                       # [P, D]
        dots = bf16_bits_to_f64(qi[q]) @ K.T                             # [H, P]
        s = (np.asarray(w[q], dtype=np.float64)[:, None] * np.maximum(dots, 0.0)).sum(axis=0)
        ok = (np.asarray(pool_valid[base:base + P]) != 0) & \
             (np.asarray(pool_start[base:base + P]).astype(np.int64) + kpool - 1 <= int(q_pos[q]))
        s32 = s.astype(np.float32)
        s32[s32 == 0] = 0.0
        scores[q, :P] = np.where(ok, s32, -np.inf)
        cand[q, :P] = ok
    return scores, cand


# ---------------------------------------------------------------------------
# a4: pool top-k
# ---------------------------------------------------------------------------


def topk_pools(scores, cand, select_k_: int, queries: Optional[Iterable[int]] = None,
               row_len=None):
    """[Q, select_k] pool ids: the k_eff = min(select_k, #candidates)
    candidates ranked first by (score descending, pool id ascending), listed in
    ascending pool id; the remaining slots are -1.  Selection is a set (the
    attention is set membership), so the ascending list is its canonical form.
    row_len [Q] (optional): only the first row_len[q] entries of row q count
    (clamped to [0, row width])."""
    Q = scores.shape[0]
    sel = np.full((Q, select_k_), -1, dtype=np.int32)
    qs = range(Q) if queries is None else queries
    for q in qs:
        n = scores.shape[1] if row_len is None else min(max(int(row_len[q]), 0), scores.shape[1])
        ids = np.flatnonzero(cand[q][:n])
        if len(ids) == 0:
            continue
        s = scores[q, ids].astype(np.float64)
        order = np.lexsort((ids, -s))          # last key is primary: score desc, then id asc
        k_eff = min(select_k_, len(ids))
        sel[q, :k_eff] = np.sort(ids[order[:k_eff]])
    return sel


# ---------------------------------------------------------------------------
# a5: selection expansion  [Atlas DSA page, Traps: fully written -1 sentinel]
# ---------------------------------------------------------------------------


def expand_selection(sel, pool_start, pool_off, q_req, kpool: int, out_width_: int):
    """tok[q, j*kpool + s] = pool_start[sel[q,j]] + s for a selected pool j,
    -1 where sel is -1 and in every slot past select_k*kpool; every element
    of the [Q, out_width] row is written."""
    Q, K = sel.shape
    tok = np.full((Q, out_width_), -1, dtype=np.int32)
    for q in range(Q):
        base = int(pool_off[int(q_req[q])])
        for j in np.flatnonzero(sel[q] >= 0):
            st = int(pool_start[base + int(sel[q, j])])
            tok[q, j * kpool:(j + 1) * kpool] = st + np.arange(kpool)
    return tok


def select_tail(tok, valid, tok_off, q_req, q_pos, kpool: int, select_k_: int):
    """always_select_tail  [Atlas DSA page, Glm5NextDsaConfig::out_width: the
    tail adds kpool - 1 slots to the emitted row].

    For a query at request-local position t of request r, with first valid row
    f: the pools that are candidates for it are the full pools ending at or
    before t, P_t = floor((t + 1 - f) / kpool) of them; the rows after them up
    to t, f + P_t*kpool .. t (fewer than kpool rows), are the query's tail.
    Its valid rows, in ascending order, go to the slots select_k*kpool,
    select_k*kpool + 1, ...; the other tail slots are -1.  Nothing else of the
    row changes.  A query before f has no tail."""
    tok = np.array(tok, dtype=np.int32, copy=True)
    first, _ = kpool_geometry(valid, tok_off, kpool)
    base = select_k_ * kpool
    tok[:, base:base + kpool - 1] = -1
    for q in range(tok.shape[0]):
        r = int(q_req[q])
        f, t = int(first[r]), int(q_pos[q])
        if f < 0 or t < f:
            continue
        lo = f + ((t + 1 - f) // kpool) * kpool
        rows = [x for x in range(lo, t + 1) if valid[int(tok_off[r]) + x]]
        assert len(rows) <= kpool - 1
        tok[q, base:base + len(rows)] = rows
    return tok


# ---------------------------------------------------------------------------
# a6: NoPE MLA over the selected tokens  [Atlas DSA page, Traps (NoPE) and the
# MASKED_ATTN_MAX_KEYS note: a per-row gather equals the dense set-membership
# mask]
# ---------------------------------------------------------------------------


def latent_rows_f64(ckv, ckv_scale, rows) -> np.ndarray:
    """Decode latent rows: bf16 bits, or fp8-e4m3 codes times the row scale."""
    if ckv_scale is None:
        return bf16_bits_to_f64(ckv[rows])
    return fp8_e4m3_to_f64(ckv[rows]) * np.asarray(ckv_scale, dtype=np.float64)[rows][:, None]


def sparse_mla_decode(q, ckv, ckv_scale, kv_off, q_req, tok, sm_scale: float,
                      queries: Optional[Iterable[int]] = None,
                      heads: Optional[Iterable[int]] = None) -> dict:
    """For every query q and head h, over the selected ids j (tok >= 0), with
    row = kv_off[r] + tok[q,j] and c = the latent row (qk_rope_head_dim = 0,
    so keys and values are both the kv_lora-wide latent):
    l_j = sm_scale * <Q[q,h], c_j>, O = sum_j softmax(l)_j c_j, lse = log sum_j
    exp l_j.  O is rounded once to bf16; an empty row gives O = 0, lse = -inf."""
    tok = np.asarray(tok)
    base = np.asarray(kv_off, dtype=np.int64)[np.asarray(q_req, dtype=np.int64)]
    rows = np.where(tok >= 0, base[:, None] + tok.astype(np.int64), -1)
    return attend_rows(q, ckv, ckv_scale, rows, sm_scale, queries, heads)


def paged_rows(block_table, page_rows: int, r: int, t) -> np.ndarray:
    """Physical cache row of request r's logical positions t in a paged latent
    cache (the block-table paged decode of the Atlas DSA page's
    MASKED_ATTN_MAX_KEYS note): the cache is a pool of pages of page_rows rows;
    block b = t // page_rows of request r sits in physical page
    block_table[r, b], at row t % page_rows of it.  Reading: block_table is
    [B, max_blocks] row-major, page ids index pages from the start of the
    cache."""
    t = np.asarray(t, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[r, t // page_rows] * page_rows + t % page_rows


def kv_index(tok, q_req, block_table, page_rows: int) -> np.ndarray:
    """The physical index row of every query (the page's step taps keep the
    logical selection and the physical indices apart): paged_rows of each
    selected id, -1 where tok is -1."""
    tok = np.asarray(tok)
    out = np.full(tok.shape, -1, dtype=np.int64)
    for qq in range(tok.shape[0]):
        sel = tok[qq] >= 0
        out[qq, sel] = paged_rows(block_table, page_rows, int(q_req[qq]), tok[qq, sel])
    return out


def sparse_mla_decode_paged(q, ckv, ckv_scale, block_table, page_rows: int, q_req, tok,
                            sm_scale: float, queries: Optional[Iterable[int]] = None,
                            heads: Optional[Iterable[int]] = None) -> dict:
    """sparse_mla_decode over a paged latent cache: the selected logical ids
    are mapped to physical rows through the block table (kv_index), then the
    same attention.  Also returns the physical index rows as "kvidx"."""
    rows = kv_index(tok, q_req, block_table, page_rows)
    res = attend_rows(q, ckv, ckv_scale, rows, sm_scale, queries, heads)
    res["kvidx"] = rows
    return res


def attend_rows(q, ckv, ckv_scale, rows, sm_scale: float,
                queries: Optional[Iterable[int]] = None,
                heads: Optional[Iterable[int]] = None) -> dict:
    """The attention of sparse_mla_decode over explicit cache rows: rows[q, j]
    is a row of ckv, or -1 for no token."""
    Q, Hm, L = q.shape
    out64 = np.zeros((Q, Hm, L), dtype=np.float64)
    lse = np.full((Q, Hm), -np.inf, dtype=np.float64)
    qs = range(Q) if queries is None else queries
    hs = np.arange(Hm) if heads is None else np.asarray(list(heads))
    for qq in qs:
        t = np.asarray(rows[qq])
        t = t[t >= 0]
        if len(t) == 0:
            continue
        assert len(np.unique(t)) == len(t), "duplicate rows in one selection row"
        C = latent_rows_f64(ckv, ckv_scale, t.astype(np.int64))                    # [n, L]
        Qh = bf16_bits_to_f64(q[qq][hs])                                           # [h, L]
        logits = sm_scale * (Qh @ C.T)                                             # [h, n]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        z = e.sum(axis=1, keepdims=True)
        out64[qq, hs] = (e @ C) / z
        lse[qq, hs] = (m + np.log(z))[:, 0]
    return {"out": f64_to_bf16_bits(out64), "out_f64": out64, "lse": lse}


# ---------------------------------------------------------------------------
# the whole chain
# ---------------------------------------------------------------------------


def dsa_step(x: dict, kpool: int, select_k_: int, out_width_: int, pstride: int,
             eps: float, sm_scale: float, new_from=None, prev=None,
             queries: Optional[Iterable[int]] = None, always_select_tail: bool = False,
             seq_len=None, post_ln: bool = True) -> dict:
    """One pass of the whole path on the numpy arrays of one input set, in the
    order of the pipeline diagram: head gate, compression, scores, top-k,
    expansion (with the tail when always_select_tail), sparse MLA.
    ``queries`` restricts the per-query stages (and the compression to those
    queries' requests).  ``seq_len``: live lengths (request_rows);
    ``post_ln=False``: the k rows were normalised when stored, so the
    compression applies no LayerNorm."""
    qlist = None if queries is None else list(queries)
    reqs = None if qlist is None else sorted({int(x["q_req"][q]) for q in qlist})
    w = head_gate(x["hidden"], x["W"])
    comp = kpool_compress(x["k"], x["gate"], x["ape"], x["valid"], x["tok_off"], x["pool_off"],
                          x["ln_w"] if post_ln else None, x["ln_b"] if post_ln else None, eps,
                          kpool, new_from=new_from, prev=prev, requests=reqs, seq_len=seq_len)
    scores, cand = index_scores(x["qi"], w, comp["keys"], comp["pool_start"], comp["pool_valid"],
                                x["pool_off"], comp["n_pools"], x["q_req"], x["q_pos"], kpool,
                                pstride, queries=qlist)
    sel = topk_pools(scores, cand, select_k_, queries=qlist)
    tok = expand_selection(sel, comp["pool_start"], x["pool_off"], x["q_req"], kpool, out_width_)
    if always_select_tail:
        tok = select_tail(tok, x["valid"], x["tok_off"], x["q_req"], x["q_pos"], kpool, select_k_)
    mla = sparse_mla_decode(x["q_mla"], x["ckv"], x.get("ckv_scale"), x["kv_off"], x["q_req"],
                            tok, sm_scale, queries=qlist)
    return {"w": w, **comp, "scores": scores, "cand": cand, "sel": sel, "tok": tok, **mla}
