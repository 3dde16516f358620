"""Comparison rules between the HIP path and the oracle.

* integers (pool starts, validity, counts, candidate flags, selections, token
  ids) must match exactly when the stage is fed the oracle's inputs;
* head-gate: max |diff| <= 1e-5 (fp32 with another summation order; the split-K
  head-gate of stkernel PR #227 measured 2.4e-6);
* pooled keys: at most 1 bf16 ulp apart (fp32 vs fp64 arithmetic before the one
  rounding to bf16), or, for an output near zero where the LayerNorm's
  (x - mean) * rstd * w + b cancels, within KEY_ABS_REL of the row's largest
  |key|: the fp32 evaluation carries an absolute error of a few 2^-24 of the
  row's scale, which is many ulps of a tiny value;
* scores: |diff| <= 1e-5 * max |score| of the row, -inf exactly where the
  oracle has it;
* MLA output: per (query, head) row, max |O - O_ref| / max |O_ref| <= 2e-2
  (bf16 P and bf16 output rounding); lse within 1e-3 absolute;
* top-k, stage-isolated and chained alike: the selection equals the oracle's,
  or every pool in the symmetric difference scores (by the oracle) within
  GAP_REL of the oracle's boundary score b (the k_eff-th best), with the same
  number of pools.  The rule is the same in a chained run: the oracle is never
  fed the GPU's keys or scores.
* a chained row whose selection differs from the oracle's under that rule is
  still checked end to end: it is one of the selections the rule allows, so its
  ids must be the oracle's expansion of it and its attention output the
  oracle's attention over those ids (check_chained_rows).
"""
import numpy as np

import oracle as O

GATE_TOL = 1e-5
KEY_ABS_REL = 2.0 ** -18
SCORE_REL = 1e-5
MLA_REL = 2e-2
LSE_ABS = 1e-3
GAP_REL = 1e-5     # boundary rule: selections may differ only within this gap


def bf16_ulp_diff(a, b):
    """Distance in bf16 ulps between two arrays of bf16 bit patterns."""
    def ordered(x):
        x = np.asarray(x).astype(np.uint16).astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


def check_gate(w_gpu, w_ref):
    d = np.max(np.abs(w_gpu.astype(np.float64) - w_ref.astype(np.float64))) if w_ref.size else 0.0
    assert d <= GATE_TOL, f"head-gate max|diff| {d:.3g} > {GATE_TOL}"
    return d


def check_compress(g, ref, requests=None, pool_off=None):
    """g, ref: dicts of keys/pool_start/pool_valid/n_pools (numpy)."""
    if requests is None:
        sl = slice(None)
        assert np.array_equal(g["n_pools"], ref["n_pools"]), "n_pools"
        idx = np.arange(len(ref["pool_start"]))
    else:
        assert np.array_equal(g["n_pools"][requests], ref["n_pools"][requests]), "n_pools"
        idx = np.concatenate([np.arange(pool_off[r], pool_off[r + 1]) for r in requests])
    assert np.array_equal(g["pool_start"][idx], ref["pool_start"][idx]), "pool_start"
    assert np.array_equal(g["pool_valid"][idx], ref["pool_valid"][idx]), "pool_valid"
    kg, kr = g["keys"][idx], ref["keys"][idx]
    u = bf16_ulp_diff(kg, kr)
    if u.max(initial=0) > 1:
        fg, fr = O.bf16_bits_to_f64(kg), O.bf16_bits_to_f64(kr)
        scale = np.abs(fr).max(axis=1, keepdims=True)
        far = (u > 1) & (np.abs(fg - fr) > KEY_ABS_REL * scale)
        i, j = np.unravel_index(np.argmax(u), u.shape)
        print(f"[keys] {int((u > 1).sum())} elements > 1 ulp; worst {int(u[i, j])} ulps: "
              f"gpu {fg[i, j]:.6g} ref {fr[i, j]:.6g} row max {scale[i, 0]:.4g}")
        assert not far.any(), f"{int(far.sum())} key elements beyond 1 ulp and {KEY_ABS_REL:.2g} of the row"
    return int((u > 0).sum())


def check_scores(s_gpu, c_gpu, s_ref, c_ref, rows=None):
    rows = range(s_ref.shape[0]) if rows is None else rows
    worst = 0.0
    for q in rows:
        assert np.array_equal(c_gpu[q], c_ref[q]), f"cand row {q}"
        fin = np.isfinite(s_ref[q])
        assert np.array_equal(np.isfinite(s_gpu[q]), fin), f"-inf pattern row {q}"
        if fin.any():
            scale = max(np.abs(s_ref[q][fin]).max(), 1e-30)
            d = np.abs(s_gpu[q][fin].astype(np.float64) - s_ref[q][fin]).max() / scale
            worst = max(worst, d)
            assert d <= SCORE_REL, f"scores row {q}: rel diff {d:.3g}"
    return worst


def boundary_ok(sel_g, sel_r, s_ref, rel):
    """Selections equal, or every disagreeing pool scores within rel of the
    oracle's k-th score."""
    a = set(int(x) for x in sel_g if x >= 0)
    b = set(int(x) for x in sel_r if x >= 0)
    if a == b:
        return True, 0
    if len(a) != len(b):
        return False, len(a ^ b)
    kth = min(float(s_ref[p]) for p in b)
    finite = s_ref[np.isfinite(s_ref)]
    tol = rel * max(abs(kth), 1e-6 * np.abs(finite).max())
    ok = all(abs(float(s_ref[p]) - kth) <= tol for p in a ^ b)
    return ok, len(a ^ b)


def check_sel_form(sel_row):
    """A selection row is strictly ascending pool ids followed by -1s."""
    sel_row = np.asarray(sel_row)
    n = int((sel_row >= 0).sum())
    assert np.all(sel_row[:n] >= 0) and np.all(sel_row[n:] == -1), "-1 before a pool id"
    assert np.all(np.diff(sel_row[:n]) > 0), "selection not strictly ascending"


def oracle_expect(xo, spec, pool_start):
    """expect(q, sel_row) for check_chained_rows: the oracle's expansion (with
    the tail when the shape has always_select_tail) and attention for
    selection sel_row of query q, on the oracle inputs ``xo`` and the oracle's
    pool starts."""
    def expect(q, sel_row):
        qq = np.array([q])
        q_req = np.asarray(xo["q_req"])[qq]
        tok = O.expand_selection(np.asarray(sel_row)[None], pool_start, xo["pool_off"], q_req,
                                 spec.kpool, spec.out_width)
        if spec.always_select_tail:
            tok = O.select_tail(tok, xo["valid"], xo["tok_off"], q_req, np.asarray(xo["q_pos"])[qq],
                                spec.kpool, spec.select_k)
        att = O.sparse_mla_decode(np.asarray(xo["q_mla"])[qq], xo["ckv"], xo.get("ckv_scale"),
                                  xo["kv_off"], q_req, tok, spec.sm_scale)
        return tok[0], att["out_f64"][0], att["lse"][0]
    return expect


def check_chained_rows(sel_g, tok_g, out_g, lse_g, ref, expect, rows=None):
    """The chained rule for the selection, ids and attention of each row.

    The selection must satisfy the boundary rule (GAP_REL) against the
    oracle's.  Where it equals the oracle's, ids are exact and the attention
    is compared with the oracle's.  Where it differs (a boundary swap), it is
    one of the selections the rule allows: its ids must equal expect(q, sel)[0]
    exactly and its attention expect's attention.  Returns the number of
    pools swapped over all rows."""
    rows = range(ref["sel"].shape[0]) if rows is None else rows
    swapped = 0
    for q in rows:
        check_sel_form(sel_g[q])
        ok, nd = boundary_ok(sel_g[q], ref["sel"][q], ref["scores"][q], GAP_REL)
        assert ok, f"selection row {q}: {nd} pools differ away from the boundary"
        if nd == 0:
            assert np.array_equal(tok_g[q], ref["tok"][q]), f"ids row {q}"
            check_mla(out_g, lse_g, ref["out_f64"], ref["lse"], rows=[q])
        else:
            swapped += nd
            tok_e, out_e, lse_e = expect(q, sel_g[q])
            assert np.array_equal(tok_g[q], tok_e), f"ids row {q} (swapped selection)"
            check_mla(np.asarray(out_g)[q:q + 1], np.asarray(lse_g)[q:q + 1], out_e[None],
                      lse_e[None])
    return swapped


def check_sel_exact(sel_g, sel_r, rows=None):
    rows = range(sel_r.shape[0]) if rows is None else rows
    for q in rows:
        assert np.array_equal(sel_g[q], sel_r[q]), f"sel row {q}"
        v = sel_g[q][sel_g[q] >= 0]
        assert np.all(np.diff(v) > 0), "selection not strictly ascending"


def check_mla(out_g_bits, lse_g, out_ref_f64, lse_ref, rows=None):
    og = O.bf16_bits_to_f64(out_g_bits)
    rows = range(out_ref_f64.shape[0]) if rows is None else rows
    worst = 0.0
    for q in rows:
        for h in range(out_ref_f64.shape[1]):
            ref = out_ref_f64[q, h]
            m = np.abs(ref).max()
            if m == 0:
                assert np.all(og[q, h] == 0), f"empty row q={q} h={h} not zero"
                assert np.isneginf(lse_g[q, h]) and np.isneginf(lse_ref[q, h])
                continue
            d = np.abs(og[q, h] - ref).max() / m
            worst = max(worst, d)
            assert d <= MLA_REL, f"MLA q={q} h={h}: rel err {d:.3g}"
            assert abs(float(lse_g[q, h]) - lse_ref[q, h]) <= LSE_ABS, f"lse q={q} h={h}"
    return worst
