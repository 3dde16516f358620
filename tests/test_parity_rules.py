"""The comparison rules of tests/parity.py, on the CPU: each rule passes what
the oracle allows and fails a planted mistake.  Mistakes are planted in copies
of the oracle's own outputs; no GPU is involved."""
import numpy as np
import pytest

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W


@pytest.fixture(scope="module")
def tiny():
    spec = W.spec_by_name("tiny")
    xn = W.make_inputs(spec, seed=0).numpy()
    ref = O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                     spec.sm_scale)
    return spec, xn, ref


def _swap_case(spec, xn, ref, q=1):
    """A copy of the oracle's outputs with a tie planted at the boundary of row
    q (the best unselected candidate given the score of the k-th selected
    pool), and the other selection that tie allows, with the oracle's ids and
    attention for it.  (Row 1 of the tiny shape: its boundary score is not 0,
    so the relative rule has a scale.)"""
    r = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
    sel = r["sel"][q][r["sel"][q] >= 0]
    s = r["scores"][q].astype(np.float64)
    b = int(min(sel, key=lambda p: (s[p], -p)))          # the k-th best selected pool
    out_of = [p for p in np.flatnonzero(r["cand"][q]) if p not in set(sel.tolist())]
    c = int(max(out_of, key=lambda p: (s[p], -p)))       # the best pool left out
    r["scores"][q, c] = r["scores"][q, b]
    alt = np.full_like(r["sel"][q], -1)
    keep = np.sort(np.array([p for p in sel if p != b] + [c]))
    alt[:len(keep)] = keep
    expect = PT.oracle_expect(xn, spec, r["pool_start"])
    tok_a, out_a, lse_a = expect(q, alt)
    sel_g, tok_g = r["sel"].copy(), r["tok"].copy()
    out_g = O.f64_to_bf16_bits(r["out_f64"]).copy()
    lse_g = r["lse"].astype(np.float32).copy()
    sel_g[q], tok_g[q] = alt, tok_a
    out_g[q] = O.f64_to_bf16_bits(out_a)
    lse_g[q] = lse_a
    return r, expect, sel_g, tok_g, out_g, lse_g, b, c


def test_equal_chain_passes(tiny):
    spec, xn, ref = tiny
    out_g = O.f64_to_bf16_bits(ref["out_f64"])
    nd = PT.check_chained_rows(ref["sel"], ref["tok"], out_g, ref["lse"].astype(np.float32), ref,
                               PT.oracle_expect(xn, spec, ref["pool_start"]))
    assert nd == 0


def test_boundary_swap_is_checked_end_to_end(tiny):
    spec, xn, ref = tiny
    r, expect, sel_g, tok_g, out_g, lse_g, b, c = _swap_case(spec, xn, ref)
    assert PT.check_chained_rows(sel_g, tok_g, out_g, lse_g, r, expect) == 2
    # the swapped row's ids must be the expansion of its own selection ...
    bad = tok_g.copy()
    bad[1] = ref["tok"][1]
    with pytest.raises(AssertionError, match="swapped selection"):
        PT.check_chained_rows(sel_g, bad, out_g, lse_g, r, expect)
    # ... and its attention the attention over those ids, not the oracle's row
    bad_out = out_g.copy()
    bad_out[1] = O.f64_to_bf16_bits(ref["out_f64"][1])
    with pytest.raises(AssertionError, match="MLA"):
        PT.check_chained_rows(sel_g, tok_g, bad_out, lse_g, r, expect)


def test_swap_away_from_the_boundary_fails(tiny):
    spec, xn, ref = tiny
    # the same swap without the planted tie: the left-out pool scores below b
    # by far more than 1e-5 of b
    _, expect, sel_g, tok_g, out_g, lse_g, b, c = _swap_case(spec, xn, ref)
    s = ref["scores"][1].astype(np.float64)
    assert abs(s[c] - s[b]) > 1e-5 * abs(s[b])
    with pytest.raises(AssertionError, match="away from the boundary"):
        PT.check_chained_rows(sel_g, tok_g, out_g, lse_g, ref, expect)


def test_gap_rule_is_relative_1e5(tiny):
    spec, xn, ref = tiny
    r, expect, sel_g, tok_g, out_g, lse_g, b, c = _swap_case(spec, xn, ref)
    kth = float(r["scores"][1, b])
    assert kth > 0
    for rel, ok in ((0.9e-5, True), (1.1e-5, False)):
        r2 = dict(r)
        r2["scores"] = r["scores"].copy()
        r2["scores"][1, c] = np.float32(kth * (1 - rel))
        got, _ = PT.boundary_ok(sel_g[1], r2["sel"][1], r2["scores"][1], PT.GAP_REL)
        assert got == ok, rel


def test_selection_form(tiny):
    spec, xn, ref = tiny
    out_g = O.f64_to_bf16_bits(ref["out_f64"])
    sel = ref["sel"].copy()
    sel[0, :2] = sel[0, 1::-1]                        # same set, not ascending
    with pytest.raises(AssertionError, match="ascending"):
        PT.check_chained_rows(sel, ref["tok"], out_g, ref["lse"], ref,
                              PT.oracle_expect(xn, spec, ref["pool_start"]))
    sel = ref["sel"].copy()
    sel[0, 0] = -1                                    # a pool dropped: sizes differ
    with pytest.raises(AssertionError):
        PT.check_chained_rows(sel, ref["tok"], out_g, ref["lse"], ref,
                              PT.oracle_expect(xn, spec, ref["pool_start"]))


def test_holes_shape_has_the_cases_it_names():
    """The holes parity shape holds what its GPU tests are meant to cover: an
    invalid pool inside a request, a hole inside a decode tail, and a request
    whose only full pool holds a hole."""
    spec = W.spec_by_name("medium_holes")
    xn = W.make_inputs(spec, seed=0).numpy()
    ref = O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                     spec.sm_scale, always_select_tail=True)
    po = xn["pool_off"]
    inner = [r for r in range(spec.B)
             if np.any(ref["pool_valid"][po[r]:po[r] + ref["n_pools"][r]][1:-1] == 0)]
    assert inner, "no invalid pool inside a request"
    only = [r for r in range(spec.B)
            if ref["n_pools"][r] == 1 and ref["pool_valid"][po[r]] == 0]
    assert only, "no request whose only pool is holed"
    base = spec.select_k * spec.kpool
    tails = ref["tok"][:, base:]
    # a tail with a gap: a -1 slot before a later id is impossible (ids are
    # packed), so look for a tail that skips a row: two ids more than 1 apart
    skipped = [q for q in range(spec.Q) if (tails[q] >= 0).sum() >= 2
               and np.any(np.diff(tails[q][tails[q] >= 0]) > 1)]
    assert skipped, "no tail with a hole"
    # invalid pools are never candidates
    for q in range(spec.Q):
        r = int(xn["q_req"][q])
        pv = ref["pool_valid"][po[r]:po[r] + ref["n_pools"][r]]
        assert not np.any(ref["cand"][q][:len(pv)][pv == 0])


def _online_softmax(xn, spec, tok, rescale=True):
    """The attention as a lazily rebased online softmax over sub-chunks of 32
    ids in selection order (reference maximum moved only when a sub-chunk's
    log2-domain logits exceed it by more than 8), fp64 throughout; with
    rescale=False a moved reference leaves the earlier output and sum as
    they were.  Returns bf16 output bits and lse like the library's call."""
    Q, Hm, L = xn["q_mla"].shape
    out = np.zeros((Q, Hm, L))
    lse = np.full((Q, Hm), -np.inf)
    for q in range(Q):
        ids = tok[q][tok[q] >= 0]
        if len(ids) == 0:
            continue
        r = int(xn["q_req"][q])
        lat = O.latent_rows_f64(xn["ckv"], xn["ckv_scale"], int(xn["kv_off"][r]) + ids)
        x = (O.bf16_bits_to_f64(xn["q_mla"][q]) @ lat.T) * spec.sm_scale / np.log(2.0)
        m = np.full(Hm, -np.inf)
        acc = np.zeros((Hm, L))
        l = np.zeros(Hm)
        for s0 in range(0, len(ids), 32):
            xs = x[:, s0:s0 + 32]
            mloc = xs.max(axis=1)
            move = mloc > m + 8.0
            if rescale:
                a = np.where(move & np.isfinite(m), np.exp2(m - mloc), 1.0)
                acc *= a[:, None]
                l *= a
            m = np.where(move, mloc, m)
            p = np.exp2(xs - m[:, None])
            l += p.sum(axis=1)
            acc += p @ lat[s0:s0 + 32]
        out[q] = acc / l[:, None]
        lse[q] = (m + np.log2(l)) * np.log(2.0)
    return O.f64_to_bf16_bits(out), lse.astype(np.float32)


def test_growing_logits_catch_a_missing_rescale():
    """The GPU growing-logits inputs (tests/test_gpu_mla_rescale.py) separate
    a correct online softmax from one that skips the rescale when its
    reference maximum moves: the first passes the attention tolerance, the
    second fails it."""
    import test_gpu_mla_rescale as G
    spec = W.spec_by_name("medium")
    x = W.make_inputs(spec, seed=11)
    G._growing_rows(x, spec)
    tok = G._ascending_selection(spec, seed=11).numpy()
    xn = x.numpy()
    want = O.sparse_mla_decode(xn["q_mla"], xn["ckv"], xn["ckv_scale"], xn["kv_off"],
                               xn["q_req"], tok, spec.sm_scale)
    good_o, good_l = _online_softmax(xn, spec, tok, rescale=True)
    PT.check_mla(good_o, good_l, want["out_f64"], want["lse"])
    bad_o, bad_l = _online_softmax(xn, spec, tok, rescale=False)
    with pytest.raises(AssertionError):
        PT.check_mla(bad_o, bad_l, want["out_f64"], want["lse"])
