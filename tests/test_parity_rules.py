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
