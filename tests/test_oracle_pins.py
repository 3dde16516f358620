"""Pins of the CPU oracle against facts fixed outside it: hand-worked examples
(tests/golden), closed forms, library routines for special cases, and brute
force on tiny inputs.  Each is chosen so that a plausible slip in the oracle
(softmax over the wrong axis, RMSNorm instead of LayerNorm, a dropped bias,
relu in the wrong place, a transposed operand, an off-by-one at the causal
boundary, a wrong tie order) fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def bf16(x):
    """float32 -> bf16 bits with torch's own conversion (round to nearest even)."""
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_on_f32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40])])
    x = x.astype(np.float32)
    assert np.array_equal(O.f64_to_bf16_bits(x.astype(np.float64)), bf16(x))


def test_bf16_rounding_halfway_and_single_rounding():
    # 1 + 2^-8 is halfway between 1 (0x3F80) and 1 + 2^-7 (0x3F81): ties to even.
    assert O.f64_to_bf16_bits(1 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 0x3F81 and 0x3F82: ties to even -> 0x3F82.
    assert O.f64_to_bf16_bits(1 + 3 * 2.0 ** -8) == 0x3F82
    # Just above halfway must round up; rounding through float32 first would not.
    assert O.f64_to_bf16_bits(1 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert O.f64_to_bf16_bits(-(1 + 2.0 ** -8 + 2.0 ** -30)) == 0xBF81
    assert np.all(O.bf16_bits_to_f64(np.uint16([0x3F80, 0xC000, 0x0001])) ==
                  np.array([1.0, -2.0, 2.0 ** -133]))


def test_fp8_e4m3_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = O.fp8_e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert O.fp8_e4m3_to_f64(np.uint8([0x7E]))[0] == 448.0      # largest finite
    assert O.fp8_e4m3_to_f64(np.uint8([0x01]))[0] == 2.0 ** -9  # smallest subnormal


# ---------------------------------------------------------------------------
# configuration rules
# ---------------------------------------------------------------------------

def test_config_rules_from_page():
    g = gold("config_rules.json")
    for c in g["select_k"]:
        assert O.select_k(c["index_topk"], c["kpool"], c["n_pools"]) == c["expect"]
    for c in g["out_width"]:
        assert O.out_width(c["index_topk"], c["kpool"], c["tail"]) == c["expect"]


# ---------------------------------------------------------------------------
# a1 head gate
# ---------------------------------------------------------------------------

def test_head_gate_brute_force_and_one_hot():
    rng = np.random.default_rng(2)
    h = rng.integers(-8, 8, (3, 5)).astype(np.float32)
    W = rng.integers(-8, 8, (5, 2)).astype(np.float32)
    got = O.head_gate(h, W)
    for m in range(3):
        for n in range(2):
            acc = 0.0
            for k in range(5):
                acc += float(h[m, k]) * float(W[k, n])
            assert got[m, n] == acc
    # a one-hot row of hidden picks the matching row of W (catches W.T)
    W2 = rng.standard_normal((6, 4)).astype(np.float32)
    e = np.zeros((1, 6), np.float32)
    e[0, 3] = 1.0
    assert np.array_equal(O.head_gate(e, W2)[0], W2[3])


# ---------------------------------------------------------------------------
# a2 geometry and compression
# ---------------------------------------------------------------------------

def _compress(k_f32, gate_f32, ape_f32, valid, kpool, ln_w, ln_b, eps=1e-5, caps=None, tok_off=None,
              new_from=None, prev=None):
    T, D = k_f32.shape
    tok_off = np.array([0, T], np.int32) if tok_off is None else np.asarray(tok_off, np.int32)
    if caps is None:
        caps = [(tok_off[r + 1] - tok_off[r]) // kpool for r in range(len(tok_off) - 1)]
    pool_off = np.concatenate([[0], np.cumsum(caps)]).astype(np.int32)
    return O.kpool_compress(bf16(k_f32), bf16(gate_f32), bf16(ape_f32), np.asarray(valid, np.uint8),
                            tok_off, pool_off, np.float32(ln_w), np.float32(ln_b), eps, kpool,
                            new_from=new_from, prev=prev), pool_off


def test_geometry_tiny_golden():
    g = gold("geometry_tiny.json")
    valid = np.ones(g["T"], np.uint8)
    valid[:g["pad"]] = 0
    first, n = O.kpool_geometry(valid, np.array([0, g["T"]]), g["kpool"])
    assert first[0] == g["first"] and n[0] == g["n_pools"]
    rng = np.random.default_rng(3)
    D = 8
    out, _ = _compress(rng.standard_normal((g["T"], D)), rng.standard_normal((g["T"], D)),
                       rng.standard_normal((g["kpool"], D)), valid, g["kpool"], np.ones(D), np.zeros(D))
    assert list(out["pool_start"][:g["n_pools"]]) == g["pool_starts"]
    assert np.all(out["pool_valid"][:g["n_pools"]] == 1)
    # capacity 128 // 4 = 32 slots: the two past the 30 pools are sentinels
    assert list(out["pool_start"][g["n_pools"]:]) == [-1, -1]
    assert np.all(out["keys"][g["n_pools"]:] == 0)
    # the dropped rows influence nothing: changing them leaves every key equal
    k2 = rng.standard_normal((g["T"], D))
    k3 = k2.copy()
    k3[g["dropped_rows"]] += 100.0
    a, _ = _compress(k2, np.zeros((g["T"], D)), np.zeros((g["kpool"], D)), valid, g["kpool"], np.ones(D), np.zeros(D))
    b, _ = _compress(k3, np.zeros((g["T"], D)), np.zeros((g["kpool"], D)), valid, g["kpool"], np.ones(D), np.zeros(D))
    assert np.array_equal(a["keys"], b["keys"])


def test_compress_worked_example_golden():
    g = gold("compress_worked.json")
    k = np.array(g["k"], np.float32)
    D = k.shape[1]
    out, _ = _compress(k, np.zeros_like(k), np.zeros((2, D)), np.ones(2), g["kpool"],
                       g["ln_w"], g["ln_b"], eps=g["eps"])
    expect = np.array([eval(e, {"sqrt": math.sqrt}) for e in g["key"]])
    assert np.array_equal(out["keys"][0], O.f64_to_bf16_bits(expect))


def test_slot_softmax_sums_to_one_per_channel():
    rng = np.random.default_rng(4)
    g = rng.standard_normal((50, 8, 16)) * 3
    a = O.slot_weights(g, rng.standard_normal((8, 16)))
    assert np.max(np.abs(a.sum(axis=1) - 1.0)) < 1e-12
    assert np.all(a > 0)


def test_softmax_runs_over_slots_per_channel():
    # gate is +40 on slot (c mod kpool) of channel c: the pooled value of channel
    # c is then k[slot c mod kpool, c]; a softmax over channels or over pools
    # would give something else.
    kpool, D = 4, 8
    rng = np.random.default_rng(5)
    k = rng.standard_normal((kpool, D)).astype(np.float32)
    gate = np.zeros((kpool, D), np.float32)
    for c in range(D):
        gate[c % kpool, c] = 40.0
    out, _ = _compress(k, gate, np.zeros((kpool, D)), np.ones(kpool), kpool, np.ones(D), np.zeros(D), eps=0.0)
    x = np.array([O.bf16_bits_to_f64(bf16(k))[c % kpool, c] for c in range(D)])
    y = (x - x.mean()) / np.sqrt(((x - x.mean()) ** 2).mean())
    assert np.max(np.abs(O.bf16_bits_to_f64(out["keys"][0]) - y)) <= 2.0 ** -7 * np.abs(y).max()


def test_one_hot_ape_selects_a_slot():
    kpool, D, P = 8, 32, 6
    rng = np.random.default_rng(6)
    k = rng.standard_normal((kpool * P, D)).astype(np.float32)
    gate = rng.standard_normal((kpool * P, D)).astype(np.float32)
    ape = np.zeros((kpool, D), np.float32)
    ape[5] = 40.0
    out, _ = _compress(k, gate, ape, np.ones(kpool * P), kpool, np.ones(D), np.zeros(D), eps=0.0)
    kb = O.bf16_bits_to_f64(bf16(k)).reshape(P, kpool, D)[:, 5, :]
    y = (kb - kb.mean(1, keepdims=True)) / np.sqrt(kb.var(1, keepdims=True))
    assert np.max(np.abs(O.bf16_bits_to_f64(out["keys"][:P]) - y)) <= 2.0 ** -7 * np.abs(y).max()


def test_constant_gate_gives_mean_and_layernorm_matches_torch():
    kpool, D, P = 4, 64, 10
    rng = np.random.default_rng(7)
    k = (rng.standard_normal((kpool * P, D)) + 3.0).astype(np.float32)   # nonzero mean
    gate = np.full((kpool * P, D), 0.75, np.float32)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    b = (0.1 * rng.standard_normal(D)).astype(np.float32)
    out, _ = _compress(k, gate, np.zeros((kpool, D)), np.ones(kpool * P), kpool, w, b, eps=1e-5)
    mean = torch.tensor(O.bf16_bits_to_f64(bf16(k)).reshape(P, kpool, D).mean(axis=1))
    ref = torch.nn.functional.layer_norm(mean, (D,), torch.tensor(w, dtype=torch.float64),
                                         torch.tensor(b, dtype=torch.float64), 1e-5).numpy()
    assert np.array_equal(out["keys"][:P], O.f64_to_bf16_bits(ref))


def test_kpool_one_is_per_row_layernorm():
    D, T, pad = 32, 40, 3
    rng = np.random.default_rng(8)
    k = rng.standard_normal((T, D)).astype(np.float32)
    gate = rng.standard_normal((T, D)).astype(np.float32)
    valid = np.ones(T)
    valid[:pad] = 0
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    b = (0.1 * rng.standard_normal(D)).astype(np.float32)
    out, _ = _compress(k, gate, rng.standard_normal((1, D)), valid, 1, w, b)
    rows = torch.tensor(O.bf16_bits_to_f64(bf16(k))[pad:])
    ref = torch.nn.functional.layer_norm(rows, (D,), torch.tensor(w, dtype=torch.float64),
                                         torch.tensor(b, dtype=torch.float64), 1e-5).numpy()
    assert np.array_equal(out["keys"][:T - pad], O.f64_to_bf16_bits(ref))
    assert list(out["pool_start"][:T - pad]) == list(range(pad, T))


def test_layernorm_bias_is_applied():
    D = 16
    rng = np.random.default_rng(9)
    b = rng.standard_normal(D).astype(np.float32)
    out, _ = _compress(rng.standard_normal((4, D)), rng.standard_normal((4, D)), np.zeros((4, D)),
                       np.ones(4), 4, np.zeros(D), b)
    assert np.array_equal(out["keys"][0], bf16(b))


def test_left_padding_shift_invariance():
    kpool, D, T = 4, 32, 61
    rng = np.random.default_rng(10)
    k = rng.standard_normal((T, D)).astype(np.float32)
    g = rng.standard_normal((T, D)).astype(np.float32)
    ape = rng.standard_normal((kpool, D)).astype(np.float32)
    w, b = np.ones(D), np.zeros(D)
    a, _ = _compress(k, g, ape, np.ones(T), kpool, w, b)
    for n in (1, 3, 7):
        kp = np.concatenate([rng.standard_normal((n, D)), k]).astype(np.float32)
        gp = np.concatenate([rng.standard_normal((n, D)), g]).astype(np.float32)
        v = np.concatenate([np.zeros(n), np.ones(T)])
        c, _ = _compress(kp, gp, ape, v, kpool, w, b)
        P = T // kpool
        assert c["n_pools"][0] == a["n_pools"][0] == P
        assert np.array_equal(c["keys"][:P], a["keys"][:P])
        assert np.array_equal(c["pool_start"][:P] - n, a["pool_start"][:P])


def test_pool_with_a_hole_is_invalid_but_keeps_its_place():
    kpool, D, T = 4, 16, 24
    rng = np.random.default_rng(11)
    v = np.ones(T)
    v[2] = 0          # before the first valid row? no: row 0 is valid, so this is a hole in pool 0
    v[13] = 0         # hole in pool 3
    out, _ = _compress(rng.standard_normal((T, D)), rng.standard_normal((T, D)), np.zeros((kpool, D)),
                       v, kpool, np.ones(D), np.zeros(D))
    assert out["n_pools"][0] == 6
    assert list(out["pool_valid"][:6]) == [0, 1, 1, 0, 1, 1]
    assert list(out["pool_start"][:6]) == [0, 4, 8, 12, 16, 20]


def test_all_invalid_request_has_no_pools():
    out, _ = _compress(np.ones((9, 8)), np.ones((9, 8)), np.zeros((4, 8)), np.zeros(9), 4, np.ones(8), np.zeros(8))
    assert out["n_pools"][0] == 0
    assert np.all(out["pool_start"] == -1)


def test_incremental_recompress_equals_full():
    kpool, D = 4, 32
    lens = [37, 64, 5]
    rng = np.random.default_rng(12)
    T = sum(lens)
    tok_off = np.concatenate([[0], np.cumsum(lens)])
    k = rng.standard_normal((T, D)).astype(np.float32)
    g = rng.standard_normal((T, D)).astype(np.float32)
    ape = rng.standard_normal((kpool, D))
    v = np.ones(T)
    v[0] = 0
    a, _ = _compress(k, g, ape, v, kpool, np.ones(D), np.zeros(D), tok_off=tok_off)
    new_from = np.array([30, 57, 2])
    k2, g2 = k.copy(), g.copy()
    for r in range(3):
        lo = tok_off[r] + new_from[r]
        k2[lo:tok_off[r + 1]] = rng.standard_normal((tok_off[r + 1] - lo, D))
        g2[lo:tok_off[r + 1]] = rng.standard_normal((tok_off[r + 1] - lo, D))
    full, _ = _compress(k2, g2, ape, v, kpool, np.ones(D), np.zeros(D), tok_off=tok_off)
    inc, _ = _compress(k2, g2, ape, v, kpool, np.ones(D), np.zeros(D), tok_off=tok_off,
                       new_from=new_from, prev=a)
    for key in ("keys", "pool_start", "pool_valid", "n_pools"):
        assert np.array_equal(full[key], inc[key])
    assert not np.array_equal(full["keys"], a["keys"])


# ---------------------------------------------------------------------------
# a3 scores
# ---------------------------------------------------------------------------

def _scores_setup(rng, P=9, H=3, D=8, kpool=2, q_pos=None):
    keys = bf16(rng.standard_normal((P, D)))
    qi = bf16(rng.standard_normal((1, H, D)))
    start = np.arange(P, dtype=np.int32) * kpool
    pvalid = np.ones(P, np.uint8)
    return keys, qi, start, pvalid, np.array([0, P], np.int32), np.array([P], np.int32)


def test_scores_brute_force_loops():
    rng = np.random.default_rng(13)
    keys, qi, start, pv, poff, npools = _scores_setup(rng)
    w = np.float32([[0.5, -1.25, 2.0]])
    s, c = O.index_scores(qi, w, keys, start, pv, poff, npools, np.int32([0]), np.int32([100]), 2, 12)
    kf, qf = O.bf16_bits_to_f64(keys), O.bf16_bits_to_f64(qi)
    for p in range(9):
        tot = 0.0
        for h in range(3):
            d = sum(qf[0, h, i] * kf[p, i] for i in range(8))
            tot += float(w[0, h]) * (d if d > 0 else 0.0)
        assert s[0, p] == np.float32(tot) or (tot == 0 and s[0, p] == 0)
    assert np.all(c[0, :9] == 1) and np.all(c[0, 9:] == 0) and np.all(np.isneginf(s[0, 9:]))


def test_scores_single_head_unit_weight_is_relu_dot():
    rng = np.random.default_rng(14)
    keys, qi, start, pv, poff, npools = _scores_setup(rng, H=1)
    s, _ = O.index_scores(qi, np.float32([[1.0]]), keys, start, pv, poff, npools,
                          np.int32([0]), np.int32([100]), 2, 9)
    ref = np.maximum(O.bf16_bits_to_f64(keys) @ O.bf16_bits_to_f64(qi[0, 0]), 0).astype(np.float32)
    assert np.array_equal(s[0], ref)
    assert not np.any(np.signbit(s[0]))      # relu zeros are +0


def test_scores_causal_boundary_golden():
    g = gold("causal_worked.json")
    rng = np.random.default_rng(15)
    P = g["T"] // g["kpool"]
    keys = bf16(rng.standard_normal((P, 8)))
    start = (np.arange(P) * g["kpool"]).astype(np.int32)
    for case in g["cases"]:
        s, c = O.index_scores(bf16(rng.standard_normal((1, 2, 8))), np.float32([[1, 1]]), keys, start,
                              np.ones(P, np.uint8), np.int32([0, P]), np.int32([P]), np.int32([0]),
                              np.int32([case["q_pos"]]), g["kpool"], P)
        assert list(c[0]) == case["cand"]
        assert np.all(np.isneginf(s[0][c[0] == 0]))


def test_scores_invalid_pool_is_not_a_candidate():
    rng = np.random.default_rng(16)
    keys, qi, start, pv, poff, npools = _scores_setup(rng)
    pv[4] = 0
    s, c = O.index_scores(qi, np.float32([[1, 1, 1]]), keys, start, pv, poff, npools,
                          np.int32([0]), np.int32([100]), 2, 9)
    assert c[0, 4] == 0 and np.isneginf(s[0, 4]) and c[0].sum() == 8


# ---------------------------------------------------------------------------
# a4 top-k
# ---------------------------------------------------------------------------

def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(17)
    for trial in range(300):
        P = int(rng.integers(1, 40))
        kk = int(rng.integers(1, 12))
        s = rng.choice(np.float32([-2.0, -0.5, 0.0, 0.5, 1.0, 3.0]), size=P).astype(np.float32)
        c = (rng.random(P) < 0.7).astype(np.uint8)
        s = np.where(c == 1, s, -np.inf).astype(np.float32)
        sel = O.topk_pools(s[None], c[None], kk)[0]
        cands = [(float(s[p]), p) for p in range(P) if c[p]]
        best = sorted(cands, key=lambda t: (-t[0], t[1]))[:kk]
        expect = sorted(p for _, p in best)
        assert list(sel[:len(expect)]) == expect
        assert np.all(sel[len(expect):] == -1)


def test_topk_row_len_brute_force():
    """A row length keeps only the row's leading entries: brute force over the
    cut row, with lengths of 0, inside the row, the width and past it."""
    rng = np.random.default_rng(23)
    for trial in range(200):
        P = int(rng.integers(1, 30))
        kk = int(rng.integers(1, 10))
        Q = 4
        s = rng.choice(np.float32([-1.0, 0.0, 0.25, 2.0, 5.0]), size=(Q, P)).astype(np.float32)
        c = (rng.random((Q, P)) < 0.8).astype(np.uint8)
        lens = np.array([0, int(rng.integers(0, P + 1)), P, P + 7], dtype=np.int32)
        sel = O.topk_pools(s, c, kk, row_len=lens)
        for q in range(Q):
            n = min(int(lens[q]), P)
            cands = [(float(s[q, p]), p) for p in range(n) if c[q, p]]
            expect = sorted(p for _, p in sorted(cands, key=lambda t: (-t[0], t[1]))[:kk])
            assert list(sel[q, :len(expect)]) == expect
            assert np.all(sel[q, len(expect):] == -1)


def test_topk_no_candidates_all_minus_one():
    sel = O.topk_pools(np.full((2, 5), -np.inf, np.float32), np.zeros((2, 5), np.uint8), 3)
    assert np.all(sel == -1)


# ---------------------------------------------------------------------------
# a5 expansion
# ---------------------------------------------------------------------------

def test_expand_worked_example_golden():
    g = gold("expand_worked.json")
    tok = O.expand_selection(np.int32([g["sel"]]), np.int32(g["pool_start"]), np.int32([0, 3]),
                             np.int32([0]), g["kpool"], g["out_width"])
    assert list(tok[0]) == g["tok"]


# ---------------------------------------------------------------------------
# a6 sparse MLA
# ---------------------------------------------------------------------------

def _mla_case(rng, T=40, Hm=4, L=512, n_sel=None, fp8=False, Q=1):
    q = bf16(rng.standard_normal((Q, Hm, L)))
    lat = rng.standard_normal((T, L)) / math.sqrt(L)
    if fp8:
        scale = (np.abs(lat).max(1) / 448).astype(np.float32)
        codes = torch.tensor(lat / scale[:, None], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return q, codes, scale
    return q, bf16(lat), None


def test_mla_equals_dense_sdpa_when_all_rows_selected():
    # With every full-pool row selected, the gathered attention is the dense
    # attention over those rows (the dense mask of set membership).
    rng = np.random.default_rng(18)
    for fp8 in (False, True):
        q, ckv, scale = _mla_case(rng, fp8=fp8)
        rows = np.arange(3, 39)
        tok = np.full((1, 48), -1, np.int32)
        tok[0, 5:5 + len(rows)] = rows[::-1]       # order and -1 holes do not matter
        res = O.sparse_mla_decode(q, ckv, scale, np.int32([0]), np.int32([0]), tok, 0.7)
        if scale is None:
            C = torch.from_numpy(ckv[rows].astype(np.int16)).view(torch.bfloat16).to(torch.float64)
        else:
            C = torch.from_numpy(ckv[rows]).view(torch.float8_e4m3fn).to(torch.float64) \
                * torch.from_numpy(scale[rows]).to(torch.float64)[:, None]
        Qt = torch.from_numpy(q[0].astype(np.int16)).view(torch.bfloat16).to(torch.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(Qt[None], C[None], C[None], scale=0.7)[0]
        assert np.max(np.abs(res["out_f64"][0] - ref.numpy())) < 1e-12
        lref = torch.logsumexp(0.7 * Qt @ C.T, dim=1).numpy()
        assert np.max(np.abs(res["lse"][0] - lref)) < 1e-12


def test_mla_closed_forms():
    rng = np.random.default_rng(19)
    q, ckv, _ = _mla_case(rng)
    C = O.bf16_bits_to_f64(ckv)
    # one selected token: O is that row, lse is its logit
    tok = np.int32([[-1, 17, -1, -1]])
    r = O.sparse_mla_decode(q, ckv, None, np.int32([2]), np.int32([0]), tok, 1.0)
    assert np.array_equal(r["out_f64"][0], np.broadcast_to(C[19], (4, 512)))
    assert np.allclose(r["lse"][0], O.bf16_bits_to_f64(q[0]) @ C[19], rtol=0, atol=1e-12)
    # zero query: uniform weights, O is the mean row, lse = log n
    z = np.zeros_like(q)
    tok = np.int32([[0, 1, 2, 3, 4]])
    r = O.sparse_mla_decode(z, ckv, None, np.int32([0]), np.int32([0]), tok, 1.0)
    assert np.allclose(r["out_f64"][0], C[:5].mean(0)[None], rtol=0, atol=1e-15)
    assert np.allclose(r["lse"][0], math.log(5), rtol=0, atol=1e-15)
    # empty row: zero output, lse -inf
    r = O.sparse_mla_decode(q, ckv, None, np.int32([0]), np.int32([0]), np.int32([[-1, -1]]), 1.0)
    assert np.all(r["out"] == 0) and np.all(np.isneginf(r["lse"]))


def test_mla_sm_scale_scales_logits():
    rng = np.random.default_rng(20)
    q, ckv, _ = _mla_case(rng)
    tok = np.int32([[1, 5, 9, 30]])
    a = O.sparse_mla_decode(q, ckv, None, np.int32([0]), np.int32([0]), tok, 2.0)
    q2 = O.f64_to_bf16_bits(2 * O.bf16_bits_to_f64(q))        # doubling is exact in bf16
    b = O.sparse_mla_decode(q2, ckv, None, np.int32([0]), np.int32([0]), tok, 1.0)
    assert np.max(np.abs(a["out_f64"] - b["out_f64"])) < 1e-14


# ---- always_select_tail ------------------------------------------------------

def test_select_tail_worked_example_golden():
    g = json.load(open(os.path.join(GOLD, "tail_worked.json")))
    valid = np.array(g["valid"], dtype=np.uint8)
    q = len(g["q_pos"])
    out = O.select_tail(np.array(g["tok_in"], dtype=np.int32), valid, np.array([0, g["T"]]),
                        np.zeros(q, dtype=np.int32), np.array(g["q_pos"]), g["kpool"], g["select_k"])
    assert np.array_equal(out, np.array(g["tok_out"]))


def test_select_tail_brute_force_against_pool_geometry():
    """The tail of a query at t, row by row: a valid row at or after the first
    valid row and at or before t that lies in no full pool ending at or before
    t -- the pools taken from the compression's pool starts, not from the
    tail's own arithmetic."""
    rng = np.random.default_rng(21)
    for trial in range(60):
        kpool = int(rng.integers(1, 9))
        B = 3
        lengths = rng.integers(1, 60, size=B)
        tok_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        valid = np.ones(int(tok_off[-1]), dtype=np.uint8)
        for r in range(B):
            pad = int(rng.integers(0, lengths[r] + 1))
            valid[tok_off[r]:tok_off[r] + pad] = 0
            if rng.random() < 0.5 and lengths[r] > pad + 2:      # a hole after f
                valid[tok_off[r] + int(rng.integers(pad + 1, lengths[r]))] = 0
        pool_off = np.concatenate([[0], np.cumsum(lengths // kpool)]).astype(np.int64)
        D = 8
        z = np.zeros((int(tok_off[-1]), D), dtype=np.uint16)
        comp = O.kpool_compress(z, z, np.zeros((kpool, D), np.uint16), valid, tok_off, pool_off,
                                np.ones(D), np.zeros(D), 1e-5, kpool)
        q_req = np.repeat(np.arange(B), 4)
        q_pos = np.array([int(rng.integers(0, lengths[r])) for r in q_req])
        q_pos[::4] = lengths[q_req[::4]] - 1                       # one decode query each
        select_k = 2
        tok_in = np.full((len(q_req), select_k * kpool + kpool - 1), -1, dtype=np.int32)
        out = O.select_tail(tok_in, valid, tok_off, q_req, q_pos, kpool, select_k)
        for q in range(len(q_req)):
            r, t = int(q_req[q]), int(q_pos[q])
            starts = [int(comp["pool_start"][pool_off[r] + p]) for p in range(int(comp["n_pools"][r]))]
            v = valid[tok_off[r]:tok_off[r + 1]]
            nz = np.flatnonzero(v)
            f = int(nz[0]) if len(nz) else -1
            want = []
            for x in range(0, t + 1):
                if not v[x] or f < 0 or x < f:
                    continue
                if any(s <= x <= s + kpool - 1 and s + kpool - 1 <= t for s in starts):
                    continue
                want.append(x)
            got = [int(x) for x in out[q, select_k * kpool:] if x >= 0]
            assert got == want, (trial, q, got, want)
            assert len(got) <= kpool - 1
            assert np.all(out[q, :select_k * kpool] == -1)


def test_select_tail_decode_closed_form():
    """Decode (t = T-1) with no holes: the tail is exactly the trailing partial
    pool, rows f + P*kpool .. T-1 of the geometry."""
    valid = np.array([0] * 3 + [1] * 30, dtype=np.uint8)
    tok_off = np.array([0, 33])
    first, n_pools = O.kpool_geometry(valid, tok_off, 4)
    out = O.select_tail(np.full((1, 8 + 3), -1, np.int32), valid, tok_off, np.array([0]),
                        np.array([32]), 4, 2)
    lo = int(first[0] + n_pools[0] * 4)
    assert list(out[0, 8:8 + (33 - lo)]) == list(range(lo, 33))
    assert lo == 31 and out[0, 10] == -1


# ---- paged latent cache ------------------------------------------------------

def test_paged_kv_index_worked_example_golden():
    g = gold("paged_worked.json")
    for c in g["cases"]:
        got = O.kv_index(np.array(c["tok"]), np.array(c["q_req"]), np.array(c["block_table"]),
                         c["page_rows"])
        assert np.array_equal(got, np.array(c["kvidx"]))


def _scatter_pages(ckv, scale, kv_off, lengths, page_rows, rng):
    """Lay each request's rows into pages taken in a random order from a pool
    that also holds junk pages, one row at a time; returns the paged cache and
    its block table."""
    nblk = [(n + page_rows - 1) // page_rows for n in lengths]
    n_pages = sum(nblk) + 3
    order = rng.permutation(n_pages)
    pages = np.empty((n_pages * page_rows,) + ckv.shape[1:], dtype=ckv.dtype)
    pages[...] = rng.integers(0, 1 << 14, size=pages.shape).astype(ckv.dtype)   # junk rows
    pscale = None if scale is None else rng.uniform(0.5, 2.0, n_pages * page_rows)
    table = np.zeros((len(lengths), max(nblk) + 2), dtype=np.int32)
    k = 0
    for r, n in enumerate(lengths):
        for b in range(nblk[r]):
            table[r, b] = order[k]
            k += 1
        for t in range(n):
            dst = table[r, t // page_rows] * page_rows + t % page_rows
            pages[dst] = ckv[kv_off[r] + t]
            if scale is not None:
                pscale[dst] = scale[kv_off[r] + t]
    return pages, pscale, table


@pytest.mark.parametrize("page_rows", [1, 3, 16])
def test_paged_mla_equals_flat_over_shuffled_pages(page_rows):
    """The same logical rows laid out in shuffled pages (among junk pages) give
    exactly the flat cache's attention, in bf16 and fp8."""
    rng = np.random.default_rng(22)
    lengths = [37, 20, 45]
    kv_off = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    for fp8 in (False, True):
        q, ckv, scale = _mla_case(rng, fp8=fp8, T=int(sum(lengths)), Q=4)
        q_req = np.array([0, 1, 2, 2])
        tok = np.full((4, 24), -1, dtype=np.int32)
        for qq, r in enumerate(q_req):
            ids = rng.choice(lengths[r], size=min(18, lengths[r]), replace=False)
            tok[qq, rng.choice(24, size=len(ids), replace=False)] = ids
        flat = O.sparse_mla_decode(q, ckv, scale, kv_off, q_req, tok, 0.9)
        pages, pscale, table = _scatter_pages(ckv, scale, kv_off, lengths, page_rows, rng)
        paged = O.sparse_mla_decode_paged(q, pages, pscale, table, page_rows, q_req, tok, 0.9)
        assert np.array_equal(paged["out_f64"], flat["out_f64"])
        assert np.array_equal(paged["lse"], flat["lse"])
        assert np.all((paged["kvidx"] >= 0) == (tok >= 0))


def test_paged_identity_table_is_the_flat_cache():
    """page_rows = 1 and block_table[r, b] = kv_off[r] + b is the flat layout."""
    rng = np.random.default_rng(23)
    q, ckv, _ = _mla_case(rng, T=30, Q=2)
    kv_off = np.array([0, 11])
    table = np.stack([np.arange(19), 11 + np.arange(19)])
    tok = np.int32([[0, 4, 10, -1], [18, 3, -1, 7]])
    flat = O.sparse_mla_decode(q, ckv, None, kv_off, np.array([0, 1]), tok, 1.0)
    paged = O.sparse_mla_decode_paged(q, ckv, None, table, 1, np.array([0, 1]), tok, 1.0)
    assert np.array_equal(paged["out"], flat["out"])
    assert np.array_equal(paged["kvidx"], np.int64([[0, 4, 10, -1], [29, 14, -1, 18]]))


# ---- the cache-write side: live lengths, indexer_store, write_geom -----------

def _regions(rng, B=3, cap=(40, 60), D=16):
    lengths = rng.integers(cap[0], cap[1], size=B)
    tok_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    n = int(tok_off[-1])
    k = bf16(rng.standard_normal((n, D)))
    gate = bf16(rng.standard_normal((n, D)))
    valid = (rng.random(n) < 0.97).astype(np.uint8)
    return lengths, tok_off, k, gate, valid


def test_live_length_equals_truncated_region():
    """Compression over live lengths inside larger regions equals compression
    of the regions cut to those lengths: rows past a live length (junk,
    mostly valid) have no influence."""
    rng = np.random.default_rng(31)
    for kpool in (1, 3, 4, 8):
        lengths, tok_off, k, gate, valid = _regions(rng)
        D = k.shape[1]
        ape = bf16(rng.standard_normal((kpool, D)))
        lw, lb = 1 + 0.1 * rng.standard_normal(D), 0.1 * rng.standard_normal(D)
        seq_len = np.array([int(rng.integers(0, n + 1)) for n in lengths])
        seq_len[0] = lengths[0]
        pool_off = np.concatenate([[0], np.cumsum(lengths // kpool)]).astype(np.int64)
        got = O.kpool_compress(k, gate, ape, valid, tok_off, pool_off, lw, lb, 1e-5, kpool,
                               seq_len=seq_len)
        cut = [np.arange(tok_off[r], tok_off[r] + seq_len[r]) for r in range(len(lengths))]
        idx = np.concatenate(cut)
        toff2 = np.concatenate([[0], np.cumsum(seq_len)]).astype(np.int64)
        want = O.kpool_compress(k[idx], gate[idx], ape, valid[idx], toff2, pool_off, lw, lb, 1e-5,
                                kpool)
        for name in ("keys", "pool_start", "pool_valid", "n_pools"):
            assert np.array_equal(got[name], want[name]), (kpool, name)


def test_compress_without_layernorm():
    """The k_normed reading: no LayerNorm after pooling.  kpool 1 stores each
    row's key as the row itself; a constant gate with no ape gives the slots'
    mean, rounded once."""
    rng = np.random.default_rng(32)
    lengths, tok_off, k, gate, valid = _regions(rng, B=2)
    valid[:] = 1
    D = k.shape[1]
    pool_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    r1 = O.kpool_compress(k, gate, np.zeros((1, D), np.uint16), valid, tok_off, pool_off, None,
                          None, 1e-5, 1)
    assert np.array_equal(r1["keys"], k)
    g0 = np.zeros_like(gate)
    pool_off4 = np.concatenate([[0], np.cumsum(lengths // 4)]).astype(np.int64)
    r4 = O.kpool_compress(k, g0, np.zeros((4, D), np.uint16), valid, tok_off, pool_off4, None,
                          None, 1e-5, 4)
    for r in range(2):
        for p in range(int(r4["n_pools"][r])):
            rows = tok_off[r] + 4 * p + np.arange(4)
            mean = O.bf16_bits_to_f64(k[rows]).sum(axis=0) / 4
            assert np.array_equal(r4["keys"][pool_off4[r] + p], O.f64_to_bf16_bits(mean))


def test_indexer_store_places_rows_and_marks_them_valid():
    rng = np.random.default_rng(33)
    lengths, tok_off, k, gate, valid = _regions(rng, B=4)
    D = k.shape[1]
    valid[:] = 0
    pos = np.array([0, int(lengths[1]) - 1, int(lengths[2]), -1])   # first, last, past, before
    k_new, g_new = bf16(rng.standard_normal((4, D))), bf16(rng.standard_normal((4, D)))
    out = O.indexer_store(k, gate, valid, tok_off, pos, k_new, g_new)
    written = {int(tok_off[0]): 0, int(tok_off[1]) + int(lengths[1]) - 1: 1}
    for row in range(len(valid)):
        if row in written:
            r = written[row]
            assert np.array_equal(out["k"][row], k_new[r]) and np.array_equal(out["gate"][row], g_new[r])
            assert out["valid"][row] == 1
        else:
            assert np.array_equal(out["k"][row], k[row]) and out["valid"][row] == 0
    # with the LayerNorm: torch's layer_norm in float64, rounded by torch to bf16
    lw, lb = 1 + 0.1 * rng.standard_normal(D), 0.1 * rng.standard_normal(D)
    out = O.indexer_store(k, gate, valid, tok_off, pos, k_new, g_new, lw, lb, 1e-5)
    x = torch.from_numpy(k_new.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    y = torch.nn.functional.layer_norm(x, (D,), torch.from_numpy(lw), torch.from_numpy(lb), 1e-5)
    yb = y.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(out["k"][int(tok_off[0])], yb[0])
    assert np.array_equal(out["gate"][int(tok_off[0])], g_new[0])


def test_k_normed_variant_equals_post_pool_norm_at_kpool_one():
    """With one slot per pool, normalising each row when it is stored and
    pooling without a LayerNorm gives the same keys as pooling then
    normalising."""
    rng = np.random.default_rng(34)
    lengths, tok_off, k, gate, valid = _regions(rng, B=2)
    valid[:] = 1
    D = k.shape[1]
    lw, lb = 1 + 0.1 * rng.standard_normal(D), 0.1 * rng.standard_normal(D)
    pool_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    ape = np.zeros((1, D), np.uint16)
    post = O.kpool_compress(k, gate, ape, valid, tok_off, pool_off, lw, lb, 1e-5, 1)
    kn = k.copy()
    for r in range(2):
        for t in range(int(lengths[r])):
            st = O.indexer_store(kn, gate, valid, tok_off, np.array([t, -1]) if r == 0 else
                                 np.array([-1, t]), k[[tok_off[r] + t] * 2], gate[[0, 0]], lw, lb,
                                 1e-5)
            kn = st["k"]
    pre = O.kpool_compress(kn, gate, ape, valid, tok_off, pool_off, None, None, 1e-5, 1)
    assert np.array_equal(pre["keys"], post["keys"])


def test_write_geom_worked_example_golden():
    g = gold("write_geom_worked.json")
    out = O.write_geom(np.array(g["seq_len"]), np.array(g["block_table"]), g["page_rows"])
    for name in ("q_req", "q_pos", "new_from", "slot"):
        assert list(out[name]) == g[name], name


def test_decode_steps_over_live_lengths_equal_full_recompression():
    """A run of decode steps that each store one row at the live length, grow
    it by one and recompress from the stored row (write_geom's new_from)
    keeps the pools equal to a full compression at every step."""
    rng = np.random.default_rng(35)
    kpool, D, B = 4, 16, 3
    lengths, tok_off, k, gate, valid = _regions(rng, B=B, cap=(30, 40), D=D)
    valid[:] = 1
    valid[tok_off[1]:tok_off[1] + 3] = 0                    # left padding in request 1
    ape = bf16(rng.standard_normal((kpool, D)))
    lw, lb = 1 + 0.1 * rng.standard_normal(D), 0.1 * rng.standard_normal(D)
    pool_off = np.concatenate([[0], np.cumsum(lengths // kpool)]).astype(np.int64)
    seq_len = np.array([5, 0, 9])
    state = O.kpool_compress(k, gate, ape, valid, tok_off, pool_off, lw, lb, 1e-5, kpool,
                             seq_len=seq_len)
    for step in range(14):
        pos = seq_len.copy()
        st = O.indexer_store(k, gate, valid, tok_off, pos, bf16(rng.standard_normal((B, D))),
                             bf16(rng.standard_normal((B, D))))
        k, gate, valid = st["k"], st["gate"], st["valid"]
        seq_len = seq_len + 1
        geo = O.write_geom(seq_len)
        assert np.array_equal(geo["new_from"], pos)
        state = O.kpool_compress(k, gate, ape, valid, tok_off, pool_off, lw, lb, 1e-5, kpool,
                                 new_from=geo["new_from"], prev=state, seq_len=seq_len)
        full = O.kpool_compress(k, gate, ape, valid, tok_off, pool_off, lw, lb, 1e-5, kpool,
                                seq_len=seq_len)
        for name in ("keys", "pool_start", "pool_valid", "n_pools"):
            assert np.array_equal(state[name], full[name]), (step, name)
