"""GPU parity of every stage against the CPU oracle on parity shapes that span
several tiles with ragged tails.  Each stage is first fed the ORACLE's
upstream outputs (stage isolation), then the whole chain runs on the GPU and
is compared with the chained rules of tests/parity.py."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


@pytest.fixture(scope="module", params=W.PARITY_SHAPES)
def case(request):
    _need_gpu()
    from sparse_attention_fp32_amd.pipeline import DsaStep  # noqa: F401  (loads libdsa)
    spec = W.spec_by_name(request.param)
    x = W.make_inputs(spec, seed=0)
    xn = x.numpy()
    ref = O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                     spec.sm_scale, always_select_tail=spec.always_select_tail)
    return spec, xn, ref, x.to("cuda")


# shapes a case applies to (the case fixture is parametrized over them
# directly, so no case is collected where it cannot run)
TAIL_SHAPES = [n for n in W.PARITY_SHAPES if W.spec_by_name(n).always_select_tail]
MULTI_QUERY_SHAPES = [n for n in W.PARITY_SHAPES if W.spec_by_name(n).Q >= 2]
SUBRANGE_Q0 = 4
SUBRANGE_SHAPES = [n for n in W.PARITY_SHAPES if W.spec_by_name(n).Q > SUBRANGE_Q0]


def _step(xg):
    from sparse_attention_fp32_amd.pipeline import DsaStep
    return DsaStep(xg)


def _poison(t):
    t.view(torch.uint8).fill_(0xFF)


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_head_gate(case):
    spec, xn, ref, xg = case
    _say(f"head_gate {spec.name}")
    st = _step(xg)
    _poison(st.w)
    st.head_gate()
    PT.check_gate(_np(st.w), ref["w"])


def test_head_gate_repeat_keeps_workspace_clean(case):
    spec, xn, ref, xg = case
    _say(f"head_gate x3 {spec.name}")
    st = _step(xg)
    for _ in range(3):
        st.head_gate()
    PT.check_gate(_np(st.w), ref["w"])
    assert int(st.ws_gate[:4].view(torch.int32).item() if st.ws_gate.numel() >= 4 else 0) == 0


# (M, K, N): row path at its upper bound, MFMA path with ragged row tiles, waves
# left without K steps, N < 16 and N = 1, and the LDS path (K % 16 != 0)
# up to 512 rows one workgroup per row; above, 16 rows per workgroup on fp32
# MFMA (K % 16 == 0) or the LDS-tiled loop
GATE_SHAPES = [(16, 4096, 16), (17, 16, 16), (33, 48, 7), (100, 4096, 16), (63, 2064, 1),
               (40, 1000, 16), (20, 4104, 5), (512, 4096, 16), (513, 2064, 16),
               (600, 4096, 5), (530, 1000, 7), (1041, 48, 16)]


@pytest.mark.parametrize("M,K,N", GATE_SHAPES)
def test_head_gate_shapes(M, K, N):
    _need_gpu()
    from sparse_attention_fp32_amd import dsa
    _say(f"head_gate shape M={M} K={K} N={N}")
    h, Wm = W.gate_operands(M, K, N, seed=M * 7 + N)
    w = torch.empty(M, N, dtype=torch.float32, device="cuda")
    _poison(w)
    ws = torch.zeros(max(1, dsa.head_gate_workspace_size(M, K, N)), dtype=torch.uint8,
                     device="cuda")
    dsa.dsa_head_gate(h.cuda(), Wm.cuda(), w, ws)
    PT.check_gate(_np(w), O.head_gate(h.numpy(), Wm.numpy()))


def test_kpool_compress(case):
    spec, xn, ref, xg = case
    _say(f"kpool_compress {spec.name}")
    st = _step(xg)
    for t in (st.keys, st.pool_start, st.pool_valid, st.n_pools):
        _poison(t)
    st.compress()
    g = {"keys": _np(st.keys).view(np.uint16), "pool_start": _np(st.pool_start),
         "pool_valid": _np(st.pool_valid), "n_pools": _np(st.n_pools)}
    ncap = int(xn["pool_off"][-1])
    g = {k: (v[:ncap] if k != "n_pools" else v) for k, v in g.items()}
    flips = PT.check_compress(g, ref)
    _say(f"keys differing by 1 ulp: {flips} of {ref['keys'].size}")


def test_kpool_compress_incremental(case):
    spec, xn, ref, xg = case
    _say(f"kpool_compress incremental {spec.name}")
    st = _step(xg)
    st.compress()
    # a decode step appends (here: rewrites) the newest row of every request
    k2, g2 = xg.k.clone(), xg.gate.clone()
    offs = xn["tok_off"]
    gen = torch.Generator(device="cuda").manual_seed(7)
    for r in range(spec.B):
        last = int(offs[r + 1]) - 1
        k2[last] = torch.randn(spec.index_dim, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
        g2[last] = torch.randn(spec.index_dim, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    xg2 = W.Inputs(**{**xg.__dict__, "k": k2, "gate": g2})
    st.x = xg2
    st.compress(incremental=True)
    x2 = dict(xn, k=k2.cpu().numpy(), gate=g2.cpu().numpy())
    ref2 = O.kpool_compress(x2["k"], x2["gate"], x2["ape"], x2["valid"], x2["tok_off"],
                            x2["pool_off"], x2["ln_w"], x2["ln_b"], spec.eps, spec.kpool)
    ncap = int(xn["pool_off"][-1])
    g = {"keys": _np(st.keys).view(np.uint16)[:ncap], "pool_start": _np(st.pool_start)[:ncap],
         "pool_valid": _np(st.pool_valid)[:ncap], "n_pools": _np(st.n_pools)}
    PT.check_compress(g, ref2)


# Left padding that the first-valid-row scan must cross in several rounds, at
# every alignment of the request's first row: 2 valid rows after 39998 padding
# rows, a request with no valid row, one of a single row, a first valid row on
# a 4 KiB boundary, and short requests inside one 16-byte chunk.
EDGE_PADS = W.Spec("scan_edges", lengths=[40000, 21000, 20, 16, 1, 4100, 7, 33, 5],
                   pads=[39998, 20485, 19, 16, 0, 4096, 3, 0, 4], kpool=4, index_heads=4,
                   index_dim=128, hidden=256, select_k=4, out_width=16, mla_heads=8)


@pytest.mark.parametrize("live", [False, True])
def test_kpool_compress_first_valid_edges(live):
    """Full compression, then the incremental call (whose scan runs where no
    cached pool gives the first valid row), against the oracle; with live
    lengths that end the scan inside the padding of some requests."""
    _need_gpu()
    spec = EDGE_PADS
    _say(f"kpool_compress first-valid edges live={live}")
    x = W.make_inputs(spec, seed=3)
    xn = x.numpy()
    xg = x.to("cuda")
    st = _step(xg)
    seq = None
    if live:
        seq = np.array([39999, 20490, 20, 16, 1, 4096, 5, 33, 4], dtype=np.int32)
        st.seq_len = torch.from_numpy(seq).cuda()
    ref = O.kpool_compress(xn["k"], xn["gate"], xn["ape"], xn["valid"], xn["tok_off"],
                           xn["pool_off"], xn["ln_w"], xn["ln_b"], spec.eps, spec.kpool,
                           seq_len=seq)
    ncap = int(xn["pool_off"][-1])

    def got():
        return {"keys": _np(st.keys).view(np.uint16)[:ncap], "pool_start": _np(st.pool_start)[:ncap],
                "pool_valid": _np(st.pool_valid)[:ncap], "n_pools": _np(st.n_pools)}
    for t in (st.keys, st.pool_start, st.pool_valid, st.n_pools):
        _poison(t)
    st.compress()
    PT.check_compress(got(), ref)
    if live:
        xg.new_from.copy_(torch.from_numpy(np.maximum(seq - 1, 0)))
    _poison(st.n_pools)
    st.compress(incremental=True)
    PT.check_compress(got(), ref)


@pytest.mark.parametrize("fused", [False, True])
def test_kpool_compress_incremental_multi(case, fused):
    """A step that rewrote the last kpool+1 rows of every request: several
    pools per request are touched, the first and last of them in any
    alignment with the request's first valid row."""
    from sparse_attention_fp32_amd import dsa
    spec, xn, ref, xg = case
    _say(f"kpool_compress incremental kpool+1 rows {spec.name} fused={fused}")
    st = _step(xg)
    st.compress()
    n = spec.kpool + 1
    offs = xn["tok_off"]
    k2, g2 = xg.k.clone(), xg.gate.clone()
    gen = torch.Generator(device="cuda").manual_seed(11)
    nf = []
    for r in range(spec.B):
        T = int(offs[r + 1] - offs[r])
        lo = max(T - n, 0)
        nf.append(lo)
        for row in range(int(offs[r]) + lo, int(offs[r + 1])):
            k2[row] = torch.randn(spec.index_dim, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            g2[row] = torch.randn(spec.index_dim, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    nf_t = torch.tensor(nf, dtype=torch.int32, device="cuda")
    x = xg
    if fused:
        dsa.dsa_gate_compress(x.hidden, x.W, st.gate_part, k2, g2, x.ape, x.valid, x.tok_off,
                              x.pool_off, x.ln_w, x.ln_b, spec.eps, spec.kpool, st.max_cap, st.keys,
                              st.pool_start, st.pool_valid, st.n_pools, new_from=nf_t, max_new=n)
    else:
        dsa.dsa_kpool_compress(k2, g2, x.ape, x.valid, x.tok_off, x.pool_off, x.ln_w, x.ln_b,
                               spec.eps, spec.kpool, st.max_cap, st.keys, st.pool_start,
                               st.pool_valid, st.n_pools, new_from=nf_t, max_new=n)
    ref2 = O.kpool_compress(k2.cpu().numpy(), g2.cpu().numpy(), xn["ape"], xn["valid"], xn["tok_off"],
                            xn["pool_off"], xn["ln_w"], xn["ln_b"], spec.eps, spec.kpool)
    ncap = int(xn["pool_off"][-1])
    g = {"keys": _np(st.keys).view(np.uint16)[:ncap], "pool_start": _np(st.pool_start)[:ncap],
         "pool_valid": _np(st.pool_valid)[:ncap], "n_pools": _np(st.n_pools)}
    PT.check_compress(g, ref2)


def _load_oracle_front(st, ref):
    ncap = len(ref["pool_start"])
    st.w.copy_(torch.from_numpy(ref["w"]))
    st.keys[:ncap].copy_(torch.from_numpy(ref["keys"].view(np.int16)))
    st.pool_start[:ncap].copy_(torch.from_numpy(ref["pool_start"]))
    st.pool_valid[:ncap].copy_(torch.from_numpy(ref["pool_valid"]))
    st.n_pools.copy_(torch.from_numpy(ref["n_pools"]))


def test_index_scores_isolated(case):
    spec, xn, ref, xg = case
    _say(f"index_scores {spec.name}")
    st = _step(xg)
    _load_oracle_front(st, ref)
    _poison(st.scores)
    _poison(st.cand)
    st.index_scores()
    worst = PT.check_scores(_np(st.scores), _np(st.cand), ref["scores"], ref["cand"])
    _say(f"scores worst rel diff {worst:.3g}")


def test_topk_isolated(case):
    spec, xn, ref, xg = case
    _say(f"topk {spec.name}")
    st = _step(xg)
    st.scores.copy_(torch.from_numpy(ref["scores"]))
    st.cand.copy_(torch.from_numpy(ref["cand"]))
    _poison(st.sel)
    st.topk()
    PT.check_sel_exact(_np(st.sel), ref["sel"])


def test_expand_isolated(case):
    spec, xn, ref, xg = case
    _say(f"expand {spec.name}")
    st = _step(xg)
    _load_oracle_front(st, ref)
    st.sel.copy_(torch.from_numpy(ref["sel"]))
    _poison(st.tok)
    st.expand()
    assert np.array_equal(_np(st.tok), ref["tok"])


@pytest.mark.parametrize("case", TAIL_SHAPES, indirect=True)
def test_select_tail_isolated(case):
    """The tail alone, on the oracle's expansion without it."""
    from sparse_attention_fp32_amd import dsa
    spec, xn, ref, xg = case
    _say(f"select_tail {spec.name}")
    st = _step(xg)
    _load_oracle_front(st, ref)
    pre = O.expand_selection(ref["sel"], ref["pool_start"], xn["pool_off"], xn["q_req"], spec.kpool,
                             spec.out_width)
    st.tok.copy_(torch.from_numpy(pre))
    dsa.dsa_select_tail(xg.valid, xg.tok_off, st.pool_start, xg.pool_off, st.n_pools, xg.q_req,
                        xg.q_pos, spec.kpool, spec.select_k, st.tok)
    assert np.array_equal(_np(st.tok), ref["tok"])
    # every query of this shape has a tail slot in use or a -1 there, never a stale id
    base = spec.select_k * spec.kpool
    assert np.any(ref["tok"][:, base:] >= 0)


def test_mla_isolated(case):
    spec, xn, ref, xg = case
    _say(f"sparse_mla {spec.name}")
    st = _step(xg)
    st.tok.copy_(torch.from_numpy(ref["tok"]))
    _poison(st.out)
    _poison(st.lse)
    st.mla()
    worst = PT.check_mla(_np(st.out), _np(st.lse), ref["out_f64"], ref["lse"])
    _say(f"MLA worst rel err {worst:.3g}")


def test_mla_fp8_every_code():
    """fp8 latent rows holding every finite E4M3 code (subnormals, both zeros,
    448) in every lane position: the attention against the oracle's decode of
    the same codes."""
    _need_gpu()
    spec = W.spec_by_name("medium_fp8")
    _say("sparse_mla fp8 every code")
    x = W.make_inputs(spec, seed=5)
    T, L = x.ckv.shape
    codes = (np.arange(T * L, dtype=np.int64).reshape(T, L) * 7 + np.arange(T)[:, None]) % 256
    codes[(codes & 0x7F) == 0x7F] = 0          # the two NaN codes
    x.ckv.copy_(torch.from_numpy(codes.astype(np.uint8)))
    xn = x.numpy()
    tok = W.random_selection(spec, seed=5)
    xg = x.to("cuda")
    st = _step(xg)
    st.tok.copy_(tok)
    _poison(st.out)
    _poison(st.lse)
    st.mla()
    want = O.sparse_mla_decode(xn["q_mla"], xn["ckv"], xn["ckv_scale"], xn["kv_off"], xn["q_req"],
                               tok.numpy(), spec.sm_scale)
    worst = PT.check_mla(_np(st.out), _np(st.lse), want["out_f64"], want["lse"])
    _say(f"MLA fp8 every code worst rel err {worst:.3g}")


def test_chain(case):
    spec, xn, ref, xg = case
    _say(f"chain {spec.name}")
    st = _step(xg)
    st.run()
    PT.check_gate(_np(st.w), ref["w"])
    nd = PT.check_chained_rows(_np(st.sel), _np(st.tok), _np(st.out), _np(st.lse), ref,
                               PT.oracle_expect(xn, spec, ref["pool_start"]))
    _say(f"chain {spec.name}: boundary swaps {nd}")


@pytest.mark.parametrize("case", MULTI_QUERY_SHAPES, indirect=True)
def test_determinism_and_duplicate_rows(case):
    spec, xn, ref, xg = case
    _say(f"determinism {spec.name}")
    # make query 1 an exact copy of query 0 (same request, position, vectors)
    d = dict(xg.__dict__)
    for name in ("hidden", "qi", "q_mla", "q_req", "q_pos"):
        t = d[name].clone()
        t[1] = t[0]
        d[name] = t
    x2 = W.Inputs(**d)
    st = _step(x2)
    st.run()
    a = [_np(t).copy() for t in (st.w, st.scores, st.sel, st.tok, st.out, st.lse)]
    st.run()
    b = [_np(t) for t in (st.w, st.scores, st.sel, st.tok, st.out, st.lse)]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "run-to-run difference"
    for u in a:
        assert np.array_equal(u[0].view(np.uint8), u[1].view(np.uint8)), "duplicate rows split"


# --- fused decode calls -------------------------------------------------------

def _oracle_gate_partials(xn, ns):
    """Head-gate partials of ns equal K slices, each from the oracle's head-gate
    on that slice (so their sum is the oracle's w up to fp32 rounding)."""
    K = xn["hidden"].shape[1]
    if ns == 1:
        return O.head_gate(xn["hidden"], xn["W"])[None]
    s = K // ns
    return np.stack([O.head_gate(xn["hidden"][:, i * s:(i + 1) * s], xn["W"][i * s:(i + 1) * s])
                     for i in range(ns)])


def test_fused_gate_compress(case):
    spec, xn, ref, xg = case
    _say(f"gate_compress {spec.name}")
    st = _step(xg)
    for t in (st.keys, st.pool_start, st.pool_valid, st.n_pools, st.gate_part):
        _poison(t)
    st.gate_compress()
    ns = st.nslices
    part = _np(st.gate_part)[:ns * spec.Q * spec.index_heads].reshape(
        spec.Q, ns, spec.index_heads).transpose(1, 0, 2)     # query-major on the device
    if ns > 1:
        PT.check_gate(part, _oracle_gate_partials(xn, ns))
    PT.check_gate(part.astype(np.float64).sum(axis=0), ref["w"])
    ncap = int(xn["pool_off"][-1])
    g = {"keys": _np(st.keys).view(np.uint16)[:ncap], "pool_start": _np(st.pool_start)[:ncap],
         "pool_valid": _np(st.pool_valid)[:ncap], "n_pools": _np(st.n_pools)}
    PT.check_compress(g, ref)


def test_fused_index_scores_isolated(case):
    spec, xn, ref, xg = case
    _say(f"index_scores_gated {spec.name}")
    st = _step(xg)
    _load_oracle_front(st, ref)
    part = _oracle_gate_partials(xn, st.nslices)               # [ns, Q, H]
    st.gate_part[:part.size].copy_(torch.from_numpy(
        np.ascontiguousarray(part.transpose(1, 0, 2)).reshape(-1)))   # query-major
    for t in (st.scores, st.cand, st.w):
        _poison(t)
    st.index_scores_gated()
    PT.check_gate(_np(st.w), ref["w"])
    worst = PT.check_scores(_np(st.scores), _np(st.cand), ref["scores"], ref["cand"])
    _say(f"gated scores worst rel diff {worst:.3g}")


@pytest.mark.parametrize("ns", [1, 7, 16, 17, 32, 33, 64])
def test_gated_scores_slice_counts(case, ns):
    """The gated scores for every count of head-gate slices the library
    takes (up to 64, uneven slices): the partials are the oracle's head-gate
    over each slice of K, so they add up to the oracle's w."""
    spec, xn, ref, xg = case
    _say(f"index_scores_gated {spec.name} with {ns} slices")
    from sparse_attention_fp32_amd import dsa
    st = _step(xg)
    _load_oracle_front(st, ref)
    parts = [O.head_gate(xn["hidden"][:, c], xn["W"][c])
             for c in np.array_split(np.arange(xn["hidden"].shape[1]), ns)]
    part = torch.from_numpy(np.ascontiguousarray(
        np.stack(parts, axis=1).astype(np.float32)).reshape(-1)).cuda()   # [Q, ns, H]
    for t in (st.scores, st.cand, st.w):
        _poison(t)
    x = st.x
    dsa.dsa_index_scores_gated(x.qi, part, ns, st.w, st.keys, st.pool_start, st.pool_valid,
                               x.pool_off, st.n_pools, x.q_req, x.q_pos, spec.kpool, st.scores,
                               st.cand)
    PT.check_gate(_np(st.w), ref["w"])
    PT.check_scores(_np(st.scores), _np(st.cand), ref["scores"], ref["cand"])


@pytest.mark.parametrize("case", SUBRANGE_SHAPES, indirect=True)
def test_gated_scores_query_subrange(case):
    """The gated scores on a run of queries q0.. of the batch (the per-query
    arrays, the query-major head-gate partials among them, passed from q0 on)
    give those queries' rows of the whole call."""
    spec, xn, ref, xg = case
    q0 = SUBRANGE_Q0
    _say(f"index_scores_gated {spec.name} on queries {q0}..{spec.Q - 1}")
    from sparse_attention_fp32_amd import dsa
    st = _step(xg)
    _load_oracle_front(st, ref)
    part = _oracle_gate_partials(xn, st.nslices)               # [ns, Q, H]
    st.gate_part[:part.size].copy_(torch.from_numpy(
        np.ascontiguousarray(part.transpose(1, 0, 2)).reshape(-1)))
    H, ns = spec.index_heads, st.nslices
    n = spec.Q - q0
    scores = torch.empty(n, st.pstride, dtype=torch.float32, device="cuda")
    cand = torch.empty(n, st.pstride, dtype=torch.uint8, device="cuda")
    w = torch.empty(n, H, dtype=torch.float32, device="cuda")
    for t in (scores, cand, w):
        _poison(t)
    x = st.x
    sub = st.gate_part[:spec.Q * ns * H].view(spec.Q, ns * H)[q0:]
    dsa.dsa_index_scores_gated(x.qi[q0:], sub, ns, w, st.keys, st.pool_start, st.pool_valid,
                               x.pool_off, st.n_pools, x.q_req[q0:], x.q_pos[q0:], spec.kpool,
                               scores, cand)
    PT.check_gate(_np(w), ref["w"][q0:])
    PT.check_scores(_np(scores), _np(cand), ref["scores"][q0:], ref["cand"][q0:])


def test_fused_topk_expand_isolated(case):
    spec, xn, ref, xg = case
    _say(f"topk_expand {spec.name}")
    st = _step(xg)
    _load_oracle_front(st, ref)
    st.scores.copy_(torch.from_numpy(ref["scores"]))
    st.cand.copy_(torch.from_numpy(ref["cand"]))
    _poison(st.sel)
    _poison(st.tok)
    st.topk_expand()
    PT.check_sel_exact(_np(st.sel), ref["sel"])
    assert np.array_equal(_np(st.tok), ref["tok"])


def test_fused_chain(case):
    spec, xn, ref, xg = case
    _say(f"fused chain {spec.name}")
    st = _step(xg)
    for t in (st.w, st.scores, st.cand, st.sel, st.tok, st.out, st.lse):
        _poison(t)
    st.run_fused()
    PT.check_gate(_np(st.w), ref["w"])
    nd = PT.check_chained_rows(_np(st.sel), _np(st.tok), _np(st.out), _np(st.lse), ref,
                               PT.oracle_expect(xn, spec, ref["pool_start"]))
    _say(f"fused chain {spec.name}: boundary swaps {nd}")
    # the cached-pool step after it gives the same outputs (nothing changed)
    a = [_np(t).copy() for t in (st.w, st.scores, st.sel, st.tok, st.out, st.lse)]
    st.run_fused(incremental=True)
    b = [_np(t) for t in (st.w, st.scores, st.sel, st.tok, st.out, st.lse)]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "incremental fused step differs"
