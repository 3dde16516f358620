"""GPU parity of the attention stage over a paged latent cache
(dsa_sparse_mla_decode_paged) against the oracle's paged attention.

Each case copies the latent rows into pages taken in a seeded random order
among junk pages (workloads.make_paged_cache).  The physical index rows are
integers and must match exactly; the outputs follow the attention tolerance.
The kernel runs the flat kernel's arithmetic on the same rows in the same
order, so its outputs must also equal the flat call's bit for bit.

Page sizes: 1 (a table row longer than the staged part, so entries are also
read from memory), 7 (not a power of two), 64 (the serving page)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu

PAGES = (1, 7, 64)


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(scope="module", params=W.PARITY_SHAPES)
def case(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd.pipeline import DsaStep  # noqa: F401  (loads libdsa)
    spec = W.spec_by_name(request.param)
    x = W.make_inputs(spec, seed=0)
    xn = x.numpy()
    ref = O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                     spec.sm_scale, always_select_tail=spec.always_select_tail)
    return spec, xn, ref, x.to("cuda")


def _paged_oracle(xn, pc, spec, tok, queries=None):
    scale = None if pc.ckv_scale is None else pc.ckv_scale.cpu().numpy()
    return O.sparse_mla_decode_paged(xn["q_mla"], pc.ckv.cpu().numpy(), scale,
                                     pc.block_table.cpu().numpy(), pc.page_rows, xn["q_req"], tok,
                                     spec.sm_scale, queries=queries)


def _run_both(st, pc):
    """Paged call (with the index rows) then the flat call on the same tok."""
    for t in (st.out, st.lse):
        t.view(torch.uint8).fill_(0xFF)
    st.mla_paged(pc, kvidx=True)
    st.kvidx.fill_(0x7ABC)
    st.mla_paged(pc, kvidx=True)     # a second call rewrites every index
    out_p, lse_p, kv = _np(st.out).copy(), _np(st.lse).copy(), _np(st.kvidx).copy()
    st.mla()
    return out_p, lse_p, kv, _np(st.out), _np(st.lse)


@pytest.mark.parametrize("page_rows", PAGES)
def test_paged_mla_isolated(case, page_rows):
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec, xn, ref, xg = case
    _say(f"paged mla {spec.name} page_rows={page_rows}")
    pc = W.make_paged_cache(xg, page_rows)
    st = DsaStep(xg)
    st.tok.copy_(torch.from_numpy(ref["tok"]))
    out_p, lse_p, kv, out_f, lse_f = _run_both(st, pc)
    want = _paged_oracle(xn, pc, spec, ref["tok"])
    assert np.array_equal(kv, want["kvidx"]), "physical index rows"
    worst = PT.check_mla(out_p, lse_p, want["out_f64"], want["lse"])
    assert np.array_equal(out_p.view(np.uint16), out_f.view(np.uint16)), "paged vs flat output"
    assert np.array_equal(lse_p.view(np.uint32), lse_f.view(np.uint32)), "paged vs flat lse"
    _say(f"paged mla worst rel err {worst:.3g}")


def test_paged_fused_chain(case):
    """The fused decode step with the paged attention: its selection is the
    GPU's own, so the paged result is compared with the flat call's on it and
    with the oracle on the rows whose selection equals the oracle's."""
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec, xn, ref, xg = case
    _say(f"paged fused chain {spec.name}")
    pc = W.make_paged_cache(xg, 16, seed=1)
    st = DsaStep(xg)
    st.run_fused(incremental=False, paged=pc)
    st.run_fused(incremental=True, paged=pc)
    out_p, lse_p = _np(st.out).copy(), _np(st.lse).copy()
    tok_g = _np(st.tok)
    st.mla()
    assert np.array_equal(out_p.view(np.uint16), _np(st.out).view(np.uint16))
    assert np.array_equal(lse_p.view(np.uint32), _np(st.lse).view(np.uint32))
    want = _paged_oracle(xn, pc, spec, ref["tok"])
    for q in range(spec.Q):
        if np.array_equal(tok_g[q], ref["tok"][q]):
            PT.check_mla(out_p, lse_p, want["out_f64"], want["lse"], rows=[q])


FULL = {   # workload: (page rows, sampled queries)
    "decode32k": (64, [0, 5, 15]),
    "longctx": (16, [0, 3]),       # 8192 blocks in the longest table row
    "mixed64": (64, [0, 17, 40, 63]),
}


@pytest.mark.parametrize("name", sorted(FULL))
def test_paged_mla_fullsize(name):
    """Full-size workloads in the launch configuration of the step: every
    physical index row exactly, sampled queries against the oracle, all
    queries bit-equal to the flat call."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd.pipeline import DsaStep
    page_rows, sample = FULL[name]
    spec = W.spec_by_name(name)
    _say(f"paged fullsize {name}: inputs")
    x = W.make_inputs(spec, seed=0)
    xn = x.numpy()
    xg = x.to("cuda")
    tok = W.random_selection(spec, seed=0)
    pc = W.make_paged_cache(xg, page_rows)
    st = DsaStep(xg)
    st.tok.copy_(tok)
    _say(f"paged fullsize {name}: GPU, {pc.n_pages} pages, table {tuple(pc.block_table.shape)}")
    out_p, lse_p, kv, out_f, lse_f = _run_both(st, pc)
    table = pc.block_table.cpu().numpy()
    assert np.array_equal(kv, O.kv_index(tok.numpy(), xn["q_req"], table, page_rows))
    assert np.array_equal(out_p.view(np.uint16), out_f.view(np.uint16))
    assert np.array_equal(lse_p.view(np.uint32), lse_f.view(np.uint32))
    _say(f"paged fullsize {name}: oracle on queries {sample}")
    want = _paged_oracle(xn, pc, spec, tok.numpy(), queries=sample)
    worst = PT.check_mla(out_p, lse_p, want["out_f64"], want["lse"], rows=sample)
    _say(f"paged fullsize {name}: ok, worst rel err {worst:.3g}")
