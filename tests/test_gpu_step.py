"""GPU: the step executor (dsa_decode_step, one host call per decode step).

Its results must be those of the fused calls made one by one (the same
kernels), bit for bit: full and cached-pool steps, flat and paged attention,
the tail on the shapes that ask for it.  The executor's own step is also held
to the oracle's chain, and captured in a HIP graph whose replays (with eager
work between them) must each give the eager result."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu

# every output of the step; the first four are the compression's, which a
# cached-pool step updates only where the newest rows land
OUTS = ("keys", "pool_start", "pool_valid", "n_pools", "w", "scores", "cand", "sel", "tok",
        "out", "lse")
STEP_OUTS = OUTS[4:]


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


@pytest.fixture(scope="module", params=W.PARITY_SHAPES)
def case(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd.pipeline import DsaStep  # noqa: F401  (loads libdsa)
    spec = W.spec_by_name(request.param)
    x = W.make_inputs(spec, seed=3)
    xn = x.numpy()
    ref = O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                     spec.sm_scale, always_select_tail=spec.always_select_tail)
    return spec, xn, ref, x.to("cuda")


def _poison(st, names):
    for n in names:
        getattr(st, n).view(torch.uint8).fill_(0xFF)


def _snap(st, names=OUTS, kvidx=False):
    torch.cuda.synchronize()
    out = [getattr(st, n).cpu().numpy().view(np.uint8).copy() for n in names]
    if kvidx:
        out.append(st.kvidx.cpu().numpy().view(np.uint8).copy())
    return out


def _same(a, b, what):
    for i, (u, v) in enumerate(zip(a, b)):
        assert np.array_equal(u, v), f"{what}: output {i} differs"


def _fused(st, incremental, pc):
    st.run_fused(incremental=incremental, paged=pc)


def test_step_equals_fused_calls(case):
    spec, xn, ref, xg = case
    from sparse_attention_fp32_amd.pipeline import DsaStep
    _say(f"decode step executor {spec.name}")
    st = DsaStep(xg)
    full, inc = st.step_args(incremental=False), st.step_args(incremental=True)
    # full step: every output from scratch
    _poison(st, OUTS)
    _fused(st, False, None)
    a = _snap(st)
    _poison(st, OUTS)
    st.run_step(full)
    b = _snap(st)
    _same(a, b, "full step")
    PT.check_gate(_np(st.w), ref["w"])
    nd = PT.check_chained_rows(_np(st.sel), _np(st.tok), _np(st.out), _np(st.lse), ref,
                               PT.oracle_expect(xn, spec, ref["pool_start"]))
    # cached-pool step over those pools
    _poison(st, STEP_OUTS)
    _fused(st, True, None)
    a = _snap(st)
    _poison(st, STEP_OUTS)
    st.run_step(inc)
    _same(a, _snap(st), "cached-pool step")
    _say(f"decode step executor {spec.name}: equal to the calls, boundary swaps {nd}")


@pytest.mark.parametrize("post_ln", (True, False))
def test_step_live_lengths(post_ln):
    """Live lengths inside the requests' regions (seq_len) and rows stored
    normalised (post_ln False): the executor passes both to the compression."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec = W.spec_by_name("medium_live")
    _say(f"decode step executor live lengths post_ln={post_ln}")
    xg = W.make_inputs(spec, seed=5).to("cuda")
    st = DsaStep(xg)
    st.seq_len = torch.tensor(spec.live_lengths(), dtype=torch.int32, device="cuda")
    st.post_ln = post_ln
    for incremental in (False, True):
        names = STEP_OUTS if incremental else OUTS
        args = st.step_args(incremental=incremental)
        _poison(st, names)
        _fused(st, incremental, None)
        a = _snap(st)
        _poison(st, names)
        st.run_step(args)
        _same(a, _snap(st), f"live step incremental={incremental}")


@pytest.mark.parametrize("page_rows", (7, 64))
def test_step_paged_equals_fused_calls(case, page_rows):
    spec, xn, ref, xg = case
    from sparse_attention_fp32_amd.pipeline import DsaStep
    _say(f"decode step executor paged {spec.name} page_rows={page_rows}")
    st = DsaStep(xg)
    pc = W.make_paged_cache(xg, page_rows, seed=4)
    st.run_fused()
    args = st.step_args(incremental=True, paged=pc, kvidx=True)
    _poison(st, STEP_OUTS)
    st.kvidx.fill_(-7)
    st.run_fused(incremental=True)           # (the flat attention: tok, sel, ... as below)
    st.mla_paged(pc, kvidx=True)
    a = _snap(st, kvidx=True)
    _poison(st, STEP_OUTS)
    st.kvidx.fill_(-7)
    st.run_step(args)
    _same(a, _snap(st, kvidx=True), "paged step")
    # the paged attention equals the flat one (the same rows through the table)
    out_p = _np(st.out).copy()
    _fused(st, True, None)
    assert np.array_equal(out_p.view(np.uint8), _np(st.out).view(np.uint8))


def test_step_in_graph(case):
    """dsa_decode_step captured in a graph: three replays, each after eager
    work that overwrites the outputs, each equal to the eager step."""
    spec, xn, ref, xg = case
    from sparse_attention_fp32_amd.pipeline import DsaStep
    _say(f"decode step executor in a graph {spec.name}")
    st = DsaStep(xg)
    st.run_fused()
    args = st.step_args(incremental=True)
    st.run_step(args)
    want = _snap(st)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run_step(args)                     # warm on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run_step(args)
    for rep in range(3):
        _poison(st, STEP_OUTS)
        torch.cuda.synchronize()
        g.replay()
        _same(want, _snap(st), f"graph replay {rep}")


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()
