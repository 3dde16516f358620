"""Parity at the five workloads' full sizes, in the launch configuration the
bench times, on outputs the oracle computes for a sample of queries.  Each
stage is also run isolated on the oracle's upstream outputs for those
queries."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu

SAMPLES = {
    "tiny": [0, 1],
    "decode32k": [0, 3, 9, 15],
    "longctx": [0, 1, 2, 3],
    "prefill4k": [0, 1, 2, 3, 100, 254, 255, 1000, 2047, 4095],
    "mixed64": None,   # the six mostly-padded requests plus six others
    "decode262k": [0],
}


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("name", W.WORKLOADS)
def test_fullsize(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec = W.spec_by_name(name)
    sample = SAMPLES[name]
    if sample is None:
        short = [i for i, p in enumerate(spec.pads) if p > 0]
        sample = sorted(short + [i for i in range(spec.Q) if i not in short][:6])
    _say(f"fullsize {name}: generating inputs")
    x = W.make_inputs(spec, seed=0)
    xn = x.numpy()
    xg = x.to("cuda")
    reqs = sorted({int(xn["q_req"][q]) for q in sample})

    _say(f"fullsize {name}: oracle on queries {sample}")
    ref = O.dsa_step(xn, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                     spec.sm_scale, queries=sample, always_select_tail=spec.always_select_tail)

    ncap = int(xn["pool_off"][-1])

    def check_chained(st, label):
        PT.check_gate(_np(st.w), ref["w"])
        g = {"keys": _np(st.keys).view(np.uint16)[:ncap], "pool_start": _np(st.pool_start)[:ncap],
             "pool_valid": _np(st.pool_valid)[:ncap], "n_pools": _np(st.n_pools)}
        flips = PT.check_compress(g, ref, requests=reqs, pool_off=xn["pool_off"])
        ndiff = PT.check_chained_rows(_np(st.sel), _np(st.tok), _np(st.out), _np(st.lse), ref,
                                      PT.oracle_expect(xn, spec, ref["pool_start"]), rows=sample)
        _say(f"fullsize {name}: {label} ok; key ulp flips in sample {flips}, boundary swaps {ndiff}")

    # the fused decode calls the bench times: full compression, then the cached-pool step
    _say(f"fullsize {name}: fused GPU chain")
    stf = DsaStep(xg)
    stf.run_fused(incremental=False)
    stf.run_fused(incremental=True)
    check_chained(stf, "fused chain")
    del stf

    _say(f"fullsize {name}: GPU chain of the six calls (full compression, then the cached-pool step)")
    st = DsaStep(xg)
    st.run(incremental=False)
    st.run(incremental=True)
    check_chained(st, "chain")

    # stage isolation on the sampled queries: oracle inputs into the GPU buffers
    idx = np.concatenate([np.arange(xn["pool_off"][r], xn["pool_off"][r + 1]) for r in reqs])
    ti = torch.from_numpy(idx).cuda()
    st.keys[ti] = torch.from_numpy(ref["keys"][idx].view(np.int16)).cuda()
    st.pool_start[ti] = torch.from_numpy(ref["pool_start"][idx]).cuda()
    st.pool_valid[ti] = torch.from_numpy(ref["pool_valid"][idx]).cuda()
    st.n_pools.copy_(torch.from_numpy(ref["n_pools"]))
    st.w.copy_(torch.from_numpy(ref["w"]))
    st.index_scores()
    PT.check_scores(_np(st.scores), _np(st.cand), ref["scores"], ref["cand"], rows=sample)
    tq = torch.tensor(sample).cuda()
    st.scores[tq] = torch.from_numpy(ref["scores"][sample]).cuda()
    st.cand[tq] = torch.from_numpy(ref["cand"][sample]).cuda()
    st.topk()
    PT.check_sel_exact(_np(st.sel), ref["sel"], rows=sample)
    st.sel[tq] = torch.from_numpy(ref["sel"][sample]).cuda()
    st.expand()
    tok2 = _np(st.tok)
    for q in sample:
        assert np.array_equal(tok2[q], ref["tok"][q]), f"tok q={q}"
    st.tok[tq] = torch.from_numpy(ref["tok"][sample]).cuda()
    st.mla()
    worst = PT.check_mla(_np(st.out), _np(st.lse), ref["out_f64"], ref["lse"], rows=sample)
    _say(f"fullsize {name}: isolated stages ok, MLA worst rel err {worst:.3g}")
