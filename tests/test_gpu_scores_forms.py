"""The index scores' query-block form (many queries per request, as in
prefill) at every key width it is built for and at narrow head counts,
against the oracle: plain weights and head-gate partials of several slice
counts.  Each shape has at least 256 queries and enough 8-query blocks times
256-pool blocks (>= 256) for the library to take that form; the queries of
one request are followed by eighteen of a request with at most one full pool
(one 8-query block entirely its own) and then by another request's, so some
blocks span requests."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu

# (name, index heads H, key width D, kpool)
FORMS = [("h12_d64_k8", 12, 64, 8), ("h4_d32_k4", 4, 32, 4), ("h16_d256_k2", 16, 256, 2),
         ("h16_d128_k4", 16, 128, 4)]


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def _spec(name, H, D, kpool):
    rng = np.random.default_rng(H * 1000 + D + kpool)
    lengths, pads = [2600, 33, 1500], [7, 30, 0]
    # queries 704..711 all belong to request 1, which has no full pool for
    # kpool >= 4 (a block of its own); 696..703 and 712..719 span requests
    q_req = [0] * 700 + [1] * 18 + [2] * 385
    q_pos = sorted(int(x) for x in rng.integers(0, 2600, size=700)) + \
        list(range(32, 14, -1)) + list(range(0, 1500, 3))[:385]
    return W.Spec(name, lengths=lengths, pads=pads, kpool=kpool, index_heads=H, index_dim=D,
                  hidden=256, select_k=8, out_width=8 * kpool, mla_heads=8, q_req=q_req,
                  q_pos=q_pos)


@pytest.mark.parametrize("name,H,D,kpool", FORMS)
def test_query_block_scores(name, H, D, kpool):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd import dsa
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec = _spec(name, H, D, kpool)
    Q, pst = spec.Q, spec.pstride()
    assert Q >= 256 and math.ceil(pst / 256) * math.ceil(Q / 8) >= 256
    _say(f"query-block scores {name}: Q={Q} pstride={pst}")
    x = W.make_inputs(spec, seed=7)
    xn = x.numpy()
    comp = O.kpool_compress(xn["k"], xn["gate"], xn["ape"], xn["valid"], xn["tok_off"],
                            xn["pool_off"], xn["ln_w"], xn["ln_b"], spec.eps, kpool)
    w = O.head_gate(xn["hidden"], xn["W"])
    ref_s, ref_c = O.index_scores(xn["qi"], w, comp["keys"], comp["pool_start"],
                                  comp["pool_valid"], xn["pool_off"], comp["n_pools"],
                                  xn["q_req"], xn["q_pos"], kpool, pst)
    st = DsaStep(x.to("cuda"))
    ncap = len(comp["pool_start"])
    st.w.copy_(torch.from_numpy(w))
    st.keys[:ncap].copy_(torch.from_numpy(comp["keys"].view(np.int16)))
    st.pool_start[:ncap].copy_(torch.from_numpy(comp["pool_start"]))
    st.pool_valid[:ncap].copy_(torch.from_numpy(comp["pool_valid"]))
    st.n_pools.copy_(torch.from_numpy(comp["n_pools"]))

    def scores_now():
        torch.cuda.synchronize()
        return st.scores.cpu().numpy(), st.cand.cpu().numpy()

    st.scores.view(torch.uint8).fill_(0xFF)
    st.cand.fill_(0xFF)
    st.index_scores()
    PT.check_scores(*scores_now(), ref_s, ref_c)

    K = xn["hidden"].shape[1]
    for ns in (1, 3, 40):
        parts = [O.head_gate(xn["hidden"][:, c], xn["W"][c])
                 for c in np.array_split(np.arange(K), ns)]
        part = torch.from_numpy(np.stack(parts, axis=1).astype(np.float32).reshape(-1)).cuda()  # [Q, ns, H]
        st.scores.view(torch.uint8).fill_(0xFF)
        st.cand.fill_(0xFF)
        st.w.view(torch.uint8).fill_(0xFF)
        xg = st.x
        dsa.dsa_index_scores_gated(xg.qi, part, ns, st.w, st.keys, st.pool_start, st.pool_valid,
                                   xg.pool_off, st.n_pools, xg.q_req, xg.q_pos, kpool, st.scores,
                                   st.cand)
        torch.cuda.synchronize()
        PT.check_gate(st.w.cpu().numpy(), w)
        PT.check_scores(*scores_now(), ref_s, ref_c)
