"""The single-chunk attention of prefill-sized batches (one chunk per query,
so no partials; workgroups placed XCD-aware, both head blocks of a query on
one XCD), bf16 and fp8 rows.

Each case runs the flat call and the paged call over a copy of the same rows
in shuffled pages, and the two must agree bit for bit (the same arithmetic on
the same rows).  Sampled queries -- the first, the last, empty ones and a
seeded draw -- are checked against the oracle's attention.  Ids are drawn per
query from its request's rows, with -1 slots inside and at the end of the row
and some rows with no id at all; 1097 queries (not a multiple of the eight
XCDs, so the order's padding workgroups leave at once) and 4100."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import dsa
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def _ids(rng, spec, q_req):
    """[Q, out_width] ids: distinct rows of each query's request, some -1 slots
    inside the row, a -1 tail, and every 97th row empty."""
    tok = np.full((len(q_req), spec.out_width), -1, dtype=np.int32)
    for q, r in enumerate(q_req):
        if q % 97 == 5:
            continue
        T = spec.lengths[r]
        n = min(int(rng.integers(1, spec.out_width + 1)), T)
        tok[q, :n] = rng.choice(T, size=n, replace=False)
        holes = rng.random(n) < 0.05
        tok[q, :n][holes] = -1
    return tok


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("nq", [1097, 4100])
def test_mla_single_chunk_large_batch(fp8, nq):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    base = W.spec_by_name("medium_prefill")
    rng = np.random.default_rng(1000 + nq + int(fp8))
    q_req = sorted(int(r) for r in rng.integers(0, base.B, size=nq))
    q_pos = [base.lengths[r] - 1 for r in q_req]
    spec = dataclasses.replace(base, latent_fp8=fp8, q_req=q_req, q_pos=q_pos)
    _say(f"single-chunk attention: {nq} queries, {'fp8' if fp8 else 'bf16'} rows")
    x = W.make_inputs(spec, seed=7, device="cuda")
    tok = _ids(rng, spec, q_req)
    Hm, L = spec.mla_heads, spec.latent
    tok_g = torch.from_numpy(tok).cuda()
    q_req_g = torch.tensor(q_req, dtype=torch.int32, device="cuda")
    dt = dsa.LATENT_FP8_E4M3 if fp8 else dsa.LATENT_BF16
    n_ws = dsa.sparse_mla_decode_workspace_size(nq, Hm, L, spec.out_width, dt)
    assert n_ws == 0, "one chunk per query: no partials"
    outs = []
    for paged in (False, True):
        out = torch.full((nq, Hm, L), -1, dtype=torch.int16, device="cuda")
        lse = torch.full((nq, Hm), float("nan"), dtype=torch.float32, device="cuda")
        if paged:
            pc = W.make_paged_cache(x, 16, seed=3)
            dsa.dsa_sparse_mla_decode_paged(x.q_mla, pc.ckv, pc.ckv_scale, pc.block_table,
                                            pc.page_rows, q_req_g, tok_g, spec.sm_scale, out, lse)
        else:
            dsa.dsa_sparse_mla_decode(x.q_mla, x.ckv, x.ckv_scale, x.kv_off, q_req_g, tok_g,
                                      spec.sm_scale, out, lse)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    (of, lf), (op, lp) = outs
    assert np.array_equal(of, op), "flat and paged outputs differ"
    assert np.array_equal(lf.view(np.uint32), lp.view(np.uint32)), "lse differs"
    empty = [q for q in range(nq) if not (tok[q] >= 0).any()]
    assert empty, "the case must hold empty rows"
    sample = sorted({0, nq - 1, *empty[:3], *(int(v) for v in rng.choice(nq, 20, replace=False))})
    xn = x.numpy()
    ref = O.sparse_mla_decode(xn["q_mla"], xn["ckv"], xn["ckv_scale"], xn["kv_off"],
                              np.asarray(q_req), tok, spec.sm_scale, queries=sample)
    worst = PT.check_mla(of, lf, ref["out_f64"], ref["lse"], rows=sample)
    _say(f"single-chunk attention: flat and paged bit-equal; oracle rel err {worst:.2e} "
         f"on {len(sample)} queries")
