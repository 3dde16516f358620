"""GPU parity of the attention's online softmax when a head's running maximum
keeps growing (Atlas glm5next_dsa page, the MASKED_ATTN_MAX_KEYS note: the
serving kernel keeps an online softmax).

The kernel moves a head's reference maximum only when a later sub-chunk's
logits exceed it by more than 2^8 (log2 domain) and then rescales that head's
partial output and sum.  With the configs' N(0,1) inputs the first sub-chunk's
maximum is almost never exceeded by that much, so those paths would go
untested.  Here every request's latent rows grow with their position -- row t
is scaled by 2^(6t/T_r), so logits end up to 64 times their starting size --
and each query's selection lists its ids in ascending order, so the logits of
a workgroup's later sub-chunks keep overtaking the reference (the shape with
sm_scale 1/sqrt(512) grows by 2^(10.5 t/T_r) instead, for the same range of
logits).  bf16 rows are
scaled and rounded to bf16 (RNE) before the call, fp8 rows through their row
scale; both sides get the same bits.  Flat and paged caches, one and several
chunks per query."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = ("medium", "medium_fp8", "medium_pairs", "medium_prefill")


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _growing_rows(x, spec):
    """Scale request r's row t by 2^(g t / T_r), in place (CPU tensors), with
    g = 6 + log2(1 / sm_scale)."""
    kv_off = x.kv_off.numpy()
    g = 6.0 + np.log2(1.0 / spec.sm_scale)
    f = np.ones(x.ckv.shape[0], dtype=np.float64)
    for r, T in enumerate(spec.lengths):
        t = np.arange(T, dtype=np.float64)
        f[kv_off[r]:kv_off[r] + T] = 2.0 ** (g * t / max(T, 1))
    if spec.latent_fp8:
        x.ckv_scale.copy_(torch.from_numpy((x.ckv_scale.numpy().astype(np.float64) * f)
                                           .astype(np.float32)))
    else:
        rows = O.bf16_bits_to_f64(x.ckv.numpy()) * f[:, None]
        x.ckv.copy_(torch.from_numpy(O.f64_to_bf16_bits(rows).view(np.int16)))


def _overtakes(xn, spec, tok):
    """Fraction of (query, head) rows whose log2-domain logits, in selection
    order, rise more than 2^8 above the maximum of their first 32 ids (so the
    kernel's reference maximum must move and O be rescaled)."""
    hits = rows = 0
    for q in range(tok.shape[0]):
        ids = tok[q][tok[q] >= 0]
        if len(ids) <= 32:
            continue
        r = int(xn["q_req"][q])
        lat = O.latent_rows_f64(xn["ckv"], xn["ckv_scale"], int(xn["kv_off"][r]) + ids)
        lg = (O.bf16_bits_to_f64(xn["q_mla"][q]) @ lat.T) * spec.sm_scale / np.log(2.0)
        hits += int(np.sum(lg[:, 32:].max(axis=1) > lg[:, :32].max(axis=1) + 8.0))
        rows += lg.shape[0]
    return hits / max(rows, 1)


def _ascending_selection(spec, seed):
    """Random ids per query (W.random_selection), sorted ascending into the
    slots that hold ids; the -1 slots stay where they were."""
    tok = W.random_selection(spec, seed=seed).numpy()
    for q in range(tok.shape[0]):
        slots = np.nonzero(tok[q] >= 0)[0]
        tok[q, slots] = np.sort(tok[q, slots])
    return torch.from_numpy(tok)


@pytest.mark.parametrize("paged", (False, True))
@pytest.mark.parametrize("name", SHAPES)
def test_mla_growing_logits(name, paged):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec = W.spec_by_name(name)
    _say(f"sparse_mla growing logits {name} paged={paged}")
    x = W.make_inputs(spec, seed=11)
    _growing_rows(x, spec)
    tok = _ascending_selection(spec, seed=11)
    xn = x.numpy()
    xg = x.to("cuda")
    st = DsaStep(xg)
    st.tok.copy_(tok)
    for t in (st.out, st.lse):
        t.view(torch.uint8).fill_(0xFF)
    if paged:
        pc = W.make_paged_cache(xg, 7, seed=11)
        st.mla_paged(pc)
    else:
        st.mla()
    want = O.sparse_mla_decode(xn["q_mla"], xn["ckv"], xn["ckv_scale"], xn["kv_off"], xn["q_req"],
                               tok.numpy(), spec.sm_scale)
    worst = PT.check_mla(_np(st.out), _np(st.lse), want["out_f64"], want["lse"])
    # the inputs do what they are for: most rows' logits rise by more than
    # the 2^8 (log2) the reference tolerates
    frac = _overtakes(xn, spec, tok.numpy())
    assert frac >= 0.5, frac
    _say(f"growing logits {name} paged={paged}: worst rel err {worst:.3g}, "
         f"rows that move their reference: {frac:.0%}")


# Selections wide enough that a query's ids split into 32 and 64 chunks, so
# the merge of the chunk partials runs in several batches of 16 and (with the
# growing rows and ascending ids) every later batch raises the running max.
WIDE = [
    W.Spec("wide4096", lengths=[9000, 12000], pads=[0, 5], kpool=4, index_heads=16,
           index_dim=128, hidden=512, select_k=1024, out_width=4096, mla_heads=64),
    W.Spec("wide8192_fp8", lengths=[20000], pads=[3], kpool=4, index_heads=16,
           index_dim=128, hidden=512, select_k=2048, out_width=8192, mla_heads=64,
           latent_fp8=True),
]


@pytest.mark.parametrize("paged", (False, True))
@pytest.mark.parametrize("spec", WIDE, ids=[s.name for s in WIDE])
def test_mla_wide_selection(spec, paged):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd.pipeline import DsaStep
    _say(f"sparse_mla wide selection {spec.name} paged={paged}")
    x = W.make_inputs(spec, seed=12)
    _growing_rows(x, spec)
    tok = _ascending_selection(spec, seed=12)
    xn = x.numpy()
    xg = x.to("cuda")
    st = DsaStep(xg)
    st.tok.copy_(tok)
    for t in (st.out, st.lse):
        t.view(torch.uint8).fill_(0xFF)
    if paged:
        st.mla_paged(W.make_paged_cache(xg, 64, seed=12))
    else:
        st.mla()
    want = O.sparse_mla_decode(xn["q_mla"], xn["ckv"], xn["ckv_scale"], xn["kv_off"], xn["q_req"],
                               tok.numpy(), spec.sm_scale)
    worst = PT.check_mla(_np(st.out), _np(st.lse), want["out_f64"], want["lse"])
    _say(f"wide selection {spec.name} paged={paged}: worst rel err {worst:.3g}")
