"""GPU parity of the cache-write side of a decode step against the oracle:
live lengths inside larger request regions (compression reads only the live
rows), compression of rows normalised when stored (no LayerNorm after
pooling), dsa_indexer_store, dsa_write_geom, and a captured graph of whole
decode steps replayed while the live lengths grow -- the geometry comes from
the device each replay, so every replay must match the oracle at its own
lengths."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16_rows(rng, shape):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16)


def _check_rows(got, want, label):
    """Stored k rows: equal, or (LayerNorm rows) within the key rule."""
    PT.check_compress({"keys": got, "pool_start": np.zeros(len(got), np.int32),
                       "pool_valid": np.zeros(len(got), np.uint8), "n_pools": np.zeros(1, np.int32)},
                      {"keys": want, "pool_start": np.zeros(len(want), np.int32),
                       "pool_valid": np.zeros(len(want), np.uint8), "n_pools": np.zeros(1, np.int32)})


@pytest.mark.parametrize("post_ln", [True, False])
@pytest.mark.parametrize("name", ["medium", "medium_fp8", "medium_live"])
def test_compress_live_lengths(name, post_ln):
    _need_gpu()
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec = W.spec_by_name(name)
    _say(f"compress live lengths {name} post_ln={post_ln}")
    x = W.make_inputs(spec, seed=0)
    xn = x.numpy()
    rng = np.random.default_rng(40)
    seq = np.array([int(rng.integers(0, n + 1)) for n in spec.lengths], dtype=np.int32)
    seq[0] = spec.lengths[0] - int(rng.integers(1, 9))
    ref = O.kpool_compress(xn["k"], xn["gate"], xn["ape"], xn["valid"], xn["tok_off"],
                           xn["pool_off"], xn["ln_w"] if post_ln else None,
                           xn["ln_b"] if post_ln else None, spec.eps, spec.kpool, seq_len=seq)
    xg = x.to("cuda")
    for fused in (False, True):
        st = DsaStep(xg)
        st.seq_len = torch.from_numpy(seq).cuda()
        st.post_ln = post_ln
        for t in (st.keys, st.pool_start, st.pool_valid, st.n_pools):
            t.view(torch.uint8).fill_(0xFF)
        if fused:
            st.gate_compress(incremental=False)
        else:
            st.compress(incremental=False)
        ncap = int(xn["pool_off"][-1])
        g = {"keys": _np(st.keys).view(np.uint16)[:ncap], "pool_start": _np(st.pool_start)[:ncap],
             "pool_valid": _np(st.pool_valid)[:ncap], "n_pools": _np(st.n_pools)}
        PT.check_compress(g, ref)


@pytest.mark.parametrize("post_ln", [True, False])
def test_indexer_store(post_ln):
    _need_gpu()
    from sparse_attention_fp32_amd import dsa
    spec = W.spec_by_name("medium_fp8")
    x = W.make_inputs(spec, seed=0)
    xn = x.numpy()
    xg = x.to("cuda")
    rng = np.random.default_rng(41)
    B, D = spec.B, spec.index_dim
    n = spec.lengths
    pos = np.array([0, n[1] - 1, n[2], -3], dtype=np.int32)   # first, last, past, before
    kn, gn = _bf16_rows(rng, (B, D)), _bf16_rows(rng, (B, D))
    _say(f"indexer_store post_ln={post_ln}")
    ln = (None, None) if post_ln else (xn["ln_w"], xn["ln_b"])
    ref = O.indexer_store(xn["k"], xn["gate"], xn["valid"], xn["tok_off"], pos, kn.numpy(),
                          gn.numpy(), ln[0], ln[1], spec.eps)
    dsa.dsa_indexer_store(kn.cuda(), gn.cuda(), torch.from_numpy(pos).cuda(), xg.tok_off, xg.k,
                          xg.gate, xg.valid, ln_w=None if post_ln else xg.ln_w,
                          ln_b=None if post_ln else xg.ln_b, eps=spec.eps)
    assert np.array_equal(_np(xg.gate), ref["gate"].astype(np.int16))
    assert np.array_equal(_np(xg.valid), ref["valid"])
    kg = _np(xg.k).view(np.uint16)
    if post_ln:
        assert np.array_equal(kg, ref["k"].view(np.uint16))
    else:
        _check_rows(kg, ref["k"].view(np.uint16), "stored rows")


def test_write_geom():
    _need_gpu()
    from sparse_attention_fp32_amd import dsa
    rng = np.random.default_rng(42)
    B, page_rows = 37, 16
    seq = rng.integers(0, 3000, size=B).astype(np.int32)
    seq[[3, 20]] = 0
    nblk = (seq + page_rows - 1) // page_rows
    n_pages = int(nblk.sum()) + 5
    table = np.zeros((B, int(nblk.max()) + 1), dtype=np.int32)
    perm = rng.permutation(n_pages)
    k = 0
    for r in range(B):
        table[r, :nblk[r]] = perm[k:k + nblk[r]]
        k += nblk[r]
    want = O.write_geom(seq, table, page_rows)
    out = {n: torch.full((B,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
           for n in ("q_req", "q_pos", "new_from", "slot")}
    dsa.dsa_write_geom(torch.from_numpy(seq).cuda(), out["q_pos"], q_req=out["q_req"],
                       new_from=out["new_from"], slot=out["slot"],
                       block_table=torch.from_numpy(table).cuda(), page_rows=page_rows,
                       n_pages=n_pages)
    for n in out:
        assert np.array_equal(_np(out[n]), want[n]), n


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("post_ln", [True, False])
def test_live_decode_graph(post_ln, fused):
    """One captured graph per variant: write_geom -> indexer_store -> the fused
    step over cached pools with the paged attention (fused: the first three
    as one dsa_gate_compress_live launch).  Between replays the host only
    writes the new live lengths and the staged rows into device buffers; each
    replay is checked against the oracle at its lengths."""
    _need_gpu()
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec = W.spec_by_name("medium_live")
    B, D = spec.B, spec.index_dim
    x = W.make_inputs(spec, seed=0)
    xn = x.numpy()
    xg = x.to("cuda")
    st = DsaStep(xg)
    st.post_ln = post_ln
    seq = np.array(spec.live, dtype=np.int32)
    st.seq_len = torch.from_numpy(seq).cuda()
    pc = W.make_paged_cache(xg, 16, seed=3)
    table = pc.block_table.cpu().numpy()
    slot = torch.empty(B, dtype=torch.int32, device="cuda")
    # the state before the first step: geometry and every pool at the initial lengths
    st.write_geom(pc, slot)
    st.gate_compress(incremental=False)
    k_new = torch.zeros(B, D, dtype=torch.int16, device="cuda")
    gate_new = torch.zeros(B, D, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run_live(k_new, gate_new, paged=pc, slot=slot, fused=fused)
    torch.cuda.synchronize()

    k, gate, valid = xn["k"].copy(), xn["gate"].copy(), xn["valid"].copy()
    ln = (None, None) if post_ln else (xn["ln_w"], xn["ln_b"])
    rng = np.random.default_rng(43)
    for step in range(6):
        grow = np.ones(B, dtype=np.int32)
        if step % 2:
            grow[1] = 0          # request 1 rewrites its newest row on odd steps
        seq = seq + grow
        kn, gn = _bf16_rows(rng, (B, D)), _bf16_rows(rng, (B, D))
        st.seq_len.copy_(torch.from_numpy(seq))
        k_new.copy_(kn)
        gate_new.copy_(gn)
        _say(f"live decode post_ln={post_ln} fused={fused} step {step}: lengths {seq.tolist()}")
        g.replay()
        torch.cuda.synchronize()

        geo = O.write_geom(seq, table, pc.page_rows)
        outs = [("q_req", xg.q_req), ("q_pos", xg.q_pos), ("new_from", xg.new_from)]
        if not fused:
            outs.append(("slot", slot))
        for name, t in outs:
            assert np.array_equal(_np(t), geo[name]), (step, name)
        stored = O.indexer_store(k, gate, valid, xn["tok_off"], geo["new_from"], kn.numpy(),
                                 gn.numpy(), ln[0], ln[1], spec.eps)
        k, gate, valid = stored["k"], stored["gate"], stored["valid"]
        assert np.array_equal(_np(xg.valid), valid)
        assert np.array_equal(_np(xg.gate).view(np.uint16), gate.view(np.uint16))
        kg = _np(xg.k).view(np.uint16)
        if post_ln:
            assert np.array_equal(kg, k.view(np.uint16))
        else:
            _check_rows(kg, k.view(np.uint16), "stored rows")
        xo = dict(xn, k=k, gate=gate, valid=valid, q_req=geo["q_req"], q_pos=geo["q_pos"])
        ref = O.dsa_step(xo, spec.kpool, spec.select_k, spec.out_width, spec.pstride(), spec.eps,
                         spec.sm_scale, always_select_tail=True, seq_len=seq, post_ln=post_ln)
        ncap = int(xn["pool_off"][-1])
        gk = {"keys": _np(st.keys).view(np.uint16)[:ncap], "pool_start": _np(st.pool_start)[:ncap],
              "pool_valid": _np(st.pool_valid)[:ncap], "n_pools": _np(st.n_pools)}
        PT.check_compress(gk, ref)
        PT.check_gate(_np(st.w), ref["w"])
        nd = PT.check_chained_rows(_np(st.sel), _np(st.tok), _np(st.out), _np(st.lse), ref,
                                   PT.oracle_expect(xo, spec, ref["pool_start"]))
        _say(f"live decode step {step}: boundary swaps {nd}")


@pytest.mark.parametrize("post_ln", [True, False])
def test_live_call_equals_three_calls(post_ln):
    """dsa_gate_compress_live leaves every buffer bit-equal to write_geom +
    indexer_store + gate_compress, step after step, including steps that
    complete a pool and an empty request that receives its first row."""
    _need_gpu()
    from sparse_attention_fp32_amd.pipeline import DsaStep
    spec = W.spec_by_name("medium_live")
    B, D = spec.B, spec.index_dim
    x = W.make_inputs(spec, seed=0)
    steps = []
    seq0 = np.array([901, 0, 1990], dtype=np.int32)
    for _ in range(2):
        st = DsaStep(x.to("cuda"))
        st.post_ln = post_ln
        st.seq_len = torch.from_numpy(seq0).cuda()
        st.write_geom()
        st.gate_compress(incremental=False)
        steps.append(st)
    rng = np.random.default_rng(44)
    seq = seq0.copy()
    for step in range(9):
        seq = seq + 1
        kn, gn = _bf16_rows(rng, (B, D)).cuda(), _bf16_rows(rng, (B, D)).cuda()
        _say(f"live call vs three calls post_ln={post_ln} step {step}: {seq.tolist()}")
        for i, st in enumerate(steps):
            st.seq_len.copy_(torch.from_numpy(seq))
            if i == 0:
                st.write_geom()
                st.store(kn, gn)
                st.gate_compress(incremental=True)
            else:
                st.gate_compress_live(kn, gn)
        a, b = steps
        for name in ("k", "gate", "valid", "q_req", "q_pos", "new_from"):
            assert np.array_equal(_np(getattr(a.x, name)).view(np.uint8),
                                  _np(getattr(b.x, name)).view(np.uint8)), (step, name)
        for name in ("keys", "pool_start", "pool_valid", "n_pools", "gate_part"):
            assert np.array_equal(_np(getattr(a, name)).view(np.uint8),
                                  _np(getattr(b, name)).view(np.uint8)), (step, name)
