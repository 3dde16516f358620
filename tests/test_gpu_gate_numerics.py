"""The head-gate numerics report of stkernel pull request #227 ("indexer fp32
head-gate split-K", its numerics bullet), on this library: 2,480 rows of the
decode product [16, 4096] x [4096, 16] in fp32, drawn over 155 seeds, through
the separate call and through the fused split-K path (partials written by the
gate+compress launch, added in slice order by the gated index scores), each
against the oracle's fp64 product.  Reported per path, as the page reports its
own: max |diff|, max |diff| relative to the row's largest |w|, top-1 head flips
and top-4 head set changes.  Asserted: max |diff| <= 1e-5, and no flip and no
set change except where the oracle's own gap at that rank is within the
tolerance (a tie the tolerance allows either way)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import parity as PT
from sparse_attention_fp32_amd import workloads as W

pytestmark = pytest.mark.gpu

M, K, N = 16, 4096, 16
SEEDS = 155                       # 155 x 16 = 2,480 rows


def _say(msg):
    sys.stdout.write(f"\n[gpu-case] {msg}\n")
    sys.stdout.flush()


def _report(name, w_gpu, w_ref):
    d = np.abs(w_gpu.astype(np.float64) - w_ref)
    rowmax = np.abs(w_ref).max(axis=1, keepdims=True)
    rel = float((d / rowmax).max())
    order_r = np.argsort(-w_ref, axis=1, kind="stable")
    order_g = np.argsort(-w_gpu.astype(np.float64), axis=1, kind="stable")
    srt = -np.sort(-w_ref, axis=1)
    gap1 = srt[:, 0] - srt[:, 1]          # the oracle's margin of its top-1 head
    gap4 = srt[:, 3] - srt[:, 4]          # ... and of its top-4 set
    flip1 = order_r[:, 0] != order_g[:, 0]
    set4 = np.array([set(a[:4]) != set(b[:4]) for a, b in zip(order_r, order_g)])
    tie = 2 * PT.GATE_TOL
    _say(f"head-gate {name}: {w_ref.shape[0]} rows, max|diff| {d.max():.3g}, "
         f"max|diff|/row max {rel:.3g}, top-1 flips {int(flip1.sum())}, "
         f"top-4 set changes {int(set4.sum())} (oracle gaps within {tie:g}: "
         f"top-1 {int((gap1 <= tie).sum())}, top-4 {int((gap4 <= tie).sum())})")
    assert d.max() <= PT.GATE_TOL, f"{name}: max|diff| {d.max():.3g}"
    assert not np.any(flip1 & (gap1 > tie)), f"{name}: top-1 flips away from a tie"
    assert not np.any(set4 & (gap4 > tie)), f"{name}: top-4 set changes away from a tie"
    return float(d.max()), rel, int(flip1.sum()), int(set4.sum())


def test_head_gate_numerics_report():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd import dsa
    from sparse_attention_fp32_amd.pipeline import DsaStep
    # a small cache (the fused path's compression runs beside the head-gate; only w is read)
    spec = W.Spec("gate_report", lengths=[64] * M, pads=[0] * M, kpool=4, index_heads=N,
                  index_dim=128, hidden=K, select_k=4, out_width=16, mla_heads=8)
    x = W.make_inputs(spec, seed=0).to("cuda")
    st = DsaStep(x)
    assert st.nslices > 1, "the fused path must take the split-K form at this shape"
    w_sep = np.empty((SEEDS * M, N), dtype=np.float32)
    w_fus = np.empty_like(w_sep)
    w_ref = np.empty((SEEDS * M, N), dtype=np.float64)
    sep = torch.empty(M, N, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(1, dsa.head_gate_workspace_size(M, K, N)), dtype=torch.uint8,
                     device="cuda")
    _say(f"head-gate report: {SEEDS} draws of [{M},{K}]x[{K},{N}], {st.nslices} K slices fused")
    for i in range(SEEDS):
        h, Wm = W.gate_operands(M, K, N, seed=10_000 + i)
        x.hidden.copy_(h)
        x.W.copy_(Wm)
        dsa.dsa_head_gate(x.hidden, x.W, sep, ws)
        st.gate_compress()
        st.index_scores_gated()
        torch.cuda.synchronize()
        rows = slice(i * M, (i + 1) * M)
        w_sep[rows] = sep.cpu().numpy()
        w_fus[rows] = st.w.cpu().numpy()
        w_ref[rows] = O.head_gate(h.numpy(), Wm.numpy())
    _report("separate call", w_sep, w_ref)
    _report("fused split-K", w_fus, w_ref)
