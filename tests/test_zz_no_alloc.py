"""dsa_sparse_mla_decode_noalloc (the attention call without a workspace
argument, for callers that cannot allocate) against dsa_sparse_mla_decode with
a workspace, through the C ABI: two calls in a row on the same GPU, the second
on a smaller input, each bit-equal to the workspace call on the same inputs
(the same kernels) and within the attention tolerance of the oracle; a call
whose partials would not fit the fixed array is refused before any launch."""
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


def _case(name, seed):
    spec = W.spec_by_name(name)
    x = W.make_inputs(spec, seed=seed)
    tok = W.random_selection(spec, seed=seed)
    return spec, x, tok


def test_noalloc_equals_workspace_call_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd import dsa
    # first the larger input (14 MiB of partials), then a smaller one (0.3 MiB)
    for name, seed in (("medium_pairs", 21), ("medium_fp8", 22)):
        spec, x, tok = _case(name, seed)
        xn = x.numpy()
        xg = x.to("cuda")
        tg = tok.cuda()
        dt = dsa.LATENT_FP8_E4M3 if spec.latent_fp8 else dsa.LATENT_BF16
        need = dsa.sparse_mla_decode_workspace_size(spec.Q, spec.mla_heads, spec.latent,
                                                    spec.out_width, dt)
        _say(f"noalloc attention {name}: Q={spec.Q} out_width={spec.out_width} "
             f"partials {need} bytes of {dsa.MLA_SCRATCH_BYTES}")
        assert 0 < need <= dsa.MLA_SCRATCH_BYTES
        outs = []
        for noalloc in (False, True):
            out = torch.empty(spec.Q, spec.mla_heads, spec.latent, dtype=torch.int16, device="cuda")
            lse = torch.empty(spec.Q, spec.mla_heads, dtype=torch.float32, device="cuda")
            out.view(torch.uint8).fill_(0xFF)
            lse.view(torch.uint8).fill_(0xFF)
            if noalloc:
                dsa.dsa_sparse_mla_decode_noalloc(xg.q_mla, xg.ckv, xg.ckv_scale, xg.kv_off,
                                                  xg.q_req, tg, spec.sm_scale, out, lse)
            else:
                ws = torch.empty(need, dtype=torch.uint8, device="cuda")
                dsa.dsa_sparse_mla_decode(xg.q_mla, xg.ckv, xg.ckv_scale, xg.kv_off, xg.q_req, tg,
                                          spec.sm_scale, out, lse, ws)
            outs.append((_np(out), _np(lse)))
        (o_ws, l_ws), (o_na, l_na) = outs
        assert np.array_equal(o_ws.view(np.uint16), o_na.view(np.uint16)), f"{name}: out differs"
        assert np.array_equal(l_ws.view(np.uint32), l_na.view(np.uint32)), f"{name}: lse differs"
        want = O.sparse_mla_decode(xn["q_mla"], xn["ckv"], xn["ckv_scale"], xn["kv_off"],
                                   xn["q_req"], tok.numpy(), spec.sm_scale)
        worst = PT.check_mla(o_na, l_na, want["out_f64"], want["lse"])
        _say(f"noalloc attention {name}: bit-equal to the workspace call, worst rel err {worst:.3g}")


def test_noalloc_refuses_oversized_before_launch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_fp32_amd import dsa
    # 256 queries of 4096 ids with 64 heads: more partials than the fixed array
    Q, Hm, L, ow = 256, 64, 512, 4096
    need = dsa.sparse_mla_decode_workspace_size(Q, Hm, L, ow, dsa.LATENT_BF16)
    assert need > dsa.MLA_SCRATCH_BYTES
    _say(f"noalloc attention refuses {need} bytes")
    q = torch.zeros(Q, Hm, L, dtype=torch.int16, device="cuda")
    ckv = torch.zeros(64, L, dtype=torch.int16, device="cuda")
    kv_off = torch.zeros(1, dtype=torch.int32, device="cuda")
    q_req = torch.zeros(Q, dtype=torch.int32, device="cuda")
    tok = torch.full((Q, ow), -1, dtype=torch.int32, device="cuda")
    out = torch.full((Q, Hm, L), 0x1234, dtype=torch.int16, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_sparse_mla_decode_noalloc(q, ckv, None, kv_off, q_req, tok, 1.0, out)
    assert e.value.code == dsa.DSA_ERR_UNSUPPORTED
    assert bool((out == 0x1234).all()), "outputs touched by a refused call"
