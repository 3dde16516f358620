"""Top-k on adversarial score rows, exact against the oracle: ties, all-equal
rows, negative rows, rows spanning more than 15 octaves, rows with fewer
candidates than select_k, and every per-thread register tile size."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_fp32_amd import dsa

pytestmark = pytest.mark.gpu


def _rows(rng, Q, P, kind):
    if kind == "normal":
        s = rng.standard_normal((Q, P)) * 20
    elif kind == "ties":
        s = rng.choice([-1.0, 0.0, 0.5, 2.0, 2.5, 7.0], size=(Q, P))
    elif kind == "equal":
        s = np.full((Q, P), 3.25)
    elif kind == "negative":
        s = -np.abs(rng.standard_normal((Q, P))) - 1.0
    elif kind == "wide":     # magnitudes spread over ~80 octaves, both signs
        s = rng.standard_normal((Q, P)) * 2.0 ** rng.integers(-40, 40, size=(Q, P))
    elif kind == "zeros":    # +0 and -0 must tie
        s = np.where(rng.random((Q, P)) < 0.5, 0.0, -0.0)
    else:
        raise KeyError(kind)
    return s.astype(np.float32)


CASES = [(P, k, kind) for P in (30, 1000, 1024, 2047, 4096, 8192, 16384)
         for k in (1, 64, 512) for kind in ("normal", "ties", "wide")]
CASES += [(8192, 512, "equal"), (8192, 512, "negative"), (4096, 100, "zeros"),
          (16384, 256, "negative"), (1024, 2000, "normal")]


@pytest.mark.parametrize("P,k,kind", CASES)
def test_topk_exact(P, k, kind):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(hash((P, k, kind)) & 0xFFFF)
    Q = 6
    s = _rows(rng, Q, P, kind)
    c = (rng.random((Q, P)) < 0.8).astype(np.uint8)
    c[1] = 0                          # a row without candidates
    c[2, :] = 0
    c[2, : min(P, 3)] = 1             # a row with fewer candidates than most k
    s = np.where(c == 1, s, -np.inf).astype(np.float32)
    ref = O.topk_pools(s, c, k)
    sg, cg = torch.from_numpy(s).cuda(), torch.from_numpy(c).cuda()
    out = torch.full((Q, k), 12345, dtype=torch.int32, device="cuda")
    dsa.dsa_topk_pools(sg, cg, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
