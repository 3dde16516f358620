"""Top-k on adversarial score rows, exact against the oracle: ties, all-equal
rows, negative rows, rows spanning more than 15 octaves, rows with fewer
candidates than select_k, every per-thread register tile size, and rows
longer than the register tile (up to 65,536 pools, the pools of a 262,144-row
context at kpool 4)."""
import zlib

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
          (16384, 256, "negative"), (1024, 2000, "normal"),
          # budgets above the 2048 staged in LDS take the direct-store path
          (16384, 4000, "normal"), (8192, 3000, "ties"), (4096, 2049, "wide")]
# rows longer than one register step (16384 pools), read again on each pass:
# 262,144 rows at kpool 4 give 65,536 pools
CASES += [(P, k, kind) for P in (16385, 32768, 65536) for k in (1, 512)
          for kind in ("normal", "ties", "wide")]
CASES += [(65536, 512, "equal"), (65536, 512, "negative"), (40000, 100, "zeros"),
          (65536, 2048, "normal"), (65536, 4000, "ties"), (32768, 20000, "wide")]
# rows of one pass that take two stages in 2048-pool blocks (the fused call
# keeps the candidates in its token row when they fit)
CASES += [(6000, 200, "wide"), (16384, 256, "ties"), (12289, 255, "zeros")]


def _seed(*parts):
    """A seed that is the same in every process (str hashes are salted)."""
    return zlib.crc32(repr(parts).encode())


def _case_rows(P, k, kind):
    rng = np.random.default_rng(_seed(P, k, kind))
    Q = 6
    s = _rows(rng, Q, P, kind)
    c = (rng.random((Q, P)) < 0.8).astype(np.uint8)
    c[1] = 0                          # a row without candidates
    c[2, :] = 0
    c[2, : min(P, 3)] = 1             # a row with fewer candidates than most k
    s = np.where(c == 1, s, -np.inf).astype(np.float32)
    return rng, s, c


@pytest.mark.parametrize("kpool", [3, 8])
@pytest.mark.parametrize("P,k,kind", CASES)
def test_topk_expand_exact(P, k, kind, kpool):
    """The fused top-k + expansion: sel as the oracle's top-k, tok as the
    oracle's expansion of it (one request per row, pool starts spaced by
    kpool from a random first row, a -1 tail).  With kpool 8 the token row
    holds the first stage's candidates of a long row (two-stage select)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng, s, c = _case_rows(P, k, kind)
    Q = s.shape[0]
    out_width = k * kpool + 5
    pool_off = np.arange(Q + 1, dtype=np.int32) * P
    first = rng.integers(0, 50, size=Q)
    pool_start = np.concatenate([f + kpool * np.arange(P) for f in first]).astype(np.int32)
    q_req = np.arange(Q, dtype=np.int32)
    ref_sel = O.topk_pools(s, c, k)
    ref_tok = O.expand_selection(ref_sel, pool_start, pool_off, q_req, kpool, out_width)
    sel = torch.full((Q, k), 12345, dtype=torch.int32, device="cuda")
    tok = torch.full((Q, out_width), 12345, dtype=torch.int32, device="cuda")
    dsa.dsa_topk_expand(torch.from_numpy(s).cuda(), torch.from_numpy(c).cuda(),
                        torch.from_numpy(pool_start).cuda(), torch.from_numpy(pool_off).cuda(),
                        torch.from_numpy(q_req).cuda(), kpool, sel, tok)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), ref_sel)
    assert np.array_equal(tok.cpu().numpy(), ref_tok)


def _exact_pools(P, k, kind, with_ws):
    rng = np.random.default_rng(_seed(P, k, kind))
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
    ws = None
    if with_ws:
        n = dsa.topk_pools_workspace_size(Q, P, k)
        blk = 16384 if P > 16384 else (2048 if P >= 4096 and 8 * k <= 2048 else 0)
        assert (n > 0) == (blk > 0 and -(-P // blk) * k <= 16384), n
        if n:
            ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    dsa.dsa_topk_pools(sg, cg, out, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("P,k,kind", CASES)
def test_topk_exact(P, k, kind):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _exact_pools(P, k, kind, with_ws=False)


# long rows whose first-stage candidates fit stage 2 (blocks x k <= 16384)
TWO_STAGE_CASES = [c for c in CASES if c[0] > 16384 and -(-c[0] // 16384) * c[1] <= 16384]
# rows of one register pass that keep at most an eighth of each 2048-pool block
# take two stages in 2048-pool blocks: exact cases at and past the thresholds
# (4096 pools, 8 * k == 2048), a ragged last block, and rows just outside the
# rule (one pass)
SMALL_BLOCK_CASES = [c for c in CASES if 4096 <= c[0] <= 16384 and 8 * c[1] <= 2048]
SMALL_BLOCK_CASES += [(4096, 256, "ties"), (4095, 256, "normal"), (6000, 200, "wide"),
                      (16384, 256, "equal"), (16384, 256, "ties"), (12289, 255, "zeros"),
                      (8192, 257, "normal")]
TWO_STAGE_CASES += SMALL_BLOCK_CASES


@pytest.mark.parametrize("P,k,kind", TWO_STAGE_CASES)
def test_topk_exact_two_stage(P, k, kind):
    """dsa_topk_pools with its workspace: rows longer than one pass in
    registers, and rows that keep at most an eighth of each 2048-pool block,
    take the two-stage select."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _exact_pools(P, k, kind, with_ws=True)


ROW_LEN_CASES = [(P, k, kind) for P in (30, 2047, 8192, 16384, 65536) for k in (1, 64, 512)
                 for kind in ("normal", "ties")] + [(4096, 2049, "wide"), (8192, 3000, "ties"),
                                                    (40000, 3000, "ties")]


@pytest.mark.parametrize("P,k,kind", ROW_LEN_CASES)
@pytest.mark.parametrize("fused", [False, True])
def test_topk_row_len(P, k, kind, fused):
    """Rows cut by row_len (0, negative, inside the row, the width, past it):
    only the leading entries count, in both calls."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng, s, c = _case_rows(P, k, kind)
    Q = s.shape[0]
    lens = np.array([0, P, int(rng.integers(1, P + 1)), -5, P + 100,
                     int(rng.integers(0, P + 1))], dtype=np.int32)[:Q]
    ref_sel = O.topk_pools(s, c, k, row_len=lens)
    sg, cg = torch.from_numpy(s).cuda(), torch.from_numpy(c).cuda()
    lg = torch.from_numpy(lens).cuda()
    if not fused:
        # without and with the workspace (two stages for rows past one pass)
        n = dsa.topk_pools_workspace_size(Q, P, k)
        for ws in (None, torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None):
            sel = torch.full((Q, k), 12345, dtype=torch.int32, device="cuda")
            dsa.dsa_topk_pools(sg, cg, sel, ws=ws, row_len=lg)
            torch.cuda.synchronize()
            assert np.array_equal(sel.cpu().numpy(), ref_sel)
        return
    # kpool 8: the token row holds a long row's first-stage candidates
    for kpool in (2, 8):
        out_width = k * kpool + 1
        pool_off = np.arange(Q + 1, dtype=np.int32) * P
        pool_start = np.concatenate([7 + kpool * np.arange(P)] * Q).astype(np.int32)
        q_req = np.arange(Q, dtype=np.int32)
        ref_tok = O.expand_selection(ref_sel, pool_start, pool_off, q_req, kpool, out_width)
        sel = torch.full((Q, k), 12345, dtype=torch.int32, device="cuda")
        tok = torch.full((Q, out_width), 12345, dtype=torch.int32, device="cuda")
        dsa.dsa_topk_expand(sg, cg, torch.from_numpy(pool_start).cuda(),
                            torch.from_numpy(pool_off).cuda(), torch.from_numpy(q_req).cuda(),
                            kpool, sel, tok, row_len=lg)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), ref_sel)
        assert np.array_equal(tok.cpu().numpy(), ref_tok)
