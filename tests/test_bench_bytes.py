"""The bench's algorithmic bytes (the numerator of every roofline figure it
prints), checked against totals worked out by hand from the definition:
inputs read once, outputs written once, a key or latent row that several
queries of one request use counted once."""
import numpy as np

import bench
from sparse_attention_fp32_amd import workloads as W


def test_decode32k_bytes():
    s = W.spec_by_name("decode32k")      # 16 requests, one query each
    xn = {"q_req": np.arange(16, dtype=np.int32)}
    n_pools = np.full(16, 8192, dtype=np.int32)
    tok = (np.arange(16 * 2048, dtype=np.int32).reshape(16, 2048) * 7) % 32768
    b = bench.algorithmic_bytes(s, xn, n_pools, tok)
    # head-gate: hidden [16, 4096] + W [4096, 16] + w [16, 16], f32
    assert b["head_gate"] == 4 * (16 * 4096 + 4096 * 16 + 16 * 16) == 525312
    # scores: 131072 pools x (256 B key + 4 B start + 1 B valid), qi + w per
    # query (16 heads x (256 + 4) B), score + flag per slot, three ints per query
    assert b["index_scores"] == 131072 * 261 + 16 * 16 * 260 + 16 * 8192 * 5 + 16 * 12
    # attention: 32768 distinct bf16 rows of 1 KiB, q and out (64 x 512 bf16
    # each), ids, lse, two ints per query
    assert b["sparse_mla_decode"] == (32768 * 1024 + 16 * 64 * 512 * 2 * 2 + 16 * 2048 * 4
                                      + 16 * 64 * 4 + 16 * 8) == 35786880
    # the fused calls: partials of 32 K-slices written and read back instead of w,
    # sel never read back
    part = 4 * 16 * 16 * 32
    assert b["gate_compress"] == b["head_gate"] - 4 * 16 * 16 + part + b["kpool_compress"]
    assert b["index_scores_gated"] == b["index_scores"] + part
    assert b["topk_expand"] == b["topk_pools"] + b["expand_selection"] - 16 * 512 * 4
    assert sum(b[k] for k in bench.STAGES) == 72200024


def test_shared_rows_count_once():
    s = W.spec_by_name("prefill4k")      # 4096 queries of one request
    xn = {"q_req": np.zeros(4096, dtype=np.int32)}
    n_pools = np.array([1024], dtype=np.int32)
    same = np.tile(np.arange(256, dtype=np.int32), (4096, 1))   # every query: rows 0..255
    holes = same.copy()
    holes[:, ::2] = -1                                            # half of them
    b_same = bench.algorithmic_bytes(s, xn, n_pools, same)
    b_holes = bench.algorithmic_bytes(s, xn, n_pools, holes)
    fixed = 4096 * 64 * 512 * 2 * 2 + 4096 * 256 * 4 + 4096 * 64 * 4 + 4096 * 8
    assert b_same["sparse_mla_decode"] == 256 * 1024 + fixed
    assert b_holes["sparse_mla_decode"] == 128 * 1024 + fixed
    # the request's 1024 pools are read once, not once per query
    assert b_same["index_scores"] == (1024 * 261 + 4096 * 16 * 260 + 4096 * 1024 * 5
                                      + 4096 * 12)
