"""The C ABI on the CPU: libdsa.so loads, exports every function include/dsa.h
declares, and refuses bad host arguments with the documented code before it
touches the GPU (no valid launch is attempted here)."""
import ctypes
import os

import pytest

from sparse_attention_fp32_amd import dsa

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="libdsa.so not built")

INV, UNS = dsa.DSA_ERR_INVALID_ARG, dsa.DSA_ERR_UNSUPPORTED
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails validation first
NUL = ctypes.c_void_p(None)
MIS = ctypes.c_void_p(0x1004)    # a pointer that is not 16-byte aligned


def _misaligned(code):
    return code == INV and "16-byte aligned" in dsa.last_error()


def test_exports_every_declared_function():
    names = dsa.header_functions()
    assert len(names) == 25
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
        getattr(dsa.lib(), n)
    assert dsa.abi_version() == 4


def _code(fn, *args):
    return fn(*args)


def test_head_gate_errors():
    L = dsa.lib()
    assert L.dsa_head_gate(FAKE, FAKE, FAKE, 4, 4096, 0, NUL, 0, NUL) == INV
    assert L.dsa_head_gate(FAKE, FAKE, FAKE, 4, 4096, 17, NUL, 0, NUL) == INV
    assert "N=17" in dsa.last_error()
    assert L.dsa_head_gate(FAKE, FAKE, FAKE, 4, 0, 16, NUL, 0, NUL) == INV
    assert L.dsa_head_gate(FAKE, FAKE, FAKE, -1, 16, 16, NUL, 0, NUL) == INV
    assert L.dsa_head_gate(NUL, FAKE, FAKE, 4, 4096, 16, FAKE, 1 << 20, NUL) == INV
    assert _misaligned(L.dsa_head_gate(FAKE, MIS, FAKE, 40, 4096, 16, NUL, 0, NUL))
    # no workspace is needed on either path
    assert dsa.head_gate_workspace_size(16, 4096, 16) == 0
    assert dsa.head_gate_workspace_size(4096, 4096, 16) == 0
    assert L.dsa_head_gate(FAKE, FAKE, FAKE, 0, 4096, 16, NUL, 0, NUL) == dsa.DSA_OK  # no-op


def _compress(kpool=4, D=128, B=2, max_cap=10, new_from=NUL, max_new=0, k=FAKE, ln_w=FAKE,
              ln_b=FAKE):
    return dsa.lib().dsa_kpool_compress(k, FAKE, FAKE, FAKE, FAKE, FAKE, NUL, ln_w, ln_b, 1e-5, B,
                                        D, kpool, max_cap, new_from, max_new, FAKE, FAKE, FAKE,
                                        FAKE, NUL)


def test_kpool_compress_errors():
    # the page's validate(): kpool 0 and kpool above the 8-slot bound are refused
    assert _compress(kpool=0) == INV
    assert _compress(kpool=9) == INV
    assert "never truncated" in dsa.last_error()
    assert _compress(D=96) == UNS
    assert _compress(D=512) == UNS
    assert _compress(B=-1) == INV
    assert _compress(max_cap=-1) == INV
    assert _compress(new_from=FAKE, max_new=0) == INV
    assert _compress(k=NUL) == INV
    assert _misaligned(_compress(k=MIS))
    assert _compress(B=70000, max_cap=4) == UNS      # beyond the launch grid
    assert _compress(ln_w=NUL) == INV             # both LayerNorm vectors, or neither
    assert "both" in dsa.last_error()
    assert _compress(B=0) == dsa.DSA_OK


def test_index_scores_errors():
    L = dsa.lib()
    def call(H=16, D=128, kpool=4, pstride=100, Q=3, qi=FAKE):
        return L.dsa_index_scores(qi, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, Q, H, D,
                                  kpool, pstride, FAKE, FAKE, NUL)
    assert call(H=0) == INV
    assert call(H=17) == INV
    assert call(D=100) == UNS
    assert call(kpool=9) == INV
    assert call(pstride=0) == INV
    assert call(Q=-2) == INV
    assert call(qi=NUL) == INV
    assert _misaligned(call(qi=MIS))
    assert call(Q=0) == dsa.DSA_OK


def test_topk_errors():
    L = dsa.lib()
    assert L.dsa_topk_pools(FAKE, FAKE, NUL, 4, 100, 0, FAKE, NUL, 0, NUL) == INV
    assert L.dsa_topk_pools(FAKE, FAKE, NUL, 4, 0, 8, FAKE, NUL, 0, NUL) == INV
    # no row-length cap: a long row passes validation (NULL sel then fails it)
    assert L.dsa_topk_pools(FAKE, FAKE, NUL, 4, 1 << 20, 8, NUL, NUL, 0, NUL) == INV
    assert "NULL" in dsa.last_error()
    assert L.dsa_topk_pools(NUL, FAKE, NUL, 4, 100, 8, FAKE, NUL, 0, NUL) == INV
    assert _misaligned(L.dsa_topk_pools(FAKE, MIS, NUL, 4, 100, 8, FAKE, NUL, 0, NUL))
    assert _misaligned(L.dsa_topk_pools(FAKE, FAKE, MIS, 4, 100, 8, FAKE, NUL, 0, NUL))
    assert dsa.topk_pools_workspace_size(16, 8192, 512) == 0
    # rows past one pass in registers: room for each row's first-stage candidates
    assert dsa.topk_pools_workspace_size(2, 65536, 512) == 2 * 4 * 512 * 4
    assert dsa.topk_pools_workspace_size(2, 65536, 8192) == 0   # candidates past stage 2's reach
    # rows of one pass that keep at most an eighth of each 2048-pool block:
    # two stages in 2048-pool blocks (ceil(P / 2048) blocks of k candidates)
    assert dsa.topk_pools_workspace_size(4, 16384, 256) == 4 * 8 * 256 * 4
    assert dsa.topk_pools_workspace_size(4, 4096, 256) == 4 * 2 * 256 * 4
    assert dsa.topk_pools_workspace_size(3, 6000, 200) == 3 * 3 * 200 * 4
    assert dsa.topk_pools_workspace_size(4, 4095, 256) == 0     # below 4096 pools
    assert dsa.topk_pools_workspace_size(4, 8192, 257) == 0     # a block keeps more than 1/8


def test_expand_errors():
    L = dsa.lib()
    def call(select_k=4, kpool=4, out_width=16, flags=0, sel=FAKE):
        return L.dsa_expand_selection(sel, FAKE, FAKE, FAKE, 2, select_k, kpool, out_width, flags, FAKE, NUL)
    # out_width must hold select_k * kpool ids (the page's topk % kpool rule)
    assert call(out_width=15) == INV
    assert call(kpool=0) == INV
    assert call(kpool=9) == INV
    assert call(select_k=0) == INV
    assert call(flags=1) == UNS          # always_select_tail: not built
    assert call(flags=2) == INV
    assert call(sel=NUL) == INV
    assert _misaligned(call(sel=MIS))
    assert L.dsa_expand_selection(FAKE, FAKE, FAKE, FAKE, 70000, 4, 4, 16, 0, FAKE, NUL) == UNS


def test_sparse_mla_errors():
    L = dsa.lib()
    def call(L_=512, Hm=64, out_width=2048, dt=0, scale=NUL, Q=16, ws=NUL, wsb=0, q=FAKE):
        return L.dsa_sparse_mla_decode(q, FAKE, scale, dt, FAKE, FAKE, FAKE, Q, Hm, L_, out_width,
                                       1.0, FAKE, NUL, ws, wsb, NUL)
    # the page's validate(): the latent must be exactly 512 wide; zero heads refused
    assert call(L_=576) == UNS
    assert "512" in dsa.last_error()
    assert call(Hm=0) == INV
    assert call(out_width=0) == INV
    assert call(dt=7) == INV
    assert call(dt=1, scale=NUL) == INV           # fp8 without row scales
    need = dsa.sparse_mla_decode_workspace_size(16, 64, 512, 2048, 0)
    assert need > 0
    assert call(ws=FAKE, wsb=need - 1) == INV
    assert call(q=NUL, ws=FAKE, wsb=need) == INV
    assert _misaligned(call(q=MIS, ws=FAKE, wsb=need))
    assert _misaligned(call(ws=MIS, wsb=need))
    assert call(Q=0) == dsa.DSA_OK


def test_fused_call_errors():
    L = dsa.lib()
    # split rule: K/128 partials for 1 <= M <= 64 and K a multiple of 128 (<= 64 slices)
    assert dsa.gate_split_count(16, 4096, 16) == 32
    assert dsa.gate_split_count(2, 256, 4) == 2
    assert dsa.gate_split_count(4096, 4096, 16) == 1      # dense head-gate writes w
    assert dsa.gate_split_count(16, 4000, 16) == 1
    assert dsa.gate_split_count(16, 128 * 65, 16) == 1
    assert dsa.gate_split_count(16, 4096, 17) == 0
    assert dsa.gate_compress_workspace_size(16, 4096, 16) == 32 * 16 * 16 * 4
    assert dsa.gate_compress_workspace_size(4096, 4096, 16) == 4096 * 16 * 4

    def gc(M=16, K=4096, N=16, part_bytes=32 * 16 * 16 * 4, kpool=4, B=2, hidden=FAKE):
        return L.dsa_gate_compress(hidden, FAKE, M, K, N, FAKE, part_bytes, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, NUL, FAKE, FAKE, 1e-5, B, 128, kpool, 10, NUL, 0,
                                   FAKE, FAKE, FAKE, FAKE, NUL)
    assert gc(N=17) == INV
    assert gc(part_bytes=32 * 16 * 16 * 4 - 1) == INV
    assert "need" in dsa.last_error()
    assert gc(kpool=9) == INV
    assert gc(hidden=NUL) == INV
    assert _misaligned(gc(hidden=MIS))
    assert gc(M=0, B=0) == dsa.DSA_OK

    def sg(nslices=32, H=16, Q=3):
        return L.dsa_index_scores_gated(FAKE, FAKE, nslices, NUL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, Q, H, 128, 4, 100, FAKE, FAKE, NUL)
    assert sg(nslices=0) == INV
    assert sg(nslices=65) == INV
    assert sg(H=17) == INV
    assert _misaligned(L.dsa_index_scores_gated(FAKE, MIS, 32, NUL, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, FAKE, 3, 16, 128, 4, 100, FAKE, FAKE, NUL))
    assert sg(Q=0) == dsa.DSA_OK

    def te(select_k=4, kpool=4, out_width=16, flags=0, tok=FAKE):
        return L.dsa_topk_expand(FAKE, FAKE, NUL, 2, 100, select_k, FAKE, FAKE, FAKE, kpool,
                                 out_width, flags, FAKE, tok, NUL)
    assert te(out_width=15) == INV
    assert te(select_k=0) == INV
    assert te(kpool=9) == INV
    assert te(flags=1) == UNS          # bit 0 reserved: dsa_select_tail writes the tail
    assert te(tok=NUL) == INV
    assert _misaligned(te(tok=MIS))


def test_select_tail_errors():
    L = dsa.lib()
    def call(kpool=4, select_k=2, out_width=11, Q=3, tok=FAKE):
        return L.dsa_select_tail(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, Q, kpool, select_k,
                                 out_width, tok, NUL)
    assert call(out_width=10) == INV          # select_k*kpool + kpool-1 slots needed
    assert "kpool-1" in dsa.last_error()
    assert call(kpool=0) == INV
    assert call(kpool=9) == INV
    assert call(select_k=0) == INV
    assert call(Q=-1) == INV
    assert call(tok=NUL) == INV
    assert _misaligned(call(tok=MIS))
    assert call(Q=0) == dsa.DSA_OK
    assert call(kpool=1, out_width=2) == dsa.DSA_OK   # kpool 1 has no tail slots


def test_sparse_mla_paged_errors():
    L = dsa.lib()
    need = dsa.sparse_mla_decode_workspace_size(16, 64, 512, 2048, 0)
    def call(L_=512, bt_stride=512, page_rows=64, n_pages=9000, Q=16, bt=FAKE, ws=FAKE, wsb=need):
        return L.dsa_sparse_mla_decode_paged(FAKE, FAKE, NUL, 0, bt, bt_stride, page_rows, n_pages,
                                             FAKE, FAKE, Q, 64, L_, 2048, 1.0, FAKE, NUL, NUL, ws,
                                             wsb, NUL)
    assert call(L_=576) == UNS
    assert call(bt_stride=0) == INV
    assert call(page_rows=0) == INV
    assert "page_rows=0" in dsa.last_error()
    assert call(n_pages=0) == INV
    assert call(n_pages=1 << 20, page_rows=4096) == UNS     # 2^32 rows
    assert call(bt=NUL) == INV
    assert _misaligned(call(bt=MIS))
    assert call(wsb=need - 1) == INV
    assert call(Q=0) == dsa.DSA_OK


def test_cache_write_errors():
    L = dsa.lib()
    def geom(B=3, slot=NUL, bt=NUL, bt_stride=0, page_rows=0, n_pages=0, seq_len=FAKE):
        return L.dsa_write_geom(seq_len, B, bt, bt_stride, page_rows, n_pages, NUL, FAKE, NUL, slot,
                                NUL)
    assert geom(B=-1) == INV
    assert geom(slot=FAKE) == INV                   # a slot needs the block table
    assert "block table" in dsa.last_error()
    assert geom(slot=FAKE, bt=FAKE, bt_stride=4, page_rows=0, n_pages=3) == INV
    assert geom(seq_len=NUL) == INV
    assert _misaligned(geom(seq_len=MIS))
    assert geom(B=0) == dsa.DSA_OK

    def store(B=2, D=128, ln_w=NUL, ln_b=NUL, pos=FAKE, eps=1e-5):
        return L.dsa_indexer_store(FAKE, FAKE, pos, FAKE, ln_w, ln_b, eps, B, D, FAKE, FAKE, FAKE,
                                   NUL)
    assert store(D=96) == UNS
    assert store(ln_w=FAKE) == INV
    assert store(eps=-1.0) == INV
    assert store(pos=NUL) == INV
    assert _misaligned(store(pos=MIS))
    assert store(B=-1) == INV
    assert store(B=0) == dsa.DSA_OK

    def live(ln_w=FAKE, ln_b=FAKE, kpool=4, seq_len=FAKE, N=16, part_bytes=32 * 16 * 16 * 4):
        return L.dsa_gate_compress_live(FAKE, FAKE, 16, 4096, N, FAKE, part_bytes, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, seq_len, FAKE, FAKE, ln_w, ln_b, 0, 1e-5,
                                        2, 128, kpool, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        NUL)
    assert live(ln_w=NUL, ln_b=NUL) == INV          # the LayerNorm is required here
    assert live(ln_w=NUL) == INV
    assert live(kpool=9) == INV
    assert live(seq_len=NUL) == INV
    assert _misaligned(live(seq_len=MIS))
    assert live(N=17) == INV
    assert live(part_bytes=4) == INV


def test_lane_read_errors():
    L = dsa.lib()
    assert L.dsa_lane_read(FAKE, 17, FAKE, NUL) == INV
    assert L.dsa_lane_read(NUL, 16, FAKE, NUL) == INV
    assert _misaligned(L.dsa_lane_read(MIS, 16, FAKE, NUL))
    assert L.dsa_lane_read(NUL, 0, NUL, NUL) == dsa.DSA_OK


def test_mla_noalloc_errors():
    """The allocation-free attention call refuses before it looks for its
    array or launches: partials beyond the fixed array, and the workspace
    call's own argument errors."""
    L = dsa.lib()
    f = L.dsa_sparse_mla_decode_noalloc
    assert f(FAKE, FAKE, NUL, 0, FAKE, FAKE, FAKE, 256, 64, 512, 4096, 1.0, FAKE, NUL, NUL) == UNS
    assert "fixed" in dsa.last_error()
    assert dsa.sparse_mla_decode_workspace_size(256, 64, 512, 4096, 0) > dsa.MLA_SCRATCH_BYTES
    assert f(FAKE, FAKE, NUL, 0, FAKE, FAKE, FAKE, 4, 64, 576, 2048, 1.0, FAKE, NUL, NUL) == UNS
    assert f(FAKE, FAKE, NUL, 0, FAKE, FAKE, FAKE, 4, 0, 512, 2048, 1.0, FAKE, NUL, NUL) == INV
    assert f(FAKE, FAKE, NUL, 1, FAKE, FAKE, FAKE, 4, 64, 512, 2048, 1.0, FAKE, NUL, NUL) == INV
    assert f(FAKE, FAKE, NUL, 0, FAKE, FAKE, FAKE, 0, 64, 512, 2048, 1.0, FAKE, NUL, NUL) == dsa.DSA_OK


def _step_args(**kw):
    """A dsa_decode_step_args for the 32K decode shape (16 queries, 8192 pools
    per row, 64 attention heads) with fake device pointers; fields in kw
    override."""
    a = dsa.DecodeStepArgs()
    a.struct_bytes = dsa.lib().dsa_decode_step_args_size()
    Q, K, H, D, kpool = 16, 4096, 16, 128, 4
    ns = dsa.gate_split_count(Q, K, H)
    for name, kind in dsa.DecodeStepArgs._fields_:
        if kind is ctypes.c_void_p:
            setattr(a, name, FAKE)
    a.M, a.K, a.H = Q, K, H
    a.gate_part_bytes = dsa.gate_compress_workspace_size(Q, K, H)
    a.seq_len = a.row_len = a.kvidx = a.block_table = NUL
    a.eps, a.B, a.D, a.kpool, a.max_cap, a.max_new = 1e-5, 16, D, kpool, 8192, 1
    a.Q, a.pstride, a.select_k, a.out_width = Q, 8192, 512, 2048
    a.ckv_scale = NUL
    a.latent_dtype, a.Hm, a.L, a.sm_scale = dsa.LATENT_BF16, 64, 512, 0.04
    a.mla_ws_bytes = dsa.sparse_mla_decode_workspace_size(Q, 64, 512, 2048, 0)
    assert ns > 1 and a.gate_part_bytes > 0 and a.mla_ws_bytes > 0
    for k_, v in kw.items():
        setattr(a, k_, v)
    return a


def _step(a):
    return dsa.lib().dsa_decode_step(ctypes.byref(a) if a is not None else NUL, NUL)


def test_decode_step_errors():
    """The step executor checks the arguments of every call it makes before it
    launches any: a bad argument of its last call (the attention) is reported
    as that call's error, not as a failed launch of its first call (the
    arguments of the first calls here are valid, and this host has no GPU)."""
    assert ctypes.sizeof(dsa.DecodeStepArgs) == dsa.lib().dsa_decode_step_args_size()
    assert _step(None) == INV
    assert _step(_step_args(struct_bytes=8)) == INV
    assert "struct_bytes" in dsa.last_error()
    assert _step(_step_args(M=8)) == INV                       # the gate's rows are the queries
    assert _step(_step_args(kpool=9)) == INV                   # the compression's validate()
    assert "kpool=9" in dsa.last_error()
    assert _step(_step_args(gate_part_bytes=4)) == INV
    assert _step(_step_args(qi=MIS)) == INV                    # the gated scores
    assert "dsa_index_scores_gated" in dsa.last_error()
    assert _step(_step_args(select_k=0)) == INV                # top-k + expansion
    assert "dsa_topk_expand" in dsa.last_error()
    assert _step(_step_args(select_tail=1, out_width=2048)) == INV   # no room for the tail slots
    assert "dsa_select_tail" in dsa.last_error()
    assert _step(_step_args(L=576)) == UNS                     # the attention, last
    assert "dsa_sparse_mla_decode" in dsa.last_error()
    assert _step(_step_args(mla_ws_bytes=16)) == INV
    assert _step(_step_args(latent_dtype=dsa.LATENT_FP8_E4M3)) == INV   # fp8 without row scales
    # the paged attention when a block table is given
    assert _step(_step_args(block_table=FAKE, bt_stride=0, page_rows=64, n_pages=8)) == INV
    assert "dsa_sparse_mla_decode_paged" in dsa.last_error()
