"""Device buffers for one DSA decode step and the six library calls in
pipeline order.  Allocation is torch's; every step of the computation is a
libdsa call."""
from __future__ import annotations

import torch

from . import dsa
from .workloads import Inputs


class DsaStep:
    """Owns the outputs and workspaces of one pass over one resident input set.

    ``run(incremental=True)`` is a decode step over cached pools: the pools
    that hold the newest row of each request are recompressed and every other
    stage runs in full.

    ``seq_len`` (a [B] i32 device tensor, or None) gives live lengths inside
    the requests' regions; ``post_ln=False`` compresses rows that were
    normalised when stored (no LayerNorm after pooling)."""

    def __init__(self, x: Inputs, stream=None):
        s = x.spec
        dev = x.k.device
        assert dev.type == "cuda", "DsaStep needs inputs resident on the GPU"
        self.x, self.spec, self.stream = x, s, stream
        self.seq_len = None
        self.post_ln = True
        Q, B, H, D = s.Q, s.B, s.index_heads, s.index_dim
        ncap = int(sum(s.pool_caps()))
        self.max_cap = max(s.pool_caps()) if s.B else 0
        self.pstride = s.pstride()
        i32 = dict(dtype=torch.int32, device=dev)
        self.w = torch.empty(Q, H, dtype=torch.float32, device=dev)
        self.ws_gate = torch.zeros(max(1, dsa.head_gate_workspace_size(Q, s.hidden, H)),
                                   dtype=torch.uint8, device=dev)
        self.keys = torch.empty(max(1, ncap), D, dtype=torch.int16, device=dev)
        self.pool_start = torch.empty(max(1, ncap), **i32)
        self.pool_valid = torch.empty(max(1, ncap), dtype=torch.uint8, device=dev)
        self.n_pools = torch.empty(B, **i32)
        self.scores = torch.empty(Q, self.pstride, dtype=torch.float32, device=dev)
        self.cand = torch.empty(Q, self.pstride, dtype=torch.uint8, device=dev)
        self.sel = torch.empty(Q, s.select_k, **i32)
        ntk = dsa.topk_pools_workspace_size(Q, self.pstride, s.select_k)
        self.ws_topk = torch.empty(ntk, dtype=torch.uint8, device=dev) if ntk else None
        self.tok = torch.empty(Q, s.out_width, **i32)
        self.out = torch.empty(Q, s.mla_heads, s.latent, dtype=torch.int16, device=dev)
        self.lse = torch.empty(Q, s.mla_heads, dtype=torch.float32, device=dev)
        # fused path: head-gate partials (or w itself when the split does not apply)
        self.nslices = dsa.gate_split_count(Q, s.hidden, H)
        self.gate_part = torch.empty(max(1, dsa.gate_compress_workspace_size(Q, s.hidden, H) // 4),
                                     dtype=torch.float32, device=dev)
        dt = dsa.LATENT_FP8_E4M3 if s.latent_fp8 else dsa.LATENT_BF16
        self.ws_mla = torch.empty(max(1, dsa.sparse_mla_decode_workspace_size(
            Q, s.mla_heads, s.latent, s.out_width, dt)), dtype=torch.uint8, device=dev)

    # -- stages -------------------------------------------------------------
    def head_gate(self):
        dsa.dsa_head_gate(self.x.hidden, self.x.W, self.w, self.ws_gate, stream=self.stream)

    def compress(self, incremental: bool = False):
        x = self.x
        lw, lb = (x.ln_w, x.ln_b) if self.post_ln else (None, None)
        dsa.dsa_kpool_compress(x.k, x.gate, x.ape, x.valid, x.tok_off, x.pool_off, lw, lb,
                               self.spec.eps, self.spec.kpool, self.max_cap, self.keys,
                               self.pool_start, self.pool_valid, self.n_pools,
                               new_from=x.new_from if incremental else None,
                               max_new=1 if incremental else 0, seq_len=self.seq_len,
                               stream=self.stream)

    def index_scores(self):
        x = self.x
        dsa.dsa_index_scores(x.qi, self.w, self.keys, self.pool_start, self.pool_valid, x.pool_off,
                             self.n_pools, x.q_req, x.q_pos, self.spec.kpool, self.scores,
                             self.cand, stream=self.stream)

    def topk(self):
        dsa.dsa_topk_pools(self.scores, self.cand, self.sel, ws=self.ws_topk, stream=self.stream)

    def expand(self):
        dsa.dsa_expand_selection(self.sel, self.pool_start, self.x.pool_off, self.x.q_req,
                                 self.spec.kpool, self.tok, stream=self.stream)
        self.tail()

    def tail(self):
        """always_select_tail: the query's own recent rows after the pools' tokens."""
        if self.spec.always_select_tail:
            x = self.x
            dsa.dsa_select_tail(x.valid, x.tok_off, self.pool_start, x.pool_off, self.n_pools,
                                x.q_req, x.q_pos, self.spec.kpool, self.spec.select_k, self.tok,
                                stream=self.stream)

    def mla(self):
        x = self.x
        dsa.dsa_sparse_mla_decode(x.q_mla, x.ckv, x.ckv_scale, x.kv_off, x.q_req, self.tok,
                                  self.spec.sm_scale, self.out, self.lse, self.ws_mla,
                                  stream=self.stream)

    def mla_paged(self, pc, kvidx: bool = False):
        """The MLA over a paged copy of the latent cache (a workloads.PagedCache);
        with kvidx, the physical index rows go to self.kvidx."""
        x = self.x
        if kvidx and getattr(self, "kvidx", None) is None:
            self.kvidx = torch.empty(self.spec.Q, self.spec.out_width, dtype=torch.int32,
                                     device=x.k.device)
        dsa.dsa_sparse_mla_decode_paged(x.q_mla, pc.ckv, pc.ckv_scale, pc.block_table,
                                        pc.page_rows, x.q_req, self.tok, self.spec.sm_scale,
                                        self.out, self.lse, self.ws_mla,
                                        kvidx=self.kvidx if kvidx else None, stream=self.stream)

    # -- fused decode calls (same outputs, fewer launches) ---------------------
    def gate_compress(self, incremental: bool = False):
        x = self.x
        lw, lb = (x.ln_w, x.ln_b) if self.post_ln else (None, None)
        dsa.dsa_gate_compress(x.hidden, x.W, self.gate_part, x.k, x.gate, x.ape, x.valid, x.tok_off,
                              x.pool_off, lw, lb, self.spec.eps, self.spec.kpool,
                              self.max_cap, self.keys, self.pool_start, self.pool_valid,
                              self.n_pools, new_from=x.new_from if incremental else None,
                              max_new=1 if incremental else 0, seq_len=self.seq_len,
                              stream=self.stream)

    def index_scores_gated(self):
        x = self.x
        dsa.dsa_index_scores_gated(x.qi, self.gate_part, self.nslices, self.w, self.keys,
                                   self.pool_start, self.pool_valid, x.pool_off, self.n_pools,
                                   x.q_req, x.q_pos, self.spec.kpool, self.scores, self.cand,
                                   stream=self.stream)

    def topk_expand(self):
        dsa.dsa_topk_expand(self.scores, self.cand, self.pool_start, self.x.pool_off, self.x.q_req,
                            self.spec.kpool, self.sel, self.tok, stream=self.stream)
        self.tail()

    def run_fused(self, incremental: bool = False, paged=None):
        """The decode step through the fused calls: four calls, five launches
        (the MLA over ``paged``, a workloads.PagedCache, when given)."""
        self.gate_compress(incremental)
        self.index_scores_gated()
        self.topk_expand()
        if paged is None:
            self.mla()
        else:
            self.mla_paged(paged)

    # -- the whole fused step from one host call -------------------------------
    def step_args(self, incremental: bool = False, paged=None, kvidx: bool = False):
        """The arguments of dsa_decode_step for this set: the fused calls of
        run_fused (with the tail when the shape asks for it), marshalled once;
        pass the result to run_step."""
        x, s = self.x, self.spec
        lw, lb = (x.ln_w, x.ln_b) if self.post_ln else (None, None)
        if kvidx and getattr(self, "kvidx", None) is None:
            self.kvidx = torch.empty(s.Q, s.out_width, dtype=torch.int32, device=x.k.device)
        return dsa.decode_step_args(
            x.hidden, x.W, self.gate_part, x.k, x.gate, x.ape, x.valid, x.tok_off, x.pool_off,
            lw, lb, s.eps, s.kpool, self.max_cap, self.keys, self.pool_start, self.pool_valid,
            self.n_pools, x.qi, self.w, x.q_req, x.q_pos, self.scores, self.cand, self.sel,
            self.tok, x.q_mla, x.ckv if paged is None else paged.ckv,
            x.ckv_scale if paged is None else paged.ckv_scale, s.sm_scale, self.out, self.lse,
            self.ws_mla, kv_off=x.kv_off, new_from=x.new_from if incremental else None,
            max_new=1 if incremental else 0, seq_len=self.seq_len,
            select_tail=s.always_select_tail,
            block_table=None if paged is None else paged.block_table,
            page_rows=0 if paged is None else paged.page_rows,
            kvidx=self.kvidx if kvidx else None)

    def run_step(self, args):
        """One dsa_decode_step call with arguments from step_args."""
        dsa.dsa_decode_step(args, stream=self.stream)

    # -- the cache-write side of a decode step --------------------------------
    def write_geom(self, paged=None, slot=None):
        """q_req, q_pos and new_from of the inputs (one query per request)
        from self.seq_len; with a paged cache and a slot buffer, the physical
        row of each request's newest position."""
        x = self.x
        dsa.dsa_write_geom(self.seq_len, x.q_pos, q_req=x.q_req, new_from=x.new_from, slot=slot,
                           block_table=None if paged is None else paged.block_table,
                           page_rows=0 if paged is None else paged.page_rows,
                           n_pages=0 if paged is None else paged.n_pages, stream=self.stream)

    def store(self, k_new, gate_new):
        """The step's staged indexer rows at new_from (normalised when
        post_ln is False)."""
        x = self.x
        lw, lb = (None, None) if self.post_ln else (x.ln_w, x.ln_b)
        dsa.dsa_indexer_store(k_new, gate_new, x.new_from, x.tok_off, x.k, x.gate, x.valid,
                              ln_w=lw, ln_b=lb, eps=self.spec.eps, stream=self.stream)

    def gate_compress_live(self, k_new, gate_new):
        """Geometry, row store, head-gate and incremental compression in one launch."""
        x = self.x
        dsa.dsa_gate_compress_live(x.hidden, x.W, self.gate_part, x.k, x.gate, x.ape, x.valid,
                                   x.tok_off, x.pool_off, self.seq_len, k_new, gate_new, x.ln_w,
                                   x.ln_b, not self.post_ln, self.spec.eps, self.spec.kpool,
                                   self.max_cap, self.keys, self.pool_start, self.pool_valid,
                                   self.n_pools, x.q_req, x.q_pos, x.new_from, stream=self.stream)

    def run_live(self, k_new, gate_new, paged=None, slot=None, fused: bool = False):
        """A whole decode step from the live lengths: geometry, the row store,
        then the fused step over cached pools.  fused: the first three in the
        compression launch (dsa_gate_compress_live; no slot is written)."""
        if fused:
            self.gate_compress_live(k_new, gate_new)
        else:
            self.write_geom(paged, slot)
            self.store(k_new, gate_new)
            self.gate_compress(incremental=True)
        self.index_scores_gated()
        self.topk_expand()
        if paged is None:
            self.mla()
        else:
            self.mla_paged(paged)

    def run(self, incremental: bool = False):
        self.head_gate()
        self.compress(incremental)
        self.index_scores()
        self.topk()
        self.expand()
        self.mla()
