"""Seeded synthetic inputs for the DSA decode path.

This module only draws random numbers and lays them out; it computes nothing
the method computes (no pooling, no geometry beyond buffer capacities, no
scores).  Both the CPU oracle (through the tests) and the GPU library (through
the tests and the bench) are fed from here, and from nowhere else.

Five named workloads follow the shapes of the GLM-5.3-Flash DSA layer
described on the Atlas ``glm5next_dsa`` page (section "Shape of the pipeline"
and the ``Glm5NextDsaConfig`` fields): an indexer of 16 heads x 128 dims with
kpool pooling, a 512-wide NoPE latent, 64 MLA heads.

* ``tiny``       one sequence of 128 rows, 5 padding rows, kpool 4, 4 indexer
                 heads x 32 dims, head-gate [2,256]x[256,4], 8 MLA heads.
* ``decode32k``  16 requests x 32768 cached rows, one decode query each.
* ``longctx``    4 ragged requests {131072, 98304, 65537, 40000} rows with
                 0..63 padding rows each, kpool 8, sharper gate logits.
* ``prefill4k``  one causal sequence of 4096 rows with 4096 queries.
* ``mixed64``    64 requests with log-uniform lengths in [1024, 65536], six of
                 them mostly padding, fp8-e4m3 latent with a per-row scale.
* ``decode262k`` one request of 262,144 cached rows (the context GLM-5.3 is
                 advertised at, per the page's MASKED_ATTN_MAX_KEYS note):
                 65,536 pools in one score row.

``N(0, v)`` below always names the variance ``v``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np
import torch


@dataclasses.dataclass
class Spec:
    name: str
    lengths: List[int]            # T_r: cache rows per request, padding included
    pads: List[int]               # leading rows with valid = 0 per request
    kpool: int
    index_heads: int              # H
    index_dim: int                # D
    hidden: int                   # K of the head-gate product
    select_k: int
    out_width: int
    mla_heads: int                # Hm
    latent: int = 512             # L
    q_req: Optional[List[int]] = None   # query -> request (default: one per request)
    q_pos: Optional[List[int]] = None   # query position (default: last row)
    gate_var: float = 1.0
    latent_fp8: bool = False
    sm_scale: float = 1.0
    eps: float = 1e-5
    always_select_tail: bool = False  # out_width then holds select_k*kpool + kpool-1 ids
    live: Optional[List[int]] = None  # live lengths inside the regions (None: the whole regions)
    holes: Optional[List[Tuple[int, int]]] = None  # (request, local row) with valid = 0 after
    #                                                the padding (validity holes)

    @property
    def B(self) -> int:
        return len(self.lengths)

    @property
    def Q(self) -> int:
        return len(self.query_req())

    def query_req(self) -> List[int]:
        return list(self.q_req) if self.q_req is not None else list(range(self.B))

    def query_pos(self) -> List[int]:
        if self.q_pos is not None:
            return list(self.q_pos)
        n = self.live_lengths()
        return [n[r] - 1 for r in self.query_req()]

    def live_lengths(self) -> List[int]:
        return list(self.live) if self.live is not None else list(self.lengths)

    def total_rows(self) -> int:
        return int(sum(self.lengths))

    def pool_caps(self) -> List[int]:
        """Pool slots reserved per request: enough for rows // kpool pools."""
        return [t // self.kpool for t in self.lengths]

    def pstride(self) -> int:
        return max(1, max(self.pool_caps()))


def _log_uniform_lengths(n: int, lo: int, hi: int, seed: int) -> List[int]:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 101])))
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(math.floor(math.exp(x))) for x in u]


def spec_by_name(name: str, seed: int = 0) -> Spec:
    if name == "tiny":
        return Spec(name, lengths=[128], pads=[5], kpool=4, index_heads=4, index_dim=32,
                    hidden=256, select_k=4, out_width=16, mla_heads=8,
                    q_req=[0, 0], q_pos=[127, 127])
    if name == "decode32k":
        return Spec(name, lengths=[32768] * 16, pads=[0] * 16, kpool=4, index_heads=16,
                    index_dim=128, hidden=4096, select_k=512, out_width=2048, mla_heads=64)
    if name == "longctx":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 102])))
        pads = [int(x) for x in rng.integers(0, 64, size=4)]
        return Spec(name, lengths=[131072, 98304, 65537, 40000], pads=pads, kpool=8,
                    index_heads=16, index_dim=128, hidden=4096, select_k=256,
                    out_width=2048, mla_heads=64, gate_var=2.0)
    if name == "decode262k":   # one request at the 262,144-token context the model advertises
        return Spec(name, lengths=[262144], pads=[0], kpool=4, index_heads=16, index_dim=128,
                    hidden=4096, select_k=512, out_width=2048, mla_heads=64)
    if name == "prefill4k":
        return Spec(name, lengths=[4096], pads=[0], kpool=4, index_heads=16, index_dim=128,
                    hidden=4096, select_k=64, out_width=256, mla_heads=64,
                    q_req=[0] * 4096, q_pos=list(range(4096)))
    if name == "mixed64":
        lengths = _log_uniform_lengths(64, 1024, 65536, seed)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 103])))
        short = rng.choice(64, size=6, replace=False)
        pads = [0] * 64
        for r in short:
            n_valid = int(rng.integers(1, 512))       # fewer than 512 valid rows
            pads[int(r)] = lengths[int(r)] - n_valid
        return Spec(name, lengths=lengths, pads=pads, kpool=4, index_heads=16,
                    index_dim=128, hidden=4096, select_k=128, out_width=512,
                    mla_heads=64, latent_fp8=True)
    # Parity shapes: oracle-seconds sizes that still span several tiles and
    # leave ragged tails in every kernel's grid.
    if name == "medium":
        return Spec(name, lengths=[1000, 517, 2053], pads=[3, 0, 61], kpool=4, index_heads=16,
                    index_dim=128, hidden=1024, select_k=100, out_width=404, mla_heads=64,
                    q_req=[0, 0, 1, 2, 2], q_pos=[999, 480, 516, 2052, 700])
    if name == "medium_tail":    # the medium shape with always_select_tail
        return Spec(name, lengths=[1000, 517, 2053], pads=[3, 0, 61], kpool=4, index_heads=16,
                    index_dim=128, hidden=1024, select_k=100, out_width=403, mla_heads=64,
                    q_req=[0, 0, 1, 2, 2], q_pos=[999, 480, 516, 2052, 62],
                    always_select_tail=True)
    if name == "medium_pairs":   # 32 queries x 1100 ids: seven attention chunks of 160 ids,
        # the last one short; a third of the queries sit mid-context (fewer candidates)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 106])))
        lengths = [2600, 1900, 3100]
        q_req = [0] * 11 + [1] * 10 + [2] * 11
        q_pos = []
        for r in q_req:
            n = lengths[r]
            q_pos.append(n - 1 if len(q_pos) % 3 else int(rng.integers(n // 3, n - 1)))
        return Spec(name, lengths=lengths, pads=[0, 11, 40], kpool=4, index_heads=16,
                    index_dim=128, hidden=512, select_k=275, out_width=1100, mla_heads=64,
                    q_req=q_req, q_pos=q_pos)
    if name == "medium_live":    # live lengths inside larger regions, one query per request
        # (with holes inside the live rows: a mid-request pool, and the tail of request 2)
        return Spec(name, lengths=[1000, 517, 2053], pads=[3, 0, 61], kpool=4, index_heads=16,
                    index_dim=128, hidden=1024, select_k=100, out_width=403, mla_heads=64,
                    always_select_tail=True, live=[901, 398, 1990],
                    holes=[(0, 500), (1, 200), (2, 1989)])
    if name == "medium_prefill":  # causal prefill of two sequences and a request with no
        # full pool: many queries per request (the index scores' query-block form), one
        # block of 16 queries spanning all three requests, a short last block, and a
        # query before its sequence's first valid row
        q_req = [0] * 683 + [1] * 3 + [2] * 411
        q_pos = [3] + list(range(9, 4100, 6)) + [69, 68, 67] + list(range(0, 2051, 5))
        return Spec(name, lengths=[4100, 70, 2051], pads=[9, 67, 0], kpool=4, index_heads=16,
                    index_dim=128, hidden=512, select_k=32, out_width=128, mla_heads=64,
                    q_req=q_req, q_pos=q_pos)
    if name == "medium_holes":   # validity holes after the first valid row: one just after
        # it and two mid-request (those pools are not candidates), a hole inside two
        # queries' tails, and a request whose only full pool holds a hole (no candidate)
        return Spec(name, lengths=[1000, 517, 2053, 7], pads=[3, 0, 61, 2], kpool=4,
                    index_heads=16, index_dim=128, hidden=1024, select_k=100, out_width=403,
                    mla_heads=64, q_req=[0, 0, 1, 2, 2, 3], q_pos=[999, 206, 514, 2051, 700, 6],
                    always_select_tail=True,
                    holes=[(0, 4), (0, 205), (0, 403), (1, 513), (2, 1000), (2, 2050), (3, 4)])
    if name == "medium_fp8":
        return Spec(name, lengths=[777, 1500, 96, 2500], pads=[0, 17, 95, 5], kpool=8,
                    index_heads=12, index_dim=64, hidden=768, select_k=40, out_width=330,
                    mla_heads=40, latent_fp8=True, sm_scale=1.0 / math.sqrt(512))
    raise KeyError(name)


WORKLOADS = ("tiny", "decode32k", "longctx", "prefill4k", "mixed64", "decode262k")
PARITY_SHAPES = ("tiny", "medium", "medium_fp8", "medium_tail", "medium_pairs", "medium_prefill",
                 "medium_holes")


@dataclasses.dataclass
class Inputs:
    """Every tensor one pass of the path reads.  bf16 tensors are carried as
    int16 bit patterns, fp8 as uint8 codes, so that both sides see the same
    bytes whatever the device."""
    spec: Spec
    hidden: torch.Tensor      # [M, hidden] f32 (M = Q)
    W: torch.Tensor           # [hidden, H] f32
    k: torch.Tensor           # [sumT, D] bf16 bits
    gate: torch.Tensor        # [sumT, D] bf16 bits
    ape: torch.Tensor         # [kpool, D] bf16 bits
    valid: torch.Tensor       # [sumT] u8
    tok_off: torch.Tensor     # [B+1] i32
    pool_off: torch.Tensor    # [B+1] i32
    ln_w: torch.Tensor        # [D] f32 (bf16-representable)
    ln_b: torch.Tensor        # [D] f32 (bf16-representable)
    qi: torch.Tensor          # [Q, H, D] bf16 bits
    q_req: torch.Tensor       # [Q] i32
    q_pos: torch.Tensor       # [Q] i32
    new_from: torch.Tensor    # [B] i32: first row appended by this decode step
    q_mla: torch.Tensor       # [Q, Hm, L] bf16 bits
    ckv: torch.Tensor         # [sumT, L] bf16 bits, or uint8 fp8-e4m3 codes
    ckv_scale: Optional[torch.Tensor]  # [sumT] f32 for fp8, else None
    kv_off: torch.Tensor      # [B] i32

    def to(self, device) -> "Inputs":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Inputs(**kw)

    def numpy(self) -> dict:
        out = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                out[f.name] = v.detach().cpu().numpy()
            elif f.name != "spec":
                out[f.name] = v
        return out


class _Streams:
    """One independently seeded torch generator per tensor name."""

    def __init__(self, seed: int, device: str):
        self.seed = seed
        self.device = device
        self.n = 0

    def gen(self) -> torch.Generator:
        self.n += 1
        g = torch.Generator(device=self.device)
        g.manual_seed(int(np.random.SeedSequence([self.seed, self.n]).generate_state(1)[0]))
        return g

    def normal(self, shape, std: float = 1.0, mean: float = 0.0) -> torch.Tensor:
        x = torch.randn(*shape, generator=self.gen(), device=self.device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if mean != 0.0:
            x.add_(mean)
        return x


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).view(torch.int16)


def _fp8_rows(x: torch.Tensor):
    """Store rows of x as OCP fp8-e4m3 codes with one f32 scale per row
    (scale = row amax / 448, the format's largest finite value)."""
    amax = x.abs().amax(dim=1).clamp_min(1e-30)
    scale = (amax / 448.0).to(torch.float32)
    y = (x / scale[:, None]).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def make_inputs(spec: Spec, seed: int = 0, device: str = "cpu") -> Inputs:
    s = _Streams(seed, device)
    B, Q, T = spec.B, spec.Q, spec.total_rows()
    H, D, L, Hm, K = spec.index_heads, spec.index_dim, spec.latent, spec.mla_heads, spec.hidden
    i32 = dict(dtype=torch.int32, device=device)

    hidden = s.normal((Q, K))
    W = s.normal((K, H), std=1.0 / math.sqrt(K))
    k = _bf16_bits(s.normal((T, D)))
    gate = _bf16_bits(s.normal((T, D), std=math.sqrt(spec.gate_var)))
    ape = _bf16_bits(s.normal((spec.kpool, D)))
    ln_w = s.normal((D,), std=math.sqrt(0.02), mean=1.0).to(torch.bfloat16).to(torch.float32)
    ln_b = s.normal((D,), std=math.sqrt(0.02)).to(torch.bfloat16).to(torch.float32)

    offs = np.concatenate([[0], np.cumsum(spec.lengths)]).astype(np.int32)
    caps = np.concatenate([[0], np.cumsum(spec.pool_caps())]).astype(np.int32)
    valid = torch.ones(T, dtype=torch.uint8, device=device)
    for r, p in enumerate(spec.pads):
        if p:
            valid[int(offs[r]):int(offs[r]) + p] = 0
    for r, row in spec.holes or ():
        assert 0 <= row < spec.lengths[r], (r, row)
        valid[int(offs[r]) + row] = 0

    qi = _bf16_bits(s.normal((Q, H, D)))
    q_mla = _bf16_bits(s.normal((Q, Hm, L)))
    lat = s.normal((T, L), std=1.0 / math.sqrt(L))
    if spec.latent_fp8:
        ckv, ckv_scale = _fp8_rows(lat)
    else:
        ckv, ckv_scale = _bf16_bits(lat), None
    del lat

    return Inputs(
        spec=spec, hidden=hidden, W=W, k=k, gate=gate, ape=ape, valid=valid,
        tok_off=torch.tensor(offs, **i32), pool_off=torch.tensor(caps, **i32),
        ln_w=ln_w, ln_b=ln_b, qi=qi,
        q_req=torch.tensor(spec.query_req(), **i32),
        q_pos=torch.tensor(spec.query_pos(), **i32),
        new_from=torch.tensor([max(t - 1, 0) for t in spec.live_lengths()], **i32),
        q_mla=q_mla, ckv=ckv, ckv_scale=ckv_scale,
        kv_off=torch.tensor(offs[:-1], **i32),
    )


@dataclasses.dataclass
class PagedCache:
    """The latent cache of an input set laid out in pages."""
    ckv: torch.Tensor                  # [n_pages * page_rows, L] bf16 bits or fp8 codes
    ckv_scale: Optional[torch.Tensor]  # [n_pages * page_rows] f32 for fp8, else None
    block_table: torch.Tensor          # [B, bt_stride] i32
    page_rows: int

    @property
    def n_pages(self) -> int:
        return self.ckv.shape[0] // self.page_rows


def make_paged_cache(x: Inputs, page_rows: int, seed: int = 0, spare_pages: int = 3,
                     extra_blocks: int = 1) -> PagedCache:
    """Copy the latent rows of ``x`` into pages of ``page_rows`` rows.  Page 0
    and ``spare_pages`` more hold junk rows (large values, so that reading
    one changes a result); every request's blocks take the other pages in a
    seeded random order, and the rows past its length in its last page are
    junk too.  The table has ``extra_blocks`` columns more than the longest
    request needs; entries past a request's blocks name page 0."""
    s = x.spec
    dev = x.ckv.device
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 104, page_rows])))
    nblk = [(t + page_rows - 1) // page_rows for t in s.lengths]
    n_pages = 1 + spare_pages + sum(nblk)
    order = 1 + rng.permutation(n_pages - 1)
    table = np.zeros((s.B, max(nblk) + extra_blocks), dtype=np.int32)
    k = 0
    for r in range(s.B):
        table[r, :nblk[r]] = order[k:k + nblk[r]]
        k += nblk[r]
    st = _Streams(int(rng.integers(1 << 30)), str(dev))
    junk = st.normal((n_pages * page_rows, s.latent), std=50.0)
    if s.latent_fp8:
        ckv, scale = _fp8_rows(junk)
    else:
        ckv, scale = _bf16_bits(junk), None
    del junk
    # destination row of every logical row, request by request
    dst = []
    for r in range(s.B):
        t = np.arange(s.lengths[r], dtype=np.int64)
        dst.append(table[r, t // page_rows].astype(np.int64) * page_rows + t % page_rows)
    dst_t = torch.from_numpy(np.concatenate(dst)).to(dev)
    ckv[dst_t] = x.ckv
    if scale is not None:
        scale[dst_t] = x.ckv_scale
    return PagedCache(ckv=ckv, ckv_scale=scale, block_table=torch.from_numpy(table).to(dev),
                      page_rows=page_rows)


def gate_operands(M: int, K: int, N: int, seed: int = 0):
    """hidden [M,K] and W [K,N] (f32) drawn as make_inputs draws them, for
    head-gate shapes outside the named workloads."""
    s = _Streams(seed, "cpu")
    return s.normal((M, K)), s.normal((K, N), std=1.0 / math.sqrt(K))


def random_selection(spec: Spec, seed: int = 0, holes: float = 0.1) -> torch.Tensor:
    """A selection row per query for running the attention stage on its own:
    distinct request-local ids drawn uniformly from the query's request, in
    random order, with about ``holes`` of the slots left at -1.  [Q, out_width]
    i32 on the CPU."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 105])))
    q_req = spec.query_req()
    tok = np.full((spec.Q, spec.out_width), -1, dtype=np.int32)
    for q, r in enumerate(q_req):
        n = min(spec.out_width, spec.lengths[r])
        ids = rng.choice(spec.lengths[r], size=n, replace=False)
        keep = rng.random(n) >= holes
        slots = rng.permutation(spec.out_width)[:n]
        tok[q, slots[keep]] = ids[keep]
    return torch.from_numpy(tok)
