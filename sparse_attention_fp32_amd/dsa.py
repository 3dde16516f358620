"""Thin ctypes binding over libdsa.so (see include/dsa.h).

Every function here only marshals arguments: it checks that tensors live on
the GPU with the dtype and contiguity the C ABI expects, turns them into device
pointers, and passes torch's current HIP stream.  All arithmetic runs in the
library's HIP kernels.  There is no CPU fallback: if libdsa.so is missing the
import of a call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dsa.h")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_LAUNCH = 0, 1, 2, 3
LATENT_BF16, LATENT_FP8_E4M3 = 0, 1
MAX_KPOOL, KV_LORA, MAX_INDEX_HEADS = 8, 512, 16
MLA_SCRATCH_BYTES = 32 << 20

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

_SIGS = {
    "dsa_abi_version": (_I, []),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_head_gate_workspace_size": (_Z, [_I, _I, _I]),
    "dsa_head_gate": (_I, [_P, _P, _P, _I, _I, _I, _P, _Z, _P]),
    "dsa_kpool_compress": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _I, _I, _I, _I, _P,
                                _I, _P, _P, _P, _P, _P]),
    "dsa_index_scores": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "dsa_topk_pools_workspace_size": (_Z, [_I, _I, _I]),
    "dsa_topk_pools": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _Z, _P]),
    "dsa_expand_selection": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "dsa_sparse_mla_decode_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "dsa_sparse_mla_decode": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P,
                                   _Z, _P]),
    "dsa_sparse_mla_decode_paged": (_I, [_P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _I, _I, _I, _I,
                                         _F, _P, _P, _P, _P, _Z, _P]),
    "dsa_sparse_mla_decode_noalloc": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _F, _P,
                                           _P, _P]),
    "dsa_gate_split_count": (_I, [_I, _I, _I]),
    "dsa_gate_compress_workspace_size": (_Z, [_I, _I, _I]),
    "dsa_gate_compress": (_I, [_P, _P, _I, _I, _I, _P, _Z, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _F, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "dsa_write_geom": (_I, [_P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P]),
    "dsa_lane_read": (_I, [_P, _Z, _P, _P]),
    "dsa_indexer_store": (_I, [_P, _P, _P, _P, _P, _P, _F, _I, _I, _P, _P, _P, _P]),
    "dsa_gate_compress_live": (_I, [_P, _P, _I, _I, _I, _P, _Z, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _I, _F, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                    _P]),
    "dsa_index_scores_gated": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                    _I, _P, _P, _P]),
    "dsa_topk_expand": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _I, _I, _I, _P, _P, _P]),
    "dsa_select_tail": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "dsa_decode_step_args_size": (_Z, []),
    "dsa_decode_step": (_I, [_P, _P]),
}


class DsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdsa error {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libdsa.so (built in-tree by sparse_attention_fp32_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_attention_fp32_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def header_functions() -> list:
    """Names of the functions include/dsa.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def last_error() -> str:
    return lib().dsa_last_error().decode()


def abi_version() -> int:
    return lib().dsa_abi_version()


def _check(code: int):
    if code != DSA_OK:
        raise DsaError(code, last_error())


def _stream(stream) -> _P:
    s = torch.cuda.current_stream() if stream is None else stream
    return _P(s.cuda_stream)


def _dev(t: Optional[torch.Tensor], dtype, name: str, allow_none: bool = False) -> _P:
    if t is None:
        if allow_none:
            return _P(None)
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _P(t.data_ptr())


_BF = (torch.int16, torch.uint16, torch.bfloat16)   # bf16 bits in any 16-bit container
_I32 = torch.int32
_U8 = (torch.uint8, torch.bool)


# --- workspace sizes -------------------------------------------------------

def head_gate_workspace_size(M: int, K: int, N: int) -> int:
    return lib().dsa_head_gate_workspace_size(M, K, N)


def topk_pools_workspace_size(Q: int, pstride: int, select_k: int) -> int:
    return lib().dsa_topk_pools_workspace_size(Q, pstride, select_k)


def sparse_mla_decode_workspace_size(Q: int, Hm: int, L: int, out_width: int, latent_dtype: int) -> int:
    return lib().dsa_sparse_mla_decode_workspace_size(Q, Hm, L, out_width, latent_dtype)


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return _P(None), 0
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return _P(ws.data_ptr()), ws.numel() * ws.element_size()


# --- the six calls ---------------------------------------------------------

def dsa_head_gate(hidden, W, w, ws=None, stream=None) -> None:
    M, K = hidden.shape
    N = W.shape[1]
    wp, wb = _ws(ws)
    _check(lib().dsa_head_gate(_dev(hidden, torch.float32, "hidden"), _dev(W, torch.float32, "W"),
                               _dev(w, torch.float32, "w"), M, K, N, wp, wb, _stream(stream)))


def dsa_kpool_compress(k, gate, ape, valid, tok_off, pool_off, ln_w, ln_b, eps: float, kpool: int,
                       max_cap: int, keys, pool_start, pool_valid, n_pools, new_from=None,
                       max_new: int = 0, seq_len=None, stream=None) -> None:
    """ln_w = ln_b = None: rows normalised when stored (no LayerNorm here);
    seq_len: live lengths [B] i32 (None: the whole regions)."""
    B = tok_off.numel() - 1
    D = k.shape[1]
    _check(lib().dsa_kpool_compress(
        _dev(k, _BF, "k"), _dev(gate, _BF, "gate"), _dev(ape, _BF, "ape"), _dev(valid, _U8, "valid"),
        _dev(tok_off, _I32, "tok_off"), _dev(pool_off, _I32, "pool_off"),
        _dev(seq_len, _I32, "seq_len", allow_none=True),
        _dev(ln_w, torch.float32, "ln_w", allow_none=True),
        _dev(ln_b, torch.float32, "ln_b", allow_none=True), float(eps), B, D,
        kpool, max_cap, _dev(new_from, _I32, "new_from", allow_none=True), int(max_new),
        _dev(keys, _BF, "keys"), _dev(pool_start, _I32, "pool_start"),
        _dev(pool_valid, _U8, "pool_valid"), _dev(n_pools, _I32, "n_pools"), _stream(stream)))


def dsa_index_scores(qi, w, keys, pool_start, pool_valid, pool_off, n_pools, q_req, q_pos,
                     kpool: int, scores, cand, stream=None) -> None:
    Q, H, D = qi.shape
    pstride = scores.shape[1]
    _check(lib().dsa_index_scores(
        _dev(qi, _BF, "qi"), _dev(w, torch.float32, "w"), _dev(keys, _BF, "keys"),
        _dev(pool_start, _I32, "pool_start"), _dev(pool_valid, _U8, "pool_valid"),
        _dev(pool_off, _I32, "pool_off"), _dev(n_pools, _I32, "n_pools"), _dev(q_req, _I32, "q_req"),
        _dev(q_pos, _I32, "q_pos"), Q, H, D, kpool, pstride, _dev(scores, torch.float32, "scores"),
        _dev(cand, _U8, "cand"), _stream(stream)))


def dsa_topk_pools(scores, cand, sel, ws=None, stream=None, row_len=None) -> None:
    """row_len: [Q] i32 (only the first row_len[q] entries of row q count) or None."""
    Q, pstride = scores.shape
    if row_len is not None and row_len.numel() < Q:
        raise ValueError(f"row_len holds {row_len.numel()} entries, need {Q}")
    select_k = sel.shape[1]
    wp, wb = _ws(ws)
    _check(lib().dsa_topk_pools(_dev(scores, torch.float32, "scores"), _dev(cand, _U8, "cand"),
                                _dev(row_len, _I32, "row_len", allow_none=True), Q, pstride,
                                select_k, _dev(sel, _I32, "sel"), wp, wb, _stream(stream)))


def dsa_expand_selection(sel, pool_start, pool_off, q_req, kpool: int, tok, flags: int = 0,
                         stream=None) -> None:
    Q, select_k = sel.shape
    out_width = tok.shape[1]
    _check(lib().dsa_expand_selection(
        _dev(sel, _I32, "sel"), _dev(pool_start, _I32, "pool_start"), _dev(pool_off, _I32, "pool_off"),
        _dev(q_req, _I32, "q_req"), Q, select_k, kpool, out_width, flags, _dev(tok, _I32, "tok"),
        _stream(stream)))


def dsa_sparse_mla_decode(q, ckv, ckv_scale, kv_off, q_req, tok, sm_scale: float, out, lse=None,
                          ws=None, stream=None) -> None:
    Q, Hm, L = q.shape
    out_width = tok.shape[1]
    fp8 = ckv.dtype in (torch.uint8, torch.float8_e4m3fn)
    dt = LATENT_FP8_E4M3 if fp8 else LATENT_BF16
    wp, wb = _ws(ws)
    _check(lib().dsa_sparse_mla_decode(
        _dev(q, _BF, "q"), _dev(ckv, (torch.uint8, torch.float8_e4m3fn) if fp8 else _BF, "ckv"),
        _dev(ckv_scale, torch.float32, "ckv_scale", allow_none=not fp8), dt,
        _dev(kv_off, _I32, "kv_off"), _dev(q_req, _I32, "q_req"), _dev(tok, _I32, "tok"), Q, Hm, L,
        out_width, float(sm_scale), _dev(out, _BF, "out"), _dev(lse, torch.float32, "lse", allow_none=True),
        wp, wb, _stream(stream)))


def dsa_sparse_mla_decode_noalloc(q, ckv, ckv_scale, kv_off, q_req, tok, sm_scale: float, out,
                                  lse=None, stream=None) -> None:
    """dsa_sparse_mla_decode with the library's fixed per-GPU workspace (no
    workspace argument; the call allocates nothing)."""
    Q, Hm, L = q.shape
    out_width = tok.shape[1]
    fp8 = ckv.dtype in (torch.uint8, torch.float8_e4m3fn)
    dt = LATENT_FP8_E4M3 if fp8 else LATENT_BF16
    _check(lib().dsa_sparse_mla_decode_noalloc(
        _dev(q, _BF, "q"), _dev(ckv, (torch.uint8, torch.float8_e4m3fn) if fp8 else _BF, "ckv"),
        _dev(ckv_scale, torch.float32, "ckv_scale", allow_none=not fp8), dt,
        _dev(kv_off, _I32, "kv_off"), _dev(q_req, _I32, "q_req"), _dev(tok, _I32, "tok"), Q, Hm, L,
        out_width, float(sm_scale), _dev(out, _BF, "out"), _dev(lse, torch.float32, "lse", allow_none=True),
        _stream(stream)))


def dsa_sparse_mla_decode_paged(q, ckv, ckv_scale, block_table, page_rows: int, q_req, tok,
                                sm_scale: float, out, lse=None, ws=None, kvidx=None,
                                stream=None) -> None:
    """ckv: [n_pages * page_rows, L] (bf16 bits, or fp8 codes with ckv_scale);
    block_table: [B, bt_stride] i32; kvidx: optional [Q, out_width] i32 output."""
    Q, Hm, L = q.shape
    out_width = tok.shape[1]
    fp8 = ckv.dtype in (torch.uint8, torch.float8_e4m3fn)
    dt = LATENT_FP8_E4M3 if fp8 else LATENT_BF16
    if page_rows < 1 or ckv.shape[0] % page_rows:
        raise ValueError(f"cache of {ckv.shape[0]} rows is not a whole number of {page_rows}-row pages")
    if fp8 and (ckv_scale is None or ckv_scale.numel() < ckv.shape[0]):
        raise ValueError("fp8 cache needs one scale per cache row")
    wp, wb = _ws(ws)
    _check(lib().dsa_sparse_mla_decode_paged(
        _dev(q, _BF, "q"), _dev(ckv, (torch.uint8, torch.float8_e4m3fn) if fp8 else _BF, "ckv"),
        _dev(ckv_scale, torch.float32, "ckv_scale", allow_none=not fp8), dt,
        _dev(block_table, _I32, "block_table"), block_table.shape[1], int(page_rows),
        ckv.shape[0] // page_rows, _dev(q_req, _I32, "q_req"), _dev(tok, _I32, "tok"), Q, Hm, L,
        out_width, float(sm_scale), _dev(out, _BF, "out"),
        _dev(lse, torch.float32, "lse", allow_none=True),
        _dev(kvidx, _I32, "kvidx", allow_none=True), wp, wb, _stream(stream)))


# --- fused decode calls ----------------------------------------------------

def gate_split_count(M: int, K: int, N: int) -> int:
    return lib().dsa_gate_split_count(M, K, N)


def gate_compress_workspace_size(M: int, K: int, N: int) -> int:
    return lib().dsa_gate_compress_workspace_size(M, K, N)


def dsa_gate_compress(hidden, W, gate_part, k, gate, ape, valid, tok_off, pool_off, ln_w, ln_b,
                      eps: float, kpool: int, max_cap: int, keys, pool_start, pool_valid, n_pools,
                      new_from=None, max_new: int = 0, seq_len=None, stream=None) -> None:
    M, K = hidden.shape
    N = W.shape[1]
    B = tok_off.numel() - 1
    D = k.shape[1]
    gp, gb = _ws(gate_part)
    if gate_part is not None and gate_part.dtype != torch.float32:
        raise ValueError("gate_part must be float32")
    _check(lib().dsa_gate_compress(
        _dev(hidden, torch.float32, "hidden"), _dev(W, torch.float32, "W"), M, K, N, gp, gb,
        _dev(k, _BF, "k"), _dev(gate, _BF, "gate"), _dev(ape, _BF, "ape"), _dev(valid, _U8, "valid"),
        _dev(tok_off, _I32, "tok_off"), _dev(pool_off, _I32, "pool_off"),
        _dev(seq_len, _I32, "seq_len", allow_none=True),
        _dev(ln_w, torch.float32, "ln_w", allow_none=True),
        _dev(ln_b, torch.float32, "ln_b", allow_none=True), float(eps), B, D,
        kpool, max_cap, _dev(new_from, _I32, "new_from", allow_none=True), int(max_new),
        _dev(keys, _BF, "keys"), _dev(pool_start, _I32, "pool_start"),
        _dev(pool_valid, _U8, "pool_valid"), _dev(n_pools, _I32, "n_pools"), _stream(stream)))


class DecodeStepArgs(ctypes.Structure):
    """The C struct dsa_decode_step_args (include/dsa.h), field for field;
    ctypes lays it out by the same C rules, and dsa_decode_step_args_size()
    checks that it did."""
    _fields_ = [
        ("struct_bytes", _Z),
        ("hidden", _P), ("W", _P), ("M", _I), ("K", _I), ("H", _I),
        ("gate_part", _P), ("gate_part_bytes", _Z),
        ("k", _P), ("gate", _P), ("ape", _P), ("valid", _P), ("tok_off", _P), ("pool_off", _P),
        ("seq_len", _P), ("ln_w", _P), ("ln_b", _P), ("eps", _F),
        ("B", _I), ("D", _I), ("kpool", _I), ("max_cap", _I),
        ("new_from", _P), ("max_new", _I),
        ("keys", _P), ("pool_start", _P), ("pool_valid", _P), ("n_pools", _P),
        ("qi", _P), ("w", _P), ("q_req", _P), ("q_pos", _P), ("Q", _I), ("pstride", _I),
        ("scores", _P), ("cand", _P),
        ("row_len", _P), ("select_k", _I), ("out_width", _I), ("topk_flags", _I),
        ("select_tail", _I), ("sel", _P), ("tok", _P),
        ("q_mla", _P), ("ckv", _P), ("ckv_scale", _P), ("latent_dtype", _I), ("Hm", _I),
        ("L", _I), ("sm_scale", _F), ("kv_off", _P), ("out", _P), ("lse", _P),
        ("mla_ws", _P), ("mla_ws_bytes", _Z),
        ("block_table", _P), ("bt_stride", _I), ("page_rows", _I), ("n_pages", _I),
        ("kvidx", _P),
    ]


class DecodeStep:
    """A filled dsa_decode_step_args and the tensors its pointers point into
    (held here, so they outlive every call made with it)."""

    def __init__(self, args: DecodeStepArgs, tensors: list):
        self.args = args
        self.tensors = tensors


def decode_step_args(hidden, W, gate_part, k, gate, ape, valid, tok_off, pool_off, ln_w, ln_b,
                     eps: float, kpool: int, max_cap: int, keys, pool_start, pool_valid, n_pools,
                     qi, w, q_req, q_pos, scores, cand, sel, tok, q_mla, ckv, ckv_scale,
                     sm_scale: float, out, lse, mla_ws, kv_off=None, new_from=None,
                     max_new: int = 0, seq_len=None, row_len=None, topk_flags: int = 0,
                     select_tail: bool = False, block_table=None, page_rows: int = 0,
                     kvidx=None) -> DecodeStep:
    """Marshals the arguments of one dsa_decode_step: those of
    dsa_gate_compress, dsa_index_scores_gated, dsa_topk_expand,
    dsa_select_tail (when select_tail) and dsa_sparse_mla_decode (or its paged
    form when block_table is given), checked as those wrappers check them."""
    M, K = hidden.shape
    Q, H, D = qi.shape
    if W.shape[1] != H or k.shape[1] != D:
        raise ValueError(f"head-gate width {W.shape[1]} / key width {k.shape[1]} differ from "
                         f"qi's {H} heads of {D}")
    if gate_part.dtype != torch.float32:
        raise ValueError("gate_part must be float32")
    Qm, Hm, L = q_mla.shape
    if Qm != Q or scores.shape[0] != Q:
        raise ValueError("q_mla, qi and scores must hold the same queries")
    if row_len is not None and row_len.numel() < Q:
        raise ValueError(f"row_len holds {row_len.numel()} entries, need {Q}")
    fp8 = ckv.dtype in (torch.uint8, torch.float8_e4m3fn)
    gp, gb = _ws(gate_part)
    wp, wb = _ws(mla_ws)
    a = DecodeStepArgs()
    a.struct_bytes = ctypes.sizeof(DecodeStepArgs)
    a.hidden, a.W = _dev(hidden, torch.float32, "hidden"), _dev(W, torch.float32, "W")
    a.M, a.K, a.H = M, K, H
    a.gate_part, a.gate_part_bytes = gp, gb
    a.k, a.gate, a.ape = _dev(k, _BF, "k"), _dev(gate, _BF, "gate"), _dev(ape, _BF, "ape")
    a.valid = _dev(valid, _U8, "valid")
    a.tok_off, a.pool_off = _dev(tok_off, _I32, "tok_off"), _dev(pool_off, _I32, "pool_off")
    a.seq_len = _dev(seq_len, _I32, "seq_len", allow_none=True)
    a.ln_w = _dev(ln_w, torch.float32, "ln_w", allow_none=True)
    a.ln_b = _dev(ln_b, torch.float32, "ln_b", allow_none=True)
    a.eps, a.B, a.D, a.kpool, a.max_cap = float(eps), tok_off.numel() - 1, D, kpool, max_cap
    a.new_from, a.max_new = _dev(new_from, _I32, "new_from", allow_none=True), int(max_new)
    a.keys, a.pool_start = _dev(keys, _BF, "keys"), _dev(pool_start, _I32, "pool_start")
    a.pool_valid, a.n_pools = _dev(pool_valid, _U8, "pool_valid"), _dev(n_pools, _I32, "n_pools")
    a.qi, a.w = _dev(qi, _BF, "qi"), _dev(w, torch.float32, "w", allow_none=True)
    a.q_req, a.q_pos = _dev(q_req, _I32, "q_req"), _dev(q_pos, _I32, "q_pos")
    a.Q, a.pstride = Q, scores.shape[1]
    a.scores, a.cand = _dev(scores, torch.float32, "scores"), _dev(cand, _U8, "cand")
    a.row_len = _dev(row_len, _I32, "row_len", allow_none=True)
    a.select_k, a.out_width = sel.shape[1], tok.shape[1]
    a.topk_flags, a.select_tail = int(topk_flags), int(bool(select_tail))
    a.sel, a.tok = _dev(sel, _I32, "sel"), _dev(tok, _I32, "tok")
    a.q_mla = _dev(q_mla, _BF, "q_mla")
    a.ckv = _dev(ckv, (torch.uint8, torch.float8_e4m3fn) if fp8 else _BF, "ckv")
    a.ckv_scale = _dev(ckv_scale, torch.float32, "ckv_scale", allow_none=not fp8)
    a.latent_dtype = LATENT_FP8_E4M3 if fp8 else LATENT_BF16
    a.Hm, a.L, a.sm_scale = Hm, L, float(sm_scale)
    a.out, a.lse = _dev(out, _BF, "out"), _dev(lse, torch.float32, "lse", allow_none=True)
    a.mla_ws, a.mla_ws_bytes = wp, wb
    if block_table is None:
        a.kv_off = _dev(kv_off, _I32, "kv_off")
        a.block_table = _P(None)
    else:
        if page_rows < 1 or ckv.shape[0] % page_rows:
            raise ValueError(f"cache of {ckv.shape[0]} rows is not a whole number of "
                             f"{page_rows}-row pages")
        if fp8 and (ckv_scale is None or ckv_scale.numel() < ckv.shape[0]):
            raise ValueError("fp8 cache needs one scale per cache row")
        a.kv_off = _dev(kv_off, _I32, "kv_off", allow_none=True)
        a.block_table = _dev(block_table, _I32, "block_table")
        a.bt_stride, a.page_rows = block_table.shape[1], int(page_rows)
        a.n_pages = ckv.shape[0] // page_rows
        a.kvidx = _dev(kvidx, _I32, "kvidx", allow_none=True)
    keep = [t for t in (hidden, W, gate_part, k, gate, ape, valid, tok_off, pool_off, ln_w, ln_b,
                        keys, pool_start, pool_valid, n_pools, qi, w, q_req, q_pos, scores, cand,
                        sel, tok, q_mla, ckv, ckv_scale, out, lse, mla_ws, kv_off, new_from,
                        seq_len, row_len, block_table, kvidx) if t is not None]
    return DecodeStep(a, keep)


def dsa_decode_step(step: DecodeStep, stream=None) -> None:
    """One decode step (include/dsa.h, dsa_decode_step) from arguments that
    decode_step_args marshalled."""
    _check(lib().dsa_decode_step(ctypes.byref(step.args), _stream(stream)))


# --- the cache-write side --------------------------------------------------

def dsa_write_geom(seq_len, q_pos, q_req=None, new_from=None, slot=None, block_table=None,
                   page_rows: int = 0, n_pages: int = 0, stream=None) -> None:
    B = seq_len.numel()
    bt_stride = block_table.shape[1] if block_table is not None else 0
    _check(lib().dsa_write_geom(
        _dev(seq_len, _I32, "seq_len"), B, _dev(block_table, _I32, "block_table", allow_none=True),
        bt_stride, int(page_rows), int(n_pages), _dev(q_req, _I32, "q_req", allow_none=True),
        _dev(q_pos, _I32, "q_pos"), _dev(new_from, _I32, "new_from", allow_none=True),
        _dev(slot, _I32, "slot", allow_none=True), _stream(stream)))


def dsa_indexer_store(k_new, gate_new, pos, tok_off, k, gate, valid, ln_w=None, ln_b=None,
                      eps: float = 1e-5, stream=None) -> None:
    B, D = k_new.shape
    _check(lib().dsa_indexer_store(
        _dev(k_new, _BF, "k_new"), _dev(gate_new, _BF, "gate_new"), _dev(pos, _I32, "pos"),
        _dev(tok_off, _I32, "tok_off"), _dev(ln_w, torch.float32, "ln_w", allow_none=True),
        _dev(ln_b, torch.float32, "ln_b", allow_none=True), float(eps), B, D, _dev(k, _BF, "k"),
        _dev(gate, _BF, "gate"), _dev(valid, _U8, "valid"), _stream(stream)))


def dsa_index_scores_gated(qi, gate_part, nslices: int, w, keys, pool_start, pool_valid, pool_off,
                           n_pools, q_req, q_pos, kpool: int, scores, cand, stream=None) -> None:
    Q, H, D = qi.shape
    pstride = scores.shape[1]
    _check(lib().dsa_index_scores_gated(
        _dev(qi, _BF, "qi"), _dev(gate_part, torch.float32, "gate_part"), int(nslices),
        _dev(w, torch.float32, "w", allow_none=True), _dev(keys, _BF, "keys"),
        _dev(pool_start, _I32, "pool_start"), _dev(pool_valid, _U8, "pool_valid"),
        _dev(pool_off, _I32, "pool_off"), _dev(n_pools, _I32, "n_pools"), _dev(q_req, _I32, "q_req"),
        _dev(q_pos, _I32, "q_pos"), Q, H, D, kpool, pstride, _dev(scores, torch.float32, "scores"),
        _dev(cand, _U8, "cand"), _stream(stream)))


def dsa_topk_expand(scores, cand, pool_start, pool_off, q_req, kpool: int, sel, tok, flags: int = 0,
                    stream=None, row_len=None) -> None:
    Q, pstride = scores.shape
    if row_len is not None and row_len.numel() < Q:
        raise ValueError(f"row_len holds {row_len.numel()} entries, need {Q}")
    select_k = sel.shape[1]
    out_width = tok.shape[1]
    _check(lib().dsa_topk_expand(
        _dev(scores, torch.float32, "scores"), _dev(cand, _U8, "cand"),
        _dev(row_len, _I32, "row_len", allow_none=True), Q, pstride, select_k,
        _dev(pool_start, _I32, "pool_start"), _dev(pool_off, _I32, "pool_off"),
        _dev(q_req, _I32, "q_req"), kpool, out_width, flags, _dev(sel, _I32, "sel"),
        _dev(tok, _I32, "tok"), _stream(stream)))


def dsa_select_tail(valid, tok_off, pool_start, pool_off, n_pools, q_req, q_pos, kpool: int,
                    select_k: int, tok, stream=None) -> None:
    Q, out_width = tok.shape
    _check(lib().dsa_select_tail(
        _dev(valid, _U8, "valid"), _dev(tok_off, _I32, "tok_off"), _dev(pool_start, _I32, "pool_start"),
        _dev(pool_off, _I32, "pool_off"), _dev(n_pools, _I32, "n_pools"), _dev(q_req, _I32, "q_req"),
        _dev(q_pos, _I32, "q_pos"), Q, kpool, select_k, out_width, _dev(tok, _I32, "tok"),
        _stream(stream)))


def dsa_gate_compress_live(hidden, W, gate_part, k, gate, ape, valid, tok_off, pool_off, seq_len,
                           k_new, gate_new, ln_w, ln_b, normed_rows: bool, eps: float, kpool: int,
                           max_cap: int, keys, pool_start, pool_valid, n_pools, q_req, q_pos,
                           new_from, stream=None) -> None:
    M, K = hidden.shape
    N = W.shape[1]
    B = tok_off.numel() - 1
    D = k.shape[1]
    gp, gb = _ws(gate_part)
    _check(lib().dsa_gate_compress_live(
        _dev(hidden, torch.float32, "hidden"), _dev(W, torch.float32, "W"), M, K, N, gp, gb,
        _dev(k, _BF, "k"), _dev(gate, _BF, "gate"), _dev(ape, _BF, "ape"), _dev(valid, _U8, "valid"),
        _dev(tok_off, _I32, "tok_off"), _dev(pool_off, _I32, "pool_off"),
        _dev(seq_len, _I32, "seq_len"), _dev(k_new, _BF, "k_new"), _dev(gate_new, _BF, "gate_new"),
        _dev(ln_w, torch.float32, "ln_w"), _dev(ln_b, torch.float32, "ln_b"), int(bool(normed_rows)),
        float(eps), B, D, kpool, max_cap, _dev(keys, _BF, "keys"),
        _dev(pool_start, _I32, "pool_start"), _dev(pool_valid, _U8, "pool_valid"),
        _dev(n_pools, _I32, "n_pools"), _dev(q_req, _I32, "q_req"), _dev(q_pos, _I32, "q_pos"),
        _dev(new_from, _I32, "new_from"), _stream(stream)))


def dsa_lane_read(src, sink, stream=None) -> None:
    """The HBM read lane: one coalesced read of src (a contiguous GPU tensor)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _check(lib().dsa_lane_read(_P(src.data_ptr()), src.numel() * src.element_size(),
                               _dev(sink, (torch.int32, torch.uint32), "sink"), _stream(stream)))
