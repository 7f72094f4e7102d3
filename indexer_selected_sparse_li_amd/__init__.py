"""Index-selection sparse attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of liblisfa.so (include/lisfa.h).  It only
marshals torch device tensors into pointers and sizes; every step of the
layer runs in the library's HIP kernels.  PyTorch provides device memory and
streams.  If the library has not been built, every call raises.

Entry points (same names as the C ABI):
  li_score(...)        lightning-indexer scores  [R, ld] fp32
  topk_select(...)     per-row Top-K index lists [R, K] int32
  li_topk(...)         scores and Top-K in one step (decode rows: one launch,
                       the scores stay on chip) -> index lists [R, K] int32
  sparse_mla_attn(...) sparse MLA attention      [R, H, D_latent] bf16 (+ lse)
  li_topk_sfa(...)     all three in one call on one stream
  li_topk_sfa_noalloc(...)  the same with no workspace: the library's static
                       per-GPU scratch array (for callers that cannot allocate)
One GPU's share of a context-parallel split:
  topk_candidates(...)         local Top-K of a shard as (position, score) pairs
  topk_merge(...)              the K best of the gathered candidates
  sparse_mla_attn_partial(...) fp32 partial attention over the shard's rows
  lse_combine(...)             log-sum-exp merge of the gathered partials
  zigzag_share(...), zigzag_restore(...)  Zigzag partition of prefill rows
Indexer prolog:
  indexer_q_quant(...)  dynamic fp8 / MXFP8 quantisation of indexer queries
  indexer_k_store(...)  LayerNorm of new keys and their store into the key cache
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import torch

from . import _lib as _c

__all__ = ["KVCache", "LisfaError", "li_score", "li_topk", "li_topk_plan", "topk_select", "sparse_mla_attn", "li_topk_sfa", "li_topk_sfa_noalloc",
           "topk_candidates", "topk_merge", "sparse_mla_attn_partial", "lse_combine", "zigzag_share",
           "zigzag_restore", "indexer_q_quant", "indexer_k_store", "indexer_prolog", "workspace_size", "load",
           "status_string"]


class LisfaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} (status {code})")


def load():
    return _c.load()


def status_string(code: int) -> str:
    return _c.load().lisfa_status_string(code).decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("tensors passed to the library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclasses.dataclass
class KVCache:
    """A cache of fixed-width rows (indexer keys or MLA latent rows).

    data:        [num_slots, width] bf16, or uint8 e4m3 codes
    scale:       fp8: fp32 [num_slots // scale_group], or fp32 [num_slots,
                 ceil(width / 128)] for one scale per 128-element tile (latent
                 cache); mxfp8 (uint8 scale): E8M0 bytes [num_slots, width // 32]
    block_table: paged layout: int32 [num_seqs, blocks_per_seq]
    seq_base:    contiguous layout: int64 [num_seqs] first slot of each sequence
    """
    data: torch.Tensor
    scale: Optional[torch.Tensor] = None
    scale_group: int = 1
    block_table: Optional[torch.Tensor] = None
    block_size: int = 64
    seq_base: Optional[torch.Tensor] = None

    @property
    def fp8(self) -> bool:
        return self.data.dtype == torch.uint8

    @property
    def mx(self) -> bool:
        return self.fp8 and self.scale is not None and self.scale.dtype == torch.uint8

    @property
    def tile_scaled(self) -> bool:
        """fp8 rows with one fp32 scale per 128-element tile: scale [num_slots, ceil(width / 128)]."""
        return self.fp8 and self.scale is not None and self.scale.dtype == torch.float32 and self.scale.dim() == 2

    @property
    def dtype_code(self) -> int:
        if self.mx:
            return _c.LISFA_MXFP8
        if self.tile_scaled:
            return _c.LISFA_FP8_TILE128
        return _c.LISFA_FP8_E4M3 if self.fp8 else _c.LISFA_BF16

    def c_struct(self) -> _c.Cache:
        d = self.data
        if d.dim() != 2:
            raise ValueError("cache data must be [num_slots, width]")
        nseq = (self.block_table.shape[0] if self.block_table is not None
                else self.seq_base.shape[0] if self.seq_base is not None else 0)
        if self.block_table is not None and self.block_table.dtype != torch.int32:
            raise ValueError("block_table must be int32")
        if self.seq_base is not None and self.seq_base.dtype != torch.int64:
            raise ValueError("seq_base must be int64")
        if self.fp8 and (self.scale is None or self.scale.dtype not in (torch.float32, torch.uint8)):
            raise ValueError("fp8 caches need fp32 scales (e4m3) or uint8 E8M0 scales (mxfp8)")
        if self.tile_scaled and (tuple(self.scale.shape) != (d.shape[0], (d.shape[1] + 127) // 128)
                                 or not self.scale.is_contiguous()):
            raise ValueError("tile scales must be fp32 [num_slots, ceil(width / 128)], contiguous")
        return _c.Cache(
            data=_ptr(d), num_slots=d.shape[0],
            dtype=self.dtype_code,
            row_stride_bytes=d.stride(0) * d.element_size(),
            scale=_ptr(self.scale), scale_group_tokens=self.scale_group,
            block_size=self.block_size, block_table=_ptr(self.block_table),
            bt_stride=self.block_table.shape[1] if self.block_table is not None else 0,
            num_seqs=nseq, seq_base_slot=_ptr(self.seq_base))


def _check(code: int, where: str):
    if code != _c.LISFA_OK:
        raise LisfaError(code, where)


def _indexer_args(q_idx, w, k_cache, row_seq, row_pos, max_visible, q_scale, rows_per_group):
    R, H_I, D_I = q_idx.shape
    if q_scale is not None and q_scale.dtype not in (torch.float32, torch.uint8):
        raise ValueError("q_scale must be fp32 (e4m3) or uint8 E8M0 (mxfp8)")
    per_head = q_scale is not None and q_scale.dtype == torch.float32 and q_scale.dim() == 2
    for t, dt in ((w, torch.float32), (row_seq, torch.int32), (row_pos, torch.int32)):
        if t.dtype != dt:
            raise ValueError(f"expected {dt}, got {t.dtype}")
    return _c.IndexerArgs(
        q=_ptr(q_idx), q_scale=_ptr(q_scale), q_scale_per_head=int(per_head), w=_ptr(w),
        k_cache=k_cache.c_struct(), row_seq=_ptr(row_seq), row_pos=_ptr(row_pos),
        R=R, H_I=H_I, D_I=D_I, rows_per_group=rows_per_group, max_visible=int(max_visible))


def _mla_args(q, kv_cache, row_seq, D_latent, softmax_scale):
    R, H, D_qk = q.shape
    if q.dtype != torch.bfloat16:
        raise ValueError("MLA queries must be bf16")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D_qk)   # the usual 1/sqrt(latent + rope)
    return _c.MlaArgs(q=_ptr(q), kv_cache=kv_cache.c_struct(), row_seq=_ptr(row_seq), R=R, H=H,
                      D_latent=D_latent, D_rope=D_qk - D_latent, softmax_scale=float(softmax_scale))


def workspace_size(op: int, R: int, max_visible: int, K: int, H: int, D_latent: int) -> int:
    return int(_c.load().lisfa_workspace_size(op, R, max_visible, K, H, D_latent))


# Workspaces the binding owns, one per (device, stream), grown on demand and
# reused: calls on one stream run in order, so they never overlap in it.
_WS_CACHE = {}


def _workspace(ws: Optional[torch.Tensor], need: int, device, stream=None) -> Optional[torch.Tensor]:
    """The caller's workspace (checked against `need`), or the binding's cached
    one for this device and stream.  A caller that passes no workspace gets a
    buffer that stays allocated for later calls on the same stream; pass one
    explicitly to control its lifetime."""
    if need == 0:
        return ws
    if ws is not None:
        if ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {need}")
        return ws
    dev = torch.device(device)
    st = _stream(stream)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), st)
    cur = _WS_CACHE.get(key)
    if cur is None or cur.numel() < need:
        # the caching allocator may hand a freed block to other work on its own
        # stream; record the stream that uses this one so that cannot happen early
        cur = torch.empty(need, dtype=torch.uint8, device=dev)
        if st != torch.cuda.current_stream(dev).cuda_stream:
            cur.record_stream(torch.cuda.ExternalStream(st, device=dev))
        _WS_CACHE[key] = cur
    return cur


def li_score(q_idx, w, k_cache: KVCache, row_seq, row_pos, scores, max_visible: int,
             q_scale=None, rows_per_group: int = 1, stream=None):
    """scores[r, s] for s <= row_pos[r]; scores is [R, ld] fp32 with ld >= max_visible."""
    lib = _c.load()
    a = _indexer_args(q_idx, w, k_cache, row_seq, row_pos, max_visible, q_scale, rows_per_group)
    if scores.dtype != torch.float32 or scores.dim() != 2:
        raise ValueError("scores must be [R, ld] fp32")
    _check(lib.li_score(ctypes.byref(a), _ptr(scores), scores.shape[1], _stream(stream)), "li_score")
    return scores


def li_topk(q_idx, w, k_cache: KVCache, row_seq, row_pos, K: int, idx, max_visible: int, q_scale=None,
            rows_per_group: int = 1, workspace=None, stream=None):
    """idx[r] = ascending positions of the K largest indexer scores of row r
    (those li_score would write), -1 padded; the scores are not returned."""
    lib = _c.load()
    a = _indexer_args(q_idx, w, k_cache, row_seq, row_pos, max_visible, q_scale, rows_per_group)
    R = a.R
    if idx.dtype != torch.int32 or tuple(idx.shape) != (R, K):
        raise ValueError("idx must be [R, K] int32")
    need = lib.lisfa_workspace_size(_c.LISFA_OP_LI_TOPK, R, max_visible, K, 0, 0)
    ws = _workspace(workspace, need, q_idx.device, stream)
    _check(lib.li_topk(ctypes.byref(a), K, _ptr(idx), _ptr(ws) if (ws is not None and need) else None, need,
                       _stream(stream)), "li_topk")
    return idx


def li_topk_plan(q_idx, w, k_cache: KVCache, row_seq, row_pos, K: int, max_visible: int, q_scale=None,
                 rows_per_group: int = 1, layer: bool = False) -> int:
    """Workgroups per row of the fused score + Top-K launch for these
    arguments, or 0 when the separate score and Top-K kernels run (host query,
    no GPU work); layer=True answers for the index step of li_topk_sfa."""
    a = _indexer_args(q_idx, w, k_cache, row_seq, row_pos, max_visible, q_scale, rows_per_group)
    n = int(_c.load().li_topk_plan(ctypes.byref(a), K, int(bool(layer))))
    if n < 0:
        raise LisfaError(n, "li_topk_plan")
    return n


def topk_select(scores, row_pos, K: int, idx, workspace=None, stream=None):
    """idx[r] = ascending positions of the K largest scores[r, :row_pos[r]+1], -1 padded."""
    lib = _c.load()
    if idx.dtype != torch.int32 or tuple(idx.shape) != (scores.shape[0], K):
        raise ValueError("idx must be [R, K] int32")
    R, ld = scores.shape
    need = lib.lisfa_workspace_size(_c.LISFA_OP_TOPK, R, ld, K, 0, 0)
    ws = _workspace(workspace, need, scores.device, stream)
    _check(lib.topk_select(_ptr(scores), ld, _ptr(row_pos), R, K, _ptr(idx),
                           _ptr(ws) if (ws is not None and need) else None, need, _stream(stream)),
           "topk_select")
    return idx


def topk_candidates(scores, row_pos, K: int, cand_pos, cand_score, pos_offset=None, workspace=None,
                    stream=None):
    """Local Top-K of one context shard: (logical position, score) pairs,
    positions ascending, (-1, -inf) padded; local position t of row r is
    logical position t + pos_offset[r]."""
    lib = _c.load()
    R, ld = scores.shape
    for t, dt in ((cand_pos, torch.int32), (cand_score, torch.float32)):
        if t.dtype != dt or tuple(t.shape) != (R, K):
            raise ValueError(f"candidate outputs must be [R, K] {dt}")
    need = lib.lisfa_workspace_size(_c.LISFA_OP_TOPK_CANDIDATES, R, ld, K, 0, 0)
    ws = _workspace(workspace, need, scores.device, stream)
    _check(lib.topk_candidates(_ptr(scores), ld, _ptr(row_pos), R, K, _ptr(pos_offset), _ptr(cand_pos),
                               _ptr(cand_score), _ptr(ws) if (ws is not None and need) else None, need,
                               _stream(stream)), "topk_candidates")
    return cand_pos, cand_score


def topk_merge(cand_score, cand_pos, K: int, idx, idx_score=None, ordered: bool = False, stream=None):
    """The K best of each row's gathered candidates ([R, n]); ascending positions."""
    lib = _c.load()
    R, n = cand_pos.shape
    if cand_score.shape != cand_pos.shape or cand_score.dtype != torch.float32 or cand_pos.dtype != torch.int32:
        raise ValueError("candidates must be [R, n] fp32 scores and int32 positions")
    if idx.dtype != torch.int32 or tuple(idx.shape) != (R, K):
        raise ValueError("idx must be [R, K] int32")
    _check(lib.topk_merge(_ptr(cand_score), _ptr(cand_pos), n, R, n, K, int(ordered), _ptr(idx),
                          _ptr(idx_score), _stream(stream)), "topk_merge")
    return idx


def sparse_mla_attn(q, kv_cache: KVCache, row_seq, idx, out, lse=None, softmax_scale: Optional[float] = None,
                    workspace=None, stream=None):
    """out[r, h] = softmax attention of q[r, h] over the latent rows named by idx[r]."""
    lib = _c.load()
    R, H, D_qk = q.shape
    D_latent = out.shape[2]
    K = idx.shape[1]
    a = _mla_args(q, kv_cache, row_seq, D_latent, softmax_scale)
    need = lib.lisfa_workspace_size(_c.LISFA_OP_SPARSE_MLA, R, 0, K, H, D_latent)
    ws = _workspace(workspace, need, q.device, stream)
    _check(lib.sparse_mla_attn(ctypes.byref(a), _ptr(idx), K, _ptr(out), _ptr(lse),
                               _ptr(ws) if ws is not None else None, need, _stream(stream)),
           "sparse_mla_attn")
    return out, lse


def sparse_mla_attn_partial(q, kv_cache: KVCache, row_seq, idx, out, lse, shard_range=None,
                            softmax_scale: Optional[float] = None, workspace=None, stream=None):
    """fp32 partial attention of one context shard over the rows of idx
    (logical positions) inside shard_range[r] = (lo, hi); kv_cache addresses
    the shard's rows by local position (logical - lo)."""
    lib = _c.load()
    R, H, D_qk = q.shape
    D_latent = out.shape[2]
    K = idx.shape[1]
    if out.dtype != torch.float32 or lse is None or lse.dtype != torch.float32:
        raise ValueError("partial outputs are fp32 out [R, H, D_latent] and lse [R, H]")
    a = _mla_args(q, kv_cache, row_seq, D_latent, softmax_scale)
    need = lib.lisfa_workspace_size(_c.LISFA_OP_SPARSE_MLA_PARTIAL, R, 0, K, H, D_latent)
    ws = _workspace(workspace, need, q.device, stream)
    _check(lib.sparse_mla_attn_partial(ctypes.byref(a), _ptr(idx), K, _ptr(shard_range), _ptr(out), _ptr(lse),
                                       _ptr(ws) if ws is not None else None, need, _stream(stream)),
           "sparse_mla_attn_partial")
    return out, lse


def lse_combine(part_out, part_lse, out, lse=None, stream=None):
    """Merge G partial results [G, R, H, D] (fp32, with lse [G, R, H]) into out [R, H, D] bf16."""
    lib = _c.load()
    G, R, H, D = part_out.shape
    if part_out.dtype != torch.float32 or part_lse.dtype != torch.float32 or tuple(part_lse.shape) != (G, R, H):
        raise ValueError("partials must be fp32 [G, R, H, D] and [G, R, H]")
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (R, H, D):
        raise ValueError("out must be [R, H, D] bf16")
    _check(lib.lse_combine(_ptr(part_out), _ptr(part_lse), G, R, H, D, _ptr(out), _ptr(lse), _stream(stream)),
           "lse_combine")
    return out, lse


def zigzag_share(n: int, G: int, g: int):
    """The two [start, end) row ranges GPU g of G takes under the Zigzag partition."""
    r = (ctypes.c_int64 * 4)()
    _check(_c.load().lisfa_zigzag_share(n, G, g, r), "lisfa_zigzag_share")
    return [(r[0], r[1]), (r[2], r[3])]


def zigzag_restore(src, dst, G: int, stream=None):
    """dst[t] = row t in original order, from src holding the gathered shares."""
    lib = _c.load()
    if src.shape != dst.shape or src.dtype != dst.dtype:
        raise ValueError("src and dst must have the same shape and dtype")
    n = src.shape[0]
    row_bytes = src[0].numel() * src.element_size() if n else 0
    _check(lib.zigzag_restore(_ptr(src), _ptr(dst), n, G, row_bytes, _stream(stream)), "zigzag_restore")
    return dst


def indexer_q_quant(q, fmt: str, q_out, q_scale_out, stream=None):
    """Quantise bf16 indexer queries [R, H_I, D_I]: fmt "fp8" (fp32 scale per
    row) or "mxfp8" (E8M0 scale per 32 elements); codes into q_out (uint8)."""
    lib = _c.load()
    R, H_I, D_I = q.shape
    if q.dtype != torch.bfloat16 or q_out.dtype != torch.uint8 or tuple(q_out.shape) != (R, H_I, D_I):
        raise ValueError("q must be bf16 and q_out uint8 of the same shape")
    dt = {"fp8": _c.LISFA_FP8_E4M3, "mxfp8": _c.LISFA_MXFP8}[fmt]
    want = (torch.float32, (R,)) if fmt == "fp8" else (torch.uint8, (R, H_I, D_I // 32))
    if q_scale_out.dtype != want[0] or tuple(q_scale_out.shape) != want[1]:
        raise ValueError(f"q_scale_out must be {want[0]} {want[1]}")
    _check(lib.indexer_q_quant(_ptr(q), R, H_I, D_I, dt, _ptr(q_out), _ptr(q_scale_out), _stream(stream)),
           "indexer_q_quant")
    return q_out, q_scale_out


def indexer_k_store(k, tok_seq, tok_pos, k_cache: KVCache, gamma=None, beta=None, eps: float = 1e-6,
                    normalize: bool = True, stream=None):
    """LayerNorm (optional) of new bf16 keys [T, D_I] and their store into
    k_cache at (tok_seq, tok_pos) in the cache's format."""
    lib = _c.load()
    T, D_I = k.shape
    if k.dtype != torch.bfloat16:
        raise ValueError("k must be bf16")
    for t in (gamma, beta):
        if t is not None and (t.dtype != torch.float32 or t.numel() != D_I):
            raise ValueError("gamma / beta must be fp32 [D_I]")
    c = k_cache.c_struct()
    _check(lib.indexer_k_store(_ptr(k), T, D_I, _ptr(gamma), _ptr(beta), float(eps), int(normalize), _ptr(tok_seq),
                               _ptr(tok_pos), ctypes.byref(c), _stream(stream)), "indexer_k_store")


_SIDE_STREAMS = {}


def _side_streams(device):
    """Two streams per device for the prolog, created once (default priority)."""
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _SIDE_STREAMS:
        _SIDE_STREAMS[key] = (torch.cuda.Stream(device=key), torch.cuda.Stream(device=key))
    return _SIDE_STREAMS[key]


def indexer_prolog(q, fmt: Optional[str], q_out, q_scale_out, k, tok_seq, tok_pos, k_cache: KVCache, gamma=None,
                   beta=None, eps: float = 1e-6, normalize: bool = True, mode: str = "fused", stream=None):
    """The indexer prolog of one step ahead of li_score: LayerNorm and store
    of the new keys into k_cache, and the dynamic quantisation of the queries
    (fmt "fp8" / "mxfp8"; None for bf16 queries, which need none).  The two
    parts are independent ("Day0 Inference Adaptation ... for a New Model",
    section 3.2, overlaps them on separate streams).  mode:
      "fused"   - one launch whose workgroups split between the two (default);
      "streams" - the two calls on two side streams that fork from `stream`
                  and that `stream` then waits for;
      "serial"  - the two calls in turn on `stream`.
    Every mode writes the same bytes, and everything launched next on
    `stream` sees them."""
    main = stream if stream is not None else torch.cuda.current_stream(q.device)
    if mode == "fused" and fmt is not None:
        lib = _c.load()
        R, H_I, D_I = q.shape
        T = k.shape[0]
        if q.dtype != torch.bfloat16 or q_out.dtype != torch.uint8 or tuple(q_out.shape) != (R, H_I, D_I):
            raise ValueError("q must be bf16 and q_out uint8 of the same shape")
        if k.dtype != torch.bfloat16 or tuple(k.shape) != (T, D_I):
            raise ValueError("k must be bf16 [T, D_I] with the queries' D_I")
        want = (torch.float32, (R,)) if fmt == "fp8" else (torch.uint8, (R, H_I, D_I // 32))
        if q_scale_out.dtype != want[0] or tuple(q_scale_out.shape) != want[1]:
            raise ValueError(f"q_scale_out must be {want[0]} {want[1]}")
        for t in (gamma, beta):
            if t is not None and (t.dtype != torch.float32 or t.numel() != D_I):
                raise ValueError("gamma / beta must be fp32 [D_I]")
        dt = {"fp8": _c.LISFA_FP8_E4M3, "mxfp8": _c.LISFA_MXFP8}[fmt]
        c = k_cache.c_struct()
        _check(lib.indexer_prolog(_ptr(q), R, H_I, D_I, dt, _ptr(q_out), _ptr(q_scale_out), _ptr(k), T, _ptr(gamma),
                                  _ptr(beta), float(eps), int(normalize), _ptr(tok_seq), _ptr(tok_pos),
                                  ctypes.byref(c), _stream(main)), "indexer_prolog")
        return
    if mode in ("serial", "fused"):
        indexer_k_store(k, tok_seq, tok_pos, k_cache, gamma=gamma, beta=beta, eps=eps, normalize=normalize,
                        stream=main)
        if fmt is not None:
            indexer_q_quant(q, fmt, q_out, q_scale_out, stream=main)
        return
    if mode != "streams":
        raise ValueError(f"unknown prolog mode {mode!r}")
    s_k, s_q = _side_streams(q.device)
    ready = torch.cuda.Event()
    ready.record(main)
    s_k.wait_event(ready)
    indexer_k_store(k, tok_seq, tok_pos, k_cache, gamma=gamma, beta=beta, eps=eps, normalize=normalize, stream=s_k)
    done_k = torch.cuda.Event()
    done_k.record(s_k)
    used = {s_k: [k, tok_seq, tok_pos, gamma, beta, k_cache.data, k_cache.scale, k_cache.block_table,
                  k_cache.seq_base]}
    if fmt is not None:
        s_q.wait_event(ready)
        indexer_q_quant(q, fmt, q_out, q_scale_out, stream=s_q)
        done_q = torch.cuda.Event()
        done_q.record(s_q)
        main.wait_event(done_q)
        used[s_q] = [q, q_out, q_scale_out]
    main.wait_event(done_k)
    if not torch.cuda.is_current_stream_capturing():
        # the caching allocator must not hand these blocks to other work before the side streams finish
        for st, ts in used.items():
            for t in ts:
                if t is not None:
                    t.record_stream(st)


def li_topk_sfa(q_idx, w, k_cache: KVCache, q, kv_cache: KVCache, row_seq, row_pos, K: int,
                max_visible: int, out, lse=None, idx_out=None, q_scale=None, rows_per_group: int = 1,
                softmax_scale: Optional[float] = None, workspace=None, stream=None):
    """The whole layer on one stream: scores -> Top-K -> sparse attention."""
    lib = _c.load()
    R, H, D_qk = q.shape
    D_latent = out.shape[2]
    ia = _indexer_args(q_idx, w, k_cache, row_seq, row_pos, max_visible, q_scale, rows_per_group)
    ma = _mla_args(q, kv_cache, row_seq, D_latent, softmax_scale)
    need = lib.lisfa_workspace_size(_c.LISFA_OP_FUSED, R, max_visible, K, H, D_latent)
    ws = _workspace(workspace, need, q.device, stream)
    _check(lib.li_topk_sfa(ctypes.byref(ia), ctypes.byref(ma), K, _ptr(idx_out), _ptr(out), _ptr(lse),
                           _ptr(ws), need, _stream(stream)), "li_topk_sfa")
    return out, lse


def li_topk_sfa_noalloc(q_idx, w, k_cache: KVCache, q, kv_cache: KVCache, row_seq, row_pos, K: int,
                        max_visible: int, out, lse=None, idx_out=None, q_scale=None, rows_per_group: int = 1,
                        softmax_scale: Optional[float] = None, stream=None):
    """li_topk_sfa without a workspace: the library's static scratch array of
    the GPU serves as one (nothing is allocated, so the call can be captured in
    a HIP graph or run where allocation is not allowed).  Calls that overlap in
    time on one GPU share that array and must be serialised by the caller."""
    lib = _c.load()
    ia = _indexer_args(q_idx, w, k_cache, row_seq, row_pos, max_visible, q_scale, rows_per_group)
    ma = _mla_args(q, kv_cache, row_seq, out.shape[2], softmax_scale)
    _check(lib.li_topk_sfa_noalloc(ctypes.byref(ia), ctypes.byref(ma), K, _ptr(idx_out), _ptr(out), _ptr(lse),
                                   _stream(stream)), "li_topk_sfa_noalloc")
    return out, lse
