"""CPU oracle for the index-selection sparse attention layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code,
tables or helpers with the HIP library and is deliberately slow and plain:
NumPy in float64, one query row at a time, no blocking or fusion.

What it computes (for one query row r of sequence b at position p):

1. Indexer relevance scores ("Large Language Model Inference Acceleration in
   Practice", section 1.2 Lightning Indexer; "Kimi New Model Open Source ...
   on Ascend", section 3: relevance scoring, head-weight weighting, Top-K).
   The pages describe the three steps in words only; the concrete form used
   throughout this library is
       score[s] = sum_j w[j] * max(0, q_idx[j, :] . k_idx[s, :])   for s <= p
   (causal: a query sees every cached position up to and including its own).
2. Top-K selection: the K largest scores among the p+1 visible positions,
   equal scores at the K-th place resolved toward the lower position; when
   p+1 <= K every visible position is kept.  The selected positions are
   returned in ascending order and padded with -1 to length K (the pages
   say only that the indexer outputs "the list of selected indices").
3. Sparse attention over the selected rows of the MLA latent cache (section
   1.2 Sparse Flash Attention; "Day0 ... for a New Model", section 3.1):
   every latent row is [latent (D_latent) | rope (D_rope)] and is shared by
   all H heads; the value is the latent part.  For head h:
       z_k = scale * q[h, :] . row_k,  p = softmax(z),
       out[h] = sum_k p_k * row_k[:D_latent],  lse[h] = log(sum_k exp(z_k)).

Storage decoding: bf16 values arrive as their 16-bit patterns, fp8 values as
OCP e4m3 codes ("... for Kimi K3.1 Pro", section 4 and "Large Language Model
Inference Acceleration in Practice", section 4 name FP8 caches; the e4m3
format itself is the OCP 8-bit floating point definition: 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN).
Scaled values are code_value * scale, evaluated in float64.

FP8 latent cache with tile scales ("Day0 Inference Adaptation and
Performance Optimization for Kimi K3.1 Pro", section 4; "Large Language Model
Inference Acceleration in Practice", section 4 and its table of formats): e4m3
codes quantised per token, per head and per tile of 128 elements.  The MLA
latent row is one vector shared by all heads, so a row of width W carries
ceil(W / 128) fp32 scales, scale j covering columns [128 j, 128 j + 128) (the
last tile of a 576-wide row holds the 64 rope columns).  The pages fix the
tile size only; one fp32 factor per tile is the reading taken here.  Values are
code_value * scale[slot, column // 128].

MXFP8 indexer ("Day0 Inference Adaptation and Performance Optimization for
Kimi K3.1 Pro", section 4 and "... for a New Model", section 4: indexer
queries and keys in MXFP8 with one shared scale per group of 32 elements):
the block format is the OCP Microscaling (MX) definition - e4m3 elements and
one E8M0 scale per 32 consecutive elements of a row, the scale byte e
standing for 2^(e - 127) (e = 255 is NaN).  Values are code_value * 2^(e-127).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


# ----------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  A bf16 value is the upper half
    of the float32 with the same sign, exponent and leading mantissa bits."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_table() -> np.ndarray:
    """Value of each of the 256 OCP e4m3 codes, from the format definition."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes).astype(np.intp)]


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> float64: byte e is 2^(e - 127); 255 is NaN."""
    e = np.asarray(codes).astype(np.int64)
    out = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, out)


def decode_mx(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """MX block values: codes [..., n] e4m3, scales [..., n / block] E8M0."""
    v = decode_e4m3(codes)
    return v * np.repeat(decode_e8m0(scales), block, axis=-1)


def _decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype in ("fp8", "mxfp8", "fp8_tile128"):
        return decode_e4m3(arr)
    raise ValueError(dtype)


KV_TILE = 128   # elements per scale tile of the tile-scaled fp8 latent cache


def decode_tile_scaled(codes: np.ndarray, scales: np.ndarray, tile: int = KV_TILE) -> np.ndarray:
    """Rows of e4m3 codes [n, W] with fp32 scales [n, ceil(W / tile)]: element
    (i, c) = code_value * scales[i, c // tile], float64."""
    codes = np.asarray(codes)
    col_tile = np.arange(codes.shape[-1]) // tile
    return decode_e4m3(codes) * np.asarray(scales, dtype=np.float64)[..., col_tile]


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """float64 -> OCP e4m3 codes: saturate to +-448, then round to the nearest
    representable value, ties to the even code (even mantissa)."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), 448.0)
    pos = _E4M3[:0x7F]                        # codes 0x00..0x7E, increasing values
    hi = np.clip(np.searchsorted(pos, mag, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = pos[hi] - mag
    d_lo = mag - pos[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def mx_quantize(x: np.ndarray, block: int = 32):
    """OCP MX conversion of rows x [..., n] (n a multiple of block) to MXFP8:
    per block, shared exponent = floor(log2(max |x|)) - 8 (8 = exponent of
    e4m3's largest normal), clamped to [-127, 127]; elements x / 2^shared
    encoded as e4m3 (saturating, round to nearest even).  A block of zeros
    gets scale 2^0 (the definition leaves it free).  Returns (codes uint8,
    scale bytes uint8)."""
    x = np.asarray(x, dtype=np.float64)
    g = x.reshape(x.shape[:-1] + (x.shape[-1] // block, block))
    amax = np.abs(g).max(axis=-1)
    _, ex = np.frexp(amax)                   # amax = m * 2^ex, m in [0.5, 1)
    shared = np.where(amax > 0, ex - 1 - 8, 0)
    shared = np.clip(shared, -127, 127)
    codes = encode_e4m3(g / np.ldexp(1.0, shared)[..., None])
    return codes.reshape(x.shape), (shared + 127).astype(np.uint8)


# ----------------------------------------------------------------------------
# cache addressing
# ----------------------------------------------------------------------------

def slots(inp: Dict, seq: int, positions: np.ndarray) -> np.ndarray:
    """Physical slot of each logical position of a sequence.  Paged caches
    map position p to block_table[seq][p // block_size] * block_size +
    p % block_size ("Kimi New Model Open Source ...", section 3: the indexer
    reads the key cache stored in pages); contiguous caches start the
    sequence at seq_base[seq]."""
    pos = np.asarray(positions, dtype=np.int64)
    if inp.get("block_table") is not None:
        bs = int(inp["block_size"])
        blk = inp["block_table"][seq][pos // bs].astype(np.int64)
        return blk * bs + pos % bs
    return int(inp["seq_base"][seq]) + pos


def indexer_keys(inp: Dict, seq: int, n: int) -> np.ndarray:
    """Keys of positions 0..n-1 of a sequence, dequantised, [n, D_I] float64."""
    sl = slots(inp, seq, np.arange(n))
    if inp["indexer_dtype"] == "mxfp8":
        return decode_mx(inp["k_data"][sl], inp["k_scale"][sl])
    k = _decode(inp["k_data"][sl], inp["indexer_dtype"])
    if inp["indexer_dtype"] == "fp8":
        k = k * inp["k_scale"][sl].astype(np.float64)[:, None]
    return k


def latent_rows(inp: Dict, seq: int, positions: np.ndarray) -> np.ndarray:
    """Latent cache rows [latent | rope] of the given positions, float64."""
    sl = slots(inp, seq, positions)
    if inp["kv_dtype"] == "fp8_tile128":
        return decode_tile_scaled(inp["kv_data"][sl], inp["kv_scale"][sl])
    rows = _decode(inp["kv_data"][sl], inp["kv_dtype"])
    if inp["kv_dtype"] == "fp8":
        g = int(inp["kv_scale_group"])
        rows = rows * inp["kv_scale"][sl // g].astype(np.float64)[:, None]
    return rows


def indexer_query(inp: Dict, r: int) -> np.ndarray:
    if inp["indexer_dtype"] == "mxfp8":
        return decode_mx(inp["q_idx"][r], inp["q_scale"][r])
    q = _decode(inp["q_idx"][r], inp["indexer_dtype"])
    if inp["indexer_dtype"] == "fp8":
        qs = np.asarray(inp["q_scale"][r], dtype=np.float64)
        q = q * (qs if qs.ndim == 0 else qs[:, None])
    return q


def mla_query(inp: Dict, r: int) -> np.ndarray:
    return decode_bf16(inp["q"][r])


# ----------------------------------------------------------------------------
# the three steps
# ----------------------------------------------------------------------------

def indexer_scores(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """score[s] = sum_j w[j] * ReLU(q_idx[j] . keys[s]); all float64.
    q_idx [H_I, D_I], w [H_I], keys [n, D_I] -> [n]."""
    dots = keys @ q_idx.T                     # [n, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def select_topk(scores: np.ndarray, K: int) -> np.ndarray:
    """Positions of the K largest scores, ties toward the lower position,
    ascending, -1 padded to K.  A stable sort of the negated scores keeps
    equal scores in position order (and treats -0.0 and +0.0 as equal)."""
    n = scores.shape[0]
    take = min(K, n)
    order = np.argsort(-scores, kind="stable")[:take]
    out = np.full(K, -1, dtype=np.int64)
    out[:take] = np.sort(order)
    return out


def sparse_mla(q: np.ndarray, rows: np.ndarray, D_v: int, scale: float,
               return_probs: bool = False):
    """Softmax attention of every head over the selected rows.
    q [H, D_qk], rows [m, D_qk] -> out [H, D_v], lse [H] (natural log).
    With no selected row the output is 0 and lse is -inf."""
    H = q.shape[0]
    m = rows.shape[0]
    if m == 0:
        out = np.zeros((H, D_v))
        lse = np.full(H, -np.inf)
        return (out, lse, np.zeros((H, 0))) if return_probs else (out, lse)
    z = scale * (q @ rows.T)                  # [H, m]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    out = p @ rows[:, :D_v]
    lse = zmax[:, 0] + np.log(l[:, 0])
    return (out, lse, p) if return_probs else (out, lse)


# ----------------------------------------------------------------------------
# one query row, end to end
# ----------------------------------------------------------------------------

def layer_row(inp: Dict, r: int, K: Optional[int] = None) -> Dict[str, np.ndarray]:
    K = int(inp["K"]) if K is None else K
    seq = int(inp["row_seq"][r])
    p = int(inp["row_pos"][r])
    n = p + 1
    keys = indexer_keys(inp, seq, n)
    sc = indexer_scores(indexer_query(inp, r), inp["w"][r].astype(np.float64), keys)
    idx = select_topk(sc, K)
    sel = idx[idx >= 0]
    rows = latent_rows(inp, seq, sel)
    out, lse = sparse_mla(mla_query(inp, r), rows, int(inp["D_latent"]),
                          float(inp["softmax_scale"]))
    return dict(scores=sc, idx=idx, out=out, lse=lse)


def attend_row(inp: Dict, r: int, idx: np.ndarray):
    """Sparse attention of row r over a given index list (-1 entries skipped)."""
    seq = int(inp["row_seq"][r])
    sel = np.asarray(idx)
    sel = sel[sel >= 0]
    rows = latent_rows(inp, seq, sel)
    return sparse_mla(mla_query(inp, r), rows, int(inp["D_latent"]),
                      float(inp["softmax_scale"]))


def scores_row(inp: Dict, r: int) -> np.ndarray:
    seq = int(inp["row_seq"][r])
    n = int(inp["row_pos"][r]) + 1
    return indexer_scores(indexer_query(inp, r), inp["w"][r].astype(np.float64),
                          indexer_keys(inp, seq, n))
