"""Plain, slow CPU oracle for the W4A16 MoE expert layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

Sources. "Chord page" is the article on the vLLM x Novita AI release of Chord,
an INT4 W4A16 MoE operator for Kimi K2.x (aihot.vn). "DFlash audit" is the
Kimi-K3 PP + DFlash migration audit. Each function names the passage it
follows. Where the pages leave a step open, the reading taken is stated next
to the code.

Arithmetic. Floating point is float64 throughout, which is exact or nearly
exact for every step: a dequantised weight is an exact product rounded once to
BF16, dot products of BF16 values are accumulated in float64, and the only
other rounding is the BF16 intermediate ``a`` (the second GEMM's BF16 input).
The reference output stays unrounded (float64).

Parity status: every function here is pinned by tests/test_oracle_pins.py
(library special cases, closed forms, brute force, invariants, hand-worked
fixtures under tests/golden/, including the comparison metrics and the
permutation). The full-size layer outputs are trusted through those pins; the
pages print no worked numerical example of the layer.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")      # largest finite BF16
SENTINEL_NAN_BITS = 0x7FC0


# --------------------------------------------------------------------------
# BF16 storage
# --------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round to nearest BF16, ties to even; returns uint16 bit patterns.

    Works on float64 input directly (no intermediate float32 rounding). For a
    finite |x| with leading-bit exponent p, the BF16 spacing is
    2**(max(p, -126) - 7); |x| divided by that spacing is rounded with rint
    (ties to even) and scaled back, which is exact in float64. Results above
    the largest finite BF16 become infinity; NaN becomes the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    ax = np.abs(x)
    finite = np.isfinite(x)
    with np.errstate(all="ignore"):
        _, e = np.frexp(ax)                       # ax = m * 2**e, 0.5 <= m < 1
        spacing = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
        r = np.rint(ax / spacing) * spacing
    r = np.where(finite, r, ax)
    r = np.where(r > BF16_MAX, np.inf, r)
    r = np.copysign(r, x)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[...] = bits
    out[np.isnan(x)] = SENTINEL_NAN_BITS
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) to float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Weights: uint4 packed eight per int32, BF16 scale per 32 along K
# --------------------------------------------------------------------------

def unpack_nibbles(words) -> np.ndarray:
    """Unpack int32 words [..., K/8] to uint4 values q [..., K].

    Reading: eight nibbles per word, low nibble first, packed along K (the
    reduction axis); nibble i of a word is bits [4i, 4i+4) and holds
    k = 8*word_index + i. The shift is logical (the word is read unsigned).
    Chord page, "TL;DR" / "vLLM integration" (uint4, group-32 schema).
    """
    u = np.asarray(words).view(np.uint32) if np.asarray(words).dtype == np.int32 \
        else np.asarray(words).astype(np.uint32)
    shifts = np.arange(8, dtype=np.uint32) * 4
    q = (u[..., :, None] >> shifts) & np.uint32(0xF)
    return q.reshape(*u.shape[:-1], u.shape[-1] * 8).astype(np.uint8)


def dequant(words, scale_bits) -> np.ndarray:
    """Dequantise to BF16: W[n, k] = bf16(f(q[n,k] - 8) * f(s[n, k // 32])).

    Subtract-then-scale with zero point 8; the product of a small integer and a
    BF16 scale is exact in float64 and rounded once (the unfused BF16 rounding
    order that the Chord page's decode kernel keeps; "H200 and Blackwell
    indexed decode"). Returns uint16 BF16 bit patterns [..., N, K].
    """
    words = np.asarray(words)
    scale_bits = np.asarray(scale_bits)
    assert words.shape[:-1] == scale_bits.shape[:-1] and words.shape[-1] == 4 * scale_bits.shape[-1]
    if words.ndim > 2 or words.shape[0] <= 64:
        q = unpack_nibbles(words).astype(np.float64) - 8.0
        s_full = np.repeat(bf16_to_f64(scale_bits), 32, axis=-1)
        return bf16_round(q * s_full)
    # rows are independent: work on 64 at a time to keep temporaries small
    out = np.empty((words.shape[0], words.shape[1] * 8), dtype=np.uint16)
    for r in range(0, words.shape[0], 64):
        out[r:r + 64] = dequant(words[r:r + 64], scale_bits[r:r + 64])
    return out


# --------------------------------------------------------------------------
# Token -> expert alignment (indexed layout)
# --------------------------------------------------------------------------

def align(topk_ids, E: int, block: int) -> dict:
    """Sort routed rows by expert, padding each expert to a multiple of block.

    The indexed layout keeps activations unpadded and puts the padding in the
    routing indices as sentinels (Chord page, "Grouped SM90 kernels", Fig. 3).
    Readings taken:
      * a routed row is the flat index f = t*topk + j of topk_ids[t, j];
        ids outside [0, E) route nowhere and are dropped;
      * c_e = number of rows routed to expert e; p_e = ceil(c_e/block)*block
        (an expert with no rows gets no block);
      * offsets = exclusive prefix sum of p (length E+1), total = offsets[E];
      * sorted_ids[offsets[e] + r] = the r-th row of expert e in ascending
        flat order (a stable sort), r < c_e; every other slot up to
        cap = T*topk + E*(block-1) holds the sentinel T*topk;
      * block_expert[b] = e for b*block in [offsets[e], offsets[e+1]), else -1;
        its length is ceil(cap / block).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    n = T * k
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    padded = -(-counts // block) * block
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    cap = n + E * (block - 1)
    sorted_ids = np.full(cap, n, dtype=np.int64)
    for e in range(E):
        rows = np.flatnonzero(flat == e)            # ascending flat order
        sorted_ids[offsets[e]:offsets[e] + rows.size] = rows
    nblocks = -(-cap // block)
    block_expert = np.full(nblocks, -1, dtype=np.int64)
    for e in range(E):
        block_expert[offsets[e] // block:offsets[e + 1] // block] = e
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                sorted_ids=sorted_ids.astype(np.int32), block_expert=block_expert.astype(np.int32),
                total=int(offsets[E]), cap=int(cap), block=int(block), sentinel=int(n))


def ep_local_ids(topk_ids, expert_map) -> np.ndarray:
    """Routing ids of one GPU's share of the experts under expert parallelism
    (the grouped backend's H200 EP8 scope, Chord page, "Grouped SM90
    kernels"): a global id g in [0, len(expert_map)) becomes expert_map[g],
    the share's local expert or -1 for one held elsewhere; any other id
    becomes -1. Rows with -1 contribute nothing, as ids outside [0, E) do.
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    m = np.asarray(expert_map).astype(np.int64)
    ok = (ids >= 0) & (ids < m.size)
    return np.where(ok, m[np.clip(ids, 0, max(m.size - 1, 0))], -1).astype(np.int32)


def permute(x_bits, al: dict, topk: int) -> np.ndarray:
    """Gather activation rows into the sorted, padded order of an alignment.

    Row p of the result is x[sorted_ids[p] // topk] for a routed slot and a
    zero row for a sentinel slot; there are cap rows. This is the gather the
    indexed layout leaves to the kernel: unpadded activations, padding carried
    by sentinel indices (Chord page, "Grouped SM90 kernels", Fig. 3).
    """
    x = np.asarray(x_bits)
    sid = al["sorted_ids"].astype(np.int64)
    out = np.zeros((sid.size, x.shape[1]), dtype=np.uint16)
    ok = sid < al["sentinel"]
    out[ok] = x[sid[ok] // topk]
    return out


def contiguous_layout(x_bits, topk_ids, E: int, block: int = 128, rows: int | None = None):
    """Build the contiguous grouped layout from a routing.

    Each expert's rows are contiguous and padded to a multiple of ``block``
    (128 on the Chord page, "Grouped SM90 kernels", Fig. 3). Returns
    (a [M_pad, H] bf16 bits, m_indices int32[M_pad] with -1 on pad rows,
    row_src int32[M_pad] = t*topk+j or -1). M_pad is the aligned total, or
    ``rows`` if given (extra rows are padding).
    """
    T, k = np.asarray(topk_ids).shape
    al = align(topk_ids, E, block)
    m_pad = al["total"] if rows is None else rows
    assert m_pad >= al["total"] and m_pad % block == 0
    a = np.zeros((m_pad, np.asarray(x_bits).shape[1]), dtype=np.uint16)
    sid = al["sorted_ids"][:al["total"]].astype(np.int64)
    ok = sid < al["sentinel"]
    a[:al["total"]][ok] = np.asarray(x_bits)[sid[ok] // k]
    m_idx = np.full(m_pad, -1, dtype=np.int32)
    row_src = np.full(m_pad, -1, dtype=np.int32)
    be = np.repeat(al["block_expert"][:al["total"] // block], block)
    m_idx[:al["total"]][ok] = be[ok]
    row_src[:al["total"]][ok] = sid[ok]
    return a, m_idx, row_src


# --------------------------------------------------------------------------
# Expert FFN and the three layouts
# --------------------------------------------------------------------------

def silu(z):
    """SiLU z / (1 + exp(-z)) in float64 (the gate of SwiGLU)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x_rows_bits, w13_bits, w2_bits):
    """One expert on a set of rows: W13 GEMM, SwiGLU, W2 GEMM.

    h = x . W13^T (float64, unrounded); gate = h[:, :I], up = h[:, I:]
    (reading: W13 rows [0, I) are the gate projection, [I, 2I) the up
    projection); a = bf16(silu(gate) * up) is the BF16 input of the second
    GEMM; y = a . W2^T (float64, unrounded).
    Returns (h, a_bits, y).
    """
    x = bf16_to_f64(x_rows_bits)
    w13 = bf16_to_f64(w13_bits)
    I = w13.shape[0] // 2
    h = x @ w13.T
    a_bits = bf16_round(silu(h[:, :I]) * h[:, I:])
    y = bf16_to_f64(a_bits) @ bf16_to_f64(w2_bits).T
    return h, a_bits, y


# --------------------------------------------------------------------------
# Unfused steps with BF16 hand-offs (the GEMM-level contract the Chord page
# times in "Grouped SM90 kernels" and "H200 prefill and TP8": routing,
# activation and communication outside the GEMMs)
# --------------------------------------------------------------------------

def gate_up_rows(x_rows_bits, w13_bits) -> np.ndarray:
    """First grouped GEMM with a BF16 output: bf16(x . W13^T), float64 dot
    products rounded once. Columns follow W13's rows: gate [0, I), up
    [I, 2I)."""
    return bf16_round(bf16_to_f64(x_rows_bits) @ bf16_to_f64(w13_bits).T)


def swiglu_rows(h_bits) -> np.ndarray:
    """SwiGLU of BF16 rows [.., 2I]: a = bf16(silu(g) * u), g = h[:, :I] and
    u = h[:, I:] widened exactly (as in expert_ffn, from BF16 inputs)."""
    h = bf16_to_f64(h_bits)
    I = h.shape[-1] // 2
    return bf16_round(silu(h[..., :I]) * h[..., I:])


def down_rows(a_bits, w2_bits) -> np.ndarray:
    """Second grouped GEMM with a BF16 output: bf16(a . W2^T)."""
    return bf16_round(bf16_to_f64(a_bits) @ bf16_to_f64(w2_bits).T)


def _expert_weights(weights, e):
    if callable(weights):
        return weights(e)
    return tuple(w[e] for w in weights)


class _DequantCache:
    def __init__(self, weights):
        self.weights = weights
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            w13_q, w13_s, w2_q, w2_s = _expert_weights(self.weights, e)
            self.cache[e] = (dequant(w13_q, w13_s), dequant(w2_q, w2_s))
        return self.cache[e]


def moe_indexed(x_bits, topk_ids, topk_w, weights, E: int, tokens=None, keep=False):
    """Indexed-layout MoE layer: out[t] = sum_j w[t,j] * y(t, j).

    Each routed row (t, j) runs through expert topk_ids[t, j] (expert_ffn) and
    the top-k-weighted combine adds the rows per token in ascending j, in
    float64, without rounding the result. Reading: the routing weight applies
    after the second GEMM; ids outside [0, E) contribute nothing.

    ``weights`` is (w13_q[E], w13_s[E], w2_q[E], w2_s[E]) or a callable
    e -> that tuple. ``tokens`` restricts the computation to those tokens
    (rows of the result follow ``tokens``). With ``keep`` the per-row h, a, y
    are returned keyed by flat index.
    """
    x = np.asarray(x_bits)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_w).astype(np.float64)
    T, k = ids.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    H = x.shape[1]
    Y = np.zeros((tok.size, k, H), dtype=np.float64)
    wq = _DequantCache(weights)
    rows_h, rows_a, rows_y = {}, {}, {}
    for e in range(E):
        sel = np.argwhere(ids[tok] == e)              # (position in tok, j)
        if sel.size == 0:
            continue
        w13, w2 = wq(e)
        h, a, y = expert_ffn(x[tok[sel[:, 0]]], w13, w2)
        Y[sel[:, 0], sel[:, 1]] = y
        if keep:
            for r, (ti, j) in enumerate(sel):
                f = int(tok[ti]) * k + int(j)
                rows_h[f], rows_a[f], rows_y[f] = h[r], a[r], y[r]
    out = combine(Y, w[tok])
    if keep:
        return out, dict(h=rows_h, a=rows_a, y=rows_y)
    return out


def combine(Y, topk_w) -> np.ndarray:
    """Top-k-weighted combine: out[t] = sum_j topk_w[t, j] * Y[t, j], the
    terms added in ascending j in float64 and left unrounded. Y is
    [T, topk, H] (zero for a row routed nowhere), topk_w is [T, topk].
    Reading: the routing weight multiplies the second GEMM's output (the
    north-star statement's "top-k-weighted combine"; the Chord page's timings
    exclude it, "Measurements")."""
    Y = np.asarray(Y, dtype=np.float64)
    w = np.asarray(topk_w).astype(np.float64)
    out = np.zeros((Y.shape[0], Y.shape[2]), dtype=np.float64)
    for j in range(Y.shape[1]):
        out += w[:, j][:, None] * Y[:, j]
    return out


def moe_contiguous(a_bits, m_indices, weights, row_src=None, topk_w=None, T=None, topk=None,
                   keep=False):
    """Contiguous-layout MoE layer.

    Rows of ``a`` are grouped by expert, each expert padded to a 128-row
    boundary; m_indices gives each row's expert and -1 marks padding (Chord
    page, "Grouped SM90 kernels", Fig. 3). Every non-pad row runs through its
    expert. Without ``row_src`` the result is y per row ([M_pad, H], NaN on
    pad rows). With ``row_src`` (row -> t*topk+j, -1 on pads) the rows are
    combined per token as in moe_indexed ([T, H]).
    """
    a = np.asarray(a_bits)
    m_idx = np.asarray(m_indices)
    M, H = a.shape
    y_all = np.full((M, H), np.nan)
    wq = _DequantCache(weights)
    a_rows = {}
    for e in np.unique(m_idx[m_idx >= 0]):
        rows = np.flatnonzero(m_idx == e)
        w13, w2 = wq(int(e))
        _, aa, y = expert_ffn(a[rows], w13, w2)
        y_all[rows] = y
        if keep:
            for r, row in enumerate(rows):
                a_rows[int(row)] = aa[r]
    if row_src is None:
        return (y_all, a_rows) if keep else y_all
    src = np.asarray(row_src)
    w = np.asarray(topk_w).astype(np.float64)
    Y = np.zeros((T, topk, H))
    ok = (src >= 0) & (m_idx >= 0)
    f = src[ok].astype(np.int64)
    Y[f // topk, f % topk] = y_all[ok]
    out = combine(Y, w)
    return (out, a_rows) if keep else out


def moe_masked(a3_bits, masked_m, weights, keep=False):
    """Masked-layout MoE layer.

    a3 [E, max_m, H] reserves a fixed row budget per expert and masked_m[e]
    is the number of valid rows; the output is flat [E*max_m, H] and rows
    beyond the valid count carry nothing (Chord page, "Grouped SM90 kernels").
    Reading: masked_m is clamped to [0, max_m]; invalid output rows are NaN
    here (unspecified for an implementation).
    """
    a3 = np.asarray(a3_bits)
    E, max_m, H = a3.shape
    out = np.full((E * max_m, H), np.nan)
    wq = _DequantCache(weights)
    a_rows = {}
    for e in range(E):
        m = int(min(max(int(masked_m[e]), 0), max_m))
        if m == 0:
            continue
        w13, w2 = wq(e)
        _, aa, y = expert_ffn(a3[e, :m], w13, w2)
        out[e * max_m:e * max_m + m] = y
        if keep:
            for r in range(m):
                a_rows[e * max_m + r] = aa[r]
    return (out, a_rows) if keep else out


# --------------------------------------------------------------------------
# Tolerance
# --------------------------------------------------------------------------

def compare(got, ref) -> dict:
    """Relative Frobenius error, max-abs error over rms(ref), and the BF16
    output-rounding floor max|bf16(ref) - ref| / rms(ref), in float64 over the
    elements given."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    diff = g - r
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    nref = float(np.linalg.norm(r))
    floor = float(np.max(np.abs(bf16_to_f64(bf16_round(r)) - r))) / rms if rms > 0 else 0.0
    return dict(rel_fro=float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff)),
                max_abs_over_rms=float(np.max(np.abs(diff))) / rms if rms > 0 else float(np.max(np.abs(diff), initial=0.0)),
                bf16_floor=floor, rms=rms, n=int(r.size))
