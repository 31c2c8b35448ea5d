"""Oracle for one decoder-layer forward over a hybrid (chunked-prefill + decode) batch.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP path: it derives token positions, page slots,
norms, rotary embeddings, attention and the gated FFN on its own, in float64
with numpy (the linear layers use numpy's matrix product; every other
reduction is an elementwise product followed by numpy's sum over one axis, so
each output row depends only on that row's inputs, not on the batch around it).

Sources (the pages):
  [notes]  "Sarathi-Serve reading notes" (zhongzhuzhou.org, 2026-05-20):
           §1.6 linear-layer cost, §2.3/§3.1 chunked prefills, §3.2 hybrid
           batches, §3.4 scheduling loop, §3.5 paged KV, §7.5b chunked
           attention work identity, §7.6 worked Yi-34B iteration.
  [cp]     "Chunked Prefill" (bowenzhou.top): "mechanism" (chunks continue the
           KV through paged blocks) and the hybrid-iteration roofline.

What the layer computes.  The pages never write a layer out; they state that a
chunk's tokens attend to everything earlier chunks of the same prompt wrote
plus, causally, themselves ([notes] §3.1, §7.5b), that a decode attends to its
own cached context ([notes] §3.2), and that all tokens of the batch share the
linear layers ([notes] §1.6, [cp] roofline).  The decoder block itself is the
pre-norm Llama/Mistral form (RMSNorm, rotary embedding on q/k, grouped-query
attention, SwiGLU FFN, two residual adds, no biases).  Readings taken where the
pages are silent:
  * RMSNorm eps = 1e-5 (from dims); gains multiply after normalisation.
  * RoPE: rotate-half pairing (i, i + d/2), inv_freq_i = theta^(-2i/d),
    theta from dims (1e4); angles and cos/sin in float64.
  * Softmax scale 1/sqrt(d); q head h reads kv head floor(h / g), g = n_q/n_kv.
  * A decode's context length counts tokens already cached: its token sits at
    position ctx, is appended there and attends ctx + 1 keys -- a 1-token
    chunk whose prefix is ctx.
  * Sequence order is chunks (argument order) then decodes; tokens are packed
    in that order.
  * Storage precision.  "bf16 layer" is read as: every activation tensor that
    passes between steps is held in bf16 -- the normed input, q/k/v after the
    rotary embedding (k/v are what the bf16 KV cache stores), the attention
    output, the normed residual and the gated FFN activation -- while the
    residual stream x, h1, y stays fp32.  With ``storage="bf16"`` the oracle
    computes every step exactly (float64) from its stored inputs and rounds its
    output once to that storage type (round to nearest even).  With
    ``storage="exact"`` nothing is rounded.

FP8 KV storage (kv_fp8 = 1; not on the pages, which keep K/V in the layer's
own precision): each K or V element is stored as the OCP e4m3fn code of
x / scale, with the per-layer K and V scales the caller passes (float32).
Codes round to nearest with ties to the even code and saturate at +-448 (the
format's largest finite value; 0x7F / 0xFF are NaN and mark unwritten slots).
The quotient x / scale is taken in single precision (see ``fp8_quotient``), and
attention reads code * scale.

FP8 projections (w8a8 = 1; not on the pages, which name FP8 only as moving
the compute/bandwidth knee): the weights are e4m3 codes with one float32 scale
per output channel (row of the [d_out][d_in] matrix), and the four
projection inputs -- the normed input xn, the attention output o, the normed
residual h1n and the SwiGLU output a -- are stored as e4m3 codes of
value / scale with one static float32 scale each (x_scale, o_scale, h_scale,
a_scale), taken as for the KV cache (``fp8_quotient``, nearest-even,
saturating).  A projection is then (codes_a * s_a) . (codes_w * s_w)^T,
computed exactly.  q, the KV cache (bf16 or its own FP8) and the fp32
residual stream are unchanged.

Page layout of the oracle's own cache: ``k[page][kv_head][slot][d]`` (logical
order, float64); a sequence's position p lives in page
``block_table[s][p // page_size]`` at slot ``p % page_size`` ([notes] §3.5,
[cp] "mechanism": KV continues across chunks through paged blocks).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Dict, Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# number formats


def bf16_bits_to_float(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


_BLOCK_ROWS = 2048
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        _POOL = concurrent.futures.ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


def _by_row_blocks(fn, x: np.ndarray, *args) -> np.ndarray:
    """fn applied to blocks of rows of a large 2-D array on a thread pool
    (numpy releases the GIL inside its loops).  Only for functions that act on
    each element or each row on its own, so the result is bit-identical to
    fn(x, *args) -- a matter of speed for the 32768-token prompt."""
    if x.ndim != 2 or x.shape[0] <= _BLOCK_ROWS or x.size < (1 << 22):
        return fn(x, *args)
    starts = range(0, x.shape[0], _BLOCK_ROWS)
    parts = list(_pool().map(lambda r0: fn(x[r0:r0 + _BLOCK_ROWS], *args), starts))
    return np.concatenate(parts, axis=0)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one step
    (no intermediate float32).  bf16 keeps 8 significant bits and float32's
    exponent range; below 2**-126 the spacing is fixed at 2**-133."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 2 and x.size >= (1 << 22):
        return _by_row_blocks(_round_bf16, x)
    return _round_bf16(x)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)                      # xf = m * 2**e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 8, -133))  # spacing of bf16 values near xf
    r = np.rint(xf / q) * q                  # np.rint rounds half to even
    over = np.abs(r) > 3.3895313892515355e38   # largest finite bf16
    r[over] = np.copysign(np.inf, xf[over])
    out[finite] = r
    return out


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(x) -> np.ndarray:
    """float64 values already on the bf16 grid -> bit patterns."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# batch layout: which token sits at which position of which sequence


@dataclass
class TokenLayout:
    seq: np.ndarray       # int64 [T]  sequence of each packed token
    pos: np.ndarray       # int64 [T]  position of the token in its sequence
    q_start: np.ndarray   # int64 [S+1] first packed token of each sequence
    cached: np.ndarray    # int64 [S]  tokens already cached before this batch
    kv_len: np.ndarray    # int64 [S]  cached + new tokens


def token_layout(chunk_len: Sequence[int], chunk_prefix: Sequence[int],
                 decode_ctx: Sequence[int]) -> TokenLayout:
    """Chunk i of a prompt covers positions [prefix, prefix + len) ([notes] §3.1:
    chunk i covers [(i-1)C, iC)); a decode is one token at position ctx.
    Chunks first, then decodes ([notes] §3.2 hybrid batch)."""
    cached = [int(p) for p in chunk_prefix] + [int(c) for c in decode_ctx]
    new = [int(n) for n in chunk_len] + [1] * len(decode_ctx)
    seq, pos, q_start = [], [], [0]
    for s, (c, n) in enumerate(zip(cached, new)):
        for j in range(n):
            seq.append(s)
            pos.append(c + j)
        q_start.append(q_start[-1] + n)
    cached_a = np.array(cached, dtype=np.int64)
    return TokenLayout(np.array(seq, dtype=np.int64), np.array(pos, dtype=np.int64),
                       np.array(q_start, dtype=np.int64), cached_a,
                       cached_a + np.array(new, dtype=np.int64))


def page_of(block_table: np.ndarray, seq: int, pos: int, page_size: int):
    """Physical (page, slot) of position ``pos`` of sequence ``seq``."""
    page = int(block_table[seq][pos // page_size])
    return page, pos % page_size


def hybrid_batch_budget(n_decodes: int, chunk_takes: Sequence[int], tau: int):
    """Token accounting of one hybrid batch ([notes] §3.2, §3.4): decodes are
    admitted first (one token each), then chunk pieces; returns the budget left
    after the decodes and after each chunk, and the batch's token count.
    Raises if the batch exceeds tau."""
    left = [tau - n_decodes]
    for c in chunk_takes:
        left.append(left[-1] - int(c))
    total = n_decodes + sum(int(c) for c in chunk_takes)
    if total > tau:
        raise ValueError(f"hybrid batch of {total} tokens exceeds the budget {tau}")
    return left, total


# ----------------------------------------------------------------------------
# the oracle's paged KV cache


# ----------------------------------------------------------------------------
# FP8 e4m3 KV cache (optional storage type)
#
# OCP 8-bit floating point, E4M3 ("e4m3fn"): sign bit, 4 exponent bits with
# bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals (m/8) * 2^-6;
# other fields (1 + m/8) * 2^(e - 7).  No infinities; code 0x7F (and 0xFF) is
# NaN, so the largest finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).
# Reading for the cache: a value x is stored as e4m3(x / scale), rounded to
# the nearest code value with ties to the even code, magnitudes past 448
# saturating to 448; it is read back as value(code) * scale.


def _e4m3_magnitude(code: int) -> float:
    e, m = code >> 3, code & 7
    if e == 0:
        return (m / 8.0) * 2.0 ** -6
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_MAG = np.array([_e4m3_magnitude(c) for c in range(127)])   # codes 0x00..0x7E, increasing


def e4m3_encode(x) -> np.ndarray:
    """float array -> uint8 e4m3 codes (round to nearest, ties to even code,
    saturating at +-448, NaN -> 0x7F with the input's sign)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), _E4M3_MAG[-1])
    hi = np.clip(np.searchsorted(_E4M3_MAG, a, side="left"), 0, 126)   # first code >= a
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_MAG[hi] - a
    d_lo = a - _E4M3_MAG[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return (code | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = np.concatenate([_E4M3_MAG, [np.nan]])[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def fp8_quotient(x, scale) -> np.ndarray:
    """x / scale as the FP8 code is taken from it: in single precision, x
    rounded to float32 times the float32 reciprocal of the float32 scale.  The
    pages fix no precision for this step; where x / scale lies at (or within
    float32 rounding of) the midpoint of two codes, the precision decides the
    code, so the kernels' single-precision product is the definition here."""
    inv = np.float32(1.0) / np.float32(scale)
    return (np.asarray(x, dtype=np.float64).astype(np.float32) * inv).astype(np.float64)


def fp8_store(x, scale) -> np.ndarray:
    """The value an e4m3 store of x with the given scale reads back:
    decode(encode(x / scale)) * scale, the quotient as in ``fp8_quotient``."""
    return e4m3_decode(e4m3_encode(fp8_quotient(x, scale))) * np.float64(np.float32(scale))


def fp8_weight(codes, row_scales) -> np.ndarray:
    """Weights [d_out][d_in] from e4m3 codes and one float32 scale per
    output row."""
    s = np.asarray(row_scales, dtype=np.float32).astype(np.float64)
    return e4m3_decode(codes) * s[:, None]


class PagedCache:
    """K and V pages in logical order [kv_head][slot][d], float64.

    Pages are held sparsely: a page comes into being, filled with NaN, the
    first time something is written to it, so a cache over a large pool costs
    only the pages actually used.  Reading a slot nobody wrote returns NaN."""

    def __init__(self, num_pages: int, n_kv: int, page_size: int, head_dim: int, kv_fp8: int = 0,
                 k_scale: float = 1.0, v_scale: float = 1.0):
        self.num_pages = num_pages
        self.n_kv = n_kv
        self.page_size = page_size
        self.head_dim = head_dim
        self.pages: Dict[int, np.ndarray] = {}   # page -> [2 (K, V)][n_kv][slot][d]
        # FP8 storage: written values are quantised (e4m3(x / scale)); pages
        # hold the values read back, codes the stored bytes (0x7F where unwritten).
        # The scales are single-precision numbers (as a caller hands them over)
        self.kv_fp8 = int(kv_fp8)
        self.scales = (np.float32(k_scale), np.float32(v_scale))
        self.codes: Dict[int, np.ndarray] = {}

    def _page(self, page: int) -> np.ndarray:
        if not 0 <= page < self.num_pages:
            raise IndexError(f"page {page} outside the pool of {self.num_pages}")
        pg = self.pages.get(page)
        if pg is None:
            pg = np.full((2, self.n_kv, self.page_size, self.head_dim), np.nan)
            self.pages[page] = pg
        return pg

    def write(self, block_table, seq: int, pos: int, k_row: np.ndarray, v_row: np.ndarray):
        page, slot = page_of(block_table, seq, pos, self.page_size)
        pg = self._page(page)
        if self.kv_fp8:
            cd = self.codes.setdefault(page, np.full(pg.shape, 0x7F, dtype=np.uint8))
            for i, (row, sc) in enumerate(((k_row, self.scales[0]), (v_row, self.scales[1]))):
                cd[i, :, slot, :] = e4m3_encode(fp8_quotient(row, sc))
                pg[i, :, slot, :] = e4m3_decode(cd[i, :, slot, :]) * np.float64(sc)
            return
        pg[0, :, slot, :] = k_row
        pg[1, :, slot, :] = v_row

    def load_prefix(self, block_table, seq: int, k_rows: np.ndarray, v_rows: np.ndarray):
        """Place already-cached K/V (positions 0..len-1) of ``seq``."""
        for pos in range(k_rows.shape[0]):
            self.write(block_table, seq, pos, k_rows[pos], v_rows[pos])

    def gather(self, block_table, seq: int, length: int):
        """Keys/values of positions 0..length-1 of ``seq``: [length][n_kv][d]."""
        ks = np.empty((length, self.n_kv, self.head_dim))
        vs = np.empty_like(ks)
        for pos in range(length):
            page, slot = page_of(block_table, seq, pos, self.page_size)
            pg = self.pages.get(page)
            if pg is None:
                ks[pos] = vs[pos] = np.nan
            else:
                ks[pos] = pg[0, :, slot, :]
                vs[pos] = pg[1, :, slot, :]
        return ks, vs

    def dense(self):
        """Whole pool as (K, V), each [num_pages][n_kv][slot][d]; NaN where unwritten."""
        shp = (self.num_pages, self.n_kv, self.page_size, self.head_dim)
        k = np.full(shp, np.nan)
        v = np.full(shp, np.nan)
        for page, pg in self.pages.items():
            k[page] = pg[0]
            v[page] = pg[1]
        return k, v


# ----------------------------------------------------------------------------
# layer pieces


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, row-wise."""
    return _by_row_blocks(_rmsnorm, np.asarray(x), gain, eps)


def _rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """angle[t][i] = pos_t * theta^(-2i/d), i < d/2."""
    half = head_dim // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(u: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of u[t][head][d] by position pos[t]."""
    d = u.shape[-1]
    half = d // 2
    ang = rope_angles(pos, d, theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def linear(x: np.ndarray, w: np.ndarray):
    """y = x . w^T for w stored [d_out][d_in]; returns y and the flop count
    2 * n * d_in * d_out of the product ([notes] §1.6).

    numpy's BLAS sends products with very few rows to dedicated small-matrix
    routines whose summation order differs from the general one; fewer than 16
    rows are therefore padded with zero rows, so that every row's result is
    independent of how many rows share the call."""
    n, d_in = x.shape
    d_out = w.shape[0]
    if n < 16:
        y = (np.concatenate([x, np.zeros((16 - n, d_in))]) @ w.T)[:n]
    else:
        y = x @ w.T
    return y, 2 * n * d_in * d_out


def paged_attention(q: np.ndarray, tok_seq: np.ndarray, tok_pos: np.ndarray,
                    cache: PagedCache, block_table: np.ndarray, n_kv: int):
    """Attention of queries q[i][head][d] over their own sequences' paged KV.

    Query i (sequence tok_seq[i], position tok_pos[i]) sees exactly keys
    0..tok_pos[i] of its sequence -- a chunk's token sees every earlier chunk's KV plus,
    causally, its own chunk ([notes] §3.1, §7.5b); a decode sees its whole
    context plus itself.  Scores q.k / sqrt(d), softmax (max first, then
    exp(s - max), then the weighted sum of V over the total weight); q head h
    reads kv head h // (n_q / n_kv).  Returns o[i][head][d] and the number of
    (query, key) pairs attended.
    """
    n, nq, d = q.shape
    g = nq // n_kv
    scale = 1.0 / math.sqrt(d)
    o = np.zeros((n, nq, d), dtype=np.float64)
    pairs = 0
    by_seq: Dict[int, list] = {}
    for i in range(n):
        by_seq.setdefault(int(tok_seq[i]), []).append(i)
    for s, idx in by_seq.items():
        length = int(np.max(np.asarray(tok_pos)[idx])) + 1
        ks, vs = cache.gather(block_table, s, length)

        def one_row(i):
            p = int(tok_pos[i])
            for h in range(nq):
                kvh = h // g
                kk, vv = ks[:p + 1, kvh], vs[:p + 1, kvh]
                sc = np.sum(kk * q[i, h], axis=1) * scale      # q . k_j / sqrt(d)
                e = np.exp(sc - np.max(sc))
                o[i, h] = np.sum(e[:, None] * vv, axis=0) / np.sum(e)
            return p + 1

        # rows are independent; long contexts run on a thread pool (same
        # arithmetic per row, so the same result)
        if length >= 4096 and len(idx) > 1:
            pairs += sum(_pool().map(one_row, idx))
        else:
            pairs += sum(one_row(i) for i in idx)
    return o, pairs


# ----------------------------------------------------------------------------
# the layer


@dataclass
class LayerResult:
    y: np.ndarray            # [len(rows)][H]
    rows: np.ndarray         # packed token indices of y's rows
    pairs: int               # (query, key) pairs attended by the computed rows
    linear_flops: int        # 2 n d_in d_out summed over the products actually run
    attn_out: Optional[np.ndarray] = None   # [len(rows)][n_q*d] (stored precision)
    stored: Optional[Dict[str, np.ndarray]] = None   # every stored activation (keep_stored)


def layer_forward(dims, w: Dict[str, np.ndarray], x: np.ndarray, chunk_len, chunk_prefix,
                  decode_ctx, block_table: np.ndarray, cache: PagedCache,
                  storage: str = "bf16", rows: Optional[Sequence[int]] = None,
                  keep_attn: bool = False, keep_stored: bool = False,
                  perturb: Optional[Callable[[str, np.ndarray], np.ndarray]] = None) -> LayerResult:
    """One pre-norm decoder layer over the hybrid batch; writes the batch's new
    K/V into ``cache`` and returns y for ``rows`` (all tokens by default).

    ``w`` holds float64 arrays: w_q [n_q d][H], w_k, w_v [n_kv d][H],
    w_o [H][n_q d], w_g, w_u [F][H], w_d [H][F], g_attn, g_ffn [H].
    K/V are computed for every token (the cache needs them); steps after the
    projections run only for ``rows`` -- exact for those rows.

    Test hooks (both off by default, leaving the arithmetic above untouched):
    ``keep_stored`` returns every stored activation (xn, q, k, v, o, h1, h1n,
    a; xn of the rows, and as xn_all of every token) in ``LayerResult.stored``; ``perturb(name, value)`` is applied to each
    of those values, and to y, right before it is rounded to its storage type
    -- how sensitive the result is to a change of size ulp(fp32) at one
    storage point (the conditioning of the layer under its own roundings).
    """
    hook = perturb if perturb is not None else (lambda name, a: a)
    if storage == "bf16":
        rb, rf = round_bf16, round_f32
    elif storage == "exact":
        rb = rf = (lambda a: a)
    else:
        raise ValueError(storage)
    act = lambda a, name: rb(hook(name, a))
    res = lambda a, name: rf(hook(name, a))
    lay = token_layout(chunk_len, chunk_prefix, decode_ctx)
    T = len(lay.seq)
    d = dims.head_dim
    nq, nkv = dims.n_q_heads, dims.n_kv_heads
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    x = np.asarray(x, dtype=np.float64)
    flops = 0
    # projection inputs: bf16 storage, or e4m3 codes with a static scale
    if getattr(dims, "w8a8", 0):
        gin = lambda a, name, scale: fp8_store(hook(name, a), getattr(dims, scale))
    else:
        gin = lambda a, name, scale: act(a, name)

    # a1: RMSNorm of the input (all tokens: K/V need it)
    xn = gin(rmsnorm(x, w["g_attn"], dims.rms_eps), "xn", "x_scale")
    # a2 + a3: projections and rotary embedding
    k, f = linear(xn, w["w_k"]); flops += f
    v, f = linear(xn, w["w_v"]); flops += f
    q, f = linear(xn[rows], w["w_q"]); flops += f
    k = rope(k.reshape(T, nkv, d), lay.pos, dims.rope_theta)
    v = v.reshape(T, nkv, d)
    q = act(rope(q.reshape(len(rows), nq, d), lay.pos[rows], dims.rope_theta), "q")
    # a bf16 cache stores bf16(k), bf16(v); an FP8 cache quantises the unrounded
    # values itself (e4m3(x / scale))
    if getattr(dims, "kv_fp8", 0) != cache.kv_fp8:
        raise ValueError("cache storage type does not match dims.kv_fp8")
    if cache.kv_fp8:
        k, v = hook("k", k), hook("v", v)
    else:
        k, v = act(k, "k"), act(v, "v")

    # a4: new K/V go into the paged cache at their sequence positions
    for t in range(T):
        cache.write(block_table, int(lay.seq[t]), int(lay.pos[t]), k[t], v[t])

    # a5: each token attends causally to positions 0..pos of its own sequence
    o, pairs = paged_attention(q, lay.seq[rows], lay.pos[rows], cache, block_table, nkv)
    o = gin(o.reshape(len(rows), nq * d), "o", "o_scale")

    # a6: output projection + residual
    ao, f = linear(o, w["w_o"]); flops += f
    h1 = res(x[rows] + ao, "h1")
    # a7 + a8: RMSNorm, gate/up projections and SwiGLU
    h1n = gin(rmsnorm(h1, w["g_ffn"], dims.rms_eps), "h1n", "h_scale")
    gt, f1 = linear(h1n, w["w_g"])
    up, f2 = linear(h1n, w["w_u"])
    a = gin(silu(gt) * up, "a", "a_scale")
    # a9: down projection + residual
    dn, f3 = linear(a, w["w_d"])
    flops += f1 + f2 + f3
    y = res(h1 + dn, "y")
    stored = dict(xn=xn[rows], xn_all=xn, q=q, k=k, v=v, o=o, h1=h1, h1n=h1n, a=a) if keep_stored else None
    return LayerResult(y, rows, pairs, flops, o if keep_attn else None, stored)


def weights_to_float(wbits: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Layer parameters as float64: bf16 bit patterns, or (w8a8) projection
    matrices as e4m3 codes with row scales under "s_" + name."""
    out = {}
    for k, v in wbits.items():
        if k.startswith("s_"):
            continue
        if ("s_" + k) in wbits:
            out[k] = fp8_weight(v, wbits["s_" + k])
        else:
            out[k] = bf16_bits_to_float(v)
    return out
