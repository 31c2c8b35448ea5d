"""Shared pieces of the GPU parity tests: running the oracle on a workload,
sampling rows at full size, and comparing results."""
from __future__ import annotations

import sys
import time

import numpy as np

from oracle import hybrid_layer as O

# floating-point bar: bf16 inputs, fp32 accumulation vs the oracle
TOL_REL_L2 = 1e-2
TOL_MAX_ABS = 5e-2


def log(*a):
    print(f"[{time.strftime('%H:%M:%S')}]", *a, flush=True)
    sys.stdout.flush()


def oracle_cache(wl, seqs=None, prefixes=True):
    b, d = wl.batch, wl.dims
    cache = O.PagedCache(b.num_pages, d.n_kv_heads, d.page_size, d.head_dim, kv_fp8=getattr(d, "kv_fp8", 0),
                         k_scale=getattr(d, "k_scale", 1.0), v_scale=getattr(d, "v_scale", 1.0))
    if prefixes:
        for s in (range(b.n_seq) if seqs is None else seqs):
            if s < len(wl.prefix_k) and wl.prefix_k[s].shape[0]:
                cache.load_prefix(b.block_table, s, O.bf16_bits_to_float(wl.prefix_k[s]),
                                  O.bf16_bits_to_float(wl.prefix_v[s]))
    return cache


def oracle_forward(wl, x=None, rows=None, storage="bf16", cache=None, batch=None, keep_attn=False):
    b = wl.batch if batch is None else batch
    w = O.weights_to_float(wl.weights)
    cache = oracle_cache(wl) if cache is None else cache
    x = wl.x if x is None else x
    r = O.layer_forward(wl.dims, w, x.astype(np.float64), b.chunk_len, b.chunk_prefix, b.decode_ctx,
                        b.block_table, cache, storage=storage, rows=rows, keep_attn=keep_attn)
    return r, cache


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return rel, mx


def assert_close(got, ref, what="", max_abs=TOL_MAX_ABS, rel_l2=TOL_REL_L2):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel, mx = errors(got, ref)
    log(f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e} (|ref|max={np.max(np.abs(ref)):.3f}, "
        f"bounds {rel_l2:.3e} / {max_abs:.3e})")
    assert rel <= rel_l2 and mx <= max_abs, (what, rel, mx)
    return rel, mx


def conditioning_floor(wl, rows, cache_seqs, seed=0, eps=1e-7):
    """Max-abs change of the oracle's own output (bf16 storage) when its input
    x is multiplied by 1 + eps N(0, 1), eps = 1e-7 by default: the size of the
    rounding cascade any implementation whose arithmetic differs from float64
    by an fp32 ulp must show on these rows (each storage point turns a
    perturbation eps into one-step flips with probability eps/ulp)."""
    rng = np.random.default_rng(seed)
    x = wl.x.astype(np.float64)
    xp = x * (1.0 + eps * rng.standard_normal(x.shape))
    y0, _ = oracle_forward(wl, x=x, rows=rows, cache=oracle_cache(wl, seqs=cache_seqs))
    y1, _ = oracle_forward(wl, x=xp, rows=rows, cache=oracle_cache(wl, seqs=cache_seqs))
    return errors(y1.y, y0.y)


# relative error of one FP8 MFMA's sum, as a fraction of the sum of |products|
# (measured worst: about 1800 fp32 ulps, 2^-13)
FP8_MFMA_REL_ERR = 2.0 ** -13


def w8a8_bound(wl, rows=None, cache_seqs=None):
    """Max-abs bar for FP8 projections.  A relative error of the FP8 MFMA's
    summation (FP8_MFMA_REL_ERR) moves a pre-quantisation value across an e4m3
    rounding boundary now and then, and such a code is a full e4m3 step (6 to
    12 %) away from the oracle's; the flips propagate through the layer.  The
    bars are the literal ones, or twice the oracle's own response to a
    relative perturbation of its input of that size where that is larger.
    Returns keyword arguments for assert_close."""
    frel, fmax = conditioning_floor(wl, rows, cache_seqs, eps=FP8_MFMA_REL_ERR)
    bars = dict(rel_l2=max(TOL_REL_L2, 2.0 * frel), max_abs=max(TOL_MAX_ABS, 2.0 * fmax))
    log(f"{wl.name}: oracle response to a {FP8_MFMA_REL_ERR:.1e} relative input perturbation: "
        f"rel_l2={frel:.3e} max_abs={fmax:.3e}; bars {bars['rel_l2']:.3e} / {bars['max_abs']:.3e}")
    return bars


def sample_rows(wl, n_random=48, seed=0):
    """Rows for full-size parity: first/last token of every chunk, tokens at
    attention-tile and page boundaries, every decode, plus random rows."""
    b = wl.batch
    lay = O.token_layout(b.chunk_len, b.chunk_prefix, b.decode_ctx)
    T = len(lay.seq)
    rows = set()
    for s in range(b.n_chunks):
        a, e = int(lay.q_start[s]), int(lay.q_start[s + 1])
        rows.update([a, a + 1, e - 2, e - 1])
        for t in range(a, e):
            p = int(lay.pos[t])
            if p % 16 in (0, 15) and (t - a) % 5 == 0:
                rows.add(t)
        for t in range(a, e, 32):
            rows.add(t)
    rows.update(range(int(lay.q_start[b.n_chunks]), T))
    rng = np.random.default_rng(seed)
    rows.update(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T))


def expected_cache_bits(cache, num_pages):
    """Oracle cache as bf16 bit patterns in logical order; NaN -> 0x7FC0."""
    k, v = cache.dense()
    def bits(a):
        out = np.full(a.shape, 0x7FC0, dtype=np.uint16)
        fin = ~np.isnan(a)
        out[fin] = O.bf16_bits(a[fin])
        return out
    return bits(k), bits(v)


# FP8 projections: gfx950's e4m3 MFMA (16x16x128) sums its 128 products to
# about 16 significant bits (measured: mean 200, worst 1800 fp32 ulps of the
# sum of |products| per instruction, against a few ulps for fp32 summation of
# exact products), so more new K/V values sit one bf16 step from the oracle's.
MIN_IDENTICAL_W8A8 = 0.95


def new_values_close(g_bits, e_vals, what, min_identical=0.99):
    """New K/V written by the layer: the GPU rounds an fp32 sum to bf16, the
    oracle a float64 one, so a value may land one bf16 step away, and a value
    near zero (cancellation in the dot product) may differ by the fp32
    accumulation error.  Bound: |g - e| <= ulp(e) + 1e-3 max|e|, ulp(e) the
    bf16 spacing at e (2^(floor(log2|e|) - 7)), with at least 99 % of the
    values bit-identical."""
    g = O.bf16_bits_to_float(g_bits)
    e = np.asarray(e_vals, dtype=np.float64)
    assert np.all(np.isfinite(e)) and np.all(np.isfinite(g)), f"{what}: non-finite value"
    same = O.bf16_bits(e) == g_bits
    err = np.abs(g - e)
    ulp = np.ldexp(1.0, np.frexp(e)[1] - 8)
    bound = ulp + 1e-3 * np.max(np.abs(e))
    frac = 1.0 - float(np.mean(same)) if same.size else 0.0
    log(f"{what}: {frac * 100:.3f}% of new values not bit-identical, max |diff| {err.max(initial=0):.2e}")
    assert np.all(err <= bound), f"{what}: {int(np.sum(err > bound))} values out of bound"
    assert frac <= 1.0 - min_identical, (what, frac)


def expected_cache_codes(cache):
    """Oracle FP8 cache as e4m3 codes in logical order; 0x7F (NaN) where unwritten."""
    shp = (cache.num_pages, cache.n_kv, cache.page_size, cache.head_dim)
    k = np.full(shp, 0x7F, dtype=np.uint8)
    v = np.full(shp, 0x7F, dtype=np.uint8)
    for page, cd in cache.codes.items():
        k[page] = cd[0]
        v[page] = cd[1]
    return k, v


def new_codes_close(g_codes, e_codes, what, min_identical=0.99):
    """New FP8 K/V written by the layer: both sides encode x / scale with the
    same rounding, but the GPU's x is an fp32 sum and the oracle's a float64
    one, so a value at a rounding boundary may land one code step away.
    Bound, on the decoded codes: |g - e| <= the e4m3 spacing at e (2^(e - 3)
    for normal e, 2^-9 below 2^-6) + 1e-3 max|e|, with at least 99 % of the
    codes identical."""
    g = O.e4m3_decode(g_codes)
    e = O.e4m3_decode(e_codes)
    assert np.all(np.isfinite(e)) and np.all(np.isfinite(g)), f"{what}: NaN code"
    same = g_codes == e_codes
    err = np.abs(g - e)
    mag = np.maximum(np.abs(e), 2.0 ** -6)
    step = np.ldexp(1.0, np.frexp(mag)[1] - 4)
    bound = step + 1e-3 * np.max(np.abs(e), initial=0.0)
    frac = 1.0 - float(np.mean(same)) if same.size else 0.0
    log(f"{what}: {frac * 100:.3f}% of new codes not identical, max |diff| {err.max(initial=0):.2e}")
    assert np.all(err <= bound), f"{what}: {int(np.sum(err > bound))} codes out of bound"
    assert frac <= 1.0 - min_identical, (what, frac)


def compare_cache(gpu_kv, cache, num_pages, written_pages_slots=None, what="cache", min_identical=0.99):
    """Bit-exact everywhere the batch did not write (prefixes, NaN decoys and
    tails).  At the batch's new slots: bit-exact if ``written_pages_slots`` is
    None (a pure copy), else ``new_values_close`` (bf16) or ``new_codes_close``
    (FP8 codes)."""
    gk, gv = gpu_kv
    if cache.kv_fp8:
        ek, ev = expected_cache_codes(cache)
        dk, dv = ek, ev
        close = new_codes_close
    else:
        ek, ev = expected_cache_bits(cache, num_pages)
        dk, dv = cache.dense()
        close = new_values_close
    assert gk.dtype == ek.dtype and gk.shape == ek.shape, (what, gk.dtype, gk.shape, ek.shape)
    for name, g, e, dense in (("K", gk, ek, dk), ("V", gv, ev, dv)):
        diff = g != e
        if written_pages_slots is None:
            assert not diff.any(), f"{what} {name}: {int(diff.sum())} elements differ"
            continue
        mask = np.zeros(g.shape, dtype=bool)
        for page, slot in written_pages_slots:
            mask[page, :, slot, :] = True
        assert not (diff & ~mask).any(), f"{what} {name}: bytes outside the new slots changed"
        close(g[mask], dense[mask], f"{what} {name}", min_identical)
