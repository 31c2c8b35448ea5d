"""Shared pieces of the GPU parity tests: running the oracle on a workload,
sampling rows at full size, and comparing results."""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

from oracle import hybrid_layer as O
from chunked_prefill_hybrid_layer_amd import workloads as W

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


def oracle_forward(wl, x=None, rows=None, storage="bf16", cache=None, batch=None, keep_attn=False,
                   keep_stored=False):
    b = wl.batch if batch is None else batch
    w = O.weights_to_float(wl.weights)
    cache = oracle_cache(wl) if cache is None else cache
    x = wl.x if x is None else x
    r = O.layer_forward(wl.dims, w, x.astype(np.float64), b.chunk_len, b.chunk_prefix, b.decode_ctx,
                        b.block_table, cache, storage=storage, rows=rows, keep_attn=keep_attn,
                        keep_stored=keep_stored)
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


# ---------------------------------------------------------------- workloads shared by tests and golden files

# small layers for full-output parity (ragged chunks starting mid-page, decodes
# around page boundaries; g = n_q / n_kv = 4, 7, 1, 16).  The last two give
# the decodes up to twelve attention partials (contexts of 3 K keys in
# 256-key ranges), so the merge takes four lane groups per decode (token,
# head), at d = 64 and 128; g16_d128 takes two.
SMALL = {
    "g4_d128": dict(n_q=8, n_kv=2, head_dim=128),
    "g7_d128": dict(n_q=14, n_kv=2, head_dim=128, hidden=896 + 128, ffn=1536),
    "g1_d64": dict(n_q=4, n_kv=4, head_dim=64, hidden=256, ffn=512),
    "g16_d128": dict(n_q=16, n_kv=1, head_dim=128, chunk_len=(40,), chunk_prefix=(1100,),
                     decode_ctx=(0, 2047, 5)),
    "g1_d64_many_partials": dict(n_q=4, n_kv=4, head_dim=64, hidden=256, ffn=512, chunk_len=(40,),
                                 chunk_prefix=(3000,), decode_ctx=(3000, 1500, 7, 2900)),
    "g4_d128_many_partials": dict(n_q=8, n_kv=2, head_dim=128, chunk_len=(40,), chunk_prefix=(3000,),
                                  decode_ctx=(3000, 1500, 3)),
}


def gemm_plan_workload(case):
    """Full-size token counts whose GEMM tile / K-split plans the named
    configurations do not reach (see the test that uses them)."""
    dims, cl, cp, n_dec = {
        "yi_T512": (W.YI, [448], [1000], 64),
        "mistral_T2048": (W.MISTRAL, [2000], [300], 48),
        "mistral_T200": (W.MISTRAL, [184], [700], 16),
        "mistral_T700": (W.MISTRAL, [660], [900], 40),
        "yi_T256": (W.YI, [224], [800], 32),
        "mistral_T1000": (W.MISTRAL, [960], [500], 40),
    }[case]
    rng = np.random.default_rng(11)
    ctx = rng.integers(1, 1500, size=n_dec).astype(np.int32)
    return W.build_workload(case, dims, cl, cp, ctx, 3)


# Cases whose max-abs bar (and, with FP8 projections, rel-L2 bar) is derived
# from the oracle's own conditioning floor because the literal bar lies below
# it.  name -> (workload builder, random rows sampled at full size or None for
# every row, relative input perturbation of the floor, derive the rel-L2 bar
# too).  eps 1e-7: an fp32-level difference; FP8_MFMA_REL_ERR: the FP8 MFMA's
# summation error.
FP8_MFMA_REL_ERR = 2.0 ** -13
DERIVED_BAR_CASES = {
    "yi_tau2048": (lambda: W.yi_tau2048(0), 24, 1e-7, False),
    "yi_tau2048_tp2": (lambda: W.yi_tau2048_tp2(0), 16, 1e-7, False),
    "yi_T512": (lambda: gemm_plan_workload("yi_T512"), 16, 1e-7, False),
    "yi_T256": (lambda: gemm_plan_workload("yi_T256"), 16, 1e-7, False),
    "mistral_tau512_w8a8": (lambda: W.with_w8a8(W.mistral_tau512(0)), 48, FP8_MFMA_REL_ERR, True),
    "mistral_T2048_w8a8": (lambda: W.with_w8a8(gemm_plan_workload("mistral_T2048")), 16, FP8_MFMA_REL_ERR, True),
    "yi_T512_w8a8": (lambda: W.with_w8a8(gemm_plan_workload("yi_T512")), 16, FP8_MFMA_REL_ERR, True),
    "small_g7_d128_w8a8": (lambda: W.with_w8a8(W.small(2, **SMALL["g7_d128"])), None, FP8_MFMA_REL_ERR, True),
}
FLOOR_ROWS = 96          # the floor is measured on the first 96 of the sampled rows
FLOORS_JSON = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "conditioning_floors.json")


def rows_digest(rows) -> str:
    return hashlib.sha256(np.asarray(rows, dtype=np.int64).tobytes()).hexdigest()[:16]


def derived_bars(name, rows):
    """Bars of a DERIVED_BAR_CASES case from the stored floors
    (tests/golden/conditioning_floors.json, written by
    tests/golden/make_conditioning_floors.py from the oracle alone): twice the
    floor where that exceeds the literal bar.  ``rows``: the rows the test
    compares (checked against the rows the floor was measured on)."""
    with open(FLOORS_JSON) as f:
        rec = json.load(f)[name]
    floor_rows = rows if rows is None else np.asarray(rows)[:FLOOR_ROWS]
    want = "all" if floor_rows is None else rows_digest(floor_rows)
    assert rec["rows"] == want, f"{name}: rows differ from those the stored floor was measured on"
    bars = dict(max_abs=max(TOL_MAX_ABS, 2.0 * rec["floor_max_abs"]), rel_l2=TOL_REL_L2)
    if DERIVED_BAR_CASES[name][3]:
        bars["rel_l2"] = max(TOL_REL_L2, 2.0 * rec["floor_rel_l2"])
    log(f"{name}: stored oracle floor (input perturbation {rec['eps']:.1e}) rel_l2={rec['floor_rel_l2']:.3e} "
        f"max_abs={rec['floor_max_abs']:.3e}; bars {bars['rel_l2']:.3e} / {bars['max_abs']:.3e}"
        + ("" if bars["max_abs"] == TOL_MAX_ABS else f" (literal max-abs {TOL_MAX_ABS} is below twice the floor)"))
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


# fraction of values (bf16 bits or e4m3 codes) the GPU must store identically
# to the oracle at each storage point: the normed input is computed from the
# same x on both sides, q from identical xn by an fp32 product; the attention
# output differs by its bf16 probabilities, and what follows inherits that
STORED_MIN_IDENTICAL = {"xn": 0.99, "q": 0.9, "o": 0.5, "h1n": 0.5, "act": 0.3}


def compare_stored(gpu, ref, dims, what, max_rel=5e-2):
    """The activations the layer stores between its steps (DeviceLayer.stored)
    against the oracle's (LayerResult.stored), every row: the normed input xn,
    the rotated q, the attention output o, the residual h1 (fp32), the normed
    residual h1n and the SwiGLU output.  bf16 values are compared as bits;
    with FP8 projections xn, o, h1n and the SwiGLU output are compared as
    e4m3 codes, the oracle's being the code of its stored value over that
    input's own scale -- so a scale used at the wrong storage point makes
    nearly every code differ.  Upstream differences of one rounding step
    cascade through later points, so later points agree less often; the
    bounds are on the fraction of identical values and on the relative L2
    distance of the values (h1, an fp32 sum, on its relative distance alone)."""
    f8 = bool(getattr(dims, "w8a8", 0))
    scales = {"xn": dims.x_scale, "o": dims.o_scale, "h1n": dims.h_scale, "act": dims.a_scale}
    res = {}
    for gname, oname in (("xn", "xn"), ("q", "q"), ("o", "o"), ("h1", "h1"), ("h1n", "h1n"), ("act", "a")):
        g = gpu[gname]
        e = np.asarray(ref[oname], dtype=np.float64).reshape(g.shape)
        if gname == "h1":
            gv = g.astype(np.float64)
            rel = float(np.linalg.norm(gv - e) / max(np.linalg.norm(e), 1e-30))
            log(f"{what} stored h1 (fp32): rel_l2 {rel:.2e}")
            assert np.all(np.isfinite(gv)) and rel <= max_rel, (what, gname, rel)
            res[gname] = (None, rel)
            continue
        elif f8 and gname in scales:
            sc = np.float64(np.float32(scales[gname]))
            same = g == O.e4m3_encode(e / sc)        # e is a code value times the scale, exactly
            gv = O.e4m3_decode(g) * sc
        else:
            gv = O.bf16_bits_to_float(g)
            same = g == O.bf16_bits(e)
        assert np.all(np.isfinite(gv)), f"{what} stored {gname}: non-finite value"
        rel = float(np.linalg.norm(gv - e) / max(np.linalg.norm(e), 1e-30))
        ident = float(np.mean(same))
        res[gname] = (ident, rel)
        log(f"{what} stored {gname}{' (e4m3 codes)' if f8 and gname in scales else ''}: "
            f"{ident * 100:.2f}% identical, rel_l2 {rel:.2e}")
        assert ident >= STORED_MIN_IDENTICAL[gname] and rel <= max_rel, (what, gname, ident, rel)
    return res


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


def w8a8_kv_extra_bound(wl, stored, gpu_stored):
    """Per-element error allowance of the new K and V rows with FP8
    projections, [T][n_kv][d] each, from two sources:
      * the FP8 MFMA sums its products to about 16 significant bits (worst
        measured 2^-13 of the sum of |products| per instruction), so a K or V
        value may move by up to that fraction of sum_i |xn_i w_i| -- more than
        one bf16 step where the sum cancels: twice 2^-13 of |xn| . |W|^T;
      * the projection's input itself: an xn code the GPU's fp32 norm put one
        e4m3 step from the oracle's (a value at a code boundary) moves the
        output by that step times the weight: |xn_gpu - xn| . |W|^T, with
        xn_gpu the codes the GPU stored (DeviceLayer.stored).
    For K the two dims a rotary pair mixes are added."""
    d = wl.dims
    w = O.weights_to_float(wl.weights)
    xn = stored["xn_all"]
    xg = O.e4m3_decode(gpu_stored["xn"]) * np.float64(np.float32(d.x_scale))
    dx = np.abs(xg - xn)
    xa = np.abs(xn)
    T, D, nkv = xa.shape[0], d.head_dim, d.n_kv_heads
    wk, wv = np.abs(w["w_k"]).T, np.abs(w["w_v"]).T
    bk = ((2.0 * FP8_MFMA_REL_ERR) * (xa @ wk) + dx @ wk).reshape(T, nkv, D)
    bv = ((2.0 * FP8_MFMA_REL_ERR) * (xa @ wv) + dx @ wv).reshape(T, nkv, D)
    half = D // 2
    pair = bk[..., :half] + bk[..., half:]
    bk = np.concatenate([pair, pair], axis=-1)
    return bk, bv


def new_values_close(g_bits, e_vals, what, min_identical=0.99, extra=None):
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
    if extra is not None:
        bound = bound + extra
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


def compare_cache(gpu_kv, cache, num_pages, written_pages_slots=None, what="cache", min_identical=0.99,
                  extra_kv=None):
    """Bit-exact everywhere the batch did not write (prefixes, NaN decoys and
    tails).  At the batch's new slots: bit-exact if ``written_pages_slots`` is
    None (a pure copy), else ``new_values_close`` (bf16) or ``new_codes_close``
    (FP8 codes).  extra_kv: per-token allowances ([T][n_kv][d] for K and V,
    tokens in the order of written_pages_slots) added to the bf16 bound."""
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
    for idx, (name, g, e, dense) in enumerate((("K", gk, ek, dk), ("V", gv, ev, dv))):
        diff = g != e
        if written_pages_slots is None:
            assert not diff.any(), f"{what} {name}: {int(diff.sum())} elements differ"
            continue
        mask = np.zeros(g.shape, dtype=bool)
        extra = None if extra_kv is None else np.zeros(g.shape)
        for t, (page, slot) in enumerate(written_pages_slots):
            mask[page, :, slot, :] = True
            if extra is not None:
                extra[page, :, slot, :] = extra_kv[idx][t]
        assert not (diff & ~mask).any(), f"{what} {name}: bytes outside the new slots changed"
        if extra is None:
            close(g[mask], dense[mask], f"{what} {name}", min_identical)
        else:
            close(g[mask], dense[mask], f"{what} {name}", min_identical, extra=extra[mask])
