"""Long-prompt chunking on the GPU at full size (Mistral-7B-shaped layer): a
32768-token prompt run as 64 chunks of 512, each co-batched with 64 decodes
(the batches composed by the stall-free scheduler, hb_schedule_iteration),
against the same prompt as one unchunked prefill.  Chunked prefill computes
exactly what the unchunked prefill computes ("Chunked Prefill", mechanism;
"Sarathi-Serve reading notes" §3.1), so the prompt rows of both runs agree
with each other and with the oracle, which evaluates sampled rows exactly
(K/V for all 32768 tokens, then attention and FFN for the sample).  The
prompt also runs alone as chunks of 128 and of 2048 tokens (the chunk-size
sweep's extremes), against the same oracle rows.  Decode rows of early,
middle and late iterations are checked against the oracle too: their
contexts hold K/V the layer wrote in earlier iterations, which the oracle
recomputes from those iterations' inputs (a token's K/V depend only on its
own input and position), so a decode at iteration i is the last row of a
prefill of its i + 1 generated tokens over its cached context."""
import numpy as np
import pytest
import torch

from oracle import hybrid_layer as O
from chunked_prefill_hybrid_layer_amd import workloads as W
from chunked_prefill_hybrid_layer_amd.runtime import DeviceLayer, schedule_batch
from tests.helpers import TOL_MAX_ABS, TOL_REL_L2, assert_close, errors, log

pytestmark = pytest.mark.gpu


DECODE_CHECK_ITERS = (1, 32, 63)
DECODE_CHECK_N = 8


def _run_chunked(lp, layer):
    """The iterations come from the stall-free scheduler (hb_schedule_iteration,
    token budget = chunk + decodes): the prompt is request 0, the decodes
    requests 1..n; each iteration's batch must be the configuration's.
    Returns the prompt rows and {iteration: decode rows [n_dec][H]} for the
    iterations in DECODE_CHECK_ITERS."""
    L, C = lp.prompt_len, lp.chunk
    prompt = np.concatenate([[L], lp.decode_ctx0])
    cached = np.concatenate([[0], lp.decode_ctx0]).astype(np.int64)
    y_prompt = np.empty((L, lp.dims.hidden), np.float32)
    y_dec = {}
    i = 0
    while cached[0] < L:
        cl, cp, dc, bt, order = schedule_batch(C + lp.n_dec, C, prompt, cached, lp.block_table, lp.num_pages)
        b = lp.batch(i)
        assert np.array_equal(cl, b.chunk_len) and np.array_equal(cp, b.chunk_prefix)
        assert np.array_equal(dc, b.decode_ctx) and np.array_equal(bt, b.block_table)
        prep = layer.prepare(cl, cp, dc, bt, C + lp.n_dec)
        x = torch.from_numpy(np.concatenate([lp.prompt_x[cp[0]:cp[0] + cl[0]],
                                             lp.decode_x[i][order[len(cl):] - 1]])).cuda()
        y = torch.empty_like(x)
        layer.forward(prep, x, y)
        y_prompt[cp[0]:cp[0] + cl[0]] = y[:cl[0]].cpu().numpy()
        if i in DECODE_CHECK_ITERS:
            yd = np.empty((lp.n_dec, lp.dims.hidden), np.float32)
            yd[order[len(cl):] - 1] = y[cl[0]:].cpu().numpy()
            y_dec[i] = yd
        cached[order[:len(cl)]] += cl
        cached[order[len(cl):]] += 1
        i += 1
    assert i == lp.n_iter
    torch.cuda.synchronize()
    return y_prompt, y_dec


def _run_prompt_alone(lp, layer, chunk):
    """The prompt alone as consecutive chunks of ``chunk`` tokens."""
    L = lp.prompt_len
    bt = np.ascontiguousarray(lp.block_table[:1])
    y_prompt = np.empty((L, lp.dims.hidden), np.float32)
    for p0 in range(0, L, chunk):
        prep = layer.prepare([chunk], [p0], [], bt, chunk)
        x = torch.from_numpy(lp.prompt_x[p0:p0 + chunk]).cuda()
        y = torch.empty_like(x)
        layer.forward(prep, x, y)
        y_prompt[p0:p0 + chunk] = y.cpu().numpy()
    torch.cuda.synchronize()
    return y_prompt


def _oracle_decode_rows(lp, w, it, decs):
    """Oracle output of decode j at iteration ``it``: the last row of a prefill
    of its it + 1 generated tokens (inputs of iterations 0..it, positions
    ctx0..ctx0+it) over its synthesized cached context."""
    d = lp.dims
    out = []
    for j in decs:
        bt = np.ascontiguousarray(lp.block_table[1 + j:2 + j])
        cache = O.PagedCache(lp.num_pages, d.n_kv_heads, d.page_size, d.head_dim)
        cache.load_prefix(bt, 0, O.bf16_bits_to_float(lp.prefix_k[1 + j]), O.bf16_bits_to_float(lp.prefix_v[1 + j]))
        x = lp.decode_x[:it + 1, j].astype(np.float64)
        r = O.layer_forward(d, w, x, [it + 1], [int(lp.decode_ctx0[j])], [], bt, cache, rows=[it])
        out.append(r.y[0])
    return np.stack(out)


def test_long_prompt_chunked_matches_unchunked_and_oracle():
    log("long prompt: generating the 32768-token workload")
    lp = W.long_prompt(0)
    d, L = lp.dims, lp.prompt_len
    max_pos = int(max(L, int(np.max(lp.decode_ctx0)) + lp.n_iter)) + 1
    log(f"long prompt: chunked run ({lp.n_iter} scheduled iterations of {lp.chunk} + {lp.n_dec} decodes)")
    l1 = DeviceLayer(d, lp.weights, lp.num_pages, max_pos)
    l1.fill_prefixes(lp.block_table, range(1, 1 + lp.n_dec), lp.prefix_k, lp.prefix_v)
    y_chunked, y_dec = _run_chunked(lp, l1)
    log("long prompt: unchunked run")
    l2 = DeviceLayer(d, lp.weights, lp.num_pages, max_pos)
    ub = lp.unchunked_batch()
    prep = l2.prepare(ub.chunk_len, ub.chunk_prefix, ub.decode_ctx, ub.block_table, ub.token_budget)
    x = torch.from_numpy(lp.prompt_x).cuda()
    y = torch.empty_like(x)
    l2.forward(prep, x, y)
    y_full = y.cpu().numpy()
    del x, y
    # Both runs approximate the same exact result with different summation
    # groupings (attention key splits of 1024 vs 16384 keys, GEMM plans for
    # 576 vs 32768 tokens), so they agree to the oracle tolerance.
    rel, mx = errors(y_chunked, y_full)
    log(f"long prompt: chunked vs unchunked over all {L} rows: rel_l2={rel:.3e} max_abs={mx:.3e}")
    for lo, hi in ((0, 1024), (L // 2 - 512, L // 2 + 512), (L - 1024, L)):
        r_, m_ = errors(y_chunked[lo:hi], y_full[lo:hi])
        log(f"long prompt:   rows [{lo}, {hi}): rel_l2={r_:.3e} max_abs={m_:.3e}")
    assert rel <= TOL_REL_L2 and mx <= TOL_MAX_ABS

    # prompt K/V in the two caches: equal up to the bf16 rounding of the projections
    k1, v1 = l1.cache_logical()
    k2, v2 = l2.cache_logical()
    pages = lp.block_table[0][:L // d.page_size]
    for name, a, b in (("K", k1[pages], k2[pages]), ("V", v1[pages], v2[pages])):
        diff = a != b
        frac = float(diff.mean())
        log(f"long prompt: prompt {name} cache, chunked vs unchunked: {frac * 100:.3f}% not bit-identical")
        assert frac <= 0.01
        fa, fb = O.bf16_bits_to_float(a[diff]), O.bf16_bits_to_float(b[diff])
        assert np.all(np.isfinite(fa)) and np.all(np.isfinite(fb))
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(fa), np.abs(fb)))[1] - 8)
        assert np.all(np.abs(fa - fb) <= ulp + 1e-3 * np.nanmax(np.abs(O.bf16_bits_to_float(a))))
    del k1, v1, k2, v2, l1, l2
    torch.cuda.empty_cache()

    y_alone = {}
    for c in (128, 2048):
        log(f"long prompt: the prompt alone as {L // c} chunks of {c}")
        lc = DeviceLayer(d, lp.weights, lp.num_pages, max_pos)
        y_alone[c] = _run_prompt_alone(lp, lc, c)
        del lc
        torch.cuda.empty_cache()

    rng = np.random.default_rng(4)
    spread = range(0, lp.n_iter, 9)
    rows = sorted(set([i * lp.chunk for i in spread] + [i * lp.chunk + lp.chunk - 1 for i in spread] +
                      [L - 1] + rng.choice(L, 8, replace=False).tolist()))
    log(f"long prompt: oracle on {len(rows)} sampled rows (K/V for all {L} tokens)")
    cache = O.PagedCache(lp.num_pages, d.n_kv_heads, d.page_size, d.head_dim)
    r = O.layer_forward(d, O.weights_to_float(lp.weights), lp.prompt_x.astype(np.float64), [L], [0], [],
                        np.ascontiguousarray(lp.block_table[:1]), cache, rows=rows)
    assert r.pairs == sum(p + 1 for p in rows)
    assert_close(y_full[rows], r.y, "unchunked vs oracle (sampled rows)")
    assert_close(y_chunked[rows], r.y, "chunked vs oracle (sampled rows)")
    for c, yc in y_alone.items():
        assert_close(yc[rows], r.y, f"prompt alone in chunks of {c} vs oracle (sampled rows)")

    w = O.weights_to_float(lp.weights)
    decs = np.random.default_rng(5).choice(lp.n_dec, DECODE_CHECK_N, replace=False)
    for it in DECODE_CHECK_ITERS:
        ref = _oracle_decode_rows(lp, w, it, decs)
        assert_close(y_dec[it][decs], ref, f"decode rows of iteration {it} vs oracle ({len(decs)} decodes)")
