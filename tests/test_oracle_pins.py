"""Pins for the oracle: each check ties an oracle function to something other
than itself -- a value the pages print, a closed form, an invariant the pages
state, a special case with a known answer, an independent library routine, or
brute force on tiny inputs.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import hybrid_layer as O
from chunked_prefill_hybrid_layer_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 3,
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 65504, 1e-40, 3e38], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_single_step_closed_forms():
    # ties go to the even significand
    assert O.round_bf16(np.array([1 + 2**-8]))[0] == 1.0
    assert O.round_bf16(np.array([1 + 3 * 2**-8]))[0] == 1 + 2**-6
    # a value just above a tie rounds up; going through float32 first would lose that
    assert O.round_bf16(np.array([1 + 2**-8 + 2**-40]))[0] == 1 + 2**-7
    assert O.round_bf16(np.array([-2.0**-130]))[0] == -2.0**-130  # subnormal grid 2^-133
    assert O.round_bf16(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------- batch layout

def test_worked_example_token_accounting():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_yi34b.json")))
    e = g["expected"]
    ra, rb = g["R_A"], g["R_B"]
    left, total = O.hybrid_batch_budget(g["n_decodes"], [ra["chunk"], rb["chunk"]], g["tau"])
    assert left == [e["budget_after_decodes"], e["budget_after_R_A"], e["budget_after_R_B"]]
    assert total == e["total_tokens"]
    assert ra["prompt_len"] - ra["cached_before"] == e["R_A_prefill_remaining_before"]
    ctx = [100, 250, 3000, 17, 64, 999]
    lay = O.token_layout([ra["chunk"], rb["chunk"]], [ra["cached_before"], rb["cached_before"]], ctx)
    assert len(lay.seq) == e["total_tokens"]
    assert lay.kv_len[0] == e["R_A_kv_len_after"]
    assert lay.kv_len[1] == e["R_B_kv_len_after"]
    assert ra["prompt_len"] - lay.kv_len[0] == e["R_A_remaining_prefill_after"]
    assert e["R_A_remaining_prefill_after"] - g["chunk_size"] == e["R_A_tail_after_next_chunk"]
    assert list(lay.q_start) == [0, 1024, 1824, 1825, 1826, 1827, 1828, 1829, 1830]
    with pytest.raises(ValueError):
        O.hybrid_batch_budget(g["n_decodes"], [ra["chunk"], rb["chunk"]], e["total_tokens"] - 1)


def test_chunk_i_covers_its_prompt_slice():
    # chunk i (1-based) of size C covers positions [(i-1)C, iC)
    C = 64
    for i in range(1, 5):
        lay = O.token_layout([C], [(i - 1) * C], [])
        assert list(lay.pos) == list(range((i - 1) * C, i * C))
    lay = O.token_layout([3], [5], [0, 7])
    assert list(lay.pos) == [5, 6, 7, 0, 7]
    assert list(lay.seq) == [0, 0, 0, 1, 2]
    assert list(lay.kv_len) == [8, 1, 8]


def test_page_of_follows_block_table():
    bt = np.array([[7, 2, 9], [4, 0, -1]])
    assert O.page_of(bt, 0, 0, 16) == (7, 0)
    assert O.page_of(bt, 0, 17, 16) == (2, 1)
    assert O.page_of(bt, 0, 47, 16) == (9, 15)
    assert O.page_of(bt, 1, 16, 16) == (0, 0)


# ---------------------------------------------------------------- small pieces

def test_rmsnorm_closed_forms():
    eps = 1e-5
    gain = np.array([1.0, 2.0, 0.5, -1.0])
    c = 3.0
    got = O.rmsnorm(np.full((1, 4), c), gain, eps)
    assert np.allclose(got, c / math.sqrt(c * c + eps) * gain, rtol=1e-15, atol=0)
    got = O.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), eps)
    assert np.allclose(got, np.array([[3.0, 4.0]]) / math.sqrt(12.5 + eps), rtol=1e-15, atol=0)


def test_rope_closed_forms():
    theta = 10000.0
    u = np.array([[[0.3, -1.7]]])                     # d = 2: one pair, frequency 1
    for p in (0, 1, 5, 1000):
        got = O.rope(u, np.array([p]), theta)[0, 0]
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(got, [0.3 * c + 1.7 * s, -1.7 * c + 0.3 * s], rtol=0, atol=1e-14)
    # d = 4: pairs (0, 2) at frequency 1 and (1, 3) at theta^(-1/2); rotate-half pairing
    u = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    p = 7
    got = O.rope(u, np.array([p]), theta)[0, 0]
    a0, a1 = p * 1.0, p * theta ** -0.5
    exp = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
           3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    assert np.allclose(got, exp, rtol=0, atol=1e-13)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    assert np.array_equal(O.rope(q, np.array([0]), 1e4), q)       # position 0 is identity
    r = O.rope(q, np.array([123]), 1e4)
    assert np.allclose(r[..., :32] ** 2 + r[..., 32:] ** 2, q[..., :32] ** 2 + q[..., 32:] ** 2,
                       rtol=1e-12)
    # <R(m) q, R(n) k> depends on m - n only
    def dot(m, n):
        return float(np.sum(O.rope(q, np.array([m]), 1e4) * O.rope(k, np.array([n]), 1e4)))
    for (m, n, dlt) in [(10, 3, 40), (0, 17, 1000), (500, 499, 7)]:
        assert math.isclose(dot(m, n), dot(m + dlt, n + dlt), rel_tol=1e-9, abs_tol=1e-9)


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert math.isclose(s[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(s[2], -1 / (1 + math.e), rel_tol=1e-15)
    assert math.isclose(s[3], 40.0, rel_tol=1e-15)
    assert abs(s[4]) < 1e-15


def test_linear_against_brute_force_loops_and_flop_count():
    rng = np.random.default_rng(3)
    n, d_in, d_out = 3, 5, 4
    x = rng.standard_normal((n, d_in))
    w = rng.standard_normal((d_out, d_in))
    y, flops = O.linear(x, w)
    ops = 0
    ref = [[0.0] * d_out for _ in range(n)]
    for i in range(n):
        for j in range(d_out):
            acc = 0.0
            for kk in range(d_in):
                acc += x[i][kk] * w[j][kk]
                ops += 2
            ref[i][j] = acc
    assert np.allclose(y, np.array(ref), rtol=1e-14, atol=1e-14)
    assert flops == ops == 2 * n * d_in * d_out
    # one-hot rows pick out weight columns
    eye = np.eye(d_in)
    assert np.array_equal(O.linear(eye, w)[0], w.T)


# ---------------------------------------------------------------- attention

def _cache_with(keys, vals, page_size=4, n_pages=None, seed=0):
    """Put one sequence's K/V (positions 0..L-1) on shuffled pages."""
    L, nkv, d = keys.shape
    need = (L + page_size - 1) // page_size
    n_pages = n_pages or need + 3
    rng = np.random.default_rng(seed)
    pages = rng.permutation(n_pages)[:need]
    bt = np.full((1, need), -1, dtype=np.int64)
    bt[0] = pages
    cache = O.PagedCache(n_pages, nkv, page_size, d)
    cache.load_prefix(bt, 0, keys, vals)
    return cache, bt


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(4)
    L, d = 6, 4
    keys = rng.standard_normal((L, 1, d))
    vals = rng.standard_normal((L, 1, d))
    cache, bt = _cache_with(keys, vals)
    q = rng.standard_normal((3, 1, d))
    pos = np.array([5, 2, 0])
    o, pairs = O.paged_attention(q, np.zeros(3, int), pos, cache, bt, 1)
    assert pairs == 6 + 3 + 1
    for i in range(3):
        w = [math.exp(sum(q[i, 0, c] * keys[j, 0, c] for c in range(d)) / math.sqrt(d))
             for j in range(pos[i] + 1)]
        tot = sum(w)
        for c in range(d):
            ref = sum(w[j] * vals[j, 0, c] for j in range(pos[i] + 1)) / tot
            assert math.isclose(o[i, 0, c], ref, rel_tol=1e-12, abs_tol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    d = 8
    keys = rng.standard_normal((9, 1, d))
    vals = rng.standard_normal((9, 1, d))
    cache, bt = _cache_with(keys, vals)
    # a token at position 0 sees only itself: o = v_0 exactly
    o, _ = O.paged_attention(rng.standard_normal((1, 1, d)), [0], [0], cache, bt, 1)
    assert np.array_equal(o[0, 0], vals[0, 0])
    # q = 0: equal weights, o = mean of the visible values
    o, _ = O.paged_attention(np.zeros((1, 1, d)), [0], [8], cache, bt, 1)
    assert np.allclose(o[0, 0], vals[:9, 0].mean(axis=0), rtol=1e-13, atol=1e-14)
    # identical value rows: o equals that row
    same = np.repeat(vals[:1], 9, axis=0)
    c2, bt2 = _cache_with(keys, same)
    o, _ = O.paged_attention(rng.standard_normal((1, 1, d)) * 3, [0], [8], c2, bt2, 1)
    assert np.allclose(o[0, 0], same[0, 0], rtol=1e-14, atol=1e-15)
    # huge logits stay finite; a key ahead by > 800 in score takes all the weight
    kq = np.zeros((9, 1, d)); kq[3, 0, 0] = 1.0
    c3, bt3 = _cache_with(kq, vals)
    qq = np.zeros((1, 1, d)); qq[0, 0, 0] = 5000.0
    o, _ = O.paged_attention(qq, [0], [8], c3, bt3, 1)
    assert np.array_equal(o[0, 0], vals[3, 0])


def test_attention_gqa_equals_duplicated_kv_heads():
    rng = np.random.default_rng(6)
    d, L = 8, 11
    keys = rng.standard_normal((L, 2, d))
    vals = rng.standard_normal((L, 2, d))
    c_g, bt = _cache_with(keys, vals)
    c_f, bt_f = _cache_with(np.repeat(keys, 3, axis=1), np.repeat(vals, 3, axis=1))
    q = rng.standard_normal((2, 6, d))
    pos = np.array([10, 4])
    o_g, _ = O.paged_attention(q, [0, 0], pos, c_g, bt, 2)      # g = 3
    o_f, _ = O.paged_attention(q, [0, 0], pos, c_f, bt_f, 6)    # g = 1
    assert np.array_equal(o_g, o_f)


def test_attention_page_permutation_invariant():
    rng = np.random.default_rng(7)
    keys = rng.standard_normal((37, 2, 8))
    vals = rng.standard_normal((37, 2, 8))
    q = rng.standard_normal((5, 4, 8))
    pos = np.array([36, 0, 15, 16, 20])
    outs = []
    for seed in range(3):
        c, bt = _cache_with(keys, vals, n_pages=20, seed=seed)
        outs.append(O.paged_attention(q, np.zeros(5, int), pos, c, bt, 2)[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# ---------------------------------------------------------------- the layer

def _tiny_float(seed=0, **kw):
    wl = W.build_workload("t", W.Dims(64, 4, 2, 16, 96), [1], [0], [], seed, x_std=1.0, **kw)
    return wl, O.weights_to_float(wl.weights)


def _prompt_run(dims, w, x, chunks, storage, bt, num_pages):
    """Run one prompt through the layer as consecutive chunks of the given sizes."""
    cache = O.PagedCache(num_pages, dims.n_kv_heads, dims.page_size, dims.head_dim)
    ys, pairs, start = [], 0, 0
    for c in chunks:
        r = O.layer_forward(dims, w, x[start:start + c], [c], [start], [], bt, cache, storage)
        ys.append(r.y)
        pairs += r.pairs
        start += c
    return np.concatenate(ys), cache, pairs


@pytest.mark.parametrize("storage", ["bf16", "exact"])
def test_chunked_prefill_equals_unchunked(storage):
    """Running a prompt as N chunks equals one unchunked prefill ([notes] §3.1,
    §7.5b): same outputs, same cache, same (query, key) work L(L+1)/2."""
    dims = W.TINY
    wl = W.tiny(0)
    w = O.weights_to_float(wl.weights)
    L = 256
    rng = np.random.default_rng(8)
    x = O.bf16_bits_to_float(W.f32_to_bf16_bits(rng.standard_normal((L, dims.hidden)).astype(np.float32)))
    bt, num_pages = W.deal_block_tables(np.array([L]), dims.page_size, np.random.default_rng(9))
    ref_y, ref_cache, ref_pairs = _prompt_run(dims, w, x, [L], storage, bt, num_pages)
    assert ref_pairs == L * (L + 1) // 2
    for chunks in ([64] * 4, [50, 78, 128], [1] * 5 + [251], [200, 56]):
        y, cache, pairs = _prompt_run(dims, w, x, chunks, storage, bt, num_pages)
        assert pairs == L * (L + 1) // 2
        assert np.array_equal(y, ref_y), chunks
        ck, cv = cache.dense()
        rk, rv = ref_cache.dense()
        assert np.array_equal(ck, rk, equal_nan=True)
        assert np.array_equal(cv, rv, equal_nan=True)


def test_chunk_pair_count_closed_form():
    """Chunk k of size C attends (k-1)C^2 + C(C+1)/2 pairs ([notes] §7.5b)."""
    dims = W.Dims(32, 2, 1, 16, 32)
    wl = W.build_workload("p", dims, [1], [0], [], 0)
    w = O.weights_to_float(wl.weights)
    C, K = 8, 5
    x = np.random.default_rng(0).standard_normal((C * K, 32))
    bt, npg = W.deal_block_tables(np.array([C * K]), 16, np.random.default_rng(1))
    cache = O.PagedCache(npg, 1, 16, 16)
    for k in range(1, K + 1):
        r = O.layer_forward(dims, w, x[(k - 1) * C:k * C], [C], [(k - 1) * C], [], bt, cache)
        assert r.pairs == (k - 1) * C * C + C * (C + 1) // 2


def test_decode_equals_last_row_of_prefill():
    dims = W.Dims(64, 4, 2, 16, 96)
    wl = W.build_workload("d", dims, [1], [0], [], 0)
    w = O.weights_to_float(wl.weights)
    n = 21
    x = np.random.default_rng(1).standard_normal((n, 64))
    bt, npg = W.deal_block_tables(np.array([n]), 16, np.random.default_rng(2))
    full, _, _ = _prompt_run(dims, w, x, [n], "bf16", bt, npg)
    cache = O.PagedCache(npg, 2, 16, 16)
    O.layer_forward(dims, w, x[:n - 1], [n - 1], [0], [], bt, cache)
    r = O.layer_forward(dims, w, x[n - 1:], [], [], [n - 1], bt, cache)
    assert np.array_equal(r.y[0], full[n - 1])


def test_layer_linear_flops_are_2_T_psi():
    """The batch's linear work is 2 * T * Psi with Psi the layer's projection
    parameter count (every token passes every matrix once; [notes] §1.6,
    [cp] hybrid-iteration roofline 2(c+b)Psi)."""
    wl = W.small(0, n_q=4, n_kv=2, head_dim=16, hidden=64, ffn=96, chunk_len=(9,), chunk_prefix=(3,),
                 decode_ctx=(5, 1))
    w = O.weights_to_float(wl.weights)
    psi = sum(wl.weights[k].size for k in ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d"))
    cache = O.PagedCache(wl.batch.num_pages, 2, 16, 16)
    for s, (k, v) in enumerate(zip(wl.prefix_k, wl.prefix_v)):
        cache.load_prefix(wl.batch.block_table, s, O.bf16_bits_to_float(k), O.bf16_bits_to_float(v))
    b = wl.batch
    r = O.layer_forward(wl.dims, w, wl.x, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, cache)
    assert r.linear_flops == 2 * b.n_tokens * psi


def test_layer_residual_paths():
    wl, w = _tiny_float()
    dims = wl.dims
    x = wl.x.astype(np.float64)
    for zero in (("w_o", "w_d"),):
        w0 = dict(w)
        for k in zero:
            w0[k] = np.zeros_like(w[k])
        cache = O.PagedCache(wl.batch.num_pages, 2, 16, 16)
        r = O.layer_forward(dims, w0, x, [1], [0], [], wl.batch.block_table, cache)
        assert np.array_equal(r.y, x)


def test_layer_composition_transparent_weights():
    """With W_q = W_k = 0 every visible key gets equal weight, so with identity
    W_v, W_o and W_d = 0 the layer returns x + (running mean of rmsnorm(x) over
    positions 0..p) -- checked with plain loops."""
    dims = W.Dims(hidden=8, n_q_heads=2, n_kv_heads=2, head_dim=4, ffn_dim=8)
    H = 8
    w = {"w_q": np.zeros((8, 8)), "w_k": np.zeros((8, 8)), "w_v": np.eye(8), "w_o": np.eye(8),
         "w_g": np.ones((8, 8)), "w_u": np.ones((8, 8)), "w_d": np.zeros((8, 8)),
         "g_attn": np.linspace(0.5, 1.5, 8), "g_ffn": np.ones(8)}
    rng = np.random.default_rng(11)
    x = rng.standard_normal((7, H))
    bt = np.array([[2, 0]])
    cache = O.PagedCache(3, 2, 16, 4)
    r = O.layer_forward(dims, w, x, [7], [0], [], bt, cache, storage="exact")
    xn = []
    for t in range(7):
        ms = sum(v * v for v in x[t]) / H
        xn.append([x[t][c] / math.sqrt(ms + dims.rms_eps) * w["g_attn"][c] for c in range(H)])
    for t in range(7):
        for c in range(H):
            mean = sum(xn[j][c] for j in range(t + 1)) / (t + 1)
            assert math.isclose(r.y[t][c], x[t][c] + mean, rel_tol=1e-12, abs_tol=1e-12)


def test_layer_writes_only_its_slots():
    wl = W.small(0, n_q=4, n_kv=2, head_dim=16, hidden=64, ffn=96, chunk_len=(9,), chunk_prefix=(3,),
                 decode_ctx=(5, 0))
    w = O.weights_to_float(wl.weights)
    b = wl.batch
    cache = O.PagedCache(b.num_pages, 2, 16, 16)
    for s, (k, v) in enumerate(zip(wl.prefix_k, wl.prefix_v)):
        cache.load_prefix(b.block_table, s, O.bf16_bits_to_float(k), O.bf16_bits_to_float(v))
    before_k = cache.dense()[0]
    O.layer_forward(wl.dims, w, wl.x, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, cache)
    after_k = cache.dense()[0]
    changed = ~((after_k == before_k) | (np.isnan(after_k) & np.isnan(before_k)))
    # new positions: chunk 3..11, decode0 5, decode1 0 -> 9 + 1 + 1 token slots, each n_kv*d values
    assert changed.sum() == 11 * 2 * 16
    # every written value is on the bf16 grid and finite
    assert np.all(np.isfinite(after_k[changed]))
    assert np.array_equal(O.round_bf16(after_k[changed]), after_k[changed])


def test_layer_ffn_composition():
    """With W_v = 0 the attention output is 0, so h1 = x; with W_g = I,
    W_u = 2 I and W_d = I the layer returns x + silu(n) * 2 n, n = rmsnorm(x)
    -- checked with plain loops (gate goes through silu, up does not)."""
    H = 8
    dims = W.Dims(hidden=H, n_q_heads=2, n_kv_heads=1, head_dim=4, ffn_dim=H)
    rng = np.random.default_rng(12)
    w = {"w_q": rng.standard_normal((8, 8)), "w_k": rng.standard_normal((4, 8)), "w_v": np.zeros((4, 8)),
         "w_o": rng.standard_normal((8, 8)), "w_g": np.eye(H), "w_u": 2 * np.eye(H), "w_d": np.eye(H),
         "g_attn": np.ones(H), "g_ffn": np.linspace(0.8, 1.2, H)}
    x = rng.standard_normal((3, H))
    cache = O.PagedCache(2, 1, 16, 4)
    r = O.layer_forward(dims, w, x, [3], [0], [], np.array([[1]]), cache, storage="exact")
    for t in range(3):
        ms = sum(v * v for v in x[t]) / H
        for c in range(H):
            n = x[t][c] / math.sqrt(ms + dims.rms_eps) * w["g_ffn"][c]
            ref = x[t][c] + n / (1 + math.exp(-n)) * 2 * n
            assert math.isclose(r.y[t][c], ref, rel_tol=1e-12, abs_tol=1e-12)


def test_bf16_storage_points():
    wl = W.small(0, n_q=4, n_kv=2, head_dim=16, hidden=64, ffn=96, chunk_len=(9,), chunk_prefix=(0,),
                 decode_ctx=())
    w = O.weights_to_float(wl.weights)
    b = wl.batch
    cache = O.PagedCache(b.num_pages, 2, 16, 16)
    r = O.layer_forward(wl.dims, w, wl.x, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, cache,
                        keep_attn=True)
    assert np.array_equal(O.round_bf16(r.attn_out), r.attn_out)
    assert np.array_equal(O.round_f32(r.y), r.y)
    r2 = O.layer_forward(wl.dims, w, wl.x, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table,
                         O.PagedCache(b.num_pages, 2, 16, 16), storage="exact", keep_attn=True)
    assert not np.array_equal(O.round_bf16(r2.attn_out), r2.attn_out)
    # the two precisions agree to bf16 accuracy
    assert np.max(np.abs(r.y - r2.y)) < 0.05


def test_row_block_evaluation_is_bit_identical():
    """Large inputs of round_bf16 and rmsnorm are evaluated in row blocks on a
    thread pool; each element (row) sees the same arithmetic, so the result is
    bit-identical to the single-call evaluation."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6000, 1024)) * np.exp(rng.uniform(-30, 30, (6000, 1)))
    x[5, :7] = [0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38 * 1.001, 1e-45, np.nan]
    a = O.round_bf16(x)
    b = O._round_bf16(x)
    assert np.array_equal(a, b, equal_nan=True)
    g = rng.standard_normal(1024)
    assert np.array_equal(O.rmsnorm(x[6:], g, 1e-5), O._rmsnorm(x[6:], g, 1e-5))


# ---------------------------------------------------------------- FP8 e4m3 KV storage

def test_e4m3_code_points_from_the_format_definition():
    """OCP 8-bit floating point E4M3: sign, 4 exponent bits (bias 7), 3
    mantissa bits, subnormals below 2^-6, NaN at 0x7F, largest finite 448."""
    cases = {0.0: 0x00, 1.0: 0x38, -2.0: 0xC0, 448.0: 0x7E, 2.0 ** -6: 0x08, 2.0 ** -9: 0x01,
             0.5: 0x30, 1.125: 0x39, 240.0: 0x77, 256.0: 0x78, 3.25: 0x45, -0.875: 0xB6}
    for x, code in cases.items():
        assert int(O.e4m3_encode(x)) == code, (x, hex(int(O.e4m3_encode(x))))
        assert float(O.e4m3_decode(np.uint8(code))) == x
    assert int(O.e4m3_encode(-0.0)) == 0x80
    assert np.isnan(O.e4m3_decode(np.uint8(0x7F))) and np.isnan(O.e4m3_decode(np.uint8(0xFF)))


def test_e4m3_rounds_to_nearest_even_and_saturates():
    # midpoints go to the even code (the code's last bit is the mantissa's)
    ties = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
            7.5 * 2.0 ** -9: 0x08, 464.0: 0x7E, 2.5 * 2.0 ** -9: 0x02}
    for x, code in ties.items():
        assert int(O.e4m3_encode(x)) == code, (x, hex(int(O.e4m3_encode(x))))
    # just off a midpoint goes to the nearer code
    assert int(O.e4m3_encode(1.0625 + 1e-9)) == 0x39
    assert int(O.e4m3_encode(1.1875 - 1e-9)) == 0x39
    # beyond the largest finite magnitude: saturation, not NaN
    for x in (449.0, 480.0, 1e6, np.inf):
        assert int(O.e4m3_encode(x)) == 0x7E and int(O.e4m3_encode(-x)) == 0xFE


def test_e4m3_round_trip_and_monotonicity():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    assert np.all(O.e4m3_encode(vals) == np.where(vals == 0, codes, codes))   # -0 keeps its sign bit
    pos = O.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    # every value maps to a code whose value is within half a step of it
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 9, 20000)
    x = x[np.abs(x) <= 448]
    y = O.e4m3_decode(O.e4m3_encode(x))
    mag = np.abs(x)
    idx = np.clip(np.searchsorted(pos, mag), 1, 126)
    step = pos[idx] - pos[idx - 1]
    assert np.all(np.abs(y - x) <= step / 2 + 1e-300)


def test_fp8_cache_stores_quantised_values():
    c = O.PagedCache(4, 2, 16, 64, kv_fp8=1, k_scale=0.0625, v_scale=0.25)
    bt = np.array([[2, 0]], dtype=np.int32)
    k = np.linspace(-3, 3, 128).reshape(2, 64)
    v = np.linspace(-100, 100, 128).reshape(2, 64)
    c.write(bt, 0, 5, k, v)
    kk, vv = c.gather(bt, 0, 6)
    assert np.array_equal(kk[5], O.e4m3_decode(O.e4m3_encode(k / 0.0625)) * 0.0625)
    assert np.array_equal(vv[5], O.e4m3_decode(O.e4m3_encode(v / 0.25)) * 0.25)
    assert np.all(np.isnan(kk[:5])) and np.all(c.codes[2][:, :, :5, :] == 0x7F)
    # half an e4m3 step: |x / scale| <= 48 lies in binades up to [32, 64), step 4
    assert np.max(np.abs(kk[5] - k)) <= 0.0625 * 4 / 2


def test_fp8_quotient_is_single_precision():
    """Worked by hand.  Scale 0.03 as float32 is 0.029999999329447746; its
    reciprocal 33.33333407839... rounds to the float32 33.333335876464844
    (neighbours 33.333332061767578 and 33.333335876464844, 2^-18 apart).
    0.75 times that is 25 + 2^-19 exactly, a float32, just above the midpoint
    25 of the codes 24 (0x5C) and 26 (0x5D): code 0x5D.  The float64 quotient
    0.75 / 0.03 is exactly 25, which would tie to the even code 0x5C."""
    q = O.fp8_quotient(np.array([0.75, -0.75]), 0.03)
    assert q[0] == 25 + 2.0 ** -19 and q[1] == -q[0]
    assert list(O.e4m3_encode(q)) == [0x5D, 0xDD]
    assert int(O.e4m3_encode(0.75 / 0.03)) == 0x5C
    # a power-of-two scale divides exactly
    x = np.array([1.0625, -3.0, 2.0 ** -10, 1000.0])
    assert np.array_equal(O.fp8_quotient(x, 2.0 ** -4), x * 16)
    c = O.PagedCache(1, 1, 16, 32, kv_fp8=1, k_scale=0.03, v_scale=0.03)
    c.write(np.array([[0]], dtype=np.int32), 0, 0, np.full((1, 32), 0.75), np.full((1, 32), -0.75))
    assert np.all(c.codes[0][0] == np.where(np.arange(16)[:, None] == 0, 0x5D, 0x7F))
    assert np.all(c.pages[0][1, 0, 0] == -26 * np.float64(np.float32(0.03)))


# ---------------------------------------------------------------- FP8 projections (w8a8)

def test_fp8_weight_rows_take_their_own_scale():
    """Row n of a projection is codes[n] * scale[n] (one scale per output
    channel, taken as float32): worked by hand."""
    codes = np.full((3, 4), 0x38, dtype=np.uint8)    # 1.0
    codes[1, 2] = 0xC0                                 # -2.0
    codes[2, 0] = 0x01                                 # 2^-9 (smallest subnormal)
    w = O.fp8_weight(codes, [0.5, 2.0, 0.25])
    assert np.array_equal(w, [[0.5] * 4, [2.0, 2.0, -4.0, 2.0], [2.0 ** -11, 0.25, 0.25, 0.25]])
    assert O.fp8_weight(np.array([[0x38]], np.uint8), [0.1])[0, 0] == np.float64(np.float32(0.1))
    wts = O.weights_to_float({"w_o": codes, "s_w_o": np.array([0.5, 2.0, 0.25], np.float32),
                              "g_ffn": np.array([0x3F80], np.uint16)})
    assert set(wts) == {"w_o", "g_ffn"} and np.array_equal(wts["w_o"], w) and wts["g_ffn"][0] == 1.0


def test_fp8_store_reads_back_codes_times_scale():
    s = 2.0 ** -4
    # values that are codes * scale come back unchanged
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    v = O.e4m3_decode(codes) * s
    assert np.array_equal(O.fp8_store(v, s), v) and np.array_equal(O.fp8_store(-v, s), -v)
    # others: nearest code, within half a step (relative 2^-4 for normals)
    x = np.random.default_rng(3).standard_normal(10000)
    y = O.fp8_store(x, s)
    normal = np.abs(x) >= 2.0 ** -6 * s
    assert np.all(np.abs(y - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * 1.0000001)
    assert np.all(np.abs(y - x)[~normal] <= 2.0 ** -10 * s)
    # scale equivariance for a power-of-two factor, saturation at 448 * scale
    assert np.array_equal(O.fp8_store(4 * x, 4 * s), 4 * y)
    assert O.fp8_store(np.array([1e6, -1e6]), 0.01).tolist() == [448 * np.float64(np.float32(0.01)),
                                                                  -448 * np.float64(np.float32(0.01))]


def test_w8a8_layer_within_the_quantisation_error_of_the_exact_layer():
    """With FP8 weights, the w8a8 layer differs from the exact layer over the
    same (decoded) weights only by the e4m3 storage of the four projection
    inputs: a relative error of at most 2^-4 per stored value (about 2^-4 /
    sqrt(3) rms), so the layer's update y - x moves by a few percent, not by
    factors (a missing or misplaced scale) and not by zero (no quantisation)."""
    from chunked_prefill_hybrid_layer_amd import workloads as W
    wl = W.with_w8a8(W.small(2, n_q=4, n_kv=2, head_dim=64, chunk_len=(20,), chunk_prefix=(5,),
                             decode_ctx=(3, 17), hidden=128, ffn=256))
    b = wl.batch
    w = O.weights_to_float(wl.weights)
    def run(dims, storage):
        cache = O.PagedCache(b.num_pages, dims.n_kv_heads, dims.page_size, dims.head_dim)
        for s in range(b.n_seq):
            cache.load_prefix(b.block_table, s, O.bf16_bits_to_float(wl.prefix_k[s]),
                              O.bf16_bits_to_float(wl.prefix_v[s]))
        return O.layer_forward(dims, w, wl.x, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, cache,
                               storage=storage).y
    import dataclasses
    y8 = run(wl.dims, "exact")
    ye = run(dataclasses.replace(wl.dims, w8a8=0), "exact")
    d8, de = y8 - wl.x, ye - wl.x
    rel = np.linalg.norm(d8 - de) / np.linalg.norm(de)
    assert 1e-3 < rel < 0.1, rel


def test_w8a8_each_projection_input_takes_its_own_scale():
    """The four stored projection inputs are e4m3 codes times their own scale
    (x_scale for the normed input, o_scale for the attention output, h_scale
    for the normed residual, a_scale for the SwiGLU output), worked out from
    the format definition and the layer's formulas on the stored values: each
    lies on its own scale's grid and, with scales whose ratios are not powers
    of two, not on the others'; the normed input, the normed residual and the
    SwiGLU output equal their formulas quantised with their own scale."""
    from chunked_prefill_hybrid_layer_amd import workloads as W
    wl = W.with_w8a8(W.small(2, n_q=4, n_kv=2, head_dim=64, chunk_len=(20,), chunk_prefix=(5,),
                             decode_ctx=(3, 17), hidden=128, ffn=256))
    d, b = wl.dims, wl.batch
    scales = {"xn": d.x_scale, "o": d.o_scale, "h1n": d.h_scale, "a": d.a_scale}
    assert len({np.float32(s) for s in scales.values()}) == 4
    w = O.weights_to_float(wl.weights)
    cache = O.PagedCache(b.num_pages, d.n_kv_heads, d.page_size, d.head_dim)
    for s in range(b.n_seq):
        cache.load_prefix(b.block_table, s, O.bf16_bits_to_float(wl.prefix_k[s]), O.bf16_bits_to_float(wl.prefix_v[s]))
    st = O.layer_forward(d, w, wl.x, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, cache,
                         keep_stored=True).stored

    def on_grid(v, s):
        q = v / np.float64(np.float32(s))
        return O.e4m3_decode(O.e4m3_encode(q)) == q

    for name, s in scales.items():
        assert np.all(on_grid(st[name], s)), name
        for other, s2 in scales.items():
            if other != name:
                assert np.mean(on_grid(st[name], s2)) < 0.5, (name, other)

    def q8(v, s):   # e4m3 store of v with scale s: code of v * (1/s) in single precision, read back * s
        s32 = np.float32(s)
        code = O.e4m3_encode(np.asarray(v, np.float64).astype(np.float32) * (np.float32(1.0) / s32))
        return O.e4m3_decode(code) * np.float64(s32)

    x = wl.x.astype(np.float64)
    for t in (0, 7, x.shape[0] - 1):
        ms = sum(float(v) * float(v) for v in x[t]) / d.hidden
        ref = [x[t, c] / math.sqrt(ms + d.rms_eps) * w["g_attn"][c] for c in range(d.hidden)]
        assert np.array_equal(st["xn"][t], q8(ref, d.x_scale))
        h1 = st["h1"][t]
        ms = sum(float(v) * float(v) for v in h1) / d.hidden
        ref = [h1[c] / math.sqrt(ms + d.rms_eps) * w["g_ffn"][c] for c in range(d.hidden)]
        assert np.array_equal(st["h1n"][t], q8(ref, d.h_scale))
        hn = st["h1n"][t]
        ref = []
        for f in range(d.ffn_dim):
            gt = sum(hn[c] * w["w_g"][f, c] for c in range(d.hidden))
            up = sum(hn[c] * w["w_u"][f, c] for c in range(d.hidden))
            ref.append(gt / (1.0 + math.exp(-gt)) * up)
        got, exp = st["a"][t], q8(ref, d.a_scale)
        # the plain loops sum in another order than the matrix product: a value
        # within rounding of a code midpoint may land one code away
        assert np.mean(got == exp) > 0.99
        assert np.all(np.abs(got - exp) <= np.abs(exp) * 2.0 ** -3 + 2.0 ** -9 * d.a_scale)
