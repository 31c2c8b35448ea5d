"""Host side of the C ABI (no GPU needed): the library loads and exports every
declared entry point; hb_pack_metadata agrees bit for bit with the oracle's
own token layout and page slots, rejects every invalid batch, and builds
attention work lists that partition each token's keys."""
import json
import os
import re

import numpy as np
import pytest

from oracle import hybrid_layer as O
from chunked_prefill_hybrid_layer_amd import workloads as W
from chunked_prefill_hybrid_layer_amd import hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "hb.h")).read()
    declared = sorted(set(re.findall(r"\b(hb_[a-z_]+)\s*\(", text)))
    assert declared == sorted(hb.EXPORTS)
    for name in declared:
        assert hasattr(hb.lib, name), name


def _pack(dims, cl, cp, dc, bt, num_pages, tau=None):
    tau = int(np.sum(cl)) + len(dc) if tau is None else tau
    return hb.pack_metadata(hb.make_dims(dims), cl, cp, dc, bt, num_pages, tau)


def _random_batch(rng, n_chunks, n_dec, max_len=300):
    cl = rng.integers(1, max_len, n_chunks)
    cp = rng.integers(0, max_len * 3, n_chunks)
    dc = rng.integers(0, max_len * 4, n_dec)
    kv = np.concatenate([cp + cl, dc + 1])
    bt, npg = W.deal_block_tables(kv, 16, rng, max_pages=int(((kv + 15) // 16).max()) + 3)
    return cl, cp, dc, bt, npg


@pytest.mark.parametrize("seed", range(6))
def test_pack_matches_oracle_layout_and_slots(seed):
    rng = np.random.default_rng(100 + seed)
    dims = [W.MISTRAL, W.YI, W.TINY][seed % 3]
    cl, cp, dc, bt, npg = _random_batch(rng, int(rng.integers(0, 4)), int(rng.integers(1, 40)))
    blob, T = _pack(dims, cl, cp, dc, bt, npg)
    lay = O.token_layout(cl, cp, dc)
    assert T == len(lay.seq)
    h = hb.header(blob)
    assert h.magic == hb.META_MAGIC and h.n_tokens == T and h.n_seq == len(cl) + len(dc)
    assert np.array_equal(hb.meta_array(blob, "q_start"), lay.q_start)
    assert np.array_equal(hb.meta_array(blob, "cached"), lay.cached)
    assert np.array_equal(hb.meta_array(blob, "kv_len"), lay.kv_len)
    assert np.array_equal(hb.meta_array(blob, "tok_seq"), lay.seq)
    assert np.array_equal(hb.meta_array(blob, "tok_pos"), lay.pos)
    slots = [O.page_of(bt, int(s), int(p), 16) for s, p in zip(lay.seq, lay.pos)]
    assert np.array_equal(hb.meta_array(blob, "slot"), [pg * 16 + sl for pg, sl in slots])
    assert np.array_equal(hb.meta_array(blob, "block_table").reshape(bt.shape), bt)
    assert h.max_kv_len == int(lay.kv_len.max())
    assert hb.meta_bytes(hb.make_dims(dims), h.n_seq, T, bt.shape[1]) >= h.bytes


@pytest.mark.parametrize("seed", range(6))
def test_attention_work_lists_partition_keys(seed):
    """Every token's attention items cover keys [0, pos+1) of its sequence
    exactly once, in split order, and its partial slots are contiguous."""
    rng = np.random.default_rng(200 + seed)
    dims = [W.MISTRAL, W.YI, W.TINY][seed % 3]
    cl, cp, dc, bt, npg = _random_batch(rng, int(rng.integers(1, 4)), int(rng.integers(0, 30)), max_len=2500)
    blob, T = _pack(dims, cl, cp, dc, bt, npg)
    lay = O.token_layout(cl, cp, dc)
    h = hb.header(blob)
    pos = hb.meta_array(blob, "tok_pos")
    poff = hb.meta_array(blob, "part_off")
    pcnt = hb.meta_array(blob, "part_cnt")
    covered = {t: [] for t in range(T)}
    for kind in ("chunk", "decode"):
        for seq, tok0, n_tok, k0, k1, split, n_split, _ in hb.attn_items(blob, kind):
            assert k0 < k1 and n_tok >= 1 and 0 <= split < n_split and k0 % 16 == 0
            g = dims.n_q_heads // dims.n_kv_heads
            if kind == "decode":   # decodes, and chunk pieces whose rows fit the 16-row decode tile
                assert n_tok == (1 if seq >= len(cl) else cl[seq]) and n_tok * g <= 16
            else:
                assert seq < len(cl) and cl[seq] * g > 16 and n_tok <= h.chunk_q_tile and k0 % 64 == 0
            for t in range(tok0, tok0 + n_tok):
                assert lay.seq[t] == seq and pcnt[t] == n_split
                covered[t].append((split, k0, k1))
    # partial slots only for tokens with more than one key range, contiguous in token order
    multi = pcnt > 1
    assert int(pcnt[multi].sum()) == h.n_partials and int(multi.sum()) == h.n_merge_tokens
    assert np.all(poff[~multi] == -1)
    assert np.array_equal(poff[multi], np.concatenate([[0], np.cumsum(pcnt[multi])[:-1]]).astype(np.int64))
    for t in range(T):
        c = sorted(covered[t])
        assert [s for s, _, _ in c] == list(range(pcnt[t]))
        assert c[0][1] == 0 and c[-1][2] >= pos[t] + 1
        for (_, _, a1), (_, b0, _) in zip(c, c[1:]):
            assert a1 == b0


@pytest.mark.parametrize("seed", range(4))
def test_append_runs_cover_each_token_once_within_a_page(seed):
    """The KV append runs list every packed token once, in order; a run stays
    inside one page and its slots are consecutive and equal the tokens' own
    slots."""
    rng = np.random.default_rng(300 + seed)
    cl, cp, dc, bt, npg = _random_batch(rng, int(rng.integers(0, 4)), int(rng.integers(1, 30)))
    blob, T = _pack(W.TINY, cl, cp, dc, bt, npg)
    runs = hb.append_runs(blob)
    slot = hb.meta_array(blob, "slot")
    assert runs[:, 0].tolist() == list(np.concatenate([[0], np.cumsum(runs[:, 1])[:-1]]))
    assert int(runs[:, 1].sum()) == T and np.all(runs[:, 1] >= 1) and np.all(runs[:, 3] == 0)
    for tok0, n, s0, _ in runs:
        assert s0 % 16 + n <= 16
        assert np.array_equal(slot[tok0:tok0 + n], s0 + np.arange(n))


def _expected_chunk_split(dims, cl, cp, slots=512, min_steps=4):
    """The rule for the keys per chunk item, restated: the smallest number of
    64-key tiles per item (at least min_steps) whose workgroups (items x kv
    heads) fit one round of `slots`; when none does, half a slot's share of
    the work (total tiles x kv heads / (2 slots))."""
    qt = 128 // (dims.n_q_heads // dims.n_kv_heads)
    steps = []
    for n, p in zip(cl, cp):
        for t0 in range(0, n, qt):
            steps.append(-(-(p + t0 + min(qt, n - t0)) // 64))
    wgs = lambda per: sum(-(-x // per) for x in steps) * dims.n_kv_heads
    if wgs(max(steps)) <= slots:
        per = next(p for p in range(min(min_steps, max(steps)), max(steps) + 1) if wgs(p) <= slots)
    else:
        per = max(min_steps, -(-sum(steps) * dims.n_kv_heads // (2 * slots)))
    return 64 * per, steps


@pytest.mark.parametrize("case", ["prompt_32768", "chunk_512_over_3000", "yi_tau2048_chunks", "small_chunk"])
def test_chunk_key_split_follows_the_workgroup_rule(case):
    """Chunk items: the keys per item follow the stated rule (one round of
    512 workgroups where a split fits it, else half a slot's share of the
    work); each tile's items are as equal as whole 64-key tiles allow and
    cover its keys once; tiles left whole have no partial result.  A
    32768-token prompt is unsplit (8192 workgroups already), so nothing is
    merged."""
    dims, cl, cp = {
        "prompt_32768": (W.MISTRAL, [32768], [0]),
        "chunk_512_over_3000": (W.MISTRAL, [512], [3000]),
        "yi_tau2048_chunks": (W.YI, [768, 768], [0, 6144]),
        "small_chunk": (W.MISTRAL, [64], [1792]),
    }[case]
    kv = np.array(cl) + np.array(cp)
    bt, npg = W.deal_block_tables(kv, 16, np.random.default_rng(2))
    blob, _ = _pack(dims, cl, cp, [], bt, npg)
    h = hb.header(blob)
    want, _ = _expected_chunk_split(dims, cl, cp)
    items = hb.attn_items(blob, "chunk")
    pos = hb.meta_array(blob, "tok_pos")
    pcnt = hb.meta_array(blob, "part_cnt")
    assert h.chunk_kv_split == min(want, 1 << 30)
    per = h.chunk_kv_split // 64
    for tok0 in np.unique(items[:, 1]):
        r = items[items[:, 1] == tok0]
        r = r[np.argsort(r[:, 5])]
        key_end = pos[tok0 + r[0, 2] - 1] + 1
        steps = (key_end + 63) // 64
        n = int(r[0, 6])
        assert len(r) == n == -(-steps // per)
        assert r[0, 3] == 0 and np.all(r[1:, 3] == r[:-1, 4]) and r[-1, 4] == key_end
        lens = (64 * np.ceil(r[:, 4] / 64) - r[:, 3]) // 64
        assert lens.max() - lens.min() <= 1 and lens.max() <= per
        assert np.all(pcnt[tok0:tok0 + r[0, 2]] == n)
    if case == "prompt_32768":
        assert h.n_partials == 0 and h.n_merge_tokens == 0 and np.all(items[:, 6] == 1)
        assert h.n_chunk_items == 32768 // h.chunk_q_tile
    if case == "chunk_512_over_3000":
        assert h.n_chunk_items * dims.n_kv_heads <= 512 and h.chunk_kv_split == 896


def test_large_decode_batch_widens_the_decode_key_split():
    """512 decodes of 1000-6000 context keys: the decode split grows past its
    256-key minimum (at most 1024, the page ids one decode wave can hold), the
    items still cover every decode's keys exactly once, and both item lists
    run longest key range first (chunk items in 256-key buckets).  32 decodes,
    whose 256-key items would spill just past one round of the machine (3072
    waves), take the smallest multiple of 32 keys that fits them in one."""
    rng = np.random.default_rng(7)
    dc = rng.integers(1000, 6000, 512)
    cl, cp = np.array([64]), np.array([100])
    kv = np.concatenate([cp + cl, dc + 1])
    bt, npg = W.deal_block_tables(kv, 16, rng)
    blob, T = _pack(W.YI, cl, cp, dc, bt, npg)
    h = hb.header(blob)
    assert 256 < h.decode_kv_split <= 1024
    assert h.n_decode_items * W.YI.n_kv_heads <= 16384 or h.decode_kv_split == 1024
    items = hb.attn_items(blob, "decode")
    pcnt = hb.meta_array(blob, "part_cnt")
    assert np.array_equal(pcnt[64:], (dc + 1 + h.decode_kv_split - 1) // h.decode_kv_split)
    assert np.array_equal(items[:, 6], pcnt[items[:, 1]])
    for kind in ("chunk", "decode"):
        r = hb.attn_items(blob, kind)
        ln = r[:, 4] - r[:, 3]
        if kind == "chunk":   # 256-key buckets, split-major within a bucket
            ln = ln // 256
        assert np.all(ln[:-1] >= ln[1:]), kind
    for t in range(64, T):
        r = items[items[:, 1] == t]
        r = r[np.argsort(r[:, 5])]
        assert r[0, 3] == 0 and np.all(r[1:, 3] == r[:-1, 4]) and r[-1, 4] == dc[t - 64] + 1
    small = dc[:32]
    kv2 = np.concatenate([cp + cl, small + 1])
    bt2, npg2 = W.deal_block_tables(kv2, 16, rng)
    blob2, _ = _pack(W.YI, cl, cp, small, bt2, npg2)
    h2 = hb.header(blob2)
    waves = lambda split: int(np.sum((small + 1 + split - 1) // split)) * W.YI.n_kv_heads
    assert waves(256) > 3072
    assert h2.decode_kv_split % 32 == 0 and waves(h2.decode_kv_split) <= 3072 < waves(h2.decode_kv_split - 32)
    assert h2.n_decode_items * W.YI.n_kv_heads == waves(h2.decode_kv_split)
    # 8 decodes fit one round at 256 keys and keep it
    blob3, _ = _pack(W.YI, cl, cp, small[:8], bt2, npg2)
    assert hb.header(blob3).decode_kv_split == 256


def test_worked_example_through_pack():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "worked_example_yi34b.json")))
    e = g["expected"]
    ra, rb = g["R_A"], g["R_B"]
    ctx = [100, 250, 3000, 17, 64, 999]
    cl, cp = [ra["chunk"], rb["chunk"]], [ra["cached_before"], rb["cached_before"]]
    kv = np.array([cp[0] + cl[0], cp[1] + cl[1]] + [c + 1 for c in ctx])
    bt, npg = W.deal_block_tables(kv, 16, np.random.default_rng(0))
    blob, T = _pack(W.YI, cl, cp, ctx, bt, npg, tau=g["tau"])
    assert T == e["total_tokens"]
    assert list(hb.meta_array(blob, "q_start")) == [0, 1024, 1824, 1825, 1826, 1827, 1828, 1829, 1830]
    kvl = hb.meta_array(blob, "kv_len")
    assert kvl[0] == e["R_A_kv_len_after"] and kvl[1] == e["R_B_kv_len_after"]
    with pytest.raises(hb.HbError) as ei:
        _pack(W.YI, cl, cp, ctx, bt, npg, tau=e["total_tokens"] - 1)
    assert ei.value.name == "HB_E_BUDGET"


def _err(fn):
    with pytest.raises(hb.HbError) as ei:
        fn()
    return ei.value.name


def test_pack_rejects_invalid_batches():
    d = W.TINY
    bt = np.array([[0, 1, -1], [2, -1, -1]], dtype=np.int32)
    ok = lambda **kw: _pack(d, kw.get("cl", [20]), kw.get("cp", [5]), kw.get("dc", [3]), kw.get("bt", bt),
                           kw.get("npg", 4), kw.get("tau"))
    ok()
    assert _err(lambda: ok(tau=20)) == "HB_E_BUDGET"
    assert _err(lambda: ok(cl=[0])) == "HB_E_LENGTH"
    assert _err(lambda: ok(cp=[-1])) == "HB_E_LENGTH"
    assert _err(lambda: ok(dc=[-2])) == "HB_E_LENGTH"
    assert _err(lambda: ok(npg=2)) == "HB_E_PAGE"                        # page 2 outside the pool
    assert _err(lambda: ok(bt=np.array([[0, -1, -1], [2, -1, -1]]))) == "HB_E_PAGE"   # needed entry is -1
    assert _err(lambda: ok(bt=np.array([[0, 1, -1], [1, -1, -1]]))) == "HB_E_ALIAS"
    assert _err(lambda: ok(cl=[40], bt=np.array([[0, 1], [2, -1]]))) == "HB_E_PAGE"  # 45 keys > 2 pages
    assert _err(lambda: ok(cl=[], cp=[], dc=[], bt=np.zeros((0, 3)))) == "HB_E_SHAPE"
    bad = W.Dims(256, 4, 4, 96, 512)
    assert _err(lambda: _pack(bad, [4], [0], [], np.array([[0]]), 1)) == "HB_E_SHAPE"
    bad = W.Dims(256, 6, 4, 64, 512)
    assert _err(lambda: _pack(bad, [4], [0], [], np.array([[0]]), 1)) == "HB_E_SHAPE"
    bad = W.Dims(256, 34, 2, 64, 512)   # group 17
    assert _err(lambda: _pack(bad, [4], [0], [], np.array([[0]]), 1)) == "HB_E_SHAPE"
    bad = W.Dims(16384 + 128, 4, 4, 64, 512)   # hidden above the row kernels' register budget
    assert _err(lambda: _pack(bad, [4], [0], [], np.array([[0]]), 1)) == "HB_E_SHAPE"
    # FP8 cache settings: kv_fp8 is 0 or 1, its scales finite and positive
    _pack(W.Dims(256, 4, 4, 64, 512, kv_fp8=1, k_scale=0.0625, v_scale=3.0), [4], [0], [], np.array([[0]]), 1)
    for kw in (dict(kv_fp8=2), dict(kv_fp8=1, k_scale=0.0), dict(kv_fp8=1, v_scale=-1.0),
               dict(kv_fp8=1, k_scale=float("nan")), dict(kv_fp8=1, v_scale=float("inf"))):
        bad = W.Dims(256, 4, 4, 64, 512, **kw)
        assert _err(lambda: _pack(bad, [4], [0], [], np.array([[0]]), 1)) == "HB_E_SHAPE", kw
    # FP8 projection settings: w8a8 is 0 or 1, its four input scales finite and positive
    _pack(W.Dims(256, 4, 4, 64, 512, w8a8=1, x_scale=0.5, o_scale=2.0, h_scale=0.1, a_scale=1.0), [4], [0], [],
          np.array([[0]]), 1)
    for kw in (dict(w8a8=3), dict(w8a8=1, x_scale=0.0), dict(w8a8=1, o_scale=-2.0), dict(w8a8=1, h_scale=float("nan")),
               dict(w8a8=1, a_scale=float("inf"))):
        bad = W.Dims(256, 4, 4, 64, 512, **kw)
        assert _err(lambda: _pack(bad, [4], [0], [], np.array([[0]]), 1)) == "HB_E_SHAPE", kw
    # a too-small buffer is reported, and nothing is written
    dims = hb.make_dims(d)
    with pytest.raises(hb.HbError) as ei:
        hb.pack_metadata(dims, [20], [5], [3], bt, 4, 100, capacity=64)
    assert ei.value.name == "HB_E_CAPACITY"


def test_rope_table_matches_oracle_angles():
    for dims in (W.TINY, W.MISTRAL):
        tab = hb.rope_table(hb.make_dims(dims), 5000)
        ang = O.rope_angles(np.arange(5000), dims.head_dim, dims.rope_theta)
        assert np.allclose(tab[..., 0], np.cos(ang), rtol=0, atol=1.2e-7)
        assert np.allclose(tab[..., 1], np.sin(ang), rtol=0, atol=1.2e-7)
        assert np.all(tab[0, :, 0] == 1.0) and np.all(tab[0, :, 1] == 0.0)


def test_workspace_size_covers_buffers():
    wl = W.mistral_tau512(0)
    b = wl.batch
    dims = hb.make_dims(wl.dims)
    blob, T = hb.pack_metadata(dims, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.num_pages,
                               b.token_budget)
    h = hb.header(blob)
    need = hb.workspace_bytes(dims, blob)
    d = wl.dims
    floor = T * (d.hidden * (2 + 4 + 2) + d.n_q_heads * d.head_dim * 4 + d.ffn_dim * 2) + \
        h.n_partials * d.n_q_heads * (d.head_dim + 2) * 4
    # plus fp32 split-K partials of at most 8 slices of the widest split projection
    split_max = 8 * T * max(d.qkv_dim, d.hidden) * 4
    assert floor <= need <= floor + split_max + 16 * 256


@pytest.mark.parametrize("w8a8", [0, 1])
def test_workspace_views_are_disjoint_regions_of_the_workspace(w8a8):
    """hb_workspace_views_of: the six stored activations sit in disjoint,
    16-byte aligned regions inside hb_workspace_bytes, each large enough for
    its [T][width] rows (one byte per element for the FP8 codes)."""
    import dataclasses
    wl = W.small(2, n_q=8, n_kv=2, head_dim=128)
    d = dataclasses.replace(wl.dims, w8a8=w8a8, **(W.FP8_ACT_SCALES if w8a8 else {}))
    b = wl.batch
    dims = hb.make_dims(d)
    blob, T = hb.pack_metadata(dims, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.num_pages,
                               b.token_budget)
    v = hb.workspace_views(dims, blob)
    need = hb.workspace_bytes(dims, blob)
    el = 1 if w8a8 else 2
    size = {"xn": d.hidden * el, "q": d.n_q_heads * d.head_dim * 2, "o": d.n_q_heads * d.head_dim * el,
            "h1": d.hidden * 4, "h1n": d.hidden * el, "act": d.ffn_dim * el}
    spans = sorted((v[n], v[n] + T * size[n], n) for n in size)
    for (a0, a1, n), (b0, _, m) in zip(spans, spans[1:]):
        assert a1 <= b0, (n, m)
    assert all(s0 % 16 == 0 and s1 <= need for s0, s1, _ in spans)
    with pytest.raises(hb.HbError):
        hb.workspace_views(dims, np.zeros(64, np.uint8))


def test_tampered_metadata_is_rejected():
    """The library reads the blob's arrays at the offsets its header names
    (the host the partial counts, the kernels all of them): a header whose
    counts or offsets do not fit the blob is refused with HB_E_META before
    anything reads it."""
    wl = W.small(2, n_q=8, n_kv=2, head_dim=128)
    b = wl.batch
    dims = hb.make_dims(wl.dims)
    blob, T = hb.pack_metadata(dims, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.num_pages,
                               b.token_budget)
    assert hb.workspace_bytes(dims, blob) > 0
    edits = [("n_decodes", T + 1), ("n_tokens", -1), ("n_seq", 0), ("off_part_cnt", None),
             ("off_block_table", -8), ("bytes", 64), ("n_decode_items", 1 << 30)]
    for field, value in edits:
        bad = blob.copy()
        h = hb.MetaHeader.from_buffer(bad)
        setattr(h, field, int(h.bytes) if value is None else value)
        with pytest.raises(hb.HbError, match="counts or array offsets"):
            hb.workspace_bytes(dims, bad)


def test_schedule_worked_example():
    """The worked Yi-34B iteration ("Sarathi-Serve reading notes" §7.6): tau
    2048, chunk 1024, six running decodes, R_A mid-prefill (4500-token prompt,
    1024 cached), R_B new (800 tokens).  The batch takes the 6 decodes, R_A's
    next 1024-token chunk and all of R_B: 1830 tokens; afterwards R_A has 2452
    prompt tokens left and R_B decodes."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "worked_example_yi34b.json")))
    e = g["expected"]
    ra, rb = g["R_A"], g["R_B"]
    ctx = [100, 250, 3000, 17, 64, 999]
    prompt = [ra["prompt_len"], rb["prompt_len"]] + ctx
    cached = [ra["cached_before"], rb["cached_before"]] + ctx
    cr, cl, cp, dr, dc = hb.schedule_iteration(g["tau"], g["chunk_size"], prompt, cached)
    assert list(dr) == [2, 3, 4, 5, 6, 7] and list(dc) == ctx
    assert list(cr) == [0, 1] and list(cl) == [ra["chunk"], rb["chunk"]] and list(cp) == cached[:2]
    assert int(cl.sum()) + len(dr) == e["total_tokens"]
    after = np.array(cached)
    after[cr] += cl
    after[dr] += 1
    assert prompt[0] - after[0] == e["R_A_remaining_prefill_after"] and after[1] == prompt[1]
    assert prompt[0] - cached[0] == e["R_A_prefill_remaining_before"]
    # the next iteration: R_B now decodes, R_A takes its next chunk
    cr2, cl2, _, dr2, _ = hb.schedule_iteration(g["tau"], g["chunk_size"], prompt, after)
    assert list(dr2) == [1, 2, 3, 4, 5, 6, 7] and list(cr2) == [0] and list(cl2) == [1024]


def test_schedule_reproduces_the_long_prompt_iterations():
    """Driving the 32768-token prompt and its 64 decodes through the
    scheduler (tau = 512 + 64, chunk 512) gives exactly the hand-built
    iterations: chunk i at prefix 512 i, every decode advancing by one."""
    lp = W.long_prompt(0, n_dec=64)
    prompt = np.concatenate([[lp.prompt_len], lp.decode_ctx0])
    cached = np.concatenate([[0], lp.decode_ctx0]).astype(np.int64)
    from chunked_prefill_hybrid_layer_amd.runtime import schedule_batch
    for i in range(lp.n_iter):
        cl, cp, dc, bt, order = schedule_batch(lp.chunk + lp.n_dec, lp.chunk, prompt, cached, lp.block_table,
                                               lp.num_pages)
        b = lp.batch(i)
        assert np.array_equal(cl, b.chunk_len) and np.array_equal(cp, b.chunk_prefix)
        assert np.array_equal(dc, b.decode_ctx) and np.array_equal(bt, b.block_table)
        cached[order[:len(cl)]] += cl
        cached[order[len(cl):]] += 1
    assert cached[0] == lp.prompt_len


def test_schedule_budget_edges_and_errors():
    # more decodes than the budget: the first tau decode in array order, no chunk
    cr, cl, cp, dr, dc = hb.schedule_iteration(3, 16, [5, 5, 5, 5, 100], [5, 6, 7, 8, 0])
    assert list(dr) == [0, 1, 2] and len(cr) == 0
    # the budget runs out inside the queue: the last chunk is cut, later requests wait
    cr, cl, cp, dr, dc = hb.schedule_iteration(100, 64, [300, 50, 70, 9], [10, 0, 0, 9])
    assert list(dr) == [3] and list(cr) == [0, 1] and list(cl) == [64, 35] and list(cp) == [10, 0]
    # a chunk never passes its prompt's end
    cr, cl, cp, dr, dc = hb.schedule_iteration(1000, 512, [700], [500])
    assert list(cl) == [200]
    # nothing to do
    cr, cl, cp, dr, dc = hb.schedule_iteration(8, 8, [], [])
    assert len(cr) == 0 and len(dr) == 0
    assert _err(lambda: hb.schedule_iteration(0, 8, [4], [0])) == "HB_E_SHAPE"
    assert _err(lambda: hb.schedule_iteration(8, 0, [4], [0])) == "HB_E_SHAPE"
    assert _err(lambda: hb.schedule_iteration(8, 8, [0], [0])) == "HB_E_LENGTH"
    assert _err(lambda: hb.schedule_iteration(8, 8, [4], [-1])) == "HB_E_LENGTH"
