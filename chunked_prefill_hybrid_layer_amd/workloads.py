"""Seeded synthetic inputs for the hybrid-batch decoder layer.

This module only draws random numbers and lays out caller-side arrays
(weights, activations, batch composition, block tables, cached K/V contents).
It holds none of the layer's arithmetic and none of the paged-KV indexing:
positions, slots, norms, projections and attention live in the library and,
independently, in the oracle.  Both sides consume exactly the arrays built
here.

Batch composition follows the hybrid batches of the Sarathi-Serve reading
notes (zhongzhuzhou.org), §3.2 "Stall-free hybrid batching": prefill-chunk
tokens of one or more prompts plus one token per running decode, with the
total under a token budget tau.  Packing order is chunks first (argument
order), then decodes.

Value recipe (the pages give none; these are readings):
  * projection weights N(0, 0.02), norm gains 1 + 0.02 N(0, 1), all rounded
    to bf16;
  * layer input x ~ N(0, x_std) rounded to bf16 and stored as fp32;
  * cached K/V of synthesized prefixes N(0, 1) rounded to bf16;
  * block tables: the pool holds every page the batch needs plus 12.5 %
    decoy pages; a seeded permutation of the pool is dealt out in sequence
    order, so no page is shared; unused table entries are -1.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
import os
from typing import Dict, List, Optional

import numpy as np

PAGE_SIZE = 16


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


_BLOCK = 1 << 22            # elements per independently seeded block
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures as cf
        _POOL = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def normal_bf16(seed: np.random.SeedSequence, shape, std: float = 1.0, mean: float = 0.0,
                parallel: bool = True) -> np.ndarray:
    """mean + std * N(0, 1), rounded to bf16 bits.  The flat array is cut into
    fixed blocks, each drawn from its own child of ``seed``, so the values do
    not depend on how many threads draw them."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nblk = (n + _BLOCK - 1) // _BLOCK
    kids = seed.spawn(nblk)

    def work(i):
        lo, hi = i * _BLOCK, min(n, (i + 1) * _BLOCK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = f32_to_bf16_bits(v)

    if parallel and nblk > 1:
        list(_pool().map(work, range(nblk)))
    else:
        for i in range(nblk):
            work(i)
    return out.reshape(shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Dims:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    page_size: int = PAGE_SIZE
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    kv_fp8: int = 0            # 1: FP8 e4m3 KV cache with the scales below
    k_scale: float = 1.0
    v_scale: float = 1.0
    w8a8: int = 0              # 1: FP8 e4m3 projections (weights and their inputs)
    x_scale: float = 1.0       # static scales of the four projection inputs
    o_scale: float = 1.0
    h_scale: float = 1.0
    a_scale: float = 1.0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass
class Batch:
    """One hybrid batch: chunk pieces (new tokens + already-cached prefix)
    and decodes (context already cached), with per-sequence block tables.

    Sequence order (= block-table row order) is the chunks, then the decodes.
    """
    chunk_len: np.ndarray          # int32 [n_chunks]
    chunk_prefix: np.ndarray       # int32 [n_chunks]
    decode_ctx: np.ndarray         # int32 [n_decodes]
    block_table: np.ndarray        # int32 [n_seq][max_pages], -1 = unused
    num_pages: int
    token_budget: int

    @property
    def n_chunks(self) -> int:
        return int(len(self.chunk_len))

    @property
    def n_decodes(self) -> int:
        return int(len(self.decode_ctx))

    @property
    def n_seq(self) -> int:
        return self.n_chunks + self.n_decodes

    @property
    def n_tokens(self) -> int:
        return int(np.sum(self.chunk_len)) + self.n_decodes

    def cached_lengths(self) -> np.ndarray:
        """Tokens already in the cache per sequence (chunk prefix / decode context)."""
        return np.concatenate([self.chunk_prefix, self.decode_ctx]).astype(np.int64)

    def new_lengths(self) -> np.ndarray:
        return np.concatenate([self.chunk_len, np.ones(self.n_decodes, np.int32)]).astype(np.int64)


@dataclass
class Workload:
    name: str
    dims: Dims
    weights: Dict[str, np.ndarray]     # bf16 bits; projections [d_out][d_in]
    x: np.ndarray                      # float32 [T][H], bf16-representable
    batch: Batch
    # cached K/V contents per sequence, logical order [len][n_kv][d] as bf16 bits
    prefix_k: List[np.ndarray] = field(default_factory=list)
    prefix_v: List[np.ndarray] = field(default_factory=list)
    meta: Dict[str, object] = field(default_factory=dict)


# --------------------------------------------------------------------------
# building blocks


def _streams(seed: int, n: int = 6):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def make_weights(dims: Dims, rng: np.random.Generator, std: float = 0.02) -> Dict[str, np.ndarray]:
    H, d, F = dims.hidden, dims.head_dim, dims.ffn_dim
    shapes = {
        "w_q": (dims.n_q_heads * d, H),
        "w_k": (dims.n_kv_heads * d, H),
        "w_v": (dims.n_kv_heads * d, H),
        "w_o": (H, dims.n_q_heads * d),
        "w_g": (F, H),
        "w_u": (F, H),
        "w_d": (H, F),
    }
    root = np.random.SeedSequence(int(rng.integers(2**63)))
    kids = root.spawn(len(shapes) + 2)
    w = {}
    for kid, (name, shp) in zip(kids, shapes.items()):
        w[name] = normal_bf16(kid, shp, std)
    w["g_attn"] = normal_bf16(kids[-2], (H,), 0.02, 1.0)
    w["g_ffn"] = normal_bf16(kids[-1], (H,), 0.02, 1.0)
    return w


WEIGHT_SHAPES = ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d")


def make_weights_fp8(dims: Dims, seed: np.random.SeedSequence, rms: float = 0.02) -> Dict[str, np.ndarray]:
    """Projection matrices as e4m3 codes drawn bit field by bit field: random
    sign, exponent field uniform in 4..11, mantissa field uniform in 0..7
    (magnitudes 1/8 .. 30, log-uniform), and one float32 scale per output row,
    rms / 9 * U(0.5, 1.5), so that the weights' rms is about ``rms``.  Norm
    gains as in make_weights."""
    H, d, F = dims.hidden, dims.head_dim, dims.ffn_dim
    shapes = {"w_q": (dims.n_q_heads * d, H), "w_k": (dims.n_kv_heads * d, H), "w_v": (dims.n_kv_heads * d, H),
              "w_o": (H, dims.n_q_heads * d), "w_g": (F, H), "w_u": (F, H), "w_d": (H, F)}
    kids = seed.spawn(len(shapes) + 2)
    w = {}
    for kid, (name, shp) in zip(kids, shapes.items()):
        g = np.random.Generator(np.random.PCG64(kid))
        sign = g.integers(0, 2, size=shp, dtype=np.uint8) << 7
        expo = g.integers(4, 12, size=shp, dtype=np.uint8) << 3
        mant = g.integers(0, 8, size=shp, dtype=np.uint8)
        w[name] = (sign | expo | mant).astype(np.uint8)
        w["s_" + name] = (np.float32(rms / 9.0) * g.uniform(0.5, 1.5, size=shp[0]).astype(np.float32)).astype(np.float32)
    w["g_attn"] = normal_bf16(kids[-2], (H,), 0.02, 1.0)
    w["g_ffn"] = normal_bf16(kids[-1], (H,), 0.02, 1.0)
    return w


# static projection-input scales of the synthetic FP8 workloads: N(0, 1)-sized
# xn and h1n, attention outputs within +-4, SwiGLU outputs within +-50, all
# inside e4m3's +-448 over the scale.  Distinct, none a power of two and no
# ratio of two of them a power of two: e4m3 has a floating exponent, so a
# value quantised and read back with a scale 2^k times the right one lands on
# the same grid, and a swap of two such scales would be invisible
FP8_ACT_SCALES = dict(x_scale=0.07, o_scale=0.03, h_scale=0.05, a_scale=0.13)


def make_activations(n_tokens: int, hidden: int, rng: np.random.Generator, std: float) -> np.ndarray:
    x = rng.standard_normal((n_tokens, hidden), dtype=np.float32) * np.float32(std)
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def deal_block_tables(kv_lens: np.ndarray, page_size: int, rng: np.random.Generator,
                      decoy_frac: float = 0.125, max_pages: Optional[int] = None):
    """Deal a shuffled page pool to sequences needing ceil(kv_len/page) pages each."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    need = (kv_lens + page_size - 1) // page_size
    total = int(need.sum())
    num_pages = total + max(1, int(np.ceil(total * decoy_frac)))
    perm = rng.permutation(num_pages).astype(np.int32)
    mp = int(need.max()) if max_pages is None else int(max_pages)
    bt = np.full((len(kv_lens), max(mp, 1)), -1, dtype=np.int32)
    cur = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[cur:cur + n]
        cur += int(n)
    return bt, num_pages


def synth_prefix(length: int, dims: Dims, seed: np.random.SeedSequence, std: float = 1.0):
    shp = (int(length), dims.n_kv_heads, dims.head_dim)
    ks, vs = seed.spawn(2)
    return normal_bf16(ks, shp, std, parallel=False), normal_bf16(vs, shp, std, parallel=False)


def build_workload(name: str, dims: Dims, chunk_len, chunk_prefix, decode_ctx, seed: int,
                   x_std: float = 1.0, token_budget: Optional[int] = None,
                   synth_prefixes: bool = True, max_pages: Optional[int] = None,
                   cache_std: float = 1.0) -> Workload:
    rw, rx, _rl, rb, rc, _ = _streams(seed)
    chunk_len = np.asarray(chunk_len, dtype=np.int32)
    chunk_prefix = np.asarray(chunk_prefix, dtype=np.int32)
    decode_ctx = np.asarray(decode_ctx, dtype=np.int32)
    cached = np.concatenate([chunk_prefix, decode_ctx]).astype(np.int64)
    new = np.concatenate([chunk_len, np.ones(len(decode_ctx), np.int32)]).astype(np.int64)
    bt, num_pages = deal_block_tables(cached + new, dims.page_size, rb, max_pages=max_pages)
    T = int(new.sum())
    batch = Batch(chunk_len, chunk_prefix, decode_ctx, bt, num_pages,
                  int(token_budget) if token_budget is not None else T)
    w = make_weights(dims, rw)
    x = make_activations(T, dims.hidden, rx, x_std)
    wl = Workload(name, dims, w, x, batch)
    if synth_prefixes:
        # one child stream per sequence, so any subset can be regenerated alone
        children = np.random.SeedSequence(int(rc.integers(2**63))).spawn(len(cached))
        kv = list(_pool().map(lambda s: synth_prefix(int(cached[s]), dims, children[s], cache_std),
                              range(len(cached))))
        wl.prefix_k = [k for k, _ in kv]
        wl.prefix_v = [v for _, v in kv]
    return wl


# --------------------------------------------------------------------------
# named workloads (shapes and length mixes of the pages' configurations)

TINY = Dims(hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=512)
MISTRAL = Dims(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn_dim=14336)
YI = Dims(hidden=7168, n_q_heads=56, n_kv_heads=8, head_dim=128, ffn_dim=20480)


def _lognormal_ctx(rng, n, median, cap, sigma=1.0):
    c = np.rint(rng.lognormal(np.log(median), sigma, size=n))
    return np.clip(np.minimum(c, cap), 1, None).astype(np.int32)


def tiny(seed: int = 0) -> Workload:
    """Tiny layer: one 256-token prompt whose 3rd 64-token chunk (prefix 128)
    runs with 4 decodes of context 16/40/77/128.  Weights and activations
    N(0, 0.02).  The prompt's own prefix is not synthesized: callers produce it
    by running chunks 1 and 2 through the layer (see ``tiny_prompt_chunks``)."""
    wl = build_workload("tiny", TINY, [64], [128], [16, 40, 77, 128], seed,
                        x_std=0.02, synth_prefixes=True)
    wl.meta["prompt_len"] = 256
    wl.meta["chunk_size"] = 64
    return wl


def tiny_prompt_chunks(wl: Workload, seed: int = 0):
    """Inputs for chunks 1 and 2 of the tiny prompt (positions 0..127): x rows
    drawn from their own stream so chunk 3's x stays that of ``tiny``."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    return [make_activations(64, wl.dims.hidden, rng, 0.02) for _ in range(2)]


def mistral_tau512(seed: int = 0) -> Workload:
    """Mistral-7B-shaped layer, tau = 512: one 480-token chunk with prefix
    U{0..3584} plus 32 decodes with context U{512..4096}."""
    _, _, rl, _, _, _ = _streams(seed)
    prefix = int(rl.integers(0, 3584, endpoint=True))
    ctx = rl.integers(512, 4096, size=32, endpoint=True).astype(np.int32)
    wl = build_workload("mistral_tau512", MISTRAL, [480], [prefix], ctx, seed, token_budget=512)
    return wl


def tau_sweep(tau: int, seed: int = 0) -> Workload:
    """tau sweep point: one chunk of tau-64 tokens (prefix 1792) plus 64
    decodes with context lognormal(median 1024, sigma 1) capped at 8192."""
    _, _, rl, _, _, _ = _streams(seed)
    ctx = _lognormal_ctx(rl, 64, 1024, 8192)
    return build_workload(f"tau_sweep_{tau}", MISTRAL, [tau - 64], [1792], ctx, seed,
                          token_budget=tau)


def yi_tau2048(seed: int = 0) -> Workload:
    """Yi-34B-shaped layer, tau = 2048: chunks of 768 at prefixes 0 and 6144
    plus 512 decodes with context lognormal(median 2048, sigma 1) capped at 16384."""
    _, _, rl, _, _, _ = _streams(seed)
    ctx = _lognormal_ctx(rl, 512, 2048, 16384)
    return build_workload("yi_tau2048", YI, [768, 768], [0, 6144], ctx, seed, token_budget=2048)


def spec_verify(seed: int = 0, n_req: int = 128, q_len: int = 4) -> Workload:
    """Speculative-decoding verify batch on the Mistral-7B-shaped layer: 128
    requests each checking 3 drafted tokens at once ("Sarathi-Serve reading
    notes" §7.4), i.e. pieces of 4 new tokens whose prefix is the request's
    whole context; contexts lognormal(median 1024, sigma 1) capped at 8192;
    512 tokens."""
    _, _, rl, _, _, _ = _streams(seed)
    ctx = _lognormal_ctx(rl, n_req, 1024, 8192)
    return build_workload("spec_verify", MISTRAL, [q_len] * n_req, ctx, [], seed, token_budget=n_req * q_len)


# FP8 KV cache scales of the synthetic workloads (powers of two, K and V
# different): N(0, 1)-sized K/V over the scale stay far inside e4m3's +-448
# and far above its subnormals (2^-6)
FP8_K_SCALE = 2.0 ** -4
FP8_V_SCALE = 2.0 ** -3


def with_kv_fp8(wl: Workload, k_scale: float = FP8_K_SCALE, v_scale: float = FP8_V_SCALE) -> Workload:
    """The same workload with an FP8 e4m3 KV cache (prefixes are quantised
    when they are written)."""
    wl.dims = dataclasses.replace(wl.dims, kv_fp8=1, k_scale=float(k_scale), v_scale=float(v_scale))
    wl.name += "_kvfp8"
    return wl


def with_w8a8(wl: Workload, seed: int = 0) -> Workload:
    """The same workload with FP8 projections: fresh e4m3 weight codes and row
    scales (make_weights_fp8) and the static input scales FP8_ACT_SCALES."""
    wl.dims = dataclasses.replace(wl.dims, w8a8=1, **FP8_ACT_SCALES)
    wl.weights = make_weights_fp8(wl.dims, np.random.SeedSequence([seed, 8]))
    wl.name += "_w8a8"
    return wl


YI_TP2 = Dims(hidden=7168, n_q_heads=28, n_kv_heads=4, head_dim=128, ffn_dim=10240)


def yi_tau2048_tp2(seed: int = 0) -> Workload:
    """One GPU's share of the Yi-34B-shaped layer under 2-way tensor
    parallelism: half the q and kv heads (28 / 4, g = 7) and half the FFN
    (10240), full hidden size, over the batch of yi_tau2048 (its lengths and
    block tables; the KV pool holds this GPU's 4 kv heads)."""
    _, _, rl, _, _, _ = _streams(seed)
    ctx = _lognormal_ctx(rl, 512, 2048, 16384)
    return build_workload("yi_tau2048_tp2", YI_TP2, [768, 768], [0, 6144], ctx, seed, token_budget=2048)


def small(seed: int = 0, n_q: int = 8, n_kv: int = 2, head_dim: int = 128,
          chunk_len=(77, 130), chunk_prefix=(45, 0), decode_ctx=(1, 15, 16, 17, 200, 333, 1000),
          hidden: int = 512, ffn: int = 1024) -> Workload:
    """Small layer for full-output parity: several GEMM and attention tiles,
    ragged chunks starting mid-page, decodes around page boundaries."""
    d = Dims(hidden=hidden, n_q_heads=n_q, n_kv_heads=n_kv, head_dim=head_dim, ffn_dim=ffn)
    return build_workload(f"small_g{n_q // n_kv}_d{head_dim}", d, list(chunk_len), list(chunk_prefix),
                          list(decode_ctx), seed)


@dataclass
class LongPrompt:
    """A long prompt run as successive chunks, each co-batched with the same
    set of decodes (stall-free: every decode advances by one token per
    iteration), next to the same prompt as one unchunked prefill."""
    dims: Dims
    weights: Dict[str, np.ndarray]
    prompt_x: np.ndarray            # [L][H] float32, bf16-representable
    chunk: int
    decode_ctx0: np.ndarray         # [n_dec] contexts at iteration 0
    decode_x: np.ndarray            # [n_iter][n_dec][H]
    block_table: np.ndarray         # [1 + n_dec][max_pages]: the prompt, then the decodes
    num_pages: int
    prefix_k: list = field(default_factory=list)   # per sequence (the prompt's is empty)
    prefix_v: list = field(default_factory=list)

    @property
    def prompt_len(self) -> int:
        return int(self.prompt_x.shape[0])

    @property
    def n_iter(self) -> int:
        return self.prompt_len // self.chunk

    @property
    def n_dec(self) -> int:
        return len(self.decode_ctx0)

    def batch(self, i: int) -> Batch:
        """Iteration i: chunk i of the prompt (prefix i * chunk) + every decode."""
        return Batch(np.array([self.chunk], np.int32), np.array([i * self.chunk], np.int32),
                     (self.decode_ctx0 + i).astype(np.int32), self.block_table, self.num_pages,
                     self.chunk + self.n_dec)

    def x(self, i: int) -> np.ndarray:
        return np.concatenate([self.prompt_x[i * self.chunk:(i + 1) * self.chunk], self.decode_x[i]])

    def unchunked_batch(self) -> Batch:
        L = self.prompt_len
        return Batch(np.array([L], np.int32), np.array([0], np.int32), np.zeros(0, np.int32),
                     np.ascontiguousarray(self.block_table[:1]), self.num_pages, L)


def long_prompt(seed: int = 0, prompt_len: int = 32768, chunk: int = 512, n_dec: int = 64,
                ctx_lo: int = 1024, ctx_hi: int = 8192, dims: Dims = None) -> LongPrompt:
    """Long-prompt chunking on the Mistral-7B-shaped layer: a 32768-token
    prompt as 64 chunks of 512, each co-batched with 64 decodes whose contexts
    start uniform in [1024, 8192] and grow by one per iteration; x ~ N(0, 1)
    (fresh decode inputs each iteration); decode prefixes N(0, 1) bf16."""
    dims = MISTRAL if dims is None else dims
    assert prompt_len % chunk == 0
    rw, rx, rl, rb, rc, _ = _streams(seed)
    n_iter = prompt_len // chunk
    ctx0 = rl.integers(ctx_lo, ctx_hi + 1, size=n_dec).astype(np.int32)
    kv_lens = np.concatenate([[prompt_len], ctx0.astype(np.int64) + n_iter])
    bt, num_pages = deal_block_tables(kv_lens, dims.page_size, rb)
    w = make_weights(dims, rw)
    xs = np.random.SeedSequence(int(rx.integers(2**63))).spawn(2)
    prompt_x = bf16_bits_to_f32(normal_bf16(xs[0], (prompt_len, dims.hidden), 1.0))
    decode_x = bf16_bits_to_f32(normal_bf16(xs[1], (n_iter, n_dec, dims.hidden), 1.0))
    lp = LongPrompt(dims, w, prompt_x, chunk, ctx0, decode_x, bt, num_pages)
    children = np.random.SeedSequence(int(rc.integers(2**63))).spawn(n_dec)
    kv = list(_pool().map(lambda j: synth_prefix(int(ctx0[j]), dims, children[j]), range(n_dec)))
    empty = np.zeros((0, dims.n_kv_heads, dims.head_dim), np.uint16)
    lp.prefix_k = [empty] + [k for k, _ in kv]
    lp.prefix_v = [empty] + [v for _, v in kv]
    return lp
