"""Conditioning of the layer under its own bf16 storage roundings (CPU, the
oracle alone).

Every activation that passes between steps is stored in bf16 (the layer's
precision contract), so a change of one fp32 ulp in a value just before it is
rounded flips the stored value by one bf16 step with probability about
change / ulp(bf16).  A flip at an early storage point changes every later
pre-rounding value by far more than an fp32 ulp, and the next storage point
then flips many of its values; after a few points the rounding of the later
activations is as good as independent.  That sets a floor under the
agreement any implementation that accumulates in fp32 can reach with the
float64 oracle: the oracle's own output moves by that much when its input
moves by 1e-7 relative.

These tests pin where the floor lies relative to the literal bars
(rel-L2 <= 1e-2, max-abs <= 5e-2) for the two layer shapes of the
configurations, and which storage points drive it:
  * Yi-34B-shaped (hidden 7168, 56/8 heads, FFN 20480): the max-abs floor is
    above 5e-2, so no fp32-accumulating implementation meets the literal
    max-abs bar on this shape; rel-L2 stays far below 1e-2;
  * Mistral-7B-shaped (hidden 4096, 32/8 heads, FFN 14336): the floor is
    below both bars (on the most sensitive rows, a chunk at prefix 0, it
    reaches about 0.04 of the 0.05 max-abs bar), which therefore apply as
    stated;
  * the cascade starts at the attention inputs: a perturbation of the normed
    input alone reproduces the whole floor, one of the SwiGLU output alone
    only a small part of it.
Worked iteration context: "Sarathi-Serve reading notes" §7.6 (the Yi-34B
iteration the Yi configuration mirrors)."""
import numpy as np
import pytest

from oracle import hybrid_layer as O
from chunked_prefill_hybrid_layer_amd import workloads as W

EPS = 1e-7


def _batch(dims, seed=0):
    """One 64-token chunk at prefix 0 (the rows most sensitive to their own
    chunk's K/V) plus 8 decodes with lognormal contexts (median 2048)."""
    rl = np.random.default_rng(seed)
    ctx = np.clip(np.minimum(np.rint(rl.lognormal(np.log(2048), 1.0, 8)), 16384), 1, None).astype(np.int32)
    return W.build_workload("floor", dims, [64], [0], ctx, seed)


class _Layer:
    def __init__(self, dims):
        self.wl = _batch(dims)
        self.w = O.weights_to_float(self.wl.weights)
        self.x = self.wl.x.astype(np.float64)

    def run(self, x=None, perturb=None):
        wl, b = self.wl, self.wl.batch
        cache = O.PagedCache(b.num_pages, wl.dims.n_kv_heads, 16, wl.dims.head_dim)
        for s in range(b.n_seq):
            if wl.prefix_k[s].shape[0]:
                cache.load_prefix(b.block_table, s, O.bf16_bits_to_float(wl.prefix_k[s]),
                                  O.bf16_bits_to_float(wl.prefix_v[s]))
        return O.layer_forward(wl.dims, self.w, self.x if x is None else x, b.chunk_len, b.chunk_prefix,
                               b.decode_ctx, b.block_table, cache, perturb=perturb).y

    def floor(self, point):
        """(rel-L2, max-abs) change of y when the value at one storage point
        (or the input x) is multiplied by 1 + EPS N(0, 1) before rounding."""
        rng = np.random.default_rng(1)
        if point == "x":
            y1 = self.run(x=self.x * (1 + EPS * rng.standard_normal(self.x.shape)))
        else:
            hook = lambda name, a: a * (1 + EPS * rng.standard_normal(a.shape)) if name == point else a
            y1 = self.run(perturb=hook)
        y0 = self.y0
        return float(np.linalg.norm(y1 - y0) / np.linalg.norm(y0)), float(np.max(np.abs(y1 - y0)))


@pytest.fixture(scope="module")
def yi():
    lay = _Layer(W.YI)
    lay.y0 = lay.run()
    return lay


def test_perturb_hook_off_is_the_plain_layer(yi):
    """The hook that passes every value through leaves the result bit-identical."""
    assert np.array_equal(yi.run(perturb=lambda name, a: a), yi.y0)


def test_yi_shape_floor_is_above_the_literal_max_abs(yi):
    rel, mx = yi.floor("x")
    print(f"Yi-shaped floor (input x 1e-7 relative): rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert mx > 5e-2          # the literal max-abs bar is below the oracle's own floor
    assert rel < 2.5e-3       # rel-L2 keeps a wide margin under its 1e-2 bar


def test_yi_shape_floor_comes_from_the_attention_inputs(yi):
    """A 1e-7 relative change of the normed input alone (before its bf16
    rounding) reproduces the floor; the same change of the SwiGLU output alone
    (the last storage point) moves y by a small fraction of it."""
    _, mx_xn = yi.floor("xn")
    _, mx_a = yi.floor("a")
    _, mx_h1n = yi.floor("h1n")
    print(f"Yi-shaped floor by storage point: xn {mx_xn:.3e}, h1n {mx_h1n:.3e}, a {mx_a:.3e}")
    assert mx_xn > 5e-2
    assert mx_a < 1e-2 and mx_a < 0.2 * mx_xn
    assert mx_h1n < mx_xn


def test_mistral_shape_floor_is_below_the_literal_bars():
    lay = _Layer(W.MISTRAL)
    lay.y0 = lay.run()
    rel, mx = lay.floor("x")
    print(f"Mistral-shaped floor (input x 1e-7 relative): rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert mx < 5e-2 and rel < 2.5e-3
