"""hb_layer_forward_static_scratch: the layer forward on the library's static
device scratch (no workspace argument, for callers that cannot allocate),
against hb_layer_forward with a caller workspace on the same inputs.  Both run
the same kernels with the same plans, so the outputs and the caches they leave
are bit-identical.  Two calls in a row, the second with a smaller batch: the
scratch keeps the first call's contents, which must not matter."""
import ctypes

import numpy as np
import pytest

from chunked_prefill_hybrid_layer_amd import workloads as W
from tests.helpers import assert_close, gemm_plan_workload, log, oracle_forward, sample_rows


def test_static_scratch_rejects_a_batch_beyond_its_size():
    """A batch whose workspace exceeds the 128 MiB scratch is refused on the
    host, before any HIP call (so this runs without a GPU: the device
    pointers are never touched)."""
    from chunked_prefill_hybrid_layer_amd import hb
    d = W.MISTRAL
    L = 8192
    bt, npg = W.deal_block_tables(np.array([L]), 16, np.random.default_rng(0))
    dims = hb.make_dims(d)
    blob, T = hb.pack_metadata(dims, [L], [0], [], bt, npg, L)
    need = hb.workspace_bytes(dims, blob)
    assert need > hb.STATIC_SCRATCH_BYTES
    fake = 1 << 40
    w = hb.Weights(*([fake] * 9), *([0] * 7))
    st = hb.lib.hb_layer_forward_static_scratch(ctypes.byref(dims), ctypes.byref(w),
                                                blob.ctypes.data_as(ctypes.c_void_p), fake, fake, L + 1, fake,
                                                fake + 256, fake, fake, 0)
    assert st == 7, hb.lib.hb_last_error_detail()         # HB_E_CAPACITY
    detail = hb.lib.hb_last_error_detail().decode()
    assert "static scratch" in detail and str(need) in detail


@pytest.mark.gpu
def test_static_scratch_forward_matches_workspace_forward():
    import torch
    from chunked_prefill_hybrid_layer_amd import hb
    from chunked_prefill_hybrid_layer_amd.runtime import DeviceLayer, stream_handle
    assert torch.cuda.is_available(), "GPU test"
    # the tau = 512 Mistral-shaped batch (about 111 MB of workspace), then a
    # 200-token batch of the same layer shape
    for wl in (W.mistral_tau512(0), gemm_plan_workload("mistral_T200")):
        b = wl.batch
        log(f"static scratch: {wl.name} T={b.n_tokens}")
        maxpos = int(np.max(b.cached_lengths() + b.new_lengths())) + 1
        layers = []
        for _ in range(2):
            L = DeviceLayer(wl.dims, wl.weights, b.num_pages, maxpos)
            L.fill_prefixes(b.block_table, range(b.n_seq), wl.prefix_k, wl.prefix_v)
            layers.append(L)
        la, lb = layers
        prep_a = la.prepare(b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.token_budget)
        prep_b = lb.prepare(b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.token_budget)
        need = hb.workspace_bytes(la.hd, prep_a.blob)
        log(f"static scratch: workspace need {need} of {hb.STATIC_SCRATCH_BYTES} bytes")
        assert need <= hb.STATIC_SCRATCH_BYTES
        x = torch.from_numpy(np.ascontiguousarray(wl.x, dtype=np.float32)).cuda()
        ya, yb = torch.empty_like(x), torch.full_like(x, float("nan"))
        la.forward(prep_a, x, ya)
        hb.layer_forward_static_scratch(lb.hd, lb.hw, prep_b.blob, prep_b.meta_dev.data_ptr(), lb.rope.data_ptr(),
                                        lb.rope_max_pos, x.data_ptr(), yb.data_ptr(), lb.k_cache.data_ptr(),
                                        lb.v_cache.data_ptr(), stream_handle())
        torch.cuda.synchronize()
        ya, yb = ya.cpu().numpy(), yb.cpu().numpy()
        assert np.all(np.isfinite(yb))
        assert np.array_equal(ya, yb), f"{wl.name}: static-scratch output differs from the workspace forward"
        for name, a, c in zip("KV", la.cache_logical(), lb.cache_logical()):
            assert np.array_equal(a, c), f"{wl.name}: {name} cache differs"
        # and against the oracle, on sampled rows, at the floating-point bar
        rows = sample_rows(wl, n_random=16)[:64]
        from oracle import hybrid_layer as O
        from tests.helpers import oracle_cache
        lay = O.token_layout(b.chunk_len, b.chunk_prefix, b.decode_ctx)
        cache = oracle_cache(wl, seqs=sorted(set(int(s) for s in lay.seq[rows])))
        r, _ = oracle_forward(wl, rows=rows, cache=cache)
        assert_close(yb[rows], r.y, f"static scratch {wl.name} vs oracle")
        del layers, la, lb, x
        torch.cuda.empty_cache()
