#!/usr/bin/env python3
"""Hybrid-batch decoder layer on one MI355X: tokens/s at tau = 512 on the
Mistral-7B-shaped layer (one 480-token prefill chunk + 32 decodes), with the
dominant kernel's roofline fraction and the CPU oracle timed beside it.

One step = the whole hot path over one batch: hb_pack_metadata on the host
into a pinned buffer, the asynchronous copy of the blob to the device, and
hb_layer_forward (RMSNorm, QKV + RoPE + KV append, hybrid attention, O +
residual, RMSNorm, gate/up + SwiGLU, down + residual).  Weights, KV cache and
activations are resident in HBM before the timed region.  Four independent
copies of weights and KV pools are used in turn so that the 256 MB
Infinity Cache cannot serve a step from the previous step's data.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --sweep-tau      # token budget 128 .. 2048, one line per tau
    python bench.py --kv-append      # hb_kv_append GB/s at T = 32768
    python bench.py --long-prompt    # 32768-token prompt, 64 chunks of 512 vs unchunked
    python bench.py --chunk-sweep    # the same prompt alone at chunk sizes 128 .. 2048
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
STAGE_EVERY = 8                # timed steps per step that records the per-stage HIP events
SETTLE_MS = 25.0               # untimed forwards before the warm-up steps (GPU power-state ramp)


def workload_by_name(name):
    from chunked_prefill_hybrid_layer_amd import workloads as W
    if name == "mistral_tau512":
        return W.mistral_tau512(0)
    if name.startswith("tau_sweep_"):
        return W.tau_sweep(int(name.rsplit("_", 1)[1]), 0)
    if name == "yi_tau2048":
        return W.yi_tau2048(0)
    if name == "yi_tau2048_tp2":
        return W.yi_tau2048_tp2(0)
    if name == "tiny":
        return W.tiny(0)
    if name == "spec_verify":
        return W.spec_verify(0)
    raise SystemExit(f"unknown workload {name}")


def stage_model(wl):
    """Algorithmic work of each stage for one launch: (flops, bytes, bound)."""
    from chunked_prefill_hybrid_layer_amd import hb
    d, b = wl.dims, wl.batch
    T = b.n_tokens
    H, nq, nkv, D, F = d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn_dim
    cached = b.cached_lengths()
    new = b.new_lengths()
    # attention (query, key) pairs: a token at position p sees p+1 keys.  Chunk
    # pieces whose (token, head) rows fit the decode kernel's 16-row tile
    # (new tokens x group <= 16) run on the decode kernel; their keys are read
    # once for all their rows.
    g = nq // nkv
    on_dec = b.chunk_len * g <= 16
    chunk_pairs, dec_pairs, chunk_kv_keys, dec_kv_keys = 0, 0, 0, 0
    for c, n, dp in zip(b.chunk_prefix, b.chunk_len, on_dec):
        pairs = int(n) * int(c) + int(n) * (int(n) + 1) // 2
        if dp:
            dec_pairs += pairs
            dec_kv_keys += int(c) + int(n)
        else:
            chunk_pairs += pairs
            chunk_kv_keys += int(c) + int(n)
    dec_pairs += int(np.sum(b.decode_ctx.astype(np.int64) + 1))
    dec_kv_keys += int(np.sum(b.decode_ctx.astype(np.int64) + 1))
    kv_elem = 1 if getattr(d, "kv_fp8", 0) else 2            # bytes per cached K/V element
    kv_bytes_per_key = nkv * D * 2 * kv_elem                # K and V
    we = 1 if getattr(d, "w8a8", 0) else 2                   # bytes per weight / projection-input element
    blob, _ = hb.pack_metadata(hb.make_dims(d), b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table,
                               b.num_pages, b.token_budget)
    npart = hb.header(blob).n_partials
    part_bytes = npart * nq * (D + 2) * 4
    m = {
        "rmsnorm_attn": (0, T * H * 4 + T * H * we + H * 2, "hbm"),
        "qkv_rope_append": (2 * T * H * (nq + 2 * nkv) * D,
                            (nq + 2 * nkv) * D * H * we + T * H * we + T * nq * D * 2 + T * 2 * nkv * D * kv_elem,
                            "mfma"),
        "attn_chunk": (4 * chunk_pairs * nq * D, chunk_kv_keys * kv_bytes_per_key, "mfma"),
        "attn_decode": (4 * dec_pairs * nq * D, dec_kv_keys * kv_bytes_per_key, "hbm"),
        "attn_merge": (0, part_bytes + T * nq * D * we, "hbm"),
        "o_proj_residual": (2 * T * nq * D * H, nq * D * H * we + T * nq * D * we + 2 * T * H * 4, "mfma"),
        "rmsnorm_ffn": (0, T * H * 4 + T * H * we + H * 2, "hbm"),
        "gate_up_swiglu": (2 * T * H * 2 * F, 2 * F * H * we + T * H * we + T * F * we, "mfma"),
        "down_residual": (2 * T * F * H, F * H * we + T * F * we + 2 * T * H * 4, "mfma"),
    }
    return m


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gate_up_swiglu": ["chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"],
    "qkv_rope_append": ["chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"],
    "o_proj_residual": ["chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"],
    "down_residual": ["chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"],
    "attn_chunk": ["chunked_prefill_hybrid_layer_amd/csrc/attention.hip"],
    "attn_decode": ["chunked_prefill_hybrid_layer_amd/csrc/attention.hip"],
    "attn_merge": ["chunked_prefill_hybrid_layer_amd/csrc/attention.hip"],
    "rmsnorm_attn": ["chunked_prefill_hybrid_layer_amd/csrc/elementwise.hip"],
    "rmsnorm_ffn": ["chunked_prefill_hybrid_layer_amd/csrc/elementwise.hip"],
}


def measured_traffic(stage, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(workload, {}).get(stage)
    if not e or e.get("source_hash") != source_hash(KERNEL_SOURCES[stage]):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl, stride=4):
    """The oracle (float64 numpy) on every `stride`-th packed token of the same
    batch; K/V of all tokens are computed since the cache needs them, and the
    cached prefixes of the sampled rows' sequences are loaded."""
    from oracle import hybrid_layer as O
    b = wl.batch
    rows = np.arange(0, b.n_tokens, stride)
    lay = O.token_layout(b.chunk_len, b.chunk_prefix, b.decode_ctx)
    need = sorted(set(int(s) for s in lay.seq[rows]))
    cache = _oracle_cache(O, wl)
    for s in need:
        if wl.prefix_k[s].shape[0]:
            cache.load_prefix(b.block_table, s, O.bf16_bits_to_float(wl.prefix_k[s]),
                              O.bf16_bits_to_float(wl.prefix_v[s]))
    w = O.weights_to_float(wl.weights)
    t0 = time.perf_counter()
    O.layer_forward(wl.dims, w, wl.x.astype(np.float64), b.chunk_len, b.chunk_prefix, b.decode_ctx,
                    b.block_table, cache, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": _oracle_threads(), "cpu_model": _cpu_model(),
            "kind": "oracle",
            "sample": (f"all {b.n_tokens} packed tokens" if stride == 1 else
                       f"{len(rows)} of the {b.n_tokens} packed tokens (every {stride}th; K/V for all {b.n_tokens})") +
                      f" of the same batch, float64 numpy oracle, {dt:.1f} s"}


def _oracle_cache(O, wl):
    d = wl.dims
    return O.PagedCache(wl.batch.num_pages, d.n_kv_heads, d.page_size, d.head_dim, kv_fp8=d.kv_fp8,
                        k_scale=d.k_scale, v_scale=d.v_scale)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_whole(wl, reps=10):
    """The oracle on the whole batch, median of `reps` calls (small configs)."""
    from oracle import hybrid_layer as O
    b = wl.batch
    w = O.weights_to_float(wl.weights)
    ts = []
    for _ in range(reps):
        cache = _oracle_cache(O, wl)
        for s in range(b.n_seq):
            if wl.prefix_k[s].shape[0]:
                cache.load_prefix(b.block_table, s, O.bf16_bits_to_float(wl.prefix_k[s]),
                                  O.bf16_bits_to_float(wl.prefix_v[s]))
        t0 = time.perf_counter()
        O.layer_forward(wl.dims, w, wl.x.astype(np.float64), b.chunk_len, b.chunk_prefix, b.decode_ctx,
                        b.block_table, cache)
        ts.append(time.perf_counter() - t0)
    dt = float(np.median(ts))
    return {"value": b.n_tokens / dt, "unit": "tokens/s", "cores": _oracle_threads(), "cpu_model": _cpu_model(),
            "kind": "oracle", "sample": f"all {b.n_tokens} packed tokens, median of {reps} calls "
                                        f"({dt * 1e3:.1f} ms each), float64 numpy oracle"}


def _oracle_threads():
    threads = int(os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or
                  len(os.sched_getaffinity(0)))
    return min(threads, len(os.sched_getaffinity(0)))


def bench_batch(wl, name, steps, warmup, copies, calibrate_copy=False):
    """Time `steps` layer steps over one fixed hybrid batch; returns the
    result line (without cpu_baseline)."""
    import torch
    from chunked_prefill_hybrid_layer_amd import hb
    from chunked_prefill_hybrid_layer_amd.runtime import DeviceLayer, stream_handle

    d, b = wl.dims, wl.batch
    T = b.n_tokens
    max_pos = int(np.max(b.cached_lengths() + b.new_lengths())) + 1
    layers = []
    for _ in range(copies):
        L = DeviceLayer(d, wl.weights, b.num_pages, max_pos)
        L.fill_prefixes(b.block_table, range(b.n_seq), wl.prefix_k, wl.prefix_v)
        layers.append(L)
    hd = hb.make_dims(d)
    x = torch.from_numpy(wl.x).cuda()
    y = torch.empty_like(x)
    # metadata: a ring of pinned host blobs and device blobs
    RING, REC = 32, 16
    blob0 = hb.pack_metadata(hd, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.num_pages,
                             b.token_budget)[0]
    size = blob0.nbytes
    pin = [torch.empty(size, dtype=torch.uint8, pin_memory=True) for _ in range(RING)]
    pin_np = [p.numpy() for p in pin]
    dev = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(RING)]
    ws = torch.empty(hb.workspace_bytes(hd, blob0), dtype=torch.uint8, device="cuda")
    stream = stream_handle()
    # per-step host work is one C call each for packing and for the forward
    packers = [hb.Packer(hd, b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.num_pages,
                         b.token_budget, pin_np[j]) for j in range(RING)]
    fwds = [[hb.Forward(hd, L.hw, pin_np[j], dev[j].data_ptr(), L.rope.data_ptr(), L.rope_max_pos, x.data_ptr(),
                        y.data_ptr(), L.k_cache.data_ptr(), L.v_cache.data_ptr(), ws.data_ptr(), ws.numel(), stream)
             for j in range(RING)] for L in layers]
    # Step s packs its metadata into pinned buffer s % RING and copies it to
    # device buffer s % RING on its own stream, one step ahead.  The compute
    # stream never waits on that stream: the host confirms the copy has
    # completed before it enqueues the step's forward.  A device buffer is
    # refilled only after the forward that read it RING steps earlier has
    # finished: the compute stream records an event after every REC-th forward
    # (each packet between two kernels leaves a bubble of about 6-8 us, so not
    # after every one: every 16th costs about 0.4 us a step), and the copy
    # waits for the first one at or after it.
    compute = torch.cuda.current_stream()
    upload = torch.cuda.Stream()
    copied = [torch.cuda.Event() for _ in range(RING)]
    for e in copied:
        e.record(upload)
    done = {}

    def upload_step(s):
        j = s % RING
        copied[j].synchronize()                # the copy that last read pinned buffer j is done
        packers[j]()
        if s >= RING:
            upload.wait_event(done[(s - RING) // REC])
        with torch.cuda.stream(upload):
            dev[j].copy_(pin[j], non_blocking=True)
        copied[j].record(upload)

    def forward_step(s, events=None):
        j = s % RING
        copied[j].synchronize()                # this step's metadata is on the device
        fwds[s % len(layers)][j](events)
        if s % REC == REC - 1:
            ev = torch.cuda.Event()
            ev.record(compute)
            done[s // REC] = ev
            done.pop(s // REC - RING // REC - 2, None)

    s_next = 0
    upload_step(0)

    def run_step(events=None):
        nonlocal s_next
        upload_step(s_next + 1)
        forward_step(s_next, events)
        s_next += 1

    # The GPU leaves its idle power state over the first ~15 ms under load; a
    # run whose warm-up is shorter times that ramp (--warmup 5 --steps 20
    # measured 0.386-0.394 ms per step against 0.356 ms steady, and the same
    # after 0.5 s of idle following a longer warm-up).  Untimed forwards keep
    # the device busy for SETTLE_MS before the warm-up steps.
    settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - settle0 < SETTLE_MS * 1e-3:
        for _ in range(8):
            run_step()
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        run_step()
    torch.cuda.synchronize()
    nst = hb.NUM_STAGES
    model = stage_model(wl)
    w8a8 = bool(getattr(d, "w8a8", 0))
    # projections (and attention's QK/PV) on MFMA: the projections' peak sets the
    # roofline of MFMA-bound stages (attention stays bf16; its stages are not
    # the dominant ones in either precision)
    peak_mfma = PEAK_FP8_TFLOPS if w8a8 else PEAK_BF16_TFLOPS

    def t_ideal(sname):
        fl, by, _ = model[sname]
        return max(fl / (peak_mfma * 1e12), by / (PEAK_HBM_GBS * 1e9))

    # The dominant kernel (the stage with the largest roofline time) is timed
    # live in the timed region: on every STAGE_EVERY-th timed step, two HIP
    # events bracket that stage alone (each event recorded between two kernels
    # leaves a gap of about 6 us on the stream, so only two, and not on every
    # step).  The breakdown of all stages comes from a separate pass afterwards.
    dom = max(hb.STAGE_NAMES, key=t_ideal)
    kd = hb.STAGE_NAMES.index(dom)
    inst = [i for i in range(steps) if i % STAGE_EVERY == STAGE_EVERY - 1] or [steps - 1]
    dom_ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in inst}
    for e0, e1 in dom_ev.values():   # torch creates the hipEvent on first record
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    ev_arrays = {i: hb.make_events([None] * kd + [e0.cuda_event, e1.cuda_event] + [None] * (nst - kd - 1))
                 for i, (e0, e1) in dom_ev.items()}
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    host_s = np.zeros(steps)
    t_start.record()
    for i in range(steps):
        h0 = time.perf_counter()
        run_step(ev_arrays.get(i))
        host_s[i] = time.perf_counter() - h0
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / steps
    dom_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in dom_ev.values()]))
    if calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.int32, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    # step-time distribution: a separate, untimed pass with an event at every
    # step boundary (each adds its own bubble to the step it opens)
    NPCT = 32
    pct_ev = [torch.cuda.Event(enable_timing=True) for _ in range(NPCT + 1)]
    for i in range(NPCT):
        pct_ev[i].record()
        run_step()
    pct_ev[NPCT].record()
    torch.cuda.synchronize()
    step_ms = np.array([pct_ev[i].elapsed_time(pct_ev[i + 1]) for i in range(NPCT)])
    # stage breakdown: a separate pass with every stage's events on every step
    NBRK = 8
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(NBRK)]
    for row in bev:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    barr = [hb.make_events([e.cuda_event for e in row]) for row in bev]
    for i in range(NBRK):
        run_step(barr[i])
    torch.cuda.synchronize()
    brk_ms = np.array([bev[i][0].elapsed_time(bev[i][nst]) for i in range(NBRK)])
    stage_ms = np.array([[bev[i][k].elapsed_time(bev[i][k + 1]) for k in range(nst)] for i in range(NBRK)])
    stage_mean = stage_ms.mean(axis=0)

    # A split O projection's reduce applies the FFN RMSNorm and is timed with
    # the O stage; the norm's own stage is then empty, and its bytes go to O.
    i_norm, i_o = hb.STAGE_NAMES.index("rmsnorm_ffn"), hb.STAGE_NAMES.index("o_proj_residual")
    if stage_mean[i_norm] < 1e-3:
        fo, bo, so = model["o_proj_residual"]
        model["o_proj_residual"] = (fo, bo + model["rmsnorm_ffn"][1], so)
        model["rmsnorm_ffn"] = (0, 0, "hbm")
    stages = {}
    t_roof = 0.0
    for k, sname in enumerate(hb.STAGE_NAMES):
        fl, by, bound = model[sname]
        t = float(stage_mean[k]) * 1e-3
        ti = t_ideal(sname)
        t_roof += ti
        stages[sname] = {"ms": round(float(stage_mean[k]), 5),
                         "tflops": round(fl / t / 1e12, 2) if t > 1e-7 else None,
                         "gbs": round(by / t / 1e9, 1) if t > 1e-7 else None, "bound": bound,
                         "roofline_frac": round(ti / t, 4) if t > 1e-7 else None}
    fl, by, bound = model[dom]
    tdom = dom_ms * 1e-3
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(fl / tdom / 1e12, 2), "peak": peak_mfma,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(by / tdom / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom, name)
    roof["kernel"] = dom
    roof["per_launch"] = {"flops": fl, "bytes": by}
    roof["timed_launches"] = len(dom_ev)
    roof["longest_stage_in_breakdown"] = max(hb.STAGE_NAMES, key=lambda n: stages[n]["ms"])

    return {
        "metric": "hybrid-layer tokens/s at tau=512 (Mistral-7B-shaped layer) + % of MFMA/HBM roofline",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "settle_forwards": n_settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 projections, bf16 attention" if w8a8 else "bf16",
        "data": "synthetic",
        "config": {"workload": name, "hidden": d.hidden, "n_q_heads": d.n_q_heads,
                   "n_kv_heads": d.n_kv_heads, "head_dim": d.head_dim, "ffn_dim": d.ffn_dim,
                   "tokens": T, "chunks": [int(c) for c in b.chunk_len],
                   "chunk_prefix": [int(c) for c in b.chunk_prefix], "decodes": b.n_decodes,
                   "decode_ctx_mean": float(np.mean(b.decode_ctx)) if b.n_decodes else 0.0,
                   "token_budget": b.token_budget, "page_size": d.page_size, "copies_rotated": copies,
                   "kv_cache": ("fp8_e4m3 (k_scale %g, v_scale %g)" % (d.k_scale, d.v_scale)) if d.kv_fp8
                   else "bf16",
                   "projections": ("fp8_e4m3 (row-scaled weights, input scales %g/%g/%g/%g)" %
                                   (d.x_scale, d.o_scale, d.h_scale, d.a_scale)) if w8a8 else "bf16"},
        "layer_iters_per_s": round(1e3 / ms, 1),
        "layer_roofline_frac": round(t_roof / (ms * 1e-3), 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)],
        "step_ms_note": "p10/p50/p90 from a separate pass of %d steps with an event at every step boundary" % NPCT,
        "breakdown_step_ms_p50": round(float(np.median(brk_ms)), 5),
        "breakdown_steps": NBRK,
        "host_issue_ms_p50": round(float(np.median(host_s)) * 1e3, 4),
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "stages": stages,
    }


def sclk_mhz():
    """Current shader clock of cuda:0 from the driver's sysfs table (the entry
    marked '*' in pp_dpm_sclk of the device's PCI function), or None.  Read as
    a file: no helper program is started."""
    import torch
    try:
        pr = torch.cuda.get_device_properties(0)
        dev = "%04x:%02x:%02x.0" % (getattr(pr, "pci_domain_id", 0), pr.pci_bus_id, pr.pci_device_id)
        with open(os.path.join("/sys/bus/pci/devices", dev, "pp_dpm_sclk")) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return line.split(":", 1)[1].replace("*", "").strip()
    except Exception:
        return None
    return None


TAU_SWEEP = (128, 256, 512, 1024, 2048)


def sweep_tau(args):
    """Token-budget sweep on the Mistral-7B-shaped layer: one chunk of tau-64
    tokens (prefix 1792) + 64 decodes per point.  One line per tau, then a
    summary with the GEMM stages' time per token against the weight-streaming
    and MFMA bounds, which locates the compute/bandwidth knee."""
    from chunked_prefill_hybrid_layer_amd import workloads as W
    points = []
    gemm = ("qkv_rope_append", "o_proj_residual", "gate_up_swiglu", "down_residual")
    suffix = ("_w8a8" if args.w8a8 else "") + ("_kvfp8" if args.kv_fp8 else "")

    def variant(wl):
        if args.w8a8:
            wl = W.with_w8a8(wl)
        if args.kv_fp8:
            wl = W.with_kv_fp8(wl)
        return wl
    wbytes = 1 if args.w8a8 else 2
    peak = PEAK_FP8_TFLOPS if args.w8a8 else PEAK_BF16_TFLOPS
    # a discarded first point: clocks settle during the first few hundred steps of a process
    bench_batch(variant(W.tau_sweep(TAU_SWEEP[0], 0)), "warm-up", args.steps, args.warmup, 1)
    for tau in TAU_SWEEP:
        wl = variant(W.tau_sweep(tau, 0))
        out = bench_batch(wl, f"tau_sweep_{tau}{suffix}", args.steps, args.warmup, args.copies)
        out["metric"] = "hybrid-layer tokens/s, token-budget sweep (Mistral-7B-shaped layer)"
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(wl, stride=max(1, tau // 512))
        print(json.dumps(out), flush=True)
        d = wl.dims
        psi = d.hidden * (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim + d.n_q_heads * d.head_dim * d.hidden + \
            3 * d.hidden * d.ffn_dim
        t_gemm = sum(out["stages"][g]["ms"] for g in gemm) * 1e-3
        points.append({"tau": tau, "tokens_per_s": out["value"], "ms_per_step": out["ms_per_step"],
                       "gemm_ms": round(t_gemm * 1e3, 4),
                       "gemm_tflops": round(2 * tau * psi / t_gemm / 1e12, 1),
                       "gemm_weight_gbs": round(wbytes * psi / t_gemm / 1e9, 1),
                       "gemm_bound_ms": round(max(wbytes * psi / (PEAK_HBM_GBS * 1e9),
                                                  2 * tau * psi / (peak * 1e12)) * 1e3, 4)})
    # algorithmic knee: n* = bytes_w * FLOPS / (2 BW) (bf16: 2 bytes at 2.5 PFLOP/s;
    # FP8: 1 byte at 5.0 PFLOP/s -- the same n*)
    knee = wbytes * peak * 1e12 / (2 * PEAK_HBM_GBS * 1e9)
    print(json.dumps({"metric": "tau sweep summary" + (" (" + suffix[1:] + ")" if suffix else ""), "points": points,
                      "knee_tokens_algorithmic": round(knee, 1)}), flush=True)


def kv_append_bench(args, n_tokens=32768):
    """hb_kv_append of one n_tokens-token prompt (prefix 0) into a shuffled page
    pool: achieved GB/s over read + write of K and V."""
    import torch
    from chunked_prefill_hybrid_layer_amd import hb
    from chunked_prefill_hybrid_layer_amd import workloads as W
    from chunked_prefill_hybrid_layer_amd.runtime import DeviceLayer, stream_handle
    d = W.MISTRAL
    bt, num_pages = W.deal_block_tables(np.array([n_tokens]), d.page_size, np.random.default_rng(0))
    hd = hb.make_dims(d)
    blob, T = hb.pack_metadata(hd, [n_tokens], [0], [], bt, num_pages, n_tokens)
    meta = torch.from_numpy(blob).cuda()
    k = torch.randint(-2**15, 2**15, (T, d.n_kv_heads * d.head_dim), dtype=torch.int16, device="cuda")
    v = torch.randint(-2**15, 2**15, (T, d.n_kv_heads * d.head_dim), dtype=torch.int16, device="cuda")
    caches = []
    for _ in range(2):
        caches.append((torch.empty((num_pages, d.n_kv_heads, d.page_size, d.head_dim), dtype=torch.int16,
                                   device="cuda"),
                       torch.empty((num_pages, d.n_kv_heads, d.head_dim, d.page_size), dtype=torch.int16,
                                   device="cuda")))
    st = stream_handle()

    def run(i):
        kc, vc = caches[i & 1]
        hb.kv_append(hd, blob, meta.data_ptr(), k.data_ptr(), v.data_ptr(), k.stride(0), kc.data_ptr(),
                     vc.data_ptr(), st)

    for i in range(args.warmup):
        run(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    by = 2 * 2 * T * d.n_kv_heads * d.head_dim * 2       # K and V, read and write, bf16
    print(json.dumps({"metric": "kv_append GB/s (one 32768-token prompt, Mistral-7B kv shape)",
                      "value": round(by / us / 1e3, 1), "unit": "GB/s", "us_per_launch": round(us, 2),
                      "bytes_per_launch": by, "tokens": T, "steps": args.steps, "warmup": args.warmup,
                      "roofline": {"bound": "hbm", "achieved": round(by / us / 1e3, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                                   "traffic": None}}), flush=True)


def _stage_events(n):
    import torch
    from chunked_prefill_hybrid_layer_amd import hb
    nst = hb.NUM_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(n)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    return evs, [hb.make_events([e.cuda_event for e in row]) for row in evs]


def _run_chunked(lp, with_decodes=True):
    """All iterations of a LongPrompt on a fresh layer, metadata and inputs
    staged on the device first; one untimed pass, then a timed one.  Returns
    (total ms, per-stage ms summed over iterations, prompt rows of y)."""
    import torch
    from chunked_prefill_hybrid_layer_amd import hb
    from chunked_prefill_hybrid_layer_amd.runtime import DeviceLayer
    d, C = lp.dims, lp.chunk
    max_pos = int(max(lp.prompt_len, int(np.max(lp.decode_ctx0, initial=0)) + lp.n_iter)) + 1
    layer = DeviceLayer(d, lp.weights, lp.num_pages, max_pos)
    if lp.n_dec:
        layer.fill_prefixes(lp.block_table, range(1, 1 + lp.n_dec), lp.prefix_k, lp.prefix_v)
    preps, xs = [], []
    for i in range(lp.n_iter):
        b = lp.batch(i)
        preps.append(layer.prepare(b.chunk_len, b.chunk_prefix, b.decode_ctx, b.block_table, b.token_budget))
        xs.append(torch.from_numpy(lp.x(i)).cuda())
    ys = [torch.empty_like(x) for x in xs]
    ev, arr = _stage_events(lp.n_iter)
    nst = hb.NUM_STAGES

    def go(events=None):
        for i in range(lp.n_iter):
            layer.forward(preps[i], xs[i], ys[i], None if events is None else events[i])

    go()                              # warm-up (rewrites the same K/V values)
    torch.cuda.synchronize()
    # the total comes from a pass without stage events (each leaves a bubble of
    # about 6 us between kernels); the stage split from a second, instrumented one
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    go()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    go(arr)
    torch.cuda.synchronize()
    st = np.array([[ev[i][k].elapsed_time(ev[i][k + 1]) for k in range(nst)] for i in range(lp.n_iter)])
    y = torch.cat([y[:C] for y in ys]).cpu().numpy()
    del layer, xs, ys
    torch.cuda.empty_cache()
    return ms, st.sum(axis=0), y


def _run_unchunked(lp):
    import torch
    from chunked_prefill_hybrid_layer_amd import hb
    from chunked_prefill_hybrid_layer_amd.runtime import DeviceLayer
    d, L = lp.dims, lp.prompt_len
    layer = DeviceLayer(d, lp.weights, lp.num_pages, L + 1)
    ub = lp.unchunked_batch()
    prep = layer.prepare(ub.chunk_len, ub.chunk_prefix, ub.decode_ctx, ub.block_table, ub.token_budget)
    x = torch.from_numpy(lp.prompt_x).cuda()
    y = torch.empty_like(x)
    ev, arr = _stage_events(1)
    nst = hb.NUM_STAGES
    layer.forward(prep, x, y)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    layer.forward(prep, x, y)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    layer.forward(prep, x, y, arr[0])
    torch.cuda.synchronize()
    st = np.array([ev[0][k].elapsed_time(ev[0][k + 1]) for k in range(nst)])
    out = y.cpu().numpy()
    del layer, x, y
    torch.cuda.empty_cache()
    return ms, st, out


def _long_prompt_cpu_baseline(lp, n_rows=24):
    """Row-sampled oracle on the unchunked prompt: K/V of all its tokens, then
    attention and FFN for n_rows rows spread over the prompt."""
    from oracle import hybrid_layer as O
    L = lp.prompt_len
    rows = np.unique(np.linspace(0, L - 1, n_rows).astype(np.int64))
    cache = O.PagedCache(lp.num_pages, lp.dims.n_kv_heads, lp.dims.page_size, lp.dims.head_dim)
    w = O.weights_to_float(lp.weights)
    t0 = time.perf_counter()
    O.layer_forward(lp.dims, w, lp.prompt_x.astype(np.float64), [L], [0], [],
                    np.ascontiguousarray(lp.block_table[:1]), cache, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s (row-sampled)", "cores": _oracle_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"{len(rows)} rows spread over the {L}-token prompt (K/V for all {L} tokens), float64 numpy "
                      f"oracle, {dt:.1f} s; a full {L}-row oracle pass would take about "
                      f"{dt * L / len(rows) / 3600:.1f} h at this rate (an upper bound: K/V are shared)"}


def long_prompt_bench(args):
    """A 32768-token prompt as 64 chunks of 512 co-batched with 64 decodes,
    against one unchunked 32768-token prefill: end-to-end time, the
    attention stages' time (same (query, key) pairs in both), and agreement of
    the prompt rows."""
    from chunked_prefill_hybrid_layer_amd import hb
    from chunked_prefill_hybrid_layer_amd import workloads as W
    lp = W.long_prompt(0)
    d, L, C = lp.dims, lp.prompt_len, lp.chunk
    ms_c, st_c, y_chunk = _run_chunked(lp)
    ms_u, st_u, y_full = _run_unchunked(lp)
    rel = float(np.linalg.norm(y_chunk.astype(np.float64) - y_full) / np.linalg.norm(y_full.astype(np.float64)))
    mx = float(np.max(np.abs(y_chunk - y_full)))
    names = list(hb.STAGE_NAMES)
    ia = names.index("attn_chunk")
    pairs = L * (L + 1) // 2
    attn_c, attn_u = float(st_c[ia]), float(st_u[ia])
    out = {
        "metric": "long-prompt chunking: 32768-token prompt as 64 chunks of 512 (+64 decodes each) vs unchunked",
        "chunked_ms_total": round(ms_c, 3), "chunked_ms_per_iteration": round(ms_c / lp.n_iter, 4),
        "chunked_tokens_per_s": round(lp.n_iter * (C + lp.n_dec) / (ms_c * 1e-3), 1),
        "unchunked_ms": round(ms_u, 3), "unchunked_tokens_per_s": round(L / (ms_u * 1e-3), 1),
        "prompt_attention_pairs": pairs,
        "attn_chunk_ms": {"chunked_sum": round(attn_c, 3), "unchunked": round(attn_u, 3),
                          "recompute_overhead": round(attn_c / attn_u - 1.0, 4),
                          "chunked_tflops": round(4 * pairs * d.n_q_heads * d.head_dim / (attn_c * 1e-3) / 1e12, 1),
                          "unchunked_tflops": round(4 * pairs * d.n_q_heads * d.head_dim / (attn_u * 1e-3) / 1e12, 1)},
        "stage_ms": {n: {"chunked_sum": round(float(st_c[k]), 3), "unchunked": round(float(st_u[k]), 3)}
                     for k, n in enumerate(names)},
        "prompt_rows_chunked_vs_unchunked": {"rel_l2": rel, "max_abs": mx},
        "dtype": "bf16", "data": "synthetic", "n_gpus": 1}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _long_prompt_cpu_baseline(lp)
    print(json.dumps(out), flush=True)


CHUNK_SWEEP = (128, 256, 512, 1024, 2048)


def chunk_sweep_bench(args):
    """The 32768-token prompt alone, chunked at C in 128 .. 2048, against the
    unchunked prefill: the chunk-attention stage summed over the iterations
    (identical (query, key) pairs at every C) and the whole prompt's time."""
    from chunked_prefill_hybrid_layer_amd import hb
    from chunked_prefill_hybrid_layer_amd import workloads as W
    names = list(hb.STAGE_NAMES)
    ia = names.index("attn_chunk")
    base = W.long_prompt(0, n_dec=0)
    ms_u, st_u, y_full = _run_unchunked(base)
    attn_u = float(st_u[ia])
    pts = []
    for C in (args.chunk_sizes or CHUNK_SWEEP):
        lp = W.long_prompt(0, chunk=C, n_dec=0)
        ms_c, st_c, y = _run_chunked(lp)
        rel = float(np.linalg.norm(y.astype(np.float64) - y_full) / np.linalg.norm(y_full.astype(np.float64)))
        pts.append({"chunk": C, "iterations": lp.n_iter, "prompt_ms": round(ms_c, 3),
                    "attn_chunk_ms": round(float(st_c[ia]), 3),
                    "recompute_overhead": round(float(st_c[ia]) / attn_u - 1.0, 4),
                    "attn_merge_ms": round(float(st_c[names.index("attn_merge")]), 3),
                    "gemm_ms": round(float(sum(st_c[names.index(n)] for n in
                                             ("qkv_rope_append", "o_proj_residual", "gate_up_swiglu",
                                              "down_residual"))), 3),
                    "rel_l2_vs_unchunked": rel})
        print(json.dumps({"metric": "chunk-size sweep, 32768-token prompt", **pts[-1]}), flush=True)
    print(json.dumps({"metric": "chunk-size sweep summary (32768-token prompt, Mistral-7B-shaped layer)",
                      "unchunked_ms": round(ms_u, 3), "unchunked_attn_chunk_ms": round(attn_u, 3),
                      "points": pts}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mistral_tau512")
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="FP8 e4m3 KV cache (k_scale 2^-4, v_scale 2^-3) instead of bf16")
    ap.add_argument("--w8a8", action="store_true",
                    help="FP8 e4m3 projections (weights and their inputs) on the FP8 MFMA")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy 256 MiB device-to-device once (counter calibration)")
    ap.add_argument("--sweep-tau", action="store_true", help="token-budget sweep, one line per tau")
    ap.add_argument("--kv-append", action="store_true", help="hb_kv_append GB/s on a 32768-token prompt")
    ap.add_argument("--long-prompt", action="store_true",
                    help="32768-token prompt: 64 chunks of 512 with 64 decodes vs unchunked")
    ap.add_argument("--chunk-sizes", type=lambda v: [int(c) for c in v.split(",")], default=None,
                    help="chunk sizes of --chunk-sweep (comma-separated; default 128,256,512,1024,2048)")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="32768-token prompt alone at chunk sizes 128 .. 2048 vs unchunked")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the hybrid-batch layer runs on one GPU; --gpus above 1 is not supported "
                                   "(data-parallel replicas would each run their own batches, weights and "
                                   "KV pool with no exchange)"}))
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.sweep_tau:
        return sweep_tau(args)
    if args.kv_append:
        return kv_append_bench(args)
    if args.long_prompt:
        return long_prompt_bench(args)
    if args.chunk_sweep:
        return chunk_sweep_bench(args)
    wl = workload_by_name(args.workload)
    name = args.workload
    from chunked_prefill_hybrid_layer_amd import workloads as W
    if args.w8a8:
        wl = W.with_w8a8(wl)
        name += "_w8a8"
    if args.kv_fp8:
        wl = W.with_kv_fp8(wl)
        name += "_kvfp8"
    out = bench_batch(wl, name, args.steps, args.warmup, args.copies, args.calibrate_copy)
    out["sclk_mhz"] = sclk_mhz()
    if not args.no_cpu_baseline:
        if args.workload == "tiny":
            out["cpu_baseline"] = cpu_baseline_whole(wl)
        else:
            # about 10 s of oracle work on a 16-core host
            out["cpu_baseline"] = cpu_baseline(wl, stride=1 if wl.batch.n_tokens <= 1024 else 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
