"""Summaries of rocprofv3 output for the layer's kernels.

    # per-kernel durations (from --kernel-trace --stats CSV output)
    python -m chunked_prefill_hybrid_layer_amd.profiling stats <dir>/<run>_kernel_stats.csv

    # per-phase kernel time of a run made of several batches (bench.py
    # --long-prompt / --chunk-sweep): the trace is cut into layer forwards
    # (each starts with the RMSNorm that feeds the QKV projection); a phase
    # NAME:NxP is P passes of N forwards, of which the middle one is summed
    python -m chunked_prefill_hybrid_layer_amd.profiling phases <dir>/<run>_kernel_trace.csv NAME:NxP ...

    # the launches of one forward in order, each with its median duration over
    # the forwards of the trace that run the same launch sequence (the
    # projections O and down share a kernel; their order tells them apart)
    python -m chunked_prefill_hybrid_layer_amd.profiling sequence <dir>/<run>_kernel_trace.csv

    # HBM bytes per launch from two --pmc runs (FETCH_SIZE, then WRITE_SIZE),
    # scaled by what the same counters read for the plain 256 MiB copy that
    # `bench.py --calibrate-copy` issues
    python -m chunked_prefill_hybrid_layer_amd.profiling traffic FETCH.csv WRITE.csv [--json-for WORKLOAD]

The counters report KiB per dispatch; the copy reads and writes exactly
COPY_BYTES, which turns each counter into bytes (factor = COPY_BYTES /
(counter KiB * 1024)).
"""
from __future__ import annotations

import collections
import csv
import sys

COPY_BYTES = 256 << 20
COPY_KERNEL_HINTS = ("copyBuffer", "copy_kernel", "CatArrayBatchedCopy", "vectorized_elementwise_kernel")

LAYER_KERNELS = {
    "rmsnorm_kernel": "rmsnorm",
    "gemm_kernel<0": "qkv_rope_append",
    "gemm_sub_kernel<0": "qkv_rope_append",
    "gemm_spec_kernel<0": "qkv_rope_append",
    "gemm_specw_kernel<0": "qkv_rope_append",
    "gemm_f8w_kernel<0": "qkv_rope_append",
    "qkv_reduce_kernel": "qkv_split_reduce",
    "attn_chunk_kernel": "attn_chunk",
    "attn_decode_kernel": "attn_decode",
    "attn_merge_kernel": "attn_merge",
    "gemm_kernel<1": "o_proj / down (residual)",
    "gemm_sub_kernel<1": "o_proj / down (residual)",
    "gemm_spec_kernel<1": "o_proj / down (residual)",
    "gemm_specw_kernel<1": "o_proj / down (residual)",
    "gemm_f8w_kernel<1": "o_proj / down (residual)",
    "splitk_reduce_kernel": "split-K reduce (+rmsnorm)",
    "gemm_kernel<2": "gate_up_swiglu",
    "gemm_sub_kernel<2": "gate_up_swiglu",
    "gemm_spec_kernel<2": "gate_up_swiglu",
    "gemm_specw_kernel<2": "gate_up_swiglu",
    "gemm_f8w_kernel<2": "gate_up_swiglu",
    "kv_append_kernel": "kv_append",
}


def short_name(kernel: str) -> str:
    for k, v in LAYER_KERNELS.items():
        if k in kernel:
            return v
    return kernel[:48]


def kernel_stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        calls = int(r["Calls"])
        avg = float(r["AverageNs"]) / 1e3
        tot = float(r["TotalDurationNs"]) / 1e3
        pct = float(r.get("Percentage", 0.0))
        out.append(f"| {short_name(name)} (`{name[:70]}`) | {calls} | {avg:.2f} | {tot:.1f} | {pct:.2f} |")
    return "\n".join(out)


def forwards(trace_csv: str):
    """Layer forwards of a kernel trace, in time order: lists of (short
    name, duration us, start ns).  A forward starts at an RMSNorm launch
    directly followed by a QKV projection launch; launches of other kernels
    (copies, fills) are left out."""
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    ks = [(short_name(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3,
           int(r["Start_Timestamp"])) for r in rows]
    ks = [k for k in ks if k[0] in set(LAYER_KERNELS.values())]
    out = []
    for i, k in enumerate(ks):
        if k[0] == "rmsnorm" and i + 1 < len(ks) and ks[i + 1][0] == "qkv_rope_append":
            out.append([])
        if out:
            out[-1].append(k)
    return out


def phases(trace_csv: str, specs):
    fw = forwards(trace_csv)
    need = sum(n * p for _, n, p in specs)
    if need != len(fw):
        raise SystemExit(f"trace holds {len(fw)} forwards, the phases describe {need}")
    lines = ["| phase | forwards | span ms | " + " | ".join(sorted(set(LAYER_KERNELS.values()))) + " |",
             "|---|---:|---:|" + "---:|" * len(set(LAYER_KERNELS.values()))]
    names = sorted(set(LAYER_KERNELS.values()))
    i = 0
    res = {}
    for name, n, p in specs:
        passes = [fw[i + j * n:i + (j + 1) * n] for j in range(p)]
        i += n * p
        mid = passes[p // 2]
        tot = collections.defaultdict(float)
        for f in mid:
            for k, d, _ in f:
                tot[k] += d
        span = (mid[-1][-1][2] + mid[-1][-1][1] * 1e3 - mid[0][0][2]) / 1e6
        res[name] = dict(tot)
        lines.append(f"| {name} | {n} | {span:.3f} | " + " | ".join(f"{tot.get(k, 0.0) / 1e3:.3f}" for k in names) + " |")
    return "\n".join(lines), res


def sequence(trace_csv: str) -> str:
    fw = forwards(trace_csv)
    if not fw:
        return "no layer forward found in the trace (an RMSNorm launch followed by a QKV projection)"
    seqs = collections.Counter(tuple(k for k, _, _ in f) for f in fw)
    common, n = seqs.most_common(1)[0]
    same = [f for f in fw if tuple(k for k, _, _ in f) == common]
    lines = [f"{n} of {len(fw)} forwards run this launch sequence; median over them (us)", "",
             "| # | kernel | median us |", "|---:|---|---:|"]
    total = 0.0
    for i, k in enumerate(common):
        d = sorted(f[i][1] for f in same)
        med = d[len(d) // 2]
        total += med
        lines.append(f"| {i} | {k} | {med:.2f} |")
    lines.append(f"| | sum | {total:.2f} |")
    return "\n".join(lines)


def _per_kernel(path: str, counter: str):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv: str, write_csv: str):
    """Mean bytes per launch (read, write) per kernel, copy-calibrated."""
    f = _per_kernel(fetch_csv, "FETCH_SIZE")
    w = _per_kernel(write_csv, "WRITE_SIZE")
    copy = [k for k in f if any(h in k for h in COPY_KERNEL_HINTS)]
    if not copy:
        raise SystemExit("no copy dispatch found for calibration")
    # the largest copy dispatch is the 256 MiB calibration copy
    ck = max(copy, key=lambda k: max(f[k]))
    fk = COPY_BYTES / (max(f[ck]) * 1024.0)
    wk = COPY_BYTES / (max(w[ck]) * 1024.0) if ck in w and max(w[ck]) > 0 else 1.0
    res = {}
    for k in f:
        rd = sum(f[k]) / len(f[k]) * 1024.0 * fk
        wr = (sum(w[k]) / len(w[k]) * 1024.0 * wk) if k in w else 0.0
        res[k] = {"read_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr, "launches": len(f[k])}
    return res, {"copy_kernel": ck, "fetch_factor": fk, "write_factor": wk}


# kernels whose launches map to exactly one layer stage (name fragment -> stage, source)
STAGE_OF_KERNEL = {
    "gemm_kernel<2": ("gate_up_swiglu", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_sub_kernel<2": ("gate_up_swiglu", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_spec_kernel<2": ("gate_up_swiglu", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_specw_kernel<2": ("gate_up_swiglu", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_f8w_kernel<2": ("gate_up_swiglu", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_kernel<0": ("qkv_rope_append", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_sub_kernel<0": ("qkv_rope_append", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_spec_kernel<0": ("qkv_rope_append", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_specw_kernel<0": ("qkv_rope_append", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "gemm_f8w_kernel<0": ("qkv_rope_append", "chunked_prefill_hybrid_layer_amd/csrc/gemm.hip"),
    "attn_chunk_kernel": ("attn_chunk", "chunked_prefill_hybrid_layer_amd/csrc/attention.hip"),
    "attn_decode_kernel": ("attn_decode", "chunked_prefill_hybrid_layer_amd/csrc/attention.hip"),
    "attn_merge_kernel": ("attn_merge", "chunked_prefill_hybrid_layer_amd/csrc/attention.hip"),
}


def write_traffic_json(res, cal, workload: str, path: str, root: str):
    import hashlib
    import json
    import os
    data = json.load(open(path)) if os.path.exists(path) else {}
    entry = data.setdefault(workload, {})
    for k, v in res.items():
        for frag, (stage, src) in STAGE_OF_KERNEL.items():
            if frag in k:
                h = hashlib.sha256(open(os.path.join(root, src), "rb").read()).hexdigest()[:16]
                entry[stage] = {"bytes_per_launch": round(v["bytes_per_launch"]),
                                "read_bytes": round(v["read_bytes"]), "write_bytes": round(v["write_bytes"]),
                                "source_hash": h, "calibration": cal}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print(kernel_stats(argv[1]))
    elif len(argv) >= 2 and argv[0] == "sequence":
        print(sequence(argv[1]))
    elif len(argv) >= 3 and argv[0] == "phases":
        specs = []
        for a in argv[2:]:
            name, np_ = a.split(":")
            n, p = np_.split("x")
            specs.append((name, int(n), int(p)))
        print("kernel time summed per phase (ms), middle pass of each phase")
        print(phases(argv[1], specs)[0])
    elif len(argv) >= 3 and argv[0] == "traffic":
        res, cal = traffic(argv[1], argv[2])
        if len(argv) >= 5:   # ... --json-for WORKLOAD: update profiles/traffic.json
            import os
            root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
            write_traffic_json(res, cal, argv[4], os.path.join(root, "profiles", "traffic.json"), root)
        print(f"calibration: {cal}")
        print("| kernel | launches | read MB | write MB | total MB |")
        print("|---|---:|---:|---:|---:|")
        for k, v in sorted(res.items(), key=lambda kv: -kv[1]["bytes_per_launch"]):
            print(f"| {short_name(k)} | {v['launches']} | {v['read_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} | "
                  f"{v['bytes_per_launch'] / 1e6:.2f} |")
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
