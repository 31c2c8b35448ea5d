"""ctypes binding of libhb.so (the C ABI declared in include/hb.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels or its host C++ code.  Importing this module fails loudly if the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

# One HIP runtime per process: torch ships its own libamdhip64, so it is loaded
# first and libhb.so then binds to that same runtime (device pointers and
# streams handed over from torch stay valid).
try:
    import torch  # noqa: F401
except ImportError:  # host-only use (metadata packing) works without torch
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
# HB_LIB_PATH: another build of the same library (the host tests use it for a
# host-sanitized build)
LIB_PATH = os.environ.get("HB_LIB_PATH") or os.path.join(_HERE, "libhb.so")

HB_OK = 0
STATUS_NAMES = ["HB_OK", "HB_E_NULL", "HB_E_SHAPE", "HB_E_LENGTH", "HB_E_BUDGET", "HB_E_PAGE",
                "HB_E_ALIAS", "HB_E_CAPACITY", "HB_E_HIP", "HB_E_META"]
META_MAGIC = 0x31424D48


class HbError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{self.name}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("kv_fp8", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float), ("w8a8", ctypes.c_int32),
                ("x_scale", ctypes.c_float), ("o_scale", ctypes.c_float), ("h_scale", ctypes.c_float),
                ("a_scale", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d", "g_attn", "g_ffn",
                 "s_q", "s_k", "s_v", "s_o", "s_g", "s_u", "s_d")]


class AttnItem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("seq", "tok0", "n_tok", "key0", "key1", "split", "n_split", "reserved")]


class MetaHeader(ctypes.Structure):
    _fields_ = ([("magic", ctypes.c_uint32), ("version", ctypes.c_uint32)] +
                [(n, ctypes.c_int32) for n in
                 ("n_seq", "n_chunks", "n_decodes", "n_tokens", "page_size", "max_pages", "num_pages",
                  "max_kv_len", "n_kv_heads", "group", "head_dim", "n_q_heads", "chunk_q_tile",
                  "chunk_kv_split", "decode_kv_split", "n_chunk_items", "n_decode_items", "n_partials",
                  "n_append_runs", "n_merge_tokens")] +
                [("bytes", ctypes.c_int64)] +
                [(n, ctypes.c_int64) for n in
                 ("off_q_start", "off_cached", "off_kv_len", "off_tok_seq", "off_tok_pos", "off_slot",
                  "off_part_off", "off_part_cnt", "off_block_table", "off_chunk_items", "off_decode_items",
                  "off_append_runs")])


class WorkspaceViews(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("xn", "q", "o", "h1", "h1n", "act")]


class Request(ctypes.Structure):
    _fields_ = [("prompt_len", ctypes.c_int32), ("cached", ctypes.c_int32)]


EXPORTS = ["hb_meta_bytes", "hb_pack_metadata", "hb_schedule_iteration", "hb_rope_table", "hb_workspace_bytes",
           "hb_workspace_views_of", "hb_kv_append", "hb_layer_forward", "hb_layer_forward_static_scratch",
           "hb_status_str", "hb_last_error_detail"]
STATIC_SCRATCH_BYTES = 128 << 20


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m chunked_prefill_hybrid_layer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.hb_meta_bytes.argtypes = [ctypes.POINTER(Dims), I32, I32, I32]
    lib.hb_meta_bytes.restype = SZ
    lib.hb_pack_metadata.argtypes = [ctypes.POINTER(Dims), I32, I32P, I32P, I32, I32P, I32P, I32, I32, I32,
                                     P, SZ, ctypes.POINTER(SZ), I32P]
    lib.hb_pack_metadata.restype = ctypes.c_int
    lib.hb_schedule_iteration.argtypes = [I32, I32, I32, ctypes.POINTER(Request), I32P, I32P, I32P, I32P, I32P,
                                          I32P, I32P]
    lib.hb_schedule_iteration.restype = ctypes.c_int
    lib.hb_rope_table.argtypes = [ctypes.POINTER(Dims), I32, ctypes.POINTER(ctypes.c_float)]
    lib.hb_rope_table.restype = ctypes.c_int
    lib.hb_workspace_bytes.argtypes = [ctypes.POINTER(Dims), P]
    lib.hb_workspace_bytes.restype = SZ
    lib.hb_workspace_views_of.argtypes = [ctypes.POINTER(Dims), P, ctypes.POINTER(WorkspaceViews)]
    lib.hb_workspace_views_of.restype = ctypes.c_int
    lib.hb_kv_append.argtypes = [ctypes.POINTER(Dims), P, P, P, P, I64, P, P, P]
    lib.hb_kv_append.restype = ctypes.c_int
    lib.hb_layer_forward.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), P, P, P, I32, P, P, P, P,
                                     P, SZ, P, ctypes.POINTER(ctypes.c_void_p)]
    lib.hb_layer_forward.restype = ctypes.c_int
    lib.hb_layer_forward_static_scratch.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), P, P, P, I32, P,
                                                    P, P, P, P]
    lib.hb_layer_forward_static_scratch.restype = ctypes.c_int
    lib.hb_status_str.argtypes = [ctypes.c_int]
    lib.hb_status_str.restype = ctypes.c_char_p
    lib.hb_last_error_detail.argtypes = []
    lib.hb_last_error_detail.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(status: int):
    if status != HB_OK:
        raise HbError(status, lib.hb_last_error_detail().decode())


def make_dims(d) -> Dims:
    """hb_dims from any object with the layer-shape attributes."""
    return Dims(d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn_dim, d.page_size,
                float(d.rms_eps), float(d.rope_theta), int(getattr(d, "kv_fp8", 0)),
                float(getattr(d, "k_scale", 1.0)), float(getattr(d, "v_scale", 1.0)),
                int(getattr(d, "w8a8", 0)), *[float(getattr(d, n, 1.0)) for n in
                                              ("x_scale", "o_scale", "h_scale", "a_scale")])


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def meta_bytes(dims: Dims, n_seq: int, n_tokens: int, max_pages: int) -> int:
    return int(lib.hb_meta_bytes(ctypes.byref(dims), n_seq, n_tokens, max_pages))


def pack_metadata(dims: Dims, chunk_len: Sequence[int], chunk_prefix: Sequence[int],
                  decode_ctx: Sequence[int], block_table: np.ndarray, num_pages: int,
                  token_budget: int, capacity: Optional[int] = None,
                  out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, int]:
    """Returns (blob as a uint8 array, packed token count).  With ``out`` (a
    uint8 array, e.g. a pinned buffer) the blob is written there in one call."""
    cl, cp, dc = _i32(chunk_len), _i32(chunk_prefix), _i32(decode_ctx)
    bt = _i32(block_table)
    if bt.ndim != 2:
        raise ValueError("block_table must be 2-D [n_seq][max_pages]")
    need = ctypes.c_size_t(0)
    ntok = ctypes.c_int32(0)
    if out is not None:
        _check(lib.hb_pack_metadata(ctypes.byref(dims), len(cl), _ptr(cl), _ptr(cp), len(dc), _ptr(dc), _ptr(bt),
                                    bt.shape[1], int(num_pages), int(token_budget),
                                    out.ctypes.data_as(ctypes.c_void_p), out.nbytes, ctypes.byref(need),
                                    ctypes.byref(ntok)))
        return out[:need.value], int(ntok.value)
    _check(lib.hb_pack_metadata(ctypes.byref(dims), len(cl), _ptr(cl), _ptr(cp), len(dc), _ptr(dc), _ptr(bt),
                                bt.shape[1], int(num_pages), int(token_budget), None, 0, ctypes.byref(need),
                                ctypes.byref(ntok)))
    cap = need.value if capacity is None else capacity
    blob = np.zeros(max(cap, 1), dtype=np.uint8)
    _check(lib.hb_pack_metadata(ctypes.byref(dims), len(cl), _ptr(cl), _ptr(cp), len(dc), _ptr(dc), _ptr(bt),
                                bt.shape[1], int(num_pages), int(token_budget),
                                blob.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(need),
                                ctypes.byref(ntok)))
    return blob[:need.value], int(ntok.value)


def header(blob: np.ndarray) -> MetaHeader:
    return MetaHeader.from_buffer_copy(blob[:ctypes.sizeof(MetaHeader)].tobytes())


def meta_array(blob: np.ndarray, name: str) -> np.ndarray:
    """int32 array of the blob by header field name (e.g. 'slot', 'tok_pos', 'block_table')."""
    h = header(blob)
    counts = {"q_start": h.n_seq + 1, "cached": h.n_seq, "kv_len": h.n_seq, "tok_seq": h.n_tokens,
              "tok_pos": h.n_tokens, "slot": h.n_tokens, "part_off": h.n_tokens, "part_cnt": h.n_tokens,
              "block_table": h.n_seq * h.max_pages}
    off = getattr(h, "off_" + name)
    return np.frombuffer(blob, dtype=np.int32, count=counts[name], offset=off).copy()


def attn_items(blob: np.ndarray, kind: str) -> np.ndarray:
    h = header(blob)
    n = h.n_chunk_items if kind == "chunk" else h.n_decode_items
    off = h.off_chunk_items if kind == "chunk" else h.off_decode_items
    return np.frombuffer(blob, dtype=np.int32, count=8 * n, offset=off).reshape(n, 8).copy()


def schedule_iteration(token_budget: int, chunk_size: int, prompt_len, cached):
    """hb_schedule_iteration over requests (prompt_len[i], cached[i]); returns
    (chunk_req, chunk_len, chunk_prefix, decode_req, decode_ctx) as int32 arrays."""
    n = len(prompt_len)
    reqs = (Request * max(n, 1))(*[Request(int(p), int(c)) for p, c in zip(prompt_len, cached)])
    outs = [np.zeros(max(n, 1), np.int32) for _ in range(5)]
    nc, nd = ctypes.c_int32(0), ctypes.c_int32(0)
    ptr = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(lib.hb_schedule_iteration(int(token_budget), int(chunk_size), n, reqs, ptr(outs[0]), ptr(outs[1]),
                                     ptr(outs[2]), ctypes.byref(nc), ptr(outs[3]), ptr(outs[4]), ctypes.byref(nd)))
    c, d = nc.value, nd.value
    return outs[0][:c], outs[1][:c], outs[2][:c], outs[3][:d], outs[4][:d]


def append_runs(blob: np.ndarray) -> np.ndarray:
    """KV append runs as an int32 array [n_runs][4] = (tok0, n_tok, slot0, 0)."""
    h = header(blob)
    return np.frombuffer(blob, dtype=np.int32, count=4 * h.n_append_runs, offset=h.off_append_runs).reshape(
        h.n_append_runs, 4).copy()


def rope_table(dims: Dims, max_pos: int) -> np.ndarray:
    out = np.empty((max_pos, dims.head_dim // 2, 2), dtype=np.float32)
    _check(lib.hb_rope_table(ctypes.byref(dims), int(max_pos),
                             out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


def workspace_bytes(dims: Dims, blob: np.ndarray) -> int:
    n = int(lib.hb_workspace_bytes(ctypes.byref(dims), blob.ctypes.data_as(ctypes.c_void_p)))
    if n == 0:
        raise HbError(9, "workspace size query failed: " + lib.hb_last_error_detail().decode())
    return n


def workspace_views(dims: Dims, blob: np.ndarray) -> dict:
    """Byte offsets of the stored activations (xn, q, o, h1, h1n, act) in the workspace."""
    v = WorkspaceViews()
    _check(lib.hb_workspace_views_of(ctypes.byref(dims), blob.ctypes.data_as(ctypes.c_void_p), ctypes.byref(v)))
    return {n: int(getattr(v, n)) for n, _ in WorkspaceViews._fields_}


def kv_append(dims: Dims, blob: np.ndarray, meta_dev: int, k: int, v: int, row_stride: int,
              k_cache: int, v_cache: int, stream: int = 0):
    _check(lib.hb_kv_append(ctypes.byref(dims), blob.ctypes.data_as(ctypes.c_void_p), meta_dev, k, v,
                            int(row_stride), k_cache, v_cache, stream))


NUM_STAGES = 9
STAGE_NAMES = ("rmsnorm_attn", "qkv_rope_append", "attn_chunk", "attn_decode", "attn_merge",
               "o_proj_residual", "rmsnorm_ffn", "gate_up_swiglu", "down_residual")


def layer_forward(dims: Dims, weights: Weights, blob: np.ndarray, meta_dev: int, rope_cs: int,
                  rope_max_pos: int, x: int, y: int, k_cache: int, v_cache: int, workspace: int,
                  workspace_bytes_: int, stream: int = 0, stage_events: Optional[Sequence[int]] = None):
    """stage_events: None, or NUM_STAGES + 1 hipEvent_t handles (e.g. torch.cuda.Event().cuda_event)."""
    ev = None
    if stage_events is not None:
        if len(stage_events) != NUM_STAGES + 1:
            raise ValueError(f"need {NUM_STAGES + 1} stage events")
        ev = (ctypes.c_void_p * len(stage_events))(*stage_events)
    _check(lib.hb_layer_forward(ctypes.byref(dims), ctypes.byref(weights), blob.ctypes.data_as(ctypes.c_void_p),
                                meta_dev, rope_cs, int(rope_max_pos), x, y, k_cache, v_cache, workspace,
                                int(workspace_bytes_), stream, ev))


def layer_forward_static_scratch(dims: Dims, weights: Weights, blob: np.ndarray, meta_dev: int, rope_cs: int,
                                 rope_max_pos: int, x: int, y: int, k_cache: int, v_cache: int, stream: int = 0):
    """hb_layer_forward on the library's static scratch (no workspace argument)."""
    _check(lib.hb_layer_forward_static_scratch(ctypes.byref(dims), ctypes.byref(weights),
                                               blob.ctypes.data_as(ctypes.c_void_p), meta_dev, rope_cs,
                                               int(rope_max_pos), x, y, k_cache, v_cache, stream))


class Packer:
    """hb_pack_metadata bound once to fixed input arrays and an output buffer,
    so that a per-iteration call is one C call (the arrays may be refilled in
    place between calls; their shapes must not change)."""

    def __init__(self, dims: Dims, chunk_len, chunk_prefix, decode_ctx, block_table, num_pages: int,
                 token_budget: int, out: np.ndarray):
        self.arrays = [_i32(chunk_len), _i32(chunk_prefix), _i32(decode_ctx), _i32(block_table)]
        cl, cp, dc, bt = self.arrays
        self.dims, self.out = dims, out
        self.need = ctypes.c_size_t(0)
        self.ntok = ctypes.c_int32(0)
        self.args = (ctypes.byref(dims), len(cl), _ptr(cl), _ptr(cp), len(dc), _ptr(dc), _ptr(bt), bt.shape[1],
                     int(num_pages), int(token_budget), out.ctypes.data_as(ctypes.c_void_p), out.nbytes,
                     ctypes.byref(self.need), ctypes.byref(self.ntok))

    def __call__(self) -> int:
        _check(lib.hb_pack_metadata(*self.args))
        return self.need.value


class Forward:
    """hb_layer_forward bound once to its buffers; call(events) enqueues one
    layer forward (events: None or a ctypes array from make_events)."""

    def __init__(self, dims: Dims, weights: Weights, meta_host: np.ndarray, meta_dev: int, rope_cs: int,
                 rope_max_pos: int, x: int, y: int, k_cache: int, v_cache: int, workspace: int,
                 workspace_bytes_: int, stream: int = 0):
        self.keep = (dims, weights, meta_host)
        self.args = (ctypes.byref(dims), ctypes.byref(weights), meta_host.ctypes.data_as(ctypes.c_void_p),
                     meta_dev, rope_cs, int(rope_max_pos), x, y, k_cache, v_cache, workspace, int(workspace_bytes_),
                     stream)

    def __call__(self, events=None):
        _check(lib.hb_layer_forward(*self.args, events))


def make_events(handles: Sequence[Optional[int]]):
    """ctypes array of NUM_STAGES + 1 hipEvent_t handles for Forward.__call__
    (None entries are not recorded)."""
    if len(handles) != NUM_STAGES + 1:
        raise ValueError(f"need {NUM_STAGES + 1} stage events")
    return (ctypes.c_void_p * len(handles))(*handles)
