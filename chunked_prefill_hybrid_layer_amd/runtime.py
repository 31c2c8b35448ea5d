"""Device-side state for driving the library from Python.

torch provides device memory, host-to-device copies and the stream; every
computation is one of the library's entry points (hb.py).  This module holds
weights, the paged KV cache, the rotary table and the workspace for one layer.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from . import hb

BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
WEIGHT_NAMES = ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d", "g_attn", "g_ffn")
SCALE_NAMES = ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d")   # row scales of FP8 projections


def to_device_u16(a: np.ndarray, device) -> torch.Tensor:
    """uint16 bit patterns -> int16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device)


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def schedule_batch(token_budget: int, chunk_size: int, prompt_len, cached, block_table: np.ndarray,
                   num_pages: int):
    """One stall-free iteration (hb_schedule_iteration) over requests with the
    given prompt lengths and cached token counts, as the arguments of
    hb_pack_metadata: returns (chunk_len, chunk_prefix, decode_ctx,
    block-table rows in packed order, request index of each sequence)."""
    cr, cl, cp, dr, dc = hb.schedule_iteration(token_budget, chunk_size, prompt_len, cached)
    order = np.concatenate([cr, dr]).astype(np.int64)
    return cl, cp, dc, np.ascontiguousarray(block_table[order]), order


@dataclass
class Prepared:
    """A hybrid batch's metadata on host and device."""
    blob: np.ndarray
    meta_dev: torch.Tensor
    n_tokens: int

    @property
    def header(self):
        return hb.header(self.blob)


class DeviceLayer:
    """Weights, paged KV cache (NaN-filled: unwritten slots are poison), rotary
    table and workspace of one decoder layer on one GPU.  With dims.kv_fp8 the
    cache holds one-byte FP8 e4m3 codes (NaN code 0x7F as poison), else bf16."""

    def __init__(self, dims, weights: dict, num_pages: int, rope_max_pos: int, device: str = "cuda"):
        self.dims = dims
        self.hd = hb.make_dims(dims)
        self.device = device
        # bf16 bit patterns; with dims.w8a8 the projections are e4m3 codes
        # (uint8) with float32 row scales under "s_" + name
        self.w = {}
        for n in WEIGHT_NAMES:
            a = weights[n]
            self.w[n] = (torch.from_numpy(np.ascontiguousarray(a)).to(device) if a.dtype == np.uint8
                         else to_device_u16(a, device))
        scales = [0] * len(SCALE_NAMES)
        if getattr(dims, "w8a8", 0):
            for i, n in enumerate(SCALE_NAMES):
                t = torch.from_numpy(np.ascontiguousarray(weights["s_" + n], dtype=np.float32)).to(device)
                self.w["s_" + n] = t
                scales[i] = t.data_ptr()
        self.hw = hb.Weights(*[self.w[n].data_ptr() for n in WEIGHT_NAMES], *scales)
        self.num_pages = int(num_pages)
        # K page blocks are [head_dim/32][page_size][32]; V page blocks [head_dim][page_size]
        self.kv_fp8 = bool(getattr(dims, "kv_fp8", 0))
        fill, dt = (E4M3_NAN, torch.uint8) if self.kv_fp8 else (BF16_NAN, torch.int16)
        self.k_cache = torch.full((self.num_pages, dims.n_kv_heads, dims.head_dim // 32, dims.page_size, 32),
                                  fill, dtype=dt, device=device)
        self.v_cache = torch.full((self.num_pages, dims.n_kv_heads, dims.head_dim, dims.page_size), fill,
                                  dtype=dt, device=device)
        self._np_cache = np.uint8 if self.kv_fp8 else np.uint16
        self.rope_max_pos = int(rope_max_pos)
        self.rope = torch.from_numpy(hb.rope_table(self.hd, self.rope_max_pos)).to(device)
        self.ws: Optional[torch.Tensor] = None

    # -- metadata ---------------------------------------------------------
    def prepare(self, chunk_len, chunk_prefix, decode_ctx, block_table, token_budget=None) -> Prepared:
        T = int(np.sum(chunk_len)) + len(decode_ctx)
        blob, n = hb.pack_metadata(self.hd, chunk_len, chunk_prefix, decode_ctx, block_table, self.num_pages,
                                   T if token_budget is None else token_budget)
        meta_dev = torch.from_numpy(blob).to(self.device)
        return Prepared(blob, meta_dev, n)

    def _workspace(self, prep: Prepared) -> torch.Tensor:
        need = hb.workspace_bytes(self.hd, prep.blob)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws

    # -- entry points -----------------------------------------------------
    def append(self, prep: Prepared, k: torch.Tensor, v: torch.Tensor):
        """hb_kv_append of k, v [T][n_kv][d] (int16 bf16 bits) at the batch's slots."""
        row_stride = k.stride(0)
        hb.kv_append(self.hd, prep.blob, prep.meta_dev.data_ptr(), k.data_ptr(), v.data_ptr(), row_stride,
                     self.k_cache.data_ptr(), self.v_cache.data_ptr(), stream_handle())

    def forward(self, prep: Prepared, x: torch.Tensor, y: torch.Tensor, stage_events=None):
        ws = self._workspace(prep)
        hb.layer_forward(self.hd, self.hw, prep.blob, prep.meta_dev.data_ptr(), self.rope.data_ptr(),
                         self.rope_max_pos, x.data_ptr(), y.data_ptr(), self.k_cache.data_ptr(),
                         self.v_cache.data_ptr(), ws.data_ptr(), ws.numel(), stream_handle(), stage_events)

    def fill_prefixes(self, block_table: np.ndarray, seqs: Sequence[int], prefix_k, prefix_v):
        """Write already-cached K/V (positions 0..len-1) of the given sequences
        through hb_kv_append, as one batch of prefix-0 chunks."""
        rows = [s for s in seqs if s < len(prefix_k) and prefix_k[s].shape[0] > 0]
        if not rows:
            return
        lens = [int(prefix_k[s].shape[0]) for s in rows]
        bt = np.ascontiguousarray(block_table[rows])
        prep = self.prepare(lens, [0] * len(rows), [], bt)
        k = to_device_u16(np.concatenate([prefix_k[s] for s in rows]), self.device)
        v = to_device_u16(np.concatenate([prefix_v[s] for s in rows]), self.device)
        self.append(prep, k, v)
        torch.cuda.synchronize()

    # -- views for checking ---------------------------------------------------
    def stored(self, prep: Prepared) -> dict:
        """The activations the last forward of ``prep`` stored between its
        steps (hb_workspace_views_of), copied to the host: xn, o, h1n, act as
        bf16 bits (uint16), or with FP8 projections as e4m3 codes (uint8); q as
        bf16 bits; h1 as float32.  Rows in packed-token order."""
        d, T = self.dims, prep.n_tokens
        offs = hb.workspace_views(self.hd, prep.blob)
        f8 = bool(getattr(d, "w8a8", 0))
        width = {"xn": d.hidden, "q": d.n_q_heads * d.head_dim, "o": d.n_q_heads * d.head_dim,
                 "h1": d.hidden, "h1n": d.hidden, "act": d.ffn_dim}
        out = {}
        for name, n in width.items():
            if name == "h1":
                dt, nb = torch.float32, 4
            elif name != "q" and f8:
                dt, nb = torch.uint8, 1
            else:
                dt, nb = torch.int16, 2
            raw = self.ws[offs[name]:offs[name] + T * n * nb]
            a = raw.view(dt).reshape(T, n).cpu().numpy()
            out[name] = a.view(np.uint16) if dt == torch.int16 else a
        return out

    def cache_logical(self):
        """(K, V) in logical order [page][kv][slot][d]: bf16 bits as uint16, or
        FP8 e4m3 codes as uint8."""
        P, nkv, c, p, _ = self.k_cache.shape
        k = self.k_cache.cpu().numpy().view(self._np_cache).transpose(0, 1, 3, 2, 4).reshape(P, nkv, p, c * 32)
        v = self.v_cache.cpu().numpy().view(self._np_cache).transpose(0, 1, 3, 2)
        return np.ascontiguousarray(k), np.ascontiguousarray(v)

    def gather_kv(self, pages, slots):
        """K and V rows at (page, slot) pairs [n][kv][d]: bf16 bits as uint16, or
        FP8 e4m3 codes as uint8."""
        pg = torch.as_tensor(np.asarray(pages), device=self.device)
        sl = torch.as_tensor(np.asarray(slots), device=self.device)
        k = self.k_cache[pg, :, :, sl, :]                       # [n][kv][d/32][32]
        v = self.v_cache.permute(0, 1, 3, 2)[pg, :, sl, :]      # [n][kv][d]
        n, nkv = k.shape[0], k.shape[1]
        return (k.reshape(n, nkv, -1).cpu().numpy().view(self._np_cache),
                v.cpu().numpy().view(self._np_cache))
