// Host side of the hybrid-batch layer library: batch validation, packed-token
// metadata, rotary table, workspace sizing and error reporting.  No HIP calls.
//
// A hybrid batch ("Sarathi-Serve reading notes", §3.2) packs chunk pieces of
// one or more prompts with one token per running decode, under a token budget
// tau.  A chunk piece of length L with prefix P covers prompt positions
// [P, P+L) (§3.1: chunk i covers [(i-1)C, iC)); its KV is appended to the
// prompt's pages and continues the prefix ("Chunked Prefill", mechanism).

#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "hb_internal.h"

namespace hb {

static thread_local std::string g_err;

void set_error(const std::string& msg) { g_err = msg; }

hb_status fail(hb_status s, const std::string& msg) {
  g_err = std::string(hb_status_str(s)) + ": " + msg;
  return s;
}

hb_status check_dims(const hb_dims* d) {
  if (!d) return fail(HB_E_NULL, "dims is NULL");
  if (d->hidden <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->ffn_dim <= 0)
    return fail(HB_E_SHAPE, "non-positive dimension");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(HB_E_SHAPE, "head_dim must be 64 or 128");
  if (d->n_q_heads % d->n_kv_heads) return fail(HB_E_SHAPE, "n_q_heads % n_kv_heads != 0");
  if (d->n_q_heads / d->n_kv_heads > kMaxGroup) return fail(HB_E_SHAPE, "group n_q/n_kv above 16");
  if (d->hidden % 128 || d->ffn_dim % 128 || (d->n_q_heads * d->head_dim) % 128 ||
      (d->n_kv_heads * d->head_dim) % 128)
    return fail(HB_E_SHAPE, "hidden, ffn_dim, n_q*d and n_kv*d must be multiples of 128");
  if (d->hidden > 16384) return fail(HB_E_SHAPE, "hidden above 16384");
  if (d->page_size != kPageSize) return fail(HB_E_SHAPE, "page_size must be 16");
  if (!(d->rms_eps >= 0.0f) || !(d->rope_theta > 0.0f)) return fail(HB_E_SHAPE, "bad eps or theta");
  if (d->kv_fp8 != 0 && d->kv_fp8 != 1) return fail(HB_E_SHAPE, "kv_fp8 must be 0 or 1");
  if (d->kv_fp8 && !(std::isfinite(d->k_scale) && d->k_scale > 0.0f && std::isfinite(d->v_scale) &&
                     d->v_scale > 0.0f))
    return fail(HB_E_SHAPE, "FP8 KV cache needs finite positive k_scale and v_scale");
  if (d->w8a8 != 0 && d->w8a8 != 1) return fail(HB_E_SHAPE, "w8a8 must be 0 or 1");
  if (d->w8a8) {
    for (float sc : {d->x_scale, d->o_scale, d->h_scale, d->a_scale})
      if (!(std::isfinite(sc) && sc > 0.0f))
        return fail(HB_E_SHAPE, "FP8 projections need finite positive x/o/h/a scales");
  }
  return HB_OK;
}

WsLayout ws_layout(const hb_dims& d, int T, int n_partials) {
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  size_t t = (size_t)T;
  w.xn = take(t * d.hidden * 2);
  w.q = take(t * d.n_q_heads * d.head_dim * 2);
  w.o = take(t * d.n_q_heads * d.head_dim * 2);
  w.h1 = take(t * d.hidden * 4);
  w.h1n = take(t * d.hidden * 2);
  w.act = take(t * d.ffn_dim * 2);
  w.part_o = take((size_t)n_partials * d.n_q_heads * d.head_dim * 4);
  w.part_ml = take((size_t)n_partials * d.n_q_heads * 2 * 4);
  // split-K partials: the largest need among the QKV, O and down projections,
  // planned exactly as the layer plans them (the FP8 plans may split differently)
  const int nqkv = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  const bool f8 = d.w8a8 != 0;
  const GemmPlan pq = gemm_plan(kGemmQkvRope, T, nqkv, d.hidden, f8);
  const GemmPlan po = gemm_plan(kGemmResidual, T, d.hidden, d.n_q_heads * d.head_dim, f8);
  const GemmPlan pd = gemm_plan(kGemmResidual, T, d.hidden, d.ffn_dim, f8);
  size_t part = 0;
  if (pq.splits > 1) part = std::max(part, (size_t)pq.splits * t * nqkv);
  if (po.splits > 1) part = std::max(part, (size_t)po.splits * t * d.hidden);
  if (pd.splits > 1) part = std::max(part, (size_t)pd.splits * t * d.hidden);
  w.gemm_part = take(part * 4);
  w.total = off;
  return w;
}

hb_status check_meta(const hb_dims* d, const void* meta_host) {
  if (!meta_host) return fail(HB_E_NULL, "meta_host is NULL");
  const hb_meta_header* h = (const hb_meta_header*)meta_host;
  if (h->magic != HB_META_MAGIC || h->version != kMetaVersion) return fail(HB_E_META, "bad metadata magic/version");
  if (h->n_kv_heads != d->n_kv_heads || h->n_q_heads != d->n_q_heads || h->head_dim != d->head_dim ||
      h->page_size != d->page_size || h->group != d->n_q_heads / d->n_kv_heads)
    return fail(HB_E_META, "metadata was built for other dims");
  // counts consistent and every array inside the blob (the host reads some
  // of them, the kernels all of them at these offsets)
  const int64_t hdr = (int64_t)sizeof(hb_meta_header);
  auto in_blob = [&](int64_t off, int64_t count, int64_t elem) {
    return count >= 0 && off >= hdr && off <= h->bytes && count * elem <= h->bytes - off;
  };
  const int64_t S = h->n_seq, T = h->n_tokens;
  if (S < 1 || T < 0 || h->n_decodes < 0 || h->n_decodes > T || h->n_chunks < 0 || h->max_pages < 1 ||
      h->n_partials < 0 || h->n_merge_tokens < 0 || h->n_merge_tokens > T || h->bytes < hdr ||
      !in_blob(h->off_q_start, S + 1, 4) || !in_blob(h->off_cached, S, 4) || !in_blob(h->off_kv_len, S, 4) ||
      !in_blob(h->off_tok_seq, T, 4) || !in_blob(h->off_tok_pos, T, 4) || !in_blob(h->off_slot, T, 4) ||
      !in_blob(h->off_part_off, T, 4) || !in_blob(h->off_part_cnt, T, 4) ||
      !in_blob(h->off_block_table, S * h->max_pages, 4) ||
      !in_blob(h->off_chunk_items, h->n_chunk_items, (int64_t)sizeof(hb_attn_item)) ||
      !in_blob(h->off_decode_items, h->n_decode_items, (int64_t)sizeof(hb_attn_item)) ||
      !in_blob(h->off_append_runs, h->n_append_runs, (int64_t)sizeof(hb_append_run)))
    return fail(HB_E_META, "metadata counts or array offsets do not fit the blob");
  return HB_OK;
}

}  // namespace hb

using namespace hb;

extern "C" {

const char* hb_status_str(hb_status s) {
  switch (s) {
    case HB_OK: return "HB_OK";
    case HB_E_NULL: return "HB_E_NULL";
    case HB_E_SHAPE: return "HB_E_SHAPE";
    case HB_E_LENGTH: return "HB_E_LENGTH";
    case HB_E_BUDGET: return "HB_E_BUDGET";
    case HB_E_PAGE: return "HB_E_PAGE";
    case HB_E_ALIAS: return "HB_E_ALIAS";
    case HB_E_CAPACITY: return "HB_E_CAPACITY";
    case HB_E_HIP: return "HB_E_HIP";
    case HB_E_META: return "HB_E_META";
  }
  return "HB_E_UNKNOWN";
}

const char* hb_last_error_detail(void) { return g_err.c_str(); }

size_t hb_meta_bytes(const hb_dims* dims, int32_t n_seq, int32_t n_tokens, int32_t max_pages) {
  if (check_dims(dims) != HB_OK || n_seq < 1 || n_tokens < 1 || max_pages < 1) return 0;
  size_t S = n_seq, T = n_tokens, P = max_pages;
  size_t max_keys = P * kPageSize;
  int qt = chunk_q_tile(dims->n_q_heads / dims->n_kv_heads);
  size_t tiles = T / qt + S;                                     // chunk tiles (>= 1 token each)
  size_t csplit = (max_keys + kChunkMinKeys - 1) / kChunkMinKeys + 1;
  size_t dsplit = (max_keys + kDecodeKvSplit - 1) / kDecodeKvSplit;
  size_t items = tiles * csplit + S * dsplit;
  size_t runs = T + S;                                           // a run per page a sequence touches
  size_t ints = (S + 1) + 3 * S + 5 * T + S * P;
  return align_up(sizeof(hb_meta_header), 64) + align_up(ints * 4 + 16 * 9, 64) +
         items * sizeof(hb_attn_item) + runs * sizeof(hb_append_run) + 64;
}

hb_status hb_pack_metadata(const hb_dims* dims, int32_t n_chunks, const int32_t* chunk_len,
                           const int32_t* chunk_prefix_len, int32_t n_decodes,
                           const int32_t* decode_ctx_len, const int32_t* block_table,
                           int32_t max_pages, int32_t num_pages, int32_t token_budget,
                           void* meta_host, size_t meta_capacity, size_t* meta_bytes_out,
                           int32_t* n_tokens_out) {
  try {
    hb_status st = check_dims(dims);
    if (st != HB_OK) return st;
    if (!meta_bytes_out) return fail(HB_E_NULL, "meta_bytes_out is NULL");
    if (n_chunks < 0 || n_decodes < 0 || n_chunks + n_decodes < 1)
      return fail(HB_E_SHAPE, "need at least one sequence");
    if ((n_chunks && (!chunk_len || !chunk_prefix_len)) || (n_decodes && !decode_ctx_len) || !block_table)
      return fail(HB_E_NULL, "length or block-table array is NULL");
    if (max_pages < 1 || num_pages < 1) return fail(HB_E_SHAPE, "max_pages and num_pages must be >= 1");
    const int S = n_chunks + n_decodes;
    const int p = dims->page_size;
    if ((int64_t)num_pages * p >= (int64_t)1 << 31) return fail(HB_E_PAGE, "page pool too large for int32 slots");

    // lengths and the token budget (tau bounds decode + chunk tokens, §3.2)
    std::vector<int32_t> cached(S), newtok(S);
    int64_t T = 0;
    for (int s = 0; s < S; ++s) {
      if (s < n_chunks) {
        if (chunk_len[s] < 1) return fail(HB_E_LENGTH, "chunk " + std::to_string(s) + " has length < 1");
        if (chunk_prefix_len[s] < 0) return fail(HB_E_LENGTH, "chunk " + std::to_string(s) + " has negative prefix");
        cached[s] = chunk_prefix_len[s];
        newtok[s] = chunk_len[s];
      } else {
        int32_t c = decode_ctx_len[s - n_chunks];
        if (c < 0) return fail(HB_E_LENGTH, "decode " + std::to_string(s - n_chunks) + " has negative context");
        cached[s] = c;
        newtok[s] = 1;
      }
      if ((int64_t)cached[s] + newtok[s] >= ((int64_t)1 << 30))
        return fail(HB_E_LENGTH, "sequence " + std::to_string(s) + " too long");
      T += newtok[s];
    }
    if (T > token_budget)
      return fail(HB_E_BUDGET, std::to_string(T) + " tokens exceed the budget " + std::to_string(token_budget));
    if (T >= ((int64_t)1 << 30)) return fail(HB_E_LENGTH, "too many tokens");

    // block tables: every needed entry valid and no page used twice
    std::vector<uint8_t> used((size_t)num_pages, 0);
    int max_kv = 0;
    for (int s = 0; s < S; ++s) {
      int kv = cached[s] + newtok[s];
      max_kv = std::max(max_kv, kv);
      int need = (kv + p - 1) / p;
      if (need > max_pages)
        return fail(HB_E_PAGE, "sequence " + std::to_string(s) + " needs " + std::to_string(need) +
                                   " pages, table rows hold " + std::to_string(max_pages));
      const int32_t* row = block_table + (size_t)s * max_pages;
      for (int b = 0; b < need; ++b) {
        int32_t e = row[b];
        if (e < 0 || e >= num_pages)
          return fail(HB_E_PAGE, "block_table[" + std::to_string(s) + "][" + std::to_string(b) + "] = " +
                                     std::to_string(e) + " outside [0, " + std::to_string(num_pages) + ")");
        if (used[e]) return fail(HB_E_ALIAS, "page " + std::to_string(e) + " referenced twice");
        used[e] = 1;
      }
    }

    // attention work lists: chunk tiles split over the key range, decodes split over their context
    const int g = dims->n_q_heads / dims->n_kv_heads;
    const int qt = chunk_q_tile(g);
    std::vector<int32_t> q_start(S + 1), kv_len(S);
    q_start[0] = 0;
    for (int s = 0; s < S; ++s) {
      q_start[s + 1] = q_start[s] + newtok[s];
      kv_len[s] = cached[s] + newtok[s];
    }
    // Which sequences take the decode kernel: every decode, and every chunk
    // piece short enough that its (token, head) rows fit the decode kernel's
    // 16-row tile (new tokens x group <= 16: a speculative-verify step of E
    // drafted tokens is a piece of E + 1 tokens over its context, "Sarathi-
    // Serve reading notes" §7.4).  Each row masks the keys past its own
    // position.  The other chunk pieces go to the chunk kernel's 128-row tiles.
    auto decode_path = [&](int s) { return s >= n_chunks || newtok[s] * g <= kMaxGroup; };
    // Chunk items.  The keys [0, key_end) of a chunk query tile are cut into
    // n runs of whole 64-key tiles, as equal as whole tiles allow (the last
    // run ends at key_end), n = ceil(tiles / per).  per, the 64-key tiles an
    // item takes at most, is the smallest (and at least kChunkMinKeys / 64)
    // for which the workgroups (items x kv heads) fit one round of the
    // machine, kChunkSlots: every workgroup then starts at once and the
    // nearly equal items end together.  Fewer, longer items would leave
    // slots idle; more would put a second round on some CUs and add partial
    // results to write and merge.  When no split fits one round, items take
    // at most half of a slot's share of the work (per = total 64-key tiles
    // x kv heads / (2 kChunkSlots)), so that longest-first ordering can
    // balance the rounds; tiles shorter than that stay whole.  A tile that
    // stays whole (n = 1) writes its output directly.
    const int64_t nkv = dims->n_kv_heads;
    std::vector<int64_t> tile_steps;
    for (int s = 0; s < n_chunks; ++s)
      if (!decode_path(s))
        for (int t0 = q_start[s]; t0 < q_start[s + 1]; t0 += qt)
        tile_steps.push_back((cached[s] + (t0 - q_start[s]) + std::min(qt, q_start[s + 1] - t0) + 63) / 64);
    int64_t max_steps = 1;
    for (int64_t x : tile_steps) max_steps = std::max(max_steps, x);
    auto workgroups = [&](int64_t per) {
      int64_t n = 0;
      for (int64_t x : tile_steps) n += (x + per - 1) / per;
      return n * nkv;
    };
    int64_t total_steps = 0;
    for (int64_t x : tile_steps) total_steps += x;
    int64_t per = std::max<int64_t>(kChunkMinKeys / 64, (total_steps * nkv + 2 * kChunkSlots - 1) / (2 * kChunkSlots));
    if (workgroups(max_steps) <= kChunkSlots) {   // non-increasing in per: bisect
      int64_t lo = std::min<int64_t>(kChunkMinKeys / 64, max_steps), hi = max_steps;
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (workgroups(mid) <= kChunkSlots) hi = mid;
        else lo = mid + 1;
      }
      per = lo;
    }
    const int csplit = (int)std::min<int64_t>(per * 64, 1 << 30);
    std::vector<int32_t> part_off((size_t)T), part_cnt((size_t)T);
    std::vector<hb_attn_item> citems, ditems;
    int64_t np = 0, n_merge = 0;
    for (int s = 0; s < n_chunks; ++s) {
      if (decode_path(s)) continue;
      for (int t0 = q_start[s]; t0 < q_start[s + 1]; t0 += qt) {
        int n = std::min(qt, q_start[s + 1] - t0);
        int key_end = cached[s] + (t0 - q_start[s]) + n;  // last token's position + 1
        const int64_t steps = (key_end + 63) / 64;
        const int nsplit = (int)((steps + per - 1) / per);
        for (int j = 0; j < nsplit; ++j) {
          hb_attn_item it{};
          it.seq = s;
          it.tok0 = t0;
          it.n_tok = n;
          it.key0 = (int)(64 * (steps * j / nsplit));
          it.key1 = std::min<int64_t>(key_end, 64 * (steps * (j + 1) / nsplit));
          it.split = j;
          it.n_split = nsplit;
          citems.push_back(it);
        }
        for (int t = t0; t < t0 + n; ++t) {
          part_cnt[t] = nsplit;
          part_off[t] = nsplit > 1 ? (int32_t)np : -1;
          if (nsplit > 1) {
            np += nsplit;
            ++n_merge;
          }
        }
      }
    }
    // Item order (the kernels take items in list order; the output does not
    // depend on it, partials are indexed by split).  Longest key ranges
    // first, so the long ones start early and the short ones fill in behind
    // them -- compared in 256-key buckets, and within a bucket split-major:
    // the items of the chunks' tiles that cover about the same key range run
    // next to each other and share those keys' K/V in L2.
    std::stable_sort(citems.begin(), citems.end(), [](const hb_attn_item& x, const hb_attn_item& y) {
      return x.split < y.split;
    });
    std::stable_sort(citems.begin(), citems.end(), [](const hb_attn_item& x, const hb_attn_item& y) {
      return (x.key1 - x.key0) / 256 > (y.key1 - y.key0) / 256;
    });
    // Keys per decode item: kDecodeKvSplit, unless its (item, kv head) waves
    // would spill past one round of the machine (kDecodeSlots) while a
    // longer split, still a multiple of kDecodeKeyStep and at most
    // kDecodeKvSplitMax, fits them in one: then the smallest such split, so
    // that no nearly empty second round trails the stream.  A batch too large
    // for one round keeps kDecodeKvSplit, doubled while it would still make
    // more than kDecodeWavesTarget waves: past that the split buys no
    // parallelism, only partial results to write and merge.
    int dsplit = kDecodeKvSplit;
    auto decode_items = [&](int split) {
      int64_t n = 0;
      for (int s = 0; s < S; ++s)
        if (decode_path(s)) n += (kv_len[s] + split - 1) / split;
      return n;
    };
    const int64_t nkv_d = dims->n_kv_heads;
    if (decode_items(dsplit) * nkv_d > kDecodeSlots && decode_items(kDecodeKvSplitMax) * nkv_d <= kDecodeSlots) {
      int lo = kDecodeKvSplit / kDecodeKeyStep, hi = kDecodeKvSplitMax / kDecodeKeyStep;   // in key steps
      while (lo < hi) {   // decode_items is non-increasing in the split: bisect
        const int mid = (lo + hi) / 2;
        if (decode_items(mid * kDecodeKeyStep) * nkv_d <= kDecodeSlots) hi = mid;
        else lo = mid + 1;
      }
      dsplit = lo * kDecodeKeyStep;
    }
    while (dsplit < kDecodeKvSplitMax && decode_items(dsplit) * nkv_d > kDecodeWavesTarget)
      dsplit = std::min(2 * dsplit, kDecodeKvSplitMax);   // an item's page ids fill at most one wave's lanes
    for (int s = 0; s < S; ++s) {
      if (!decode_path(s)) continue;
      const int t = q_start[s], n = newtok[s];
      const int nsplit = (kv_len[s] + dsplit - 1) / dsplit;
      for (int j = 0; j < nsplit; ++j) {
        hb_attn_item it{};
        it.seq = s;
        it.tok0 = t;
        it.n_tok = n;
        it.key0 = j * dsplit;
        it.key1 = std::min(kv_len[s], (j + 1) * dsplit);
        it.split = j;
        it.n_split = nsplit;
        ditems.push_back(it);
      }
      for (int u = t; u < t + n; ++u) {
        part_cnt[u] = nsplit;
        part_off[u] = nsplit > 1 ? (int32_t)np : -1;
        if (nsplit > 1) {
          np += nsplit;
          ++n_merge;
        }
      }
    }
    std::stable_sort(ditems.begin(), ditems.end(), [](const hb_attn_item& x, const hb_attn_item& y) {
      return x.key1 - x.key0 > y.key1 - y.key0;
    });
    if (np >= ((int64_t)1 << 31)) return fail(HB_E_CAPACITY, "too many attention partials");

    // KV append runs: each sequence's new tokens, cut where a page ends
    std::vector<hb_append_run> runs;
    for (int s = 0; s < S; ++s) {
      const int32_t* row = block_table + (size_t)s * max_pages;
      for (int t = q_start[s]; t < q_start[s + 1];) {
        const int pos = cached[s] + (t - q_start[s]);
        const int n = std::min(p - pos % p, q_start[s + 1] - t);
        hb_append_run r{};
        r.tok0 = t;
        r.n_tok = n;
        r.slot0 = row[pos / p] * p + pos % p;
        runs.push_back(r);
        t += n;
      }
    }

    // blob layout
    size_t off = align_up(sizeof(hb_meta_header), 64);
    auto take = [&](size_t bytes) {
      size_t at = off;
      off = align_up(off + bytes, 16);
      return (int64_t)at;
    };
    hb_meta_header h{};
    h.magic = HB_META_MAGIC;
    h.version = kMetaVersion;
    h.n_seq = S;
    h.n_chunks = n_chunks;
    h.n_decodes = n_decodes;
    h.n_tokens = (int32_t)T;
    h.page_size = p;
    h.max_pages = max_pages;
    h.num_pages = num_pages;
    h.max_kv_len = max_kv;
    h.n_kv_heads = dims->n_kv_heads;
    h.group = g;
    h.head_dim = dims->head_dim;
    h.n_q_heads = dims->n_q_heads;
    h.chunk_q_tile = qt;
    h.chunk_kv_split = csplit;
    h.decode_kv_split = dsplit;
    h.n_chunk_items = (int32_t)citems.size();
    h.n_decode_items = (int32_t)ditems.size();
    h.n_partials = (int32_t)np;
    h.n_append_runs = (int32_t)runs.size();
    h.n_merge_tokens = (int32_t)n_merge;
    h.off_q_start = take((S + 1) * 4);
    h.off_cached = take(S * 4);
    h.off_kv_len = take(S * 4);
    h.off_tok_seq = take(T * 4);
    h.off_tok_pos = take(T * 4);
    h.off_slot = take(T * 4);
    h.off_part_off = take(T * 4);
    h.off_part_cnt = take(T * 4);
    h.off_block_table = take((size_t)S * max_pages * 4);
    h.off_chunk_items = take(citems.size() * sizeof(hb_attn_item));
    h.off_decode_items = take(ditems.size() * sizeof(hb_attn_item));
    h.off_append_runs = take(runs.size() * sizeof(hb_append_run));
    h.bytes = (int64_t)align_up(off, 64);
    *meta_bytes_out = (size_t)h.bytes;
    if (n_tokens_out) *n_tokens_out = (int32_t)T;
    if (!meta_host) return HB_OK;
    if (meta_capacity < (size_t)h.bytes)
      return fail(HB_E_CAPACITY, "metadata needs " + std::to_string(h.bytes) + " bytes, buffer holds " +
                                     std::to_string(meta_capacity));

    char* base = (char*)meta_host;
    memset(base, 0, (size_t)h.bytes);
    memcpy(base, &h, sizeof(h));
    auto arr = [&](int64_t o) { return (int32_t*)(base + o); };
    memcpy(arr(h.off_q_start), q_start.data(), (S + 1) * 4);
    memcpy(arr(h.off_cached), cached.data(), S * 4);
    memcpy(arr(h.off_kv_len), kv_len.data(), S * 4);
    int32_t* tseq = arr(h.off_tok_seq);
    int32_t* tpos = arr(h.off_tok_pos);
    int32_t* tslot = arr(h.off_slot);
    for (int s = 0; s < S; ++s) {
      const int32_t* row = block_table + (size_t)s * max_pages;
      for (int t = q_start[s]; t < q_start[s + 1]; ++t) {
        int pos = cached[s] + (t - q_start[s]);
        tseq[t] = s;
        tpos[t] = pos;
        tslot[t] = row[pos / p] * p + pos % p;
      }
    }
    memcpy(arr(h.off_part_off), part_off.data(), T * 4);
    memcpy(arr(h.off_part_cnt), part_cnt.data(), T * 4);
    memcpy(arr(h.off_block_table), block_table, (size_t)S * max_pages * 4);
    if (!citems.empty()) memcpy(base + h.off_chunk_items, citems.data(), citems.size() * sizeof(hb_attn_item));
    if (!ditems.empty()) memcpy(base + h.off_decode_items, ditems.data(), ditems.size() * sizeof(hb_attn_item));
    memcpy(base + h.off_append_runs, runs.data(), runs.size() * sizeof(hb_append_run));
    return HB_OK;
  } catch (const std::bad_alloc&) {
    return fail(HB_E_CAPACITY, "host allocation failed");
  } catch (...) {
    return fail(HB_E_SHAPE, "unexpected exception");
  }
}

hb_status hb_schedule_iteration(int32_t token_budget, int32_t chunk_size, int32_t n_requests,
                                const hb_request* requests, int32_t* chunk_req, int32_t* chunk_len,
                                int32_t* chunk_prefix, int32_t* n_chunks_out, int32_t* decode_req,
                                int32_t* decode_ctx, int32_t* n_decodes_out) {
  if (!n_chunks_out || !n_decodes_out) return fail(HB_E_NULL, "schedule: NULL count output");
  if (n_requests < 0 || token_budget < 1 || chunk_size < 1)
    return fail(HB_E_SHAPE, "schedule: n_requests < 0, token_budget < 1 or chunk_size < 1");
  if (n_requests > 0 && (!requests || !chunk_req || !chunk_len || !chunk_prefix || !decode_req || !decode_ctx))
    return fail(HB_E_NULL, "schedule: NULL array");
  for (int i = 0; i < n_requests; ++i)
    if (requests[i].prompt_len < 1 || requests[i].cached < 0)
      return fail(HB_E_LENGTH, "schedule: request " + std::to_string(i) + " has prompt_len < 1 or cached < 0");
  int64_t n = 0;
  int nd = 0, nc = 0;
  // 1. decodes first: every request whose prompt is fully cached, one token each
  for (int i = 0; i < n_requests && n < token_budget; ++i) {
    if (requests[i].cached < requests[i].prompt_len) continue;
    decode_req[nd] = i;
    decode_ctx[nd] = requests[i].cached;
    ++nd;
    ++n;
  }
  // 2. then one chunk per prefilling request, in queue order, while budget remains
  for (int i = 0; i < n_requests && n < token_budget; ++i) {
    const int64_t remaining = (int64_t)requests[i].prompt_len - requests[i].cached;
    if (remaining <= 0) continue;
    const int64_t take = std::min<int64_t>(std::min<int64_t>(chunk_size, remaining), token_budget - n);
    chunk_req[nc] = i;
    chunk_len[nc] = (int32_t)take;
    chunk_prefix[nc] = requests[i].cached;
    ++nc;
    n += take;
  }
  *n_chunks_out = nc;
  *n_decodes_out = nd;
  return HB_OK;
}

hb_status hb_rope_table(const hb_dims* dims, int32_t max_pos, float* host_out) {
  hb_status st = check_dims(dims);
  if (st != HB_OK) return st;
  if (!host_out) return fail(HB_E_NULL, "host_out is NULL");
  if (max_pos < 1) return fail(HB_E_LENGTH, "max_pos must be >= 1");
  const int d = dims->head_dim, half = d / 2;
  const double theta = dims->rope_theta;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -(2.0 * i) / d);
    for (int64_t pos = 0; pos < max_pos; ++pos) {
      double a = (double)pos * inv_freq;
      host_out[(pos * half + i) * 2 + 0] = (float)cos(a);
      host_out[(pos * half + i) * 2 + 1] = (float)sin(a);
    }
  }
  return HB_OK;
}

size_t hb_workspace_bytes(const hb_dims* dims, const void* meta_host) {
  if (check_dims(dims) != HB_OK || check_meta(dims, meta_host) != HB_OK) return 0;
  const hb_meta_header* h = (const hb_meta_header*)meta_host;
  return ws_layout(*dims, h->n_tokens, h->n_partials).total;
}

hb_status hb_workspace_views_of(const hb_dims* dims, const void* meta_host, hb_workspace_views* out) {
  if (!out) return fail(HB_E_NULL, "workspace_views: NULL out");
  hb_status st = check_dims(dims);
  if (st != HB_OK) return st;
  st = check_meta(dims, meta_host);
  if (st != HB_OK) return st;
  const hb_meta_header* h = (const hb_meta_header*)meta_host;
  const WsLayout L = ws_layout(*dims, h->n_tokens, h->n_partials);
  out->xn = (int64_t)L.xn;
  out->q = (int64_t)L.q;
  out->o = (int64_t)L.o;
  out->h1 = (int64_t)L.h1;
  out->h1n = (int64_t)L.h1n;
  out->act = (int64_t)L.act;
  return HB_OK;
}

}  // extern "C"
