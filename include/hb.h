/*
 * hb.h -- C ABI of the hybrid-batch decoder-layer library (MI355X, gfx950).
 *
 * One decoder-layer forward over a hybrid batch: prefill chunks, whose tokens
 * attend to their prompt's already-cached prefix plus causally to their own
 * chunk, packed together with single-token decodes that attend to their own
 * paged KV; every token of the batch shares the QKV, O and SwiGLU projections.
 *
 * Sources:
 *   "Sarathi-Serve reading notes" (zhongzhuzhou.org): §3.1 chunked prefills
 *   (chunk i covers positions [(i-1)C, iC), writes their KV and attends to all
 *   KV of earlier chunks), §3.2 stall-free hybrid batches (decode tokens plus
 *   chunk tokens under a token budget tau), §3.5 paged KV cache, §1.6 the
 *   linear-layer cost model.
 *   "Chunked Prefill" (bowenzhou.top): "mechanism" (chunks continue the KV
 *   through paged blocks) and the hybrid-iteration roofline.
 *
 * Conventions shared by every entry point
 *   - bf16 values travel as uint16_t bit patterns; fp32 as float.
 *   - Sequence order: the n_chunks chunk pieces in argument order, then the
 *     n_decodes decodes.  Packed token order follows the sequence order; a
 *     chunk's tokens are consecutive, a decode contributes one token.
 *   - A chunk piece of length L with prefix P holds positions [P, P+L) of its
 *     prompt; a decode with context C is one token at position C (C tokens are
 *     already cached; it attends C+1 keys, itself included).
 *   - KV cache (bf16, or FP8 e4m3 with dims->kv_fp8), two separate device
 *     arrays, page size p = 16:
 *       K: [num_pages][n_kv_heads][head_dim/32][p][32]   (32-dim slices, each
 *          token-major: dims 32c..32c+31 of a page's 16 tokens are one
 *          contiguous block, 1 KB in bf16, 512 B in FP8)
 *       V: [num_pages][n_kv_heads][head_dim][p]   (dim-major inside a page)
 *     Position pos of sequence s lives in page block_table[s][pos / p] at
 *     in-page slot pos % p.  Unused block-table entries are -1 and are never
 *     read; pages no sequence references are never touched.
 *   - Ownership: the caller allocates and frees every host and device buffer
 *     (metadata, workspace, caches, weights, activations).  The library keeps
 *     no pointer after a call returns, allocates no memory, and holds no
 *     global mutable state apart from a thread-local error string.
 *   - Device entry points only enqueue work on `stream` (a hipStream_t; NULL
 *     is the default stream) and return; buffers must stay alive until the
 *     stream has finished that work.
 *   - Errors: every function returns hb_status; no C++ exception crosses the
 *     ABI.  All argument checks happen on the host before anything is
 *     enqueued, so on an error nothing has been written or launched.
 *     hb_last_error_detail() describes the most recent failure of the calling
 *     thread.
 */
#ifndef HB_H_
#define HB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HB_OK = 0,
  HB_E_NULL = 1,      /* a required pointer is NULL */
  HB_E_SHAPE = 2,     /* unsupported or inconsistent dimensions */
  HB_E_LENGTH = 3,    /* a length is out of range (chunk <= 0, prefix/context < 0) */
  HB_E_BUDGET = 4,    /* the batch holds more tokens than the token budget tau */
  HB_E_PAGE = 5,      /* a needed block-table entry is outside [0, num_pages),
                         or a sequence needs more pages than a table row holds */
  HB_E_ALIAS = 6,     /* one physical page is referenced twice */
  HB_E_CAPACITY = 7,  /* a caller buffer (metadata, workspace, rope table) is too small */
  HB_E_HIP = 8,       /* a HIP launch or runtime call failed */
  HB_E_META = 9       /* the metadata blob is not one hb_pack_metadata wrote for these dims
                         (bad magic or version, other dims, or counts and array offsets
                         that do not fit the blob's size) */
} hb_status;

/* Layer shape.  Supported: head_dim 64 or 128; n_q_heads % n_kv_heads == 0
 * with group g = n_q_heads / n_kv_heads <= 16; hidden, ffn_dim, n_q_heads *
 * head_dim and n_kv_heads * head_dim multiples of 128; hidden <= 16384;
 * page_size 16. */
typedef struct {
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn_dim;
  int32_t page_size;
  float rms_eps;     /* RMSNorm epsilon, e.g. 1e-5 */
  float rope_theta;  /* rotary base, e.g. 1e4 */
  /* KV cache element type.  0: bf16.  1: FP8 e4m3 (OCP e4m3fn: exponent bias
   * 7, largest finite 448, no infinities, NaN 0x7F/0xFF), one byte per
   * element: the cache holds e4m3(x / scale) rounded to nearest even and
   * saturated to +-448, and attention reads code value * scale.  x / scale is
   * evaluated in single precision as x times the float reciprocal of scale
   * (the precision decides codes at midpoints).  K/V inputs must be finite
   * (NaN inputs are outside the contract).  The scales are per layer, come from
   * the caller, must be finite and > 0 (HB_E_SHAPE otherwise) and are ignored
   * for bf16. */
  int32_t kv_fp8;
  float k_scale;
  float v_scale;
  /* Projection precision.  0: bf16 weights and inputs.  1: FP8 e4m3 on the
   * gfx950 FP8 matrix cores: the projection weights are e4m3 codes with one
   * float scale per output channel (hb_weights s_*), and the four projection
   * inputs -- the normed input (into QKV), the attention output (into O), the
   * normed residual (into gate/up) and the SwiGLU output (into down) -- are
   * stored as e4m3 codes of value / scale with the static per-layer scales
   * below (quotient in single precision as for the FP8 cache, nearest even,
   * saturating).  A projection is (a codes * scale) . (w codes * row scale)^T
   * with fp32 accumulation.  q, the KV cache and the fp32 residual stream are
   * unaffected.  Scales must be finite and > 0 (HB_E_SHAPE otherwise). */
  int32_t w8a8;
  float x_scale, o_scale, h_scale, a_scale;
} hb_dims;

/* Device pointers to the layer's parameters.  Projection matrices are
 * row-major [d_out][d_in], bf16 bits (or e4m3 codes with dims->w8a8):
 *   w_q [n_q*d][hidden], w_k and w_v [n_kv*d][hidden], w_o [hidden][n_q*d],
 *   w_g and w_u [ffn][hidden], w_d [hidden][ffn];  g_attn, g_ffn [hidden]
 * (bf16 bits).  With dims->w8a8, s_q .. s_d hold one float scale per output
 * channel (d_out entries each; row n of a matrix is codes[n] * s[n]); they
 * are not read otherwise. */
typedef struct {
  const void *w_q, *w_k, *w_v, *w_o, *w_g, *w_u, *w_d;
  const uint16_t *g_attn, *g_ffn;
  const float *s_q, *s_k, *s_v, *s_o, *s_g, *s_u, *s_d;
} hb_weights;

/* ---------------------------------------------------------------------------
 * Packed-token metadata.  hb_pack_metadata writes one self-contained blob:
 * this header followed by int32 arrays at the given byte offsets.  All
 * internal references are offsets, so the blob is copied verbatim to the
 * device (one hipMemcpyAsync of `bytes` bytes).
 */
#define HB_META_MAGIC 0x31424D48u /* "HMB1" */

typedef struct {
  int32_t seq;      /* sequence index */
  int32_t tok0;     /* first packed token of the tile */
  int32_t n_tok;    /* tokens in the tile (1 for a decode) */
  int32_t key0;     /* keys [key0, key1) of the sequence handled by this item */
  int32_t key1;
  int32_t split;    /* index of this key range among the tile's ranges */
  int32_t n_split;  /* number of key ranges of the tile (1: the item writes the
                       attention output itself, no partial result) */
  int32_t reserved;
} hb_attn_item;

/* A run of consecutive packed tokens of one sequence whose K/V land in one
 * page at consecutive slots: tokens [tok0, tok0 + n_tok) go to slots
 * slot0 .. slot0 + n_tok - 1 (slot0 = page * page_size + first in-page slot). */
typedef struct {
  int32_t tok0;
  int32_t n_tok;    /* 1 .. page_size */
  int32_t slot0;
  int32_t reserved;
} hb_append_run;

typedef struct {
  uint32_t magic;
  uint32_t version;
  int32_t n_seq, n_chunks, n_decodes, n_tokens;
  int32_t page_size, max_pages;     /* block-table row length */
  int32_t num_pages;                /* size of the page pool the tables index */
  int32_t max_kv_len;               /* max over sequences of cached + new */
  int32_t n_kv_heads, group, head_dim, n_q_heads;   /* dims the work lists were built for */
  int32_t chunk_q_tile;             /* tokens per chunk attention tile */
  int32_t chunk_kv_split;           /* keys per chunk attention item, at most */
  int32_t decode_kv_split;          /* keys per decode attention item */
  int32_t n_chunk_items, n_decode_items;
  int32_t n_partials;               /* attention partial results (part_cnt summed over the
                                       tokens with more than one) */
  int32_t n_append_runs;            /* KV append runs (hb_append_run) */
  int32_t n_merge_tokens;           /* tokens whose attention has more than one partial */
  int64_t bytes;                    /* size of the whole blob */
  /* byte offsets from the start of the blob */
  int64_t off_q_start;     /* int32 [n_seq + 1]  first packed token of each sequence */
  int64_t off_cached;      /* int32 [n_seq]      tokens cached before this batch */
  int64_t off_kv_len;      /* int32 [n_seq]      cached + new tokens */
  int64_t off_tok_seq;     /* int32 [n_tokens]   sequence of each token */
  int64_t off_tok_pos;     /* int32 [n_tokens]   position of each token in its sequence */
  int64_t off_slot;        /* int32 [n_tokens]   page * page_size + in-page slot */
  int64_t off_part_off;    /* int32 [n_tokens]   first attention partial of each token (-1: none) */
  int64_t off_part_cnt;    /* int32 [n_tokens]   key ranges of each token's attention (1: its
                              item writes the output directly, no partial) */
  int64_t off_block_table; /* int32 [n_seq][max_pages] copy of the caller's tables */
  int64_t off_chunk_items; /* hb_attn_item [n_chunk_items] */
  int64_t off_decode_items;/* hb_attn_item [n_decode_items] */
  int64_t off_append_runs; /* hb_append_run [n_append_runs], in packed-token order */
} hb_meta_header;

/* Upper bound of the blob size for any batch of n_seq sequences, n_tokens
 * tokens and max_pages_per_seq table columns under these dims; 0 on bad
 * arguments. */
size_t hb_meta_bytes(const hb_dims *dims, int32_t n_seq, int32_t n_tokens,
                     int32_t max_pages_per_seq);

/* Validate one hybrid batch and build its packed-token metadata (host only;
 * makes no HIP call).
 *
 * The batch is the stall-free hybrid batch of the "Sarathi-Serve reading
 * notes" §3.2: one token for each running decode plus prefill chunk pieces,
 * together at most the token budget tau.  A chunk piece continues its
 * prompt: the i-th chunk of size C covers prompt positions [(i-1)C, iC), and
 * the (i-1)C tokens before it are already cached (§3.1; here any prefix
 * length).  K/V live in fixed-size pages reached through per-sequence block
 * tables (§3.5 paged KV; "Chunked Prefill", mechanism: each chunk's K/V go
 * into the blocks the next chunk reads).
 *
 *   chunk_len[n_chunks], chunk_prefix_len[n_chunks]: new tokens and
 *     already-cached prefix of each chunk piece (chunk_len >= 1, prefix >= 0).
 *   decode_ctx_len[n_decodes]: tokens already cached per decode (>= 0).
 *   block_table[(n_chunks + n_decodes) * max_pages_per_seq]: row-major page
 *     tables in sequence order; entries -1 past a sequence's last page.
 *   num_pages: size of the page pool; token_budget: tau.
 *   meta_host: output blob, meta_capacity bytes; may be NULL to query the size.
 *   meta_bytes_out: receives the blob size (required).
 *   n_tokens_out: receives the packed token count (may be NULL).
 *
 * Checks (first failure wins): HB_E_NULL, HB_E_SHAPE (dims, max_pages < 1,
 * n_chunks + n_decodes < 1), HB_E_LENGTH, HB_E_BUDGET (tokens > tau),
 * HB_E_PAGE (needed entry outside [0, num_pages), more pages needed than
 * max_pages_per_seq, num_pages * page_size >= 2^31), HB_E_ALIAS (a page used
 * by two table entries), HB_E_CAPACITY (meta_capacity too small).
 * Nothing is written to meta_host unless the result is HB_OK. */
hb_status hb_pack_metadata(const hb_dims *dims, int32_t n_chunks, const int32_t *chunk_len,
                           const int32_t *chunk_prefix_len, int32_t n_decodes,
                           const int32_t *decode_ctx_len, const int32_t *block_table,
                           int32_t max_pages_per_seq, int32_t num_pages, int32_t token_budget,
                           void *meta_host, size_t meta_capacity, size_t *meta_bytes_out,
                           int32_t *n_tokens_out);

/* ---------------------------------------------------------------------------
 * Stall-free batch composition ("Sarathi-Serve reading notes" §3.4, the
 * scheduling loop; §7.6, a worked iteration).  Host only, no HIP calls.
 *
 * A request is described by its prompt length and the number of its tokens
 * already in the KV cache.  It is decoding once cached >= prompt_len (its next
 * token sits at position `cached`), otherwise its prompt is being prefilled.
 * One iteration takes, in this order:
 *   1. every decoding request, one token each, in array order, while the
 *      budget lasts (the pages add all decodes; more decodes than the budget
 *      is a case they do not cover, and the later ones wait);
 *   2. then, walking the prefilling requests in array order (the queue
 *      order), one chunk each of min(chunk_size, prompt_len - cached,
 *      budget left) tokens, until the budget is spent.
 * Output, in hb_pack_metadata's sequence order: the chunks (request index,
 * length, prefix = cached) then the decodes (request index, context =
 * cached).  Output arrays hold n_requests entries each.  The caller advances
 * each request's `cached` by what it was given after running the iteration.
 * Errors: HB_E_NULL, HB_E_SHAPE (n_requests < 0, token_budget < 1,
 * chunk_size < 1), HB_E_LENGTH (prompt_len < 1 or cached < 0). */
typedef struct {
  int32_t prompt_len;
  int32_t cached;
} hb_request;

hb_status hb_schedule_iteration(int32_t token_budget, int32_t chunk_size, int32_t n_requests,
                                const hb_request *requests, int32_t *chunk_req, int32_t *chunk_len,
                                int32_t *chunk_prefix, int32_t *n_chunks_out, int32_t *decode_req,
                                int32_t *decode_ctx, int32_t *n_decodes_out);

/* Rotary table for positions 0..max_pos-1 (host only): host_out[pos][i][0..1]
 * = (cos, sin)(pos * theta^(-2i/head_dim)), i < head_dim/2, computed in double
 * and rounded to float.  host_out holds max_pos * head_dim floats. */
hb_status hb_rope_table(const hb_dims *dims, int32_t max_pos, float *host_out);

/* Device workspace hb_layer_forward needs for the batch described by
 * meta_host; 0 on bad arguments. */
size_t hb_workspace_bytes(const hb_dims *dims, const void *meta_host);

/* Where hb_layer_forward leaves the activations it stores between the layer's
 * steps (the precision contract of the layer: each of these is what the next
 * step reads), as byte offsets into the workspace.  T = the batch's packed
 * tokens, rows in packed-token order:
 *   xn   [T][hidden]  normed input (into QKV)
 *   q    [T][n_q*d]   queries after RoPE, bf16, natural dim order
 *   o    [T][n_q*d]   attention output (into O)
 *   h1   [T][hidden]  x + o W_o^T, fp32
 *   h1n  [T][hidden]  normed residual (into gate/up)
 *   act  [T][ffn]     SwiGLU output (into down)
 * xn, o, h1n and act are bf16, or with dims->w8a8 one-byte e4m3 codes of
 * value / (x_scale, o_scale, h_scale, a_scale) with rows that many bytes
 * apart.  The contents are valid once the forward has completed on its
 * stream and until the workspace is used again.  For checking and debugging;
 * nothing else reads them.  Errors as hb_workspace_bytes (HB_E_NULL for a
 * NULL out). */
typedef struct {
  int64_t xn, q, o, h1, h1n, act;
} hb_workspace_views;

hb_status hb_workspace_views_of(const hb_dims *dims, const void *meta_host, hb_workspace_views *out);

/* KV append ("Chunked Prefill", mechanism: each chunk writes its KV into the
 * paged blocks): for every packed token t, k[t] and v[t] ([n_kv][head_dim]
 * bf16, consecutive tokens `row_stride` elements apart) go to slot[t] of the
 * K and V caches (as FP8 codes of k / k_scale, v / v_scale with
 * dims->kv_fp8).  Only those slots change.  meta_host / meta_dev: the blob
 * from hb_pack_metadata and its byte-identical device copy. */
hb_status hb_kv_append(const hb_dims *dims, const void *meta_host, const void *meta_dev,
                       const uint16_t *k, const uint16_t *v, int64_t row_stride,
                       void *k_cache, void *v_cache, void *stream);

/* One decoder-layer forward over the hybrid batch (device): one layer of
 * the iteration the "Sarathi-Serve reading notes" schedule in §3.4 (the whole
 * batch passes through the model once), with every token of the batch in the
 * same linear layers (§1.6: their cost depends on the token count, not on
 * which request a token belongs to; "Chunked Prefill", hybrid-iteration
 * roofline) and each token attending to its own sequence only: a chunk token
 * at position p sees keys 0..p of its prompt, the cached prefix plus its own
 * chunk causally (§3.1, §7.5b: query i of chunk k sees (k-1)C + i keys), a
 * decode sees its whole context plus itself (§3.2).  Steps:
 *   xn  = RMSNorm(x) * g_attn                                  (bf16)
 *   q,k,v = xn W_q^T, xn W_k^T, xn W_v^T; RoPE(q, k) by position (bf16)
 *   k, v appended to the cache at the tokens' slots
 *   o   = softmax(q K^T / sqrt(d)) V over keys 0..pos of the token's own
 *         sequence, q head h using kv head h / g                (bf16)
 *   h1  = x + o W_o^T                                           (fp32)
 *   a   = silu(RMSNorm(h1) g_ffn W_g^T) * (RMSNorm(h1) g_ffn W_u^T)  (bf16)
 *   y   = h1 + a W_d^T                                          (fp32)
 * x, y: [n_tokens][hidden] fp32 device arrays (may not alias).
 * rope_cs: device copy of hb_rope_table(dims, rope_max_pos); every position
 * in the batch must be < rope_max_pos (else HB_E_CAPACITY).
 * workspace: device buffer of at least hb_workspace_bytes(dims, meta_host).
 * The caches must hold the prefix/context K/V of every sequence and at least
 * the num_pages pages the metadata was packed for.
 * stage_events: NULL, or HB_NUM_STAGES + 1 caller-created hipEvent_t handles;
 * event i is recorded on `stream` right before stage i is launched and event
 * HB_NUM_STAGES after the last stage, so elapsed(event i, event i+1) is the
 * device time of stage i.  A NULL handle is skipped (each recorded event
 * leaves a gap of a few microseconds between two kernels, so a caller timing
 * one stage passes only its two events).  A failing event record returns HB_E_HIP (the
 * stages enqueued before it stay enqueued).  Where a split O projection's
 * reduce also applies the FFN RMSNorm, that reduce is timed with the O stage
 * and the rmsnorm_ffn stage is empty; the merge stage is empty when no token
 * has more than one attention partial.  Stages, in launch order: */
#define HB_NUM_STAGES 9
#define HB_STAGE_NAMES                                                              \
  { "rmsnorm_attn", "qkv_rope_append", "attn_chunk", "attn_decode", "attn_merge", \
    "o_proj_residual", "rmsnorm_ffn", "gate_up_swiglu", "down_residual" }
hb_status hb_layer_forward(const hb_dims *dims, const hb_weights *w, const void *meta_host,
                           const void *meta_dev, const float *rope_cs, int32_t rope_max_pos,
                           const float *x, float *y, void *k_cache, void *v_cache,
                           void *workspace, size_t workspace_bytes, void *stream,
                           void *const *stage_events);

/* hb_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * of HB_STATIC_SCRATCH_BYTES (128 MiB) inside the library: each GPU the
 * library is loaded on holds one until the process ends, and its device
 * address is looked up on the first call on that device (the device current
 * at the call; `stream` must belong to it).  This call allocates nothing and
 * calls no allocating routine; the caller still passes inputs, outputs,
 * caches and metadata as for hb_layer_forward.  Every call on one GPU uses
 * that GPU's one array, which keeps the last call's contents: calls that
 * overlap on one GPU (other streams, other threads) race; serialise them.
 * Nothing in the scratch needs to start at zero.  Errors: as hb_layer_forward;
 * HB_E_CAPACITY, before anything is enqueued, when the batch needs more than
 * HB_STATIC_SCRATCH_BYTES of workspace (hb_workspace_bytes gives the need). */
#define HB_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
hb_status hb_layer_forward_static_scratch(const hb_dims *dims, const hb_weights *w, const void *meta_host,
                                          const void *meta_dev, const float *rope_cs, int32_t rope_max_pos,
                                          const float *x, float *y, void *k_cache, void *v_cache,
                                          void *stream);

const char *hb_status_str(hb_status s);
const char *hb_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* HB_H_ */
