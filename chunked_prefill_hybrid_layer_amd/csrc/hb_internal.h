// Internal definitions shared by the host code and the HIP kernels of the
// hybrid-batch layer library.  Not part of the public ABI (see include/hb.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/hb.h"

namespace hb {

// --- attention tiling (fixed by the kernels; recorded in the metadata) -----
constexpr int kChunkRows = 128;       // (token, head) rows per chunk attention tile
constexpr int kChunkKeyTile = 64;     // keys staged per step (4 pages of 16)
constexpr int kChunkMinKeys = 256;    // keys per chunk attention item at least, where a tile is split
constexpr int kChunkSlots = 512;      // chunk workgroups the machine runs at once (2 per CU x 256 CUs)
constexpr int kDecodeKeyStep = 32;    // keys per decode step (2 pages)
constexpr int kDecodeKvSplit = 256;   // keys per decode attention item, at least (multiple of 32)
constexpr int kDecodeKvSplitMax = 1024;  // at most: the decode kernel holds an item's page ids one per lane
constexpr int kDecodeWavesTarget = 16384;  // decode items x kv heads beyond which the decode split doubles
constexpr int kDecodeSlots = 3072;    // decode waves the machine runs at once (3 per SIMD x 1024 SIMDs)
constexpr int kPageSize = 16;
constexpr uint32_t kMetaVersion = 3;
constexpr int kMaxGroup = 16;         // decode path holds a kv group in one 16-row MFMA tile

// --- GEMM -------------------------------------------------------------------
constexpr int kNumCU = 256;           // MI355X compute units (tile / split-K planning)

inline int chunk_q_tile(int group) { return group >= kChunkRows ? 1 : kChunkRows / group; }

// Thread-local error detail.
void set_error(const std::string& msg);
hb_status fail(hb_status s, const std::string& msg);

// Validates dims against what the kernels support.
hb_status check_dims(const hb_dims* d);

// Byte layout of the device workspace for one batch.
struct WsLayout {
  size_t xn, q, o, h1, h1n, act, part_o, part_ml, gemm_part, total;
};
WsLayout ws_layout(const hb_dims& d, int n_tokens, int n_partials);

// Validates a metadata blob against dims (magic, version, dims it was built for).
hb_status check_meta(const hb_dims* d, const void* meta_host);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace hb

// Device-side launch helpers (defined in the .hip files).
namespace hb {

struct DevMeta {            // device pointers into the copied metadata blob
  const int32_t* q_start;
  const int32_t* cached;
  const int32_t* kv_len;
  const int32_t* tok_seq;
  const int32_t* tok_pos;
  const int32_t* slot;
  const int32_t* part_off;
  const int32_t* part_cnt;
  const int32_t* block_table;
  const hb_attn_item* chunk_items;
  const hb_attn_item* decode_items;
  const hb_append_run* append_runs;
  int n_append_runs;
};
DevMeta dev_meta(const hb_meta_header* h, const void* meta_dev);

typedef struct ihipStream_t* stream_t;

// out: bf16, or with out_inv_scale > 0 FP8 e4m3 codes of value * out_inv_scale
hb_status launch_rmsnorm(const float* x, const uint16_t* gain, void* out, int rows, int hidden,
                         float eps, stream_t s, float out_inv_scale = 0.0f);
hb_status launch_kv_append(const hb_dims& d, const DevMeta& m, int n_tokens, const uint16_t* k,
                           const uint16_t* v, int64_t row_stride, void* kc, void* vc, stream_t s);

enum GemmMode { kGemmQkvRope = 0, kGemmResidual = 1, kGemmSwiglu = 2 };

struct GemmArgs {
  int mode;
  // f8: A and the weights are FP8 e4m3 codes.  Then K and lda count 16-bit
  // units (two codes each), so that every address computation is the bf16
  // one over the same bytes; acc is scaled by a_scale * (row scale of the
  // weight row) and a SwiGLU output is written as codes of out * out_inv_scale.
  int f8;
  const float* ws0;
  const float* ws1;
  const float* ws2;
  float a_scale, out_inv_scale;
  const uint16_t* a;  // [M][K] bf16
  int lda;
  int M, N, K;
  // weights: QKV concatenates w0 (n0 rows), w1 (n1 rows), w2; SwiGLU pairs w0 (gate) and w1 (up);
  // the residual mode uses w0 only.
  const uint16_t* w0;
  const uint16_t* w1;
  const uint16_t* w2;
  int n0, n1;
  // residual: out_f = res + acc
  const float* res;
  float* out_f;
  int ldo;
  // SwiGLU / QKV bf16 output
  uint16_t* out_b;
  // QKV epilogue; the caches hold bf16, or FP8 e4m3 codes of x * inv_scale
  const float* rope;
  const int32_t* tok_pos;
  const int32_t* slot;
  void* k_cache;
  void* v_cache;
  int kv_fp8;
  float k_inv_scale, v_inv_scale;
  int n_q_heads, n_kv_heads, head_dim;
  // split-K partials [splits][M][N] fp32 (used when the plan splits K)
  float* part;
};
// Tile configuration (an index into the kernel's tile table) and split-K
// factor the GEMM launcher uses for a problem; the QKV launch reduces its own
// split, residual-mode callers reduce with launch_splitk_reduce.
struct GemmPlan {
  int tile, splits;
};
GemmPlan gemm_plan(int mode, int M, int N, int K, bool f8 = false);
hb_status launch_gemm(const GemmArgs& g, stream_t s);
// norm_out: bf16, or with norm_inv_scale > 0 FP8 e4m3 codes of value * norm_inv_scale
hb_status launch_splitk_reduce(const float* part, int splits, const float* res, float* out, int M, int N,
                               const uint16_t* gain, void* norm_out, float eps, stream_t s,
                               float norm_inv_scale = 0.0f);

struct AttnArgs {
  const uint16_t* q;       // [T][n_q * d]
  const void* k_cache;     // bf16, or FP8 e4m3 codes (value = code * scale)
  const void* v_cache;
  int kv_fp8;
  float k_scale, v_scale;
  DevMeta meta;
  int max_pages;
  int n_q_heads, n_kv_heads, head_dim, group;
  int n_chunk_items, n_decode_items, n_tokens;
  int n_merge_tokens;      // tokens with more than one partial (0: no merge pass)
  int merge_tok0;          // first decode token
  int merge_groups;        // lane groups per decode (token, head) pair in the merge (1, 2 or 4)
  float* part_o;           // [n_partials][n_q][d]
  float* part_ml;          // [n_partials][n_q][2]
  void* out;               // [T][n_q * d] bf16, or FP8 codes of o * out_inv_scale (> 0)
  float out_inv_scale;
};
// Attention in up to three launches (chunk items, decode items, merge of the
// tokens with more than one partial); ev, if not NULL, holds the events to
// record before each launch (3 entries).
hb_status launch_attention(const AttnArgs& a, stream_t s, void* const* ev);
// The merge's first decode token and lane groups per decode (token, head)
// pair, from the host copy of the metadata.
void merge_plan(const hb_meta_header* h, const void* meta_host, int* tok0, int* groups);

}  // namespace hb
