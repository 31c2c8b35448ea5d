// Device entry points of the hybrid-batch layer library: hb_kv_append and
// hb_layer_forward.  Validation happens here, on the host, before anything is
// enqueued; the kernels assume validated metadata.
//
// hb_layer_forward is the one-layer slice of the serving iteration
// run_iteration(B) of the "Sarathi-Serve reading notes" (§3.4): the hybrid
// batch B (decodes plus chunk pieces under tau, §3.2) passes once through
//   RMSNorm -> QKV projection (+RoPE, +KV append) -> paged hybrid attention ->
//   O projection (+residual) -> RMSNorm -> gate/up projection (+SwiGLU) ->
//   down projection (+residual).

#include <mutex>

#include "device_common.h"

namespace hb {

DevMeta dev_meta(const hb_meta_header* h, const void* meta_dev) {
  const char* b = (const char*)meta_dev;
  DevMeta m;
  m.q_start = (const int32_t*)(b + h->off_q_start);
  m.cached = (const int32_t*)(b + h->off_cached);
  m.kv_len = (const int32_t*)(b + h->off_kv_len);
  m.tok_seq = (const int32_t*)(b + h->off_tok_seq);
  m.tok_pos = (const int32_t*)(b + h->off_tok_pos);
  m.slot = (const int32_t*)(b + h->off_slot);
  m.part_off = (const int32_t*)(b + h->off_part_off);
  m.part_cnt = (const int32_t*)(b + h->off_part_cnt);
  m.block_table = (const int32_t*)(b + h->off_block_table);
  m.chunk_items = (const hb_attn_item*)(b + h->off_chunk_items);
  m.decode_items = (const hb_attn_item*)(b + h->off_decode_items);
  m.append_runs = (const hb_append_run*)(b + h->off_append_runs);
  m.n_append_runs = h->n_append_runs;
  return m;
}

}  // namespace hb

using namespace hb;

#define HB_TRY(expr)                 \
  do {                               \
    hb_status _st = (expr);          \
    if (_st != HB_OK) return _st;    \
  } while (0)

extern "C" hb_status hb_kv_append(const hb_dims* dims, const void* meta_host, const void* meta_dev,
                                  const uint16_t* k, const uint16_t* v, int64_t row_stride, void* k_cache,
                                  void* v_cache, void* stream) {
  HB_TRY(check_dims(dims));
  HB_TRY(check_meta(dims, meta_host));
  if (!meta_dev || !k || !v || !k_cache || !v_cache) return fail(HB_E_NULL, "kv_append: NULL pointer");
  if (row_stride < (int64_t)dims->n_kv_heads * dims->head_dim || row_stride % 8)
    return fail(HB_E_SHAPE, "kv_append: row_stride must be >= n_kv*head_dim and a multiple of 8");
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15)
    return fail(HB_E_SHAPE, "kv_append: buffers must be 16-byte aligned");
  const hb_meta_header* h = (const hb_meta_header*)meta_host;
  return launch_kv_append(*dims, dev_meta(h, meta_dev), h->n_tokens, k, v, row_stride, k_cache, v_cache,
                          (stream_t)stream);
}

// ---------------------------------------------------------------------------
// Static scratch of hb_layer_forward_static_scratch, for callers that cannot
// allocate: the workspace of one forward (stored activations, attention and
// split-K partial results) in a file-scope device array, one per GPU the
// library runs on, held until the process ends.  In host code `scratch` is a
// host-side stand-in, not a device address: its device address is looked up
// once per device (hipGetSymbolAddress, with the device current) and only
// that address is handed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the current device's scratch (looked up on the first
// call on that device).
static hb_status static_scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(HB_E_HIP, "static scratch: no current device (or device index >= 64)");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HB_E_HIP, std::string("static scratch: hipGetSymbolAddress failed: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HB_OK;
}

// The forward of both entry points; static_ws: the workspace is the static
// scratch (workspace and workspace_bytes are ignored).
static hb_status layer_forward_impl(const hb_dims* dims, const hb_weights* w, const void* meta_host,
                                    const void* meta_dev, const float* rope_cs, int32_t rope_max_pos,
                                    const float* x, float* y, void* k_cache, void* v_cache, void* workspace,
                                    size_t workspace_bytes, void* stream, void* const* stage_events,
                                    bool static_ws) {
  HB_TRY(check_dims(dims));
  HB_TRY(check_meta(dims, meta_host));
  if (!w || !meta_dev || !rope_cs || !x || !y || !k_cache || !v_cache || (!static_ws && !workspace))
    return fail(HB_E_NULL, "layer_forward: NULL pointer");
  if (!w->w_q || !w->w_k || !w->w_v || !w->w_o || !w->w_g || !w->w_u || !w->w_d || !w->g_attn || !w->g_ffn)
    return fail(HB_E_NULL, "layer_forward: NULL weight");
  const bool f8 = dims->w8a8 != 0;
  if (f8 && (!w->s_q || !w->s_k || !w->s_v || !w->s_o || !w->s_g || !w->s_u || !w->s_d))
    return fail(HB_E_NULL, "layer_forward: FP8 projections need every weight row scale");
  if ((const void*)x == (const void*)y) return fail(HB_E_SHAPE, "layer_forward: x and y alias");
  const hb_meta_header* h = (const hb_meta_header*)meta_host;
  if (h->max_kv_len > rope_max_pos)
    return fail(HB_E_CAPACITY, "rope table holds " + std::to_string(rope_max_pos) + " positions, batch reaches " +
                                   std::to_string(h->max_kv_len));
  const int T = h->n_tokens;
  const WsLayout L = ws_layout(*dims, T, h->n_partials);
  if (static_ws && L.total > kStaticScratchBytes)
    return fail(HB_E_CAPACITY, "layer_forward_static_scratch: the batch needs " + std::to_string(L.total) +
                                   " bytes of workspace, the static scratch holds " +
                                   std::to_string(kStaticScratchBytes));
  if (!static_ws && workspace_bytes < L.total)
    return fail(HB_E_CAPACITY, "workspace needs " + std::to_string(L.total) + " bytes");
  const uintptr_t al = (uintptr_t)workspace | (uintptr_t)x | (uintptr_t)y | (uintptr_t)k_cache |
                       (uintptr_t)v_cache | (uintptr_t)rope_cs | (uintptr_t)w->w_q | (uintptr_t)w->w_k |
                       (uintptr_t)w->w_v | (uintptr_t)w->w_o | (uintptr_t)w->w_g | (uintptr_t)w->w_u |
                       (uintptr_t)w->w_d | (uintptr_t)w->g_attn | (uintptr_t)w->g_ffn;
  if (al & 15) return fail(HB_E_SHAPE, "layer_forward: device buffers must be 16-byte aligned");
  if (static_ws) HB_TRY(static_scratch_ptr(&workspace));

  const stream_t s = (stream_t)stream;
  // optional per-stage timing events (see HB_STAGE_NAMES)
  auto mark = [&](int i) -> hb_status {
    if (stage_events && stage_events[i] && hipEventRecord((hipEvent_t)stage_events[i], (hipStream_t)stream) != hipSuccess)
      return fail(HB_E_HIP, "layer_forward: stage event record failed");
    return HB_OK;
  };
  const DevMeta m = dev_meta(h, meta_dev);
  char* ws = (char*)workspace;
  uint16_t* xn = (uint16_t*)(ws + L.xn);
  uint16_t* qb = (uint16_t*)(ws + L.q);
  uint16_t* ob = (uint16_t*)(ws + L.o);
  float* h1 = (float*)(ws + L.h1);
  uint16_t* h1n = (uint16_t*)(ws + L.h1n);
  uint16_t* act = (uint16_t*)(ws + L.act);
  const int H = dims->hidden, d = dims->head_dim, nq = dims->n_q_heads, nkv = dims->n_kv_heads;
  const int F = dims->ffn_dim;

  // a1: RMSNorm of the input
  HB_TRY(mark(0));
  HB_TRY(launch_rmsnorm(x, w->g_attn, xn, T, H, dims->rms_eps, s, f8 ? 1.0f / dims->x_scale : 0.0f));

  // a2-a4: QKV projection, RoPE, KV append
  GemmArgs g{};
  g.mode = kGemmQkvRope;
  g.a = xn;
  g.lda = H;
  g.M = T;
  g.N = (nq + 2 * nkv) * d;
  g.K = H;
  g.w0 = static_cast<const uint16_t*>(w->w_q);
  g.w1 = static_cast<const uint16_t*>(w->w_k);
  g.w2 = static_cast<const uint16_t*>(w->w_v);
  g.f8 = f8;
  g.ws0 = w->s_q;
  g.ws1 = w->s_k;
  g.ws2 = w->s_v;
  g.a_scale = dims->x_scale;
  g.n0 = nq * d;
  g.n1 = nkv * d;
  g.out_b = qb;
  g.rope = rope_cs;
  g.tok_pos = m.tok_pos;
  g.slot = m.slot;
  g.k_cache = k_cache;
  g.v_cache = v_cache;
  g.kv_fp8 = dims->kv_fp8;
  g.k_inv_scale = dims->kv_fp8 ? 1.0f / dims->k_scale : 1.0f;
  g.v_inv_scale = dims->kv_fp8 ? 1.0f / dims->v_scale : 1.0f;
  g.n_q_heads = nq;
  g.n_kv_heads = nkv;
  g.head_dim = d;
  g.part = (float*)(ws + L.gemm_part);
  HB_TRY(mark(1));
  HB_TRY(launch_gemm(g, s));

  // a5: hybrid attention over the paged cache
  AttnArgs at{};
  at.q = qb;
  at.k_cache = k_cache;
  at.v_cache = v_cache;
  at.kv_fp8 = dims->kv_fp8;
  at.k_scale = dims->kv_fp8 ? dims->k_scale : 1.0f;
  at.v_scale = dims->kv_fp8 ? dims->v_scale : 1.0f;
  at.meta = m;
  at.max_pages = h->max_pages;
  at.n_q_heads = nq;
  at.n_kv_heads = nkv;
  at.head_dim = d;
  at.group = nq / nkv;
  at.n_chunk_items = h->n_chunk_items;
  at.n_decode_items = h->n_decode_items;
  at.n_tokens = T;
  at.n_merge_tokens = h->n_merge_tokens;
  merge_plan(h, meta_host, &at.merge_tok0, &at.merge_groups);
  at.part_o = (float*)(ws + L.part_o);
  at.part_ml = (float*)(ws + L.part_ml);
  at.out = ob;
  at.out_inv_scale = f8 ? 1.0f / dims->o_scale : 0.0f;
  HB_TRY(launch_attention(at, s, stage_events ? stage_events + 2 : nullptr));

  // a6: O projection + residual, a7: RMSNorm (split-K: the reduce adds the
  // residual and normalises in one pass)
  float* gpart = (float*)(ws + L.gemm_part);
  const GemmPlan po = gemm_plan(kGemmResidual, T, H, nq * d, f8);
  const GemmPlan pd = gemm_plan(kGemmResidual, T, H, F, f8);
  GemmArgs go{};
  go.mode = kGemmResidual;
  go.a = ob;
  go.lda = nq * d;
  go.M = T;
  go.N = H;
  go.K = nq * d;
  go.w0 = static_cast<const uint16_t*>(w->w_o);
  go.f8 = f8;
  go.ws0 = w->s_o;
  go.a_scale = dims->o_scale;
  go.res = x;
  go.out_f = h1;
  go.ldo = H;
  go.part = gpart;
  // Stage events: a split O's reduce (which adds the residual) belongs to the
  // O stage, as down's reduce belongs to the down stage; it also applies the
  // FFN RMSNorm, whose own stage is then empty.
  HB_TRY(mark(5));
  HB_TRY(launch_gemm(go, s));
  const float h_inv = f8 ? 1.0f / dims->h_scale : 0.0f;
  if (po.splits > 1) {
    HB_TRY(launch_splitk_reduce(gpart, po.splits, x, h1, T, H, w->g_ffn, h1n, dims->rms_eps, s, h_inv));
    HB_TRY(mark(6));
  } else {
    HB_TRY(mark(6));
    HB_TRY(launch_rmsnorm(h1, w->g_ffn, h1n, T, H, dims->rms_eps, s, h_inv));
  }

  // a8: gate/up projection + SwiGLU
  GemmArgs gu{};
  gu.mode = kGemmSwiglu;
  gu.a = h1n;
  gu.lda = H;
  gu.M = T;
  gu.N = 2 * F;
  gu.K = H;
  gu.w0 = static_cast<const uint16_t*>(w->w_g);
  gu.w1 = static_cast<const uint16_t*>(w->w_u);
  gu.f8 = f8;
  gu.ws0 = w->s_g;
  gu.ws1 = w->s_u;
  gu.a_scale = dims->h_scale;
  gu.out_inv_scale = f8 ? 1.0f / dims->a_scale : 0.0f;
  gu.out_b = act;
  gu.ldo = F;
  HB_TRY(mark(7));
  HB_TRY(launch_gemm(gu, s));

  // a9: down projection + residual
  GemmArgs gd{};
  gd.mode = kGemmResidual;
  gd.a = act;
  gd.lda = F;
  gd.M = T;
  gd.N = H;
  gd.K = F;
  gd.w0 = static_cast<const uint16_t*>(w->w_d);
  gd.f8 = f8;
  gd.ws0 = w->s_d;
  gd.a_scale = dims->a_scale;
  gd.res = h1;
  gd.out_f = y;
  gd.ldo = H;
  gd.part = gpart;
  HB_TRY(mark(8));
  HB_TRY(launch_gemm(gd, s));
  if (pd.splits > 1) HB_TRY(launch_splitk_reduce(gpart, pd.splits, h1, y, T, H, nullptr, nullptr, 0.f, s));
  HB_TRY(mark(9));
  return HB_OK;
}

extern "C" hb_status hb_layer_forward(const hb_dims* dims, const hb_weights* w, const void* meta_host,
                                      const void* meta_dev, const float* rope_cs, int32_t rope_max_pos,
                                      const float* x, float* y, void* k_cache, void* v_cache,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* stage_events) {
  return layer_forward_impl(dims, w, meta_host, meta_dev, rope_cs, rope_max_pos, x, y, k_cache, v_cache, workspace,
                            workspace_bytes, stream, stage_events, false);
}

extern "C" hb_status hb_layer_forward_static_scratch(const hb_dims* dims, const hb_weights* w, const void* meta_host,
                                                     const void* meta_dev, const float* rope_cs,
                                                     int32_t rope_max_pos, const float* x, float* y, void* k_cache,
                                                     void* v_cache, void* stream) {
  return layer_forward_impl(dims, w, meta_host, meta_dev, rope_cs, rope_max_pos, x, y, k_cache, v_cache, nullptr, 0,
                            stream, nullptr, true);
}
