// Varlen hybrid attention over the paged KV cache for gfx950.
//
// Every packed token t of sequence s at position pos attends to keys
// 0..pos of s: a chunk token sees all KV written by the prompt's earlier
// chunks plus, causally, its own chunk ("Sarathi-Serve reading notes" §3.1,
// §7.5b); a decode token sees its whole context plus itself (§3.2).
// Scores are q.k/sqrt(d); q head h reads kv head h/g.
//
// Work is split over key ranges (hb_attn_item); each item writes an
// unnormalised partial (o, running max m, weight sum l) per (token, head) and
// a merge pass combines a token's partials.  The two item kinds run on
// different kernels:
//   decode: one wave per (item, kv head).  The g query heads of the kv group
//     form one 16-row MFMA tile.  S^T = K Q^T and O^T = V^T P^T, so that K
//     rows and V^T rows (the V cache is dim-major inside a page) are MFMA
//     fragments loaded straight from HBM as 16- and 8-byte vectors, and the
//     probabilities never leave the lanes that computed them.  The path is a
//     bandwidth-bound stream over the cached context.
//   chunk: one 256-thread workgroup per (item, kv head) holds up to 128
//     (token, head) rows, 32 per wave; 64-key tiles (4 pages) of K and V are
//     staged through double-buffered, swizzled LDS and shared by the 4 waves.

#include <math.h>

#include "device_common.h"

namespace hb {

__device__ __forceinline__ uint2 keep_first(uint2 v, int n) {
  // keep the first n (0..4) bf16 values of a 4-value vector, zero the rest
  if (n >= 4) return v;
  if (n <= 0) return make_uint2(0u, 0u);
  if (n == 1) return make_uint2(v.x & 0xffffu, 0u);
  if (n == 2) return make_uint2(v.x, 0u);
  return make_uint2(v.x, v.y & 0xffffu);
}

// Probabilities enter the PV product as two bf16 fragments, p = hi + lo with
// hi = bf16(p) and lo = bf16(p - hi): about 16 significant bits.  A single bf16
// P would put a 2^-9 relative error on every weight, and since o is an average
// of values that largely cancel, that error does not shrink with the number
// of keys.
__device__ __forceinline__ void split_p(const float* p, bf16x8& hi, bf16x8& lo) {
  uint32_t h[8];
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f2bf(p[e]);
    r[e] = p[e] - bf2f((uint16_t)h[e]);
  }
  uint4 uh, ul;
  uh.x = h[0] | (h[1] << 16);
  uh.y = h[2] | (h[3] << 16);
  uh.z = h[4] | (h[5] << 16);
  uh.w = h[6] | (h[7] << 16);
  ul.x = pack2bf(r[0], r[1]);
  ul.y = pack2bf(r[2], r[3]);
  ul.z = pack2bf(r[4], r[5]);
  ul.w = pack2bf(r[6], r[7]);
  hi = as_bf16x8(uh);
  lo = as_bf16x8(ul);
}

// ----------------------------------------------------------------------------
// decode items
template <int D>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a, float scale_log2) {
  constexpr int KK = D / 32;  // MFMA k-steps over the head dim
  constexpr int NJ = D / 16;  // 16-dim output blocks
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item_idx = blockIdx.x * 4 + wave;
  if (item_idx >= a.n_decode_items) return;
  const int kvh = blockIdx.y;
  const hb_attn_item it = a.meta.decode_items[item_idx];
  const int g = a.group, nq = a.n_q_heads, nkv = a.n_kv_heads;
  const int r = lane & 15, qd = lane >> 4;
  const int t = it.tok0;
  const int32_t* bt = a.meta.block_table + (size_t)it.seq * a.max_pages;

  bf16x8 qf[KK];
  {
    const uint16_t* qrow = a.q + (size_t)t * nq * D + (size_t)(kvh * g + r) * D + qd * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = (r < g) ? as_bf16x8(*reinterpret_cast<const uint4*>(qrow + kk * 32)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const size_t hs = (size_t)16 * D;  // elements of one (page, kv head) block

  for (int kb = it.key0; kb < it.key1; kb += 32) {
    const bool has1 = kb + 16 < it.key1;
    const int pg0 = bt[kb >> 4];
    const int pg1 = has1 ? bt[(kb >> 4) + 1] : pg0;
    const uint16_t* K0 = a.k_cache + ((size_t)pg0 * nkv + kvh) * hs;
    const uint16_t* K1 = a.k_cache + ((size_t)pg1 * nkv + kvh) * hs;
    const uint16_t* V0 = a.v_cache + ((size_t)pg0 * nkv + kvh) * hs;
    const uint16_t* V1 = a.v_cache + ((size_t)pg1 * nkv + kvh) * hs;
    uint4 k0[KK], k1[KK];
    uint2 v0[NJ], v1[NJ];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k0[kk] = *reinterpret_cast<const uint4*>(K0 + r * D + kk * 32 + qd * 8);
#pragma unroll
    for (int j = 0; j < NJ; ++j) v0[j] = *reinterpret_cast<const uint2*>(V0 + (j * 16 + r) * 16 + qd * 4);
    if (has1) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) k1[kk] = *reinterpret_cast<const uint4*>(K1 + r * D + kk * 32 + qd * 8);
#pragma unroll
      for (int j = 0; j < NJ; ++j) v1[j] = *reinterpret_cast<const uint2*>(V1 + (j * 16 + r) * 16 + qd * 4);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) k1[kk] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) v1[j] = make_uint2(0, 0);
    }
    // S^T tiles: s0[i] = score(key kb + 4qd + i, row r), s1[i] = score(key kb + 16 + 4qd + i, row r)
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s0 = mfma16x16x32(as_bf16x8(k0[kk]), qf[kk], s0);
    if (has1) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) s1 = mfma16x16x32(as_bf16x8(k1[kk]), qf[kk], s1);
    }
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (kb + 4 * qd + i < it.key1) ? s0[i] * scale_log2 : -INFINITY;
      sv[4 + i] = (kb + 16 + 4 * qd + i < it.key1) ? s1[i] * scale_log2 : -INFINITY;
    }
    float mb = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mb = fmaxf(mb, sv[e]);
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mn = fmaxf(m, mb);
    const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m - mn);
    float ps[8], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ps[e] = (sv[e] == -INFINITY) ? 0.f : exp2f(sv[e] - mn);
      lsum += ps[e];
    }
    l = l * alpha + lsum;
    m = mn;
    bf16x8 pf, pfl;
    split_p(ps, pf, pfl);
    if (kb + 32 > it.key1) {  // tail: values past the last key may be poisoned
      const int n0 = it.key1 - (kb + 4 * qd), n1 = it.key1 - (kb + 16 + 4 * qd);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        v0[j] = keep_first(v0[j], n0);
        v1[j] = keep_first(v1[j], n1);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[j] *= alpha;
      const bf16x8 vf = as_bf16x8(make_uint4(v0[j].x, v0[j].y, v1[j].x, v1[j].y));
      acc[j] = mfma16x16x32(vf, pf, acc[j]);
      acc[j] = mfma16x16x32(vf, pfl, acc[j]);
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (r < g) {
    const int head = kvh * g + r;
    const size_t pidx = (size_t)a.meta.part_off[t] + it.split;
    float* po = a.part_o + (pidx * nq + head) * D;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      *reinterpret_cast<float4*>(po + j * 16 + qd * 4) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    if (qd == 0) {
      a.part_ml[(pidx * nq + head) * 2 + 0] = m;
      a.part_ml[(pidx * nq + head) * 2 + 1] = l;
    }
  }
}

// ----------------------------------------------------------------------------
// chunk items
template <int D>
__global__ __launch_bounds__(256) void attn_chunk_kernel(AttnArgs a, float scale_log2) {
  constexpr int KK = D / 32;
  constexpr int NJ = D / 16;
  constexpr int KCH = D / 8;      // 16-byte chunks per K row
  constexpr int PAGE = 16 * D;    // elements per (page, kv head) block
  constexpr int NLD = D / 32;     // 16-byte chunks each thread moves per operand per tile
  __shared__ __align__(16) uint16_t Ks[2][4 * PAGE];
  __shared__ __align__(16) uint16_t Vs[2][4 * PAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const hb_attn_item it = a.meta.chunk_items[blockIdx.x];
  const int kvh = blockIdx.y;
  const int g = a.group, nq = a.n_q_heads, nkv = a.n_kv_heads;
  const int r = lane & 15, qd = lane >> 4;
  const int32_t* bt = a.meta.block_table + (size_t)it.seq * a.max_pages;

  bf16x8 qf[2][KK];
  int rpos[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = wave * 32 + rb * 16 + r;
    const int tl = row / g, hq = row - tl * g;
    const bool valid = tl < it.n_tok;
    const int t = it.tok0 + tl;
    rpos[rb] = valid ? a.meta.tok_pos[t] : -1;
    const uint16_t* qrow = a.q + (size_t)t * nq * D + (size_t)(kvh * g + hq) * D + qd * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[rb][kk] = valid ? as_bf16x8(*reinterpret_cast<const uint4*>(qrow + kk * 32)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  f32x4 acc[2][NJ];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  uint4 kr[NLD], vr[NLD];
  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int ci = tid + 256 * u;
      const int pg = ci / (2 * D), within = ci % (2 * D);
      const int key_base = kt + pg * 16;
      if (key_base < it.key1) {
        const int page = bt[key_base >> 4];
        const size_t base = ((size_t)page * nkv + kvh) * PAGE + (size_t)within * 8;
        kr[u] = *reinterpret_cast<const uint4*>(a.k_cache + base);
        uint4 v = *reinterpret_cast<const uint4*>(a.v_cache + base);
        // V chunk `within` holds dim within/2, keys 8*(within&1) .. +7 of the page
        const int nvalid = it.key1 - (key_base + 8 * (within & 1));
        const uint2 lo = keep_first(make_uint2(v.x, v.y), nvalid);
        const uint2 hi = keep_first(make_uint2(v.z, v.w), nvalid - 4);
        vr[u] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int ci = tid + 256 * u;
      const int pg = ci / (2 * D), within = ci % (2 * D);
      const int key = within / KCH, c = within % KCH;
      *reinterpret_cast<uint4*>(&Ks[buf][(pg * 16 + key) * D + (c ^ (key & (KCH - 1))) * 8]) = kr[u];
      const int dd = within >> 1, hf = within & 1, s = (dd >> 3) & 3;
      uint16_t* vrow = &Vs[buf][pg * PAGE + dd * 16];
      *reinterpret_cast<uint2*>(vrow + ((2 * hf) ^ s) * 4) = make_uint2(vr[u].x, vr[u].y);
      *reinterpret_cast<uint2*>(vrow + ((2 * hf + 1) ^ s) * 4) = make_uint2(vr[u].z, vr[u].w);
    }
  };

  const int ntiles = (it.key1 - it.key0 + 63) / 64;
  gload(it.key0);
  lstore(0);
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int kt = it.key0 + ti * 64;
    const int cur = ti & 1;
    if (ti + 1 < ntiles) gload(kt + 64);
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[kb][1] = s[kb][0];
      const int key = kb * 16 + r;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int c = kk * 4 + qd;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[cur][key * D + (c ^ (key & (KCH - 1))) * 8]);
        s[kb][0] = mfma16x16x32(kf, qf[0][kk], s[kb][0]);
        s[kb][1] = mfma16x16x32(kf, qf[1][kk], s[kb][1]);
      }
    }
    bf16x8 pf[2][2], pfl[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float sv[16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt + kb * 16 + 4 * qd + i;
          sv[kb * 4 + i] = (key <= rpos[rb] && key < it.key1) ? s[kb][rb][i] * scale_log2 : -INFINITY;
        }
      float mb = sv[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mb = fmaxf(mb, sv[e]);
      mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      const float mn = fmaxf(m[rb], mb);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m[rb] - mn);
      float ps[16], lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ps[e] = (sv[e] == -INFINITY) ? 0.f : exp2f(sv[e] - mn);
        lsum += ps[e];
      }
      l[rb] = l[rb] * alpha + lsum;
      m[rb] = mn;
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[rb][j] *= alpha;
      // keys 32c + 4qd + e (e < 4) and 32c + 16 + 4qd + (e - 4) (e >= 4)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float p8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p8[e] = ps[(2 * c) * 4 + e];
          p8[4 + e] = ps[(2 * c + 1) * 4 + e];
        }
        split_p(p8, pf[rb][c], pfl[rb][c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int dd = j * 16 + r, sw = (dd >> 3) & 3;
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vs[cur][(2 * c) * PAGE + dd * 16 + (qd ^ sw) * 4]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vs[cur][(2 * c + 1) * PAGE + dd * 16 + (qd ^ sw) * 4]);
        const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[0][j] = mfma16x16x32(vf, pf[0][c], acc[0][j]);
        acc[1][j] = mfma16x16x32(vf, pf[1][c], acc[1][j]);
        acc[0][j] = mfma16x16x32(vf, pfl[0][c], acc[0][j]);
        acc[1][j] = mfma16x16x32(vf, pfl[1][c], acc[1][j]);
      }
    }
    if (ti + 1 < ntiles) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float lt = l[rb];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int row = wave * 32 + rb * 16 + r;
    const int tl = row / g, hq = row - tl * g;
    if (tl < it.n_tok) {
      const int t = it.tok0 + tl;
      const int head = kvh * g + hq;
      const size_t pidx = (size_t)a.meta.part_off[t] + it.split;
      float* po = a.part_o + (pidx * nq + head) * D;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        *reinterpret_cast<float4*>(po + j * 16 + qd * 4) =
            make_float4(acc[rb][j][0], acc[rb][j][1], acc[rb][j][2], acc[rb][j][3]);
      if (qd == 0) {
        a.part_ml[(pidx * nq + head) * 2 + 0] = m[rb];
        a.part_ml[(pidx * nq + head) * 2 + 1] = lt;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// merge: o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, one wave per (token, head)
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nq = a.n_q_heads;
  if (wid >= (int64_t)a.n_tokens * nq) return;
  const int t = (int)(wid / nq), h = (int)(wid % nq);
  const int p0 = a.meta.part_off[t], pc = a.meta.part_cnt[t];
  float M = -INFINITY;
  for (int p = 0; p < pc; ++p) M = fmaxf(M, a.part_ml[((size_t)(p0 + p) * nq + h) * 2]);
  float L = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int p = 0; p < pc; ++p) {
    const size_t pr = (size_t)(p0 + p) * nq + h;
    const float mp = a.part_ml[pr * 2], lp = a.part_ml[pr * 2 + 1];
    const float w = (mp == -INFINITY) ? 0.f : exp2f(mp - M);
    L += w * lp;
    const float* src = a.part_o + pr * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += w * src[e];
  }
  const float inv = 1.0f / L;
  uint16_t* dst = a.out + (size_t)t * nq * D + (size_t)h * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = f2bf(o[e] * inv);
}

template <int D>
static hb_status launch_attention_d(const AttnArgs& a, stream_t s, void* const* ev) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipStream_t st = (hipStream_t)s;
  if (ev) hipEventRecord((hipEvent_t)ev[0], st);
  if (a.n_chunk_items > 0)
    hipLaunchKernelGGL(attn_chunk_kernel<D>, dim3(a.n_chunk_items, a.n_kv_heads), dim3(256), 0, st, a, scale_log2);
  if (ev) hipEventRecord((hipEvent_t)ev[1], st);
  if (a.n_decode_items > 0)
    hipLaunchKernelGGL(attn_decode_kernel<D>, dim3((a.n_decode_items + 3) / 4, a.n_kv_heads), dim3(256), 0, st, a,
                       scale_log2);
  if (ev) hipEventRecord((hipEvent_t)ev[2], st);
  const int64_t waves = (int64_t)a.n_tokens * a.n_q_heads;
  hipLaunchKernelGGL(attn_merge_kernel<D>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return HB_OK;
}

hb_status launch_attention(const AttnArgs& a, stream_t s, void* const* ev) {
  if (a.n_tokens <= 0) return HB_OK;
  return a.head_dim == 128 ? launch_attention_d<128>(a, s, ev) : launch_attention_d<64>(a, s, ev);
}

}  // namespace hb
