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
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack2bf(p[2 * e], p[2 * e + 1]);
    const float r0 = p[2 * e] - __uint_as_float(h[e] << 16);
    const float r1 = p[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u);
    l[e] = pack2bf(r0, r1);
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
  lo = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------------------
// decode items
//
// One step covers 32 keys (2 pages).  The item's page ids (at most 16: a
// decode item spans at most kDecodeKvSplit = 256 keys) sit one per lane and
// are broadcast with readlane, so no step waits on a block-table load.  The
// K/V of a step sit in one register buffer (138 VGPRs): three waves per SIMD
// keep more bytes in flight than two double-buffered ones did (measured).

// Issue the K (4 x 16 B per page) and V^T (8 x 8 B per page) fragment loads of
// the step starting at key KB into buffer set SFX.  With K stored in 32-dim
// slices of the page, each K load instruction reads one contiguous 1 KB
// block (16 keys x 32 dims) and each V^T load 16 dims x 16 keys (512 B); the
// loads are nontemporal (the KV is read once).
#define DEC_LOAD(KB, SFX)                                                                     \
  {                                                                                           \
    const int _j = ((KB) - it.key0) >> 4;                                                     \
    const bool _has1 = (KB) + 16 < it.key1;                                                   \
    const int _pg0 = __builtin_amdgcn_readlane(my_pg, _j);                                    \
    const int _pg1 = __builtin_amdgcn_readlane(my_pg, _has1 ? _j + 1 : _j);                   \
    const uint16_t* _K0 = a.k_cache + ((size_t)_pg0 * nkv + kvh) * hs + r * 32 + qd * 8;      \
    const uint16_t* _K1 = a.k_cache + ((size_t)_pg1 * nkv + kvh) * hs + r * 32 + qd * 8;      \
    const uint16_t* _V0 = a.v_cache + ((size_t)_pg0 * nkv + kvh) * hs + r * 16 + qd * 4;      \
    const uint16_t* _V1 = a.v_cache + ((size_t)_pg1 * nkv + kvh) * hs + r * 16 + qd * 4;      \
    _Pragma("unroll") for (int kk = 0; kk < KK; ++kk)                                         \
        k0##SFX[kk] = load_stream16(_K0 + kk * 512); \
    _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj)                                         \
        v0##SFX[jj] = load_stream8(_V0 + jj * 256); \
    if (_has1) {                                                                              \
      _Pragma("unroll") for (int kk = 0; kk < KK; ++kk)                                       \
          k1##SFX[kk] = load_stream16(_K1 + kk * 512); \
      _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj)                                       \
          v1##SFX[jj] = load_stream8(_V1 + jj * 256); \
    } else {                                                                                  \
      _Pragma("unroll") for (int kk = 0; kk < KK; ++kk) k1##SFX[kk] = make_uint4(0, 0, 0, 0); \
      _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) v1##SFX[jj] = make_uint2(0, 0);       \
    }                                                                                         \
  }

// Scores, online softmax and PV for the step starting at key KB from buffer SFX.
#define DEC_COMPUTE(KB, SFX)                                                                  \
  {                                                                                           \
    const bool _has1 = (KB) + 16 < it.key1;                                                   \
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;                                            \
    _Pragma("unroll") for (int kk = 0; kk < KK; ++kk)                                         \
        s0 = mfma16x16x32(as_bf16x8(k0##SFX[kk]), qf[kk], s0);                               \
    if (_has1) {                                                                              \
      _Pragma("unroll") for (int kk = 0; kk < KK; ++kk)                                       \
          s1 = mfma16x16x32(as_bf16x8(k1##SFX[kk]), qf[kk], s1);                             \
    }                                                                                         \
    /* raw scores; keys past the item's end are masked (tail step only) */                   \
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};                   \
    if ((KB) + 32 > it.key1) {                                                                \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                         \
        if ((KB) + 4 * qd + i >= it.key1) sv[i] = -INFINITY;                                  \
        if ((KB) + 16 + 4 * qd + i >= it.key1) sv[4 + i] = -INFINITY;                         \
      }                                                                                       \
    }                                                                                         \
    float mb = sv[0];                                                                         \
    _Pragma("unroll") for (int e = 1; e < 8; ++e) mb = fmaxf(mb, sv[e]);                      \
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));                                                   \
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));                                                   \
    /* running max in log2 units; the first step always has a valid key */                    \
    const float mn = fmaxf(m, mb * scale_log2);                                               \
    const float alpha = fast_exp2(m - mn);                                                    \
    float ps[8], lsum = 0.f;                                                                  \
    _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                           \
      ps[e] = fast_exp2(fmaf(sv[e], scale_log2, -mn));                                        \
      lsum += ps[e];                                                                          \
    }                                                                                         \
    l = l * alpha + lsum;                                                                     \
    m = mn;                                                                                   \
    bf16x8 pf, pfl;                                                                           \
    split_p(ps, pf, pfl);                                                                     \
    if ((KB) + 32 > it.key1) { /* tail: values past the last key may be poisoned */           \
      const int n0 = it.key1 - ((KB) + 4 * qd), n1 = it.key1 - ((KB) + 16 + 4 * qd);         \
      _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) {                                     \
        v0##SFX[jj] = keep_first(v0##SFX[jj], n0);                                            \
        v1##SFX[jj] = keep_first(v1##SFX[jj], n1);                                            \
      }                                                                                       \
    }                                                                                         \
    _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) {                                       \
      acc[jj] *= alpha;                                                                       \
      const bf16x8 vf =                                                                       \
          as_bf16x8(make_uint4(v0##SFX[jj].x, v0##SFX[jj].y, v1##SFX[jj].x, v1##SFX[jj].y));  \
      acc[jj] = mfma16x16x32(vf, pf, acc[jj]);                                                \
      acc[jj] = mfma16x16x32(vf, pfl, acc[jj]);                                               \
    }                                                                                         \
  }

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_decode_kernel(AttnArgs a, float scale_log2) {
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
  const int npg = (it.key1 - it.key0 + 15) >> 4;
  const int my_pg = (lane < npg) ? bt[(it.key0 >> 4) + lane] : 0;

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

  uint4 k0A[KK], k1A[KK];
  uint2 v0A[NJ], v1A[NJ];
  for (int kb = it.key0; kb < it.key1; kb += 32) {
    DEC_LOAD(kb, A);
    DEC_COMPUTE(kb, A);
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

#undef DEC_LOAD
#undef DEC_COMPUTE

// ----------------------------------------------------------------------------
// chunk items
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_chunk_kernel(AttnArgs a, float scale_log2) {
  constexpr int KK = D / 32;
  constexpr int NJ = D / 16;
  constexpr int KCH = D / 8;      // 16-byte chunks per K row
  constexpr int PAGE = 16 * D;    // elements per (page, kv head) block
  constexpr int NLD = D / 32;     // 16-byte chunks each thread moves per operand per tile
  __shared__ __align__(16) uint16_t Ks[2][4 * PAGE];
  __shared__ __align__(16) uint16_t Vs[2][4 * PAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // kv head fastest: workgroups go round-robin over the 8 XCDs, so kv head h
  // runs on XCD h mod 8 and the prefix K/V every query tile of that head
  // re-reads stays in that XCD's L2
  const hb_attn_item it = a.meta.chunk_items[blockIdx.x / a.n_kv_heads];
  const int kvh = blockIdx.x % a.n_kv_heads;
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

  // The item's page ids, staged in LDS a window of 64 pages (16 key tiles) at
  // a time, double-buffered: window w sits in pids[w & 1].  Window w + 1 is
  // staged at the first tile of window w; the buffer it overwrites (window
  // w - 1) was last read two iterations earlier, and its first reader comes
  // after at least one barrier.
  __shared__ int pids[2][64];
  const int npg = (it.key1 - it.key0 + 15) >> 4;
#define STAGE_PIDS(W)                                                                         \
  if (tid < 64 && (W) * 64 + tid < npg) pids[(W) & 1][tid] = bt[(it.key0 >> 4) + (W) * 64 + tid];
  STAGE_PIDS(0);
  __syncthreads();

  // thread tid moves 16-byte chunk ci = tid + 256 u of the 4-page tile:
  // page ci / (2 D), chunk `within` = ci % (2 D) of that (page, kv head) block
  uint4 kr[NLD], vr[NLD];
#define CHUNK_GLOAD(KT)                                                                       \
  _Pragma("unroll") for (int u = 0; u < NLD; ++u) {                                           \
    const int ci = tid + 256 * u;                                                             \
    const int pg = ci / (2 * D), within = ci % (2 * D);                                       \
    const int key_base = (KT) + pg * 16;                                                      \
    if (key_base < it.key1) {                                                                 \
      const int pi = (key_base - it.key0) >> 4;                                               \
      const int page = pids[(pi >> 6) & 1][pi & 63];                                          \
      const size_t base = ((size_t)page * nkv + kvh) * PAGE + (size_t)within * 8;             \
      kr[u] = *reinterpret_cast<const uint4*>(a.k_cache + base);                              \
      vr[u] = *reinterpret_cast<const uint4*>(a.v_cache + base);                              \
    } else {                                                                                  \
      kr[u] = make_uint4(0, 0, 0, 0);                                                         \
      vr[u] = make_uint4(0, 0, 0, 0);                                                         \
    }                                                                                         \
  }
  // K rows go to Ks swizzled by key; V^T chunk `within` holds dim within / 2,
  // keys 8 (within & 1) .. +7 of its page: values past the item's last key are
  // zeroed (the cache may hold poison there), and each 4-key group is placed at
  // group ^ ((dim >> 2) & 3): the PV fragment reads (ds_read_b64) then have no bank conflicts.
#define CHUNK_LSTORE(KT, BUF)                                                                 \
  _Pragma("unroll") for (int u = 0; u < NLD; ++u) {                                           \
    const int ci = tid + 256 * u;                                                             \
    const int pg = ci / (2 * D), within = ci % (2 * D);                                       \
    /* K chunk `within` of the page block [D/32][16][32]: slot key, 8-dim chunk c */          \
    const int key = (within >> 2) & 15, c = (within >> 6) * 4 + (within & 3);                \
    *reinterpret_cast<uint4*>(&Ks[BUF][(pg * 16 + key) * D + (c ^ (key & (KCH - 1))) * 8]) = kr[u]; \
    const int nvalid = it.key1 - ((KT) + pg * 16 + 8 * (within & 1));                         \
    const uint2 lo = keep_first(make_uint2(vr[u].x, vr[u].y), nvalid);                        \
    const uint2 hi = keep_first(make_uint2(vr[u].z, vr[u].w), nvalid - 4);                    \
    const int dd = within >> 1, hf = within & 1, sw = (dd >> 2) & 3;                          \
    uint16_t* vrow = &Vs[BUF][pg * PAGE + dd * 16];                                           \
    *reinterpret_cast<uint2*>(vrow + ((2 * hf) ^ sw) * 4) = lo;                               \
    *reinterpret_cast<uint2*>(vrow + ((2 * hf + 1) ^ sw) * 4) = hi;                           \
  }

  const int ntiles = (it.key1 - it.key0 + 63) / 64;
  const int first_pos = a.meta.tok_pos[it.tok0];
  CHUNK_GLOAD(it.key0);
  CHUNK_LSTORE(it.key0, 0);
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int kt = it.key0 + ti * 64;
    const int cur = ti & 1;
    if ((ti & 15) == 0) STAGE_PIDS((ti >> 4) + 1);
    if (ti + 1 < ntiles) {
      CHUNK_GLOAD(kt + 64);
    }
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
    // causal / end-of-range masks matter only on tiles reaching past the first
    // row's position or past the item's last key (wave-uniform test)
    const bool need_mask = (kt + 64 > it.key1) || (kt + 63 > first_pos);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float sv[16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[kb * 4 + i] = s[kb][rb][i];
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt + kb * 16 + 4 * qd + i;
            if (!(key <= rpos[rb] && key < it.key1)) sv[kb * 4 + i] = -INFINITY;
          }
      }
      float mb = sv[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mb = fmaxf(mb, sv[e]);
      mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      const float mn = fmaxf(m[rb], mb * scale_log2);   // log2 units; -inf while a row saw no key
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(m[rb] - ms);
      float ps[16], lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ps[e] = fast_exp2(fmaf(sv[e], scale_log2, -ms));
        lsum += ps[e];
      }
      l[rb] = l[rb] * alpha + lsum;
      m[rb] = mn;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[rb][j] *= alpha;
      }
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
        const int dd = j * 16 + r, sw = (dd >> 2) & 3;
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vs[cur][(2 * c) * PAGE + dd * 16 + (qd ^ sw) * 4]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vs[cur][(2 * c + 1) * PAGE + dd * 16 + (qd ^ sw) * 4]);
        const bf16x8 vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[0][j] = mfma16x16x32(vf, pf[0][c], acc[0][j]);
        acc[1][j] = mfma16x16x32(vf, pf[1][c], acc[1][j]);
        acc[0][j] = mfma16x16x32(vf, pfl[0][c], acc[0][j]);
        acc[1][j] = mfma16x16x32(vf, pfl[1][c], acc[1][j]);
      }
    }
    if (ti + 1 < ntiles) {
      CHUNK_LSTORE(kt + 64, cur ^ 1);
    }
    __syncthreads();
  }
#undef CHUNK_GLOAD
#undef CHUNK_LSTORE
#undef STAGE_PIDS

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
// merge: o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over a token's
// partials, in one pass with a running maximum (the sums are rescaled when it
// grows), four partials in flight at a time, in partial order (deterministic).
// D/4 lanes per (token, head), each owning 4 consecutive dims.  A partial that
// saw no key of its token has m = -inf and weight 0.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int LPH = D / 4;                 // lanes per (token, head)
  constexpr int PER_BLOCK = 256 / LPH;
  const int sub = threadIdx.x / LPH, l4 = threadIdx.x % LPH;
  const int64_t wid = (int64_t)blockIdx.x * PER_BLOCK + sub;
  const int nq = a.n_q_heads;
  if (wid >= (int64_t)a.n_tokens * nq) return;
  const int t = (int)(wid / nq), h = (int)(wid % nq);
  const int p0 = a.meta.part_off[t], pc = a.meta.part_cnt[t];
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + (size_t)p0 * nq + h;
  const float* src = a.part_o + ((size_t)p0 * nq + h) * D + l4 * 4;
  float M = -INFINITY, L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#define MERGE_STEP(U)                                                                          \
  {                                                                                            \
    float2 mv[U];                                                                              \
    float4 v[U];                                                                               \
    _Pragma("unroll") for (int u = 0; u < U; ++u) {                                            \
      mv[u] = ml[(size_t)(p + u) * nq];                                                        \
      v[u] = *reinterpret_cast<const float4*>(src + (size_t)(p + u) * nq * D);                 \
    }                                                                                          \
    float mb = mv[0].x;                                                                        \
    _Pragma("unroll") for (int u = 1; u < U; ++u) mb = fmaxf(mb, mv[u].x);                     \
    const float mn = fmaxf(M, mb);                                                             \
    if (mn != -INFINITY) {                                                                     \
      const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - mn);                             \
      L *= sc;                                                                                 \
      o.x *= sc; o.y *= sc; o.z *= sc; o.w *= sc;                                              \
      _Pragma("unroll") for (int u = 0; u < U; ++u) {                                          \
        const float w = (mv[u].x == -INFINITY) ? 0.f : fast_exp2(mv[u].x - mn);                \
        L += w * mv[u].y;                                                                      \
        o.x += w * v[u].x; o.y += w * v[u].y; o.z += w * v[u].z; o.w += w * v[u].w;            \
      }                                                                                        \
      M = mn;                                                                                  \
    }                                                                                          \
  }
  int p = 0;
  for (; p + 4 <= pc; p += 4) MERGE_STEP(4);
  for (; p < pc; ++p) MERGE_STEP(1);
#undef MERGE_STEP
  const float inv = 1.0f / L;
  uint2 pk;
  pk.x = pack2bf(o.x * inv, o.y * inv);
  pk.y = pack2bf(o.z * inv, o.w * inv);
  *reinterpret_cast<uint2*>(a.out + (size_t)t * nq * D + (size_t)h * D + l4 * 4) = pk;
}

template <int D>
static hb_status launch_attention_d(const AttnArgs& a, stream_t s, void* const* ev) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipStream_t st = (hipStream_t)s;
  if (ev) hipEventRecord((hipEvent_t)ev[0], st);
  if (a.n_chunk_items > 0)
    hipLaunchKernelGGL(attn_chunk_kernel<D>, dim3((unsigned)a.n_chunk_items * a.n_kv_heads), dim3(256), 0, st, a,
                       scale_log2);
  if (ev) hipEventRecord((hipEvent_t)ev[1], st);
  if (a.n_decode_items > 0)
    hipLaunchKernelGGL(attn_decode_kernel<D>, dim3((a.n_decode_items + 3) / 4, a.n_kv_heads), dim3(256), 0, st, a,
                       scale_log2);
  if (ev) hipEventRecord((hipEvent_t)ev[2], st);
  const int64_t pairs = (int64_t)a.n_tokens * a.n_q_heads, per_block = 256 / (D / 4);
  hipLaunchKernelGGL(attn_merge_kernel<D>, dim3((unsigned)((pairs + per_block - 1) / per_block)), dim3(256), 0, st,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return HB_OK;
}

hb_status launch_attention(const AttnArgs& a, stream_t s, void* const* ev) {
  if (a.n_tokens <= 0) return HB_OK;
  return a.head_dim == 128 ? launch_attention_d<128>(a, s, ev) : launch_attention_d<64>(a, s, ev);
}

}  // namespace hb
