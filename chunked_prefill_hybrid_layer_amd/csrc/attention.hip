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
//     form one 16-row MFMA tile -- for a chunk piece of a few tokens (n x g
//     <= 16: a speculative-verify step) the n tokens' g heads, each row
//     masking the keys past its own position.  S^T = K Q^T and O^T = V^T P^T, so that K
//     rows and V^T rows (the V cache is dim-major inside a page) are MFMA
//     fragments loaded straight from HBM as 16- and 8-byte vectors, and the
//     probabilities never leave the lanes that computed them.  The path is a
//     bandwidth-bound stream over the cached context.  A workgroup is one
//     wave, and the grid runs kv head fastest: the kv heads of an item start
//     together and read the same pages, whose blocks for all kv heads are
//     adjacent in memory (Yi tau=2048 decode 1.20 -> 1.16 ms, 64 decodes at
//     tau=128 86 -> 80 us, against four items per workgroup item-fastest).
//   chunk: one 256-thread workgroup per (item, kv head) holds up to 128
//     (token, head) rows, 32 per wave; 64-key tiles (4 pages) of K and V are
//     staged through double-buffered, swizzled LDS and shared by the 4 waves.

#include <math.h>

#include <algorithm>

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

__device__ __forceinline__ uint4 keep_first8(uint4 v, int n) {
  // keep the first n (0..8) bf16 values of an 8-value vector, zero the rest
  const uint2 lo = keep_first(make_uint2(v.x, v.y), n);
  const uint2 hi = keep_first(make_uint2(v.z, v.w), n - 4);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Decode items: probabilities enter the PV product as two bf16 fragments,
// p = hi + lo with hi = bf16(p) and lo = bf16(p - hi), about 16 significant
// bits (a single bf16 P puts a relative error up to 2^-9 on every weight).  The
// decode kernel is bound by HBM, so the second MFMA per step is free there; the
// chunk kernel, which is not, uses a single bf16 P (see its comment).
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

// Four consecutive output dims starting at element oi of the [T][n_q * d]
// attention output: (v0..v3) * inv as bf16, or as FP8 codes of that over the
// O projection's input scale.  The merge writes its outputs the same way, so a
// token written straight from its one attention item gets the arithmetic of a
// one-partial merge.
__device__ __forceinline__ void store_out4(const AttnArgs& a, size_t oi, float v0, float v1, float v2, float v3,
                                           float inv) {
  if (a.out_inv_scale > 0.0f) {
    const float q = a.out_inv_scale;
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.out) + oi) =
        pack4fp8(v0 * inv * q, v1 * inv * q, v2 * inv * q, v3 * inv * q);
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + oi) =
        make_uint2(pack2bf(v0 * inv, v1 * inv), pack2bf(v2 * inv, v3 * inv));
  }
}

// ----------------------------------------------------------------------------
// decode items
//
// One step covers 32 keys (2 pages).  The item's page ids (at most 64: a
// decode item spans at most kDecodeKvSplitMax = 1024 keys) sit one per lane and
// are broadcast with readlane, so no step waits on a block-table load.  The
// K/V of a step sit in one register buffer (138 VGPRs): three waves per SIMD
// keep more bytes in flight than two double-buffered ones did (measured).
//
// Key order.  Lane l = (qd = l / 16, r = l % 16).  The two QK MFMAs of a step
// take their A rows from permuted keys: row i of MFMA h is key
// 8 (i / 4) + 4 h + i % 4 of the step, so the 4 scores lane l receives from
// MFMA h are keys 8 qd + 4 h .. + 3, and the lane ends up with the 8
// consecutive keys 8 qd .. 8 qd + 7.  Those are exactly the keys of the PV
// MFMA's B operand (P^T) in that lane, and its A operand (V^T: dim r, the
// same 8 keys) is one 16-byte run of the dim-major V page (page qd / 2,
// slots 8 (qd % 2) .. + 7).  So P stays in its lanes, and each V^T load moves
// 1 KB (16 dims x 32 keys) like each K load does.  The K row of MFMA h in lane
// l is key 8 (r / 4) + 4 h + r % 4: page r / 8, slot 8 ((r / 4) % 2) + 4 h +
// r % 4.

// Issue the K (2 x D/32 loads of 16 B) and V^T (D/16 loads of 16 B) fragment
// loads of the step starting at key KB.  Each K load instruction reads 16 keys
// x 32 dims (1 KB) in 64-byte runs, each V^T load 16 dims x 32 keys (1 KB) in
// 16-byte runs; the loads are nontemporal (the KV is read once).  Without a
// second page, its lanes read the first page again (the keys are masked).
#define DEC_ADDR(KB)                                                                          \
  const int _j = ((KB) - it.key0) >> 4;                                                       \
  const bool _has1 = (KB) + 16 < it.key1;                                                     \
  const int _pg0 = __builtin_amdgcn_readlane(my_pg, _j);                                      \
  const int _pg1 = __builtin_amdgcn_readlane(my_pg, _has1 ? _j + 1 : _j);                     \
  const size_t _kb = ((size_t)((r >> 3) ? _pg1 : _pg0) * nkv + kvh) * hs + kslot * 32 + qd * 8; \
  const size_t _vb = ((size_t)((qd >> 1) ? _pg1 : _pg0) * nkv + kvh) * hs + r * 16 + (qd & 1) * 8;

#define DEC_LOAD(KB)                                                                          \
  {                                                                                           \
    DEC_ADDR(KB)                                                                              \
    const uint16_t* _K = static_cast<const uint16_t*>(a.k_cache) + _kb;                       \
    const uint16_t* _V = static_cast<const uint16_t*>(a.v_cache) + _vb;                       \
    _Pragma("unroll") for (int kk = 0; kk < KK; ++kk) {                                       \
      k0[kk] = load_stream16(_K + kk * 512);                                                  \
      k1[kk] = load_stream16(_K + kk * 512 + 4 * 32);                                         \
    }                                                                                         \
    _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) vv[jj] = load_stream16(_V + jj * 256);  \
  }

// FP8 cache: the same fragments as codes (byte offsets equal the bf16 element
// offsets) into raw buffer I.
#define DEC_LOAD8(KB, I)                                                                      \
  {                                                                                           \
    DEC_ADDR(KB)                                                                              \
    const uint8_t* _K = static_cast<const uint8_t*>(a.k_cache) + _kb;                         \
    const uint8_t* _V = static_cast<const uint8_t*>(a.v_cache) + _vb;                         \
    _Pragma("unroll") for (int kk = 0; kk < KK; ++kk) {                                       \
      k0r[I][kk] = load_stream8(_K + kk * 512);                                               \
      k1r[I][kk] = load_stream8(_K + kk * 512 + 4 * 32);                                      \
    }                                                                                         \
    _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) vr[I][jj] = load_stream8(_V + jj * 256); \
  }

// Raw buffer I widened (exactly) into the bf16 buffers.
#define DEC_WIDEN(I)                                                                          \
  {                                                                                           \
    _Pragma("unroll") for (int kk = 0; kk < KK; ++kk) {                                       \
      k0[kk] = fp8x8_bf16x8(k0r[I][kk]);                                                      \
      k1[kk] = fp8x8_bf16x8(k1r[I][kk]);                                                      \
    }                                                                                         \
    _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) vv[jj] = fp8x8_bf16x8(vr[I][jj]);       \
  }

// Scores, online softmax and PV for the step starting at key KB.
#define DEC_COMPUTE(KB)                                                                       \
  {                                                                                           \
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;                                            \
    _Pragma("unroll") for (int kk = 0; kk < KK; ++kk) {                                       \
      s0 = mfma16x16x32(as_bf16x8(k0[kk]), qf[kk], s0);                                       \
      s1 = mfma16x16x32(as_bf16x8(k1[kk]), qf[kk], s1);                                       \
    }                                                                                         \
    /* raw scores of keys KB + 8 qd + e for this lane's row; keys past the  */                \
    /* item's end or past the row's own position are masked                 */                \
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};                   \
    const int _nv = it.key1 - ((KB) + 8 * qd); /* keys of the item among this lane's 8 */     \
    if ((KB) + 32 > lim0) {                                                                   \
      const int _ns = lim - ((KB) + 8 * qd);   /* ... and at or before the row's position */  \
      _Pragma("unroll") for (int e = 0; e < 8; ++e)                                           \
        if (e >= _ns) sv[e] = -INFINITY;                                                      \
    }                                                                                         \
    float mb = sv[0];                                                                         \
    _Pragma("unroll") for (int e = 1; e < 8; ++e) mb = fmaxf(mb, sv[e]);                      \
    mb = fmaxf(mb, xor16(mb));                                                                \
    mb = fmaxf(mb, xor32(mb));                                                                \
    /* running max in log2 units (-inf while the row has seen no key: a     */                \
    /* multi-token row may see none in a step, or in a whole item)          */                \
    const float mn = fmaxf(m, mb * scale_log2);                                               \
    const float ms = (mn == -INFINITY) ? 0.f : mn;                                            \
    const float alpha = fast_exp2(m - ms);                                                    \
    float ps[8], lsum = 0.f;                                                                  \
    _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                           \
      ps[e] = fast_exp2(fmaf(sv[e], scale_log2, -ms));                                        \
      lsum += ps[e];                                                                          \
    }                                                                                         \
    l = l * alpha + lsum;                                                                     \
    m = mn;                                                                                   \
    bf16x8 pf, pfl;                                                                           \
    split_p(ps, pf, pfl);                                                                     \
    if ((KB) + 32 > it.key1) { /* tail: values past the last key may be poisoned */           \
      _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) vv[jj] = keep_first8(vv[jj], _nv);    \
    }                                                                                         \
    _Pragma("unroll") for (int jj = 0; jj < NJ; ++jj) {                                       \
      acc[jj] *= alpha;                                                                       \
      const bf16x8 vf = as_bf16x8(vv[jj]);                                                    \
      acc[jj] = mfma16x16x32(vf, pf, acc[jj]);                                                \
      acc[jj] = mfma16x16x32(vf, pfl, acc[jj]);                                               \
    }                                                                                         \
  }

// F8: the cache holds FP8 e4m3 codes; scale_log2 carries k_scale and the
// partials are scaled by v_scale.
template <int D, bool F8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_decode_kernel(AttnArgs a, float scale_log2) {
  constexpr int KK = D / 32;  // MFMA k-steps over the head dim
  constexpr int NJ = D / 16;  // 16-dim output blocks
  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.x % a.n_kv_heads;
  const int item_idx = blockIdx.x / a.n_kv_heads;
  if (item_idx >= a.n_decode_items) return;
  const hb_attn_item it = a.meta.decode_items[item_idx];
  const int g = a.group, nq = a.n_q_heads, nkv = a.n_kv_heads;
  const int r = lane & 15, qd = lane >> 4;
  // MFMA row r is (token tl, head hq) of the item's n_tok tokens (n_tok x g <=
  // 16; a decode is one token).  Row r sees keys < lim: the item's end, or
  // its own position + 1 if that is earlier; lim0 (the first token's) is the
  // smallest over the rows, so steps ending at or before it need no mask.
  const int tl = r / g, hq = r - tl * g;
  const bool valid = tl < it.n_tok;
  const int lim = valid ? min(it.key1, a.meta.tok_pos[it.tok0 + tl] + 1) : it.key1;
  const int lim0 = min(it.key1, a.meta.tok_pos[it.tok0] + 1);
  const int kslot = 8 * ((r >> 2) & 1) + (r & 3);   // K slot of MFMA 0's row r (MFMA 1: + 4)
  const int t = it.tok0;
  const int32_t* bt = a.meta.block_table + (size_t)it.seq * a.max_pages;
  const int npg = (it.key1 - it.key0 + 15) >> 4;
  const int my_pg = (lane < npg) ? bt[(it.key0 >> 4) + lane] : 0;

  bf16x8 qf[KK];
  {
    const uint16_t* qrow = a.q + (size_t)(t + (valid ? tl : 0)) * nq * D + (size_t)(kvh * g + hq) * D + qd * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = valid ? as_bf16x8(*reinterpret_cast<const uint4*>(qrow + kk * 32)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const size_t hs = (size_t)16 * D;  // elements of one (page, kv head) block

  uint4 k0[KK], k1[KK], vv[NJ];
  if constexpr (F8) {
    // two steps' codes in flight (the bytes of one bf16 step), each widened
    // just before its MFMAs
    uint2 k0r[2][KK], k1r[2][KK], vr[2][NJ];
    for (int kb = it.key0; kb < it.key1; kb += 64) {
      const bool second = kb + 32 < it.key1;
      DEC_LOAD8(kb, 0);
      if (second) DEC_LOAD8(kb + 32, 1);
      DEC_WIDEN(0);
      DEC_COMPUTE(kb);
      if (second) {
        DEC_WIDEN(1);
        DEC_COMPUTE(kb + 32);
      }
    }
  } else {
    for (int kb = it.key0; kb < it.key1; kb += 32) {
      DEC_LOAD(kb);
      DEC_COMPUTE(kb);
    }
  }
  l += xor16(l);
  l += xor32(l);
  if (valid) {
    const int head = kvh * g + hq, tok = t + tl;
    const float vsc = F8 ? a.v_scale : 1.0f;
    if (it.n_split == 1) {
      // the whole context in one item: normalise and write the output
      const float inv = 1.0f / l;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        store_out4(a, ((size_t)tok * nq + head) * D + j * 16 + qd * 4, acc[j][0] * vsc, acc[j][1] * vsc,
                   acc[j][2] * vsc, acc[j][3] * vsc, inv);
    } else {
      const size_t pidx = (size_t)a.meta.part_off[tok] + it.split;
      float* po = a.part_o + (pidx * nq + head) * D;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        *reinterpret_cast<float4*>(po + j * 16 + qd * 4) =
            make_float4(acc[j][0] * vsc, acc[j][1] * vsc, acc[j][2] * vsc, acc[j][3] * vsc);
      if (qd == 0) {
        a.part_ml[(pidx * nq + head) * 2 + 0] = m;
        a.part_ml[(pidx * nq + head) * 2 + 1] = l;
      }
    }
  }
}

#undef DEC_ADDR
#undef DEC_LOAD
#undef DEC_LOAD8
#undef DEC_WIDEN
#undef DEC_COMPUTE

// ----------------------------------------------------------------------------
// chunk items
//
// One 256-thread workgroup per (item, kv head): up to 128 (token, head) rows,
// 32 per wave, one 32-column block of v_mfma_f32_32x32x16_bf16.  Keys go in
// tiles of 64 (4 pages).  Per tile:
//   S^T = K Q^T   (2 key blocks of 32 x D/16 k-steps; Q stays in registers)
//   online softmax on the 32 x 64 scores (lane l holds row l % 32 and 32 of
//   its 64 keys; the other 32 sit in lane l ^ 32)
//   O^T += V^T P^T (D/32 dim blocks x 4 key steps of 16), P as bf16.
//
// K/V reach LDS with direct-to-LDS loads (global_load_lds_dwordx4): wave w
// moves page w of the tile, D/32 1 KB loads each of K and V, double-buffered
// over tiles with one barrier per tile.  Each lane's global address is chosen
// so that the LDS image comes out XOR-swizzled on 16-byte chunks:
//   K image [page 4][dim half D/64][slot 16][64 dims]: 128-byte rows, chunk c
//     of slot t's row at c ^ ((t >> 1) & 7); one 1 KB load fills 8 slots of
//     one half, gathering from two of the cache's 32-dim slices.
//   V image [page 4][dim D][16 keys]: the cache's own (dim-major) page layout;
//     half h (keys 8h..8h+7) of dim row d sits at h ^ ((d >> 3) & 1).
// Both fragment reads are ds_read_b128 without bank conflicts (measured with
// SQ_LDS_BANK_CONFLICT on these exact access patterns: the previous swizzles,
// c ^ f(t) on 64-byte rows and h ^ ((d >> 2) & 1), cost 4 conflict cycles per
// read and 1.7x the read time).
//
// Key order.  The rows of the QK MFMA are a permutation of the 32 keys of a
// block: MFMA row i is key kperm(i).  With it, the 16 scores lane l receives
// for a block are keys 16 (v >> 3) + 8 (l >> 5) + (v & 7), v = 0..15: eight
// consecutive keys per half.  These are exactly the 8 consecutive keys the PV
// MFMA wants in lane l, so P goes from the score registers into the PV
// operand with no data movement, and each V^T fragment is one 16-byte read.
//
// Keys at or past the item's end (a partly used last page, pages past the
// item) are masked to -inf in S; their V entries in LDS are zeroed on the
// item's last tile, since a stale or poisoned value times a zero weight would
// still be NaN.  The weight sum l adds the bf16 probabilities the PV product
// uses, so numerator and denominator carry the same rounding.

constexpr float kLazyMax = 8.0f;

__device__ __forceinline__ int kswz(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int kperm(int i) {
  return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}


// F8: the cache holds FP8 e4m3 codes.  Pages then come through registers
// (each wave loads its page's codes, widens them exactly to bf16 and writes the
// same LDS images the direct-to-LDS loads produce); scale_log2 carries
// k_scale and the partials are scaled by v_scale.
template <int D, bool F8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_chunk_kernel(AttnArgs a, float scale_log2) {
  constexpr int NS = D / 32;      // 1 KB K or V loads per page = PV dim blocks
  constexpr int NH = D / 64;      // 128-byte dim halves of a K row
  constexpr int KS = D / 16;      // QK k-steps
  constexpr int PAGE = 16 * D;    // elements per (page, kv head) block
  constexpr int TILE = 4 * PAGE;  // elements of K (or of V) per 64-key tile
  __shared__ __align__(1024) uint16_t lds[2][2 * TILE];  // [stage][K image | V image]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // kv head fastest: workgroups go round-robin over the 8 XCDs, so kv head h
  // runs on XCD h mod 8 and the prefix K/V every query tile of that head
  // re-reads stays in that XCD's L2
  const hb_attn_item it = a.meta.chunk_items[blockIdx.x / a.n_kv_heads];
  const int kvh = blockIdx.x % a.n_kv_heads;
  const int g = a.group, nq = a.n_q_heads, nkv = a.n_kv_heads;
  const int col = lane & 31, hh = lane >> 5;
  const int32_t* bt = a.meta.block_table + (size_t)it.seq * a.max_pages + (it.key0 >> 4);
  const int npg = (it.key1 - it.key0 + 15) >> 4;
  const int ntiles = (it.key1 - it.key0 + 63) >> 6;

  // Page ids of this wave's pages (page 4 j + wave of the item for tile j),
  // one per lane for a window of 64 tiles, broadcast with readlane.  The
  // first window is requested before Q, so the first tile's loads wait only
  // for it and Q's loads overlap them.  Window w + 1 (if the item has one) is
  // requested at the first tile of window w into pnext and taken over when
  // its first tile is issued, 63 tiles later.
  // The loads are unconditional (indexes clamped into the item, results
  // selected afterwards): a load under a branch makes every later wait a
  // wait for all loads.
  auto fetch_window = [&](int w) {
    const int pi = 4 * (64 * w + lane) + wave;
    const int v = bt[max(0, min(pi, npg - 1))];
    return pi < npg ? v : 0;
  };
  int pcur = fetch_window(0), pnext = 0;

  // this lane's query row and its Q^T fragments (dims 16 ks + 8 hh .. +7)
  const int row = wave * 32 + col;
  const int tl = row / g, hq = row - tl * g;
  const bool valid = tl < it.n_tok;
  const int t = it.tok0 + tl;
  const int tq = valid ? t : it.tok0;   // rows past the item's tokens read its first row
  const int rpos_l = a.meta.tok_pos[tq];
  const int rpos = valid ? rpos_l : -1;
  bf16x8 qf[KS];
  {
    const uint16_t* qrow = a.q + ((size_t)tq * nq + kvh * g + hq) * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 u = *reinterpret_cast<const uint4*>(qrow + ks * 16);
      qf[ks] = as_bf16x8(valid ? u : make_uint4(0, 0, 0, 0));
    }
  }

  // LDS fragment offsets (elements, stage 0).  K: MFMA row col of key block kb
  // is key 32 kb + kperm(col): page 2 kb + (col >> 4), slot kperm(col) & 15;
  // k-step ks reads dim half ks >> 2, chunk (2 ks + hh) & 7 of that half.
  // V: dim row 32 db + col of page p, half hh.
  const int kslot = kperm(col) & 15;
  const int koff = ((col >> 4) * NH * 16 + kslot) * 64;
  int kch[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kch[j] = (((2 * j + hh) & 7) ^ kswz(kslot)) * 8;
  const int voff = TILE + col * 16 + ((hh ^ ((col >> 3) & 1)) * 8);

  // DMA lane offsets inside a 1 KB load.  K load (half h, slots 8 b .. 8 b + 7)
  // of a page: lane -> slot 8 b + lane / 8, LDS chunk lane % 8, which holds
  // logical chunk c = (lane % 8) ^ kswz(slot): dims 64 h + 8 c .. +7, in the
  // cache's slice 2 h + c / 4 at chunk c % 4.  V (dim lane / 2 of the block,
  // LDS half lane % 2) fetches half (lane % 2) ^ ((dim >> 3) & 1).
  int kdma[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int sl = 8 * b + (lane >> 3), c = (lane & 7) ^ kswz(sl);
    kdma[b] = ((c >> 2) * 16 + sl) * 32 + (c & 3) * 8;
  }
  const int vdma = (lane >> 1) * 16 + (((lane & 1) ^ ((lane >> 4) & 1)) * 8);

  auto issue_tile = [&](int tile, int st) {
    // wave-uniform: does the tile have this wave's page?
    if (4 * tile + wave < npg) {
      const int page = __builtin_amdgcn_readlane(pcur, tile & 63);
      const size_t base = ((size_t)page * nkv + kvh) * PAGE;
      const uint16_t* kg = static_cast<const uint16_t*>(a.k_cache) + base;
      const uint16_t* vg = static_cast<const uint16_t*>(a.v_cache) + base + vdma;
      uint16_t* dst = &lds[st][0];
      // K: load s = 2 h + b covers half h, slots 8 b .. 8 b + 7 (page image
      // [half][slot][64]: element offset 512 s within the page's image)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        __builtin_amdgcn_global_load_lds((const void*)(kg + (s >> 1) * 1024 + kdma[s & 1]),
                                         (lds_ptr_t)(dst + (wave * NS + s) * 512), 16, 0, 0);
#pragma unroll
      for (int u = 0; u < NS; ++u)
        __builtin_amdgcn_global_load_lds((const void*)(vg + u * 512), (lds_ptr_t)(dst + TILE + wave * PAGE + u * 512), 16, 0,
                                         0);
    }
  };

  // FP8 pages: a page block is D * 16 bytes, loaded as D / 64 units of 1 KB
  // (16 bytes per lane).  Unit L of K holds slice L / 32, slot (L / 2) % 16,
  // dims 16 (L % 2) .. +15 of that slice; unit L of V is dim row L.
  constexpr int NL8 = D / 64;
  uint4 kr8[NL8], vr8[NL8];
  auto load_tile8 = [&](int tile) {
    if (4 * tile + wave < npg) {
      const int page = __builtin_amdgcn_readlane(pcur, tile & 63);
      const size_t base = ((size_t)page * nkv + kvh) * PAGE + lane * 16;
#pragma unroll
      for (int u = 0; u < NL8; ++u) {
        kr8[u] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k_cache) + base + u * 1024);
        vr8[u] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v_cache) + base + u * 1024);
      }
    }
  };
  auto store_tile8 = [&](int tile, int st) {
    if (4 * tile + wave < npg) {
      uint16_t* kimg = &lds[st][0] + wave * PAGE;      // [dim half][slot][64]
      uint16_t* vimg = &lds[st][TILE] + wave * PAGE;   // [dim][16 keys]
#pragma unroll
      for (int u = 0; u < NL8; ++u) {
        const int L = u * 64 + lane;
        const int sl = (L >> 1) & 15, c0 = ((L >> 5) & 1) * 4 + 2 * (L & 1);
        uint16_t* krow = kimg + ((L >> 6) * 16 + sl) * 64;
        *reinterpret_cast<uint4*>(krow + ((c0 ^ kswz(sl)) * 8)) = fp8x8_bf16x8(make_uint2(kr8[u].x, kr8[u].y));
        *reinterpret_cast<uint4*>(krow + (((c0 + 1) ^ kswz(sl)) * 8)) = fp8x8_bf16x8(make_uint2(kr8[u].z, kr8[u].w));
        uint16_t* vrow = vimg + L * 16;
        const int sw = (L >> 3) & 1;
        *reinterpret_cast<uint4*>(vrow + sw * 8) = fp8x8_bf16x8(make_uint2(vr8[u].x, vr8[u].y));
        *reinterpret_cast<uint4*>(vrow + (sw ^ 1) * 8) = fp8x8_bf16x8(make_uint2(vr8[u].z, vr8[u].w));
      }
    }
  };

  f32x16 acc[NS];
#pragma unroll
  for (int db = 0; db < NS; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int first_pos = a.meta.tok_pos[it.tok0];

  if (F8) {
    load_tile8(0);
    store_tile8(0, 0);
  } else {
    issue_tile(0, 0);
  }
  for (int ti = 0; ti < ntiles; ++ti) {
    const int kt = it.key0 + ti * 64;
    const int cur = ti & 1;
    // tile ti has landed for every wave (each wave's own direct-to-LDS loads
    // are complete before it reaches the barrier), and every wave is done
    // with tile ti - 1
    WAIT_VMCNT(0);
    __syncthreads();
    if ((ti & 63) == 0 && ti + 64 < ntiles) pnext = fetch_window((ti >> 6) + 1);
    if (ti + 1 < ntiles) {
      if (((ti + 1) & 63) == 0) pcur = pnext;
      if (F8) load_tile8(ti + 1);
      else issue_tile(ti + 1, cur ^ 1);
    }
    if (kt + 64 > it.key1) {
      // last tile, partly past the item's end: zero V of keys >= key1
      uint16_t* vimg = &lds[cur][TILE];
      for (int c = tid; c < 4 * D * 2; c += 256) {
        const int p = c / (2 * D), dim = (c >> 1) % D, hs = c & 1;
        const int nvalid = it.key1 - (kt + 16 * p + 8 * (hs ^ ((dim >> 3) & 1)));
        if (nvalid < 8) {
          uint4* ch = reinterpret_cast<uint4*>(vimg + p * PAGE + dim * 16 + hs * 8);
          *ch = nvalid <= 0 ? make_uint4(0, 0, 0, 0) : keep_first8(*ch, nvalid);
        }
      }
      __syncthreads();
    }
    const uint16_t* kimg = &lds[cur][0];
    // The QK and PV MFMAs run at raised wave priority, the softmax at the
    // normal one: of the two waves of a SIMD (from two co-resident items),
    // the one in an MFMA phase then issues each MFMA as soon as the pipe
    // frees, and the other's softmax fills the issue slots in between.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);

    // QK: the two key blocks' accumulation chains alternate, and the fragment
    // reads run four ahead of the MFMAs that use them
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
    bf16x8 kf[2 * KS];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i)   // i = 2 ks + kb
      kf[i] = *reinterpret_cast<const bf16x8*>(kimg + (i & 1) * 2 * NS * 512 + koff + ((i >> 1) >> 2) * 1024 +
                                               kch[(i >> 1) & 3]);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) s[i & 1] = mfma32x32x16(kf[i], qf[i >> 1], s[i & 1]);
    // V fragments of the tile, read now so that their latency hides under the
    // softmax (vf[q * NS + db]: key step q, dim block db)
    bf16x8 vf[4 * NS];
#pragma unroll
    for (int i = 0; i < 4 * NS; ++i)
      vf[i] = *reinterpret_cast<const bf16x8*>(kimg + voff + (i / NS) * PAGE + (i % NS) * 512);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // causal / end-of-range masks matter only on tiles reaching past the first
    // row's position or past the item's last key (wave-uniform test)
    if ((kt + 64 > it.key1) || (kt + 63 > first_pos)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt + 32 * kb + 16 * (v >> 3) + 8 * hh + (v & 7);
          if (!(key <= rpos && key < it.key1)) s[kb][v] = -INFINITY;
        }
    }
    // row maximum (NaN-propagating maximum: v_maximum3_f32 chains, no operand
    // canonicalisation)
    float mb = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = kb ? 0 : 1; v < 16; ++v) mb = __builtin_elementwise_maximum(mb, s[kb][v]);
    mb = __builtin_elementwise_maximum(mb, xor32(mb)) * scale_log2;
    // The reference maximum m of a row (log2 units; -inf while the row saw no
    // key) moves only when a tile exceeds it by more than kLazyMax: the
    // probabilities then stay below 2^kLazyMax, and the accumulator rescale
    // (a wave-uniform branch) is skipped on most tiles.  o and l are scaled by
    // the same 2^-m, so the result does not depend on where m sits.
    const bool grow = mb > m + kLazyMax;
    const float mn = grow ? mb : m;
    const float ms = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = grow ? fast_exp2(m - ms) : 1.0f;
    m = mn;
    // probabilities as bf16 pairs: pk[kb][j] holds keys of score registers 2j, 2j + 1
    uint32_t pk[2][8];
    float lsum = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pk[kb][j] = pack2bf(fast_exp2(fmaf(s[kb][2 * j], scale_log2, -ms)),
                            fast_exp2(fmaf(s[kb][2 * j + 1], scale_log2, -ms)));
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[kb][j]), ones, lsum, false);
      }
    l = l * alpha + lsum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < NS; ++db) acc[db] *= alpha;
    }
    // key step q = 2 kb + h covers the tile's page q: keys 16 q + 8 hh .. +7 in this lane
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 pb = as_bf16x8(make_uint4(pk[q >> 1][4 * (q & 1)], pk[q >> 1][4 * (q & 1) + 1],
                                             pk[q >> 1][4 * (q & 1) + 2], pk[q >> 1][4 * (q & 1) + 3]));
#pragma unroll
      for (int db = 0; db < NS; ++db) acc[db] = mfma32x32x16(vf[q * NS + db], pb, acc[db]);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // FP8: the next tile's codes, loaded before this tile's compute, go into
    // the other LDS images (every wave finished reading them before this
    // iteration's barrier)
    if (F8 && ti + 1 < ntiles) store_tile8(ti + 1, cur ^ 1);
  }

  l += xor32(l);
  if (valid) {
    const int head = kvh * g + hq;
    const float vsc = F8 ? a.v_scale : 1.0f;
    // acc[db][v] is dim 32 db + 8 (v >> 2) + 4 hh + (v & 3)
    if (it.n_split == 1) {
      // all of the tile's keys in one item: normalise and write the output
      const float inv = 1.0f / l;
      const size_t ob = ((size_t)t * nq + head) * D + 4 * hh;
#pragma unroll
      for (int db = 0; db < NS; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          store_out4(a, ob + 32 * db + 8 * j, acc[db][4 * j] * vsc, acc[db][4 * j + 1] * vsc,
                     acc[db][4 * j + 2] * vsc, acc[db][4 * j + 3] * vsc, inv);
    } else {
      const size_t pidx = (size_t)a.meta.part_off[t] + it.split;
      float* po = a.part_o + (pidx * nq + head) * D + 4 * hh;
#pragma unroll
      for (int db = 0; db < NS; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(po + 32 * db + 8 * j) =
              make_float4(acc[db][4 * j] * vsc, acc[db][4 * j + 1] * vsc, acc[db][4 * j + 2] * vsc,
                          acc[db][4 * j + 3] * vsc);
      if (hh == 0) {
        a.part_ml[(pidx * nq + head) * 2 + 0] = m;
        a.part_ml[(pidx * nq + head) * 2 + 1] = l;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// merge: o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over a token's
// partials, with a running maximum (the sums are rescaled when it grows), in
// a fixed order (deterministic).  D/4 lanes per lane group, each owning 4
// consecutive dims.  A partial that saw no key of its token has m = -inf and
// weight 0.
//
// Partials first, first + stride, ... (count of them) of the (token, head)
// pair whose first partial is p0, into the running (M, L, o): rounds of four
// loaded together, slots past the last counting as empty (m = -inf).
template <int D>
__device__ __forceinline__ void merge_partials(const AttnArgs& a, int h, int l4, int p0, int first, int stride,
                                               int count, float& M, float& L, float4& o) {
  const int nq = a.n_q_heads;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + (size_t)(p0 + first) * nq + h;
  const float* src = a.part_o + ((size_t)(p0 + first) * nq + h) * D + l4 * 4;
  for (int p = 0; p < count; p += 4) {
    float2 mv[4];
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (p + u < count) {
        const size_t q = (size_t)(p + u) * stride;
        mv[u] = ml[q * nq];
        v[u] = *reinterpret_cast<const float4*>(src + q * nq * D);
      } else {
        mv[u] = make_float2(-INFINITY, 0.f);
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    const float mb = fmaxf(fmaxf(mv[0].x, mv[1].x), fmaxf(mv[2].x, mv[3].x));
    const float mn = fmaxf(M, mb);
    if (mn != -INFINITY) {
      const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - mn);
      L *= sc;
      o.x *= sc; o.y *= sc; o.z *= sc; o.w *= sc;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = (mv[u].x == -INFINITY) ? 0.f : fast_exp2(mv[u].x - mn);
        L += w * mv[u].y;
        o.x += w * v[u].x; o.y += w * v[u].y; o.z += w * v[u].z; o.w += w * v[u].w;
      }
      M = mn;
    }
  }
}

// One lane group per (token, head) pair, except with G > 1: the decode
// tokens [a.merge_tok0, n_tokens) then take G lane groups per pair, in the
// workgroups from chunk_blocks on.  Group g merges partials g, g + G, ..., and
// group 0 combines the groups' results through LDS in group order, so a pair
// with up to 4 G partials takes one round of loads.  With G = 1 every token
// takes the plain running-maximum pass.
constexpr int kMergeMaxGroups = 4;

template <int D, int G>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int chunk_blocks) {
  constexpr int LPH = D / 4;                       // lanes per group
  constexpr int PER_BLOCK = 256 / LPH;             // lane groups per workgroup
  static_assert(PER_BLOCK % G == 0, "whole (token, head) pairs per workgroup");
  const int sub = threadIdx.x / LPH, l4 = threadIdx.x % LPH;
  const int nq = a.n_q_heads;
  if (G == 1 || (int)blockIdx.x < chunk_blocks) {
    const int64_t wid = (int64_t)blockIdx.x * PER_BLOCK + sub;
    if (wid >= (int64_t)(G == 1 ? a.n_tokens : a.merge_tok0) * nq) return;
    const int t = (int)(wid / nq), h = (int)(wid % nq);
    const int p0 = a.meta.part_off[t], pc = a.meta.part_cnt[t];
    if (pc <= 1) return;   // written by its one attention item
    float M = -INFINITY, L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    merge_partials<D>(a, h, l4, p0, 0, 1, pc, M, L, o);
    // FP8: codes of o / o_scale (the O projection's input)
    store_out4(a, (size_t)t * nq * D + (size_t)h * D + l4 * 4, o.x, o.y, o.z, o.w, 1.0f / L);
    return;
  }
  // decode tokens, G groups per pair: every thread of these workgroups
  // reaches the barrier
  __shared__ float4 sm_o[PER_BLOCK][LPH];
  __shared__ float2 sm_ml[PER_BLOCK];
  const int pair = sub / G, grp = sub % G;
  const int64_t wid = (int64_t)a.merge_tok0 * nq + (int64_t)((int)blockIdx.x - chunk_blocks) * (PER_BLOCK / G) + pair;
  int t = 0, h = 0, p0 = 0, pc = 0;
  if (wid < (int64_t)a.n_tokens * nq) {
    t = (int)(wid / nq);
    h = (int)(wid % nq);
    p0 = a.meta.part_off[t];
    pc = a.meta.part_cnt[t];
  }
  const bool active = pc > 1;   // else none, or written by its one attention item
  float M = -INFINITY, L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (active && grp < pc) merge_partials<D>(a, h, l4, p0, grp, G, (pc - grp + G - 1) / G, M, L, o);
  sm_o[sub][l4] = o;
  if (l4 == 0) sm_ml[sub] = make_float2(M, L);
  __syncthreads();
  if (!active || grp != 0) return;
  float Mx = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) Mx = fmaxf(Mx, sm_ml[sub + g].x);
  float Lx = 0.f;
  float4 ox = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float2 mlg = sm_ml[sub + g];
    const float w = (mlg.x == -INFINITY) ? 0.f : fast_exp2(mlg.x - Mx);
    const float4 og = sm_o[sub + g][l4];
    Lx += w * mlg.y;
    ox.x += w * og.x; ox.y += w * og.y; ox.z += w * og.z; ox.w += w * og.w;
  }
  store_out4(a, (size_t)t * nq * D + (size_t)h * D + l4 * 4, ox.x, ox.y, ox.z, ox.w, 1.0f / Lx);
}

// Lane groups per decode (token, head) pair, from the packed partial counts.
// Chunk tokens keep one: their few partials (the tile's key splits) load in
// one or two rounds, and grouping them measured slower (at tau = 128, 8
// partials each: 9.2-10.1 us for the whole merge with two groups against
// 8.0-8.5 with one).  Decode tokens take the fewest groups (1, 2 or 4)
// that minimise the region's residency rounds (workgroups over the 8 per CU
// that fit: 4 waves each, about 52 VGPRs) times the load rounds of its
// longest pair: at tau = 128 (64 decodes, up to 26 partials) four groups took
// the merge kernel from 8.0 to 5.2 us; at Yi tau = 2048 (28672 decode
// pairs, mostly 2-5 partials) more workgroups cost more rounds than they save
// (four groups: 27 -> 32 us), and the plan keeps one.
void merge_plan(const hb_meta_header* h, const void* meta_host, int* tok0, int* groups) {
  const int T = h->n_tokens, nq = h->n_q_heads;
  const int per_block = 1024 / h->head_dim;           // lane groups per 256-thread workgroup
  const int32_t* pc = reinterpret_cast<const int32_t*>(static_cast<const char*>(meta_host) + h->off_part_cnt);
  *tok0 = T - h->n_decodes;                           // decodes are the last tokens of the packed order
  *groups = 1;
  int max_pc = 0;
  for (int t = *tok0; t < T; ++t) max_pc = std::max(max_pc, (int)pc[t]);
  if (max_pc <= 4) return;
  const int64_t pairs = (int64_t)h->n_decodes * nq;
  int64_t best = -1;
  for (int g = 1; g <= kMergeMaxGroups; g *= 2) {
    const int64_t wgs = (pairs * g + per_block - 1) / per_block;
    const int64_t cost = ((wgs + 8 * kNumCU - 1) / (8 * kNumCU)) * ((max_pc + 4 * g - 1) / (4 * g));
    if (best < 0 || cost < best) {
      best = cost;
      *groups = g;
    }
  }
}

template <int D, bool F8>
static hb_status launch_attention_d(const AttnArgs& a, stream_t s, void* const* ev) {
  // FP8: keys are code * k_scale, so k_scale joins the score scale
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D) * (F8 ? a.k_scale : 1.0f);
  hipStream_t st = (hipStream_t)s;
  auto mark = [&](int i) -> bool { return !ev || !ev[i] || hipEventRecord((hipEvent_t)ev[i], st) == hipSuccess; };
  // one workgroup per (item, kv head): the grid's x extent holds at most 2^31 - 1
  if ((int64_t)a.n_chunk_items * a.n_kv_heads > INT32_MAX || (int64_t)a.n_decode_items * a.n_kv_heads > INT32_MAX)
    return fail(HB_E_SHAPE, "attention: more (item, kv head) pairs than one grid holds");
  if (!mark(0)) return fail(HB_E_HIP, "attention: stage event record failed");
  if (a.n_chunk_items > 0)
    hipLaunchKernelGGL((attn_chunk_kernel<D, F8>), dim3((unsigned)a.n_chunk_items * a.n_kv_heads), dim3(256), 0, st, a,
                       scale_log2);
  if (!mark(1)) return fail(HB_E_HIP, "attention: stage event record failed");
  if (a.n_decode_items > 0)
    hipLaunchKernelGGL((attn_decode_kernel<D, F8>), dim3((unsigned)a.n_decode_items * a.n_kv_heads), dim3(64), 0, st,
                       a, scale_log2);
  if (!mark(2)) return fail(HB_E_HIP, "attention: stage event record failed");
  if (a.n_merge_tokens > 0) {
    const int64_t per_block = 256 / (D / 4), nq = a.n_q_heads, G = a.merge_groups;
    if (G != 1 && G != 2 && G != kMergeMaxGroups) return fail(HB_E_SHAPE, "attention merge: 1, 2 or 4 lane groups");
    if (a.merge_tok0 < 0 || a.merge_tok0 > a.n_tokens) return fail(HB_E_SHAPE, "attention merge: bad decode start");
    const int64_t first = G == 1 ? a.n_tokens : a.merge_tok0;   // tokens of one group per pair
    const int64_t chunk_blocks = (first * nq + per_block - 1) / per_block;
    const int64_t blocks = chunk_blocks + ((a.n_tokens - first) * nq * G + per_block - 1) / per_block;
    if (blocks > INT32_MAX) return fail(HB_E_SHAPE, "attention merge: grid too large");
    const dim3 grid((unsigned)blocks);
    if (G == 1) hipLaunchKernelGGL((attn_merge_kernel<D, 1>), grid, dim3(256), 0, st, a, (int)chunk_blocks);
    else if (G == 2) hipLaunchKernelGGL((attn_merge_kernel<D, 2>), grid, dim3(256), 0, st, a, (int)chunk_blocks);
    else hipLaunchKernelGGL((attn_merge_kernel<D, kMergeMaxGroups>), grid, dim3(256), 0, st, a, (int)chunk_blocks);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return HB_OK;
}

hb_status launch_attention(const AttnArgs& a, stream_t s, void* const* ev) {
  if (a.n_tokens <= 0) return HB_OK;
  if (a.kv_fp8)
    return a.head_dim == 128 ? launch_attention_d<128, true>(a, s, ev) : launch_attention_d<64, true>(a, s, ev);
  return a.head_dim == 128 ? launch_attention_d<128, false>(a, s, ev) : launch_attention_d<64, false>(a, s, ev);
}

}  // namespace hb
