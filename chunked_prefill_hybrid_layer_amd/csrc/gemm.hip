// Packed-token projections for gfx950: C[M][N] = A[M][K] . W[N][K]^T with
// bf16 operands and fp32 accumulation on MFMA (v_mfma_f32_16x16x32_bf16).
//
// Every token of the hybrid batch -- chunk and decode alike -- goes through
// the same projections, which is what makes the linear-layer cost depend on
// the batch's token count n ("Sarathi-Serve reading notes" §1.6: T_math =
// 2 n d_in d_out / FLOPS, T_mem = (d_in d_out bytes_w + n d_in bytes_a) / BW;
// "Chunked Prefill", hybrid-iteration roofline 2(c+b)Psi).
//
// Tiles (workgroup BM x BN, K stages of 64):
//   128 x 128 / 128 x 96, 8 waves (2 per SIMD): more, smaller tiles where the
//                        256-row ones leave CUs idle or need a K split (the
//                        128 x 96 one gives a 512-token, 6144-wide QKV exactly
//                        256 tiles with no split)
//   256 x 128, 8 waves
//   256 x 256 / 256 x 224, 8 waves: half the L2 and LDS operand traffic per
//                        flop of 256 x 128; the 224-wide tile makes
//                        Mistral-size gate/up exactly 256 tiles for 256 CUs.
// A planner picks tile and K split per problem from a cost model fitted to
// measured times.
// Two waves per SIMD: on gfx950 one wave per SIMD issues back-to-back
// independent 16x16x32 MFMAs at about two thirds of the rate two waves reach
// (measured).  Both operands are K-contiguous and reach LDS through
// direct-to-LDS loads (global_load_lds_dwordx4, no VGPR staging), one 1 KB
// wave load landing contiguously; the global address of every lane is chosen
// so that the LDS image is XOR-swizzled on 16-byte chunks and the MFMA
// fragment reads are bank-conflict free.  The MFMA operand fragments of the
// next K step are read from LDS into registers while the MFMAs of the current
// one run (sched_group_barrier interleaves them).  The narrow tiles keep a
// ring of 3-4 LDS stages; the wide tiles keep two 64 KB stages with one
// barrier per stage (see gemm_sub_kernel).  Workgroups are renumbered so that
// each XCD (own L2) walks a contiguous run of tiles, M fastest, and keeps to
// one K slice of a split (block_tile).
//
// Split-K (grid.z > 1, when the tiles alone leave CUs idle): each K slice writes an fp32 partial tile and a reduce kernel adds the slices in a
// fixed order (results do not depend on timing) before applying the epilogue.
//
// Epilogues (the accumulator tile is staged through LDS as fp32, except
// SwiGLU, which stages only its bf16 or FP8 outputs):
//   QKV:      RoPE (rotate-half, table-driven) on q and k; q -> bf16 buffer;
//             k and v -> the paged KV cache at the tokens' slots (KV append).
//             The weight rows are read in an order that interleaves the two
//             halves of every head, so that each rotated pair is two adjacent
//             GEMM columns and any tile width holds whole pairs.
//   residual: out = res + acc (fp32).
//   SwiGLU:   each 16-column MFMA block holds eight FFN units, their gate rows
//             in its first eight columns and the matching up rows in the last
//             eight; out = silu(gate) * up (bf16, or FP8 codes), formed in
//             registers after one lane swap.

#include <cmath>

#include "device_common.h"

namespace hb {

// Workgroup tile configurations.  WM x WN waves each own a (BM/WM) x (BN/WN)
// block of 16x16 MFMA tiles; a stage holds BK columns of K for the A rows and
// the weight rows of the tile.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int NST_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NST = NST_;
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int FM = BM / WM / 16, FN = BN / WN / 16;  // 16-row / 16-column blocks per wave
  static constexpr int KS = BK / 32;                          // MFMA K steps per stage
  static constexpr int CPR = BK / 8;                          // 16-byte chunks per LDS row
  static constexpr int RPL = 64 / CPR;                        // rows per 1 KB wave load
  static constexpr int STAGE_ELEMS = (BM + BN) * BK;
  static constexpr int MAIN_LDS = NST * STAGE_ELEMS * 2;
  static constexpr int CS_LD = BN + 4;                        // fp32 staging row stride
  static constexpr int EPI_ROWS = BM * CS_LD * 4 <= 160 * 1024 - 4096 ? BM : BM / 2;
  static constexpr int EPI_LDS = EPI_ROWS * CS_LD * 4;
  static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
  static constexpr int TOTAL_LOADS = (BM + BN) / RPL;         // 1 KB loads per stage
  static constexpr int LOADS = (TOTAL_LOADS + WAVES - 1) / WAVES;  // per wave (some waves one fewer)
  static_assert((BM + BN) % RPL == 0, "stage rows must split into whole wave loads");
  static_assert(EPI_ROWS % (BM / WM) == 0, "epilogue passes must hold whole waves");
};
using Tile128W8 = Tile<128, 128, 64, 4, 2, 4>;  // ring pipeline, 8 waves (two per SIMD)
using Tile128N96 = Tile<128, 96, 64, 4, 2, 4>;  // ring pipeline, 8 waves
using Tile256 = Tile<256, 128, 64, 4, 2, 3>;    // ring pipeline (gemm_kernel)
using TileW256 = Tile<256, 256, 64, 4, 2, 2>;   // sub-step pipeline (gemm_sub_kernel)
using TileW224 = Tile<256, 224, 64, 4, 2, 2>;   // sub-step pipeline (gemm_sub_kernel)

// Bank-conflict-free placement of 16-byte chunk c of LDS row r, as measured
// with SQ_LDS_BANK_CONFLICT on gfx950 for the MFMA fragment reads (16
// consecutive rows, one chunk column per 16 lanes): eight consecutive lanes
// must land in distinct 16-byte bank groups of a 256-byte window.
//   128-byte rows: c ^ (r & 7)   ((r ^ (r >> 3)) & 7 conflicted on 60 % of cycles)
//    64-byte rows: c ^ ((r >> 1) & 3)   (c ^ (r & 3) conflicted on half of them)
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return CPR == 8 ? c ^ (r & 7) : c ^ ((r >> 1) & 3);
}

// Cache policy of the weight rows' direct-to-LDS loads in the 256-row
// sub-step and wave-specialised kernels when at most kStreamWeightsMaxRowTiles
// row tiles share each weight tile: sc0 | nt (miss the CU's L1, stream through
// L2).  The activation rows are re-read by every tile column; streamed
// weights leave L2 to them, which lowers the average load latency that bounds
// the stage loop (measured: 256x224 gate/up and specialised down at 512
// tokens 3-7 % faster).  With more row tiles the weight tile itself is re-read
// and streaming it costs: at 8 row tiles O lost 5 % while down gained 5 %, at
// 128 row tiles (a 32768-token prefill) gate/up lost 6 %.  The 128-row ring
// kernel keeps the default policy: streaming there lost 4-22 % (QKV, O, down;
// it gained only on gate/up at 128 tokens).  Activation rows always load with
// the default policy.
constexpr int kWeightLoadPolicy = 3;
constexpr int kStreamWeightsMaxRowTiles = 2;

template <int MODE, int BN>
__device__ __forceinline__ const uint16_t* weight_row(const GemmArgs& g, int n, int n0) {
  if (MODE == kGemmQkvRope) {
    // GEMM columns run over each head with the two halves interleaved:
    // column 2j of a head is dim j, column 2j + 1 is dim j + d/2, so every
    // rotated pair sits in two adjacent columns of one tile
    const int d = g.head_dim, h = n / d, p = n - h * d;
    n = h * d + (p >> 1) + (p & 1) * (d >> 1);
    if (n < g.n0) return g.w0 + (size_t)n * g.K;
    if (n < g.n0 + g.n1) return g.w1 + (size_t)(n - g.n0) * g.K;
    return g.w2 + (size_t)(n - g.n0 - g.n1) * g.K;
  } else if (MODE == kGemmSwiglu) {
    // tile column c: unit n0/2 + 8 (c / 16) + c % 8, gate for c % 16 < 8, else up
    const int c = n - n0, unit = n0 / 2 + (c >> 4) * 8 + (c & 7);
    return ((c & 8) ? g.w1 : g.w0) + (size_t)unit * g.K;
  } else {
    return g.w0 + (size_t)n * g.K;
  }
}
// FP8 projections: the scale of the weight row behind GEMM column n (the
// same mapping as weight_row).
template <int MODE, int BN>
__device__ __forceinline__ float weight_scale(const GemmArgs& g, int n, int n0) {
  if (MODE == kGemmQkvRope) {
    const int d = g.head_dim, h = n / d, p = n - h * d;
    n = h * d + (p >> 1) + (p & 1) * (d >> 1);
    if (n < g.n0) return g.ws0[n];
    if (n < g.n0 + g.n1) return g.ws1[n - g.n0];
    return g.ws2[n - g.n0 - g.n1];
  } else if (MODE == kGemmSwiglu) {
    const int c = n - n0, unit = n0 / 2 + (c >> 4) * 8 + (c & 7);
    return (c & 8) ? g.ws1[unit] : g.ws0[unit];
  } else {
    return g.ws0[n];
  }
}

// QKV output of token m, GEMM columns n .. n + 7 (n a multiple of 8): dims
// i0 .. i0 + 3 (x0) and i0 + d/2 .. i0 + d/2 + 3 (x1) of one head, where
// i0 = (n mod d) / 2.  q and k are rotated by the token's position (rotate-
// half: dim i pairs with dim i + d/2), q goes to the q buffer, k and v to the
// paged cache at the token's slot (bf16, or FP8 codes of x / scale).  q and K
// stores are 8 bytes (4 in FP8); V (dim-major in a page) takes one store per dim.
// The rotation's cos/sin pairs of dims i0 .. i0 + 3 at the token's position
// and the token's cache slot, requested on their own so that a caller can
// issue them before its other loads.
struct QkvTokenData {
  float4 cs01, cs23;
  int slot;
};
__device__ __forceinline__ QkvTokenData qkv_token_data(const GemmArgs& g, int m, int n) {
  const int d = g.head_dim, half = d >> 1;
  const int hb = n / d, i0 = (n - hb * d) >> 1;
  const int c = hb * d + i0;
  QkvTokenData t;
  t.slot = g.slot[m];
  if (c < (g.n_q_heads + g.n_kv_heads) * d) {
    const float4* rp = reinterpret_cast<const float4*>(g.rope + ((size_t)g.tok_pos[m] * half + i0) * 2);
    t.cs01 = rp[0];
    t.cs23 = rp[1];
  }
  return t;
}

__device__ __forceinline__ void qkv_store4(const GemmArgs& g, int m, int n, const float (&x0)[4],
                                           const float (&x1)[4], const QkvTokenData& td) {
  const int d = g.head_dim, half = d >> 1;
  const int qdim = g.n_q_heads * d, kdim = g.n_kv_heads * d;
  const int hb = n / d, i0 = (n - hb * d) >> 1;
  const int c = hb * d + i0;  // natural column of dim i0
  if (c < qdim + kdim) {
    const float4 cs01 = td.cs01, cs23 = td.cs23;
    const float cs[4] = {cs01.x, cs01.z, cs23.x, cs23.z}, sn[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
    float y0[4], y1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y0[e] = x0[e] * cs[e] - x1[e] * sn[e];
      y1[e] = x1[e] * cs[e] + x0[e] * sn[e];
    }
    const uint2 lo = make_uint2(pack2bf(y0[0], y0[1]), pack2bf(y0[2], y0[3]));
    const uint2 hi = make_uint2(pack2bf(y1[0], y1[1]), pack2bf(y1[2], y1[3]));
    if (c < qdim) {
      uint16_t* qo = g.out_b + (size_t)m * qdim + c;
      *reinterpret_cast<uint2*>(qo) = lo;
      *reinterpret_cast<uint2*>(qo + half) = hi;
    } else if (g.kv_fp8) {
      // FP8 K page block: [d/32][16 slots][32] codes of k / k_scale
      const int kvh = (c - qdim) / d;
      const int sl = td.slot;
      uint8_t* kb = static_cast<uint8_t*>(g.k_cache) + ((size_t)(sl >> 4) * g.n_kv_heads + kvh) * 16 * d +
                    (sl & 15) * 32;
      const float s = g.k_inv_scale;
      *reinterpret_cast<uint32_t*>(kb + (i0 >> 5) * 512 + (i0 & 31)) =
          pack4fp8(y0[0] * s, y0[1] * s, y0[2] * s, y0[3] * s);
      *reinterpret_cast<uint32_t*>(kb + ((i0 + half) >> 5) * 512 + ((i0 + half) & 31)) =
          pack4fp8(y1[0] * s, y1[1] * s, y1[2] * s, y1[3] * s);
    } else {
      const int kvh = (c - qdim) / d;
      const int sl = td.slot;
      // K page block: [d/32][16 slots][32]; dims i0 .. i0 + 3 share a 32-dim slice
      uint16_t* kb = static_cast<uint16_t*>(g.k_cache) + ((size_t)(sl >> 4) * g.n_kv_heads + kvh) * 16 * d +
                     (sl & 15) * 32;
      *reinterpret_cast<uint2*>(kb + (i0 >> 5) * 512 + (i0 & 31)) = lo;
      *reinterpret_cast<uint2*>(kb + ((i0 + half) >> 5) * 512 + ((i0 + half) & 31)) = hi;
    }
  } else {
    const int kvh = (c - qdim - kdim) / d;
    const int sl = td.slot;
    const size_t vo = (((size_t)(sl >> 4) * g.n_kv_heads + kvh) * d + i0) * 16 + (sl & 15);
    if (g.kv_fp8) {
      uint8_t* vp = static_cast<uint8_t*>(g.v_cache) + vo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vp[e * 16] = fp8_code(x0[e] * g.v_inv_scale);
        vp[(half + e) * 16] = fp8_code(x1[e] * g.v_inv_scale);
      }
    } else {
      uint16_t* vp = static_cast<uint16_t*>(g.v_cache) + vo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vp[e * 16] = f2bf(x0[e]);
        vp[(half + e) * 16] = f2bf(x1[e]);
      }
    }
  }
}


// Which tile (tm, tn) and K slice z a workgroup takes.  Workgroups reach the
// eight XCDs (each with its own L2) round-robin in launch order, x fastest,
// then z.  Each XCD gets a contiguous run of tiles, M fastest, so the row
// tiles that share a weight tile run on one XCD.  With a K split into z
// slices (8 % z == 0) each XCD also keeps to one slice, 8 / z XCDs per slice:
// the slice's activation columns, which every tile of the XCD reads, can then
// stay in its L2, where handing every XCD tiles of every slice made each one
// stream the whole activation matrix (the 4-way split down projection at 512
// tokens read its 14.7 MB of activations once per XCD).
struct BlockTile {
  int tm, tn, z;
};
__device__ __forceinline__ bool xcd_slices() {
  return ((gridDim.x * gridDim.z) & 7) == 0 && (8 % gridDim.z) == 0;
}
__device__ __forceinline__ int block_slice() {
  if (!xcd_slices()) return blockIdx.z;
  const int xcd = (blockIdx.x + gridDim.x * blockIdx.z) & 7;
  return xcd / (8 / gridDim.z);
}
__device__ __forceinline__ BlockTile block_tile(int tiles_m) {
  int tile = blockIdx.x, z = blockIdx.z;
  if (xcd_slices()) {
    const int L = blockIdx.x + gridDim.x * blockIdx.z;   // launch order
    const int xcd = L & 7, i = L >> 3, per_slice = 8 / gridDim.z;
    z = xcd / per_slice;
    tile = (xcd % per_slice) * (gridDim.x * gridDim.z / 8) + i;
  }
  return BlockTile{tile % tiles_m, tile / tiles_m, z};
}

// Epilogue, in passes of EPI_ROWS tile rows staged through LDS as fp32:
// acc[i][j][e] is C[wm*WROWS + i*16 + 4*(lane>>4) + e][wn*WCOLS + j*16 + (lane&15)].
template <int MODE, class TL, bool F8 = true>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, f32x4 (&acc)[TL::FM][TL::FN], unsigned char* smem,
                                              int m0, int n0, int wm, int wn, int lane, int tid) {
  constexpr int BM = TL::BM, BN = TL::BN, NT = TL::THREADS, FM = TL::FM, FN = TL::FN;
  constexpr int WROWS = BM / TL::WM, WCOLS = BN / TL::WN, CS_LD = TL::CS_LD;
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int ER = TL::EPI_ROWS;
  if (F8 && g.f8) {   // codes -> values: input scale times the weight row's scale, per column
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WCOLS + j * 16 + (lane & 15);
      const float sc = g.a_scale * weight_scale<MODE, BN>(g, n, n0);
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][j] *= sc;
    }
  }
#pragma unroll
  for (int p = 0; p < BM / ER; ++p) {
    if (p > 0) __syncthreads();
    if (wm * WROWS >= p * ER && wm * WROWS < (p + 1) * ER) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Cs[(wm * WROWS - p * ER + i * 16 + 4 * (lane >> 4) + e) * CS_LD + wn * WCOLS + j * 16 + (lane & 15)] =
                acc[i][j][e];
    }
    __syncthreads();
    const int mb = m0 + p * ER;   // first token of this pass
    if (gridDim.z > 1) {  // split-K: raw fp32 partial into this workgroup's slice
      float* out = g.part + (size_t)block_slice() * g.M * g.N;
      for (int idx = tid; idx < ER * BN / 4; idx += NT) {
        const int r = idx / (BN / 4), c4 = idx % (BN / 4);
        const int m = mb + r;
        if (m >= g.M) continue;
        *reinterpret_cast<float4*>(out + (size_t)m * g.N + n0 + c4 * 4) =
            *reinterpret_cast<const float4*>(Cs + r * CS_LD + c4 * 4);
      }
    } else if (MODE == kGemmResidual) {
      for (int idx = tid; idx < ER * BN / 4; idx += NT) {
        const int r = idx / (BN / 4), c4 = idx % (BN / 4);
        const int m = mb + r;
        if (m >= g.M) continue;
        float4 o = *reinterpret_cast<const float4*>(Cs + r * CS_LD + c4 * 4);
        const float4 rr = *reinterpret_cast<const float4*>(g.res + (size_t)m * g.ldo + n0 + c4 * 4);
        o.x += rr.x;
        o.y += rr.y;
        o.z += rr.z;
        o.w += rr.w;
        *reinterpret_cast<float4*>(g.out_f + (size_t)m * g.ldo + n0 + c4 * 4) = o;
      }
    } else if (MODE == kGemmSwiglu) {
      const int f0 = n0 / 2;
      for (int idx = tid; idx < ER * (BN / 8); idx += NT) {
        const int r = idx / (BN / 8), c4 = idx % (BN / 8);
        const int m = mb + r;
        if (m >= g.M) continue;
        // units 4 c4 .. 4 c4 + 3: gate columns 16 (c4 / 2) + 4 (c4 % 2) .. +3, up 8 further
        const float* gr = Cs + r * CS_LD + (c4 >> 1) * 16 + (c4 & 1) * 4;
        const float* ur = gr + 8;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = gr[e];
          o[e] = z / (1.0f + __expf(-z)) * ur[e];
        }
        if (g.f8) {   // the down projection's input: FP8 codes of out / a_scale
          const float q = g.out_inv_scale;
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(g.out_b) + (size_t)m * g.ldo + f0 + c4 * 4) =
              pack4fp8(o[0] * q, o[1] * q, o[2] * q, o[3] * q);
        } else {
          uint2 pk;
          pk.x = pack2bf(o[0], o[1]);
          pk.y = pack2bf(o[2], o[3]);
          *reinterpret_cast<uint2*>(g.out_b + (size_t)m * g.ldo + f0 + c4 * 4) = pk;
        }
      }
    } else {  // QKV + RoPE + KV append: one thread per (token, 4 rotated pairs)
      for (int idx = tid; idx < ER * (BN / 8); idx += NT) {
        const int r = idx / (BN / 8), c8 = idx % (BN / 8);
        const int m = mb + r;
        if (m >= g.M) continue;
        const float4 a = *reinterpret_cast<const float4*>(Cs + r * CS_LD + c8 * 8);
        const float4 b = *reinterpret_cast<const float4*>(Cs + r * CS_LD + c8 * 8 + 4);
        const float x0[4] = {a.x, a.z, b.x, b.z}, x1[4] = {a.y, a.w, b.y, b.w};
        qkv_store4(g, m, n0 + c8 * 8, x0, x1, qkv_token_data(g, m, n0 + c8 * 8));
      }
    }
  }
}

// SwiGLU epilogue of the bf16 kernels.  Every SwiGLU tile orders its columns
// so that each 16-column MFMA block holds eight FFN units: column c is unit
// n0/2 + 8 (c / 16) + c % 8, a gate row for c % 16 < 8 and the matching up
// row for c % 16 >= 8 (weight_row).  acc[i][j][e] is tile row
// wm*WROWS + i*16 + 4*(lane>>4) + e, column wn*WCOLS + j*16 + (lane&15), so a
// unit's gate and up values sit in lanes l and l ^ 8 of a 16-lane row.  A gate
// lane swaps its rows e = 2, 3 for the partner's up values of rows 0, 1 (a
// row_ror:8 DPP move, which within 16 lanes is exactly lane ^ 8), and each
// lane forms two outputs: unit wn*WCOLS/2 + 8j + lane % 8, rows e = 0, 1 (gate
// lanes) or 2, 3 (up lanes).  The bf16 outputs are staged row-major in LDS (one
// pass) and written out in 16-byte chunks.  The arithmetic is the staged
// epilogue's, so outputs are bit-identical; it saves the fp32 tile's LDS round
// trip (wide specialised gate/up at 512 tokens: 106-107 -> 101-104 us).
// F8OUT (FP8 projections): each lane first scales its values by the input
// scale and its column's weight-row scale, and the outputs are e4m3 codes of
// out / a_scale (one byte each).
// has_acc: the calling wave holds an accumulator block (not a producer).
template <class TL, bool F8OUT = false>
__device__ __forceinline__ void swiglu_epilogue_regs(const GemmArgs& g, f32x4 (&acc)[TL::FM][TL::FN],
                                                     unsigned char* smem, int m0, int n0, bool has_acc, int wm,
                                                     int wn, int lane, int tid) {
  constexpr int BM = TL::BM, FM = TL::FM, FN = TL::FN, WROWS = BM / TL::WM, WCOLS = TL::BN / TL::WN;
  constexpr int UNITS = TL::BN / 2;
  // staging row stride in output elements (units + pad, rows 16-byte aligned)
  constexpr int OLD = F8OUT ? UNITS + 16 : UNITS + 8;
  constexpr int EB = F8OUT ? 1 : 2;             // bytes per output element
  constexpr int CPRO = UNITS * EB / 16;         // 16-byte output chunks per row
  static_assert(BM * OLD * EB <= TL::LDS, "output staging fits the kernel's LDS");
  static_assert((UNITS * EB) % 16 == 0, "rows of whole 16-byte chunks");
  uint16_t* ob = reinterpret_cast<uint16_t*>(smem);
  uint8_t* ob8 = smem;
  if (has_acc) {
    const bool gate_lane = (lane & 8) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        f32x4 a4 = acc[i][j];
        if (F8OUT)   // codes -> values: input scale times this lane's column (weight row) scale
          a4 *= g.a_scale * weight_scale<kGemmSwiglu, TL::BN>(g, n0 + wn * WCOLS + j * 16 + (lane & 15), n0);
        const float s0 = gate_lane ? a4[2] : a4[0], s1 = gate_lane ? a4[3] : a4[1];
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s0), 0x128, 0xf, 0xf, false));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s1), 0x128, 0xf, 0xf, false));
        const float g0 = gate_lane ? a4[0] : r0, g1 = gate_lane ? a4[1] : r1;
        const float u0 = gate_lane ? r0 : a4[2], u1 = gate_lane ? r1 : a4[3];
        const float o0 = g0 / (1.0f + __expf(-g0)) * u0, o1 = g1 / (1.0f + __expf(-g1)) * u1;
        const int row = wm * WROWS + i * 16 + 4 * (lane >> 4) + (gate_lane ? 0 : 2);
        const int unit = wn * (WCOLS / 2) + j * 8 + (lane & 7);
        if (F8OUT) {   // the down projection's input: FP8 codes of out / a_scale
          ob8[row * OLD + unit] = fp8_code(o0 * g.out_inv_scale);
          ob8[(row + 1) * OLD + unit] = fp8_code(o1 * g.out_inv_scale);
        } else {
          const uint32_t pk = pack2bf(o0, o1);
          ob[row * OLD + unit] = (uint16_t)(pk & 0xffffu);
          ob[(row + 1) * OLD + unit] = (uint16_t)(pk >> 16);
        }
      }
  }
  __syncthreads();
  const int f0 = n0 / 2;
  uint8_t* out = reinterpret_cast<uint8_t*>(g.out_b);
  for (int idx = tid; idx < BM * CPRO; idx += TL::THREADS) {
    const int r = idx / CPRO, c = idx % CPRO;
    const int m = m0 + r;
    if (m >= g.M) continue;
    *reinterpret_cast<uint4*>(out + ((size_t)m * g.ldo + f0) * EB + c * 16) =
        *reinterpret_cast<const uint4*>(smem + (size_t)r * OLD * EB + c * 16);
  }
}

// bf16 kernels: SwiGLU in registers, the other modes through gemm_epilogue
// (F8SCALE: whether that instantiation keeps the runtime FP8 column-scale
// branch; each kernel keeps the variant its register allocation was tuned
// with: compiling it out made the 256 x 128 specialised kernel spill 4 VGPRs).
template <int MODE, class TL, bool F8SCALE = true>
__device__ __forceinline__ void gemm_epilogue_bf16(const GemmArgs& g, f32x4 (&acc)[TL::FM][TL::FN], unsigned char* smem,
                                                   int m0, int n0, bool has_acc, int wm, int wn, int lane, int tid) {
  if (MODE == kGemmSwiglu)   // never split: the planner keeps SwiGLU whole
    swiglu_epilogue_regs<TL>(g, acc, smem, m0, n0, has_acc, wm, wn, lane, tid);
  else
    gemm_epilogue<MODE, TL, F8SCALE>(g, acc, smem, m0, n0, wm, wn, lane, tid);
}

// F8: A and the weights are e4m3 codes (K counted in 16-bit units, so a 64-unit
// stage row is 128 codes).  The LDS images, loads and swizzles are the bf16
// ones; a lane's MFMA operand is the two 16-byte chunks qd and 4 + qd of its
// row (the chunks the two bf16 K steps read), one 16x16x128 MFMA per stage.
template <int MODE, class TL, bool F8>
__global__ __launch_bounds__(TL::THREADS) void gemm_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, NST = TL::NST, SE = TL::STAGE_ELEMS;
  constexpr int NL = TL::LOADS, NT = TL::THREADS, FM = TL::FM, FN = TL::FN, KS = TL::KS, CPR = TL::CPR;
  constexpr int RPL = TL::RPL, WROWS = BM / TL::WM, WCOLS = BN / TL::WN, CS_LD = TL::CS_LD;
  __shared__ __align__(16) unsigned char smem[TL::LDS];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int tiles_m = (g.M + BM - 1) / BM;
  const BlockTile btile = block_tile(tiles_m);
  const int tm = btile.tm, tn = btile.tn;
  const int m0 = tm * BM, n0 = tn * BN;
  // K slice of this workgroup (split-K along grid.z)
  const int nk = (g.K / BK) / gridDim.z;
  const int k_first = btile.z * nk;

  // DMA mapping: load q = wave + WAVES * i covers rows [RPL q, RPL q + RPL) of
  // the stage image (A rows first, then B rows); lane l lands at row
  // RPL q + l / CPR, chunk l % CPR, i.e. it loads logical chunk (l % CPR) ^ f(row).
  // When the loads of a stage do not divide evenly over the waves, the waves
  // short of one repeat the stage's last load (same bytes to the same LDS
  // address), so that every wave counts the same number of loads per stage.
  // bf16: waves 0-3 issue a stage's loads right after the barrier, waves 4-7
  // after the stage's MFMAs: the two waves of a SIMD issue at different times,
  // so one of them has MFMAs to issue while the other waits on its load queue.
  // (FP8 keeps every wave issuing after the barrier: its fragment registers
  // leave no room for the longer live ranges.)
  const bool late = !F8 && wave >= 4;
  const uint16_t* gsrc[NL];
  int ldst[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = min(wave + TL::WAVES * i, TL::TOTAL_LOADS - 1);
    const int r = RPL * q + lane / CPR;                      // row of the stage image
    const int rr = r < BM ? r : r - BM;                       // row within A or B
    const int c = swz<CPR>(rr, lane % CPR);
    gsrc[i] = (r < BM ? g.a + (size_t)min(m0 + rr, g.M - 1) * g.lda : weight_row<MODE, BN>(g, n0 + rr, n0)) +
              (size_t)k_first * BK + c * 8;
    ldst[i] = RPL * q * BK;
  }
#define ISSUE_STAGE(KT)                                                                              \
  {                                                                                                  \
    uint16_t* _st = lds + ((KT) % NST) * SE;                                                         \
    _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                   \
        __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)(KT) * BK),                 \
                                         (lds_ptr_t)(_st + ldst[i]), 16, 0, 0);                      \
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA operand fragments.  The MFMAs of a stage run column block by column
  // block (j outer); B fragment j of the next stage is read into fb[kk][j]
  // right after its last use, the A fragments of the next stage go to the
  // other half of fa.  So the LDS reads of stage kt+1 overlap the MFMAs of
  // stage kt with one A buffer extra, not a full second fragment set.
  bf16x8 fa[2][KS][FM], fb[KS][FN];
#define FRAG_A(B, KK, I, AS)                                                                     \
  {                                                                                              \
    const int _r = wm * WROWS + (I) * 16 + (lane & 15);                                          \
    fa[B][KK][I] = *reinterpret_cast<const bf16x8*>((AS) + _r * BK + swz<CPR>(_r, (KK) * 4 + (lane >> 4)) * 8); \
  }
#define FRAG_B(KK, J, BS)                                                                        \
  {                                                                                              \
    const int _r = wn * WCOLS + (J) * 16 + (lane & 15);                                          \
    fb[KK][J] = *reinterpret_cast<const bf16x8*>((BS) + _r * BK + swz<CPR>(_r, (KK) * 4 + (lane >> 4)) * 8); \
  }
#define LOAD_FRAGS(B, KT)                                                                        \
  {                                                                                              \
    const uint16_t* _as = lds + ((KT) % NST) * SE;                                               \
    const uint16_t* _bs = _as + BM * BK;                                                         \
    _Pragma("unroll") for (int kk = 0; kk < KS; ++kk) {                                          \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) FRAG_A(B, kk, i, _as);                      \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) FRAG_B(kk, j, _bs);                         \
    }                                                                                            \
  }
  // MFMAs of the stage in fa[CUR]/fb; with NEXT, the fragments of stage KT1
  // are read in between (A into fa[NXT]).
#define MFMAS(CUR, NXT, KT1, NEXT)                                                               \
  {                                                                                              \
    const uint16_t* _as = lds + ((KT1) % NST) * SE;                                              \
    const uint16_t* _bs = _as + BM * BK;                                                         \
    _Pragma("unroll") for (int kk = 0; kk < KS; ++kk)                                            \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                             \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                             \
        acc[i][j] = mfma16x16x32(fa[CUR][kk][i], fb[kk][j], acc[i][j]);                          \
      if (NEXT) {                                                                                \
        FRAG_B(kk, j, _bs);                                                                      \
        if (j < FM) FRAG_A(NXT, kk, j, _as);                                                     \
        if (j == FN - 1) _Pragma("unroll") for (int i = FN; i < FM; ++i) FRAG_A(NXT, kk, i, _as); \
      }                                                                                          \
    }                                                                                            \
  }
  // One stage: wait until stage KT+1 has landed in LDS (own loads, then every
  // wave's via the barrier), refill the buffer of stage KT (every wave holds
  // its fragments in registers by now), then the MFMAs of stage KT with the
  // fragment reads of stage KT+1 in between.
  static_assert(FN >= FM, "A fragments are read alongside the first FM column blocks");
  constexpr int LEAD = NST;   // stages issued ahead of the one computed

  // FP8 operands: 32 codes per lane (chunks qd and 4 + qd of the row).  The
  // chunks are read as bf16x8, the type the bf16 path reads: read as uint4,
  // the compiler put a wait for every in-flight direct-to-LDS load before each
  // LDS read of the stage loop, which serialised the prefetch.
  i32x8 fa8[2][FM], fb8[FN];
#define FRAG8(DST, BASE, R)                                                                      \
  {                                                                                              \
    const int _r = (R);                                                                          \
    const bf16x8 _lo = *reinterpret_cast<const bf16x8*>((BASE) + _r * BK + swz<CPR>(_r, (lane >> 4)) * 8); \
    const bf16x8 _hi = *reinterpret_cast<const bf16x8*>((BASE) + _r * BK + swz<CPR>(_r, 4 + (lane >> 4)) * 8); \
    DST = cat_i32x8(__builtin_bit_cast(uint4, _lo), __builtin_bit_cast(uint4, _hi));             \
  }
#define LOAD_FRAGS8(B, KT)                                                                       \
  {                                                                                              \
    const uint16_t* _as = lds + ((KT) % NST) * SE;                                               \
    const uint16_t* _bs = _as + BM * BK;                                                         \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) FRAG8(fa8[B][i], _as, wm * WROWS + i * 16 + (lane & 15)); \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) FRAG8(fb8[j], _bs, wn * WCOLS + j * 16 + (lane & 15)); \
  }
#define MFMAS8(CUR, NXT, KT1, NEXT)                                                              \
  {                                                                                              \
    const uint16_t* _as = lds + ((KT1) % NST) * SE;                                              \
    const uint16_t* _bs = _as + BM * BK;                                                         \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                             \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                             \
        acc[i][j] = mfma16x16x128_f8(fa8[CUR][i], fb8[j], acc[i][j]);                            \
      if (NEXT) {                                                                                \
        FRAG8(fb8[j], _bs, wn * WCOLS + j * 16 + (lane & 15));                                   \
        if (j < FM) FRAG8(fa8[NXT][j < FM ? j : 0], _as, wm * WROWS + j * 16 + (lane & 15));      \
      }                                                                                          \
    }                                                                                            \
  }
#define STEP(CUR, NXT, KT)                                                                       \
  {                                                                                              \
    const int _later = min(LEAD - 2, nk - 2 - (KT));                                             \
    if (_later >= 3) WAIT_VMCNT(3 * NL);                                                         \
    else if (_later == 2) WAIT_VMCNT(2 * NL);                                                    \
    else if (_later == 1) WAIT_VMCNT(NL);                                                        \
    else WAIT_VMCNT(0);                                                                          \
    WAIT_LGKM0();                                                                                \
    __builtin_amdgcn_s_barrier();                                                                \
    asm volatile("" ::: "memory");                                                               \
    if (!late && (KT) + LEAD < nk) ISSUE_STAGE((KT) + LEAD);                                   \
    if constexpr (F8) {                                                                          \
      MFMAS8(CUR, NXT, (KT) + 1, true);                                                          \
      _Pragma("unroll") for (int _j = 0; _j < FM; ++_j) {                                        \
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                      \
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                                       \
      }                                                                                          \
      _Pragma("unroll") for (int _j = FM; _j < FN; ++_j) {                                       \
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                      \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                       \
      }                                                                                          \
    } else {                                                                                     \
      MFMAS(CUR, NXT, (KT) + 1, true);                                                           \
      _Pragma("unroll") for (int _k = 0; _k < KS; ++_k) {                                        \
        _Pragma("unroll") for (int _j = 0; _j < FM; ++_j) {                                      \
          __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                    \
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                     \
        }                                                                                        \
        _Pragma("unroll") for (int _j = FM; _j < FN; ++_j) {                                     \
          __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                    \
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
    if (late && (KT) + LEAD < nk) ISSUE_STAGE((KT) + LEAD);                                    \
  }

#pragma unroll
  for (int s = 0; s < LEAD; ++s)
    if (s < nk) ISSUE_STAGE(s);
  {
    const int later = min(LEAD - 1, nk - 1);
    if (later >= 3) WAIT_VMCNT(3 * NL);
    else if (later == 2) WAIT_VMCNT(2 * NL);
    else if (later == 1) WAIT_VMCNT(NL);
    else WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (F8) {
      LOAD_FRAGS8(0, 0);
    } else {
      LOAD_FRAGS(0, 0);
    }
  }
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    STEP(0, 1, kt);
    STEP(1, 0, kt + 1);
  }
  if (kt + 1 < nk) {
    STEP(0, 1, kt);
    WAIT_LGKM0();
    if constexpr (F8) {
      MFMAS8(1, 0, 0, false);
    } else {
      MFMAS(1, 0, 0, false);
    }
  } else {
    WAIT_LGKM0();
    if constexpr (F8) {
      MFMAS8(0, 1, 0, false);
    } else {
      MFMAS(0, 1, 0, false);
    }
  }
#undef STEP
#undef MFMAS
#undef MFMAS8
#undef LOAD_FRAGS8
#undef FRAG8
#undef LOAD_FRAGS
#undef FRAG_A
#undef FRAG_B
#undef ISSUE_STAGE
  WAIT_VMCNT(0);
  __syncthreads();

  if (F8 && MODE == kGemmSwiglu)
    swiglu_epilogue_regs<TL, true>(g, acc, smem, m0, n0, true, wm, wn, lane, tid);
  else if (F8)
    gemm_epilogue<MODE, TL>(g, acc, smem, m0, n0, wm, wn, lane, tid);
  else
    gemm_epilogue_bf16<MODE, TL>(g, acc, smem, m0, n0, true, wm, wn, lane, tid);
}

// Sub-step pipeline (stages of BK = 64, two LDS buffers, one barrier per
// stage): the operand fragments of each 32-deep K sub-step are read from LDS
// during the MFMAs of the sub-step before it.  The barrier sits between the
// two sub-steps of a stage: by then every wave has read the second half of
// the stage into registers, so the DMA refills that buffer with the stage
// after next while the second half is computed.  B fragments are single-
// buffered except the last two column blocks, whose reads are issued first,
// so the reads that must finish before the barrier are never the last issued.
template <int MODE, class TL>
__global__ __launch_bounds__(TL::THREADS) void gemm_sub_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, SE = TL::STAGE_ELEMS;
  constexpr int FM = TL::FM, FN = TL::FN, CPR = TL::CPR, RPL = TL::RPL;
  constexpr int WROWS = BM / TL::WM, WCOLS = BN / TL::WN;
  static_assert(TL::NST == 2 && TL::KS == 2 && FN >= FM + 2, "sub-step pipeline layout");
  __shared__ __align__(16) unsigned char smem[TL::LDS];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int tiles_m = (g.M + BM - 1) / BM;
  const BlockTile btile = block_tile(tiles_m);
  const int tm = btile.tm, tn = btile.tn;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (g.K / BK) / gridDim.z;
  const int k_first = btile.z * nk;

  // Load split: the A rows' loads (activations, L2-resident) go to waves
  // 4-7, the weight rows' loads (first touch from HBM) to waves 0-3.  Waves
  // 0-3 issue right after the barrier, waves 4-7 after the MFMAs of the second
  // sub-step, so the two waves of a SIMD issue at different times and one of
  // them always has MFMAs to issue while the other waits on its load queue;
  // the loads with the longer latency get the longer slack.
  constexpr int LA = BM / RPL, LB = TL::BN / RPL;          // A and weight loads per stage
  constexpr int NLA = LA / 4, NLB = (LB + 3) / 4;
  constexpr int NLS = NLA > NLB ? NLA : NLB;
  static_assert(LA % 4 == 0 && TL::WAVES == 8, "load split layout");
  const bool a_side = wave >= 4;
  const int nl = a_side ? NLA : (LB / 4 + ((wave & 3) < LB % 4 ? 1 : 0));
  const bool stream_w = tiles_m <= kStreamWeightsMaxRowTiles;
  const uint16_t* gsrc[NLS];
  int ldst[NLS];
#pragma unroll
  for (int i = 0; i < NLS; ++i) {
    const int q = a_side ? (wave & 3) + 4 * i : LA + min((wave & 3) + 4 * i, LB - 1);
    const int r = RPL * q + lane / CPR;
    const int rr = r < BM ? r : r - BM;
    const int c = swz<CPR>(rr, lane % CPR);
    gsrc[i] = (r < BM ? g.a + (size_t)min(m0 + rr, g.M - 1) * g.lda : weight_row<MODE, BN>(g, n0 + rr, n0)) +
              (size_t)k_first * BK + c * 8;
    ldst[i] = RPL * q * BK;
  }
#define ISSUE_STAGE(KT)                                                                              \
  {                                                                                                  \
    uint16_t* _st = lds + ((KT) & 1) * SE;                                                           \
    _Pragma("unroll") for (int i = 0; i < NLS; ++i)                                                  \
      if (i < nl) {                                                                                  \
        if (a_side || !stream_w)                                                                     \
          __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)(KT) * BK),               \
                                           (lds_ptr_t)(_st + ldst[i]), 16, 0, 0);                    \
        else                                                                                         \
          __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)(KT) * BK),               \
                                           (lds_ptr_t)(_st + ldst[i]), 16, 0, kWeightLoadPolicy);    \
      }                                                                                              \
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa[2][FM], fb[FN - 2], fbl[2][2];
  const int arow = wm * WROWS + (lane & 15), brow = wn * WCOLS + (lane & 15);
#define RD(BASE, R, KK) \
  (*reinterpret_cast<const bf16x8*>((BASE) + (R) * BK + swz<CPR>((R), (KK) * 4 + (lane >> 4)) * 8))
  // compute the sub-step held in fa[CUR], fb, fbl[CUR]; with NEXT, read the
  // fragments of sub-step (stage S1, half KK1) in between.
#define SUBSTEP(CUR, NXT, S1, KK1, NEXT)                                                          \
  {                                                                                               \
    const uint16_t* _as = lds + ((S1) & 1) * SE;                                                  \
    const uint16_t* _bs = _as + BM * BK;                                                          \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                              \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                              \
        acc[i][j] = mfma16x16x32(fa[CUR][i], j < FN - 2 ? fb[j < FN - 2 ? j : 0] : fbl[CUR][j - (FN - 2) >= 0 ? j - (FN - 2) : 0], acc[i][j]); \
      if (NEXT) {                                                                                 \
        if (j == 0) {                                                                             \
          fbl[NXT][0] = RD(_bs, brow + (FN - 2) * 16, KK1);                                      \
          fbl[NXT][1] = RD(_bs, brow + (FN - 1) * 16, KK1);                                      \
        }                                                                                         \
        if (j < FN - 2) fb[j < FN - 2 ? j : 0] = RD(_bs, brow + j * 16, KK1);                     \
        if (j >= 1 && j <= FM) fa[NXT][j >= 1 && j <= FM ? j - 1 : 0] = RD(_as, arow + (j - 1) * 16, KK1); \
      }                                                                                           \
    }                                                                                             \
    if (NEXT) {                                                                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                                          \
      _Pragma("unroll") for (int _j = 1; _j <= FM; ++_j) {                                        \
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                       \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                        \
      }                                                                                           \
      _Pragma("unroll") for (int _j = FM + 1; _j < FN - 2; ++_j) {                                \
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                       \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                        \
      }                                                                                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * FM, 0);                                     \
    }                                                                                             \
  }

  ISSUE_STAGE(0);
  WAIT_VMCNT(0);
  if (nk > 1) ISSUE_STAGE(1);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  {
    const uint16_t* _as = lds;
    const uint16_t* _bs = _as + BM * BK;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = RD(_as, arow + i * 16, 0);
#pragma unroll
    for (int j = 0; j < FN - 2; ++j) fb[j] = RD(_bs, brow + j * 16, 0);
    fbl[0][0] = RD(_bs, brow + (FN - 2) * 16, 0);
    fbl[0][1] = RD(_bs, brow + (FN - 1) * 16, 0);
  }
  for (int st = 0; st + 1 < nk; ++st) {
    SUBSTEP(0, 1, st, 1, true);
    WAIT_VMCNT(0);   // stage st+1 (the only one in flight) has landed
    WAIT_LGKM0();    // this wave's reads of the second half of stage st are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (!a_side && st + 2 < nk) ISSUE_STAGE(st + 2);
    SUBSTEP(1, 0, st + 1, 0, true);
    if (a_side && st + 2 < nk) ISSUE_STAGE(st + 2);
  }
  SUBSTEP(0, 1, nk - 1, 1, true);
  SUBSTEP(1, 0, 0, 0, false);
#undef SUBSTEP
#undef RD
#undef ISSUE_STAGE
  WAIT_VMCNT(0);
  __syncthreads();
  gemm_epilogue_bf16<MODE, TL>(g, acc, smem, m0, n0, true, wm, wn, lane, tid);
}

// FP8 wide tiles (256 x 224, 256 x 256).  A 64-unit stage row is 128 codes,
// so one 16x16x128 MFMA per (i, j) covers a stage and the bf16 sub-step split
// has no FP8 counterpart; with the fragments of the next stage held in
// registers as the ring kernel does, these tiles spill.  Here two LDS stages
// and one barrier per stage: after the barrier every wave is done with the
// stage before (its buffer is refilled with the next stage at once) and the
// current stage has landed; the stage's A fragments are read first, the B
// fragments one column block ahead of its MFMAs.  The next stage's loads
// have one stage of MFMAs to land.  The loads and LDS images are the ring
// kernel's (K counted in 16-bit units), the weight rows stream through L2
// under the same rule as the bf16 wide tiles.  (A schedule that gave the
// weight rows two stages of slack -- all B fragments read first, a second
// barrier, then the B rows of the stage after next -- measured the same:
// 65-66 us on the 512-token gate/up, 242 us at 2048 tokens.)
template <int MODE, class TL>
__global__ __launch_bounds__(TL::THREADS) void gemm_f8w_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, SE = TL::STAGE_ELEMS;
  constexpr int NL = TL::LOADS, FM = TL::FM, FN = TL::FN, CPR = TL::CPR, RPL = TL::RPL;
  constexpr int WROWS = BM / TL::WM, WCOLS = BN / TL::WN;
  static_assert(TL::NST == 2, "two LDS stages");
  __shared__ __align__(16) unsigned char smem[TL::LDS];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const int tiles_m = (g.M + BM - 1) / BM;
  const BlockTile btile = block_tile(tiles_m);
  const int tm = btile.tm, tn = btile.tn;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (g.K / BK) / gridDim.z;
  const int k_first = btile.z * nk;

  // DMA mapping of the ring kernel: load q = wave + WAVES * i covers rows
  // [RPL q, RPL q + RPL) of the stage image; waves short of a load repeat the
  // stage's last one.
  const bool stream_w = tiles_m <= kStreamWeightsMaxRowTiles;
  const uint16_t* gsrc[NL];
  int ldst[NL];
  bool wrow[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = min(wave + TL::WAVES * i, TL::TOTAL_LOADS - 1);
    const int r = RPL * q + lane / CPR;
    const int rr = r < BM ? r : r - BM;
    const int c = swz<CPR>(rr, lane % CPR);
    gsrc[i] = (r < BM ? g.a + (size_t)min(m0 + rr, g.M - 1) * g.lda : weight_row<MODE, BN>(g, n0 + rr, n0)) +
              (size_t)k_first * BK + c * 8;
    ldst[i] = RPL * q * BK;
    wrow[i] = stream_w && RPL * q >= BM;   // wave-uniform: a load's rows are all A or all weights
  }
#define ISSUE_STAGE(KT)                                                                              \
  {                                                                                                  \
    uint16_t* _st = lds + ((KT) & 1) * SE;                                                           \
    _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                                 \
      if (wrow[i])                                                                                   \
        __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)(KT) * BK),                 \
                                         (lds_ptr_t)(_st + ldst[i]), 16, 0, kWeightLoadPolicy);      \
      else                                                                                           \
        __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)(KT) * BK),                 \
                                         (lds_ptr_t)(_st + ldst[i]), 16, 0, 0);                      \
    }                                                                                                \
  }
  // 32 codes per lane: 16-byte chunks qd and 4 + qd of the row (read as
  // bf16x8, the type the bf16 path reads)
#define FRAG8(DST, BASE, R)                                                                      \
  {                                                                                              \
    const int _r = (R);                                                                          \
    const bf16x8 _lo = *reinterpret_cast<const bf16x8*>((BASE) + _r * BK + swz<CPR>(_r, (lane >> 4)) * 8); \
    const bf16x8 _hi = *reinterpret_cast<const bf16x8*>((BASE) + _r * BK + swz<CPR>(_r, 4 + (lane >> 4)) * 8); \
    DST = cat_i32x8(__builtin_bit_cast(uint4, _lo), __builtin_bit_cast(uint4, _hi));             \
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  i32x8 fa[FM], fb[2];
  const int arow = wm * WROWS + (lane & 15), brow = wn * WCOLS + (lane & 15);

  ISSUE_STAGE(0);
  for (int kt = 0; kt < nk; ++kt) {
    WAIT_VMCNT(0);   // stage kt (the only one in flight) has landed
    WAIT_LGKM0();    // this wave's reads of stage kt - 1 are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 1 < nk) ISSUE_STAGE(kt + 1);
    const uint16_t* as = lds + (kt & 1) * SE;
    const uint16_t* bs = as + BM * BK;
#pragma unroll
    for (int i = 0; i < FM; ++i) FRAG8(fa[i], as, arow + i * 16);
    FRAG8(fb[0], bs, brow);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (j + 1 < FN) FRAG8(fb[(j + 1) & 1], bs, brow + (j + 1) * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][j] = mfma16x16x128_f8(fa[i], fb[j & 1], acc[i][j]);
    }
  }
#undef FRAG8
#undef ISSUE_STAGE
  WAIT_VMCNT(0);
  __syncthreads();
  if (MODE == kGemmSwiglu)
    swiglu_epilogue_regs<TL, true>(g, acc, smem, m0, n0, true, wm, wn, lane, tid);
  else
    gemm_epilogue<MODE, TL>(g, acc, smem, m0, n0, wm, wn, lane, tid);
}

// Wave-specialised pipeline.  Consumer waves 0-3 (one per SIMD) run every
// MFMA of the tile, each a 64-row block across all BN columns; producer waves
// 4-7 (the other wave of each SIMD) issue every direct-to-LDS load, into a
// ring of NST stages.  A wave whose vector-memory queue is full stalls at its
// next load; with the loads kept out of the MFMA waves' instruction streams,
// that stall no longer holds up MFMA issue.  The consumers follow the
// sub-step schedule (fragments of the next 32-deep sub-step read during the
// MFMAs of the current one); the one barrier per stage, between its two
// sub-steps, tells the producers that the buffer read last is free and the
// consumers that the next stage has landed.
template <int BM_, int BN_, int NST_>
struct SpecTile {
  static constexpr int BM = BM_, BN = BN_, BK = 64, NST = NST_;
  static constexpr int WM = 4, WN = 1;                          // consumer blocks
  static constexpr int CONSUMERS = 4, PRODUCERS = 4, WAVES = 8, THREADS = 512;
  static constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
  static constexpr int KS = BK / 32, CPR = BK / 8, RPL = 64 / CPR;
  static constexpr int STAGE_ELEMS = (BM + BN) * BK;
  static constexpr int TOTAL_LOADS = (BM + BN) / RPL;
  static constexpr int LOADS = TOTAL_LOADS / PRODUCERS;          // per producer wave and stage
  static constexpr int MAIN_LDS = NST * STAGE_ELEMS * 2;
  static constexpr int CS_LD = BN + 4;
  static constexpr int EPI_ROWS = BM * CS_LD * 4 <= 160 * 1024 - 4096 ? BM : BM / 2;
  static constexpr int EPI_LDS = EPI_ROWS * CS_LD * 4;
  static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
  static_assert(TOTAL_LOADS % PRODUCERS == 0, "stage loads must split evenly over the producers");
  static_assert((BM / RPL) % PRODUCERS == 0, "A rows fill whole load indices of every producer");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};
using TileS256 = SpecTile<256, 128, 3>;

template <int MODE, class TL>
__global__ __launch_bounds__(TL::THREADS) void gemm_spec_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BK = TL::BK, NST = TL::NST, SE = TL::STAGE_ELEMS;
  constexpr int NL = TL::LOADS, FM = TL::FM, FN = TL::FN, CPR = TL::CPR, RPL = TL::RPL;
  constexpr int WROWS = BM / TL::WM;
  static_assert(TL::KS == 2 && FN >= FM + 2 && NST >= 2 && NST <= 4, "sub-step pipeline layout");
  static_assert(3 * NL <= 63, "vmcnt counts at most 63 loads");
  __shared__ __align__(16) unsigned char smem[TL::LDS];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = (g.M + BM - 1) / BM;
  const BlockTile btile = block_tile(tiles_m);
  const int tm = btile.tm, tn = btile.tn;
  const int m0 = tm * BM, n0 = tn * TL::BN;
  const int nk = (g.K / BK) / gridDim.z;
  const int k_first = btile.z * nk;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int wm = wave;   // consumer block row; producers stage nothing in the epilogue

  if (wave >= TL::CONSUMERS) {
    wm = 1 << 20;
    // producer p issues loads q = p + PRODUCERS * i of every stage: rows
    // [RPL q, RPL q + RPL) of the stage image (A rows, then weight rows), lane
    // l at row RPL q + l / CPR, swizzled chunk (l % CPR) ^ f(row)
    const int p = wave - TL::CONSUMERS;
    const bool stream_w = tiles_m <= kStreamWeightsMaxRowTiles;
    const uint16_t* gsrc[NL];
    int ldst[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = p + TL::PRODUCERS * i;
      const int r = RPL * q + lane / CPR;
      const int rr = r < BM ? r : r - BM;
      const int c = swz<CPR>(rr, lane % CPR);
      gsrc[i] = (r < BM ? g.a + (size_t)min(m0 + rr, g.M - 1) * g.lda : weight_row<MODE, TL::BN>(g, n0 + rr, n0)) +
                (size_t)k_first * BK + c * 8;
      ldst[i] = RPL * q * BK;
    }
    auto issue = [&](int kt) {
      uint16_t* st = lds + (kt % NST) * SE;
#pragma unroll
      for (int i = 0; i < NL; ++i) {   // loads i < (BM / RPL) / PRODUCERS are A rows
        if (i < (BM / RPL) / TL::PRODUCERS || !stream_w)
          __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)kt * BK), (lds_ptr_t)(st + ldst[i]), 16, 0,
                                           0);
        else
          __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)kt * BK), (lds_ptr_t)(st + ldst[i]), 16, 0,
                                           kWeightLoadPolicy);
      }
    };
#pragma unroll
    for (int s = 0; s < NST; ++s)
      if (s < nk) issue(s);
    // wait until at most N stages of this wave's loads are in flight
    auto wait_stages = [&](int n) {
      if (n >= 3) WAIT_VMCNT(3 * NL);
      else if (n == 2) WAIT_VMCNT(2 * NL);
      else if (n == 1) WAIT_VMCNT(NL);
      else WAIT_VMCNT(0);
    };
    // stage 0 landed: the loads of the stages after it may still be in flight
    wait_stages(min(NST, nk) - 1);
    __builtin_amdgcn_s_barrier();
    for (int st = 0; st + 1 < nk; ++st) {
      // stage st + 1 landed (stages issued so far: up to st + NST - 1)
      wait_stages(min(st + NST, nk) - (st + 2));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // every consumer has read stage st: refill its buffer
      if (st + NST < nk) issue(st + NST);
    }
    WAIT_VMCNT(0);
  } else {
    bf16x8 fa[2][FM], fb[FN - 2], fbl[2][2];
    const int arow = wave * WROWS + (lane & 15), brow = lane & 15;
#define RD(BASE, R, KK) \
  (*reinterpret_cast<const bf16x8*>((BASE) + (R) * BK + swz<CPR>((R), (KK) * 4 + (lane >> 4)) * 8))
    // compute the sub-step held in fa[CUR], fb, fbl[CUR]; with NEXT, read the
    // fragments of sub-step KK1 of the stage in buffer B1 in between.
#define SUBSTEP(CUR, NXT, B1, KK1, NEXT)                                                          \
  {                                                                                               \
    const uint16_t* _as = lds + (B1) * SE;                                                        \
    const uint16_t* _bs = _as + BM * BK;                                                          \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                              \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                              \
        acc[i][j] = mfma16x16x32(fa[CUR][i], j < FN - 2 ? fb[j < FN - 2 ? j : 0] : fbl[CUR][j - (FN - 2) >= 0 ? j - (FN - 2) : 0], acc[i][j]); \
      if (NEXT) {                                                                                 \
        if (j == 0) {                                                                             \
          fbl[NXT][0] = RD(_bs, brow + (FN - 2) * 16, KK1);                                      \
          fbl[NXT][1] = RD(_bs, brow + (FN - 1) * 16, KK1);                                      \
        }                                                                                         \
        if (j < FN - 2) fb[j < FN - 2 ? j : 0] = RD(_bs, brow + j * 16, KK1);                     \
        if (j >= 1 && j <= FM) fa[NXT][j >= 1 && j <= FM ? j - 1 : 0] = RD(_as, arow + (j - 1) * 16, KK1); \
      }                                                                                           \
    }                                                                                             \
    if (NEXT) {                                                                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                                          \
      _Pragma("unroll") for (int _j = 1; _j <= FM; ++_j) {                                        \
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                       \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                        \
      }                                                                                           \
      _Pragma("unroll") for (int _j = FM + 1; _j < FN - 2; ++_j) {                                \
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);                                       \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                        \
      }                                                                                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * FM, 0);                                     \
    }                                                                                             \
  }
    __builtin_amdgcn_s_barrier();   // stage 0 has landed
    asm volatile("" ::: "memory");
    {
      const uint16_t* _as = lds;
      const uint16_t* _bs = _as + BM * BK;
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[0][i] = RD(_as, arow + i * 16, 0);
#pragma unroll
      for (int j = 0; j < FN - 2; ++j) fb[j] = RD(_bs, brow + j * 16, 0);
      fbl[0][0] = RD(_bs, brow + (FN - 2) * 16, 0);
      fbl[0][1] = RD(_bs, brow + (FN - 1) * 16, 0);
    }
    int b0 = 0;   // buffer of stage st
    for (int st = 0; st + 1 < nk; ++st) {
      const int b1 = b0 + 1 == NST ? 0 : b0 + 1;
      SUBSTEP(0, 1, b0, 1, true);
      WAIT_LGKM0();   // this wave's reads of stage st are done
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      SUBSTEP(1, 0, b1, 0, true);
      b0 = b1;
    }
    SUBSTEP(0, 1, b0, 1, true);
    SUBSTEP(1, 0, 0, 0, false);
#undef SUBSTEP
#undef RD
  }
  __syncthreads();
  gemm_epilogue_bf16<MODE, TL>(g, acc, smem, m0, n0, wave < TL::CONSUMERS, wm, 0, lane, tid);
}

// Wide wave-specialised pipeline (256 x 224): 12 waves, three per SIMD.
// Consumer waves 0-7 (two per SIMD) each hold a 64 x 112 accumulator block
// (112 VGPRs) and run its MFMAs; producer waves 8-11 issue every
// direct-to-LDS load of a stage (15 each) into two 60 KB stages.  Three waves
// per SIMD leave 168 VGPRs a wave, so a consumer reads the A fragments of a
// 32-deep sub-step when it starts and each B fragment one column block ahead
// of its MFMAs, and the other consumer of its SIMD hides those reads.  One
// barrier per stage: after it every consumer is done with the stage before
// (its buffer takes the stage after next) and the next stage has landed.
template <int BM_, int BN_>
struct SpecWTile {
  static constexpr int BM = BM_, BN = BN_, BK = 64, NST = 2;
  static constexpr int WM = 4, WN = 2;                          // consumer blocks
  static constexpr int CONSUMERS = WM * WN, PRODUCERS = 4, WAVES = CONSUMERS + PRODUCERS, THREADS = 64 * WAVES;
  static constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
  static constexpr int KS = BK / 32, CPR = BK / 8, RPL = 64 / CPR;
  static constexpr int STAGE_ELEMS = (BM + BN) * BK;
  static constexpr int TOTAL_LOADS = (BM + BN) / RPL;
  static constexpr int LOADS = TOTAL_LOADS / PRODUCERS;
  static constexpr int MAIN_LDS = NST * STAGE_ELEMS * 2;
  static constexpr int CS_LD = BN + 4;
  static constexpr int EPI_ROWS = BM * CS_LD * 4 <= 160 * 1024 - 4096 ? BM : BM / 2;
  static constexpr int EPI_LDS = EPI_ROWS * CS_LD * 4;
  static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
  static_assert(TOTAL_LOADS % PRODUCERS == 0, "stage loads must split evenly over the producers");
  static_assert((BM / RPL) % PRODUCERS == 0, "A rows fill whole load indices of every producer");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(EPI_ROWS % (BM / WM) == 0, "epilogue passes must hold whole consumer blocks");
};
using TileSW224 = SpecWTile<256, 224>;


template <int MODE, class TL>
__global__ __launch_bounds__(TL::THREADS) __attribute__((amdgpu_waves_per_eu(3))) void gemm_specw_kernel(GemmArgs g) {
  constexpr int BM = TL::BM, BK = TL::BK, SE = TL::STAGE_ELEMS;
  constexpr int NL = TL::LOADS, FM = TL::FM, FN = TL::FN, CPR = TL::CPR, RPL = TL::RPL;
  constexpr int WROWS = BM / TL::WM, WCOLS = TL::BN / TL::WN;
  static_assert(TL::KS == 2 && TL::NST == 2, "two 64-deep stages of two sub-steps");
  static_assert(NL <= 31, "vmcnt counts at most 63 loads");
  __shared__ __align__(16) unsigned char smem[TL::LDS];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = (g.M + BM - 1) / BM;
  const BlockTile btile = block_tile(tiles_m);
  const int tm = btile.tm, tn = btile.tn;
  const int m0 = tm * BM, n0 = tn * TL::BN;
  const int nk = (g.K / BK) / gridDim.z;
  const int k_first = btile.z * nk;

  // accumulators: set in each branch, so they are not live through the
  // producers' loop
  f32x4 acc[FM][FN];
  // consumer block (wm, wn); producers stage nothing in the epilogue
  int wm = wave % TL::WM, wn = wave / TL::WM;

  if (wave >= TL::CONSUMERS) {
    wm = 1 << 20;
    wn = 0;
    const int p = wave - TL::CONSUMERS;
    const bool stream_w = tiles_m <= kStreamWeightsMaxRowTiles;
    const uint16_t* gsrc[NL];
    int ldst[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = p + TL::PRODUCERS * i;   // row group: A rows, then B rows
      const int r = RPL * q + lane / CPR;
      const int rr = r < BM ? r : r - BM;
      const int c = swz<CPR>(rr, lane % CPR);
      gsrc[i] = (r < BM ? g.a + (size_t)min(m0 + rr, g.M - 1) * g.lda : weight_row<MODE, TL::BN>(g, n0 + rr, n0)) +
                (size_t)k_first * BK + c * 8;
      ldst[i] = RPL * q * BK;
    }
    auto issue = [&](int kt) {
      uint16_t* st = lds + (kt & 1) * SE;
#pragma unroll
      for (int i = 0; i < NL; ++i) {   // loads i < (BM / RPL) / PRODUCERS are A rows
        if (i < (BM / RPL) / TL::PRODUCERS || !stream_w)
          __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)kt * BK), (lds_ptr_t)(st + ldst[i]), 16, 0,
                                           0);
        else
          __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)kt * BK), (lds_ptr_t)(st + ldst[i]), 16, 0,
                                           kWeightLoadPolicy);
      }
    };
    issue(0);
    if (nk > 1) issue(1);
    // stage 0 landed (stage 1 may still be in flight)
    if (nk > 1) WAIT_VMCNT(NL);
    else WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    for (int st = 0; st + 1 < nk; ++st) {
      WAIT_VMCNT(0);   // stage st + 1 (the only one in flight) has landed
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // every consumer is done with stage st: refill its buffer
      if (st + 2 < nk) issue(st + 2);
    }
    WAIT_VMCNT(0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa[FM], fb[2];
    const int arow = wm * WROWS + (lane & 15), brow = wn * WCOLS + (lane & 15);
#define RD(BASE, R, KK) \
  (*reinterpret_cast<const bf16x8*>((BASE) + (R) * BK + swz<CPR>((R), (KK) * 4 + (lane >> 4)) * 8))
    __builtin_amdgcn_s_barrier();   // stage 0 has landed
    asm volatile("" ::: "memory");
    for (int st = 0; st < nk; ++st) {
      const uint16_t* as = lds + (st & 1) * SE;
      const uint16_t* bs = as + BM * BK;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = RD(as, arow + i * 16, kk);
        fb[0] = RD(bs, brow, kk);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (j + 1 < FN) fb[(j + 1) & 1] = RD(bs, brow + (j + 1) * 16, kk);
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j] = mfma16x16x32(fa[i], fb[j & 1], acc[i][j]);
        }
      }
      if (st + 1 < nk) {
        WAIT_LGKM0();   // this wave's reads of stage st are done
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
#undef RD
  }
  __syncthreads();
  gemm_epilogue_bf16<MODE, TL, false>(g, acc, smem, m0, n0, wave < TL::CONSUMERS, wm, wn, lane, tid);
}

// y[m][:] = res[m][:] + sum_z part[z][m][:] (z in order); with norm_out, also
// norm_out[m][:] = bf16(y / sqrt(mean(y^2) + eps) * gain).  One workgroup of
// NT threads per row; the row stays in registers (N <= NT * 4 * MAXCH).  All
// slices of a chunk are loaded before any is added (up to kMaxSplits), so a
// thread waits on memory once per chunk, not once per slice; the sum keeps the
// slice order.
constexpr int kMaxSplits = 8;   // the planner splits K at most 8 ways

template <int NT, int MAXCH>
__global__ __launch_bounds__(NT) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                           const float* __restrict__ res, float* __restrict__ out,
                                                           int M, int N, const uint16_t* __restrict__ gain,
                                                           void* __restrict__ norm_out, float eps,
                                                           float norm_inv_scale) {
  constexpr int NW = NT / 64;
  __shared__ float red[NW];
  const int m = blockIdx.x;
  const int n4 = N >> 2;
  float4 v[MAXCH];
  float ss = 0.f;
  // the norm's gains are requested with the row, not after the row sum
  uint2 gg[MAXCH];
  if (norm_out) {
#pragma unroll
    for (int k = 0; k < MAXCH; ++k) {
      const int i = threadIdx.x + NT * k;
      if (i < n4) gg[k] = reinterpret_cast<const uint2*>(gain)[i];
    }
  }
#pragma unroll
  for (int k = 0; k < MAXCH; ++k) {
    const int i = threadIdx.x + NT * k;
    if (i < n4) {
      float4 p[kMaxSplits];
#pragma unroll
      for (int z = 0; z < kMaxSplits; ++z)
        if (z < splits) p[z] = reinterpret_cast<const float4*>(part + ((size_t)z * M + m) * N)[i];
      v[k] = reinterpret_cast<const float4*>(res + (size_t)m * N)[i];
#pragma unroll
      for (int z = 0; z < kMaxSplits; ++z) {
        if (z < splits) {
          v[k].x += p[z].x;
          v[k].y += p[z].y;
          v[k].z += p[z].z;
          v[k].w += p[z].w;
        }
      }
      reinterpret_cast<float4*>(out + (size_t)m * N)[i] = v[k];
      ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
  }
  if (!norm_out) return;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < NW; w += 2) total += red[w] + red[w + 1];
  const float rs = 1.0f / sqrtf(total / (float)N + eps);
#pragma unroll
  for (int k = 0; k < MAXCH; ++k) {
    const int i = threadIdx.x + NT * k;
    if (i < n4) {
      const float y0 = v[k].x * rs * bf2f((uint16_t)(gg[k].x & 0xffff)), y1 = v[k].y * rs * bf2f((uint16_t)(gg[k].x >> 16));
      const float y2 = v[k].z * rs * bf2f((uint16_t)(gg[k].y & 0xffff)), y3 = v[k].w * rs * bf2f((uint16_t)(gg[k].y >> 16));
      if (norm_inv_scale > 0.0f) {   // FP8 codes of the normed row / scale
        const float q = norm_inv_scale;
        reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(norm_out) + (size_t)m * N)[i] =
            pack4fp8(y0 * q, y1 * q, y2 * q, y3 * q);
      } else {
        reinterpret_cast<uint2*>(static_cast<uint16_t*>(norm_out) + (size_t)m * N)[i] =
            make_uint2(pack2bf(y0, y1), pack2bf(y2, y3));
      }
    }
  }
}

// QKV after split-K: sum the slices (in order) of 8 consecutive GEMM columns
// (4 rotated pairs), then the QKV epilogue.  One thread per (token, 8 columns).
__global__ __launch_bounds__(256) void qkv_reduce_kernel(GemmArgs g, int splits) {
  const int groups = g.N / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)g.M * groups) return;
  const int m = (int)(idx / groups), n = (int)(idx % groups) * 8;
  // the position -> rotation-table chain is requested first, so that it
  // overlaps the slices' loads instead of following them
  const QkvTokenData td = qkv_token_data(g, m, n);
  float4 u[kMaxSplits], v[kMaxSplits];   // every slice loaded before any is added
#pragma unroll
  for (int z = 0; z < kMaxSplits; ++z) {
    if (z < splits) {
      const float4* row = reinterpret_cast<const float4*>(g.part + ((size_t)z * g.M + m) * g.N + n);
      u[z] = row[0];
      v[z] = row[1];
    }
  }
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
#pragma unroll
  for (int z = 0; z < kMaxSplits; ++z) {
    if (z < splits) {
      a.x += u[z].x; a.y += u[z].y; a.z += u[z].z; a.w += u[z].w;
      b.x += v[z].x; b.y += v[z].y; b.z += v[z].z; b.w += v[z].w;
    }
  }
  const float x0[4] = {a.x, a.z, b.x, b.z}, x1[4] = {a.y, a.w, b.y, b.w};
  qkv_store4(g, m, n, x0, x1, td);
}

enum { kTile256 = 1, kTileW256 = 2, kTileW224 = 3, kTile128W8 = 4, kTile128N96 = 5, kTileS256 = 6, kTileSW224 = 7 };

// Estimated time of one GEMM under a tile choice, fitted (least squares, 37
// measured tile/split choices on the Mistral-7B- and Yi-34B-shaped
// projections, most within 5 %) to
//   rounds * 2 BM BN (K / splits + 545) / (per-CU peak * eff) * (0.776 + 0.224 f)
//   + split-K partials written and read once at 6.5 TB/s,
// where rounds = ceil(tiles / 256 CUs), f = tiles / (rounds * 256) is how full
// the rounds are (a part-filled machine runs each busy CU faster), and 545
// K columns stand for a tile's pipeline fill and epilogue.  The wide
// wave-specialised kernel gains nothing from a part-filled machine (its four
// producer waves set its load rate, not the memory system): it takes f = 1.
template <class TL>
static double plan_cost(int M, int N, int K, int splits, double eff, bool fill_gain) {
  const double tiles = (double)((M + TL::BM - 1) / TL::BM) * (N / TL::BN) * splits;
  const double rounds = std::ceil(tiles / kNumCU);
  const double fill = fill_gain ? tiles / (rounds * kNumCU) : 1.0;
  const double per_cu = 2.5e15 / kNumCU * eff;   // flop/s
  const double t_tile = 2.0 * TL::BM * TL::BN * ((double)K / splits + 545.0) / per_cu;
  const double t_part = splits > 1 ? 2.0 * splits * (double)M * N * 4 / 6.5e12 : 0.0;
  return rounds * t_tile * (0.776 + 0.224 * fill) + t_part;
}

template <class TL>
static void plan_try(GemmPlan& best, double& best_cost, int tile, int mode, int M, int N, int K, double eff,
                     bool fill_gain = true) {
  if (N % TL::BN || K % TL::BK) return;
  const int nk = K / TL::BK;
  for (int splits = 1; splits <= 8; splits *= 2) {
    if (splits > 1 && (mode == kGemmSwiglu || nk % splits || nk / splits < 2 * TL::NST)) break;
    const double c = plan_cost<TL>(M, N, K, splits, eff, fill_gain);
    if (c < best_cost) {
      best_cost = c;
      best.tile = tile;
      best.splits = splits;
    }
  }
}

// Efficiencies: fraction of the MFMA peak per busy CU with every CU busy (fit
// to measured times of the bf16 kernels on the Mistral- and Yi-shaped
// projections; 256x224 set so that it beats 256x256 where both apply, as
// measured in the layer).  FP8 (f8): K counts codes; the plan is made for
// K / 2 units (same bytes and the same MFMA cycles per stage as bf16), on the
// ring-pipeline tiles and the FP8 wide tiles; the FP8 ring kernel keeps the
// unskewed load issue, so its 256x128 tile keeps the earlier fit.  FP8
// 256x224 measured 66 us on the 512-token gate/up (0.46) and 236 us at 2048
// tokens (0.52); 256x256 93 us on the 2048-token QKV (0.35, where the
// 256x128 ring tile takes 86 us).  The wide wave-specialised 256x224 kernel
// (bf16 only) measured 100-102 us on the Mistral-shaped 512-token gate/up
// against 103-105 on the sub-step kernel, 193 vs 196 at 1024 tokens and 376
// vs 406 (256x128 specialised) at 2048, but 170 vs 158 us at 576 tokens (1.5
// rounds) and 7.45 vs 6.21 ms at 32768 (256x256 sub-step), where the
// activation rows no longer stay in L2: it is tried up to 2048 rows only.
GemmPlan gemm_plan(int mode, int M, int N, int K, bool f8) {
  GemmPlan p{kTile128W8, 1};
  double cost = 1e30;
  if (f8) K /= 2;
  plan_try<Tile128W8>(p, cost, kTile128W8, mode, M, N, K, 0.344);
  plan_try<Tile128N96>(p, cost, kTile128N96, mode, M, N, K, f8 ? 0.291 : 0.31);
  if (M < 256) return p;
  plan_try<Tile256>(p, cost, kTile256, mode, M, N, K, f8 ? 0.426 : 0.445);
  if (f8) {   // the FP8 wide-tile kernel (gemm_f8w_kernel), fit to its layer timings
    plan_try<TileW256>(p, cost, kTileW256, mode, M, N, K, 0.35);
    plan_try<TileW224>(p, cost, kTileW224, mode, M, N, K, 0.47);
    return p;
  }
  plan_try<TileS256>(p, cost, kTileS256, mode, M, N, K, 0.49);
  plan_try<TileW256>(p, cost, kTileW256, mode, M, N, K, 0.53);
  plan_try<TileW224>(p, cost, kTileW224, mode, M, N, K, 0.485);
  if (M <= 2048) plan_try<TileSW224>(p, cost, kTileSW224, mode, M, N, K, 0.55, false);
  return p;
}

template <class TL>
static void launch_sub(const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid((unsigned)(((g.M + TL::BM - 1) / TL::BM) * (g.N / TL::BN)), 1, splits);
  switch (g.mode) {
    case kGemmQkvRope: hipLaunchKernelGGL((gemm_sub_kernel<kGemmQkvRope, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    case kGemmResidual: hipLaunchKernelGGL((gemm_sub_kernel<kGemmResidual, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_sub_kernel<kGemmSwiglu, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
  }
}

template <class TL>
static void launch_spec(const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid((unsigned)(((g.M + TL::BM - 1) / TL::BM) * (g.N / TL::BN)), 1, splits);
  switch (g.mode) {
    case kGemmQkvRope: hipLaunchKernelGGL((gemm_spec_kernel<kGemmQkvRope, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    case kGemmResidual: hipLaunchKernelGGL((gemm_spec_kernel<kGemmResidual, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_spec_kernel<kGemmSwiglu, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
  }
}

template <class TL>
static void launch_specw(const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid((unsigned)(((g.M + TL::BM - 1) / TL::BM) * (g.N / TL::BN)), 1, splits);
  switch (g.mode) {
    case kGemmQkvRope: hipLaunchKernelGGL((gemm_specw_kernel<kGemmQkvRope, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    case kGemmResidual: hipLaunchKernelGGL((gemm_specw_kernel<kGemmResidual, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_specw_kernel<kGemmSwiglu, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
  }
}

template <class TL>
static void launch_f8w(const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid((unsigned)(((g.M + TL::BM - 1) / TL::BM) * (g.N / TL::BN)), 1, splits);
  switch (g.mode) {
    case kGemmQkvRope: hipLaunchKernelGGL((gemm_f8w_kernel<kGemmQkvRope, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    case kGemmResidual: hipLaunchKernelGGL((gemm_f8w_kernel<kGemmResidual, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_f8w_kernel<kGemmSwiglu, TL>), grid, dim3(TL::THREADS), 0, s, g); break;
  }
}

template <class TL, bool F8>
static void launch_tile(const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid((unsigned)(((g.M + TL::BM - 1) / TL::BM) * (g.N / TL::BN)), 1, splits);
  switch (g.mode) {
    case kGemmQkvRope: hipLaunchKernelGGL((gemm_kernel<kGemmQkvRope, TL, F8>), grid, dim3(TL::THREADS), 0, s, g); break;
    case kGemmResidual: hipLaunchKernelGGL((gemm_kernel<kGemmResidual, TL, F8>), grid, dim3(TL::THREADS), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_kernel<kGemmSwiglu, TL, F8>), grid, dim3(TL::THREADS), 0, s, g); break;
  }
}

hb_status launch_gemm(const GemmArgs& ga, stream_t s) {
  if (ga.M <= 0) return HB_OK;
  if (ga.N % 128 || ga.K % (ga.f8 ? 128 : 64)) return fail(HB_E_SHAPE, "gemm N/K not multiples of 128/64 (FP8: 128/128)");
  if (ga.mode < kGemmQkvRope || ga.mode > kGemmSwiglu) return fail(HB_E_SHAPE, "bad gemm mode");
  if (ga.f8 && (!ga.ws0 || (ga.mode != kGemmResidual && !ga.ws1) || (ga.mode == kGemmQkvRope && !ga.ws2)))
    return fail(HB_E_NULL, "FP8 gemm needs the weight row scales");
  const GemmPlan p = gemm_plan(ga.mode, ga.M, ga.N, ga.K, ga.f8 != 0);
  GemmArgs g = ga;
  if (g.f8) {   // count K and lda in 16-bit units (two codes)
    g.K /= 2;
    g.lda /= 2;
  }
  if (p.splits > 1 && !g.part) return fail(HB_E_NULL, "gemm split-K needs a partial buffer");
  if (g.f8) {
    if (p.tile == kTile256) launch_tile<Tile256, true>(g, p.splits, (hipStream_t)s);
    else if (p.tile == kTileW224) launch_f8w<TileW224>(g, p.splits, (hipStream_t)s);
    else if (p.tile == kTileW256) launch_f8w<TileW256>(g, p.splits, (hipStream_t)s);
    else if (p.tile == kTile128N96) launch_tile<Tile128N96, true>(g, p.splits, (hipStream_t)s);
    else launch_tile<Tile128W8, true>(g, p.splits, (hipStream_t)s);
  } else if (p.tile == kTileS256) launch_spec<TileS256>(g, p.splits, (hipStream_t)s);
  else if (p.tile == kTileW224) launch_sub<TileW224>(g, p.splits, (hipStream_t)s);
  else if (p.tile == kTileSW224) launch_specw<TileSW224>(g, p.splits, (hipStream_t)s);
  else if (p.tile == kTileW256) launch_sub<TileW256>(g, p.splits, (hipStream_t)s);
  else if (p.tile == kTile256) launch_tile<Tile256, false>(g, p.splits, (hipStream_t)s);
  else if (p.tile == kTile128W8) launch_tile<Tile128W8, false>(g, p.splits, (hipStream_t)s);
  else if (p.tile == kTile128N96) launch_tile<Tile128N96, false>(g, p.splits, (hipStream_t)s);
  else launch_tile<Tile128W8, false>(g, p.splits, (hipStream_t)s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("gemm launch: ") + hipGetErrorString(e));
  if (p.splits > 1 && g.mode == kGemmQkvRope) {
    const int64_t n = (int64_t)g.M * (g.N / 8);
    hipLaunchKernelGGL(qkv_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)s, g,
                       p.splits);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(HB_E_HIP, std::string("qkv reduce launch: ") + hipGetErrorString(e));
  }
  return HB_OK;
}

hb_status launch_splitk_reduce(const float* part, int splits, const float* res, float* out, int M, int N,
                               const uint16_t* gain, void* norm_out, float eps, stream_t s, float norm_inv_scale) {
  if (M <= 0) return HB_OK;
  if (N > 16384) return fail(HB_E_SHAPE, "split-K reduce: row above 16384");
  if (splits < 1 || splits > kMaxSplits) return fail(HB_E_SHAPE, "split-K reduce: 1..8 slices");
  // A row per workgroup; with fewer rows than the machine has CUs, 1024
  // threads a row (more loads in flight per row), else 256.
  if (M < kNumCU)
    hipLaunchKernelGGL((splitk_reduce_kernel<1024, 4>), dim3(M), dim3(1024), 0, (hipStream_t)s, part, splits, res, out,
                       M, N, gain, norm_out, eps, norm_inv_scale);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<256, 16>), dim3(M), dim3(256), 0, (hipStream_t)s, part, splits, res, out,
                       M, N, gain, norm_out, eps, norm_inv_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("split-K reduce launch: ") + hipGetErrorString(e));
  return HB_OK;
}

}  // namespace hb
