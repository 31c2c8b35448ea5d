// Packed-token projections for gfx950: C[M][N] = A[M][K] . W[N][K]^T with
// bf16 operands and fp32 accumulation on MFMA (v_mfma_f32_16x16x32_bf16).
//
// Every token of the hybrid batch -- chunk and decode alike -- goes through
// the same projections, which is what makes the linear-layer cost depend on
// the batch's token count n ("Sarathi-Serve reading notes" §1.6: T_math =
// 2 n d_in d_out / FLOPS, T_mem = (d_in d_out bytes_w + n d_in bytes_a) / BW;
// "Chunked Prefill", hybrid-iteration roofline 2(c+b)Psi).
//
// Tiling: WM x 2 waves, each owning a 64x64 output block, so a workgroup tile
// is (64 WM) x 128 with K steps of 64.  WM = 4 (256x128, 512 threads, two
// waves per SIMD) serves batches of 256+ tokens, WM = 2 (128x128) smaller
// ones.  Both operands are K-contiguous.  A ring of LDS stages (3 x 48 KB or
// 4 x 32 KB) is filled by direct-to-LDS loads (global_load_lds_dwordx4, no VGPR
// staging) issued two or three K steps ahead to cover L2/HBM latency.  Each
// 1 KB wave load lands contiguously in LDS; the global address of every lane
// is chosen so that the LDS image is XOR-swizzled on 16-byte chunks and the
// MFMA fragment reads are bank-conflict free.  Workgroups are renumbered so
// that each XCD (own L2) walks a contiguous run of tiles, M fastest: the M
// tiles sharing a weight tile run on one XCD.
//
// Split-K (grid.z > 1, when the tiles alone do not cover the 256 CUs): each
// K slice writes an fp32 partial tile and a reduce kernel adds the slices in a
// fixed order (results do not depend on timing) before applying the epilogue.
//
// Epilogues (the accumulator tile is staged through LDS as fp32):
//   QKV:      RoPE (rotate-half, table-driven) on q and k; q -> bf16 buffer;
//             k and v -> the paged KV cache at the tokens' slots (KV append).
//   residual: out = res + acc (fp32).
//   SwiGLU:   the tile's 128 columns are 64 gate rows and the 64 up rows of
//             the same FFN units; out = silu(gate) * up (bf16).

#include "device_common.h"

namespace hb {

constexpr int BN = kGemmBN, BK = kGemmBK;
constexpr int CS_LD = BN + 4;  // fp32 staging row stride (floats)

template <int WM>
struct Cfg {
  static constexpr int BM = 64 * WM;
  static constexpr int THREADS = 128 * WM;
  static constexpr int WAVES = 2 * WM;
  static constexpr int NST = WM == 2 ? 4 : 3;                 // LDS pipeline stages
  static constexpr int STAGE_ELEMS = (BM + BN) * BK;          // bf16 per stage
  static constexpr int LOADS = (BM + BN) / 8 / WAVES;         // 1 KB DMA loads per wave and stage
  static constexpr int MAIN_LDS = NST * STAGE_ELEMS * 2;
  static constexpr int EPI_LDS = BM * CS_LD * 4;
  static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
};

// 16-byte chunk c of LDS row r (128 B) is stored at chunk c ^ (r & 7).  For the
// fragment reads (16 consecutive rows, one chunk column per 16 lanes) this is
// free of bank conflicts on gfx950, as measured with SQ_LDS_BANK_CONFLICT; the
// (r ^ (r >> 3)) variant spent 60 % of its LDS cycles in conflicts.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

template <int MODE>
__device__ __forceinline__ const uint16_t* weight_row(const GemmArgs& g, int n, int n0) {
  if (MODE == kGemmQkvRope) {
    if (n < g.n0) return g.w0 + (size_t)n * g.K;
    if (n < g.n0 + g.n1) return g.w1 + (size_t)(n - g.n0) * g.K;
    return g.w2 + (size_t)(n - g.n0 - g.n1) * g.K;
  } else if (MODE == kGemmSwiglu) {
    const int f0 = n0 / 2, c = n - n0;
    return (c < BN / 2) ? g.w0 + (size_t)(f0 + c) * g.K : g.w1 + (size_t)(f0 + c - BN / 2) * g.K;
  } else {
    return g.w0 + (size_t)n * g.K;
  }
}

// QKV output of token m, columns c and c + d/2 of one head (c within the first
// half): q and k are rotated by the token's position, q goes to the q buffer,
// k and v to the paged cache at the token's slot.
__device__ __forceinline__ void qkv_store_pair(const GemmArgs& g, int m, int c, float x0, float x1) {
  const int d = g.head_dim, half = d >> 1;
  const int qdim = g.n_q_heads * d, kdim = g.n_kv_heads * d;
  const int i = c % d;
  if (c < qdim + kdim) {
    const int pos = g.tok_pos[m];
    const float2 cs = *reinterpret_cast<const float2*>(g.rope + ((size_t)pos * half + i) * 2);
    const uint16_t y0 = f2bf(x0 * cs.x - x1 * cs.y);
    const uint16_t y1 = f2bf(x1 * cs.x + x0 * cs.y);
    if (c < qdim) {
      uint16_t* qo = g.out_b + (size_t)m * qdim + c;
      qo[0] = y0;
      qo[half] = y1;
    } else {
      const int kvh = (c - qdim) / d;
      const int sl = g.slot[m];
      uint16_t* kp = g.k_cache + (((size_t)(sl >> 4) * g.n_kv_heads + kvh) * 16 + (sl & 15)) * d + i;
      kp[0] = y0;
      kp[half] = y1;
    }
  } else {
    const int kvh = (c - qdim - kdim) / d;
    const int sl = g.slot[m];
    uint16_t* vp = g.v_cache + (((size_t)(sl >> 4) * g.n_kv_heads + kvh) * d + i) * 16 + (sl & 15);
    vp[0] = f2bf(x0);
    vp[half * 16] = f2bf(x1);
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

template <int MODE, int WM>
__global__ __launch_bounds__(Cfg<WM>::THREADS) void gemm_kernel(GemmArgs g) {
  using C = Cfg<WM>;
  constexpr int BM = C::BM, NST = C::NST, SE = C::STAGE_ELEMS, NL = C::LOADS, NT = C::THREADS;
  __shared__ __align__(16) unsigned char smem[C::LDS];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (g.M + BM - 1) / BM;
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  // K slice of this workgroup (split-K along grid.z)
  const int nk = (g.K / BK) / gridDim.z;
  const int k_first = blockIdx.z * nk;

  // DMA mapping: load q = wave + WAVES * i covers rows [8q, 8q + 8) of the
  // stage image (A rows first, then B rows); lane l lands at row 8q + l/8,
  // chunk l%8, i.e. it loads logical chunk (l%8) ^ f(row).
  const uint16_t* gsrc[NL];
  int ldst[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = wave + C::WAVES * i;
    const int r = 8 * q + (lane >> 3);                       // row of the stage image
    const int rr = r < BM ? r : r - BM;                       // row within A or B
    const int c = swz(rr, lane & 7);
    gsrc[i] = (r < BM ? g.a + (size_t)min(m0 + rr, g.M - 1) * g.lda : weight_row<MODE>(g, n0 + rr, n0)) +
              (size_t)k_first * BK + c * 8;
    ldst[i] = 8 * q * BK;
  }
#define ISSUE_STAGE(KT)                                                                              \
  {                                                                                                  \
    uint16_t* _st = lds + ((KT) % NST) * SE;                                                         \
    _Pragma("unroll") for (int i = 0; i < NL; ++i)                                                   \
        __builtin_amdgcn_global_load_lds((const void*)(gsrc[i] + (size_t)(KT) * BK),                 \
                                         (lds_ptr_t)(_st + ldst[i]), 16, 0, 0);                      \
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) ISSUE_STAGE(s);

  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most the loads of the stages issued after it
    // (NL per stage and wave) are outstanding
    const int later = min(NST - 2, nk - 1 - kt);
    if (later >= 2) WAIT_VMCNT(2 * NL);
    else if (later == 1) WAIT_VMCNT(NL);
    else WAIT_VMCNT(0);
    // every wave's part of stage kt is in LDS and stage kt-1 is no longer read.
    // A plain s_barrier: __syncthreads() would add a fence that waits for all
    // in-flight stages; the empty asm keeps LDS accesses on their side.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + NST - 1 < nk) ISSUE_STAGE(kt + NST - 1);
    const uint16_t* as = lds + (kt % NST) * SE;
    const uint16_t* bs = as + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const bf16x8*>(as + r * BK + swz(r, c) * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + r * BK + swz(r, c) * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
    }
  }
#undef ISSUE_STAGE
  WAIT_VMCNT(0);
  __syncthreads();

  // stage the fp32 tile in LDS: acc[i][j][e] is C[wm*64+i*16+4*(lane>>4)+e][wn*64+j*16+(lane&15)]
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Cs[(wm * 64 + i * 16 + 4 * (lane >> 4) + e) * CS_LD + wn * 64 + j * 16 + (lane & 15)] = acc[i][j][e];
  __syncthreads();

  if (gridDim.z > 1) {  // split-K: raw fp32 partial into slice blockIdx.z
    float* out = g.part + (size_t)blockIdx.z * g.M * g.N;
    for (int idx = tid; idx < BM * BN / 4; idx += NT) {
      const int r = idx / (BN / 4), c4 = idx % (BN / 4);
      const int m = m0 + r;
      if (m >= g.M) continue;
      *reinterpret_cast<float4*>(out + (size_t)m * g.N + n0 + c4 * 4) =
          *reinterpret_cast<const float4*>(Cs + r * CS_LD + c4 * 4);
    }
  } else if (MODE == kGemmResidual) {
    for (int idx = tid; idx < BM * BN / 4; idx += NT) {
      const int r = idx / (BN / 4), c4 = idx % (BN / 4);
      const int m = m0 + r;
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
    for (int idx = tid; idx < BM * (BN / 8); idx += NT) {
      const int r = idx / (BN / 8), c4 = idx % (BN / 8);
      const int m = m0 + r;
      if (m >= g.M) continue;
      const float* gr = Cs + r * CS_LD + c4 * 4;
      const float* ur = gr + BN / 2;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = gr[e];
        o[e] = z / (1.0f + __expf(-z)) * ur[e];
      }
      uint2 pk;
      pk.x = pack2bf(o[0], o[1]);
      pk.y = pack2bf(o[2], o[3]);
      *reinterpret_cast<uint2*>(g.out_b + (size_t)m * g.ldo + f0 + c4 * 4) = pk;
    }
  } else {  // QKV + RoPE + KV append: one thread per (token, rotated pair)
    const int half = g.head_dim >> 1;
    for (int idx = tid; idx < BM * (BN / 2); idx += NT) {
      const int r = idx / (BN / 2), pp = idx % (BN / 2);
      const int m = m0 + r;
      if (m >= g.M) continue;
      const int c = (pp / half) * g.head_dim + pp % half;  // column within the tile
      qkv_store_pair(g, m, n0 + c, Cs[r * CS_LD + c], Cs[r * CS_LD + c + half]);
    }
  }
}

// y[m][:] = res[m][:] + sum_z part[z][m][:] (z in order); with norm_out, also
// norm_out[m][:] = bf16(y / sqrt(mean(y^2) + eps) * gain).  One workgroup per row.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            const float* __restrict__ res, float* __restrict__ out,
                                                            int M, int N, const uint16_t* __restrict__ gain,
                                                            uint16_t* __restrict__ norm_out, float eps) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int n4 = N >> 2;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += 256) {
    float4 v = reinterpret_cast<const float4*>(res + (size_t)m * N)[i];
    for (int z = 0; z < splits; ++z) {
      const float4 p = reinterpret_cast<const float4*>(part + ((size_t)z * M + m) * N)[i];
      v.x += p.x;
      v.y += p.y;
      v.z += p.z;
      v.w += p.w;
    }
    reinterpret_cast<float4*>(out + (size_t)m * N)[i] = v;
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  if (!norm_out) return;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = 1.0f / sqrtf(total / (float)N + eps);
  for (int i = threadIdx.x; i < n4; i += 256) {
    const float4 v = reinterpret_cast<const float4*>(out + (size_t)m * N)[i];
    const uint2 gg = reinterpret_cast<const uint2*>(gain)[i];
    uint2 o;
    o.x = pack2bf(v.x * rs * bf2f((uint16_t)(gg.x & 0xffff)), v.y * rs * bf2f((uint16_t)(gg.x >> 16)));
    o.y = pack2bf(v.z * rs * bf2f((uint16_t)(gg.y & 0xffff)), v.w * rs * bf2f((uint16_t)(gg.y >> 16)));
    reinterpret_cast<uint2*>(norm_out + (size_t)m * N)[i] = o;
  }
}

// QKV after split-K: sum the slices of each rotated column pair, then the QKV
// epilogue.  One thread per (token, pair).
__global__ __launch_bounds__(256) void qkv_reduce_kernel(GemmArgs g, int splits) {
  const int half = g.head_dim >> 1, pairs = g.N / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)g.M * pairs) return;
  const int m = (int)(idx / pairs), p = (int)(idx % pairs);
  const int c = (p / half) * g.head_dim + p % half;
  float x0 = 0.f, x1 = 0.f;
  for (int z = 0; z < splits; ++z) {
    const float* row = g.part + ((size_t)z * g.M + m) * g.N;
    x0 += row[c];
    x1 += row[c + half];
  }
  qkv_store_pair(g, m, c, x0, x1);
}

GemmPlan gemm_plan(int mode, int M, int N, int K) {
  GemmPlan p;
  p.wm = M >= 256 ? 4 : 2;
  const int bm = 64 * p.wm, nst = p.wm == 2 ? 4 : 3;
  const int tiles = ((M + bm - 1) / bm) * (N / BN);
  const int nk = K / BK;
  p.splits = 1;
  if (mode != kGemmSwiglu)
    while (p.splits < 8 && tiles * p.splits < kNumCU && nk % (2 * p.splits) == 0 && nk / (2 * p.splits) >= nst)
      p.splits *= 2;
  return p;
}

template <int WM>
static void launch_wm(const GemmArgs& g, dim3 grid, hipStream_t s) {
  constexpr int T = Cfg<WM>::THREADS;
  switch (g.mode) {
    case kGemmQkvRope: hipLaunchKernelGGL((gemm_kernel<kGemmQkvRope, WM>), grid, dim3(T), 0, s, g); break;
    case kGemmResidual: hipLaunchKernelGGL((gemm_kernel<kGemmResidual, WM>), grid, dim3(T), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_kernel<kGemmSwiglu, WM>), grid, dim3(T), 0, s, g); break;
  }
}

hb_status launch_gemm(const GemmArgs& g, stream_t s) {
  if (g.M <= 0) return HB_OK;
  if (g.N % BN || g.K % BK) return fail(HB_E_SHAPE, "gemm N/K not multiples of the tile");
  if (g.mode < kGemmQkvRope || g.mode > kGemmSwiglu) return fail(HB_E_SHAPE, "bad gemm mode");
  const GemmPlan p = gemm_plan(g.mode, g.M, g.N, g.K);
  if (p.splits > 1 && !g.part) return fail(HB_E_NULL, "gemm split-K needs a partial buffer");
  const int bm = 64 * p.wm;
  const dim3 grid((unsigned)(((g.M + bm - 1) / bm) * (g.N / BN)), 1, p.splits);
  if (p.wm == 4) launch_wm<4>(g, grid, (hipStream_t)s);
  else launch_wm<2>(g, grid, (hipStream_t)s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("gemm launch: ") + hipGetErrorString(e));
  if (p.splits > 1 && g.mode == kGemmQkvRope) {
    const int64_t n = (int64_t)g.M * (g.N / 2);
    hipLaunchKernelGGL(qkv_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)s, g,
                       p.splits);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(HB_E_HIP, std::string("qkv reduce launch: ") + hipGetErrorString(e));
  }
  return HB_OK;
}

hb_status launch_splitk_reduce(const float* part, int splits, const float* res, float* out, int M, int N,
                               const uint16_t* gain, uint16_t* norm_out, float eps, stream_t s) {
  if (M <= 0) return HB_OK;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(M), dim3(256), 0, (hipStream_t)s, part, splits, res, out, M, N, gain,
                     norm_out, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("split-K reduce launch: ") + hipGetErrorString(e));
  return HB_OK;
}

}  // namespace hb
