// Packed-token projections for gfx950: C[M][N] = A[M][K] . W[N][K]^T with
// bf16 operands and fp32 accumulation on MFMA (v_mfma_f32_16x16x32_bf16).
//
// Every token of the hybrid batch -- chunk and decode alike -- goes through
// the same projections, which is what makes the linear-layer cost depend on
// the batch's token count n ("Sarathi-Serve reading notes" §1.6: T_math =
// 2 n d_in d_out / FLOPS, T_mem = (d_in d_out bytes_w + n d_in bytes_a) / BW;
// "Chunked Prefill", hybrid-iteration roofline 2(c+b)Psi).
//
// Tiling: 256 threads (4 waves, 2x2), 128x128 output tile, K step 64.  Both
// operands are K-contiguous, staged through double-buffered LDS with an XOR
// swizzle on 16-byte chunks so the MFMA fragment reads are bank-conflict free.
// One barrier per K step: the next step's global loads are issued before the
// MFMAs of the current step and written to the other LDS buffer after them.
// Workgroups are renumbered so that each XCD (own L2) walks a contiguous run
// of tiles, M fastest: the M tiles sharing a weight tile run on one XCD.
//
// Epilogues (the accumulator tile is staged through LDS as fp32):
//   QKV:      RoPE (rotate-half, table-driven) on q and k; q -> bf16 buffer;
//             k and v -> the paged KV cache at the tokens' slots (KV append).
//   residual: out = res + acc (fp32).
//   SwiGLU:   the tile's 128 columns are 64 gate rows and the 64 up rows of
//             the same FFN units; out = silu(gate) * up (bf16).

#include "device_common.h"

namespace hb {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int CS_LD = BN + 4;  // fp32 staging row stride (floats)
constexpr int kMainLds = 2 * (BM + BN) * BK * 2;
constexpr int kEpiLds = BM * CS_LD * 4;
constexpr int kGemmLds = kMainLds > kEpiLds ? kMainLds : kEpiLds;

// 16-byte chunk c of LDS row r is stored at chunk swz(r, c): within any 8 or 16
// consecutive rows the same logical chunk lands in distinct bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

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

template <int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ __align__(16) unsigned char smem[kGemmLds];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * BM * BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (g.M + BM - 1) / BM;
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  // global -> LDS mapping: 4 passes of 32 rows x 8 chunks of 16 bytes
  const int lr = tid >> 3, lc = tid & 7;
  const uint16_t* ga0 = g.a + (size_t)min(m0 + lr, g.M - 1) * g.lda + lc * 8;
  const uint16_t* ga1 = g.a + (size_t)min(m0 + lr + 32, g.M - 1) * g.lda + lc * 8;
  const uint16_t* ga2 = g.a + (size_t)min(m0 + lr + 64, g.M - 1) * g.lda + lc * 8;
  const uint16_t* ga3 = g.a + (size_t)min(m0 + lr + 96, g.M - 1) * g.lda + lc * 8;
  const uint16_t* gb0 = weight_row<MODE>(g, n0 + lr, n0) + lc * 8;
  const uint16_t* gb1 = weight_row<MODE>(g, n0 + lr + 32, n0) + lc * 8;
  const uint16_t* gb2 = weight_row<MODE>(g, n0 + lr + 64, n0) + lc * 8;
  const uint16_t* gb3 = weight_row<MODE>(g, n0 + lr + 96, n0) + lc * 8;
  // LDS element offsets of this thread's 4 chunks (rows lr + 32p, chunk lc)
  const int so0 = (lr) * BK + swz(lr, lc) * 8;
  const int so1 = (lr + 32) * BK + swz(lr + 32, lc) * 8;
  const int so2 = (lr + 64) * BK + swz(lr + 64, lc) * 8;
  const int so3 = (lr + 96) * BK + swz(lr + 96, lc) * 8;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = g.K / BK;
  uint4 ra0 = *reinterpret_cast<const uint4*>(ga0), ra1 = *reinterpret_cast<const uint4*>(ga1);
  uint4 ra2 = *reinterpret_cast<const uint4*>(ga2), ra3 = *reinterpret_cast<const uint4*>(ga3);
  uint4 rb0 = *reinterpret_cast<const uint4*>(gb0), rb1 = *reinterpret_cast<const uint4*>(gb1);
  uint4 rb2 = *reinterpret_cast<const uint4*>(gb2), rb3 = *reinterpret_cast<const uint4*>(gb3);
  *reinterpret_cast<uint4*>(As + so0) = ra0;
  *reinterpret_cast<uint4*>(As + so1) = ra1;
  *reinterpret_cast<uint4*>(As + so2) = ra2;
  *reinterpret_cast<uint4*>(As + so3) = ra3;
  *reinterpret_cast<uint4*>(Bs + so0) = rb0;
  *reinterpret_cast<uint4*>(Bs + so1) = rb1;
  *reinterpret_cast<uint4*>(Bs + so2) = rb2;
  *reinterpret_cast<uint4*>(Bs + so3) = rb3;
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int ko = (kt + 1) * BK;
      ra0 = *reinterpret_cast<const uint4*>(ga0 + ko);
      ra1 = *reinterpret_cast<const uint4*>(ga1 + ko);
      ra2 = *reinterpret_cast<const uint4*>(ga2 + ko);
      ra3 = *reinterpret_cast<const uint4*>(ga3 + ko);
      rb0 = *reinterpret_cast<const uint4*>(gb0 + ko);
      rb1 = *reinterpret_cast<const uint4*>(gb1 + ko);
      rb2 = *reinterpret_cast<const uint4*>(gb2 + ko);
      rb3 = *reinterpret_cast<const uint4*>(gb3 + ko);
    }
    const uint16_t* as = As + cur * BM * BK;
    const uint16_t* bs = Bs + cur * BN * BK;
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
    if (more) {
      uint16_t* an = As + (cur ^ 1) * BM * BK;
      uint16_t* bn = Bs + (cur ^ 1) * BN * BK;
      *reinterpret_cast<uint4*>(an + so0) = ra0;
      *reinterpret_cast<uint4*>(an + so1) = ra1;
      *reinterpret_cast<uint4*>(an + so2) = ra2;
      *reinterpret_cast<uint4*>(an + so3) = ra3;
      *reinterpret_cast<uint4*>(bn + so0) = rb0;
      *reinterpret_cast<uint4*>(bn + so1) = rb1;
      *reinterpret_cast<uint4*>(bn + so2) = rb2;
      *reinterpret_cast<uint4*>(bn + so3) = rb3;
    }
    __syncthreads();
  }

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

  if (MODE == kGemmResidual) {
    for (int idx = tid; idx < BM * BN / 4; idx += 256) {
      const int r = idx / (BN / 4), c4 = idx % (BN / 4);
      const int m = m0 + r;
      if (m >= g.M) continue;
      const float4 a = *reinterpret_cast<const float4*>(Cs + r * CS_LD + c4 * 4);
      const float4 rr = *reinterpret_cast<const float4*>(g.res + (size_t)m * g.ldo + n0 + c4 * 4);
      float4 o;
      o.x = rr.x + a.x;
      o.y = rr.y + a.y;
      o.z = rr.z + a.z;
      o.w = rr.w + a.w;
      *reinterpret_cast<float4*>(g.out_f + (size_t)m * g.ldo + n0 + c4 * 4) = o;
    }
  } else if (MODE == kGemmSwiglu) {
    const int f0 = n0 / 2;
    for (int idx = tid; idx < BM * (BN / 8); idx += 256) {
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
  } else {  // QKV + RoPE + KV append
    const int d = g.head_dim, half = d >> 1;
    const int qdim = g.n_q_heads * d, kdim = g.n_kv_heads * d;
    const int nkv = g.n_kv_heads;
    if (n0 < qdim + kdim) {
      const bool is_q = n0 < qdim;
      for (int idx = tid; idx < BM * (BN / 2); idx += 256) {
        const int r = idx / (BN / 2), pp = idx % (BN / 2);
        const int m = m0 + r;
        if (m >= g.M) continue;
        const int hh = pp / half, i = pp % half;
        const int clo = hh * d + i, chi = clo + half;
        const int pos = g.tok_pos[m];
        const float2 cs = *reinterpret_cast<const float2*>(g.rope + ((size_t)pos * half + i) * 2);
        const float x0 = Cs[r * CS_LD + clo], x1 = Cs[r * CS_LD + chi];
        const uint16_t y0 = f2bf(x0 * cs.x - x1 * cs.y);
        const uint16_t y1 = f2bf(x1 * cs.x + x0 * cs.y);
        if (is_q) {
          uint16_t* qo = g.out_b + (size_t)m * qdim + n0;
          qo[clo] = y0;
          qo[chi] = y1;
        } else {
          const int kvh = (n0 - qdim) / d + hh;
          const int sl = g.slot[m];
          uint16_t* kp = g.k_cache + (((size_t)(sl >> 4) * nkv + kvh) * 16 + (sl & 15)) * d;
          kp[i] = y0;
          kp[i + half] = y1;
        }
      }
    } else {
      for (int idx = tid; idx < BM * BN; idx += 256) {
        const int c = idx / BM, r = idx % BM;  // consecutive threads: consecutive tokens
        const int m = m0 + r;
        if (m >= g.M) continue;
        const int hh = c / d, i = c % d;
        const int kvh = (n0 - qdim - kdim) / d + hh;
        const int sl = g.slot[m];
        g.v_cache[(((size_t)(sl >> 4) * nkv + kvh) * d + i) * 16 + (sl & 15)] = f2bf(Cs[r * CS_LD + c]);
      }
    }
  }
}

hb_status launch_gemm(const GemmArgs& g, stream_t s) {
  if (g.M <= 0) return HB_OK;
  if (g.N % BN || g.K % BK) return fail(HB_E_SHAPE, "gemm N/K not multiples of the tile");
  const unsigned tiles = (unsigned)(((g.M + BM - 1) / BM) * (g.N / BN));
  switch (g.mode) {
    case kGemmQkvRope:
      hipLaunchKernelGGL(gemm_kernel<kGemmQkvRope>, dim3(tiles), dim3(256), 0, (hipStream_t)s, g);
      break;
    case kGemmResidual:
      hipLaunchKernelGGL(gemm_kernel<kGemmResidual>, dim3(tiles), dim3(256), 0, (hipStream_t)s, g);
      break;
    case kGemmSwiglu:
      hipLaunchKernelGGL(gemm_kernel<kGemmSwiglu>, dim3(tiles), dim3(256), 0, (hipStream_t)s, g);
      break;
    default:
      return fail(HB_E_SHAPE, "bad gemm mode");
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("gemm launch: ") + hipGetErrorString(e));
  return HB_OK;
}

}  // namespace hb
