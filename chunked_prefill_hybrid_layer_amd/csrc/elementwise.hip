// RMSNorm and paged KV append for gfx950.
//
// RMSNorm: out = x / sqrt(mean(x^2) + eps) * gain, fp32 in, bf16 out; one
// 256-thread workgroup per token row, float4 loads, wave + LDS reduction.
//
// KV append ("Chunked Prefill", mechanism: each chunk writes its KV into the
// paged blocks so the next chunk continues from it; "Sarathi-Serve reading
// notes" §3.1): dim i of token t's K row goes to K[page][kvh][i / 32][slot][i % 32],
// its V row to V[page][kvh][:][slot], page = slot[t] / 16, slot = slot[t] % 16.

#include "device_common.h"

namespace hb {

// The row stays in registers between the sum of squares and the scaling:
// up to kNormMaxChunks float4 per thread (hidden <= 256 * 4 * kNormMaxChunks).
constexpr int kNormMaxChunks = 16;

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x,
                                                      const uint16_t* __restrict__ gain,
                                                      void* __restrict__ out, int hidden, float eps,
                                                      float out_inv_scale) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * hidden);
  const int n4 = hidden >> 2;
  const uint2* g2 = reinterpret_cast<const uint2*>(gain);
  float4 v[kNormMaxChunks];
  uint2 gg[kNormMaxChunks];   // gains requested with the row, not after its sum
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kNormMaxChunks; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < n4) {
      v[k] = xr[i];
      gg[k] = g2[i];
      ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(total / (float)hidden + eps);
  const bool f8 = out_inv_scale > 0.0f;   // FP8 codes of the normed row / scale
  uint2* orow = reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)row * hidden);
  uint32_t* crow = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + (size_t)row * hidden);
#pragma unroll
  for (int k = 0; k < kNormMaxChunks; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < n4) {
      const float y0 = v[k].x * r * bf2f((uint16_t)(gg[k].x & 0xffff)), y1 = v[k].y * r * bf2f((uint16_t)(gg[k].x >> 16));
      const float y2 = v[k].z * r * bf2f((uint16_t)(gg[k].y & 0xffff)), y3 = v[k].w * r * bf2f((uint16_t)(gg[k].y >> 16));
      if (f8) {
        crow[i] = pack4fp8(y0 * out_inv_scale, y1 * out_inv_scale, y2 * out_inv_scale, y3 * out_inv_scale);
      } else {
        orow[i] = make_uint2(pack2bf(y0, y1), pack2bf(y2, y3));
      }
    }
  }
}

hb_status launch_rmsnorm(const float* x, const uint16_t* gain, void* out, int rows, int hidden,
                         float eps, stream_t s, float out_inv_scale) {
  if (rows <= 0) return HB_OK;
  if (hidden > 256 * 4 * kNormMaxChunks) return fail(HB_E_SHAPE, "rmsnorm: hidden above 16384");
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, (hipStream_t)s, x, gain, out, hidden, eps,
                     out_inv_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("rmsnorm launch: ") + hipGetErrorString(e));
  return HB_OK;
}

// One wave per (append run, kv head): a run is up to 16 consecutive tokens
// of one sequence landing in one page at consecutive slots (built by
// hb_pack_metadata).  K is stored in 32-dim slices of the page ([d/32][16][32]),
// so each slice of the run's rows is a contiguous copy.  V is stored transposed in the page ([d][16 slots]), so
// the run's V rows are staged in LDS and written back row by row of d: a
// full page is one contiguous block (two lanes per d row), a partial page
// writes only its own slots.  F8: the cache holds FP8 e4m3 codes of x / scale
// (kinv, vinv are 1 / scale), one byte per element, same layout.
template <int D, bool F8>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, int64_t row_stride,
                                                        const hb_append_run* __restrict__ runs, int n_runs,
                                                        int nkv, void* __restrict__ kcv, void* __restrict__ vcv,
                                                        float kinv, float vinv) {
  constexpr int CPT = D / 8;  // 16-byte chunks per token row
  __shared__ __align__(16) uint16_t vs[4][16 * D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const bool active = item < (int64_t)n_runs * nkv;
  int n = 0, s0 = 0, tok0 = 0, h = 0;
  size_t pb = 0;   // elements (= bytes in F8) from the cache start to the (page, kv head) block
  if (active) {
    const hb_append_run run = runs[item / nkv];
    h = (int)(item % nkv);
    n = run.n_tok;
    tok0 = run.tok0;
    s0 = run.slot0 & 15;
    pb = ((size_t)(run.slot0 >> 4) * nkv + h) * (size_t)(16 * D);
  }
  for (int idx = lane; idx < n * CPT; idx += 64) {
    const int i = idx / CPT, c = idx % CPT;
    const size_t src = (size_t)(tok0 + i) * row_stride + (size_t)h * D + c * 8;
    // K page block [D/32][16][32]: dims 8c..8c+7 of slot s0+i
    const size_t kd = pb + (size_t)(c >> 2) * 512 + (size_t)(s0 + i) * 32 + (c & 3) * 8;
    const uint4 kr = *reinterpret_cast<const uint4*>(k + src);
    if (F8) {
      const uint32_t w[4] = {kr.x, kr.y, kr.z, kr.w};
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = bf2f((uint16_t)(w[j] & 0xffff)) * kinv;
        f[2 * j + 1] = bf2f((uint16_t)(w[j] >> 16)) * kinv;
      }
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(kcv) + kd) =
          make_uint2(pack4fp8(f[0], f[1], f[2], f[3]), pack4fp8(f[4], f[5], f[6], f[7]));
    } else {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(kcv) + kd) = kr;
    }
    *reinterpret_cast<uint4*>(&vs[wave][i * D + c * 8]) = *reinterpret_cast<const uint4*>(v + src);
  }
  __syncthreads();
  for (int idx = lane; idx < 2 * D; idx += 64) {
    const int dd = idx >> 1, hf = idx & 1;          // d row, first or second 8 slots
    const int lo = max(s0, 8 * hf), hi = min(s0 + n, 8 * hf + 8);
    if (lo >= hi) continue;
    const size_t vd = pb + (size_t)dd * 16 + 8 * hf;
    if (F8) {
      uint8_t* dst = static_cast<uint8_t*>(vcv) + vd;
      if (lo == 8 * hf && hi == 8 * hf + 8) {
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = bf2f(vs[wave][(8 * hf + j - s0) * D + dd]) * vinv;
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack4fp8(f[0], f[1], f[2], f[3]), pack4fp8(f[4], f[5], f[6], f[7]));
      } else {
        for (int sl = lo; sl < hi; ++sl) dst[sl - 8 * hf] = fp8_code(bf2f(vs[wave][(sl - s0) * D + dd]) * vinv);
      }
    } else {
      uint16_t* dst = static_cast<uint16_t*>(vcv) + vd;
      if (lo == 8 * hf && hi == 8 * hf + 8) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = (uint32_t)vs[wave][(8 * hf + 2 * j - s0) * D + dd] |
                 ((uint32_t)vs[wave][(8 * hf + 2 * j + 1 - s0) * D + dd] << 16);
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        for (int sl = lo; sl < hi; ++sl) dst[sl - 8 * hf] = vs[wave][(sl - s0) * D + dd];
      }
    }
  }
}

hb_status launch_kv_append(const hb_dims& d, const DevMeta& m, int n_tokens, const uint16_t* k,
                           const uint16_t* v, int64_t row_stride, void* kc, void* vc, stream_t s) {
  if (n_tokens <= 0 || m.n_append_runs <= 0) return HB_OK;
  const int64_t items = (int64_t)m.n_append_runs * d.n_kv_heads;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  const float kinv = d.kv_fp8 ? 1.0f / d.k_scale : 1.0f, vinv = d.kv_fp8 ? 1.0f / d.v_scale : 1.0f;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, (hipStream_t)s, k, v, row_stride, m.append_runs,
                       m.n_append_runs, d.n_kv_heads, kc, vc, kinv, vinv);
  };
  if (d.head_dim == 128) {
    if (d.kv_fp8) go(kv_append_kernel<128, true>); else go(kv_append_kernel<128, false>);
  } else {
    if (d.kv_fp8) go(kv_append_kernel<64, true>); else go(kv_append_kernel<64, false>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("kv_append launch: ") + hipGetErrorString(e));
  return HB_OK;
}

}  // namespace hb
