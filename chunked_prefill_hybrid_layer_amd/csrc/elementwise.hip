// RMSNorm and paged KV append for gfx950.
//
// RMSNorm: out = x / sqrt(mean(x^2) + eps) * gain, fp32 in, bf16 out; one
// 256-thread workgroup per token row, float4 loads, wave + LDS reduction.
//
// KV append ("Chunked Prefill", mechanism: each chunk writes its KV into the
// paged blocks so the next chunk continues from it; "Sarathi-Serve reading
// notes" §3.1): token t's K row goes to K[page][kvh][slot][:], its V row to
// V[page][kvh][:][slot], page = slot[t] / 16, slot = slot[t] % 16.

#include "device_common.h"

namespace hb {

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x,
                                                      const uint16_t* __restrict__ gain,
                                                      uint16_t* __restrict__ out, int hidden, float eps) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * hidden);
  const int n4 = hidden >> 2;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n4; i += 256) {
    float4 v = xr[i];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(total / (float)hidden + eps);
  uint2* orow = reinterpret_cast<uint2*>(out + (size_t)row * hidden);
  const uint2* g2 = reinterpret_cast<const uint2*>(gain);
  for (int i = threadIdx.x; i < n4; i += 256) {
    float4 v = xr[i];
    uint2 gg = g2[i];
    float g0 = bf2f((uint16_t)(gg.x & 0xffff)), g1 = bf2f((uint16_t)(gg.x >> 16));
    float g2f = bf2f((uint16_t)(gg.y & 0xffff)), g3 = bf2f((uint16_t)(gg.y >> 16));
    uint2 o;
    o.x = pack2bf(v.x * r * g0, v.y * r * g1);
    o.y = pack2bf(v.z * r * g2f, v.w * r * g3);
    orow[i] = o;
  }
}

hb_status launch_rmsnorm(const float* x, const uint16_t* gain, uint16_t* out, int rows, int hidden,
                         float eps, stream_t s) {
  if (rows <= 0) return HB_OK;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, (hipStream_t)s, x, gain, out, hidden, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("rmsnorm launch: ") + hipGetErrorString(e));
  return HB_OK;
}

// One thread per (token, kv head, 8-element chunk of d).
template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, int64_t row_stride,
                                                        const int32_t* __restrict__ slot, int n_tokens, int nkv,
                                                        uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
  constexpr int CH = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)n_tokens * nkv * CH;
  if (idx >= total) return;
  const int c = (int)(idx % CH);
  const int h = (int)((idx / CH) % nkv);
  const int t = (int)(idx / ((int64_t)CH * nkv));
  const int sl = slot[t];
  const int page = sl >> 4, off = sl & 15;
  const size_t src = (size_t)t * row_stride + (size_t)h * D + c * 8;
  const uint4 kk = *reinterpret_cast<const uint4*>(k + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(v + src);
  const size_t pb = ((size_t)page * nkv + h) * (size_t)(16 * D);
  *reinterpret_cast<uint4*>(kc + pb + (size_t)off * D + c * 8) = kk;
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
  uint16_t* vbase = vc + pb + (size_t)(c * 8) * 16 + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vbase[(2 * e) * 16] = (uint16_t)(w[e] & 0xffff);
    vbase[(2 * e + 1) * 16] = (uint16_t)(w[e] >> 16);
  }
}

hb_status launch_kv_append(const hb_dims& d, const DevMeta& m, int n_tokens, const uint16_t* k,
                           const uint16_t* v, int64_t row_stride, uint16_t* kc, uint16_t* vc, stream_t s) {
  if (n_tokens <= 0) return HB_OK;
  const int64_t total = (int64_t)n_tokens * d.n_kv_heads * (d.head_dim / 8);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(kv_append_kernel<128>, dim3(blocks), dim3(256), 0, (hipStream_t)s, k, v, row_stride,
                       m.slot, n_tokens, d.n_kv_heads, kc, vc);
  else
    hipLaunchKernelGGL(kv_append_kernel<64>, dim3(blocks), dim3(256), 0, (hipStream_t)s, k, v, row_stride,
                       m.slot, n_tokens, d.n_kv_heads, kc, vc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HB_E_HIP, std::string("kv_append launch: ") + hipGetErrorString(e));
  return HB_OK;
}

}  // namespace hb
