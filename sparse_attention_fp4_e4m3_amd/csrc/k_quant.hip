// k_quant.hip -- quantize-on-write of 512-channel KV latents to FP4, of
// local-window latents to FP8, and of indexer keys to MXFP4.
//
// Cache format of "FP4 cache entries, and why they're safe" (course brief
// "DeepSeek-V4.1-Flash"): E2M1 elements, one E4M3 scale per 16 channels, no
// second-level global scale, 256 + 32 = 288 bytes per entry.  Scale choice
// and rounding are the plainest reading of that section: s = E4M3(amax/6)
// round-to-nearest-even (6 = largest E2M1 value), elements E2M1(x/s)
// round-to-nearest-even.
//
// Layout: 32 lanes per token, lane g owns group g (16 channels = 64 B of
// fp32 input or 32 B of bf16), so a wave covers two tokens with fully
// coalesced loads; each lane writes 8 code bytes and 1 scale byte.
// HBM-bound: 2 KiB (fp32) or 1 KiB (bf16) read + 288 B written per token.
#include "csa2_common.h"

namespace csa2 {
namespace {

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// nearest E2M1 code, ties to even code, |q| > 6 -> 6, sign kept.
// Thresholds: midpoints .25 .75 1.25 1.75 2.5 3.5 5; at a midpoint the even
// code wins, hence '>' above an even neighbour and '>=' below one.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const float a = fabsf(q);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(q) >> 28) & 8u);
}

template <int DT>
__global__ __launch_bounds__(256) void k_quant_fp4(const void* __restrict__ x, int64_t n, int64_t stride,
                                                   const int64_t* __restrict__ dst_rows, uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, int64_t cap) {
  const int64_t tok = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int g = threadIdx.x & 31;
  if (tok >= n) return;
  const int64_t dst = dst_rows ? dst_rows[tok] : tok;
  if (dst < 0 || dst >= cap) return;
  float v[16];
  if (DT == CSA2_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + tok * stride + g * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 t = p[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + tok * stride + g * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 t = p[i];
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sb = e4m3_code(__fdiv_rn(amax, 6.0f));
  const float s = e4m3_value(sb);
  uint32_t lo = 0, hi = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) lo |= e2m1_code(__fdiv_rn(v[i], s)) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hi |= e2m1_code(__fdiv_rn(v[8 + i], s)) << (4 * i);
  }
  *reinterpret_cast<uint2*>(codes + dst * kCodeBytes + g * 8) = make_uint2(lo, hi);
  scales[dst * kGroups + g] = (uint8_t)sb;
}

// Local-window entries: one signed E4M3 byte per channel (the brief's
// "FP4 cache entries, and why they're safe" keeps the local sliding-window
// cache in FP8; no scale is named, so values are stored as they are):
// nearest value, ties to the even code, |x| > 448 saturating to 448, the
// sign bit copied from x (a negative value that rounds to zero gives 0x80).
// Same thread layout as k_quant_fp4; each lane writes 16 bytes.
template <int DT>
__global__ __launch_bounds__(256) void k_quant_fp8(const void* __restrict__ x, int64_t n, int64_t stride,
                                                   const int64_t* __restrict__ dst_rows, uint8_t* __restrict__ codes,
                                                   int64_t cap) {
  const int64_t tok = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int g = threadIdx.x & 31;
  if (tok >= n) return;
  const int64_t dst = dst_rows ? dst_rows[tok] : tok;
  if (dst < 0 || dst >= cap) return;
  uint32_t u[16];  // fp32 bits of the lane's 16 channels
  if (DT == CSA2_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + tok * stride + g * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 t = p[i];
      u[4 * i] = t.x; u[4 * i + 1] = t.y; u[4 * i + 2] = t.z; u[4 * i + 3] = t.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + tok * stride + g * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 t = p[i];
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u[8 * i + 2 * k] = w[k] << 16;
        u[8 * i + 2 * k + 1] = w[k] & 0xFFFF0000u;
      }
    }
  }
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t b = e4m3_code(__uint_as_float(u[i] & 0x7FFFFFFFu)) | ((u[i] >> 24) & 0x80u);
    out[i >> 2] |= b << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(codes + dst * kDim + g * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

// Indexer keys in OCP MXFP4 (64 channels = two blocks of 32 sharing an E8M0
// scale each), converted as the OCP Microscaling specification gives it:
// X = 2^(floor(log2 amax) - 2) -- for a normal amax with biased exponent E
// that is E8M0 code E - 2; a zero or subnormal amax gives code 0 -- then
// E2M1(x / X) with the FP4 element rounding above.  One thread per block of
// 32 channels writes 16 code bytes and 1 scale byte.
template <int DT>
__global__ __launch_bounds__(256) void k_quant_mx(const void* __restrict__ x, int64_t n, int64_t stride,
                                                  const int64_t* __restrict__ dst_rows, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales, int64_t cap) {
  const int64_t tok = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 1;
  const int blk = threadIdx.x & 1;
  if (tok >= n) return;
  const int64_t dst = dst_rows ? dst_rows[tok] : tok;
  if (dst < 0 || dst >= cap) return;
  float v[32];
  if (DT == CSA2_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + tok * stride + blk * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 t = p[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + tok * stride + blk * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 t = p[i];
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const uint32_t sb = (uint32_t)max(e - 2, 0);
  const float X = __uint_as_float(sb ? (sb << 23) : 0x00400000u);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) out[i >> 3] |= e2m1_code(__fdiv_rn(v[i], X)) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(codes + dst * 32 + blk * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  scales[dst * 2 + blk] = (uint8_t)sb;
}

// Visible entries of query rows when each cache entry folds m consecutive
// tokens (entry e covers tokens m*e .. m*e + m - 1; "The global branch" in the
// course brief: the encoder layers compress m = 2 tokens per entry): a query
// at token position t sees the entries whose whole block lies at or before t,
// (t + 1) / m of them; t < 0 sees none.
__global__ __launch_bounds__(256) void k_visible(const int64_t* __restrict__ pos, int m, int n,
                                                 int32_t* __restrict__ vis) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t t = pos[i];
  const int64_t e = t < 0 ? 0 : (t + 1) / m;
  vis[i] = (int32_t)(e > 0x7FFFFFFF ? 0x7FFFFFFF : e);
}

}  // namespace

hipError_t launch_visible(const int64_t* pos, int m, int n, int32_t* vis, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_visible, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, pos, m, n, vis);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const void* x, int x_dtype, int64_t n, int64_t stride, const int64_t* dst_rows,
                                 uint8_t* codes, uint8_t* scales, int64_t cap, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(n, 128)), block(256);
  auto& ev = profile_events(CSA2_KERNEL_QUANT_MXFP4);
  if (ev.start) (void)hipEventRecord(ev.start, s);
  if (x_dtype == CSA2_F32)
    hipLaunchKernelGGL(k_quant_mx<CSA2_F32>, grid, block, 0, s, x, n, stride, dst_rows, codes, scales, cap);
  else
    hipLaunchKernelGGL(k_quant_mx<CSA2_BF16>, grid, block, 0, s, x, n, stride, dst_rows, codes, scales, cap);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, int x_dtype, int64_t n, int64_t stride, const int64_t* dst_rows,
                               uint8_t* codes, int64_t cap, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(n, 8)), block(256);
  auto& ev = profile_events(CSA2_KERNEL_QUANT_FP8);
  if (ev.start) (void)hipEventRecord(ev.start, s);
  if (x_dtype == CSA2_F32)
    hipLaunchKernelGGL(k_quant_fp8<CSA2_F32>, grid, block, 0, s, x, n, stride, dst_rows, codes, cap);
  else
    hipLaunchKernelGGL(k_quant_fp8<CSA2_BF16>, grid, block, 0, s, x, n, stride, dst_rows, codes, cap);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int x_dtype, int64_t n, int64_t stride, const int64_t* dst_rows,
                           uint8_t* codes, uint8_t* scales, int64_t cap, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(n, 8)), block(256);
  auto& ev = profile_events(CSA2_KERNEL_QUANT);
  if (ev.start) (void)hipEventRecord(ev.start, s);
  if (x_dtype == CSA2_F32)
    hipLaunchKernelGGL(k_quant_fp4<CSA2_F32>, grid, block, 0, s, x, n, stride, dst_rows, codes, scales, cap);
  else
    hipLaunchKernelGGL(k_quant_fp4<CSA2_BF16>, grid, block, 0, s, x, n, stride, dst_rows, codes, scales, cap);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
  return hipGetLastError();
}

}  // namespace csa2
