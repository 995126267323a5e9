// csa2_common.h -- shared host/device declarations of the gfx950 CSA2 library.
// Internal header: not part of the C ABI (include/csa2.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

constexpr int kDim = 512;       // latent channels per cache entry
constexpr int kGroup = 16;      // channels per E4M3 scale
constexpr int kGroups = 32;     // scales per entry
constexpr int kCodeBytes = 256; // E2M1 bytes per entry
constexpr int kIdxDim = 64;     // indexer head dim
constexpr int kBlock = 8;       // hierarchical pool block

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// per-kernel event recording (measurement hook of the C ABI)
struct ProfileEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfileEvents& profile_events(int kernel_id);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are pre-validated.

hipError_t launch_quantize(const void* x, int x_dtype, int64_t n, int64_t stride, const int64_t* dst_rows,
                           uint8_t* codes, uint8_t* scales, int64_t cap, hipStream_t s);

size_t topk_workspace_bytes(int mode, int R, int H, int max_visible, int pool_stride, int pool_size);
int topk_max_visible();

// k_dtype CSA2_MXFP4: idx_k = codes [rows][32], idx_ks = E8M0 scales [rows][2]; else idx_ks unused
hipError_t launch_index_topk(int mode, int R, const void* idx_q, int q_dtype, int H, const void* idx_k,
                             const uint8_t* idx_ks, int k_dtype,
                             const int64_t* row_start, const int32_t* row_visible, int max_visible,
                             const int32_t* pool, const int32_t* pool_len, int pool_stride, int top_k,
                             int32_t* out_idx, int pool_size, int32_t* out_pool, int32_t* out_pool_len,
                             void* ws, hipStream_t s);

hipError_t launch_quantize_mxfp4(const void* x, int x_dtype, int64_t n, int64_t stride, const int64_t* dst_rows,
                                 uint8_t* codes, uint8_t* scales, int64_t cap, hipStream_t s);

// row_visible of query rows at token positions pos when each entry folds m tokens
hipError_t launch_visible(const int64_t* pos, int m, int n, int32_t* vis, hipStream_t s);

hipError_t launch_quantize_fp8(const void* x, int x_dtype, int64_t n, int64_t stride, const int64_t* dst_rows,
                               uint8_t* codes, int64_t cap, hipStream_t s);

// Attention workspace: the first kAttnCounterBytes hold the arrival counters of
// split launches that merge their own partials; they are zero before the first
// call and every call leaves them zero.  Split partials follow them.
constexpr size_t kAttnCounterBytes = 4096;

// window = true: one more partial slot per (row, head) for the local window
size_t attn_workspace_bytes(int R, int Hq, int q_dtype, int top_k, bool window);

// decode attention with 32-head workgroups (bf16 queries) and the merge of its key splits; a local
// window joins when that merge runs inside the launch, as a partial the window kernel writes first
// (normalized fp32 [R][Hq][2][512], slot 1, with its (max, sum) [R][Hq][2]) in the last
// attn_dec_window_bytes of the workspace
bool attn_dec_applies(int R, int Hq, int q_dtype, int top_k, bool window);
size_t attn_dec_window_bytes(int R, int Hq);
size_t attn_dec_workspace_bytes(int R, int Hq, int top_k, bool window);
hipError_t launch_attn_dec(int R, const void* q, int Hq, const uint8_t* codes, const uint8_t* scales,
                           const int64_t* row_start, const int32_t* idx, int top_k, const int32_t* row_visible,
                           float softmax_scale, void* out, int out_dtype, float* lse, const float* win_o,
                           const float* win_m, const float* win_l, void* ws, hipStream_t s);

// top_k may be 0 when a window is given (win != nullptr): the window alone is attended
hipError_t launch_sparse_attn(int R, const void* q, int q_dtype, int Hq, const uint8_t* codes, const uint8_t* scales,
                              const int64_t* row_start, const int32_t* idx, int top_k, const int32_t* row_visible,
                              uint8_t* win, const int64_t* win_start, const int32_t* win_len,
                              const void* new_x, int new_x_dtype, int64_t new_x_stride, const int64_t* new_rows,
                              float softmax_scale, void* out, int out_dtype, float* lse, void* ws, hipStream_t s);

// ------------------------------------------------------------ device helpers
// Workgroup barrier for LDS traffic only.  HIP's __syncthreads() also waits
// for every outstanding global load (s_waitcnt vmcnt(0)), which would drain
// register prefetches issued ahead of the barrier; this one waits for this
// wave's LDS operations only, so global loads stay in flight across it.
// Use it only where the data exchanged through the barrier lives in LDS.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// nearest E4M3 (E4M3FN) code of v >= 0, ties to even, saturating at 448
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0.015625f) {  // below 2^-6: subnormal grid m * 2^-9 (scaling by 512 is exact)
    return (uint32_t)__float2int_rn(v * 512.0f);
  }
  const uint32_t u = __float_as_uint(v);
  const uint32_t e = (u >> 23) - 120u;  // rebias 127 -> 7
  const uint32_t man = u & 0x7FFFFFu;
  const uint32_t keep = man >> 20, rest = man & 0xFFFFFu;
  uint32_t code = (e << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1u;  // carries into the exponent
  return code;
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace csa2
