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

// radix digits over the 31 value bits of a non-negative fp32 score
constexpr int kBins1 = 2048, kBins2 = 2048, kBins3 = 512;
constexpr int kShift1 = 20, kShift2 = 9;

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

struct TopkWorkspace {
  // carved from the caller's workspace
  float* qf;             // [R, H, 64] fp32 copy of the indexer queries
  float* scores;         // [R, n_pad] fp32 (Full: positions; Reindex: pool slots)
  float* bmax;           // [R, nb_pad] fp32 block maxima (Full with pool)
  uint32_t* hist;        // [2 series][R][kBins1 + kBins2 + kBins3]
  uint32_t* counts;      // [2 series][R][chunks][2]
  int64_t n_pad, nb_pad;
  int chunks, bchunks;
};

size_t topk_workspace_bytes(int mode, int R, int H, int max_visible, int pool_stride, int pool_size);

hipError_t launch_index_topk(int mode, int R, const void* idx_q, int q_dtype, int H, const void* idx_k, int k_dtype,
                             const int64_t* row_start, const int32_t* row_visible, int max_visible,
                             const int32_t* pool, const int32_t* pool_len, int pool_stride, int top_k,
                             int32_t* out_idx, int pool_size, int32_t* out_pool, int32_t* out_pool_len,
                             void* ws, hipStream_t s);

size_t attn_workspace_bytes(int R, int Hq, int q_dtype, int top_k);

hipError_t launch_sparse_attn(int R, const void* q, int q_dtype, int Hq, const uint8_t* codes, const uint8_t* scales,
                              const int64_t* row_start, const int32_t* idx, int top_k, const int32_t* row_visible,
                              float softmax_scale, void* out, int out_dtype, float* lse, void* ws, hipStream_t s);

// ------------------------------------------------------------ device helpers
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
#endif

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace csa2
