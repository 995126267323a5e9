// csa2_api.cpp -- the extern "C" boundary: argument checks, workspace sizing,
// dispatch to the gfx950 launchers.  Checks read host-visible arguments only;
// no call synchronizes, allocates or copies.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "csa2_common.h"

namespace csa2 {

static thread_local std::string g_last_error;
static ProfileEvents g_events[16];

ProfileEvents& profile_events(int id) { return g_events[(id >= 0 && id < 16) ? id : 0]; }

static int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

static int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA2_OK;
  return fail(CSA2_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------- the library's scratch
// csa2_sparse_attn_noalloc keeps the split partials and merge counters of its
// launches in this array instead of a caller's workspace.  On the host the
// array's name stands for a host-side shadow, not device memory: host code
// takes the device address from hipGetSymbolAddress, once per device, and
// passes only that address to kernels.
constexpr size_t kStaticScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

__global__ void k_clear_u64(uint64_t* p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0;
}

// Device address of the current device's scratch, looked up on the first call
// on that device, which also clears the merge counters on stream s (the array
// starts zero-filled and every call leaves the counters zero).
static int32_t static_scratch(const char* fn, hipStream_t s, void** out);
static bool dtype_ok(int32_t d) { return d == CSA2_F32 || d == CSA2_BF16; }
static size_t dtype_size(int32_t d) { return d == CSA2_F32 ? 4 : 2; }

static int32_t static_scratch(const char* fn, hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CSA2_E_UNSUPPORTED, "%s: device %d (the library keeps scratch for devices 0..%d)", fn, dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(CSA2_E_HIP, "%s: hipGetSymbolAddress(scratch) gave a null address", fn);
    constexpr int n = (int)(kAttnCounterBytes / 8);
    hipLaunchKernelGGL(k_clear_u64, dim3((n + 255) / 256), dim3(256), 0, s, static_cast<uint64_t*>(p), n);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

// checks shared by csa2_sparse_attn and csa2_sparse_attn_noalloc (all but the workspace)
static int32_t sparse_attn_args(const char* fn, int32_t n_rows, const void* q, int32_t q_dtype, int32_t n_heads,
                                int32_t head_dim, const uint8_t* kv_codes, const uint8_t* kv_scales,
                                const int64_t* row_kv_start, const int32_t* idx, int32_t top_k, float softmax_scale,
                                const void* out, int32_t out_dtype) {
  if (n_rows < 0) return fail(CSA2_E_INVALID, "%s: n_rows < 0", fn);
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return fail(CSA2_E_INVALID, "%s: dtype is not F32/BF16", fn);
  if (head_dim != kDim) return fail(CSA2_E_UNSUPPORTED, "%s: head_dim %d (only 512 is built)", fn, head_dim);
  if (n_heads < 16 || n_heads > 128 || n_heads % 16)
    return fail(CSA2_E_INVALID, "%s: n_heads %d must be a multiple of 16 in 16..128", fn, n_heads);
  if (top_k < 1) return fail(CSA2_E_INVALID, "%s: top_k %d < 1", fn, top_k);
  if (!(softmax_scale == softmax_scale)) return fail(CSA2_E_INVALID, "%s: softmax_scale is NaN", fn);
  if (n_rows == 0) return CSA2_OK;
  if (!q || !kv_codes || !kv_scales || !row_kv_start || !idx || !out)
    return fail(CSA2_E_INVALID, "%s: null buffer", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(kv_codes, 16) || !aligned(kv_scales, 8))
    return fail(CSA2_E_INVALID, "%s: q/out/kv_codes must be 16-byte and kv_scales 8-byte aligned", fn);
  return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" {

const char* csa2_last_error(void) { return g_last_error.c_str(); }

int32_t csa2_profile_kernel_events(int32_t kernel_id, void* start_event, void* stop_event) {
  if (kernel_id < CSA2_KERNEL_QUANT || kernel_id > CSA2_KERNEL_QUANT_MXFP4)
    return fail(CSA2_E_INVALID, "csa2_profile_kernel_events: unknown kernel id %d", kernel_id);
  g_events[kernel_id].start = static_cast<hipEvent_t>(start_event);
  g_events[kernel_id].stop = static_cast<hipEvent_t>(stop_event);
  return CSA2_OK;
}

int32_t csa2_quantize_kv_fp4(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t x_row_stride,
                             const int64_t* dst_rows, uint8_t* kv_codes, uint8_t* kv_scales, int64_t cap_rows,
                             void* stream) {
  if (n_tokens < 0) return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: n_tokens < 0");
  if (!dtype_ok(x_dtype)) return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: x_dtype %d is not F32/BF16", x_dtype);
  if (n_tokens == 0) return CSA2_OK;
  if (!x || !kv_codes || !kv_scales) return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: null buffer");
  if (x_row_stride < kDim) return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: x_row_stride %lld < 512",
                                       (long long)x_row_stride);
  if (!aligned(x, 16) || (x_row_stride * (int64_t)dtype_size(x_dtype)) % 16 != 0)
    return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: x rows must be 16-byte aligned");
  if (!aligned(kv_codes, 8)) return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: kv_codes must be 8-byte aligned");
  if (cap_rows <= 0) return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: cap_rows <= 0");
  if (!dst_rows && n_tokens > cap_rows)
    return fail(CSA2_E_INVALID, "csa2_quantize_kv_fp4: n_tokens %lld > cap_rows %lld", (long long)n_tokens,
                (long long)cap_rows);
  return hip_status(launch_quantize(x, x_dtype, n_tokens, x_row_stride, dst_rows, kv_codes, kv_scales, cap_rows,
                                    static_cast<hipStream_t>(stream)),
                    "csa2_quantize_kv_fp4");
}

size_t csa2_index_topk_workspace_size(int32_t mode, int32_t n_rows, int32_t n_heads, int32_t max_visible,
                                      int32_t pool_stride, int32_t top_k, int32_t pool_size) {
  (void)top_k;
  if (n_rows <= 0 || n_heads <= 0) return 0;
  return topk_workspace_bytes(mode, n_rows, n_heads, max_visible < 0 ? 0 : max_visible,
                              pool_stride < 0 ? 0 : pool_stride, pool_size < 0 ? 0 : pool_size);
}

}  // extern "C"

// one validation and dispatch for both key formats (fn names the caller)
static int32_t index_topk(const char* fn, int32_t mode, int32_t n_rows, const void* idx_q, int32_t q_dtype,
                          int32_t n_heads, int32_t head_dim, const void* idx_k, const uint8_t* idx_ks,
                          int32_t k_dtype, int32_t k_heads, const int64_t* row_kv_start, const int32_t* row_visible,
                          int32_t max_visible, const int32_t* pool, const int32_t* pool_len, int32_t pool_stride,
                          int32_t top_k, int32_t* out_idx, int32_t pool_size, int32_t block_size, int32_t* out_pool,
                          int32_t* out_pool_len, void* workspace, size_t workspace_bytes, void* stream) {
  const bool mx = k_dtype == CSA2_MXFP4;
  if (mode != CSA2_FULL && mode != CSA2_REINDEX && mode != CSA2_FULL_SHARED)
    return fail(CSA2_E_INVALID, "%s: unknown mode %d", fn, mode);
  if (n_rows < 0) return fail(CSA2_E_INVALID, "%s: n_rows < 0", fn);
  if (!dtype_ok(q_dtype) || !(mx || dtype_ok(k_dtype))) return fail(CSA2_E_INVALID, "%s: dtype is not F32/BF16", fn);
  if (head_dim != kIdxDim) return fail(CSA2_E_UNSUPPORTED, "%s: head_dim %d (only 64 is built)", fn, head_dim);
  if (k_heads != 1)
    return fail(CSA2_E_UNSUPPORTED, "%s: k_heads %d (only one key shared by the query heads is built)", fn, k_heads);
  if (n_heads < 1 || n_heads > 32) return fail(CSA2_E_UNSUPPORTED, "%s: n_heads %d outside 1..32", fn, n_heads);
  if (top_k < 1 || top_k > CSA2_MAX_TOP_K) return fail(CSA2_E_INVALID, "%s: top_k %d outside 1..%d", fn, top_k,
                                                       CSA2_MAX_TOP_K);
  if (max_visible < 0) return fail(CSA2_E_INVALID, "%s: max_visible < 0", fn);
  if (max_visible > topk_max_visible())
    return fail(CSA2_E_UNSUPPORTED, "%s: max_visible %d above the built limit %d", fn, max_visible, topk_max_visible());
  if (mode == CSA2_REINDEX && pool_stride > 65536)
    return fail(CSA2_E_UNSUPPORTED, "%s: pool_stride %d above 65536", fn, pool_stride);
  if (n_rows == 0) return CSA2_OK;
  if (!idx_q || !idx_k || (mx && !idx_ks) || !row_kv_start || !row_visible || !out_idx)
    return fail(CSA2_E_INVALID, "%s: null buffer", fn);
  if (!aligned(idx_k, 16)) return fail(CSA2_E_INVALID, "%s: idx_k must be 16-byte aligned", fn);
  if (mx && !aligned(idx_ks, 2)) return fail(CSA2_E_INVALID, "%s: idx_k_scales must be 2-byte aligned", fn);
  if (mode == CSA2_REINDEX) {
    if (!pool) return fail(CSA2_E_INVALID, "%s: REINDEX needs a pool", fn);
    if (pool_stride < 1) return fail(CSA2_E_INVALID, "%s: REINDEX needs pool_stride >= 1", fn);
    if (pool_size != 0) return fail(CSA2_E_INVALID, "%s: REINDEX does not emit a pool (pool_size must be 0)", fn);
  }
  if (mode != CSA2_REINDEX && pool_size != 0) {
    if (pool_size < 0 || block_size != kBlock || pool_size % kBlock != 0)
      return fail(CSA2_E_INVALID, "%s: pool_size %d must be a positive multiple of block_size 8 (got %d)", fn,
                  pool_size, block_size);
    if (!out_pool || !out_pool_len) return fail(CSA2_E_INVALID, "%s: pool outputs are null", fn);
  }
  const size_t need = topk_workspace_bytes(mode, n_rows, n_heads, max_visible, pool_stride, pool_size);
  if (!workspace || workspace_bytes < need)
    return fail(CSA2_E_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(CSA2_E_INVALID, "%s: workspace must be 256-byte aligned", fn);
  return hip_status(launch_index_topk(mode, n_rows, idx_q, q_dtype, n_heads, idx_k, idx_ks, k_dtype, row_kv_start,
                                      row_visible, max_visible, pool, pool_len, pool_stride, top_k, out_idx,
                                      mode != CSA2_REINDEX ? pool_size : 0, out_pool, out_pool_len, workspace,
                                      static_cast<hipStream_t>(stream)),
                    fn);
}

extern "C" {

int32_t csa2_index_topk(int32_t mode, int32_t n_rows, const void* idx_q, int32_t q_dtype, int32_t n_heads,
                        int32_t head_dim, const void* idx_k, int32_t k_dtype, int32_t k_heads,
                        const int64_t* row_kv_start,
                        const int32_t* row_visible, int32_t max_visible, const int32_t* pool,
                        const int32_t* pool_len, int32_t pool_stride, int32_t top_k, int32_t* out_idx,
                        int32_t pool_size, int32_t block_size, int32_t* out_pool, int32_t* out_pool_len,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (k_dtype == CSA2_MXFP4)
    return fail(CSA2_E_INVALID, "csa2_index_topk: MXFP4 keys go through csa2_index_topk_mxfp4");
  return index_topk("csa2_index_topk", mode, n_rows, idx_q, q_dtype, n_heads, head_dim, idx_k, nullptr, k_dtype,
                    k_heads, row_kv_start, row_visible, max_visible, pool, pool_len, pool_stride, top_k, out_idx, pool_size,
                    block_size, out_pool, out_pool_len, workspace, workspace_bytes, stream);
}

int32_t csa2_index_topk_mxfp4(int32_t mode, int32_t n_rows, const void* idx_q, int32_t q_dtype, int32_t n_heads,
                              int32_t head_dim, const uint8_t* idx_k_codes, const uint8_t* idx_k_scales,
                              int32_t k_heads, const int64_t* row_kv_start, const int32_t* row_visible, int32_t max_visible,
                              const int32_t* pool, const int32_t* pool_len, int32_t pool_stride, int32_t top_k,
                              int32_t* out_idx, int32_t pool_size, int32_t block_size, int32_t* out_pool,
                              int32_t* out_pool_len, void* workspace, size_t workspace_bytes, void* stream) {
  return index_topk("csa2_index_topk_mxfp4", mode, n_rows, idx_q, q_dtype, n_heads, head_dim, idx_k_codes,
                    idx_k_scales, CSA2_MXFP4, k_heads, row_kv_start, row_visible, max_visible, pool, pool_len, pool_stride,
                    top_k, out_idx, pool_size, block_size, out_pool, out_pool_len, workspace, workspace_bytes, stream);
}

int32_t csa2_quantize_idx_mxfp4(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t x_row_stride,
                                const int64_t* dst_rows, uint8_t* k_codes, uint8_t* k_scales, int64_t cap_rows,
                                void* stream) {
  const char* fn = "csa2_quantize_idx_mxfp4";
  if (n_tokens < 0) return fail(CSA2_E_INVALID, "%s: n_tokens < 0", fn);
  if (!dtype_ok(x_dtype)) return fail(CSA2_E_INVALID, "%s: x_dtype %d is not F32/BF16", fn, x_dtype);
  if (n_tokens == 0) return CSA2_OK;
  if (!x || !k_codes || !k_scales) return fail(CSA2_E_INVALID, "%s: null buffer", fn);
  if (x_row_stride < kIdxDim) return fail(CSA2_E_INVALID, "%s: x_row_stride %lld < 64", fn, (long long)x_row_stride);
  if (!aligned(x, 16) || (x_row_stride * (int64_t)dtype_size(x_dtype)) % 16)
    return fail(CSA2_E_INVALID, "%s: x rows must be 16-byte aligned", fn);
  if (!aligned(k_codes, 16) || !aligned(k_scales, 2))
    return fail(CSA2_E_INVALID, "%s: k_codes must be 16-byte and k_scales 2-byte aligned", fn);
  if (cap_rows <= 0) return fail(CSA2_E_INVALID, "%s: cap_rows <= 0", fn);
  if (!dst_rows && n_tokens > cap_rows)
    return fail(CSA2_E_INVALID, "%s: n_tokens %lld > cap_rows %lld", fn, (long long)n_tokens, (long long)cap_rows);
  return hip_status(launch_quantize_mxfp4(x, x_dtype, n_tokens, x_row_stride, dst_rows, k_codes, k_scales, cap_rows,
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

int32_t csa2_visible_entries(const int64_t* token_pos, int32_t tokens_per_entry, int32_t n_rows,
                             int32_t* row_visible, void* stream) {
  const char* fn = "csa2_visible_entries";
  if (n_rows < 0) return fail(CSA2_E_INVALID, "%s: n_rows < 0", fn);
  if (tokens_per_entry < 1) return fail(CSA2_E_INVALID, "%s: tokens_per_entry %d < 1", fn, tokens_per_entry);
  if (n_rows == 0) return CSA2_OK;
  if (!token_pos || !row_visible) return fail(CSA2_E_INVALID, "%s: null buffer", fn);
  return hip_status(launch_visible(token_pos, tokens_per_entry, n_rows, row_visible, static_cast<hipStream_t>(stream)),
                    fn);
}

size_t csa2_sparse_attn_workspace_size(int32_t n_rows, int32_t n_heads, int32_t q_dtype, int32_t top_k) {
  if (n_rows <= 0 || n_heads <= 0 || n_heads % 16 || top_k <= 0 || !dtype_ok(q_dtype)) return 0;
  return attn_workspace_bytes(n_rows, n_heads, q_dtype, top_k, false);
}

int32_t csa2_sparse_attn(int32_t n_rows, const void* q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                         const uint8_t* kv_codes, const uint8_t* kv_scales, const int64_t* row_kv_start,
                         const int32_t* idx, int32_t top_k, const int32_t* row_visible, float softmax_scale,
                         void* out, int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const char* fn = "csa2_sparse_attn";
  const int32_t rc = sparse_attn_args(fn, n_rows, q, q_dtype, n_heads, head_dim, kv_codes, kv_scales, row_kv_start,
                                      idx, top_k, softmax_scale, out, out_dtype);
  if (rc != CSA2_OK || n_rows == 0) return rc;
  const size_t need = attn_workspace_bytes(n_rows, n_heads, q_dtype, top_k, false);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CSA2_E_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
  if (need && !aligned(workspace, 256)) return fail(CSA2_E_INVALID, "%s: workspace must be 256-byte aligned", fn);
  return hip_status(launch_sparse_attn(n_rows, q, q_dtype, n_heads, kv_codes, kv_scales, row_kv_start, idx, top_k,
                                       row_visible, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, softmax_scale,
                                       out, out_dtype, lse,
                                       workspace, static_cast<hipStream_t>(stream)),
                    fn);
}

int32_t csa2_sparse_attn_noalloc(int32_t n_rows, const void* q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                                 const uint8_t* kv_codes, const uint8_t* kv_scales, const int64_t* row_kv_start,
                                 const int32_t* idx, int32_t top_k, const int32_t* row_visible, float softmax_scale,
                                 void* out, int32_t out_dtype, float* lse, void* stream) {
  const char* fn = "csa2_sparse_attn_noalloc";
  const int32_t rc = sparse_attn_args(fn, n_rows, q, q_dtype, n_heads, head_dim, kv_codes, kv_scales, row_kv_start,
                                      idx, top_k, softmax_scale, out, out_dtype);
  if (rc != CSA2_OK || n_rows == 0) return rc;
  const size_t need = attn_workspace_bytes(n_rows, n_heads, q_dtype, top_k, false);
  if (need > kStaticScratchBytes)
    return fail(CSA2_E_WORKSPACE, "%s: the call needs %zu bytes of scratch, more than the %zu the library holds "
                "(csa2_sparse_attn takes a workspace of any size)", fn, need, kStaticScratchBytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need) {
    const int32_t r2 = static_scratch(fn, s, &ws);
    if (r2 != CSA2_OK) return r2;
  }
  return hip_status(launch_sparse_attn(n_rows, q, q_dtype, n_heads, kv_codes, kv_scales, row_kv_start, idx, top_k,
                                       row_visible, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, softmax_scale,
                                       out, out_dtype, lse, ws, s),
                    fn);
}

int32_t csa2_quantize_swa_fp8(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t x_row_stride,
                              const int64_t* dst_rows, uint8_t* win_codes, int64_t cap_rows, void* stream) {
  const char* fn = "csa2_quantize_swa_fp8";
  if (n_tokens < 0) return fail(CSA2_E_INVALID, "%s: n_tokens < 0", fn);
  if (!dtype_ok(x_dtype)) return fail(CSA2_E_INVALID, "%s: x_dtype %d is not F32/BF16", fn, x_dtype);
  if (n_tokens == 0) return CSA2_OK;
  if (!x || !win_codes) return fail(CSA2_E_INVALID, "%s: null buffer", fn);
  if (x_row_stride < kDim) return fail(CSA2_E_INVALID, "%s: x_row_stride %lld < 512", fn, (long long)x_row_stride);
  if (!aligned(x, 16) || (x_row_stride * (int64_t)dtype_size(x_dtype)) % 16)
    return fail(CSA2_E_INVALID, "%s: x rows must be 16-byte aligned", fn);
  if (!aligned(win_codes, 16)) return fail(CSA2_E_INVALID, "%s: win_codes must be 16-byte aligned", fn);
  if (cap_rows <= 0) return fail(CSA2_E_INVALID, "%s: cap_rows <= 0", fn);
  if (!dst_rows && n_tokens > cap_rows)
    return fail(CSA2_E_INVALID, "%s: n_tokens %lld > cap_rows %lld", fn, (long long)n_tokens, (long long)cap_rows);
  return hip_status(launch_quantize_fp8(x, x_dtype, n_tokens, x_row_stride, dst_rows, win_codes, cap_rows,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

size_t csa2_sparse_attn_swa_workspace_size(int32_t n_rows, int32_t n_heads, int32_t q_dtype, int32_t top_k) {
  if (n_rows <= 0 || n_heads <= 0 || n_heads % 16 || top_k < 0 || !dtype_ok(q_dtype)) return 0;
  return attn_workspace_bytes(n_rows, n_heads, q_dtype, top_k, true);
}

int32_t csa2_sparse_attn_swa(int32_t n_rows, const void* q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                             const uint8_t* kv_codes, const uint8_t* kv_scales, const int64_t* row_kv_start,
                             const int32_t* idx, int32_t top_k, const int32_t* row_visible,
                             uint8_t* win_codes, const int64_t* row_win_start, const int32_t* row_win_len,
                             const void* new_x, int32_t new_x_dtype, int64_t new_x_stride, const int64_t* new_rows,
                             float softmax_scale, void* out, int32_t out_dtype, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const char* fn = "csa2_sparse_attn_swa";
  if (n_rows < 0) return fail(CSA2_E_INVALID, "%s: n_rows < 0", fn);
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return fail(CSA2_E_INVALID, "%s: dtype is not F32/BF16", fn);
  if (head_dim != kDim) return fail(CSA2_E_UNSUPPORTED, "%s: head_dim %d (only 512 is built)", fn, head_dim);
  if (n_heads < 16 || n_heads > 128 || n_heads % 16)
    return fail(CSA2_E_INVALID, "%s: n_heads %d must be a multiple of 16 in 16..128", fn, n_heads);
  if (top_k < 0) return fail(CSA2_E_INVALID, "%s: top_k %d < 0", fn, top_k);
  if (!(softmax_scale == softmax_scale)) return fail(CSA2_E_INVALID, "%s: softmax_scale is NaN", fn);
  if (n_rows == 0) return CSA2_OK;
  if (!q || !out || !win_codes || !row_win_start || !row_win_len) return fail(CSA2_E_INVALID, "%s: null buffer", fn);
  if (top_k > 0 && (!kv_codes || !kv_scales || !row_kv_start || !idx))
    return fail(CSA2_E_INVALID, "%s: null cache or index buffer with top_k > 0", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(win_codes, 16))
    return fail(CSA2_E_INVALID, "%s: q/out/win_codes must be 16-byte aligned", fn);
  if (top_k > 0 && (!aligned(kv_codes, 16) || !aligned(kv_scales, 8)))
    return fail(CSA2_E_INVALID, "%s: kv_codes must be 16-byte and kv_scales 8-byte aligned", fn);
  if (new_x) {
    if (!dtype_ok(new_x_dtype)) return fail(CSA2_E_INVALID, "%s: new_x_dtype %d is not F32/BF16", fn, new_x_dtype);
    if (!new_rows) return fail(CSA2_E_INVALID, "%s: new_x without new_rows", fn);
    if (new_x_stride < kDim) return fail(CSA2_E_INVALID, "%s: new_x_stride %lld < 512", fn, (long long)new_x_stride);
    if (!aligned(new_x, 16) || (new_x_stride * (int64_t)dtype_size(new_x_dtype)) % 16)
      return fail(CSA2_E_INVALID, "%s: new_x rows must be 16-byte aligned", fn);
  }
  const size_t need = attn_workspace_bytes(n_rows, n_heads, q_dtype, top_k, true);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CSA2_E_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
  if (need && !aligned(workspace, 256)) return fail(CSA2_E_INVALID, "%s: workspace must be 256-byte aligned", fn);
  return hip_status(launch_sparse_attn(n_rows, q, q_dtype, n_heads, kv_codes, kv_scales, row_kv_start, idx, top_k,
                                       row_visible, win_codes, row_win_start, row_win_len, new_x, new_x_dtype,
                                       new_x_stride, new_rows, softmax_scale, out, out_dtype, lse, workspace,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
