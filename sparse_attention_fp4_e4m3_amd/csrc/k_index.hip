// k_index.hip -- indexer scoring, exact top-K selection and the hierarchical
// candidate pool on gfx950.
//
// Sources: "The global branch: compress, index, select" and "The
// hierarchical indexer" (course brief "DeepSeek-V4.1-Flash"); "The Paper"
// (talk write-up "DeepSeek V4.1 Flash: pushing the limits") for the Full /
// Reindex modes.  The pages give no score formula; the reading used is
// score = sum_h ReLU(q_h . k) with one shared key per entry, evaluated in a
// fixed fp32 order (fmaf chain over channels from +0, ReLU, left-to-right
// head sum) so that selection is reproducible bit for bit.
//
// Pipeline of one csa2_index_topk call (one stream, no host sync):
//   k_prep           indexer queries -> fp32, zero the radix histograms
//   k_scan_full      (Full)    every visible entry: score, block max, and the
//                              first radix histogram, fused; HBM-bound on the
//                              128 B (bf16) key rows
//   k_score_pool     (Reindex) pool entries only, same score
//   k_radix_pass<2>  second 11-bit digit histogram inside the threshold bin
//   k_radix_pass<3>  last 9-bit digit histogram
//   k_select_count   exact threshold T; per-chunk counts of > T and == T
//   k_select_write   ordered compaction: positions ascending, ties to the
//                    lower position, -1 padding; expands selected blocks
//                    into the pool
// Scores are non-negative fp32, so their bit patterns order like uint32;
// invalid slots carry -1.0 (sign bit set) and are never counted.
#include <algorithm>
#include <type_traits>

#include "csa2_common.h"

namespace csa2 {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanKeysPerThread = 2;
constexpr int kScanIters = 4;
constexpr int kScanChunk = kScanThreads * kScanKeysPerThread * kScanIters;  // 2048 positions
constexpr int kSelChunk = 8192;                                            // radix pass chunk
constexpr int kHistWords = kBins1 + kBins2 + kBins3;

struct Series {
  const float* arr;      // [R, stride] scores (sign bit set = invalid)
  int64_t stride;
  uint32_t* hist;        // [R, kHistWords]
  uint32_t* counts;      // [R, chunks, 2]
  uint32_t* state;       // [R, 4]: T, need_ties, all_flag, nsel
  int chunks;
  int K;
};

struct SelArgs {
  Series s[2];
  int nseries;
  int mode;                 // CSA2_FULL / CSA2_REINDEX
  const int32_t* row_visible;
  int max_visible;
  int pool_stride;
  const int32_t* pool;      // Reindex: slot -> position
  int32_t* out_idx;         // [R, K]
  int32_t* out_pool;        // [R, pool_size]
  int32_t* out_pool_len;    // [R]
  int pool_size;
};

__device__ __forceinline__ int row_len(const SelArgs& a, int series, int r) {
  if (a.mode == CSA2_REINDEX) return a.pool_stride;
  int v = a.row_visible[r];
  v = v < 0 ? 0 : (v > a.max_visible ? a.max_visible : v);
  return series == 0 ? v : (v + kBlock - 1) / kBlock;
}

__device__ __forceinline__ int visible_of(const int32_t* rv, int r, int maxv) {
  int v = rv[r];
  return v < 0 ? 0 : (v > maxv ? maxv : v);
}

// ------------------------------------------------------------ block scans
// 256 threads = 4 waves of 64.
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t* lds, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t t = lds[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__device__ __forceinline__ uint32_t block_flag_prefix(bool f, uint32_t* lds, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(f);
  const uint32_t lp = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) lds[wave] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t t = lds[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + lp;
}

// Bin holding the K-th largest element of a histogram (bins scanned from
// the top).  Returns -1 when the histogram holds fewer than K elements.
// *above = elements in higher bins, *total = all elements.
__device__ int find_bin(const uint32_t* __restrict__ h, int nbins, uint32_t K, uint32_t* above, uint32_t* total,
                        uint32_t* lds) {
  const int per = nbins / 256;
  const int hi = nbins - threadIdx.x * per;  // this thread: bins [hi-per, hi), descending
  uint32_t local = 0;
  for (int b = hi - 1; b >= hi - per; --b) local += h[b];
  uint32_t tot;
  const uint32_t before = block_excl_sum(local, lds, &tot);
  if (threadIdx.x == 0) lds[8] = 0xFFFFFFFFu;
  __syncthreads();
  if (before < K && K <= before + local) {
    uint32_t c = before;
    for (int b = hi - 1; b >= hi - per; --b) {
      const uint32_t n = h[b];
      if (K <= c + n) {
        lds[8] = (uint32_t)b;
        lds[9] = c;
        break;
      }
      c += n;
    }
  }
  __syncthreads();
  const uint32_t bin = lds[8], ab = lds[9];
  __syncthreads();
  *total = tot;
  *above = (bin == 0xFFFFFFFFu) ? tot : ab;
  return (bin == 0xFFFFFFFFu) ? -1 : (int)bin;
}

struct Threshold {
  uint32_t T;       // exact 31-bit key of the K-th largest element
  uint32_t need;    // ties at T to take (>= 1) unless all
  uint32_t nsel;    // elements selected = min(K, valid)
  bool all;         // fewer than K valid elements: select every valid one
};

// levels: how many digits are resolved (1..3); returns partial info for the
// radix passes and the full threshold at level 3.
__device__ Threshold resolve(const uint32_t* __restrict__ hist, uint32_t K, int levels, uint32_t* lds, int* b1o,
                             int* b2o) {
  Threshold t{0u, 0u, 0u, false};
  uint32_t above1, total;
  const int b1 = find_bin(hist, kBins1, K, &above1, &total, lds);
  *b1o = b1;
  if (b1 < 0) {
    t.all = true;
    t.nsel = total;
    return t;
  }
  t.nsel = K;
  if (levels < 2) return t;
  uint32_t above2, tot2;
  const int b2 = find_bin(hist + kBins1, kBins2, K - above1, &above2, &tot2, lds);
  *b2o = b2;
  if (levels < 3) return t;
  uint32_t above3, tot3;
  const int b3 = find_bin(hist + kBins1 + kBins2, kBins3, K - above1 - above2, &above3, &tot3, lds);
  t.T = ((uint32_t)b1 << kShift1) | ((uint32_t)b2 << kShift2) | (uint32_t)b3;
  t.need = K - above1 - above2 - above3;
  return t;
}

// ------------------------------------------------------------ the score
// fmaf chain over channels from +0, ReLU, heads summed left to right.
template <int KDT>
__device__ __forceinline__ void load_key(const void* __restrict__ k, int64_t row, float (&kv)[kIdxDim]) {
  if (KDT == CSA2_BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(k) + row * kIdxDim);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 t = __builtin_nontemporal_load(p + i);
      const uint32_t w[4] = {t[0], t[1], t[2], t[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kv[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        kv[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(k) + row * kIdxDim);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4 t = __builtin_nontemporal_load(p + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) kv[4 * i + j] = __uint_as_float(t[j]);
    }
  }
}

// scores of NK keys against H heads (H a template constant, or 0 = runtime hr)
template <int H, int NK>
__device__ __forceinline__ void score_keys(const float* __restrict__ q, int hr, const float (&kv)[NK][kIdxDim],
                                           float (&out)[NK]) {
  if constexpr (H > 0) {
    float acc[NK][H];
#pragma unroll
    for (int n = 0; n < NK; ++n)
#pragma unroll
      for (int h = 0; h < H; ++h) acc[n][h] = 0.0f;
#pragma unroll
    for (int c = 0; c < kIdxDim; ++c)
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const float qv = q[h * kIdxDim + c];
#pragma unroll
        for (int n = 0; n < NK; ++n) acc[n][h] = __builtin_fmaf(qv, kv[n][c], acc[n][h]);
      }
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      float s = acc[n][0] > 0.0f ? acc[n][0] : 0.0f;
#pragma unroll
      for (int h = 1; h < H; ++h) s = __fadd_rn(s, acc[n][h] > 0.0f ? acc[n][h] : 0.0f);
      out[n] = s;
    }
  } else {
#pragma unroll
    for (int n = 0; n < NK; ++n) out[n] = 0.0f;
    for (int h = 0; h < hr; ++h) {
      float acc[NK];
#pragma unroll
      for (int n = 0; n < NK; ++n) acc[n] = 0.0f;
#pragma unroll
      for (int c = 0; c < kIdxDim; ++c) {
        const float qv = q[h * kIdxDim + c];
#pragma unroll
        for (int n = 0; n < NK; ++n) acc[n] = __builtin_fmaf(qv, kv[n][c], acc[n]);
      }
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        const float rel = acc[n] > 0.0f ? acc[n] : 0.0f;
        out[n] = (h == 0) ? rel : __fadd_rn(out[n], rel);
      }
    }
  }
}

// ------------------------------------------------------------ kernels

__global__ __launch_bounds__(256) void k_prep(const void* __restrict__ idx_q, int q_dtype, int64_t nq,
                                              float* __restrict__ qf, uint32_t* __restrict__ hist, int64_t nhist) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += stride)
    qf[i] = (q_dtype == CSA2_BF16) ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(idx_q)[i] << 16)
                                   : static_cast<const float*>(idx_q)[i];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nhist; i += stride) hist[i] = 0u;
}

__device__ __forceinline__ void flush_hist(uint32_t* __restrict__ g, const uint32_t* __restrict__ l, int n) {
  for (int b = threadIdx.x; b < n; b += blockDim.x) {
    const uint32_t v = l[b];
    if (v) atomicAdd(g + b, v);
  }
}

template <int KDT, int H, bool POOL>
__global__ __launch_bounds__(kScanThreads) void k_scan_full(
    const float* __restrict__ qf, int hr, const void* __restrict__ idx_k, const int64_t* __restrict__ row_start,
    const int32_t* __restrict__ row_visible, int max_vis, float* __restrict__ scores, int64_t n_pad,
    float* __restrict__ bmax, int64_t nb_pad, uint32_t* __restrict__ hist_s, uint32_t* __restrict__ hist_b) {
  __shared__ uint32_t h1[kBins1];
  __shared__ uint32_t hb[POOL ? kBins1 : 1];
  const int r = blockIdx.y;
  const int vis = visible_of(row_visible, r, max_vis);
  const int base = blockIdx.x * kScanChunk;
  if (base >= vis) return;
  for (int b = threadIdx.x; b < kBins1; b += kScanThreads) {
    h1[b] = 0u;
    if (POOL) hb[b] = 0u;
  }
  __syncthreads();
  const float* q = qf + (int64_t)r * (H > 0 ? H : hr) * kIdxDim;
  const int64_t rs = row_start[r];
  float* srow = scores + (int64_t)r * n_pad;
  for (int it = 0; it < kScanIters; ++it) {
    int j[kScanKeysPerThread];
    float kv[kScanKeysPerThread][kIdxDim];
#pragma unroll
    for (int n = 0; n < kScanKeysPerThread; ++n) {
      j[n] = base + (it * kScanKeysPerThread + n) * kScanThreads + threadIdx.x;
      const int jj = j[n] < vis ? j[n] : vis - 1;  // tail lanes reload a valid row, result dropped
      load_key<KDT>(idx_k, rs + jj, kv[n]);
    }
    float s[kScanKeysPerThread];
    score_keys<H, kScanKeysPerThread>(q, hr, kv, s);
#pragma unroll
    for (int n = 0; n < kScanKeysPerThread; ++n) {
      const bool ok = j[n] < vis;
      if (ok) {
        srow[j[n]] = s[n];
        atomicAdd(&h1[__float_as_uint(s[n]) >> kShift1], 1u);
      }
      if (POOL) {
        // block of 8 consecutive positions = 8 consecutive lanes
        float m = ok ? s[n] : -1.0f;
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        if (ok && (threadIdx.x & 7) == 0) {
          bmax[(int64_t)r * nb_pad + j[n] / kBlock] = m;
          atomicAdd(&hb[__float_as_uint(m) >> kShift1], 1u);
        }
      }
    }
  }
  __syncthreads();
  flush_hist(hist_s + (int64_t)r * kHistWords, h1, kBins1);
  if (POOL) flush_hist(hist_b + (int64_t)r * kHistWords, hb, kBins1);
}

template <int KDT, int H>
__global__ __launch_bounds__(kScanThreads) void k_score_pool(
    const float* __restrict__ qf, int hr, const void* __restrict__ idx_k, const int64_t* __restrict__ row_start,
    const int32_t* __restrict__ row_visible, int max_vis, const int32_t* __restrict__ pool,
    const int32_t* __restrict__ pool_len, int pool_stride, float* __restrict__ scores, int64_t n_pad,
    uint32_t* __restrict__ hist_s) {
  __shared__ uint32_t h1[kBins1];
  const int r = blockIdx.y;
  const int base = blockIdx.x * kScanChunk;
  if (base >= pool_stride) return;
  for (int b = threadIdx.x; b < kBins1; b += kScanThreads) h1[b] = 0u;
  __syncthreads();
  const int vis = visible_of(row_visible, r, max_vis);
  int plen = pool_len ? pool_len[r] : pool_stride;
  plen = plen < 0 ? 0 : (plen > pool_stride ? pool_stride : plen);
  const float* q = qf + (int64_t)r * (H > 0 ? H : hr) * kIdxDim;
  const int64_t rs = row_start[r];
  const int32_t* prow = pool + (int64_t)r * pool_stride;
  float* srow = scores + (int64_t)r * n_pad;
  for (int it = 0; it < kScanIters; ++it) {
    int i[kScanKeysPerThread];
    bool ok[kScanKeysPerThread];
    float kv[kScanKeysPerThread][kIdxDim];
#pragma unroll
    for (int n = 0; n < kScanKeysPerThread; ++n) {
      i[n] = base + (it * kScanKeysPerThread + n) * kScanThreads + threadIdx.x;
      const int p = (i[n] < plen) ? prow[i[n]] : -1;
      ok[n] = p >= 0 && p < vis;
      if (ok[n]) {
        load_key<KDT>(idx_k, rs + p, kv[n]);
      } else {
#pragma unroll
        for (int c = 0; c < kIdxDim; ++c) kv[n][c] = 0.0f;
      }
    }
    float s[kScanKeysPerThread];
    score_keys<H, kScanKeysPerThread>(q, hr, kv, s);
#pragma unroll
    for (int n = 0; n < kScanKeysPerThread; ++n) {
      if (i[n] < pool_stride) srow[i[n]] = ok[n] ? s[n] : -1.0f;
      if (ok[n]) atomicAdd(&h1[__float_as_uint(s[n]) >> kShift1], 1u);
    }
  }
  __syncthreads();
  flush_hist(hist_s + (int64_t)r * kHistWords, h1, kBins1);
}

// Histogram of the next digit over elements that match the resolved prefix.
template <int LEVEL>
__global__ __launch_bounds__(256) void k_radix_pass(SelArgs a) {
  __shared__ uint32_t lh[LEVEL == 2 ? kBins2 : kBins3];
  __shared__ uint32_t red[16];
  const int series = blockIdx.z, r = blockIdx.y, c = blockIdx.x;
  if (series >= a.nseries) return;
  const Series& S = a.s[series];
  const int n = row_len(a, series, r);
  const int base = c * kSelChunk;
  if (base >= n) return;
  const uint32_t* hist = S.hist + (int64_t)r * kHistWords;
  int b1 = -1, b2 = -1;
  const Threshold t = resolve(hist, (uint32_t)S.K, LEVEL - 1, red, &b1, &b2);
  if (t.all) return;
  constexpr int NB = LEVEL == 2 ? kBins2 : kBins3;
  for (int b = threadIdx.x; b < NB; b += 256) lh[b] = 0u;
  __syncthreads();
  const float* arr = S.arr + (int64_t)r * S.stride;
  const int end = min(n, base + kSelChunk);
  for (int i = base + threadIdx.x; i < end; i += 256) {
    const uint32_t key = __float_as_uint(arr[i]);
    if (key >> 31) continue;
    if ((int)(key >> kShift1) != b1) continue;
    if (LEVEL == 2) {
      atomicAdd(&lh[(key >> kShift2) & (kBins2 - 1)], 1u);
    } else {
      if ((int)((key >> kShift2) & (kBins2 - 1)) != b2) continue;
      atomicAdd(&lh[key & (kBins3 - 1)], 1u);
    }
  }
  __syncthreads();
  flush_hist(S.hist + (int64_t)r * kHistWords + (LEVEL == 2 ? kBins1 : kBins1 + kBins2), lh, NB);
}

__global__ __launch_bounds__(256) void k_select_count(SelArgs a) {
  __shared__ uint32_t red[16];
  const int series = blockIdx.z, r = blockIdx.y, c = blockIdx.x;
  if (series >= a.nseries) return;
  const Series& S = a.s[series];
  const int n = row_len(a, series, r);
  const int base = c * kSelChunk;
  if (base >= n && c != 0) return;
  int b1, b2;
  const Threshold t = resolve(S.hist + (int64_t)r * kHistWords, (uint32_t)S.K, 3, red, &b1, &b2);
  if (c == 0 && threadIdx.x == 0) {
    uint32_t* st = S.state + (int64_t)r * 4;
    st[0] = t.T;
    st[1] = t.need;
    st[2] = t.all ? 1u : 0u;
    st[3] = t.nsel;
  }
  if (base >= n) return;
  const float* arr = S.arr + (int64_t)r * S.stride;
  const int end = min(n, base + kSelChunk);
  uint32_t gt = 0, eq = 0;
  for (int i = base + threadIdx.x; i < end; i += 256) {
    const uint32_t key = __float_as_uint(arr[i]);
    if (key >> 31) continue;
    if (t.all || key > t.T) ++gt;
    else if (key == t.T) ++eq;
  }
  uint32_t tg, te;
  block_excl_sum(gt, red, &tg);
  block_excl_sum(eq, red, &te);
  if (threadIdx.x == 0) {
    uint32_t* cnt = S.counts + ((int64_t)r * S.chunks + c) * 2;
    cnt[0] = tg;
    cnt[1] = te;
  }
}

__global__ __launch_bounds__(256) void k_select_write(SelArgs a) {
  __shared__ uint32_t red[16];
  __shared__ uint32_t pre[2];
  const int series = blockIdx.z, r = blockIdx.y, c = blockIdx.x;
  if (series >= a.nseries) return;
  const Series& S = a.s[series];
  const int n = row_len(a, series, r);
  const int base = c * kSelChunk;
  const uint32_t* st = S.state + (int64_t)r * 4;
  const uint32_t T = st[0], need = st[1], nsel = st[3];
  const bool all = st[2] != 0u;
  const int vis = (a.mode == CSA2_FULL) ? visible_of(a.row_visible, r, a.max_visible) : 0;
  // padding and the pool length (chunk 0)
  if (c == 0) {
    if (series == 0) {
      int32_t* o = a.out_idx + (int64_t)r * S.K;
      for (int i = (int)nsel + threadIdx.x; i < S.K; i += 256) o[i] = -1;
    } else {
      // pool length: full blocks except a partial last block if it was kept
      const int nb = n;  // blocks of this row
      int plen = (int)nsel * kBlock;
      if (nsel > 0 && (vis % kBlock) != 0) {
        const uint32_t lastkey = __float_as_uint(S.arr[(int64_t)r * S.stride + nb - 1]);
        bool kept;
        if (all) kept = true;
        else if (lastkey > T) kept = true;
        else if (lastkey == T) {
          // the last block is the highest-index tie: kept iff every tie is taken
          uint32_t ties = 0;
          const uint32_t* cnt = S.counts + (int64_t)r * S.chunks * 2;
          const int nch = (nb + kSelChunk - 1) / kSelChunk;
          for (int k = 0; k < nch; ++k) ties += cnt[2 * k + 1];
          kept = need >= ties;
        } else kept = false;
        if (kept) plen -= kBlock - (vis % kBlock);
      }
      int32_t* o = a.out_pool + (int64_t)r * a.pool_size;
      for (int i = plen + threadIdx.x; i < a.pool_size; i += 256) o[i] = -1;
      if (threadIdx.x == 0) a.out_pool_len[r] = plen;
    }
  }
  if (base >= n) return;
  // selections and ties in earlier chunks
  if (threadIdx.x == 0) {
    uint32_t gtb = 0, eqb = 0;
    const uint32_t* cnt = S.counts + (int64_t)r * S.chunks * 2;
    for (int k = 0; k < c; ++k) {
      gtb += cnt[2 * k];
      eqb += cnt[2 * k + 1];
    }
    pre[0] = gtb + (all ? 0u : min(eqb, need));
    pre[1] = eqb;
  }
  __syncthreads();
  uint32_t out_pos = pre[0];
  uint32_t ties_seen = pre[1];
  __syncthreads();
  const float* arr = S.arr + (int64_t)r * S.stride;
  const int end = min(n, base + kSelChunk);
  for (int i0 = base; i0 < end; i0 += 256) {
    const int i = i0 + threadIdx.x;
    const uint32_t key = (i < end) ? __float_as_uint(arr[i]) : 0x80000000u;
    const bool valid = !(key >> 31);
    const bool tie = valid && !all && key == T;
    uint32_t ntie;
    const uint32_t tr = block_flag_prefix(tie, red, &ntie);
    const bool sel = valid && (all || key > T || (tie && ties_seen + tr < need));
    uint32_t nsel_it;
    const uint32_t sr = block_flag_prefix(sel, red, &nsel_it);
    if (sel) {
      const uint32_t p = out_pos + sr;
      if (p >= nsel) {
        // unreachable when the threshold is consistent; keeps every store in bounds
      } else if (series == 0) {
        const int32_t pos = (a.mode == CSA2_FULL) ? i : a.pool[(int64_t)r * a.pool_stride + i];
        a.out_idx[(int64_t)r * S.K + p] = pos;
      } else {
        int32_t* o = a.out_pool + (int64_t)r * a.pool_size + (int64_t)p * kBlock;
#pragma unroll
        for (int m = 0; m < kBlock; ++m) {
          const int pos = i * kBlock + m;
          if (pos < vis) o[m] = pos;
        }
      }
    }
    out_pos += nsel_it;
    ties_seen += ntie;
  }
}

template <int KDT, int H, bool POOL>
void launch_scoring(int mode, dim3 grid, hipStream_t s, const float* qf, int hr, const void* idx_k,
                    const int64_t* row_start, const int32_t* row_visible, int max_vis, const int32_t* pool,
                    const int32_t* pool_len, int pool_stride, const TopkWorkspace& w, uint32_t* hist_b) {
  if (mode == CSA2_FULL)
    hipLaunchKernelGGL((k_scan_full<KDT, H, POOL>), grid, dim3(kScanThreads), 0, s, qf, hr, idx_k, row_start,
                       row_visible, max_vis, w.scores, w.n_pad, w.bmax, w.nb_pad, w.hist, hist_b);
  else
    hipLaunchKernelGGL((k_score_pool<KDT, H>), grid, dim3(kScanThreads), 0, s, qf, hr, idx_k, row_start,
                       row_visible, max_vis, pool, pool_len, pool_stride, w.scores, w.n_pad, w.hist);
}

template <int KDT, bool POOL>
void dispatch_heads(int H, int mode, dim3 grid, hipStream_t s, const float* qf, const void* idx_k,
                    const int64_t* row_start, const int32_t* row_visible, int max_vis, const int32_t* pool,
                    const int32_t* pool_len, int pool_stride, const TopkWorkspace& w, uint32_t* hist_b) {
  if (H == 8)
    launch_scoring<KDT, 8, POOL>(mode, grid, s, qf, H, idx_k, row_start, row_visible, max_vis, pool, pool_len,
                                 pool_stride, w, hist_b);
  else if (H == 4)
    launch_scoring<KDT, 4, POOL>(mode, grid, s, qf, H, idx_k, row_start, row_visible, max_vis, pool, pool_len,
                                 pool_stride, w, hist_b);
  else
    launch_scoring<KDT, 0, POOL>(mode, grid, s, qf, H, idx_k, row_start, row_visible, max_vis, pool, pool_len,
                                 pool_stride, w, hist_b);
}

struct Carve {
  char* p;
  size_t off = 0;
  template <class T>
  T* take(size_t count) {
    T* r = reinterpret_cast<T*>(p ? p + off : nullptr);
    off += (count * sizeof(T) + 255) & ~size_t(255);
    return r;
  }
};

struct Layout {
  TopkWorkspace w;
  uint32_t* hist_b;
  uint32_t* counts_b;
  uint32_t* state;
  size_t bytes;
};

Layout layout(void* base, int mode, int R, int H, int max_visible, int pool_stride, int pool_size) {
  Layout L{};
  Carve c{static_cast<char*>(base)};
  const int64_t n = (mode == CSA2_FULL) ? max_visible : pool_stride;
  L.w.n_pad = round_up(n > 0 ? n : 1, 64);
  L.w.chunks = (int)ceil_div(n > 0 ? n : 1, kSelChunk);
  const bool pool_on = mode == CSA2_FULL && pool_size > 0;
  const int64_t nb = pool_on ? ceil_div(max_visible, kBlock) : 0;
  L.w.nb_pad = round_up(nb > 0 ? nb : 1, 64);
  L.w.bchunks = (int)ceil_div(nb > 0 ? nb : 1, kSelChunk);
  L.w.qf = c.take<float>((size_t)R * H * kIdxDim);
  L.w.hist = c.take<uint32_t>((size_t)R * kHistWords * (pool_on ? 2 : 1));
  L.hist_b = pool_on ? L.w.hist + (size_t)R * kHistWords : nullptr;
  L.w.counts = c.take<uint32_t>((size_t)R * L.w.chunks * 2);
  L.counts_b = pool_on ? c.take<uint32_t>((size_t)R * L.w.bchunks * 2) : nullptr;
  L.state = c.take<uint32_t>((size_t)R * 8);
  L.w.scores = c.take<float>((size_t)R * L.w.n_pad);
  L.w.bmax = pool_on ? c.take<float>((size_t)R * L.w.nb_pad) : nullptr;
  L.bytes = c.off;
  return L;
}

}  // namespace

size_t topk_workspace_bytes(int mode, int R, int H, int max_visible, int pool_stride, int pool_size) {
  return layout(nullptr, mode, R, H, max_visible, pool_stride, pool_size).bytes;
}

hipError_t launch_index_topk(int mode, int R, const void* idx_q, int q_dtype, int H, const void* idx_k, int k_dtype,
                             const int64_t* row_start, const int32_t* row_visible, int max_visible,
                             const int32_t* pool, const int32_t* pool_len, int pool_stride, int top_k,
                             int32_t* out_idx, int pool_size, int32_t* out_pool, int32_t* out_pool_len, void* ws,
                             hipStream_t s) {
  const bool pool_on = mode == CSA2_FULL && pool_size > 0;
  Layout L = layout(ws, mode, R, H, max_visible, pool_stride, pool_size);
  const int64_t nq = (int64_t)R * H * kIdxDim;
  const int64_t nhist = (int64_t)R * kHistWords * (pool_on ? 2 : 1);
  hipLaunchKernelGGL(k_prep, dim3((unsigned)std::min<int64_t>(2048, ceil_div(std::max(nq, nhist), 256))), dim3(256),
                     0, s, idx_q, q_dtype, nq, L.w.qf, L.w.hist, nhist);

  // scoring
  const int64_t n = (mode == CSA2_FULL) ? max_visible : pool_stride;
  if (n > 0) {
    const dim3 grid((unsigned)ceil_div(n, kScanChunk), (unsigned)R);
    auto& ev = profile_events(mode == CSA2_FULL ? CSA2_KERNEL_INDEX_SCAN : CSA2_KERNEL_REINDEX_SCORE);
    if (ev.start) hipEventRecord(ev.start, s);
    const TopkWorkspace& w = L.w;
    if (k_dtype == CSA2_BF16) {
      if (pool_on)
        dispatch_heads<CSA2_BF16, true>(H, mode, grid, s, w.qf, idx_k, row_start, row_visible, max_visible, pool,
                                        pool_len, pool_stride, w, L.hist_b);
      else
        dispatch_heads<CSA2_BF16, false>(H, mode, grid, s, w.qf, idx_k, row_start, row_visible, max_visible, pool,
                                         pool_len, pool_stride, w, L.hist_b);
    } else {
      if (pool_on)
        dispatch_heads<CSA2_F32, true>(H, mode, grid, s, w.qf, idx_k, row_start, row_visible, max_visible, pool,
                                       pool_len, pool_stride, w, L.hist_b);
      else
        dispatch_heads<CSA2_F32, false>(H, mode, grid, s, w.qf, idx_k, row_start, row_visible, max_visible, pool,
                                        pool_len, pool_stride, w, L.hist_b);
    }
    if (ev.stop) hipEventRecord(ev.stop, s);
  }

  // selection
  SelArgs a{};
  a.mode = mode;
  a.row_visible = row_visible;
  a.max_visible = max_visible;
  a.pool_stride = pool_stride;
  a.pool = pool;
  a.out_idx = out_idx;
  a.out_pool = out_pool;
  a.out_pool_len = out_pool_len;
  a.pool_size = pool_size;
  a.nseries = pool_on ? 2 : 1;
  a.s[0] = Series{L.w.scores, L.w.n_pad, L.w.hist, L.w.counts, L.state, L.w.chunks, top_k};
  if (pool_on) a.s[1] = Series{L.w.bmax, L.w.nb_pad, L.hist_b, L.counts_b, L.state + (size_t)R * 4, L.w.bchunks,
                               pool_size / kBlock};
  const int gx = std::max(L.w.chunks, pool_on ? L.w.bchunks : 1);
  const dim3 grid((unsigned)gx, (unsigned)R, (unsigned)a.nseries);
  hipLaunchKernelGGL(k_radix_pass<2>, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_radix_pass<3>, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_select_count, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_select_write, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
