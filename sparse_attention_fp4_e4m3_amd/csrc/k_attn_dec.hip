// k_attn_dec.hip -- decode sparse attention over FP4 cache entries with
// 32-head workgroups on v_mfma_f32_32x32x16_f16, and its split-K merge.
//
// What it computes ("The Paper" in the talk write-up "DeepSeek V4.1 Flash:
// pushing the limits": K and V are the same Main KV entry; "The global
// branch" in the course brief "DeepSeek-V4.1-Flash": one 512-dim latent per
// entry shared by every query head, so decode attention is one small GEMM
// per row): for row r and head h, softmax over the selected entries of
// softmax_scale * q . x_hat, then the weighted sum of the x_hat.
//
// Numerics.  x_hat = E2M1 code * E4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16.  A head's bf16 query is
// multiplied by the power of two 2^sh that puts its largest magnitude in
// [2^14, 2^15); 2^-sh is folded into that head's logit scale.  The scaled
// values convert to fp16 exactly down to 2^-28 of the head's maximum (the
// fp16 normal range), whatever the query's own range.  Both products run on
// fp16 MFMA with fp32 accumulation; probabilities are rounded to fp16 and the
// row sums add those same rounded values.  Split partials are normalized
// outputs stored in fp16 (relative 2^-11) with fp32 maxima and sums.
//
// Work split.  A workgroup of 8 waves owns one (row, 32 heads, key split)
// and walks its keys in chunks of 256, 32 keys per wave:
//  * QK^T: wave w gathers keys [32w, 32w+32) of the chunk straight from HBM
//    into registers (lane = key, lane/32 = channel half), dequantizes them
//    into the A operand and multiplies with the 32 heads' queries (LDS) as
//    the B operand: S^T[key][head] in one 32x32 accumulator.
//  * softmax: per-head maxima and sums of the 8 waves meet in LDS; the
//    online maximum rescales the running outputs between chunks.
//  * PV: wave w owns channels [64w, 64w+64) of every head.  The raw FP4
//    rows are staged in LDS as they arrived; ds_read_b64_tr_b4 hands each
//    lane one channel of 16 consecutive keys (the K-contiguous B operand),
//    so each conversion yields two keys of one channel, multiplied by those
//    keys' scales (staged as fp16, transposed, by the QK lanes).
//  Every FP4 element is dequantized once for QK^T and once for PV.
// Split-K: each (row, head group) has S workgroups; each writes its
// normalized fp16 partial straight from its accumulators (device-scope stores,
// no transpose) and its (max, sum) per head, and k_dec_combine merges the S
// partials in fixed split order, so results are deterministic.
// A row's local window ("The Paper" in the talk write-up: the selected
// entries and the recent window share one softmax) joins as one more
// partial: the window kernel writes it (normalized fp32, with its (max, sum))
// before this launch, and the in-launch merge weighs it after the splits.
#include <algorithm>

#include "csa2_common.h"

namespace csa2 {
namespace {

constexpr int kT = 512;        // threads per workgroup (8 waves, two per SIMD)
constexpr int kHG = 32;        // heads per workgroup
constexpr int kChunk = 256;    // keys per chunk (32 per wave)
constexpr int kQS = 520;       // fp16 per staged query row (512 + 8 pad)
constexpr int kCS = 272;       // bytes per staged code row (256 + 16 pad: transposed reads hit distinct banks)
constexpr int kSS = 264;       // fp16 per staged scale row [group][key] (256 keys + 8 pad)
constexpr int kPS = 264;       // fp16 per probability row [head][key]
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplits = 8;   // key splits per (row, head group)
constexpr int kMaxPairs = 256;  // (row, 32-head group) pairs; more rows take the 64-head prefill kernel
static_assert(kMaxPairs * 16 <= (int)kAttnCounterBytes, "arrival and done counters of every pair");
constexpr int kMergeParts = 4;  // merge workgroups per pair: one 16-byte piece of every attention lane each
constexpr int kSpinMax = 1 << 21;  // bounded wait of a merge workgroup (about 100 ms at 128 clocks per poll)

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

struct DecArgs {
  const uint16_t* q;        // [R][Hq][512] bf16
  int Hq;
  const uint8_t* codes;     // [rows][256]
  const uint8_t* scales;    // [rows][32]
  const int64_t* row_start;
  const int32_t* idx;       // [R][top_k]
  int top_k;
  const int32_t* row_visible;
  float c2;                 // softmax_scale * log2(e)
  void* out;
  int out_dtype;
  float* lse;
  const float* win_o;       // the local window's partial, written before this launch, or null:
                            // normalized fp32 [R][Hq][2][512] (slot 1), its (max, sum) in win_m, win_l [R][Hq][2]
  const float* win_m;
  const float* win_l;
  int splits;               // S
  int kps;                  // keys per split (multiple of kChunk)
  int xcd_map;              // 1: the S splits of a (row, head group) share blockIdx.x % 8
  int grp;                  // xcd_map: consecutive pairs that share an XCD (a row's head groups, which
                            // gather the same entries, when rows come in multiples of 8; else 1)
  _Float16* ws_o;           // [pairs][S][wave][piece 4][lane][8] normalized partials in accumulator order
  float* ws_ml;             // [pairs][32 heads][S][2] (max in log2 units, sum)
  uint64_t* counters;       // [pairs][cstride]: attention arrivals, merge parts done in the first two words
                            // (zero between calls); null: the merge runs as a launch of its own
  int cstride;              // words between pairs' counters: one 128-byte line per pair when they fit
  int nattn;                // attention workgroups (pairs x S); higher blockIdx.x are merge workgroups
};

struct __align__(16) SmemDec {
  _Float16 q[kHG * kQS];
  union {
    uint8_t cs[kChunk * kCS];          // raw code rows of the chunk
    _Float16 ob[kHG * 512];             // epilogue: the fp16 partial, row-major
  } u;
  _Float16 ss[32 * kSS];                // scales [group][key]
  _Float16 ps[kHG * kPS];               // probabilities [head][key]
  float red_max[8][kHG];
  float red_sum[8][kHG];
  float c2h[kHG];
  float alpha[kHG];
  float ifin[kHG];
  __align__(16) float om[16][kMaxSplits];  // merge workgroups: weights of the splits of their 16 heads
  float omw[16];                           // and of the window's partial
  int flag;
};

__device__ __forceinline__ uint32_t h2u(half2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2v u2h(uint32_t u) { return __builtin_bit_cast(half2v, u); }

template <int SEL>
__device__ __forceinline__ half2v fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 cat4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8, u32x4{a, b, c, d});
}

// lanes l and l^32 hold the same head (32x32 accumulator column) for the two key halves
__device__ __forceinline__ float half_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// One chunk's raw bytes in a lane's registers, in the order they are loaded:
// code piece i = 16 bytes [16*(lane%16), +16) of key 4*i + lane/16 of the
// wave's 32 keys (four whole rows per load instruction: 8 cache lines), and
// the scale bytes [16*h2, +16) of key l32 (the key this lane scores).
struct RawKey {
  u32x4 c[8];
  u32x4 s;
};

// index slots of the lane's 9 loads (8 code pieces, then the scale load)
struct Slots {
  int32_t j[9];
};

__device__ __forceinline__ void load_slots(Slots& S, const DecArgs& a, int r, int kc0, int kend, int w, int lane) {
  const int32_t* row = a.idx + (int64_t)r * a.top_k;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = kc0 + 32 * w + 4 * i + (lane >> 4);
    S.j[i] = row[slot < kend ? slot : kend - 1];
  }
  const int slot = kc0 + 32 * w + (lane & 31);
  S.j[8] = row[slot < kend ? slot : kend - 1];
}

// Gather of one chunk: an invalid slot reads cache row 0 (always present) so
// that every load is issued without a branch.  Only the scale load's key is
// masked (its scales are zeroed and its logits set to -inf); the codes of an
// invalid key are finite E2M1 values and meet zero scales.
__device__ __forceinline__ void gather(RawKey& k, const DecArgs& a, const Slots& S, int64_t rs, int vis, int kc0,
                                       int kend, int w, int lane, uint32_t& valid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = kc0 + 32 * w + 4 * i + (lane >> 4);
    const bool ok = (slot < kend) & ((uint32_t)S.j[i] < (uint32_t)vis);
    const int64_t row = ok ? rs + S.j[i] : 0;
    k.c[i] = *reinterpret_cast<const u32x4*>(a.codes + row * kCodeBytes + 16 * (lane & 15));
  }
  const int slot = kc0 + 32 * w + (lane & 31);
  const bool ok = (slot < kend) & ((uint32_t)S.j[8] < (uint32_t)vis);
  valid = ok;
  const int64_t row = ok ? rs + S.j[8] : 0;
  k.s = *reinterpret_cast<const u32x4*>(a.scales + row * kGroups + 16 * (lane >> 5));
}

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float h_lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu)); }
__device__ __forceinline__ float h_hi(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }

// A merge workgroup: merges piece pc (tile pc >> 1, accumulator rows 8*(pc&1) .. +7: 16 heads x 256
// channels) of the S partials of one (row, head group) once their S attention workgroups have
// arrived.  Merge workgroups have higher blockIdx.x than every attention workgroup, so each starts only
// once every attention workgroup has been placed on a CU, and it waits for its pair by polling the
// arrival counter (bounded: past kSpinMax polls it writes NaN).  The S attention workgroups and the merge
// workgroups of a pair share blockIdx.x % 8, hence one XCC and one L2: workgroups are dispatched to the
// XCCs round-robin in blockIdx order, though not always from XCC 0 (graph launches start elsewhere).
// Each arrival adds 1 to the count and 1 to a 4-bit field of its XCC, and a merge workgroup proceeds only
// when the field of its own XCC holds all S arrivals (else NaN): the partials, stored before each arrival
// is counted, are then in its L2 and are read back past this CU's L1 (agent-scope loads).  The last merge
// workgroup of a pair to finish resets both counters for the next call.
// Pair of the t-th (pair, ...) slot of XCD x: XCD x holds the groups of grp consecutive pairs numbered
// x, x + 8, x + 16, ...
__device__ __forceinline__ int xcd_pair(int t, int x, int grp) { return (8 * (t / grp) + x) * grp + t % grp; }

__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7u; }

__device__ __forceinline__ void merge_part(const DecArgs& a, SmemDec& sm) {
  const int j = (int)blockIdx.x - a.nattn;
  const int jx = j >> 3, x = j & 7;
  const int pair = xcd_pair(jx / kMergeParts, x, a.grp), pc = jx % kMergeParts;
  const int S = a.splits;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31, tt = pc >> 1, jj = pc & 1;
  const int nhg = a.Hq / kHG;
  const int r = pair / nhg, h0 = (pair % nhg) * kHG;
  if (tid == 0) {
    uint64_t c = 0;
    int it = 0;
    for (; it < kSpinMax; ++it) {
      c = __hip_atomic_load(&a.counters[a.cstride * pair], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int)(c & 255u) >= S) break;
      __builtin_amdgcn_s_sleep(2);
    }
    sm.flag = (it < kSpinMax && (int)((c >> (8 + 4 * xcc_id())) & 15u) == S) ? 1 : 0;
  }
  lds_barrier();
  const bool ok = sm.flag != 0;
  // threads 0..15: the (max, sum) pairs of head 16*jj + tid, issued first (they are needed first);
  // then every thread's piece pc of (split s, wave w, lane): 16 bytes each, all in flight, from L2
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(a.ws_ml, 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.ws_o, 0, 0x7FFFFFFF, 0x00020000);
  u32x2 ml[kMaxSplits];
  if (tid < 16) {
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
      const uint32_t e = (uint32_t)(((size_t)pair * kHG + 16 * jj + tid) * S + (s2 < S ? s2 : 0));
      ml[s2] = __builtin_amdgcn_raw_buffer_load_b64(rm, (int)(8u * e), 0, 16);
    }
  }
  u32x4 v[kMaxSplits];
#pragma unroll
  for (int s2 = 0; s2 < kMaxSplits; ++s2) {
    const uint32_t off = (uint32_t)((((((size_t)pair * S + (s2 < S ? s2 : 0)) * 8 + w) * 4 + pc) * 64 + lane) * 16);
    v[s2] = __builtin_amdgcn_raw_buffer_load_b128(ro, (int)off, 0, 16);
  }
  // the window's partial (an earlier launch wrote it): this thread's 8 outputs, its heads' (max, sum)
  float wo[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wm = -INFINITY, wl = 0.0f;
  if (a.win_o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t hh = (int64_t)r * a.Hq + h0 + 16 * jj + 8 * (e >> 2) + 4 * h2 + (e & 3);
      wo[e] = a.win_o[(hh * 2 + 1) * kDim + 64 * w + 32 * tt + l32];
    }
    if (tid < 16) {
      const int64_t hh = (int64_t)r * a.Hq + h0 + 16 * jj + tid;
      wm = a.win_m[hh * 2 + 1];
      wl = a.win_l[hh * 2 + 1];
    }
  }
  // weights of the splits of each head, in fixed split order, then the window's
  if (tid < 16) {
    float M = wm;
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2)
      if (s2 < S) M = fmaxf(M, __uint_as_float(ml[s2][0]));
    float wg[kMaxSplits], L = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
      wg[s2] = (s2 < S && M != -INFINITY)
                   ? __builtin_amdgcn_exp2f(__uint_as_float(ml[s2][0]) - M) * __uint_as_float(ml[s2][1])
                   : 0.0f;
      L += wg[s2];
    }
    const float ww = M != -INFINITY ? __builtin_amdgcn_exp2f(wm - M) * wl : 0.0f;  // 0 without a window
    L += ww;
    const float iL = L > 0.0f ? 1.0f / L : 0.0f;
    *reinterpret_cast<floatx4*>(&sm.om[tid][0]) = floatx4{wg[0] * iL, wg[1] * iL, wg[2] * iL, wg[3] * iL};
    *reinterpret_cast<floatx4*>(&sm.om[tid][4]) = floatx4{wg[4] * iL, wg[5] * iL, wg[6] * iL, wg[7] * iL};
    sm.omw[tid] = ww * iL;
    if (a.lse && tt == 0)
      a.lse[(int64_t)r * a.Hq + h0 + 16 * jj + tid] = !ok ? __builtin_nanf("") : L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  }
  lds_barrier();  // (the piece loads stay in flight)
  // rows i = 8*jj + e of this lane: head 8*(i/4) + 4*h2 + i%4 (= 16*jj + local head), channel 64w + 32tt + l32
  floatx4 wv[8][2];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int hl = 8 * (e >> 2) + 4 * h2 + (e & 3);
    wv[e][0] = *reinterpret_cast<const floatx4*>(&sm.om[hl][0]);
    wv[e][1] = *reinterpret_cast<const floatx4*>(&sm.om[hl][4]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < kMaxSplits; ++s2) {
    if (s2 >= S) break;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += wv[2 * k][s2 >> 2][s2 & 3] * h_lo(v[s2][k]);
      acc[2 * k + 1] += wv[2 * k + 1][s2 >> 2][s2 & 3] * h_hi(v[s2][k]);
    }
  }
  if (a.win_o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += sm.omw[8 * (e >> 2) + 4 * h2 + (e & 3)] * wo[e];
  }
  const int64_t ob = ((int64_t)r * a.Hq + h0 + 16 * jj) * kDim + 64 * w + 32 * tt + l32;
  const float bad = __builtin_nanf("");
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t o = ob + (int64_t)(8 * (e >> 2) + 4 * h2 + (e & 3)) * kDim;
    const float val = ok ? acc[e] : bad;
    if (a.out_dtype == CSA2_F32) __builtin_nontemporal_store(val, static_cast<float*>(a.out) + o);
    else __builtin_nontemporal_store((uint16_t)bf16_rne(val), static_cast<uint16_t*>(a.out) + o);
  }
  // every merge workgroup of the pair has seen all S arrivals once the last one gets here
  if (tid == 0) {
    const uint64_t d = __hip_atomic_fetch_add(&a.counters[a.cstride * pair + 1], uint64_t(1), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (d == kMergeParts - 1) {
      __hip_atomic_store(&a.counters[a.cstride * pair], uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.counters[a.cstride * pair + 1], uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// MULTI: splits of more than one chunk (the next chunk's rows are gathered
// into registers while the current one is processed)
template <bool MULTI>
__global__ __launch_bounds__(kT, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_dec(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  SmemDec& sm = *reinterpret_cast<SmemDec*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;

  if (a.counters && (int)blockIdx.x >= a.nattn) {
    merge_part(a, sm);
    return;
  }
  // (pair, split): with xcd_map the S splits of one (row, head group) run on
  // one XCD (workgroups are dispatched round-robin over the 8 XCDs), so its
  // queries are read from HBM once and then hit that XCD's L2; with grp > 1
  // the other head groups of the row are there too, and the entries they
  // gather as well come from that L2
  const int S = a.splits;
  const int L = blockIdx.x;
  int pair, split;
  if (a.xcd_map) {
    const int jx = L >> 3;
    split = jx % S;
    pair = xcd_pair(jx / S, L & 7, a.grp);
  } else {
    split = L % S;
    pair = L / S;
  }
  const int nhg = a.Hq / kHG;
  const int r = pair / nhg, hg = pair % nhg;
  const int h0 = hg * kHG;
  const int kbeg = split * a.kps;
  const int kend = min(a.top_k, kbeg + a.kps);
  const int nch = kend > kbeg ? (kend - kbeg + kChunk - 1) / kChunk : 0;
  const int myslot = 32 * w + l32;  // the key this lane scores, within a chunk

  // ---- prologue: the queries, then chunk 0's indices and rows in flight
  const int hq = tid >> 4, qc0 = 32 * (tid & 15);  // thread t stages head t/16, channels [32*(t%16), +32)
  u32x4 qv[4];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.q + ((int64_t)r * a.Hq + h0 + hq) * kDim + qc0);
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = src[i];
  }
  const int vis = a.row_visible ? a.row_visible[r] : 0x7FFFFFFF;
  const int64_t rs = a.row_start[r];
  RawKey bufA, bufB;
  uint32_t vA = 0, vB = 0;
  Slots sl;
  // every split holds at least one key (kbeg < top_k), so chunk 0 is gathered without a branch: a branch
  // here would make the queries' first use wait for the gather as well
  load_slots(sl, a, r, kbeg, kend, w, lane);
  gather(bufA, a, sl, rs, vis, kbeg, kend, w, lane, vA);
  if (MULTI && nch > 1) load_slots(sl, a, r, kbeg + kChunk, kend, w, lane);
  {
    // the 16 threads of a head are 16 lanes of one wave
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) mx = max(mx, max((qv[i][k] << 16) & 0x7FFFFFFFu, qv[i][k] & 0x7FFF0000u));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    // shift sh puts the head's largest magnitude in [2^14, 2^15); 2^sh and 2^-sh are normal floats
    const int E = (int)(mx >> 23) - 127;
    const int sh = mx == 0 ? 0 : min(126, max(-126, 14 - E));
    const float up = __uint_as_float((uint32_t)(127 + sh) << 23);
    if ((tid & 15) == 0) sm.c2h[hq] = a.c2 * __uint_as_float((uint32_t)(127 - sh) << 23);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const _Float16 lo = (_Float16)(__uint_as_float(qv[i][k] << 16) * up);
        const _Float16 hi = (_Float16)(__uint_as_float(qv[i][k] & 0xFFFF0000u) * up);
        o[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<u32x4*>(&sm.q[hq * kQS + qc0 + 8 * i]) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }

  floatx16 O[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) O[t] = floatx16{};
  float m_run = -INFINITY, l_run = 0.0f;  // head l32 (replicated over the lane halves and waves)
  lds_barrier();  // queries and head scales staged; chunk 0's loads stay in flight
  const float c2h = sm.c2h[l32];

  auto chunk = [&](int c, RawKey& cur, uint32_t vcur, RawKey& nxt, uint32_t& vnxt) {
    const int kc0 = kbeg + c * kChunk;
    if (MULTI && c + 1 < nch) {
      gather(nxt, a, sl, rs, vis, kc0 + kChunk, kend, w, lane, vnxt);
      if (c + 2 < nch) load_slots(sl, a, r, kc0 + 2 * kChunk, kend, w, lane);
    }
    if (c > 0) lds_barrier();  // the previous chunk's PV reads of cs / ss / ps are done (gathers stay in flight)
    // stage the raw code rows (read back by this wave for QK^T and by every wave for PV)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(&sm.u.cs[(32 * w + 4 * i + (lane >> 4)) * kCS + 16 * (lane & 15)]) = cur.c[i];
    if (!vcur) cur.s = u32x4{0u, 0u, 0u, 0u};  // an invalid key's values are 0
    // scales of the lane's 16 groups as fp16 pairs (group 2i, 2i+1) -> stage [group][key]
    uint32_t sp[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sp[2 * i] = h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.s[i], 1.0f, false));
      sp[2 * i + 1] = h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.s[i], 1.0f, true));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t* d = reinterpret_cast<uint16_t*>(&sm.ss[(16 * h2 + 2 * i) * kSS + myslot]);
      d[0] = (uint16_t)(sp[i] & 0xFFFFu);
      d[kSS] = (uint16_t)(sp[i] >> 16);
    }
    // this lane's key row, channels [256*h2, +256), from the rows its own wave staged
    u32x4 kw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kw[j] = *reinterpret_cast<const u32x4*>(&sm.u.cs[myslot * kCS + 128 * h2 + 16 * j]);

    // ---- QK^T: S^T[key][head] over 512 channels; K-step ks covers channels 256*h2 + 8*ks .. +7.
    // Query fragments are read from LDS four K-steps ahead (the scheduling barriers keep the reads
    // where they are written); even and odd K-steps accumulate separately.
    floatx16 St0 = floatx16{}, St1 = floatx16{};
    const _Float16* qrow = &sm.q[l32 * kQS + 256 * h2];
    half8 bq[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) bq[k] = *reinterpret_cast<const half8*>(qrow + 8 * k);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      const uint32_t word = kw[ks >> 2][ks & 3];
      const uint32_t pr = sp[ks >> 2];                       // groups 4*(ks>>2) .. : pair (2i, 2i+1)
      const uint32_t sv = ((ks >> 1) & 1) ? (pr >> 16) : (pr & 0xFFFFu);
      const half2v s2 = u2h(sv | (sv << 16));
      const half8 av = cat4(h2u(fp4x2<0>(word) * s2), h2u(fp4x2<1>(word) * s2), h2u(fp4x2<2>(word) * s2),
                            h2u(fp4x2<3>(word) * s2));
      if (ks & 1) St1 = mfma32(av, bq[ks & 3], St1);
      else St0 = mfma32(av, bq[ks & 3], St0);
      if (ks + 4 < 32) bq[ks & 3] = *reinterpret_cast<const half8*>(qrow + 8 * (ks + 4));
      __builtin_amdgcn_sched_barrier(0);
    }
    const floatx16 St = St0 + St1;

    // ---- softmax over the chunk: lane holds head l32, keys 8*(i/4) + 4*h2 + i%4 of this wave
    const uint32_t vm = (uint32_t)__ballot(vcur);  // bit k: key k of this wave (lanes 0..31)
    float z[16];
    float mx = -INFINITY;
    // the logits, masked per key only when some key of the wave is invalid (a uniform branch)
    if (vm == 0xFFFFFFFFu) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        z[i] = St[i] * c2h;
        mx = fmaxf(mx, z[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * h2 + (i & 3);
        z[i] = ((vm >> key) & 1u) ? St[i] * c2h : -INFINITY;
        mx = fmaxf(mx, z[i]);
      }
    }
    mx = half_max(mx);
    if (lane < 32) sm.red_max[w][lane] = mx;
    lds_barrier();
    // half h2 of the wave takes waves 4h2 .. 4h2+3, the two halves then meet across lanes
    const float mc = half_max(fmaxf(fmaxf(sm.red_max[4 * h2][l32], sm.red_max[4 * h2 + 1][l32]),
                                    fmaxf(sm.red_max[4 * h2 + 2][l32], sm.red_max[4 * h2 + 3][l32])));
    const float m_new = fmaxf(m_run, mc);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 while nothing has been seen
    m_run = m_new;
    float sum = 0.0f;
    uint32_t pw[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const _Float16 p0 = (_Float16)__builtin_amdgcn_exp2f(z[i] - m_use);
      const _Float16 p1 = (_Float16)__builtin_amdgcn_exp2f(z[i + 1] - m_use);
      sum = __builtin_amdgcn_fdot2(half2v{p0, p1}, half2v{1.0f16, 1.0f16}, sum, false);  // p0 + p1 + sum in fp32
      pw[i >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, p0) | ((uint32_t)__builtin_bit_cast(uint16_t, p1) << 16);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<u32x2*>(&sm.ps[l32 * kPS + 32 * w + 8 * g + 4 * h2]) = u32x2{pw[2 * g], pw[2 * g + 1]};
    sum = half_sum(sum);
    if (lane < 32) sm.red_sum[w][lane] = sum;
    if (w == 0 && lane < 32) sm.alpha[lane] = alpha;
    lds_barrier();
    const float ls = half_sum((sm.red_sum[4 * h2][l32] + sm.red_sum[4 * h2 + 1][l32]) +
                              (sm.red_sum[4 * h2 + 2][l32] + sm.red_sum[4 * h2 + 3][l32]));  // same bits in both halves
    l_run = l_run * alpha + ls;

    // ---- PV: O[head][channel] for channels [64w, 64w+64), two 32-channel tiles
    if (c > 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 al = *reinterpret_cast<const floatx4*>(&sm.alpha[8 * g + 4 * h2]);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) O[t][4 * g + e] *= al[e];
      }
    }
    const int lg = (lane >> 4) & 1;  // which 16 channels of the 32-channel tile this lane converts
    // operands of 32 keys: two transposed code reads, their scales, the probabilities of two K-steps;
    // the next 32 keys' are read while the current ones are converted and multiplied
    struct PvIn {
      i32x2 tr[2];
      u32x4 sc[2][2];
      half8 ap[2];
    };
    auto pv_load = [&](PvIn& in, int kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint8_t* p = &sm.u.cs[(kb + 16 * h2 + (lane & 15)) * kCS + 32 * w + 16 * t + 8 * lg];
        in.tr[t] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(const_cast<uint8_t*>(p)));
        const _Float16* sg = &sm.ss[(4 * w + 2 * t + lg) * kSS + kb + 16 * h2];
        in.sc[t][0] = *reinterpret_cast<const u32x4*>(sg);
        in.sc[t][1] = *reinterpret_cast<const u32x4*>(sg + 8);
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
        in.ap[sub] = *reinterpret_cast<const half8*>(&sm.ps[l32 * kPS + kb + 16 * h2 + 8 * sub]);
    };
    PvIn pin[2];
    pv_load(pin[0], 0);
#pragma unroll
    for (int t8 = 0; t8 < kChunk / 32; ++t8) {
      if (t8 + 1 < kChunk / 32) pv_load(pin[(t8 + 1) & 1], 32 * (t8 + 1));
      __builtin_amdgcn_sched_barrier(0);
      const PvIn& in = pin[t8 & 1];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t word = (uint32_t)in.tr[t][sub];
          const u32x4 s4 = in.sc[t][sub];
          const half8 bv = cat4(h2u(fp4x2<0>(word) * u2h(s4[0])), h2u(fp4x2<1>(word) * u2h(s4[1])),
                                h2u(fp4x2<2>(word) * u2h(s4[2])), h2u(fp4x2<3>(word) * u2h(s4[3])));
          O[t] = mfma32(in.ap[sub], bv, O[t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (MULTI) {
    for (int c = 0; c < nch; ++c) {
      chunk(c, bufA, vA, bufB, vB);
      bufA = bufB;  // the next chunk's registers (moves)
      vA = vB;
    }
  } else if (nch > 0) {
    chunk(0, bufA, vA, bufB, vB);
  }

  // ---- epilogue: lane holds O[head 8*(i/4) + 4*h2 + i%4][channel 64w + 32t + l32]; every lane
  // knows its head l32's (max, sum); one reciprocal per head, shared through LDS
  if (w == 0 && lane < 32) sm.ifin[lane] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  lds_barrier();
  float inv[16];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const floatx4 iv = *reinterpret_cast<const floatx4*>(&sm.ifin[8 * g + 4 * h2]);
#pragma unroll
    for (int e = 0; e < 4; ++e) inv[4 * g + e] = iv[e];
  }

  if (S == 1) {
    // one split: the output directly
    const int64_t ob = ((int64_t)r * a.Hq + h0) * kDim + 64 * w + l32;
    if (a.out_dtype == CSA2_F32) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          __builtin_nontemporal_store(O[t][i] * inv[i],
                                      static_cast<float*>(a.out) + ob + (8 * (i >> 2) + 4 * h2 + (i & 3)) * kDim + 32 * t);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          static_cast<uint16_t*>(a.out)[ob + (8 * (i >> 2) + 4 * h2 + (i & 3)) * kDim + 32 * t] =
              (uint16_t)bf16_rne(O[t][i] * inv[i]);
    }
    if (a.lse && w == 0 && lane < 32)
      a.lse[(int64_t)r * a.Hq + h0 + lane] = l_run > 0.0f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    return;
  }

  // ---- split partial: the lane's 32 normalized outputs in fp16, in accumulator order: piece p = 2t + j
  // of every lane of the wave is one contiguous KiB (each store instruction writes whole lines)
  const size_t pbase = (size_t)pair * S + split;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(a.ws_o, 0, 0x7FFFFFFF, 0x00020000);
  const uint32_t pofs = (uint32_t)(((pbase * 8 + w) * 256 + lane) * 16);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = 8 * j + 2 * k;
        pk[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[t][i] * inv[i])) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(O[t][i + 1] * inv[i + 1])) << 16);
      }
      // device-scope stores (written through to memory, the line kept in this XCD's L2): the merge reads
      // them back from L2, and the kernel does not end with 8 MB of them dirty in L2
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{pk[0], pk[1], pk[2], pk[3]}, rw,
                                             (int)(pofs + 1024u * (uint32_t)(2 * t + j)), 0, 16);
    }
  if (w == 0 && lane < 32)
    *reinterpret_cast<float2*>(a.ws_ml + (((size_t)pair * kHG + lane) * S + split) * 2) = make_float2(m_run, l_run);
  if (!a.counters) return;
  // arrival, once this workgroup's stores have reached L2: the count and this XCC's field
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    __hip_atomic_fetch_add(&a.counters[a.cstride * pair], uint64_t(1) | (uint64_t(1) << (8 + 4 * xcc_id())),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The merge of the key splits: one workgroup of 256 threads per (row, head
// group, wave of the attention workgroup).  The weights of the splits of
// each head (w_s = 2^(m_s - M) l_s / sum) come first, in fixed split order;
// then thread (j, lane) merges 16 bytes of that lane's partial (8 heads of
// one channel) over the splits, every split's load issued before any use,
// and the merged outputs go out in head-major order through LDS.
__global__ __launch_bounds__(256) void k_dec_combine(DecArgs a) {
  __shared__ float om[kHG][kMaxSplits];
  const int pair = blockIdx.x >> 3, w = blockIdx.x & 7;
  const int t = threadIdx.x, lane = t & 63, j = t >> 6;
  const int S = a.splits;
  const int nhg = a.Hq / kHG;
  const int r = pair / nhg, h0 = (pair % nhg) * kHG;
  // partial loads first: lane's 16-byte piece j (tile j>>1, accumulator rows 8*(j&1) .. +7)
  u32x4 v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const size_t pb = (size_t)pair * S + (s < S ? s : 0);
    v[s] = reinterpret_cast<const u32x4*>(a.ws_o)[(pb * 8 + w) * 256 + t];
  }
  // weights of the splits of each head, in fixed split order
  __shared__ float2 mls[kHG * kMaxSplits];
  if (t < kHG * S) mls[t] = reinterpret_cast<const float2*>(a.ws_ml)[(size_t)pair * kHG * S + t];
  __syncthreads();
  if (t < kHG) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, mls[t * S + s].x);
    float wg[kMaxSplits], L = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      wg[s] = (s < S && M != -INFINITY) ? __builtin_amdgcn_exp2f(mls[t * S + s].x - M) * mls[t * S + s].y : 0.0f;
      L += wg[s];
    }
    const float iL = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) om[t][s] = wg[s] * iL;
    if (a.lse && w == 0) a.lse[(int64_t)r * a.Hq + h0 + t] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const int h2 = lane >> 5, l32 = lane & 31, tt = j >> 1;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s >= S) break;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i0 = 8 * (j & 1) + 2 * k;  // accumulator rows i0, i0 + 1
      acc[2 * k] += om[8 * (i0 >> 2) + 4 * h2 + (i0 & 3)][s] * h_lo(v[s][k]);
      acc[2 * k + 1] += om[8 * ((i0 + 1) >> 2) + 4 * h2 + ((i0 + 1) & 3)][s] * h_hi(v[s][k]);
    }
  }
  // through LDS to head-major order: 32 heads x 64 channels, then 32 contiguous bytes per thread
  __shared__ float ot[kHG][64 + 4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = 8 * (j & 1) + e;
    ot[8 * (i >> 2) + 4 * h2 + (i & 3)][32 * tt + l32] = acc[e];
  }
  __syncthreads();
  const int oh = t >> 3, oc = 8 * (t & 7);
  const int64_t o = ((int64_t)r * a.Hq + h0 + oh) * kDim + 64 * w + oc;
  const floatx4 v0 = *reinterpret_cast<const floatx4*>(&ot[oh][oc]), v1 = *reinterpret_cast<const floatx4*>(&ot[oh][oc + 4]);
  if (a.out_dtype == CSA2_F32) {
    reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + o)[0] = v0;
    reinterpret_cast<floatx4*>(static_cast<float*>(a.out) + o)[1] = v1;
  } else {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + o) =
        u32x4{bf16_rne(v0[0]) | (bf16_rne(v0[1]) << 16), bf16_rne(v0[2]) | (bf16_rne(v0[3]) << 16),
              bf16_rne(v1[0]) | (bf16_rne(v1[1]) << 16), bf16_rne(v1[2]) | (bf16_rne(v1[3]) << 16)};
  }
}

struct DecPlan {
  int pairs, splits, kps;
  bool xcd;
};

// Key splits so that about 256 workgroups run: (row, 32-head group) pairs x
// splits, at most one split per 256-key chunk and at most kMaxSplits.
DecPlan dec_plan(int R, int Hq, int top_k) {
  DecPlan p{};
  p.pairs = R * (Hq / kHG);
  const int max_chunks = (int)ceil_div(top_k, kChunk);
  int s = (int)std::min<int64_t>(std::min(max_chunks, kMaxSplits), std::max<int64_t>(1, ceil_div(256, p.pairs)));
  p.kps = (int)round_up(ceil_div(top_k, s), kChunk);
  p.splits = (int)ceil_div(top_k, p.kps);
  p.xcd = p.splits > 1 && p.pairs % 8 == 0;
  return p;
}

}  // namespace

bool attn_dec_applies(int R, int Hq, int q_dtype, int top_k, bool window) {
  if (q_dtype != CSA2_BF16 || Hq % kHG != 0 || top_k < 1) return false;
  const int64_t pairs = (int64_t)R * (Hq / kHG);
  // rows x 64-head groups that fill the chip take the 64-head prefill kernel
  if ((Hq / 16) % 4 == 0 && (int64_t)R * (Hq / 64) >= 256) return false;
  if (pairs > kMaxPairs) return false;
  if (!window) return true;
  // a window joins as one more term of the in-launch merge, so only plans that merge in the launch take it
  const DecPlan p = dec_plan(R, Hq, top_k);
  return p.splits > 1 && p.xcd;
}

size_t attn_dec_window_bytes(int R, int Hq) {
  const size_t n = (size_t)R * Hq * 2;
  return round_up(n * kDim * 4, 256) + 2 * round_up(n * 4, 256);
}

size_t attn_dec_workspace_bytes(int R, int Hq, int top_k, bool window) {
  const DecPlan p = dec_plan(R, Hq, top_k);
  if (p.splits <= 1) return 0;
  const size_t n = (size_t)p.pairs * p.splits;
  return kAttnCounterBytes + round_up(n * kHG * 512 * 2, 256) + round_up(n * kHG * 8, 256) +
         (window ? attn_dec_window_bytes(R, Hq) : 0);
}

hipError_t launch_attn_dec(int R, const void* q, int Hq, const uint8_t* codes, const uint8_t* scales,
                           const int64_t* row_start, const int32_t* idx, int top_k, const int32_t* row_visible,
                           float softmax_scale, void* out, int out_dtype, float* lse, const float* win_o,
                           const float* win_m, const float* win_l, void* ws, hipStream_t s) {
  const DecPlan p = dec_plan(R, Hq, top_k);
  if (win_o && !(p.splits > 1 && p.xcd)) return hipErrorInvalidValue;  // only the in-launch merge takes a window
  DecArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.Hq = Hq;
  a.codes = codes;
  a.scales = scales;
  a.row_start = row_start;
  a.idx = idx;
  a.top_k = top_k;
  a.row_visible = row_visible;
  a.c2 = softmax_scale * kLog2e;
  a.out = out;
  a.out_dtype = out_dtype;
  a.lse = lse;
  a.win_o = win_o;
  a.win_m = win_m;
  a.win_l = win_l;
  a.splits = p.splits;
  a.kps = p.kps;
  a.xcd_map = p.xcd ? 1 : 0;
  a.grp = R % 8 == 0 ? Hq / kHG : 1;
  a.nattn = p.pairs * p.splits;
  int nmerge = 0;
  if (p.splits > 1) {
    const size_t n = (size_t)p.pairs * p.splits;
    char* b = static_cast<char*>(ws);
    if (p.xcd) {
      a.counters = reinterpret_cast<uint64_t*>(b);
      // each pair's counters on a line of their own when the pairs allow it (the arrivals and polls of
      // different pairs then do not queue on one line), else packed down to 16 bytes
      a.cstride = std::max(2, std::min(16, (int)(kAttnCounterBytes / 8) / p.pairs));
      nmerge = kMergeParts * p.pairs;
    }
    a.ws_o = reinterpret_cast<_Float16*>(b + kAttnCounterBytes);
    a.ws_ml = reinterpret_cast<float*>(b + kAttnCounterBytes + round_up(n * kHG * 512 * 2, 256));
  }
  const bool multi = p.kps > kChunk;
  auto kern = multi ? k_attn_dec<true> : k_attn_dec<false>;
  static bool configured[2] = {false, false};
  if (!configured[multi]) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sizeof(SmemDec));
    configured[multi] = true;
  }
  auto& ev = profile_events(CSA2_KERNEL_ATTN);
  if (ev.start) (void)hipEventRecord(ev.start, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.nattn + nmerge)), dim3(kT), sizeof(SmemDec), s, a);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits <= 1 || a.counters) return e;
  auto& ec = profile_events(CSA2_KERNEL_ATTN_COMBINE);
  if (ec.start) (void)hipEventRecord(ec.start, s);
  hipLaunchKernelGGL(k_dec_combine, dim3((unsigned)(p.pairs * 8)), dim3(256), 0, s, a);
  if (ec.stop) (void)hipEventRecord(ec.stop, s);
  return hipGetLastError();
}

}  // namespace csa2
