// k_attn.hip -- gather + FP4 dequant + online-softmax sparse attention on
// gfx950 MFMA, with a deterministic split-K combine.
//
// What it computes ("The Paper" in the talk write-up "DeepSeek V4.1 Flash:
// pushing the limits": K and V are the same Main KV entry; "The global
// branch" in the course brief "DeepSeek-V4.1-Flash": one 512-dim latent per
// entry shared by all query heads): for a row r and head h, softmax over the
// selected entries of softmax_scale * q . x_hat, then the weighted sum of the
// x_hat.  x_hat = E2M1 code * E4M3 scale is exact in fp16, so both products
// run on fp16 MFMA (v_mfma_f32_16x16x32_f16, fp32 accumulate): bf16 queries
// convert to fp16 exactly; fp32 queries are split into hi + lo fp16 halves.
// Probabilities are rounded to fp16 for the PV product and the row sums add
// up those same rounded values.
//
// Work split.  A workgroup (8 waves, two per SIMD so that one wave's memory,
// LDS and exp latency overlaps the other's math) owns one (row, group of
// 16*NHT heads, key split) and walks its keys in steps of 128:
//  * QK^T, keys split across waves: wave w takes keys [16w, 16w+16) of the
//    step and every head of the group.  Its lanes load their key's 288-byte
//    row straight from HBM into registers (prefetched a whole step ahead)
//    and dequantize it into the A operand (key rows); queries sit in LDS as
//    the B operand.  The result S^T gives each lane 4 keys of one head.
//  * softmax: per-wave maxima and sums meet in LDS (lane reductions use
//    permlane swaps).  The reference maximum of a head only moves when the
//    new maximum exceeds it by more than 2^8, so the running output is
//    rarely rescaled; the final division by the same-reference sum makes
//    the result independent of that choice.
//  * PV, output channels and key halves split across waves: wave w produces
//    channels [128(w%4), +128) of every head over keys [64(w/4), +64) of the
//    step, from raw codes staged in LDS.  A lane owns 8 consecutive
//    channels; nibbles of two keys are interleaved with bit operations so
//    that each converted fp16 pair holds two keys of one channel (the
//    K-contiguous B operand layout), and all 8 channels share one scale
//    pair.  The two key halves are summed through LDS at the end.
// Every FP4 element is dequantized once for QK^T and once for PV per
// workgroup.  The split partials total rows x heads x splits x 512 fp32, so
// the launch plan trades head tiles per workgroup against key splits.
#include <type_traits>

#include "csa2_common.h"

namespace csa2 {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kStep = 128;           // keys per step (16 per wave in QK^T)
constexpr int kCsStride = 272;       // bytes per staged code row (256 + 16 pad)
constexpr int kScStride = 136;       // fp16 per staged scale row (128 keys + 8 pad)
constexpr int kPStride = 136;        // fp16 per probability row
constexpr int kQStride = 520;        // fp16 per query row (512 + 8 pad)
constexpr int kOStride = 516;        // fp32 per row of the epilogue reduction buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;        // log2 headroom before the reference maximum moves
constexpr int kWinMax = 128;         // local window entries per row
constexpr int kWStride = 520;        // bytes per staged window entry: entries 8 apart land 16 banks apart

__device__ __forceinline__ uint32_t h2_bits(half2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2v bits_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// two E2M1 codes (byte SEL of w: low nibble first) -> two fp16 values
template <int SEL>
__device__ __forceinline__ half2v fp4x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// two E4M3 bytes (half SEL of w) -> two fp16 values
template <bool SEL>
__device__ __forceinline__ half2v e4m3x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, SEL);
}

__device__ __forceinline__ floatx4 mfma(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 cat4(half2v a, half2v b, half2v c, half2v d) {
  return __builtin_bit_cast(half8, u32x4{h2_bits(a), h2_bits(b), h2_bits(c), h2_bits(d)});
}

struct AttnArgs {
  const void* q;
  int Hq;
  const uint8_t* codes;
  const uint8_t* scales;
  const int64_t* row_start;
  const int32_t* idx;
  int top_k;
  const int32_t* row_visible;
  float c2;              // softmax_scale * log2(e)
  void* out;
  int out_dtype;
  float* lse;
  int slots;             // partials per (row, head): key splits (+1 for the window); 1 = write out directly
  int keys_per_split;    // multiple of kStep
  float* ws_o;           // [R, Hq, slots, 512] partial outputs, normalized
  float* ws_m;           // [R, Hq, slots] reference maxima (log2 units)
  float* ws_l;           // [R, Hq, slots] sums
  uint8_t* win;              // local window entries [*, 512] signed E4M3 bytes (written only with new_x)
  const int64_t* win_start;  // [R] first window entry of each row
  const int32_t* win_len;    // [R] window entries of each row (clamped to [0, kWinMax])
  const void* new_x;         // optional: row r's newest token [R][new_x_stride] of new_x_dtype ...
  int new_x_dtype;
  int64_t new_x_stride;
  const int64_t* new_rows;   // ... written to window row new_rows[r] (< 0: none) by this call
};

// Row r's newest window token, written by the attention call itself (one launch
// fewer per layer in decode, where every row has its own window).  Before a
// workgroup barrier every thread encodes one channel of x[r] as signed E4M3 (as
// the FP8 quantize call does) into a 512-byte LDS row, and workgroups of head
// group 0 store it to the window; after the barrier the 4 lanes (q4 = 0..3) of
// the entry slot the token occupies in the row's window take their 128 bytes
// from LDS in place of the ones they loaded, which may predate the write.
__device__ __forceinline__ void encode_fresh(const AttnArgs& a, int r, int hg, uint8_t* fresh) {
  const int64_t dst = a.new_rows[r];
  if (dst < 0) return;
  const int t = threadIdx.x;  // one channel per thread (512 threads)
  const uint32_t u = a.new_x_dtype == CSA2_F32
                         ? __float_as_uint(static_cast<const float*>(a.new_x)[r * a.new_x_stride + t])
                         : (uint32_t)static_cast<const uint16_t*>(a.new_x)[r * a.new_x_stride + t] << 16;
  const uint8_t b = (uint8_t)(e4m3_code(__uint_as_float(u & 0x7FFFFFFFu)) | ((u >> 24) & 0x80u));
  fresh[t] = b;
  if (hg == 0) a.win[dst * kDim + t] = b;
}

// after the barrier: true if this lane's entry is the fresh one (its c[] now holds it)
__device__ __forceinline__ bool take_fresh(const AttnArgs& a, int r, int key, int len, int q4, const uint8_t* fresh,
                                           u32x4 (&c)[8]) {
  const int64_t dst = a.new_rows[r];
  if (dst < 0 || dst - a.win_start[r] != key || key >= len) return false;
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = *reinterpret_cast<const u32x4*>(fresh + 128 * q4 + 16 * i);
  return true;
}

// byte offset of staged code row k.  Rows are padded to 272 bytes and each
// group of 8 rows inside a 32-row block is shifted by another 64 bytes, so
// the rows 8 apart that one PV k-group reads land 16 banks apart.
constexpr int kCsBlock = 32 * kCsStride + 3 * 64;
__device__ __forceinline__ int cs_off(int k) {
  return (k >> 5) * kCsBlock + (k & 31) * kCsStride + 64 * ((k >> 3) & 3);
}

// Staged operands, probabilities and per-wave maxima and sums are double
// buffered by step parity: a wave writes those of step s+1 before the one
// barrier of that step, while slower waves may still read those of step s.
template <int NHT, bool SPLITQ>
struct Smem {
  static constexpr int kQRows = 16 * NHT * (SPLITQ ? 2 : 1);
  union {
    struct {
      _Float16 q[kQRows * kQStride];
      uint8_t cs[2][(kStep / 32) * kCsBlock];
      _Float16 sct[2][kGroups * kScStride];
      _Float16 p[2][16 * NHT * kPStride];
    } s;
    float ored[16 * NHT * kOStride];  // after the key loop: outputs of the second key half
  } u;
  float red_max[2][kWaves][64];
  float red_sum[2][kWaves][64];
  float alpha[64];
  float lfin[64];
};

// lane reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// byte permute: bytes of {hi:lo} picked by the four selector bytes (0..3 = lo, 4..7 = hi)
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

struct Raw {
  u32x4 c[4];  // code bytes [64*q4, 64*q4+64) of the lane's key
  u32x2 s;     // scale bytes [8*q4, 8*q4+8)
};

// Branch-free gather: an invalid key loads row 0 of the cache (always
// present) and is masked before use (mask_raw), so every load is issued
// unconditionally and the compiler keeps them all in flight.
__device__ __forceinline__ void load_raw(Raw& R, const AttnArgs& a, int64_t rs, int vis, int32_t j, int i,
                                         int kend, uint32_t& valid, int q4) {
  const bool ok = (i < kend) & ((uint32_t)j < (uint32_t)vis);
  valid = ok;
  const int64_t row = ok ? rs + j : 0;
  const u32x4* pc = reinterpret_cast<const u32x4*>(a.codes + row * kCodeBytes + 64 * q4);
#pragma unroll
  for (int c = 0; c < 4; ++c) R.c[c] = pc[c];
  R.s = *reinterpret_cast<const u32x2*>(a.scales + row * kGroups + 8 * q4);
}

// An invalid key's scales are zeroed, so its dequantized values are 0 in PV
// (its codes are finite E2M1 values whatever row was read; its logits are
// masked separately).
__device__ __forceinline__ void mask_raw(Raw& R, uint32_t valid) {
  R.s[0] = valid ? R.s[0] : 0u;
  R.s[1] = valid ? R.s[1] : 0u;
}

// index stored in key slot i of row r, clamped to the split's last slot
// (kend > kbeg >= 0).  Slots >= kend are rejected later by load_raw; the
// loaded value is not inspected here, so the load can stay in flight.
__device__ __forceinline__ int32_t load_idx(const AttnArgs& a, int r, int i, int kend) {
  return a.idx[(int64_t)r * a.top_k + (i < kend ? i : kend - 1)];
}

template <int NHT, bool SPLITQ, int QDT>
__global__ __launch_bounds__(kThreads, 1) void k_sparse_attn(AttnArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem<NHT, SPLITQ>& sm = *reinterpret_cast<Smem<NHT, SPLITQ>*>(smem_raw);
  auto& ss = sm.u.s;
  constexpr int HG = 16 * NHT;
  constexpr int NQ = SPLITQ ? 2 : 1;
  constexpr bool kFastSoftmax = NHT == 2;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int cq = w & 3, kh = w >> 2;  // PV role: channel quarter, key half
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int h0 = hg * HG;
  const int kbeg = split * a.keys_per_split;
  const int kend = min(a.top_k, kbeg + a.keys_per_split);
  const int nsteps = kend > kbeg ? (kend - kbeg + kStep - 1) / kStep : 0;
  const int vis = a.row_visible ? a.row_visible[r] : 0x7FFFFFFF;
  const int64_t rs = a.row_start[r];
  const int myslot = 16 * w + n16;  // this lane's key within a step (QK^T role)

  // ---- prologue: indices of steps 0 and 1, the keys of step 0 in flight, queries to LDS.
  // Every load below and in the step prefetch is unconditional: slots past
  // the split end read the split's last index slot and the gather then
  // reads cache row 0, so no branch makes the compiler wait for loads early.
  uint32_t vA = 0, vB = 0;
  Raw bufA, bufB;
  const int32_t j0 = load_idx(a, r, kbeg + myslot, kend);
  int32_t jn = load_idx(a, r, kbeg + kStep + myslot, kend);
  load_raw(bufA, a, rs, vis, j0, kbeg + myslot, kend, vA, q4);
  {
    // HG heads x 512 channels in 16-byte pieces; all loads issued before any conversion
    if (QDT == CSA2_BF16) {
      constexpr int NP = HG * kDim / 8 / kThreads;  // pieces per thread
      const uint16_t* qb = static_cast<const uint16_t*>(a.q) + ((int64_t)r * a.Hq + h0) * kDim;
      u32x4 v[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int p = tid + kThreads * i;
        v[i] = *reinterpret_cast<const u32x4*>(qb + (int64_t)(p / (kDim / 8)) * kDim + (p % (kDim / 8)) * 8);
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int p = tid + kThreads * i;
        half8 hv;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hv[2 * k] = (_Float16)__uint_as_float(v[i][k] << 16);
          hv[2 * k + 1] = (_Float16)__uint_as_float(v[i][k] & 0xFFFF0000u);
        }
        *reinterpret_cast<half8*>(&ss.q[(p / (kDim / 8)) * kQStride + (p % (kDim / 8)) * 8]) = hv;
      }
    } else {
      constexpr int NP = HG * kDim / 4 / kThreads;
      const float* qf = static_cast<const float*>(a.q) + ((int64_t)r * a.Hq + h0) * kDim;
      floatx4 v[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int p = tid + kThreads * i;
        v[i] = *reinterpret_cast<const floatx4*>(qf + (int64_t)(p / (kDim / 4)) * kDim + (p % (kDim / 4)) * 4);
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int p = tid + kThreads * i;
        const int h = p / (kDim / 4), c4 = (p % (kDim / 4)) * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const _Float16 hi = (_Float16)v[i][k];
          ss.q[h * kQStride + c4 + k] = hi;
          if (SPLITQ) ss.q[(HG + h) * kQStride + c4 + k] = (_Float16)(v[i][k] - (float)hi);
        }
      }
    }
  }
  __syncthreads();

  floatx4 O[NHT][8];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int t = 0; t < 8; ++t) O[ht][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mref[NHT], lrun[NHT];  // per head 16*ht + n16 (softmax role), replicated over q4 and waves
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    mref[ht] = -INFINITY;
    lrun[ht] = 0.0f;
  }

  // One step over keys [kstep0, kstep0+128) held in `cur`; at its start the
  // gather of the next step is issued into `nxt` (a whole step ahead) and the
  // index of the step after that is loaded (past the end: harmless in-bounds
  // loads whose keys are masked).
  auto step = [&](int st, Raw& cur, uint32_t vcur, Raw& nxt, uint32_t& vnxt) {
    const int kstep0 = kbeg + st * kStep;
    load_raw(nxt, a, rs, vis, jn, kstep0 + kStep + myslot, kend, vnxt, q4);
    jn = load_idx(a, r, kstep0 + 2 * kStep + myslot, kend);
    mask_raw(cur, vcur);
    // scale bytes of groups 8*q4 .. 8*q4+7 -> fp16
    half2v sc[4];
    sc[0] = e4m3x2_to_h2<false>(cur.s[0]);
    sc[1] = e4m3x2_to_h2<true>(cur.s[0]);
    sc[2] = e4m3x2_to_h2<false>(cur.s[1]);
    sc[3] = e4m3x2_to_h2<true>(cur.s[1]);

    // ---- QK^T: S^T[key][head] for this wave's 16 keys
    floatx4 S[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) S[ht] = floatx4{0.f, 0.f, 0.f, 0.f};
    // query fragments are read from LDS two K-steps ahead of their use
    constexpr int NB = NHT * NQ;
    half8 bq[3][NB];
    auto load_bq = [&](half8* dst, int ks) {
#pragma unroll
      for (int ht = 0; ht < NB; ++ht)
        dst[ht] = *reinterpret_cast<const half8*>(&ss.q[(16 * ht + n16) * kQStride + 128 * q4 + 8 * ks]);
    };
    load_bq(bq[0], 0);
    load_bq(bq[1], 1);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      // K-step ks covers channels 128*q4 + 8*ks .. +7 on both operands
      if (ks + 2 < 16) load_bq(bq[(ks + 2) % 3], ks + 2);
      const uint32_t word = cur.c[ks >> 2][ks & 3];
      const half2v s1 = sc[ks >> 2];
      const half2v sv = (ks & 2) ? __builtin_shufflevector(s1, s1, 1, 1) : __builtin_shufflevector(s1, s1, 0, 0);
      const half8 av = cat4(fp4x2_to_h2<0>(word) * sv, fp4x2_to_h2<1>(word) * sv, fp4x2_to_h2<2>(word) * sv,
                            fp4x2_to_h2<3>(word) * sv);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        S[ht] = mfma(av, bq[ks % 3][ht], S[ht]);
        if (SPLITQ) S[ht] = mfma(av, bq[ks % 3][NHT + ht], S[ht]);
      }
    }

    // ---- softmax.  The reference maximum of each head is kept lazily: it
    // only moves when a new maximum exceeds it by more than 2^kLazy.
    // Two-tile workgroups (long key loops) first take the probabilities
    // against the current references and publish them with the per-wave
    // maxima and sums behind one barrier; every wave reads the same maxima
    // and takes the same decision: if a reference has to move (always at the
    // first step with a valid key), the probabilities are recomputed behind
    // a second barrier.  One-tile workgroups (short key loops, where that
    // first attempt rarely pays) exchange the maxima first.  Both give the
    // same probabilities.  Staged data are double buffered by step parity
    // in the first scheme, since a wave writes those of step s+1 before its
    // barrier while slower waves may still read those of step s.
    const int pb = kFastSoftmax ? (st & 1) : 0;
    const unsigned long long vm = __ballot(vcur);
    float mx[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      mx[ht] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (vm >> (4 * q4 + i)) & 1ull;
        const float z = ok ? S[ht][i] * a.c2 : -INFINITY;
        S[ht][i] = z;
        mx[ht] = fmaxf(mx[ht], z);
      }
      mx[ht] = rows_max(mx[ht]);
    }
    // probabilities of this wave's keys against the references muse; sums to red_sum
    auto probs = [&](int ht, float muse) {
      const int h = 16 * ht + n16;
      _Float16 pv[4];
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = (_Float16)__builtin_amdgcn_exp2f(S[ht][i] - muse);
        sum += (float)pv[i];
      }
      *reinterpret_cast<u32x2*>(&ss.p[pb][h * kPStride + 16 * w + 4 * q4]) =
          u32x2{h2_bits(half2v{pv[0], pv[1]}), h2_bits(half2v{pv[2], pv[3]})};
      sum = rows_sum(sum);
      if (q4 == 0) sm.red_sum[pb][w][h] = sum;
    };
    auto stage = [&]() {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4*>(&ss.cs[pb][cs_off(myslot) + 64 * q4 + 16 * c]) = cur.c[c];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ss.sct[pb][(8 * q4 + 2 * g) * kScStride + myslot] = sc[g][0];
        ss.sct[pb][(8 * q4 + 2 * g + 1) * kScStride + myslot] = sc[g][1];
      }
    };
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      if (kFastSoftmax) probs(ht, mref[ht] == -INFINITY ? 0.0f : mref[ht]);
      if (q4 == 0) sm.red_max[pb][w][16 * ht + n16] = mx[ht];
    }
    if (kFastSoftmax) stage();
    lds_barrier();  // B1: maxima (and, first scheme, probabilities, sums, staged codes) visible;
                    // every wave is past the PV of the previous step
    if (!kFastSoftmax) stage();

    float mstep[NHT];
    bool move = false;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      mstep[ht] = sm.red_max[pb][0][h];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) mstep[ht] = fmaxf(mstep[ht], sm.red_max[pb][ww][h]);
      move |= mstep[ht] > mref[ht] + kLazy;  // (true for any valid key while the reference is -inf)
    }
    const bool slow = !kFastSoftmax || __ballot(move) != 0ull;  // the same in every wave
    float alpha[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) alpha[ht] = 1.0f;
    if (slow) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const int h = 16 * ht + n16;
        const float mnew = (mstep[ht] > mref[ht] + kLazy) ? mstep[ht] : mref[ht];
        const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
        alpha[ht] = (mnew == mref[ht]) ? 1.0f : __builtin_amdgcn_exp2f(mref[ht] - muse);
        mref[ht] = mnew;
        probs(ht, muse);
        if (q4 == 0 && w == 0) sm.alpha[h] = alpha[ht];
      }
      lds_barrier();  // B2: probabilities, sums, alpha (and, second scheme, staged codes) visible
    }

#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      float add = sm.red_sum[pb][0][h];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) add += sm.red_sum[pb][ww][h];
      lrun[ht] = lrun[ht] * alpha[ht] + add;
    }

    // ---- PV: channels 128*cq + 8*n16 + t (t = 0..7) of every head over keys [64kh, 64kh+64);
    // rescale only when a reference moved
    if (slow && st > 0) {
      float al[NHT][4];
      bool moved = false;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          al[ht][i] = sm.alpha[16 * ht + 4 * q4 + i];
          moved |= al[ht][i] != 1.0f;
        }
      if (__ballot(moved)) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 8; ++t) O[ht][t][i] *= al[ht][i];
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int key0 = 64 * kh + 32 * kk + 8 * q4;  // this lane's 8 keys (k-slots 0..7)
      // channels 128*cq + 8*n16 .. +7: one 32-bit code word per key
      uint32_t W[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        W[k] = *reinterpret_cast<const uint32_t*>(&ss.cs[pb][cs_off(key0 + k) + 64 * cq + 4 * n16]);
      // the 8 channels share scale group 8*cq + n16/2
      const u32x4 spw = *reinterpret_cast<const u32x4*>(&ss.sct[pb][(8 * cq + (n16 >> 1)) * kScStride + key0]);
      // byte b of E[p]: channel 2b of keys (2p, 2p+1); byte b of D[p]: channel 2b+1
      uint32_t E[4], D[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t wa = W[2 * p], wb = W[2 * p + 1];
        E[p] = (wa & 0x0F0F0F0Fu) | ((wb << 4) & 0xF0F0F0F0u);
        D[p] = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);
      }
      half8 av[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        av[ht] = *reinterpret_cast<const half8*>(&ss.p[pb][(16 * ht + n16) * kPStride + key0]);
      // tile t (channel 128*cq + 8*n16 + t) is converted just before its products
      auto tile = [&](auto sel_c, const uint32_t(&src)[4], int t) {
        constexpr int SEL = decltype(sel_c)::value;
        u32x4 b;
#pragma unroll
        for (int p = 0; p < 4; ++p) b[p] = h2_bits(fp4x2_to_h2<SEL>(src[p]) * bits_h2(spw[p]));
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) O[ht][t] = mfma(av[ht], __builtin_bit_cast(half8, b), O[ht][t]);
      };
      tile(std::integral_constant<int, 0>{}, E, 0);
      tile(std::integral_constant<int, 0>{}, D, 1);
      tile(std::integral_constant<int, 1>{}, E, 2);
      tile(std::integral_constant<int, 1>{}, D, 3);
      tile(std::integral_constant<int, 2>{}, E, 4);
      tile(std::integral_constant<int, 2>{}, D, 5);
      tile(std::integral_constant<int, 3>{}, E, 6);
      tile(std::integral_constant<int, 3>{}, D, 7);
    }
  };
  for (int st = 0; st < nsteps; st += 2) {
    step(st, bufA, vA, bufB, vB);
    if (st + 1 < nsteps) step(st + 1, bufB, vB, bufA, vA);
  }

  // ---- epilogue: the second key half hands its outputs over through LDS
  __syncthreads();  // every wave is past its last PV: the staging area is free
  const int ch = 128 * cq + 8 * n16;
  if (kh == 1) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4* dst = reinterpret_cast<float4*>(&sm.u.ored[(16 * ht + 4 * q4 + i) * kOStride + ch]);
        dst[0] = make_float4(O[ht][0][i], O[ht][1][i], O[ht][2][i], O[ht][3][i]);
        dst[1] = make_float4(O[ht][4][i], O[ht][5][i], O[ht][6][i], O[ht][7][i]);
      }
  }
  if (w == 0 && q4 == 0) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) sm.lfin[16 * ht + n16] = lrun[ht];
  }
  __syncthreads();
  if (kh == 0) {
    const int64_t rowh = (int64_t)r * a.Hq + h0;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * ht + 4 * q4 + i;
        const float L = sm.lfin[h];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const float4* src = reinterpret_cast<const float4*>(&sm.u.ored[h * kOStride + ch]);
        const float4 o0 = src[0], o1 = src[1];
        float v[8] = {O[ht][0][i] + o0.x, O[ht][1][i] + o0.y, O[ht][2][i] + o0.z, O[ht][3][i] + o0.w,
                      O[ht][4][i] + o1.x, O[ht][5][i] + o1.y, O[ht][6][i] + o1.z, O[ht][7][i] + o1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] *= inv;
        if (a.slots > 1) {
          // streaming stores: the partials are read once, by the combine kernel
          floatx4* dst = reinterpret_cast<floatx4*>(a.ws_o + ((rowh + h) * a.slots + split) * kDim + ch);
          __builtin_nontemporal_store(floatx4{v[0], v[1], v[2], v[3]}, dst);
          __builtin_nontemporal_store(floatx4{v[4], v[5], v[6], v[7]}, dst + 1);
        } else if (a.out_dtype == CSA2_F32) {
          float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + (rowh + h) * kDim + ch);
          dst[0] = make_float4(v[0], v[1], v[2], v[3]);
          dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          uint32_t pk[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t lo = __float_as_uint(v[2 * k]), hi = __float_as_uint(v[2 * k + 1]);
            lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
            hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
            pk[k] = lo | (hi << 16);
          }
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (rowh + h) * kDim + ch) =
              make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
      }
    }
    if (w == 0 && q4 == 0) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const int h = 16 * ht + n16;
        if (a.slots == 1) {
          if (a.lse) a.lse[rowh + h] = lrun[ht] > 0.0f ? (mref[ht] + __log2f(lrun[ht])) * kLn2 : -INFINITY;
        } else {
          a.ws_m[(rowh + h) * a.slots + split] = mref[ht];
          a.ws_l[(rowh + h) * a.slots + split] = lrun[ht];
        }
      }
    }
  }
}

// ---- Pipelined workgroups (bf16 queries, 16 or 32 heads).  Waves 0-3 and
// 4-7 take different roles so that the two waves sharing a SIMD run
// different code at the same time instead of meeting at every barrier with
// the same work.  Iteration i has two phases, each ended by a barrier:
//  * waves 0-3 (QK^T role) score step i: phase 1 gathers and dequantizes
//    their 32 keys (two 16-key tiles, the gather of step i+1 in flight) and
//    runs QK^T with the query fragments shared by both tiles, then
//    publishes per-wave maxima; phase 2 moves the lazy references, writes
//    the probabilities and sums and stages the raw codes and scales of step
//    i in buffer i%2;
//  * waves 4-7 (PV role) run PV for step i-1 from buffer (i-1)%2, half of
//    its keys per phase; wave 4+c owns channels [128c, 128c+128) of every
//    head over all keys of the step (no key halves, so each writes its own
//    channels at the end).
// The running sums live in the QK^T waves (updated one iteration later from
// the published sums), the outputs in the PV waves, which rescale them by
// the published factors when a reference moved.
template <int NHT, int KT>
struct SmemPP {
  static constexpr int kKeys = 64 * KT;  // keys per step
  _Float16 q[16 * NHT * kQStride];
  uint8_t cs[2][(kKeys / 32) * kCsBlock];
  _Float16 sct[2][kGroups * kScStride];
  _Float16 p[2][16 * NHT * kPStride];
  float red_max[4][64];
  float red_sum[4][64];
  float alpha[64];
  float lfin[64];
};

template <int NHT, int KT>
__global__ __launch_bounds__(kThreads, 1) void k_attn_pp(AttnArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  SmemPP<NHT, KT>& sm = *reinterpret_cast<SmemPP<NHT, KT>*>(smem_raw);
  constexpr int kKeys = SmemPP<NHT, KT>::kKeys;  // keys per step: KT 16-key tiles per QK^T wave
  constexpr int HG = 16 * NHT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so each role branches as a whole
  const int n16 = lane & 15, q4 = lane >> 4;
  const bool qk_role = w < 4;
  const int c4 = w & 3;  // QK^T: key quarter of the step; PV: channel quarter
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int h0 = hg * HG;
  const int kbeg = split * a.keys_per_split;
  const int kend = min(a.top_k, kbeg + a.keys_per_split);
  const int nsteps = kend > kbeg ? (kend - kbeg + kKeys - 1) / kKeys : 0;
  const int vis = a.row_visible ? a.row_visible[r] : 0x7FFFFFFF;
  const int64_t rs = a.row_start[r];
  const int64_t rowh = (int64_t)r * a.Hq + h0;
  int slot[KT];  // QK^T role: this lane's keys within a step
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) slot[kt] = 16 * KT * c4 + 16 * kt + n16;

  Raw bufA[KT], bufB[KT];
  uint32_t vA[KT], vB[KT];
  int32_t jn[KT];
  if (qk_role) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int32_t j0 = load_idx(a, r, kbeg + slot[kt], kend);
      jn[kt] = load_idx(a, r, kbeg + kKeys + slot[kt], kend);
      load_raw(bufA[kt], a, rs, vis, j0, kbeg + slot[kt], kend, vA[kt], q4);
    }
  }
  {
    constexpr int NP = HG * kDim / 8 / kThreads;  // 16-byte query pieces per thread
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + rowh * kDim;
    u32x4 v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      v[i] = *reinterpret_cast<const u32x4*>(qb + (int64_t)(p / (kDim / 8)) * kDim + (p % (kDim / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      half8 hv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hv[2 * k] = (_Float16)__uint_as_float(v[i][k] << 16);
        hv[2 * k + 1] = (_Float16)__uint_as_float(v[i][k] & 0xFFFF0000u);
      }
      *reinterpret_cast<half8*>(&sm.q[(p / (kDim / 8)) * kQStride + (p % (kDim / 8)) * 8]) = hv;
    }
  }
  __syncthreads();

  // Each role runs a loop of its own with the same barriers (two per
  // iteration, nsteps + 1 iterations), so only one role's state is live in
  // either loop.
  if (qk_role) {
    // lazy references and running sums per head 16*ht + n16 (replicated over q4 and waves)
    float mref[NHT], lrun[NHT], alpha_prev[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      mref[ht] = -INFINITY;
      lrun[ht] = 0.0f;
      alpha_prev[ht] = 1.0f;
    }
    auto iter = [&](int it, Raw (&cur)[KT], uint32_t (&vcur)[KT], Raw (&nxt)[KT], uint32_t (&vnxt)[KT]) {
      const int bw = it & 1;
      half2v sc[KT][4];
      floatx4 S[KT][NHT];
      // ---------------- phase 1
      if (it > 0) {  // running sums of step it-1
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          const int h = 16 * ht + n16;
          const float add = (sm.red_sum[0][h] + sm.red_sum[1][h]) + (sm.red_sum[2][h] + sm.red_sum[3][h]);
          lrun[ht] = lrun[ht] * alpha_prev[ht] + add;
        }
      }
      if (it < nsteps) {
        const int kstep0 = kbeg + it * kKeys;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          load_raw(nxt[kt], a, rs, vis, jn[kt], kstep0 + kKeys + slot[kt], kend, vnxt[kt], q4);
          jn[kt] = load_idx(a, r, kstep0 + 2 * kKeys + slot[kt], kend);
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          mask_raw(cur[kt], vcur[kt]);
          sc[kt][0] = e4m3x2_to_h2<false>(cur[kt].s[0]);
          sc[kt][1] = e4m3x2_to_h2<true>(cur[kt].s[0]);
          sc[kt][2] = e4m3x2_to_h2<false>(cur[kt].s[1]);
          sc[kt][3] = e4m3x2_to_h2<true>(cur[kt].s[1]);
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) S[kt][ht] = floatx4{0.f, 0.f, 0.f, 0.f};
        half8 bq[2][NHT];
        auto load_bq = [&](half8* dst, int ks) {
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
            dst[ht] = *reinterpret_cast<const half8*>(&sm.q[(16 * ht + n16) * kQStride + 128 * q4 + 8 * ks]);
        };
        load_bq(bq[0], 0);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          if (ks + 1 < 16) load_bq(bq[(ks + 1) & 1], ks + 1);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const uint32_t word = cur[kt].c[ks >> 2][ks & 3];
            const half2v s1 = sc[kt][ks >> 2];
            const half2v sv = (ks & 2) ? __builtin_shufflevector(s1, s1, 1, 1) : __builtin_shufflevector(s1, s1, 0, 0);
            const half8 av = cat4(fp4x2_to_h2<0>(word) * sv, fp4x2_to_h2<1>(word) * sv,
                                  fp4x2_to_h2<2>(word) * sv, fp4x2_to_h2<3>(word) * sv);
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) S[kt][ht] = mfma(av, bq[ks & 1][ht], S[kt][ht]);
          }
        }
        // scaled, masked logits and the per-wave maxima (keys 16*KT*c4 + 16*kt + 4*q4 + i)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const unsigned long long vm = __ballot(vcur[kt]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool ok = (vm >> (4 * q4 + i)) & 1ull;
              const float z = ok ? S[kt][ht][i] * a.c2 : -INFINITY;
              S[kt][ht][i] = z;
              mx = fmaxf(mx, z);
            }
          }
          mx = rows_max(mx);
          if (q4 == 0) sm.red_max[c4][16 * ht + n16] = mx;
        }
      }
      lds_barrier();
      // ---------------- phase 2: references, probabilities, sums, staging of step it
      if (it < nsteps) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          const int h = 16 * ht + n16;
          const float mstep = fmaxf(fmaxf(sm.red_max[0][h], sm.red_max[1][h]), fmaxf(sm.red_max[2][h], sm.red_max[3][h]));
          const float mnew = (mstep > mref[ht] + kLazy) ? mstep : mref[ht];
          const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
          alpha_prev[ht] = (mnew == mref[ht]) ? 1.0f : __builtin_amdgcn_exp2f(mref[ht] - muse);
          mref[ht] = mnew;
          float sum = 0.0f;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            _Float16 pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pv[i] = (_Float16)__builtin_amdgcn_exp2f(S[kt][ht][i] - muse);
              sum += (float)pv[i];
            }
            *reinterpret_cast<u32x2*>(&sm.p[bw][h * kPStride + 16 * KT * c4 + 16 * kt + 4 * q4]) =
                u32x2{h2_bits(half2v{pv[0], pv[1]}), h2_bits(half2v{pv[2], pv[3]})};
          }
          sum = rows_sum(sum);
          if (q4 == 0) {
            sm.red_sum[c4][h] = sum;
            if (c4 == 0) sm.alpha[h] = alpha_prev[ht];
          }
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x4*>(&sm.cs[bw][cs_off(slot[kt]) + 64 * q4 + 16 * c]) = cur[kt].c[c];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            sm.sct[bw][(8 * q4 + 2 * g) * kScStride + slot[kt]] = sc[kt][g][0];
            sm.sct[bw][(8 * q4 + 2 * g + 1) * kScStride + slot[kt]] = sc[kt][g][1];
          }
        }
      }
      lds_barrier();
    };
    for (int it = 0; it <= nsteps; it += 2) {
      iter(it, bufA, vA, bufB, vB);
      if (it + 1 <= nsteps) iter(it + 1, bufB, vB, bufA, vA);
    }
    // epilogue: running sums to the PV waves through LDS
    if (c4 == 0 && q4 == 0) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) sm.lfin[16 * ht + n16] = lrun[ht];
    }
    __syncthreads();
    if (c4 == 0 && q4 == 0) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const int h = 16 * ht + n16;
        if (a.slots == 1) {
          if (a.lse) a.lse[rowh + h] = lrun[ht] > 0.0f ? (mref[ht] + __log2f(lrun[ht])) * kLn2 : -INFINITY;
        } else {
          a.ws_m[(rowh + h) * a.slots + split] = mref[ht];
          a.ws_l[(rowh + h) * a.slots + split] = lrun[ht];
        }
      }
    }
  } else {
    // outputs of channels 128*c4 + 8*n16 + t, heads 16*ht + 4*q4 + i
    floatx4 O[NHT][8];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int t = 0; t < 8; ++t) O[ht][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // PV over keys [32kk, 32kk+32) of the step staged in buffer b
    auto pv_part = [&](int b, int kk) {
      const int key0 = 32 * kk + 8 * q4;
      uint32_t W[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        W[k] = *reinterpret_cast<const uint32_t*>(&sm.cs[b][cs_off(key0 + k) + 64 * c4 + 4 * n16]);
      const u32x4 spw = *reinterpret_cast<const u32x4*>(&sm.sct[b][(8 * c4 + (n16 >> 1)) * kScStride + key0]);
      uint32_t E[4], D[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t wa = W[2 * p], wb = W[2 * p + 1];
        E[p] = (wa & 0x0F0F0F0Fu) | ((wb << 4) & 0xF0F0F0F0u);
        D[p] = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);
      }
      half8 av[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) av[ht] = *reinterpret_cast<const half8*>(&sm.p[b][(16 * ht + n16) * kPStride + key0]);
      auto tile = [&](auto sel_c, const uint32_t(&src)[4], int t) {
        constexpr int SEL = decltype(sel_c)::value;
        u32x4 bb;
#pragma unroll
        for (int p = 0; p < 4; ++p) bb[p] = h2_bits(fp4x2_to_h2<SEL>(src[p]) * bits_h2(spw[p]));
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) O[ht][t] = mfma(av[ht], __builtin_bit_cast(half8, bb), O[ht][t]);
      };
      tile(std::integral_constant<int, 0>{}, E, 0);
      tile(std::integral_constant<int, 0>{}, D, 1);
      tile(std::integral_constant<int, 1>{}, E, 2);
      tile(std::integral_constant<int, 1>{}, D, 3);
      tile(std::integral_constant<int, 2>{}, E, 4);
      tile(std::integral_constant<int, 2>{}, D, 5);
      tile(std::integral_constant<int, 3>{}, E, 6);
      tile(std::integral_constant<int, 3>{}, D, 7);
    };
    for (int it = 0; it <= nsteps; ++it) {
      const int br = (it & 1) ^ 1;
      // ---------------- phase 1: rescale when a reference moved at step it-1, then all but the
      // last 32 keys of the step
      if (it > 0) {
        float al[NHT][4];
        bool moved = false;
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            al[ht][i] = sm.alpha[16 * ht + 4 * q4 + i];
            moved |= al[ht][i] != 1.0f;
          }
        if (__ballot(moved)) {
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int t = 0; t < 8; ++t) O[ht][t][i] *= al[ht][i];
        }
#pragma unroll
        for (int kk = 0; kk < 2 * KT - 1; ++kk) pv_part(br, kk);
      }
      lds_barrier();
      // ---------------- phase 2: the last 32 keys
      if (it > 0) pv_part(br, 2 * KT - 1);
      lds_barrier();
    }
    __syncthreads();
    // epilogue: each PV wave writes its channels of every head
    const int ch = 128 * c4 + 8 * n16;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * ht + 4 * q4 + i;
        const float L = sm.lfin[h];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = O[ht][t][i] * inv;
        if (a.slots > 1) {
          floatx4* dst = reinterpret_cast<floatx4*>(a.ws_o + ((rowh + h) * a.slots + split) * kDim + ch);
          __builtin_nontemporal_store(floatx4{v[0], v[1], v[2], v[3]}, dst);
          __builtin_nontemporal_store(floatx4{v[4], v[5], v[6], v[7]}, dst + 1);
        } else if (a.out_dtype == CSA2_F32) {
          float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + (rowh + h) * kDim + ch);
          dst[0] = make_float4(v[0], v[1], v[2], v[3]);
          dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          uint32_t pk[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t lo = __float_as_uint(v[2 * k]), hi = __float_as_uint(v[2 * k + 1]);
            lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
            hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
            pk[k] = lo | (hi << 16);
          }
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (rowh + h) * kDim + ch) =
              make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
      }
    }
  }
}

// ---- 64-head workgroups (bf16 queries) for batches whose rows alone fill
// the chip.  Every key is then dequantized once per 64 heads instead of once
// per 32, for QK^T and for PV.  QK^T is as above with four head tiles; PV
// gives wave w the channels [64w, 64w+64) of all 64 heads over all keys of
// the step: a lane owns the 4 channels 64w + 4*n16 + t (t = 0..3, one per
// output tile, all in one scale group), reads their 16-bit code pieces and
// interleaves two keys' nibbles per byte, two key pairs per 32-bit word, so
// that each converted fp16 pair again holds two keys of one channel.  With
// no key halves, each wave writes its own channels at the end.
struct SmemWide {
  _Float16 q[64 * kQStride];
  union {
    struct {
      uint8_t cs[(kStep / 32) * kCsBlock];
      _Float16 sct[kGroups * kScStride];
    } f;                            // FP4 steps: staged codes and scales
    uint8_t wc[kWinMax * kWStride];  // the window step: staged FP8 entries
  } u;
  _Float16 p[64 * kPStride];
  float red_max[kWaves][64];
  float red_sum[kWaves][64];
  float alpha[64];
  float lfin[64];
  int moved;            // 1: some head's reference moved in this step (written before its second barrier)
  uint8_t fresh[kDim];  // the row's newest window token, when the call writes it
};

__global__ __launch_bounds__(kThreads, 1) void k_sparse_attn_wide(AttnArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  SmemWide& sm = *reinterpret_cast<SmemWide*>(smem_raw);
  constexpr int NHT = 4, HG = 64;
  static_assert(kWaves == 8, "the cross-wave reductions give each of the 4 lane groups two waves");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int split = blockIdx.x, r = blockIdx.y, hg = blockIdx.z;
  const int h0 = hg * HG;
  const int kbeg = split * a.keys_per_split;
  const int kend = min(a.top_k, kbeg + a.keys_per_split);
  const int nsteps = kend > kbeg ? (kend - kbeg + kStep - 1) / kStep : 0;
  const int vis = a.row_visible ? a.row_visible[r] : 0x7FFFFFFF;
  const int64_t rs = a.row_start[r];
  const int myslot = 16 * w + n16;  // this lane's key within a step (QK^T role)

  // ---- prologue (as in k_sparse_attn): indices, the keys of step 0 in flight, queries to LDS
  uint32_t vA = 0, vB = 0;
  Raw bufA, bufB;
  const int32_t j0 = load_idx(a, r, kbeg + myslot, kend);
  int32_t jn = load_idx(a, r, kbeg + kStep + myslot, kend);
  load_raw(bufA, a, rs, vis, j0, kbeg + myslot, kend, vA, q4);
  {
    constexpr int NP = HG * kDim / 8 / kThreads;  // 16-byte pieces per thread
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + ((int64_t)r * a.Hq + h0) * kDim;
    u32x4 v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      v[i] = *reinterpret_cast<const u32x4*>(qb + (int64_t)(p / (kDim / 8)) * kDim + (p % (kDim / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      half8 hv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hv[2 * k] = (_Float16)__uint_as_float(v[i][k] << 16);
        hv[2 * k + 1] = (_Float16)__uint_as_float(v[i][k] & 0xFFFF0000u);
      }
      *reinterpret_cast<half8*>(&sm.q[(p / (kDim / 8)) * kQStride + (p % (kDim / 8)) * 8]) = hv;
    }
  }
  __syncthreads();

  floatx4 O[NHT][4];  // [head tile][channel 64w + 4*n16 + t]: heads 16*ht + 4*q4 + i
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int t = 0; t < 4; ++t) O[ht][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mref[NHT], lrun[NHT];  // per head 16*ht + n16 (softmax role), replicated over q4 and waves
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    mref[ht] = -INFINITY;
    lrun[ht] = 0.0f;
  }
  const int cb = 32 * w + 2 * n16;     // byte of this lane's PV channels in a code row
  const int grp = 4 * w + (n16 >> 2);  // their scale group

  auto step = [&](int st, Raw& cur, uint32_t vcur, Raw& nxt, uint32_t& vnxt) {
    const int kstep0 = kbeg + st * kStep;
    load_raw(nxt, a, rs, vis, jn, kstep0 + kStep + myslot, kend, vnxt, q4);
    jn = load_idx(a, r, kstep0 + 2 * kStep + myslot, kend);
    mask_raw(cur, vcur);
    half2v sc[4];
    sc[0] = e4m3x2_to_h2<false>(cur.s[0]);
    sc[1] = e4m3x2_to_h2<true>(cur.s[0]);
    sc[2] = e4m3x2_to_h2<false>(cur.s[1]);
    sc[3] = e4m3x2_to_h2<true>(cur.s[1]);

    // ---- QK^T: S^T[key][head] for this wave's 16 keys and the 64 heads
    floatx4 S[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) S[ht] = floatx4{0.f, 0.f, 0.f, 0.f};
    half8 bq[2][NHT];  // query fragments, one K-step ahead
    auto load_bq = [&](half8* dst, int ks) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        dst[ht] = *reinterpret_cast<const half8*>(&sm.q[(16 * ht + n16) * kQStride + 128 * q4 + 8 * ks]);
    };
    load_bq(bq[0], 0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks + 1 < 16) load_bq(bq[(ks + 1) & 1], ks + 1);
      const uint32_t word = cur.c[ks >> 2][ks & 3];
      const half2v s1 = sc[ks >> 2];
      const half2v sv = (ks & 2) ? __builtin_shufflevector(s1, s1, 1, 1) : __builtin_shufflevector(s1, s1, 0, 0);
      const half8 av = cat4(fp4x2_to_h2<0>(word) * sv, fp4x2_to_h2<1>(word) * sv, fp4x2_to_h2<2>(word) * sv,
                            fp4x2_to_h2<3>(word) * sv);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) S[ht] = mfma(av, bq[ks & 1][ht], S[ht]);
    }

    // ---- softmax (maxima exchanged first, then probabilities; lazy references as above)
    const unsigned long long vm = __ballot(vcur);
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (vm >> (4 * q4 + i)) & 1ull;
        const float z = ok ? S[ht][i] * a.c2 : -INFINITY;
        S[ht][i] = z;
        mx = fmaxf(mx, z);
      }
      mx = rows_max(mx);
      if (q4 == 0) sm.red_max[w][16 * ht + n16] = mx;
    }
    lds_barrier();  // B1: maxima visible; every wave is past the previous PV
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(&sm.u.f.cs[cs_off(myslot) + 64 * q4 + 16 * c]) = cur.c[c];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sm.u.f.sct[(8 * q4 + 2 * g) * kScStride + myslot] = sc[g][0];
      sm.u.f.sct[(8 * q4 + 2 * g + 1) * kScStride + myslot] = sc[g][1];
    }
    float alpha[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      // lane group q4 takes waves 2q4 and 2q4+1, the four groups then meet across lanes
      const float mstep = rows_max(fmaxf(sm.red_max[2 * q4][h], sm.red_max[2 * q4 + 1][h]));
      const float mnew = (mstep > mref[ht] + kLazy) ? mstep : mref[ht];
      const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
      alpha[ht] = (mnew == mref[ht]) ? 1.0f : __builtin_amdgcn_exp2f(mref[ht] - muse);
      mref[ht] = mnew;
      _Float16 pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = (_Float16)__builtin_amdgcn_exp2f(S[ht][i] - muse);
      // the rounded probabilities summed two per instruction in fp32 (v_dot2 with ones)
      float sum = __builtin_amdgcn_fdot2(half2v{pv[0], pv[1]}, half2v{1.0f16, 1.0f16}, 0.0f, false);
      sum = __builtin_amdgcn_fdot2(half2v{pv[2], pv[3]}, half2v{1.0f16, 1.0f16}, sum, false);
      *reinterpret_cast<u32x2*>(&sm.p[h * kPStride + 16 * w + 4 * q4]) =
          u32x2{h2_bits(half2v{pv[0], pv[1]}), h2_bits(half2v{pv[2], pv[3]})};
      sum = rows_sum(sum);
      if (q4 == 0) {
        sm.red_sum[w][h] = sum;
        if (w == 0) sm.alpha[h] = alpha[ht];
      }
    }
    if (w == 0) {
      // whether any head's reference moved this step (wave 0's lanes hold every head)
      bool mv = false;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) mv |= alpha[ht] != 1.0f;
      const bool any = __ballot(mv) != 0ull;
      if (lane == 0) sm.moved = any ? 1 : 0;
    }
    lds_barrier();  // B2: probabilities, sums, alpha and staged codes visible
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      const float add = rows_sum(sm.red_sum[2 * q4][h] + sm.red_sum[2 * q4 + 1][h]);  // same order in every lane
      lrun[ht] = lrun[ht] * alpha[ht] + add;
    }
    // the outputs rescaled only in a step where some head's reference moved (one LDS word read)
    if (st > 0 && sm.moved) {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = sm.alpha[16 * ht + 4 * q4 + i];
#pragma unroll
          for (int t = 0; t < 4; ++t) O[ht][t][i] *= al;
        }
    }

    // ---- PV over the step's 128 keys, 32 per K-step: this lane's keys key0 .. key0+7
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int key0 = 32 * kk + 8 * q4;
      uint32_t W[8];  // the 4 code nibbles (channels 64w + 4*n16 .. +3) of each key
#pragma unroll
      for (int k = 0; k < 8; ++k) W[k] = *reinterpret_cast<const uint16_t*>(&sm.u.f.cs[cs_off(key0 + k) + cb]);
      const u32x4 spw = *reinterpret_cast<const u32x4*>(&sm.u.f.sct[grp * kScStride + key0]);
      // bytes of E: channel 0 of keys (0,1), channel 2 of keys (0,1), channel 0 of keys (2,3),
      // channel 2 of keys (2,3) (first two key pairs; the second word the next two); D: channels 1, 3
      uint32_t E[2], D[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t A = W[4 * h2] | (W[4 * h2 + 2] << 16), B = W[4 * h2 + 1] | (W[4 * h2 + 3] << 16);
        E[h2] = (A & 0x0F0F0F0Fu) | ((B << 4) & 0xF0F0F0F0u);
        D[h2] = ((A >> 4) & 0x0F0F0F0Fu) | (B & 0xF0F0F0F0u);
      }
      half8 av[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        av[ht] = *reinterpret_cast<const half8*>(&sm.p[(16 * ht + n16) * kPStride + key0]);
      // tile t: channel 64w + 4*n16 + t; key pairs 0..3 from bytes (lo, hi) of the two words
      auto tile = [&](auto lo_c, const uint32_t(&src)[2], int t) {
        constexpr int LO = decltype(lo_c)::value;  // byte of the first key pair of a word (0 or 1)
        const u32x4 b = u32x4{h2_bits(fp4x2_to_h2<LO>(src[0]) * bits_h2(spw[0])),
                              h2_bits(fp4x2_to_h2<LO + 2>(src[0]) * bits_h2(spw[1])),
                              h2_bits(fp4x2_to_h2<LO>(src[1]) * bits_h2(spw[2])),
                              h2_bits(fp4x2_to_h2<LO + 2>(src[1]) * bits_h2(spw[3]))};
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) O[ht][t] = mfma(av[ht], __builtin_bit_cast(half8, b), O[ht][t]);
      };
      tile(std::integral_constant<int, 0>{}, E, 0);
      tile(std::integral_constant<int, 0>{}, D, 1);
      tile(std::integral_constant<int, 1>{}, E, 2);
      tile(std::integral_constant<int, 1>{}, D, 3);
    }
  };
  for (int st = 0; st < nsteps; st += 2) {
    step(st, bufA, vA, bufB, vB);
    if (st + 1 < nsteps) step(st + 1, bufB, vB, bufA, vA);
  }

  // ---- the row's local window as one more step (FP8 entries, no gather, no scales): lane
  // loads bytes [128 q4, +128) of entry `myslot`, converts them for QK^T, stages them for PV
  // (the staging area of the FP4 steps, free once every wave is past their PV), and PV
  // transposes each lane's 4-byte channel pieces of 8 entries with byte permutes.
  if (a.win) {
    const int len = min(max(a.win_len[r], 0), kWinMax);
    u32x4 c[8];
    if (myslot < len) {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.win + (a.win_start[r] + myslot) * kDim + 128 * q4);
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (a.new_x) {
      encode_fresh(a, r, hg, sm.fresh);
      lds_barrier();
      (void)take_fresh(a, r, myslot, len, q4, sm.fresh, c);
    }
    floatx4 S[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) S[ht] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint32_t w0 = c[ks >> 1][2 * (ks & 1)], w1 = c[ks >> 1][2 * (ks & 1) + 1];
      const half8 av = cat4(e4m3x2_to_h2<false>(w0), e4m3x2_to_h2<true>(w0), e4m3x2_to_h2<false>(w1),
                            e4m3x2_to_h2<true>(w1));
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        S[ht] = mfma(av, *reinterpret_cast<const half8*>(&sm.q[(16 * ht + n16) * kQStride + 128 * q4 + 8 * ks]),
                     S[ht]);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = (16 * w + 4 * q4 + i < len) ? S[ht][i] * a.c2 : -INFINITY;
        S[ht][i] = z;
        mx = fmaxf(mx, z);
      }
      mx = rows_max(mx);
      if (q4 == 0) sm.red_max[w][16 * ht + n16] = mx;
    }
    lds_barrier();  // maxima visible; every wave is past the last FP4 PV
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&sm.u.wc[myslot * kWStride + 128 * q4 + 16 * i]) = c[i];
    float alpha[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      // lane group q4 takes waves 2q4 and 2q4+1, the four groups then meet across lanes
      const float mstep = rows_max(fmaxf(sm.red_max[2 * q4][h], sm.red_max[2 * q4 + 1][h]));
      const float mnew = (mstep > mref[ht] + kLazy) ? mstep : mref[ht];
      const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
      alpha[ht] = (mnew == mref[ht]) ? 1.0f : __builtin_amdgcn_exp2f(mref[ht] - muse);
      mref[ht] = mnew;
      _Float16 pv[4];
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = (_Float16)__builtin_amdgcn_exp2f(S[ht][i] - muse);
        sum += (float)pv[i];
      }
      *reinterpret_cast<u32x2*>(&sm.p[h * kPStride + 16 * w + 4 * q4]) =
          u32x2{h2_bits(half2v{pv[0], pv[1]}), h2_bits(half2v{pv[2], pv[3]})};
      sum = rows_sum(sum);
      if (q4 == 0) {
        sm.red_sum[w][h] = sum;
        if (w == 0) sm.alpha[h] = alpha[ht];
      }
    }
    lds_barrier();  // probabilities, sums, alpha and staged entries visible
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      const float add = rows_sum(sm.red_sum[2 * q4][h] + sm.red_sum[2 * q4 + 1][h]);  // same order in every lane
      lrun[ht] = lrun[ht] * alpha[ht] + add;
    }
    {
      float al[NHT][4];
      bool moved = false;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          al[ht][i] = sm.alpha[16 * ht + 4 * q4 + i];
          moved |= al[ht][i] != 1.0f;
        }
      if (__ballot(moved)) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) O[ht][t][i] *= al[ht][i];
      }
    }
    const int cw = 64 * w + 4 * n16;  // this lane's 4 PV channels
    const int kk_end = (len + 31) >> 5;
    for (int kk = 0; kk < kk_end; ++kk) {
      const int e0 = 32 * kk + 8 * q4;
      uint32_t W[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) W[k] = *reinterpret_cast<const uint32_t*>(&sm.u.wc[(e0 + k) * kWStride + cw]);
      uint32_t T[2][4];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t a01 = perm(W[4 * g + 1], W[4 * g], 0x05010400u), b01 = perm(W[4 * g + 1], W[4 * g], 0x07030602u);
        const uint32_t a23 = perm(W[4 * g + 3], W[4 * g + 2], 0x05010400u),
                       b23 = perm(W[4 * g + 3], W[4 * g + 2], 0x07030602u);
        T[g][0] = perm(a23, a01, 0x05040100u);
        T[g][1] = perm(a23, a01, 0x07060302u);
        T[g][2] = perm(b23, b01, 0x05040100u);
        T[g][3] = perm(b23, b01, 0x07060302u);
      }
      half8 av[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) av[ht] = *reinterpret_cast<const half8*>(&sm.p[(16 * ht + n16) * kPStride + e0]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const half8 b = cat4(e4m3x2_to_h2<false>(T[0][t]), e4m3x2_to_h2<true>(T[0][t]), e4m3x2_to_h2<false>(T[1][t]),
                             e4m3x2_to_h2<true>(T[1][t]));
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) O[ht][t] = mfma(av[ht], b, O[ht][t]);
      }
    }
  }

  // ---- epilogue: each wave writes its 64 channels of the 64 heads
  if (w == 0 && q4 == 0) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) sm.lfin[16 * ht + n16] = lrun[ht];
  }
  __syncthreads();
  const int64_t rowh = (int64_t)r * a.Hq + h0;
  const int ch = 64 * w + 4 * n16;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * ht + 4 * q4 + i;
      const float L = sm.lfin[h];
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const float v0 = O[ht][0][i] * inv, v1 = O[ht][1][i] * inv, v2 = O[ht][2][i] * inv, v3 = O[ht][3][i] * inv;
      if (a.slots > 1) {
        floatx4* dst = reinterpret_cast<floatx4*>(a.ws_o + ((rowh + h) * a.slots + split) * kDim + ch);
        __builtin_nontemporal_store(floatx4{v0, v1, v2, v3}, dst);
      } else if (a.out_dtype == CSA2_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (rowh + h) * kDim + ch) = make_float4(v0, v1, v2, v3);
      } else {
        const float vv[4] = {v0, v1, v2, v3};
        uint32_t pk[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          uint32_t lo = __float_as_uint(vv[2 * k]), hi = __float_as_uint(vv[2 * k + 1]);
          lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
          hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
          pk[k] = lo | (hi << 16);
        }
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + (rowh + h) * kDim + ch) = make_uint2(pk[0], pk[1]);
      }
    }
  }
  if (w == 0 && q4 == 0) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      if (a.slots == 1) {
        if (a.lse) a.lse[rowh + h] = lrun[ht] > 0.0f ? (mref[ht] + __log2f(lrun[ht])) * kLn2 : -INFINITY;
      } else {
        a.ws_m[(rowh + h) * a.slots + split] = mref[ht];
        a.ws_l[(rowh + h) * a.slots + split] = lrun[ht];
      }
    }
  }
}

// ---- local sliding window.  A row's window (at most 128 entries of one
// signed E4M3 byte per channel, K = V like a Main KV entry) is one step of
// the loop above with no gather and no scales: a workgroup owns one (row,
// group of 16*NHT heads); lane (w, n16, q4) loads bytes [128 q4, +128) of
// window entry 16w + n16 into registers, converts them pairwise to fp16
// (exact: every E4M3 value is an fp16 value) as the QK^T A operand, and
// stages them in LDS for PV.  PV gives wave w channels [64w, 64w+64) as in
// the 64-head kernel: a lane reads the 4 bytes at channel 64w + 4*n16 of 8
// consecutive entries and transposes them with byte permutes so that each
// fp16 pair holds two entries of one channel.  The result is a partial
// (normalized output, maximum, sum) in the last slot, merged by the combine
// with the key splits of the selected entries, or the output itself when
// nothing else is attended.
template <int NHT, bool SPLITQ>
struct SmemSwa {
  static constexpr int kQRows = 16 * NHT * (SPLITQ ? 2 : 1);
  _Float16 q[kQRows * kQStride];
  uint8_t wc[kWinMax * kWStride];
  _Float16 p[16 * NHT * kPStride];
  float red_max[kWaves][64];
  float red_sum[kWaves][64];
  uint8_t fresh[kDim];  // the row's newest window token, when the call writes it
};

template <int NHT, bool SPLITQ, int QDT>
__global__ __launch_bounds__(kThreads, 1) void k_swa_attn(AttnArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  using Sm = SmemSwa<NHT, SPLITQ>;
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  constexpr int HG = 16 * NHT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int r = blockIdx.x, hg = blockIdx.y;
  const int h0 = hg * HG;
  const int len = min(max(a.win_len[r], 0), kWinMax);
  const int key = 16 * w + n16;  // this lane's entry in QK^T

  u32x4 c[8];  // bytes [128 q4, +128) of entry `key`
  if (key < len) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.win + (a.win_start[r] + key) * kDim + 128 * q4);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = src[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = u32x4{0u, 0u, 0u, 0u};
  }
  if (a.new_x) encode_fresh(a, r, hg, sm.fresh);
  // queries to LDS as fp16 (fp32 queries as hi + lo halves, rows HG.. the lo halves)
  if (QDT == CSA2_BF16) {
    constexpr int NP = HG * kDim / 8 / kThreads;
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + ((int64_t)r * a.Hq + h0) * kDim;
    u32x4 v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      v[i] = *reinterpret_cast<const u32x4*>(qb + (int64_t)(p / (kDim / 8)) * kDim + (p % (kDim / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      half8 hv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hv[2 * k] = (_Float16)__uint_as_float(v[i][k] << 16);
        hv[2 * k + 1] = (_Float16)__uint_as_float(v[i][k] & 0xFFFF0000u);
      }
      *reinterpret_cast<half8*>(&sm.q[(p / (kDim / 8)) * kQStride + (p % (kDim / 8)) * 8]) = hv;
    }
  } else {
    constexpr int NP = HG * kDim / 4 / kThreads;
    const float* qf = static_cast<const float*>(a.q) + ((int64_t)r * a.Hq + h0) * kDim;
    floatx4 v[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      v[i] = *reinterpret_cast<const floatx4*>(qf + (int64_t)(p / (kDim / 4)) * kDim + (p % (kDim / 4)) * 4);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + kThreads * i;
      const int h = p / (kDim / 4), c4 = (p % (kDim / 4)) * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const _Float16 hi = (_Float16)v[i][k];
        sm.q[h * kQStride + c4 + k] = hi;
        if (SPLITQ) sm.q[(HG + h) * kQStride + c4 + k] = (_Float16)(v[i][k] - (float)hi);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&sm.wc[key * kWStride + 128 * q4 + 16 * i]) = c[i];
  __syncthreads();
  // the fresh entry replaces the loaded one in registers and in its staged row (read by PV after the
  // softmax barrier)
  if (a.new_x && take_fresh(a, r, key, len, q4, sm.fresh, c)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&sm.wc[key * kWStride + 128 * q4 + 16 * i]) = c[i];
  }

  // ---- QK^T: S^T[entry][head]; K-step ks covers channels 128*q4 + 8*ks .. +7 on both operands
  constexpr int NQ = SPLITQ ? 2 : 1;
  floatx4 S[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) S[ht] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const uint32_t w0 = c[ks >> 1][2 * (ks & 1)], w1 = c[ks >> 1][2 * (ks & 1) + 1];
    const half8 av = cat4(e4m3x2_to_h2<false>(w0), e4m3x2_to_h2<true>(w0), e4m3x2_to_h2<false>(w1),
                          e4m3x2_to_h2<true>(w1));
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
      for (int qh = 0; qh < NQ; ++qh) {
        const half8 bq = *reinterpret_cast<const half8*>(&sm.q[(16 * (qh * NHT + ht) + n16) * kQStride + 128 * q4 + 8 * ks]);
        S[ht] = mfma(av, bq, S[ht]);
      }
    }
  }

  // ---- softmax over the window: lane holds entries 16w + 4q4 + i of head 16ht + n16
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = (16 * w + 4 * q4 + i < len) ? S[ht][i] * a.c2 : -INFINITY;
      S[ht][i] = z;
      mx = fmaxf(mx, z);
    }
    mx = rows_max(mx);
    if (q4 == 0) sm.red_max[w][16 * ht + n16] = mx;
  }
  __syncthreads();
  float mrow[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + n16;
    float m = sm.red_max[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) m = fmaxf(m, sm.red_max[ww][h]);
    mrow[ht] = m;
    const float muse = (m == -INFINITY) ? 0.0f : m;
    _Float16 pv[4];
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = (_Float16)__builtin_amdgcn_exp2f(S[ht][i] - muse);
      sum += (float)pv[i];
    }
    *reinterpret_cast<u32x2*>(&sm.p[h * kPStride + 16 * w + 4 * q4]) =
        u32x2{h2_bits(half2v{pv[0], pv[1]}), h2_bits(half2v{pv[2], pv[3]})};
    sum = rows_sum(sum);
    if (q4 == 0) sm.red_sum[w][h] = sum;
  }
  __syncthreads();

  // ---- PV: wave w, channels 64w + 4*n16 + t (tile t), all window entries
  floatx4 O[NHT][4];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int t = 0; t < 4; ++t) O[ht][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int cb = 64 * w + 4 * n16;
  const int kk_end = (len + 31) >> 5;  // 32-entry K-steps holding a valid entry
  for (int kk = 0; kk < kk_end; ++kk) {
    const int e0 = 32 * kk + 8 * q4;
    uint32_t W[8];  // channels cb .. cb+3 of entries e0 .. e0+7
#pragma unroll
    for (int k = 0; k < 8; ++k) W[k] = *reinterpret_cast<const uint32_t*>(&sm.wc[(e0 + k) * kWStride + cb]);
    // 4x4 byte transposes: T[t] of a group of 4 entries holds channel t of each
    uint32_t T[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t a01 = perm(W[4 * g + 1], W[4 * g], 0x05010400u), b01 = perm(W[4 * g + 1], W[4 * g], 0x07030602u);
      const uint32_t a23 = perm(W[4 * g + 3], W[4 * g + 2], 0x05010400u),
                     b23 = perm(W[4 * g + 3], W[4 * g + 2], 0x07030602u);
      T[g][0] = perm(a23, a01, 0x05040100u);
      T[g][1] = perm(a23, a01, 0x07060302u);
      T[g][2] = perm(b23, b01, 0x05040100u);
      T[g][3] = perm(b23, b01, 0x07060302u);
    }
    half8 av[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) av[ht] = *reinterpret_cast<const half8*>(&sm.p[(16 * ht + n16) * kPStride + e0]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half8 b = cat4(e4m3x2_to_h2<false>(T[0][t]), e4m3x2_to_h2<true>(T[0][t]), e4m3x2_to_h2<false>(T[1][t]),
                           e4m3x2_to_h2<true>(T[1][t]));
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) O[ht][t] = mfma(av[ht], b, O[ht][t]);
    }
  }

  // ---- epilogue: the partial of the last slot, or the output when it is the only one
  const int64_t rowh = (int64_t)r * a.Hq + h0;
  const int slot = a.slots - 1;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * ht + 4 * q4 + i;
      float L = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) L += sm.red_sum[ww][h];
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const float v0 = O[ht][0][i] * inv, v1 = O[ht][1][i] * inv, v2 = O[ht][2][i] * inv, v3 = O[ht][3][i] * inv;
      if (a.slots > 1) {
        floatx4* dst = reinterpret_cast<floatx4*>(a.ws_o + ((rowh + h) * a.slots + slot) * kDim + cb);
        __builtin_nontemporal_store(floatx4{v0, v1, v2, v3}, dst);
      } else if (a.out_dtype == CSA2_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (rowh + h) * kDim + cb) = make_float4(v0, v1, v2, v3);
      } else {
        const float vv[4] = {v0, v1, v2, v3};
        uint32_t pk[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          uint32_t lo = __float_as_uint(vv[2 * k]), hi = __float_as_uint(vv[2 * k + 1]);
          lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
          hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
          pk[k] = lo | (hi << 16);
        }
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + (rowh + h) * kDim + cb) = make_uint2(pk[0], pk[1]);
      }
    }
  }
  if (w == 0 && q4 == 0) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = 16 * ht + n16;
      float L = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) L += sm.red_sum[ww][h];
      if (a.slots == 1) {
        if (a.lse) a.lse[rowh + h] = L > 0.0f ? (mrow[ht] + __log2f(L)) * kLn2 : -INFINITY;
      } else {
        a.ws_m[(rowh + h) * a.slots + slot] = mrow[ht];
        a.ws_l[(rowh + h) * a.slots + slot] = L;
      }
    }
  }
}

// one (row, head) per workgroup of 128 threads, 4 channels per thread;
// splits merged in fixed order with a running maximum, 8 splits per batch of
// loads: o = sum_s w_s l_s o_s / sum_s w_s l_s,  w_s = 2^(m_s - max m)
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_m,
                                                      const float* __restrict__ ws_l, int splits, void* out,
                                                      int out_dtype, float* lse) {
  const int64_t rh = blockIdx.x;
  const float* m = ws_m + rh * splits;
  const float* l = ws_l + rh * splits;
  float M = -INFINITY, L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float4 v[8];
    float mm[8], ll[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = s0 + k < splits ? s0 + k : splits - 1;
      v[k] = reinterpret_cast<const float4*>(ws_o + (rh * splits + s) * kDim)[threadIdx.x];
      mm[k] = s0 + k < splits ? m[s] : -INFINITY;
      ll[k] = l[s];
    }
    float bm = mm[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) bm = fmaxf(bm, mm[k]);
    const float Mn = fmaxf(M, bm);
    if (Mn == -INFINITY) continue;  // every split so far is empty
    const float sc = __builtin_amdgcn_exp2f(M - Mn);  // 0 while M is still -inf
    L *= sc;
    acc.x *= sc;
    acc.y *= sc;
    acc.z *= sc;
    acc.w *= sc;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float wl = __builtin_amdgcn_exp2f(mm[k] - Mn) * ll[k];  // 0 for empty or missing splits
      L += wl;
      acc.x += wl * v[k].x;
      acc.y += wl * v[k].y;
      acc.z += wl * v[k].z;
      acc.w += wl * v[k].w;
    }
    M = Mn;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const float v[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if (out_dtype == CSA2_F32) {
    reinterpret_cast<float4*>(static_cast<float*>(out) + rh * kDim)[threadIdx.x] = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint32_t pk[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t lo = __float_as_uint(v[2 * k]), hi = __float_as_uint(v[2 * k + 1]);
      lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
      hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
      pk[k] = lo | (hi << 16);
    }
    reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + rh * kDim)[threadIdx.x] = make_uint2(pk[0], pk[1]);
  }
  if (lse && threadIdx.x == 0) lse[rh] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

struct Plan {
  int nht, head_groups, splits, keys_per_split;
  bool splitq;
  bool wide;  // 64-head workgroups (k_sparse_attn_wide)
};

// Launch plan.  A workgroup takes 32 heads (16 if the head count is an odd
// number of 16-head tiles) and, when rows x head groups do not fill the
// chip, the keys are split so that >= 256 workgroups run.  Small batches
// (at most 64 row x 16-head tiles) take 16 heads per workgroup: each key is
// then dequantized by twice as many workgroups, but half as many key splits
// fill the chip, which halves the split partials written here and read by
// the combine (measured faster at 4 and 16 rows of 64 heads, slower at 32).
// fp32 queries (hi and lo halves) always take 16 heads: 32 would not fit the
// double-buffered staging in LDS.  When rows x 64-head groups alone fill the
// chip (bf16 queries), workgroups take 64 heads and no keys are split.
Plan plan(int R, int Hq, int q_dtype, int top_k) {
  Plan p{};
  p.splitq = q_dtype == CSA2_F32;
  const int tiles = Hq / 16;
  const int max_splits = (int)std::max<int64_t>(1, ceil_div(top_k, kStep));
  p.wide = !p.splitq && tiles % 4 == 0 && (int64_t)R * (tiles / 4) >= 256;
  if (p.wide) {
    p.nht = 4;
    p.head_groups = tiles / 4;
    p.keys_per_split = (int)round_up(top_k, kStep);
    p.splits = 1;
    return p;
  }
  p.nht = (tiles % 2 == 0 && (int64_t)R * tiles > 64 && !p.splitq) ? 2 : 1;
  p.head_groups = tiles / p.nht;
  const int64_t base = (int64_t)R * p.head_groups;
  const int splits = (int)std::min<int64_t>(max_splits, std::max<int64_t>(1, ceil_div(256, base)));
  p.keys_per_split = (int)round_up(ceil_div(top_k, splits), kStep);
  p.splits = (int)ceil_div(top_k, p.keys_per_split);
  return p;
}

template <int NHT, int KT>
hipError_t go_pp(const Plan& p, int R, const AttnArgs& a, hipStream_t s) {
  auto kern = k_attn_pp<NHT, KT>;
  const size_t lds = sizeof(SmemPP<NHT, KT>);
  static bool configured = false;
  if (!configured) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.splits, R, p.head_groups), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int NHT, bool SPLITQ, int QDT>
hipError_t go(const Plan& p, int R, const AttnArgs& a, hipStream_t s) {
  auto kern = k_sparse_attn<NHT, SPLITQ, QDT>;
  const size_t lds = sizeof(Smem<NHT, SPLITQ>);
  static bool configured = false;
  if (!configured) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.splits, R, p.head_groups), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int NHT, bool SPLITQ, int QDT>
hipError_t go_swa(int R, int head_groups, const AttnArgs& a, hipStream_t s) {
  auto kern = k_swa_attn<NHT, SPLITQ, QDT>;
  const size_t lds = sizeof(SmemSwa<NHT, SPLITQ>);
  static bool configured = false;
  if (!configured) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(R, head_groups), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

// partial slots per (row, head): the key splits of the selected entries
// plus one for the window kernel (the 64-head kernel takes the window as one
// more step of its own loop instead); 1 means the only kernel writes the output
int attn_slots(int R, int Hq, int q_dtype, int top_k, bool window) {
  if (top_k == 0) return 1;
  const Plan p = plan(R, Hq, q_dtype, top_k);
  return p.splits + (window && !p.wide ? 1 : 0);
}

}  // namespace

size_t attn_workspace_bytes(int R, int Hq, int q_dtype, int top_k, bool window) {
  if (attn_dec_applies(R, Hq, q_dtype, top_k, window)) return attn_dec_workspace_bytes(R, Hq, top_k, window);
  const int slots = attn_slots(R, Hq, q_dtype, top_k, window);
  if (slots <= 1) return 0;
  const size_t n = (size_t)R * Hq * slots;
  return kAttnCounterBytes + ((n * kDim * 4 + 255) & ~size_t(255)) + 2 * ((n * 4 + 255) & ~size_t(255));
}

hipError_t launch_sparse_attn(int R, const void* q, int q_dtype, int Hq, const uint8_t* codes, const uint8_t* scales,
                              const int64_t* row_start, const int32_t* idx, int top_k, const int32_t* row_visible,
                              uint8_t* win, const int64_t* win_start, const int32_t* win_len,
                              const void* new_x, int new_x_dtype, int64_t new_x_stride, const int64_t* new_rows,
                              float softmax_scale, void* out, int out_dtype, float* lse, void* ws, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const bool window = win != nullptr;
  const bool dec = attn_dec_applies(R, Hq, q_dtype, top_k, window);
  if (dec && !window)
    return launch_attn_dec(R, q, Hq, codes, scales, row_start, idx, top_k, row_visible, softmax_scale, out, out_dtype,
                           lse, nullptr, nullptr, nullptr, ws, s);
  const Plan p = top_k > 0 && !dec ? plan(R, Hq, q_dtype, top_k) : Plan{};
  AttnArgs a{};
  a.q = q;
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
  a.slots = attn_slots(R, Hq, q_dtype, top_k, window);
  a.keys_per_split = p.keys_per_split;
  a.win = win;
  a.win_start = win_start;
  a.win_len = win_len;
  a.new_x = new_x;
  a.new_x_dtype = new_x_dtype;
  a.new_x_stride = new_x_stride;
  a.new_rows = new_rows;
  if (dec) {
    // the window first, as a partial (slot 1 of two) that the decode kernel's merge takes as one more term
    const size_t n = (size_t)R * Hq * 2;
    char* b = static_cast<char*>(ws) + attn_dec_workspace_bytes(R, Hq, top_k, false);
    a.slots = 2;
    a.ws_o = reinterpret_cast<float*>(b);
    b += (n * kDim * 4 + 255) & ~size_t(255);
    a.ws_m = reinterpret_cast<float*>(b);
    b += (n * 4 + 255) & ~size_t(255);
    a.ws_l = reinterpret_cast<float*>(b);
    auto& ew = profile_events(CSA2_KERNEL_SWA_ATTN);
    if (ew.start) (void)hipEventRecord(ew.start, s);
    const hipError_t e = go_swa<1, false, CSA2_BF16>(R, Hq / 16, a, s);
    if (ew.stop) (void)hipEventRecord(ew.stop, s);
    if (e != hipSuccess) return e;
    return launch_attn_dec(R, q, Hq, codes, scales, row_start, idx, top_k, row_visible, softmax_scale, out, out_dtype,
                           lse, a.ws_o, a.ws_m, a.ws_l, ws, s);
  }
  if (a.slots > 1) {
    const size_t n = (size_t)R * Hq * a.slots;
    char* b = static_cast<char*>(ws) + kAttnCounterBytes;
    a.ws_o = reinterpret_cast<float*>(b);
    b += (n * kDim * 4 + 255) & ~size_t(255);
    a.ws_m = reinterpret_cast<float*>(b);
    b += (n * 4 + 255) & ~size_t(255);
    a.ws_l = reinterpret_cast<float*>(b);
  }
  hipError_t e = hipSuccess;
  if (top_k > 0) {
    auto& ev = profile_events(CSA2_KERNEL_ATTN);
    if (ev.start) (void)hipEventRecord(ev.start, s);
    if (p.wide) {
      const size_t lds = sizeof(SmemWide);
      static bool configured = false;
      if (!configured) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_sparse_attn_wide),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        configured = true;
      }
      hipLaunchKernelGGL(k_sparse_attn_wide, dim3(p.splits, R, p.head_groups), dim3(kThreads), lds, s, a);
      e = hipGetLastError();
    } else if (q_dtype == CSA2_BF16) {
      // splits of at least two steps take the pipelined kernel (its first and last
      // iterations run one role only, which a single step cannot amortize)
      const bool pipelined = p.keys_per_split >= 2 * kStep;
      if (p.nht == 2) e = pipelined ? go_pp<2, 2>(p, R, a, s) : go<2, false, CSA2_BF16>(p, R, a, s);
      else e = pipelined ? go_pp<1, 2>(p, R, a, s) : go<1, false, CSA2_BF16>(p, R, a, s);
    } else {
      e = go<1, true, CSA2_F32>(p, R, a, s);
    }
    if (ev.stop) (void)hipEventRecord(ev.stop, s);
    if (e != hipSuccess) return e;
  }
  if (window && !(top_k > 0 && p.wide)) {
    // 64-head workgroups when rows alone fill the chip (bf16 queries), else 16
    const int tiles = Hq / 16;
    const bool wide = q_dtype == CSA2_BF16 && tiles % 4 == 0 && (int64_t)R * (tiles / 4) >= 256;
    auto& ew = profile_events(CSA2_KERNEL_SWA_ATTN);
    if (ew.start) (void)hipEventRecord(ew.start, s);
    if (wide) e = go_swa<4, false, CSA2_BF16>(R, tiles / 4, a, s);
    else if (q_dtype == CSA2_BF16) e = go_swa<1, false, CSA2_BF16>(R, tiles, a, s);
    else e = go_swa<1, true, CSA2_F32>(R, tiles, a, s);
    if (ew.stop) (void)hipEventRecord(ew.stop, s);
    if (e != hipSuccess) return e;
  }
  if (a.slots > 1) {
    auto& ec = profile_events(CSA2_KERNEL_ATTN_COMBINE);
    if (ec.start) (void)hipEventRecord(ec.start, s);
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)((int64_t)R * Hq)), dim3(128), 0, s, a.ws_o, a.ws_m, a.ws_l,
                       a.slots, out, out_dtype, lse);
    if (ec.stop) (void)hipEventRecord(ec.stop, s);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace csa2
