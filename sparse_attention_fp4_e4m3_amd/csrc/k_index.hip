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
//   k_prep      (Full) indexer queries -> fp32 ([channel quad][head][4]
//               order); zero the first-digit histograms
//   k_score     Full: every visible entry; Reindex: the pool entries.  Key
//               rows are staged through LDS with fully coalesced 16-byte
//               loads (the next tile prefetched into registers), queries
//               reach every lane through scalar loads (Full over bf16 / fp32
//               keys) or broadcast LDS loads of a once-staged copy (Reindex,
//               MXFP4 keys), each thread runs the H fmaf chains of one key.  Full also writes the 8-entry block maxima and
//               builds the first radix histogram (12 bits) of scores and
//               block maxima in the same pass.  HBM-bound on the key rows.
//   k_collect   (Full) every wave compacts, in position order, the entries
//               whose first digit reaches the threshold bin into its own
//               slice of a candidate list (no block-wide syncs)
//   k_finalize  one workgroup per row and series selects among the
//               candidates (Full) or pool slots (Reindex), held in LDS;
//               Reindex counts the first digit of the pool's scores here
//               (its scoring reads the queries as given and counts nothing)
// Exact selection: three radix digits give the K-th largest key, then an
// ordered compaction writes positions ascending, ties to the lower position,
// -1 padding; selected blocks expand into the pool.
// Scores are non-negative fp32, so their bit patterns order like uint32;
// invalid slots carry -1.0 (sign bit set) and are never counted.
#include <algorithm>
#include <type_traits>

#include "csa2_common.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kFinThreads = 1024;
constexpr int kSub = 2048;  // elements per collect wave (one candidate slice)
// radix digits over the 31 value bits: 12 / 11 / 8
constexpr int kD1 = 4096, kD2 = 2048, kD3 = 256;
constexpr int kS1 = 19, kS2 = 8;
constexpr int kScanSlots = 768;  // resident scan workgroups on 256 CUs (3 each)
constexpr int kMaxHeads = 32;
constexpr int kListRows = 64;  // grid rows of a pass over a device-side row list
constexpr int kQPrepared = -1;  // query "dtype" of a Reindex scan reading the prepared fp32 block

// One wave scores 64 keys at a time (one key per lane).  The keys' rows are
// loaded with fully coalesced 16-byte pieces, staged in the wave's own LDS
// area and read back one row per lane, so no workgroup barrier is needed
// between tiles and the waves of a workgroup drift freely.
//
// MXFP4 keys (32 code bytes + 2 E8M0 scale bytes per key, in two arrays) are
// not staged: each lane loads its own key's 32 bytes (two 16-byte loads; the
// wave's two loads cover 2 KiB of consecutive rows) and its 2 scale bytes,
// and widens the codes to fp32 itself (exact: E2M1 value times a power of two).
template <int KDT>
struct KeyTile {
  static constexpr bool kMx = KDT == CSA2_MXFP4;
  static constexpr int kBytes = KDT == CSA2_BF16 ? 128 : (kMx ? 32 : 256);  // one indexer key row (codes)
  static constexpr int kKeys = 64;                             // keys per wave tile
  static constexpr int kStride = kBytes + 16;                  // padded LDS row
  static constexpr int kPieces = kBytes / 16;                  // 16-byte pieces per row
  static constexpr int kPerLane = kKeys * kPieces / 64;        // 8 (bf16), 16 (fp32) or 2 (MXFP4, own key)
  static constexpr int kWaveBytes = kMx ? 0 : kKeys * kStride;  // LDS per wave
};
constexpr int kWavesPerWG = kThreads / 64;
constexpr int kWGKeys = kWavesPerWG * 64;  // keys per workgroup tile (one wave tile per wave)

__device__ __forceinline__ int clampv(int v, int maxv) { return v < 0 ? 0 : (v > maxv ? maxv : v); }

// ------------------------------------------------------------ block helpers

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts of
// 1, 2, 4, 8 within each 16-lane row, then the row totals carried across
// rows by broadcasting lane 15 (to rows 1, 3) and lane 31 (to rows 2, 3).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over the block; *total = the block sum.  lds >= NT/64 words.  LDS_ONLY: the
// barriers wait for LDS operations only, so global loads in flight stay in flight.
template <int NT, bool LDS_ONLY = false>
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t* lds, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_sum(v);
  if (lane == 63) lds[wave] = x;
  if (LDS_ONLY) lds_barrier();
  else __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = lds[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  if (LDS_ONLY) lds_barrier();
  else __syncthreads();
  *total = tot;
  return before + x - v;
}

// Bin holding the K-th largest element of a histogram of NB bins in global
// or shared memory (bins scanned from the top); -1 when it holds fewer than
// K.  *above = elements in higher bins, *total = all elements.  Each thread
// owns NB/NT consecutive bins, all loaded at once.  lds >= 20 words.
template <int NT, int NB>
__device__ __forceinline__ int find_bin(const uint32_t* h, uint32_t K, uint32_t* above, uint32_t* total, uint32_t* lds) {
  static_assert(NB % NT == 0, "bins per thread");
  constexpr int PER = NB / NT;
  const int hi = NB - (int)threadIdx.x * PER;  // this thread: bins [hi-PER, hi), descending
  uint32_t c[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) c[k] = h[hi - 1 - k];
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) local += c[k];
  uint32_t tot;
  const uint32_t before = block_excl_sum<NT>(local, lds, &tot);
  if (threadIdx.x == 0) lds[16] = 0xFFFFFFFFu;
  __syncthreads();
  if (before < K && K <= before + local) {
    uint32_t run = before, ab = 0;
    int bin = -1;
#pragma unroll
    for (int k = 0; k < PER; ++k) {  // this thread's bins from the top
      if (bin < 0 && K <= run + c[k]) {
        bin = hi - 1 - k;
        ab = run;
      }
      run += c[k];
    }
    lds[16] = (uint32_t)bin;
    lds[17] = ab;
  }
  __syncthreads();
  const uint32_t bin = lds[16], ab = lds[17];
  __syncthreads();
  *total = tot;
  *above = (bin == 0xFFFFFFFFu) ? tot : ab;
  return (bin == 0xFFFFFFFFu) ? -1 : (int)bin;
}

// find_bin for a histogram in LDS that the block has finished (a barrier
// since its last update): wave 0 alone scans it and publishes the bin, so the
// block meets at two barriers instead of four.  Lane l owns the NB/64
// consecutive bins below NB - l*NB/64 (lane 0 the highest), summed per
// 16-byte group; the lane holding the K-th largest element descends through
// its group sums, then through the four bins of that group.
template <int NB>
__device__ __forceinline__ int find_bin_wave(const uint32_t* h, uint32_t K, uint32_t* above, uint32_t* total,
                                             uint32_t* lds) {
  static_assert(NB % 256 == 0, "whole 16-byte groups per lane");
  constexpr int PER = NB / 64, NG = PER / 4;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int lo = NB - (lane + 1) * PER;  // this lane: bins [lo, lo + PER)
    const u32x4* p = reinterpret_cast<const u32x4*>(h + lo);
    uint32_t gs[NG];
    uint32_t local = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const u32x4 v = p[g];
      gs[g] = (v[0] + v[1]) + (v[2] + v[3]);
      local += gs[g];
    }
    const uint32_t incl = wave_incl_sum(local);
    const uint32_t before = incl - local;
    const uint32_t tot = (uint32_t)__shfl((int)incl, 63, 64);
    if (lane == 0) {
      lds[16] = 0xFFFFFFFFu;  // (overwritten below by the lane that holds the K-th element)
      lds[18] = tot;
    }
    if (before < K && K <= incl) {
      uint32_t run = before;
      int gsel = 0;
      bool found = false;
#pragma unroll
      for (int g = NG - 1; g >= 0; --g) {
        const bool here = !found && K <= run + gs[g];
        gsel = here ? g : gsel;
        run += (!found && !here) ? gs[g] : 0u;
        found = found || here;
      }
      const u32x4 v = p[gsel];
      int bin = lo + 4 * gsel;
      found = false;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const bool here = !found && K <= run + v[e];
        bin = here ? lo + 4 * gsel + e : bin;
        run += (!found && !here) ? v[e] : 0u;
        found = found || here;
      }
      lds[16] = (uint32_t)bin;
      lds[17] = run;
    }
  }
  lds_barrier();
  const uint32_t bin = lds[16], ab = lds[17], tot = lds[18];
  lds_barrier();
  *total = tot;
  *above = (bin == 0xFFFFFFFFu) ? tot : ab;
  return (bin == 0xFFFFFFFFu) ? -1 : (int)bin;
}

__device__ __forceinline__ void flush_hist(uint32_t* __restrict__ g, const uint32_t* __restrict__ l, int n) {
  for (int b = threadIdx.x; b < n; b += blockDim.x) {
    const uint32_t v = l[b];
    if (v) atomicAdd(g + b, v);
  }
}

// ------------------------------------------------------------ kernels

__global__ __launch_bounds__(256) void k_prep(const void* __restrict__ idx_q, int q_dtype, int R, int H,
                                              float* __restrict__ qf, uint32_t* __restrict__ hist, int64_t nhist) {
  const int64_t nq = (int64_t)R * H * kIdxDim;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += stride) {
    const int64_t r = i / (H * kIdxDim);
    const int rem = (int)(i % (H * kIdxDim));
    const int h = rem / kIdxDim, c = rem % kIdxDim;
    const float v = (q_dtype == CSA2_BF16) ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(idx_q)[i] << 16)
                                           : static_cast<const float*>(idx_q)[i];
    qf[r * H * kIdxDim + ((c >> 2) * H + h) * 4 + (c & 3)] = v;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nhist; i += stride) hist[i] = 0u;
}

// zero the approximate path's histograms and accumulators (three arrays and, if given, one word)
__global__ __launch_bounds__(256) void k_zero(uint32_t* __restrict__ x, int64_t nx, uint32_t* __restrict__ y,
                                              int64_t ny, uint32_t* __restrict__ z, int64_t nz,
                                              uint32_t* __restrict__ one) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nx; i += stride) x[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ny; i += stride) y[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nz; i += stride) z[i] = 0u;
  if (one && blockIdx.x == 0 && threadIdx.x == 0) *one = 0u;
}

struct ScoreArgs {
  int H;
  const void* idx_k;
  const uint8_t* idx_ks;      // MXFP4 keys: E8M0 scales [rows][2]
  const int64_t* row_start;
  const int32_t* row_visible;
  int max_visible;
  const int32_t* pool;        // Reindex
  const int32_t* pool_len;
  int pool_stride;
  float* scores;              // [R][n_pad]
  int64_t n_pad;
  float* bmax;                // [R][nb_pad]
  int64_t nb_pad;
  uint32_t* hist_s;           // [R][kD1]
  uint32_t* hist_b;           // [R][kD1]
  int tiles_per_wg;
  const uint32_t* row_list;   // non-null: grid row i scores rows row_list[i], row_list[i + gridDim.y], ...
  const uint32_t* row_count;  //   (of *row_count listed rows)
  int shared_start;           // every row reads the segment at row_start[0]
};

template <int KDT>
struct Staged {
  u32x4 v[KeyTile<KDT>::kPerLane];
  uint32_t sc;  // MXFP4: the two scale bytes of this lane's key
  int32_t pos;  // Reindex: the entry position of this lane's own slot (-1: none)
};

// E8M0 byte -> 2^(b - 127) as fp32 (b = 0: the subnormal 2^-127); the codec never writes 255
__device__ __forceinline__ float e8m0_f(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

// First-digit histograms are kept as packed 16-bit counters (two bins per
// word): a workgroup scores at most 255 x 256 entries, so no counter overflows.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin) { atomicAdd(&h[bin >> 1], 1u << (16 * (bin & 1))); }

__device__ __forceinline__ void flush_packed(uint32_t* __restrict__ g, const uint32_t* __restrict__ l) {
  for (int w = threadIdx.x; w < kD1 / 2; w += blockDim.x) {
    const uint32_t v = l[w];
    if (v & 0xFFFFu) atomicAdd(g + 2 * w, v & 0xFFFFu);
    if (v >> 16) atomicAdd(g + 2 * w + 1, v >> 16);
  }
}

// HC: compile-time head count (0 = runtime a.H, at most 32).  Full reads the
// prepared fp32 queries (qsrc: [row][channel quad][head][4]); Reindex reads the
// caller's queries as they are (qsrc: [row][head][64] of dtype QDT), so it needs
// no preparation kernel, and builds no histogram (its selection counts the
// pool's scores itself).
// One workgroup scores the slots [tile0 * 256, (tile0 + ntl) * 256) of row r (clipped to the row):
// wave w takes the 64-key tiles w, w + 4, ...  Returns early (the whole workgroup) when the range
// holds no slot.
template <int KDT, int HC, bool REINDEX, bool POOL, int QDT>
__device__ __forceinline__ void score_rows(const ScoreArgs& a, const void* __restrict__ qsrc, uint8_t* smem, int r,
                                           int64_t tile0, int ntl) {
  using T = KeyTile<KDT>;
  constexpr int NACC = HC > 0 ? HC : kMaxHeads;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint8_t* tile = smem + wv * T::kWaveBytes;                                       // this wave's rows
  uint32_t* h1 = reinterpret_cast<uint32_t*>(smem + kWavesPerWG * T::kWaveBytes);  // kD1/2 packed
  uint32_t* hb = h1 + kD1 / 2;                                                     // kD1/2 packed (POOL)
  // queries [quad][head][4]: after the histograms (Full), or where they would start (Reindex has none)
  float* sq = reinterpret_cast<float*>(REINDEX ? h1 : hb + (POOL ? kD1 / 2 : 0));

  const int H = HC > 0 ? HC : a.H;
  const int vis = clampv(a.row_visible[r], a.max_visible);
  int plen = 0;
  if (REINDEX) plen = a.pool_len ? clampv(a.pool_len[r], a.pool_stride) : a.pool_stride;
  const int n = REINDEX ? plen : vis;  // slots scored: Reindex, the pool's valid length
  const int64_t base0 = tile0 * kWGKeys;
  if (base0 >= n) return;
  const int ntiles = (int)std::min<int64_t>(ntl, ceil_div(n - base0, kWGKeys));
  if (!REINDEX) {
    for (int b = threadIdx.x; b < kD1 / 2; b += kThreads) {
      h1[b] = 0u;
      if (POOL) hb[b] = 0u;
    }
  }
  // Reindex and MXFP4 keys: the row's queries to LDS as fp32 in [channel quad][head][4] order (Full: the
  // prepared block, already in that order; Reindex: the caller's [head][64] queries, bf16 widened): every
  // lane reads a quad's H x 4 values as same-address (broadcast) LDS loads, which the compiler issues
  // ahead of their use.  Full over bf16 / fp32 keys, whose key rows already come from LDS, keeps scalar
  // loads of the prepared block (measured: LDS queries there halve its rate), and so does Reindex over
  // such keys when a prepared block exists (QDT = kQPrepared: the prefill rescoring).
  constexpr bool kLdsQ = (REINDEX && QDT != kQPrepared) || T::kMx;
  for (int i = threadIdx.x; kLdsQ && i < H * kIdxDim; i += kThreads) {
    float v;
    if constexpr (REINDEX) {
      const int h = i / kIdxDim, c = i % kIdxDim;
      const int64_t at = ((int64_t)r * H + h) * kIdxDim + c;
      v = QDT == CSA2_BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(qsrc)[at] << 16)
                           : static_cast<const float*>(qsrc)[at];
      sq[((c >> 2) * H + h) * 4 + (c & 3)] = v;
    } else {
      sq[i] = static_cast<const float*>(qsrc)[(int64_t)r * H * kIdxDim + i];
    }
  }
  __syncthreads();
  const int64_t rs = a.row_start[a.shared_start ? 0 : r];
  const uint8_t* kbase = static_cast<const uint8_t*>(a.idx_k);
  float* srow = a.scores + (int64_t)r * a.n_pad;
  const int32_t* prow = REINDEX ? a.pool + (int64_t)r * a.pool_stride : nullptr;

  // entry position of slot i (Full: the slot itself; Reindex: the pool entry), -1 if invalid
  auto position = [&](int64_t i) -> int64_t {
    if (REINDEX) {
      const int p = (i < plen) ? prow[i] : -1;
      return (p >= 0 && p < vis) ? p : -1;
    }
    return i < vis ? i : -1;
  };
  // piece id = lane + 64*i -> key id / kPieces, piece id % kPieces (coalesced 16-byte pieces).
  // Slots without a visible entry load some valid key row instead (Full: the
  // last visible one; Reindex: row 0 of the key array) and their scores are
  // discarded below; the loaded values are not inspected here, so the loads
  // of the next tile stay in flight while the current one is scored.
  auto load_tile = [&](int64_t base, Staged<KDT>& st) {
    if constexpr (T::kMx) {
      // own key: slot base + lane (Full: clamped to the last visible entry; Reindex: its pool entry, else row 0)
      int64_t row;
      if (!REINDEX) {
        row = rs + std::min<int64_t>(base + lane, (int64_t)vis - 1);
      } else {
        st.pos = (int32_t)position(base + lane);
        row = st.pos >= 0 ? rs + st.pos : 0;
      }
      const u32x4* pc = reinterpret_cast<const u32x4*>(kbase + row * 32);
      st.v[0] = __builtin_nontemporal_load(pc);
      st.v[1] = __builtin_nontemporal_load(pc + 1);
      st.sc = *reinterpret_cast<const uint16_t*>(a.idx_ks + row * 2);
      return;
    }
    if (!REINDEX) {
      // Full: 32-bit offsets into the row's key segment (at most 2^21 entries of 256 bytes)
      const uint8_t* kseg = kbase + rs * T::kBytes;
      if (base + T::kKeys <= vis) {
        // a wholly visible tile: piece i of this lane is 1 KiB after piece i-1
        const uint32_t off0 = (uint32_t)(base + lane / T::kPieces) * T::kBytes + (lane % T::kPieces) * 16u;
#pragma unroll
        for (int i = 0; i < T::kPerLane; ++i)
          st.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kseg + off0 + 1024u * i));
      } else {
#pragma unroll
        for (int i = 0; i < T::kPerLane; ++i) {
          const int id = lane + 64 * i;
          const uint32_t row = (uint32_t)std::min<int64_t>(base + id / T::kPieces, (int64_t)vis - 1);
          st.v[i] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(kseg + row * T::kBytes + (id % T::kPieces) * 16u));
        }
      }
      return;
    }
    // Reindex: each lane reads its own slot's pool entry once; the lanes loading a key's pieces take it
    // from that lane
    st.pos = (int32_t)position(base + lane);
#pragma unroll
    for (int i = 0; i < T::kPerLane; ++i) {
      const int id = lane + 64 * i;
      const int k = id / T::kPieces, piece = id % T::kPieces;
      const int32_t pos = __shfl(st.pos, k, 64);
      const int64_t row = pos >= 0 ? rs + pos : 0;
      st.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + row * T::kBytes) + piece);
    }
  };

  // wave tiles of this workgroup: wave wv takes tiles wv, wv + 4, ... (64 keys each); the
  // next tile's loads are in flight while the current one is scored
  const int nwt = (int)std::min<int64_t>((int64_t)ntiles * kWavesPerWG, ceil_div(n - base0, T::kKeys));
  auto tile_base = [&](int j) { return base0 + (int64_t)j * T::kKeys; };
  auto score_tile = [&](int j, Staged<KDT>& st) {
    const int64_t base = tile_base(j);
    const int32_t own = st.pos;  // (st is refilled with the next tile below)
    u32x4 mc[2] = {st.v[0], st.v[T::kPerLane > 1 ? 1 : 0]};  // MXFP4: this key's codes, kept in registers
    float mx0 = 0.0f, mx1 = 0.0f;                             // MXFP4: the two block scales
    if constexpr (T::kMx) {
      mx0 = e8m0_f(st.sc & 0xFFu);
      mx1 = e8m0_f(st.sc >> 8);
    } else {
      // (the LDS operations of one wave execute in order: the previous tile's reads are done)
#pragma unroll
      for (int i = 0; i < T::kPerLane; ++i) {
        const int id = lane + 64 * i;
        *reinterpret_cast<u32x4*>(tile + (id / T::kPieces) * T::kStride + (id % T::kPieces) * 16) = st.v[i];
      }
    }
    if (j + kWavesPerWG < nwt) load_tile(tile_base(j + kWavesPerWG), st);

    // the H fmaf chains of key `lane`, channels in order
    float acc[NACC];
#pragma unroll
    for (int h = 0; h < NACC; ++h) acc[h] = 0.0f;
    const uint8_t* row = tile + lane * T::kStride;
#pragma unroll(T::kMx ? 16 : 2)  // MXFP4: full, so the code words stay in registers
    for (int c4 = 0; c4 < 16; ++c4) {
      float kv[4];
      if constexpr (T::kMx) {
        // channels 4 c4 .. +3: code bytes 2 c4, 2 c4 + 1 (low nibble first), block c4 / 8
        const uint32_t wd = mc[c4 >> 3][(c4 >> 1) & 3] >> (16 * (c4 & 1));  // its two bytes, low half
        const float X = c4 < 8 ? mx0 : mx1;
        const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 0);
        const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 1);
        kv[0] = __fmul_rn(lo[0], X);
        kv[1] = __fmul_rn(lo[1], X);
        kv[2] = __fmul_rn(hi[0], X);
        kv[3] = __fmul_rn(hi[1], X);
      } else if (KDT == CSA2_BF16) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(row + c4 * 8);
        kv[0] = __uint_as_float(w[0] << 16);
        kv[1] = __uint_as_float(w[0] & 0xFFFF0000u);
        kv[2] = __uint_as_float(w[1] << 16);
        kv[3] = __uint_as_float(w[1] & 0xFFFF0000u);
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(row + c4 * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[e] = __uint_as_float(w[e]);
      }
      // the H x 4 query values of this channel quad: broadcast LDS loads
      const float* qrow = kLdsQ ? sq + c4 * H * 4 : static_cast<const float*>(qsrc) + (int64_t)r * H * kIdxDim + c4 * H * 4;
      if constexpr (HC > 0) {
#pragma unroll
        for (int h = 0; h < HC; ++h) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[h] = __builtin_fmaf(qrow[h * 4 + e], kv[e], acc[h]);
        }
      } else {
#pragma unroll
        for (int h = 0; h < kMaxHeads; ++h) {
          if (h < H) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[h] = __builtin_fmaf(qrow[h * 4 + e], kv[e], acc[h]);
          }
        }
      }
    }
    // ReLU as an integer max on the bits: a positive float keeps its bits,
    // anything else (negative, -0) becomes +0, exactly x > 0 ? x : 0
    auto relu = [](float x) { return __int_as_float(max(__float_as_int(x), 0)); };
    float sc = relu(acc[0]);
#pragma unroll
    for (int h = 1; h < NACC; ++h)
      if (HC > 0 || h < H) sc = __fadd_rn(sc, relu(acc[h]));
    const int64_t i = base + lane;
    const bool ok = REINDEX ? own >= 0 : i < vis;
    if (i < n) srow[i] = ok ? sc : -1.0f;
    if (!REINDEX && ok) hist_add(h1, __float_as_uint(sc) >> kS1);
    if (POOL) {
      // a block of 8 consecutive positions = 8 consecutive lanes; scores are
      // >= +0 or -1.0 (invalid), so their bits order like int32
      int m = __float_as_int(ok ? sc : -1.0f);
      m = max(m, __shfl_xor(m, 1, 64));
      m = max(m, __shfl_xor(m, 2, 64));
      m = max(m, __shfl_xor(m, 4, 64));
      if (ok && (lane & 7) == 0) {
        a.bmax[(int64_t)r * a.nb_pad + i / kBlock] = __int_as_float(m);
        hist_add(hb, (uint32_t)m >> kS1);
      }
    }
  };
  if (wv < nwt) {
    Staged<KDT> st;
    load_tile(tile_base(wv), st);
    for (int j = wv; j < nwt; j += kWavesPerWG) score_tile(j, st);
  }
  if (REINDEX) return;
  __syncthreads();
  flush_packed(a.hist_s + (int64_t)r * kD1, h1);
  if (POOL) flush_packed(a.hist_b + (int64_t)r * kD1, hb);
}

template <int KDT, int HC, bool REINDEX, bool POOL, int QDT>
__global__ __launch_bounds__(kThreads, 3) void k_score(ScoreArgs a, const void* __restrict__ qsrc) {
  extern __shared__ __align__(16) uint8_t smem[];
  int r = (int)blockIdx.y;
  if (a.row_list) {  // grid row i scores the i-th listed row, if there is one
    if (blockIdx.y >= *a.row_count) return;
    r = (int)a.row_list[blockIdx.y];
  }
  score_rows<KDT, HC, REINDEX, POOL, QDT>(a, qsrc, smem, r, (int64_t)blockIdx.x * a.tiles_per_wg, a.tiles_per_wg);
}

// Full over rows of different lengths: the grid's workgroups share the batch's 256-entry tiles
// evenly (about 1/gridDim.x of them each, in row order), so short rows leave no workgroup idle.
// Each workgroup takes the row lengths (at most 256 rows, one per thread), their tile prefix sums,
// and scores its range row segment by row segment, flushing each row's histograms.
template <int KDT, int HC, bool POOL>
__global__ __launch_bounds__(kThreads, 3) void k_scan_even(ScoreArgs a, const void* __restrict__ qsrc, int R) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t xs[8];
  const int i = threadIdx.x;
  const uint32_t tl = i < R ? (uint32_t)ceil_div(clampv(a.row_visible[i], a.max_visible), kWGKeys) : 0u;
  uint32_t total;
  const uint32_t ex = block_excl_sum<kThreads>(tl, xs, &total);
  uint32_t cur = (uint32_t)((uint64_t)total * blockIdx.x / gridDim.x);
  const uint32_t end = (uint32_t)((uint64_t)total * (blockIdx.x + 1) / gridDim.x);
  while (cur < end) {
    if (tl > 0u && ex <= cur && cur < ex + tl) {  // the row holding tile `cur`
      xs[4] = (uint32_t)i;
      xs[5] = ex;
      xs[6] = ex + tl;
    }
    __syncthreads();
    const int r = (int)xs[4];
    const uint32_t lo = xs[5], seg = min(end, xs[6]);
    __syncthreads();
    score_rows<KDT, HC, false, POOL, CSA2_F32>(a, qsrc, smem, r, (int64_t)(cur - lo), (int)(seg - cur));
    __syncthreads();  // (the histogram flush has read the LDS counters before the next segment zeroes them)
    cur = seg;
  }
}

struct Series {
  const float* arr;      // [R, stride] keys (sign bit set = invalid)
  int64_t stride;
  const uint32_t* hist;  // [R, kD1] first-digit histogram of the scores
  uint32_t* thr;         // [R, 2] Full: threshold bin (-1: fewer than K valid) and the count above it
  float* cand_key;       // [R, 2*stride] candidate keys (Full): per-slice lists, then the packed list
  int32_t* cand_pos;     // [R, 2*stride] candidate positions (Full)
  uint32_t* counts;      // [R, nsub] candidates per slice (Full)
  int nsub;              // slices of kSub elements
  int K;
};

struct SelArgs {
  Series s[2];
  int nseries;
  int mode;
  const int32_t* row_visible;
  int max_visible;
  int pool_stride;
  const int32_t* pool;
  int32_t* out_idx;      // [R, K]
  int32_t* out_pool;     // [R, pool_size]
  int32_t* out_pool_len; // [R]
  int pool_size;
  const int32_t* pool_len;   // Reindex: valid slots per row (null = pool_stride)
  const uint32_t* row_list;  // non-null: grid row i selects for rows row_list[i], row_list[i + grid rows], ...
  const uint32_t* row_count; //   (of *row_count listed rows)
  int by_len;                // Reindex: split each row by its valid slots, not its capacity
  // the prefill rescoring's certification (null: none): a row whose exact selection does not prove the
  // sampled bound cert_thi[r] is appended to cert_list (count *cert_count) with its first-digit histogram
  // cert_xhist[r] zeroed, for the exact fallback that follows
  const float* cert_thi;
  uint32_t* cert_list;
  uint32_t* cert_count;
  uint32_t* cert_xhist;
};

__device__ __forceinline__ int series_len(const SelArgs& a, int series, int r) {
  if (a.mode == CSA2_REINDEX) return a.pool_len ? clampv(a.pool_len[r], a.pool_stride) : a.pool_stride;
  const int v = clampv(a.row_visible[r], a.max_visible);
  return series == 0 ? v : (v + kBlock - 1) / kBlock;
}

constexpr int kFinCap = 16384;  // candidates a finalize workgroup keeps in LDS (16 per thread)

// where candidate c of a row's list sits in its source arrays: Full, slice
// lo = the largest s with pre[s] <= c (a fixed-step search without branches)
__device__ __forceinline__ int64_t fin_src(bool full, int nsub, const uint32_t* pre, uint32_t c) {
  if (!full) return c;
  int lo = 0;
#pragma unroll
  for (int step = 512; step > 0; step >>= 1) {
    const int t = lo + step;
    lo = (t <= nsub && pre[min(t, nsub)] <= c) ? t : lo;
  }
  return (int64_t)lo * kSub + (c - pre[lo]);
}

// Loads the candidates [w0, w1) of this wave (MAXCH chunks of 64, all loads
// in flight together: slots past the run read entry 0 of the row and, like
// slots at or past nvalid, are masked afterwards), finds the first digit for
// Reindex (its barriers wait for the loads), then keeps, in order, the valid
// candidates whose first digit reaches it: they go to lkey/lpos[w0 ...].
// Returns their count.
template <int NT, int MAXCH>
__device__ __forceinline__ uint32_t fin_gather(const Series& S, int r, bool full, int nsub, const uint32_t* pre,
                                              const uint32_t* sk, const int32_t* sp, uint32_t w0, uint32_t w1,
                                              uint32_t nvalid, int& b0, uint32_t& above0, uint32_t* red,
                                              uint32_t* lkey, int32_t* lpos) {
  const int lane = threadIdx.x & 63;
  const int nch = (int)((w1 - w0 + 63u) / 64u);
  uint32_t kr[MAXCH];
  int32_t pr[MAXCH];
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const uint32_t c = w0 + 64u * j + lane;
    const int64_t at = (j < nch && c < w1) ? fin_src(full, nsub, pre, c) : 0;
    kr[j] = sk[at];
    pr[j] = sp[at];
  }
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const uint32_t c = w0 + 64u * j + lane;
    kr[j] = (j < nch && c < w1 && c < nvalid) ? kr[j] : 0x80000000u;
  }
  if (!full) {
    // Reindex: the first-digit histogram of the row's valid scores, counted here
    // in the candidate area (written only after find_bin has read it)
    for (int b = threadIdx.x; b < kD1; b += NT) lkey[b] = 0u;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < MAXCH; ++j)
      if (!(kr[j] >> 31)) atomicAdd(&lkey[kr[j] >> kS1], 1u);
    lds_barrier();
    uint32_t total0;
    b0 = find_bin_wave<kD1>(lkey, (uint32_t)S.K, &above0, &total0, red);
  }
  const uint32_t lo_key = b0 < 0 ? 0u : ((uint32_t)b0 << kS1);  // smaller keys cannot be selected
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const bool keep = !(kr[j] >> 31) && kr[j] >= lo_key;
    const unsigned long long m = __ballot(keep);
    if (keep) {
      const uint32_t at =
          w0 + cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      lkey[at] = kr[j];
      lpos[at] = pr[j];
    }
    cnt += (uint32_t)__popcll(m);
  }
  return cnt;
}

// The prefill rescoring's certification of the sampled bound thi, taken on the exact scores: if at
// least K candidates have an exact score of at least thi, the K-th largest exact score over all
// entries is at least thi, so every entry of the exact top-K (ties included) has A + eps >= thi - eps_max
// and is a candidate.  That holds when the K-th largest exact candidate score T reaches thi (scores are
// non-negative, so their bits order like the values), or, with fewer than K candidates, when every
// visible entry is one.  A row that fails joins the exact fallback's list, its first-digit histogram
// zeroed here (before that scan); rows whose candidates overflowed (count -1) are on the list already.
template <int NT>
__device__ __forceinline__ void certify_row(const SelArgs& a, int r, int n, int vis, bool all, uint32_t T,
                                            uint32_t* flag) {
  if (threadIdx.x == 0) {
    bool ok = true;
    if (a.pool_len[r] >= 0 && vis > 0) ok = all ? n >= vis : T >= __float_as_uint(a.cert_thi[r]);
    if (!ok) a.cert_list[atomicAdd(a.cert_count, 1u)] = (uint32_t)r;
    *flag = ok ? 1u : 0u;
  }
  __syncthreads();
  if (*flag == 0u) {
    u32x4* h = reinterpret_cast<u32x4*>(a.cert_xhist + (int64_t)r * kD1);
    for (int i = threadIdx.x; i < kD1 / 4; i += NT) h[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Exact selection for one (row, series) by one workgroup of NT threads.
// The first radix digit comes from the scan's histogram (Full: the bin
// k_collect used; Reindex: found here).  Candidates: Full -> the per-slice
// lists written by k_collect, in slice order; Reindex -> every pool slot.
// Wave w owns the candidates [w0, w1) of that order.  Up to kFinCap of them
// are loaded at once and only those that can still be selected are kept, in
// order, in LDS (each wave then works on its own run); beyond kFinCap
// (massive ties, very large pools) they are read from global memory, a Full
// row's list first packed into the second half of its candidate arrays.
// Two more digits give the exact K-th largest key T; the ordered compaction
// then writes positions ascending, taking ties at T in candidate order
// (= ascending position), and pads with -1.
template <int NT, int series, int CAP = kFinCap>
__device__ __forceinline__ void finalize_row(const SelArgs& a, int r, uint32_t* hist, uint32_t* hist2,
                                             uint32_t* pre,
                             uint32_t* red, uint32_t* lkey, int32_t* lpos) {
  constexpr int NW = NT / 64;
  const Series& S = a.s[series];
  const int n = series_len(a, series, r);
  const bool full = a.mode == CSA2_FULL;
  const int vis = clampv(a.row_visible[r], a.max_visible);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the two digit histograms start at zero (ordered by the barriers below)
  for (int b = threadIdx.x; b < NT; b += NT) hist[b] = 0u;
  for (int b = threadIdx.x; b < kD2; b += NT) hist2[b] = 0u;
  uint32_t M;
  uint32_t above0 = 0;
  int b0 = -1;
  int nsub = 0;
  const uint32_t* sk;
  const int32_t* sp;
  // Full with at most kSpec slices per wave: wave w owns slices [s_lo, s_hi) of the row's candidate
  // lists (k_collect wrote slice s's candidates, in position order, from offset s * kSub), and the
  // first 64 candidates of each are loaded before the slice counts have arrived
  constexpr int kSpec = 16;
  int s_lo = 0, s_hi = 0;
  bool by_slice = false;
  uint32_t kr[kSpec];
  int32_t pr[kSpec];
  if (full) {
    nsub = (n + kSub - 1) / kSub;
    sk = reinterpret_cast<const uint32_t*>(S.cand_key) + (int64_t)r * 2 * S.stride;
    sp = S.cand_pos + (int64_t)r * 2 * S.stride;
    const int spw = (nsub + NW - 1) / NW;
    by_slice = spw <= kSpec;
    s_lo = min(nsub, wave * spw);
    s_hi = min(nsub, s_lo + spw);
    // the slice counts first: the prefix sums wait for them alone, the candidate loads stay in flight
    const uint32_t c_first = ((int)threadIdx.x < nsub) ? S.counts[(int64_t)r * S.nsub + threadIdx.x] : 0u;
    if (by_slice) {
#pragma unroll
      for (int j = 0; j < kSpec; ++j) {
        const int sl = s_lo + j;
        const int64_t at = sl < s_hi ? (int64_t)sl * kSub + lane : 0;
        kr[j] = sk[at];
        pr[j] = sp[at];
      }
    }
    b0 = (int)S.thr[2 * r];
    above0 = S.thr[2 * r + 1];
    // pre[1027] (past the largest slice count's prefix) flags a slice of more than 64 candidates
    if (threadIdx.x == 0) pre[1027] = 0u;
    uint32_t carry = 0;
    for (int s0 = 0; s0 < nsub; s0 += NT) {
      const int s = s0 + threadIdx.x;
      const uint32_t c = s0 == 0 ? c_first : ((s < nsub) ? S.counts[(int64_t)r * S.nsub + s] : 0u);
      uint32_t tot;
      const uint32_t ex = block_excl_sum<NT, true>(c, red, &tot);  // (its barriers order the flag's reset)
      if (s < nsub) pre[s] = carry + ex;
      if (c > 64u) pre[1027] = 1u;
      carry += tot;
    }
    if (threadIdx.x == 0) pre[nsub] = carry;
    lds_barrier();
    M = pre[nsub];
    // candidates clustered in position (a slice of more than 64) leave the early loads short:
    // the row is then split evenly over the waves instead
    by_slice = by_slice && pre[1027] == 0u;
  } else {
    // the row is split by its pool capacity when that fits, so the candidate
    // loads need not wait for the pool length (slots past it are masked);
    // sparsely filled lists (the prefill candidates) by their length instead
    M = (a.pool_stride <= CAP && !a.by_len) ? (uint32_t)a.pool_stride : (uint32_t)n;
    sk = reinterpret_cast<const uint32_t*>(S.arr) + (int64_t)r * S.stride;
    sp = a.pool + (int64_t)r * a.pool_stride;
  }
  const uint32_t per_w = ((M + NW - 1) / NW + 63u) & ~63u;
  uint32_t w0 = min(M, (uint32_t)wave * per_w);
  const uint32_t w1 = min(M, w0 + per_w);
  // The threshold digits and the ordered compaction over this wave's run [w0, cend) of keys/posr,
  // instantiated once for candidates in LDS and once for candidates in global memory: a pointer that
  // could be either would turn every access into a flat one, whose waits also cover the global stores
  // in flight.
  auto phases = [&](const uint32_t* keys, const int32_t* posr, const uint32_t cend, auto in_lds) {
    // ---- exact threshold: digits 2 and 3 among the candidates of the first digit's bin
    uint32_t need = 0;
    uint32_t prefix = 0;
    const bool all = b0 < 0;  // fewer than K valid entries: every valid candidate is selected
    if (!all) {
      uint32_t K = (uint32_t)S.K - above0;
      prefix = (uint32_t)b0;
      int shift_hi = kS1;
  #pragma unroll 1
      for (int lev = 1; lev < 3; ++lev) {
        const int sh = lev == 1 ? kS2 : 0;
        const int nb = lev == 1 ? kD2 : kD3;
        uint32_t* h = lev == 1 ? hist2 : hist;
  #pragma unroll 4
        for (uint32_t c = w0 + lane; c < cend; c += 64) {
          const uint32_t key = keys[c];
          if (!(key >> 31) && (key >> shift_hi) == prefix) atomicAdd(&h[(key >> sh) & (nb - 1)], 1u);
        }
        lds_barrier();
        uint32_t above, total;
        const int b = lev == 1 ? find_bin_wave<kD2>(hist2, K, &above, &total, red)
                               : find_bin_wave<kD3>(hist, K, &above, &total, red);
        prefix = (prefix << (shift_hi - sh)) | (uint32_t)b;
        shift_hi = sh;
        K -= above;
      }
      need = K;  // ties at T to take, in candidate order
    }
    const uint32_t T = prefix;  // the full 31-bit key of the K-th largest
    // (the prefill rescoring: pre[] is unused by Reindex rows, its word 1026 carries the verdict)
    if (a.cert_thi) certify_row<NT>(a, r, n, vis, all, T, pre + 1026);

    // ---- ordered compaction over each wave's run, 64 candidates at a time
    auto is_gt = [&](uint32_t key) { return !(key >> 31) && (all || key > T); };
    auto is_eq = [&](uint32_t key) { return !(key >> 31) && !all && key == T; };
    uint32_t gt = 0, eq = 0;
    for (uint32_t c0 = w0; c0 < cend; c0 += 64) {
      const uint32_t c = c0 + lane;
      const uint32_t key = c < cend ? keys[c] : 0x80000000u;
      gt += (uint32_t)__popcll(__ballot(is_gt(key)));
      eq += (uint32_t)__popcll(__ballot(is_eq(key)));
    }
    if (lane == 0) {
      red[wave] = gt;
      red[NW + wave] = eq;
    }
    lds_barrier();
    uint32_t gt_before = 0, eq_before = 0, tot_gt = 0;
  #pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const uint32_t g = red[ww], e = red[NW + ww];
      gt_before += ww < wave ? g : 0u;
      eq_before += ww < wave ? e : 0u;
      tot_gt += g;
    }
    lds_barrier();
    const uint32_t nsel = all ? tot_gt : (uint32_t)S.K;
    uint32_t out = gt_before + (all ? 0u : min(eq_before, need));
    uint32_t ties = eq_before;
    bool last_block_kept = false;
    for (uint32_t c0 = w0; c0 < cend; c0 += 64) {
      const uint32_t c = c0 + lane;
      const bool in = c < cend;
      const uint32_t key = in ? keys[c] : 0x80000000u;
      // in LDS the position is read with the key (one wait for both); in global memory only for the
      // selected candidates
      int32_t pos = 0;
      if constexpr (decltype(in_lds)::value) pos = posr[in ? c : w0];
      const bool e = is_eq(key);
      const unsigned long long me = __ballot(e);
      const uint32_t rank =
          ties + __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
      const bool sel = is_gt(key) || (e && rank < need);
      const unsigned long long ms = __ballot(sel);
      const uint32_t at =
          out + __builtin_amdgcn_mbcnt_hi((uint32_t)(ms >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ms, 0u));
      if (sel && at < nsel) {
        if constexpr (!decltype(in_lds)::value) pos = posr[c];
        if constexpr (series == 0) {
          a.out_idx[(int64_t)r * S.K + at] = pos;
        } else {
          int32_t* o = a.out_pool + (int64_t)r * a.pool_size + (int64_t)at * kBlock;
  #pragma unroll
          for (int m = 0; m < kBlock; ++m) o[m] = (pos * kBlock + m < vis) ? pos * kBlock + m : -1;
          if (pos == n - 1) last_block_kept = true;
        }
      }
      out += (uint32_t)__popcll(ms);
      ties += (uint32_t)__popcll(me);
    }
    // ---- padding and pool length
    if constexpr (series == 0) {
      int32_t* o = a.out_idx + (int64_t)r * S.K;
      for (int i = (int)nsel + threadIdx.x; i < S.K; i += NT) o[i] = -1;
    } else {
      if (threadIdx.x == 0) red[0] = 0u;
      lds_barrier();
      if (last_block_kept) red[0] = 1u;
      lds_barrier();
      // the partial last block is the highest block, hence the last one written
      int plen = (int)nsel * kBlock;
      if (red[0] && (vis % kBlock) != 0) plen -= kBlock - (vis % kBlock);
      int32_t* o = a.out_pool + (int64_t)r * a.pool_size;
      for (int i = (int)nsel * kBlock + threadIdx.x; i < a.pool_size; i += NT) o[i] = -1;
      if (threadIdx.x == 0) a.out_pool_len[r] = plen;
    }
  };
  if (M <= (uint32_t)CAP) {
  if (by_slice) {
    // candidate c of the row's order sits at LDS slot c: the wave's run is [pre[s_lo], pre[s_hi]);
    // every collected candidate reaches the threshold bin, so all are kept
#pragma unroll
    for (int j = 0; j < kSpec; ++j) {
      const int sl = s_lo + j;
      if (sl < s_hi) {
        const uint32_t base = pre[sl], cs = pre[sl + 1] - base;
        if ((uint32_t)lane < cs) {
          lkey[base + lane] = kr[j];
          lpos[base + lane] = pr[j];
        }
      }
    }
    w0 = pre[s_lo];
    phases(lkey, lpos, pre[s_hi], std::true_type{});
  } else {
    const int nchmax = (int)(per_w / 64u);  // uniform
    const uint32_t nv = full ? M : (uint32_t)n;  // Reindex: the valid slots
    uint32_t sw;
    if (nchmax <= 2) sw = fin_gather<NT, 2>(S, r, full, nsub, pre, sk, sp, w0, w1, nv, b0, above0, red, lkey, lpos);
    else if (nchmax <= 4) sw = fin_gather<NT, 4>(S, r, full, nsub, pre, sk, sp, w0, w1, nv, b0, above0, red, lkey, lpos);
    else if (nchmax <= 8) sw = fin_gather<NT, 8>(S, r, full, nsub, pre, sk, sp, w0, w1, nv, b0, above0, red, lkey, lpos);
    else sw = fin_gather<NT, 16>(S, r, full, nsub, pre, sk, sp, w0, w1, nv, b0, above0, red, lkey, lpos);
    // (each wave reads back only its own run; LDS operations of a wave execute in order)
    phases(lkey, lpos, w0 + sw, std::true_type{});
  }
  } else {
    const uint32_t* gk;
    const int32_t* gp;
    if (full) {
      uint32_t* dk = reinterpret_cast<uint32_t*>(S.cand_key) + (int64_t)r * 2 * S.stride + S.stride;
      int32_t* dp = S.cand_pos + (int64_t)r * 2 * S.stride + S.stride;
#pragma unroll 4
      for (uint32_t c = threadIdx.x; c < M; c += NT) {
        const int64_t at = fin_src(full, nsub, pre, c);
        dk[c] = sk[at];
        dp[c] = sp[at];
      }
      __syncthreads();
      gk = dk;
      gp = dp;
    } else {
      // Reindex beyond the LDS capacity: the first-digit histogram from the scores in place
      for (int b = threadIdx.x; b < kD1; b += NT) lkey[b] = 0u;
      __syncthreads();
      for (int c = threadIdx.x; c < n; c += NT) {
        const uint32_t key = sk[c];
        if (!(key >> 31)) atomicAdd(&lkey[key >> kS1], 1u);
      }
      __syncthreads();
      uint32_t total0;
      b0 = find_bin_wave<kD1>(lkey, (uint32_t)S.K, &above0, &total0, red);
      gk = sk;
      gp = sp;
    }
    phases(gk, gp, w1, std::false_type{});
  }
}

// Full mode: each wave compacts its slice of kSub elements, keeping those
// whose first digit is at least the threshold bin (all valid ones when the
// row holds fewer than K).
__device__ __forceinline__ void collect_row(const SelArgs& a, int series, int r, uint32_t* red) {
  const Series& S = a.s[series];
  const int n = series_len(a, series, r);
  const int64_t wg_base = (int64_t)blockIdx.x * 4 * kSub;
  if (wg_base >= n && blockIdx.x != 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = wg_base + (int64_t)wave * kSub;
  const int end = (int)std::min<int64_t>(n, base + kSub);  // <= base for a wave past the end
  const float* arr = S.arr + (int64_t)r * S.stride;
  // the slice's keys are in flight while the threshold bin is found
  constexpr int kPer = kSub / 64;  // 32 elements per lane
  const int last = n > 0 ? n - 1 : 0;  // the row's score array holds at least kSub slots
  float v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = (int)base + 64 * k + lane;
    v[k] = arr[i < end ? i : last];
  }
  uint32_t above, total;
  const int b1 = find_bin<kThreads, kD1>(S.hist + (int64_t)r * kD1, (uint32_t)S.K, &above, &total, red);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    S.thr[2 * r] = (uint32_t)b1;
    S.thr[2 * r + 1] = above;
  }
  const uint32_t thr = b1 < 0 ? 0u : (uint32_t)b1;
  if (base >= n) return;
  const int sub = (int)(base / kSub);
  float* ck = S.cand_key + (int64_t)r * 2 * S.stride + base;
  int32_t* cp = S.cand_pos + (int64_t)r * 2 * S.stride + base;
  uint32_t cnt = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = (int)base + 64 * k + lane;
    const uint32_t key = __float_as_uint(v[k]);
    const bool take = i < end && !(key >> 31) && (key >> kS1) >= thr;
    const unsigned long long m = __ballot(take);
    if (take) {
      const uint32_t at = cnt + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      ck[at] = v[k];
      cp[at] = i;
    }
    cnt += (uint32_t)__popcll(m);
  }
  if (lane == 0) S.counts[(int64_t)r * S.nsub + sub] = cnt;
}

// LIST: the rows of a device-side list (a grid of at most kListRows rows, looping over the list),
// else grid row r collects for row r
template <bool LIST>
__global__ __launch_bounds__(kThreads) void k_collect(SelArgs a) {
  __shared__ uint32_t red[32];
  const int series = blockIdx.z;
  if (series >= a.nseries) return;
  if constexpr (!LIST) {
    collect_row(a, series, (int)blockIdx.y, red);
  } else {
    const uint32_t nl = *a.row_count;
    for (uint32_t li = blockIdx.y; li < nl; li += gridDim.y) {
      collect_row(a, series, (int)a.row_list[li], red);
      __syncthreads();  // (red reused by the next listed row)
    }
  }
}

constexpr size_t kFinLdsWords = kFinThreads + kD2 + 1028 + 32 + 2 * (size_t)kFinCap;

__global__ __launch_bounds__(kFinThreads) void k_finalize(SelArgs a) {
  extern __shared__ __align__(16) uint32_t fsm[];
  uint32_t* hist = fsm;                       // kFinThreads (last digit)
  uint32_t* hist2 = hist + kFinThreads;       // kD2 (second digit)
  uint32_t* pre = hist2 + kD2;                // 1025
  uint32_t* red = pre + 1028;                 // 32
  uint32_t* lkey = red + 32;                  // kFinCap
  int32_t* lpos = reinterpret_cast<int32_t*>(lkey + kFinCap);
  if ((int)blockIdx.y >= a.nseries) return;
  // one instantiation per series (entries, blocks), so neither carries the other's branches
  auto one = [&](int r) {
    if (blockIdx.y == 0) finalize_row<kFinThreads, 0>(a, r, hist, hist2, pre, red, lkey, lpos);
    else finalize_row<kFinThreads, 1>(a, r, hist, hist2, pre, red, lkey, lpos);
  };
  int r = (int)blockIdx.x;
  if (a.row_list) {  // workgroup i selects for the i-th listed row, if there is one
    if (blockIdx.x >= *a.row_count) return;
    r = (int)a.row_list[blockIdx.x];
  }
  one(r);
}

// The prefill rescoring's selection (Reindex over candidate lists split by their length, thousands of
// rows): 512-thread workgroups keeping up to 4,096 candidates in LDS, three per CU (at most 80 VGPRs),
// so three rows' selections overlap on every CU (a longer list is selected from global memory).
// Measured on the 4,096-row chunk: 3.48 -> 3.41 ms (two per CU at 87 VGPRs: 3.43 ms).
constexpr int kFinSmallThreads = 512;
constexpr int kFinSmallCap = 4096;
constexpr size_t kFinSmallLdsWords = kFinSmallThreads + kD2 + 1028 + 32 + 2 * (size_t)kFinSmallCap;

__global__ __launch_bounds__(kFinSmallThreads) __attribute__((amdgpu_waves_per_eu(6))) void k_finalize_small(SelArgs a) {
  extern __shared__ __align__(16) uint32_t fsm[];
  uint32_t* hist = fsm;
  uint32_t* hist2 = hist + kFinSmallThreads;
  uint32_t* pre = hist2 + kD2;
  uint32_t* red = pre + 1028;
  uint32_t* lkey = red + 32;
  int32_t* lpos = reinterpret_cast<int32_t*>(lkey + kFinSmallCap);
  finalize_row<kFinSmallThreads, 0, kFinSmallCap>(a, (int)blockIdx.x, hist, hist2, pre, red, lkey, lpos);
}

// ------------------------------------------------------------ prefill: approximate MFMA passes
//
// When every query row reads the same key segment (a prefill chunk over one
// cache), the indexer scores form a GEMM of (rows x heads) against keys.  The
// chunk's rows are first scored with bf16 MFMA (fp32 accumulate): one pass
// builds each row's first-digit histogram of the approximate scores A, a
// second pass marks as candidates every entry whose A could still belong to
// the exact top-K.  Let E be the exact score (the fmaf-chain definition) and
// S the real-number score.  The MFMA dot and the exact chain each differ from
// S by at most gamma_64 * sum_c |q_c k_c| per head, and the head sums by at
// most gamma_7 of their size, with gamma_n = n u / (1 - n u); u = 2^-23 covers
// any fp32 summation order with round-to-nearest or truncation.  By
// Cauchy-Schwarz sum_c |q_c k_c| <= |q_h| |k|, so
//   |A - E| <= eps_j = c |k_j| sum_h |q_h|,   c = 2 (gamma_64 + gamma_7 (1 + gamma_64)),
// taken here with further safety factors.  The bound lo(b), the lower edge
// of the histogram bin that holds a sampled order statistic of A, marks as
// candidates the entries with A_j + eps_j >= lo(b) - eps_max; they are
// rescored exactly and selected exactly.  The bound is proven afterwards, on
// the exact scores: if at least K candidates have E >= lo(b), every entry of
// the exact top-K (ties included) has E_j >= lo(b), so A_j + eps_j >= lo(b)
// and it is a candidate: the result is the exact top-K.  A row that fails that
// test, or whose candidates overflow the list, falls back to the exact full
// scan.

// query rows per workgroup of the approximate passes: each key a wave loads feeds
// every row of its workgroup (16 rows for up to 8 heads; 8 keep 16 heads in registers)
template <int H>
__host__ __device__ constexpr int pf_rows() { return H <= 8 ? 16 : 8; }
constexpr int kPfRange = 32768;  // keys per workgroup of the candidate pass
constexpr int kPfCap = 16384;    // candidates kept per row (more: exact fallback for that row)
constexpr int kPfSample = 16;    // the provisional bound samples every 16th 32-key step
// error constant c of the bound above for H heads, with a factor 8 of safety
// on top (so the margin stays valid even if an accumulator kept fewer bits)
__host__ __device__ constexpr float pf_err(int H) { return 16.0f * (64.0f + (float)H) * 1.1920929e-07f; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct PfArgs {
  const uint16_t* q;          // [R][H][64] bf16 indexer queries
  const uint8_t* k;           // indexer keys: bf16 rows of 128 bytes, or MXFP4 codes (32 bytes per key)
  const uint8_t* ks;          // MXFP4 keys: E8M0 scales [rows][2] (null: bf16 keys)
  const int64_t* row_start;   // segment start = row_start[0]
  const int32_t* row_visible; // [R]
  int max_visible;
  int R;
  int K;
  float* knorm;               // [max_visible] |k_j| bound
  uint32_t* kmax;             // [1] max |k_j| (float bits)
  float* qn;                  // [R] sum_h |q_h| bound
  uint32_t* hist;             // [R][kD1] first-digit histograms of A over a sample of the keys
  float* plo;                 // [R] candidate bound lo(b) - eps_max (+inf: no candidates, the exact fallback)
  float* thi;                 // [R] sampled bound lo(b) that the exact selection certifies
  int sample;                 // MODE 0: every sample-th 32-key step
  uint32_t target;            // entries the threshold bin must cover (K, or more for a sample)
  uint32_t* bits;             // [R][nwords] candidate bitmap
  int nwords;
  int32_t* cand;              // [R][kPfCap] candidate positions, ascending
  int32_t* ccnt;              // [R] candidates (-1 on overflow)
  uint32_t* over_list;        // [R] the rows for the exact fallback (candidates overflow, or the bound is not
                              // certified), in no particular order
  uint32_t* nover;            // their count (zeroed by the call's first kernels)
  uint32_t* xhist;            // [R][kD1] the exact path's first-digit histograms (zeroed for listed rows)
};

// max(x, +0) as one integer max: negative floats (sign bit set, -0 included) compare below 0
__device__ __forceinline__ float relu0(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// norms: one thread per key of the shared segment, then one per (row, head) query
// Key norms (MXFP4: one thread per key; bf16: eight lanes per key, 16 coalesced bytes each, summed
// across the eight lanes; the order of the sum does not matter for the bound: 64 terms of rounding
// stay far below the 1e-5 margin the norm is widened by) over a grid-stride loop, their maximum (one
// atomic per workgroup), and each row's sum of query-head norms (one thread per row and head).
__global__ __launch_bounds__(256) void k_pf_norms(PfArgs a, int H) {
  __shared__ uint32_t wmax[4];
  const int64_t seg = a.row_start[0];
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t m = 0u;  // largest norm seen (non-negative floats order like their bits)
  if (!a.ks) {
    const int64_t nthreads = ((int64_t)a.max_visible * 8 + 63) & ~int64_t(63);  // whole waves
    for (int64_t t = t0; t < nthreads; t += stride) {
      const int64_t i = t >> 3;
      const int part = (int)(t & 7);
      float ss = 0.0f;
      if (i < a.max_visible) {
        const u32x4 v = reinterpret_cast<const u32x4*>(a.k + (seg + i) * 128)[part];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xFFFF0000u);
          ss = __builtin_fmaf(lo, lo, ss);
          ss = __builtin_fmaf(hi, hi, ss);
        }
      }
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 4, 64);
      if (i < a.max_visible) {
        const float nrm = __fsqrt_rn(ss) * 1.00001f;
        if (part == 0) a.knorm[i] = nrm;
        m = max(m, __float_as_uint(nrm));
      }
    }
  } else {
    for (int64_t i = t0; i < a.max_visible; i += stride) {
      // MXFP4: the exact values E2M1(code) * 2^(scale - 127)
      const u32x4* row = reinterpret_cast<const u32x4*>(a.k + (seg + i) * 32);
      const uint32_t sc = *reinterpret_cast<const uint16_t*>(a.ks + (seg + i) * 2);
      float ss = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const u32x4 v = row[b];
        const float X = e8m0_f(b ? sc >> 8 : sc & 0xFFu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[e], 1.0f, 0);
          const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[e], 1.0f, 1);
          const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[e], 1.0f, 2);
          const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[e], 1.0f, 3);
          const float x[8] = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float y = __fmul_rn(x[k], X);
            ss = __builtin_fmaf(y, y, ss);
          }
        }
      }
      const float nrm = __fsqrt_rn(ss) * 1.00001f;
      a.knorm[i] = nrm;
      m = max(m, __float_as_uint(nrm));
    }
  }
  m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 8, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 4, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (b) atomicMax(a.kmax, b);
  }
  for (int64_t i = t0; i < (int64_t)a.R * H; i += stride) {
    const u32x4* row = reinterpret_cast<const u32x4*>(a.q + i * 64);
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const u32x4 v = row[p];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xFFFF0000u);
        ss = __builtin_fmaf(lo, lo, ss);
        ss = __builtin_fmaf(hi, hi, ss);
      }
    }
    atomicAdd(&a.qn[i / H], __fsqrt_rn(ss) * 1.00001f);
  }
}

// MODE 0: first-digit histogram of A per row.  MODE 1: candidate bitmap.
// A workgroup (4 waves) takes pf_rows<H>() rows; MODE 0 all keys, MODE 1 one
// range of kPfRange keys.  Each wave walks 32-key steps (two 16-key MFMA
// tiles, keys [32p, 32p+32) for p = w, w+4, ...), two steps in flight:
// B operand = the keys, loaded straight from global; A operand = the rows'
// queries held in registers.  The rows go in groups of four; M tile t of a
// group holds heads [4t, 4t+4) of its four rows (M row 4*row + head - 4t),
// so the accumulator lanes of row group g = lane/16 hold four heads of row g
// for key lane%16 in every tile, and each lane sums its row's H ReLU'd heads
// by itself: every (row, key) score lives in exactly one lane.  In MODE 1 a
// step yields one whole bitmap word per row, stored directly.
// MX: MXFP4 keys, widened to the bf16 B operand in registers (exact: an E2M1 value times a power of two).
template <int MODE, int H, bool MX>
__global__ __launch_bounds__(256, 2) void k_pf_pass(PfArgs a) {
  constexpr int kPfRows = pf_rows<H>();
  static_assert(H % 4 == 0 && kPfRows % 4 == 0, "heads and rows in fours");
  constexpr int TG = H / 4;             // M tiles per group of four rows
  constexpr int NG = kPfRows / 4;       // row groups
  extern __shared__ __align__(16) uint32_t pl[];  // MODE 0: kPfRows x kD1/2 packed counters
  // the wave index as a uniform value, so that the step positions derived from it are too
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n16 = lane & 15, g = lane >> 4;
  const int r0 = blockIdx.x * kPfRows;
  const int64_t seg = a.row_start[0];

  int kend = 0;
#pragma unroll
  for (int i = 0; i < kPfRows; ++i)
    if (r0 + i < a.R) kend = max(kend, clampv(a.row_visible[r0 + i], a.max_visible));
  const int kbeg = MODE == 0 ? 0 : (int)blockIdx.y * kPfRange;
  const int klim = MODE == 0 ? kend : min(kend, kbeg + kPfRange);
  if (kbeg >= klim) return;

  if (MODE == 0) {
    for (int i = threadIdx.x; i < kPfRows * kD1 / 2; i += 256) pl[i] = 0u;
  }

  // A operand of tile t of row group rg: M row n16 = (row 4rg + n16/4, head 4t + n16%4), channels 32ks + 8g
  bf16x8 qa[NG][TG][2];
#pragma unroll
  for (int rg = 0; rg < NG; ++rg) {
    const int row = r0 + 4 * rg + n16 / 4;
#pragma unroll
    for (int t = 0; t < TG; ++t) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (row < a.R)
          v = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)row * H + 4 * t + n16 % 4) * 64 + 32 * ks + 8 * g);
        qa[rg][t][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }
  // this lane's output row in row group rg: 4rg + g; key lane n16 of each 16-key tile
  // the smallest visible end of the workgroup's rows: steps wholly below it need no per-key bound test
  int vmin = klim;
#pragma unroll
  for (int i = 0; i < kPfRows; ++i)
    if (r0 + i < a.R) vmin = min(vmin, clampv(a.row_visible[r0 + i], a.max_visible));
  int vis[NG], rowo[NG];
  uint32_t* wrow[NG];  // MODE 1: this row's bitmap (stored by lane n16 == 0), null past the last row
  float lo[NG], cq[NG];
#pragma unroll
  for (int rg = 0; rg < NG; ++rg) {
    const int row = r0 + 4 * rg + g;
    rowo[rg] = row;
    wrow[rg] = row < a.R ? a.bits + (int64_t)row * a.nwords : nullptr;
    vis[rg] = row < a.R ? min(clampv(a.row_visible[row], a.max_visible), klim) : 0;
    lo[rg] = 0.0f;
    cq[rg] = 0.0f;
    if (MODE == 1 && row < a.R) {
      lo[rg] = a.plo[row];
      cq[rg] = a.qn[row] * pf_err(H);
    }
  }
  if (MODE == 0) __syncthreads();

  const int sample = MODE == 0 ? a.sample : 1;
  const int nsteps = ((klim - kbeg + 31) / 32 + sample - 1) / sample;  // steps this workgroup takes
  struct Step {
    u32x4 b[2][2];  // [tile][k step]
    float kn[2];
  };
  const uint8_t* kseg = a.k + seg * (MX ? 32 : 128);  // uniform base: loads take a 32-bit lane offset
  auto load_step = [&](int p, Step& st) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t j = (uint32_t)min(kbeg + 32 * p * sample + 16 * tt + n16, klim - 1);
      if constexpr (MX) {
        // channels 8g .. 8g+7 (block 0) and 32+8g .. (block 1): one code word each; bf16 values
        // packed as the loaded bf16 rows are (low half = even channel)
        const uint32_t c0 = *reinterpret_cast<const uint32_t*>(kseg + j * 32u + 4u * (uint32_t)g);
        const uint32_t c1 = *reinterpret_cast<const uint32_t*>(kseg + j * 32u + 16u + 4u * (uint32_t)g);
        st.b[tt][0] = u32x4{c0, 0u, 0u, 0u};
        st.b[tt][1] = u32x4{c1, 0u, 0u, 0u};
        st.kn[tt] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(a.ks + (seg + j) * 2));  // scales
        if (MODE == 1) st.b[tt][0][1] = __float_as_uint(a.knorm[j]);
      } else {
        const uint32_t off = j * 128u + 16u * (uint32_t)g;
        st.b[tt][0] = *reinterpret_cast<const u32x4*>(kseg + off);
        st.b[tt][1] = *reinterpret_cast<const u32x4*>(kseg + off + 64u);
        st.kn[tt] = MODE == 1 ? a.knorm[j] : 0.0f;
      }
    }
  };
  // MXFP4: the loaded code words and scales -> the bf16 B operand and the key norm (in place)
  auto widen = [&](Step& st) {
    if constexpr (MX) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint32_t sc = __float_as_uint(st.kn[tt]);
        const float kn = MODE == 1 ? __uint_as_float(st.b[tt][0][1]) : 0.0f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const uint32_t c = st.b[tt][blk][0];
          const float X = e8m0_f(blk ? sc >> 8 : sc & 0xFFu);
          // the power-of-two scale applied by the conversion itself (exact: an E2M1 value times 2^k)
          auto pk = [](auto v) { return __builtin_bit_cast(uint32_t, v); };
          st.b[tt][blk] = u32x4{pk(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, X, 0)),
                                pk(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, X, 1)),
                                pk(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, X, 2)),
                                pk(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, X, 3))};
        }
        st.kn[tt] = kn;
      }
    }
  };
  // the products of one row group in one step: its (key tile, head tile) accumulators
  auto products_rg = [&](int rg, const Step& st, floatx4 (&acc)[2][TG]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        floatx4 c = floatx4{0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rg][t][0], __builtin_bit_cast(bf16x8, st.b[tt][0]), c, 0, 0, 0);
        acc[tt][t] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rg][t][1], __builtin_bit_cast(bf16x8, st.b[tt][1]), c, 0, 0, 0);
      }
  };
  // every accumulator of a step first, so the epilogue reads results issued well before it
  auto products = [&](const Step& st, floatx4 (&acc)[NG][2][TG]) {
#pragma unroll
    for (int rg = 0; rg < NG; ++rg) products_rg(rg, st, acc[rg]);
  };
  // approximate score of (row 4rg + g, key lane of a tile): ReLU per head, summed over the row's heads
  auto score = [&](const floatx4 (&acc)[TG]) {
    float sc = 0.0f;
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float part = (relu0(acc[t][0]) + relu0(acc[t][1])) + (relu0(acc[t][2]) + relu0(acc[t][3]));
      sc = t == 0 ? part : sc + part;
    }
    return sc;
  };

  // wave step i (keys of step p = w + 4i) sits in slot i % 3: while step i is
  // scored, steps i+1 and i+2 are in flight (each slot is refilled with the
  // step two ahead before it is used, no register copies)
  Step sA, sB, sC;
  load_step(min(w, nsteps - 1), sA);
  load_step(min(w + 4, nsteps - 1), sB);
  auto body = [&](int p, Step& cur, Step& ahead) {
    load_step(min(p + 8, nsteps - 1), ahead);  // clamped: always in bounds
    const int j0 = kbeg + 32 * p * sample;
    widen(cur);
    if (MODE == 0) {
      floatx4 acc[NG][2][TG];
      products(cur, acc);
#pragma unroll
      for (int rg = 0; rg < NG; ++rg)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const float sc = score(acc[rg][tt]);
          if (j0 + 16 * tt + n16 < vis[rg]) hist_add(pl + (rowo[rg] - r0) * (kD1 / 2), __float_as_uint(sc) >> kS1);
        }
    } else {
      // ballots built straight from the compares (the int-predicate __ballot would turn each compare
      // into a 0/1 value and compare that again); the per-key bound test only in steps that reach a
      // row's visible end (a uniform branch: j0 and vmin are wave-uniform)
      // Row group rg's products are issued beside the epilogue of row group rg - 1 (independent
      // work for the matrix and vector units of one wave), and the bitmap words are stored at the
      // end of the step, so the step is one block the scheduler can interleave.
      auto marks = [&](auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        floatx4 acc[NG][2][TG];
        uint32_t word[NG];
        auto epilogue = [&](int rg) {
          unsigned long long m[2];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const float sc = score(acc[rg][tt]);
            const bool ok = FULL || j0 + 16 * tt + n16 < vis[rg];
            m[tt] = __builtin_amdgcn_ballot_w64(ok && __builtin_fmaf(cq[rg], cur.kn[tt], sc) >= lo[rg]);
          }
          // bitmap word of row g: its 16 keys of each tile (lanes 16g .. 16g+15)
          word[rg] = ((uint32_t)(m[0] >> (16 * g)) & 0xFFFFu) | ((uint32_t)(m[1] >> (16 * g)) << 16);
        };
        products_rg(0, cur, acc[0]);
#pragma unroll
        for (int rg = 1; rg < NG; ++rg) {
          products_rg(rg, cur, acc[rg]);
          epilogue(rg - 1);
        }
        epilogue(NG - 1);
        if (n16 == 0) {
#pragma unroll
          for (int rg = 0; rg < NG; ++rg)
            if (wrow[rg]) wrow[rg][j0 / 32] = word[rg];
        }
      };
      if (j0 + 32 <= vmin) marks(std::true_type{});
      else marks(std::false_type{});
    }
  };
  // whole rounds of three steps (no conditional step in the loop body, so the
  // waits for the loads in flight stay exact), then the last steps
  int p0 = w;
  for (; p0 + 8 < nsteps; p0 += 12) {
    body(p0, sA, sC);
    body(p0 + 4, sB, sA);
    body(p0 + 8, sC, sB);
  }
  if (p0 < nsteps) body(p0, sA, sC);
  if (p0 + 4 < nsteps) body(p0 + 4, sB, sA);
  if (MODE == 0) {
    __syncthreads();
    for (int i = threadIdx.x; i < kPfRows * (kD1 / 2); i += 256) {
      const int rloc = i / (kD1 / 2), wd = i % (kD1 / 2);
      const uint32_t v = pl[i];
      if (r0 + rloc < a.R && v) {
        uint32_t* gh = a.hist + (int64_t)(r0 + rloc) * kD1 + 2 * wd;
        if (v & 0xFFFFu) atomicAdd(gh, v & 0xFFFFu);
        if (v >> 16) atomicAdd(gh + 1, v >> 16);
      }
    }
  }
}

// per row: the bin holding the target-th largest sampled approximate score -> candidate bound.  A row
// whose sample is too small to place it gets no candidates (+inf): its exact selection then fails the
// certification and it takes the exact fallback.
__global__ __launch_bounds__(256) void k_pf_thresh(PfArgs a, int H) {
  __shared__ uint32_t red[32];
  const int r = blockIdx.x;
  uint32_t above, total;
  const int b = find_bin<256, kD1>(a.hist + (int64_t)r * kD1, a.target, &above, &total, red);
  if (threadIdx.x == 0) {
    if (b < 0) {
      a.plo[r] = INFINITY;
      a.thi[r] = INFINITY;
    } else {
      const float edge = __uint_as_float((uint32_t)b << kS1);
      const float emax = a.qn[r] * pf_err(H) * __uint_as_float(*a.kmax);
      a.plo[r] = (edge - emax) - 1e-6f * edge;  // nudged down: rounding of the subtraction
      a.thi[r] = edge;
    }
  }
}

// per row: candidate bitmap -> ascending positions (or the overflow flag).
// Wave w owns a contiguous quarter of the row's words: a first pass counts
// its bits (coalesced 64-word loads), one barrier gives each wave its output
// offset, and a second pass expands 64 words at a time: a DPP prefix sum of
// the lanes' bit counts places each lane's positions, written one bit per
// lane per store, so a store's lanes write neighbouring slots.
__global__ __launch_bounds__(256) void k_pf_compact(PfArgs a) {
  __shared__ uint32_t red[4];
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vis = clampv(a.row_visible[r], a.max_visible);
  const int nw = (vis + 31) / 32;
  const uint32_t* bw = a.bits + (int64_t)r * a.nwords;
  int32_t* out = a.cand + (int64_t)r * kPfCap;
  const int per = ((nw + 3) / 4 + 63) & ~63;
  const int w0 = min(nw, wave * per), w1 = min(nw, w0 + per);
  uint32_t cnt = 0;
  for (int i = w0 + lane; i < w1; i += 64) cnt += __popc(bw[i]);
  cnt = wave_incl_sum(cnt);
  if (lane == 63) red[wave] = cnt;
  __syncthreads();
  uint32_t base = 0, total = 0;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    base += ww < wave ? red[ww] : 0u;
    total += red[ww];
  }
  if (total <= (uint32_t)kPfCap) {
    for (int i0 = w0; i0 < w1; i0 += 64) {
      const int i = i0 + lane;
      uint32_t m = i < w1 ? bw[i] : 0u;
      const uint32_t c = (uint32_t)__popc(m);
      const uint32_t incl = wave_incl_sum(c);
      uint32_t at = base + incl - c;
      base += (uint32_t)__shfl((int)incl, 63, 64);
      while (__ballot(m != 0u)) {
        if (m) {
          out[at++] = 32 * i + (__ffs(m) - 1);
          m &= m - 1u;
        }
      }
    }
  }
  const bool overflow = total > (uint32_t)kPfCap;
  if (threadIdx.x == 0) {
    a.ccnt[r] = overflow ? -1 : (int32_t)total;
    if (overflow) a.over_list[atomicAdd(a.nover, 1u)] = (uint32_t)r;
  }
  if (overflow) {  // this row takes the exact full scan, whose first-digit histogram starts at zero
    u32x4* h = reinterpret_cast<u32x4*>(a.xhist + (int64_t)r * kD1);
    for (int i = threadIdx.x; i < kD1 / 4; i += 256) h[i] = u32x4{0u, 0u, 0u, 0u};
  }
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
  // exact path (Full and Reindex; the per-row fallback of the shared-segment mode)
  float* qf;
  uint32_t* hist;  // [2][R][kD1] first-digit histograms (Full: entries, blocks; Reindex: the second)
  uint32_t* thr[2];  // [R][2] threshold bins found by k_collect (Full)
  float* scores;
  float* bmax;
  float* cand_key[2];
  int32_t* cand_pos[2];
  uint32_t* counts[2];
  int64_t n_pad, nb_pad;
  int nsub, nbsub;
  // shared-segment (prefill) approximate path
  float* knorm;
  uint32_t* kmax;
  float* qn;
  uint32_t* phist;
  float* plo;
  float* thi;
  uint32_t* bits;
  int nwords;
  int32_t* cand;
  int32_t* ccnt;
  uint32_t* over_list;
  uint32_t* nover;
  float* cscore;   // [R][kPfCap] exact scores of the candidates
  size_t bytes;
};

Layout layout(void* base, int mode, int R, int H, int max_visible, int pool_stride, int pool_size) {
  Layout L{};
  Carve c{static_cast<char*>(base)};
  const bool shared = mode == CSA2_FULL_SHARED;
  const bool full = mode == CSA2_FULL || shared;
  const int64_t n = full ? max_visible : pool_stride;
  const bool pool_on = full && pool_size > 0;
  const int64_t nb = pool_on ? ceil_div(max_visible, kBlock) : 0;
  L.n_pad = round_up(std::max<int64_t>(n, 1), kSub);
  L.nb_pad = round_up(std::max<int64_t>(nb, 1), kSub);
  L.nsub = (int)(L.n_pad / kSub);
  L.nbsub = (int)(L.nb_pad / kSub);
  L.qf = c.take<float>((size_t)R * H * kIdxDim);
  L.hist = c.take<uint32_t>((size_t)R * kD1 * 2);
  L.thr[0] = c.take<uint32_t>((size_t)R * 2);
  L.thr[1] = c.take<uint32_t>((size_t)R * 2);
  L.scores = c.take<float>((size_t)R * L.n_pad);
  L.bmax = pool_on ? c.take<float>((size_t)R * L.nb_pad) : nullptr;
  if (full) {
    L.cand_key[0] = c.take<float>((size_t)R * 2 * L.n_pad);
    L.cand_pos[0] = c.take<int32_t>((size_t)R * 2 * L.n_pad);
    L.counts[0] = c.take<uint32_t>((size_t)R * L.nsub);
  }
  if (pool_on) {
    L.cand_key[1] = c.take<float>((size_t)R * 2 * L.nb_pad);
    L.cand_pos[1] = c.take<int32_t>((size_t)R * 2 * L.nb_pad);
    L.counts[1] = c.take<uint32_t>((size_t)R * L.nbsub);
  }
  if (shared && !pool_on) {
    L.nwords = (int)ceil_div(std::max<int64_t>(max_visible, 1), 32);
    L.knorm = c.take<float>((size_t)std::max(max_visible, 1));
    L.kmax = c.take<uint32_t>(1);
    L.qn = c.take<float>((size_t)R);
    L.phist = c.take<uint32_t>((size_t)R * kD1);
    L.plo = c.take<float>((size_t)R);
    L.thi = c.take<float>((size_t)R);
    L.bits = c.take<uint32_t>((size_t)R * L.nwords);
    L.cand = c.take<int32_t>((size_t)R * kPfCap);
    L.ccnt = c.take<int32_t>((size_t)R);
    L.over_list = c.take<uint32_t>((size_t)R);
    L.nover = c.take<uint32_t>(1);
    L.cscore = c.take<float>((size_t)R * kPfCap);
  }
  L.bytes = c.off;
  return L;
}

// even_rows > 0: the Full scan with the batch's tiles shared evenly (k_scan_even over that many rows)
template <int KDT, int HC, bool REINDEX, bool POOL, int QDT>
void launch_score(const ScoreArgs& sa, const void* qsrc, dim3 grid, hipStream_t s, int even_rows) {
  using T = KeyTile<KDT>;
  const size_t lds = (size_t)kWavesPerWG * T::kWaveBytes + (REINDEX ? 0 : (size_t)kD1 / 2 * 4 * (POOL ? 2 : 1)) +
                     ((REINDEX || T::kMx) ? (size_t)(HC > 0 ? HC : kMaxHeads) * kIdxDim * 4 : 0);
  if constexpr (!REINDEX && QDT == CSA2_F32) {
    if (even_rows > 0) {
      auto kern = k_scan_even<KDT, HC, POOL>;
      static bool configured = false;
      if (!configured) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
        configured = true;
      }
      hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, sa, qsrc, even_rows);
      return;
    }
  }
  auto kern = k_score<KDT, HC, REINDEX, POOL, QDT>;
  static bool configured = false;
  if (!configured) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    configured = true;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, sa, qsrc);
}

template <int KDT, bool REINDEX, bool POOL, int QDT>
void dispatch_heads(int H, const ScoreArgs& sa, const void* qsrc, dim3 grid, hipStream_t s, int even_rows = 0) {
  if (H == 8) launch_score<KDT, 8, REINDEX, POOL, QDT>(sa, qsrc, grid, s, even_rows);
  else if (H == 4) launch_score<KDT, 4, REINDEX, POOL, QDT>(sa, qsrc, grid, s, even_rows);
  else launch_score<KDT, 0, REINDEX, POOL, QDT>(sa, qsrc, grid, s, even_rows);
}

}  // namespace

size_t topk_workspace_bytes(int mode, int R, int H, int max_visible, int pool_stride, int pool_size) {
  return layout(nullptr, mode, R, H, max_visible, pool_stride, pool_size).bytes;
}

int topk_max_visible() { return 1024 * kSub; }

namespace {

// the exact path: scan (Full: every visible entry; Reindex: the pool), then
// the exact selection; a row list restricts it to the listed rows
// the prefill rescoring's certification: bounds, the fallback list and its count, the exact histograms
struct Cert {
  const float* thi;
  uint32_t* list;
  uint32_t* count;
  uint32_t* xhist;
};

void run_exact(const Layout& L, int mode, bool shared, int R, int q_dtype, int H, const void* idx_k,
               const uint8_t* idx_ks, int k_dtype,
               const int64_t* row_start, const int32_t* row_visible, int max_visible, const int32_t* pool,
               const int32_t* pool_len, int pool_stride, int top_k, int32_t* out_idx, int pool_size,
               int32_t* out_pool, int32_t* out_pool_len, float* scores,
               int64_t score_stride, bool prep_done, bool record, const void* idx_q, hipStream_t s,
               const uint32_t* row_list = nullptr, const uint32_t* row_count = nullptr,
               const Cert* cert = nullptr) {
  const bool full = mode == CSA2_FULL;
  // a row list (rows known only on the device, usually none): the scan and the selection keep a grid
  // row per possible row (workgroups past the list's length exit at once); the collection, whose grid is
  // widest, takes at most kListRows grid rows that loop over the list
  const int Rg = row_list ? std::min(R, kListRows) : R;
  const bool pool_on = full && pool_size > 0;
  if (!prep_done && full) {  // (Reindex reads the queries as given and counts in its selection)
    const int64_t nq = (int64_t)R * H * kIdxDim;
    const int64_t nhist = (int64_t)R * kD1 * 2;
    hipLaunchKernelGGL(k_prep, dim3((unsigned)std::min<int64_t>(2048, ceil_div(std::max(nq, nhist), 256))),
                       dim3(256), 0, s, idx_q, q_dtype, R, H, L.qf, L.hist, nhist);
  }
  const int64_t n = full ? max_visible : pool_stride;
  if (n > 0) {
    ScoreArgs sa{};
    sa.H = H;
    sa.idx_k = idx_k;
    sa.idx_ks = idx_ks;
    sa.row_start = row_start;
    sa.row_visible = row_visible;
    sa.max_visible = max_visible;
    sa.pool = pool;
    sa.pool_len = pool_len;
    sa.pool_stride = pool_stride;
    sa.scores = scores;
    sa.n_pad = score_stride;
    sa.bmax = L.bmax;
    sa.nb_pad = L.nb_pad;
    // Reindex counts into the second histogram, so that the shared-segment mode's
    // rescoring (Reindex over candidate lists) leaves the first one to its Full fallback
    sa.hist_s = full ? L.hist : L.hist + (size_t)R * kD1;
    sa.hist_b = L.hist + (size_t)R * kD1;
    sa.row_list = row_list;
    sa.row_count = row_count;
    sa.shared_start = shared ? 1 : 0;
    // Full: about three workgroups per CU over the whole batch (each scans
    // tiles_per_wg x 256 consecutive entries); Reindex: 256 pool slots each
    // (at most 255 tiles = 65,280 entries per workgroup: its packed 16-bit histogram counters cannot overflow)
    const int64_t tiles = ceil_div(n, (int64_t)kWGKeys);
    sa.tiles_per_wg =
        (int)std::min<int64_t>(255, ceil_div(tiles, std::max<int64_t>(1, ceil_div((int64_t)kScanSlots, R))));
    dim3 grid((unsigned)ceil_div(tiles, (int64_t)sa.tiles_per_wg), (unsigned)R);
    // Full decode batches of up to 256 rows: the tiles shared evenly over the grid (rows of different
    // lengths leave no workgroup idle); at most 255 tiles per workgroup (its packed histogram counters)
    const int even = (full && !shared && !row_list && R <= kThreads) ? R : 0;
    if (even) grid = dim3((unsigned)std::max<int64_t>(kScanSlots, ceil_div((int64_t)R * tiles, 255)), 1u);
    auto& ev = profile_events(full ? CSA2_KERNEL_INDEX_SCAN : CSA2_KERNEL_REINDEX_SCORE);
    if (record && ev.start) (void)hipEventRecord(ev.start, s);
    const bool qbf = q_dtype == CSA2_BF16;
    // the prefill rescoring (Reindex over the candidate lists) reads the block k_prep laid out
    const bool prepared = !full && shared && prep_done;
    if (prepared && k_dtype == CSA2_BF16) dispatch_heads<CSA2_BF16, true, false, kQPrepared>(H, sa, L.qf, grid, s);
    else if (prepared && k_dtype == CSA2_F32) dispatch_heads<CSA2_F32, true, false, kQPrepared>(H, sa, L.qf, grid, s);
    else if (k_dtype == CSA2_MXFP4) {
      if (!full && qbf) dispatch_heads<CSA2_MXFP4, true, false, CSA2_BF16>(H, sa, idx_q, grid, s);
      else if (!full) dispatch_heads<CSA2_MXFP4, true, false, CSA2_F32>(H, sa, idx_q, grid, s);
      else if (pool_on) dispatch_heads<CSA2_MXFP4, false, true, CSA2_F32>(H, sa, L.qf, grid, s, even);
      else dispatch_heads<CSA2_MXFP4, false, false, CSA2_F32>(H, sa, L.qf, grid, s, even);
    } else if (k_dtype == CSA2_BF16) {
      if (!full && qbf) dispatch_heads<CSA2_BF16, true, false, CSA2_BF16>(H, sa, idx_q, grid, s);
      else if (!full) dispatch_heads<CSA2_BF16, true, false, CSA2_F32>(H, sa, idx_q, grid, s);
      else if (pool_on) dispatch_heads<CSA2_BF16, false, true, CSA2_F32>(H, sa, L.qf, grid, s, even);
      else dispatch_heads<CSA2_BF16, false, false, CSA2_F32>(H, sa, L.qf, grid, s, even);
    } else {
      if (!full && qbf) dispatch_heads<CSA2_F32, true, false, CSA2_BF16>(H, sa, idx_q, grid, s);
      else if (!full) dispatch_heads<CSA2_F32, true, false, CSA2_F32>(H, sa, idx_q, grid, s);
      else if (pool_on) dispatch_heads<CSA2_F32, false, true, CSA2_F32>(H, sa, L.qf, grid, s, even);
      else dispatch_heads<CSA2_F32, false, false, CSA2_F32>(H, sa, L.qf, grid, s, even);
    }
    if (record && ev.stop) (void)hipEventRecord(ev.stop, s);
  }

  SelArgs a{};
  a.mode = mode;
  a.row_visible = row_visible;
  a.max_visible = max_visible;
  a.pool_stride = pool_stride;
  a.pool = pool;
  a.pool_len = pool_len;
  a.by_len = shared ? 1 : 0;  // the prefill candidate lists are mostly empty
  if (cert) {
    a.cert_thi = cert->thi;
    a.cert_list = cert->list;
    a.cert_count = cert->count;
    a.cert_xhist = cert->xhist;
  }
  a.row_list = row_list;
  a.row_count = row_count;
  a.out_idx = out_idx;
  a.out_pool = out_pool;
  a.out_pool_len = out_pool_len;
  a.pool_size = pool_size;
  a.nseries = pool_on ? 2 : 1;
  a.s[0] = Series{scores, score_stride, full ? L.hist : L.hist + (size_t)R * kD1, L.thr[0], L.cand_key[0],
                  L.cand_pos[0], L.counts[0], L.nsub, top_k};
  if (pool_on)
    a.s[1] = Series{L.bmax, L.nb_pad, L.hist + (size_t)R * kD1, L.thr[1], L.cand_key[1], L.cand_pos[1], L.counts[1],
                    L.nbsub,
                    pool_size / kBlock};
  if (full) {
    const int gx = (int)ceil_div(std::max(L.nsub, pool_on ? L.nbsub : 1), 4);
    if (row_list)
      hipLaunchKernelGGL(k_collect<true>, dim3((unsigned)gx, (unsigned)Rg, (unsigned)a.nseries), dim3(kThreads), 0, s,
                         a);
    else
      hipLaunchKernelGGL(k_collect<false>, dim3((unsigned)gx, (unsigned)R, (unsigned)a.nseries), dim3(kThreads), 0, s,
                         a);
  }
  if (a.by_len && !row_list && mode == CSA2_REINDEX) {  // the prefill rescoring's selection
    const size_t lds = kFinSmallLdsWords * 4;
    static bool configured_small = false;
    if (!configured_small) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_finalize_small),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      configured_small = true;
    }
    hipLaunchKernelGGL(k_finalize_small, dim3((unsigned)R), dim3(kFinSmallThreads), lds, s, a);
    return;
  }
  const size_t lds = kFinLdsWords * 4;
  static bool configured = false;
  if (!configured) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_finalize), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    configured = true;
  }
  hipLaunchKernelGGL(k_finalize, dim3((unsigned)R, (unsigned)a.nseries), dim3(kFinThreads), lds, s, a);
}

template <int H, bool MX>
void launch_pf_pass(int mode, const PfArgs& p, int R, int max_visible, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(R, pf_rows<H>()), mode == 0 ? 1u : (unsigned)ceil_div(max_visible, kPfRange));
  const size_t lds = mode == 0 ? (size_t)pf_rows<H>() * kD1 / 2 * 4 : 0;
  static bool configured[2] = {false, false};
  if (mode == 0) {
    if (!configured[0]) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_pf_pass<0, H, MX>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      configured[0] = true;
    }
    hipLaunchKernelGGL((k_pf_pass<0, H, MX>), grid, dim3(256), lds, s, p);
  } else {
    if (!configured[1]) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_pf_pass<1, H, MX>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      configured[1] = true;
    }
    hipLaunchKernelGGL((k_pf_pass<1, H, MX>), grid, dim3(256), lds, s, p);
  }
}

}  // namespace

bool topk_uses_prefill_path(int mode, int q_dtype, int k_dtype, int H, int pool_size) {
  return mode == CSA2_FULL_SHARED && pool_size == 0 && q_dtype == CSA2_BF16 &&
         (k_dtype == CSA2_BF16 || k_dtype == CSA2_MXFP4) && (H == 4 || H == 8 || H == 16);
}

hipError_t launch_index_topk(int mode, int R, const void* idx_q, int q_dtype, int H, const void* idx_k,
                             const uint8_t* idx_ks, int k_dtype,
                             const int64_t* row_start, const int32_t* row_visible, int max_visible,
                             const int32_t* pool, const int32_t* pool_len, int pool_stride, int top_k,
                             int32_t* out_idx, int pool_size, int32_t* out_pool, int32_t* out_pool_len, void* ws,
                             hipStream_t s) {
  const bool shared = mode == CSA2_FULL_SHARED;
  const int emode = shared ? CSA2_FULL : mode;
  Layout L = layout(ws, mode, R, H, max_visible, pool_stride, pool_size);
  if (!topk_uses_prefill_path(mode, q_dtype, k_dtype, H, pool_size)) {
    run_exact(L, emode, shared, R, q_dtype, H, idx_k, idx_ks, k_dtype, row_start, row_visible, max_visible, pool, pool_len,
              pool_stride, top_k, out_idx, pool_size, out_pool, out_pool_len, L.scores, L.n_pad, false, true,
              idx_q, s);
    return hipGetLastError();
  }
  // shared segment: approximate MFMA passes -> candidates -> exact rescoring and selection
  PfArgs p{};
  p.q = static_cast<const uint16_t*>(idx_q);
  p.k = static_cast<const uint8_t*>(idx_k);
  p.ks = k_dtype == CSA2_MXFP4 ? idx_ks : nullptr;
  p.row_start = row_start;
  p.row_visible = row_visible;
  p.max_visible = max_visible;
  p.R = R;
  p.K = top_k;
  p.knorm = L.knorm;
  p.kmax = L.kmax;
  p.qn = L.qn;
  p.hist = L.phist;
  p.plo = L.plo;
  p.thi = L.thi;
  p.sample = 1;
  p.target = (uint32_t)top_k;
  p.bits = L.bits;
  p.nwords = L.nwords;
  p.cand = L.cand;
  p.ccnt = L.ccnt;
  p.over_list = L.over_list;
  p.nover = L.nover;
  p.xhist = L.hist;
  {
    // the queries for the exact path (fallback rows); the approximate histogram, the key-norm maximum,
    // the query norms and the fallback list's count zeroed; the exact path's histograms of listed rows
    // are zeroed by the kernel that lists them (k_pf_compact, the rescoring's selection)
    const int64_t nq = (int64_t)R * H * kIdxDim;
    hipLaunchKernelGGL(k_prep, dim3((unsigned)std::min<int64_t>(2048, ceil_div(nq, 256))), dim3(256), 0, s, idx_q,
                       q_dtype, R, H, L.qf, L.hist, (int64_t)0);
    hipLaunchKernelGGL(k_zero, dim3((unsigned)std::min<int64_t>(2048, ceil_div((int64_t)R * kD1, 256))), dim3(256),
                       0, s, L.phist, (int64_t)R * kD1, L.phist, (int64_t)0, L.phist, (int64_t)0, L.kmax);
    hipLaunchKernelGGL(k_zero, dim3((unsigned)ceil_div((int64_t)R, 256)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(L.qn), (int64_t)R, L.nover, (int64_t)0, L.nover, (int64_t)0,
                       L.nover);
  }
  const int64_t nn = std::max<int64_t>((int64_t)max_visible * (k_dtype == CSA2_MXFP4 ? 1 : 8), (int64_t)R * H);
  hipLaunchKernelGGL(k_pf_norms, dim3((unsigned)std::min<int64_t>(1024, ceil_div(nn, 256))), dim3(256), 0, s, p, H);
  auto& ev = profile_events(CSA2_KERNEL_INDEX_SCAN);
  if (ev.start) (void)hipEventRecord(ev.start, s);
  auto pass = [&](int mode, const PfArgs& pa) {
    if (pa.ks) {
      if (H == 4) launch_pf_pass<4, true>(mode, pa, R, max_visible, s);
      else if (H == 8) launch_pf_pass<8, true>(mode, pa, R, max_visible, s);
      else launch_pf_pass<16, true>(mode, pa, R, max_visible, s);
    } else {
      if (H == 4) launch_pf_pass<4, false>(mode, pa, R, max_visible, s);
      else if (H == 8) launch_pf_pass<8, false>(mode, pa, R, max_visible, s);
      else launch_pf_pass<16, false>(mode, pa, R, max_visible, s);
    }
  };
  // 1. a provisional bound per row from a 1/kPfSample sample of the keys, with headroom
  PfArgs ps = p;
  ps.hist = L.phist;
  ps.sample = kPfSample;
  ps.target = (uint32_t)ceil_div((int64_t)top_k * 3, 2 * kPfSample);
  pass(0, ps);
  hipLaunchKernelGGL(k_pf_thresh, dim3((unsigned)R), dim3(256), 0, s, ps, H);
  // 2. the candidate pass over every key
  pass(1, ps);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
  hipLaunchKernelGGL(k_pf_compact, dim3((unsigned)R), dim3(256), 0, s, p);
  // exact scores of the candidates and the exact selection among them (Reindex over the candidate lists),
  // which also certifies each row's bound on the exact scores and lists the rows that fail
  const Cert cert{L.thi, L.over_list, L.nover, L.hist};
  run_exact(L, CSA2_REINDEX, true, R, q_dtype, H, idx_k, idx_ks, k_dtype, row_start, row_visible, max_visible, L.cand,
            L.ccnt, kPfCap, top_k, out_idx, 0, nullptr, nullptr, L.cscore, kPfCap, true, true, idx_q, s, nullptr,
            nullptr, &cert);
  // listed rows (candidates overflowed, or the bound not certified): the exact full scan and selection,
  // for those rows only
  run_exact(L, CSA2_FULL, true, R, q_dtype, H, idx_k, idx_ks, k_dtype, row_start, row_visible, max_visible, nullptr,
            nullptr, 0, top_k, out_idx, 0, nullptr, nullptr, L.scores, L.n_pad, true, false, idx_q, s,
            L.over_list, L.nover);
  return hipGetLastError();
}

}  // namespace csa2
