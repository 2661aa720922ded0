// Per-row top-K selection on gfx950 (the M^sel step of the atlas DeepSeek-V3.2-Exp
// MoE-block step list; row layout int32 [batch, query, min(K, keys)] from the
// nnterp deepseek_v32 page, section 03).
//
// Order: score descending, then index ascending (equal scores go to the lower
// index).  -0 == +0; NaN and -inf are never selected.  The chosen indices are
// written in ascending order and the row is padded with -1.
//
// One 1024-thread workgroup selects from up to 32768 elements held in
// registers (thread i owns a contiguous run of E elements, so the output is
// compacted in index order by a block-wide prefix sum).  The K-th largest key
// is found exactly by a radix select over the order-preserving 32-bit key
// (12 + 10 + 10 bits, MSB first) with LDS histograms; the first pass uses 12
// bits (sign, exponent and 3 mantissa bits) so that score distributions
// concentrated in a few binades still spread over many bins.  As soon as the
// bin holding the K-th key has at most 16 elements, those are ranked
// directly (by key, then index) instead of running the remaining passes; the
// count of selectable keys comes from the first histogram.
//
// Rows longer than one workgroup's capacity are reduced in two stages: each
// chunk of the row yields its own exact top-K candidates (key, index), in
// index order, and a second pass selects the top-K of the candidates.  This is
// exact: an element of the row's top-K has fewer than K elements ahead of it
// in the (score, index) order within its chunk, so it survives its chunk.
// Rows whose candidates would not fit one merge workgroup (more than 16
// chunks of K, or K of a chunk or more) take the two-launch long-row select
// described before its kernels.
//
// Inside the whole path, causal query rows hold scores only up to their
// query's position; the rest of such a row's memory is masked to key 0.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kChunkElems = 32 * kTopkThreads;  // stage-1 chunk (E = 32)
constexpr int kPass1Bins = 4096;                 // 12 bits
constexpr int kPassBins = 1024;                  // 10 bits (passes 2 and 3)
constexpr int kSmallCand = 16;                   // boundary bins this small are ranked by one wave

struct alignas(16) TopkLds {
  uint32_t hist[2][kPass1Bins];     // ping-pong: pass p counts into hist[p & 1]
  uint32_t wave_tot[2][kTopkWaves];  // ping-pong scan scratch (16-byte aligned rows)
  uint32_t sel[3][2];                // per pass: boundary bin, count above it
  uint32_t cand_key[kSmallCand];
  int32_t cand_idx[kSmallCand];
  uint32_t cand_take[kSmallCand];
  uint32_t total;
  uint32_t ncand;
};

// Exclusive prefix sum over the workgroup in thread order: the sum of the
// values of all lower threads; *total gets the sum over all threads.  One
// barrier; `wave_tot` must not be reused before the next barrier.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  static_assert(kTopkWaves % 4 == 0, "wave totals read 4 at a time");
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < kTopkWaves / 4; ++q) {
    const uint4 t4 = reinterpret_cast<const uint4*>(wave_tot)[q];
    const uint32_t t[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      before += (4 * q + e < wave) ? t[e] : 0u;
      tot += t[e];
    }
  }
  *total = tot;
  return before + inc - v;
}

// Bins [NB - (t+1)*per, NB - t*per) belong to thread t (scanned from the top):
// find the bin where the running count from the top reaches k_rem; the owner
// thread records it and the count above it in sel.  Returns the histogram's
// total (no bin is recorded when it is below k_rem).  A thread's bins are
// read once, with one 16-byte read when it owns four.
template <int NB>
__device__ __forceinline__ uint32_t find_boundary(const uint32_t* hist, uint32_t k_rem,
                                                  uint32_t* wave_tot, uint32_t* sel) {
  constexpr int per = NB / kTopkThreads;
  static_assert(per == 1 || per == 4, "bins per thread");
  const int hi_bin = NB - static_cast<int>(threadIdx.x) * per;  // exclusive
  uint32_t c[per];  // c[k]: bin hi_bin - 1 - k
  if constexpr (per == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(hist + hi_bin - 4);
    c[0] = v.w; c[1] = v.z; c[2] = v.y; c[3] = v.x;
  } else {
    c[0] = hist[hi_bin - 1];
  }
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) local += c[k];
  uint32_t tot;
  uint32_t acc = block_exclusive_scan(local, wave_tot, &tot);
#pragma unroll
  for (int k = 0; k < per; ++k) {
    if (acc < k_rem && k_rem <= acc + c[k]) {
      sel[0] = static_cast<uint32_t>(hi_bin - 1 - k);
      sel[1] = acc;
    }
    acc += c[k];
  }
  return tot;
}

// The keys row `row` holds: n_in; with causal_T > 0 (rows of causal queries,
// causal_T of them per sequence) only the ones its query sees, [0, L_b - T +
// t + 1) for row (b, t), L_b the sequence's length (seq_lens[b] clamped to
// [0, n_in], or n_in), the count clamped to [0, n_in]; whatever the rest of
// the row's memory holds counts as key 0.
__device__ __forceinline__ int row_keys(int64_t row, int n_in, int causal_T, const int32_t* seq_lens) {
  if (causal_T <= 0) return n_in;
  const int t = static_cast<int>(row % causal_T);
  const int L = seq_lens == nullptr ? n_in : min(max(seq_lens[row / causal_T], 0), n_in);
  return min(max(L - causal_T + t + 1, 0), n_in);
}

// SRC_CAND: elements come from a candidate list (key, index) instead of fp32
// scores.  OUT_CAND: the result is a candidate list (key and index written).
// VEC: every thread's run of E inputs starts 16-byte aligned (16-byte loads).
template <int E, bool SRC_CAND, bool OUT_CAND, bool VEC>
__global__ void __launch_bounds__(kTopkThreads, (E <= 16 && !SRC_CAND && !OUT_CAND) ? 8 : 1)
topk_select(int n_in, int causal_T, const int32_t* __restrict__ seq_lens, int64_t in_stride, int chunk_elems,
            const float* __restrict__ scores, const uint32_t* __restrict__ cand_key_in,
            const int32_t* __restrict__ cand_idx_in, int K_out, int32_t* __restrict__ idx_out,
            uint32_t* __restrict__ cand_key_out) {
  __shared__ TopkLds lds;
  debug_poison_lds<sizeof(lds)>(&lds);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int chunk = blockIdx.x;
  // this workgroup's elements: [elem0, elem0 + n) of the row's input, of the
  // [elem0, elem0 + n_mem) it holds in memory
  const int elem0 = chunk * chunk_elems;
  const int n_mem = min(chunk_elems, n_in - elem0);
  const int n = min(n_mem, row_keys(row, n_in, causal_T, seq_lens) - elem0);
  const int64_t in_base = row * in_stride + elem0;
  const int64_t out_base = (row * gridDim.x + chunk) * static_cast<int64_t>(K_out);

  // ---- thread t owns elements [E t, E t + E): keys in registers ----
  uint32_t key[E];
  int32_t id[SRC_CAND ? E : 1];  // candidate indices; a score's index is its position
  const int i0 = tid * E;
  if (VEC && i0 + E <= n_mem) {
#pragma unroll
    for (int j = 0; j < E; j += 4) {
      if constexpr (SRC_CAND) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(cand_key_in + in_base + i0 + j);
        const int4 d4 = *reinterpret_cast<const int4*>(cand_idx_in + in_base + i0 + j);
        key[j] = k4.x; key[j + 1] = k4.y; key[j + 2] = k4.z; key[j + 3] = k4.w;
        id[j] = d4.x; id[j + 1] = d4.y; id[j + 2] = d4.z; id[j + 3] = d4.w;
      } else {
        const float4 f4 = *reinterpret_cast<const float4*>(scores + in_base + i0 + j);
        key[j] = score_key(f4.x); key[j + 1] = score_key(f4.y);
        key[j + 2] = score_key(f4.z); key[j + 3] = score_key(f4.w);
      }
    }
    // a run that reaches past the row's n elements (what the memory holds
    // there is not a score of this row): those count as key 0
    if (i0 + E > n) {
#pragma unroll
      for (int j = 0; j < E; ++j) key[j] &= 0u - static_cast<uint32_t>(i0 + j < n);
    }
  } else {
    // the chunk's ragged end (or rows not 16-byte aligned): every load issued
    // before any is used, at positions clamped into the chunk's memory,
    // elements past n masked to key 0 (a branch per element would wait for
    // each load in turn)
    const int last = max(n, 1) - 1;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = min(i0 + j, last);
      if constexpr (SRC_CAND) {
        key[j] = cand_key_in[in_base + i];
        id[j] = cand_idx_in[in_base + i];
      } else {
        key[j] = score_key(scores[in_base + i]);
      }
    }
#pragma unroll
    for (int j = 0; j < E; ++j) key[j] &= 0u - static_cast<uint32_t>(i0 + j < n);
  }
  // the row index of element j of this thread (keys of elements past the
  // input are 0, so they are never taken and their index is never used)
  auto index_of = [&](int j) -> int32_t {
    if constexpr (SRC_CAND) return id[j];
    else return elem0 + i0 + j;
  };
  // clear both histograms while the loads are in flight
  for (int i = tid; i < 2 * kPass1Bins; i += kTopkThreads) (&lds.hist[0][0])[i] = 0u;
  if (tid == 0) lds.ncand = 0u;
  __syncthreads();

  // ---- pass 1: 12-bit histogram of the selectable keys (key 0 is not) ----
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (key[j] != 0u) atomicAdd(&lds.hist[0][key[j] >> 20], 1u);
  __syncthreads();
  // the boundary bin of the K-th largest key; the total is the count of
  // selectable keys
  const uint32_t nvalid =
      find_boundary<kPass1Bins>(lds.hist[0], static_cast<uint32_t>(K_out), lds.wave_tot[0], lds.sel[0]);
  __syncthreads();
  const uint32_t ksel = min(static_cast<uint32_t>(K_out), nvalid);

  // Selection rule, set below: keys > thr_hi are taken; keys with
  // (key & mask) == prefix are the boundary candidates, of which k_rem are
  // taken (by larger key, then lower index).
  uint32_t prefix = 0u, mask = 0u, k_rem = ksel;
  uint32_t cnt = 0u;  // candidates in the boundary bin
  bool all = nvalid <= static_cast<uint32_t>(K_out);
  if (!all) {
    prefix = lds.sel[0][0] << 20;
    mask = 0xfff00000u;
    k_rem -= lds.sel[0][1];
    cnt = lds.hist[0][lds.sel[0][0]];
    constexpr int kShift[2] = {10, 0};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (cnt <= kSmallCand) break;  // workgroup-uniform
      uint32_t* h = lds.hist[(p + 1) & 1];
      if (p == 1)  // hist[0] is free again once pass 2's boundary is known
        for (int i = tid; i < kPassBins; i += kTopkThreads) h[i] = 0u;
      if (p == 1) __syncthreads();
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (key[j] != 0u && (key[j] & mask) == prefix) atomicAdd(&h[(key[j] >> kShift[p]) & (kPassBins - 1)], 1u);
      __syncthreads();
      (void)find_boundary<kPassBins>(h, k_rem, lds.wave_tot[(p + 1) & 1], lds.sel[p + 1]);
      __syncthreads();
      const uint32_t bin = lds.sel[p + 1][0];
      prefix |= bin << kShift[p];
      mask |= static_cast<uint32_t>(kPassBins - 1) << kShift[p];
      k_rem -= lds.sel[p + 1][1];
      cnt = h[bin];
    }
  }

  // ---- decide which elements are taken ----
  uint32_t take = 0;  // bit j: element j of this thread is taken
  // the compaction scan's scratch: the one not read since the last barrier
  uint32_t* cscan = lds.wave_tot[1];
  if (all) {
#pragma unroll
    for (int j = 0; j < E; ++j) take |= static_cast<uint32_t>(key[j] != 0u) << j;
  } else if (cnt <= kSmallCand) {
    // rank the few boundary candidates directly
    // element j's list slot (< kSmallCand: 4 bits) in nibble j % 8 of slot4[j / 8]
    static_assert(kSmallCand <= 16, "slots in 4 bits");
    uint32_t is_cand = 0;  // bit j: element j is a boundary candidate
    uint32_t slot4[(E + 7) / 8];
#pragma unroll
    for (int q = 0; q < (E + 7) / 8; ++q) slot4[q] = 0u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if (key[j] != 0u && (key[j] & mask) == prefix) {
        const uint32_t s = atomicAdd(&lds.ncand, 1u);
        lds.cand_key[s] = key[j];
        lds.cand_idx[s] = index_of(j);
        is_cand |= 1u << j;
        slot4[j / 8] |= s << (4 * (j % 8));
      }
    }
    __syncthreads();
    if (tid < 64) {  // wave 0: lane i holds candidate i; the others come by readlane
      const bool have = tid < static_cast<int>(cnt);
      const uint32_t mk = have ? lds.cand_key[tid] : 0u;
      const int32_t mi = have ? lds.cand_idx[tid] : 0;
      uint32_t rank = 0;
      for (uint32_t u = 0; u < cnt; ++u) {
        const uint32_t uk = __builtin_amdgcn_readlane(mk, u);
        const int32_t ui = __builtin_amdgcn_readlane(mi, u);
        rank += (uk > mk || (uk == mk && ui < mi)) ? 1u : 0u;
      }
      if (have) lds.cand_take[tid] = rank < k_rem;
    }
    __syncthreads();
    const uint32_t thr_hi = prefix | ~mask;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      bool t = key[j] > thr_hi;
      if ((is_cand >> j) & 1u) t = lds.cand_take[(slot4[j / 8] >> (4 * (j % 8))) & 15u] != 0u;
      take |= static_cast<uint32_t>(t) << j;
    }
  } else {
    // three full passes: prefix is the exact boundary key; the first k_rem of
    // its equal keys (in index order) are taken
    uint32_t n_eq = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) n_eq += key[j] == prefix;
    uint32_t tot;
    uint32_t eq_before = block_exclusive_scan(n_eq, lds.wave_tot[1], &tot);
    cscan = lds.wave_tot[0];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      bool t = key[j] > prefix;
      if (key[j] == prefix) {
        t = eq_before < k_rem;
        ++eq_before;
      }
      take |= static_cast<uint32_t>(t) << j;
    }
  }

  // ---- compaction in index order ----
  uint32_t tot;
  uint32_t pos = block_exclusive_scan(__builtin_popcount(take), cscan, &tot);
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (((take >> j) & 1u) && pos < static_cast<uint32_t>(K_out)) {  // pos < ksel <= K_out by construction
      idx_out[out_base + pos] = index_of(j);
      if constexpr (OUT_CAND) cand_key_out[out_base + pos] = key[j];
      ++pos;
    }
  }
  for (int j = static_cast<int>(ksel) + tid; j < K_out; j += kTopkThreads) {
    idx_out[out_base + j] = -1;
    if constexpr (OUT_CAND) cand_key_out[out_base + j] = 0u;
  }
}

template <bool SRC_CAND, bool OUT_CAND>
dsa_status_t run_select(int per_wg, bool vec, dim3 grid, int n_in, int causal_T, const int32_t* seq_lens,
                        int64_t in_stride,
                        int chunk_elems, const float* scores, const uint32_t* ck_in,
                        const int32_t* ci_in, int K_out, int32_t* idx_out, uint32_t* ck_out,
                        hipStream_t stream) {
  LaunchTimer timer;
#define DSA_TOPK_LAUNCH(EV, VEC)                                                                \
  hipExtLaunchKernelGGL(topk_select<EV, SRC_CAND, OUT_CAND, VEC>, grid, dim3(kTopkThreads), 0,  \
                        stream, timer.start(), timer.stop(), 0, n_in, causal_T, seq_lens,       \
                        in_stride, chunk_elems,                                                 \
                        scores, ck_in, ci_in, K_out, idx_out, ck_out)
  if (per_wg <= 8 * kTopkThreads) {
    if (vec) DSA_TOPK_LAUNCH(8, true); else DSA_TOPK_LAUNCH(8, false);
  } else if (per_wg <= 16 * kTopkThreads) {
    if (vec) DSA_TOPK_LAUNCH(16, true); else DSA_TOPK_LAUNCH(16, false);
  } else {
    if (vec) DSA_TOPK_LAUNCH(32, true); else DSA_TOPK_LAUNCH(32, false);
  }
#undef DSA_TOPK_LAUNCH
  return timer.done(SRC_CAND ? "topk_merge" : OUT_CAND ? "topk_chunk" : "topk_select");
}

// ---------------------------------------------------------------------------
// Long rows (more keys than one workgroup holds), in two launches over the
// row's chunks of kLongChunk keys, one workgroup per chunk.  The chunks of a
// row meet through per-row words of the workspace guarded by the call's tag,
// so nothing needs zeroing beforehand:
//   meet[0] = tag << 24 | arrivals of launch 1 << 12   (12-bit counts)
//   meet[1] = the tag once the row's histogram has been zeroed for this call
//   meet[2] = tag << 24 | arrivals of launch 2         (24-bit count)
// A word holding another tag is stale (an earlier call, or whatever the
// workspace held) and counts as zero.
//  1. topk_long_hist: a chunk's 12-bit histogram of its selectable keys is
//     added into the row's with device-scope atomics; the row's first
//     arriving workgroup zeroes the row's histogram first and publishes the
//     tag in meet[1], which later arrivals wait for (the first one is
//     already running, so the wait ends).
//  2. topk_long_gather: every workgroup finds the bin holding the row's K-th
//     key from the complete histogram and stores its chunk's selectable keys
//     in that bin or above it (every selectable key when the row has at most
//     K) as (key, index) pairs, in index order, into the chunk's slot (device-
//     scope stores).  The row's last arriving workgroup narrows the K-th key
//     k_T from the pairs inside the boundary bin (two 10-bit levels) and,
//     where keys equal to k_T must be split by index, the highest index taken
//     i_T (three 9-bit levels, lowest index first); it writes the indices of
//     the pairs with key > k_T, or key == k_T and index <= i_T, in chunk
//     order (so ascending), pads the row with -1, and marks the row's words
//     stale so that a replay of the same call starts afresh.
// The same (score, index) order as the single-workgroup select.
// ---------------------------------------------------------------------------
constexpr int kLongThreads = 1024;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kLongE = 4;                             // keys per thread
constexpr int kLongChunk = kLongThreads * kLongE;     // 4096 keys per workgroup
constexpr int kLongBins = 4096;                       // 12-bit first level
constexpr int kLongBins2 = 1024;                      // 10-bit key levels
constexpr int kLongBins3 = 512;                       // 9-bit index levels
constexpr int kLongMaxChunks = 2048;                  // chunk offsets in the tail's LDS
constexpr int kLongMeetWords = 4;                     // uint64 per row
constexpr int kLongHeld = 8;                          // pairs per thread in the tail's registers

// exclusive prefix sum over the workgroup's threads; *total gets the sum.
// One barrier; wave_tot must not be written again before the next barrier.
__device__ __forceinline__ uint32_t long_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kLongWaves; ++w) {
    const uint32_t t = wave_tot[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  *total = tot;
  return before + inc - v;
}

// The bin where the running count reaches k (from the top bin down when DESC,
// from bin 0 up otherwise) and the count before it, into sel[0], sel[1]
// (published by the caller's next barrier); returns the histogram's total.
template <int NB, bool DESC>
__device__ __forceinline__ uint32_t long_boundary(const uint32_t* h, uint32_t k, uint32_t* wave_tot,
                                                  uint32_t* sel) {
  constexpr int per = NB / kLongThreads > 0 ? NB / kLongThreads : 1;
  const int t = static_cast<int>(threadIdx.x);
  uint32_t c[per];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    const int i = t * per + j;
    c[j] = i < NB ? h[DESC ? NB - 1 - i : i] : 0u;
    local += c[j];
  }
  uint32_t tot;
  uint32_t acc = long_scan(local, wave_tot, &tot);
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (acc < k && k <= acc + c[j]) {
      const int i = t * per + j;
      sel[0] = static_cast<uint32_t>(DESC ? NB - 1 - i : i);
      sel[1] = acc;
    }
    acc += c[j];
  }
  return tot;
}

// This thread's kLongE keys of the chunk starting at c0 of a row of S scores
// in memory, of which the first n count (the rest are key 0: never
// selectable); thread t holds keys [kLongE t, kLongE t + kLongE).  Loads are
// all issued before any is used (positions clamped into the row), then masked.
template <bool VEC>
__device__ __forceinline__ void long_load(const float* row_scores, int S, int n, int c0, uint32_t (&key)[kLongE]) {
  const int i0 = c0 + static_cast<int>(threadIdx.x) * kLongE;
  if (VEC && i0 + kLongE <= S) {
    const float4 f4 = *reinterpret_cast<const float4*>(row_scores + i0);  // read again by the second launch
    key[0] = score_key(f4.x); key[1] = score_key(f4.y); key[2] = score_key(f4.z); key[3] = score_key(f4.w);
  } else {
#pragma unroll
    for (int j = 0; j < kLongE; ++j) key[j] = score_key(row_scores[min(i0 + j, S - 1)]);
  }
#pragma unroll
  for (int j = 0; j < kLongE; ++j) key[j] &= 0u - static_cast<uint32_t>(i0 + j < n);
}

// Arrival on a tagged word: returns the arrival count including this one
// (1 for the arrival that installs the call's tag).  A compare and swap is
// retried only while the word is stale.
__device__ __forceinline__ uint32_t long_arrive(uint64_t* word, uint64_t tag, uint64_t one, uint64_t count_mask) {
  uint64_t old = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if ((old >> 24) == tag) {
      const uint64_t prev = __hip_atomic_fetch_add(word, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return static_cast<uint32_t>(((prev / one) & count_mask) + 1);
    }
    if (__hip_atomic_compare_exchange_strong(word, &old, (tag << 24) | one, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return 1u;
  }
}

template <bool VEC>
__global__ void __launch_bounds__(kLongThreads)
topk_long_hist(int S, int causal_T, const int32_t* __restrict__ seq_lens, const float* __restrict__ scores,
               uint64_t* __restrict__ meet, uint32_t* __restrict__ hist, uint64_t tag) {
  __shared__ uint32_t h[kLongBins];
  __shared__ uint32_t first;
  debug_poison_lds<sizeof(h)>(h);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  uint32_t key[kLongE];
  long_load<VEC>(scores + row * S, S, row_keys(row, S, causal_T, seq_lens), blockIdx.x * kLongChunk, key);
  for (int i = tid; i < kLongBins; i += kLongThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kLongE; ++j)
    if (key[j] != 0u) atomicAdd(&h[key[j] >> 20], 1u);
  uint64_t* st = meet + row * kLongMeetWords;
  uint32_t* gh = hist + row * kLongBins;
  if (tid == 0) first = long_arrive(st, tag, uint64_t(1) << 12, 0xfffu) == 1u ? 1u : 0u;
  __syncthreads();
  if (first) {  // the first arrival: a zeroed row histogram, then the tag
    for (int i = tid; i < kLongBins; i += kLongThreads)
      __hip_atomic_store(gh + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) __hip_atomic_store(st + 1, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (tid == 0) {  // wait for the first arrival's zeroing (it is running)
    for (int spin = 0; spin < kSelWaitSpins &&
                       __hip_atomic_load(st + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag;
         ++spin)
      __builtin_amdgcn_s_sleep(4);
  }
  __syncthreads();
  for (int i = tid; i < kLongBins; i += kLongThreads) {
    const uint32_t c = h[i];
    if (c != 0u) __hip_atomic_fetch_add(gh + i, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool VEC>
__global__ void __launch_bounds__(kLongThreads)
topk_long_gather(int S, int causal_T, const int32_t* __restrict__ seq_lens, int K, int nchunk,
                 const float* __restrict__ scores, uint64_t* __restrict__ meet,
                 const uint32_t* __restrict__ hist, uint32_t* __restrict__ counts, uint64_t* __restrict__ pairs,
                 int32_t* __restrict__ idx_out, uint64_t tag) {
  // the row histogram; in the tail, [0, 1024) the narrowing histograms and
  // [1024, 1024 + nchunk] the chunks' pair offsets
  __shared__ __attribute__((aligned(16))) uint32_t h[kLongBins];
  __shared__ uint32_t wave_tot[2][kLongWaves];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t last;
  debug_poison_lds<sizeof(h)>(h);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int chunk = blockIdx.x;
  const int c0 = chunk * kLongChunk;
  uint32_t key[kLongE];
  long_load<VEC>(scores + row * S, S, row_keys(row, S, causal_T, seq_lens), c0, key);
  reinterpret_cast<u32x4_t*>(h)[tid] = reinterpret_cast<const u32x4_t*>(hist + row * kLongBins)[tid];
  __syncthreads();
  const uint32_t nvalid = long_boundary<kLongBins, true>(h, static_cast<uint32_t>(K), wave_tot[0], sel);
  __syncthreads();
  const bool all = nvalid <= static_cast<uint32_t>(K);
  const uint32_t b1 = all ? 0u : sel[0];
  const uint32_t above1 = all ? 0u : sel[1];
  // the chunk's pairs: selectable keys in the boundary bin or above, index order
  uint32_t in = 0u;
#pragma unroll
  for (int j = 0; j < kLongE; ++j) in |= static_cast<uint32_t>(key[j] != 0u && (key[j] >> 20) >= b1) << j;
  uint32_t m;
  uint32_t pos = long_scan(static_cast<uint32_t>(__builtin_popcount(in)), wave_tot[1], &m);
  uint64_t* slot = pairs + (row * nchunk + chunk) * static_cast<int64_t>(kLongChunk);
  const int i0 = c0 + tid * kLongE;
#pragma unroll
  for (int j = 0; j < kLongE; ++j)
    if ((in >> j) & 1u)
      __hip_atomic_store(slot + pos++, (static_cast<uint64_t>(key[j]) << 32) | static_cast<uint32_t>(i0 + j),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) __hip_atomic_store(counts + row * nchunk + chunk, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's pair stores are complete
  __syncthreads();
  uint64_t* st = meet + row * kLongMeetWords;
  if (tid == 0) last = long_arrive(st + 2, tag, 1u, 0xffffffu) == static_cast<uint32_t>(nchunk) ? 1u : 0u;
  __syncthreads();
  if (!last) return;

  // ---- the row's last workgroup: every chunk's pairs are stored ----
  uint32_t* offs = h + kLongBins2;  // offs[c] = pairs before chunk c, offs[nchunk] = all
  {
    uint32_t cnt[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = 2 * tid + q;
      cnt[q] = c < nchunk ? __hip_atomic_load(counts + row * nchunk + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0u;
    }
    uint32_t tot;
    const uint32_t before = long_scan(cnt[0] + cnt[1], wave_tot[0], &tot);
    if (2 * tid < nchunk) offs[2 * tid] = before;
    if (2 * tid + 1 < nchunk) offs[2 * tid + 1] = before + cnt[0];
    if (tid == 0) offs[nchunk] = tot;
  }
  __syncthreads();
  const uint32_t M = offs[nchunk];
  const uint64_t* row_pairs = pairs + row * nchunk * static_cast<int64_t>(kLongChunk);
  // Pairs in chunk order are visited in rounds of kLongHeld * kLongThreads:
  // thread t holds pairs base + kLongHeld t + r in registers.  A row with at
  // most one round of pairs (the usual case) loads them once; a larger one
  // reloads its rounds on every pass.  A pair's chunk: binary search over
  // offs, all of a thread's searches in lockstep.
  constexpr uint32_t kRound = kLongHeld * kLongThreads;
  int top = nchunk > 1 ? 1 : 0;   // the largest power of two <= nchunk - 1
  while (top != 0 && 2 * top <= nchunk - 1) top *= 2;
  uint64_t held[kLongHeld];
  auto load_round = [&](uint32_t base) {
    int c[kLongHeld];
#pragma unroll
    for (int r = 0; r < kLongHeld; ++r) c[r] = 0;
    const uint32_t v0 = base + static_cast<uint32_t>(tid) * kLongHeld;
    for (int step = top; step > 0; step >>= 1)
#pragma unroll
      for (int r = 0; r < kLongHeld; ++r) {
        const int nc = c[r] + step;
        if (nc < nchunk && offs[nc] <= v0 + r) c[r] = nc;
      }
#pragma unroll
    for (int r = 0; r < kLongHeld; ++r) {
      const uint32_t v = v0 + r;
      held[r] = v < M ? __hip_atomic_load(row_pairs + static_cast<int64_t>(c[r]) * kLongChunk + (v - offs[c[r]]),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : 0u;
    }
  };
  const bool one_round = M <= kRound;
  if (one_round) load_round(0);
  // f(pair) for every pair (pairs past M are 0: key 0, never counted)
  auto visit = [&](auto&& f) {
    for (uint32_t base = 0; base < M; base += kRound) {
      if (!one_round) load_round(base);
#pragma unroll
      for (int r = 0; r < kLongHeld; ++r) f(held[r]);
    }
  };
  uint32_t k_t = 1u;               // selected: key > k_t, or key == k_t and index <= i_t
  uint32_t i_t = 0xffffffffu;
  const uint32_t ksel = all ? nvalid : static_cast<uint32_t>(K);
  if (!all) {
    uint32_t k_rem = static_cast<uint32_t>(K) - above1;   // from the boundary bin: 1 .. its size
    uint32_t prefix = b1 << 20;
#pragma unroll 1
    for (int lvl = 0; lvl < 2; ++lvl) {
      const int shift = lvl == 0 ? 10 : 0;
      const uint32_t mask = lvl == 0 ? 0xfff00000u : 0xfffffc00u;
      h[tid] = 0u;
      __syncthreads();
      visit([&](uint64_t pr) {
        const uint32_t kk = static_cast<uint32_t>(pr >> 32);
        if (kk != 0u && (kk & mask) == prefix) atomicAdd(&h[(kk >> shift) & (kLongBins2 - 1)], 1u);
      });
      __syncthreads();
      (void)long_boundary<kLongBins2, true>(h, k_rem, wave_tot[lvl], sel);
      __syncthreads();
      prefix |= sel[0] << shift;
      k_rem -= sel[1];
    }
    k_t = prefix;                                 // the exact K-th key; k_rem of its equals are taken
    const uint32_t n_eq = h[k_t & (kLongBins2 - 1)];
    if (n_eq > k_rem) {
      // equal keys split by index: the k_rem-th smallest index among them
      uint32_t iprefix = 0u, imask = 0u, i_rem = k_rem;
#pragma unroll 1
      for (int lvl = 0; lvl < 3; ++lvl) {
        const int shift = 18 - 9 * lvl;
        __syncthreads();
        if (tid < kLongBins3) h[tid] = 0u;
        __syncthreads();
        visit([&](uint64_t pr) {
          const uint32_t ii = static_cast<uint32_t>(pr);
          if (static_cast<uint32_t>(pr >> 32) == k_t && (ii & imask) == iprefix)
            atomicAdd(&h[(ii >> shift) & (kLongBins3 - 1)], 1u);
        });
        __syncthreads();
        (void)long_boundary<kLongBins3, false>(h, i_rem, wave_tot[lvl & 1], sel);
        __syncthreads();
        iprefix |= sel[0] << shift;
        imask |= static_cast<uint32_t>(kLongBins3 - 1) << shift;
        i_rem -= sel[1];
      }
      i_t = iprefix;
    }
  }
  // the selected pairs in chunk order: ascending indices
  int32_t* out = idx_out + row * K;
  uint32_t written = 0u;
  int it = 0;
#pragma unroll 1
  for (uint32_t base = 0; base < M; base += kRound, ++it) {
    if (!one_round) load_round(base);
    uint32_t take = 0u;
#pragma unroll
    for (int r = 0; r < kLongHeld; ++r) {
      const uint32_t kk = static_cast<uint32_t>(held[r] >> 32);
      const uint32_t ii = static_cast<uint32_t>(held[r]);
      const bool t = kk != 0u && (all || kk > k_t || (kk == k_t && ii <= i_t));
      take |= static_cast<uint32_t>(t) << r;
    }
    uint32_t tot;
    uint32_t p = written + long_scan(static_cast<uint32_t>(__builtin_popcount(take)), wave_tot[it & 1], &tot);
#pragma unroll
    for (int r = 0; r < kLongHeld; ++r)
      if (((take >> r) & 1u) && p < static_cast<uint32_t>(K))  // p < ksel by construction
        out[p++] = static_cast<int32_t>(static_cast<uint32_t>(held[r]));
    written += tot;
  }
  for (int j = static_cast<int>(ksel) + tid; j < K; j += kLongThreads) out[j] = -1;
  if (tid == 0) {
    __hip_atomic_store(st, (tag | kTagStale) << 24, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st + 1, tag | kTagStale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st + 2, (tag | kTagStale) << 24, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct TopkPlan {
  int chunks;      // chunks per row (1 = one workgroup per row)
  int chunk_elems;
  bool long_rows;  // the two-launch long-row select
};

// Rows longer than one workgroup's capacity: exact per-chunk candidates and
// one merge workgroup per row, with the smaller chunk (16 K elements) when
// its candidate lists still fit the merge, since it spreads stage 1 over
// twice the workgroups, else 32 K.  Rows whose candidates fit neither (more
// than 16 chunks of K, or K of a chunk or more) take the long-row select.
TopkPlan plan(const dsa_shape_t& s) {
  TopkPlan p{1, s.S, false};
  if (s.S <= kChunkElems) return p;
  const int64_t K = k_eff(s);
  for (int ce = kChunkElems / 2; ce <= kChunkElems; ce *= 2) {
    const int64_t chunks = (s.S + ce - 1) / ce;
    if (chunks * K <= kChunkElems && K < ce) {
      p.chunk_elems = ce;
      p.chunks = static_cast<int>(chunks);
      return p;
    }
  }
  p.long_rows = true;
  p.chunk_elems = kLongChunk;
  p.chunks = (s.S + kLongChunk - 1) / kLongChunk;
  return p;
}

// long-row workspace: per row the meeting words, the 12-bit histogram, the
// chunks' pair counts and a slot of kLongChunk pairs per chunk
struct LongWs {
  size_t meet_words, hist_words, cnt_words, pair_words;  // uint64, uint32, uint32, uint64
};
LongWs long_ws(const dsa_shape_t& s, const TopkPlan& p) {
  const size_t rows = static_cast<size_t>(s.B) * s.T;
  return LongWs{rows * kLongMeetWords, rows * kLongBins, (rows * p.chunks + 63) / 64 * 64,
                rows * p.chunks * static_cast<size_t>(kLongChunk)};
}

}  // namespace

size_t topk_workspace_bytes(const dsa_shape_t& s) {
  const TopkPlan p = plan(s);
  if (p.chunks == 1) return 0;
  if (p.long_rows) {
    const LongWs w = long_ws(s, p);
    return (w.meet_words + w.pair_words) * sizeof(uint64_t) + (w.hist_words + w.cnt_words) * sizeof(uint32_t);
  }
  const size_t rows = static_cast<size_t>(s.B) * s.T;
  return rows * p.chunks * k_eff(s) * (sizeof(uint32_t) + sizeof(int32_t));
}

dsa_status_t topk_check(const dsa_shape_t& s) {
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  if (rows > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "topk: B*T = %lld exceeds 65535 rows",
                static_cast<long long>(rows));
  const TopkPlan p = plan(s);
  if (p.long_rows && p.chunks > kLongMaxChunks)
    return fail(DSA_ERR_UNSUPPORTED, "topk: S = %d exceeds the long-row select's %d keys", s.S,
                kLongMaxChunks * kLongChunk);
  return DSA_OK;
}

namespace {
dsa_status_t long_rows_launch(const dsa_shape_t& s, const TopkPlan& p, const float* scores, int causal_T,
                              const int32_t* seq_lens, int32_t* idx, void* ws, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  const int K = k_eff(s);
  const LongWs w = long_ws(s, p);
  uint64_t* meet = static_cast<uint64_t*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(meet + w.meet_words);
  uint32_t* counts = hist + w.hist_words;
  uint64_t* pairs = reinterpret_cast<uint64_t*>(counts + w.cnt_words);
  const uint64_t tag = next_call_tag();
  const bool vec = s.S % 4 == 0;
  const dim3 grid(p.chunks, rows), block(kLongThreads);
  {
    LaunchTimer t;
    if (vec)
      hipExtLaunchKernelGGL(topk_long_hist<true>, grid, block, 0, stream, t.start(), t.stop(), 0, s.S, causal_T,
                            seq_lens, scores, meet, hist, tag);
    else
      hipExtLaunchKernelGGL(topk_long_hist<false>, grid, block, 0, stream, t.start(), t.stop(), 0, s.S, causal_T,
                            seq_lens, scores, meet, hist, tag);
    const dsa_status_t st = t.done("topk_long_hist");
    if (st != DSA_OK) return st;
  }
  LaunchTimer t;
  if (vec)
    hipExtLaunchKernelGGL(topk_long_gather<true>, grid, block, 0, stream, t.start(), t.stop(), 0, s.S, causal_T,
                          seq_lens, K, p.chunks, scores, meet, hist, counts, pairs, idx, tag);
  else
    hipExtLaunchKernelGGL(topk_long_gather<false>, grid, block, 0, stream, t.start(), t.stop(), 0, s.S, causal_T,
                          seq_lens, K, p.chunks, scores, meet, hist, counts, pairs, idx, tag);
  return t.done("topk_long_gather");
}

dsa_status_t topk_launches(const dsa_shape_t& s, const float* scores, int causal_T, const int32_t* seq_lens,
                           int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  dsa_status_t st = topk_check(s);
  if (st != DSA_OK) return st;
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  const int K = k_eff(s);
  const TopkPlan p = plan(s);
  if (p.chunks == 1) {
    return run_select<false, false>(s.S, s.S % 4 == 0, dim3(1, rows), s.S, causal_T, seq_lens, s.S, s.S,
                                    scores, nullptr, nullptr, K, idx, nullptr, stream);
  }
  const size_t need = topk_workspace_bytes(s);
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "topk: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (p.long_rows) return long_rows_launch(s, p, scores, causal_T, seq_lens, idx, ws, stream);
  const int64_t n2 = static_cast<int64_t>(p.chunks) * K;
  int32_t* cand_idx = static_cast<int32_t*>(ws);
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(cand_idx + rows * n2);
  st = run_select<false, true>(p.chunk_elems, s.S % 4 == 0, dim3(p.chunks, rows), s.S, causal_T, seq_lens,
                               s.S, p.chunk_elems, scores, nullptr, nullptr, K, cand_idx, cand_key, stream);
  if (st != DSA_OK) return st;
  return run_select<true, false>(static_cast<int>(n2), n2 % 4 == 0, dim3(1, rows), static_cast<int>(n2), 0,
                                 nullptr, n2, static_cast<int>(n2), nullptr, cand_key, cand_idx, K, idx, nullptr,
                                 stream);
}
}  // namespace

dsa_status_t launch_topk(const dsa_shape_t& s, const float* scores, const int32_t* seq_lens, bool causal_rows,
                         int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  dsa_status_t st = topk_launches(s, scores, causal_rows ? s.T : 0, seq_lens, idx, ws, ws_bytes, stream);
#ifdef DSA_DEBUG
  if (st == DSA_OK)
    st = debug_check_idx(static_cast<int64_t>(s.B) * s.T, k_eff(s), s.S, true, idx, stream, "top-K output");
#endif
  return st;
}

}  // namespace dsa
