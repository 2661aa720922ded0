// Top-K of one score row by one 256-thread workgroup, from a 12-bit
// histogram of the row that is already complete and the row's fp32 scores in
// global memory (the M^sel step of the atlas DeepSeek-V3.2-Exp MoE-block step
// list; row layout int32 [min(K, keys)] ascending, padded with -1, from the
// nnterp deepseek_v32 page, section 03).
//
// Order: score descending, then index ascending; -0 == +0; NaN and -inf are
// never selected (their key is 0).  The K-th largest key is narrowed MSB
// first over the order-preserving 32-bit key, 12 + 10 + 10 bits: the given
// histogram fixes the top 12.  One pass over the row then marks every
// element above the boundary bin in an LDS bitmap and copies the elements of
// the boundary bin (key, index) into an LDS list, whose 10-bit histograms fix
// the remaining bits until the boundary bin holds few enough elements to be
// ranked directly (by key, then index) or the key is exact (then its equal
// elements are taken in index order through a second bitmap).  Only when the
// boundary bin is too large for the list do 10-bit passes over the row come
// first.  Each thread finally owns a contiguous run of bitmap words, so a
// block prefix sum of their counts places the indices in ascending order.
//
// Scores and histogram are read with device-scope loads: other workgroups
// wrote them (with device-scope stores and atomics) and this workgroup must
// not read a stale cached copy.
#pragma once
#include "dsa_device.h"

namespace dsa {
namespace sel {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBins1 = 4096;     // the first level: 12 bits (sign, exponent, 3 mantissa bits)
constexpr int kBins2 = 1024;     // the later levels: 10 bits each
constexpr int kDirect = 64;      // boundary bins this small are ranked by one wave
constexpr int kList = 4096;      // boundary elements held in LDS
constexpr int kMaxRow = 262144;  // longest row: the two bitmaps take 2 x 32 KB
constexpr int kBatch = 16;       // row reads in flight per thread (16 bytes each)
constexpr int kSc1 = 16;         // cache policy of a device-scope load (sc1)

struct alignas(16) Lds {
  uint32_t hist[kBins1];
  uint32_t bits[2 * (kMaxRow / 32)];  // selected, then equal-to-the-exact-boundary
  uint32_t list_key[kList];
  int32_t list_idx[kList];
  uint32_t small_key[kDirect];
  int32_t small_idx[kDirect];
  uint32_t wave_tot[2][kWaves];
  uint32_t sel_bin, sel_above;
  uint32_t nlist, nsmall;
};

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// Exclusive prefix sum over the 256 threads in thread order; *total gets the
// sum.  One barrier; wave_tot must not be reused before the next barrier.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = wave_tot[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  *total = tot;
  return before + inc - v;
}

// Bins [NB - (t+1) per, NB - t per) belong to thread t (scanned from the
// top): the bin where the running count from the top reaches k_rem and the
// count above it go to sel_bin / sel_above (nothing is recorded when the
// histogram's total is below k_rem, which is returned).
template <int NB>
__device__ __forceinline__ uint32_t find_boundary(Lds& L, uint32_t k_rem, int slot) {
  constexpr int per = NB / kThreads;
  const int hi_bin = NB - static_cast<int>(threadIdx.x) * per;  // exclusive
  uint32_t c[per];
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    c[k] = L.hist[hi_bin - 1 - k];
    local += c[k];
  }
  uint32_t tot;
  uint32_t acc = block_scan(local, L.wave_tot[slot], &tot);
#pragma unroll
  for (int k = 0; k < per; ++k) {
    if (acc < k_rem && k_rem <= acc + c[k]) {
      L.sel_bin = static_cast<uint32_t>(hi_bin - 1 - k);
      L.sel_above = acc;
    }
    acc += c[k];
  }
  return tot;
}

// Visits every element of the row: f(index, key).  Thread t takes 4
// consecutive elements per round of 1024, kBatch rounds read before any is
// used (device-scope buffer loads; reads past the row return 0 and are not
// visited).
template <typename F>
__device__ __forceinline__ void for_each_row(__amdgpu_buffer_rsrc_t row, int S, F&& f) {
  const int t4 = 4 * static_cast<int>(threadIdx.x);
  for (int base = 0; base < S; base += kBatch * 4 * kThreads) {
    u32x4v v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      v[b] = __builtin_amdgcn_raw_buffer_load_b128(row, 4 * (base + 4 * kThreads * b + t4), 0, kSc1);
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = base + 4 * kThreads * b + t4 + e;
        if (i < S) f(i, score_key(__uint_as_float(v[b][e])));
      }
  }
}

// One narrowing level: a 10-bit histogram of the elements still in the
// boundary bin (visit(g) calls g(key) for each candidate element), then the
// new boundary; updates prefix / mask / k_rem / cnt.
template <typename V>
__device__ __forceinline__ void narrow(Lds& L, int shift, V&& visit, uint32_t& prefix, uint32_t& mask,
                                       uint32_t& k_rem, uint32_t& cnt, int slot) {
  const int tid = threadIdx.x;
  __syncthreads();  // every thread is done with the previous histogram
  for (int i = tid; i < kBins2; i += kThreads) L.hist[i] = 0u;
  __syncthreads();
  const uint32_t pf = prefix, mk = mask;
  visit([&](uint32_t key) {
    if ((key & mk) == pf) atomicAdd(&L.hist[(key >> shift) & (kBins2 - 1)], 1u);
  });
  __syncthreads();
  (void)find_boundary<kBins2>(L, k_rem, slot);
  __syncthreads();
  const uint32_t bin = L.sel_bin;
  prefix |= bin << shift;
  mask |= static_cast<uint32_t>(kBins2 - 1) << shift;
  k_rem -= L.sel_above;
  cnt = L.hist[bin];
}

// The selection.  row_ptr: the row's S scores; ghist: its 12-bit histogram
// of selectable keys (key != 0; bin = key >> 20); out: K int32.  All 256
// threads call it; L lives in LDS.
__device__ void select_row(Lds& L, const float* row_ptr, int S, const uint32_t* ghist, int K,
                           int32_t* out) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t row =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row_ptr), 0, 4 * S, 0x00020000);
  {  // the histogram: all of a thread's reads in flight at once
    const __amdgpu_buffer_rsrc_t gh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(ghist), 0, 4 * kBins1, 0x00020000);
    constexpr int kPer = kBins1 / (4 * kThreads);  // 16-byte reads per thread
    u32x4v h[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      h[k] = __builtin_amdgcn_raw_buffer_load_b128(gh, 16 * (tid + kThreads * k), 0, kSc1);
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      *reinterpret_cast<u32x4v*>(&L.hist[4 * (tid + kThreads * k)]) = h[k];
  }
  if (tid == 0) {
    L.nlist = 0u;
    L.nsmall = 0u;
  }
  __syncthreads();
  const uint32_t nvalid = find_boundary<kBins1>(L, static_cast<uint32_t>(K), 0);
  __syncthreads();
  const uint32_t ksel = min(static_cast<uint32_t>(K), nvalid);
  const bool all = nvalid <= static_cast<uint32_t>(K);
  // keys > (prefix | ~mask) are taken; keys with (key & mask) == prefix are
  // the boundary candidates (cnt of them), of which k_rem are taken
  uint32_t prefix = 0u, mask = 0u, k_rem = ksel, cnt = 0u;
  int level = 1;  // levels fixed so far: 12, then 10 and 10 bits
  constexpr int kShift[3] = {20, 10, 0};
  if (!all) {
    prefix = L.sel_bin << 20;
    mask = 0xfff00000u;
    k_rem -= L.sel_above;
    cnt = L.hist[L.sel_bin];
    // boundary bins too large for the LDS list: narrow over the row first
    while (cnt > static_cast<uint32_t>(kList) && level < 3) {
      narrow(L, kShift[level], [&](auto g) {
        for_each_row(row, S, [&](int, uint32_t key) {
          if (key != 0u) g(key);
        });
      }, prefix, mask, k_rem, cnt, level & 1);
      ++level;
    }
  }
  const int nwords = (S + 31) >> 5;
  uint32_t* selw = L.bits;
  uint32_t* eqw = L.bits + nwords;
  const bool list = !all && cnt <= static_cast<uint32_t>(kList);
  __syncthreads();
  for (int i = tid; i < 2 * nwords; i += kThreads) L.bits[i] = 0u;
  __syncthreads();
  {
    const uint32_t thr_hi = prefix | ~mask, pf = prefix, mk = mask;
    for_each_row(row, S, [&](int i, uint32_t key) {
      if (key == 0u) return;
      if (all || key > thr_hi) {
        atomicOr(&selw[i >> 5], 1u << (i & 31));
      } else if ((key & mk) == pf) {
        if (list) {
          const uint32_t s = atomicAdd(&L.nlist, 1u);
          if (s < static_cast<uint32_t>(kList)) {  // cnt <= kList of them (bound kept regardless)
            L.list_key[s] = key;
            L.list_idx[s] = i;
          }
        } else {
          atomicOr(&eqw[i >> 5], 1u << (i & 31));  // exact key, more equal elements than the list holds
        }
      }
    });
  }
  __syncthreads();
  if (list) {
    const int n = static_cast<int>(min(L.nlist, static_cast<uint32_t>(kList)));
    while (cnt > static_cast<uint32_t>(kDirect) && level < 3) {
      narrow(L, kShift[level], [&](auto g) {
        for (int c = tid; c < n; c += kThreads) g(L.list_key[c]);
      }, prefix, mask, k_rem, cnt, level & 1);
      ++level;
    }
    const bool direct = cnt <= static_cast<uint32_t>(kDirect);
    const uint32_t thr_hi = prefix | ~mask;
    __syncthreads();
    for (int c = tid; c < n; c += kThreads) {
      const uint32_t key = L.list_key[c];
      const int i = L.list_idx[c];
      if (key > thr_hi) {
        atomicOr(&selw[i >> 5], 1u << (i & 31));
      } else if ((key & mask) == prefix) {
        if (direct) {
          const uint32_t s = atomicAdd(&L.nsmall, 1u);
          if (s < static_cast<uint32_t>(kDirect)) {
            L.small_key[s] = key;
            L.small_idx[s] = i;
          }
        } else {
          atomicOr(&eqw[i >> 5], 1u << (i & 31));  // the key is exact: ties by index
        }
      }
    }
    __syncthreads();
    if (direct && tid < 64) {  // wave 0: lane i holds candidate i, the others come by readlane
      const uint32_t m = min(L.nsmall, static_cast<uint32_t>(kDirect));
      const bool have = tid < static_cast<int>(m);
      const uint32_t mk = have ? L.small_key[tid] : 0u;
      const int32_t mi = have ? L.small_idx[tid] : 0;
      uint32_t rank = 0;
      for (uint32_t u = 0; u < m; ++u) {
        const uint32_t uk = __builtin_amdgcn_readlane(mk, u);
        const int32_t ui = __builtin_amdgcn_readlane(mi, u);
        rank += (uk > mk || (uk == mk && ui < mi)) ? 1u : 0u;
      }
      if (have && rank < k_rem) atomicOr(&selw[mi >> 5], 1u << (mi & 31));
    }
    __syncthreads();
  }
  // compaction: thread t owns words [w0, w1); the selected elements, and the
  // first k_rem equal-to-the-boundary elements in index order
  const int per = (nwords + kThreads - 1) / kThreads;
  const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
  uint32_t nsel = 0, neq = 0;
  for (int w = w0; w < w1; ++w) {
    nsel += __builtin_popcount(selw[w]);
    neq += __builtin_popcount(eqw[w]);
  }
  uint32_t tot;
  uint32_t pos = block_scan(nsel, L.wave_tot[0], &tot);
  uint32_t eq_before = block_scan(neq, L.wave_tot[1], &tot);
  pos += min(eq_before, k_rem);  // equal elements taken by lower threads come first
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = selw[w];
    uint32_t e = eqw[w];
    while (e) {
      const uint32_t b = e & (~e + 1u);
      if (eq_before < k_rem) bits |= b;
      ++eq_before;
      e ^= b;
    }
    while (bits) {
      const int b = __builtin_ctz(bits);
      if (pos < static_cast<uint32_t>(K)) out[pos] = 32 * w + b;
      ++pos;
      bits &= bits - 1u;
    }
  }
  for (int j = static_cast<int>(ksel) + tid; j < K; j += kThreads) out[j] = -1;
}

}  // namespace sel
}  // namespace dsa
