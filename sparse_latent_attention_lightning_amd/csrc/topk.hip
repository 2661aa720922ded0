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

// SRC_CAND: elements come from a candidate list (key, index) instead of fp32
// scores.  OUT_CAND: the result is a candidate list (key and index written).
// VEC: every thread's run of E inputs starts 16-byte aligned (16-byte loads).
template <int E, bool SRC_CAND, bool OUT_CAND, bool VEC>
__global__ void __launch_bounds__(kTopkThreads, (E <= 16 && !SRC_CAND && !OUT_CAND) ? 8 : 1)
topk_select(int n_in, int64_t in_stride, int chunk_elems,
            const float* __restrict__ scores, const uint32_t* __restrict__ cand_key_in,
            const int32_t* __restrict__ cand_idx_in, int K_out, int32_t* __restrict__ idx_out,
            uint32_t* __restrict__ cand_key_out) {
  __shared__ TopkLds lds;
  debug_poison_lds<sizeof(lds)>(&lds);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int chunk = blockIdx.x;
  // this workgroup's elements: [elem0, elem0 + n) of the row's input
  const int elem0 = chunk * chunk_elems;
  const int n = min(chunk_elems, n_in - elem0);
  const int64_t in_base = row * in_stride + elem0;
  const int64_t out_base = (row * gridDim.x + chunk) * static_cast<int64_t>(K_out);

  // ---- thread t owns elements [E t, E t + E): keys in registers ----
  uint32_t key[E];
  int32_t id[SRC_CAND ? E : 1];  // candidate indices; a score's index is its position
  const int i0 = tid * E;
  if (VEC && i0 + E <= n) {
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
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = i0 + j;
      if (i < n) {
        if constexpr (SRC_CAND) {
          key[j] = cand_key_in[in_base + i];
          id[j] = cand_idx_in[in_base + i];
        } else {
          key[j] = score_key(scores[in_base + i]);
        }
      } else {
        key[j] = 0u;
        if constexpr (SRC_CAND) id[j] = -1;
      }
    }
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
dsa_status_t run_select(int per_wg, bool vec, dim3 grid, int n_in, int64_t in_stride,
                        int chunk_elems, const float* scores, const uint32_t* ck_in,
                        const int32_t* ci_in, int K_out, int32_t* idx_out, uint32_t* ck_out,
                        hipStream_t stream) {
  LaunchTimer timer;
#define DSA_TOPK_LAUNCH(EV, VEC)                                                                \
  hipExtLaunchKernelGGL(topk_select<EV, SRC_CAND, OUT_CAND, VEC>, grid, dim3(kTopkThreads), 0,  \
                        stream, timer.start(), timer.stop(), 0, n_in, in_stride, chunk_elems,   \
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

struct TopkPlan {
  int chunks;      // stage-1 chunks per row (1 = single stage)
  int chunk_elems;
};

// Rows longer than one workgroup's capacity: the smaller chunk (16 K
// elements) when its candidate lists still fit one merge workgroup, since it
// spreads stage 1 over twice the workgroups; else 32 K.
TopkPlan plan(const dsa_shape_t& s) {
  TopkPlan p{1, s.S};
  if (s.S > kChunkElems) {
    const int64_t K = k_eff(s);
    p.chunk_elems = kChunkElems;
    for (int ce = kChunkElems / 2; ce <= kChunkElems; ce *= 2) {
      const int64_t chunks = (s.S + ce - 1) / ce;
      if (chunks * K <= kChunkElems && K < ce) {
        p.chunk_elems = ce;
        break;
      }
    }
    p.chunks = (s.S + p.chunk_elems - 1) / p.chunk_elems;
  }
  return p;
}

}  // namespace

size_t topk_workspace_bytes(const dsa_shape_t& s) {
  const TopkPlan p = plan(s);
  if (p.chunks == 1) return 0;
  const size_t rows = static_cast<size_t>(s.B) * s.T;
  return rows * p.chunks * k_eff(s) * (sizeof(uint32_t) + sizeof(int32_t));
}

dsa_status_t topk_check(const dsa_shape_t& s) {
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  if (rows > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "topk: B*T = %lld exceeds 65535 rows",
                static_cast<long long>(rows));
  const TopkPlan p = plan(s);
  const int K = k_eff(s);
  if (p.chunks > 1 && (static_cast<int64_t>(p.chunks) * K > kChunkElems || K >= p.chunk_elems))
    return fail(DSA_ERR_UNSUPPORTED, "topk: S = %d with K = %d needs more than two stages", s.S, K);
  return DSA_OK;
}

namespace {
dsa_status_t topk_launches(const dsa_shape_t& s, const float* scores, int32_t* idx, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  dsa_status_t st = topk_check(s);
  if (st != DSA_OK) return st;
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  const int K = k_eff(s);
  const TopkPlan p = plan(s);
  if (p.chunks == 1) {
    return run_select<false, false>(s.S, s.S % 4 == 0, dim3(1, rows), s.S, s.S, s.S, scores,
                                    nullptr, nullptr, K, idx, nullptr, stream);
  }
  const int64_t n2 = static_cast<int64_t>(p.chunks) * K;
  const size_t need = topk_workspace_bytes(s);
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "topk: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  int32_t* cand_idx = static_cast<int32_t*>(ws);
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(cand_idx + rows * n2);
  st = run_select<false, true>(p.chunk_elems, s.S % 4 == 0, dim3(p.chunks, rows), s.S,
                                            s.S, p.chunk_elems, scores, nullptr, nullptr, K,
                                            cand_idx, cand_key, stream);
  if (st != DSA_OK) return st;
  return run_select<true, false>(static_cast<int>(n2), n2 % 4 == 0, dim3(1, rows),
                                 static_cast<int>(n2), n2, static_cast<int>(n2), nullptr, cand_key,
                                 cand_idx, K, idx, nullptr, stream);
}
}  // namespace

dsa_status_t launch_topk(const dsa_shape_t& s, const float* scores, int32_t* idx, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  dsa_status_t st = topk_launches(s, scores, idx, ws, ws_bytes, stream);
#ifdef DSA_DEBUG
  if (st == DSA_OK)
    st = debug_check_idx(static_cast<int64_t>(s.B) * s.T, k_eff(s), s.S, true, idx, stream, "top-K output");
#endif
  return st;
}

}  // namespace dsa
