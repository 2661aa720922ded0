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
// is found exactly by a 3-pass radix select over the order-preserving 32-bit
// key (12 + 10 + 10 bits, MSB first) with LDS histograms; the first pass uses
// 12 bits (sign, exponent and 3 mantissa bits) so that score distributions
// concentrated in a few binades still spread over many bins.
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

struct BlockScanLds {
  uint32_t wave_tot[kTopkWaves];
};

// Exclusive prefix sum over the workgroup in thread order; returns the sum of
// the values of all lower threads and sets *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, BlockScanLds& lds,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) lds.wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const uint32_t t = lds.wave_tot[i];
    before += (i < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();  // wave_tot is reused by the next scan
  *total = tot;
  return before + inc - v;
}

// SRC_CAND: elements come from a candidate list (key, index) instead of fp32
// scores.  OUT_CAND: the result is a candidate list (key and index written).
template <int E, bool SRC_CAND, bool OUT_CAND>
__global__ void __launch_bounds__(kTopkThreads)
topk_select(int n_in, int64_t in_stride, int chunk_elems,
            const float* __restrict__ scores, const uint32_t* __restrict__ cand_key_in,
            const int32_t* __restrict__ cand_idx_in, int K_out, int32_t* __restrict__ idx_out,
            uint32_t* __restrict__ cand_key_out) {
  __shared__ uint32_t hist[4096];
  __shared__ BlockScanLds scan_lds;
  __shared__ uint32_t sel_bin, sel_above;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int chunk = blockIdx.x;
  // this workgroup's elements: [elem0, elem0 + n) of the row's input
  const int elem0 = chunk * chunk_elems;
  const int n = min(chunk_elems, n_in - elem0);
  const int64_t in_base = row * in_stride + elem0;
  const int64_t out_base = (row * gridDim.x + chunk) * static_cast<int64_t>(K_out);

  uint32_t key[E];
  int32_t id[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = tid * E + j;
    if (i < n) {
      if constexpr (SRC_CAND) {
        key[j] = cand_key_in[in_base + i];
        id[j] = cand_idx_in[in_base + i];
      } else {
        key[j] = score_key(scores[in_base + i]);
        id[j] = elem0 + i;
      }
    } else {
      key[j] = 0u;
      id[j] = -1;
    }
  }

  // ---- how many selectable elements, and how many to take ----
  uint32_t nvalid_local = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) nvalid_local += key[j] != 0u;
  uint32_t nvalid;
  (void)block_exclusive_scan(nvalid_local, scan_lds, &nvalid);

  uint32_t thr = 0u;      // keys > thr are taken ...
  uint32_t take_eq = 0u;  // ... and the first take_eq keys == thr (by index)
  const uint32_t ksel = min(static_cast<uint32_t>(K_out), nvalid);
  if (nvalid > static_cast<uint32_t>(K_out)) {
    uint32_t prefix = 0u, mask = 0u, k_rem = ksel;
    constexpr int kShift[3] = {20, 10, 0};
    constexpr int kBits[3] = {12, 10, 10};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int shift = kShift[p], nb = 1 << kBits[p];
      for (int i = tid; i < nb; i += kTopkThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (key[j] != 0u && (key[j] & mask) == prefix)
          atomicAdd(&hist[(key[j] >> shift) & (nb - 1)], 1u);
      __syncthreads();
      // thread t owns bins [nb - (t+1)*per, nb - t*per), scanned from the top
      const int per = (nb + kTopkThreads - 1) / kTopkThreads;
      const int hi_bin = nb - tid * per;  // exclusive
      uint32_t local = 0;
      for (int k = 1; k <= per; ++k)
        if (hi_bin - k >= 0) local += hist[hi_bin - k];
      uint32_t tot;
      uint32_t acc = block_exclusive_scan(local, scan_lds, &tot);
      for (int k = 1; k <= per; ++k) {
        const int bin = hi_bin - k;
        if (bin < 0) break;
        const uint32_t c = hist[bin];
        if (acc < k_rem && k_rem <= acc + c) {
          sel_bin = static_cast<uint32_t>(bin);
          sel_above = acc;
        }
        acc += c;
      }
      __syncthreads();
      prefix |= sel_bin << shift;
      mask |= static_cast<uint32_t>(nb - 1) << shift;
      k_rem -= sel_above;
      __syncthreads();  // sel_bin / hist reused by the next pass
    }
    thr = prefix;
    take_eq = k_rem;
  }

  // ---- compaction in index order ----
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    n_gt += key[j] > thr;
    n_eq += (key[j] == thr) && (thr != 0u);
  }
  uint32_t tot;
  const uint32_t packed_before = block_exclusive_scan((n_gt << 16) | n_eq, scan_lds, &tot);
  uint32_t eq_before = packed_before & 0xffffu;
  const uint32_t gt_before = packed_before >> 16;
  uint32_t pos = gt_before + min(eq_before, take_eq);
#pragma unroll
  for (int j = 0; j < E; ++j) {
    bool take = key[j] > thr;
    if (key[j] == thr && thr != 0u) {
      take = eq_before < take_eq;
      ++eq_before;
    }
    if (take && pos < static_cast<uint32_t>(K_out)) {  // pos < ksel <= K_out by construction
      idx_out[out_base + pos] = id[j];
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
dsa_status_t run_select(int per_wg, dim3 grid, int n_in, int64_t in_stride, int chunk_elems,
                        const float* scores, const uint32_t* ck_in, const int32_t* ci_in,
                        int K_out, int32_t* idx_out, uint32_t* ck_out, hipStream_t stream) {
#define DSA_TOPK_LAUNCH(EV)                                                               \
  hipExtLaunchKernelGGL(topk_select<EV, SRC_CAND, OUT_CAND>, grid, dim3(kTopkThreads), 0, stream, \
                        timer.start(), timer.stop(), 0, n_in, in_stride, chunk_elems, scores,     \
                        ck_in, ci_in, K_out, idx_out, ck_out)
  LaunchTimer timer;
  if (per_wg <= 8 * kTopkThreads) DSA_TOPK_LAUNCH(8);
  else if (per_wg <= 16 * kTopkThreads) DSA_TOPK_LAUNCH(16);
  else DSA_TOPK_LAUNCH(32);
#undef DSA_TOPK_LAUNCH
  return timer.done(SRC_CAND ? "topk_merge" : OUT_CAND ? "topk_chunk" : "topk_select");
}

struct TopkPlan {
  int chunks;      // stage-1 chunks per row (1 = single stage)
  int chunk_elems;
};

TopkPlan plan(const dsa_shape_t& s) {
  TopkPlan p{1, s.S};
  if (s.S > kChunkElems) {
    p.chunk_elems = kChunkElems;
    p.chunks = (s.S + kChunkElems - 1) / kChunkElems;
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

dsa_status_t launch_topk(const dsa_shape_t& s, const float* scores, int32_t* idx, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  if (rows > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "topk: B*T = %lld exceeds 65535 rows",
                static_cast<long long>(rows));
  const int K = k_eff(s);
  const TopkPlan p = plan(s);
  if (p.chunks == 1) {
    return run_select<false, false>(s.S, dim3(1, rows), s.S, s.S, s.S, scores, nullptr, nullptr,
                                    K, idx, nullptr, stream);
  }
  const int64_t n2 = static_cast<int64_t>(p.chunks) * K;
  if (n2 > kChunkElems || K >= p.chunk_elems)
    return fail(DSA_ERR_UNSUPPORTED, "topk: S = %d with K = %d needs more than two stages", s.S, K);
  const size_t need = topk_workspace_bytes(s);
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "topk: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  int32_t* cand_idx = static_cast<int32_t*>(ws);
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(cand_idx + rows * n2);
  dsa_status_t st = run_select<false, true>(p.chunk_elems, dim3(p.chunks, rows), s.S, s.S,
                                            p.chunk_elems, scores, nullptr, nullptr, K, cand_idx,
                                            cand_key, stream);
  if (st != DSA_OK) return st;
  return run_select<true, false>(static_cast<int>(n2), dim3(1, rows), static_cast<int>(n2), n2,
                                 static_cast<int>(n2), nullptr, cand_key, cand_idx, K, idx,
                                 nullptr, stream);
}

}  // namespace dsa
