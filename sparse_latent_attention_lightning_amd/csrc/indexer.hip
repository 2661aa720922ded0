// Lightning-indexer scores on gfx950.
//
// S[b,t,s] = idx_scale * sum_h w[b,t,h] * ReLU(q_idx[b,t,h,:] . k_idx[b,s,:])
// for s <= q_pos(t) = S - T + t, and -inf for later keys (atlas.klimoza.dev,
// DeepSeek-V3.2-Exp MoE block, "All 43 steps": the index score S^I and the
// causal mask M added to it).  The head sum accumulates in fp32 and the
// prefactor multiplies it once, after the sum.
//
// Two kernels:
//  * indexer_mfma: 64 heads x 128 dims (the V3.2 indexer), bf16 or e4m3.
//    One wave scores 16 keys at a time as a [64 heads] x [16 keys] MFMA tile
//    (heads on the M side, keys on the N side, the 128 dims as the reduction),
//    loading each key row straight from global memory into the MFMA operand
//    registers: every key byte is read once, with no LDS round trip.  The
//    query tile sits in registers for the wave's whole key range.  ReLU, the
//    head weights and the head sum run on the accumulator registers: each
//    lane holds 16 heads of one key, sums them, and two cross-lane adds finish
//    the 64-head reduction.
//  * indexer_generic: any HI x DI, f32 / bf16 / e4m3, plain fp32 VALU loops.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

template <int WDT>
__device__ __forceinline__ float load_w(const void* w, int64_t i) {
  if constexpr (WDT == DSA_BF16)
    return bf16_to_f32(static_cast<const uint16_t*>(w)[i]);
  else
    return static_cast<const float*>(w)[i];
}

template <int IDT>
__device__ __forceinline__ float load_idx(const void* p, int64_t i) {
  if constexpr (IDT == DSA_BF16)
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else if constexpr (IDT == DSA_FP8_E4M3)
    return e4m3_to_f32(static_cast<const uint8_t*>(p)[i]);
  else
    return static_cast<const float*>(p)[i];
}

// ---------------------------------------------------------------------------
// generic kernel: one thread per (query row, key); the query row and its head
// weights are staged in LDS as fp32.
// ---------------------------------------------------------------------------
template <int IDT, int WDT>
__global__ void __launch_bounds__(256)
indexer_generic(int T, int S, int HI, int DI, float idx_scale, const void* __restrict__ q_idx,
                const uint8_t* __restrict__ q_sf, const void* __restrict__ k_idx,
                const uint8_t* __restrict__ k_sf, const void* __restrict__ w,
                float* __restrict__ scores) {
  extern __shared__ float smem[];
  float* qs = smem;             // [HI * DI]
  float* ws = smem + HI * DI;   // [HI]
  const int64_t row = blockIdx.y;  // b * T + t
  const int b = static_cast<int>(row / T);
  const int t = static_cast<int>(row % T);
  const int q_pos = S - T + t;
  const int nblk = DI / 128;
  for (int i = threadIdx.x; i < HI * DI; i += blockDim.x) {
    float v = load_idx<IDT>(q_idx, row * HI * DI + i);
    if constexpr (IDT == DSA_FP8_E4M3)
      v *= ue8m0_to_f32(q_sf[(row * HI + i / DI) * nblk + (i % DI) / 128]);
    qs[i] = v;
  }
  for (int h = threadIdx.x; h < HI; h += blockDim.x) ws[h] = load_w<WDT>(w, row * HI + h);
  __syncthreads();
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  float out;
  if (s > q_pos) {
    out = -__builtin_inff();
  } else {
    const int64_t krow = static_cast<int64_t>(b) * S + s;
    float acc = 0.f;
    for (int h = 0; h < HI; ++h) {
      float dot = 0.f;
      for (int d = 0; d < DI; ++d) {
        float kv = load_idx<IDT>(k_idx, krow * DI + d);
        if constexpr (IDT == DSA_FP8_E4M3) kv *= ue8m0_to_f32(k_sf[krow * nblk + d / 128]);
        dot = fmaf(qs[h * DI + d], kv, dot);
      }
      acc = fmaf(ws[h], fmaxf(dot, 0.f), acc);
    }
    out = idx_scale * acc;
  }
  scores[row * S + s] = out;
}

// ---------------------------------------------------------------------------
// MFMA kernel, HI = 64, DI = 128.
//
// MFMA 16x16x32 operand layouts (lane l, g = l / 16, n = l % 16):
//   A (16 x 32): lane holds row n, reduction elements 8g .. 8g+7
//   B (32 x 16): lane holds column n, reduction elements 8g .. 8g+7
//   C (16 x 16): lane holds rows 4g .. 4g+3 of column n
// Rows are heads (4 blocks of 16), columns are keys.  The 128-wide reduction
// is split in 4 steps; the dims of step ks in lane group g are chosen so that
// a lane's 4 steps cover one contiguous run of the key row: bf16 uses dims
// 32*ks + 8*g + e (each step is one 16-byte load per lane, a 64-byte run per
// key), fp8 uses dims 32*g + 8*ks + e (each lane loads 32 contiguous bytes).
// ---------------------------------------------------------------------------
constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kIdxWaves = 4;
constexpr int kKeysPerWave = 128;   // 8 tiles of 16 keys
constexpr int kTilesPerGroup = 4;    // tiles whose loads are issued together
constexpr int kQStrideBf16 = kIdxDim + 8;   // padded LDS row (elements)
constexpr int kQStrideFp8 = kIdxDim + 16;   // padded LDS row (bytes)

template <bool FP8, int WDT>
__global__ void __launch_bounds__(kIdxWaves * 64)
indexer_mfma(int T, int S, float idx_scale, const void* __restrict__ q_idx,
             const uint8_t* __restrict__ q_sf, const void* __restrict__ k_idx,
             const uint8_t* __restrict__ k_sf, const void* __restrict__ w,
             float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kIdxHeads * kQStrideBf16 * 2];
  __shared__ float w_lds[kIdxHeads];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int64_t row = blockIdx.y;  // b * T + t
  const int b = static_cast<int>(row / T);
  const int t = static_cast<int>(row % T);
  const int q_pos = S - T + t;
  const int s_lim = min(S, q_pos + 1);  // keys [0, s_lim) are visible

  const int s_begin = (blockIdx.x * kIdxWaves + wave) * kKeysPerWave;
  const int s_end = min(S, s_begin + kKeysPerWave);
  const bool active = s_begin < S && s_begin < s_lim;  // this wave has visible keys
  const int64_t kbase = static_cast<int64_t>(b) * S;
  // Key rows of a group of kTilesPerGroup 16-key tiles (keys past the visible
  // range load row s_lim - 1, so every address stays in bounds).
  auto load_group = [&](int s0, u32x4_t (&kb)[kTilesPerGroup][4], float (&ksc)[kTilesPerGroup]) {
#pragma unroll
    for (int j = 0; j < kTilesPerGroup; ++j) {
      const int s = min(s0 + 16 * j + n, s_lim - 1);
      if constexpr (!FP8) {
        const u32x4_t* kr = reinterpret_cast<const u32x4_t*>(
            static_cast<const uint16_t*>(k_idx) + (kbase + s) * kIdxDim);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[j][ks] = __builtin_nontemporal_load(kr + 4 * ks + g);
      } else {
        const u32x4_t* kr = reinterpret_cast<const u32x4_t*>(
            static_cast<const uint8_t*>(k_idx) + (kbase + s) * kIdxDim);
        kb[j][0] = __builtin_nontemporal_load(kr + 2 * g);
        kb[j][1] = __builtin_nontemporal_load(kr + 2 * g + 1);
        ksc[j] = ue8m0_to_f32(k_sf[kbase + s]);
      }
    }
  };
  // the first key group goes out before the query is staged: both latencies overlap
  u32x4_t kb0[kTilesPerGroup][4], kb1[kTilesPerGroup][4];
  float ksc0[kTilesPerGroup] = {}, ksc1[kTilesPerGroup] = {};
  if (active) load_group(s_begin, kb0, ksc0);

  // ---- stage the query row (and w, times the query scales for fp8) ----
  if constexpr (!FP8) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint16_t*>(q_idx) + row * kIdxHeads * kIdxDim);
    for (int i = threadIdx.x; i < kIdxHeads * kIdxDim / 8; i += blockDim.x) {
      const int h = i / (kIdxDim / 8), c = i % (kIdxDim / 8);
      *reinterpret_cast<u32x4_t*>(q_lds + (h * kQStrideBf16 + c * 8) * 2) = src[i];
    }
  } else {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint8_t*>(q_idx) + row * kIdxHeads * kIdxDim);
    for (int i = threadIdx.x; i < kIdxHeads * kIdxDim / 16; i += blockDim.x) {
      const int h = i / (kIdxDim / 16), c = i % (kIdxDim / 16);
      *reinterpret_cast<u32x4_t*>(q_lds + h * kQStrideFp8 + c * 16) = src[i];
    }
  }
  for (int h = threadIdx.x; h < kIdxHeads; h += blockDim.x) {
    float wv = load_w<WDT>(w, row * kIdxHeads + h);
    if constexpr (FP8) wv *= ue8m0_to_f32(q_sf[row * kIdxHeads + h]);
    w_lds[h] = wv;
  }
  __syncthreads();

  if (s_begin >= S) return;
  float* out_row = scores + row * S;

  if (s_begin >= s_lim) {  // every key of this wave is in the future
    for (int s = s_begin + lane; s < s_end; s += 64) out_row[s] = -__builtin_inff();
    return;
  }

  // ---- query operand (A) and head weights in registers ----
  bf16x8_t qa[4][4];
  long qa8[4][4];
  float wreg[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int h = mb * 16 + n;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if constexpr (!FP8)
        qa[mb][ks] = *reinterpret_cast<const bf16x8_t*>(q_lds + (h * kQStrideBf16 + 32 * ks + 8 * g) * 2);
      else
        qa8[mb][ks] = *reinterpret_cast<const long*>(q_lds + h * kQStrideFp8 + 32 * g + 8 * ks);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wreg[mb][i] = w_lds[mb * 16 + 4 * g + i];
  }

  auto score_group = [&](int s0, const u32x4_t (&kb)[kTilesPerGroup][4],
                         const float (&ksc)[kTilesPerGroup]) {
#pragma unroll
    for (int j = 0; j < kTilesPerGroup; ++j) {
      f32x4_t acc[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if constexpr (!FP8) {
            acc[mb] = mfma16x16x32_bf16(qa[mb][ks], __builtin_bit_cast(bf16x8_t, kb[j][ks]), acc[mb]);
          } else {
            // 32 contiguous bytes per lane: step ks takes bytes 8ks .. 8ks+7
            const u32x4_t half = kb[j][ks >> 1];
            const long kv = (ks & 1) ? (static_cast<long>(half[3]) << 32 | half[2])
                                     : (static_cast<long>(half[1]) << 32 | half[0]);
            acc[mb] = mfma16x16x32_fp8(qa8[mb][ks], kv, acc[mb]);
          }
        }
      }
      float part = 0.f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wreg[mb][i], fmaxf(acc[mb][i], 0.f), part);
      part = xor16_sum(part);
      part = xor32_sum(part);
      const int s = s0 + 16 * j + n;
      if (g == 0 && s < s_end) {
        float v;
        if constexpr (FP8) v = idx_scale * (part * ksc[j]);
        else v = idx_scale * part;
        out_row[s] = (s < s_lim) ? v : -__builtin_inff();
      }
    }
  };

  // two-stage pipeline: the next group's key rows load while this group scores
  constexpr int kGroupKeys = 16 * kTilesPerGroup;
#pragma unroll
  for (int grp = 0; grp < kKeysPerWave / kGroupKeys; grp += 2) {
    const int s0 = s_begin + grp * kGroupKeys;
    const int s1 = s0 + kGroupKeys;
    if (s1 < s_end) load_group(s1, kb1, ksc1);
    if (s0 < s_end) score_group(s0, kb0, ksc0);
    if (s1 + kGroupKeys < s_end) load_group(s1 + kGroupKeys, kb0, ksc0);
    if (s1 < s_end) score_group(s1, kb1, ksc1);
  }
}

template <int IDT, int WDT>
dsa_status_t run_generic(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                         const void* k_idx, const uint8_t* k_sf, const void* w, float* scores,
                         hipStream_t stream) {
  const size_t lds = (static_cast<size_t>(s.HI) * s.DI + s.HI) * sizeof(float);
  if (lds > 64 * 1024)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: HI*DI = %d too large for the generic kernel",
                s.HI * s.DI);
  dim3 grid((s.S + 255) / 256, s.B * s.T);
  LaunchTimer timer;
  hipExtLaunchKernelGGL(indexer_generic<IDT, WDT>, grid, dim3(256), lds, stream, timer.start(),
                        timer.stop(), 0, s.T, s.S, s.HI, s.DI, s.idx_scale, q_idx, q_sf, k_idx,
                        k_sf, w, scores);
  return timer.done("indexer_generic");
}

template <bool FP8, int WDT>
dsa_status_t run_mfma(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                      const void* k_idx, const uint8_t* k_sf, const void* w, float* scores,
                      hipStream_t stream) {
  const int keys_per_block = kIdxWaves * kKeysPerWave;
  dim3 grid((s.S + keys_per_block - 1) / keys_per_block, s.B * s.T);
  LaunchTimer timer;
  hipExtLaunchKernelGGL(indexer_mfma<FP8, WDT>, grid, dim3(kIdxWaves * 64), 0, stream,
                        timer.start(), timer.stop(), 0, s.T, s.S, s.idx_scale, q_idx, q_sf, k_idx,
                        k_sf, w, scores);
  return timer.done("indexer_mfma");
}

}  // namespace

dsa_status_t launch_indexer(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                            const void* k_idx, const uint8_t* k_sf, const void* w,
                            float* scores, hipStream_t stream) {
  if (static_cast<int64_t>(s.B) * s.T > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: B*T = %lld exceeds 65535 query rows",
                static_cast<long long>(s.B) * s.T);
  const bool v32 = s.HI == kIdxHeads && s.DI == kIdxDim;
  const bool wbf = s.w_dtype == DSA_BF16;
  if (v32 && s.idx_dtype == DSA_BF16)
    return wbf ? run_mfma<false, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream)
               : run_mfma<false, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream);
  if (v32 && s.idx_dtype == DSA_FP8_E4M3)
    return wbf ? run_mfma<true, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream)
               : run_mfma<true, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream);
  switch (s.idx_dtype) {
    case DSA_F32:
      return wbf ? run_generic<DSA_F32, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream)
                 : run_generic<DSA_F32, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream);
    case DSA_BF16:
      return wbf ? run_generic<DSA_BF16, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream)
                 : run_generic<DSA_BF16, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream);
    case DSA_FP8_E4M3:
      return wbf ? run_generic<DSA_FP8_E4M3, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream)
                 : run_generic<DSA_FP8_E4M3, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, scores, stream);
  }
  return fail(DSA_ERR_UNSUPPORTED, "indexer: unknown idx_dtype %d", s.idx_dtype);
}

}  // namespace dsa
