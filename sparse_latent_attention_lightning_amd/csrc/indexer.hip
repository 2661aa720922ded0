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

// ---------------------------------------------------------------------------
// Query-blocked MFMA kernel for many queries per sequence (prefill), bf16,
// HI = 64, DI = 128.
//
// The index scores of a prefill chunk are a dense contraction: [T queries x
// 64 heads] x [128 dims] x [S keys], with the ReLU-weighted head sum applied
// to every 64-head column.  Streaming the key rows once per query (as the
// decode kernel does) would make the kernel bound by key traffic, so here a
// block of 8 waves takes 8 consecutive queries of one sequence, one per wave,
// and streams every key the 8 of them see through LDS once:
//  * keys move in 64-key chunks (16 KB) through a ring of 4 LDS buffers,
//    copied global -> LDS by the DMA path, two 1 KB copies per wave per chunk;
//    a key row is 256 bytes = 16 pieces of 16 bytes, and piece c of row r sits
//    in slot c ^ ((r & 7) << 1) of the row, so that the operand reads (lane
//    (g, n): row n, piece 4 ks + g) touch all 64 banks in every cycle;
//  * each wave keeps its query's 64 x 128 Q^I tile as MFMA A operands (64
//    VGPRs) and its 64 head weights for the block's whole key range;
//  * per 16-key tile: 16 MFMAs (4 head blocks x 4 reduction steps), then ReLU,
//    weight and the in-lane part of the head sum on the accumulators (each
//    lane holds 16 heads of one key); the MFMAs of tile u + 1 are issued
//    before the VALU work of tile u, so the two overlap;
//  * the cross-lane part of the head sum of a chunk's 4 tiles is one
//    reduce-scatter (3 lane swaps, 3 adds) that leaves the 64 scores of the
//    chunk one per lane, stored as one 256-byte run.
// Blocks run longest first (the causal key range grows with the query index),
// which balances the triangular work over the CUs.
// ---------------------------------------------------------------------------
constexpr int kPfWaves = 8;                                  // queries per block
constexpr int kPfChunkKeys = 64;
constexpr int kPfRowBytes = kIdxDim * 2;                     // 256
constexpr int kPfChunkBytes = kPfChunkKeys * kPfRowBytes;    // 16 KB
constexpr int kPfBuffers = 4;
constexpr int kPfMinQueries = 8;   // fewer queries per sequence use the per-query kernel
static_assert(kPfChunkBytes == kPfWaves * 2 * 1024, "two 1 KB copies per wave per chunk");

template <int WDT>
__global__ void __launch_bounds__(kPfWaves * 64)
indexer_prefill(int T, int S, int n_qblk, float idx_scale, const uint16_t* __restrict__ q_idx,
                const uint16_t* __restrict__ k_idx, const void* __restrict__ w,
                float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kPfBuffers * kPfChunkBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int nb = gridDim.x / n_qblk;                 // sequences
  const int qb = n_qblk - 1 - static_cast<int>(blockIdx.x) / nb;   // longest first
  const int b = static_cast<int>(blockIdx.x) % nb;
  const int t0 = qb * kPfWaves;
  const int t = t0 + wave;
  const bool has_q = t < T;
  const int tq = min(t, T - 1);
  const int q_pos = S - T + tq;
  const int kend = S - T + min(t0 + kPfWaves, T);    // keys [0, kend) are visible to some query
  const int nchunks = (kend + kPfChunkKeys - 1) / kPfChunkKeys;
  const int64_t kbase = static_cast<int64_t>(b) * S;
  const uint32_t kb_lds = lds_addr(kbuf);

  // chunk c -> buffer c % kPfBuffers; this wave copies rows 8 wave .. 8 wave + 7
  // (keys past S - 1 load row S - 1: every address stays in bounds)
  auto issue_chunk = [&](int c) {
    const uint32_t dst = kb_lds + (c % kPfBuffers) * kPfChunkBytes + wave * 2048;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wave * 8 + i * 4 + (lane >> 4);
      const int piece = (lane & 15) ^ ((r & 7) << 1);
      const int key = min(c * kPfChunkKeys + r, S - 1);
      lds_dma_16(k_idx + (kbase + key) * kIdxDim + piece * 8, dst + i * 1024);
    }
  };
#pragma unroll
  for (int c = 0; c < kPfBuffers - 1; ++c)
    if (c < nchunks) issue_chunk(c);

  // ---- the query tile (A operands) and head weights, in registers ----
  const int64_t row = static_cast<int64_t>(b) * T + tq;
  const bf16x8_t* qrow = reinterpret_cast<const bf16x8_t*>(q_idx + row * kIdxHeads * kIdxDim);
  bf16x8_t qa[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[mb][ks] = __builtin_nontemporal_load(qrow + (16 * mb + n) * (kIdxDim / 8) + 4 * ks + g);
  float wreg[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) wreg[mb][i] = load_w<WDT>(w, row * kIdxHeads + 16 * mb + 4 * g + i);

  float* out_row = scores + row * S;

  // one 16-key tile: 16 MFMAs into acc (key operands read from LDS)
  auto tile_mfma = [&](const uint8_t* buf, int u, f32x4_t (&acc)[4]) {
    bf16x8_t kb[4];
    const uint8_t* rp = buf + (16 * u + n) * kPfRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kb[ks] = *reinterpret_cast<const bf16x8_t*>(rp + 16 * ((4 * ks + g) ^ ((n & 7) << 1)));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x16x32_bf16(qa[mb][ks], kb[ks], acc[mb]);
  };
  // ReLU, head weights and the in-lane part of the head sum
  auto tile_part = [&](const f32x4_t (&acc)[4]) -> float {
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      p0 = fmaf(wreg[mb][0], fmaxf(acc[mb][0], 0.f), p0);
      p1 = fmaf(wreg[mb][1], fmaxf(acc[mb][1], 0.f), p1);
      p0 = fmaf(wreg[mb][2], fmaxf(acc[mb][2], 0.f), p0);
      p1 = fmaf(wreg[mb][3], fmaxf(acc[mb][3], 0.f), p1);
    }
    return p0 + p1;
  };
  // cross-lane part of the head sum for the 4 tiles of chunk c: afterwards
  // lane l holds the full sum of part[l / 16] for key n, i.e. key 64 c + l
  auto chunk_store = [&](int c, const float (&part)[4]) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
    const auto d = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
    const float h0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float h1 = __uint_as_float(d[0]) + __uint_as_float(d[1]);
    const auto e = __builtin_amdgcn_permlane16_swap(__float_as_uint(h0), __float_as_uint(h1), false, false);
    const float v = idx_scale * (__uint_as_float(e[0]) + __uint_as_float(e[1]));
    const int key = c * kPfChunkKeys + lane;
    if (has_q && key < S) __builtin_nontemporal_store(key <= q_pos ? v : -__builtin_inff(), out_row + key);
  };

  f32x4_t acc0[4], acc1[4];
  float part[4];
  for (int c = 0; c < nchunks; ++c) {
    // chunk c has landed: the copies issued after it are those of chunks
    // c + 1 .. min(c + kPfBuffers - 2, nchunks - 1), two per chunk (the first
    // chunk also waits for the query loads, issued after the copies)
    const int later = min(kPfBuffers - 2, nchunks - 1 - c);
    if (c == 0 || later <= 0)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    __syncthreads();   // every wave's copies of chunk c are in; chunk c - 1 is consumed
    if (c + kPfBuffers - 1 < nchunks) issue_chunk(c + kPfBuffers - 1);
    const uint8_t* buf = kbuf + (c % kPfBuffers) * kPfChunkBytes;
    tile_mfma(buf, 0, acc0);
    if (c > 0) {
      part[3] = tile_part(acc1);
      chunk_store(c - 1, part);
    }
    tile_mfma(buf, 1, acc1);
    part[0] = tile_part(acc0);
    tile_mfma(buf, 2, acc0);
    part[1] = tile_part(acc1);
    tile_mfma(buf, 3, acc1);
    part[2] = tile_part(acc0);
  }
  if (nchunks > 0) {
    part[3] = tile_part(acc1);
    chunk_store(nchunks - 1, part);
  }
  // keys past the block's last chunk are in every query's future
  if (has_q) {
    const int k0 = nchunks * kPfChunkKeys;
    if ((S & 3) == 0) {
      const f32x4_t ninf = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
      for (int k = k0 + 4 * lane; k < S; k += 256)
        __builtin_nontemporal_store(ninf, reinterpret_cast<f32x4_t*>(out_row + k));
    } else {
      for (int k = k0 + lane; k < S; k += 64) __builtin_nontemporal_store(-__builtin_inff(), out_row + k);
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming MFMA kernel for few queries per sequence (decode), bf16, HI = 64,
// DI = 128.
//
// Decode reads every key row of the sequence once per query: the kernel is a
// stream of k^I from HBM.  Each wave owns 256 consecutive keys and moves them
// through a private ring of four 8 KB LDS buffers with whole-line direct
// copies (global_load_lds_dwordx4: 1 KB of contiguous key rows per
// instruction), three 32-key chunks in flight while one is scored; per-lane
// operand loads, whose 16 lanes per key row touch 64-byte pieces, stream
// slower.  No barrier is needed after the query is staged (each wave reads
// only what it copied).  The operands are read as in the prefill kernel (row
// r's piece c in slot c ^ ((r & 7) << 1)), and every two chunks (4 tiles)
// finish with the same reduce-scatter, so each wave keeps its 256 scores in 4
// registers and stores them at the end, after its last load.
// ---------------------------------------------------------------------------
constexpr int kStWaves = 4;
constexpr int kStChunkKeys = 32;                              // keys per chunk
constexpr int kStChunkBytes = kStChunkKeys * kIdxDim * 2;     // 8 KB
constexpr int kStBuffers = 4;                                 // per wave
constexpr int kStChunks = 8;                                  // chunks per wave
constexpr int kStKeysPerBlock = kStWaves * kStChunks * kStChunkKeys;  // 1024
constexpr int kStCopies = kStChunkBytes / 1024;               // 8 copies per chunk

template <int WDT>
__global__ void __launch_bounds__(kStWaves * 64)
indexer_stream(int T, int S, int nkb, float idx_scale, const uint16_t* __restrict__ q_idx,
               const uint16_t* __restrict__ k_idx, const void* __restrict__ w,
               float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kStWaves * kStBuffers * kStChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kIdxHeads * kQStrideBf16 * 2];
  __shared__ float w_lds[kIdxHeads];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int64_t row = blockIdx.x / nkb;  // b * T + t
  const int kb = static_cast<int>(blockIdx.x % nkb);
  const int b = static_cast<int>(row / T);
  const int t = static_cast<int>(row % T);
  const int s_lim = min(S, S - T + t + 1);  // keys [0, s_lim) are visible
  const int s_begin = (kb * kStWaves + wave) * (kStChunks * kStChunkKeys);
  const int s_end = min(S, s_begin + kStChunks * kStChunkKeys);
  const int s_vis = min(s_end, s_lim);  // this wave scores [s_begin, s_vis)
  const int nch = s_vis > s_begin ? (s_vis - s_begin + kStChunkKeys - 1) / kStChunkKeys : 0;
  const int64_t kbase = static_cast<int64_t>(b) * S;
  const uint32_t wlds = lds_addr(kbuf) + wave * kStBuffers * kStChunkBytes;

  // chunk c -> buffer c % 4; copy i covers chunk rows 4i .. 4i+3 (keys past
  // the visible range load row s_vis - 1: every address stays in bounds)
  auto issue_chunk = [&](int c) {
    const uint32_t dst = wlds + (c % kStBuffers) * kStChunkBytes;
#pragma unroll
    for (int i = 0; i < kStCopies; ++i) {
      const int r = 4 * i + (lane >> 4);
      const int piece = (lane & 15) ^ ((r & 7) << 1);
      const int key = min(s_begin + c * kStChunkKeys + r, s_vis - 1);
      lds_dma_16_nt(k_idx + (kbase + key) * kIdxDim + piece * 8, dst + 1024 * i);
    }
  };
#pragma unroll
  for (int c = 0; c < kStBuffers - 1; ++c)
    if (c < nch) issue_chunk(c);

  // ---- stage the query row and the head weights ----
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(q_idx + row * kIdxHeads * kIdxDim);
    for (int i = threadIdx.x; i < kIdxHeads * kIdxDim / 8; i += blockDim.x) {
      const int h = i / (kIdxDim / 8), c = i % (kIdxDim / 8);
      *reinterpret_cast<u32x4_t*>(q_lds + (h * kQStrideBf16 + c * 8) * 2) = src[i];
    }
    for (int h = threadIdx.x; h < kIdxHeads; h += blockDim.x) w_lds[h] = load_w<WDT>(w, row * kIdxHeads + h);
  }
  __syncthreads();

  float* out_row = scores + row * S;
  if (nch == 0) {  // every key of this wave is in the future (or past S)
    for (int s = s_begin + lane; s < s_end; s += 64) out_row[s] = -__builtin_inff();
    return;
  }
  bf16x8_t qa[4][4];
  float wreg[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int h = mb * 16 + n;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[mb][ks] = *reinterpret_cast<const bf16x8_t*>(q_lds + (h * kQStrideBf16 + 32 * ks + 8 * g) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) wreg[mb][i] = w_lds[mb * 16 + 4 * g + i];
  }

  float res[kStChunks / 2];  // chunks 2j, 2j+1: 64 scores, key s_begin + 64 j + lane
  float part[4];
#pragma unroll
  for (int c = 0; c < kStChunks; ++c) {
    if (c < nch) {  // wave-uniform
      // chunk c has landed; chunks up to c + 3 go out behind it
      const int ahead = min(kStBuffers - 2, nch - 1 - c);  // copies issued after chunk c
      if (ahead >= 2)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else if (ahead == 1)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (c + kStBuffers - 1 < nch) issue_chunk(c + kStBuffers - 1);
      const uint8_t* buf = kbuf + (wave * kStBuffers + (c % kStBuffers)) * kStChunkBytes;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t kv[4];
        const uint8_t* rp = buf + (16 * u + n) * (kIdxDim * 2);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kv[ks] = *reinterpret_cast<const bf16x8_t*>(rp + 16 * ((4 * ks + g) ^ ((n & 7) << 1)));
        f32x4_t acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x16x32_bf16(qa[mb][ks], kv[ks], acc[mb]);
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          p0 = fmaf(wreg[mb][0], fmaxf(acc[mb][0], 0.f), p0);
          p1 = fmaf(wreg[mb][1], fmaxf(acc[mb][1], 0.f), p1);
          p0 = fmaf(wreg[mb][2], fmaxf(acc[mb][2], 0.f), p0);
          p1 = fmaf(wreg[mb][3], fmaxf(acc[mb][3], 0.f), p1);
        }
        part[2 * (c & 1) + u] = p0 + p1;
      }
    } else {
      part[2 * (c & 1)] = 0.f;
      part[2 * (c & 1) + 1] = 0.f;
    }
    if (c & 1) {  // cross-lane head sum of 4 tiles: lane l ends with key 64 (c / 2) + l
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float h0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
      const float h1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(h0), __float_as_uint(h1), false, false);
      res[c >> 1] = idx_scale * (__uint_as_float(z[0]) + __uint_as_float(z[1]));
    }
  }
  // ---- the wave's scores: one 256-byte run per two chunks; future keys -inf ----
#pragma unroll
  for (int j = 0; j < kStChunks / 2; ++j) {
    const int s = s_begin + 64 * j + lane;
    if (s < s_end) __builtin_nontemporal_store(s < s_lim ? res[j] : -__builtin_inff(), out_row + s);
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

template <int WDT>
dsa_status_t run_stream(const dsa_shape_t& s, const void* q_idx, const void* k_idx, const void* w,
                        float* scores, hipStream_t stream) {
  const int nkb = (s.S + kStKeysPerBlock - 1) / kStKeysPerBlock;
  const int64_t blocks = static_cast<int64_t>(s.B) * s.T * nkb;
  if (blocks > 0x7fffffff)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: %lld key blocks", static_cast<long long>(blocks));
  LaunchTimer timer;
  hipExtLaunchKernelGGL(indexer_stream<WDT>, dim3(static_cast<unsigned>(blocks)), dim3(kStWaves * 64),
                        0, stream, timer.start(), timer.stop(), 0, s.T, s.S, nkb, s.idx_scale,
                        static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), w,
                        scores);
  return timer.done("indexer_stream");
}

template <int WDT>
dsa_status_t run_prefill(const dsa_shape_t& s, const void* q_idx, const void* k_idx,
                         const void* w, float* scores, hipStream_t stream) {
  const int n_qblk = (s.T + kPfWaves - 1) / kPfWaves;
  const int64_t blocks = static_cast<int64_t>(n_qblk) * s.B;
  if (blocks > 0x7fffffff)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: %lld query blocks", static_cast<long long>(blocks));
  LaunchTimer timer;
  hipExtLaunchKernelGGL(indexer_prefill<WDT>, dim3(static_cast<unsigned>(blocks)),
                        dim3(kPfWaves * 64), 0, stream, timer.start(), timer.stop(), 0, s.T, s.S,
                        n_qblk, s.idx_scale, static_cast<const uint16_t*>(q_idx),
                        static_cast<const uint16_t*>(k_idx), w, scores);
  return timer.done("indexer_prefill");
}

}  // namespace

dsa_status_t launch_indexer(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                            const void* k_idx, const uint8_t* k_sf, const void* w,
                            float* scores, hipStream_t stream) {
  const bool v32 = s.HI == kIdxHeads && s.DI == kIdxDim;
  const bool wbf = s.w_dtype == DSA_BF16;
  if (v32 && s.idx_dtype == DSA_BF16 && s.T >= kPfMinQueries)
    return wbf ? run_prefill<DSA_BF16>(s, q_idx, k_idx, w, scores, stream)
               : run_prefill<DSA_F32>(s, q_idx, k_idx, w, scores, stream);
  if (v32 && s.idx_dtype == DSA_BF16)
    return wbf ? run_stream<DSA_BF16>(s, q_idx, k_idx, w, scores, stream)
               : run_stream<DSA_F32>(s, q_idx, k_idx, w, scores, stream);
  // the per-query kernels put the query row on grid.y
  if (static_cast<int64_t>(s.B) * s.T > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: B*T = %lld exceeds 65535 query rows",
                static_cast<long long>(s.B) * s.T);
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
