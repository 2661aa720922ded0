// Lightning-indexer scores on gfx950.
//
// S[b,t,s] = idx_scale * sum_h w[b,t,h] * ReLU(q_idx[b,t,h,:] . k_idx[b,s,:])
// for s <= q_pos(t) = S - T + t, and -inf for later keys (atlas.klimoza.dev,
// DeepSeek-V3.2-Exp MoE block, "All 43 steps": the index score S^I and the
// causal mask M added to it).  The head sum accumulates in fp32 and the
// prefactor multiplies it once, after the sum.
//
// Three kernels:
//  * indexer_stream (few queries per sequence, 64 heads x 128 dims, bf16 or
//    e4m3): each wave streams a run of key rows through its own LDS ring with
//    whole-line direct copies and scores them on MFMAs against the query tile
//    it keeps in registers.
//  * indexer_prefill (8 or more queries per sequence, bf16): 4 queries per
//    workgroup share every key chunk through LDS.
//  * indexer_generic: any HI x DI, f32 / bf16 / e4m3, plain fp32 VALU loops.
// ReLU, the head weights and the head sum run on the MFMA accumulator
// registers: each lane holds 16 heads of one key and sums them, and lane
// swaps finish the 64-head reduction.
#include "dsa_device.h"
#include "dsa_internal.h"
#include "select_row.h"

namespace dsa {
namespace {

template <int WDT>
__device__ __forceinline__ float load_w(const void* w, int64_t i) {
  if constexpr (WDT == DSA_BF16)
    return bf16_to_f32(static_cast<const uint16_t*>(w)[i]);
  else
    return static_cast<const float*>(w)[i];
}

// Keys of sequence b: all S, or its own context length in a ragged batch
// (clamped to [0, S]); its T queries are its last T positions.
__device__ __forceinline__ int seq_len(const int32_t* seq_lens, int b, int S) {
  return seq_lens == nullptr ? S : min(max(seq_lens[b], 0), S);
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
                const int32_t* __restrict__ seq_lens, float* __restrict__ scores) {
  extern __shared__ float smem[];
  float* qs = smem;             // [HI * DI]
  float* ws = smem + HI * DI;   // [HI]
  const int64_t row = blockIdx.y;  // b * T + t
  const int b = static_cast<int>(row / T);
  const int t = static_cast<int>(row % T);
  const int q_pos = seq_len(seq_lens, b, S) - T + t;
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
// MFMA kernels, HI = 64, DI = 128.
//
// MFMA 16x16x32 operand layouts (lane l, g = l / 16, n = l % 16):
//   A (16 x 32): lane holds row n, reduction elements 8g .. 8g+7
//   B (32 x 16): lane holds column n, reduction elements 8g .. 8g+7
//   C (16 x 16): lane holds rows 4g .. 4g+3 of column n
// Rows are heads (4 blocks of 16), columns are keys.  The 128-wide reduction
// is split in 4 steps; the dims of step ks in lane group g are chosen so that
// a lane's 4 steps cover one contiguous run of the key row: bf16 uses dims
// 32*ks + 8*g + e (each step one 16-byte read per lane, a 64-byte run per
// key), fp8 uses dims 32*g + 8*ks + e (32 contiguous bytes per lane).
// ---------------------------------------------------------------------------
constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;

// ---------------------------------------------------------------------------
// Query-blocked MFMA kernel for many queries per sequence (prefill), bf16,
// HI = 64, DI = 128.
//
// The index scores of a prefill chunk are a dense contraction: [T queries x
// 64 heads] x [128 dims] x [S keys], with the ReLU-weighted head sum applied
// to every 64-head column.  Streaming the key rows once per query (as the
// decode kernel does) would make the kernel bound by key traffic, so here a
// block of 8 waves (two per SIMD, one block per CU) takes 8 consecutive
// queries of one sequence, one per wave, and streams every key the 8 of them
// see through LDS once:
//  * keys move in 64-key chunks (16 KB) through a ring of 8 LDS buffers (six
//    chunks in flight while one is scored), copied global -> LDS by the DMA
//    path, two 1 KB copies per wave per chunk;
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
constexpr int kPfWaves = 4;                                  // e4m3: queries per block
constexpr int kPfChunkKeys = 64;
constexpr int kPfRowBytes = kIdxDim * 2;                     // 256
constexpr int kPfChunkBytes = kPfChunkKeys * kPfRowBytes;    // 16 KB
constexpr int kPfBuffers = 4;                                // e4m3: chunks in the LDS ring
constexpr int kPfMinQueries = 8;   // fewer queries per sequence use the per-query kernel
constexpr int kPfQueries = 8;      // bf16: queries (waves) per block, one block per CU
constexpr int kPfRing = 8;         // bf16: chunks in the LDS ring (128 KB)
constexpr int kPfCopies = kPfChunkBytes / 1024 / kPfQueries;  // 1 KB copies per wave per chunk
static_assert(kPfCopies * kPfQueries * 1024 == kPfChunkBytes, "whole copies per wave");

template <int WDT>
__global__ void __launch_bounds__(kPfQueries * 64)
indexer_prefill(int T, int S, int n_qblk, float idx_scale, const uint16_t* __restrict__ q_idx,
                const uint16_t* __restrict__ k_idx, const void* __restrict__ w,
                const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                int full_rows) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kPfRing * kPfChunkBytes];
  debug_poison_lds<sizeof(kbuf)>(kbuf);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int nb = gridDim.x / n_qblk;                 // sequences
  const int qb = n_qblk - 1 - static_cast<int>(blockIdx.x) / nb;   // longest first
  const int b = static_cast<int>(blockIdx.x) % nb;
  const int t0 = qb * kPfQueries;
  const int t = t0 + wave;
  const bool has_q = t < T;
  const int tq = min(t, T - 1);
  const int L = seq_len(seq_lens, b, S);
  const int q_pos = L - T + tq;
  const int kend = max(0, L - T + min(t0 + kPfQueries, T));  // keys [0, kend) are visible to some query
  const int nchunks = (kend + kPfChunkKeys - 1) / kPfChunkKeys;
  const int64_t kbase = static_cast<int64_t>(b) * S;
  const uint32_t kb_lds = lds_addr(kbuf);

  // chunk c -> buffer c % kPfRing; this wave copies chunk rows
  // 4 kPfCopies wave .. 4 kPfCopies (wave + 1) - 1
  // (keys past S - 1 load row S - 1: every address stays in bounds)
  auto issue_chunk = [&](int c) {
    const uint32_t dst = kb_lds + (c % kPfRing) * kPfChunkBytes + wave * kPfCopies * 1024;
#pragma unroll
    for (int i = 0; i < kPfCopies; ++i) {
      const int r = (wave * kPfCopies + i) * 4 + (lane >> 4);
      const int piece = (lane & 15) ^ ((r & 7) << 1);
      const int key = min(c * kPfChunkKeys + r, S - 1);
      lds_dma_16(k_idx + (kbase + key) * kIdxDim + piece * 8, dst + i * 1024);
    }
  };
#pragma unroll
  for (int c = 0; c < kPfRing - 1; ++c)
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
    // c + 1 .. min(c + kPfRing - 2, nchunks - 1), two per chunk (the first
    // chunk also waits for the query loads, issued after the copies)
    const int later = c == 0 ? 0 : max(0, min(kPfRing - 2, nchunks - 1 - c));
    switch (later) {
      case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPfCopies) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPfCopies) : "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kPfCopies) : "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kPfCopies) : "memory"); break;
      case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * kPfCopies) : "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * kPfCopies) : "memory"); break;
    }
    __syncthreads();   // every wave's copies of chunk c are in; chunk c - 1 is consumed
    if (c + kPfRing - 1 < nchunks) issue_chunk(c + kPfRing - 1);
    const uint8_t* buf = kbuf + (c % kPfRing) * kPfChunkBytes;
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
  if (has_q && full_rows) {
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
// Query-blocked e4m3 kernel for many queries per sequence (prefill): the
// design of indexer_prefill on gfx950's 16x16x128 f8f6f4 product.
//  * keys move in 128-key chunks (128 bytes per key: 16 KB) through a ring of
//    4 LDS buffers, four 1 KB copies per wave per chunk; piece c of row r in
//    slot c ^ ((r >> 1) & 7), lane (g, n) reads pieces 2g and 2g + 1 of row n
//    (its 32 bytes of the key for the one product per 16 keys and head
//    block), every bank once per cycle;
//  * the chunk's 128 ue8m0 key scales follow it into the buffer (each wave
//    copies 32 of them as 4-byte pieces, so every wave counts the same
//    copies);
//  * each wave keeps its query's 64 x 128 codes as four A operands (32
//    VGPRs) and its head weights times the query scales of the heads;
//  * per 16-key tile: 4 products (one per head block), then ReLU, weight and
//    the in-lane head sum; the products of tile u + 1 are issued before the
//    VALU work of tile u;
//  * per 64 keys one reduce-scatter leaves one key's sum per lane, which is
//    multiplied by that key's scale (a power of two: it commutes exactly
//    with the ReLU and the head sum) and by the prefactor.
// The key scale bytes are copied as 4-byte pieces, so the launcher sends only
// sequence lengths that are multiples of 4 here (others: indexer_stream).
// ---------------------------------------------------------------------------
constexpr int kPf8ChunkKeys = 128;
constexpr int kPf8RowBytes = kIdxDim;                           // 128
constexpr int kPf8KeyBytes = kPf8ChunkKeys * kPf8RowBytes;      // 16 KB
constexpr int kPf8Stride = kPf8KeyBytes + kPf8ChunkKeys;        // keys, then their scales
constexpr int kPf8Copies = kPf8KeyBytes / 1024 / kPfWaves;      // 4: 1 KB copies per wave
constexpr int kPf8Ops = kPf8Copies + 1;                         // memory ops per wave per chunk
static_assert(kPf8Copies * kPfWaves * 1024 == kPf8KeyBytes, "whole copies per wave");

template <int WDT>
__global__ void __launch_bounds__(kPfWaves * 64)
indexer_prefill_fp8(int T, int S, int n_qblk, float idx_scale, const uint8_t* __restrict__ q_idx,
                    const uint8_t* __restrict__ q_sf, const uint8_t* __restrict__ k_idx,
                    const uint8_t* __restrict__ k_sf, const void* __restrict__ w,
                    const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                    int full_rows) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kPfBuffers * kPf8Stride];
  debug_poison_lds<sizeof(kbuf)>(kbuf);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int nb = gridDim.x / n_qblk;                                // sequences
  const int qb = n_qblk - 1 - static_cast<int>(blockIdx.x) / nb;    // longest first
  const int b = static_cast<int>(blockIdx.x) % nb;
  const int t0 = qb * kPfWaves;
  const int t = t0 + wave;
  const bool has_q = t < T;
  const int tq = min(t, T - 1);
  const int L = seq_len(seq_lens, b, S);
  const int q_pos = L - T + tq;
  const int kend = max(0, L - T + min(t0 + kPfWaves, T));  // keys [0, kend) are visible to some query
  const int nchunks = (kend + kPf8ChunkKeys - 1) / kPf8ChunkKeys;
  const int64_t kbase = static_cast<int64_t>(b) * S;
  const uint32_t kb_lds = lds_addr(kbuf);

  // chunk c -> buffer c % kPfBuffers; this wave copies rows 32 wave .. 32
  // wave + 31 (8 rows per 1 KB copy) and the scales of the same 32 keys
  // (keys past S - 1 load row S - 1, scale pieces stay inside the row)
  auto issue_chunk = [&](int c) {
    const uint32_t dst = kb_lds + (c % kPfBuffers) * kPf8Stride;
#pragma unroll
    for (int i = 0; i < kPf8Copies; ++i) {
      const int r = (wave * kPf8Copies + i) * 8 + (lane >> 3);
      const int piece = (lane & 7) ^ ((r >> 1) & 7);
      const int key = min(c * kPf8ChunkKeys + r, S - 1);
      lds_dma_16(k_idx + (kbase + key) * kPf8RowBytes + piece * 16, dst + (wave * kPf8Copies + i) * 1024);
    }
    const int key4 = min(c * kPf8ChunkKeys + 32 * wave + 4 * (lane & 7), S - 4);
    if (lane < 8) lds_dma_4(k_sf + kbase + key4, dst + kPf8KeyBytes + 32 * wave);
  };
#pragma unroll
  for (int c = 0; c < kPfBuffers - 1; ++c)
    if (c < nchunks) issue_chunk(c);

  // ---- the query's codes (A operands) and head weights, in registers ----
  const int64_t row = static_cast<int64_t>(b) * T + tq;
  i32x8_t qa[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const u32x4_t* hp = reinterpret_cast<const u32x4_t*>(q_idx + (row * kIdxHeads + 16 * mb + n) * kIdxDim + 32 * g);
    const u32x4_t lo = __builtin_nontemporal_load(hp);
    const u32x4_t hi = __builtin_nontemporal_load(hp + 1);
    qa[mb] = i32x8_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                     static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                     static_cast<int>(hi[2]), static_cast<int>(hi[3])};
  }
  float wreg[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t hh = row * kIdxHeads + 16 * mb + 4 * g + i;
      wreg[mb][i] = load_w<WDT>(w, hh) * ue8m0_to_f32(q_sf[hh]);
    }

  float* out_row = scores + row * S;

  // one 16-key tile: 4 products into acc (key operands read from LDS)
  auto tile_mfma = [&](const uint8_t* buf, int u, f32x4_t (&acc)[4]) {
    const uint8_t* rp = buf + (16 * u + n) * kPf8RowBytes;
    const int f = (n >> 1) & 7;  // (row >> 1) & 7 of row 16 u + n
    const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(rp + 16 * ((2 * g) ^ f));
    const u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(rp + 16 * ((2 * g + 1) ^ f));
    const i32x8_t kk = {static_cast<int>(k0[0]), static_cast<int>(k0[1]), static_cast<int>(k0[2]),
                        static_cast<int>(k0[3]), static_cast<int>(k1[0]), static_cast<int>(k1[1]),
                        static_cast<int>(k1[2]), static_cast<int>(k1[3])};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x16x128_e4m3(qa[mb], kk, f32x4_t{0.f, 0.f, 0.f, 0.f});
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
  // cross-lane head sum of 4 tiles: lane l ends with key 64 h + l of chunk c
  auto half_store = [&](const uint8_t* buf, int c, int h, const float (&part)[4]) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
    const auto d = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
    const float h0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float h1 = __uint_as_float(d[0]) + __uint_as_float(d[1]);
    const auto e = __builtin_amdgcn_permlane16_swap(__float_as_uint(h0), __float_as_uint(h1), false, false);
    const float ks = ue8m0_to_f32(buf[kPf8KeyBytes + 64 * h + lane]);
    const float v = idx_scale * ((__uint_as_float(e[0]) + __uint_as_float(e[1])) * ks);
    const int key = c * kPf8ChunkKeys + 64 * h + lane;
    if (has_q && key < S) __builtin_nontemporal_store(key <= q_pos ? v : -__builtin_inff(), out_row + key);
  };

  f32x4_t acc0[4], acc1[4];
  float part[4];
  for (int c = 0; c < nchunks; ++c) {
    // chunk c has landed: the copies issued after it are those of chunks
    // c + 1 .. min(c + kPfBuffers - 2, nchunks - 1), kPf8Ops per chunk (the
    // first chunk also waits for the query loads, issued after the copies)
    const int later = min(kPfBuffers - 2, nchunks - 1 - c);
    if (c == 0 || later <= 0)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPf8Ops) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPf8Ops) : "memory");
    __syncthreads();   // every wave's copies of chunk c are in; chunk c - 1 is consumed
    if (c + kPfBuffers - 1 < nchunks) issue_chunk(c + kPfBuffers - 1);
    const uint8_t* buf = kbuf + (c % kPfBuffers) * kPf8Stride;
    tile_mfma(buf, 0, acc0);
#pragma unroll
    for (int u = 1; u < 8; ++u) {
      if (u & 1) tile_mfma(buf, u, acc1); else tile_mfma(buf, u, acc0);
      part[(u - 1) & 3] = (u & 1) ? tile_part(acc0) : tile_part(acc1);
      if (u == 4) half_store(buf, c, 0, part);
    }
    part[3] = tile_part(acc1);
    half_store(buf, c, 1, part);
  }
  // keys past the block's last chunk are in every query's future
  if (has_q && full_rows) {
    const int k0 = nchunks * kPf8ChunkKeys;
    for (int k = k0 + lane; k < S; k += 64) __builtin_nontemporal_store(-__builtin_inff(), out_row + k);
  }
}

// ---------------------------------------------------------------------------
// Streaming MFMA kernel for few queries per sequence (decode), HI = 64,
// DI = 128, bf16 or e4m3.
//
// Decode reads every key row of the sequence once per query: the kernel is a
// stream of k^I from HBM.  Each wave owns a run of consecutive keys and moves
// them through a private ring of four 8 KB LDS buffers with whole-line direct
// copies (global_load_lds_dwordx4: 1 KB of contiguous key rows per
// instruction), three chunks in flight while one is scored; per-lane operand
// loads, whose 16 lanes per key row touch 64-byte pieces, stream slower.  No
// barrier is needed after the query is staged (each wave reads only what it
// copied).
//  * bf16: a key row is 256 bytes, a chunk 32 keys (two 16-key tiles); row
//    r's 16-byte piece c sits in slot c ^ ((r & 7) << 1) and operand step ks
//    of lane (g, n) reads piece 4 ks + g of row n, as in the prefill kernel.
//  * e4m3: a key row is 128 bytes, a chunk 64 keys (four tiles); piece c of
//    row r sits in slot c ^ ((r >> 1) & 7), and lane (g, n) reads pieces 2g
//    and 2g + 1 of row n (its 32 contiguous bytes, the dims of the four
//    fp8 MFMA steps).  Every 16 lanes of a 16-byte read then cover the 64
//    banks once.  The key block scales (one byte per key row) multiply the
//    head sums at the end; the query block scales are folded into w.
// Every 4 tiles finish with a reduce-scatter of the head sums (3 lane swaps,
// 3 adds) that leaves one key's score per lane, so each wave keeps its scores
// in a few registers and stores them at the end, after its last copy.
// ---------------------------------------------------------------------------
constexpr int kStWaves = 4;
constexpr int kStChunkBytes = 8192;                           // per chunk
constexpr int kStBuffers = 4;                                 // per wave
constexpr int kStChunks = 8;                                  // chunks per wave
constexpr int kStCopies = kStChunkBytes / 1024;               // 8 copies per chunk

template <bool FP8>
struct StreamShape {
  static constexpr int kRowBytes = FP8 ? kIdxDim : 2 * kIdxDim;
  static constexpr int kChunkKeys = kStChunkBytes / kRowBytes;  // 64 / 32
  static constexpr int kTiles = kChunkKeys / 16;                // per chunk
  static constexpr int kWaveKeys = kStChunks * kChunkKeys;      // 512 / 256
  static constexpr int kBlockKeys = kStWaves * kWaveKeys;       // 2048 / 1024
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;         // 8 / 4
  static constexpr int kResults = kWaveKeys / 64;               // scores per lane
};

// The fused selection (SELECT): the key-block workgroups of a query row meet
// through two per-row words of the caller's workspace and a 12-bit histogram
// of the row.
//   state[0] = tag (40 bits) << 24 | arrivals (12 bits) << 12 | flushes (12 bits)
//   state[1] = the tag once the row's histogram has been zeroed for this call
// The tag is the call's own (bit 39 clear); a state with another tag is
// stale (an earlier call, or whatever the workspace held) and counts as
// zero.  A workgroup, once its scores are stored (device-scope stores) and
// its block's histogram is built in LDS, arrives: the first arrival of the
// call zeroes the row's histogram and then publishes the tag in state[1];
// every later arrival waits for that (the first arrival is already running,
// so the wait ends), then adds its block histogram to the row's with device
// atomics and counts a flush.  The workgroup whose flush completes the count
// has the whole row: it selects the row's top-K (select_row.h) and writes
// idx, then marks both words stale (tag with bit 39 set), so that a replay
// of the same call starts afresh.  The scores never leave the workspace.

struct SelectArgs {
  int32_t* idx;       // [rows, K]
  int K;
  uint64_t* state;    // [rows, 2]
  uint32_t* hist;     // [rows, 4096]
  uint64_t tag;
};

template <bool FP8, int WDT, bool SELECT>
__global__ void __launch_bounds__(kStWaves * 64)
indexer_stream(int T, int S, int nkb, float idx_scale, const uint8_t* __restrict__ q_idx,
               const uint8_t* __restrict__ q_sf, const uint8_t* __restrict__ k_idx,
               const uint8_t* __restrict__ k_sf, const void* __restrict__ w,
               const int32_t* __restrict__ seq_lens, float* __restrict__ scores, SelectArgs sa) {
  using Sh = StreamShape<FP8>;
  static_assert(!SELECT || sizeof(sel::Lds) <= kStWaves * kStBuffers * kStChunkBytes,
                "the selection's scratch fits the idle key ring");
  constexpr int kWBytes = kIdxHeads * (WDT == DSA_BF16 ? 2 : 4);
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kStWaves * kStBuffers * kStChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kIdxHeads * Sh::kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[kWBytes];
  __shared__ __attribute__((aligned(16))) uint8_t qsf_lds[kIdxHeads];
  debug_poison_lds<sizeof(kbuf)>(kbuf);
  debug_poison_lds<sizeof(q_lds)>(q_lds);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int64_t row = blockIdx.x / nkb;  // b * T + t
  const int kb = static_cast<int>(blockIdx.x % nkb);
  const int b = static_cast<int>(row / T);
  const int t = static_cast<int>(row % T);
  const int L = seq_len(seq_lens, b, S);
  const int s_lim = max(0, min(L, L - T + t + 1));  // keys [0, s_lim) are visible
  const int s_begin = (kb * kStWaves + wave) * Sh::kWaveKeys;
  const int s_end = min(S, s_begin + Sh::kWaveKeys);
  const int s_vis = min(s_end, s_lim);  // this wave scores [s_begin, s_vis)
  const int nch = s_vis > s_begin ? (s_vis - s_begin + Sh::kChunkKeys - 1) / Sh::kChunkKeys : 0;
  const int64_t kbase = static_cast<int64_t>(b) * S;
  const uint32_t wlds = lds_addr(kbuf) + wave * kStBuffers * kStChunkBytes;

  // e4m3 key scale bytes, one per score this lane ends with (issued first:
  // they retire before every copy, so the copy waits below cover them; the
  // key is clamped into [0, s_vis - 1], or is row 0 when nothing is visible)
  uint8_t ksb[Sh::kResults];
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < Sh::kResults; ++j)
      ksb[j] = k_sf[kbase + max(0, min(s_begin + 64 * j + lane, s_vis - 1))];
  }

  // Key rows and query rows share one LDS layout: copy i of a 1 KB block
  // covers rows kRowsPerCopy * i ..; lane l writes slot l % (row / 16) of row
  // kRowsPerCopy * i + l / (row / 16), which holds the piece
  // swizzled into it (bf16: slot ^ ((r & 7) << 1), e4m3: slot ^ ((r >> 1) & 7)).
  auto copy_piece = [&](int i, int& r, int& piece) {
    if constexpr (FP8) {
      r = 8 * i + (lane >> 3);
      piece = (lane & 7) ^ ((r >> 1) & 7);
    } else {
      r = 4 * i + (lane >> 4);
      piece = (lane & 15) ^ ((r & 7) << 1);
    }
  };
  // ---- the query row, the head weights (and the query scales) go out first,
  // as whole-line copies into LDS; the compiler sees no load it must wait for ----
  {
    constexpr int kQCopies = kIdxHeads * Sh::kRowBytes / 1024 / kStWaves;  // per wave: 4 / 2
    const uint8_t* qrow = q_idx + row * kIdxHeads * Sh::kRowBytes;
#pragma unroll
    for (int j = 0; j < kQCopies; ++j) {
      const int i = wave * kQCopies + j;
      int r, piece;
      copy_piece(i, r, piece);
      lds_dma_16(qrow + r * Sh::kRowBytes + piece * 16, lds_addr(q_lds) + 1024 * i);
    }
    if (wave == 0 && lane < kWBytes / 16)
      lds_dma_16(static_cast<const uint8_t*>(w) + row * kWBytes + 16 * lane, lds_addr(w_lds));
    if constexpr (FP8)
      if (wave == 1 && lane < kIdxHeads / 16)
        lds_dma_16(q_sf + row * kIdxHeads + 16 * lane, lds_addr(qsf_lds));
  }

  // chunk c -> buffer c % 4 (keys past the visible range load row s_vis - 1:
  // every address stays in bounds)
  auto issue_chunk = [&](int c) {
    const uint32_t dst = wlds + (c % kStBuffers) * kStChunkBytes;
#pragma unroll
    for (int i = 0; i < kStCopies; ++i) {
      int r, piece;
      copy_piece(i, r, piece);
      const int key = min(s_begin + c * Sh::kChunkKeys + r, s_vis - 1);
      lds_dma_16_nt(k_idx + (kbase + key) * Sh::kRowBytes + piece * 16, dst + 1024 * i);
    }
  };
#pragma unroll
  for (int c = 0; c < kStBuffers - 1; ++c)
    if (c < nch) issue_chunk(c);
  // the query copies are older than the chunks' 8 copies each
  if (nch >= 3)
    asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (nch == 2)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (nch == 1)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave's query copies are in

  float* out_row = scores + row * S;
  if (!SELECT && nch == 0) {  // every key of this wave is in the future (or past S)
    for (int s = s_begin + lane; s < s_end; s += 64) out_row[s] = -__builtin_inff();
    return;
  }
  bf16x8_t qa[4][4];
  long qa8[4][4];
  float wreg[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int h = mb * 16 + n;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // dims 32 g + 8 ks (e4m3) or 32 ks + 8 g (bf16) of head h: its piece,
      // through the row's swizzle
      if constexpr (FP8)
        qa8[mb][ks] = *reinterpret_cast<const long*>(
            q_lds + h * Sh::kRowBytes + 16 * ((2 * g + (ks >> 1)) ^ ((h >> 1) & 7)) + 8 * (ks & 1));
      else
        qa[mb][ks] = *reinterpret_cast<const bf16x8_t*>(
            q_lds + h * Sh::kRowBytes + 16 * ((4 * ks + g) ^ ((h & 7) << 1)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = mb * 16 + 4 * g + i;
      float wv = load_w<WDT>(w_lds, hh);
      if constexpr (FP8) wv *= ue8m0_to_f32(qsf_lds[hh]);
      wreg[mb][i] = wv;
    }
  }

  // e4m3: the head block's 32 query bytes of this lane (dims 32 g .. 32 g + 31)
  i32x8_t qa128[4];
  if constexpr (FP8) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qa128[mb][2 * ks] = static_cast<int>(static_cast<uint64_t>(qa8[mb][ks]) & 0xffffffffu);
        qa128[mb][2 * ks + 1] = static_cast<int>(static_cast<uint64_t>(qa8[mb][ks]) >> 32);
      }
  }
  float res[Sh::kResults];  // lane l: key s_begin + 64 j + l
  float part[4];
#pragma unroll
  for (int c = 0; c < kStChunks; ++c) {
    constexpr int kT = Sh::kTiles;
    const int p0 = (c * kT) & 3;  // first part slot of this chunk
    if (c < nch) {  // wave-uniform
      // chunk c has landed; chunks up to c + 3 go out behind it
      const int ahead = min(kStBuffers - 2, nch - 1 - c);  // chunks issued after chunk c
      if (ahead >= 2)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else if (ahead == 1)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (c + kStBuffers - 1 < nch) issue_chunk(c + kStBuffers - 1);
      const uint8_t* buf = kbuf + (wave * kStBuffers + (c % kStBuffers)) * kStChunkBytes;
#pragma unroll
      for (int u = 0; u < kT; ++u) {
        const uint8_t* rp = buf + (16 * u + n) * Sh::kRowBytes;
        f32x4_t acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
          // one 16x16x128 e4m3 product per head block: lane (g, n) holds
          // dims 32 g .. 32 g + 31 of key n, in the byte order of the
          // query's fragment (pieces 2 g and 2 g + 1 of the row)
          const int f = (n >> 1) & 7;  // (row >> 1) & 7 of row 16 u + n
          const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(rp + 16 * ((2 * g) ^ f));
          const u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(rp + 16 * ((2 * g + 1) ^ f));
          const i32x8_t kk = {static_cast<int>(k0[0]), static_cast<int>(k0[1]), static_cast<int>(k0[2]),
                              static_cast<int>(k0[3]), static_cast<int>(k1[0]), static_cast<int>(k1[1]),
                              static_cast<int>(k1[2]), static_cast<int>(k1[3])};
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x16x128_e4m3(qa128[mb], kk, acc[mb]);
        } else {
          bf16x8_t kv[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            kv[ks] = *reinterpret_cast<const bf16x8_t*>(rp + 16 * ((4 * ks + g) ^ ((n & 7) << 1)));
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x16x32_bf16(qa[mb][ks], kv[ks], acc[mb]);
        }
        float h0 = 0.f, h1 = 0.f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          h0 = fmaf(wreg[mb][0], fmaxf(acc[mb][0], 0.f), h0);
          h1 = fmaf(wreg[mb][1], fmaxf(acc[mb][1], 0.f), h1);
          h0 = fmaf(wreg[mb][2], fmaxf(acc[mb][2], 0.f), h0);
          h1 = fmaf(wreg[mb][3], fmaxf(acc[mb][3], 0.f), h1);
        }
        part[p0 + u] = h0 + h1;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kT; ++u) part[p0 + u] = 0.f;
    }
    if (((c + 1) * kT) % 4 == 0) {  // cross-lane head sum of 4 tiles: lane l ends with key 64 j + l
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float e0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
      const float e1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(e0), __float_as_uint(e1), false, false);
      res[(c * kT) / 4] = __uint_as_float(z[0]) + __uint_as_float(z[1]);
    }
  }
  // ---- the wave's scores: one 256-byte run per 64 keys; future keys -inf ----
  float sv[Sh::kResults];
#pragma unroll
  for (int j = 0; j < Sh::kResults; ++j) {
    const int s = s_begin + 64 * j + lane;
    float v;
    if constexpr (FP8) v = idx_scale * (res[j] * ue8m0_to_f32(ksb[j]));
    else v = idx_scale * res[j];
    sv[j] = s < s_lim ? v : -__builtin_inff();
    if constexpr (SELECT) {
      if (s < s_end) __hip_atomic_store(out_row + s, sv[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (s < s_end) __builtin_nontemporal_store(sv[j], out_row + s);
    }
  }
  if constexpr (SELECT) {
    // ---- the block's histogram, the row's meeting, the last one selects ----
    __shared__ uint32_t sel_flag;
    const int tid = threadIdx.x;
    uint32_t* lh = reinterpret_cast<uint32_t*>(kbuf);  // every wave is past its last chunk
    __syncthreads();
    for (int i = tid; i < sel::kBins1; i += kStWaves * 64) lh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < Sh::kResults; ++j) {
      const uint32_t key = score_key(sv[j]);
      if (s_begin + 64 * j + lane < s_end && key != 0u) atomicAdd(&lh[key >> 20], 1u);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's score stores are complete
    __syncthreads();
    uint64_t* st = sa.state + 2 * row;
    uint32_t* gh = sa.hist + row * sel::kBins1;
    if (tid == 0) {
      // once the call's tag is in the word, arrivals only add; a compare and
      // swap installs the tag (the first arrival) and is retried only while
      // the word is stale
      uint64_t old = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool first = false;
      for (;;) {
        if ((old >> 24) == sa.tag) {
          __hip_atomic_fetch_add(st, uint64_t(1) << 12, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        if (__hip_atomic_compare_exchange_strong(st, &old, (sa.tag << 24) | (uint64_t(1) << 12),
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
          first = true;
          break;
        }
      }
      sel_flag = first ? 1u : 0u;
    }
    __syncthreads();
    if (sel_flag) {  // the first arrival: a zeroed row histogram, then the tag
      for (int i = tid; i < sel::kBins1; i += kStWaves * 64)
        __hip_atomic_store(gh + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) __hip_atomic_store(st + 1, sa.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (tid == 0) {  // wait for the first arrival's zeroing (it is running)
      for (int spin = 0; spin < kSelWaitSpins &&
                         __hip_atomic_load(st + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != sa.tag;
           ++spin)
        __builtin_amdgcn_s_sleep(4);
    }
    __syncthreads();
    for (int i = tid; i < sel::kBins1; i += kStWaves * 64) {
      const uint32_t c = lh[i];
      if (c != 0u) __hip_atomic_fetch_add(gh + i, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's histogram adds are complete
    __syncthreads();
    if (tid == 0) {
      const uint64_t old = __hip_atomic_fetch_add(st, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sel_flag = (static_cast<int>(old & 0xfffu) + 1 == nkb) ? 1u : 0u;
    }
    __syncthreads();
    if (!sel_flag) return;
    sel::Lds& L = *reinterpret_cast<sel::Lds*>(kbuf);
    sel::select_row(L, out_row, S, gh, sa.K, sa.idx + row * sa.K);
    if (tid == 0) {
      __hip_atomic_store(st, (sa.tag | kTagStale) << 24, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(st + 1, sa.tag | kTagStale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int IDT, int WDT>
dsa_status_t run_generic(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                         const void* k_idx, const uint8_t* k_sf, const void* w,
                         const int32_t* seq_lens, float* scores, hipStream_t stream) {
  const size_t lds = (static_cast<size_t>(s.HI) * s.DI + s.HI) * sizeof(float);
  if (lds > 64 * 1024)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: HI*DI = %d too large for the generic kernel",
                s.HI * s.DI);
  dim3 grid((s.S + 255) / 256, s.B * s.T);
  LaunchTimer timer;
  hipExtLaunchKernelGGL(indexer_generic<IDT, WDT>, grid, dim3(256), lds, stream, timer.start(),
                        timer.stop(), 0, s.T, s.S, s.HI, s.DI, s.idx_scale, q_idx, q_sf, k_idx,
                        k_sf, w, seq_lens, scores);
  return timer.done("indexer_generic");
}

template <bool FP8, int WDT, bool SELECT = false>
dsa_status_t run_stream(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                        const void* k_idx, const uint8_t* k_sf, const void* w,
                        const int32_t* seq_lens, float* scores, hipStream_t stream,
                        SelectArgs sa = SelectArgs{}) {
  constexpr int kBlockKeys = StreamShape<FP8>::kBlockKeys;
  const int nkb = (s.S + kBlockKeys - 1) / kBlockKeys;
  const int64_t blocks = static_cast<int64_t>(s.B) * s.T * nkb;
  if (blocks > 0x7fffffff)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: %lld key blocks", static_cast<long long>(blocks));
  LaunchTimer timer;
  hipExtLaunchKernelGGL((indexer_stream<FP8, WDT, SELECT>), dim3(static_cast<unsigned>(blocks)),
                        dim3(kStWaves * 64), 0, stream, timer.start(), timer.stop(), 0, s.T, s.S,
                        nkb, s.idx_scale, static_cast<const uint8_t*>(q_idx), q_sf,
                        static_cast<const uint8_t*>(k_idx), k_sf, w, seq_lens, scores, sa);
  return timer.done(SELECT ? "indexer_select" : "indexer_stream");
}

template <int WDT>
dsa_status_t run_prefill_fp8(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                             const void* k_idx, const uint8_t* k_sf, const void* w,
                             const int32_t* seq_lens, float* scores, bool full_rows, hipStream_t stream) {
  const int n_qblk = (s.T + kPfWaves - 1) / kPfWaves;
  const int64_t blocks = static_cast<int64_t>(n_qblk) * s.B;
  if (blocks > 0x7fffffff)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: %lld query blocks", static_cast<long long>(blocks));
  LaunchTimer timer;
  hipExtLaunchKernelGGL(indexer_prefill_fp8<WDT>, dim3(static_cast<unsigned>(blocks)),
                        dim3(kPfWaves * 64), 0, stream, timer.start(), timer.stop(), 0, s.T, s.S,
                        n_qblk, s.idx_scale, static_cast<const uint8_t*>(q_idx), q_sf,
                        static_cast<const uint8_t*>(k_idx), k_sf, w, seq_lens, scores, full_rows ? 1 : 0);
  return timer.done("indexer_prefill_fp8");
}

template <int WDT>
dsa_status_t run_prefill(const dsa_shape_t& s, const void* q_idx, const void* k_idx,
                         const void* w, const int32_t* seq_lens, float* scores, bool full_rows,
                         hipStream_t stream) {
  const int n_qblk = (s.T + kPfQueries - 1) / kPfQueries;
  const int64_t blocks = static_cast<int64_t>(n_qblk) * s.B;
  if (blocks > 0x7fffffff)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: %lld query blocks", static_cast<long long>(blocks));
  LaunchTimer timer;
  hipExtLaunchKernelGGL(indexer_prefill<WDT>, dim3(static_cast<unsigned>(blocks)),
                        dim3(kPfQueries * 64), 0, stream, timer.start(), timer.stop(), 0, s.T, s.S,
                        n_qblk, s.idx_scale, static_cast<const uint16_t*>(q_idx),
                        static_cast<const uint16_t*>(k_idx), w, seq_lens, scores, full_rows ? 1 : 0);
  return timer.done("indexer_prefill");
}

}  // namespace

bool indexer_select_applies(const dsa_shape_t& s) {
  return s.HI == kIdxHeads && s.DI == kIdxDim && s.T < kPfMinQueries && s.S <= sel::kMaxRow &&
         (s.idx_dtype == DSA_BF16 || s.idx_dtype == DSA_FP8_E4M3) &&
         static_cast<int64_t>(s.B) * s.T <= 65535;
}

size_t indexer_select_workspace_bytes(const dsa_shape_t& s) {
  const size_t rows = static_cast<size_t>(s.B) * s.T;
  return rows * (2 * sizeof(uint64_t) + sel::kBins1 * sizeof(uint32_t));
}

dsa_status_t launch_indexer_select(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                                   const void* k_idx, const uint8_t* k_sf, const void* w,
                                   const int32_t* seq_lens, float* scores, int32_t* idx,
                                   void* sel_ws, uint64_t tag, hipStream_t stream) {
  if (!indexer_select_applies(s))
    return fail(DSA_ERR_UNSUPPORTED, "indexer_select: shape not covered by the fused selection");
  const size_t rows = static_cast<size_t>(s.B) * s.T;
  SelectArgs sa;
  sa.idx = idx;
  sa.K = k_eff(s);
  sa.state = static_cast<uint64_t*>(sel_ws);
  sa.hist = reinterpret_cast<uint32_t*>(static_cast<char*>(sel_ws) + rows * 2 * sizeof(uint64_t));
  sa.tag = tag & (kTagStale - 1);
  const bool wbf = s.w_dtype == DSA_BF16;
  if (s.idx_dtype == DSA_BF16)
    return wbf ? run_stream<false, DSA_BF16, true>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream, sa)
               : run_stream<false, DSA_F32, true>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream, sa);
  return wbf ? run_stream<true, DSA_BF16, true>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream, sa)
             : run_stream<true, DSA_F32, true>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream, sa);
}

dsa_status_t launch_indexer(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                            const void* k_idx, const uint8_t* k_sf, const void* w,
                            const int32_t* seq_lens, float* scores, bool full_rows,
                            hipStream_t stream) {
  const bool v32 = s.HI == kIdxHeads && s.DI == kIdxDim;
  const bool wbf = s.w_dtype == DSA_BF16;
  if (v32 && s.idx_dtype == DSA_BF16 && s.T >= kPfMinQueries)
    return wbf ? run_prefill<DSA_BF16>(s, q_idx, k_idx, w, seq_lens, scores, full_rows, stream)
               : run_prefill<DSA_F32>(s, q_idx, k_idx, w, seq_lens, scores, full_rows, stream);
  if (v32 && s.idx_dtype == DSA_BF16)
    return wbf ? run_stream<false, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream)
               : run_stream<false, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream);
  if (v32 && s.idx_dtype == DSA_FP8_E4M3 && s.T >= kPfMinQueries && s.S % 4 == 0)
    return wbf ? run_prefill_fp8<DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, full_rows, stream)
               : run_prefill_fp8<DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, full_rows, stream);
  if (v32 && s.idx_dtype == DSA_FP8_E4M3)
    return wbf ? run_stream<true, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream)
               : run_stream<true, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream);
  // the generic kernel puts the query row on grid.y
  if (static_cast<int64_t>(s.B) * s.T > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: B*T = %lld exceeds 65535 query rows",
                static_cast<long long>(s.B) * s.T);
  switch (s.idx_dtype) {
    case DSA_F32:
      return wbf ? run_generic<DSA_F32, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream)
                 : run_generic<DSA_F32, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream);
    case DSA_BF16:
      return wbf ? run_generic<DSA_BF16, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream)
                 : run_generic<DSA_BF16, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream);
    case DSA_FP8_E4M3:
      return wbf ? run_generic<DSA_FP8_E4M3, DSA_BF16>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream)
                 : run_generic<DSA_FP8_E4M3, DSA_F32>(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, stream);
  }
  return fail(DSA_ERR_UNSUPPORTED, "indexer: unknown idx_dtype %d", s.idx_dtype);
}

}  // namespace dsa
