// Sparse latent attention in absorbed form on gfx950.
//
// For each query row (b, t) and head h, over the keys j listed in idx[b,t,:]
// (entries -1 or outside [0, S) skipped, duplicates counted as written):
//   logit_j = sm_scale * (q[h, 0:Dc] . c_j + q[h, Dc:Dc+Dr] . r_j),  kv_j = [c_j ; r_j]
//   o[h, :] = sum_j softmax(logit)_j c_j,   lse[h] = log sum_j exp(logit_j)
// (atlas.klimoza.dev, DeepSeek-V3.2-Exp MoE block, "All 43 steps": keys
// [K^C ; k^R] with the same rotary key for every head, values c W_UV; taken in
// absorbed form, q_lat = W_UK q^C, so every head reads the same 576-wide
// row.  nnterp deepseek_v32, sections 03/04: zero probability outside the
// selection, each row sums to one over it.)
//
// Kernels:
//  * mla_mfma (H = 128, Dc = 512, Dr = 64, bf16): one workgroup of 4 waves
//    (one per SIMD) takes one query row and one split of its index list.  All
//    128 heads share each gathered tile of 32 selected key rows, copied
//    straight from global memory into LDS (row-major, swizzled) and read
//    twice: directly for the logits and through transposing LDS reads for the
//    value product.  Wave w owns heads 32w..32w+31: logits^T = K_tile . Q^T on
//    32x32x16 MFMAs (keys on M, heads on N), an online softmax in fp32 with
//    exp2 against a fixed reference max, and O^T += V^T . P^T (latent dims on
//    M, heads on N) with P^T taken straight from the logit accumulators.  A
//    ring of 4 LDS tiles holds the tile of the value product, the tile of the
//    logits and two tiles whose copies are in flight.  With too few query
//    rows to give every CU a workgroup even at the finest split, a workgroup
//    of 2 waves takes 64 heads instead (two workgroups per split, on one XCD,
//    gathering the same rows): twice the workgroups, half the query block
//    and half the partials per workgroup.
//  * mla_combine: merges split partials (o_s, lse_s) with weights
//    exp(lse_s - lse), deterministically (fixed split order, no atomics).
//  * mla_generic: any shape, fp32 VALU loops, two passes over the index row.
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DT>
__device__ __forceinline__ float load_mla(const void* p, int64_t i) {
  if constexpr (DT == DSA_BF16)
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else
    return static_cast<const float*>(p)[i];
}

template <int DT>
__device__ __forceinline__ void store_mla(void* p, int64_t i, float v) {
  if constexpr (DT == DSA_BF16)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else
    static_cast<float*>(p)[i] = v;
}

// ---------------------------------------------------------------------------
// generic kernel: one workgroup per (head, query row)
// ---------------------------------------------------------------------------
template <int DT>
__global__ void __launch_bounds__(256)
mla_generic(int T, int S, int H, int Dc, int Dr, int W, float sm_scale,
            const void* __restrict__ q, const void* __restrict__ kv,
            const int32_t* __restrict__ idx, void* __restrict__ o, float* __restrict__ lse) {
  extern __shared__ float smem[];
  const int D = Dc + Dr;
  float* qs = smem;            // [D]
  float* logit = smem + D;     // [W]
  __shared__ float red[256 / 64];
  const int h = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int b = static_cast<int>(row / T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = threadIdx.x; d < D; d += blockDim.x) qs[d] = load_mla<DT>(q, (row * H + h) * D + d);
  __syncthreads();
  float mloc = -__builtin_inff();
  for (int j = threadIdx.x; j < W; j += blockDim.x) {
    const int s = idx[row * W + j];
    float x = -__builtin_inff();
    if (s >= 0 && s < S) {
      const int64_t kr = (static_cast<int64_t>(b) * S + s) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], load_mla<DT>(kv, kr + d), dot);
      x = sm_scale * dot;
    }
    logit[j] = x;
    mloc = fmaxf(mloc, x);
  }
  mloc = wave_max(mloc);
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < 4; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  float lloc = 0.f;
  if (m != -__builtin_inff()) {
    for (int j = threadIdx.x; j < W; j += blockDim.x) {
      const float p = __expf(logit[j] - m);  // exp(-inf) = 0 for skipped entries
      logit[j] = p;
      lloc += p;
    }
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[wave] = lloc;
  __syncthreads();
  const float l = red[0] + red[1] + red[2] + red[3];
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  for (int d = threadIdx.x; d < Dc; d += blockDim.x) {
    float acc = 0.f;
    if (l > 0.f) {
      for (int j = 0; j < W; ++j) {
        const int s = idx[row * W + j];
        if (s < 0 || s >= S) continue;
        acc = fmaf(logit[j], load_mla<DT>(kv, (static_cast<int64_t>(b) * S + s) * D + d), acc);
      }
    }
    store_mla<DT>(o, (row * H + h) * Dc + d, acc * inv_l);
  }
  if (lse != nullptr && threadIdx.x == 0)
    lse[row * H + h] = l > 0.f ? m + __logf(l) : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// MFMA kernel, H = 128, Dc = 512, Dr = 64, bf16
//
// One workgroup of 4 waves (one per SIMD, 512 registers each) takes one query
// row and one split of its index list; wave w owns heads 32w .. 32w+31.  All
// 128 heads share each gathered tile of 32 selected key rows.
//
// Both products run on v_mfma_f32_32x32x16_bf16 (lane l, h = l / 32,
// m = l % 32):
//   A (32 x 16): lane holds row m, reduction elements 8h .. 8h+7
//   B (16 x 32): lane holds column m, reduction elements 8h .. 8h+7
//   C (32 x 32): register i holds row 8(i/4) + 4h + i%4 of column m
// A wave issues about one instruction per 4 cycles and this MFMA holds the
// matrix pipe for 32 cycles (also as one dependent accumulation chain), so
// the loop is laid out to spend well under 8 other instructions per MFMA.
//
// logits^T (32 keys x 32 heads) = K_tile (A, from LDS) . Q^T (B, registers),
// 36 steps of 16 dims in one chain: lane (h, m) ends with head m and keys
// 8(i/4) + 4h + i%4.  The softmax is per lane (one head, 16 keys) plus one
// lane swap across the halves.  O^T (512 dims x 32 heads) += V^T (A) . P^T
// (B) in 16 dim blocks x 2 key steps: P^T is the lane's own probabilities
// (key step s takes registers 8s .. 8s+7, so B slot 8h + e holds key
// 16s + 8(e/4) + 4h + e%4), and V^T comes from the row-major key tile through
// the transposing read ds_read_b64_tr_b16 (within 16 lanes, lane i receives
// element i%4 of the 8-byte chunks loaded by lanes 4j + i/4, j = 0..3): lane
// 4j + q of 16-lane group (h, d) loads dims 32db + 16d + 4q .. +3 of key
// 16s + 4h + j, and of key 16s + 8 + 4h + j for the other half of its slots.
//
// Iteration t computes logits(t), then the softmax of tile t interleaved with
// the value product of tile t - 1: with a fixed reference max (below) the two
// are independent, and the softmax's VALU work fills the issue slots the
// value MFMAs leave free.
//
// Key tile in LDS (38 KiB): latent part of row r at byte 1088 r (1 KiB + 64 B
// pad), 16-byte piece p at (p & ~3) | ((p & 3) ^ ((r >> 2) & 3)); rotary part
// in a region of its own at byte 34816, row r at 128 r, piece p' at
// p' ^ ((r >> 1) & 7).  The LDS has 64 banks of 4 bytes; a 16-byte read
// serves two 8-lane groups per cycle (lanes 0-7 with 24-31, 8-15 with 16-23,
// 32-39 with 56-63, 40-47 with 48-55) and a transposing 8-byte read lanes
// 0-31, then 32-63 (measured with the bank conflict counter on gfx950).  With
// this placement every read of the loop touches each bank once per cycle.
//
// Tiles are filled by direct global->LDS copies (global_load_lds_dwordx4:
// lane l of a wave writes 16 B at the wave's LDS base + 16 l): wave w copies
// the latent parts of rows R w .. R w + R - 1 (R = 8 with 4 waves, 16 with
// 2; one 1 KiB run each) and the rotary parts of the same rows (8 rows per
// copy), spread over its logits steps.  A ring of 4 tiles holds the tile of the value
// product, the tile of the logits and two tiles in flight.  Before the first
// tile the ring stages the query (one buffer per wave), after the last one
// the output (bf16 [head][dims], stored as whole 1 KiB head rows).
// ---------------------------------------------------------------------------
constexpr int kH = 128, kDc = 512, kDr = 64, kD = kDc + kDr;
constexpr int kTileKeys = 32;
constexpr int kBuffers = 4;                  // LDS tile ring
constexpr int kLatStride = 1088;             // bytes per latent row in LDS (1024 + 64 pad)
constexpr int kRopeBase = kTileKeys * kLatStride;            // byte offset of the rotary region
constexpr int kTileBytes = kRopeBase + kTileKeys * kDr * 2;  // 38912
constexpr int kKSteps = kD / 16;             // 36 logits reduction steps of 16 dims
constexpr int kLatSteps = kDc / 16;          // 32 of them over the latent part
constexpr int kDimBlocks = kDc / 32;         // 16 value blocks of 32 dims
constexpr int kPvSteps = 2 * kDimBlocks;     // value MFMAs per tile (2 key steps)
constexpr int kReadAhead = 4;                // logits A-operand reads issued ahead of their MFMAs
constexpr int kVAhead = 4;                   // value A operands (2 reads each) issued ahead
constexpr float kRefSlack = 32.0f;           // log2 units: p <= 2^32 against the reference max
constexpr int kIdxWin = 1024;                // index entries staged in LDS at a time (4 waves)

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) const char lds_char_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

struct MlaTile {
  uint8_t bytes[kTileBytes];
};

// slot of 16-byte piece p in a row whose 4-piece groups are permuted by f
__device__ __forceinline__ int swz4(int p, int f) { return (p & ~3) | ((p & 3) ^ f); }
__device__ __forceinline__ int lat_f(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

// Address arithmetic on LDS pointers stays in the 32-bit LDS address space, so
// constant offsets fold into the instructions' offset fields.
__device__ __forceinline__ short4_t lds_read_tr16(lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

__device__ __forceinline__ f32x16_t mfma32x32x16_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                                      const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The logits chain keeps its accumulator in VGPRs (the value product holds
// all AGPRs): issued through asm, whose register constraints pin the class.
// Consecutive MFMAs of one chain (same destination and srcC) need no wait
// states; the closing nops cover those before VALU reads of the result.
__device__ __forceinline__ void mfma32_first(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_acc(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// (the result passes through the nops, so no reader can move above them)
__device__ __forceinline__ void mfma32_drain(f32x16_t& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}

// max of three without the NaN-quieting the compiler adds around maxnum on
// values it cannot prove canonical (the logits are finite or -inf)
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// two fp32 -> packed bf16 pair (low half = a), round to nearest even, one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{a, b}, bf16x2v_t));
}

// NW waves (4: heads 0..127; 2: a head half, 64 heads from head0).  1-D grid
// of rows * nsplit * (4 / NW) workgroups.  With xcd_map, the workgroups of
// one query row share an XCD (workgroups are dealt to the 8 XCDs
// round-robin), so its 147 KB query block and, with 2 waves, the key rows
// both head halves gather are fetched once into that XCD's L2.
// nsplit == 1: writes o (bf16) and lse directly; otherwise writes bf16
// partials part_o [rows, nsplit, H, Dc] (already divided by the split's own
// sum) and part_lse [rows, H, nsplit] (natural log; -inf for an empty split).
template <int NW>
__global__ void __launch_bounds__(NW * 64, 1)
mla_mfma(int T, int S, int W, int kps, int nsplit, int xcd_map, float sm_scale,
         const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
         const int32_t* __restrict__ idx, uint16_t* __restrict__ o, float* __restrict__ lse,
         uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(1024))) MlaTile tiles[kBuffers];
  // a window of the split's index entries as key rows (-1: skipped entry)
  // index window: 4 entries per thread (4 waves: 1024, 2 waves: 512)
  constexpr int kWin = kIdxWin * NW / 4;
  constexpr int kWinTiles = kWin / kTileKeys;
  __shared__ __attribute__((aligned(16))) int32_t idxw[kWin];
  static_assert(NW == 4 || NW == 2, "4 waves (128 heads) or 2 waves (64 heads) per workgroup");
  constexpr int kThreads = NW * 64;
  constexpr int kRowsPerWave = kTileKeys / NW;        // tile rows each wave copies: 8 or 16
  constexpr int kRopeCopies = kRowsPerWave / 8;       // their rotary parts, 8 rows per 1 KiB copy
  constexpr int kCopies = kRowsPerWave + kRopeCopies; // copies per wave per tile: 9 or 18
  constexpr int kCopyStep = kKSteps / kCopies;        // logits steps per copy: 4 or 2
  constexpr int kWinPer = kWin / kThreads;            // index window entries per thread
  static_assert(kCopyStep * kCopies == kKSteps && kCopyStep >= 2, "copies spread over the logits steps");
  __shared__ int32_t last_valid[NW];  // per wave: the split's last valid entry it saw
  debug_poison_lds<sizeof(tiles)>(tiles);
  debug_poison_lds<sizeof(idxw)>(idxw);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, m = lane & 31;
  const int L = blockIdx.x;
  // workgroups per query row: the splits, times 2 head halves with 2 waves
  constexpr int kHalves = 4 / NW;
  const int nsh = nsplit * kHalves;
  int sh;
  int64_t row;
  if (xcd_map) {
    sh = (L >> 3) % nsh;
    row = static_cast<int64_t>(L / (8 * nsh)) * 8 + (L & 7);
  } else {
    sh = L % nsh;
    row = L / nsh;
  }
  const int sp = sh / kHalves;
  const int head0 = (sh % kHalves) * 32 * NW;  // the workgroup's first head
  const int b = static_cast<int>(row / T);
  const int j0 = sp * kps;
  const int nj = max(0, min(W, j0 + kps) - j0);
  int ntiles;  // tiles up to the split's last valid entry (set with the first index window)
  const uint16_t* kv_seq = kv + static_cast<int64_t>(b) * S * kD;

  // The split's index entries go through LDS a window at a time: thread i
  // loads entries i, i + 256, ... of the window (past the split's end: -1).
  const int32_t* idx_row = idx + row * W;
  const int j_end = j0 + nj;
  int win[kWinPer];
  auto load_window = [&](int w) {
#pragma unroll
    for (int u = 0; u < kWinPer; ++u) {
      const int j = j0 + w * kWin + tid + u * kThreads;
      win[u] = j < j_end ? idx_row[j] : -1;
    }
  };
  auto store_window = [&]() {
#pragma unroll
    for (int u = 0; u < kWinPer; ++u)
      idxw[tid + u * kThreads] = (win[u] >= 0 && win[u] < S) ? win[u] : -1;
  };

  // Query operand (B of logits^T): qf[ks] = head 32w + m, dims 16ks + 8h .. +8,
  // i.e. 16-byte piece 2ks + h of the head's row.  Wave w's 32 heads are one
  // contiguous 36 KiB run of q, copied with whole-line copies into ring buffer
  // w (head n at byte 1152 n, piece p in slot p ^ ((n >> 1) & 7): rows 72
  // slots apart, so the operand reads touch every bank once per cycle).  The
  // copies go out before the index window's loads, so both latencies overlap;
  // the 8 splits of a query row share an XCD and 7 of them find it in L2.
  bf16x8_t qf[kKSteps];
  {
    const char* qsrc = reinterpret_cast<const char*>(q + (row * kH + head0 + 32 * wave) * kD);
    const uint32_t qlds = lds_addr(tiles[wave].bytes);
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
#pragma unroll 4
    for (int i = 0; i < 32 * kD * 2 / 1024; ++i) {
      const int x = 1024 * i + 16 * ln;  // staging byte this lane's copy lands on
      const int n = x / (kD * 2), slot = (x - n * (kD * 2)) >> 4;
      lds_dma_16(qsrc + n * (kD * 2) + 16 * (slot ^ ((n >> 1) & 7)), qlds + 1024 * i);
    }
  }
  load_window(0);
  // The split ends after its last valid entry: the entries past it add
  // nothing (top-K rows of queries with fewer than K visible keys end in -1
  // padding, which this drops).  Entries beyond the first window are read
  // here once more only for splits longer than the window.
  {
    int last = -1;
#pragma unroll
    for (int u = 0; u < kWinPer; ++u)
      if (win[u] >= 0 && win[u] < S) last = j0 + tid + u * kThreads;
    for (int j = j0 + kWin + tid; j < j_end; j += kThreads) {
      const int e = idx_row[j];
      if (e >= 0 && e < S) last = j;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    if (lane == 0) last_valid[wave] = last;
  }
  store_window();   // waits for the window's loads, and so for the query copies issued before them
  __syncthreads();  // the first index window and the last valid entries are published
  {
    int last = last_valid[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) last = max(last, last_valid[w]);
    const int nj_used = last >= j0 ? last - j0 + 1 : 0;
    ntiles = __builtin_amdgcn_readfirstlane((nj_used + kTileKeys - 1) / kTileKeys);
  }
  {
    lds_char_t* qst = (lds_char_t*)(tiles[wave].bytes) + m * (kD * 2);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qf[ks] = *(__attribute__((address_space(3))) const bf16x8_t*)(
          qst + 16 * ((2 * ks + hl) ^ ((m >> 1) & 7)));
  }
  f32x16_t oacc[kDimBlocks];  // O^T: oacc[db][i] = O[head 32w + m][32db + 8(i/4) + 4h + i%4]
#pragma unroll
  for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_ref = -__builtin_inff();  // reference max (log2 units) of head 32w + m
  float l_run = 0.f;
  const float scale2 = sm_scale * kLog2e;

  // Wave w copies tile rows R w .. R w + R - 1 (R = kRowsPerWave; latent and
  // rotary parts), reading their key rows from the index window.  Skipped entries copy key row 0 of the sequence: their
  // logits are replaced by -inf, so their probabilities are exactly zero and
  // (finite) rows add nothing to O.
  // the sequence's base address, wave-uniform (the copies take it in SGPRs)
  const char* kvb;
  {
    const uint64_t a = reinterpret_cast<uint64_t>(kv_seq);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    kvb = reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
  }
  // latent copy of row R w + k: lane ln's 16-byte slot holds piece swz4(ln, f),
  // f = lat_f(R w + k), the same for each group of 4 rows
  int lat_lo[kRowsPerWave / 4];
#pragma unroll
  for (int g4 = 0; g4 < kRowsPerWave / 4; ++g4)
    lat_lo[g4] = 16 * swz4(lane, lat_f(kRowsPerWave * wave + 4 * g4));
  // rotary copy c: lane ln takes row R w + 8c + ln/8, slot ln % 8
  int rope_r[kRopeCopies], rope_lo[kRopeCopies];
#pragma unroll
  for (int c = 0; c < kRopeCopies; ++c) {
    rope_r[c] = kRowsPerWave * wave + 8 * c + (lane >> 3);
    rope_lo[c] = 2 * kDc + 16 * ((lane & 7) ^ rope_swz(rope_r[c]));
  }
  struct TileCopies {
    const int32_t* wrow;  // the tile's 32 index entries in the window
    uint32_t lds;
  };
  // the tile's validity mask (bit r: tile row r holds a valid key), formed by
  // every wave for itself from the index entries when the tile's copies go
  // out (`entry`: entry lane & 31, read earlier so that its latency stays
  // hidden); kept in scalar registers until the tile's logits
  auto tile_mask = [&](int entry) { return static_cast<uint32_t>(__ballot(entry >= 0)); };
  auto prep_tile = [&](int t) {
    TileCopies c;
    c.wrow = &idxw[(t % kWinTiles) * kTileKeys];
    c.lds = lds_addr(tiles[(t + 2) % kBuffers].bytes);
    return c;
  };
  // key row of copy k (k < R: tile row R w + k, all lanes; then the rotary
  // copies, row rope_r[k - R] per lane), read from the index window just
  // before the copy goes out (skipped: row 0)
  auto copy_key = [&](const TileCopies& c, int k) {
    return k < kRowsPerWave ? c.wrow[kRowsPerWave * wave + k] : c.wrow[rope_r[k - kRowsPerWave] & 31];
  };
  // byte offsets within the sequence fit 32 bits (S * 1152 < 2^32, checked on the host)
  auto copy_row = [&](const TileCopies& c, int k, int s) {
    // opaque, here at the use: the key read stays in flight until the copy,
    // and the row offset is formed per lane on the VALU, not the scalar unit
    asm volatile("" : "+v"(s));
    s = max(s, 0);
    const int lo = k < kRowsPerWave ? lat_lo[k >> 2] : rope_lo[k - kRowsPerWave];
    // (wave-uniform; readfirstlane keeps it in a scalar register for m0)
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        k < kRowsPerWave ? c.lds + kLatStride * (kRowsPerWave * wave + k)
                         : c.lds + kRopeBase + 1024 * (kRopeCopies * wave + k - kRowsPerWave));
    lds_dma_16_sbase(kvb, static_cast<uint32_t>(s) * static_cast<uint32_t>(kD * 2) + lo, dst);
  };
  // all of a tile's copies at once (start-up): the key reads go out together
  auto issue_tile = [&](int t) {
    const TileCopies c = prep_tile(t);
    int keys[kCopies];
#pragma unroll
    for (int k = 0; k < kCopies; ++k) keys[k] = copy_key(c, k);
    const uint32_t vm = tile_mask(c.wrow[lane & 31]);
#pragma unroll
    for (int k = 0; k < kCopies; ++k) copy_row(c, k, keys[k]);
    return vm;
  };
  // wait until at most `pending` later tiles' copies of this wave are in flight
  auto wait_tiles = [&](int pending) {
    static_assert(kCopies < 64, "vmcnt immediate");
    if (pending <= 0)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopies) : "memory");
  };

  // LDS byte offsets.  Logits A operand of step ks: row m, piece 2ks + h:
  // latent steps at aoff[ks & 1] + 64 (ks >> 1), rotary steps at roff[ks - 32].
  int aoff[2], roff[4];
#pragma unroll
  for (int par = 0; par < 2; ++par) aoff[par] = kLatStride * m + 16 * ((2 * par + hl) ^ lat_f(m));
#pragma unroll
  for (int k = 0; k < 4; ++k) roff[k] = kRopeBase + 128 * m + 16 * ((2 * k + hl) ^ rope_swz(m));
  // Transposing reads of key step s, dim block db: lane (h, d, j, q) reads
  // dims 32db + 16d + 4q of key 16s + 4h + j (vbase[0]) or 16s + 8 + 4h + j
  // (vbase[1]); lat_f of those rows is h, resp. 2 + h.
  int vbase[2];
  {
    const int dh = (lane >> 4) & 1, j = (lane >> 2) & 3, qd = lane & 3;
    vbase[0] = kLatStride * (4 * hl + j) + 16 * ((2 * dh + (qd >> 1)) ^ hl) + 8 * (qd & 1);
    vbase[1] = kLatStride * (8 + 4 * hl + j) + 16 * ((2 * dh + (qd >> 1)) ^ (2 + hl)) + 8 * (qd & 1);
  }

  // start-up: every wave has its query in registers, the ring is free; tiles
  // 0 and 1 go out
  __syncthreads();
  // masks of the tile of the next logits and of the one after it
  uint32_t vm_a = 0u, vm_b = 0u;
  if (ntiles > 0) vm_a = issue_tile(0);
  if (ntiles > 1) vm_b = issue_tile(1);

  // Online softmax with a fixed reference max per head: the first tile with a
  // valid key sets it, and p = 2^(x - ref) stays below 2^kRefSlack as long as
  // no later logit exceeds the reference by more than the slack.  If one does
  // (never for sane data), the whole split is run once more with the true
  // maximum as reference, so O is only ever zeroed, never rescaled.  The
  // decision is workgroup-uniform (barriers stay matched).
  float m_seen = -__builtin_inff();
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
#pragma unroll
      for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
      l_run = 0.f;
      m_ref = m_seen;
    }
    bool overflow = false;
    if (pass == 1 && ntiles > kWinTiles) {  // the window moved on: back to the first
      load_window(0);
      store_window();
      __syncthreads();
    }
    if (pass == 1) {
      if (ntiles > 0) vm_a = issue_tile(0);
      if (ntiles > 1) vm_b = issue_tile(1);
    }

    f32x16_t sacc;   // logits^T of the current tile (raw dot products)
    bf16x8_t pb[2];  // P^T of the previous tile, key steps 0 and 1
    u32x4_t pn[2];   // P^T of the current tile, being formed (bf16 pairs)

    // ---- logits^T of tile it, with the copies of tile it + 2 ----
    // COPIES: with the copies of the tile two ahead (all but the last two tiles)
    auto logits = [&](auto copies_tag, lds_char_t* cur, const TileCopies& nxt, uint32_t& vm_nxt) {
      constexpr bool copies = decltype(copies_tag)::value;
      auto aload = [&](int ks) {
        const int off = ks < kLatSteps ? aoff[ks & 1] + 64 * (ks >> 1) : roff[ks - kLatSteps];
        return *(__attribute__((address_space(3))) const bf16x8_t*)(cur + off);
      };
      bf16x8_t ka[kReadAhead];
#pragma unroll
      for (int ks = 0; ks < kReadAhead; ++ks) ka[ks] = aload(ks);
      int key = copies ? copy_key(nxt, 0) : 0;
      const int entry = copies ? nxt.wrow[lane & 31] : 0;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks == 0)
          mfma32_first(sacc, ka[0], qf[0]);
        else
          mfma32_acc(sacc, ka[ks % kReadAhead], qf[ks]);
        if (ks + kReadAhead < kKSteps) ka[ks % kReadAhead] = aload(ks + kReadAhead);
        // copy k of the tile two ahead goes out with step C k + 1 (C =
        // kCopyStep), the key row of copy k + 1 is read right after, with
        // step C k + C - 1 (the same step when C = 2)
        if (ks % kCopyStep == 1 && ks / kCopyStep < kCopies && copies) copy_row(nxt, ks / kCopyStep, key);
        if (ks % kCopyStep == kCopyStep - 1 && ks / kCopyStep + 1 < kCopies && copies)
          key = copy_key(nxt, ks / kCopyStep + 1);
        if (ks == 6 && copies) vm_nxt = tile_mask(entry);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma32_drain(sacc);
    };

    // ---- softmax of the current tile in small phases, one per value step of
    // the previous tile, each a few independent instructions (the wave issues
    // in order, so a phase must not wait on its own results): two max chains,
    // the lane swap, the reference update, then a three-stage pipeline over
    // the 16 probabilities (scale and shift, exp2, sum and pack) ----
    float t0 = 0.f, t1 = 0.f, tm = 0.f, negm = 0.f, ps0 = 0.f, ps1 = 0.f;
    float xq[2] = {0.f, 0.f}, pq[2] = {0.f, 0.f};  // in-flight arguments / probabilities
    bool first = false;
    auto sm_phase = [&](int k) {
      if (k < 7) {  // max over the 16 logits, chains t0 (even phases) and t1 (odd)
        const int i = k < 2 ? 3 * k : 2 * k + 2;  // first register of this phase
        if (k == 0) t0 = max3_f32(sacc[0], sacc[1], sacc[2]);
        else if (k == 1) t1 = max3_f32(sacc[3], sacc[4], sacc[5]);
        else if (k & 1) t1 = max3_f32(t1, sacc[i], sacc[i + 1]);
        else t0 = max3_f32(t0, sacc[i], sacc[i + 1]);
      } else if (k == 7) {
        t0 = max3_f32(t0, t1, t1);
      } else if (k == 8) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t0), __float_as_uint(t0), false, false);
        t0 = max3_f32(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
      } else if (k == 9) {
        tm = t0 * scale2;  // -inf when the tile has no valid key
        first = m_ref == -__builtin_inff();
      } else if (k == 10) {
        m_seen = max3_f32(m_seen, tm, tm);
        if (first) m_ref = tm;  // O and l of this head are still 0
      } else if (k == 11) {
        overflow |= tm > m_ref + kRefSlack;
        negm = (m_ref == -__builtin_inff()) ? 0.f : -m_ref;
      } else if (k < 12 + 18) {  // j = k - 12: argument of j, exp2 of j - 1, sum of j - 2
        const int j = k - 12;
        if (j >= 2) {
          const int e = j - 2;
          if (e & 1) {
            ps1 = e == 1 ? pq[1] : ps1 + pq[1];
            pn[e >> 3][(e >> 1) & 3] = pack_bf16x2(pq[0], pq[1]);
          } else {
            ps0 = e == 0 ? pq[0] : ps0 + pq[0];
          }
        }
        // v_exp_f32 directly: arguments are <= kRefSlack, -inf gives 0
        if (j >= 1 && j <= 16) pq[(j - 1) & 1] = __builtin_amdgcn_exp2f(xq[(j - 1) & 1]);
        if (j < 16) xq[j & 1] = __builtin_fmaf(sacc[j], scale2, negm);
      } else {
        const float ps = ps0 + ps1;
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
        l_run += __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
    };
    constexpr int kSmPhases = 12 + 18 + 1;

    // ---- value product of the previous tile (in buffer `prv`), with the
    // softmax phases of the current tile when SM ----
    auto sm_pv = [&](auto sm_tag, auto pv_tag, lds_char_t* prv) {
      constexpr bool SM = decltype(sm_tag)::value;
      constexpr bool PV = decltype(pv_tag)::value;
      if constexpr (PV) {
        auto vload = [&](int st) {
          const int s = st >> 4, db = st & 15;
          const short4_t lo = lds_read_tr16(prv + vbase[0] + kLatStride * 16 * s + 64 * db);
          const short4_t hi = lds_read_tr16(prv + vbase[1] + kLatStride * 16 * s + 64 * db);
          return __builtin_bit_cast(
              bf16x8_t, short8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        };
        bf16x8_t va[kVAhead];
#pragma unroll
        for (int st = 0; st < kVAhead; ++st) va[st] = vload(st);
#pragma unroll
        for (int st = 0; st < kPvSteps; ++st) {
          const int s = st >> 4, db = st & 15;
          oacc[db] = mfma32x32x16_bf16(va[st % kVAhead], pb[s], oacc[db]);
          if (st + kVAhead < kPvSteps) va[st % kVAhead] = vload(st + kVAhead);
          if constexpr (SM)
            if (st < kSmPhases) sm_phase(st);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (SM)
#pragma unroll
          for (int k = kPvSteps; k < kSmPhases; ++k) sm_phase(k);
      } else {
#pragma unroll
        for (int k = 0; k < kSmPhases; ++k) sm_phase(k);
      }
    };
    using yes = std::true_type;
    using no = std::false_type;

    // wait for tile it, publish it, send out the copies of tile it + 2 and
    // compute its logits (skipped rows: -inf)
    auto front = [&](int it) {
      wait_tiles(min(1, ntiles - 1 - it));
      __syncthreads();  // every wave's copies of tile `it` are in; tile it-2 is consumed
      const bool copies = it + 2 < ntiles;
      TileCopies nxt;
      if (copies) {
        const int t = it + 2;
        if (t % kWinTiles == 0) {  // next index window (splits longer than one window)
          load_window(t / kWinTiles);
          store_window();
          __syncthreads();
        }
        nxt = prep_tile(t);
      }
      lds_char_t* cur = (lds_char_t*)(tiles[(it + 2) % kBuffers].bytes);
      const uint32_t vm = vm_a;  // tile it
      uint32_t vm_nxt = 0u;      // tile it + 2
      if (copies)
        logits(std::true_type{}, cur, nxt, vm_nxt);
      else
        logits(std::false_type{}, cur, nxt, vm_nxt);
      vm_a = vm_b;
      vm_b = vm_nxt;
      if (vm != 0xffffffffu) {  // skipped rows in this tile: their logits are -inf
        const uint32_t bits = (vm >> (4 * hl)) & 0x0f0f0f0fu;  // bit 8(i/4) + i%4: key of register i
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!((bits >> (8 * (i >> 2) + (i & 3))) & 1u)) sacc[i] = -__builtin_inff();
      }
    };
    if (ntiles > 0) {
      front(0);
      sm_pv(yes{}, no{}, nullptr);
      pb[0] = __builtin_bit_cast(bf16x8_t, pn[0]);
      pb[1] = __builtin_bit_cast(bf16x8_t, pn[1]);
    }
    for (int it = 1; it < ntiles; ++it) {
      front(it);
      sm_pv(yes{}, yes{}, (lds_char_t*)(tiles[(it + 1) % kBuffers].bytes));  // tile it - 1
      pb[0] = __builtin_bit_cast(bf16x8_t, pn[0]);
      pb[1] = __builtin_bit_cast(bf16x8_t, pn[1]);
    }
    // the last tile's value product
    if (ntiles > 0) sm_pv(no{}, yes{}, (lds_char_t*)(tiles[(ntiles + 1) % kBuffers].bytes));
    // every copy has landed (the ring is reused by a second pass)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!__syncthreads_or(pass == 0 && overflow)) break;
  }

  // ---- epilogue: normalise, stage [head][dims] in bf16 through the idle
  // ring (rows 1040 B apart), then store whole 1 KiB head rows: wave w reads
  // back only the rows it wrote, so no barrier separates the two ----
  constexpr int kStageStride = 1040;
  static_assert(kH * kStageStride <= kBuffers * kTileBytes, "output staging fits the ring");
  char* stage = reinterpret_cast<char*>(tiles[0].bytes);
  {
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    char* srow = stage + kStageStride * (32 * wave + m) + 8 * hl;
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x16_t& a = oacc[db];
        const u32x2_t v = {pack_bf16x2(a[4 * u] * inv_l, a[4 * u + 1] * inv_l),
                           pack_bf16x2(a[4 * u + 2] * inv_l, a[4 * u + 3] * inv_l)};
        *reinterpret_cast<u32x2_t*>(srow + 64 * db + 16 * u) = v;
      }
    uint16_t* dst = (nsplit == 1 ? o + row * kH * kDc : part_o + (row * nsplit + sp) * kH * kDc) + head0 * kDc;
#pragma unroll 4
    for (int k = 0; k < 32; ++k) {
      const int hh = 32 * wave + k;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + kStageStride * hh + 16 * lane);
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(dst + hh * kDc) + 16 * lane) = v;
    }
  }
  if (hl == 0) {
    const int h = head0 + 32 * wave + m;
    const float v = l_run > 0.f ? (m_ref + __log2f(l_run)) * kLn2 : -__builtin_inff();
    if (nsplit > 1)
      part_lse[(row * kH + h) * nsplit + sp] = v;
    else if (lse != nullptr)
      lse[row * kH + h] = v;
  }
}

// Merge of the split partials: one wave per (query row, head), lane l covers
// latent dims 8l .. 8l+7 (Dc = 512).  lse = log sum_s exp(lse_s);
// o = sum_s exp(lse_s - lse) o_s.  Fixed split order, no atomics:
// deterministic.  NS (the split count, a template argument for the counts the
// planner uses) unrolls everything: the NS partial loads and the wave's NS
// contiguous lse values (scalar loads) are all issued before the first wait.
// Every split's partial is written (an empty split holds zeros with weight 0).
// With xcd_map (rows a multiple of 8), workgroup L merges heads of row
// 8 (L / 256) + L % 8: the XCD that wrote the row's partials (mla_mfma's
// xcd_map) also merges them.
template <int NS>
__global__ void __launch_bounds__(256)
mla_combine(int nsplit_rt, int xcd_map, int64_t total_heads, const uint16_t* __restrict__ part_o,
            const float* __restrict__ part_lse, uint16_t* __restrict__ o, float* __restrict__ lse) {
  const int64_t L = blockIdx.x;
  const int64_t hq = xcd_map ? (L >> 8) * 256 + (L & 7) * 32 + ((L >> 3) & 31) : L;  // 4-head group
  const int64_t rh = __builtin_amdgcn_readfirstlane(hq * 4 + (threadIdx.x >> 6));  // row * H + head
  if (rh >= total_heads) return;
  const int nsplit = NS > 0 ? NS : nsplit_rt;
  const int lane = threadIdx.x & 63;
  const int64_t row = rh / kH;
  const int h = static_cast<int>(rh - row * kH);
  const float* ls = part_lse + rh * nsplit;
  const uint16_t* po = part_o + (row * nsplit * kH + h) * kDc + 8 * lane;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f, m_use = 0.f;
  auto add = [&](float wgt, const u32x4_t& pv) {
    wsum += wgt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(wgt, __uint_as_float(pv[e] << 16), acc[2 * e]);
      acc[2 * e + 1] = fmaf(wgt, __uint_as_float(pv[e] & 0xffff0000u), acc[2 * e + 1]);
    }
  };
  if constexpr (NS > 0) {
    u32x4_t pv[NS];
    float lv[NS];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) pv[sp] = *reinterpret_cast<const u32x4_t*>(po + static_cast<int64_t>(sp) * kH * kDc);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) lv[sp] = ls[sp];
    float m = -__builtin_inff();
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) m = fmaxf(m, lv[sp]);
    m_use = m == -__builtin_inff() ? 0.f : m;
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) add(__expf(lv[sp] - m_use), pv[sp]);  // exp(-inf) = 0
  } else {
    float m = -__builtin_inff();
    for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, ls[sp]);
    m_use = m == -__builtin_inff() ? 0.f : m;
    for (int sp = 0; sp < nsplit; ++sp)
      add(__expf(ls[sp] - m_use), *reinterpret_cast<const u32x4_t*>(po + static_cast<int64_t>(sp) * kH * kDc));
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const u32x4_t ov = {f32x2_to_bf16x2(acc[0] * inv, acc[1] * inv), f32x2_to_bf16x2(acc[2] * inv, acc[3] * inv),
                      f32x2_to_bf16x2(acc[4] * inv, acc[5] * inv), f32x2_to_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4_t*>(o + rh * kDc + 8 * lane) = ov;
  if (lse != nullptr && lane == 0) lse[rh] = wsum > 0.f ? m_use + __logf(wsum) : -__builtin_inff();
}

struct MlaPlan {
  bool mfma;
  int splits;
  int kps;  // index entries per split (multiple of the tile)
  int nw;   // waves per workgroup: 4 (128 heads) or 2 (64 heads, two workgroups per split)
};

MlaPlan plan(const dsa_shape_t& s) {
  MlaPlan p{false, 1, k_eff(s), 4};
  if (!(s.H == kH && s.Dc == kDc && s.Dr == kDr && s.mla_dtype == DSA_BF16)) return p;
  p.mfma = true;
  const int W = k_eff(s);
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  const int cus = device_info().cu_count;
  // one workgroup per CU: split until every CU has a workgroup, but keep at
  // least 4 tiles per split
  int splits = 1;
  while (rows * splits < cus && W / (splits * 2) >= 4 * kTileKeys) splits *= 2;
  int kps = (W + splits - 1) / splits;
  kps = (kps + kTileKeys - 1) / kTileKeys * kTileKeys;
  splits = (W + kps - 1) / kps;
  p.splits = splits < 1 ? 1 : splits;
  p.kps = kps;
  // still fewer workgroups than CUs: split the heads as well, two workgroups
  // of 64 heads per split, placed on one XCD (each gathers the same rows)
  if (rows * p.splits * 2 <= cus) p.nw = 2;
  return p;
}

}  // namespace

size_t mla_workspace_bytes(const dsa_shape_t& s) {
  const MlaPlan p = plan(s);
  if (!p.mfma || p.splits == 1) return 0;
  const size_t rows = static_cast<size_t>(s.B) * s.T;
  const size_t po = rows * p.splits * s.H * static_cast<size_t>(s.Dc) * sizeof(uint16_t);
  return (po + 255) / 256 * 256 + rows * p.splits * s.H * sizeof(float);
}

dsa_status_t mla_check(const dsa_shape_t& s) {
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  if (rows > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: B*T = %lld exceeds 65535 rows",
                static_cast<long long>(rows));
  if (plan(s).mfma) {
    if (static_cast<int64_t>(s.S) * kD * 2 > 0xffffffffLL)
      return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: S = %d key rows exceed 4 GiB per sequence", s.S);
  } else if ((static_cast<size_t>(s.Dc) + s.Dr + k_eff(s)) * sizeof(float) > 64 * 1024) {
    return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: D + K = %d too large for the generic kernel",
                s.Dc + s.Dr + k_eff(s));
  }
  return DSA_OK;
}

dsa_status_t launch_sparse_mla(const dsa_shape_t& s, const void* q, const void* kv,
                               const int32_t* idx, void* o, float* lse, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  {
    const dsa_status_t st = mla_check(s);
    if (st != DSA_OK) return st;
  }
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  const int W = k_eff(s);
#ifdef DSA_DEBUG
  {
    const dsa_status_t st = debug_check_idx(rows, W, s.S, false, idx, stream, "attention index rows");
    if (st != DSA_OK) return st;
  }
#endif
  const MlaPlan p = plan(s);
  if (p.mfma) {
    uint16_t* part_o = nullptr;
    float* part_lse = nullptr;
    if (p.splits > 1) {
      const size_t need = mla_workspace_bytes(s);
      if (ws == nullptr || ws_bytes < need)
        return fail(DSA_ERR_WORKSPACE, "sparse_mla: workspace of %zu bytes needed, %zu given",
                    need, ws_bytes);
      part_o = static_cast<uint16_t*>(ws);
      const size_t po = static_cast<size_t>(rows) * p.splits * s.H * s.Dc * sizeof(uint16_t);
      part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + (po + 255) / 256 * 256);
    }
    const int xcd_map = (p.splits > 1 && rows % 8 == 0) ? 1 : 0;
    const unsigned wgs = static_cast<unsigned>(rows * p.splits * (4 / p.nw));
    LaunchTimer timer;
    auto attend = [&](auto kernel) {
      hipExtLaunchKernelGGL(kernel, dim3(wgs), dim3(p.nw * 64), 0, stream, timer.start(), timer.stop(), 0,
                            s.T, s.S, W, p.kps, p.splits, xcd_map, s.sm_scale,
                            static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,
                            static_cast<uint16_t*>(o), lse, part_o, part_lse);
    };
    if (p.nw == 2)
      attend(mla_mfma<2>);
    else
      attend(mla_mfma<4>);
    dsa_status_t st = timer.done("mla_mfma");
    if (st != DSA_OK || p.splits == 1) return st;
    const int64_t total_heads = rows * kH;
    LaunchTimer ctimer;
    const dim3 cgrid(static_cast<unsigned>((total_heads + 3) / 4));
    auto combine = [&](auto kernel) {
      hipExtLaunchKernelGGL(kernel, cgrid, dim3(256), 0, stream, ctimer.start(), ctimer.stop(), 0,
                            p.splits, xcd_map, total_heads, static_cast<const uint16_t*>(part_o),
                            static_cast<const float*>(part_lse), static_cast<uint16_t*>(o), lse);
    };
    switch (p.splits) {
      case 2: combine(mla_combine<2>); break;
      case 4: combine(mla_combine<4>); break;
      case 8: combine(mla_combine<8>); break;
      case 16: combine(mla_combine<16>); break;
      default: combine(mla_combine<0>); break;
    }
    return ctimer.done("mla_combine");
  }
  const size_t lds = (static_cast<size_t>(s.Dc) + s.Dr + W) * sizeof(float);
  LaunchTimer timer;
  const dim3 grid(s.H, static_cast<unsigned>(rows));
  if (s.mla_dtype == DSA_BF16)
    hipExtLaunchKernelGGL(mla_generic<DSA_BF16>, grid, dim3(256), lds, stream, timer.start(),
                          timer.stop(), 0, s.T, s.S, s.H, s.Dc, s.Dr, W, s.sm_scale, q, kv, idx, o, lse);
  else
    hipExtLaunchKernelGGL(mla_generic<DSA_F32>, grid, dim3(256), lds, stream, timer.start(),
                          timer.stop(), 0, s.T, s.S, s.H, s.Dc, s.Dr, W, s.sm_scale, q, kv, idx, o, lse);
  return timer.done("mla_generic");
}

}  // namespace dsa
