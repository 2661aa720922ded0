// Sparse latent attention in absorbed form on gfx950.
//
// For each query row (b, t) and head h, over the keys j listed in idx[b,t,:]
// (entries -1 or outside [0, S) skipped, duplicates counted as written):
//   logit_j = sm_scale * (q[h, 0:Dc] . c_j + q[h, Dc:Dc+Dr] . r_j),  kv_j = [c_j ; r_j]
//   o[h, :] = sum_j softmax(logit)_j c_j,   lse[h] = log sum_j exp(logit_j)
// (atlas.klimoza.dev, DeepSeek-V3.2-Exp MoE block, "All 43 steps": keys
// [K^C ; k^R] with one rotary key shared by all heads, values c W_UV; taken in
// absorbed form, q_lat = W_UK q^C, so every head reads the same 576-wide
// row.  nnterp deepseek_v32, sections 03/04: zero probability outside the
// selection, each row sums to one over it.)
//
// Kernels:
//  * mla_mfma (H = 128, Dc = 512, Dr = 64, bf16): one workgroup of 8 waves
//    takes one query row and one split of its index list.  All 128 heads share
//    each gathered key tile: 32 selected rows are copied straight from global
//    memory into LDS (row-major, swizzled) and read twice, directly for the
//    logits and through transposing LDS reads for the value product.  Wave w
//    owns heads 16w..16w+15: logits^T = K_tile . Q^T on MFMA (keys on M,
//    heads on N), an online softmax in fp32 with exp2, and O^T += V^T . P^T on
//    MFMA (latent dims on M, heads on N) with P^T taken straight from the
//    logit accumulators.  A ring of 3 LDS tiles keeps the next tile's copies
//    in flight during the current tile's MFMAs.
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
// row and one split of its index list; wave w owns heads 32w .. 32w+31 as two
// groups of 16 (group c: heads 32w + 16c .. +15).  All 128 heads share each
// gathered tile of 32 selected key rows, and every operand a wave reads from
// LDS feeds two MFMAs, one per group.
//
// MFMA 16x16x32 bf16 operand layouts (lane l, g = l / 16, n = l % 16):
//   A (16 x 32): lane holds row n, reduction elements 8g .. 8g+7
//   B (32 x 16): lane holds column n, reduction elements 8g .. 8g+7
//   C (16 x 16): register i holds row 4g + i of column n
//
// logits^T (2 blocks of 16 keys x 16 heads, per group) = K_tile (A, from LDS)
// . Q^T (B, registers), reduced over the 576 dims in 18 steps of 32: four
// independent accumulation chains.  Lane (g, n) ends with head n of each
// group and keys 4g + i and 16 + 4g + i.
//
// O^T (512 dims x 16 heads, per group) += V^T (A) . P^T (B), reduced over the
// 32 keys in one MFMA per 16 dims.  P^T comes straight from the logit
// accumulators: its B-operand slot 8g + e holds key 4g + e (e < 4) or
// 16 + 4g + e - 4 (e >= 4).  V^T is read from the same row-major key tile with
// the transposing LDS load ds_read_b64_tr_b16: within a 16-lane group, lane i
// receives element (i % 4) of the 8-byte chunk loaded by lane 4j + i/4, for
// j = 0..3.  So lane 4j + c of group g loads dims 16db + 4c .. +3 of tile row
// 4g + j (+16 for the second half of its slots), and lane i ends up with 4 key
// slots of dim 16db + i: half of its A operand.
//
// Key tile in LDS (38 KiB): latent part of row r (64 pieces of 16 B) at byte
// 1088 r, piece c stored at c ^ f(r), f(r) = 2 ((r >> 2) & 1); rotary part (8
// pieces) in a region of its own at byte 34816, row r at 128 r, piece c' at
// c' ^ ((r >> 1) & 7).  The LDS has 64 banks of 4 bytes.  A 16-byte read takes
// 4 cycles, each serving two groups of 8 lanes: lanes 0-7 with 24-31, 8-15
// with 16-23, 32-39 with 56-63 and 40-47 with 48-55 (measured with the bank
// conflict counter on gfx950); a transposing 8-byte read serves 32 lanes per
// cycle.  With this placement the logits reads, the transposing reads and the
// epilogue staging touch every bank once per cycle, and every read is one
// base register plus a compile-time offset.
//
// The tile is filled by direct global->LDS copies (global_load_lds_dwordx4:
// lane l of a wave writes 16 B at the wave's LDS base + 16 l): wave w copies
// the latent parts of rows 8w .. 8w+7 (one 1 KiB run of global memory each)
// and the rotary parts of the same rows.  A ring of 4 tiles keeps up to three
// later tiles' copies in flight during the current tile's MFMAs.
// ---------------------------------------------------------------------------
constexpr int kH = 128, kDc = 512, kDr = 64, kD = kDc + kDr;
constexpr int kMlaWaves = 4;                 // wave w owns heads 32w .. 32w+31
constexpr int kMlaThreads = kMlaWaves * 64;
constexpr int kTileKeys = 32;
constexpr int kBuffers = 4;                  // LDS tile ring
constexpr int kCopiesPerTile = 9;            // copies per wave per tile: 8 latent rows + rotary parts
constexpr int kLatStride = 1088;             // bytes per latent row in LDS (1024 + 64 pad)
constexpr int kRopeBase = kTileKeys * kLatStride;            // byte offset of the rotary region
constexpr int kTileBytes = kRopeBase + kTileKeys * kDr * 2;  // 38912
constexpr int kKSteps = kD / 32;             // 18 logits reduction steps
constexpr int kLatSteps = kDc / 32;          // 16 of them over the latent part
constexpr int kReadAhead = 6;                // logits A-operand reads issued ahead of their MFMAs
constexpr int kVAhead = 4;                   // value A operands (2 reads each) issued ahead
constexpr float kRefSlack = 32.0f;           // log2 units: p <= 2^32 against the reference max
constexpr int kStageStride = 528;            // epilogue staging row: 256 bf16 + 16 B pad
constexpr int kIdxWin = 1024;                // index entries staged in LDS at a time
constexpr int kWinTiles = kIdxWin / kTileKeys;
constexpr int kWinPerThread = kIdxWin / kMlaThreads;
constexpr int kQStageBytes = 16 * kD * 2;    // one wave's query rows of one group, staged in the ring
static_assert(kMlaWaves * kQStageBytes <= 2 * kTileBytes, "query staging fits ring buffers 0-1");

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) const char lds_char_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// a zero key row: skipped index entries load it, so their LDS rows are zero
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[kD];

struct MlaTile {
  uint8_t bytes[kTileBytes];
};


__device__ __forceinline__ int lat_swz(int r) { return ((r >> 2) & 1) << 1; }  // f(r)
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

// Slot of 16-byte piece p (0..71) within a staged query row of head hq
// (0..15): the latent pieces are XOR-swizzled within aligned groups of 16 by
// hq >> 1, the rotary pieces within their group of 8 likewise (an involution,
// so the same function maps slots back to pieces).  The operand reads (lane
// (g, n): head n, piece 4ks + g; rows 1152 B = 32 banks apart) then touch
// every bank once per cycle of the 16-byte read.
__device__ __forceinline__ int qpiece_slot(int p, int hq) {
  return p < 64 ? ((p & ~15) | ((p ^ (hq >> 1)) & 15)) : (64 | ((p - 64) ^ ((hq >> 1) & 7)));
}

// Address arithmetic on LDS pointers stays in the 32-bit LDS address space, so
// constant offsets fold into the instructions' offset fields.
__device__ __forceinline__ short4_t lds_read_tr16(lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
}

// 1-D grid of rows * nsplit workgroups.  With xcd_map, the splits of one query
// row share an XCD (workgroups are dealt to the 8 XCDs round-robin), so its
// 147 KB query block is fetched once into that XCD's L2.
// nsplit == 1: writes o (bf16) and lse directly; otherwise writes bf16
// partials part_o [rows, nsplit, H, Dc] (already divided by the split's own
// sum) and part_lse [rows, H, nsplit] (natural log; -inf for an empty split).
__global__ void __launch_bounds__(kMlaThreads, 1)
mla_mfma(int T, int S, int W, int kps, int nsplit, int xcd_map, float sm_scale,
         const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
         const int32_t* __restrict__ idx, uint16_t* __restrict__ o, float* __restrict__ lse,
         uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(1024))) MlaTile tiles[kBuffers];
  // a window of the split's index entries as key rows (-1: skipped entry)
  __shared__ __attribute__((aligned(16))) int32_t idxw[kIdxWin];
  // validity of each tile's rows (bit r: tile row r holds a valid key), written
  // when the tile's copies are issued, kBuffers - 1 iterations before its use
  __shared__ uint32_t vmask[kBuffers + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int L = blockIdx.x;
  int sp;
  int64_t row;
  if (xcd_map) {
    sp = (L >> 3) % nsplit;
    row = static_cast<int64_t>(L / (8 * nsplit)) * 8 + (L & 7);
  } else {
    sp = L % nsplit;
    row = L / nsplit;
  }
  const int b = static_cast<int>(row / T);
  const int j0 = sp * kps;
  const int nj = max(0, min(W, j0 + kps) - j0);
  const int ntiles = (nj + kTileKeys - 1) / kTileKeys;
  const uint16_t* kv_seq = kv + static_cast<int64_t>(b) * S * kD;

  // The split's index entries go through LDS a window at a time: thread i
  // loads entries i, i + 256, ... of the window (past the split's end: -1).
  const int32_t* idx_row = idx + row * W;
  const int j_end = j0 + nj;
  int win[kWinPerThread];
  auto load_window = [&](int w) {
#pragma unroll
    for (int u = 0; u < kWinPerThread; ++u) {
      const int j = j0 + w * kIdxWin + tid + u * kMlaThreads;
      win[u] = j < j_end ? idx_row[j] : -1;
    }
  };
  auto store_window = [&]() {
#pragma unroll
    for (int u = 0; u < kWinPerThread; ++u)
      idxw[tid + u * kMlaThreads] = (win[u] >= 0 && win[u] < S) ? win[u] : -1;
  };

  // Query operand (B of logits^T): qf[c][ks] = head 32w + 16c + n, dims
  // 32ks + 8g .. +8.  Wave w's 16 heads of group c are one contiguous 18 KiB
  // run of q; each group goes through ring buffers 0-1 with whole-line copies,
  // placed so that the operand reads are free of bank conflicts: head hq
  // (0..15) at byte 1152 hq, its 16-byte piece p at slot qpiece_slot(p, hq).
  // Meanwhile tiles 0 and 1 land in buffers 2 and 3 (tile t uses ring buffer
  // (t + 2) % 4).
  bf16x8_t qf[2][kKSteps];
  load_window(0);
  store_window();
  __syncthreads();  // the first index window is published
  const char* qsrc = reinterpret_cast<const char*>(q + (row * kH + 32 * wave) * kD);
  auto stage_q = [&](int c) {
    const uint32_t qlds = lds_addr(tiles) + wave * kQStageBytes;
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
#pragma unroll 2
    for (int i = 0; i < kQStageBytes / 1024; ++i) {
      const int x = 1024 * i + 16 * ln;  // staging byte this lane's copy lands on
      const int hq = x / (kD * 2), slot = (x - hq * kD * 2) >> 4;
      lds_dma_16(qsrc + (16 * c + hq) * (kD * 2) + 16 * qpiece_slot(slot, hq), qlds + 1024 * i);
    }
  };
  auto read_q = [&](int c) {
    lds_char_t* qst = (lds_char_t*)(tiles[0].bytes) + wave * kQStageBytes;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qf[c][ks] = *(__attribute__((address_space(3))) const bf16x8_t*)(
          qst + n * (kD * 2) + 16 * qpiece_slot(4 * ks + g, n));
  };
  f32x4_t oacc[2][kDc / 16];  // O^T: oacc[c][db][i] = O[head 32w + 16c + n][16db + 4g + i]
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int db = 0; db < kDc / 16; ++db) oacc[c][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-__builtin_inff(), -__builtin_inff()};  // reference max (log2 units) per group
  float l_run[2] = {0.f, 0.f};
  const float scale2 = sm_scale * kLog2e;

  // Wave w copies tile rows 8w .. 8w+7 (latent and rotary parts), reading
  // their key rows from the index window; wave 0 also publishes the tile's
  // validity mask.
  // Byte offset, from the sequence's first key row, of the zero row that
  // skipped entries copy: one select per copy instead of a branch.
  const int64_t zero_off = reinterpret_cast<const char*>(g_zero_row) - reinterpret_cast<const char*>(kv_seq);
  // A tile's copies: prep_tile reads the wave's 8 key rows from the index
  // window (two broadcast reads, one LDS round trip) and publishes the tile's
  // validity mask (wave 0); copy_row(k) then issues copy k of 9 (8 latent
  // rows, then the rotary parts).  Each lane forms its own source address, so
  // no value goes through SGPRs.  The main loop spreads the nine copies over
  // the logits MFMAs, so their issue cost hides under matrix work.
  struct TileCopies {
    int sl[8];  // key rows of tile rows 8w .. 8w+7 (-1: skipped)
    int sr;     // key row of tile row 8w + lane/8 (rotary copy)
    uint32_t lds;
  };
  auto prep_tile = [&](int t) {
    TileCopies c;
    const int32_t* wrow = &idxw[(t % kWinTiles) * kTileKeys];
    const int ln = __lane_id();
    if (wave == 0) {
      const uint32_t m = static_cast<uint32_t>(__ballot(wrow[ln & 31] >= 0));
      if (ln == 0) vmask[t % (kBuffers + 1)] = m;
    }
    const int4 s4a = *reinterpret_cast<const int4*>(wrow + 8 * wave);
    const int4 s4b = *reinterpret_cast<const int4*>(wrow + 8 * wave + 4);
    c.sl[0] = s4a.x; c.sl[1] = s4a.y; c.sl[2] = s4a.z; c.sl[3] = s4a.w;
    c.sl[4] = s4b.x; c.sl[5] = s4b.y; c.sl[6] = s4b.z; c.sl[7] = s4b.w;
    c.sr = wrow[8 * wave + (ln >> 3)];
    c.lds = lds_addr(tiles[(t + 2) % kBuffers].bytes);
    return c;
  };
  const char* kvb = reinterpret_cast<const char*>(kv_seq);
  auto copy_row = [&](const TileCopies& c, int k) {
    // an opaque copy of the lane id: the per-copy address math is redone at
    // each copy instead of being kept live across the loop in registers
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
    if (k < 8) {  // latent part of row r: its 16-byte slot `ln` holds piece ln ^ f(r)
      const int r = 8 * wave + k;
      const int64_t off = c.sl[k] >= 0 ? static_cast<int64_t>(c.sl[k]) * (kD * 2) : zero_off;
      lds_dma_16(kvb + off + 16 * (ln ^ lat_swz(r)), c.lds + kLatStride * r);
    } else {  // rotary parts of rows 8w .. 8w+7: lane l takes row 8w + l/8
      const int r = 8 * wave + (ln >> 3);
      const int64_t off = c.sr >= 0 ? static_cast<int64_t>(c.sr) * (kD * 2) : zero_off;
      lds_dma_16(kvb + off + 2 * kDc + 16 * ((ln & 7) ^ rope_swz(r)), c.lds + kRopeBase + 1024 * wave);
    }
  };
  auto issue_tile = [&](int t) {
    const TileCopies c = prep_tile(t);
#pragma unroll
    for (int k = 0; k < kCopiesPerTile; ++k) copy_row(c, k);
  };
  // wait until at most `pending` later tiles' copies of this wave are in flight
  auto wait_tiles = [&](int pending) {
    static_assert(kBuffers == 4 && kCopiesPerTile == 9, "vmcnt immediates");
    if (pending <= 0)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (pending == 1)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  };

  // LDS byte offsets.  Logits A operand of step ks for key block mb: row
  // 16mb + n, piece 4ks + g, stored at 4ks + (g ^ f(row)) (latent steps) or in
  // the rotary region (steps 16, 17).
  int aoff[2], roff[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int r = 16 * mb + n;
    aoff[mb] = kLatStride * r + 16 * (g ^ lat_swz(r));
#pragma unroll
    for (int kr = 0; kr < 2; ++kr) roff[mb][kr] = kRopeBase + 128 * r + 16 * ((4 * kr + g) ^ rope_swz(r));
  }
  // Transposing reads: lane (g, jq, cq) reads tile row 4g + jq + 16h, dims
  // 16db + 4cq: piece 2db + cq/2, byte 8(cq&1).  (2db + y) ^ f = 4(db/2) + ((2(db&1) + y) ^ f),
  // so each (h, db parity) has one base and db/2 moves it by 64 bytes.
  const int jq = n >> 2, cq = n & 3;
  int voff[2][2];  // [h][db parity]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 4 * g + jq + 16 * h;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      voff[h][par] = kLatStride * r + 16 * ((2 * par + (cq >> 1)) ^ lat_swz(r)) + 8 * (cq & 1);
  }

  // start-up: the query in two halves, tiles 0 and 1 meanwhile
  stage_q(0);
  for (int t = 0; t < 2 && t < ntiles; ++t) issue_tile(t);
  // loads complete in issue order: wait for the query half, not the tiles
  if (ntiles >= 2)
    asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  else if (ntiles == 1)
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  read_q(0);
  __syncthreads();  // every wave has read its first half: the staging is free
  stage_q(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  read_q(1);
  __syncthreads();  // buffers 0-1 are free again; tiles 0 and 1 are in

  // Online softmax with a fixed reference max per head: the first tile with a
  // valid key sets it, and p = 2^(x - ref) stays below 2^kRefSlack as long as
  // no later logit exceeds the reference by more than the slack.  If one does
  // (never for sane data), the whole split is run once more with the true
  // maximum as reference, so O is only ever zeroed, never rescaled.  The
  // decision is workgroup-uniform (barriers stay matched).
  float m_seen[2] = {-__builtin_inff(), -__builtin_inff()};
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int db = 0; db < kDc / 16; ++db) oacc[c][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        l_run[c] = 0.f;
        m_ref[c] = m_seen[c];
      }
    }
    bool overflow = false;
    if (pass == 1 && ntiles > kWinTiles) {  // the window moved on: back to the first
      load_window(0);
      store_window();
      __syncthreads();
    }
    for (int t = pass == 0 ? 2 : 0; t < kBuffers - 1 && t < ntiles; ++t) issue_tile(t);
    for (int it = 0; it < ntiles; ++it) {
      wait_tiles(min(kBuffers - 2, ntiles - 1 - it));
      __syncthreads();  // every wave's copies of tile `it` are in; tile it-1 is consumed
      const bool copies = it + kBuffers - 1 < ntiles;
      TileCopies nxt;
      if (copies) {
        const int t = it + kBuffers - 1;
        if (t % kWinTiles == 0) {  // next index window (splits longer than kIdxWin)
          load_window(t / kWinTiles);
          store_window();
          __syncthreads();
        }
        nxt = prep_tile(t);
      }
      lds_char_t* cur = (lds_char_t*)(tiles[(it + 2) % kBuffers].bytes);
      // validity of rows 4g + i (block 0) and 16 + 4g + i (block 1)
      const uint32_t valid = vmask[it % (kBuffers + 1)] >> (4 * g);

      // ---- logits^T: 2 key blocks x 2 head groups, four chains ----
      f32x4_t sacc[2][2];  // [mb][c]
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int c = 0; c < 2; ++c) sacc[mb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      {
        // software pipeline over the 36 (ks, mb) key-tile reads: the read of
        // step st + kReadAhead is issued with the two MFMAs of step st
        constexpr int kSteps = 2 * kKSteps;
        auto aload = [&](int st) {
          const int ks = st >> 1, mb = st & 1;
          const int off = ks < kLatSteps ? aoff[mb] + 64 * ks : roff[mb][ks - kLatSteps];
          return *(__attribute__((address_space(3))) const bf16x8_t*)(cur + off);
        };
        bf16x8_t ka[kReadAhead];
#pragma unroll
        for (int st = 0; st < kReadAhead; ++st) ka[st] = aload(st);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          const int ks = st >> 1, mb = st & 1;
          sacc[mb][0] = mfma16x16x32_bf16(ka[st % kReadAhead], qf[0][ks], sacc[mb][0]);
          sacc[mb][1] = mfma16x16x32_bf16(ka[st % kReadAhead], qf[1][ks], sacc[mb][1]);
          if (st + kReadAhead < kSteps) ka[st % kReadAhead] = aload(st + kReadAhead);
          // copy k of the tile kBuffers - 1 ahead goes out with step 4k + 1
          if (st % 4 == 1 && st / 4 < kCopiesPerTile && copies) copy_row(nxt, st / 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax weights (lane: head n of each group; keys 16mb + 4g + i) ----
      bf16x8_t pb[2];  // B operands of the value product: slot 8g + e
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float x[2][4];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[mb][i] = ((valid >> (16 * mb + i)) & 1) ? sacc[mb][c][i] * scale2 : -__builtin_inff();
            tmax = fmaxf(tmax, x[mb][i]);
          }
        tmax = xor16_max(tmax);
        tmax = xor32_max(tmax);
        m_seen[c] = fmaxf(m_seen[c], tmax);
        if (m_ref[c] == -__builtin_inff()) m_ref[c] = tmax;  // O and l of this head are still 0
        overflow |= tmax > m_ref[c] + kRefSlack;
        const float m_use = (m_ref[c] == -__builtin_inff()) ? 0.f : m_ref[c];
        float psum = 0.f;
        u32x4_t pw;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // v_exp_f32 directly: arguments are <= kRefSlack, -inf gives 0
          const float p0 = __builtin_amdgcn_exp2f(x[e >> 2][e & 3] - m_use);
          const float p1 = __builtin_amdgcn_exp2f(x[e >> 2][(e & 3) + 1] - m_use);
          psum += p0 + p1;
          pw[e >> 1] = f32x2_to_bf16x2(p0, p1);
        }
        pb[c] = __builtin_bit_cast(bf16x8_t, pw);
        psum = xor16_sum(psum);
        psum = xor32_sum(psum);
        l_run[c] += psum;
      }

      // ---- O^T += V^T . P^T, both groups per V^T operand ----
      {
        // ds_read_b64_tr_b16 takes no folded offset: an opaque per-tile copy of
        // the bases keeps each read's address add next to the read
        int vbase[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            vbase[h][par] = voff[h][par];
            asm volatile("" : "+v"(vbase[h][par]));
          }
        auto vload = [&](int db) {
          const short4_t lo = lds_read_tr16(cur + vbase[0][db & 1] + 64 * (db >> 1));
          const short4_t hi = lds_read_tr16(cur + vbase[1][db & 1] + 64 * (db >> 1));
          return __builtin_bit_cast(
              bf16x8_t, short8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        };
        bf16x8_t va[kVAhead];
#pragma unroll
        for (int db = 0; db < kVAhead; ++db) va[db] = vload(db);
#pragma unroll
        for (int db = 0; db < kDc / 16; ++db) {
          oacc[0][db] = mfma16x16x32_bf16(va[db % kVAhead], pb[0], oacc[0][db]);
          oacc[1][db] = mfma16x16x32_bf16(va[db % kVAhead], pb[1], oacc[1][db]);
          if (db + kVAhead < kDc / 16) va[db % kVAhead] = vload(db + kVAhead);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // every copy has landed (the ring is reused by a second pass)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!__syncthreads_or(pass == 0 && overflow)) break;
  }

  // ---- epilogue: normalise, stage [head][dims] through LDS, coalesced stores ----
  uint16_t* dst = nsplit == 1 ? o + row * kH * kDc : part_o + (row * nsplit + sp) * kH * kDc;
  char* stage = reinterpret_cast<char*>(tiles[0].bytes);  // 128 rows x 528 B (the ring is idle)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // the ring / the previous half of the staging is free
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float inv_l = l_run[c] > 0.f ? 1.f / l_run[c] : 0.f;
      const int h = 32 * wave + 16 * c + n;
#pragma unroll
      for (int dq = 0; dq < kDc / 32; ++dq) {
        const f32x4_t& a = oacc[c][16 * half + dq];
        const u32x2_t v = {f32x2_to_bf16x2(a[0] * inv_l, a[1] * inv_l),
                           f32x2_to_bf16x2(a[2] * inv_l, a[3] * inv_l)};
        *reinterpret_cast<u32x2_t*>(stage + kStageStride * h + 2 * (16 * dq + 4 * g)) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < (kH * kDc / 2 * 2) / (16 * kMlaThreads); ++k) {  // 16 x 16 B per thread
      const int cidx = tid + kMlaThreads * k;  // 16-byte chunk: head cidx / 32, part cidx % 32
      const int hh = cidx >> 5, part = cidx & 31;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + kStageStride * hh + 16 * part);
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(dst + hh * kDc) + 512 * half + 16 * part) = v;
    }
  }
  if (g == 0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int h = 32 * wave + 16 * c + n;
      const float v = l_run[c] > 0.f ? (m_ref[c] + __log2f(l_run[c])) * kLn2 : -__builtin_inff();
      if (nsplit > 1)
        part_lse[(row * kH + h) * nsplit + sp] = v;
      else if (lse != nullptr)
        lse[row * kH + h] = v;
    }
  }
}

// Merge of the split partials: one wave per (query row, head), lane l covers
// latent dims 8l .. 8l+7 (Dc = 512).  lse = log sum_s exp(lse_s);
// o = sum_s exp(lse_s - lse) o_s.  Fixed split order, no atomics:
// deterministic.  The wave's split lse values are one contiguous run, read
// through the scalar cache.
__global__ void __launch_bounds__(256)
mla_combine(int nsplit, int64_t total_heads, const uint16_t* __restrict__ part_o,
            const float* __restrict__ part_lse, uint16_t* __restrict__ o, float* __restrict__ lse) {
  const int64_t rh = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));  // row * H + head
  if (rh >= total_heads) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = rh / kH;
  const int h = static_cast<int>(rh - row * kH);
  const float* ls = part_lse + rh * nsplit;
  float m = -__builtin_inff();
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, ls[sp]);
  const float m_use = m == -__builtin_inff() ? 0.f : m;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  const uint16_t* po = part_o + (row * nsplit * kH + h) * kDc + 8 * lane;
  // every split's partial is written (an empty split holds zeros with weight
  // 0), so all loads are issued unconditionally
#pragma unroll 8
  for (int sp = 0; sp < nsplit; ++sp) {
    const float wgt = __expf(ls[sp] - m_use);  // exp(-inf) = 0
    const u32x4_t pv = *reinterpret_cast<const u32x4_t*>(po + static_cast<int64_t>(sp) * kH * kDc);
    wsum += wgt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(wgt, __uint_as_float(pv[e] << 16), acc[2 * e]);
      acc[2 * e + 1] = fmaf(wgt, __uint_as_float(pv[e] & 0xffff0000u), acc[2 * e + 1]);
    }
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
};

MlaPlan plan(const dsa_shape_t& s) {
  MlaPlan p{false, 1, k_eff(s)};
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

dsa_status_t launch_sparse_mla(const dsa_shape_t& s, const void* q, const void* kv,
                               const int32_t* idx, void* o, float* lse, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(s.B) * s.T;
  if (rows > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: B*T = %lld exceeds 65535 rows",
                static_cast<long long>(rows));
  const int W = k_eff(s);
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
    LaunchTimer timer;
    hipExtLaunchKernelGGL(mla_mfma, dim3(static_cast<unsigned>(rows * p.splits)), dim3(kMlaThreads), 0,
                          stream, timer.start(), timer.stop(), 0, s.T, s.S, W, p.kps, p.splits, xcd_map,
                          s.sm_scale, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv),
                          idx, static_cast<uint16_t*>(o), lse, part_o, part_lse);
    dsa_status_t st = timer.done("mla_mfma");
    if (st != DSA_OK || p.splits == 1) return st;
    const int64_t total_heads = rows * kH;
    LaunchTimer ctimer;
    hipExtLaunchKernelGGL(mla_combine, dim3(static_cast<unsigned>((total_heads + 3) / 4)), dim3(256), 0,
                          stream, ctimer.start(), ctimer.stop(), 0, p.splits, total_heads,
                          static_cast<const uint16_t*>(part_o), static_cast<const float*>(part_lse),
                          static_cast<uint16_t*>(o), lse);
    return ctimer.done("mla_combine");
  }
  const size_t lds = (static_cast<size_t>(s.Dc) + s.Dr + W) * sizeof(float);
  if (lds > 64 * 1024)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: D + K = %d too large for the generic kernel",
                s.Dc + s.Dr + W);
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
