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
//    each gathered key tile: 32 selected rows are loaded with coalesced
//    16-byte loads and written to LDS twice, row-major for the logits and
//    transposed (latent part) for the value product.  Wave w owns heads
//    16w..16w+15: logits^T = K_tile . Q^T on MFMA (keys on M, heads on N), an
//    online softmax in fp32 with exp2, and O += P . V on MFMA (heads on M,
//    latent dims on N) with P taken straight from the logit accumulators.
//    LDS is double-buffered: the next tile's rows load into registers during
//    the current tile's MFMAs.
//  * mla_combine: merges split partials (o_s, lse_s) with weights
//    exp(lse_s - lse), deterministically (fixed split order, no atomics).
//  * mla_generic: any shape, fp32 VALU loops, two passes over the index row.
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
// MFMA 32x32x16 bf16 operand layouts (lane l, G = l / 32, n = l % 32):
//   A (32 x 16): lane holds row n, reduction elements 8G .. 8G+7
//   B (16 x 32): lane holds column n, reduction elements 8G .. 8G+7
//   C (32 x 32): register i holds row 8*(i/4) + 4G + (i%4) of column n
//
// Key tile in LDS (38 KiB): latent part of row m (64 pieces of 16 B) at byte
// 1088 m, piece c stored at c ^ ((m >> 2) & 3); rotary part (8 pieces) in a
// region of its own at byte 34816, row m at 128 m, piece c' at c' ^ ((m >> 1) & 7).
// The LDS has 64 banks of 4 bytes (a 16-byte read pass serves 16 lanes, an
// 8-byte pass 32 lanes).  The 1088-byte row stride shifts consecutive rows by
// 4 bank quads and the 2-bit XOR spreads groups of 4 rows, so the logits
// operand reads (16 rows, one piece) and the transposing value reads (4 rows x
// 4 pieces) both touch every bank once per pass, and every read is one base
// register plus a compile-time offset.  The tile is filled by direct
// global->LDS copies (global_load_lds_dwordx4: lane l of a wave writes 16 B at
// the wave's LDS base + 16 l); wave w copies the latent parts of tile rows
// 8w .. 8w+7 (one 1 KiB run of global memory each) and their rotary parts.  The gather needs no registers and runs asynchronously with the MFMAs.
//
// logits^T (32 keys x 32 heads) = K_tile (A, from LDS) . Q^T (B, registers),
// reduction over the 576 dims in 36 steps of 16.  MFMA row m is tile row m.
//
// O (32 heads x 512) += P (A) . V (B), reduction over the 32 keys in two
// MFMAs (kk = 0, 1).  P comes straight from the logit accumulators: lane
// (G, n) holds head n and MFMA rows 8*(i/4) + 4G + i%4; its A-operand slot
// 8G + e of MFMA kk is accumulator i = 8kk + e, i.e. MFMA row
// 16kk + 8(e/4) + 4G + e%4.  V is read from the same row-major tile with the
// transposing LDS load ds_read_b64_tr_b16: within a 16-lane group, lane i
// receives element (i % 4) of the 8-byte chunk loaded by lane 4j + i/4, for
// j = 0..3.  So lane 4j + c of a group loads 4 latent dims (base + 4c) of the
// key in slot (base slot + j), and each lane ends up with 4 consecutive key
// slots of one latent dim: half of its B operand.
// ---------------------------------------------------------------------------
constexpr int kH = 128, kDc = 512, kDr = 64, kD = kDc + kDr;
constexpr int kMlaWaves = 4;                 // wave w owns heads 32w .. 32w+31
constexpr int kMlaThreads = kMlaWaves * 64;
constexpr int kTileKeys = 32;
constexpr int kPieces = kD / 8;              // 16-byte pieces per key row (72)
constexpr int kTileLoads = kTileKeys * kPieces / 64;       // wave-wide 1 KiB copies per tile (36)
constexpr int kLoadsPerWave = kTileLoads / kMlaWaves;      // 9: 8 latent rows + 8 rotary parts
constexpr int kBuffers = 3;                  // LDS tile ring: 2 tiles in flight during compute
constexpr int kLatStride = 1088;             // bytes per latent row in LDS (1024 + 64 pad)
constexpr int kRopeBase = kTileKeys * kLatStride;       // byte offset of the rotary region
constexpr int kTileBytes = kRopeBase + kTileKeys * kDr * 2;  // 38912
constexpr int kReadAhead = 6;                // logits A-operand reads issued ahead of their MFMA
constexpr int kVAhead = 4;                   // value B-operand (2 reads each) issued ahead
constexpr float kRefSlack = 32.0f;           // log2 units: p <= 2^32 against the reference max
// The query operand (36 steps x 8 bf16 per lane) does not fit in registers next
// to the 512 fp32 accumulators of O; its last kQLdsSteps steps live in LDS.
constexpr int kQLdsSteps = 11;
constexpr int kQRegSteps = kD / 16 - kQLdsSteps;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// a zero key row: skipped index entries load it, so their LDS rows are zero
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[kD];

struct MlaTile {
  uint8_t bytes[kTileBytes];
};

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char*)(p)));
}

// 16-byte global -> LDS copy per lane: lane l writes LDS [lds + 16 l] (lds is
// wave-uniform).  Issued through asm so the compiler does not hold back the
// current tile's LDS reads behind it; completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes a tile (loads retire in
// issue order, so vmcnt(N) means all but the last N copies have landed).
// m0 is declared clobbered; the compiler sets m0 itself before each of its own
// uses and this kernel has no other, so the reserved-register warning is moot.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma_16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// wait until at most `groups` tiles' copies of this wave are still in flight
__device__ __forceinline__ void wait_tiles_in_flight(int groups) {
  static_assert(kLoadsPerWave == 9 && kBuffers == 3, "vmcnt immediates assume 9 copies per tile");
  if (groups >= 1)
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ int lat_swz(int m) { return (m >> 2) & 3; }
__device__ __forceinline__ int rope_swz(int m) { return (m >> 1) & 7; }

__device__ __forceinline__ f32x16_t mfma32x32x16_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                                      const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) const char lds_char_t;

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
// sum) and part_lse [rows, nsplit, H] (natural log; -inf for an empty split).
__global__ void __launch_bounds__(kMlaThreads, 1)
mla_mfma(int T, int S, int W, int kps, int nsplit, int xcd_map, float sm_scale,
         const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
         const int32_t* __restrict__ idx, uint16_t* __restrict__ o, float* __restrict__ lse,
         uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(1024))) MlaTile tiles[kBuffers];
  __shared__ uint32_t vmask[kBuffers];  // per tile buffer: bit r = tile row r holds a valid key
  // query steps kQRegSteps.. of each wave: [step][wave][G][head n][8 bf16]
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kQLdsSteps][kMlaWaves][2][32][8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5, n = lane & 31;
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

  // query operand (B of logits^T): head 32*wave + n, dims 16ks + 8G .. +8;
  // steps < kQRegSteps stay in registers, the rest go to LDS
  bf16x8_t qf[kQRegSteps];
  {
    const uint16_t* qh = q + (row * kH + 32 * wave + n) * kD;
#pragma unroll
    for (int ks = 0; ks < kQRegSteps; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qh + 16 * ks + 8 * G);
#pragma unroll
    for (int ks = kQRegSteps; ks < kD / 16; ++ks)
      *reinterpret_cast<bf16x8_t*>(qlds[ks - kQRegSteps][wave][G][n]) =
          *reinterpret_cast<const bf16x8_t*>(qh + 16 * ks + 8 * G);
    // consume the loads here: later vmcnt waits then only see the tile copies
#pragma unroll
    for (int ks = 0; ks < kQRegSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  f32x16_t oacc[kDc / 32];
#pragma unroll
  for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;
  float m_ref = -__builtin_inff();  // reference max (log2 units) of head 32*wave + n
  float l_run = 0.f;
  const float scale2 = sm_scale * kLog2e;

  // Wave w gathers tile rows 8w .. 8w+7.  Their index entries come through
  // scalar loads one tile ahead (skipped or out-of-range entries become -1);
  // the wave publishes their validity as byte w of the tile's mask word.
  const int32_t* idx_row = idx + row * W;
  const int j_end = j0 + nj;
  typedef __attribute__((__vector_size__(8 * sizeof(int32_t)))) int32_t i32x8_t;
  auto tile_rows = [&](int t, int (&sr)[8]) {
    const int j = j0 + t * kTileKeys + 8 * wave;
    if (j + 8 <= j_end) {  // one 32-byte scalar load
      i32x8_t v;
      __builtin_memcpy(&v, idx_row + j, sizeof v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sr[e] = (v[e] >= 0 && v[e] < S) ? v[e] : -1;
    } else {               // the ragged end of the split
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int sv = idx_row[min(j + e, j_end - 1)];
        if (j + e >= j_end || sv < 0 || sv >= S) sv = -1;
        sr[e] = sv;
      }
    }
  };
  auto issue_tile = [&](int t, const int (&sr)[8]) {
    MlaTile& dst = tiles[t % kBuffers];
    // an opaque copy of the lane id: the per-copy address math below is redone
    // at each issue instead of being kept live across the loop in registers
    int lane = __lane_id();
    asm volatile("" : "+v"(lane));
    uint32_t mask8 = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) mask8 |= static_cast<uint32_t>(sr[e] >= 0) << e;
    if (lane == 0) reinterpret_cast<uint8_t*>(&vmask[t % kBuffers])[wave] = static_cast<uint8_t>(mask8);
    // latent part of row r = 8w + e: its 16-byte slot `lane` holds piece lane ^ F(r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * wave + e;
      const uint16_t* src =
          (sr[e] >= 0 ? kv_seq + static_cast<int64_t>(sr[e]) * kD : g_zero_row) + 8 * (lane ^ lat_swz(r));
      lds_dma_16(src, lds_addr(dst.bytes) + kLatStride * r);
    }
    // rotary parts of rows 8w .. 8w+7: lane l takes row 8w + l/8
    {
      const int e = lane >> 3, r = 8 * wave + e;
      int sv = sr[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) sv = e == k ? sr[k] : sv;
      const uint16_t* src = (sv >= 0 ? kv_seq + static_cast<int64_t>(sv) * kD : g_zero_row) + kDc +
                            8 * ((lane & 7) ^ rope_swz(r));
      lds_dma_16(src, lds_addr(dst.bytes) + kRopeBase + 1024 * wave);
    }
  };

  // LDS byte offsets.  Logits A operand of step ks: row n, piece 2ks + G.
  // Latent steps: piece 4(ks/2) + (2(ks&1) + G), stored at 4(ks/2) + ((2(ks&1) + G) ^ F(n)).
  int aoff[2], roff[4];
#pragma unroll
  for (int par = 0; par < 2; ++par) aoff[par] = kLatStride * n + 16 * ((2 * par + G) ^ lat_swz(n));
#pragma unroll
  for (int kr = 0; kr < 4; ++kr) roff[kr] = kRopeBase + 128 * n + 16 * ((2 * kr + G) ^ rope_swz(n));
  // Transposing reads: lane (q16, jq, cq) reads MFMA row m = 16kk + 8h + 4(q16/2) + jq,
  // latent dims 32nb + 16(q16&1) + 4cq: piece 4nb + y, y = 2(q16&1) + cq/2, byte 8(cq&1);
  // F(m) = (2h + q16/2) & 3, so the stored piece is 4nb + (y ^ F(m)).
  const int q16 = lane >> 4, jq = (lane & 15) >> 2, cq = lane & 3;
  const int y = 2 * (q16 & 1) + (cq >> 1);
  int voff[2][2];  // [kk][h]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = 16 * kk + 8 * h + 4 * (q16 >> 1) + jq;
      voff[kk][h] = kLatStride * m + 16 * (y ^ lat_swz(m)) + 8 * (cq & 1);
    }

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
      for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;
      l_run = 0.f;
      m_ref = m_seen;
    }
    bool overflow = false;
    int srn[8];  // index entries of the next tile to issue
    if (ntiles > 0) tile_rows(0, srn);
    for (int t = 0; t < kBuffers - 1 && t < ntiles; ++t) {
      issue_tile(t, srn);
      if (t + 1 < ntiles) tile_rows(t + 1, srn);
    }
    for (int it = 0; it < ntiles; ++it) {
      // tile `it` has landed once at most the copies of the later issued tiles remain
      wait_tiles_in_flight(min(kBuffers - 2, ntiles - 1 - it));
      __syncthreads();  // every wave's copies of tile `it` are in; tile it-1 is consumed
      if (it + kBuffers - 1 < ntiles) {
        issue_tile(it + kBuffers - 1, srn);
        if (it + kBuffers < ntiles) tile_rows(it + kBuffers, srn);
      }
      lds_char_t* cur = (lds_char_t*)(tiles[it % kBuffers].bytes);
      // validity of the tile rows; accumulator i sits on row 8(i/4) + 4G + i%4
      const uint32_t valid = vmask[it % kBuffers] >> (4 * G);

      // ---- logits^T: 32 keys x 32 heads ----
      f32x16_t sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      {
        // software pipeline: the LDS read of step ks + kReadAhead is issued with
        // the MFMA of step ks; sched_barrier keeps each pair in place
        auto aload = [&](int ks) {
          const int off = ks < kDc / 16 ? aoff[ks & 1] + 64 * (ks >> 1) : roff[ks - kDc / 16];
          return *(__attribute__((address_space(3))) const bf16x8_t*)(cur + off);
        };
        auto qload = [&](int ks) {
          return *reinterpret_cast<const bf16x8_t*>(qlds[ks - kQRegSteps][wave][G][n]);
        };
        bf16x8_t ka[kReadAhead], qb[kReadAhead];
#pragma unroll
        for (int ks = 0; ks < kReadAhead; ++ks) {
          ka[ks] = aload(ks);
          if (ks >= kQRegSteps) qb[ks] = qload(ks);
        }
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
          sacc = mfma32x32x16_bf16(ka[ks % kReadAhead],
                                   ks < kQRegSteps ? qf[ks] : qb[ks % kReadAhead], sacc);
          const int nx = ks + kReadAhead;
          if (nx < kD / 16) {
            ka[ks % kReadAhead] = aload(nx);
            if (nx >= kQRegSteps) qb[ks % kReadAhead] = qload(nx);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax weights (lane: head n, accumulator i = MFMA row 8(i/4) + 4G + i%4) ----
      float x[16];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = ((valid >> (8 * (i >> 2) + (i & 3))) & 1) ? sacc[i] * scale2 : -__builtin_inff();
        tmax = fmaxf(tmax, x[i]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      m_seen = fmaxf(m_seen, tmax);
      if (m_ref == -__builtin_inff()) m_ref = tmax;  // O and l of this head are still 0
      overflow |= tmax > m_ref + kRefSlack;
      const float m_use = (m_ref == -__builtin_inff()) ? 0.f : m_ref;
      float psum = 0.f;
      bf16x8_t pa[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4_t pw;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = exp2f(x[8 * kk + e] - m_use);
          const float p1 = exp2f(x[8 * kk + e + 1] - m_use);
          psum += p0 + p1;
          pw[e >> 1] = static_cast<uint32_t>(f32_to_bf16(p0)) |
                       (static_cast<uint32_t>(f32_to_bf16(p1)) << 16);
        }
        pa[kk] = __builtin_bit_cast(bf16x8_t, pw);
      }
      psum += __shfl_xor(psum, 32, 64);
      l_run += psum;

      // ---- O += P . V ----
      {
        // software pipeline over the 32 (kk, nb) steps: the two transposing reads
        // of step st + kVAhead are issued with the MFMA of step st
        constexpr int kSteps = 2 * (kDc / 32);
        // ds_read_b64_tr_b16 takes no folded offset: an opaque per-tile copy of
        // the bases keeps each read's address add next to the read instead of
        // 64 precomputed addresses living across the loop
        int vbase[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            vbase[kk][h] = voff[kk][h];
            asm volatile("" : "+v"(vbase[kk][h]));
          }
        bf16x8_t vb[kVAhead];
        auto vload = [&](int st) {
          const int kk = st / (kDc / 32), nb = st % (kDc / 32);
          const short4_t lo = lds_read_tr16(cur + vbase[kk][0] + 64 * nb);
          const short4_t hi = lds_read_tr16(cur + vbase[kk][1] + 64 * nb);
          return __builtin_bit_cast(
              bf16x8_t, short8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        };
#pragma unroll
        for (int st = 0; st < kVAhead; ++st) vb[st] = vload(st);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          const int kk = st / (kDc / 32), nb = st % (kDc / 32);
          oacc[nb] = mfma32x32x16_bf16(pa[kk], vb[st % kVAhead], oacc[nb]);
          if (st + kVAhead < kSteps) vb[st % kVAhead] = vload(st + kVAhead);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // every copy has landed (the ring is reused by a second pass)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!__syncthreads_or(pass == 0 && overflow)) break;
  }

  // ---- epilogue: oacc[nb][i] = O[head 32*wave + 8(i/4) + 4G + i%4][32nb + n] ----
  float inv_l[16], lse_h[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int src = 8 * (i >> 2) + 4 * G + (i & 3);
    const float l = __shfl(l_run, src, 64);
    const float m = __shfl(m_ref, src, 64);
    inv_l[i] = l > 0.f ? 1.f / l : 0.f;
    lse_h[i] = l > 0.f ? (m + __log2f(l)) * kLn2 : -__builtin_inff();
  }
  const int hbase = 32 * wave + 4 * G;
  uint16_t* dst = nsplit == 1 ? o + (row * kH) * kDc : part_o + ((row * nsplit + sp) * kH) * kDc;
  float* dst_lse = nsplit == 1 ? lse : part_lse + (row * nsplit + sp - row) * kH;
#pragma unroll
  for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = hbase + 8 * (i >> 2) + (i & 3);
      dst[h * kDc + 32 * nb + n] = f32_to_bf16(oacc[nb][i] * inv_l[i]);
    }
  if (dst_lse != nullptr && n == 0)
#pragma unroll
    for (int i = 0; i < 16; ++i) dst_lse[row * kH + hbase + 8 * (i >> 2) + (i & 3)] = lse_h[i];
}

// Merge of the split partials: thread = 8 consecutive latent dims of one head.
// lse = log sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.  Fixed split
// order, no atomics: deterministic.
template <int DT>
__global__ void __launch_bounds__(256)
mla_combine(int H, int Dc, int nsplit, int64_t total_vec, const uint16_t* __restrict__ part_o,
            const float* __restrict__ part_lse, void* __restrict__ o, float* __restrict__ lse) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // 8-dim vector id
  if (v >= total_vec) return;
  const int per_row = H * Dc / 8;
  const int64_t row = v / per_row;
  const int rem = static_cast<int>(v % per_row);
  const int h = rem / (Dc / 8), d0 = (rem % (Dc / 8)) * 8;
  float m = -__builtin_inff();
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, part_lse[(row * nsplit + sp) * H + h]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -__builtin_inff()) {
    for (int sp = 0; sp < nsplit; ++sp) {
      const float ls = part_lse[(row * nsplit + sp) * H + h];
      if (ls == -__builtin_inff()) continue;
      const float wgt = __expf(ls - m);
      wsum += wgt;
      const u32x4_t pv = *reinterpret_cast<const u32x4_t*>(
          part_o + ((row * nsplit + sp) * H + h) * Dc + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(wgt, __uint_as_float(pv[e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(wgt, __uint_as_float(pv[e] & 0xffff0000u), acc[2 * e + 1]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) store_mla<DT>(o, (row * H + h) * Dc + d0 + e, acc[e] * inv);
  if (lse != nullptr && d0 == 0) lse[row * H + h] = wsum > 0.f ? m + __logf(wsum) : -__builtin_inff();
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
    mla_mfma<<<dim3(static_cast<unsigned>(rows * p.splits)), kMlaThreads, 0, stream>>>(
        s.T, s.S, W, p.kps, p.splits, xcd_map, s.sm_scale, static_cast<const uint16_t*>(q),
        static_cast<const uint16_t*>(kv), idx, static_cast<uint16_t*>(o), lse, part_o, part_lse);
    dsa_status_t st = check_launch("mla_mfma");
    if (st != DSA_OK || p.splits == 1) return st;
    const int64_t total_vec = rows * s.H * s.Dc / 8;
    mla_combine<DSA_BF16><<<dim3(static_cast<unsigned>((total_vec + 255) / 256)), 256, 0, stream>>>(
        s.H, s.Dc, p.splits, total_vec, part_o, part_lse, o, lse);
    return check_launch("mla_combine");
  }
  const size_t lds = (static_cast<size_t>(s.Dc) + s.Dr + W) * sizeof(float);
  if (lds > 64 * 1024)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_mla: D + K = %d too large for the generic kernel",
                s.Dc + s.Dr + W);
  if (s.mla_dtype == DSA_BF16)
    mla_generic<DSA_BF16><<<dim3(s.H, rows), 256, lds, stream>>>(s.T, s.S, s.H, s.Dc, s.Dr, W,
                                                                 s.sm_scale, q, kv, idx, o, lse);
  else
    mla_generic<DSA_F32><<<dim3(s.H, rows), 256, lds, stream>>>(s.T, s.S, s.H, s.Dc, s.Dr, W,
                                                                s.sm_scale, q, kv, idx, o, lse);
  return check_launch("mla_generic");
}

}  // namespace dsa
