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
// Key tile in LDS: 32 selected rows of 576 bf16, 1152 B apart (no padding),
// each row cut in 72 pieces of 16 B; piece c of row r sits at physical piece
// c ^ (r & 7).  The tile is filled by direct global->LDS loads
// (global_load_lds_dwordx4: lane l of a wave writes 16 B at the wave's LDS
// base + 16 l), so the gather needs no registers and runs asynchronously
// with the MFMAs of the previous tile.
//
// logits^T (32 keys x 32 heads) = K_tile (A, from LDS) . Q^T (B, registers),
// reduction over the 576 dims in 36 steps of 16.  MFMA row m reads the tile's
// row pi(m), pi(8a + 4b + j) = 8a + 2j + b (a permutation inside each group
// of 8 rows).
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
//
// With the row permutation and the piece swizzle, both LDS read patterns
// (8 lanes x 16 B on 8 rows of one column; 4 rows x 32 B for the transposing
// read) touch each of the 32 banks once per pass.
// ---------------------------------------------------------------------------
constexpr int kH = 128, kDc = 512, kDr = 64, kD = kDc + kDr;
constexpr int kMlaWaves = 4;                 // wave w owns heads 32w .. 32w+31
constexpr int kMlaThreads = kMlaWaves * 64;
constexpr int kTileKeys = 32;
constexpr int kPieces = kD / 8;              // 16-byte pieces per key row (72)
constexpr int kTileLoads = kTileKeys * kPieces / 64;       // wave-wide 1 KiB loads per tile (36)
constexpr int kLoadsPerWave = kTileLoads / kMlaWaves;      // 9
constexpr int kMaxSplitKeys = 2048;          // index entries one workgroup stages in LDS
constexpr float kRefSlack = 32.0f;           // log2 units: p <= 2^32 against the reference max

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// a zero key row: skipped index entries load it, so their LDS rows are zero
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[kD];

struct MlaTile {
  uint16_t k[kTileKeys * kD];
};

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char*)(p)));
}

// 16-byte global -> LDS copy per lane: lane l writes LDS [lds + 16 l] (lds is
// wave-uniform).  Issued through asm so the compiler does not hold back the
// current tile's LDS reads behind it; completion is awaited explicitly with
// s_waitcnt vmcnt(0) before the barrier that publishes the tile.
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

__device__ __forceinline__ int tile_row(int m) {  // pi(m)
  return (m & ~7) | ((m & 3) << 1) | ((m >> 2) & 1);
}

// byte offset of (row r, logical piece c) in a tile
__device__ __forceinline__ int tile_off(int r, int c) { return r * (kD * 2) + 16 * (c ^ (r & 7)); }

__device__ __forceinline__ f32x16_t mfma32x32x16_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                                      const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_t*)((__attribute__((address_space(3))) char*)(p)));
}

// grid: (splits, rows).  Split sp covers index entries [sp*kps, (sp+1)*kps).
// splits == 1: writes o (bf16) and lse directly; otherwise writes fp32 partials
// part_o [rows, splits, H, Dc] (already divided by the split's own sum) and
// part_lse [rows, splits, H] (natural log; -inf for an empty split).
__global__ void __launch_bounds__(kMlaThreads, 1)
mla_mfma(int T, int S, int W, int kps, float sm_scale, const uint16_t* __restrict__ q,
         const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
         uint16_t* __restrict__ o, float* __restrict__ lse, float* __restrict__ part_o,
         float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(1024))) MlaTile tiles[2];
  __shared__ int32_t sidx[kMaxSplitKeys];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5, n = lane & 31;
  const int sp = blockIdx.x, nsplit = gridDim.x;
  const int64_t row = blockIdx.y;
  const int b = static_cast<int>(row / T);
  const int j0 = sp * kps;
  const int nj = max(0, min(W, j0 + kps) - j0);
  const int ntiles = (nj + kTileKeys - 1) / kTileKeys;
  const uint16_t* kv_seq = kv + static_cast<int64_t>(b) * S * kD;

  // stage this split's index entries (skipped entries become -1)
  for (int j = tid; j < ntiles * kTileKeys; j += kMlaThreads) {
    int s = j < nj ? idx[row * W + j0 + j] : -1;
    sidx[j] = (s >= 0 && s < S) ? s : -1;
  }

  // query operand (B of logits^T): head 32*wave + n, dims 16ks + 8G .. +8
  bf16x8_t qf[kD / 16];
  {
    const uint16_t* qh = q + (row * kH + 32 * wave + n) * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qh + 16 * ks + 8 * G);
  }

  f32x16_t oacc[kDc / 32];
#pragma unroll
  for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;
  float m_ref = -__builtin_inff();  // reference max (log2 units) of head 32*wave + n
  float l_run = 0.f;
  const float scale2 = sm_scale * kLog2e;
  __syncthreads();  // sidx ready

  // gather: wave-wide load k covers tile slots 64k .. 64k+63 (slot = row*72 + physical piece)
  auto issue_tile = [&](int t, MlaTile& dst) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int k = wave + kMlaWaves * i;
      const int L = 64 * k + lane;
      const int r = L / kPieces, c = (L % kPieces) ^ (r & 7);
      const int s = sidx[t * kTileKeys + r];
      const uint16_t* src = (s >= 0 ? kv_seq + static_cast<int64_t>(s) * kD : g_zero_row) + 8 * c;
      lds_dma_16(src, lds_addr(dst.k) + 1024 * k);
    }
  };

  // LDS byte offsets.  Logits A operand: row pi(n), logical piece 2ks + G;
  // with ks = 4a + bb, (2ks + G) ^ x = 8a + ((2bb + G) ^ x), x = row & 7.
  const int ar = tile_row(n);
  int aoff[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) aoff[bb] = ar * (kD * 2) + 16 * ((2 * bb + G) ^ (ar & 7));
  // Transposing reads: lane (q16, jq, cq) reads MFMA rows 16kk + 8h + 4(q16/2) + jq,
  // latent dims d = 32nb + y*4 + 4(cq&1)... as piece 4nb + y, y = 2(q16&1) + cq/2,
  // byte 8(cq&1).  (4nb + y) ^ x = 4(nb ^ (x>>2)) + ((y ^ x) & 3): even nb move by
  // +64*(x>>2) bytes, odd nb by -64*(x>>2).
  const int q16 = lane >> 4, jq = (lane & 15) >> 2, cq = lane & 3;
  const int y = 2 * (q16 & 1) + (cq >> 1);
  int voff[2][2][2];  // [kk][h][nb parity]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = tile_row(16 * kk + 8 * h + 4 * (q16 >> 1) + jq);
      const int x = r & 7;
      const int base = r * (kD * 2) + 16 * ((y ^ x) & 3) + 8 * (cq & 1);
      voff[kk][h][0] = base + 64 * (x >> 2);
      voff[kk][h][1] = base - 64 * (x >> 2);
    }

  // Online softmax with a fixed reference max per head: the first tile with a
  // valid key sets it, and p = 2^(x - ref) stays below 2^kRefSlack after
  // that as long as no later logit exceeds the reference by more than the
  // slack.  If one does (never for sane data), the whole split is run once
  // more with the true maximum as reference, so O is only ever zeroed, never
  // rescaled.  The decision is workgroup-uniform (barriers stay matched).
  float m_seen = -__builtin_inff();
  bool rerun = false;  // workgroup-uniform
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
#pragma unroll
      for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;
      l_run = 0.f;
      m_ref = m_seen;
    }
    if (ntiles > 0) issue_tile(0, tiles[0]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    bool overflow = false;
    for (int it = 0; it < ntiles; ++it) {
      const char* cur = reinterpret_cast<const char*>(tiles[it & 1].k);
      if (it + 1 < ntiles) issue_tile(it + 1, tiles[(it + 1) & 1]);

      // ---- logits^T: 32 keys x 32 heads ----
      f32x16_t sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8_t ka =
            *reinterpret_cast<const bf16x8_t*>(cur + aoff[ks & 3] + 128 * (ks >> 2));
        sacc = mfma32x32x16_bf16(ka, qf[ks], sacc);
      }

      // ---- softmax weights (lane: head n, MFMA rows 8(i/4) + 4G + i%4) ----
      float x[16];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * G + (i & 3);
        x[i] = sidx[it * kTileKeys + tile_row(m)] >= 0 ? sacc[i] * scale2 : -__builtin_inff();
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
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int nb = 0; nb < kDc / 32; ++nb) {
          const short4_t lo = lds_read_tr16(cur + voff[kk][0][nb & 1] + 64 * nb);
          const short4_t hi = lds_read_tr16(cur + voff[kk][1][nb & 1] + 64 * nb);
          const bf16x8_t vb = __builtin_bit_cast(
              bf16x8_t, short8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          oacc[nb] = mfma32x32x16_bf16(pa[kk], vb, oacc[nb]);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (__syncthreads_or(pass == 0 && overflow)) {
        rerun = true;
        break;
      }
    }
    if (!rerun || pass == 1) break;
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
  if (nsplit == 1) {
#pragma unroll
    for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = hbase + 8 * (i >> 2) + (i & 3);
        o[(row * kH + h) * kDc + 32 * nb + n] = f32_to_bf16(oacc[nb][i] * inv_l[i]);
      }
    if (lse != nullptr && n == 0)
#pragma unroll
      for (int i = 0; i < 16; ++i) lse[row * kH + hbase + 8 * (i >> 2) + (i & 3)] = lse_h[i];
  } else {
    float* po = part_o + ((row * nsplit + sp) * kH) * kDc;
#pragma unroll
    for (int nb = 0; nb < kDc / 32; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = hbase + 8 * (i >> 2) + (i & 3);
        po[h * kDc + 32 * nb + n] = oacc[nb][i] * inv_l[i];
      }
    if (n == 0)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        part_lse[(row * nsplit + sp) * kH + hbase + 8 * (i >> 2) + (i & 3)] = lse_h[i];
  }
}

// grid: (H, rows), 128 threads; thread handles Dc / 128 latent dims
template <int DT>
__global__ void __launch_bounds__(128)
mla_combine(int H, int Dc, int nsplit, const float* __restrict__ part_o,
            const float* __restrict__ part_lse, void* __restrict__ o, float* __restrict__ lse) {
  const int h = blockIdx.x;
  const int64_t row = blockIdx.y;
  float m = -__builtin_inff();
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, part_lse[(row * nsplit + sp) * H + h]);
  float wsum = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float ls = part_lse[(row * nsplit + sp) * H + h];
    wsum += ls == -__builtin_inff() ? 0.f : __expf(ls - m);
  }
  const float lse_tot = wsum > 0.f ? m + __logf(wsum) : -__builtin_inff();
  for (int d = threadIdx.x; d < Dc; d += blockDim.x) {
    float acc = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float ls = part_lse[(row * nsplit + sp) * H + h];
      if (ls == -__builtin_inff()) continue;
      acc = fmaf(__expf(ls - lse_tot), part_o[((row * nsplit + sp) * H + h) * Dc + d], acc);
    }
    store_mla<DT>(o, (row * H + h) * Dc + d, acc);
  }
  if (lse != nullptr && threadIdx.x == 0) lse[row * H + h] = lse_tot;
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
  // least 4 tiles per split and at most kMaxSplitKeys entries per workgroup
  int splits = 1;
  while (rows * splits < cus && W / (splits * 2) >= 4 * kTileKeys) splits *= 2;
  while ((W + splits - 1) / splits > kMaxSplitKeys) splits *= 2;
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
  return rows * p.splits * s.H * (static_cast<size_t>(s.Dc) + 1) * sizeof(float);
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
    if (p.splits == 1) {
      mla_mfma<<<dim3(1, rows), kMlaThreads, 0, stream>>>(
          s.T, s.S, W, p.kps, s.sm_scale, static_cast<const uint16_t*>(q),
          static_cast<const uint16_t*>(kv), idx, static_cast<uint16_t*>(o), lse, nullptr, nullptr);
      return check_launch("mla_mfma");
    }
    const size_t need = mla_workspace_bytes(s);
    if (ws == nullptr || ws_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "sparse_mla: workspace of %zu bytes needed, %zu given", need,
                  ws_bytes);
    float* part_o = static_cast<float*>(ws);
    float* part_lse = part_o + static_cast<size_t>(rows) * p.splits * s.H * s.Dc;
    mla_mfma<<<dim3(p.splits, rows), kMlaThreads, 0, stream>>>(
        s.T, s.S, W, p.kps, s.sm_scale, static_cast<const uint16_t*>(q),
        static_cast<const uint16_t*>(kv), idx, nullptr, nullptr, part_o, part_lse);
    dsa_status_t st = check_launch("mla_mfma");
    if (st != DSA_OK) return st;
    mla_combine<DSA_BF16><<<dim3(s.H, rows), 128, 0, stream>>>(s.H, s.Dc, p.splits, part_o,
                                                               part_lse, o, lse);
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
