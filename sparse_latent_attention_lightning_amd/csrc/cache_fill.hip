// Cache fill and indexer inputs on gfx950: the step before the sparse path.
//
// For each new token with hidden state x (the attention input) the joint
// projection p = W x covers four blocks (atlas.klimoza.dev, DeepSeek-V3.2-Exp
// MoE block, "All 43 steps": c^KV = x W_DKV, k^pe = x W_KR, w = x W_w; the
// indexer key projection wk and its k_norm from the nnterp deepseek_v32
// module tree; the [512, 64] split of the joint down-projection, then the
// latent norm and the key rotation, from the mla-kv excerpt of the atlas
// "DeepSeek-V3.2-Exp · Attention input" page):
//   c^KV = p[0:512]     -> RMSNorm (eps 1e-6) times the gain       -> kv row 0..511
//   k^pe = p[512:576]   -> pair (2i, 2i+1) turned by the token's
//                          angle i into dims i and i + 32           -> kv row 512..575
//   k^I  = p[576:704]   -> LayerNorm (eps 1e-6), gain and bias      -> indexer key row
//                          (bf16, or E4M3 codes with one ue8m0 scale)
//   w    = p[704:768]   -> the head weights of the token's query
// The rotary layout for this model (the nnterp deepseek_v32 page, section
// 03): the projection's dims 2i and 2i+1 form a pair that lands in rotary
// dims i and i + 32.
//
// Kernels:
//  * fill_gemm_skinny (few tokens, a decode step): p = x W^T on 32x32x16
//    bf16 MFMAs with fp32 partial sums over slices of the hidden dimension,
//    so that the weights stream through many workgroups at once;
//    fill_gemm_tiled (many tokens): 128 x 128 tiles through an LDS ring.
//    Both operands are contiguous along the reduction (W in Linear layout,
//    one output per row); both take a batch of such products (one per head
//    for the absorption products) and, when one slice covers the reduction,
//    write the finished bf16 / fp32 values (the tiled kernel also E4M3 codes
//    with one ue8m0 scale per 128-output tile, and the absorbed query's
//    rotary part).
//  * fill_rows: one workgroup per token sums the partials in a fixed order
//    (deterministic), then the norms, the rotation, the quantiser, and the
//    scatter into the caches' rows; q_rows does the same for the indexer
//    query's heads.
//  * the absorption products either side of the sparse attention (see the
//    section further down): uk_transpose (W_UK in reduction-contiguous
//    form), q_rope (the query's rotary part), gemm_finish (slice sums of the
//    output projection).
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kFillLat = 512, kFillRope = 64, kFillIdx = 128, kFillW = 64;
constexpr int kFillCols = kFillLat + kFillRope + kFillIdx + kFillW;  // 768
constexpr int kGemmKStep = 64;                  // reduction width per iteration
constexpr int kGemmRows = 32;                   // tokens per workgroup of the few-token kernel
constexpr float kNormEps = 1e-6f;

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4v_t;

// Operands of a batch of products p_b = x_b W_b^T (one per head for the
// absorption products, a batch of 1 otherwise): token n of batch b is the row
// x + b sx + n ldx (D contiguous elements), output j of batch b the row
// W + b sw + j D.  Partial sums go to part[(b slices + slice) N ncols]; a
// product over one slice may instead write its result straight to
// out + b so + n ldo + j (kernels instantiated with OUT = DSA_BF16 / DSA_F32).
struct GemmOperands {
  const uint16_t* x;
  const uint16_t* W;
  int64_t ldx, sx, sw;
  void* out;
  int64_t ldo, so;
  uint8_t* out_sf;  // E4M3 output: one ue8m0 scale byte per (row, 128-output tile)
  // the absorbed query's rotary part (tiled kernel, finished output, 4
  // output tiles: tile b takes pairs 8b .. 8b+7): pair (2i, 2i+1) of x's
  // elements rope_at .. rope_at + 63 turned by angle i into out elements
  // rope_to + i and rope_to + 32 + i (null: none)
  const float* rope_cos;
  const float* rope_sin;
  int rope_at, rope_to;
};
constexpr int kOutPartial = -1;

// element (t, j) of batch b: a partial sum, or the finished value
template <int OUT>
__device__ __forceinline__ void gemm_store(const GemmOperands& g, float* part, int64_t pidx, int bt,
                                           int t, int j, float v) {
  if constexpr (OUT == kOutPartial) {
    part[pidx] = v;
  } else {
    const int64_t o = bt * g.so + t * g.ldo + j;
    if constexpr (OUT == DSA_BF16)
      static_cast<uint16_t*>(g.out)[o] = f32_to_bf16(v);
    else
      static_cast<float*>(g.out)[o] = v;
  }
}

// fp32 -> OCP E4M3FN code, round to nearest with ties to the even code;
// |v| <= 448 (the caller's scale guarantees it; larger saturates to 448)
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9, rint ties to even
    return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // 8 = smallest normal
  }
  // keep 3 mantissa bits: add half an ulp of the 3-bit mantissa (minus one
  // when the kept lsb is 0, so exact halves go to the even code), then cut
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  const int e = static_cast<int>(r >> 23) - 127;  // -6 .. 8
  uint32_t code = (static_cast<uint32_t>(e + 7) << 3) | ((r >> 20) & 7u);
  if (code > 0x7Eu) code = 0x7Eu;  // 448 is the largest finite code
  return sign | code;
}

// e of the ue8m0 scale 2^e of a block with largest magnitude amax: the
// smallest integer with 448 2^e >= amax (0 for an all-zero block), but not
// below -127, the smallest scale the byte e + 127 can hold (a block whose
// largest magnitude is under 448 2^-127 keeps that scale; its codes then
// stay within range).  With amax = M 2^E (1 <= M < 2) and 448 = 1.75 2^8:
// e = E - 8 when M <= 1.75, else E - 7.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t u = __float_as_uint(amax);
  const int E = static_cast<int>(u >> 23) - 127;  // -127 for a subnormal amax
  const int e = E - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// max over the wave's 64 lanes on lane moves (no LDS): xor 1 and 2 within
// quads, the half-row and row mirrors (8 and 16 lanes), then the 16- and
// 32-lane swaps of gfx950 (row r of the first operand trades places with row
// r - 1 of the second: the two results hold both rows' maxima)
__device__ __forceinline__ float wave_max_lanes(float v) {
  auto dpp = [](float x, int ctrl) -> float {
    switch (ctrl) {  // the control must be a constant
      case 0xB1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
      case 0x141: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    }
  };
  v = fmaxf(v, dpp(v, 0xB1));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp(v, 0x4E));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp(v, 0x141));  // row_half_mirror
  v = fmaxf(v, dpp(v, 0x140));  // row_mirror
  const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
  const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
}

// v / 2^e (a multiplication by an exact power of two where 2^-e is a normal float)
__device__ __forceinline__ float scale_down(float v, int e) {
  return (e >= -126 && e <= 126) ? v * __uint_as_float(static_cast<uint32_t>(127 - e) << 23)
                                 : ldexpf(v, -e);
}

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Few tokens (a decode step): the weights are the traffic, and they should
// be in flight all at once.  Workgroup = one 32-output tile of one slice of
// the hidden dimension; its 4 waves take consecutive runs of kSkinnyChunks
// 64-wide chunks each, issue every load of their run before the first MFMA,
// and add their accumulators through LDS, so one partial per workgroup
// reaches memory.  grid: (output tiles of 32, token blocks, batch x slices).
//
// Loads read whole rows: load s of a chunk gives lane l the 16-byte piece
// l & 7 of row 8 s + l / 8 (8 rows x 128 contiguous bytes per instruction;
// a lane per row of the MFMA layout would touch 32 rows, four times the
// cache lines per instruction, and runs at about half the rate).  Each
// chunk then goes through the wave's own 8 KB of LDS into the MFMA layout
// (row r's piece c in slot tile_slot(r, c): conflict-free both ways).
constexpr int kSkinnyChunks = 4;
constexpr int kSkinnyWaves = 4;

__device__ __forceinline__ int tile_slot(int r, int piece) { return piece ^ (r & 7) ^ ((r >> 3) & 1); }

template <int OUT>
__global__ void __launch_bounds__(kSkinnyWaves * 64)
fill_gemm_skinny(int N, int D, int ncols, int slices, GemmOperands g, float* __restrict__ part) {
  __shared__ float red[kSkinnyWaves - 1][16][64];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kSkinnyWaves][2][kGemmRows * 128];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5, m = lane & 31;
  const int m0 = blockIdx.y * kGemmRows;
  const int c0 = blockIdx.x * 32;
  const int nchunks = D / kGemmKStep;
  const int bt = blockIdx.z / slices, sl = blockIdx.z - bt * slices;
  const int ch0 = (sl * kSkinnyWaves + wave) * kSkinnyChunks;
  const int lr = lane >> 3, lp = lane & 7;  // this lane's row (within 8) and piece
  u32x4v_t a[kSkinnyChunks][4], b[kSkinnyChunks][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4v_t* ap = reinterpret_cast<const u32x4v_t*>(
        g.x + bt * g.sx + static_cast<int64_t>(min(m0 + 8 * s + lr, N - 1)) * g.ldx + 8 * lp);
    const u32x4v_t* bp = reinterpret_cast<const u32x4v_t*>(
        g.W + bt * g.sw + static_cast<int64_t>(c0 + 8 * s + lr) * D + 8 * lp);
#pragma unroll
    for (int j = 0; j < kSkinnyChunks; ++j) {
      const int ch = min(ch0 + j, nchunks - 1);  // past the end: a valid chunk, not used
      a[j][s] = ap[ch * (kGemmKStep / 8)];
      b[j][s] = __builtin_nontemporal_load(bp + ch * (kGemmKStep / 8));
    }
  }
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  uint8_t* xs = stage[wave][0];
  uint8_t* ws = stage[wave][1];
#pragma unroll
  for (int j = 0; j < kSkinnyChunks; ++j) {
    if (ch0 + j < nchunks) {  // wave-uniform
      // the wave's LDS is its own and the LDS runs one wave's operations in
      // order: the previous chunk's reads are done before these writes land
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 8 * s + lr;
        *reinterpret_cast<u32x4v_t*>(xs + r * 128 + 16 * tile_slot(r, lp)) = a[j][s];
        *reinterpret_cast<u32x4v_t*>(ws + r * 128 + 16 * tile_slot(r, lp)) = b[j][s];
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int piece = 2 * s4 + hl;
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(xs + m * 128 + 16 * tile_slot(m, piece));
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(ws + m * 128 + 16 * tile_slot(m, piece));
        acc = mfma32(av, bv, acc);
      }
    }
  }
  if (wave > 0)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave - 1][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
    const int64_t pbase = static_cast<int64_t>(blockIdx.z) * N * ncols;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = acc[i];
#pragma unroll
      for (int u = 0; u < kSkinnyWaves - 1; ++u) v += red[u][i][lane];
      const int t = m0 + 8 * (i >> 2) + 4 * hl + (i & 3);
      if (t < N) gemm_store<OUT>(g, part, pbase + static_cast<int64_t>(t) * ncols + c0 + m, bt, t, c0 + m, v);
    }
  }
}

// Many tokens (prefill): a tiled product.  Workgroup = 128 tokens x 128
// outputs, wave w = a 64 x 64 quarter (2 x 2 tiles of 32 x 32); the
// reduction moves in 64-wide chunks through a ring of kTStages LDS stages
// (per stage an A tile of 128 token rows and a B tile of 128 weight rows,
// 128 bytes each), filled by direct global -> LDS copies that run
// kTStages - 1 chunks ahead.  A row's 16-byte piece c sits in slot
// c ^ (r & 7) ^ ((r >> 3) & 1), so that the operand reads (32 rows, one piece
// each) touch every bank once per cycle.
constexpr int kTM = 128, kTN = 128;
constexpr int kXcds = 8;  // accelerator dies of the MI355X, one L2 each
constexpr int kTTile = kTM * kGemmKStep * 2;  // 16 KB per operand tile
constexpr int kTCopies = kTTile / 1024 / 4;   // copies per wave per operand tile

// STAGES = 4 (the ring above, one workgroup per CU) or 2 (half the LDS: two
// workgroups per CU hide each other's load latency; each chunk then waits
// for its own copies).  The launches use 2: measured faster for every
// reduction tried (the 8-chunk absorbed output of 16384 tokens 700 us
// against 790, the 112-chunk cache fill 250 us against 270).
template <int OUT, int STAGES>
__global__ void __launch_bounds__(256, 4 / STAGES)
fill_gemm_tiled(int N, int D, int ncols, GemmOperands g, float* __restrict__ part) {
  static_assert(STAGES == 4 || STAGES == 2, "ring depth");
  constexpr int kTStages = STAGES;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kTStages][2][kTTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, m = lane & 31;
  // XCD-aware order: workgroup i is dispatched to XCD i % 8, each XCD with
  // its own L2; give every XCD a contiguous run of tiles (output tile fastest)
  // so that the tiles sharing a token block, and a batch's weights, meet in
  // one L2 instead of being fetched by every XCD
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int per_xcd = total / kXcds;
  const int w_id = lin < per_xcd * kXcds ? (lin % kXcds) * per_xcd + lin / kXcds : lin;
  const int bx = w_id % gx, by = (w_id / gx) % gy, bz = w_id / (gx * gy);
  const int m0 = by * kTM, n0 = bx * kTN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nk = D / kGemmKStep;
  const uint16_t* x = g.x + bz * g.sx;
  const uint16_t* W = g.W + bz * g.sw;
  part += static_cast<int64_t>(bz) * N * ncols;
  // copy j of an operand tile covers its rows 8j .. 8j+7; lane l writes slot
  // l & 7 of row 8j + l / 8 (rows past the last token load the last token)
  auto issue = [&](int c) {
    const int st = c % kTStages;
#pragma unroll
    for (int i = 0; i < kTCopies; ++i) {
      const int j = wave * kTCopies + i;
      const int r = 8 * j + (lane >> 3);
      const int piece = tile_slot(r, lane & 7);
      const int64_t k = static_cast<int64_t>(c) * kGemmKStep + piece * 8;
      lds_dma_16(x + min(m0 + r, N - 1) * g.ldx + k, lds_addr(ring[st][0]) + 1024 * j);
      lds_dma_16(W + static_cast<int64_t>(n0 + r) * D + k, lds_addr(ring[st][1]) + 1024 * j);
    }
  };
#pragma unroll
  for (int c = 0; c < kTStages - 1; ++c)
    if (c < nk) issue(c);
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  for (int c = 0; c < nk; ++c) {
    // chunk c has landed: the copies issued after it are those of the next
    // min(kTStages - 2, nk - 1 - c) chunks, 2 kTCopies each
    const int later = min(kTStages - 2, nk - 1 - c);
    static_assert(kTCopies == 4, "vmcnt immediates");
    if (later >= 2)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's copies of chunk c are in; chunk c - 1 is consumed
    if (c + kTStages - 1 < nk) issue(c + kTStages - 1);
    const uint8_t* At = ring[c % kTStages][0];
    const uint8_t* Bt = ring[c % kTStages][1];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int piece = 2 * s4 + hl;
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra = wm + 32 * t + m, rb = wn + 32 * t + m;
        a[t] = *reinterpret_cast<const bf16x8_t*>(At + ra * 128 + 16 * tile_slot(ra, piece));
        b[t] = *reinterpret_cast<const bf16x8_t*>(Bt + rb * 128 + 16 * tile_slot(rb, piece));
      }
#pragma unroll
      for (int ta = 0; ta < 2; ++ta)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[ta][tb] = mfma32(a[ta], b[tb], acc[ta][tb]);
    }
  }
  // register i of tile (ta, tb): token m0 + wm + 32 ta + 8 (i / 4) + 4 h + i % 4,
  // output n0 + wn + 32 tb + m
  if constexpr (OUT == DSA_FP8_E4M3) {
    // E4M3 codes with one ue8m0 scale per (token, 128-output tile), the
    // quantiser of the indexer keys: the fp32 tile goes through the idle
    // ring, then each wave finishes whole token rows (2 outputs per lane)
    static_assert(kTM * kTN * 4 <= sizeof(ring), "fp32 tile in the ring");
    __syncthreads();  // every wave is done with the ring
    float* tile = reinterpret_cast<float*>(&ring[0][0][0]);
#pragma unroll
    for (int ta = 0; ta < 2; ++ta)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          tile[(wm + 32 * ta + 8 * (i >> 2) + 4 * hl + (i & 3)) * kTN + wn + 32 * tb + m] = acc[ta][tb][i];
    __syncthreads();
    // wave w takes rows w + 4 k, eight independent rows at a time (one wave
    // per SIMD here: the rows' dependent chains overlap only within a wave)
    uint8_t* codes = static_cast<uint8_t*>(g.out) + bz * g.so;
    constexpr int kRowsAtOnce = 8;
#pragma unroll 1
    for (int r0 = wave; r0 < kTM && m0 + r0 < N; r0 += 4 * kRowsAtOnce) {
      float2 v[kRowsAtOnce];
      float am[kRowsAtOnce];
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u)
        v[u] = reinterpret_cast<const float2*>(tile + (r0 + 4 * u) * kTN)[lane];
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u) am[u] = fmaxf(fabsf(v[u].x), fabsf(v[u].y));
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u) am[u] = wave_max_lanes(am[u]);
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u) {
        const int t = m0 + r0 + 4 * u;
        const int e = ue8m0_exponent(am[u]);
        const uint32_t c = e4m3_code(scale_down(v[u].x, e)) | (e4m3_code(scale_down(v[u].y, e)) << 8);
        if (t < N) {
          *reinterpret_cast<uint16_t*>(codes + static_cast<int64_t>(t) * g.ldo + n0 + 2 * lane) =
              static_cast<uint16_t>(c);
          if (lane == 0)
            g.out_sf[(static_cast<int64_t>(bz) * N + t) * (ncols / kTN) + bx] = static_cast<uint8_t>(e + 127);
        }
      }
    }
  } else if constexpr (OUT == DSA_BF16 || OUT == DSA_F32) {
    // finished values: the tile goes through the idle ring so that each
    // token's 128 outputs leave as whole 16-byte pieces of its row
    using T = typename std::conditional<OUT == DSA_BF16, uint16_t, float>::type;
    constexpr int kPer = 16 / sizeof(T);  // elements per 16-byte piece
    static_assert(kTM * kTN * sizeof(T) <= sizeof(ring), "output tile in the ring");
    __syncthreads();  // every wave is done with the ring
    T* tile = reinterpret_cast<T*>(&ring[0][0][0]);
#pragma unroll
    for (int ta = 0; ta < 2; ++ta)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = acc[ta][tb][i];
          T* dst = tile + (wm + 32 * ta + 8 * (i >> 2) + 4 * hl + (i & 3)) * kTN + wn + 32 * tb + m;
          if constexpr (OUT == DSA_BF16) *dst = f32_to_bf16(v);
          else *dst = v;
        }
    __syncthreads();
    T* out = static_cast<T*>(g.out) + bz * g.so;
    constexpr int kPieces = kTM * kTN / kPer;  // of the whole tile
#pragma unroll
    for (int k = 0; k < kPieces / 256; ++k) {
      const int piece = k * 256 + static_cast<int>(threadIdx.x);
      const int r = piece / (kTN / kPer), cp = piece % (kTN / kPer);
      const int t = m0 + r;
      if (t < N)
        *reinterpret_cast<u32x4v_t*>(out + static_cast<int64_t>(t) * g.ldo + n0 + kPer * cp) =
            *reinterpret_cast<const u32x4v_t*>(tile + r * kTN + kPer * cp);
    }
    if (g.rope_cos != nullptr) {
      // the 32 pairs split over the 4 output tiles (8 each); a thread's 4
      // (token, pair) items load everything before any arithmetic
      constexpr int kPairs = 8, kItems = kTM * kPairs / 256;
      uint32_t pr[kItems];
      float cs[kItems], sn[kItems];
#pragma unroll
      for (int u = 0; u < kItems; ++u) {
        const int it = static_cast<int>(threadIdx.x) + 256 * u;
        const int t = min(m0 + it / kPairs, N - 1), i = bx * kPairs + it % kPairs;
        pr[u] = *reinterpret_cast<const uint32_t*>(x + t * g.ldx + g.rope_at + 2 * i);
        cs[u] = g.rope_cos[static_cast<int64_t>(t) * 32 + i];
        sn[u] = g.rope_sin[static_cast<int64_t>(t) * 32 + i];
      }
#pragma unroll
      for (int u = 0; u < kItems; ++u) {
        const int it = static_cast<int>(threadIdx.x) + 256 * u;
        const int t = m0 + it / kPairs, i = bx * kPairs + it % kPairs;
        if (t >= N) continue;
        const float a = bf16_to_f32(static_cast<uint16_t>(pr[u])), b = bf16_to_f32(static_cast<uint16_t>(pr[u] >> 16));
        T* o = out + static_cast<int64_t>(t) * g.ldo + g.rope_to + i;
        if constexpr (OUT == DSA_BF16) {
          o[0] = f32_to_bf16(a * cs[u] - b * sn[u]);
          o[32] = f32_to_bf16(a * sn[u] + b * cs[u]);
        } else {
          o[0] = a * cs[u] - b * sn[u];
          o[32] = a * sn[u] + b * cs[u];
        }
      }
    }
  } else {
#pragma unroll
    for (int ta = 0; ta < 2; ++ta)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = m0 + wm + 32 * ta + 8 * (i >> 2) + 4 * hl + (i & 3);
        if (t < N)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const int j = n0 + wn + 32 * tb + m;
            gemm_store<OUT>(g, part, static_cast<int64_t>(t) * ncols + j, bz, t, j, acc[ta][tb][i]);
          }
      }
  }
}

// Many tokens with a long reduction: 256 tokens x 128 outputs per workgroup,
// wave w = 128 x 64 (4 x 2 MFMA tiles), so each operand read from LDS feeds
// more MFMAs than the 128 x 128 kernel's 2 x 2 (6 reads per 8 MFMAs against
// 4 per 4); a 3-stage ring of 48 KB stages (A 32 KB, B 16 KB), direct
// copies two chunks ahead, the same swizzle.  Partial or finished bf16 /
// fp32 output (the latter staged through the ring as 16-byte row pieces).
constexpr int kWM = 256, kWStages = 3;
constexpr int kWATile = kWM * kGemmKStep * 2;     // 32 KB
constexpr int kWACopies = kWATile / 1024 / 4;     // 8 per wave
constexpr int kWStage = kWATile + kTTile;         // 48 KB

template <int OUT>
__global__ void __launch_bounds__(256, 1)
fill_gemm_wide(int N, int D, int ncols, GemmOperands g, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kWStages][kWStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, m = lane & 31;
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int per_xcd = total / kXcds;
  const int w_id = lin < per_xcd * kXcds ? (lin % kXcds) * per_xcd + lin / kXcds : lin;
  const int bx = w_id % gx, by = (w_id / gx) % gy, bz = w_id / (gx * gy);
  const int m0 = by * kWM, n0 = bx * kTN;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 64;
  const int nk = D / kGemmKStep;
  const uint16_t* x = g.x + bz * g.sx;
  const uint16_t* W = g.W + bz * g.sw;
  part += static_cast<int64_t>(bz) * N * ncols;
  auto issue = [&](int c) {
    uint8_t* st = ring[c % kWStages];
#pragma unroll
    for (int i = 0; i < kWACopies; ++i) {  // A rows 8j .. 8j + 7, j < 32
      const int j = wave * kWACopies + i;
      const int r = 8 * j + (lane >> 3);
      const int64_t k = static_cast<int64_t>(c) * kGemmKStep + tile_slot(r, lane & 7) * 8;
      lds_dma_16(x + min(m0 + r, N - 1) * g.ldx + k, lds_addr(st) + 1024 * j);
    }
#pragma unroll
    for (int i = 0; i < kTCopies; ++i) {  // B rows 8j .. 8j + 7, j < 16
      const int j = wave * kTCopies + i;
      const int r = 8 * j + (lane >> 3);
      const int64_t k = static_cast<int64_t>(c) * kGemmKStep + tile_slot(r, lane & 7) * 8;
      lds_dma_16(W + static_cast<int64_t>(n0 + r) * D + k, lds_addr(st + kWATile) + 1024 * j);
    }
  };
#pragma unroll
  for (int c = 0; c < kWStages - 1; ++c)
    if (c < nk) issue(c);
  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  static_assert(kWACopies + kTCopies == 12 && kWStages == 3, "vmcnt immediate: one chunk = 12 copies per wave");
  for (int c = 0; c < nk; ++c) {
    // chunk c has landed when at most the next chunk's 12 copies are out
    if (c + 1 < nk)
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's copies of chunk c are in; chunk c - 1 is consumed
    if (c + kWStages - 1 < nk) issue(c + kWStages - 1);
    const uint8_t* At = ring[c % kWStages];
    const uint8_t* Bt = At + kWATile;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int piece = 2 * s4 + hl;
      bf16x8_t a[4], b[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ra = wm + 32 * t + m;
        a[t] = *reinterpret_cast<const bf16x8_t*>(At + ra * 128 + 16 * tile_slot(ra, piece));
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rb = wn + 32 * t + m;
        b[t] = *reinterpret_cast<const bf16x8_t*>(Bt + rb * 128 + 16 * tile_slot(rb, piece));
      }
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[ta][tb] = mfma32(a[ta], b[tb], acc[ta][tb]);
    }
  }
  // register i of tile (ta, tb): token m0 + wm + 32 ta + 8 (i / 4) + 4 h + i % 4,
  // output n0 + wn + 32 tb + m
  if constexpr (OUT == DSA_FP8_E4M3) {
    // E4M3 codes with one ue8m0 scale per (token, 128-output tile), the
    // quantiser of the indexer keys: the fp32 tile goes through the idle
    // ring, then each wave finishes whole token rows (2 outputs per lane)
    static_assert(kWM * kTN * 4 <= sizeof(ring), "fp32 tile in the ring");
    __syncthreads();  // every wave is done with the ring
    float* tile = reinterpret_cast<float*>(&ring[0][0]);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          tile[(wm + 32 * ta + 8 * (i >> 2) + 4 * hl + (i & 3)) * kTN + wn + 32 * tb + m] = acc[ta][tb][i];
    __syncthreads();
    // wave w takes rows w + 4 k, eight independent rows at a time (one wave
    // per SIMD here: the rows' dependent chains overlap only within a wave)
    uint8_t* codes = static_cast<uint8_t*>(g.out) + bz * g.so;
    constexpr int kRowsAtOnce = 8;
#pragma unroll 1
    for (int r0 = wave; r0 < kWM && m0 + r0 < N; r0 += 4 * kRowsAtOnce) {
      float2 v[kRowsAtOnce];
      float am[kRowsAtOnce];
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u)
        v[u] = reinterpret_cast<const float2*>(tile + (r0 + 4 * u) * kTN)[lane];
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u) am[u] = fmaxf(fabsf(v[u].x), fabsf(v[u].y));
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u) am[u] = wave_max_lanes(am[u]);
#pragma unroll
      for (int u = 0; u < kRowsAtOnce; ++u) {
        const int t = m0 + r0 + 4 * u;
        const int e = ue8m0_exponent(am[u]);
        const uint32_t c = e4m3_code(scale_down(v[u].x, e)) | (e4m3_code(scale_down(v[u].y, e)) << 8);
        if (t < N) {
          *reinterpret_cast<uint16_t*>(codes + static_cast<int64_t>(t) * g.ldo + n0 + 2 * lane) =
              static_cast<uint16_t>(c);
          if (lane == 0)
            g.out_sf[(static_cast<int64_t>(bz) * N + t) * (ncols / kTN) + bx] = static_cast<uint8_t>(e + 127);
        }
      }
    }
  } else if constexpr (OUT == DSA_BF16 || OUT == DSA_F32) {
    using T = typename std::conditional<OUT == DSA_BF16, uint16_t, float>::type;
    constexpr int kPer = 16 / sizeof(T);
    static_assert(kWM * kTN * sizeof(T) <= sizeof(ring), "output tile in the ring");
    __syncthreads();  // every wave is done with the ring
    T* tile = reinterpret_cast<T*>(&ring[0][0]);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = acc[ta][tb][i];
          T* dst = tile + (wm + 32 * ta + 8 * (i >> 2) + 4 * hl + (i & 3)) * kTN + wn + 32 * tb + m;
          if constexpr (OUT == DSA_BF16) *dst = f32_to_bf16(v);
          else *dst = v;
        }
    __syncthreads();
    T* out = static_cast<T*>(g.out) + bz * g.so;
    constexpr int kPieces = kWM * kTN / kPer;
#pragma unroll
    for (int k = 0; k < kPieces / 256; ++k) {
      const int piece = k * 256 + static_cast<int>(threadIdx.x);
      const int r = piece / (kTN / kPer), cp = piece % (kTN / kPer);
      const int t = m0 + r;
      if (t < N)
        *reinterpret_cast<u32x4v_t*>(out + static_cast<int64_t>(t) * g.ldo + n0 + kPer * cp) =
            *reinterpret_cast<const u32x4v_t*>(tile + r * kTN + kPer * cp);
    }
  } else {
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = m0 + wm + 32 * ta + 8 * (i >> 2) + 4 * hl + (i & 3);
        if (t < N)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const int j = n0 + wn + 32 * tb + m;
            gemm_store<OUT>(g, part, static_cast<int64_t>(t) * ncols + j, bz, t, j, acc[ta][tb][i]);
          }
      }
  }
}

// sum over a workgroup of 256 threads (4 waves); red: 4 floats of LDS
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();  // red may be reused
  return r;
}

// One workgroup of 256 threads per token.
template <int KVDT, int KDT, int WDT>
__global__ void __launch_bounds__(256)
fill_rows(int N, int slices, const float* __restrict__ part, const float* __restrict__ kv_gamma,
          const float* __restrict__ k_gamma, const float* __restrict__ k_beta,
          const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
          const int64_t* __restrict__ slots, void* __restrict__ kv_cache,
          void* __restrict__ k_cache, uint8_t* __restrict__ k_sf, void* __restrict__ w_out) {
  __shared__ float p[kFillCols];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int n = blockIdx.x;
  const int64_t slot = slots[n];
  // the projection: partial sums in slice order
  // (three outputs per thread, four slices per step: the loads of a step are
  // independent; the sum runs in slice order)
  {
    const float* src = part + static_cast<int64_t>(n) * kFillCols + tid;
    const int64_t stride = static_cast<int64_t>(N) * kFillCols;
    float acc[3] = {0.f, 0.f, 0.f};
    int sl = 0;
    for (; sl + 4 <= slices; sl += 4) {
      float v[4][3];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 3; ++q) v[u][q] = src[(sl + u) * stride + 256 * q];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 3; ++q) acc[q] += v[u][q];
    }
    for (; sl < slices; ++sl)
#pragma unroll
      for (int q = 0; q < 3; ++q) acc[q] += src[sl * stride + 256 * q];
#pragma unroll
    for (int q = 0; q < 3; ++q) p[tid + 256 * q] = acc[q];
  }
  __syncthreads();

  // c^KV: RMSNorm over 512 dims (two per thread)
  const float c0v = p[tid], c1v = p[tid + 256];
  const float ms = block_sum(c0v * c0v + c1v * c1v, red) * (1.0f / kFillLat);
  const float inv_rms = 1.0f / sqrtf(ms + kNormEps);
  // k^I: LayerNorm over 128 dims (threads 0..127), mean then squared deviations
  const float y = tid < kFillIdx ? p[kFillLat + kFillRope + tid] : 0.f;
  const float mean = block_sum(y, red) * (1.0f / kFillIdx);
  const float dev = tid < kFillIdx ? y - mean : 0.f;
  const float var = block_sum(dev * dev, red) * (1.0f / kFillIdx);
  const float z = tid < kFillIdx ? dev * (1.0f / sqrtf(var + kNormEps)) * k_gamma[tid] + k_beta[tid] : 0.f;

  if (slot >= 0) {
    // kv row: [normalised latent ; rotated key]
    auto put_kv = [&](int i, float v) {
      if constexpr (KVDT == DSA_BF16)
        static_cast<uint16_t*>(kv_cache)[slot * (kFillLat + kFillRope) + i] = f32_to_bf16(v);
      else
        static_cast<float*>(kv_cache)[slot * (kFillLat + kFillRope) + i] = v;
    };
    put_kv(tid, c0v * inv_rms * kv_gamma[tid]);
    put_kv(tid + 256, c1v * inv_rms * kv_gamma[tid + 256]);
    if (tid < kFillRope / 2) {
      const float cs = rope_cos[static_cast<int64_t>(n) * (kFillRope / 2) + tid];
      const float sn = rope_sin[static_cast<int64_t>(n) * (kFillRope / 2) + tid];
      const float a = p[kFillLat + 2 * tid], b = p[kFillLat + 2 * tid + 1];
      put_kv(kFillLat + tid, a * cs - b * sn);
      put_kv(kFillLat + kFillRope / 2 + tid, a * sn + b * cs);
    }
  }
  // indexer key row
  if constexpr (KDT == DSA_FP8_E4M3) {
    // the scale 2^e: the smallest e with 448 2^e >= max |z| (an all-zero row: e = 0)
    float amax = tid < kFillIdx ? fabsf(z) : 0.f;
    amax = wave_max(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(red[0], red[1]);
    const int e = ue8m0_exponent(amax);
    if (slot >= 0 && tid < kFillIdx) {
      static_cast<uint8_t*>(k_cache)[slot * kFillIdx + tid] =
          static_cast<uint8_t>(e4m3_code(ldexpf(z, -e)));
      if (tid == 0) k_sf[slot] = static_cast<uint8_t>(e + 127);
    }
  } else {
    if (slot >= 0 && tid < kFillIdx) {
      if constexpr (KDT == DSA_BF16)
        static_cast<uint16_t*>(k_cache)[slot * kFillIdx + tid] = f32_to_bf16(z);
      else
        static_cast<float*>(k_cache)[slot * kFillIdx + tid] = z;
    }
  }
  // head weights of the token's query
  if (tid < kFillW) {
    const float v = p[kFillLat + kFillRope + kFillIdx + tid];
    if constexpr (WDT == DSA_BF16)
      static_cast<uint16_t*>(w_out)[static_cast<int64_t>(n) * kFillW + tid] = f32_to_bf16(v);
    else
      static_cast<float*>(w_out)[static_cast<int64_t>(n) * kFillW + tid] = v;
  }
}

struct FillPlan {
  int row_blocks, slices, chunks_per_slice;
  bool skinny;
};

// ncols: outputs of the projection (a multiple of 128)
FillPlan fill_plan(int N, int D, int ncols) {
  FillPlan p;
  p.row_blocks = (N + kGemmRows - 1) / kGemmRows;
  const int nchunks = D / kGemmKStep;
  // few tokens (fewer 128 x 128 tiles than CUs): 32-output tiles, each
  // workgroup a kSkinnyWaves x kSkinnyChunks-chunk slice
  p.skinny = ((N + kTM - 1) / kTM) * (ncols / kTN) < device_info().cu_count;
  if (p.skinny) {
    p.chunks_per_slice = kSkinnyWaves * kSkinnyChunks;
    p.slices = (nchunks + p.chunks_per_slice - 1) / p.chunks_per_slice;
    return p;
  }
  // otherwise 128 x 128 tiles over the whole hidden dimension
  p.chunks_per_slice = nchunks;
  p.slices = 1;
  return p;
}

template <int KVDT, int KDT, int WDT>
dsa_status_t run_rows(int N, int slices, const float* part, const float* kv_gamma,
                      const float* k_gamma, const float* k_beta, const float* rope_cos,
                      const float* rope_sin, const int64_t* slots, void* kv_cache, void* k_cache,
                      uint8_t* k_sf, void* w_out, hipStream_t stream) {
  LaunchTimer timer;
  hipExtLaunchKernelGGL(fill_rows<KVDT, KDT, WDT>, dim3(N), dim3(256), 0, stream, timer.start(),
                        timer.stop(), 0, N, slices, part, kv_gamma, k_gamma, k_beta, rope_cos,
                        rope_sin, slots, kv_cache, k_cache, k_sf, w_out);
  return timer.done("fill_rows");
}

template <int KVDT, int KDT>
dsa_status_t run_rows_w(int wdt, int N, int slices, const float* part, const float* kv_gamma,
                        const float* k_gamma, const float* k_beta, const float* rope_cos,
                        const float* rope_sin, const int64_t* slots, void* kv_cache,
                        void* k_cache, uint8_t* k_sf, void* w_out, hipStream_t stream) {
  return wdt == DSA_BF16
             ? run_rows<KVDT, KDT, DSA_BF16>(N, slices, part, kv_gamma, k_gamma, k_beta, rope_cos,
                                             rope_sin, slots, kv_cache, k_cache, k_sf, w_out, stream)
             : run_rows<KVDT, KDT, DSA_F32>(N, slices, part, kv_gamma, k_gamma, k_beta, rope_cos,
                                            rope_sin, slots, kv_cache, k_cache, k_sf, w_out, stream);
}

// The indexer query of each token (Q^I = c^Q wq_b, the nnterp module
// tree's wq_b, 1536 -> 64 heads x 128): one wave per (token, head) adds the
// slices of its 128 outputs (two per lane) and writes them as bf16 / fp32,
// or as E4M3 codes with the head's ue8m0 scale (the quantiser of the keys).
constexpr int kQHeads = 64, kQDim = 128, kQCols = kQHeads * kQDim;  // 8192

template <int QDT>
__global__ void __launch_bounds__(256)
q_rows(int N, int slices, const float* __restrict__ part, void* __restrict__ q_out,
       uint8_t* __restrict__ q_sf) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t col = static_cast<int64_t>(h) * kQDim + 2 * lane;
  const float* src = part + static_cast<int64_t>(n) * kQCols + col;
  const int64_t stride = static_cast<int64_t>(N) * kQCols;
  float v0 = 0.f, v1 = 0.f;
  for (int sl = 0; sl < slices; ++sl) {  // slice order: deterministic
    v0 += src[sl * stride];
    v1 += src[sl * stride + 1];
  }
  const int64_t o = static_cast<int64_t>(n) * kQCols + col;
  if constexpr (QDT == DSA_FP8_E4M3) {
    const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const int e = ue8m0_exponent(amax);
    uint8_t* q = static_cast<uint8_t*>(q_out);
    q[o] = static_cast<uint8_t>(e4m3_code(ldexpf(v0, -e)));
    q[o + 1] = static_cast<uint8_t>(e4m3_code(ldexpf(v1, -e)));
    if (lane == 0) q_sf[static_cast<int64_t>(n) * kQHeads + h] = static_cast<uint8_t>(e + 127);
  } else if constexpr (QDT == DSA_BF16) {
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(q_out) + o)[0] = f32x2_to_bf16x2(v0, v1);
  } else {
    static_cast<float*>(q_out)[o] = v0;
    static_cast<float*>(q_out)[o + 1] = v1;
  }
}

size_t projection_workspace_bytes(int N, int D, int ncols, int batch = 1) {
  const FillPlan p = fill_plan(N, D, ncols * batch);
  return static_cast<size_t>(batch) * p.slices * N * ncols * sizeof(float);
}

// p = x W^T into fp32 partials (p.slices of them, [N, ncols] each), or, for
// out_dtype DSA_BF16 / DSA_F32 and one slice, straight into g.out
// 256-token tiles pay off with a long reduction (at least 16 chunks) and at
// least two workgroups per CU (measured: the output projection of 16384
// tokens 5047 -> 4146 us, the bf16 indexer query 660 -> 551 us; the cache
// fill's 384 workgroups and the 8-chunk absorbed output got slower)
template <int OUT>
bool wide_tiles(int N, int D, int ncols, int batch, const GemmOperands& g) {
  if (OUT == kOutPartial || g.rope_cos != nullptr || D < 16 * kGemmKStep) return false;
  const int64_t wgs = static_cast<int64_t>(ncols / kTN) * ((N + kWM - 1) / kWM) * batch;
  return wgs >= 2 * static_cast<int64_t>(device_info().cu_count);
}

template <int OUT>
dsa_status_t launch_projection_as(const FillPlan& p, int N, int D, int ncols, int batch,
                                  const GemmOperands& g, float* part, const char* name,
                                  hipStream_t stream) {
  LaunchTimer timer;
  if (p.skinny)
    hipExtLaunchKernelGGL(fill_gemm_skinny<OUT>, dim3(ncols / 32, p.row_blocks, batch * p.slices),
                          dim3(kSkinnyWaves * 64), 0, stream, timer.start(), timer.stop(), 0, N, D,
                          ncols, p.slices, g, part);
  else if (wide_tiles<OUT>(N, D, ncols, batch, g))
    hipExtLaunchKernelGGL(fill_gemm_wide<OUT>, dim3(ncols / kTN, (N + kWM - 1) / kWM, batch),
                          dim3(256), 0, stream, timer.start(), timer.stop(), 0, N, D, ncols, g,
                          part);
  else
    hipExtLaunchKernelGGL((fill_gemm_tiled<OUT, 2>), dim3(ncols / kTN, (N + kTM - 1) / kTM, batch),
                          dim3(256), 0, stream, timer.start(), timer.stop(), 0, N, D, ncols, g,
                          part);
  return timer.done(name);
}

dsa_status_t launch_projection(const FillPlan& p, int N, int D, int ncols, int batch,
                               const GemmOperands& g, float* part, const char* name,
                               hipStream_t stream, int out_dtype = kOutPartial) {
  if (out_dtype != kOutPartial && p.slices != 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: a direct output needs one slice, the plan has %d", name,
                p.slices);
  if (out_dtype == DSA_BF16)
    return launch_projection_as<DSA_BF16>(p, N, D, ncols, batch, g, part, name, stream);
  if (out_dtype == DSA_F32)
    return launch_projection_as<DSA_F32>(p, N, D, ncols, batch, g, part, name, stream);
  return launch_projection_as<kOutPartial>(p, N, D, ncols, batch, g, part, name, stream);
}

// one projection of a batch of 1: x [N, D], W [ncols, D]
GemmOperands plain(const void* x, const void* W, int D) {
  return GemmOperands{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), D, 0, 0,
                      nullptr, 0, 0, nullptr, nullptr, nullptr, 0, 0};
}

// ---------------------------------------------------------------------------
// Absorption products either side of the sparse attention (the step list of
// the atlas.klimoza.dev DeepSeek-V3.2-Exp page: k^C = c^KV W_UK, v = c^KV
// W_UV; kv_b_proj 512 -> 128 heads x (128 + 128) and o_proj 16384 -> 7168
// in the nnterp module tree).  Absorbed, head h's query meets the latent
// rows through q_lat,h = W_UK,h q^C_h and its output leaves through
// W_UV,h o_lat,h, then wo.  kv_b_proj's Linear rows come per head: rows
// 256 h .. 256 h + 127 are W_UK,h (key dims), the next 128 W_UV,h.
constexpr int kLat = 512, kNope = 128, kVDim = 128, kQRope = 64;
constexpr int kQbDim = kNope + kQRope;       // 192: q_b_proj's per-head output
constexpr int kQDimOut = kLat + kQRope;      // 576: the sparse attention's query
constexpr int kKvbRows = kNope + kVDim;      // 256 kv_b_proj rows per head

// W_UK,h in reduction-contiguous form: wuk_t[h][c][e] = kv_b[256 h + e][c].
// Workgroup = 64 latent columns of one head: the 128 x 64 block goes through
// LDS (rows padded by 4 bytes), then out as 64 rows of 128 elements.
__global__ void __launch_bounds__(256)
uk_transpose(const uint16_t* __restrict__ kvb, uint16_t* __restrict__ wuk_t) {
  __shared__ uint16_t tile[kNope][64 + 2];
  const int h = blockIdx.y, c0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const uint16_t* src = kvb + static_cast<int64_t>(h) * kKvbRows * kLat + c0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // 128 rows x 8 pieces of 8 elements
    const int piece = tid + 256 * k;
    const int e = piece >> 3, c = (piece & 7) * 8;
    const u32x4v_t v = *reinterpret_cast<const u32x4v_t*>(src + static_cast<int64_t>(e) * kLat + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      tile[e][c + 2 * u] = static_cast<uint16_t>(v[u]);
      tile[e][c + 2 * u + 1] = static_cast<uint16_t>(v[u] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = wuk_t + (static_cast<int64_t>(h) * kLat + c0) * kNope;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // 64 rows x 16 pieces
    const int piece = tid + 256 * k;
    const int c = piece >> 4, e = (piece & 15) * 8;
    u32x4v_t v;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = static_cast<uint32_t>(tile[e + 2 * u][c]) | (static_cast<uint32_t>(tile[e + 2 * u + 1][c]) << 16);
    *reinterpret_cast<u32x4v_t*>(dst + static_cast<int64_t>(c) * kNope + e) = v;
  }
}

// The rotary part of the absorbed query: pair (2i, 2i + 1) of the head's
// q^pe turned by the token's angle i into dims 512 + i and 544 + i (the
// layout of the cached rotary key, so that q and k share it).  One thread
// per (token, head, pair).
template <int ODT>
__global__ void __launch_bounds__(256)
q_rope(int N, int H, const uint16_t* __restrict__ qb, const float* __restrict__ rope_cos,
       const float* __restrict__ rope_sin, void* __restrict__ q) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= static_cast<int64_t>(N) * H * (kQRope / 2)) return;
  const int i = static_cast<int>(id & 31);
  const int64_t nh = id >> 5;
  const int n = static_cast<int>(nh / H);
  const uint32_t pr = *reinterpret_cast<const uint32_t*>(qb + nh * kQbDim + kNope + 2 * i);
  const float a = bf16_to_f32(static_cast<uint16_t>(pr)), b = bf16_to_f32(static_cast<uint16_t>(pr >> 16));
  const float c = rope_cos[static_cast<int64_t>(n) * 32 + i], sn = rope_sin[static_cast<int64_t>(n) * 32 + i];
  const float r0 = a * c - b * sn, r1 = a * sn + b * c;
  const int64_t o = nh * kQDimOut + kLat + i;
  if constexpr (ODT == DSA_BF16) {
    static_cast<uint16_t*>(q)[o] = f32_to_bf16(r0);
    static_cast<uint16_t*>(q)[o + kQRope / 2] = f32_to_bf16(r1);
  } else {
    static_cast<float*>(q)[o] = r0;
    static_cast<float*>(q)[o + kQRope / 2] = r1;
  }
}

// out[t, j] = sum of the partials in slice order (deterministic); one thread
// per 4 outputs
template <int ODT>
__global__ void __launch_bounds__(256)
gemm_finish(int N, int ncols, int slices, const float* __restrict__ part, void* __restrict__ out) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(N) * ncols;
  if (4 * id >= total) return;
  const float4* src = reinterpret_cast<const float4*>(part) + id;
  const int64_t stride = total / 4;
  float4 v = src[0];
  for (int sl = 1; sl < slices; ++sl) {
    const float4 u = src[sl * stride];
    v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
  }
  if constexpr (ODT == DSA_BF16) {
    uint2 r;
    r.x = f32x2_to_bf16x2(v.x, v.y);
    r.y = f32x2_to_bf16x2(v.z, v.w);
    reinterpret_cast<uint2*>(out)[id] = r;
  } else {
    reinterpret_cast<float4*>(out)[id] = v;
  }
}

template <int ODT>
dsa_status_t run_q_rope(int N, int H, const void* qb, const float* rope_cos, const float* rope_sin,
                        void* q, hipStream_t stream) {
  LaunchTimer timer;
  const int64_t threads = static_cast<int64_t>(N) * H * (kQRope / 2);
  hipExtLaunchKernelGGL(q_rope<ODT>, dim3(static_cast<uint32_t>((threads + 255) / 256)), dim3(256), 0,
                        stream, timer.start(), timer.stop(), 0, N, H,
                        static_cast<const uint16_t*>(qb), rope_cos, rope_sin, q);
  return timer.done("q_rope");
}

}  // namespace

dsa_status_t launch_absorb_prepare(int H, const void* kv_b, void* wuk_t, hipStream_t stream) {
  if (H == 0) return DSA_OK;
  LaunchTimer timer;
  hipExtLaunchKernelGGL(uk_transpose, dim3(kLat / 64, H), dim3(256), 0, stream, timer.start(),
                        timer.stop(), 0, static_cast<const uint16_t*>(kv_b),
                        static_cast<uint16_t*>(wuk_t));
  return timer.done("uk_transpose");
}

dsa_status_t launch_absorb_query(int N, int H, const void* qb, const void* wuk_t,
                                 const float* rope_cos, const float* rope_sin, int q_dtype, void* q,
                                 hipStream_t stream) {
  if (N == 0 || H == 0) return DSA_OK;
  // per head: [N, 128] x [128 -> 512], written into q[:, h, 0:512]
  const GemmOperands g{static_cast<const uint16_t*>(qb), static_cast<const uint16_t*>(wuk_t),
                       static_cast<int64_t>(H) * kQbDim, kQbDim,
                       static_cast<int64_t>(kLat) * kNope, q,
                       static_cast<int64_t>(H) * kQDimOut, kQDimOut};
  const FillPlan p = fill_plan(N, kNope, kLat * H);
  static_assert(kLat / 128 * 8 == kQRope / 2, "the tiled kernel's 4 output tiles take 8 pairs each");
  // few tokens: the tiled kernel turns the rotary part too (one launch less:
  // 7.9 us against 7.7 + 4.4 for 32 tokens); for many tokens the extra loads
  // in every workgroup's epilogue cost more than the separate pass (16384
  // tokens: 1246 us against 858 + 190)
  constexpr int kFuseRopeTokens = 1024;
  if (!p.skinny && N <= kFuseRopeTokens) {
    GemmOperands gr = g;
    gr.rope_cos = rope_cos;
    gr.rope_sin = rope_sin;
    gr.rope_at = kNope;
    gr.rope_to = kLat;
    return launch_projection(p, N, kNope, kLat, H, gr, nullptr, "absorb_q_gemm", stream, q_dtype);
  }
  dsa_status_t st = launch_projection(p, N, kNope, kLat, H, g, nullptr, "absorb_q_gemm", stream, q_dtype);
  if (st != DSA_OK) return st;
  return q_dtype == DSA_BF16 ? run_q_rope<DSA_BF16>(N, H, qb, rope_cos, rope_sin, q, stream)
                             : run_q_rope<DSA_F32>(N, H, qb, rope_cos, rope_sin, q, stream);
}

dsa_status_t launch_absorb_output(int N, int H, const void* o_lat, const void* kv_b, int out_dtype,
                                  void* premix, hipStream_t stream) {
  if (N == 0 || H == 0) return DSA_OK;
  // per head: [N, 512] x [512 -> 128] with W_UV,h = kv_b rows 256 h + 128 ..
  const GemmOperands g{static_cast<const uint16_t*>(o_lat),
                       static_cast<const uint16_t*>(kv_b) + static_cast<int64_t>(kNope) * kLat,
                       static_cast<int64_t>(H) * kLat, kLat,
                       static_cast<int64_t>(kKvbRows) * kLat, premix,
                       static_cast<int64_t>(H) * kVDim, kVDim};
  const FillPlan p = fill_plan(N, kLat, kVDim * H);
  return launch_projection(p, N, kLat, kVDim, H, g, nullptr, "absorb_o_gemm", stream, out_dtype);
}

size_t output_projection_workspace_bytes(int N, int Din, int Dout) {
  const FillPlan p = fill_plan(N, Din, Dout);
  return p.slices > 1 ? projection_workspace_bytes(N, Din, Dout) : 0;
}

dsa_status_t launch_output_projection(int N, int Din, int Dout, const void* premix, const void* wo,
                                      int out_dtype, void* out, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  if (N == 0) return DSA_OK;
  const FillPlan p = fill_plan(N, Din, Dout);
  GemmOperands g = plain(premix, wo, Din);
  if (p.slices == 1) {
    g.out = out;
    g.ldo = Dout;
    return launch_projection(p, N, Din, Dout, 1, g, nullptr, "wo_gemm", stream, out_dtype);
  }
  const size_t need = projection_workspace_bytes(N, Din, Dout);
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "output projection: workspace of %zu bytes needed, %zu given",
                need, ws_bytes);
  float* part = static_cast<float*>(ws);
  dsa_status_t st = launch_projection(p, N, Din, Dout, 1, g, part, "wo_gemm", stream);
  if (st != DSA_OK) return st;
  LaunchTimer timer;
  const int64_t threads = static_cast<int64_t>(N) * Dout / 4;
  const dim3 grid(static_cast<uint32_t>((threads + 255) / 256));
  if (out_dtype == DSA_BF16)
    hipExtLaunchKernelGGL(gemm_finish<DSA_BF16>, grid, dim3(256), 0, stream, timer.start(),
                          timer.stop(), 0, N, Dout, p.slices, part, out);
  else
    hipExtLaunchKernelGGL(gemm_finish<DSA_F32>, grid, dim3(256), 0, stream, timer.start(),
                          timer.stop(), 0, N, Dout, p.slices, part, out);
  return timer.done("wo_finish");
}

size_t cache_fill_workspace_bytes(int N, int D) { return projection_workspace_bytes(N, D, kFillCols); }

size_t indexer_query_workspace_bytes(int N, int Dq) {
  // many tokens: the tiled kernel writes the query itself (no partials)
  return fill_plan(N, Dq, kQCols).skinny ? projection_workspace_bytes(N, Dq, kQCols) : 0;
}

dsa_status_t launch_cache_fill(int N, int D, const void* x, const void* W, const float* kv_gamma,
                               const float* k_gamma, const float* k_beta, const float* rope_cos,
                               const float* rope_sin, const int64_t* slots, int kv_dtype,
                               void* kv_cache, int k_dtype, void* k_cache, uint8_t* k_sf,
                               int w_dtype, void* w_out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (N == 0) return DSA_OK;
  const FillPlan p = fill_plan(N, D, kFillCols);
  const size_t need = projection_workspace_bytes(N, D, kFillCols);
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "cache fill: workspace of %zu bytes needed, %zu given", need,
                ws_bytes);
  float* part = static_cast<float*>(ws);
  {
    const dsa_status_t st =
        launch_projection(p, N, D, kFillCols, 1, plain(x, W, D), part, "fill_gemm", stream);
    if (st != DSA_OK) return st;
  }
#define DSA_FILL_ROWS(KV, K)                                                                    \
  run_rows_w<KV, K>(w_dtype, N, p.slices, part, kv_gamma, k_gamma, k_beta, rope_cos, rope_sin, \
                    slots, kv_cache, k_cache, k_sf, w_out, stream)
  if (kv_dtype == DSA_BF16) {
    if (k_dtype == DSA_FP8_E4M3) return DSA_FILL_ROWS(DSA_BF16, DSA_FP8_E4M3);
    if (k_dtype == DSA_BF16) return DSA_FILL_ROWS(DSA_BF16, DSA_BF16);
    return DSA_FILL_ROWS(DSA_BF16, DSA_F32);
  }
  if (k_dtype == DSA_FP8_E4M3) return DSA_FILL_ROWS(DSA_F32, DSA_FP8_E4M3);
  if (k_dtype == DSA_BF16) return DSA_FILL_ROWS(DSA_F32, DSA_BF16);
  return DSA_FILL_ROWS(DSA_F32, DSA_F32);
#undef DSA_FILL_ROWS
}

dsa_status_t launch_indexer_query(int N, int Dq, const void* cq, const void* wq_b, int q_dtype,
                                  void* q_out, uint8_t* q_sf, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (N == 0) return DSA_OK;
  const FillPlan p = fill_plan(N, Dq, kQCols);
  if (!p.skinny) {
    // one 128-output tile = one head: the tiled kernel writes the finished
    // query (E4M3 codes and the head's scale, or bf16 / fp32) itself
    GemmOperands g = plain(cq, wq_b, Dq);
    g.out = q_out;
    g.ldo = kQCols;
    g.out_sf = q_sf;
    if (q_dtype != DSA_FP8_E4M3)
      return launch_projection(p, N, Dq, kQCols, 1, g, nullptr, "q_gemm", stream, q_dtype);
    LaunchTimer timer;
    if (wide_tiles<DSA_FP8_E4M3>(N, Dq, kQCols, 1, g)) {
      hipExtLaunchKernelGGL(fill_gemm_wide<DSA_FP8_E4M3>, dim3(kQCols / kTN, (N + kWM - 1) / kWM, 1),
                            dim3(256), 0, stream, timer.start(), timer.stop(), 0, N, Dq, kQCols, g, nullptr);
      return timer.done("q_gemm");
    }
    const dim3 grid(kQCols / kTN, (N + kTM - 1) / kTM, 1);
    hipExtLaunchKernelGGL((fill_gemm_tiled<DSA_FP8_E4M3, 2>), grid, dim3(256), 0, stream,
                          timer.start(), timer.stop(), 0, N, Dq, kQCols, g, nullptr);
    return timer.done("q_gemm");
  }
  const size_t need = projection_workspace_bytes(N, Dq, kQCols);
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "indexer query: workspace of %zu bytes needed, %zu given",
                need, ws_bytes);
  float* part = static_cast<float*>(ws);
  dsa_status_t st = launch_projection(p, N, Dq, kQCols, 1, plain(cq, wq_b, Dq), part, "q_gemm", stream);
  if (st != DSA_OK) return st;
  LaunchTimer timer;
  const dim3 grid(N, kQHeads / 4);
  if (q_dtype == DSA_FP8_E4M3)
    hipExtLaunchKernelGGL(q_rows<DSA_FP8_E4M3>, grid, dim3(256), 0, stream, timer.start(),
                          timer.stop(), 0, N, p.slices, part, q_out, q_sf);
  else if (q_dtype == DSA_BF16)
    hipExtLaunchKernelGGL(q_rows<DSA_BF16>, grid, dim3(256), 0, stream, timer.start(),
                          timer.stop(), 0, N, p.slices, part, q_out, q_sf);
  else
    hipExtLaunchKernelGGL(q_rows<DSA_F32>, grid, dim3(256), 0, stream, timer.start(),
                          timer.stop(), 0, N, p.slices, part, q_out, q_sf);
  return timer.done("q_rows");
}

}  // namespace dsa
