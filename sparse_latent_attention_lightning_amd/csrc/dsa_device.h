// Device-side helpers shared by the libdsa kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): gfx950 converts
// in hardware (v_cvt_pk_bf16_f32), branch-free
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// two fp32 -> packed bf16 pair (low half = a), round to nearest even
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// OCP E4M3FN byte -> fp32 (exact); used by the generic kernels only.
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xfu;
  const uint32_t m = c & 0x7u;
  if (e == 0xfu && m == 0x7u) return __uint_as_float(0x7fc00000u);
  float v;
  if (e == 0)
    v = static_cast<float>(m) * 0.001953125f;  // m/8 * 2^-6
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1+m/8)*2^(e-7)
  return __uint_as_float(__float_as_uint(v) | s);
}

// ue8m0 scale byte -> 2^(byte-127) as fp32 (bytes 0 and 255 are not used by
// the block quantiser; 0 maps to 2^-127 (a subnormal), 255 to NaN).
__device__ __forceinline__ float ue8m0_to_f32(uint8_t b) {
  if (b == 0xffu) return __uint_as_float(0x7fc00000u);
  if (b == 0) return __uint_as_float(0x00400000u);
  return __uint_as_float(static_cast<uint32_t>(b) << 23);
}

// Workgroups of one launch that meet through words of the caller's
// workspace tag those words with the call's own 39-bit tag; a word holding
// another tag is stale and counts as zero.  The meeting's last workgroup
// marks the words stale (tag with bit 39 set) so that a replay of the same
// call starts afresh.  A workgroup that waits for another, already running,
// one polls at most kSelWaitSpins rounds of about 256 cycles.
constexpr uint64_t kTagStale = uint64_t(1) << 39;
constexpr int kSelWaitSpins = 1 << 20;

// Order-preserving key of an fp32 score: larger score -> larger key.
// -0 is folded into +0; NaN and -inf map to 0, which no selectable score
// reaches (the smallest selectable key, that of -FLT_MAX, is 0x00800000).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                      // -0 -> +0
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;    // NaN
  if (u == 0xff800000u) return 0u;                   // -inf
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves (no
// LDS round trips): shifts by 1, 2, 4 and 8 lanes within each 16-lane row
// (lanes shifted in from outside the row add 0), then the row totals are
// broadcast forward (lane 15 of rows 0 and 2 into rows 1 and 3, lane 31 into
// rows 2 and 3; rows outside the row mask keep `old` = 0 and add nothing)
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 1, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 2, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 4, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowShr + 8, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowBcast15, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, kRowBcast31, 0xc, 0xf, false);
  return v;
}

// Butterfly steps across lane distance 16 and 32 on the VALU (v_permlane16_swap
// / v_permlane32_swap with both operands the same value: each lane ends with
// its own value and its partner's, in some order, so any symmetric op works).
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Debug builds (-DDSA_DEBUG): fill an LDS buffer with 0xff bytes before its
// first use (NaN as bf16 or fp32, -1 as int32: a skipped key), so that a read
// of LDS nothing wrote shows up in the results.  Every thread of the
// workgroup calls it; it ends with a barrier.  Other builds: nothing.
template <int BYTES>
__device__ __forceinline__ void debug_poison_lds(void* p) {
#ifdef DSA_DEBUG
  static_assert(BYTES % 16 == 0, "whole 16-byte pieces");
  u32x4_t* q = static_cast<u32x4_t*>(p);
  for (int i = threadIdx.x; i < BYTES / 16; i += blockDim.x) q[i] = u32x4_t{~0u, ~0u, ~0u, ~0u};
  __syncthreads();
#else
  (void)p;
#endif
}

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
// uses and the kernels that call this have no other, so the reserved-register
// warning is moot.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma_16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
// The same copy with the nontemporal hint: data streamed once does not
// displace cached data of the kernels that follow.
__device__ __forceinline__ void lds_dma_16_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
// 4-byte global -> LDS copy per lane: lane l writes LDS [lds + 4 l] (the
// source 4-byte aligned; lanes outside exec copy nothing).  Counted like the
// 16-byte copies.
__device__ __forceinline__ void lds_dma_4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
// The same copy from a wave-uniform 64-bit base plus a 32-bit per-lane byte
// offset (the saddr form: no 64-bit address arithmetic per lane).
__device__ __forceinline__ void lds_dma_16_sbase(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ f32x4_t mfma16x16x32_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                                     const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// gfx950's 16x16x128 product of OCP e4m3 operands (format 0 for both, unit
// E8M0 scales 127): lane (g, n) supplies 32 bytes of row n of each operand;
// C as for every 16x16 product (lane (g, n): rows 4 g .. 4 g + 3, column n)
__device__ __forceinline__ f32x4_t mfma16x16x128_e4m3(const i32x8_t& a, const i32x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ f32x4_t mfma16x16x32_fp8(long a, long b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

}  // namespace dsa
