// Device-side checks of index rows for debug builds (-DDSA_DEBUG); other
// builds compile nothing from this file.
//
// The top-K rows (the M^sel step of the atlas DeepSeek-V3.2-Exp MoE-block
// step list) hold min(K, keys) int32 entries, ascending, padded with -1 (the
// nnterp deepseek_v32 page, section 03).  Caller-written rows given to the
// attention may hold -1 anywhere and repeat entries; entries outside [0, S)
// other than -1 are skipped by the release build and rejected by this one.
#include "dsa_device.h"
#include "dsa_internal.h"

#ifdef DSA_DEBUG
namespace dsa {
namespace {

// [0]: entries outside [-1, S); [1]: order violations (sorted rows only)
__device__ unsigned int g_idx_bad[2];

__global__ void debug_idx_clear() {
  if (threadIdx.x < 2) g_idx_bad[threadIdx.x] = 0u;
}

__global__ void __launch_bounds__(256)
debug_idx_scan(int64_t n, int W, int S, int sorted, const int32_t* __restrict__ idx) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t v = idx[i];
  if (v < -1 || v >= S) atomicAdd(&g_idx_bad[0], 1u);
  if (sorted && i % W != 0) {
    const int32_t u = idx[i - 1];
    if (v != -1 && (u == -1 || u >= v)) atomicAdd(&g_idx_bad[1], 1u);
  }
}

}  // namespace

dsa_status_t debug_check_idx(int64_t rows, int W, int S, bool sorted, const int32_t* idx,
                             hipStream_t stream, const char* what) {
  const int64_t n = rows * W;
  if (n == 0) return DSA_OK;
  hipLaunchKernelGGL(debug_idx_clear, dim3(1), dim3(64), 0, stream);
  hipLaunchKernelGGL(debug_idx_scan, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, n, W,
                     S, sorted ? 1 : 0, idx);
  dsa_status_t st = check_launch("debug_idx_scan");
  if (st != DSA_OK) return st;
  unsigned int bad[2] = {0u, 0u};
  if (hipMemcpyFromSymbolAsync(bad, HIP_SYMBOL(g_idx_bad), sizeof(bad), 0, hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(DSA_ERR_HIP, "debug check of %s: %s", what, hipGetErrorString(hipGetLastError()));
  if (bad[0] != 0u || bad[1] != 0u)
    return fail(DSA_ERR_INVALID_ARG, "debug check of %s: %u entries outside [-1, %d), %u out of order", what,
                bad[0], S, bad[1]);
  return DSA_OK;
}

}  // namespace dsa
#endif
