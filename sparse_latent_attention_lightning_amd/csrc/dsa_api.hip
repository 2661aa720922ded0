// libdsa C ABI: argument validation, dispatch and workspace layout.
// The operations are defined in include/dsa.h (with the passages of the pages
// each one follows); the kernels live in indexer.hip, topk.hip and
// sparse_mla.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <random>
#include <utility>
#include <vector>

#include "dsa.h"
#include "dsa_internal.h"

namespace dsa {

namespace {
thread_local char g_last_error[512] = "";

constexpr size_t kAlign = 256;  // workspace sub-buffers start on 256-byte boundaries

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_bytes(int32_t dt) {
  switch (dt) {
    case DSA_F32: return 4;
    case DSA_BF16: return 2;
    case DSA_FP8_E4M3: return 1;
  }
  return 0;
}

dsa_status_t check_shape(const dsa_shape_t* s) {
  if (s == nullptr) return fail(DSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B <= 0 || s->T <= 0 || s->S <= 0)
    return fail(DSA_ERR_INVALID_ARG, "B, T, S must be positive (got %d, %d, %d)", s->B, s->T, s->S);
  if (s->T > s->S) return fail(DSA_ERR_INVALID_ARG, "T = %d exceeds S = %d", s->T, s->S);
  if (s->HI <= 0 || s->DI <= 0) return fail(DSA_ERR_INVALID_ARG, "HI and DI must be positive");
  if (s->H <= 0 || s->Dc <= 0 || s->Dr < 0)
    return fail(DSA_ERR_INVALID_ARG, "H and Dc must be positive and Dr non-negative");
  if (s->K <= 0) return fail(DSA_ERR_INVALID_ARG, "K must be positive (got %d)", s->K);
  if (s->idx_dtype != DSA_F32 && s->idx_dtype != DSA_BF16 && s->idx_dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_INVALID_ARG, "unknown idx_dtype %d", s->idx_dtype);
  if (s->w_dtype != DSA_F32 && s->w_dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "w_dtype must be F32 or BF16 (got %d)", s->w_dtype);
  if (s->mla_dtype != DSA_F32 && s->mla_dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "mla_dtype must be F32 or BF16 (got %d)", s->mla_dtype);
  if (s->idx_dtype == DSA_FP8_E4M3 && s->DI % 128 != 0)
    return fail(DSA_ERR_INVALID_ARG, "fp8 indexer needs DI %% 128 == 0 (got %d)", s->DI);
  const int64_t rows = static_cast<int64_t>(s->B) * s->T;
  if (rows * s->S > (int64_t(1) << 40))
    return fail(DSA_ERR_UNSUPPORTED, "B*T*S too large");
  if ((static_cast<int64_t>(s->Dc + s->Dr) * dtype_bytes(s->mla_dtype)) % 16 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "(Dc + Dr) rows must be a multiple of 16 bytes");
  return DSA_OK;
}

dsa_status_t need(const void* p, const char* name) {
  if (p == nullptr) return fail(DSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return DSA_OK;
}

dsa_status_t check_indexer_args(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                                const void* k_idx, const uint8_t* k_sf, const void* w,
                                const float* scores) {
  dsa_status_t st;
  if ((st = need(q_idx, "q_idx")) || (st = need(k_idx, "k_idx")) || (st = need(w, "w")) ||
      (st = need(scores, "scores")))
    return st;
  if (s.idx_dtype == DSA_FP8_E4M3) {
    if (q_sf == nullptr || k_sf == nullptr)
      return fail(DSA_ERR_INVALID_ARG, "fp8 indexer needs q_sf and k_sf");
  }
  return DSA_OK;
}

// context lengths of a ragged batch: nullable (all S); else 4-byte aligned
dsa_status_t check_seq_lens(const int32_t* seq_lens) {
  if (seq_lens != nullptr && (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0)
    return fail(DSA_ERR_INVALID_ARG, "seq_lens is not 4-byte aligned");
  return DSA_OK;
}

dsa_status_t check_mla_args(const void* q, const void* kv, const int32_t* idx, const void* o) {
  dsa_status_t st;
  if ((st = need(q, "q")) || (st = need(kv, "kv")) || (st = need(idx, "idx")) ||
      (st = need(o, "o")))
    return st;
  return DSA_OK;
}

// dsa_forward's workspace: the scores, the selection (when idx_out is NULL),
// the top-K's scratch, then the attention's scratch
struct ForwardLayout {
  size_t scores, idx, topk_ws, mla_ws, total;
};

ForwardLayout forward_layout(const dsa_shape_t& s) {
  const size_t rows = static_cast<size_t>(s.B) * s.T;
  ForwardLayout L{};
  L.scores = 0;
  L.idx = align_up(rows * s.S * sizeof(float));
  L.topk_ws = L.idx + align_up(rows * k_eff(s) * sizeof(int32_t));
  L.mla_ws = L.topk_ws + align_up(topk_workspace_bytes(s));
  L.total = L.mla_ws + align_up(mla_workspace_bytes(s));
  return L;
}

// dsa_indexer_topk's workspace: the scores, then the per-row state
size_t indexer_topk_scores_bytes(const dsa_shape_t& s) {
  return align_up(static_cast<size_t>(s.B) * s.T * s.S * sizeof(float));
}
size_t indexer_topk_total_bytes(const dsa_shape_t& s) {
  return indexer_topk_scores_bytes(s) + align_up(indexer_select_workspace_bytes(s));
}

}  // namespace

// A tag per call of a launch whose workgroups meet through the workspace:
// distinct across calls of this process (a random start plus a counter), 39 bits.
uint64_t next_call_tag() {
  static std::atomic<uint64_t> counter{0};
  static const uint64_t salt = [] {
    std::random_device rd;
    return (static_cast<uint64_t>(rd()) << 32) ^ rd();
  }();
  return (salt + counter.fetch_add(1, std::memory_order_relaxed)) & ((uint64_t(1) << 39) - 1);
}

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

dsa_status_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DSA_OK;
}

size_t forward_workspace_bytes(const dsa_shape_t& s) { return forward_layout(s).total; }

// The whole path on a workspace of forward_workspace_bytes(s) bytes at `base`
// (the shape is checked, the workspace size is the caller's business).
dsa_status_t forward_on(const dsa_shape_t& s, const int32_t* seq_lens, const void* q_idx,
                        const uint8_t* q_sf, const void* k_idx, const uint8_t* k_sf, const void* w,
                        const void* q, const void* kv, int32_t* idx_out, void* o, float* lse,
                        char* base, hipStream_t hs) {
  dsa_status_t st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  const ForwardLayout L = forward_layout(s);
  float* scores = reinterpret_cast<float*>(base + L.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + L.idx);
  if ((st = check_indexer_args(s, q_idx, q_sf, k_idx, k_sf, w, scores)) != DSA_OK) return st;
  if ((st = check_mla_args(q, kv, idx, o)) != DSA_OK) return st;
  // every step's shape limits before the first launch: a failing call enqueues nothing
  if ((st = topk_check(s)) != DSA_OK || (st = mla_check(s)) != DSA_OK) return st;
  // the scores stay in the workspace: the top-K ignores each row past its
  // query's position, so the indexer need not write the keys there
  if ((st = launch_indexer(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, false, hs)) != DSA_OK)
    return st;
  if ((st = launch_topk(s, scores, seq_lens, true, idx, base + L.topk_ws, L.mla_ws - L.topk_ws, hs)) !=
      DSA_OK)
    return st;
  return launch_sparse_mla(s, q, kv, idx, o, lse, base + L.mla_ws, L.total - L.mla_ws, hs);
}

// ---- the library's own scratch memory (dsa_forward_noalloc) ---------------
// A file-scope device array: every GPU the library runs on holds its own copy
// (kNoallocScratchBytes) from the library's load until the process ends.  In
// host code `noalloc_scratch` names only a host-side stand-in; the device
// address of a GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is handed to
// kernels.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t noalloc_scratch[kNoallocScratchBytes];

namespace {
// the device address of `noalloc_scratch` on the current device (nullptr and
// the error recorded when the runtime cannot give it)
char* noalloc_scratch_ptr() {
  static std::mutex mu;
  static std::vector<char*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    fail(DSA_ERR_HIP, "forward_noalloc: hipGetDevice failed");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<size_t>(dev) >= ptrs.size()) ptrs.resize(dev + 1, nullptr);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (e != hipSuccess || p == nullptr) {
      fail(DSA_ERR_HIP, "forward_noalloc: hipGetSymbolAddress of the scratch array: %s",
           hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = static_cast<char*>(p);
  }
  return ptrs[dev];
}
}  // namespace

// ---- kernel timing sessions ----------------------------------------------
namespace {
constexpr size_t kTimingCap = 65536;

struct TimedLaunch {
  const char* name;  // set by done(); nullptr while the launch is being enqueued
  hipEvent_t start, stop;
};

struct TimingSession {
  std::mutex mu;
  std::atomic<bool> active{false};
  long generation = 0;
  std::vector<TimedLaunch> launches;
  std::vector<hipEvent_t> pool;  // 2 events per launch slot, reused across sessions
  std::vector<std::pair<const char*, int>> dropped;
};

TimingSession& timing() {
  static TimingSession t;
  return t;
}
}  // namespace

LaunchTimer::LaunchTimer() {
  TimingSession& T = timing();
  if (!T.active.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lock(T.mu);
  if (!T.active.load(std::memory_order_relaxed)) return;
  gen_ = T.generation;
  if (T.launches.size() >= kTimingCap) {
    slot_ = -2;  // counted in done()
    return;
  }
  const size_t i = T.launches.size();
  while (T.pool.size() < 2 * (i + 1)) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    T.pool.push_back(e);
  }
  TimedLaunch rec{nullptr, T.pool[2 * i], T.pool[2 * i + 1]};
  T.launches.push_back(rec);
  start_ = rec.start;
  stop_ = rec.stop;
  slot_ = static_cast<long>(i);
}

dsa_status_t LaunchTimer::done(const char* what) {
  const dsa_status_t st = check_launch(what);
  if (slot_ == -1) return st;
  TimingSession& T = timing();
  std::lock_guard<std::mutex> lock(T.mu);
  if (!T.active.load(std::memory_order_relaxed) || gen_ != T.generation) return st;
  if (slot_ == -2) {
    for (auto& d : T.dropped)
      if (d.first == what) {
        ++d.second;
        return st;
      }
    T.dropped.emplace_back(what, 1);
    return st;
  }
  if (st == DSA_OK) T.launches[static_cast<size_t>(slot_)].name = what;
  return st;
}

const DeviceInfo& device_info() {
  static std::mutex mu;
  static std::vector<DeviceInfo> cache;
  static std::vector<bool> have;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<size_t>(dev) >= cache.size()) {
    cache.resize(dev + 1);
    have.resize(dev + 1, false);
  }
  if (!have[dev]) {
    hipDeviceProp_t p{};
    DeviceInfo info{256, 160 * 1024};
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
      info.cu_count = p.multiProcessorCount;
      info.max_lds = p.sharedMemPerBlock;
    }
    cache[dev] = info;
    have[dev] = true;
  }
  return cache[dev];
}

}  // namespace dsa

using namespace dsa;

extern "C" {

dsa_status_t dsa_indexer_scores_ragged(const dsa_shape_t* shape, const int32_t* seq_lens,
                                       const void* q_idx, const uint8_t* q_sf,
                                       const void* k_idx, const uint8_t* k_sf, const void* w,
                                       float* scores, void* stream) {
  g_last_error[0] = '\0';
  dsa_status_t st = check_shape(shape);
  if (st != DSA_OK) return st;
  if ((st = check_indexer_args(*shape, q_idx, q_sf, k_idx, k_sf, w, scores)) != DSA_OK) return st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  return launch_indexer(*shape, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, true,
                        static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_indexer_scores(const dsa_shape_t* shape, const void* q_idx, const uint8_t* q_sf,
                                const void* k_idx, const uint8_t* k_sf, const void* w,
                                float* scores, void* stream) {
  return dsa_indexer_scores_ragged(shape, nullptr, q_idx, q_sf, k_idx, k_sf, w, scores, stream);
}

dsa_status_t dsa_topk(const dsa_shape_t* shape, const float* scores, int32_t* idx, void* ws,
                      size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  dsa_status_t st = check_shape(shape);
  if (st != DSA_OK) return st;
  if ((st = need(scores, "scores")) || (st = need(idx, "idx"))) return st;
  if (ws != nullptr && !aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  return launch_topk(*shape, scores, nullptr, false, idx, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_indexer_topk(const dsa_shape_t* shape, const int32_t* seq_lens,
                              const void* q_idx, const uint8_t* q_sf, const void* k_idx,
                              const uint8_t* k_sf, const void* w, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  dsa_status_t st = check_shape(shape);
  if (st != DSA_OK) return st;
  const dsa_shape_t& s = *shape;
  if (!indexer_select_applies(s))
    return fail(DSA_ERR_UNSUPPORTED,
                "indexer_topk: covers HI = 64, DI = 128, BF16 or FP8 keys, T < 8 and S <= 262144 "
                "(got HI = %d, DI = %d, T = %d, S = %d)", s.HI, s.DI, s.T, s.S);
  const size_t ws_need = indexer_topk_total_bytes(s);
  if (ws == nullptr || ws_bytes < ws_need)
    return fail(DSA_ERR_WORKSPACE, "indexer_topk: workspace of %zu bytes needed, %zu given", ws_need,
                ws_bytes);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base);
  if ((st = check_indexer_args(s, q_idx, q_sf, k_idx, k_sf, w, scores)) != DSA_OK) return st;
  if ((st = need(idx, "idx")) != DSA_OK) return st;
  st = launch_indexer_select(s, q_idx, q_sf, k_idx, k_sf, w, seq_lens, scores, idx,
                             base + indexer_topk_scores_bytes(s), next_call_tag(), static_cast<hipStream_t>(stream));
#ifdef DSA_DEBUG
  if (st == DSA_OK)
    st = debug_check_idx(static_cast<int64_t>(s.B) * s.T, k_eff(s), s.S, true, idx,
                         static_cast<hipStream_t>(stream), "fused top-K output");
#endif
  return st;
}

dsa_status_t dsa_sparse_mla_fwd(const dsa_shape_t* shape, const void* q, const void* kv,
                                const int32_t* idx, void* o, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  dsa_status_t st = check_shape(shape);
  if (st != DSA_OK) return st;
  if ((st = check_mla_args(q, kv, idx, o)) != DSA_OK) return st;
  if (ws != nullptr && !aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  return launch_sparse_mla(*shape, q, kv, idx, o, lse, ws, ws_bytes,
                           static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_forward_ragged(const dsa_shape_t* shape, const int32_t* seq_lens,
                                const void* q_idx, const uint8_t* q_sf, const void* k_idx,
                                const uint8_t* k_sf, const void* w, const void* q, const void* kv,
                                int32_t* idx_out, void* o, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  dsa_status_t st = check_shape(shape);
  if (st != DSA_OK) return st;
  const ForwardLayout L = forward_layout(*shape);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(DSA_ERR_WORKSPACE, "forward: workspace of %zu bytes needed, %zu given", L.total,
                ws_bytes);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  return forward_on(*shape, seq_lens, q_idx, q_sf, k_idx, k_sf, w, q, kv, idx_out, o, lse,
                    static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_forward(const dsa_shape_t* shape, const void* q_idx, const uint8_t* q_sf,
                         const void* k_idx, const uint8_t* k_sf, const void* w, const void* q,
                         const void* kv, int32_t* idx_out, void* o, float* lse, void* ws,
                         size_t ws_bytes, void* stream) {
  return dsa_forward_ragged(shape, nullptr, q_idx, q_sf, k_idx, k_sf, w, q, kv, idx_out, o, lse,
                            ws, ws_bytes, stream);
}

dsa_status_t dsa_forward_noalloc(const dsa_shape_t* shape, const void* q_idx, const uint8_t* q_sf,
                                 const void* k_idx, const uint8_t* k_sf, const void* w, const void* q,
                                 const void* kv, int32_t* idx_out, void* o, float* lse, void* stream) {
  g_last_error[0] = '\0';
  dsa_status_t st = check_shape(shape);
  if (st != DSA_OK) return st;
  const size_t need = forward_workspace_bytes(*shape);
  if (need > kNoallocScratchBytes)
    return fail(DSA_ERR_WORKSPACE,
                "forward_noalloc: this shape needs %zu bytes of scratch; the library's own scratch "
                "holds %zu (use dsa_forward with a workspace)", need, kNoallocScratchBytes);
  char* base = noalloc_scratch_ptr();
  if (base == nullptr) return DSA_ERR_HIP;
  return forward_on(*shape, nullptr, q_idx, q_sf, k_idx, k_sf, w, q, kv, idx_out, o, lse, base,
                    static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_cache_fill(int32_t N, int32_t D, const void* x, const void* W,
                            const float* kv_gamma, const float* k_gamma, const float* k_beta,
                            const float* rope_cos, const float* rope_sin, const int64_t* slots,
                            int32_t kv_dtype, void* kv_cache, int32_t k_dtype, void* k_cache,
                            uint8_t* k_sf, int32_t w_dtype, void* w_out, void* ws,
                            size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (N < 0 || D <= 0 || D % 64 != 0)
    return fail(DSA_ERR_INVALID_ARG, "cache fill: N = %d, D = %d (D must be a positive multiple of 64)",
                N, D);
  if (kv_dtype != DSA_BF16 && kv_dtype != DSA_F32)
    return fail(DSA_ERR_UNSUPPORTED, "cache fill: kv_dtype %d", kv_dtype);
  if (k_dtype != DSA_BF16 && k_dtype != DSA_F32 && k_dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "cache fill: k_dtype %d", k_dtype);
  if (w_dtype != DSA_BF16 && w_dtype != DSA_F32)
    return fail(DSA_ERR_UNSUPPORTED, "cache fill: w_dtype %d", w_dtype);
  if (N == 0) return DSA_OK;
  dsa_status_t st;
  if ((st = need(x, "x")) || (st = need(W, "W")) || (st = need(kv_gamma, "kv_gamma")) ||
      (st = need(k_gamma, "k_gamma")) || (st = need(k_beta, "k_beta")) ||
      (st = need(rope_cos, "rope_cos")) || (st = need(rope_sin, "rope_sin")) ||
      (st = need(slots, "slots")) || (st = need(kv_cache, "kv_cache")) ||
      (st = need(k_cache, "k_cache")) || (st = need(w_out, "w_out")))
    return st;
  if (k_dtype == DSA_FP8_E4M3 && k_sf == nullptr)
    return fail(DSA_ERR_INVALID_ARG, "cache fill: k_sf is NULL with an FP8 indexer key");
  if (ws != nullptr && !aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  return launch_cache_fill(N, D, x, W, kv_gamma, k_gamma, k_beta, rope_cos, rope_sin, slots,
                           kv_dtype, kv_cache, k_dtype, k_cache, k_sf, w_dtype, w_out, ws,
                           ws_bytes, static_cast<hipStream_t>(stream));
}

size_t dsa_cache_fill_workspace_bytes(int32_t N, int32_t D) {
  if (N < 0 || D <= 0 || D % 64 != 0) return static_cast<size_t>(-1);
  return N == 0 ? 0 : cache_fill_workspace_bytes(N, D);
}

dsa_status_t dsa_indexer_query(int32_t N, int32_t Dq, const void* cq, const void* wq_b,
                               int32_t q_dtype, void* q_out, uint8_t* q_sf, void* ws,
                               size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (N < 0 || Dq <= 0 || Dq % 64 != 0)
    return fail(DSA_ERR_INVALID_ARG, "indexer query: N = %d, Dq = %d (Dq must be a positive multiple of 64)",
                N, Dq);
  if (q_dtype != DSA_BF16 && q_dtype != DSA_F32 && q_dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "indexer query: q_dtype %d", q_dtype);
  if (N == 0) return DSA_OK;
  dsa_status_t st;
  if ((st = need(cq, "cq")) || (st = need(wq_b, "wq_b")) || (st = need(q_out, "q_out"))) return st;
  if (q_dtype == DSA_FP8_E4M3 && q_sf == nullptr)
    return fail(DSA_ERR_INVALID_ARG, "indexer query: q_sf is NULL with FP8 output");
  if (ws != nullptr && !aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  return launch_indexer_query(N, Dq, cq, wq_b, q_dtype, q_out, q_sf, ws, ws_bytes,
                              static_cast<hipStream_t>(stream));
}

size_t dsa_indexer_query_workspace_bytes(int32_t N, int32_t Dq) {
  if (N < 0 || Dq <= 0 || Dq % 64 != 0) return static_cast<size_t>(-1);
  return N == 0 ? 0 : indexer_query_workspace_bytes(N, Dq);
}

dsa_status_t dsa_absorb_prepare(int32_t H, const void* kv_b, void* w_uk_t, void* stream) {
  g_last_error[0] = '\0';
  if (H < 0) return fail(DSA_ERR_INVALID_ARG, "absorb prepare: H = %d", H);
  if (H == 0) return DSA_OK;
  dsa_status_t st;
  if ((st = need(kv_b, "kv_b")) || (st = need(w_uk_t, "w_uk_t"))) return st;
  return launch_absorb_prepare(H, kv_b, w_uk_t, static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_absorb_query(int32_t N, int32_t H, const void* qb, const void* w_uk_t,
                              const float* rope_cos, const float* rope_sin, int32_t q_dtype,
                              void* q, void* stream) {
  g_last_error[0] = '\0';
  if (N < 0 || H < 0) return fail(DSA_ERR_INVALID_ARG, "absorb query: N = %d, H = %d", N, H);
  if (q_dtype != DSA_BF16 && q_dtype != DSA_F32)
    return fail(DSA_ERR_UNSUPPORTED, "absorb query: q_dtype %d", q_dtype);
  if (N == 0 || H == 0) return DSA_OK;
  dsa_status_t st;
  if ((st = need(qb, "qb")) || (st = need(w_uk_t, "w_uk_t")) || (st = need(rope_cos, "rope_cos")) ||
      (st = need(rope_sin, "rope_sin")) || (st = need(q, "q")))
    return st;
  return launch_absorb_query(N, H, qb, w_uk_t, rope_cos, rope_sin, q_dtype, q,
                             static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_absorb_output(int32_t N, int32_t H, const void* o_lat, const void* kv_b,
                               int32_t out_dtype, void* out, void* stream) {
  g_last_error[0] = '\0';
  if (N < 0 || H < 0) return fail(DSA_ERR_INVALID_ARG, "absorb output: N = %d, H = %d", N, H);
  if (out_dtype != DSA_BF16 && out_dtype != DSA_F32)
    return fail(DSA_ERR_UNSUPPORTED, "absorb output: out_dtype %d", out_dtype);
  if (N == 0 || H == 0) return DSA_OK;
  dsa_status_t st;
  if ((st = need(o_lat, "o_lat")) || (st = need(kv_b, "kv_b")) || (st = need(out, "out"))) return st;
  return launch_absorb_output(N, H, o_lat, kv_b, out_dtype, out, static_cast<hipStream_t>(stream));
}

static bool output_projection_dims_ok(int32_t N, int32_t Din, int32_t Dout) {
  return N >= 0 && Din > 0 && Din % 64 == 0 && Dout > 0 && Dout % 128 == 0;
}

dsa_status_t dsa_output_projection(int32_t N, int32_t Din, int32_t Dout, const void* premix,
                                   const void* wo, int32_t out_dtype, void* out, void* ws,
                                   size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (!output_projection_dims_ok(N, Din, Dout))
    return fail(DSA_ERR_INVALID_ARG,
                "output projection: N = %d, Din = %d, Dout = %d (Din a positive multiple of 64, "
                "Dout of 128)", N, Din, Dout);
  if (out_dtype != DSA_BF16 && out_dtype != DSA_F32)
    return fail(DSA_ERR_UNSUPPORTED, "output projection: out_dtype %d", out_dtype);
  if (N == 0) return DSA_OK;
  dsa_status_t st;
  if ((st = need(premix, "premix")) || (st = need(wo, "wo")) || (st = need(out, "out"))) return st;
  if (ws != nullptr && !aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  return launch_output_projection(N, Din, Dout, premix, wo, out_dtype, out, ws, ws_bytes,
                                  static_cast<hipStream_t>(stream));
}

size_t dsa_output_projection_workspace_bytes(int32_t N, int32_t Din, int32_t Dout) {
  if (!output_projection_dims_ok(N, Din, Dout)) return static_cast<size_t>(-1);
  return N == 0 ? 0 : output_projection_workspace_bytes(N, Din, Dout);
}

size_t dsa_workspace_bytes(const dsa_shape_t* shape, int32_t entry) {
  if (check_shape(shape) != DSA_OK) return static_cast<size_t>(-1);
  switch (entry) {
    case DSA_ENTRY_TOPK: return topk_workspace_bytes(*shape);
    case DSA_ENTRY_SPARSE_MLA: return mla_workspace_bytes(*shape);
    case DSA_ENTRY_FORWARD: return forward_layout(*shape).total;
    case DSA_ENTRY_INDEXER_TOPK:
      if (!indexer_select_applies(*shape)) {
        fail(DSA_ERR_UNSUPPORTED, "indexer_topk does not cover this shape");
        return static_cast<size_t>(-1);
      }
      return indexer_topk_total_bytes(*shape);
  }
  fail(DSA_ERR_INVALID_ARG, "unknown entry %d", entry);
  return static_cast<size_t>(-1);
}

dsa_status_t dsa_timing_begin(void) {
  g_last_error[0] = '\0';
  TimingSession& T = timing();
  std::lock_guard<std::mutex> lock(T.mu);
  if (T.active.load()) return fail(DSA_ERR_INVALID_ARG, "timing: a session is already active");
  T.launches.clear();
  T.dropped.clear();
  ++T.generation;
  T.active.store(true);
  return DSA_OK;
}

dsa_status_t dsa_timing_end(dsa_kernel_time_t* out, int32_t max_out, int32_t* n_out) {
  g_last_error[0] = '\0';
  if (out == nullptr && max_out > 0) return fail(DSA_ERR_INVALID_ARG, "timing: out is NULL");
  TimingSession& T = timing();
  std::lock_guard<std::mutex> lock(T.mu);
  if (!T.active.load()) return fail(DSA_ERR_INVALID_ARG, "timing: no active session");
  T.active.store(false);
  std::vector<dsa_kernel_time_t> recs;
  auto find = [&](const char* name) -> dsa_kernel_time_t& {
    for (auto& r : recs)
      if (std::strncmp(r.name, name, sizeof r.name - 1) == 0) return r;
    dsa_kernel_time_t r{};
    std::snprintf(r.name, sizeof r.name, "%s", name);
    recs.push_back(r);
    return recs.back();
  };
  dsa_status_t st = DSA_OK;
  for (const TimedLaunch& L : T.launches) {
    if (L.name == nullptr) continue;  // its stop event was never recorded
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(L.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, L.start, L.stop);
    if (e != hipSuccess) {
      st = fail(DSA_ERR_HIP, "timing: %s: %s", L.name, hipGetErrorString(e));
      continue;
    }
    dsa_kernel_time_t& r = find(L.name);
    r.min_ms = r.launches == 0 ? ms : std::min(r.min_ms, static_cast<double>(ms));
    r.max_ms = std::max(r.max_ms, static_cast<double>(ms));
    r.total_ms += ms;
    ++r.launches;
  }
  for (const auto& d : T.dropped) find(d.first).dropped += d.second;
  T.launches.clear();
  T.dropped.clear();
  for (int32_t i = 0; i < max_out && i < static_cast<int32_t>(recs.size()); ++i) out[i] = recs[i];
  if (n_out != nullptr) *n_out = static_cast<int32_t>(recs.size());
  return st;
}

const char* dsa_status_str(dsa_status_t status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_last_error; }

}  // extern "C"
