// Host-side declarations shared by the libdsa translation units.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// Device facts the launch heuristics need, cached once per device.
struct DeviceInfo {
  int cu_count;
  size_t max_lds;
};
const DeviceInfo& device_info();

// Records a failure detail for dsa_last_error() and returns `st`.
dsa_status_t fail(dsa_status_t st, const char* fmt, ...);
// Checks the last launch on this thread.
dsa_status_t check_launch(const char* what);

// Times one kernel launch for dsa_timing_*: construct it right before the
// launch, pass start()/stop() to hipExtLaunchKernelGGL (the runtime stamps
// them with the dispatch's own begin and end), call done() right after (it
// checks the launch like check_launch).  Outside a timing session the events
// are null and the launch is a plain one.
class LaunchTimer {
 public:
  LaunchTimer();
  hipEvent_t start() const { return start_; }
  hipEvent_t stop() const { return stop_; }
  dsa_status_t done(const char* what);

 private:
  hipEvent_t start_ = nullptr, stop_ = nullptr;
  long slot_ = -1;  // record index in the session; -1 not timed, -2 beyond the capacity
  long gen_ = 0;    // the session the slot belongs to
};

// A tag per call of a launch whose workgroups meet through the workspace:
// distinct across calls of this process (39 bits).
uint64_t next_call_tag();

inline int32_t k_eff(const dsa_shape_t& s) { return s.K < s.S ? s.K : s.S; }

// ---- index scores -------------------------------------------------------
// seq_lens: device int32 [B] context lengths of a ragged batch, or nullptr.
// full_rows: every score of a row is written (keys past the query's position
// get -inf); false lets the many-query kernels leave the keys past a query
// block's last visible one unwritten, for a consumer that ignores each row
// past its query's position (launch_topk with causal_rows).
dsa_status_t launch_indexer(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                            const void* k_idx, const uint8_t* k_sf, const void* w,
                            const int32_t* seq_lens, float* scores, bool full_rows,
                            hipStream_t stream);

// The index scores with the top-K selection fused in (decode: fewer than 8
// queries per sequence, V3.2 indexer shapes): scores go to `scores` (scratch),
// the selection to idx [rows, K_eff]; sel_ws holds the per-row meeting state
// and histograms (indexer_select_workspace_bytes), tag is the call's own.
bool indexer_select_applies(const dsa_shape_t& s);
size_t indexer_select_workspace_bytes(const dsa_shape_t& s);
dsa_status_t launch_indexer_select(const dsa_shape_t& s, const void* q_idx, const uint8_t* q_sf,
                                   const void* k_idx, const uint8_t* k_sf, const void* w,
                                   const int32_t* seq_lens, float* scores, int32_t* idx,
                                   void* sel_ws, uint64_t tag, hipStream_t stream);

// ---- top-k -------------------------------------------------------------
// DSA_OK when launch_topk has kernels for the shape, else the failure (set
// with fail) it would return; launches nothing.
dsa_status_t topk_check(const dsa_shape_t& s);
size_t topk_workspace_bytes(const dsa_shape_t& s);
// causal_rows: row (b, t) holds scores only for its causally visible keys
// [0, L_b - T + t + 1) (L_b = seq_lens[b] clamped to [0, S], or S without
// seq_lens; the length clamped to [0, S]); whatever the rest of the row's
// memory holds is ignored.  Else every row holds S scores.
dsa_status_t launch_topk(const dsa_shape_t& s, const float* scores, const int32_t* seq_lens,
                         bool causal_rows, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

// ---- cache fill and indexer inputs ---------------------------------------
size_t cache_fill_workspace_bytes(int N, int D);
size_t indexer_query_workspace_bytes(int N, int Dq);
// ---- absorption products ---------------------------------------------------
dsa_status_t launch_absorb_prepare(int H, const void* kv_b, void* wuk_t, hipStream_t stream);
dsa_status_t launch_absorb_query(int N, int H, const void* qb, const void* wuk_t,
                                 const float* rope_cos, const float* rope_sin, int q_dtype, void* q,
                                 hipStream_t stream);
dsa_status_t launch_absorb_output(int N, int H, const void* o_lat, const void* kv_b, int out_dtype,
                                  void* premix, hipStream_t stream);
size_t output_projection_workspace_bytes(int N, int Din, int Dout);
dsa_status_t launch_output_projection(int N, int Din, int Dout, const void* premix, const void* wo,
                                      int out_dtype, void* out, void* ws, size_t ws_bytes,
                                      hipStream_t stream);
dsa_status_t launch_indexer_query(int N, int Dq, const void* cq, const void* wq_b, int q_dtype,
                                  void* q_out, uint8_t* q_sf, void* ws, size_t ws_bytes,
                                  hipStream_t stream);
dsa_status_t launch_cache_fill(int N, int D, const void* x, const void* W, const float* kv_gamma,
                               const float* k_gamma, const float* k_beta, const float* rope_cos,
                               const float* rope_sin, const int64_t* slots, int kv_dtype,
                               void* kv_cache, int k_dtype, void* k_cache, uint8_t* k_sf,
                               int w_dtype, void* w_out, void* ws, size_t ws_bytes,
                               hipStream_t stream);

// ---- debug builds (-DDSA_DEBUG) -------------------------------------------
#ifdef DSA_DEBUG
// Checks rows x W index entries on the device and waits for the result: every
// entry in [-1, S), and with `sorted` the valid entries of each row strictly
// ascending with the -1 padding after them.  Fails with DSA_ERR_INVALID_ARG
// naming `what` otherwise.  Synchronizes `stream` (not for graph capture).
dsa_status_t debug_check_idx(int64_t rows, int W, int S, bool sorted, const int32_t* idx,
                             hipStream_t stream, const char* what);
#endif

// ---- the whole path ------------------------------------------------------
// Workspace bytes of dsa_forward, and the path on such a workspace at `base`
// (shape already checked; pointers, alignment and seq_lens checked here).
size_t forward_workspace_bytes(const dsa_shape_t& s);
dsa_status_t forward_on(const dsa_shape_t& s, const int32_t* seq_lens, const void* q_idx,
                        const uint8_t* q_sf, const void* k_idx, const uint8_t* k_sf, const void* w,
                        const void* q, const void* kv, int32_t* idx_out, void* o, float* lse,
                        char* base, hipStream_t stream);

// ---- sparse latent attention ------------------------------------------
// As topk_check, for launch_sparse_mla.
dsa_status_t mla_check(const dsa_shape_t& s);
size_t mla_workspace_bytes(const dsa_shape_t& s);
dsa_status_t launch_sparse_mla(const dsa_shape_t& s, const void* q, const void* kv,
                               const int32_t* idx, void* o, float* lse, void* ws,
                               size_t ws_bytes, hipStream_t stream);

}  // namespace dsa
