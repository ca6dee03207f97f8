// Internal declarations shared by the host API and the kernel translation units.
// Nothing here is part of the C ABI (include/clsa.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/clsa.h"

namespace clsa {

// Rows no longer than this are selected by one workgroup holding the whole row in LDS;
// longer rows use the multi-workgroup histogram select.
constexpr int kLdsRowCap = 12288;
// Bins of the first histogram level of the multi-workgroup select (top 12 key bits).
constexpr int kHist1Bins = 4096;
// Per-row state words of the multi-workgroup select.
constexpr int kTopkStateWords = 16;
// Scores handled by one workgroup of the multi-workgroup select passes.
constexpr int kTopkChunk = 8192;
// Keys per attention tile.
constexpr int kAttnTile = 64;
// fp32 words per split partial record: acc[128], m, l, 2 words of padding (16-byte records).
constexpr int kPartStride = 132;
// Default rows per prefill chunk of clsa_step.
constexpr int kPrefillChunkRows = 1024;

// ---- host-side plan (pure functions, no HIP) ------------------------------------------------
struct TopkPlan {
  bool multi_wg = false;   // long rows: histogram select over many workgroups
  size_t hist_off = 0, state_off = 0, sure_off = 0, cand_off = 0;
  size_t bytes = 0;
};

struct AttnPlan {
  int group = 0;           // hq / hkv query heads per KV head
  int qrows = 0;           // query rows per (row, KV head) = n_layers_call * group
  int qblocks = 0;         // blocks of 64 query rows
  int splits = 1;          // the selected rows are split over this many workgroups
  int keys_per_split = 0;  // multiple of kAttnTile
  size_t part_bytes = 0;   // fp32 partials (m, l, acc[128]) when splits > 1
};

struct StepPlan {
  TopkPlan topk;
  AttnPlan attn;
  int chunk_rows = 0;      // prefill: rows per chunk; decode: R
  int64_t ld_scores = 0;   // workspace scores leading dimension
  size_t scores_off = 0, scores_bytes = 0;
  size_t topk_off = 0;
  size_t part_off = 0;
  size_t ksel_off = 0, vsel_off = 0, sel_bytes = 0;
  size_t total = 0;
};

// Validation.  Each returns CLSA_OK or an error status and fills `err`.
clsa_status check_dims(const clsa_dims* d, std::string& err);
clsa_status check_rows(const clsa_dims* d, const clsa_rows* r, std::string& err);
clsa_status check_ptr(const void* p, const char* name, std::string& err);
clsa_status check_ptr_opt(const void* p, const char* name, std::string& err);

TopkPlan plan_topk(const clsa_dims* d, const clsa_rows* r);
AttnPlan plan_attn(const clsa_dims* d, int n_rows, int n_layers_call);
StepPlan plan_step(const clsa_dims* d, const clsa_rows* r, int schedule, bool user_scores, bool user_sel,
                   int prefill_chunk_rows);
size_t workspace_bytes(const clsa_dims* d, const clsa_rows* r, int schedule);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline float softmax_scale(const clsa_dims* d) {
  return d->sm_scale > 0.f ? d->sm_scale : 1.0f / 11.313708498984761f;  // 1/sqrt(128)
}

// ---- kernel launchers (defined in the .hip translation units) --------------------------------
// All return hipSuccess-or-error as an int (0 = success) so this header needs no HIP include.
struct RowsDev {
  int mode, n_rows, seq, pos0, max_row_len;
  const int32_t* cu;  // device cu_seqlens
};

int launch_index_scores_decode(const RowsDev& rows, int d_idx, int64_t total_tokens, const uint16_t* q_idx,
                               const uint16_t* k_idx, float* scores, int64_t ld, void* stream);
int launch_index_scores_prefill(const RowsDev& rows, int d_idx, const uint16_t* q_idx, const uint16_t* k_idx,
                                float* scores, int64_t ld, void* stream);
int launch_topk(const RowsDev& rows, int k, const TopkPlan& plan, const float* scores, int64_t ld,
                int32_t* idx, int32_t* count, void* ws, void* stream);
int launch_gather(const RowsDev& rows, int k, int hkv, const uint16_t* kc, const uint16_t* vc,
                  const int32_t* idx, const int32_t* count, uint16_t* ks, uint16_t* vs, void* stream);
int launch_attn(const RowsDev& rows, int k, int hq, int hkv, int n_layers_call, float scale,
                const AttnPlan& plan, const uint16_t* q, int64_t q_stride, const uint16_t* ksel,
                const uint16_t* vsel, const uint16_t* kc, const uint16_t* vc, const int32_t* idx,
                const int32_t* count, uint16_t* out, int64_t o_stride, void* part, void* stream);
const char* device_error_string(int err);

}  // namespace clsa
