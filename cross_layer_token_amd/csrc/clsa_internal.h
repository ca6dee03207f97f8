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
// Tokens per workgroup of the decode score kernel (also the histogram partial granularity).
// Decode: the sequences' tokens, concatenated as they lie in the cache, are cut into segments of
// about total / kIdxMinWorkgroups tokens (idx_seg_for), so that every workgroup streams the same
// share of K_idx whatever the mix of sequence lengths; a segment may hold the end of one sequence
// and the start of the next.  Prefill rows and scores from the caller: per-row chunks of
// kIdxChunkMax when that still gives kIdxMinWorkgroups workgroups, else halved down to
// kIdxChunkMin (idx_chunk_for).
constexpr int kIdxChunkMax = 8192;
constexpr int kIdxChunkMin = 1024;
constexpr int kIdxMinWorkgroups = 256;
// First histogram level of the long-row select: the top kTopkBinBits bits of the score key
// (sign, exponent and the two leading mantissa bits), so a bin spans a factor of 1.25 in value
// and the candidates at or above the bin holding the k-th score stay a few percent of the row
// whatever the scale of the scores (one bin of sign and high exponent bits alone spans a factor
// of 4 and can hold a fifth of the row).
constexpr int kTopkBinBits = 11;
constexpr int kTopkBins = 1 << kTopkBinBits;
static_assert(kIdxChunkMax < 65536, "histogram partials hold uint16 counts");
// Scores classified by one workgroup of the long-row select, and the most spans of a row.
constexpr int kSelectSpan = 8192;
constexpr int kMaxSelectSpans = 2048;
static_assert((int64_t)kSelectSpan * kMaxSelectSpans >= CLSA_MAX_ROW_LEN, "spans cover the longest row");
// The layer-batched decode step may finish the long-row selection inside the attention
// workgroups (each keeps its split's token ids in LDS) when a split holds at most this many keys.
constexpr int kFusedMaxIds = 2048;
// Keys per attention tile.
constexpr int kAttnTile = 64;
// Upper bound on the splits of the selected rows of one (row, KV head, query block).
constexpr int kMaxAttnSplits = 16;
// Attention: (row, KV head, query block) blocks at or above this count run 4-wave workgroups,
// two per CU, with no key split; below it, 8-wave workgroups (one per CU) and the keys are split
// until about CLSA_ATTN_TARGET_WGS workgroups exist.
constexpr int kAttnManyBlocks = 512;
#ifndef CLSA_ATTN_TARGET_WGS
#define CLSA_ATTN_TARGET_WGS 256
#endif
// fp32 words of one attention split partial per (row, KV head, query block): 4 waves x 64 lanes
// x (32 accumulators + m + l).
constexpr int kAttnPartFloats = 4 * 34 * 64;
// Default rows per prefill chunk of clsa_step.
constexpr int kPrefillChunkRows = 1024;
// The per-layer decode schedule gathers K_S/V_S of this many bytes at most at a time (a chunk of
// rows), so that the compact buffers the L attention passes re-read stay in the 256 MB Infinity
// Cache.
constexpr size_t kPerLayerResidentBytes = (size_t)192 << 20;

// ---- host-side plan (pure functions, no HIP) ------------------------------------------------
struct TopkPlan {
  bool multi_wg = false;   // long rows: histogram select over many workgroups
  int hist_chunk = 0;      // tokens per histogram partial (the score kernel's segment or chunk)
  int hist_chunks = 0;     // histogram partials per row (a decode row may straddle one more segment)
  int spans = 0;           // select workgroups per row (kSelectSpan scores each)
  size_t hpart_off = 0;    // uint16 [R, hist_chunks, kTopkBins]: per-piece partials (full or windowed)
  size_t hinfo_off = 0;    // uint32 [R, hist_chunks]: window start | full flag of each partial
  size_t cnt_off = 0;      // uint32 [R, spans]
  size_t slot_off = 0;     // uint2 [R, max_row_len]: per-span ordered lists (key, index)
  size_t list_off = 0;     // uint2 [R, max_row_len]: the concatenated list, when it overflows LDS
  size_t rowinfo_off = 0;  // uint32 [R, 2]: first-level bin t1 and the count above it
  size_t bytes = 0;
};

struct AttnPlan {
  int group = 0;           // hq / hkv query heads per KV head
  int qrows = 0;           // query rows per (row, KV head) = n_layers_call * group
  int qblocks = 0;         // blocks of 16 wpt query rows
  int teams = 2;           // teams per workgroup (1 or 2)
  int wpt = 4;             // waves per team (4, or 2 for rows of at most 32 query rows with many blocks)
  bool pair = false;       // many blocks: team t takes KV head 2p + t of the pair p (whole stages, no splits)
  int splits = 1;          // the selected rows are split over this many workgroups
  int keys_per_split = 0;  // multiple of kAttnTile
  size_t part_bytes = 0;   // fp32 partials [splits, R, hkv, qblocks, kAttnPartFloats] when splits > 1
  int tickets = 0;         // uint32 words of ticket memory: one per (row, KV head, query block)
};

// Ticket words live in one region that the first kernel of a call clears; every ticket is
// reset by the workgroup that consumes it, so later launches of the same call can reuse it.
struct StepPlan {
  TopkPlan topk;
  AttnPlan attn;
  int chunk_rows = 0;      // prefill: rows per chunk; decode: R
  int sel_chunk_rows = 0;  // per-layer decode: rows whose compact K_S/V_S are gathered at once
  int64_t ld_scores = 0;   // workspace scores leading dimension
  size_t ticket_off = 0;   // attention tickets
  int n_tickets = 0;
  size_t scores_off = 0, scores_bytes = 0;
  size_t topk_off = 0;
  size_t part_off = 0;
  size_t ksel_off = 0, vsel_off = 0, sel_bytes = 0;
  bool fused_select = false;  // the attention workgroups finish the long-row selection
  size_t total = 0;
};

// Validation.  Each returns CLSA_OK or an error status and fills `err`.
clsa_status check_dims(const clsa_dims* d, std::string& err);
clsa_status check_rows(const clsa_dims* d, const clsa_rows* r, std::string& err);
clsa_status check_ptr(const void* p, const char* name, std::string& err);
clsa_status check_ptr_opt(const void* p, const char* name, std::string& err);

TopkPlan plan_topk(const clsa_dims* d, const clsa_rows* r);
// Tokens per workgroup of the decode score kernel for n_rows rows of at most max_row_len tokens.
int idx_chunk_for(int n_rows, int max_row_len);
int idx_seg_for(int64_t total_tokens);
// n_rows: rows of this launch (buffer sizes); split_rows: rows that decide the split count
// (0 = n_rows).
AttnPlan plan_attn(const clsa_dims* d, int n_rows, int n_layers_call, int split_rows);
StepPlan plan_step(const clsa_dims* d, const clsa_rows* r, int schedule, bool user_scores, bool user_sel,
                   int prefill_chunk_rows);
size_t workspace_bytes(const clsa_dims* d, const clsa_rows* r, int schedule, int prefill_chunk_rows);
// Standalone calls: [tickets][plan buffers].
size_t topk_workspace(const clsa_dims* d, const clsa_rows* r);
size_t attn_workspace(const AttnPlan& a);


// Host and device: the selection positions [*kbeg, *kend) that split `split` of a (row, KV head)
// block reads, when each split takes kps positions and the row holds `count` selected tokens of at
// most k.  count is clamped into [0, k] first, so an out-of-range count from a caller cannot send a
// read of idx (or of a compact K_S/V_S row) past the row's k entries: kend <= k always.
#if defined(__HIPCC__)
#define CLSA_HOST_DEVICE __host__ __device__
#else
#define CLSA_HOST_DEVICE
#endif
CLSA_HOST_DEVICE inline void split_key_range(int count, int k, int split, int kps, int* kbeg, int* kend) {
  const int cnt = count < 0 ? 0 : (count > k ? k : count);
  const int b = split * kps;
  *kbeg = b;
  *kend = b + kps < cnt ? b + kps : cnt;
}

// Prefill routing scores: the causal tiles of kPfTile rows x kPfTile token columns.  Row block rb
// (rows kPfTile rb .. of the call) has column blocks 0 .. (pos0 + its last row) / kPfTile: c0 + rb of
// them for every block but the last (c0 = ceil(pos0 / kPfTile) + 1), so tile t lies in the row block
// whose prefix P(rb) = rb c0 + rb (rb - 1) / 2 is the largest at or below t.
constexpr int kPfTile = 128;
struct PrefillGrid {
  int c0;        // column blocks of row block 0
  int last_rb;   // last row block
  int64_t tiles; // tiles holding a visible entry
};
CLSA_HOST_DEVICE inline int64_t pf_prefix(int64_t rb, int c0) { return rb * c0 + rb * (rb - 1) / 2; }
inline PrefillGrid prefill_grid(int pos0, int n_rows) {
  PrefillGrid g;
  g.c0 = (pos0 + kPfTile - 1) / kPfTile + 1;
  g.last_rb = (n_rows - 1) / kPfTile;
  g.tiles = pf_prefix(g.last_rb, g.c0) + (int64_t)(pos0 + n_rows - 1) / kPfTile + 1;
  return g;
}
// Row block and column block of tile t < g.tiles.
CLSA_HOST_DEVICE inline void prefill_tile(const PrefillGrid& g, int64_t t, int* rb_out, int* cb_out) {
  int64_t rb;
  if (t >= pf_prefix(g.last_rb, g.c0)) {
    rb = g.last_rb;
  } else {
    // P(rb) <= t  <=>  rb <= (sqrt((2 c0 - 1)^2 + 8 t) - (2 c0 - 1)) / 2; then fix the rounding
    const double b = 2.0 * g.c0 - 1.0;
    rb = (int64_t)((__builtin_sqrt(b * b + 8.0 * (double)t) - b) * 0.5);
    while (rb > 0 && pf_prefix(rb, g.c0) > t) --rb;
    while (rb < g.last_rb && pf_prefix(rb + 1, g.c0) <= t) ++rb;
  }
  *rb_out = (int)rb;
  *cb_out = (int)(t - pf_prefix(rb, g.c0));
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline size_t ticket_region(int words) { return words ? align_up((size_t)words * 4, 256) : 0; }
inline float softmax_scale(const clsa_dims* d) {
  return d->sm_scale > 0.f ? d->sm_scale : 1.0f / 11.313708498984761f;  // 1/sqrt(128)
}

// Distillation target and loss (eq. 4-5): keys per KL partial, and the workspace layout.
constexpr int kDistillKeyBlock = 256;
// The KL pass's causal tiles of kDistillRowBlock positions x kDistillKeyBlock keys, row-block-major.
// Full row block r (positions pos0 + 32 r .. pos0 + 32 r + 31) sees key blocks
// 0 .. floor((pos0 + 32 r + 31) / 256) = floor((a + r) / 8), with a = floor((pos0 + 31) / 32); the
// last row block, possibly partial, sees key blocks 0 .. floor((pos0 + n_rows - 1) / 256).
constexpr int kDistillRowBlock = 32;
static_assert(kDistillKeyBlock == 8 * kDistillRowBlock, "eight row blocks per key block");
CLSA_HOST_DEVICE inline int64_t kl_floor8_sum(int64_t x) {  // sum over y < x of floor(y / 8)
  const int64_t q = x >> 3, r = x & 7;
  return 4 * q * (q - 1) + r * q;
}
// tiles of the full row blocks below r
CLSA_HOST_DEVICE inline int64_t kl_prefix(int64_t a, int64_t r) { return r + kl_floor8_sum(a + r) - kl_floor8_sum(a); }
CLSA_HOST_DEVICE inline int64_t kl_tile_count(int pos0, int n_rows) {
  const int64_t a = (pos0 + 31) / 32;
  const int64_t last_rb = (n_rows - 1) / kDistillRowBlock;
  return kl_prefix(a, last_rb) + ((int64_t)pos0 + n_rows - 1) / kDistillKeyBlock + 1;
}
// Row block and key block of tile t < kl_tile_count(pos0, n_rows): a binary search over the prefix.
CLSA_HOST_DEVICE inline void kl_tile(int pos0, int n_rows, int64_t t, int* rb_out, int* kb_out) {
  const int64_t a = (pos0 + 31) / 32;
  const int last_rb = (n_rows - 1) / kDistillRowBlock;
  const int64_t last0 = kl_prefix(a, last_rb);
  int rb = last_rb;
  if (t < last0) {
    int lo = 0, hi = last_rb;  // prefix(lo) <= t < prefix(hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (kl_prefix(a, mid) <= t) lo = mid; else hi = mid;
    }
    rb = lo;
  }
  *rb_out = rb;
  *kb_out = (int)(t - kl_prefix(a, rb));
}
struct DistillPlan {
  int n_kb = 0;           // key blocks of kDistillKeyBlock per row
  int64_t kl_tiles = 0;   // workgroups of the KL pass: kl_tile_count(pos0, n_rows)
  size_t lse2_off = 0;    // fp32 [R, L * hq]
  size_t lse_i_off = 0;   // fp32 [R]
  size_t part_off = 0;    // fp32 [R, n_kb]
  size_t bytes = 0;
};
DistillPlan plan_distill(const clsa_dims* d, const clsa_rows* r);

// ---- kernel launchers (defined in the .hip translation units) --------------------------------
// All return hipSuccess-or-error as an int (0 = success) so this header needs no HIP include.
struct RowsDev {
  int mode, n_rows, seq, pos0, max_row_len;
  int64_t total_tokens;
  const int32_t* cu;  // device cu_seqlens
};

// `clear` (n_clear words) is zeroed by the launch before any other kernel of the call reads it.
// seg: tokens per workgroup over the concatenated sequences (idx_seg_for).  hpart / hinfo (with
// topk): also write, for every (row, segment) piece, the top-k histogram partial at slot
// segment - floor(cu[row] / seg) of the row's hpart_chunks.
int launch_index_scores_decode(const RowsDev& rows, int d_idx, int seg, const uint16_t* q_idx, int64_t q_stride,
                               const uint16_t* k_idx, float* scores, int64_t ld, uint16_t* hpart, uint32_t* hinfo,
                               int topk, int hpart_chunks, uint32_t* clear, int n_clear, void* stream);
int launch_index_scores_prefill(const RowsDev& rows, int d_idx, const uint16_t* q_idx, const uint16_t* k_idx,
                                float* scores, int64_t ld, uint32_t* clear, int n_clear, void* stream);
// have_hist: the score kernel already wrote the histogram partials.
// finish = false (long rows only): the select stops after writing the span lists and each row's
// first-level bin; the attention launched with SelectIn finishes the selection.
int launch_topk(const RowsDev& rows, int k, const TopkPlan& plan, const float* scores, int64_t ld,
                int32_t* idx, int32_t* count, void* ws, bool have_hist, void* stream, bool finish = true);
// Where the attention finds a row's unfinished selection (see launch_topk with finish = false).
struct SelectIn {
  const void* slot = nullptr;        // uint2 [R, max_row_len] span lists
  const uint32_t* cnt = nullptr;     // [R, spans]
  const uint32_t* rowinfo = nullptr; // [R, 2]
  int spans = 0;
};
int launch_gather(const RowsDev& rows, int k, int hkv, const uint16_t* kc, const uint16_t* vc,
                  const int32_t* idx, const int32_t* count, uint16_t* ks, uint16_t* vs, void* stream);
// tickets_clear: the tickets are known to be zero (cleared earlier in the call).
int launch_attn(const RowsDev& rows, int k, int hq, int hkv, int n_layers_call, float scale,
                const AttnPlan& plan, const uint16_t* q, int64_t q_stride, const uint16_t* ksel,
                const uint16_t* vsel, const uint16_t* kc, const uint16_t* vc, const int32_t* idx,
                const int32_t* count, uint16_t* out, int64_t o_stride, void* part, uint32_t* tickets,
                bool tickets_clear, void* stream, const SelectIn* sel = nullptr, int32_t* idx_out = nullptr,
                int32_t* count_out = nullptr);
int launch_index_project(int batch, int d_idx, int d_model, int hkv, int64_t total_tokens, const uint16_t* h,
                         const uint16_t* wq, const uint16_t* wk, const int32_t* cu, uint16_t* q_idx, uint16_t* k_idx,
                         const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache,
                         void* stream);
int launch_distill(const RowsDev& rows, int64_t total_tokens, int L, int hq, int hkv, float scale, const uint16_t* q,
                   int64_t q_stride, const uint16_t* k, const float* scores, int64_t ld, float* kl, float* loss,
                   void* ws, const DistillPlan& plan, void* stream);
const char* device_error_string(int err);

// Static device scratch of clsa_step_no_alloc (no_alloc.hip): its size, and the address of the
// current device's copy (looked up once per device; 0 = success, else a HIP error with `err` set).
constexpr size_t kNoAllocScratchBytes = CLSA_NO_ALLOC_SCRATCH_BYTES;
int no_alloc_scratch(void** ptr, std::string& err);

}  // namespace clsa
