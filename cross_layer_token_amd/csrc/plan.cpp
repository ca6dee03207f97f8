// Host-side validation and workspace planning of the CLSA ABI.  Pure C++: no HIP call is made
// here, so every error path can be exercised on a machine without a GPU.
#include <cstdint>
#include <cstdio>
#include <string>

#include "clsa_internal.h"

namespace clsa {

namespace {
clsa_status fail(std::string& err, clsa_status s, const std::string& msg) {
  err = msg;
  return s;
}
}  // namespace

clsa_status check_ptr(const void* p, const char* name, std::string& err) {
  if (p == nullptr) return fail(err, CLSA_ERR_INVALID_ARGUMENT, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(err, CLSA_ERR_INVALID_ARGUMENT, std::string(name) + " is not 16-byte aligned");
  return CLSA_OK;
}

clsa_status check_ptr_opt(const void* p, const char* name, std::string& err) {
  if (p != nullptr && reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(err, CLSA_ERR_INVALID_ARGUMENT, std::string(name) + " is not 16-byte aligned");
  return CLSA_OK;
}

clsa_status check_dims(const clsa_dims* d, std::string& err) {
  if (d == nullptr) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->batch < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "batch must be >= 1");
  if (d->topk < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "topk must be >= 1");
  if (d->n_layers < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "n_layers must be >= 1");
  if (d->hq < 1 || d->hkv < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "hq and hkv must be >= 1");
  if (d->hq % d->hkv != 0) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "hq must be a multiple of hkv");
  if (d->head_dim != CLSA_HEAD_DIM) return fail(err, CLSA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (d->d_idx != 64 && d->d_idx != 128) return fail(err, CLSA_ERR_UNSUPPORTED, "d_idx must be 64 or 128");
  if (d->topk > CLSA_MAX_TOPK) return fail(err, CLSA_ERR_UNSUPPORTED, "topk above CLSA_MAX_TOPK");
  if (d->sm_scale != d->sm_scale) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "sm_scale is NaN");
  return CLSA_OK;
}

clsa_status check_rows(const clsa_dims* d, const clsa_rows* r, std::string& err) {
  if (r == nullptr) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows is NULL");
  if (r->mode != CLSA_MODE_DECODE && r->mode != CLSA_MODE_PREFILL)
    return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows.mode must be CLSA_MODE_DECODE or CLSA_MODE_PREFILL");
  if (r->n_rows < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows.n_rows must be >= 1");
  if (r->max_row_len < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows.max_row_len must be >= 1");
  if (r->max_row_len > CLSA_MAX_ROW_LEN) return fail(err, CLSA_ERR_UNSUPPORTED, "rows.max_row_len too large");
  if (r->total_tokens < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows.total_tokens must be >= 1");
  if (r->mode == CLSA_MODE_DECODE) {
    if (r->n_rows != d->batch) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "decode requires n_rows == batch");
  } else {
    if (r->seq < 0 || r->seq >= d->batch) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows.seq out of range");
    if (r->pos0 < 0) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows.pos0 must be >= 0");
    if ((int64_t)r->pos0 + r->n_rows != (int64_t)r->max_row_len)
      return fail(err, CLSA_ERR_INVALID_ARGUMENT, "prefill requires max_row_len == pos0 + n_rows");
  }
  if (r->max_row_len > r->total_tokens)
    return fail(err, CLSA_ERR_INVALID_ARGUMENT, "rows.max_row_len exceeds total_tokens");
  if (r->cu_seqlens_host != nullptr) {
    const int32_t* cu = r->cu_seqlens_host;
    if (cu[0] != 0) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
    for (int b = 0; b < d->batch; ++b) {
      const int64_t n = (int64_t)cu[b + 1] - cu[b];
      if (n < 0) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "cu_seqlens is not non-decreasing");
      if (r->mode == CLSA_MODE_DECODE) {
        if (n < 1) return fail(err, CLSA_ERR_INVALID_ARGUMENT, "decode sequence of length 0");
        if (n > r->max_row_len)
          return fail(err, CLSA_ERR_INVALID_ARGUMENT, "a sequence is longer than rows.max_row_len");
      }
    }
    if (cu[d->batch] != r->total_tokens)
      return fail(err, CLSA_ERR_INVALID_ARGUMENT, "cu_seqlens[batch] != rows.total_tokens");
    if (r->mode == CLSA_MODE_PREFILL && (int64_t)cu[r->seq + 1] - cu[r->seq] < (int64_t)r->pos0 + r->n_rows)
      return fail(err, CLSA_ERR_INVALID_ARGUMENT, "prefill rows reach past the end of their sequence");
  }
  return CLSA_OK;
}

int idx_chunk_for(int n_rows, int max_row_len) {
  int chunk = kIdxChunkMax;
  while (chunk > kIdxChunkMin && (int64_t)n_rows * ((max_row_len + chunk - 1) / chunk) < kIdxMinWorkgroups) chunk >>= 1;
  return chunk;
}

int idx_seg_for(int64_t total_tokens) {
  int64_t seg = (total_tokens + kIdxMinWorkgroups - 1) / kIdxMinWorkgroups;
  seg = (seg + 63) / 64 * 64;
  return (int)(seg < kIdxChunkMin ? kIdxChunkMin : (seg > kIdxChunkMax ? kIdxChunkMax : seg));
}

TopkPlan plan_topk(const clsa_dims* d, const clsa_rows* r) {
  TopkPlan p;
  p.multi_wg = r->max_row_len > kLdsRowCap;
  if (!p.multi_wg) return p;
  const size_t R = (size_t)r->n_rows;
  // decode partials come per (row, segment of the concatenated sequences), so a row may straddle
  // one segment more than its length needs
  const bool decode = r->mode == CLSA_MODE_DECODE;
  p.hist_chunk = decode ? idx_seg_for(r->total_tokens) : idx_chunk_for(r->n_rows, r->max_row_len);
  p.hist_chunks = (r->max_row_len + p.hist_chunk - 1) / p.hist_chunk + (decode ? 1 : 0);
  p.spans = (r->max_row_len + kSelectSpan - 1) / kSelectSpan;
  size_t off = 0;
  p.hpart_off = off;
  off = align_up(off + R * p.hist_chunks * kTopkBins * 2, 256);
  p.hinfo_off = off;
  off = align_up(off + R * p.hist_chunks * 4, 256);
  p.cnt_off = off;
  off = align_up(off + R * p.spans * 4, 256);
  p.slot_off = off;
  off = align_up(off + R * (size_t)r->max_row_len * 8, 256);
  p.list_off = off;
  off = align_up(off + R * (size_t)r->max_row_len * 8, 256);
  p.rowinfo_off = off;
  off = align_up(off + R * 8, 256);
  p.bytes = off;
  (void)d;
  return p;
}

AttnPlan plan_attn(const clsa_dims* d, int n_rows, int n_layers_call, int split_rows) {
  AttnPlan p;
  p.group = d->hq / d->hkv;
  p.qrows = n_layers_call * p.group;
  p.qblocks = (p.qrows + 63) / 64;
  // the split count depends on split_rows only, so every chunk of a call splits alike
  const int64_t base = (int64_t)(split_rows > 0 ? split_rows : n_rows) * d->hkv * p.qblocks;
  const int tiles = (d->topk + kAttnTile - 1) / kAttnTile;
  p.teams = base >= kAttnManyBlocks ? 1 : 2;
  if (p.teams == 1 && p.qrows > 32 && p.qblocks == 1 && d->hkv % 2 == 0) {
    // many blocks of more than 32 query rows: one eight-wave workgroup per (row, pair of KV heads),
    // a team per head, in lockstep (two four-wave workgroups per CU drift apart, and the kernel
    // waits for the one that fell behind); one round of workgroups, no splits
    p.teams = 2;
    p.pair = true;
    p.keys_per_split = tiles * kAttnTile;
    return p;
  }
  if (p.teams == 1 && p.qrows <= 32) {
    // one team of four waves would leave half of them (two SIMDs of the CU) without MFMA work:
    // two teams of two waves split each stage's tiles instead
    p.teams = 2;
    p.wpt = 2;
    p.qblocks = (p.qrows + 31) / 32;
  }
  int splits = 1;
  if (p.teams == 2 && base < CLSA_ATTN_TARGET_WGS) splits = (int)((CLSA_ATTN_TARGET_WGS + base - 1) / base);
  if (splits > kMaxAttnSplits) splits = kMaxAttnSplits;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int tiles_per_split = (tiles + splits - 1) / splits;
  p.splits = (tiles + tiles_per_split - 1) / tiles_per_split;
  p.keys_per_split = tiles_per_split * kAttnTile;
  if (p.splits > 1) {
    p.part_bytes = align_up((size_t)p.splits * n_rows * d->hkv * p.qblocks * kAttnPartFloats * 4, 256);
    p.tickets = (int)((int64_t)n_rows * d->hkv * p.qblocks);
  }
  return p;
}

StepPlan plan_step(const clsa_dims* d, const clsa_rows* r, int schedule, bool user_scores, bool user_sel,
                   int prefill_chunk_rows) {
  StepPlan s;
  const bool prefill = r->mode == CLSA_MODE_PREFILL;
  s.chunk_rows = prefill ? (prefill_chunk_rows > 0 ? prefill_chunk_rows : kPrefillChunkRows) : r->n_rows;
  if (s.chunk_rows > r->n_rows) s.chunk_rows = r->n_rows;
  clsa_rows chunk = *r;
  chunk.n_rows = s.chunk_rows;
  if (prefill) chunk.max_row_len = r->max_row_len;  // a chunk never sees more than the last row
  s.topk = plan_topk(d, &chunk);
  // one attention pass over all L layers, or one pass per layer (per-layer schedule, and the
  // per-layer routing ablation, which also routes once per layer)
  const int lc = schedule == CLSA_SCHEDULE_LAYER_BATCHED ? d->n_layers : 1;
  // every chunk (the shorter tail included) splits like the whole call, so results do not
  // depend on the chunk size; buffers are sized for the largest chunk
  s.attn = plan_attn(d, s.chunk_rows, lc, r->n_rows);
  const bool compact = schedule == CLSA_SCHEDULE_PER_LAYER && !prefill;
  if (compact) {
    // the gather and the L attention passes run over chunks of rows whose K_S/V_S fit
    // kPerLayerResidentBytes; each chunk splits for its own size (a function of the sizes alone),
    // so the partials and tickets cover both the full chunk and the shorter tail
    const size_t row_sel = (size_t)2 * d->hkv * d->topk * CLSA_HEAD_DIM * 2;  // K and V of one row
    int64_t rows_fit = (int64_t)(kPerLayerResidentBytes / row_sel);
    if (rows_fit < 1) rows_fit = 1;
    s.sel_chunk_rows = rows_fit < r->n_rows ? (int)rows_fit : r->n_rows;
    const int tail = r->n_rows % s.sel_chunk_rows;
    s.attn = plan_attn(d, s.sel_chunk_rows, 1, s.sel_chunk_rows);
    if (tail > 0) {
      const AttnPlan t = plan_attn(d, tail, 1, tail);
      if (t.part_bytes > s.attn.part_bytes) s.attn.part_bytes = t.part_bytes;
      if (t.tickets > s.attn.tickets) s.attn.tickets = t.tickets;
    }
  }
  s.ld_scores = (int64_t)align_up((size_t)r->max_row_len, 64);
  s.fused_select = !prefill && schedule == CLSA_SCHEDULE_LAYER_BATCHED && s.topk.multi_wg && s.attn.teams == 2 && s.attn.wpt == 4 &&
                   s.attn.keys_per_split <= kFusedMaxIds;
  size_t off = 0;
  s.ticket_off = off;
  s.n_tickets = s.attn.tickets;
  off += ticket_region(s.n_tickets);
  if (!user_scores) {
    s.scores_off = off;
    s.scores_bytes = align_up((size_t)s.chunk_rows * s.ld_scores * 4, 256);
    off += s.scores_bytes;
  }
  s.topk_off = off;
  off += s.topk.bytes;
  s.part_off = off;
  off += s.attn.part_bytes;
  if (compact && !user_sel) {
    s.sel_bytes = align_up((size_t)s.sel_chunk_rows * d->hkv * d->topk * CLSA_HEAD_DIM * 2, 256);
    s.ksel_off = off;
    off += s.sel_bytes;
    s.vsel_off = off;
    off += s.sel_bytes;
  }
  s.total = off;
  return s;
}

size_t topk_workspace(const clsa_dims* d, const clsa_rows* r) {
  return plan_topk(d, r).bytes;
}

size_t attn_workspace(const AttnPlan& a) { return ticket_region(a.tickets) + a.part_bytes; }

DistillPlan plan_distill(const clsa_dims* d, const clsa_rows* r) {
  DistillPlan p;
  const size_t R = (size_t)r->n_rows;
  p.n_kb = (r->max_row_len + kDistillKeyBlock - 1) / kDistillKeyBlock;
  p.kl_tiles = kl_tile_count(r->pos0, r->n_rows);
  size_t off = 0;
  p.lse2_off = off;
  off = align_up(off + R * d->n_layers * d->hq * 4, 256);
  p.lse_i_off = off;
  off = align_up(off + R * 4, 256);
  p.part_off = off;
  off = align_up(off + R * p.n_kb * 4, 256);
  p.bytes = off;
  return p;
}

size_t workspace_bytes(const clsa_dims* d, const clsa_rows* r, int schedule, int prefill_chunk_rows) {
  size_t m = topk_workspace(d, r);
  // a standalone clsa_sparse_attn call may cover any number of layers up to L
  for (int l = 1; l <= d->n_layers; ++l) {
    const size_t a = attn_workspace(plan_attn(d, r->n_rows, l, 0));
    if (a > m) m = a;
  }
  const StepPlan s = plan_step(d, r, schedule, false, false, prefill_chunk_rows);
  if (s.total > m) m = s.total;
  return m < 256 ? 256 : m;
}

}  // namespace clsa
