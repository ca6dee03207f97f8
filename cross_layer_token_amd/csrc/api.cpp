// The C ABI of include/clsa.h: validate on the host, then enqueue the kernels on the stream.
#include <cstring>
#include <string>

#include "clsa_internal.h"

using namespace clsa;

namespace {

thread_local std::string g_last_error;

clsa_status set_error(clsa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

// Every check writes its message into g_err; CLSA_TRY forwards it to the thread-local slot.
#define CLSA_TRY(expr)                              \
  do {                                              \
    const clsa_status _s = (expr);                  \
    if (_s != CLSA_OK) return set_error(_s, g_err); \
  } while (0)

thread_local std::string g_err;

clsa_status device_status(int err, const char* what) {
  if (err == 0) return CLSA_OK;
  return set_error(CLSA_ERR_DEVICE, std::string(what) + ": " + device_error_string(err));
}

RowsDev rows_dev(const clsa_rows* r, const int32_t* cu) {
  RowsDev d;
  d.mode = r->mode;
  d.n_rows = r->n_rows;
  d.seq = r->seq;
  d.pos0 = r->pos0;
  d.max_row_len = r->max_row_len;
  d.total_tokens = r->total_tokens;
  d.cu = cu;
  return d;
}

clsa_status check_common(const clsa_dims* dims, const clsa_rows* rows) {
  CLSA_TRY(check_dims(dims, g_err));
  CLSA_TRY(check_rows(dims, rows, g_err));
  return CLSA_OK;
}

clsa_status check_ld(int64_t ld, const clsa_rows* rows, const char* name) {
  if (ld < rows->max_row_len) return set_error(CLSA_ERR_INVALID_ARGUMENT, std::string(name) + " < rows.max_row_len");
  if (ld % 4 != 0) return set_error(CLSA_ERR_INVALID_ARGUMENT, std::string(name) + " must be a multiple of 4");
  return CLSA_OK;
}

clsa_status check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return CLSA_OK;
  if (ws == nullptr || have < need)
    return set_error(CLSA_ERR_WORKSPACE, "workspace of " + std::to_string(have) + " bytes given, " +
                                             std::to_string(need) + " needed");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return set_error(CLSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return CLSA_OK;
}

clsa_status check_attn_strides(const clsa_dims* d, int lc, int64_t q_stride, int64_t o_stride) {
  const int64_t need = (int64_t)lc * d->hq * CLSA_HEAD_DIM;
  if (q_stride < need || o_stride < need)
    return set_error(CLSA_ERR_INVALID_ARGUMENT, "row stride smaller than n_layers_call * hq * 128");
  if (q_stride % 8 != 0 || o_stride % 8 != 0)
    return set_error(CLSA_ERR_INVALID_ARGUMENT, "row strides must be multiples of 8 elements");
  return CLSA_OK;
}

}  // namespace

extern "C" {

const char* clsa_status_string(clsa_status s) {
  switch (s) {
    case CLSA_OK: return "CLSA_OK";
    case CLSA_ERR_INVALID_ARGUMENT: return "CLSA_ERR_INVALID_ARGUMENT";
    case CLSA_ERR_UNSUPPORTED: return "CLSA_ERR_UNSUPPORTED";
    case CLSA_ERR_WORKSPACE: return "CLSA_ERR_WORKSPACE";
    case CLSA_ERR_DEVICE: return "CLSA_ERR_DEVICE";
  }
  return "CLSA_STATUS_UNKNOWN";
}

const char* clsa_last_error_message(void) { return g_last_error.c_str(); }

int32_t clsa_abi_version(void) { return CLSA_ABI_VERSION; }

size_t clsa_workspace_bytes(const clsa_dims* dims, const clsa_rows* rows, int32_t schedule,
                            int32_t prefill_chunk_rows) {
  if (check_common(dims, rows) != CLSA_OK) return 0;
  if (schedule != CLSA_SCHEDULE_LAYER_BATCHED && schedule != CLSA_SCHEDULE_PER_LAYER &&
      schedule != CLSA_SCHEDULE_PER_LAYER_ROUTING) {
    set_error(CLSA_ERR_INVALID_ARGUMENT, "unknown schedule");
    return 0;
  }
  if (prefill_chunk_rows < 0) {
    set_error(CLSA_ERR_INVALID_ARGUMENT, "prefill_chunk_rows must be >= 0");
    return 0;
  }
  return workspace_bytes(dims, rows, schedule, prefill_chunk_rows);
}

clsa_status clsa_index_scores(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* q_idx,
                              const clsa_bf16* k_idx, const int32_t* cu_seqlens, float* scores, int64_t ld_scores,
                              clsa_stream stream) {
  g_last_error.clear();
  CLSA_TRY(check_common(dims, rows));
  CLSA_TRY(check_ptr(q_idx, "q_idx", g_err));
  CLSA_TRY(check_ptr(k_idx, "k_idx", g_err));
  CLSA_TRY(check_ptr(cu_seqlens, "cu_seqlens", g_err));
  CLSA_TRY(check_ptr(scores, "scores", g_err));
  if (clsa_status s = check_ld(ld_scores, rows, "ld_scores"); s != CLSA_OK) return s;
  const RowsDev rd = rows_dev(rows, cu_seqlens);
  int e;
  if (rows->mode == CLSA_MODE_DECODE)
    e = launch_index_scores_decode(rd, dims->d_idx, idx_seg_for(rows->total_tokens), q_idx, dims->d_idx, k_idx,
                                   scores, ld_scores, nullptr, nullptr, 0, 0, nullptr, 0, stream);
  else
    e = launch_index_scores_prefill(rd, dims->d_idx, q_idx, k_idx, scores, ld_scores, nullptr, 0, stream);
  return device_status(e, "clsa_index_scores");
}

clsa_status clsa_index_project(const clsa_dims* dims, const clsa_rows* rows, int32_t d_model, const clsa_bf16* h,
                               const clsa_bf16* w_q_idx, const clsa_bf16* w_k_idx, const int32_t* cu_seqlens,
                               clsa_bf16* q_idx, clsa_bf16* k_idx, const clsa_bf16* k_new, const clsa_bf16* v_new,
                               clsa_bf16* k_cache, clsa_bf16* v_cache, clsa_stream stream) {
  g_last_error.clear();
  CLSA_TRY(check_common(dims, rows));
  if (rows->mode != CLSA_MODE_DECODE)
    return set_error(CLSA_ERR_UNSUPPORTED, "clsa_index_project appends one new token per sequence: DECODE rows only");
  if (d_model < 32 || d_model > CLSA_MAX_D_MODEL || d_model % 32 != 0)
    return set_error(CLSA_ERR_UNSUPPORTED, "d_model must be a multiple of 32 in [32, CLSA_MAX_D_MODEL]");
  CLSA_TRY(check_ptr(h, "h", g_err));
  CLSA_TRY(check_ptr(w_q_idx, "w_q_idx", g_err));
  CLSA_TRY(check_ptr(w_k_idx, "w_k_idx", g_err));
  CLSA_TRY(check_ptr(cu_seqlens, "cu_seqlens", g_err));
  CLSA_TRY(check_ptr(q_idx, "q_idx", g_err));
  CLSA_TRY(check_ptr(k_idx, "k_idx", g_err));
  if ((k_new == nullptr) != (v_new == nullptr))
    return set_error(CLSA_ERR_INVALID_ARGUMENT, "k_new and v_new must be given together");
  if (k_new != nullptr) {
    CLSA_TRY(check_ptr(k_new, "k_new", g_err));
    CLSA_TRY(check_ptr(v_new, "v_new", g_err));
    CLSA_TRY(check_ptr(k_cache, "k_cache", g_err));
    CLSA_TRY(check_ptr(v_cache, "v_cache", g_err));
  }
  return device_status(launch_index_project(dims->batch, dims->d_idx, d_model, dims->hkv, rows->total_tokens, h,
                                            w_q_idx, w_k_idx, cu_seqlens, q_idx, k_idx, k_new, v_new, k_cache,
                                            v_cache, stream),
                       "clsa_index_project");
}

size_t clsa_distill_workspace_bytes(const clsa_dims* dims, const clsa_rows* rows) {
  if (check_common(dims, rows) != CLSA_OK) return 0;
  if (rows->mode != CLSA_MODE_PREFILL) {
    set_error(CLSA_ERR_UNSUPPORTED, "the distillation loss is defined on PREFILL rows");
    return 0;
  }
  return plan_distill(dims, rows).bytes;
}

clsa_status clsa_distill_kl(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* q, int64_t q_row_stride,
                            const clsa_bf16* k_cache, const int32_t* cu_seqlens, const float* scores,
                            int64_t ld_scores, float* kl, float* loss, void* workspace, size_t workspace_bytes_,
                            clsa_stream stream) {
  g_last_error.clear();
  CLSA_TRY(check_common(dims, rows));
  if (rows->mode != CLSA_MODE_PREFILL)
    return set_error(CLSA_ERR_UNSUPPORTED, "the distillation loss is defined on PREFILL rows");
  CLSA_TRY(check_ptr(q, "q", g_err));
  CLSA_TRY(check_ptr(k_cache, "k_cache", g_err));
  CLSA_TRY(check_ptr(cu_seqlens, "cu_seqlens", g_err));
  CLSA_TRY(check_ptr(scores, "scores", g_err));
  CLSA_TRY(check_ptr(kl, "kl", g_err));
  if (loss != nullptr && reinterpret_cast<uintptr_t>(loss) % 4 != 0)
    return set_error(CLSA_ERR_INVALID_ARGUMENT, "loss is not 4-byte aligned");
  if (clsa_status s = check_ld(ld_scores, rows, "ld_scores"); s != CLSA_OK) return s;
  if (clsa_status s = check_attn_strides(dims, dims->n_layers, q_row_stride, q_row_stride); s != CLSA_OK) return s;
  const DistillPlan plan = plan_distill(dims, rows);
  if (clsa_status s = check_workspace(workspace, workspace_bytes_, plan.bytes); s != CLSA_OK) return s;
  return device_status(launch_distill(rows_dev(rows, cu_seqlens), rows->total_tokens, dims->n_layers, dims->hq, dims->hkv,
                                      softmax_scale(dims), q, q_row_stride, k_cache, scores, ld_scores, kl, loss,
                                      workspace, plan, stream),
                       "clsa_distill_kl");
}

clsa_status clsa_topk(const clsa_dims* dims, const clsa_rows* rows, const int32_t* cu_seqlens, const float* scores,
                      int64_t ld_scores, int32_t* idx, int32_t* count, void* workspace, size_t workspace_bytes_,
                      clsa_stream stream) {
  g_last_error.clear();
  CLSA_TRY(check_common(dims, rows));
  CLSA_TRY(check_ptr(cu_seqlens, "cu_seqlens", g_err));
  CLSA_TRY(check_ptr(scores, "scores", g_err));
  CLSA_TRY(check_ptr(idx, "idx", g_err));
  CLSA_TRY(check_ptr(count, "count", g_err));
  if (clsa_status s = check_ld(ld_scores, rows, "ld_scores"); s != CLSA_OK) return s;
  const TopkPlan plan = plan_topk(dims, rows);
  if (clsa_status s = check_workspace(workspace, workspace_bytes_, topk_workspace(dims, rows)); s != CLSA_OK)
    return s;
  const RowsDev rd = rows_dev(rows, cu_seqlens);
  return device_status(launch_topk(rd, dims->topk, plan, scores, ld_scores, idx, count, workspace, false, stream),
                       "clsa_topk");
}

clsa_status clsa_gather_kv(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* k_cache,
                           const clsa_bf16* v_cache, const int32_t* cu_seqlens, const int32_t* idx,
                           const int32_t* count, clsa_bf16* k_sel, clsa_bf16* v_sel, clsa_stream stream) {
  g_last_error.clear();
  CLSA_TRY(check_common(dims, rows));
  CLSA_TRY(check_ptr(k_cache, "k_cache", g_err));
  CLSA_TRY(check_ptr(v_cache, "v_cache", g_err));
  CLSA_TRY(check_ptr(cu_seqlens, "cu_seqlens", g_err));
  CLSA_TRY(check_ptr(idx, "idx", g_err));
  CLSA_TRY(check_ptr(count, "count", g_err));
  CLSA_TRY(check_ptr(k_sel, "k_sel", g_err));
  CLSA_TRY(check_ptr(v_sel, "v_sel", g_err));
  const RowsDev rd = rows_dev(rows, cu_seqlens);
  return device_status(
      launch_gather(rd, dims->topk, dims->hkv, k_cache, v_cache, idx, count, k_sel, v_sel, stream), "clsa_gather_kv");
}

clsa_status clsa_sparse_attn(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* q, int64_t q_row_stride,
                             int32_t n_layers_call, const clsa_bf16* k_sel, const clsa_bf16* v_sel,
                             const clsa_bf16* k_cache, const clsa_bf16* v_cache, const int32_t* cu_seqlens,
                             const int32_t* idx, const int32_t* count, clsa_bf16* out, int64_t out_row_stride,
                             void* workspace, size_t workspace_bytes_, clsa_stream stream) {
  g_last_error.clear();
  CLSA_TRY(check_common(dims, rows));
  if (n_layers_call < 1 || n_layers_call > dims->n_layers)
    return set_error(CLSA_ERR_UNSUPPORTED, "n_layers_call must be in [1, n_layers]");
  CLSA_TRY(check_ptr(q, "q", g_err));
  CLSA_TRY(check_ptr(out, "out", g_err));
  CLSA_TRY(check_ptr(count, "count", g_err));
  CLSA_TRY(check_ptr(cu_seqlens, "cu_seqlens", g_err));
  const bool compact = k_sel != nullptr || v_sel != nullptr;
  if (compact) {
    CLSA_TRY(check_ptr(k_sel, "k_sel", g_err));
    CLSA_TRY(check_ptr(v_sel, "v_sel", g_err));
  } else {
    CLSA_TRY(check_ptr(k_cache, "k_cache", g_err));
    CLSA_TRY(check_ptr(v_cache, "v_cache", g_err));
    CLSA_TRY(check_ptr(idx, "idx", g_err));
  }
  if (clsa_status s = check_attn_strides(dims, n_layers_call, q_row_stride, out_row_stride); s != CLSA_OK) return s;
  const AttnPlan plan = plan_attn(dims, rows->n_rows, n_layers_call, 0);
  if (clsa_status s = check_workspace(workspace, workspace_bytes_, attn_workspace(plan)); s != CLSA_OK) return s;
  const RowsDev rd = rows_dev(rows, cu_seqlens);
  char* ws = static_cast<char*>(workspace);
  return device_status(launch_attn(rd, dims->topk, dims->hq, dims->hkv, n_layers_call, softmax_scale(dims), plan, q,
                                   q_row_stride, compact ? k_sel : nullptr, compact ? v_sel : nullptr, k_cache,
                                   v_cache, idx, count, out, out_row_stride, ws + ticket_region(plan.tickets),
                                   reinterpret_cast<uint32_t*>(ws), false, stream),
                       "clsa_sparse_attn");
}

}  // extern "C"

namespace {

// Every check of clsa_step's arguments except the workspace.
clsa_status check_step_args(const clsa_dims* dims, const clsa_rows* rows, const clsa_step_args* a) {
  CLSA_TRY(check_common(dims, rows));
  if (a == nullptr) return set_error(CLSA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->schedule != CLSA_SCHEDULE_LAYER_BATCHED && a->schedule != CLSA_SCHEDULE_PER_LAYER &&
      a->schedule != CLSA_SCHEDULE_PER_LAYER_ROUTING)
    return set_error(CLSA_ERR_INVALID_ARGUMENT, "unknown schedule");
  if (a->prefill_chunk_rows < 0) return set_error(CLSA_ERR_INVALID_ARGUMENT, "prefill_chunk_rows must be >= 0");
  CLSA_TRY(check_ptr(a->q_idx, "q_idx", g_err));
  CLSA_TRY(check_ptr(a->k_idx, "k_idx", g_err));
  CLSA_TRY(check_ptr(a->k_cache, "k_cache", g_err));
  CLSA_TRY(check_ptr(a->v_cache, "v_cache", g_err));
  CLSA_TRY(check_ptr(a->cu_seqlens, "cu_seqlens", g_err));
  CLSA_TRY(check_ptr(a->q, "q", g_err));
  CLSA_TRY(check_ptr(a->out, "out", g_err));
  CLSA_TRY(check_ptr(a->idx, "idx", g_err));
  CLSA_TRY(check_ptr(a->count, "count", g_err));
  CLSA_TRY(check_ptr_opt(a->scores, "scores", g_err));
  CLSA_TRY(check_ptr_opt(a->k_sel, "k_sel", g_err));
  CLSA_TRY(check_ptr_opt(a->v_sel, "v_sel", g_err));
  if ((a->k_sel == nullptr) != (a->v_sel == nullptr))
    return set_error(CLSA_ERR_INVALID_ARGUMENT, "k_sel and v_sel must both be given or both be NULL");
  if (a->scores != nullptr)
    if (clsa_status s = check_ld(a->ld_scores, rows, "ld_scores"); s != CLSA_OK) return s;
  const bool prefill = rows->mode == CLSA_MODE_PREFILL;
  if (a->schedule == CLSA_SCHEDULE_PER_LAYER_ROUTING) {
    if (prefill) return set_error(CLSA_ERR_UNSUPPORTED, "per-layer routing is a DECODE schedule");
    if (a->scores != nullptr || a->k_sel != nullptr)
      return set_error(CLSA_ERR_INVALID_ARGUMENT, "per-layer routing takes no scores, k_sel or v_sel");
  }
  return CLSA_OK;
}

}  // namespace

extern "C" {

clsa_status clsa_step(const clsa_dims* dims, const clsa_rows* rows, const clsa_step_args* a, void* workspace,
                      size_t workspace_bytes_, clsa_stream stream) {
  g_last_error.clear();
  if (clsa_status s = check_step_args(dims, rows, a); s != CLSA_OK) return s;
  const bool prefill = rows->mode == CLSA_MODE_PREFILL;
  const StepPlan sp = plan_step(dims, rows, a->schedule, a->scores != nullptr, a->k_sel != nullptr,
                                a->prefill_chunk_rows);
  if (clsa_status s = check_workspace(workspace, workspace_bytes_, sp.total); s != CLSA_OK) return s;

  char* ws = static_cast<char*>(workspace);
  const int L = dims->n_layers, hq = dims->hq, hkv = dims->hkv, k = dims->topk;
  const int64_t row_elems = (int64_t)L * hq * CLSA_HEAD_DIM;
  const float scale = softmax_scale(dims);
  const int chunk = sp.chunk_rows;
  // attention tickets, one per (row, KV head, query block); the chunk's first kernel clears them
  uint32_t* tickets = reinterpret_cast<uint32_t*>(ws + sp.ticket_off);
  uint32_t* attn_tickets = tickets;
  if (a->schedule == CLSA_SCHEDULE_PER_LAYER_ROUTING) {
    // the ablation: score, select and attend once per layer, each layer with its own query
    const RowsDev rd = rows_dev(rows, a->cu_seqlens);
    const TopkPlan tp = plan_topk(dims, rows);
    char* topk_ws = ws + sp.topk_off;
    float* scores = reinterpret_cast<float*>(ws + sp.scores_off);
    const AttnPlan ap = plan_attn(dims, rows->n_rows, 1, rows->n_rows);
    const int R = rows->n_rows;
    const int iseg = tp.multi_wg ? tp.hist_chunk : idx_seg_for(rows->total_tokens);
    // as in the layer-batched step, the attention workgroups finish each layer's long-row selection
    const bool fused = tp.multi_wg && ap.teams == 2 && ap.wpt == 4 && ap.keys_per_split <= kFusedMaxIds;
    SelectIn sel;
    if (fused) {
      sel.slot = topk_ws + tp.slot_off;
      sel.cnt = reinterpret_cast<const uint32_t*>(topk_ws + tp.cnt_off);
      sel.rowinfo = reinterpret_cast<const uint32_t*>(topk_ws + tp.rowinfo_off);
      sel.spans = tp.spans;
    }
    for (int l = 0; l < L; ++l) {
      uint16_t* hpart = tp.multi_wg ? reinterpret_cast<uint16_t*>(topk_ws + tp.hpart_off) : nullptr;
      uint32_t* hinfo = tp.multi_wg ? reinterpret_cast<uint32_t*>(topk_ws + tp.hinfo_off) : nullptr;
      int e = launch_index_scores_decode(rd, dims->d_idx, iseg, a->q_idx + (int64_t)l * dims->d_idx,
                                         (int64_t)L * dims->d_idx, a->k_idx, scores, sp.ld_scores, hpart, hinfo, k,
                                         tp.hist_chunks, tickets, sp.n_tickets, stream);
      if (e) return device_status(e, "clsa_step: index scores of a layer");
      int32_t* idx = a->idx + (int64_t)l * R * k;
      int32_t* count = a->count + (int64_t)l * R;
      e = launch_topk(rd, k, tp, scores, sp.ld_scores, idx, count, topk_ws, tp.multi_wg, stream,
                      !fused);
      if (e) return device_status(e, "clsa_step: top-k of a layer");
      e = launch_attn(rd, k, hq, hkv, 1, scale, ap, a->q + (int64_t)l * hq * CLSA_HEAD_DIM, row_elems, nullptr,
                      nullptr, a->k_cache, a->v_cache, idx, count, a->out + (int64_t)l * hq * CLSA_HEAD_DIM, row_elems,
                      ws + sp.part_off, attn_tickets, true, stream, fused ? &sel : nullptr, idx, count);
      if (e) return device_status(e, "clsa_step: attention of a layer");
    }
    return CLSA_OK;
  }
  for (int c0 = 0; c0 < rows->n_rows; c0 += chunk) {
    clsa_rows cr = *rows;
    cr.n_rows = rows->n_rows - c0 < chunk ? rows->n_rows - c0 : chunk;
    if (prefill) {
      cr.pos0 = rows->pos0 + c0;
      cr.max_row_len = cr.pos0 + cr.n_rows;
    }
    const RowsDev rd = rows_dev(&cr, a->cu_seqlens);
    float* scores;
    int64_t ld;
    if (a->scores != nullptr) {
      scores = a->scores + (int64_t)c0 * a->ld_scores;
      ld = a->ld_scores;
    } else {
      scores = reinterpret_cast<float*>(ws + sp.scores_off);
      ld = sp.ld_scores;
    }
    const TopkPlan tp = plan_topk(dims, &cr);
    char* topk_ws = ws + sp.topk_off;
    const clsa_bf16* q_idx = a->q_idx + (int64_t)c0 * dims->d_idx;
    int e;
    bool have_hist = false;
    if (prefill) {
      e = launch_index_scores_prefill(rd, dims->d_idx, q_idx, a->k_idx, scores, ld, tickets, sp.n_tickets, stream);
    } else {
      uint16_t* hpart = tp.multi_wg ? reinterpret_cast<uint16_t*>(topk_ws + tp.hpart_off) : nullptr;
      uint32_t* hinfo = tp.multi_wg ? reinterpret_cast<uint32_t*>(topk_ws + tp.hinfo_off) : nullptr;
      have_hist = tp.multi_wg;
      const int seg = tp.multi_wg ? tp.hist_chunk : idx_seg_for(cr.total_tokens);
      e = launch_index_scores_decode(rd, dims->d_idx, seg, q_idx, dims->d_idx, a->k_idx, scores, ld, hpart, hinfo,
                                     k, tp.hist_chunks, tickets, sp.n_tickets, stream);
    }
    if (e) return device_status(e, "clsa_step: index scores");
    int32_t* idx = a->idx + (int64_t)c0 * k;
    int32_t* count = a->count + c0;
    // the layer-batched decode step lets the attention workgroups finish the long-row selection
    e = launch_topk(rd, k, tp, scores, ld, idx, count, topk_ws, have_hist, stream, !sp.fused_select);
    if (e) return device_status(e, "clsa_step: top-k");
    const clsa_bf16* q = a->q + (int64_t)c0 * row_elems;
    clsa_bf16* out = a->out + (int64_t)c0 * row_elems;
    if (a->schedule == CLSA_SCHEDULE_LAYER_BATCHED) {
      const AttnPlan ap = plan_attn(dims, cr.n_rows, L, rows->n_rows);
      SelectIn sel;
      if (sp.fused_select) {
        sel.slot = topk_ws + tp.slot_off;
        sel.cnt = reinterpret_cast<const uint32_t*>(topk_ws + tp.cnt_off);
        sel.rowinfo = reinterpret_cast<const uint32_t*>(topk_ws + tp.rowinfo_off);
        sel.spans = tp.spans;
      }
      e = launch_attn(rd, k, hq, hkv, L, scale, ap, q, row_elems, nullptr, nullptr, a->k_cache, a->v_cache, idx, count,
                      out, row_elems, ws + sp.part_off, attn_tickets, true, stream, sp.fused_select ? &sel : nullptr,
                      idx, count);
      if (e) return device_status(e, "clsa_step: attention");
    } else if (prefill) {
      // prefill rows gather their own selections inside the attention (no compact buffer)
      const AttnPlan ap = plan_attn(dims, cr.n_rows, 1, rows->n_rows);
      for (int l = 0; l < L; ++l) {
        e = launch_attn(rd, k, hq, hkv, 1, scale, ap, q + (int64_t)l * hq * CLSA_HEAD_DIM, row_elems, nullptr, nullptr,
                        a->k_cache, a->v_cache, idx, count, out + (int64_t)l * hq * CLSA_HEAD_DIM, row_elems,
                        ws + sp.part_off, attn_tickets, true, stream);
        if (e) return device_status(e, "clsa_step: attention layer");
      }
    } else {
      // decode: gather K_S/V_S of a chunk of rows into the compact buffers, then the L passes over
      // them while they are cache-resident; decode row r is sequence r, so a chunk's rows are the
      // sequences s0.. and read cu_seqlens from s0
      const int sc = sp.sel_chunk_rows;
      const size_t sel_row = (size_t)hkv * k * CLSA_HEAD_DIM;
      for (int s0 = 0; s0 < cr.n_rows; s0 += sc) {
        RowsDev rs = rd;
        rs.n_rows = cr.n_rows - s0 < sc ? cr.n_rows - s0 : sc;
        rs.cu = rd.cu + s0;
        const AttnPlan ap = plan_attn(dims, rs.n_rows, 1, rs.n_rows);
        clsa_bf16* ksel = a->k_sel ? a->k_sel + s0 * sel_row : reinterpret_cast<clsa_bf16*>(ws + sp.ksel_off);
        clsa_bf16* vsel = a->v_sel ? a->v_sel + s0 * sel_row : reinterpret_cast<clsa_bf16*>(ws + sp.vsel_off);
        const int32_t* cidx = idx + (int64_t)s0 * k;
        const int32_t* ccnt = count + s0;
        e = launch_gather(rs, k, hkv, a->k_cache, a->v_cache, cidx, ccnt, ksel, vsel, stream);
        if (e) return device_status(e, "clsa_step: gather");
        const clsa_bf16* cq = q + (int64_t)s0 * row_elems;
        clsa_bf16* cout = out + (int64_t)s0 * row_elems;
        for (int l = 0; l < L; ++l) {
          e = launch_attn(rs, k, hq, hkv, 1, scale, ap, cq + (int64_t)l * hq * CLSA_HEAD_DIM, row_elems, ksel, vsel,
                          a->k_cache, a->v_cache, cidx, ccnt, cout + (int64_t)l * hq * CLSA_HEAD_DIM, row_elems,
                          ws + sp.part_off, attn_tickets, true, stream);
          if (e) return device_status(e, "clsa_step: attention layer");
        }
      }
    }
  }
  return CLSA_OK;
}

clsa_status clsa_step_no_alloc(const clsa_dims* dims, const clsa_rows* rows, const clsa_step_args* args,
                               clsa_stream stream) {
  g_last_error.clear();
  if (clsa_status s = check_step_args(dims, rows, args); s != CLSA_OK) return s;
  const StepPlan sp = plan_step(dims, rows, args->schedule, args->scores != nullptr, args->k_sel != nullptr,
                                args->prefill_chunk_rows);
  if (sp.total > kNoAllocScratchBytes)
    return set_error(CLSA_ERR_UNSUPPORTED, "clsa_step_no_alloc: this call needs " + std::to_string(sp.total) +
                                               " bytes of scratch; the static scratch holds " +
                                               std::to_string(kNoAllocScratchBytes) +
                                               " (use clsa_step with a workspace, smaller prefill chunks, or "
                                               "caller-owned scores / k_sel / v_sel)");
  void* ws = nullptr;
  if (int e = no_alloc_scratch(&ws, g_err); e != 0) return set_error(CLSA_ERR_DEVICE, "clsa_step_no_alloc: " + g_err);
  return clsa_step(dims, rows, args, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
