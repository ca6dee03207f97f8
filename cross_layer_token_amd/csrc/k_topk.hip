// Token-level TopK(I_t, k) - the second half of the routing equation on the picx.dev summary of
// "You Only Index Once" (Methodology > Architecture Overview, eq. 2), computed once per step.
//
// Selection rule: the first m = min(k, n) tokens in the order (score descending, index
// ascending), written in ascending index order.  Scores are mapped to order-preserving 32-bit
// keys; the m-th largest key T is found by radix select on integer histograms; then every token
// with key > T is taken, plus the lowest-index tokens with key == T until m are taken.  All
// decisions are integer counts, so the result is unique and independent of thread timing.
//
// Short rows (<= kLdsRowCap): one workgroup per row holds the row's keys in LDS.
// Long rows: a first-level histogram of the top key bits comes in partials (written by the
// score kernel, or by k_topk_hist_partials); each select workgroup sums them, finds the bin
// holding T, and compacts its span's scores at or above that bin in index order; a second kernel
// with one workgroup per row (or the attention workgroups) finishes the selection over that
// short list.  No workgroup ever waits for another.
#include "select_common.h"

namespace clsa {

namespace {

constexpr int kRowThreads = 512;

__device__ void write_all(int32_t* out, int32_t* count, int r, int n, int k) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) out[(int64_t)r * k + i] = i < n ? i : -1;
  if (threadIdx.x == 0) count[r] = n;
}

// ---------------------------------------------------------------------------- short rows
// The bin (from the top bin down) whose cumulative count first reaches `need` among kTopkBins
// 16-bit counts packed two per word (bin b in half b & 1 of word b >> 1): res[0] = the bin,
// res[1] = the count of the bins above it.  NT threads each own kTopkBins / NT consecutive bins;
// all must call it; it ends with __syncthreads().
static_assert(kLdsRowCap < 65536, "a short row's bin counts fit 16 bits");

template <int NT>
__device__ void find_packed_bin_from_top(const uint32_t* hpk, int need, int* scan, int* res) {
  constexpr int B = kTopkBins / NT;
  static_assert(kTopkBins % NT == 0, "whole bins per thread");
  const int hi = kTopkBins - 1 - B * (int)threadIdx.x;
  int h[B], loc = 0;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int b = hi - j;
    h[j] = (int)((hpk[b >> 1] >> ((b & 1) * 16)) & 0xFFFFu);
    loc += h[j];
  }
  int total;
  int run = block_exclusive_scan(loc, scan, &total);
#pragma unroll
  for (int j = 0; j < B; ++j) {
    if (run < need && run + h[j] >= need) {
      res[0] = hi - j;
      res[1] = run;
    }
    run += h[j];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kRowThreads) void k_topk_rows_lds(RowsDev rw, const float* __restrict__ scores,
                                                                 int64_t ld, int k, int32_t* __restrict__ out,
                                                                 int32_t* __restrict__ count) {
  // the row's keys: dynamic LDS sized for the launch's longest row (at most kLdsRowCap keys), so
  // that shorter rows leave room for more workgroups per CU
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hpk[kTopkBins / 2];  // the first level's counts, 16 bits each (a row holds < 2^16 keys)
  __shared__ uint32_t hist[256];           // the 8-bit passes
  __shared__ int scan[2 * kRowThreads / 64];
  __shared__ int res[2];
  const int r = blockIdx.x;
  const int n = row_len(rw, r);
  const int m = n < k ? n : k;
  if (m == n) {
    write_all(out, count, r, n, k);
    return;
  }
  const float* srow = scores + (int64_t)r * ld;
  for (int i = threadIdx.x; i < kTopkBins / 2; i += blockDim.x) hpk[i] = 0u;
  __syncthreads();
  // First level: the top kTopkBinBits key bits (sign, exponent, two mantissa bits), the same bins
  // as the long-row select, counted in 16-bit halves of LDS words.
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint32_t key = score_key(srow[i]);
    const uint32_t bin = key >> (32 - kTopkBinBits);
    keys[i] = key;
    atomicAdd(&hpk[bin >> 1], 1u << ((bin & 1u) * 16u));
  }
  __syncthreads();
  find_packed_bin_from_top<kRowThreads>(hpk, m, scan, res);
  uint32_t prefix = (uint32_t)res[0] << (32 - kTopkBinBits), pmask = ~0u << (32 - kTopkBinBits);
  int need = m - res[1];
  auto key_at = [&](int i) { return keys[i]; };
  // then 8-bit passes below it, the last aligned to bit 0 (its window overlaps bits the prefix
  // already fixes, which then match)
  for (int shift = 32 - kTopkBinBits - 8;; shift -= 8) {
    if (shift < 0) shift = 0;
    radix_pass8(hist, n, key_at, prefix, pmask, shift, need, res);
    if (shift == 0) break;
  }
  const uint32_t T = prefix;  // the m-th largest key; `need` ties at T are taken
  // ordered compaction: thread t owns the contiguous element range [t*E, t*E + E)
  const int E = (n + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * E;
  int gt = 0, eq = 0;
  for (int j = 0; j < E; ++j) {
    const int i = i0 + j;
    if (i < n) {
      const uint32_t key = keys[i];
      gt += key > T;
      eq += key == T;
    }
  }
  int gt_before, eq_before, t0, t1;
  block_exclusive_scan2(gt, eq, scan, &gt_before, &eq_before, &t0, &t1);
  int32_t* orow = out + (int64_t)r * k;
  for (int j = 0; j < E; ++j) {
    const int i = i0 + j;
    if (i < n) {
      const uint32_t key = keys[i];
      const bool take = key > T || (key == T && eq_before < need);
      if (take) orow[gt_before + (eq_before < need ? eq_before : need)] = i;
      gt_before += key > T;
      eq_before += key == T;
    }
  }
  for (int i = m + threadIdx.x; i < k; i += blockDim.x) orow[i] = -1;
  if (threadIdx.x == 0) count[r] = m;
}

// ---------------------------------------------------------------------------- long rows
struct SelectArgs {
  RowsDev rw;
  const float* scores;
  int64_t ld;
  int k;
  int32_t* out;
  int32_t* count;
  uint16_t* hpart;        // [R, hist_chunks, kTopkBins] per-piece histograms of key >> (32 - kTopkBinBits)
  uint32_t* hinfo;        // [R, hist_chunks] window start | full flag of each partial (write_hist_partial)
  int hist_chunk;         // tokens per partial
  int hist_chunks;
  int hist_flat;          // 1: the decode score kernel's partials, one per (row, segment of the
                          // concatenated sequences); 0: per-row chunks from k_topk_hist_partials
  int span_flat;          // 1 (decode): blockIdx.x enumerates the (row, span) pairs that exist
  uint32_t* cnt;          // [R, spans]
  int spans;
  uint2* slot;            // [R, max_row_len]
  uint2* list;            // [R, max_row_len]
  uint32_t* rowinfo;      // [R, 2]: t1 and the count above it
};

constexpr int kSelThreads = 1024;
constexpr int kHistThreads = 256;

// Histogram partials of the scores (used when no score kernel produced them).
__global__ __launch_bounds__(kHistThreads) void k_topk_hist_partials(SelectArgs a) {
  __shared__ uint32_t hist[kTopkBins];
  __shared__ int scan[2 * kHistThreads / 64];
  __shared__ int res[4];
  const int r = blockIdx.y, c = blockIdx.x;
  const int n = row_len(a.rw, r);
  const int t0 = c * a.hist_chunk;
  if (t0 >= n || (n <= a.k)) return;
  const int t1 = t0 + a.hist_chunk < n ? t0 + a.hist_chunk : n;
  for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  const float* srow = a.scores + (int64_t)r * a.ld;
  constexpr int PER = 8;
  for (int i0 = t0 + threadIdx.x; i0 < t1; i0 += PER * kHistThreads) {
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = i0 + j * kHistThreads;
      v[j] = i < t1 ? srow[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (i0 + j * kHistThreads < t1) atomicAdd(&hist[score_key(v[j]) >> (32 - kTopkBinBits)], 1u);
  }
  __syncthreads();
  uint32_t* hp = reinterpret_cast<uint32_t*>(a.hpart + ((int64_t)r * a.hist_chunks + c) * kTopkBins);
  write_hist_partial<kHistThreads>(hist, t1 - t0, a.k, hp, a.hinfo + (int64_t)r * a.hist_chunks + c, scan, res);
}

// Long-row select, first kernel.  Workgroup (span, row) handles scores [span * kSelectSpan,
// +kSelectSpan).
//  1. Sum the row's histogram partials (exact from the largest window start up, see
//     write_hist_partial); find the bin t1 holding the m-th largest key.
//  2. Append (key, index) of every score whose bin is >= t1 to the span's slot, in index order,
//     and publish the span's count; span 0 publishes t1 and the count above it.
// The selection is then finished by k_topk_finish, or by the attention workgroups themselves.
static_assert(kMaxSelectSpans % kSelThreads == 0, "whole spans per select thread");
static_assert(kSelectSpan == kSelThreads * 8, "each select thread classifies 8 consecutive scores");

// Finds, in the kTopkBins-bin LDS histogram, the bin d (from the top bin down) whose cumulative
// count first reaches `need`, and publishes res[0] = d, res[1] = count of the bins above d.
// Thread t owns bins kTopkBins - 1 - 2t and kTopkBins - 2 - 2t; a block scan gives each thread
// the count above its pair.  All threads must call it; it ends with __syncthreads().
__device__ __forceinline__ void find_bin_from_top(const uint32_t* hist, int need, int* scan, int* res) {
  static_assert(kTopkBins == 2 * kSelThreads, "one bin pair per select thread");
  const int hi = kTopkBins - 1 - 2 * (int)threadIdx.x;
  const int h0 = (int)hist[hi], h1 = (int)hist[hi - 1];
  int total;
  const int above = block_exclusive_scan(h0 + h1, scan, &total);
  if (above < need && above + h0 >= need) {
    res[0] = hi;
    res[1] = above;
  } else if (above + h0 < need && above + h0 + h1 >= need) {
    res[0] = hi - 1;
    res[1] = above + h0;
  }
  __syncthreads();
}

// Decode: the (row, span) pair of flat workgroup w, enumerating each row's ceil(n / kSelectSpan)
// spans row after row (the grid holds an upper bound of them, so that a ragged batch launches no
// workgroup per span of its longest row for every row); {-1, -1} when w is past the last pair.
// All threads call it; it ends with __syncthreads().
__device__ int2 flat_span(const RowsDev& rw, int w, int* scan, int* found) {
  if (threadIdx.x == 0) {
    found[0] = -1;
    found[1] = -1;
  }
  int base = 0;
  for (int r0 = 0; r0 < rw.n_rows; r0 += kSelThreads) {  // uniform across the workgroup
    const int r = r0 + (int)threadIdx.x;
    const int n = r < rw.n_rows ? row_len(rw, r) : 0;
    const int c = (n + kSelectSpan - 1) / kSelectSpan;
    int total;
    const int pre = base + block_exclusive_scan(c, scan, &total);
    if (c > 0 && w >= pre && w < pre + c) {
      found[0] = r;
      found[1] = w - pre;
    }
    base += total;
  }
  __syncthreads();
  return make_int2(found[0], found[1]);
}

__global__ __launch_bounds__(kSelThreads) void k_topk_select(SelectArgs a) {
  __shared__ uint32_t hist[kTopkBins];
  __shared__ int scan[2 * kSelThreads / 64];
  __shared__ int res[2];
  __shared__ int any_full;
  __shared__ int found[2];
  int r = blockIdx.y, sp = blockIdx.x;
  if (a.span_flat) {
    const int2 rs = flat_span(a.rw, blockIdx.x, scan, found);
    if (rs.x < 0) return;
    r = rs.x;
    sp = rs.y;
  }
  const int n = row_len(a.rw, r);
  const int m = n < a.k ? n : a.k;
  const int s0 = sp * kSelectSpan;
  if (s0 >= n) return;
  const int s1 = s0 + kSelectSpan < n ? s0 + kSelectSpan : n;
  int32_t* orow = a.out + (int64_t)r * a.k;
  if (m == n) {  // every visible token is selected
    for (int i = s0 + threadIdx.x; i < s1; i += blockDim.x) orow[i] = i;
    if (sp == 0) {
      for (int i = n + threadIdx.x; i < a.k; i += blockDim.x) orow[i] = -1;
      if (threadIdx.x == 0) a.count[r] = n;
    }
    return;
  }
  // this thread's 8 consecutive scores (loaded first; the latency overlaps the histogram)
  const float* srow = a.scores + (int64_t)r * a.ld;
  const int i0 = s0 + threadIdx.x * 8;
  float x[8];
  if (i0 + 7 < s1) {
    const float4 v0 = *reinterpret_cast<const float4*>(srow + i0);
    const float4 v1 = *reinterpret_cast<const float4*>(srow + i0 + 4);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = i0 + j < s1 ? srow[i0 + j] : 0.f;
  }
  // 1. the row's histogram from the partials (exact from the largest window start up); a decode
  //    row's partials are those of the segments its tokens cu[r] .. cu[r] + n - 1 fall in
  const int hoff = a.hist_flat ? a.rw.cu[r] : 0;  // token offsets fit in 32 bits
  const int nch_row = (hoff + n - 1) / a.hist_chunk - hoff / a.hist_chunk + 1;
  const int nch = nch_row < a.hist_chunks ? nch_row : a.hist_chunks;
  sum_hist_partials<kSelThreads>(reinterpret_cast<const uint32_t*>(a.hpart + (int64_t)r * a.hist_chunks * kTopkBins),
                                 a.hinfo + (int64_t)r * a.hist_chunks, nch, hist, &any_full);
  find_bin_from_top(hist, m, scan, res);
  const uint32_t t1 = (uint32_t)res[0];
  const int above1 = res[1];
  // 2. ordered compaction of the span's scores with bin >= t1 into the span's slot
  uint32_t key[8];
  int c = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    key[j] = score_key(x[j]);
    c += (i0 + j < s1) && (key[j] >> (32 - kTopkBinBits)) >= t1;
  }
  int tot;
  int pos = block_exclusive_scan(c, scan, &tot);
  uint2* slot = a.slot + (int64_t)r * a.rw.max_row_len + s0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if ((i0 + j < s1) && (key[j] >> (32 - kTopkBinBits)) >= t1) {
      slot[pos] = make_uint2(key[j], (uint32_t)(i0 + j));
      ++pos;
    }
  }
  if (threadIdx.x == 0) {
    a.cnt[(int64_t)r * a.spans + sp] = (uint32_t)tot;
    if (sp == 0) {
      a.rowinfo[2 * r] = t1;
      a.rowinfo[2 * r + 1] = (uint32_t)above1;
    }
  }
}

// Long-row select, second kernel: one workgroup per row concatenates the span lists (in span
// order, so in token order; in LDS when they fit, else in the workspace), refines the exact m-th
// largest key T over the remaining key bits, and writes the selection in token order: keys above
// T, then the lowest-index ties at T up to m.
__global__ __launch_bounds__(kSelThreads) void k_topk_finish(SelectArgs a) {
  __shared__ uint32_t hist[512];
  __shared__ int scan[2 * kSelThreads / 64];
  __shared__ int res[4];
  __shared__ int span_pre[kMaxSelectSpans + 1];
  __shared__ uint2 list_lds[kListLds];
  const int r = blockIdx.x;
  const int n = row_len(a.rw, r);
  const int m = n < a.k ? n : a.k;
  if (m == n) return;  // every visible token is selected, written by the select
  // the span lists and counts come from the previous kernel: plain loads, requested at once
  CandidateLoads<kSelThreads, 1, kMaxSelectSpans> cq;
  const uint2* rslot = a.slot + (int64_t)r * a.rw.max_row_len;
  const int nsp = (n + kSelectSpan - 1) / kSelectSpan;
  request_candidates(cq, rslot, a.cnt + (int64_t)r * a.spans, nsp, n);
  const uint32_t t1 = a.rowinfo[2 * r];
  const int above1 = (int)a.rowinfo[2 * r + 1];
  uint2* glist = a.list + (int64_t)r * a.rw.max_row_len;
  const int L = complete_candidates(cq, rslot, nsp, span_pre, scan, list_lds, glist);
  int32_t* orow = a.out + (int64_t)r * a.k;
  auto emit = [&](int pos, int32_t tok) { orow[pos] = tok; };
  if (L <= kListLds) {
    static_assert(kListLds % kSelThreads == 0, "the LDS list fits the threads' registers");
    refine_and_emit_regs<kListLds / kSelThreads>(list_lds, L, m, t1, above1, hist, scan, res, emit);
  } else {
    refine_and_emit([&](int i) { return glist[i]; }, L, m, t1, above1, hist, scan, res, emit);
  }
  for (int i = m + threadIdx.x; i < a.k; i += blockDim.x) orow[i] = -1;
  if (threadIdx.x == 0) a.count[r] = m;
}

}  // namespace

int launch_topk(const RowsDev& rows, int k, const TopkPlan& plan, const float* scores, int64_t ld, int32_t* idx,
                int32_t* count, void* ws, bool have_hist, void* stream, bool finish) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!plan.multi_wg) {
    const size_t key_bytes = (size_t)(rows.max_row_len < kLdsRowCap ? rows.max_row_len : kLdsRowCap) * sizeof(uint32_t);
    hipLaunchKernelGGL(k_topk_rows_lds, dim3(rows.n_rows), dim3(kRowThreads), key_bytes, s, rows, scores, ld, k, idx,
                       count);
    return (int)hipGetLastError();
  }
  char* w = static_cast<char*>(ws);
  SelectArgs a;
  a.rw = rows;
  a.scores = scores;
  a.ld = ld;
  a.k = k;
  a.out = idx;
  a.count = count;
  a.hpart = reinterpret_cast<uint16_t*>(w + plan.hpart_off);
  a.hinfo = reinterpret_cast<uint32_t*>(w + plan.hinfo_off);
  a.hist_chunk = plan.hist_chunk;
  a.hist_chunks = plan.hist_chunks;
  a.hist_flat = have_hist ? 1 : 0;
  // decode rows: one workgroup per (row, span) that exists, at most T / kSelectSpan + R of them
  const bool flat = rows.mode == CLSA_MODE_DECODE;
  const int64_t flat_wgs = (rows.total_tokens + kSelectSpan - 1) / kSelectSpan + rows.n_rows;
  const bool use_flat = flat && flat_wgs < (int64_t)plan.spans * rows.n_rows;
  a.span_flat = use_flat ? 1 : 0;
  a.cnt = reinterpret_cast<uint32_t*>(w + plan.cnt_off);
  a.spans = plan.spans;
  a.slot = reinterpret_cast<uint2*>(w + plan.slot_off);
  a.list = reinterpret_cast<uint2*>(w + plan.list_off);
  a.rowinfo = reinterpret_cast<uint32_t*>(w + plan.rowinfo_off);
  if (!have_hist)
    hipLaunchKernelGGL(k_topk_hist_partials, dim3(plan.hist_chunks, rows.n_rows), dim3(kHistThreads), 0, s, a);
  if (use_flat)
    hipLaunchKernelGGL(k_topk_select, dim3((unsigned)flat_wgs), dim3(kSelThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_topk_select, dim3(plan.spans, rows.n_rows), dim3(kSelThreads), 0, s, a);
  if (finish) hipLaunchKernelGGL(k_topk_finish, dim3(rows.n_rows), dim3(kSelThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace clsa
