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
// Long rows: a first-level histogram of the top key bits comes in per-chunk partials (written
// by the score kernel, or by k_topk_hist_partials); each select workgroup sums them, finds the
// bin holding T, and compacts its span's scores at or above that bin in index order; the last
// workgroup of the row (one atomic ticket per workgroup, nothing contended) finishes the
// selection over that short list.  No workgroup ever waits for another.
#include "device_common.h"

namespace clsa {

namespace {

constexpr int kRowThreads = 512;
constexpr int kPassThreads = 256;

// Find the bin d (scanning from the top bin down) whose cumulative count from the top first
// reaches `need`; returns d and sets *above = count of bins above d.  hist has nb bins in LDS;
// one thread finds it and publishes via res[0..1].  Contains __syncthreads().
__device__ void find_bin_from_top(const uint32_t* hist, int nb, int need, int* scan_scratch, int* res) {
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int u0 = threadIdx.x * per;
  int local = 0;
  for (int j = 0; j < per; ++j) {
    const int u = u0 + j;
    if (u < nb) local += (int)hist[nb - 1 - u];
  }
  int total;
  int run = block_exclusive_scan(local, scan_scratch, &total);
  for (int j = 0; j < per; ++j) {
    const int u = u0 + j;
    if (u < nb) {
      const int h = (int)hist[nb - 1 - u];
      if (run < need && run + h >= need) {
        res[0] = nb - 1 - u;
        res[1] = run;
      }
      run += h;
    }
  }
  __syncthreads();
}

// Find the bin d (scanning from the bottom bin up) whose cumulative count first reaches need;
// returns via res[0] = d, res[1] = count below d.
__device__ void find_bin_from_bottom(const uint32_t* hist, int nb, int need, int* scan_scratch, int* res) {
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int u0 = threadIdx.x * per;
  int local = 0;
  for (int j = 0; j < per; ++j)
    if (u0 + j < nb) local += (int)hist[u0 + j];
  int total;
  int run = block_exclusive_scan(local, scan_scratch, &total);
  for (int j = 0; j < per; ++j) {
    const int u = u0 + j;
    if (u < nb) {
      const int h = (int)hist[u];
      if (run < need && run + h >= need) {
        res[0] = u;
        res[1] = run;
      }
      run += h;
    }
  }
  __syncthreads();
}

__device__ void write_all(int32_t* out, int32_t* count, int r, int n, int k) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) out[(int64_t)r * k + i] = i < n ? i : -1;
  if (threadIdx.x == 0) count[r] = n;
}

// ---------------------------------------------------------------------------- short rows
__global__ __launch_bounds__(kRowThreads) void k_topk_rows_lds(RowsDev rw, const float* __restrict__ scores,
                                                                 int64_t ld, int k, int32_t* __restrict__ out,
                                                                 int32_t* __restrict__ count) {
  __shared__ uint32_t keys[kLdsRowCap];
  __shared__ uint32_t hist[2048];
  __shared__ int scan[kRowThreads / 64 + 1];
  __shared__ int res[2];
  const int r = blockIdx.x;
  const int n = row_len(rw, r);
  const int m = n < k ? n : k;
  if (m == n) {
    write_all(out, count, r, n, k);
    return;
  }
  const float* srow = scores + (int64_t)r * ld;
  for (int i = threadIdx.x; i < n; i += blockDim.x) keys[i] = score_key(srow[i]);
  uint32_t prefix = 0, pmask = 0;
  int need = m;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int nb = 1 << widths[pass];
    const int sh = shifts[pass];
    for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t key = keys[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin_from_top(hist, nb, need, scan, res);
    prefix |= (uint32_t)res[0] << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    need -= res[1];
    __syncthreads();
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
  int tot;
  int gt_before = block_exclusive_scan(gt, scan, &tot);
  int eq_before = block_exclusive_scan(eq, scan, &tot);
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
  uint16_t* hpart;        // [R, hist_chunks, kTopkBins] per-chunk histograms of key >> (32 - kTopkBinBits)
  int hist_chunks;
  uint32_t* ticket;       // [R], zero on entry
  uint32_t* cnt;          // [R, spans]
  int spans;
  uint2* slot;            // [R, max_row_len]
  uint2* list;            // [R, max_row_len]
};

constexpr int kSelThreads = 1024;
constexpr int kHistThreads = 256;

// Histogram partials of the scores (used when no score kernel produced them); clears the tickets.
__global__ __launch_bounds__(kHistThreads) void k_topk_hist_partials(SelectArgs a) {
  __shared__ uint32_t hist[kTopkBins];
  const int r = blockIdx.y, c = blockIdx.x;
  if (r == 0 && c == 0)
    for (int i = threadIdx.x; i < a.rw.n_rows; i += blockDim.x) a.ticket[i] = 0u;
  const int n = row_len(a.rw, r);
  const int t0 = c * kIdxChunk;
  if (t0 >= n || (n <= a.k)) return;
  const int t1 = t0 + kIdxChunk < n ? t0 + kIdxChunk : n;
  for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  const float* srow = a.scores + (int64_t)r * a.ld;
  constexpr int PER = kIdxChunk / kHistThreads;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = t0 + threadIdx.x + j * kHistThreads;
    v[j] = i < t1 ? srow[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (t0 + (int)threadIdx.x + j * kHistThreads < t1) atomicAdd(&hist[score_key(v[j]) >> (32 - kTopkBinBits)], 1u);
  __syncthreads();
  uint16_t* hp = a.hpart + ((int64_t)r * a.hist_chunks + c) * kTopkBins;
  for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) hp[i] = (uint16_t)hist[i];
}

// Long-row select.  Workgroup (span, row) handles scores [span * kSelectSpan, +kSelectSpan).
//  1. Sum the row's histogram partials; find the bin t1 holding the m-th largest key.
//  2. Append (key, index) of every score whose bin is >= t1 to the span's slot, in index order.
//  3. The last workgroup of the row (ticket) concatenates the span lists (still in index order),
//     refines the exact m-th largest key T over the remaining key bits, and writes the output:
//     keys above T, then the lowest-index ties at T up to m, in list (= index) order.
constexpr int kListLds = 5120;   // (key, index) pairs the last workgroup keeps in LDS
constexpr int kCopyBatch = 6;    // list loads each thread keeps in flight

__global__ __launch_bounds__(kSelThreads) void k_topk_select(SelectArgs a) {
  __shared__ uint32_t hist[kTopkBins];
  __shared__ int scan[kSelThreads / 64 + 1];
  __shared__ int res[2];
  __shared__ int flag[1];
  __shared__ int span_pre[kSelThreads + 1];
  __shared__ uint2 list_lds[kListLds];
  const int r = blockIdx.y, sp = blockIdx.x;
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
  // 1. row histogram from the partials (thread t owns bins 2t, 2t+1), 32 partials per round
  {
    const int nch = (n + kIdxChunk - 1) / kIdxChunk;
    const uint32_t* hp = reinterpret_cast<const uint32_t*>(a.hpart + (int64_t)r * a.hist_chunks * kTopkBins);
    uint32_t lo = 0, hi = 0;
    for (int c = 0; c < nch; c += 32) {
      uint32_t w[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) w[j] = c + j < nch ? hp[(int64_t)(c + j) * (kTopkBins / 2) + threadIdx.x] : 0u;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        lo += w[j] & 0xFFFFu;
        hi += w[j] >> 16;
      }
    }
    hist[2 * threadIdx.x] = lo;
    hist[2 * threadIdx.x + 1] = hi;
  }
  __syncthreads();
  find_bin_from_top(hist, kTopkBins, m, scan, res);
  const uint32_t t1 = (uint32_t)res[0];
  const int above1 = res[1];
  // 2. ordered compaction of the span's scores with bin >= t1
  const float* srow = a.scores + (int64_t)r * a.ld;
  uint2* slot = a.slot + (int64_t)r * a.rw.max_row_len + s0;
  constexpr int ROUND = kSelThreads * 4;
  constexpr int ROUNDS = kSelectSpan / ROUND;
  float4 v[ROUNDS];
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    const int i = s0 + q * ROUND + threadIdx.x * 4;
    v[q] = i + 3 < s1 ? *reinterpret_cast<const float4*>(srow + i)
                      : make_float4(i < s1 ? srow[i] : 0.f, i + 1 < s1 ? srow[i + 1] : 0.f,
                                    i + 2 < s1 ? srow[i + 2] : 0.f, 0.f);
  }
  int written = 0;
#pragma unroll
  for (int q = 0; q < ROUNDS; ++q) {
    const int i = s0 + q * ROUND + threadIdx.x * 4;
    const float x[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
    uint32_t key[4];
    bool f[4];
    int c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      key[j] = score_key(x[j]);
      f[j] = (i + j < s1) && (key[j] >> (32 - kTopkBinBits)) >= t1;
      c += f[j];
    }
    int tot;
    int pos = written + block_exclusive_scan(c, scan, &tot);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (f[j]) st_dev(reinterpret_cast<uint64_t*>(slot + pos++), ((uint64_t)(uint32_t)(i + j) << 32) | key[j]);
    written += tot;
  }
  if (threadIdx.x == 0) st_dev(&a.cnt[(int64_t)r * a.spans + sp], (uint32_t)written);
  // 3. the last workgroup of the row finishes the selection
  const int nsp = (n + kSelectSpan - 1) / kSelectSpan;
  if (!arrive_last(&a.ticket[r], (uint32_t)nsp, flag)) return;
  // concatenate the span lists (spans in order, so the list stays in index order); the list
  // lives in LDS when it fits, else in the workspace
  int L = 0;
  {
    const int mine = threadIdx.x < nsp ? (int)ld_dev(&a.cnt[(int64_t)r * a.spans + threadIdx.x]) : 0;
    const int pre = block_exclusive_scan(mine, scan, &L);
    if (threadIdx.x < nsp) span_pre[threadIdx.x] = pre;
    if (threadIdx.x == 0) span_pre[nsp] = L;
    __syncthreads();
  }
  uint2* list = L <= kListLds ? list_lds : a.list + (int64_t)r * a.rw.max_row_len;
  {
    const uint2* rslot = a.slot + (int64_t)r * a.rw.max_row_len;
    for (int p0 = 0; p0 < L; p0 += kSelThreads * kCopyBatch) {
      uint64_t v[kCopyBatch];
      int at[kCopyBatch];
#pragma unroll
      for (int j = 0; j < kCopyBatch; ++j) {
        const int p = p0 + j * kSelThreads + threadIdx.x;
        at[j] = p;
        v[j] = 0;
        if (p < L) {
          int lo = 0, hi = nsp - 1;  // span holding list position p
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (span_pre[mid] <= p) lo = mid; else hi = mid - 1;
          }
          v[j] = ld_dev(reinterpret_cast<const uint64_t*>(rslot + (int64_t)lo * kSelectSpan + (p - span_pre[lo])));
        }
      }
#pragma unroll
      for (int j = 0; j < kCopyBatch; ++j)
        if (at[j] < L) list[at[j]] = make_uint2((uint32_t)v[j], (uint32_t)(v[j] >> 32));
    }
    __syncthreads();
  }
  // refine T below the first level: bits [20:10], then [9:0]
  int need = m - above1;
  uint32_t prefix = t1 << (32 - kTopkBinBits), pmask = ~0u << (32 - kTopkBinBits);
  const int shifts[2] = {10, 0};
  const int widths[2] = {32 - kTopkBinBits - 10, 10};
  for (int pass = 0; pass < 2; ++pass) {
    const int nb = 1 << widths[pass];
    const int sh = shifts[pass];
    for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < L; i += blockDim.x) {
      const uint32_t key = list[i].x;
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin_from_top(hist, nb, need, scan, res);
    prefix |= (uint32_t)res[0] << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    need -= res[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  // ordered output over contiguous per-thread ranges of the list
  const int E = (L + blockDim.x - 1) / blockDim.x;
  const int p0 = threadIdx.x * E;
  int gt = 0, eq = 0;
  for (int j = 0; j < E; ++j) {
    const int p = p0 + j;
    if (p < L) {
      const uint32_t key = list[p].x;
      gt += key > T;
      eq += key == T;
    }
  }
  int tot;
  int gt_before = block_exclusive_scan(gt, scan, &tot);
  int eq_before = block_exclusive_scan(eq, scan, &tot);
  for (int j = 0; j < E; ++j) {
    const int p = p0 + j;
    if (p < L) {
      const uint2 e = list[p];
      const bool take = e.x > T || (e.x == T && eq_before < need);
      if (take) orow[gt_before + (eq_before < need ? eq_before : need)] = (int32_t)e.y;
      gt_before += e.x > T;
      eq_before += e.x == T;
    }
  }
  for (int i = m + threadIdx.x; i < a.k; i += blockDim.x) orow[i] = -1;
  if (threadIdx.x == 0) a.count[r] = m;
}

}  // namespace

int launch_topk(const RowsDev& rows, int k, const TopkPlan& plan, const float* scores, int64_t ld, int32_t* idx,
                int32_t* count, void* ws, uint32_t* tickets, bool have_hist, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!plan.multi_wg) {
    hipLaunchKernelGGL(k_topk_rows_lds, dim3(rows.n_rows), dim3(kRowThreads), 0, s, rows, scores, ld, k, idx, count);
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
  a.hist_chunks = plan.hist_chunks;
  a.ticket = tickets;
  a.cnt = reinterpret_cast<uint32_t*>(w + plan.cnt_off);
  a.spans = plan.spans;
  a.slot = reinterpret_cast<uint2*>(w + plan.slot_off);
  a.list = reinterpret_cast<uint2*>(w + plan.list_off);
  if (!have_hist)
    hipLaunchKernelGGL(k_topk_hist_partials, dim3(plan.hist_chunks, rows.n_rows), dim3(kHistThreads), 0, s, a);
  hipLaunchKernelGGL(k_topk_select, dim3(plan.spans, rows.n_rows), dim3(kSelThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace clsa
