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
// Long rows: many workgroups per row.  Pass 1 builds a per-row histogram of the top 12 key
// bits; the last workgroup of a row (atomic ticket) finds the bin holding T.  Pass 2 appends
// the tokens above that bin ("sure") and inside it ("candidates") to per-row lists; the last
// workgroup of the row refines T and the index cut-off among the candidates and writes the
// ascending index list through an LDS bitmap.
#include "device_common.h"

namespace clsa {

namespace {

constexpr int kRowThreads = 512;
constexpr int kPassThreads = 256;
constexpr int kBitmapWords = 4096;  // 2^17 tokens per bitmap segment

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
// Per-row state words (uint32): 0 done1, 1 done2, 2 nsure, 3 ncand, 4 t1, 5 above1, 6 need1
struct LongRowsArgs {
  RowsDev rw;
  const float* scores;
  int64_t ld;
  int k;
  int32_t* out;
  int32_t* count;
  uint32_t* hist1;  // [R, kHist1Bins]
  uint32_t* state;  // [R, kTopkStateWords]
  int32_t* sure;    // [R, k]
  uint2* cand;      // [R, max_row_len] (key, index)
};

__global__ void k_topk_clear(uint32_t* __restrict__ hist1, uint32_t* __restrict__ state, int n_rows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)n_rows * kHist1Bins) hist1[i] = 0;
  if (i < (int64_t)n_rows * kTopkStateWords) state[i] = 0;
}

__device__ __forceinline__ bool last_block_of_row(uint32_t* ticket, int nchunks, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) flag[0] = atomicAdd(ticket, 1u) == (uint32_t)(nchunks - 1);
  __syncthreads();
  const bool last = flag[0] != 0;
  if (last) __threadfence();
  return last;
}

__global__ __launch_bounds__(kPassThreads) void k_topk_hist(LongRowsArgs a) {
  __shared__ uint32_t hist[kHist1Bins];
  __shared__ int scan[kPassThreads / 64 + 1];
  __shared__ int res[2];
  __shared__ int flag[1];
  const int r = blockIdx.y;
  const int n = row_len(a.rw, r);
  const int m = n < a.k ? n : a.k;
  const int c0 = blockIdx.x * kTopkChunk;
  if (c0 >= n) return;
  if (m == n) {  // every visible token is selected: identity list, no histogram needed
    const int c1 = c0 + kTopkChunk < n ? c0 + kTopkChunk : n;
    for (int i = c0 + threadIdx.x; i < c1; i += blockDim.x) a.out[(int64_t)r * a.k + i] = i;
    if (blockIdx.x == 0) {
      for (int i = n + threadIdx.x; i < a.k; i += blockDim.x) a.out[(int64_t)r * a.k + i] = -1;
      if (threadIdx.x == 0) a.count[r] = n;
    }
    return;
  }
  for (int i = threadIdx.x; i < kHist1Bins; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const float* srow = a.scores + (int64_t)r * a.ld;
  const int c1 = c0 + kTopkChunk < n ? c0 + kTopkChunk : n;
  for (int i = c0 + threadIdx.x; i < c1; i += blockDim.x) atomicAdd(&hist[score_key(srow[i]) >> 20], 1u);
  __syncthreads();
  uint32_t* g = a.hist1 + (int64_t)r * kHist1Bins;
  for (int i = threadIdx.x; i < kHist1Bins; i += blockDim.x)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
  const int nchunks = (n + kTopkChunk - 1) / kTopkChunk;
  uint32_t* st = a.state + (int64_t)r * kTopkStateWords;
  if (!last_block_of_row(&st[0], nchunks, flag)) return;
  for (int i = threadIdx.x; i < kHist1Bins; i += blockDim.x) hist[i] = __hip_atomic_load(&g[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  find_bin_from_top(hist, kHist1Bins, m, scan, res);
  if (threadIdx.x == 0) {
    st[4] = (uint32_t)res[0];
    st[5] = (uint32_t)res[1];
    st[6] = (uint32_t)(m - res[1]);
  }
}

__global__ __launch_bounds__(kPassThreads) void k_topk_collect(LongRowsArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t bitmap[kBitmapWords];
  __shared__ int scan[kPassThreads / 64 + 1];
  __shared__ int res[2];
  __shared__ int flag[1];
  const int r = blockIdx.y;
  const int n = row_len(a.rw, r);
  const int m = n < a.k ? n : a.k;
  const int c0 = blockIdx.x * kTopkChunk;
  if (c0 >= n || m == n) return;
  uint32_t* st = a.state + (int64_t)r * kTopkStateWords;
  const uint32_t t1 = st[4];
  const float* srow = a.scores + (int64_t)r * a.ld;
  int32_t* sure = a.sure + (int64_t)r * a.k;
  uint2* cand = a.cand + (int64_t)r * a.rw.max_row_len;
  const int c1 = c0 + kTopkChunk < n ? c0 + kTopkChunk : n;
  const int lane = threadIdx.x & 63;
  for (int base = c0; base < c1; base += blockDim.x) {
    const int i = base + threadIdx.x;
    uint32_t key = 0, bin = 0;
    const bool valid = i < c1;
    if (valid) {
      key = score_key(srow[i]);
      bin = key >> 20;
    }
    const bool is_sure = valid && bin > t1;
    const bool is_cand = valid && bin == t1;
    // wave-aggregated appends
    const uint64_t ms = __ballot(is_sure);
    const uint64_t mc = __ballot(is_cand);
    uint32_t ps = 0, pc = 0;
    if (lane == 0) {
      if (ms) ps = atomicAdd(&st[2], (uint32_t)__popcll(ms));
      if (mc) pc = atomicAdd(&st[3], (uint32_t)__popcll(mc));
    }
    ps = __shfl(ps, 0, 64);
    pc = __shfl(pc, 0, 64);
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    if (is_sure) sure[ps + __popcll(ms & below)] = i;
    if (is_cand) cand[pc + __popcll(mc & below)] = make_uint2(key, (uint32_t)i);
  }
  const int nchunks = (n + kTopkChunk - 1) / kTopkChunk;
  if (!last_block_of_row(&st[1], nchunks, flag)) return;

  // ---- last workgroup of the row: refine the threshold among the candidates -------------------
  const int nsure = (int)__hip_atomic_load(&st[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int ncand = (int)__hip_atomic_load(&st[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int need = (int)st[6];
  uint32_t prefix = t1 << 20, pmask = 0xFFF00000u;
  const int shifts[2] = {9, 0};
  const int widths[2] = {11, 9};
  int eq_count = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int nb = 1 << widths[pass];
    const int sh = shifts[pass];
    for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < ncand; i += blockDim.x) {
      const uint32_t key = __builtin_nontemporal_load(&cand[i].x);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin_from_top(hist, nb, need, scan, res);
    prefix |= (uint32_t)res[0] << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    need -= res[1];
    if (pass == 1) eq_count = (int)hist[res[0]];
    __syncthreads();
  }
  const uint32_t T = prefix;
  // index cut-off among the keys equal to T: the need-th smallest index
  uint32_t jstar = 0xFFFFFFFFu;
  if (need < eq_count) {
    uint32_t ip = 0, im = 0;
    int need_i = need;
    const int ishift[3] = {20, 10, 0};
    const int iwidth[3] = {11, 10, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int nb = 1 << iwidth[pass];
      const int sh = ishift[pass];
      for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < ncand; i += blockDim.x) {
        const uint2 c = cand[i];
        if (c.x == T && (c.y & im) == ip) atomicAdd(&hist[(c.y >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      find_bin_from_bottom(hist, nb, need_i, scan, res);
      ip |= (uint32_t)res[0] << sh;
      im |= (uint32_t)(nb - 1) << sh;
      need_i -= res[1];
      __syncthreads();
    }
    jstar = ip;
  }
  // ---- ascending output through an LDS bitmap, one 2^17-token segment at a time --------------
  int32_t* orow = a.out + (int64_t)r * a.k;
  int written = 0;
  const int seg_bits = kBitmapWords * 32;
  for (int s0 = 0; s0 < n; s0 += seg_bits) {
    for (int i = threadIdx.x; i < kBitmapWords; i += blockDim.x) bitmap[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nsure; i += blockDim.x) {
      const int j = sure[i] - s0;
      if (j >= 0 && j < seg_bits) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
    for (int i = threadIdx.x; i < ncand; i += blockDim.x) {
      const uint2 c = cand[i];
      const bool take = c.x > T || (c.x == T && c.y <= jstar);
      const int j = (int)c.y - s0;
      if (take && j >= 0 && j < seg_bits) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    constexpr int WPT = kBitmapWords / kPassThreads;  // words per thread
    int local = 0;
    for (int w = 0; w < WPT; ++w) local += __popc(bitmap[threadIdx.x * WPT + w]);
    int tot;
    int pos = written + block_exclusive_scan(local, scan, &tot);
    for (int w = 0; w < WPT; ++w) {
      uint32_t bits = bitmap[threadIdx.x * WPT + w];
      const int tok0 = s0 + (threadIdx.x * WPT + w) * 32;
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < a.k) orow[pos] = tok0 + b;
        ++pos;
      }
    }
    written += tot;
    __syncthreads();
  }
  for (int i = m + threadIdx.x; i < a.k; i += blockDim.x) orow[i] = -1;
  if (threadIdx.x == 0) a.count[r] = m;
}

}  // namespace

int launch_topk(const RowsDev& rows, int k, const TopkPlan& plan, const float* scores, int64_t ld, int32_t* idx,
                int32_t* count, void* ws, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!plan.multi_wg) {
    hipLaunchKernelGGL(k_topk_rows_lds, dim3(rows.n_rows), dim3(kRowThreads), 0, s, rows, scores, ld, k, idx, count);
    return (int)hipGetLastError();
  }
  char* w = static_cast<char*>(ws);
  LongRowsArgs a;
  a.rw = rows;
  a.scores = scores;
  a.ld = ld;
  a.k = k;
  a.out = idx;
  a.count = count;
  a.hist1 = reinterpret_cast<uint32_t*>(w + plan.hist_off);
  a.state = reinterpret_cast<uint32_t*>(w + plan.state_off);
  a.sure = reinterpret_cast<int32_t*>(w + plan.sure_off);
  a.cand = reinterpret_cast<uint2*>(w + plan.cand_off);
  const int64_t nclear = (int64_t)rows.n_rows * kHist1Bins;
  hipLaunchKernelGGL(k_topk_clear, dim3((unsigned)((nclear + 255) / 256)), dim3(256), 0, s, a.hist1, a.state,
                     rows.n_rows);
  const dim3 grid((rows.max_row_len + kTopkChunk - 1) / kTopkChunk, rows.n_rows);
  hipLaunchKernelGGL(k_topk_hist, grid, dim3(kPassThreads), 0, s, a);
  hipLaunchKernelGGL(k_topk_collect, grid, dim3(kPassThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace clsa
