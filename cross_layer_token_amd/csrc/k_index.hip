// Routing scores I_t[j] = q_idx,t . K_idx[j] - the first half of the routing equation on the
// picx.dev summary of "You Only Index Once" (Methodology > Architecture Overview, eq. 2).
//
// Decode: a bandwidth-bound GEMV that streams every K_idx row exactly once.  Workgroups own
// equal slices of the packed token axis (so ragged batches are balanced by tokens, not by
// sequences); a slice that crosses a sequence boundary is processed per sequence segment.
// Each 16-byte K_idx chunk meets the query chunk in v_dot2 (bf16 x bf16 -> fp32), and the
// per-lane partial sums of 16 rows are reduce-scattered over the row's lanes with DPP, so that
// every lane ends up owning one finished row score.
//
// Prefill: the causal product Q_idx K_idx^T on the matrix cores (bf16 MFMA 16x16x32, fp32
// accumulate), skipping tiles above the diagonal.
#include "device_common.h"

namespace clsa {

namespace {

__device__ __forceinline__ float dot8(const uint4& k, const uint4& q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x), __builtin_bit_cast(bf16x2_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y), __builtin_bit_cast(bf16x2_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z), __builtin_bit_cast(bf16x2_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w), __builtin_bit_cast(bf16x2_t, q.w), acc, false);
  return acc;
}

// One reduce-scatter step over the lane bit M: of the 2H partial sums a lane holds, keep the
// half selected by its own bit M and add the partner's copy of that half.
template <int M, int H>
__device__ __forceinline__ void rs_step(float* p, int sub) {
  const bool upper = (sub & M) != 0;
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const float lo = p[j], hi = p[j + H];
    const float send = upper ? lo : hi;
    const float keep = upper ? hi : lo;
    p[j] = keep + dpp_partner<M>(send);
  }
}

constexpr int kIdxThreads = 256;

template <int D>
__global__ __launch_bounds__(kIdxThreads) void k_index_scores_decode(const uint16_t* __restrict__ q_idx,
                                                                       const uint16_t* __restrict__ k_idx,
                                                                       const int32_t* __restrict__ cu, int batch,
                                                                       int64_t total_tokens, int max_row_len,
                                                                       float* __restrict__ scores, int64_t ld,
                                                                       int chunk) {
  constexpr int LPR = D / 8;   // lanes per K_idx row (16 bytes each)
  constexpr int NG = 64 / LPR; // row groups per wave
  constexpr int NR = LPR;      // rows per lane per iteration: one finished row per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = lane / LPR, sub = lane % LPR;
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int64_t t1 = t0 + chunk < total_tokens ? t0 + chunk : total_tokens;
  if (t0 >= t1) return;
  // sequence holding t0: the largest b < batch with cu[b] <= t0
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t0) lo = mid; else hi = mid - 1;
  }
  int b = lo;
  int64_t t = t0;
  while (t < t1) {
    while (b < batch - 1 && (int64_t)cu[b + 1] <= t) ++b;
    const int64_t seq_end = (int64_t)cu[b + 1];
    const int64_t seg_end = seq_end < t1 ? seq_end : t1;
    if (seg_end <= t) break;  // inconsistent cu_seqlens: nothing valid left in this slice
    const int64_t base = cu[b];
    const uint4 qv = *reinterpret_cast<const uint4*>(q_idx + (size_t)b * D + sub * 8);
    float* srow = scores + (int64_t)b * ld;
    for (int64_t it = t + wave * 64; it < seg_end; it += (kIdxThreads / 64) * 64) {
      uint4 kv[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int64_t row = it + i * NG + lg;
        kv[i] = row < seg_end ? load_stream16(k_idx + row * D + sub * 8)
                              : make_uint4(0u, 0u, 0u, 0u);
      }
      float p[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) p[i] = dot8(kv[i], qv, 0.f);
      if constexpr (LPR == 16) {
        rs_step<8, 8>(p, sub);
        rs_step<4, 4>(p, sub);
        rs_step<2, 2>(p, sub);
        rs_step<1, 1>(p, sub);
      } else {
        rs_step<4, 4>(p, sub);
        rs_step<2, 2>(p, sub);
        rs_step<1, 1>(p, sub);
      }
      const int64_t row = it + sub * NG + lg;
      if (row < seg_end) {
        const int64_t local = row - base;
        if (local < max_row_len) srow[local] = p[0];
      }
    }
    t = seg_end;
  }
}

// Prefill: rows i (query positions pos0 + i of sequence `seq`), columns j (tokens of the same
// sequence); only j <= pos0 + i is computed and written.  64 x 64 tile per workgroup, each wave
// 16 rows x 64 columns.
template <int D>
__global__ __launch_bounds__(256) void k_index_scores_prefill(const uint16_t* __restrict__ q_idx,
                                                               const uint16_t* __restrict__ k_idx,
                                                               const int32_t* __restrict__ cu, int seq, int pos0,
                                                               int n_rows, float* __restrict__ scores, int64_t ld) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int last_row = (r0 + 63 < n_rows - 1) ? r0 + 63 : n_rows - 1;
  if (c0 > pos0 + last_row) return;  // tile entirely above the causal diagonal
  const int64_t base = cu[seq];
  const int wr0 = r0 + wave * 16;
  if (wr0 >= n_rows) return;
  const int l16 = lane & 15, grp = lane >> 4;
  bf16x8_t a[KS];
  {
    const int row = wr0 + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < n_rows) v = *reinterpret_cast<const uint4*>(q_idx + (int64_t)row * D + ks * 32 + grp * 8);
      a[ks] = bitcast<bf16x8_t>(v);
    }
  }
  const int ncols = pos0 + n_rows;  // tokens any row of this call may see
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int col = c0 + nt * 16 + l16;
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (col < ncols) v = *reinterpret_cast<const uint4*>(k_idx + (base + col) * D + ks * 32 + grp * 8);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bitcast<bf16x8_t>(v), acc, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wr0 + grp * 4 + j;
      if (row < n_rows && col <= pos0 + row) scores[(int64_t)row * ld + col] = acc[j];
    }
  }
}

}  // namespace

int launch_index_scores_decode(const RowsDev& rows, int d_idx, int64_t total_tokens, const uint16_t* q_idx,
                               const uint16_t* k_idx, float* scores, int64_t ld, void* stream) {
  const int chunk = 4096;
  const int64_t nblk = (total_tokens + chunk - 1) / chunk;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d_idx == 128)
    hipLaunchKernelGGL(k_index_scores_decode<128>, dim3((unsigned)nblk), dim3(kIdxThreads), 0, s, q_idx, k_idx,
                       rows.cu, rows.n_rows, total_tokens, rows.max_row_len, scores, ld, chunk);
  else
    hipLaunchKernelGGL(k_index_scores_decode<64>, dim3((unsigned)nblk), dim3(kIdxThreads), 0, s, q_idx, k_idx,
                       rows.cu, rows.n_rows, total_tokens, rows.max_row_len, scores, ld, chunk);
  return (int)hipGetLastError();
}

int launch_index_scores_prefill(const RowsDev& rows, int d_idx, const uint16_t* q_idx, const uint16_t* k_idx,
                                float* scores, int64_t ld, void* stream) {
  const int ncols = rows.pos0 + rows.n_rows;
  dim3 grid((ncols + 63) / 64, (rows.n_rows + 63) / 64);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d_idx == 128)
    hipLaunchKernelGGL(k_index_scores_prefill<128>, grid, dim3(256), 0, s, q_idx, k_idx, rows.cu, rows.seq,
                       rows.pos0, rows.n_rows, scores, ld);
  else
    hipLaunchKernelGGL(k_index_scores_prefill<64>, grid, dim3(256), 0, s, q_idx, k_idx, rows.cu, rows.seq,
                       rows.pos0, rows.n_rows, scores, ld);
  return (int)hipGetLastError();
}

const char* device_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace clsa
