// Routing scores I_t[j] = q_idx,t . K_idx[j] - the first half of the routing equation on the
// picx.dev summary of "You Only Index Once" (Methodology > Architecture Overview, eq. 2).
//
// Decode: a bandwidth-bound GEMV that streams every K_idx row exactly once.  A workgroup owns
// one equal segment of all the sequences' tokens.  Each 16-byte K_idx chunk meets the query
// chunk in v_dot2 (bf16 x bf16 -> fp32), and the per-lane partial sums of 16 rows are
// reduce-scattered over the row's lanes with DPP, so that every lane ends up owning one finished
// row score.  When asked, the
// workgroup also histograms the top key bits of its scores (the first level of the top-k
// select) and publishes the part of the histogram the select needs (write_hist_partial), which
// saves the select a pass over the scores.
//
// Prefill: the causal product Q_idx K_idx^T on the matrix cores (bf16 MFMA 16x16x32, fp32
// accumulate) over the causal tiles only, each K_idx tile staged once in LDS.
#include "select_common.h"

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

// One workgroup = one segment of `seg` tokens of the sequences concatenated as they lie in the
// cache (K_idx rows cu[b] .. cu[b + 1] - 1 belong to sequence b), so every workgroup streams the
// same share of K_idx whatever the mix of sequence lengths.  It walks the pieces of the sequences
// its segment overlaps, in order; each piece is scored with its sequence's query.  Each wave takes
// 64 rows per iteration (16 per lane, one 16-byte piece of each) and requests the next
// iteration's rows before reducing the current ones, so every wave keeps a full set of loads in
// flight.  Besides the scores it can write, for every piece of a sequence longer than topk, the
// histogram of the top kTopkBinBits key bits (for the top-k select), at slot
// segment - floor(cu[b] / seg) of the sequence's partials, and clear the select's per-row tickets
// (consumed by later kernels on the same stream).  Every K_idx row read lies inside the segment,
// so the reads stay inside [0, total) whatever cu holds.
template <int D>
__global__ __launch_bounds__(kIdxThreads) void k_index_scores_decode(const uint16_t* __restrict__ q_idx,
                                                                       int64_t q_stride,
                                                                       const uint16_t* __restrict__ k_idx,
                                                                       const int32_t* __restrict__ cu, int n_rows,
                                                                       int max_row_len, int seg, int64_t total,
                                                                       float* __restrict__ scores, int64_t ld,
                                                                       uint16_t* __restrict__ hpart,
                                                                       uint32_t* __restrict__ hinfo, int topk,
                                                                       int hpart_chunks, uint32_t* __restrict__ clear,
                                                                       int n_clear) {
  constexpr int LPR = D / 8;   // lanes per K_idx row (16 bytes each)
  constexpr int NG = 64 / LPR; // row groups per wave
  constexpr int NR = LPR;      // rows per lane per iteration: one finished row per lane
  constexpr int STEP = (kIdxThreads / 64) * 64;
  __shared__ uint32_t hist[kTopkBins];
  __shared__ int scan[2 * kIdxThreads / 64];
  __shared__ int res[4];
  __shared__ int first_row, first_lo, first_hi;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = lane / LPR, sub = lane % LPR;
  const int w = blockIdx.x;
  if (clear != nullptr && w == 0)
    for (int i = threadIdx.x; i < n_clear; i += blockDim.x) clear[i] = 0u;
  // token offsets fit in 32 bits (cu_seqlens is int32): g0 = w * seg <= total - 1
  const int g0 = w * seg;
  const int g1 = (int)(total - g0 < seg ? total : g0 + seg);
  // The first piece starts at g0, and K_idx rows are addressed by token alone: that piece's first
  // iteration is requested before the search below (rows past the piece but inside the segment
  // are read and not stored).
  uint4 kv[NR];
  {
    const uint16_t* kseg = k_idx + sub * 8;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int row = g0 + wave * 64 + i * NG + lg;
      kv[i] = row < g1 ? load_stream16(kseg + (int64_t)row * D) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  bool prefetched = true;
  // the sequence holding token g0 (cu[b] <= g0 < cu[b + 1]); none found: nothing to do
  if (threadIdx.x == 0) first_row = n_rows;
  __syncthreads();
  for (int j = threadIdx.x; j < n_rows; j += blockDim.x) {
    const int c0 = cu[j], c1 = cu[j + 1];
    if (c0 <= g0 && g0 < c1) {
      first_row = j;
      first_lo = c0;
      first_hi = c1;
    }
  }
  __syncthreads();
  // the first sequence's bounds come from the search; each later one starts where the previous
  // one ends, so only its end is loaded
  int c0 = first_lo, c1 = first_hi;
  for (int b = first_row; b < n_rows; ++b) {
    if (b != first_row) {
      c0 = c1;
      c1 = cu[b + 1];
    }
    if (c0 >= g1) break;
    int n = c1 - c0;
    n = n < 0 ? 0 : (n > max_row_len ? max_row_len : n);
    const int lo = g0 > c0 ? g0 : c0;
    const int64_t e = (int64_t)c0 + n;
    const int hi = (int)(e < g1 ? e : g1);
    if (lo >= hi) continue;
    const int t0 = lo - c0, t1 = hi - c0;  // the piece, in the sequence's own positions
    const int slot = w - c0 / seg;
    const int64_t rs = c0;
    const bool do_hist = hpart != nullptr && n > topk && slot >= 0 && slot < hpart_chunks;
    if (do_hist) {
      for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) hist[i] = 0u;
      __syncthreads();
    }
    const uint16_t* kbase = k_idx + rs * D + sub * 8;
    const uint4 qv = *reinterpret_cast<const uint4*>(q_idx + (int64_t)b * q_stride + sub * 8);
    float* srow = scores + (int64_t)b * ld;
    auto load = [&](int it) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int row = it + i * NG + lg;
        kv[i] = row < t1 ? load_stream16(kbase + (int64_t)row * D) : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    int it = t0 + wave * 64;
    if (!(prefetched && lo == g0) && it < t1) load(it);  // else kv holds this iteration's rows already
    prefetched = false;
    for (; it < t1; it += STEP) {
      float p[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) p[i] = dot8(kv[i], qv, 0.f);
      if (it + STEP < t1) load(it + STEP);
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
      const int row = it + sub * NG + lg;
      if (row < t1) {
        srow[row] = p[0];
        if (do_hist) atomicAdd(&hist[score_key(p[0]) >> (32 - kTopkBinBits)], 1u);
      }
    }
    if (do_hist) {
      __syncthreads();
      // bins 2i and 2i + 1 as the low and high halves of one word (counts <= seg <= 65535)
      uint32_t* hp = reinterpret_cast<uint32_t*>(hpart + ((int64_t)b * hpart_chunks + slot) * kTopkBins);
      write_hist_partial<kIdxThreads>(hist, t1 - t0, topk, hp, hinfo + (int64_t)b * hpart_chunks + slot, scan, res);
      __syncthreads();  // hist is read by the partial's write before the next piece clears it
    }
  }
}

// Prefill: the causal product Q_idx K_idx^T.  Rows i are the query positions pos0 + i of sequence
// `seq`, columns j the tokens of that sequence; only j <= pos0 + i is written.  The grid enumerates
// only the 128 x 128 tiles (128 rows of the call x 128 token columns) that hold a visible entry:
// row block rb (rows 128 rb ..) has column blocks 0 .. (pos0 + its last row) / 128, that is c0 + rb
// of them for every block but the last (c0 = ceil(pos0 / 128) + 1), so tile t lies in the row
// block whose prefix P(rb) = rb c0 + rb (rb - 1) / 2 is the largest at or below t.
// The workgroup stages its 128 K_idx rows once in LDS (16-byte chunks XOR-swizzled by the row, so
// the fragment reads of 16 rows x 4 chunks hit 64 distinct banks) and each of its four waves takes
// a quarter of the query rows.  The product runs transposed, S^T = K Q^T, on bf16 MFMA 16x16x32: a lane's four
// accumulators are then four consecutive columns of one row, stored as one 16-byte write, and a
// store instruction covers 64 contiguous bytes of 16 rows.
constexpr int kPfThreads = 256;

template <int D>
__global__ __launch_bounds__(kPfThreads) void k_index_scores_prefill(const uint16_t* __restrict__ q_idx,
                                                                      const uint16_t* __restrict__ k_idx,
                                                                      const int32_t* __restrict__ cu, int seq, int pos0,
                                                                      int n_rows, float* __restrict__ scores, int64_t ld,
                                                                      PrefillGrid grid, uint32_t* __restrict__ clear,
                                                                      int n_clear) {
  constexpr int KS = D / 32;                       // MFMA k-steps
  constexpr int CH = D / 8;                        // 16-byte chunks per K_idx row
  constexpr int WROWS = kPfTile / (kPfThreads / 64);  // query rows per wave
  constexpr int RPW = WROWS / 16;                  // 16-row MFMA blocks per wave
  static_assert(RPW >= 1 && kPfTile * CH % kPfThreads == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t kt[kPfTile * D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  if (clear != nullptr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_clear; i += blockDim.x) clear[i] = 0u;
  const int64_t base = cu[seq];
  const int ncols = pos0 + n_rows;  // tokens any row of this call sees
  // Workgroup ids are dealt to the 8 XCDs in turn, so workgroup b takes tile (b % 8) per_xcd + b / 8:
  // each XCD then works through one contiguous band of row blocks, and its L2 holds that band's
  // queries and the keys they see instead of every tile's inputs.
  const int64_t per_xcd = (grid.tiles + 7) / 8;
  for (int64_t b = blockIdx.x; b < 8 * per_xcd; b += gridDim.x) {
    const int64_t t = (b % 8) * per_xcd + b / 8;
    if (t >= grid.tiles) continue;  // the padding of the last band (uniform in the workgroup)
    int rb, cb;
    prefill_tile(grid, t, &rb, &cb);
    const int r0 = rb * kPfTile;  // first row of the tile
    const int k0 = cb * kPfTile;  // first token column
    __syncthreads();  // the previous tile's fragment reads are done
    // stage the tile's K_idx rows (columns past the call's last token read that token, unused)
#pragma unroll
    for (int i = 0; i < kPfTile * CH / kPfThreads; ++i) {
      const int e = i * kPfThreads + threadIdx.x;
      const int key = e / CH, ch = e % CH;
      const int col = k0 + key < ncols ? k0 + key : ncols - 1;
      const uint4 v = load16(k_idx + (base + col) * D + ch * 8);
      *reinterpret_cast<uint4*>(kt + key * D + ((ch ^ (key & (CH - 1))) * 8)) = v;
    }
    // this wave's query fragments: rows r0 + WROWS wave + 16 rblk + l16, d = 32 ks + 8 grp ..
    bf16x8_t qf[RPW][KS];
#pragma unroll
    for (int rblk = 0; rblk < RPW; ++rblk) {
      const int row = r0 + wave * WROWS + rblk * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < n_rows) v = load16(q_idx + (int64_t)row * D + ks * 32 + grp * 8);
        qf[rblk][ks] = bitcast<bf16x8_t>(v);
      }
    }
    __syncthreads();
    const int wrow0 = r0 + wave * WROWS;
    if (wrow0 >= n_rows || k0 > pos0 + wrow0 + WROWS - 1) continue;  // no visible entry for this wave
#pragma unroll
    for (int kb = 0; kb < kPfTile / 16; ++kb) {
      const int key = kb * 16 + l16;
      floatx4_t acc[RPW];
#pragma unroll
      for (int rblk = 0; rblk < RPW; ++rblk) acc[rblk] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(kt + key * D + (((ks * 4 + grp) ^ (key & (CH - 1))) * 8));
#pragma unroll
        for (int rblk = 0; rblk < RPW; ++rblk)
          acc[rblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a), qf[rblk][ks], acc[rblk], 0, 0, 0);
      }
      // acc[rblk][j]: row wrow0 + 16 rblk + l16, column k0 + 16 kb + 4 grp + j
      const int col = k0 + kb * 16 + grp * 4;
#pragma unroll
      for (int rblk = 0; rblk < RPW; ++rblk) {
        const int row = wrow0 + rblk * 16 + l16;
        if (row >= n_rows) continue;
        const int lim = pos0 + row;  // last visible column of the row
        float* p = scores + (int64_t)row * ld + col;
        if (col + 3 <= lim) {
          *reinterpret_cast<floatx4_t*>(p) = acc[rblk];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (col + j <= lim) p[j] = acc[rblk][j];
        }
      }
    }
  }
}

}  // namespace

int launch_index_scores_decode(const RowsDev& rows, int d_idx, int seg, const uint16_t* q_idx, int64_t q_stride,
                               const uint16_t* k_idx, float* scores, int64_t ld, uint16_t* hpart, uint32_t* hinfo,
                               int topk, int hpart_chunks, uint32_t* clear, int n_clear, void* stream) {
  const int64_t segs = (rows.total_tokens + seg - 1) / seg;
  const dim3 grid((unsigned)(segs > 0 ? segs : 1));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d_idx == 128)
    hipLaunchKernelGGL(k_index_scores_decode<128>, grid, dim3(kIdxThreads), 0, s, q_idx, q_stride, k_idx, rows.cu,
                       rows.n_rows, rows.max_row_len, seg, rows.total_tokens, scores, ld, hpart, hinfo, topk,
                       hpart_chunks, clear, n_clear);
  else
    hipLaunchKernelGGL(k_index_scores_decode<64>, grid, dim3(kIdxThreads), 0, s, q_idx, q_stride, k_idx, rows.cu,
                       rows.n_rows, rows.max_row_len, seg, rows.total_tokens, scores, ld, hpart, hinfo, topk,
                       hpart_chunks, clear, n_clear);
  return (int)hipGetLastError();
}

int launch_index_scores_prefill(const RowsDev& rows, int d_idx, const uint16_t* q_idx, const uint16_t* k_idx,
                                float* scores, int64_t ld, uint32_t* clear, int n_clear, void* stream) {
  const PrefillGrid g = prefill_grid(rows.pos0, rows.n_rows);
  // one workgroup per tile, up to a cap beyond which workgroups loop over tiles
  const int64_t cap = (int64_t)1 << 20;
  const int64_t padded = (g.tiles + 7) / 8 * 8;  // whole rounds over the 8 XCDs
  const dim3 grid((unsigned)(padded < cap ? padded : cap));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d_idx == 128)
    hipLaunchKernelGGL(k_index_scores_prefill<128>, grid, dim3(kPfThreads), 0, s, q_idx, k_idx, rows.cu, rows.seq,
                       rows.pos0, rows.n_rows, scores, ld, g, clear, n_clear);
  else
    hipLaunchKernelGGL(k_index_scores_prefill<64>, grid, dim3(kPfThreads), 0, s, q_idx, k_idx, rows.cu, rows.seq,
                       rows.pos0, rows.n_rows, scores, ld, g, clear, n_clear);
  return (int)hipGetLastError();
}

const char* device_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace clsa
