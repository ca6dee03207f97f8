// The step before the routing: the shared indexer's projections of each decode sequence's new
// token (picx.dev summary of "You Only Index Once", Methodology > Architecture Overview, eq. 1:
// Q_idx = H W_idx^Q, K_idx = H W_idx^K) and the append of that token to the caches.
//
// out[b, j] = sum_c h[b, c] * w[j, c] over the 2 * d_idx channels [query | key]: a skinny
// product (a few sequences x 128 or 256 channels x d_model) whose time is the time to move the
// operands through the compute units.  One CU streams only some tens of GB/s (its outstanding
// misses bound it), so the work is cut into small output tiles - 4 sequences x 4 channels over
// the whole of d_model, one workgroup each - which spreads the weights over every CU (256
// workgroups of 64 KB each for 16 sequences at d_model 4096) and needs no reduction across
// workgroups.  Each thread takes 16-byte pieces of d_model from the 8 operand rows and
// accumulates the 16 dot products with v_dot2_f32_bf16 in fp32; the workgroup then sums the
// threads' partials in a fixed order (LDS, then a 16-lane DPP butterfly), so the result does not
// depend on timing.  Results are rounded to bf16 (nearest, ties to even): query channels go to
// q_idx[b], key channels to the sequence's last row of k_idx.  B more workgroups copy the new K
// and V rows into the caches, one sequence each.
#include "device_common.h"

namespace clsa {

namespace {

constexpr int kProjThreads = 256;
constexpr int kTile = 4;            // sequences and channels per workgroup
constexpr int kPieceRounds = 2;     // 16-byte pieces per operand row each thread has in flight

struct ProjArgs {
  const uint16_t* h;      // [B, d_model]
  const uint16_t* wq;     // [d_idx, d_model]
  const uint16_t* wk;     // [d_idx, d_model]
  const int32_t* cu;      // [B + 1]
  uint16_t* q_idx;        // [B, d_idx]
  uint16_t* k_idx;        // [T, d_idx]
  const uint16_t* k_new;  // [B, hkv, 128] or null
  const uint16_t* v_new;  // [B, hkv, 128] or null
  uint16_t* k_cache;      // [T, hkv, 128]
  uint16_t* v_cache;      // [T, hkv, 128]
  int64_t total_tokens;
  int batch, d_idx, d_model, hkv;
  int ch_tiles, proj_tiles;  // channel tiles (2 d_idx / 4); projection workgroups
};

// Cache row of sequence b's new token (its last position), or -1 if the sequence is empty or
// reaches past the cache: then nothing is written for it.
__device__ __forceinline__ int64_t new_token_row(const ProjArgs& a, int b) {
  const int64_t beg = a.cu[b], end = a.cu[b + 1];
  return (end > beg && beg >= 0 && end <= a.total_tokens) ? end - 1 : -1;
}

// acc + sum of the 8 bf16 products of two 16-byte pieces (fp32, in element-pair order)
__device__ __forceinline__ float dot8(const uint4& x, const uint4& y, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.x), __builtin_bit_cast(bf16x2_t, y.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.y), __builtin_bit_cast(bf16x2_t, y.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.z), __builtin_bit_cast(bf16x2_t, y.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.w), __builtin_bit_cast(bf16x2_t, y.w), acc, false);
  return acc;
}

// Copy sequence b's new K and V rows (hkv * 128 bf16 each) into its last cache row.
__device__ void append_kv(const ProjArgs& a, int b) {
  const int per = a.hkv * 128 / 8;  // 16-byte pieces per token row
  const int64_t row = new_token_row(a, b);
  constexpr int kUnroll = 4;
  for (int i0 = threadIdx.x; i0 < 2 * per; i0 += kUnroll * kProjThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kProjThreads;
      if (i < 2 * per) v[u] = load16((i < per ? a.k_new : a.v_new) + ((int64_t)b * per + (i < per ? i : i - per)) * 8);
    }
    if (row < 0) continue;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kProjThreads;
      if (i < 2 * per)
        *reinterpret_cast<uint4*>((i < per ? a.k_cache : a.v_cache) + (row * per + (i < per ? i : i - per)) * 8) = v[u];
    }
  }
}

__global__ __launch_bounds__(kProjThreads) void k_index_project(ProjArgs a) {
  if ((int)blockIdx.x >= a.proj_tiles) {  // K / V append, one sequence per workgroup
    if (a.k_new != nullptr) append_kv(a, (int)blockIdx.x - a.proj_tiles);
    return;
  }
  const int ch0 = (blockIdx.x % a.ch_tiles) * kTile;  // the tile never straddles query and key
  const int b0 = (blockIdx.x / a.ch_tiles) * kTile;
  // output of thread t with t % 16 == 0: (sequence b0 + t / 64, channel ch0 + (t / 16) % 4); the
  // cache row a key channel goes to is requested now, alongside the operands
  const int j = threadIdx.x >> 4;
  const int out_b = b0 + (j >> 2), out_ch = ch0 + (j & 3);
  const bool writes = (threadIdx.x & 15) == 0 && out_b < a.batch;
  const int64_t key_row = (writes && out_ch >= a.d_idx) ? new_token_row(a, out_b) : -1;
  const uint16_t* hr[kTile];
  const uint16_t* wr[kTile];
#pragma unroll
  for (int i = 0; i < kTile; ++i) {
    const int b = b0 + i < a.batch ? b0 + i : a.batch - 1;  // rows past the batch are read, not written
    hr[i] = a.h + (int64_t)b * a.d_model;
    const int ch = ch0 + i;
    wr[i] = ch < a.d_idx ? a.wq + (int64_t)ch * a.d_model : a.wk + (int64_t)(ch - a.d_idx) * a.d_model;
  }
  float acc[kTile * kTile];
#pragma unroll
  for (int k = 0; k < kTile * kTile; ++k) acc[k] = 0.f;
  const int pieces = a.d_model / 8;
  for (int p0 = threadIdx.x; p0 < pieces; p0 += kPieceRounds * kProjThreads) {
    uint4 hv[kPieceRounds][kTile], wv[kPieceRounds][kTile];
#pragma unroll
    for (int u = 0; u < kPieceRounds; ++u) {
      const int p = p0 + u * kProjThreads;
#pragma unroll
      for (int i = 0; i < kTile; ++i) {
        hv[u][i] = make_uint4(0u, 0u, 0u, 0u);
        wv[u][i] = make_uint4(0u, 0u, 0u, 0u);
        if (p < pieces) {
          hv[u][i] = load16(hr[i] + (int64_t)p * 8);
          wv[u][i] = load16(wr[i] + (int64_t)p * 8);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPieceRounds; ++u)
#pragma unroll
      for (int s = 0; s < kTile; ++s)
#pragma unroll
        for (int c = 0; c < kTile; ++c) acc[s * kTile + c] = dot8(hv[u][s], wv[u][c], acc[s * kTile + c]);
  }
  // fixed-order reduction: output j sums thread slots q, q + 16, ..., q + 240 in lane q of a
  // 16-lane row, then the row's 16 lanes are combined by a butterfly (every lane ends with the
  // same value)
  __shared__ float red[kTile * kTile][kProjThreads];
#pragma unroll
  for (int k = 0; k < kTile * kTile; ++k) red[k][threadIdx.x] = acc[k];
  __syncthreads();
  const int q = threadIdx.x & 15;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kProjThreads / 16; ++i) s += red[j][i * 16 + q];
  s += dpp_partner<8>(s);
  s += dpp_partner<4>(s);
  s += dpp_partner<2>(s);
  s += dpp_partner<1>(s);
  if (writes) {
    const uint16_t v = (uint16_t)f32_to_bf16(s);
    if (out_ch < a.d_idx) a.q_idx[(int64_t)out_b * a.d_idx + out_ch] = v;
    else if (key_row >= 0) a.k_idx[key_row * a.d_idx + (out_ch - a.d_idx)] = v;
  }
}

}  // namespace

int launch_index_project(int batch, int d_idx, int d_model, int hkv, int64_t total_tokens, const uint16_t* h,
                         const uint16_t* wq, const uint16_t* wk, const int32_t* cu, uint16_t* q_idx, uint16_t* k_idx,
                         const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache,
                         void* stream) {
  ProjArgs a;
  a.h = h;
  a.wq = wq;
  a.wk = wk;
  a.cu = cu;
  a.q_idx = q_idx;
  a.k_idx = k_idx;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.total_tokens = total_tokens;
  a.batch = batch;
  a.d_idx = d_idx;
  a.d_model = d_model;
  a.hkv = hkv;
  a.ch_tiles = 2 * d_idx / kTile;
  a.proj_tiles = a.ch_tiles * ((batch + kTile - 1) / kTile);
  const int copies = k_new != nullptr ? batch : 0;
  hipLaunchKernelGGL(k_index_project, dim3((unsigned)(a.proj_tiles + copies)), dim3(kProjThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace clsa
