// The multi-layer distillation target and loss (picx.dev summary of "You Only Index Once",
// Methodology, Multi-Layer Distillation, eq. 4-5): for every prefill position t,
//   A_t = 1/(L Hq) sum over layers l and query heads h of softmax_j(q_t^(l,h) . k_j^(g(h)) * scale)
//   KL_t = KL(A_t || softmax_j(I_t)) = sum_j A_tj (ln A_tj - ln softmax(I_t)_j),   j = 0..t,
// and the loss, the mean of KL_t over the positions.  The attention scale is the layers' own
// 1/sqrt(head_dim) and KV head g(h) = floor(h Hkv / Hq), as in the attention of the step.
//
// A_t needs every (layer, head) distribution normalised before they are summed, so there are
// two passes over the keys, both on bf16 MFMA (16x16x32, fp32 accumulate) with the exp2-domain
// softmax of the attention kernel:
//  1. k_distill_stats: the log2 normaliser of each (position, layer, head).  Workgroup = 16
//     positions x up to 32 (layer, head) pairs of one KV head; each wave keeps 4 pairs x 16
//     positions of queries in registers, the KV head's keys stream through LDS in 64-key tiles,
//     S^T = K Q^T, and the running max and sum stay in the lane that owns the query column
//     (the max is raised lazily, only past a growth of 2^8).
//  2. k_distill_kl: A over a tile of 32 positions x 256 keys.  Each wave keeps its 64 keys of
//     the current KV head in registers; the (layer, head) pairs' query blocks stream through LDS
//     (double-buffered), and exp2(s * c - lse2) is added into lane-local accumulators, so the
//     sum over the L * Hq pairs needs no exchange.  The tile's KL terms are then summed in a
//     fixed order into one partial per (position, 256-key block).
// k_row_lse gives the log-sum-exp of each row of I, k_distill_rowsum sums the partials of every
// position and k_distill_loss the rows, each in a fixed order, so the results do not depend on
// timing.  The vector ALU, not the matrix cores, bounds both passes: every score costs one exp2,
// one fma and one add, against 1/16 of a 16x16x32 MFMA for the q.k products.
#include "device_common.h"

namespace clsa {

namespace {

constexpr int kTileKeys = 64;
constexpr int kTileBytes = kTileKeys * CLSA_HEAD_DIM * 2;  // 16 KB: 64 rows of 256 bytes
constexpr int kDstWaves = 8;
constexpr int kDstThreads = 64 * kDstWaves;
constexpr int kStatRows = 16;                          // positions per stats workgroup
constexpr int kStatPairsPerWave = 4;
constexpr int kStatPairs = kDstWaves * kStatPairsPerWave;
constexpr int kStatTilesPerStep = 2;                    // 64-key tiles per LDS step
constexpr int kStatPieces = kTileKeys * 16 / kDstThreads;  // 16-byte pieces of a key tile per thread
static_assert(kStatPieces * kDstThreads == kTileKeys * 16, "whole tile pieces per thread");
// KL pass: four-wave workgroups of 32 positions x 256 keys, three per CU (each wave keeps its 64
// keys of the current KV head in registers and accumulates 64 keys x 32 positions of A)
constexpr int kKlWaves = 4;
constexpr int kKlThreads = 64 * kKlWaves;
constexpr int kKlBlocksPerCU = 3;
constexpr int kKlRows = kDistillRowBlock;                // positions per KL workgroup
constexpr int kKlTq = kKlRows / 16;                      // 16-position MFMA blocks
constexpr int kKlKeysPerWave = 64;
constexpr int kKlKeys = kKlWaves * kKlKeysPerWave;       // keys per KL workgroup
constexpr int kKlPieces = kKlRows * 16 / kKlThreads;     // 16-byte query pieces per thread per pair
constexpr int kKlQBytes = kKlRows * CLSA_HEAD_DIM * 2;   // one (layer, head) query block in LDS
constexpr int kKlPairsPerStep = 2;                       // (layer, head) query blocks per LDS step
static_assert(kKlPieces * kKlThreads == kKlRows * 16, "whole query pieces per thread");
static_assert(kKlKeys == kDistillKeyBlock, "key block of the KL partials");
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleLog2 = 8.f;

struct DistillArgs {
  int pos0, n_rows, seq;  // rows: positions pos0 .. pos0 + n_rows - 1 of sequence seq
  const int32_t* cu;
  int64_t total_tokens;   // rows of the cache; no key read goes past it
  int L, hq, hkv, group, pairs_per_g, n_kb;
  float c;                // softmax scale * log2(e)
  const uint16_t* q;      // row i at q + i * q_stride: [L, hq, 128]
  int64_t q_stride;
  const uint16_t* k;      // [T, hkv, 128]
  const float* scores;    // [n_rows, ld]
  int64_t ld;
  float* lse2;            // [n_rows, L * hq]: log2 of each (row, layer, head) softmax normaliser
  float* lse_i;           // [n_rows]: natural log-sum-exp of the row's scores
  float* part;            // [n_rows, n_kb]
  float* kl;              // [n_rows]
  float* loss;            // [1] or null
  int64_t kl_tiles;       // workgroups of the KL pass, one per causal tile
};

// Byte offset, in a tile of 64 rows x 128 bf16, of the 16-byte chunk `chunk` of row `row`: chunk
// slot chunk ^ (row & 15), so that row stores and 16-lane fragment reads spread over the banks.
__device__ __forceinline__ int tile_off(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// ---------------------------------------------------------------------------------------------
// log-sum-exp of each row of the scores (natural log), over the row's visible tokens
__global__ __launch_bounds__(256) void k_row_lse(DistillArgs a) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  const int n = a.pos0 + i + 1;
  const float* s = a.scores + (int64_t)i * a.ld;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < n; j += 256) mx = fmaxf(mx, s[j]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = threadIdx.x; j < n; j += 256) sum += __builtin_amdgcn_exp2f((s[j] - mx) * 1.4426950408889634f);
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) a.lse_i[i] = mx + __builtin_amdgcn_logf((red[0] + red[1]) + (red[2] + red[3])) * kLn2;
}

// ---------------------------------------------------------------------------------------------
// pass 1: log2 normaliser of every (position, layer, head)
__global__ __launch_bounds__(kDstThreads) void k_distill_stats(DistillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStatTilesPerStep * kTileKeys * CLSA_HEAD_DIM];
  char* const lds_bytes = reinterpret_cast<char*>(lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  // row blocks last first: a block's work grows with its positions, so within each KV head the
  // longest blocks are dispatched first and the grid ends on short ones
  const int r0 = (int)(gridDim.x - 1 - blockIdx.x) * kStatRows;
  const int g = blockIdx.y % a.hkv, chunk = blockIdx.y / a.hkv;
  const int last_row = (r0 + kStatRows < a.n_rows ? r0 + kStatRows : a.n_rows) - 1;
  const int t_lo = a.pos0 + r0, t_hi = a.pos0 + last_row;  // keys 0 .. t_hi are read
  const int64_t seq_base = a.cu[a.seq];
  const int key_cap = (int)min((int64_t)t_hi, a.total_tokens - 1 - seq_base);  // loads stay in the cache
  // this lane's query column: position t of row r0 + l16 (rows past the block repeat the last)
  const int row = r0 + l16 <= last_row ? r0 + l16 : last_row;
  const int t = a.pos0 + row;
  const int p0 = chunk * kStatPairs + wave * kStatPairsPerWave;
  const bool wave_active = p0 < a.pairs_per_g;
  bf16x8_t qf[kStatPairsPerWave][4];
  int qh[kStatPairsPerWave];  // layer * hq + head of each query block, -1 when past the pairs
#pragma unroll
  for (int qb = 0; qb < kStatPairsPerWave; ++qb) {
    const int p = p0 + qb;
    qh[qb] = p < a.pairs_per_g ? (p / a.group) * a.hq + g * a.group + p % a.group : -1;
    const uint16_t* qp = a.q + (int64_t)row * a.q_stride + (int64_t)(qh[qb] < 0 ? 0 : qh[qb]) * CLSA_HEAD_DIM;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (qh[qb] >= 0) v = load16(qp + kk * 32 + grp * 8);
      qf[qb][kk] = bitcast<bf16x8_t>(v);
    }
  }
  // loader: 64 keys x 16 chunks per tile, kStatPieces pieces per thread; keys past t_hi re-read t_hi
  const int64_t kbase = (seq_base * a.hkv + g) * CLSA_HEAD_DIM;
  int lkey[kStatPieces], lchunk[kStatPieces], soff[kStatPieces];
#pragma unroll
  for (int i = 0; i < kStatPieces; ++i) {
    const int piece = threadIdx.x + i * kDstThreads;
    lkey[i] = piece >> 4;
    lchunk[i] = piece & 15;
    soff[i] = tile_off(lkey[i], lchunk[i]);
  }
  uint4 rk[kStatTilesPerStep][kStatPieces];
  auto load_step = [&](int st) {
#pragma unroll
    for (int u = 0; u < kStatTilesPerStep; ++u)
#pragma unroll
      for (int i = 0; i < kStatPieces; ++i) {
        int key = (st * kStatTilesPerStep + u) * kTileKeys + lkey[i];
        key = key < key_cap ? key : key_cap;
        rk[u][i] = load16(a.k + kbase + (int64_t)key * a.hkv * CLSA_HEAD_DIM + lchunk[i] * 8);
      }
  };
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = tile_off(l16, 4 * kk + grp);
  float m_run[kStatPairsPerWave], l_run[kStatPairsPerWave];
#pragma unroll
  for (int qb = 0; qb < kStatPairsPerWave; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float c = a.c;
  // One 64-key tile: S^T = K Q^T for the wave's 4 pairs x 16 positions, then the online max and
  // sum of each query column.
  auto compute_tile = [&](const char* tb, int tile) {
    floatx4_t s[kStatPairsPerWave][4];
#pragma unroll
    for (int qb = 0; qb < kStatPairsPerWave; ++qb)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) s[qb][mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // one block of 16 keys at a time, the next block's K fragments read from LDS meanwhile
    uint4 av[2][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) av[0][kk] = *reinterpret_cast<const uint4*>(tb + koff[kk]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt + 1 < 4) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) av[(mt + 1) & 1][kk] = *reinterpret_cast<const uint4*>(tb + koff[kk] + (mt + 1) * 4096);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int qb = 0; qb < kStatPairsPerWave; ++qb)
          s[qb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(av[mt & 1][kk]), qf[qb][kk], s[qb][mt], 0, 0, 0);
    }
    // s[qb][mt][j]: q . k of key tile * 64 + 16 mt + 4 grp + j, query column l16; keys past the
    // column's position are masked (only tiles reaching past the block's first position have any)
    if (tile * kTileKeys + kTileKeys - 1 > t_lo) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tile * kTileKeys + mt * 16 + grp * 4 + j > t)
#pragma unroll
            for (int qb = 0; qb < kStatPairsPerWave; ++qb) s[qb][mt][j] = -INFINITY;
    }
    // The maxima use the NaN-propagating maximum: three operands per instruction and no
    // canonicalisation of the MFMA results, which the IEEE maxNum of fmaxf needs on each input
    // (the scores are finite or -inf, so both give the same value).
    auto max3 = [](float x, float y, float z) {
      return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
    };
#pragma unroll
    for (int qb = 0; qb < kStatPairsPerWave; ++qb) {
      const floatx4_t* v = s[qb];  // 16 scores: a tree of eight three-operand maxima
      float mx = max3(max3(v[0][0], v[0][1], v[0][2]), max3(v[0][3], v[1][0], v[1][1]),
                      max3(v[1][2], v[1][3], v[2][0]));
      mx = max3(mx, max3(v[2][1], v[2][2], v[2][3]), max3(v[3][0], v[3][1], v[3][2]));
      mx = __builtin_elementwise_maximum(mx, v[3][3]);
      if (__any(mx * c > m_run[qb] + kRescaleLog2)) {
        mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 16, 64));
        mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32, 64));
        const float m_new = __builtin_elementwise_maximum(m_run[qb], mx * c);
        l_run[qb] *= __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
      }
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += __builtin_amdgcn_exp2f(fmaf(s[qb][mt][j], c, -m_run[qb]));
      l_run[qb] += sum;
    }
  };
  // steps of kStatTilesPerStep tiles: the next step is loaded while this one is computed, and the
  // workgroup meets at one barrier per step
  const int ntiles = t_hi / kTileKeys + 1;
  const int steps = (ntiles + kStatTilesPerStep - 1) / kStatTilesPerStep;
  load_step(0);
  for (int st = 0; st < steps; ++st) {
    char* sb = lds_bytes + (st & 1) * kStatTilesPerStep * kTileBytes;
#pragma unroll
    for (int u = 0; u < kStatTilesPerStep; ++u)
#pragma unroll
      for (int i = 0; i < kStatPieces; ++i) *reinterpret_cast<uint4*>(sb + u * kTileBytes + soff[i]) = rk[u][i];
    __syncthreads();  // one barrier per step: buffer st & 1 was last read two steps ago
    if (st + 1 < steps) load_step(st + 1);
    if (!wave_active) continue;
#pragma unroll
    for (int u = 0; u < kStatTilesPerStep; ++u) {
      const int tile = st * kStatTilesPerStep + u;
      if (tile < ntiles) compute_tile(sb + u * kTileBytes, tile);
    }
  }
  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < kStatPairsPerWave; ++qb) {
    float l = l_run[qb] + __shfl_xor(l_run[qb], 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (grp == 0 && r0 + l16 <= last_row && qh[qb] >= 0)
      a.lse2[(int64_t)(r0 + l16) * a.L * a.hq + qh[qb]] = m_run[qb] + __builtin_amdgcn_logf(l);
  }
}

// ---------------------------------------------------------------------------------------------
// pass 2: A over 32 positions x 256 keys, then the tile's KL terms per position
__global__ __launch_bounds__(kKlThreads, kKlBlocksPerCU) void k_distill_kl(DistillArgs a) {
  // two steps of kKlPairsPerStep (layer, head) query blocks: the next step is loaded while this
  // one is computed, and the workgroup meets at one barrier per step
  __shared__ __attribute__((aligned(16))) uint16_t qlds[2 * kKlPairsPerStep * kKlRows * CLSA_HEAD_DIM];
  __shared__ float llds[2][kKlPairsPerStep][kKlRows];
  __shared__ float red[kKlWaves][kKlRows];
  char* const q_bytes = reinterpret_cast<char*>(qlds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  // one workgroup per causal tile (kl_tile in clsa_internal.h), and no others: a 2-D grid over
  // every (key block, row block) pair holds about as many tiles past the diagonal as before it,
  // and those workgroups, though they exit at once, still wait for a free slot to be dispatched
  // (on the 8192-position workload fewer than half the slots were busy, and the pass took 3.8 ms
  // instead of 2.4)
  const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  if (tile >= a.kl_tiles) return;  // the last grid row of a call with more than 2^23 tiles
  int kb, rb;
  kl_tile(a.pos0, a.n_rows, tile, &rb, &kb);
  const int r0 = rb * kKlRows;
  const int last_row = (r0 + kKlRows < a.n_rows ? r0 + kKlRows : a.n_rows) - 1;
  const int t_hi = a.pos0 + last_row;
  const int k0 = kb * kKlKeys;
  if (k0 > t_hi) return;  // not a tile of the list (never true for tiles below kl_tile_count)
  const int wk0 = k0 + wave * kKlKeysPerWave;
  const bool wave_active = wk0 <= t_hi;
  const int P = a.L * a.hq;
  // query-block loader: kKlRows rows x 16 chunks, kKlPieces pieces per thread
  int lrow[kKlPieces], lchunk[kKlPieces], soff[kKlPieces];
#pragma unroll
  for (int i = 0; i < kKlPieces; ++i) {
    const int piece = threadIdx.x + i * kKlThreads;
    lrow[i] = piece >> 4;
    lchunk[i] = piece & 15;
    soff[i] = tile_off(lrow[i], lchunk[i]);
    if (r0 + lrow[i] > last_row) lrow[i] = last_row - r0;
  }
  uint4 rq[kKlPairsPerStep][kKlPieces];
  float rl[kKlPairsPerStep];
  // pair index pi = g * pairs_per_g + p  ->  (layer p / group, head g * group + p % group)
  auto pair_qh = [&](int pi) {
    const int g = pi / a.pairs_per_g, p = pi % a.pairs_per_g;
    return (p / a.group) * a.hq + g * a.group + p % a.group;
  };
  auto load_step = [&](int st) {
#pragma unroll
    for (int u = 0; u < kKlPairsPerStep; ++u) {
      const int pi = st * kKlPairsPerStep + u;
      const int qh = pair_qh(pi < P ? pi : P - 1);  // past the last pair: re-read it, unused
#pragma unroll
      for (int i = 0; i < kKlPieces; ++i)
        rq[u][i] = load16(a.q + (int64_t)(r0 + lrow[i]) * a.q_stride + (int64_t)qh * CLSA_HEAD_DIM + lchunk[i] * 8);
      if (threadIdx.x < kKlRows) {
        const int rr = r0 + threadIdx.x <= last_row ? r0 + threadIdx.x : last_row;
        rl[u] = a.lse2[(int64_t)rr * P + qh];
      }
    }
  };
  int qoff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qoff[kk] = tile_off(l16, 4 * kk + grp);
  // this wave's keys: rows wk0 + 16 mt + l16 of the A operand (clamped for the loads)
  const int64_t seq_base = a.cu[a.seq];
  const int key_cap = (int)min((int64_t)t_hi, a.total_tokens - 1 - seq_base);  // loads stay in the cache
  const int64_t kbase = seq_base * a.hkv * CLSA_HEAD_DIM;
  int64_t krow[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    int key = wk0 + mt * 16 + l16;
    key = key < key_cap ? key : key_cap;
    krow[mt] = kbase + (int64_t)key * a.hkv * CLSA_HEAD_DIM + grp * 8;
  }
  bf16x8_t kf[4][4];
  floatx4_t abar[4][kKlTq];  // [mt][tq]: key wk0 + 16 mt + 4 grp + j, row r0 + 16 tq + l16
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int tq = 0; tq < kKlTq; ++tq) abar[mt][tq] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const float c = a.c;
  // One (layer, head) pair: S^T = K Q^T for the wave's 64 keys x kKlRows positions, and
  // exp2(s c - lse2) into the accumulators, one block of 16 positions at a time.  Keys past a
  // position get meaningless values here; they are never read back.
  auto compute_pair = [&](const char* qb, const float* lse_row) {
#pragma unroll
    for (int tq = 0; tq < kKlTq; ++tq) {
      bf16x8_t qv[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qv[kk] = bitcast<bf16x8_t>(*reinterpret_cast<const uint4*>(qb + qoff[kk] + tq * 4096));
      floatx4_t s[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) s[mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt][kk], qv[kk], s[mt], 0, 0, 0);
      const float lse = lse_row[tq * 16 + l16];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) abar[mt][tq][j] += __builtin_amdgcn_exp2f(fmaf(s[mt][j], c, -lse));
    }
  };
  const int steps = (P + kKlPairsPerStep - 1) / kKlPairsPerStep;
  load_step(0);
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
#pragma unroll
    for (int u = 0; u < kKlPairsPerStep; ++u) {
      char* qb = q_bytes + (buf * kKlPairsPerStep + u) * kKlQBytes;
#pragma unroll
      for (int i = 0; i < kKlPieces; ++i) *reinterpret_cast<uint4*>(qb + soff[i]) = rq[u][i];
      if (threadIdx.x < kKlRows) llds[buf][u][threadIdx.x] = rl[u];
    }
    __syncthreads();  // one barrier per step: buffer buf was last read two steps ago
    if (st + 1 < steps) load_step(st + 1);
    if (!wave_active) continue;
#pragma unroll
    for (int u = 0; u < kKlPairsPerStep; ++u) {
      const int pi = st * kKlPairsPerStep + u;
      if (pi >= P) break;
      if (pi % a.pairs_per_g == 0) {  // a new KV head: this wave's 64 keys of it
        const int g = pi / a.pairs_per_g;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            kf[mt][kk] = bitcast<bf16x8_t>(load16(a.k + krow[mt] + g * CLSA_HEAD_DIM + kk * 32));
      }
      compute_pair(q_bytes + (buf * kKlPairsPerStep + u) * kKlQBytes, llds[buf][u]);
    }
  }
  // KL terms of the tile: sum over the visible keys j of A (ln A - (I_j - lse_I))
  const float inv = 1.f / (float)P;
  float klp[kKlTq];
#pragma unroll
  for (int tq = 0; tq < kKlTq; ++tq) {
    klp[tq] = 0.f;
    const int row = r0 + tq * 16 + l16;
    if (!wave_active || row > last_row) continue;
    const int t = a.pos0 + row;
    const float lse_i = a.lse_i[row];
    const float* srow = a.scores + (int64_t)row * a.ld;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int key0 = wk0 + mt * 16 + grp * 4;
      if (key0 > t) continue;
      const float4 iv = *reinterpret_cast<const float4*>(srow + key0);
      const float ivs[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float av = abar[mt][tq][j] * inv;
        // weights below the smallest normal float add less than 1e-36 and are skipped, so the
        // logarithm never meets a flushed denormal
        if (key0 + j <= t && av >= 1.17549435e-38f)
          klp[tq] += av * (__builtin_amdgcn_logf(av) * kLn2 - (ivs[j] - lse_i));
      }
    }
  }
#pragma unroll
  for (int tq = 0; tq < kKlTq; ++tq) {
    float v = klp[tq] + __shfl_xor(klp[tq], 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (grp == 0) red[wave][tq * 16 + l16] = v;
  }
  __syncthreads();
  if (threadIdx.x < kKlRows && r0 + (int)threadIdx.x <= last_row) {
    float v = red[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kKlWaves; ++w) v += red[w][threadIdx.x];
    a.part[(int64_t)(r0 + threadIdx.x) * a.n_kb + kb] = v;
  }
}

// ---------------------------------------------------------------------------------------------
// KL of every row: one wave per row, lane b holding the partials of key blocks b, b + 64, ...
// summed by a fixed butterfly
constexpr int kRowSumThreads = 256;
__global__ __launch_bounds__(kRowSumThreads) void k_distill_rowsum(DistillArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = (int)blockIdx.x * (kRowSumThreads / 64) + (int)(threadIdx.x >> 6);
  if (i >= a.n_rows) return;
  const int nkb = (a.pos0 + i) / kKlKeys + 1;
  const float* p = a.part + (int64_t)i * a.n_kb;
  float v = 0.f;
  for (int b = lane; b < nkb; b += 64) v += p[b];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) a.kl[i] = v;
}

// the loss: mean of the rows' KL, thread t summing rows t, t + 1024, ... then a fixed tree
constexpr int kLossThreads = 1024;
__global__ __launch_bounds__(kLossThreads) void k_distill_loss(DistillArgs a) {
  __shared__ float red[kLossThreads / 64];
  float mine = 0.f;
  for (int i = threadIdx.x; i < a.n_rows; i += kLossThreads) mine += a.kl[i];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o, 64);
  if (lane == 0) red[wave] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int w = 0; w < kLossThreads / 64; ++w) s += red[w];
    a.loss[0] = s / (float)a.n_rows;
  }
}

}  // namespace

int launch_distill(const RowsDev& rows, int64_t total_tokens, int L, int hq, int hkv, float scale, const uint16_t* q,
                   int64_t q_stride, const uint16_t* k, const float* scores, int64_t ld, float* kl, float* loss,
                   void* ws, const DistillPlan& plan, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  DistillArgs a;
  a.pos0 = rows.pos0;
  a.n_rows = rows.n_rows;
  a.seq = rows.seq;
  a.cu = rows.cu;
  a.total_tokens = total_tokens;
  a.L = L;
  a.hq = hq;
  a.hkv = hkv;
  a.group = hq / hkv;
  a.pairs_per_g = L * a.group;
  a.n_kb = plan.n_kb;
  a.c = scale * 1.4426950408889634f;
  a.q = q;
  a.q_stride = q_stride;
  a.k = k;
  a.scores = scores;
  a.ld = ld;
  a.lse2 = reinterpret_cast<float*>(w + plan.lse2_off);
  a.lse_i = reinterpret_cast<float*>(w + plan.lse_i_off);
  a.part = reinterpret_cast<float*>(w + plan.part_off);
  a.kl = kl;
  a.loss = loss;
  const int chunks = (a.pairs_per_g + kStatPairs - 1) / kStatPairs;
  hipLaunchKernelGGL(k_row_lse, dim3((unsigned)rows.n_rows), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_distill_stats, dim3((unsigned)((rows.n_rows + kStatRows - 1) / kStatRows), (unsigned)(hkv * chunks)),
                     dim3(kDstThreads), 0, s, a);
  a.kl_tiles = plan.kl_tiles;
  // at most 2^23 workgroups per grid row (2^31 threads), further rows for larger calls
  const unsigned kl_x = (unsigned)(plan.kl_tiles < (1 << 23) ? plan.kl_tiles : (1 << 23));
  const unsigned kl_y = (unsigned)((plan.kl_tiles + kl_x - 1) / kl_x);
  hipLaunchKernelGGL(k_distill_kl, dim3(kl_x, kl_y), dim3(kKlThreads), 0, s, a);
  hipLaunchKernelGGL(k_distill_rowsum, dim3((unsigned)((rows.n_rows + kRowSumThreads / 64 - 1) / (kRowSumThreads / 64))),
                     dim3(kRowSumThreads), 0, s, a);
  if (loss != nullptr) hipLaunchKernelGGL(k_distill_loss, dim3(1), dim3(kLossThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace clsa
