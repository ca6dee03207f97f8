// Sparse attention over the shared selection (picx.dev summary of "You Only Index Once",
// Methodology > Architecture Overview, eq. 3: every cross-decoder layer attends to the same
// selected rows K_{S_t}, V_{S_t} of the one shared cache), with the softmax(QK^T/sqrt(d))V of
// the zhichai.net explainer (Background: Attention and Its Limits), and the Selector that
// gathers those rows (same explainer, CLSA: Sharing the Index Across Layers).
//
// One workgroup owns (query row r, KV head g, a block of up to 64 query rows, a split of the
// selected keys), or, with many blocks, (row r, a pair of adjacent KV heads), a team per head.
// The query rows of a KV head are all layers x the heads of its GQA group, so in the
// layer-batched schedule every K/V tile brought into LDS serves L * Hq / Hkv queries.
// The selected keys stream through LDS in stages of two 64-key tiles; the next stage's K/V rows
// are loaded into registers while the current one is computed.  Per tile: S^T = K Q^T and
// O^T += V^T P^T on bf16 MFMA 16x16x32 with fp32 accumulate; the online softmax (exp2 domain)
// keeps every statistic of a query in the lane that owns the query's column.  When the keys
// are split over several workgroups, each writes fp32 partials (m, l, acc) with device-scope
// stores and the last to arrive (atomic ticket) recombines them, so no separate pass is
// launched and no workgroup needs a device-wide cache flush.
#include "select_common.h"

namespace clsa {

namespace {

constexpr int kAttnWaveThreads = 256;  // threads of one team (four waves)
constexpr int kAttnPartWave = 34 * 64;             // floats per wave: acc 32 x 64 lanes, m, l
constexpr int kAttnPartWG = 4 * kAttnPartWave;     // floats per workgroup partial (team 0's four waves)
static_assert(kAttnPartWG == kAttnPartFloats, "partial record layout");

struct AttnArgs {
  RowsDev rw;
  int k, hq, hkv, lc, group, qrows, qblocks, splits, kps;
  float scale_log2;
  const uint16_t* q;
  int64_t q_stride;
  const uint16_t* ksrc;  // compact buffer [R, hkv, k, 128] or cache [T, hkv, 128]
  const uint16_t* vsrc;
  const int32_t* idx;
  const int32_t* count;
  uint16_t* out;
  int64_t o_stride;
  float* part;         // [splits, R, hkv, qblocks, kAttnPartWG] in the lanes' layout
  uint32_t* tickets;   // [R, hkv, qblocks], zero on entry, reset by their last workgroup
  // the row's unfinished selection (SELECT = true): span lists, their counts, t1 and the count
  // above it; one workgroup of each row writes the finished selection to idx_out / count_out
  const uint2* sel_slot;
  const uint32_t* sel_cnt;
  const uint32_t* sel_rowinfo;
  int sel_spans;
  int32_t* idx_out;
  int32_t* count_out;
};

// LDS of the selection finished inside the workgroup (nothing when SELECT = false).
template <bool SELECT>
struct SelectLds {};
template <>
struct SelectLds<true> {
  uint32_t hist[512];
  int scan[2 * 2 * kAttnWaveThreads / 64];
  int res[2];
  int span_pre[kMaxSelectSpans + 1];
  int32_t ids[kFusedMaxIds];  // this split's token ids, in selection order
};

// Four outputs scaled by inv, rounded to bf16 (round to nearest even) and stored as 8 bytes.
__device__ __forceinline__ void store_out4(uint16_t* p, const floatx4_t& v, float inv) {
  const bf16x2_t lo = {(__bf16)(v[0] * inv), (__bf16)(v[1] * inv)};
  const bf16x2_t hi = {(__bf16)(v[2] * inv), (__bf16)(v[3] * inv)};
  *reinterpret_cast<uint2*>(p) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// LDS tile layout: a tile holds 64 rows (keys) of 128 bf16 in row order; the 16-byte chunk c of
// row r sits at chunk slot c ^ (r & 15).  Row stores, K fragment reads and the transposed V
// reads then all spread over the banks without padding.

typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4_t lds_shortx4_t;

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i reads 4
// consecutive bf16 at its own address and receives element (i % 4) of the 4 values read by lanes
// 4k + i / 4, k = 0..3.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  const shortx4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// One stage = 2 tiles of 64 keys in LDS (2 x 32 KB).  A workgroup is TEAMS teams of WPT waves
// that all serve the same 16 WPT query rows (one 16-column MFMA block per wave):
//  * TEAMS = 2, WPT = 4 (one 8-wave workgroup per CU): team t computes tile t of every stage, so
//    each wave does one tile per stage; at the end the two teams merge their (m, l, acc) through
//    LDS.  Used when there are few (row, KV head) blocks and the keys are split across
//    workgroups.
//  * TEAMS = 1, WPT = 4 (two 4-wave workgroups per CU): every wave computes both tiles.  Used
//    when there are many blocks, so that two rows' gathers are in flight per CU.
//  * TEAMS = 2, WPT = 2 (two 4-wave workgroups per CU): as TEAMS = 1 for rows of at most 32
//    query rows (prefill: L x Hq / Hkv = 32), where one team of four waves would leave two of
//    them, and so two of the CU's four SIMDs, without MFMA work.
// The next stage's rows are in flight into registers while the current one is computed.
constexpr int kAttnTiles = 2;
// log2 of the growth of the running max that is absorbed without rescaling (P <= 2^this).
constexpr float kRescaleLog2 = 8.f;
// Split partials fetched per round trip by the combining workgroup.
constexpr int kCombineBatch = 4;

// SELECT (with FROM_CACHE, TEAMS = 2 and WPT = 4): the workgroup first finishes the row's
// long-row selection itself from the span lists of the select (see k_topk_select) and
// keeps its split's token ids in LDS, instead of reading them from idx.
// PAIR (TEAMS = 2, WPT = 4, no splits): team t takes KV head 2p + t of the workgroup's pair p,
// with its own tiles, loader and output, over the same selected keys; the teams pass the same
// barriers, so they stay in lockstep.
template <bool FROM_CACHE, int TEAMS, bool SELECT = false, int WPT = 4, bool PAIR = false>
__global__ __launch_bounds__(64 * WPT * TEAMS, 64 * WPT * TEAMS == 512 ? 1 : 2) void k_sparse_attn(AttnArgs a) {
  constexpr int NTH = 64 * WPT * TEAMS;            // threads
  constexpr int QB = 16 * WPT;                     // query rows per block
  constexpr int STAGE = kAttnTiles * kAttnTile;
  constexpr int TILE_ELEMS = kAttnTile * CLSA_HEAD_DIM;
  constexpr int HEADS = PAIR ? 2 : 1;              // KV heads per workgroup
  constexpr int HEAD_LDS = 2 * kAttnTiles * TILE_ELEMS;  // one head's K and V tiles, elements
  constexpr int LT = NTH / HEADS;                  // threads loading one head's rows
  constexpr int TPT = PAIR ? kAttnTiles : kAttnTiles / TEAMS;  // tiles each team computes per stage
  constexpr int TPP = LT / 256;                    // tiles the loader covers per group of 4 pieces
  constexpr int LPT = 4 * (kAttnTiles / TPP);      // K (and V) pieces each thread loads per stage
  static_assert(NTH == 256 || NTH == 512, "four or eight waves");
  static_assert(!SELECT || WPT == 4, "the fused selection runs on eight-wave workgroups");
  static_assert(TEAMS == 1 || TEAMS == 2, "one or two teams");
  static_assert(!PAIR || (TEAMS == 2 && WPT == 4), "a pair is two teams of four waves");
  // per head: K of tile t at t * TILE_ELEMS, V of tile t at (kAttnTiles + t) * TILE_ELEMS; the
  // same memory holds the team exchange at the end
  __shared__ __attribute__((aligned(16))) uint16_t lds[HEADS * HEAD_LDS];
  __shared__ int flag[1];
  __shared__ SelectLds<SELECT> sl;
  static_assert(!SELECT || (FROM_CACHE && TEAMS == 2), "the fused selection reads the cache with two teams");
  static_assert(kListLds * sizeof(uint2) <= sizeof(lds), "the candidate list fits the tile buffers");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int team = wave / WPT, tw = wave % WPT;
  const int l16 = lane & 15, grp = lane >> 4;
  int bid = blockIdx.x;
  const int split = bid % a.splits;
  bid /= a.splits;
  const int qb = bid % a.qblocks;
  const int gblk = bid / a.qblocks;                 // KV head, or pair of heads
  const int g = PAIR ? 2 * gblk + team : gblk;      // this team's KV head
  const int r = blockIdx.y;
  // The fused selection's loads (span counts, the first entries of the span lists, t1 and the count
  // above it) are requested first, bounded by the buffers' extents rather than by the row length,
  // whose own load would otherwise have to complete before them.
  CandidateLoads<NTH, 2, kMaxSelectSpans> cq;
  uint32_t sel_t1 = 0u, sel_above1 = 0u;
  if constexpr (SELECT) {
    request_candidates(cq, a.sel_slot + (int64_t)r * a.rw.max_row_len, a.sel_cnt + (int64_t)r * a.sel_spans,
                              a.sel_spans, a.rw.max_row_len);
    sel_t1 = a.sel_rowinfo[2 * r];
    sel_above1 = a.sel_rowinfo[2 * r + 1];
  }
  // the row's selected tokens: the fused selection's count, or the caller's (clamped into [0, k]
  // by split_key_range, so no position read lies past the row's k entries of idx or K_S/V_S)
  const int cnt = SELECT ? min(a.k, row_len(a.rw, r)) : a.count[r];
  int kbeg, kend;
  split_key_range(cnt, a.k, split, a.kps, &kbeg, &kend);

  // this lane's query column: query row qr -> (layer, head) of the GQA group of KV head g
  const int qr = qb * QB + tw * 16 + l16;
  const bool wave_active = qb * QB + tw * 16 < a.qrows;
  const bool q_valid = qr < a.qrows;
  const int layer = q_valid ? qr / a.group : 0;
  const int head = g * a.group + (q_valid ? qr % a.group : 0);
  bf16x8_t qf[4];
  {
    const uint16_t* qp = a.q + (int64_t)r * a.q_stride + ((int64_t)layer * a.hq + head) * CLSA_HEAD_DIM;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (q_valid) v = *reinterpret_cast<const uint4*>(qp + s * 32 + grp * 8);
      qf[s] = bitcast<bf16x8_t>(v);
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  floatx4_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int seq = row_seq(a.rw, r);
  const int64_t tok_base = FROM_CACHE ? (int64_t)a.rw.cu[seq] : 0;
  const int32_t* irow = a.idx + (int64_t)r * a.k;
  // token ids are clamped into the row's visible tokens, so that no index can send a load
  // outside the cache (valid selections are unchanged by it)
  const int tok_last = FROM_CACHE ? max(row_len(a.rw, r) - 1, 0) : 0;
  auto tok = [&](int id) { return id < 0 ? 0 : (id > tok_last ? tok_last : id); };
  // The fused selection: this split's token ids (selection positions kbeg .. kend - 1) into LDS.
  const int nk = kend > kbeg ? kend - kbeg : 0;
  if constexpr (SELECT) {
    const int n = row_len(a.rw, r);
    if (n <= a.k) {  // every visible token is selected (the select wrote idx and count already)
      for (int i = threadIdx.x; i < nk; i += blockDim.x) sl.ids[i] = kbeg + i;
    } else {
      const uint32_t t1 = sel_t1;
      const int above1 = (int)sel_above1;
      const int nsp = (n + kSelectSpan - 1) / kSelectSpan;
      const uint2* rslot = a.sel_slot + (int64_t)r * a.rw.max_row_len;
      uint2* list_lds = reinterpret_cast<uint2*>(lds);  // the tiles are not in use yet
      const int L = complete_candidates(cq, rslot, nsp, sl.span_pre, sl.scan, list_lds, nullptr);
      const bool writer = split == 0 && qb == 0 && gblk == 0;  // the same for every thread of the workgroup
      int32_t* orow = a.idx_out + (int64_t)r * a.k;
      auto emit = [&](int pos, int32_t t) {
        if (pos >= kbeg && pos < kend) sl.ids[pos - kbeg] = t;
        if (writer) orow[pos] = t;
      };
      if (L <= kListLds) {
        static_assert(kListLds % NTH == 0, "the LDS list fits the threads' registers");
        refine_and_emit_regs<kListLds / NTH>(list_lds, L, cnt, t1, above1, sl.hist, sl.scan, sl.res, emit);
      } else {
        // too many candidates for LDS: read them in place, span found by binary search
        auto at = [&](int i) {
          int lo = 0, hi = nsp - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sl.span_pre[mid] <= i) lo = mid;
            else hi = mid - 1;
          }
          return rslot[(int64_t)lo * kSelectSpan + (i - sl.span_pre[lo])];
        };
        refine_and_emit(at, L, cnt, t1, above1, sl.hist, sl.scan, sl.res, emit);
      }
      if (writer) {
        for (int i = cnt + threadIdx.x; i < a.k; i += blockDim.x) orow[i] = -1;
        if (threadIdx.x == 0) a.count_out[r] = cnt;
      }
    }
    __syncthreads();  // the ids are complete, and the list in the tile buffers is read no more
  }
  auto sel_id = [&](int key) {  // token id at selection position key of this split (SELECT)
    if constexpr (SELECT) {
      const int p = key - kbeg;
      return (p >= 0 && p < nk) ? sl.ids[p] : 0;
    } else {
      return key;
    }
  };
  // loader mapping: thread -> one 16-byte chunk of head_dim of keys 4 (ld_key4 % 16) + i (i < 4)
  // of the tiles ld_key4 / 16 + TPP * t (t < kAttnTiles / TPP)
  const int ltid = PAIR ? (int)threadIdx.x % LT : (int)threadIdx.x;  // loader thread of this head
  const int ld_chunk = ltid & 15;
  const int ld_key4 = ltid >> 4;  // 0 .. 16 TPP - 1
  auto piece_key = [&](int p) {           // stage-relative key of load piece p (< LPT)
    return ((ld_key4 >> 4) + TPP * (p >> 2)) * kAttnTile + (ld_key4 & 15) * 4 + (p & 3);
  };
  // the next stage's K and V pieces of this thread, in flight while the current stage is computed
  uint4 rk[LPT], rv[LPT];
  // Keys past the end of this split are clamped to its last key: the load stays inside the
  // selection (a finite row that is part of this attention anyway) and the key is masked out
  // of the softmax, so no load needs a branch.
  const int klast = kend - 1;
  auto load_ids = [&](int kt, int (&ids)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int key = kt + piece_key(i);
      ids[i] = key < klast ? key : klast;
      if (SELECT) ids[i] = sel_id(ids[i]);
      else if (FROM_CACHE) ids[i] = irow[ids[i]];  // clamped when used, so the load is not waited for here
    }
  };
  // 64-bit base of this (row, KV head) once, and 64-bit row offsets: a row may see 2^24 tokens of
  // hkv * 128 elements
  const int row_elems = FROM_CACHE ? a.hkv * CLSA_HEAD_DIM : CLSA_HEAD_DIM;
  const int64_t base_off = FROM_CACHE ? (tok_base * a.hkv + g) * CLSA_HEAD_DIM
                                      : (((int64_t)r * a.hkv + g) * a.k) * CLSA_HEAD_DIM;
  const uint16_t* kbase = a.ksrc + base_off + ld_chunk * 8;
  const uint16_t* vbase = a.vsrc + base_off + ld_chunk * 8;
  auto load_stage = [&](const int (&ids)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int64_t off = (int64_t)(FROM_CACHE ? tok(ids[i]) : ids[i]) * row_elems;
      rk[i] = load16(kbase + off);
      rv[i] = load16(vbase + off);
    }
  };
  // Per-lane byte offsets into a tile (swizzled layout), fixed for the whole kernel; the parts that
  // depend on the loop variables are compile-time immediates.
  //   row stores: piece p -> its tile and row, chunk ld_chunk
  //   K fragment: row mt*16 + l16, chunk 4kk + grp  -> slot (grp ^ l16) ^ 4kk
  //   V^T fragment (transposed read): row 32kk + 4grp + l16/4 (+16), head_dim 16ht + 4(l16 % 4)
  //     -> slot (2ht + (l16/2 % 2)) ^ (4grp + l16/4) = z ^ 2ht, byte 8 (l16 % 2) inside the chunk
  char* const lds_bytes = reinterpret_cast<char*>(lds) + (PAIR ? team * HEAD_LDS * 2 : 0);  // this head's tiles
  int soff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int key = piece_key(i);
    const int row = key & (kAttnTile - 1);
    soff[i] = (key / kAttnTile) * TILE_ELEMS * 2 + row * 256 + ((ld_chunk ^ (row & 15)) << 4);
  }
  // fragment offsets inside tile 0; tile t adds t * TILE_ELEMS * 2 bytes
  int koff[4];
  const int gx = grp ^ l16;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = l16 * 256 + ((gx ^ (4 * kk)) << 4);
  int voff[8];
  {
    const int y = 4 * grp + (l16 >> 2);
    const int z = ((l16 >> 1) & 1) ^ y;
#pragma unroll
    for (int ht = 0; ht < 8; ++ht) voff[ht] = kAttnTiles * TILE_ELEMS * 2 + y * 256 + ((z ^ (2 * ht)) << 4) + 8 * (l16 & 1);
  }
  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      *reinterpret_cast<uint4*>(lds_bytes + soff[i]) = rk[i];
      *reinterpret_cast<uint4*>(lds_bytes + kAttnTiles * TILE_ELEMS * 2 + soff[i]) = rv[i];
    }
  };
  const float scale = a.scale_log2;
  // One tile of the stage: S^T = K Q^T, online softmax in the exp2 domain, O^T += V^T P^T.
  // The running max m_run is only raised when some score of the wave exceeds it by more than
  // 2^kRescaleLog2; until then P = 2^(s - m_run) <= 2^kRescaleLog2 is used as is.  Numerator and
  // denominator share the same m_run, so the result does not depend on when it is raised, and the
  // common case needs neither a cross-lane reduction nor a rescale of acc.
  auto compute_tile = [&](int tile, int nvalid) {
    const char* tb = lds_bytes + tile * TILE_ELEMS * 2;  // this tile's K; its V sits at voff + tb
    floatx4_t s[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      floatx4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 av = *reinterpret_cast<const uint4*>(tb + koff[kk] + mt * 4096);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(av), qf[kk], c, 0, 0, 0);
      }
      s[mt] = c;
    }
    // s[mt][j]: raw q.k of key 16mt + 4grp + j of the tile, query column l16
    if (nvalid < kAttnTile) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (mt * 16 + grp * 4 + j >= nvalid) s[mt][j] = -INFINITY;
    }
    // the NaN-propagating maximum: three operands per instruction and no canonicalisation of the
    // MFMA results, which fmaxf's IEEE maxNum needs on each input (the scores are finite or -inf,
    // so both give the same value)
    auto max3 = [](float x, float y, float z) {
      return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
    };
    float mx = max3(max3(s[0][0], s[0][1], s[0][2]), max3(s[0][3], s[1][0], s[1][1]), max3(s[1][2], s[1][3], s[2][0]));
    mx = max3(mx, max3(s[2][1], s[2][2], s[2][3]), max3(s[3][0], s[3][1], s[3][2]));
    mx = __builtin_elementwise_maximum(mx, s[3][3]);
    if (__any(mx * scale > m_run + kRescaleLog2)) {
      mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 16, 64));
      mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32, 64));
      const float m_new = __builtin_elementwise_maximum(m_run, mx * scale);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= corr;
    }
    // P^T operand of k-step kk (keys 32kk .. 32kk + 31): slots 0..3 <- keys 32kk + 4grp + j,
    // slots 4..7 <- keys 32kk + 16 + 4grp + j
    bf16x8_t pb[2];
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = __builtin_amdgcn_exp2f(fmaf(s[2 * kk + h][j], scale, -m_run));
          psum += p[j];
        }
        w[2 * h] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)p[0], (__bf16)p[1]});
        w[2 * h + 1] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)p[2], (__bf16)p[3]});
      }
      pb[kk] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    }
    l_run += psum;
#pragma unroll
    for (int ht = 0; ht < 8; ++ht) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const char* vb = tb + voff[ht] + kk * 8192;
        const uint2 v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(vb));
        const uint2 v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(vb + 4096));
        acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(make_uint4(v0.x, v0.y, v1.x, v1.y)),
                                                          pb[kk], acc[ht], 0, 0, 0);
      }
    }
  };

  // Stage 0 is requested before the selection count has arrived: its keys are clamped into the
  // index row, and padding entries (-1, past the count) are replaced by the split's first entry,
  // which is selected whenever the split is not empty; when it is padding too (empty split,
  // nothing is computed) token 0 of the row is read.  Only keys below the count reach the
  // softmax, so the replaced rows never contribute.
  if constexpr (SELECT) {
    int ids0[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int key = kbeg + piece_key(i);
      ids0[i] = tok(sel_id(key < klast ? key : klast));
    }
    load_stage(ids0);
  } else {
    int ids0[LPT];
    const int kfirst = kbeg < a.k - 1 ? kbeg : a.k - 1;
    const int id_first = FROM_CACHE ? irow[kfirst] : 0;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      int key = kbeg + piece_key(i);
      key = key < a.k - 1 ? key : a.k - 1;
      if (FROM_CACHE) {
        int id = irow[key];
        id = id >= 0 ? id : id_first;
        key = tok(id);
      }
      ids0[i] = key;
    }
    load_stage(ids0);
  }
  // the next stage's rows are requested before this stage is computed
  int ids_next[LPT];
  if (kbeg < kend) load_ids(kbeg + STAGE, ids_next);
  // inside the loop kend > kbeg, so every clamped key lies in [kbeg, kend); after the last
  // stage the request for the "next" one re-reads the split's last row and is not used
  for (int kt = kbeg; kt < kend; kt += STAGE) {
    store_stage();
    __syncthreads();
    load_stage(ids_next);
    load_ids(kt + 2 * STAGE, ids_next);
    if (wave_active) {
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const int tile = PAIR ? t : team + TEAMS * t;
        const int nvalid = kend - (kt + tile * kAttnTile);  // keys of this tile
        if (nvalid > 0) compute_tile(tile, nvalid < kAttnTile ? nvalid : kAttnTile);
      }
    }
    __syncthreads();
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // Merge team 1 into team 0 through LDS (the tiles are free after the loop's last barrier):
  // per wave [acc: 8 ht x 4 j x 64 lanes][m: 64][l: 64], fp32.
  float* xch = reinterpret_cast<float*>(lds) + tw * kAttnPartWave;
  static_assert(WPT * kAttnPartWave * 4 <= (int)sizeof(lds), "team exchange fits the tiles");
  if (TEAMS == 2 && !PAIR && team == 1 && wave_active) {
#pragma unroll
    for (int ht = 0; ht < 8; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j) xch[(ht * 4 + j) * 64 + lane] = acc[ht][j];
    xch[32 * 64 + lane] = m_run;
    xch[33 * 64 + lane] = l_run;
  }
  if (TEAMS == 2 && !PAIR) __syncthreads();
  if (TEAMS == 2 && !PAIR && team == 0 && wave_active) {
    const float m1 = xch[32 * 64 + lane], l1 = xch[33 * 64 + lane];
    const float M = fmaxf(m_run, m1);
    if (M != -INFINITY) {  // both -inf: no keys in this split
      const float c0 = __builtin_amdgcn_exp2f(m_run - M), c1 = __builtin_amdgcn_exp2f(m1 - M);
      l_run = l_run * c0 + l1 * c1;
#pragma unroll
      for (int ht = 0; ht < 8; ++ht)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[ht][j] = acc[ht][j] * c0 + xch[(ht * 4 + j) * 64 + lane] * c1;
      m_run = M;
    }
  }
  // acc[ht][j]: head_dim ht*16 + grp*4 + j of this lane's query (team 0 holds the workgroup's result)
  uint16_t* op = a.out + (int64_t)r * a.o_stride + ((int64_t)layer * a.hq + head) * CLSA_HEAD_DIM;
  if (a.splits == 1) {
    if ((!PAIR && team != 0) || !q_valid) return;  // paired teams each hold their own head's result
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int ht = 0; ht < 8; ++ht) store_out4(op + ht * 16 + grp * 4, acc[ht], inv);
    return;
  }
  // Split partial of this workgroup, in the lanes' own layout (each store instruction of a wave
  // covers 256 contiguous bytes).  The last split of this (row, KV head, query block) to arrive
  // recombines them.
  const int64_t wg_rec = (((int64_t)r * a.hkv + g) * a.qblocks + qb) * kAttnPartWG;
  const int64_t split_stride = (int64_t)a.rw.n_rows * a.hkv * a.qblocks * kAttnPartWG;
  float* pw = a.part + wg_rec + tw * kAttnPartWave;
  if (team == 0) {
    float* pp = pw + split * split_stride;
#pragma unroll
    for (int ht = 0; ht < 8; ++ht)
#pragma unroll
      for (int j = 0; j < 4; ++j) st_dev(pp + (ht * 4 + j) * 64 + lane, acc[ht][j]);
    st_dev(pp + 32 * 64 + lane, m_run);
    st_dev(pp + 33 * 64 + lane, l_run);
  }
  uint32_t* ticket = a.tickets + ((int64_t)r * a.hkv + g) * a.qblocks + qb;
  if (!arrive_last(ticket, (uint32_t)a.splits, flag)) return;
  if (team != 0 || !q_valid) return;
  // Recombine the splits in split order, so that whichever workgroup arrives last computes
  // exactly the same result: a running (M, den, tot) absorbs split s as
  //   M' = max(M, m_s),  tot' = 2^(M - M') tot + 2^(m_s - M') acc_s,  den' likewise with l_s.
  // The partials of up to kCombineBatch splits are requested together (one round trip per batch).
  float M = -INFINITY, den = 0.f;
  float tot[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) tot[i] = 0.f;
  for (int s0 = 0; s0 < a.splits; s0 += kCombineBatch) {
    float mb[kCombineBatch], lb[kCombineBatch], vb[kCombineBatch][32];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int s2 = s0 + b;
      if (s2 >= a.splits || s2 == split) continue;
      const float* ps = pw + s2 * split_stride;
#pragma unroll
      for (int i = 0; i < 32; ++i) vb[b][i] = ld_dev(ps + i * 64 + lane);
      mb[b] = ld_dev(ps + 32 * 64 + lane);
      lb[b] = ld_dev(ps + 33 * 64 + lane);
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int s2 = s0 + b;
      if (s2 >= a.splits) break;
      if (s2 == split) {
        mb[b] = m_run;
        lb[b] = l_run;
#pragma unroll
        for (int ht = 0; ht < 8; ++ht)
#pragma unroll
          for (int j = 0; j < 4; ++j) vb[b][ht * 4 + j] = acc[ht][j];
      }
      if (mb[b] == -INFINITY) continue;  // a split with no keys
      const float m_new = fmaxf(M, mb[b]);
      const float c_old = __builtin_amdgcn_exp2f(M - m_new);
      const float c_new = __builtin_amdgcn_exp2f(mb[b] - m_new);
      M = m_new;
      den = den * c_old + lb[b] * c_new;
#pragma unroll
      for (int i = 0; i < 32; ++i) tot[i] = tot[i] * c_old + vb[b][i] * c_new;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int ht = 0; ht < 8; ++ht) {
    const floatx4_t o = {tot[ht * 4], tot[ht * 4 + 1], tot[ht * 4 + 2], tot[ht * 4 + 3]};
    store_out4(op + ht * 16 + grp * 4, o, inv);
  }
}

// ---------------------------------------------------------------------------- prefill rows
// Prefill attention: every query row (position) has its own selection, so its K/V rows are
// gathered for it alone and never reused by another row.  One workgroup = (row r, KV head g, block
// of up to 32 query rows, i.e. (layer, head) pairs of g's GQA group).  Its four waves take
// interleaved 32-key tiles of the row's selection, and each wave computes all 32 query columns of
// its tile: two 16-column MFMA blocks share every K and V fragment, which halves the LDS reads per
// MFMA against one 16-column block per wave.  A wave loads its tile's K and V rows (16 lanes per
// 256-byte row, so every quarter-wave reads whole rows) into LDS buffers of its own, so the waves
// never wait for each other inside the loop; the next tile's rows are in flight while a tile is
// computed.  The four waves' (m, l, acc) are merged in LDS at the end, in wave order.
constexpr int kPfaKeys = 32;     // keys per tile
constexpr int kPfaWaves = 4;
constexpr int kPfaCols = 32;     // query columns per workgroup (and per wave)
constexpr int kPfaPart = 68;     // floats per lane of a wave's merge record: acc 2 x 8 x 4, m 2, l 2
constexpr int kPfaIds = 2048;    // selection positions whose token ids sit in LDS at a time
constexpr int kPfaTileBytes = kPfaKeys * CLSA_HEAD_DIM * 2;  // one tile of K (or V)
constexpr int kPfaWaveBytes = 2 * kPfaTileBytes;             // a wave's K and V tiles
constexpr int kPfaLds = (kPfaWaves - 1) * kPfaPart * 64 * 4 > kPfaWaves * kPfaWaveBytes
                            ? (kPfaWaves - 1) * kPfaPart * 64 * 4
                            : kPfaWaves * kPfaWaveBytes;
// Buffer resource word 3 for plain (unformatted) dword loads on gfx9-family chips.
constexpr int kBufferWord3 = 0x00020000;

// Token ids of the row's selection are staged in LDS, kPfaIds positions at a time, already
// clamped into the row's tokens (and positions past the count set to token 0, a valid row that the
// softmax masks), so the loop reads 8 ids with two LDS reads and forms each row address with one
// 24-bit multiply-add.  BUF: the rows are read with buffer loads, whose 32-bit byte offset from
// the (sequence, KV head) base covers every visible row (checked at launch); otherwise with 64-bit
// global addresses.
template <bool BUF>
__global__ __launch_bounds__(64 * kPfaWaves, 2) void k_prefill_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kPfaLds];
  __shared__ __attribute__((aligned(16))) int ids[kPfaIds];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int qb = blockIdx.x % a.qblocks;
  const int g = blockIdx.x / a.qblocks;
  const int r = blockIdx.y;
  int kbeg, cnt;  // the row's selection positions 0 .. cnt - 1 (count clamped into [0, k])
  split_key_range(a.count[r], a.k, 0, a.k, &kbeg, &cnt);

  // query columns 16 cb + l16 of the block -> (layer, head)
  bf16x8_t qf[2][4];
  int layer[2], head[2];
  bool qvalid[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int qr = qb * kPfaCols + cb * 16 + l16;
    qvalid[cb] = qr < a.qrows;
    layer[cb] = qvalid[cb] ? qr / a.group : 0;
    head[cb] = g * a.group + (qvalid[cb] ? qr % a.group : 0);
    const uint16_t* qp = a.q + (int64_t)r * a.q_stride + ((int64_t)layer[cb] * a.hq + head[cb]) * CLSA_HEAD_DIM;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (qvalid[cb]) v = load16(qp + kk * 32 + grp * 8);
      qf[cb][kk] = bitcast<bf16x8_t>(v);
    }
  }

  const int seq = row_seq(a.rw, r);
  const int64_t tok_base = (int64_t)a.rw.cu[seq];
  const int tok_last = max(row_len(a.rw, r) - 1, 0);
  const int32_t* irow = a.idx + (int64_t)r * a.k;
  const int row_elems = a.hkv * CLSA_HEAD_DIM;
  const uint32_t row_bytes = (uint32_t)row_elems * 2u;
  // the (sequence, KV head) base; the lane reads 16-byte chunk l16 of every row it loads
  const int64_t base_el = (tok_base * a.hkv + g) * CLSA_HEAD_DIM;
  const uint16_t* kbase = a.ksrc + base_el;
  const uint16_t* vbase = a.vsrc + base_el;
  const uint32_t lane_off = (uint32_t)l16 * 16u;
  __amdgpu_buffer_rsrc_t rk, rv;
  if constexpr (BUF) {
    const int nrec = (int)((uint32_t)tok_last * row_bytes + 256u);  // bytes up to the last visible row
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nrec, kBufferWord3);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nrec, kBufferWord3);
  }
  // the lane loads chunk l16 of tile keys 8 grp + i (i < 8)
  uint4 kr[8], vr[8];
  auto load_tile = [&](int tile) {
    const int4 i0 = *reinterpret_cast<const int4*>(&ids[tile * kPfaKeys + grp * 8]);
    const int4 i1 = *reinterpret_cast<const int4*>(&ids[tile * kPfaKeys + grp * 8 + 4]);
    const int id[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (BUF) {
        // exact in 24 bits: the launch keeps row_bytes below 2^24 and max_row_len * row_bytes
        // below 2^31, so the id is below 2^23 and the product below 2^31
        const uint32_t off = __umul24((uint32_t)id[i], row_bytes) + lane_off;
        kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
        vr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
      } else {
        const int64_t off = (int64_t)id[i] * row_elems + l16 * 8;
        kr[i] = load16(kbase + off);
        vr[i] = load16(vbase + off);
      }
    }
  };

  // this wave's tiles: key row kr, 16-byte chunk c at slot c ^ (kr & 15) (see the tile layout above)
  char* const kbuf = lds + wave * kPfaWaveBytes;
  char* const vbuf = kbuf + kPfaTileBytes;
  int soff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = grp * 8 + i;
    soff[i] = key * 256 + ((l16 ^ (key & 15)) << 4);
  }
  // K fragment (mt, kk): key 16 mt + l16, chunk 4 kk + grp; mt adds 16 rows = 4096 bytes
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = l16 * 256 + ((((kk * 4) + grp) ^ l16) << 4);
  int voff[8];
  {
    const int y = 4 * grp + (l16 >> 2);
    const int z = ((l16 >> 1) & 1) ^ y;
#pragma unroll
    for (int ht = 0; ht < 8; ++ht) voff[ht] = y * 256 + ((z ^ (2 * ht)) << 4) + 8 * (l16 & 1);
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  floatx4_t acc[2][8];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[cb][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const float scale = a.scale_log2;

  for (int c0 = 0; c0 < cnt; c0 += kPfaIds) {
    const int clen = min(kPfaIds, cnt - c0);
    const int ctiles = (clen + kPfaKeys - 1) / kPfaKeys;
    if (c0 > 0) __syncthreads();  // every wave is done with the previous ids
    for (int i = threadIdx.x; i < ctiles * kPfaKeys; i += blockDim.x) {
      const int id = i < clen ? irow[c0 + i] : 0;
      ids[i] = id < 0 ? 0 : (id > tok_last ? tok_last : id);
    }
    __syncthreads();
    int t = wave;
    if (t < ctiles) load_tile(t);
    for (; t < ctiles; t += kPfaWaves) {
      // this tile's rows into the wave's buffers (the previous tile's reads have completed: their
      // values fed its MFMAs), then the next tile's loads
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<uint4*>(kbuf + soff[i]) = kr[i];
        *reinterpret_cast<uint4*>(vbuf + soff[i]) = vr[i];
      }
      if (t + kPfaWaves < ctiles) load_tile(t + kPfaWaves);
      // S^T = K Q^T: s[mt][cb][j] = q . k of key 16 mt + 4 grp + j, query column 16 cb + l16
      floatx4_t s[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        floatx4_t c0v = {0.f, 0.f, 0.f, 0.f}, c1v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8_t kfrag = bitcast<bf16x8_t>(*reinterpret_cast<const uint4*>(kbuf + koff[kk] + mt * 4096));
          c0v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qf[0][kk], c0v, 0, 0, 0);
          c1v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qf[1][kk], c1v, 0, 0, 0);
        }
        s[mt][0] = c0v;
        s[mt][1] = c1v;
      }
      const int nvalid = clen - t * kPfaKeys;
      if (nvalid < kPfaKeys) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (mt * 16 + grp * 4 + j >= nvalid) {
              s[mt][0][j] = -INFINITY;
              s[mt][1][j] = -INFINITY;
            }
      }
      // online softmax (exp2 domain) per query column, with the lazy rescale of the decode kernel;
      // P^T operand slots 0..3 <- keys 4 grp + j, slots 4..7 <- keys 16 + 4 grp + j.  The tile
      // maximum uses the NaN-propagating maximum (three operands per instruction; the scores are
      // finite or -inf).
      bf16x8_t pb[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float mx = __builtin_elementwise_maximum(s[0][cb][0], s[0][cb][1]);
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[0][cb][2], s[0][cb][3]));
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[1][cb][0], s[1][cb][1]));
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[1][cb][2], s[1][cb][3]));
        if (__any(mx * scale > m_run[cb] + kRescaleLog2)) {
          mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 16, 64));
          mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32, 64));
          const float m_new = fmaxf(m_run[cb], mx * scale);
          const float corr = __builtin_amdgcn_exp2f(m_run[cb] - m_new);
          m_run[cb] = m_new;
          l_run[cb] *= corr;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[cb][i] *= corr;
        }
        uint32_t w[4];
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          float p[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[j] = __builtin_amdgcn_exp2f(fmaf(s[mt][cb][j], scale, -m_run[cb]));
            psum += p[j];
          }
          w[2 * mt] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)p[0], (__bf16)p[1]});
          w[2 * mt + 1] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)p[2], (__bf16)p[3]});
        }
        l_run[cb] += psum;
        pb[cb] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
      // O^T += V^T P^T, one V^T fragment per 16 head dims shared by both column blocks
#pragma unroll
      for (int ht = 0; ht < 8; ++ht) {
        const uint2 v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(vbuf + voff[ht]));
        const uint2 v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(vbuf + voff[ht] + 4096));
        const bf16x8_t va = bitcast<bf16x8_t>(make_uint4(v0.x, v0.y, v1.x, v1.y));
        acc[0][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0], acc[0][ht], 0, 0, 0);
        acc[1][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[1], acc[1][ht], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    l_run[cb] += __shfl_xor(l_run[cb], 16, 64);
    l_run[cb] += __shfl_xor(l_run[cb], 32, 64);
  }
  // merge waves 1..3 into wave 0 through LDS (the tile buffers are free once every wave is past
  // its loop)
  __syncthreads();
  float* rec = reinterpret_cast<float*>(lds);
  if (wave > 0) {
    float* pw = rec + (wave - 1) * kPfaPart * 64;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int ht = 0; ht < 8; ++ht)
#pragma unroll
        for (int j = 0; j < 4; ++j) pw[((cb * 8 + ht) * 4 + j) * 64 + lane] = acc[cb][ht][j];
      pw[(64 + cb) * 64 + lane] = m_run[cb];
      pw[(66 + cb) * 64 + lane] = l_run[cb];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w2 = 1; w2 < kPfaWaves; ++w2) {
    const float* pw = rec + (w2 - 1) * kPfaPart * 64;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float m1 = pw[(64 + cb) * 64 + lane], l1 = pw[(66 + cb) * 64 + lane];
      const float M = fmaxf(m_run[cb], m1);
      if (M == -INFINITY) continue;  // neither has keys
      const float c0 = __builtin_amdgcn_exp2f(m_run[cb] - M), c1 = __builtin_amdgcn_exp2f(m1 - M);
      l_run[cb] = l_run[cb] * c0 + l1 * c1;
#pragma unroll
      for (int ht = 0; ht < 8; ++ht)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[cb][ht][j] = acc[cb][ht][j] * c0 + pw[((cb * 8 + ht) * 4 + j) * 64 + lane] * c1;
      m_run[cb] = M;
    }
  }
  // acc[cb][ht][j]: head dim 16 ht + 4 grp + j of query column 16 cb + l16
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    if (!qvalid[cb]) continue;
    uint16_t* op = a.out + (int64_t)r * a.o_stride + ((int64_t)layer[cb] * a.hq + head[cb]) * CLSA_HEAD_DIM;
    const float inv = l_run[cb] > 0.f ? 1.f / l_run[cb] : 0.f;
#pragma unroll
    for (int ht = 0; ht < 8; ++ht) store_out4(op + ht * 16 + grp * 4, acc[cb][ht], inv);
  }
}

__global__ void k_clear_u32(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Selector: k_sel[r, g, i, :] = k_cache[cu[seq] + idx[r, i], g, :] for i < count[r], zero after.
constexpr int kGatherTok = 16;
__global__ __launch_bounds__(256) void k_gather_kv(RowsDev rw, int k, int hkv, const uint16_t* __restrict__ kc,
                                                    const uint16_t* __restrict__ vc, const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ count, uint16_t* __restrict__ ksel,
                                                    uint16_t* __restrict__ vsel) {
  const int r = blockIdx.y;
  const int cnt = count[r];
  const int64_t base = rw.cu[row_seq(rw, r)];
  const int tok_last = max(row_len(rw, r) - 1, 0);
  const int per_tok = hkv * 16;  // 16-byte chunks per token
  const int total = kGatherTok * per_tok;
  for (int c = threadIdx.x; c < total; c += blockDim.x) {
    const int t = c / per_tok;
    const int rem = c - t * per_tok;
    const int g = rem >> 4, ch = rem & 15;
    const int i = blockIdx.x * kGatherTok + t;
    if (i >= k) continue;
    const int64_t dst = (((int64_t)r * hkv + g) * k + i) * CLSA_HEAD_DIM + ch * 8;
    uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
    if (i < cnt) {
      int id = idx[(int64_t)r * k + i];
      id = id < 0 ? 0 : (id > tok_last ? tok_last : id);  // stays inside the row's tokens
      const int64_t src = ((base + id) * hkv + g) * CLSA_HEAD_DIM + ch * 8;
      kv = *reinterpret_cast<const uint4*>(kc + src);
      vv = *reinterpret_cast<const uint4*>(vc + src);
    }
    *reinterpret_cast<uint4*>(ksel + dst) = kv;
    *reinterpret_cast<uint4*>(vsel + dst) = vv;
  }
}

}  // namespace

int launch_attn(const RowsDev& rows, int k, int hq, int hkv, int n_layers_call, float scale, const AttnPlan& plan,
                const uint16_t* q, int64_t q_stride, const uint16_t* ksel, const uint16_t* vsel, const uint16_t* kc,
                const uint16_t* vc, const int32_t* idx, const int32_t* count, uint16_t* out, int64_t o_stride,
                void* part, uint32_t* tickets, bool tickets_clear, void* stream, const SelectIn* sel,
                int32_t* idx_out, int32_t* count_out) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  AttnArgs a;
  a.rw = rows;
  a.k = k;
  a.hq = hq;
  a.hkv = hkv;
  a.lc = n_layers_call;
  a.group = plan.group;
  a.qrows = plan.qrows;
  a.qblocks = plan.qblocks;
  a.splits = plan.splits;
  a.kps = plan.keys_per_split;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.q = q;
  a.q_stride = q_stride;
  const bool from_cache = ksel == nullptr;
  a.ksrc = from_cache ? kc : ksel;
  a.vsrc = from_cache ? vc : vsel;
  a.idx = idx;
  a.count = count;
  a.out = out;
  a.o_stride = o_stride;
  a.part = static_cast<float*>(part);
  a.tickets = tickets;
  a.sel_slot = sel ? static_cast<const uint2*>(sel->slot) : nullptr;
  a.sel_cnt = sel ? sel->cnt : nullptr;
  a.sel_rowinfo = sel ? sel->rowinfo : nullptr;
  a.sel_spans = sel ? sel->spans : 0;
  a.idx_out = idx_out;
  a.count_out = count_out;
  const bool fused = sel != nullptr;
  if (rows.mode == CLSA_MODE_PREFILL && from_cache && !fused) {
    // prefill rows: each gathers its own selection; no key splits, no partials
    a.qblocks = (plan.qrows + kPfaCols - 1) / kPfaCols;
    const dim3 grid((unsigned)(a.qblocks * hkv), (unsigned)rows.n_rows);
    // buffer loads when a 32-bit byte offset reaches every visible row (device row lengths are
    // clamped to max_row_len) and the row stride fits the 24-bit multiply that forms it
    const int64_t row_bytes = (int64_t)hkv * CLSA_HEAD_DIM * 2;
    if ((int64_t)rows.max_row_len * row_bytes <= (int64_t)INT32_MAX && row_bytes < ((int64_t)1 << 24))
      hipLaunchKernelGGL(k_prefill_attn<true>, grid, dim3(64 * kPfaWaves), 0, s, a);
    else
      hipLaunchKernelGGL(k_prefill_attn<false>, grid, dim3(64 * kPfaWaves), 0, s, a);
    return (int)hipGetLastError();
  }
  if (fused && (plan.teams != 2 || plan.wpt != 4 || ksel != nullptr || plan.keys_per_split > kFusedMaxIds || idx_out == nullptr ||
                count_out == nullptr))
    return (int)hipErrorInvalidValue;
  if (plan.splits > 1 && !tickets_clear)
    hipLaunchKernelGGL(k_clear_u32, dim3((plan.tickets + 255) / 256), dim3(256), 0, s, tickets, plan.tickets);
  if (plan.pair && (plan.splits != 1 || plan.teams != 2 || plan.wpt != 4 || hkv % 2 != 0))
    return (int)hipErrorInvalidValue;
  const int gblocks = plan.pair ? hkv / 2 : hkv;
  const dim3 grid((unsigned)(plan.splits * plan.qblocks * gblocks), (unsigned)rows.n_rows);
  const dim3 block((unsigned)(64 * plan.wpt * plan.teams));
  if (plan.pair) {
    if (fused)
      hipLaunchKernelGGL((k_sparse_attn<true, 2, true, 4, true>), grid, block, 0, s, a);
    else if (from_cache)
      hipLaunchKernelGGL((k_sparse_attn<true, 2, false, 4, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_sparse_attn<false, 2, false, 4, true>), grid, block, 0, s, a);
  } else if (plan.teams == 2 && plan.wpt == 2) {
    if (fused) return (int)hipErrorInvalidValue;
    if (from_cache)
      hipLaunchKernelGGL((k_sparse_attn<true, 2, false, 2>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_sparse_attn<false, 2, false, 2>), grid, block, 0, s, a);
  } else if (plan.teams == 2) {
    if (fused)
      hipLaunchKernelGGL((k_sparse_attn<true, 2, true>), grid, block, 0, s, a);
    else if (from_cache)
      hipLaunchKernelGGL((k_sparse_attn<true, 2>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_sparse_attn<false, 2>), grid, block, 0, s, a);
  } else {
    if (from_cache)
      hipLaunchKernelGGL((k_sparse_attn<true, 1>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_sparse_attn<false, 1>), grid, block, 0, s, a);
  }
  return (int)hipGetLastError();
}

int launch_gather(const RowsDev& rows, int k, int hkv, const uint16_t* kc, const uint16_t* vc, const int32_t* idx,
                  const int32_t* count, uint16_t* ks, uint16_t* vs, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((k + kGatherTok - 1) / kGatherTok), (unsigned)rows.n_rows);
  hipLaunchKernelGGL(k_gather_kv, grid, dim3(256), 0, s, rows, k, hkv, kc, vc, idx, count, ks, vs);
  return (int)hipGetLastError();
}

}  // namespace clsa
