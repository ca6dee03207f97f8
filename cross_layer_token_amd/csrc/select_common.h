// The steps of the long-row top-k select (TopK(I_t, k) of eq. 2 in the picx.dev summary of
// "You Only Index Once", Methodology > Architecture Overview) that more than one kernel runs:
// the histogram partials (score kernel, select), and the finish over the candidates (the
// select's finishing kernel, and the attention workgroups that finish the selection themselves).
//
// The candidates of a row are the (key, token) pairs whose first-level bin is at or above the bin
// t1 holding the m-th largest key.  Span s of the row (kSelectSpan scores) holds cnt[s] of them
// at slot + s * kSelectSpan, in token order, so the spans concatenated in order are in token
// order too.  The m-th largest key T is refined with 8-bit radix passes over the candidates;
// then every key above T is taken, and the lowest-token ties at T until m are taken.
#pragma once

#include "device_common.h"

namespace clsa {

constexpr int kListLds = 8192;   // (key, token) pairs a finishing workgroup keeps in LDS
constexpr int kCopyBatch = 8;    // list loads each lane keeps in flight
constexpr int kSpecPerLane = 4;  // span entries each lane requests before the span counts arrive

// One radix pass over 8 key bits: histogram of the keys that match the prefix found so far, then
// the bin holding the need-th largest.  Ends with __syncthreads().
template <typename KeyAt>
__device__ __forceinline__ void radix_pass8(uint32_t* hist, int count, KeyAt key_at, uint32_t& prefix,
                                            uint32_t& pmask, int shift, int& need, int* res) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < count; i += blockDim.x) {
    const uint32_t key = key_at(i);
    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  find_bin256_from_top(hist, need, res);
  prefix |= (uint32_t)res[0] << shift;
  pmask |= 255u << shift;
  need -= res[1];
}

// ---- windowed histogram partials ------------------------------------------------------------
// A chunk of at least m keys can bound the row's first-level bin t1 (the bin of the row's m-th
// largest key) from below by the bin lo of its own m-th largest key, since the row's m-th largest
// is at least the chunk's.  So the chunk publishes its histogram only from lo up, kHistWin bins,
// when its top bin lies inside that window; otherwise (or with fewer than m keys) it publishes
// all kTopkBins bins.  Summing every chunk's partial as it stands gives exact counts for every bin
// at or above the largest lo, t1 among them, which is all the top-down search for t1 reads.
// Layout per chunk: kTopkBins / 2 words (bins 2i and 2i + 1 in the halves of word i; a window
// uses the first kHistWin / 2 words, bins lo + 2i and lo + 2i + 1), and one info word lo | full.
constexpr int kHistWin = 128;
constexpr uint32_t kHistFull = 1u << 31;

// Two searches of find_bin_from_top_block in one scan: res[0], res[1] for need0 and res[2],
// res[3] for need1 (1 <= need <= the histogram's total).  Ends with __syncthreads().
template <int NT>
__device__ void find_two_bins_from_top_block(const uint32_t* hist, int need0, int need1, int* scan, int* res) {
  static_assert(kTopkBins % NT == 0, "whole bins per thread");
  constexpr int B = kTopkBins / NT;
  const int hi = kTopkBins - 1 - B * (int)threadIdx.x;
  int h[B], loc = 0;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    h[j] = (int)hist[hi - j];
    loc += h[j];
  }
  int total;
  int run = block_exclusive_scan(loc, scan, &total);
#pragma unroll
  for (int j = 0; j < B; ++j) {
    if (run < need0 && run + h[j] >= need0) {
      res[0] = hi - j;
      res[1] = run;
    }
    if (run < need1 && run + h[j] >= need1) {
      res[2] = hi - j;
      res[3] = run;
    }
    run += h[j];
  }
  __syncthreads();
}

// Writes a chunk's partial from its complete LDS histogram of len keys (NT threads, all calling).
template <int NT>
__device__ void write_hist_partial(const uint32_t* hist, int len, int m, uint32_t* hp, uint32_t* info, int* scan,
                                   int* res) {
  int lo = 0;
  bool full = true;
  if (m >= 1 && len >= m) {
    find_two_bins_from_top_block<NT>(hist, 1, m, scan, res);
    lo = res[2];
    full = res[0] - lo >= kHistWin;
  }
  if (full) {
    for (int i = threadIdx.x; i < kTopkBins / 2; i += NT) hp[i] = hist[2 * i] | (hist[2 * i + 1] << 16);
  } else {
    for (int i = threadIdx.x; i < kHistWin / 2; i += NT) {
      const int b = lo + 2 * i;
      const uint32_t h0 = b < kTopkBins ? hist[b] : 0u, h1 = b + 1 < kTopkBins ? hist[b + 1] : 0u;
      hp[i] = h0 | (h1 << 16);
    }
  }
  if (threadIdx.x == 0) *info = (uint32_t)lo | (full ? kHistFull : 0u);
}

// Sums the row's chunk partials into the LDS histogram hist (NT threads; nch chunks, the partial
// of chunk c at hp + c * kTopkBins / 2).  Windows: window words and info words are requested
// kSumBatch chunk groups at a time, added with LDS atomics, and hist is cleared while the first
// batch is in flight.  Full partials (pieces shorter than k) are summed in a second pass, only when
// there are any: thread t owns word t (bins 2t and 2t + 1) of every partial and adds it over all
// full partials in registers, with kFullBatch chunks' words in flight at a time, then adds the two
// sums to hist.  Ends with __syncthreads().
template <int NT>
__device__ void sum_hist_partials(const uint32_t* hp, const uint32_t* info, int nch, uint32_t* hist, int* any_full) {
  constexpr int kWords = kHistWin / 2;
  constexpr int kGroup = NT / kWords;  // chunks per pass
  constexpr int kSumBatch = 8;
  constexpr int kFullBatch = 16;
  const int w = threadIdx.x % kWords, cg = threadIdx.x / kWords;
  if (threadIdx.x == 0) *any_full = 0;
  bool cleared = false, full_seen = false;
  for (int cb = 0; cb < nch; cb += kGroup * kSumBatch) {
    uint32_t iv[kSumBatch], wv[kSumBatch];
#pragma unroll
    for (int p = 0; p < kSumBatch; ++p) {
      const int c = cb + p * kGroup + cg;
      iv[p] = c < nch ? info[c] : 0u;
      wv[p] = c < nch ? hp[(int64_t)c * (kTopkBins / 2) + w] : 0u;
    }
    if (!cleared) {
      for (int i = threadIdx.x; i < kTopkBins; i += NT) hist[i] = 0u;
      __syncthreads();
      cleared = true;
    }
#pragma unroll
    for (int p = 0; p < kSumBatch; ++p) {
      const int c = cb + p * kGroup + cg;
      if (c >= nch) continue;
      if (iv[p] & kHistFull) {
        full_seen = true;
      } else {
        const int b = (int)(iv[p] & (kTopkBins - 1)) + 2 * w;
        if ((wv[p] & 0xFFFFu) && b < kTopkBins) atomicAdd(&hist[b], wv[p] & 0xFFFFu);
        if ((wv[p] >> 16) && b + 1 < kTopkBins) atomicAdd(&hist[b + 1], wv[p] >> 16);
      }
    }
  }
  if (!cleared)
    for (int i = threadIdx.x; i < kTopkBins; i += NT) hist[i] = 0u;
  if (full_seen) *any_full = 1;
  __syncthreads();
  if (*any_full == 0) return;
  for (int t = threadIdx.x; t < kTopkBins / 2; t += NT) {
    uint32_t lo = 0u, hi = 0u;
    for (int c0 = 0; c0 < nch; c0 += kFullBatch) {
      uint32_t iv[kFullBatch], v[kFullBatch];
      // unconditional loads of a clamped chunk (predicated loads would each get their own wait),
      // masked when added
#pragma unroll
      for (int j = 0; j < kFullBatch; ++j) {
        const int c = c0 + j < nch ? c0 + j : nch - 1;
        iv[j] = info[c];
        v[j] = hp[(int64_t)c * (kTopkBins / 2) + t];  // inside the partial whatever its kind
      }
#pragma unroll
      for (int j = 0; j < kFullBatch; ++j) {
        const bool take = c0 + j < nch && (iv[j] & kHistFull);
        lo += take ? (v[j] & 0xFFFFu) : 0u;
        hi += take ? (v[j] >> 16) : 0u;
      }
    }
    if (lo) atomicAdd(&hist[2 * t], lo);
    if (hi) atomicAdd(&hist[2 * t + 1], hi);
  }
  __syncthreads();
}

// Candidate collection, in two halves so that its loads can be issued before the row length is
// known.  request_candidates loads the span counts of this thread (spans tid * SPT .. + SPT - 1)
// and the first kSpecPerLane * 64 entries of the first NSPEC spans of every wave, bounded by
// span_bound spans and len_bound entries (the buffers' extents, or the row's own).
// complete_candidates then gathers the counts of the row's nsp spans into span_pre[0..nsp]
// (prefix counts, span_pre[nsp] = L) and returns L.  When L <= kListLds the span lists are
// concatenated into list_lds, otherwise into list_global when it is given; with neither the lists
// stay in the spans.  The spans come from an earlier kernel, so plain loads see them.
// complete_candidates ends with __syncthreads().
template <int NT, int NSPEC, int kMaxSpansSel>
struct CandidateLoads {
  static_assert(kMaxSpansSel % NT == 0, "whole spans per thread");
  static constexpr int SPT = kMaxSpansSel / NT;  // span counts per thread
  uint64_t spec[NSPEC][kSpecPerLane];
  uint32_t c[SPT];
};

__device__ __forceinline__ uint64_t load_entry(const uint2* p) { return *reinterpret_cast<const uint64_t*>(p); }

template <int NT, int NSPEC, int kMaxSpansSel>
__device__ __forceinline__ void request_candidates(CandidateLoads<NT, NSPEC, kMaxSpansSel>& q, const uint2* slot,
                                                   const uint32_t* cnt, int span_bound, int len_bound) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < NSPEC; ++u) {
    const int sp = wave + u * kWaves;
#pragma unroll
    for (int j = 0; j < kSpecPerLane; ++j) {
      const int e = sp * kSelectSpan + j * 64 + lane;
      q.spec[u][j] = (sp < span_bound && e < len_bound) ? load_entry(slot + e) : 0;
    }
  }
#pragma unroll
  for (int i = 0; i < q.SPT; ++i) {
    const int sp = threadIdx.x * q.SPT + i;
    q.c[i] = sp < span_bound ? cnt[sp] : 0u;
  }
}

template <int NT, int NSPEC, int kMaxSpansSel>
__device__ int complete_candidates(const CandidateLoads<NT, NSPEC, kMaxSpansSel>& q, const uint2* slot, int nsp,
                                   int* span_pre, int* scan, uint2* list_lds, uint2* list_global) {
  constexpr int kWaves = NT / 64;
  constexpr int SPT = kMaxSpansSel / NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int L = 0;
  {
    int c[SPT], mine = 0;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int sp = threadIdx.x * SPT + i;
      c[i] = sp < nsp ? (int)q.c[i] : 0;  // counts past the row's spans are not the row's
      mine += c[i];
    }
    int pre = block_exclusive_scan(mine, scan, &L);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int sp = threadIdx.x * SPT + i;
      if (sp < nsp) span_pre[sp] = pre;
      pre += c[i];
    }
    if (threadIdx.x == 0) span_pre[nsp] = L;
    __syncthreads();
  }
  uint2* list = L <= kListLds ? list_lds : list_global;
  if (list == nullptr) return L;
  for (int sp2 = wave, u = 0; sp2 < nsp; sp2 += kWaves, ++u) {
    const int base = span_pre[sp2], cnt_s = span_pre[sp2 + 1] - base;
    const uint2* src = slot + (int64_t)sp2 * kSelectSpan;
    int e0 = 0;
    if (u < NSPEC) {
#pragma unroll
      for (int uu = 0; uu < NSPEC; ++uu) {
        if (uu != u) continue;
#pragma unroll
        for (int j = 0; j < kSpecPerLane; ++j) {
          const int e = j * 64 + lane;
          if (e < cnt_s) list[base + e] = make_uint2((uint32_t)q.spec[uu][j], (uint32_t)(q.spec[uu][j] >> 32));
        }
      }
      e0 = kSpecPerLane * 64;
    }
    for (; e0 < cnt_s; e0 += kCopyBatch * 64) {
      uint64_t v[kCopyBatch];
#pragma unroll
      for (int j = 0; j < kCopyBatch; ++j) {
        const int e = e0 + j * 64 + lane;
        v[j] = e < cnt_s ? load_entry(src + e) : 0;
      }
#pragma unroll
      for (int j = 0; j < kCopyBatch; ++j) {
        const int e = e0 + j * 64 + lane;
        if (e < cnt_s) list[base + e] = make_uint2((uint32_t)v[j], (uint32_t)(v[j] >> 32));
      }
    }
  }
  __syncthreads();
  return L;
}

// Refines the m-th largest key T below the first level (bin t1, `above1` keys in higher bins)
// with 8-bit passes over the L candidates entry_at(0..L-1) (in token order), the last pass
// aligned to bit 0 (its window overlaps bits the prefix already fixes, which then match), and
// calls emit(position, token) for every selected candidate, position = its rank in token order
// among the selected (0 .. m-1).  Every thread calls this; it ends without a barrier after the
// emits.
template <typename EntryAt, typename Emit>
__device__ void refine_and_emit(EntryAt entry_at, int L, int m, uint32_t t1, int above1, uint32_t* hist, int* scan,
                                int* res, Emit emit) {
  int need = m - above1;
  uint32_t prefix = t1 << (32 - kTopkBinBits), pmask = ~0u << (32 - kTopkBinBits);
  auto key_at = [&](int i) { return entry_at(i).x; };
  for (int shift = 32 - kTopkBinBits - 8;; shift -= 8) {
    if (shift < 0) shift = 0;
    radix_pass8(hist, L, key_at, prefix, pmask, shift, need, res);
    if (shift == 0) break;
  }
  const uint32_t T = prefix;
  // ordered output over contiguous per-thread ranges of the candidates
  const int E = (L + (int)blockDim.x - 1) / (int)blockDim.x;
  const int p0 = threadIdx.x * E;
  int gt = 0, eq = 0;
  for (int j = 0; j < E; ++j) {
    const int p = p0 + j;
    if (p < L) {
      const uint32_t key = key_at(p);
      gt += key > T;
      eq += key == T;
    }
  }
  int gt_before, eq_before, tg, te;
  block_exclusive_scan2(gt, eq, scan, &gt_before, &eq_before, &tg, &te);
  for (int j = 0; j < E; ++j) {
    const int p = p0 + j;
    if (p < L) {
      const uint2 e = entry_at(p);
      const bool take = e.x > T || (e.x == T && eq_before < need);
      const int pos = gt_before + (eq_before < need ? eq_before : need);
      if (take && pos < m) emit(pos, (int32_t)e.y);
      gt_before += e.x > T;
      eq_before += e.x == T;
    }
  }
}

// refine_and_emit for a candidate list in LDS of at most blockDim.x * EMAX entries: each thread
// keeps its contiguous range of E = ceil(L / blockDim.x) entries in registers for all passes, and
// the 8-bit passes alternate between the two 256-bin halves of hist2 (one half is cleared while
// the other is searched), so a pass costs two barriers and no list reads.  Same selection, same
// positions.  Every thread calls this; it ends without a barrier after the emits.
template <int EMAX, typename Emit>
__device__ void refine_and_emit_regs(const uint2* list, int L, int m, uint32_t t1, int above1, uint32_t* hist2,
                                     int* scan, int* res, Emit emit) {
  const int E = (L + (int)blockDim.x - 1) / (int)blockDim.x;  // <= EMAX, checked by the caller
  const int p0 = threadIdx.x * E;
  uint32_t key[EMAX];
  int32_t tok[EMAX];
  bool ok[EMAX];
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    ok[j] = j < E && p0 + j < L;
    const uint2 e = ok[j] ? list[p0 + j] : make_uint2(0u, 0u);
    key[j] = e.x;
    tok[j] = (int32_t)e.y;
  }
  for (int i = threadIdx.x; i < 512; i += blockDim.x) hist2[i] = 0u;
  __syncthreads();
  int need = m - above1;
  uint32_t prefix = t1 << (32 - kTopkBinBits), pmask = ~0u << (32 - kTopkBinBits);
  int half = 0;
  for (int shift = 32 - kTopkBinBits - 8;; shift -= 8) {
    if (shift < 0) shift = 0;
    uint32_t* h = hist2 + 256 * half;
#pragma unroll
    for (int j = 0; j < EMAX; ++j)
      if (ok[j] && (key[j] & pmask) == prefix) atomicAdd(&h[(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    // the other half was last searched in the previous pass (finished by its barrier) and is next
    // counted into after this pass's barrier
    uint32_t* o = hist2 + 256 * (half ^ 1);
    for (int i = threadIdx.x; i < 256; i += blockDim.x) o[i] = 0u;
    find_bin256_from_top(h, need, res);
    prefix |= (uint32_t)res[0] << shift;
    pmask |= 255u << shift;
    need -= res[1];
    if (shift == 0) break;
    half ^= 1;
  }
  const uint32_t T = prefix;
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    gt += ok[j] && key[j] > T;
    eq += ok[j] && key[j] == T;
  }
  int gt_before, eq_before, tg, te;
  block_exclusive_scan2(gt, eq, scan, &gt_before, &eq_before, &tg, &te);
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    if (ok[j]) {
      const bool take = key[j] > T || (key[j] == T && eq_before < need);
      const int pos = gt_before + (eq_before < need ? eq_before : need);
      if (take && pos < m) emit(pos, tok[j]);
      gt_before += key[j] > T;
      eq_before += key[j] == T;
    }
  }
}

}  // namespace clsa
