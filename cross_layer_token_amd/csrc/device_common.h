// Device helpers shared by the CLSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "clsa_internal.h"

namespace clsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp32 -> bf16 round-to-nearest-even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map of a score to an unsigned key: a larger score gives a larger key.
// -0.0 is mapped like +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int row_seq(const RowsDev& rw, int r) { return rw.mode == CLSA_MODE_DECODE ? r : rw.seq; }

// Tokens row r sees, clamped to the host bound so that no write leaves the caller's buffers.
__device__ __forceinline__ int row_len(const RowsDev& rw, int r) {
  if (rw.mode == CLSA_MODE_DECODE) {
    const int n = rw.cu[r + 1] - rw.cu[r];
    return n < 0 ? 0 : (n > rw.max_row_len ? rw.max_row_len : n);
  }
  return rw.pos0 + r + 1;
}

// 16-byte streaming load that is not expected to be reused (non-temporal hint).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Plain 16-byte load through a native vector type (a uint4 struct copy can become a memcpy into
// private memory).
__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T>
__device__ __forceinline__ T bitcast(const uint4& v) {
  return __builtin_bit_cast(T, v);
}

// DPP lane exchange inside rows of 16 lanes.  The pairing partner of each step has the
// opposite bit `M` of the lane id and the same higher bits (8: rotate by 8; 4: mirror inside
// half-rows; 2 and 1: quad permutes).
template <int M>
__device__ __forceinline__ float dpp_partner(float v) {
  int x = __float_as_int(v);
  if constexpr (M == 8) x = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);       // row_ror:8
  else if constexpr (M == 4) x = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  else if constexpr (M == 2) x = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  else x = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);                          // quad_perm 1,0,3,2
  return __int_as_float(x);
}

// ---- handing data from one workgroup to another inside a kernel ----------------------------
// A device-scope fence (__threadfence) writes back and invalidates the whole L2 of the XCD; done
// by every workgroup it serialises the chip.  Instead, data that another workgroup will read is
// stored with device-scope relaxed atomic stores (written through to the device coherence point),
// each thread waits for its stores to complete, and the reader uses device-scope relaxed atomic
// loads.  The one atomic ticket per workgroup then orders "all producers done" before the reads.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_memory() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Every thread calls this after storing (with st_dev) what the last workgroup will read.  Returns
// true in all threads of the workgroup that arrives last (of `arrivals`), which also resets the
// ticket to zero for the next launch.  `flag` is one int of LDS.
__device__ __forceinline__ bool arrive_last(uint32_t* ticket, uint32_t arrivals, int* flag) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag[0] = prev == arrivals - 1;
    if (prev == arrivals - 1) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return flag[0] != 0;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2, 4, 8 inside each row
// of 16 lanes, then the last lane of row 0 (row_bcast15) and of rows 0-1 (row_bcast31) is added
// to the rows above.  Lanes whose DPP source is outside the row receive 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Block-wide exclusive scan of one (or two) ints per thread (blockDim.x a multiple of 64,
// <= 1024).  `scratch` holds at least 2 * (blockDim.x / 64) ints.  Returns the exclusive prefix and
// sets *total.  Contains two __syncthreads(); scratch may be reused after it returns.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = scratch[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__device__ __forceinline__ void block_exclusive_scan2(int v0, int v1, int* scratch, int* out0, int* out1,
                                                      int* total0, int* total1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int i0 = wave_inclusive_scan(v0), i1 = wave_inclusive_scan(v1);
  if (lane == 63) {
    scratch[wave] = i0;
    scratch[nw + wave] = i1;
  }
  __syncthreads();
  int b0 = 0, b1 = 0, a0 = 0, a1 = 0;
  for (int w = 0; w < nw; ++w) {
    const int t0 = scratch[w], t1 = scratch[nw + w];
    b0 += w < wave ? t0 : 0;
    b1 += w < wave ? t1 : 0;
    a0 += t0;
    a1 += t1;
  }
  __syncthreads();
  *out0 = b0 + i0 - v0;
  *out1 = b1 + i1 - v1;
  *total0 = a0;
  *total1 = a1;
}

// Wave 0 finds, in a 256-bin LDS histogram, the bin d (from the top bin down) whose cumulative
// count first reaches `need`, and publishes res[0] = d, res[1] = count of the bins above d.  All
// threads must call it; it ends with __syncthreads().
__device__ __forceinline__ void find_bin256_from_top(const uint32_t* hist, int need, int* res) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // lane owns bins 255 - 4 lane .. 252 - 4 lane (descending)
    int h[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = (int)hist[255 - 4 * lane - j];
      loc += h[j];
    }
    int run = wave_inclusive_scan(loc) - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run < need && run + h[j] >= need) {
        res[0] = 255 - 4 * lane - j;
        res[1] = run;
      }
      run += h[j];
    }
  }
  __syncthreads();
}

}  // namespace clsa
