// Device filler of the seeded synthetic inputs (the same generator as clsa_synth/gen.py, written
// for the GPU so that multi-GiB caches are produced in HBM without a host copy).  It holds none of
// the CLSA method's arithmetic.
//
//   mix(z): SplitMix64 output function of z + 0x9E3779B97F4A7C15 (Steele, Lea & Flood 2014)
//   key    = mix(mix(seed) ^ tensor_id);   draw j of element i = mix(key + 4 i + j)
//   uniform integer in [lo, hi]: lo + (((draw0 >> 32) * (hi - lo + 1)) >> 32), divided by den
//   ~N(0,1): (sum of the twelve 16-bit fields of draws 0..2 - 393210) / 65536
//   fp32 -> bf16: round to nearest even on the bit pattern
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t host_mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void k_fill_uniform(uint16_t* __restrict__ out, int64_t n, uint64_t key, int lo, int hi, float inv_den) {
  const uint64_t m = (uint64_t)(hi - lo + 1);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t x = mix(key + (uint64_t)i * 4ull);
    const int v = lo + (int)(((x >> 32) * m) >> 32);
    out[i] = to_bf16((float)v * inv_den);
  }
}

__global__ void k_fill_normal(uint16_t* __restrict__ out, int64_t n, uint64_t key) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t total = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint64_t x = mix(key + (uint64_t)i * 4ull + (uint64_t)j);
      total += (int64_t)(x & 0xFFFFull) + (int64_t)((x >> 16) & 0xFFFFull) + (int64_t)((x >> 32) & 0xFFFFull) +
               (int64_t)(x >> 48);
    }
    out[i] = to_bf16((float)(total - 393210) / 65536.0f);
  }
}

// k_idx[token, :] = 2 * q_idx[src, :] for every (token, src) pair.
__global__ void k_plant(uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ q_idx,
                        const int64_t* __restrict__ pairs, int n_pairs, int d) {
  const int p = blockIdx.x;
  if (p >= n_pairs) return;
  const int64_t tok = pairs[2 * p], src = pairs[2 * p + 1];
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    const float v = __uint_as_float((uint32_t)q_idx[src * d + c] << 16);
    k_idx[tok * d + c] = to_bf16(2.0f * v);
  }
}

uint64_t tensor_key(uint64_t seed, uint32_t tid) { return host_mix(host_mix(seed) ^ (uint64_t)tid); }

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

extern "C" {

int synth_fill_uniform_int(uint16_t* out, int64_t n, uint64_t seed, uint32_t tensor_id, int lo, int hi, int den,
                           void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fill_uniform, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, out, n,
                     tensor_key(seed, tensor_id), lo, hi, 1.0f / (float)den);
  return (int)hipGetLastError();
}

int synth_fill_normal(uint16_t* out, int64_t n, uint64_t seed, uint32_t tensor_id, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fill_normal, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, out, n,
                     tensor_key(seed, tensor_id));
  return (int)hipGetLastError();
}

int synth_plant_needles(uint16_t* k_idx, const uint16_t* q_idx, const int64_t* pairs_dev, int n_pairs, int d,
                        void* stream) {
  if (n_pairs <= 0) return 0;
  hipLaunchKernelGGL(k_plant, dim3(n_pairs), dim3(128), 0, (hipStream_t)stream, k_idx, q_idx, pairs_dev, n_pairs, d);
  return (int)hipGetLastError();
}

uint64_t synth_tensor_key(uint64_t seed, uint32_t tensor_id) { return tensor_key(seed, tensor_id); }

}  // extern "C"
