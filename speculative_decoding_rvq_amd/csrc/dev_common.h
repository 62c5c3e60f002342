// Device helpers shared by the CodePredictor round kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cps {

constexpr int kBlock = 256;  // every kernel runs 4 wave64s per workgroup
constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// One 16-byte weight chunk: 4 fp32 or 8 bf16 values, unpacked to fp32.
template <typename WT> struct Chunk;
template <> struct Chunk<float> {
  using T = float4;
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const float4& v, float* o) {
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct Chunk<uint16_t> {
  using T = uint4;
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float* o) {
    o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
    o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
  }
};

// Row `row` of a table stored as WT, converted to fp32 element `i`.
template <typename WT> __device__ __forceinline__ float load_elem(const WT* p, size_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// ----------------------------------------------------------- reductions ----
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Block-wide reductions over 256 threads; `red` is 4+ words of LDS.  Every
// thread gets the result.  Fixed tree order: deterministic.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  v = wave_max_u64(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  uint64_t a = red[0] > red[1] ? red[0] : red[1];
  uint64_t b = red[2] > red[3] ? red[2] : red[3];
  return a > b ? a : b;
}
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  uint32_t a = red[0] > red[1] ? red[0] : red[1];
  uint32_t b = red[2] > red[3] ? red[2] : red[3];
  return a > b ? a : b;
}
__device__ __forceinline__ int block_sum_i(int v, int* red) {
  v = wave_sum_i(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Exclusive prefix sum of one int per thread over the block (thread order).
// `red` needs 4 words of LDS.  Returns the exclusive prefix; *total = sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  int inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(inc, o, kWave);
    if (l >= o) inc += n;
  }
  __syncthreads();
  if (l == kWave - 1) red[w] = inc;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += red[i];
  *total = red[0] + red[1] + red[2] + red[3];
  return base + inc - v;
}

// ------------------------------------------------------------- Philox ----
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11, section 4): ten rounds of
// the 4-word multiply/xor S-box with a Weyl-advanced 2-word key.
__device__ __forceinline__ uint32_t philox_word0(uint64_t seed, uint32_t c0, uint32_t c1) {
  uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = 0u;
  uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * x0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * x2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ x1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ x3 ^ k1;
    x1 = static_cast<uint32_t>(p1);
    x3 = static_cast<uint32_t>(p0);
    x0 = n0;
    x2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return x0;
}

enum Purpose : uint32_t { kDraft = 0, kAccept = 1, kTarget = 2 };

// Uniform of one frame decision: 24 random bits of word 0 of
// Philox4x32-10(counter = (depth, purpose, 0, 0), key = seed), in [0, 1).
__device__ __forceinline__ float frame_uniform(uint64_t seed, int depth, uint32_t purpose) {
  return static_cast<float>(philox_word0(seed, static_cast<uint32_t>(depth), purpose) >> 8) *
         (1.0f / 16777216.0f);
}

// Order-preserving float -> uint32 key (larger float -> larger key); +0 and
// -0 map to the same key.
__device__ __forceinline__ uint32_t float_key(float z) {
  uint32_t u = __float_as_uint(z);
  if (z == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Near-tie thresholds and flag bits (same values as the C header).
constexpr float kEpsAccept = 1e-5f;
constexpr double kEpsGap = 1e-4;
constexpr double kEpsCdf = 1e-5;
constexpr uint32_t kFlagTopk = 1u, kFlagArgmax = 2u, kFlagCdf = 4u, kFlagAccept = 8u;

// LDS scratch the block sampler needs: compacted support of up to V entries.
struct SampleSmem {
  int idx[4096];
  float w[4096];
  int red[8];
  int result[2];
};

// Sample(w, u) over a row whose weights are produced by `weight(i)`,
// i in [0, V), V a multiple of 256: the entries with w_i > 0 in ascending
// code order, a sequential float32 running sum, t = u * sum, first entry
// whose running sum exceeds t.  Result for every thread: the code, and the
// CDF near-tie flag through *flag.  Returns -1 if no weight is positive.
template <typename WF>
__device__ int block_sample(WF weight, int V, float u, SampleSmem& sm, bool* flag) {
  const int per = V / kBlock;
  const int base = threadIdx.x * per;
  int cnt = 0;
  for (int j = 0; j < per; ++j) cnt += weight(base + j) > 0.0f ? 1 : 0;
  int total;
  int off = block_exclusive_scan(cnt, sm.red, &total);
  for (int j = 0; j < per; ++j) {
    const float wv = weight(base + j);
    if (wv > 0.0f) {
      sm.idx[off] = base + j;
      sm.w[off] = wv;
      ++off;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int code = -1, near = 0;
    if (total > 0) {
#pragma clang fp contract(off)
      float tot = 0.0f;
      for (int i = 0; i < total; ++i) tot = tot + sm.w[i];
      const float t = u * tot;
      const double eps = static_cast<double>(tot) * kEpsCdf;
      float run = 0.0f;
      int pos = total - 1;
      for (int i = 0; i < total; ++i) {
        const float before = run;
        run = run + sm.w[i];
        if (t < run) {
          pos = i;
          const bool lo = i > 0 && fabs(static_cast<double>(t) - static_cast<double>(before)) < eps;
          const bool hi = i + 1 < total && fabs(static_cast<double>(run) - static_cast<double>(t)) < eps;
          near = (lo || hi) ? 1 : 0;
          break;
        }
        if (i == total - 1) {  // t == sum after rounding: the last entry
          near = (i > 0 && fabs(static_cast<double>(t) - static_cast<double>(before)) < eps) ? 1 : 0;
        }
      }
      code = sm.idx[pos];
    }
    sm.result[0] = code;
    sm.result[1] = near;
  }
  __syncthreads();
  *flag = sm.result[1] != 0;
  const int code = sm.result[0];
  __syncthreads();
  return code;
}

}  // namespace cps
