// Device helpers shared by the CodePredictor round kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "kernels.h"

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

// Activation rows that feed the packed matrix-core projections are carried
// as two fp16 pieces, x ~ hi + lo: hi = fp16(x) and lo = fp16(x - hi), both
// rounded to nearest even (x - hi is exact in fp32).  hi + lo holds x to 22
// significant bits, or to 2^-25 in absolute terms when lo is subnormal;
// fp16 x fp16 products are exact in fp32.  A value outside fp16's range
// (|x| >= 65504, or NaN) sets the caller's overflow flag and is carried as
// +-65504, so what it feeds stays finite (and wrong: the caller reports the
// flag).  kPieces (two) in kernels.h.
constexpr float kF16Max = 65504.0f;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// The two pieces of x0, x1, packed two values per word (x0 in the low half).
__device__ __forceinline__ void split2_pair(float x0, float x1, uint32_t& hi, uint32_t& lo, bool& bad) {
  bad |= !(fabsf(x0) < kF16Max) || !(fabsf(x1) < kF16Max);
  x0 = fminf(fmaxf(x0, -kF16Max), kF16Max);  // NaN -> -65504
  x1 = fminf(fmaxf(x1, -kF16Max), kF16Max);
  const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
  const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
  const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
  hi = f16_bits(h0) | (f16_bits(h1) << 16);
  lo = f16_bits(l0) | (f16_bits(l1) << 16);
}

// Eight consecutive values y of row `row`, columns k .. k+7 (k % 8 == 0),
// split into their two pieces and stored as one fragment entry per piece in
// a chunk-major plane buffer with T row tiles: row tile t = row / 16, K
// chunk c = k / 32, piece p at ((c * T + t) * 2 + p) * 64 16-byte entries,
// fragment lane (row % 16) + 16 ((k % 32) / 8).  Returns whether a value
// was outside fp16's range (the caller raises the overflow flag for rows
// whose outputs are used).
__device__ __forceinline__ bool split_store8(uint16_t* planes, int T, int row, int k, const float (&y)[8]) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  uint32_t hp[4], lp[4];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 8; i += 2) split2_pair(y[i], y[i + 1], hp[i / 2], lp[i / 2], bad);
  const int L = row % 16 + 16 * ((k % 32) / 8);
  u32x4_t* dst =
      reinterpret_cast<u32x4_t*>(planes) + (static_cast<size_t>(k / 32) * T + row / 16) * kPieces * 64 + L;
  dst[0] = u32x4_t{hp[0], hp[1], hp[2], hp[3]};
  dst[64] = u32x4_t{lp[0], lp[1], lp[2], lp[3]};
  return bad;
}

// Four consecutive values y of row `row`, columns k .. k+3 (k % 4 == 0):
// half of a fragment entry per piece (8 bytes), same layout as split_store8.
__device__ __forceinline__ bool split_store4(uint16_t* planes, int T, int row, int k, const float (&y)[4]) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  uint32_t h0, h1, l0, l1;
  bool bad = false;
  split2_pair(y[0], y[1], h0, l0, bad);
  split2_pair(y[2], y[3], h1, l1, bad);
  const int L = row % 16 + 16 * ((k % 32) / 8);
  uint16_t* dst = planes + ((static_cast<size_t>(k / 32) * T + row / 16) * kPieces * 64 + L) * 8 + (k % 8);
  *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{h0, h1};
  *reinterpret_cast<u32x2_t*>(dst + 64 * 8) = u32x2_t{l0, l1};
  return bad;
}

// The overflow flag of a split row: raised for rows at a position (pos
// nullable: every row).  Inactive rows run through the projections with
// whatever their buffers hold, and their outputs are never used.
__device__ __forceinline__ void flag_overflow(int* ovf, const int* pos, int row) {
  if (ovf != nullptr && (pos == nullptr || pos[row] >= 0)) *ovf = 1;
}

// Row `row` of a table stored as WT, converted to fp32 element `i`.
template <typename WT> __device__ __forceinline__ float load_elem(const WT* p, size_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// ----------------------------------------------------------- reductions ----
// Cross-lane steps use DPP (row rotations / shifts / broadcasts inside the
// VALU) and readlane, not LDS permutes.  Fixed association order:
// deterministic.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ uint32_t lane_u(uint32_t v, int l) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}

// row_ror:n control words (rotate within each row of 16 lanes)
constexpr int kRor8 = 0x128, kRor4 = 0x124, kRor2 = 0x122, kRor1 = 0x121;

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kRor8>(v);
  v += dpp_f<kRor4>(v);
  v += dpp_f<kRor2>(v);
  v += dpp_f<kRor1>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kRor8>(v));
  v = fmaxf(v, dpp_f<kRor4>(v));
  v = fmaxf(v, dpp_f<kRor2>(v));
  v = fmaxf(v, dpp_f<kRor1>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, static_cast<uint32_t>(dpp_i<kRor8>(static_cast<int>(v))));
  v = umax32(v, static_cast<uint32_t>(dpp_i<kRor4>(static_cast<int>(v))));
  v = umax32(v, static_cast<uint32_t>(dpp_i<kRor2>(static_cast<int>(v))));
  v = umax32(v, static_cast<uint32_t>(dpp_i<kRor1>(static_cast<int>(v))));
  return umax32(umax32(lane_u(v, 0), lane_u(v, 16)), umax32(lane_u(v, 32), lane_u(v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  v = mn(v, static_cast<uint32_t>(dpp_i<kRor8>(static_cast<int>(v))));
  v = mn(v, static_cast<uint32_t>(dpp_i<kRor4>(static_cast<int>(v))));
  v = mn(v, static_cast<uint32_t>(dpp_i<kRor2>(static_cast<int>(v))));
  v = mn(v, static_cast<uint32_t>(dpp_i<kRor1>(static_cast<int>(v))));
  return mn(mn(lane_u(v, 0), lane_u(v, 16)), mn(lane_u(v, 32), lane_u(v, 48)));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kRor8>(v);
  v += dpp_i<kRor4>(v);
  v += dpp_i<kRor2>(v);
  v += dpp_i<kRor1>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
// Largest 64-bit key of the wave (compared as unsigned).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32);
  const uint32_t mhi = wave_max_u32(hi);
  const uint32_t lo = hi == mhi ? static_cast<uint32_t>(v) : 0u;
  return (static_cast<uint64_t>(mhi) << 32) | wave_max_u32(lo);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each
// row of 16 (row_shr 1, 2, 4, 8 with zero fill), then the row totals carried
// across rows with row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Block barrier ordering LDS accesses only: global stores still in flight
// are not waited for (the workgroup-scope fence of a full barrier would).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS written by some lanes of a wave, then read by others of the same wave:
// a wave's LDS accesses are performed in order, so only the compiler needs
// holding back.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Block-wide reductions over 256 threads; `red` is 4+ words of LDS.  Every
// thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  lds_sync();
  if (l == 0) red[w] = v;
  lds_sync();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  v = wave_max_u64(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  lds_sync();
  if (l == 0) red[w] = v;
  lds_sync();
  uint64_t a = red[0] > red[1] ? red[0] : red[1];
  uint64_t b = red[2] > red[3] ? red[2] : red[3];
  return a > b ? a : b;
}
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  lds_sync();
  if (l == 0) red[w] = v;
  lds_sync();
  return umax32(umax32(red[0], red[1]), umax32(red[2], red[3]));
}
__device__ __forceinline__ int block_sum_i(int v, int* red) {
  v = wave_sum_i(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  lds_sync();
  if (l == 0) red[w] = v;
  lds_sync();
  return red[0] + red[1] + red[2] + red[3];
}

// Exclusive prefix sum of one int per thread over the block (thread order).
// `red` needs 4 words of LDS.  Returns the exclusive prefix; *total = sum.
template <int NW = kBlock / kWave>
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int inc = wave_incl_scan(v);
  lds_sync();
  if (l == kWave - 1) red[w] = inc;
  lds_sync();
  int base = 0, t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    base += i < w ? red[i] : 0;
    t += red[i];
  }
  *total = t;
  return base + inc - v;
}

// The rows of one lm_head: indices i < n, ascending, with head[i] == h.  The
// block keeps positions [first, first + cap) of that list in rows[0..cap)
// (-1 past its end) and returns how many it kept; NT threads in the block,
// `red` is NT / 64 ints of LDS.
template <int NT = kBlock>
__device__ __forceinline__ int head_rows_slice(const int* head, int n, int h, int first, int cap, int* rows,
                                               int* red) {
  for (int i = threadIdx.x; i < cap; i += NT) rows[i] = -1;
  int base = 0;
  for (int r0 = 0; r0 < n; r0 += NT) {
    const int i = r0 + threadIdx.x;
    const bool hit = i < n && head[i] == h;
    int total;
    const int pos = base + block_exclusive_scan<NT / kWave>(hit ? 1 : 0, red, &total);  // barriers inside
    if (hit && pos >= first && pos < first + cap) rows[pos - first] = i;
    base += total;
  }
  __syncthreads();
  return min(max(base - first, 0), cap);
}

// ------------------------------------------------------------- Philox ----
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11, section 4): ten rounds of
// the 4-word multiply/xor S-box with a Weyl-advanced 2-word key.
__device__ __forceinline__ uint32_t philox_word0(uint64_t seed, uint32_t c0, uint32_t c1, uint32_t c2 = 0u) {
  uint32_t x0 = c0, x1 = c1, x2 = c2, x3 = 0u;
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
// Philox4x32-10(counter = (depth, purpose, index, 0), key = seed), in [0, 1).
// index 0 for the chain window; a tree window numbers the draws of a depth
// and the children tested at a node.
__device__ __forceinline__ float frame_uniform(uint64_t seed, int depth, uint32_t purpose, uint32_t index = 0u) {
  return static_cast<float>(philox_word0(seed, static_cast<uint32_t>(depth), purpose, index) >> 8) *
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

// One wave: Sample over the list w[0..total) in list order (entries with
// w = 0 are skipped, as Sample skips non-positive weights).  Lane 0 turns w
// into its running sums in place, sequentially in float32; t = u * sum; the
// first running sum above t is then found 64 entries at a time by ballot.
// *code = idx of the chosen entry (-1 if no entry is positive); *near = the
// CDF near-tie flag (t within 1e-5 * sum of a boundary of the chosen entry
// that has a positive entry on its other side; positions among the positive
// entries come from per-block positivity masks, lane c holding block c's).
// Needs: w 16-byte aligned and zero from total up to the next multiple of 32;
// total <= 4096; all 64 lanes active.
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  return (static_cast<uint64_t>(lane_u(static_cast<uint32_t>(v >> 32), l)) << 32) |
         lane_u(static_cast<uint32_t>(v), l);
}

// The first half of list_draw: the positivity masks of w[0..total) and lane
// 0's running sums in place.  Several list_search calls with different u can
// then share one prefix.
struct ListSums {
  uint64_t mine;  // positivity mask of block `lane`
  int npos, last;
};

__device__ __forceinline__ ListSums list_prefix(float* w, int total) {
  const int lane = threadIdx.x % kWave;
  uint64_t mine = 0;  // positivity mask of block `lane`
  int npos = 0, last = -1;
  for (int c0 = 0, c = 0; c0 < total; c0 += kWave, ++c) {
    const int i = c0 + lane;
    const uint64_t m = __ballot(i < total && w[min(i, total - 1)] > 0.0f);
    if (lane == c) mine = m;
    npos += __popcll(m);
    if (m) last = c0 + 63 - __clzll(static_cast<long long>(m));
  }
  if (npos == 0) return ListSums{mine, 0, last};
  if (lane == 0) {
    float carry = 0.0f;
    for (int c0 = 0; c0 < total; c0 += 32) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const float4 q = *reinterpret_cast<const float4*>(&w[c0 + i]);
        v[i] = q.x;
        v[i + 1] = q.y;
        v[i + 2] = q.z;
        v[i + 3] = q.w;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        carry = carry + v[i];
        v[i] = carry;
      }
#pragma unroll
      for (int i = 0; i < 32; i += 4)
        *reinterpret_cast<float4*>(&w[c0 + i]) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    }
  }
  wave_lds_sync();
  return ListSums{mine, npos, last};
}

// The second half: the entry whose running sum first exceeds u * sum.
template <typename IT>
__device__ __forceinline__ void list_search(const float* w, const IT* idx, int total, const ListSums& ls, float u,
                                            int* code, int* near) {
  const int lane = threadIdx.x % kWave;
  const uint64_t mine = ls.mine;
  const int npos = ls.npos, last = ls.last;
  *code = -1;
  *near = 0;
  if (npos == 0) return;
  const float tot = w[total - 1];
  const float t = u * tot;
  const double eps = static_cast<double>(tot) * kEpsCdf;
  for (int c0 = 0, c = 0; c0 < total; c0 += kWave, ++c) {
    const int i = c0 + lane;
    const uint64_t hit = __ballot(i < total && t < w[min(i, total - 1)]);
    if (hit) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      const int pos = c0 + l;
      const float run = w[pos];
      const float before = pos > 0 ? w[pos - 1] : 0.0f;
      // positive entries before the chosen one
      const int pb = wave_sum_i(lane < c ? __popcll(mine) : 0) +
                     __popcll(lane_u64(mine, c) & ((1ull << l) - 1ull));
      const bool lo = pb > 0 && fabs(static_cast<double>(t) - static_cast<double>(before)) < eps;
      const bool hi = pb + 1 < npos && fabs(static_cast<double>(run) - static_cast<double>(t)) < eps;
      *code = static_cast<int>(idx[pos]);
      *near = (lo || hi) ? 1 : 0;
      return;
    }
  }
  // t == sum after rounding: the last positive entry owns the top end
  const float before_last = last > 0 ? w[last - 1] : 0.0f;
  *code = static_cast<int>(idx[last]);
  *near = (npos > 1 && fabs(static_cast<double>(t) - static_cast<double>(before_last)) < eps) ? 1 : 0;
}

template <typename IT>
__device__ __forceinline__ void list_draw(float* w, const IT* idx, int total, float u, int* code, int* near) {
  const ListSums ls = list_prefix(w, total);
  list_search(w, idx, total, ls, u, code, near);
}

}  // namespace cps
