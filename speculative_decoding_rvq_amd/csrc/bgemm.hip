// Batched projections and lm_heads on the matrix cores: bf16 weights, fp32
// activations (many activation rows: streams x verify rows).
//
// C[m][n] = sum_k x_m[k] * W[n][k], W row-major [out][in].
//
// Every fp32 activation is split into three bf16 pieces by truncation,
// x = hi + mid + lo (split3), and the tile runs v_mfma_f32_16x16x32_bf16
// once per piece into one fp32 accumulator.  bf16 x bf16 products are exact
// in fp32, so the result is the fp32 dot product up to summation order.
//
// Tiling: a block owns (16 FM) x (16 FN) outputs and its four wave64s split
// K in quarters: a wave reads its activation and weight fragments straight
// from global memory in the MFMA operand layout (lane l: row l % 16, k =
// 8 (l / 16) .. +7 of each 32-wide chunk), splits its activation fragments
// in registers and keeps two chunks of loads in flight.  Loads are
// unconditional and held in native vectors, so the compiler's waits count
// exactly the chunk being consumed.  The four partial tiles (and the rows'
// partial sums of squares) meet in LDS and are added in wave order: the
// result does not depend on timing.  Many small tiles fill the chip without
// any cross-block reduction.
//
// RMSNorm: x * g is split; the rows' sums of squares are accumulated on the
// way and 1/sqrt(mean + eps) scales the outputs.  Epilogues: residual add,
// SwiGLU (columns 0..TN/2-1 of a tile are gate rows, TN/2..TN-1 the matching
// up rows), Q write plus K/V append at the row's position, lm_head logits for
// rows grouped by head (final-normed rows written once).
#include "dev_common.h"
#include "kernels.h"

namespace cps {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = kBlock / kWave;  // 4: K quarters

// Weight row read for output column n of the launch (SwiGLU tiles of TN
// columns: TN/2 gate rows, then the matching up rows).
template <typename WT, int MODE, int TN>
__device__ __forceinline__ const WT* bweight_row(const GemvArgs& a, const WT* W0, int n) {
  if (MODE == kQKV) {
    const WT* W1 = static_cast<const WT*>(a.W1);
    const WT* W2 = static_cast<const WT*>(a.W2);
    if (n < a.qdim) return W0 + static_cast<size_t>(n) * a.K;
    if (n < a.qdim + a.kvdim) return W1 + static_cast<size_t>(n - a.qdim) * a.K;
    return W2 + static_cast<size_t>(n - a.qdim - a.kvdim) * a.K;
  }
  if (MODE == kSwiGLU) {
    const WT* W1 = static_cast<const WT*>(a.W1);
    const int tile = n / TN, c = n % TN;
    const int f = tile * (TN / 2) + (c % (TN / 2));
    return (c < TN / 2 ? W0 : W1) + static_cast<size_t>(f) * a.K;
  }
  return W0 + static_cast<size_t>(n) * a.K;
}

template <int MODE, int FM, int FN, bool NORM>
__global__ __launch_bounds__(kBlock) void bgemm_kernel(const GemvArgs a) {
  using WT = uint16_t;  // bf16 bit patterns
  constexpr int TM = 16 * FM, TN = 16 * FN;
  __shared__ float part[kWaves][TM][TN + 1];
  __shared__ float ssq_s[kWaves][TM];
  __shared__ float rinv_s[TM];
  __shared__ int rows_s[TM];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * TN;

  // ---- the block's activation rows ----
  const WT* W0 = static_cast<const WT*>(a.W0);
  int count;
  if (MODE == kHead) {
    const int j = blockIdx.z;  // head j+1: its rows, ascending, slice blockIdx.y
    __shared__ int red_h[4];
    count = head_rows_slice(a.head, a.M, j + 1, blockIdx.y * TM, TM, rows_s, red_h);
    if (count <= 0) return;
    W0 = W0 + static_cast<size_t>(j) * static_cast<size_t>(a.head_stride);
  } else {
    const int m0 = blockIdx.y * TM;
    count = min(TM, a.M - m0);
    if (tid < TM) rows_s[tid] = tid < count ? m0 + tid : -1;
  }
  __syncthreads();

  // ---- this lane's operand rows; a missing row reads X row 0 (masked) ----
  const float* xr[FM];
  bool xv[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int row = rows_s[16 * f + li];
    xv[f] = row >= 0;
    xr[f] = a.X + static_cast<size_t>(row >= 0 ? row / a.xdiv : 0) * a.ldx;
  }
  const WT* wr[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) wr[f] = bweight_row<WT, MODE, TN>(a, W0, n0 + 16 * f + li);
  const int cw = a.K / 32 / kWaves;          // chunks of this wave (even)
  const int kbase = wave * cw * 32 + 8 * lg;  // lane's first k

  struct Frag {  // one chunk of this lane's operands (native vectors)
    floatx4 x[FM][2];
    floatx4 g[2];
    u32x4 w[FN];  // 8 bf16 per weight fragment
  };
  auto fetch = [&](int c) __attribute__((always_inline)) {
    Frag f;
    const int k = kbase + c * 32;
#pragma unroll
    for (int i = 0; i < FN; ++i) f.w[i] = *reinterpret_cast<const u32x4*>(wr[i] + k);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      f.x[i][0] = *reinterpret_cast<const floatx4*>(xr[i] + k);
      f.x[i][1] = *reinterpret_cast<const floatx4*>(xr[i] + k + 4);
    }
    if constexpr (NORM) {
      f.g[0] = *reinterpret_cast<const floatx4*>(a.norm_g + k);
      f.g[1] = *reinterpret_cast<const floatx4*>(a.norm_g + k + 4);
    } else {
      f.g[0] = f.g[1] = floatx4{1.0f, 1.0f, 1.0f, 1.0f};
    }
    return f;
  };

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float ss[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) ss[f] = 0.0f;

  auto compute = [&](const Frag& fr) __attribute__((always_inline)) {
    float xs[FM][8];  // this lane's x (* g) values of the chunk
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = xv[f] ? fr.x[f][e / 4][e % 4] : 0.0f;
        ss[f] += x * x;
        xs[f][e] = NORM ? x * fr.g[e / 4][e % 4] : x;
      }
    bf16x8 ap[FM][3];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      uint32_t hp[4], mp[4], lp[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t h0, m0, l0, h1, m1, l1;
        split3(xs[f][e], h0, m0, l0);
        split3(xs[f][e + 1], h1, m1, l1);
        hp[e / 2] = h0 | (h1 << 16);
        mp[e / 2] = m0 | (m1 << 16);
        lp[e / 2] = l0 | (l1 << 16);
      }
      ap[f][0] = __builtin_bit_cast(bf16x8, u32x4{hp[0], hp[1], hp[2], hp[3]});
      ap[f][1] = __builtin_bit_cast(bf16x8, u32x4{mp[0], mp[1], mp[2], mp[3]});
      ap[f][2] = __builtin_bit_cast(bf16x8, u32x4{lp[0], lp[1], lp[2], lp[3]});
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int n = 0; n < FN; ++n)
          acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap[f][p], __builtin_bit_cast(bf16x8, fr.w[n]),
                                                              acc[f][n], 0, 0, 0);
  };

  // ---- K loop: two chunks in flight (the chunk count is even; the
  // fetches past the end re-read the last chunk and are not used) ----
  Frag f0 = fetch(0);
  __builtin_amdgcn_sched_barrier(0);
  Frag f1 = fetch(1);
  __builtin_amdgcn_sched_barrier(0);
  for (int c = 0; c < cw; c += 2) {
    compute(f0);
    __builtin_amdgcn_sched_barrier(0);
    f0 = fetch(min(c + 2, cw - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(f1);
    __builtin_amdgcn_sched_barrier(0);
    f1 = fetch(min(c + 3, cw - 1));
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- partial tiles and sums of squares -> LDS, added in wave order ----
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int n = 0; n < FN; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][16 * f + 4 * lg + i][16 * n + li] = acc[f][n][i];
  if (NORM) {
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      float t = ss[f];
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      if (lg == 0) ssq_s[wave][16 * f + li] = t;
    }
  }
  __syncthreads();
  if (NORM && tid < TM) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += ssq_s[w][tid];
    rinv_s[tid] = 1.0f / sqrtf(t / static_cast<float>(a.K) + a.eps);
  }
  __syncthreads();
  auto tile_val = [&](int r, int c) {
    float v = part[0][r][c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += part[w][r][c];
    return NORM ? v * rinv_s[r] : v;
  };

  // final-normed rows for the heads' caller (the column tiles split K)
  if (MODE == kHead && NORM && a.xnorm_out != nullptr) {
    const int k4 = a.K / 4;
    const int per = (k4 + gridDim.x - 1) / gridDim.x;
    const int c0 = blockIdx.x * per, c1 = min(k4, c0 + per);
    const int w = c1 - c0;
    for (int idx = tid; w > 0 && idx < count * w; idx += kBlock) {
      const int r = idx / w, c = 4 * (c0 + idx % w);
      const int row = rows_s[r];
      const float4 x = *reinterpret_cast<const float4*>(a.X + static_cast<size_t>(row / a.xdiv) * a.ldx + c);
      const float4 g = *reinterpret_cast<const float4*>(a.norm_g + c);
      const float ri = rinv_s[r];
      *reinterpret_cast<float4*>(a.xnorm_out + static_cast<size_t>(row) * a.K + c) =
          make_float4(x.x * g.x * ri, x.y * g.y * ri, x.z * g.z * ri, x.w * g.w * ri);
    }
  }

  // ---- fused epilogue ----
  if (MODE == kSwiGLU) {
    for (int idx = tid; idx < TM * (TN / 2); idx += kBlock) {
      const int r = idx / (TN / 2), c = idx % (TN / 2);
      const int row = rows_s[r];
      if (row < 0) continue;
      const float g = tile_val(r, c), u = tile_val(r, c + TN / 2);
      const float sg = g / (1.0f + expf(-g));
      a.Y[static_cast<size_t>(row) * a.ldy + blockIdx.x * (TN / 2) + c] = sg * u;
    }
    return;
  }
  for (int idx = tid; idx < TM * TN; idx += kBlock) {
    const int r = idx / TN, c = idx % TN;
    const int row = rows_s[r];
    if (row < 0) continue;
    const float val = tile_val(r, c);
    const int o = n0 + c;
    if (MODE == kAdd) {
      a.Y[static_cast<size_t>(row) * a.ldy + o] += val;
    } else if (MODE == kHead) {
      a.Y[static_cast<size_t>(row) * a.ldy + o] = val;
    } else if (MODE == kQKV) {
      if (o < a.qdim) {
        a.Y[static_cast<size_t>(row) * a.ldy + o] = val;
      } else {
        const int pp = a.pos[row];
        if (pp >= 0 && pp < a.kv_positions) {
          const int b = row / a.rows_per_stream;
          float* base = a.kv + static_cast<size_t>(b) * a.kv_sb + static_cast<size_t>(pp) * a.kvdim;
          const int oo = o - a.qdim;
          if (oo < a.kvdim) base[oo] = val;
          else base[a.kv_vo + (oo - a.kvdim)] = val;
        }
      }
    }
  }
}

template <int FM, int FN, bool NORM>
hipError_t launch_t(int mode, const GemvArgs& a, dim3 grid, hipStream_t s) {
  switch (mode) {
    case kAdd: hipLaunchKernelGGL((bgemm_kernel<kAdd, FM, FN, NORM>), grid, dim3(kBlock), 0, s, a); break;
    case kSwiGLU: hipLaunchKernelGGL((bgemm_kernel<kSwiGLU, FM, FN, NORM>), grid, dim3(kBlock), 0, s, a); break;
    case kQKV: hipLaunchKernelGGL((bgemm_kernel<kQKV, FM, FN, NORM>), grid, dim3(kBlock), 0, s, a); break;
    case kHead: hipLaunchKernelGGL((bgemm_kernel<kHead, FM, FN, NORM>), grid, dim3(kBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FM, int FN>
hipError_t launch_f(int mode, const GemvArgs& a, dim3 grid, hipStream_t s) {
  return a.norm_g != nullptr ? launch_t<FM, FN, true>(mode, a, grid, s)
                             : launch_t<FM, FN, false>(mode, a, grid, s);
}

}  // namespace

// bf16 weights only: fp32 weights keep the fp32 kernels of mfma_impl.h,
// which measured faster on the small fp32 shapes.
hipError_t launch_bgemm(int wdtype, int mode, int fm, int fn, const GemvArgs& a, dim3 grid, hipStream_t s) {
  if (wdtype != CP_SPEC_BF16) return hipErrorInvalidValue;
  if (fm == 1 && fn == 4) return launch_f<1, 4>(mode, a, grid, s);
  if (fm == 2 && fn == 4) return launch_f<2, 4>(mode, a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace cps
