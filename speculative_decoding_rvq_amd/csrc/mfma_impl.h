// Skinny GEMM on the matrix cores for many activation rows (batched streams).
//
// C[m][n] = sum_k x_m[k] * W[n][k] for M activation rows (M = streams x rows),
// W row-major [out][in].  Block tile 64 x 64, four waves of 32 x 32 (2 x 2
// MFMA tiles of 16 x 16), K in steps of 32 staged through LDS.
//
// fp32 weights: v_mfma_f32_16x16x4_f32; within a 32-wide K step lane group g
// supplies k = 8g + s to sub-step s, so a lane reads eight consecutive k of
// its row with two 16-byte LDS loads.
// bf16 weights: v_mfma_f32_16x16x32_bf16.  The activations stay float32: each
// x is split into three bf16 pieces hi + mid + lo that add up to x exactly
// (8 + 8 + 8 significant bits), and the tile runs three MFMAs, one per piece,
// into the same fp32 accumulator.  Every product is exact in fp32, so the
// result is the fp32 dot product up to summation order.
//
// RMSNorm: x * g is staged; the rows' sums of squares are accumulated while
// staging and 1/sqrt(mean + eps) scales the outputs.  Epilogue through an LDS
// copy of the C tile: residual add, SwiGLU (columns 0..31 of a tile are gate
// rows f0..f0+31, columns 32..63 the matching up rows), Q write plus K/V
// append at the row's position, or lm_head logits for rows grouped by head.
#pragma once

#include <type_traits>

#include "dev_common.h"
#include "kernels.h"

namespace cps {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTM = kMfmaTM, kTN = kMfmaTN, kTK = kMfmaTK;

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Output slot n of the launch -> weight row (mode dependent).  SwiGLU tiles of
// TN columns hold TN/2 gate rows then the TN/2 matching up rows.
template <typename WT, int MODE, int TN = kMfmaTN>
__device__ __forceinline__ const WT* gemm_weight_row(const GemvArgs& a, const WT* W0, int n) {
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

// Final-normed activation rows for the heads' caller (x * g * rinv): the
// column tiles of a row tile split K between them, float4 at a time, so each
// block writes a short slice.
__device__ __forceinline__ void write_xnorm(const GemvArgs& a, const int* rows_s, const float* rinv_s,
                                            int count) {
  const int k4 = a.K / 4;
  const int per = (k4 + gridDim.x - 1) / gridDim.x;
  const int c0 = blockIdx.x * per, c1 = min(k4, c0 + per);
  const int w = c1 - c0;
  if (w <= 0) return;
  for (int idx = threadIdx.x; idx < count * w; idx += kBlock) {
    const int r = idx / w, c = 4 * (c0 + idx % w);
    const int row = rows_s[r];
    if (row % a.xdiv != 0) continue;  // one writer per X row
    const float4 x = *reinterpret_cast<const float4*>(a.X + static_cast<size_t>(row / a.xdiv) * a.ldx + c);
    const float4 g = *reinterpret_cast<const float4*>(a.norm_g + c);
    const float ri = rinv_s[r];
    *reinterpret_cast<float4*>(a.xnorm_out + static_cast<size_t>(row / a.xdiv) * a.K + c) =
        make_float4(x.x * g.x * ri, x.y * g.y * ri, x.z * g.z * ri, x.w * g.w * ri);
  }
}

// lm_head rows m with k = m % xdiv in 1..hbK: head j+1 applied to draft
// offset b_k (added to the row's logits); 0 otherwise.
__device__ __forceinline__ float head_bias(const GemvArgs& a, int j, int row, int o) {
  const int k = row % a.xdiv;
  if (a.hb == nullptr || k < 1 || k > a.hbK) return 0.0f;
  return a.hb[(static_cast<size_t>(j) * a.hbK + (k - 1)) * a.N + o];
}

struct GemmSmemF32 {
  float A[kTM][kTK + 4];
  float B[kTN][kTK + 4];
};
struct GemmSmemBF16 {
  uint16_t A[3][kTM][kTK + 8];
  uint16_t B[kTN][kTK + 8];
};

template <typename WT, int MODE>
__global__ __launch_bounds__(kBlock) void mfma_gemm_kernel(const GemvArgs a) {
  constexpr bool kBf16 = sizeof(WT) == 2;
  using Smem = typename std::conditional<kBf16, GemmSmemBF16, GemmSmemF32>::type;
  __shared__ union {
    Smem s;
    float C[kTM][kTN + 1];
  } sm;
  __shared__ int rows_s[kTM];  // global activation row of each tile row (-1: none)
  __shared__ float rinv_s[kTM];
  __shared__ float ssq[kTM][4];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kTN;

  // ---- which activation rows this tile covers ----
  const WT* W0 = static_cast<const WT*>(a.W0);
  int count;
  if (MODE == kHead) {
    const int j = blockIdx.z;  // head j+1: its rows, ascending, slice blockIdx.y
    __shared__ int red_h[4];
    count = head_rows_slice(a.head, a.M, j + 1, blockIdx.y * kTM, kTM, rows_s, red_h);
    if (count <= 0) return;
    W0 = W0 + static_cast<size_t>(j) * static_cast<size_t>(a.head_stride);
  } else {
    const int m0 = blockIdx.y * kTM;
    count = min(kTM, a.M - m0);
    if (tid < kTM) rows_s[tid] = tid < count ? m0 + tid : -1;
  }
  __syncthreads();

  // staging roles: thread t -> tile row t/4, k sub-range (t%4)*8 .. +7
  const int sr = tid >> 2, sk = (tid & 3) * 8;
  const int arow = rows_s[sr];
  const float* xrow = arow >= 0 ? a.X + static_cast<size_t>(arow / a.xdiv) * a.ldx : nullptr;
  const WT* wrow = gemm_weight_row<WT, MODE>(a, W0, n0 + sr);
  const bool norm = a.norm_g != nullptr;
  float ss = 0.0f;

  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nsteps = a.K / kTK;
  // global -> register prefetch of one K step
  float4 xa0, xa1;
  typename std::conditional<kBf16, uint4, float4>::type wb0, wb1;
  auto fetch = [&](int step) {
    const int k = step * kTK + sk;
    if (xrow) {
      xa0 = *reinterpret_cast<const float4*>(xrow + k);
      xa1 = *reinterpret_cast<const float4*>(xrow + k + 4);
    } else {
      xa0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      xa1 = xa0;
    }
    if constexpr (kBf16) {
      wb0 = *reinterpret_cast<const uint4*>(wrow + k);
    } else {
      wb0 = *reinterpret_cast<const float4*>(wrow + k);
      wb1 = *reinterpret_cast<const float4*>(wrow + k + 4);
    }
  };
  fetch(0);
  for (int step = 0; step < nsteps; ++step) {
    // ---- registers -> LDS (activation * gain, split into pieces for bf16) ----
    float x[8] = {xa0.x, xa0.y, xa0.z, xa0.w, xa1.x, xa1.y, xa1.z, xa1.w};
    const int kg = step * kTK + sk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss += x[e] * x[e];
      if (norm) x[e] *= a.norm_g[kg + e];
    }
    __syncthreads();  // previous step's fragments have been read
    if constexpr (kBf16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = bf16_rne_bits(x[e]);
        const float r1 = x[e] - __uint_as_float(h << 16);
        const uint32_t m = bf16_rne_bits(r1);
        const float r2 = r1 - __uint_as_float(m << 16);
        sm.s.A[0][sr][sk + e] = static_cast<uint16_t>(h);
        sm.s.A[1][sr][sk + e] = static_cast<uint16_t>(m);
        sm.s.A[2][sr][sk + e] = static_cast<uint16_t>(__float_as_uint(r2) >> 16);  // exact
      }
      *reinterpret_cast<uint4*>(&sm.s.B[sr][sk]) = wb0;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.s.A[sr][sk + e] = x[e];
      *reinterpret_cast<float4*>(&sm.s.B[sr][sk]) = wb0;
      *reinterpret_cast<float4*>(&sm.s.B[sr][sk + 4]) = wb1;
    }
    __syncthreads();
    if (step + 1 < nsteps) fetch(step + 1);
    // ---- MFMAs of this step ----
    if constexpr (kBf16) {
      bf16x8 af[2][3], bfr[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
          af[mt][pc] = *reinterpret_cast<const bf16x8*>(&sm.s.A[pc][wm * 32 + mt * 16 + li][lg * 8]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        bfr[nt] = *reinterpret_cast<const bf16x8*>(&sm.s.B[wn * 32 + nt * 16 + li][lg * 8]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int pc = 0; pc < 3; ++pc)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt][pc], bfr[nt], acc[mt][nt], 0, 0, 0);
    } else {
      float av[2][8], bv[2][8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const float4 p0 = *reinterpret_cast<const float4*>(&sm.s.A[wm * 32 + mt * 16 + li][lg * 8]);
        const float4 p1 = *reinterpret_cast<const float4*>(&sm.s.A[wm * 32 + mt * 16 + li][lg * 8 + 4]);
        av[mt][0] = p0.x; av[mt][1] = p0.y; av[mt][2] = p0.z; av[mt][3] = p0.w;
        av[mt][4] = p1.x; av[mt][5] = p1.y; av[mt][6] = p1.z; av[mt][7] = p1.w;
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float4 p0 = *reinterpret_cast<const float4*>(&sm.s.B[wn * 32 + nt * 16 + li][lg * 8]);
        const float4 p1 = *reinterpret_cast<const float4*>(&sm.s.B[wn * 32 + nt * 16 + li][lg * 8 + 4]);
        bv[nt][0] = p0.x; bv[nt][1] = p0.y; bv[nt][2] = p0.z; bv[nt][3] = p0.w;
        bv[nt][4] = p1.x; bv[nt][5] = p1.y; bv[nt][6] = p1.z; bv[nt][7] = p1.w;
      }
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mt][s], bv[nt][s], acc[mt][nt], 0, 0, 0);
    }
  }

  // ---- per-row 1/rms (the four staging threads of a row hold partial sums) ----
  if (norm) {
    ssq[sr][tid & 3] = ss;
    __syncthreads();
    if (tid < kTM)
      rinv_s[tid] = 1.0f / sqrtf((ssq[tid][0] + ssq[tid][1] + ssq[tid][2] + ssq[tid][3]) /
                                     static_cast<float>(a.K) + a.eps);
  }
  __syncthreads();  // all fragment reads done: the staging area becomes C
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm.C[wm * 32 + mt * 16 + lg * 4 + i][wn * 32 + nt * 16 + li] = acc[mt][nt][i];
  __syncthreads();

  // final-normed rows for the heads' caller (once per row, by the first n tile)
  if (MODE == kHead && norm && a.xnorm_out != nullptr) write_xnorm(a, rows_s, rinv_s, count);

  // ---- fused epilogue ----
  if (MODE == kSwiGLU) {
    for (int idx = tid; idx < kTM * (kTN / 2); idx += kBlock) {
      const int r = idx / (kTN / 2), c = idx % (kTN / 2);
      const int row = rows_s[r];
      if (row < 0) continue;
      float g = sm.C[r][c], u = sm.C[r][c + kTN / 2];
      if (norm) {
        g *= rinv_s[r];
        u *= rinv_s[r];
      }
      const float sg = g / (1.0f + expf(-g));
      a.Y[static_cast<size_t>(row) * a.ldy + blockIdx.x * (kTN / 2) + c] = sg * u;
    }
    return;
  }
  for (int idx = tid; idx < kTM * kTN; idx += kBlock) {
    const int r = idx / kTN, c = idx % kTN;
    const int row = rows_s[r];
    if (row < 0) continue;
    float val = sm.C[r][c];
    if (norm) val *= rinv_s[r];
    const int o = n0 + c;
    if (MODE == kAdd) {
      a.Y[static_cast<size_t>(row) * a.ldy + o] += val;
    } else if (MODE == kHead) {
      a.Y[static_cast<size_t>(row) * a.ldy + o] = val + head_bias(a, blockIdx.z, row, o);
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

template <typename WT>
hipError_t launch_mfma_t(int mode, const GemvArgs& a, dim3 grid, hipStream_t s) {
  switch (mode) {
    case kAdd: hipLaunchKernelGGL((mfma_gemm_kernel<WT, kAdd>), grid, dim3(kBlock), 0, s, a); break;
    case kSwiGLU: hipLaunchKernelGGL((mfma_gemm_kernel<WT, kSwiGLU>), grid, dim3(kBlock), 0, s, a); break;
    case kQKV: hipLaunchKernelGGL((mfma_gemm_kernel<WT, kQKV>), grid, dim3(kBlock), 0, s, a); break;
    case kHead: hipLaunchKernelGGL((mfma_gemm_kernel<WT, kHead>), grid, dim3(kBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K variant for problems with few output tiles (small hidden sizes, few
// rows per head): a block owns a (16 FM) x (16 FN) tile and its four waves
// take a quarter of K each, reading their fragments straight from global
// memory (lane l: row l % 16, k = 8 (l / 16) .. +7 of each 32-wide chunk, the
// same k assignment as above) with up to U chunks in flight.  The partial
// tiles and the rows' partial sums of squares meet in LDS and are added in a
// fixed order, so the result does not depend on timing.
template <typename WT, int MODE, int FM, int FN>
__global__ __launch_bounds__(kBlock) void mfma_splitk_kernel(const GemvArgs a) {
  constexpr bool kBf16 = sizeof(WT) == 2;
  constexpr int TM = 16 * FM, TN = 16 * FN;
  constexpr int U = FM + FN >= 3 ? 2 : 4;
  constexpr int kWaves = kBlock / kWave;
  __shared__ float part[kWaves][TM][TN + 1];
  __shared__ float ssq_s[kWaves][TM];
  __shared__ float rinv_s[TM];
  __shared__ int rows_s[TM];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * TN;

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

  const float* xr[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int row = rows_s[16 * f + li];
    xr[f] = row >= 0 ? a.X + static_cast<size_t>(row / a.xdiv) * a.ldx : nullptr;
  }
  const WT* wr[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) wr[f] = gemm_weight_row<WT, MODE, TN>(a, W0, n0 + 16 * f + li);
  const bool norm = a.norm_g != nullptr;

  const int kw = a.K / kWaves;            // this wave's K range
  const int kbeg = wave * kw + 8 * lg;    // lane's first k
  const int nch = kw / kTK;

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float ss[FM];
#pragma unroll
  for (int f = 0; f < FM; ++f) ss[f] = 0.0f;

  using WV = typename std::conditional<kBf16, uint4, float4>::type;
  constexpr int kWV = kBf16 ? 1 : 2;  // 16-byte weight loads per chunk and fragment
  for (int c0 = 0; c0 < nch; c0 += U) {
    float4 xa[U][FM][2];
    WV wb[U][FN][kWV];
    float4 ga[U][2];
    // ---- issue every load of the group ----
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u >= nch) break;
      const int k = kbeg + (c0 + u) * kTK;
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int v = 0; v < kWV; ++v) wb[u][f][v] = *reinterpret_cast<const WV*>(wr[f] + k + v * (8 / kWV));
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        if (xr[f]) {
          xa[u][f][0] = *reinterpret_cast<const float4*>(xr[f] + k);
          xa[u][f][1] = *reinterpret_cast<const float4*>(xr[f] + k + 4);
        } else {
          xa[u][f][0] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          xa[u][f][1] = xa[u][f][0];
        }
      }
      if (norm) {
        ga[u][0] = *reinterpret_cast<const float4*>(a.norm_g + k);
        ga[u][1] = *reinterpret_cast<const float4*>(a.norm_g + k + 4);
      }
    }
    // ---- MFMAs of the group ----
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u >= nch) break;
      const float g[8] = {ga[u][0].x, ga[u][0].y, ga[u][0].z, ga[u][0].w,
                          ga[u][1].x, ga[u][1].y, ga[u][1].z, ga[u][1].w};
      float x[FM][8];
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const float4 p0 = xa[u][f][0], p1 = xa[u][f][1];
        x[f][0] = p0.x; x[f][1] = p0.y; x[f][2] = p0.z; x[f][3] = p0.w;
        x[f][4] = p1.x; x[f][5] = p1.y; x[f][6] = p1.z; x[f][7] = p1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ss[f] += x[f][e] * x[f][e];
          if (norm) x[f][e] *= g[e];
        }
      }
      if constexpr (kBf16) {
        bf16x8 ap[FM][3];
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t h = bf16_rne_bits(x[f][e]);
            const float r1 = x[f][e] - __uint_as_float(h << 16);
            const uint32_t mm = bf16_rne_bits(r1);
            const float r2 = r1 - __uint_as_float(mm << 16);
            ap[f][0][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(h));
            ap[f][1][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(mm));
            ap[f][2][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(__float_as_uint(r2) >> 16));
          }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const bf16x8 bw = __builtin_bit_cast(bf16x8, wb[u][fn][0]);
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int pc = 0; pc < 3; ++pc)
              acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap[fm][pc], bw, acc[fm][fn], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const float4 q0 = wb[u][fn][0], q1 = wb[u][fn][1];
          const float w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
          for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
              acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[fm][s], w[s], acc[fm][fn], 0, 0, 0);
        }
      }
    }
  }

  // ---- partial tiles and sums of squares -> LDS ----
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][16 * fm + 4 * lg + i][16 * fn + li] = acc[fm][fn][i];
  if (norm) {
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      float t = ss[f];
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      if (lg == 0) ssq_s[wave][16 * f + li] = t;
    }
  }
  __syncthreads();
  if (norm && tid < TM) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += ssq_s[w][tid];
    rinv_s[tid] = 1.0f / sqrtf(t / static_cast<float>(a.K) + a.eps);
  }
  __syncthreads();

  if (MODE == kHead && norm && a.xnorm_out != nullptr) write_xnorm(a, rows_s, rinv_s, count);
  auto tile_val = [&](int r, int c) {
    float v = part[0][r][c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += part[w][r][c];
    return norm ? v * rinv_s[r] : v;
  };
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
      a.Y[static_cast<size_t>(row) * a.ldy + o] = val + head_bias(a, blockIdx.z, row, o);
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

template <typename WT, int FM, int FN>
hipError_t launch_splitk_mode(int mode, const GemvArgs& a, dim3 grid, hipStream_t s) {
  switch (mode) {
    case kAdd: hipLaunchKernelGGL((mfma_splitk_kernel<WT, kAdd, FM, FN>), grid, dim3(kBlock), 0, s, a); break;
    case kSwiGLU: hipLaunchKernelGGL((mfma_splitk_kernel<WT, kSwiGLU, FM, FN>), grid, dim3(kBlock), 0, s, a); break;
    case kQKV: hipLaunchKernelGGL((mfma_splitk_kernel<WT, kQKV, FM, FN>), grid, dim3(kBlock), 0, s, a); break;
    case kHead: hipLaunchKernelGGL((mfma_splitk_kernel<WT, kHead, FM, FN>), grid, dim3(kBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// tile: 0 = 64 x 64 LDS-staged, 1 = 32 x 32 split-K, 2 = 16 x 16 split-K
template <typename WT>
hipError_t launch_mfma_t(int mode, int tile, const GemvArgs& a, dim3 grid, hipStream_t s) {
  switch (tile) {
    case 0: return launch_mfma_t<WT>(mode, a, grid, s);
    case 1: return launch_splitk_mode<WT, 2, 2>(mode, a, grid, s);
    case 2: return launch_splitk_mode<WT, 1, 1>(mode, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cps