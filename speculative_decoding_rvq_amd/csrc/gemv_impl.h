// Skinny matrix-vector kernel for few activation rows (one stream: M <= 8).
//
// Y[m][o] = sum_k W[o][k] * x_m[k] for the M activation rows x_m, with W
// row-major [out][in] in fp32 or bf16 (weights are streamed once per launch,
// 16 bytes per lane per load, consecutive lanes on consecutive chunks).
// Each workgroup keeps its M activation rows in registers (RMSNorm applied
// in the prologue when requested); thread kt of a row group owns K-chunks
// kt, kt+KT, ... so every weight row is read by KT lanes at once.  Partial
// sums of RPG output rows x MT activation rows are folded with a wave
// transpose-reduction (each shuffle halves the live values) and, when a row
// spans several waves, through LDS.  The epilogue is fused: residual add,
// SwiGLU gate/up product, Q write plus K/V append at the row's position, or
// per-row lm_head logits.
#pragma once

#include "dev_common.h"
#include "kernels.h"

namespace cps {

// Reduce NV values held by every lane of a wave.  Afterwards lane l holds
// the wave-wide sum of value l / (64 / NV) (for every lane of its group).
template <int NV>
__device__ __forceinline__ float wave_transpose_reduce(float (&v)[NV]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int s = 0; (NV >> s) > 1; ++s) {
    const int c = NV >> s;
    const int o = 32 >> s;
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < c / 2; ++i) {
      const float send = up ? v[i] : v[i + c / 2];
      const float keep = up ? v[i + c / 2] : v[i];
      v[i] = keep + __shfl_xor(send, o, kWave);
    }
  }
#pragma unroll
  for (int o = (kWave / NV) >> 1; o > 0; o >>= 1) v[0] += __shfl_xor(v[0], o, kWave);
  return v[0];
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

template <typename WT, int MODE, int MT, int SPT>
__global__ __launch_bounds__(kBlock) void gemv_kernel(const GemvArgs a) {
  using C = Chunk<WT>;
  using VT = typename C::T;
  constexpr int VEC = C::N;
  constexpr int RPG = kRPG;
  constexpr int NV = RPG * MT;
  static_assert(NV <= kWave, "too many partial sums per lane");
  __shared__ float part[4][NV];
  __shared__ float tot[4][NV];
  __shared__ float red[8];

  const int KT = a.kt;
  const int RG = kBlock / KT;
  const int tid = threadIdx.x;
  const int rg = tid / KT, kt = tid % KT;
  const int wave = tid / kWave, lane = tid % kWave;
  const int m0 = blockIdx.y * MT;
  const int Mloc = min(MT, a.M - m0);
  if (Mloc <= 0) return;

  const WT* W0 = static_cast<const WT*>(a.W0);
  const WT* W1 = static_cast<const WT*>(a.W1);
  const WT* W2 = static_cast<const WT*>(a.W2);
  if (MODE == kHead) {
    const int h = a.head[m0];
    if (h <= 0 || h > a.n_heads) return;
    W0 = W0 + static_cast<size_t>(h - 1) * static_cast<size_t>(a.head_stride);
  }

  // ---- activation rows into registers (optionally RMSNormed) ----
  float xr[MT][SPT][VEC];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int seg = kt + KT * j;
      if (m < Mloc) {
        const float* xp = a.X + static_cast<size_t>((m0 + m) / a.xdiv) * a.ldx + seg * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 v = *reinterpret_cast<const float4*>(xp + e);
          xr[m][j][e] = v.x; xr[m][j][e + 1] = v.y; xr[m][j][e + 2] = v.z; xr[m][j][e + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) xr[m][j][e] = 0.0f;
      }
    }
  }
  if (a.norm_g != nullptr) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss += xr[m][j][e] * xr[m][j][e];
      // every row group holds a full copy of the row: divide by RG
      const float total = block_sum(ss, red);
      const float rinv = 1.0f / sqrtf(total / static_cast<float>(RG * a.K) + a.eps);
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int k0 = (kt + KT * j) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) xr[m][j][e] = xr[m][j][e] * rinv * a.norm_g[k0 + e];
      }
    }
    if (a.xnorm_out != nullptr && blockIdx.x == 0 && rg == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < Mloc) {
#pragma unroll
          for (int j = 0; j < SPT; ++j) {
            float* op = a.xnorm_out + static_cast<size_t>(m0 + m) * a.K + (kt + KT * j) * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) op[e] = xr[m][j][e];
          }
        }
      }
    }
  }

  // ---- stream the weight rows ----
  const int stride = gridDim.x * RG;
  for (int ubase = blockIdx.x * RG; ubase < a.units; ubase += stride) {
    const int u = ubase + rg;
    const int uu = u < a.units ? u : a.units - 1;
    const WT* wr[RPG];
#pragma unroll
    for (int rp = 0; rp < RPG; ++rp) {
      if (MODE == kSwiGLU) {
        const int o = uu * (RPG / 2) + (rp % (RPG / 2));
        wr[rp] = (rp < RPG / 2 ? W0 : W1) + static_cast<size_t>(o) * a.K;
      } else if (MODE == kQKV) {
        const int o = uu * RPG + rp;
        if (o < a.qdim) wr[rp] = W0 + static_cast<size_t>(o) * a.K;
        else if (o < a.qdim + a.kvdim) wr[rp] = W1 + static_cast<size_t>(o - a.qdim) * a.K;
        else wr[rp] = W2 + static_cast<size_t>(o - a.qdim - a.kvdim) * a.K;
      } else {
        wr[rp] = W0 + static_cast<size_t>(uu * RPG + rp) * a.K;
      }
    }
    VT wv[RPG][SPT];
#pragma unroll
    for (int rp = 0; rp < RPG; ++rp)
#pragma unroll
      for (int j = 0; j < SPT; ++j)
        wv[rp][j] = *reinterpret_cast<const VT*>(wr[rp] + (kt + KT * j) * VEC);
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = 0.0f;
#pragma unroll
    for (int rp = 0; rp < RPG; ++rp)
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        float w[VEC];
        C::unpack(wv[rp][j], w);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[rp * MT + m] = fmaf(w[e], xr[m][j][e], v[rp * MT + m]);
      }

    const float r = wave_transpose_reduce<NV>(v);
    constexpr int LPV = kWave / NV;
    if ((lane % LPV) == 0) part[wave][lane / LPV] = r;
    __syncthreads();
    const int WPR = KT / kWave;
    if (tid < RG * NV) {
      const int g = tid / NV, idx = tid % NV;
      float s = 0.0f;
      for (int w = 0; w < WPR; ++w) s += part[g * WPR + w][idx];
      tot[g][idx] = s;
    }
    __syncthreads();

    // ---- fused epilogue ----
    if (MODE == kSwiGLU) {
      constexpr int NO = (RPG / 2) * MT;
      if (tid < RG * NO) {
        const int g = tid / NO, i = (tid % NO) / MT, m = tid % MT;
        const int ug = ubase + g;
        if (ug < a.units && m < Mloc) {
          const float gv = tot[g][i * MT + m];
          const float uv = tot[g][(i + RPG / 2) * MT + m];
          a.Y[static_cast<size_t>(m0 + m) * a.ldy + ug * (RPG / 2) + i] = silu_f(gv) * uv;
        }
      }
    } else if (tid < RG * NV) {
      const int g = tid / NV, rp = (tid % NV) / MT, m = tid % MT;
      const int ug = ubase + g;
      if (ug < a.units && m < Mloc) {
        const float val = tot[g][rp * MT + m];
        const int o = ug * RPG + rp;
        const int row = m0 + m;
        if (MODE == kAdd) {
          a.Y[static_cast<size_t>(row) * a.ldy + o] += val;
        } else if (MODE == kHead || MODE == kStore) {
          a.Y[static_cast<size_t>(row) * a.ldy + o] = val;
        } else if (MODE == kQKV) {
          if (o < a.qdim) {
            a.Y[static_cast<size_t>(row) * a.ldy + o] = val;
          } else {
            const int p = a.pos[row];
            if (p >= 0 && p < a.kv_positions) {
              const int b = row / a.rows_per_stream;
              float* base = a.kv + static_cast<size_t>(b) * a.kv_sb + static_cast<size_t>(p) * a.kvdim;
              const int oo = o - a.qdim;
              if (oo < a.kvdim) base[oo] = val;
              else base[a.kv_vo + (oo - a.kvdim)] = val;
            }
          }
        }
      }
    }
  }
}

// Host-side dispatch for one weight type.
template <typename WT>
hipError_t launch_gemv_t(int mode, int mt, const GemvArgs& a, int grid_x, int grid_y, hipStream_t s) {
  constexpr int VEC = Chunk<WT>::N;
  const int spt = a.K / (VEC * a.kt);
  dim3 grid(grid_x, grid_y), block(kBlock);
#define CPS_GEMV_CASE(MODE_, MT_, SPT_)                                         \
  if (mode == MODE_ && mt == MT_ && spt == SPT_) {                              \
    hipLaunchKernelGGL((gemv_kernel<WT, MODE_, MT_, SPT_>), grid, block, 0, s, a); \
    return hipGetLastError();                                                   \
  }
#define CPS_GEMV_SPT(MODE_, MT_) \
  CPS_GEMV_CASE(MODE_, MT_, 1)   \
  CPS_GEMV_CASE(MODE_, MT_, 2)   \
  CPS_GEMV_CASE(MODE_, MT_, 3)   \
  CPS_GEMV_CASE(MODE_, MT_, 4)
#define CPS_GEMV_MT(MODE_) \
  CPS_GEMV_SPT(MODE_, 2)   \
  CPS_GEMV_SPT(MODE_, 4)   \
  CPS_GEMV_SPT(MODE_, 8)
  CPS_GEMV_MT(kAdd)
  CPS_GEMV_MT(kSwiGLU)
  CPS_GEMV_MT(kQKV)
  CPS_GEMV_SPT(kHead, 1)
#undef CPS_GEMV_MT
#undef CPS_GEMV_SPT
#undef CPS_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace cps
