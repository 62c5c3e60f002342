// Skinny matrix-vector kernel for few activation rows (one stream: M <= 8).
//
// Y[m][o] = sum_k W[o][k] * x_m[k], W row-major [out][in] in fp32 or bf16.
//
// Work layout: a row group of KT threads (64, 128 or 256) covers the whole K
// of RPG weight rows; thread kt owns 16-byte chunks kt, kt+KT, ... of each
// row, so a row is read by KT consecutive lanes (coalesced).  A block has
// 256 / KT row groups.  The thread keeps the matching slices of the M
// activation rows in registers, so every weight byte is loaded once and used
// for M fused multiply-adds.
//
// Latency: the activation rows are loaded first, then the weights of the
// block's first unit.  RMSNorm's 1/sqrt(mean+eps) is a
// per-row scalar applied to the dot products in the epilogue, so the rows'
// sums of squares are reduced together with the dot products: partial sums
// are folded within DPP rows of 16 lanes (four rotations) and across rows and
// waves through LDS, behind a single barrier.  The epilogue is fused:
// residual add, SwiGLU product (gate and up partials summed by one thread),
// Q write plus K/V append at the row's position, per-row lm_head logits (with
// the final-normed hidden state written once).
#pragma once

#include "dev_common.h"
#include "kernels.h"

namespace cps {


// Sum over the 16 lanes of each DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kRor8>(v);
  v += dpp_f<kRor4>(v);
  v += dpp_f<kRor2>(v);
  v += dpp_f<kRor1>(v);
  return v;
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// Weight row read for output slot `o` of the launch.
template <typename WT, int MODE, int RPG>
__device__ __forceinline__ const WT* weight_row(const GemvArgs& a, const WT* W0, int o) {
  if (MODE == kQKV) {
    const WT* W1 = static_cast<const WT*>(a.W1);
    const WT* W2 = static_cast<const WT*>(a.W2);
    if (o < a.qdim) return W0 + static_cast<size_t>(o) * a.K;
    if (o < a.qdim + a.kvdim) return W1 + static_cast<size_t>(o - a.qdim) * a.K;
    return W2 + static_cast<size_t>(o - a.qdim - a.kvdim) * a.K;
  }
  if (MODE == kSwiGLU) {
    // unit u covers outputs u*H2 .. u*H2+H2-1 (H2 = RPG/2): slots below H2
    // are gate rows, the rest the matching up rows
    constexpr int H2 = RPG / 2;
    const WT* W1 = static_cast<const WT*>(a.W1);
    const int u = o / RPG, rp = o % RPG;
    const int f = u * H2 + (rp % H2);
    return (rp < H2 ? W0 : W1) + static_cast<size_t>(f) * a.K;
  }
  return W0 + static_cast<size_t>(o) * a.K;
}

// Where a block's activation rows come from.  The default reads row m / xdiv
// of a.X and a K/V append's position from a.pos; a custom source (kCustom)
// provides prepare() (called by every thread once the first weights are in
// flight), load(m, k, x): the VEC values of the block's row m from column k,
// and pos(m), for the rows m0 .. m0 + MT - 1 of a launch with one row tile
// per block row.
struct XRows {
  static constexpr bool kCustom = false;
  __device__ void prepare() const {}
  template <int VEC>
  __device__ void load(int, int, float4 (&)[VEC / 4]) const {}
  __device__ int pos(int) const { return -1; }
};

// One block of the GEMV: block (bx, by) of a grid gdx blocks wide (after any
// remapping).  WT weight type, MODE epilogue, MT activation rows per tile,
// SPT 16-byte chunks per thread per row.
template <typename WT, int MODE, int MT, int SPT, typename Rows>
__device__ __forceinline__ void gemv_block(const GemvArgs& a, int bx, int by, int gdx, const Rows& rows) {
  using C = Chunk<WT>;
  using VT = typename C::T;
  constexpr int VEC = C::N;
  constexpr int RPG = gemv_rpg(SPT);
  constexpr int NV = RPG * MT;
  // per DPP row: NV dot-product partials, then MT sums of squares (RMSNorm)
  __shared__ float part[kBlock / 16][NV + MT];

  const int KT = a.kt;
  const int RG = kBlock / KT;
  const int rows16 = KT / 16;  // DPP rows per row group
  const int tid = threadIdx.x;
  const int rg = tid / KT, kt = tid % KT;
  const int lane = tid % kWave;
  const int m0 = MODE == kHeadG ? 0 : by * MT;
  if (MODE != kHeadG && a.M - m0 <= 0) return;

  const WT* W0 = static_cast<const WT*>(a.W0);
  // kHeadG: the block's rows are slice q of the rows of head j + 1
  __shared__ int rows_s[MODE == kHeadG ? MT : 1];
  int hsel = 0;  // the block's head (lm_head modes)
  if (MODE == kHead) {
    hsel = a.head[m0];
    if (hsel <= 0 || hsel > a.n_heads) return;
  }
  int Mg = 0;
  if (MODE == kHeadG) {
    __shared__ int red_g[kBlock / kWave];
    const int j = blockIdx.y / a.hslices, q = blockIdx.y % a.hslices;
    Mg = head_rows_slice(a.head, a.M, j + 1, q * MT, MT, rows_s, red_g);
    if (Mg <= 0) return;
    hsel = j + 1;
  }
  if (MODE == kHead || MODE == kHeadG)
    W0 = W0 + static_cast<size_t>(hsel - 1) * static_cast<size_t>(a.head_stride);
  // activation row m of the block
  auto row_of = [&](int m) { return MODE == kHeadG ? rows_s[m] : m0 + m; };
  const int Mloc = MODE == kHeadG ? Mg : min(MT, a.M - m0);
  const int stride = gdx * RG;
  int ubase = bx * RG;

  // ---- the activation rows first, then the first unit's weights: the rows
  // were written by the previous kernel and come back from the memory side
  // of the L2, so their round trip overlaps the weight stream (issued the
  // other way round, every projection took 0.5-1.2 us longer).  The gain is
  // read once per chunk, not once per row: every vector memory instruction
  // counts at one stream, more than the bytes it moves. ----
  const bool norm = a.norm_g != nullptr;
  VT wv[RPG][SPT];
  auto load_first_weights = [&]() __attribute__((always_inline)) {
    const int u = min(ubase + rg, a.units - 1);
#pragma unroll
    for (int rp = 0; rp < RPG; ++rp) {
      const WT* wr = weight_row<WT, MODE, RPG>(a, W0, u * RPG + rp);
#pragma unroll
      for (int j = 0; j < SPT; ++j) wv[rp][j] = *reinterpret_cast<const VT*>(wr + (kt + KT * j) * VEC);
    }
  };
  if constexpr (Rows::kCustom) {
    // a custom source finds its rows first (prepare: loads and a barrier),
    // so the weights go out before it
    load_first_weights();
    __builtin_amdgcn_sched_barrier(0);
    rows.prepare();
  }
  float4 xv[MT][SPT][VEC / 4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        if constexpr (Rows::kCustom) {
          if (e == 0) rows.template load<VEC>(m, (kt + KT * j) * VEC, xv[m][j]);
        } else {
          xv[m][j][e / 4] =
              m < Mloc ? *reinterpret_cast<const float4*>(a.X + static_cast<size_t>(row_of(m) / a.xdiv) * a.ldx +
                                                          (kt + KT * j) * VEC + e)
                       : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
  if constexpr (Rows::kCustom) {
    // block column 0 also leaves the rows in a.X (the round's row buffer:
    // the residual stream the later projections add to)
    if (bx == 0 && rg == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < Mloc) {
#pragma unroll
          for (int j = 0; j < SPT; ++j)
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
              *reinterpret_cast<float4*>(const_cast<float*>(a.X) + static_cast<size_t>(m0 + m) * a.ldx +
                                         (kt + KT * j) * VEC + e) = xv[m][j][e / 4];
        }
    }
  }
  float4 gv[SPT][VEC / 4];
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      gv[j][e / 4] = norm ? *reinterpret_cast<const float4*>(a.norm_g + (kt + KT * j) * VEC + e)
                          : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!Rows::kCustom) load_first_weights();
  __builtin_amdgcn_sched_barrier(0);
  float xr[MT][SPT][VEC];
  float ss[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    ss[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const float4 v = xv[m][j][e / 4], g = gv[j][e / 4];
        ss[m] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        xr[m][j][e] = v.x * g.x;
        xr[m][j][e + 1] = v.y * g.y;
        xr[m][j][e + 2] = v.z * g.z;
        xr[m][j][e + 3] = v.w * g.w;
      }
  }

  // thread (g, idx) of the epilogue owns slot idx / MT of unit g, row idx % MT
  const bool owner = tid < RG * NV;
  const int g = owner ? tid / NV : 0, idx = owner ? tid % NV : 0;
  float ri = 1.0f;  // 1/rms of the owner's row, known after the first reduction

  // epilogue operands that do not depend on the dot products (the residual
  // value of a residual add, the row's position of a K/V append), loaded
  // with the unit's weights rather than after the reduction
  float yold = 0.0f, yold_n = 0.0f;
  int ppos = -1, ppos_n = -1;
  auto epi_load = [&](int ub, float& y, int& pp) {
    const int rp = idx / MT, m = idx % MT, u = ub + g;
    if (!owner || u >= a.units || m >= Mloc) return;
    const int row = m0 + m;
    if (MODE == kAdd) y = a.Y[static_cast<size_t>(row) * a.ldy + u * RPG + rp];
    if (MODE == kQKV) pp = Rows::kCustom ? rows.pos(m) : a.pos[row];
  };
  epi_load(ubase, yold, ppos);

  // ---- units ----
  for (bool first = true; ubase < a.units; ubase += stride, first = false) {
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
    // next unit's weights go out before the reduction
    const int nb = ubase + stride;
    if (nb < a.units) {
      const int u = min(nb + rg, a.units - 1);
#pragma unroll
      for (int rp = 0; rp < RPG; ++rp) {
        const WT* wr = weight_row<WT, MODE, RPG>(a, W0, u * RPG + rp);
#pragma unroll
        for (int j = 0; j < SPT; ++j) wv[rp][j] = *reinterpret_cast<const VT*>(wr + (kt + KT * j) * VEC);
      }
      epi_load(nb, yold_n, ppos_n);
    }
    // fold 16 lanes per DPP row (dot products and, the first time, the sums
    // of squares), then the DPP rows of the row group in LDS: one barrier
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = row16_sum(v[i]);
    if (first && norm) {
#pragma unroll
      for (int m = 0; m < MT; ++m) ss[m] = row16_sum(ss[m]);
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) part[tid >> 4][i] = v[i];
      if (first && norm) {
#pragma unroll
        for (int m = 0; m < MT; ++m) part[tid >> 4][NV + m] = ss[m];
      }
    }
    __syncthreads();
    if (first && norm) {
      // every row group holds a full copy of each row: row group 0's sums
      if (owner) {
        float t = 0.0f;
        for (int q = 0; q < rows16; ++q) t += part[q][NV + idx % MT];
        ri = 1.0f / sqrtf(t / static_cast<float>(a.K) + a.eps);
      }
      if ((MODE == kHead || MODE == kHeadG) && a.xnorm_out != nullptr && bx == 0 && rg == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m >= Mloc || row_of(m) % a.xdiv != 0) continue;
          float t = 0.0f;
          for (int q = 0; q < rows16; ++q) t += part[q][NV + m];
          const float r0 = 1.0f / sqrtf(t / static_cast<float>(a.K) + a.eps);
          float* dst = a.xnorm_out + static_cast<size_t>(row_of(m) / a.xdiv) * a.K;
#pragma unroll
          for (int j = 0; j < SPT; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) dst[(kt + KT * j) * VEC + e] = xr[m][j][e] * r0;
        }
      }
    }
    // ---- fused epilogue ----
    if (owner) {
      const int rp = idx / MT, m = idx % MT;
      const int u = ubase + g;
      if (MODE == kSwiGLU) {
        // slots below RPG/2 are gate values, the rest the matching up values
        constexpr int H2 = RPG / 2;
        if (rp < H2 && u < a.units && m < Mloc) {
          const int iu = (rp + H2) * MT + m;
          float gate = 0.0f, up = 0.0f;
          for (int q = 0; q < rows16; ++q) {
            gate += part[g * rows16 + q][idx];
            up += part[g * rows16 + q][iu];
          }
          a.Y[static_cast<size_t>(m0 + m) * a.ldy + H2 * u + rp] = silu_f(gate * ri) * (up * ri);
        }
      } else if (u < a.units && m < Mloc) {
        float val = 0.0f;
        for (int q = 0; q < rows16; ++q) val += part[g * rows16 + q][idx];
        val *= ri;
        const int o = u * RPG + rp;
        const int row = row_of(m);
        if (MODE == kAdd) {
          a.Y[static_cast<size_t>(row) * a.ldy + o] = yold + val;
        } else if (MODE == kHead || MODE == kHeadG) {
          const int k = row % a.xdiv;
          if (a.hb != nullptr && k >= 1 && k <= a.hbK)
            val += a.hb[(static_cast<size_t>(hsel - 1) * a.hbK + (k - 1)) * a.N + o];
          a.Y[static_cast<size_t>(row) * a.ldy + o] = val;
        } else if (MODE == kStore) {
          a.Y[static_cast<size_t>(row) * a.ldy + o] = val;
        } else if (MODE == kQKV) {
          if (o < a.qdim) {
            a.Y[static_cast<size_t>(row) * a.ldy + o] = val;
          } else {
            const int pp = ppos;
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
    yold = yold_n, ppos = ppos_n;
    if (nb < a.units) __syncthreads();  // part[] is rewritten by the next unit
  }
}

template <typename WT, int MODE, int MT, int SPT>
__global__ __launch_bounds__(kBlock) void gemv_kernel(const GemvArgs a) {
  // Several row tiles read the same weight rows.  Blocks go to the eight
  // XCDs in turn (linear id modulo 8): the row tiles of one weight slice are
  // given to consecutive blocks of one XCD, so all but the first read the
  // slice from that XCD's L2.
  int bx = blockIdx.x, by = blockIdx.y;
  if (MODE != kHeadG && gridDim.y > 1 && gridDim.x % 8 == 0) {
    const int L = blockIdx.x + gridDim.x * blockIdx.y;
    const int i = L / 8;
    by = i % gridDim.y;
    bx = (i / gridDim.y) * 8 + L % 8;
  }
  gemv_block<WT, MODE, MT, SPT>(a, bx, by, gridDim.x, XRows{});
}

// Host-side dispatch for one weight type: MT in {1, 2, 4, 8}, SPT in 1..4.
template <typename WT>
hipError_t launch_gemv_t(int mode, int mt, const GemvArgs& a, int grid_x, int grid_y, hipStream_t s) {
  constexpr int VEC = Chunk<WT>::N;
  const int spt = a.K / (VEC * a.kt);
  dim3 grid(grid_x, grid_y), block(kBlock);
#define CPS_GEMV_CASE(MODE_, MT_, SPT_)                                                 \
  if (mode == MODE_ && mt == MT_ && spt == SPT_) {                                      \
    hipLaunchKernelGGL((gemv_kernel<WT, MODE_, MT_, SPT_>), grid, block, 0, s, a);     \
    return hipGetLastError();                                                           \
  }
#define CPS_GEMV_SPT(MODE_, MT_) \
  CPS_GEMV_CASE(MODE_, MT_, 1)   \
  CPS_GEMV_CASE(MODE_, MT_, 2)   \
  CPS_GEMV_CASE(MODE_, MT_, 3)   \
  CPS_GEMV_CASE(MODE_, MT_, 4)
#define CPS_GEMV_MT(MODE_) \
  CPS_GEMV_SPT(MODE_, 1)   \
  CPS_GEMV_SPT(MODE_, 2)   \
  CPS_GEMV_SPT(MODE_, 4)   \
  CPS_GEMV_SPT(MODE_, 8)
  CPS_GEMV_MT(kAdd)
  CPS_GEMV_MT(kSwiGLU)
  CPS_GEMV_MT(kQKV)
  CPS_GEMV_SPT(kHead, 1)
  CPS_GEMV_SPT(kHeadG, 2)
  CPS_GEMV_SPT(kHeadG, 4)
  CPS_GEMV_SPT(kHeadG, 8)
#undef CPS_GEMV_MT
#undef CPS_GEMV_SPT
#undef CPS_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace cps
