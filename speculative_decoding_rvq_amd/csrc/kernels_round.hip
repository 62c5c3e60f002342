// Attention, top-k softmax + sampling, acceptance and the round control
// kernels of CodePredictor speculative decoding.
#include <mutex>
#include <type_traits>

#include "dev_common.h"
#include "kernels.h"
#include "gemv_impl.h"
#include "topk_impl.h"
#include "accept_impl.h"

namespace cps {

hipError_t launch_gemv_f32(int mode, int mt, const GemvArgs& a, int gx, int gy, hipStream_t s);
hipError_t launch_gemv_bf16(int mode, int mt, const GemvArgs& a, int gx, int gy, hipStream_t s);

hipError_t launch_gemv(int wdtype, int mode, int mt, const GemvArgs& a, int grid_x, int grid_y,
                       hipStream_t s) {
  return wdtype == CP_SPEC_BF16 ? launch_gemv_bf16(mode, mt, a, grid_x, grid_y, s)
                                : launch_gemv_f32(mode, mt, a, grid_x, grid_y, s);
}

hipError_t launch_mfma_f32(int mode, int tile, const GemvArgs& a, dim3 grid, hipStream_t s);
hipError_t launch_mfma_bf16(int mode, int tile, const GemvArgs& a, dim3 grid, hipStream_t s);

hipError_t launch_mfma(int wdtype, int mode, int tile, const GemvArgs& a, dim3 grid, hipStream_t s) {
  return wdtype == CP_SPEC_BF16 ? launch_mfma_bf16(mode, tile, a, grid, s)
                                : launch_mfma_f32(mode, tile, a, grid, s);
}

// ---------------------------------------------------------------------------
// Causal attention over the in-frame positions of one stream and one KV head.
//
// Phase 1 loads (float4) K of positions 0..max row position, rotated by RoPE
// on the way into LDS, V, and the rotated queries of the group's (row, query
// head) pairs; a thread takes its items two at a time, both items' loads
// before either's stores, so one memory round trip covers them.  Phase 2: a
// 16-lane DPP row per pair, lane l scoring positions l and l + 16; the row's
// max and sum (DPP rotations) give the softmax weights (positions above the
// row's own are masked).  Phase 3: each thread produces four consecutive
// output dimensions of one pair.
template <int D>
__global__ __launch_bounds__(kBlock) void attention_kernel(const AttnArgs a) {
  extern __shared__ float smem[];
  constexpr int half = D / 2;
  constexpr int H4 = half / 4;  // float4s per half row
  constexpr int KS = D + 4;     // padded K row stride (rows on different banks)
  const int b = blockIdx.x, g = blockIdx.y;
  const int R = a.R;
  const int kvdim = a.nkv * D;
  const int qdim = a.nq * D;
  const int group = a.nq / a.nkv;
  const int npair = R * group;
  __shared__ int pos_s[CP_SPEC_MAX_WINDOW];
  if (threadIdx.x < R) pos_s[threadIdx.x] = a.pos[b * R + threadIdx.x];
  __syncthreads();
  int maxp = -1;
  for (int r = 0; r < R; ++r) maxp = max(maxp, pos_s[r]);
  if (maxp < 0 || maxp >= a.G) return;  // no active row, or outside the frame
  const int np = maxp + 1;
  float* Ks = smem;                  // [np][KS]
  float* Vs = Ks + a.G * KS;         // [np][D]
  float* Qs = Vs + a.G * D;          // [npair][D]
  float* S = Qs + npair * D;         // [npair][32]
  const float* kb = a.kv + static_cast<size_t>(b) * a.kv_sb + g * D;
  const float* vb = kb + a.kv_vo;

  // ---- phase 1: K (rotated), V, Q (rotated) into LDS; a thread's items
  // two at a time, both items' loads issued before either's stores ----
  const int nk = np * H4, nq = npair * H4;
  struct Item {
    float4 x1, x2, v1, v2, c01, c23;
  };
  auto load_item = [&](int it, Item& m) {
    if (it < nk) {
      const int p = it / H4, i4 = (it % H4) * 4;
      m.x1 = *reinterpret_cast<const float4*>(kb + p * kvdim + i4);
      m.x2 = *reinterpret_cast<const float4*>(kb + p * kvdim + i4 + half);
      m.v1 = *reinterpret_cast<const float4*>(vb + p * kvdim + i4);
      m.v2 = *reinterpret_cast<const float4*>(vb + p * kvdim + i4 + half);
      m.c01 = *reinterpret_cast<const float4*>(a.rope + p * half + i4);      // cos,sin x2
      m.c23 = *reinterpret_cast<const float4*>(a.rope + p * half + i4 + 2);
    } else if (it < nk + nq) {
      const int jt = it - nk;
      const int pr = jt / H4, i4 = (jt % H4) * 4;
      const int r = pr / group, j = pr % group;
      const float* qrow = a.Q + static_cast<size_t>(b * R + r) * qdim + (g * group + j) * D;
      const int pq = max(pos_s[r], 0);
      m.x1 = *reinterpret_cast<const float4*>(qrow + i4);
      m.x2 = *reinterpret_cast<const float4*>(qrow + i4 + half);
      m.c01 = *reinterpret_cast<const float4*>(a.rope + pq * half + i4);
      m.c23 = *reinterpret_cast<const float4*>(a.rope + pq * half + i4 + 2);
    }
  };
  auto store_item = [&](int it, const Item& m) {
    if (it >= nk + nq) return;
    int i4;
    float* dst;
    if (it < nk) {
      const int p = it / H4;
      i4 = (it % H4) * 4;
      dst = Ks + p * KS;
      *reinterpret_cast<float4*>(Vs + p * D + i4) = m.v1;
      *reinterpret_cast<float4*>(Vs + p * D + i4 + half) = m.v2;
    } else {
      const int jt = it - nk;
      i4 = (jt % H4) * 4;
      dst = Qs + (jt / H4) * D;
    }
    const float4 k1 = m.x1, k2 = m.x2, c01 = m.c01, c23 = m.c23;
    dst[i4 + 0] = k1.x * c01.x - k2.x * c01.y;  dst[i4 + half + 0] = k2.x * c01.x + k1.x * c01.y;
    dst[i4 + 1] = k1.y * c01.z - k2.y * c01.w;  dst[i4 + half + 1] = k2.y * c01.z + k1.y * c01.w;
    dst[i4 + 2] = k1.z * c23.x - k2.z * c23.y;  dst[i4 + half + 2] = k2.z * c23.x + k1.z * c23.y;
    dst[i4 + 3] = k1.w * c23.z - k2.w * c23.w;  dst[i4 + half + 3] = k2.w * c23.z + k1.w * c23.w;
  };
  for (int it = threadIdx.x; it < nk + nq; it += 2 * kBlock) {
    Item m0, m1;
    load_item(it, m0);
    load_item(it + kBlock, m1);
    store_item(it, m0);
    store_item(it + kBlock, m1);
  }
  __syncthreads();

  // ---- phase 2: scores and softmax.  32 lanes per pair (eight pairs per
  // block pass): lane l scores positions l % 16 and l % 16 + 16 over one
  // half of the head dimensions, the two halves meet by a lane exchange;
  // the row's max and sum fold by DPP rotations within each 16-lane row ----
  {
    const int l32 = threadIdx.x & 31, prow = threadIdx.x >> 5;
    const int l16 = l32 & 15, hd = l32 >> 4;
    for (int pr0 = 0; pr0 < npair; pr0 += kBlock / 32) {
      const int pr = pr0 + prow;
      const bool live_pair = pr < npair;
      const int pp = live_pair ? pos_s[pr / group] : -1;
      float sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = l16 + 16 * h;
        float part = 0.0f;
        if (p <= pp) {
          const float4* q4 = reinterpret_cast<const float4*>(Qs + pr * D + hd * half);
          const float4* k4 = reinterpret_cast<const float4*>(Ks + p * KS + hd * half);
          float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int i = 0; i < H4; ++i) {
            const float4 x = q4[i], y = k4[i];
            acc[0] = fmaf(x.x, y.x, acc[0]);
            acc[1] = fmaf(x.y, y.y, acc[1]);
            acc[2] = fmaf(x.z, y.z, acc[2]);
            acc[3] = fmaf(x.w, y.w, acc[3]);
          }
          part = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
        // lanes l and l ^ 16 hold the two halves of one score (same p, pp)
        const float other = __shfl_xor(part, 16);
        sc[h] = p <= pp ? (hd == 0 ? part + other : other + part) * a.scale : -INFINITY;
      }
      float mx = fmaxf(sc[0], sc[1]);
      mx = fmaxf(mx, dpp_f<kRor8>(mx));
      mx = fmaxf(mx, dpp_f<kRor4>(mx));
      mx = fmaxf(mx, dpp_f<kRor2>(mx));
      mx = fmaxf(mx, dpp_f<kRor1>(mx));
      const float e0 = l16 <= pp ? expf(sc[0] - mx) : 0.0f;
      const float e1 = l16 + 16 <= pp ? expf(sc[1] - mx) : 0.0f;
      float sum = e0 + e1;
      sum += dpp_f<kRor8>(sum);
      sum += dpp_f<kRor4>(sum);
      sum += dpp_f<kRor2>(sum);
      sum += dpp_f<kRor1>(sum);
      if (live_pair && pp >= 0 && hd == 0) {
        S[pr * 32 + l16] = e0 / sum;  // zero past the row's own position
        S[pr * 32 + l16 + 16] = e1 / sum;
      }
    }
  }
  __syncthreads();

  // ---- phase 3: four output dimensions of one pair per thread (fp32
  // rows, or their split pieces for the O projection).  Every row's weights
  // are zero past its own position, so all threads run the block's np
  // positions: a uniform trip count, unrolled, its LDS reads in flight
  // together ----
  constexpr int D4 = D / 4;
  for (int idx = threadIdx.x; idx < npair * D4; idx += kBlock) {
    const int pr = idx / D4, i4 = (idx % D4) * 4;
    const int r = pr / group, j = pr % group;
    const int pp = pos_s[r];
    if (pp < 0) continue;
    const float* srow = S + pr * 32;
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int p = 0; p < np; ++p) {
      const float w = srow[p];
      const float4 v = *reinterpret_cast<const float4*>(Vs + p * D + i4);
      o[0] = fmaf(w, v.x, o[0]);
      o[1] = fmaf(w, v.y, o[1]);
      o[2] = fmaf(w, v.z, o[2]);
      o[3] = fmaf(w, v.w, o[3]);
    }
    const int row = b * R + r, k = (g * group + j) * D + i4;
    if (a.planes != nullptr) {
      if (split_store4(a.planes, a.ptiles, row, k, o)) flag_overflow(a.ovf, nullptr, row);  // active rows only
    } else {
      *reinterpret_cast<float4*>(a.out + static_cast<size_t>(row) * qdim + k) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

size_t attention_smem_bytes(int G, int d, int R, int group) {
  const size_t npair = static_cast<size_t>(R) * group;
  return (static_cast<size_t>(G) * (2 * d + 4) + npair * d + npair * 32) * sizeof(float);
}

hipError_t attention_allow_smem(int d, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  switch (d) {
#define CPS_ATT_ATTR(D_) \
  case D_:               \
    return hipFuncSetAttribute(reinterpret_cast<const void*>(attention_kernel<D_>), \
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
    CPS_ATT_ATTR(8) CPS_ATT_ATTR(16) CPS_ATT_ATTR(32) CPS_ATT_ATTR(64) CPS_ATT_ATTR(128)
#undef CPS_ATT_ATTR
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnArgs& a, int B, hipStream_t s) {
  const size_t shm = attention_smem_bytes(a.G, a.d, a.R, a.nq / a.nkv);
  switch (a.d) {
#define CPS_ATT(D_)                                                                          \
  case D_:                                                                                   \
    hipLaunchKernelGGL(attention_kernel<D_>, dim3(B, a.nkv), dim3(kBlock), shm, s, a); \
    break;
    CPS_ATT(8) CPS_ATT(16) CPS_ATT(32) CPS_ATT(64) CPS_ATT(128)
#undef CPS_ATT
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void rmsnorm_rows_kernel(const float* x, float* y,
                                                              const float* g, int H, float eps) {
  __shared__ float red[8];
  const float* xr = x + static_cast<size_t>(blockIdx.x) * H;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < H; i += kBlock) ss += xr[i] * xr[i];
  const float tot = block_sum(ss, red);
  const float rinv = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
  float* yr = y + static_cast<size_t>(blockIdx.x) * H;
  for (int i = threadIdx.x; i < H; i += kBlock) yr[i] = xr[i] * rinv * g[i];
}

hipError_t launch_rmsnorm_rows(const float* x, float* y, const float* g, int rows, int H, float eps,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(rows), dim3(kBlock), 0, s, x, y, g, H, eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Component: n_rows independent rows.
__global__ __launch_bounds__(kBlock) void topk_rows_kernel(const TopkArgs a) {
  extern __shared__ float4 row_dyn[];
  __shared__ SelSmem S;
  __shared__ uint64_t red64[4];
  __shared__ uint32_t red32[4];
  const int r = blockIdx.x;
  const float* z = a.logits + static_cast<size_t>(r) * a.V;
  float* pr = a.probs ? a.probs + static_cast<size_t>(r) * a.V : nullptr;
  const bool samp = a.u != nullptr && !a.greedy;
  const float u = samp ? a.u[r] : 0.0f;
  dispatch_vpt(a.V, [&](auto vpt) {
    constexpr int VPT = decltype(vpt)::value;
    float zv[VPT];
    load_row<VPT>(z, zv);
    if (a.greedy) {
      const TopkResult res = argmax_regs<VPT>(zv, red64, red32);
      if (threadIdx.x == 0) {
        if (a.codes) a.codes[r] = res.code;
        if (a.flags) a.flags[r] = res.flags;
      }
      return;
    }
    const RowLds L = row_lds(row_dyn, a.V, false);
    store_row<VPT>(zv, L.z);
    int total;
    uint32_t flags = 0;
    if (!topk_list<VPT>(zv, a.k, a.T, L, S, pr, &total, &flags)) return;
    int code = -1, near = 0;
    if (samp) list_draw(L.lw, L.lidx, total, u, &code, &near);
    if (near) flags |= kFlagCdf;
    if (threadIdx.x == 0) {
      if (a.codes) a.codes[r] = code;
      if (a.flags) a.flags[r] = flags;
    }
  });
}

hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(a.n_rows), dim3(kBlock), row_lds_bytes(a.V, false), s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Component accept (cp_spec_accept, cp_spec_walk_step): the decode round's
// acceptance functions on caller data.  The caller hands over dense rows;
// the positive entries of p become the list walk_step reads (the decode
// round's target kernel hands it the top-k list, which holds the same
// positive entries in the same order).

// The positive entries of a dense row held in registers (thread t owning
// codes [t*VPT, (t+1)*VPT)) as a list in ascending code order: L.lw the
// weights, L.lidx the codes, zero from the count up to the next multiple of
// 32.  Every thread gets the count; the list is published by a barrier.
template <int VPT>
__device__ int dense_to_list(const float (&pv)[VPT], const RowLds& L, int* red) {
  const int base = threadIdx.x * VPT;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) cnt += pv[j] > 0.0f ? 1 : 0;
  int total;
  int off = block_exclusive_scan(cnt, red, &total);
#pragma unroll
  for (int j = 0; j < VPT; ++j)
    if (pv[j] > 0.0f) {
      L.lw[off] = pv[j];
      L.lidx[off] = static_cast<uint16_t>(base + j);
      ++off;
    }
  if (threadIdx.x < 32 && total + static_cast<int>(threadIdx.x) < ((total + 31) & ~31))
    L.lw[total + threadIdx.x] = 0.0f;
  lds_sync();
  return total;
}

// One block per (offset row r, stream b) of a chain round: row r < gamma
// tests draft r + 1, row gamma draws the bonus; greedy rows take their
// argmax.  tcode / tflags [B][W + 1] as the decode round's target kernel
// writes them.
__global__ __launch_bounds__(kBlock) void accept_rows_kernel(const AcceptArgs a) {
  extern __shared__ float4 row_dyn[];
  __shared__ uint64_t red64[4];
  __shared__ uint32_t red32[4];
  __shared__ int redi[4];
  const int r = blockIdx.x, b = blockIdx.y;
  const int W = a.W, V = a.V;
  const int gamma = min(max(a.gamma[b], 0), W);
  const size_t orow = static_cast<size_t>(b) * (W + 1) + r;
  if (r > gamma) {
    if (threadIdx.x == 0) {
      a.tcode[orow] = -1;
      a.tflags[orow] = 0u;
    }
    return;
  }
  dispatch_vpt(V, [&](auto vpt) {
    constexpr int VPT = decltype(vpt)::value;
    float pv[VPT];
    load_row<VPT>(a.p + orow * V, pv);
    if (a.greedy) {
      const TopkResult res = argmax_regs<VPT>(pv, red64, red32);
      if (threadIdx.x == 0) {
        a.tcode[orow] = res.code;
        a.tflags[orow] = res.flags;
      }
      return;
    }
    const bool test = r < gamma;
    const RowLds L = row_lds(row_dyn, V, true);
    if (test) {
      float qv[VPT];
      load_row<VPT>(a.q + (static_cast<size_t>(b) * W + r) * V, qv);
      store_row<VPT>(qv, L.q);
    }
    const int total = dense_to_list<VPT>(pv, L, redi);
    if (threadIdx.x >= kWave) return;
    const int d = test ? a.draft[static_cast<size_t>(b) * W + r] : -1;
    const float ua = test ? a.u_acc[static_cast<size_t>(b) * W + r] : 0.0f;
    const float ut = a.u_tgt[orow];
    uint32_t flags = 0;
    int code = -1;
    const int acc = walk_step(L, total, V, test ? 1 : 0, [&](int) { return d; }, [&](int) { return ua; }, ut,
                              &code, &flags);
    if (acc == 0) flags |= kRowAccepted;
    if (threadIdx.x == 0) {
      a.tcode[orow] = code;
      a.tflags[orow] = flags;
    }
  });
}

// One wave per stream: the round's outcome from its rows (chain_outcome).
__global__ __launch_bounds__(kBlock) void accept_outcome_kernel(const AcceptArgs a) {
  const int b = blockIdx.x * (kBlock / kWave) + static_cast<int>(threadIdx.x / kWave);
  if (b >= a.B) return;  // the whole wave
  const int l = static_cast<int>(threadIdx.x % kWave);
  const int W = a.W;
  const int gamma = min(max(a.gamma[b], 0), W);
  const int dc = l < gamma ? a.draft[static_cast<size_t>(b) * W + l] : 0;
  const int tc = l <= gamma ? a.tcode[static_cast<size_t>(b) * (W + 1) + l] : 0;
  const uint32_t tf = l <= gamma ? a.tflags[static_cast<size_t>(b) * (W + 1) + l] : 0u;
  int code;
  const ChainOutcome o = chain_outcome(gamma, a.greedy != 0, dc, tc, tf, &code);
  const int n = o.n_acc + 1;
  if (l <= W) a.codes_out[static_cast<size_t>(b) * (W + 1) + l] = l < n ? code : -1;
  if (l == 0) {
    a.n_out[b] = n;
    if (a.flags_out) a.flags_out[b] = o.accept | o.cdf;
  }
}

hipError_t launch_accept_rows(const AcceptArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(accept_rows_kernel, dim3(a.W + 1, a.B), dim3(kBlock), row_lds_bytes(a.V, true), s, a);
  constexpr int kStreamsPerBlock = kBlock / kWave;
  hipLaunchKernelGGL(accept_outcome_kernel, dim3((a.B + kStreamsPerBlock - 1) / kStreamsPerBlock), dim3(kBlock), 0,
                     s, a);
  return hipGetLastError();
}

// Scratch of the allocation-free component accept: the rows' steps
// (tcode, then tflags) of up to kNoAllocRows rows, one copy per GPU, held
// until the process ends.  Host code takes its device address from
// hipGetSymbolAddress (noalloc_accept_scratch); the symbol's host-side name
// is not a device address.
static __device__ __align__(256) uint32_t scratch[2 * kNoAllocRows];

hipError_t noalloc_accept_scratch(int** tcode, uint32_t** tflags) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
      e = hipGetSymbolAddress(&ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        ptr[dev] = nullptr;
        return e;
      }
    }
    p = ptr[dev];
  }
  *tcode = static_cast<int*>(p);
  *tflags = static_cast<uint32_t*>(p) + kNoAllocRows;
  return hipSuccess;
}

// One block per row of cp_spec_walk_step: the row's children tested in order
// against its draft distribution, then the draw (walk_step).
__global__ __launch_bounds__(kBlock) void walk_rows_kernel(const WalkArgs a) {
  extern __shared__ float4 row_dyn[];
  __shared__ int redi[4];
  const int i = blockIdx.x;
  const int V = a.V;
  const int nk = min(max(a.nchild[i], 0), a.maxc);
  dispatch_vpt(V, [&](auto vpt) {
    constexpr int VPT = decltype(vpt)::value;
    float pv[VPT];
    load_row<VPT>(a.p + static_cast<size_t>(i) * V, pv);
    const RowLds L = row_lds(row_dyn, V, true);
    if (nk > 0) {
      float qv[VPT];
      load_row<VPT>(a.q + static_cast<size_t>(i) * V, qv);
      store_row<VPT>(qv, L.q);
    }
    const int total = dense_to_list<VPT>(pv, L, redi);
    if (threadIdx.x >= kWave) return;
    const size_t cb = static_cast<size_t>(i) * a.maxc;
    uint32_t flags = 0;
    int code = -1;
    const int acc = walk_step(L, total, V, nk, [&](int k) { return a.child[cb + k]; },
                              [&](int k) { return a.u_acc[cb + k]; }, a.u_tgt[i], &code, &flags);
    if (threadIdx.x == 0) {
      a.acc_out[i] = acc;
      a.code_out[i] = code;
      if (a.flags_out) a.flags_out[i] = flags;
    }
  });
}

hipError_t launch_walk_rows(const WalkArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(walk_rows_kernel, dim3(a.n), dim3(kBlock), row_lds_bytes(a.V, true), s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Round control.

// Copy one input row into the verify rows: E_table[code] (fp32 or bf16).
__device__ __forceinline__ void embed_row(const RoundArgs& r, int table, int code, float* dst) {
  code = min(max(code, 0), r.V - 1);  // codes come from [0, V); never index outside
  const size_t off = (static_cast<size_t>(table) * r.V + code) * r.H;
  if (r.wbf16) {
    const uint16_t* e = static_cast<const uint16_t*>(r.embed) + off;
    for (int i = threadIdx.x; i < r.H; i += kBlock) dst[i] = bf16_to_f32(e[i]);
  } else {
    const float* e = static_cast<const float*>(r.embed) + off;
    for (int i = threadIdx.x; i < r.H; i += kBlock) dst[i] = e[i];
  }
}

// The same by threads i = 0..n-1 of a group (8 bf16 or 4 fp32 values per
// thread per step when the rows are 16-byte aligned).  bf16 rows: up to
// kGatherRun steps' loads are issued before the first store, so a row costs
// one memory round trip, not one per step.
constexpr int kGatherRun = 4;
__device__ __forceinline__ void embed_row_span(const RoundArgs& r, int table, int code, float* dst, int i0,
                                               int n) {
  code = min(max(code, 0), r.V - 1);
  const size_t off = (static_cast<size_t>(table) * r.V + code) * r.H;
  const bool dst_al = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
  if (r.wbf16) {
    const uint16_t* e = static_cast<const uint16_t*>(r.embed) + off;
    if ((r.H & 7) == 0 && dst_al && (reinterpret_cast<uintptr_t>(e) & 15u) == 0) {
      const int step = n * 8;
      for (int i = i0 * 8; i < r.H; i += kGatherRun * step) {
        uint4 v[kGatherRun];
#pragma unroll
        for (int j = 0; j < kGatherRun; ++j)
          if (i + j * step < r.H) v[j] = *reinterpret_cast<const uint4*>(e + i + j * step);
#pragma unroll
        for (int j = 0; j < kGatherRun; ++j) {
          if (i + j * step >= r.H) break;
          float* d = dst + i + j * step;
          *reinterpret_cast<float4*>(d) = make_float4(bf16lo(v[j].x), bf16hi(v[j].x), bf16lo(v[j].y), bf16hi(v[j].y));
          *reinterpret_cast<float4*>(d + 4) = make_float4(bf16lo(v[j].z), bf16hi(v[j].z), bf16lo(v[j].w), bf16hi(v[j].w));
        }
      }
    } else {
      for (int i = i0; i < r.H; i += n) dst[i] = bf16_to_f32(e[i]);
    }
  } else {
    const float* e = static_cast<const float*>(r.embed) + off;
    if ((r.H & 3) == 0 && dst_al && (reinterpret_cast<uintptr_t>(e) & 15u) == 0) {
      for (int i = i0 * 4; i < r.H; i += n * 4)
        *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(e + i);
    } else {
      for (int i = i0; i < r.H; i += n) dst[i] = e[i];
    }
  }
}

__device__ __forceinline__ uint64_t frame_seed(const StreamState& st) {
  return (static_cast<uint64_t>(st.seed_hi) << 32) | st.seed_lo;
}
__device__ __forceinline__ void set_frame_seed(StreamState& st, uint64_t seed) {
  st.seed_lo = static_cast<uint32_t>(seed);
  st.seed_hi = static_cast<uint32_t>(seed >> 32);
}

// Fused drafts: the heads of verify row rr of stream b in the next heads
// launch, given its target head th (0 = inactive row): column 0 the target,
// column k = 1..W the candidate draft of offset k, head th + k while the
// round that row rr would end can draft that far (k <= min(N-1, G-2-th)).
// Called by every thread; thread i < W + 1 writes column i.
__device__ __forceinline__ void fused_row_heads(const RoundArgs& r, int b, int rr, int th, int i) {
  if (i > r.W) return;
  int v = 0;
  if (th > 0) v = i == 0 ? th : (i <= min(r.N - 1, r.G - 2 - th) ? th + i : 0);
  r.fhead[(static_cast<size_t>(b) * r.R + rr) * (r.W + 1) + i] = v;
}

// Prefill of frame f for stream b: rows [h_frame, E_0[c_0]] at positions 0, 1
// and head 1 on row 1.  Rows wider than the block are copied with every load
// issued before the stores (16-byte pieces when aligned): one memory round
// trip per row instead of one per H / kBlock step.
__device__ void setup_prefill(const RoundArgs& r, const CallDesc& c, int b, int f) {
  float* x = r.X + static_cast<size_t>(b) * r.R * r.H;
  const float* hf = c.h_frame + (static_cast<size_t>(f) * c.B + b) * r.H;
  const int c0 = c.c0[static_cast<size_t>(f) * c.B + b];
  if (r.fold) {
    // (the rows: the folded Q/K/V launch reads them itself and leaves them
    // in X)
  } else if (r.H > kBlock) {
    if ((r.H & 3) == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(hf)) & 15u) == 0) {
      const int step = kBlock * 4;
      for (int i = threadIdx.x * 4; i < r.H; i += kGatherRun * step) {
        float4 v[kGatherRun];
#pragma unroll
        for (int j = 0; j < kGatherRun; ++j)
          if (i + j * step < r.H) v[j] = *reinterpret_cast<const float4*>(hf + i + j * step);
#pragma unroll
        for (int j = 0; j < kGatherRun; ++j) {
          if (i + j * step >= r.H) break;
          *reinterpret_cast<float4*>(x + i + j * step) = v[j];
        }
      }
    } else {
      for (int i = threadIdx.x; i < r.H; i += kBlock) x[i] = hf[i];
    }
    embed_row_span(r, 0, c0, x + r.H, threadIdx.x, kBlock);
  } else {
    for (int i = threadIdx.x; i < r.H; i += kBlock) x[i] = hf[i];
    embed_row(r, 0, c0, x + r.H);
  }
  if (threadIdx.x == 0) {
    c.out_codes[(static_cast<size_t>(f) * c.B + b) * r.G] = c0;
    for (int i = 0; i < r.R; ++i) {
      r.pos[b * r.R + i] = i < 2 ? i : -1;
      r.thead[b * r.R + i] = i == 1 ? 1 : 0;
    }
    for (int t = 0; t < r.W; ++t) r.dhead[b * r.W + t] = 0;
  }
  if (r.fused) {  // row 1 scores c_1 and drafts the first round from h_1
    const int W1 = r.W + 1;
    if (static_cast<int>(threadIdx.x) < r.R * W1)
      fused_row_heads(r, b, threadIdx.x / W1, threadIdx.x / W1 == 1 ? 1 : 0, threadIdx.x % W1);
  }
}

__global__ __launch_bounds__(kBlock) void round_init_kernel(const RoundArgs r, const CallDesc c) {
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0) {
    *r.call = c;
    *r.ovf = 0;  // no activation has left fp16's range in this call yet
  }
  constexpr int kStatWords = sizeof(cp_spec_stats) / sizeof(long long);
  if (threadIdx.x < kStatWords) reinterpret_cast<long long*>(r.sstats + b)[threadIdx.x] = 0;
  StreamState st{};
  if (c.F > 0) {
    setup_prefill(r, c, b, 0);
    st.mode = r.fold ? kModeFresh : kModePrefill;
    set_frame_seed(st, c.seeds[b]);
  } else {
    st.mode = kModeDone;
    if (threadIdx.x == 0) {
      for (int i = 0; i < r.R; ++i) {
        r.pos[b * r.R + i] = -1;
        r.thead[b * r.R + i] = 0;
      }
      for (int t = 0; t < r.W; ++t) r.dhead[b * r.W + t] = 0;
    }
    if (r.fused && static_cast<int>(threadIdx.x) < r.R * (r.W + 1))
      fused_row_heads(r, b, threadIdx.x / (r.W + 1), 0, threadIdx.x % (r.W + 1));
  }
  if (threadIdx.x == 0) r.st[b] = st;
  if (r.tnodes > 0 && threadIdx.x == 0) r.ncode[static_cast<size_t>(b) * kTreeSlots] = 0;  // no K/V move pending
}

hipError_t launch_round_init(const RoundArgs& r, const CallDesc& c, hipStream_t s) {
  hipLaunchKernelGGL(round_init_kernel, dim3(c.B), dim3(kBlock), 0, s, r, c);
  return hipGetLastError();
}

// Draft distributions q_t and proposals d_t of every stream (block (t-1, b)),
// plus the verify input row E_{s+t}[d_t].
__global__ __launch_bounds__(kBlock) void draft_topk_kernel(const RoundArgs r) {
  extern __shared__ float4 row_dyn[];
  __shared__ SelSmem S;
  __shared__ uint64_t red64[4];
  __shared__ uint32_t red32[4];
  const int t = blockIdx.x + 1, b = blockIdx.y;
  const size_t row = static_cast<size_t>(b) * r.W + (t - 1);
  dispatch_vpt(r.V, [&](auto vpt) {
    constexpr int VPT = decltype(vpt)::value;
    // the state goes out first, then the row (it always exists), so that the
    // draw's uniform is computed while the row is still in flight
    const StreamState st = r.st[b];
    float zv[VPT];
    load_row<VPT>(r.dlogits + row * r.V, zv);
    if (st.mode != kModeSpec) return;
    const float u = r.greedy ? 0.0f : frame_uniform(frame_seed(st), st.s + t, kDraft);
    // verify row 0 = E_s[c_s]: gathered by the block of offset 1, while the
    // draft rows are sampled
    float* x0 = r.X + static_cast<size_t>(b) * r.R * r.H;
    if (t > st.gamma) {  // gamma = 0: only row 0 to fill
      if (t == 1) embed_row(r, st.s, st.last, x0);
      return;
    }
    float* xrow = r.X + (static_cast<size_t>(b) * r.R + t) * r.H;
    if (r.greedy) {
      if (t == 1) embed_row(r, st.s, st.last, x0);
      const TopkResult res = argmax_regs<VPT>(zv, red64, red32);
      if (threadIdx.x == 0) {
        r.dcode[row] = res.code;
        r.dflags[row] = res.flags;
      }
      embed_row(r, st.s + t, res.code, xrow);
      return;
    }
    const RowLds L = row_lds(row_dyn, r.V, false);
    store_row<VPT>(zv, L.z);
    int total;
    uint32_t flags = 0;
    if (!topk_list<VPT>(zv, r.top_k, r.T, L, S, r.q + row * r.V, &total, &flags)) {
      if (t == 1) embed_row_span(r, st.s, st.last, x0, threadIdx.x - kWave, kBlock - kWave);
      return;
    }
    // wave 0 finishes the row: the draw, then the next input row
    int code, near;
    list_draw(L.lw, L.lidx, total, u, &code, &near);
    if (near) flags |= kFlagCdf;
    if (threadIdx.x == 0) {
      r.dcode[row] = code;
      r.dflags[row] = flags;
    }
    embed_row_span(r, st.s + t, code, xrow, threadIdx.x, kWave);
  });
}

hipError_t launch_draft_topk(const RoundArgs& r, hipStream_t s) {
  if (r.W <= 0 || r.N < 2) return hipSuccess;
  hipLaunchKernelGGL(draft_topk_kernel, dim3(r.W, r.B), dim3(kBlock), row_lds_bytes(r.V, false), s, r);
  return hipGetLastError();
}

// Target distribution p_r of every verify row that has a head, and the
// row's step of the acceptance walk (walk_step), all rows of all streams in
// parallel:
//   chain row r < gamma tests draft offset t = r+1 (one child): accept d_t
//     iff U(s+t, accept) < p_r(d_t) / q_t(d_t); if not, the row draws its
//     residual sample norm(max(0, p_r - q_t)) with U(s+t, target);
//   row gamma draws the bonus from p_gamma with U(s+gamma+1, target);
//   prefill row 1 draws c_1 from p_1 with U(1, target);
//   tree row v tests its node's active children in node order with
//     U(depth, accept, k) and draws from the last residual with
//     U(depth, target) when none is accepted.
// Each row's outcome depends on that row alone, so the sequential scan
// reduces to "first rejected offset" (chain) or a walk over the rows'
// decisions (tree) in the accept kernel.  tcode holds the draft code
// (accepted) or the row's draw; tflags the row's top-k / argmax flags, its
// accept-test and CDF near ties, and kRowAccepted (chain) or the accepted
// child + 1 in bits 16..23 (tree).
// Fused drafts: block (rr, k >= 1) forms row rr's candidate draft of offset
// k instead: q = TopKSoftmax of its logits (dense, kept for the next round's
// test), the draw with U(depth, draft) (greedy: the argmax), its flags.
template <int VPT>
__device__ void candidate_draft(const RoundArgs& r, int b, int rr, int k, SelSmem& S, float4* row_dyn,
                                uint64_t* red64, uint32_t* red32) {
  const size_t frow = (static_cast<size_t>(b) * r.R + rr) * (r.W + 1) + k;
  const int head = r.fhead[frow];
  const StreamState st = r.fold ? r.st_out[b] : r.st[b];  // (fold: the staged state is this round's)
  float zv[VPT];
  load_row<VPT>(r.tlogits + frow * r.V, zv);
  if (head <= 0 || st.mode == kModeDone) return;
  const size_t crow = (static_cast<size_t>(b) * r.R + rr) * r.W + (k - 1);
  if (r.greedy) {
    const TopkResult res = argmax_regs<VPT>(zv, red64, red32);
    if (threadIdx.x == 0) {
      r.ccode[crow] = res.code;
      r.cflags[crow] = res.flags;
    }
    return;
  }
  const float u = frame_uniform(frame_seed(st), head, kDraft);
  const RowLds L = row_lds(row_dyn, r.V, true);
  store_row<VPT>(zv, L.z);
  int total;
  uint32_t flags = 0;
  if (!topk_list<VPT>(zv, r.top_k, r.T, L, S, r.cq + crow * r.V, &total, &flags)) return;
  int code, near;
  list_draw(L.lw, L.lidx, total, u, &code, &near);
  if (near) flags |= kFlagCdf;
  if (threadIdx.x == 0) {
    r.ccode[crow] = code;
    r.cflags[crow] = flags;
  }
}

__global__ __launch_bounds__(kBlock) void target_topk_kernel(const RoundArgs r) {
  extern __shared__ float4 row_dyn[];
  __shared__ SelSmem S;
  __shared__ uint64_t red64[4];
  __shared__ uint32_t red32[4];
  const int W1 = r.fused ? r.W + 1 : 1;
  const int rr = blockIdx.x / W1, kc = blockIdx.x % W1, b = blockIdx.y;
  const size_t row = static_cast<size_t>(b) * r.R + rr;
  if (r.fold && blockIdx.x == 0) {
    // the accept step folded into this pass's first projection left the
    // stream's state and drafts in staging copies, which this launch reads;
    // the next pass's first projection reads them in place
    constexpr int kStW = sizeof(StreamState) / 4;
    const int t = threadIdx.x;
    if (t < kStW) {
      reinterpret_cast<int*>(r.st + b)[t] = reinterpret_cast<const int*>(r.st_out + b)[t];
    } else if (t >= kWave && t < kWave + r.W) {
      const size_t i = static_cast<size_t>(b) * r.W + (t - kWave);
      r.dcode[i] = r.dcode_out[i];
      r.dflags[i] = r.dflags_out[i];
    }
  }
  dispatch_vpt(r.V, [&](auto vpt) {
    constexpr int VPT = decltype(vpt)::value;
    if (kc > 0) {
      candidate_draft<VPT>(r, b, rr, kc, S, row_dyn, red64, red32);
      return;
    }
    const int base = threadIdx.x * VPT;
    // every load that depends only on the block goes out at once (one memory
    // round trip, not three): the row's head and the stream's state first, so
    // that the uniforms are computed while the rest is in flight, then the
    // logits and the draft distribution this row may test against (the
    // chain's row rr tests draft offset rr + 1, which exists for rr < W; a
    // tree row tests the children of its node, drafted at depth dep[rr] + 1)
    const int head = r.thead[row];
    const StreamState st = r.fold ? r.st_out[b] : r.st[b];  // (fold: the staged state is this round's)
    float zv[VPT];
    load_row<VPT>(r.tlogits + row * W1 * r.V, zv);
    const int qi = r.tnodes > 0 ? r.dep[rr] : rr;
    const bool has_q = !r.greedy && qi < r.W;
    float qv[VPT];
    int dd = -1;
    if (has_q) {
      const float* qrow = r.q + (static_cast<size_t>(b) * r.W + qi) * r.V;
#pragma unroll
      for (int j = 0; j < VPT; ++j) qv[j] = qrow[base + j];
      if (r.tnodes == 0) dd = (r.fold ? r.dcode_out : r.dcode)[static_cast<size_t>(b) * r.W + rr];
    }
    // (a finished stream's heads are zero already; testing its mode here keeps
    // the state load ahead of this branch)
    if (head <= 0 || st.mode == kModeDone) return;
    const bool spec = st.mode == kModeSpec;
    if (r.greedy) {
      const TopkResult res = argmax_regs<VPT>(zv, red64, red32);
      if (threadIdx.x == 0) {
        r.tcode[row] = res.code;
        r.tflags[row] = res.flags;
      }
      return;
    }
    // the row's children: chain row rr < gamma tests draft rr + 1; a tree
    // row its node's children within the round's depth
    const int gamma = spec ? st.gamma : 0;
    __shared__ int kids_s[kMaxTree];  // a tree row's active children, node order
    int nk = 0;
    if (r.tnodes == 0) {
      nk = spec && rr < gamma ? 1 : 0;
    } else if (spec) {
      for (int ch = 1; ch <= r.tnodes; ++ch)
        if (r.par[ch] == rr && r.dep[ch] <= gamma) {
          if (threadIdx.x == 0) kids_s[nk] = ch;
          ++nk;
        }
    }
    const uint64_t seed = frame_seed(st);
    const int depth = spec ? st.s + (r.tnodes > 0 ? r.dep[rr] : rr) + 1 : 1;
    const float ut = frame_uniform(seed, depth, kTarget);
    const float ua0 = nk > 0 ? frame_uniform(seed, depth, kAccept) : 0.0f;
    const RowLds L = row_lds(row_dyn, r.V, true);
    store_row<VPT>(zv, L.z);
    if (nk > 0) store_row<VPT>(qv, L.q);
    int total;
    uint32_t flags = 0;
    if (!topk_list<VPT>(zv, r.top_k, r.T, L, S, nullptr, &total, &flags)) return;
    // wave 0: the row's step of the walk
    int code = -1, acc;
    if (r.tnodes == 0) {
      acc = walk_step(L, total, r.V, nk, [&](int) { return dd; }, [&](int) { return ua0; }, ut, &code, &flags);
      if (acc == 0) flags |= kRowAccepted;
    } else {
      acc = walk_step(L, total, r.V, nk,
                      [&](int k) { return r.ncode[static_cast<size_t>(b) * kTreeSlots + kids_s[k]]; },
                      [&](int k) { return k == 0 ? ua0 : frame_uniform(seed, depth, kAccept, k); }, ut, &code,
                      &flags);
      if (acc >= 0) {
        flags |= static_cast<uint32_t>(kids_s[acc] + 1) << 16;
        code = -1;
      }
    }
    if (threadIdx.x == 0) {
      r.tcode[row] = code;
      r.tflags[row] = flags;
    }
  });
}

hipError_t launch_target_topk(const RoundArgs& r, hipStream_t s) {
  const int W1 = r.fused ? r.W + 1 : 1;
  hipLaunchKernelGGL(target_topk_kernel, dim3(r.R * W1, r.B), dim3(kBlock), row_lds_bytes(r.V, true), s, r);
  return hipGetLastError();
}

// Near-tie flag bits -> the four near-tie counters (stats words).
__device__ __forceinline__ void count_flags(uint32_t f, cp_spec_stats* cnt) {
  if (f & kFlagTopk) ++cnt->near_tie_topk;
  if (f & kFlagArgmax) ++cnt->near_tie_argmax;
  if (f & kFlagCdf) ++cnt->near_tie_cdf;
  if (f & kFlagAccept) ++cnt->near_tie_accept;
}

// Fused drafts, next round of stream b at committed depth s with gamma
// drafts: the candidate set of the verify row that ended this round (hrow,
// whose output is h_s) becomes the round's drafts (codes, flags and dense
// distributions, as the draft kernel leaves them), the verify rows E_s[c_s]
// and E_{s+t}[d_t] are gathered, and the rows' heads for the next heads
// launch are set.  cc / cf: that row's candidate codes and flags, already
// read (so the gather's loads go out at once).  Every thread of the block
// calls it.
__device__ void fused_next_round(const RoundArgs& r, int b, int s, int gamma, int hrow, int last, const int* cc,
                                 const uint32_t* cf) {
  const int tid = threadIdx.x;
  const size_t cb = (static_cast<size_t>(b) * r.R + hrow) * r.W;
  const int V4 = r.V / 4;
  const float4* src = reinterpret_cast<const float4*>(r.cq + cb * r.V);
  float4* dst = reinterpret_cast<float4*>(r.q + static_cast<size_t>(b) * r.W * r.V);
  for (int i = tid; i < gamma * V4; i += kBlock) dst[i] = src[i];
  if (tid < gamma) {
    r.dcode_out[static_cast<size_t>(b) * r.W + tid] = cc[tid];
    r.dflags_out[static_cast<size_t>(b) * r.W + tid] = cf[tid];
  }
  // the gamma + 1 verify rows side by side, a group of threads each (with
  // the fold, the next pass's Q/K/V launch reads them itself and leaves
  // them in X)
  const int nrow = gamma + 1, per = kBlock / nrow;
  const int k = tid / per;
  if (k < nrow && !r.fold) {
    const int code = k == 0 ? last : cc[k - 1];
    embed_row_span(r, s + k, code, r.X + (static_cast<size_t>(b) * r.R + k) * r.H, tid - k * per, per);
  }
  const int W1 = r.W + 1;
  if (tid < r.R * W1) {
    const int rr = tid / W1;
    fused_row_heads(r, b, rr, rr <= gamma ? s + 1 + rr : 0, tid % W1);
  }
}

// Candidate rows of h_{s+n} held in registers while the outcome is decided:
// up to kHrowF4 float4 per thread, i.e. R * H <= 8192.
constexpr int kHrowF4 = 8;

// Accept, commit, truncate, and set up the stream's next round (or frame).
// The rows' outcomes come from the target kernel: n = first rejected offset
// (or gamma + 1), committed codes = the accepted drafts, then row n-1's
// sample.  Greedy: accept while d_t equals row t-1's argmax.
//
// Latency: every load that depends only on the stream index goes out at once
// (state, call, the rows' codes and flags, the stream's counters, and all R
// output rows, one of which becomes h_{s+n}); one thread then decides, and
// the block writes.  Counters stay per stream (no device-wide atomics inside
// the round); they are added to the caller's totals once per call.
// The accept step of stream b, by one block of kBlock threads.  It reads the
// round's state from r.st / r.dcode / r.dflags and writes the next round's to
// r.st_out / r.dcode_out / r.dflags_out.
__device__ void accept_step(const RoundArgs& r, int b) {
  __shared__ StreamState st_s;
  __shared__ CallDesc c_s;
  __shared__ cp_spec_stats cnt_s;
  __shared__ int tcode_s[CP_SPEC_MAX_WINDOW], dcode_s[CP_SPEC_MAX_WINDOW];
  __shared__ uint32_t tflags_s[CP_SPEC_MAX_WINDOW], dflags_s[CP_SPEC_MAX_WINDOW];
  // fused drafts: every verify row's candidate codes and flags
  __shared__ int ccode_s[CP_SPEC_MAX_WINDOW * CP_SPEC_MAX_WINDOW];
  __shared__ uint32_t cflags_s[CP_SPEC_MAX_WINDOW * CP_SPEC_MAX_WINDOW];
  __shared__ int sh_n, sh_hrow;
  constexpr int kStW = sizeof(StreamState) / 4, kCallW = sizeof(CallDesc) / 4;
  constexpr int kCntW = sizeof(cp_spec_stats) / 8;
  static_assert(kStW <= 32 && kCallW <= 32 && kCntW <= 32, "state words");
  const int tid = threadIdx.x;
  const size_t rb = static_cast<size_t>(b) * r.R;

  // ---- every independent load at once ----
  if (tid < kStW) {
    reinterpret_cast<int*>(&st_s)[tid] = reinterpret_cast<const int*>(r.st + b)[tid];
  } else if (tid >= 32 && tid < 32 + kCallW) {
    reinterpret_cast<int*>(&c_s)[tid - 32] = reinterpret_cast<const int*>(r.call)[tid - 32];
  } else if (tid >= 64 && tid < 64 + kCntW) {
    reinterpret_cast<long long*>(&cnt_s)[tid - 64] = reinterpret_cast<const long long*>(r.sstats + b)[tid - 64];
  } else if (tid >= 96 && tid < 96 + r.R) {
    tcode_s[tid - 96] = r.tcode[rb + tid - 96];
    tflags_s[tid - 96] = r.tflags[rb + tid - 96];
  } else if (tid >= 112 && tid < 112 + r.W) {
    dcode_s[tid - 112] = r.dcode[static_cast<size_t>(b) * r.W + tid - 112];
    dflags_s[tid - 112] = r.dflags[static_cast<size_t>(b) * r.W + tid - 112];
  } else if (r.fused && tid >= 128 && tid < 128 + r.R * r.W) {
    ccode_s[tid - 128] = r.ccode[rb * r.W + tid - 128];
    cflags_s[tid - 128] = r.cflags[rb * r.W + tid - 128];
  }
  const int H4 = r.H / 4;
  const int nf4 = r.R * H4;
  const bool held = nf4 <= kHrowF4 * kBlock;
  float4 hv[kHrowF4];
  if (held) {
    const float4* src = reinterpret_cast<const float4*>(r.Hout + rb * r.H);
#pragma unroll
    for (int i = 0; i < kHrowF4; ++i) {
      const int q = tid + i * kBlock;
      if (q < nf4) hv[i] = src[q];
    }
  }
  __syncthreads();
  StreamState st = st_s;
  if (st.mode == kModeDone || st.mode == kModeFresh) {
    // nothing to commit: a finished stream, or a call's first pass (the
    // init kernel set up its rows)
    if (tid == 0 && r.st_out != r.st) {
      if (st.mode == kModeFresh) st.mode = kModePrefill;
      r.st_out[b] = st;
    }
    return;
  }
  const CallDesc& c = c_s;
  const size_t fb = static_cast<size_t>(st.f) * c.B + b;
  int* out = c.out_codes + fb * r.G;

  // ---- the decision (wave 0; lane l holds draft l + 1 and row l) ----
  if (tid < kWave) {
    cp_spec_stats& cnt = cnt_s;
    const int l = tid;
    if (st.mode == kModePrefill) {
      if (l == 0) {
        const uint32_t f = tflags_s[1] & ~kRowAccepted;
        count_flags(f, &cnt);
        if (f) st_s.flags |= 1u << 1;
        out[1] = st_s.last = tcode_s[1];
        ++cnt.prefill_passes;
        sh_n = 1;
        sh_hrow = 1;
        st_s.s = 1;
      }
    } else {
      const int s = st.s, gamma = st.gamma;
      const int dc = l < gamma ? dcode_s[l] : 0;
      const uint32_t df = l < gamma ? dflags_s[l] : 0u;
      const int tc = l <= gamma ? tcode_s[l] : 0;
      const uint32_t tf = l <= gamma ? tflags_s[l] : 0u;
      int code;
      const ChainOutcome o = chain_outcome(gamma, r.greedy != 0, dc, tc, tf, &code);
      const int n_acc = o.n_acc, n = n_acc + 1;
      // near ties of the decisions the outcome used: drafts 1..n_acc + 1
      // (the last one tested), rows 0..n_acc; draft l + 1 and row l both
      // mark depth s + 1 + l
      const uint32_t dfu = l < min(n_acc + 1, gamma) ? df : 0u;
      const uint32_t rfu = l <= n_acc ? (tf & (kFlagTopk | kFlagArgmax)) : 0u;
      const uint32_t marked = static_cast<uint32_t>(__ballot(dfu != 0u || rfu != 0u));
      auto both = [&](uint32_t bit) {
        return __popcll(__ballot((dfu & bit) != 0u)) + __popcll(__ballot((rfu & bit) != 0u));
      };
      const int n_topk = both(kFlagTopk), n_argmax = both(kFlagArgmax);
      const int n_cdf = both(kFlagCdf) + (o.cdf != 0u ? 1 : 0);
      const int n_accept = both(kFlagAccept) + __popc(o.accept);
      const int last = __shfl(code, n_acc);
      if (l <= n_acc) out[s + 1 + l] = code;
      if (l < gamma) {  // one counter word per lane
        ++cnt.proposed[l];
        if (l < n_acc) ++cnt.accepted[l];
      }
      if (l == 0) {
        cnt.near_tie_topk += n_topk;
        cnt.near_tie_argmax += n_argmax;
        cnt.near_tie_cdf += n_cdf;
        cnt.near_tie_accept += n_accept;
        uint32_t fl = st.flags | (marked << (s + 1)) | (o.accept << (s + 1));
        if (o.cdf) fl |= 1u << (s + n);
        st_s.last = last;
        ++cnt.rounds;
        if (n_acc == gamma) ++cnt.bonus;
        st_s.flags = fl;
        st_s.s = s + n;
        sh_n = n;
        sh_hrow = n - 1;
      }
    }
    if (l == 0 && st_s.s >= r.G - 1) {  // frame complete
      if (c.out_flags) c.out_flags[fb] = st_s.flags;
      ++cnt.frames;
      cnt.codes += r.G - 1;
    }
  }
  __syncthreads();
  st = st_s;

  // ---- h_{s+n} = output row n-1 (prefill: row 1), and with position-aware
  // offsets the next round's draft inputs h_{s+n} + b_t, t = 1..W (b_t = 0
  // past K) ----
  {
    const int hrow = sh_hrow;
    float4* dst = reinterpret_cast<float4*>(r.hstate + static_cast<size_t>(b) * r.H);
    float4* dx = r.K > 0 ? reinterpret_cast<float4*>(r.dX + static_cast<size_t>(b) * r.W * r.H) : nullptr;
    const float4* off = reinterpret_cast<const float4*>(r.doff);
    auto put = [&](int k4, float4 v) {
      dst[k4] = v;
      if (dx != nullptr)
        for (int t = 0; t < r.W; ++t) {
          float4 o = v;
          if (t < r.K) {
            const float4 bt = off[t * H4 + k4];
            o.x += bt.x, o.y += bt.y, o.z += bt.z, o.w += bt.w;
          }
          dx[t * H4 + k4] = o;
        }
    };
    if (held) {
#pragma unroll
      for (int i = 0; i < kHrowF4; ++i) {
        const int q = tid + i * kBlock;
        if (q < nf4 && q / H4 == hrow) put(q % H4, hv[i]);
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(r.Hout + (rb + hrow) * r.H);
      for (int i = tid; i < H4; i += kBlock) put(i, src[i]);
    }
  }
  if (tid < kCntW)
    reinterpret_cast<long long*>(r.sstats + b)[tid] = reinterpret_cast<const long long*>(&cnt_s)[tid];

  // ---- next round of this stream ----
  if (st.s >= r.G - 1) {
    st.f += 1;
    st.s = 0;
    st.flags = 0;
    st.gamma = 0;
    if (st.f >= c.F) {
      st.mode = kModeDone;
      if (tid < r.R) {
        r.pos[rb + tid] = -1;
        r.thead[rb + tid] = 0;
      }
      if (tid < r.W) r.dhead[static_cast<size_t>(b) * r.W + tid] = 0;
      if (r.fused && tid < r.R * (r.W + 1)) fused_row_heads(r, b, tid / (r.W + 1), 0, tid % (r.W + 1));
    } else {
      st.mode = kModePrefill;
      set_frame_seed(st, c.seeds[static_cast<size_t>(st.f) * c.B + b]);
      setup_prefill(r, c, b, st.f);
    }
  } else {
    const int s = st.s;
    const int gamma = r.N == 0 ? 0 : min(r.N - 1, r.G - 2 - s);
    st.gamma = gamma;
    st.mode = kModeSpec;
    // verify row 0 = E_s[c_s]: the draft kernel gathers it when it runs
    if (r.N < 2) embed_row(r, s, st.last, r.X + rb * r.H);
    if (tid < r.R) {
      r.pos[rb + tid] = tid <= gamma ? s + 1 + tid : -1;
      r.thead[rb + tid] = tid <= gamma ? s + 1 + tid : 0;
    }
    if (tid < r.W) r.dhead[static_cast<size_t>(b) * r.W + tid] = tid + 1 <= gamma ? s + tid + 1 : 0;
    if (r.fused)
      fused_next_round(r, b, s, gamma, sh_hrow, st.last, ccode_s + sh_hrow * r.W, cflags_s + sh_hrow * r.W);
  }
  if (tid == 0) r.st_out[b] = st;
}

__global__ __launch_bounds__(kBlock) void round_accept_kernel(const RoundArgs r) { accept_step(r, blockIdx.x); }

hipError_t launch_round_accept(const RoundArgs& r, hipStream_t s) {
  hipLaunchKernelGGL(round_accept_kernel, dim3(r.B), dim3(kBlock), 0, s, r);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The accept step folded into the next pass's first projection.
//
// A row of the fold's Q/K/V launch: where its values come from (null: a zero
// row; fp32 or the tables' type) and its position (-1: inactive).
struct FoldRow {
  const void* p;
  int bf16;
  int pos;
};

template <int MT>
__device__ void fold_rows(const RoundArgs& r, int m0, int M, FoldRow* out);

// The GEMV's custom row source: the block's FoldRows (LDS), found by
// fold_rows in prepare().
template <int MT>
struct FoldRows {
  static constexpr bool kCustom = true;
  const RoundArgs& r;
  int m0, M;
  FoldRow* rows;
  __device__ void prepare() const { fold_rows<MT>(r, m0, M, rows); }
  template <int VEC>
  __device__ void load(int m, int k, float4 (&x)[VEC / 4]) const {
    const FoldRow fr = rows[m];
    if (fr.p == nullptr) {
#pragma unroll
      for (int i = 0; i < VEC / 4; ++i) x[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      return;
    }
    if (fr.bf16) {
      const uint16_t* e = static_cast<const uint16_t*>(fr.p) + k;
      if ((reinterpret_cast<uintptr_t>(e) & 7u) == 0) {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
          const uint2 v = *reinterpret_cast<const uint2*>(e + 4 * i);
          x[i] = make_float4(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y));
        }
      } else {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i)
          x[i] = make_float4(bf16_to_f32(e[4 * i]), bf16_to_f32(e[4 * i + 1]), bf16_to_f32(e[4 * i + 2]),
                             bf16_to_f32(e[4 * i + 3]));
      }
    } else {
      const float* f = static_cast<const float*>(fr.p) + k;
      if ((reinterpret_cast<uintptr_t>(f) & 15u) == 0) {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) x[i] = *reinterpret_cast<const float4*>(f + 4 * i);
      } else {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) x[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
      }
    }
  }
  __device__ int pos(int m) const { return rows[m].pos; }
};

// Rows m0 .. m0 + MT - 1 (of M) of the fold's Q/K/V launch.  For each stream
// with rows there, the outcome of the round the last pass verified, as the
// accept step takes it (chain_outcome on the rows' steps; a prefill commits
// row 1's code), then the next round's input rows and positions: E_s[c_s] and
// E_{s+t}[d_t] with the drafts of the row that ended the round, or, after a
// frame, the next frame's prefill rows [h_frame, E_0[c_0]].  Wave w takes the
// block's w-th stream (R >= 2 and MT <= 8: at most four).  Every thread of
// the block calls it.
template <int MT>
__device__ void fold_rows(const RoundArgs& r, int m0, int M, FoldRow* out) {
  // rows past M (and rows no stream claims) stay zero rows
  if (threadIdx.x < MT) out[threadIdx.x] = FoldRow{nullptr, 0, -1};
  __syncthreads();
  const int w = static_cast<int>(threadIdx.x) / kWave, l = static_cast<int>(threadIdx.x) % kWave;
  const int b = m0 / r.R + w;
  if (w < 4 && b < r.B && b * r.R < m0 + MT) {
    // every load that does not depend on the outcome at once: the state, the
    // rows' steps (lane l: row l), the drafts (lane l: d_{l+1}) and every
    // row's candidate codes (lane l: entry l of [R][W])
    const size_t rb = static_cast<size_t>(b) * r.R;
    const StreamState st = r.st[b];
    const CallDesc* c = r.call;
    const int cF = c->F, cB = c->B;
    const float* hframe = c->h_frame;
    const int* c0 = c->c0;
    const int tc = l < r.R ? r.tcode[rb + l] : 0;
    const uint32_t tf = l < r.R ? r.tflags[rb + l] : 0u;
    const int dc = l < r.W ? r.dcode[static_cast<size_t>(b) * r.W + l] : 0;
    const int cc = l < r.R * r.W ? r.ccode[rb * r.W + l] : 0;
    int mode = st.mode, f = st.f, s = st.s, last = st.last, hrow = 0;
    bool pre = mode == kModeFresh;  // the next rows are frame f's prefill
    if (mode == kModePrefill || mode == kModeSpec) {
      int n = 1;
      if (mode == kModePrefill) {
        hrow = 1;
        last = __shfl(tc, 1);
      } else {
        const int gamma = st.gamma;
        int code;
        const ChainOutcome o = chain_outcome(gamma, r.greedy != 0, l < gamma ? dc : 0, l <= gamma ? tc : 0,
                                             l <= gamma ? tf : 0u, &code);
        n = o.n_acc + 1;
        hrow = n - 1;
        last = __shfl(code, o.n_acc);
      }
      s = (mode == kModePrefill ? 0 : s) + n;
      mode = kModeSpec;
      if (s >= r.G - 1) {  // frame complete
        f += 1;
        mode = f >= cF ? kModeDone : kModePrefill;
        pre = mode == kModePrefill;
      }
    }
    const int gamma = mode == kModeSpec ? (r.N == 0 ? 0 : min(r.N - 1, r.G - 2 - s)) : 0;
    // lane l: row l's draft code, d_l of the row that ended the round
    const int ccl = __shfl(cc, min(max(hrow * r.W + l - 1, 0), kWave - 1));
    const int rr = l, row = b * r.R + rr, m = row - m0;
    if (rr < r.R && m >= 0 && m < MT) {
      FoldRow fr{nullptr, 0, -1};
      if (row < M && mode != kModeDone) {
        const size_t fb = static_cast<size_t>(f) * cB + b;
        int table = -1, code = 0;
        if (pre) {
          if (rr == 0) fr = FoldRow{hframe + fb * r.H, 0, 0};
          if (rr == 1) table = 0, code = c0[fb], fr.pos = 1;
        } else if (rr <= gamma) {
          table = s + rr;
          code = rr == 0 ? last : ccl;
          fr.pos = s + 1 + rr;
        }
        if (table >= 0) {
          code = min(max(code, 0), r.V - 1);  // codes come from [0, V); never index outside
          const size_t off = (static_cast<size_t>(table) * r.V + code) * r.H;
          fr.p = r.wbf16 ? static_cast<const void*>(static_cast<const uint16_t*>(r.embed) + off)
                         : static_cast<const void*>(static_cast<const float*>(r.embed) + off);
          fr.bf16 = r.wbf16;
        }
      }
      out[m] = fr;
    }
  }
  __syncthreads();
}

// Grid: r.B accept blocks, then gdx x gdy GEMV blocks (one-dimensional).
template <typename WT, int MT, int SPT>
__global__ __launch_bounds__(kBlock) void gemv_fold_kernel(const GemvArgs a, const RoundArgs r, int gdx, int gdy) {
  const int L = blockIdx.x;
  if (L < r.B) {
    accept_step(r, L);
    return;
  }
  // as gemv_kernel's: the row tiles of one weight slice on one XCD
  const int Lg = L - r.B;
  int bx = Lg % gdx, by = Lg / gdx;
  if (gdy > 1 && gdx % 8 == 0) {
    const int i = Lg / 8;
    by = i % gdy;
    bx = (i / gdy) * 8 + Lg % 8;
  }
  __shared__ FoldRow rows_s[MT];
  gemv_block<WT, kQKV, MT, SPT>(a, bx, by, gdx, FoldRows<MT>{r, by * MT, a.M, rows_s});
}

template <typename WT>
hipError_t launch_gemv_fold_t(int mt, const GemvArgs& a, const RoundArgs& r, int gx, int gy, hipStream_t s) {
  constexpr int VEC = Chunk<WT>::N;
  const int spt = a.K / (VEC * a.kt);
  if (r.R < 2 || a.rows_per_stream != r.R || a.M != r.B * r.R) return hipErrorInvalidValue;
  const dim3 grid(r.B + gx * gy), block(kBlock);
#define CPS_FOLD_CASE(MT_, SPT_)                                                                \
  if (mt == MT_ && spt == SPT_) {                                                               \
    hipLaunchKernelGGL((gemv_fold_kernel<WT, MT_, SPT_>), grid, block, 0, s, a, r, gx, gy);    \
    return hipGetLastError();                                                                   \
  }
#define CPS_FOLD_MT(MT_) CPS_FOLD_CASE(MT_, 1) CPS_FOLD_CASE(MT_, 2) CPS_FOLD_CASE(MT_, 3) CPS_FOLD_CASE(MT_, 4)
  CPS_FOLD_MT(1)
  CPS_FOLD_MT(2)
  CPS_FOLD_MT(4)
  CPS_FOLD_MT(8)
#undef CPS_FOLD_MT
#undef CPS_FOLD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_fold(int wdtype, int mt, const GemvArgs& a, const RoundArgs& r, int gx, int gy,
                            hipStream_t s) {
  return wdtype == CP_SPEC_BF16 ? launch_gemv_fold_t<uint16_t>(mt, a, r, gx, gy, s)
                                : launch_gemv_fold_t<float>(mt, a, r, gx, gy, s);
}

// ---------------------------------------------------------------------------
// The codec part of the Talker's next input for finished frames: row i is
// the sum over groups g = 0..G-1 of E_g[codes[i][g]], added in group order
// in float32.  A code outside [0, V) makes the row NaN.  One block per row,
// four channels per thread per step.
__global__ __launch_bounds__(kBlock) void talker_feedback_kernel(const void* embed, int wbf16, int G, int V, int H,
                                                                 const int* codes, float* out) {
  __shared__ int code_s[64];
  __shared__ int bad_s;
  const int row = blockIdx.x;
  if (threadIdx.x == 0) bad_s = 0;
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += kBlock) {
    const int c = codes[static_cast<size_t>(row) * G + g];
    const bool ok = c >= 0 && c < V;
    code_s[g] = ok ? c : 0;
    if (!ok) bad_s = 1;
  }
  __syncthreads();
  const float nan = __uint_as_float(0x7FC00000u);
  float* dst = out + static_cast<size_t>(row) * H;
  for (int i = threadIdx.x * 4; i < H; i += kBlock * 4) {
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    for (int g = 0; g < G; ++g) {
      const size_t off = (static_cast<size_t>(g) * V + code_s[g]) * H + i;
      if (wbf16) {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(embed) + off);
        a0 += bf16lo(v.x); a1 += bf16hi(v.x); a2 += bf16lo(v.y); a3 += bf16hi(v.y);
      } else {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(embed) + off);
        a0 += v.x; a1 += v.y; a2 += v.z; a3 += v.w;
      }
    }
    if (bad_s) a0 = a1 = a2 = a3 = nan;
    *reinterpret_cast<float4*>(dst + i) = make_float4(a0, a1, a2, a3);
  }
}

hipError_t launch_talker_feedback(const void* embed, int wbf16, int G, int V, int H, const int* codes, int n,
                                  float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (G > 64 || H % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(talker_feedback_kernel, dim3(n), dim3(kBlock), 0, s, embed, wbf16, G, V, H, codes, out);
  return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void stats_flush_kernel(const cp_spec_stats* sstats, int B,
                                                             cp_spec_stats* out) {
  constexpr int kW = sizeof(cp_spec_stats) / sizeof(long long);
  const int i = threadIdx.x;
  if (i >= kW) return;
  long long t = 0;
  for (int b = 0; b < B; ++b) t += reinterpret_cast<const long long*>(sstats + b)[i];
  if (t) atomicAdd(reinterpret_cast<unsigned long long*>(out) + i, static_cast<unsigned long long>(t));
}

hipError_t launch_stats_flush(const cp_spec_stats* sstats, int B, cp_spec_stats* out, hipStream_t s) {
  hipLaunchKernelGGL(stats_flush_kernel, dim3(1), dim3(kBlock), 0, s, sstats, B, out);
  return hipGetLastError();
}


// ===========================================================================
// Tree-shaped verify window ("RVQ Position Aware Speculative Decoding ...",
// section 2.2 and Figure 2).  Node 0 is the root (row 0, the committed code
// c_s); node i = row i sits at depth dep[i], proposes the code of depth
// s + dep[i] and keeps its K/V in slot G + i - 1 of the stream's cache (the
// frame's G positions come first) until the round commits it.  Every node draws its code from its depth's draft
// distribution; the walk tests a node's children in order with min(1, p'/q)
// and replaces p' by norm(max(0, p' - q)) after each rejection.
// ===========================================================================

// Draft side: block (d-1, b) forms q_d (dense, for the walk) and draws the
// code of every node of depth d from it (draw index j = the node's number
// among the nodes of depth d, node order), then gathers each node's verify
// input E_{s+d}[code]; the block of depth 1 also gathers row 0 = E_s[c_s].
// Per-depth flags (top-k boundary, any draw's CDF near tie) go to dflags.
// The previous round's accepted tree nodes' K/V: slot G + a - 1 -> position
// s + 1 + dep[a] for every node a on the path from the root to node v, every
// layer, K and V.  The round's tree accept kernel leaves (s, v) in
// ncode[b][0]; the W draft blocks of the stream share the move (block
// `part`), a node at a time with all of a node's loads before its stores.
// It runs before the round's projections write new node K/V into the slots.
__device__ void tree_kv_move(const RoundArgs& r, int b, int s, int v, int part) {
  float* kvb = r.kv + static_cast<size_t>(b) * r.kv_sb;
  const int kv4 = r.kvdim / 4, n4 = 2 * r.L * kv4;
  const int nthr = r.W * kBlock;
  constexpr int Q = 4;
  for (int a = v; a > 0 && a <= r.tnodes; a = r.par[a]) {
    const size_t src = static_cast<size_t>(r.G + a - 1) * r.kvdim;
    const size_t dst = static_cast<size_t>(s + 1 + r.dep[a]) * r.kvdim;
    for (int i0 = part * kBlock + threadIdx.x; i0 < n4; i0 += Q * nthr) {
      float4 t[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int i = min(i0 + q * nthr, n4 - 1);
        const float* lay = kvb + static_cast<size_t>(i / kv4) * r.Gk * r.kvdim;
        t[q] = *reinterpret_cast<const float4*>(lay + src + (i % kv4) * 4);
      }
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int i = i0 + q * nthr;
        if (i < n4) {
          float* lay = kvb + static_cast<size_t>(i / kv4) * r.Gk * r.kvdim;
          *reinterpret_cast<float4*>(lay + dst + (i % kv4) * 4) = t[q];
        }
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void tree_draft_kernel(const RoundArgs r) {
  extern __shared__ float4 row_dyn[];
  __shared__ SelSmem S;
  __shared__ int tcode_s[kMaxTree], tnode_s[kMaxTree], nd_s;
  __shared__ int rank_s[kTreeSlots];  // greedy: the depth's top m + 1 codes in order
  const int d = blockIdx.x + 1, b = blockIdx.y;
  const size_t row = static_cast<size_t>(b) * r.W + (d - 1);
  dispatch_vpt(r.V, [&](auto vpt) {
    constexpr int VPT = decltype(vpt)::value;
    float zv[VPT];
    load_row<VPT>(r.dlogits + row * r.V, zv);  // before the state: the row always exists
    const StreamState st = r.st[b];
    const int pend = r.ncode[static_cast<size_t>(b) * kTreeSlots];
    if (st.mode != kModeSpec) return;
    if (pend > 0) tree_kv_move(r, b, pend >> 8, pend & 0xFF, d - 1);
    float* x0 = r.X + static_cast<size_t>(b) * r.R * r.H;
    if (d > st.gamma) {  // no node this round at this depth: only row 0 to fill
      if (d == 1) embed_row(r, st.s, st.last, x0);
      return;
    }
    const RowLds L = row_lds(row_dyn, r.V, false);
    store_row<VPT>(zv, L.z);
    int total;
    uint32_t flags = 0;
    // greedy: the nodes' codes are the depth's m highest draft logits, the
    // k-th child of a parent taking the k-th (m = the most children of a
    // parent at this depth); the top-m + 1 set comes from the top-k
    // selection, its order from wave 0's ranking
    int m = 0;
    if (r.greedy) {
      for (int p = 0; p <= r.tnodes; ++p) {
        if (p > 0 && r.dep[p] != d - 1) continue;
        int n = 0;
        for (int i = 1; i <= r.tnodes; ++i) n += r.par[i] == p ? 1 : 0;
        m = max(m, n);
      }
    }
    const int kk = r.greedy ? m + 1 : r.top_k;
    const float T = r.greedy ? 1.0f : r.T;
    if (topk_list<VPT>(zv, kk, T, L, S, r.greedy ? nullptr : r.q + row * r.V, &total, &flags)) {
      const uint64_t seed = frame_seed(st);
      if (r.greedy) {
        // wave 0: rank the set by (logit desc, code asc); tcode_s[k] = the
        // k-th highest; a gap under 1e-4 among the first m + 1 flags the
        // depth
        const int lane = threadIdx.x % kWave;
        if (lane < total) {
          const int ci = L.lidx[lane];
          const float zi = L.z[ci];
          int rank = 0;
          for (int j = 0; j < total; ++j) {
            const int cj = L.lidx[j];
            const float zj = L.z[cj];
            rank += (zj > zi || (zj == zi && cj < ci)) ? 1 : 0;
          }
          rank_s[rank] = ci;
        }
        wave_lds_sync();
        bool near = false;
        if (lane + 1 < total)
          near = static_cast<double>(L.z[rank_s[lane]]) - static_cast<double>(L.z[rank_s[lane + 1]]) < kEpsGap;
        flags = __ballot(near) ? kFlagArgmax : 0u;
        int nd = 0;
        for (int i = 1; i <= r.tnodes; ++i) {
          if (r.dep[i] != d) continue;
          int rank = 0;  // i's place among its parent's children
          for (int j = 1; j < i; ++j) rank += r.par[j] == r.par[i] ? 1 : 0;
          if (threadIdx.x == 0) {
            tcode_s[nd] = rank_s[rank];
            tnode_s[nd] = i;
            r.ncode[static_cast<size_t>(b) * kTreeSlots + i] = rank_s[rank];
          }
          ++nd;
        }
        if (threadIdx.x == 0) {
          r.dflags[row] = flags;
          nd_s = nd;
        }
      } else {
        // wave 0: every draw of the depth from one set of running sums
        const ListSums ls = list_prefix(L.lw, total);
        int nd = 0;  // nodes of depth d
        for (int i = 1; i <= r.tnodes; ++i) {
          if (r.dep[i] != d) continue;
          int code, near;
          list_search(L.lw, L.lidx, total, ls, frame_uniform(seed, st.s + d, kDraft, nd), &code, &near);
          if (near) flags |= kFlagCdf;
          if (threadIdx.x == 0) {
            tcode_s[nd] = code;
            tnode_s[nd] = i;
            r.ncode[static_cast<size_t>(b) * kTreeSlots + i] = code;
          }
          ++nd;
        }
        if (threadIdx.x == 0) {
          r.dflags[row] = flags;
          nd_s = nd;
        }
      }
    } else if (d == 1) {  // meanwhile the other waves gather row 0
      embed_row_span(r, st.s, st.last, x0, threadIdx.x - kWave, kBlock - kWave);
    }
    __syncthreads();
    // every node's verify input, the nodes side by side (a group of threads each)
    const int nd = nd_s;
    const int per = kBlock / nd;
    const int k = threadIdx.x / per;
    if (k < nd)
      embed_row_span(r, st.s + d, tcode_s[k], r.X + (static_cast<size_t>(b) * r.R + tnode_s[k]) * r.H,
                     threadIdx.x - k * per, per);
  });
}

hipError_t launch_tree_draft(const RoundArgs& r, hipStream_t s) {
  hipLaunchKernelGGL(tree_draft_kernel, dim3(r.W, r.B), dim3(kBlock), row_lds_bytes(r.V, false), s, r);
  return hipGetLastError();
}

// Attention of the tree window over rows r0 .. r0 + RB - 1 of one stream
// and one KV head (grid z: row chunks of RB rows).  Keys: the cache
// positions 0..P-1 (P = 1 + the largest row position below G: the committed
// prefix and the root) and the node slots G + i - 1 of the active node rows,
// at most 128.  A row at a position below G (the root, or a prefill row) is
// causal over the prefix; node row i sits at logical position pos[0] +
// dep[i] and sees the whole prefix plus the nodes in anc[i] (itself and its
// ancestors).  K is rotated by its logical position, Q by its row's.
// Phases as in attention_kernel; in phase 2 the 32 lanes of a (row, query
// head) pair take the keys 32 apart.
template <int D>
__global__ __launch_bounds__(kBlock) void tree_attention_kernel(const AttnArgs a) {
  extern __shared__ float smem[];
  constexpr int half = D / 2;
  constexpr int H4 = half / 4;
  constexpr int KS = D + 4;
  const int b = blockIdx.x, g = blockIdx.y;
  const int R = a.R, r0 = blockIdx.z * a.RB;
  const int nr = min(a.RB, R - r0);
  const int kvdim = a.nkv * D;
  const int qdim = a.nq * D;
  const int group = a.nq / a.nkv;
  const int npair = nr * group;
  const int kstr = (a.Gk + 31) & ~31;  // score row stride
  __shared__ int pos_s[kTreeSlots], qp_s[kTreeSlots], dep_s[kTreeSlots];
  __shared__ uint64_t anc_s[kTreeSlots];
  __shared__ int kslot_s[kMaxKeys], klp_s[kMaxKeys], knode_s[kMaxKeys];
  // the rows' positions, depths and masks in LDS (indexing the argument
  // block per lane would turn into memory loads)
  for (int i = threadIdx.x; i < R; i += kBlock) {
    pos_s[i] = a.pos[b * R + i];
    dep_s[i] = a.dep[i];
    anc_s[i] = a.anc[i];
  }
  __syncthreads();
  // the key list, every entry by its own thread: prefix slots 0..P-1, then
  // the active node rows in row order
  int P = 0, nnode = 0;
  for (int r = 0; r < R; ++r) {
    const int pr = pos_s[r];
    if (pr >= 0 && pr < a.G) P = max(P, pr + 1);
    if (r > 0 && pr >= a.G && pr < a.Gk) ++nnode;
  }
  const int p0 = pos_s[0];
  const int np = P + nnode;
  for (int i = threadIdx.x; i < P; i += kBlock) kslot_s[i] = i, klp_s[i] = i, knode_s[i] = 0;
  for (int r = threadIdx.x; r < R; r += kBlock) {
    const int pr = pos_s[r];
    qp_s[r] = pr < 0 ? -1 : (pr < a.G ? pr : (pr < a.Gk ? p0 + dep_s[r] : -1));
    if (r > 0 && pr >= a.G && pr < a.Gk) {
      int before = 0;
      for (int i = 1; i < r; ++i) before += (pos_s[i] >= a.G && pos_s[i] < a.Gk) ? 1 : 0;
      if (P + before < kMaxKeys) kslot_s[P + before] = pr, klp_s[P + before] = p0 + dep_s[r], knode_s[P + before] = r;
    }
  }
  __syncthreads();
  if (P == 0 || np > kMaxKeys || np > a.Gk || nr <= 0) return;  // no active row (np <= G + nodes)
  float* Ks = smem;                  // [np][KS]
  float* Vs = Ks + a.Gk * KS;        // [np][D]
  float* Qs = Vs + a.Gk * D;         // [npair][D]
  float* S = Qs + a.RB * group * D;  // [npair][kstr]
  const float* kb = a.kv + static_cast<size_t>(b) * a.kv_sb + g * D;
  const float* vb = kb + a.kv_vo;

  // ---- phase 1: K (rotated), V, Q (rotated) into LDS; a thread's items
  // two at a time, both items' loads issued before either's stores ----
  const int nk = np * H4, nq = npair * H4;
  struct Item {
    float4 x1, x2, v1, v2, c01, c23;
  };
  auto load_item = [&](int it, Item& m) {
    if (it < nk) {
      const int p = it / H4, i4 = (it % H4) * 4;
      const int sl = kslot_s[p], lp = klp_s[p];
      m.x1 = *reinterpret_cast<const float4*>(kb + sl * kvdim + i4);
      m.x2 = *reinterpret_cast<const float4*>(kb + sl * kvdim + i4 + half);
      m.v1 = *reinterpret_cast<const float4*>(vb + sl * kvdim + i4);
      m.v2 = *reinterpret_cast<const float4*>(vb + sl * kvdim + i4 + half);
      m.c01 = *reinterpret_cast<const float4*>(a.rope + lp * half + i4);
      m.c23 = *reinterpret_cast<const float4*>(a.rope + lp * half + i4 + 2);
    } else if (it < nk + nq) {
      const int jt = it - nk;
      const int pr = jt / H4, i4 = (jt % H4) * 4;
      const int r = r0 + pr / group, j = pr % group;
      const float* qrow = a.Q + static_cast<size_t>(b * R + r) * qdim + (g * group + j) * D;
      const int pq = max(qp_s[r], 0);
      m.x1 = *reinterpret_cast<const float4*>(qrow + i4);
      m.x2 = *reinterpret_cast<const float4*>(qrow + i4 + half);
      m.c01 = *reinterpret_cast<const float4*>(a.rope + pq * half + i4);
      m.c23 = *reinterpret_cast<const float4*>(a.rope + pq * half + i4 + 2);
    }
  };
  auto store_item = [&](int it, const Item& m) {
    if (it >= nk + nq) return;
    int i4;
    float* dst;
    if (it < nk) {
      const int p = it / H4;
      i4 = (it % H4) * 4;
      dst = Ks + p * KS;
      *reinterpret_cast<float4*>(Vs + p * D + i4) = m.v1;
      *reinterpret_cast<float4*>(Vs + p * D + i4 + half) = m.v2;
    } else {
      const int jt = it - nk;
      i4 = (jt % H4) * 4;
      dst = Qs + (jt / H4) * D;
    }
    const float4 k1 = m.x1, k2 = m.x2, c01 = m.c01, c23 = m.c23;
    dst[i4 + 0] = k1.x * c01.x - k2.x * c01.y;  dst[i4 + half + 0] = k2.x * c01.x + k1.x * c01.y;
    dst[i4 + 1] = k1.y * c01.z - k2.y * c01.w;  dst[i4 + half + 1] = k2.y * c01.z + k1.y * c01.w;
    dst[i4 + 2] = k1.z * c23.x - k2.z * c23.y;  dst[i4 + half + 2] = k2.z * c23.x + k1.z * c23.y;
    dst[i4 + 3] = k1.w * c23.z - k2.w * c23.w;  dst[i4 + half + 3] = k2.w * c23.z + k1.w * c23.w;
  };
  for (int it = threadIdx.x; it < nk + nq; it += 2 * kBlock) {
    Item m0, m1;
    load_item(it, m0);
    load_item(it + kBlock, m1);
    store_item(it, m0);
    store_item(it + kBlock, m1);
  }
  __syncthreads();

  // ---- phase 2: scores and softmax, 32 lanes per pair, keys 32 apart ----
  for (int base = 0; base < npair * 32; base += kBlock) {
    const int idx = base + threadIdx.x;
    const int pr = idx >> 5, lane = idx & 31;
    const bool live_pair = pr < npair;
    const int r = live_pair ? r0 + pr / group : 0;
    const int qp = live_pair ? qp_s[r] : -1;
    float* srow = S + (live_pair ? pr : 0) * kstr;
    float mx = -INFINITY;
    for (int p = lane; p < np; p += 32) {
      bool ok = live_pair && qp >= 0;
      if (ok) ok = p < P ? kslot_s[p] <= qp : ((anc_s[r] >> knode_s[p]) & 1ull) != 0ull;
      float sc = -INFINITY;
      if (ok) {
        const float4* q4 = reinterpret_cast<const float4*>(Qs + pr * D);
        const float4* k4 = reinterpret_cast<const float4*>(Ks + p * KS);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
          const float4 x = q4[i], y = k4[i];
          acc += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
        }
        sc = acc * a.scale;
      }
      if (live_pair) srow[p] = sc;
      mx = fmaxf(mx, sc);
    }
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
    float sum = 0.0f;
    for (int p = lane; p < np; p += 32) {
      const float sc = live_pair ? srow[p] : -INFINITY;
      const float e = sc == -INFINITY ? 0.0f : expf(sc - mx);
      if (live_pair) srow[p] = e;
      sum += e;
    }
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 32);
    if (live_pair)
      for (int p = lane; p < np; p += 32) srow[p] = sum > 0.0f ? srow[p] / sum : 0.0f;
  }
  __syncthreads();

  // ---- phase 3: eight output dimensions of one pair per thread ----
  constexpr int D8 = D / 8;
  for (int idx = threadIdx.x; idx < npair * D8; idx += kBlock) {
    const int pr = idx / D8, i8 = (idx % D8) * 8;
    const int r = r0 + pr / group, j = pr % group;
    if (qp_s[r] < 0) continue;
    const float* srow = S + pr * kstr;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
    for (int p = 0; p < np; ++p) {
      const float w = srow[p];
      const float4 v0 = *reinterpret_cast<const float4*>(Vs + p * D + i8);
      const float4 v1 = *reinterpret_cast<const float4*>(Vs + p * D + i8 + 4);
      o[0] += w * v0.x; o[1] += w * v0.y; o[2] += w * v0.z; o[3] += w * v0.w;
      o[4] += w * v1.x; o[5] += w * v1.y; o[6] += w * v1.z; o[7] += w * v1.w;
    }
    const int row = b * R + r, k = (g * group + j) * D + i8;
    if (a.planes != nullptr) {
      if (split_store8(a.planes, a.ptiles, row, k, o)) flag_overflow(a.ovf, nullptr, row);  // active rows only
    } else {
      float* dst = a.out + static_cast<size_t>(row) * qdim + k;
      *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

size_t tree_attention_smem_bytes(int Gk, int d, int RB, int group) {
  const size_t npair = static_cast<size_t>(RB) * group;
  const size_t kstr = (static_cast<size_t>(Gk) + 31) / 32 * 32;
  return (static_cast<size_t>(Gk) * (2 * d + 4) + npair * d + npair * kstr) * sizeof(float);
}

hipError_t tree_attention_allow_smem(int d, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  switch (d) {
#define CPS_TATT_ATTR(D_) \
  case D_:                \
    return hipFuncSetAttribute(reinterpret_cast<const void*>(tree_attention_kernel<D_>), \
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
    CPS_TATT_ATTR(8) CPS_TATT_ATTR(16) CPS_TATT_ATTR(32) CPS_TATT_ATTR(64) CPS_TATT_ATTR(128)
#undef CPS_TATT_ATTR
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_tree_attention(const AttnArgs& a, int B, hipStream_t s) {
  if (a.RB < 1 || a.Gk > kMaxKeys || a.R > kTreeSlots) return hipErrorInvalidValue;
  const size_t shm = tree_attention_smem_bytes(a.Gk, a.d, a.RB, a.nq / a.nkv);
  const dim3 grid(B, a.nkv, (a.R + a.RB - 1) / a.RB);
  switch (a.d) {
#define CPS_TATT(D_)                                                                              \
  case D_:                                                                                        \
    hipLaunchKernelGGL(tree_attention_kernel<D_>, grid, dim3(kBlock), shm, s, a);                 \
    break;
    CPS_TATT(8) CPS_TATT(16) CPS_TATT(32) CPS_TATT(64) CPS_TATT(128)
#undef CPS_TATT
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Accept side of the tree window, one block per stream.  Every node's step
// of the walk was decided by its row in the target kernel (accepted child,
// or the row's draw); thread 0 follows the decisions from the root.  Then
// the path is committed, its nodes' K/V move from their slots (G + i - 1) to
// their positions, h_{s+n} = the last node's output row, and the stream's
// next round (or frame) is set up.
__global__ __launch_bounds__(kBlock) void tree_accept_kernel(const RoundArgs r) {
  __shared__ StreamState st_s;
  __shared__ CallDesc c_s;
  __shared__ cp_spec_stats cnt_s;
  __shared__ uint32_t tfl_s[kTreeSlots], dfl_s[CP_SPEC_MAX_WINDOW];
  __shared__ int tcode_s[kTreeSlots], ncode_s[kTreeSlots];
  __shared__ int par_s[kTreeSlots], dep_s[kTreeSlots];
  __shared__ int v_s, n_s;
  constexpr int kStW = sizeof(StreamState) / 4, kCallW = sizeof(CallDesc) / 4;
  constexpr int kCntW = sizeof(cp_spec_stats) / 8;
  static_assert(kStW <= 32 && kCallW <= 32 && kCntW <= 32, "state words");
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t rb = static_cast<size_t>(b) * r.R;
  // ---- every independent load at once ----
  if (tid < kStW) {
    reinterpret_cast<int*>(&st_s)[tid] = reinterpret_cast<const int*>(r.st + b)[tid];
  } else if (tid >= 32 && tid < 32 + kCallW) {
    reinterpret_cast<int*>(&c_s)[tid - 32] = reinterpret_cast<const int*>(r.call)[tid - 32];
  } else if (tid >= 64 && tid < 64 + kCntW) {
    reinterpret_cast<long long*>(&cnt_s)[tid - 64] = reinterpret_cast<const long long*>(r.sstats + b)[tid - 64];
  } else if (tid >= 128 && tid < 128 + kTreeSlots) {
    const int i = tid - 128;
    tfl_s[i] = i < r.R ? r.tflags[rb + i] : 0u;
    tcode_s[i] = i < r.R ? r.tcode[rb + i] : -1;
    ncode_s[i] = r.ncode[static_cast<size_t>(b) * kTreeSlots + i];
    if (i < CP_SPEC_MAX_WINDOW) dfl_s[i] = i < r.W ? r.dflags[static_cast<size_t>(b) * r.W + i] : 0u;
    par_s[i] = r.par[i];
    dep_s[i] = r.dep[i];
  }
  __syncthreads();
  StreamState st = st_s;
  if (st.mode == kModeDone) return;
  const CallDesc& c = c_s;
  const size_t fb = static_cast<size_t>(st.f) * c.B + b;
  int* out = c.out_codes + fb * r.G;
  const bool spec = st.mode == kModeSpec;
  const int s = st.s, gamma = st.gamma;
  if (tid == 0) {
    cp_spec_stats& cnt = cnt_s;
    if (!spec) {  // prefill: c_1 is row 1's draw (greedy: its argmax)
      const uint32_t f = tfl_s[1] & (kFlagTopk | kFlagCdf | kFlagArgmax);
      count_flags(f, &cnt);
      if (f) st_s.flags |= 1u << 1;
      out[1] = st_s.last = tcode_s[1];
      ++cnt.prefill_passes;
      st_s.s = 1;
      v_s = 1;
      n_s = 1;
    } else {
      uint32_t fl = 0u;
      int v = 0, n = 0;
      for (;;) {  // the walk: at most one node per depth
        const uint32_t tf = tfl_s[v];
        const int j = s + dep_s[v] + 1;
        // the rows the walk visits used their top-k set (greedy: argmax)
        const uint32_t ft = tf & (kFlagTopk | kFlagArgmax);
        if (ft) {
          count_flags(ft, &cnt);
          fl |= 1u << j;
        }
        int dec = -1;  // the accepted child
        if (r.greedy) {
          // the first active child whose code equals the row's argmax
          for (int ch = 1; ch <= r.tnodes && dec < 0; ++ch)
            if (par_s[ch] == v && dep_s[ch] <= gamma && ncode_s[ch] == tcode_s[v]) dec = ch;
          if (dec < 0) {
            out[s + n + 1] = st_s.last = tcode_s[v];
            ++n;
            break;
          }
        } else {
          if (tf & kFlagAccept) {
            ++cnt.near_tie_accept;
            fl |= 1u << j;
          }
          dec = static_cast<int>((tf >> 16) & 0xFFu) - 1;
          if (dec < 1 || dec > r.tnodes) {
            if (tf & kFlagCdf) {
              ++cnt.near_tie_cdf;
              fl |= 1u << j;
            }
            out[s + n + 1] = st_s.last = tcode_s[v];
            ++n;
            break;
          }
        }
        out[s + n + 1] = ncode_s[dec];
        ++n;
        v = dec;
      }
      // the draft depths whose candidates the walk tested: 1..n (depth n's
      // children were tested at the last visited node)
      for (int d = 1; d <= min(n, gamma); ++d) {
        const uint32_t f = dfl_s[d - 1];
        count_flags(f, &cnt);
        if (f) fl |= 1u << (s + d);
      }
    st_s.flags |= fl;
      v_s = v;
      n_s = n;
    }
  }
  __syncthreads();
  const int v = v_s, n = n_s;

  if (spec) {
    if (tid == 0) {
      ++cnt_s.rounds;
      for (int d = 1; d <= gamma; ++d) {
        ++cnt_s.proposed[d - 1];
        if (d <= n - 1) ++cnt_s.accepted[d - 1];
      }
      bool leaf = true;
      for (int ch = 1; ch <= r.tnodes; ++ch)
        if (par_s[ch] == v && dep_s[ch] <= gamma) leaf = false;
      if (leaf) ++cnt_s.bonus;
      st_s.s = s + n;
    }
  }
  // the accepted nodes' K/V move to their positions in the next round's draft
  // kernel: ncode[b][0] = s << 8 | v, or 0 when nothing moves (no node
  // accepted, a prefill round, or the frame complete)
  if (tid == 0) {
    const bool move = spec && v > 0 && s + n < r.G - 1;
    r.ncode[static_cast<size_t>(b) * kTreeSlots] = move ? (s << 8) | v : 0;
  }
  if (tid == 0 && st_s.s >= r.G - 1) {  // frame complete
    if (c.out_flags) c.out_flags[fb] = st_s.flags;
    ++cnt_s.frames;
    cnt_s.codes += r.G - 1;
  }
  __syncthreads();
  st = st_s;

  // ---- h_{s+n} = the last path node's output row (prefill: row 1), and
  // with position-aware offsets the next round's draft inputs ----
  {
    const int H4 = r.H / 4;
    const float4* src = reinterpret_cast<const float4*>(r.Hout + (rb + v) * r.H);
    float4* dst = reinterpret_cast<float4*>(r.hstate + static_cast<size_t>(b) * r.H);
    float4* dx = r.K > 0 ? reinterpret_cast<float4*>(r.dX + static_cast<size_t>(b) * r.W * r.H) : nullptr;
    const float4* off = reinterpret_cast<const float4*>(r.doff);
    for (int i = tid; i < H4; i += kBlock) {
      const float4 hv = src[i];
      dst[i] = hv;
      if (dx != nullptr)
        for (int t = 0; t < r.W; ++t) {
          float4 o = hv;
          if (t < r.K) {
            const float4 bt = off[t * H4 + i];
            o.x += bt.x, o.y += bt.y, o.z += bt.z, o.w += bt.w;
          }
          dx[t * H4 + i] = o;
        }
    }
  }
  if (tid < kCntW)
    reinterpret_cast<long long*>(r.sstats + b)[tid] = reinterpret_cast<const long long*>(&cnt_s)[tid];

  // ---- next round of this stream ----
  if (st.s >= r.G - 1) {
    st.f += 1;
    st.s = 0;
    st.flags = 0;
    st.gamma = 0;
    if (st.f >= c.F) {
      st.mode = kModeDone;
      if (tid < r.R) {
        r.pos[rb + tid] = -1;
        r.thead[rb + tid] = 0;
      }
      if (tid < r.W) r.dhead[static_cast<size_t>(b) * r.W + tid] = 0;
    } else {
      st.mode = kModePrefill;
      set_frame_seed(st, c.seeds[static_cast<size_t>(st.f) * c.B + b]);
      setup_prefill(r, c, b, st.f);
    }
  } else {
    const int s2 = st.s;
    const int g2 = min(r.tdepth, r.G - 2 - s2);
    st.gamma = g2;
    st.mode = kModeSpec;
    if (tid < r.R) {
      const bool act = tid == 0 || dep_s[tid] <= g2;
      r.pos[rb + tid] = tid == 0 ? s2 + 1 : (act ? r.G + tid - 1 : -1);  // node i: slot G + i - 1
      r.thead[rb + tid] = act ? s2 + 1 + dep_s[tid] : 0;
    }
    if (tid < r.W) r.dhead[static_cast<size_t>(b) * r.W + tid] = tid + 1 <= g2 ? s2 + tid + 1 : 0;
  }
  if (tid == 0) r.st[b] = st;
}

hipError_t launch_tree_accept(const RoundArgs& r, hipStream_t s) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3(r.B), dim3(kBlock), 0, s, r);
  return hipGetLastError();
}

}  // namespace cps
