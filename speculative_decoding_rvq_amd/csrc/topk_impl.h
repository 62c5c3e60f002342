// Temperature/top-k softmax of one row of logits, and optional sampling, by
// one block of 256 threads; thread t owns codes [t*VPT, (t+1)*VPT).
//
// Which codes are in the top-k set: order by (logit desc, code asc) and take
// the first k.  Found without sorting the row:
//   1. the row's largest and smallest logits (one block reduction);
//   2. a 2048-bin histogram of floor((zmax - z) * 2047 / (zmax - zmin)); the
//      bin index never decreases as z decreases, so the bins before the one
//      in which the running count reaches k hold members only, the bins after
//      it non-members only;
//   3. the entries of that boundary bin (a handful for smooth rows) are
//      ranked exactly by pairwise comparison in the (logit desc, code asc)
//      order, and the first k - (count before the bin) of them are admitted.
// A boundary bin of more than 256 entries (heavy ties or clustering) falls
// back to an MSB-first radix select on order-preserving 32-bit keys (four
// passes of 8 bits), which gives the exact k-th key; entries equal to it are
// admitted in ascending code order.
// Probabilities are exp((z - zmax) / T) / sum on the set, zero elsewhere;
// sampling walks them straight from registers.
#pragma once

#include <type_traits>

#include "dev_common.h"

namespace cps {

constexpr int kSelBins = 2048;  // value bins of the selection histogram
constexpr int kMaxCand = 256;   // boundary-bin entries ranked exactly

struct TopkSmem {
  union {
    struct {
      uint32_t hist[kSelBins];
      uint32_t cand_key[kMaxCand];
      int cand_id[kMaxCand];
      uint8_t verdict[4096];  // boundary-bin entries: admitted or not, by code
    } sel;
    SampleSmem samp;  // sampling runs after the selection is done
  };
  uint32_t red_mm[8];   // wave max / min keys
  int red_scan[4];      // wave totals of the bin-count scan
  float red_sum[4];     // wave softmax sums
  uint32_t red_kth[4];  // wave smallest member keys
  uint32_t red_out[4];  // wave largest non-member keys
  uint64_t red64[4];
  uint32_t red32[4];
  int redi[8];
  int bsel[4];          // boundary bin, count before it, its size, candidates
  int rsel[2];          // radix digit / remaining
};

struct TopkResult {
  int code;
  uint32_t flags;
};

// Exact k-th largest key by radix select; member[] gets the top-k set.
template <int VPT>
__device__ void radix_members(const uint32_t* key, int k, bool* member, TopkSmem& sm) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int rem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    lds_sync();
    sm.sel.hist[tid] = 0;
    lds_sync();
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      if ((key[j] & pmask) == prefix) atomicAdd(&sm.sel.hist[(key[j] >> shift) & 255u], 1u);
    lds_sync();
    // thread t looks at digit 255 - t: inclusive count of digits >= it
    const int c = static_cast<int>(sm.sel.hist[255 - tid]);
    int total;
    const int excl = block_exclusive_scan(c, sm.redi, &total);
    if (excl < rem && excl + c >= rem) {
      sm.rsel[0] = 255 - tid;
      sm.rsel[1] = rem - excl;
    }
    lds_sync();
    prefix |= static_cast<uint32_t>(sm.rsel[0]) << shift;
    pmask |= 255u << shift;
    rem = sm.rsel[1];
  }
  const uint32_t kth = prefix;
  // ties at the k-th key: the `rem` lowest codes among them are admitted
  int eq = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) eq += key[j] == kth ? 1 : 0;
  int eq_total;
  int rank = block_exclusive_scan(eq, sm.redi + 4, &eq_total);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    if (key[j] > kth) {
      member[j] = true;
    } else if (key[j] == kth) {
      member[j] = rank < rem;
      ++rank;
    } else {
      member[j] = false;
    }
  }
}

// The row's logits come in registers (zv: codes [t*VPT, (t+1)*VPT) of
// thread t), so that callers can issue the loads before anything else.
// pv receives the thread's VPT probabilities (left unset when greedy).
template <int VPT>
__device__ __forceinline__ TopkResult topk_regs(const float (&zv)[VPT], int k, float T,
                                                bool greedy, bool do_sample, float u, float* probs,
                                                TopkSmem& sm, float (&pv)[VPT]) {
  constexpr int V = VPT * kBlock;
  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int base = tid * VPT;
  uint32_t key[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) key[j] = float_key(zv[j]);
  TopkResult res{-1, 0u};
  if (greedy) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const uint64_t c = (static_cast<uint64_t>(key[j]) << 32) |
                         static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(base + j));
      best = c > best ? c : best;
    }
    best = block_max_u64(best, sm.red64);
    const int arg = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    uint32_t second = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      if (base + j != arg) second = key[j] > second ? key[j] : second;
    second = block_max_u32(second, sm.red32);
    res.code = arg;
    if (V > 1) {
      const double gap = static_cast<double>(key_float(static_cast<uint32_t>(best >> 32))) -
                         static_cast<double>(key_float(second));
      if (gap < kEpsGap) res.flags |= kFlagArgmax;
    }
    return res;
  }

  // ---- 1. largest and smallest key; the histogram is cleared meanwhile ----
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    kmax = umax32(kmax, key[j]);
    kmin = key[j] < kmin ? key[j] : kmin;
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  lds_sync();  // the previous row's readers of this LDS are done
  if (lane == 0) {
    sm.red_mm[w] = kmax;
    sm.red_mm[4 + w] = kmin;
  }
  const bool select = k < V;
#pragma unroll
  for (int i = 0; i < kSelBins / kBlock; ++i) sm.sel.hist[tid * (kSelBins / kBlock) + i] = 0u;
  if (tid == 0) sm.bsel[3] = 0;
  lds_sync();
  kmax = umax32(umax32(sm.red_mm[0], sm.red_mm[1]), umax32(sm.red_mm[2], sm.red_mm[3]));
  kmin = sm.red_mm[4];
#pragma unroll
  for (int i = 5; i < 8; ++i) kmin = sm.red_mm[i] < kmin ? sm.red_mm[i] : kmin;
  const float zmax = key_float(kmax);

  bool member[VPT];
  if (!select) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) member[j] = true;
  } else if (kmax == kmin) {  // one value everywhere: the k lowest codes
#pragma unroll
    for (int j = 0; j < VPT; ++j) member[j] = base + j < k;
  } else {
    const float scale = static_cast<float>(kSelBins - 1) / (zmax - key_float(kmin));
    const bool binned = scale > 0.0f && scale <= 3.0e38f;
    auto bin_of = [&](float zz) {
      return static_cast<int>(fminf((zmax - zz) * scale, static_cast<float>(kSelBins - 1)));
    };
    int bstar = 0, cstar = kSelBins + kMaxCand;
    if (binned) {
      // ---- 2. bin histogram and the boundary bin ----
#pragma unroll
      for (int j = 0; j < VPT; ++j) atomicAdd(&sm.sel.hist[bin_of(zv[j])], 1u);
      lds_sync();
      constexpr int BPT = kSelBins / kBlock;
      int cnt[BPT];
      int s = 0;
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        cnt[i] = static_cast<int>(sm.sel.hist[tid * BPT + i]);
        s += cnt[i];
      }
      const int inc = wave_incl_scan(s);
      if (lane == kWave - 1) sm.red_scan[w] = inc;
      lds_sync();
      int excl = inc - s;
      for (int i = 0; i < w; ++i) excl += sm.red_scan[i];
      if (excl < k && excl + s >= k) {
        int c = excl;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          if (c < k && c + cnt[i] >= k) {
            sm.bsel[0] = tid * BPT + i;
            sm.bsel[1] = c;
            sm.bsel[2] = cnt[i];
          }
          c += cnt[i];
        }
      }
      lds_sync();
      bstar = sm.bsel[0];
      cstar = sm.bsel[2];
    }
    if (cstar <= kMaxCand) {
      const int rem = k - sm.bsel[1];
      uint32_t at = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int b = bin_of(zv[j]);
        member[j] = b < bstar || (b == bstar && rem == cstar);
        if (b == bstar) at |= 1u << j;
      }
      if (rem < cstar) {
        // ---- 3. rank the boundary bin's entries exactly ----
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
          if (at & (1u << j)) {
            const int slot = atomicAdd(&sm.bsel[3], 1);
            sm.sel.cand_key[slot] = key[j];
            sm.sel.cand_id[slot] = base + j;
          }
        }
        lds_sync();
        if (tid < cstar) {
          const uint32_t ki = sm.sel.cand_key[tid];
          const int ii = sm.sel.cand_id[tid];
          int rank = 0;
          for (int m = 0; m < cstar; ++m) {
            const uint32_t km = sm.sel.cand_key[m];
            rank += (km > ki || (km == ki && sm.sel.cand_id[m] < ii)) ? 1 : 0;
          }
          sm.sel.verdict[ii] = rank < rem ? 1 : 0;
        }
        lds_sync();
#pragma unroll
        for (int j = 0; j < VPT; ++j)
          if (at & (1u << j)) member[j] = sm.sel.verdict[base + j] != 0;
      }
    } else {
      radix_members<VPT>(key, k, member, sm);
    }
  }

  // ---- softmax on the set; smallest member and largest non-member keys
  // (boundary gap) in the same block reduction ----
  float e[VPT];
  float part = 0.0f;
  uint32_t kth = 0xFFFFFFFFu, out_best = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    e[j] = member[j] ? expf((zv[j] - zmax) / T) : 0.0f;
    part += e[j];
    if (member[j]) kth = key[j] < kth ? key[j] : kth;
    else out_best = umax32(out_best, key[j]);
  }
  part = wave_sum(part);
  kth = wave_min_u32(kth);
  out_best = wave_max_u32(out_best);
  if (lane == 0) {
    sm.red_sum[w] = part;
    sm.red_kth[w] = kth;
    sm.red_out[w] = out_best;
  }
  lds_sync();
  const float Z = (sm.red_sum[0] + sm.red_sum[1]) + (sm.red_sum[2] + sm.red_sum[3]);
  if (select) {
    kth = sm.red_kth[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) kth = sm.red_kth[i] < kth ? sm.red_kth[i] : kth;
    out_best = umax32(umax32(sm.red_out[0], sm.red_out[1]), umax32(sm.red_out[2], sm.red_out[3]));
    const double gap = static_cast<double>(key_float(kth)) - static_cast<double>(key_float(out_best));
    if (gap < kEpsGap) res.flags |= kFlagTopk;
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) pv[j] = e[j] / Z;
  if (do_sample) {
    bool near = false;
    res.code = sample_regs<VPT>(pv, u, sm.samp, &near);
    if (near) res.flags |= kFlagCdf;
  }
  // stores last: the barriers above do not wait for them
  if (probs != nullptr) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) probs[base + j] = pv[j];
  }
  return res;
}

// Thread t's VPT logits of a row.
template <int VPT>
__device__ __forceinline__ void load_row(const float* __restrict__ z, float (&zv)[VPT]) {
#pragma unroll
  for (int j = 0; j < VPT; ++j) zv[j] = z[threadIdx.x * VPT + j];
}

template <int VPT>
__device__ __forceinline__ TopkResult topk_row(const float* __restrict__ z, int k, float T,
                                               bool greedy, bool do_sample, float u, float* probs,
                                               TopkSmem& sm, float (&pv)[VPT]) {
  float zv[VPT];
  load_row<VPT>(z, zv);
  return topk_regs<VPT>(zv, k, T, greedy, do_sample, u, probs, sm, pv);
}

template <typename F>
__device__ __forceinline__ void dispatch_vpt(int V, F&& f) {
  switch (V / kBlock) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    case 16: f(std::integral_constant<int, 16>{}); break;
    default: break;
  }
}

}  // namespace cps
