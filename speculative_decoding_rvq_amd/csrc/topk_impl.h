// Temperature/top-k softmax of one row of logits and the draw from it, by one
// block of 256 threads; thread t owns codes [t*VPT, (t+1)*VPT).
//
// Which codes are in the top-k set: order by (logit desc, code asc) and take
// the first k.  Found without sorting the row:
//   1. the row's largest and smallest logits (one block reduction);
//   2. a 2048-bin histogram of floor((zmax - z) * 2047 / (zmax - zmin)); the
//      bin index never decreases as z decreases, so the bins before the one
//      in which the running count reaches k hold members only, the bins after
//      it non-members only.  Every wave finds that boundary bin from the
//      histogram by itself;
//   3. the entries of the boundary bin (a handful for smooth rows) are ranked
//      exactly in the (logit desc, code asc) order, and the first
//      k - (count before the bin) of them are admitted.
// A boundary bin of more than 256 entries (heavy ties or clustering) falls
// back to an MSB-first radix select on order-preserving 32-bit keys (four
// passes of 8 bits), which gives the exact k-th key; entries equal to it are
// admitted in ascending code order.
// The block meets at three barriers; from then on wave 0 works alone: it
// ranks the boundary bin, compacts the set in ascending code order, and
// forms p = exp((z - zmax) / T) / sum on it (zero elsewhere), ready for
// list_draw.
#pragma once

#include <type_traits>

#include "dev_common.h"

namespace cps {

constexpr int kSelBins = 2048;  // value bins of the selection histogram
constexpr int kMaxCand = 256;   // boundary-bin entries ranked exactly

// Fixed-size LDS of one row's selection.
struct SelSmem {
  uint32_t ckey[kMaxCand];  // boundary-bin candidates: keys and codes
  int ccode[kMaxCand];
  uint8_t verdict[4096];    // candidates: admitted or not, by code
  uint16_t mmask[kBlock];   // per thread: member bits, candidate bits
  uint16_t cmask[kBlock];
  uint32_t red_mm[8];       // wave max / min keys
  uint32_t red_out[4];      // wave largest non-member keys
  int redi[8];
  int rsel[2];              // radix digit / remaining
  int ncand;
};

// V-sized LDS of one row, carved from dynamic shared memory: the logits, the
// draft probabilities (target rows), and a region holding the selection
// histogram, later the compacted set (weights, then 16-bit codes).
struct RowLds {
  float* z;
  float* q;
  uint32_t* hist;
  float* lw;
  uint16_t* lidx;
};
__host__ __device__ constexpr int row_lds_region(int V) {
  return 6 * V > 4 * kSelBins ? 6 * V : 4 * kSelBins;
}
__host__ __device__ constexpr size_t row_lds_bytes(int V, bool with_q) {
  return static_cast<size_t>(4 * V * (with_q ? 2 : 1) + row_lds_region(V));
}
// base: 16-byte aligned; V a multiple of 256, so every array stays aligned.
__device__ __forceinline__ RowLds row_lds(void* base, int V, bool with_q) {
  RowLds L;
  L.z = static_cast<float*>(base);
  L.q = with_q ? L.z + V : nullptr;
  unsigned char* a = static_cast<unsigned char*>(base) + 4 * V * (with_q ? 2 : 1);
  L.hist = reinterpret_cast<uint32_t*>(a);
  L.lw = reinterpret_cast<float*>(a);
  L.lidx = reinterpret_cast<uint16_t*>(a + 4 * V);
  return L;
}

struct TopkResult {
  int code;
  uint32_t flags;
};

// Thread t's VPT logits of a row.
template <int VPT>
__device__ __forceinline__ void load_row(const float* __restrict__ z, float (&zv)[VPT]) {
#pragma unroll
  for (int j = 0; j < VPT; ++j) zv[j] = z[threadIdx.x * VPT + j];
}

// ... and back into an LDS row.
template <int VPT>
__device__ __forceinline__ void store_row(const float (&v)[VPT], float* dst) {
  float* d = dst + threadIdx.x * VPT;
  if constexpr (VPT % 4 == 0) {
#pragma unroll
    for (int j = 0; j < VPT; j += 4)
      *reinterpret_cast<float4*>(d + j) = make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]);
  } else {
#pragma unroll
    for (int j = 0; j < VPT; ++j) d[j] = v[j];
  }
}

// Exact k-th largest key by radix select; member[] gets the top-k set.
// hist: 256 words of LDS; redi: 8 ints; rsel: 2 ints.
template <int VPT>
__device__ void radix_members(const uint32_t* key, int k, bool* member, uint32_t* hist, int* redi,
                              int* rsel) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int rem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    lds_sync();
    hist[tid] = 0;
    lds_sync();
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      if ((key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
    lds_sync();
    // thread t looks at digit 255 - t: inclusive count of digits >= it
    const int c = static_cast<int>(hist[255 - tid]);
    int total;
    const int excl = block_exclusive_scan(c, redi, &total);
    if (excl < rem && excl + c >= rem) {
      rsel[0] = 255 - tid;
      rsel[1] = rem - excl;
    }
    lds_sync();
    prefix |= static_cast<uint32_t>(rsel[0]) << shift;
    pmask |= 255u << shift;
    rem = rsel[1];
  }
  const uint32_t kth = prefix;
  // ties at the k-th key: the `rem` lowest codes among them are admitted
  int eq = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) eq += key[j] == kth ? 1 : 0;
  int eq_total;
  int rank = block_exclusive_scan(eq, redi + 4, &eq_total);
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

// Greedy choice of a row held in registers (zv: codes [t*VPT, (t+1)*VPT) of
// thread t): argmax with ties to the lowest code, and the top-2 gap flag.
// red64 / red32: 4 words of LDS each.
template <int VPT>
__device__ __forceinline__ TopkResult argmax_regs(const float (&zv)[VPT], uint64_t* red64, uint32_t* red32) {
  constexpr int V = VPT * kBlock;
  const int base = threadIdx.x * VPT;
  uint32_t key[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) key[j] = float_key(zv[j]);
  TopkResult res{-1, 0u};
  uint64_t best = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const uint64_t c = (static_cast<uint64_t>(key[j]) << 32) |
                       static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(base + j));
    best = c > best ? c : best;
  }
  best = block_max_u64(best, red64);
  const int arg = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
  uint32_t second = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j)
    if (base + j != arg) second = key[j] > second ? key[j] : second;
  second = block_max_u32(second, red32);
  res.code = arg;
  if (V > 1) {
    const double gap = static_cast<double>(key_float(static_cast<uint32_t>(best >> 32))) -
                       static_cast<double>(key_float(second));
    if (gap < kEpsGap) res.flags |= kFlagArgmax;
  }
  return res;
}

// The top-k set and its softmax for a row held in registers (zv), which the
// caller has also stored into L.z (and the draft row into L.q) before the
// call; the first barrier here publishes both.  Returns false in waves 1-3,
// which have nothing left to do, and true in wave 0, where then
//   L.lidx[0..*total)  the set's codes in ascending order,
//   L.lw[0..*total)    their probabilities (zero up to a multiple of 32),
//   *flags             |= the boundary flag when k < V (k-th largest minus
//                      (k+1)-th largest logit below 1e-4).
// dense, when set, receives every code's probability (zero outside the
// set); its stores are left in flight.
template <int VPT>
__device__ bool topk_list(const float (&zv)[VPT], int k, float T, const RowLds& L, SelSmem& S, float* dense,
                          int* total_out, uint32_t* flags) {
  constexpr int V = VPT * kBlock;
  constexpr int CPL = 4 * VPT;  // codes per lane of wave 0 (4 threads' worth)
  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const int base = tid * VPT;
  uint32_t key[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) key[j] = float_key(zv[j]);

  // ---- 1. largest and smallest key; the histogram is cleared meanwhile ----
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    kmax = umax32(kmax, key[j]);
    kmin = key[j] < kmin ? key[j] : kmin;
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  if (lane == 0) {
    S.red_mm[w] = kmax;
    S.red_mm[4 + w] = kmin;
  }
  {
    uint4* h = reinterpret_cast<uint4*>(L.hist) + tid * (kSelBins / kBlock / 4);
#pragma unroll
    for (int i = 0; i < kSelBins / kBlock / 4; ++i) h[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid == 0) S.ncand = 0;
  lds_sync();
  kmax = umax32(umax32(S.red_mm[0], S.red_mm[1]), umax32(S.red_mm[2], S.red_mm[3]));
  kmin = S.red_mm[4];
#pragma unroll
  for (int i = 5; i < 8; ++i) kmin = S.red_mm[i] < kmin ? S.red_mm[i] : kmin;
  const float zmax = key_float(kmax);

  uint32_t mm = 0, cm = 0;  // member / boundary-candidate bits of the thread's codes
  uint32_t outk = 0;        // largest key of a definite non-member
  int rem = 0;              // candidates to admit
  bool ranked = false;      // block-uniform: the boundary bin needs ranking
  if (k >= V) {
    mm = (1u << VPT) - 1u;
  } else if (kmax == kmin) {  // one value everywhere: the k lowest codes
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      if (base + j < k) mm |= 1u << j;
      else outk = umax32(outk, key[j]);
    }
  } else {
    const float scale = static_cast<float>(kSelBins - 1) / (zmax - key_float(kmin));
    const bool binned = scale > 0.0f && scale <= 3.0e38f;
    auto bin_of = [&](float zz) {
      return static_cast<int>(fminf((zmax - zz) * scale, static_cast<float>(kSelBins - 1)));
    };
    int bstar = 0, before = 0, cstar = kSelBins + kMaxCand;
    if (binned) {
      // ---- 2. bin histogram; each wave finds the boundary bin ----
#pragma unroll
      for (int j = 0; j < VPT; ++j) atomicAdd(&L.hist[bin_of(zv[j])], 1u);
      lds_sync();
      uint32_t h[32];
      const uint4* hp = reinterpret_cast<const uint4*>(L.hist) + lane * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = hp[i];
        h[4 * i] = v.x;
        h[4 * i + 1] = v.y;
        h[4 * i + 2] = v.z;
        h[4 * i + 3] = v.w;
      }
      int s = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) s += static_cast<int>(h[i]);
      const int inc = wave_incl_scan(s);
      const int lb = __ffsll(static_cast<unsigned long long>(__ballot(inc >= k))) - 1;
      int c = inc - s, bb = 0, bc = 0, bn = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int hi = static_cast<int>(h[i]);
        if (c < k && c + hi >= k) {
          bb = 32 * lane + i;
          bc = c;
          bn = hi;
        }
        c += hi;
      }
      bstar = __builtin_amdgcn_readlane(bb, lb);
      before = __builtin_amdgcn_readlane(bc, lb);
      cstar = __builtin_amdgcn_readlane(bn, lb);
    }
    if (cstar <= kMaxCand) {
      rem = k - before;
      ranked = rem < cstar;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int b = bin_of(zv[j]);
        if (b < bstar || (b == bstar && !ranked)) {
          mm |= 1u << j;
        } else if (b == bstar) {
          cm |= 1u << j;
          const int slot = atomicAdd(&S.ncand, 1);
          S.ckey[slot] = key[j];
          S.ccode[slot] = base + j;
        } else {
          outk = umax32(outk, key[j]);
        }
      }
    } else {
      bool member[VPT];
      radix_members<VPT>(key, k, member, L.hist, S.redi, S.rsel);
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (member[j]) mm |= 1u << j;
        else outk = umax32(outk, key[j]);
      }
    }
  }
  if (dense != nullptr) {
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      if (!((mm | cm) & (1u << j))) dense[base + j] = 0.0f;
  }
  outk = wave_max_u32(outk);
  if (lane == 0) S.red_out[w] = outk;
  S.mmask[tid] = static_cast<uint16_t>(mm);
  S.cmask[tid] = static_cast<uint16_t>(cm);
  lds_sync();
  if (w != 0) return false;

  // ---- 3. wave 0: the boundary bin, the compacted set, the softmax ----
  outk = umax32(umax32(S.red_out[0], S.red_out[1]), umax32(S.red_out[2], S.red_out[3]));
  uint64_t M = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) M |= static_cast<uint64_t>(S.mmask[4 * lane + i]) << (i * VPT);
  if (ranked) {
    const int nc = S.ncand;
    uint32_t rej = 0;
    for (int s = lane; s < nc; s += kWave) {
      const uint32_t ks = S.ckey[s];
      const int cs = S.ccode[s];
      int rank = 0;
      for (int m = 0; m < nc; ++m) {
        const uint32_t km = S.ckey[m];
        rank += (km > ks || (km == ks && S.ccode[m] < cs)) ? 1 : 0;
      }
      const bool adm = rank < rem;
      S.verdict[cs] = adm ? 1 : 0;
      if (!adm) {
        rej = umax32(rej, ks);
        if (dense != nullptr) dense[cs] = 0.0f;
      }
    }
    outk = umax32(outk, wave_max_u32(rej));
    wave_lds_sync();
    uint64_t C = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) C |= static_cast<uint64_t>(S.cmask[4 * lane + i]) << (i * VPT);
    while (C) {
      const int b = __ffsll(static_cast<unsigned long long>(C)) - 1;
      C &= C - 1;
      if (S.verdict[lane * CPL + b]) M |= 1ull << b;
    }
  }
  const int n = __popcll(M);
  const int inc = wave_incl_scan(n);
  const int total = __builtin_amdgcn_readlane(inc, kWave - 1);
  int off = inc - n;
  while (M) {
    const int b = __ffsll(static_cast<unsigned long long>(M)) - 1;
    M &= M - 1;
    L.lidx[off++] = static_cast<uint16_t>(lane * CPL + b);
  }
  if (lane < 32 && total + lane < ((total + 31) & ~31)) L.lw[total + lane] = 0.0f;
  wave_lds_sync();
  uint32_t kth = 0xFFFFFFFFu;
  float part = 0.0f;
  for (int i = lane; i < total; i += kWave) {
    const float z = L.z[L.lidx[i]];
    const uint32_t kz = float_key(z);
    kth = kz < kth ? kz : kth;
    const float e = expf((z - zmax) / T);
    L.lw[i] = e;
    part += e;
  }
  const float Z = wave_sum(part);
  for (int i = lane; i < total; i += kWave) {
    const float p = L.lw[i] / Z;
    L.lw[i] = p;
    if (dense != nullptr) dense[L.lidx[i]] = p;
  }
  if (k < V) {
    kth = wave_min_u32(kth);
    const double gap = static_cast<double>(key_float(kth)) - static_cast<double>(key_float(outk));
    if (gap < kEpsGap) *flags |= kFlagTopk;
  }
  wave_lds_sync();
  *total_out = total;
  return true;
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
