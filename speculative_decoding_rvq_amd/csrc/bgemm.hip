// Batched projections and lm_heads on the matrix cores: bf16 weights, fp32
// activations (many activation rows: streams x verify rows).
//
// C[m][n] = sum_k x_m[k] * W[n][k].
//
// Every fp32 activation is carried as two fp16 pieces, x ~ hi + lo
// (split2_pair: 22 significant bits), and the weights as fp16 copies of the
// bf16 values times 2^S, one S per packed matrix (exact: a bf16 value has 8
// significant bits, and S puts the matrix's largest value just below 2^15).
// The tile runs v_mfma_f32_16x16x32_f16 once per piece into one fp32
// accumulator; fp16 x fp16 products are exact in fp32, so the result is the
// fp32 dot product of W and hi + lo up to summation order, then times 2^-S.
//
// Memory traffic is what bounds these shapes, so both operands are read in
// whole cache lines:
//  * weights are packed once, at create, in MFMA fragment order: for each
//    16-column tile and 32-wide K chunk, 64 lanes x 8 fp16 (1 KB) with lane
//    l holding W[16 t + l % 16][32 c + 8 (l / 16) .. +7], chunk-major (the
//    tiles of one chunk side by side).  A wave reads a B fragment as one
//    contiguous 1 KB load;
//  * projection inputs arrive pre-split by the producing kernel (two planes
//    in fragment order); the lm_heads' rows are read row-major, a quad of
//    lanes per 128-byte row segment, each lane holding the 8 values of one
//    fragment entry, split in registers and written as whole entries to a
//    small XOR-swizzled LDS stage private to the wave (no block barrier in
//    the K loop, no bank conflicts on either side).
// Tiling: a block owns (16 FM) x (16 FN) outputs; its wave64s split K: four
// (one a SIMD) once the grid has a block per compute unit, eight (two a
// SIMD, so one's MFMAs cover the other's waits) on smaller grids.  Each wave
// keeps its next two chunks' loads in flight.  The partial tiles (and the
// rows' partial sums of squares) meet in LDS and are added in a fixed order:
// the result does not depend on timing.
//
// RMSNorm: x * g is split; the rows' sums of squares are accumulated on the
// way and 1/sqrt(mean + eps) scales the outputs.  Epilogues: residual add,
// SwiGLU (columns 0..TN/2-1 of a tile are gate rows, TN/2..TN-1 the matching
// up rows), Q write plus K/V append at the row's position, lm_head logits for
// rows grouped by head (final-normed rows written once).
#include <algorithm>

#include "dev_common.h"
#include "kernels.h"

namespace cps {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef f16x8_t h8;


// Packed layouts are chunk-major: fragment (tile t, K chunk c) of a matrix
// packed with NT tiles per chunk is the 1 KB at (c * NT + t) * 512 bf16, so
// the fragments that waves load together (neighbouring tiles of one chunk)
// are neighbours in memory and spread over the cache channels.
__device__ __forceinline__ size_t frag_at(int t, int c, int NT) {
  return (static_cast<size_t>(c) * NT + t) * 512;
}

// Packed 16-column tile j of the block's tile: its tile index in W0 (or, for
// the SwiGLU up half, in W1).
template <int MODE, int FN>
__device__ __forceinline__ int btile(int bx, int j) {
  if (MODE == kSwiGLU) {  // gate tiles, then the matching up tiles
    constexpr int H = FN / 2;
    return bx * H + (j % H);
  }
  return bx * FN + j;
}

// The output tile of this block.  Blocks are dispatched to the eight XCDs in
// turn (linear block id modulo 8), and each XCD's L2 serves only its own
// blocks.  So each XCD takes a contiguous range of column tiles, and its
// blocks, in dispatch order, sweep that range in groups of 32 tiles (GR row
// tiles x GC column tiles): the blocks resident on one XCD at a time share
// their weight and activation tiles through its L2.  Grids of at most one
// block per compute unit (all resident at once) and grids that do not split
// that way keep the plain order.
__device__ __forceinline__ void block_tile(int* bx, int* by) {
  constexpr int kXcd = 8, kGroup = 32;
  const int NBX = gridDim.x, NBY = gridDim.y;
  const int cpx = NBX / kXcd;
  const int GC = cpx >= 8 ? 8 : cpx, GR = GC > 0 ? kGroup / GC : 0;
  if (NBX * NBY <= 256 || NBX % kXcd || GC == 0 || kGroup % GC || cpx % GC || NBY % GR) {
    *bx = blockIdx.x;
    *by = blockIdx.y;
    return;
  }
  const int L = blockIdx.x + NBX * blockIdx.y;
  const int x = L % kXcd, i = L / kXcd;
  const int g = i / kGroup, j = i % kGroup, gpc = cpx / GC;
  *bx = x * cpx + (g % gpc) * GC + j % GC;
  *by = (g / gpc) * GR + j / GC;
}

// Finishes a lane's share of one fragment pair: va / vb are the scaled sums
// of four consecutive columns of row `row` in fragments a and b.  SwiGLU: a
// gate and its up values, oa the column of the activations; otherwise oa /
// ob are the output columns of the two fragments (32 adjacent columns for
// the residual add).  pp: the row's position (Q/K/V).  Lanes 16 apart hold
// the same row (the residual add's sums of squares fold over them).
// The residual add's operands that do not depend on the products: the old
// values at columns oa / ob and the next projection's gains there.
struct AddOps {
  floatx4 ya, yb, ga, gb;
};
__device__ __forceinline__ AddOps add_operands(const GemvArgs& a, int row, int oa, int ob) {
  AddOps o;
  o.ya = *reinterpret_cast<const floatx4*>(a.Y + static_cast<size_t>(row) * a.ldy + oa);
  o.yb = *reinterpret_cast<const floatx4*>(a.Y + static_cast<size_t>(row) * a.ldy + ob);
  if (a.out_planes != nullptr && a.out_g != nullptr) {
    o.ga = *reinterpret_cast<const floatx4*>(a.out_g + oa);
    o.gb = *reinterpret_cast<const floatx4*>(a.out_g + ob);
  } else {
    o.ga = o.gb = floatx4{1.0f, 1.0f, 1.0f, 1.0f};
  }
  return o;
}
// ops: the residual add's operands when loaded earlier (else loaded here).
template <int MODE>
__device__ __forceinline__ void finish_pair(const GemvArgs& a, int row, int pp, int lg, const float (&va)[4],
                                            const float (&vb)[4], int oa, int ob, const AddOps* ops = nullptr) {
  if (MODE == kSwiGLU) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = va[i] / (1.0f + expf(-va[i])) * vb[i];
    if (a.out_planes != nullptr) {
      if (split_store4(a.out_planes, a.out_ptiles, row, oa, y)) flag_overflow(a.ovf, a.pos, row);
    } else {
      *reinterpret_cast<floatx4*>(a.Y + static_cast<size_t>(row) * a.ldy + oa) = floatx4{y[0], y[1], y[2], y[3]};
    }
    return;
  }
  if (MODE == kAdd) {
    const AddOps o = ops != nullptr ? *ops : add_operands(a, row, oa, ob);
    float xa[4], xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xa[i] = o.ya[i] + va[i];
      xb[i] = o.yb[i] + vb[i];
    }
    *reinterpret_cast<floatx4*>(a.Y + static_cast<size_t>(row) * a.ldy + oa) = floatx4{xa[0], xa[1], xa[2], xa[3]};
    *reinterpret_cast<floatx4*>(a.Y + static_cast<size_t>(row) * a.ldy + ob) = floatx4{xb[0], xb[1], xb[2], xb[3]};
    if (a.out_planes != nullptr) {
      // the next normed projection's input: x * g split, and the row's sum
      // of squares over these 32 columns (four lanes of the row)
      float ya4[4], yb4[4], ssr = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ssr = fmaf(xa[i], xa[i], ssr);
        ya4[i] = xa[i] * o.ga[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ssr = fmaf(xb[i], xb[i], ssr);
        yb4[i] = xb[i] * o.gb[i];
      }
      bool bad = split_store4(a.out_planes, a.out_ptiles, row, oa, ya4);
      bad |= split_store4(a.out_planes, a.out_ptiles, row, ob, yb4);
      if (bad) flag_overflow(a.ovf, a.pos, row);
      ssr += __shfl_xor(ssr, 16);
      ssr += __shfl_xor(ssr, 32);
      if (lg == 0) a.out_ssp[static_cast<size_t>(row) * (a.N / 32) + oa / 32] = ssr;
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int o = h ? ob : oa;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = h ? vb[i] : va[i];
    if (MODE == kHead) {
      // rows of draft offset k = row % xdiv add head . b_k
      const int ko = row % a.xdiv;
      if (a.hb != nullptr && ko >= 1 && ko <= a.hbK) {
        const floatx4 bias =
            *reinterpret_cast<const floatx4*>(a.hb + (static_cast<size_t>(blockIdx.z) * a.hbK + (ko - 1)) * a.N + o);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += bias[i];
      }
      *reinterpret_cast<floatx4*>(a.Y + static_cast<size_t>(row) * a.ldy + o) = floatx4{v[0], v[1], v[2], v[3]};
    } else if (MODE == kQKV) {
      if (o < a.qdim) {
        *reinterpret_cast<floatx4*>(a.Y + static_cast<size_t>(row) * a.ldy + o) = floatx4{v[0], v[1], v[2], v[3]};
      } else if (pp >= 0 && pp < a.kv_positions) {
        const int b = row / a.rows_per_stream;
        float* base = a.kv + static_cast<size_t>(b) * a.kv_sb + static_cast<size_t>(pp) * a.kvdim;
        const int oo = o - a.qdim;
        float* dst = oo < a.kvdim ? base + oo : base + a.kv_vo + (oo - a.kvdim);
        *reinterpret_cast<floatx4*>(dst) = floatx4{v[0], v[1], v[2], v[3]};
      }
    }
  }
}

// NW waves, each taking 1/NW of K: eight while the grid has fewer blocks
// than compute units (more loads in flight per block), four from a block per
// compute unit on (the partial tiles then meet in one exchange, not two).
template <int MODE, int FM, int FN, bool NORM, bool PL, int NW>
__global__ __launch_bounds__(NW * kWave) void bgemm_kernel(const GemvArgs a) {
  static_assert(NW == 4 || NW == 8, "waves of a K-split block");
  constexpr int kGT = NW * kWave;
  constexpr int TM = 16 * FM, TN = 16 * FN;
  constexpr int SW = PL ? 1 : NW;  // stage: only the in-kernel split uses it
  struct StageT { u32x4 f[SW][FM * kPieces][kWave]; };  // split fragments of one chunk
  // partial tiles in fragment order (lane l's four values of fragment
  // (f, n) as one 16-byte entry), four slots
  struct PartT { floatx4 v[4][FM * FN][kWave]; float ssq[NW][TM]; };
  __shared__ union {
    StageT stage;
    PartT part;
  } sm;
  __shared__ float rinv_s[TM];
  __shared__ int rows_s[TM];
  __shared__ int pos_s[TM];  // Q/K/V: the rows' positions

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  int bx = blockIdx.x, by = blockIdx.y;
  if (MODE != kHead) block_tile(&bx, &by);
  const int li = lane & 15, lg = lane >> 4;

  // ---- the block's activation rows ----
  const uint16_t* W0 = static_cast<const uint16_t*>(a.W0);
  int tile0 = 0;  // lm_heads: the head's first tile
  int count;
  if (MODE == kHead) {
    const int j = blockIdx.z;  // head j+1: its rows, ascending, slice blockIdx.y
    __shared__ int red_h[NW];
    count = head_rows_slice<kGT>(a.head, a.M, j + 1, by * TM, TM, rows_s, red_h);
    if (count <= 0) return;
    tile0 = j * (a.N / 16);
  } else {
    const int m0 = by * TM;
    count = min(TM, a.M - m0);
    if (tid < TM) rows_s[tid] = tid < count ? m0 + tid : -1;
  }
  __syncthreads();

  // ---- operand pointers.  Activations: for row tile f, lane l reads row
// 16 f + l / 4, k 8 (l % 4) .. +7 of each chunk (a quad covers one 128-byte
// row segment) and so holds exactly fragment entry (l / 4) + 16 (l % 4).  A
// missing row reads X row 0: its outputs and sum of squares are never used.
  const int cw = a.K / 32 / NW;  // chunks of this wave (even, >= 2)
  const int c0 = wave * cw;
  // Grids of at most one block per compute unit (every operand stays in the
  // L2 of its XCD): blocks start their K walk at different chunks, so that
  // the blocks that share a tile do not all miss on the same lines at once.
  // Larger grids run in several waves of blocks: there the blocks of a group
  // walk K together and share each chunk through the L2.
  const bool stagger = MODE == kHead || gridDim.x * gridDim.y <= 256;
  const int rot = stagger ? (bx / 8 + 2 * by + blockIdx.z) % cw : 0;
  auto rc = [&](int step) { const int c = step + rot; return c >= cw ? c - cw : c; };
  const int kl = 8 * (lane & 3);
  const float* xb = a.X + c0 * 32 + kl;
  int xo[FM];  // row offsets in floats
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int row = rows_s[16 * f + (lane >> 2)];
    xo[f] = (row >= 0 ? row / a.xdiv : 0) * a.ldx;
  }
  const float* gr = NORM ? a.norm_g + c0 * 32 + kl : nullptr;
  const uint16_t* wr[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const uint16_t* Wm = (MODE == kSwiGLU && j >= FN / 2) ? static_cast<const uint16_t*>(a.W1) : W0;
    wr[j] = Wm + frag_at(tile0 + btile<MODE, FN>(bx, j), c0, a.wtiles) + lane * 8;
  }
  const size_t wstep = static_cast<size_t>(a.wtiles) * 512;  // one chunk further

  struct BFrag {  // ... and weight fragments
    u32x4 w[FN];
  };
  auto fetch_b = [&](int c) __attribute__((always_inline)) {
    BFrag f;
#pragma unroll
    for (int j = 0; j < FN; ++j) f.w[j] = *reinterpret_cast<const u32x4*>(wr[j] + rc(c) * wstep);
    return f;
  };
  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  float ss[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) ss[i] = 0.0f;

  // Epilogue operands that do not depend on the products.  Pre-split
  // RMSNorm rows' sums of squares per 32-wide K chunk (TPR neighbouring
  // threads read a row's, each a contiguous run) and the Q/K/V rows'
  // positions are loaded after the K loop; the residual add's old values and
  // next gains of the pairs this wave finishes go out after the first chunks
  // and stay in flight during the K loop.
  constexpr int TPR = kGT / TM;
  constexpr int kRun = 8;
  constexpr int U = FM * (FN / 2);          // fragment pairs of the tile
  constexpr int UPW = (U + NW - 1) / NW;    // ... finished per wave
  const int np = a.K / 32, per = np / TPR;
  const int srow = rows_s[tid / TPR];
  const float* sp = (PL && NORM) ? a.ssp + static_cast<size_t>(srow >= 0 ? srow : 0) * np + (tid % TPR) * per
                                 : nullptr;
  float sv[kRun];
  int pv = -1;
  // (not for the widest tile at eight waves, whose registers are full)
  constexpr bool kPreAdd = MODE == kAdd && (NW == 4 || FM * FN <= 16);
  AddOps pre[kPreAdd ? UPW : 1];
  const int n0col = bx * TN;
  const int c4 = 4 * lg;
  // pair u: fragments (f, na) and (f, nb), na = j and nb = j + FN / 2 for
  // SwiGLU (a gate tile and its up tile), na = 2 j and nb = 2 j + 1
  // otherwise (32 adjacent columns)
  auto pair_of = [&](int u, int& f, int& j, int& na, int& nb) {
    f = u / (FN / 2);
    j = u % (FN / 2);
    na = MODE == kSwiGLU ? j : 2 * j;
    nb = MODE == kSwiGLU ? j + FN / 2 : 2 * j + 1;
  };
  auto epilogue_loads = [&]() __attribute__((always_inline)) {
    if constexpr (kPreAdd) {
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        const int u = wave + NW * i;
        int f, j, na, nb;
        pair_of(u < U ? u : 0, f, j, na, nb);
        const int row = rows_s[16 * f + li];
        if (u < U && row >= 0) pre[i] = add_operands(a, row, n0col + 16 * na + c4, n0col + 16 * nb + c4);
      }
    }
  };
  if constexpr (PL) {
    // activations pre-split: plane p of row tile t, chunk c is the 1 KB
    // fragment at ((c * T + t) * 2 + p) * 512 fp16 (T row tiles)
    const uint16_t* ab = a.planes + (static_cast<size_t>(c0) * a.ptiles + by * FM) * kPieces * 512 + lane * 8;
    const size_t astep = static_cast<size_t>(a.ptiles) * kPieces * 512;
    struct PFrag {
      u32x4 x[FM][kPieces];
    };
    auto fetch_p = [&](int c) __attribute__((always_inline)) {
      PFrag f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int p = 0; p < kPieces; ++p)
          f.x[i][p] = *reinterpret_cast<const u32x4*>(ab + rc(c) * astep + (i * kPieces + p) * 512);
      return f;
    };
    auto mma_p = [&](const PFrag& fa, const BFrag& fb) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < kPieces; ++p)
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int n = 0; n < FN; ++n)
            acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, fb.w[n]),
                                                               __builtin_bit_cast(h8, fa.x[f][p]), acc[f][n], 0, 0, 0);
    };
    // two chunks of loads in flight, issued in the loop's order (the wait
    // counts before each chunk's MFMAs then cover only that chunk); the
    // last two chunks' MFMAs follow the loop, with nothing more to fetch
    // (deeper prefetch, four chunks, measured no faster)
    PFrag pa0 = fetch_p(0);
    BFrag pb0 = fetch_b(0);
    __builtin_amdgcn_sched_barrier(0);
    PFrag pa1 = fetch_p(1);
    BFrag pb1 = fetch_b(1);
    __builtin_amdgcn_sched_barrier(0);
    epilogue_loads();
    __builtin_amdgcn_sched_barrier(0);
    for (int c = 0; c + 2 < cw; c += 2) {
      mma_p(pa0, pb0);
      __builtin_amdgcn_sched_barrier(0);
      pa0 = fetch_p(c + 2);
      __builtin_amdgcn_sched_barrier(0);
      pb0 = fetch_b(c + 2);
      __builtin_amdgcn_sched_barrier(0);
      mma_p(pa1, pb1);
      __builtin_amdgcn_sched_barrier(0);
      pa1 = fetch_p(c + 3);
      __builtin_amdgcn_sched_barrier(0);
      pb1 = fetch_b(c + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    mma_p(pa0, pb0);
    __builtin_amdgcn_sched_barrier(0);
    mma_p(pa1, pb1);
  } else {
  struct AFrag {  // one chunk of this lane's activation loads
    floatx4 x[FM][2];
    floatx4 g[2];
  };
  auto fetch_a = [&](int step) __attribute__((always_inline)) {
    const int c = rc(step);
    AFrag f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      f.x[i][0] = *reinterpret_cast<const floatx4*>(xb + xo[i] + c * 32);
      f.x[i][1] = *reinterpret_cast<const floatx4*>(xb + xo[i] + c * 32 + 4);
    }
    if constexpr (NORM) {
      f.g[0] = *reinterpret_cast<const floatx4*>(gr + c * 32);
      f.g[1] = *reinterpret_cast<const floatx4*>(gr + c * 32 + 4);
    } else {
      f.g[0] = f.g[1] = floatx4{1.0f, 1.0f, 1.0f, 1.0f};
    }
    return f;
  };


  // Stage slots are XOR-swizzled, entry e at e ^ (((e >> 4) & 3) << 1), so
  // that both this lane mapping's writes and the fragment reads (lane e reads
  // entry e) hit eight distinct 16-byte bank groups per eight lanes.
  auto slot = [](int e) { return e ^ (((e >> 4) & 3) << 1); };
  const int wslot = slot((lane >> 2) + 16 * (lane & 3));
  const int rslot = slot(lane);
  // split x * g of one chunk into the wave's LDS stage: two fp16 pieces,
  // two values per word
  bool bad = false;
  auto split_store = [&](const AFrag& fr) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      uint32_t hp[4], lp[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float x0 = fr.x[i][e / 4][e % 4], x1 = fr.x[i][e / 4][e % 4 + 1];
        ss[i] = fmaf(x0, x0, ss[i]);
        ss[i] = fmaf(x1, x1, ss[i]);
        const float y0 = NORM ? x0 * fr.g[e / 4][e % 4] : x0;
        const float y1 = NORM ? x1 * fr.g[e / 4][e % 4 + 1] : x1;
        split2_pair(y0, y1, hp[e / 2], lp[e / 2], bad);
      }
      sm.stage.f[wave][i * kPieces + 0][wslot] = u32x4{hp[0], hp[1], hp[2], hp[3]};
      sm.stage.f[wave][i * kPieces + 1][wslot] = u32x4{lp[0], lp[1], lp[2], lp[3]};
    }
  };
  auto mma = [&](const BFrag& fb) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      h8 ap[FM];
#pragma unroll
      for (int f = 0; f < FM; ++f) ap[f] = __builtin_bit_cast(h8, sm.stage.f[wave][f * kPieces + p][rslot]);
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int n = 0; n < FN; ++n)
          acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, fb.w[n]), ap[f], acc[f][n], 0,
                                                             0, 0);
    }
  };

  // ---- K loop (an even number of chunks per wave), two chunks of loads in
  // flight per operand: a chunk's activation registers are refilled as soon
  // as they are split, its weight registers once its MFMAs are issued; the
  // last two chunks follow the loop (issued in the loop's order, see
  // above) ----
  AFrag fa0 = fetch_a(0);
  __builtin_amdgcn_sched_barrier(0);
  BFrag fb0 = fetch_b(0);
  __builtin_amdgcn_sched_barrier(0);
  AFrag fa1 = fetch_a(1);
  __builtin_amdgcn_sched_barrier(0);
  BFrag fb1 = fetch_b(1);
  __builtin_amdgcn_sched_barrier(0);
  for (int c = 0; c + 2 < cw; c += 2) {
    wave_lds_sync();  // the previous chunk's fragment reads are done
    split_store(fa0);
    __builtin_amdgcn_sched_barrier(0);
    fa0 = fetch_a(c + 2);
    __builtin_amdgcn_sched_barrier(0);
    wave_lds_sync();
    mma(fb0);
    __builtin_amdgcn_sched_barrier(0);
    fb0 = fetch_b(c + 2);
    __builtin_amdgcn_sched_barrier(0);
    wave_lds_sync();
    split_store(fa1);
    __builtin_amdgcn_sched_barrier(0);
    fa1 = fetch_a(c + 3);
    __builtin_amdgcn_sched_barrier(0);
    wave_lds_sync();
    mma(fb1);
    __builtin_amdgcn_sched_barrier(0);
    fb1 = fetch_b(c + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  wave_lds_sync();
  split_store(fa0);
  wave_lds_sync();
  mma(fb0);
  wave_lds_sync();
  split_store(fa1);
  wave_lds_sync();
  mma(fb1);
  if (bad) flag_overflow(a.ovf, nullptr, 0);  // the heads' rows are all in use

  }

  // ---- the partial tiles meet in LDS in a fixed order.  Eight waves:
  // waves 4-7 hand theirs to waves 0-3 (w + w+4), which store the four
  // sums; four waves store their own.  One more barrier and every wave reads
  // the four sums of the fragments it finishes as (s0 + s1) + (s2 + s3).
  // Entries are 16 bytes per lane, in lane order: no bank conflicts.  The
  // rows' partial sums of squares go along. ----
  // every wave past its last stage read (stage and part share LDS; the
  // pre-split path at four waves never touches the stage)
  // the rows' sums of squares and positions: all loads at once, in flight
  // during the tile exchange (issued during the K loop instead they slowed
  // gate/up and Q/K/V)
  if constexpr (PL && NORM) {
#pragma unroll
    for (int i = 0; i < kRun; ++i) sv[i] = (srow >= 0 && i < per) ? sp[i] : 0.0f;
  }
  if (MODE == kQKV && tid < TM && rows_s[tid] >= 0) pv = a.pos[rows_s[tid]];
  if (!PL || NW == 8) __syncthreads();
  if (NORM && !PL) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float t = ss[i];
      t += __shfl_xor(t, 1);
      t += __shfl_xor(t, 2);
      if ((lane & 3) == 0) sm.part.ssq[wave][16 * i + (lane >> 2)] = t;
    }
  }
  if (NW == 8) {
    if (wave >= 4) {
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int n = 0; n < FN; ++n) sm.part.v[wave - 4][f * FN + n][lane] = acc[f][n];
    }
    __syncthreads();
    if (wave < 4) {  // slot `wave` is this wave's alone from here on
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int n = 0; n < FN; ++n) {
          acc[f][n] += sm.part.v[wave][f * FN + n][lane];
          sm.part.v[wave][f * FN + n][lane] = acc[f][n];
        }
    }
  } else {
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int n = 0; n < FN; ++n) sm.part.v[wave][f * FN + n][lane] = acc[f][n];
  }
  if constexpr (PL && NORM) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < kRun; ++i)
      if (i < per) t += sv[i];
    for (int i = kRun; i < per; ++i) t += srow >= 0 ? sp[i] : 0.0f;
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) t += __shfl_xor(t, o);
    if (tid % TPR == 0) rinv_s[tid / TPR] = 1.0f / sqrtf(t / static_cast<float>(a.K) + a.eps);
  }
  if (MODE == kQKV && tid < TM) pos_s[tid] = pv;
  __syncthreads();
  auto rinv_of = [&](int r) {
    if constexpr (PL) {
      return rinv_s[r];
    } else {
      float t = (sm.part.ssq[0][r] + sm.part.ssq[1][r]) + (sm.part.ssq[2][r] + sm.part.ssq[3][r]);
      if (NW == 8)
        t = ((sm.part.ssq[0][r] + sm.part.ssq[4][r]) + (sm.part.ssq[1][r] + sm.part.ssq[5][r])) +
            ((sm.part.ssq[2][r] + sm.part.ssq[6][r]) + (sm.part.ssq[3][r] + sm.part.ssq[7][r]));
      return 1.0f / sqrtf(t / static_cast<float>(a.K) + a.eps);
    }
  };

  // final-normed rows for the heads' caller (the column tiles split K)
  if (MODE == kHead && NORM && a.xnorm_out != nullptr) {
    const int k4 = a.K / 4;
    const int per = (k4 + gridDim.x - 1) / gridDim.x;
    const int q0 = bx * per, q1 = min(k4, q0 + per);
    const int w = q1 - q0;
    for (int idx = tid; w > 0 && idx < count * w; idx += kGT) {
      const int r = idx / w, c = 4 * (q0 + idx % w);
      const int row = rows_s[r];
      if (row % a.xdiv != 0) continue;  // one writer per X row
      const float4 x = *reinterpret_cast<const float4*>(a.X + static_cast<size_t>(row / a.xdiv) * a.ldx + c);
      const float4 g = *reinterpret_cast<const float4*>(a.norm_g + c);
      const float ri = rinv_of(r);
      *reinterpret_cast<float4*>(a.xnorm_out + static_cast<size_t>(row / a.xdiv) * a.K + c) =
          make_float4(x.x * g.x * ri, x.y * g.y * ri, x.z * g.z * ri, x.w * g.w * ri);
    }
  }

  // ---- each wave finishes fragment pairs u = wave, wave + NW, ... (pair_of).
  // Lane l holds row 16 f + l % 16 and, of each fragment, the four columns
  // 4 (l / 16) .. +3, so every store writes 16 (fp32) or 8 (fp16) bytes. ----
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int u = wave + NW * i;
    if (u >= U) break;
    int f, j, na, nb;
    pair_of(u, f, j, na, nb);
    const int r = 16 * f + li;
    const int row = rows_s[r];
    const float rs = NORM ? rinv_of(r) : 1.0f;
    float va[4], vb[4];
    {
      const floatx4 a0 = sm.part.v[0][f * FN + na][lane], a1 = sm.part.v[1][f * FN + na][lane];
      const floatx4 a2 = sm.part.v[2][f * FN + na][lane], a3 = sm.part.v[3][f * FN + na][lane];
      const floatx4 b0 = sm.part.v[0][f * FN + nb][lane], b1 = sm.part.v[1][f * FN + nb][lane];
      const floatx4 b2 = sm.part.v[2][f * FN + nb][lane], b3 = sm.part.v[3][f * FN + nb][lane];
      const float wa = a.wscale0, wb = MODE == kSwiGLU ? a.wscale1 : a.wscale0;  // 2^-S, exact
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        va[i] = ((a0[i] + a1[i]) + (a2[i] + a3[i])) * wa * rs;
        vb[i] = ((b0[i] + b1[i]) + (b2[i] + b3[i])) * wb * rs;
      }
    }
    if (row < 0) continue;
    if (MODE == kSwiGLU)
      finish_pair<MODE>(a, row, -1, lg, va, vb, bx * (TN / 2) + 16 * j + c4, 0);
    else
      finish_pair<MODE>(a, row, MODE == kQKV ? pos_s[r] : -1, lg, va, vb, n0col + 16 * na + c4,
                        n0col + 16 * nb + c4, kPreAdd ? &pre[i] : nullptr);
  }
}

// ---------------------------------------------------------------------------
// Large batches: 128 x 192 block tiles whose operand chunks are staged in LDS
// and shared by the block's four waves.  Each wave owns a 64 x 96 sub-tile
// over the whole K, so there are no partial tiles to exchange; the epilogue
// runs from its registers (finish_pair).  A chunk (32 of K) is 16 KB of
// activation pieces (eight row tiles, two planes) and 12 KB of weight
// fragments, copied global -> registers -> LDS by all 256 threads (seven
// 16-byte entries each, consecutive threads on consecutive entries), two
// chunks ahead of the MFMAs; one barrier per chunk.  Two blocks fit a
// compute unit.  SwiGLU: wave column wn takes gate tiles 3 wn .. 3 wn + 2 and
// the matching up tiles, so its gate and up values meet in its registers.
constexpr int kLW = 4;            // waves of a staged block
constexpr int kLT = kLW * kWave;  // 256 threads

// FM x FN fragments per wave, waves 2 x 2 (launched with 4 x 6).
template <int MODE, bool NORM, int FM, int FN>
__global__ __launch_bounds__(kLT, 2) void bgemm_lds_kernel(const GemvArgs a) {
  constexpr int BM = 2 * FM, BN = 2 * FN;
  constexpr int TM = 16 * BM, TN = 16 * BN;
  constexpr int AE = BM * kPieces * kWave;  // activation entries of a chunk
  constexpr int SE = AE + BN * kWave;       // + weight entries
  constexpr int PT = SE / kLT, PA = AE / kLT;
  static_assert(SE % kLT == 0 && AE % kLT == 0, "stage entries per thread");
  __shared__ u32x4 stg[2][SE];
  __shared__ float rinv_s[TM];
  __shared__ int rows_s[TM];
  __shared__ int pos_s[TM];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int li = lane & 15, lg = lane >> 4;
  int bx = blockIdx.x, by = blockIdx.y;
  block_tile(&bx, &by);
  const int m0 = by * TM;
  if (tid < TM) {
    const bool in = m0 + tid < a.M;
    rows_s[tid] = in ? m0 + tid : -1;
    pos_s[tid] = (MODE == kQKV && in) ? a.pos[m0 + tid] : -1;
  }

  // ---- the thread's stage entries: PA of activations, then weights.
  // Sources as a wave-uniform byte base (scalar registers) plus the lane's
  // 32-bit offset: entry i of thread t is activation entry t + 256 i, or
  // lane t % 64 of weight tile j = wave + 4 (i - PA) of the block. ----
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const char* abase = reinterpret_cast<const char*>(a.planes) + static_cast<size_t>(by) * BM * kPieces * 1024;
  const char* bbase[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    bbase[i] = nullptr;
    if (i >= PA) {
      const int j = wave_u + kLW * (i - PA);
      const bool up = MODE == kSwiGLU && j >= BN / 2;
      const int t = MODE == kSwiGLU ? bx * (BN / 2) + (up ? j - BN / 2 : j) : bx * BN + j;
      bbase[i] = reinterpret_cast<const char*>((up ? a.W1 : a.W0)) + frag_at(t, 0, a.wtiles) * 2;
    }
  }
  const uint32_t avo = static_cast<uint32_t>(tid) * 16, bvo = static_cast<uint32_t>(lane) * 16;
  const size_t astep = static_cast<size_t>(a.ptiles) * kPieces * 1024;  // bytes per chunk
  const size_t wstep = static_cast<size_t>(a.wtiles) * 1024;
  struct Pre {
    u32x4 v[PT];
  };
  auto load = [&](int c) __attribute__((always_inline)) {
    Pre q;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const char* src = i < PA ? abase + static_cast<size_t>(c) * astep + i * kLT * 16 + avo
                               : bbase[i] + static_cast<size_t>(c) * wstep + bvo;
      q.v[i] = *reinterpret_cast<const u32x4*>(src);
    }
    return q;
  };
  auto store = [&](int sidx, const Pre& q) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PT; ++i) stg[sidx][tid + i * kLT] = q.v[i];
  };
  // the wave's B tiles in the stage
  int bt[FN];
#pragma unroll
  for (int n = 0; n < FN; ++n)
    bt[n] = MODE == kSwiGLU ? (n < FN / 2 ? wn * (FN / 2) + n : BN / 2 + wn * (FN / 2) + n - FN / 2) : wn * FN + n;

  floatx4 acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int n = 0; n < FN; ++n) acc[f][n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // the wave's fragments of a chunk, all read before its MFMAs
  struct Frags {
    u32x4 w[FN];
    u32x4 x[FM][kPieces];
  };
  auto frags = [&](int sidx) __attribute__((always_inline)) {
    Frags g;
#pragma unroll
    for (int n = 0; n < FN; ++n) g.w[n] = stg[sidx][AE + bt[n] * kWave + lane];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int p = 0; p < kPieces; ++p) g.x[f][p] = stg[sidx][((wm * FM + f) * kPieces + p) * kWave + lane];
    return g;
  };
  auto mma = [&](const Frags& g) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int p = 0; p < kPieces; ++p)
#pragma unroll
        for (int n = 0; n < FN; ++n)
          acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, g.w[n]),
                                                             __builtin_bit_cast(h8, g.x[f][p]), acc[f][n], 0, 0, 0);
  };

  // ---- prologue: chunks 0 and 1 in flight, the rows' RMSNorm scales ----
  const int nc = a.K / 32;
  Pre P0 = load(0);
  Pre P1 = load(min(1, nc - 1));
  if constexpr (NORM) {
    // TPR threads per row, each summing its share of the row's per-chunk
    // sums of squares in order, then folded by a butterfly
    constexpr int TPR = kLT / TM;
    const int r = tid / TPR, per = nc / TPR;
    const int row = m0 + r < a.M ? m0 + r : 0;
    const float* sp = a.ssp + static_cast<size_t>(row) * nc + (tid % TPR) * per;
    float t = 0.0f;
    for (int i = 0; i < per; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(sp + i);
      t += v.x;
      t += v.y;
      t += v.z;
      t += v.w;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) t += __shfl_xor(t, o);
    if (tid % TPR == 0) rinv_s[r] = 1.0f / sqrtf(t / static_cast<float>(a.K) + a.eps);
  }
  store(0, P0);
  if (nc > 2) P0 = load(2);
  __syncthreads();
  // chunk c: the wave's fragments out of stage c % 2; chunk c + 1 (register
  // buffer (c + 1) % 2) into the other stage, read by no wave since the last
  // barrier, and that buffer reloaded with chunk c + 3; then the MFMAs and
  // one barrier
  auto step = [&](int c, int sidx, Pre& nxt) __attribute__((always_inline)) {
    const Frags g = frags(sidx);
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < nc) {
      store(sidx ^ 1, nxt);
      if (c + 3 < nc) nxt = load(c + 3);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(g);
    __syncthreads();
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, 0, P1);
    if (c + 1 < nc) step(c + 1, 1, P0);
  }

  // ---- epilogue from registers: pairs (f, na) and (f, nb) as in
  // bgemm_kernel ----
  const int c4 = 4 * lg;
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int j = 0; j < FN / 2; ++j) {
      const int na = MODE == kSwiGLU ? j : 2 * j, nb = MODE == kSwiGLU ? j + FN / 2 : 2 * j + 1;
      const int r = 16 * (wm * FM + f) + li;
      const int row = rows_s[r];
      const float rs = NORM ? rinv_s[r] : 1.0f;
      const float wa = a.wscale0, wbs = MODE == kSwiGLU ? a.wscale1 : a.wscale0;  // 2^-S, exact
      float va[4], vb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        va[i] = acc[f][na][i] * wa * rs;
        vb[i] = acc[f][nb][i] * wbs * rs;
      }
      if (row < 0) continue;
      if (MODE == kSwiGLU)
        finish_pair<MODE>(a, row, -1, lg, va, vb, bx * (TN / 2) + 16 * (wn * (FN / 2) + j) + c4, 0);
      else
        finish_pair<MODE>(a, row, MODE == kQKV ? pos_s[r] : -1, lg, va, vb, bx * TN + 16 * (wn * FN + na) + c4,
                          bx * TN + 16 * (wn * FN + nb) + c4);
    }
}

template <int FM, int FN, bool NORM, int NW>
hipError_t launch_t(int mode, const GemvArgs& a, dim3 grid, hipStream_t s) {
  const bool pl = a.planes != nullptr;
  const dim3 block(NW * kWave);
  switch (mode) {
    // projections read pre-split rows; the lm_heads (rows gathered per head)
    // split in the kernel
    case kAdd:
      if (!pl) return hipErrorInvalidValue;
      hipLaunchKernelGGL((bgemm_kernel<kAdd, FM, FN, NORM, true, NW>), grid, block, 0, s, a);
      break;
    case kSwiGLU:
      if (!pl) return hipErrorInvalidValue;
      hipLaunchKernelGGL((bgemm_kernel<kSwiGLU, FM, FN, NORM, true, NW>), grid, block, 0, s, a);
      break;
    case kQKV:
      if (!pl) return hipErrorInvalidValue;
      hipLaunchKernelGGL((bgemm_kernel<kQKV, FM, FN, NORM, true, NW>), grid, block, 0, s, a);
      break;
    case kHead:  // 32-row tiles (rows gathered per head)
      if constexpr (FM == 2) {
        if (pl) return hipErrorInvalidValue;
        hipLaunchKernelGGL((bgemm_kernel<kHead, FM, FN, NORM, false, NW>), grid, block, 0, s, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FM, int FN>
hipError_t launch_f(int mode, int nw, const GemvArgs& a, dim3 grid, hipStream_t s) {
  const bool norm = a.norm_g != nullptr;
  if (nw == 4) return norm ? launch_t<FM, FN, true, 4>(mode, a, grid, s) : launch_t<FM, FN, false, 4>(mode, a, grid, s);
  if constexpr (FM * FN <= 24) {  // the 64 x 128 tile at eight waves would spill
    if (nw == 8) return norm ? launch_t<FM, FN, true, 8>(mode, a, grid, s) : launch_t<FM, FN, false, 8>(mode, a, grid, s);
  }
  return hipErrorInvalidValue;
}

// Split pass: rows [0, M) of X (times g when set) into two fp16 planes in
// fragment order, rows up to the next multiple of 64 zero; with g, per row
// the sums of squares of x over each 32-wide K chunk.  Block (row tile, K
// block): 16 rows x 256 values; wave w takes fragment entries of chunks
// w and w + 4 of the block (lane = fragment lane), so the four entries of
// one row and chunk sit in lanes l, l +- 16, l +- 32 of one wave.
__global__ __launch_bounds__(kBlock) void split_rows_kernel(const float* X, int ldx, int M, int K, const float* g,
                                                            uint16_t* planes, float* ssp, int* ovf,
                                                            const int* pos) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int mt = blockIdx.x, kb = blockIdx.y;
  const int row = 16 * mt + lane % 16;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 8 * kb + wave + 4 * h;
    const int k = 32 * c + 8 * (lane / 16);
    float v[8], y[8];
    if (row < M) {
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(X + static_cast<size_t>(row) * ldx + k);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(X + static_cast<size_t>(row) * ldx + k + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = x0[i];
        v[i + 4] = x1[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float ss = 0.0f;
    if (g != nullptr) {
      const floatx4 g0 = *reinterpret_cast<const floatx4*>(g + k);
      const floatx4 g1 = *reinterpret_cast<const floatx4*>(g + k + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = v[i] * g0[i];
        y[i + 4] = v[i + 4] * g1[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = v[i];
    }
    if (split_store8(planes, gridDim.x, row, k, y)) flag_overflow(ovf, pos, row);
    if (g != nullptr) {
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      if (lane < 16 && row < M) ssp[static_cast<size_t>(row) * (K / 32) + c] = ss;
    }
  }
}

// Packs one bf16 matrix [N][K] (row-major, N % 16 == 0, K % 32 == 0), times
// `scale` (a power of two), as fp16 into fragment order at tiles t0.. of a
// chunk-major packed matrix with NT tiles per chunk: thread t writes one
// fragment entry (8 values).
__global__ __launch_bounds__(kBlock) void pack_frag_kernel(const uint16_t* W, int N, int K, uint16_t* P, int NT,
                                                           int t0, float scale) {
  const size_t t = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x;
  const size_t total = static_cast<size_t>(N / 16) * (K / 32) * kWave;
  if (t >= total) return;
  const int l = static_cast<int>(t % kWave);
  const size_t blk = t / kWave;
  const int c = static_cast<int>(blk % (K / 32));
  const int tile = static_cast<int>(blk / (K / 32));
  const uint16_t* src = W + static_cast<size_t>(tile * 16 + l % 16) * K + c * 32 + 8 * (l / 16);
  uint16_t* dst = P + frag_at(t0 + tile, c, NT) + l * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    dst[e] = static_cast<uint16_t>(f16_bits(static_cast<_Float16>(bf16_to_f32(src[e]) * scale)));
}

// *out = max |W| over n bf16 values, as float bits (non-negative floats
// order like their bit patterns).
__global__ __launch_bounds__(kBlock) void absmax_bf16_kernel(const uint16_t* W, size_t n, uint32_t* out) {
  __shared__ float red[kBlock / kWave];
  float m = 0.0f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * kBlock)
    m = fmaxf(m, fabsf(bf16_to_f32(W[i])));
  m = wave_max(m);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  // one atomic per block (a word that every wave hit serialised them)
  if (threadIdx.x == 0)
    atomicMax(out, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

}  // namespace

// bf16 weights only (packed by pack_fragments); fp32 weights keep the fp32
// kernels of mfma_impl.h.
hipError_t launch_bgemm(int wdtype, int mode, int fm, int fn, int nw, const GemvArgs& a, dim3 grid, hipStream_t s) {
  if (wdtype != CP_SPEC_BF16) return hipErrorInvalidValue;
  if (a.K % (64 * nw)) return hipErrorInvalidValue;  // an even number of chunks per wave
  if (fm == 2 && fn == 2) return launch_f<2, 2>(mode, nw, a, grid, s);
  if (fm == 2 && fn == 4) return launch_f<2, 4>(mode, nw, a, grid, s);
  if (fm == 2 && fn == 8) return launch_f<2, 8>(mode, nw, a, grid, s);
  if (fm == 4 && fn == 4) return launch_f<4, 4>(mode, nw, a, grid, s);
  if (fm == 4 && fn == 6) return launch_f<4, 6>(mode, nw, a, grid, s);
  if (fm == 4 && fn == 8) return launch_f<4, 8>(mode, nw, a, grid, s);
  return hipErrorInvalidValue;
}

// The staged tile for a shape, as 10 fm + fn, or 0: 128 x 192 (wave tiles
// of 4 x 6 fragments) where it gives every compute unit a block.  (Measured
// at wide-256: 128 x 128 tiles on half the compute units, and 64 x 128 tiles
// for the O and down projections, ran slower than bgemm_kernel.)
int bgemm_lds_tile(int mode, int N, int K, int M, int ptiles) {
  if (mode != kSwiGLU && mode != kQKV && mode != kAdd) return 0;
  if (M < kLdsMinRows || K % 512 || ptiles * 16 < M) return 0;
  const int cols = mode == kSwiGLU ? 2 * N : N;
  static const int kTiles[1][2] = {{4, 6}};
  for (const auto& t : kTiles) {
    const int bm = 2 * t[0], tn = 32 * t[1];
    if (ptiles % bm || cols % tn || (mode == kSwiGLU && N % (tn / 2))) continue;
    if (cols / tn * (ptiles / bm) >= kLdsMinBlocks) return 10 * t[0] + t[1];
  }
  return 0;
}

hipError_t launch_bgemm_lds(int mode, bool norm, const GemvArgs& a, hipStream_t s) {
  const int tile = a.planes == nullptr ? 0 : bgemm_lds_tile(mode, a.N, a.K, a.M, a.ptiles);
  if (tile == 0) return hipErrorInvalidValue;
  const int fm = tile / 10, fn = tile % 10;
  const int cols = mode == kSwiGLU ? 2 * a.N : a.N;
  const dim3 grid(cols / (32 * fn), a.ptiles / (2 * fm));
#define CPS_LDS_CASE(MODE_, FM_, FN_)                                                                   \
  if (mode == MODE_ && fm == FM_ && fn == FN_) {                                                       \
    if (norm) hipLaunchKernelGGL((bgemm_lds_kernel<MODE_, true, FM_, FN_>), grid, dim3(kLT), 0, s, a);   \
    else hipLaunchKernelGGL((bgemm_lds_kernel<MODE_, false, FM_, FN_>), grid, dim3(kLT), 0, s, a);       \
    return hipGetLastError();                                                                          \
  }
#define CPS_LDS_MODE(MODE_) CPS_LDS_CASE(MODE_, 4, 6)
  CPS_LDS_MODE(kSwiGLU)
  CPS_LDS_MODE(kQKV)
  CPS_LDS_MODE(kAdd)
#undef CPS_LDS_MODE
#undef CPS_LDS_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_split_rows(const float* X, int ldx, int M, int K, const float* g, uint16_t* planes, float* ssp,
                             int* ovf, const int* pos, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (K % 256 || ldx % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_rows_kernel, dim3((M + 63) / 64 * 4, K / 256), dim3(kBlock), 0, s, X, ldx, M, K, g,
                     planes, ssp, ovf, pos);
  return hipGetLastError();
}

hipError_t pack_fragments(const uint16_t* W, int N, int K, uint16_t* P, int NT, int t0, int S, hipStream_t s) {
  if (N % 16 || K % 32 || N <= 0 || K <= 0 || t0 < 0 || t0 + N / 16 > NT || S < -100 || S > 100)
    return hipErrorInvalidValue;
  const size_t total = static_cast<size_t>(N / 16) * (K / 32) * kWave;
  hipLaunchKernelGGL(pack_frag_kernel, dim3(static_cast<unsigned>((total + kBlock - 1) / kBlock)), dim3(kBlock),
                     0, s, W, N, K, P, NT, t0, ldexpf(1.0f, S));
  return hipGetLastError();
}

hipError_t launch_absmax_bf16(const uint16_t* W, size_t n, uint32_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + kBlock - 1) / kBlock, 1024);
  hipLaunchKernelGGL(absmax_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, W, n, out);
  return hipGetLastError();
}

}  // namespace cps
