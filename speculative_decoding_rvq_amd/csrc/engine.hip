// Host side of the CodePredictor speculative-decoding library: validation,
// workspace carving, the round sequence (captured once into a hipGraph per
// stream count and replayed), the frame loop, and the C ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <utility>
#include <array>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

using namespace cps;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define CPS_HIP(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(CP_SPEC_EHIP, std::string(#call) + ": " + hipGetErrorString(e_));    \
  } while (0)

struct Shape {
  int L, H, nq, nkv, d, F, G, V, wdt, N, greedy, top_k, maxB;
  float theta, eps, T;
  int R, W, qdim, kvdim;
  int vec;  // weight elements per 16-byte chunk
  int K;    // position-aware draft offsets (0 = none)
  int fd;   // next round's drafts formed in the verify tail
  // tree window (T = 0: the chain): nodes, depth, parent and depth of node
  // i (node 0 = the root), K/V positions per stream (the frame's G plus one
  // slot per node)
  int tn, td, Gk;
  int par[kTreeSlots], dep[kTreeSlots];
  int tw;   // the most nodes at one depth (rows that share a head)
  int trb;  // tree attention: rows per block
};

struct Layout {
  size_t st, call, sstats, dhead, thead, pos, hstate, dX, X, Hout, ncode, Q, attn, act, kv, dlogits, q, dcode, dflags,
      tlogits, p, tcode, tflags, rope, packed, planes, ssp, fhead, cq, ccode, cflags, hb, st2, dcode2, dflags2, ovf,
      total;
};

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Threads covering one weight row's K in the GEMV: the largest of 256, 128,
// 64 that divides the row's 16-byte chunks with at most 4 chunks per thread.
int choose_kt(int K, int vec) {
  if (K % vec) return 0;
  const int segs = K / vec;
  for (int kt : {256, 128, 64})
    if (segs % kt == 0 && segs / kt <= 4) return kt;
  return 0;
}

int validate(const cp_spec_cfg* c, Shape* s, bool* warn_ar) {
  if (!c) return fail(CP_SPEC_EINVAL, "cfg is null");
  *warn_ar = false;
  if (c->layers < 1 || c->hidden < 1 || c->q_heads < 1 || c->kv_heads < 1 || c->head_dim < 2 ||
      c->ffn < 1 || c->vocab < 1 || c->max_streams < 1)
    return fail(CP_SPEC_EINVAL, "non-positive shape in cfg");
  if (c->code_groups < 2) return fail(CP_SPEC_EINVAL, "code_groups must be >= 2");
  if (c->q_heads % c->kv_heads) return fail(CP_SPEC_EINVAL, "q_heads must be a multiple of kv_heads");
  if (c->head_dim % 2) return fail(CP_SPEC_EINVAL, "head_dim must be even");
  if (c->weight_dtype != CP_SPEC_F32 && c->weight_dtype != CP_SPEC_BF16)
    return fail(CP_SPEC_EINVAL, "weight_dtype must be CP_SPEC_F32 or CP_SPEC_BF16");
  if (c->verify_size == 1)
    return fail(CP_SPEC_EINVAL, "verify_size 1 leaves no draft slot (valid: 0 = off, 2..8)");
  if (c->verify_size < 0 || c->verify_size > CP_SPEC_MAX_WINDOW)
    return fail(CP_SPEC_EINVAL, "verify_size must be 0 (off) or 2..8");
  if (!c->greedy) {
    if (!(c->temperature > 0.0f)) return fail(CP_SPEC_EINVAL, "temperature must be > 0");
    if (c->top_k < 1 || c->top_k > c->vocab) return fail(CP_SPEC_EINVAL, "top_k must be in 1..vocab");
  }
  if (c->draft_offsets < 0 || c->draft_offsets > CP_SPEC_MAX_OFFSETS)
    return fail(CP_SPEC_EINVAL, "draft_offsets must be in 0..8");
  if (c->tree_nodes < 0 || c->tree_nodes > CP_SPEC_MAX_TREE)
    return fail(CP_SPEC_EINVAL, "tree_nodes must be in 0..63");
  for (int i = 1; i <= c->tree_nodes; ++i)
    if (c->tree_parent[i - 1] < 0 || c->tree_parent[i - 1] >= i)
      return fail(CP_SPEC_EINVAL, "tree_parent[i-1] must be in 0..i-1");
  if (c->fused_draft != 0 && c->fused_draft != 1) return fail(CP_SPEC_EINVAL, "fused_draft must be 0 or 1");
  if (c->fused_draft && c->tree_nodes > 0)
    return fail(CP_SPEC_EUNSUPPORTED, "fused_draft runs chain windows only");
  if (c->tree_nodes > 0) {
    int dep[kTreeSlots] = {0};
    for (int i = 1; i <= c->tree_nodes; ++i) {
      dep[i] = dep[c->tree_parent[i - 1]] + 1;
      if (dep[i] > CP_SPEC_MAX_WINDOW - 1) return fail(CP_SPEC_EINVAL, "tree depth must be at most 7");
    }
    if (c->code_groups + c->tree_nodes > kMaxKeys)
      return fail(CP_SPEC_EUNSUPPORTED, "code_groups + tree_nodes must be at most 128");
  }
  if (c->vocab > CP_SPEC_MAX_VOCAB)
    return fail(CP_SPEC_EUNSUPPORTED, "vocab above the small-vocabulary bound (4096)");
  const int vpt = c->vocab / 256;
  if (c->vocab % 256 || (vpt & (vpt - 1)))
    return fail(CP_SPEC_EUNSUPPORTED, "vocab must be 256 * 2^i (256..4096)");
  if (c->code_groups > CP_SPEC_MAX_GROUPS) return fail(CP_SPEC_EUNSUPPORTED, "code_groups > 32");
  if (c->head_dim != 8 && c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64 &&
      c->head_dim != 128)
    return fail(CP_SPEC_EUNSUPPORTED, "head_dim must be 8, 16, 32, 64 or 128");
  Shape& s_ = *s;
  s_.L = c->layers; s_.H = c->hidden; s_.nq = c->q_heads; s_.nkv = c->kv_heads; s_.d = c->head_dim;
  s_.F = c->ffn; s_.G = c->code_groups; s_.V = c->vocab; s_.wdt = c->weight_dtype;
  s_.N = c->verify_size; s_.greedy = c->greedy ? 1 : 0;
  s_.top_k = c->greedy ? 1 : c->top_k; s_.maxB = c->max_streams;
  s_.theta = c->rope_theta; s_.eps = c->rms_eps; s_.T = c->greedy ? 1.0f : c->temperature;
  s_.qdim = s_.nq * s_.d; s_.kvdim = s_.nkv * s_.d;
  s_.vec = s_.wdt == CP_SPEC_BF16 ? 8 : 4;
  if (s_.N > 0 && s_.G < 3) {
    *warn_ar = true;  // no depth to draft: the autoregressive loop
    s_.N = 0;
  }
  if (c->tree_nodes > 0 && s_.G < 3) *warn_ar = true;  // nothing to draft: the autoregressive loop
  s_.tn = s_.td = 0;
  s_.par[0] = -1;
  s_.dep[0] = 0;
  if (c->tree_nodes > 0 && !*warn_ar) {
    s_.tn = c->tree_nodes;
    for (int i = 1; i <= s_.tn; ++i) {
      s_.par[i] = c->tree_parent[i - 1];
      s_.dep[i] = s_.dep[s_.par[i]] + 1;
      s_.td = std::max(s_.td, s_.dep[i]);
    }
    s_.N = s_.td + 1;  // codes a round commits at most
  }
  for (int i = s_.tn + 1; i < kTreeSlots; ++i) s_.par[i] = -1, s_.dep[i] = 0;
  s_.tw = 1;
  for (int d = 1; d <= s_.td; ++d) {
    int n = 0;
    for (int i = 1; i <= s_.tn; ++i) n += s_.dep[i] == d ? 1 : 0;
    s_.tw = std::max(s_.tw, n);
  }
  s_.Gk = s_.G + s_.tn;
  s_.R = s_.tn > 0 ? s_.tn + 1 : std::max(s_.N, 2);
  s_.W = s_.tn > 0 ? s_.td : std::max(s_.N - 1, 1);
  s_.K = s_.N >= 2 ? c->draft_offsets : 0;  // no drafts, no offsets
  s_.fd = (c->fused_draft && s_.N >= 2 && s_.tn == 0) ? 1 : 0;
  for (int K : {s_.H, s_.qdim, s_.F})
    if (!choose_kt(K, s_.vec))
      return fail(CP_SPEC_EUNSUPPORTED, "matrix width " + std::to_string(K) +
                                            " not tileable (multiple of 256 fp32 / 512 bf16 "
                                            "elements, at most 4 chunks per thread)");
  for (int N_ : {s_.qdim + 2 * s_.kvdim, s_.H, s_.V, s_.kvdim, s_.qdim})
    if (N_ % kRPGHost) return fail(CP_SPEC_EUNSUPPORTED, "output width must be a multiple of 4");
  if (s_.F % 2) return fail(CP_SPEC_EUNSUPPORTED, "ffn must be even");
  // tree attention: the most rows per block (a power of two) whose tile fits
  s_.trb = 0;
  if (s_.tn > 0)
    for (int rb = 64; rb >= 1 && !s_.trb; rb /= 2)
      if (tree_attention_smem_bytes(s_.Gk, s_.d, rb, s_.nq / s_.nkv) <= 160 * 1024) s_.trb = std::min(rb, s_.R);
  if (attention_smem_bytes(s_.G, s_.d, s_.R, s_.nq / s_.nkv) > 160 * 1024 || (s_.tn > 0 && s_.trb == 0))
    return fail(CP_SPEC_EUNSUPPORTED, "attention tile (positions x head_dim x query group) exceeds LDS");
  return CP_SPEC_OK;
}


// Streams from which the round's projections and heads run on the matrix
// cores (64-row tiles); below it the GEMV streams each weight once per few rows.
constexpr int kMfmaMinStreams = 8;
constexpr int kMfmaMinRows = 32;
constexpr int kFillBlocks = 256;  // one block per compute unit

// Waves per K-split block for a grid of `blocks` blocks with work: eight
// below one block per compute unit, four from there on.
int bgemm_waves(long blocks) { return blocks >= kFillBlocks ? 4 : 8; }

// bf16 weights in MFMA fragment order for the batched path: only when many
// rows can occur and every matrix tiles (N % 16, K % 128).
bool packs_weights(const Shape& s) {
  if (s.wdt != CP_SPEC_BF16) return false;
  if (s.maxB * s.R < kMfmaMinRows && s.maxB < kMfmaMinStreams) return false;
  return s.H % 128 == 0 && s.qdim % 128 == 0 && s.F % 128 == 0 && s.kvdim % 16 == 0 && s.V % 16 == 0;
}

// Per layer: QKV (stacked), O, gate, up, down; then the stacked lm_heads.
size_t packed_layer_elems(const Shape& s) {
  const size_t H = s.H, F = s.F;
  return (s.qdim + 2 * static_cast<size_t>(s.kvdim)) * H + H * s.qdim + 2 * F * H + H * F;
}
size_t packed_elems(const Shape& s) {
  if (!packs_weights(s)) return 0;
  return packed_layer_elems(s) * s.L + static_cast<size_t>(s.G - 1) * s.V * s.H;
}

Layout make_layout(const Shape& s) {
  Layout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t B = s.maxB, R = s.R, W = s.W, f4 = sizeof(float), i4 = sizeof(int);
  l.st = take(B * sizeof(StreamState));
  l.call = take(sizeof(CallDesc));
  l.sstats = take(B * sizeof(cp_spec_stats));
  l.dhead = take(std::max<size_t>(B * W, CP_SPEC_MAX_OFFSETS) * i4);  // (also create's scratch)
  l.thead = take(B * R * i4);
  l.pos = take(B * R * i4);
  l.hstate = take(B * s.H * f4);
  l.dX = take(s.K > 0 && !s.fd ? B * W * s.H * f4 : 0);  // draft inputs h_s + b_t
  l.X = take(B * R * s.H * f4);
  l.Hout = take(B * R * s.H * f4);
  l.Q = take(B * R * s.qdim * f4);
  l.attn = take(B * R * s.qdim * f4);
  l.act = take(B * R * s.F * f4);
  l.kv = take(B * static_cast<size_t>(s.L) * 2 * s.Gk * s.kvdim * f4);
  l.ncode = take(B * kTreeSlots * i4);  // tree window: the code of every node
  l.dlogits = take(B * W * s.V * f4);
  l.q = take(B * W * s.V * f4);
  l.dcode = take(B * W * i4);
  l.dflags = take(B * W * i4);
  // fused drafts: the target rows' logits and every row's candidate drafts'
  // logits side by side ([B][R][W + 1][V], column 0 the target)
  const size_t W1 = s.fd ? W + 1 : 1;
  l.tlogits = take(B * R * W1 * s.V * f4);
  l.fhead = take(s.fd ? B * R * W1 * i4 : 0);
  l.cq = take(s.fd ? B * R * W * s.V * f4 : 0);
  l.ccode = take(s.fd ? B * R * W * i4 : 0);
  l.cflags = take(s.fd ? B * R * W * i4 : 0);
  l.hb = take(s.fd && s.K > 0 ? static_cast<size_t>(s.G - 1) * s.K * s.V * f4 : 0);
  // the accept step folded into the next pass's first projection: staging
  // copies of the stream state and drafts
  l.st2 = take(s.fd ? B * sizeof(StreamState) : 0);
  l.dcode2 = take(s.fd ? B * W * i4 : 0);
  l.dflags2 = take(s.fd ? B * W * i4 : 0);
  l.p = take(B * R * s.V * f4);
  // (also the component accept's per-row scratch, [B][width + 1])
  const size_t Rt = std::max<size_t>(R, CP_SPEC_MAX_WINDOW);
  l.tcode = take(B * Rt * i4);
  l.tflags = take(B * Rt * i4);
  l.rope = take(static_cast<size_t>(s.G) * (s.d / 2) * sizeof(float2));
  l.packed = take(packed_elems(s) * sizeof(uint16_t));
  // pre-split activation planes (two fp16 per value) and partial sums of
  // squares of the batched projections' input rows
  const size_t prow = packs_weights(s) ? (B * R + 63) / 64 * 64 : 0;
  const size_t kmax = std::max({static_cast<size_t>(s.H), static_cast<size_t>(s.qdim), static_cast<size_t>(s.F)});
  l.planes = take(2 * prow * kmax * kPieces * sizeof(uint16_t));  // two alternating buffers
  l.ssp = take(prow * (kmax / 32) * f4);
  l.ovf = take(2 * sizeof(uint32_t));  // activation outside fp16's range; create's scratch word
  l.total = off;
  return l;
}

}  // namespace

struct cp_spec {
  Shape sh;
  Layout lo;
  char* ws;
  const void* embed;
  const void* heads;
  const float* fnorm;
  const float* doff = nullptr;  // [K][H] draft offsets (borrowed)
  std::vector<std::array<const void*, 9>> layers;
  // fragment-packed bf16 copies (batched path): per layer QKV, O, gate, up,
  // down; the lm_heads; all null when the weights are not packed
  std::vector<std::array<const uint16_t*, 5>> packed;
  const uint16_t* packed_heads = nullptr;
  // 2^-S of each packed matrix (the packed fp16 copy holds W * 2^S)
  std::vector<std::array<float, 5>> pscale;
  float hscale = 1.0f;
  hipStream_t cap_stream = nullptr;
  hipGraphExec_t graph = nullptr;
  int graph_B = -1;
  bool use_graph = true;
  bool use_fold = true;

  template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  long long kv_sb() const { return static_cast<long long>(sh.L) * 2 * sh.Gk * sh.kvdim; }

  RoundArgs round_args(int B) const {
    RoundArgs r{};
    r.B = B; r.R = sh.R; r.W = sh.W; r.G = sh.G; r.V = sh.V; r.H = sh.H; r.N = sh.N;
    r.greedy = sh.greedy; r.top_k = sh.top_k; r.L = sh.L; r.T = sh.T;
    r.tnodes = sh.tn; r.tdepth = sh.td; r.Gk = sh.Gk; r.kvdim = sh.kvdim;
    for (int i = 0; i < kTreeSlots; ++i) r.par[i] = sh.par[i], r.dep[i] = sh.dep[i];
    r.kv = at<float>(lo.kv);
    r.kv_sb = kv_sb();
    r.ncode = at<int>(lo.ncode);
    r.wbf16 = sh.wdt == CP_SPEC_BF16;
    r.embed = embed;
    r.st = at<StreamState>(lo.st);
    r.call = at<CallDesc>(lo.call);
    r.sstats = at<cp_spec_stats>(lo.sstats);
    r.dhead = at<int>(lo.dhead);
    r.thead = at<int>(lo.thead);
    r.pos = at<int>(lo.pos);
    r.hstate = at<float>(lo.hstate);
    r.K = sh.fd ? 0 : sh.K;  // fused drafts: the offsets enter through the heads' table
    r.doff = doff;
    r.dX = sh.K > 0 && !sh.fd ? at<float>(lo.dX) : nullptr;
    r.fused = sh.fd;
    r.ovf = at<int>(lo.ovf);
    r.fhead = sh.fd ? at<int>(lo.fhead) : nullptr;
    r.cq = sh.fd ? at<float>(lo.cq) : nullptr;
    r.ccode = sh.fd ? at<int>(lo.ccode) : nullptr;
    r.cflags = sh.fd ? at<uint32_t>(lo.cflags) : nullptr;
    r.X = at<float>(lo.X);
    r.Hout = at<float>(lo.Hout);
    r.dlogits = at<float>(lo.dlogits);
    r.q = at<float>(lo.q);
    r.dcode = at<int>(lo.dcode);
    r.dflags = at<uint32_t>(lo.dflags);
    r.tlogits = at<float>(lo.tlogits);
    r.p = at<float>(lo.p);
    r.tcode = at<int>(lo.tcode);
    r.tflags = at<uint32_t>(lo.tflags);
    r.st_out = r.st;
    r.dcode_out = r.dcode;
    r.dflags_out = r.dflags;
    if (fold_accept(B)) {
      r.fold = 1;
      r.st_out = at<StreamState>(lo.st2);
      r.dcode_out = at<int>(lo.dcode2);
      r.dflags_out = at<uint32_t>(lo.dflags2);
    }
    return r;
  }
  // Whether the round's accept step runs inside the next pass's first
  // projection (fused drafts, chain window, layer 0's Q/K/V on the GEMV).
  bool fold_accept(int B) const {
    return sh.fd && sh.tn == 0 && sh.R >= 2 && B * sh.R < kMfmaMinRows && use_fold;
  }
};

namespace {

// Activation rows per GEMV tile: enough for M when it is small, bounded so
// that the activation slices a thread keeps (rows x chunks x 16 bytes) stay
// within 96 registers.
int mt_for(int M, int spt, int vec) {
  int mt = M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8));
  while (mt > 1 && mt * spt * vec > 96) mt >>= 1;
  return mt;
}

bool mfma_fits(int mode, const GemvArgs& a) {
  if (a.K % kMfmaTK) return false;
  return mode == kSwiGLU ? a.N % (kMfmaTN / 2) == 0 : a.N % kMfmaTN == 0;
}

// Block tile (16 fm) x (16 fn) of the packed bf16 kernel for M rows: the
// largest that still gives every compute unit a block, else the one with the
// most blocks; false when no tile divides the columns or K is not a
// multiple of 512 (up to eight waves, each an even number of 32-wide
// chunks).  64 x 128 only for the residual adds, always at four waves: it
// cut the O and down projections' L2-to-CU bytes per compute unit by a third
// at 1024 rows (Q/K/V ran slower on it than on 64 x 96).
bool bgemm_tile(int mode, int N, int K, int M, int* fm_out, int* fn_out) {
  static const int kTiles[5][2] = {{4, 8}, {4, 6}, {4, 4}, {2, 4}, {2, 2}};
  if (K % 512) return false;
  int best = -1, best_blocks = 0;
  for (int i = 0; i < 5; ++i) {
    const int fm = kTiles[i][0], fn = kTiles[i][1];
    if (fn == 8 && mode != kAdd) continue;
    const bool fits = mode == kSwiGLU ? N % (8 * fn) == 0 : N % (16 * fn) == 0;
    if (!fits) continue;
    const int cols = mode == kSwiGLU ? 2 * N : N;
    const int blocks = cols / (16 * fn) * ((M + 16 * fm - 1) / (16 * fm));
    if (blocks >= kFillBlocks) {
      best = i;
      break;
    }
    if (fn == 8) continue;  // not below a full grid (its blocks take four waves)
    if (blocks > best_blocks) best = i, best_blocks = blocks;
  }
  if (best < 0) return false;
  *fm_out = kTiles[best][0];
  *fn_out = kTiles[best][1];
  return true;
}

// One skinny projection: Y (op) W . rows(X).  Many rows: matrix-core tiles
// (bf16: over the fragment-packed copies pk0 / pk1 of W0 / W1).
int gemv(const cp_spec* h, hipStream_t s, int mode, GemvArgs a, const uint16_t* pk0 = nullptr,
         const uint16_t* pk1 = nullptr, const RoundArgs* fold = nullptr) {
  if (a.M <= 0) return CP_SPEC_OK;
  if (fold != nullptr && a.M >= kMfmaMinRows) return fail(CP_SPEC_EINVAL, "folded accept step off the GEMV path");
  int fm, fn;
  if (a.planes != nullptr && !bgemm_tile(mode, a.N, a.K, a.M, &fm, &fn))
    return fail(CP_SPEC_EINVAL, "pre-split rows without a matrix-core tile");
  const bool head_mode = mode == kHead || mode == kHeadG;
  if (pk0 != nullptr && !head_mode && a.M >= kMfmaMinRows && bgemm_tile(mode, a.N, a.K, a.M, &fm, &fn)) {
    const int cols = mode == kSwiGLU ? a.N * 2 : a.N;
    a.W0 = pk0;
    a.W1 = pk1;
    if (a.planes == nullptr) {
      // the activation rows split once, then the tiles read the pieces (the
      // decoder layers' own path has them split by the producing kernel)
      uint16_t* planes = h->at<uint16_t>(h->lo.planes);
      float* ssp = h->at<float>(h->lo.ssp);
      CPS_HIP(launch_split_rows(a.X, a.ldx, a.M, a.K, a.norm_g, planes, ssp, a.ovf, a.pos, s));
      a.planes = planes;
      a.ptiles = (a.M + 63) / 64 * 4;
      a.ssp = ssp;
    }
    a.wtiles = a.N / 16;  // per packed matrix (SwiGLU: gate and up each)
    if (bgemm_lds_tile(mode, a.N, a.K, a.M, a.ptiles) != 0) {
      CPS_HIP(launch_bgemm_lds(mode, a.norm_g != nullptr, a, s));
      return CP_SPEC_OK;
    }
    const dim3 grid(cols / (16 * fn), (a.M + 16 * fm - 1) / (16 * fm));
    CPS_HIP(launch_bgemm(h->sh.wdt, mode, fm, fn, bgemm_waves(static_cast<long>(grid.x) * grid.y), a, grid, s));
    return CP_SPEC_OK;
  }
  if (!head_mode && a.M >= kMfmaMinRows && mfma_fits(mode, a)) {
    // the largest tile that still gives the chip enough blocks
    const int cols = mode == kSwiGLU ? a.N * 2 : a.N;  // tile columns (gate and up side by side)
    int tile = kTile64, t = 64;
    if (a.K % (4 * kMfmaTK) == 0) {
      if (cols / 64 * ((a.M + 63) / 64) < kFillBlocks) {
        tile = kTile32, t = 32;
        if (cols / 32 * ((a.M + 31) / 32) < kFillBlocks) tile = kTile16, t = 16;
      }
    }
    CPS_HIP(launch_mfma(h->sh.wdt, mode, tile, a, dim3(cols / t, (a.M + t - 1) / t), s));
    return CP_SPEC_OK;
  }
  const int vec = h->sh.vec;
  a.kt = choose_kt(a.K, vec);
  if (!a.kt) return fail(CP_SPEC_EUNSUPPORTED, "untileable K");
  const int spt = a.K / (vec * a.kt);
  const int rg = 256 / a.kt;
  const int rpg = gemv_rpg(spt);
  a.units = mode == kSwiGLU ? a.N / (rpg / 2) : a.N / rpg;
  const int gx = std::min((a.units + rg - 1) / rg, 4096);
  int mt, gy;
  if (mode == kHead) {
    mt = 1;
    gy = a.M;
  } else if (mode == kHeadG) {
    // a head's rows in slices of two per block: the slices of one weight
    // slice run on one XCD (block columns keep their XCD across the grid's
    // rows), so all but the first read it from that XCD's L2.  Measured at
    // one stream with fused drafts against up to 8 rows per block: 0.6 us
    // per pass faster at N = 4, 4 us at N = 8.  a.hslices comes in as the
    // most rows one head can have and leaves as the slices per head
    const int rph = std::max(a.hslices, 1);
    mt = 2;
    a.hslices = (rph + mt - 1) / mt;
    gy = a.n_heads * a.hslices;
  } else {
    mt = mt_for(a.M, spt, vec);
    // residual adds, the Q/K/V launch that runs the accept step, and Q/K/V
    // over at most four rows: two rows per block at most.  A thread loads two
    // fp32 activation vectors per 16-byte weight chunk and row, so four rows
    // make the activation loads twice the weight loads; with two rows per
    // block the second row tile reads the same weight slice from its XCD's
    // L2 (gemv_kernel's block order).  Measured at one stream: down 4.54 ->
    // 4.03 us, O 3.41 -> 3.35, 2.5-4.5 % more codes/s on every one-stream
    // workload; the SwiGLU projection (5.4 -> 5.7 us) keeps its wider tiles,
    // and so does the plain Q/K/V at eight rows (6.1 -> 7.0 us; 2 us per
    // pass slower at N = 8).
    if (mode == kAdd || fold != nullptr || (mode == kQKV && a.M <= 4)) mt = std::min(mt, 2);
    gy = (a.M + mt - 1) / mt;
  }
  if (fold != nullptr) {
    if (mode != kQKV) return fail(CP_SPEC_EINVAL, "folded accept step outside the Q/K/V GEMV");
    CPS_HIP(launch_gemv_fold(h->sh.wdt, mt, a, *fold, gx, gy, s));
    return CP_SPEC_OK;
  }
  CPS_HIP(launch_gemv(h->sh.wdt, mode, mt, a, gx, gy, s));
  return CP_SPEC_OK;
}

// Whether the decoder layers over M rows run on the matrix cores with the
// activation split folded into the producing kernels: the attention kernel
// writes the O projection's input pieces, the SwiGLU epilogue the down
// projection's, the residual-add epilogues the next normed projection's (x *
// gain, plus the rows' partial sums of squares).  Two plane buffers
// alternate: every kernel reads one and writes the other.
bool fused_planes(const cp_spec* h, int M) {
  if (h->packed.empty() || M < kMfmaMinRows) return false;
  const Shape& s = h->sh;
  int fm, fn;
  return s.d % 8 == 0 && bgemm_tile(kQKV, s.qdim + 2 * s.kvdim, s.H, M, &fm, &fn) &&
         bgemm_tile(kAdd, s.H, s.qdim, M, &fm, &fn) && bgemm_tile(kSwiGLU, s.F, s.H, M, &fm, &fn) &&
         bgemm_tile(kAdd, s.H, s.F, M, &fm, &fn);
}

// One decoder kernel of layer l over B*R rows of X at positions `pos`
// (fused: see fused_planes; layer 0's Q/K/V input is split by the caller).
// fold: layer 0 of a round whose previous accept step runs inside its Q/K/V
// launch.
int layer_kernel(const cp_spec* h, hipStream_t s, int kind, int l, int B, int R, float* X,
                 const int* pos, float* kv, bool fused = false, const RoundArgs* fold = nullptr) {
  const Shape& sh = h->sh;
  const int M = B * R;
  float* Q = h->at<float>(h->lo.Q);
  float* attn = h->at<float>(h->lo.attn);
  float* act = h->at<float>(h->lo.act);
  const auto& w = h->layers[l];
  const uint16_t* const* pk = h->packed.empty() ? nullptr : h->packed[l].data();
  auto pw = [&](int i) { return pk ? pk[i] : nullptr; };
  float* kvl = kv + l * 2LL * sh.Gk * sh.kvdim;
  const long long kv_vo = static_cast<long long>(sh.Gk) * sh.kvdim;
  GemvArgs a{};
  a.xdiv = 1;
  a.M = M;
  a.eps = sh.eps;
  a.ovf = h->at<int>(h->lo.ovf);
  a.pos = pos;  // the overflow flag ignores inactive rows
  a.wscale0 = a.wscale1 = 1.0f;
  const float* psc = h->pscale.empty() ? nullptr : h->pscale[l].data();
  auto sc = [&](int i) { return psc ? psc[i] : 1.0f; };
  uint16_t* P0 = h->at<uint16_t>(h->lo.planes);
  uint16_t* P1 = P0 + static_cast<size_t>((M + 63) / 64 * 64) *
                          std::max({sh.H, sh.qdim, sh.F}) * kPieces;  // within the second buffer
  float* S = h->at<float>(h->lo.ssp);
  const int T = (M + 63) / 64 * 4;
  switch (kind) {
    case CP_SPEC_KERNEL_QKV:
      a.W0 = w[1]; a.W1 = w[2]; a.W2 = w[3];
      a.N = sh.qdim + 2 * sh.kvdim; a.K = sh.H;
      a.X = X; a.ldx = sh.H; a.norm_g = static_cast<const float*>(w[0]);
      a.Y = Q; a.ldy = sh.qdim;
      a.qdim = sh.qdim; a.kvdim = sh.kvdim; a.kv = kvl; a.kv_sb = h->kv_sb();
      a.kv_vo = kv_vo; a.rows_per_stream = R; a.pos = pos; a.kv_positions = sh.Gk;
      if (fused) a.planes = P0, a.ptiles = T, a.ssp = S;
      a.wscale0 = sc(0);
      return gemv(h, s, kQKV, a, pw(0), nullptr, fold);
    case CP_SPEC_KERNEL_ATTENTION: {
      AttnArgs at{};
      at.Q = Q; at.out = attn; at.kv = kvl; at.kv_sb = h->kv_sb(); at.kv_vo = kv_vo; at.pos = pos;
      at.rope = h->at<float2>(h->lo.rope); at.R = R; at.nq = sh.nq; at.nkv = sh.nkv; at.d = sh.d;
      at.G = sh.G; at.scale = 1.0f / std::sqrt(static_cast<float>(sh.d));
      if (fused) at.planes = P1, at.ptiles = T;
      at.ovf = h->at<int>(h->lo.ovf);
      if (sh.tn > 0) {  // tree window: node slots and ancestor masks
        at.Gk = sh.Gk;
        at.RB = sh.trb;
        for (int i = 0; i < kTreeSlots; ++i) {
          at.dep[i] = sh.dep[i];
          at.anc[i] = (i >= 1 && i <= sh.tn) ? (1ull << i) | at.anc[sh.par[i]] : 0ull;
        }
        CPS_HIP(launch_tree_attention(at, B, s));
        return CP_SPEC_OK;
      }
      CPS_HIP(launch_attention(at, B, s));
      return CP_SPEC_OK;
    }
    case CP_SPEC_KERNEL_O_PROJ:
      a.W0 = w[4]; a.N = sh.H; a.K = sh.qdim; a.X = attn; a.ldx = sh.qdim; a.Y = X; a.ldy = sh.H;
      if (fused) {
        a.planes = P1, a.ptiles = T;
        a.out_planes = P0, a.out_ptiles = T, a.out_g = static_cast<const float*>(w[5]), a.out_ssp = S;
      }
      a.wscale0 = sc(1);
      return gemv(h, s, kAdd, a, pw(1));
    case CP_SPEC_KERNEL_GATE_UP:
      a.W0 = w[6]; a.W1 = w[7]; a.N = sh.F; a.K = sh.H; a.X = X; a.ldx = sh.H;
      a.norm_g = static_cast<const float*>(w[5]); a.Y = act; a.ldy = sh.F;
      if (fused) a.planes = P0, a.ptiles = T, a.ssp = S, a.out_planes = P1, a.out_ptiles = T;
      a.wscale0 = sc(2);
      a.wscale1 = sc(3);
      return gemv(h, s, kSwiGLU, a, pw(2), pw(3));
    case CP_SPEC_KERNEL_DOWN:
      a.W0 = w[8]; a.N = sh.H; a.K = sh.F; a.X = act; a.ldx = sh.F; a.Y = X; a.ldy = sh.H;
      if (fused) {
        a.planes = P1, a.ptiles = T;
        if (l + 1 < sh.L)  // the next layer's Q/K/V input
          a.out_planes = P0, a.out_ptiles = T, a.out_g = static_cast<const float*>(h->layers[l + 1][0]),
          a.out_ssp = S;
      }
      a.wscale0 = sc(4);
      return gemv(h, s, kAdd, a, pw(4));
    default:
      return fail(CP_SPEC_EINVAL, "not a decoder kernel kind");
  }
}

const int kLayerKinds[5] = {CP_SPEC_KERNEL_QKV, CP_SPEC_KERNEL_ATTENTION, CP_SPEC_KERNEL_O_PROJ,
                            CP_SPEC_KERNEL_GATE_UP, CP_SPEC_KERNEL_DOWN};

// All decoder layers over B*R rows of X at positions `pos`, cache `kv`.
int run_layers(const cp_spec* h, hipStream_t s, int B, int R, float* X, const int* pos, float* kv,
               const RoundArgs* fold = nullptr) {
  const bool fused = fused_planes(h, B * R);
  if (fold != nullptr && fused) return fail(CP_SPEC_EINVAL, "folded accept step with pre-split rows");
  if (fused)  // layer 0's Q/K/V input: the rows as the round left them
    CPS_HIP(launch_split_rows(X, h->sh.H, B * R, h->sh.H, static_cast<const float*>(h->layers[0][0]),
                              h->at<uint16_t>(h->lo.planes), h->at<float>(h->lo.ssp), h->at<int>(h->lo.ovf), pos, s));
  for (int l = 0; l < h->sh.L; ++l)
    for (int kind : kLayerKinds) {
      const int rc = layer_kernel(h, s, kind, l, B, R, X, pos, kv, fused, l == 0 ? fold : nullptr);
      if (rc) return rc;
    }
  return CP_SPEC_OK;
}

// lm_head logits of M rows (row m reads X row m / xdiv, head head[m], 0 =
// skip).  per_head > 0: on the matrix cores, rows grouped by head (each block
// finds its head's rows itself), at most per_head rows per head.  Else the
// GEMV: rows_per_head > 0 groups the rows of a head in one block (at most
// that many per head), 0 runs one block per row.  hb: per head and draft
// offset, the head applied to the offset, added to rows m with m % xdiv in
// 1..K (see GemvArgs).
int head_logits(const cp_spec* h, hipStream_t s, int M, const float* X, int xdiv, const int* head,
                const float* norm_g, float* xnorm_out, float* logits, int per_head = 0, int rows_per_head = 0,
                const float* hb = nullptr) {
  GemvArgs a{};
  a.W0 = h->heads; a.N = h->sh.V; a.K = h->sh.H; a.X = X; a.ldx = h->sh.H; a.xdiv = xdiv; a.M = M;
  a.norm_g = norm_g; a.eps = h->sh.eps; a.Y = logits; a.ldy = h->sh.V; a.head = head;
  a.head_stride = static_cast<long long>(h->sh.V) * h->sh.H; a.xnorm_out = xnorm_out;
  a.n_heads = h->sh.G - 1;
  a.hb = hb;
  a.hbK = hb != nullptr ? h->sh.K : 0;
  a.wscale0 = a.wscale1 = h->hscale;
  a.ovf = h->at<int>(h->lo.ovf);
  if (per_head > 0 && h->packed_heads != nullptr && a.N % 64 == 0 && a.K % 512 == 0) {
    // bf16, packed heads: 32 x 128 tiles per head where, at the average
    // rows per head, they still give every compute unit a block (each column
    // tile re-reads and splits its rows' fp32 activations: wide tiles halve
    // that), else 32 x 64
    a.W0 = h->packed_heads;
    a.wtiles = a.n_heads * (a.N / 16);
    const int slices = (per_head + 31) / 32;
    const int avg = (M + a.n_heads - 1) / a.n_heads;
    const int fn = a.N % 128 == 0 && a.N / 128 * ((avg + 31) / 32) * a.n_heads >= kFillBlocks ? 8 : 4;
    // four waves only for the wide tiles on a full grid (measured: the
    // 32 x 64 tiles keep eight, whose in-kernel split is latency-bound)
    const long busy = static_cast<long>(a.N / (16 * fn)) * ((avg + 31) / 32) * a.n_heads;  // blocks with rows
    const int nw = fn == 8 ? bgemm_waves(busy) : 8;
    CPS_HIP(launch_bgemm(h->sh.wdt, kHead, 2, fn, nw, a, dim3(a.N / (16 * fn), slices, a.n_heads), s));
    return CP_SPEC_OK;
  }
  if (per_head > 0 && mfma_fits(kHead, a)) {
    // tiles by the average rows per head
    const int avg = (M + a.n_heads - 1) / a.n_heads;
    const bool big = a.N / 64 * ((avg + 63) / 64) * a.n_heads >= kFillBlocks || a.K % (4 * kMfmaTK);
    const int t = big ? 64 : 32;
    const dim3 grid(a.N / t, (per_head + t - 1) / t, a.n_heads);
    CPS_HIP(launch_mfma(h->sh.wdt, kHead, big ? kTile64 : kTile32, a, grid, s));
    return CP_SPEC_OK;
  }
  if (rows_per_head > 0) {
    a.hslices = rows_per_head;
    return gemv(h, s, kHeadG, a);
  }
  return gemv(h, s, kHead, a);
}

// The whole round for B streams: draft GEMV -> draft sample -> verify pass ->
// per-row heads -> target softmax -> accept/commit/truncate.
int enqueue_round(const cp_spec* h, hipStream_t s, int B) {
  const Shape& sh = h->sh;
  const RoundArgs r = h->round_args(B);
  int rc;
  // many streams: lm_heads on the matrix cores, at most one row per stream
  // and head in the draft row set; in the verify row set a tree's nodes of
  // one depth share their head (tw of them)
  const int per_head = B >= kMfmaMinStreams ? B : 0;
  const int per_head_t = per_head * sh.tw;
  const int rows_head_t = sh.tn > 0 ? B * sh.tw : 0;  // few streams: grouped GEMV
  if (sh.fd) {
    // drafts were formed last round; this round's verify tail forms the
    // next ones: rows (stream, verify row r, k) with k = 0 the target head
    // and k = 1..W row r's candidate drafts (at most R rows of a stream per
    // head)
    // with the fold, layer 0's Q/K/V launch also commits the previous round
    if ((rc = run_layers(h, s, B, sh.R, r.X, r.pos, h->at<float>(h->lo.kv), r.fold ? &r : nullptr))) return rc;
    const int W1 = sh.W + 1;
    if ((rc = head_logits(h, s, B * sh.R * W1, r.X, W1, r.fhead, h->fnorm, r.Hout, r.tlogits,
                          per_head > 0 ? B * sh.R : 0, B * sh.R,
                          sh.K > 0 ? h->at<float>(h->lo.hb) : nullptr)))
      return rc;
    CPS_HIP(launch_target_topk(r, s));
    if (!r.fold) CPS_HIP(launch_round_accept(r, s));
    return CP_SPEC_OK;
  }
  if (sh.N >= 2) {
    // draft rows read h_s, or h_s + b_t when the drafter has offsets
    const float* dx = r.K > 0 ? r.dX : r.hstate;
    if ((rc = head_logits(h, s, B * sh.W, dx, r.K > 0 ? 1 : sh.W, r.dhead, nullptr, nullptr, r.dlogits,
                          per_head)))
      return rc;
    CPS_HIP(sh.tn > 0 ? launch_tree_draft(r, s) : launch_draft_topk(r, s));
  }
  if ((rc = run_layers(h, s, B, sh.R, r.X, r.pos, h->at<float>(h->lo.kv)))) return rc;
  if ((rc = head_logits(h, s, B * sh.R, r.X, 1, r.thead, h->fnorm, r.Hout, r.tlogits, per_head_t,
                        rows_head_t)))
    return rc;
  CPS_HIP(launch_target_topk(r, s));
  CPS_HIP(sh.tn > 0 ? launch_tree_accept(r, s) : launch_round_accept(r, s));
  return CP_SPEC_OK;
}

int ensure_graph(cp_spec* h, int B) {
  if (h->graph && h->graph_B == B) return CP_SPEC_OK;
  if (h->graph) {
    hipGraphExecDestroy(h->graph);
    h->graph = nullptr;
    h->graph_B = -1;
  }
  hipGraph_t g = nullptr;
  CPS_HIP(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
  const int rc = enqueue_round(h, h->cap_stream, B);
  const hipError_t e = hipStreamEndCapture(h->cap_stream, &g);
  if (rc) {
    if (g) hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return fail(CP_SPEC_EHIP, std::string("graph capture: ") + hipGetErrorString(e));
  const hipError_t ei = hipGraphInstantiate(&h->graph, g, nullptr, nullptr, 0);
  hipGraphDestroy(g);
  if (ei != hipSuccess) return fail(CP_SPEC_EHIP, std::string("graph instantiate: ") + hipGetErrorString(ei));
  h->graph_B = B;
  return CP_SPEC_OK;
}

// Rounds a stream still needs at the least: every round commits at most
// max(N, 1) codes and every frame starts with its prefill pass.
long long rounds_lower_bound(const Shape& sh, const StreamState& st, int F) {
  const int nw = std::max(sh.N, 1);
  const long long per_frame = 1 + (sh.G - 2 + nw - 1) / nw;
  if (st.mode == kModeDone) return 0;
  // (with the accept step folded into the next pass, a state is the round
  // just verified, not yet committed: still at least one pass)
  if (st.mode == kModePrefill || st.mode == kModeFresh) return static_cast<long long>(F - st.f) * per_frame;
  return (sh.G - 1 - st.s + nw - 1) / nw + static_cast<long long>(F - st.f - 1) * per_frame;
}

}  // namespace

extern "C" {

const char* cp_spec_last_error(void) { return g_err.c_str(); }

size_t cp_spec_workspace_bytes(const cp_spec_cfg* cfg) {
  Shape s{};
  bool warn = false;
  if (validate(cfg, &s, &warn) < 0) return 0;
  return make_layout(s).total;
}

int cp_spec_create(const cp_spec_weights* w, const cp_spec_cfg* cfg, void* d_workspace,
                   size_t workspace_bytes, cp_spec** out) {
  if (!out) return fail(CP_SPEC_EINVAL, "out is null");
  *out = nullptr;
  Shape s{};
  bool warn = false;
  const int rc = validate(cfg, &s, &warn);
  if (rc < 0) return rc;
  if (!w || !w->embed || !w->heads || !w->final_norm || !w->layer)
    return fail(CP_SPEC_EINVAL, "weights incomplete");
  const Layout lo = make_layout(s);
  if (!d_workspace || workspace_bytes < lo.total)
    return fail(CP_SPEC_EWORKSPACE, "workspace smaller than cp_spec_workspace_bytes()");
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256)
    return fail(CP_SPEC_EWORKSPACE, "workspace must be 256-byte aligned");
  for (int i = 0; i < 9 * s.L; ++i)
    if (!w->layer[i]) return fail(CP_SPEC_EINVAL, "null layer weight pointer");
  if (cfg->draft_offsets > 0 &&
      (!w->draft_offsets || reinterpret_cast<uintptr_t>(w->draft_offsets) % 16))
    return fail(CP_SPEC_EINVAL, "draft_offsets > 0 needs a 16-byte aligned offset array");

  cp_spec* h = new cp_spec();
  h->sh = s;
  h->lo = lo;
  h->ws = static_cast<char*>(d_workspace);
  h->embed = w->embed;
  h->heads = w->heads;
  h->fnorm = w->final_norm;
  h->doff = s.K > 0 ? w->draft_offsets : nullptr;
  h->layers.resize(s.L);
  for (int l = 0; l < s.L; ++l)
    for (int j = 0; j < 9; ++j) h->layers[l][j] = w->layer[9 * l + j];

  // RoPE table, angle = position * theta^(-2i/d), evaluated in double.
  std::vector<float2> rope(static_cast<size_t>(s.G) * (s.d / 2));
  for (int p = 0; p < s.G; ++p)
    for (int i = 0; i < s.d / 2; ++i) {
      const double ang = p * std::pow(static_cast<double>(s.theta), -2.0 * i / s.d);
      rope[static_cast<size_t>(p) * (s.d / 2) + i] =
          make_float2(static_cast<float>(std::cos(ang)), static_cast<float>(std::sin(ang)));
    }
  hipError_t e = hipMemset(d_workspace, 0, lo.total);
  if (e == hipSuccess)
    e = hipMemcpy(h->at<char>(lo.rope), rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = attention_allow_smem(s.d, attention_smem_bytes(s.G, s.d, s.R, s.nq / s.nkv));
  if (e == hipSuccess && s.tn > 0)
    e = tree_attention_allow_smem(s.d, tree_attention_smem_bytes(s.Gk, s.d, s.trb, s.nq / s.nkv));
  if (e == hipSuccess && packs_weights(s)) {
    // fragment-packed copies of every bf16 matrix (read once, here)
    uint16_t* p = h->at<uint16_t>(lo.packed);
    // a packed matrix of NT tiles per chunk from row-stacked sources
    // as fp16 times 2^S, S putting the matrix's largest |w| just below 2^15
    // (every bf16 value of magnitude 2^(-S-17) or more is then exact); the
    // kernels multiply their sums by 2^-S
    uint32_t* d_max = h->at<uint32_t>(lo.ovf);  // scratch word
    auto pack = [&](std::initializer_list<std::pair<const void*, int>> parts, int K, float* wscale) {
      int N = 0;
      for (const auto& pr : parts) N += pr.second;
      uint16_t* dst = p;
      uint32_t mbits = 0;
      if (e == hipSuccess) e = hipMemset(d_max, 0, sizeof(uint32_t));
      for (const auto& pr : parts)
        if (e == hipSuccess)
          e = launch_absmax_bf16(static_cast<const uint16_t*>(pr.first), static_cast<size_t>(pr.second) * K, d_max,
                                 nullptr);
      if (e == hipSuccess) e = hipMemcpy(&mbits, d_max, sizeof(uint32_t), hipMemcpyDeviceToHost);
      float mx = 0.0f;
      std::memcpy(&mx, &mbits, sizeof(float));
      int ex = 0;
      if (mx > 0.0f) std::frexp(mx, &ex);  // mx < 2^ex
      const int S = mx > 0.0f ? 15 - ex : 0;
      *wscale = std::ldexp(1.0f, -S);
      int t0 = 0;
      for (const auto& pr : parts) {
        if (e == hipSuccess)
          e = pack_fragments(static_cast<const uint16_t*>(pr.first), pr.second, K, dst, N / 16, t0, S, nullptr);
        t0 += pr.second / 16;
      }
      p += static_cast<size_t>(N) * K;
      return dst;
    };
    h->packed.resize(s.L);
    h->pscale.resize(s.L);
    for (int l = 0; l < s.L; ++l) {
      const auto& wl = h->layers[l];
      auto& pk = h->packed[l];
      auto& ps = h->pscale[l];
      pk[0] = pack({{wl[1], s.qdim}, {wl[2], s.kvdim}, {wl[3], s.kvdim}}, s.H, &ps[0]);  // Q, K, V tiles
      pk[1] = pack({{wl[4], s.H}}, s.qdim, &ps[1]);
      pk[2] = pack({{wl[6], s.F}}, s.H, &ps[2]);
      pk[3] = pack({{wl[7], s.F}}, s.H, &ps[3]);
      pk[4] = pack({{wl[8], s.H}}, s.F, &ps[4]);
    }
    h->packed_heads = pack({{h->heads, (s.G - 1) * s.V}}, s.H, &h->hscale);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemset(d_max, 0, sizeof(uint32_t));
  }
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking);
  if (e == hipSuccess && s.fd && s.K > 0) {
    // fused drafts with offsets: hb[j-1][t-1][:] = head_j . b_t, added to
    // the candidate rows' logits (head_j (h + b_t) = head_j h + head_j b_t)
    int* d_hd = h->at<int>(lo.dhead);  // K head indices, scratch
    std::vector<int> hd(s.K);
    for (int j = 1; j <= s.G - 1 && e == hipSuccess; ++j) {
      std::fill(hd.begin(), hd.end(), j);
      e = hipMemcpy(d_hd, hd.data(), s.K * sizeof(int), hipMemcpyHostToDevice);
      if (e != hipSuccess) break;
      float* dst = h->at<float>(lo.hb) + static_cast<size_t>(j - 1) * s.K * s.V;
      if (head_logits(h, h->cap_stream, s.K, h->doff, 1, d_hd, nullptr, nullptr, dst) != CP_SPEC_OK) {
        e = hipErrorLaunchFailure;
        break;
      }
      e = hipStreamSynchronize(h->cap_stream);
    }
    if (e == hipSuccess) e = hipMemset(d_hd, 0, s.maxB * s.W * sizeof(int));
  }
  if (e != hipSuccess) {
    delete h;
    return fail(CP_SPEC_EHIP, std::string("create: ") + hipGetErrorString(e));
  }
  *out = h;
  if (warn) {
    g_err = "fewer than two drafted depths available: autoregressive loop";
    return CP_SPEC_WARN_AR_FALLBACK;
  }
  return CP_SPEC_OK;
}

void cp_spec_destroy(cp_spec* h) {
  if (!h) return;
  if (h->graph) hipGraphExecDestroy(h->graph);
  if (h->cap_stream) hipStreamDestroy(h->cap_stream);
  delete h;
}

int cp_spec_decode_frames(cp_spec* h, void* stream, int32_t n_streams, int32_t n_frames,
                          const float* d_h_frame, const int32_t* d_c0, const uint64_t* d_seeds,
                          int32_t* d_out_codes, uint32_t* d_out_flags, cp_spec_stats* d_stats) {
  if (!h) return fail(CP_SPEC_EINVAL, "null handle");
  if (n_streams < 1 || n_streams > h->sh.maxB)
    return fail(CP_SPEC_EINVAL, "n_streams outside 1..max_streams");
  if (n_frames < 0) return fail(CP_SPEC_EINVAL, "n_frames < 0");
  if (n_frames == 0) return CP_SPEC_OK;
  if (!d_h_frame || !d_c0 || !d_seeds || !d_out_codes)
    return fail(CP_SPEC_EINVAL, "null input/output pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = n_streams;
  const RoundArgs r = h->round_args(B);
  CallDesc c{};
  c.h_frame = d_h_frame; c.c0 = d_c0; c.seeds = d_seeds; c.out_codes = d_out_codes;
  c.out_flags = d_out_flags; c.F = n_frames; c.B = B;
  if (h->use_graph) {
    const int rc = ensure_graph(h, B);
    if (rc) return rc;
  }
  CPS_HIP(launch_round_init(r, c, s));
  std::vector<StreamState> st(B);
  const int nw = std::max(h->sh.N, 1);
  long long chunk = static_cast<long long>(n_frames) * (1 + (h->sh.G - 2 + nw - 1) / nw);
  const long long cap = static_cast<long long>(n_frames) * h->sh.G + 16;
  long long launched = 0;
  for (;;) {
    for (long long i = 0; i < chunk; ++i) {
      if (h->use_graph) {
        CPS_HIP(hipGraphLaunch(h->graph, s));
      } else {
        const int rc = enqueue_round(h, s, B);
        if (rc) return rc;
      }
    }
    launched += chunk;
    CPS_HIP(hipMemcpyAsync(st.data(), r.st, B * sizeof(StreamState), hipMemcpyDeviceToHost, s));
    CPS_HIP(hipStreamSynchronize(s));
    long long need = 0;
    for (int b = 0; b < B; ++b) need = std::max(need, rounds_lower_bound(h->sh, st[b], n_frames));
    if (need == 0) break;
    if (launched > cap) return fail(CP_SPEC_EHIP, "round loop did not terminate");
    chunk = need;
  }
  if (d_stats) CPS_HIP(launch_stats_flush(r.sstats, B, d_stats, s));
  int ovf = 0;
  CPS_HIP(hipMemcpyAsync(&ovf, r.ovf, sizeof(int), hipMemcpyDeviceToHost, s));
  CPS_HIP(hipStreamSynchronize(s));
  if (ovf)
    return fail(CP_SPEC_EUNSUPPORTED,
                "an activation reached |x| >= 65504, outside the fp16 range of the matrix-core projections: "
                "this call's codes are not valid");
  return CP_SPEC_OK;
}

int cp_spec_get_stats(const cp_spec_stats* d_stats, void* stream, cp_spec_stats* host_out) {
  if (!d_stats || !host_out) return fail(CP_SPEC_EINVAL, "null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  CPS_HIP(hipMemcpyAsync(host_out, d_stats, sizeof(cp_spec_stats), hipMemcpyDeviceToHost, s));
  CPS_HIP(hipStreamSynchronize(s));
  return CP_SPEC_OK;
}

int cp_spec_head_logits(cp_spec* h, void* stream, int32_t n_rows, const float* d_x,
                        const int32_t* d_head, int32_t apply_final_norm, float* d_logits) {
  if (!h) return fail(CP_SPEC_EINVAL, "null handle");
  if (n_rows < 0 || n_rows > h->sh.maxB * h->sh.R) return fail(CP_SPEC_EINVAL, "n_rows out of range");
  if (n_rows == 0) return CP_SPEC_OK;
  if (!d_x || !d_head || !d_logits) return fail(CP_SPEC_EINVAL, "null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // many rows: grouped by head on the matrix cores (any number per head)
  return head_logits(h, s, n_rows, d_x, 1, d_head, apply_final_norm ? h->fnorm : nullptr, nullptr,
                     d_logits, n_rows >= kMfmaMinRows ? n_rows : 0, n_rows);
}

int cp_spec_topk_sample(cp_spec* h, void* stream, int32_t n_rows, const float* d_logits,
                        const float* d_u, float* d_probs, int32_t* d_codes, uint32_t* d_flags) {
  if (!h) return fail(CP_SPEC_EINVAL, "null handle");
  if (n_rows < 0) return fail(CP_SPEC_EINVAL, "n_rows < 0");
  if (n_rows == 0) return CP_SPEC_OK;
  if (!d_logits) return fail(CP_SPEC_EINVAL, "null logits");
  TopkArgs a{};
  a.logits = d_logits; a.probs = d_probs; a.codes = d_codes; a.flags = d_flags; a.u = d_u;
  a.V = h->sh.V; a.k = h->sh.top_k; a.greedy = h->sh.greedy; a.T = h->sh.T; a.n_rows = n_rows;
  CPS_HIP(launch_topk_rows(a, static_cast<hipStream_t>(stream)));
  return CP_SPEC_OK;
}

int cp_spec_talker_feedback(cp_spec* h, void* stream, int32_t n_rows, const int32_t* d_codes, float* d_out) {
  if (!h) return fail(CP_SPEC_EINVAL, "null handle");
  if (n_rows < 0) return fail(CP_SPEC_EINVAL, "n_rows < 0");
  if (n_rows == 0) return CP_SPEC_OK;
  if (!d_codes || !d_out) return fail(CP_SPEC_EINVAL, "null pointer");
  const Shape& sh = h->sh;
  if (sh.G > 64 || sh.H % 4) return fail(CP_SPEC_EUNSUPPORTED, "feedback needs G <= 64 and H % 4 == 0");
  if (reinterpret_cast<uintptr_t>(d_out) % 16 ||
      reinterpret_cast<uintptr_t>(h->embed) % (sh.wdt == CP_SPEC_BF16 ? 8 : 16))
    return fail(CP_SPEC_EINVAL, "misaligned embedding tables or output");
  CPS_HIP(launch_talker_feedback(h->embed, sh.wdt == CP_SPEC_BF16, sh.G, sh.V, sh.H, d_codes, n_rows, d_out,
                                 static_cast<hipStream_t>(stream)));
  return CP_SPEC_OK;
}

int cp_spec_accept(cp_spec* h, void* stream, int32_t n_streams, int32_t width, const int32_t* d_gamma,
                   const int32_t* d_draft, const float* d_q, const float* d_p,
                   const float* d_u_accept, const float* d_u_target, int32_t* d_n, int32_t* d_codes,
                   uint32_t* d_flags) {
  if (!h) return fail(CP_SPEC_EINVAL, "null handle");
  if (n_streams < 0 || n_streams > h->sh.maxB || width < 0 || width > CP_SPEC_MAX_WINDOW - 1)
    return fail(CP_SPEC_EINVAL, "n_streams/width out of range");
  if (n_streams == 0) return CP_SPEC_OK;
  if (!d_gamma || !d_draft || !d_p || !d_n || !d_codes || (!h->sh.greedy && (!d_q || !d_u_accept || !d_u_target)))
    return fail(CP_SPEC_EINVAL, "null pointer");
  AcceptArgs a{};
  a.B = n_streams; a.W = width; a.V = h->sh.V; a.greedy = h->sh.greedy; a.gamma = d_gamma;
  a.draft = d_draft; a.q = d_q; a.p = d_p; a.u_acc = d_u_accept; a.u_tgt = d_u_target; a.n_out = d_n;
  a.codes_out = d_codes; a.flags_out = d_flags;
  a.tcode = h->at<int>(h->lo.tcode);  // the round's own per-row outcome buffers
  a.tflags = h->at<uint32_t>(h->lo.tflags);
  CPS_HIP(launch_accept_rows(a, static_cast<hipStream_t>(stream)));
  return CP_SPEC_OK;
}

int cp_spec_accept_noalloc(void* stream, int32_t vocab, int32_t greedy, int32_t n_streams, int32_t width,
                           const int32_t* d_gamma, const int32_t* d_draft, const float* d_q, const float* d_p,
                           const float* d_u_accept, const float* d_u_target, int32_t* d_n, int32_t* d_codes,
                           uint32_t* d_flags) {
  const int vpt = vocab / 256;
  if (vocab < 256 || vocab > CP_SPEC_MAX_VOCAB || vocab % 256 || (vpt & (vpt - 1)))
    return fail(CP_SPEC_EINVAL, "vocab must be 256 * 2^i (256..4096)");
  if (n_streams < 0 || width < 0 || width > CP_SPEC_MAX_WINDOW - 1)
    return fail(CP_SPEC_EINVAL, "n_streams < 0 or width outside 0..7");
  if (static_cast<long long>(n_streams) * (width + 1) > kNoAllocRows)
    return fail(CP_SPEC_EINVAL, "n_streams * (width + 1) exceeds the static scratch (65536 rows)");
  if (n_streams == 0) return CP_SPEC_OK;
  if (!d_gamma || !d_draft || !d_p || !d_n || !d_codes || (!greedy && (!d_q || !d_u_accept || !d_u_target)))
    return fail(CP_SPEC_EINVAL, "null pointer");
  AcceptArgs a{};
  a.B = n_streams; a.W = width; a.V = vocab; a.greedy = greedy ? 1 : 0; a.gamma = d_gamma;
  a.draft = d_draft; a.q = d_q; a.p = d_p; a.u_acc = d_u_accept; a.u_tgt = d_u_target; a.n_out = d_n;
  a.codes_out = d_codes; a.flags_out = d_flags;
  CPS_HIP(noalloc_accept_scratch(&a.tcode, &a.tflags));
  CPS_HIP(launch_accept_rows(a, static_cast<hipStream_t>(stream)));
  return CP_SPEC_OK;
}

int cp_spec_walk_step(cp_spec* h, void* stream, int32_t n_rows, int32_t max_children, const float* d_p,
                      const float* d_q, const int32_t* d_n_children, const int32_t* d_children,
                      const float* d_u_accept, const float* d_u_target, int32_t* d_accepted, int32_t* d_codes,
                      uint32_t* d_flags) {
  if (!h) return fail(CP_SPEC_EINVAL, "null handle");
  if (h->sh.greedy) return fail(CP_SPEC_EUNSUPPORTED, "walk_step decodes stochastically only");
  if (n_rows < 0 || max_children < 1 || max_children > 64)
    return fail(CP_SPEC_EINVAL, "n_rows < 0 or max_children outside 1..64");
  if (n_rows == 0) return CP_SPEC_OK;
  if (!d_p || !d_q || !d_n_children || !d_children || !d_u_accept || !d_u_target || !d_accepted || !d_codes)
    return fail(CP_SPEC_EINVAL, "null pointer");
  WalkArgs a{};
  a.n = n_rows; a.V = h->sh.V; a.maxc = max_children; a.p = d_p; a.q = d_q; a.nchild = d_n_children;
  a.child = d_children; a.u_acc = d_u_accept; a.u_tgt = d_u_target; a.acc_out = d_accepted;
  a.code_out = d_codes; a.flags_out = d_flags;
  CPS_HIP(launch_walk_rows(a, static_cast<hipStream_t>(stream)));
  return CP_SPEC_OK;
}

int cp_spec_decoder_forward(cp_spec* h, void* stream, int32_t n_streams, int32_t rows_per_stream,
                            float* d_x, const int32_t* d_pos, float* d_kv) {
  if (!h) return fail(CP_SPEC_EINVAL, "null handle");
  if (n_streams < 0 || n_streams > h->sh.maxB || rows_per_stream < 1 || rows_per_stream > h->sh.R)
    return fail(CP_SPEC_EINVAL, "n_streams/rows_per_stream out of range");
  if (n_streams == 0) return CP_SPEC_OK;
  if (!d_x || !d_pos || !d_kv) return fail(CP_SPEC_EINVAL, "null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rc = run_layers(h, s, n_streams, rows_per_stream, d_x, d_pos, d_kv);
  if (rc) return rc;
  CPS_HIP(launch_rmsnorm_rows(d_x, d_x, h->fnorm, n_streams * rows_per_stream, h->sh.H, h->sh.eps, s));
  return CP_SPEC_OK;
}

int cp_spec_time_kernel(cp_spec* h, void* stream, int32_t n_streams, int32_t kind, int32_t iters,
                        cp_spec_kernel_timing* out) {
  if (!h || !out) return fail(CP_SPEC_EINVAL, "null pointer");
  if (n_streams < 1 || n_streams > h->sh.maxB) return fail(CP_SPEC_EINVAL, "n_streams out of range");
  if (kind < 0 || kind >= CP_SPEC_KERNEL_KINDS) return fail(CP_SPEC_EINVAL, "unknown kernel kind");
  if (iters < 1) return fail(CP_SPEC_EINVAL, "iters < 1");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Shape& sh = h->sh;
  const int B = n_streams, R = sh.R, W = sh.W, G = sh.G;
  const RoundArgs r = h->round_args(B);
  // rows at mid-frame positions s0+1.., one distinct head per row
  const int s0 = std::max(0, G - 1 - R);
  std::vector<int> pos(static_cast<size_t>(B) * R), thead(static_cast<size_t>(B) * R);
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < R; ++i) {
      pos[b * R + i] = s0 + 1 + i;
      thead[b * R + i] = std::min(s0 + 1 + i, G - 1);
    }
  // head tables for the draft GEMV: variant v uses heads 1 + (v*W + t) % (G-1)
  const bool grouped = B >= kMfmaMinStreams;
  const bool fused = fused_planes(h, B * R);
  const int per_head = grouped ? B : 0;
  const int nvar = G - 1;
  std::vector<int> dvar(static_cast<size_t>(nvar) * B * W);
  for (int v = 0; v < nvar; ++v)
    for (int b = 0; b < B; ++b)
      for (int t = 0; t < W; ++t) dvar[(static_cast<size_t>(v) * B + b) * W + t] = 1 + (v * W + t) % (G - 1);
  int* d_dvar = reinterpret_cast<int*>(r.q);  // scratch: the draft-distribution buffer
  CPS_HIP(hipMemcpyAsync(r.pos, pos.data(), pos.size() * sizeof(int), hipMemcpyHostToDevice, s));
  CPS_HIP(hipMemcpyAsync(r.thead, thead.data(), thead.size() * sizeof(int), hipMemcpyHostToDevice, s));
  CPS_HIP(hipMemcpyAsync(d_dvar, dvar.data(), dvar.size() * sizeof(int), hipMemcpyHostToDevice, s));
  CPS_HIP(hipStreamSynchronize(s));

  const double ws = sh.wdt == CP_SPEC_BF16 ? 2.0 : 4.0;
  const double M = static_cast<double>(B) * R, H = sh.H, F = sh.F, V = sh.V;
  const double qd = sh.qdim, kvd = sh.kvdim;
  double bytes = 0, flops = 0, rows = M;
  switch (kind) {
    case CP_SPEC_KERNEL_DRAFT_HEADS:
      rows = static_cast<double>(B) * W;
      bytes = std::min(W, G - 1) * V * H * ws + rows * (H + V) * 4;
      flops = 2 * rows * V * H;
      break;
    case CP_SPEC_KERNEL_QKV:
      bytes = (qd + 2 * kvd) * H * ws + M * (H + qd + 2 * kvd) * 4;
      flops = 2 * M * (qd + 2 * kvd) * H;
      break;
    case CP_SPEC_KERNEL_ATTENTION: {
      const double np = s0 + R;
      bytes = B * np * 2 * kvd * 4 + M * 2 * qd * 4;
      flops = 4 * M * np * qd;
      break;
    }
    case CP_SPEC_KERNEL_O_PROJ:
      bytes = H * qd * ws + M * (qd + 2 * H) * 4;
      flops = 2 * M * H * qd;
      break;
    case CP_SPEC_KERNEL_GATE_UP:
      bytes = 2 * F * H * ws + M * (H + F) * 4;
      flops = 4 * M * F * H;
      break;
    case CP_SPEC_KERNEL_DOWN:
      bytes = H * F * ws + M * (F + 2 * H) * 4;
      flops = 2 * M * H * F;
      break;
    case CP_SPEC_KERNEL_TARGET_HEADS:
      bytes = std::min(R, G - 1) * V * H * ws + M * (2 * H + V) * 4;
      flops = 2 * M * V * H;
      break;
  }
  auto launch = [&](hipStream_t ls, int i) -> int {
    if (kind == CP_SPEC_KERNEL_DRAFT_HEADS)
      return head_logits(h, ls, B * W, r.K > 0 ? r.dX : r.hstate, r.K > 0 ? 1 : W,
                         d_dvar + static_cast<size_t>(i % nvar) * B * W, nullptr, nullptr, r.dlogits, per_head);
    if (kind == CP_SPEC_KERNEL_TARGET_HEADS)
      return head_logits(h, ls, B * R, r.X, 1, r.thead, h->fnorm, r.Hout, r.tlogits, per_head);
    return layer_kernel(h, ls, kind, i % sh.L, B, R, r.X, r.pos, h->at<float>(h->lo.kv), fused);
  };
  // the layers as the round runs them; one pass first fills every buffer
  // a kind reads
  if (fused) {
    const int rc0 = run_layers(h, s, B, R, r.X, r.pos, h->at<float>(h->lo.kv));
    if (rc0) return rc0;
  }
  int rc = launch(s, 0);  // warm the launch path
  if (rc) return rc;
  CPS_HIP(hipStreamSynchronize(s));
  // the launches as one graph, like the decode round
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  CPS_HIP(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
  for (int i = 0; i < iters && !rc; ++i) rc = launch(h->cap_stream, i);
  const hipError_t ec = hipStreamEndCapture(h->cap_stream, &g);
  if (rc) {
    if (g) hipGraphDestroy(g);
    return rc;
  }
  if (ec != hipSuccess) return fail(CP_SPEC_EHIP, std::string("timing capture: ") + hipGetErrorString(ec));
  const hipError_t ei = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  hipGraphDestroy(g);
  if (ei != hipSuccess) return fail(CP_SPEC_EHIP, std::string("timing instantiate: ") + hipGetErrorString(ei));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t et = hipGraphLaunch(ge, s);  // warm
  if (et == hipSuccess) et = hipEventCreate(&e0);
  if (et == hipSuccess) et = hipEventCreate(&e1);
  if (et == hipSuccess) et = hipEventRecord(e0, s);
  if (et == hipSuccess) et = hipGraphLaunch(ge, s);
  if (et == hipSuccess) et = hipEventRecord(e1, s);
  if (et == hipSuccess) et = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (et == hipSuccess) et = hipEventElapsedTime(&ms, e0, e1);
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  hipGraphExecDestroy(ge);
  if (et != hipSuccess) return fail(CP_SPEC_EHIP, std::string("timing: ") + hipGetErrorString(et));
  out->avg_us = 1e3 * ms / iters;
  out->bytes_per_launch = bytes;
  out->flops_per_launch = flops;
  out->launches = iters;
  out->rows = static_cast<int32_t>(rows);
  out->reserved = 0;
  if (kind == CP_SPEC_KERNEL_DRAFT_HEADS || kind == CP_SPEC_KERNEL_TARGET_HEADS)
    out->matrix_cores = grouped && sh.V % kMfmaTN == 0 && sh.H % kMfmaTK == 0;
  else if (kind == CP_SPEC_KERNEL_ATTENTION)
    out->matrix_cores = 0;
  else {
    GemvArgs t{};
    int mode = kAdd;
    t.K = kind == CP_SPEC_KERNEL_O_PROJ ? sh.qdim : kind == CP_SPEC_KERNEL_DOWN ? sh.F : sh.H;
    t.N = kind == CP_SPEC_KERNEL_QKV ? sh.qdim + 2 * sh.kvdim : kind == CP_SPEC_KERNEL_GATE_UP ? sh.F : sh.H;
    if (kind == CP_SPEC_KERNEL_QKV) mode = kQKV;
    if (kind == CP_SPEC_KERNEL_GATE_UP) mode = kSwiGLU;
    out->matrix_cores = B * R >= kMfmaMinRows && mfma_fits(mode, t);
  }
  return CP_SPEC_OK;
}

}  // extern "C"
