// Kernel argument blocks and launchers of the CodePredictor round.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cp_spec.h"

namespace cps {

constexpr int kRPGHost = 4;   // output widths must be multiples of this

// Tree window: nodes (the root not counted), per-stream node slots (slot 0
// of a stream's node-code array holds the pending K/V move), and the most
// attention keys of a row (the frame's positions plus the nodes).
constexpr int kMaxTree = CP_SPEC_MAX_TREE;
constexpr int kTreeSlots = kMaxTree + 1;
constexpr int kMaxKeys = 128;

// GEMV weight rows per row group per unit: 4, or 2 when a thread holds three
// or more 16-byte chunks of each row.
__host__ __device__ constexpr int gemv_rpg(int spt) { return spt >= 3 ? 2 : 4; }

// Matrix-core tiles: 64 activation rows x 64 outputs, K steps of 32.
constexpr int kMfmaTM = 64, kMfmaTN = 64, kMfmaTK = 32;

enum GemvMode : int {
  kStore = 0,   // Y[m][o] = acc
  kAdd = 1,     // Y[m][o] += acc             (residual add)
  kSwiGLU = 2,  // Y[m][o] = silu(gate) * up  (W0 = gate, W1 = up)
  kQKV = 3,     // q -> Y, k/v -> KV cache at the row's position
  kHead = 4,    // per-row lm_head: W = heads[head[m] - 1]
  kHeadG = 5,   // lm_heads, rows grouped by head: each head's weights read
                // once for all its rows (few rows; the matrix-core paths
                // group by head themselves)
};

struct GemvArgs {
  const void* W0;
  const void* W1;
  const void* W2;
  int N;          // output rows (kQKV: qdim + 2*kvdim; kSwiGLU: ffn)
  int K;          // reduction length
  const float* X; // activation rows
  int ldx;
  int xdiv;       // activation row of output row m is m / xdiv
  int M;          // activation rows
  const float* norm_g;  // nullable: RMSNorm(x) * g applied to X rows first
  float eps;
  float* Y;
  int ldy;
  // kQKV
  int qdim, kvdim;
  float* kv;            // [B][L][2][G][nkv][d] base of this layer: + b*kv_sb
  long long kv_sb;      // floats per stream in the cache
  long long kv_vo;      // offset of V from K inside a layer
  int rows_per_stream;  // R
  int kv_positions;     // G: positions per stream in the cache
  const int* pos;       // [M] position of each row, -1 = inactive
  // kHead
  const int* head;      // [M] head index 1..n_heads, 0 = skip
  int n_heads;          // G-1
  long long head_stride;  // elements per head matrix (V*H)
  float* xnorm_out;     // nullable: normalised X rows written here, by the
                        // rows m with m % xdiv == 0, at X row m / xdiv
  // lm_heads: row m with k = m % xdiv in 1..hbK adds hb[(head - 1) * hbK +
  // k - 1][o] to its logits (the heads applied to the draft offsets b_k)
  const float* hb;
  int hbK;
  int hslices;          // kHeadG: row slices of MT per head (grid y = heads x slices)
  // tiling (host-chosen)
  int kt;     // threads covering one row's K (64/128/256)
  int units;  // number of RPG-row output units
  // matrix-core path: W0 / W1 fragment-packed with wtiles tiles per chunk;
  // activations pre-split by launch_split_rows (nullable) into ptiles row
  // tiles
  int wtiles;
  const uint16_t* planes;
  int ptiles;
  const float* ssp;  // [M][K / 32] partial sums of squares (with norm_g)
  // ... and the next projection's input, written by this one's epilogue
  // (SwiGLU: the activations; residual add: the new rows times out_g, with
  // their partial sums of squares in out_ssp [M][N / 32]); nullable
  uint16_t* out_planes;
  int out_ptiles;
  const float* out_g;
  float* out_ssp;
  // packed fp16 weights hold W * 2^S (one S per packed matrix): the tile's
  // sums are multiplied by wscale0 (W0) / wscale1 (W1, the SwiGLU up half)
  float wscale0, wscale1;
  int* ovf;  // set when an activation of a row in use (pos null or pos[row] >= 0) split for the matrix cores leaves fp16's range
};

struct AttnArgs {
  const float* Q;     // [B*R][qdim]
  float* out;         // [B*R][qdim]
  uint16_t* planes;   // nullable: out split for the O projection instead
  int ptiles;         // (planes) row tiles
  int* ovf;           // (planes) see GemvArgs
  const float* kv;    // layer base, + b*kv_sb
  long long kv_sb;
  long long kv_vo;
  const int* pos;     // [B*R]
  const float2* rope; // [G][d/2] (cos, sin)
  int R, nq, nkv, d, G;
  float scale;
  // tree window: K/V positions per stream (G + nodes), rows per block (the
  // grid's third axis covers the R rows), node depths, and per row the nodes
  // it attends to (bit i = node i, itself included)
  int Gk, RB;
  int dep[kTreeSlots];
  uint64_t anc[kTreeSlots];
};

struct TopkArgs {
  const float* logits;  // row r at logits + r*V
  float* probs;         // nullable
  int* codes;           // nullable
  uint32_t* flags;      // nullable
  const float* u;       // nullable (component call: uniforms per row)
  int V, k, greedy;
  float T;
  int n_rows;
};

struct AcceptArgs {  // component accept of a chain round
  int B, W, V, greedy;
  const int* gamma;
  const int* draft;
  const float* q;
  const float* p;
  const float* u_acc;
  const float* u_tgt;
  int* n_out;
  int* codes_out;
  uint32_t* flags_out;
  int* tcode;         // scratch [B][W + 1]: each row's step
  uint32_t* tflags;   // scratch [B][W + 1]
};

struct WalkArgs {  // component walk step: one node row each
  int n, V, maxc;
  const float* p;       // [n][V]
  const float* q;       // [n][V]
  const int* nchild;    // [n]
  const int* child;     // [n][maxc]
  const float* u_acc;   // [n][maxc]
  const float* u_tgt;   // [n]
  int* acc_out;
  int* code_out;
  uint32_t* flags_out;  // nullable
};

// Per-stream state of the round engine.
struct StreamState {
  int f;       // frame being decoded
  int s;       // committed depth (c_0..c_s committed, c_s not yet fed)
  int gamma;   // drafts in the coming round
  int mode;    // kModePrefill / kModeSpec / kModeDone / kModeFresh
  uint32_t flags;
  int last;                   // c_s, the last committed code
  uint32_t seed_lo, seed_hi;  // the frame's Philox key
};
// kModeFresh (accept folded into the first projection): the call's first
// pass, whose rows are frame f's prefill and which has no outcome to commit
enum { kModePrefill = 0, kModeSpec = 1, kModeDone = 2, kModeFresh = 3 };

// Arguments of one decode call, written on device by the init kernel so the
// captured round graph can be replayed for any call.
struct CallDesc {
  const float* h_frame;
  const int* c0;
  const uint64_t* seeds;
  int* out_codes;
  uint32_t* out_flags;
  int F, B;
};

struct RoundArgs {
  // shapes
  int B, R, W, G, V, H, N, greedy, top_k, L;
  float T;
  int wbf16;
  // weights
  const void* embed;
  // state and buffers
  StreamState* st;
  CallDesc* call;
  cp_spec_stats* sstats;  // [B] per-stream counters of the current call
  int* dhead;   // [B][W]
  int* thead;   // [B][R]
  int* pos;     // [B][R]
  float* hstate;   // [B][H]
  int K;              // position-aware draft offsets (0 = none)
  const float* doff;  // [K][H] b_t at row t-1
  float* dX;          // [B][W][H] draft inputs h_s + b_t (K > 0)
  // tree window (T > 0): nodes, depth, node parents and depths, the K/V
  // cache of the round's streams, every node's code
  int tnodes, tdepth, Gk, kvdim;
  int par[kTreeSlots], dep[kTreeSlots];
  float* kv;          // [B][L][2][Gk][kvdim]
  long long kv_sb;
  int* ncode;         // [B][kTreeSlots]
  float* X;        // [B][R][H]
  float* Hout;     // [B][R][H]
  float* dlogits;  // [B][W][V]
  float* q;        // [B][W][V]
  int* dcode;      // [B][W]
  uint32_t* dflags;  // [B][W]
  float* tlogits;  // [B][R][V]; fused drafts: [B][R][W + 1][V], column 0
  float* p;        // [B][R][V]
  int* ovf;        // activation outside fp16's range (cleared by the init kernel)
  // fused drafts: rows (b, r, k) of the heads launch (k = 0 target, k >= 1
  // row r's candidate draft of offset k), their heads, and every row's
  // candidate drafts (distributions, codes, flags) until the accept step
  // keeps the set of the row that ends the round
  int fused;
  int* fhead;      // [B][R][W + 1]
  float* cq;       // [B][R][W][V]
  int* ccode;      // [B][R][W]
  uint32_t* cflags;  // [B][R][W]
  int* tcode;      // [B][R]
  uint32_t* tflags;  // [B][R]
  // where the accept step writes the stream state and the next round's
  // drafts: st / dcode / dflags themselves, or, with the accept step folded
  // into the next pass's first projection (fold), staging copies: the
  // projection's other blocks still read the old ones; the target softmax
  // launch reads the staged ones and moves them into place
  int fold;
  StreamState* st_out;
  int* dcode_out;
  uint32_t* dflags_out;
};

// Launchers.  All asynchronous on `s`.
hipError_t launch_gemv(int wdtype, int mode, int mt, const GemvArgs& a, int grid_x, int grid_y,
                       hipStream_t s);
// Layer 0's Q/K/V GEMV with the previous round's accept step folded in
// (r.fold): r.B extra blocks run the accept step (into r.st_out /
// r.dcode_out / r.dflags_out), and the GEMV blocks take the same outcome from
// r.st, r.tcode / r.tflags, r.dcode and r.ccode and read their rows from the
// embedding tables or h_frame directly.  Grid gx x gy GEMV blocks as for
// launch_gemv, plus the accept blocks.
hipError_t launch_gemv_fold(int wdtype, int mt, const GemvArgs& a, const RoundArgs& r, int gx, int gy,
                            hipStream_t s);
// tile: kTile64 (64 x 64, LDS-staged), kTile32 / kTile16 (split-K over the
// block's four waves; K a multiple of 128).
enum MfmaTile { kTile64 = 0, kTile32 = 1, kTile16 = 2 };
hipError_t launch_mfma(int wdtype, int mode, int tile, const GemvArgs& a, dim3 grid, hipStream_t s);
// Matrix-core projections with in-block split-K over fragment-packed bf16
// weights (W0 / W1 packed by pack_fragments): block tile (16 fm) x (16 fn),
// (fm, fn) in {(2, 2), (2, 4), (2, 8), (4, 4), (4, 6), (4, 8)}, K a multiple
// of 512; nw waves per block (4 or 8, each taking K / nw; (4, 8) only 4); grid
// (columns / tile, rows / tile) or, lm_heads, (V / tile, row tiles, heads).
hipError_t launch_bgemm(int wdtype, int mode, int fm, int fn, int nw, const GemvArgs& a, dim3 grid, hipStream_t s);
// Large batches (kLdsMinRows rows or more): 128 x 192 block tiles staged in
// LDS, four waves of 64 x 96 over the whole K; bgemm_lds_tile gives the
// tile (10 fm + fn) or 0 when the shape does not yield kLdsMinBlocks blocks
// of it.  Pre-split rows only (a.planes); kSwiGLU, kQKV and kAdd.
constexpr int kLdsMinRows = 512;
constexpr int kLdsMinBlocks = 256;
int bgemm_lds_tile(int mode, int N, int K, int M, int ptiles);
hipError_t launch_bgemm_lds(int mode, bool norm, const GemvArgs& a, hipStream_t s);
// One bf16 matrix [N][K] row-major, times 2^S, as fp16 in MFMA fragment
// order (N % 16 == 0, K % 32 == 0), at tiles t0 .. t0 + N/16 - 1 of a
// chunk-major packed matrix with NT tiles per chunk: fragment (tile t, K
// chunk c) is 64 lanes x 8 fp16 at ((c * NT + t) * 64 + lane) * 8, lane l
// holding W[16 t + l % 16][32 c + 8 (l / 16) + 0..7] * 2^S.
hipError_t pack_fragments(const uint16_t* W, int N, int K, uint16_t* P, int NT, int t0, int S, hipStream_t s);
// *out = the largest |W| of n bf16 values, as float bits (*out must be 0
// before).
hipError_t launch_absmax_bf16(const uint16_t* W, size_t n, uint32_t* out, hipStream_t s);
// Activation pieces per value in the planes of the batched projections.
constexpr int kPieces = 2;
// Rows [0, M) of X (times g when set) split into two fp16 planes in
// fragment order for launch_bgemm (a.planes): with T = ceil(M / 64) * 4 row
// tiles, row tile t, K chunk c, plane p at ((c * T + t) * 2 + p) * 512 fp16;
// rows from M up to 64 T are zero.  With g,
// ssp[m][j] = sum of x^2 over K chunk j (32 wide).  K % 256 == 0.  A value
// outside fp16's range in row m sets *ovf (nullable) when pos (nullable) is
// null or pos[m] >= 0.
hipError_t launch_split_rows(const float* X, int ldx, int M, int K, const float* g, uint16_t* planes, float* ssp,
                             int* ovf, const int* pos, hipStream_t s);
// LDS the attention kernel needs, and raising its limit above 64 KB (once,
// before any launch).
size_t attention_smem_bytes(int G, int d, int R, int group);
hipError_t attention_allow_smem(int d, size_t bytes);
hipError_t launch_attention(const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_rmsnorm_rows(const float* x, float* y, const float* g, int rows, int H, float eps,
                               hipStream_t s);
hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t s);
// Every row's step of the walk, then each stream's outcome (two kernels).
hipError_t launch_accept_rows(const AcceptArgs& a, hipStream_t s);
// Rows of the allocation-free accept's static scratch, and the device
// address of the current GPU's copy (looked up once per device).
constexpr int kNoAllocRows = 65536;
constexpr int kMaxDevices = 64;
hipError_t noalloc_accept_scratch(int** tcode, uint32_t** tflags);
hipError_t launch_walk_rows(const WalkArgs& a, hipStream_t s);
hipError_t launch_round_init(const RoundArgs& r, const CallDesc& c, hipStream_t s);
hipError_t launch_draft_topk(const RoundArgs& r, hipStream_t s);
hipError_t launch_target_topk(const RoundArgs& r, hipStream_t s);
hipError_t launch_round_accept(const RoundArgs& r, hipStream_t s);
// Tree window: node draws, ancestor-masked attention, the walk and commit.
hipError_t launch_tree_draft(const RoundArgs& r, hipStream_t s);
// LDS of one tree-attention block (RB rows of a stream, one KV head).
size_t tree_attention_smem_bytes(int Gk, int d, int RB, int group);
hipError_t tree_attention_allow_smem(int d, size_t bytes);
hipError_t launch_tree_attention(const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_tree_accept(const RoundArgs& r, hipStream_t s);
// Adds the B per-stream counters to *out (one block; fixed order).
hipError_t launch_stats_flush(const cp_spec_stats* sstats, int B, cp_spec_stats* out, hipStream_t s);
// out[i][:] = sum over g < G of E_g[codes[i * G + g]] (float32, group
// order); G <= 64, H % 4 == 0, the embedding rows 8-byte (bf16) or 16-byte
// (fp32) aligned.
hipError_t launch_talker_feedback(const void* embed, int wbf16, int G, int V, int H, const int* codes, int n,
                                  float* out, hipStream_t s);

}  // namespace cps
