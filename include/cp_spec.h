/*
 * cp_spec.h -- C ABI of the MI355X CodePredictor speculative-decoding library.
 *
 * One round of in-frame RVQ speculative decoding, as the TensorRT-Edge-LLM
 * user guide "CodePredictor Speculative Decoding" describes it (sections "Why
 * the draft is free" and "How a round works"):
 *   draft   apply head_{s+t} to the held hidden state h_s, t = 1..N-1, as one
 *           batched GEMV over the stacked later-depth lm_heads, and sample a
 *           proposal from each temperature/top-k distribution;
 *   verify  one causal decoder pass over the committed depth plus the drafts;
 *   accept  exact speculative sampling (min(1, p/q), residual norm(p - q)+,
 *           bonus from the trailing distribution), or argmax equality when
 *           decoding greedily (Lesson 8, "Two exact algorithms");
 *   commit  the accepted codes and truncate the per-frame KV (Lesson 8,
 *           section 07, "treat each round as a transaction").
 *
 * Conventions shared by every entry point:
 *   - All pointers named d_* are device pointers on the current HIP device;
 *     the caller owns all device memory (weights, inputs, outputs, workspace,
 *     statistics).  The library never allocates device memory.
 *   - `stream` is a hipStream_t passed as void*; every call is asynchronous on
 *     it unless stated otherwise.  Results are valid after the stream syncs.
 *   - Matrices are row-major [out][in].  Weights are float32 or bfloat16 bit
 *     patterns (uint16) as cfg.weight_dtype says; norm gains are float32.
 *   - Return value: CP_SPEC_OK, a positive warning, or a negative error.  On
 *     a negative return nothing was launched; cp_spec_last_error() gives a
 *     message (thread-local, valid until the next call on the same thread).
 */
#ifndef CP_SPEC_H
#define CP_SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define CP_SPEC_OK 0
/* Speculation disabled for this model, the autoregressive loop is used:
 * fewer than three RVQ depths (guide, "Limitations": automatic fallback). */
#define CP_SPEC_WARN_AR_FALLBACK 1
#define CP_SPEC_EINVAL (-1)       /* bad argument (e.g. verify_size 1 or > 8) */
#define CP_SPEC_EUNSUPPORTED (-2) /* shape outside the kernels' bounds        */
#define CP_SPEC_EHIP (-3)         /* a HIP runtime call failed                */
#define CP_SPEC_EWORKSPACE (-4)   /* workspace too small / misaligned         */

#define CP_SPEC_F32 0
#define CP_SPEC_BF16 1

/* Kernel bounds.  The vocabulary bound is the "small-vocabulary" bound of the
 * guide's "Kernels" section: a whole row of logits is held on chip. */
#define CP_SPEC_MAX_VOCAB 4096
#define CP_SPEC_MAX_GROUPS 32
#define CP_SPEC_MAX_WINDOW 8
#define CP_SPEC_MAX_TREE 63   /* tree window nodes (the root not counted) */
#define CP_SPEC_MAX_OFFSETS 8

/* Near-tie flag bits reported per decision by the component entry points. */
#define CP_SPEC_FLAG_TOPK 1u   /* k-th minus (k+1)-th largest logit < 1e-4    */
#define CP_SPEC_FLAG_ARGMAX 2u /* top-2 logit gap < 1e-4 (greedy)             */
#define CP_SPEC_FLAG_CDF 4u    /* sample point within 1e-5*sum of a boundary  */
#define CP_SPEC_FLAG_ACCEPT 8u /* |u - p(d)/q(d)| < 1e-5                      */

typedef struct cp_spec cp_spec; /* opaque handle */

typedef struct cp_spec_cfg {
  int32_t layers;       /* decoder layers L                                  */
  int32_t hidden;       /* H                                                 */
  int32_t q_heads;      /* query heads                                       */
  int32_t kv_heads;     /* key/value heads (grouped-query when < q_heads)    */
  int32_t head_dim;     /* d (even)                                          */
  int32_t ffn;          /* SwiGLU intermediate width                         */
  int32_t code_groups;  /* G: RVQ depths per frame (c_0 .. c_{G-1})          */
  int32_t vocab;        /* V: codebook size of every depth                   */
  int32_t weight_dtype; /* CP_SPEC_F32 or CP_SPEC_BF16                       */
  float rope_theta;     /* RoPE base                                         */
  float rms_eps;        /* RMSNorm epsilon                                   */
  int32_t verify_size;  /* N: 0 = off (autoregressive loop), else 2..8: the  */
                        /* committed depth plus N-1 drafted depths (guide,   */
                        /* "Options", --cpSpecVerifySize; 1 is rejected)     */
  int32_t greedy;       /* 1 = argmax decoding (exact greedy verification)   */
  float temperature;    /* > 0 unless greedy                                 */
  int32_t top_k;        /* 1..V unless greedy                                */
  int32_t max_streams;  /* largest n_streams any call will pass              */
  int32_t draft_offsets;/* K: position-aware draft offsets b_1..b_K, 0..8    */
                        /* ("RVQ Position Aware ...", section 2.2, Fig. 3):  */
                        /* draft offset t <= K scores with head_{s+t} the    */
                        /* state h_s + b_t, t > K the state h_s; only the    */
                        /* draft distributions q change. 0 = no offsets.     */
  /* 1: the next round's drafts are formed in this round's verify tail ("RVQ
   * Position Aware ...", section 2.2 and Figure 3: one call verifies and
   * drafts).  Every verify row that can end the round (and the prefill's
   * row 1) also scores the heads of the depths after it, with the offsets
   * when draft_offsets > 0, in the same lm_head launch as the target rows;
   * their drafts are drawn in the target softmax launch, and the accept
   * step keeps the set of the row that ends the round.  Below 32 verify rows
   * the accept step runs inside the next pass's first (Q/K/V) launch, whose
   * projection blocks read the next rows from the tables themselves.  The drafts and the
   * committed codes are those of fused_draft 0; the separate draft GEMV and
   * draft softmax launches are gone, the heads launch scores up to
   * max(N, 2) x N rows per stream instead of max(N, 2).  Chain windows only
   * (EUNSUPPORTED with a tree); ignored when verify_size < 2. */
  int32_t fused_draft;
  /* Tree-shaped verify window ("RVQ Position Aware ...", section 2.2 and
   * Figure 2).  tree_nodes = T in 1..63 replaces the chain window
   * (verify_size is then ignored; the verify block has T + 1 rows); 0 = the
   * chain.  tree_parent[i - 1] is the parent of node i (0 = the root, the
   * committed code; a parent precedes its children); depth at most 7.
   * Sampled: a node at depth d draws the code of depth s + d from that
   * depth's draft distribution (the j-th node of the depth with uniform
   * index j); the round walks down from the root testing a node's children
   * in order with min(1, p'/q) and replacing p' by norm(max(0, p' - q))
   * after each rejection, and draws from p' when no child is accepted.
   * Greedy: the k-th child of a node proposes the k-th highest draft logit
   * of its depth; the walk takes the first child equal to the node's target
   * argmax, else commits that argmax.  Nodes deeper than the frame allows
   * are left out of a round.  Sibling rows share their lm_head: the heads
   * launch reads each head once for all of them.
   * CP_SPEC_EUNSUPPORTED when the attention tile cannot fit LDS. */
  int32_t tree_nodes;
  int32_t tree_parent[CP_SPEC_MAX_TREE];
} cp_spec_cfg;

typedef struct cp_spec_weights {
  const void* embed;       /* [G][V][H]: table j embeds code c_j             */
  const void* heads;       /* [G-1][V][H]: lm_head j (scores c_j) at j-1      */
  const float* final_norm; /* [H]                                            */
  /* Host array of layers*9 device pointers, per layer in this order:
   * attn_norm[H] (f32), wq[nq*d][H], wk[nkv*d][H], wv[nkv*d][H], wo[H][nq*d],
   * ffn_norm[H] (f32), w_gate[F][H], w_up[F][H], w_down[H][F].
   * Read during cp_spec_create only; the device pointers are borrowed. */
  const void* const* layer;
  /* [K][H] f32 device, b_t at row t-1, 16-byte aligned; borrowed and read by
   * every decode call; required when cfg.draft_offsets > 0, else ignored. */
  const float* draft_offsets;
} cp_spec_weights;

/* Device-side statistics, accumulated (never cleared) by decode calls. */
typedef struct cp_spec_stats {
  int64_t frames;          /* frames completed                               */
  int64_t codes;           /* codes committed (G-1 per frame)                */
  int64_t prefill_passes;  /* frame bootstrap passes                         */
  int64_t rounds;          /* verify passes after the prefill                */
  int64_t proposed[CP_SPEC_MAX_OFFSETS]; /* drafts proposed at offset t=i+1  */
  int64_t accepted[CP_SPEC_MAX_OFFSETS]; /* drafts accepted at offset t=i+1  */
  int64_t bonus;           /* rounds whose drafts were all accepted          */
  int64_t near_tie_accept, near_tie_argmax, near_tie_cdf, near_tie_topk;
} cp_spec_stats;

/* Bytes of device workspace cp_spec_create needs for `cfg` (256-byte
 * aligned base required).  0 if cfg is invalid (see cp_spec_last_error). */
size_t cp_spec_workspace_bytes(const cp_spec_cfg* cfg);

/* Validate cfg, borrow the weights, carve the caller's workspace and upload
 * the RoPE table (synchronous: the device must be idle with respect to the
 * workspace).  Errors: EINVAL for verify_size 1 or > 8, non-positive shapes,
 * q_heads not a multiple of kv_heads, odd head_dim, temperature <= 0 or
 * top_k outside 1..V when sampling; EUNSUPPORTED for V > 4096, G > 32, or
 * matrix widths the kernels do not tile; EWORKSPACE when bytes is short.
 * Returns CP_SPEC_WARN_AR_FALLBACK (handle still created) when G < 3 with
 * verify_size > 0: every frame then runs the autoregressive loop. */
int cp_spec_create(const cp_spec_weights* w, const cp_spec_cfg* cfg,
                   void* d_workspace, size_t workspace_bytes, cp_spec** out);

void cp_spec_destroy(cp_spec* h);
const char* cp_spec_last_error(void);

/* Decode n_frames frames for each of n_streams independent streams.
 *   d_h_frame   [F][B][H] f32  talker hidden state of each frame (position 0)
 *   d_c0        [F][B]    i32  the frame's first code (from the talker)
 *   d_seeds     [F][B]    u64  Philox4x32-10 key of each frame
 *   d_out_codes [F][B][G] i32  out: c_0..c_{G-1} ([..][0] = c0)
 *   d_out_flags [F][B]    u32  out, nullable: bit j set when a decision at
 *                              depth j was a near tie (see CP_SPEC_FLAG_*)
 *   d_stats     cp_spec_stats  device, nullable: counters are added to it
 * A frame is a pure function of (weights, h_frame, c0, seed): frames of one
 * stream run in order, streams advance independently (ragged acceptance).
 * Host-synchronising: returns after the last frame has been decoded.
 * Errors: EINVAL for n_streams outside 1..max_streams or n_frames < 0;
 * EUNSUPPORTED, after the call has run, when an activation entering a
 * matrix-core projection (bf16 weights, 32 or more rows in a pass) reached
 * |x| >= 65504: those projections carry activations as two fp16 pieces, and
 * the call's codes are then not valid. */
int cp_spec_decode_frames(cp_spec* h, void* stream, int32_t n_streams,
                          int32_t n_frames, const float* d_h_frame,
                          const int32_t* d_c0, const uint64_t* d_seeds,
                          int32_t* d_out_codes, uint32_t* d_out_flags,
                          cp_spec_stats* d_stats);

/* Copy device statistics to the host (synchronises `stream`). */
int cp_spec_get_stats(const cp_spec_stats* d_stats, void* stream,
                      cp_spec_stats* host_out);

/* ---- component entry points: one step of the round each ----------------
 * Each runs the code cp_spec_decode_frames runs for that step, on caller
 * data, so each step can be checked on its own: head_logits and
 * decoder_forward launch the round's own projection, attention and head
 * kernels; topk_sample, accept and walk_step launch thin kernels around the
 * round's device functions (the top-k softmax and inverse-CDF draw, the
 * acceptance walk step and the chain outcome scan).  They use the handle's
 * workspace as scratch: calls on one handle must not overlap.  With bf16
 * weights and 32 or more rows, head_logits and decoder_forward run their
 * projections on the matrix cores with activations carried as two fp16
 * pieces: an activation of magnitude 65504 or more (or NaN) there is
 * carried as +-65504, so the outputs it feeds are finite but wrong, and
 * these two calls do not report it (decode_frames does, as EUNSUPPORTED). */

/* Stacked-head logits (draft GEMV, guide "Why the draft is free"; per-row
 * verify heads, guide "Limitations"):
 *   logits[r][:] = head_{d_head[r]} . (apply_final_norm ? RMSNorm_final(x[r])
 *                                                        : x[r])
 * d_x [n_rows][H] f32, d_head [n_rows] i32 in 1..G-1 (0 = skip the row),
 * d_logits [n_rows][V] f32.  n_rows <= max_streams * max(N, 2). */
int cp_spec_head_logits(cp_spec* h, void* stream, int32_t n_rows,
                        const float* d_x, const int32_t* d_head,
                        int32_t apply_final_norm, float* d_logits);

/* Temperature/top-k softmax and inverse-CDF sampling of each row (guide,
 * "Kernels"; Lesson 8, "Exact stochastic decoding"):
 *   probs[r] = TopKSoftmax(logits[r]; T, k)  (zero off the top-k support,
 *              ties at the k-th logit go to the lower code id)
 *   codes[r] = Sample(probs[r], u[r]): sequential float32 inverse CDF over
 *              the positive entries in ascending code order
 * Greedy handles: codes[r] = argmax (ties to the lower id), probs untouched.
 * d_u nullable (no sampling: codes[r] = -1 when not greedy); d_probs
 * nullable; d_flags [n_rows] u32 nullable (CP_SPEC_FLAG_* bits). */
int cp_spec_topk_sample(cp_spec* h, void* stream, int32_t n_rows,
                        const float* d_logits, const float* d_u,
                        float* d_probs, int32_t* d_codes, uint32_t* d_flags);

/* Accept scan of one round per stream (guide, "How a round works", step 3):
 *   for t = 1..gamma[b]: accept d_t iff u_accept[b][t-1] < p[t-1](d_t) /
 *   q[t-1](d_t) (float32); at the first rejection emit
 *   Sample(max(0, p[t-1] - q[t-1]), u_target[b][t-1]) (p[t-1] itself when
 *   that residual is all zero) and stop; if all are accepted emit
 *   Sample(p[gamma], u_target[b][gamma]).  Sample is the float32 inverse CDF
 *   over the positive entries in ascending code order.
 * Greedy handles: d_q and the uniforms are ignored, d_p holds target logits
 * rows and the argmax-equality rule applies.
 *   d_gamma [B] i32 in 0..width; d_draft [B][width] i32;
 *   d_q [B][width][V] f32; d_p [B][width+1][V] f32;
 *   d_u_accept [B][width] f32; d_u_target [B][width+1] f32;
 *   d_n out [B] i32 (codes committed, 1..gamma+1);
 *   d_codes out [B][width+1] i32 (the committed codes, in depth order);
 *   d_flags out [B] u32 nullable (bit t-1: near tie at offset t, either the
 *   accept test of a tested offset or the CDF of the committed draw).
 * Every row is decided in parallel by the step the decode round's target
 * kernel takes (one child per row), then the outcome scan its accept step
 * runs (one wave per stream); the rows' steps go through the workspace.
 * Errors: EINVAL for n_streams outside 0..max_streams, width outside 0..7,
 * null pointers. */
int cp_spec_accept(cp_spec* h, void* stream, int32_t n_streams, int32_t width,
                   const int32_t* d_gamma, const int32_t* d_draft,
                   const float* d_q, const float* d_p,
                   const float* d_u_accept, const float* d_u_target,
                   int32_t* d_n, int32_t* d_codes, uint32_t* d_flags);

/* cp_spec_accept without a handle and without allocating: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, rule and results
 * as cp_spec_accept, with the vocabulary size (256 * 2^i, up to 4096) and the
 * greedy switch given directly.  The rows' steps go through a static
 * scratch array of 65536 rows (512 KiB) that the library keeps on each GPU
 * it runs on until the process ends; nothing is allocated, and every row of
 * the scratch a call reads it has written first.  All calls on one GPU
 * share that array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 * Errors: EINVAL for a bad vocab, n_streams < 0, width outside 0..7,
 * n_streams * (width + 1) > 65536, null pointers; EHIP if the scratch
 * address cannot be looked up. */
int cp_spec_accept_noalloc(void* stream, int32_t vocab, int32_t greedy,
                           int32_t n_streams, int32_t width,
                           const int32_t* d_gamma, const int32_t* d_draft,
                           const float* d_q, const float* d_p,
                           const float* d_u_accept, const float* d_u_target,
                           int32_t* d_n, int32_t* d_codes, uint32_t* d_flags);

/* One node's step of the tree walk ("RVQ Position Aware ...", section 2.2,
 * Figure 2: the standard acceptance rule with residual resampling applied
 * along the tree), the step the decode round's target kernel takes for every
 * tree row.  For each row i, with p' = p[i] and q = q[i] (the draft
 * distribution of the children's depth):
 *   for k = 0..n_children[i]-1: x = children[i][k]; accept x iff
 *     u_accept[i][k] < p'(x) / q(x) (float32) and stop; else p' <-
 *     max(0, p' - q) (kept when nothing stays positive), divided by its
 *     sequential float32 sum in ascending code order when another child
 *     follows;
 *   none accepted: code = Sample(p', u_target[i]).
 *   d_p, d_q [n][V] f32; d_n_children [n] i32 (clamped to 0..max_children);
 *   d_children [n][max_children] i32; d_u_accept [n][max_children] f32;
 *   d_u_target [n] f32;
 *   d_accepted out [n] i32: index of the accepted child, or -1;
 *   d_codes out [n] i32: the accepted child's code, or the draw;
 *   d_flags out [n] u32 nullable (CP_SPEC_FLAG_ACCEPT for any test within
 *   1e-5 of its uniform, CP_SPEC_FLAG_CDF for the draw).
 * Errors: EINVAL for n_rows < 0, max_children outside 1..64, null pointers;
 * EUNSUPPORTED on a greedy handle. */
int cp_spec_walk_step(cp_spec* h, void* stream, int32_t n_rows,
                      int32_t max_children, const float* d_p, const float* d_q,
                      const int32_t* d_n_children, const int32_t* d_children,
                      const float* d_u_accept, const float* d_u_target,
                      int32_t* d_accepted, int32_t* d_codes, uint32_t* d_flags);

/* One causal decoder pass over rows_per_stream rows of each stream (the
 * verify pass, guide "How a round works", step 2):
 *   d_x [B][R][H] f32   in: input rows; out: final-RMSNormed hidden states
 *   d_pos [B][R] i32    position of each row (-1 = inactive row); a stream's
 *                       active rows must be consecutive positions, and every
 *                       position below its first row must already be in KV
 *   d_kv  [B][L][2][G][n_kv][d] f32  per-frame cache: K (before RoPE) at
 *                       [..][0], V at [..][1]; rows write their position and
 *                       attend to positions <= their own.
 * n_streams <= max_streams, rows_per_stream <= max(N, 2). */
int cp_spec_decoder_forward(cp_spec* h, void* stream, int32_t n_streams,
                            int32_t rows_per_stream, float* d_x,
                            const int32_t* d_pos, float* d_kv);

/* The codec part of the Talker's next input for finished frames (SGLang-Omni
 * note, the Talker / CodePredictor hand-off paragraph; "RVQ Position Aware
 * ...", section 2.1): for each row i,
 *   d_out[i][:] = sum over g = 0..G-1 of E_g[d_codes[i][g]]
 * added in group order in float32 (the text projection the Talker adds is
 * not part of the CodePredictor).  d_codes [n_rows][G] i32 device (the
 * layout of cp_spec_decode_frames' out_codes, n_rows = frames x streams);
 * d_out [n_rows][H] f32 device, 16-byte aligned, caller-owned.  A row with a
 * code outside [0, V) is written as NaN.  Asynchronous on `stream`.
 * Errors: EINVAL for n_rows < 0, null pointers or misaligned buffers;
 * EUNSUPPORTED for G > 64 or H not a multiple of 4. */
int cp_spec_talker_feedback(cp_spec* h, void* stream, int32_t n_rows,
                            const int32_t* d_codes, float* d_out);

/* ---- measurement --------------------------------------------------------
 * Kernel kinds of the round, for cp_spec_time_kernel. */
#define CP_SPEC_KERNEL_DRAFT_HEADS 0  /* stacked-head draft GEMV            */
#define CP_SPEC_KERNEL_QKV 1          /* RMSNorm + Q/K/V GEMV + KV append   */
#define CP_SPEC_KERNEL_ATTENTION 2    /* in-frame causal attention          */
#define CP_SPEC_KERNEL_O_PROJ 3       /* output projection + residual       */
#define CP_SPEC_KERNEL_GATE_UP 4      /* RMSNorm + gate/up GEMV + SwiGLU    */
#define CP_SPEC_KERNEL_DOWN 5         /* down projection + residual         */
#define CP_SPEC_KERNEL_TARGET_HEADS 6 /* final RMSNorm + per-row heads      */
#define CP_SPEC_KERNEL_KINDS 7

typedef struct cp_spec_kernel_timing {
  double avg_us;           /* mean device time per launch                   */
  double bytes_per_launch; /* algorithmic bytes: weights read once plus the */
                           /* activation rows read and written              */
  double flops_per_launch; /* 2 * rows * weight elements                    */
  int32_t launches;
  int32_t rows;            /* activation rows per launch                    */
  int32_t matrix_cores;    /* 1: the launch ran on MFMA tiles, 0: GEMV or   */
                           /* vector code                                   */
  int32_t reserved;
} cp_spec_kernel_timing;

/* Time one kernel of the round in its decode launch configuration for
 * n_streams streams: `iters` launches, captured into one HIP graph (as the
 * decode round is) and replayed between two HIP events recorded on
 * `stream`, cycling through the layers (or through distinct heads) so
 * consecutive launches read different weights.  Rows sit at mid-frame
 * positions with one distinct head each.  Overwrites the handle's
 * workspace (decode state included); synchronises `stream`. */
int cp_spec_time_kernel(cp_spec* h, void* stream, int32_t n_streams,
                        int32_t kind, int32_t iters,
                        cp_spec_kernel_timing* out);

#ifdef __cplusplus
}
#endif
#endif /* CP_SPEC_H */
