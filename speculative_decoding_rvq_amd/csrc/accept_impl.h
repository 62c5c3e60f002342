// The acceptance step of a round, as device functions that every kernel
// taking an acceptance decision calls: the decode round's target kernel
// (chain and tree windows) and the component kernels behind cp_spec_accept
// and cp_spec_walk_step.
//
// Exact speculative sampling (TensorRT-Edge-LLM guide "CodePredictor
// Speculative Decoding", "How a round works", step 3; Lesson 8, section 02,
// exact stochastic decoding): a proposal x drawn from q is kept with
// probability min(1, p(x)/q(x)); after a rejection the position is drawn from
// norm(max(0, p - q)).  The tree window ("RVQ Position Aware ...", section 2.2
// and Figure 2) applies the same rule to the children of a node one after
// another, each rejection replacing p by the normalised residual.
#pragma once

#include "dev_common.h"
#include "topk_impl.h"

namespace cps {

// Row outcome bits next to the near-tie flags: the row's tested child was
// accepted (chain rows); tree rows keep the accepted child + 1 in bits 16..23.
constexpr uint32_t kRowAccepted = 1u << 8;

// One verify row's step of the walk, run by wave 0 of the row's block.
//   p    the row's target distribution as a list: L.lw[0..total) weights,
//        L.lidx their codes in ascending order, zero from `total` up to the
//        next multiple of 32 (p is zero off the list);
//   q    the draft distribution of the children's depth, dense in L.q (read
//        only when nk > 0);
//   x(k) the code of child k, k = 0..nk-1, tested in this order.
// Child k is accepted iff ua(k) < p'(x)/q(x) in float32, with p' = p for the
// first child; a code outside [0, V) has q = 1 and p' = 0 (rejected).  After
// a rejection p' becomes max(0, p' - q) entrywise (kept as it is when no
// entry would stay positive), divided by its sequential float32 sum in
// ascending code order when another child follows.  With no child accepted
// the row draws Sample(p', ut) (inverse CDF over the positive entries).
// Returns the accepted child's index, or -1 with *code = the draw.  *flags
// |= kFlagAccept when a test's |u - p'/q| < 1e-5, kFlagCdf for a draw's CDF
// near tie.  L.lw is overwritten.  All 64 lanes of wave 0 must call it.
template <typename XF, typename UAF>
__device__ int walk_step(const RowLds& L, int total, int V, int nk, XF x, UAF ua, float ut, int* code,
                         uint32_t* flags) {
  const int lane = threadIdx.x % kWave;
  for (int k = 0; k < nk; ++k) {
    const int xc = x(k);
    const float qd = (xc >= 0 && xc < V) ? L.q[xc] : 1.0f;
    float pd = 0.0f;
    for (int i = lane; i < total; i += kWave)
      if (L.lidx[i] == xc) pd = L.lw[i];
    pd = wave_max(pd);  // the only matching entry, p >= 0 elsewhere
    const float ratio = pd / qd;
    const float u = ua(k);
    if (fabs(static_cast<double>(u) - static_cast<double>(ratio)) < kEpsAccept) *flags |= kFlagAccept;
    if (u < ratio) {
      *code = xc;
      return k;
    }
    // the residual lives on p's list (p is zero elsewhere); with no positive
    // entry p' is kept
    bool pos = false;
    for (int i = lane; i < total; i += kWave) pos |= L.lw[i] - L.q[L.lidx[i]] > 0.0f;
    if (__ballot(pos)) {
      for (int i = lane; i < total; i += kWave) L.lw[i] = fmaxf(L.lw[i] - L.q[L.lidx[i]], 0.0f);
      wave_lds_sync();
    }
    if (k + 1 < nk) {  // another child is tested on p': normalise it
      float tot = 0.0f;
      if (lane == 0)
        for (int i = 0; i < total; ++i)
          if (L.lw[i] > 0.0f) tot = tot + L.lw[i];
      tot = __shfl(tot, 0);
      for (int i = lane; i < total; i += kWave) L.lw[i] = L.lw[i] / tot;
      wave_lds_sync();
    }
  }
  int near = 0;
  list_draw(L.lw, L.lidx, total, ut, code, &near);
  if (near) *flags |= kFlagCdf;
  return -1;
}

// The outcome of a chain round from its rows' steps.
//   dcode[t-1]         draft of offset t = 1..gamma;
//   tcode[r], tflags[r] row r's step: greedy, its argmax (and kFlagArgmax);
//                      sampled, the tested draft when kRowAccepted, else the
//                      row's draw (residual after a rejection, the bonus on
//                      row gamma), with its kFlagAccept / kFlagCdf bits.
// Greedy: drafts are kept while d_t equals row t-1's argmax (Lesson 8,
// section 02).  Sampled: while row t-1 accepted.  The round commits
// n = n_acc + 1 codes: codes[0..n_acc) the kept drafts, codes[n_acc] row
// n_acc's code.  Near ties of decisions the outcome used: accept, bit t-1 for
// each tested offset t <= min(n_acc + 1, gamma); cdf, bit n_acc for the
// committed draw.
struct ChainOutcome {
  int n_acc;
  uint32_t accept, cdf;
};

// One wave decides: lane l holds draft l + 1 (dc, l < gamma) and row l's
// step (tc, tf, l <= gamma); every lane of the wave calls it, and lane l
// gets the code it commits in *code (valid for l <= n_acc).
__device__ __forceinline__ ChainOutcome chain_outcome(int gamma, bool greedy, int dc, int tc, uint32_t tf,
                                                      int* code) {
  const int l = static_cast<int>(threadIdx.x % kWave);
  const bool kept = l < gamma && (greedy ? dc == tc : (tf & kRowAccepted) != 0u);
  ChainOutcome o{0, 0u, 0u};
  // the first lane not kept (lanes from gamma on never are): n_acc <= gamma
  o.n_acc = __builtin_ctzll(static_cast<unsigned long long>(__ballot(!kept)));
  if (!greedy) {
    const int tested = min(o.n_acc + 1, gamma);
    o.accept = static_cast<uint32_t>(__ballot(l < tested && (tf & kFlagAccept) != 0u));
    o.cdf = static_cast<uint32_t>(__ballot(l == o.n_acc && (tf & kFlagCdf) != 0u));
  }
  *code = l < o.n_acc ? dc : tc;
  return o;
}

}  // namespace cps
