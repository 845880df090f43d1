// Fused speculative-verify decode on gfx950.
//
// Method ("Noyaux d'inférence", section "1. Le décodage KDA": the state after any accepted
// prefix of draft tokens is fixed by those tokens' projected inputs, so only the projected
// inputs are cached and the accepted states are rebuilt on chip; replayed tokens, the bonus
// token and the next draft window share one recurrent loop fused with the short
// convolution, input normalisation, gating, the recurrence and output normalisation.
// AMD blog "Dentro de los esfuerzos de optimización de Kimi K3", section 3: one launch that
// writes straight into the destination buffer; section 5: tiles own disjoint value columns
// and walk the same tokens in order.)
//
// Work decomposition: one workgroup of NW waves per (request, head): 4 for large batches
// (three workgroups per CU), 8 when the batch leaves most CUs idle, so that the head's
// per-token work spreads over two waves per SIMD. The head's fp32 state (d_k x d_v) is read
// from HBM once, lives in registers for every token (wave w owns value columns
// [D/NW w, D/NW (w + 1)); lane (row group rg = lane / 8, column group cg = lane % 8) holds
// rows D/8 rg .. + D/8 - 1 of its D/(8 NW) columns), and is written back twice: after the
// replayed drafts (state_acc) and after the bonus token (state, in place). A lane's rows and
// the order of every sum do not depend on NW, so all widths give the same bits.
//
// Tokens go in blocks of eight. The whole block's projected inputs are loaded one block
// ahead; the block's input stage (causal convolution, SiLU, decay and output gates, L2 norms
// of q and k) runs for all its tokens at once, parallel over channels and tokens; each wave
// then replays its columns through the block's tokens with no barrier (column sums over the
// key rows are reduced inside the wave); the block's outputs get their RMS normalisation
// together at the end. Per token, with the state columns independent:
//   k_s = sum_i (a_i k_i) S_ij,  q_s = sum_i (a_i q_i) S_ij     (both on the old state)
//   e_j = v_j - k_s;  S_ij <- a_i S_ij + (beta k_i) e_j;  o_j = q_s + beta (q . k) e_j
// which equals decaying first, correcting, then reading out S^T q. Every per-token quantity is
// computed by the same operations in the same order whatever the token's position in its
// block, so a replayed state is bit-identical to the state the same tokens reach one launch
// at a time.
#include "kda_common.h"
#include "kda_decode.h"

namespace kda {

// sigmoid with the hardware exponential and reciprocal (a few ulp; saturates correctly: an
// overflowing exponential gives 0, a vanishing one 1)
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// A wave-uniform value held in scalar registers and opaque to the optimiser, so that a
// per-lane choice between two launch parameters stays a register select instead of becoming
// a per-lane load from the parameter block (which costs a memory round trip before the
// address it feeds is known).
template <typename T>
__device__ __forceinline__ T in_sgpr(T x) {
  asm volatile("" : "+s"(x));
  return x;
}
// (pointers keep the global address space, so that their loads stay global loads)
#define KDA_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ const KDA_GLOBAL __bf16* in_sgpr_global(const __bf16* x) {
  auto g = (const KDA_GLOBAL __bf16*)x;
  asm volatile("" : "+s"(g));
  return g;
}

template <int D, int W, typename Tout, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 3 : 1) void decode_replay_kernel(DecodeParams p) {
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(W >= 1 && W <= 4, "convolution width");
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  static_assert(D % (8 * NW) == 0, "at least one value column per lane");
  constexpr int NT = 64 * NW;         // threads
  constexpr int NB = 8;               // tokens per block
  constexpr int RPL = D / 8;          // rows of S per lane
  constexpr int CPW = D / NW;         // value columns per wave
  constexpr int CPL = CPW / 8;        // value columns per lane
  constexpr int C3 = 3 * D;           // convolved channels q, k, v
  constexpr int CPG = D / 32;         // channels per thread in the 32-thread token groups
  // small batches (latency-bound) fetch the first block's new-window rows before the accepted
  // count arrives, and keep them when it is 0; large batches (HBM-bound) never spend the loads
  constexpr bool kSpeculate = NW > 4;

  const int rh = blockIdx.x;
  const int r = __builtin_amdgcn_readfirstlane(rh / p.H);   // (scalar: uniform loads)
  const int h = __builtin_amdgcn_readfirstlane(rh % p.H);
  const int H = p.H;
  int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int rg = lane >> 3;
  const int cg = lane & 7;
  const int col0 = CPW * w + CPL * cg;   // first value column of this lane
  const int row0 = RPL * rg;             // first key row of this lane

  // one block's per-token vectors: convolved q, k (then a q^, a k^ with the L2-normalised
  // q^, k^), v, decay a, beta k^, output gate, pre-norm output
  __shared__ __attribute__((aligned(16))) float s_q[NB][D], s_k[NB][D], s_v[NB][D], s_a[NB][D];
  __shared__ __attribute__((aligned(16))) float s_bk[NB][D], s_z[NB][D], s_o[NB][D];
  __shared__ float s_beta[NB];
  // one block's projected inputs as loaded (q, k, v, g, z rows of each token) and its betas
  constexpr int kRows = 5;
  __shared__ __attribute__((aligned(16))) __bf16 s_raw[NB][kRows][D];
  __shared__ float s_rbeta[NB];
  __shared__ float s_nrm[NB][3];        // 1/|q|, 1/|k|, (q . k) of the normalised vectors

  // Loads are issued in the order their data is needed: the request's accepted count, the
  // convolution tails and taps, the first block of inputs, then the state (first read by
  // the recurrence, after the block's input stage).
  int n_acc = p.n_acc[r];
  int n_new = p.n_new;
  if (p.n_new_r) n_new = __builtin_amdgcn_readfirstlane(p.n_new_r[r]);

  // ---- input-stage role (whole waves): threads [0, D) own q and k channel tid; [D, 2D) own
  // v, g and z channel tid - D. Each keeps the causal-convolution tail of its channels in
  // registers.
  const bool role_qk = w < D / 64;
  const bool role_v = w >= D / 64 && w < 2 * D / 64;
  const int ch = role_qk ? tid : tid - D;
  float tail_a[3] = {0.f, 0.f, 0.f}, tail_b[3] = {0.f, 0.f, 0.f};
  float wa[4] = {0.f, 0.f, 0.f, 0.f}, wb[4] = {0.f, 0.f, 0.f, 0.f};
  const size_t tbase = (size_t(r) * H + h) * C3 * (W - 1);
  const size_t wbase = size_t(h) * C3 * W;
  const int ca = role_qk ? ch : 2 * D + ch;   // q channel or v channel
  const int cb = ch + D;                      // k channel (q/k role only)
  if (role_qk || role_v) {
#pragma unroll
    for (int m = 0; m < W - 1; ++m) {
      tail_a[m] = p.conv_tail[tbase + size_t(ca) * (W - 1) + m];
      if (role_qk) tail_b[m] = p.conv_tail[tbase + size_t(cb) * (W - 1) + m];
    }
#pragma unroll
    for (int m = 0; m < W; ++m) {
      wa[m] = p.conv_w[wbase + size_t(ca) * W + m];
      if (role_qk) wb[m] = p.conv_w[wbase + size_t(cb) * W + m];
    }
  }



  // ---- projected inputs of one block: replay slots 1..n_acc of the previous window, then
  // slots 0..n_new-1 of the current one. They are fetched one block ahead in 16-byte pieces
  // (thread tid takes pieces tid, tid + NT, ...) into registers and written to s_raw once
  // the block before has been replayed. Piece c is part c % kPPR of row kind
  // f = c / (NB kPPR) of token (c / kPPR) % NB: the kind, and with it the base pointer, is
  // the same across a wave, and every lane loads (rows past the end read a present row), so
  // the loads of a block go out back to back with no wait between them.
  constexpr int kPPR = D * 2 / 16;                  // 16-byte pieces per row
  constexpr int kPPF = NB * kPPR;                   // pieces per row kind
  constexpr int kPieces = kRows * kPPF;             // per block
  constexpr int kPPT = (kPieces + NT - 1) / NT;     // per thread
  static_assert(kPPF % 64 == 0 && kPieces % 64 == 0, "whole waves per row kind");
  bf16x8 praw[kPPT];
  __bf16 pbeta = __bf16(0.f);   // raw bits, converted when staged
  int n_tok = 0;
  const int prev_slots = in_sgpr(p.prev_slots), cur_slots = in_sgpr(p.cur_slots);
  auto token_row = [&](int t) -> size_t {
    const bool replay = t < n_acc;
    const int slot = replay ? t + 1 : t - n_acc;
    const int slots = replay ? prev_slots : cur_slots;
    return (size_t(r) * slots + slot) * H + h;
  };
  using GB = const KDA_GLOBAL __bf16;
  using GB8 = const KDA_GLOBAL bf16x8;
  auto row_base = [&](int f, bool replay) -> GB* {
    switch (f) {
      case 0: return replay ? in_sgpr_global(p.prev_q) : in_sgpr_global(p.cur_q);
      case 1: return replay ? in_sgpr_global(p.prev_k) : in_sgpr_global(p.cur_k);
      case 2: return replay ? in_sgpr_global(p.prev_v) : in_sgpr_global(p.cur_v);
      case 3: return replay ? in_sgpr_global(p.prev_g) : in_sgpr_global(p.cur_g);
      default: return in_sgpr_global(p.cur_z);
    }
  };
  auto fetch_block = [&](int tb) {
#pragma unroll
    for (int m = 0; m < kPPT; ++m) {
      const int c = tid + NT * m;
      if (NT * (m + 1) > kPieces && c >= kPieces) break;   // whole waves
      const int f = __builtin_amdgcn_readfirstlane(c / kPPF);
      const int i = (c / kPPR) % NB, part = c % kPPR;
      const int t = tb + i;
      const bool replay = t < n_acc;
      // rows past the end, and z of replayed tokens (never used), read a present row
      const bool use = t < n_tok && !(f == 4 && replay);
      GB* base = use ? row_base(f, replay) : in_sgpr_global(p.cur_q);
      const size_t row = use ? token_row(t) : size_t(0);
      praw[m] = *reinterpret_cast<GB8*>(base + row * D + 8 * part);
    }
    if (w == 0) {   // lanes below NB carry the block's betas
      const int t = tb + (lane < NB ? lane : 0);
      const bool use = lane < NB && t < n_tok;
      GB* bb = use && t < n_acc ? in_sgpr_global(p.prev_beta) : in_sgpr_global(p.cur_beta);
      pbeta = bb[use ? token_row(t) : size_t(0)];
    }
  };
  auto stage_block = [&]() {
#pragma unroll
    for (int m = 0; m < kPPT; ++m) {
      const int c = tid + NT * m;
      if (NT * (m + 1) > kPieces && c >= kPieces) break;
      const int f = c / kPPF, i = (c / kPPR) % NB, part = c % kPPR;
      *reinterpret_cast<bf16x8*>(&s_raw[i][f][8 * part]) = praw[m];
    }
    if (tid < NB) s_rbeta[tid] = (float)pbeta;
  };
  // the first block of the new window alone (token t = slot t), in bounds whatever the
  // accepted count: slots below n_new exist for every request
  auto fetch_first_new = [&]() {
#pragma unroll
    for (int m = 0; m < kPPT; ++m) {
      const int c = tid + NT * m;
      if (NT * (m + 1) > kPieces && c >= kPieces) break;
      const int f = __builtin_amdgcn_readfirstlane(c / kPPF);
      const int i = (c / kPPR) % NB, part = c % kPPR;
      const size_t row = i < p.n_new ? (size_t(r) * cur_slots + i) * H + h : size_t(0);
      praw[m] = *reinterpret_cast<GB8*>(row_base(f, false) + row * D + 8 * part);
    }
    if (w == 0) {
      const int i = lane < NB && lane < p.n_new ? lane : 0;
      pbeta = p.cur_beta[(size_t(r) * cur_slots + i) * H + h];
    }
  };
  // ---- state tile into registers
  const size_t sbase = (size_t(r) * H + h) * D * D;
  float S[RPL][CPL];
  auto load_state = [&]() {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const float* src = p.state + sbase + size_t(row0 + i) * D + col0;
      if constexpr (CPL == 4) {
        // read once: a streaming (non-temporal) load
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
#pragma unroll
        for (int j = 0; j < 4; ++j) S[i][j] = x[j];
      } else if constexpr (CPL == 2) {
        const f32x2 x = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(src));
        S[i][0] = x[0];
        S[i][1] = x[1];
      } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) S[i][j] = src[j];
      }
    }
  };
  // (small batches: the state's loads go out before the accepted count is waited for)
  if constexpr (kSpeculate) {
    fetch_first_new();
    load_state();
  }
  n_acc = n_acc < 0 ? 0 : (n_acc > p.prev_slots - 1 ? p.prev_slots - 1 : n_acc);
  if (p.n_new_r) n_new = n_new < 1 ? 1 : (n_new > p.n_new ? p.n_new : n_new);
  n_tok = n_acc + n_new;
  if (!kSpeculate || n_acc > 0) fetch_block(0);
  if constexpr (!kSpeculate) load_state();




  stage_block();
  lds_barrier();

  for (int tb = 0; tb < n_tok; tb += NB) {
    const int nb = min(NB, n_tok - tb);
    // lane coordinates re-derived per block: the LDS and global addresses built from them are
    // recomputed here (a few integer ops) instead of being hoisted out of the loop and kept
    // live across it
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, rg = lane >> 3, cg = lane & 7;
    const int col0 = CPW * w + CPL * cg, row0 = RPL * rg;
    const int ch = role_qk ? tid : tid - D;

    // ---------------- input stage of the block: causal conv, SiLU, gates -----------------
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i >= nb) continue;
      const int t = tb + i;
      if (role_qk) {
        const float xa = (float)s_raw[i][0][ch], xb = (float)s_raw[i][1][ch];
        float ya = wa[W - 1] * xa, yb = wb[W - 1] * xb;
#pragma unroll
        for (int m = 0; m < W - 1; ++m) {
          ya += wa[m] * tail_a[m];
          yb += wb[m] * tail_b[m];
        }
#pragma unroll
        for (int m = 0; m + 1 < W - 1; ++m) {
          tail_a[m] = tail_a[m + 1];
          tail_b[m] = tail_b[m + 1];
        }
        if constexpr (W > 1) {
          tail_a[W - 2] = xa;
          tail_b[W - 2] = xb;
        }
        if (p.act) {
          ya = ya * sigmoidf_(ya);
          yb = yb * sigmoidf_(yb);
        }
        s_q[i][ch] = ya;
        s_k[i][ch] = yb;
      } else if (role_v) {
        const float xa = (float)s_raw[i][2][ch], xg = (float)s_raw[i][3][ch];
        const float xz = (float)s_raw[i][4][ch];
        float ya = wa[W - 1] * xa;
#pragma unroll
        for (int m = 0; m < W - 1; ++m) ya += wa[m] * tail_a[m];
#pragma unroll
        for (int m = 0; m + 1 < W - 1; ++m) tail_a[m] = tail_a[m + 1];
        if constexpr (W > 1) tail_a[W - 2] = xa;
        if (p.act) ya = ya * sigmoidf_(ya);
        s_v[i][ch] = ya;
        // exp(max(-softplus(x), g_min)) = max(sigmoid(-x), e^{g_min})
        s_a[i][ch] = fmaxf(sigmoidf_(-xg), p.decay_floor);
        s_z[i][ch] = t >= n_acc ? sigmoidf_(xz) : 0.f;
      }
      if (t == n_acc && (role_qk || role_v)) {
        // bonus token: the convolution tail it leaves is the new committed tail
#pragma unroll
        for (int m = 0; m < W - 1; ++m) {
          p.conv_tail[tbase + size_t(ca) * (W - 1) + m] = tail_a[m];
          if (role_qk) p.conv_tail[tbase + size_t(cb) * (W - 1) + m] = tail_b[m];
        }
      }
    }
    if (tid < nb) s_beta[tid] = sigmoidf_(s_rbeta[tid]);
    lds_barrier();

    // the next block's inputs load while this block is replayed
    const bool more = tb + NB < n_tok;
    if (more) fetch_block(tb + NB);

    // L2 norms of q and k and their dot product: 32 threads per token, fixed order
    {
      const int i = tid >> 5, l = tid & 31;
      float sq = 0.f, sk = 0.f, sqk = 0.f;
      if (i < nb) {
#pragma unroll
        for (int m = 0; m < CPG; ++m) {
          const float qv = s_q[i][l + 32 * m], kv = s_k[i][l + 32 * m];
          sq = fmaf(qv, qv, sq);
          sk = fmaf(kv, kv, sk);
          sqk = fmaf(qv, kv, sqk);
        }
      }
      // sums over the 32 lanes of the group (lanes 0-7, then 8 and 16 apart)
      sq = sum_xor16(sum_xor8(sum_mirror8(sum_xor2(sum_xor1(sq)))));
      sk = sum_xor16(sum_xor8(sum_mirror8(sum_xor2(sum_xor1(sk)))));
      sqk = sum_xor16(sum_xor8(sum_mirror8(sum_xor2(sum_xor1(sqk)))));
      if (l == 0 && i < nb) {
        const float iq = 1.f / sqrtf(sq + p.eps_l2);
        const float ik = 1.f / sqrtf(sk + p.eps_l2);
        s_nrm[i][0] = iq;
        s_nrm[i][1] = ik;
        s_nrm[i][2] = sqk * iq * ik;
      }
    }
    lds_barrier();
    // per-row factors of the recurrence, once per token and channel
#pragma unroll
    for (int m = 0; m < (NB * D + NT - 1) / NT; ++m) {
      const int idx = tid + NT * m;
      const int i = idx / D, c = idx % D;
      if (idx < NB * D && i < nb) {
        const float a = s_a[i][c];
        const float kn = s_k[i][c] * s_nrm[i][1];
        s_k[i][c] = a * kn;
        s_q[i][c] = a * (s_q[i][c] * s_nrm[i][0]);
        s_bk[i][c] = s_beta[i] * kn;
      }
    }
    lds_barrier();

    if (tb == 0 && n_acc == 0 && p.state_acc) {
      // no accepted drafts: the accepted state is the committed entering state
#pragma unroll
      for (int ii = 0; ii < RPL; ++ii) {
        float* dst = p.state_acc + sbase + size_t(row0 + ii) * D + col0;
        if constexpr (CPL == 4) {
          __builtin_nontemporal_store(f32x4{S[ii][0], S[ii][1], S[ii][2], S[ii][3]},
                                      reinterpret_cast<f32x4*>(dst));
        } else if constexpr (CPL == 2) {
          __builtin_nontemporal_store(f32x2{S[ii][0], S[ii][1]}, reinterpret_cast<f32x2*>(dst));
        } else {
#pragma unroll
          for (int j = 0; j < CPL; ++j) dst[j] = S[ii][j];
        }
      }
    }
    // ---------------- recurrence: this wave's columns through the block's tokens ----------
#pragma unroll 1
    for (int i = 0; i < nb; ++i) {
      const int t = tb + i;
      const bool output = t >= n_acc;
      const float qk = s_nrm[i][2];
      const float beta = s_beta[i];
      // the lane's rows of the token's read-out factors (a k^, a q^), every read issued
      // before the first is used so that their LDS latencies overlap
      f32x4 ak[RPL / 4], aq[RPL / 4];
#pragma unroll
      for (int m = 0; m < RPL / 4; ++m) {
        ak[m] = *reinterpret_cast<const f32x4*>(&s_k[i][row0 + 4 * m]);
        aq[m] = *reinterpret_cast<const f32x4*>(&s_q[i][row0 + 4 * m]);
      }
      float ks[CPL], qs[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        ks[j] = 0.f;
        qs[j] = 0.f;
      }
      // (replayed drafts produce no output: their read-out sums are skipped)
      if (output) {
#pragma unroll
        for (int m = 0; m < RPL / 4; ++m)
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              ks[j] = fmaf(ak[m][u], S[4 * m + u][j], ks[j]);
              qs[j] = fmaf(aq[m][u], S[4 * m + u][j], qs[j]);
            }
      } else {
#pragma unroll
        for (int m = 0; m < RPL / 4; ++m)
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < CPL; ++j) ks[j] = fmaf(ak[m][u], S[4 * m + u][j], ks[j]);
      }
      // the update's factors (a, beta k^), read while the column sums are reduced
      f32x4 fa[RPL / 4], fb[RPL / 4];
#pragma unroll
      for (int m = 0; m < RPL / 4; ++m) {
        fa[m] = *reinterpret_cast<const f32x4*>(&s_a[i][row0 + 4 * m]);
        fb[m] = *reinterpret_cast<const f32x4*>(&s_bk[i][row0 + 4 * m]);
      }
      // sum over the 8 row groups (lanes cg, cg + 8, ..., cg + 56), fixed butterfly order
#pragma unroll
      for (int j = 0; j < CPL; ++j) ks[j] = sum_xor32(sum_xor16(sum_xor8(ks[j])));
      if (output) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) qs[j] = sum_xor32(sum_xor16(sum_xor8(qs[j])));
      }
      float e[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) e[j] = s_v[i][col0 + j] - ks[j];
#pragma unroll
      for (int m = 0; m < RPL / 4; ++m)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < CPL; ++j)
            S[4 * m + u][j] = fmaf(fb[m][u], e[j], fa[m][u] * S[4 * m + u][j]);
      if (output && rg == 0) {
        // each column is held by 8 lanes; row group 0 writes it
#pragma unroll
        for (int j = 0; j < CPL; ++j) s_o[i][col0 + j] = p.scale * fmaf(beta * qk, e[j], qs[j]);
      }
      float* dst_state = nullptr;
      if (t == n_acc - 1) dst_state = p.state_acc;   // after the accepted drafts
      if (t == n_acc) dst_state = p.state;           // after the bonus token
      if (dst_state) {
#pragma unroll
        for (int ii = 0; ii < RPL; ++ii) {
          float* dst = dst_state + sbase + size_t(row0 + ii) * D + col0;
          if constexpr (CPL == 4) {
            // written once, read by a later launch: streaming (non-temporal) stores
            __builtin_nontemporal_store(f32x4{S[ii][0], S[ii][1], S[ii][2], S[ii][3]},
                                        reinterpret_cast<f32x4*>(dst));
          } else if constexpr (CPL == 2) {
            __builtin_nontemporal_store(f32x2{S[ii][0], S[ii][1]}, reinterpret_cast<f32x2*>(dst));
          } else {
#pragma unroll
            for (int j = 0; j < CPL; ++j) dst[j] = S[ii][j];
          }
        }
      }
    }
    if (more) stage_block();   // s_raw of this block was last read before the first barrier
    lds_barrier();

    // ---------------- gated RMS normalisation of the block's outputs ----------------------
    // 32 threads per token, CPG consecutive channels each; the sum of squares in a fixed
    // order (the thread's channels, then the same butterfly as the input norms)
    if (tid < 32 * NB) {
      const int i = tid >> 5, l = tid & 31;
      const int t = tb + i;
      const bool live = i < nb && t >= n_acc;
      const int c0 = CPG * l;
      float ov[CPG];
      float osq = 0.f;
#pragma unroll
      for (int m = 0; m < CPG; ++m) {
        ov[m] = live ? s_o[i][c0 + m] : 0.f;
        osq = fmaf(ov[m], ov[m], osq);
      }
      osq = sum_xor16(sum_xor8(sum_mirror8(sum_xor2(sum_xor1(osq)))));
      if (live) {
        const float rinv = 1.f / sqrtf(osq / float(D) + p.eps_rms);
        Tout* dst = reinterpret_cast<Tout*>(p.o) + ((size_t(r) * p.n_new + (t - n_acc)) * H + h) * D;
        // one vector store per thread
#pragma unroll
        for (int m = 0; m < CPG; ++m)
          ov[m] = ov[m] * rinv * p.norm_w[c0 + m] * s_z[i][c0 + m];
        if constexpr (CPG == 4 && sizeof(Tout) == 2)
          *reinterpret_cast<bf16x4*>(dst + c0) =
              bf16x4{(__bf16)ov[0], (__bf16)ov[1], (__bf16)ov[2], (__bf16)ov[3]};
        else if constexpr (CPG == 4)
          *reinterpret_cast<f32x4*>(dst + c0) = f32x4{ov[0], ov[1], ov[2], ov[3]};
        else if constexpr (CPG == 2 && sizeof(Tout) == 2)
          *reinterpret_cast<bf16x2*>(dst + c0) = bf16x2{(__bf16)ov[0], (__bf16)ov[1]};
        else
          *reinterpret_cast<f32x2*>(dst + c0) = f32x2{ov[0], ov[1]};
      }
    }
    if (more) lds_barrier();   // the next block rewrites the shared vectors
  }
}

template <int D, int W, int NW>
static hipError_t launch_decode_nw(const DecodeParams& p, hipStream_t stream) {
  if (p.out_f32)
    hipLaunchKernelGGL((decode_replay_kernel<D, W, float, NW>), dim3(p.R * p.H), dim3(64 * NW),
                       0, stream, p);
  else
    hipLaunchKernelGGL((decode_replay_kernel<D, W, __bf16, NW>), dim3(p.R * p.H), dim3(64 * NW),
                       0, stream, p);
  return hipGetLastError();
}

template <int D, int W>
static hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (p.waves) {
    case 4: return launch_decode_nw<D, W, 4>(p, stream);
    case 8: return launch_decode_nw<D, W, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static hipError_t launch_decode_w(const DecodeParams& p, hipStream_t stream) {
  switch (p.conv_width) {
    case 1: return launch_decode<D, 1>(p, stream);
    case 2: return launch_decode<D, 2>(p, stream);
    case 3: return launch_decode<D, 3>(p, stream);
    case 4: return launch_decode<D, 4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_replay(const DecodeParams& p, hipStream_t stream) {
  if (p.D == 128) return launch_decode_w<128>(p, stream);
  if (p.D == 64) return launch_decode_w<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
