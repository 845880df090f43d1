// Chunked KDA prefill on gfx950.
//
// Method ("Noyaux KDA et FlashKDA", sections "FlashKDA : le noyau par blocs" and "Le rôle de
// la décroissance bornée"; AMD blog "Dentro de los esfuerzos de optimización de Kimi K3",
// "Nota técnica: Precisión del KDA y memoria on-chip"). For a chunk of C = 64 tokens entering
// with state S (d_k x d_v), with Gamma the in-chunk cumulative floored log-decay per key
// channel:
//   A[r,s] = beta_r sum_i k[r,i] k[s,i] e^{Gamma[r,i]-Gamma[s,i]}   (s < r)
//   T      = (I + A)^{-1}                      fp32, unit lower triangular
//   U      = T diag(beta) (V - (K * e^Gamma) S)
//   M[r,s] = sum_i q[r,i] k[s,i] e^{Gamma[r,i]-Gamma[s,i]}        (s <= r)
//   O      = scale ((Q * e^Gamma) S + M U)
//   S     <- diag(e^{Gamma_L}) S + (K * e^{Gamma_L - Gamma})^T U
// (U is the chunk's block of beta-weighted delta errors; applying T to V - K_Gamma S keeps
// the prediction error in fp32 before the triangular solve.)
//
// Exponent safety: e^{Gamma_r - Gamma_s} is never formed as e^{Gamma_r} e^{-Gamma_s} over the
// whole chunk (that overflows fp32). The chunk is cut into four 16-token sub-blocks. Row
// operands are referenced to the start of their sub-block (rho = e^{lambda} <= 1), column
// operands to its end (kappa <= 1); the gap between two sub-blocks is a per-channel product
// of whole-sub-block decays (<= 1). Inside a diagonal sub-block the column operand is k / rho,
// at most e^{16 |g_min|}: the floor keeps it finite, which is what lets every causal tile,
// diagonal ones included, run as a dense matrix product.
//
// Precision. The inverse is fp32 end to end (fp32 inputs, fp32 16x16x4 MFMA accumulation)
// and rounded only once complete. The model's outputs are heavy-tailed (a read-out is a sum
// of products of near-Gaussian factors, max |o| ~ 10-30 x RMS), so a single bf16 rounding of
// a dominant factor would cost up to ~2.5% of the output RMS. Three kinds of operands avoid it:
//  * fp16 (11-bit significand, one MFMA) for factors bounded well inside the fp16 range:
//    Q e^Gamma, K e^Gamma and K e^{Gamma_L - Gamma} (at most 1 for unit-norm q, k) and the
//    state S in its products with them. With unit keys, beta in [0, 1] and g <= 0 a token adds
//    at most v_c^2 to the squared norm of state column c, so |S| stays below
//    sqrt(|h0 column|^2 + sum_t v_{t,c}^2), far inside fp16's 65504;
//  * fp16 hi + lo pairs (~22 bits, two or three MFMAs) for M (at most 1) and U, whose rows are
//    the tokens' weighted errors beta (v - S'^T k), bounded like S;
//  * bf16 hi + lo pairs (~16 bits, three MFMAs: hi*hi + lo*hi + hi*lo) where a factor can be
//    large or tiny: T diag(beta), V - K_Gamma S, and the operands of M's diagonal blocks,
//    whose in-block decay ratios reach e^{16 |g_min|}.
// A itself takes single bf16 operands (with an fp32 accumulation and an fp32 inverse); the
// emulation of every rounding point showed no gain from splitting them.
//
// Work decomposition: one workgroup (4 waves) per (sequence, head, 64-wide value tile).
// Value columns of S never mix, so each wave owns 16 columns of S in its MFMA accumulators
// for the whole sequence (the state never leaves registers between chunks). The four waves
// share the per-chunk prologue through LDS.
#include <type_traits>

#include "kda_chunk_io.h"
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <class Pol, int DK>
struct ChunkLayout {
  using E = typename Pol::E;
  // Row strides of 2 dwords modulo 32 banks: the 16 rows read by one 16-lane group of an
  // MFMA fragment load land on distinct bank pairs (conflict-free 8-byte reads).
  static constexpr int kPadE = sizeof(E) == 2 ? 4 : 4;
  static constexpr int LDP = DK + kPadE;   // row-major [64 tokens][DK] tiles
  static constexpr int LDT = 64 + kPadE;   // [rows][64 tokens] tiles
  static constexpr int LDA = 64 + 4;       // fp32 A / T working matrix
  static constexpr int kLo = Pol::kSplit ? 1 : 0;
  static constexpr size_t tP = size_t(64) * LDP * sizeof(E);
  static constexpr size_t tT = size_t(DK) * LDT * sizeof(E);
  static constexpr size_t t64 = size_t(64) * LDT * sizeof(E);
  // ---- region X, prologue view: q rho (hi, lo), k / rho (hi, lo), k rho, k kappa
  static constexpr size_t oQr = 0;
  static constexpr size_t oQrLo = oQr + tP;
  static constexpr size_t oKd = oQrLo + kLo * tP;
  static constexpr size_t oKdLo = oKd + tP;
  static constexpr size_t oKr = oKdLo + kLo * tP;
  static constexpr size_t oKc = oKr + tP;
  static constexpr size_t kXA = oKc + tP;
  // ---- region X, recurrence view: Q e^Gamma (fp16) over q rho and K e^Gamma (fp16) over
  //      k / rho, row for row (a thread rewrites in place the elements it reads back), then
  //      (K e^{GL-Gamma})^T (fp16) over k rho, which is dead by then
  static constexpr size_t oQg = oQr;
  static constexpr size_t oKg = oKd;
  static constexpr size_t oKhT = oKr;
  static constexpr size_t kXD = oKhT + tT;
  static constexpr size_t kX = kXA > kXD ? kXA : kXD;
  // ---- region Y: fp32 A / T
  static constexpr size_t oA = kX;
  static constexpr size_t kY = size_t(64) * LDA * 4;
  // ---- region Z: M (fp16 hi, lo); region W: T diag(beta) (bf16 hi, lo), both written during the prologue
  //      while region X still holds the prologue tiles
  static constexpr size_t oM = oA + kY;
  static constexpr size_t oMLo = oM + t64;
  static constexpr size_t oT = oMLo + kLo * t64;
  static constexpr size_t oTLo = oT + t64;
  // ---- small
  static constexpr size_t oBeta = oTLo + kLo * t64;
  static constexpr size_t oBP = oBeta + 64 * 4;        // [4][DK] sub-block decay products
  static constexpr size_t oDecay = oBP + 4 * DK * 4;   // [DK] whole-chunk decay
  static constexpr size_t kBytes = oDecay + DK * 4;
  static_assert(kBytes <= 160 * 1024, "LDS budget of one CDNA4 compute unit");
};

// t * b split into a hi + lo pair: hi rounds the fp32 product, lo is the exact remainder
// rounded (one explicit fma), so the bits never depend on whether the compiler fuses the
// product into the subtraction
template <class Pol>
__device__ __forceinline__ void store_split_prod(typename Pol::E* hi, typename Pol::E* lo,
                                                 int idx, float t, float b) {
  using E = typename Pol::E;
  const E h = from_f32<E>(t * b);
  hi[idx] = h;
  if constexpr (Pol::kSplit) lo[idx] = from_f32<E>(fmaf(t, b, -to_f32(h)));
}
__device__ __forceinline__ void split_prod_bf16(float t, float b, __bf16& h, __bf16& l) {
  h = (__bf16)(t * b);
  l = (__bf16)fmaf(t, b, -(float)h);
}
// one element as an fp16 hi + lo pair (fp32 for fp32 inputs)
template <class Pol>
__device__ __forceinline__ void store_split_r(typename Pol::ER* hi, typename Pol::ER* lo, int idx,
                                              float x) {
  using R = typename Pol::ER;
  const R h = R(x);
  hi[idx] = h;
  if constexpr (Pol::kSplit) lo[idx] = R(x - float(h));
}

// Row-block IA of A and (kM) row-block 3 - IA of M for one wave. Column operands: k / rho on
// the diagonal block, k kappa next to it, k kappa times the decay gap further down. Without M
// (the transition pass) block (3, 0) moves from wave 3 to wave 0, so the waves run 8, 8, 12
// and 12 MFMAs instead of 4 to 16.
template <class Pol, class L, int DK, int IA, bool kM>
__device__ __forceinline__ void am_rows(const typename Pol::E* sKr, const typename Pol::E* sKd,
                                        const typename Pol::E* sKdLo, const typename Pol::E* sKc,
                                        const typename Pol::E* sQr, const typename Pol::E* sQrLo,
                                        const float* sBP, const float* sBeta, float* sA,
                                        typename Pol::ER* sM, typename Pol::ER* sMLo,
                                        typename Pol::E* sT, typename Pol::E* sTLo, int ln, int q4) {
  using Frag = typename Pol::Frag;
  constexpr int NS = Pol::slices(DK);
  constexpr int IM = 3 - IA;
  constexpr bool kTake30 = !kM && IA == 0;   // this wave also computes A block (3, 0)
  constexpr int kJ0 = (!kM && IA == 3) ? 1 : 0;   // first column block of the row
  // M block (3, 0) moves from wave 0 to wave 3 (bf16 inputs, where M's off-diagonal column
  // operands are rebuilt pairs): the waves then run 10, 11, 9 and 10 MFMAs per k-slice and
  // 2, 2, 1 and 1 rebuilt blocks, instead of 13, 11, 9, 7 and 3, 2, 1, 0
  constexpr bool kM30 = kM && Pol::kSplit && IA == 3;
  constexpr int kMJ0 = (kM && Pol::kSplit && IM == 3) ? 1 : 0;   // first M column block
  // gap between sub-blocks i and j (i - j >= 2): the whole-sub-block decays strictly between
  // them, (2, 0) -> P_1, (3, 1) -> P_2, (3, 0) -> P_1 P_2 (sBP row b holds P_b per channel)
  const float* P1 = sBP + DK;
  const float* P2 = sBP + 2 * DK;
  f32x4 accA[4], accM[4], acc30 = zero4(), accM30 = zero4();
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    accA[jb] = zero4();
    accM[jb] = zero4();
  }
#pragma unroll
  for (int pp = 0; pp < NS; ++pp) {
    const Frag rowA = Pol::load(sKr, L::LDP, 16 * IA + ln, pp, q4);
    Frag rowM, colA[4], colM[4], colMl[4], dKl, dQl, rowM3, dQl3, colM30, colM30l;
    if constexpr (kM) rowM = Pol::load(sQr, L::LDP, 16 * IM + ln, pp, q4);
    if constexpr (kM30) {
      const float* const fac[3] = {sBP, sBP + DK, sBP + 2 * DK};
      rowM3 = Pol::load(sQr, L::LDP, 48 + ln, pp, q4);
      dQl3 = Pol::load(sQrLo, L::LDP, 48 + ln, pp, q4);
      Pol::template load_pair_scaled<3>(sKd, sKdLo, L::LDP, ln, pp, q4, fac, colM30, colM30l);
    }
#pragma unroll
    for (int jb = kJ0; jb <= IA; ++jb) {
      if (jb == IA) colA[jb] = Pol::load(sKd, L::LDP, 16 * jb + ln, pp, q4);
      else if (jb == IA - 1) colA[jb] = Pol::load(sKc, L::LDP, 16 * jb + ln, pp, q4);
      else if (jb == 0 && IA == 3) colA[jb] = Pol::load_scaled2(sKc, L::LDP, ln, pp, q4, P1, P2);
      else colA[jb] = Pol::load_scaled(sKc, L::LDP, 16 * jb + ln, pp, q4, jb == 0 ? P1 : P2);
    }
#pragma unroll
    for (int jb = kMJ0; jb <= IM; ++jb) {
      if constexpr (!kM) break;
      if (jb == IM) {
        colM[jb] = Pol::load(sKd, L::LDP, 16 * jb + ln, pp, q4);
      } else if constexpr (Pol::kSplit) {
        // off-diagonal blocks: k kappa times the decay gap, k / rho times the decays of the
        // sub-blocks jb .. IM - 1, rebuilt from the k / rho pair as a pair (a single bf16 k
        // kappa here was the largest error source of the outputs)
        const float* const fac[3] = {sBP + jb * DK, sBP + (jb + 1) * DK, sBP + (jb + 2) * DK};
        if (IM - jb == 1)
          Pol::template load_pair_scaled<1>(sKd, sKdLo, L::LDP, 16 * jb + ln, pp, q4, fac, colM[jb], colMl[jb]);
        else if (IM - jb == 2)
          Pol::template load_pair_scaled<2>(sKd, sKdLo, L::LDP, 16 * jb + ln, pp, q4, fac, colM[jb], colMl[jb]);
        else
          Pol::template load_pair_scaled<3>(sKd, sKdLo, L::LDP, 16 * jb + ln, pp, q4, fac, colM[jb], colMl[jb]);
      } else {
        if (jb == IM - 1) colM[jb] = Pol::load(sKc, L::LDP, 16 * jb + ln, pp, q4);
        else if (jb == 0 && IM == 3) colM[jb] = Pol::load_scaled2(sKc, L::LDP, ln, pp, q4, P1, P2);
        else colM[jb] = Pol::load_scaled(sKc, L::LDP, 16 * jb + ln, pp, q4, jb == 0 ? P1 : P2);
      }
    }
    if constexpr (Pol::kSplit && kM) {
      dKl = Pol::load(sKdLo, L::LDP, 16 * IM + ln, pp, q4);
      dQl = Pol::load(sQrLo, L::LDP, 16 * IM + ln, pp, q4);
    }
#pragma unroll
    for (int jb = kJ0; jb <= IA; ++jb) accA[jb] = Pol::mma(colA[jb], rowA, accA[jb]);
    if constexpr (kTake30) {
      const Frag row3 = Pol::load(sKr, L::LDP, 48 + ln, pp, q4);
      acc30 = Pol::mma(Pol::load_scaled2(sKc, L::LDP, ln, pp, q4, P1, P2), row3, acc30);
    }
    if constexpr (kM) {
#pragma unroll
      for (int jb = kMJ0; jb <= IM; ++jb) accM[jb] = Pol::mma(colM[jb], rowM, accM[jb]);
      if constexpr (kM30) accM30 = Pol::mma(colM30, rowM3, accM30);
      if constexpr (Pol::kSplit) {
        accM[IM] = Pol::mma(dKl, rowM, accM[IM]);
#pragma unroll
        for (int jb = kMJ0; jb < IM; ++jb) accM[jb] = Pol::mma(colMl[jb], rowM, accM[jb]);
        if constexpr (kM30) accM30 = Pol::mma(colM30l, rowM3, accM30);
        // the lo half of q rho on every block of the row
#pragma unroll
        for (int jb = kMJ0; jb <= IM; ++jb) accM[jb] = Pol::mma(colM[jb], dQl, accM[jb]);
        if constexpr (kM30) accM30 = Pol::mma(colM30, dQl3, accM30);
      }
    }
  }
  // register e of block (row i, column jb): row 16 i + ln, column 16 jb + 4 q4 + e
  const int ra = 16 * IA + ln, rm = 16 * IM + ln;
  const float br = sBeta[ra];
#pragma unroll
  for (int jb = kJ0; jb <= IA; ++jb) {
    f32x4 outv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * jb + 4 * q4 + e;
      outv[e] = (jb == IA && s >= ra) ? 0.f : br * accA[jb][e];
    }
    *reinterpret_cast<f32x4*>(sA + ra * L::LDA + 16 * jb + 4 * q4) = outv;
  }
  if constexpr (kTake30) {
    const float b3 = sBeta[48 + ln];
    *reinterpret_cast<f32x4*>(sA + (48 + ln) * L::LDA + 4 * q4) = b3 * acc30;
  }
#pragma unroll
  for (int jb = kMJ0; jb <= IM; ++jb) {
    if constexpr (!kM) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * jb + 4 * q4 + e;
      store_split_r<Pol>(sM, sMLo, rm * L::LDT + s, (jb == IM && s > rm) ? 0.f : accM[jb][e]);
    }
  }
  if constexpr (kM30) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      store_split_r<Pol>(sM, sMLo, (48 + ln) * L::LDT + 4 * q4 + e, accM30[e]);
  }
  // Diagonal block IA of T = (I + A)^{-1} in fp32, by right-looking substitution: the quad of
  // lanes 4 jc .. 4 jc + 3 solves column jc, lane part pp holding rows pp, pp + 4, pp + 8,
  // pp + 12. Once x_s is final its owner broadcasts it inside the quad and it is removed from
  // every row (the block is zero on and above its diagonal, so later rows only). The block
  // was written just above by other lanes of this wave: a wave-scope fence orders those LDS
  // writes before the reads.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  {
    const int lane = 16 * q4 + ln;
    const int jc = lane >> 2, pp = lane & 3;
    const float* Ab = sA + 16 * IA * L::LDA + 16 * IA;
    f32x4 arow[4][4];   // rows pp + 4 i, columns 4 m .. 4 m + 3
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        arow[i][m] = *reinterpret_cast<const f32x4*>(Ab + (pp + 4 * i) * L::LDA + 4 * m);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (pp + 4 * i == jc) ? 1.f : 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 15; ++s2) {
      float xs;
      switch (s2 & 3) {
        case 0: xs = quad_bcast<0>(x[s2 >> 2]); break;
        case 1: xs = quad_bcast<1>(x[s2 >> 2]); break;
        case 2: xs = quad_bcast<2>(x[s2 >> 2]); break;
        default: xs = quad_bcast<3>(x[s2 >> 2]); break;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = fmaf(-arow[i][s2 >> 2][s2 & 3], xs, x[i]);
    }
    const float bj = sBeta[16 * IA + jc];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * IA + pp + 4 * i;
      sA[r * L::LDA + 16 * IA + jc] = x[i];
      store_split_prod<Pol>(sT, sTLo, r * L::LDT + 16 * IA + jc, x[i], bj);
    }
  }
}

// four consecutive elements (8 bytes for bf16, 16 for fp32) and their hi / lo split
template <class Pol>
__device__ __forceinline__ void store4(typename Pol::E* dst, const float* x) {
  if constexpr (sizeof(typename Pol::E) == 2)
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  else
    *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
}

// four consecutive elements as read-out operands (fp16 for bf16 inputs)
template <class Pol>
__device__ __forceinline__ void store4r(typename Pol::ER* dst, const float* x) {
  if constexpr (sizeof(typename Pol::ER) == 2)
    *reinterpret_cast<f16x4*>(dst) = __builtin_convertvector((f32x4{x[0], x[1], x[2], x[3]}), f16x4);
  else
    *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
}

template <class Pol>
__device__ __forceinline__ void store4_split(typename Pol::E* hi, typename Pol::E* lo,
                                             const float* x) {
  if constexpr (Pol::kSplit) {
    bf16x4 a, c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = (__bf16)x[e];
      c[e] = (__bf16)(x[e] - (float)a[e]);
    }
    *reinterpret_cast<bf16x4*>(hi) = a;
    *reinterpret_cast<bf16x4*>(lo) = c;
  } else {
    store4<Pol>(hi, x);
  }
}

// Activations of the raw token stage, with the hardware reciprocal and exponential (each
// within an ulp or two of fp32; the stage's outputs then pass through bf16 and fp16 operands)
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
__device__ __forceinline__ float silu_fast(float x) { return x * sigmoid_fast(x); }

// Prep pass: copy one chunk's serial-step operands from their LDS tiles to its slot, in
// fragment order (wave w writes fragments w, w + 4, ...; one 16-byte store per lane each).
template <class Pol, class L, int DK>
__device__ __forceinline__ void prep_store(char* slot, const typename Pol::ER* sKg,
                                           const typename Pol::ER* sQg, const typename Pol::E* sT,
                                           const typename Pol::E* sTLo, const typename Pol::ER* sM,
                                           const typename Pol::ER* sMLo,
                                           const typename Pol::ER* sKhT, const float* sDecay,
                                           int w, int lane, int ln, int q4) {
  using OS = OpSlot<DK>;
  constexpr int NS = OS::NS;
  // streaming stores: the slot is read back by the walk, a launch later (from HBM, not L2)
  auto put = [&](int f, auto frag) {
    static_assert(sizeof(frag) == 16, "one 16-byte fragment per lane");
    __builtin_nontemporal_store(
        frag, reinterpret_cast<decltype(frag)*>(slot + size_t(f) * 1024 + lane * 16));
  };
  for (int f = w; f < 4 * NS; f += 4) {
    put(OS::fKg + f, Pol::load_r(sKg, L::LDP, 16 * (f / NS) + ln, f % NS, q4));
    put(OS::fQg + f, Pol::load_r(sQg, L::LDP, 16 * (f / NS) + ln, f % NS, q4));
  }
  for (int i = w; i < 6; i += 4) {
    const int rb = i < 2 ? i : (i < 4 ? 2 : 3), pp = i < 2 ? 0 : (i & 1);
    put(OS::fT + i, Pol::load(sT, L::LDT, 16 * rb + ln, pp, q4));
    put(OS::fTLo + i, Pol::load(sTLo, L::LDT, 16 * rb + ln, pp, q4));
    put(OS::fM + i, Pol::load_r(sM, L::LDT, 16 * rb + ln, pp, q4));
    put(OS::fMLo + i, Pol::load_r(sMLo, L::LDT, 16 * rb + ln, pp, q4));
  }
  for (int f = w; f < 2 * OS::NTD; f += 4)
    put(OS::fKh + f, Pol::load_r(sKhT, L::LDT, 16 * (f / 2) + ln, f % 2, q4));
  if (w == 0 && lane < DK / 4)
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(sDecay + 4 * lane),
                                reinterpret_cast<f32x4*>(slot + size_t(OS::kDecay) * 1024 +
                                                         lane * 16));
}

// kOut false: the transition pass of the segment-parallel path, which keeps only the state
// (no M, no Q e^Gamma tile, no output products, q is never read).
// kPrep true: pass 1 of the two-pass prefill. One workgroup per (sequence, group of chunks,
// head) runs the prologue of each chunk and stores the serial step's operands to the chunk's
// slot instead of running the step (no state, values or outputs).
template <class Pol, typename Tio, typename Tout, int DK, bool kOut, bool kPrep = false,
          bool kRaw = false>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkParams p) {
  using L = ChunkLayout<Pol, DK>;
  using E = typename Pol::E;
  using Frag = typename Pol::Frag;
  using ER = typename Pol::ER;
  using FragR = typename Pol::FragR;
  using PM = ProMap<DK>;
  constexpr int TPT = PM::kTPT;            // tokens per thread in the prologue
  constexpr int NS = Pol::slices(DK);      // k-slices over key channels
  constexpr int NT = Pol::slices(64);      // k-slices over the chunk's tokens
  constexpr int NTD = DK / 16;             // 16-row tiles of S per wave
  constexpr int VT = 64;

  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  E* sQr = reinterpret_cast<E*>(smem + L::oQr);
  E* sQrLo = reinterpret_cast<E*>(smem + L::oQrLo);
  E* sKd = reinterpret_cast<E*>(smem + L::oKd);
  E* sKdLo = reinterpret_cast<E*>(smem + L::oKdLo);
  E* sKr = reinterpret_cast<E*>(smem + L::oKr);
  E* sKc = reinterpret_cast<E*>(smem + L::oKc);
  ER* sQg = reinterpret_cast<ER*>(smem + L::oQg);
  ER* sKhT = reinterpret_cast<ER*>(smem + L::oKhT);
  ER* sKg = reinterpret_cast<ER*>(smem + L::oKg);
  E* sT = reinterpret_cast<E*>(smem + L::oT);
  E* sTLo = reinterpret_cast<E*>(smem + L::oTLo);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  ER* sM = reinterpret_cast<ER*>(smem + L::oM);
  ER* sMLo = reinterpret_cast<ER*>(smem + L::oMLo);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
  float* sBP = reinterpret_cast<float*>(smem + L::oBP);
  float* sDecay = reinterpret_cast<float*>(smem + L::oDecay);

  // ---- which (sequence, segment, head, state tile): the tiles of one unit share an XCD
  int vt;
  const int unit = block_unit(blockIdx.x, p.n_vt, &vt);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int DV = p.dv;
  const int h = unit % H;
  const int sj = unit / H;              // global segment index n * n_seg + j
  const int n = p.seq0 + sj / p.n_seg;
  const int j = sj % p.n_seg;
  const int mode = p.mode;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int q4 = lane >> 4;   // k-group of the lane inside an MFMA fragment
  const int ln = lane & 15;   // row / column of the lane inside a 16x16 tile

  int bos, eos;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
  } else {
    bos = n * p.seq_len;
    eos = bos + p.seq_len;
  }
  // operand slot of the sequence's first chunk (prep pass)
  const long long seq_slot0 = seq_first_slot(bos, p.slot_tok0, n, p.seq0);
  const int seq_bos = bos;
  {
    // chunk-aligned contiguous segments
    int c_lo;
    segment_range(seq_bos, eos, j, p.n_seg, &bos, &eos, &c_lo);
  }
  // transition mode: tiles [0, DK/64) hold P (zero values, identity start), the rest Q
  const bool p_tile = mode == kModeTransition && vt < DK / 64;
  // column of v feeding this tile (P tiles read none; their address stays at column 0)
  const int vcol0 = p_tile ? 0 : (mode == kModeTransition ? vt - DK / 64 : vt) * VT;
  const int ldS = mode == kModeTransition ? DK + DV : DV;                // state row stride
  Tout* __restrict__ go = reinterpret_cast<Tout*>(p.o);
  const int col0 = vt * VT + 16 * w;   // first state column owned by this wave

  // ---- entering state in accumulator layout: tile t, register e = row 16t + 4 q4 + e
  f32x4 S[NTD];
  const float* s_in = nullptr;
  if (mode == kModeForward && p.h0) s_in = p.h0 + (size_t(n) * H + h) * DK * DV;
  if (mode == kModeReplay) s_in = p.ws_sin + (size_t(sj) * H + h) * DK * DV;
#pragma unroll
  for (int t = 0; t < NTD; ++t) {
    if constexpr (kPrep) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * t + 4 * q4 + e;
      float x = 0.f;
      if (s_in) x = s_in[size_t(c) * DV + col0 + ln];
      if (p_tile) x = (c == col0 + ln) ? 1.f : 0.f;
      S[t][e] = x;
    }
  }

  // strictly upper sub-blocks of M and T' stay zero for the whole sequence
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int r = idx >> 6, s = idx & 63;
    if ((s >> 4) > (r >> 4)) {
      sM[r * L::LDT + s] = ER(0.f);
      sT[r * L::LDT + s] = from_f32<E>(0.f);
      if constexpr (Pol::kSplit) {
        sMLo[r * L::LDT + s] = ER(0.f);
        sTLo[r * L::LDT + s] = from_f32<E>(0.f);
      }
    }
  }

  RawChunk<Tio, DK, kRaw> raw;

  // raw projections: the convolution taps of this thread's q and k channels (prologue
  // mapping) and of its value channels (value-convolution mapping), right-aligned in a window
  // of four (tap 3 multiplies the current token, tap 3 - i the token i before it; taps
  // beyond the width are zero), and the leaving tail
  float wq[4][4], wk[4][4], wv[4][4];
  if constexpr (kRaw) {
    constexpr int C3 = 3 * DK;   // raw mode: d_v = d_k
    const int W = p.conv_width;
    const int cq0 = 4 * (lane % PM::kLPT);
    const int cv0 = 4 * (tid % (DK / 4));
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int mw = m - (4 - W);   // the tap of the width-W window
        const bool on = mw >= 0;
        wq[c][m] = on ? p.conv_w[(size_t(h) * C3 + cq0 + c) * W + mw] : 0.f;
        wk[c][m] = on ? p.conv_w[(size_t(h) * C3 + DK + cq0 + c) * W + mw] : 0.f;
        wv[c][m] = on ? p.conv_w[(size_t(h) * C3 + 2 * DK + cv0 + c) * W + mw] : 0.f;
      }
    // the sequence's leaving tail: its last W - 1 raw inputs (older ones from the entering
    // tail when it is shorter), written by the workgroup of the group holding its last chunk
    const int seq_eos = p.cu_seqlens ? p.cu_seqlens[n + 1] : seq_bos + p.seq_len;
    const int len = seq_eos - seq_bos;
    const bool last_group = (len == 0 && j == 0) || (bos < eos && eos == seq_eos);
    if (p.conv_tail_out && W > 1 && last_group) {
      const size_t tb = (size_t(n) * H + h) * C3 * (W - 1);
      for (int idx = tid; idx < C3 * (W - 1); idx += 256) {
        const int ch = idx / (W - 1), m = idx % (W - 1);
        int slot;
        const int pos = raw_tail_out_row(seq_bos, seq_eos, W, m, &slot);
        float val = 0.f;
        if (pos >= 0) {
          const __bf16* src = ch < DK ? reinterpret_cast<const __bf16*>(p.q)
                                      : ch < 2 * DK ? reinterpret_cast<const __bf16*>(p.k)
                                                    : reinterpret_cast<const __bf16*>(p.v);
          const int cc = ch < DK ? ch : ch < 2 * DK ? ch - DK : ch - 2 * DK;
          val = (float)src[(size_t(pos) * H + h) * DK + cc];
        } else if (p.conv_tail_in) {
          val = p.conv_tail_in[tb + size_t(ch) * (W - 1) + slot];
        }
        p.conv_tail_out[tb + size_t(ch) * (W - 1) + m] = val;
      }
    }
  }

  if (bos < eos)
    load_chunk_any<kPrep ? kLoadAll & ~kLoadV : (kOut ? kLoadAll : kLoadAll & ~kLoadQ), Tio, DK, 0,
                   8, kRaw>(raw, p, bos, min(kChunk, eos - bos), w, lane, h, vcol0);

  // raw mode: a chunk's convolution history (the q, k rows before each thread's first
  // token) and its raw value rows (value mapping: 4 channels x kTPV tokens per thread, plus
  // the three rows before), loaded one chunk ahead like the other inputs. Rows before the
  // sequence come from the entering tail when they are used.
  using VM = RawValueMap<DK>;
  constexpr int kTPV = VM::kTPV;
  bf16x4 pre_hq[3], pre_hk[3], pre_v[kTPV + 3];
  auto raw_prefetch = [&](int cs, int L, int lane_) {
    const int W = p.conv_width;
    const int rb0_ = 16 * w + (lane_ / PM::kLPT) * TPT;
    const int c0_ = 4 * (lane_ % PM::kLPT);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      // rows of the chunk's own sequence up to its last row only (raw_history_row)
      const int tok = raw_history_row(cs, L, rb0_, i, W, seq_bos);
      pre_hq[i] = pre_hk[i] = bf16x4{};
      if (tok >= 0) {
        const size_t off = (size_t(tok) * H + h) * DK + c0_;
        pre_hq[i] = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(p.q) + off);
        pre_hk[i] = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(p.k) + off);
      }
    }
    const int cv0 = VM::cv0(tid), tv0 = VM::tv0(tid);
#pragma unroll
    for (int i = 0; i < kTPV + 3; ++i) {
      const int tok = raw_value_row(cs, L, tv0, i, W, seq_bos);
      pre_v[i] = bf16x4{};
      if (tok >= 0)
        pre_v[i] = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(p.v) +
                                                    (size_t(tok) * H + h) * DK + cv0);
    }
  };
  if constexpr (kRaw)
    if (bos < eos) raw_prefetch(bos, min(kChunk, eos - bos), lane);

  const int lane0 = lane, q4_0 = q4, ln0 = ln;
  for (int cstart = bos; cstart < eos; cstart += kChunk) {
    const int Lc = min(kChunk, eos - cstart);
    // lane coordinates re-derived per chunk: the LDS addresses built from them are then
    // recomputed in the loop (a few integer ops) instead of being hoisted out of it, where
    // dozens of them would stay live in registers for the whole sequence
    int lane = lane0, q4 = q4_0, ln = ln0;
    asm volatile("" : "+v"(lane), "+v"(q4), "+v"(ln));
    // the next chunk's raw inputs are loaded in small pieces spread over this chunk, once the
    // prologue has consumed the current ones: issuing them never waits on a full memory
    // pipeline and their HBM latency is covered
    const bool more = cstart + kChunk < eos;
    const int nstart = cstart + kChunk, nLc = min(kChunk, eos - nstart);
#define KDA_PREFETCH(parts, lo, hi) \
  if (more) load_chunk_any<parts, Tio, DK, lo, hi, kRaw>(raw, p, nstart, nLc, w, lane, h, vcol0)

    // ================= prologue 1: decay factors and operand tiles ======================
    // rho = e^{lambda} (decay from the sub-block start to token r, inclusive) <= 1;
    // kappa = P / rho (decay after token r to the sub-block end) <= 1; 1/rho <= e^{16|g_min|}
    const int grp = lane / PM::kLPT;
    const int c0 = 4 * (lane % PM::kLPT);
    const int rb0 = 16 * w + grp * TPT;   // first token row of this thread
    float rho[TPT][4], qv[TPT][4], kv[TPT][4];
    float ex[TPT][4];                      // per-token decays e^{max(g, g_min)}
    float lp[4] = {1.f, 1.f, 1.f, 1.f};   // running decay over this thread's tokens
    // e^{max(g, g_min)} = 2^{max(g log2 e, g_min log2 e)}: scaling by log2 e first makes the
    // floor a single max (the product needs no NaN quieting) and feeds v_exp_f32 directly
    const float gmin2 = p.g_min * kLog2e;
    // rows past the end of a ragged last chunk count as zero keys and queries with no decay
    // raw projections: causal depthwise convolution (history from the rows before this
    // thread's first token, or the entering tail before the sequence), optional SiLU, and
    // the L2 norm of each token's q and k over its d_k channels (a sum across the kLPT lanes
    // holding the row)
    float qin[TPT][4], kin[TPT][4];
    if constexpr (kRaw) {
      const int W = p.conv_width;
      constexpr int C3 = 3 * DK;   // raw mode: d_v = d_k
      float hq[3][4], hk[3][4];   // raw q, k of tokens rb0 - 1 - i
#pragma unroll
      for (int i = 0; i < 3; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          hq[i][c] = (float)pre_hq[i][c];   // zero where not loaded
          hk[i][c] = (float)pre_hk[i][c];
        }
        // rows before the sequence: the entering tail's slot of that token, oldest first
        const int m = raw_history_tail_slot(cstart, rb0, i, W, seq_bos);
        if (m >= 0 && p.conv_tail_in) {
          const size_t tb = (size_t(n) * H + h) * C3 * (W - 1);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            hq[i][c] = p.conv_tail_in[tb + size_t(c0 + c) * (W - 1) + m];
            hk[i][c] = p.conv_tail_in[tb + size_t(DK + c0 + c) * (W - 1) + m];
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // window tap m multiplies token t - 3 + m (history rows before the thread's first)
          float yq = 0.f, yk = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int d = t - 3 + m;   // token offset inside this thread's rows
            if (d < -3) continue;
            const float xq = d >= 0 ? to_f32(raw.q[d < 0 ? 0 : d][c]) : hq[d < 0 ? -d - 1 : 0][c];
            const float xk = d >= 0 ? to_f32(raw.k[d < 0 ? 0 : d][c]) : hk[d < 0 ? -d - 1 : 0][c];
            yq = fmaf(wq[c][m], xq, yq);
            yk = fmaf(wk[c][m], xk, yk);
          }
          if (p.act) {
            yq = silu_fast(yq);
            yk = silu_fast(yk);
          }
          qin[t][c] = yq;
          kin[t][c] = yk;
          ssq = fmaf(yq, yq, ssq);
          ssk = fmaf(yk, yk, ssk);
        }
        ssq = sum_xor8(sum_mirror8(sum_xor2(sum_xor1(ssq))));
        ssk = sum_xor8(sum_mirror8(sum_xor2(sum_xor1(ssk))));
        if constexpr (PM::kLPT == 32) {
          ssq = sum_xor16(ssq);
          ssk = sum_xor16(ssk);
        }
        const float rq = __builtin_amdgcn_rsqf(ssq + p.eps_l2);
        const float rk = __builtin_amdgcn_rsqf(ssk + p.eps_l2);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          qin[t][c] *= rq;
          kin[t][c] *= rk;
        }
      }
      // the chunk's convolved values for the walk (fp32: after the activation they reach
      // ~15 x their RMS, and one bf16 rounding of them costs several % of the outputs' RMS):
      // thread = 4 value channels x kTPV tokens
      {
        const int cv0 = VM::cv0(tid), tv0 = VM::tv0(tid);
        float xv[kTPV + 3][4];
#pragma unroll
        for (int i = 0; i < kTPV + 3; ++i) {
#pragma unroll
          for (int c = 0; c < 4; ++c) xv[i][c] = (float)pre_v[i][c];   // zero where not loaded
          const int m = raw_value_tail_slot(cstart, Lc, tv0, i, W, seq_bos);
          if (m >= 0 && p.conv_tail_in) {
            const size_t tb = (size_t(n) * H + h) * C3 * (W - 1);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              xv[i][c] = p.conv_tail_in[tb + size_t(2 * DK + cv0 + c) * (W - 1) + m];
          }
        }
#pragma unroll
        for (int t = 0; t < kTPV; ++t) {
          const int tok = cstart + tv0 + t;
          if (tok >= cstart + Lc) continue;
          float y[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc = fmaf(wv[c][m], xv[t + m][c], acc);
            y[c] = p.act ? silu_fast(acc) : acc;
          }
          *reinterpret_cast<f32x4*>(p.v_conv + (size_t(tok) * H + h) * DK + cv0) =
              f32x4{y[0], y[1], y[2], y[3]};
        }
      }
      // the next chunk's history and value rows: a whole chunk to land
      if (more) raw_prefetch(nstart, nLc, lane);
    }
    auto raw_in = [&](auto full) {
      constexpr bool kFull = decltype(full)::value;
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const bool valid = kFull || rb0 + t < Lc;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (kRaw) {
            // decay e^{max(-softplus(x), g_min)} = max(sigmoid(-x), e^{g_min})
            const float x = (float)raw.g[t][c];
            ex[t][c] = valid ? fmaxf(sigmoid_fast(-x), p.decay_floor) : 1.f;
            kv[t][c] = valid ? kin[t][c] : 0.f;
            qv[t][c] = valid ? qin[t][c] : 0.f;
          } else {
            const float gt = valid ? fmaxf(raw.g[t][c] * kLog2e, gmin2) : 0.f;
            ex[t][c] = __builtin_amdgcn_exp2f(gt);
            kv[t][c] = valid ? to_f32(raw.k[t][c]) : 0.f;
            qv[t][c] = (kOut && valid) ? to_f32(raw.q[t][c]) : 0.f;
          }
          lp[c] *= ex[t][c];
          rho[t][c] = lp[c];
        }
      }
    };
    if (Lc == kChunk) raw_in(std::true_type{});
    else raw_in(std::false_type{});
    // decay of the earlier token groups of the sub-block (exclusive prefix product across
    // lanes) and of the whole sub-block; every lane of a channel gets the same bits
    float bp[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float pre;
      if constexpr (PM::kNG == 2) {
        const float o = __shfl_xor(lp[c], 32);
        pre = grp ? o : 1.f;
        bp[c] = lp[c] * o;
      } else {
        static_assert(PM::kNG == 4, "token groups per sub-block");
        const float a = __shfl_xor(lp[c], 16);
        const float pair = lp[c] * a;
        const float b2 = __shfl_xor(pair, 32);
        pre = ((grp & 2) ? b2 : 1.f) * ((grp & 1) ? a : 1.f);
        bp[c] = pair * b2;
      }
#pragma unroll
      for (int t = 0; t < TPT; ++t) rho[t][c] *= pre;
    }
    float beta_r;
    if constexpr (kRaw)
      beta_r = (16 * w + lane < Lc) ? sigmoid_fast((float)raw.beta) : 0.f;
    else
      beta_r = (16 * w + lane < Lc) ? raw.beta : 0.f;
    // 1 / rho from one reciprocal per channel: 1/rho_t = (1/rho_last) x the decays after t
    float rinv_next[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) rinv_next[c] = __builtin_amdgcn_rcpf(rho[TPT - 1][c]);
#pragma unroll
    for (int t = TPT - 1; t >= 0; --t) {
      float xq[4], xkd[4], xkr[4], xkc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float rh = rho[t][c];
        const float rinv = rinv_next[c];
        if (t > 0) rinv_next[c] = rinv * ex[t][c];
        const float k0 = kv[t][c];
        xq[c] = qv[t][c] * rh;
        xkd[c] = k0 * rinv;
        xkr[c] = k0 * rh;
        xkc[c] = xkd[c] * bp[c];
        qv[t][c] = xq[c];    // q rho
        kv[t][c] = xkr[c];   // k rho
        rho[t][c] = xkc[c];  // k kappa
      }
      const int idx = (rb0 + t) * L::LDP + c0;
      if constexpr (kOut) store4_split<Pol>(sQr + idx, sQrLo + idx, xq);
      store4_split<Pol>(sKd + idx, sKdLo + idx, xkd);
      store4<Pol>(sKr + idx, xkr);
      store4<Pol>(sKc + idx, xkc);
    }
    if (grp == 0) *reinterpret_cast<f32x4*>(sBP + w * DK + c0) = f32x4{bp[0], bp[1], bp[2], bp[3]};
    if (lane < 16) sBeta[16 * w + lane] = beta_r;
    lds_barrier();

    // ---- chunk-level factors from the four sub-block products of each channel (read-only
    //      here; the whole-chunk decay is first read after two more barriers)
    float fs[4], fe[4];
    {
      f32x4 Pb[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) Pb[bb] = *reinterpret_cast<const f32x4*>(sBP + bb * DK + c0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        fs[c] = 1.f;
        fe[c] = 1.f;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          if (bb < w) fs[c] *= Pb[bb][c];
          if (bb > w) fe[c] *= Pb[bb][c];
        }
      }
      if (w == 0 && grp == 0)
        *reinterpret_cast<f32x4*>(sDecay + c0) = Pb[0] * Pb[1] * Pb[2] * Pb[3];
    }


    // ================= prologue 2: A (fp32) and M (hi, lo) sub-blocks ====================
    // wave w: row-block w of A (blocks (w, j <= w)) and row-block 3 - w of M, 40 - 4 w MFMAs
    // (M takes the lo half of q rho on every block, and of k / rho on its diagonal block). The
    // row blocks are compile-time per wave so each slice's fragment loads issue together.
    switch (w) {
      case 0: am_rows<Pol, L, DK, 0, kOut>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, sBeta, sA, sM, sMLo, sT, sTLo, ln, q4); break;
      case 1: am_rows<Pol, L, DK, 1, kOut>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, sBeta, sA, sM, sMLo, sT, sTLo, ln, q4); break;
      case 2: am_rows<Pol, L, DK, 2, kOut>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, sBeta, sA, sM, sMLo, sT, sTLo, ln, q4); break;
      default: am_rows<Pol, L, DK, 3, kOut>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, sBeta, sA, sM, sMLo, sT, sTLo, ln, q4); break;
    }
    KDA_PREFETCH(kLoadG, 0, 4);
    lds_barrier();

    // ================= prologue 3: recurrence operand tiles; off-diagonal inverse ===========
    {
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const int idx = (rb0 + t) * L::LDP + c0;
        float xq[4], xk[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          xq[c] = qv[t][c] * fs[c];   // q e^{Gamma}
          xk[c] = kv[t][c] * fs[c];   // k e^{Gamma}
        }
        if constexpr (kOut) store4r<Pol>(sQg + idx, xq);
        store4r<Pol>(sKg + idx, xk);
      }
      KDA_PREFETCH(kLoadG, 4, 6);
      // (K e^{Gamma_L - Gamma})^T: channel rows, this thread's TPT consecutive tokens
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int t4 = 0; t4 < TPT; t4 += 4) {
          float col[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) col[e] = rho[t4 + e][c] * fe[c];
          const int idx = (c0 + c) * L::LDT + rb0 + t4;
          store4r<Pol>(sKhT + idx, col);
        }
      }
      KDA_PREFETCH(kLoadG, 6, 8);
    }
    // T = (I + A)^{-1} in fp32, by 16x16 blocks. The diagonal blocks came with A (one per
    // wave); waves 1 and 3 now run level 1 on fp32 MFMA (16x16x4): T_10 = -T_11 A_10 T_00,
    // T_32 = -T_33 A_32 T_22. After a barrier, level 2 fills the lower-left 32x32 block
    // -T_[23][23] A_[23][01] T_[01][01], one 16x16 block per wave (T_20, T_21, T_30, T_31).
    // T_ij (i > j) is stored in the free upper position (j, i) so that A_ij stays readable;
    // every block also goes out as T'_ij = T_ij diag(beta) (hi, lo) for the serial step.
    auto tblk = [&](int bi, int bj) -> float* {
      return bi == bj ? sA + 16 * bi * L::LDA + 16 * bi : sA + 16 * bj * L::LDA + 16 * bi;
    };
    auto ablk = [&](int bi, int bj) -> const float* { return sA + 16 * bi * L::LDA + 16 * bj; };
    // X += A_blk * T_blk (16x16x16, natural k order: k-step kk2 takes k = 4 kk2 + q4) and
    // Y += T_blk * X with X in accumulator layout (k-step e takes rows 4 q4 + e).
    // Two independent accumulations issued alternately, so that consecutive MFMAs never wait
    // on each other: Xa += A1 T1 and Xb += A2 T2; a single product A T split over its k range
    // (Xa: k < 8, Xb: k >= 8); and the same for products with a register operand.
    auto mm_acc2 = [&](f32x4& Xa, const float* A1, const float* T1, f32x4& Xb, const float* A2,
                       const float* T2) {
#pragma unroll
      for (int kk2 = 0; kk2 < 4; ++kk2) {
        Xa = mma_f32(A1[ln * L::LDA + 4 * kk2 + q4], T1[(4 * kk2 + q4) * L::LDA + ln], Xa);
        Xb = mma_f32(A2[ln * L::LDA + 4 * kk2 + q4], T2[(4 * kk2 + q4) * L::LDA + ln], Xb);
      }
    };
    auto mm_acc_split = [&](f32x4& Xa, f32x4& Xb, const float* Ab, const float* Tb) {
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        Xa = mma_f32(Ab[ln * L::LDA + 4 * kk2 + q4], Tb[(4 * kk2 + q4) * L::LDA + ln], Xa);
        Xb = mma_f32(Ab[ln * L::LDA + 4 * kk2 + 8 + q4], Tb[(4 * kk2 + 8 + q4) * L::LDA + ln], Xb);
      }
    };
    auto mm_reg2 = [&](f32x4& Ya, const float* T1, f32x4 X1, f32x4& Yb, const float* T2, f32x4 X2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Ya = mma_f32(T1[ln * L::LDA + 4 * q4 + e], X1[e], Ya);
        Yb = mma_f32(T2[ln * L::LDA + 4 * q4 + e], X2[e], Yb);
      }
    };
    auto mm_reg_split = [&](f32x4& Ya, f32x4& Yb, const float* Tb, f32x4 X) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        Ya = mma_f32(Tb[ln * L::LDA + 4 * q4 + e], X[e], Ya);
        Yb = mma_f32(Tb[ln * L::LDA + 4 * q4 + e + 2], X[e + 2], Yb);
      }
    };
    // T_ij = -Y into sA (fp32, for later blocks) and T'_ij = T_ij diag(beta) into sT (hi, lo)
    auto put = [&](int bi, int bj, f32x4 Y) {
      float* To = tblk(bi, bj);
      const float bcol = sBeta[16 * bj + ln];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        To[(4 * q4 + e) * L::LDA + ln] = -Y[e];
        store_split_prod<Pol>(sT, sTLo, (16 * bi + 4 * q4 + e) * L::LDT + 16 * bj + ln, -Y[e],
                              bcol);
      }
    };
    if (w & 1) {
      const int lo = w - 1;   // diagonal pair (lo, lo + 1)
      f32x4 Xa = zero4(), Xb = zero4(), Ya = zero4(), Yb = zero4();
      mm_acc_split(Xa, Xb, ablk(lo + 1, lo), tblk(lo, lo));
      mm_reg_split(Ya, Yb, tblk(lo + 1, lo + 1), Xa + Xb);
      put(lo + 1, lo, Ya + Yb);
    }
    lds_barrier();
    KDA_PREFETCH(kLoadK, 0, 4);
    if constexpr (kOut) KDA_PREFETCH(kLoadQ, 0, 4);
    {
      const int bj = w & 1;          // column block 0 or 1
      const bool row3 = w >= 2;      // row block 2 or 3
      // X_2j, X_3j = A_[2|3],[01] T_[01],j, each accumulated in two halves
      f32x4 X2a = zero4(), X2b = zero4(), X3a = zero4(), X3b = zero4();
      if (bj == 0) {
        mm_acc2(X2a, ablk(2, 0), tblk(0, 0), X2b, ablk(2, 1), tblk(1, 0));
        if (row3) mm_acc2(X3a, ablk(3, 0), tblk(0, 0), X3b, ablk(3, 1), tblk(1, 0));
      } else {
        mm_acc_split(X2a, X2b, ablk(2, 1), tblk(1, 1));
        if (row3) mm_acc_split(X3a, X3b, ablk(3, 1), tblk(1, 1));
      }
      f32x4 Ya = zero4(), Yb = zero4();
      if (!row3) mm_reg_split(Ya, Yb, tblk(2, 2), X2a + X2b);
      else mm_reg2(Ya, tblk(3, 2), X2a + X2b, Yb, tblk(3, 3), X3a + X3b);
      put(row3 ? 3 : 2, bj, Ya + Yb);
    }
    KDA_PREFETCH(kLoadK, 4, 8);
    if constexpr (kOut) KDA_PREFETCH(kLoadQ, 4, 8);
    lds_barrier();


    if constexpr (kPrep) {
      char* slot = p.ws_ops + (size_t(seq_slot0 + (cstart - seq_bos) / kChunk) * H + h) *
                                  OpSlot<DK>::kBytes;
      prep_store<Pol, L, DK>(slot, sKg, sQg, sT, sTLo, sM, sMLo, sKhT, sDecay, w, lane, ln, q4);
      KDA_PREFETCH(kLoadB, 0, 8);
    } else {
      // ================= serial step: this wave's 16 value columns ============================

      // Each product loads a batch of A fragments from LDS first and then issues its MFMAs, so
      // several LDS reads are in flight per wave (one wave per SIMD hides nothing otherwise).
      // S as fp16 B fragments, shared by the two products with decayed keys and queries
      FragR Sr[NS];
  #pragma unroll
      for (int pp = 0; pp < NS; ++pp) Sr[pp] = Pol::from_acc_r(S, pp);
      // X = (K e^Gamma) S - V, in fp32
      // (the values stay packed in the raw registers until here)
      f32x4 X[4];
  #pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        float vx[4];
  #pragma unroll
        for (int e = 0; e < 4; ++e) vx[e] = to_f32(raw.v[rb][e]);
        quad_transpose(vx, lane);   // now token 16 rb + 4 q4 + e, column 16 w + ln
        if (Lc == kChunk && !p_tile) {
  #pragma unroll
          for (int e = 0; e < 4; ++e) X[rb][e] = -vx[e];
        } else {
  #pragma unroll
          for (int e = 0; e < 4; ++e) X[rb][e] = (16 * rb + 4 * q4 + e < Lc && !p_tile) ? -vx[e] : 0.f;
        }
      }
      KDA_PREFETCH(kLoadV | kLoadB, 0, 8);
  #pragma unroll
      for (int pp = 0; pp < NS; ++pp) {
        FragR kg[4];
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb) kg[rb] = Pol::load_r(sKg, L::LDP, 16 * rb + ln, pp, q4);
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb) X[rb] = Pol::mma_r(kg[rb], Sr[pp], X[rb]);
      }
      f32x4 U[4], O[4];
      // O = (Q e^Gamma) S, independent of X: its MFMAs cover the latency of the X products
  #pragma unroll
      for (int pp = 0; pp < NS; ++pp) {
        if constexpr (!kOut) break;
        FragR qg[4];
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb) qg[rb] = Pol::load_r(sQg, L::LDP, 16 * rb + ln, pp, q4);
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb) O[rb] = Pol::mma_r(qg[rb], Sr[pp], pp == 0 ? zero4() : O[rb]);
      }
      // U = T' (V - K_Gamma S) = -T' X
      Frag Xh[NT], Xl[NT];
  #pragma unroll
      for (int pp = 0; pp < NT; ++pp) Pol::from_acc_split(X, pp, Xh[pp], Xl[pp]);
  #pragma unroll
      for (int pp = 0; pp < NT; ++pp) {
        Frag th[4], tl[4];
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (pp < Pol::slices_blocks(rb + 1)) {
            th[rb] = Pol::load(sT, L::LDT, 16 * rb + ln, pp, q4);
            if constexpr (Pol::kSplit) tl[rb] = Pol::load(sTLo, L::LDT, 16 * rb + ln, pp, q4);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          if (pp < Pol::slices_blocks(rb + 1)) U[rb] = Pol::mma(th[rb], Xh[pp], pp == 0 ? zero4() : U[rb]);
        if constexpr (Pol::kSplit) {
  #pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            if (pp < Pol::slices_blocks(rb + 1)) U[rb] = Pol::mma(tl[rb], Xh[pp], U[rb]);
  #pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            if (pp < Pol::slices_blocks(rb + 1)) U[rb] = Pol::mma(th[rb], Xl[pp], U[rb]);
        }
      }
  #pragma unroll
      for (int rb = 0; rb < 4; ++rb) U[rb] = -U[rb];
      // O += M U and S += K^T U with fp16 operands: U as an fp16 hi + lo pair, M as one too,
      // K e^{Gamma_L - Gamma} (at most 1) as a single fp16
      FragR Uh[NT], Ul[NT];
  #pragma unroll
      for (int pp = 0; pp < NT; ++pp) Pol::from_acc_split_r(U, pp, Uh[pp], Ul[pp]);
  #pragma unroll
      for (int pp = 0; pp < NT; ++pp) {
        if constexpr (!kOut) break;
        FragR mh[4], ml[4];
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (pp < Pol::slices_blocks(rb + 1)) {
            mh[rb] = Pol::load_r(sM, L::LDT, 16 * rb + ln, pp, q4);
            if constexpr (Pol::kSplit) ml[rb] = Pol::load_r(sMLo, L::LDT, 16 * rb + ln, pp, q4);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          if (pp < Pol::slices_blocks(rb + 1)) O[rb] = Pol::mma_r(mh[rb], Uh[pp], O[rb]);
        if constexpr (Pol::kSplit) {
  #pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            if (pp < Pol::slices_blocks(rb + 1)) O[rb] = Pol::mma_r(ml[rb], Uh[pp], O[rb]);
  #pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            if (pp < Pol::slices_blocks(rb + 1)) O[rb] = Pol::mma_r(mh[rb], Ul[pp], O[rb]);
        }
      }
      // S <- diag(e^{Gamma_L}) S + (K e^{Gamma_L - Gamma})^T U
  #pragma unroll
      for (int t = 0; t < NTD; ++t) {
  #pragma unroll
        for (int e = 0; e < 4; ++e) S[t][e] *= sDecay[16 * t + 4 * q4 + e];
      }
  #pragma unroll
      for (int pp = 0; pp < NT; ++pp) {
  #pragma unroll
        for (int t0 = 0; t0 < NTD; t0 += 4) {
          FragR kh[4];
  #pragma unroll
          for (int t = 0; t < 4; ++t) kh[t] = Pol::load_r(sKhT, L::LDT, 16 * (t0 + t) + ln, pp, q4);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int t = 0; t < 4; ++t) S[t0 + t] = Pol::mma_r(kh[t], Uh[pp], S[t0 + t]);
          if constexpr (Pol::kSplit) {
  #pragma unroll
            for (int t = 0; t < 4; ++t) S[t0 + t] = Pol::mma_r(kh[t], Ul[pp], S[t0 + t]);
          }
        }
      }
      // output, after the state update so that the last O products complete under it: a quad
      // transpose gives each lane four consecutive columns of token 16 rb + 4 q4 + lane % 4
      if constexpr (kOut) {
        const int tq = 4 * q4 + (ln & 3);
        const uint32_t lo_el = uint32_t((tq * H + h) * DV + col0 + 4 * (ln >> 2));
  #pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          float ox[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) ox[e] = p.scale * O[rb][e];
          quad_transpose(ox, lane);
          Tout* row = go + size_t(cstart + 16 * rb) * H * DV;
          if (16 * rb + tq < Lc) {
            if constexpr (sizeof(Tout) == 2)
              *reinterpret_cast<bf16x4*>(row + lo_el) =
                  bf16x4{(__bf16)ox[0], (__bf16)ox[1], (__bf16)ox[2], (__bf16)ox[3]};
            else
              *reinterpret_cast<f32x4*>(row + lo_el) = f32x4{ox[0], ox[1], ox[2], ox[3]};
          }
        }
      }
    }
    if constexpr (!kPrep)
      if (mode == kModeForward)
        write_checkpoint<DK, NTD>(p, S, seq_bos, cstart + Lc, Lc, h, col0, q4, ln);
    lds_barrier();
#undef KDA_PREFETCH
  }

  if constexpr (kPrep) return;
  float* s_out = nullptr;
  if (mode == kModeForward && p.ht) s_out = p.ht + (size_t(n) * H + h) * DK * DV;
  if (mode == kModeTransition) s_out = p.ws_pq + (size_t(sj) * H + h) * DK * ldS;
  if (s_out) {
#pragma unroll
    for (int t = 0; t < NTD; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * t + 4 * q4 + e;
        s_out[size_t(c) * ldS + col0 + ln] = S[t][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Pass 1 of the two-launch prefill for bf16 inputs: each chunk's prologue, stored to its operand
// slot. The arithmetic is chunk_fwd_kernel's prologue operation for operation, per key channel
// and per product accumulator, so the slot holds the same bits as the operands that kernel
// computes for its serial step. What differs is where the data lives:
//  * channels go in passes of 64: in pass h a thread takes channels 64 h + CPT l .. + CPT - 1
//    (l = lane % (d_k / 4), CPT = 2 at d_k = 128, 4 at 64) of the same tokens as there, so
//    each channel's decay products see the same operations in the same order; the prologue
//    tiles hold 64 channels and A and M accumulate over the passes;
//  * the serial step's operands go from registers straight to the slot: Q e^Gamma, K e^Gamma
//    and (K e^{Gamma_L - Gamma})^T per pass, M from its accumulators, T diag(beta) from the
//    fp32 inverse once complete; no LDS holds them.
// LDS: six 64-channel tiles, the fp32 A / T matrix and small vectors, 72 KB: two workgroups
// per compute unit, so one workgroup's loads and stores run under the other's products.
template <int DK>
struct PrepLayout {
  static constexpr int PW = 64;              // channels per pass
  static constexpr int LDP = PW + 4;         // tile row stride: 2 dwords modulo 32 banks
  static constexpr int LDA = 64 + 4;         // fp32 A / T working matrix
  static constexpr size_t tP = size_t(64) * LDP * 2;
  static constexpr size_t oQr = 0;
  static constexpr size_t oQrLo = oQr + tP;
  static constexpr size_t oKd = oQrLo + tP;
  static constexpr size_t oKdLo = oKd + tP;
  static constexpr size_t oKr = oKdLo + tP;
  static constexpr size_t oKc = oKr + tP;
  static constexpr size_t oA = oKc + tP;
  static constexpr size_t oBeta = oA + size_t(64) * LDA * 4;   // two chunks' betas
  static constexpr size_t oBP = oBeta + 2 * 64 * 4;             // [4][DK] sub-block decays
  static constexpr size_t oDecay = oBP + 4 * DK * 4;            // [DK] whole-chunk decay
  static constexpr size_t kBytes = oDecay + DK * 4;
  static_assert(2 * kBytes <= 160 * 1024, "two workgroups per compute unit");
};

// Products of one channel pass for wave IA: row block IA of A and row block IM = 3 - IA of M
// (M block (3, 0) on wave 3, as in am_rows), over the pass's two k-slices (global slices
// 2 h and 2 h + 1), into accumulators kept across the passes. Same loads and MFMAs, in the same
// order per accumulator, as am_rows in forward mode.
template <int DK, int IA>
__device__ __forceinline__ void prep_am_pass(const __bf16* sKr, const __bf16* sKd,
                                             const __bf16* sKdLo, const __bf16* sKc,
                                             const __bf16* sQr, const __bf16* sQrLo,
                                             const float* sBP, int hp, f32x4 (&accA)[4],
                                             f32x4 (&accM)[4], f32x4& accM30, int ln, int q4) {
  using Pol = PolBF16;
  using Frag = Pol::Frag;
  using L = PrepLayout<DK>;
  constexpr int IM = 3 - IA;
  constexpr bool kM30 = IA == 3;
  constexpr int kMJ0 = IM == 3 ? 1 : 0;
  const float* P1 = sBP + DK;
  const float* P2 = sBP + 2 * DK;
  // (one slice at a time: the fragments of both slices at once do not fit the registers of
  // two waves per SIMD)
#pragma unroll 1
  for (int pl = 0; pl < 2; ++pl) {
    const int pp = 2 * hp + pl;   // global k-slice (factor columns); pl indexes the tiles
    const Frag rowA = Pol::load(sKr, L::LDP, 16 * IA + ln, pl, q4);
    Frag rowM, colA[4], colM[4], colMl[4], dKl, dQl, rowM3, dQl3, colM30, colM30l;
    rowM = Pol::load(sQr, L::LDP, 16 * IM + ln, pl, q4);
    if constexpr (kM30) {
      const float* const fac[3] = {sBP, sBP + DK, sBP + 2 * DK};
      rowM3 = Pol::load(sQr, L::LDP, 48 + ln, pl, q4);
      dQl3 = Pol::load(sQrLo, L::LDP, 48 + ln, pl, q4);
      Pol::template load_pair_scaled_at<3>(sKd, sKdLo, L::LDP, ln, pl, pp, q4, fac, colM30, colM30l);
    }
#pragma unroll
    for (int jb = 0; jb <= IA; ++jb) {
      if (jb == IA) colA[jb] = Pol::load(sKd, L::LDP, 16 * jb + ln, pl, q4);
      else if (jb == IA - 1) colA[jb] = Pol::load(sKc, L::LDP, 16 * jb + ln, pl, q4);
      else if (jb == 0 && IA == 3) colA[jb] = Pol::load_scaled2_at(sKc, L::LDP, ln, pl, pp, q4, P1, P2);
      else colA[jb] = Pol::load_scaled_at(sKc, L::LDP, 16 * jb + ln, pl, pp, q4, jb == 0 ? P1 : P2);
    }
#pragma unroll
    for (int jb = kMJ0; jb <= IM; ++jb) {
      if (jb == IM) {
        colM[jb] = Pol::load(sKd, L::LDP, 16 * jb + ln, pl, q4);
      } else {
        const float* const fac[3] = {sBP + jb * DK, sBP + (jb + 1) * DK, sBP + (jb + 2) * DK};
        if (IM - jb == 1)
          Pol::template load_pair_scaled_at<1>(sKd, sKdLo, L::LDP, 16 * jb + ln, pl, pp, q4, fac, colM[jb], colMl[jb]);
        else if (IM - jb == 2)
          Pol::template load_pair_scaled_at<2>(sKd, sKdLo, L::LDP, 16 * jb + ln, pl, pp, q4, fac, colM[jb], colMl[jb]);
        else
          Pol::template load_pair_scaled_at<3>(sKd, sKdLo, L::LDP, 16 * jb + ln, pl, pp, q4, fac, colM[jb], colMl[jb]);
      }
    }
    dKl = Pol::load(sKdLo, L::LDP, 16 * IM + ln, pl, q4);
    dQl = Pol::load(sQrLo, L::LDP, 16 * IM + ln, pl, q4);
#pragma unroll
    for (int jb = 0; jb <= IA; ++jb) accA[jb] = Pol::mma(colA[jb], rowA, accA[jb]);
#pragma unroll
    for (int jb = kMJ0; jb <= IM; ++jb) accM[jb] = Pol::mma(colM[jb], rowM, accM[jb]);
    if constexpr (kM30) accM30 = Pol::mma(colM30, rowM3, accM30);
    accM[IM] = Pol::mma(dKl, rowM, accM[IM]);
#pragma unroll
    for (int jb = kMJ0; jb < IM; ++jb) accM[jb] = Pol::mma(colMl[jb], rowM, accM[jb]);
    if constexpr (kM30) accM30 = Pol::mma(colM30l, rowM3, accM30);
#pragma unroll
    for (int jb = kMJ0; jb <= IM; ++jb) accM[jb] = Pol::mma(colM[jb], dQl, accM[jb]);
    if constexpr (kM30) accM30 = Pol::mma(colM30, dQl3, accM30);
  }
}

// After the passes: A's row block into the fp32 matrix, M's blocks straight to the slot (fp16
// hi and lo fragments; zeros for the strictly upper block sharing a fragment with the
// diagonal one), and the diagonal block of T = (I + A)^{-1} by the same fp32 substitution as
// am_rows (T diag(beta) is formed later, from the fp32 matrix).
template <int DK, int IA>
__device__ __forceinline__ void prep_am_finish(const f32x4 (&accA)[4], const f32x4 (&accM)[4],
                                               const f32x4& accM30, const float* sBeta,
                                               float* sA, char* slot, int ln, int q4) {
  using L = PrepLayout<DK>;
  using OS = OpSlot<DK>;
  constexpr int IM = 3 - IA;
  constexpr bool kM30 = IA == 3;
  constexpr int kMJ0 = IM == 3 ? 1 : 0;
  const int lane = 16 * q4 + ln;
  const int ra = 16 * IA + ln, rm = 16 * IM + ln;
  const float br = sBeta[ra];
#pragma unroll
  for (int jb = 0; jb <= IA; ++jb) {
    f32x4 outv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * jb + 4 * q4 + e;
      outv[e] = (jb == IA && s >= ra) ? 0.f : br * accA[jb][e];
    }
    *reinterpret_cast<f32x4*>(sA + ra * L::LDA + 16 * jb + 4 * q4) = outv;
  }
  // M block (row block i, column block jb): register e is column 16 jb + 4 q4 + e of row
  // 16 i + ln, i.e. half jb % 2 of this lane's 16 bytes in fragment (i, jb / 2)
  auto put_m = [&](int i, int jb, f32x4 x) {
    f16x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 h = (_Float16)x[e];
      hi[e] = h;
      lo[e] = (_Float16)(x[e] - float(h));
    }
    const int f = OS::tri(i, jb / 2);
    char* dst = slot + lane * 16 + (jb & 1) * 8;
    *reinterpret_cast<f16x4*>(dst + size_t(OS::fM + f) * 1024) = hi;
    *reinterpret_cast<f16x4*>(dst + size_t(OS::fMLo + f) * 1024) = lo;
  };
#pragma unroll
  for (int jb = kMJ0; jb <= IM; ++jb) {
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * jb + 4 * q4 + e;
      x[e] = (jb == IM && s > rm) ? 0.f : accM[jb][e];
    }
    put_m(IM, jb, x);
  }
  if constexpr (IM % 2 == 0) put_m(IM, IM + 1, zero4());   // strictly upper, same fragment
  if constexpr (kM30) put_m(3, 0, accM30);
  // diagonal block IA of T, as in am_rows
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  {
    const int jc = lane >> 2, pp = lane & 3;
    const float* Ab = sA + 16 * IA * L::LDA + 16 * IA;
    f32x4 arow[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        arow[i][m] = *reinterpret_cast<const f32x4*>(Ab + (pp + 4 * i) * L::LDA + 4 * m);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (pp + 4 * i == jc) ? 1.f : 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 15; ++s2) {
      float xs;
      switch (s2 & 3) {
        case 0: xs = quad_bcast<0>(x[s2 >> 2]); break;
        case 1: xs = quad_bcast<1>(x[s2 >> 2]); break;
        case 2: xs = quad_bcast<2>(x[s2 >> 2]); break;
        default: xs = quad_bcast<3>(x[s2 >> 2]); break;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = fmaf(-arow[i][s2 >> 2][s2 & 3], xs, x[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sA[(16 * IA + pp + 4 * i) * L::LDA + 16 * IA + jc] = x[i];
  }
}

// A 32-bit word moved from lane l ^ 1 (quad_perm), l ^ 8 (row rotation by eight) or l ^ 4
// (swizzle) of the wave.
__device__ __forceinline__ uint32_t word_xor1(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), kQuadXor1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t word_xor8(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t word_xor4(uint32_t x) {
  return uint32_t(__builtin_amdgcn_ds_swizzle(int(x), 0x101F));   // and 0x1f, xor 4
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}

// The prep pass's Q e^Gamma and K e^Gamma of one channel pass (products qv fs, kv fs rounded
// to fp16 as before, then exchanged, not recomputed) written as whole 16-byte lane rows of
// their fragments. Thread (grp, li) holds channels c0 .. c0 + CPT - 1 of tokens rb0 .. rb0 +
// TPT - 1. With CPT = 2 the partner l ^ 1 holds channels c0 ^ 2 and l ^ 8 channels c0 ^ 16;
// with CPT = 4 the partner l ^ 4 holds channels c0 ^ 16.
template <int DK, int CPT, int TPT>
__device__ __forceinline__ void store_qk_rows(const float (&qv)[TPT][CPT],
                                              const float (&kv)[TPT][CPT], const float (&fs)[CPT],
                                              char* fq, char* fk, int w, int li, int rb0, int c0,
                                              int lane) {
  constexpr int NS = DK / 32;
  static_assert((CPT == 2 && TPT == 8) || (CPT == 4 && TPT == 4), "prep thread map");
  // u[m][t][j]: word j (channels 2 j, 2 j + 1 of the thread) of token t, matrix m (q, k)
  uint32_t u[2][TPT][CPT / 2];
#pragma unroll
  for (int t = 0; t < TPT; ++t)
#pragma unroll
    for (int j = 0; j < CPT / 2; ++j) {
      u[0][t][j] = pack_f16x2(qv[t][2 * j] * fs[2 * j], qv[t][2 * j + 1] * fs[2 * j + 1]);
      u[1][t][j] = pack_f16x2(kv[t][2 * j] * fs[2 * j], kv[t][2 * j + 1] * fs[2 * j + 1]);
    }
  // p[m][i]: channels 4 q .. 4 q + 3 (two words) of token tok1(i), four of them
  uint32_t pw[2][4][2];
  int tok1_base;
  if constexpr (CPT == 2) {
    // lanes l and l ^ 1: the even one keeps tokens 0..3 and takes its partner's words of
    // them, the odd one keeps tokens 4..7
    const bool odd = (lane & 1) != 0;
    tok1_base = odd ? 4 : 0;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t r = word_xor1(odd ? u[m][i][0] : u[m][4 + i][0]);
        pw[m][i][0] = odd ? r : u[m][i][0];
        pw[m][i][1] = odd ? u[m][4 + i][0] : r;
      }
  } else {
    tok1_base = 0;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[m][i][0] = u[m][i][0];
        pw[m][i][1] = u[m][i][CPT / 2 - 1];
      }
  }
  // lanes holding channel groups 4 q and 16 + 4 q: the lower keeps tokens 0, 1 of its four,
  // the upper tokens 2, 3; each ends with two 16-byte rows
  const bool up = CPT == 2 ? (lane & 8) != 0 : (lane & 4) != 0;
  const int q = CPT == 2 ? (li % 8) / 2 : li % 4;
  const int slice = c0 / 32;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tt = tok1_base + (up ? 2 : 0) + i;
    const int r = rb0 + tt;
    char* dq = fq + size_t(w * NS + slice) * 1024 + size_t(16 * q + r % 16) * 16;
    char* dk = fk + size_t(w * NS + slice) * 1024 + size_t(16 * q + r % 16) * 16;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint32_t r0, r1;
      if constexpr (CPT == 2) {
        r0 = word_xor8(up ? pw[m][i][0] : pw[m][2 + i][0]);
        r1 = word_xor8(up ? pw[m][i][1] : pw[m][2 + i][1]);
      } else {
        r0 = word_xor4(up ? pw[m][i][0] : pw[m][2 + i][0]);
        r1 = word_xor4(up ? pw[m][i][1] : pw[m][2 + i][1]);
      }
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 row = up ? u32x4{r0, r1, pw[m][2 + i][0], pw[m][2 + i][1]}
                           : u32x4{pw[m][i][0], pw[m][i][1], r0, r1};
      *reinterpret_cast<u32x4*>(m == 0 ? dq : dk) = row;
    }
  }
}

template <int DK>
__global__ __launch_bounds__(256, 2) void chunk_prep_kernel(ChunkParams p) {
  using L = PrepLayout<DK>;
  using OS = OpSlot<DK>;
  using PM = ProMap<DK>;
  constexpr int TPT = PM::kTPT;          // tokens per thread
  constexpr int NPASS = DK / 64;         // channel passes
  constexpr int CPT = 4 / NPASS;         // channels per thread and pass
  using GV = float __attribute__((ext_vector_type(CPT)));
  using BV = __bf16 __attribute__((ext_vector_type(CPT)));

  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  __bf16* sQr = reinterpret_cast<__bf16*>(smem + L::oQr);
  __bf16* sQrLo = reinterpret_cast<__bf16*>(smem + L::oQrLo);
  __bf16* sKd = reinterpret_cast<__bf16*>(smem + L::oKd);
  __bf16* sKdLo = reinterpret_cast<__bf16*>(smem + L::oKdLo);
  __bf16* sKr = reinterpret_cast<__bf16*>(smem + L::oKr);
  __bf16* sKc = reinterpret_cast<__bf16*>(smem + L::oKc);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  float* sBetaAll = reinterpret_cast<float*>(smem + L::oBeta);
  float* sBP = reinterpret_cast<float*>(smem + L::oBP);
  float* sDecay = reinterpret_cast<float*>(smem + L::oDecay);

  int sub;
  const int unit = block_unit(blockIdx.x, 1, &sub);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int h = unit % H;
  const int sj = unit / H;
  const int n = p.seq0 + sj / p.n_seg;
  const int j = sj % p.n_seg;
  int bos, eos;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
  } else {
    bos = n * p.seq_len;
    eos = bos + p.seq_len;
  }
  const long long seq_slot0 = seq_first_slot(bos, p.slot_tok0, n, p.seq0);
  const int seq_bos = bos;
  {
    int c_lo;
    segment_range(seq_bos, eos, j, p.n_seg, &bos, &eos, &c_lo);
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int q4 = lane >> 4;
  const int ln = lane & 15;
  const int grp = lane / PM::kLPT;
  const int li = lane % PM::kLPT;
  const int rb0 = 16 * w + grp * TPT;          // first token row of this thread
  const float gmin2 = p.g_min * kLog2e;
  const __bf16* gq = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* gk = reinterpret_cast<const __bf16*>(p.k);

  int cnum = 0;
  for (int cstart = bos; cstart < eos; cstart += kChunk, ++cnum) {
    const int Lc = min(kChunk, eos - cstart);
    float* sBeta = sBetaAll + 64 * (cnum & 1);
    char* slot = p.ws_ops + (size_t(seq_slot0 + (cstart - seq_bos) / kChunk) * H + h) * OS::kBytes;
    float beta_r;
    {
      const int bl = lane & 15;
      const int r = 16 * w + bl;
      beta_r = p.beta[size_t(r < Lc ? cstart + r : cstart) * H + h];
      beta_r = r < Lc ? beta_r : 0.f;
    }
    if (lane < 16) sBeta[16 * w + lane] = beta_r;

    f32x4 accA[4], accM[4], accM30 = zero4();
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      accA[jb] = zero4();
      accM[jb] = zero4();
    }
#pragma unroll
    for (int hp = 0; hp < NPASS; ++hp) {
      const int c0 = 64 * hp + CPT * li;   // first channel of the thread in this pass
      const int tc0 = CPT * li;            // its column in the 64-channel tiles
      // ---- this pass's inputs (rows past a ragged chunk's end read its first row; their
      //      values are masked below)
      GV gin[TPT];
      BV kin[TPT], qin[TPT];
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const int r = rb0 + t;
        const size_t row = (size_t(r < Lc ? cstart + r : cstart) * H + h) * DK + c0;
        gin[t] = *reinterpret_cast<const GV*>(p.g + row);
        kin[t] = *reinterpret_cast<const BV*>(gk + row);
        qin[t] = *reinterpret_cast<const BV*>(gq + row);
      }
      // ---- decay factors, as in chunk_fwd_kernel's prologue, per channel
      float rho[TPT][CPT], qv[TPT][CPT], kv[TPT][CPT], ex[TPT][CPT];
      float lp[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) lp[c] = 1.f;
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const bool valid = rb0 + t < Lc;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const float gt = valid ? fmaxf(gin[t][c] * kLog2e, gmin2) : 0.f;
          ex[t][c] = __builtin_amdgcn_exp2f(gt);
          kv[t][c] = valid ? (float)kin[t][c] : 0.f;
          qv[t][c] = valid ? (float)qin[t][c] : 0.f;
          lp[c] *= ex[t][c];
          rho[t][c] = lp[c];
        }
      }
      float bp[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        float pre;
        if constexpr (PM::kNG == 2) {
          const float o = __shfl_xor(lp[c], 32);
          pre = grp ? o : 1.f;
          bp[c] = lp[c] * o;
        } else {
          static_assert(PM::kNG == 4, "token groups per sub-block");
          const float a = __shfl_xor(lp[c], 16);
          const float pair = lp[c] * a;
          const float b2 = __shfl_xor(pair, 32);
          pre = ((grp & 2) ? b2 : 1.f) * ((grp & 1) ? a : 1.f);
          bp[c] = pair * b2;
        }
#pragma unroll
        for (int t = 0; t < TPT; ++t) rho[t][c] *= pre;
      }
      float rinv_next[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) rinv_next[c] = __builtin_amdgcn_rcpf(rho[TPT - 1][c]);
#pragma unroll
      for (int t = TPT - 1; t >= 0; --t) {
        BV qh, ql, dh, dl, kr, kc;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const float rh = rho[t][c];
          const float rinv = rinv_next[c];
          if (t > 0) rinv_next[c] = rinv * ex[t][c];
          const float k0 = kv[t][c];
          const float xq = qv[t][c] * rh;
          const float xkd = k0 * rinv;
          const float xkr = k0 * rh;
          const float xkc = xkd * bp[c];
          qv[t][c] = xq;
          kv[t][c] = xkr;
          rho[t][c] = xkc;
          qh[c] = (__bf16)xq;
          ql[c] = (__bf16)(xq - (float)qh[c]);
          dh[c] = (__bf16)xkd;
          dl[c] = (__bf16)(xkd - (float)dh[c]);
          kr[c] = (__bf16)xkr;
          kc[c] = (__bf16)xkc;
        }
        const int idx = (rb0 + t) * L::LDP + tc0;
        *reinterpret_cast<BV*>(sQr + idx) = qh;
        *reinterpret_cast<BV*>(sQrLo + idx) = ql;
        *reinterpret_cast<BV*>(sKd + idx) = dh;
        *reinterpret_cast<BV*>(sKdLo + idx) = dl;
        *reinterpret_cast<BV*>(sKr + idx) = kr;
        *reinterpret_cast<BV*>(sKc + idx) = kc;
      }
      if (grp == 0) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) sBP[w * DK + c0 + c] = bp[c];
      }
      lds_barrier();
      // ---- this pass's recurrence operands, straight to the slot: Q e^Gamma and K e^Gamma
      //      (token rows, fragment (w, channel / 32)) and (K e^{Gamma_L - Gamma})^T (channel
      //      rows, fragment (channel / 16, token / 32)), fp16
      {
        float fs[CPT], fe[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          float pb[4];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) pb[bb] = sBP[bb * DK + c0 + c];
          fs[c] = 1.f;
          fe[c] = 1.f;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            if (bb < w) fs[c] *= pb[bb];
            if (bb > w) fe[c] *= pb[bb];
          }
          if (w == 0 && grp == 0) sDecay[c0 + c] = pb[0] * pb[1] * pb[2] * pb[3];
        }
        // Channel c0 of token row r sits in lane 16 ((c0 % 16) / 4) + r % 16 of fragment
        // (r / 16, c0 / 32), bytes from 8 ((c0 % 32) / 16) + 2 (c0 % 4): a lane's 16 bytes are
        // channels 4 q .. 4 q + 3 and 16 + 4 q .. 16 + 4 q + 3 of one token, held here by two
        // (d_k = 64) or four (d_k = 128) threads. They swap fp16 words across lanes (DPP, or
        // a swizzle for the lane distance 4) until each holds whole 16-byte rows of two tokens,
        // so both operands leave with two 16-byte stores a thread instead of one store per
        // token (the vector-memory queue takes one instruction per 64 lanes whatever its width).
        store_qk_rows<DK, CPT, TPT>(qv, kv, fs, slot + size_t(OS::fQg) * 1024,
                                    slot + size_t(OS::fKg) * 1024, w, li, rb0, c0, lane);
        // channel row c0 + c, tokens rb0 + t4 .. + 3: lane 16 ((token % 16) / 4) + channel % 16
        // of fragment (channel / 16, token / 32), bytes from 8 ((token % 32) / 16)
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int ch = c0 + c;
#pragma unroll
          for (int t4 = 0; t4 < TPT; t4 += 4) {
            const int r = rb0 + t4;
            f16x4 col;
#pragma unroll
            for (int e = 0; e < 4; ++e) col[e] = (_Float16)(rho[t4 + e][c] * fe[c]);
            const size_t o = size_t(OS::fKh + 2 * (ch / 16) + r / 32) * 1024 +
                             size_t(16 * ((r % 16) / 4) + ch % 16) * 16 + ((r % 32) / 16) * 8;
            *reinterpret_cast<f16x4*>(slot + o) = col;
          }
        }
      }
      // ---- A and M products over this pass's two k-slices
      switch (w) {
        case 0: prep_am_pass<DK, 0>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, hp, accA, accM, accM30, ln, q4); break;
        case 1: prep_am_pass<DK, 1>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, hp, accA, accM, accM30, ln, q4); break;
        case 2: prep_am_pass<DK, 2>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, hp, accA, accM, accM30, ln, q4); break;
        default: prep_am_pass<DK, 3>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sBP, hp, accA, accM, accM30, ln, q4); break;
      }
      lds_barrier();   // the tiles are rewritten by the next pass (or the next chunk)
    }
    // ---- A's row blocks, M to the slot, diagonal blocks of T
    switch (w) {
      case 0: prep_am_finish<DK, 0>(accA, accM, accM30, sBeta, sA, slot, ln, q4); break;
      case 1: prep_am_finish<DK, 1>(accA, accM, accM30, sBeta, sA, slot, ln, q4); break;
      case 2: prep_am_finish<DK, 2>(accA, accM, accM30, sBeta, sA, slot, ln, q4); break;
      default: prep_am_finish<DK, 3>(accA, accM, accM30, sBeta, sA, slot, ln, q4); break;
    }
    lds_barrier();
    // ---- off-diagonal blocks of T, as in chunk_fwd_kernel (level 1 on waves 1 and 3, then
    //      one level-2 block per wave); T_ij (i > j) in the free upper position (j, i)
    auto tblk = [&](int bi, int bj) -> float* {
      return bi == bj ? sA + 16 * bi * L::LDA + 16 * bi : sA + 16 * bj * L::LDA + 16 * bi;
    };
    auto ablk = [&](int bi, int bj) -> const float* { return sA + 16 * bi * L::LDA + 16 * bj; };
    auto mm_acc2 = [&](f32x4& Xa, const float* A1, const float* T1, f32x4& Xb, const float* A2,
                       const float* T2) {
#pragma unroll
      for (int kk2 = 0; kk2 < 4; ++kk2) {
        Xa = mma_f32(A1[ln * L::LDA + 4 * kk2 + q4], T1[(4 * kk2 + q4) * L::LDA + ln], Xa);
        Xb = mma_f32(A2[ln * L::LDA + 4 * kk2 + q4], T2[(4 * kk2 + q4) * L::LDA + ln], Xb);
      }
    };
    auto mm_acc_split = [&](f32x4& Xa, f32x4& Xb, const float* Ab, const float* Tb) {
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        Xa = mma_f32(Ab[ln * L::LDA + 4 * kk2 + q4], Tb[(4 * kk2 + q4) * L::LDA + ln], Xa);
        Xb = mma_f32(Ab[ln * L::LDA + 4 * kk2 + 8 + q4], Tb[(4 * kk2 + 8 + q4) * L::LDA + ln], Xb);
      }
    };
    auto mm_reg2 = [&](f32x4& Ya, const float* T1, f32x4 X1, f32x4& Yb, const float* T2, f32x4 X2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Ya = mma_f32(T1[ln * L::LDA + 4 * q4 + e], X1[e], Ya);
        Yb = mma_f32(T2[ln * L::LDA + 4 * q4 + e], X2[e], Yb);
      }
    };
    auto mm_reg_split = [&](f32x4& Ya, f32x4& Yb, const float* Tb, f32x4 X) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        Ya = mma_f32(Tb[ln * L::LDA + 4 * q4 + e], X[e], Ya);
        Yb = mma_f32(Tb[ln * L::LDA + 4 * q4 + e + 2], X[e + 2], Yb);
      }
    };
    auto put = [&](int bi, int bj, f32x4 Y) {
      float* To = tblk(bi, bj);
#pragma unroll
      for (int e = 0; e < 4; ++e) To[(4 * q4 + e) * L::LDA + ln] = -Y[e];
    };
    if (w & 1) {
      const int lo = w - 1;
      f32x4 Xa = zero4(), Xb = zero4(), Ya = zero4(), Yb = zero4();
      mm_acc_split(Xa, Xb, ablk(lo + 1, lo), tblk(lo, lo));
      mm_reg_split(Ya, Yb, tblk(lo + 1, lo + 1), Xa + Xb);
      put(lo + 1, lo, Ya + Yb);
    }
    lds_barrier();
    {
      const int bj = w & 1;
      const bool row3 = w >= 2;
      f32x4 X2a = zero4(), X2b = zero4(), X3a = zero4(), X3b = zero4();
      if (bj == 0) {
        mm_acc2(X2a, ablk(2, 0), tblk(0, 0), X2b, ablk(2, 1), tblk(1, 0));
        if (row3) mm_acc2(X3a, ablk(3, 0), tblk(0, 0), X3b, ablk(3, 1), tblk(1, 0));
      } else {
        mm_acc_split(X2a, X2b, ablk(2, 1), tblk(1, 1));
        if (row3) mm_acc_split(X3a, X3b, ablk(3, 1), tblk(1, 1));
      }
      f32x4 Ya = zero4(), Yb = zero4();
      if (!row3) mm_reg_split(Ya, Yb, tblk(2, 2), X2a + X2b);
      else mm_reg2(Ya, tblk(3, 2), X2a + X2b, Yb, tblk(3, 3), X3a + X3b);
      put(row3 ? 3 : 2, bj, Ya + Yb);
    }
    lds_barrier();
    // ---- T diag(beta) (bf16 hi and lo) of the 6 lower fragments, from the fp32 matrix: lane
    //      (q4, ln) holds row 16 rb + ln, columns 32 pp + 16 hh + 4 q4 + e; and the decay
    for (int i = w; i < 6; i += 4) {
      const int rb = i < 2 ? i : (i < 4 ? 2 : 3), pp = i < 2 ? 0 : (i & 1);
      const int r = 16 * rb + ln;
      bf16x8 hi, lo;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int c = 32 * pp + 16 * (e8 >> 2) + 4 * q4 + (e8 & 3);
        const int cb = c >> 4;
        float t;
        if (cb > rb) t = 0.f;
        else if (cb == rb) t = sA[r * L::LDA + c];
        else t = sA[(16 * cb + ln) * L::LDA + 16 * rb + (c & 15)];
        __bf16 h, l;
        split_prod_bf16(t, sBeta[c], h, l);   // as store_split_prod
        hi[e8] = h;
        lo[e8] = l;
      }
      __builtin_nontemporal_store(hi, reinterpret_cast<bf16x8*>(slot + size_t(OS::fT + i) * 1024 + lane * 16));
      __builtin_nontemporal_store(lo, reinterpret_cast<bf16x8*>(slot + size_t(OS::fTLo + i) * 1024 + lane * 16));
    }
    if (w == 0 && lane < DK / 4)
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(sDecay + 4 * lane),
                                  reinterpret_cast<f32x4*>(slot + size_t(OS::kDecay) * 1024 + lane * 16));
  }
}

template <class Pol, typename Tio, typename Tout, int DK>
static hipError_t launch_one(const ChunkParams& p, hipStream_t stream) {
  const int groups = (p.n_units + 7) / 8;
  const dim3 grid(groups * 8 * p.n_vt);
  if (p.mode == kModeTransition)
    hipLaunchKernelGGL((chunk_fwd_kernel<Pol, Tio, Tout, DK, false>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((chunk_fwd_kernel<Pol, Tio, Tout, DK, true>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(const ChunkParams& base, int prep_groups, int dk,
                             hipStream_t stream, bool raw) {
  if (!base.ws_ops || !base.q || !base.k || !base.g || !base.beta || base.H < 1 ||
      base.n_seqs < 1 || prep_groups < 1 || (!base.cu_seqlens && base.seq_len < 0))
    return hipErrorInvalidValue;
  if (op_slot_bytes(dk) != (dk == 128 ? OpSlot<128>::kBytes : OpSlot<64>::kBytes))
    return hipErrorInvalidValue;
  ChunkParams prep = base;
  prep.mode = kModePrep;
  prep.n_seg = prep_groups;
  prep.n_vt = 1;
  prep.n_units = base.n_seqs * prep_groups * base.H;
  prep.o = nullptr;
  prep.ht = nullptr;
  prep.h0 = nullptr;
  prep.ws_pq = nullptr;
  prep.ws_sin = nullptr;
  prep.ckpt = nullptr;
  const dim3 grid((prep.n_units + 7) / 8 * 8);
  if (raw && (!base.conv_w || !base.v || !base.v_conv || base.conv_width < 1 ||
              base.conv_width > 4 || base.dv != dk))
    return hipErrorInvalidValue;
  if (dk == 128 && raw)
    hipLaunchKernelGGL((chunk_fwd_kernel<PolBF16, __bf16, float, 128, true, true, true>), grid,
                       dim3(256), 0, stream, prep);
  else if (dk == 128)
    hipLaunchKernelGGL((chunk_prep_kernel<128>), grid, dim3(256), 0, stream, prep);
  else if (dk == 64 && raw)
    hipLaunchKernelGGL((chunk_fwd_kernel<PolBF16, __bf16, float, 64, true, true, true>), grid,
                       dim3(256), 0, stream, prep);
  else if (dk == 64)
    hipLaunchKernelGGL((chunk_prep_kernel<64>), grid, dim3(256), 0, stream, prep);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Consistency of a launch description with the kernel's index arithmetic: every unit maps to
// a valid (sequence, segment, head) and every tile to columns inside the state it writes.
static bool chunk_params_consistent(const ChunkParams& p, int dk) {
  if (p.H < 1 || p.n_seqs < 1 || p.n_seg < 1 || p.n_vt < 1 || p.dv < 64 || p.dv % 64) return false;
  if ((long long)p.n_units != (long long)p.n_seqs * p.n_seg * p.H) return false;
  if (!p.q || !p.k || !p.v || !p.g || !p.beta) return false;
  if (!p.cu_seqlens && p.seq_len < 0) return false;
  switch (p.mode) {
    case kModeForward:
      return p.n_seg == 1 && p.n_vt == p.dv / 64 && p.o;
    case kModeTransition:
      return p.n_vt == (dk + p.dv) / 64 && (dk % 64) == 0 && p.ws_pq;
    case kModeReplay:
      return p.n_vt == p.dv / 64 && p.ws_sin && p.o;
    default:
      return false;
  }
}

hipError_t launch_chunk_fwd(const ChunkParams& p, int io_dtype, int out_dtype, int dk,
                            hipStream_t stream) {
  if (!chunk_params_consistent(p, dk)) return hipErrorInvalidValue;
  if (io_dtype == 1) {
    if (out_dtype == 1) {
      if (dk == 128) return launch_one<PolBF16, __bf16, __bf16, 128>(p, stream);
      if (dk == 64) return launch_one<PolBF16, __bf16, __bf16, 64>(p, stream);
    } else {
      if (dk == 128) return launch_one<PolBF16, __bf16, float, 128>(p, stream);
      if (dk == 64) return launch_one<PolBF16, __bf16, float, 64>(p, stream);
    }
  } else {
    if (dk == 64) return launch_one<PolF32, float, float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
