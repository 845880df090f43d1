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
// a dominant factor would cost up to ~2.5% of the output RMS. Every factor on the dominant
// paths (T diag(beta), the diagonal blocks of M and their operands, M, U, V - K_Gamma S,
// Q e^Gamma, S in the read-out, K e^{Gamma_L - Gamma}) is therefore carried as a hi + lo pair
// of bf16 values and multiplied with three bf16 MFMAs (hi*hi + lo*hi + hi*lo): ~16 mantissa
// bits on matrix cores at 3/16 of the cost of fp32 MFMA.
//
// Work decomposition: one workgroup (4 waves) per (sequence, head, 64-wide value tile).
// Value columns of S never mix, so each wave owns 16 columns of S in its MFMA accumulators
// for the whole sequence (the state never leaves registers between chunks). The four waves
// share the per-chunk prologue through LDS.
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
  // ---- region X, recurrence view: Q e^Gamma (hi, lo), (K e^{GL-Gamma})^T (hi, lo),
  //      K e^Gamma, T diag(beta) (hi, lo)
  static constexpr size_t oQg = 0;
  static constexpr size_t oQgLo = oQg + tP;
  static constexpr size_t oKhT = oQgLo + kLo * tP;
  static constexpr size_t oKhTLo = oKhT + tT;
  static constexpr size_t oKg = oKhTLo + kLo * tT;
  static constexpr size_t oT = oKg + tP;
  static constexpr size_t oTLo = oT + t64;
  static constexpr size_t kXD = oTLo + kLo * t64;
  static constexpr size_t kX = kXA > kXD ? kXA : kXD;
  // ---- region Y: fp32 A / T, later V^T of the value tile
  static constexpr size_t oA = kX;
  static constexpr size_t oVT = kX;
  static constexpr size_t kY = size_t(64) * LDA * 4 > t64 ? size_t(64) * LDA * 4 : t64;
  // ---- region Z: M (hi, lo)
  static constexpr size_t oM = oA + kY;
  static constexpr size_t oMLo = oM + t64;
  // ---- small
  static constexpr size_t oBeta = oMLo + kLo * t64;
  static constexpr size_t oBP = oBeta + 64 * 4;        // [4][DK] sub-block decay products
  static constexpr size_t oDecay = oBP + 4 * DK * 4;   // [DK] whole-chunk decay
  static constexpr size_t oPair = oDecay + DK * 4;     // [3][DK] gaps between sub-blocks
  static constexpr size_t kBytes = oPair + 3 * DK * 4;
  static_assert(kBytes <= 160 * 1024, "LDS budget of one CDNA4 compute unit");
};

template <class Pol>
__device__ __forceinline__ void store_split(typename Pol::E* hi, typename Pol::E* lo, int idx,
                                            float x) {
  using E = typename Pol::E;
  const E h = from_f32<E>(x);
  hi[idx] = h;
  if constexpr (Pol::kSplit) lo[idx] = from_f32<E>(x - to_f32(h));
}

// 16 consecutive values (one 16-token column of a transposed tile) with vector stores
template <class Pol>
__device__ __forceinline__ void store16(typename Pol::E* dst, const float* x) {
  if constexpr (sizeof(typename Pol::E) == 2) {
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<bf16x4*>(dst + e) =
          bf16x4{(__bf16)x[e], (__bf16)x[e + 1], (__bf16)x[e + 2], (__bf16)x[e + 3]};
  } else {
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<f32x4*>(dst + e) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};
  }
}

template <class Pol>
__device__ __forceinline__ void store16_split(typename Pol::E* hi, typename Pol::E* lo,
                                              const float* x) {
  if constexpr (Pol::kSplit) {
#pragma unroll
    for (int e0 = 0; e0 < 16; e0 += 4) {
      bf16x4 a, c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = (__bf16)x[e0 + e];
        c[e] = (__bf16)(x[e0 + e] - (float)a[e]);
      }
      *reinterpret_cast<bf16x4*>(hi + e0) = a;
      *reinterpret_cast<bf16x4*>(lo + e0) = c;
    }
  } else {
    store16<Pol>(hi, x);
  }
}

// CPT consecutive channels of one token row
template <class Pol, int CPT>
__device__ __forceinline__ void store_row(typename Pol::E* dst, const float* x) {
  if constexpr (CPT == 2 && sizeof(typename Pol::E) == 2) {
    *reinterpret_cast<bf16x2*>(dst) = bf16x2{(__bf16)x[0], (__bf16)x[1]};
  } else {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) dst[cc] = from_f32<typename Pol::E>(x[cc]);
  }
}

template <class Pol, int CPT>
__device__ __forceinline__ void store_row_split(typename Pol::E* hi, typename Pol::E* lo,
                                                const float* x) {
  if constexpr (Pol::kSplit && CPT == 2) {
    const bf16x2 h = bf16x2{(__bf16)x[0], (__bf16)x[1]};
    *reinterpret_cast<bf16x2*>(hi) = h;
    *reinterpret_cast<bf16x2*>(lo) =
        bf16x2{(__bf16)(x[0] - (float)h[0]), (__bf16)(x[1] - (float)h[1])};
  } else {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) store_split<Pol>(hi, lo, cc, x[cc]);
  }
}

// Row-block IA of A and row-block 3 - IA of M for one wave. Column operands: k / rho on the
// diagonal block, k kappa next to it, k kappa times the decay gap further down.
template <class Pol, class L, int DK, int IA>
__device__ __forceinline__ void am_rows(const typename Pol::E* sKr, const typename Pol::E* sKd,
                                        const typename Pol::E* sKdLo, const typename Pol::E* sKc,
                                        const typename Pol::E* sQr, const typename Pol::E* sQrLo,
                                        const float* sPair, const float* sBeta, float* sA,
                                        typename Pol::E* sM, typename Pol::E* sMLo, int ln, int q4) {
  using Frag = typename Pol::Frag;
  constexpr int NS = Pol::slices(DK);
  constexpr int IM = 3 - IA;
  // gap factor index of a pair (i, j) with i - j >= 2: (2,0) -> 0, (3,1) -> 1, (3,0) -> 2
  constexpr int gapA0 = IA == 2 ? 0 : 2, gapA1 = 1;
  constexpr int gapM0 = IM == 2 ? 0 : 2, gapM1 = 1;
  f32x4 accA[4], accM[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    accA[jb] = zero4();
    accM[jb] = zero4();
  }
#pragma unroll
  for (int pp = 0; pp < NS; ++pp) {
    const Frag rowA = Pol::load(sKr, L::LDP, 16 * IA + ln, pp, q4);
    const Frag rowM = Pol::load(sQr, L::LDP, 16 * IM + ln, pp, q4);
    Frag colA[4], colM[4], dKl, dQl;
#pragma unroll
    for (int jb = 0; jb <= IA; ++jb) {
      if (jb == IA) colA[jb] = Pol::load(sKd, L::LDP, 16 * jb + ln, pp, q4);
      else if (jb == IA - 1) colA[jb] = Pol::load(sKc, L::LDP, 16 * jb + ln, pp, q4);
      else colA[jb] = Pol::load_scaled(sKc, L::LDP, 16 * jb + ln, pp, q4,
                                       sPair + (jb == 0 ? gapA0 : gapA1) * DK);
    }
#pragma unroll
    for (int jb = 0; jb <= IM; ++jb) {
      if (jb == IM) colM[jb] = Pol::load(sKd, L::LDP, 16 * jb + ln, pp, q4);
      else if (jb == IM - 1) colM[jb] = Pol::load(sKc, L::LDP, 16 * jb + ln, pp, q4);
      else colM[jb] = Pol::load_scaled(sKc, L::LDP, 16 * jb + ln, pp, q4,
                                       sPair + (jb == 0 ? gapM0 : gapM1) * DK);
    }
    if constexpr (Pol::kSplit) {
      dKl = Pol::load(sKdLo, L::LDP, 16 * IM + ln, pp, q4);
      dQl = Pol::load(sQrLo, L::LDP, 16 * IM + ln, pp, q4);
    }
#pragma unroll
    for (int jb = 0; jb <= IA; ++jb) accA[jb] = Pol::mma(colA[jb], rowA, accA[jb]);
#pragma unroll
    for (int jb = 0; jb <= IM; ++jb) accM[jb] = Pol::mma(colM[jb], rowM, accM[jb]);
    if constexpr (Pol::kSplit) {
      accM[IM] = Pol::mma(dKl, rowM, accM[IM]);
      accM[IM] = Pol::mma(colM[IM], dQl, accM[IM]);
    }
  }
  // register e of block (row i, column jb): row 16 i + ln, column 16 jb + 4 q4 + e
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
#pragma unroll
  for (int jb = 0; jb <= IM; ++jb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * jb + 4 * q4 + e;
      store_split<Pol>(sM, sMLo, rm * L::LDT + s, (jb == IM && s > rm) ? 0.f : accM[jb][e]);
    }
  }
}

// Raw inputs of one chunk held by one thread: CPT key channels x 16 tokens of its
// sub-block, one value column x 16 tokens, and (lanes < 16) one beta.
template <typename Tio, int CPT>
struct RawChunk {
  float g[16][CPT];
  Tio k[16][CPT];
  Tio q[16][CPT];
  Tio v[16];
  float beta;
};

template <typename Tio, int DK, int CPT>
__device__ __forceinline__ void load_chunk(RawChunk<Tio, CPT>& x, const ChunkParams& p,
                                           int cstart, int Lc, int w, int lane, int h,
                                           int vcol0, bool p_tile) {
  const Tio* __restrict__ gq = reinterpret_cast<const Tio*>(p.q);
  const Tio* __restrict__ gk = reinterpret_cast<const Tio*>(p.k);
  const Tio* __restrict__ gv = reinterpret_cast<const Tio*>(p.v);
  const int H = p.H;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int r = 16 * w + t;
    const int tok = cstart + (r < Lc ? r : 0);   // rows past the end read a valid row
    const size_t base = (size_t(tok) * H + h) * DK + CPT * lane;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      x.g[t][cc] = p.g[base + cc];
      x.k[t][cc] = gk[base + cc];
      x.q[t][cc] = gq[base + cc];
    }
    x.v[t] = gv[(size_t(tok) * H + h) * p.dv + vcol0 + lane];
  }
  x.beta = 0.f;
  if (lane < 16) {
    const int r = 16 * w + lane;
    x.beta = p.beta[size_t(cstart + (r < Lc ? r : 0)) * H + h];
  }
  (void)p_tile;
}

template <class Pol, typename Tio, typename Tout, int DK>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkParams p) {
  using L = ChunkLayout<Pol, DK>;
  using E = typename Pol::E;
  using Frag = typename Pol::Frag;
  constexpr int CPT = DK / 64;             // key channels per thread in the prologue
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
  E* sQg = reinterpret_cast<E*>(smem + L::oQg);
  E* sQgLo = reinterpret_cast<E*>(smem + L::oQgLo);
  E* sKhT = reinterpret_cast<E*>(smem + L::oKhT);
  E* sKhTLo = reinterpret_cast<E*>(smem + L::oKhTLo);
  E* sKg = reinterpret_cast<E*>(smem + L::oKg);
  E* sT = reinterpret_cast<E*>(smem + L::oT);
  E* sTLo = reinterpret_cast<E*>(smem + L::oTLo);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  E* sVT = reinterpret_cast<E*>(smem + L::oVT);
  E* sM = reinterpret_cast<E*>(smem + L::oM);
  E* sMLo = reinterpret_cast<E*>(smem + L::oMLo);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
  float* sBP = reinterpret_cast<float*>(smem + L::oBP);
  float* sDecay = reinterpret_cast<float*>(smem + L::oDecay);
  float* sPair = reinterpret_cast<float*>(smem + L::oPair);

  // ---- which (sequence, segment, head, state tile): the tiles of one unit share an XCD
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int rest = b >> 3;
  const int vt = rest % p.n_vt;
  const int unit = (rest / p.n_vt) * 8 + xcd;
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int DV = p.dv;
  const int h = unit % H;
  const int sj = unit / H;              // global segment index n * n_seg + j
  const int n = sj / p.n_seg;
  const int j = sj % p.n_seg;
  const int mode = p.mode;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
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
  if (p.n_seg > 1) {
    // chunk-aligned contiguous segments: segment j holds chunks [j nc / n_seg, (j+1) nc / n_seg)
    const long long nc = (eos - bos + kChunk - 1) / kChunk;
    const int c_lo = int((j * nc) / p.n_seg);
    const int c_hi = int(((j + 1) * nc) / p.n_seg);
    const int seg_bos = bos + kChunk * c_lo;
    eos = min(eos, bos + kChunk * c_hi);
    bos = seg_bos;
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
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * t + 4 * q4 + e;
      float x = 0.f;
      if (s_in) x = s_in[size_t(c) * DV + col0 + ln];
      if (p_tile) x = (c == col0 + ln) ? 1.f : 0.f;
      S[t][e] = x;
    }
  }

  // strictly upper sub-blocks of M stay zero for the whole sequence
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int r = idx >> 6, s = idx & 63;
    if ((s >> 4) > (r >> 4)) {
      sM[r * L::LDT + s] = from_f32<E>(0.f);
      if constexpr (Pol::kSplit) sMLo[r * L::LDT + s] = from_f32<E>(0.f);
    }
  }

  RawChunk<Tio, CPT> raw;

  for (int cstart = bos; cstart < eos; cstart += kChunk) {
    const int Lc = min(kChunk, eos - cstart);
    load_chunk<Tio, DK, CPT>(raw, p, cstart, Lc, w, lane, h, vcol0, p_tile);

    // ================= prologue 1: decay factors and operand tiles ======================
    // rho = e^{lambda} (decay from the sub-block start to token r, inclusive) <= 1;
    // kappa = P / rho (decay after token r to the sub-block end) <= 1; 1/rho <= e^{16|g_min|}
    float qr[16][CPT], kr[16][CPT], kc[16][CPT], vv[16];
    float bp[CPT];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) bp[cc] = 1.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const bool valid = 16 * w + t < Lc;
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        const float gt = valid ? fmaxf(raw.g[t][cc], p.g_min) : 0.f;
        bp[cc] *= __expf(gt);
        kr[t][cc] = bp[cc];                           // rho, for now
        kc[t][cc] = valid ? to_f32(raw.k[t][cc]) : 0.f;
        qr[t][cc] = valid ? to_f32(raw.q[t][cc]) : 0.f;
      }
      vv[t] = (valid && !p_tile) ? to_f32(raw.v[t]) : 0.f;
    }
    const float beta_r = (16 * w + lane < Lc) ? raw.beta : 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int r = 16 * w + t;
      float xq[CPT], xkd[CPT], xkr[CPT], xkc[CPT];
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        const float rho = kr[t][cc];
        const float rinv = __builtin_amdgcn_rcpf(rho);
        const float k0 = kc[t][cc];
        xq[cc] = qr[t][cc] * rho;
        xkd[cc] = k0 * rinv;
        xkr[cc] = k0 * rho;
        xkc[cc] = k0 * (bp[cc] * rinv);
        qr[t][cc] = xq[cc];      // q rho
        kr[t][cc] = xkr[cc];     // k rho
        kc[t][cc] = xkc[cc];     // k kappa
      }
      const int idx = r * L::LDP + CPT * lane;
      store_row_split<Pol, CPT>(sQr + idx, sQrLo + idx, xq);
      store_row_split<Pol, CPT>(sKd + idx, sKdLo + idx, xkd);
      store_row<Pol, CPT>(sKr + idx, xkr);
      store_row<Pol, CPT>(sKc + idx, xkc);
    }
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) sBP[w * DK + CPT * lane + cc] = bp[cc];
    if (lane < 16) sBeta[16 * w + lane] = beta_r;
    __syncthreads();

    // ---- chunk-level factors from the four sub-block products of each channel
    float fs[CPT], fe[CPT];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = CPT * lane + cc;
      const float Pb[4] = {sBP[c], sBP[DK + c], sBP[2 * DK + c], sBP[3 * DK + c]};
      fs[cc] = 1.f;
      fe[cc] = 1.f;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        if (bb < w) fs[cc] *= Pb[bb];
        if (bb > w) fe[cc] *= Pb[bb];
      }
      if (w == 0) {
        sDecay[c] = Pb[0] * Pb[1] * Pb[2] * Pb[3];
        sPair[c] = Pb[1];                   // gap for sub-block pair (2, 0)
        sPair[DK + c] = Pb[2];              // (3, 1)
        sPair[2 * DK + c] = Pb[1] * Pb[2];  // (3, 0)
      }
    }
    __syncthreads();

    // ================= prologue 2: A (fp32) and M (hi, lo) sub-blocks ====================
    // wave w: row-block w of A (blocks (w, j <= w)) and row-block 3 - w of M; every wave runs
    // 28 MFMAs (M's diagonal block uses split operands). The row blocks are compile-time per
    // wave so each slice's fragment loads issue together.
    switch (w) {
      case 0: am_rows<Pol, L, DK, 0>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sPair, sBeta, sA, sM, sMLo, ln, q4); break;
      case 1: am_rows<Pol, L, DK, 1>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sPair, sBeta, sA, sM, sMLo, ln, q4); break;
      case 2: am_rows<Pol, L, DK, 2>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sPair, sBeta, sA, sM, sMLo, ln, q4); break;
      default: am_rows<Pol, L, DK, 3>(sKr, sKd, sKdLo, sKc, sQr, sQrLo, sPair, sBeta, sA, sM, sMLo, ln, q4); break;
    }
    __syncthreads();

    // ================= prologue 3: recurrence operand tiles; fp32 inverse =================
    if (w == 0) {
      // diagonal sub-blocks: lane = (block bi, column jc); right-looking substitution in fp32:
      // once x_s is final it is removed from every later row
      const int bi = lane >> 4, jc = lane & 15;
      const float* Ab = sA + 16 * bi * L::LDA + 16 * bi;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == jc) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 15; ++s) {
#pragma unroll
        for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-Ab[r * L::LDA + s], x[s], x[r]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sA[(16 * bi + r) * L::LDA + 16 * bi + jc] = x[r];
    }
    {
      const int c0 = CPT * lane;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int r = 16 * w + t;
        float xq[CPT], xk[CPT];
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
          xq[cc] = qr[t][cc] * fs[cc];   // q e^{Gamma}
          xk[cc] = kr[t][cc] * fs[cc];   // k e^{Gamma}
        }
        store_row_split<Pol, CPT>(sQg + r * L::LDP + c0, sQgLo + r * L::LDP + c0, xq);
        store_row<Pol, CPT>(sKg + r * L::LDP + c0, xk);
      }
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        float col[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) col[t] = kc[t][cc] * fe[cc];   // k e^{Gamma_L - Gamma}
        store16_split<Pol>(sKhT + (c0 + cc) * L::LDT + 16 * w, sKhTLo + (c0 + cc) * L::LDT + 16 * w, col);
      }
    }
    __syncthreads();
    // off-diagonal sub-blocks on fp32 MFMA (16x16x4) in two levels:
    //   level 1: T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22
    //   level 2: the lower-left 32x32 block -T_[23][23] A_[23][01] T_[01][01], one 16x16 block
    //   per wave (T_20, T_21, T_30, T_31).
    // T_ij (i > j) is stored in the free upper position (j, i) so that A_ij stays readable.
    auto tblk = [&](int bi, int bj) -> float* {
      return bi == bj ? sA + 16 * bi * L::LDA + 16 * bi : sA + 16 * bj * L::LDA + 16 * bi;
    };
    auto ablk = [&](int bi, int bj) -> const float* { return sA + 16 * bi * L::LDA + 16 * bj; };
    // X += A_blk * T_blk (16x16x16, natural k order)
    auto mm_acc = [&](f32x4 X, const float* Ab, const float* Tb) -> f32x4 {
#pragma unroll
      for (int kk2 = 0; kk2 < 4; ++kk2)
        X = mma_f32(Ab[ln * L::LDA + 4 * kk2 + q4], Tb[(4 * kk2 + q4) * L::LDA + ln], X);
      return X;
    };
    // Y += T_blk * X with X in accumulator layout (slice e holds rows 4 q4 + e)
    auto mm_reg = [&](f32x4 Y, const float* Tb, f32x4 X) -> f32x4 {
#pragma unroll
      for (int e = 0; e < 4; ++e) Y = mma_f32(Tb[ln * L::LDA + 4 * q4 + e], X[e], Y);
      return Y;
    };
    auto put = [&](int bi, int bj, f32x4 Y) {
      float* To = tblk(bi, bj);
#pragma unroll
      for (int e = 0; e < 4; ++e) To[(4 * q4 + e) * L::LDA + ln] = -Y[e];
    };
    if (w < 2) {
      const int lo = 2 * w;   // (1, 0) or (3, 2)
      const f32x4 X = mm_acc(zero4(), ablk(lo + 1, lo), tblk(lo, lo));
      put(lo + 1, lo, mm_reg(zero4(), tblk(lo + 1, lo + 1), X));
    }
    __syncthreads();
    {
      const int bj = w & 1;          // column block 0 or 1
      const bool row3 = w >= 2;      // row block 2 or 3
      f32x4 X2, X3 = zero4();        // X_2j, X_3j = A_[2|3],[01] T_[01],j
      if (bj == 0) {
        X2 = mm_acc(mm_acc(zero4(), ablk(2, 0), tblk(0, 0)), ablk(2, 1), tblk(1, 0));
        if (row3) X3 = mm_acc(mm_acc(zero4(), ablk(3, 0), tblk(0, 0)), ablk(3, 1), tblk(1, 0));
      } else {
        X2 = mm_acc(zero4(), ablk(2, 1), tblk(1, 1));
        if (row3) X3 = mm_acc(zero4(), ablk(3, 1), tblk(1, 1));
      }
      f32x4 Y;
      if (!row3) Y = mm_reg(zero4(), tblk(2, 2), X2);
      else Y = mm_reg(mm_reg(zero4(), tblk(3, 2), X2), tblk(3, 3), X3);
      put(row3 ? 3 : 2, bj, Y);
    }
    __syncthreads();

    // T' = T diag(beta), rounded once complete (hi, lo): thread = (row r, 16 columns)
    {
      const int r = tid >> 2;
      const int s0 = 16 * (tid & 3);
      const float* Tb = tblk(r >> 4, s0 >> 4) + (r & 15) * L::LDA;
      float row[16];
#pragma unroll
      for (int u = 0; u < 16; u += 4) {
        const f32x4 tv = *reinterpret_cast<const f32x4*>(Tb + u);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(sBeta + s0 + u);
#pragma unroll
        for (int e = 0; e < 4; ++e) row[u + e] = (s0 + u + e <= r) ? tv[e] * bv[e] : 0.f;
      }
      store16_split<Pol>(sT + r * L::LDT + s0, sTLo + r * L::LDT + s0, row);
    }
    __syncthreads();
    // value tile, transposed, into region Y (A / T are dead now)
    store16<Pol>(sVT + lane * L::LDT + 16 * w, vv);
    __syncthreads();

    // ================= serial step: this wave's 16 value columns ============================
    // Each product loads a batch of A fragments from LDS first and then issues its MFMAs, so
    // several LDS reads are in flight per wave (one wave per SIMD hides nothing otherwise).
    Frag Sh[NS], Sl[NS];
#pragma unroll
    for (int pp = 0; pp < NS; ++pp) Pol::from_acc_split(S, pp, Sh[pp], Sl[pp]);
    f32x4 U[4], O[4];
    // O = (Q e^Gamma) S first, while S is split
#pragma unroll
    for (int pp = 0; pp < NS; ++pp) {
      Frag qh[4], ql[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        qh[rb] = Pol::load(sQg, L::LDP, 16 * rb + ln, pp, q4);
        if constexpr (Pol::kSplit) ql[rb] = Pol::load(sQgLo, L::LDP, 16 * rb + ln, pp, q4);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        O[rb] = Pol::mma(qh[rb], Sh[pp], pp == 0 ? zero4() : O[rb]);
        if constexpr (Pol::kSplit) {
          O[rb] = Pol::mma(ql[rb], Sh[pp], O[rb]);
          O[rb] = Pol::mma(qh[rb], Sl[pp], O[rb]);
        }
      }
    }
    // X = (K e^Gamma) S - V, in fp32
    f32x4 X[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const E* vsrc = sVT + (16 * w + ln) * L::LDT + 16 * rb + 4 * q4;
#pragma unroll
      for (int e = 0; e < 4; ++e) X[rb][e] = -to_f32(vsrc[e]);
    }
#pragma unroll
    for (int pp = 0; pp < NS; ++pp) {
      Frag kg[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) kg[rb] = Pol::load(sKg, L::LDP, 16 * rb + ln, pp, q4);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) X[rb] = Pol::mma(kg[rb], Sh[pp], X[rb]);
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
      for (int rb = 0; rb < 4; ++rb) {
        if (pp < Pol::slices_blocks(rb + 1)) {
          U[rb] = Pol::mma(th[rb], Xh[pp], pp == 0 ? zero4() : U[rb]);
          if constexpr (Pol::kSplit) {
            U[rb] = Pol::mma(tl[rb], Xh[pp], U[rb]);
            U[rb] = Pol::mma(th[rb], Xl[pp], U[rb]);
          }
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) U[rb] = -U[rb];
    // O += M U
    Frag Uh[NT], Ul[NT];
#pragma unroll
    for (int pp = 0; pp < NT; ++pp) Pol::from_acc_split(U, pp, Uh[pp], Ul[pp]);
#pragma unroll
    for (int pp = 0; pp < NT; ++pp) {
      Frag mh[4], ml[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (pp < Pol::slices_blocks(rb + 1)) {
          mh[rb] = Pol::load(sM, L::LDT, 16 * rb + ln, pp, q4);
          if constexpr (Pol::kSplit) ml[rb] = Pol::load(sMLo, L::LDT, 16 * rb + ln, pp, q4);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (pp < Pol::slices_blocks(rb + 1)) {
          O[rb] = Pol::mma(mh[rb], Uh[pp], O[rb]);
          if constexpr (Pol::kSplit) {
            O[rb] = Pol::mma(ml[rb], Uh[pp], O[rb]);
            O[rb] = Pol::mma(mh[rb], Ul[pp], O[rb]);
          }
        }
      }
    }
    if (mode != kModeTransition) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * q4 + e;
          if (r < Lc)
            go[(size_t(cstart + r) * H + h) * DV + col0 + ln] = from_f32<Tout>(p.scale * O[rb][e]);
        }
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
        Frag kh[4], kl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          kh[t] = Pol::load(sKhT, L::LDT, 16 * (t0 + t) + ln, pp, q4);
          if constexpr (Pol::kSplit) kl[t] = Pol::load(sKhTLo, L::LDT, 16 * (t0 + t) + ln, pp, q4);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          S[t0 + t] = Pol::mma(kh[t], Uh[pp], S[t0 + t]);
          if constexpr (Pol::kSplit) {
            S[t0 + t] = Pol::mma(kl[t], Uh[pp], S[t0 + t]);
            S[t0 + t] = Pol::mma(kh[t], Ul[pp], S[t0 + t]);
          }
        }
      }
    }
    __syncthreads();
  }

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

template <class Pol, typename Tio, typename Tout, int DK>
static hipError_t launch_one(const ChunkParams& p, hipStream_t stream) {
  const int groups = (p.n_units + 7) / 8;
  const dim3 grid(groups * 8 * p.n_vt);
  hipLaunchKernelGGL((chunk_fwd_kernel<Pol, Tio, Tout, DK>), grid, dim3(256), 0, stream, p);
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
