// Chunked backward of the KDA recurrence on gfx950: 16-token chunks, every product on fp32
// matrix cores (v_mfma_f32_16x16x4_f32).
//
// The pages give the forward only ("Noyaux KDA et FlashKDA", section "FlashKDA : le noyau par
// blocs": the chunked kernel serves training as well as prefill). This file differentiates the
// chunk form of that forward. Per chunk of C = 16 tokens (G: the in-chunk cumulative sum of the
// floored log-decays, per key channel; G_C its value after the last token):
//
//   K_G = K e^G,  Q_G = Q e^G,  K^ = K e^(G_C - G)
//   A = tril(diag(beta) K_G (K e^-G)^T, -1),  T = (I + A)^-1,  M = tril(Q_G (K e^-G)^T)
//   X0 = V - K_G S0,  Y = diag(beta) X0,  U = T Y
//   O = s (Q_G S0 + M U),  S_C = e^(G_C) S0 + K^^T U
//
// and, going back with dS = dL/dS_C:
//
//   dU = s M^T dO + K^ dS,  dY = T^T dU,  dV = diag(beta) dY,  dT = dU Y^T,
//   dA = -T^T dT T^T (strictly lower),  dM = s dO U^T (lower),
//   dS0 = e^(G_C) dS + s Q_G^T dO - K_G^T diag(beta) dY,
//
// the pairwise terms of A and M giving each token's query-side and key-side key gradients,
// and the log-decay gradient q dq + k dk(query side) - k dk(key side) plus the chunk-end
// terms, summed in reverse over the chunk (tests/test_backward_chunk_form.py checks these
// formulas against the per-token chain rule in fp64). With 16 tokens the decay factors stay
// inside fp32 (|G| <= 16 x 5.4); the pairwise factors e^(G_t - G_s) are formed as
// e^(G_t - G_m) e^(G_m - G_s) around the chunk's mid value G_m, so no factor exceeds e^44.
//
// Three launches:
//   1. cbwd_fwd_kernel: one wave per (sequence, head, 16-column tile) walks the chunks
//      forward and stores each chunk's entering state S0, X0 and U;
//   2. cbwd_rev_kernel: the same waves walk back, storing dS (the gradient of the state
//      leaving each chunk), dU and dY, writing dv, and dh0 at the sequence start;
//   3. cbwd_grad_kernel: one workgroup per (chunk, head) forms dq, dk, dbeta and dg.
// Sums over value columns happen inside launch 3 in a fixed order: results are deterministic.
#include "kda_bwd.h"
#include "kda_common.h"

namespace kda {

namespace {

constexpr int kC = kCBChunk;

// chunk slot of chunk c of sequence n (whose first token is bos)
__device__ __forceinline__ long long cb_slot(int bos, int n, int c) {
  return (long long)(bos / kC) + n + c;
}

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p, size_t i) {
  return to_f32(p[i]);
}

// 1 or 0. Rows past a ragged chunk's end are loaded from a row inside it (the index stays in
// bounds) and scaled by 0: a load made only under a condition is followed by a wait for it
// where the branches join, which would serialise a loop of such loads.
__device__ __forceinline__ float keep_f(bool keep) { return keep ? 1.f : 0.f; }
template <typename T>
__device__ __forceinline__ float ld_keep(const T* p, size_t i, bool keep) {
  return to_f32(p[i]) * keep_f(keep);
}

// four consecutive elements as fp32 (16- or 8-byte aligned)
__device__ __forceinline__ f32x4 ld4(const float* p, size_t i) {
  return *reinterpret_cast<const f32x4*>(p + i);
}
__device__ __forceinline__ f32x4 ld4(const __bf16* p, size_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  f32x4 r;
  r[0] = __builtin_bit_cast(float, u.x << 16);
  r[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
  r[2] = __builtin_bit_cast(float, u.y << 16);
  r[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
  return r;
}

// One wave's prologue of a chunk for the walks: the in-chunk decays of its key channels
// (lane, lane + 64, ...), written to LDS as the operand tiles the chunk's products read.
// Token-major tiles have rows of LK floats, channel-major ones rows of LT.
template <typename Tio, int DK, bool kRev>
struct WalkTiles {
  static constexpr int CPL = DK / 64;
  static constexpr int LK = DK + 1;   // (odd strides: the 16 rows a product reads hit 16 banks)
  static constexpr int LT = kC + 1;
  float* Kg;     // token-major K e^G (forward), or channel-major (reverse)
  float* Kh;     // channel-major K e^(G_C - G) (forward), or token-major (reverse)
  float* QgT;    // channel-major Q e^G (reverse only)
  float* Kq;     // token-major K e^(G - G_m)
  float* Kk;     // token-major K e^(G_m - G)
  float* Qq;     // token-major Q e^(G - G_m) (reverse only)
  float* eGC;    // e^(G_C) per channel
  float* beta;   // per token

  __device__ void build(const CBwdParams& p, int cs, int L, int h, int lane) const {
    const int H = p.H;
    const Tio* gk = reinterpret_cast<const Tio*>(p.k);
    const Tio* gq = reinterpret_cast<const Tio*>(p.q);
    float G[kC][CPL], kv[kC][CPL], qv[kC][CPL];
    float acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      const bool valid = t < L;
      const size_t row = (size_t(valid ? cs + t : cs) * H + h) * DK;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int ch = lane + 64 * i;
        const float gv = p.g[row + ch];
        acc[i] += fmaxf(gv, p.g_min) * keep_f(valid);
        G[t][i] = acc[i];
        kv[t][i] = ld_keep(gk, row + ch, valid);
        if constexpr (kRev) qv[t][i] = ld_keep(gq, row + ch, valid);
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int ch = lane + 64 * i;
      const float gc = G[kC - 1][i];
      const float gm = 0.5f * (G[0][i] + gc);
      eGC[ch] = __expf(gc);
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        const float eg = __expf(G[t][i]);
        const float eh = __expf(gc - G[t][i]);
        const float em = __expf(G[t][i] - gm);
        const float emi = __expf(gm - G[t][i]);
        Kq[t * LK + ch] = kv[t][i] * em;
        Kk[t * LK + ch] = kv[t][i] * emi;
        if constexpr (!kRev) {
          Kg[t * LK + ch] = kv[t][i] * eg;
          Kh[ch * LT + t] = kv[t][i] * eh;
        } else {
          Kg[ch * LT + t] = kv[t][i] * eg;
          Kh[t * LK + ch] = kv[t][i] * eh;
          QgT[ch * LT + t] = qv[t][i] * eg;
          Qq[t * LK + ch] = qv[t][i] * em;
        }
      }
    }
    if (lane < kC) beta[lane] = lane < L ? p.beta[size_t(cs + lane) * H + h] : 0.f;
  }
};

// 16 x 16 product over the key channels: D[t][s] = sum_c X[t][c] Y[s][c] (token-major tiles)
template <int DK>
__device__ __forceinline__ f32x4 gram16(const float* X, const float* Y, int ln, int q4) {
  constexpr int LK = DK + 1;
  f32x4 acc = zero4();
#pragma unroll
  for (int kk = 0; kk < DK / 4; ++kk) {
    const int c = (DK / 4) * q4 + kk;
    acc = mma_f32(X[ln * LK + c], Y[ln * LK + c], acc);
  }
  return acc;
}

// T = (I + A)^-1 for the strictly lower A[t][s] = beta_t B[t][s] (B stored with row stride 17):
// lane j < 16 solves column j by forward substitution into sT (row stride 20)
__device__ __forceinline__ void invert16(const float* sB, const float* sBeta, float* sT, int lane) {
  if (lane < kC) {
    float x[kC];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float v = (i == lane) ? 1.f : 0.f;
      const float bi = sBeta[i];
#pragma unroll
      for (int m = 0; m < i; ++m) v = fmaf(-bi * sB[i * 17 + m], x[m], v);
      x[i] = v;
      sT[i * 20 + lane] = v;
    }
  }
}

// a wave's own LDS writes made visible to its other lanes
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

// ---- 1. forward walk: S0, X0 and U of every chunk
template <typename Tio, int DK>
__global__ __launch_bounds__(64) void cbwd_fwd_kernel(CBwdParams p) {
  constexpr int DV = DK, NTD = DK / 16;
  using WT = WalkTiles<Tio, DK, false>;
  constexpr int LK = WT::LK, LT = WT::LT;
  __shared__ float sKg[kC * LK], sKq[kC * LK], sKk[kC * LK];
  __shared__ float sKhT[DK * LT];
  __shared__ float sB[kC * 17], sT[kC * 20], sGC[DK], sBeta[kC];

  int ct;
  const int unit = block_unit(blockIdx.x, p.n_ct, &ct);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int h = unit % H, n = unit / H;
  const int bos = p.cu_seqlens ? p.cu_seqlens[n] : n * p.seq_len;
  const int eos = p.cu_seqlens ? p.cu_seqlens[n + 1] : bos + p.seq_len;
  const int lane = threadIdx.x, q4 = lane >> 4, ln = lane & 15;
  const int col = 16 * ct + ln;
  const Tio* gv = reinterpret_cast<const Tio*>(p.v);
  const WT tiles{sKg, sKhT, nullptr, sKq, sKk, nullptr, sGC, sBeta};

  // the state tile in accumulator layout: block rb, register r = row 16 rb + 4 q4 + r
  f32x4 S[NTD];
  const size_t st_off = (size_t(n) * H + h) * DK * DV;
#pragma unroll
  for (int rb = 0; rb < NTD; ++rb) S[rb] = zero4();
  if (p.h0) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[rb][r] = p.h0[st_off + size_t(16 * rb + 4 * q4 + r) * DV + col];
  }

  int c = 0;
  for (int cs = bos; cs < eos; cs += kC, ++c) {
    const int L = min(kC, eos - cs);
    const size_t blk = size_t(cb_slot(bos, n, c)) * H + h;
    tiles.build(p, cs, L, h, lane);
    wave_sync();
    {
      const f32x4 b = gram16<DK>(sKq, sKk, ln, q4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * q4 + r;
        sB[t * 17 + ln] = ln < t ? b[r] : 0.f;
      }
    }
    wave_sync();
    invert16(sB, sBeta, sT, lane);
    wave_sync();
    // the state entering the chunk
    float* s0 = p.S0 + blk * DK * DV;
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s0[size_t(16 * rb + 4 * q4 + r) * DV + col] = S[rb][r];
    // X = K_G S (k order: the state's own register order)
    f32x4 X = zero4();
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) X = mma_f32(sKg[ln * LK + 16 * rb + 4 * q4 + r], S[rb][r], X);
    // X0 = V - X, Y = diag(beta) X0 (rows past a ragged chunk's end stay zero)
    f32x4 X0, Y;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q4 + r;
      const float vv = ld_f32(gv, (size_t(t < L ? cs + t : cs) * H + h) * DV + col);
      X0[r] = (vv - X[r]) * keep_f(t < L);
      Y[r] = sBeta[t] * X0[r];
    }
    // U = T Y
    f32x4 U = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) U = mma_f32(sT[ln * 20 + 4 * q4 + kk], Y[kk], U);
    float* wx = p.X0 + blk * kC * DV;
    float* wu = p.U + blk * kC * DV;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      wx[size_t(4 * q4 + r) * DV + col] = X0[r];
      wu[size_t(4 * q4 + r) * DV + col] = U[r];
    }
    // S = e^(G_C) S + K^^T U
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[rb][r] *= sGC[16 * rb + 4 * q4 + r];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        S[rb] = mma_f32(sKhT[(16 * rb + ln) * LT + 4 * q4 + kk], U[kk], S[rb]);
    }
    wave_sync();   // the next chunk rewrites the tiles
  }
}

// ---- 2. reverse walk: dS, dU, dY of every chunk, dv, and dh0
template <typename Tio, int DK>
__global__ __launch_bounds__(64) void cbwd_rev_kernel(CBwdParams p) {
  constexpr int DV = DK, NTD = DK / 16;
  using WT = WalkTiles<Tio, DK, true>;
  constexpr int LK = WT::LK, LT = WT::LT;
  __shared__ float sKh[kC * LK], sKq[kC * LK], sKk[kC * LK], sQq[kC * LK];
  __shared__ float sKgT[DK * LT], sQgT[DK * LT];
  __shared__ float sB[kC * 17], sM[kC * 17], sT[kC * 20], sGC[DK], sBeta[kC];

  int ct;
  const int unit = block_unit(blockIdx.x, p.n_ct, &ct);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int h = unit % H, n = unit / H;
  const int bos = p.cu_seqlens ? p.cu_seqlens[n] : n * p.seq_len;
  const int eos = p.cu_seqlens ? p.cu_seqlens[n + 1] : bos + p.seq_len;
  const int lane = threadIdx.x, q4 = lane >> 4, ln = lane & 15;
  const int col = 16 * ct + ln;
  const Tio* gdo = reinterpret_cast<const Tio*>(p.d_o);
  const WT tiles{sKgT, sKh, sQgT, sKq, sKk, sQq, sGC, sBeta};

  f32x4 D[NTD];
  const size_t st_off = (size_t(n) * H + h) * DK * DV;
#pragma unroll
  for (int rb = 0; rb < NTD; ++rb) D[rb] = zero4();
  if (p.dht) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) D[rb][r] = p.dht[st_off + size_t(16 * rb + 4 * q4 + r) * DV + col];
  }

  const int nch = (eos - bos + kC - 1) / kC;
  for (int c = nch - 1; c >= 0; --c) {
    const int cs = bos + kC * c;
    const int L = min(kC, eos - cs);
    const size_t blk = size_t(cb_slot(bos, n, c)) * H + h;
    tiles.build(p, cs, L, h, lane);
    wave_sync();
    {
      const f32x4 b = gram16<DK>(sKq, sKk, ln, q4);
      const f32x4 m = gram16<DK>(sQq, sKk, ln, q4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * q4 + r;
        sB[t * 17 + ln] = ln < t ? b[r] : 0.f;
        sM[t * 17 + ln] = ln <= t ? m[r] : 0.f;
      }
    }
    wave_sync();
    invert16(sB, sBeta, sT, lane);
    wave_sync();
    // the gradient of the state leaving the chunk
    float* ds = p.dS + blk * DK * DV;
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) ds[size_t(16 * rb + 4 * q4 + r) * DV + col] = D[rb][r];
    // s dO as the products' right operand: token 4 q4 + kk, this lane's column
    float sdo[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int t = 4 * q4 + kk;
      sdo[kk] = p.scale * ld_keep(gdo, (size_t(t < L ? cs + t : cs) * H + h) * DV + col, t < L);
    }
    // dU = M^T (s dO) + K^ D
    f32x4 dU = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) dU = mma_f32(sM[(4 * q4 + kk) * 17 + ln], sdo[kk], dU);
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dU = mma_f32(sKh[ln * LK + 16 * rb + 4 * q4 + r], D[rb][r], dU);
    // dY = T^T dU
    f32x4 dY = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) dY = mma_f32(sT[(4 * q4 + kk) * 20 + ln], dU[kk], dY);
    float* wdu = p.dU + blk * kC * DV;
    float* wdy = p.dY + blk * kC * DV;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q4 + r;
      wdu[size_t(t) * DV + col] = dU[r];
      wdy[size_t(t) * DV + col] = dY[r];
      if (t < L) p.dv[(size_t(cs + t) * H + h) * DV + col] = sBeta[t] * dY[r];
    }
    // D = e^(G_C) D + Q_G^T (s dO) - K_G^T diag(beta) dY
    float bdy[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bdy[kk] = -sBeta[4 * q4 + kk] * dY[kk];
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) D[rb][r] *= sGC[16 * rb + 4 * q4 + r];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        D[rb] = mma_f32(sQgT[(16 * rb + ln) * LT + 4 * q4 + kk], sdo[kk], D[rb]);
        D[rb] = mma_f32(sKgT[(16 * rb + ln) * LT + 4 * q4 + kk], bdy[kk], D[rb]);
      }
    }
    wave_sync();
  }
  if (p.dh0) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p.dh0[st_off + size_t(16 * rb + 4 * q4 + r) * DV + col] = D[rb][r];
  }
}

// ---- 3. gradients of one chunk: dq, dk, dbeta and dg. One workgroup (DK / 16 waves) per
// (chunk slot, head); workgroups of unused slots exit.
template <typename Tio, int DK>
__global__ __launch_bounds__(4 * DK) void cbwd_grad_kernel(CBwdParams p) {
  constexpr int DV = DK, NT = 4 * DK;
  constexpr int LK = DK + 1, LV = DV + 4;
  __shared__ float sKq[kC * LK], sKk[kC * LK], sQq[kC * LK];
  __shared__ float sG[kC * LK];   // G, then each token's log-decay gradient
  __shared__ __attribute__((aligned(16))) float sdO[kC * LV], sU[kC * LV], sdY[kC * LV];
  __shared__ float sB[kC * 17], sdT[kC * 17], sdM[kC * 17], sW[kC * 17], sT[kC * 20];
  __shared__ float sGm[DK], sGC[DK], sExtra[DK], sBeta[kC], sdb[kC];

  const int H = p.H;
  const int h = int(blockIdx.x % unsigned(H));
  const long long slot = blockIdx.x / unsigned(H);
  // the sequence whose slots hold this one: the last n with floor(bos_n / 16) + n <= slot
  auto first_tok = [&](int i) -> long long {
    return p.cu_seqlens ? (long long)p.cu_seqlens[i] : (long long)i * p.seq_len;
  };
  int lo = 0, hi = p.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first_tok(mid) / kC + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  const int n = lo;
  const long long bos = first_tok(n), eos = first_tok(n + 1);
  const long long c = slot - (bos / kC + n);
  if (c < 0 || bos + kC * c >= eos) return;
  const int cs = int(bos + kC * c);
  const int L = int(min((long long)kC, eos - cs));
  const size_t blk = size_t(slot) * H + h;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, q4 = lane >> 4, ln = lane & 15;
  const Tio* gq = reinterpret_cast<const Tio*>(p.q);
  const Tio* gk = reinterpret_cast<const Tio*>(p.k);
  const Tio* gdo = reinterpret_cast<const Tio*>(p.d_o);
  const float* wX0 = p.X0 + blk * kC * DV;
  const float* wdU = p.dU + blk * kC * DV;

  // 1. the in-chunk decays and the key/query tiles (one thread per key channel), and s dO,
  // U and dY (the other threads)
  if (tid < DK) {
    float G[kC], kv[kC], qv[kC];
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      const bool valid = t < L;
      const size_t row = (size_t(valid ? cs + t : cs) * H + h) * DK + tid;
      acc += fmaxf(p.g[row], p.g_min) * keep_f(valid);
      G[t] = acc;
      kv[t] = ld_keep(gk, row, valid);
      qv[t] = ld_keep(gq, row, valid);
    }
    const float gc = G[kC - 1];
    const float gm = 0.5f * (G[0] + gc);
    sGm[tid] = gm;
    sGC[tid] = gc;
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      const float em = __expf(G[t] - gm), emi = __expf(gm - G[t]);
      sKq[t * LK + tid] = kv[t] * em;
      sKk[t * LK + tid] = kv[t] * emi;
      sQq[t * LK + tid] = qv[t] * em;
      sG[t * LK + tid] = G[t];
    }
  } else {
    // a third of the threads per tile (DK of them, whole waves), four 4-element groups each
    const int u = tid - DK, tile = u / DK, v = u % DK;
    f32x4 x[4];
    if (tile == 0) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int e = v + DK * it, t = e / (DV / 4), j = 4 * (e % (DV / 4));
        x[it] = (p.scale * keep_f(t < L)) * ld4(gdo, (size_t(t < L ? cs + t : cs) * H + h) * DV + j);
      }
    } else {
      const float* src = (tile == 1 ? p.U : p.dY) + blk * kC * DV;
#pragma unroll
      for (int it = 0; it < 4; ++it) x[it] = ld4(src, 4 * size_t(v + DK * it));
    }
    float* dst = tile == 0 ? sdO : tile == 1 ? sU : sdY;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = v + DK * it, t = e / (DV / 4), j = 4 * (e % (DV / 4));
      *reinterpret_cast<f32x4*>(dst + t * LV + j) = x[it];
    }
    if (tid - DK < kC) sBeta[tid - DK] = tid - DK < L ? p.beta[size_t(cs + tid - DK) * H + h] : 0.f;
  }
  lds_barrier();

  // 2. the 16 x 16 matrices, one wave each
  if (w == 0) {
    // dT = dU Y^T with Y = diag(beta) X0 (value order j = 16 i + 4 q4 + e)
    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < DV / 16; ++i) {
      const f32x4 a = ld4(wdU, size_t(ln) * DV + 16 * i + 4 * q4);
      const f32x4 b = ld4(wX0, size_t(ln) * DV + 16 * i + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mma_f32(a[e], b[e], acc);
    }
    const float bl = sBeta[ln];
#pragma unroll
    for (int r = 0; r < 4; ++r) sdT[(4 * q4 + r) * 17 + ln] = acc[r] * bl;
  } else if (w == 1) {
    // dM = (s dO) U^T, on s <= t
    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < DV / 16; ++i) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(sdO + ln * LV + 16 * i + 4 * q4);
      const f32x4 b = *reinterpret_cast<const f32x4*>(sU + ln * LV + 16 * i + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mma_f32(a[e], b[e], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q4 + r;
      sdM[t * 17 + ln] = ln <= t ? acc[r] : 0.f;
    }
  } else if (w == 2) {
    // B and T = (I + diag(beta) B)^-1, as in the walks
    const f32x4 b = gram16<DK>(sKq, sKk, ln, q4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q4 + r;
      sB[t * 17 + ln] = ln < t ? b[r] : 0.f;
    }
    wave_sync();
    invert16(sB, sBeta, sT, lane);
  } else if (w == 3) {
    // first part of dbeta: X0 . dY per token, four lanes a token
    const int t = lane >> 2, part = lane & 3;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < DV / 16; ++i) {
      const int j = 16 * i + 4 * part;
      const f32x4 x = ld4(wX0, size_t(t) * DV + j);
      const f32x4 y = *reinterpret_cast<const f32x4*>(sdY + t * LV + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(x[e], y[e], acc);
    }
    acc = sum_xor2(sum_xor1(acc));
    if (part == 0) sdb[t] = acc;
  }
  lds_barrier();

  // 3. dA = -T^T dT T^T (strictly lower), dB = diag(beta) dA, and dbeta
  if (w == 0) {
    f32x4 P = zero4();   // dT T^T, k order m = 4 kk + q4
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int m = 4 * kk + q4;
      P = mma_f32(sdT[ln * 17 + m], sT[ln * 20 + m], P);
    }
    f32x4 A = zero4();   // T^T P, k order: P's own registers
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) A = mma_f32(sT[(4 * q4 + kk) * 20 + ln], P[kk], A);
    float db[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q4 + r;
      const float a = ln < t ? -A[r] : 0.f;
      sW[t * 17 + ln] = sBeta[t] * a;
      db[r] = sum_xor8(sum_mirror8(sum_xor2(sum_xor1(a * sB[t * 17 + ln]))));
    }
    if (ln == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * q4 + r;
        if (t < L) p.dbeta[size_t(cs + t) * H + h] = sdb[t] + db[r];
      }
    }
  }
  lds_barrier();

  // 4. per key channel c = 16 w + ln: the products with the chunk's states and the pairwise
  // terms, in accumulator layout (row t = 4 q4 + r)
  const int ch = 16 * w + ln;
  f32x4 aQ = zero4(), aKg = zero4(), aKh = zero4();
  float rs = 0.f;
  {
    const float* s0 = p.S0 + blk * DK * DV + size_t(ch) * DV;
    const float* ds = p.dS + blk * DK * DV + size_t(ch) * DV;
#pragma unroll 4
    for (int i = 0; i < DV / 16; ++i) {
      const int j = 16 * i + 4 * q4;
      const f32x4 bs = ld4(s0, j), bd = ld4(ds, j);
      const f32x4 ao = *reinterpret_cast<const f32x4*>(sdO + ln * LV + j);
      const f32x4 ay = *reinterpret_cast<const f32x4*>(sdY + ln * LV + j);
      const f32x4 au = *reinterpret_cast<const f32x4*>(sU + ln * LV + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        aQ = mma_f32(ao[e], bs[e], aQ);     // (s dO) S0^T
        aKg = mma_f32(ay[e], bs[e], aKg);   // dY S0^T
        aKh = mma_f32(au[e], bd[e], aKh);   // U dS^T
        rs = fmaf(bs[e], bd[e], rs);        // rowsum(S0 * dS)
      }
    }
  }
  rs = sum_xor32(sum_xor16(rs));
  f32x4 dqM = zero4(), dkAq = zero4(), dkMk = zero4(), dkAk = zero4();
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int m = 4 * kk + q4;
    const float kk_ = sKk[m * LK + ch], qq_ = sQq[m * LK + ch], kq_ = sKq[m * LK + ch];
    dqM = mma_f32(sdM[ln * 17 + m], kk_, dqM);    // dM (K e^-G)
    dkAq = mma_f32(sW[ln * 17 + m], kk_, dkAq);   // dB (K e^-G)
    dkMk = mma_f32(sdM[m * 17 + ln], qq_, dkMk);  // dM^T Q_G
    dkAk = mma_f32(sW[m * 17 + ln], kq_, dkAk);   // dB^T K_G
  }

  // 5. dq, dk, and each token's log-decay gradient (query side + key side -)
  const float gm = sGm[ch], gc = sGC[ch];
  float khs = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * q4 + r;
    const bool valid = t < L;
    const float G = sG[t * LK + ch];
    const float eg = __expf(G), em = __expf(G - gm), emi = __expf(gm - G), eh = __expf(gc - G);
    const size_t row = (size_t(valid ? cs + t : cs) * H + h) * DK + ch;
    const float qv = ld_keep(gq, row, valid), kv = ld_keep(gk, row, valid);
    const float dq = aQ[r] * eg + dqM[r] * em;
    const float dkq = -sBeta[t] * aKg[r] * eg + dkAq[r] * em;
    const float dkk = (dkAk[r] + dkMk[r]) * emi;
    const float dkh = aKh[r] * eh;
    if (valid) {
      p.dq[row] = dq;
      p.dk[row] = dkq + dkk + dkh;
    }
    sG[t * LK + ch] = valid ? qv * dq + kv * (dkq - dkk - dkh) : 0.f;
    khs = fmaf(kv, dkh, khs);
  }
  khs = sum_xor32(sum_xor16(khs));
  // the gradient of G_C: the leaving state's decay and the key-side factors e^(G_C - G)
  if (q4 == 0) sExtra[ch] = khs + __expf(gc) * rs;
  lds_barrier();

  // 6. dg_t = dL/dG_C + sum over t' >= t of the per-token gradients (0 where g is floored)
  if (tid < DK) {
    float run = sExtra[tid];
    for (int t = kC - 1; t >= 0; --t) {
      run += sG[t * LK + tid];
      if (t < L) {
        const size_t row = (size_t(cs + t) * H + h) * DK + tid;
        p.dg[row] = p.g[row] > p.g_min ? run : 0.f;
      }
    }
  }
}

template <typename Tio, int DK>
static hipError_t launch_cbwd(const CBwdParams& p, hipStream_t stream) {
  const dim3 walk((p.n_units + 7) / 8 * 8 * p.n_ct);
  hipLaunchKernelGGL((cbwd_fwd_kernel<Tio, DK>), walk, dim3(64), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((cbwd_rev_kernel<Tio, DK>), walk, dim3(64), 0, stream, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((cbwd_grad_kernel<Tio, DK>), dim3(unsigned(p.n_slots * p.H)), dim3(4 * DK),
                     0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd_mfma(const CBwdParams& p, int io_dtype, int dk, hipStream_t stream) {
  if (p.n_ct != dk / 16 || p.n_units != p.n_seqs * p.H || p.H < 1 || p.n_seqs < 1 ||
      p.n_slots != cbwd_slots(p.T, p.n_seqs) || p.n_slots * p.H > 0x7fffffffLL)
    return hipErrorInvalidValue;
  if (dk == 128) return io_dtype == 1 ? launch_cbwd<__bf16, 128>(p, stream)
                                      : launch_cbwd<float, 128>(p, stream);
  if (dk == 64) return io_dtype == 1 ? launch_cbwd<__bf16, 64>(p, stream)
                                     : launch_cbwd<float, 64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
