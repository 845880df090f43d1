// Ordered scan of segment summaries for the segment-parallel prefill.
//
// "Noyaux KDA et FlashKDA", section "Le parallélisme de contexte intra-appareil": each
// segment's state transition is evaluated without its incoming state and the transitions
// are then composed exactly to recover every segment's initial state; AMD blog "Dentro de los
// esfuerzos de optimización de Kimi K3", section 5: an ordered scan of the group summaries
// gives each group's initial state, after which the groups replay their tokens in parallel.
//
// A summary is the affine map S_out = P S_in + Q of one segment (P: d_k x d_k, Q: d_k x d_v,
// stored side by side as [P | Q]). The scan walks the segments of one sequence in order:
//   S_in(0) = h0,  S_in(j + 1) = P_j S_in(j) + Q_j,  final state = S_in(n_seg).
// Value columns stay independent, so one workgroup (4 waves x 16 columns) owns a 64-column
// slice of one (sequence, head) and keeps it in MFMA accumulators. For bf16 inputs P_j is
// staged through LDS as a hi + lo pair of bf16 values and multiplied with three bf16 MFMAs per
// product (hi*hi + lo*hi + hi*lo, ~16 mantissa bits), S_in(j) split the same way in
// registers. For fp32 inputs (held to 1e-4 x RMS) P_j stays fp32 in LDS and the products run
// on fp32 MFMA (v_mfma_f32_16x16x4_f32), with S_in(j) as its own operand.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <int DK, bool kF32>
__global__ __launch_bounds__(256) void segment_scan_kernel(ScanParams p) {
  using Pol = PolBF16;
  using Frag = PolBF16::Frag;
  constexpr int LDP = DK + 8;
  constexpr int LDF = DK + 1;   // fp32 rows: 16 consecutive rows fall in distinct banks
  constexpr int NS = DK / 32;
  constexpr int NTD = DK / 16;
  // bf16: P as (hi, lo) pairs; fp32: P itself in the same bytes
  constexpr size_t kPBytes = kF32 ? size_t(DK) * LDF * 4 : size_t(2) * DK * LDP * 2;
  __shared__ __attribute__((aligned(16))) char smem[kPBytes];
  __bf16* sPh = reinterpret_cast<__bf16*>(smem);
  __bf16* sPl = sPh + DK * LDP;
  float* sPf = reinterpret_cast<float*>(smem);

  const int n_vt = p.dv / 64;
  const int vt = blockIdx.x % n_vt;
  const int nh = blockIdx.x / n_vt;       // n * H + h
  const int n = nh / p.H;
  const int h = nh % p.H;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int q4 = lane >> 4;
  const int ln = lane & 15;
  const int DV = p.dv;
  const int ldpq = DK + DV;
  const int col = vt * 64 + 16 * w + ln;  // value column of this lane

  f32x4 S[NTD];
  const float* h0 = p.h0 ? p.h0 + size_t(nh) * DK * DV : nullptr;
#pragma unroll
  for (int t = 0; t < NTD; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) S[t][e] = h0 ? h0[size_t(16 * t + 4 * q4 + e) * DV + col] : 0.f;

  int bos, eos;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
  } else {
    bos = n * p.seq_len;
    eos = bos + p.seq_len;
  }
  const long long nc = (eos - bos + 63) / 64;

  // P_j and Q_j are read one step ahead into registers (16-byte pieces of the thread's rows of
  // P; Q in the accumulator layout of S), so their HBM latency hides under the previous step
  // (a load of Q_j in its own step would also be ordered after that step's S_in stores).
  constexpr int kPPT = DK * DK / (4 * 256);   // f32x4 pieces of P per thread
  f32x4 pr[kPPT], qn[NTD];
  auto fetch = [&](int j) {
    const float* pq = p.pq + ((size_t(n) * p.n_seg + j) * p.H + h) * DK * ldpq;
#pragma unroll
    for (int i = 0; i < kPPT; ++i) {
      const int idx = (tid + 256 * i) * 4;
      pr[i] = *reinterpret_cast<const f32x4*>(pq + size_t(idx / DK) * ldpq + idx % DK);
    }
#pragma unroll
    for (int t = 0; t < NTD; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) qn[t][e] = pq[size_t(16 * t + 4 * q4 + e) * ldpq + DK + col];
  };
  if (p.n_seg > 0) fetch(0);

  for (int j = 0; j < p.n_seg; ++j) {
    const size_t seg = (size_t(n) * p.n_seg + j) * p.H + h;
    // entering state of segment j
    float* sin = p.sin + seg * DK * DV;
#pragma unroll
    for (int t = 0; t < NTD; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) sin[size_t(16 * t + 4 * q4 + e) * DV + col] = S[t][e];
    // a segment without tokens is the identity map: the state passes through unchanged
    // (its summary was never written; the registers are refilled with the next one)
    if ((j * nc) / p.n_seg == ((j + 1) * nc) / p.n_seg) {
      if (j + 1 < p.n_seg) fetch(j + 1);
      continue;
    }

    // P_j into LDS, row = key channel: (hi, lo) bf16, or fp32
#pragma unroll
    for (int i = 0; i < kPPT; ++i) {
      const int idx = (tid + 256 * i) * 4;
      const int r = idx / DK, c = idx % DK;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (kF32) {
          sPf[r * LDF + c + e] = pr[i][e];
        } else {
          const __bf16 hi = (__bf16)pr[i][e];
          sPh[r * LDP + c + e] = hi;
          sPl[r * LDP + c + e] = (__bf16)(pr[i][e] - (float)hi);
        }
      }
    }
    lds_barrier();

    // S <- P_j S + Q_j
    if constexpr (kF32) {
      // k-slice s of the fp32 MFMA takes key rows 16 (s / 4) + 4 q4 + s % 4: the B operand
      // is then this lane's own accumulator register S[s / 4][s % 4]
      f32x4 Sold[NTD];
#pragma unroll
      for (int t = 0; t < NTD; ++t) Sold[t] = S[t];
#pragma unroll
      for (int t = 0; t < NTD; ++t) S[t] = qn[t];
      if (j + 1 < p.n_seg) fetch(j + 1);
#pragma unroll
      for (int t = 0; t < NTD; ++t) {
        const float* prow = sPf + (16 * t + ln) * LDF + 4 * q4;
#pragma unroll
        for (int s2 = 0; s2 < DK / 4; ++s2)
          S[t] = mma_f32(prow[16 * (s2 >> 2) + (s2 & 3)], Sold[s2 >> 2][s2 & 3], S[t]);
      }
    } else {
      Frag Sh[NS], Sl[NS];
#pragma unroll
      for (int pp = 0; pp < NS; ++pp) Pol::from_acc_split(S, pp, Sh[pp], Sl[pp]);
#pragma unroll
      for (int t = 0; t < NTD; ++t) S[t] = qn[t];
      if (j + 1 < p.n_seg) fetch(j + 1);
#pragma unroll
      for (int pp = 0; pp < NS; ++pp) {
#pragma unroll
        for (int t = 0; t < NTD; ++t) {
          const Frag ah = Pol::load(sPh, LDP, 16 * t + ln, pp, q4);
          S[t] = Pol::mma(ah, Sh[pp], S[t]);
          S[t] = Pol::mma(Pol::load(sPl, LDP, 16 * t + ln, pp, q4), Sh[pp], S[t]);
          S[t] = Pol::mma(ah, Sl[pp], S[t]);
        }
      }
    }
    lds_barrier();
  }
  if (p.ht) {
    float* ht = p.ht + size_t(nh) * DK * DV;
#pragma unroll
    for (int t = 0; t < NTD; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) ht[size_t(16 * t + 4 * q4 + e) * DV + col] = S[t][e];
  }
}

hipError_t launch_segment_scan(const ScanParams& p, int dk, hipStream_t stream) {
  if (p.N < 1 || p.H < 1 || p.n_seg < 1 || p.dv < 64 || p.dv % 64 || !p.pq || !p.sin)
    return hipErrorInvalidValue;
  const dim3 grid(p.N * p.H * (p.dv / 64));
  if (dk == 128 && p.f32)
    hipLaunchKernelGGL((segment_scan_kernel<128, true>), grid, dim3(256), 0, stream, p);
  else if (dk == 128)
    hipLaunchKernelGGL((segment_scan_kernel<128, false>), grid, dim3(256), 0, stream, p);
  else if (dk == 64 && p.f32)
    hipLaunchKernelGGL((segment_scan_kernel<64, true>), grid, dim3(256), 0, stream, p);
  else if (dk == 64)
    hipLaunchKernelGGL((segment_scan_kernel<64, false>), grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kda
