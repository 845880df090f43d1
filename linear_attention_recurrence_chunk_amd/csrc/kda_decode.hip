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
// Work decomposition: one workgroup (4 waves) per (request, head). The head's fp32 state
// (d_k x d_v) is read from HBM once, lives in registers for every token of the loop (wave w
// owns value columns [32w, 32w + 32); lane (row group rg = lane / 8, column group cg =
// lane % 8) holds rows 16 rg .. 16 rg + 15 of columns 4 cg .. 4 cg + 3), and is written back
// twice: after the replayed drafts (state_acc) and after the bonus token (state, in place).
// Column sums over the 128 key rows are reduced inside the wave (lanes that share cg), so the
// recurrence needs no LDS traffic and no barrier.
//
// Per token, with the state columns independent:
//   k_s = sum_i (a_i k_i) S_ij,  q_s = sum_i (a_i q_i) S_ij     (both on the old state)
//   e_j = v_j - k_s;  S_ij <- a_i S_ij + (beta k_i) e_j;  o_j = q_s + beta (q . k) e_j
// which equals decaying first, correcting, then reading out S^T q. The operation order is
// fixed and identical for replayed, bonus and draft tokens, so a replayed state is
// bit-identical to the state the same tokens reach one launch at a time.
#include "kda_common.h"
#include "kda_decode.h"

namespace kda {

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

struct RawToken {
  float a, b, g, z, beta;
};

// Raw inputs a thread needs for token t of its request: replay slots 1..n_acc of the
// previous window, then slots 0..n_new-1 of the current one. Threads of the q/k role read
// q and k of their channel, threads of the v role read v, g, z and (channel 0) beta.
template <int D>
__device__ __forceinline__ RawToken load_raw(const DecodeParams& p, int r, int t, int n_acc,
                                             int ch, bool role_qk, bool role_v) {
  const bool replay = t < n_acc;
  const int slot = replay ? t + 1 : t - n_acc;
  const int slots = replay ? p.prev_slots : p.cur_slots;
  const size_t tok = (size_t(r) * slots + slot) * p.H + blockIdx.x % p.H;
  RawToken x = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (role_qk) {
    x.a = (float)(replay ? p.prev_q : p.cur_q)[tok * D + ch];
    x.b = (float)(replay ? p.prev_k : p.cur_k)[tok * D + ch];
  } else if (role_v) {
    x.a = (float)(replay ? p.prev_v : p.cur_v)[tok * D + ch];
    x.g = (float)(replay ? p.prev_g : p.cur_g)[tok * D + ch];
    if (!replay) x.z = (float)p.cur_z[tok * D + ch];
    if (ch == 0) x.beta = (float)(replay ? p.prev_beta : p.cur_beta)[tok];
  }
  return x;
}

template <int D, int W, typename Tout>
__global__ __launch_bounds__(256) void decode_replay_kernel(DecodeParams p) {
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(W >= 1 && W <= 4, "convolution width");
  constexpr int RPL = D / 8;          // rows of S per lane
  constexpr int CPW = D / 4;          // value columns per wave
  constexpr int CPL = CPW / 8;        // value columns per lane
  constexpr int C3 = 3 * D;           // convolved channels q, k, v

  const int rh = blockIdx.x;
  const int r = rh / p.H;
  const int h = rh % p.H;
  const int H = p.H;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int rg = lane >> 3;
  const int cg = lane & 7;
  const int col0 = CPW * w + CPL * cg;   // first value column of this lane
  const int row0 = RPL * rg;             // first key row of this lane

  // per-token values shared through LDS, double-buffered by token parity
  __shared__ float s_q[2][D], s_k[2][D], s_a[2][D], s_v[2][D], s_z[2][D];
  __shared__ float s_red[2][4][3];      // per wave: sum q^2, sum k^2, sum q k
  __shared__ float s_beta[2];
  __shared__ float s_osq[2][4];         // per wave: sum o^2 over its columns

  // ---- state tile into registers
  const size_t sbase = (size_t(r) * H + h) * D * D;
  float S[RPL][CPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const float* src = p.state + sbase + size_t(row0 + i) * D + col0;
    if constexpr (CPL == 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = x[j];
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) S[i][j] = src[j];
    }
  }

  // ---- input-stage role: threads [0, D) own q and k channel tid; [D, 2D) own v, g and z
  // channel tid - D. Each keeps the causal-convolution tail of its channels in registers.
  const bool role_qk = tid < D;
  const bool role_v = tid >= D && tid < 2 * D;
  const int ch = role_qk ? tid : tid - D;
  float tail_a[3] = {0.f, 0.f, 0.f}, tail_b[3] = {0.f, 0.f, 0.f};
  float wa[4] = {0.f, 0.f, 0.f, 0.f}, wb[4] = {0.f, 0.f, 0.f, 0.f};
  const size_t tbase = (size_t(r) * H + h) * C3 * (W - 1);
  const size_t wbase = size_t(h) * C3 * W;
  if (role_qk || role_v) {
    const int ca = role_qk ? ch : 2 * D + ch;   // q channel or v channel
    const int cb = ch + D;                      // k channel (q/k role only)
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

  int n_acc = p.n_acc[r];
  n_acc = n_acc < 0 ? 0 : (n_acc > p.prev_slots - 1 ? p.prev_slots - 1 : n_acc);
  const int n_tok = n_acc + p.n_new;

  if (n_acc == 0 && p.state_acc) {
    // no accepted drafts: the accepted state is the committed entering state
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      float* dst = p.state_acc + sbase + size_t(row0 + i) * D + col0;
#pragma unroll
      for (int j = 0; j < CPL; ++j) dst[j] = S[i][j];
    }
  }

  RawToken nx = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (n_tok > 0) nx = load_raw<D>(p, r, 0, n_acc, ch, role_qk, role_v);

  for (int t = 0; t < n_tok; ++t) {
    const int buf = t & 1;
    const bool replay = t < n_acc;
    const bool output = !replay;
    const float xa = nx.a, xb = nx.b, xg = nx.g, xz = nx.z, xbeta = nx.beta;
    if (t + 1 < n_tok) nx = load_raw<D>(p, r, t + 1, n_acc, ch, role_qk, role_v);

    // ---------------- input stage: causal conv, SiLU, gates -------------------------------
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    if (role_qk) {
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
      s_q[buf][ch] = ya;
      s_k[buf][ch] = yb;
      sq = ya * ya;
      sk = yb * yb;
      sqk = ya * yb;
    } else if (role_v) {
      float ya = wa[W - 1] * xa;
#pragma unroll
      for (int m = 0; m < W - 1; ++m) ya += wa[m] * tail_a[m];
#pragma unroll
      for (int m = 0; m + 1 < W - 1; ++m) tail_a[m] = tail_a[m + 1];
      if constexpr (W > 1) tail_a[W - 2] = xa;
      if (p.act) ya = ya * sigmoidf_(ya);
      s_v[buf][ch] = ya;
      // exp(max(-softplus(x), g_min)) = max(sigmoid(-x), e^{g_min})
      s_a[buf][ch] = fmaxf(1.f / (1.f + expf(xg)), p.decay_floor);
      s_z[buf][ch] = output ? sigmoidf_(xz) : 0.f;
      if (ch == 0) s_beta[buf] = sigmoidf_(xbeta);
    }
    // norms of q and k: reduce inside the wave, one partial per wave
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sq += __shfl_xor(sq, off);
      sk += __shfl_xor(sk, off);
      sqk += __shfl_xor(sqk, off);
    }
    if (lane == 0) {
      s_red[buf][w][0] = sq;
      s_red[buf][w][1] = sk;
      s_red[buf][w][2] = sqk;
    }
    __syncthreads();

    // ---------------- recurrence on this lane's block of S --------------------------------
    const float nq2 = s_red[buf][0][0] + s_red[buf][1][0] + s_red[buf][2][0] + s_red[buf][3][0];
    const float nk2 = s_red[buf][0][1] + s_red[buf][1][1] + s_red[buf][2][1] + s_red[buf][3][1];
    const float nqk = s_red[buf][0][2] + s_red[buf][1][2] + s_red[buf][2][2] + s_red[buf][3][2];
    const float iq = 1.f / sqrtf(nq2 + p.eps_l2);
    const float ik = 1.f / sqrtf(nk2 + p.eps_l2);
    const float beta = s_beta[buf];
    const float qk = nqk * iq * ik;    // (q . k) of the normalised vectors
    float ak[RPL], aq[RPL], bk[RPL], av[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const float a = s_a[buf][row0 + i];
      const float kn = s_k[buf][row0 + i] * ik;
      av[i] = a;
      ak[i] = a * kn;
      aq[i] = a * (s_q[buf][row0 + i] * iq);
      bk[i] = beta * kn;
    }
    float ks[CPL], qs[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      ks[j] = 0.f;
      qs[j] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        ks[j] = fmaf(ak[i], S[i][j], ks[j]);
        qs[j] = fmaf(aq[i], S[i][j], qs[j]);
      }
    }
    // sum over the 8 row groups (lanes cg, cg + 8, ..., cg + 56), fixed butterfly order
#pragma unroll
    for (int off = 8; off <= 32; off <<= 1) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        ks[j] += __shfl_xor(ks[j], off);
        qs[j] += __shfl_xor(qs[j], off);
      }
    }
    float e[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) e[j] = s_v[buf][col0 + j] - ks[j];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) S[i][j] = fmaf(bk[i], e[j], av[i] * S[i][j]);
    }

    float ov[CPL];
    if (output) {
      float osq = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        ov[j] = p.scale * fmaf(beta * qk, e[j], qs[j]);
        osq += ov[j] * ov[j];
      }
      // each column is held by 8 lanes; count it once (row group 0)
      osq = rg == 0 ? osq : 0.f;
#pragma unroll
      for (int off = 1; off <= 4; off <<= 1) osq += __shfl_xor(osq, off);
      if (lane == 0) s_osq[buf][w] = osq;
    }
    if (replay && t == n_acc - 1 && p.state_acc) {
      // state after the accepted drafts
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        float* dst = p.state_acc + sbase + size_t(row0 + i) * D + col0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) dst[j] = S[i][j];
      }
    }
    __syncthreads();

    if (output) {
      const float tot = s_osq[buf][0] + s_osq[buf][1] + s_osq[buf][2] + s_osq[buf][3];
      const float rinv = 1.f / sqrtf(tot / float(D) + p.eps_rms);
      if (rg == 0) {
        const int j_out = t - n_acc;
        Tout* dst = reinterpret_cast<Tout*>(p.o) + ((size_t(r) * p.n_new + j_out) * H + h) * D + col0;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          dst[j] = from_f32<Tout>(ov[j] * rinv * p.norm_w[col0 + j] * s_z[buf][col0 + j]);
      }
      if (t == n_acc) {
        // bonus token: the new committed state and convolution tail
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
          float* dst = p.state + sbase + size_t(row0 + i) * D + col0;
#pragma unroll
          for (int j = 0; j < CPL; ++j) dst[j] = S[i][j];
        }
        if (role_qk || role_v) {
          const int ca = role_qk ? ch : 2 * D + ch;
          const int cb = ch + D;
#pragma unroll
          for (int m = 0; m < W - 1; ++m) {
            p.conv_tail[tbase + size_t(ca) * (W - 1) + m] = tail_a[m];
            if (role_qk) p.conv_tail[tbase + size_t(cb) * (W - 1) + m] = tail_b[m];
          }
        }
      }
    }
  }
}

template <int D, int W>
static hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.out_f32)
    hipLaunchKernelGGL((decode_replay_kernel<D, W, float>), dim3(p.R * p.H), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_replay_kernel<D, W, __bf16>), dim3(p.R * p.H), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
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
