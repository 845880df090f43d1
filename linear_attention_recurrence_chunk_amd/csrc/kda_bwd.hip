// Backward of the KDA recurrence on gfx950: the gradients of kda_chunk_fwd's outputs o and
// final state with respect to q, k, v, g, beta and h0.
//
// The pages give the forward only ("Noyaux KDA et FlashKDA", section "FlashKDA : le noyau par
// blocs": FlashKDA serves training as well as prefill). These kernels differentiate the same
// per-token update, in reverse token order:
//
//   forward   a = exp(max(g_t, g_min));  S' = diag(a) S_prev;  e = v_t - S'^T k_t;
//             S = S' + beta_t k_t e^T;  o_t = scale S^T q_t
//   backward  D += scale q_t do_t^T;  dq_t = scale S do_t;  de = beta_t D^T k_t;  dv_t = de;
//             dk_t = beta_t D e - S' de;  dbeta_t = k_t^T D e;  D' = D - k_t de^T;
//             dg_t = a (rowsum(S_prev * D')) where g_t > g_min, else 0;  D = diag(a) D'
//
// with D = dL/dS starting from dL/d(final state); dh0 is D at the sequence start.
//
// Value columns of S and D never mix, so one workgroup owns a 16-column tile of one (sequence,
// head): 4 waves x 64 lanes, lane = (row group, column), each thread DK / 16 consecutive key
// rows of one column. Everything is fp32 vector arithmetic (no matrix cores: one token at a
// time). Per workgroup:
//   1. a forward pass over the sequence stores the state at every 8th token (the workspace's
//      checkpoints; fp32, so the states match the per-token definition to rounding);
//   2. the sub-chunks of 8 tokens are taken in reverse: the 9 states of one are recomputed
//      from its checkpoint into registers, then its tokens are differentiated in reverse.
// Sums over value columns (dq, dk, dg and dbeta) are partial per tile; a second kernel adds
// the tiles in a fixed order, so results are deterministic. dv and dh0 are complete per tile.
#include "kda_bwd.h"
#include "kda_chunk_io.h"
#include "kda_common.h"

namespace kda {

// RPT consecutive elements of one row of an io-type tensor, as fp32
template <typename T, int RPT>
__device__ __forceinline__ void load_rows(const T* src, float (&x)[RPT]) {
  if constexpr (sizeof(T) == 2) {
    static_assert(RPT % 4 == 0, "bf16 rows load in quads");
#pragma unroll
    for (int i = 0; i < RPT; i += 4) {
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(src + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[i + e] = (float)a[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < RPT; i += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(src + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[i + e] = a[e];
    }
  }
}

// Sum over the 16 lanes of a DPP row (the 16 columns of a row group) of RPT row values,
// scattered: lane l ends with the total of row rows_reduced_row(l) (lanes that share bits 3..1
// for RPT = 8, bits 3..2 for RPT = 4, hold the same row and the same bits).
template <int RPT>
__device__ __forceinline__ float rows_reduce(const float (&x)[RPT], int lane) {
  const bool h3 = (lane & 8) != 0, h2 = (lane & 4) != 0;
  constexpr int kA = RPT / 2;
  float a[kA];
#pragma unroll
  for (int i = 0; i < kA; ++i) {
    // partner l ^ 8 (row rotation by eight): keep one half of the rows, send the other
    const float keep = h3 ? x[kA + i] : x[i];
    const float send = h3 ? x[i] : x[kA + i];
    a[i] = keep + dpp_mov<0x128>(send);
  }
  constexpr int kB = kA / 2;
  float b[kB];
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    // partner 7 - l inside each eight (row half mirror): lanes 0-3 keep the lower half
    const float keep = h2 ? a[kB + i] : a[i];
    const float send = h2 ? a[i] : a[kB + i];
    b[i] = keep + dpp_mov<0x141>(send);
  }
  float c;
  if constexpr (kB == 2) {
    const bool h1 = (lane & 2) != 0;
    const float keep = h1 ? b[1] : b[0];
    const float send = h1 ? b[0] : b[1];
    c = keep + quad_perm<kQuadXor2>(send);
  } else {
    static_assert(kB == 1, "rows per thread: 4 or 8");
    c = sum_xor2(b[0]);
  }
  return sum_xor1(c);
}
template <int RPT>
__device__ __forceinline__ int rows_reduced_row(int lane) {
  if constexpr (RPT == 8) return ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 + ((lane >> 1) & 1);
  else return ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
}
// the one lane of each group holding the same row that writes it
template <int RPT>
__device__ __forceinline__ bool rows_writer(int lane) {
  return RPT == 8 ? (lane & 1) == 0 : (lane & 3) == 0;
}

template <typename Tio, int DK>
__global__ __launch_bounds__(256, 3) void chunk_bwd_tile_kernel(BwdParams p) {
  constexpr int RPT = DK / 16;   // key rows per thread
  constexpr int DV = DK;
  constexpr int SUB = kBwdSub;
  __shared__ float sRed[2][4][16];

  int ct;
  const int unit = block_unit(blockIdx.x, p.n_ct, &ct);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int h = unit % H;
  const int n = unit / H;
  int bos, eos;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
  } else {
    bos = n * p.seq_len;
    eos = bos + p.seq_len;
  }
  const int len = eos - bos;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;
  const int r0 = (4 * w + (lane >> 4)) * RPT;   // first key row of this thread
  const int col = 16 * ct + c;                  // its value column
  const float gmin = p.g_min;
  const Tio* gq = reinterpret_cast<const Tio*>(p.q);
  const Tio* gk = reinterpret_cast<const Tio*>(p.k);
  const Tio* gv = reinterpret_cast<const Tio*>(p.v);
  const Tio* gdo = reinterpret_cast<const Tio*>(p.d_o);
  const size_t state_off = (size_t(n) * H + h) * DK * DV;   // [N, H, DK, DV] of this unit

  // sum over all 128 (or 64) key rows of a column: the thread's rows, the wave's four row
  // groups (lanes c, c + 16, c + 32, c + 48), then the four waves through LDS, added in a
  // fixed order so every thread of the column gets the same bits
  int par = 0;
  auto col_reduce = [&](float x) -> float {
    x = sum_xor32(sum_xor16(x));
    if (lane < 16) sRed[par][w][lane] = x;
    lds_barrier();
    const float s = ((sRed[par][0][c] + sRed[par][1][c]) + sRed[par][2][c]) + sRed[par][3][c];
    par ^= 1;
    return s;
  };

  // one token's inputs for this thread, as loaded: every loop below loads the next token's
  // while the current one is computed, so a step does not wait for memory
  struct In {
    float g[RPT], k[RPT], beta, v;
  };
  auto load_in = [&](int t, In& x) {
    const size_t row = (size_t(t) * H + h) * DK + r0;
#pragma unroll
    for (int i = 0; i < RPT; i += 4) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(p.g + row + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) x.g[i + e] = a4[e];
    }
    load_rows<Tio, RPT>(gk + row, x.k);
    x.beta = p.beta[size_t(t) * H + h];
    x.v = to_f32(gv[(size_t(t) * H + h) * DV + col]);
  };
  // the reverse step's extra inputs: q rows and the output gradient of the column
  struct InB {
    float q[RPT], d_o;
  };
  auto load_inb = [&](int t, InB& x) {
    load_rows<Tio, RPT>(gq + (size_t(t) * H + h) * DK + r0, x.q);
    x.d_o = to_f32(gdo[(size_t(t) * H + h) * DV + col]);
  };
  // one token's decays and keys
  struct Tok {
    float a[RPT], k[RPT], beta;
    bool live[RPT];
  };
  auto decode = [&](const In& in, Tok& x) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      x.live[i] = in.g[i] > gmin;
      x.a[i] = __expf(fmaxf(in.g[i], gmin));
      x.k[i] = in.k[i];
    }
    x.beta = in.beta;
  };
  // S <- S' + beta k e^T for one token; returns e (this thread's column)
  auto fwd_step = [&](const In& in, const float (&Sin)[RPT], float (&Sout)[RPT]) -> float {
    Tok x;
    decode(in, x);
    const float vc = in.v;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      Sout[i] = x.a[i] * Sin[i];
      part = fmaf(Sout[i], x.k[i], part);
    }
    const float e = vc - col_reduce(part);
#pragma unroll
    for (int i = 0; i < RPT; ++i) Sout[i] = fmaf(x.beta * x.k[i], e, Sout[i]);
    return e;
  };

  // ---- 1. forward pass: the state at the start of every sub-chunk into the checkpoints
  const long long slot0 = (long long)(bos / SUB) + n;   // first checkpoint slot of the sequence
  auto ckpt_ptr = [&](int j) {
    return p.ckpt + ((size_t(slot0 + j) * H + h) * DK + r0) * DV + col;
  };
  float S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = p.h0 ? p.h0[state_off + size_t(r0 + i) * DV + col] : 0.f;
  const int nsub = (len + SUB - 1) / SUB;
  In cur;
  if (len > 0) load_in(bos, cur);
  for (int j = 0; j < nsub; ++j) {
    float* cp = ckpt_ptr(j);
#pragma unroll
    for (int i = 0; i < RPT; ++i) cp[size_t(i) * DV] = S[i];
    const int t0 = bos + SUB * j, t1 = min(eos, t0 + SUB);
    for (int t = t0; t < t1; ++t) {
      In nxt;
      if (t + 1 < eos) load_in(t + 1, nxt);
      float Sn[RPT];
      fwd_step(cur, S, Sn);
#pragma unroll
      for (int i = 0; i < RPT; ++i) S[i] = Sn[i];
      cur = nxt;
    }
  }

  // ---- 2. reverse over the sub-chunks
  float D[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    D[i] = p.dht ? p.dht[state_off + size_t(r0 + i) * DV + col] : 0.f;
  const int rsel = rows_reduced_row<RPT>(lane);
  const bool writer = rows_writer<RPT>(lane);
  const size_t part_stride = size_t(p.n_ct) * p.T * H * DK;   // from one partial sum to the next
  for (int j = nsub - 1; j >= 0; --j) {
    const int t0 = bos + SUB * j;
    const int L = min(SUB, eos - t0);
    float Ss[SUB + 1][RPT];   // Ss[i]: the state after i tokens of the sub-chunk
    float es[SUB];
    {
      const float* cp = ckpt_ptr(j);
#pragma unroll
      for (int i = 0; i < RPT; ++i) Ss[0][i] = cp[size_t(i) * DV];
    }
    {
      In in;
      load_in(t0, in);
      static_for<0, SUB>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (i < L) {
          In nxt;
          if (i + 1 < L) load_in(t0 + i + 1, nxt);
          es[i] = fwd_step(in, Ss[i], Ss[i + 1]);
          in = nxt;
        }
      });
    }
    static_for<0, SUB>([&](auto ic) {
      constexpr int i = SUB - 1 - decltype(ic)::value;
      if (i >= L) return;
      const int t = t0 + i;
      // (loaded at the step: the sub-chunk's states leave no registers for a look-ahead)
      In inr;
      InB inb;
      load_in(t, inr);
      load_inb(t, inb);
      Tok x;
      decode(inr, x);
      float qv[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) qv[r] = inb.q[r];
      const float doc = inb.d_o;
      const float e = es[i];
      float rq[RPT], rk[RPT], ra[RPT];
      float pde = 0.f, pb = 0.f;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        D[r] = fmaf(p.scale * qv[r], doc, D[r]);
        rq[r] = p.scale * Ss[i + 1][r] * doc;
        pde = fmaf(D[r], x.k[r], pde);
        pb = fmaf(x.k[r] * D[r], e, pb);
      }
      const float de = x.beta * col_reduce(pde);
      if (w == 0 && lane < 16) p.dv[(size_t(t) * H + h) * DV + col] = de;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const float sp = x.a[r] * Ss[i][r];                  // S'
        rk[r] = x.beta * D[r] * e - sp * de;                 // dk's terms of this column
        const float dp = D[r] - x.k[r] * de;                 // D'
        ra[r] = x.live[r] ? dp * Ss[i][r] : 0.f;             // dg / a's terms
        D[r] = x.a[r] * dp;
      }
      const float sq = rows_reduce<RPT>(rq, lane);
      const float sk = rows_reduce<RPT>(rk, lane);
      const float sa = rows_reduce<RPT>(ra, lane);
      if (writer) {
        const size_t o = ((size_t(ct) * p.T + t) * H + h) * DK + r0 + rsel;
        p.part[o] = sq;
        p.part[part_stride + o] = sk;
        p.part[2 * part_stride + o] = sa;
      }
      // dbeta: k^T D e over this wave's rows and columns
      pb = sum_xor32(sum_xor16(sum_xor8(sum_mirror8(sum_xor2(sum_xor1(pb))))));
      if (lane == 0) p.part_beta[(size_t(4 * ct + w) * p.T + t) * H + h] = pb;
    });
  }
  if (p.dh0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) p.dh0[state_off + size_t(r0 + i) * DV + col] = D[i];
  }
}

// dq, dk, dg (sums over the tiles, in tile order) and dbeta; one thread per (token, head) and
// four consecutive key rows, 16-byte loads and stores
template <int DK>
__global__ __launch_bounds__(256) void chunk_bwd_reduce_kernel(BwdParams p) {
  const long long idx4 = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total4 = p.T * p.H * DK / 4;
  if (idx4 >= total4) return;
  const long long idx = 4 * idx4;
  const long long th = idx / DK;   // t * H + h
  const size_t stride = size_t(p.n_ct) * p.T * p.H * DK;
  const size_t tile = size_t(p.T) * p.H * DK;
  f32x4 sq = zero4(), sk = zero4(), sa = zero4();
  for (int ct = 0; ct < p.n_ct; ++ct) {
    const size_t o = size_t(ct) * tile + size_t(idx);
    sq += *reinterpret_cast<const f32x4*>(p.part + o);
    sk += *reinterpret_cast<const f32x4*>(p.part + stride + o);
    sa += *reinterpret_cast<const f32x4*>(p.part + 2 * stride + o);
  }
  const f32x4 g = *reinterpret_cast<const f32x4*>(p.g + idx);
  f32x4 dg;
#pragma unroll
  for (int e = 0; e < 4; ++e) dg[e] = g[e] > p.g_min ? __expf(g[e]) * sa[e] : 0.f;
  *reinterpret_cast<f32x4*>(p.dq + idx) = sq;
  *reinterpret_cast<f32x4*>(p.dk + idx) = sk;
  *reinterpret_cast<f32x4*>(p.dg + idx) = dg;
  if (idx % DK == 0) {
    float sb = 0.f;
    for (int i = 0; i < 4 * p.n_ct; ++i) sb += p.part_beta[size_t(i) * p.T * p.H + size_t(th)];
    p.dbeta[th] = sb;
  }
}

template <typename Tio, int DK>
static hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  const dim3 grid((p.n_units + 7) / 8 * 8 * p.n_ct);
  hipLaunchKernelGGL((chunk_bwd_tile_kernel<Tio, DK>), grid, dim3(256), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long total4 = p.T * p.H * DK / 4;
  if (total4 == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_bwd_reduce_kernel<DK>), dim3(unsigned((total4 + 255) / 256)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const BwdParams& p, int io_dtype, int dk, hipStream_t stream) {
  if (p.n_ct != dk / 16 || p.n_units != p.n_seqs * p.H || p.H < 1 || p.n_seqs < 1)
    return hipErrorInvalidValue;
  if (dk == 128) return io_dtype == 1 ? launch_bwd<__bf16, 128>(p, stream)
                                      : launch_bwd<float, 128>(p, stream);
  if (dk == 64) return io_dtype == 1 ? launch_bwd<__bf16, 64>(p, stream)
                                     : launch_bwd<float, 64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
