// The KDA recurrence in 16-token chunks on gfx950, every product on fp32 matrix cores
// (v_mfma_f32_16x16x4_f32): the backward, and the fp32 prefill at d = 128.
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
// The backward's four launches:
//   0. cbwd_prep_kernel: one workgroup per (chunk, head) forms the chunk's operand block: the
//      decayed tiles K_G, K^, Q_G, T, M, e^(G_C) and beta;
//   1. cbwd_fwd_kernel: one wave per (sequence, head, 16-column tile) walks the chunks
//      forward and stores the entering state S0 of even chunks, X0 and U of every chunk;
//   2. cbwd_rev_kernel: the same waves walk back, storing dS (the gradient of the state
//      leaving a chunk) of odd chunks and of the last (see kAdvanceDS), dU and dY of every
//      chunk, writing dv, and dh0 at the sequence start;
//   3. cbwd_grad_kernel: one workgroup per (chunk, head) rebuilds the state its walk did not
//      keep from the neighbouring chunk's (the walk's own update), then forms dq, dk, dbeta
//      and dg.
// The fp32 prefill: the same operand pass, then c16_prefill_kernel, the forward walk producing
// o = s (Q_G S0 + M U), the final state and checkpoints.
// The walks stage each chunk's operand block into LDS (global-to-LDS loads) while the previous
// chunk is computed, so their chains hold the state products only. Sums over value columns
// happen inside launch 3 in a fixed order: results are deterministic.
#include "kda_bwd.h"
#include "kda_common.h"

namespace kda {

namespace {

constexpr int kC = kCBChunk;

// chunk slot of chunk c of the launch's sequence i (whose first token is sbos tokens after the
// launch's slot origin)
__device__ __forceinline__ long long cb_slot(int sbos, int i, int c) {
  return (long long)(sbos / kC) + i + c;
}

// first token of the launch's sequence i (i = n_seqs: the end of the last one)
__device__ __forceinline__ int seq_first_token(const CBwdParams& p, int i) {
  return p.cu_seqlens ? p.cu_seqlens[p.seq0 + i] : (p.seq0 + i) * p.seq_len;
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

// The operand block of one (chunk slot, head), in floats: the [16][DK] tiles K_G, K^ and Q_G
// (element (t, c) at t DK + (c ^ swz(t))), T and M ([16][16] row-major), e^(G_C) per key channel
// and beta per token. The forward walk stages the first kFwd floats, the reverse walk all.
template <int DK>
struct OpBlock {
  static constexpr int kKG = 0;
  static constexpr int kKH = 16 * DK;
  static constexpr int kT = 32 * DK;
  static constexpr int kEGC = kT + 256;
  static constexpr int kBeta = kEGC + DK;
  static constexpr int kFwd = kBeta + 16;
  static constexpr int kQG = kFwd;
  static constexpr int kM = kQG + 16 * DK;
  static constexpr int kFloats = kM + 256;
  static_assert(kFwd % 4 == 0 && kFloats % 4 == 0, "16-byte units");
  static_assert(kFloats == cbwd_op_floats(DK), "workspace layout");
};
// The swizzle of the tiles' rows (an XOR on bits 2..5 of the channel): both access patterns of
// the walks read 64 distinct banks: lanes along the tokens reading four consecutive channels
// each (one 16-byte read: the XOR keeps aligned groups of four together), and lanes along the
// channels with four token groups.
__device__ __forceinline__ int swz(int t) { return 4 * t; }

// Copies the 16 x 16 tile of a chunk (rows cs + t, or cs for t >= L; columns col0 ..
// col0 + 15 of rows ld elements apart) from global src to LDS dst, row-major (one wave; the LDS
// address of a global-to-LDS load is its wave-uniform base plus 16 bytes per lane).
// Asynchronous: the data is there once the wave's vector-memory count has drained.
template <typename Tio>
__device__ __forceinline__ void stage_vtile(const Tio* src, size_t ld, int cs, int L, int col0,
                                            float* dst, int lane) {
  constexpr int kPer = sizeof(Tio);          // 16-byte units per row
  constexpr int kEl = 16 / sizeof(Tio);      // elements per unit
  if (lane < 16 * kPer) {
    const int t = lane / kPer, part = lane % kPer;
    const Tio* g = src + size_t(t < L ? cs + t : cs) * ld + col0 + kEl * part;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(g), dst, 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stores a 16 x 16 tile held in accumulator layout (lane (q4, ln), register r: row 4 q4 + r,
// column ln) to row-major dst (rows ld floats apart) with one 16-byte store per lane: after a
// transpose inside each quad of lanes, lane (q4, ln) holds row 4 q4 + (ln & 3), columns
// 4 (ln >> 2) .. + 3.
__device__ __forceinline__ void store_tile16(float* dst, size_t ld, f32x4 a, int lane) {
  float x[4] = {a[0], a[1], a[2], a[3]};
  quad_transpose(x, lane);
  const int q4 = (lane >> 4) & 3, ln = lane & 15;
  *reinterpret_cast<f32x4*>(dst + size_t(4 * q4 + (ln & 3)) * ld + 4 * (ln >> 2)) =
      f32x4{x[0], x[1], x[2], x[3]};
}

// The chunk that a chunk slot holds: the launch's sequence i (the last one whose first slot
// floor((bos_i - slot_tok0) / 16) + i is at most slot), the chunk's first token and length.
// False for slots that no chunk uses. c_out (optional): the chunk's index in its sequence.
__device__ __forceinline__ bool slot_chunk(const CBwdParams& p, long long slot, int* cs_out,
                                           int* L_out, int* c_out = nullptr,
                                           int* eos_out = nullptr) {
  auto first_tok = [&](int i) -> long long { return seq_first_token(p, i); };
  int lo = 0, hi = p.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((first_tok(mid) - p.slot_tok0) / kC + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  const long long bos = first_tok(lo), eos = first_tok(lo + 1);
  const long long c = slot - ((bos - p.slot_tok0) / kC + lo);
  if (c < 0 || bos + kC * c >= eos) return false;
  *cs_out = int(bos + kC * c);
  *L_out = int(min((long long)kC, eos - *cs_out));
  if (c_out) *c_out = int(c);
  if (eos_out) *eos_out = int(eos);
  return true;
}

// Which leaving-state gradients dS the reverse walk writes. With kAdvanceDS only those of odd
// chunks and of each sequence's last chunk: the gradient pass advances an even chunk's from the
// chunk after it, D = e^(G_C') D' + Q_G'^T (s dO') - K_G'^T diag(beta') dY' (the walk's own
// update). It stages that chunk's dY and dO in LDS; for fp32 inputs at d_k = 128 the extra
// tile would cost the gradient pass its second workgroup per CU, so there every dS is written.
template <typename Tio, int DK>
constexpr bool kAdvanceDS = sizeof(Tio) == 2 || DK == 64;

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
// lane j < 16 solves column j by forward substitution into sT (row stride 20) and, when gT is
// set, into gT (row stride 16)
__device__ __forceinline__ void invert16(const float* sB, const float* sBeta, float* sT,
                                         float* gT, int lane) {
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
      if (gT) gT[i * 16 + lane] = v;
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

// ---- 0. operand blocks: one workgroup (one thread per key channel) per (chunk slot, head)
template <typename Tio, int DK>
__global__ __launch_bounds__(DK) void cbwd_prep_kernel(CBwdParams p) {
  using OB = OpBlock<DK>;
  constexpr int LK = DK + 1;
  __shared__ float sKq[kC * LK], sKk[kC * LK], sQq[kC * LK];
  __shared__ float sB[kC * 17], sT[kC * 20], sBeta[kC];
  const int H = p.H;
  const int h = int(blockIdx.x % unsigned(H));
  const long long slot = blockIdx.x / unsigned(H);
  int cs, L;
  if (!slot_chunk(p, slot, &cs, &L)) return;
  float* ob = p.ops + (size_t(slot) * H + h) * OB::kFloats;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, q4 = lane >> 4, ln = lane & 15;
  const Tio* gq = reinterpret_cast<const Tio*>(p.q);
  const Tio* gk = reinterpret_cast<const Tio*>(p.k);
  // beta of token tid (threads below kC), loaded before the block's stores: after them it
  // would wait for its round trip alone, the stores possibly aliasing it
  const float beta_raw = p.beta[size_t(tid < L ? cs + tid : cs) * H + h];
  {
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
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      const float eg = __expf(G[t]), eh = __expf(gc - G[t]);
      const float em = __expf(G[t] - gm), emi = __expf(gm - G[t]);
      const int sa = t * DK + (tid ^ swz(t));
      ob[OB::kKG + sa] = kv[t] * eg;
      ob[OB::kKH + sa] = kv[t] * eh;
      ob[OB::kQG + sa] = qv[t] * eg;
      sKq[t * LK + tid] = kv[t] * em;
      sKk[t * LK + tid] = kv[t] * emi;
      sQq[t * LK + tid] = qv[t] * em;
    }
    ob[OB::kEGC + tid] = __expf(gc);
  }
  if (tid < kC) {
    const float b = tid < L ? beta_raw : 0.f;
    sBeta[tid] = b;
    ob[OB::kBeta + tid] = b;
  }
  lds_barrier();
  if (w == 0) {
    const f32x4 b = gram16<DK>(sKq, sKk, ln, q4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q4 + r;
      sB[t * 17 + ln] = ln < t ? b[r] : 0.f;
    }
    wave_sync();
    invert16(sB, sBeta, sT, ob + OB::kT, lane);
  }
  if (w == DK / 64 - 1) {
    const f32x4 m = gram16<DK>(sQq, sKk, ln, q4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q4 + r;
      ob[OB::kM + t * 16 + ln] = ln <= t ? m[r] : 0.f;
    }
  }
}

// The walks: a workgroup of four waves per (sequence, head, group of four 16-column tiles);
// wave w owns tile 4 sub + w. The waves walk the same chunks and share each chunk's operand
// block in LDS, double-buffered: while a chunk is computed, the next chunk's block and the
// 16 x 16 input tiles are copied in. One barrier per chunk publishes the staged buffer and
// frees the one just read. (At 8192 x 96, d = 128: 192 workgroups, one per CU and one
// computing wave per SIMD; with two waves per workgroup, 384 of them, the backward took 7.6
// instead of 6.5 ms.)
constexpr int kWalkWaves = 4;

// Copies a block of N4 16-byte units from global src to LDS dst, 64 units per instruction;
// wave w of the walk issues instructions w, w + kWalkWaves, ... (asynchronous, as above)
template <int N4>
__device__ __forceinline__ void stage_block_half(const float* src, float* dst, int w, int lane) {
#pragma unroll
  for (int i = 0; i < N4 / 64; ++i)
    if (i % kWalkWaves == w)
      __builtin_amdgcn_global_load_lds(src + 4 * (64 * i + lane), dst + 256 * i, 16, 0, 0);
  if constexpr (N4 % 64 != 0) {
    if ((N4 / 64) % kWalkWaves == w && lane < N4 % 64)
      __builtin_amdgcn_global_load_lds(src + 4 * (64 * (N4 / 64) + lane), dst + 256 * (N4 / 64),
                                       16, 0, 0);
  }
}

// The backward's two walks add memory waves to the four that compute: wave kLoader stages
// each chunk's operand block and input tiles into LDS a chunk ahead, and wave kStorer (in the
// reverse walk kStorers waves from it) writes the results the computing waves leave in LDS
// (double-buffered, one buffer per chunk parity) to global memory. A 16-byte store or a 1 KiB
// global-to-LDS load holds the compute unit's vector-memory queue for tens of cycles and a
// wave stalls in order until the queue takes it; in the computing waves these stalls took
// 35-45% of each chunk step. Each memory wave waits only for its own accesses (the loader for
// its loads before each barrier; the stores are never waited for), and all waves of the
// workgroup pass the same barriers.
constexpr int kLoader = kWalkWaves, kStorer = kWalkWaves + 1;
// the forward walk has one storer, the reverse walk (whose dS tiles its storers transpose,
// see copy_cols) two
constexpr int kFwdThreads = 64 * (kWalkWaves + 2);
constexpr int kStorers = 2;
constexpr int kRevThreads = 64 * (kWalkWaves + 1 + kStorers);
constexpr int kOutLd = 68;   // row stride (floats) of the LDS result tiles: 64 columns + 4

// All N4 16-byte units of a block, issued by one wave.
template <int N4>
__device__ __forceinline__ void stage_block_all(const float* src, float* dst, int lane) {
#pragma unroll
  for (int w = 0; w < kWalkWaves; ++w) stage_block_half<N4>(src, dst, w, lane);
}

// A 16 x 16 accumulator tile into a row-major LDS tile of kOutLd-float rows, 16 bytes a lane
// (the quad transpose of store_tile16).
__device__ __forceinline__ void put_tile16(float* dst, f32x4 a, int lane) {
  float x[4] = {a[0], a[1], a[2], a[3]};
  quad_transpose(x, lane);
  const int q4 = (lane >> 4) & 3, ln = lane & 15;
  *reinterpret_cast<f32x4*>(dst + (4 * q4 + (ln & 3)) * kOutLd + 4 * (ln >> 2)) =
      f32x4{x[0], x[1], x[2], x[3]};
}

// The storer's copy of `rows` rows of a workgroup's 64 columns from an LDS result tile to
// row-major global memory (rows ld floats apart): 4 rows per instruction, eight loads from LDS
// in flight ahead of their stores. Rows at or past `keep` are not written.
template <int kRows>
__device__ __forceinline__ void copy_rows(const float* src, float* dst, size_t ld, int keep,
                                          int lane) {
  const int rr = lane >> 4, cc = 4 * (lane & 15);
  constexpr int kGroup = kRows / 4 < 8 ? kRows / 4 : 8;
#pragma unroll
  for (int i0 = 0; i0 < kRows / 4; i0 += kGroup) {
    f32x4 v[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
      v[j] = *reinterpret_cast<const f32x4*>(src + (4 * (i0 + j) + rr) * kOutLd + cc);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int row = 4 * (i0 + j) + rr;
      if (row < keep) *reinterpret_cast<f32x4*>(dst + size_t(row) * ld + cc) = v[j];
    }
  }
}

// The storer's copy of a workgroup's DK x 64 state tile that the computing waves left in LDS
// in their accumulator layout, column-major (column c of the tile at c * (DK + 4), rows
// contiguous: each lane's 16-byte write is four rows of one column, no transpose on the
// computing waves' chain). Quad (lane / 4) reads four rows of columns 4 quad .. + 3, one column
// a lane, the quad transposes them, and lane j stores row 4 i + j, 16 bytes of four columns, to
// row-major dst (rows ld floats apart): eight reads in flight ahead of their stores.
template <int DK>
__device__ __forceinline__ void copy_cols(const float* src, float* dst, size_t ld, int lane,
                                          int part) {
  constexpr int kLd = DK + 4;
  constexpr int kPer = DK / 4 / kStorers;   // 4-row groups of one storer
  static_assert(kPer % 8 == 0, "whole groups of eight");
  const int qd = lane >> 2, j = lane & 3;
#pragma unroll
  for (int i0 = part * kPer; i0 < (part + 1) * kPer; i0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = *reinterpret_cast<const f32x4*>(src + (4 * qd + j) * kLd + 4 * (i0 + k));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float x[4] = {v[k][0], v[k][1], v[k][2], v[k][3]};
      quad_transpose(x, lane);
      *reinterpret_cast<f32x4*>(dst + size_t(4 * (i0 + k) + j) * ld + 4 * qd) =
          f32x4{x[0], x[1], x[2], x[3]};
    }
  }
}

// ---- 1. forward walk: S0 of even chunks, X0 and U of every chunk
template <typename Tio, int DK>
__global__ __launch_bounds__(kFwdThreads) void cbwd_fwd_kernel(CBwdParams p) {
  constexpr int DV = DK, NTD = DK / 16;
  using OB = OpBlock<DK>;
  // per buffer: the block's first kFwd floats, then the four 16 x 16 value tiles
  constexpr int kTile = 64 * int(sizeof(Tio));   // floats of one tile
  constexpr int kBuf = OB::kFwd + kWalkWaves * kTile;
  // results of a chunk: the next chunk's entering state S (DK rows), X0 and U (16 rows each)
  constexpr int kOS = 0, kOX = DK * kOutLd, kOU = kOX + 16 * kOutLd, kOut = kOU + 16 * kOutLd;
  __shared__ __attribute__((aligned(16))) float sb0[kBuf], sb1[kBuf];
  __shared__ __attribute__((aligned(16))) float so[2][kOut];

  int sub;
  const int unit = block_unit(blockIdx.x, p.n_ct / kWalkWaves, &sub);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int h = unit % H, n = unit / H;
  const int bos = seq_first_token(p, n), eos = seq_first_token(p, n + 1);
  const int sbos = bos - p.slot_tok0;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q4 = lane >> 4, ln = lane & 15;
  const int nch = (eos - bos + kC - 1) / kC;
  if (nch == 0) return;
  const float* ops0 = p.ops + (size_t(cb_slot(sbos, n, 0)) * H + h) * OB::kFloats;
  const size_t ops_stride = size_t(H) * OB::kFloats;
  const int col0 = 64 * sub;   // the workgroup's first state column

  if (w == kLoader) {
    const Tio* gv = reinterpret_cast<const Tio*>(p.v) + size_t(h) * DV;
    // a chunk's operand block and the four value tiles (the last chunk's again at the end:
    // nothing is staged conditionally); the buffer was last read in the chunk before last
    auto stage = [&](int c, float* dst) {
      const int cs = bos + kC * c;
      stage_block_all<OB::kFwd / 4>(ops0 + c * ops_stride, dst, lane);
#pragma unroll
      for (int t = 0; t < kWalkWaves; ++t)
        stage_vtile(gv, size_t(H) * DV, cs, min(kC, eos - cs), col0 + 16 * t,
                    dst + OB::kFwd + t * kTile, lane);
    };
    stage(0, sb0);
    wait_vmem();
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
      stage(min(c + 1, nch - 1), (c & 1) ? sb0 : sb1);
      wait_vmem();
      lds_barrier();
    }
    return;
  }
  if (w == kStorer) {
    // interval c (after barrier c - 1) writes what chunk c - 1 left: S0 of chunk c when c is
    // even, X0 and U of chunk c - 1 (for c = 0 the entering state only). The gradient pass
    // advances an odd chunk's entering state from the even one before it.
    auto s0_of = [&](int c) { return p.S0 + (size_t(cb_slot(sbos, n, c)) * H + h) * DK * DV; };
    lds_barrier();
    for (int c = 0; c <= nch; ++c) {
      const float* src = so[(c + 1) & 1];
      if (c < nch && c % 2 == 0) copy_rows<DK>(src + kOS, s0_of(c) + col0, DV, DK, lane);
      if (c > 0) {
        const size_t blk = size_t(cb_slot(sbos, n, c - 1)) * H + h;
        copy_rows<16>(src + kOX, p.X0 + blk * kC * DV + col0, DV, 16, lane);
        copy_rows<16>(src + kOU, p.U + blk * kC * DV + col0, DV, 16, lane);
      }
      if (c < nch) lds_barrier();
    }
    return;
  }

  const int ct = kWalkWaves * sub + w;
  const int col = 16 * ct + ln;
  // the state tile in accumulator layout: block rb, register r = row 16 rb + 4 q4 + r
  f32x4 S[NTD];
  const size_t st_off = (size_t(p.seq0 + n) * H + h) * DK * DV;
#pragma unroll
  for (int rb = 0; rb < NTD; ++rb) S[rb] = zero4();
  if (p.h0) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[rb][r] = p.h0[st_off + size_t(16 * rb + 4 * q4 + r) * DV + col];
  }
  // the entering state goes out through buffer 1 (the storer's interval 0 reads it)
#pragma unroll
  for (int rb = 0; rb < NTD; ++rb) put_tile16(so[1] + kOS + 16 * rb * kOutLd + 16 * w, S[rb], lane);
  lds_barrier();

  for (int c = 0; c < nch; ++c) {
    const float* cur = (c & 1) ? sb1 : sb0;
    float* out = so[c & 1];
    const int cs = bos + kC * c, L = min(kC, eos - cs);
    const int sl = swz(ln);
    // X = K_G S (k order: the state's own register order)
    f32x4 X = zero4();
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(cur + OB::kKG + ln * DK + ((16 * rb + 4 * q4) ^ sl));
#pragma unroll
      for (int r = 0; r < 4; ++r) X = mma_f32(a[r], S[rb][r], X);
    }
    // X0 = V - X, Y = diag(beta) X0 (rows past a ragged chunk's end are zero)
    const f32x4 bt = *reinterpret_cast<const f32x4*>(cur + OB::kBeta + 4 * q4);
    const Tio* vt = reinterpret_cast<const Tio*>(cur + OB::kFwd + w * kTile);
    f32x4 X0, Y;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      X0[r] = (to_f32(vt[(4 * q4 + r) * 16 + ln]) - X[r]) * keep_f(4 * q4 + r < L);
      Y[r] = bt[r] * X0[r];
    }
    // U = T Y
    f32x4 U = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) U = mma_f32(cur[OB::kT + ln * 16 + 4 * q4 + kk], Y[kk], U);
    put_tile16(out + kOX + 16 * w, X0, lane);
    put_tile16(out + kOU + 16 * w, U, lane);
    // S = e^(G_C) S + K^^T U
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb) {
      const f32x4 e = *reinterpret_cast<const f32x4*>(cur + OB::kEGC + 16 * rb + 4 * q4);
      S[rb] *= e;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int t = 4 * q4 + kk;
        S[rb] = mma_f32(cur[OB::kKH + t * DK + ((16 * rb + ln) ^ swz(t))], U[kk], S[rb]);
      }
    }
    if (c + 1 < nch && (c + 1) % 2 == 0) {
#pragma unroll
      for (int rb = 0; rb < NTD; ++rb) put_tile16(out + kOS + 16 * rb * kOutLd + 16 * w, S[rb], lane);
    }
    // publishes the next staged buffer and this chunk's results; frees the buffer just read
    lds_barrier();
  }
}

// ---- 2. reverse walk: dS (see kAdvanceDS), dU, dY of every chunk, dv, and dh0
template <typename Tio, int DK>
__global__ __launch_bounds__(kRevThreads) void cbwd_rev_kernel(CBwdParams p) {
  constexpr int DV = DK, NTD = DK / 16;
  using OB = OpBlock<DK>;
  // per buffer: the operand block, then the four 16 x 16 tiles of output gradients
  constexpr int kTile = 64 * int(sizeof(Tio));
  constexpr int kBuf = OB::kFloats + kWalkWaves * kTile;
  // results of a chunk: dS (the gradient of the state leaving it; the 64 columns of DK + 4
  // floats each, column-major, see copy_cols), dU, dY, dv (row-major)
  static_assert(64 * (DK + 4) <= DK * kOutLd, "the column-major dS tile fits its region");
  constexpr int kOD = 0, kOdU = DK * kOutLd, kOdY = kOdU + 16 * kOutLd, kOdv = kOdY + 16 * kOutLd,
                kOut = kOdv + 16 * kOutLd;
  __shared__ __attribute__((aligned(16))) float sb0[kBuf], sb1[kBuf];
  __shared__ __attribute__((aligned(16))) float so[2][kOut];

  int sub;
  const int unit = block_unit(blockIdx.x, p.n_ct / kWalkWaves, &sub);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int h = unit % H, n = unit / H;
  const int bos = seq_first_token(p, n), eos = seq_first_token(p, n + 1);
  const int sbos = bos - p.slot_tok0;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q4 = lane >> 4, ln = lane & 15;
  const int nch = (eos - bos + kC - 1) / kC;
  const float* ops0 = p.ops + (size_t(cb_slot(sbos, n, 0)) * H + h) * OB::kFloats;
  const size_t ops_stride = size_t(H) * OB::kFloats;
  const int col0 = 64 * sub;

  if (w == kLoader) {
    const Tio* gdo = reinterpret_cast<const Tio*>(p.d_o) + size_t(h) * DV;
    auto stage = [&](int c, float* dst) {
      const int cs = bos + kC * c;
      stage_block_all<OB::kFloats / 4>(ops0 + c * ops_stride, dst, lane);
#pragma unroll
      for (int t = 0; t < kWalkWaves; ++t)
        stage_vtile(gdo, size_t(H) * DV, cs, min(kC, eos - cs), col0 + 16 * t,
                    dst + OB::kFloats + t * kTile, lane);
    };
    if (nch > 0) {
      stage(nch - 1, sb0);
      wait_vmem();
      lds_barrier();
      for (int i = 0; i < nch; ++i) {
        stage(max(nch - 2 - i, 0), (i & 1) ? sb0 : sb1);
        wait_vmem();
        lds_barrier();
      }
    }
    return;
  }
  if (w >= kStorer) {
    // interval i (after barrier i - 1) writes what iteration i - 1 (chunk nch - i) left; the
    // two storers take half of dS's rows each, dU and dY the first, dv the second
    const int sp = w - kStorer;
    if (nch > 0) {
      lds_barrier();
      for (int i = 1; i <= nch; ++i) {
        lds_barrier();
        const float* src = so[(i - 1) & 1];
        const int c = nch - i, cs = bos + kC * c, L = min(kC, eos - cs);
        const size_t blk = size_t(cb_slot(sbos, n, c)) * H + h;
        if (!kAdvanceDS<Tio, DK> || (c & 1) || c == nch - 1)
          copy_cols<DK>(src + kOD, p.dS + blk * DK * DV + col0, DV, lane, sp);
        if (sp == 0) {
          copy_rows<16>(src + kOdU, p.dU + blk * kC * DV + col0, DV, 16, lane);
          copy_rows<16>(src + kOdY, p.dY + blk * kC * DV + col0, DV, 16, lane);
        } else {
          copy_rows<16>(src + kOdv, p.dv + (size_t(cs) * H + h) * DV + col0, size_t(H) * DV, L,
                        lane);
        }
      }
    }
    return;
  }

  const int ct = kWalkWaves * sub + w;
  const int col = 16 * ct + ln;
  f32x4 D[NTD];
  const size_t st_off = (size_t(p.seq0 + n) * H + h) * DK * DV;
#pragma unroll
  for (int rb = 0; rb < NTD; ++rb) D[rb] = zero4();
  if (p.dht) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) D[rb][r] = p.dht[st_off + size_t(16 * rb + 4 * q4 + r) * DV + col];
  }
  if (nch > 0) {
    lds_barrier();
    for (int i = 0; i < nch; ++i) {
      const int c = nch - 1 - i;
      const float* cur = (i & 1) ? sb1 : sb0;
      float* out = so[i & 1];
      // the gradient of the state leaving the chunk, as the accumulators hold it (column
      // 16 w + ln, rows 16 rb + 4 q4 .. + 3), where it is kept
      if (!kAdvanceDS<Tio, DK> || (c & 1) || c == nch - 1) {
#pragma unroll
        for (int rb = 0; rb < NTD; ++rb)
          *reinterpret_cast<f32x4*>(out + kOD + (16 * w + ln) * (DK + 4) + 16 * rb + 4 * q4) = D[rb];
      }
      const int cs = bos + kC * c, L = min(kC, eos - cs);
      const int sl = swz(ln);
      // s dO as the products' right operand: token 4 q4 + kk, this lane's column
      const Tio* dt = reinterpret_cast<const Tio*>(cur + OB::kFloats + w * kTile);
      float sdo[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sdo[kk] = (p.scale * keep_f(4 * q4 + kk < L)) * to_f32(dt[(4 * q4 + kk) * 16 + ln]);
      // dU = M^T (s dO) + K^ D
      f32x4 dU = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) dU = mma_f32(cur[OB::kM + (4 * q4 + kk) * 16 + ln], sdo[kk], dU);
#pragma unroll
      for (int rb = 0; rb < NTD; ++rb) {
        const f32x4 a =
            *reinterpret_cast<const f32x4*>(cur + OB::kKH + ln * DK + ((16 * rb + 4 * q4) ^ sl));
#pragma unroll
        for (int r = 0; r < 4; ++r) dU = mma_f32(a[r], D[rb][r], dU);
      }
      // dY = T^T dU
      f32x4 dY = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) dY = mma_f32(cur[OB::kT + (4 * q4 + kk) * 16 + ln], dU[kk], dY);
      const f32x4 bt = *reinterpret_cast<const f32x4*>(cur + OB::kBeta + 4 * q4);
      put_tile16(out + kOdU + 16 * w, dU, lane);
      put_tile16(out + kOdY + 16 * w, dY, lane);
      // dv = diag(beta) dY (row-major, like the tiles above; the storer drops rows past L)
      put_tile16(out + kOdv + 16 * w, bt * dY, lane);
      // D = e^(G_C) D + Q_G^T (s dO) - K_G^T diag(beta) dY
      float bdy[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bdy[kk] = -bt[kk] * dY[kk];
#pragma unroll
      for (int rb = 0; rb < NTD; ++rb) {
        const f32x4 e = *reinterpret_cast<const f32x4*>(cur + OB::kEGC + 16 * rb + 4 * q4);
        D[rb] *= e;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int t = 4 * q4 + kk;
          const int a = t * DK + ((16 * rb + ln) ^ swz(t));
          D[rb] = mma_f32(cur[OB::kQG + a], sdo[kk], D[rb]);
          D[rb] = mma_f32(cur[OB::kKG + a], bdy[kk], D[rb]);
        }
      }
      lds_barrier();
    }
  }
  if (p.dh0) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p.dh0[st_off + size_t(16 * rb + 4 * q4 + r) * DV + col] = D[rb][r];
  }
}

// ---- the fp32 prefill at d = 128: the forward walk of the same chunk form, producing
// o = s (Q_G S0 + M U) per chunk, the final state and checkpoints. Workgroups as above (four
// computing waves, four 16-column tiles of one (sequence, head), and the loader wave kLoader
// staging the whole operand block and the value tiles); the computing waves store o.
constexpr int kPrefillThreads = 64 * (kWalkWaves + 1);
template <int DK>
__global__ __launch_bounds__(kPrefillThreads) void c16_prefill_kernel(CBwdParams p) {
  using Tio = float;
  constexpr int DV = DK, NTD = DK / 16;
  using OB = OpBlock<DK>;
  constexpr int kTile = 64 * int(sizeof(Tio));
  constexpr int kBuf = OB::kFloats + kWalkWaves * kTile;
  __shared__ __attribute__((aligned(16))) float sb0[kBuf], sb1[kBuf];

  int sub;
  const int unit = block_unit(blockIdx.x, p.n_ct / kWalkWaves, &sub);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int h = unit % H, n = unit / H;
  const int bos = seq_first_token(p, n), eos = seq_first_token(p, n + 1);
  const int sbos = bos - p.slot_tok0;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q4 = lane >> 4, ln = lane & 15;
  const Tio* gv = reinterpret_cast<const Tio*>(p.v) + size_t(h) * DV;
  const int nch = (eos - bos + kC - 1) / kC;
  const float* ops0 = p.ops + (size_t(cb_slot(sbos, n, 0)) * H + h) * OB::kFloats;
  const size_t ops_stride = size_t(H) * OB::kFloats;

  if (w == kLoader) {
    // a chunk's operand block and the four value tiles (the last chunk's again at the end:
    // nothing is staged conditionally); the buffer was last read in the chunk before last
    auto stage = [&](int c, float* dst) {
      const int cs = bos + kC * c;
      stage_block_all<OB::kFloats / 4>(ops0 + c * ops_stride, dst, lane);
#pragma unroll
      for (int t = 0; t < kWalkWaves; ++t)
        stage_vtile(gv, size_t(H) * DV, cs, min(kC, eos - cs), 64 * sub + 16 * t,
                    dst + OB::kFloats + t * kTile, lane);
    };
    if (nch > 0) {
      stage(0, sb0);
      wait_vmem();
      lds_barrier();
      for (int c = 0; c < nch; ++c) {
        stage(min(c + 1, nch - 1), (c & 1) ? sb0 : sb1);
        wait_vmem();
        lds_barrier();
      }
    }
    return;
  }

  const int ct = kWalkWaves * sub + w;
  const int col = 16 * ct + ln;
  const int sl = swz(ln);

  f32x4 S[NTD];
  const size_t st_off = (size_t(p.seq0 + n) * H + h) * DK * DV;
#pragma unroll
  for (int rb = 0; rb < NTD; ++rb) S[rb] = zero4();
  if (p.h0) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[rb][r] = p.h0[st_off + size_t(16 * rb + 4 * q4 + r) * DV + col];
  }
  // the state, row-major at dst (this wave's 16 columns)
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb) store_tile16(dst + size_t(16 * rb) * DV + 16 * ct, DV, S[rb], lane);
  };
  // K S with the [16][DK] tile at offset off of buffer b (k order: the state's register order)
  auto tile_times_state = [&](const float* b, int off) {
    f32x4 x = zero4();
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(b + off + ln * DK + ((16 * rb + 4 * q4) ^ sl));
#pragma unroll
      for (int r = 0; r < 4; ++r) x = mma_f32(a[r], S[rb][r], x);
    }
    return x;
  };
  if (nch > 0) lds_barrier();
  for (int c = 0; c < nch; ++c) {
    const float* cur = (c & 1) ? sb1 : sb0;
    const int cs = bos + kC * c, L = min(kC, eos - cs);
    // X = K_G S and the inter-chunk part of the output, Q_G S
    const f32x4 X = tile_times_state(cur, OB::kKG);
    f32x4 O = tile_times_state(cur, OB::kQG);
    // X0 = V - X, Y = diag(beta) X0 (rows past a ragged chunk's end are zero), U = T Y
    const f32x4 bt = *reinterpret_cast<const f32x4*>(cur + OB::kBeta + 4 * q4);
    const Tio* vt = reinterpret_cast<const Tio*>(cur + OB::kFloats + w * kTile);
    f32x4 Y;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Y[r] = bt[r] * ((vt[(4 * q4 + r) * 16 + ln] - X[r]) * keep_f(4 * q4 + r < L));
    f32x4 U = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) U = mma_f32(cur[OB::kT + ln * 16 + 4 * q4 + kk], Y[kk], U);
    // the intra-chunk part, M U
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) O = mma_f32(cur[OB::kM + ln * 16 + 4 * q4 + kk], U[kk], O);
    // S = e^(G_C) S + K^^T U
#pragma unroll
    for (int rb = 0; rb < NTD; ++rb) {
      S[rb] *= *reinterpret_cast<const f32x4*>(cur + OB::kEGC + 16 * rb + 4 * q4);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int t = 4 * q4 + kk;
        S[rb] = mma_f32(cur[OB::kKH + t * DK + ((16 * rb + ln) ^ swz(t))], U[kk], S[rb]);
      }
    }
    // publishes the next staged buffer, frees the one just read
    lds_barrier();
    {
      // o rows of this chunk: after a quad transpose lane (q4, ln) holds token
      // 4 q4 + (ln & 3), columns 4 (ln >> 2) .. + 3 of this tile
      float x[4] = {O[0], O[1], O[2], O[3]};
      quad_transpose(x, lane);
      const int t = 4 * q4 + (ln & 3);
      if (t < L)
        *reinterpret_cast<f32x4*>(p.o + (size_t(cs + t) * H + h) * DV + 16 * ct + 4 * (ln >> 2)) =
            f32x4{p.scale * x[0], p.scale * x[1], p.scale * x[2], p.scale * x[3]};
    }
    // the state after a multiple of ckpt_every tokens of the sequence
    const int done = kC * (c + 1);
    if (p.ckpt && done <= eos - bos && done % p.ckpt_every == 0)
      store_state(p.ckpt + (size_t(bos / p.ckpt_every + done / p.ckpt_every - 1) * H + h) * DK * DV);
  }
  if (p.ht) store_state(p.ht + st_off);
}

// ---- 3. gradients of one chunk: dq, dk, dbeta and dg. One workgroup (DK / 16 waves) per
// (chunk slot, head); workgroups of unused slots exit.
template <typename Tio, int DK>
__global__ __launch_bounds__(4 * DK) void cbwd_grad_kernel(CBwdParams p) {
  constexpr int DV = DK;
  constexpr int LK = DK + 1, LV = DV + 4;
  constexpr bool kAdv = kAdvanceDS<Tio, DK>;
  constexpr int LVn = DV + 16 / int(sizeof(Tio));   // row stride of the chunk after's dO
  __shared__ float sKq[kC * LK], sKk[kC * LK], sQq[kC * LK];
  __shared__ float sG[kC * LK];   // G, then each token's log-decay gradient
  __shared__ __attribute__((aligned(16))) float sdO[kC * LV], sU[kC * LV], sdY[kC * LV];
  // U of the chunk before (odd chunks), or dY of the chunk after (even chunks, kAdv)
  __shared__ __attribute__((aligned(16))) float sUp[kC * LV];
  // dO of the chunk after as loaded (even chunks, kAdv)
  __shared__ __attribute__((aligned(16))) Tio sdOn[kAdv ? kC * LVn : 8];
  __shared__ float sB[kC * 17], sdT[kC * 17], sdM[kC * 17], sW[kC * 17], sT[kC * 20];
  __shared__ float sGm[DK], sGC[DK], sExtra[DK], sBeta[kC], sdb[kC];

  const int H = p.H;
  const int h = int(blockIdx.x % unsigned(H));
  const long long slot = blockIdx.x / unsigned(H);
  int cs, L, ci, eos;
  if (!slot_chunk(p, slot, &cs, &L, &ci, &eos)) return;
  const size_t blk = size_t(slot) * H + h;
  // the forward walk keeps the entering states of even chunks; an odd chunk's is advanced
  // here from the one before it (the same sequence's previous slot). With kAdv the reverse walk
  // keeps the leaving-state gradients of odd chunks and of the last; an even chunk's is
  // advanced here from the one after it (the next slot, its first token csn, Ln tokens).
  const bool odd = (ci & 1) != 0;
  const int csn = cs + kC, Ln = min(kC, eos - csn);
  const bool ds_next = kAdv && !odd && Ln > 0;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, q4 = lane >> 4, ln = lane & 15;
  const Tio* gq = reinterpret_cast<const Tio*>(p.q);
  const Tio* gk = reinterpret_cast<const Tio*>(p.k);
  const Tio* gdo = reinterpret_cast<const Tio*>(p.d_o);
  const float* wX0 = p.X0 + blk * kC * DV;
  const float* wdU = p.dU + blk * kC * DV;

  // 1. the in-chunk decays and the key/query tiles (one thread per key channel), and s dO,
  // U and dY (the other threads). The key-channel threads keep which of their tokens' g lie
  // above the floor (bit t) for step 6, so that no load of g waits behind a store there.
  unsigned live = 0;
  if (tid < DK) {
    float G[kC], kv[kC], qv[kC];
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      const bool valid = t < L;
      const size_t row = (size_t(valid ? cs + t : cs) * H + h) * DK + tid;
      const float gv = p.g[row];
      live |= (gv > p.g_min ? 1u : 0u) << t;
      acc += fmaxf(gv, p.g_min) * keep_f(valid);
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
    if ((odd && tile == 1) || (ds_next && tile == 2)) {
      const float* src = odd ? p.U + (blk - H) * kC * DV : p.dY + (blk + H) * kC * DV;
#pragma unroll
      for (int it = 0; it < 4; ++it) x[it] = ld4(src, 4 * size_t(v + DK * it));
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int e = v + DK * it, t = e / (DV / 4), j = 4 * (e % (DV / 4));
        *reinterpret_cast<f32x4*>(sUp + t * LV + j) = x[it];
      }
    }
    if constexpr (kAdv) {
      if (ds_next && tile == 0) {
        // rows past the chunk after's end read its first row (scaled by 0 where used)
        using V4 = Tio __attribute__((ext_vector_type(4)));
        V4 y[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int e = v + DK * it, t = e / (DV / 4), j = 4 * (e % (DV / 4));
          y[it] = *reinterpret_cast<const V4*>(gdo + (size_t(t < Ln ? csn + t : csn) * H + h) * DV + j);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int e = v + DK * it, t = e / (DV / 4), j = 4 * (e % (DV / 4));
          *reinterpret_cast<V4*>(sdOn + t * LVn + j) = y[it];
        }
      }
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
    invert16(sB, sBeta, sT, nullptr, lane);
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
    // S0 of an odd chunk: e^(G_C) S0' + K^'^T U' from the chunk before (' marks its values),
    // the forward walk's update with the same products in the same order, here transposed:
    // lane (q4, ln) gets channel ch, value columns j .. j + 3 of column block i
    // dS of an even chunk (kAdv): the reverse walk's update from the chunk after, likewise
    using OB = OpBlock<DK>;
    const float* s0 = p.S0 + (odd ? blk - H : blk) * DK * DV + size_t(ch) * DV;
    const float* ds = p.dS + (ds_next ? blk + H : blk) * DK * DV + size_t(ch) * DV;
    float ech = 1.f, khp[4] = {0.f, 0.f, 0.f, 0.f};
    if (odd) {
      const float* ob = p.ops + (blk - H) * OB::kFloats;
      ech = ob[OB::kEGC + ch];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int t = 4 * q4 + kk;
        khp[kk] = ob[OB::kKH + t * DK + (ch ^ swz(t))];
      }
    }
    float egn = 1.f, qgn[4] = {0.f, 0.f, 0.f, 0.f}, kgn[4] = {0.f, 0.f, 0.f, 0.f};
    float nbt[4] = {0.f, 0.f, 0.f, 0.f};   // -beta of the chunk after's tokens
    if (ds_next) {
      const float* ob = p.ops + (blk + H) * OB::kFloats;
      egn = ob[OB::kEGC + ch];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int t = 4 * q4 + kk;
        const int a = t * DK + (ch ^ swz(t));
        qgn[kk] = ob[OB::kQG + a];
        kgn[kk] = ob[OB::kKG + a];
        nbt[kk] = -ob[OB::kBeta + t];
      }
    }
#pragma unroll 4
    for (int i = 0; i < DV / 16; ++i) {
      const int j = 16 * i + 4 * q4;
      f32x4 bs = ld4(s0, j);
      f32x4 bd = ld4(ds, j);
      if (odd) {
        bs *= ech;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          bs = mma_f32(sUp[(4 * q4 + kk) * LV + 16 * i + ln], khp[kk], bs);
      }
      if constexpr (kAdv) {
        if (ds_next) {
          bd *= egn;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int t = 4 * q4 + kk;
            const float sdo = (p.scale * keep_f(t < Ln)) * to_f32(sdOn[t * LVn + 16 * i + ln]);
            bd = mma_f32(sdo, qgn[kk], bd);
            bd = mma_f32(nbt[kk] * sUp[t * LV + 16 * i + ln], kgn[kk], bd);
          }
        }
      }
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

  // 5. dq, dk, and each token's log-decay gradient (query side + key side -); the four
  // tokens' q and k are loaded before the first store (the stores could alias them)
  const float gm = sGm[ch], gc = sGC[ch];
  float khs = 0.f;
  float qv4[4], kv4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * q4 + r;
    const bool valid = t < L;
    const size_t row = (size_t(valid ? cs + t : cs) * H + h) * DK + ch;
    qv4[r] = ld_keep(gq, row, valid);
    kv4[r] = ld_keep(gk, row, valid);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * q4 + r;
    const bool valid = t < L;
    const float G = sG[t * LK + ch];
    const float eg = __expf(G), em = __expf(G - gm), emi = __expf(gm - G), eh = __expf(gc - G);
    const size_t row = (size_t(valid ? cs + t : cs) * H + h) * DK + ch;
    const float qv = qv4[r], kv = kv4[r];
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
      if (t < L) p.dg[(size_t(cs + t) * H + h) * DK + tid] = (live >> t) & 1u ? run : 0.f;
    }
  }
}

template <typename Tio, int DK>
static hipError_t launch_cbwd(const CBwdParams& p, hipStream_t stream) {
  const dim3 walk((p.n_units + 7) / 8 * 8 * (p.n_ct / kWalkWaves));
  const dim3 chunks(unsigned(p.n_slots * p.H));
  hipLaunchKernelGGL((cbwd_prep_kernel<Tio, DK>), chunks, dim3(DK), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((cbwd_fwd_kernel<Tio, DK>), walk, dim3(kFwdThreads), 0, stream, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((cbwd_rev_kernel<Tio, DK>), walk, dim3(kRevThreads), 0, stream, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((cbwd_grad_kernel<Tio, DK>), chunks, dim3(4 * DK), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_c16_prefill(const CBwdParams& p, int dk, hipStream_t stream) {
  if (dk != 128 || p.n_ct != dk / 16 || p.n_ct % kWalkWaves != 0 ||
      p.n_units != p.n_seqs * p.H || p.H < 1 || p.n_seqs < 1 || !p.ops || !p.o ||
      (p.ckpt && (p.ckpt_every < 64 || p.ckpt_every % 64 != 0)) || p.n_slots * p.H > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const dim3 walk((p.n_units + 7) / 8 * 8 * (p.n_ct / kWalkWaves));
  hipLaunchKernelGGL((cbwd_prep_kernel<float, 128>), dim3(unsigned(p.n_slots * p.H)), dim3(128), 0,
                     stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((c16_prefill_kernel<128>), walk, dim3(kPrefillThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd_mfma(const CBwdParams& p, int io_dtype, int dk, hipStream_t stream) {
  if (p.n_ct != dk / 16 || p.n_ct % kWalkWaves != 0 || p.n_units != p.n_seqs * p.H || p.H < 1 ||
      p.n_seqs < 1 ||
      p.n_slots != cbwd_slots(p.T, p.n_seqs) || p.n_slots * p.H > 0x7fffffffLL)
    return hipErrorInvalidValue;
  if (dk == 128) return io_dtype == 1 ? launch_cbwd<__bf16, 128>(p, stream)
                                      : launch_cbwd<float, 128>(p, stream);
  if (dk == 64) return io_dtype == 1 ? launch_cbwd<__bf16, 64>(p, stream)
                                     : launch_cbwd<float, 64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kda
