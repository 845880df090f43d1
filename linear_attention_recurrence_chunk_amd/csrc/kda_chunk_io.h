// Pieces shared by the chunk kernel (one-launch prefill and prep pass) and the walk kernel:
// the per-thread mapping and loads of a chunk's raw inputs, and the layout of the operand
// slots the prep pass writes and the walk reads.
#pragma once

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// N input elements of one thread, bf16 ones two to a register
template <typename T, int N>
struct Packed {
  T x[N];
  __device__ __forceinline__ float get(int i) const { return to_f32(x[i]); }
  __device__ __forceinline__ void set(int i, T a) { x[i] = a; }
};
template <int N>
struct Packed<__bf16, N> {
  bf16x2 x[N / 2];
  __device__ __forceinline__ float get(int i) const { return (float)x[i >> 1][i & 1]; }
  __device__ __forceinline__ void set(int i, __bf16 a) { x[i >> 1][i & 1] = a; }
};

// four consecutive elements of one input row (one vector load)
template <typename T> struct Quad;
template <> struct Quad<__bf16> { using type = bf16x4; };
template <> struct Quad<float> { using type = f32x4; };

// Prologue thread mapping: wave w owns the 16-token sub-block w; inside it, lane = (token group
// grp, channel quad c4) with DK / 4 lanes per token row, so each thread holds DK / 16
// consecutive tokens (16 w + grp DK / 16 + t) of four consecutive key channels (4 c4 ..).
template <int DK>
struct ProMap {
  static constexpr int kLPT = DK / 4;      // lanes per token row
  static constexpr int kNG = 64 / kLPT;    // token groups per sub-block
  static constexpr int kTPT = DK / 16;     // tokens per thread
};

// Raw inputs of one chunk held by one thread: g, k, q of its prologue elements; for each of
// the four 16-token row blocks rb, four value columns 16 w + 4 (lane % 16 / 4) .. + 3 of token
// 16 rb + 4 (lane / 16) + lane % 4 (a quad transpose turns them into MFMA accumulator layout);
// and (lanes < 16) the beta of token 16 w + lane. With kRawG the gates arrive as raw bf16
// projections (log-decay and beta before their activations) instead of fp32 values.
template <typename Tio, int DK, bool kRawG = false>
struct RawChunk {
  static constexpr int kTPT = ProMap<DK>::kTPT;
  using Tg = std::conditional_t<kRawG, __bf16, float>;
  typename Quad<Tg>::type g[kTPT];
  typename Quad<Tio>::type k[kTPT], q[kTPT], v[4];
  Tg beta;
};

// Loads of one chunk. Token offsets are wave-uniform (scalar address arithmetic) and each lane
// adds a fixed 32-bit byte offset. With kFull false (the last, ragged chunk of a sequence)
// rows past its end read the chunk's first row instead, which always exists.
// Address of a lane's element: base + uniform_elems + lane_elems (elements of type E), read
// as type T; with kFull false and !ok, base + fallback_elems instead.
template <bool kFull, typename E, typename T>
__device__ __forceinline__ const T* lane_ptr(const void* base, size_t uniform_elems,
                                             uint32_t lane_elems, bool ok, size_t fallback_elems) {
  const E* b = reinterpret_cast<const E*>(base);
  const char* u = reinterpret_cast<const char*>(b + uniform_elems);
  const char* a = u + lane_elems * uint32_t(sizeof(E));
  if constexpr (!kFull) a = ok ? a : reinterpret_cast<const char*>(b + fallback_elems);
  return reinterpret_cast<const T*>(a);
}

// Pieces of a chunk's raw inputs, loaded separately so that their issue can be spread over
// the previous chunk: kind G, K or Q for the thread's tokens [kLo, kHi) out of eight (scaled to
// its token count), V (values) or B (beta).
enum : int { kLoadG = 1, kLoadK = 2, kLoadQ = 4, kLoadV = 8, kLoadB = 16, kLoadAll = 31 };

template <bool kFull, int kParts, typename Tio, int DK, int kLo = 0, int kHi = 8, bool kRawG = false>
__device__ __forceinline__ void load_chunk(RawChunk<Tio, DK, kRawG>& x, const ChunkParams& p,
                                           int cstart, int Lc, int w, int lane, int h, int vcol0) {
  using M = ProMap<DK>;
  using Q4 = typename Quad<Tio>::type;
  using Tg = typename RawChunk<Tio, DK, kRawG>::Tg;
  using G4 = typename Quad<Tg>::type;
  const int H = p.H;
  const int grp = lane / M::kLPT;
  const int c0 = 4 * (lane % M::kLPT);
  const size_t row = size_t(H) * DK;                 // elements from one token to the next
  // prologue elements: token cstart + 16 w + grp kTPT + t, channels c0 .. c0 + 3
  const uint32_t lk = uint32_t((grp * M::kTPT * H + h) * DK + c0);
  const size_t fk = (size_t(cstart) * H + h) * DK + c0;   // fallback: the chunk's first row
  const size_t u0 = size_t(cstart + 16 * w) * row;
#pragma unroll
  for (int t = kLo * M::kTPT / 8; t < kHi * M::kTPT / 8; ++t) {
    const bool ok = 16 * w + grp * M::kTPT + t < Lc;
    const size_t u = u0 + size_t(t) * row;
    if constexpr ((kParts & kLoadG) != 0) x.g[t] = *lane_ptr<kFull, Tg, G4>(p.g, u, lk, ok, fk);
    if constexpr ((kParts & kLoadK) != 0) x.k[t] = *lane_ptr<kFull, Tio, Q4>(p.k, u, lk, ok, fk);
    if constexpr ((kParts & kLoadQ) != 0) x.q[t] = *lane_ptr<kFull, Tio, Q4>(p.q, u, lk, ok, fk);
  }
  if constexpr ((kParts & kLoadV) != 0) {
    // values: token cstart + 16 rb + 4 q4 + lane % 4, columns vcol0 + 16 w + 4 (ln / 4) .. + 3
    const int q4 = lane >> 4, ln = lane & 15;
    const int vc = vcol0 + 16 * w + 4 * (ln >> 2);
    const uint32_t lv = uint32_t(((4 * q4 + (ln & 3)) * H + h) * p.dv + vc);
    const size_t fv = (size_t(cstart) * H + h) * p.dv + vc;
    const size_t vrow = size_t(H) * p.dv;
    const size_t v0 = size_t(cstart) * vrow;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const bool ok = 16 * rb + 4 * q4 + (ln & 3) < Lc;
      x.v[rb] = *lane_ptr<kFull, Tio, Q4>(p.v, v0 + size_t(16 * rb) * vrow, lv, ok, fv);
    }
  }
  if constexpr ((kParts & kLoadB) == 0) return;
  // beta of token 16 w + lane % 16 (every lane loads, so that the register is only ever
  // written by loads; lanes 16-63 repeat lanes 0-15 and are not used)
  {
    const int bl = lane & 15;
    const bool ok = 16 * w + bl < Lc;
    const uint32_t lb = uint32_t((16 * w + bl) * H + h);
    const size_t fb = size_t(cstart) * H + h;
    x.beta = *lane_ptr<kFull, Tg, Tg>(p.beta, size_t(cstart) * H, lb, ok, fb);
  }
}

template <int kParts, typename Tio, int DK, int kLo = 0, int kHi = 8, bool kRawG = false>
__device__ __forceinline__ void load_chunk_any(RawChunk<Tio, DK, kRawG>& x, const ChunkParams& p,
                                               int cstart, int Lc, int w, int lane, int h,
                                               int vcol0) {
  if (Lc == kChunk)
    load_chunk<true, kParts, Tio, DK, kLo, kHi, kRawG>(x, p, cstart, Lc, w, lane, h, vcol0);
  else
    load_chunk<false, kParts, Tio, DK, kLo, kHi, kRawG>(x, p, cstart, Lc, w, lane, h, vcol0);
}

// One chunk-head's serial-step operands, written by the prep pass of the two-pass prefill and
// read by its walk: MFMA fragments in lane order (64 lanes x 16 bytes = 1 KiB per fragment),
// so a wave moves one fragment as one contiguous block, and the walk's LDS reads of them are
// conflict-free without padding. The last block holds the whole-chunk decay (DK fp32).
template <int DK>
struct OpSlot {
  static constexpr int NS = DK / 32;    // k-slices over key channels
  static constexpr int NTD = DK / 16;   // 16-row tiles over key channels
  static constexpr int fKg = 0;         // K e^Gamma (fp16), fragment (rb, pp) at rb NS + pp
  static constexpr int fQg = 4 * NS;    // Q e^Gamma (fp16), same order
  static constexpr int fT = 8 * NS;     // T diag(beta) hi (bf16): the 6 lower fragments
  static constexpr int fTLo = fT + 6;   //   and lo
  static constexpr int fM = fT + 12;    // M hi (fp16): the 6 lower fragments
  static constexpr int fMLo = fT + 18;  //   and lo
  static constexpr int fKh = fT + 24;   // (K e^{Gamma_L - Gamma})^T (fp16), (t, pp) at 2 t + pp
  static constexpr int kDecay = fKh + 2 * NTD;
  static constexpr int kBlocks = kDecay + 1;
  static constexpr size_t kBytes = size_t(kBlocks) * 1024;
  static_assert(DK * 4 <= 1024, "the decay fits one block");
  // the lower fragments of a 64 x 64 operand in slice order: row block rb takes slices
  // pp < (rb + 2) / 2, i.e. (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
  static constexpr __host__ __device__ int tri(int rb, int pp) { return (rb == 3 ? 4 : rb) + pp; }
};

// Checkpoint of the state after a full chunk that ends a multiple of p.ckpt_every tokens into
// its sequence (forward mode; seq_bos is the sequence's first token). S holds this wave's 16
// columns (from col0) in MFMA accumulator layout.
template <int DK, int NTD>
__device__ __forceinline__ void write_checkpoint(const ChunkParams& p, const f32x4 (&S)[NTD],
                                                 int seq_bos, int cend, int Lc, int h, int col0,
                                                 int q4, int ln) {
  const int done = cend - seq_bos;   // tokens of the sequence processed so far
  if (!p.ckpt || Lc != kChunk || done % p.ckpt_every != 0) return;
  const size_t slot = size_t(seq_bos / p.ckpt_every + done / p.ckpt_every - 1);
  float* dst = p.ckpt + (slot * p.H + h) * size_t(DK) * p.dv + col0 + ln;
#pragma unroll
  for (int t = 0; t < NTD; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[size_t(16 * t + 4 * q4 + e) * p.dv] = S[t][e];
}

}  // namespace kda
