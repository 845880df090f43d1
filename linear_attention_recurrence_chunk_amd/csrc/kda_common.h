// Device helpers shared by the libkda kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_index.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;   // log2(e), rounded to fp32
constexpr int kWave = 64;
constexpr int kSub = 16;     // tokens per sub-block (one MFMA tile edge)
constexpr int kNumSub = kChunk / kSub;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// ---------------------------------------------------------------------------------------------
// MFMA policies. A 16x16 fp32 accumulator tile holds element (row m, col n) in lane
// n + 16 * (m / 4), register m % 4. An operand fragment of lane l belongs to row/column
// l % 16 and k-group l / 16. Every fragment here uses the same k-order inside a slice, chosen
// so that the accumulator registers of the tiles covering a slice ARE the B fragment of that
// slice: a result can feed the next product with no data movement. LDS fragments are read in
// the same order, so A and B always agree.
// ---------------------------------------------------------------------------------------------

// bf16 operands, v_mfma_f32_16x16x32_bf16. Slice p covers k in [32p, 32p + 32); element e of
// k-group q is k = 32p + 16 * (e / 4) + 4q + e % 4.
struct PolBF16 {
  using E = __bf16;
  using Frag = bf16x8;
  static constexpr int kSlice = 32;
  static constexpr bool kSplit = true;  // products that need it use hi + lo operand pairs
  __device__ static __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr int slices(int k) { return k / 32; }
  // slices covering the first nb 16-wide blocks of k
  static constexpr int slices_blocks(int nb) { return (nb + 1) / 2; }
  __device__ static __forceinline__ Frag load(const E* tile, int ld, int row, int p, int q) {
    const E* base = tile + row * ld + 32 * p + 4 * q;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(base);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // fragment scaled per k by fac[k] (fp32), rounded once to bf16
  __device__ static __forceinline__ Frag load_scaled(const E* tile, int ld, int row, int p,
                                                     int q, const float* fac) {
    return load_scaled_at(tile, ld, row, p, p, q, fac);
  }
  // the same with the tile's slice p and the factors' slice pf given apart (tiles that hold
  // only part of the channels)
  __device__ static __forceinline__ Frag load_scaled_at(const E* tile, int ld, int row, int p,
                                                        int pf, int q, const float* fac) {
    const E* base = tile + row * ld + 32 * p + 4 * q;
    const float* fb = fac + 32 * pf + 4 * q;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(base);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + 16);
    f32x4 flo = *reinterpret_cast<const f32x4*>(fb);
    f32x4 fhi = *reinterpret_cast<const f32x4*>(fb + 16);
    Frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (__bf16)((float)lo[e] * flo[e]);
      r[e + 4] = (__bf16)((float)hi[e] * fhi[e]);
    }
    return r;
  }
  // as load_scaled with the per-channel factor fac1 * fac2
  __device__ static __forceinline__ Frag load_scaled2(const E* tile, int ld, int row, int p,
                                                      int q, const float* fac1,
                                                      const float* fac2) {
    return load_scaled2_at(tile, ld, row, p, p, q, fac1, fac2);
  }
  __device__ static __forceinline__ Frag load_scaled2_at(const E* tile, int ld, int row, int p,
                                                         int pf, int q, const float* fac1,
                                                         const float* fac2) {
    const E* base = tile + row * ld + 32 * p + 4 * q;
    const int o = 32 * pf + 4 * q;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(base);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + 16);
    f32x4 alo = *reinterpret_cast<const f32x4*>(fac1 + o);
    f32x4 ahi = *reinterpret_cast<const f32x4*>(fac1 + o + 16);
    f32x4 blo = *reinterpret_cast<const f32x4*>(fac2 + o);
    f32x4 bhi = *reinterpret_cast<const f32x4*>(fac2 + o + 16);
    Frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (__bf16)((float)lo[e] * (alo[e] * blo[e]));
      r[e + 4] = (__bf16)((float)hi[e] * (ahi[e] * bhi[e]));
    }
    return r;
  }
  // A bf16 hi + lo pair of tiles, recombined per k in fp32, scaled by the product of NF
  // per-k factors (fp32, multiplied in order) and split again into a bf16 hi + lo pair: the
  // scaled operand keeps the pair's ~16 significant bits instead of one bf16's 8
  template <int NF>
  __device__ static __forceinline__ void load_pair_scaled(const E* thi, const E* tlo, int ld,
                                                          int row, int p, int q,
                                                          const float* const (&fac)[3],
                                                          Frag& h, Frag& l) {
    load_pair_scaled_at<NF>(thi, tlo, ld, row, p, p, q, fac, h, l);
  }
  template <int NF>
  __device__ static __forceinline__ void load_pair_scaled_at(const E* thi, const E* tlo, int ld,
                                                             int row, int p, int pf, int q,
                                                             const float* const (&fac)[3],
                                                             Frag& h, Frag& l) {
    const int ot = 32 * p + 4 * q;
    const int o = 32 * pf + 4 * q;
    const E* bh = thi + row * ld + ot;
    const E* bl = tlo + row * ld + ot;
    const bf16x4 h0 = *reinterpret_cast<const bf16x4*>(bh);
    const bf16x4 h1 = *reinterpret_cast<const bf16x4*>(bh + 16);
    const bf16x4 l0 = *reinterpret_cast<const bf16x4*>(bl);
    const bf16x4 l1 = *reinterpret_cast<const bf16x4*>(bl + 16);
    f32x4 f0 = *reinterpret_cast<const f32x4*>(fac[0] + o);
    f32x4 f1 = *reinterpret_cast<const f32x4*>(fac[0] + o + 16);
#pragma unroll
    for (int i = 1; i < NF; ++i) {
      f0 *= *reinterpret_cast<const f32x4*>(fac[i] + o);
      f1 *= *reinterpret_cast<const f32x4*>(fac[i] + o + 16);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = ((float)h0[e] + (float)l0[e]) * f0[e];
      const float x1 = ((float)h1[e] + (float)l1[e]) * f1[e];
      h[e] = (__bf16)x0;
      h[e + 4] = (__bf16)x1;
      l[e] = (__bf16)(x0 - (float)h[e]);
      l[e + 4] = (__bf16)(x1 - (float)h[e + 4]);
    }
  }
  // B fragment of slice p from accumulator tiles acc[2p] and acc[2p + 1], as a hi + lo pair:
  // hi = bf16(x), lo = bf16(x - hi)
  __device__ static __forceinline__ void from_acc_split(const f32x4* acc, int p, Frag& hi,
                                                        Frag& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = acc[2 * p + (e >> 2)][e & 3];
      const __bf16 xh = (__bf16)x;
      hi[e] = xh;
      lo[e] = (__bf16)(x - (float)xh);
    }
  }
  // fp16 operands (v_mfma_f32_16x16x32_f16, same k-order) for the products whose factors are
  // bounded well inside the fp16 range: an 11-bit significand in one MFMA, where a single
  // bf16 (8 bits) would need a hi + lo pair and three MFMAs
  using ER = _Float16;
  using FragR = f16x8;
  __device__ static __forceinline__ f32x4 mma_r(FragR a, FragR b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ FragR load_r(const ER* tile, int ld, int row, int p, int q) {
    const ER* base = tile + row * ld + 32 * p + 4 * q;
    f16x4 lo = *reinterpret_cast<const f16x4*>(base);
    f16x4 hi = *reinterpret_cast<const f16x4*>(base + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ static __forceinline__ FragR from_acc_r(const f32x4* acc, int p) {
    const f32x4 a = acc[2 * p], b = acc[2 * p + 1];
    const f16x4 ra = __builtin_convertvector(a, f16x4), rb = __builtin_convertvector(b, f16x4);
    return __builtin_shufflevector(ra, rb, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // fp16 hi + lo pair (~22 significant bits): hi = fp16(x), lo = fp16(x - hi)
  __device__ static __forceinline__ void from_acc_split_r(const f32x4* acc, int p, FragR& hi,
                                                          FragR& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = acc[2 * p + (e >> 2)][e & 3];
      const _Float16 xh = (_Float16)x;
      hi[e] = xh;
      lo[e] = (_Float16)(x - (float)xh);
    }
  }
};

// fp32 operands, v_mfma_f32_16x16x4_f32. Slice p covers rows {16 (p/4) + 4q + p%4 : q}.
struct PolF32 {
  using E = float;
  using Frag = float;
  static constexpr int kSlice = 4;
  static constexpr bool kSplit = false;  // fp32 operands need no second part
  __device__ static __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static constexpr int slices(int k) { return k / 4; }
  static constexpr int slices_blocks(int nb) { return 4 * nb; }
  __device__ static __forceinline__ Frag load(const E* tile, int ld, int row, int p, int q) {
    return tile[row * ld + 16 * (p >> 2) + 4 * q + (p & 3)];
  }
  __device__ static __forceinline__ Frag load_scaled(const E* tile, int ld, int row, int p,
                                                     int q, const float* fac) {
    const int kk = 16 * (p >> 2) + 4 * q + (p & 3);
    return tile[row * ld + kk] * fac[kk];
  }
  __device__ static __forceinline__ Frag load_scaled2(const E* tile, int ld, int row, int p,
                                                      int q, const float* fac1,
                                                      const float* fac2) {
    const int kk = 16 * (p >> 2) + 4 * q + (p & 3);
    return tile[row * ld + kk] * (fac1[kk] * fac2[kk]);
  }
  __device__ static __forceinline__ Frag from_acc(const f32x4* acc, int p) {
    return acc[p >> 2][p & 3];
  }
  __device__ static __forceinline__ void from_acc_split(const f32x4* acc, int p, Frag& hi,
                                                        Frag& lo) {
    hi = acc[p >> 2][p & 3];
    lo = 0.f;
  }
  using ER = float;
  using FragR = float;
  __device__ static __forceinline__ f32x4 mma_r(FragR a, FragR b, f32x4 c) { return mma(a, b, c); }
  __device__ static __forceinline__ FragR load_r(const ER* tile, int ld, int row, int p, int q) {
    return load(tile, ld, row, p, q);
  }
  __device__ static __forceinline__ FragR from_acc_r(const f32x4* acc, int p) { return from_acc(acc, p); }
  __device__ static __forceinline__ void from_acc_split_r(const f32x4* acc, int p, FragR& hi,
                                                          FragR& lo) {
    from_acc_split(acc, p, hi, lo);
  }
};

// fp32 MFMA on a natural k-order (used by the triangular inverse): slice s holds k = 4s + q.
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Cross-lane moves inside each quad of four lanes (DPP quad_perm: lane i of the quad reads
// lane sel[i]).
template <int kCtrl>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl,
                                                            0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;   // [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;   // [2, 3, 0, 1]
template <int kSrc>
__device__ __forceinline__ float quad_bcast(float v) {
  return quad_perm<kSrc * 0x55>(v);   // [kSrc, kSrc, kSrc, kSrc]
}

// Workgroup barrier that orders LDS only: global loads and stores stay in flight across it
// (a full barrier's fence waits for every outstanding global access, stores included). For
// kernels whose threads never read global memory that another thread of the workgroup
// wrote during the launch; data staged by global-to-LDS loads is waited for by each wave
// (vmcnt) before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sums across lanes without LDS traffic (DPP and the gfx950 row-swap instructions). Each
// returns x + x' where x' is the value of the partner lane named; both partners get the same
// bits (fp32 addition commutes).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_xor1(float x) { return x + quad_perm<0xB1>(x); }
__device__ __forceinline__ float sum_xor2(float x) { return x + quad_perm<0x4E>(x); }
// partner 7 - l inside each group of eight (after sum_xor1 and sum_xor2 this completes the
// sum over the eight lanes)
__device__ __forceinline__ float sum_mirror8(float x) { return x + dpp_mov<0x141>(x); }
// partner l ^ 8 inside each row of sixteen (row rotation by eight)
__device__ __forceinline__ float sum_xor8(float x) { return x + dpp_mov<0x128>(x); }
// partner l ^ 16: v_permlane16_swap exchanges the odd rows of one copy with the even rows of
// the other, so the two results hold x[l] and x[l ^ 16] in row order in every lane
__device__ __forceinline__ float sum_xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, unsigned(r[0])) + __builtin_bit_cast(float, unsigned(r[1]));
}
// partner l ^ 32, with v_permlane32_swap on the two halves of the wave
__device__ __forceinline__ float sum_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, unsigned(r[0])) + __builtin_bit_cast(float, unsigned(r[1]));
}

// 4 x 4 transpose across a quad: lane a of the quad holds row a in x[0..3] and afterwards
// holds column a (two exchange stages: 2 x 2 blocks, then the off-diagonal pair of blocks).
__device__ __forceinline__ void quad_transpose(float x[4], int lane) {
  const bool odd = (lane & 1) != 0, up = (lane & 2) != 0;
  float r0 = quad_perm<kQuadXor1>(odd ? x[0] : x[1]);
  float r1 = quad_perm<kQuadXor1>(odd ? x[2] : x[3]);
  x[0] = odd ? r0 : x[0];
  x[1] = odd ? x[1] : r0;
  x[2] = odd ? r1 : x[2];
  x[3] = odd ? x[3] : r1;
  r0 = quad_perm<kQuadXor2>(up ? x[0] : x[2]);
  r1 = quad_perm<kQuadXor2>(up ? x[1] : x[3]);
  x[0] = up ? r0 : x[0];
  x[1] = up ? r1 : x[1];
  x[2] = up ? x[2] : r0;
  x[3] = up ? x[3] : r1;
}

}  // namespace kda
