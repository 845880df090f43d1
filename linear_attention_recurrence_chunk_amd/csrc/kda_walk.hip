// Pass 2 of the two-launch prefill on gfx950: the serial chunk walk over the operand slots
// the prep pass of the chunk kernel writes (see kda_chunk.hip for the method and the
// precision design of the products).
#include "kda_chunk_io.h"
#include "kda_common.h"
#include "kda_internal.h"


namespace kda {

// The walk's products as a fixed sequence of stages, each one group of operand fragments
// (at most eight) and the MFMAs that consume them, in an order that keeps the state's chain
// (X, its split, U, its split, the state update) short: the products with decayed queries
// (O) fill the MFMA unit while the splits run. Every accumulator sees its products in the
// same order as in the chunk kernel's serial step.
template <int DK, bool kOut = true>
struct WalkPlan {
  using OS = OpSlot<DK>;
  static constexpr int NS = OS::NS;
  static constexpr int NTD = OS::NTD;
  enum : int { kK, kQ, kT, kKh, kM };
  // K 0..NS-1 | Q 0..kQ1-1 | T 0,1 | Q kQ1..NS-1 | Kh (pp, t0) | M 0,1; without outputs there
  // are no Q and M stages
  static constexpr int kQ1 = kOut ? NS / 2 : 0;        // Q stages before the X split
  static constexpr int sQ1 = NS;
  static constexpr int sT = sQ1 + kQ1;
  static constexpr int sQ2 = sT + 2;
  static constexpr int sKh = sQ2 + (kOut ? NS - kQ1 : 0);
  static constexpr int sM = sKh + 2 * (NTD / 4);
  static constexpr int kStages = sM + (kOut ? 2 : 0);
  static constexpr int kAfterK = NS - 1;                // load the next chunk's values
  static constexpr int kAfterQ1 = sT - 1;               // split X
  static constexpr int kAfterQ2 = sKh - 1;              // negate and split U
  static constexpr __host__ __device__ int kind(int s) {
    return s < sQ1 ? kK : s < sT ? kQ : s < sQ2 ? kT : s < sKh ? kQ : s < sM ? kKh : kM;
  }
  // slice of the stage (the k-slice for K and Q, the token slice for T, M and Kh)
  static constexpr __host__ __device__ int pp(int s) {
    return s < sQ1 ? s
         : s < sT ? s - sQ1
         : s < sQ2 ? s - sT
         : s < sKh ? kQ1 + s - sQ2
         : s < sM ? (s - sKh) / (NTD / 4)
         : s - sM;
  }
  // first 16-row tile of the state updated by a Kh stage
  static constexpr __host__ __device__ int t0(int s) { return 4 * ((s - sKh) % (NTD / 4)); }
  static constexpr __host__ __device__ int count(int s) {
    return (kind(s) == kT || kind(s) == kM) ? (pp(s) == 0 ? 8 : 4) : 4;
  }
  // the slot blocks the walk reads, in fetch order (without outputs: no Q e^Gamma and no M)
  static constexpr int kFetched = kOut ? OS::kBlocks : 4 * NS + 12 + (OS::kBlocks - OS::fKh);
  static constexpr __host__ __device__ int fetched(int j) {
    return kOut ? j
         : j < 4 * NS ? OS::fKg + j
         : j < 4 * NS + 12 ? OS::fT + (j - 4 * NS)
         : OS::fKh + (j - 4 * NS - 12);
  }
  // fragment k of stage s
  static constexpr __host__ __device__ int frag(int s, int k) {
    const int kd = kind(s), p = pp(s);
    if (kd == kK) return OS::fKg + k * NS + p;
    if (kd == kQ) return OS::fQg + k * NS + p;
    if (kd == kKh) return OS::fKh + 2 * (t0(s) + k) + p;
    // T and M: hi of the stage's row blocks, then lo
    const int nr = p == 0 ? 4 : 2, rb0 = p == 0 ? 0 : 2;
    const int hi = kd == kT ? OS::fT : OS::fM, lo = kd == kT ? OS::fTLo : OS::fMLo;
    const int i = k < nr ? k : k - nr;
    return (k < nr ? hi : lo) + OS::tri(rb0 + i, p);
  }
};

// Pass 2 of the two-pass prefill: the serial walk over the chunks of one (sequence, head,
// 64-column state tile), with the prologue's operands read from the chunks' slots. The step is
// the chunk kernel's serial step, operation for operation, so the two paths agree bit for bit.
// Slots stream into two LDS buffers by direct global-to-LDS loads: the next chunk's slot is in
// flight while the current one is consumed, and the next chunk's values load into registers.
// kMem (one state tile per workgroup): a fifth wave issues every slot load. A 1 KiB
// global-to-LDS load occupies the compute unit's vector-memory queue for tens of cycles, and a
// wave stalls in order until the queue takes its load; the waves that compute would otherwise
// spend about a quarter of each chunk step issuing them. The fifth wave shares a SIMD with one
// of them, so every wave is held to 256 registers and the fragment look-ahead is one stage.
template <typename Tio, typename Tout, int DK, bool kOut, int kTPW, bool kMem>
__global__ __launch_bounds__(256 * kTPW + (kMem ? 64 : 0)) void chunk_walk_kernel(ChunkParams p) {
  using Pol = PolBF16;
  using Frag = typename Pol::Frag;
  using FragR = typename Pol::FragR;
  using OS = OpSlot<DK>;
  constexpr int NS = OS::NS;
  constexpr int NT = Pol::slices(64);
  constexpr int NTD = OS::NTD;
  constexpr int VT = 64;
  static_assert(2 * OS::kBytes <= 160 * 1024, "two slots fit the LDS of one compute unit");

  __shared__ __attribute__((aligned(16))) char smem[2 * OS::kBytes];

  // ---- which (sequence, segment, head) and which kTPW state tiles of it (four waves per
  //      tile): the workgroups of one unit share an XCD
  int vg;
  const int unit = block_unit(blockIdx.x, p.n_vt / kTPW, &vg);
  if (unit >= p.n_units) return;
  const int H = p.H;
  const int DV = p.dv;
  const int h = unit % H;
  const int sj = unit / H;              // global segment index n * n_seg + j
  const int n = p.seq0 + (p.n_order > 0 ? int(p.order[sj / p.n_seg]) : sj / p.n_seg);
  const int j = sj % p.n_seg;
  const int mode = p.mode;

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave in the workgroup
  const int w = wid & 3;                                       // wave in its state tile
  const int vt = vg * kTPW + (wid >> 2);
  const int lane = tid & 63;
  const int q4 = lane >> 4;
  const int ln = lane & 15;

  int bos, eos;
  if (p.cu_seqlens) {
    bos = p.cu_seqlens[n];
    eos = p.cu_seqlens[n + 1];
  } else {
    bos = n * p.seq_len;
    eos = bos + p.seq_len;
  }
  // operand slot of the sequence's first chunk, then the segment's chunk range (chunk-aligned
  // contiguous segments: segment j holds chunks [j nc / n_seg, (j+1) nc / n_seg))
  long long slot0 = seq_first_slot(bos, p.slot_tok0, n, p.seq0);
  {
    int c_lo;
    segment_range(bos, eos, j, p.n_seg, &bos, &eos, &c_lo);
    slot0 += c_lo;
  }
  const int nchunks = (eos - bos + kChunk - 1) / kChunk;
  const char* ws_head = p.ws_ops + (size_t(slot0) * H + h) * OS::kBytes;
  const size_t slot_stride = size_t(H) * OS::kBytes;   // from one chunk's slot to the next
  // transition: tiles [0, DK/64) hold P (zero values, identity start), the rest Q
  const bool p_tile = !kOut && vt < DK / 64;
  const int vcol0 = p_tile ? 0 : (kOut ? vt : vt - DK / 64) * VT;   // column of v feeding the tile
  const int col0 = vt * VT + 16 * w;   // first state column owned by this wave
  const int ldS = kOut ? DV : DK + DV;   // row stride of the state this tile writes
  Tout* __restrict__ go = reinterpret_cast<Tout*>(p.o);
  using Plan = WalkPlan<DK, kOut>;

  if constexpr (kMem) {
    if (wid == 4 * kTPW) {
      // the load wave: moves each chunk's slot into LDS a chunk ahead (the waves that compute
      // issue no slot loads, so they never stall on the memory pipeline's queue for them)
      auto fetch_all = [&](int ci, char* dst) {
        const char* src = ws_head + size_t(ci) * slot_stride;
#pragma unroll
        for (int jf = 0; jf < Plan::kFetched; ++jf) {
          const int f = Plan::fetched(jf);
          __builtin_amdgcn_global_load_lds(src + size_t(f) * 1024 + lane * 16, dst + f * 1024, 16,
                                           0, 0);
        }
      };
      if (nchunks > 0) fetch_all(0, smem);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      for (int ci = 0; ci < nchunks; ++ci) {
        if (ci + 1 < nchunks) fetch_all(ci + 1, smem + ((ci + 1) & 1) * OS::kBytes);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
      }
      return;
    }
  }

  // ---- entering state in accumulator layout: tile t, register e = row 16t + 4 q4 + e
  f32x4 S[NTD];
  const float* s_in = nullptr;
  if (mode == kModeWalk && p.h0) s_in = p.h0 + (size_t(n) * H + h) * DK * DV;
  if (mode == kModeReplay) s_in = p.ws_sin + (size_t(sj) * H + h) * DK * DV;
  if (s_in) {
    // all loads in flight together
    const float* src = s_in + col0 + ln;
#pragma unroll
    for (int t = 0; t < NTD; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[t][e] = src[size_t(16 * t + 4 * q4 + e) * DV];
  } else {
#pragma unroll
    for (int t = 0; t < NTD; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[t][e] = (p_tile && 16 * t + 4 * q4 + e == col0 + ln) ? 1.f : 0.f;
  }

  // waves 0..3 (one per SIMD) move blocks wid, wid + 4, ... of the fragment ranges the walk
  // reads (without outputs: no Q e^Gamma and no M) of chunk ci's slot into buffer dst; with
  // two tiles per workgroup the other wave of each SIMD issues none, so it computes while its
  // partner waits for the memory pipeline to take the loads (the global address is a
  // wave-uniform block address plus the lane's 16-byte offset)
  auto fetch_range = [&](const char* src, char* dst, int f0, int f1) {
    if (wid < 4) {
#pragma unroll
      for (int i = 0; i < (OS::kBlocks + 3) / 4; ++i) {
        const int f = f0 + wid + 4 * i;
        if (f < f1)
          __builtin_amdgcn_global_load_lds(src + size_t(f) * 1024 + lane * 16, dst + f * 1024,
                                           16, 0, 0);
      }
    }
  };
  auto fetch_slot = [&](int ci, char* dst) {
    const char* src = ws_head + size_t(ci) * slot_stride;
    if constexpr (kOut) {
      fetch_range(src, dst, 0, OS::kBlocks);
    } else {
      fetch_range(src, dst, OS::fKg, OS::fKg + 4 * NS);
      fetch_range(src, dst, OS::fT, OS::fTLo + 6);
      fetch_range(src, dst, OS::fKh, OS::kBlocks);
    }
  };

  RawChunk<Tio, DK> raw;
  // values of the chunk about to start, in accumulator layout and negated: the initial X
  const int tq = 4 * q4 + (ln & 3);
  f32x4 X0[4];
  auto values_to_x0 = [&](int L) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      float vx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vx[e] = to_f32(raw.v[rb][e]);
      quad_transpose(vx, lane);   // token 16 rb + 4 q4 + e, column 16 w + ln
      if (L == kChunk && !p_tile) {
#pragma unroll
        for (int e = 0; e < 4; ++e) X0[rb][e] = -vx[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) X0[rb][e] = (16 * rb + 4 * q4 + e < L && !p_tile) ? -vx[e] : 0.f;
      }
    }
  };
  if (nchunks > 0) {
    if constexpr (!kMem) fetch_slot(0, smem);
    if (!p_tile)
      load_chunk_any<kLoadV, Tio, DK>(raw, p, bos, min(kChunk, eos - bos), w, lane, h, vcol0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    values_to_x0(min(kChunk, eos - bos));
  }
  lds_barrier();

  // outputs of a chunk, transposed (lane: token 16 rb + tq, four consecutive columns)
  const uint32_t lo_el = uint32_t((tq * H + h) * DV + col0 + 4 * (ln >> 2));
  auto store_out = [&](const f32x4* Oc, int cst, int L) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      float ox[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ox[e] = p.scale * Oc[rb][e];
      quad_transpose(ox, lane);
      Tout* row = go + size_t(cst + 16 * rb) * H * DV;
      if (16 * rb + tq < L) {
        if constexpr (sizeof(Tout) == 2)
          *reinterpret_cast<bf16x4*>(row + lo_el) =
              bf16x4{(__bf16)ox[0], (__bf16)ox[1], (__bf16)ox[2], (__bf16)ox[3]};
        else
          *reinterpret_cast<f32x4*>(row + lo_el) = f32x4{ox[0], ox[1], ox[2], ox[3]};
      }
    }
  };

  using V16 = int __attribute__((ext_vector_type(4)));
  f32x4 O[4];
  for (int ci = 0; ci < nchunks; ++ci) {
    const int cstart = bos + ci * kChunk;
    const int Lc = min(kChunk, eos - cstart);
    const char* cur = smem + (ci & 1) * OS::kBytes;
    const bool more = ci + 1 < nchunks;
    // the next slot streams in behind this chunk (issued first: it has the whole chunk to land)
    if constexpr (!kMem) {
      if (more) fetch_slot(ci + 1, smem + ((ci + 1) & 1) * OS::kBytes);
    }

    // the state as fp16 B fragments (both products with decayed keys and queries), then its
    // decay for the update: S is not read again before S += K^T U
    FragR Sr[NS];
#pragma unroll
    for (int pp = 0; pp < NS; ++pp) Sr[pp] = Pol::from_acc_r(S, pp);
    {
      const float* decay = reinterpret_cast<const float*>(cur + OS::kDecay * 1024);
#pragma unroll
      for (int t = 0; t < NTD; ++t) {
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(decay + 16 * t + 4 * q4);
        S[t] *= dv4;
      }
    }

    // The products run as a fixed sequence of stages (Plan): each stage's fragments are read
    // from LDS two stages ahead of its MFMAs, into three rotating register buffers.
    // stages of fragment look-ahead: two with one wave per SIMD; one with two waves per SIMD
    // (both waves' registers fit the SIMD's file only then)
    constexpr int kAhead = kTPW == 1 && !kMem ? 2 : 1;
    V16 fb[kAhead + 1][8];
    auto load_stage = [&](int st, V16* dst) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k < Plan::count(st))
          dst[k] = *reinterpret_cast<const V16*>(cur + Plan::frag(st, k) * 1024 + lane * 16);
    };
    auto R = [](V16 x) { return __builtin_bit_cast(FragR, x); };
    auto B = [](V16 x) { return __builtin_bit_cast(Frag, x); };
    f32x4 X[4], U[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) X[rb] = X0[rb];
    Frag Xh[NT], Xl[NT];
    FragR Uh[NT], Ul[NT];
    static_for<0, kAhead>([&](auto a) { load_stage(decltype(a)::value, fb[decltype(a)::value]); });
    static_for<0, Plan::kStages>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      if constexpr (st + kAhead < Plan::kStages) load_stage(st + kAhead, fb[(st + kAhead) % (kAhead + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      V16* f = fb[st % (kAhead + 1)];
      constexpr int kind = Plan::kind(st), pp = Plan::pp(st);
      if constexpr (kind == Plan::kK) {
        // X = (K e^Gamma) S - V
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) X[rb] = Pol::mma_r(R(f[rb]), Sr[pp], X[rb]);
      } else if constexpr (kind == Plan::kQ) {
        // O = (Q e^Gamma) S
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) O[rb] = Pol::mma_r(R(f[rb]), Sr[pp], pp == 0 ? zero4() : O[rb]);
      } else if constexpr (kind == Plan::kT) {
        // U = T' (V - K_Gamma S) = -T' X; stage pp holds hi then lo of row blocks rb0..3
        constexpr int kMax = 4;
        const int rb0 = pp == 0 ? 0 : 2, nr = pp == 0 ? 4 : 2;
#pragma unroll
        for (int i = 0; i < kMax; ++i)
          if (i < nr) U[rb0 + i] = Pol::mma(B(f[i]), Xh[pp], pp == 0 ? zero4() : U[rb0 + i]);
#pragma unroll
        for (int i = 0; i < kMax; ++i)
          if (i < nr) U[rb0 + i] = Pol::mma(B(f[nr + i]), Xh[pp], U[rb0 + i]);
#pragma unroll
        for (int i = 0; i < kMax; ++i)
          if (i < nr) U[rb0 + i] = Pol::mma(B(f[i]), Xl[pp], U[rb0 + i]);
      } else if constexpr (kind == Plan::kKh) {
        // S += (K e^{Gamma_L - Gamma})^T U, U as an fp16 hi + lo pair
        const int t0 = Plan::t0(st);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t0 + t] = Pol::mma_r(R(f[t]), Uh[pp], S[t0 + t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t0 + t] = Pol::mma_r(R(f[t]), Ul[pp], S[t0 + t]);
      } else {
        // O += M U, M and U as fp16 hi + lo pairs
        const int rb0 = pp == 0 ? 0 : 2, nr = pp == 0 ? 4 : 2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nr) O[rb0 + i] = Pol::mma_r(R(f[i]), Uh[pp], O[rb0 + i]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nr) O[rb0 + i] = Pol::mma_r(R(f[nr + i]), Uh[pp], O[rb0 + i]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nr) O[rb0 + i] = Pol::mma_r(R(f[i]), Ul[pp], O[rb0 + i]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // work off the state's chain, placed where the products above keep the MFMA unit busy
      if constexpr (st == Plan::kAfterK) {
        // the next chunk's values
        if (more && !p_tile) {
          const int nstart = cstart + kChunk;
          load_chunk_any<kLoadV, Tio, DK>(raw, p, nstart, min(kChunk, eos - nstart), w, lane, h,
                                          vcol0);
        }
      }
      if constexpr (st == Plan::kAfterQ1) {
#pragma unroll
        for (int q = 0; q < NT; ++q) Pol::from_acc_split(X, q, Xh[q], Xl[q]);
      }
      if constexpr (st == Plan::kAfterQ2) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) U[rb] = -U[rb];
#pragma unroll
        for (int q = 0; q < NT; ++q) Pol::from_acc_split_r(U, q, Uh[q], Ul[q]);
      }
    });
    if (mode == kModeWalk) write_checkpoint<DK, NTD>(p, S, bos, cstart + Lc, Lc, h, col0, q4, ln);
    if (more) {
      // the next slot (and values) must have landed before any wave reads them; this
      // chunk's output stores are issued after the wait, so it never waits on them
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      values_to_x0(min(kChunk, eos - cstart - kChunk));
    }
    if constexpr (kOut) store_out(O, cstart, Lc);
    lds_barrier();
  }

  float* s_out = nullptr;
  if (mode == kModeWalk && p.ht) s_out = p.ht + (size_t(n) * H + h) * DK * DV;
  if (mode == kModeTransition) s_out = p.ws_pq + (size_t(sj) * H + h) * DK * ldS;
  if (s_out) {
#pragma unroll
    for (int t = 0; t < NTD; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_out[size_t(16 * t + 4 * q4 + e) * ldS + col0 + ln] = S[t][e];
  }
}

// Tv: the values' type (bf16 inputs, or the fp32 convolved values of the raw prefill)
template <typename Tv, typename Tout, int DK, int kTPW>
static hipError_t launch_walk_tpw(const ChunkParams& p, hipStream_t stream) {
  // one state tile per workgroup: four waves that compute and a fifth that loads the slots
  constexpr bool kMem = kTPW == 1;
  const dim3 grid((p.n_units + 7) / 8 * 8 * (p.n_vt / kTPW));
  const dim3 block(256 * kTPW + (kMem ? 64 : 0));
  if (p.mode == kModeTransition)
    hipLaunchKernelGGL((chunk_walk_kernel<Tv, Tout, DK, false, kTPW, kMem>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((chunk_walk_kernel<Tv, Tout, DK, true, kTPW, kMem>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename Tout, int DK>
static hipError_t launch_walk(const ChunkParams& p, hipStream_t stream, bool v_f32) {
  if (v_f32) {
    // (the raw prefill: forward walks only)
    if (p.mode == kModeTransition) return hipErrorInvalidValue;
    if (p.walk_tpw == 2) return launch_walk_tpw<float, Tout, DK, 2>(p, stream);
    return launch_walk_tpw<float, Tout, DK, 1>(p, stream);
  }
  if (p.walk_tpw == 2) return launch_walk_tpw<__bf16, Tout, DK, 2>(p, stream);
  return launch_walk_tpw<__bf16, Tout, DK, 1>(p, stream);
}

hipError_t launch_chunk_walk(const ChunkParams& p, int out_dtype, int dk, hipStream_t stream,
                             bool v_f32) {
  if (!p.ws_ops || !p.v || p.H < 1 || p.n_seqs < 1 || p.n_seg < 1 || p.dv != dk ||
      (long long)p.n_units != (long long)p.n_seqs * p.n_seg * p.H ||
      (!p.cu_seqlens && p.seq_len < 0))
    return hipErrorInvalidValue;
  if ((p.walk_tpw != 1 && p.walk_tpw != 2) || p.n_vt % p.walk_tpw != 0) return hipErrorInvalidValue;
  switch (p.mode) {
    case kModeWalk:
      if (p.n_seg != 1 || p.n_vt != p.dv / 64 || !p.o) return hipErrorInvalidValue;
      break;
    case kModeTransition:
      if (p.n_vt != (dk + p.dv) / 64 || !p.ws_pq) return hipErrorInvalidValue;
      break;
    case kModeReplay:
      if (p.n_vt != p.dv / 64 || !p.ws_sin || !p.o) return hipErrorInvalidValue;
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (dk == 128) return out_dtype == 1 ? launch_walk<__bf16, 128>(p, stream, v_f32)
                                       : launch_walk<float, 128>(p, stream, v_f32);
  if (dk == 64) return out_dtype == 1 ? launch_walk<__bf16, 64>(p, stream, v_f32)
                                      : launch_walk<float, 64>(p, stream, v_f32);
  return hipErrorInvalidValue;
}

}  // namespace kda
