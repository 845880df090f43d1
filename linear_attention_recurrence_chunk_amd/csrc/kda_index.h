// Index arithmetic of the prefill kernels that decides which rows of the caller's buffers a
// workgroup touches: the workgroup -> (sequence, segment, head) decoding, segment and slot
// ranges, and the raw-projection prep pass's convolution rows. The kernels call these
// functions, and a host program (tests/addrcheck) calls the same ones to replay every access of
// a launch against the allocation extents on the CPU. Plain C++: no HIP types.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#if defined(__HIPCC__)
#define KDA_HD __host__ __device__ __forceinline__
#else
#define KDA_HD inline
#endif

namespace kda {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kMaxOrder = 256;   // sequences a walk can reorder (launch-parameter bytes)

// Workgroup b of a grid of (units rounded up to 8) x per_unit workgroups: the per_unit
// workgroups of one unit get block ids that agree mod 8, so they run on one XCD. Returns the
// unit (possibly >= the unit count: such workgroups exit) and sets *sub to the workgroup's
// index inside its unit.
KDA_HD int block_unit(int b, int per_unit, int* sub) {
  const int xcd = b & 7;
  const int rest = b >> 3;
  *sub = rest % per_unit;
  return (rest / per_unit) * 8 + xcd;
}

// Chunk-aligned contiguous segments of a sequence [seq_bos, seq_eos): segment j of n_seg holds
// chunks [j nc / n_seg, (j + 1) nc / n_seg). Sets its token range and first chunk.
KDA_HD void segment_range(int seq_bos, int seq_eos, int j, int n_seg, int* bos, int* eos,
                          int* c_lo) {
  if (n_seg <= 1) {
    *bos = seq_bos;
    *eos = seq_eos;
    *c_lo = 0;
    return;
  }
  const long long nc = (seq_eos - seq_bos + kChunk - 1) / kChunk;
  const int lo = int((j * nc) / n_seg);
  const int hi = int(((j + 1) * nc) / n_seg);
  *c_lo = lo;
  *bos = seq_bos + kChunk * lo;
  *eos = seq_eos < seq_bos + kChunk * hi ? seq_eos : seq_bos + kChunk * hi;
}

// Operand slot of a sequence's first chunk: sequence n (first token seq_bos) of a group that
// starts at sequence seq0 and token slot_tok0 uses slots from (seq_bos - slot_tok0) / 64 +
// (n - seq0) on, so packed sequences never share one.
KDA_HD long long seq_first_slot(int seq_bos, int slot_tok0, int n, int seq0) {
  return (long long)((seq_bos - slot_tok0) >> 6) + (n - seq0);
}

// ---- raw-projection prep pass (short causal convolution of width W <= 4 over q, k and v)

// Thread mapping of the value convolution: thread tid owns value channels cv0 .. cv0 + 3 of
// kTPV consecutive tokens from tv0 (DK / 4 channel quads over the 256 threads).
template <int DK>
struct RawValueMap {
  static constexpr int kQuads = DK / 4;
  static constexpr int kTPV = 64 / (256 / kQuads);
  static KDA_HD int cv0(int tid) { return 4 * (tid % kQuads); }
  static KDA_HD int tv0(int tid) { return kTPV * (tid / kQuads); }
};

// Convolution history of the prologue's q and k: the row i + 1 tokens before a thread's first
// token (chunk row rb0) of the chunk starting at cs with L rows. The token whose input row the
// thread loads, or -1 when it loads none: rows of taps the width does not reach, rows before
// the sequence (they come from the entering tail), and rows past the chunk's last one (threads
// whose rows lie past a ragged last chunk discard their outputs).
KDA_HD int raw_history_row(int cs, int L, int rb0, int i, int W, int seq_bos) {
  const int tok = cs + rb0 - 1 - i;
  return (i + 1 < W && tok >= seq_bos && tok < cs + L) ? tok : -1;
}

// The entering-tail slot (oldest first, W - 1 per channel) of that history row when it lies
// before the sequence and the width reaches it, else -1.
KDA_HD int raw_history_tail_slot(int cs, int rb0, int i, int W, int seq_bos) {
  const int tok = cs + rb0 - 1 - i;
  return (i + 1 < W && tok < seq_bos) ? (W - 1) - (seq_bos - tok) : -1;
}

// Rows of the value convolution: window entry i (0 .. kTPV + 2) of a thread whose tokens start
// at chunk row tv0 is token cs + tv0 - 3 + i. The token whose input row it loads, or -1: taps
// the width does not reach, rows past the chunk's last one, rows before the sequence.
KDA_HD int raw_value_row(int cs, int L, int tv0, int i, int W, int seq_bos) {
  const int tok = cs + tv0 - 3 + i;
  return (i >= 4 - W && tok < cs + L && tok >= seq_bos) ? tok : -1;
}

// The entering-tail slot of window entry i when it lies before the sequence, else -1.
KDA_HD int raw_value_tail_slot(int cs, int L, int tv0, int i, int W, int seq_bos) {
  const int tok = cs + tv0 - 3 + i;
  return (i >= 4 - W && tok < cs + L && tok < seq_bos) ? (W - 1) - (seq_bos - tok) : -1;
}

// Entry m (oldest first) of a sequence's leaving tail: the last W - 1 raw inputs. The input row
// it copies, or -1 when the sequence is shorter than the tail and the entry comes from the
// entering tail, at slot *tail_slot.
KDA_HD int raw_tail_out_row(int seq_bos, int seq_eos, int W, int m, int* tail_slot) {
  const int pos = seq_eos - (W - 1) + m;
  *tail_slot = pos >= seq_bos ? -1 : m + (seq_eos - seq_bos);
  return pos >= seq_bos ? pos : -1;
}

// ---- host-side plan of the two-launch prefill (which groups, slots and workspace regions)

// Operand slots: chunk c of sequence n (bos_n its first token) uses slot (bos_n / 64) + n + c,
// so slots never collide and there are at most total_tokens / 64 + n_seqs + 1 of them (for a
// group of sequences: its tokens and its sequence count).
inline long long op_slot_count(long long total_tokens, long long n_seqs) {
  return total_tokens / 64 + n_seqs + 1;
}
// bytes of one (slot, head) operand block for key width dk (MFMA fragments of 1 KiB each plus
// one block for the whole-chunk decay)
inline size_t op_slot_bytes(int dk) { return size_t(8 * (dk / 32) + 24 + 2 * (dk / 16) + 1) * 1024; }

inline size_t two_pass_workspace_bytes(int64_t T, int64_t N, int H, int dk) {
  return size_t(op_slot_count(T, N)) * size_t(H) * op_slot_bytes(dk);
}

// fp32 convolved values of the raw-projection prefill, [T, H, dv], rounded up to 256 bytes
inline size_t raw_vconv_bytes(int64_t T, int H, int dv) {
  return (size_t(T) * H * dv * 4 + 255) / 256 * 256;
}

// Chunks per workgroup of the prep pass (its loop prefetches each chunk's inputs during the
// previous one)
constexpr int kPrepChunks = 8;

inline int64_t max_seq_len(const int32_t* cu_seqlens_host, int N, int seq_len) {
  if (!cu_seqlens_host) return seq_len;
  int64_t m = 0;
  for (int i = 0; i < N; ++i) {
    const int64_t len = int64_t(cu_seqlens_host[i + 1]) - cu_seqlens_host[i];
    m = len > m ? len : m;
  }
  return m;
}

// chunk groups per sequence of the prep pass
inline int prep_groups(const int32_t* cu_seqlens_host, int N, int seq_len) {
  const int64_t max_chunks = (max_seq_len(cu_seqlens_host, N, seq_len) + 63) / 64;
  const int64_t groups = (max_chunks + kPrepChunks - 1) / kPrepChunks;
  return groups < 1 ? 1 : int(groups);
}

// The order in which a walk takes the sequences n0 .. n1 - 1 of a group: longest first, ties
// in sequence order. Fills order[0 .. m) with sequence offsets and returns m, or 0 (own order)
// without offsets, for a single sequence or more than kMaxOrder of them.
inline int walk_order(const int32_t* cu_seqlens_host, int n0, int n1, uint16_t* order) {
  const int m = n1 - n0;
  if (!cu_seqlens_host || m < 2 || m > kMaxOrder) return 0;
  for (int i = 0; i < m; ++i) order[i] = uint16_t(i);
  auto len = [&](uint16_t i) { return cu_seqlens_host[n0 + i + 1] - cu_seqlens_host[n0 + i]; };
  std::stable_sort(order, order + m, [&](uint16_t a, uint16_t b) { return len(a) > len(b); });
  return m;
}

// Consecutive groups of whole sequences, each as long as need(tokens, sequences) fits the
// budget (at least one sequence per group); run(n0, n1, first token, tokens) is called for
// each in order and the first status other than ok is returned. Sequences are independent, so
// nothing passes between groups.
template <class Need, class Run>
int for_each_group(int N, const int32_t* cu_seqlens_host, int seq_len, size_t budget, Need need,
                   Run run, int ok) {
  auto first_tok = [&](int n) -> int64_t {
    return cu_seqlens_host ? int64_t(cu_seqlens_host[n]) : int64_t(n) * seq_len;
  };
  for (int n0 = 0; n0 < N;) {
    int n1 = n0 + 1;
    while (n1 < N && need(first_tok(n1 + 1) - first_tok(n0), n1 + 1 - n0) <= budget) ++n1;
    const int rc = run(n0, n1, first_tok(n0), first_tok(n1) - first_tok(n0));
    if (rc != ok) return rc;
    n0 = n1;
  }
  return ok;
}

}  // namespace kda
