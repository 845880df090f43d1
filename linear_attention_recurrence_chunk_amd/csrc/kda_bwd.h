// Launch parameters of the 16-token chunk form of the recurrence on fp32 matrix cores: the
// backward (gradients of kda_chunk_fwd's outputs) and the fp32 prefill at d = 128.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// 16-token chunks, every product on fp32 matrix cores
constexpr int kCBChunk = 16;

struct CBwdParams {
  const void* q;            // [T, H, DK] io dtype
  const void* k;
  const void* v;            // [T, H, DV]
  const float* g;           // [T, H, DK]
  const float* beta;        // [T, H]
  const float* h0;          // [N, H, DK, DV] or null (zeros)
  const void* d_o;          // [T, H, DV] io dtype: dL/do
  const float* dht;         // [N, H, DK, DV] or null (zeros)
  const int32_t* cu_seqlens;  // device [N + 1] or null (fixed length seq_len)
  int seq_len, n_seqs, H, n_ct;   // n_ct: 16-column state tiles per head (DV / 16)
  int n_units;              // n_seqs * H
  // the launch's sequences i = 0 .. n_seqs - 1 are the call's sequences seq0 + i (first token
  // bos); their chunk slots count from token slot_tok0 (a group of sequences of the prefill)
  int seq0, slot_tok0;
  long long T;              // tokens in all
  long long n_slots;        // chunk slots: T / 16 + N + 1
  float scale, g_min;
  float* dq;                // [T, H, DK] fp32 outputs
  float* dk;
  float* dv;                // [T, H, DV]
  float* dg;                // [T, H, DK]
  float* dbeta;             // [T, H]
  float* dh0;               // [N, H, DK, DV] or null
  // workspace, per chunk slot and head; chunk c of sequence n (first token bos_n) uses slot
  // floor(bos_n / 16) + n + c
  float* S0;                // [slots, H, DK, DV] state entering the chunk
  float* dS;                // [slots, H, DK, DV] dL/d(state leaving the chunk)
  float* U;                 // [slots, H, 16, DV] T diag(beta) (V - K_Gamma S0)
  float* X0;                // [slots, H, 16, DV] V - K_Gamma S0
  float* dU;                // [slots, H, 16, DV]
  float* dY;                // [slots, H, 16, DV] T^T dU
  float* ops;               // [slots, H, cbwd_op_floats(DK)] per-chunk operand blocks
  // the prefill's outputs
  float* o;                 // [T, H, DV]
  float* ht;                // [N, H, DK, DV] or null
  float* ckpt;              // [floor(T / ckpt_every), H, DK, DV] or null
  int ckpt_every;           // a multiple of 64 when ckpt is set
};

// floats of one (chunk slot, head) operand block: three 16 x dk tiles, two 16 x 16 matrices,
// dk decay factors and 16 betas
inline constexpr size_t cbwd_op_floats(int dk) { return 49 * size_t(dk) + 528; }

inline long long cbwd_slots(long long T, long long N) { return T / kCBChunk + N + 1; }

// Workspace bytes of the chunked backward for T tokens in N sequences
inline size_t cbwd_workspace_bytes(long long T, long long N, int H, int dk, int dv) {
  return size_t(cbwd_slots(T, N)) * H *
         (2 * size_t(dk) * dv + 4 * size_t(kCBChunk) * dv + cbwd_op_floats(dk)) * 4;
}

// Points p's workspace arrays into ws (at least cbwd_workspace_bytes(p.T, p.n_seqs, p.H, dk,
// dv) bytes, 16-byte aligned); p.T, p.n_seqs and p.H must be set.
inline void cbwd_bind_workspace(CBwdParams& p, void* ws, int dk, int dv) {
  const size_t slots = size_t(cbwd_slots(p.T, p.n_seqs));
  const size_t st = slots * p.H * dk * dv;          // one [slots, H, dk, dv] array
  const size_t rows = slots * p.H * kCBChunk * dv;  // one [slots, H, 16, dv] array
  float* f = static_cast<float*>(ws);
  p.S0 = f;
  p.dS = f + st;
  p.U = f + 2 * st;
  p.X0 = f + 2 * st + rows;
  p.dU = f + 2 * st + 2 * rows;
  p.dY = f + 2 * st + 3 * rows;
  p.ops = f + 2 * st + 4 * rows;
}

hipError_t launch_chunk_bwd_mfma(const CBwdParams& p, int io_dtype, int dk, hipStream_t stream);

// Workspace bytes of the fp32 prefill at d = 128 for T tokens in N sequences: the operand blocks
inline size_t c16_prefill_workspace_bytes(long long T, long long N, int H, int dk) {
  return size_t(cbwd_slots(T, N)) * H * cbwd_op_floats(dk) * 4;
}

// The fp32 prefill (o, ht, checkpoints) of the launch's sequences: the operand pass, then the
// walk. p.ops holds c16_prefill_workspace_bytes of the launch's tokens and sequences.
hipError_t launch_c16_prefill(const CBwdParams& p, int dk, hipStream_t stream);

}  // namespace kda
