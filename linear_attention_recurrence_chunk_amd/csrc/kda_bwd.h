// Launch parameters of the backward of the recurrence (gradients of kda_chunk_fwd's outputs).
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
};

inline long long cbwd_slots(long long T, long long N) { return T / kCBChunk + N + 1; }

// Workspace bytes of the chunked backward for T tokens in N sequences
inline size_t cbwd_workspace_bytes(long long T, long long N, int H, int dk, int dv) {
  return size_t(cbwd_slots(T, N)) * H * (2 * size_t(dk) * dv + 4 * size_t(kCBChunk) * dv) * 4;
}

hipError_t launch_chunk_bwd_mfma(const CBwdParams& p, int io_dtype, int dk, hipStream_t stream);

}  // namespace kda
