// Launch parameters of the backward of the recurrence (gradients of kda_chunk_fwd's outputs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct BwdParams {
  const void* q;            // [T, H, DK] io dtype
  const void* k;
  const void* v;            // [T, H, DV]
  const float* g;           // [T, H, DK]
  const float* beta;        // [T, H]
  const float* h0;          // [N, H, DK, DV] or null (zeros)
  const void* d_o;          // [T, H, DV] io dtype: dL/do
  const float* dht;         // [N, H, DK, DV] or null (zeros): dL/d(final state)
  const int32_t* cu_seqlens;  // device [N + 1] or null (fixed length seq_len)
  int seq_len, n_seqs, H, n_ct;   // n_ct: 16-column state tiles per head (DV / 16)
  int n_units;              // n_seqs * H
  long long T;              // tokens in all
  float scale, g_min;
  // outputs (fp32)
  float* dq;                // [T, H, DK]
  float* dk;
  float* dv;                // [T, H, DV]
  float* dg;                // [T, H, DK]
  float* dbeta;             // [T, H]
  float* dh0;               // [N, H, DK, DV] or null
  // workspace
  float* ckpt;              // [T / 16 + N + 1, H, DK, DV] states at every 16th token
  float* part;              // [3, n_ct, T, H, DK] per-tile sums of dq, dk, da
  float* part_beta;         // [4 n_ct, T, H] per-wave sums of dbeta
};

// tokens between the backward's state checkpoints (a sub-chunk, recomputed in registers)
constexpr int kBwdSub = 8;

inline long long bwd_ckpt_slots(long long T, long long N) { return T / kBwdSub + N + 1; }

// Workspace bytes of the backward for T tokens in N sequences
inline size_t bwd_workspace_bytes(long long T, long long N, int H, int dk, int dv) {
  const long long n_ct = dv / 16;
  const size_t ckpt = size_t(bwd_ckpt_slots(T, N)) * H * dk * dv * 4;
  const size_t part = size_t(3) * n_ct * T * H * dk * 4;
  const size_t part_beta = size_t(4) * n_ct * T * H * 4;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(ckpt) + up(part) + up(part_beta);
}

hipError_t launch_chunk_bwd(const BwdParams& p, int io_dtype, int dk, hipStream_t stream);

}  // namespace kda
