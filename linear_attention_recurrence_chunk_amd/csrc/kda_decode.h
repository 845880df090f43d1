// Launch parameters of the fused decode-replay kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeParams {
  int R, H, D, conv_width, n_new, prev_slots, cur_slots, act;
  const int32_t* n_acc;     // [R]
  const int32_t* n_new_r;   // [R] new tokens per request (clamped to [1, n_new]) or null
  const __bf16* prev_q;     // [R, prev_slots, H, D] ...
  const __bf16* prev_k;
  const __bf16* prev_v;
  const __bf16* prev_g;
  const __bf16* prev_beta;  // [R, prev_slots, H]
  const __bf16* cur_q;      // [R, cur_slots, H, D] ...
  const __bf16* cur_k;
  const __bf16* cur_v;
  const __bf16* cur_g;
  const __bf16* cur_beta;
  const __bf16* cur_z;
  const float* conv_w;      // [H, 3D, W]
  const float* norm_w;      // [D]
  float* state;             // [R, H, D, D] in: committed, out: after the bonus token
  float* state_acc;         // [R, H, D, D] or null
  float* conv_tail;         // [R, H, 3D, W - 1]
  void* o;                  // [R, n_new, H, D] bf16 or fp32 (n_new: the most per request)
  int out_f32;
  int waves;                // waves per workgroup: 4 or 8
  float scale, decay_floor, eps_l2, eps_rms;
};

// Waves per decode workgroup (one workgroup per request and head): 4 while the workgroups
// fill the device (three per CU), 8 when at most half the compute units get one, so that a
// head's per-token work spreads over two waves per SIMD (same results either way).
inline int decode_waves(long long units, int cus) { return units * 2 <= cus ? 8 : 4; }

hipError_t launch_decode_replay(const DecodeParams& p, hipStream_t stream);

}  // namespace kda
