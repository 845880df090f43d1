// Host-side plumbing shared between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// One launch of the chunk kernel. A "unit" is one (sequence, head) pair; every unit is
// processed by n_vt workgroups, one per 64-column value tile.
struct ChunkParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* h0;          // [N, H, dk, dv] or null (zeros)
  const int32_t* cu_seqlens;  // device [N + 1] or null (fixed length seq_len)
  void* o;                  // [T, H, dv] output dtype
  float* ht;                // [N, H, dk, dv] or null
  int seq_len;              // tokens per sequence when cu_seqlens is null
  int n_seqs;
  int H;
  int dv;                   // full value width (row stride of v / o / states)
  int n_vt;                 // value tiles per unit
  int n_units;              // n_seqs * H
  float scale;
  float g_min;
};

hipError_t launch_chunk_fwd(const ChunkParams& p, int io_dtype, int out_dtype, int dk,
                            hipStream_t stream);

}  // namespace kda
