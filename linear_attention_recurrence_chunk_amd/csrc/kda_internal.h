// Host-side plumbing shared between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_index.h"

namespace kda {

// What one launch of the chunk kernel computes.
enum ChunkMode : int {
  kModeForward = 0,     // outputs o and the final state of whole sequences
  kModeTransition = 1,  // per segment: (P, Q) with S_out = P S_in + Q, no outputs
  kModeReplay = 2,      // per segment: outputs o from the segment's entering state
  kModePrep = 3,        // two-pass prefill, pass 1: per chunk and head, the serial step's
                        // operands into ws_ops (no state, no values, no outputs)
  kModeWalk = 4,        // two-pass prefill, pass 2: the serial chunk walk from ws_ops
};


// One launch of the chunk kernel. A "unit" is one (sequence, segment, head) triple (one
// segment per sequence in forward mode); every unit is processed by n_vt workgroups, one per
// 64-column tile of its state (d_v columns, or d_k + d_v columns [P | Q] in transition mode).
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
  int n_units;              // n_seqs * n_seg * H
  int n_seg;                // segments per sequence (1 in forward mode)
  int mode;                 // ChunkMode
  float* ws_pq;             // transition: [N, n_seg, H, dk, dk + dv]
  float* ws_sin;            // replay: [N, n_seg, H, dk, dv] entering states
  char* ws_ops;             // prep / walk: operand slots [chunk slot][H] (see op_slot_count)
  int walk_tpw;             // walk: state tiles per workgroup, 1 or 2 (2 needs n_vt even)
  // forward / walk mode: states at every ckpt_every tokens of each sequence (a multiple of
  // 64; 0 for none). The state after token bos_n + (j + 1) ckpt_every - 1 of sequence n goes
  // to [floor(bos_n / ckpt_every) + j, H, dk, dv] of ckpt.
  float* ckpt;
  int ckpt_every;
  // a group of whole sequences (two-launch prefill with a workspace smaller than the whole
  // batch needs): unit sequence index n runs sequence seq0 + n, and operand slots count from
  // token slot_tok0 (the group's first token): chunk c of sequence m (first token bos_m) uses
  // slot ((bos_m - slot_tok0) / 64) + (m - seq0) + c. Both 0 otherwise.
  int seq0;
  int slot_tok0;
  // walk: the order in which its workgroups take the group's sequences, longest first, so that
  // the long ones do not start last (n_order > 0: unit sequence u runs sequence
  // seq0 + order[u]; groups of more than kMaxOrder sequences keep their own order)
  int n_order;
  uint16_t order[kMaxOrder];
  // prep mode with raw projections (q, k, v, g, beta before the short convolution, the L2
  // norms and the gate activations, all bf16): taps [H, 2 dk + dv, conv_width] (q, k, v
  // channels), entering convolution tails [N, H, 2 dk + dv, conv_width - 1] (null: zeros),
  // leaving tails (same shape), and the convolved values [T, H, dv] fp32 the walk reads
  const float* conv_w;
  const float* conv_tail_in;
  float* conv_tail_out;
  float* v_conv;
  int conv_width;
  int act;
  float eps_l2;
  float decay_floor;        // e^{g_min}
  float scale;
  float g_min;
};

// Ordered scan over segment summaries: S_in(0) = h0, S_in(j + 1) = P_j S_in(j) + Q_j.
struct ScanParams {
  const float* pq;          // [N, n_seg, H, dk, dk + dv]
  const float* h0;          // [N, H, dk, dv] or null
  float* sin;               // [N, n_seg, H, dk, dv]
  float* ht;                // [N, H, dk, dv] or null
  const int32_t* cu_seqlens;  // device [N + 1] or null (fixed length seq_len)
  int seq_len;
  int N, n_seg, H, dv;
  int f32;                  // 1: fp32 products (fp32 io), 0: split bf16 (bf16 io)
};

hipError_t launch_segment_scan(const ScanParams& p, int dk, hipStream_t stream);

hipError_t launch_chunk_fwd(const ChunkParams& p, int io_dtype, int out_dtype, int dk,
                            hipStream_t stream);

// Two-pass prefill (bf16 inputs). The prep pass runs over (sequence, group of chunks, head),
// prep_groups groups per sequence, and fills the operand slots in base.ws_ops from q, k, g,
// beta (no other field of base is read). A walk then runs over (sequence, segment, head,
// state tile) in mode kModeWalk (whole sequences: o and ht), kModeTransition (segment
// summaries [P | Q] into ws_pq) or kModeReplay (o from the entering states in ws_sin).
hipError_t launch_chunk_prep(const ChunkParams& base, int prep_groups, int dk,
                             hipStream_t stream, bool raw = false);
hipError_t launch_chunk_walk(const ChunkParams& p, int out_dtype, int dk, hipStream_t stream,
                             bool v_f32 = false);

}  // namespace kda
