/*
 * libkda: the KDA gated delta-rule recurrence on AMD Instinct MI355X (gfx950).
 *
 * Each attention head of each sequence carries a fixed fp32 state S of d_k x d_v (rows are
 * key channels, columns value channels) that every token updates serially
 * ("Noyaux KDA et FlashKDA", section "Le conflit fondamental"). Per token t:
 *
 *     a_t  = exp(max(g_t, g_min))              per key channel; the floor is section
 *                                              "Le rôle de la décroissance bornée"
 *     S'   = diag(a_t) S                       decay first,
 *     S    = S' + beta_t k_t (v_t - S'^T k_t)^T  then the beta-weighted delta correction,
 *     o_t  = scale * S^T q_t                   then the read-out (sees token t).
 *
 * The update order is a reading: the pages never print the equation.
 *
 * Conventions shared by every entry point:
 *  - Pointers named without a _host suffix are DEVICE pointers (hipMalloc'ed or torch
 *    tensors); every call is asynchronous on `stream` (a hipStream_t, NULL = the default
 *    stream) and returns once the kernels are queued.
 *  - The library never allocates, frees or synchronises. Callers own every buffer.
 *  - Tensors are dense, row-major, with the shapes given below; all pointers must be 16-byte
 *    aligned.
 *  - States are stored head-contiguous, [.., H, d_k, d_v], so each head is one contiguous
 *    byte range ("Inférence : cache KV, décodage, quantification", section on prefill/decode
 *    disaggregation).
 *  - Every argument is validated on the host BEFORE anything is launched; on error nothing
 *    is launched, no output is touched and a negative kda_status is returned. Validation
 *    makes no HIP call. Device-side values (cu_seqlens on the device, n_acc) are trusted to
 *    match their host description; n_acc is clamped into range on the device.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 1

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL_ARG = -1,            /* a required pointer is NULL */
  KDA_ERR_BAD_SHAPE = -2,           /* a size is out of range or inconsistent */
  KDA_ERR_BAD_DTYPE = -3,           /* io_dtype is not a kda_dtype */
  KDA_ERR_MISALIGNED = -4,          /* a pointer is not 16-byte aligned */
  KDA_ERR_BAD_SEQLENS = -5,         /* cu_seqlens_host not 0-based, non-decreasing, ending at T */
  KDA_ERR_WORKSPACE_TOO_SMALL = -6, /* workspace_bytes below kda_segment_cp_workspace_size */
  KDA_ERR_UNSUPPORTED = -7,         /* valid but not implemented (d_k, d_v, dtype combination) */
  KDA_ERR_LAUNCH_FAILED = -8,       /* the HIP runtime rejected a launch */
  KDA_ERR_ALIASING = -9,            /* an output overlaps an input it must not overlap */
  KDA_ERR_BAD_VALUE = -10,          /* a scalar is out of range (g_min, eps, scale not finite) */
  KDA_ERR_SCRATCH_TOO_SMALL = -11   /* kda_chunk_fwd_noalloc: the longest sequence's operand
                                       slots exceed KDA_NOALLOC_SCRATCH_BYTES */
} kda_status;

typedef enum kda_dtype {
  KDA_F32 = 0,  /* IEEE binary32 */
  KDA_BF16 = 1  /* bfloat16 */
} kda_dtype;

/*
 * kda_chunk_fwd: chunked prefill of the recurrence over one or several packed sequences
 * ("Noyaux KDA et FlashKDA", section "FlashKDA : le noyau par blocs": parallel inside a
 * 64-token chunk, serial across chunks; AMD blog "Dentro de los esfuerzos de optimización de
 * Kimi K3", "Nota técnica: Precisión del KDA y memoria on-chip": per-chunk inverse of the
 * unit lower-triangular dependency matrix in fp32, rounded to bf16 only once complete).
 *
 *   q, k     [T_total, H, d_k]  io_dtype
 *   v        [T_total, H, d_v]  io_dtype
 *   g        [T_total, H, d_k]  fp32 log-decay per key channel (floored at g_min inside)
 *   beta     [T_total, H]       fp32
 *   h0       [N, H, d_k, d_v]   fp32 entering state per sequence, or NULL for zeros
 *   o        [T_total, H, d_v]  out_dtype output: KDA_F32, or io_dtype (written once; a bf16
 *                               output is the round-to-nearest-even of the fp32 result)
 *   ht       [N, H, d_k, d_v]   fp32 final state per sequence, or NULL to skip it
 *
 * Sequences: with cu_seqlens == cu_seqlens_host == NULL there are N = batch sequences of
 * seq_len tokens each, T_total = batch * seq_len (a [batch, seq_len, H, d] tensor).
 * Otherwise batch must be 1, both cu_seqlens (device) and cu_seqlens_host (host copy of the
 * same N + 1 int32 offsets) are given, N = n_seqs and T_total = seq_len = cu_seqlens_host[N].
 * Chunks restart at every sequence start; a sequence of length 0 copies h0 to ht.
 *
 * Supported: io_dtype KDA_BF16 with d_k = d_v in {64, 128}; KDA_F32 with d_k = d_v in
 * {64, 128} (fp32 output).
 * g_min must lie in [-5.4, 0] (the in-chunk exponent range stays finite in fp32);
 * g values above 0 are accepted but are not decays. o must not overlap any input; ht may
 * alias h0 (in-place state update).
 *
 * Numeric range (KDA_BF16): several of the chunk's matrix products take fp16 operands (max
 * 65504): the decayed queries and keys, the state, the tokens' weighted errors
 * beta (v - S'^T k) and the in-chunk attention scores. They stay in range in the method's
 * regime: q and k of unit L2 norm per token and head, beta in [0, 1], g <= 0. There every
 * token adds at most v_c^2 to the squared norm of state column c, so
 * |S| <= sqrt(|h0 column c|^2 + sum_t v_{t,c}^2) and each error is at most |v| + that bound;
 * keys or queries far from unit norm, or a sum above ~1e9, can give non-finite outputs.
 * Nothing checks this at run time (the library never synchronises). Both forms are tested
 * just inside the bound (sums of about 6e8, from scaled values and from a scaled entering
 * state; tests/test_gpu_range.py): outputs finite, within 1.5e-2 x RMS of the fp64 oracle.
 *
 * Workspace and launches. With workspace == NULL the call is one launch: each workgroup owns
 * one (sequence, head, 64-column state tile) and computes every chunk's token-parallel
 * prologue and then its serial step. With a workspace (KDA_BF16 only) the call is two
 * launches, the split of a token-parallel stage from the serial recurrence that the AMD blog
 * describes in section 5: (1) the prologue of every (chunk, head) runs in parallel over the
 * whole device and stores the serial step's operands (about 73 KiB per chunk and head at
 * d_k = 128) in the workspace; (2) the serial walk per (sequence, head, state tile) reads
 * them back. Both paths give bit-identical o and ht. A workspace of at least
 * kda_chunk_fwd_workspace_size(..., KDA_CHUNK_WS_TWO_PASS, ...) bytes takes the whole batch
 * in one prep and one walk; a smaller one (at least the KDA_CHUNK_WS_MIN size: the longest
 * sequence's slots) takes consecutive groups of whole sequences that fit, two launches per
 * group, with the same results. Each walk starts a group's longest sequences first (up to
 * 256 sequences per group; scheduling only, the results do not depend on it). The workspace
 * must be 16-byte aligned and overlap no other
 * argument; its contents on entry are ignored and on return are undefined. KDA_F32 at
 * d_k = 64 ignores the workspace (one launch). KDA_F32 at d_k = 128 always takes two launches
 * through a workspace, in the 16-token chunk form with every product in fp32 on the matrix
 * cores (the form kda_chunk_bwd uses): (1) per 16-token chunk and head, the decayed tiles
 * K e^G, K e^(G_C - G), Q e^G, the inverse T, the matrix M, e^(G_C) and beta (26.6 KiB at
 * d_k = 128); (2) the walk per (sequence, head, four 16-column state tiles), o = scale (Q e^G S0
 * + M U) per chunk. Without a workspace it returns KDA_ERR_WORKSPACE_TOO_SMALL; the same
 * grouping of whole sequences applies.
 *
 * State checkpoints (prefix-cache resume points; the prefill hands states on to later
 * requests, "Inférence : cache KV, décodage, quantification", prefill/decode disaggregation):
 * with ckpt_every > 0 (a multiple of 64) the state after every ckpt_every tokens of each
 * sequence is written to ckpt_states, fp32 [floor(T_total / ckpt_every), H, d_k, d_v]: the
 * state after the first (j + 1) * ckpt_every tokens of sequence n (n-th sequence starting at
 * token bos_n) goes to slot floor(bos_n / ckpt_every) + j. Slots of different sequences never
 * collide; slots no sequence reaches are left untouched. Passing a checkpoint as h0 for the
 * rest of its sequence reproduces the rest of the original call's o and ht bit for bit.
 * ckpt_every = 0 writes none (ckpt_states may be NULL).
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                  const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                  int num_heads, int d_k, int d_v, int io_dtype, int out_dtype, float scale,
                  float g_min, void* o, float* ht, int ckpt_every, float* ckpt_states,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Policies of kda_chunk_fwd_workspace_size. */
#define KDA_CHUNK_WS_AUTO 0     /* size of the path the library recommends (0: one launch) */
#define KDA_CHUNK_WS_TWO_PASS 1 /* the whole batch in one prep and one walk */
#define KDA_CHUNK_WS_MIN 2      /* the least the two-launch path accepts (longest sequence) */

/*
 * Bytes of workspace kda_chunk_fwd uses for the given sizes (same batch / seq_len / n_seqs /
 * cu_seqlens_host conventions as kda_chunk_fwd; cu_seqlens_host may be NULL, then packed
 * sequences are sized as if one of them held every token). Slots: a batch or group of
 * sequences with T tokens and N sequences needs (T / 64 + N + 1) x num_heads slots of
 * 74,752 B (d_k = 128) or 50,176 B (d_k = 64). KDA_F32 at d_k = 128: (T / 16 + N + 1) x
 * num_heads operand blocks of 27,200 B (the policies as for KDA_BF16, KDA_CHUNK_WS_AUTO
 * capping the size like a large batch's). 0 for KDA_F32 at d_k = 64 and unsupported widths.
 * KDA_CHUNK_WS_AUTO returns the whole-batch size while the one-launch workgroups
 * (sequences x heads x d_v / 64) do not exceed the current device's compute units (the
 * prologue then sits on every serial chain); beyond that, min(whole batch, max(8 GiB, longest
 * sequence)): groups of sequences, which measured faster than one launch on a 64-sequence
 * varlen batch as well.
 */
int kda_chunk_fwd_workspace_size(int batch, int seq_len, int n_seqs,
                                 const int32_t* cu_seqlens_host, int num_heads, int d_k,
                                 int d_v, int io_dtype, int policy, size_t* bytes);

/*
 * kda_chunk_fwd_noalloc: kda_chunk_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation. Arguments,
 * validation and results are those of kda_chunk_fwd without the workspace; the caller still
 * passes every input and output. With KDA_BF16 the call takes the two-launch path, its operand
 * slots in a static device array of KDA_NOALLOC_SCRATCH_BYTES (256 MiB) that the library holds
 * on every GPU it runs on until the process ends: the whole batch in one prep and one walk when
 * its slots fit, else consecutive groups of whole sequences, with the same bits as
 * kda_chunk_fwd. A sequence of T tokens needs floor(T / 64) + 2 slots of 74,752 B per head at
 * d_k = 128 (50,176 B at 64), so it may have up to (floor(KDA_NOALLOC_SCRATCH_BYTES /
 * (74,752 x num_heads)) - 1) x 64 - 1 tokens: 2,303 at 96 heads, 19,071 at 12; a longer one
 * returns KDA_ERR_SCRATCH_TOO_SMALL before anything runs. KDA_F32 at d_k = 64 runs the
 * one-launch path and uses no scratch; at d_k = 128 its operand blocks (27,200 B per 16 tokens
 * and head, floor(T / 16) + 2 per sequence) go in the same array (up to 1,615 tokens per
 * sequence at 96 heads, 13,135 at 12).
 *
 * The call allocates and frees nothing (no hipMalloc, hipFree or allocating library routine).
 * The first call on a device, with that device current, looks up the array's device address
 * (hipGetSymbolAddress) and keeps it; call with the stream's device current. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (concurrent streams, or
 * threads without ordering) race on it and must be serialised by the caller. Its contents are
 * overwritten by each call before they are read.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* h0, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                          int num_heads, int d_k, int d_v, int io_dtype, int out_dtype,
                          float scale, float g_min, void* o, float* ht, int ckpt_every,
                          float* ckpt_states, void* stream);

/*
 * kda_chunk_bwd: gradients of kda_chunk_fwd's outputs (training; "Noyaux KDA et FlashKDA",
 * section "FlashKDA : le noyau par blocs": the kernel serves training as well as prefill). The
 * pages give no backward; this is reverse-mode differentiation of the per-token update above.
 * Token by token, going back from D = dL/dS = dht at each sequence's end:
 *
 *   D += scale q_t do_t^T;  dq_t = scale S_t do_t;  de = beta_t D^T k_t;  dv_t = de;
 *   dk_t = beta_t D e_t - S'_t de;  dbeta_t = k_t^T D e_t;  D' = D - k_t de^T;
 *   dg_t = a_t * rowsum(S_{t-1} * D') where g_t > g_min, else 0 (the floor is flat);
 *   D = diag(a_t) D';  dh0 = D at the sequence start
 *
 * (e_t = v_t - S'_t^T k_t, S'_t = diag(a_t) S_{t-1}). The library evaluates the same gradients
 * in chunk form, 16 tokens at a time, in fp32 on the matrix cores: a parallel pass forms each
 * chunk's operands, a forward walk stores each chunk's entering state, a reverse walk each
 * chunk's leaving-state gradient (all in the workspace), and one workgroup per chunk then forms
 * dq, dk, dbeta and dg from them.
 *
 *   q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch, seq_len, n_seqs, num_heads,
 *   d_k, d_v, io_dtype, scale, g_min: as for kda_chunk_fwd (the forward's inputs)
 *   d_o      [T_total, H, d_v]   io_dtype   dL/do
 *   dht      [N, H, d_k, d_v]    fp32       dL/d(final state), or NULL for zeros
 *   dq, dk   [T_total, H, d_k]   fp32 outputs
 *   dv       [T_total, H, d_v]   fp32
 *   dg       [T_total, H, d_k]   fp32 (with respect to the raw g, before the floor)
 *   dbeta    [T_total, H]        fp32
 *   dh0      [N, H, d_k, d_v]    fp32, or NULL to skip it
 *   workspace  at least kda_chunk_bwd_workspace_size bytes, 16-byte aligned, overlapping no
 *              argument; its contents on entry are ignored, on return undefined.
 *
 * Supported: io_dtype KDA_BF16 or KDA_F32 with d_k = d_v in {64, 128}. Outputs must not overlap
 * any input or each other. Results are deterministic (every sum is taken in a fixed order, no
 * atomics). Four launches on the stream: the operand pass, the forward walk, the reverse walk,
 * the per-chunk gradients.
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                  const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                  int num_heads, int d_k, int d_v, int io_dtype, float scale, float g_min,
                  const void* d_o, const float* dht, float* dq, float* dk, float* dv, float* dg,
                  float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Workspace bytes of kda_chunk_bwd: (T_total / 16 + N + 1) chunk slots x H x (2 d_k d_v +
 * 64 d_v + 49 d_k + 528) x 4 (per 16-token chunk and head, fp32: the entering state and the
 * leaving state's gradient, four 16 x d_v row blocks, and the chunk's operand block: three
 * 16 x d_k decayed tiles, two 16 x 16 matrices, d_k decay factors and 16 betas). Same batch /
 * seq_len / n_seqs conventions as kda_chunk_fwd_workspace_size.
 */
int kda_chunk_bwd_workspace_size(int batch, int seq_len, int n_seqs, int num_heads, int d_k,
                                 int d_v, size_t* bytes);

/*
 * kda_chunk_fwd_raw: the prefill from raw projections, with the short convolution, the input
 * norms and the gate activations fused into the prep pass of the two-launch form (the same
 * token stage as kda_decode_replay: "Noyaux d'inférence", section "1. Le décodage KDA", fused
 * short convolution, input normalisation and gating; here on the prefill side, so the
 * convolved and normalised q, k and the activated gates never travel through HBM).
 *
 *   q_raw, k_raw, g_raw  [T_total, H, d_k] bf16 projections before the convolution / gate
 *   v_raw                [T_total, H, d_v] bf16
 *   beta_raw             [T_total, H] bf16
 *   conv_w               [H, 2 d_k + d_v, conv_width] fp32, channel order q, k, v; tap
 *                        conv_width - 1 multiplies the current token
 *   conv_tail_in         [N, H, 2 d_k + d_v, conv_width - 1] fp32 raw inputs before each
 *                        sequence, oldest first (a restored prefix), or NULL for zeros
 *   conv_tail_out        same shape, or NULL: each sequence's last conv_width - 1 raw inputs
 *                        (older ones from conv_tail_in when it is shorter); must not overlap
 *                        conv_tail_in
 * Per token, as in kda_decode_replay: depthwise causal convolution of q, k, v over the raw
 * inputs, SiLU when act == 1, q and k scaled by 1 / sqrt(sum x^2 + eps_l2),
 * beta = sigmoid(beta_raw), g = max(-softplus(g_raw), g_min); then the recurrence of
 * kda_chunk_fwd (h0, ht, o, scale, packed sequences as there). The convolved values are
 * stored once, in fp32, for the serial walk. Supported: d_k = d_v in {64, 128}, conv_width in
 * 1..4. `workspace` (16-byte aligned) holds the convolved values and the operand slots: with
 * kda_chunk_fwd_raw_workspace_size(...) bytes those of the whole batch; with less, down to
 * that size for the longest sequence alone, consecutive groups of whole sequences run one
 * after the other, each group a prep pass and a walk (sequences are independent, so the
 * result is the same bits). Below that, KDA_ERR_WORKSPACE_TOO_SMALL.
 */
int kda_chunk_fwd_raw(const void* q_raw, const void* k_raw, const void* v_raw,
                      const void* g_raw, const void* beta_raw, const float* conv_w,
                      const float* conv_tail_in, float* conv_tail_out, const float* h0,
                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int batch,
                      int seq_len, int n_seqs, int num_heads, int d_k, int d_v, int conv_width,
                      int act, float eps_l2, float scale, float g_min, void* o, float* ht,
                      int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace kda_chunk_fwd_raw needs (batch / seq_len / n_seqs as in kda_chunk_fwd). */
int kda_chunk_fwd_raw_workspace_size(int batch, int seq_len, int n_seqs, int num_heads, int d_k,
                                     int d_v, size_t* bytes);

/*
 * Bytes of device workspace kda_segment_cp_fwd needs for the given sizes (batch / seq_len /
 * n_seqs as in kda_chunk_fwd; n_segments = 0 asks for the automatic choice). For KDA_BF16
 * inputs with d_k = d_v in {64, 128} the size includes the operand slots of the two-launch
 * form (see kda_chunk_fwd); for KDA_F32 it is the segment summaries and entering states only.
 * Returns KDA_OK and writes *bytes, or a negative status.
 */
int kda_segment_cp_workspace_size(int batch, int seq_len, int n_seqs, int num_heads, int d_k,
                                  int d_v, int io_dtype, int n_segments, size_t* bytes);

/*
 * kda_segment_cp_fwd: segment-parallel prefill for few heads over long sequences
 * ("Noyaux KDA et FlashKDA", section "Le parallélisme de contexte intra-appareil"; AMD blog
 * section 5: group summaries, ordered scan, parallel replay).
 *
 * Same tensors, conventions and supported sizes as kda_chunk_fwd. Every sequence is cut into
 * up to n_segments contiguous, chunk-aligned segments (1..256). With n_segments = 0 the
 * library picks at most 64 from a cost model over the device's compute units and the longest
 * sequence; when that choice is one segment (the heads alone fill the device) the call is
 * the plain forward pass, exactly as kda_chunk_fwd (the workspace query still returns the
 * size for 64 segments). Otherwise the steps on `stream` are: (1) each segment's affine
 * summary (P, Q) with S_out = P S_in + Q, computed without its entering state; (2) an ordered
 * scan that composes the summaries into every segment's exact entering state and the final
 * state; (3) all segments replay their tokens in parallel from those states. The result
 * equals kda_chunk_fwd up to rounding.
 *
 * `workspace` is caller-owned device memory, 16-byte aligned, overlapping no other argument;
 * its contents on entry are ignored. With at least kda_segment_cp_workspace_size(...) bytes
 * and bf16 inputs, the steps use the two-launch form: one prep pass over every chunk and head
 * writes the chunks' operand slots, and (1) and (3) are walks over those slots. With less,
 * but at least the size the query returns for KDA_F32 inputs, (1) and (3) run the one-launch
 * kernel, which recomputes each chunk's prologue for every state tile.
 */
int kda_segment_cp_fwd(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* h0, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                       int num_heads, int d_k, int d_v, int io_dtype, int out_dtype,
                       float scale, float g_min, void* o, float* ht, int n_segments,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * One window of cached projected inputs for decode: raw (pre-convolution, pre-activation)
 * per-token projections, all bf16, each [R, slots, H, .]. z is the output-gate input and is
 * only read for the current window (it may be NULL in the previous one).
 */
typedef struct kda_token_window {
  const void* q;     /* [R, slots, H, d_k] */
  const void* k;     /* [R, slots, H, d_k] */
  const void* v;     /* [R, slots, H, d_v] */
  const void* g;     /* [R, slots, H, d_k] raw decay gate; g = max(-softplus(raw), g_min) */
  const void* beta;  /* [R, slots, H]      raw; beta = sigmoid(raw) */
  const void* z;     /* [R, slots, H, d_v] raw output gate; sigmoid(z) scales the output */
  int slots;
} kda_token_window;

/*
 * kda_decode_replay: fused speculative-verify decode ("Noyaux d'inférence", section
 * "1. Le décodage KDA": cache only projected inputs, replay accepted drafts on chip instead
 * of snapshotting S, one loop over replayed, bonus and draft tokens fused with short
 * convolution, input normalisation, gating and output normalisation; AMD blog section 3:
 * one launch that writes straight to the destination buffer; section 5: tiles own disjoint
 * value columns and walk the same tokens in order).
 *
 * Per request r and head h, starting from the committed state state[r, h] (the state after
 * the previous call's bonus token) and conv_tail[r, h]:
 *   1. replay slots 1 .. n_acc[r] of `prev` (the accepted drafts of the previous window;
 *      slot 0 was the previous bonus, already committed): no output;
 *   2. state_acc[r, h] <- S (skipped when state_acc is NULL);
 *   3. slot 0 of `cur` (the bonus token), output o[r, 0, h]; state[r, h] <- S and
 *      conv_tail[r, h] <- tail (the new committed values);
 *   4. slots 1 .. n_r - 1 of `cur` (the next draft window), outputs o[r, j, h]; their
 *      states are never written. n_r = n_new, or n_new_per_request[r] clamped to
 *      [1, n_new] when that array is given (irregular batches: requests whose draft windows
 *      differ in length; rows j >= n_r of o[r] are left untouched).
 * Each token: depthwise causal convolution of width conv_width over the raw q, k, v
 * channels with the tail of the last conv_width - 1 raw inputs; SiLU if act == 1;
 * q and k scaled by 1 / sqrt(sum x^2 + eps_l2); beta = sigmoid; g = max(-softplus, g_min);
 * the recurrence step above; o = scale * S^T q, then o * rsqrt(mean(o^2) + eps_rms) *
 * norm_w * sigmoid(z). The token step is one code path with a fixed operation order, so a
 * replayed state is bit-identical to the state the same tokens reach one launch at a time.
 *
 *   n_acc      [R] int32 device, clamped to [0, prev->slots - 1]
 *   n_new_per_request  [R] int32 device or NULL (all requests take n_new tokens)
 *   conv_w     [H, 2 d_k + d_v, conv_width] fp32, channel order q, k, v; tap conv_width - 1
 *              multiplies the current token
 *   norm_w     [d_v] fp32, shared by all heads
 *   state      [R, H, d_k, d_v] fp32, read then overwritten in place with S after the bonus
 *   state_acc  [R, H, d_k, d_v] fp32 or NULL; must not overlap state
 *   conv_tail  [R, H, 2 d_k + d_v, conv_width - 1] fp32, oldest first, updated in place
 *              (may be NULL when conv_width == 1)
 *   o          [R, n_new, H, d_v] out_dtype: KDA_BF16, or KDA_F32 (a bf16 output is the
 *              round-to-nearest-even of the fp32 result)
 *
 * Supported: d_k = d_v = 128 or 64, conv_width in 1..4, 1 <= n_new <= cur->slots,
 * prev->slots in 1..16, act in {0, 1}, eps_l2 > 0, eps_rms >= 0.
 */
int kda_decode_replay(int n_requests, int num_heads, int d_k, int d_v, int conv_width,
                      int n_new, const int32_t* n_acc, const int32_t* n_new_per_request,
                      const kda_token_window* prev,
                      const kda_token_window* cur, const float* conv_w, const float* norm_w,
                      float scale, float g_min, float eps_l2, float eps_rms, int act,
                      float* state, float* state_acc, float* conv_tail, void* o,
                      int out_dtype, void* stream);

/* Static description of a status code (never NULL). */
const char* kda_status_string(int status);

/* KDA_VERSION of the built library. */
int kda_version(void);

/* The hipError_t of the last failed launch in this thread (0 if none). */
int kda_last_launch_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
