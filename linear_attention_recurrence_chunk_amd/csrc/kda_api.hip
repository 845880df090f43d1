// C ABI of libkda: argument validation (host only, no HIP call) and kernel dispatch.
#include <algorithm>
#include <mutex>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/kda.h"
#include "kda_bwd.h"
#include "kda_decode.h"
#include "kda_internal.h"

// Operand slots of kda_chunk_fwd_noalloc, held by the library on every GPU it runs on for the
// life of the process. Host code never passes this name to a kernel or a copy: it is a host
// stand-in for the symbol, and the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

using kda::max_seq_len;
using kda::prep_groups;
using kda::raw_vconv_bytes;
using kda::two_pass_workspace_bytes;

thread_local int g_last_launch_error = 0;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* ptr, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(ptr);
  return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

size_t dsize(int io_dtype) { return io_dtype == KDA_BF16 ? 2 : 4; }

constexpr int kMaxSegments = 256;
constexpr int kAutoSegments = 64;

// [P | Q] summaries plus entering states, fp32, for every (sequence, segment, head)
size_t segment_workspace_bytes(int N, int H, int dk, int dv, int ns) {
  return size_t(N) * ns * H * dk * (size_t(dk) + 2 * size_t(dv)) * 4;
}

// Shared validation of the prefill entry points. Fills the sequence count and token total.
int validate_prefill(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* h0, const int32_t* cu_seqlens,
                     const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                     int num_heads, int d_k, int d_v, int io_dtype, int out_dtype,
                     float scale, float g_min, const void* o, const float* ht, int* out_N,
                     int64_t* out_T, size_t gate_bytes = 4, bool f32_wide = false) {
  if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_NULL_ARG;
  if (io_dtype != KDA_F32 && io_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (out_dtype != io_dtype && out_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
  if (num_heads <= 0 || d_k <= 0 || d_v <= 0 || batch < 0 || seq_len < 0)
    return KDA_ERR_BAD_SHAPE;
  if (!isfinite(scale) || !isfinite(g_min) || g_min < -5.4f || g_min > 0.f)
    return KDA_ERR_BAD_VALUE;

  int N;
  int64_t T;
  if (cu_seqlens || cu_seqlens_host) {
    if (!cu_seqlens || !cu_seqlens_host) return KDA_ERR_NULL_ARG;
    if (batch != 1 || n_seqs < 0) return KDA_ERR_BAD_SHAPE;
    if (!aligned16(cu_seqlens)) return KDA_ERR_MISALIGNED;
    if (cu_seqlens_host[0] != 0) return KDA_ERR_BAD_SEQLENS;
    for (int i = 0; i < n_seqs; ++i)
      if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return KDA_ERR_BAD_SEQLENS;
    if (cu_seqlens_host[n_seqs] != seq_len) return KDA_ERR_BAD_SEQLENS;
    N = n_seqs;
    T = seq_len;
  } else {
    if (n_seqs != batch) return KDA_ERR_BAD_SHAPE;
    N = batch;
    T = int64_t(batch) * seq_len;
  }
  if (T * num_heads * (int64_t)(d_k > d_v ? d_k : d_v) >= (int64_t(1) << 40))
    return KDA_ERR_BAD_SHAPE;

  const bool ok_bf16 = io_dtype == KDA_BF16 && d_k == d_v && (d_k == 64 || d_k == 128);
  // fp32 inputs: d = 64 everywhere; d = 128 for kda_chunk_fwd (the 16-token chunk form)
  const bool ok_f32 = io_dtype == KDA_F32 && d_k == d_v && (d_k == 64 || (f32_wide && d_k == 128));
  if (!ok_bf16 && !ok_f32) return KDA_ERR_UNSUPPORTED;

  const void* ptrs[] = {q, k, v, g, beta, o, h0, ht};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;

  const size_t es = dsize(io_dtype);
  const Range rq = range_of(q, size_t(T) * num_heads * d_k * es);
  const Range rk = range_of(k, size_t(T) * num_heads * d_k * es);
  const Range rv = range_of(v, size_t(T) * num_heads * d_v * es);
  const Range rg = range_of(g, size_t(T) * num_heads * d_k * gate_bytes);
  const Range rb = range_of(beta, size_t(T) * num_heads * gate_bytes);
  const Range rh0 = range_of(h0, h0 ? size_t(N) * num_heads * d_k * d_v * 4 : 0);
  const Range ro = range_of(o, size_t(T) * num_heads * d_v * dsize(out_dtype));
  const Range rht = range_of(ht, ht ? size_t(N) * num_heads * d_k * d_v * 4 : 0);
  for (Range in : {rq, rk, rv, rg, rb, rh0})
    if (overlaps(ro, in)) return KDA_ERR_ALIASING;
  for (Range in : {rq, rk, rv, rg, rb, ro})
    if (overlaps(rht, in)) return KDA_ERR_ALIASING;
  if (overlaps(rht, rh0) && rht.lo != rh0.lo) return KDA_ERR_ALIASING;  // only exact in-place
  *out_N = N;
  *out_T = T;
  return KDA_OK;
}

int launch_status(hipError_t err) {
  if (err != hipSuccess) {
    g_last_launch_error = static_cast<int>(err);
    return KDA_ERR_LAUNCH_FAILED;
  }
  return KDA_OK;
}

// Compute units of the current device (one query per process and device).
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Automatic segment count (at most kAutoSegments, the size the workspace query assumes): the
// one minimising a cost in units of one chunk step of the chunk kernel, with the passes
// running in rounds of one workgroup per compute unit. A transition step costs ~0.75 of a
// replay step (no output products) and a scan step ~0.9. One segment means the plain
// forward kernel (no transition, no scan).
int auto_segments(int N, int H, int dk, int dv, int64_t max_chunks, int cus) {
  auto rounds = [&](int64_t wgs) { return double((wgs + cus - 1) / cus); };
  double best = rounds(int64_t(N) * H * (dv / 64)) * double(max_chunks);
  int best_n = 1;
  const int hi = int(max_chunks < kAutoSegments ? max_chunks : kAutoSegments);
  for (int n = 2; n <= hi; ++n) {
    const double per_seg = double((max_chunks + n - 1) / n);
    const double cost = rounds(int64_t(N) * n * H * ((dk + dv) / 64)) * per_seg * 0.75 +
                        0.9 * n + rounds(int64_t(N) * n * H * (dv / 64)) * per_seg;
    if (cost < best) {
      best = cost;
      best_n = n;
    }
  }
  return best_n;
}

// workspace the automatic policy asks for when the batch runs in groups of sequences
constexpr size_t kGroupedWorkspace = size_t(8) << 30;


// The one-launch path leaves compute units idle when its (sequence, head, state tile)
// workgroups do not fill them; its per-chunk prologue then sits on every workgroup's serial
// chain, which the two-launch path takes off it.
bool two_pass_wanted(int64_t N, int H, int dv) {
  return N * H * (dv / 64) <= int64_t(compute_units());
}

// The walk takes a group's sequences longest first (ties in sequence order): with more
// workgroups than compute units, a long sequence dispatched last would finish alone.
void set_walk_order(kda::ChunkParams& gp, const int32_t* cu_seqlens_host, int n0, int n1) {
  gp.n_order = kda::walk_order(cu_seqlens_host, n0, n1, gp.order);
}

// Consecutive groups of whole sequences (kda::for_each_group) with the library's status codes
template <class Need, class Run>
int for_each_group(int N, const int32_t* cu_seqlens_host, int seq_len, size_t budget, Need need,
                   Run run) {
  return kda::for_each_group(N, cu_seqlens_host, seq_len, budget, need, run, KDA_OK);
}

// The launch parameters of one group: its sequences n0 .. n1 - 1, operand slots counted from
// its first token
kda::ChunkParams group_params(const kda::ChunkParams& p, int n0, int n1, int64_t tok0) {
  kda::ChunkParams gp = p;
  gp.seq0 = n0;
  gp.slot_tok0 = int(tok0);
  gp.n_seqs = n1 - n0;
  gp.n_units = (n1 - n0) * p.H;
  return gp;
}

// Automatic segment count of the two-launch segment path (at most kAutoSegments): the count
// minimising a cost in units of one walk chunk step with one state tile per workgroup
// (~3.7 us on MI355X). The prep pass is the same for every count. A walk runs in rounds of
// one workgroup per compute unit (its LDS holds two operand slots); a step of a two-tile
// workgroup costs 1.13 units, a transition step 0.85 of the corresponding output step, and
// the ordered scan 1.5 units per segment (fitted to measured launch times).
double walk_cost(int64_t units, int n_vt, int64_t chunks, bool transition, int cus) {
  const int tpw = (n_vt % 2 == 0 && units * n_vt > int64_t(cus)) ? 2 : 1;
  const int64_t wgs = units * n_vt / tpw;
  const double rounds = double((wgs + cus - 1) / cus);
  return rounds * double(chunks) * (tpw == 2 ? 1.13 : 1.0) * (transition ? 0.85 : 1.0);
}

int auto_segments_two_pass(int N, int H, int dk, int dv, int64_t max_chunks, int cus) {
  double best = walk_cost(int64_t(N) * H, dv / 64, max_chunks, false, cus);
  int best_n = 1;
  const int hi = int(max_chunks < kAutoSegments ? max_chunks : kAutoSegments);
  for (int n = 2; n <= hi; ++n) {
    const int64_t per_seg = (max_chunks + n - 1) / n;
    const int64_t units = int64_t(N) * n * H;
    const double cost = walk_cost(units, (dk + dv) / 64, per_seg, true, cus) + 1.5 * n +
                        walk_cost(units, dv / 64, per_seg, false, cus);
    if (cost < best) {
      best = cost;
      best_n = n;
    }
  }
  return best_n;
}

// State tiles per walk workgroup. One tile (four waves, one per SIMD) keeps the serial chain
// shortest and wins while the workgroups fit on the compute units in one round; beyond that
// two tiles per workgroup (eight waves, two per SIMD, sharing every slot load) finish the
// rounds sooner.
int walk_tiles_per_wg(int64_t units, int n_vt) {
  return (n_vt % 2 == 0 && units * n_vt > int64_t(compute_units())) ? 2 : 1;
}

// the two-launch form needs bf16 inputs and equal key and value widths of 64 or 128
bool two_pass_supported(int io_dtype, int dk, int dv) {
  return io_dtype == KDA_BF16 && dk == dv && (dk == 64 || dk == 128);
}

int check_workspace_aliasing(const void* ws, size_t need, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, const float* h0,
                             const void* o, const float* ht, int64_t T, int N, int H, int dk,
                             int dv, int io_dtype, int out_dtype) {
  const size_t es = dsize(io_dtype);
  const Range rws = range_of(ws, need);
  const Range all[] = {
      range_of(q, size_t(T) * H * dk * es), range_of(k, size_t(T) * H * dk * es),
      range_of(v, size_t(T) * H * dv * es), range_of(g, size_t(T) * H * dk * 4),
      range_of(beta, size_t(T) * H * 4), range_of(h0, h0 ? size_t(N) * H * dk * dv * 4 : 0),
      range_of(o, size_t(T) * H * dv * dsize(out_dtype)),
      range_of(ht, ht ? size_t(N) * H * dk * dv * 4 : 0)};
  for (Range x : all)
    if (overlaps(rws, x)) return KDA_ERR_ALIASING;
  return KDA_OK;
}

// The device address of this GPU's scratch (the current device's), looked up on the first
// call on each device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int device_scratch(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_launch_error = err != hipSuccess ? int(err) : int(hipErrorInvalidDevice);
    return KDA_ERR_LAUNCH_FAILED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr) {
      g_last_launch_error = err != hipSuccess ? int(err) : int(hipErrorInvalidSymbol);
      return KDA_ERR_LAUNCH_FAILED;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_version(void) { return KDA_VERSION; }

int kda_last_launch_error(void) { return g_last_launch_error; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_ARG: return "a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
    case KDA_ERR_BAD_DTYPE: return "unknown io dtype";
    case KDA_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case KDA_ERR_BAD_SEQLENS: return "cu_seqlens must start at 0, not decrease and end at T";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than required";
    case KDA_ERR_UNSUPPORTED: return "unsupported size / dtype combination";
    case KDA_ERR_LAUNCH_FAILED: return "kernel launch failed";
    case KDA_ERR_ALIASING: return "an output overlaps an input";
    case KDA_ERR_BAD_VALUE: return "a scalar argument is out of range";
    case KDA_ERR_SCRATCH_TOO_SMALL:
      return "a sequence's operand slots exceed the no-allocation entry point's static scratch";
    default: return "unknown status";
  }
}

int kda_chunk_fwd_workspace_size(int batch, int seq_len, int n_seqs,
                                 const int32_t* cu_seqlens_host, int num_heads, int d_k, int d_v,
                                 int io_dtype, int policy, size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_ARG;
  if (io_dtype != KDA_F32 && io_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (policy != KDA_CHUNK_WS_AUTO && policy != KDA_CHUNK_WS_TWO_PASS &&
      policy != KDA_CHUNK_WS_MIN)
    return KDA_ERR_BAD_VALUE;
  if (batch < 0 || seq_len < 0 || n_seqs < 0 || num_heads <= 0 || d_k <= 0 || d_v <= 0)
    return KDA_ERR_BAD_SHAPE;
  *bytes = 0;
  const bool c16 = io_dtype == KDA_F32 && d_k == 128 && d_v == 128;
  if (!c16 && (io_dtype != KDA_BF16 || d_k != d_v || (d_k != 64 && d_k != 128))) return KDA_OK;
  // packed sequences: batch 1, seq_len = T_total; otherwise n_seqs = batch
  const bool packed = cu_seqlens_host || (batch == 1 && n_seqs != 1);
  const int64_t T = packed ? int64_t(seq_len) : int64_t(batch) * seq_len;
  const int64_t N = packed ? n_seqs : batch;
  auto need = [&](int64_t tokens, int64_t seqs) {
    return c16 ? kda::c16_prefill_workspace_bytes(tokens, seqs, num_heads, d_k)
               : two_pass_workspace_bytes(tokens, seqs, num_heads, d_k);
  };
  const size_t full = need(T, N);
  // the largest single sequence (a group needs at least that); without the offsets of packed
  // sequences, the whole token count
  const int64_t longest = packed ? (cu_seqlens_host ? max_seq_len(cu_seqlens_host, int(N), 0) : T)
                                 : int64_t(seq_len);
  const size_t one = need(longest, 1);
  if (policy == KDA_CHUNK_WS_TWO_PASS) {
    *bytes = full;
  } else if (policy == KDA_CHUNK_WS_MIN) {
    *bytes = one < full ? one : full;
  } else if (!c16 && two_pass_wanted(N, num_heads, d_v)) {
    *bytes = full;
  } else {
    // enough (sequence, head, tile) units to fill the device: groups of sequences through a
    // workspace of at most kGroupedWorkspace bytes (at least the longest sequence's need)
    size_t cap = kGroupedWorkspace > one ? kGroupedWorkspace : one;
    *bytes = cap < full ? cap : full;
  }
  return KDA_OK;
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                  const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                  int num_heads, int d_k, int d_v, int io_dtype, int out_dtype, float scale,
                  float g_min, void* o, float* ht, int ckpt_every, float* ckpt_states,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int N = 0;
  int64_t T = 0;
  const int st = validate_prefill(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch,
                                  seq_len, n_seqs, num_heads, d_k, d_v, io_dtype, out_dtype, scale,
                                  g_min, o, ht, &N, &T, 4, true);
  if (st != KDA_OK) return st;
  if (ckpt_every < 0 || ckpt_every % 64 != 0) return KDA_ERR_BAD_SHAPE;
  if (ckpt_every > 0 && T / ckpt_every == 0) ckpt_every = 0;   // no sequence reaches a slot
  if (ckpt_every > 0) {
    if (!ckpt_states) return KDA_ERR_NULL_ARG;
    if (!aligned16(ckpt_states)) return KDA_ERR_MISALIGNED;
    const size_t es = dsize(io_dtype);
    const Range rc = range_of(ckpt_states, size_t(T / ckpt_every) * num_heads * d_k * d_v * 4);
    const Range all[] = {
        range_of(q, size_t(T) * num_heads * d_k * es), range_of(k, size_t(T) * num_heads * d_k * es),
        range_of(v, size_t(T) * num_heads * d_v * es), range_of(g, size_t(T) * num_heads * d_k * 4),
        range_of(beta, size_t(T) * num_heads * 4),
        range_of(h0, h0 ? size_t(N) * num_heads * d_k * d_v * 4 : 0),
        range_of(o, size_t(T) * num_heads * d_v * dsize(out_dtype)),
        range_of(ht, ht ? size_t(N) * num_heads * d_k * d_v * 4 : 0),
        range_of(workspace, workspace ? workspace_bytes : 0)};
    for (Range x : all)
      if (overlaps(rc, x)) return KDA_ERR_ALIASING;
  }
  // fp32 at d = 128: the 16-token chunk form, always through a workspace of operand blocks
  const bool c16 = io_dtype == KDA_F32 && d_k == 128;
  if (c16) {
    auto c16_need = [&](int64_t tokens, int64_t seqs) {
      return kda::c16_prefill_workspace_bytes(tokens, seqs, num_heads, d_k);
    };
    const size_t need = c16_need(T, N);
    const size_t need_min = c16_need(max_seq_len(cu_seqlens_host, N, seq_len), 1);
    if (!workspace || workspace_bytes < (need_min < need ? need_min : need))
      return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
    const int rc = check_workspace_aliasing(workspace, workspace_bytes < need ? workspace_bytes : need,
                                            q, k, v, g, beta, h0, o, ht, T, N, num_heads, d_k, d_v,
                                            io_dtype, out_dtype);
    if (rc != KDA_OK) return rc;
    if (N == 0) return KDA_OK;
    kda::CBwdParams cp{};
    cp.q = q;
    cp.k = k;
    cp.v = v;
    cp.g = g;
    cp.beta = beta;
    cp.h0 = h0;
    cp.cu_seqlens = cu_seqlens;
    cp.seq_len = cu_seqlens ? 0 : seq_len;
    cp.H = num_heads;
    cp.n_ct = d_v / 16;
    cp.scale = scale;
    cp.g_min = g_min;
    cp.o = static_cast<float*>(o);
    cp.ht = ht;
    cp.ckpt = ckpt_every > 0 ? ckpt_states : nullptr;
    cp.ckpt_every = ckpt_every > 0 ? ckpt_every : 64;
    cp.ops = static_cast<float*>(workspace);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // consecutive groups of whole sequences whose operand blocks fit the workspace
    return for_each_group(N, cu_seqlens_host, seq_len, workspace_bytes, c16_need,
                          [&](int n0, int n1, int64_t tok0, int64_t tokens) {
                            kda::CBwdParams gp = cp;
                            gp.seq0 = n0;
                            gp.slot_tok0 = int(tok0);
                            gp.n_seqs = n1 - n0;
                            gp.n_units = (n1 - n0) * num_heads;
                            gp.T = tokens;
                            gp.n_slots = kda::cbwd_slots(tokens, n1 - n0);
                            return launch_status(kda::launch_c16_prefill(gp, d_k, s));
                          });
  }
  const bool two_pass = workspace != nullptr && io_dtype == KDA_BF16;
  size_t need = 0;
  if (two_pass) {
    // the whole batch at once, or groups of whole sequences; a group needs at least the
    // longest sequence's slots
    need = two_pass_workspace_bytes(T, N, num_heads, d_k);
    const size_t need_min =
        two_pass_workspace_bytes(max_seq_len(cu_seqlens_host, N, seq_len), 1, num_heads, d_k);
    if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
    if (workspace_bytes < (need_min < need ? need_min : need)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    const int rc = check_workspace_aliasing(workspace, workspace_bytes < need ? workspace_bytes : need,
                                            q, k, v, g, beta, h0, o, ht, T, N, num_heads, d_k, d_v,
                                            io_dtype, out_dtype);
    if (rc != KDA_OK) return rc;
  }
  if (N == 0) return KDA_OK;
  kda::ChunkParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.cu_seqlens = cu_seqlens;
  p.o = o;
  p.ht = ht;
  p.seq_len = cu_seqlens ? 0 : seq_len;
  p.n_seqs = N;
  p.H = num_heads;
  p.dv = d_v;
  p.n_vt = d_v / 64;
  p.n_seg = 1;
  p.mode = kda::kModeForward;
  p.n_units = N * num_heads;
  p.scale = scale;
  p.g_min = g_min;
  p.ckpt = ckpt_every > 0 ? ckpt_states : nullptr;
  p.ckpt_every = ckpt_every > 0 ? ckpt_every : 64;
  if (two_pass) {
    p.mode = kda::kModeWalk;
    p.ws_ops = static_cast<char*>(workspace);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // consecutive groups of whole sequences whose slots fit the workspace (one group when it
    // holds the whole batch)
    return for_each_group(
        N, cu_seqlens_host, seq_len, workspace_bytes,
        [&](int64_t tokens, int64_t seqs) {
          return two_pass_workspace_bytes(tokens, seqs, num_heads, d_k);
        },
        [&](int n0, int n1, int64_t tok0, int64_t) {
          kda::ChunkParams gp = group_params(p, n0, n1, tok0);
          const int32_t* cu_g = cu_seqlens_host ? cu_seqlens_host + n0 : nullptr;
          int rc = launch_status(
              kda::launch_chunk_prep(gp, prep_groups(cu_g, n1 - n0, seq_len), d_k, s));
          if (rc != KDA_OK) return rc;
          gp.walk_tpw = walk_tiles_per_wg(gp.n_units, gp.n_vt);
          set_walk_order(gp, cu_seqlens_host, n0, n1);
          return launch_status(kda::launch_chunk_walk(gp, out_dtype, d_k, s));
        });
  }
  return launch_status(
      kda::launch_chunk_fwd(p, io_dtype, out_dtype, d_k, static_cast<hipStream_t>(stream)));
}

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* h0, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                          int num_heads, int d_k, int d_v, int io_dtype, int out_dtype,
                          float scale, float g_min, void* o, float* ht, int ckpt_every,
                          float* ckpt_states, void* stream) {
  // kda_chunk_fwd's own validation, with no workspace (host only, launches nothing)
  int N = 0;
  int64_t T = 0;
  const int st = validate_prefill(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch,
                                  seq_len, n_seqs, num_heads, d_k, d_v, io_dtype, out_dtype, scale,
                                  g_min, o, ht, &N, &T, 4, true);
  if (st != KDA_OK) return st;
  const bool c16 = io_dtype == KDA_F32 && d_k == 128;
  if (io_dtype != KDA_BF16 && !c16)   // one launch, no scratch
    return kda_chunk_fwd(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch, seq_len,
                         n_seqs, num_heads, d_k, d_v, io_dtype, out_dtype, scale, g_min, o, ht,
                         ckpt_every, ckpt_states, nullptr, 0, stream);
  // a group holds at least one whole sequence: the longest one's slots must fit
  const int64_t longest = max_seq_len(cu_seqlens_host, N, seq_len);
  const size_t one = c16 ? kda::c16_prefill_workspace_bytes(longest, 1, num_heads, d_k)
                         : two_pass_workspace_bytes(longest, 1, num_heads, d_k);
  if (one > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH_TOO_SMALL;
  if (N == 0) return KDA_OK;
  void* ws = nullptr;
  const int rc = device_scratch(&ws);
  if (rc != KDA_OK) return rc;
  return kda_chunk_fwd(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch, seq_len, n_seqs,
                       num_heads, d_k, d_v, io_dtype, out_dtype, scale, g_min, o, ht, ckpt_every,
                       ckpt_states, ws, KDA_NOALLOC_SCRATCH_BYTES, stream);
}

int kda_chunk_bwd_workspace_size(int batch, int seq_len, int n_seqs, int num_heads, int d_k,
                                 int d_v, size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_ARG;
  if (batch < 0 || seq_len < 0 || n_seqs < 0 || num_heads <= 0 || d_k <= 0 || d_v <= 0)
    return KDA_ERR_BAD_SHAPE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
  const bool packed = batch == 1 && n_seqs != 1;
  const int64_t T = packed ? int64_t(seq_len) : int64_t(batch) * seq_len;
  const int64_t N = packed ? n_seqs : batch;
  *bytes = kda::cbwd_workspace_bytes(T, N, num_heads, d_k, d_v);
  return KDA_OK;
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                  const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                  int num_heads, int d_k, int d_v, int io_dtype, float scale, float g_min,
                  const void* d_o, const float* dht, float* dq, float* dk, float* dv, float* dg,
                  float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!d_o || !dq || !dk || !dv || !dg || !dbeta || !workspace) return KDA_ERR_NULL_ARG;
  if (io_dtype != KDA_F32 && io_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
  // the forward's checks (shapes, sequences, values), with d_o standing in for its output;
  // fp32 inputs are validated as bf16 ones of the same widths (the backward takes both)
  int N = 0;
  int64_t T = 0;
  const int st = validate_prefill(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch,
                                  seq_len, n_seqs, num_heads, d_k, d_v, KDA_BF16, KDA_BF16, scale,
                                  g_min, d_o, nullptr, &N, &T, 4);
  if (st != KDA_OK) return st;
  const size_t es = dsize(io_dtype);
  const void* ptrs[] = {d_o, dht, dq, dk, dv, dg, dbeta, dh0, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
  const size_t need = kda::cbwd_workspace_bytes(T, N, num_heads, d_k, d_v);
  if (workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
  {
    const size_t st_bytes = size_t(N) * num_heads * d_k * d_v * 4;
    const Range in[] = {
        range_of(q, size_t(T) * num_heads * d_k * es), range_of(k, size_t(T) * num_heads * d_k * es),
        range_of(v, size_t(T) * num_heads * d_v * es), range_of(g, size_t(T) * num_heads * d_k * 4),
        range_of(beta, size_t(T) * num_heads * 4), range_of(h0, h0 ? st_bytes : 0),
        range_of(d_o, size_t(T) * num_heads * d_v * es), range_of(dht, dht ? st_bytes : 0)};
    const Range out[] = {
        range_of(dq, size_t(T) * num_heads * d_k * 4), range_of(dk, size_t(T) * num_heads * d_k * 4),
        range_of(dv, size_t(T) * num_heads * d_v * 4), range_of(dg, size_t(T) * num_heads * d_k * 4),
        range_of(dbeta, size_t(T) * num_heads * 4), range_of(dh0, dh0 ? st_bytes : 0),
        range_of(workspace, need)};
    const int n_out = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < n_out; ++i) {
      for (Range x : in)
        if (overlaps(out[i], x)) return KDA_ERR_ALIASING;
      for (int j = i + 1; j < n_out; ++j)
        if (overlaps(out[i], out[j])) return KDA_ERR_ALIASING;
    }
  }
  if (N == 0) return KDA_OK;
  kda::CBwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.d_o = d_o;
  p.dht = dht;
  p.cu_seqlens = cu_seqlens;
  p.seq_len = cu_seqlens ? 0 : seq_len;
  p.n_seqs = N;
  p.H = num_heads;
  p.n_ct = d_v / 16;
  p.n_units = N * num_heads;
  p.T = T;
  p.n_slots = kda::cbwd_slots(T, N);
  p.scale = scale;
  p.g_min = g_min;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dg = dg;
  p.dbeta = dbeta;
  p.dh0 = dh0;
  kda::cbwd_bind_workspace(p, workspace, d_k, d_v);
  return launch_status(
      kda::launch_chunk_bwd_mfma(p, io_dtype, d_k, static_cast<hipStream_t>(stream)));
}

int kda_chunk_fwd_raw_workspace_size(int batch, int seq_len, int n_seqs, int num_heads, int d_k,
                                     int d_v, size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_ARG;
  if (batch < 0 || seq_len < 0 || n_seqs < 0 || num_heads <= 0 || d_k <= 0 || d_v <= 0)
    return KDA_ERR_BAD_SHAPE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
  const bool packed = batch == 1 && n_seqs != 1;
  const int64_t T = packed ? int64_t(seq_len) : int64_t(batch) * seq_len;
  const int64_t N = packed ? n_seqs : batch;
  *bytes = raw_vconv_bytes(T, num_heads, d_v) + two_pass_workspace_bytes(T, N, num_heads, d_k);
  return KDA_OK;
}

int kda_chunk_fwd_raw(const void* q_raw, const void* k_raw, const void* v_raw,
                      const void* g_raw, const void* beta_raw, const float* conv_w,
                      const float* conv_tail_in, float* conv_tail_out, const float* h0,
                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int batch,
                      int seq_len, int n_seqs, int num_heads, int d_k, int d_v, int conv_width,
                      int act, float eps_l2, float scale, float g_min, void* o, float* ht,
                      int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!conv_w || !workspace) return KDA_ERR_NULL_ARG;
  if (conv_width < 1 || conv_width > 4) return KDA_ERR_BAD_SHAPE;
  if (act != 0 && act != 1) return KDA_ERR_BAD_VALUE;
  if (!(eps_l2 > 0.f) || !isfinite(eps_l2)) return KDA_ERR_BAD_VALUE;
  if (d_k != d_v) return KDA_ERR_UNSUPPORTED;
  // the same shape, sequence and aliasing checks as kda_chunk_fwd with bf16 inputs (g and
  // beta bf16 too)
  int N = 0;
  int64_t T = 0;
  const int st = validate_prefill(q_raw, k_raw, v_raw, static_cast<const float*>(g_raw),
                                  static_cast<const float*>(beta_raw), h0, cu_seqlens,
                                  cu_seqlens_host, batch, seq_len, n_seqs, num_heads, d_k, d_v,
                                  KDA_BF16, out_dtype, scale, g_min, o, ht, &N, &T, 2);
  if (st != KDA_OK) return st;
  const void* ptrs[] = {conv_w, conv_tail_in, conv_tail_out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
  if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
  // the whole batch at once, or groups of whole sequences: a group needs the convolved values
  // and operand slots of its own tokens, at least those of the longest sequence
  auto raw_bytes = [&](int64_t tokens, int64_t seqs) {
    return raw_vconv_bytes(tokens, num_heads, d_v) +
           two_pass_workspace_bytes(tokens, seqs, num_heads, d_k);
  };
  const size_t need_all = raw_bytes(T, N);
  const size_t need_min = raw_bytes(max_seq_len(cu_seqlens_host, N, seq_len), 1);
  if (workspace_bytes < (need_min < need_all ? need_min : need_all))
    return KDA_ERR_WORKSPACE_TOO_SMALL;
  const size_t need = workspace_bytes < need_all ? workspace_bytes : need_all;
  const size_t C3 = size_t(2 * d_k + d_v);
  const size_t tail_bytes = size_t(N) * num_heads * C3 * size_t(conv_width - 1) * 4;
  {
    const Range rws = range_of(workspace, need);
    const Range rout = range_of(conv_tail_out, conv_tail_out ? tail_bytes : 0);
    const Range rin = range_of(conv_tail_in, conv_tail_in ? tail_bytes : 0);
    const Range all[] = {
        range_of(q_raw, size_t(T) * num_heads * d_k * 2), range_of(k_raw, size_t(T) * num_heads * d_k * 2),
        range_of(v_raw, size_t(T) * num_heads * d_v * 2), range_of(g_raw, size_t(T) * num_heads * d_k * 2),
        range_of(beta_raw, size_t(T) * num_heads * 2),
        range_of(h0, h0 ? size_t(N) * num_heads * d_k * d_v * 4 : 0),
        range_of(o, size_t(T) * num_heads * d_v * dsize(out_dtype)),
        range_of(ht, ht ? size_t(N) * num_heads * d_k * d_v * 4 : 0),
        range_of(conv_w, size_t(num_heads) * C3 * conv_width * 4)};
    for (Range x : all) {
      if (overlaps(rws, x)) return KDA_ERR_ALIASING;
      if (overlaps(rout, x)) return KDA_ERR_ALIASING;
    }
    // the leaving tail is written while other workgroups still read the entering one
    if (overlaps(rout, rin) || overlaps(rout, rws) || overlaps(rin, rws)) return KDA_ERR_ALIASING;
  }
  if (N == 0) return KDA_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  kda::ChunkParams p{};
  p.q = q_raw;
  p.k = k_raw;
  p.v = v_raw;
  p.g = static_cast<const float*>(g_raw);         // bf16 data; the raw prep reads it as such
  p.beta = static_cast<const float*>(beta_raw);
  p.h0 = h0;
  p.cu_seqlens = cu_seqlens;
  p.o = o;
  p.ht = ht;
  p.seq_len = cu_seqlens ? 0 : seq_len;
  p.n_seqs = N;
  p.H = num_heads;
  p.dv = d_v;
  p.n_vt = d_v / 64;
  p.n_seg = 1;
  p.n_units = N * num_heads;
  p.scale = scale;
  p.g_min = g_min;
  p.ckpt_every = 64;
  p.conv_w = conv_w;
  p.conv_tail_in = conv_tail_in;
  p.conv_tail_out = conv_tail_out;
  p.conv_width = conv_width;
  p.act = act;
  p.eps_l2 = eps_l2;
  p.decay_floor = expf(g_min);
  p.mode = kda::kModeWalk;
  return for_each_group(
      N, cu_seqlens_host, seq_len, workspace_bytes, raw_bytes,
      [&](int n0, int n1, int64_t tok0, int64_t tokens) {
        kda::ChunkParams gp = group_params(p, n0, n1, tok0);
        // the kernels index the convolved values by global token: the group's region is
        // handed over as a base shifted back by its first token (64-bit address arithmetic,
        // so every address they form lies inside the region)
        const uintptr_t vbase = reinterpret_cast<uintptr_t>(workspace) -
                                uintptr_t(tok0) * uintptr_t(num_heads) * uintptr_t(d_v) * 4u;
        gp.v_conv = reinterpret_cast<float*>(vbase);
        gp.ws_ops = static_cast<char*>(workspace) + raw_vconv_bytes(tokens, num_heads, d_v);
        const int32_t* cu_g = cu_seqlens_host ? cu_seqlens_host + n0 : nullptr;
        int rc = launch_status(
            kda::launch_chunk_prep(gp, prep_groups(cu_g, n1 - n0, seq_len), d_k, s, true));
        if (rc != KDA_OK) return rc;
        // the walk reads the convolved values
        gp.v = gp.v_conv;
        gp.walk_tpw = 1;   // (the fp32-value walk has no register room for two waves per SIMD)
        set_walk_order(gp, cu_seqlens_host, n0, n1);
        return launch_status(kda::launch_chunk_walk(gp, out_dtype, d_k, s, true));
      });
}

int kda_segment_cp_workspace_size(int batch, int seq_len, int n_seqs, int num_heads, int d_k,
                                  int d_v, int io_dtype, int n_segments, size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_ARG;
  if (io_dtype != KDA_F32 && io_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (batch < 0 || seq_len < 0 || n_seqs < 0 || num_heads <= 0 || d_k <= 0 || d_v <= 0)
    return KDA_ERR_BAD_SHAPE;
  if (n_segments < 0 || n_segments > kMaxSegments) return KDA_ERR_BAD_SHAPE;
  const int ns = n_segments == 0 ? kAutoSegments : n_segments;
  const int64_t T = batch == 1 && n_seqs != 1 ? int64_t(seq_len) : int64_t(batch) * seq_len;
  const int64_t N = batch == 1 && n_seqs != 1 ? n_seqs : batch;
  *bytes = segment_workspace_bytes(int(N), num_heads, d_k, d_v, ns);
  if (two_pass_supported(io_dtype, d_k, d_v)) *bytes += two_pass_workspace_bytes(T, N, num_heads, d_k);
  return KDA_OK;
}

int kda_segment_cp_fwd(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* h0, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                       int num_heads, int d_k, int d_v, int io_dtype, int out_dtype,
                       float scale, float g_min, void* o, float* ht, int n_segments,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int N = 0;
  int64_t T = 0;
  const int st = validate_prefill(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch,
                                  seq_len, n_seqs, num_heads, d_k, d_v, io_dtype, out_dtype, scale,
                                  g_min, o, ht, &N, &T);
  if (st != KDA_OK) return st;
  if (n_segments < 0 || n_segments > kMaxSegments) return KDA_ERR_BAD_SHAPE;
  int ns = n_segments == 0 ? kAutoSegments : n_segments;
  const size_t need = segment_workspace_bytes(N, num_heads, d_k, d_v, ns);
  const size_t need_ops = two_pass_supported(io_dtype, d_k, d_v)
                              ? two_pass_workspace_bytes(T, N, num_heads, d_k) : 0;
  if (!workspace) return KDA_ERR_NULL_ARG;
  if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
  if (workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
  // a workspace that also holds the operand slots runs the two-launch form
  const bool two_pass = need_ops > 0 && workspace_bytes >= need + need_ops;
  {
    const int rc = check_workspace_aliasing(workspace, two_pass ? need + need_ops : need, q, k, v,
                                            g, beta, h0, o, ht, T, N, num_heads, d_k, d_v,
                                            io_dtype, out_dtype);
    if (rc != KDA_OK) return rc;
  }
  if (N == 0) return KDA_OK;
  const int64_t max_chunks = (max_seq_len(cu_seqlens_host, N, seq_len) + 63) / 64;
  if (n_segments == 0)
    ns = two_pass ? auto_segments_two_pass(N, num_heads, d_k, d_v, max_chunks, compute_units())
                  : auto_segments(N, num_heads, d_k, d_v, max_chunks, compute_units());
  float* ws_pq = static_cast<float*>(workspace);
  float* ws_sin = ws_pq + size_t(N) * ns * num_heads * d_k * (d_k + d_v);
  char* ws_ops = static_cast<char*>(workspace) + need;
  const hipStream_t s = static_cast<hipStream_t>(stream);

  kda::ChunkParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.cu_seqlens = cu_seqlens;
  p.o = o;
  p.ht = nullptr;
  p.seq_len = cu_seqlens ? 0 : seq_len;
  p.n_seqs = N;
  p.H = num_heads;
  p.dv = d_v;
  p.scale = scale;
  p.g_min = g_min;
  p.ws_ops = two_pass ? ws_ops : nullptr;
  if (two_pass) {
    // one prep pass serves every walk below
    const int rc = launch_status(
        kda::launch_chunk_prep(p, prep_groups(cu_seqlens_host, N, seq_len), d_k, s));
    if (rc != KDA_OK) return rc;
  }
  if (ns == 1 && n_segments == 0) {
    // one segment: the entering state is h0, so the forward pass is the whole job
    p.ht = ht;
    p.n_vt = d_v / 64;
    p.n_seg = 1;
    p.n_units = N * num_heads;
    if (two_pass) {
      p.mode = kda::kModeWalk;
      p.walk_tpw = walk_tiles_per_wg(p.n_units, p.n_vt);
      return launch_status(kda::launch_chunk_walk(p, out_dtype, d_k, s));
    }
    p.mode = kda::kModeForward;
    return launch_status(kda::launch_chunk_fwd(p, io_dtype, out_dtype, d_k, s));
  }
  p.n_seg = ns;
  p.n_units = N * ns * num_heads;
  p.ws_pq = ws_pq;
  p.ws_sin = ws_sin;
  // (1) segment summaries [P | Q] over the widened state, without entering states
  p.mode = kda::kModeTransition;
  p.n_vt = (d_k + d_v) / 64;
  p.walk_tpw = walk_tiles_per_wg(p.n_units, p.n_vt);
  int rc = launch_status(two_pass ? kda::launch_chunk_walk(p, out_dtype, d_k, s)
                                  : kda::launch_chunk_fwd(p, io_dtype, out_dtype, d_k, s));
  if (rc != KDA_OK) return rc;
  // (2) ordered scan: every segment's entering state and the final state
  kda::ScanParams sp{};
  sp.pq = ws_pq;
  sp.h0 = h0;
  sp.sin = ws_sin;
  sp.ht = ht;
  sp.cu_seqlens = cu_seqlens;
  sp.seq_len = cu_seqlens ? 0 : seq_len;
  sp.N = N;
  sp.n_seg = ns;
  sp.H = num_heads;
  sp.dv = d_v;
  sp.f32 = io_dtype == KDA_F32;
  rc = launch_status(kda::launch_segment_scan(sp, d_k, s));
  if (rc != KDA_OK) return rc;
  // (3) all segments replay their tokens in parallel
  p.mode = kda::kModeReplay;
  p.n_vt = d_v / 64;
  p.walk_tpw = walk_tiles_per_wg(p.n_units, p.n_vt);
  return launch_status(two_pass ? kda::launch_chunk_walk(p, out_dtype, d_k, s)
                                : kda::launch_chunk_fwd(p, io_dtype, out_dtype, d_k, s));
}

int kda_decode_replay(int n_requests, int num_heads, int d_k, int d_v, int conv_width,
                      int n_new, const int32_t* n_acc, const int32_t* n_new_per_request,
                      const kda_token_window* prev,
                      const kda_token_window* cur, const float* conv_w, const float* norm_w,
                      float scale, float g_min, float eps_l2, float eps_rms, int act,
                      float* state, float* state_acc, float* conv_tail, void* o,
                      int out_dtype, void* stream) {
  if (!prev || !cur) return KDA_ERR_NULL_ARG;
  if (!n_acc || !conv_w || !norm_w || !state || !o) return KDA_ERR_NULL_ARG;
  if (!conv_tail && conv_width != 1) return KDA_ERR_NULL_ARG;
  if (out_dtype != KDA_BF16 && out_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
  if (!prev->q || !prev->k || !prev->v || !prev->g || !prev->beta) return KDA_ERR_NULL_ARG;
  if (!cur->q || !cur->k || !cur->v || !cur->g || !cur->beta || !cur->z) return KDA_ERR_NULL_ARG;
  if (n_requests < 0 || num_heads <= 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_BAD_SHAPE;
  if (conv_width < 1 || conv_width > 4) return KDA_ERR_BAD_SHAPE;
  if (prev->slots < 1 || prev->slots > 16 || cur->slots < 1 || cur->slots > 16)
    return KDA_ERR_BAD_SHAPE;
  if (n_new < 1 || n_new > cur->slots) return KDA_ERR_BAD_SHAPE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
  if (act != 0 && act != 1) return KDA_ERR_BAD_VALUE;
  if (!isfinite(scale) || !isfinite(g_min) || g_min > 0.f || !(eps_l2 > 0.f) ||
      !(eps_rms >= 0.f) || !isfinite(eps_l2) || !isfinite(eps_rms))
    return KDA_ERR_BAD_VALUE;
  const void* ptrs[] = {n_acc, n_new_per_request, prev->q, prev->k, prev->v, prev->g,
                        prev->beta, cur->q,
                        cur->k,   cur->v,  cur->g,  cur->beta, cur->z, conv_w,   norm_w,
                        state,    state_acc, conv_tail, o};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
  const size_t R = size_t(n_requests), H = size_t(num_heads), D = size_t(d_k);
  const size_t C3 = 3 * D;
  const Range rstate = range_of(state, R * H * D * D * 4);
  const Range racc = range_of(state_acc, state_acc ? R * H * D * D * 4 : 0);
  const Range rtail = range_of(conv_tail, R * H * C3 * size_t(conv_width - 1) * 4);
  const Range ro = range_of(o, R * size_t(n_new) * H * D * dsize(out_dtype));
  const Range ins[] = {
      range_of(n_acc, R * 4), range_of(n_new_per_request, n_new_per_request ? R * 4 : 0),
      range_of(prev->q, R * prev->slots * H * D * 2), range_of(prev->k, R * prev->slots * H * D * 2),
      range_of(prev->v, R * prev->slots * H * D * 2), range_of(prev->g, R * prev->slots * H * D * 2),
      range_of(prev->beta, R * prev->slots * H * 2),
      range_of(cur->q, R * cur->slots * H * D * 2), range_of(cur->k, R * cur->slots * H * D * 2),
      range_of(cur->v, R * cur->slots * H * D * 2), range_of(cur->g, R * cur->slots * H * D * 2),
      range_of(cur->beta, R * cur->slots * H * 2), range_of(cur->z, R * cur->slots * H * D * 2),
      range_of(conv_w, H * C3 * size_t(conv_width) * 4), range_of(norm_w, D * 4)};
  for (Range out : {rstate, racc, rtail, ro})
    for (Range in : ins)
      if (overlaps(out, in)) return KDA_ERR_ALIASING;
  if (overlaps(rstate, racc) || overlaps(rstate, ro) || overlaps(rstate, rtail) ||
      overlaps(racc, ro) || overlaps(racc, rtail) || overlaps(ro, rtail))
    return KDA_ERR_ALIASING;
  if (n_requests == 0) return KDA_OK;

  kda::DecodeParams p{};
  p.R = n_requests;
  p.H = num_heads;
  p.D = d_k;
  p.conv_width = conv_width;
  p.n_new = n_new;
  p.prev_slots = prev->slots;
  p.cur_slots = cur->slots;
  p.act = act;
  p.n_acc = n_acc;
  p.n_new_r = n_new_per_request;
  p.prev_q = static_cast<const __bf16*>(prev->q);
  p.prev_k = static_cast<const __bf16*>(prev->k);
  p.prev_v = static_cast<const __bf16*>(prev->v);
  p.prev_g = static_cast<const __bf16*>(prev->g);
  p.prev_beta = static_cast<const __bf16*>(prev->beta);
  p.cur_q = static_cast<const __bf16*>(cur->q);
  p.cur_k = static_cast<const __bf16*>(cur->k);
  p.cur_v = static_cast<const __bf16*>(cur->v);
  p.cur_g = static_cast<const __bf16*>(cur->g);
  p.cur_beta = static_cast<const __bf16*>(cur->beta);
  p.cur_z = static_cast<const __bf16*>(cur->z);
  p.conv_w = conv_w;
  p.norm_w = norm_w;
  p.state = state;
  p.state_acc = state_acc;
  p.conv_tail = conv_tail;
  p.o = o;
  p.out_f32 = out_dtype == KDA_F32 ? 1 : 0;
  p.scale = scale;
  p.decay_floor = expf(g_min);
  p.eps_l2 = eps_l2;
  p.eps_rms = eps_rms;
  p.waves = kda::decode_waves(int64_t(n_requests) * num_heads, compute_units());
  return launch_status(kda::launch_decode_replay(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
