// C ABI of libkda: argument validation (host only, no HIP call) and kernel dispatch.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

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

// Shared validation of the prefill entry points. Fills the sequence count and token total.
int validate_prefill(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* h0, const int32_t* cu_seqlens,
                     const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                     int num_heads, int d_k, int d_v, int io_dtype, int out_dtype,
                     float scale, float g_min, const void* o, const float* ht, int* out_N,
                     int64_t* out_T) {
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
  const bool ok_f32 = io_dtype == KDA_F32 && d_k == 64 && d_v == 64;
  if (!ok_bf16 && !ok_f32) return KDA_ERR_UNSUPPORTED;

  const void* ptrs[] = {q, k, v, g, beta, o, h0, ht};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;

  const size_t es = dsize(io_dtype);
  const Range rq = range_of(q, size_t(T) * num_heads * d_k * es);
  const Range rk = range_of(k, size_t(T) * num_heads * d_k * es);
  const Range rv = range_of(v, size_t(T) * num_heads * d_v * es);
  const Range rg = range_of(g, size_t(T) * num_heads * d_k * 4);
  const Range rb = range_of(beta, size_t(T) * num_heads * 4);
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
    default: return "unknown status";
  }
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                  const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                  int num_heads, int d_k, int d_v, int io_dtype, int out_dtype, float scale,
                  float g_min, void* o, float* ht, void* stream) {
  int N = 0;
  int64_t T = 0;
  const int st = validate_prefill(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch,
                                  seq_len, n_seqs, num_heads, d_k, d_v, io_dtype, out_dtype, scale,
                                  g_min, o, ht, &N, &T);
  if (st != KDA_OK) return st;
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
  p.n_units = N * num_heads;
  p.scale = scale;
  p.g_min = g_min;
  return launch_status(
      kda::launch_chunk_fwd(p, io_dtype, out_dtype, d_k, static_cast<hipStream_t>(stream)));
}

int kda_segment_cp_workspace_size(int n_seqs, int num_heads, int d_k, int d_v, int n_segments,
                                  size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_ARG;
  (void)n_seqs; (void)num_heads; (void)d_k; (void)d_v; (void)n_segments;
  return KDA_ERR_UNSUPPORTED;
}

int kda_segment_cp_fwd(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* h0, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_host, int batch, int seq_len, int n_seqs,
                       int num_heads, int d_k, int d_v, int io_dtype, int out_dtype,
                       float scale, float g_min, void* o, float* ht, int n_segments,
                       void* workspace,
                       size_t workspace_bytes, void* stream) {
  int N = 0;
  int64_t T = 0;
  const int st = validate_prefill(q, k, v, g, beta, h0, cu_seqlens, cu_seqlens_host, batch,
                                  seq_len, n_seqs, num_heads, d_k, d_v, io_dtype, out_dtype, scale,
                                  g_min, o, ht, &N, &T);
  if (st != KDA_OK) return st;
  (void)n_segments; (void)workspace; (void)workspace_bytes; (void)stream;
  return KDA_ERR_UNSUPPORTED;
}

int kda_decode_replay(int n_requests, int num_heads, int d_k, int d_v, int conv_width,
                      int n_new, const int32_t* n_acc, const kda_token_window* prev,
                      const kda_token_window* cur, const float* conv_w, const float* norm_w,
                      float scale, float g_min, float eps_l2, float eps_rms, int act,
                      float* state, float* state_acc, float* conv_tail, void* o,
                      void* stream) {
  (void)n_requests; (void)num_heads; (void)d_k; (void)d_v; (void)conv_width; (void)n_new;
  (void)n_acc; (void)prev; (void)cur; (void)conv_w; (void)norm_w; (void)scale; (void)g_min;
  (void)eps_l2; (void)eps_rms; (void)act; (void)state; (void)state_acc; (void)conv_tail;
  (void)o; (void)stream;
  return KDA_ERR_UNSUPPORTED;
}

}  // extern "C"
