// CPU replay of every global-memory access of the raw-projection prefill (kda_chunk_fwd_raw):
// its grouping of sequences, the prep pass in raw mode (chunk_fwd_kernel with kPrep and kRaw)
// and the walk over fp32 values (chunk_walk_kernel with float values, one state tile per
// workgroup). The row and slot arithmetic comes from kda_index.h, the header the kernels call;
// the loop structure (which rows each thread touches in which chunk) follows the kernels. Each
// access is checked against the extent of the buffer it addresses, and the walk's reads of
// convolved values and slots against what the prep pass wrote.
//
// Built with g++ by tests/test_raw_addressing.py; no GPU, no HIP.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../linear_attention_recurrence_chunk_amd/csrc/kda_index.h"

namespace {

using namespace kda;

enum Buf { kQ, kK, kV, kG, kBeta, kConvW, kTailIn, kTailOut, kVConv, kOps, kH0, kO, kHt, kNumBufs };
const char* kNames[kNumBufs] = {"q", "k", "v", "g", "beta", "conv_w", "conv_tail_in",
                                "conv_tail_out", "v_conv", "ws_ops", "h0", "o", "ht"};

struct Config {
  int n_seqs;
  const int32_t* cu;   // host offsets [n_seqs + 1] or null (fixed length)
  int seq_len;         // tokens per sequence (fixed length) or the total (packed)
  int H, DK, W;
  int has_tail_in, has_tail_out, has_h0, has_ht, out_bytes;
  long long workspace_bytes;   // 0: the whole batch's need
  int legacy_history_rows;     // 1: history rows bounded below only (the code that faulted)
};

struct Checker {
  const Config& c;
  long long T;
  long long extent[kNumBufs];
  // group-relative regions of the workspace: v_conv [lo, hi) in the shifted base's bytes
  long long vconv_lo = 0, vconv_hi = 0;
  std::vector<uint8_t> vconv_written;   // per (token, head, channel quad) of the group
  std::vector<uint8_t> slot_written;    // per (slot, head) of the group
  long long group_tok0 = 0;
  long long n_oob = 0, n_unwritten = 0, n_access = 0;
  std::string report;

  explicit Checker(const Config& cfg) : c(cfg) {
    T = c.cu ? c.cu[c.n_seqs] : (long long)c.n_seqs * c.seq_len;
    const long long C3 = 3LL * c.DK;
    const long long H = c.H, DK = c.DK;
    extent[kQ] = extent[kK] = extent[kV] = extent[kG] = T * H * DK * 2;
    extent[kBeta] = T * H * 2;
    extent[kConvW] = H * C3 * c.W * 4;
    extent[kTailIn] = c.has_tail_in ? (long long)c.n_seqs * H * C3 * (c.W - 1) * 4 : 0;
    extent[kTailOut] = c.has_tail_out ? (long long)c.n_seqs * H * C3 * (c.W - 1) * 4 : 0;
    extent[kH0] = extent[kHt] = (long long)c.n_seqs * H * DK * DK * 4;
    extent[kO] = T * H * DK * c.out_bytes;
    extent[kVConv] = extent[kOps] = 0;   // per group
  }

  void note(const char* what, int buf, long long off, long long size, const char* where) {
    if (report.size() < 1500) {
      char line[256];
      snprintf(line, sizeof line, "%s %s bytes [%lld, %lld) of %lld (%s)\n", what, kNames[buf],
               off, off + size, buf == kVConv ? vconv_hi : extent[buf], where);
      report += line;
    }
  }

  // an access of size bytes at byte offset off of buffer buf
  void acc(int buf, long long off, long long size, const char* where) {
    ++n_access;
    long long lo = 0, hi = extent[buf];
    if (buf == kVConv) lo = vconv_lo, hi = vconv_hi;
    if (off < lo || off + size > hi) {
      ++n_oob;
      note("out of bounds:", buf, off, size, where);
    }
  }
};

template <int DK>
struct RawPlan {
  // prologue mapping (as in the kernels' ProMap)
  static constexpr int kLPT = DK / 4;
  static constexpr int kTPT = DK / 16;
  using VM = RawValueMap<DK>;
  static constexpr int kTPV = VM::kTPV;
};

// history row of the code that faulted: bounded below by the sequence start only
int legacy_history_row(int cs, int /*L*/, int rb0, int i, int W, int seq_bos) {
  const int tok = cs + rb0 - 1 - i;
  return (i + 1 < W && tok >= seq_bos) ? tok : -1;
}

template <int DK>
void prep_group(Checker& ck, int n0, int n1, long long tok0, int groups) {
  using P = RawPlan<DK>;
  const Config& c = ck.c;
  const int H = c.H, W = c.W;
  const long long C3 = 3LL * DK;
  const size_t SB = op_slot_bytes(DK);
  const int n_seqs = n1 - n0;
  const int n_units = n_seqs * groups * H;
  const int grid = (n_units + 7) / 8 * 8;
  for (int b = 0; b < grid; ++b) {
    int vt;
    const int unit = block_unit(b, 1, &vt);
    if (unit >= n_units) continue;
    const int h = unit % H;
    const int sj = unit / H;
    const int n = n0 + sj / groups;
    const int j = sj % groups;
    const int seq_bos = c.cu ? c.cu[n] : n * c.seq_len;
    const int seq_eos = c.cu ? c.cu[n + 1] : seq_bos + c.seq_len;
    const long long seq_slot0 = seq_first_slot(seq_bos, int(tok0), n, n0);
    int bos, eos, c_lo;
    segment_range(seq_bos, seq_eos, j, groups, &bos, &eos, &c_lo);
    const int len = seq_eos - seq_bos;
    const bool last_group = (len == 0 && j == 0) || (bos < eos && eos == seq_eos);
    const long long tb = ((long long)n * H + h) * C3 * (W - 1);
    for (int tid = 0; tid < 256; ++tid) {
      const int w = tid >> 6, lane = tid & 63;
      const int cq0 = 4 * (lane % P::kLPT);
      const int cv0 = P::VM::cv0(tid), tv0 = P::VM::tv0(tid);
      // taps
      for (int ch = 0; ch < 4; ++ch)
        for (int m = 0; m < 4; ++m) {
          const int mw = m - (4 - W);
          if (mw < 0) continue;
          ck.acc(kConvW, ((h * C3 + cq0 + ch) * W + mw) * 4, 4, "taps q");
          ck.acc(kConvW, ((h * C3 + DK + cq0 + ch) * W + mw) * 4, 4, "taps k");
          ck.acc(kConvW, ((h * C3 + 2 * DK + cv0 + ch) * W + mw) * 4, 4, "taps v");
        }
      // leaving tail
      if (c.has_tail_out && W > 1 && last_group) {
        for (int idx = tid; idx < C3 * (W - 1); idx += 256) {
          const int ch = idx / (W - 1), m = idx % (W - 1);
          int slot;
          const int pos = raw_tail_out_row(seq_bos, seq_eos, W, m, &slot);
          if (pos >= 0) {
            const int buf = ch < DK ? kQ : ch < 2 * DK ? kK : kV;
            const int cc = ch % DK;
            ck.acc(buf, (((long long)pos * H + h) * DK + cc) * 2, 2, "leaving tail row");
          } else if (c.has_tail_in) {
            ck.acc(kTailIn, (tb + (long long)ch * (W - 1) + slot) * 4, 4, "leaving tail slot");
          }
          ck.acc(kTailOut, (tb + (long long)ch * (W - 1) + m) * 4, 4, "leaving tail write");
        }
      }
      // a chunk's prologue inputs (g, k, q bf16 quads; beta) with the ragged-chunk fallback to
      // the chunk's first row
      auto load_chunk = [&](int cs, int L) {
        const int grp = lane / P::kLPT;
        for (int t = 0; t < P::kTPT; ++t) {
          const int r = 16 * w + grp * P::kTPT + t;
          const long long row = r < L ? cs + r : cs;
          const long long off = ((row * H + h) * DK + cq0) * 2;
          ck.acc(kG, off, 8, "chunk g");
          ck.acc(kK, off, 8, "chunk k");
          ck.acc(kQ, off, 8, "chunk q");
        }
        const int r = 16 * w + (lane & 15);
        const long long row = r < L ? cs + r : cs;
        ck.acc(kBeta, (row * H + h) * 2, 2, "chunk beta");
      };
      // convolution history rows and value rows of a chunk
      auto raw_prefetch = [&](int cs, int L) {
        const int rb0 = 16 * w + (lane / P::kLPT) * P::kTPT;
        for (int i = 0; i < 3; ++i) {
          const int tok = c.legacy_history_rows ? legacy_history_row(cs, L, rb0, i, W, seq_bos)
                                                : raw_history_row(cs, L, rb0, i, W, seq_bos);
          if (tok < 0) continue;
          const long long off = (((long long)tok * H + h) * DK + cq0) * 2;
          ck.acc(kQ, off, 8, "history q");
          ck.acc(kK, off, 8, "history k");
        }
        for (int i = 0; i < P::kTPV + 3; ++i) {
          const int tok = raw_value_row(cs, L, tv0, i, W, seq_bos);
          if (tok < 0) continue;
          ck.acc(kV, (((long long)tok * H + h) * DK + cv0) * 2, 8, "value row");
        }
      };
      if (bos < eos) {
        load_chunk(bos, std::min(kChunk, eos - bos));
        raw_prefetch(bos, std::min(kChunk, eos - bos));
      }
      for (int cstart = bos; cstart < eos; cstart += kChunk) {
        const int Lc = std::min(kChunk, eos - cstart);
        const int rb0 = 16 * w + (lane / P::kLPT) * P::kTPT;
        for (int i = 0; i < 3; ++i) {
          const int m = raw_history_tail_slot(cstart, rb0, i, W, seq_bos);
          if (m < 0 || !c.has_tail_in) continue;
          for (int ch = 0; ch < 4; ++ch) {
            ck.acc(kTailIn, (tb + (long long)(cq0 + ch) * (W - 1) + m) * 4, 4, "history tail q");
            ck.acc(kTailIn, (tb + (long long)(DK + cq0 + ch) * (W - 1) + m) * 4, 4,
                   "history tail k");
          }
        }
        for (int i = 0; i < P::kTPV + 3; ++i) {
          const int m = raw_value_tail_slot(cstart, Lc, tv0, i, W, seq_bos);
          if (m < 0 || !c.has_tail_in) continue;
          for (int ch = 0; ch < 4; ++ch)
            ck.acc(kTailIn, (tb + (long long)(2 * DK + cv0 + ch) * (W - 1) + m) * 4, 4,
                   "value tail");
        }
        for (int t = 0; t < P::kTPV; ++t) {
          const int tok = cstart + tv0 + t;
          if (tok >= cstart + Lc) continue;
          const long long off = (((long long)tok * H + h) * DK + cv0) * 4;
          ck.acc(kVConv, off, 16, "convolved value write");
          const long long e = ((tok - ck.group_tok0) * H + h) * (DK / 4) + cv0 / 4;
          if (e >= 0 && e < (long long)ck.vconv_written.size()) ck.vconv_written[e] = 1;
        }
        const bool more = cstart + kChunk < eos;
        if (more) {
          const int nstart = cstart + kChunk, nLc = std::min(kChunk, eos - nstart);
          raw_prefetch(nstart, nLc);
          load_chunk(nstart, nLc);
        }
        const long long slot = seq_slot0 + (cstart - seq_bos) / kChunk;
        ck.acc(kOps, (long long)((slot * H + h) * SB), (long long)SB, "slot write");
        const long long si = slot * H + h;
        if (si >= 0 && si < (long long)ck.slot_written.size()) ck.slot_written[si] = 1;
      }
    }
  }
}

template <int DK>
void walk_group(Checker& ck, int n0, int n1, long long tok0) {
  const Config& c = ck.c;
  const int H = c.H, DV = DK;
  const size_t SB = op_slot_bytes(DK);
  const int n_vt = DV / 64;
  const int n_seqs = n1 - n0;
  const int n_units = n_seqs * H;
  uint16_t order[kMaxOrder];
  const int n_order = walk_order(c.cu, n0, n1, order);
  const int grid = (n_units + 7) / 8 * 8 * n_vt;
  for (int b = 0; b < grid; ++b) {
    int vg;
    const int unit = block_unit(b, n_vt, &vg);
    if (unit >= n_units) continue;
    const int h = unit % H;
    const int sj = unit / H;
    const int n = n0 + (n_order > 0 ? int(order[sj]) : sj);
    const int seq_bos = c.cu ? c.cu[n] : n * c.seq_len;
    const int seq_eos = c.cu ? c.cu[n + 1] : seq_bos + c.seq_len;
    long long slot0 = seq_first_slot(seq_bos, int(tok0), n, n0);
    int bos, eos, c_lo;
    segment_range(seq_bos, seq_eos, 0, 1, &bos, &eos, &c_lo);
    slot0 += c_lo;
    const int nchunks = (eos - bos + kChunk - 1) / kChunk;
    const int vt = vg;
    for (int ci = 0; ci < nchunks; ++ci) {
      const long long si = (slot0 + ci) * H + h;
      ck.acc(kOps, si * (long long)SB, (long long)SB, "slot read");
      if (si < 0 || si >= (long long)ck.slot_written.size() || !ck.slot_written[si]) {
        ++ck.n_unwritten;
        ck.note("unwritten:", kOps, si * (long long)SB, (long long)SB, "slot read");
      }
    }
    for (int tid = 0; tid < 256; ++tid) {
      const int w = tid >> 6, lane = tid & 63;
      const int q4 = lane >> 4, ln = lane & 15;
      const int col0 = vt * 64 + 16 * w;
      const long long sbase = ((long long)n * H + h) * DK * DV;
      for (int t = 0; t < DK / 16; ++t)
        for (int e = 0; e < 4; ++e) {
          const long long el = sbase + (long long)(16 * t + 4 * q4 + e) * DV + col0 + ln;
          if (c.has_h0) ck.acc(kH0, el * 4, 4, "h0 read");
          if (c.has_ht) ck.acc(kHt, el * 4, 4, "ht write");
        }
      const int vc = vt * 64 + 16 * w + 4 * (ln >> 2);
      const int tq = 4 * q4 + (ln & 3);
      for (int cstart = bos; cstart < eos; cstart += kChunk) {
        const int L = std::min(kChunk, eos - cstart);
        for (int rb = 0; rb < 4; ++rb) {
          // fp32 values, with the ragged-chunk fallback to the chunk's first row
          const int r = 16 * rb + tq;
          const long long row = r < L ? cstart + r : cstart;
          ck.acc(kVConv, ((row * H + h) * DV + vc) * 4, 16, "walk value read");
          const long long e = ((row - ck.group_tok0) * H + h) * (DK / 4) + vc / 4;
          if (e < 0 || e >= (long long)ck.vconv_written.size() || !ck.vconv_written[e]) {
            ++ck.n_unwritten;
            ck.note("unwritten:", kVConv, ((row * H + h) * DV + vc) * 4, 16, "walk value read");
          }
          if (r < L)
            ck.acc(kO, ((long long)(cstart + 16 * rb + tq) * H * DV + (long long)h * DV + vc) *
                           c.out_bytes, 4 * c.out_bytes, "output write");
        }
      }
    }
  }
}

template <int DK>
void run(Checker& ck) {
  const Config& c = ck.c;
  const int H = c.H;
  auto raw_bytes = [&](int64_t tokens, int64_t seqs) {
    return raw_vconv_bytes(tokens, H, DK) + two_pass_workspace_bytes(tokens, seqs, H, DK);
  };
  const size_t need_all = raw_bytes(ck.T, c.n_seqs);
  const size_t budget = c.workspace_bytes > 0 ? size_t(c.workspace_bytes) : need_all;
  for_each_group(
      c.n_seqs, c.cu, c.seq_len, budget, raw_bytes,
      [&](int n0, int n1, int64_t tok0, int64_t tokens) {
        // the group's regions of the workspace: convolved values first, then its slots; the
        // kernels address the values from a base shifted back by the group's first token
        const size_t vbytes = raw_vconv_bytes(tokens, H, DK);
        const size_t obytes = two_pass_workspace_bytes(tokens, n1 - n0, H, DK);
        if (vbytes + obytes > budget) {
          ++ck.n_oob;
          ck.report += "group needs more workspace than given\n";
        }
        ck.group_tok0 = tok0;
        ck.vconv_lo = (long long)tok0 * H * DK * 4;
        ck.vconv_hi = ck.vconv_lo + (long long)vbytes;
        ck.extent[kVConv] = ck.vconv_hi;
        ck.extent[kOps] = (long long)obytes;
        ck.vconv_written.assign(size_t(tokens) * H * (DK / 4), 0);
        ck.slot_written.assign(size_t(op_slot_count(tokens, n1 - n0)) * H, 0);
        const int32_t* cu_g = c.cu ? c.cu + n0 : nullptr;
        const int groups = prep_groups(cu_g, n1 - n0, c.seq_len);
        prep_group<DK>(ck, n0, n1, tok0, groups);
        walk_group<DK>(ck, n0, n1, tok0);
        return 0;
      },
      0);
}

}  // namespace

// Replays one kda_chunk_fwd_raw call. Returns the number of out-of-bounds accesses plus reads
// of workspace the prep pass never wrote; *n_access receives the number of accesses checked and
// report (report_len bytes) the first findings.
extern "C" long long kda_raw_addr_check(int n_seqs, const int32_t* cu_seqlens, int seq_len,
                                        int H, int DK, int W, int has_tail_in, int has_tail_out,
                                        int has_h0, int has_ht, int out_bytes,
                                        long long workspace_bytes, int legacy_history_rows,
                                        long long* n_access, char* report, int report_len) {
  Config c{n_seqs, cu_seqlens, seq_len, H, DK, W, has_tail_in, has_tail_out, has_h0, has_ht,
           out_bytes, workspace_bytes, legacy_history_rows};
  Checker ck(c);
  if (DK == 128) run<128>(ck);
  else if (DK == 64) run<64>(ck);
  else return -1;
  if (n_access) *n_access = ck.n_access;
  if (report && report_len > 0) {
    strncpy(report, ck.report.c_str(), size_t(report_len) - 1);
    report[report_len - 1] = 0;
  }
  return ck.n_oob + ck.n_unwritten;
}
