// plan.hpp -- host-side planning shared by the library's translation units:
// launch limits, workspace layouts of the decode schedules, and the
// arguments handed to the decode kernel launchers (whose instantiations are
// compiled separately, per head_dim, element type and set of group sizes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "adamas.h"
#include "kernels.hpp"

namespace adm_host {

using namespace adm;

constexpr int kMaxG = 8;                   // query heads per KV head
constexpr int64_t kMaxGroups = 8192;       // B*Hq and B*Hkv (control-area slots)
constexpr size_t kCtrlSelect = 0;          // u32 counters of select / decode groups
constexpr size_t kCtrlAttend = 32768;      // u32 counters of attention rows
constexpr int kMaxBudget = 1 << 20;
constexpr size_t kLdsLimit = 64 * 1024;    // per-workgroup LDS used by any kernel here
// ... except the decode chunk scan, which keeps G * chunk u16 distances: up
// to the 160 KiB a gfx950 workgroup may hold (one 1024-thread workgroup per
// compute unit either way), so grouped heads scan chunks as long as MHA ones
constexpr size_t kLdsDecodeLimit = 160 * 1024;
constexpr int64_t kComputeUnits = 256;     // MI355X; workgroups of one decode round
// Paged caches: a page holds at least one scan load of a wavefront per KV head
constexpr int kMinPageTokens = 1024, kMaxPageTokens = 16384;
constexpr int kMaxCandTile = 8192;         // candidate entries staged in LDS at once
constexpr size_t kStreamBlocks = 1024;     // adamas_stream_read: four slices per compute unit
constexpr uint32_t kDefaultWaitPolls = 1u << 20;  // polls of a group wait before it gives up

inline bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool valid_dtype(int dt) { return dt == ADAMAS_F32 || dt == ADAMAS_BF16; }
inline bool valid_dim(int d) { return d == 64 || d == 128 || d == 256; }
inline size_t nbins_padded(int D) { return (size_t)kNbinsPadded(D); }

// Calls f(std::integral_constant<int, D>{}) for a supported head_dim D.
template <class F>
inline void with_dim(int d, F&& f) {
  if (d == 256)
    f(std::integral_constant<int, 256>{});
  else if (d == 128)
    f(std::integral_constant<int, 128>{});
  else
    f(std::integral_constant<int, 64>{});
}

// Candidate layout shared by the selection kernels: per head, n_chunks slots
// of kpad u32 entries, kpad the power of two >= max(4, min(budget, chunk)).
struct SelectPlan {
  int chunk = 0, n_chunks = 0, kpad = 0, kpad_log2 = 0, mcap = 0;
  size_t cand_off = 0, end = 0, lds = 0;
};

inline void finish_select_plan(SelectPlan& p, int64_t rows, int64_t n_ctx, int budget, size_t start) {
  p.n_chunks = (int)((n_ctx + p.chunk - 1) / p.chunk);
  const int kmax = budget < p.chunk ? budget : p.chunk;
  p.kpad_log2 = 2;
  while ((1 << p.kpad_log2) < kmax) ++p.kpad_log2;
  p.kpad = 1 << p.kpad_log2;
  const int64_t m = (int64_t)p.n_chunks * p.kpad;
  p.mcap = (int)(m < kMaxCandTile ? m : kMaxCandTile);
  p.cand_off = round_up(start, 256);
  p.end = p.cand_off + (size_t)rows * (size_t)m * sizeof(uint32_t);
}

// adamas_select_topk: 1024-thread workgroups over chunks of the distances.
inline SelectPlan plan_select(int64_t rows, int64_t n_ctx, int budget, int D, size_t start) {
  SelectPlan p;
  int c = 4096;
  while (c < 16384 && c < 8 * budget) c *= 2;
  while (c > kSelectThreads && (int64_t)(c / 2) >= n_ctx) c /= 2;
  for (;;) {
    p.chunk = c;
    finish_select_plan(p, rows, n_ctx, budget, start);
    const size_t region = std::max((size_t)p.chunk * 2, (size_t)p.mcap * 4);
    p.lds = kTmpWords * 4 + nbins_padded(D) * 4 + (size_t)p.kpad * 4 + region;
    if (p.lds <= kLdsLimit || c <= kSelectThreads) break;
    c /= 2;
  }
  return p;
}

// Decode kernel LDS: scan phase (query words, histograms, distances) and the
// aliasing final phase (histogram, attention partials, indices, candidates).
inline int cand_slot(int budget, int chunk) {
  const int kmax = budget < chunk ? budget : chunk;
  int k = 4;
  while (k < kmax) k *= 2;
  return k;
}
// key_bytes: 2, or 1 for the 8-bit key variant
inline size_t decode_lds_scan(int D, int G, int c, int budget, int key_bytes = 2) {
  const int kpad = cand_slot(budget, c);
  return (size_t)(G + 1) * (D / 16) * 4 + (size_t)G * nbins_padded(D) * 4 +
         (size_t)stage_heads(G, kpad) * kpad * 4 + (size_t)G * c * key_bytes +
         (size_t)(2 + kDecodeThreads / kWave) * G * 4;
}
// sel_rows = min(budget, n_ctx) indices are kept in LDS only when attention is fused.
inline size_t decode_lds_final(int D, int sel_rows_lds, int mcap) {
  const int nw = kDecodeThreads / kWave;
  return nbins_padded(D) * 4 + (size_t)(nw + 1) * (2 + D) * 4 + (size_t)kAttendThreads / 16 * 4 +
         (size_t)((sel_rows_lds + 3) & ~3) * 4 + (size_t)mcap * 4;
}

struct AttendPlan {
  int splits = 0;
  size_t part_off = 0, end = 0;
};

inline AttendPlan plan_attend(int64_t rows, int sel_rows, int D, size_t start) {
  AttendPlan p;
  p.splits = (sel_rows + kAttendRowsPerBatch - 1) / kAttendRowsPerBatch;
  p.part_off = round_up(start, 256);
  const size_t pwp = (size_t)((2 + D + 3) & ~3);
  p.end = p.part_off + (p.splits > 1 ? (size_t)rows * p.splits * pwp * sizeof(float) : 0);
  return p;
}

struct DecodePlan {
  SelectPlan sel;
  bool u8 = false;  // k_decode keeps 8-bit keys (fewer rounds of workgroups)
  bool big = false;  // MHA chunks of 32768 tokens, two workgroups per CU, compacted by halves
  bool fuse = false;
  size_t idx_off = 0;
  AttendPlan att;
  // SPLIT schedule: per-chunk key counts [B*Hq][ncp][kNbinsHist(D)] u16 at chist_off,
  // attention partials [B*Hq][segs][2 + D padded to 4] f32 at spart_off
  bool split_ok = false;
  int ncp = 0, seg_chunks = 0, segs = 0;
  size_t chist_off = 0, spart_off = 0;
  size_t total = 0;
};
constexpr int kSplitSegChunks = 8;  // chunks per k_split_select workgroup

// LDS of k_split_select: scratch, key counts, two per-chunk arrays, and when
// the attention is fused the row list and the attention scratch.
inline size_t split_select_lds(int D, int ncp, bool fused) {
  const size_t nw = kSplitThreads / kWave, pw = 2 + D, pwp = (pw + 3) & ~3;
  size_t b = (size_t)kTmpWords * 4 + (size_t)kNbinsPadded(D) * 4 + 2 * (size_t)ncp * 4;
  if (fused) b += (size_t)kSplitFuseRows * 4 + (nw * pw + kSplitThreads / 16 + pwp) * 4;
  return b;
}

// The rest of a decode plan once its chunk (and key width) are fixed.
inline void finish_decode_plan(DecodePlan& p, int B, int Hq, int Hkv, int64_t n_ctx, int budget,
                               int D, int c);

// Whether a last-arrival launch of the plan runs two workgroups per CU (the
// OCC build): MHA launches of more than one round whose LDS allows it.
inline bool decode_two_per_cu(const DecodePlan& p, int G, int64_t wgs) {
  return G == 1 && wgs > kComputeUnits && 2 * p.sel.lds <= kLdsDecodeLimit;
}

// adamas_decode_step: 1024-thread workgroups, chunks as large as LDS allows
// (fewer candidates to merge), attention fused into the selecting workgroup
// when the selection is small (at most two 256-row batches for the group).
// allow_u8: the launch may take the 8-bit key variant of k_decode (plain
// contiguous decode steps; the ragged and paged steps keep 16-bit keys).
// allow_big: MHA launches of several rounds may take 32768-token chunks
// (not the paged step, whose wavefront stretches must stay inside a page).
inline DecodePlan plan_decode(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int D,
                              bool allow_u8 = true, bool allow_big = true) {
  DecodePlan p;
  const int G = Hq / Hkv;
  auto chunk_for = [&](int c0, int key_bytes) {
    int c = c0;
    while (c > 1024 && kTmpWords * 4 + decode_lds_scan(D, G, c, budget, key_bytes) > kLdsDecodeLimit)
      c /= 2;
    while (c > 1024 && (int64_t)(c / 2) >= n_ctx) c /= 2;
    // shorter chunks while the whole launch still fits one workgroup per
    // compute unit: more of the device streams the code cache
    while (c > 1024 && (int64_t)B * Hkv * ((n_ctx + c / 2 - 1) / (c / 2)) <= kComputeUnits)
      c /= 2;
    return c;
  };
  auto rounds = [&](int c) {
    return ((int64_t)B * Hkv * ((n_ctx + c - 1) / c) + kComputeUnits - 1) / kComputeUnits;
  };
  // 16-bit keys: at most 16384 tokens, one compaction pass of 16 per thread
  int c = chunk_for(16384, 2);
  // MHA launches of several rounds: chunks twice as long while two
  // workgroups still share a CU halve the workgroups, candidate lists and
  // final merges (the chunk is compacted a half at a time)
  if (allow_big && G == 1 && c == 16384 && rounds(c) > 1 && rounds(2 * c) < rounds(c) &&
      2 * (kTmpWords * 4 + decode_lds_scan(D, 1, 2 * c, budget, 2)) <= kLdsDecodeLimit) {
    DecodePlan q;
    q.big = true;
    finish_decode_plan(q, B, Hq, Hkv, n_ctx, budget, D, 2 * c);
    if (decode_two_per_cu(q, G, (int64_t)B * Hkv * q.sel.n_chunks)) return q;
  }
  // grouped heads whose 16-bit keys cap the chunk so that the launch takes
  // more than one round: 8-bit keys hold chunks twice as long (up to 32768
  // tokens, one compaction thread per 32), when that saves rounds and every
  // head's candidates stage at once
  if (allow_u8 && G >= 2 && D <= 128 && rounds(c) > 1) {
    const int c8 = chunk_for(32768, 1);
    if (rounds(c8) < rounds(c) && stage_heads(G, cand_slot(budget, c8)) == G) {
      c = c8;
      p.u8 = true;
    }
  }
  finish_decode_plan(p, B, Hq, Hkv, n_ctx, budget, D, c);
  return p;
}

inline void finish_decode_plan(DecodePlan& p, int B, int Hq, int Hkv, int64_t n_ctx, int budget,
                               int D, int c) {
  const int G = Hq / Hkv;
  const int64_t rows = (int64_t)B * Hq;
  p.sel.chunk = c;
  finish_select_plan(p.sel, rows, n_ctx, budget, ADAMAS_WS_CTRL_BYTES);
  const int bsel = (int)(n_ctx < budget ? n_ctx : budget);
  const int batches = G * ((bsel + kAttendRowsPerBatch - 1) / kAttendRowsPerBatch);
  p.fuse = batches <= 2;
  const int sidx_rows = p.fuse ? bsel : 0;
  // shrink the LDS candidate tile if the final phase would not fit
  while (p.sel.mcap > 256 &&
         kTmpWords * 4 + decode_lds_final(D, sidx_rows, p.sel.mcap) > kLdsDecodeLimit)
    p.sel.mcap = (p.sel.mcap / 2 + 3) & ~3;
  p.sel.lds = kTmpWords * 4 + std::max(decode_lds_scan(D, G, c, budget, p.u8 ? 1 : 2),
                                       decode_lds_final(D, sidx_rows, p.sel.mcap));
  p.idx_off = round_up(p.sel.end, 256);
  const size_t idx_end = p.idx_off + (size_t)rows * budget * sizeof(int32_t);
  p.att = plan_attend(rows, bsel, D, idx_end);
  p.ncp = (p.sel.n_chunks + 7) & ~7;
  p.split_ok = p.sel.n_chunks <= kSplitMaxChunks;
  p.seg_chunks = kSplitSegChunks;
  p.segs = (p.sel.n_chunks + kSplitSegChunks - 1) / kSplitSegChunks;
  p.chist_off = round_up(p.att.end, 256);
  size_t end = p.att.end;
  if (p.split_ok) {
    const size_t chist_end = p.chist_off + (size_t)rows * (size_t)p.ncp * kNbinsHist(D) * 2;
    p.spart_off = round_up(chist_end, 256);
    end = p.spart_off + (size_t)rows * p.segs * (size_t)((2 + D + 3) & ~3) * 4;
  }
  p.total = round_up(end, 256);
}

// More chunk candidates per head than the selecting workgroup holds in
// registers (four per thread): it would select from them in LDS tiles, and
// the separate selection is faster (1M-token MHA layer, budget 256, 32
// chunks of 256 candidates per head: 184 against 190 us).
inline bool many_candidates(const DecodePlan& p) {
  return (int64_t)p.sel.n_chunks * p.sel.kpad > 4 * kDecodeThreads;
}

// adamas_decode_step with group waits (k_decode_gs): every workgroup of the
// launch must be resident at once, so the grid is kept within one
// 1024-thread workgroup per compute unit (always resident: at most 128 VGPRs
// and 64 KiB of LDS per workgroup).  Chunks are as small as that allows
// (more compute units streaming), and no smaller than 1024 tokens.
struct GroupPlan {
  bool ok = false;
  bool u8 = false;  // k_decode_gs keeps 8-bit keys (chunks that fit the device)
  int chunk = 0, n_chunks = 0, cmax = 0;
  size_t lds = 0, hist_off = 0, part_off = 0, total = 0;
};

inline size_t decode_gs_lds(int D, int G, int c, int cmax, int key_bytes = 2) {
  const int nw = kDecodeThreads / kWave;
  const size_t pwp = (size_t)((2 + D + 3) & ~3);
  const size_t attend = ((size_t)nw * (2 + D) + kDecodeThreads / 16 + pwp) * 4;
  const size_t merge = (size_t)kGsMergeTile * pwp * 4;
  return (size_t)kTmpWords * 4 + 32 * 4 + (size_t)G * (D / 16) * 4 +
         (size_t)(G + 2) * nbins_padded(D) * 4 + (size_t)G * cmax * 4 +
         std::max({(size_t)G * c * key_bytes, attend, merge});
}

// allow_u8: the 8-bit key variant may take shapes the 16-bit one cannot
// hold at once (a forced group wait; the automatic choice does not take it:
// with tens of chunks per group its histogram exchange and merge cost more
// than the split schedule's second launch).
inline GroupPlan plan_decode_gs(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int D,
                                int64_t capacity, bool allow_u8 = false) {
  GroupPlan p;
  const int G = Hq / Hkv;
  const int64_t groups = (int64_t)B * Hkv, rows = (int64_t)B * Hq;
  const int64_t bsel = n_ctx < budget ? n_ctx : budget;
  auto cmax_of = [&](int c) { return (int)((std::min<int64_t>(bsel, c) + 3) & ~3); };
  auto chunks_of = [&](int c) { return (n_ctx + c - 1) / c; };
  int c = 16384;
  while (c > 1024 && decode_gs_lds(D, G, c, cmax_of(c)) > kLdsLimit) c /= 2;
  while (c > 1024 && groups * chunks_of(c / 2) <= capacity &&
         decode_gs_lds(D, G, c / 2, cmax_of(c / 2)) <= kLdsLimit)
    c /= 2;
  p.chunk = c;
  p.n_chunks = (int)chunks_of(c);
  p.cmax = cmax_of(c);
  p.lds = decode_gs_lds(D, G, c, p.cmax);
  const size_t nbh = (size_t)((3 * D + 1 + 7) & ~7), pwp = (size_t)((2 + D + 3) & ~3);
  p.hist_off = round_up(ADAMAS_WS_CTRL_BYTES, 256);
  p.part_off = round_up(p.hist_off + (size_t)rows * p.n_chunks * nbh * 2, 256);
  p.total = round_up(p.part_off + (size_t)rows * p.n_chunks * pwp * 4, 256);
  p.ok = p.lds <= kLdsLimit && groups * p.n_chunks <= capacity && groups <= kMaxGroups;
  // grouped heads whose 16-bit keys need more chunks than the device holds
  // at once: 8-bit keys in chunks up to 32768 tokens and the whole LDS
  if (!p.ok && allow_u8 && G >= 2 && D <= 128 && groups <= kMaxGroups) {
    auto lds8 = [&](int cc) { return decode_gs_lds(D, G, cc, cmax_of(cc), 1); };
    int c8 = 32768;
    while (c8 > 1024 && lds8(c8) > kLdsDecodeLimit) c8 /= 2;
    while (c8 > 1024 && groups * chunks_of(c8 / 2) <= capacity) c8 /= 2;
    if (lds8(c8) <= kLdsDecodeLimit && groups * chunks_of(c8) <= capacity) {
      p.u8 = true;
      p.chunk = c8;
      p.n_chunks = (int)chunks_of(c8);
      p.cmax = cmax_of(c8);
      p.lds = lds8(c8);
      p.part_off = round_up(p.hist_off + (size_t)rows * p.n_chunks * nbh * 2, 256);
      p.total = round_up(p.part_off + (size_t)rows * p.n_chunks * pwp * 4, 256);
      p.ok = true;
    }
  }
  return p;
}

struct DecodeArgs {
  const void *q, *k, *v;
  const uint8_t* kc;
  int Hq, Hkv;
  int64_t cap, n_ctx;
  int budget;
  float qscale;
  uint32_t *cand, *ctr;
  int32_t* idx;
  void* out;
  int n_sink, n_recent;
  RaggedArgs rg;  // lens == nullptr: every sequence holds n_ctx rows
  uint16_t* chist = nullptr;  // SPLIT: per-chunk key counts, selection left to k_split_select
  int ncp = 0;
  EncodeRule rule{1, 0, {}};  // rotation mode and bucketing alphas at launch
  uint32_t wait_polls = kDefaultWaitPolls;  // group-wait bound (adamas_set_wait_polls)
  uint64_t* stamps = nullptr;  // phase stamps (measurement build), or null
};

// Dynamic LDS beyond 64 KiB must be allowed per kernel before its launch.
template <class K>
inline void allow_lds(K kernel, size_t lds) {
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// Launchers of the decode kernels (decode_inst.hip), one instantiation per
// head_dim D, group size G = Hq / Hkv and element type.
template <int D, int G, bool BF>
void launch_decode_t(const DecodePlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a);
template <int D, int G, bool BF>
void launch_decode_gs_t(const GroupPlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a,
                        uint8_t* w);

}  // namespace adm_host
