// adamas.hip -- C ABI of the MI355X ADAMAS decode path (declared in
// include/adamas.h): host-side argument checks, workspace layout and kernel
// launches.  Citations refer to the ADAMAS article
// (www.lnwmold.com/news/826806) by its numbered sections.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "adamas.h"
#include "kernels.hpp"

namespace {

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

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool valid_dtype(int dt) { return dt == ADAMAS_F32 || dt == ADAMAS_BF16; }
bool valid_dim(int d) { return d == 64 || d == 128 || d == 256; }
size_t nbins_padded(int D) { return (size_t)kNbinsPadded(D); }

// Calls f(std::integral_constant<int, D>{}) for a supported head_dim D.
template <class F>
void with_dim(int d, F&& f) {
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

void finish_select_plan(SelectPlan& p, int64_t rows, int64_t n_ctx, int budget, size_t start) {
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
SelectPlan plan_select(int64_t rows, int64_t n_ctx, int budget, int D, size_t start) {
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
int cand_slot(int budget, int chunk) {
  const int kmax = budget < chunk ? budget : chunk;
  int k = 4;
  while (k < kmax) k *= 2;
  return k;
}
size_t decode_lds_scan(int D, int G, int c, int budget) {
  const int kpad = cand_slot(budget, c);
  return (size_t)(G + 1) * (D / 16) * 4 + (size_t)G * nbins_padded(D) * 4 +
         (size_t)stage_heads(G, kpad) * kpad * 4 + (size_t)G * c * 2 +
         (size_t)(2 + kDecodeThreads / kWave) * G * 4;
}
// sel_rows = min(budget, n_ctx) indices are kept in LDS only when attention is fused.
size_t decode_lds_final(int D, int sel_rows_lds, int mcap) {
  const int nw = kDecodeThreads / kWave;
  return nbins_padded(D) * 4 + (size_t)(nw + 1) * (2 + D) * 4 + (size_t)kAttendThreads / 16 * 4 +
         (size_t)((sel_rows_lds + 3) & ~3) * 4 + (size_t)mcap * 4;
}

struct AttendPlan {
  int splits = 0;
  size_t part_off = 0, end = 0;
};

AttendPlan plan_attend(int64_t rows, int sel_rows, int D, size_t start) {
  AttendPlan p;
  p.splits = (sel_rows + kAttendRowsPerBatch - 1) / kAttendRowsPerBatch;
  p.part_off = round_up(start, 256);
  const size_t pwp = (size_t)((2 + D + 3) & ~3);
  p.end = p.part_off + (p.splits > 1 ? (size_t)rows * p.splits * pwp * sizeof(float) : 0);
  return p;
}

struct DecodePlan {
  SelectPlan sel;
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
size_t split_select_lds(int D, int ncp, bool fused) {
  const size_t nw = kSplitThreads / kWave, pw = 2 + D, pwp = (pw + 3) & ~3;
  size_t b = (size_t)kTmpWords * 4 + (size_t)kNbinsPadded(D) * 4 + 2 * (size_t)ncp * 4;
  if (fused) b += (size_t)kSplitFuseRows * 4 + (nw * pw + kSplitThreads / 16 + pwp) * 4;
  return b;
}

// adamas_decode_step: 1024-thread workgroups, chunks as large as LDS allows
// (fewer candidates to merge), attention fused into the selecting workgroup
// when the selection is small (at most two 256-row batches for the group).
DecodePlan plan_decode(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int D) {
  DecodePlan p;
  const int G = Hq / Hkv;
  const int64_t rows = (int64_t)B * Hq;
  int c = 16384;
  while (c > 1024 && kTmpWords * 4 + decode_lds_scan(D, G, c, budget) > kLdsDecodeLimit) c /= 2;
  while (c > 1024 && (int64_t)(c / 2) >= n_ctx) c /= 2;
  // shorter chunks while the whole launch still fits one workgroup per
  // compute unit: more of the device streams the code cache
  while (c > 1024 && (int64_t)B * Hkv * ((n_ctx + c / 2 - 1) / (c / 2)) <= kComputeUnits) c /= 2;
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
  p.sel.lds = kTmpWords * 4 + std::max(decode_lds_scan(D, G, c, budget),
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
  return p;
}

// More chunk candidates per head than one LDS tile holds: one workgroup
// selecting from them all would take several passes over global memory.
bool many_candidates(const DecodePlan& p) {
  return (int64_t)p.sel.n_chunks * p.sel.kpad > kMaxCandTile;
}

// adamas_decode_step with group waits (k_decode_gs): every workgroup of the
// launch must be resident at once, so the grid is kept within one
// 1024-thread workgroup per compute unit (always resident: at most 128 VGPRs
// and 64 KiB of LDS per workgroup).  Chunks are as small as that allows
// (more compute units streaming), and no smaller than 1024 tokens.
struct GroupPlan {
  bool ok = false;
  int chunk = 0, n_chunks = 0, cmax = 0;
  size_t lds = 0, hist_off = 0, part_off = 0, total = 0;
};

size_t decode_gs_lds(int D, int G, int c, int cmax) {
  const int nw = kDecodeThreads / kWave;
  const size_t pwp = (size_t)((2 + D + 3) & ~3);
  const size_t attend = ((size_t)nw * (2 + D) + kDecodeThreads / 16 + pwp) * 4;
  const size_t merge = (size_t)kGsMergeTile * pwp * 4;
  return (size_t)kTmpWords * 4 + 32 * 4 + (size_t)G * (D / 16) * 4 +
         (size_t)(G + 2) * nbins_padded(D) * 4 + (size_t)G * cmax * 4 +
         std::max({(size_t)G * c * 2, attend, merge});
}

GroupPlan plan_decode_gs(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int D,
                         int64_t capacity) {
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
  return p;
}

// Workgroups of one launch that are resident together: one per compute unit.
int64_t device_capacity() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Sizing a workspace does not know the device: size for a capacity no device
// here exceeds, which gives the most chunks.
constexpr int64_t kSizingCapacity = 1024;

std::atomic<int> g_decode_mode{ADAMAS_DECODE_AUTO};
std::atomic<int> g_rotation{1};
int rotation_on() { return g_rotation.load(std::memory_order_relaxed); }

int launch_status() {
  return hipGetLastError() == hipSuccess ? ADAMAS_OK : ADAMAS_ERR_DEVICE;
}

// ---------------------------------------------------------- kernel tables
template <int D, int G>
void launch_score_t(dim3 grid, hipStream_t s, const uint8_t* qc, const uint8_t* kc, int Hq,
                    int Hkv, int64_t cap, int64_t n_ctx, int chunk, uint16_t* dist) {
  k_score<D, G><<<grid, kScoreThreads, 0, s>>>(qc, kc, Hq, Hkv, cap, n_ctx, chunk, dist);
}

template <int D>
bool dispatch_score(int G, dim3 grid, hipStream_t s, const uint8_t* qc, const uint8_t* kc,
                    int Hq, int Hkv, int64_t cap, int64_t n_ctx, int chunk, uint16_t* dist) {
  switch (G) {
#define ADM_CASE(g) \
  case g: launch_score_t<D, g>(grid, s, qc, kc, Hq, Hkv, cap, n_ctx, chunk, dist); return true;
    ADM_CASE(1) ADM_CASE(2) ADM_CASE(3) ADM_CASE(4) ADM_CASE(5) ADM_CASE(6) ADM_CASE(7)
    ADM_CASE(8)
#undef ADM_CASE
    default: return false;
  }
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
};

// Dynamic LDS beyond 64 KiB must be allowed per kernel before its launch.
template <class K>
void allow_lds(K kernel, size_t lds) {
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <int D, int G, bool BF, int RAG, bool OCC>
void launch_decode_k(const DecodePlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  allow_lds(&k_decode<D, G, BF, RAG, OCC>, p.sel.lds);
  k_decode<D, G, BF, RAG, OCC><<<grid, kDecodeThreads, p.sel.lds, s>>>(
      a.q, a.k, a.v, a.kc, a.Hq, a.Hkv, a.cap, a.n_ctx, p.sel.chunk, p.sel.n_chunks, a.budget,
      p.sel.kpad_log2, p.sel.mcap, (p.fuse && !a.chist) ? 1 : 0, a.qscale, a.cand, a.ctr, a.idx,
      a.out, a.n_sink, a.n_recent, rotation_on(), a.rg, RAG ? nullptr : a.chist,
      RAG ? 0 : a.ncp);
}

template <int D, int G, bool BF>
void launch_decode_t(const DecodePlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  // MHA launches of several rounds run two workgroups per compute unit
  // when their LDS allows it
  const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
  const bool occ = G == 1 && wgs > kComputeUnits && 2 * p.sel.lds <= kLdsDecodeLimit;
  const int rag = a.rg.lens == nullptr ? 0 : (a.rg.pages == nullptr ? 1 : 2);
  if constexpr (G == 1) {
    if (occ) {
      if (rag == 2)
        launch_decode_k<D, G, BF, 2, true>(p, grid, s, a);
      else if (rag == 1)
        launch_decode_k<D, G, BF, 1, true>(p, grid, s, a);
      else
        launch_decode_k<D, G, BF, 0, true>(p, grid, s, a);
      return;
    }
  }
  if (rag == 2)
    launch_decode_k<D, G, BF, 2, false>(p, grid, s, a);
  else if (rag == 1)
    launch_decode_k<D, G, BF, 1, false>(p, grid, s, a);
  else
    launch_decode_k<D, G, BF, 0, false>(p, grid, s, a);
}

template <int D, int G, bool BF>
void launch_decode_gs_t(const GroupPlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a,
                        uint8_t* w) {
  k_decode_gs<D, G, BF><<<grid, kDecodeThreads, p.lds, s>>>(
      a.q, a.k, a.v, a.kc, a.Hq, a.Hkv, a.cap, a.n_ctx, p.chunk, p.n_chunks, a.budget, p.cmax,
      a.qscale, reinterpret_cast<uint16_t*>(w + p.hist_off),
      reinterpret_cast<float*>(w + p.part_off), reinterpret_cast<uint32_t*>(w + kCtrlSelect),
      reinterpret_cast<uint32_t*>(w + kCtrlAttend),
      reinterpret_cast<uint32_t*>(w + ADAMAS_WS_STATUS_OFFSET), a.idx, a.out, a.n_sink,
      a.n_recent, rotation_on());
}

template <int D, bool BF>
bool dispatch_decode_gs(int G, const GroupPlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a,
                        uint8_t* w) {
  switch (G) {
#define ADM_CASE(g) \
  case g: launch_decode_gs_t<D, g, BF>(p, grid, s, a, w); return true;
    ADM_CASE(1) ADM_CASE(2) ADM_CASE(3) ADM_CASE(4) ADM_CASE(5) ADM_CASE(6) ADM_CASE(7)
    ADM_CASE(8)
#undef ADM_CASE
    default: return false;
  }
}

template <int D, bool BF>
bool dispatch_decode(int G, const DecodePlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  switch (G) {
#define ADM_CASE(g) \
  case g: launch_decode_t<D, g, BF>(p, grid, s, a); return true;
    ADM_CASE(1) ADM_CASE(2) ADM_CASE(3) ADM_CASE(4) ADM_CASE(5) ADM_CASE(6) ADM_CASE(7)
    ADM_CASE(8)
#undef ADM_CASE
    default: return false;
  }
}

template <int D, bool BF>
void launch_attend_t(dim3 grid, hipStream_t s, const void* q, const void* k, const void* v,
                     const int32_t* idx, int Hq, int Hkv, int64_t cap, int budget, float qscale,
                     float* part, uint32_t* ctr, void* out, const PageArgs* pa) {
  if (pa != nullptr)
    k_attend<D, BF, true><<<grid, kAttendThreads, 0, s>>>(q, k, v, idx, Hq, Hkv, cap, budget,
                                                          qscale, part, ctr, out, *pa);
  else
    k_attend<D, BF, false><<<grid, kAttendThreads, 0, s>>>(q, k, v, idx, Hq, Hkv, cap, budget,
                                                           qscale, part, ctr, out, PageArgs{});
}

// pa: the page table of paged K/V pools, or null for [B][Hkv][cap][D] caches
void launch_attend(int D, bool bf, dim3 grid, hipStream_t s, const void* q, const void* k,
                   const void* v, const int32_t* idx, int Hq, int Hkv, int64_t cap, int budget,
                   float qscale, float* part, uint32_t* ctr, void* out,
                   const PageArgs* pa = nullptr) {
  with_dim(D, [&](auto dc) {
    constexpr int DD = decltype(dc)::value;
    if (bf)
      launch_attend_t<DD, true>(grid, s, q, k, v, idx, Hq, Hkv, cap, budget, qscale, part, ctr,
                                out, pa);
    else
      launch_attend_t<DD, false>(grid, s, q, k, v, idx, Hq, Hkv, cap, budget, qscale, part, ctr,
                                 out, pa);
  });
}

// Score scale in the log2 domain: s2 = (q . k) * scale * log2(e).
float attend_qscale(float scale, int D) {
  const float sc = (scale == 0.0f) ? 1.0f / sqrtf((float)D) : scale;
  return sc * 1.4426950408889634f;
}

}  // namespace

extern "C" {

int adamas_version(void) { return ADAMAS_VERSION; }

const char* adamas_status_string(int status) {
  switch (status) {
    case ADAMAS_OK: return "ok";
    case ADAMAS_ERR_INVALID: return "invalid argument (null/misaligned pointer, size or range)";
    case ADAMAS_ERR_UNSUPPORTED: return "unsupported (head_dim, dtype or a size limit)";
    case ADAMAS_ERR_WORKSPACE: return "workspace missing or too small";
    case ADAMAS_ERR_DEVICE: return "device launch error";
    default: return "unknown status";
  }
}

size_t adamas_workspace_bytes(int op, int B, int Hq, int Hkv, int64_t n_ctx, int budget,
                              int head_dim) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_ctx < 1 || budget < 1 ||
      budget > kMaxBudget || !valid_dim(head_dim))
    return 0;
  if (op == ADAMAS_OP_DECODE_STEP && Hq / Hkv > kMaxG) return 0;
  const int64_t rows = (int64_t)B * Hq;
  switch (op) {
    case ADAMAS_OP_SELECT_TOPK:
      return round_up(plan_select(rows, n_ctx, budget, head_dim, ADAMAS_WS_CTRL_BYTES).end,
                      256);
    case ADAMAS_OP_SPARSE_ATTEND:
      return round_up(plan_attend(rows, budget, head_dim, ADAMAS_WS_CTRL_BYTES).end, 256);
    case ADAMAS_OP_DECODE_STEP:
      return std::max(
          plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim).total,
          plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, kSizingCapacity).total);
    default: return 0;
  }
}

int adamas_encode_keys(const void* x, int dtype, int batch, int heads, int64_t n, int head_dim,
                       uint8_t* codes, int64_t cap, int64_t pos, void* x_copy_dst,
                       hipStream_t stream) {
  if (!valid_dtype(dtype) || !valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  if (batch < 1 || heads < 1 || n < 0 || pos < 0 || cap < 1 || pos + n > cap)
    return ADAMAS_ERR_INVALID;
  if (!aligned16(x) || !aligned16(codes)) return ADAMAS_ERR_INVALID;
  if (x_copy_dst != nullptr && !aligned16(x_copy_dst)) return ADAMAS_ERR_INVALID;
  if (n == 0) return ADAMAS_OK;
  const int64_t nvec = (int64_t)batch * heads * n;
  const int64_t slots = kEncodeThreads / 16;  // one vector per 16-lane slot
  const int64_t blocks64 = (nvec + slots - 1) / slots;
  const unsigned blocks = (unsigned)(blocks64 < 8192 ? blocks64 : 8192);
  const int bf = dtype == ADAMAS_BF16;
  with_dim(head_dim, [&](auto dc) {
    k_encode<decltype(dc)::value><<<blocks, kEncodeThreads, 0, stream>>>(
        x, bf, n, nvec, codes, cap, pos, x_copy_dst, rotation_on());
  });
  return launch_status();
}

int adamas_score(const uint8_t* q_codes, const uint8_t* k_codes, int B, int Hq, int Hkv,
                 int head_dim, int64_t cap, int64_t n_ctx, uint16_t* dist, hipStream_t stream) {
  if (!valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_ctx < 0 || cap < 1 || n_ctx > cap)
    return ADAMAS_ERR_INVALID;
  if (Hq / Hkv > kMaxG || Hkv > 65535 || B > 65535 || n_ctx > INT32_MAX)
    return ADAMAS_ERR_UNSUPPORTED;
  if (!aligned16(q_codes) || !aligned16(k_codes) || !aligned16(dist)) return ADAMAS_ERR_INVALID;
  if (n_ctx == 0) return ADAMAS_OK;
  const int chunk = 4096;
  const dim3 grid((unsigned)((n_ctx + chunk - 1) / chunk), (unsigned)Hkv, (unsigned)B);
  const int G = Hq / Hkv;
  bool ok = false;
  with_dim(head_dim, [&](auto dc) {
    ok = dispatch_score<decltype(dc)::value>(G, grid, stream, q_codes, k_codes, Hq, Hkv, cap,
                                             n_ctx, chunk, dist);
  });
  if (!ok) return ADAMAS_ERR_UNSUPPORTED;
  return launch_status();
}

int adamas_select_topk_keep(const uint16_t* dist, int B, int Hq, int64_t n_ctx, int head_dim,
                            int budget, int n_sink, int n_recent, int32_t* idx, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (!valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || n_ctx < 1 || budget < 1 || n_sink < 0 || n_recent < 0)
    return ADAMAS_ERR_INVALID;
  if (budget > kMaxBudget || n_ctx > INT32_MAX || (int64_t)B * Hq > kMaxGroups || Hq > 65535 ||
      B > 65535)
    return ADAMAS_ERR_UNSUPPORTED;
  if (!aligned16(dist) || !aligned16(idx)) return ADAMAS_ERR_INVALID;
  if (ws == nullptr || !aligned16(ws)) return ADAMAS_ERR_WORKSPACE;
  const int64_t rows = (int64_t)B * Hq;
  const SelectPlan p = plan_select(rows, n_ctx, budget, head_dim, ADAMAS_WS_CTRL_BYTES);
  if (ws_bytes < round_up(p.end, 256)) return ADAMAS_ERR_WORKSPACE;
  uint8_t* w = static_cast<uint8_t*>(ws);
  const dim3 grid((unsigned)p.n_chunks, (unsigned)Hq, (unsigned)B);
  uint32_t* cand = reinterpret_cast<uint32_t*>(w + p.cand_off);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(w + kCtrlSelect);
  with_dim(head_dim, [&](auto dc) {
    k_select<decltype(dc)::value><<<grid, kSelectThreads, p.lds, stream>>>(
        dist, Hq, n_ctx, p.chunk, p.n_chunks, budget, p.kpad_log2, p.mcap, cand, ctr, idx,
        n_sink, n_recent);
  });
  return launch_status();
}

int adamas_select_topk(const uint16_t* dist, int B, int Hq, int64_t n_ctx, int head_dim,
                       int budget, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  return adamas_select_topk_keep(dist, B, Hq, n_ctx, head_dim, budget, 0, 0, idx, ws, ws_bytes,
                                 stream);
}

int adamas_sparse_attend(const void* q, const void* k, const void* v, int dtype,
                         const int32_t* idx, int B, int Hq, int Hkv, int head_dim, int64_t cap,
                         int budget, float scale, void* out, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!valid_dtype(dtype) || !valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || cap < 1 || budget < 1 || !isfinite(scale))
    return ADAMAS_ERR_INVALID;
  if (budget > kMaxBudget || (int64_t)B * Hq > kMaxGroups || Hq > 65535 || B > 65535)
    return ADAMAS_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(idx) || !aligned16(out))
    return ADAMAS_ERR_INVALID;
  if (ws == nullptr || !aligned16(ws)) return ADAMAS_ERR_WORKSPACE;
  const int64_t rows = (int64_t)B * Hq;
  const AttendPlan p = plan_attend(rows, budget, head_dim, ADAMAS_WS_CTRL_BYTES);
  if (ws_bytes < round_up(p.end, 256)) return ADAMAS_ERR_WORKSPACE;
  uint8_t* w = static_cast<uint8_t*>(ws);
  const dim3 grid((unsigned)p.splits, (unsigned)Hq, (unsigned)B);
  launch_attend(head_dim, dtype == ADAMAS_BF16, grid, stream, q, k, v, idx, Hq, Hkv, cap, budget,
                attend_qscale(scale, head_dim), reinterpret_cast<float*>(w + p.part_off),
                reinterpret_cast<uint32_t*>(w + kCtrlAttend), out);
  return launch_status();
}

}  // extern "C"

namespace {

// The last-arrival schedule: the fused decode kernel, then (when the
// selection is too large to attend inside it) the attention kernel over the
// selected rows.
int launch_last_arrival(const DecodePlan& p, const DecodeArgs& a, int B, int head_dim, bool bf,
                        uint8_t* w, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid((unsigned)p.sel.n_chunks, (unsigned)a.Hkv, (unsigned)B);
  bool ok = false;
  with_dim(head_dim, [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    ok = bf ? dispatch_decode<D, true>(G, p, grid, stream, a)
            : dispatch_decode<D, false>(G, p, grid, stream, a);
  });
  if (!ok) return ADAMAS_ERR_UNSUPPORTED;
  bool attended = false;
  if (a.chist != nullptr) {
    const int bsel = (int)(a.n_ctx < a.budget ? a.n_ctx : a.budget);
    const dim3 gsel((unsigned)p.segs, (unsigned)((int64_t)B * a.Hq));
    // attention inside the selection launch when a segment's rows fit in LDS
    const bool fa = bsel <= kSplitFuseRows;
    const SplitAttend sa{fa ? a.q : nullptr, a.k, a.v, a.Hq, a.Hkv, a.cap, a.qscale,
                         reinterpret_cast<float*>(w + p.spart_off),
                         reinterpret_cast<uint32_t*>(w + kCtrlAttend), a.out};
    const size_t lds = split_select_lds(head_dim, p.ncp, fa);
    with_dim(head_dim, [&](auto dc) {
      constexpr int D = decltype(dc)::value;
      if (bf) {
        allow_lds(&k_split_select<D, true>, lds);
        k_split_select<D, true><<<gsel, kSplitThreads, lds, stream>>>(
            a.cand, a.chist, p.sel.n_chunks, p.ncp, p.seg_chunks, p.sel.kpad_log2, p.sel.chunk,
            3 * D + 2, bsel, a.budget, a.idx, sa);
      } else {
        allow_lds(&k_split_select<D, false>, lds);
        k_split_select<D, false><<<gsel, kSplitThreads, lds, stream>>>(
            a.cand, a.chist, p.sel.n_chunks, p.ncp, p.seg_chunks, p.sel.kpad_log2, p.sel.chunk,
            3 * D + 2, bsel, a.budget, a.idx, sa);
      }
    });
    attended = fa;
  }
  if ((!p.fuse || a.chist != nullptr) && !attended) {
    const dim3 gatt((unsigned)p.att.splits, (unsigned)a.Hq, (unsigned)B);
    const PageArgs pa{a.rg.pages, a.rg.max_pages, a.rg.page_log2, a.rg.n_pages};
    launch_attend(head_dim, bf, gatt, stream, a.q, a.k, a.v, a.idx, a.Hq, a.Hkv, a.cap, a.budget,
                  a.qscale, reinterpret_cast<float*>(w + p.att.part_off),
                  reinterpret_cast<uint32_t*>(w + kCtrlAttend), a.out,
                  a.rg.pages != nullptr ? &pa : nullptr);
  }
  return launch_status();
}

}  // namespace

extern "C" {

int adamas_decode_step_keep(const void* q, const void* k, const void* v, const uint8_t* k_codes,
                            int dtype, int B, int Hq, int Hkv, int head_dim, int64_t cap,
                            int64_t n_ctx, int budget, int n_sink, int n_recent, float scale,
                            void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (!valid_dtype(dtype) || !valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || cap < 1 || n_ctx < 1 || n_ctx > cap ||
      budget < 1 || !isfinite(scale) || n_sink < 0 || n_recent < 0)
    return ADAMAS_ERR_INVALID;
  if (budget > kMaxBudget || n_ctx > INT32_MAX || Hq / Hkv > kMaxG ||
      (int64_t)B * Hq > kMaxGroups || Hq > 65535 || B > 65535)
    return ADAMAS_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_codes) || !aligned16(out))
    return ADAMAS_ERR_INVALID;
  if (idx_out != nullptr && !aligned16(idx_out)) return ADAMAS_ERR_INVALID;
  if (ws == nullptr || !aligned16(ws)) return ADAMAS_ERR_WORKSPACE;
  // the documented requirement covers both schedules, whichever runs
  if (ws_bytes < adamas_workspace_bytes(ADAMAS_OP_DECODE_STEP, B, Hq, Hkv, n_ctx, budget,
                                        head_dim))
    return ADAMAS_ERR_WORKSPACE;
  const int mode = g_decode_mode.load(std::memory_order_relaxed);
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int G = Hq / Hkv;
  const bool bf = dtype == ADAMAS_BF16;
  const DecodePlan p = plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim);
  const bool many = many_candidates(p);
  // AUTO takes group waits where the last-arrival schedule could not fuse
  // the attention (it would need a second launch) or would select from too
  // many candidates in one workgroup; failing that, the separate selection
  // for the latter
  if (mode == ADAMAS_DECODE_GROUP_WAIT || (mode == ADAMAS_DECODE_AUTO && (!p.fuse || many))) {
    const GroupPlan gp = plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, device_capacity());
    if (gp.ok) {
      if (ws_bytes < gp.total) return ADAMAS_ERR_WORKSPACE;
      DecodeArgs a{q, k, v, k_codes, Hq, Hkv, cap, n_ctx, budget, attend_qscale(scale, head_dim),
                   nullptr, nullptr, idx_out, out, n_sink, n_recent, {}};
      const dim3 grid((unsigned)gp.n_chunks, (unsigned)Hkv, (unsigned)B);
      bool ok = false;
      with_dim(head_dim, [&](auto dc) {
        constexpr int D = decltype(dc)::value;
        ok = bf ? dispatch_decode_gs<D, true>(G, gp, grid, stream, a, w)
                : dispatch_decode_gs<D, false>(G, gp, grid, stream, a, w);
      });
      if (!ok) return ADAMAS_ERR_UNSUPPORTED;
      return launch_status();
    }
    if (mode == ADAMAS_DECODE_GROUP_WAIT) return ADAMAS_ERR_UNSUPPORTED;
  }
  if (mode == ADAMAS_DECODE_SPLIT && !p.split_ok) return ADAMAS_ERR_UNSUPPORTED;
  const bool split = mode == ADAMAS_DECODE_SPLIT || (mode == ADAMAS_DECODE_AUTO && many && p.split_ok);
  if (ws_bytes < p.total) return ADAMAS_ERR_WORKSPACE;
  int32_t* idx = idx_out != nullptr       ? idx_out
                 : (p.fuse && !split) ? nullptr
                                      : reinterpret_cast<int32_t*>(w + p.idx_off);
  DecodeArgs a{q, k, v, k_codes, Hq, Hkv, cap, n_ctx, budget, attend_qscale(scale, head_dim),
               reinterpret_cast<uint32_t*>(w + p.sel.cand_off),
               reinterpret_cast<uint32_t*>(w + kCtrlSelect), idx, out, n_sink, n_recent, {}};
  if (split) {
    a.chist = reinterpret_cast<uint16_t*>(w + p.chist_off);
    a.ncp = p.ncp;
  }
  return launch_last_arrival(p, a, B, head_dim, bf, w, stream);
}

int adamas_decode_step(const void* q, const void* k, const void* v, const uint8_t* k_codes,
                       int dtype, int B, int Hq, int Hkv, int head_dim, int64_t cap,
                       int64_t n_ctx, int budget, float scale, void* out, int32_t* idx_out,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return adamas_decode_step_keep(q, k, v, k_codes, dtype, B, Hq, Hkv, head_dim, cap, n_ctx,
                                 budget, 0, 0, scale, out, idx_out, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// adamas_decode_append_step and adamas_decode_paged_step: validation shared
// by both, then one last-arrival launch (plus the attention launch when the
// selection is large).  pages == nullptr: contiguous [B][Hkv][cap] caches.
int ragged_step(const void* q, const void* k_new, const void* v_new, void* k, void* v,
                uint8_t* k_codes, const int32_t* lens, int dtype, int B, int Hq, int Hkv,
                int head_dim, int64_t cap, int64_t max_len, int budget, int n_sink, int n_recent,
                float scale, void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                hipStream_t stream, const int32_t* pages, int max_pages, int page_log2,
                int n_pages) {
  if (!valid_dtype(dtype) || !valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  const bool app = k_new != nullptr;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || cap < 1 || max_len < 1 || max_len > cap ||
      budget < 1 || !isfinite(scale) || n_sink < 0 || n_recent < 0 || (v_new != nullptr) != app)
    return ADAMAS_ERR_INVALID;
  if (budget > kMaxBudget || max_len > INT32_MAX || Hq / Hkv > kMaxG ||
      (int64_t)B * Hq > kMaxGroups || Hq > 65535 || B > 65535)
    return ADAMAS_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_codes) ||
      !aligned16(out) || lens == nullptr || reinterpret_cast<uintptr_t>(lens) % 4 != 0)
    return ADAMAS_ERR_INVALID;
  if (app && (!aligned16(k_new) || !aligned16(v_new))) return ADAMAS_ERR_INVALID;
  if (idx_out != nullptr && !aligned16(idx_out)) return ADAMAS_ERR_INVALID;
  if (ws == nullptr || !aligned16(ws)) return ADAMAS_ERR_WORKSPACE;
  if (ws_bytes < adamas_workspace_bytes(ADAMAS_OP_DECODE_STEP, B, Hq, Hkv, max_len, budget,
                                        head_dim))
    return ADAMAS_ERR_WORKSPACE;
  uint8_t* w = static_cast<uint8_t*>(ws);
  DecodePlan p = plan_decode(B, Hq, Hkv, max_len, budget, head_dim);
  if (ws_bytes < p.total) return ADAMAS_ERR_WORKSPACE;
  // paged with fused attention: the final workgroup keeps the page table row
  // in LDS after the candidate tile, when it is short and fits
  int pt_lds = 0;
  if (pages != nullptr && p.fuse && max_pages <= kDecodeThreads) {
    const size_t need = (size_t)kTmpWords * 4 +
                        decode_lds_final(head_dim, (int)std::min<int64_t>(budget, max_len),
                                         p.sel.mcap) +
                        (size_t)max_pages * 4;
    if (need <= kLdsDecodeLimit) {
      p.sel.lds = std::max(p.sel.lds, need);
      pt_lds = 1;
    }
  }
  int32_t* idx = idx_out != nullptr ? idx_out
                 : p.fuse       ? nullptr
                                : reinterpret_cast<int32_t*>(w + p.idx_off);
  DecodeArgs a{q, k, v, k_codes, Hq, Hkv, cap, max_len, budget, attend_qscale(scale, head_dim),
               reinterpret_cast<uint32_t*>(w + p.sel.cand_off),
               reinterpret_cast<uint32_t*>(w + kCtrlSelect), idx, out, n_sink, n_recent,
               RaggedArgs{lens, k_new, v_new, k, v, k_codes, pages, max_pages, page_log2,
                          n_pages, pt_lds}};
  return launch_last_arrival(p, a, B, head_dim, dtype == ADAMAS_BF16, w, stream);
}

}  // namespace

extern "C" {

int adamas_decode_append_step(const void* q, const void* k_new, const void* v_new, void* k,
                              void* v, uint8_t* k_codes, const int32_t* lens, int dtype, int B,
                              int Hq, int Hkv, int head_dim, int64_t cap, int64_t max_len,
                              int budget, int n_sink, int n_recent, float scale, void* out,
                              int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return ragged_step(q, k_new, v_new, k, v, k_codes, lens, dtype, B, Hq, Hkv, head_dim, cap,
                     max_len, budget, n_sink, n_recent, scale, out, idx_out, ws, ws_bytes, stream,
                     nullptr, 0, 0, 0);
}

int adamas_decode_paged_step(const void* q, const void* k_new, const void* v_new, void* k_pool,
                             void* v_pool, uint8_t* code_pool, const int32_t* page_table,
                             const int32_t* lens, int dtype, int B, int Hq, int Hkv, int head_dim,
                             int page_size, int n_pages, int max_pages, int64_t max_len,
                             int budget, int n_sink, int n_recent, float scale, void* out,
                             int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int page_log2 = 0;
  while (page_log2 < 30 && (1 << page_log2) < page_size) ++page_log2;
  if (page_size < kMinPageTokens || page_size > kMaxPageTokens || (1 << page_log2) != page_size)
    return ADAMAS_ERR_UNSUPPORTED;
  if (n_pages < 1 || max_pages < 1 || page_table == nullptr ||
      reinterpret_cast<uintptr_t>(page_table) % 4 != 0)
    return ADAMAS_ERR_INVALID;
  return ragged_step(q, k_new, v_new, k_pool, v_pool, code_pool, lens, dtype, B, Hq, Hkv,
                     head_dim, (int64_t)max_pages * page_size, max_len, budget, n_sink, n_recent,
                     scale, out, idx_out, ws, ws_bytes, stream, page_table, max_pages, page_log2,
                     n_pages);
}

int adamas_set_rotation(int on) {
  if (on != 0 && on != 1 && on != 2) return ADAMAS_ERR_INVALID;
  g_rotation.store(on, std::memory_order_relaxed);
  return ADAMAS_OK;
}

int adamas_set_decode_mode(int mode) {
  if (mode != ADAMAS_DECODE_AUTO && mode != ADAMAS_DECODE_LAST_ARRIVAL &&
      mode != ADAMAS_DECODE_GROUP_WAIT && mode != ADAMAS_DECODE_SPLIT)
    return ADAMAS_ERR_INVALID;
  g_decode_mode.store(mode, std::memory_order_relaxed);
  return ADAMAS_OK;
}

int adamas_decode_path(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int head_dim) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_ctx < 1 || budget < 1 ||
      budget > kMaxBudget || !valid_dim(head_dim) || Hq / Hkv > kMaxG)
    return -ADAMAS_ERR_INVALID;
  const int mode = g_decode_mode.load(std::memory_order_relaxed);
  const DecodePlan p = plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim);
  const bool many = many_candidates(p);
  if (mode == ADAMAS_DECODE_LAST_ARRIVAL) return ADAMAS_DECODE_LAST_ARRIVAL;
  if (mode == ADAMAS_DECODE_SPLIT)
    return p.split_ok ? ADAMAS_DECODE_SPLIT : -ADAMAS_ERR_UNSUPPORTED;
  if (mode == ADAMAS_DECODE_AUTO && p.fuse && !many) return ADAMAS_DECODE_LAST_ARRIVAL;
  const int64_t capacity = device_capacity();
  if (capacity <= 0) return -ADAMAS_ERR_DEVICE;
  if (plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, capacity).ok)
    return ADAMAS_DECODE_GROUP_WAIT;
  if (mode == ADAMAS_DECODE_GROUP_WAIT) return -ADAMAS_ERR_UNSUPPORTED;
  return many && p.split_ok ? ADAMAS_DECODE_SPLIT : ADAMAS_DECODE_LAST_ARRIVAL;
}

size_t adamas_stream_read_blocks(size_t bytes) {
  const size_t units = bytes / 16;
  const size_t per = (size_t)kStreamThreads * kDecodeScanDepth;
  const size_t want = (units + per - 1) / per;
  return want < kStreamBlocks ? want : kStreamBlocks;
}

int adamas_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!aligned16(src) || sink == nullptr || bytes == 0 || bytes % 16 != 0)
    return ADAMAS_ERR_INVALID;
  const int64_t units = (int64_t)(bytes / 16);
  const int64_t blocks = (int64_t)adamas_stream_read_blocks(bytes);
  const int64_t per_block = (units + blocks - 1) / blocks;
  k_stream_read<<<(unsigned)blocks, kStreamThreads, 0, stream>>>(
      static_cast<const uint4*>(src), units, per_block, sink);
  return launch_status();
}

}  // extern "C"
