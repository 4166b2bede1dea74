// adamas.hip -- C ABI of the MI355X ADAMAS decode path (declared in
// include/adamas.h): host-side argument checks, workspace layout and kernel
// launches.  Citations refer to the ADAMAS article
// (www.lnwmold.com/news/826806) by its numbered sections.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "adamas.h"
#include "plan.hpp"

namespace {

using namespace adm;
using namespace adm_host;

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
// per-head-group bucketing alphas (adamas_set_bucket_alpha); n == 0: 0.5
std::mutex g_alpha_mu;
int g_alpha_n = 0;
float g_alpha[kMaxAlphaGroups] = {};
// the encoding rule a launch takes (by value, so a launch keeps the table it
// was made with)
EncodeRule encode_rule() {
  EncodeRule r{rotation_on(), 0, {}};
  std::lock_guard<std::mutex> lk(g_alpha_mu);
  r.n_alpha = g_alpha_n;
  for (int i = 0; i < g_alpha_n; ++i) r.alpha[i] = g_alpha[i];
  return r;
}
std::atomic<uint32_t> g_wait_polls{kDefaultWaitPolls};
std::atomic<uint64_t*> g_stamps{nullptr};  // phase stamps (measurement build)
uint64_t* stamps_ptr() { return g_stamps.load(std::memory_order_relaxed); }

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
                                                          qscale, part, ctr, out, *pa,
                                                          stamps_ptr());
  else
    k_attend<D, BF, false><<<grid, kAttendThreads, 0, s>>>(q, k, v, idx, Hq, Hkv, cap, budget,
                                                           qscale, part, ctr, out, PageArgs{},
                                                           stamps_ptr());
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
  // the limits every entry point enforces (and which keep the plans' sizes
  // far from overflowing)
  if (n_ctx > INT32_MAX || (int64_t)B * Hq > kMaxGroups || Hq > 65535 || B > 65535) return 0;
  if (op == ADAMAS_OP_DECODE_STEP && Hq / Hkv > kMaxG) return 0;
  const int64_t rows = (int64_t)B * Hq;
  switch (op) {
    case ADAMAS_OP_SELECT_TOPK:
      return round_up(plan_select(rows, n_ctx, budget, head_dim, ADAMAS_WS_CTRL_BYTES).end,
                      256);
    case ADAMAS_OP_SPARSE_ATTEND:
      return round_up(plan_attend(rows, budget, head_dim, ADAMAS_WS_CTRL_BYTES).end, 256);
    case ADAMAS_OP_DECODE_STEP:
      // every schedule and key width a decode step of this shape may take
      return std::max(
          {plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim, true).total,
           plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim, false).total,
           plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim, false, false).total,
           plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, kSizingCapacity, true).total,
           plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, kComputeUnits, true).total});
    default: return 0;
  }
}

int adamas_encode_keys(const void* x, int dtype, int batch, int heads, int64_t n, int head_dim,
                       uint8_t* codes, int64_t cap, int64_t pos, void* x_copy_dst,
                       hipStream_t stream) {
  if (!valid_dtype(dtype) || !valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  if (batch < 1 || heads < 1 || n < 0 || pos < 0 || cap < 1 || pos > cap || n > cap - pos)
    return ADAMAS_ERR_INVALID;
  // x and the code cache must be addressable: batch * heads * cap rows of up
  // to 256 elements (the products below then cannot overflow)
  if (cap > (INT64_MAX / 1024) / ((int64_t)batch * heads)) return ADAMAS_ERR_INVALID;
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
        x, bf, n, nvec, codes, cap, pos, x_copy_dst, heads, encode_rule());
  });
  return launch_status();
}

int adamas_encode_keys_paged(const void* x, int dtype, int batch, int heads, int64_t n,
                             int head_dim, uint8_t* code_pool, void* x_pool,
                             const int32_t* page_table, int page_size, int n_pages,
                             int max_pages, int64_t pos, hipStream_t stream) {
  if (!valid_dtype(dtype) || !valid_dim(head_dim)) return ADAMAS_ERR_UNSUPPORTED;
  if (page_size < 1024 || page_size > 16384 || (page_size & (page_size - 1)) != 0)
    return ADAMAS_ERR_UNSUPPORTED;
  if (batch < 1 || heads < 1 || n < 0 || pos < 0 || n_pages < 1 || max_pages < 1)
    return ADAMAS_ERR_INVALID;
  const int64_t logical = (int64_t)max_pages * page_size;
  if (pos > logical || n > logical - pos) return ADAMAS_ERR_INVALID;
  // pool rows n_pages * heads * page_size of up to 256 elements must be addressable
  if ((int64_t)n_pages * heads > (INT64_MAX / 1024) / page_size) return ADAMAS_ERR_INVALID;
  if ((int64_t)batch * heads > (INT64_MAX / 1024) / (n > 0 ? n : 1)) return ADAMAS_ERR_INVALID;
  if (!aligned16(x) || !aligned16(code_pool) || page_table == nullptr ||
      (reinterpret_cast<uintptr_t>(page_table) & 3) != 0)
    return ADAMAS_ERR_INVALID;
  if (x_pool != nullptr && !aligned16(x_pool)) return ADAMAS_ERR_INVALID;
  if (n == 0) return ADAMAS_OK;
  const int64_t nvec = (int64_t)batch * heads * n;
  const int64_t slots = kEncodeThreads / 16;
  const int64_t blocks64 = (nvec + slots - 1) / slots;
  const unsigned blocks = (unsigned)(blocks64 < 8192 ? blocks64 : 8192);
  int log2 = 0;
  while ((1 << log2) < page_size) ++log2;
  const EncodePages pg{page_table, max_pages, log2, n_pages};
  with_dim(head_dim, [&](auto dc) {
    k_encode<decltype(dc)::value, true><<<blocks, kEncodeThreads, 0, stream>>>(
        x, dtype == ADAMAS_BF16, n, nvec, code_pool, 0, pos, x_pool, heads, encode_rule(), pg);
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
  // 32768-token chunks are compacted a half at a time only by the two-per-CU build
  if (p.big && !decode_two_per_cu(p, G, (int64_t)p.sel.n_chunks * a.Hkv * B))
    return ADAMAS_ERR_UNSUPPORTED;
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
                         reinterpret_cast<uint32_t*>(w + kCtrlAttend), a.out, a.stamps};
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

}  // extern "C"

namespace {

// Argument checks of a decode step (everything but the workspace).
int check_decode_args(const void* q, const void* k, const void* v, const uint8_t* k_codes,
                      int dtype, int B, int Hq, int Hkv, int head_dim, int64_t cap,
                      int64_t n_ctx, int budget, int n_sink, int n_recent, float scale,
                      const void* out, const int32_t* idx_out) {
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
  return ADAMAS_OK;
}

// no_group_wait: never the group-wait schedule (the workspace then only has
// to hold the last-arrival or split layout, DecodePlan::total).
int decode_step_impl(const void* q, const void* k, const void* v, const uint8_t* k_codes,
                     int dtype, int B, int Hq, int Hkv, int head_dim,
                     int64_t cap, int64_t n_ctx, int budget, int n_sink, int n_recent,
                     float scale, void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                     hipStream_t stream, bool no_group_wait = false) {
  const int chk = check_decode_args(q, k, v, k_codes, dtype, B, Hq, Hkv, head_dim, cap, n_ctx,
                                    budget, n_sink, n_recent, scale, out, idx_out);
  if (chk != ADAMAS_OK) return chk;
  if (ws == nullptr || !aligned16(ws)) return ADAMAS_ERR_WORKSPACE;
  // the documented requirement covers both schedules, whichever runs
  if (!no_group_wait && ws_bytes < adamas_workspace_bytes(ADAMAS_OP_DECODE_STEP, B, Hq, Hkv,
                                                          n_ctx, budget, head_dim))
    return ADAMAS_ERR_WORKSPACE;
  int mode = g_decode_mode.load(std::memory_order_relaxed);
  if (no_group_wait && mode == ADAMAS_DECODE_GROUP_WAIT) mode = ADAMAS_DECODE_AUTO;
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int G = Hq / Hkv;
  const bool bf = dtype == ADAMAS_BF16;
  const DecodePlan p = plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim);
  const bool many = many_candidates(p);
  // AUTO takes group waits where the last-arrival schedule could not fuse
  // the attention (it would need a second launch) or would select from too
  // many candidates in one workgroup; failing that, the separate selection
  // for the latter
  if (!no_group_wait &&
      (mode == ADAMAS_DECODE_GROUP_WAIT || (mode == ADAMAS_DECODE_AUTO && (!p.fuse || many)))) {
    const GroupPlan gp = plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, device_capacity(),
                                        mode == ADAMAS_DECODE_GROUP_WAIT);
    if (gp.ok) {
      if (ws_bytes < gp.total) return ADAMAS_ERR_WORKSPACE;
      DecodeArgs a{q, k, v, k_codes, Hq, Hkv, cap, n_ctx, budget, attend_qscale(scale, head_dim),
                   nullptr, nullptr, idx_out, out, n_sink, n_recent, {}};
      a.rule = encode_rule();
      a.wait_polls = g_wait_polls.load(std::memory_order_relaxed);
      a.stamps = stamps_ptr();
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
  a.rule = encode_rule();
  a.stamps = stamps_ptr();
  if (split) {
    a.chist = reinterpret_cast<uint16_t*>(w + p.chist_off);
    a.ncp = p.ncp;
  }
  return launch_last_arrival(p, a, B, head_dim, bf, w, stream);
}

}  // namespace

extern "C" {

int adamas_decode_step_keep(const void* q, const void* k, const void* v, const uint8_t* k_codes,
                            int dtype, int B, int Hq, int Hkv, int head_dim, int64_t cap,
                            int64_t n_ctx, int budget, int n_sink, int n_recent, float scale,
                            void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return decode_step_impl(q, k, v, k_codes, dtype, B, Hq, Hkv, head_dim, cap, n_ctx, budget,
                          n_sink, n_recent, scale, out, idx_out, ws, ws_bytes, stream);
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
  DecodePlan p = plan_decode(B, Hq, Hkv, max_len, budget, head_dim, false, pages == nullptr);
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
  a.rule = encode_rule();
  a.stamps = stamps_ptr();
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

int adamas_set_bucket_alpha(const float* alpha, int n) {
  static_assert(ADAMAS_MAX_ALPHA_GROUPS == kMaxAlphaGroups, "alpha table size");
  if (n < 0 || n > kMaxAlphaGroups || (n > 0 && alpha == nullptr)) return ADAMAS_ERR_INVALID;
  for (int i = 0; i < n; ++i)
    if (!(alpha[i] >= 0.0f) || !std::isfinite(alpha[i])) return ADAMAS_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_alpha_mu);
  for (int i = 0; i < n; ++i) g_alpha[i] = alpha[i];
  g_alpha_n = n;
  return ADAMAS_OK;
}

int adamas_bucket_alpha(float* alpha_out, int cap) {
  std::lock_guard<std::mutex> lk(g_alpha_mu);
  if (alpha_out != nullptr)
    for (int i = 0; i < g_alpha_n && i < cap; ++i) alpha_out[i] = g_alpha[i];
  return g_alpha_n;
}

int adamas_set_wait_polls(uint32_t polls) {
  g_wait_polls.store(polls, std::memory_order_relaxed);
  return ADAMAS_OK;
}

uint32_t adamas_wait_polls(void) { return g_wait_polls.load(std::memory_order_relaxed); }

int adamas_phase_stamps_built(void) { return kPhases ? 1 : 0; }

size_t adamas_phase_buffer_bytes(void) {
  return (size_t)kPhaseRegions * kPhaseMaxWorkgroups * kPhaseSlots * sizeof(uint64_t);
}

int adamas_set_phase_buffer(void* buf, size_t bytes) {
  if (!kPhases) return ADAMAS_ERR_UNSUPPORTED;
  if (buf != nullptr && (!aligned16(buf) || bytes < adamas_phase_buffer_bytes()))
    return ADAMAS_ERR_INVALID;
  g_stamps.store(static_cast<uint64_t*>(buf), std::memory_order_relaxed);
  return ADAMAS_OK;
}

int adamas_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

int adamas_set_decode_mode(int mode) {
  if (mode != ADAMAS_DECODE_AUTO && mode != ADAMAS_DECODE_LAST_ARRIVAL &&
      mode != ADAMAS_DECODE_GROUP_WAIT && mode != ADAMAS_DECODE_SPLIT)
    return ADAMAS_ERR_INVALID;
  g_decode_mode.store(mode, std::memory_order_relaxed);
  return ADAMAS_OK;
}

int adamas_decode_key_bytes(int B, int Hq, int Hkv, int64_t n_ctx, int budget, int head_dim) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_ctx < 1 || budget < 1 ||
      budget > kMaxBudget || !valid_dim(head_dim) || Hq / Hkv > kMaxG)
    return -ADAMAS_ERR_INVALID;
  if (n_ctx > INT32_MAX || (int64_t)B * Hq > kMaxGroups || Hq > 65535 || B > 65535)
    return -ADAMAS_ERR_UNSUPPORTED;
  // the group-wait kernel when the current mode would take it on this device
  const int path = adamas_decode_path(B, Hq, Hkv, n_ctx, budget, head_dim);
  if (path == ADAMAS_DECODE_GROUP_WAIT)
    return plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, device_capacity(),
                          g_decode_mode.load(std::memory_order_relaxed) ==
                              ADAMAS_DECODE_GROUP_WAIT)
                   .u8
               ? 1
               : 2;
  return plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim).u8 ? 1 : 2;
}

int adamas_decode_chunk_tokens(int B, int Hq, int Hkv, int64_t n_ctx, int budget,
                               int head_dim) {
  const int kb = adamas_decode_key_bytes(B, Hq, Hkv, n_ctx, budget, head_dim);
  if (kb < 0) return kb;
  if (adamas_decode_path(B, Hq, Hkv, n_ctx, budget, head_dim) == ADAMAS_DECODE_GROUP_WAIT)
    return plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, device_capacity(),
                          g_decode_mode.load(std::memory_order_relaxed) ==
                              ADAMAS_DECODE_GROUP_WAIT)
        .chunk;
  return plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim).sel.chunk;
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
  if (plan_decode_gs(B, Hq, Hkv, n_ctx, budget, head_dim, capacity,
                     mode == ADAMAS_DECODE_GROUP_WAIT).ok)
    return ADAMAS_DECODE_GROUP_WAIT;
  if (mode == ADAMAS_DECODE_GROUP_WAIT) return -ADAMAS_ERR_UNSUPPORTED;
  return many && p.split_ok ? ADAMAS_DECODE_SPLIT : ADAMAS_DECODE_LAST_ARRIVAL;
}

}  // extern "C"

namespace {

// Scratch of adamas_decode_step_static: one copy per device, resident from
// the library's load on that device until the process ends.  Host code never
// uses this name as an address (in host code it is a stand-in for the
// symbol); static_scratch() resolves the device address once per device.
static __device__ __align__(256) uint8_t scratch[ADAMAS_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

__global__ void k_zero16(uint4* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address, or null on a runtime error.  The
// first call on a device resolves the symbol and enqueues on `stream` a
// small kernel that zeroes the control bytes (the later calls rely on every
// completed call leaving them zero).
uint8_t* static_scratch(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p != nullptr) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
    return nullptr;
  k_zero16<<<16, 256, 0, stream>>>(static_cast<uint4*>(addr), ADAMAS_WS_CTRL_BYTES / 16);
  if (hipGetLastError() != hipSuccess) return nullptr;
  p = static_cast<uint8_t*>(addr);
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int adamas_decode_step_static(const void* q, const void* k, const void* v,
                              const uint8_t* k_codes, int dtype, int B, int Hq, int Hkv,
                              int head_dim, int64_t cap, int64_t n_ctx, int budget, float scale,
                              void* out, int32_t* idx_out, hipStream_t stream) {
  // every check before anything is resolved or enqueued: the arguments, then
  // the shape's scratch against the static buffer
  const int chk = check_decode_args(q, k, v, k_codes, dtype, B, Hq, Hkv, head_dim, cap, n_ctx,
                                    budget, 0, 0, scale, out, idx_out);
  if (chk != ADAMAS_OK) return chk;
  if (plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim).total > ADAMAS_STATIC_SCRATCH_BYTES)
    return ADAMAS_ERR_WORKSPACE;
  uint8_t* w = static_scratch(stream);
  if (w == nullptr) return ADAMAS_ERR_DEVICE;
  return decode_step_impl(q, k, v, k_codes, dtype, B, Hq, Hkv, head_dim, cap, n_ctx, budget, 0,
                          0, scale, out, idx_out, w, ADAMAS_STATIC_SCRATCH_BYTES, stream, true);
}

size_t adamas_static_scratch_need(int B, int Hq, int Hkv, int64_t n_ctx, int budget,
                                  int head_dim) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_ctx < 1 || budget < 1 ||
      budget > kMaxBudget || !valid_dim(head_dim) || Hq / Hkv > kMaxG)
    return 0;
  if (n_ctx > INT32_MAX || (int64_t)B * Hq > kMaxGroups || Hq > 65535 || B > 65535) return 0;
  return plan_decode(B, Hq, Hkv, n_ctx, budget, head_dim).total;
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
