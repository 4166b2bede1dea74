// decode_inst.hip -- launchers of the fused decode kernels (k_decode,
// k_decode_gs) for one head_dim (ADM_INST_D), element type (ADM_INST_BF) and
// set of group sizes (ADM_INST_GSET: 0 -> G = 1, 1 -> G = 2..4,
// 2 -> G = 5..8).  The build compiles this file once per combination, in
// parallel; adamas.hip dispatches to them.
#include "plan.hpp"

#ifndef ADM_INST_D
#error "ADM_INST_D (64, 128 or 256) must be defined"
#endif
#ifndef ADM_INST_BF
#error "ADM_INST_BF (0 or 1) must be defined"
#endif
#ifndef ADM_INST_GSET
#error "ADM_INST_GSET (0, 1 or 2) must be defined"
#endif

namespace adm_host {

template <int D, int G, bool BF, int RAG, bool OCC, bool U8 = false, bool ONE = false>
void launch_decode_k(const DecodePlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  allow_lds(&k_decode<D, G, BF, RAG, OCC, U8, ONE>, p.sel.lds);
  k_decode<D, G, BF, RAG, OCC, U8, ONE><<<grid, kDecodeThreads, p.sel.lds, s>>>(
      a.q, a.k, a.v, a.kc, a.Hq, a.Hkv, a.cap, a.n_ctx, p.sel.chunk, p.sel.n_chunks, a.budget,
      p.sel.kpad_log2, p.sel.mcap, (p.fuse && !a.chist) ? 1 : 0, a.qscale, a.cand, a.ctr, a.idx,
      a.out, a.n_sink, a.n_recent, a.rule, a.rg, RAG ? nullptr : a.chist,
      RAG ? 0 : a.ncp, a.stamps);
}

template <int D, int G, bool BF>
void launch_decode_t(const DecodePlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  // MHA launches of several rounds run two workgroups per compute unit
  // when their LDS allows it
  const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
  const bool occ = decode_two_per_cu(p, G, wgs);  // always so for 32768-token chunks
  const int rag = a.rg.lens == nullptr ? 0 : (a.rg.pages == nullptr ? 1 : 2);
  if constexpr (G >= 2 && D <= 128) {
    if (p.u8 && rag == 0) {
      launch_decode_k<D, G, BF, 0, false, true>(p, grid, s, a);
      return;
    }
  }
  // one chunk per KV head: the variant that selects and attends (or writes
  // the index rows) without a hand-over
  const bool one = rag == 0 && p.sel.n_chunks == 1 && a.chist == nullptr;
  if constexpr (G == 1) {
    if (occ) {
      if (one)
        launch_decode_k<D, G, BF, 0, true, false, true>(p, grid, s, a);
      else if (rag == 2)
        launch_decode_k<D, G, BF, 2, true>(p, grid, s, a);
      else if (rag == 1)
        launch_decode_k<D, G, BF, 1, true>(p, grid, s, a);
      else
        launch_decode_k<D, G, BF, 0, true>(p, grid, s, a);
      return;
    }
  }
  if (one)
    launch_decode_k<D, G, BF, 0, false, false, true>(p, grid, s, a);
  else if (rag == 2)
    launch_decode_k<D, G, BF, 2, false>(p, grid, s, a);
  else if (rag == 1)
    launch_decode_k<D, G, BF, 1, false>(p, grid, s, a);
  else
    launch_decode_k<D, G, BF, 0, false>(p, grid, s, a);
}

template <int D, int G, bool BF, bool U8>
void launch_decode_gs_k(const GroupPlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a,
                        uint8_t* w) {
  allow_lds(&k_decode_gs<D, G, BF, U8>, p.lds);
  k_decode_gs<D, G, BF, U8><<<grid, kDecodeThreads, p.lds, s>>>(
      a.q, a.k, a.v, a.kc, a.Hq, a.Hkv, a.cap, a.n_ctx, p.chunk, p.n_chunks, a.budget, p.cmax,
      a.qscale, reinterpret_cast<uint16_t*>(w + p.hist_off),
      reinterpret_cast<float*>(w + p.part_off), reinterpret_cast<uint32_t*>(w + kCtrlSelect),
      reinterpret_cast<uint32_t*>(w + kCtrlAttend),
      reinterpret_cast<uint32_t*>(w + ADAMAS_WS_STATUS_OFFSET), a.wait_polls, a.idx, a.out,
      a.n_sink, a.n_recent, a.rule, a.stamps);
}

template <int D, int G, bool BF>
void launch_decode_gs_t(const GroupPlan& p, dim3 grid, hipStream_t s, const DecodeArgs& a,
                        uint8_t* w) {
  if constexpr (G >= 2 && D <= 128) {
    if (p.u8) {
      launch_decode_gs_k<D, G, BF, true>(p, grid, s, a, w);
      return;
    }
  }
  launch_decode_gs_k<D, G, BF, false>(p, grid, s, a, w);
}

#define ADM_INST_G(g)                                                                        \
  template void launch_decode_t<ADM_INST_D, g, (ADM_INST_BF != 0)>(                          \
      const DecodePlan&, dim3, hipStream_t, const DecodeArgs&);                              \
  template void launch_decode_gs_t<ADM_INST_D, g, (ADM_INST_BF != 0)>(                       \
      const GroupPlan&, dim3, hipStream_t, const DecodeArgs&, uint8_t*);
#if ADM_INST_GSET == 0
ADM_INST_G(1)
#elif ADM_INST_GSET == 1
ADM_INST_G(2) ADM_INST_G(3) ADM_INST_G(4)
#else
ADM_INST_G(5) ADM_INST_G(6) ADM_INST_G(7) ADM_INST_G(8)
#endif
#undef ADM_INST_G

}  // namespace adm_host
