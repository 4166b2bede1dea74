// kernels.hpp -- the gfx950 kernels of the ADAMAS decode path.
//
// Citations refer to the ADAMAS article (www.lnwmold.com/news/826806) by its
// numbered sections: §2.1 Hadamard rotation, §2.2 bucketing, §2.3 Manhattan
// distance, §3.1 packed code cache, §5.2 token budget, §6 final attention.
#pragma once

#include "device_common.hpp"

namespace adm {

// Selection keys: bin 0 holds the tokens that are always kept (the first
// n_sink and the last n_recent of the context), bin 1 + d the others at
// Manhattan distance d (0 <= d <= 3*D).
constexpr int kNbins(int D) { return 3 * D + 2; }
constexpr int kNbinsPadded(int D) { return (kNbins(D) + 3) & ~3; }
constexpr int kNbinsHist(int D) { return (kNbins(D) + 7) & ~7; }  // u16 bins, 16-byte rows

// Key of token t: 0 if it is always kept, else 1 + its distance.
ADM_DEV uint32_t select_key(int64_t t, uint32_t d, int64_t n_sink, int64_t keep_from) {
  return (t < n_sink || t >= keep_from) ? 0u : d + 1u;
}

// The always-kept tokens of a run [t0, t0 + valid) as run-local bounds: token
// i is kept iff i < lo or i >= hi (0 <= lo, hi <= valid).
struct KeepRange {
  int lo, hi;
  ADM_DEV KeepRange(int64_t t0, int valid, int64_t n_sink, int64_t keep_from) {
    const int64_t a = n_sink - t0, z = keep_from - t0;
    lo = (int)(a < 0 ? 0 : (a > valid ? valid : a));
    hi = (int)(z < 0 ? 0 : (z > valid ? valid : z));
  }
  ADM_DEV uint32_t key(int i, uint32_t d) const { return (i < lo || i >= hi) ? 0u : d + 1u; }
  // no token of [0, n) is always kept: every key there is d + 1
  ADM_DEV bool keeps_none(int n) const { return lo == 0 && hi >= n; }
};
constexpr int kGsMergeTile = 16;  // partials merged per LDS tile (k_decode_gs)

constexpr int kEncodeThreads = 256;
constexpr int kScoreThreads = 256;
constexpr int kSelectThreads = 1024;
constexpr int kDecodeThreads = 1024;  // one workgroup of 16 wavefronts per CU
// Grouped heads stage all G heads' chunk candidates at once when G * kpad
// entries fit this many (chunk_compact_heads); else one head at a time.
constexpr int kFusedStageEntries = 8192;
ADM_HOST_DEV constexpr int stage_heads(int G, int kpad) {
  return (G >= 2 && G * kpad <= kFusedStageEntries) ? G : 1;
}
// 16-byte code loads per thread in flight in the decode scans: 64 KiB per
// workgroup per batch streams faster than 128 or 256 KiB (fewer requests
// queued per CU at the same delivered bandwidth)
constexpr int kDecodeScanDepth = 4;
constexpr int kAttendThreads = 1024;
constexpr int kAttendRowsPerSlot = 4;  // rows a 16-lane slot holds in flight
constexpr int kAttendRowsPerBatch = (kAttendThreads / 16) * kAttendRowsPerSlot;  // 256

// ------------------------------------------------------------------ encode
// §2.1 + §2.2 + §3.1 for keys (or queries): one 16-lane slot per vector
// (kEncodeThreads / 16 vectors per workgroup), grid-stride over the
// batch*heads*n vectors of x[batch*heads][n][D].
// With PG the code rows (and copies) go to pools of pages instead: token t
// of sequence b, head h, is pool row (table[b][t >> page_log2] * heads + h)
// * page + t % page; a token whose table entry is outside [0, n_pages) is
// not stored.
struct EncodePages {
  const int32_t* table;  // [batch][max_pages]
  int max_pages, page_log2, n_pages;
};

template <int D, bool PG = false>
__global__ __launch_bounds__(kEncodeThreads) void k_encode(const void* __restrict__ x,
                                                           int is_bf16, int64_t n, int64_t nvec,
                                                           uint8_t* __restrict__ codes,
                                                           int64_t cap, int64_t pos,
                                                           void* __restrict__ copy, int heads,
                                                           EncodeRule rule,
                                                           EncodePages pg = {}) {
  // a 16-lane slot per vector: lane l holds dimensions [l*EL, l*EL + EL), so
  // the butterflies of distance below EL stay in registers and the others
  // (EL, 2EL, 4EL, 8EL) are DPP exchanges inside the slot's row of 16 lanes;
  // each lane moves 16 bytes or more of the vector per access.  The rows are
  // read once and their copies not read back soon: non-temporal accesses
  // (they slow a decode streaming beside the encoder less)
  constexpr int EL = D / 16, SLOTS = kEncodeThreads / 16;
  constexpr int kGroupLanes = (D > 128 ? 128 : D) / EL;  // lanes of one absmax group
  const int l16 = threadIdx.x & 15;
  const int64_t nslots = (int64_t)gridDim.x * SLOTS;
  for (int64_t v = (int64_t)blockIdx.x * SLOTS + (threadIdx.x >> 4); v < nvec; v += nslots) {
    const int64_t bh = v / n;
    int64_t row = bh * cap + pos + (v - bh * n);
    if constexpr (PG) {
      const int64_t b = bh / heads, t = pos + (v - bh * n);
      const int32_t id = pg.table[b * pg.max_pages + (t >> pg.page_log2)];
      if (id < 0 || id >= pg.n_pages) continue;  // the same for the slot's 16 lanes
      row = (((int64_t)id * heads + (bh - b * heads)) << pg.page_log2) +
            (t & ((int64_t{1} << pg.page_log2) - 1));
    }
    const int64_t src = v * D + l16 * EL;
    float y[EL];
    if (is_bf16) {
      constexpr int NB = EL * 2;  // bytes per lane
      const uint8_t* s8 = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(x) + src);
      uint32_t w[EL / 2];
      if constexpr (NB == 8) {
        const uint2 t = *reinterpret_cast<const uint2*>(s8);
        w[0] = t.x; w[1] = t.y;
        if (copy != nullptr)
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(copy) + row * D + l16 * EL) = t;
      } else {
#pragma unroll
        for (int k = 0; k < NB / 16; ++k) {
          const uint4 t = load_stream(reinterpret_cast<const uint4*>(s8) + k);
          w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
          if (copy != nullptr)
            store_stream(
                reinterpret_cast<uint4*>(static_cast<uint16_t*>(copy) + row * D + l16 * EL) + k, t);
        }
      }
#pragma unroll
      for (int e = 0; e < EL; ++e)
        y[e] = (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : bf16_to_f32(w[e >> 1] & 0xffffu);
    } else {
      const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + src);
#pragma unroll
      for (int k = 0; k < EL / 4; ++k) {
        const uint4 t = load_stream(s4 + k);
        y[4 * k] = __uint_as_float(t.x); y[4 * k + 1] = __uint_as_float(t.y);
        y[4 * k + 2] = __uint_as_float(t.z); y[4 * k + 3] = __uint_as_float(t.w);
        if (copy != nullptr)
          store_stream(reinterpret_cast<uint4*>(static_cast<float*>(copy) + row * D + l16 * EL) + k,
                       t);
      }
    }
    if (rule.rotate == 1)
      slot_fwht<D, false>(y, l16);
    else if (rule.rotate == 2)
      slot_fwht<D, true>(y, l16);
    // §2.2: absmax of the vector's 128-dimension group, codes at -alpha*a, 0,
    // alpha*a (alpha of the vector's head; 0.5 unless set)
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < EL; ++e) a = fmaxf(a, fabsf(y[e]));
    a = fmaxf(a, lane_xor<1>(a));
    a = fmaxf(a, lane_xor<2>(a));
    if constexpr (kGroupLanes >= 8) a = fmaxf(a, lane_xor<4>(a));
    if constexpr (kGroupLanes >= 16) a = fmaxf(a, lane_xor<8>(a));
    const float t2 = rule.alpha_of((int)(bh % heads)) * a, t0 = -t2;
    // §3.1: 4 codes per byte, first code in the high bits; 16 dimensions per word
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const float val = y[e];
      const uint32_t c = (val < t0) ? 0u : (val < 0.0f) ? 1u : (val < t2) ? 2u : 3u;
      const int i = (l16 * EL + e) & 15;  // dimension index within its word
      bits |= c << (8 * (i >> 2) + 6 - 2 * (i & 3));
    }
    constexpr int kLanesPerWord = 16 / EL;
    if constexpr (kLanesPerWord >= 2) bits |= lane_xor_u32<1>(bits);
    if constexpr (kLanesPerWord >= 4) bits |= lane_xor_u32<2>(bits);
    if (l16 % kLanesPerWord == 0)
      reinterpret_cast<uint32_t*>(codes + row * (D / 4))[l16 / kLanesPerWord] = bits;
  }
}

// -------------------------------------------------------------------- scan
// §2.3: stream one chunk of packed key codes and produce, for each of the G
// query heads sharing this KV head, the Manhattan distance of every token.
// Codes are read as 16-byte units (64 codes) with non-temporal loads, U per
// thread in flight; at D = 128 a token is two units held by a lane pair whose
// partial sums are added with a DPP swap.
//
// Where a head's code units are, and which of them each lane takes: one
// contiguous stream, or pages of a pool.  A scan walks batches at `base` in
// [0, limit(units)) by step<NT, U>(); load j of a batch reads this lane's
// unit(base, j), and units from bound(units) on are read in bounds but not
// used.
struct ContigCodes {
  const uint4* p;
  template <int NT>
  ADM_DEV int unit(int base, int j) const { return base + j * NT + (int)threadIdx.x; }
  template <int NT, int U>
  static constexpr int step() { return NT * U; }
  ADM_DEV int limit(int units) const { return units; }
  ADM_DEV int bound(int units) const { return units; }
  ADM_DEV uint4 load(int u, int units) const {
    return load_stream(p + (u < units ? u : units - 1));
  }
};

// Paged code cache: each wavefront of the chunk's workgroup scans its own
// stretch of `upw` consecutive units, [w0, w0 + upw), which lies inside one
// page (pages hold >= 16 stretches and stretches start on multiples of upw),
// so the page table is read once per wavefront and every load is a plain
// offset from `page` (the pool units of this KV head in that page; poff is
// the page offset of unit w0).
struct PagedCodes {
  const uint4* page;
  int w0, upw, poff;
  template <int NT>
  ADM_DEV int unit(int base, int j) const {
    return w0 + base + j * kWave + (int)(threadIdx.x & (kWave - 1));
  }
  template <int NT, int U>
  static constexpr int step() { return kWave * U; }
  ADM_DEV int limit(int units) const {
    const int r = units - w0;
    return r < 0 ? 0 : (r < upw ? r : upw);
  }
  ADM_DEV int bound(int units) const { return units < w0 + upw ? units : w0 + upw; }
  ADM_DEV uint4 load(int u, int units) const {
    return load_stream(page + poff + ((u < bound(units) ? u : w0) - w0));
  }
};

template <int NT, int U, class Src>
ADM_DEV void scan_load(const Src& src, int units, int base, uint4 (&w)[U]) {
#pragma unroll
  for (int j = 0; j < U; ++j) w[j] = src.load(src.template unit<NT>(base, j), units);
}

template <int D, int G, int NT, int U, class Src, class Sink>
ADM_DEV void scan_units(const Src& src, const uint4 (&w)[U], int base, int units,
                        const QPlanes (&qp)[G], Sink&& sink) {
  constexpr int kUnitsPerToken = D / 64;
  const int bnd = src.bound(units);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int u = src.template unit<NT>(base, j);
    const uint32_t p0 = therm_p(w[j].x), p1 = therm_p(w[j].y);
    const uint32_t p2 = therm_p(w[j].z), p3 = therm_p(w[j].w);
    const uint32_t t0 = therm_t(w[j].x, w[j].y), t1 = therm_t(w[j].z, w[j].w);
    uint32_t dg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t s = __popc(p0 ^ qp[g].p[0]);
      s = popc_acc(p1 ^ qp[g].p[1], s);
      s = popc_acc(p2 ^ qp[g].p[2], s);
      s = popc_acc(p3 ^ qp[g].p[3], s);
      s = popc_acc(t0 ^ qp[g].t[0], s);
      s = popc_acc(t1 ^ qp[g].t[1], s);
      if constexpr (kUnitsPerToken == 2) s += swap_pair(s);
      if constexpr (kUnitsPerToken == 4) {  // a quad of lanes holds one token
        s += lane_xor_u32<1>(s);
        s += lane_xor_u32<2>(s);
      }
      dg[g] = s;
    }
    if (u < bnd && (threadIdx.x & (kUnitsPerToken - 1)) == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sink(g, u / kUnitsPerToken, dg[g]);
    }
  }
}

// Whole chunk; with `first` the caller has already issued the loads of the
// first batch (base 0) into it.
template <int D, int G, int NT, int U, class Src, class Sink>
ADM_DEV void scan_chunk(const Src& src, int valid, const QPlanes (&qp)[G], Sink&& sink,
                        const uint4 (*first)[U] = nullptr) {
  constexpr int kUnitsPerToken = D / 64, kStep = Src::template step<NT, U>();
  const int units = valid * kUnitsPerToken, lim = src.limit(units);
  int base = 0;
  if (first != nullptr) {
    if (lim > 0) scan_units<D, G, NT, U>(src, *first, 0, units, qp, sink);
    base = kStep;
  }
  for (; base < lim; base += kStep) {
    uint4 w[U];
    scan_load<NT, U>(src, units, base, w);
    scan_units<D, G, NT, U>(src, w, base, units, qp, sink);
  }
}

// scan_units with 8-bit keys (head_dim 64 and 128): each token's key
// key(tok, d) is counted in hist (exact) and stored as min(key, 255) in
// sdist8 [G][chunk].
template <int D, int G, int NT, int U, class Src, class KeyFn>
ADM_DEV void scan_units_u8(const Src& src, const uint4 (&w)[U], int base, int units,
                           const QPlanes (&qp)[G], KeyFn&& keyfn, uint32_t* shist, int nbp,
                           uint8_t* sdist8, int chunk) {
  constexpr int K = D / 64;  // lanes per token
  static_assert(K == 1 || K == 2, "8-bit keys for head_dim 64 and 128");
  const int bnd = src.bound(units);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int u = src.template unit<NT>(base, j);
    const uint32_t p0 = therm_p(w[j].x), p1 = therm_p(w[j].y);
    const uint32_t p2 = therm_p(w[j].z), p3 = therm_p(w[j].w);
    const uint32_t t0 = therm_t(w[j].x, w[j].y), t1 = therm_t(w[j].z, w[j].w);
    uint32_t dg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t s = __popc(p0 ^ qp[g].p[0]);
      s = popc_acc(p1 ^ qp[g].p[1], s);
      s = popc_acc(p2 ^ qp[g].p[2], s);
      s = popc_acc(p3 ^ qp[g].p[3], s);
      s = popc_acc(t0 ^ qp[g].t[0], s);
      s = popc_acc(t1 ^ qp[g].t[1], s);
      if constexpr (K == 2) s += swap_pair(s);
      dg[g] = s;
    }
    if (u < bnd && (threadIdx.x & (K - 1)) == 0) {
      const int tok = u / K;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t key = keyfn(tok, dg[g]);
        atomicAdd(&shist[g * nbp + key], 1u);
        sdist8[g * chunk + tok] = (uint8_t)(key < (uint32_t)kKeySat ? key : (uint32_t)kKeySat);
      }
    }
  }
}

template <int D, int G, int NT, int U, class Src, class KeyFn>
ADM_DEV void scan_chunk_u8(const Src& src, int valid, const QPlanes (&qp)[G], KeyFn&& keyfn,
                           uint32_t* shist, int nbp, uint8_t* sdist8, int chunk,
                           const uint4 (*first)[U] = nullptr) {
  constexpr int kUnitsPerToken = D / 64, kStep = Src::template step<NT, U>();
  const int units = valid * kUnitsPerToken, lim = src.limit(units);
  int base = 0;
  if (first != nullptr) {
    if (lim > 0)
      scan_units_u8<D, G, NT, U>(src, *first, 0, units, qp, keyfn, shist, nbp, sdist8, chunk);
    base = kStep;
  }
  for (; base < lim; base += kStep) {
    uint4 w[U];
    scan_load<NT, U>(src, units, base, w);
    scan_units_u8<D, G, NT, U>(src, w, base, units, qp, keyfn, shist, nbp, sdist8, chunk);
  }
}

// Query planes for this thread's part of the row (D/64 consecutive lanes hold
// one token's units; lane t of them takes words 4t..4t+3) from packed words in
// LDS.
template <int D, int G>
ADM_DEV void load_qplanes(const uint32_t* sq, QPlanes (&qp)[G]) {
  constexpr int W = D / 16;
  const int part = (int)(threadIdx.x & (D / 64 - 1));
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t* r = sq + g * W + part * 4;
    qp[g] = make_qplanes(r[0], r[1], r[2], r[3]);
  }
}

// ------------------------------------------------------------------- score
// adamas_score: grid (chunks, Hkv, B); query codes already encoded.
template <int D, int G>
__global__ __launch_bounds__(kScoreThreads) void k_score(const uint8_t* __restrict__ q_codes,
                                                         const uint8_t* __restrict__ k_codes,
                                                         int Hq, int Hkv, int64_t cap,
                                                         int64_t n_ctx, int chunk,
                                                         uint16_t* __restrict__ dist) {
  constexpr int W = D / 16;
  __shared__ uint32_t sq[G * W];
  const int c = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  for (int i = threadIdx.x; i < G * W; i += kScoreThreads)
    sq[i] = reinterpret_cast<const uint32_t*>(
        q_codes + ((int64_t)b * Hq + (int64_t)hkv * G) * (D / 4))[i];
  lds_sync();
  QPlanes qp[G];
  load_qplanes<D, G>(sq, qp);
  const int64_t t0 = (int64_t)c * chunk;
  const int valid = (int)min((int64_t)chunk, n_ctx - t0);
  const uint8_t* kbase = k_codes + (((int64_t)b * Hkv + hkv) * cap + t0) * (D / 4);
  uint16_t* drow = dist + ((int64_t)b * Hq + (int64_t)hkv * G) * n_ctx + t0;
  scan_chunk<D, G, kScoreThreads, 8>(ContigCodes{reinterpret_cast<const uint4*>(kbase)}, valid,
                                     qp, [&](int g, int tok, uint32_t d) {
    drow[(int64_t)g * n_ctx + tok] = (uint16_t)d;
  });
}

// ---------------------------------------------------------------- §6 attend
// Gather attention over a list of selected rows of one head.  A 16-lane slot
// owns a row at a time and every lane D/16 dimensions; each slot keeps
// kAttendRowsPerSlot rows' K and V in flight.  Scores stay in the log2 domain
// (q pre-multiplied by scale*log2(e)) and the slots' (m, l, o) merge by
// log-sum-exp.  On return s_res[0] = m, s_res[1] = l, s_res[2 + t] = o_t.
struct Softmax {
  float m, l;
};

template <int EL>
ADM_DEV void merge_partial(Softmax& a, float (&oa)[EL], Softmax bpart, const float (&ob)[EL]) {
  const float M = fmaxf(a.m, bpart.m);
  if (M == -INFINITY) return;
  const float wa = (a.m == -INFINITY) ? 0.0f : exp2f(a.m - M);
  const float wb = (bpart.m == -INFINITY) ? 0.0f : exp2f(bpart.m - M);
  a.l = a.l * wa + bpart.l * wb;
#pragma unroll
  for (int e = 0; e < EL; ++e) oa[e] = oa[e] * wa + ob[e] * wb;
  a.m = M;
}

// Raw element words of one lane's slice of a row (D/16 elements).
template <int D, bool BF>
struct RowRaw {
  static constexpr int EL = D / 16;
  static constexpr int WORDS = BF ? EL / 2 : EL;
  uint32_t w[WORDS];
  ADM_DEV void load(const void* base, int64_t elem) {
    if constexpr (BF) {
      const uint16_t* p = static_cast<const uint16_t*>(base) + elem;
      if constexpr (WORDS >= 4) {
#pragma unroll
        for (int i = 0; i < WORDS / 4; ++i) {
          const uint4 t = reinterpret_cast<const uint4*>(p)[i];
          w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
        }
      } else {
        const uint2 t = *reinterpret_cast<const uint2*>(p);
        w[0] = t.x; w[1] = t.y;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
#pragma unroll
      for (int i = 0; i < WORDS / 4; ++i) {
        const uint4 t = p[i];
        w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
      }
    }
  }
  ADM_DEV float at(int e) const {
    if constexpr (BF)
      return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : bf16_to_f32(w[e >> 1] & 0xffffu);
    else
      return __uint_as_float(w[e]);
  }
};

// Dot product of one lane's q and k slices (EL elements): bf16 pairs go
// through the packed bf16 dot instruction (exact products, binary32 sums).
template <int D, bool BF>
ADM_DEV float slice_dot(const RowRaw<D, BF>& q, const RowRaw<D, BF>& k) {
  float acc = 0.0f;
  if constexpr (BF) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < RowRaw<D, BF>::WORDS; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.w[i]),
                                            __builtin_bit_cast(bf2, k.w[i]), acc, false);
  } else {
#pragma unroll
    for (int e = 0; e < RowRaw<D, BF>::EL; ++e) acc += q.at(e) * k.at(e);
  }
  return acc;
}

// Gather attention over nrows selected rows of one head.  Rows go in
// batches of NS*RB (a 16-lane slot holds RB rows' K and V, every lane D/16
// dimensions).  Each wavefront keeps its own running maximum (shared by its
// 4 slots through lane exchanges, no workgroup barrier per batch), weights
// and a weighted V sum; at the end the NW wavefront partials (m, l, o) are
// merged by log-sum-exp.  On return s_res[0] = m, s_res[1] = l,
// s_res[2 + t] = o_t.  s_part holds NW*(2+D) floats plus NT/16 spare.
// With OVR, row ovr.tok (when >= 0) is read from ovr.k / ovr.v at element
// offset ovr.off instead of the cache (a row appended in the same launch).
// Unselected slots carry token -1 and never match.
struct RowOverride {
  const void* k;
  const void* v;
  int64_t tok;
  int64_t off;
};

// Rows of a paged K/V (or code) pool for one (sequence, KV head): the
// sequence's page table row pt maps its logical page t >> page_log2 to a pool
// page, and token t sits in pool row ((page * Hkv + hkv) << page_log2) plus
// its offset in the page.  Entries outside [0, n_pages) and pages past the
// table are clamped in bounds (such rows hold whatever that page holds).
struct PageMap {
  const int32_t* pt;
  int page_log2, n_pages, max_pages, hkv, Hkv;
  ADM_DEV int32_t entry(int64_t t) const {
    const int64_t pg = t >> page_log2;
    return pt[pg < max_pages - 1 ? pg : max_pages - 1];
  }
  ADM_DEV bool valid(int64_t t) const {
    const int32_t id = entry(t);
    return (t >> page_log2) < max_pages && id >= 0 && id < n_pages;
  }
  ADM_DEV int64_t row(int64_t t) const {
    int32_t id = entry(t);
    id = id < 0 ? 0 : (id < n_pages ? id : n_pages - 1);
    return (((int64_t)id * Hkv + hkv) << page_log2) + (t & ((1 << page_log2) - 1));
  }
};

template <int D, bool BF, int NT, bool OVR = false, bool PG = false>
ADM_DEV void attend_rows(const void* __restrict__ q, const void* __restrict__ k,
                         const void* __restrict__ v, int64_t qoff, int64_t kvrow0, int64_t cap,
                         const int32_t* rows, int nrows, float qscale, float* s_part,
                         float* s_res, RowOverride ovr = {}, PageMap pm = {},
                         const PhaseStamps* ps = nullptr) {
  constexpr int EL = D / 16, NS = NT / 16, NW = NT / kWave, PW = 2 + D;
  // fp32 rows are twice the bytes: half the rows per batch keeps registers in budget
  // (and D = 256 rows twice those of D = 128)
  constexpr int RB = (BF ? kAttendRowsPerSlot : kAttendRowsPerSlot / 2) / (D > 128 ? 2 : 1);
  const int l16 = threadIdx.x & 15, slot = threadIdx.x >> 4;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  RowRaw<D, BF> qr;
  qr.load(q, qoff + l16 * EL);
  float m_run = -INFINITY, l_run = 0.0f;
  float o[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) o[e] = 0.0f;
  for (int r0 = 0; r0 < nrows; r0 += NS * RB) {
    int32_t tok[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int r = r0 + slot + NS * j;
      const int32_t t = (r < nrows) ? rows[r] : -1;
      tok[j] = (t >= 0 && (int64_t)t < cap) ? t : -1;
    }
    RowRaw<D, BF> kr[RB], vr[RB];
    // unselected slots load row 0 of the head (in bounds) and are skipped below
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int64_t t = tok[j] >= 0 ? tok[j] : 0;
      const int64_t r = PG ? pm.row(t) : kvrow0 + t;
      if (OVR && tok[j] >= 0 && tok[j] == ovr.tok) {
        kr[j].load(ovr.k, ovr.off + l16 * EL);
        vr[j].load(ovr.v, ovr.off + l16 * EL);
      } else {
        kr[j].load(k, r * D + l16 * EL);
        vr[j].load(v, r * D + l16 * EL);
      }
    }
    float sc[RB];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      sc[j] = row16_sum(slice_dot<D, BF>(qr, kr[j])) * qscale;
      if (tok[j] < 0) sc[j] = -INFINITY;
      mloc = fmaxf(mloc, sc[j]);
    }
    // the wavefront's maximum over its 4 slots (lanes ^16, ^32).  No early
    // exit for a batch with nothing valid: the update below leaves the state
    // unchanged then (weights 0, correction 1 or 0 on an empty state), and a
    // branch here would let the compiler sink the V loads behind the wait for
    // K, a second memory round trip
    const float mb = xor_max<32>(xor_max<16>(mloc));
    const float mn = fmaxf(m_run, mb);
    const float corr = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - mn);
    l_run *= corr;
#pragma unroll
    for (int e = 0; e < EL; ++e) o[e] *= corr;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const float p = (tok[j] >= 0) ? exp2f(sc[j] - mn) : 0.0f;
      l_run += p;
#pragma unroll
      for (int e = 0; e < EL; ++e) o[e] += p * vr[j].at(e);
    }
    m_run = mn;
  }
  if (ps) {
    ps->mark(9);             // rows gathered, weighted (thread 0's wavefront)
    ps->mark_last_wave(13);  // ... by every wavefront
  }
  // every slot shares m_run: sum l and o over slots (lanes ^16, ^32), then waves
  l_run = xor_sum<32>(xor_sum<16>(l_run));
#pragma unroll
  for (int e = 0; e < EL; ++e) o[e] = xor_sum<32>(xor_sum<16>(o[e]));
  if (ps) ps->mark_last_wave(14);  // slot sums done by every wavefront
  float* mine = s_part + wid * PW;
  if (lane < 16) {
    if (lane == 0) {
      mine[0] = m_run;
      mine[1] = l_run;
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) mine[2 + l16 * EL + e] = o[e];
  }
  lds_sync();
  if (threadIdx.x < D) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_part[w * PW]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_part[w * PW];
      const float a = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
      L += a * s_part[w * PW + 1];
      O += a * s_part[w * PW + 2 + threadIdx.x];
    }
    s_res[2 + threadIdx.x] = O;
    if (threadIdx.x == 0) {
      s_res[0] = M;
      s_res[1] = L;
    }
  }
  lds_sync();
  if (ps) ps->mark(10);  // partials of the wavefronts merged
}

template <bool BF>
ADM_DEV void store_out(void* out, int64_t i, float val) {
  if constexpr (BF)
    static_cast<uint16_t*>(out)[i] = f32_to_bf16(val);
  else
    static_cast<float*>(out)[i] = val;
}

// adamas_sparse_attend (and the large-selection half of a decode step):
// grid (splits, Hq, B), up to kAttendRowsPerBatch rows per workgroup.  With
// more than one split, partial (m, l, o) triples are merged by the last
// workgroup of the head.  With PG, k and v are paged pools and `pages` the
// page table (PageMap; cap is then its logical capacity).
struct PageArgs {
  const int32_t* pages;  // [B][max_pages]
  int max_pages, page_log2, n_pages;
};

template <int D, bool BF, bool PG = false>
__global__ __launch_bounds__(kAttendThreads) void k_attend(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ idx, int Hq, int Hkv, int64_t cap, int budget, float qscale,
    float* __restrict__ part, uint32_t* __restrict__ counters, void* __restrict__ out,
    PageArgs pa = {}, uint64_t* __restrict__ stamps = nullptr) {
  constexpr int NT = kAttendThreads, NW = NT / kWave, PW = 2 + D;
  constexpr int PWP = (PW + 3) & ~3;  // partial rows padded to 16 bytes
  constexpr int kMergeTile = 32;
  __shared__ uint32_t s_tmp[kTmpWords];
  // phase stamps: 0 entry, 9-10 inside attend_rows, 11 partial handed over,
  // 12 merged output stored
  const PhaseStamps ps(stamps, kPhaseAttend, s_tmp);
  ps.mark(0);
  __shared__ float s_part[NW * PW + kAttendRowsPerBatch];
  __shared__ __align__(16) float s_res[PWP];
  __shared__ __align__(16) float s_tile[kMergeTile * PWP];
  const int s = blockIdx.x, hq = blockIdx.y, b = blockIdx.z, S = gridDim.x;
  const int G = Hq / Hkv;
  const int64_t row = (int64_t)b * Hq + hq;
  const int64_t kvrow0 = ((int64_t)b * Hkv + hq / G) * cap;
  const int r0 = s * kAttendRowsPerBatch;
  const int nrows = min(kAttendRowsPerBatch, budget - r0);
  const PageMap pm{PG ? pa.pages + (int64_t)b * pa.max_pages : nullptr, pa.page_log2, pa.n_pages,
                   pa.max_pages, hq / G, Hkv};
  attend_rows<D, BF, NT, false, PG>(q, k, v, row * D, kvrow0, cap, idx + row * budget + r0, nrows,
                                    qscale, s_part, s_res, RowOverride{}, pm, &ps);
  if (S == 1) {
    if (threadIdx.x < D) {
      const float L = s_res[1];
      store_out<BF>(out, row * D + threadIdx.x, L > 0.0f ? s_res[2 + threadIdx.x] / L : 0.0f);
    }
    ps.flush();
    return;
  }
  float* mine = part + (row * S + s) * PWP;
  lds_to_shared<NT>(reinterpret_cast<uint32_t*>(mine), reinterpret_cast<const uint32_t*>(s_res),
                    PWP);
  const bool last = arrive_last<NT>(&counters[row], S, s_tmp);
  ps.mark(11);
  if (!last) {
    ps.flush();
    return;
  }
  const float* pp = part + row * S * PWP;
  float M = -INFINITY, L = 0.0f, O = 0.0f;
  for (int t0 = 0; t0 < S; t0 += kMergeTile) {
    const int nt = min(kMergeTile, S - t0);
    lds_sync();
    shared_to_lds<NT>(reinterpret_cast<uint32_t*>(s_tile),
                      reinterpret_cast<const uint32_t*>(pp + t0 * PWP), nt * PWP);
    lds_sync();
    if (threadIdx.x < D) {
      for (int i = 0; i < nt; ++i) {
        const float mi = s_tile[i * PWP];
        if (mi == -INFINITY) continue;
        const float Mn = fmaxf(M, mi);
        const float a = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
        const float bb = exp2f(mi - Mn);
        L = L * a + s_tile[i * PWP + 1] * bb;
        O = O * a + s_tile[i * PWP + 2 + threadIdx.x] * bb;
        M = Mn;
      }
    }
  }
  if (threadIdx.x < D) store_out<BF>(out, row * D + threadIdx.x, L > 0.0f ? O / L : 0.0f);
  if (threadIdx.x == 0) counters[row] = 0;
  ps.mark(12);
  ps.flush();
}

// --------------------------------------------------------- §5.2 selection
// Per chunk: keep the chunk's min(budget, valid) best (D, token) as
// candidates; a token in the global top-budget is always in its chunk's
// top-budget, so the union of the chunk candidates contains the answer.  The
// last workgroup of a group (atomic arrival count) selects from the union.

// adamas_select_topk: grid (chunks, Hq, B) over uint16 distances.
template <int D>
__global__ __launch_bounds__(kSelectThreads) void k_select(
    const uint16_t* __restrict__ dist, int Hq, int64_t n_ctx, int chunk, int n_chunks,
    int budget, int kpad_log2, int mcap, uint32_t* __restrict__ cand,
    uint32_t* __restrict__ counters, int32_t* __restrict__ idx, int n_sink, int n_recent) {
  constexpr int NT = kSelectThreads, NB = kNbins(D), NBP = kNbinsPadded(D);
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* s_tmp = reinterpret_cast<uint32_t*>(smem);
  uint32_t* shist = s_tmp + kTmpWords;
  uint32_t* sstage = shist + NBP;                           // chunk candidates
  uint8_t* region = reinterpret_cast<uint8_t*>(sstage + (1 << kpad_log2));
  uint16_t* sdist = reinterpret_cast<uint16_t*>(region);   // phase 1
  uint32_t* scand = reinterpret_cast<uint32_t*>(region);   // phase 2
  const int c = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int64_t row = (int64_t)b * Hq + hq;
  for (int i = threadIdx.x; i < NBP; i += NT) shist[i] = 0;
  lds_sync();
  const int64_t t0 = (int64_t)c * chunk;
  const int valid = (int)min((int64_t)chunk, n_ctx - t0);
  const uint16_t* drow = dist + row * n_ctx + t0;
  const int64_t keep_from = n_ctx - n_recent;
  for (int t = threadIdx.x; t < valid; t += NT) {
    // values above 3*D break the caller's contract; clamp so LDS stays in bounds
    const uint32_t d = drow[t] < NB - 1 ? drow[t] : (uint32_t)(NB - 2);
    const uint32_t key = select_key(t0 + t, d, n_sink, keep_from);
    sdist[t] = (uint16_t)key;
    atomicAdd(&shist[key], 1u);
  }
  lds_sync();
  const int kc = min(budget, valid);
  const int kpad = 1 << kpad_log2;
  const Threshold thr = find_threshold<NT>(shist, NB, (uint32_t)kc, s_tmp);
  chunk_compact<NT>(sdist, valid, thr, (uint32_t)kc - thr.lt, sstage, kc, kpad, s_tmp,
                    [](uint32_t, uint32_t) {});
  lds_sync();
  lds_to_shared<NT>(cand + (row * n_chunks + c) * kpad, sstage, kpad);
  if (!arrive_last<NT>(&counters[row], n_chunks, s_tmp)) return;
  final_select<NT>(cand + row * n_chunks * kpad, n_chunks * kpad, kpad_log2, chunk, NB,
                   (int)min((int64_t)budget, n_ctx), budget, nullptr, idx + row * budget, scand,
                   mcap, shist, s_tmp);
  if (threadIdx.x == 0) counters[row] = 0;
}

// ------------------------------------------------------- fused decode step
// adamas_decode_step: grid (chunks, Hkv, B) of 1024-thread workgroups.  Each
// workgroup encodes the G query heads of its KV head (§2.1-§2.2, one
// wavefront per head), scans one chunk of codes (§2.3) keeping distances and
// a histogram in LDS, and writes the chunk's candidates.  The last workgroup
// of the KV head selects the budget for its G query heads (§5.2) and, when
// fuse_attend is set, attends over the selected rows (§6) and writes out.
// Ragged batches with the decoded token appended in the same launch
// (adamas_decode_append_step): sequence b holds lens[b] cached rows; when
// k_new is set its row lens[b] receives the step's key (codes, K) and value
// and the step attends over lens[b] + 1 rows.  n_ctx is then the host's
// bound on those lengths (the grid is planned for it); lens are clamped to
// it and to the cache.
// With a page table (the paged variant, RAG == 2) k, v and k_codes are pools
// of pages as PageMap describes, and cap is the table's logical capacity.
struct RaggedArgs {
  const int32_t* lens;         // [B]
  const void* k_new;           // [B][Hkv][D] elements, or null: nothing appended
  const void* v_new;           // [B][Hkv][D]
  void* k_cache;               // the K, V and code caches again, written at row lens[b]
  void* v_cache;
  uint8_t* code_cache;
  const int32_t* pages;        // [B][max_pages] pool page of each logical page (RAG == 2)
  int max_pages, page_log2, n_pages;
  int pt_lds;                  // 1: the final workgroup copies the table row to LDS after
                               // the candidate tile (max_pages <= kDecodeThreads)
};

// OCC: compiled for two resident workgroups per compute unit (at most 64
// VGPRs), for launches of several rounds, where one workgroup's chunk tail
// then overlaps the other's scan.
// RAG: 0 every sequence holds n_ctx rows; 1 ragged (RaggedArgs); 2 ragged
// over paged pools.
// ONE (RAG 0, 16-bit keys): launches of one chunk per KV head; with
// n_chunks == 1 the chunk's candidates are the selection (see below).
// U8 (grouped heads, head_dim <= 128, RAG 0): the chunk's keys are kept in
// LDS as min(key, 255), one byte per (head, token), which fits twice the
// chunk of 16-bit keys; a launch that would need two rounds of workgroups
// then runs in one.  Keys below a chunk threshold under 255 are exact; a
// chunk where some head's threshold reaches 255 rescans its codes half a
// chunk at a time with exact 16-bit keys.
template <int D, int G, bool BF, int RAG, bool OCC = false, bool U8 = false, bool ONE = false>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(OCC ? 8 : 1)))
void k_decode(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint8_t* __restrict__ k_codes, int Hq, int Hkv, int64_t cap, int64_t n_ctx, int chunk,
    int n_chunks, int budget, int kpad_log2, int mcap, int fuse_attend, float qscale,
    uint32_t* __restrict__ cand, uint32_t* __restrict__ counters, int32_t* __restrict__ idx,
    void* __restrict__ out, int n_sink, int n_recent, EncodeRule rule, RaggedArgs rg,
    uint16_t* __restrict__ chist, int ncp, uint64_t* __restrict__ stamps) {
  constexpr int NT = kDecodeThreads, NW = NT / kWave;
  constexpr int NB = kNbins(D), NBP = kNbinsPadded(D), W = D / 16;
  constexpr int E = D / 64, kLanesPerWord = 16 / E, PW = 2 + D;
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* s_tmp = reinterpret_cast<uint32_t*>(smem);
  // phase stamps (measurement build only): 0 entry, 1 query encoded, 2 scan
  // end, 3 chunk threshold, 4 candidates staged, 5 handed over; final
  // workgroup: 6-7 inside final_select, 8 selection done, 9-10 inside
  // attend_rows, 11 output stored
  const PhaseStamps ps(stamps, kPhaseDecode, s_tmp);
  ps.mark(0);
  uint8_t* region = smem + kTmpWords * 4;
  // phase 1 (scan) layout
  uint32_t* sq = reinterpret_cast<uint32_t*>(region);  // G query rows, then the appended key
  uint32_t* shist = sq + (G + 1) * W;
  const int n_stage = stage_heads(G, 1 << kpad_log2);
  uint32_t* sstage = shist + G * NBP;  // chunk candidates of n_stage heads
  static_assert(!U8 || (G >= 2 && D <= 128 && RAG == 0 && !OCC), "8-bit key variant");
  static_assert(!ONE || (RAG == 0 && !U8), "single-chunk variant");
  uint16_t* sdist = reinterpret_cast<uint16_t*>(sstage + n_stage * (1 << kpad_log2));
  uint8_t* sdist8 = reinterpret_cast<uint8_t*>(sdist);  // U8: [G][chunk] bytes
  uint32_t* s_fused = reinterpret_cast<uint32_t*>(
      U8 ? static_cast<void*>(sdist8 + G * chunk)
         : static_cast<void*>(sdist + G * chunk));  // 2G + NW*G words
  // phase 2 (final selection + attention) layout, aliasing phase 1
  uint32_t* fhist = reinterpret_cast<uint32_t*>(region);
  float* s_part = reinterpret_cast<float*>(fhist + NBP);
  float* s_res = s_part + NW * PW + NT / 16;  // after attend_rows' per-slot scratch
  int32_t* sidx = reinterpret_cast<int32_t*>(s_res + PW);  // fused attention only
  const int bsel_max = (int)min((int64_t)budget, n_ctx);
  uint32_t* scand =
      reinterpret_cast<uint32_t*>(sidx + (fuse_attend ? ((bsel_max + 3) & ~3) : 0));
  uint32_t* s_knew = sq + G * W;  // ragged: the appended key's code row

  // Workgroups are dealt to the 8 XCDs round-robin by linear id; rotating the
  // chunk index with the KV head spreads every chunk offset of the code cache
  // over all XCDs (a fixed offset per XCD loads some XCDs' memory paths more).
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int c = (lin % n_chunks + lin / n_chunks) % n_chunks;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int kpad = 1 << kpad_log2;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  // this sequence's rows and, when appending, the new token's position
  int64_t n_b = n_ctx, pos_new = -1;
  if constexpr (RAG) {
    const bool app = rg.k_new != nullptr;
    const int64_t lim = (cap < n_ctx ? cap : n_ctx) - (app ? 1 : 0);
    int64_t L = rg.lens[b];
    L = L < 0 ? 0 : (L > lim ? lim : L);
    n_b = L + (app ? 1 : 0);
    pos_new = app ? L : -1;
  }
  const int bsel = (int)min((int64_t)budget, n_b);
  const int active = (int)((n_b + chunk - 1) / chunk);  // chunks holding rows of this sequence
  for (int i = threadIdx.x; i < G * NBP; i += NT) shist[i] = 0;
  // the query (wavefront g holds head g, G <= NW), then the first batch of
  // codes, then the query's encoding while the codes are in flight
  static_assert(G <= NW, "one wavefront per query head");
  const int gq = wid < G ? wid : G - 1;  // spare wavefronts load a copy: no branch
  const uint4 qraw =
      load_elems_raw<E, BF>(q, ((int64_t)b * Hq + (int64_t)hkv * G + gq) * D + lane * E);
  const int64_t t0 = (int64_t)c * chunk;
  // rows of the grid's chunk (the planned bound), then of this sequence
  const int valid_grid = (int)min((int64_t)chunk, n_ctx - t0);
  [[maybe_unused]] const PageMap pmap{rg.pages + (int64_t)b * rg.max_pages, rg.page_log2,
                                      rg.n_pages, rg.max_pages, hkv, Hkv};
  const auto src = [&] {
    if constexpr (RAG == 2) {
      // this wavefront's stretch of the chunk and the pool page holding it
      constexpr int kUpt = D / 64;
      const int upp_log2 = rg.page_log2 + (kUpt == 4 ? 2 : kUpt == 2 ? 1 : 0);
      const int upw = chunk * kUpt / NW, w0 = wid * upw;
      const int64_t a = t0 * kUpt + w0;
      const int64_t pg = a >> upp_log2;
      int id = pmap.pt[pg < rg.max_pages - 1 ? pg : rg.max_pages - 1];
      id = __builtin_amdgcn_readfirstlane(id < 0 ? 0 : (id < rg.n_pages ? id : rg.n_pages - 1));
      return PagedCodes{reinterpret_cast<const uint4*>(k_codes) +
                            (((int64_t)id * Hkv + hkv) << upp_log2),
                        w0, upw, (int)(a & ((1 << upp_log2) - 1))};
    } else
      return ContigCodes{reinterpret_cast<const uint4*>(
          k_codes + (((int64_t)b * Hkv + hkv) * cap + t0) * (D / 4))};
  }();
  uint4 first[kDecodeScanDepth];
  scan_load<NT, kDecodeScanDepth>(src, valid_grid * (D / 64), 0, first);
  __builtin_amdgcn_sched_barrier(0);  // keep the code loads ahead of the wait for q
  if constexpr (RAG) {
    if (c >= active) {
      if (n_b == 0 && c == 0) {  // an empty sequence: zeros, nothing selected
        for (int g = 0; g < G; ++g) {
          const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
          if (threadIdx.x < D) store_out<BF>(out, row * D + threadIdx.x, 0.0f);
          if (idx)
            for (int j = threadIdx.x; j < budget; j += NT) idx[row * budget + j] = -1;
        }
      }
      ps.flush();
      return;  // no rows of this sequence in this chunk
    }
  }
  const int valid = (int)min((int64_t)chunk, n_b - t0);
  const bool has_new = RAG && pos_new >= t0 && pos_new < t0 + valid;
  const int valid_mem = valid - (has_new ? 1 : 0);  // rows read from the code cache
  if constexpr (RAG) {
    if (has_new && wid == NW - 1) {
      // the appended token: encode its key, write its code row and its K and
      // V rows for later steps.  Within this launch its distance comes from
      // s_knew and its K, V from k_new, v_new (the final workgroup may sit on
      // another XCD, whose L2 does not see these stores before the launch ends)
      const int64_t src = ((int64_t)b * Hkv + hkv) * D;
      const uint4 kraw = load_elems_raw<E, BF>(rg.k_new, src + lane * E);
      float y[E];
      widen_elems<E, BF>(kraw, y);
      const uint32_t word = wave_encode<D>(y, rule.rotate, rule.alpha_of(hkv));
      const int64_t crow =
          RAG == 2 ? pmap.row(pos_new) : ((int64_t)b * Hkv + hkv) * cap + pos_new;
      // a paged row whose table entry is out of range is scored but not stored
      const bool store = RAG != 2 || pmap.valid(pos_new);
      if (lane % kLanesPerWord == 0) {
        s_knew[lane / kLanesPerWord] = word;
        if (store)
          reinterpret_cast<uint32_t*>(rg.code_cache + crow * (D / 4))[lane / kLanesPerWord] = word;
      }
      constexpr int kRowBytes = D * (BF ? 2 : 4);
      if (store && lane < kRowBytes / 16) {
        const uint4 kv = reinterpret_cast<const uint4*>(
            static_cast<const uint8_t*>(rg.k_new) + src * (BF ? 2 : 4))[lane];
        const uint4 vv = reinterpret_cast<const uint4*>(
            static_cast<const uint8_t*>(rg.v_new) + src * (BF ? 2 : 4))[lane];
        reinterpret_cast<uint4*>(static_cast<uint8_t*>(rg.k_cache) + crow * kRowBytes)[lane] = kv;
        reinterpret_cast<uint4*>(static_cast<uint8_t*>(rg.v_cache) + crow * kRowBytes)[lane] = vv;
      }
    }
  }
  if (wid < G) {
    float y[E];
    widen_elems<E, BF>(qraw, y);
    const uint32_t word = wave_encode<D>(y, rule.rotate, rule.alpha_of(hkv));
    if (lane % kLanesPerWord == 0) sq[wid * W + lane / kLanesPerWord] = word;
  }
  lds_sync();
  ps.mark(1);
  QPlanes qp[G];
  load_qplanes<D, G>(sq, qp);
  const KeepRange keep(t0, valid, n_sink, n_b - n_recent);
  const auto sink = [&](int g, int tok, uint32_t key) {
    sdist[g * chunk + tok] = (uint16_t)key;
    atomicAdd(&shist[g * NBP + key], 1u);
  };
  // a chunk without always-kept tokens (the common case) skips the range test
  // (not in the paged two-per-CU build, where the second copy of the scan
  // costs spills under its 64-register cap)
  if constexpr (U8) {
    if (keep.keeps_none(valid_mem))
      scan_chunk_u8<D, G, NT, kDecodeScanDepth>(
          src, valid_mem, qp, [](int, uint32_t d) { return d + 1u; }, shist, NBP, sdist8, chunk,
          &first);
    else
      scan_chunk_u8<D, G, NT, kDecodeScanDepth>(
          src, valid_mem, qp, [&](int tok, uint32_t d) { return keep.key(tok, d); }, shist, NBP,
          sdist8, chunk, &first);
  } else if (!(OCC && RAG == 2) && keep.keeps_none(valid_mem))
    scan_chunk<D, G, NT, kDecodeScanDepth>(
        src, valid_mem, qp, [&](int g, int tok, uint32_t d) { sink(g, tok, d + 1u); }, &first);
  else
    scan_chunk<D, G, NT, kDecodeScanDepth>(
        src, valid_mem, qp, [&](int g, int tok, uint32_t d) { sink(g, tok, keep.key(tok, d)); },
        &first);
  if constexpr (RAG) {
    if (has_new && (int)threadIdx.x < G) {
      const int g = threadIdx.x, tok = valid_mem;
      const uint32_t key = keep.key(tok, code_distance<D>(sq + g * W, s_knew));
      sdist[g * chunk + tok] = (uint16_t)key;
      atomicAdd(&shist[g * NBP + key], 1u);
    }
  }
  lds_sync();
  ps.mark(2);
  if (chist != nullptr) {
    // separate selection (k_split_select): this chunk's key counts per head,
    // one row of kNbinsHist(D) u16 per (head, chunk), 8 counts per store
    constexpr int CR = kNbinsHist(D), CQ = CR / 8;
    for (int i = threadIdx.x; i < G * CQ; i += NT) {
      const int g = i / CQ, b0 = (i - g * CQ) * 8;
      const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int kb = b0 + 2 * k;
        const uint32_t lo = kb < NB ? shist[g * NBP + kb] : 0u;
        const uint32_t hi = kb + 1 < NB ? shist[g * NBP + kb + 1] : 0u;
        w[k] = lo | (hi << 16);
      }
      reinterpret_cast<uint4*>(chist + (row * ncp + c) * CR)[b0 / 8] =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  const int kc = min(budget, valid);
  // one chunk per head: its kc = bsel candidates, in token order, are the
  // selection itself, so the step needs neither their hand-over, an arrival
  // nor a final selection.  solo: the attention follows at once; solo_sel
  // (attention in a later launch): the index rows are written from here
  // (a separate instantiation, so that the multi-chunk kernels keep their
  // registers and code as they are)
  const bool one = ONE && n_chunks == 1 && chist == nullptr;
  const bool solo = one && fuse_attend && bsel <= NT && (G == 1 || n_stage == G);
  const bool solo_sel = one && !fuse_attend;
  const auto write_idx = [&](int g, const uint32_t* st) {
    const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
    for (int j = threadIdx.x; j < budget; j += NT)
      idx[row * budget + j] = j < bsel ? (int32_t)(st[j] & 0xffffu) : -1;
  };
  bool staged = false;
  if constexpr (G >= 2) {
    if (n_stage == G) {
      if constexpr (U8) {
        const bool exact = chunk_compact_heads_u8<NT, NB, G>(
            shist, NBP, sdist8, chunk, valid, (uint32_t)kc, sstage, kpad, s_fused,
            s_fused + 2 * G, &ps);
        if constexpr (3 * D + 1 >= kKeySat) {
          if (!exact) {
            // exact 16-bit keys, half a chunk at a time, in the bytes' place
            // (G halves of 16-bit keys fill the G chunks of bytes); s_tot:
            // per head the (below, at) counts of earlier halves, and the
            // count chunk_collect reports
            const int kHalf = chunk / 2;  // <= NT * kCompactTpt tokens
            uint16_t* sd16 = reinterpret_cast<uint16_t*>(sdist8);
            uint32_t* s_thr = s_fused;
            uint32_t* s_tot = s_fused + 2 * G;
            if ((int)threadIdx.x < 2 * G) s_tot[threadIdx.x] = 0u;
            QPlanes qh[G];
            load_qplanes<D, G>(sq, qh);
            for (int h0 = 0; h0 < valid; h0 += kHalf) {
              const int hv = min(kHalf, valid - h0);
              lds_sync();
              scan_chunk<D, G, NT, kDecodeScanDepth>(
                  ContigCodes{src.p + (int64_t)h0 * (D / 64)}, hv, qh,
                  [&](int g, int tok, uint32_t d) {
                    sd16[g * kHalf + tok] = (uint16_t)keep.key(h0 + tok, d);
                  });
              lds_sync();
              for (int g = 0; g < G; ++g) {
                const uint32_t t = s_thr[2 * g], quota = (uint32_t)kc - s_thr[2 * g + 1];
                const uint32_t ltp = s_tot[2 * g], eqp = s_tot[2 * g + 1];
                const uint32_t taken = eqp < quota ? eqp : quota, off = ltp + taken;
                uint32_t* o = sstage + g * kpad;
                chunk_collect<NT>(
                    sd16 + g * kHalf, hv, (int)t, quota - taken, s_tmp,
                    [&](uint32_t pos, uint32_t tok, uint32_t key) {
                      o[off + pos] = (key << 16) | (uint32_t)(h0 + (int)tok);
                    },
                    nullptr, s_tot + 2 * G);
                lds_sync();
                if (threadIdx.x == 0) {
                  const uint32_t tot = s_tot[2 * G];
                  s_tot[2 * g] = ltp + (tot & 0xffffu);
                  s_tot[2 * g + 1] = eqp + (tot >> 16);
                }
                lds_sync();
              }
            }
          }
        }
      } else {
        chunk_compact_heads<NT, NB, G>(shist, NBP, sdist, chunk, valid, (uint32_t)kc, sstage,
                                       kpad, s_fused, s_fused + 2 * G, &ps);
      }
      ps.mark(4);
      for (int g = 0; g < G; ++g) {
        const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
        if (solo_sel)
          write_idx(g, sstage + g * kpad);
        else if (!solo)
          lds_to_shared<NT>(cand + (row * n_chunks + c) * kpad, sstage + g * kpad, kpad);
      }
      staged = true;
    }
  }
  if (!staged) {
    for (int g = 0; g < G; ++g) {
      const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
      const Threshold thr = find_threshold<NT>(shist + g * NBP, NB, (uint32_t)kc, s_tmp);
      ps.mark(3);
      bool halves = false;
      if constexpr (OCC && G == 1 && RAG != 2) halves = valid > NT * kCompactTpt;
      if (!halves) {
        chunk_compact<NT>(sdist + g * chunk, valid, thr, (uint32_t)kc - thr.lt, sstage, kc,
                          kpad, s_tmp, [](uint32_t, uint32_t) {}, &ps);
      } else {
        // chunks of more than NT * kCompactTpt tokens (multi-round MHA
        // launches): one compaction pass per half, in token order; s_tot
        // holds the (below, at) threshold counts of the earlier halves and
        // the count chunk_collect reports
        constexpr int kHalf = NT * kCompactTpt;
        uint32_t* s_tot = s_fused;
        if (threadIdx.x < 2) s_tot[threadIdx.x] = 0u;
        const uint32_t quota = (uint32_t)kc - thr.lt;
        for (int h0 = 0; h0 < valid; h0 += kHalf) {
          lds_sync();
          const uint32_t ltp = s_tot[0], eqp = s_tot[1];
          const uint32_t taken = eqp < quota ? eqp : quota, off = ltp + taken;
          chunk_collect<NT>(
              sdist + g * chunk + h0, min(kHalf, valid - h0), thr.t, quota - taken, s_tmp,
              [&](uint32_t pos, uint32_t tok, uint32_t key) {
                sstage[off + pos] = (key << 16) | (uint32_t)(h0 + (int)tok);
              },
              nullptr, s_tot + 2);
          lds_sync();
          if (threadIdx.x == 0) {
            const uint32_t tot = s_tot[2];
            s_tot[0] = ltp + (tot & 0xffffu);
            s_tot[1] = eqp + (tot >> 16);
          }
        }
        for (int j = kc + (int)threadIdx.x; j < kpad; j += NT) sstage[j] = 0xFFFFFFFFu;
      }
      lds_sync();
      ps.mark(4);
      if (solo_sel)
        write_idx(g, sstage);
      else if (!solo)
        lds_to_shared<NT>(cand + (row * n_chunks + c) * kpad, sstage, kpad);
    }
  }
  if (solo_sel) {
    ps.mark(11);
    ps.flush();
    return;
  }
  if (chist != nullptr) {  // k_split_select takes it from here
    ps.mark(5);
    ps.flush();
    return;
  }
  if (solo) {
    // the token lists go to registers first (the attention's LDS overlaps the
    // staged rows), then, per head, to the index row and the attention
    int32_t mine[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      mine[g] = (int)threadIdx.x < bsel ? (int32_t)(sstage[g * kpad + threadIdx.x] & 0xffffu)
                                        : -1;
    lds_sync();
    ps.mark(8);
    const int64_t kvrow0 = ((int64_t)b * Hkv + hkv) * cap;
#pragma unroll 1
    for (int g = 0; g < G; ++g) {
      const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
      int32_t tok = mine[0];  // mine[g] by selects (a variable index would spill)
#pragma unroll
      for (int u = 1; u < G; ++u) tok = u == g ? mine[u] : tok;
      if ((int)threadIdx.x < bsel) sidx[threadIdx.x] = tok;
      if (idx) {
        for (int j = threadIdx.x; j < budget; j += NT)
          idx[row * budget + j] = j < bsel ? tok : -1;
      }
      lds_sync();
      attend_rows<D, BF, NT>(q, k, v, row * D, kvrow0, cap, sidx, bsel, qscale, s_part, s_res,
                             RowOverride{}, PageMap{}, &ps);
      if (threadIdx.x < D) {
        const float L = s_res[1];
        store_out<BF>(out, row * D + threadIdx.x, L > 0.0f ? s_res[2 + threadIdx.x] / L : 0.0f);
      }
      lds_sync();
    }
    ps.mark(11);
    ps.flush();
    return;
  }
  const bool last = arrive_last<NT>(&counters[b * Hkv + hkv], active, s_tmp);
  ps.mark(5);
  if (!last) {
    ps.flush();
    return;
  }
  const int64_t kvrow0 = ((int64_t)b * Hkv + hkv) * cap;
  // paged: the gathers below look up the sequence's page table; its row is
  // loaded now (in flight during the selection) and kept in LDS
  [[maybe_unused]] PageMap amap = pmap;
  [[maybe_unused]] int32_t pt_entry = 0;
  if constexpr (RAG == 2) {
    if (rg.pt_lds && fuse_attend && (int)threadIdx.x < rg.max_pages)
      pt_entry = pmap.pt[threadIdx.x];
  }
  for (int g = 0; g < G; ++g) {
    const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
    final_select<NT>(cand + row * n_chunks * kpad, active * kpad, kpad_log2, chunk, NB, bsel,
                     budget, fuse_attend ? sidx : nullptr, idx ? idx + row * budget : nullptr,
                     scand, mcap, fhist, s_tmp, nullptr, &ps);
    ps.mark(8);
    if constexpr (RAG == 2) {
      if (g == 0 && rg.pt_lds && fuse_attend) {
        int32_t* s_pt = reinterpret_cast<int32_t*>(scand + mcap);
        if ((int)threadIdx.x < rg.max_pages) s_pt[threadIdx.x] = pt_entry;
        lds_sync();
        amap.pt = s_pt;
      }
    }
    if (fuse_attend) {
      if constexpr (RAG)
        attend_rows<D, BF, NT, true, RAG == 2>(
            q, k, v, row * D, kvrow0, cap, sidx, bsel, qscale, s_part, s_res,
            RowOverride{rg.k_new, rg.v_new, rg.k_new != nullptr ? pos_new : -2,
                        ((int64_t)b * Hkv + hkv) * D},
            amap, &ps);
      else
        attend_rows<D, BF, NT>(q, k, v, row * D, kvrow0, cap, sidx, bsel, qscale, s_part, s_res,
                               RowOverride{}, PageMap{}, &ps);
      if (threadIdx.x < D) {
        const float L = s_res[1];
        store_out<BF>(out, row * D + threadIdx.x, L > 0.0f ? s_res[2 + threadIdx.x] / L : 0.0f);
      }
      lds_sync();
    }
  }
  if (threadIdx.x == 0) counters[b * Hkv + hkv] = 0;
  ps.mark(11);
  ps.flush();
}

// ------------------------------------- decode step, selection on its own
// When a head has too many chunk candidates for one workgroup to select
// from quickly (n_chunks * kpad well beyond what fits in LDS at once),
// k_decode publishes each chunk's candidates and its key counts per query
// head and stops, and this kernel selects.  Grid (segments, B*Hq).  Each
// workgroup sums the head's counts over the chunks (§5.2 threshold t and
// quota of ties), derives for every chunk how many of its keys lie below t
// and how many of its ties it contributes, and from their prefix sums where
// its kept tokens start in the ascending selection; its wavefronts then copy
// the kept tokens of the segment's chunks there, one chunk at a time.  Ties
// at t go to the lowest token indices: chunks are in token order, and each
// chunk's candidates are too.
//   chist [B*Hq][ncp][kNbinsHist(D)] u16 (a row of key counts per chunk),
//         ncp >= n_chunks
//   cand  [B*Hq][n_chunks][kpad] as k_decode leaves it (token order, 0xFFFFFFFF unused)
constexpr int kSplitThreads = 1024;
constexpr int kSplitMaxChunks = 2048;
constexpr int kSplitEntriesPerLane = 16;  // a wavefront loads 1024 candidates at once
constexpr int kSplitRegChunks = 4;  // count rows a wavefront holds in registers (fast path)

// With fa.q set, each workgroup also attends over the tokens it placed (its
// segment's share of the selection, staged in LDS; at most kSplitFuseRows)
// and publishes a partial (m, l, o); the last workgroup of the head merges
// them by log-sum-exp and writes the output (no separate attention launch).
// LDS (dynamic): split_select_lds(D, n_chunks, fused).
struct SplitAttend {
  const void* q;               // null: selection only
  const void* k;
  const void* v;
  int Hq, Hkv;
  int64_t cap;
  float qscale;
  float* part;                 // [B*Hq][segments][PWP] partials
  uint32_t* counters;          // [B*Hq] arrival counters, left zero
  void* out;
  uint64_t* stamps;            // phase stamps (measurement build), or null
};
constexpr int kSplitFuseRows = 8192;

template <int D, bool BF>
__global__ __launch_bounds__(kSplitThreads) void k_split_select(
    const uint32_t* __restrict__ cand, const uint16_t* __restrict__ chist, int n_chunks, int ncp,
    int chunks_per_seg, int kpad_log2, int chunk, int nbins, int bsel, int budget,
    int32_t* __restrict__ idx, SplitAttend fa) {
  constexpr int NT = kSplitThreads, NW = NT / kWave, EPL = kSplitEntriesPerLane;
  constexpr int PW = 2 + D, PWP = (PW + 3) & ~3;
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* s_tmp = reinterpret_cast<uint32_t*>(smem);
  // phase stamps: 0 entry, 1 threshold, 2 placement done, 3 tokens copied,
  // 9-10 inside attend_rows, 11 partial handed over, 12 merged output stored
  const PhaseStamps ps(fa.stamps, kPhaseSplit, s_tmp);
  ps.mark(0);
  uint32_t* s_hist = s_tmp + kTmpWords;
  uint32_t* s_first = s_hist + kNbinsPadded(D);  // first output position of the chunk's tokens
  uint32_t* s_take = s_first + ncp;               // (count below t) << 16 | ties taken
  int32_t* s_rows = reinterpret_cast<int32_t*>(s_take + ncp);  // fused: this segment's tokens
  float* s_part = reinterpret_cast<float*>(s_rows + kSplitFuseRows);
  float* s_res = s_part + NW * PW + NT / 16;
  const int64_t row = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  constexpr int CR = kNbinsHist(D), CQ = CR / 8;
  const uint16_t* h = chist + row * ncp * CR;
  // the first EPL*64 candidates of this wavefront's first chunk, loaded now
  // so that they arrive while the counts are summed
  const int kpad_pre = 1 << kpad_log2;
  const int c_pre = (int)blockIdx.x * chunks_per_seg + wid;
  const bool has_pre = c_pre < min(n_chunks, ((int)blockIdx.x + 1) * chunks_per_seg);
  uint4 pre[EPL / 4];
#pragma unroll
  for (int u = 0; u < EPL / 4; ++u) {
    const int i = lane * EPL + 4 * u;
    pre[u] = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
    if (has_pre && i < kpad_pre)
      pre[u] = *reinterpret_cast<const uint4*>(cand + ((row * n_chunks + c_pre) << kpad_log2) + i);
  }
  for (int i = threadIdx.x; i < nbins; i += NT) s_hist[i] = 0;
  for (int i = threadIdx.x; i < n_chunks; i += NT) s_first[i] = 0;
  lds_sync();
  Threshold thr;
  if (CQ <= kWave && n_chunks <= kSplitRegChunks * NW) {
    // every count in registers after one round of loads: wavefront w holds
    // the rows of chunks w, w + NW, ..., lane l their keys 8l..8l+7
    uint4 e[kSplitRegChunks];
#pragma unroll
    for (int k = 0; k < kSplitRegChunks; ++k) {
      const int c = wid + NW * k;
      e[k] = make_uint4(0u, 0u, 0u, 0u);
      if (c < n_chunks && lane < CQ) e[k] = reinterpret_cast<const uint4*>(h + (int64_t)c * CR)[lane];
    }
    // count u (0..7) of a row slice: half u & 1 of word u >> 1
    const auto count = [](const uint4& x, int u) {
      const int wi = u >> 1;
      const uint32_t w = wi < 2 ? (wi == 0 ? x.x : x.y) : (wi == 2 ? x.z : x.w);
      return (w >> (16 * (u & 1))) & 0xffffu;
    };
    if (lane < CQ) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // this lane's key 8l+u summed over its chunks
        uint32_t sum = 0;
#pragma unroll
        for (int k = 0; k < kSplitRegChunks; ++k) sum += count(e[k], u);
        if (sum && lane * 8 + u < nbins) atomicAdd(&s_hist[lane * 8 + u], sum);
      }
    }
    lds_sync();
    thr = find_threshold<NT>(s_hist, nbins, (uint32_t)bsel, s_tmp);
    // per chunk: keys below t and ties at t, one wavefront sum each
#pragma unroll
    for (int k = 0; k < kSplitRegChunks; ++k) {
      const int c = wid + NW * k;
      if (c >= n_chunks) break;  // uniform in the wavefront
      uint32_t lt = 0, eq = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kb = lane * 8 + u;
        const uint32_t n = count(e[k], u);
        lt += kb < thr.t ? n : 0u;
        eq += kb == thr.t ? n : 0u;
      }
      lt = __builtin_amdgcn_readlane(wave_scan_incl(lt), kWave - 1);
      eq = __builtin_amdgcn_readlane(wave_scan_incl(eq), kWave - 1);
      if (lane == 0) {
        s_first[c] = lt;
        s_take[c] = eq;
      }
    }
  } else {
    {  // the head's counts: P threads per key, each over every P-th chunk
      const int P = max(1, NT / nbins);
      for (int it = threadIdx.x; it < nbins * P; it += NT) {
        const int kb = it / P, p = it - kb * P;
        uint32_t sum = 0;
        for (int c = p; c < n_chunks; c += P) sum += h[(int64_t)c * CR + kb];
        if (sum) atomicAdd(&s_hist[kb], sum);
      }
    }
    lds_sync();
    thr = find_threshold<NT>(s_hist, nbins, (uint32_t)bsel, s_tmp);
    {  // per chunk: keys below t (P2 threads per chunk, every P2-th key) and ties at t
      const int P2 = max(1, NT / n_chunks);
      for (int it = threadIdx.x; it < n_chunks * P2; it += NT) {
        const int c = it % n_chunks, p = it / n_chunks;
        const uint16_t* hc = h + (int64_t)c * CR;
        uint32_t sum = 0;
#pragma unroll 4
        for (int kb = p; kb < thr.t; kb += P2) sum += hc[kb];
        if (sum) atomicAdd(&s_first[c], sum);
        if (p == 0) s_take[c] = hc[thr.t];
      }
    }
  }
  const uint32_t quota = (uint32_t)bsel - thr.lt;
  ps.mark(1);
  lds_sync();
  if (n_chunks <= kWave) {
    // prefix sums over chunks in one wavefront: where each chunk's tokens
    // start, and its share of the ties (the same arithmetic as below)
    if (wid == 0) {
      const int c = lane;
      const uint32_t lt = c < n_chunks ? s_first[c] : 0u, eq = c < n_chunks ? s_take[c] : 0u;
      const uint32_t lt_ex = wave_scan_incl(lt) - lt, eq_ex = wave_scan_incl(eq) - eq;
      const uint32_t before = eq_ex < quota ? eq_ex : quota;
      const uint32_t q = min(eq, quota - before);
      if (c < n_chunks) {
        s_first[c] = lt_ex + before;
        s_take[c] = (lt << 16) | q;
      }
    }
  } else {  // prefix sums over chunks: where each chunk's tokens start, and its share of ties
    const int tpt = (n_chunks + NT - 1) / NT, c0 = threadIdx.x * tpt;
    uint32_t lts = 0, eqs = 0;
    for (int j = 0; j < tpt; ++j)
      if (c0 + j < n_chunks) {
        lts += s_first[c0 + j];
        eqs += s_take[c0 + j];
      }
    uint32_t tot;
    uint32_t lt_ex = block_scan_incl<NT>(lts, s_tmp, &tot) - lts;
    uint32_t eq_ex = block_scan_incl<NT>(eqs, s_tmp, &tot) - eqs;
    for (int j = 0; j < tpt; ++j) {
      const int c = c0 + j;
      if (c >= n_chunks) break;
      const uint32_t lt = s_first[c], eq = s_take[c];
      // ties taken by earlier chunks, then this chunk's share.  Written so
      // that no subtraction can wrap: with `eq_ex >= quota ? 0 : min(eq,
      // quota - eq_ex)` the compiler (ROCm 7.2 clang) also folded a separate
      // min(eq_ex, quota) to eq_ex
      const uint32_t before = eq_ex < quota ? eq_ex : quota;
      const uint32_t q = min(eq, quota - before);
      s_first[c] = lt_ex + before;
      s_take[c] = (lt << 16) | q;
      lt_ex += lt;
      eq_ex += eq;
    }
  }
  lds_sync();
  ps.mark(2);
  int32_t* out = idx + row * budget;
  if (blockIdx.x == 0)
    for (int j = bsel + threadIdx.x; j < budget; j += NT) out[j] = -1;
  const uint32_t t = (uint32_t)thr.t;
  const int kpad = 1 << kpad_log2;
  const int c_lo = blockIdx.x * chunks_per_seg, c_hi = min(n_chunks, c_lo + chunks_per_seg);
  // this segment's slots of the selection: [seg0, seg1)
  const uint32_t seg0 = c_lo < n_chunks ? s_first[c_lo] : (uint32_t)bsel;
  const uint32_t seg1 = c_hi < n_chunks ? s_first[c_hi] : (uint32_t)bsel;
  const bool fused = fa.q != nullptr;
  for (int c = c_lo + wid; c < c_hi; c += NW) {
    const uint32_t tk = s_take[c], q = tk & 0xffffu, need = (tk >> 16) + q;
    if (need == 0) continue;
    uint32_t pos = s_first[c], ties = 0, got = 0;
    const uint32_t end = min(pos + need, (uint32_t)bsel);  // this chunk's slots in the selection
    const uint32_t* list = cand + ((row * n_chunks + c) << kpad_log2);
    const int32_t tok0 = c * chunk;
    for (int base = 0; base < kpad && got < need; base += EPL * kWave) {
      // EPL consecutive candidates per lane, in token order across lanes
      uint32_t v[EPL];
#pragma unroll
      for (int u = 0; u < EPL / 4; ++u) {
        const int i = base + lane * EPL + 4 * u;
        uint4 e = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
        if (base == 0 && c == c_pre)
          e = pre[u];
        else if (i < kpad)
          e = *reinterpret_cast<const uint4*>(list + i);
        v[4 * u] = e.x;
        v[4 * u + 1] = e.y;
        v[4 * u + 2] = e.z;
        v[4 * u + 3] = e.w;
      }
      uint32_t neq = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) neq += (v[j] >> 16) == t;
      const uint32_t eq_incl = wave_scan_incl(neq);
      uint32_t rank = ties + eq_incl - neq;  // ties of this chunk before this lane's
      uint32_t flags = 0, ntake = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const uint32_t d = v[j] >> 16;
        const bool take = d < t || (d == t && rank < q);
        rank += d == t;
        flags |= (take ? 1u : 0u) << j;
        ntake += take;
      }
      const uint32_t take_incl = wave_scan_incl(ntake);
      uint32_t o = pos + take_incl - ntake;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if ((flags >> j & 1u) && o < end) {
          const int32_t tok = tok0 + (int32_t)(v[j] & 0xffffu);
          out[o] = tok;
          if (fused) s_rows[o - seg0] = tok;
          ++o;
        }
      const uint32_t took = __builtin_amdgcn_readlane(take_incl, kWave - 1);
      ties += __builtin_amdgcn_readlane(eq_incl, kWave - 1);
      got += took;
      pos += took;
    }
  }
  if (!fused) {
    ps.flush();
    return;
  }
  // §6 over this segment's rows, then the log-sum-exp merge of the segments
  lds_sync();
  ps.mark(3);
  const int G = fa.Hq / fa.Hkv;
  const int b = (int)(row / fa.Hq), hq = (int)(row % fa.Hq);
  const int64_t kvrow0 = ((int64_t)b * fa.Hkv + hq / G) * fa.cap;
  attend_rows<D, BF, NT>(fa.q, fa.k, fa.v, row * D, kvrow0, fa.cap, s_rows, (int)(seg1 - seg0),
                         fa.qscale, s_part, s_res, RowOverride{}, PageMap{}, &ps);
  const int S = gridDim.x;
  if (S == 1) {
    if ((int)threadIdx.x < D) {
      const float L = s_res[1];
      store_out<BF>(fa.out, row * D + threadIdx.x, L > 0.0f ? s_res[2 + threadIdx.x] / L : 0.0f);
    }
    ps.flush();
    return;
  }
  lds_to_shared<NT>(reinterpret_cast<uint32_t*>(fa.part + (row * S + blockIdx.x) * PWP),
                    reinterpret_cast<const uint32_t*>(s_res), PWP);
  const bool last = arrive_last<NT>(&fa.counters[row], S, s_tmp);
  ps.mark(11);
  if (!last) {
    ps.flush();
    return;
  }
  // merge: partials staged through LDS (the row list is free now)
  float* s_tile = reinterpret_cast<float*>(s_rows);
  constexpr int kTile = kSplitFuseRows / PWP;
  const float* pp = fa.part + row * S * PWP;
  float M = -INFINITY, L = 0.0f, O = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kTile) {
    const int nt = min(kTile, S - s0);
    lds_sync();
    shared_to_lds<NT>(reinterpret_cast<uint32_t*>(s_tile),
                      reinterpret_cast<const uint32_t*>(pp + s0 * PWP), nt * PWP);
    lds_sync();
    if ((int)threadIdx.x < D) {
      for (int i = 0; i < nt; ++i) {
        const float mi = s_tile[i * PWP];
        if (mi == -INFINITY) continue;
        const float Mn = fmaxf(M, mi);
        const float a = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
        const float bb = exp2f(mi - Mn);
        L = L * a + s_tile[i * PWP + 1] * bb;
        O = O * a + s_tile[i * PWP + 2 + threadIdx.x] * bb;
        M = Mn;
      }
    }
  }
  if ((int)threadIdx.x < D) store_out<BF>(fa.out, row * D + threadIdx.x, L > 0.0f ? O / L : 0.0f);
  if (threadIdx.x == 0) fa.counters[row] = 0;
  ps.mark(12);
  ps.flush();
}

// ------------------------------------------ fused decode step, group wait
// adamas_decode_step when all workgroups of the launch are resident on the
// device together: grid (chunks, Hkv, B) as k_decode, the chunk workgroups
// of one KV head forming a group.  Each workgroup encodes its query heads
// and scans its chunk (§2.1-§2.3) into LDS as k_decode does, then publishes
// only the chunk's distance histograms and waits for its group.  The summed
// histograms give every workgroup each query head's budget threshold (§5.2)
// and, from the chunks before its own, how many of the threshold ties fall
// to its chunk and where its tokens go in the ascending selection; so each
// workgroup keeps its own share of the budget without exchanging candidates,
// attends over those rows (§6) and publishes a partial (m, l, o).  The last
// workgroup of the group merges the partials by log-sum-exp.
//   ghist  [B*Hq][n_chunks][NBH] u16   part [B*Hq][n_chunks][PWP] f32
//   cmax   >= min(budget, n_ctx, chunk), a multiple of 4 (LDS index rows)
// U8 (grouped heads, head_dim <= 128): the chunk's keys are kept as
// min(key, 255), one byte each, as in k_decode; a head whose group threshold
// reaches 255 re-scans the chunk half at a time with exact 16-bit keys.
template <int D, int G, bool BF, bool U8 = false>
__global__ __launch_bounds__(kDecodeThreads) void k_decode_gs(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint8_t* __restrict__ k_codes, int Hq, int Hkv, int64_t cap, int64_t n_ctx, int chunk,
    int n_chunks, int budget, int cmax, float qscale, uint16_t* __restrict__ ghist,
    float* __restrict__ part, uint32_t* __restrict__ arrive_hist,
    uint32_t* __restrict__ arrive_part, uint32_t* __restrict__ status, uint32_t max_polls,
    int32_t* __restrict__ idx, void* __restrict__ out, int n_sink, int n_recent, EncodeRule rule,
    uint64_t* __restrict__ stamps) {

  constexpr int NT = kDecodeThreads, NW = NT / kWave;
  constexpr int NB = kNbins(D), NBP = kNbinsPadded(D), NBH = kNbinsHist(D), W = D / 16;
  static_assert(G <= kTmpWords - kTmpGroupCounts, "per-head counts live in s_tmp");
  constexpr int E = D / 64, kLanesPerWord = 16 / E, PW = 2 + D, PWP = (PW + 3) & ~3;
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* s_tmp = reinterpret_cast<uint32_t*>(smem);
  uint32_t* s_sums = s_tmp + kTmpWords;
  // phase stamps: 0 entry, 2 scan end, 3 histograms published, 4 group
  // complete, 5 selection done, 9-10 inside attend_rows, 11 partial handed
  // over, 12 merged output stored
  const PhaseStamps ps(stamps, kPhaseDecode, s_tmp);
  ps.mark(0);
  uint32_t* sq = s_sums + 32;
  uint32_t* shist = sq + G * W;
  uint32_t* s_tot = shist + G * NBP;  // one head's group counts per bin: all chunks, chunks before
  uint32_t* s_bef = s_tot + NBP;
  int32_t* sidx = reinterpret_cast<int32_t*>(s_bef + NBP);
  uint8_t* region = reinterpret_cast<uint8_t*>(sidx + G * cmax);
  static_assert(!U8 || (G >= 2 && D <= 128), "8-bit key variant");
  uint16_t* sdist = reinterpret_cast<uint16_t*>(region);  // scan and selection
  uint8_t* sdist8 = region;                               // U8: [G][chunk] bytes
  float* s_part = reinterpret_cast<float*>(region);       // attention, after selection
  float* s_res = s_part + NW * PW + NT / 16;
  float* s_merge = reinterpret_cast<float*>(region);      // merge, last workgroup

  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int c = (lin % n_chunks + lin / n_chunks) % n_chunks;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const int grp = b * Hkv + hkv;
  const int64_t row0 = (int64_t)b * Hq + (int64_t)hkv * G;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  for (int i = threadIdx.x; i < G * NBP; i += NT) shist[i] = 0;
  // as k_decode: query, first batch of codes, then the query's encoding
  static_assert(G <= NW, "one wavefront per query head");
  const int gq = wid < G ? wid : G - 1;
  const uint4 qraw = load_elems_raw<E, BF>(q, (row0 + gq) * D + lane * E);
  const int64_t t0 = (int64_t)c * chunk;
  const int valid = (int)min((int64_t)chunk, n_ctx - t0);
  const uint8_t* kbase = k_codes + (((int64_t)b * Hkv + hkv) * cap + t0) * (D / 4);
  const ContigCodes src{reinterpret_cast<const uint4*>(kbase)};
  uint4 first[kDecodeScanDepth];
  scan_load<NT, kDecodeScanDepth>(src, valid * (D / 64), 0, first);
  __builtin_amdgcn_sched_barrier(0);
  if (wid < G) {
    float y[E];
    widen_elems<E, BF>(qraw, y);
    const uint32_t word = wave_encode<D>(y, rule.rotate, rule.alpha_of(hkv));
    if (lane % kLanesPerWord == 0) sq[wid * W + lane / kLanesPerWord] = word;
  }
  lds_sync();
  QPlanes qp[G];
  load_qplanes<D, G>(sq, qp);
  const KeepRange keep(t0, valid, n_sink, n_ctx - n_recent);
  const auto sink = [&](int g, int tok, uint32_t key) {
    sdist[g * chunk + tok] = (uint16_t)key;
    atomicAdd(&shist[g * NBP + key], 1u);
  };
  if constexpr (U8) {
    if (keep.keeps_none(valid))
      scan_chunk_u8<D, G, NT, kDecodeScanDepth>(
          src, valid, qp, [](int, uint32_t d) { return d + 1u; }, shist, NBP, sdist8, chunk,
          &first);
    else
      scan_chunk_u8<D, G, NT, kDecodeScanDepth>(
          src, valid, qp, [&](int tok, uint32_t d) { return keep.key(tok, d); }, shist, NBP,
          sdist8, chunk, &first);
  } else if (keep.keeps_none(valid))
    scan_chunk<D, G, NT, kDecodeScanDepth>(
        src, valid, qp, [&](int g, int tok, uint32_t d) { sink(g, tok, d + 1u); }, &first);
  else
    scan_chunk<D, G, NT, kDecodeScanDepth>(
        src, valid, qp, [&](int g, int tok, uint32_t d) { sink(g, tok, keep.key(tok, d)); },
        &first);
  lds_sync();
  ps.mark(2);

  // publish this chunk's histograms as u16 rows (counts <= chunk < 2^16)
  for (int i = threadIdx.x; i < G * (NBH / 8); i += NT) {
    const int g = i / (NBH / 8), b0 = (i % (NBH / 8)) * 8;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lo = b0 + 2 * j, hi = lo + 1;
      w[j] = (lo < NB ? shist[g * NBP + lo] : 0u) | ((hi < NB ? shist[g * NBP + hi] : 0u) << 16);
    }
    uint16_t* dst = ghist + ((row0 + g) * n_chunks + c) * NBH;
    store_shared_x4(make_rsrc(dst, NBH * 2), (uint32_t)b0 * 2u, u32x4{w[0], w[1], w[2], w[3]});
  }
  // a wait that gave up leaves the group's histograms possibly incomplete:
  // this workgroup then keeps no rows (and writes no indices), publishes an
  // empty partial and runs to its end, so the counters are still reset
  ps.mark(3);
  const bool complete = arrive_and_wait<NT>(&arrive_hist[grp], n_chunks, status, max_polls,
                                            s_tmp);
  ps.mark(4);

  // group thresholds; this chunk's share of each query head's selection
  const int bsel = (int)min((int64_t)budget, n_ctx);
  uint32_t* s_cnt = s_tmp + kTmpGroupCounts;  // rows kept per query head
  if (!complete && (int)threadIdx.x < G) s_cnt[threadIdx.x] = 0;
  uint32_t* s_grp = s_sums;  // per head: t, lt, lt_before, ties_before
  if constexpr (G == 1) {
    // one head: 16-byte row segments (8 bins of one chunk), one per thread,
    // summed into LDS with atomics, and the threshold with its counts in the
    // chunks before this one from find_group_threshold
    if (complete) {
      for (int i = threadIdx.x; i < 2 * NBP; i += NT) s_tot[i] = 0;
      lds_sync();
      constexpr int SEG = NBH / 8;
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(ghist + row0 * n_chunks * NBH, (uint32_t)(n_chunks * NBH * 2));
      for (int i0 = 0; i0 < n_chunks * SEG; i0 += NT) {
        const int i = i0 + (int)threadIdx.x;
        const int cc = i / SEG, b0 = (i % SEG) * 8;
        u32x4 h = {0u, 0u, 0u, 0u};
        if (i < n_chunks * SEG) h = load_shared_x4(r, (uint32_t)(cc * NBH + b0) * 2u);
        const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t x = (hw[j >> 1] >> (16 * (j & 1))) & 0xffffu;
          if (x != 0u && b0 + j < NB) {
            atomicAdd(&s_tot[b0 + j], x);
            if (cc < c) atomicAdd(&s_bef[b0 + j], x);
          }
        }
      }
      lds_sync();
      const uint32_t tot = (int)threadIdx.x < NB ? s_tot[threadIdx.x] : 0u;
      const uint32_t bef = (int)threadIdx.x < NB ? s_bef[threadIdx.x] : 0u;
      const GroupThreshold gt =
          find_group_threshold<NT>(tot, bef, NB, (uint32_t)bsel, s_sums, s_tmp);
      // (find_group_threshold ends with a barrier after its last use of s_sums)
      if (threadIdx.x == 0) {
        s_grp[0] = (uint32_t)gt.t;
        s_grp[1] = gt.lt;
        s_grp[2] = gt.lt_before;
        s_grp[3] = gt.ties_before;
      }
    }
    lds_sync();
  } else {
    // the group's histograms summed for every query head at once, all loads in
    // one round: thread i takes one 8-bin segment (i % (G * SEG)) of one head
    // and every P-th chunk from i / (G * SEG), adds its sums into s_grp_tot
    // (this chunk's own rows, published above, are no longer needed) and
    // keeps in registers its sum over those of its chunks before this one.
    // s_grp (in s_sums): per head t, lt, lt_before, ties_before.
    constexpr int SEG = NBH / 8, SEGS = G * SEG, P = NT / SEGS;
    static_assert(P >= 1, "one histogram segment per thread at least");
    uint32_t* s_grp_tot = shist;
    const int hseg = (int)threadIdx.x < P * SEGS ? (int)threadIdx.x % SEGS : -1;
    const int hq = (int)threadIdx.x / SEGS;
    const int hg = hseg >= 0 ? hseg / SEG : 0, hb0 = hseg >= 0 ? (hseg - hg * SEG) * 8 : 0;
    uint32_t bef8[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (complete) {
      for (int i = threadIdx.x; i < G * NBP; i += NT) s_grp_tot[i] = 0u;
      if ((int)threadIdx.x < 4 * G) s_grp[threadIdx.x] = 0u;
    }
    lds_sync();
    if (complete && hseg >= 0) {
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(ghist + (row0 + hg) * n_chunks * NBH, (uint32_t)(n_chunks * NBH * 2));
      uint32_t tot8[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      constexpr int UL = 8;  // segment loads in flight per thread
      for (int c0 = hq; c0 < n_chunks; c0 += UL * P) {
        u32x4 h[UL];
#pragma unroll
        for (int u = 0; u < UL; ++u) {
          const int cc = c0 + u * P;
          h[u] = cc < n_chunks ? load_shared_x4(r, (uint32_t)(cc * NBH + hb0) * 2u)
                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UL; ++u) {
          const uint32_t hw[4] = {h[u].x, h[u].y, h[u].z, h[u].w};
          const bool before = c0 + u * P < c;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t x = (hw[j >> 1] >> (16 * (j & 1))) & 0xffffu;
            tot8[j] += x;
            bef8[j] += before ? x : 0u;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (hb0 + j < NB && tot8[j] != 0u) atomicAdd(&s_grp_tot[hg * NBP + hb0 + j], tot8[j]);
    }
    lds_sync();
    // thresholds: wavefront g scans head g's summed bins
    if (complete && wid < G) {
      constexpr int BPL = (NB + kWave - 1) / kWave;
      const uint32_t* h = s_grp_tot + wid * NBP;
      uint32_t v[BPL], sum = 0;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        const int bin = lane * BPL + j;
        v[j] = bin < NB ? h[bin] : 0u;
        sum += v[j];
      }
      const uint32_t incl = wave_scan_incl(sum), excl = incl - sum;
      const uint32_t K = (uint32_t)bsel;
      if (excl < K && K <= incl) {
        uint32_t acc = excl, lt = 0;
        int tb = 0;
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
          if (acc < K && K <= acc + v[j]) {
            tb = lane * BPL + j;
            lt = acc;
          }
          acc += v[j];
        }
        s_grp[4 * wid] = (uint32_t)tb;
        s_grp[4 * wid + 1] = lt;
      }
    }
    lds_sync();
    // the chunks before this one: their counts below and at each threshold,
    // summed over each wavefront first (one LDS atomic per wavefront and head
    // instead of one per thread on the same two words)
    if (complete) {
      uint32_t lt_b = 0, eq_b = 0;
      if (hseg >= 0) {
        const int tb = (int)s_grp[4 * hg];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          lt_b += hb0 + j < tb ? bef8[j] : 0u;
          eq_b += hb0 + j == tb ? bef8[j] : 0u;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const bool here = hseg >= 0 && hg == g;
        const uint32_t sl = __builtin_amdgcn_readlane(wave_scan_incl(here ? lt_b : 0u), kWave - 1);
        const uint32_t se = __builtin_amdgcn_readlane(wave_scan_incl(here ? eq_b : 0u), kWave - 1);
        if (lane == 0) {
          if (sl) atomicAdd(&s_grp[4 * g + 2], sl);
          if (se) atomicAdd(&s_grp[4 * g + 3], se);
        }
      }
    }
    lds_sync();
  }
  // this chunk's share of head g's threshold ties and where its tokens start
  // in the ascending selection (no subtraction wraps)
  const auto share = [&](int g, uint32_t& mine_q, uint32_t& off) {
    const uint32_t quota = (uint32_t)bsel - s_grp[4 * g + 1];  // ties the group keeps
    const uint32_t tb = s_grp[4 * g + 3], before = tb < quota ? tb : quota;
    mine_q = quota - before;
    off = s_grp[4 * g + 2] + before;
  };
  bool heads_at_once = false;
  if constexpr (U8) {
    heads_at_once = complete;
#pragma unroll
    for (int g = 0; g < G; ++g) heads_at_once = heads_at_once && s_grp[4 * g] < (uint32_t)kKeySat;
  }
  if (heads_at_once) {
    // every head's share in one pass over the byte keys (the summed
    // histograms in shist are no longer needed: their rows hold the prefix)
    collect_heads_u8<NT, G>(
        sdist8, chunk, valid, [&](int g) { return s_grp[4 * g]; },
        [&](int g) {
          uint32_t mq, off;
          share(g, mq, off);
          return mq;
        },
        shist,
        [&](int g, uint32_t pos, uint32_t t, uint32_t) {
          const int32_t tok = (int32_t)(t0 + t);
          sidx[g * cmax + pos] = tok;
          if (idx) {
            uint32_t mq, off;
            share(g, mq, off);
            idx[(row0 + g) * budget + off + pos] = tok;
          }
        },
        s_cnt);
    if (idx && c == 0)
      for (int j = (int)threadIdx.x; j < G * (budget - bsel); j += NT) {
        const int g = j / (budget - bsel);
        idx[(row0 + g) * budget + bsel + (j - g * (budget - bsel))] = -1;
      }
  }
  for (int g = 0; g < (complete && !heads_at_once ? G : 0); ++g) {
    const int64_t row = row0 + g;
    const GroupThreshold gt{(int)s_grp[4 * g], s_grp[4 * g + 1], s_grp[4 * g + 2],
                            s_grp[4 * g + 3]};
    const uint32_t quota = (uint32_t)bsel - gt.lt;  // ties at t the whole group keeps
    // ties kept by the chunks before, then this chunk's share (no subtraction wraps)
    const uint32_t before = gt.ties_before < quota ? gt.ties_before : quota;
    const uint32_t mine_q = quota - before;
    const uint32_t off = gt.lt_before + before;
    int32_t* sg = sidx + g * cmax;
    int32_t* ig = idx ? idx + row * budget + off : nullptr;
    uint32_t kept = 0;
    if constexpr (U8) {
      if (gt.t < kKeySat) {
        kept = chunk_collect_u8<NT>(sdist8 + g * chunk, valid, gt.t, mine_q, s_tmp,
                                    [&](uint32_t pos, uint32_t t, uint32_t) {
                                      const int32_t tok = (int32_t)(t0 + t);
                                      sg[pos] = tok;
                                      if (ig) ig[pos] = tok;
                                    });
      } else if constexpr (3 * D + 1 >= kKeySat) {
        // exact 16-bit keys of head g, half a chunk at a time, written over
        // its own byte keys (a half of 16-bit keys fills one head's bytes)
        const int kHalf = chunk / 2;  // <= NT * kCompactTpt tokens
        uint16_t* sd16 = reinterpret_cast<uint16_t*>(sdist8 + g * chunk);
        uint32_t* s_half = s_tmp + kTmpHalfTotals;  // chunk_collect's totals
        QPlanes qh[G];
        load_qplanes<D, G>(sq, qh);
        uint32_t lt_prev = 0, eq_prev = 0;
        for (int h0 = 0; h0 < valid; h0 += kHalf) {
          const int hv = min(kHalf, valid - h0);
          lds_sync();
          scan_chunk<D, G, NT, kDecodeScanDepth>(
              ContigCodes{src.p + (int64_t)h0 * (D / 64)}, hv, qh,
              [&](int gg, int tok, uint32_t d) {
                if (gg == g) sd16[tok] = (uint16_t)keep.key(h0 + tok, d);
              });
          lds_sync();
          const uint32_t taken = eq_prev < mine_q ? eq_prev : mine_q, hoff = lt_prev + taken;
          kept += chunk_collect<NT>(sd16, hv, gt.t, mine_q - taken, s_tmp,
                                    [&](uint32_t pos, uint32_t t, uint32_t) {
                                      const int32_t tok = (int32_t)(t0 + h0 + (int)t);
                                      sg[hoff + pos] = tok;
                                      if (ig) ig[hoff + pos] = tok;
                                    },
                                    nullptr, s_half);
          lds_sync();
          const uint32_t tot = s_half[0];
          lt_prev += tot & 0xffffu;
          eq_prev += tot >> 16;
        }
      }
    } else {
      kept = chunk_collect<NT>(sdist + g * chunk, valid, gt.t, mine_q, s_tmp,
                               [&](uint32_t pos, uint32_t t, uint32_t) {
                                 const int32_t tok = (int32_t)(t0 + t);
                                 sg[pos] = tok;
                                 if (ig) ig[pos] = tok;
                               });
    }
    if (threadIdx.x == 0) s_cnt[g] = kept;
    if (idx && c == 0)
      for (int j = bsel + (int)threadIdx.x; j < budget; j += NT) idx[row * budget + j] = -1;
  }
  lds_sync();  // index rows complete; the distances are no longer needed
  ps.mark(5);

  const int64_t kvrow0 = ((int64_t)b * Hkv + hkv) * cap;
  for (int g = 0; g < G; ++g) {
    const int64_t row = row0 + g;
    attend_rows<D, BF, NT>(q, k, v, row * D, kvrow0, cap, sidx + g * cmax, (int)s_cnt[g], qscale,
                           s_part, s_res, RowOverride{}, PageMap{}, &ps);
    lds_to_shared<NT>(reinterpret_cast<uint32_t*>(part + (row * n_chunks + c) * PWP),
                      reinterpret_cast<const uint32_t*>(s_res), PWP);
  }
  const bool last = arrive_last<NT>(&arrive_part[grp], n_chunks, s_tmp);
  ps.mark(11);
  if (!last) {
    ps.flush();
    return;
  }
  // merge: every head's chunk partials by log-sum-exp, all heads at once;
  // tiles of nt chunks (the whole group when the chunk's key region holds
  // it) pass through LDS, thread j merging dimension j % D of head j / D.
  // One head: tiles of kGsMergeTile partials, thread j < D merging dim j.
  if constexpr (G == 1) {
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int c0 = 0; c0 < n_chunks; c0 += kGsMergeTile) {
      const int nt = min(kGsMergeTile, n_chunks - c0);
      lds_sync();
      shared_to_lds<NT>(reinterpret_cast<uint32_t*>(s_merge),
                        reinterpret_cast<const uint32_t*>(part + (row0 * n_chunks + c0) * PWP),
                        nt * PWP);
      lds_sync();
      if ((int)threadIdx.x < D) {
        for (int i = 0; i < nt; ++i) {
          const float mi = s_merge[i * PWP];
          if (mi == -INFINITY) continue;
          const float Mn = fmaxf(M, mi);
          const float a = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
          const float bb = exp2f(mi - Mn);
          L = L * a + s_merge[i * PWP + 1] * bb;
          O = O * a + s_merge[i * PWP + 2 + threadIdx.x] * bb;
          M = Mn;
        }
      }
    }
    if ((int)threadIdx.x < D) store_out<BF>(out, row0 * D + threadIdx.x, L > 0.0f ? O / L : 0.0f);
  } else {
    const int region_words = max(G * chunk * (U8 ? 1 : 2) / 4, kGsMergeTile * PWP);
    const int nt_max = max(1, region_words / (G * PWP));
    constexpr int PAIRS = (G * D + NT - 1) / NT;
    float M[PAIRS], L[PAIRS], O[PAIRS];
#pragma unroll
    for (int u = 0; u < PAIRS; ++u) {
      M[u] = -INFINITY;
      L[u] = 0.0f;
      O[u] = 0.0f;
    }
    for (int c0 = 0; c0 < n_chunks; c0 += nt_max) {
      const int nt = min(nt_max, n_chunks - c0);
      lds_sync();
      if (nt == n_chunks) {  // the group's rows are contiguous
        shared_to_lds<NT>(reinterpret_cast<uint32_t*>(s_merge),
                          reinterpret_cast<const uint32_t*>(part + row0 * n_chunks * PWP),
                          G * n_chunks * PWP);
      } else {
        for (int g = 0; g < G; ++g)
          shared_to_lds<NT>(reinterpret_cast<uint32_t*>(s_merge + g * nt * PWP),
                            reinterpret_cast<const uint32_t*>(part + ((row0 + g) * n_chunks + c0) * PWP),
                            nt * PWP);
      }
      lds_sync();
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) {
        const int j = (int)threadIdx.x + u * NT;
        if (j < G * D) {
          const int g = j / D, d = j - g * D;
          const float* pg = s_merge + g * nt * PWP;
          for (int i = 0; i < nt; ++i) {
            const float mi = pg[i * PWP];
            if (mi == -INFINITY) continue;
            const float Mn = fmaxf(M[u], mi);
            const float a = (M[u] == -INFINITY) ? 0.0f : exp2f(M[u] - Mn);
            const float bb = exp2f(mi - Mn);
            L[u] = L[u] * a + pg[i * PWP + 1] * bb;
            O[u] = O[u] * a + pg[i * PWP + 2 + d] * bb;
            M[u] = Mn;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < PAIRS; ++u) {
      const int j = (int)threadIdx.x + u * NT;
      if (j < G * D) {
        const int g = j / D, d = j - g * D;
        store_out<BF>(out, (row0 + g) * D + d, L[u] > 0.0f ? O[u] / L[u] : 0.0f);
      }
    }
  }
  if (threadIdx.x == 0) {
    arrive_hist[grp] = 0;
    arrive_part[grp] = 0;
  }
  ps.mark(12);
  ps.flush();
}

// ---------------------------------------------------------- reference read
// adamas_stream_read: each workgroup streams one contiguous slice of the
// buffer with the decode scan's loads (16 bytes per thread, kDecodeScanDepth
// in flight, non-temporal) and writes the XOR of what it read, so the reads
// cannot be dropped.
constexpr int kStreamThreads = 1024;
// (internal linkage: every translation unit that includes this header gets
// its own copy; only the library's entry point launches it)
static __global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4* __restrict__ src,
                                                                int64_t units, int64_t per_block,
                                                                uint32_t* __restrict__ sink) {
  constexpr int U = kDecodeScanDepth;
  const int64_t u0 = (int64_t)blockIdx.x * per_block;
  const int64_t u1 = min(u0 + per_block, units);
  uint32_t acc = 0;
  for (int64_t base = u0; base < u1; base += (int64_t)kStreamThreads * U) {
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t u = base + (int64_t)j * kStreamThreads + threadIdx.x;
      w[j] = load_stream(src + (u < u1 ? u : u1 - 1));
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t u = base + (int64_t)j * kStreamThreads + threadIdx.x;
      if (u < u1) acc ^= w[j].x ^ w[j].y ^ w[j].z ^ w[j].w;  // clamped loads repeat a unit
    }
  }
  __shared__ uint32_t s_acc[kStreamThreads / kWave];
  for (int m = 1; m < kWave; m <<= 1) acc ^= __shfl_xor(acc, m);
  if ((threadIdx.x & (kWave - 1)) == 0) s_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int i = 0; i < kStreamThreads / kWave; ++i) x ^= s_acc[i];
    sink[blockIdx.x] = x;
  }
}

}  // namespace adm
