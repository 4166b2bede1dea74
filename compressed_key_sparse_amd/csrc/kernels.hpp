// kernels.hpp -- the gfx950 kernels of the ADAMAS decode path.
//
// Citations refer to the ADAMAS article (www.lnwmold.com/news/826806) by its
// numbered sections: §2.1 Hadamard rotation, §2.2 bucketing, §2.3 Manhattan
// distance, §3.1 packed code cache, §5.2 token budget, §6 final attention.
#pragma once

#include "device_common.hpp"

namespace adm {

constexpr int kNbins(int D) { return 3 * D + 1; }
constexpr int kNbinsPadded(int D) { return (3 * D + 1 + 3) & ~3; }

// ------------------------------------------------------------------ encode
// §2.1 + §2.2 + §3.1 for keys (or queries): one wavefront per vector,
// grid-stride over the batch*heads*n vectors of x[batch*heads][n][D].
template <int D>
__global__ __launch_bounds__(kBlock) void k_encode(const void* __restrict__ x, int is_bf16,
                                                   int64_t n, int64_t nvec,
                                                   uint8_t* __restrict__ codes, int64_t cap,
                                                   int64_t pos, void* __restrict__ copy) {
  constexpr int E = D / 64;
  constexpr int kLanesPerWord = 16 / E;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nwaves = (int64_t)gridDim.x * (kBlock / kWave);
  for (int64_t v = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave; v < nvec; v += nwaves) {
    const int64_t bh = v / n;
    const int64_t row = bh * cap + pos + (v - bh * n);
    const int64_t src = v * D + lane * E;
    if (copy != nullptr) {
      const int64_t dst = row * D + lane * E;
      if (is_bf16) {
        if constexpr (E == 2)
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(copy) + dst) =
              *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(x) + src);
        else
          static_cast<uint16_t*>(copy)[dst] = static_cast<const uint16_t*>(x)[src];
      } else {
        if constexpr (E == 2)
          *reinterpret_cast<uint2*>(static_cast<float*>(copy) + dst) =
              *reinterpret_cast<const uint2*>(static_cast<const float*>(x) + src);
        else
          static_cast<float*>(copy)[dst] = static_cast<const float*>(x)[src];
      }
    }
    float y[E];
    load_elems<E>(x, is_bf16 != 0, src, y);
    const uint32_t word = wave_encode<D>(y);
    if (lane % kLanesPerWord == 0)
      reinterpret_cast<uint32_t*>(codes + row * (D / 4))[lane / kLanesPerWord] = word;
  }
}

// -------------------------------------------------------------------- scan
// §2.3: stream one chunk of packed key codes and produce, for each of the G
// query heads sharing this KV head, the Manhattan distance of every token.
// Codes are read as 16-byte units (64 codes); at D = 128 a token is two units
// held by a lane pair whose partial sums are added with a DPP swap.  Loads of
// U units per thread are issued before any of them is used.
template <int D, int G, int U, class Sink>
ADM_DEV void scan_chunk(const uint8_t* __restrict__ kbase, int valid, const QPlanes (&qp)[G],
                        Sink&& sink) {
  constexpr int kUnitsPerToken = D / 64;
  const int units = valid * kUnitsPerToken;
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(kbase);
  for (int base = 0; base < units; base += kBlock * U) {
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = base + j * kBlock + (int)threadIdx.x;
      w[j] = (u < units) ? src[u] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = base + j * kBlock + (int)threadIdx.x;
      const uint32_t p0 = therm_p(w[j].x), p1 = therm_p(w[j].y);
      const uint32_t p2 = therm_p(w[j].z), p3 = therm_p(w[j].w);
      const uint32_t t0 = therm_t(w[j].x, w[j].y), t1 = therm_t(w[j].z, w[j].w);
      uint32_t dg[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        uint32_t s = __popc(p0 ^ qp[g].p[0]);
        s += __popc(p1 ^ qp[g].p[1]);
        s += __popc(p2 ^ qp[g].p[2]);
        s += __popc(p3 ^ qp[g].p[3]);
        s += __popc(t0 ^ qp[g].t[0]);
        s += __popc(t1 ^ qp[g].t[1]);
        if constexpr (kUnitsPerToken == 2) s += swap_pair(s);
        dg[g] = s;
      }
      if (u < units && (kUnitsPerToken == 1 || (threadIdx.x & 1) == 0)) {
#pragma unroll
        for (int g = 0; g < G; ++g) sink(g, u / kUnitsPerToken, dg[g]);
      }
    }
  }
}

// Query planes for this thread's half of the row (D = 128: lane parity picks
// words 0-3 or 4-7; D = 64: the whole row) from packed words in LDS.
template <int D, int G>
ADM_DEV void load_qplanes(const uint32_t* sq, QPlanes (&qp)[G]) {
  constexpr int W = D / 16;
  const int half = (D == 128) ? (int)(threadIdx.x & 1) : 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t* r = sq + g * W + half * 4;
    qp[g] = make_qplanes(r[0], r[1], r[2], r[3]);
  }
}

// ------------------------------------------------------------------- score
// adamas_score: grid (chunks, Hkv, B); query codes already encoded.
template <int D, int G>
__global__ __launch_bounds__(kBlock) void k_score(const uint8_t* __restrict__ q_codes,
                                                  const uint8_t* __restrict__ k_codes, int Hq,
                                                  int Hkv, int64_t cap, int64_t n_ctx, int chunk,
                                                  uint16_t* __restrict__ dist) {
  constexpr int W = D / 16;
  __shared__ uint32_t sq[G * W];
  const int c = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  for (int i = threadIdx.x; i < G * W; i += kBlock)
    sq[i] = reinterpret_cast<const uint32_t*>(
        q_codes + ((int64_t)b * Hq + (int64_t)hkv * G) * (D / 4))[i];
  __syncthreads();
  QPlanes qp[G];
  load_qplanes<D, G>(sq, qp);
  const int64_t t0 = (int64_t)c * chunk;
  const int valid = (int)min((int64_t)chunk, n_ctx - t0);
  const uint8_t* kbase = k_codes + (((int64_t)b * Hkv + hkv) * cap + t0) * (D / 4);
  uint16_t* drow = dist + ((int64_t)b * Hq + (int64_t)hkv * G) * n_ctx + t0;
  scan_chunk<D, G, 4>(kbase, valid, qp, [&](int g, int tok, uint32_t d) {
    drow[(int64_t)g * n_ctx + tok] = (uint16_t)d;
  });
}

// --------------------------------------------------------- §5.2 selection
// Per chunk: keep the chunk's min(budget, valid) best (D, token) as
// candidates; a token in the global top-budget is always in its chunk's
// top-budget, so the union of the chunk candidates contains the answer.  The
// last workgroup of a group (atomic arrival count) selects from the union.
ADM_DEV bool arrive_last(uint32_t* counter, int n_arrivals, uint32_t* s_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(counter, 1u);
    *s_flag = (prev == (uint32_t)(n_arrivals - 1)) ? 1u : 0u;
  }
  __syncthreads();
  const bool last = *s_flag != 0;
  if (last) __threadfence();
  return last;
}

// adamas_select_topk: grid (chunks, Hq, B) over uint16 distances.
template <int D>
__global__ __launch_bounds__(kBlock) void k_select(const uint16_t* __restrict__ dist, int Hq,
                                                   int64_t n_ctx, int chunk, int n_chunks,
                                                   int budget, uint32_t* __restrict__ cand,
                                                   uint32_t* __restrict__ counters,
                                                   int32_t* __restrict__ idx) {
  constexpr int NB = kNbins(D), NBP = kNbinsPadded(D);
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* s_tmp = reinterpret_cast<uint32_t*>(smem);
  uint32_t* shist = s_tmp + 16;
  uint16_t* sdist = reinterpret_cast<uint16_t*>(shist + NBP);
  const int c = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int64_t row = (int64_t)b * Hq + hq;
  for (int i = threadIdx.x; i < NBP; i += kBlock) shist[i] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)c * chunk;
  const int valid = (int)min((int64_t)chunk, n_ctx - t0);
  const uint16_t* drow = dist + row * n_ctx + t0;
  for (int t = threadIdx.x; t < valid; t += kBlock) {
    // values above 3*D break the caller's contract; clamp so LDS stays in bounds
    const uint16_t d = drow[t] < NB ? drow[t] : (uint16_t)(NB - 1);
    sdist[t] = d;
    atomicAdd(&shist[d], 1u);
  }
  __syncthreads();
  const int kmax = min(budget, chunk);
  const int kc = min(budget, valid);
  const Threshold thr = find_threshold(shist, NB, (uint32_t)kc, s_tmp);
  chunk_compact(sdist, valid, chunk / kBlock, thr, (uint32_t)kc - thr.lt,
                cand + (row * n_chunks + c) * kmax, s_tmp);
  if (!arrive_last(&counters[row], n_chunks, &s_tmp[12])) return;
  const int valid_last = (int)(n_ctx - (int64_t)(n_chunks - 1) * chunk);
  final_select(cand + row * n_chunks * kmax, n_chunks, kmax, min(budget, valid_last), chunk,
               (int)min((int64_t)budget, n_ctx), budget, idx + row * budget, shist, NB, s_tmp);
  if (threadIdx.x == 0) counters[row] = 0;
}

// ------------------------------------------------------- fused decode step
// adamas_decode_step, selection half: grid (chunks, Hkv, B).  Each workgroup
// encodes the G query heads of its KV head (§2.1-§2.2, one wavefront per
// head), scans one chunk of codes (§2.3) keeping distances and a histogram in
// LDS, writes the chunk's candidates, and the last workgroup of the KV head
// selects the budget for its G query heads (§5.2).
template <int D, int G>
__global__ __launch_bounds__(kBlock) void k_decode_select(
    const void* __restrict__ q, int q_bf16, const uint8_t* __restrict__ k_codes, int Hq, int Hkv,
    int64_t cap, int64_t n_ctx, int chunk, int n_chunks, int budget, uint32_t* __restrict__ cand,
    uint32_t* __restrict__ counters, int32_t* __restrict__ idx) {
  constexpr int NB = kNbins(D), NBP = kNbinsPadded(D), W = D / 16;
  constexpr int E = D / 64, kLanesPerWord = 16 / E;
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* s_tmp = reinterpret_cast<uint32_t*>(smem);
  uint32_t* sq = s_tmp + 16;
  uint32_t* shist = sq + G * W;
  uint16_t* sdist = reinterpret_cast<uint16_t*>(shist + G * NBP);
  const int c = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  for (int i = threadIdx.x; i < G * NBP; i += kBlock) shist[i] = 0;
  for (int g = wid; g < G; g += kBlock / kWave) {
    float y[E];
    load_elems<E>(q, q_bf16 != 0, ((int64_t)b * Hq + (int64_t)hkv * G + g) * D + lane * E, y);
    const uint32_t word = wave_encode<D>(y);
    if (lane % kLanesPerWord == 0) sq[g * W + lane / kLanesPerWord] = word;
  }
  __syncthreads();
  QPlanes qp[G];
  load_qplanes<D, G>(sq, qp);
  const int64_t t0 = (int64_t)c * chunk;
  const int valid = (int)min((int64_t)chunk, n_ctx - t0);
  const uint8_t* kbase = k_codes + (((int64_t)b * Hkv + hkv) * cap + t0) * (D / 4);
  scan_chunk<D, G, 4>(kbase, valid, qp, [&](int g, int tok, uint32_t d) {
    sdist[g * chunk + tok] = (uint16_t)d;
    atomicAdd(&shist[g * NBP + d], 1u);
  });
  __syncthreads();
  const int kmax = min(budget, chunk);
  const int kc = min(budget, valid);
  for (int g = 0; g < G; ++g) {
    const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
    const Threshold thr = find_threshold(shist + g * NBP, NB, (uint32_t)kc, s_tmp);
    chunk_compact(sdist + g * chunk, valid, chunk / kBlock, thr, (uint32_t)kc - thr.lt,
                  cand + (row * n_chunks + c) * kmax, s_tmp);
  }
  if (!arrive_last(&counters[b * Hkv + hkv], n_chunks, &s_tmp[12])) return;
  const int valid_last = (int)(n_ctx - (int64_t)(n_chunks - 1) * chunk);
  const int bsel = (int)min((int64_t)budget, n_ctx);
  for (int g = 0; g < G; ++g) {
    const int64_t row = (int64_t)b * Hq + (int64_t)hkv * G + g;
    final_select(cand + row * n_chunks * kmax, n_chunks, kmax, min(budget, valid_last), chunk,
                 bsel, budget, idx + row * budget, shist, NB, s_tmp);
    __syncthreads();
  }
  if (threadIdx.x == 0) counters[b * Hkv + hkv] = 0;
}

// ---------------------------------------------------------------- §6 attend
// Split-K gather attention: grid (splits, Hq, B).  A workgroup takes up to
// 32 selected rows; each 16-lane slot owns two rows and every lane D/16
// dimensions.  K and V rows of a slot are loaded before any is used.  Scores
// are kept in the log2 domain (q pre-multiplied by scale*log2(e)); partial
// (m, l, o) triples merge by log-sum-exp, first across slots, then across
// splits by the last-arriving workgroup of the head.
constexpr int kAttnRowsPerSlot = 2;
constexpr int kAttnRows = 16 * kAttnRowsPerSlot;

template <int EL>
ADM_DEV void load_row_slice(const void* base, bool is_bf16, int64_t elem, float (&out)[EL]) {
  if (is_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + elem;
    if constexpr (EL == 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(p);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = bf16_to_f32(ws[i] & 0xffffu);
        out[2 * i + 1] = bf16_to_f32(ws[i] >> 16);
      }
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      out[0] = bf16_to_f32(w.x & 0xffffu);
      out[1] = bf16_to_f32(w.x >> 16);
      out[2] = bf16_to_f32(w.y & 0xffffu);
      out[3] = bf16_to_f32(w.y >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < EL / 4; ++i) {
      const float4 w = p[i];
      out[4 * i] = w.x;
      out[4 * i + 1] = w.y;
      out[4 * i + 2] = w.z;
      out[4 * i + 3] = w.w;
    }
  }
}

struct Softmax {
  float m, l;
};

// Merge (m2, l2, o2) into (m1, l1, o1); m = -inf marks an empty partial.
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

template <int D>
__global__ __launch_bounds__(kBlock) void k_attend(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    int is_bf16, const int32_t* __restrict__ idx, int Hq, int Hkv, int64_t cap, int budget,
    float qscale, float* __restrict__ part, uint32_t* __restrict__ counters,
    void* __restrict__ out) {
  constexpr int EL = D / 16;
  constexpr int RS = kAttnRowsPerSlot;
  __shared__ float s_part[kBlock / kWave][2 + D];
  __shared__ uint32_t s_flag[1];
  const int s = blockIdx.x, hq = blockIdx.y, b = blockIdx.z, S = gridDim.x;
  const int G = Hq / Hkv;
  const int64_t row = (int64_t)b * Hq + hq;
  const int64_t kvrow0 = ((int64_t)b * Hkv + hq / G) * cap;
  const int l16 = threadIdx.x & 15, slot = threadIdx.x >> 4;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const bool bf = is_bf16 != 0;

  float qv[EL];
  load_row_slice<EL>(q, bf, row * D + l16 * EL, qv);
#pragma unroll
  for (int e = 0; e < EL; ++e) qv[e] *= qscale;

  const int r0 = s * kAttnRows;
  const int r1 = min(r0 + kAttnRows, budget);
  int32_t tok[RS];
#pragma unroll
  for (int j = 0; j < RS; ++j) {
    const int r = r0 + slot + 16 * j;
    int32_t t = (r < r1) ? idx[row * budget + r] : -1;
    tok[j] = (t >= 0 && (int64_t)t < cap) ? t : -1;
  }
  float kf[RS][EL], vf[RS][EL];
#pragma unroll
  for (int j = 0; j < RS; ++j) {
    if (tok[j] >= 0) {
      load_row_slice<EL>(k, bf, (kvrow0 + tok[j]) * D + l16 * EL, kf[j]);
      load_row_slice<EL>(v, bf, (kvrow0 + tok[j]) * D + l16 * EL, vf[j]);
    }
  }
  Softmax st{-INFINITY, 0.0f};
  float o[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) o[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < RS; ++j) {
    if (tok[j] >= 0) {  // uniform across the 16 lanes of a slot
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < EL; ++e) dot += qv[e] * kf[j][e];
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) dot += __shfl_xor(dot, m);
      const float M = fmaxf(st.m, dot);
      const float corr = (st.m == -INFINITY) ? 0.0f : exp2f(st.m - M);
      const float p = exp2f(dot - M);
      st.l = st.l * corr + p;
#pragma unroll
      for (int e = 0; e < EL; ++e) o[e] = o[e] * corr + p * vf[j][e];
      st.m = M;
    }
  }
  // merge the four slots of each wavefront (lanes ^16, ^32), then the waves
#pragma unroll
  for (int m = 16; m < kWave; m <<= 1) {
    Softmax other{__shfl_xor(st.m, m), __shfl_xor(st.l, m)};
    float oo[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) oo[e] = __shfl_xor(o[e], m);
    merge_partial<EL>(st, o, other, oo);
  }
  if (lane < 16) {
    if (lane == 0) {
      s_part[wid][0] = st.m;
      s_part[wid][1] = st.l;
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) s_part[wid][2 + l16 * EL + e] = o[e];
  }
  __syncthreads();
  // thread t < D combines the waves for dimension t
  float m_all = -INFINITY, l_all = 0.0f, o_all = 0.0f;
  if (threadIdx.x < D) {
    const int dd = threadIdx.x;
    for (int w = 0; w < kBlock / kWave; ++w) m_all = fmaxf(m_all, s_part[w][0]);
    if (m_all != -INFINITY) {
      for (int w = 0; w < kBlock / kWave; ++w) {
        const float mw = s_part[w][0];
        const float a = (mw == -INFINITY) ? 0.0f : exp2f(mw - m_all);
        l_all += s_part[w][1] * a;
        o_all += s_part[w][2 + dd] * a;
      }
    }
  }
  auto store_out = [&](int dd, float val) {
    if (bf)
      static_cast<uint16_t*>(out)[row * D + dd] = f32_to_bf16(val);
    else
      static_cast<float*>(out)[row * D + dd] = val;
  };
  if (S == 1) {
    if (threadIdx.x < D) store_out(threadIdx.x, l_all > 0.0f ? o_all / l_all : 0.0f);
    return;
  }
  float* my = part + (row * S + s) * (2 + D);
  if (threadIdx.x < D) {
    my[2 + threadIdx.x] = o_all;
    if (threadIdx.x == 0) {
      my[0] = m_all;
      my[1] = l_all;
    }
  }
  if (!arrive_last(&counters[row], S, &s_flag[0])) return;
  if (threadIdx.x < D) {
    const float* ps = part + row * S * (2 + D);
    float M = -INFINITY;
    for (int i = 0; i < S; ++i) M = fmaxf(M, ps[i * (2 + D)]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
      for (int i = 0; i < S; ++i) {
        const float mi = ps[i * (2 + D)];
        const float a = (mi == -INFINITY) ? 0.0f : exp2f(mi - M);
        L += ps[i * (2 + D) + 1] * a;
        O += ps[i * (2 + D) + 2 + threadIdx.x] * a;
      }
    }
    store_out(threadIdx.x, L > 0.0f ? O / L : 0.0f);
  }
  if (threadIdx.x == 0) counters[row] = 0;
}

}  // namespace adm
