// device_common.hpp -- gfx950 device building blocks of the ADAMAS decode path.
//
// Citations refer to the ADAMAS article (www.lnwmold.com/news/826806) by its
// numbered sections: §2.1 Hadamard rotation, §2.2 three-threshold bucketing,
// §2.3 Manhattan distance on 2-bit codes, §3.1 packed code cache, §5.2 token
// budget, §6 final attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define ADM_DEV __device__ __forceinline__

namespace adm {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // every kernel here runs 4 waves per workgroup

// ---------------------------------------------------------------- elements
ADM_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// binary32 -> bfloat16, round to nearest, ties to even (NaN stays NaN).
ADM_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Load `E` consecutive elements starting at element `i` (E in {1, 2}).
template <int E>
ADM_DEV void load_elems(const void* base, bool is_bf16, int64_t i, float (&out)[E]) {
  if (is_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + i;
    if constexpr (E == 2) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      out[0] = bf16_to_f32(w & 0xffffu);
      out[1] = bf16_to_f32(w >> 16);
    } else {
      out[0] = bf16_to_f32(*p);
    }
  } else {
    const float* p = static_cast<const float*>(base) + i;
    if constexpr (E == 2) {
      float2 w = *reinterpret_cast<const float2*>(p);
      out[0] = w.x;
      out[1] = w.y;
    } else {
      out[0] = *p;
    }
  }
}

// ---------------------------------------------------------- §2.1 + §2.2
// One wavefront rotates, buckets and packs one vector of D dims.
// Lane l holds elements l*E .. l*E+E-1 (E = D/64).  The fast Walsh-Hadamard
// transform runs the butterfly stages h = 1, 2, ..., D/2 in that order; at
// each stage the element whose index has bit h clear becomes (lower + upper)
// and its partner becomes (lower - upper), each one binary32 operation, so
// the rotated values are bit-identical to a scalar loop in the same stage
// order (addition is commutative and round-to-nearest is sign-symmetric).
// Stages below E are inside a lane; the rest exchange with lane ^ (h / E).
//
// Bucketing: a = max|y| over the vector, thresholds -0.5a, 0, +0.5a, codes
// 0 if y < -a/2, 1 if y < 0, 2 if y < a/2, else 3 (strict comparisons).
//
// Packing (§3.1): four codes per byte, first code in bits 7..6; returns, on
// the lanes with (lane % (16/E)) == 0, the little-endian 32-bit word
// lane / (16/E) of the packed row (16 codes per word); other lanes return 0.
template <int D>
ADM_DEV uint32_t wave_encode(float (&y)[D / 64]) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        float a = y[e], b = y[e + h];
        y[e] = a + b;
        y[e + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float p = __shfl_xor(y[e], m);
      y[e] = upper ? (p - y[e]) : (y[e] + p);
    }
  }
  float a = fabsf(y[0]);
#pragma unroll
  for (int e = 1; e < E; ++e) a = fmaxf(a, fabsf(y[e]));
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) a = fmaxf(a, __shfl_xor(a, m));
  const float t0 = -0.5f * a;
  const float t2 = 0.5f * a;
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = y[e];
    const uint32_t c = (v < t0) ? 0u : (v < 0.0f) ? 1u : (v < t2) ? 2u : 3u;
    const int i = lane * E + e;                       // dimension index
    const int pos = 8 * ((i >> 2) & 3) + 6 - 2 * (i & 3);  // bit position in its word
    bits |= c << pos;
  }
  constexpr int kLanesPerWord = 16 / E;
#pragma unroll
  for (int m = 1; m < kLanesPerWord; m <<= 1) bits |= __shfl_xor(bits, m);
  return (lane % kLanesPerWord) == 0 ? bits : 0u;
}

// --------------------------------------------------------------- §2.3
// Manhattan distance between 2-bit codes through thermometer bit planes.
// Code c = 2h + l maps to the three bits t1 = [c >= 1] = h|l, t2 = [c >= 2] = h
// and t3 = [c >= 3] = h&l; |a - b| is the number of planes in which a and b
// differ, so a sum of |qc - kc| over 16 codes per 32-bit word is a popcount of
// XORed planes.  Per word the planes t1 (odd bit of each field) and t3 (even
// bit) share one word ("P form"); the t2 planes of two words share one more
// ("T form"): 48 plane bits per 16 codes.
ADM_DEV uint32_t therm_p(uint32_t w) {
  const uint32_t a = w | (w << 1);  // odd bit 2j+1: h | l
  const uint32_t b = w & (w >> 1);  // even bit 2j:  l & h
  return (a & 0xAAAAAAAAu) | (b & 0x55555555u);
}
ADM_DEV uint32_t therm_t(uint32_t w0, uint32_t w1) {
  return (w0 & 0xAAAAAAAAu) | ((w1 >> 1) & 0x55555555u);
}

// Query-side planes for one 16-byte unit (4 words, 64 codes).
struct QPlanes {
  uint32_t p[4];
  uint32_t t[2];
};
ADM_DEV QPlanes make_qplanes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  QPlanes r;
  r.p[0] = therm_p(w0);
  r.p[1] = therm_p(w1);
  r.p[2] = therm_p(w2);
  r.p[3] = therm_p(w3);
  r.t[0] = therm_t(w0, w1);
  r.t[1] = therm_t(w2, w3);
  return r;
}

// Swap values between lane pairs (l, l^1) with a DPP quad permutation.
ADM_DEV uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

// ----------------------------------------------------------- block scans
// Inclusive prefix sum of one u32 per thread over the 256-thread block.
// Uses s_tmp[0..3]; contains two barriers.
ADM_DEV uint32_t block_scan_incl(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == kWave - 1) s_tmp[wid] = v;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) {
    uint32_t x = s_tmp[w];
    pre += (w < wid) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + pre;
}

// ------------------------------------------------------------------ §5.2
// Threshold of a budget over a distance histogram: the smallest t with
// count(D <= t) >= K, and lt = count(D < t).  Requires 1 <= K <= total count.
struct Threshold {
  int t;
  uint32_t lt;
};
ADM_DEV Threshold find_threshold(const uint32_t* hist, int nbins, uint32_t K, uint32_t* s_tmp) {
  const int bpt = (nbins + kBlock - 1) / kBlock;
  const int b0 = threadIdx.x * bpt;
  uint32_t sum = 0;
  for (int i = 0; i < bpt; ++i)
    if (b0 + i < nbins) sum += hist[b0 + i];
  uint32_t tot;
  const uint32_t incl = block_scan_incl(sum, s_tmp, &tot);
  const uint32_t excl = incl - sum;
  if (excl < K && K <= incl) {
    uint32_t c = excl;
    for (int i = 0; i < bpt; ++i) {
      const uint32_t h = hist[b0 + i];
      if (c + h >= K) {
        s_tmp[8] = (uint32_t)(b0 + i);
        s_tmp[9] = c;
        break;
      }
      c += h;
    }
  }
  __syncthreads();
  Threshold r{(int)s_tmp[8], s_tmp[9]};
  __syncthreads();
  return r;
}

// Ordered selection inside one chunk held in LDS.  Keeps every token with
// D < t and the first `quota` tokens (lowest index) with D == t, and writes
// them in token order as (D << 16) | token to out[].  Token i is kept at
// position (#kept-lt before i) + min(#eq before i, quota).
ADM_DEV void chunk_compact(const uint16_t* sdist, int valid, int tpt, Threshold thr,
                           uint32_t quota, uint32_t* out, uint32_t* s_tmp) {
  const int t0 = threadIdx.x * tpt;
  uint32_t lt = 0, eq = 0;
  for (int i = 0; i < tpt; ++i) {
    const int t = t0 + i;
    if (t < valid) {
      const int d = sdist[t];
      lt += d < thr.t;
      eq += d == thr.t;
    }
  }
  uint32_t tot;
  const uint32_t mine = lt | (eq << 16);
  const uint32_t ex = block_scan_incl(mine, s_tmp, &tot) - mine;
  uint32_t ltb = ex & 0xffffu, eqb = ex >> 16;
  for (int i = 0; i < tpt; ++i) {
    const int t = t0 + i;
    if (t < valid) {
      const uint32_t d = sdist[t];
      if ((int)d < thr.t) {
        out[ltb + (eqb < quota ? eqb : quota)] = (d << 16) | (uint32_t)t;
        ++ltb;
      } else if ((int)d == thr.t) {
        if (eqb < quota) out[ltb + eqb] = (d << 16) | (uint32_t)t;
        ++eqb;
      }
    }
  }
}

// Final selection of one head from its chunk candidates.  cand[] holds, per
// chunk c, Kmax entries (D << 16 | token-in-chunk) in token order (the last
// chunk holds k_last), so the array is in global token order.  Keeps the
// bsel smallest (D, token) and writes the tokens, ascending, to idx[0..bsel),
// then -1 up to budget.  shist must hold nbins words of LDS.
ADM_DEV void final_select(const uint32_t* cand, int n_chunks, int kmax, int k_last, int chunk,
                          int bsel, int budget, int32_t* idx, uint32_t* shist, int nbins,
                          uint32_t* s_tmp) {
  const int M = (n_chunks - 1) * kmax + k_last;
  for (int i = threadIdx.x; i < nbins; i += kBlock) shist[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < M; i += kBlock) atomicAdd(&shist[cand[i] >> 16], 1u);
  __syncthreads();
  const Threshold thr = find_threshold(shist, nbins, (uint32_t)bsel, s_tmp);
  const uint32_t quota = (uint32_t)bsel - thr.lt;
  constexpr int kTpt = 16;
  uint32_t carry_lt = 0, carry_eq = 0;
  for (int base = 0; base < M; base += kBlock * kTpt) {
    const int i0 = base + threadIdx.x * kTpt;
    uint32_t lt = 0, eq = 0;
    for (int i = 0; i < kTpt; ++i) {
      if (i0 + i < M) {
        const int d = (int)(cand[i0 + i] >> 16);
        lt += d < thr.t;
        eq += d == thr.t;
      }
    }
    uint32_t tot;
    const uint32_t mine = lt | (eq << 16);
    const uint32_t ex = block_scan_incl(mine, s_tmp, &tot) - mine;
    uint32_t ltb = carry_lt + (ex & 0xffffu), eqb = carry_eq + (ex >> 16);
    for (int i = 0; i < kTpt; ++i) {
      const int j = i0 + i;
      if (j < M) {
        const uint32_t v = cand[j];
        const int d = (int)(v >> 16);
        const int32_t tok = (j / kmax) * chunk + (int32_t)(v & 0xffffu);
        if (d < thr.t) {
          idx[ltb + (eqb < quota ? eqb : quota)] = tok;
          ++ltb;
        } else if (d == thr.t) {
          if (eqb < quota) idx[ltb + eqb] = tok;
          ++eqb;
        }
      }
    }
    carry_lt += tot & 0xffffu;
    carry_eq += tot >> 16;
  }
  for (int j = bsel + threadIdx.x; j < budget; j += kBlock) idx[j] = -1;
}

}  // namespace adm
