// device_common.hpp -- gfx950 device building blocks of the ADAMAS decode path.
//
// Citations refer to the ADAMAS article (www.lnwmold.com/news/826806) by its
// numbered sections: §2.1 Hadamard rotation, §2.2 three-threshold bucketing,
// §2.3 Manhattan distance on 2-bit codes, §3.1 packed code cache, §5.2 token
// budget, §6 final attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define ADM_DEV __device__ __forceinline__
#define ADM_HOST_DEV __host__ __device__

namespace adm {

constexpr int kWave = 64;

// LDS scratch words used by the block-level helpers (s_tmp[0..31]).
constexpr int kTmpWaveSums = 0;   // [0, 16): per-wave partial sums
constexpr int kTmpThrT = 16;      // threshold bin
constexpr int kTmpThrLt = 17;     // count below the threshold
constexpr int kTmpFlag = 20;      // "last arrival" flag
constexpr int kTmpStamps = 32;    // phase stamps (measurement build only)

// Workgroup barrier for LDS exchanges only.  __syncthreads() also orders
// global memory, which on this target waits for every outstanding vector
// load and store; tail phases keep global loads in flight across their LDS
// barriers, so they synchronise LDS alone.
ADM_DEV void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------ phase stamps
// A measurement build (compiled with -DADAMAS_PHASES=1, libadamas_phases.so)
// records, per workgroup, the device's constant-rate wall clock at marked
// points of a kernel.  Thread 0 keeps the stamps in LDS (s_tmp[kTmpStamps,
// +2*kPhaseSlots)) and copies them to the caller's buffer when the
// workgroup exits (flush), so no global store is in flight when the kernel's
// own code waits for its memory operations; the product build compiles every
// mark away and reserves no LDS for them.  Buffer layout: [kernel
// region][workgroup][kPhaseSlots] u64, 0 = not reached.
#if defined(ADAMAS_PHASES) && ADAMAS_PHASES
constexpr bool kPhases = true;
#else
constexpr bool kPhases = false;
#endif
constexpr int kPhaseSlots = 24;
constexpr int kTmpWords = kTmpStamps + (kPhases ? 2 * kPhaseSlots : 0);
constexpr int kPhaseMaxWorkgroups = 8192;  // per kernel region
enum PhaseRegion { kPhaseDecode = 0, kPhaseSplit = 1, kPhaseAttend = 2, kPhaseRegions = 3 };
struct PhaseStamps {
  uint64_t* row;  // this workgroup's slots in the caller's buffer, or null
  uint64_t* lds;  // the stamps while the workgroup runs
  ADM_DEV PhaseStamps(uint64_t* buf, int region, uint32_t* s_tmp) : row(nullptr), lds(nullptr) {
    if constexpr (kPhases) {
      const int64_t wg = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
      if (buf != nullptr && wg < kPhaseMaxWorkgroups) {
        row = buf + ((int64_t)region * kPhaseMaxWorkgroups + wg) * kPhaseSlots;
        lds = reinterpret_cast<uint64_t*>(s_tmp + kTmpStamps);
        if (threadIdx.x == 0)
          for (int s = 0; s < kPhaseSlots; ++s) lds[s] = 0;
      }
    }
  }
  ADM_DEV void mark(int slot) const {
    if constexpr (kPhases) {
      if (lds != nullptr && threadIdx.x == 0) lds[slot] = wall_clock64();
    }
  }
  // the latest of the workgroup's wavefronts to reach this point (slots
  // marked this way must be followed by a workgroup barrier before flush)
  ADM_DEV void mark_last_wave(int slot) const {
    if constexpr (kPhases) {
      if (lds != nullptr && (threadIdx.x & (kWave - 1)) == 0)
        atomicMax(reinterpret_cast<unsigned long long*>(lds + slot),
                  (unsigned long long)wall_clock64());
    }
  }
  // copy the stamps out; at every exit of the workgroup
  ADM_DEV void flush() const {
    if constexpr (kPhases) {
      if (row != nullptr && threadIdx.x == 0)
        for (int s = 0; s < kPhaseSlots; ++s) row[s] = lds[s];
    }
  }
};

// ---------------------------------------------------------------- elements
ADM_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// binary32 -> bfloat16, round to nearest, ties to even (NaN stays NaN).
ADM_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Load `E` consecutive elements starting at element `i` (E in {1, 2, 4}).
template <int E>
ADM_DEV void load_elems(const void* base, bool is_bf16, int64_t i, float (&out)[E]) {
  if (is_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + i;
    if constexpr (E == 4) {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      out[0] = bf16_to_f32(w.x & 0xffffu);
      out[1] = bf16_to_f32(w.x >> 16);
      out[2] = bf16_to_f32(w.y & 0xffffu);
      out[3] = bf16_to_f32(w.y >> 16);
    } else if constexpr (E == 2) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      out[0] = bf16_to_f32(w & 0xffffu);
      out[1] = bf16_to_f32(w >> 16);
    } else {
      out[0] = bf16_to_f32(*p);
    }
  } else {
    const float* p = static_cast<const float*>(base) + i;
    if constexpr (E == 4) {
      const float4 w = *reinterpret_cast<const float4*>(p);
      out[0] = w.x;
      out[1] = w.y;
      out[2] = w.z;
      out[3] = w.w;
    } else if constexpr (E == 2) {
      float2 w = *reinterpret_cast<const float2*>(p);
      out[0] = w.x;
      out[1] = w.y;
    } else {
      out[0] = *p;
    }
  }
}

// The same elements as raw bits (issue the load now, widen later with
// widen_elems): E * 2 or E * 4 bytes in a uint4 (only the bytes loaded are
// set; the rest are zero).
template <int E, bool BF>
ADM_DEV uint4 load_elems_raw(const void* base, int64_t i) {
  if constexpr (BF) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + i;
    if constexpr (E == 4) {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      return make_uint4(w.x, w.y, 0u, 0u);
    } else if constexpr (E == 2) {
      return make_uint4(*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u);
    } else {
      return make_uint4(*p, 0u, 0u, 0u);
    }
  } else {
    const float* p = static_cast<const float*>(base) + i;
    if constexpr (E == 4) {
      return *reinterpret_cast<const uint4*>(p);
    } else if constexpr (E == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      return make_uint4(w.x, w.y, 0u, 0u);
    } else {
      return make_uint4(__float_as_uint(*p), 0u, 0u, 0u);
    }
  }
}
template <int E, bool BF>
ADM_DEV void widen_elems(uint4 raw, float (&out)[E]) {
  const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (BF)
      out[e] = bf16_to_f32((e & 1) ? (r[e >> 1] >> 16) : (r[e >> 1] & 0xffffu));
    else
      out[e] = __uint_as_float(r[e]);
  }
}

// Data handed from one workgroup to another within a launch (candidate
// lists, attention partials) is written and read with device-scope coherent
// accesses (the sc1 cache policy): they are coherent across the XCDs'
// separate L2 caches by themselves, so the hand-off needs no L2 write-back or
// invalidation.  Every wavefront of the writer waits for its own stores to be
// acknowledged (wait_vmem, below) before the workgroup barrier that precedes
// the arrival count, so the count is never visible before the data it
// announces.  Whole 16-byte rows are moved through buffer instructions (a
// 4-byte coherent store costs a full line of write traffic).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCachePolicyCoherent = 16;       // sc1: device-scope coherence
constexpr int kBufferDword3 = 0x00020000;      // raw 32-bit buffer (GFX9 layout)

ADM_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           kBufferDword3);
}
ADM_DEV void store_shared_x4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, kCachePolicyCoherent);
}
ADM_DEV u32x4 load_shared_x4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kCachePolicyCoherent);
}
ADM_DEV uint32_t load_shared_b32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kCachePolicyCoherent);
}
ADM_DEV uint32_t load_shared_b16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)byte_off, 0, kCachePolicyCoherent);
}
ADM_DEV void store_shared(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copy n u32 (n % 4 == 0) between LDS and a coherent global buffer (16-byte
// rows; the global side is 16-byte aligned).
template <int NT>
ADM_DEV void lds_to_shared(uint32_t* dst_global, const uint32_t* src_lds, int n) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(dst_global, (uint32_t)n * 4u);
  for (int i = threadIdx.x; i < n / 4; i += NT) {
    const uint4 v = reinterpret_cast<const uint4*>(src_lds)[i];
    store_shared_x4(r, (uint32_t)i * 16u, u32x4{v.x, v.y, v.z, v.w});
  }
}

// Copy n u32 (n % 4 == 0) written by other workgroups of this launch into LDS,
// up to 8 outstanding 16-byte coherent loads per thread.  The barrier between
// the loads and the LDS stores keeps the compiler from sinking each load into
// its store (which would serialize them).  One barrier per 32*NT elements.
template <int NT>
ADM_DEV void shared_to_lds(uint32_t* dst_lds, const uint32_t* src_global, int n) {
  constexpr int UL = 8;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src_global, (uint32_t)n * 4u);
  const int n4 = n / 4;
  for (int base = 0; base < n4; base += NT * UL) {
    u32x4 v[UL];
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      const int i = base + j * NT + (int)threadIdx.x;
      if (base + j * NT < n4) v[j] = load_shared_x4(r, (uint32_t)i * 16u);  // past n: reads 0
    }
    lds_sync();
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      const int i = base + j * NT + (int)threadIdx.x;
      if (base + j * NT < n4 && i < n4)
        reinterpret_cast<uint4*>(dst_lds)[i] = make_uint4(v[j].x, v[j].y, v[j].z, v[j].w);
    }
  }
}

// Streaming 16-byte load that is not expected to be reused (non-temporal).
ADM_DEV uint4 load_stream(const uint4* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Streaming 16-byte store of data no kernel reads back soon (non-temporal).
ADM_DEV void store_stream(uint4* p, uint4 v) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<v4u*>(p));
}

// ------------------------------------------------------- lane exchanges
// x from lane (lane ^ M) of the wavefront, without the LDS crossbar:
//   M = 1, 2: DPP quad permutations [1,0,3,2], [2,3,0,1];
//   M = 4:    DPP half-row mirror (l ^ 7 within 8 lanes), then quad [3,2,1,0] (l ^ 3);
//   M = 8:    DPP rotation by 8 within the 16-lane row;
//   M = 16, 32: v_permlane16_swap / v_permlane32_swap of x with itself, which
//   leaves x in one result and the partner lane's x in the other.
template <int CTRL>
ADM_DEV uint32_t dpp_move(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int M>
ADM_DEV uint32_t lane_xor_u32(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane mask");
  if constexpr (M == 1) return dpp_move<0xB1>(v);
  if constexpr (M == 2) return dpp_move<0x4E>(v);
  if constexpr (M == 4) return dpp_move<0x1B>(dpp_move<0x141>(v));
  if constexpr (M == 8) return dpp_move<0x128>(v);
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return r[0] == v ? r[1] : r[0];
  }
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] == v ? r[1] : r[0];
  }
}
template <int M>
ADM_DEV float lane_xor(float x) {
  return __uint_as_float(lane_xor_u32<M>(__float_as_uint(x)));
}
// x + x(lane ^ M) and max(x, x(lane ^ M)) for M = 16, 32: the two swap
// results are x and the partner's x in some order, which neither needs.
template <int M>
ADM_DEV float xor_sum(float x) {
  static_assert(M == 16 || M == 32, "row exchanges only");
  const uint32_t v = __float_as_uint(x);
  const auto r = (M == 16) ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int M>
ADM_DEV float xor_max(float x) {
  static_assert(M == 16 || M == 32, "row exchanges only");
  const uint32_t v = __float_as_uint(x);
  const auto r = (M == 16) ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
// Bucketing: a = max|y| over a group of 128 dimensions (the whole vector
// when D <= 128; at D = 256 lanes 0-31 and 32-63 hold the two groups),
// thresholds -0.5a, 0, +0.5a, codes 0 if y < -a/2, 1 if y < 0, 2 if
// y < a/2, else 3 (strict comparisons).
//
// Packing (§3.1): four codes per byte, first code in bits 7..6; returns, on
// the lanes with (lane % (16/E)) == 0, the little-endian 32-bit word
// lane / (16/E) of the packed row (16 codes per word); other lanes return 0.
// The §2.1 butterflies over one wavefront's vector (H16: every sum and
// difference one binary16 operation on binary16 inputs).
template <int D, bool H16>
ADM_DEV void wave_fwht(float (&y)[D / 64]) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & (kWave - 1);
  auto add = [](float a, float b) -> float {
    if constexpr (H16) return (float)(_Float16)((_Float16)a + (_Float16)b);
    else return a + b;
  };
  auto sub = [](float a, float b) -> float {
    if constexpr (H16) return (float)(_Float16)((_Float16)a - (_Float16)b);
    else return a - b;
  };
  if constexpr (H16) {
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = (float)(_Float16)y[e];
  }
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        float a = y[e], b = y[e + h];
        y[e] = add(a, b);
        y[e + h] = sub(a, b);
      }
    }
  }
  // butterflies across lanes: the lane with bit m clear keeps a + b, the
  // other a - b (a = the lower lane's value)
  auto stage = [&](auto mtag) {
    constexpr int m = decltype(mtag)::value;
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float p = lane_xor<m>(y[e]);
      y[e] = upper ? sub(p, y[e]) : add(y[e], p);
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
  stage(std::integral_constant<int, 16>{});
  stage(std::integral_constant<int, 32>{});
}

// The same butterflies over one vector held by a 16-lane slot of the
// wavefront, lane l16 holding the EL = D/16 consecutive dimensions
// [l16*EL, l16*EL + EL): the stages below EL pair registers of one lane, the
// stages EL, 2EL, 4EL and 8EL pair lanes l16 and l16 + h/EL inside the slot's
// 16-lane row.  Stage order and every operation are those of wave_fwht.
template <int D, bool H16>
ADM_DEV void slot_fwht(float (&y)[D / 16], int l16) {
  constexpr int EL = D / 16;
  auto add = [](float a, float b) -> float {
    if constexpr (H16) return (float)(_Float16)((_Float16)a + (_Float16)b);
    else return a + b;
  };
  auto sub = [](float a, float b) -> float {
    if constexpr (H16) return (float)(_Float16)((_Float16)a - (_Float16)b);
    else return a - b;
  };
  if constexpr (H16) {
#pragma unroll
    for (int e = 0; e < EL; ++e) y[e] = (float)(_Float16)y[e];
  }
#pragma unroll
  for (int h = 1; h < EL; h <<= 1) {
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      if ((e & h) == 0) {
        const float a = y[e], b = y[e + h];
        y[e] = add(a, b);
        y[e + h] = sub(a, b);
      }
    }
  }
  auto stage = [&](auto mtag) {
    constexpr int m = decltype(mtag)::value;
    const bool upper = (l16 & m) != 0;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const float p = lane_xor<m>(y[e]);
      y[e] = upper ? sub(p, y[e]) : add(y[e], p);
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
}

// How vectors are encoded (§2.1, §2.2).  rotate: 1 rotates in binary32; 0
// buckets the vector as it is (no §2.1; for the ablation); 2 rotates in
// binary16 (the article's FP16 advice, §6).  The outer bucketing thresholds
// of KV head h are -alpha*a and +alpha*a (one binary32 product), with
// alpha = alpha[h % n_alpha], or 0.5 (the §2.2 rule) when n_alpha is 0: the
// §3.2 tuning list lets groups of attention heads bucket with their own
// thresholds.  A query head buckets with its KV head's alpha.
constexpr int kMaxAlphaGroups = 64;
struct EncodeRule {
  int rotate;
  int n_alpha;
  float alpha[kMaxAlphaGroups];
  __host__ __device__ __forceinline__ float alpha_of(int head) const {
    return n_alpha > 0 ? alpha[head % n_alpha] : 0.5f;
  }
};

// mode: EncodeRule::rotate.  In binary16 the inputs are rounded to binary16
// and every sum and difference is one binary16 operation, carried between
// lanes as the equal binary32 value.
template <int D>
ADM_DEV uint32_t wave_encode(float (&y)[D / 64], int mode, float alpha) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & (kWave - 1);
  if (mode == 1)
    wave_fwht<D, false>(y);
  else if (mode == 2)
    wave_fwht<D, true>(y);
  float a = fabsf(y[0]);
#pragma unroll
  for (int e = 1; e < E; ++e) a = fmaxf(a, fabsf(y[e]));
  a = fmaxf(a, lane_xor<1>(a));
  a = fmaxf(a, lane_xor<2>(a));
  a = fmaxf(a, lane_xor<4>(a));
  a = fmaxf(a, lane_xor<8>(a));
  a = xor_max<16>(a);
  if constexpr (D <= 128) a = xor_max<32>(a);  // else one absmax per 32-lane half
  const float t2 = alpha * a;
  const float t0 = -t2;
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = y[e];
    const uint32_t c = (v < t0) ? 0u : (v < 0.0f) ? 1u : (v < t2) ? 2u : 3u;
    const int i = lane * E + e;                            // dimension index
    const int pos = 8 * ((i >> 2) & 3) + 6 - 2 * (i & 3);  // bit position in its word
    bits |= c << pos;
  }
  constexpr int kLanesPerWord = 16 / E;
  bits |= lane_xor_u32<1>(bits);
  bits |= lane_xor_u32<2>(bits);
  if constexpr (kLanesPerWord >= 8) bits |= lane_xor_u32<4>(bits);
  if constexpr (kLanesPerWord == 16) bits |= lane_xor_u32<8>(bits);
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

// popc(x) + acc as one instruction.  Written out so that a sum of plane
// popcounts stays a chain of accumulating counts (the compiler otherwise
// re-associates it into separate counts joined by three-input adds, two more
// VALU instructions per six counts in the scan's inner loop).
ADM_DEV uint32_t popc_acc(uint32_t x, uint32_t acc) {
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(acc));
  return r;
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

// Manhattan distance between two packed code rows of D dims (D/16 words),
// with the plane formulas of the scan (one 16-byte unit of 4 words at a time).
template <int D>
ADM_DEV uint32_t code_distance(const uint32_t* a, const uint32_t* b) {
  uint32_t s = 0;
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    const QPlanes qa = make_qplanes(a[4 * u], a[4 * u + 1], a[4 * u + 2], a[4 * u + 3]);
    const uint32_t* w = b + 4 * u;
    s += __popc(therm_p(w[0]) ^ qa.p[0]) + __popc(therm_p(w[1]) ^ qa.p[1]) +
         __popc(therm_p(w[2]) ^ qa.p[2]) + __popc(therm_p(w[3]) ^ qa.p[3]) +
         __popc(therm_t(w[0], w[1]) ^ qa.t[0]) + __popc(therm_t(w[2], w[3]) ^ qa.t[1]);
  }
  return s;
}

// Swap values between lane pairs (l, l^1) with a DPP quad permutation.
ADM_DEV uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

// ----------------------------------------------------------- block scans
// DPP controls (GFX9 data-parallel primitives on 16-lane rows).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
ADM_DEV uint32_t dpp_u32(uint32_t v) {
  // lanes whose source is outside the row, or whose row is masked off, get 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
}
template <int CTRL>
ADM_DEV float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts of 1, 2, 4, 8
// inside each 16-lane row, then row broadcasts of lanes 15 and 31 carry the
// row totals into the following rows.
ADM_DEV uint32_t wave_scan_incl(uint32_t v) {
  v += dpp_u32<kDppRowShr1>(v);
  v += dpp_u32<kDppRowShr2>(v);
  v += dpp_u32<kDppRowShr4>(v);
  v += dpp_u32<kDppRowShr8>(v);
  v += dpp_u32<kDppRowBcast15, 0xA>(v);
  v += dpp_u32<kDppRowBcast31, 0xC>(v);
  return v;
}

// Sum over each 16-lane row, returned on every lane of the row.
ADM_DEV float row16_sum(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppRowRor4>(x);
  x += dpp_f32<kDppRowRor8>(x);
  return x;
}

// Inclusive prefix sum of one u32 per thread over an NT-thread block.
// Uses s_tmp[0 .. NT/64); contains two barriers.
template <int NT>
ADM_DEV uint32_t block_scan_incl(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x >> 6;
  v = wave_scan_incl(v);
  if (lane == kWave - 1) s_tmp[kTmpWaveSums + wid] = v;
  lds_sync();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t x = s_tmp[kTmpWaveSums + w];
    pre += (w < wid) ? x : 0u;
    tot += x;
  }
  lds_sync();
  *total = tot;
  return v + pre;
}

// ------------------------------------------------------------------ §5.2
// Threshold of a budget over a distance histogram: the smallest t with
// count(D <= t) >= K, and lt = count(D < t).  Requires 1 <= K <= total count.
// Wavefront 0 does the search (one DPP scan over 64 lanes of consecutive
// bins); the result reaches every thread through LDS after one barrier.
// Two budgets K0, K1 are searched in the same pass (pass K1 = K0 for one).
struct Threshold {
  int t;
  uint32_t lt;
};
constexpr int kTmpThr1T = 18, kTmpThr1Lt = 19;

ADM_DEV void find_threshold_pair(const uint32_t* hist, int nbins, uint32_t K0, uint32_t K1,
                                 uint32_t* s_tmp, Threshold* r0, Threshold* r1) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int bpl = (nbins + kWave - 1) / kWave;
    const int b0 = lane * bpl;
    uint32_t sum = 0;
    for (int i = 0; i < bpl; ++i)
      if (b0 + i < nbins) sum += hist[b0 + i];
    const uint32_t incl = wave_scan_incl(sum);
    const uint32_t excl = incl - sum;
    const uint32_t Ks[2] = {K0, K1};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t K = Ks[w];
      if (excl < K && K <= incl) {
        uint32_t c = excl;
        for (int i = 0; i < bpl; ++i) {
          const uint32_t h = hist[b0 + i];
          if (c + h >= K) {
            s_tmp[w ? kTmpThr1T : kTmpThrT] = (uint32_t)(b0 + i);
            s_tmp[w ? kTmpThr1Lt : kTmpThrLt] = c;
            break;
          }
          c += h;
        }
      }
    }
  }
  lds_sync();
  *r0 = Threshold{(int)s_tmp[kTmpThrT], s_tmp[kTmpThrLt]};
  *r1 = Threshold{(int)s_tmp[kTmpThr1T], s_tmp[kTmpThr1Lt]};
  lds_sync();
}

// One bin per thread (nbins <= NT): DPP scan inside each wavefront, then the
// wavefront totals through LDS; the thread whose bin crosses K publishes it.
template <int NT>
ADM_DEV Threshold find_threshold(const uint32_t* hist, int nbins, uint32_t K, uint32_t* s_tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int nwb = (nbins + kWave - 1) / kWave;  // wavefronts that hold bins
  const uint32_t h = (int)threadIdx.x < nbins ? hist[threadIdx.x] : 0u;
  const uint32_t incl_w = wave_scan_incl(h);
  if (lane == kWave - 1 && wid < nwb) s_tmp[kTmpWaveSums + wid] = incl_w;
  lds_sync();
  if (wid < nwb) {
    uint32_t pre = 0;  // all wave sums read at once, the earlier ones added
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = s_tmp[kTmpWaveSums + w];
      pre += w < wid ? x : 0u;
    }
    const uint32_t incl = pre + incl_w, excl = incl - h;
    if (excl < K && K <= incl) {
      s_tmp[kTmpThrT] = threadIdx.x;
      s_tmp[kTmpThrLt] = excl;
    }
  }
  lds_sync();
  const Threshold r{(int)s_tmp[kTmpThrT], s_tmp[kTmpThrLt]};
  static_assert(NW <= 16, "wave sums live in s_tmp[0..16)");
  return r;
}

// Threshold of a budget over a group of chunks scanned by different
// workgroups.  Thread b < nbins holds tot = the group's count of distance b
// and bef = the count of distance b in the chunks before this workgroup's.
// Returns the group threshold t and lt = count(D < t) as find_threshold
// does, and for the chunks before this one lt_before = their count of D < t
// and ties_before = their count of D == t.  s_sums holds 32 words.
struct GroupThreshold {
  int t;
  uint32_t lt, lt_before, ties_before;
};
constexpr int kTmpGrpLtBefore = 21, kTmpGrpTiesBefore = 22, kTmpGroupCounts = 24;
constexpr int kTmpHalfTotals = 23;  // k_decode_gs re-scan: a half chunk's counts

template <int NT>
ADM_DEV GroupThreshold find_group_threshold(uint32_t tot, uint32_t bef, int nbins, uint32_t K,
                                            uint32_t* s_sums, uint32_t* s_tmp) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
  const int nwb = (nbins + kWave - 1) / kWave;
  if ((int)threadIdx.x >= nbins) tot = bef = 0;
  const uint32_t it = wave_scan_incl(tot), ib = wave_scan_incl(bef);
  if (lane == kWave - 1 && wid < nwb) {
    s_sums[wid] = it;
    s_sums[16 + wid] = ib;
  }
  lds_sync();
  if (wid < nwb) {
    uint32_t pt = 0, pb = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
      const uint32_t xt = s_sums[w], xb = s_sums[16 + w];
      pt += w < wid ? xt : 0u;
      pb += w < wid ? xb : 0u;
    }
    const uint32_t incl = pt + it, excl = incl - tot;
    if (excl < K && K <= incl) {
      s_tmp[kTmpThrT] = threadIdx.x;
      s_tmp[kTmpThrLt] = excl;
      s_tmp[kTmpGrpLtBefore] = pb + ib - bef;
      s_tmp[kTmpGrpTiesBefore] = bef;
    }
  }
  lds_sync();
  return GroupThreshold{(int)s_tmp[kTmpThrT], s_tmp[kTmpThrLt], s_tmp[kTmpGrpLtBefore],
                        s_tmp[kTmpGrpTiesBefore]};
}

// Threshold masks of TPT keys held two per 32-bit word (key 2i in the low
// half of word i, key 2i+1 in the high half; keys below 2^15): bit j of ge is
// set iff key j >= t, of gt iff key j > t.  The packed 16-bit differences
// (t-1-d) and (t-d) carry the answers in their sign bits; one shift and one
// and-or move word i's two sign bits to bits 2i and 16+2i, and the two halves
// are interleaved once at the end.
template <int TPT>
ADM_DEV void key_masks(const uint32_t* ws, int t, uint32_t& ge, uint32_t& gt) {
  static_assert(TPT % 8 == 0 && TPT <= 16, "sign bits of TPT/2 words fit one 16-bit half");
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const s16x2 tm1 = {(short)(t - 1), (short)(t - 1)};
  const s16x2 tt = {(short)t, (short)t};
  uint32_t ga = 0, gb = 0;
#pragma unroll
  for (int i = 0; i < TPT / 2; ++i) {
    const s16x2 dv = __builtin_bit_cast(s16x2, ws[i]);
    const uint32_t a = __builtin_bit_cast(uint32_t, (s16x2)(tm1 - dv));
    const uint32_t b = __builtin_bit_cast(uint32_t, (s16x2)(tt - dv));
    ga |= (a >> (15 - 2 * i)) & (0x00010001u << (2 * i));
    gb |= (b >> (15 - 2 * i)) & (0x00010001u << (2 * i));
  }
  ge = (ga & 0x5555u) | ((ga >> 15) & 0xAAAAu);
  gt = (gb & 0x5555u) | ((gb >> 15) & 0xAAAAu);
}

// Ordered selection inside one chunk held in LDS.  Keeps every token with
// D < t and the first `quota` tokens (lowest index) with D == t, and calls
// emit(pos, token, D) for each, pos being its rank in token order among the
// kept: (#lt before it) + min(#eq before it, quota).  Returns the number
// kept.  Thread j owns tokens [16j, 16j+16), read once with 16-byte LDS loads
// (threads past the chunk own nothing).
constexpr int kCompactTpt = 16;
// With tot_out, thread 0 gets (#below t) | (#at t) << 16 over the chunk there.
template <int NT, class Emit, int TPT = kCompactTpt>
ADM_DEV uint32_t chunk_collect(const uint16_t* sdist, int valid, int t, uint32_t quota,
                               uint32_t* s_tmp, Emit&& emit, const PhaseStamps* ps = nullptr,
                               uint32_t* tot_out = nullptr) {
  static_assert(TPT % 8 == 0 && TPT <= 16, "whole 16-byte reads, one 16-bit mask");
  const int t0 = threadIdx.x * TPT;
  uint32_t ltm = 0, eqm = 0;  // bit i: token t0+i is below / at the threshold
  uint32_t dw[TPT / 2] = {};  // the thread's distances, two per word (all <= 3*D < 2^15)
  if (t0 < valid) {
#pragma unroll
    for (int v8 = 0; v8 < TPT / 8; ++v8) {
      const uint4 w = *reinterpret_cast<const uint4*>(sdist + t0 + 8 * v8);
      dw[4 * v8] = w.x; dw[4 * v8 + 1] = w.y; dw[4 * v8 + 2] = w.z; dw[4 * v8 + 3] = w.w;
    }
    uint32_t ge, gt;
    key_masks<TPT>(dw, t, ge, gt);
    const int nv = valid - t0;  // tokens of this thread inside the chunk
    constexpr uint32_t kAll = (1u << TPT) - 1u;
    const uint32_t vmask = nv >= TPT ? kAll : ((1u << nv) - 1u);
    ltm = ~ge & vmask;
    eqm = ge & ~gt & vmask;
  }
  uint32_t tot;
  const uint32_t mine = (uint32_t)__popc(ltm) | ((uint32_t)__popc(eqm) << 16);
  if (ps) ps->mark_last_wave(17);  // masks done
  const uint32_t ex = block_scan_incl<NT>(mine, s_tmp, &tot) - mine;
  if (ps) ps->mark(18);  // prefix over the workgroup
  uint32_t ltb = ex & 0xffffu, eqb = ex >> 16;
  // visit only the flagged tokens, in order (a small fraction of the chunk)
  for (uint32_t m = ltm | eqm; m != 0; m &= m - 1) {
    const int i = __ffs(m) - 1;
    const uint32_t tok = (uint32_t)(t0 + i);
    if ((ltm >> i) & 1u) {
      uint32_t word = dw[0];
#pragma unroll
      for (int k = 1; k < TPT / 2; ++k) word = (i >> 1) == k ? dw[k] : word;
      emit(ltb + (eqb < quota ? eqb : quota), tok, (word >> (16 * (i & 1))) & 0xffffu);
      ++ltb;
    } else {
      if (eqb < quota) emit(ltb + eqb, tok, (uint32_t)t);
      ++eqb;
    }
  }
  if (ps) ps->mark_last_wave(19);  // tokens emitted
  if (tot_out != nullptr && threadIdx.x == 0) *tot_out = tot;
  const uint32_t eq_all = tot >> 16;
  return (tot & 0xffffu) + (eq_all < quota ? eq_all : quota);
}

// The chunk phase for G query heads at once (G >= 2): thresholds of all
// heads from their histograms, then the ordered selection of each head's kc
// best tokens into its own staging row, with three workgroup barriers in all
// (the per-head helpers above take about five per head).
//   hist  [G][nbp] key counts     sdist [G][chunk] keys     out [G][kpad]
// Head g keeps every token with key < t_g and the first kc - lt_g (lowest
// index) with key == t_g, in token order, as (key << 16) | token; entries
// past its kc are 0xFFFFFFFF.  s_thr holds 2G words, s_sums NW*G words.
template <int NT, int NB, int G, int TPT = kCompactTpt>
ADM_DEV void chunk_compact_heads(const uint32_t* hist, int nbp, const uint16_t* sdist, int chunk,
                                 int valid, uint32_t kc, uint32_t* out, int kpad,
                                 uint32_t* s_thr, uint32_t* s_sums,
                                 const PhaseStamps* ps = nullptr) {
  constexpr int NW = NT / kWave, BPL = (NB + kWave - 1) / kWave;
  static_assert(G <= NW, "one wavefront per head finds its threshold");
  static_assert(TPT % 8 == 0 && TPT <= 16, "whole 16-byte reads, one 16-bit mask");
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  // (1) thresholds: wavefront g scans head g's histogram, BPL bins per lane
  if (wid < G) {
    const uint32_t* h = hist + wid * nbp;
    uint32_t v[BPL], sum = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int bin = lane * BPL + j;
      v[j] = bin < NB ? h[bin] : 0u;
      sum += v[j];
    }
    const uint32_t incl = wave_scan_incl(sum), excl = incl - sum;
    if (excl < kc && kc <= incl) {  // the lane holding the kc-th smallest key
      uint32_t acc = excl, lt = 0;
      int t = 0;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {  // the bin where the count reaches kc
        if (acc < kc && kc <= acc + v[j]) {
          t = lane * BPL + j;
          lt = acc;
        }
        acc += v[j];
      }
      s_thr[2 * wid] = (uint32_t)t;
      s_thr[2 * wid + 1] = lt;
    }
  }
  // zero the staging rows' tails while the thresholds settle
  for (int i = threadIdx.x; i < G * kpad; i += NT) {
    const int g = i / kpad, j = i - g * kpad;
    if ((uint32_t)j >= kc) out[i] = 0xFFFFFFFFu;
  }
  lds_sync();
  if (ps) ps->mark(16);  // thresholds found
  // (2) this thread's TPT tokens: per head, masks of keys below / at t_g
  const int t0 = threadIdx.x * TPT;
  const int nv = valid - t0;
  constexpr uint32_t kAll = (1u << TPT) - 1u;
  const uint32_t vmask = nv >= TPT ? kAll : (nv > 0 ? ((1u << nv) - 1u) : 0u);
  uint32_t ltm[G], eqm[G], mine[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = (int)s_thr[2 * g];
    uint32_t ge = 0, gt = 0;
    if (t0 < valid) {
      uint32_t ws[TPT / 2];
#pragma unroll
      for (int v8 = 0; v8 < TPT / 8; ++v8) {
        const uint4 w = *reinterpret_cast<const uint4*>(sdist + g * chunk + t0 + 8 * v8);
        ws[4 * v8] = w.x; ws[4 * v8 + 1] = w.y; ws[4 * v8 + 2] = w.z; ws[4 * v8 + 3] = w.w;
      }
      key_masks<TPT>(ws, t, ge, gt);
    }
    ltm[g] = ~ge & vmask;
    eqm[g] = ge & ~gt & vmask;
    mine[g] = (uint32_t)__popc(ltm[g]) | ((uint32_t)__popc(eqm[g]) << 16);
  }
  if (ps) ps->mark_last_wave(17);  // masks of every head done
  // (3) prefix counts over the workgroup for every head with one barrier
  uint32_t incl[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    incl[g] = wave_scan_incl(mine[g]);
    if (lane == kWave - 1) s_sums[wid * G + g] = incl[g];
  }
  lds_sync();
  if (ps) ps->mark(18);  // prefix over the workgroup
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t pre = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) pre += w < wid ? s_sums[w * G + g] : 0u;
    const uint32_t ex = pre + incl[g] - mine[g];
    uint32_t ltb = ex & 0xffffu, eqb = ex >> 16;
    const uint32_t quota = kc - s_thr[2 * g + 1];
    const uint32_t t = s_thr[2 * g];
    uint32_t* o = out + g * kpad;
    for (uint32_t m = ltm[g] | eqm[g]; m != 0; m &= m - 1) {
      const int i = __ffs(m) - 1;
      const uint32_t tok = (uint32_t)(t0 + i);
      if ((ltm[g] >> i) & 1u) {
        const uint32_t d = sdist[g * chunk + tok];
        o[ltb + (eqb < quota ? eqb : quota)] = (d << 16) | tok;
        ++ltb;
      } else {
        if (eqb < quota) o[ltb + eqb] = (t << 16) | tok;
        ++eqb;
      }
    }
  }
  if (ps) ps->mark_last_wave(19);  // tokens emitted
  lds_sync();
}

// chunk_compact_heads over 8-bit keys: sdist8 [G][chunk] holds min(key, 255),
// the histograms the exact keys.  Thread j owns tokens [32j, 32j + 32)
// (chunk <= 32 * NT).  When every head's threshold key is below 255, a
// stored key below the threshold is exact, 255 can only mean "above it", and
// the result is chunk_compact_heads' on the exact keys; the function then
// emits and returns true.  Otherwise (some head's kc-th smallest key is 255
// or more) it emits nothing and returns false, with the thresholds in s_thr
// and the staging rows' tails already set; the caller must then select from
// exact keys.
constexpr int kKeySat = 255;
// x < u in each byte of x, for one byte value u in all four bytes, as bit 7
// of each byte of the result (the others clear).  xm = x | 0x80808080; c holds
// u in each byte (LO, u <= 128) or u - 128 (HI, u >= 128).  Per byte,
// xm - c = 0x80 + (x & 0x7F) - c_b never borrows from the next byte, and its
// bit 7 (z7) is set iff x's low seven bits are >= c_b.  LO: x < u iff x's bit
// 7 and z7 are both clear (u = 128: c_b = 128 leaves z7 clear, x < 128 iff
// bit 7 of x is); HI: iff either of them is clear.
template <bool HI>
ADM_HOST_DEV inline uint32_t bytes_below_u(uint32_t x, uint32_t xm, uint32_t c) {
  const uint32_t z = xm - c;
  return ~(HI ? (x & z) : (x | z)) & 0x80808080u;
}
// Bits 7, 15, 23, 31 of m to bits 0..3: the multiplier's four terms move bit
// 7 + 8k to 28 + k; the other products land on distinct bits (no carries)
// below 28 or past 31.
ADM_HOST_DEV inline uint32_t byte_flags_nibble(uint32_t m) { return (m * 0x00204081u) >> 28; }

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// Counts and hit mask of one thread's 32 one-byte keys k[0..32) (LDS, 16-byte
// aligned) against a threshold t <= 254: nlt = #keys < t, nle = #keys <= t,
// bit i of hit set iff k[i] <= t.  Keys from nv on (all when nv <= 0) count
// nowhere: they are read as 255, which no such threshold reaches.
ADM_DEV void byte_key_counts(const uint8_t* k, int nv, uint32_t t, uint32_t& nlt,
                             uint32_t& nle, uint32_t& hit) {
  nlt = nle = hit = 0;
  if (nv <= 0) return;
  const uint4 a = reinterpret_cast<const uint4*>(k)[0], b = reinterpret_cast<const uint4*>(k)[1];
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  if (nv < 32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int left = nv - 4 * j;
      w[j] |= left >= 4 ? 0u : (left <= 0 ? 0xFFFFFFFFu : 0xFFFFFFFFu << (8 * left));
    }
  }
  const auto pass = [&](auto hi, uint32_t c0, uint32_t c1) {
    constexpr bool HI = decltype(hi)::value;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t x = w[j], xm = x | 0x80808080u;
      const uint32_t lt = bytes_below_u<HI>(x, xm, c0), le = bytes_below_u<HI>(x, xm, c1);
      nlt += (uint32_t)__popc(lt);
      nle += (uint32_t)__popc(le);
      hit |= byte_flags_nibble(le) << (4 * j);
    }
  };
  // keys below t and below t + 1, both with the LO form while t + 1 <= 128
  if (t <= 127u)
    pass(BoolC<false>{}, t * 0x01010101u, (t + 1u) * 0x01010101u);
  else
    pass(BoolC<true>{}, (t - 128u) * 0x01010101u, (t - 127u) * 0x01010101u);
}

// The ordered selection of G heads at given thresholds over one-byte keys
// (every threshold below 255): head g keeps each token of the chunk with key
// < thr_of(g) and the first quota_of(g) (lowest index) with key ==
// thr_of(g), calling emit(g, pos, token, key) with pos its rank in token
// order among head g's kept tokens; with kept non-null, kept[g] (LDS) gets
// the number kept.  Thread j owns tokens [32j, 32j + 32) (valid <= 32 * NT);
// four keys per word are compared bytewise without borrows between bytes.
// s_sums holds NW * G words.  Ends with a workgroup barrier.
template <int NT, int G, class ThrOf, class QuotaOf, class Emit>
ADM_DEV void collect_heads_u8(const uint8_t* sdist8, int chunk, int valid, ThrOf&& thr_of,
                              QuotaOf&& quota_of, uint32_t* s_sums, Emit&& emit,
                              uint32_t* kept = nullptr, const PhaseStamps* ps = nullptr) {
  constexpr int NW = NT / kWave, TPT = 32;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  // counts of keys below t and up to t, and a 32-bit mask of this thread's
  // tokens with key <= t (the ones the emission visits)
  const int t0 = threadIdx.x * TPT;
  const int nv = valid - t0;
  uint32_t hit[G], mine[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t nlt, nle;
    byte_key_counts(sdist8 + g * chunk + t0, nv, thr_of(g), nlt, nle, hit[g]);
    mine[g] = nlt | ((nle - nlt) << 16);
  }
  if (ps) ps->mark_last_wave(17);  // masks of every head done
  uint32_t incl[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    incl[g] = wave_scan_incl(mine[g]);
    if (lane == kWave - 1) s_sums[wid * G + g] = incl[g];
  }
  lds_sync();
  if (ps) ps->mark(18);  // prefix over the workgroup
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t pre = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t s = s_sums[w * G + g];
      pre += w < wid ? s : 0u;
      all += s;
    }
    const uint32_t ex = pre + incl[g] - mine[g];
    uint32_t ltb = ex & 0xffffu, eqb = ex >> 16;
    const uint32_t quota = quota_of(g);
    const uint32_t t = thr_of(g);
    if (kept && threadIdx.x == 0) {
      const uint32_t eq_all = all >> 16;
      kept[g] = (all & 0xffffu) + (eq_all < quota ? eq_all : quota);
    }
    for (uint32_t m = hit[g]; m != 0; m &= m - 1) {
      const uint32_t tok = (uint32_t)(t0 + __ffs(m) - 1);
      const uint32_t d = sdist8[g * chunk + tok];
      if (d < t) {
        emit(g, ltb + (eqb < quota ? eqb : quota), tok, d);
        ++ltb;
      } else {
        if (eqb < quota) emit(g, ltb + eqb, tok, t);
        ++eqb;
      }
    }
  }
  if (ps) ps->mark_last_wave(19);  // tokens emitted
  lds_sync();
}

template <int NT, int NB, int G>
ADM_DEV bool chunk_compact_heads_u8(const uint32_t* hist, int nbp, const uint8_t* sdist8,
                                    int chunk, int valid, uint32_t kc, uint32_t* out, int kpad,
                                    uint32_t* s_thr, uint32_t* s_sums,
                                    const PhaseStamps* ps = nullptr) {
  constexpr int NW = NT / kWave, BPL = (NB + kWave - 1) / kWave;
  static_assert(G <= NW, "one wavefront per head finds its threshold");
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  if (wid < G) {  // thresholds, as chunk_compact_heads
    const uint32_t* h = hist + wid * nbp;
    uint32_t v[BPL], sum = 0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int bin = lane * BPL + j;
      v[j] = bin < NB ? h[bin] : 0u;
      sum += v[j];
    }
    const uint32_t incl = wave_scan_incl(sum), excl = incl - sum;
    if (excl < kc && kc <= incl) {
      uint32_t acc = excl, lt = 0;
      int t = 0;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        if (acc < kc && kc <= acc + v[j]) {
          t = lane * BPL + j;
          lt = acc;
        }
        acc += v[j];
      }
      s_thr[2 * wid] = (uint32_t)t;
      s_thr[2 * wid + 1] = lt;
    }
  }
  for (int i = threadIdx.x; i < G * kpad; i += NT) {
    const int g = i / kpad, j = i - g * kpad;
    if ((uint32_t)j >= kc) out[i] = 0xFFFFFFFFu;
  }
  lds_sync();
  if (ps) ps->mark(16);  // thresholds found
  bool exact = true;
#pragma unroll
  for (int g = 0; g < G; ++g) exact = exact && s_thr[2 * g] < (uint32_t)kKeySat;
  if (!exact) return false;
  collect_heads_u8<NT, G>(
      sdist8, chunk, valid, [&](int g) { return s_thr[2 * g]; },
      [&](int g) { return kc - s_thr[2 * g + 1]; }, s_sums,
      [&](int g, uint32_t pos, uint32_t tok, uint32_t key) {
        out[g * kpad + pos] = (key << 16) | tok;
      },
      nullptr, ps);
  return true;
}

// chunk_collect over 8-bit keys (min(key, 255), t < 255, so every key that
// is kept is exact): thread j owns tokens [32j, 32j + 32) of the chunk
// (valid <= 32 * NT), counted with bytewise compares; emit(pos, token, key)
// as chunk_collect.  With tot_out, thread 0 gets (#below t) | (#at t) << 16.
template <int NT, class Emit>
ADM_DEV uint32_t chunk_collect_u8(const uint8_t* skey, int valid, int t, uint32_t quota,
                                  uint32_t* s_tmp, Emit&& emit, uint32_t* tot_out = nullptr) {
  constexpr int TPT = 32;
  const int t0 = threadIdx.x * TPT;
  const int nv = valid - t0;
  uint32_t nlt, nle, hit;
  byte_key_counts(skey + t0, nv, (uint32_t)t, nlt, nle, hit);
  const uint32_t mine = nlt | ((nle - nlt) << 16);
  uint32_t tot;
  const uint32_t ex = block_scan_incl<NT>(mine, s_tmp, &tot) - mine;
  uint32_t ltb = ex & 0xffffu, eqb = ex >> 16;
  for (uint32_t m = hit; m != 0; m &= m - 1) {
    const uint32_t tok = (uint32_t)(t0 + __ffs(m) - 1);
    const uint32_t d = skey[tok];
    if (d < (uint32_t)t) {
      emit(ltb + (eqb < quota ? eqb : quota), tok, d);
      ++ltb;
    } else {
      if (eqb < quota) emit(ltb + eqb, tok, (uint32_t)t);
      ++eqb;
    }
  }
  if (tot_out != nullptr && threadIdx.x == 0) *tot_out = tot;
  const uint32_t eq_all = tot >> 16;
  return (tot & 0xffffu) + (eq_all < quota ? eq_all : quota);
}

// chunk_collect into out[] (LDS) as (D << 16) | token; entries [kept, pad_to)
// get the sentinel 0xFFFFFFFF.  on_kept(token, D) is called for every kept
// token.
template <int NT, int TPT = kCompactTpt, class OnKept>
ADM_DEV void chunk_compact(const uint16_t* sdist, int valid, Threshold thr, uint32_t quota,
                           uint32_t* out, int kept, int pad_to, uint32_t* s_tmp,
                           OnKept&& on_kept, const PhaseStamps* ps = nullptr) {
  auto emit = [&](uint32_t pos, uint32_t t, uint32_t d) {
    out[pos] = (d << 16) | t;
    on_kept(t, d);
  };
  chunk_collect<NT, decltype(emit)&, TPT>(sdist, valid, thr.t, quota, s_tmp, emit, ps);
  for (int j = kept + (int)threadIdx.x; j < pad_to; j += NT) out[j] = 0xFFFFFFFFu;
}

// Final selection of one head from its chunk candidates.  cand[] (global,
// written by lds_to_shared) holds n_chunks slots of 2^kpad_log2 entries (D << 16 | token in
// chunk) in token order, unused entries 0xFFFFFFFF, so the array is in global
// token order.  Keeps the bsel smallest (D, token), writes the tokens,
// ascending, to sidx[0..bsel) (LDS, if non-null) and idx[0..bsel) (global, if
// non-null) followed by -1 up to budget.  Candidates pass through LDS scand[]
// (capacity mcap) in tiles; one tile when M <= mcap.
template <int NT>
ADM_DEV void final_select_tiled(const uint32_t* cand, int M, int kpad_log2, int chunk, int nbins,
                                int bsel, int budget, int32_t* sidx, int32_t* idx,
                                uint32_t* scand, int mcap, uint32_t* shist, uint32_t* s_tmp,
                                const int32_t* slot_start);

// First token of candidate slot `slot`: slot * chunk for fixed chunks, else
// from slot_start[] (LDS) when the slots cover intervals of varying length.
ADM_DEV int32_t slot_token0(const int32_t* slot_start, int slot, int chunk) {
  return slot_start ? slot_start[slot] : slot * chunk;
}

// Up to 4*NT candidates: each thread keeps four consecutive entries in
// registers from one 16-byte coherent load; histogram, threshold and ordered
// compaction run on them directly.
template <int NT>
ADM_DEV void final_select(const uint32_t* cand, int M, int kpad_log2, int chunk, int nbins, int bsel,
                          int budget, int32_t* sidx, int32_t* idx, uint32_t* scand, int mcap,
                          uint32_t* shist, uint32_t* s_tmp, const int32_t* slot_start = nullptr,
                          const PhaseStamps* ps = nullptr) {
  if (M > 4 * NT) {
    final_select_tiled<NT>(cand, M, kpad_log2, chunk, nbins, bsel, budget, sidx, idx, scand,
                           mcap, shist, s_tmp, slot_start);
    return;
  }
  const int i0 = 4 * (int)threadIdx.x;
  u32x4 e = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  if (i0 < M) e = load_shared_x4(make_rsrc(cand, (uint32_t)M * 4u), (uint32_t)i0 * 4u);
  if ((int)threadIdx.x < nbins) shist[threadIdx.x] = 0;
  lds_sync();
  uint32_t v[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (i0 + j >= M) v[j] = 0xFFFFFFFFu;  // sentinel: no bin, never selected
    const uint32_t d = v[j] >> 16;
    if ((int)d < nbins) atomicAdd(&shist[d], 1u);
  }
  lds_sync();
  if (ps) ps->mark(6);  // candidates loaded, histogram built
  const Threshold thr = find_threshold<NT>(shist, nbins, (uint32_t)bsel, s_tmp);
  if (ps) ps->mark(7);  // threshold found
  const uint32_t quota = (uint32_t)bsel - thr.lt;
  uint32_t lt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = (int)(v[j] >> 16);
    lt += d < thr.t;
    eq += d == thr.t;
  }
  uint32_t tot;
  const uint32_t mine = lt | (eq << 16);
  if (ps) ps->mark_last_wave(20);  // counts below / at the threshold
  const uint32_t ex = block_scan_incl<NT>(mine, s_tmp, &tot) - mine;
  if (ps) ps->mark(21);  // prefix over the workgroup
  uint32_t ltb = ex & 0xffffu, eqb = ex >> 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = (int)(v[j] >> 16);
    int pos = -1;
    if (d < thr.t) {
      pos = (int)(ltb + (eqb < quota ? eqb : quota));
      ++ltb;
    } else if (d == thr.t) {
      if (eqb < quota) pos = (int)(ltb + eqb);
      ++eqb;
    }
    if (pos >= 0) {
      const int32_t tok =
          slot_token0(slot_start, (i0 + j) >> kpad_log2, chunk) + (int32_t)(v[j] & 0xffffu);
      if (sidx) sidx[pos] = tok;
      if (idx) idx[pos] = tok;
    }
  }
  if (idx)
    for (int j = bsel + threadIdx.x; j < budget; j += NT) idx[j] = -1;
  if (ps) ps->mark_last_wave(22);  // tokens placed
  lds_sync();
}

template <int NT>
ADM_DEV void final_select_tiled(const uint32_t* cand, int M, int kpad_log2, int chunk, int nbins,
                                int bsel, int budget, int32_t* sidx, int32_t* idx,
                                uint32_t* scand, int mcap, uint32_t* shist, uint32_t* s_tmp,
                                const int32_t* slot_start) {
  const bool resident = M <= mcap;
  for (int i = threadIdx.x; i < nbins; i += NT) shist[i] = 0;
  for (int base = 0; base < M; base += mcap) {
    const int n = min(mcap, M - base);
    lds_sync();
    shared_to_lds<NT>(scand, cand + base, n);
    lds_sync();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t d = scand[i] >> 16;
      if ((int)d < nbins) atomicAdd(&shist[d], 1u);
    }
  }
  lds_sync();
  const Threshold thr = find_threshold<NT>(shist, nbins, (uint32_t)bsel, s_tmp);
  const uint32_t quota = (uint32_t)bsel - thr.lt;
  uint32_t carry_lt = 0, carry_eq = 0;
  for (int base = 0; base < M; base += mcap) {
    const int n = min(mcap, M - base);
    if (!resident) {
      lds_sync();
      shared_to_lds<NT>(scand, cand + base, n);
      lds_sync();
    }
    const int tpt = (n + NT - 1) / NT;
    const int i0 = threadIdx.x * tpt;
    uint32_t lt = 0, eq = 0;
    for (int i = 0; i < tpt; ++i) {
      if (i0 + i < n) {
        const int d = (int)(scand[i0 + i] >> 16);
        lt += d < thr.t;
        eq += d == thr.t;
      }
    }
    uint32_t tot;
    const uint32_t mine = lt | (eq << 16);
    const uint32_t ex = block_scan_incl<NT>(mine, s_tmp, &tot) - mine;
    uint32_t ltb = carry_lt + (ex & 0xffffu), eqb = carry_eq + (ex >> 16);
    for (int i = 0; i < tpt; ++i) {
      const int j = i0 + i;
      if (j < n) {
        const uint32_t v = scand[j];
        const int d = (int)(v >> 16);
        int pos = -1;
        if (d < thr.t) {
          pos = (int)(ltb + (eqb < quota ? eqb : quota));
          ++ltb;
        } else if (d == thr.t) {
          if (eqb < quota) pos = (int)(ltb + eqb);
          ++eqb;
        }
        if (pos >= 0) {
          const int32_t tok =
              slot_token0(slot_start, (base + j) >> kpad_log2, chunk) + (int32_t)(v & 0xffffu);
          if (sidx) sidx[pos] = tok;
          if (idx) idx[pos] = tok;
        }
      }
    }
    carry_lt += tot & 0xffffu;
    carry_eq += tot >> 16;
  }
  if (idx)
    for (int j = bsel + threadIdx.x; j < budget; j += NT) idx[j] = -1;
  lds_sync();
}

// Wait until every vector memory access this wavefront has issued is
// complete; on gfx9-family targets stores count in vmcnt too, and a
// device-scope (sc1) store completes once it is written through to the level
// every XCD reads.  s_waitcnt immediate: vmcnt[3:0] in bits 3:0, expcnt in
// 6:4, lgkmcnt in 11:8, vmcnt[5:4] in 15:14; expcnt and lgkmcnt are left at
// their maxima (not waited for).  A workgroup-scope release fence does not
// wait for vmcnt on this target (all of a workgroup's wavefronts share one
// compute unit), so the hand-offs below wait explicitly.
constexpr int kWaitVmcnt0 = 0x0F70;
ADM_DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); }

// Count this workgroup's arrival after its coherent (sc1) hand-off stores
// completed; returns true on the last of n_arrivals workgroups, whose
// coherent loads then see every earlier workgroup's writes.  Every wavefront
// waits for its own stores (wait_vmem), the barrier orders the whole
// workgroup before the count, and the count itself is a device-scope atomic.
template <int NT>
ADM_DEV bool arrive_last(uint32_t* counter, int n_arrivals, uint32_t* s_tmp) {
  wait_vmem();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_tmp[kTmpFlag] = (prev == (uint32_t)(n_arrivals - 1)) ? 1u : 0u;
  }
  __syncthreads();
  return s_tmp[kTmpFlag] != 0;
}

// Count this workgroup's arrival as arrive_last does, then wait until all
// n_arrivals workgroups of the group have arrived.  Only for launches whose
// workgroups are all resident on the device together (the caller checks the
// grid against the device), so every awaited workgroup is running.  The wait
// is bounded: after max_polls polls it gives up, sets *status to 1 and
// returns false (on every thread of the workgroup); the caller must then not
// use the group's data (it may be incomplete) and still run to its end, so
// that every counter is left zero; that launch's results are invalid.
// Returns true when all n_arrivals workgroups have arrived.
template <int NT>
ADM_DEV bool arrive_and_wait(uint32_t* counter, int n_arrivals, uint32_t* status,
                             uint32_t max_polls, uint32_t* s_tmp) {
  wait_vmem();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t seen =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    for (uint32_t polls = 0; seen < (uint32_t)n_arrivals; ++polls) {
      if (polls >= max_polls) {
        __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      seen = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_tmp[kTmpFlag] = seen >= (uint32_t)n_arrivals ? 1u : 0u;
  }
  __syncthreads();
  return s_tmp[kTmpFlag] != 0;
}

}  // namespace adm
