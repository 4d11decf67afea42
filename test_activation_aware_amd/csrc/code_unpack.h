// Device helpers shared by the few-token projection kernels: loading one
// 64-channel step of a lane's packed codes from the tiled code layout and
// unpacking them into fp16 pairs 1024 + c (the code OR-ed into the mantissa
// of 1024.0, exact for codes below 1024), the raw-input loads of the fused
// input path, and direct-to-LDS buffer loads (also used by quantize_pack).
//
// Lane layout of a step (the A-operand layout of v_mfma_f32_32x32x16_f16):
// lane l holds row l % 32 of a 32-row tile and, in sub-step s = 0..3 of the
// step, the 8 channels 16 s + 8 (l / 32) .. + 7.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ttq {
namespace unpack {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef uint32_t u4a __attribute__((ext_vector_type(4), aligned(4)));  // 4 words at a word boundary

// 8 consecutive raw input values held in registers (fused input path)
template <typename TX>
struct XRaw {
  h8 v;
  __device__ __forceinline__ void load(const TX* p) { v = *reinterpret_cast<const h8*>(p); }
  __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  }
};
template <>
struct XRaw<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};
template <>
struct XRaw<void> {};

// raw buffer resource over [base, base + bytes) (loads past the end read 0)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nrec = (int)min<int64_t>(bytes, (int64_t)0x7FFFFFF0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

// 16 bytes per lane from a buffer into LDS; lane l lands at lds_wave_base + 16 l.
// AUX: the load's cache-policy bits (2: nontemporal, for data read once).
template <int AUX = 0>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           voff, 0, 0, AUX);
}

// Zero, as an opaque value the compiler cannot form before v is in a
// register.  A direct-to-LDS copy is not a dependence the compiler tracks for
// the LDS reads of its destination: addressing those reads with
// after_load(v), v a word of a global load issued after the copy, makes them
// wait for that load and so, since a wave's loads complete in issue order,
// for the copy.
__device__ __forceinline__ int after_load(uint32_t v) {
  int z = 0;
  asm("" : "+v"(z) : "v"(v));
  return z;
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// one step's code words of this lane (see the prefill kernel): q = 4, this
// lane half's 4 words; q = 2, the row's 4 words; q = 3, the row's 6 words;
// q = 5, words hh .. hh + 3 of each of the row's two 5-word blocks
template <int Q>
struct CodeStep {
  u4v a;
  u2v b;
};
template <>
struct CodeStep<5> {
  u4v a;
  u4v b;
};

// NT: loads with the nontemporal hint (codes streamed once per call)
template <typename V, bool NT>
__device__ __forceinline__ V load_words(const uint32_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}
template <int Q, bool NT = false>
__device__ __forceinline__ CodeStep<Q> load_codes(const uint32_t* p, int hh) {
  CodeStep<Q> c;
  if constexpr (Q == 4) {
    c.a = load_words<u4v, NT>(p + 4 * hh);
  } else if constexpr (Q == 2) {
    c.a = load_words<u4v, NT>(p);
  } else if constexpr (Q == 5) {
    c.a = load_words<u4a, NT>(p + hh);
    c.b = load_words<u4a, NT>(p + 5 + hh);
  } else {
    const u2v w01 = load_words<u2v, NT>(p);
    const u2v w23 = load_words<u2v, NT>(p + 2);
    c.b = load_words<u2v, NT>(p + 4);
    c.a = u4v{w01[0], w01[1], w23[0], w23[1]};
  }
  return c;
}

__device__ __forceinline__ uint32_t code_word(const CodeStep<3>& c, int i) { return i < 4 ? c.a[i] : c.b[i - 4]; }

// fp16 pairs 1024 + c for sub-step s of the step, this lane half
template <int Q>
__device__ __forceinline__ void code_pairs(const CodeStep<Q>& c, int s, int hh, uint32_t mask, uint32_t magic,
                                           uint32_t out[4]) {
  if constexpr (Q == 5) {
    // the 8 codes start at bit 80 (s & 1) + 8 hh of the 4 words held for
    // block s >> 1; lo / hi: codes 0-3 and 4-7 (20 bits each, from bit 0)
    const u4v& v = (s >> 1) ? c.b : c.a;
    const uint32_t o = 8u * (uint32_t)hh;
    uint32_t lo, hi;
    if ((s & 1) == 0) {
      lo = __builtin_amdgcn_alignbit(v[1], v[0], o);
      hi = __builtin_amdgcn_alignbit(v[1], v[0], o + 20u);
    } else {
      lo = __builtin_amdgcn_alignbit(v[3], v[2], o + 16u);
      hi = v[3] >> (o + 4u);
    }
    // codes 0 | 4 at bit 0 and 1 | 5 at bit 5 of ua, 2 | 6 at bit 2 and 3 | 7 at bit 7 of ub
    const uint32_t ua = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    const uint32_t ub = __builtin_amdgcn_perm(hi, lo, 0x06050201u);
    out[0] = and_or(ua, mask, magic);
    out[1] = and_or(ua >> 5, mask, magic);
    out[2] = and_or(ub >> 2, mask, magic);
    out[3] = and_or(ub >> 7, mask, magic);
    return;
  }
  uint32_t u;
  if constexpr (Q == 4) {
    u = c.a[s];
  } else if constexpr (Q == 2) {
    u = __builtin_amdgcn_perm(0u, c.a[s] >> (16 * hh), 0x0C010C00u);
  } else if constexpr (Q == 3) {
    const int bit = 3 * (16 * (s & 1) + 8 * hh);
    const int w = bit >> 5, off = bit & 31;
    const uint32_t lo = code_word(c, 3 * (s >> 1) + w);
    const uint32_t hi = (w < 2) ? code_word(c, 3 * (s >> 1) + w + 1) : 0u;
    const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)off);
    u = (win & 0xFFFu) | ((win << 4) & 0x0FFF0000u);
  }
  constexpr int SH = (Q == 4) ? 4 : (Q == 3 ? 3 : 2);
  out[0] = and_or(u, mask, magic);
#pragma unroll
  for (int j = 1; j < 4; ++j) out[j] = and_or(u >> (SH * j), mask, magic);
}

}  // namespace unpack
}  // namespace ttq
