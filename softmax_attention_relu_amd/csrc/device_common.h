// Device-side helpers for gfx950: vector types for the matrix cores, bf16
// packing, fast division and the RoPE table lookup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hla_internal.h"

namespace hla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// bf16 lives in memory as 16-bit patterns; two of them per 32-bit word,
// element 2i in the low half (little endian).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The feature map phi(x) = max(x, 0) with NaN kept (IEEE 754-2019 maximum,
// one v_maximum3_f32): a NaN input reaches every output that depends on it,
// where the maxNum of fmaxf would turn it into 0.
__device__ __forceinline__ float relu(float x) { return __builtin_elementwise_maximum(x, 0.0f); }

// Round two floats to bf16 (nearest even, v_cvt_pk_bf16_f32) and pack them.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2_t x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Low / high 16-bit halves of two words packed into one word.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv &f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// One rotated pair: which band table it reads and where its column starts.
struct RopePair {
  const float *col;  // table + 2 * k (k = pair index inside its band)
  int stride;        // floats per table row (= band width)
  int band;          // 0: t, 1: y, 2: x
};

__device__ __forceinline__ RopePair rope_pair(const RopeArgs &r, int p) {
  RopePair rp;
  const int two_p = 2 * p;
  if (two_p < r.d_t) {
    rp.col = r.cs_t + two_p;
    rp.stride = r.d_t;
    rp.band = 0;
  } else if (two_p < r.d_t + r.d_h) {
    rp.col = r.cs_h + (two_p - r.d_t);
    rp.stride = r.d_h;
    rp.band = 1;
  } else {
    rp.col = r.cs_w + (two_p - r.d_t - r.d_h);
    rp.stride = r.d_w;
    rp.band = 2;
  }
  return rp;
}

struct TokenPos {
  uint32_t t, y, x;
};

__device__ __forceinline__ TokenPos token_pos(const RopeArgs &r, uint32_t n) {
  TokenPos p;
  p.t = fast_div(n, r.div_hw);
  const uint32_t rem = n - p.t * r.hw;
  p.y = fast_div(rem, r.div_w);
  p.x = rem - p.y * r.w;
  return p;
}

// (cos, sin) of pair `rp` at token position `tp`.
__device__ __forceinline__ f32x2_t rope_cs(const RopePair &rp, const TokenPos &tp) {
  const uint32_t pos = rp.band == 0 ? tp.t : (rp.band == 1 ? tp.y : tp.x);
  return *reinterpret_cast<const f32x2_t *>(rp.col + (size_t)pos * rp.stride);
}

// Rotate (x0, x1) by the angle whose (cos, sin) is cs.
__device__ __forceinline__ void rotate(float &x0, float &x1, f32x2_t cs) {
  const float a = x0 * cs.x - x1 * cs.y;
  const float b = x0 * cs.y + x1 * cs.x;
  x0 = a;
  x1 = b;
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte store of eight bf16.
__device__ __forceinline__ void store_nt(uint16_t *p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}

// Loads of data a kernel reads exactly once, where each load instruction
// covers whole 128-byte lines (eight lanes x 16 bytes of a bf16 token row):
// non-temporal, so the stream does not displace the lines work-groups share
// (states, RoPE tables, the anchor's key tiles). Streams that use them ran
// 5-11% faster. Where several instructions read pieces of one line (8-byte
// loads, fp32 rows split over two loads) ordinary loads keep the line for the
// later pieces; a non-temporal load there fetched it again (the token-causal
// kernel slowed from 0.74 to 1.2 ms).
__device__ __forceinline__ u32x4_t load_once16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}
__device__ __forceinline__ uint4 load_once_u4(const void *p) {
  const u32x4_t v = load_once16(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Orders this wave's LDS stores before its later LDS loads (and the reverse)
// without a work-group barrier: LDS requests of one wave are served in order,
// the fence keeps the compiler from moving them across.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// cos/sin of the four pairs of one 8-dim chunk. When every band width is a
// multiple of 8 the chunk lies in one band and the four pairs are contiguous in
// its table: two aligned 16-byte loads. Otherwise each pair is looked up alone.
template <bool kAligned>
struct ChunkRope {
  RopePair p[kAligned ? 1 : 4];
  __device__ __forceinline__ void init(const RopeArgs &r, int chunk) {
#pragma unroll
    for (int j = 0; j < (kAligned ? 1 : 4); ++j) p[j] = rope_pair(r, 4 * chunk + j);
  }
  __device__ __forceinline__ void get(const TokenPos &tp, f32x2_t cs[4]) const {
    if constexpr (kAligned) {
      const uint32_t pos = p[0].band == 0 ? tp.t : (p[0].band == 1 ? tp.y : tp.x);
      const float *q = p[0].col + (size_t)pos * p[0].stride;
      const f32x4_t a = *reinterpret_cast<const f32x4_t *>(q);
      const f32x4_t b = *reinterpret_cast<const f32x4_t *>(q + 4);
      cs[0] = f32x2_t{a.x, a.y};
      cs[1] = f32x2_t{a.z, a.w};
      cs[2] = f32x2_t{b.x, b.y};
      cs[3] = f32x2_t{b.z, b.w};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) cs[j] = rope_cs(p[j], tp);
    }
  }
};

// bf16 outputs: hardware exp and reciprocal (about 1 ulp); exactly 1/2 at 0.
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float sigmoid_exact(float x) { return 1.f / (1.f + expf(-x)); }

}  // namespace hla
