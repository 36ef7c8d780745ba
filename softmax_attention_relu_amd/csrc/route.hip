// Block attention-residual (AttnRes) router (SANA-Video 2.0 summary, method
// section, router equation). Per token, with u = w + phi_t[b]:
//   r_i = 1 / sqrt(mean_c v_ic^2 + eps),  l_i = r_i * (u . v_i)
//   alpha = softmax_i(l),                 h = sum_i alpha_i v_i
// RMSNorm reduces to the scalar r_i, so each source is read from HBM once:
// a wave handles one token at a time, every lane holding 8-element chunks of
// each source in registers (chunk c of the row lives in lane c % 64); u, the
// same for every token of a batch, sits in a per-wave LDS copy, which keeps
// the kernel within 128 registers and four waves per SIMD for C <= 2048. The two
// dot products of all sources are summed over the wave in one transposed
// butterfly, then the weighted sum is formed from the registers. Sources that
// do not fit in registers are read again for the weighted sum.
#include <algorithm>

#include "device_common.h"

namespace hla {

namespace {

template <bool kBF16>
struct RouteElem;
template <>
struct RouteElem<true> {
  struct Chunk {
    uint4 w;
  };
  __device__ static Chunk load(const void *base, size_t off) {
    Chunk c;
    c.w = load_once_u4(reinterpret_cast<const uint16_t *>(base) + off);
    return c;
  }
  __device__ static void unpack(const Chunk &c, float x[8]) {
    x[0] = bf16_lo(c.w.x); x[1] = bf16_hi(c.w.x);
    x[2] = bf16_lo(c.w.y); x[3] = bf16_hi(c.w.y);
    x[4] = bf16_lo(c.w.z); x[5] = bf16_hi(c.w.z);
    x[6] = bf16_lo(c.w.w); x[7] = bf16_hi(c.w.w);
  }
  __device__ static void store(void *base, size_t off, const float y[8]) {
    store_nt(reinterpret_cast<uint16_t *>(base) + off,
             u32x4_t{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])});
  }
};
template <>
struct RouteElem<false> {
  struct Chunk {
    float4 a, b;
  };
  __device__ static Chunk load(const void *base, size_t off) {
    const float *p = reinterpret_cast<const float *>(base) + off;
    Chunk c;
    c.a = *reinterpret_cast<const float4 *>(p);
    c.b = *reinterpret_cast<const float4 *>(p + 4);
    return c;
  }
  __device__ static void unpack(const Chunk &c, float x[8]) {
    x[0] = c.a.x; x[1] = c.a.y; x[2] = c.a.z; x[3] = c.a.w;
    x[4] = c.b.x; x[5] = c.b.y; x[6] = c.b.z; x[7] = c.b.w;
  }
  __device__ static void store(void *base, size_t off, const float y[8]) {
    f32x4_t *p = reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(base) + off);
    __builtin_nontemporal_store(f32x4_t{y[0], y[1], y[2], y[3]}, p);
    __builtin_nontemporal_store(f32x4_t{y[4], y[5], y[6], y[7]}, p + 1);
  }
};

template <int kCtrl>
__device__ __forceinline__ float f32_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141, kDppQuad2301 = 0x4E, kDppQuad1032 = 0xB1;

// One step inside a row of 16 lanes: the partner (given by the DPP control,
// an involution) differs in lane bit kBit. While n > 1 values remain the step
// is transposed (lanes with the bit set keep the upper half), else it sums.
template <int kCtrl, int kBit, int VC>
__device__ __forceinline__ void row_step(float v[VC], int &n, int lane) {
  const bool hi = (lane >> kBit) & 1;
  if (n > 1) {
#pragma unroll
    for (int k = 0; k < VC / 2; ++k) {
      if (k < n / 2) {
        const float keep = hi ? v[k + n / 2] : v[k];
        const float give = hi ? v[k] : v[k + n / 2];
        v[k] = keep + f32_dpp<kCtrl>(give);
      }
    }
    n /= 2;
  } else {
    v[0] += f32_dpp<kCtrl>(v[0]);
  }
}

// Sums each of the VC values v[] over the 64 lanes of the wave (VC = 8, 16 or
// 32) in one transposed butterfly: every step pairs lanes that differ in one
// lane bit, and the two lanes of a pair keep different halves of the values
// still held, so each step halves the values per lane. v_permlane32_swap and
// v_permlane16_swap of the pair (a, b) hand lane bit 5 (bit 4) = 0 its own and
// its partner's a and bit = 1 both b's in one instruction; inside a row of 16
// the partner comes from a DPP mirror or quad permutation (an involution that
// flips the lane bit in question). After the transposed steps the remaining
// lane bits are summed out. The total of value k ends in the lanes whose bits
// 5, 4, ... spell k from the top, and is returned in red[k] for every lane.
template <int VC>
__device__ __forceinline__ void wave_sums(float v[VC], float red[VC]) {
  static_assert(VC == 8 || VC == 16 || VC == 32, "reduction width");
  const int lane = threadIdx.x & 63;
  // lane bit 5
#pragma unroll
  for (int k = 0; k < VC / 2; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + VC / 2]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  // lane bit 4
#pragma unroll
  for (int k = 0; k < VC / 4; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[k + VC / 4]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  // lane bits 3, 2, 1 inside rows: transposed while values remain, then plain sums
  int n = VC / 4;
  row_step<kDppRowMirror, 3, VC>(v, n, lane);
  row_step<kDppRowHalfMirror, 2, VC>(v, n, lane);
  row_step<kDppQuad2301, 1, VC>(v, n, lane);
  v[0] += f32_dpp<kDppQuad1032>(v[0]);  // lane bit 0
  // value k sits in the lanes whose bits 5, 4, ... (log2 VC of them) spell k
  constexpr int kBits = VC == 8 ? 3 : (VC == 16 ? 4 : 5);
#pragma unroll
  for (int k = 0; k < VC; ++k) red[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[0]), k << (6 - kBits)));
}

// One wave per token at a time; the waves of the grid take tokens in turn
// (wave w: tokens w, w + W, ...), so the running waves read one contiguous
// window of the sources. CHL: 8-element chunks per lane (C <= 512 * CHL).
// kKeep: sources kept in registers (S <= kKeep), otherwise the weighted sum
// reads the row again. SMAX: sources the reduction is sized for (S <= SMAX).
extern __shared__ __align__(16) float route_u_lds[];

template <bool kBF16, int CHL, int kKeep, int SMAX>
__global__ __launch_bounds__(256, CHL <= 4 ? 4 : 1) void route_kernel(RouteArgs a) {
  typedef RouteElem<kBF16> E;
  const int lane = threadIdx.x & 63;
  // u = w + phi_t[b] of the wave's current batch, one copy per wave in LDS
  float *ul = route_u_lds + (size_t)(threadIdx.x >> 6) * a.C;
  const long long tokens = (long long)a.B * a.T;
  const long long nwaves = (long long)gridDim.x * 4;
  const int nch = a.C / 8;
  const float inv_c = 1.f / (float)a.C;

  int ub = -1;  // batch whose u is staged
  for (long long tok = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); tok < tokens; tok += nwaves) {
    const int b = (int)(tok / a.T);
    if (b != ub) {  // u = w + phi_t[b]
      ub = b;
      wave_lds_fence();  // the previous batch's u is no longer read
#pragma unroll
      for (int c = 0; c < CHL; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
          float4 w0 = *reinterpret_cast<const float4 *>(a.w + 8 * ch);
          float4 w1 = *reinterpret_cast<const float4 *>(a.w + 8 * ch + 4);
          if (a.phi_t) {
            const float *pp = a.phi_t + (size_t)b * a.C + 8 * ch;
            const float4 p0 = *reinterpret_cast<const float4 *>(pp);
            const float4 p1 = *reinterpret_cast<const float4 *>(pp + 4);
            w0.x += p0.x; w0.y += p0.y; w0.z += p0.z; w0.w += p0.w;
            w1.x += p1.x; w1.y += p1.y; w1.z += p1.z; w1.w += p1.w;
          }
          *reinterpret_cast<float4 *>(ul + 8 * ch) = w0;
          *reinterpret_cast<float4 *>(ul + 8 * ch + 4) = w1;
        }
      }
      wave_lds_fence();
    }
    const size_t row = (size_t)tok * a.C;

    // this lane's share of sum v^2 and u.v for every source
    typename E::Chunk held[kKeep > 0 ? kKeep : 1][CHL];
    float part[2 * SMAX];
#pragma unroll
    for (int i = 0; i < SMAX; ++i) {
      float ss = 0.f, dot = 0.f;
      if (i < a.S) {
#pragma unroll
        for (int c = 0; c < CHL; ++c) {
          const int ch = lane + 64 * c;
          if (ch < nch) {
            const typename E::Chunk ck = E::load(a.v[i], row + 8 * ch);
            if (i < kKeep) held[i < kKeep ? i : 0][c] = ck;
            float x[8];
            E::unpack(ck, x);
            const f32x4_t u0 = *reinterpret_cast<const f32x4_t *>(ul + 8 * ch);
            const f32x4_t u1 = *reinterpret_cast<const f32x4_t *>(ul + 8 * ch + 4);
            const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              ss += x[t] * x[t];
              dot += uu[t] * x[t];
            }
          }
        }
      }
      part[2 * i] = ss;
      part[2 * i + 1] = dot;
    }
    float red[2 * SMAX];
    wave_sums<2 * SMAX>(part, red);

    float alpha[SMAX];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < SMAX; ++i) {
      alpha[i] = i < a.S ? red[2 * i + 1] / sqrtf(red[2 * i] * inv_c + a.eps) : -INFINITY;
      m = fmaxf(m, alpha[i]);
    }
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < SMAX; ++i) {
      alpha[i] = i < a.S ? expf(alpha[i] - m) : 0.f;
      l += alpha[i];
    }
    const float inv_l = 1.f / l;
#pragma unroll
    for (int i = 0; i < SMAX; ++i) alpha[i] *= inv_l;

#pragma unroll
    for (int c = 0; c < CHL; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        float y[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) y[t] = 0.f;
#pragma unroll
        for (int i = 0; i < SMAX; ++i) {
          if (i < a.S) {
            float x[8];
            if (i < kKeep)
              E::unpack(held[i < kKeep ? i : 0][c], x);
            else
              E::unpack(E::load(a.v[i], row + 8 * ch), x);
#pragma unroll
            for (int t = 0; t < 8; ++t) y[t] += alpha[i] * x[t];
          }
        }
        E::store(a.h, row + 8 * ch, y);
      }
    }
    if (a.alpha && lane < a.S) {
      float al = alpha[0];
#pragma unroll
      for (int i = 1; i < SMAX; ++i)
        if (lane == i) al = alpha[i];
      a.alpha[(size_t)tok * a.S + lane] = al;
    }
  }
}

// Grid of the grid-stride kernel: as many work-groups as are resident at once
// (occupancy of this instantiation, read once, times the CUs), never more than
// one wave per token.
template <bool kBF16, int CHL, int kKeep, int SMAX>
hipError_t launch_kernel(const RouteArgs &a, hipStream_t stream) {
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, route_kernel<kBF16, CHL, kKeep, SMAX>, 256,
                                                     4 * 512 * CHL * sizeof(float)) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 1;
  const long long tokens = (long long)a.B * a.T;
  const long long wgs = std::min<long long>((tokens + 3) / 4, (long long)per_cu * cus);
  hipLaunchKernelGGL((route_kernel<kBF16, CHL, kKeep, SMAX>), dim3((unsigned)wgs), dim3(256),
                     4 * (size_t)a.C * sizeof(float), stream, a);
  return hipGetLastError();
}

template <bool kBF16, int CHL, int kKeep>
hipError_t launch_smax(const RouteArgs &a, hipStream_t stream) {
  if (a.S <= 4) return launch_kernel<kBF16, CHL, kKeep, 4>(a, stream);
  if (a.S <= 8) return launch_kernel<kBF16, CHL, kKeep, 8>(a, stream);
  return launch_kernel<kBF16, CHL, kKeep, 16>(a, stream);
}

template <bool kBF16>
hipError_t launch_typed(const RouteArgs &a, hipStream_t stream) {
  const int nch = a.C / 8;
  if (nch <= 64) return launch_smax<kBF16, 1, 16>(a, stream);
  if (nch <= 128) return launch_smax<kBF16, 2, 8>(a, stream);
  if (nch <= 256) return launch_smax<kBF16, 4, 4>(a, stream);
  if (nch <= 512) return launch_smax<kBF16, 8, 2>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route(hla_dtype dt, const RouteArgs &a, hipStream_t stream) {
  return dt == HLA_BF16 ? launch_typed<true>(a, stream) : launch_typed<false>(a, stream);
}

}  // namespace hla
