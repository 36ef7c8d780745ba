// Block attention-residual (AttnRes) router (SANA-Video 2.0 summary, method
// section, router equation). Per token, with u = w + phi_t[b]:
//   r_i = 1 / sqrt(mean_c v_ic^2 + eps),  l_i = r_i * (u . v_i)
//   alpha = softmax_i(l),                 h = sum_i alpha_i v_i
// RMSNorm reduces to the scalar r_i, so each source is read from HBM once:
// one wave per token, every lane holding 8-element chunks of each source in
// registers (chunk c of the row lives in lane c % 64), wave reductions for the
// two dot products per source, then the weighted sum from registers.
// Sources that do not fit in registers take a second pass over the row.
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
    c.w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + off);
    return c;
  }
  __device__ static void unpack(const Chunk &c, float x[8]) {
    x[0] = bf16_lo(c.w.x); x[1] = bf16_hi(c.w.x);
    x[2] = bf16_lo(c.w.y); x[3] = bf16_hi(c.w.y);
    x[4] = bf16_lo(c.w.z); x[5] = bf16_hi(c.w.z);
    x[6] = bf16_lo(c.w.w); x[7] = bf16_hi(c.w.w);
  }
  __device__ static void store(void *base, size_t off, const float y[8]) {
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(base) + off) =
        make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7]));
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
    float *p = reinterpret_cast<float *>(base) + off;
    *reinterpret_cast<float4 *>(p) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// CHL: 8-element chunks per lane (C <= 512 * CHL). kKeep: sources kept in
// registers (S <= kKeep); otherwise the weighted sum re-reads the row.
template <bool kBF16, int CHL, int kKeep>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  typedef RouteElem<kBF16> E;
  const int lane = threadIdx.x & 63;
  const long long tok = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= (long long)a.B * a.T) return;  // whole wave leaves together
  const int b = (int)(tok / a.T);
  const int nch = a.C / 8;
  const size_t row = (size_t)tok * a.C;

  float u[CHL][8];
#pragma unroll
  for (int c = 0; c < CHL; ++c) {
    const int ch = lane + 64 * c;
#pragma unroll
    for (int t = 0; t < 8; ++t) u[c][t] = 0.f;
    if (ch < nch) {
      const float4 w0 = *reinterpret_cast<const float4 *>(a.w + 8 * ch);
      const float4 w1 = *reinterpret_cast<const float4 *>(a.w + 8 * ch + 4);
      u[c][0] = w0.x; u[c][1] = w0.y; u[c][2] = w0.z; u[c][3] = w0.w;
      u[c][4] = w1.x; u[c][5] = w1.y; u[c][6] = w1.z; u[c][7] = w1.w;
      if (a.phi_t) {
        const float *pp = a.phi_t + (size_t)b * a.C + 8 * ch;
        const float4 p0 = *reinterpret_cast<const float4 *>(pp);
        const float4 p1 = *reinterpret_cast<const float4 *>(pp + 4);
        u[c][0] += p0.x; u[c][1] += p0.y; u[c][2] += p0.z; u[c][3] += p0.w;
        u[c][4] += p1.x; u[c][5] += p1.y; u[c][6] += p1.z; u[c][7] += p1.w;
      }
    }
  }

  const bool keep = a.S <= kKeep;
  typename E::Chunk held[kKeep][CHL];
  float logit[kMaxSources];
  const float inv_c = 1.f / (float)a.C;
#pragma unroll
  for (int i = 0; i < kMaxSources; ++i) {
    if (i < a.S) {
      float ss = 0.f, dot = 0.f;
#pragma unroll
      for (int c = 0; c < CHL; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
          const typename E::Chunk ck = E::load(a.v[i], row + 8 * ch);
          if (keep && i < kKeep) held[i < kKeep ? i : 0][c] = ck;
          float x[8];
          E::unpack(ck, x);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            ss += x[t] * x[t];
            dot += u[c][t] * x[t];
          }
        }
      }
      ss = wave_sum(ss);
      dot = wave_sum(dot);
      logit[i] = dot / sqrtf(ss * inv_c + a.eps);
    } else {
      logit[i] = -INFINITY;
    }
  }
  float m = logit[0];
#pragma unroll
  for (int i = 1; i < kMaxSources; ++i) m = fmaxf(m, logit[i]);
  float alpha[kMaxSources];
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxSources; ++i) {
    alpha[i] = i < a.S ? expf(logit[i] - m) : 0.f;
    l += alpha[i];
  }
  const float inv_l = 1.f / l;
#pragma unroll
  for (int i = 0; i < kMaxSources; ++i) alpha[i] *= inv_l;

#pragma unroll
  for (int c = 0; c < CHL; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      float y[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxSources; ++i) {
        if (i < a.S) {
          float x[8];
          if (keep && i < kKeep)
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
    for (int i = 1; i < kMaxSources; ++i)
      if (lane == i) al = alpha[i];
    a.alpha[(size_t)tok * a.S + lane] = al;
  }
}

template <bool kBF16>
hipError_t launch_typed(const RouteArgs &a, hipStream_t stream) {
  const long long tokens = (long long)a.B * a.T;
  const dim3 grid((unsigned)((tokens + 3) / 4));
  const int nch = a.C / 8;
  if (nch <= 64)
    hipLaunchKernelGGL((route_kernel<kBF16, 1, 16>), grid, dim3(256), 0, stream, a);
  else if (nch <= 128)
    hipLaunchKernelGGL((route_kernel<kBF16, 2, 8>), grid, dim3(256), 0, stream, a);
  else if (nch <= 256)
    hipLaunchKernelGGL((route_kernel<kBF16, 4, 4>), grid, dim3(256), 0, stream, a);
  else if (nch <= 512)
    hipLaunchKernelGGL((route_kernel<kBF16, 8, 2>), grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(hla_dtype dt, const RouteArgs &a, hipStream_t stream) {
  return dt == HLA_BF16 ? launch_typed<true>(a, stream) : launch_typed<false>(a, stream);
}

}  // namespace hla
