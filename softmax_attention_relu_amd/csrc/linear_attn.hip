// ReLU-kernel linear attention with 3D RoPE after the ReLU, bidirectional and
// block-causal (SANA-Video notes, section 3.2 output equation and pseudocode;
// section 3.4 causal equation, constant-memory cache and Algorithm 1).
//
// One call runs three kernels on the caller's stream:
//   la_build  per (b, h, slab of tokens): c_j = RoPE(relu(k_j)) and
//             S_slab = sum_j c_j^T v_j on the matrix cores (bf16 operands,
//             fp32 accumulation; fp32 operands for float inputs), plus
//             z_slab = sum_j relu(k_j) on the vector ALUs. Slabs never straddle
//             a chunk boundary.
//   la_scan   per (b, h): fixed-order sum of the slab partials of each chunk
//             and an inclusive prefix over chunks, starting from the carried
//             state; writes one (KV, ksum) record per chunk and the final
//             state. A bidirectional call is the one-chunk case.
//   la_apply  per (b, h, token range inside one chunk): a_i = RoPE(relu(q_i)),
//             numerator a_i P_c on the matrix cores, denominator relu(q_i).Z_c
//             + eps, optional sigmoid gate, store.
// Memory traffic is the K/V read of the build and the Q/G read and O write of
// the apply; the fp32 partials are ~1-2% on top.
#include "device_common.h"

namespace hla {

namespace {

constexpr int kTile = 256;            // tokens per build tile (8 per thread)
constexpr int kRow16 = kTile + 8;     // bf16 elements per LDS row (16-byte pad)
constexpr int kRow32 = kTile + 4;     // float elements per LDS row (16-byte pad)
constexpr int kApplySub = 32;         // tokens per wave step in the apply

template <bool kBF16>
struct Elem;
template <>
struct Elem<true> {
  typedef uint16_t T;
  // eight consecutive elements of one row
  struct Chunk {
    uint4 w;
  };
  __device__ static Chunk load(const T *p) {
    Chunk c;
    c.w = *reinterpret_cast<const uint4 *>(p);
    return c;
  }
  __device__ static Chunk zero() {
    Chunk c;
    c.w = make_uint4(0, 0, 0, 0);
    return c;
  }
  __device__ static void unpack(const Chunk &c, float x[8]) {
    x[0] = bf16_lo(c.w.x); x[1] = bf16_hi(c.w.x);
    x[2] = bf16_lo(c.w.y); x[3] = bf16_hi(c.w.y);
    x[4] = bf16_lo(c.w.z); x[5] = bf16_hi(c.w.z);
    x[6] = bf16_lo(c.w.w); x[7] = bf16_hi(c.w.w);
  }
};
template <>
struct Elem<false> {
  typedef float T;
  struct Chunk {
    float4 a, b;
  };
  __device__ static Chunk load(const T *p) {
    Chunk c;
    c.a = *reinterpret_cast<const float4 *>(p);
    c.b = *reinterpret_cast<const float4 *>(p + 4);
    return c;
  }
  __device__ static Chunk zero() {
    Chunk c;
    c.a = make_float4(0.f, 0.f, 0.f, 0.f);
    c.b = c.a;
    return c;
  }
  __device__ static void unpack(const Chunk &c, float x[8]) {
    x[0] = c.a.x; x[1] = c.a.y; x[2] = c.a.z; x[3] = c.a.w;
    x[4] = c.b.x; x[5] = c.b.y; x[6] = c.b.z; x[7] = c.b.w;
  }
};

struct BuildArgs {
  const void *k, *v;
  int N, H, L, n_chunks, slab_tokens, slabs_per_chunk;
  RopeArgs rope;
  float *part;  // [B*H][n_chunks*slabs_per_chunk][kStateFloats]
};

// ---------------------------------------------------------------------------
// State build. 256 threads; thread t owns dims 8*(t%8) .. +7 of tokens
// 8*(t/8) .. +7 of each 256-token tile, so every load instruction of a wave
// reads eight whole 128-byte token rows. The thread rotates its pairs, then
// writes its 8x8 block transposed into LDS (dim-major, token-contiguous), the
// layout the matrix-core operands want: S = C^T V with the token axis as the
// reduction axis. Wave w accumulates the 32x32 block (w/2, w%2) of S.
template <bool kBF16>
__global__ __launch_bounds__(256) void la_build_kernel(BuildArgs a) {
  typedef Elem<kBF16> E;
  typedef typename E::T T;
  extern __shared__ __align__(16) unsigned char lds_raw[];

  const int tid = threadIdx.x;
  const int dc = tid & 7;   // dim chunk
  const int g = tid >> 3;   // token group inside the tile
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int bh = blockIdx.y;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int slab_id = blockIdx.x;
  const int chunk = slab_id / a.slabs_per_chunk;
  const int slab = slab_id - chunk * a.slabs_per_chunk;
  const int c_lo = chunk * a.L;
  const int c_hi = min(a.N, c_lo + a.L);
  const int lo = c_lo + slab * a.slab_tokens;
  const int hi = min(c_hi, lo + a.slab_tokens);

  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD + dc * 8;
  const T *kp = reinterpret_cast<const T *>(a.k) + head_base;
  const T *vp = reinterpret_cast<const T *>(a.v) + head_base;

  RopePair rp[4];
  if (a.rope.enabled) {
#pragma unroll
    for (int j = 0; j < 4; ++j) rp[j] = rope_pair(a.rope, 4 * dc + j);
  }

  float zacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zacc[i] = 0.f;
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  typename E::Chunk kr[8], vr[8];
  auto load_tile = [&](int base) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int n = base + 8 * g + r;
      if (n < hi) {
        kr[r] = E::load(kp + (size_t)n * tok_stride);
        vr[r] = E::load(vp + (size_t)n * tok_stride);
      } else {
        kr[r] = E::zero();
        vr[r] = E::zero();
      }
    }
  };

  if (lo < hi) load_tile(lo);
  for (int base = lo; base < hi; base += kTile) {
    __syncthreads();  // previous tile's operand reads are done
    // relu, key sum, rotation; transposed store into LDS
    float c[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float x[8];
      E::unpack(kr[r], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = fmaxf(x[i], 0.f);
        zacc[i] += x[i];
      }
      if (a.rope.enabled) {
        const int n = base + 8 * g + r;
        const TokenPos tp = token_pos(a.rope, (uint32_t)min(n, a.N - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) rotate(x[2 * j], x[2 * j + 1], rope_cs(rp[j], tp));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) c[r][i] = x[i];
    }
    if constexpr (kBF16) {
      uint16_t *cT = reinterpret_cast<uint16_t *>(lds_raw);
      uint16_t *vT = cT + kD * kRow16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint4 w;
        w.x = pack_bf16(c[0][i], c[1][i]);
        w.y = pack_bf16(c[2][i], c[3][i]);
        w.z = pack_bf16(c[4][i], c[5][i]);
        w.w = pack_bf16(c[6][i], c[7][i]);
        *reinterpret_cast<uint4 *>(cT + (8 * dc + i) * kRow16 + 8 * g) = w;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t wd[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint4 &q = vr[r].w;
          const uint32_t word = (i >> 1) == 0 ? q.x : (i >> 1) == 1 ? q.y : (i >> 1) == 2 ? q.z : q.w;
          wd[r] = word;
        }
        uint4 w;
        if (i & 1) {
          w.x = pack_hi16(wd[0], wd[1]); w.y = pack_hi16(wd[2], wd[3]);
          w.z = pack_hi16(wd[4], wd[5]); w.w = pack_hi16(wd[6], wd[7]);
        } else {
          w.x = pack_lo16(wd[0], wd[1]); w.y = pack_lo16(wd[2], wd[3]);
          w.z = pack_lo16(wd[4], wd[5]); w.w = pack_lo16(wd[6], wd[7]);
        }
        *reinterpret_cast<uint4 *>(vT + (8 * dc + i) * kRow16 + 8 * g) = w;
      }
    } else {
      float *cT = reinterpret_cast<float *>(lds_raw);
      float *vT = cT + kD * kRow32;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float *dst = cT + (8 * dc + i) * kRow32 + 8 * g;
        *reinterpret_cast<float4 *>(dst) = make_float4(c[0][i], c[1][i], c[2][i], c[3][i]);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(c[4][i], c[5][i], c[6][i], c[7][i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float vv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          float x[8];
          E::unpack(vr[r], x);
          vv[r] = x[i];
        }
        float *dst = vT + (8 * dc + i) * kRow32 + 8 * g;
        *reinterpret_cast<float4 *>(dst) = make_float4(vv[0], vv[1], vv[2], vv[3]);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(vv[4], vv[5], vv[6], vv[7]);
      }
    }
    __syncthreads();
    // next tile's loads fly while the matrix cores work on this one
    if (base + kTile < hi) load_tile(base + kTile);

    const int mb = wave >> 1, nb = wave & 1;
    if constexpr (kBF16) {
      const uint16_t *cT = reinterpret_cast<const uint16_t *>(lds_raw);
      const uint16_t *vT = cT + kD * kRow16;
      const uint16_t *arow = cT + (32 * mb + (lane & 31)) * kRow16 + 8 * (lane >> 5);
      const uint16_t *brow = vT + (32 * nb + (lane & 31)) * kRow16 + 8 * (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < kTile / 16; ++kk) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(arow + 16 * kk);
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(brow + 16 * kk);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      }
    } else {
      const float *cT = reinterpret_cast<const float *>(lds_raw);
      const float *vT = cT + kD * kRow32;
      const float *arow = cT + (32 * mb + (lane & 31)) * kRow32 + (lane >> 5);
      const float *brow = vT + (32 * nb + (lane & 31)) * kRow32 + (lane >> 5);
#pragma unroll 8
      for (int kk = 0; kk < kTile / 2; ++kk) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(arow[2 * kk], brow[2 * kk], acc, 0, 0, 0);
      }
    }
  }

  // partial record of this slab
  float *out = a.part + ((size_t)bh * a.n_chunks * a.slabs_per_chunk + slab_id) * kStateFloats;
  {
    const int mb = wave >> 1, nb = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * mb + 8 * i + 4 * (lane >> 5) + j;
        out[d * kD + 32 * nb + (lane & 31)] = acc[4 * i + j];
      }
  }
  // key sum: lanes with equal dc (lane bits 3..5 differ), then the four waves
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float s = zacc[i];
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    zacc[i] = s;
  }
  __syncthreads();
  float *zw = reinterpret_cast<float *>(lds_raw);  // [4][64]
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) zw[wave * kD + 8 * dc + i] = zacc[i];
  }
  __syncthreads();
  if (tid < kD) out[kD * kD + tid] = zw[tid] + zw[kD + tid] + zw[2 * kD + tid] + zw[3 * kD + tid];
}

// ---------------------------------------------------------------------------
// Fixed-order reduction of slab partials and inclusive prefix over chunks.
struct ScanArgs {
  const float *part;
  int n_chunks, slabs_per_chunk;
  const float *kv_in, *ksum_in;
  float *kv_out, *ksum_out;
  float *prefix;  // [B*H][n_chunks][kStateFloats]
};

__global__ __launch_bounds__(256) void la_scan_kernel(ScanArgs a) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= kStateFloats) return;
  const int bh = blockIdx.y;
  float run = 0.f;
  if (a.kv_in) run = idx < kD * kD ? a.kv_in[(size_t)bh * kD * kD + idx] : a.ksum_in[(size_t)bh * kD + idx - kD * kD];
  const int nsl = a.n_chunks * a.slabs_per_chunk;
  const float *p = a.part + (size_t)bh * nsl * kStateFloats + idx;
  float *pre = a.prefix + (size_t)bh * a.n_chunks * kStateFloats + idx;
  for (int c = 0; c < a.n_chunks; ++c) {
    float s = 0.f;
    for (int i = 0; i < a.slabs_per_chunk; ++i) s += p[(size_t)(c * a.slabs_per_chunk + i) * kStateFloats];
    run += s;
    pre[(size_t)c * kStateFloats] = run;
  }
  if (a.kv_out) {
    if (idx < kD * kD)
      a.kv_out[(size_t)bh * kD * kD + idx] = run;
    else
      a.ksum_out[(size_t)bh * kD + idx - kD * kD] = run;
  }
}

// ---------------------------------------------------------------------------
// Apply. Each wave handles 32 tokens per step: lane l holds token l%32 and
// the dims of its half (l/32). The numerator is computed transposed,
// O^T = P^T A^T, so the state is the matrix-core A operand (held in
// registers for the whole work-group) and each lane's B operand is a
// contiguous piece of its own token's q row; the result lands with every lane
// holding output dims of its own token, where the denominator and gate live.
struct ApplyArgs {
  const void *q, *g;
  void *o;
  int N, H, L, n_chunks, apply_tokens, apply_per_chunk;
  RopeArgs rope;
  float eps;
  const float *prefix;
};

// bf16 outputs: hardware exp and reciprocal (about 1 ulp); exactly 1/2 at 0.
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float sigmoid_exact(float x) { return 1.f / (1.f + expf(-x)); }

__global__ __launch_bounds__(256) void la_apply_bf16_kernel(ApplyArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, tl = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int chunk = blockIdx.x / a.apply_per_chunk;
  const int part = blockIdx.x - chunk * a.apply_per_chunk;
  const int c_lo = chunk * a.L;
  const int c_hi = min(a.N, c_lo + a.L);
  const int lo = c_lo + part * a.apply_tokens;
  const int hi = min(c_hi, lo + a.apply_tokens);
  if (lo >= hi) return;

  const float *P = a.prefix + ((size_t)bh * a.n_chunks + chunk) * kStateFloats;
  // A operand: P^T as hi + lo bf16 parts. Lane holds rows e = 32*mb + tl,
  // reduction index d = 16*s + 8*half + t.
  bf16x8_t shi[2][4], slo[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const float x0 = P[(16 * s + 8 * half + t) * kD + 32 * mb + tl];
        const float x1 = P[(16 * s + 8 * half + t + 1) * kD + 32 * mb + tl];
        const uint32_t hw = pack_bf16(x0, x1);
        wh[t / 2] = hw;
        wl[t / 2] = pack_bf16(x0 - bf16_lo(hw), x1 - bf16_hi(hw));
      }
      shi[mb][s] = __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
      slo[mb][s] = __builtin_bit_cast(bf16x8_t, make_uint4(wl[0], wl[1], wl[2], wl[3]));
    }
  float zr[4][8];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) zr[s][t] = P[kD * kD + 16 * s + 8 * half + t];

  RopePair rp[4][4];
  if (a.rope.enabled) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) rp[s][j] = rope_pair(a.rope, 8 * s + 4 * half + j);
  }

  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD;
  const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q) + head_base;
  const uint16_t *gp = a.g ? reinterpret_cast<const uint16_t *>(a.g) + head_base : nullptr;
  uint16_t *op = reinterpret_cast<uint16_t *>(a.o) + head_base;

  for (int sub = lo + kApplySub * wave; sub < hi; sub += 4 * kApplySub) {
    const int n = sub + tl;
    const bool valid = n < hi;
    const size_t row = (size_t)n * tok_stride;
    uint4 qr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qr[s] = valid ? *reinterpret_cast<const uint4 *>(qp + row + 16 * s + 8 * half) : make_uint4(0, 0, 0, 0);
    uint2 gr[2][4];
    if (gp) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gr[mb][i] = valid ? *reinterpret_cast<const uint2 *>(gp + row + 32 * mb + 8 * i + 4 * half) : make_uint2(0, 0);
    }
    TokenPos tp;
    if (a.rope.enabled) tp = token_pos(a.rope, (uint32_t)min(n, a.N - 1));
    float den = 0.f;
    bf16x8_t bq[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
      x[0] = bf16_lo(qr[s].x); x[1] = bf16_hi(qr[s].x);
      x[2] = bf16_lo(qr[s].y); x[3] = bf16_hi(qr[s].y);
      x[4] = bf16_lo(qr[s].z); x[5] = bf16_hi(qr[s].z);
      x[6] = bf16_lo(qr[s].w); x[7] = bf16_hi(qr[s].w);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[t] = fmaxf(x[t], 0.f);
        den += x[t] * zr[s][t];
      }
      if (a.rope.enabled) {
#pragma unroll
        for (int j = 0; j < 4; ++j) rotate(x[2 * j], x[2 * j + 1], rope_cs(rp[s][j], tp));
      }
      bq[s] = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]),
                                                      pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])));
    }
    f32x16_t acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi[mb][s], bq[s], acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo[mb][s], bq[s], acc[mb], 0, 0, 0);
      }
    }
    den += __shfl_xor(den, 32);
    const float inv = 1.f / (den + a.eps);
    if (valid) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = acc[mb][4 * i + j] * inv;
          if (gp) {
            y[0] *= sigmoid_fast(bf16_lo(gr[mb][i].x));
            y[1] *= sigmoid_fast(bf16_hi(gr[mb][i].x));
            y[2] *= sigmoid_fast(bf16_lo(gr[mb][i].y));
            y[3] *= sigmoid_fast(bf16_hi(gr[mb][i].y));
          }
          *reinterpret_cast<uint2 *>(op + row + 32 * mb + 8 * i + 4 * half) =
              make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
        }
    }
  }
}

// Float inputs: fp32 matrix cores (32x32x2) so nothing is rounded below fp32.
// Reduction index d = 32*half + s: each lane holds dims [32*half, 32*half+32)
// of its token, which keeps every RoPE pair inside one lane.
__global__ __launch_bounds__(256) void la_apply_f32_kernel(ApplyArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, tl = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int chunk = blockIdx.x / a.apply_per_chunk;
  const int part = blockIdx.x - chunk * a.apply_per_chunk;
  const int c_lo = chunk * a.L;
  const int c_hi = min(a.N, c_lo + a.L);
  const int lo = c_lo + part * a.apply_tokens;
  const int hi = min(c_hi, lo + a.apply_tokens);
  if (lo >= hi) return;

  const float *P = a.prefix + ((size_t)bh * a.n_chunks + chunk) * kStateFloats;
  float sa[2][32];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 32; ++s) sa[mb][s] = P[(32 * half + s) * kD + 32 * mb + tl];
  float zr[32];
#pragma unroll
  for (int s = 0; s < 32; ++s) zr[s] = P[kD * kD + 32 * half + s];

  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD;
  const float *qp = reinterpret_cast<const float *>(a.q) + head_base;
  const float *gp = a.g ? reinterpret_cast<const float *>(a.g) + head_base : nullptr;
  float *op = reinterpret_cast<float *>(a.o) + head_base;

  for (int sub = lo + kApplySub * wave; sub < hi; sub += 4 * kApplySub) {
    const int n = sub + tl;
    const bool valid = n < hi;
    const size_t row = (size_t)n * tok_stride;
    float x[32];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float4 v = valid ? *reinterpret_cast<const float4 *>(qp + row + 32 * half + 4 * s)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      x[4 * s] = v.x; x[4 * s + 1] = v.y; x[4 * s + 2] = v.z; x[4 * s + 3] = v.w;
    }
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      x[s] = fmaxf(x[s], 0.f);
      den += x[s] * zr[s];
    }
    if (a.rope.enabled) {
      const TokenPos tp = token_pos(a.rope, (uint32_t)min(n, a.N - 1));
#pragma unroll
      for (int j = 0; j < 16; ++j) rotate(x[2 * j], x[2 * j + 1], rope_cs(rope_pair(a.rope, 16 * half + j), tp));
    }
    f32x16_t acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < 32; ++s) acc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(sa[mb][s], x[s], acc[mb], 0, 0, 0);
    }
    den += __shfl_xor(den, 32);
    const float inv_den = den + a.eps;
    if (valid) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t off = row + 32 * mb + 8 * i + 4 * half;
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = acc[mb][4 * i + j] / inv_den;
          if (gp) {
            const float4 gv = *reinterpret_cast<const float4 *>(gp + off);
            y[0] *= sigmoid_exact(gv.x);
            y[1] *= sigmoid_exact(gv.y);
            y[2] *= sigmoid_exact(gv.z);
            y[3] *= sigmoid_exact(gv.w);
          }
          *reinterpret_cast<float4 *>(op + off) = make_float4(y[0], y[1], y[2], y[3]);
        }
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

LinearPlan plan_linear(int B, int N, int H, int chunk_tokens) {
  LinearPlan p;
  const long long L = chunk_tokens > 0 && chunk_tokens < N ? chunk_tokens : N;
  p.chunk_len = (int)L;
  p.n_chunks = (int)((N + L - 1) / L);
  const long long heads = (long long)B * H;
  // about 1024 build work-groups (4 per CU), slabs a multiple of the tile
  long long want = (heads * N + 1023) / 1024;
  long long slab = ((want + kTile - 1) / kTile) * kTile;
  if (slab < kTile) slab = kTile;
  const long long lt = ((L + kTile - 1) / kTile) * kTile;
  if (slab > lt) slab = lt;
  p.slab_tokens = (int)slab;
  p.slabs_per_chunk = (int)((L + slab - 1) / slab);
  // about 2048 apply work-groups, token ranges a multiple of 128
  long long awant = (heads * N + 2047) / 2048;
  long long at = ((awant + 127) / 128) * 128;
  if (at < 128) at = 128;
  const long long l128 = ((L + 127) / 128) * 128;
  if (at > l128) at = l128;
  p.apply_tokens = (int)at;
  p.apply_per_chunk = (int)((L + at - 1) / at);
  const size_t part_bytes = (size_t)heads * p.n_chunks * p.slabs_per_chunk * kStateFloats * sizeof(float);
  const size_t prefix_bytes = (size_t)heads * p.n_chunks * kStateFloats * sizeof(float);
  p.part_offset = 0;
  p.prefix_offset = align256(part_bytes);
  p.total_bytes = p.prefix_offset + align256(prefix_bytes);
  return p;
}

hipError_t launch_linear(hla_dtype dt, const LinearArgs &a, const LinearPlan &p, hipStream_t stream) {
  const int heads = a.B * a.H;
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(a.ws) + p.part_offset);
  float *prefix = reinterpret_cast<float *>(reinterpret_cast<char *>(a.ws) + p.prefix_offset);

  BuildArgs ba;
  ba.k = a.k;
  ba.v = a.v;
  ba.N = a.N;
  ba.H = a.H;
  ba.L = p.chunk_len;
  ba.n_chunks = p.n_chunks;
  ba.slab_tokens = p.slab_tokens;
  ba.slabs_per_chunk = p.slabs_per_chunk;
  ba.rope = a.rope;
  ba.part = part;
  const dim3 bgrid(p.n_chunks * p.slabs_per_chunk, heads);
  if (dt == HLA_BF16) {
    const size_t lds = 2 * kD * kRow16 * sizeof(uint16_t);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&la_build_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(la_build_kernel<true>, bgrid, dim3(256), lds, stream, ba);
  } else {
    const size_t lds = 2 * kD * kRow32 * sizeof(float);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&la_build_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(la_build_kernel<false>, bgrid, dim3(256), lds, stream, ba);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  ScanArgs sa;
  sa.part = part;
  sa.n_chunks = p.n_chunks;
  sa.slabs_per_chunk = p.slabs_per_chunk;
  sa.kv_in = a.kv_in;
  sa.ksum_in = a.ksum_in;
  sa.kv_out = a.kv_out;
  sa.ksum_out = a.ksum_out;
  sa.prefix = prefix;
  hipLaunchKernelGGL(la_scan_kernel, dim3((kStateFloats + 255) / 256, heads), dim3(256), 0, stream, sa);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  ApplyArgs aa;
  aa.q = a.q;
  aa.g = a.g;
  aa.o = a.o;
  aa.N = a.N;
  aa.H = a.H;
  aa.L = p.chunk_len;
  aa.n_chunks = p.n_chunks;
  aa.apply_tokens = p.apply_tokens;
  aa.apply_per_chunk = p.apply_per_chunk;
  aa.rope = a.rope;
  aa.eps = a.eps;
  aa.prefix = prefix;
  const dim3 agrid(p.n_chunks * p.apply_per_chunk, heads);
  if (dt == HLA_BF16)
    hipLaunchKernelGGL(la_apply_bf16_kernel, agrid, dim3(256), 0, stream, aa);
  else
    hipLaunchKernelGGL(la_apply_f32_kernel, agrid, dim3(256), 0, stream, aa);
  return hipGetLastError();
}

}  // namespace hla
