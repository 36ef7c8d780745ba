// ReLU-kernel linear attention with 3D RoPE after the ReLU, bidirectional and
// block-causal (SANA-Video notes, section 3.2 output equation and pseudocode;
// section 3.4 causal equation, constant-memory cache and Algorithm 1).
//
// One call runs three kernels on the caller's stream:
//   la_build  per (b, 4 heads, slab of tokens): c_j = RoPE(relu(k_j)) and
//             S_slab = sum_j c_j^T v_j on the matrix cores (bf16 operands,
//             fp32 accumulation; fp32 operands for float inputs), plus
//             z_slab = sum_j relu(k_j) on the vector ALUs. Slabs never straddle
//             a chunk boundary.
//   la_scan   per (b, h): fixed-order sum of the slab partials of each chunk
//             and an inclusive prefix over chunks, starting from the carried
//             state; writes one (KV, ksum) record per chunk and the final
//             state. A bidirectional call is the one-chunk case.
//   la_apply  per (b, 4 heads, token range inside one chunk):
//             a_i = RoPE(relu(q_i)), numerator a_i P_c on the matrix cores,
//             denominator relu(q_i).Z_c + eps, optional sigmoid gate, store.
// Work-groups are 4 waves, one head each, over the same tokens: the 4 waves'
// 128-byte rows of a token form one 512-byte span of the (B, N, H, 64)
// tensors, and heads vary fastest across the grid. Memory traffic is the K/V
// read of the build and the Q/G read and O write of the apply; the fp32
// partial states are ~2% on top.
#include <algorithm>

#include <type_traits>

#include "device_common.h"

namespace hla {

namespace {

constexpr int kHeadsPerWG = 4;        // one head per wave
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
    c.w = load_once_u4(p);
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
  const float *zw;  // kZW: per-token weight of the key sum, [B*H][N]
  int N, H, L, n_chunks, slabs_per_chunk, ngroups;
  RopeArgs rope;
  float *part;  // [B*H][n_chunks*slabs_per_chunk][kStateFloats]
};

constexpr int kWTile = 64;           // tokens per wave tile in the build
constexpr int kWRow16 = kWTile + 8;  // bf16 per LDS row (144 bytes)
constexpr int kWRow32 = kWTile + 4;  // floats per LDS row (272 bytes)
constexpr int kWaveLds16 = 2 * kD * kWRow16 * 2;  // C^T and V^T tiles of one wave
constexpr int kWaveLds32 = 2 * kD * kWRow32 * 4;

// 16-byte granule swizzle of the build's dim-major bf16 tiles. With 144-byte
// rows, flipping granule bits 1 and 2 by row bits 5 and 4 makes both access
// patterns hit 16 distinct bank groups per 16 lanes: the transposed stores
// (rows 8 apart) and the matrix-core operand loads (16 consecutive rows).
__device__ __forceinline__ int gran_swz(int row) { return (((row >> 5) & 1) << 1) | (((row >> 4) & 1) << 2); }

// RoPE of the state build for an aligned 8-dim chunk. A build lane rotates 8
// consecutive tokens, so it reads (cos, sin) from its band's table for the
// first of them and moves to the next position with the angle-addition
// identity: cos(a+u) = cos a cos u - sin a sin u, sin(a+u) = sin a cos u +
// cos a sin u, u being the band's unit angle (row 1 of the h or w table, whose
// rows start at position 0). A position that does not move by exactly one (a
// new row or frame, and the t band, whose table may start at an offset) is read
// from the table again. At most seven steps lie between a table read and its
// use, a few ulp on cos and sin.
struct RopeWalk {
  const float *col;
  int stride, band;
  bool can_step;
  f32x2_t unit[4];
  __device__ __forceinline__ void fetch(uint32_t pos, f32x2_t cs[4]) const {
    const float *q = col + (size_t)pos * stride;
    const f32x4_t a = *reinterpret_cast<const f32x4_t *>(q);
    const f32x4_t b = *reinterpret_cast<const f32x4_t *>(q + 4);
    cs[0] = f32x2_t{a.x, a.y};
    cs[1] = f32x2_t{a.z, a.w};
    cs[2] = f32x2_t{b.x, b.y};
    cs[3] = f32x2_t{b.z, b.w};
  }
  __device__ __forceinline__ void init(const RopeArgs &r, int chunk) {
    const RopePair p = rope_pair(r, 4 * chunk);
    col = p.col;
    stride = p.stride;
    band = p.band;
    can_step = band != 0 && (band == 1 ? r.h : r.w) >= 2;
    if (can_step) {
      fetch(1, unit);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) unit[j] = f32x2_t{1.f, 0.f};
    }
  }
  __device__ __forceinline__ uint32_t coord(const TokenPos &tp) const {
    return band == 0 ? tp.t : (band == 1 ? tp.y : tp.x);
  }
  // cs holds the pairs at position `from`; leave them at position `to`
  __device__ __forceinline__ void advance(uint32_t from, uint32_t to, f32x2_t cs[4]) const {
    if (to == from) return;
    if (can_step && to == from + 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float c = cs[j].x * unit[j].x - cs[j].y * unit[j].y;
        const float sn = cs[j].y * unit[j].x + cs[j].x * unit[j].y;
        cs[j] = f32x2_t{c, sn};
      }
    } else {
      fetch(to, cs);
    }
  }
};

// ---------------------------------------------------------------------------
// State build. Wave w of a work-group owns head 4*g + w of one slab and streams
// its 64-token tiles with no work-group barrier. The tiles of a chunk are dealt
// out to its S slabs in turn (slab s takes tiles s, s+S, s+2S, ...), so at any
// moment the running work-groups read one contiguous window of K and V; giving
// each slab a contiguous token range instead spaces the concurrent streams by
// a fixed stride and loses up to a fifth of the bandwidth to uneven use of the
// memory channels. Lane (dc = lane%8,
// g = lane/8) loads dims 8*dc..+7 of tokens 8*g..+7: every load instruction
// reads eight whole 128-byte token rows. The lane applies relu and RoPE, then
// stores its 8x8 block transposed into the wave's LDS tiles (dim-major,
// token-contiguous), the layout the matrix cores need because S = C^T V
// reduces over tokens. The wave accumulates all of S (four 32x32 blocks) and
// writes its slab's partial (S, z) record at the end. With kZW the key sum
// weights token j by zw_j (the gradient pass sums dden_i relu(q_i) this way).
template <bool kBF16, bool kRope, bool kAligned, bool kZW>
__global__ __launch_bounds__(256, kBF16 ? 2 : 1) void la_build_kernel(BuildArgs a) {
  typedef Elem<kBF16> E;
  typedef typename E::T T;
  extern __shared__ __align__(16) unsigned char lds_raw[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int dc = lane & 7, g = lane >> 3;
  const int half = lane >> 5, tl = lane & 31;

  const int hgroup = blockIdx.x % a.ngroups;
  const int slab_id = blockIdx.x / a.ngroups;
  const int h = kHeadsPerWG * hgroup + wave;
  if (h >= a.H) return;  // no work-group barrier follows
  const int b = blockIdx.y;
  const int bh = b * a.H + h;
  const int chunk = slab_id / a.slabs_per_chunk;
  const int slab = slab_id - chunk * a.slabs_per_chunk;
  const int c_lo = chunk * a.L;
  const int c_hi = min(a.N, c_lo + a.L);

  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD + dc * 8;
  const T *kp = reinterpret_cast<const T *>(a.k) + head_base;
  const T *vp = reinterpret_cast<const T *>(a.v) + head_base;
  const float *zwp = kZW ? a.zw + (size_t)bh * a.N : nullptr;

  // aligned bands: walk the positions; otherwise look every pair up
  RopeWalk walk;
  ChunkRope<false> cr;
  if constexpr (kRope && kAligned) walk.init(a.rope, dc);
  if constexpr (kRope && !kAligned) cr.init(a.rope, dc);

  float zacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zacc[i] = 0.f;
  f32x16_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  unsigned char *wl = lds_raw + wave * (kBF16 ? kWaveLds16 : kWaveLds32);

  const int tile_step = a.slabs_per_chunk * kWTile;
  for (int base = c_lo + slab * kWTile; base < c_hi; base += tile_step) {
    const int hi = min(c_hi, base + kWTile);
    // Every load of the tile is issued before any use: token indices past the
    // tile are clamped to its last token (always valid) and zeroed afterwards.
    typename E::Chunk kr[8], vr[8];
    f32x2_t cs[(kRope && !kAligned) ? 8 : 1][4];
    f32x2_t cur[4];
    uint32_t cpos = 0;
    // V first: it is transposed into LDS (freeing its registers) while K lands
#pragma unroll
    for (int r = 0; r < 8; ++r) vr[r] = E::load(vp + (size_t)min(base + 8 * g + r, hi - 1) * tok_stride);
#pragma unroll
    for (int r = 0; r < 8; ++r) kr[r] = E::load(kp + (size_t)min(base + 8 * g + r, hi - 1) * tok_stride);
    float zw[kZW ? 8 : 1];
    if constexpr (kZW) {
#pragma unroll
      for (int r = 0; r < 8; ++r) zw[r] = zwp[min(base + 8 * g + r, hi - 1)];
    }
    if constexpr (kRope && kAligned) {
      cpos = walk.coord(token_pos(a.rope, (uint32_t)min(base + 8 * g, hi - 1)));
      walk.fetch(cpos, cur);
    } else if constexpr (kRope) {
#pragma unroll
      for (int r = 0; r < 8; ++r) cr.get(token_pos(a.rope, (uint32_t)min(base + 8 * g + r, hi - 1)), cs[r]);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (base + 8 * g + r >= hi) vr[r] = E::zero();
    if constexpr (kBF16) {
      uint16_t *vT = reinterpret_cast<uint16_t *>(wl) + kD * kWRow16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t wd[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint4 &q = vr[r].w;
          wd[r] = (i >> 1) == 0 ? q.x : (i >> 1) == 1 ? q.y : (i >> 1) == 2 ? q.z : q.w;
        }
        uint4 w;
        if (i & 1) {
          w = make_uint4(pack_hi16(wd[0], wd[1]), pack_hi16(wd[2], wd[3]), pack_hi16(wd[4], wd[5]),
                         pack_hi16(wd[6], wd[7]));
        } else {
          w = make_uint4(pack_lo16(wd[0], wd[1]), pack_lo16(wd[2], wd[3]), pack_lo16(wd[4], wd[5]),
                         pack_lo16(wd[6], wd[7]));
        }
        const int row = 8 * dc + i;
        *reinterpret_cast<uint4 *>(vT + row * kWRow16 + 8 * (g ^ gran_swz(row))) = w;
      }
    } else {
      float *vT = reinterpret_cast<float *>(wl) + kD * kWRow32;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float vv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          float x[8];
          E::unpack(vr[r], x);
          vv[r] = x[i];
        }
        float *dst = vT + (8 * dc + i) * kWRow32 + 8 * g;
        *reinterpret_cast<float4 *>(dst) = make_float4(vv[0], vv[1], vv[2], vv[3]);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(vv[4], vv[5], vv[6], vv[7]);
      }
    }
    // relu, key sum, rotation; bf16 tiles pack token pairs right away
    float c[kBF16 ? 1 : 8][8];
    uint32_t pk[8][4];
    float prev[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (base + 8 * g + r >= hi) kr[r] = E::zero();
      float x[8];
      E::unpack(kr[r], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = relu(x[i]);
        if constexpr (kZW)
          zacc[i] += zw[r] * x[i];
        else
          zacc[i] += x[i];
      }
      if constexpr (kRope && kAligned) {
        if (r > 0) {
          const uint32_t np = walk.coord(token_pos(a.rope, (uint32_t)min(base + 8 * g + r, hi - 1)));
          walk.advance(cpos, np, cur);
          cpos = np;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) rotate(x[2 * j], x[2 * j + 1], cur[j]);
      } else if constexpr (kRope) {
#pragma unroll
        for (int j = 0; j < 4; ++j) rotate(x[2 * j], x[2 * j + 1], cs[r][j]);
      }
      if constexpr (kBF16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (r & 1)
            pk[i][r >> 1] = pack_bf16(prev[i], x[i]);
          else
            prev[i] = x[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[r][i] = x[i];
      }
    }
    if constexpr (kBF16) {
      uint16_t *cT = reinterpret_cast<uint16_t *>(wl);
      const uint16_t *vT = cT + kD * kWRow16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * dc + i;
        *reinterpret_cast<uint4 *>(cT + row * kWRow16 + 8 * (g ^ gran_swz(row))) =
            make_uint4(pk[i][0], pk[i][1], pk[i][2], pk[i][3]);
      }
      wave_lds_fence();
      const int r0 = tl, r1 = 32 + tl;
#pragma unroll
      for (int kk = 0; kk < kWTile / 16; ++kk) {
        const int G = 2 * kk + half;
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t *>(cT + r0 * kWRow16 + 8 * (G ^ gran_swz(r0)));
        const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t *>(cT + r1 * kWRow16 + 8 * (G ^ gran_swz(r1)));
        const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t *>(vT + r0 * kWRow16 + 8 * (G ^ gran_swz(r0)));
        const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t *>(vT + r1 * kWRow16 + 8 * (G ^ gran_swz(r1)));
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
      }
    } else {
      float *cT = reinterpret_cast<float *>(wl);
      const float *vT = cT + kD * kWRow32;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float *dst = cT + (8 * dc + i) * kWRow32 + 8 * g;
        *reinterpret_cast<float4 *>(dst) = make_float4(c[0][i], c[1][i], c[2][i], c[3][i]);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(c[4][i], c[5][i], c[6][i], c[7][i]);
      }
      wave_lds_fence();
      const float *a0p = cT + tl * kWRow32 + half, *a1p = cT + (32 + tl) * kWRow32 + half;
      const float *b0p = vT + tl * kWRow32 + half, *b1p = vT + (32 + tl) * kWRow32 + half;
#pragma unroll 4
      for (int kk = 0; kk < kWTile / 2; ++kk) {
        const float a0 = a0p[2 * kk], a1 = a1p[2 * kk], b0 = b0p[2 * kk], b1 = b1p[2 * kk];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
    }
    wave_lds_fence();  // the next tile's stores come after these loads
  }

  // key sum of the wave: lanes with equal dc differ in lane bits 3..5
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float s = zacc[i];
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    zacc[i] = s;
  }
  float *out = a.part + ((size_t)bh * a.n_chunks * a.slabs_per_chunk + slab_id) * kStateFloats;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) out[(32 * mb + 8 * i + 4 * half + j) * kD + 32 * nb + tl] = acc[mb][nb][4 * i + j];
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[kD * kD + 8 * dc + i] = zacc[i];
  }
}

// ---------------------------------------------------------------------------
// Fixed-order reduction of slab partials and inclusive prefix over chunks
// (inclusive suffix, from the last chunk back, for the gradient pass).
struct ScanArgs {
  const float *part;
  int n_chunks, slabs_per_chunk;
  const float *kv_in, *ksum_in;
  float *kv_out, *ksum_out;
  float *prefix;  // [B*H][n_chunks][kStateFloats]
  float *init;    // nullable: receives the incoming state (kv_in or zero) [B*H][kStateFloats]
  int reverse;    // suffix sums: chunks from the last one back
};

__global__ __launch_bounds__(256) void la_scan_kernel(ScanArgs a) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= kStateFloats) return;
  const int bh = blockIdx.y;
  float run = 0.f;
  if (a.kv_in) run = idx < kD * kD ? a.kv_in[(size_t)bh * kD * kD + idx] : a.ksum_in[(size_t)bh * kD + idx - kD * kD];
  // a copy of the incoming state for readers that run after kv_out (which may
  // alias kv_in) has been written
  if (a.init) a.init[(size_t)bh * kStateFloats + idx] = run;
  const int nsl = a.n_chunks * a.slabs_per_chunk;
  const float *p = a.part + (size_t)bh * nsl * kStateFloats + idx;
  float *pre = a.prefix + (size_t)bh * a.n_chunks * kStateFloats + idx;
  // Slabs are summed in index order from zero, then added to the running state,
  // chunk by chunk in scan order. With eight or more slabs per chunk their loads
  // go out in batches of sixteen (eight below sixteen slabs) with no store
  // between them; indices past the last slab repeat it and are not added. With
  // fewer, the (chunk, slab) partials are loaded sixteen at a time across chunks
  // before any of them is added: a prefix store could otherwise be taken to
  // alias the next chunk's partials, one memory round trip per chunk.
  const int spc = a.slabs_per_chunk;
  auto chunk_sum = [&](const float *pc, auto width_c) {
    constexpr int W = decltype(width_c)::value;
    float s = 0.f;
    for (int i = 0; i < spc; i += W) {
      float x[W];
#pragma unroll
      for (int j = 0; j < W; ++j) x[j] = pc[(size_t)min(i + j, spc - 1) * kStateFloats];
#pragma unroll
      for (int j = 0; j < W; ++j)
        if (i + j < spc) s += x[j];
    }
    return s;
  };
  if (spc >= 8) {
    for (int ci = 0; ci < a.n_chunks; ++ci) {
      const int c = a.reverse ? a.n_chunks - 1 - ci : ci;
      const float *pc = p + (size_t)c * spc * kStateFloats;
      run += spc >= 16 ? chunk_sum(pc, std::integral_constant<int, 16>{}) : chunk_sum(pc, std::integral_constant<int, 8>{});
      pre[(size_t)c * kStateFloats] = run;
    }
  } else {
    int lc = 0, ls = 0;  // next partial to load: chunk (scan order), slab
    int sc = 0, ss = 0;  // next partial to add
    float s = 0.f;
    for (int t0 = 0; t0 < nsl; t0 += 16) {
      float x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // past the end: a repeat of the last partial, never added
        const int ci = min(lc, a.n_chunks - 1);
        const int c = a.reverse ? a.n_chunks - 1 - ci : ci;
        x[j] = p[((size_t)c * spc + (lc < a.n_chunks ? ls : spc - 1)) * kStateFloats];
        if (++ls == spc) {
          ls = 0;
          ++lc;
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (t0 + j < nsl) {
          s += x[j];
          if (++ss == spc) {
            const int c = a.reverse ? a.n_chunks - 1 - sc : sc;
            run += s;
            pre[(size_t)c * kStateFloats] = run;
            s = 0.f;
            ss = 0;
            ++sc;
          }
        }
    }
  }
  if (a.kv_out) {
    if (idx < kD * kD)
      a.kv_out[(size_t)bh * kD * kD + idx] = run;
    else
      a.ksum_out[(size_t)bh * kD + idx - kD * kD] = run;
  }
}

struct ApplyArgs {
  const void *q, *g;
  void *o;
  int N, H, L, n_chunks, apply_per_chunk, ngroups;
  RopeArgs rope;
  float eps;
  const float *prefix;
  int tab_t, tab_h, tab_w;  // floats in each band's table (LDS-staged RoPE)
};

// RoPE variants of the bf16 apply
constexpr int kRopeNone = 0;    // no rotation
constexpr int kRopePair = 1;    // any band widths: each pair looked up in global memory
constexpr int kRopeGlobal = 2;  // band widths multiples of 8: two 16-byte global loads per 8 dims
constexpr int kRopeLds = 3;     // as kRopeGlobal, from a copy of the tables in LDS
constexpr int kTabLdsFloats = 9216;  // largest table set staged in LDS (36 KB)

extern __shared__ __align__(16) float la_tab_lds[];

// (cos, sin) of the four pairs of one 8-dim chunk from the LDS copy of the
// tables, laid out [t table | h table | w table].
struct ChunkRopeLds {
  int off, stride, band;
  __device__ __forceinline__ void init(const RopeArgs &r, const ApplyArgs &a, int chunk) {
    const int two_p = 8 * chunk;
    if (two_p < r.d_t) {
      off = two_p;
      stride = r.d_t;
      band = 0;
    } else if (two_p < r.d_t + r.d_h) {
      off = a.tab_t + two_p - r.d_t;
      stride = r.d_h;
      band = 1;
    } else {
      off = a.tab_t + a.tab_h + two_p - r.d_t - r.d_h;
      stride = r.d_w;
      band = 2;
    }
  }
  __device__ __forceinline__ void get(const TokenPos &tp, f32x2_t cs[4]) const {
    const uint32_t pos = band == 0 ? tp.t : (band == 1 ? tp.y : tp.x);
    const int i = off + (int)pos * stride;
    const f32x4_t a = *reinterpret_cast<const f32x4_t *>(&la_tab_lds[i]);
    const f32x4_t b = *reinterpret_cast<const f32x4_t *>(&la_tab_lds[i + 4]);
    cs[0] = f32x2_t{a.x, a.y};
    cs[1] = f32x2_t{a.z, a.w};
    cs[2] = f32x2_t{b.x, b.y};
    cs[3] = f32x2_t{b.z, b.w};
  }
};

// ---------------------------------------------------------------------------
// Apply. Wave w of a work-group owns head 4*g + w of one part of a chunk and
// walks it 32 tokens at a time; the 32-token steps of a chunk are dealt out to
// its parts in turn (part p takes steps p, p+A, p+2A, ...), for the same reason
// as the build's tiles. Q and G are loaded as whole 128-byte
// rows (lane = token 8u + lane/8, dims 8*(lane%8)..+7) and turned into the
// matrix-core lane layout through a per-wave LDS stage; O goes back through
// the stage to whole-row non-temporal stores.
// In the lane layout, lane l holds token l%32 and the dims of its half (l/32).
// The numerator is computed transposed, O^T = P^T A^T: the chunk's state P^T
// (bf16 hi + lo parts, held in registers) is the A operand and each lane's B
// operand is a contiguous piece of its own token's q row; the result lands
// with every lane holding output dims of its own token, where the denominator
// and the gate are applied. The rows of P^T are permuted (output row
// m = 8i + 4h + j of a 32x32 product holds dim 16h + 4i + j), so the 16
// results of a lane are 16 consecutive dims.
constexpr int kStageRow = kD + 8;  // bf16 per staged token row (144 bytes)

template <int kRopeMode, bool kGate>
__global__ __launch_bounds__(256, kRopeMode == kRopePair ? 1 : 2) void la_apply_bf16_kernel(ApplyArgs a) {
  constexpr bool kRope = kRopeMode != kRopeNone;
  __shared__ __align__(16) uint16_t stage_all[kHeadsPerWG][kApplySub * kStageRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, tl = lane & 31;
  const int r8 = lane >> 3, c8 = lane & 7;
  const int hgroup = blockIdx.x % a.ngroups;
  const int pid = blockIdx.x / a.ngroups;
  const int chunk = pid / a.apply_per_chunk;
  const int part = pid - chunk * a.apply_per_chunk;
  const int c_lo = chunk * a.L;
  const int c_hi = min(a.N, c_lo + a.L);
  const int first = c_lo + part * kApplySub;
  if (first >= c_hi) return;  // the same for the whole work-group
  const int sub_step = a.apply_per_chunk * kApplySub;
  if constexpr (kRopeMode == kRopeLds) {
    // copy the three tables into LDS (each a multiple of 8 floats)
    const int n4 = (a.tab_t + a.tab_h + a.tab_w) / 4;
    for (int i = tid; i < n4; i += 256) {
      const int f = 4 * i;
      const float *src = f < a.tab_t ? a.rope.cs_t + f
                                      : (f < a.tab_t + a.tab_h ? a.rope.cs_h + (f - a.tab_t)
                                                               : a.rope.cs_w + (f - a.tab_t - a.tab_h));
      *reinterpret_cast<f32x4_t *>(&la_tab_lds[f]) = *reinterpret_cast<const f32x4_t *>(src);
    }
    __syncthreads();
  }
  const int h = kHeadsPerWG * hgroup + wave;
  if (h >= a.H) return;  // no work-group barrier follows
  const int b = blockIdx.y;
  const int bh = b * a.H + h;

  // A operand: P^T as hi + lo bf16 parts. Lane holds output row tl of block
  // mb (dim 32*mb + el) and reduction index d = 16*s + 8*half + t.
  const float *P = a.prefix + ((size_t)bh * a.n_chunks + chunk) * kStateFloats;
  const int el = (((tl >> 2) & 1) << 4) | ((tl >> 3) << 2) | (tl & 3);
  bf16x8_t shi[2][4], slo[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const float x0 = P[(16 * s + 8 * half + t) * kD + 32 * mb + el];
        const float x1 = P[(16 * s + 8 * half + t + 1) * kD + 32 * mb + el];
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

  ChunkRope<kRopeMode != kRopePair> cr[4];
  ChunkRopeLds crl[4];
  if constexpr (kRopeMode == kRopeLds) {
#pragma unroll
    for (int s = 0; s < 4; ++s) crl[s].init(a.rope, a, 2 * s + half);
  } else if constexpr (kRope) {
#pragma unroll
    for (int s = 0; s < 4; ++s) cr[s].init(a.rope, 2 * s + half);
  }

  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD;
  const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q) + head_base + 8 * c8;
  const uint16_t *gp = reinterpret_cast<const uint16_t *>(a.g) + head_base + 8 * c8;
  uint16_t *op = reinterpret_cast<uint16_t *>(a.o) + head_base + 8 * c8;
  uint16_t *st = stage_all[wave];

  for (int sub = first; sub < c_hi; sub += sub_step) {
    const int hi = min(c_hi, sub + kApplySub);
    // whole-row loads; tokens past the step read the last valid token
    u32x4_t qrow[4], grow[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t n = (size_t)min(sub + 8 * u + r8, hi - 1);
      qrow[u] = load_once16(qp + n * tok_stride);
      if constexpr (kGate) grow[u] = load_once16(gp + n * tok_stride);
    }
    f32x2_t cs[kRope ? 4 : 1][4];
    if constexpr (kRope) {
      const TokenPos tp = token_pos(a.rope, (uint32_t)min(sub + tl, hi - 1));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (kRopeMode == kRopeLds)
          crl[s].get(tp, cs[s]);
        else
          cr[s].get(tp, cs[s]);
      }
    }
    // q rows -> lane layout
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4_t *>(st + (8 * u + r8) * kStageRow + 8 * c8) = qrow[u];
    wave_lds_fence();
    u32x4_t qr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qr[s] = *reinterpret_cast<const u32x4_t *>(st + tl * kStageRow + 16 * s + 8 * half);
    u32x4_t gr[2][2];
    if constexpr (kGate) {
      wave_lds_fence();
#pragma unroll
      for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4_t *>(st + (8 * u + r8) * kStageRow + 8 * c8) = grow[u];
      wave_lds_fence();
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 2; ++v)
          gr[mb][v] = *reinterpret_cast<const u32x4_t *>(st + tl * kStageRow + 32 * mb + 16 * half + 8 * v);
    }

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
        x[t] = relu(x[t]);
        den += x[t] * zr[s][t];
      }
      if constexpr (kRope) {
#pragma unroll
        for (int j = 0; j < 4; ++j) rotate(x[2 * j], x[2 * j + 1], cs[s][j]);
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
    // normalise and gate in the lane layout, back to rows through the stage
    wave_lds_fence();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = acc[mb][8 * v + j] * inv;
        if constexpr (kGate) {
          const u32x4_t gw = gr[mb][v];
          y[0] *= sigmoid_fast(bf16_lo(gw.x));
          y[1] *= sigmoid_fast(bf16_hi(gw.x));
          y[2] *= sigmoid_fast(bf16_lo(gw.y));
          y[3] *= sigmoid_fast(bf16_hi(gw.y));
          y[4] *= sigmoid_fast(bf16_lo(gw.z));
          y[5] *= sigmoid_fast(bf16_hi(gw.z));
          y[6] *= sigmoid_fast(bf16_lo(gw.w));
          y[7] *= sigmoid_fast(bf16_hi(gw.w));
        }
        *reinterpret_cast<u32x4_t *>(st + tl * kStageRow + 32 * mb + 16 * half + 8 * v) =
            u32x4_t{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
      }
    wave_lds_fence();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = sub + 8 * u + r8;
      const u32x4_t w = *reinterpret_cast<const u32x4_t *>(st + (8 * u + r8) * kStageRow + 8 * c8);
      if (n < hi) store_nt(op + (size_t)n * tok_stride, w);
    }
    wave_lds_fence();  // the next step's stage stores come after these loads
  }
}

// Float inputs: fp32 matrix cores (32x32x2) so nothing is rounded below fp32.
// Reduction index d = 32*half + s: each lane holds dims [32*half, 32*half+32)
// of its token, which keeps every RoPE pair inside one lane.
__global__ __launch_bounds__(256) void la_apply_f32_kernel(ApplyArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, tl = lane & 31;
  const int hgroup = blockIdx.x % a.ngroups;
  const int pid = blockIdx.x / a.ngroups;
  const int h = kHeadsPerWG * hgroup + wave;
  if (h >= a.H) return;
  const int b = blockIdx.y;
  const int bh = b * a.H + h;
  const int chunk = pid / a.apply_per_chunk;
  const int part = pid - chunk * a.apply_per_chunk;
  const int c_lo = chunk * a.L;
  const int c_hi = min(a.N, c_lo + a.L);
  const int first = c_lo + part * kApplySub;
  if (first >= c_hi) return;  // no work-group barrier follows
  const int sub_step = a.apply_per_chunk * kApplySub;

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

  for (int sub = first; sub < c_hi; sub += sub_step) {
    const int hi = min(c_hi, sub + kApplySub);
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
      x[s] = relu(x[s]);
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


// ---------------------------------------------------------------------------
// Token-causal apply (bf16). Token i sees the state of every token j <= i:
//   o_i = (a_i (P + sum_{j<=i, j in range} c_j^T v_j)) /
//         (phi(q_i) . (z + sum_{j<=i} phi(k_j)) + eps)
// with (P, z) the state of all tokens before the range (exclusive prefix).
// A wave owns one head of one token range and walks it in 32-token steps,
// carrying the state S (fp32, in matrix-core accumulators) and the key sum z
// (in LDS). Per step, with i the query and j the key within the step:
//   O^T  = S^T a^T                      inter-step part (S as bf16 hi + lo)
//   T^T  = C A^T, U^T = phi(K) phi(Q)^T  scores, rotated and plain
//   O^T += V^T (T^T masked to j <= i)   intra-step part (T as bf16 hi + lo)
//   den  = phi(q_i).z + sum_{j<=i} U^T[j][i] + eps
//   S   += C^T V,  z += sum_j phi(k_j)   (after this step's outputs)
// Dim order. Every product over dims uses the order the state accumulators
// hold: lane half h supplies dims d0..d0+3 and d0+8..d0+11, d0 = 32kb + 16s +
// 4h, for reduction step (kb, s). q and k are loaded in that order (8-byte
// pieces), so S's accumulator entries 8s..8s+7 are directly the A operand of
// the inter-step product. Key order. C^T and V^T go to LDS transposed with the
// keys of each group of 16 permuted (bits 2 and 3 swapped), so that the masked
// scores, read from their accumulators as the B operand of the P.V product,
// match contiguous 16-byte reads of V^T; the state update reads C^T and V^T
// with the same key order on both sides.
constexpr int kCtRow = kApplySub + 8;  // bf16 per transposed row (32 keys + pad)

struct CausalArgs {
  const uint16_t *q, *k, *v, *g;
  uint16_t *o;
  int N, H, L, n_chunks, ngroups;
  RopeArgs rope;
  float eps;
  const float *prefix;  // inclusive prefix per range: [B*H][n_chunks][kStateFloats]
  const float *init;    // state before the first range: [B*H][kStateFloats]
  int tab_t, tab_h, tab_w;  // floats in each band's table (LDS-staged RoPE)
};

__device__ __forceinline__ int key_perm(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// (cos, sin) of the two pairs of the 4-dim run starting at dim d (d % 4 == 0)
__device__ __forceinline__ f32x4_t rope_run(const RopeArgs &r, const TokenPos &tp, int d) {
  const float *col;
  int stride;
  uint32_t pos;
  if (d < r.d_t) {
    col = r.cs_t + d;
    stride = r.d_t;
    pos = tp.t;
  } else if (d < r.d_t + r.d_h) {
    col = r.cs_h + (d - r.d_t);
    stride = r.d_h;
    pos = tp.y;
  } else {
    col = r.cs_w + (d - r.d_t - r.d_h);
    stride = r.d_w;
    pos = tp.x;
  }
  return *reinterpret_cast<const f32x4_t *>(col + (size_t)pos * stride);
}

// the same from the LDS copy of the tables, laid out [t table | h table | w table]
__device__ __forceinline__ f32x4_t rope_run_lds(const RopeArgs &r, const CausalArgs &a, const TokenPos &tp, int d) {
  int i;
  if (d < r.d_t)
    i = d + (int)tp.t * r.d_t;
  else if (d < r.d_t + r.d_h)
    i = a.tab_t + (d - r.d_t) + (int)tp.y * r.d_h;
  else
    i = a.tab_t + a.tab_h + (d - r.d_t - r.d_h) + (int)tp.x * r.d_w;
  return *reinterpret_cast<const f32x4_t *>(&la_tab_lds[i]);
}

// kRopeMode: kRopeNone, kRopeGlobal (tables read from global memory) or
// kRopeLds (tables copied to LDS first: every lookup of a step would otherwise
// be a global round trip on the step's critical path)
template <int kRopeMode, bool kGate>
__global__ __launch_bounds__(256, 2) void la_causal_kernel(CausalArgs a) {
  constexpr bool kRope = kRopeMode != kRopeNone;
  __shared__ __align__(16) uint16_t ct_all[kHeadsPerWG][kD * kCtRow];
  __shared__ __align__(16) uint16_t vt_all[kHeadsPerWG][kD * kCtRow];
  __shared__ __align__(16) float z_all[kHeadsPerWG][kD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: head and bases in scalar registers
  const int half = lane >> 5, tl = lane & 31;
  const int hgroup = blockIdx.x % a.ngroups;
  const int rng = blockIdx.x / a.ngroups;
  if constexpr (kRopeMode == kRopeLds) {
    // copy the three tables into LDS (each a multiple of 4 floats)
    const int n4 = (a.tab_t + a.tab_h + a.tab_w) / 4;
    for (int i = tid; i < n4; i += 256) {
      const int f = 4 * i;
      const float *src = f < a.tab_t ? a.rope.cs_t + f
                                      : (f < a.tab_t + a.tab_h ? a.rope.cs_h + (f - a.tab_t)
                                                               : a.rope.cs_w + (f - a.tab_t - a.tab_h));
      *reinterpret_cast<f32x4_t *>(&la_tab_lds[f]) = *reinterpret_cast<const f32x4_t *>(src);
    }
    __syncthreads();
  }
  const int h = kHeadsPerWG * hgroup + wave;
  if (h >= a.H) return;  // no work-group barrier follows
  const int b = blockIdx.y;
  const int bh = b * a.H + h;
  const int lo = rng * a.L;
  const int hi_r = min(a.N, lo + a.L);
  if (lo >= hi_r) return;
  uint16_t *ct = ct_all[wave];
  uint16_t *vt = vt_all[wave];
  float *zs = z_all[wave];

  // state before the range: S[d][e] in accumulator layout (rows d, column e)
  const float *P = rng > 0 ? a.prefix + ((size_t)bh * a.n_chunks + rng - 1) * kStateFloats
                           : a.init + (size_t)bh * kStateFloats;
  const float *Pz = P + kD * kD;
  f32x16_t sacc[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[kb][nb][4 * i + j] = P[(32 * kb + 8 * i + 4 * half + j) * kD + 32 * nb + tl];
  zs[lane] = Pz[lane];
  wave_lds_fence();

  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD;
  const int kp_self = key_perm(tl);

  for (int sub = lo; sub < hi_r; sub += kApplySub) {
    const int hi = min(hi_r, sub + kApplySub);
    const int n = sub + tl;
    const bool valid = n < hi;
    // the step's rows: a wave-uniform base plus one 32-bit byte offset per lane,
    // shared by q, k, v, g and o (one layout); keeps 64-bit lane addresses out
    // of the step's registers
    const size_t step_base = head_base + (size_t)sub * tok_stride;
    const int row = min(tl, hi - 1 - sub);  // rows past the end read the last one
    const uint32_t roff = (uint32_t)row * (uint32_t)(tok_stride * sizeof(uint16_t));
    auto at = [&](const uint16_t *base, int d) {
      return reinterpret_cast<const char *>(base + step_base) + roff + d * sizeof(uint16_t);
    };

    // Every global read of the step is issued here, before any of them is
    // used (v as 16-byte pieces; q and k as 8-byte pieces in the state's dim
    // order, per reduction step; the gate pieces of the output): the step
    // waits for one memory round trip instead of one per reduction step, one
    // for the gate and one for its first V^T write.
    uint4 vp[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) vp[s] = *reinterpret_cast<const uint4 *>(at(a.v, 16 * s + 8 * half));
    uint2 qkp[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int d0 = 32 * (st >> 1) + 16 * (st & 1) + 4 * half;
      qkp[st][0] = *reinterpret_cast<const uint2 *>(at(a.q, d0));
      qkp[st][1] = *reinterpret_cast<const uint2 *>(at(a.q, d0 + 8));
      qkp[st][2] = *reinterpret_cast<const uint2 *>(at(a.k, d0));
      qkp[st][3] = *reinterpret_cast<const uint2 *>(at(a.k, d0 + 8));
    }
    uint2 gws[2][4];
    if constexpr (kGate) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) gws[mb][i] = *reinterpret_cast<const uint2 *>(at(a.g, 32 * mb + 8 * i + 4 * half));
    }
    TokenPos tp;
    if constexpr (kRope) tp = token_pos(a.rope, (uint32_t)(sub + row));
    if (!valid) {
#pragma unroll
      for (int s = 0; s < 4; ++s) vp[s] = make_uint4(0, 0, 0, 0);
    }

    // V^T to LDS: row = dim, column = permuted key
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w[4] = {vp[s].x, vp[s].y, vp[s].z, vp[s].w};
#pragma unroll
      for (int t = 0; t < 8; ++t)
        vt[(16 * s + 8 * half + t) * kCtRow + kp_self] = (uint16_t)((t & 1) ? (w[t >> 1] >> 16) : (w[t >> 1] & 0xFFFFu));
    }

    f32x16_t tacc, uacc, oacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      tacc[i] = 0.f;
      uacc[i] = 0.f;
      oacc[0][i] = 0.f;
      oacc[1][i] = 0.f;
    }
    float den_in = 0.f;
    // the key-sum slot this lane's butterfly result adds to, less 32 kb + 16 s2
    const int zt = 4 * ((lane >> 4) & 1) + 2 * ((lane >> 3) & 1) + ((lane >> 2) & 1);
    const int zslot = 4 * half + (zt < 4 ? zt : 4 + zt);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1, s2 = st & 1;
      const int d0 = 32 * kb + 16 * s2 + 4 * half;
      float fq[8], fk[8];
      uint2 q0 = qkp[st][0], q1 = qkp[st][1], k0 = qkp[st][2], k1 = qkp[st][3];
      if (!valid) q0 = q1 = k0 = k1 = make_uint2(0, 0);
      const uint32_t qw[4] = {q0.x, q0.y, q1.x, q1.y};
      const uint32_t kw[4] = {k0.x, k0.y, k1.x, k1.y};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        fq[2 * u] = relu(bf16_lo(qw[u]));
        fq[2 * u + 1] = relu(bf16_hi(qw[u]));
        fk[2 * u] = relu(bf16_lo(kw[u]));
        fk[2 * u + 1] = relu(bf16_hi(kw[u]));
      }
      // denominator against the key sum before this step
      {
        const f32x4_t z0 = *reinterpret_cast<const f32x4_t *>(zs + d0);
        const f32x4_t z1 = *reinterpret_cast<const f32x4_t *>(zs + d0 + 8);
        den_in += fq[0] * z0.x + fq[1] * z0.y + fq[2] * z0.z + fq[3] * z0.w;
        den_in += fq[4] * z1.x + fq[5] * z1.y + fq[6] * z1.z + fq[7] * z1.w;
      }
      // this step's key sum for these dims: sum over the 32 tokens (lane bits 0..4)
      {
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = fk[t];
        // lane bit 4: pairs (t, t + 4)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[t]), __float_as_uint(v[t + 4]), false,
                                                          false);
          v[t] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        const bool b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {  // lane bit 3: partner by a rotation of 8 inside the row
          const float keep = b3 ? v[t + 2] : v[t];
          const float give = b3 ? v[t] : v[t + 2];
          v[t] = keep + dpp_f32<0x128>(give);
        }
        {  // lane bit 2: row half mirror
          const float keep = b2 ? v[1] : v[0];
          const float give = b2 ? v[0] : v[1];
          v[0] = keep + dpp_f32<0x141>(give);
        }
        v[0] += dpp_f32<0x4E>(v[0]);  // lane bit 1
        v[0] += dpp_f32<0xB1>(v[0]);  // lane bit 0
        // v[0] is the sum for value 4*bit4 + 2*bit3 + bit2 of this half, which
        // sits at zs[d0 + zslot] (a lane offset plus this step's constant)
        if ((lane & 3) == 0) zs[zslot + 32 * kb + 16 * s2] += v[0];
      }
      float qa[8], kc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        qa[t] = fq[t];
        kc[t] = fk[t];
      }
      if constexpr (kRope) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f32x4_t c4;
          if constexpr (kRopeMode == kRopeLds)
            c4 = rope_run_lds(a.rope, a, tp, d0 + 8 * u);
          else
            c4 = rope_run(a.rope, tp, d0 + 8 * u);
          rotate(qa[4 * u], qa[4 * u + 1], f32x2_t{c4.x, c4.y});
          rotate(qa[4 * u + 2], qa[4 * u + 3], f32x2_t{c4.z, c4.w});
          rotate(kc[4 * u], kc[4 * u + 1], f32x2_t{c4.x, c4.y});
          rotate(kc[4 * u + 2], kc[4 * u + 3], f32x2_t{c4.z, c4.w});
        }
      }
      const uint32_t aw[4] = {pack_bf16(qa[0], qa[1]), pack_bf16(qa[2], qa[3]), pack_bf16(qa[4], qa[5]),
                              pack_bf16(qa[6], qa[7])};
      const uint32_t cw[4] = {pack_bf16(kc[0], kc[1]), pack_bf16(kc[2], kc[3]), pack_bf16(kc[4], kc[5]),
                              pack_bf16(kc[6], kc[7])};
      const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(aw[0], aw[1], aw[2], aw[3]));
      const bf16x8_t C = __builtin_bit_cast(bf16x8_t, make_uint4(cw[0], cw[1], cw[2], cw[3]));
      const bf16x8_t Qu = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16(fq[0], fq[1]), pack_bf16(fq[2], fq[3]),
                                                                  pack_bf16(fq[4], fq[5]), pack_bf16(fq[6], fq[7])));
      const bf16x8_t Ku = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16(fk[0], fk[1]), pack_bf16(fk[2], fk[3]),
                                                                  pack_bf16(fk[4], fk[5]), pack_bf16(fk[6], fk[7])));
      // C^T to LDS (row = dim, column = permuted key)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int d = t < 4 ? d0 + t : d0 + 4 + t;
        ct[d * kCtRow + kp_self] = (uint16_t)((t & 1) ? (cw[t >> 1] >> 16) : (cw[t >> 1] & 0xFFFFu));
      }
      tacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(C, A, tacc, 0, 0, 0);
      uacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ku, Qu, uacc, 0, 0, 0);
      // inter-step: O^T += S^T a^T, S entries 8*s2 .. 8*s2+7 of block (kb, mb) as hi + lo
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x0 = sacc[kb][mb][8 * s2 + 2 * u], x1 = sacc[kb][mb][8 * s2 + 2 * u + 1];
          wh[u] = pack_bf16(x0, x1);
          wl[u] = pack_bf16(x0 - bf16_lo(wh[u]), x1 - bf16_hi(wh[u]));
        }
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3])), A, oacc[mb], 0, 0, 0);
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(wl[0], wl[1], wl[2], wl[3])), A, oacc[mb], 0, 0, 0);
      }
    }
    wave_lds_fence();  // C^T, V^T and z written

    // causal mask: the lane holds keys 8i + 4*half + j of query tl
    float den = den_in + __shfl_xor(den_in, 32);
    float dsum = 0.f;
    float p[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool keep = 8 * i + 4 * half + j <= tl;
        p[4 * i + j] = keep ? tacc[4 * i + j] : 0.f;
        dsum += keep ? uacc[4 * i + j] : 0.f;
      }
    den += dsum + __shfl_xor(dsum, 32) + a.eps;
    // intra-step: O^T += V^T P^T, P as hi + lo
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float x0 = p[8 * u + 2 * w], x1 = p[8 * u + 2 * w + 1];
        wh[w] = pack_bf16(x0, x1);
        wl[w] = pack_bf16(x0 - bf16_lo(wh[w]), x1 - bf16_hi(wh[w]));
      }
      const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
      const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, make_uint4(wl[0], wl[1], wl[2], wl[3]));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t *>(vt + (32 * mb + tl) * kCtRow + 16 * u + 8 * half);
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, ph, oacc[mb], 0, 0, 0);
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pl, oacc[mb], 0, 0, 0);
      }
    }
    // state update: S += C^T V over the step's keys (same key order on both sides)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8_t cta[2], vtb[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        cta[x] = *reinterpret_cast<const bf16x8_t *>(ct + (32 * x + tl) * kCtRow + 16 * s + 8 * half);
        vtb[x] = *reinterpret_cast<const bf16x8_t *>(vt + (32 * x + tl) * kCtRow + 16 * s + 8 * half);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          sacc[kb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cta[kb], vtb[nb], sacc[kb][nb], 0, 0, 0);
    }

    // normalise, gate, store: lane holds dims 32*mb + 8i + 4*half + j of token n
    const float inv = 1.f / den;
    if (valid) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = oacc[mb][4 * i + j] * inv;
          if constexpr (kGate) {
            const uint2 gw = gws[mb][i];
            y[0] *= sigmoid_fast(bf16_lo(gw.x));
            y[1] *= sigmoid_fast(bf16_hi(gw.x));
            y[2] *= sigmoid_fast(bf16_lo(gw.y));
            y[3] *= sigmoid_fast(bf16_hi(gw.y));
          }
          *reinterpret_cast<uint2 *>(const_cast<char *>(at(a.o, 32 * mb + 8 * i + 4 * half))) =
              make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
        }
    }
    wave_lds_fence();  // the next step's LDS writes come after these reads
  }
}

template <bool kBF16, bool kRope, bool kAligned, bool kZW>
hipError_t launch_build(dim3 grid, const BuildArgs &ba, hipStream_t stream) {
  const size_t lds = 4 * (size_t)(kBF16 ? kWaveLds16 : kWaveLds32);
  const void *fn = reinterpret_cast<const void *>(&la_build_kernel<kBF16, kRope, kAligned, kZW>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((la_build_kernel<kBF16, kRope, kAligned, kZW>), grid, dim3(256), lds, stream, ba);
  return hipSuccess;
}

template <bool kBF16, bool kZW>
hipError_t launch_build_any(const RopeArgs &r, dim3 grid, const BuildArgs &ba, hipStream_t stream) {
  if (!r.enabled) return launch_build<kBF16, false, false, kZW>(grid, ba, stream);
  if (r.aligned) return launch_build<kBF16, true, true, kZW>(grid, ba, stream);
  return launch_build<kBF16, true, false, kZW>(grid, ba, stream);
}

template <int kRopeMode>
void launch_apply_bf16(bool gate, dim3 grid, const ApplyArgs &aa, hipStream_t stream) {
  const size_t lds = kRopeMode == kRopeLds ? (size_t)(aa.tab_t + aa.tab_h + aa.tab_w) * sizeof(float) : 0;
  if (gate)
    hipLaunchKernelGGL((la_apply_bf16_kernel<kRopeMode, true>), grid, dim3(256), lds, stream, aa);
  else
    hipLaunchKernelGGL((la_apply_bf16_kernel<kRopeMode, false>), grid, dim3(256), lds, stream, aa);
}

}  // namespace

LinearPlan plan_linear(int B, int N, int H, int chunk_tokens) {
  LinearPlan p;
  const long long L = chunk_tokens > 0 && chunk_tokens < N ? chunk_tokens : N;
  p.chunk_len = (int)L;
  p.n_chunks = (int)((N + L - 1) / L);
  p.ngroups = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  // Work-groups per (b, head group, chunk). Both kernels run two work-groups
  // per CU, 512 at once on the 256 CUs of an MI355X (a fixed assumption, so
  // that the workspace query needs no device). Work-groups start in grid order
  // as slots free up. The split chosen is the one, up to four rounds of
  // work-groups, whose schedule ends first, estimated from each work-group's
  // 64-token tiles plus one tile's worth of start-up: the work-groups of full
  // chunks run in rounds, and those of a shorter last chunk fill the slots the
  // last round leaves idle. The smaller split wins a tie. A chunk never gets
  // more slabs than tiles, nor more parts than 32-token steps.
  const long long per_chunk_groups = (long long)B * p.ngroups * p.n_chunks;
  const long long slots = 512;
  const long long max_split = std::max(1LL, 4 * slots / per_chunk_groups);
  const long long tiles_full = (L + kWTile - 1) / kWTile;
  const long long last_len = N - (long long)(p.n_chunks - 1) * L;
  const long long tiles_last = (last_len + kWTile - 1) / kWTile;
  const bool ragged = tiles_last < tiles_full;
  long long split = 1, best_end = -1;
  for (long long sp = 1; sp <= std::min(max_split, tiles_full); ++sp) {
    const long long groups = (long long)B * p.ngroups;
    const long long n_full = groups * (p.n_chunks - (ragged ? 1 : 0)) * sp;
    const long long n_last = ragged ? groups * sp : 0;
    const long long d_full = 1 + (tiles_full + sp - 1) / sp;
    const long long d_last = 1 + (tiles_last + sp - 1) / sp;
    const long long rounds = (n_full + slots - 1) / slots;
    const long long idle = rounds * slots - n_full;  // slots free after rounds - 1
    long long end = rounds * d_full;
    if (n_last > 0) {
      const long long small_end = idle > 0 ? (rounds - 1) * d_full + (n_last + idle - 1) / idle * d_last
                                           : rounds * d_full + (n_last + slots - 1) / slots * d_last;
      end = std::max(end, small_end);
    }
    if (best_end < 0 || end < best_end) {
      best_end = end;
      split = sp;
    }
  }
  p.slabs_per_chunk = (int)std::min(split, (L + kWTile - 1) / kWTile);
  p.apply_per_chunk = (int)std::min(split, (L + kApplySub - 1) / kApplySub);
  const long long heads = (long long)B * H;
  const size_t part_bytes = (size_t)heads * p.n_chunks * p.slabs_per_chunk * kStateFloats * sizeof(float);
  const size_t prefix_bytes = (size_t)heads * p.n_chunks * kStateFloats * sizeof(float);
  p.part_offset = 0;
  p.prefix_offset = align256(part_bytes);
  p.total_bytes = p.prefix_offset + align256(prefix_bytes);
  return p;
}

hipError_t launch_state_sums(hla_dtype dt, const StateSumArgs &sa_in, const LinearPlan &p, void *ws,
                             hipStream_t stream, float **prefix_out) {
  const int heads = sa_in.B * sa_in.H;
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + p.part_offset);
  float *prefix = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + p.prefix_offset);
  if (sa_in.zw && dt != HLA_BF16) return hipErrorInvalidValue;

  BuildArgs ba;
  ba.k = sa_in.k;
  ba.v = sa_in.v;
  ba.zw = sa_in.zw;
  ba.N = sa_in.N;
  ba.H = sa_in.H;
  ba.L = p.chunk_len;
  ba.n_chunks = p.n_chunks;
  ba.slabs_per_chunk = p.slabs_per_chunk;
  ba.ngroups = p.ngroups;
  ba.rope = sa_in.rope;
  ba.part = part;
  const dim3 bgrid(p.n_chunks * p.slabs_per_chunk * p.ngroups, sa_in.B);
  {
    hipError_t e;
    if (dt != HLA_BF16)
      e = launch_build_any<false, false>(sa_in.rope, bgrid, ba, stream);
    else if (sa_in.zw)
      e = launch_build_any<true, true>(sa_in.rope, bgrid, ba, stream);
    else
      e = launch_build_any<true, false>(sa_in.rope, bgrid, ba, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  ScanArgs sa;
  sa.part = part;
  sa.n_chunks = p.n_chunks;
  sa.slabs_per_chunk = p.slabs_per_chunk;
  sa.kv_in = sa_in.start_kv;
  sa.ksum_in = sa_in.start_ksum;
  sa.kv_out = sa_in.final_kv;
  sa.ksum_out = sa_in.final_ksum;
  sa.prefix = prefix;
  sa.init = sa_in.init_copy;
  sa.reverse = sa_in.reverse ? 1 : 0;
  hipLaunchKernelGGL(la_scan_kernel, dim3((kStateFloats + 255) / 256, heads), dim3(256), 0, stream, sa);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  *prefix_out = prefix;
  return hipSuccess;
}

// State build and scan of the forward paths; *prefix_out receives the
// inclusive prefix per chunk.
static hipError_t build_and_scan(hla_dtype dt, const LinearArgs &a, const LinearPlan &p, hipStream_t stream,
                                 float **prefix_out, float *init = nullptr) {
  StateSumArgs s;
  s.B = a.B;
  s.N = a.N;
  s.H = a.H;
  s.k = a.k;
  s.v = a.v;
  s.zw = nullptr;
  s.rope = a.rope;
  s.start_kv = a.kv_in;
  s.start_ksum = a.ksum_in;
  s.final_kv = a.kv_out;
  s.final_ksum = a.ksum_out;
  s.reverse = false;
  s.init_copy = init;
  return launch_state_sums(dt, s, p, a.ws, stream, prefix_out);
}

hipError_t launch_linear(hla_dtype dt, const LinearArgs &a, const LinearPlan &p, hipStream_t stream) {
  float *prefix = nullptr;
  {
    const hipError_t e = build_and_scan(dt, a, p, stream, &prefix);
    if (e != hipSuccess) return e;
  }
  ApplyArgs aa;
  aa.q = a.q;
  aa.g = a.g;
  aa.o = a.o;
  aa.N = a.N;
  aa.H = a.H;
  aa.L = p.chunk_len;
  aa.n_chunks = p.n_chunks;
  aa.apply_per_chunk = p.apply_per_chunk;
  aa.ngroups = p.ngroups;
  aa.rope = a.rope;
  aa.eps = a.eps;
  aa.prefix = prefix;
  aa.tab_t = aa.tab_h = aa.tab_w = 0;
  if (a.rope.enabled) {
    aa.tab_t = (int)((uint32_t)a.N / a.rope.hw) * a.rope.d_t;
    aa.tab_h = (int)a.rope.h * a.rope.d_h;
    aa.tab_w = (int)a.rope.w * a.rope.d_w;
  }
  const dim3 agrid(p.n_chunks * p.apply_per_chunk * p.ngroups, a.B);
  if (dt == HLA_BF16) {
    const bool gate = a.g != nullptr;
    const int tab_floats = aa.tab_t + aa.tab_h + aa.tab_w;
    if (!a.rope.enabled)
      launch_apply_bf16<kRopeNone>(gate, agrid, aa, stream);
    else if (!a.rope.aligned)
      launch_apply_bf16<kRopePair>(gate, agrid, aa, stream);
    else if (tab_floats <= kTabLdsFloats)
      launch_apply_bf16<kRopeLds>(gate, agrid, aa, stream);
    else
      launch_apply_bf16<kRopeGlobal>(gate, agrid, aa, stream);
  } else
    hipLaunchKernelGGL(la_apply_f32_kernel, agrid, dim3(256), 0, stream, aa);
  return hipGetLastError();
}

LinearPlan plan_linear_causal(int B, int N, int H) {
  // one work-group per (b, head group, range), about 512 in all; ranges are
  // whole 32-token steps and carry their state sequentially
  const long long groups = (long long)B * ((H + kHeadsPerWG - 1) / kHeadsPerWG);
  const long long ranges = std::max(1LL, 512 / groups);
  long long len = ((long long)N + ranges - 1) / ranges;
  len = std::max<long long>(kApplySub, (len + kApplySub - 1) / kApplySub * kApplySub);
  LinearPlan p = plan_linear(B, N, H, (int)std::min<long long>(len, N));
  p.init_offset = p.total_bytes;  // copy of the incoming state
  p.total_bytes += align256((size_t)B * H * kStateFloats * sizeof(float));
  return p;
}

template <int kRopeMode>
void launch_causal(bool gate, dim3 grid, const CausalArgs &ca, hipStream_t stream) {
  const size_t lds = kRopeMode == kRopeLds ? (size_t)(ca.tab_t + ca.tab_h + ca.tab_w) * sizeof(float) : 0;
  if (gate)
    hipLaunchKernelGGL((la_causal_kernel<kRopeMode, true>), grid, dim3(256), lds, stream, ca);
  else
    hipLaunchKernelGGL((la_causal_kernel<kRopeMode, false>), grid, dim3(256), lds, stream, ca);
}

hipError_t launch_linear_causal(const LinearArgs &a, const LinearPlan &p, hipStream_t stream) {
  float *prefix = nullptr;
  float *init = reinterpret_cast<float *>(reinterpret_cast<char *>(a.ws) + p.init_offset);
  {
    const hipError_t e = build_and_scan(HLA_BF16, a, p, stream, &prefix, init);
    if (e != hipSuccess) return e;
  }
  CausalArgs ca;
  ca.q = reinterpret_cast<const uint16_t *>(a.q);
  ca.k = reinterpret_cast<const uint16_t *>(a.k);
  ca.v = reinterpret_cast<const uint16_t *>(a.v);
  ca.g = reinterpret_cast<const uint16_t *>(a.g);
  ca.o = reinterpret_cast<uint16_t *>(a.o);
  ca.N = a.N;
  ca.H = a.H;
  ca.L = p.chunk_len;
  ca.n_chunks = p.n_chunks;
  ca.ngroups = p.ngroups;
  ca.rope = a.rope;
  ca.eps = a.eps;
  ca.prefix = prefix;
  ca.init = init;
  ca.tab_t = ca.tab_h = ca.tab_w = 0;
  if (a.rope.enabled) {
    ca.tab_t = (int)((uint32_t)a.N / a.rope.hw) * a.rope.d_t;
    ca.tab_h = (int)a.rope.h * a.rope.d_h;
    ca.tab_w = (int)a.rope.w * a.rope.d_w;
  }
  const int tab_floats = ca.tab_t + ca.tab_h + ca.tab_w;
  const dim3 grid(p.n_chunks * p.ngroups, a.B);
  const bool gate = a.g != nullptr;
  if (!a.rope.enabled)
    launch_causal<kRopeNone>(gate, grid, ca, stream);
  else if (tab_floats <= kTabLdsFloats)
    launch_causal<kRopeLds>(gate, grid, ca, stream);
  else
    launch_causal<kRopeGlobal>(gate, grid, ca, stream);
  return hipGetLastError();
}

}  // namespace hla
