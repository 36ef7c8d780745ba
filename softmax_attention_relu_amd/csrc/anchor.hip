// Gated non-causal softmax anchor attention on the bf16 matrix cores
// (SANA-Video 2.0 abstract and summary: one layer in four is a gated softmax
// anchor; textbook scaled dot-product attention with a sigmoid output gate):
//   o_i = sigmoid(g_i) * sum_j softmax_j(scale * q_i . k_j) v_j
//
// Two kernels:
//   anchor_vt  writes V of each (b, h) transposed, [64 dims][Npad tokens],
//              tokens zero-padded to a multiple of 64 and permuted inside each
//              group of 16 so that every matrix-core operand of the P.V product
//              is one contiguous 16-byte LDS read (see kernel comment).
//   anchor_fwd online-softmax attention. A work-group of 16 waves owns 512
//              query rows of one (b, h); wave w owns 32 rows. Per 64-key tile:
//                S^T = K Q^T   (A = K rows from LDS, B = Q^T held in registers)
//                softmax update in the exp2 domain, lane-local: the score layout
//                gives each lane one query row and 32 of the 64 keys
//                O^T += V^T P^T (A = V^T from LDS, B = P^T straight from the
//                score registers, rounded to bf16)
//              K and V^T tiles are double-buffered in LDS; the next tile's
//              global loads are issued before the current tile's products.
// At most 128 registers per lane keep every accumulator in VGPRs with four
// waves per SIMD; the tile's row max is combined across the two lane halves
// with v_permlane32_swap. On this chip the plain vector ALU work of the
// softmax (one FMA, one max and half a conversion per score) does not overlap
// the matrix-core work much, while exponentials largely do; that, not the
// matrix cores, sets the kernel's speed.
// The running max is refreshed lazily: rows keep their reference max until a
// tile exceeds it by more than 8 (log2 units), so exponentials stay <= 2^8
// and the O / row-sum rescale is almost never taken. The normaliser uses the
// same reference max, so the result is exact up to rounding.
#include "device_common.h"

namespace hla {

namespace {

constexpr int kBK = 64;            // keys per tile
constexpr int kKRow = kD + 8;      // bf16 per LDS row of K (144 bytes)
constexpr int kVRow = kBK + 8;     // bf16 per LDS row of V^T (144 bytes)
constexpr float kLazy = 8.0f;      // lazy max threshold, log2 units
constexpr int kWaves = 16;         // waves per work-group, 32 query rows each
constexpr int kMinWaves = 4;       // waves per SIMD the forward kernel is compiled for
static_assert(kSparseKBlock == kBK, "a named key block is one tile");
static_assert(kSparseQBlock % 32 == 0, "a query block is whole waves of 32 rows");

// Key position inside a group of 16 with bits 2 and 3 swapped. With this
// order, the 8 keys a lane feeds to one 32x32x16 product (keys 4h..4h+3 and
// 8+4h..8+4h+3 of a 16-key step, h = lane / 32) sit at positions 8h..8h+7.
// max of x over lanes l and l^32: v_permlane32_swap of a register with itself
// leaves the partner's value in one of the two results
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ int perm16(int n) { return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1); }

struct VtArgs {
  const uint16_t *v;
  uint16_t *vt;  // [B*H][64][npad]
  int N, H, npad;
};

__global__ __launch_bounds__(256) void anchor_vt_kernel(VtArgs a) {
  __shared__ uint16_t tile[kBK][kD + 2];
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int n0 = blockIdx.x * kBK;
  const size_t tok_stride = (size_t)a.H * kD;
  const uint16_t *vp = a.v + (size_t)b * a.N * tok_stride + (size_t)h * kD;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int c = tid + 256 * r;
    const int key = c >> 3, dc = c & 7;
    const int n = n0 + key;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < a.N) w = *reinterpret_cast<const uint4 *>(vp + (size_t)n * tok_stride + 8 * dc);
    uint32_t *dst = reinterpret_cast<uint32_t *>(&tile[key][8 * dc]);
    dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
  }
  __syncthreads();
  uint16_t *out = a.vt + (size_t)bh * kD * a.npad + n0;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int c = tid + 256 * r;
    const int e = c >> 3, pc = c & 7;  // dim row, 8-position chunk
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
      const int p0 = 8 * pc + t, p1 = p0 + 1;
      const int k0 = (p0 & ~15) | perm16(p0 & 15);  // perm16 is its own inverse
      const int k1 = (p1 & ~15) | perm16(p1 & 15);
      w[t / 2] = (uint32_t)tile[k0][e] | ((uint32_t)tile[k1][e] << 16);
    }
    *reinterpret_cast<uint4 *>(out + (size_t)e * a.npad + 8 * pc) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

struct FwdArgs {
  const uint16_t *q, *k, *g;
  const uint16_t *vt;
  uint16_t *o;
  int N, H, npad;
  float c;  // scale * log2(e)
  // block-sparse form: key tiles named per (b*H + h, query block), [..][max_blocks]
  const int *blocks, *counts;
  int n_qb, max_blocks;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// The row sum adds the bf16-rounded P with v_dot2 (two terms per
// instruction): the normaliser uses the same weights as the P.V product.
// kSparse: the work-group's query rows form one query block and visit only
// the 64-key tiles named for it (entries outside the key range are skipped);
// otherwise every tile in order.
template <int WAVES, int MINW, bool kSparse>
__global__ __launch_bounds__(64 * WAVES, MINW) void anchor_fwd_kernel(FwdArgs a) {
  constexpr int kThreads = 64 * WAVES;
  // 16-byte chunks of K (and of V^T) per thread per tile: 512 chunks each
  constexpr int kLoaders = kThreads < kBK * 8 ? kThreads : kBK * 8;
  constexpr int kLoads = kBK * 8 / kLoaders;
  __shared__ __align__(16) uint16_t ks[2][kBK * kKRow];
  __shared__ __align__(16) uint16_t vs[2][kD * kVRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, tl = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int q0 = blockIdx.x * (32 * WAVES) + wave * 32;

  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD;
  const uint16_t *kp = a.k + head_base;
  const uint16_t *vtp = a.vt + (size_t)bh * kD * a.npad;

  // Q^T operands: row q0 + tl, dims 16*s + 8*half .. +7
  bf16x8_t qb[4];
  {
    const int n = q0 + tl;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (n < a.N) w = *reinterpret_cast<const uint4 *>(a.q + head_base + (size_t)n * tok_stride + 16 * s + 8 * half);
      qb[s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // tile loader: K (64 keys x 8 chunks) and V^T (64 dims x 8 chunks), 16-byte
  // chunks spread over the work-group
  uint4 kreg[kLoads], vreg[kLoads];
  auto load_tile = [&](int t) {
    if (tid >= kLoaders) return;
    const int n0 = t * kBK;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + kLoaders * r;
      const int row = c >> 3, ch = c & 7;
      const int n = n0 + row;
      kreg[r] = n < a.N ? *reinterpret_cast<const uint4 *>(kp + (size_t)n * tok_stride + 8 * ch) : make_uint4(0, 0, 0, 0);
      vreg[r] = *reinterpret_cast<const uint4 *>(vtp + (size_t)row * a.npad + n0 + 8 * ch);
    }
  };
  auto store_tile = [&](int buf) {
    if (tid >= kLoaders) return;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + kLoaders * r;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<uint4 *>(&ks[buf][row * kKRow + 8 * ch]) = kreg[r];
      *reinterpret_cast<uint4 *>(&vs[buf][row * kVRow + 8 * ch]) = vreg[r];
    }
  };

  f32x16_t oacc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.f;
  float mref = -INFINITY, lsum = 0.f;

  const int ntiles = (a.N + kBK - 1) / kBK;
  // position i of the visiting order -> key tile; next(i): first usable position >= i
  const int *list = nullptr;
  int cnt = ntiles;
  if constexpr (kSparse) {
    const size_t qblk = (size_t)bh * a.n_qb + blockIdx.x;
    list = a.blocks + qblk * a.max_blocks;
    cnt = min(max(a.counts[qblk], 0), a.max_blocks);
  }
  auto tile_of = [&](int i) { return kSparse ? list[i] : i; };
  auto next = [&](int i) {
    if constexpr (kSparse) {
      while (i < cnt && (unsigned)list[i] >= (unsigned)ntiles) ++i;
    }
    return i;
  };
  int pos = next(0);
  if (pos < cnt) {
    load_tile(tile_of(pos));
    store_tile(0);
  }
  __syncthreads();
  for (int buf = 0; pos < cnt; buf ^= 1) {
    const int t = tile_of(pos);
    const int pnext = next(pos + 1);
    if (pnext < cnt) load_tile(tile_of(pnext));

    // S^T = K Q^T for the 64 keys of this tile
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t kv =
            *reinterpret_cast<const bf16x8_t *>(&ks[buf][(32 * kb + tl) * kKRow + 16 * s + 8 * half]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qb[s], sacc[kb], 0, 0, 0);
      }

    // mask keys past the end (last tile only)
    if ((t + 1) * kBK > a.N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (t * kBK + 32 * kb + 8 * i + 4 * half + j >= a.N) sacc[kb][4 * i + j] = -INFINITY;
    }

    // online softmax (exp2 domain); ts is this lane's share of the tile's row sum
    bf16x8_t pb[2][2];
    float ts;
    auto exps = [&](float nm) {
      ts = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], a.c, nm));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint4 w = make_uint4(pack_bf16(p[8 * u + 0], p[8 * u + 1]), pack_bf16(p[8 * u + 2], p[8 * u + 3]),
                                     pack_bf16(p[8 * u + 4], p[8 * u + 5]), pack_bf16(p[8 * u + 6], p[8 * u + 7]));
          pb[kb][u] = __builtin_bit_cast(bf16x8_t, w);
          const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), one, ts, false);
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), one, ts, false);
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), one, ts, false);
          ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), one, ts, false);
        }
      }
    };
    auto row_max = [&]() {
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      return max_halves(mx) * a.c;
    };
    auto rescale = [&](float mnew) {
      const float f = exp2f(mref - mnew);
      mref = mnew;
      lsum *= f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] *= f;
    };
    {
      const float mt = row_max();
      const bool bump = mt > mref + kLazy;
      if (__any(bump)) rescale(bump ? mt : mref);
      exps(-mref);
    }
    lsum += ts;

    // O^T += V^T P^T
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8_t vv =
              *reinterpret_cast<const bf16x8_t *>(&vs[buf][(32 * mb + tl) * kVRow + 32 * kb + 16 * u + 8 * half]);
          oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[kb][u], oacc[mb], 0, 0, 0);
        }

    if (pnext < cnt) {
      store_tile(buf ^ 1);  // the other buffer was last read two tiles ago
      __syncthreads();
    }
    pos = pnext;
  }

  // normalise, gate, store: lane holds row tl, dims 32*mb + 8*i + 4*half + j
  const int n = q0 + tl;
  const float l = lsum + __shfl_xor(lsum, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;  // no key visited: the output is 0
  if (n < a.N) {
    const size_t row = head_base + (size_t)n * tok_stride;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t off = row + 32 * mb + 8 * i + 4 * half;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = oacc[mb][4 * i + j] * inv;
        if (a.g) {
          const uint2 gw = *reinterpret_cast<const uint2 *>(a.g + off);
          y[0] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_lo(gw.x)));
          y[1] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_hi(gw.x)));
          y[2] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_lo(gw.y)));
          y[3] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_hi(gw.y)));
        }
        *reinterpret_cast<uint2 *>(a.o + off) = make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
      }
  }
}

}  // namespace

size_t anchor_workspace_bytes(int B, int N, int H) {
  const size_t npad = ((size_t)N + kBK - 1) / kBK * kBK;
  return (size_t)B * H * kD * npad * sizeof(uint16_t);
}

hipError_t launch_anchor(const AnchorArgs &a, hipStream_t stream) {
  const int heads = a.B * a.H;
  const int npad = (a.N + kBK - 1) / kBK * kBK;
  VtArgs va;
  va.v = reinterpret_cast<const uint16_t *>(a.v);
  va.vt = reinterpret_cast<uint16_t *>(a.ws);
  va.N = a.N;
  va.H = a.H;
  va.npad = npad;
  hipLaunchKernelGGL(anchor_vt_kernel, dim3(npad / kBK, heads), dim3(256), 0, stream, va);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  FwdArgs fa;
  fa.q = reinterpret_cast<const uint16_t *>(a.q);
  fa.k = reinterpret_cast<const uint16_t *>(a.k);
  fa.g = reinterpret_cast<const uint16_t *>(a.g);
  fa.vt = va.vt;
  fa.o = reinterpret_cast<uint16_t *>(a.o);
  fa.N = a.N;
  fa.H = a.H;
  fa.npad = npad;
  fa.c = a.scale * 1.4426950408889634f;
  fa.blocks = a.blocks;
  fa.counts = a.counts;
  fa.max_blocks = a.max_blocks;
  if (a.blocks) {
    fa.n_qb = (a.N + kSparseQBlock - 1) / kSparseQBlock;
    hipLaunchKernelGGL((anchor_fwd_kernel<kSparseQBlock / 32, kMinWaves, true>), dim3(fa.n_qb, heads),
                       dim3(2 * kSparseQBlock), 0, stream, fa);
  } else {
    fa.n_qb = 0;
    hipLaunchKernelGGL((anchor_fwd_kernel<kWaves, kMinWaves, false>),
                       dim3((a.N + 32 * kWaves - 1) / (32 * kWaves), heads), dim3(64 * kWaves), 0, stream, fa);
  }
  return hipGetLastError();
}

}  // namespace hla
