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
#include <string.h>

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

// bitmaps of the block-sparse form (dynamic LDS): the union of the work-group's
// named tiles, then one set per query block of the work-group
extern __shared__ __align__(16) uint32_t anchor_bits[];

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
    if (n < a.N) w = load_once_u4(vp + (size_t)n * tok_stride + 8 * dc);
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
  // gradient preparation (kPrep): reads dO, writes dG, dY = dO * sigmoid(g) (bf16,
  // the layout of q) and per row the log2-domain normaliser and Delta = dY . y
  const uint16_t *dO;
  uint16_t *dg, *dy;
  float *lse, *delta;  // [B*H][N]
  // optional (not kPrep): the natural-log normaliser of every row, [B*H][N]
  float *lse_out;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// The row sum adds the bf16-rounded P with v_dot2 (two terms per
// instruction): the normaliser uses the same weights as the P.V product.
// kSparse: the work-group's query rows form WAVES / 4 query blocks of 128 rows.
// The work-group walks the union of the 64-key tiles they name, in ascending
// order (two LDS bitmaps: the union and each block's own set; entries outside
// the key range name nothing, repeats count once), loading every tile once for
// all its waves; a wave computes only the tiles its own block names.
// Otherwise every tile in order. kPrep: the epilogue writes the inputs of the
// gradient kernels instead of o (y = the ungated output, s = sigmoid(g)):
// dG = dO y s (1 - s), dY = dO s (bf16), Delta = dY . y and L = mref + log2(rowsum),
// so that p_ij = exp2(c s_ij - L_i) are the normalised weights.
template <int WAVES, int MINW, bool kSparse, bool kPrep>
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
  constexpr int kBlockWaves = kSparseQBlock / 32;
  const int nwords = (ntiles + 31) >> 5;
  const uint32_t *uni = anchor_bits, *own = anchor_bits + (size_t)nwords * (1 + wave / kBlockWaves);
  if constexpr (kSparse) {
    for (int i = tid; i < nwords * (1 + WAVES / kBlockWaves); i += kThreads) anchor_bits[i] = 0u;
    __syncthreads();
    const int qb = blockIdx.x * (WAVES / kBlockWaves) + wave / kBlockWaves;
    if (wave % kBlockWaves == 0 && qb < a.n_qb) {
      const size_t qblk = (size_t)bh * a.n_qb + qb;
      const int *list = a.blocks + qblk * a.max_blocks;
      const int cnt = min(max(a.counts[qblk], 0), a.max_blocks);
      uint32_t *mine = anchor_bits + (size_t)nwords * (1 + wave / kBlockWaves);
      for (int i = lane; i < cnt; i += 64) {
        const int m = list[i];
        if ((unsigned)m < (unsigned)ntiles) {
          atomicOr(&anchor_bits[m >> 5], 1u << (m & 31));
          atomicOr(&mine[m >> 5], 1u << (m & 31));
        }
      }
    }
    __syncthreads();
  }
  // first tile >= t in the visiting order, ntiles if none
  auto next = [&](int t) {
    if constexpr (!kSparse) {
      return t;
    } else {
      int w = t >> 5;
      if (w >= nwords) return ntiles;
      uint32_t bits = uni[w] & (~0u << (t & 31));
      while (bits == 0u) {
        if (++w >= nwords) return ntiles;
        bits = uni[w];
      }
      return (w << 5) + __builtin_ctz(bits);
    }
  };
  int t = next(0);
  if (t < ntiles) {
    load_tile(t);
    store_tile(0);
  }
  __syncthreads();
  for (int buf = 0; t < ntiles; buf ^= 1) {
    const int tnext = next(t + 1);
    if (tnext < ntiles) load_tile(tnext);
    if (kSparse && !((own[t >> 5] >> (t & 31)) & 1u)) {  // not named by this wave's block
      if (tnext < ntiles) {
        store_tile(buf ^ 1);
        __syncthreads();
      }
      t = tnext;
      continue;
    }

    // S^T = K Q^T for the 64 keys of this tile; here and in the P.V product the
    // two accumulators alternate, so each product waits on the other's
    // predecessor rather than its own
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
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
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8_t vv =
              *reinterpret_cast<const bf16x8_t *>(&vs[buf][(32 * mb + tl) * kVRow + 32 * kb + 16 * u + 8 * half]);
          oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[kb][u], oacc[mb], 0, 0, 0);
        }

    if (tnext < ntiles) {
      store_tile(buf ^ 1);  // the other buffer was last read two tiles ago
      __syncthreads();
    }
    t = tnext;
  }

  // normalise, gate, store: lane holds row tl, dims 32*mb + 8*i + 4*half + j
  const int n = q0 + tl;
  const float l = lsum + __shfl_xor(lsum, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;  // no key visited: the output is 0
  if constexpr (kPrep) {
    const size_t row = head_base + (size_t)min(n, a.N - 1) * tok_stride;
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t off = row + 32 * mb + 8 * i + 4 * half;
        const uint2 ow = *reinterpret_cast<const uint2 *>(a.dO + off);
        const float dov[4] = {bf16_lo(ow.x), bf16_hi(ow.x), bf16_lo(ow.y), bf16_hi(ow.y)};
        float gv[4] = {0.f, 0.f, 0.f, 0.f};
        if (a.g) {
          const uint2 gw = *reinterpret_cast<const uint2 *>(a.g + off);
          gv[0] = bf16_lo(gw.x); gv[1] = bf16_hi(gw.x); gv[2] = bf16_lo(gw.y); gv[3] = bf16_hi(gw.y);
        }
        float dgv[4], dyv[4], y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[j] = oacc[mb][4 * i + j] * inv;
          const float sg = a.g ? __builtin_amdgcn_rcpf(1.f + __expf(-gv[j])) : 1.f;
          dgv[j] = dov[j] * y[j] * sg * (1.f - sg);
          dyv[j] = dov[j] * sg;
        }
        // Delta from the bf16 dY the dP product reads, so that sum_j dS_ij = 0
        // holds for the kernels' own dP (exactly zero gradients stay near zero)
        const uint2 dyw = make_uint2(pack_bf16(dyv[0], dyv[1]), pack_bf16(dyv[2], dyv[3]));
        part += bf16_lo(dyw.x) * y[0] + bf16_hi(dyw.x) * y[1] + bf16_lo(dyw.y) * y[2] + bf16_hi(dyw.y) * y[3];
        if (n < a.N) {
          *reinterpret_cast<uint2 *>(a.dy + off) = dyw;
          if (a.g)
            *reinterpret_cast<uint2 *>(a.dg + off) =
                make_uint2(pack_bf16(dgv[0], dgv[1]), pack_bf16(dgv[2], dgv[3]));
        }
      }
    const float delta = part + __shfl_xor(part, 32);
    if (n < a.N) {
      if (half == 0) {
        a.lse[(size_t)bh * a.N + n] = mref + log2f(l);
        a.delta[(size_t)bh * a.N + n] = delta;
      }
    }
    return;
  }
  if (n < a.N) {
    if (a.lse_out && half == 0) a.lse_out[(size_t)bh * a.N + n] = (mref + log2f(l)) * 0.6931471805599453f;
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

// ---------------------------------------------------------------------------
// Gradients. With p_ij = exp2(c s_ij - L_i) (L from the preparation pass),
// dP_ij = dY_i . v_j and dS_ij = p_ij (dP_ij - Delta_i), the gradient of the
// logit: dq_i = scale sum_j dS_ij k_j, dk_j = scale sum_i dS_ij q_i and
// dv_j = sum_i p_ij dY_i. Two kernels, no atomics: one owns keys and walks the
// query tiles (dk, dv), the other owns queries and walks the key tiles (dq).
// Both reuse the forward's layout: the scores come out with each lane holding
// one column token and 32 row tokens, which feed the next products as B
// operands straight from registers against transposed tiles whose tokens are
// permuted in groups of 16 (the V^T layout of anchor_vt).
struct BwdArgs {
  const uint16_t *q, *k, *v, *dy;  // [B][N][H][64]
  const uint16_t *qt, *dyt, *kt;   // [B*H][64][npad], tokens permuted in groups of 16
  const float *lse, *delta;        // [B*H][N]
  uint16_t *dq, *dk, *dv;
  int N, H, npad;
  float c, scale;
};

// 16 bytes at p, or zeros when ok is false (p is then not read). Written as a
// branch on purpose: a select between the loaded value and a named zero vector
// can be turned into a load through a selected pointer, which puts the zero
// vector (and the staged tile) in scratch memory.
__device__ __forceinline__ uint4 chunk_or_zero(const uint16_t *p, bool ok) {
  uint4 w = make_uint4(0, 0, 0, 0);
  if (ok) w = *reinterpret_cast<const uint4 *>(p);
  return w;
}

// B operands of 32 tokens' rows: lane (tl, half) holds token n (its wave's
// token tl), dims 16 s + 8 half .. +7 (zero past N)
__device__ __forceinline__ void row_operands(const uint16_t *base, size_t stride, int n, int half, int N,
                                             bf16x8_t x[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < N) w = *reinterpret_cast<const uint4 *>(base + (size_t)n * stride + 16 * s + 8 * half);
    x[s] = __builtin_bit_cast(bf16x8_t, w);
  }
}

// f * acc rounded to bf16; the lane holds column token n, dims 32 mb + 8 i + 4 half + j
__device__ __forceinline__ void store_cols(uint16_t *base, size_t stride, int n, int half, const f32x16_t acc[2],
                                           float f) {
  const size_t row = (size_t)n * stride;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x16_t &x = acc[mb];
      *reinterpret_cast<uint2 *>(base + row + 32 * mb + 8 * i + 4 * half) =
          make_uint2(pack_bf16(f * x[4 * i], f * x[4 * i + 1]), pack_bf16(f * x[4 * i + 2], f * x[4 * i + 3]));
    }
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void anchor_dkdv_kernel(BwdArgs a) {
  static_assert(64 * WAVES == kBK * 8, "one 16-byte chunk of each tile per thread");
  __shared__ __align__(16) uint16_t qs[2][kBK * kKRow];  // Q rows of the query tile
  __shared__ __align__(16) uint16_t ds[2][kBK * kKRow];  // dY rows
  __shared__ __align__(16) uint16_t qts[2][kD * kVRow];  // Q^T, permuted
  __shared__ __align__(16) uint16_t dts[2][kD * kVRow];  // dY^T, permuted
  __shared__ __align__(16) float ls[2][kBK], dls[2][kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, tl = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int k0 = blockIdx.x * (32 * WAVES) + wave * 32;
  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD;

  bf16x8_t kb[4], vb[4];
  row_operands(a.k + head_base, tok_stride, k0 + tl, half, a.N, kb);
  row_operands(a.v + head_base, tok_stride, k0 + tl, half, a.N, vb);
  const uint16_t *qp = a.q + head_base, *dp = a.dy + head_base;
  const uint16_t *qtp = a.qt + (size_t)bh * kD * a.npad, *dtp = a.dyt + (size_t)bh * kD * a.npad;
  const float *lsp = a.lse + (size_t)bh * a.N, *dlp = a.delta + (size_t)bh * a.N;

  const int row = tid >> 3, ch = tid & 7;
  uint4 sreg[4];
  float sf = 0.f;
  auto load_tile = [&](int t) {
    const int n0 = t * kBK, n = n0 + row;
    sreg[0] = chunk_or_zero(qp + (size_t)n * tok_stride + 8 * ch, n < a.N);
    sreg[1] = chunk_or_zero(dp + (size_t)n * tok_stride + 8 * ch, n < a.N);
    sreg[2] = *reinterpret_cast<const uint4 *>(qtp + (size_t)row * a.npad + n0 + 8 * ch);
    sreg[3] = *reinterpret_cast<const uint4 *>(dtp + (size_t)row * a.npad + n0 + 8 * ch);
    // past N: a weight of exactly 0 and no Delta (waves 0 and 1 read L and Delta)
    const int qn = n0 + (tid & (kBK - 1));
    if (tid < kBK) {
      sf = INFINITY;
      if (qn < a.N) sf = lsp[qn];
    } else if (tid < 2 * kBK) {
      sf = 0.f;
      if (qn < a.N) sf = dlp[qn];
    }
  };
  auto store_tile = [&](int buf) {
    *reinterpret_cast<uint4 *>(&qs[buf][row * kKRow + 8 * ch]) = sreg[0];
    *reinterpret_cast<uint4 *>(&ds[buf][row * kKRow + 8 * ch]) = sreg[1];
    *reinterpret_cast<uint4 *>(&qts[buf][row * kVRow + 8 * ch]) = sreg[2];
    *reinterpret_cast<uint4 *>(&dts[buf][row * kVRow + 8 * ch]) = sreg[3];
    if (tid < 2 * kBK) (tid < kBK ? ls : dls)[buf][tid & (kBK - 1)] = sf;
  };

  f32x16_t dva[2], dka[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dva[mb][i] = dka[mb][i] = 0.f;

  const int ntiles = (a.N + kBK - 1) / kBK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    // scores and dP of the tile's 64 queries (rows) against the wave's 32 keys
    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[qb][i] = pacc[qb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int off = (32 * qb + tl) * kKRow + 16 * s + 8 * half;
        sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(&qs[buf][off]), kb[s],
                                                           sacc[qb], 0, 0, 0);
        pacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(&ds[buf][off]), vb[s],
                                                           pacc[qb], 0, 0, 0);
      }
    }
    // weights and logit gradients: lane rows 32 qb + 8 i + 4 half + j
    bf16x8_t pw[2][2], sw[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float pv[16], dv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4_t L = *reinterpret_cast<const f32x4_t *>(&ls[buf][32 * qb + 8 * i + 4 * half]);
        const f32x4_t Dl = *reinterpret_cast<const f32x4_t *>(&dls[buf][32 * qb + 8 * i + 4 * half]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pj = __builtin_amdgcn_exp2f(fmaf(sacc[qb][4 * i + j], a.c, -L[j]));
          pv[4 * i + j] = pj;
          dv[4 * i + j] = pj * (pacc[qb][4 * i + j] - Dl[j]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pw[qb][u] = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16(pv[8 * u], pv[8 * u + 1]), pack_bf16(pv[8 * u + 2], pv[8 * u + 3]),
                                 pack_bf16(pv[8 * u + 4], pv[8 * u + 5]), pack_bf16(pv[8 * u + 6], pv[8 * u + 7])));
        sw[qb][u] = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16(dv[8 * u], dv[8 * u + 1]), pack_bf16(dv[8 * u + 2], dv[8 * u + 3]),
                                 pack_bf16(dv[8 * u + 4], dv[8 * u + 5]), pack_bf16(dv[8 * u + 6], dv[8 * u + 7])));
      }
    }
    // dV^T += dY^T P and dK^T += Q^T dS over the tile's queries
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int off = (32 * mb + tl) * kVRow + 32 * qb + 16 * u + 8 * half;
          dva[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(&dts[buf][off]),
                                                            pw[qb][u], dva[mb], 0, 0, 0);
          dka[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(&qts[buf][off]),
                                                            sw[qb][u], dka[mb], 0, 0, 0);
        }
    if (t + 1 < ntiles) {
      store_tile(buf ^ 1);  // the other buffer was last read two tiles ago
      __syncthreads();
    }
  }
  const int n = k0 + tl;
  if (n < a.N) {
    store_cols(a.dk + head_base, tok_stride, n, half, dka, a.scale);
    store_cols(a.dv + head_base, tok_stride, n, half, dva, 1.f);
  }
}

// Tiles of the dq kernel go global -> LDS directly (no staging registers):
// rows of 128 bytes, unpadded, with row r's 16-byte chunk c in slot c ^ (r & 7),
// so the 8 rows that one operand read touches per chunk column fall in 8
// different slots. One copy instruction moves 8 rows (64 lanes x 16 bytes).
__device__ __forceinline__ void copy_rows(const uint16_t *src, uint16_t *lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 4) void anchor_dq_kernel(BwdArgs a) {
  static_assert(WAVES == 16, "waves 0-7 copy K and V rows, waves 8-15 copy K^T rows");
  __shared__ __align__(16) uint16_t ks[2][kBK * kD];   // K rows of the key tile
  __shared__ __align__(16) uint16_t vr[2][kBK * kD];   // V rows
  __shared__ __align__(16) uint16_t kts[2][kD * kBK];  // K^T, permuted

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, tl = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int q0 = blockIdx.x * (32 * WAVES) + wave * 32;
  const size_t tok_stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)b * a.N * tok_stride + (size_t)h * kD;

  bf16x8_t qb[4], db[4];
  row_operands(a.q + head_base, tok_stride, q0 + tl, half, a.N, qb);
  row_operands(a.dy + head_base, tok_stride, q0 + tl, half, a.N, db);
  const int nq = min(q0 + tl, a.N - 1);
  const float L = a.lse[(size_t)bh * a.N + nq], Dl = a.delta[(size_t)bh * a.N + nq];
  const uint16_t *kp = a.k + head_base, *vp = a.v + head_base;
  const uint16_t *ktp = a.kt + (size_t)bh * kD * a.npad;

  // copier: wave w copies rows 8 (w % 8) .. +7; lane i takes row + i / 8 and
  // fills slot i % 8 with chunk (i % 8) ^ (row & 7)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int crow = 8 * (wv & 7) + (lane >> 3);
  const int cchunk = (lane & 7) ^ (crow & 7);
  auto issue_tile = [&](int t, int buf) {
    const int n0 = t * kBK;
    if (wv < 8) {
      const int n = min(n0 + crow, a.N - 1);  // rows past the end: finite data, weight 0
      copy_rows(kp + (size_t)n * tok_stride + 8 * cchunk, &ks[buf][512 * wv]);
      copy_rows(vp + (size_t)n * tok_stride + 8 * cchunk, &vr[buf][512 * wv]);
    } else {
      copy_rows(ktp + (size_t)crow * a.npad + n0 + 8 * cchunk, &kts[buf][512 * (wv - 8)]);
    }
  };
  // this lane's operand rows tl (+ 32 per block): chunk 2j + half sits in slot (2j + half) ^ (tl & 7)
  int roff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) roff[j] = tl * kD + 8 * ((2 * j + half) ^ (tl & 7));

  f32x16_t dqa[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[mb][i] = 0.f;

  const int ntiles = (a.N + kBK - 1) / kBK;
  issue_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // the other buffers held tile t - 1, whose readers all passed the last barrier
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    const bool tail = (t + 1) * kBK > a.N;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T and dP^T of 32 of the tile's keys (rows) against the wave's 32 queries
      f32x16_t sacc, pacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int off = 32 * kb * kD + roff[s];
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(&ks[buf][off]), qb[s], sacc,
                                                       0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(&vr[buf][off]), db[s], pacc,
                                                       0, 0, 0);
      }
      float dv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * i + j;
          float pj = __builtin_amdgcn_exp2f(fmaf(sacc[e], a.c, -L));
          if (tail && t * kBK + 32 * kb + 8 * i + 4 * half + j >= a.N) pj = 0.f;
          dv[e] = pj * (pacc[e] - Dl);
        }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8_t sw = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16(dv[8 * u], dv[8 * u + 1]), pack_bf16(dv[8 * u + 2], dv[8 * u + 3]),
                                 pack_bf16(dv[8 * u + 4], dv[8 * u + 5]), pack_bf16(dv[8 * u + 6], dv[8 * u + 7])));
        // dQ^T += K^T dS^T over these keys
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int off = 32 * mb * kBK + roff[2 * kb + u];
          dqa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(&kts[buf][off]), sw,
                                                            dqa[mb], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t + 1 has landed
      __syncthreads();
    }
  }
  const int n = q0 + tl;
  if (n < a.N) store_cols(a.dq + head_base, tok_stride, n, half, dqa, a.scale);
}

// Preparation from a saved forward: with o the gated output (o = s y, s = sigmoid(g))
// and lse its natural-log row normaliser, per row and dim
//   dY = dO s (bf16), dG = dO o (1 - s), Delta = sum_d dO o, L = lse log2(e).
// Delta is dO . o = dY . y in exact arithmetic (the recomputing preparation uses the
// bf16 dY instead, which it has next to y). Eight threads per (token, head) row,
// eight dims each.
struct PrepArgs {
  const uint16_t *o, *g, *dO;
  const float *lse;  // natural log, [B*H][N]
  uint16_t *dy, *dg;
  float *L, *delta;  // log2 units, [B*H][N]
  long long rows;    // B * N * H
  int N, H;
};

__global__ __launch_bounds__(256) void anchor_prep_saved_kernel(PrepArgs a) {
  const long long r = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const long long rr = r < a.rows ? r : a.rows - 1;  // the row's 8 threads stay together
  const size_t off = (size_t)rr * kD + 8 * part;
  const uint4 ow = *reinterpret_cast<const uint4 *>(a.o + off);
  const uint4 dw = *reinterpret_cast<const uint4 *>(a.dO + off);
  uint4 gw = make_uint4(0, 0, 0, 0);
  if (a.g) gw = *reinterpret_cast<const uint4 *>(a.g + off);
  const uint32_t ov[4] = {ow.x, ow.y, ow.z, ow.w}, dv[4] = {dw.x, dw.y, dw.z, dw.w}, gv[4] = {gw.x, gw.y, gw.z, gw.w};
  uint32_t dyw[4], dgw[4];
  float part_delta = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float dy2[2], dg2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float o = e ? bf16_hi(ov[w]) : bf16_lo(ov[w]);
      const float d = e ? bf16_hi(dv[w]) : bf16_lo(dv[w]);
      const float s = a.g ? __builtin_amdgcn_rcpf(1.f + __expf(-(e ? bf16_hi(gv[w]) : bf16_lo(gv[w])))) : 1.f;
      dy2[e] = d * s;
      dg2[e] = d * o * (1.f - s);
      part_delta += d * o;
    }
    dyw[w] = pack_bf16(dy2[0], dy2[1]);
    dgw[w] = pack_bf16(dg2[0], dg2[1]);
  }
  part_delta += __shfl_xor(part_delta, 1);
  part_delta += __shfl_xor(part_delta, 2);
  part_delta += __shfl_xor(part_delta, 4);
  if (r >= a.rows) return;
  *reinterpret_cast<uint4 *>(a.dy + off) = make_uint4(dyw[0], dyw[1], dyw[2], dyw[3]);
  if (a.g) *reinterpret_cast<uint4 *>(a.dg + off) = make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]);
  if (part == 0) {
    const int h = (int)(r % a.H);
    const long long bn = r / a.H;
    const int n = (int)(bn % a.N), b = (int)(bn / a.N);
    const size_t i = ((size_t)b * a.H + h) * a.N + n;
    a.L[i] = a.lse[i] * 1.4426950408889634f;
    a.delta[i] = part_delta;
  }
}

hipError_t launch_vt(const void *x, void *xt, int B, int N, int H, int npad, hipStream_t stream) {
  VtArgs va;
  va.v = reinterpret_cast<const uint16_t *>(x);
  va.vt = reinterpret_cast<uint16_t *>(xt);
  va.N = N;
  va.H = H;
  va.npad = npad;
  hipLaunchKernelGGL(anchor_vt_kernel, dim3(npad / kBK, B * H), dim3(256), 0, stream, va);
  return hipGetLastError();
}

}  // namespace

namespace {
// gradient workspace: V^T, Q^T, dY^T, K^T (bf16, [B*H][64][npad]), dY (bf16, the
// layout of q), L and Delta (fp32, [B*H][N])
struct BwdLayout {
  size_t vt, qt, dyt, kt, dy, lse, delta, total;
};
BwdLayout bwd_layout(int B, int N, int H) {
  const size_t npad = ((size_t)N + kBK - 1) / kBK * kBK;
  const size_t t = align256((size_t)B * H * kD * npad * sizeof(uint16_t));
  BwdLayout l;
  l.vt = 0;
  l.qt = t;
  l.dyt = 2 * t;
  l.kt = 3 * t;
  l.dy = 4 * t;
  l.lse = l.dy + align256((size_t)B * N * H * kD * sizeof(uint16_t));
  l.delta = l.lse + align256((size_t)B * H * N * sizeof(float));
  l.total = l.delta + align256((size_t)B * H * N * sizeof(float));
  return l;
}
}  // namespace

size_t anchor_backward_workspace_bytes(int B, int N, int H) { return bwd_layout(B, N, H).total; }

hipError_t launch_anchor_backward(const AnchorBwdArgs &a, hipStream_t stream) {
  const int heads = a.B * a.H;
  const int npad = (a.N + kBK - 1) / kBK * kBK;
  const BwdLayout l = bwd_layout(a.B, a.N, a.H);
  char *ws = reinterpret_cast<char *>(a.ws);
  uint16_t *vt = reinterpret_cast<uint16_t *>(ws + l.vt), *qt = reinterpret_cast<uint16_t *>(ws + l.qt);
  uint16_t *dyt = reinterpret_cast<uint16_t *>(ws + l.dyt), *kt = reinterpret_cast<uint16_t *>(ws + l.kt);
  uint16_t *dy = reinterpret_cast<uint16_t *>(ws + l.dy);
  float *lse = reinterpret_cast<float *>(ws + l.lse), *delta = reinterpret_cast<float *>(ws + l.delta);

  hipError_t e;
  FwdArgs fa;
  memset(&fa, 0, sizeof(fa));
  fa.c = a.scale * 1.4426950408889634f;
  if (a.o && a.lse) {
    // preparation from the saved forward: elementwise, no second forward pass
    PrepArgs pa;
    pa.o = reinterpret_cast<const uint16_t *>(a.o);
    pa.g = reinterpret_cast<const uint16_t *>(a.g);
    pa.dO = reinterpret_cast<const uint16_t *>(a.dO);
    pa.lse = a.lse;
    pa.dy = dy;
    pa.dg = reinterpret_cast<uint16_t *>(a.dg);
    pa.L = lse;
    pa.delta = delta;
    pa.rows = (long long)a.B * a.N * a.H;
    pa.N = a.N;
    pa.H = a.H;
    hipLaunchKernelGGL(anchor_prep_saved_kernel, dim3((unsigned)((pa.rows + 31) / 32)), dim3(256), 0, stream, pa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    if ((e = launch_vt(a.v, vt, a.B, a.N, a.H, npad, stream)) != hipSuccess) return e;
    // preparation: the forward with its epilogue writing dG, dY, L, Delta
    fa.q = reinterpret_cast<const uint16_t *>(a.q);
    fa.k = reinterpret_cast<const uint16_t *>(a.k);
    fa.g = reinterpret_cast<const uint16_t *>(a.g);
    fa.vt = vt;
    fa.N = a.N;
    fa.H = a.H;
    fa.npad = npad;
    fa.dO = reinterpret_cast<const uint16_t *>(a.dO);
    fa.dg = reinterpret_cast<uint16_t *>(a.dg);
    fa.dy = dy;
    fa.lse = lse;
    fa.delta = delta;
    hipLaunchKernelGGL((anchor_fwd_kernel<kWaves, kMinWaves, false, true>),
                       dim3((a.N + 32 * kWaves - 1) / (32 * kWaves), heads), dim3(64 * kWaves), 0, stream, fa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_vt(a.q, qt, a.B, a.N, a.H, npad, stream)) != hipSuccess) return e;
  if ((e = launch_vt(dy, dyt, a.B, a.N, a.H, npad, stream)) != hipSuccess) return e;
  if ((e = launch_vt(a.k, kt, a.B, a.N, a.H, npad, stream)) != hipSuccess) return e;

  BwdArgs ba;
  ba.q = reinterpret_cast<const uint16_t *>(a.q);
  ba.k = reinterpret_cast<const uint16_t *>(a.k);
  ba.v = reinterpret_cast<const uint16_t *>(a.v);
  ba.dy = dy;
  ba.qt = qt;
  ba.dyt = dyt;
  ba.kt = kt;
  ba.lse = lse;
  ba.delta = delta;
  ba.dq = reinterpret_cast<uint16_t *>(a.dq);
  ba.dk = reinterpret_cast<uint16_t *>(a.dk);
  ba.dv = reinterpret_cast<uint16_t *>(a.dv);
  ba.N = a.N;
  ba.H = a.H;
  ba.npad = npad;
  ba.c = fa.c;
  ba.scale = a.scale;
  constexpr int kBwdWaves = 8;
  const dim3 grid((a.N + 32 * kBwdWaves - 1) / (32 * kBwdWaves), heads);
  hipLaunchKernelGGL((anchor_dkdv_kernel<kBwdWaves>), grid, dim3(64 * kBwdWaves), 0, stream, ba);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dq: the tile's two 32-key blocks one after the other keep it within 128
  // registers, so it runs sixteen waves (four per SIMD) like the forward
  constexpr int kDqWaves = 16;
  hipLaunchKernelGGL((anchor_dq_kernel<kDqWaves>), dim3((a.N + 32 * kDqWaves - 1) / (32 * kDqWaves), heads),
                     dim3(64 * kDqWaves), 0, stream, ba);
  return hipGetLastError();
}

size_t anchor_sparse_lds_bytes(int N) {
  const size_t nwords = (((size_t)N + kBK - 1) / kBK + 31) / 32;
  return nwords * (1 + kWaves / (kSparseQBlock / 32)) * sizeof(uint32_t);
}

size_t anchor_workspace_bytes(int B, int N, int H) {
  const size_t npad = ((size_t)N + kBK - 1) / kBK * kBK;
  return (size_t)B * H * kD * npad * sizeof(uint16_t);
}

hipError_t launch_anchor(const AnchorArgs &a, hipStream_t stream) {
  const int heads = a.B * a.H;
  const int npad = (a.N + kBK - 1) / kBK * kBK;
  hipError_t e = launch_vt(a.v, a.ws, a.B, a.N, a.H, npad, stream);
  if (e != hipSuccess) return e;

  FwdArgs fa;
  memset(&fa, 0, sizeof(fa));
  fa.q = reinterpret_cast<const uint16_t *>(a.q);
  fa.k = reinterpret_cast<const uint16_t *>(a.k);
  fa.g = reinterpret_cast<const uint16_t *>(a.g);
  fa.vt = reinterpret_cast<const uint16_t *>(a.ws);
  fa.o = reinterpret_cast<uint16_t *>(a.o);
  fa.N = a.N;
  fa.H = a.H;
  fa.npad = npad;
  fa.c = a.scale * 1.4426950408889634f;
  fa.blocks = a.blocks;
  fa.counts = a.counts;
  fa.max_blocks = a.max_blocks;
  fa.lse_out = a.lse;
  if (a.blocks) {
    fa.n_qb = (a.N + kSparseQBlock - 1) / kSparseQBlock;
    hipLaunchKernelGGL((anchor_fwd_kernel<kWaves, kMinWaves, true, false>),
                       dim3((a.N + 32 * kWaves - 1) / (32 * kWaves), heads), dim3(64 * kWaves),
                       anchor_sparse_lds_bytes(a.N), stream, fa);
  } else {
    fa.n_qb = 0;
    hipLaunchKernelGGL((anchor_fwd_kernel<kWaves, kMinWaves, false, false>),
                       dim3((a.N + 32 * kWaves - 1) / (32 * kWaves), heads), dim3(64 * kWaves), 0, stream, fa);
  }
  return hipGetLastError();
}

}  // namespace hla
