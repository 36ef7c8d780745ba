// Gated non-causal softmax anchor attention on the bf16 matrix cores
// (SANA-Video 2.0 abstract and summary: one layer in four is a gated softmax
// anchor; textbook scaled dot-product attention with a sigmoid output gate):
//   o_i = sigmoid(g_i) * sum_j softmax_j(scale * q_i . k_j) v_j
//
// Two kernels:
//   anchor_vt  writes V of each (b, h) transposed, [64 dims][Npad tokens],
//              tokens zero-padded to a multiple of 64 and permuted inside each
//              group of 16 so that every matrix-core operand of the P.V product
//              is one contiguous 16-byte LDS read (see kernel comment); for
//              the forward it also records each 64-key block's largest K norm
//              and finite |v|, and writes K in fp16.
//   anchor_fwd online-softmax attention. A work-group of 16 waves owns 512
//              query rows of one (b, h); wave w owns 32 rows. Per 64-key tile:
//                S^T = K Q^T   (A = K rows from LDS, B = Q^T held in registers)
//                softmax update in the exp2 domain, lane-local: the score layout
//                gives each lane one query row and 32 of the 64 keys
//                O^T += V^T P^T (A = V^T from LDS, B = P^T straight from the
//                score registers, rounded to bf16)
//              K and V^T tiles are double-buffered in LDS; the next tile's
//              global loads are issued before the current tile's products.
//              Where a static bound on the logits holds (most inputs), the
//              scores come from fp16 products of K and Q^T pre-scaled by
//              scale log2(e), so the weights are exp2 of the products with no
//              per-score arithmetic before the exponential.
// At most 128 registers per lane keep every accumulator in VGPRs with four
// waves per SIMD; on the running-max path the tile's row max is combined
// across the two lane halves with v_permlane32_swap. The softmax's vector work
// overlaps the matrix-core work of other waves only in part; that, not the
// matrix cores alone, sets the kernel's speed.
// The running max is refreshed lazily: rows keep their reference max until a
// tile exceeds it by more than 8 (log2 units), so exponentials stay <= 2^8
// and the O / row-sum rescale is almost never taken. The normaliser uses the
// same reference max, so the result is exact up to rounding.
#include <string.h>

#include <type_traits>

#include "device_common.h"

namespace hla {

namespace {

constexpr int kBK = 64;            // keys per tile
constexpr int kKRow = kD + 8;      // bf16 per LDS row of K (144 bytes)
constexpr int kVRow = kBK + 8;     // bf16 per LDS row of V^T (144 bytes)
constexpr int kORow = kD + 8;      // bf16 per LDS row of the output stage (144 bytes)
constexpr float kLazy = 8.0f;      // lazy max threshold, log2 units
constexpr float kStatic = 48.0f;   // largest static logit bound b_i, log2 units
// bounds for the half-precision scores: c |q_i| <= 2^10, |k_j|^2 <= 2^20, |v| <= 2^40
constexpr float kHalfQ = 1024.0f;
constexpr float kHalfK2 = 1048576.0f;
constexpr float kHalfV = 1099511627776.0f;
constexpr int kLateSleep = 4;      // the late wave group's start offset, units of 64 cycles
constexpr int kVmcnt0 = 0x0F70;    // s_waitcnt immediate: vmcnt(0), other counters free
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
  // optional: the largest squared norm of the K rows of each 64-key block,
  // [B*H][npad / 64] (the forward's static logit bound)
  const uint16_t *k;
  float *kmax2;
  // optional with kmax2: the largest finite |v| element of each 64-key block
  // ([B*H][npad / 64]) and K in half precision ([B*H][npad][64], rows past N
  // zero), for the forward's half-precision scores
  float *vmax;
  uint16_t *kh;
};

// two bf16 -> two fp16 (nearest even; exact for |x| in [2^-14, 65504])
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const _Float16 lo = (_Float16)bf16_lo(w), hi = (_Float16)bf16_hi(w);
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// largest finite |x| of the two bf16 in w as a bf16 bit pattern (0 if neither
// is finite): a NaN or Inf in v reaches only its own output column, whatever
// loop the forward takes, so only finite values bound the weights' headroom
__device__ __forceinline__ uint32_t finite_abs_bits(uint32_t x) { return x < 0x7f80u ? x : 0u; }
__device__ __forceinline__ uint32_t max_abs_bits(uint32_t w) {
  return max(finite_abs_bits(w & 0x7fffu), finite_abs_bits((w >> 16) & 0x7fffu));
}

__global__ __launch_bounds__(256) void anchor_vt_kernel(VtArgs a) {
  __shared__ uint16_t tile[kBK][kD + 2];
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int n0 = blockIdx.x * kBK;
  const size_t tok_stride = (size_t)a.H * kD;
  const uint16_t *vp = a.v + (size_t)b * a.N * tok_stride + (size_t)h * kD;
  uint32_t vm = 0u;  // largest finite |v| of this thread's elements, bf16 bits
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int c = tid + 256 * r;
    const int key = c >> 3, dc = c & 7;
    const int n = n0 + key;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < a.N) w = load_once_u4(vp + (size_t)n * tok_stride + 8 * dc);
    vm = max(max(vm, max_abs_bits(w.x)), max(max_abs_bits(w.y), max(max_abs_bits(w.z), max_abs_bits(w.w))));
    uint32_t *dst = reinterpret_cast<uint32_t *>(&tile[key][8 * dc]);
    dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
  }
  if (a.kmax2) {
    __shared__ float wmax[4];
    __shared__ uint32_t wvm[4];
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + 256 * r;
      const int key = c >> 3, dc = c & 7;
      const int n = n0 + key;
      float ss = 0.f;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (n < a.N) {
        w = load_once_u4(a.k + (vp - a.v) + (size_t)n * tok_stride + 8 * dc);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += bf16_lo(ws[j]) * bf16_lo(ws[j]) + bf16_hi(ws[j]) * bf16_hi(ws[j]);
      }
      if (a.kh)
        *reinterpret_cast<uint4 *>(a.kh + ((size_t)bh * a.npad + n) * kD + 8 * dc) =
            make_uint4(bf16x2_to_f16x2(w.x), bf16x2_to_f16x2(w.y), bf16x2_to_f16x2(w.z), bf16x2_to_f16x2(w.w));
      // the key's eight chunks sit in eight consecutive lanes
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      m = fmaxf(m, ss);
    }
    m = fmaxf(m, __shfl_xor(m, 8));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) vm = max(vm, (uint32_t)__shfl_xor((int)vm, o));
    if ((tid & 63) == 0) {
      wmax[tid >> 6] = m;
      wvm[tid >> 6] = vm;
    }
    __syncthreads();
    if (tid == 0) {
      const size_t blk = (size_t)bh * (a.npad / kBK) + blockIdx.x;
      a.kmax2[blk] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
      if (a.vmax) a.vmax[blk] = __uint_as_float(max(max(wvm[0], wvm[1]), max(wvm[2], wvm[3])) << 16);
    }
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
  // static logit bound (nullable): the largest squared K norm of each 64-key
  // block of the head, [B*H][npad / 64]
  const float *kmax2;
  // half-precision scores (nullable, with kmax2): the largest finite |v| of each
  // 64-key block, [B*H][npad / 64], and K in fp16, [B*H][npad][64]
  const float *vmax;
  const uint16_t *kh;
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
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

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
  // epilogue: each wave's 32 output rows (gate in, o out), whole 128-byte rows
  __shared__ __align__(16) uint16_t ostage[kPrep ? 1 : WAVES][32 * kORow];

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
  // Q^T resident before the tile loop. Without this wait the loads may still be
  // pending on the path of the waves that stage no tile, and the compiler then
  // waits for all loads (the next tile's included) before every tile's first product.
  __builtin_amdgcn_s_waitcnt(kVmcnt0);

  // Static bound. By Cauchy-Schwarz every logit of row i obeys
  // |c s_ij| <= c |q_i| max_j |k_j| =: b_i. Softmax does not depend on the
  // reference it subtracts, so while b_i <= kStatic a row needs no running max:
  // it subtracts nothing and takes the half-precision scores below (weights
  // within 2^(+-kStatic)), decided per work-group. Otherwise (or without the
  // key norms) the running max.
  bool stat = false, half_scores = false;
  float mref = -INFINITY, lsum = 0.f;
  if (a.kmax2) {
    __shared__ float wk[WAVES];
    __shared__ uint32_t wv[WAVES];
    __shared__ int all_half;
    if (tid == 0) all_half = 1;
    const int nblk = a.npad / kBK;
    const float *km = a.kmax2 + (size_t)bh * nblk;
    const float *vx = a.vmax ? a.vmax + (size_t)bh * nblk : nullptr;
    // maxima of non-negative floats compared as bit patterns: a NaN sorts
    // above every number and so fails every bound below
    float m = 0.f;
    uint32_t mv = 0u;
    for (int i = tid; i < nblk; i += kThreads) {
      m = fmaxf(m, km[i]);
      if (vx) mv = max(mv, __float_as_uint(vx[i]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      m = fmaxf(m, __shfl_xor(m, o));
      mv = max(mv, (uint32_t)__shfl_xor((int)mv, o));
    }
    if (lane == 0) {
      wk[wave] = m;
      wv[wave] = mv;
    }
    __syncthreads();
    m = wk[0];
    mv = wv[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      m = fmaxf(m, wk[w]);
      mv = max(mv, wv[w]);
    }
    float qn = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) qn += (float)qb[s][j] * (float)qb[s][j];
    qn += __shfl_xor(qn, 32);
    const float bnd = a.c * sqrtf(qn) * sqrtf(m);
    stat = __builtin_amdgcn_readfirstlane(__all(bnd <= kStatic)) != 0;
    if (a.kh) {
      // Half-precision scores, taken by the whole work-group or not at all (the
      // K tiles it stages are fp16 or bf16): every row static, c |q_i| and
      // |k_j| small enough that fp16's subnormal range costs nothing, and |v|
      // small enough that weights up to 2^kStatic cannot overflow O
      const bool ok = stat && __float_as_uint(a.c * sqrtf(qn)) <= __float_as_uint(kHalfQ) &&
                      __float_as_uint(m) <= __float_as_uint(kHalfK2) && mv <= __float_as_uint(kHalfV);
      if (lane == 0 && !__all(ok)) all_half = 0;
      __syncthreads();
      half_scores = all_half != 0;
      if (half_scores) mref = 0.f;
    }
  }
  // Two wave groups per SIMD (bit 2 of the wave index); the second starts each
  // tile a few hundred cycles late, so the two groups' matrix-core phases fall
  // less on each other's and more on the other group's vector phase (measured
  // on the bf16-score loop: co-execution +29%; neutral on the half-precision loop).
  const bool late = (__builtin_amdgcn_readfirstlane(wave) & 4) != 0;

  // tile loader: K (64 keys x 8 chunks, bf16 from the input or fp16 from the
  // copy) and V^T (64 dims x 8 chunks), 16-byte chunks spread over the
  // work-group; rows past the end of K repeat the last row (their scores are masked)
  uint4 kreg[kLoads], vreg[kLoads];
  auto load_tile = [&](int t, auto mode_c) {
    if (tid >= kLoaders) return;
    constexpr bool kHalf = decltype(mode_c)::value == 2;
    const uint16_t *ksrc = kHalf ? a.kh + (size_t)bh * a.npad * kD : kp;
    const size_t kstride = kHalf ? (size_t)kD : tok_stride;
    const int n0 = t * kBK;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + kLoaders * r;
      const int row = c >> 3, ch = c & 7;
      const int n = min(n0 + row, a.N - 1);
      kreg[r] = *reinterpret_cast<const uint4 *>(ksrc + (size_t)n * kstride + 8 * ch);
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

  // The tile loop, in two copies that keep each within the register budget:
  // kMode 0 running max (bf16 scores), 2 half-precision scores. A work-group's
  // waves all take the same one (its K tiles are staged in one format).
  auto tile_loop = [&](auto mode_c) {
    constexpr int kMode = decltype(mode_c)::value;
    // Q^T scaled by c = scale log2(e) and rounded to fp16 (11 significant
    // bits against bf16's 8): the products then give the exponents c s_ij
    // directly, and the weights 2^(c s_ij) need no reference: |c s_ij| <= b_i
    // <= kStatic keeps them within 2^(+-kStatic)
    f16x8_t qh[4];
    if constexpr (kMode == 2) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) qh[s][j] = (_Float16)(a.c * (float)qb[s][j]);
    }
    int t = next(0);
    if (t < ntiles) {
      load_tile(t, mode_c);
      store_tile(0);
    }
    __syncthreads();
    // Code placement: the half-precision loop below runs 39.3 ms per 720p/5s
    // call when its first instruction sits 40 or 44 bytes past a 64-byte
    // boundary and 41.0-42.7 ms at the other 4-byte offsets (same instructions,
    // bitwise equal output). These no-ops, executed once, put it at 44 with
    // this compiler in the forward and in the gradient preparation (whose code
    // before the loop differs); tests/test_anchor_placement.py checks both.
    if constexpr (kMode == 2) asm volatile("s_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0");
    if constexpr (kMode == 2 && kPrep)
      asm volatile("s_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\t"
                   "s_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0\n\ts_nop 0");
    for (int buf = 0; t < ntiles; buf ^= 1) {
      const int tnext = next(t + 1);
      if (tnext < ntiles) load_tile(tnext, mode_c);
      if (late) __builtin_amdgcn_s_sleep(kLateSleep);
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
          const uint16_t *kr = &ks[buf][(32 * kb + tl) * kKRow + 16 * s + 8 * half];
          if constexpr (kMode == 2)
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8_t *>(kr), qh[s],
                                                              sacc[kb], 0, 0, 0);
          else
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(kr), qb[s],
                                                               sacc[kb], 0, 0, 0);
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

      if constexpr (kMode == 0) {
        // running max, refreshed lazily: rows keep their reference until a tile
        // exceeds it by more than kLazy (log2 units), so weights stay <= 2^kLazy
        // and the O / row-sum rescale is almost never taken
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        const float mt = max_halves(mx) * a.c;
        const bool bump = mt > mref + kLazy;
        if (__any(bump)) {
          const float mnew = bump ? mt : mref;
          const float f = exp2f(mref - mnew);
          mref = mnew;
          lsum *= f;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[mb][i] *= f;
        }
      }

      // weights in the exp2 domain, rounded to bf16 for the P.V product; the row
      // sum adds the same bf16 weights (two per v_dot2)
      bf16x8_t pb[2][2];
      float ts = 0.f;
      const float nm = -mref;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          p[i] = __builtin_amdgcn_exp2f(kMode == 2 ? sacc[kb][i] : fmaf(sacc[kb][i], a.c, nm));
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
  };
  if (half_scores)
    tile_loop(std::integral_constant<int, 2>{});
  else
    tile_loop(std::integral_constant<int, 0>{});

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
  } else {
    if (n < a.N && a.lse_out && half == 0) a.lse_out[(size_t)bh * a.N + n] = (mref + log2f(l)) * 0.6931471805599453f;
    // The wave's 32 rows pass through its LDS stage as whole 128-byte rows: the
    // gate comes in and o goes out one row per eight lanes (16 bytes each), so
    // every line is read and written whole by one instruction.
    uint16_t *st = ostage[wave];
    const int rr = lane >> 3, rc = lane & 7;  // 8 rows per pass, 16-byte chunk rc
    if (a.g) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int nr = q0 + 8 * p + rr;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (nr < a.N) w = load_once_u4(a.g + head_base + (size_t)nr * tok_stride + 8 * rc);
        *reinterpret_cast<uint4 *>(&st[(8 * p + rr) * kORow + 8 * rc]) = w;
      }
      wave_lds_fence();
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = 32 * mb + 8 * i + 4 * half;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = oacc[mb][4 * i + j] * inv;
        uint2 *sp = reinterpret_cast<uint2 *>(&st[tl * kORow + col]);
        if (a.g) {
          const uint2 gw = *sp;
          y[0] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_lo(gw.x)));
          y[1] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_hi(gw.x)));
          y[2] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_lo(gw.y)));
          y[3] *= __builtin_amdgcn_rcpf(1.f + __expf(-bf16_hi(gw.y)));
        }
        *sp = make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
      }
    wave_lds_fence();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int nr = q0 + 8 * p + rr;
      const uint4 w = *reinterpret_cast<const uint4 *>(&st[(8 * p + rr) * kORow + 8 * rc]);
      if (nr < a.N) *reinterpret_cast<uint4 *>(a.o + head_base + (size_t)nr * tok_stride + 8 * rc) = w;
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

// Tiles of the gradient kernels go global -> LDS directly (no staging registers):
// rows of 128 bytes, unpadded, with row r's 16-byte chunk c in slot
// c ^ ((r >> 1) & 7). An operand read serves 16 lanes (16 rows, one chunk
// column) per pass over the 64 banks of 4 bytes; two consecutive rows fill one
// 256-byte bank line, so rows 2m and 2m + 1 take its two halves and the eight
// values of m take eight different slots: the 16 rows hit 64 different banks.
// One copy instruction moves 8 rows (64 lanes x 16 bytes).
__device__ __forceinline__ void copy_rows(const uint16_t *src, uint16_t *lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// A pointer the compiler keeps in scalar registers (p is the same in every lane).
__device__ __forceinline__ const uint16_t *wave_uniform(const uint16_t *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint16_t *>(((uint64_t)hi << 32) | lo);
}
// The same copy from a wave-uniform base (a buffer resource in scalar
// registers) plus this lane's byte offset, which then takes one vector
// register instead of a 64-bit address.
__device__ __forceinline__ void copy_rows_from(const uint16_t *base, uint32_t byte_off, uint16_t *lds) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, byte_off, 0, 0, 0);
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 3) void anchor_dkdv_kernel(BwdArgs a) {
  static_assert(WAVES == 12, "waves 0-7 copy the four tiles, waves 8 and 9 the row statistics");
  // one block, row statistics first: a read's 16-bit immediate offset reaches
  // the first 64 KB
  struct Lds {
    float ls[2][kBK], dls[2][kBK];  // L and -Delta of the tile's queries
    uint16_t qs[2][kBK * kD];       // Q rows of the query tile
    uint16_t ds[2][kBK * kD];       // dY rows
    uint16_t qts[2][kD * kBK];      // Q^T, permuted
    uint16_t dts[2][kD * kBK];      // dY^T, permuted
  };
  __shared__ __align__(16) Lds sm;
  auto &ls = sm.ls, &dls = sm.dls;
  auto &qs = sm.qs, &ds = sm.ds, &qts = sm.qts, &dts = sm.dts;

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
  const uint16_t *qp = wave_uniform(a.q + head_base), *dp = wave_uniform(a.dy + head_base);
  const uint16_t *qtp = wave_uniform(a.qt + (size_t)bh * kD * a.npad);
  const uint16_t *dtp = wave_uniform(a.dyt + (size_t)bh * kD * a.npad);
  const float *lsp = a.lse + (size_t)bh * a.N, *dlp = a.delta + (size_t)bh * a.N;

  // copier: wave w < 8 copies rows 32 (w % 2) .. +31 of tile w / 2 (Q, dY, Q^T,
  // dY^T) in four instructions of 8 rows; lane i takes row + i / 8 and fills
  // slot i % 8 with chunk (i % 8) ^ ((row >> 1) & 7), which is the lane's chunk
  // of instruction 0 for even instructions and that ^ 4 for odd ones. Waves 8
  // and 9 load L and -Delta of the next tile into a register.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int kind = wv >> 1, grp = 4 * (wv & 1);
  const int crow = 8 * grp + (lane >> 3);  // + 8 i
  const int cchunk = (lane & 7) ^ ((crow >> 1) & 7);
  // row tiles: byte offsets of instructions 0 and 1 from the tile's first row
  // (2 and 3 add 16 rows through the scalar offset)
  const uint32_t roff0 = 2 * ((uint32_t)crow * (uint32_t)tok_stride + 8 * cchunk);
  const uint32_t roff1 = 2 * ((uint32_t)(crow + 8) * (uint32_t)tok_stride + 8 * (cchunk ^ 4));
  const uint16_t *rsrc = kind == 0 ? qp : dp;
  // transposed tiles: this lane's pointers for instructions 0 and 1
  const uint16_t *tsrc = kind == 2 ? qtp : dtp;
  const uint16_t *tp0 = tsrc + (size_t)crow * a.npad + 8 * cchunk;
  const uint16_t *tp1 = tsrc + (size_t)(crow + 8) * a.npad + 8 * (cchunk ^ 4);
  const int ntiles = (a.N + kBK - 1) / kBK;
  float sf = 0.f;
  auto issue_tile = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int n0 = t * kBK;
    // every wave loads one value per lane (waves 8 and 9 keep L and Delta; rows
    // past N read row N - 1): one definition on every path, applied when stored
    sf = (wv == 8 ? lsp : dlp)[min(n0 + lane, a.N - 1)];
    if (wv < 4) {
      uint16_t *dst = kind == 0 ? qs[buf] : ds[buf];
      const uint16_t *base = wave_uniform(rsrc + (size_t)n0 * tok_stride);
      const uint32_t skip = 2 * 16 * (uint32_t)tok_stride;  // 16 rows, in bytes
      if (n0 + kBK <= a.N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, -1,
                                                                             0x00020000);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + 512 * (grp + i)),
                                                   16, (i & 1) ? roff1 : roff0, (i >> 1) * skip, 0, 0);
        }
      } else {
        // rows past the end copy row N - 1: finite data, weight 0
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t r = (uint32_t)min(crow + 8 * i, a.N - 1 - n0);
          copy_rows_from(base, 2 * (r * (uint32_t)tok_stride + 8 * (cchunk ^ (4 * (i & 1)))), dst + 512 * (grp + i));
        }
      }
    } else if (wv < 8) {
      uint16_t *dst = kind == 2 ? qts[buf] : dts[buf];
      const size_t skip = (size_t)16 * a.npad;  // 16 rows
#pragma unroll
      for (int i = 0; i < 4; ++i)
        copy_rows(((i & 1) ? tp1 : tp0) + (i >> 1) * skip + n0, dst + 512 * (grp + i));
    }
  };
  // past N: a weight of exactly 0 and no Delta
  auto store_stats = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const bool live = t * kBK + lane < a.N;
    if (wv == 8) ls[buf][lane] = live ? sf : INFINITY;
    if (wv == 9) dls[buf][lane] = live ? -sf : 0.f;
  };
  // this lane's operand rows tl (+ 32 per block): chunk 2j + half sits in slot
  // (2j + half) ^ ((tl >> 1) & 7); byte offsets within a tile
  uint32_t roff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) roff[j] = 2 * (tl * kD + 8 * ((2 * j + half) ^ ((tl >> 1) & 7)));

  f32x16_t dva[2], dka[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dva[mb][i] = dka[mb][i] = 0.f;

  // one tile of queries from buffer buf (a compile-time constant, so every LDS
  // address is a lane offset plus an immediate); its two 32-query blocks one
  // after the other
  auto tile = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    // the other buffers held tile t - 1, whose readers all passed the last barrier
    if (t + 1 < ntiles) issue_tile(t + 1, std::integral_constant<int, buf ^ 1>{});
    const char *qbase = reinterpret_cast<const char *>(qs[buf]);
    const char *dbase = reinterpret_cast<const char *>(ds[buf]);
    const char *qtbase = reinterpret_cast<const char *>(qts[buf]);
    const char *dtbase = reinterpret_cast<const char *>(dts[buf]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // scores and dP - Delta of 32 queries (rows) against the wave's 32 keys;
      // the dP products accumulate onto -Delta of their rows
      f32x16_t sacc, pacc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4_t nd = *reinterpret_cast<const f32x4_t *>(&dls[buf][32 * qb + 8 * i + 4 * half]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sacc[4 * i + j] = 0.f;
          pacc[4 * i + j] = nd[j];
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t off = 2 * 32 * qb * kD + roff[s];
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(qbase + off), kb[s], sacc,
                                                       0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(dbase + off), vb[s], pacc,
                                                       0, 0, 0);
      }
      // weights and logit gradients: lane rows 32 qb + 8 i + 4 half + j
      float pv[16], dv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4_t L = *reinterpret_cast<const f32x4_t *>(&ls[buf][32 * qb + 8 * i + 4 * half]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pj = __builtin_amdgcn_exp2f(fmaf(sacc[4 * i + j], a.c, -L[j]));
          pv[4 * i + j] = pj;
          dv[4 * i + j] = pj * pacc[4 * i + j];
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8_t pw = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16(pv[8 * u], pv[8 * u + 1]), pack_bf16(pv[8 * u + 2], pv[8 * u + 3]),
                                 pack_bf16(pv[8 * u + 4], pv[8 * u + 5]), pack_bf16(pv[8 * u + 6], pv[8 * u + 7])));
        const bf16x8_t sw = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16(dv[8 * u], dv[8 * u + 1]), pack_bf16(dv[8 * u + 2], dv[8 * u + 3]),
                                 pack_bf16(dv[8 * u + 4], dv[8 * u + 5]), pack_bf16(dv[8 * u + 6], dv[8 * u + 7])));
        // dV^T += dY^T P and dK^T += Q^T dS over these 16 queries: rows 32 mb + tl,
        // columns 32 qb + 16 u + 8 half (chunk 4 qb + 2 u + half)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const uint32_t off = 2 * 32 * mb * kBK + roff[2 * qb + u];
          dva[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(dtbase + off), pw,
                                                            dva[mb], 0, 0, 0);
          dka[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(qtbase + off), sw,
                                                            dka[mb], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) {
      store_stats(t + 1, std::integral_constant<int, buf ^ 1>{});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t + 1 has landed
      __syncthreads();
    }
  };

  issue_tile(0, std::integral_constant<int, 0>{});
  store_stats(0, std::integral_constant<int, 0>{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
  }
  const int n = k0 + tl;
  if (n < a.N) {
    store_cols(a.dk + head_base, tok_stride, n, half, dka, a.scale);
    store_cols(a.dv + head_base, tok_stride, n, half, dva, 1.f);
  }
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 3) void anchor_dq_kernel(BwdArgs a) {
  static_assert(WAVES == 12, "waves 0-3 copy K rows, 4-7 V rows, 8-11 K^T rows, 16 rows each");
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
  const uint16_t *kp = wave_uniform(a.k + head_base), *vp = wave_uniform(a.v + head_base);
  const uint16_t *ktp = wave_uniform(a.kt + (size_t)bh * kD * a.npad);

  // copier: wave w copies rows 16 (w % 4) .. +15 of tile w / 4 (K, V, K^T) in
  // two instructions of 8 rows; lane i takes row + i / 8 and fills slot i % 8
  // with chunk (i % 8) ^ ((row >> 1) & 7). Each tile's source is a wave-uniform
  // base plus this lane's byte offset.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int kind = wv >> 2, grp = 2 * (wv & 3);
  const int crow = 8 * grp + (lane >> 3);  // and crow + 8
  const int cchunk = (lane & 7) ^ ((crow >> 1) & 7), cchunk1 = cchunk ^ 4;
  const uint32_t off0 = 2 * ((uint32_t)crow * (uint32_t)tok_stride + 8 * cchunk);
  const uint32_t off1 = 2 * ((uint32_t)(crow + 8) * (uint32_t)tok_stride + 8 * cchunk1);
  const uint16_t *src = kind == 0 ? kp : vp;
  const uint16_t *kt0 = ktp + (size_t)crow * a.npad + 8 * cchunk, *kt1 = ktp + (size_t)(crow + 8) * a.npad + 8 * cchunk1;
  const int ntiles = (a.N + kBK - 1) / kBK;
  auto issue_tile = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int n0 = t * kBK;
    uint16_t *dst = kind == 0 ? ks[buf] : kind == 1 ? vr[buf] : kts[buf];
    if (kind == 2) {
      copy_rows(kt0 + n0, dst + 512 * grp);
      copy_rows(kt1 + n0, dst + 512 * (grp + 1));
    } else {
      // rows past the end copy row N - 1: finite data, weight 0
      uint32_t o0 = off0, o1 = off1;
      if (n0 + kBK > a.N) {
        o0 = 2 * ((uint32_t)min(crow, a.N - 1 - n0) * (uint32_t)tok_stride + 8 * cchunk);
        o1 = 2 * ((uint32_t)min(crow + 8, a.N - 1 - n0) * (uint32_t)tok_stride + 8 * cchunk1);
      }
      const uint16_t *base = wave_uniform(src + (size_t)n0 * tok_stride);
      copy_rows_from(base, o0, dst + 512 * grp);
      copy_rows_from(base, o1, dst + 512 * (grp + 1));
    }
  };
  // this lane's operand rows tl (+ 32 per block): chunk 2j + half sits in slot
  // (2j + half) ^ ((tl >> 1) & 7); byte offsets within a tile
  uint32_t roff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) roff[j] = 2 * (tl * kD + 8 * ((2 * j + half) ^ ((tl >> 1) & 7)));

  f32x16_t dqa[2], ndl;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[mb][i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndl[i] = -Dl;

  // one tile of keys from buffer buf (a compile-time constant, so every LDS
  // address is a lane offset plus an immediate)
  auto tile = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    // the other buffers held tile t - 1, whose readers all passed the last barrier
    if (t + 1 < ntiles) issue_tile(t + 1, std::integral_constant<int, buf ^ 1>{});
    const bool tail = (t + 1) * kBK > a.N;
    const char *kbase = reinterpret_cast<const char *>(ks[buf]);
    const char *vbase = reinterpret_cast<const char *>(vr[buf]);
    const char *tbase = reinterpret_cast<const char *>(kts[buf]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T and dP^T - Delta of 32 of the tile's keys (rows) against the wave's
      // 32 queries: the dP products accumulate onto -Delta of their columns
      f32x16_t sacc, pacc = ndl;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t off = 2 * 32 * kb * kD + roff[s];
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(kbase + off), qb[s], sacc,
                                                       0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(vbase + off), db[s], pacc,
                                                       0, 0, 0);
      }
      float dv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) dv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e], a.c, -L));
      // only a tile that reaches past N has keys to mask (weight 0)
      if (__builtin_expect(tail, 0)) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (t * kBK + 32 * kb + 8 * (e >> 2) + 4 * half + (e & 3) >= a.N) dv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) dv[e] *= pacc[e];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8_t sw = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16(dv[8 * u], dv[8 * u + 1]), pack_bf16(dv[8 * u + 2], dv[8 * u + 3]),
                                 pack_bf16(dv[8 * u + 4], dv[8 * u + 5]), pack_bf16(dv[8 * u + 6], dv[8 * u + 7])));
        // dQ^T += K^T dS^T over these keys
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const uint32_t off = 2 * 32 * mb * kBK + roff[2 * kb + u];
          dqa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(tbase + off), sw,
                                                            dqa[mb], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t + 1 has landed
      __syncthreads();
    }
  };

  issue_tile(0, std::integral_constant<int, 0>{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
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

hipError_t launch_vt(const void *x, void *xt, int B, int N, int H, int npad, hipStream_t stream,
                     const void *k = nullptr, float *kmax2 = nullptr, float *vmax = nullptr,
                     uint16_t *kh = nullptr) {
  VtArgs va;
  va.v = reinterpret_cast<const uint16_t *>(x);
  va.vt = reinterpret_cast<uint16_t *>(xt);
  va.N = N;
  va.H = H;
  va.npad = npad;
  va.k = reinterpret_cast<const uint16_t *>(k);
  va.kmax2 = kmax2;
  va.vmax = vmax;
  va.kh = kh;
  hipLaunchKernelGGL(anchor_vt_kernel, dim3(npad / kBK, B * H), dim3(256), 0, stream, va);
  return hipGetLastError();
}

}  // namespace

namespace {
// gradient workspace: V^T, Q^T, dY^T, K^T (bf16, [B*H][64][npad]), dY (bf16, the
// layout of q), L and Delta (fp32, [B*H][N]), then for the preparation forward the
// key-block norms and value maxima (fp32, [B*H][npad / 64]) and K in fp16 ([B*H][npad][64])
struct BwdLayout {
  size_t vt, qt, dyt, kt, dy, lse, delta, kmax2, vmax, kh, total;
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
  l.kmax2 = l.delta + align256((size_t)B * H * N * sizeof(float));
  l.vmax = l.kmax2 + align256((size_t)B * H * (npad / kBK) * sizeof(float));
  l.kh = l.vmax + align256((size_t)B * H * (npad / kBK) * sizeof(float));
  l.total = l.kh + t;
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
    float *kmax2 = reinterpret_cast<float *>(ws + l.kmax2), *vmax = reinterpret_cast<float *>(ws + l.vmax);
    uint16_t *kh = reinterpret_cast<uint16_t *>(ws + l.kh);
    if ((e = launch_vt(a.v, vt, a.B, a.N, a.H, npad, stream, a.k, kmax2, vmax, kh)) != hipSuccess) return e;
    fa.kmax2 = kmax2;
    fa.vmax = vmax;
    fa.kh = kh;
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
  constexpr int kBwdWaves = 12;
  const dim3 grid((a.N + 32 * kBwdWaves - 1) / (32 * kBwdWaves), heads);
  hipLaunchKernelGGL((anchor_dkdv_kernel<kBwdWaves>), grid, dim3(64 * kBwdWaves), 0, stream, ba);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dq: the tile's two 32-key blocks one after the other; twelve waves, three
  // per SIMD
  constexpr int kDqWaves = 12;
  hipLaunchKernelGGL((anchor_dq_kernel<kDqWaves>), dim3((a.N + 32 * kDqWaves - 1) / (32 * kDqWaves), heads),
                     dim3(64 * kDqWaves), 0, stream, ba);
  return hipGetLastError();
}

size_t anchor_sparse_lds_bytes(int N) {
  const size_t nwords = (((size_t)N + kBK - 1) / kBK + 31) / 32;
  return nwords * (1 + kWaves / (kSparseQBlock / 32)) * sizeof(uint32_t);
}

namespace {
// forward workspace: V^T (bf16, [B*H][64][npad]), the key-block norms and
// value maxima (fp32, [B*H][npad / 64] each), K in fp16 ([B*H][npad][64])
struct FwdLayout {
  size_t kmax2, vmax, kh, total;
};
FwdLayout fwd_layout(int B, int N, int H) {
  const size_t npad = ((size_t)N + kBK - 1) / kBK * kBK;
  const size_t t = align256((size_t)B * H * kD * npad * sizeof(uint16_t));
  const size_t blk = align256((size_t)B * H * (npad / kBK) * sizeof(float));
  FwdLayout l;
  l.kmax2 = t;
  l.vmax = t + blk;
  l.kh = t + 2 * blk;
  l.total = l.kh + (size_t)B * H * kD * npad * sizeof(uint16_t);
  return l;
}
}  // namespace

size_t anchor_workspace_bytes(int B, int N, int H) { return fwd_layout(B, N, H).total; }

hipError_t launch_anchor(const AnchorArgs &a, hipStream_t stream) {
  const int heads = a.B * a.H;
  const int npad = (a.N + kBK - 1) / kBK * kBK;
  const FwdLayout l = fwd_layout(a.B, a.N, a.H);
  char *ws = reinterpret_cast<char *>(a.ws);
  float *kmax2 = reinterpret_cast<float *>(ws + l.kmax2), *vmax = reinterpret_cast<float *>(ws + l.vmax);
  uint16_t *kh = reinterpret_cast<uint16_t *>(ws + l.kh);
  hipError_t e = launch_vt(a.v, a.ws, a.B, a.N, a.H, npad, stream, a.k, kmax2, vmax, kh);
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
  fa.kmax2 = kmax2;
  fa.vmax = vmax;
  fa.kh = kh;
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
