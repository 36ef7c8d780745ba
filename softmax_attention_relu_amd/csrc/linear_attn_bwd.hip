// Gradients of ReLU-kernel linear attention with RoPE after the ReLU and the
// sigmoid output gate, bidirectional and block-causal (forward: SANA-Video
// notes, section 3.2 output equation; section 3.4 causal equation and
// Algorithm 1's cache). Chunk c's queries read the cache KV_c, ksum_c (the
// carried state plus every chunk up to c; one chunk for the bidirectional
// layer). With s = sigmoid(g), y = num / den and a_i = R_i relu(q_i):
//
//   dG_i = dO_i y_i s_i (1 - s_i),  dY_i = dO_i s_i
//   dnum_i = dY_i / den_i,          dden_i = -(dY_i . y_i) / den_i
//   dq_i = (R_i^T (KV_c dnum_i) + dden_i ksum_c) [q_i > 0]
//   G_c  = dKV_out + sum_{c' >= c} sum_{i in c'} a_i^T dnum_i
//   Gz_c = dksum_out + sum_{c' >= c} sum_{i in c'} dden_i relu(q_i)
//   dk_j = (R_j^T (G_c v_j) + Gz_c) [k_j > 0],  dv_j = G_c^T R_j relu(k_j)
//
// and the carried state receives G_0, Gz_0. Four steps on the caller's stream:
//   1. the forward's state build and prefix scan over (k, v): KV_c, ksum_c;
//   2. la_bwd_query, per (b, 4 heads, 32-token steps of one chunk): y again
//      from KV_c, then dG and dq; dnum (bf16) and dden (fp32) go to the
//      workspace;
//   3. the same state build over (q, dnum), its key sum weighted by dden, and
//      a suffix scan from dKV_out: G_c, Gz_c;
//   4. la_bwd_key, per (b, 4 heads, 32-token steps): dk and dv.
// Steps 2 and 4 are built like the forward's apply: one head per wave, whole
// 128-byte rows in and out through a per-wave LDS stage, the 64x64 fp32
// matrices held in registers as bf16 hi + lo matrix-core operands.
#include <algorithm>

#include "device_common.h"

namespace hla {

namespace {

constexpr int kHeads = 4;     // one head per wave
constexpr int kStep = 32;     // tokens per wave step
constexpr int kRow = kD + 8;  // bf16 per staged token row (144 bytes)

// RoPE variants
constexpr int kNoRope = 0;
constexpr int kRopeAny = 1;      // any even band widths: each pair looked up
constexpr int kRopeAligned = 2;  // band widths multiples of 8: two 16-byte loads per 8 dims

struct BwdArgs {
  const uint16_t *x0, *x1, *gate;  // query pass: q, dO, g (nullable); key pass: k, v
  uint16_t *y0, *y1, *y2;          // query pass: dq, dg, dnum; key pass: dk, dv
  float *dden;                     // query pass: [B*H][N]
  int N, H, L, n_chunks, parts_per_chunk, ngroups;
  RopeArgs rope;
  float eps;
  const float *state;  // [B*H][n_chunks][kStateFloats]: KV_c, ksum_c or G_c, Gz_c
  // the forward's saved state instead (one chunk): KV [B*H][D][D] in state,
  // ksum [B*H][D] here; null for the records above
  const float *ksum;
};

// The chunk's 64x64 matrix and its key sum (or gradient key sum)
__device__ __forceinline__ const float *state_matrix(const BwdArgs &a, int bh, int chunk) {
  return a.ksum ? a.state + (size_t)bh * kD * kD : a.state + ((size_t)bh * a.n_chunks + chunk) * kStateFloats;
}
__device__ __forceinline__ const float *state_sum(const BwdArgs &a, int bh, int chunk) {
  return a.ksum ? a.ksum + (size_t)bh * kD : state_matrix(a, bh, chunk) + kD * kD;
}

// Lane layout of a step: lane (tl = lane % 32, hf = lane / 32) holds token tl
// and the 32 dims 32*mb + 16*hf + 8*v + t (mb, v in {0, 1}, t < 8), kept as
// four 8-dim pieces [mb][v]. The matrix-core products reduce over the dims in
// this order: K step s (16 dims) takes piece [s/2][s%2] of both halves, so
// each lane's B operand is one of its own pieces.
//
// A operands of the 64x64 fp32 matrix M (row-major) for out = A b with b in
// the lane layout: kTrans gives A = M^T (out_e = sum_d M[d][e] b_d), otherwise
// A = M (out_d = sum_e M[d][e] b_e). The output rows are permuted (row
// 8i + 4h + j of block mb is dim 32*mb + 16*h + 4*i + j), so accumulator entry
// r of block mb holds dim 32*mb + 16*hf + r: again the lane layout, piece
// [mb][r / 8], element r % 8. M goes in as bf16 hi + lo parts.
template <bool kTrans>
__device__ __forceinline__ void state_operands(const float *M, int tl, int hf, bf16x8_t hi[2][4],
                                               bf16x8_t lo[2][4]) {
  const int el = (((tl >> 2) & 1) << 4) | ((tl >> 3) << 2) | (tl & 3);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kb = 32 * (s >> 1) + 16 * hf + 8 * (s & 1);
      const int m = 32 * mb + el;
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const float x0 = kTrans ? M[(kb + t) * kD + m] : M[m * kD + kb + t];
        const float x1 = kTrans ? M[(kb + t + 1) * kD + m] : M[m * kD + kb + t + 1];
        const uint32_t w = pack_bf16(x0, x1);
        wh[t / 2] = w;
        wl[t / 2] = pack_bf16(x0 - bf16_lo(w), x1 - bf16_hi(w));
      }
      hi[mb][s] = __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
      lo[mb][s] = __builtin_bit_cast(bf16x8_t, make_uint4(wl[0], wl[1], wl[2], wl[3]));
    }
}

// acc[mb] = A b over the four K steps, hi and lo parts
__device__ __forceinline__ void state_product(const bf16x8_t hi[2][4], const bf16x8_t lo[2][4],
                                              const u32x4_t b[2][2], f32x16_t acc[2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, b[s >> 1][s & 1]);
      acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi[mb][s], bb, acc[mb], 0, 0, 0);
      acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo[mb][s], bb, acc[mb], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void unpack8(const u32x4_t w, float x[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

__device__ __forceinline__ u32x4_t pack8(const float x[8]) {
  return u32x4_t{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
}

// Whole-row access: lane (r8 = lane / 8, c8 = lane % 8) moves dims 8*c8..+7 of
// tokens sub + 8u + r8 (u < 4); p already points at dims 8*c8 of token 0.
// Loads past the step read its last token (always valid).
__device__ __forceinline__ void load_rows(const uint16_t *p, size_t stride, int sub, int hi, int r8,
                                          u32x4_t rows[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t n = (size_t)min(sub + 8 * u + r8, hi - 1);
    rows[u] = load_once16(p + n * stride);
  }
}

__device__ __forceinline__ void rows_to_stage(uint16_t *st, const u32x4_t rows[4], int r8, int c8) {
#pragma unroll
  for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4_t *>(st + (8 * u + r8) * kRow + 8 * c8) = rows[u];
}

__device__ __forceinline__ void stage_to_lane(const uint16_t *st, int tl, int hf, u32x4_t x[2][2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 2; ++v)
      x[mb][v] = *reinterpret_cast<const u32x4_t *>(st + tl * kRow + 32 * mb + 16 * hf + 8 * v);
}

__device__ __forceinline__ void lane_to_stage(uint16_t *st, const u32x4_t x[2][2], int tl, int hf) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 2; ++v)
      *reinterpret_cast<u32x4_t *>(st + tl * kRow + 32 * mb + 16 * hf + 8 * v) = x[mb][v];
}

template <bool kNT>
__device__ __forceinline__ void stage_to_rows(const uint16_t *st, uint16_t *p, size_t stride, int sub, int hi, int r8,
                                              int c8) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int n = sub + 8 * u + r8;
    const u32x4_t w = *reinterpret_cast<const u32x4_t *>(st + (8 * u + r8) * kRow + 8 * c8);
    if (n < hi) {
      if constexpr (kNT)
        store_nt(p + (size_t)n * stride, w);
      else
        *reinterpret_cast<u32x4_t *>(p + (size_t)n * stride) = w;
    }
  }
}

// Per-wave position of a step: which head, chunk and token steps.
struct StepRange {
  int h, bh, chunk, first, c_hi;
};

__device__ __forceinline__ bool step_range(const BwdArgs &a, int wave, StepRange &r) {
  const int hgroup = blockIdx.x % a.ngroups;
  const int pid = blockIdx.x / a.ngroups;
  r.chunk = pid / a.parts_per_chunk;
  const int part = pid - r.chunk * a.parts_per_chunk;
  const int c_lo = r.chunk * a.L;
  r.c_hi = min(a.N, c_lo + a.L);
  r.first = c_lo + part * kStep;
  r.h = kHeads * hgroup + wave;
  r.bh = blockIdx.y * a.H + r.h;
  return r.first < r.c_hi && r.h < a.H;
}

template <int kRopeMode>
struct PieceRope {
  ChunkRope<kRopeMode == kRopeAligned> cr[2][2];
  __device__ __forceinline__ void init(const RopeArgs &r, int hf) {
    if constexpr (kRopeMode != kNoRope) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 2; ++v) cr[mb][v].init(r, 4 * mb + 2 * hf + v);
    }
  }
  __device__ __forceinline__ void get(const RopeArgs &r, int n, f32x2_t cs[2][2][4]) const {
    if constexpr (kRopeMode != kNoRope) {
      const TokenPos tp = token_pos(r, (uint32_t)n);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 2; ++v) cr[mb][v].get(tp, cs[mb][v]);
    }
  }
};

// relu of a piece, optionally its key-sum dot with z, then R (forward rotation)
template <bool kRope>
__device__ __forceinline__ u32x4_t features(const u32x4_t w, const f32x2_t cs[4], const float *z, float &dot) {
  float x[8];
  unpack8(w, x);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    x[t] = relu(x[t]);
    if (z) dot += x[t] * z[t];
  }
  if constexpr (kRope) {
#pragma unroll
    for (int j = 0; j < 4; ++j) rotate(x[2 * j], x[2 * j + 1], cs[j]);
  }
  return pack8(x);
}

// (R^T d + z) [x > 0] of a piece: d from accumulator entries 8v..8v+7
template <bool kRope>
__device__ __forceinline__ u32x4_t input_grad(const f32x16_t &acc, int v, const f32x2_t cs[4], const float z[8],
                                              float zscale, const u32x4_t xw) {
  float d[8], x[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) d[t] = acc[8 * v + t];
  if constexpr (kRope) {
#pragma unroll
    for (int j = 0; j < 4; ++j) rotate(d[2 * j], d[2 * j + 1], f32x2_t{cs[j].x, -cs[j].y});
  }
  unpack8(xw, x);
#pragma unroll
  for (int t = 0; t < 8; ++t) d[t] = x[t] > 0.f ? d[t] + zscale * z[t] : 0.f;
  return pack8(d);
}

// ---------------------------------------------------------------------------
// Query side: dG, dq, and the inputs dnum, dden of the key side's sums.
template <int kRopeMode, bool kGate>
__global__ __launch_bounds__(256, 1) void la_bwd_query_kernel(BwdArgs a) {
  constexpr bool kRope = kRopeMode != kNoRope;
  __shared__ __align__(16) uint16_t stage_all[kHeads][3][kStep * kRow];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, tl = lane & 31;
  const int r8 = lane >> 3, c8 = lane & 7;
  StepRange sr;
  if (!step_range(a, wave, sr)) return;  // no work-group barrier in this kernel

  const float *P = state_matrix(a, sr.bh, sr.chunk);
  const float *Z = state_sum(a, sr.bh, sr.chunk);
  bf16x8_t th[2][4], tlo[2][4], nh[2][4], nlo[2][4];
  state_operands<true>(P, tl, hf, th, tlo);
  state_operands<false>(P, tl, hf, nh, nlo);
  float z[2][2][8];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int t = 0; t < 8; ++t) z[mb][v][t] = Z[32 * mb + 16 * hf + 8 * v + t];
  PieceRope<kRopeMode> pr;
  pr.init(a.rope, hf);

  const size_t stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)blockIdx.y * a.N * stride + (size_t)sr.h * kD + 8 * c8;
  const uint16_t *qp = a.x0 + head_base;
  const uint16_t *dop = a.x1 + head_base;
  const uint16_t *gp = kGate ? a.gate + head_base : nullptr;
  uint16_t *dqp = a.y0 + head_base;
  uint16_t *dgp = kGate ? a.y1 + head_base : nullptr;
  uint16_t *dnp = a.y2 + head_base;
  float *ddp = a.dden + (size_t)sr.bh * a.N;
  uint16_t *stq = stage_all[wave][0], *std_ = stage_all[wave][1], *stg = stage_all[wave][2];

  for (int sub = sr.first; sub < sr.c_hi; sub += a.parts_per_chunk * kStep) {
    const int hi = min(sr.c_hi, sub + kStep);
    u32x4_t qrow[4], drow[4], grow[4];
    load_rows(qp, stride, sub, hi, r8, qrow);
    load_rows(dop, stride, sub, hi, r8, drow);
    if constexpr (kGate) load_rows(gp, stride, sub, hi, r8, grow);
    f32x2_t cs[2][2][4];
    pr.get(a.rope, min(sub + tl, hi - 1), cs);
    rows_to_stage(stq, qrow, r8, c8);
    rows_to_stage(std_, drow, r8, c8);
    if constexpr (kGate) rows_to_stage(stg, grow, r8, c8);
    wave_lds_fence();
    u32x4_t qL[2][2], dL[2][2], gL[2][2];
    stage_to_lane(stq, tl, hf, qL);
    stage_to_lane(std_, tl, hf, dL);
    if constexpr (kGate) stage_to_lane(stg, tl, hf, gL);

    // a = R relu(q) and the denominator's half dot product
    float denp = 0.f;
    u32x4_t aL[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 2; ++v) aL[mb][v] = features<kRope>(qL[mb][v], cs[mb][v], z[mb][v], denp);
    f32x16_t acc[2];
    state_product(th, tlo, aL, acc);  // num = a KV
    const float inv = 1.f / (denp + __shfl_xor(denp, 32) + a.eps);

    // y, gate, dY; dnum and the half dot dY . y
    float dot = 0.f;
    u32x4_t dnL[2][2], dgL[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        float dov[8], gv[8], dn[8], dg[8];
        unpack8(dL[mb][v], dov);
        if constexpr (kGate) unpack8(gL[mb][v], gv);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float y = acc[mb][8 * v + t] * inv;
          float dy = dov[t];
          if constexpr (kGate) {
            const float s = sigmoid_fast(gv[t]);
            dg[t] = dy * y * s * (1.f - s);
            dy *= s;
          }
          dot += dy * y;
          dn[t] = dy * inv;
        }
        dnL[mb][v] = pack8(dn);
        if constexpr (kGate) dgL[mb][v] = pack8(dg);
      }
    const float dden = -(dot + __shfl_xor(dot, 32)) * inv;

    // da = KV dnum (bf16 dnum, as stored for the key side), then dq
    state_product(nh, nlo, dnL, acc);
    u32x4_t dqL[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 2; ++v) dqL[mb][v] = input_grad<kRope>(acc[mb], v, cs[mb][v], z[mb][v], dden, qL[mb][v]);

    // back to rows through the stage (the lane reads above are done: one wave's
    // LDS requests are served in order)
    wave_lds_fence();
    lane_to_stage(stq, dqL, tl, hf);
    lane_to_stage(std_, dnL, tl, hf);
    if constexpr (kGate) lane_to_stage(stg, dgL, tl, hf);
    wave_lds_fence();
    stage_to_rows<true>(stq, dqp, stride, sub, hi, r8, c8);
    stage_to_rows<false>(std_, dnp, stride, sub, hi, r8, c8);
    if constexpr (kGate) stage_to_rows<true>(stg, dgp, stride, sub, hi, r8, c8);
    if (hf == 0 && sub + tl < hi) ddp[sub + tl] = dden;
    wave_lds_fence();  // the next step's stage stores come after these loads
  }
}

// ---------------------------------------------------------------------------
// Key side: dk = (R^T (G v) + Gz) [k > 0], dv = G^T R relu(k).
template <int kRopeMode>
__global__ __launch_bounds__(256, 1) void la_bwd_key_kernel(BwdArgs a) {
  constexpr bool kRope = kRopeMode != kNoRope;
  __shared__ __align__(16) uint16_t stage_all[kHeads][2][kStep * kRow];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, tl = lane & 31;
  const int r8 = lane >> 3, c8 = lane & 7;
  StepRange sr;
  if (!step_range(a, wave, sr)) return;  // no work-group barrier in this kernel

  const float *P = state_matrix(a, sr.bh, sr.chunk);
  const float *Z = state_sum(a, sr.bh, sr.chunk);
  bf16x8_t th[2][4], tlo[2][4], nh[2][4], nlo[2][4];
  state_operands<true>(P, tl, hf, th, tlo);
  state_operands<false>(P, tl, hf, nh, nlo);
  float z[2][2][8];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int t = 0; t < 8; ++t) z[mb][v][t] = Z[32 * mb + 16 * hf + 8 * v + t];
  PieceRope<kRopeMode> pr;
  pr.init(a.rope, hf);

  const size_t stride = (size_t)a.H * kD;
  const size_t head_base = (size_t)blockIdx.y * a.N * stride + (size_t)sr.h * kD + 8 * c8;
  const uint16_t *kp = a.x0 + head_base;
  const uint16_t *vp = a.x1 + head_base;
  uint16_t *dkp = a.y0 + head_base;
  uint16_t *dvp = a.y1 + head_base;
  uint16_t *stk = stage_all[wave][0], *stv = stage_all[wave][1];

  for (int sub = sr.first; sub < sr.c_hi; sub += a.parts_per_chunk * kStep) {
    const int hi = min(sr.c_hi, sub + kStep);
    u32x4_t krow[4], vrow[4];
    load_rows(kp, stride, sub, hi, r8, krow);
    load_rows(vp, stride, sub, hi, r8, vrow);
    f32x2_t cs[2][2][4];
    pr.get(a.rope, min(sub + tl, hi - 1), cs);
    rows_to_stage(stk, krow, r8, c8);
    rows_to_stage(stv, vrow, r8, c8);
    wave_lds_fence();
    u32x4_t kL[2][2], vL[2][2];
    stage_to_lane(stk, tl, hf, kL);
    stage_to_lane(stv, tl, hf, vL);

    float unused = 0.f;
    u32x4_t cL[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 2; ++v) cL[mb][v] = features<kRope>(kL[mb][v], cs[mb][v], nullptr, unused);
    f32x16_t acc[2];
    u32x4_t dvL[2][2], dkL[2][2];
    state_product(th, tlo, cL, acc);  // dv = G^T c
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        float x[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) x[t] = acc[mb][8 * v + t];
        dvL[mb][v] = pack8(x);
      }
    state_product(nh, nlo, vL, acc);  // dc = G v
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 2; ++v) dkL[mb][v] = input_grad<kRope>(acc[mb], v, cs[mb][v], z[mb][v], 1.f, kL[mb][v]);

    wave_lds_fence();
    lane_to_stage(stk, dkL, tl, hf);
    lane_to_stage(stv, dvL, tl, hf);
    wave_lds_fence();
    stage_to_rows<true>(stk, dkp, stride, sub, hi, r8, c8);
    stage_to_rows<true>(stv, dvp, stride, sub, hi, r8, c8);
    wave_lds_fence();  // the next step's stage stores come after these loads
  }
}

template <int kRopeMode>
void launch_bwd_kernels(bool gate, dim3 grid, const BwdArgs &qa, const BwdArgs &ka, hipStream_t stream,
                        int which) {
  if (which == 0) {
    if (gate)
      hipLaunchKernelGGL((la_bwd_query_kernel<kRopeMode, true>), grid, dim3(256), 0, stream, qa);
    else
      hipLaunchKernelGGL((la_bwd_query_kernel<kRopeMode, false>), grid, dim3(256), 0, stream, qa);
  } else {
    hipLaunchKernelGGL((la_bwd_key_kernel<kRopeMode>), grid, dim3(256), 0, stream, ka);
  }
}

void launch_bwd(const RopeArgs &r, bool gate, dim3 grid, const BwdArgs &qa, const BwdArgs &ka, hipStream_t stream,
                int which) {
  if (!r.enabled)
    launch_bwd_kernels<kNoRope>(gate, grid, qa, ka, stream, which);
  else if (r.aligned)
    launch_bwd_kernels<kRopeAligned>(gate, grid, qa, ka, stream, which);
  else
    launch_bwd_kernels<kRopeAny>(gate, grid, qa, ka, stream, which);
}

}  // namespace

LinearPlan plan_linear_backward(int B, int N, int H, int chunk_tokens) {
  LinearPlan p = plan_linear(B, N, H, chunk_tokens);
  // dnum (bf16, the layout of q) and dden (fp32, [B*H][N]) after the state regions
  p.dnum_offset = p.total_bytes;
  p.total_bytes += align256((size_t)B * N * H * kD * sizeof(uint16_t));
  p.dden_offset = p.total_bytes;
  p.total_bytes += align256((size_t)B * H * N * sizeof(float));
  return p;
}

hipError_t launch_linear_backward(const LinearBwdArgs &a, const LinearPlan &p, hipStream_t stream) {
  char *ws = reinterpret_cast<char *>(a.ws);
  uint16_t *dnum = reinterpret_cast<uint16_t *>(ws + p.dnum_offset);
  float *dden = reinterpret_cast<float *>(ws + p.dden_offset);

  // 1. forward cache per chunk
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
  s.final_kv = nullptr;
  s.final_ksum = nullptr;
  s.reverse = false;
  s.init_copy = nullptr;
  float *state = nullptr;
  hipError_t e;
  if (!a.kv_saved && (e = launch_state_sums(HLA_BF16, s, p, a.ws, stream, &state)) != hipSuccess) return e;

  BwdArgs qa;
  qa.x0 = reinterpret_cast<const uint16_t *>(a.q);
  qa.x1 = reinterpret_cast<const uint16_t *>(a.dO);
  qa.gate = reinterpret_cast<const uint16_t *>(a.g);
  qa.y0 = reinterpret_cast<uint16_t *>(a.dq);
  qa.y1 = reinterpret_cast<uint16_t *>(a.dg);
  qa.y2 = dnum;
  qa.dden = dden;
  qa.N = a.N;
  qa.H = a.H;
  qa.L = p.chunk_len;
  qa.n_chunks = p.n_chunks;
  qa.parts_per_chunk = p.apply_per_chunk;
  qa.ngroups = p.ngroups;
  qa.rope = a.rope;
  qa.eps = a.eps;
  // the query side reads the forward's saved state where it is given (one
  // chunk), the records of the build and scan otherwise
  qa.state = a.kv_saved ? a.kv_saved : state;
  qa.ksum = a.kv_saved ? a.ksum_saved : nullptr;
  BwdArgs ka = qa;
  ka.x0 = reinterpret_cast<const uint16_t *>(a.k);
  ka.x1 = reinterpret_cast<const uint16_t *>(a.v);
  ka.gate = nullptr;
  ka.y0 = reinterpret_cast<uint16_t *>(a.dk);
  ka.y1 = reinterpret_cast<uint16_t *>(a.dv);
  ka.y2 = nullptr;
  ka.dden = nullptr;
  const dim3 grid(p.n_chunks * p.apply_per_chunk * p.ngroups, a.B);

  // 2. query side
  launch_bwd(a.rope, a.g != nullptr, grid, qa, ka, stream, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // 3. key-side sums over (q, dnum), key sum weighted by dden, suffix scan
  s.k = a.q;
  s.v = dnum;
  s.zw = dden;
  s.start_kv = a.dkv_out;
  s.start_ksum = a.dksum_out;
  s.final_kv = a.dkv_in;
  s.final_ksum = a.dksum_in;
  s.reverse = true;
  e = launch_state_sums(HLA_BF16, s, p, a.ws, stream, &state);
  if (e != hipSuccess) return e;

  // 4. key side
  ka.state = state;
  ka.ksum = nullptr;
  launch_bwd(a.rope, false, grid, qa, ka, stream, 1);
  return hipGetLastError();
}

}  // namespace hla
