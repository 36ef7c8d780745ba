// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hla.h"

namespace hla {

constexpr int kD = 64;                    // the only head dimension built
constexpr int kStateFloats = kD * kD + kD; // one (KV, ksum) record: D*D state then D key sum

// Division by a fixed divisor d >= 1 for numerators 0 <= n < 2^31:
// n / d == (umulhi(n, m) + n) >> s  (round-up method with a 33-bit magic).
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << 32) * ((1ull << s) - d)) / d) + 1);
  return f;
}

// RoPE tables and grid as the kernels see them. Token n sits at
// t = n / (gh*gw), y = (n % (gh*gw)) / gw, x = n % gw.
struct RopeArgs {
  int enabled;
  int aligned;           // band widths multiples of 8 and 16-byte aligned tables
  int d_t, d_h, d_w;
  uint32_t hw, w, h;     // grid_h * grid_w, grid_w, grid_h
  FastDiv div_hw, div_w;
  const float *cs_t, *cs_h, *cs_w;
};

// How a linear-attention call is split into work-groups; computed by the
// same function for the workspace query and the launch.
struct LinearPlan {
  int n_chunks;         // ceil(N / L)
  int chunk_len;        // L (min(L, N))
  int slabs_per_chunk;  // build work-groups per (b, head group, chunk); slab s takes tiles s, s+S, ...
  int apply_per_chunk;  // apply work-groups per (b, head group, chunk); part p takes steps p, p+A, ...
  int ngroups;          // head groups of 4 (one head per wave)
  size_t part_offset, prefix_offset, total_bytes;  // workspace layout (bytes)
  size_t init_offset = 0;  // causal path: copy of the incoming state
  size_t dnum_offset = 0, dden_offset = 0;  // gradient path: query-side intermediates
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

LinearPlan plan_linear(int B, int N, int H, int chunk_tokens);

struct LinearArgs {
  int B, N, H;
  const void *q, *k, *v, *g;
  void *o;
  RopeArgs rope;
  float eps;
  const float *kv_in, *ksum_in;
  float *kv_out, *ksum_out;
  void *ws;
};

hipError_t launch_linear(hla_dtype dt, const LinearArgs &a, const LinearPlan &p, hipStream_t stream);

// Chunked state sums: per chunk sum_j RoPE(relu(k_j))^T v_j and the key sum
// sum_j w_j relu(k_j) (w_j = 1 without zw), then an inclusive scan over the
// chunks (a prefix, or a suffix when reverse) starting from start_kv/start_ksum
// (zero when null). *prefix_out (in the workspace, [B*H][n_chunks][kStateFloats])
// receives the scan; final_kv/final_ksum its last value; init_copy the start.
struct StateSumArgs {
  int B, N, H;
  const void *k, *v;
  const float *zw;  // nullable, [B*H][N] fp32 (bf16 rows only)
  RopeArgs rope;
  const float *start_kv, *start_ksum;
  float *final_kv, *final_ksum;
  bool reverse;
  float *init_copy;
};

hipError_t launch_state_sums(hla_dtype dt, const StateSumArgs &s, const LinearPlan &p, void *ws, hipStream_t stream,
                             float **prefix_out);

// Gradients of the bidirectional / block-causal path (bf16). dO, dq, dk, dv,
// dg share the (B, N, H, 64) layout of q; the cache gradients are fp32.
struct LinearBwdArgs {
  int B, N, H;
  const void *q, *k, *v, *g, *dO;
  RopeArgs rope;
  float eps;
  const float *kv_in, *ksum_in;    // nullable carried state of the forward
  const float *dkv_out, *dksum_out;  // nullable gradient of the returned cache
  void *dq, *dk, *dv, *dg;
  float *dkv_in, *dksum_in;        // nullable gradient of the carried state
  void *ws;
  // bidirectional only, nullable: the forward's state over the whole sequence
  // ([B*H][D][D] and [B*H][D]); given, the first state build is skipped
  const float *kv_saved = nullptr, *ksum_saved = nullptr;
};

LinearPlan plan_linear_backward(int B, int N, int H, int chunk_tokens);
hipError_t launch_linear_backward(const LinearBwdArgs &a, const LinearPlan &p, hipStream_t stream);

// Token-causal path (bf16, band widths multiples of 8): ranges of whole
// 32-token steps as the chunks of the state build and scan.
LinearPlan plan_linear_causal(int B, int N, int H);
hipError_t launch_linear_causal(const LinearArgs &a, const LinearPlan &p, hipStream_t stream);

constexpr int kSparseQBlock = 128;  // query rows per block of the block-sparse anchor
constexpr int kSparseKBlock = 64;   // keys per named block

struct AnchorArgs {
  int B, N, H;
  const void *q, *k, *v, *g;
  void *o;
  float scale;
  void *ws;
  const int *blocks = nullptr, *counts = nullptr;  // block-sparse form when blocks != nullptr
  int max_blocks = 0;
  float *lse = nullptr;  // optional: natural-log normaliser per row, [B*H][N]
};

size_t anchor_workspace_bytes(int B, int N, int H);
size_t anchor_sparse_lds_bytes(int N);      // bitmaps of the block-sparse form
constexpr size_t kSparseLdsLimit = 16384;  // larger N is rejected (N above ~1.6M tokens)
hipError_t launch_anchor(const AnchorArgs &a, hipStream_t stream);

struct AnchorBwdArgs {
  int B, N, H;
  const void *q, *k, *v, *g, *dO;
  void *dq, *dk, *dv, *dg;
  float scale;
  void *ws;
  // saved forward (both or neither): its gated output and row normalisers; then
  // the preparation is elementwise instead of a second forward pass
  const void *o = nullptr;
  const float *lse = nullptr;
};

size_t anchor_backward_workspace_bytes(int B, int N, int H);
hipError_t launch_anchor_backward(const AnchorBwdArgs &a, hipStream_t stream);

constexpr int kMaxSources = 16;

struct RouteArgs {
  int B, T, C, S;
  const void *v[kMaxSources];
  const float *w, *phi_t;
  float eps;
  void *h;
  float *alpha;
};

hipError_t launch_route(hla_dtype dt, const RouteArgs &a, hipStream_t stream);

}  // namespace hla
