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
};

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

// Token-causal path (bf16, band widths multiples of 8): ranges of whole
// 32-token steps as the chunks of the state build and scan.
LinearPlan plan_linear_causal(int B, int N, int H);
hipError_t launch_linear_causal(const LinearArgs &a, const LinearPlan &p, hipStream_t stream);

struct AnchorArgs {
  int B, N, H;
  const void *q, *k, *v, *g;
  void *o;
  float scale;
  void *ws;
};

size_t anchor_workspace_bytes(int B, int N, int H);
hipError_t launch_anchor(const AnchorArgs &a, hipStream_t stream);

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
