// C-ABI entry points of libhla: argument validation (before any launch),
// workspace sizing, the RoPE table helper, and dispatch to the kernel files.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <climits>

#include "hla_internal.h"

using namespace hla;

static_assert(kSparseQBlock == HLA_SPARSE_Q_BLOCK && kSparseKBlock == HLA_SPARSE_K_BLOCK,
              "block sizes of the sparse anchor as declared in hla.h");

namespace {

// Enum arguments come from C, where any int value can be passed. Their bits are
// read as an int before they are validated: loading a value outside the enum's
// range as the C++ enum type is undefined behaviour.
template <class E>
int enum_bits(const E *e) {
  static_assert(sizeof(E) == sizeof(int), "the interface's enums are int-sized");
  int v;
  memcpy(&v, e, sizeof v);
  return v;
}

bool rope_valid(const hla_rope3d *r, int N, int D) {
  if (!r) return true;
  if (r->grid_t <= 0 || r->grid_h <= 0 || r->grid_w <= 0) return false;
  if ((long long)r->grid_t * r->grid_h * r->grid_w != (long long)N) return false;
  if (r->d_t < 0 || r->d_h < 0 || r->d_w < 0) return false;
  if ((r->d_t | r->d_h | r->d_w) & 1) return false;
  if (r->d_t + r->d_h + r->d_w != D) return false;
  if ((r->d_t && !r->cs_t) || (r->d_h && !r->cs_h) || (r->d_w && !r->cs_w)) return false;
  return true;
}

RopeArgs make_rope(const hla_rope3d *r) {
  RopeArgs ra;
  memset(&ra, 0, sizeof(ra));
  if (!r) return ra;
  ra.enabled = 1;
  ra.d_t = r->d_t;
  ra.d_h = r->d_h;
  ra.d_w = r->d_w;
  ra.hw = (uint32_t)r->grid_h * (uint32_t)r->grid_w;
  ra.w = (uint32_t)r->grid_w;
  ra.h = (uint32_t)r->grid_h;
  ra.div_hw = make_fastdiv(ra.hw);
  ra.div_w = make_fastdiv(ra.w);
  ra.cs_t = r->cs_t;
  ra.cs_h = r->cs_h;
  ra.cs_w = r->cs_w;
  ra.aligned = (r->d_t % 8 == 0) && (r->d_h % 8 == 0) && (r->d_w % 8 == 0) && ((uintptr_t)r->cs_t % 16 == 0) &&
               ((uintptr_t)r->cs_h % 16 == 0) && ((uintptr_t)r->cs_w % 16 == 0);
  return ra;
}

// (batch, head) pairs index the second dimension of the launch grids, whose
// limit is 65 535; token indices fit in 31 bits and element offsets of a
// [B][N][H][64] tensor in 63.
constexpr long long kMaxBatchHeads = 65535;

bool shape_ok(int B, int N, int H) {
  if (B <= 0 || N <= 0 || H <= 0) return false;
  if ((long long)B * H > kMaxBatchHeads) return false;
  return true;
}

// the first grid dimension of the linear kernels, (chunk, slab or part, head
// group), within 31 bits (only very short chunks of very long sequences reach it)
bool plan_ok(const LinearPlan &p) {
  return (long long)p.n_chunks * std::max(p.slabs_per_chunk, p.apply_per_chunk) * p.ngroups <= INT_MAX;
}

hla_status linear_common(int dtv, int B, int N, int H, int D, int chunk_tokens, const void *q, const void *k,
                         const void *v, const void *g, const hla_rope3d *rope, float eps, const float *kv_in,
                         const float *ksum_in, float *kv_out, float *ksum_out, void *o, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!q || !k || !v || !o) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H) || chunk_tokens <= 0) return HLA_ERR_INVALID_ARG;
  if ((kv_in == nullptr) != (ksum_in == nullptr)) return HLA_ERR_INVALID_ARG;
  if ((kv_out == nullptr) != (ksum_out == nullptr)) return HLA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || isinf(eps)) return HLA_ERR_INVALID_ARG;
  if (dtv != HLA_BF16 && dtv != HLA_F32) return HLA_ERR_UNSUPPORTED;
  if (D != kD) return HLA_ERR_UNSUPPORTED;
  if (!rope_valid(rope, N, D)) return HLA_ERR_INVALID_ARG;
  const LinearPlan plan = plan_linear(B, N, H, chunk_tokens);
  if (!plan_ok(plan)) return HLA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < plan.total_bytes) return HLA_ERR_WORKSPACE;
  LinearArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.o = o;
  a.rope = make_rope(rope);
  a.eps = eps;
  a.kv_in = kv_in;
  a.ksum_in = ksum_in;
  a.kv_out = kv_out;
  a.ksum_out = ksum_out;
  a.ws = ws;
  return launch_linear(static_cast<hla_dtype>(dtv), a, plan, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

hla_status linear_bwd_common(int dtv, int B, int N, int H, int D, int chunk_tokens, const void *q,
                             const void *k, const void *v, const void *g, const hla_rope3d *rope, float eps,
                             const float *kv_in, const float *ksum_in, const void *dO, const float *dkv_out,
                             const float *dksum_out, void *dq, void *dk, void *dv, void *dg, float *dkv_in,
                             float *dksum_in, void *ws, size_t ws_bytes, hipStream_t stream,
                             const float *kv_saved = nullptr, const float *ksum_saved = nullptr) {
  if (!q || !k || !v || !dO || !dq || !dk || !dv) return HLA_ERR_INVALID_ARG;
  if ((g == nullptr) != (dg == nullptr)) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H) || chunk_tokens <= 0) return HLA_ERR_INVALID_ARG;
  if ((kv_in == nullptr) != (ksum_in == nullptr)) return HLA_ERR_INVALID_ARG;
  if ((dkv_out == nullptr) != (dksum_out == nullptr)) return HLA_ERR_INVALID_ARG;
  if ((dkv_in == nullptr) != (dksum_in == nullptr)) return HLA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || isinf(eps)) return HLA_ERR_INVALID_ARG;
  if (dtv != HLA_BF16 && dtv != HLA_F32) return HLA_ERR_UNSUPPORTED;
  if (D != kD) return HLA_ERR_UNSUPPORTED;
  if (!rope_valid(rope, N, D)) return HLA_ERR_INVALID_ARG;
  if (dtv != HLA_BF16) return HLA_ERR_UNSUPPORTED;
  const LinearPlan plan = plan_linear_backward(B, N, H, chunk_tokens);
  if (!plan_ok(plan)) return HLA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < plan.total_bytes) return HLA_ERR_WORKSPACE;
  LinearBwdArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.dO = dO;
  a.rope = make_rope(rope);
  a.eps = eps;
  a.kv_in = kv_in;
  a.ksum_in = ksum_in;
  a.dkv_out = dkv_out;
  a.dksum_out = dksum_out;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dkv_in = dkv_in;
  a.dksum_in = dksum_in;
  a.ws = ws;
  a.kv_saved = kv_saved;
  a.ksum_saved = ksum_saved;
  return launch_linear_backward(a, plan, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

}  // namespace

extern "C" {

hla_status hla_rope_table_host(int len, int pos0, int d_band, double base, float *out) {
  if (!out || len <= 0 || d_band <= 0 || (d_band & 1) || !(base > 0.0)) return HLA_ERR_INVALID_ARG;
  const int half = d_band / 2;
  for (int r = 0; r < len; ++r) {
    const double p = (double)pos0 + (double)r;
    for (int k = 0; k < half; ++k) {
      const double a = p * pow(base, -2.0 * (double)k / (double)d_band);
      out[((size_t)r * half + k) * 2] = (float)cos(a);
      out[((size_t)r * half + k) * 2 + 1] = (float)sin(a);
    }
  }
  return HLA_OK;
}

size_t hla_linear_attn_workspace(int B, int N, int H, int D) {
  if (!shape_ok(B, N, H) || D != kD) return 0;
  return plan_linear(B, N, H, N).total_bytes;
}

hla_status hla_linear_attn(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k, const void *v,
                           const void *g, const hla_rope3d *rope, float eps, void *o, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
  return linear_common(enum_bits(&dt), B, N, H, D, N > 0 ? N : 1, q, k, v, g, rope, eps, nullptr, nullptr, nullptr, nullptr, o,
                       ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free bidirectional call: the workspace is the library's own
// static device array. Each GPU the library runs on holds one copy until the
// process ends; its address on a device comes from hipGetSymbolAddress with that
// device current, taken on the first call there and kept. In host code the
// array's name is only a stand-in, so kernels get the kept address.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_on[kMaxDevices];

hla_status scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HLA_ERR_HIP;
  void *p = scratch_on[dev].load(std::memory_order_acquire);
  if (!p) {
    // idempotent: concurrent first calls on one device store the same address
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HLA_ERR_HIP;
    scratch_on[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return HLA_OK;
}
}  // namespace

size_t hla_linear_attn_noalloc_max_workspace(void) { return kScratchBytes; }

hla_status hla_linear_attn_noalloc(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                   const void *v, const void *g, const hla_rope3d *rope, float eps, void *o,
                                   hipStream_t stream) {
  // the same checks as hla_linear_attn, then the size limit, before the scratch
  // address is looked up (no device call for a rejected request)
  if (!q || !k || !v || !o) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H)) return HLA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || isinf(eps)) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 && enum_bits(&dt) != HLA_F32) return HLA_ERR_UNSUPPORTED;
  if (D != kD) return HLA_ERR_UNSUPPORTED;
  if (!rope_valid(rope, N, D)) return HLA_ERR_INVALID_ARG;
  if (plan_linear(B, N, H, N).total_bytes > kScratchBytes) return HLA_ERR_WORKSPACE;
  void *ws = nullptr;
  const hla_status st = scratch_ptr(&ws);
  if (st != HLA_OK) return st;
  // every byte of the workspace that the kernels read they first write (the
  // slab partials, then the prefix records), so nothing needs clearing
  return linear_common(enum_bits(&dt), B, N, H, D, N, q, k, v, g, rope, eps, nullptr, nullptr, nullptr, nullptr, o, ws,
                       kScratchBytes, stream);
}

size_t hla_linear_attn_chunked_workspace(int B, int N, int H, int D, int chunk_tokens) {
  if (!shape_ok(B, N, H) || D != kD || chunk_tokens <= 0) return 0;
  return plan_linear(B, N, H, chunk_tokens).total_bytes;
}

hla_status hla_linear_attn_chunked(hla_dtype dt, int B, int N, int H, int D, int chunk_tokens, const void *q,
                                   const void *k, const void *v, const void *g, const hla_rope3d *rope, float eps,
                                   const float *kv_in, const float *ksum_in, float *kv_out, float *ksum_out, void *o,
                                   void *ws, size_t ws_bytes, hipStream_t stream) {
  return linear_common(enum_bits(&dt), B, N, H, D, chunk_tokens, q, k, v, g, rope, eps, kv_in, ksum_in, kv_out, ksum_out, o, ws,
                       ws_bytes, stream);
}

size_t hla_linear_attn_causal_workspace(int B, int N, int H, int D) {
  if (!shape_ok(B, N, H) || D != kD) return 0;
  return plan_linear_causal(B, N, H).total_bytes;
}

hla_status hla_linear_attn_causal(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                  const void *v, const void *g, const hla_rope3d *rope, float eps, const float *kv_in,
                                  const float *ksum_in, float *kv_out, float *ksum_out, void *o, void *ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H)) return HLA_ERR_INVALID_ARG;
  if ((kv_in == nullptr) != (ksum_in == nullptr)) return HLA_ERR_INVALID_ARG;
  if ((kv_out == nullptr) != (ksum_out == nullptr)) return HLA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || isinf(eps)) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 && enum_bits(&dt) != HLA_F32) return HLA_ERR_UNSUPPORTED;
  if (D != kD) return HLA_ERR_UNSUPPORTED;
  if (!rope_valid(rope, N, D)) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16) return HLA_ERR_UNSUPPORTED;
  LinearArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.o = o;
  a.rope = make_rope(rope);
  if (a.rope.enabled && !a.rope.aligned) return HLA_ERR_UNSUPPORTED;
  const LinearPlan plan = plan_linear_causal(B, N, H);
  if (!plan_ok(plan)) return HLA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < plan.total_bytes) return HLA_ERR_WORKSPACE;
  a.eps = eps;
  a.kv_in = kv_in;
  a.ksum_in = ksum_in;
  a.kv_out = kv_out;
  a.ksum_out = ksum_out;
  a.ws = ws;
  return launch_linear_causal(a, plan, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

size_t hla_linear_attn_backward_workspace(int B, int N, int H, int D) {
  if (!shape_ok(B, N, H) || D != kD) return 0;
  return plan_linear_backward(B, N, H, N).total_bytes;
}

hla_status hla_linear_attn_backward(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                    const void *v, const void *g, const hla_rope3d *rope, float eps, const void *dO,
                                    void *dq, void *dk, void *dv, void *dg, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
  return linear_bwd_common(enum_bits(&dt), B, N, H, D, N > 0 ? N : 1, q, k, v, g, rope, eps, nullptr, nullptr, dO, nullptr,
                           nullptr, dq, dk, dv, dg, nullptr, nullptr, ws, ws_bytes, stream);
}

hla_status hla_linear_attn_backward_saved(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                          const void *v, const void *g, const hla_rope3d *rope, float eps,
                                          const float *kv, const float *ksum, const void *dO, void *dq, void *dk,
                                          void *dv, void *dg, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!kv || !ksum) return HLA_ERR_INVALID_ARG;
  return linear_bwd_common(enum_bits(&dt), B, N, H, D, N > 0 ? N : 1, q, k, v, g, rope, eps, nullptr, nullptr, dO, nullptr,
                           nullptr, dq, dk, dv, dg, nullptr, nullptr, ws, ws_bytes, stream, kv, ksum);
}

size_t hla_linear_attn_chunked_backward_workspace(int B, int N, int H, int D, int chunk_tokens) {
  if (!shape_ok(B, N, H) || D != kD || chunk_tokens <= 0) return 0;
  return plan_linear_backward(B, N, H, chunk_tokens).total_bytes;
}

hla_status hla_linear_attn_chunked_backward(hla_dtype dt, int B, int N, int H, int D, int chunk_tokens,
                                            const void *q, const void *k, const void *v, const void *g,
                                            const hla_rope3d *rope, float eps, const float *kv_in,
                                            const float *ksum_in, const void *dO, const float *dkv_out,
                                            const float *dksum_out, void *dq, void *dk, void *dv, void *dg,
                                            float *dkv_in, float *dksum_in, void *ws, size_t ws_bytes,
                                            hipStream_t stream) {
  return linear_bwd_common(enum_bits(&dt), B, N, H, D, chunk_tokens, q, k, v, g, rope, eps, kv_in, ksum_in, dO, dkv_out,
                           dksum_out, dq, dk, dv, dg, dkv_in, dksum_in, ws, ws_bytes, stream);
}

size_t hla_softmax_anchor_workspace(int B, int N, int H, int D) {
  if (!shape_ok(B, N, H) || D != kD) return 0;
  return anchor_workspace_bytes(B, N, H);
}

hla_status hla_softmax_anchor(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k, const void *v,
                              const void *g, float scale, void *o, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H) || !isfinite(scale) || !(scale > 0.f)) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 || D != kD) return HLA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < anchor_workspace_bytes(B, N, H)) return HLA_ERR_WORKSPACE;
  AnchorArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.o = o;
  a.scale = scale;
  a.ws = ws;
  return launch_anchor(a, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

hla_status hla_softmax_anchor_lse(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                  const void *v, const void *g, float scale, void *o, float *lse, void *ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (!lse) return HLA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H) || !isfinite(scale) || !(scale > 0.f)) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 || D != kD) return HLA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < anchor_workspace_bytes(B, N, H)) return HLA_ERR_WORKSPACE;
  AnchorArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.o = o;
  a.scale = scale;
  a.ws = ws;
  a.lse = lse;
  return launch_anchor(a, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

size_t hla_softmax_anchor_backward_workspace(int B, int N, int H, int D) {
  if (!shape_ok(B, N, H) || D != kD) return 0;
  return anchor_backward_workspace_bytes(B, N, H);
}

hla_status hla_softmax_anchor_backward(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                       const void *v, const void *g, float scale, const void *dO, void *dq,
                                       void *dk, void *dv, void *dg, void *ws, size_t ws_bytes,
                                       hipStream_t stream) {
  if (!q || !k || !v || !dO || !dq || !dk || !dv) return HLA_ERR_INVALID_ARG;
  if ((g == nullptr) != (dg == nullptr)) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H) || !isfinite(scale) || !(scale > 0.f)) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 || D != kD) return HLA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < anchor_backward_workspace_bytes(B, N, H)) return HLA_ERR_WORKSPACE;
  AnchorBwdArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.dO = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.scale = scale;
  a.ws = ws;
  return launch_anchor_backward(a, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

hla_status hla_softmax_anchor_backward_saved(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                             const void *v, const void *g, float scale, const void *o,
                                             const float *lse, const void *dO, void *dq, void *dk, void *dv, void *dg,
                                             void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!o || !lse) return HLA_ERR_INVALID_ARG;
  if (!q || !k || !v || !dO || !dq || !dk || !dv) return HLA_ERR_INVALID_ARG;
  if ((g == nullptr) != (dg == nullptr)) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H) || !isfinite(scale) || !(scale > 0.f)) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 || D != kD) return HLA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < anchor_backward_workspace_bytes(B, N, H)) return HLA_ERR_WORKSPACE;
  AnchorBwdArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.dO = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.scale = scale;
  a.ws = ws;
  a.o = o;
  a.lse = lse;
  return launch_anchor_backward(a, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

hla_status hla_softmax_anchor_block_sparse(hla_dtype dt, int B, int N, int H, int D, const void *q, const void *k,
                                           const void *v, const void *g, float scale, const int *blocks,
                                           const int *counts, int max_blocks, void *o, void *ws, size_t ws_bytes,
                                           hipStream_t stream) {
  if (!q || !k || !v || !o || !blocks || !counts) return HLA_ERR_INVALID_ARG;
  if (!shape_ok(B, N, H) || !isfinite(scale) || !(scale > 0.f) || max_blocks <= 0) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 || D != kD || anchor_sparse_lds_bytes(N) > kSparseLdsLimit) return HLA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < anchor_workspace_bytes(B, N, H)) return HLA_ERR_WORKSPACE;
  AnchorArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.o = o;
  a.scale = scale;
  a.ws = ws;
  a.blocks = blocks;
  a.counts = counts;
  a.max_blocks = max_blocks;
  return launch_anchor(a, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

hla_status hla_attnres_route(hla_dtype dt, int B, int T, int C, int S, const void *const *v, const float *w,
                             const float *phi_t, float eps, void *h, float *alpha, hipStream_t stream) {
  if (!v || !w || !h) return HLA_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || C <= 0 || (C % 8) != 0 || S < 1 || S > kMaxSources) return HLA_ERR_INVALID_ARG;
  if ((long long)B * T > (1LL << 31) - 1) return HLA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || isinf(eps)) return HLA_ERR_INVALID_ARG;
  for (int i = 0; i < S; ++i)
    if (!v[i]) return HLA_ERR_INVALID_ARG;
  if (enum_bits(&dt) != HLA_BF16 && enum_bits(&dt) != HLA_F32) return HLA_ERR_UNSUPPORTED;
  if (C > 4096) return HLA_ERR_UNSUPPORTED;
  RouteArgs a;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.T = T;
  a.C = C;
  a.S = S;
  for (int i = 0; i < S; ++i) a.v[i] = v[i];
  a.w = w;
  a.phi_t = phi_t;
  a.eps = eps;
  a.h = h;
  a.alpha = alpha;
  return launch_route(dt, a, stream) == hipSuccess ? HLA_OK : HLA_ERR_HIP;
}

const char *hla_status_string(hla_status s) {
  switch (enum_bits(&s)) {
    case HLA_OK: return "HLA_OK";
    case HLA_ERR_INVALID_ARG: return "HLA_ERR_INVALID_ARG: invalid argument";
    case HLA_ERR_UNSUPPORTED: return "HLA_ERR_UNSUPPORTED: unsupported dtype or head dimension";
    case HLA_ERR_WORKSPACE: return "HLA_ERR_WORKSPACE: workspace missing or too small";
    case HLA_ERR_HIP: return "HLA_ERR_HIP: kernel launch failed";
  }
  return "HLA_ERR_UNKNOWN";
}

}  // extern "C"
