/*
 * libhla -- token-mixing path of the SANA-Video / SANA-Video 2.0 hybrid
 * attention layer, for AMD Instinct MI355X (gfx950).
 *
 * Four operations, each a set of hand-written HIP kernels:
 *
 *   hla_linear_attn          bidirectional ReLU-kernel linear attention with 3D
 *                            RoPE after the ReLU, a RoPE-free denominator and an
 *                            optional sigmoid output gate.
 *   hla_linear_attn_chunked  block-causal variant that carries the cumulative
 *                            D x D state and key sum across chunks.
 *   hla_linear_attn_causal   token-causal variant: every token sees itself and
 *                            the tokens before it, plus a carried state.
 *   hla_linear_attn_backward, hla_linear_attn_chunked_backward
 *                            gradients of the bidirectional and block-causal
 *                            variants (inputs, gate and carried state);
 *                            hla_linear_attn_backward_saved takes the
 *                            forward's state instead of rebuilding it.
 *   hla_softmax_anchor       gated non-causal softmax attention (the periodic
 *                            full-rank anchor layer); hla_softmax_anchor_lse
 *                            also writes each row's normaliser.
 *   hla_softmax_anchor_block_sparse
 *                            the anchor restricted to caller-given key blocks.
 *   hla_softmax_anchor_backward, hla_softmax_anchor_backward_saved
 *                            gradients of the anchor, recomputing the forward
 *                            or from its saved output and normalisers.
 *   hla_attnres_route        block attention-residual (AttnRes) depth router.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Ownership: the caller allocates and owns every buffer. Tensor pointers are
 *   DEVICE pointers to contiguous memory in the layouts stated per call; the
 *   hla_rope3d struct and the array of source pointers of the router are HOST
 *   memory that is read during the call only. The library never allocates,
 *   frees or synchronises, and keeps no pointer after it returns.
 * - Asynchrony: every call enqueues its kernels on `stream` (NULL = the
 *   default stream) and returns; outputs are valid once the stream has
 *   executed them. A call enqueues kernels only (no memset or copy), so it can
 *   be captured in a HIP graph and replayed; workspace contents on entry never
 *   matter.
 * - Errors: arguments are validated before anything is launched. A rejected
 *   call returns HLA_ERR_INVALID_ARG, HLA_ERR_UNSUPPORTED or HLA_ERR_WORKSPACE
 *   and has no side effect. A failed launch returns HLA_ERR_HIP. No C++
 *   exception crosses this interface. Apart from hla_linear_attn_noalloc's
 *   static device array (see there) and caches of read-only device facts, the
 *   library holds no mutable global state, so calls from several host threads
 *   are safe.
 * - Aliasing: outputs must not overlap inputs, except kv_out == kv_in and
 *   ksum_out == ksum_in in hla_linear_attn_chunked and hla_linear_attn_causal,
 *   and dkv_in == dkv_out, dksum_in == dksum_out in
 *   hla_linear_attn_chunked_backward.
 * - Sizes: B, N, H >= 1 and B * H <= 65535 (a (batch, head) pair indexes a
 *   launch grid dimension); larger products are HLA_ERR_INVALID_ARG. The
 *   linear calls also reject a plan whose work-groups per batch element
 *   (chunks x slabs x head groups) exceed 2^31 - 1, reachable only with very
 *   short chunks of very long sequences.
 * - Numbers: HLA_BF16 tensors hold bfloat16 values, HLA_F32 tensors float.
 *   States, key sums, router queries and RoPE tables are always float.
 *   Arithmetic is float32 throughout; bf16 outputs are rounded to nearest
 *   even. Only head dimension D = 64 is built.
 * - Determinism: no floating-point atomics are used; a call repeated on the
 *   same inputs returns bitwise identical outputs.
 * - Non-finite inputs (a reading; the pages say nothing of them): nothing is
 *   checked or clamped, and NaN propagates. relu keeps NaN (relu(-Inf) = 0,
 *   relu(+Inf) = +Inf) and every sum that takes a NaN or Inf term carries it.
 *   A NaN in q_i reaches o_i only; in k_j every output row of that head (in
 *   the block-causal forms: the rows of k_j's chunk and of later chunks); in
 *   v_j[e] column e of the same rows; in g_i[e] that one element; in a router
 *   source at token t, h_t and alpha_t only. An Inf makes the outputs that
 *   take it non-finite in the same pattern. Outputs that do not depend on the
 *   value are unaffected. Gradients of non-finite inputs are unspecified.
 */
#ifndef HLA_H
#define HLA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HLA_OK = 0,
  HLA_ERR_INVALID_ARG = 1, /* null required pointer, bad size, inconsistent shapes */
  HLA_ERR_UNSUPPORTED = 2, /* a valid request the library does not implement (D != 64, ...) */
  HLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace query */
  HLA_ERR_HIP = 4          /* a kernel launch failed (hipGetLastError) */
} hla_status;

typedef enum { HLA_BF16 = 0, HLA_F32 = 1 } hla_dtype;

/*
 * 3D rotary position embedding (SANA-Video notes, section 3.2 and Figure 2(c):
 * RoPE is applied to the ReLU features of Q and K). The pages do not define the
 * rotation; this library uses the following reading:
 *   token n of a call sits at frame t, row y, column x of a grid_t x grid_h x
 *   grid_w latent grid, n = (t * grid_h + y) * grid_w + x (t-major);
 *   dims [0, d_t) rotate with t, [d_t, d_t + d_h) with y, the rest with x;
 *   inside a band, adjacent pairs (2k, 2k+1) rotate by the angle a_k of the
 *   token's coordinate: (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
 * The tables hold (cos a, sin a) as float pairs, row r for coordinate r:
 *   cs_t: [grid_t][d_t/2][2], cs_h: [grid_h][d_h/2][2], cs_w: [grid_w][d_w/2][2].
 * hla_rope_table_host fills one table; a streaming caller whose first frame is
 * global frame t0 builds cs_t with pos0 = t0.
 */
typedef struct {
  int grid_t, grid_h, grid_w; /* grid_t * grid_h * grid_w must equal N */
  int d_t, d_h, d_w;          /* even, d_t + d_h + d_w == D */
  const float *cs_t;          /* device */
  const float *cs_h;          /* device */
  const float *cs_w;          /* device */
} hla_rope3d;

/*
 * Host helper: out[r][k] = (cos a, sin a), a = (pos0 + r) * base^(-2k / d_band),
 * for r in [0, len) and k in [0, d_band/2). Angles are formed in double and
 * rounded to float. `out` is HOST memory of len * d_band floats.
 * Errors: INVALID_ARG if out is NULL, len <= 0, d_band <= 0 or odd, base <= 0.
 */
hla_status hla_rope_table_host(int len, int pos0, int d_band, double base, float *out);

/*
 * Bidirectional ReLU-kernel linear attention with RoPE after the ReLU
 * (SANA-Video notes, section 3.2: output equation and pseudocode), with an
 * optional output gate (SANA-Video 2.0 abstract: the linear layers are gated;
 * form read as sigmoid(G) times the normalised output). Per batch b, head h:
 *   a_i = RoPE_i(relu(q_i)),  c_j = RoPE_j(relu(k_j))
 *   KV  = sum_j c_j^T v_j (D x D),   z = sum_j relu(k_j)  (no RoPE)
 *   o_i = (a_i KV) / (relu(q_i) . z + eps),  then o_i *= sigmoid(g_i) if g
 * q, k, v, g, o: [B][N][H][D] of dtype `dt` (token-major, head, then dim).
 * g may be NULL (no gate); rope may be NULL (no rotation).
 * ws: device workspace of at least hla_linear_attn_workspace(B, N, H, D) bytes
 *     (its contents on entry do not matter and are overwritten). The split of
 *     the sequence into work-group slabs, and so the workspace size, is planned
 *     for 512 resident work-groups (two per CU on the 256 CUs of an MI355X), a
 *     fixed figure so that the size query needs no device; on another part the
 *     results are the same and only the schedule differs.
 * Errors: INVALID_ARG for null q/k/v/o, B, N or H <= 0, bad rope fields or a
 * rope grid whose product differs from N; UNSUPPORTED for D != 64 or an
 * unknown dtype; WORKSPACE if ws is NULL or ws_bytes is too small.
 */
size_t hla_linear_attn_workspace(int B, int N, int H, int D);
hla_status hla_linear_attn(hla_dtype dt, int B, int N, int H, int D,
                           const void *q, const void *k, const void *v, const void *g,
                           const hla_rope3d *rope, float eps,
                           void *o, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_linear_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is the library's own static
 * device array of hla_linear_attn_noalloc_max_workspace() bytes (64 MiB), one
 * per GPU, held until the process ends; the call allocates nothing and
 * returns results bitwise equal to hla_linear_attn's. Every call on one GPU
 * uses that GPU's array, so calls that overlap on one GPU (several streams or
 * host threads) race; serialise them. The caller passes inputs and outputs as
 * for hla_linear_attn; the current device must be the one that owns them.
 * Errors: as hla_linear_attn; WORKSPACE when the call needs more than the
 * static array (hla_linear_attn_workspace(B, N, H, D) above the maximum), HIP
 * when the array's address cannot be obtained on the current device.
 */
size_t hla_linear_attn_noalloc_max_workspace(void);
hla_status hla_linear_attn_noalloc(hla_dtype dt, int B, int N, int H, int D,
                                   const void *q, const void *k, const void *v, const void *g,
                                   const hla_rope3d *rope, float eps, void *o, hipStream_t stream);

/*
 * Block-causal linear attention with a constant-memory carried state
 * (SANA-Video notes, section 3.4: causal equation with the own term included,
 * the cache of cumulative states and key sums, and Algorithm 1's update).
 * Chunk c holds tokens [c L, min((c+1) L, N)), L = chunk_tokens; the last chunk
 * may be shorter. With P_c = KV_in + sum of c_j^T v_j over chunks 0..c and
 * Z_c = z_in + sum of relu(k_j) over chunks 0..c, token i of chunk c gets
 *   o_i = (a_i P_c) / (relu(q_i) . Z_c + eps),  then the optional gate.
 * kv_in [B][H][D][D] and ksum_in [B][H][D] (float, device) may both be NULL
 * for a zero state; kv_out and ksum_out receive P_last and Z_last and may both
 * be NULL (the call then does not commit its state). kv_out may equal kv_in and
 * ksum_out may equal ksum_in. Other arguments as hla_linear_attn; the rope
 * grid covers the N tokens of this call.
 * Errors: as hla_linear_attn, plus INVALID_ARG for chunk_tokens <= 0 or only one
 * of each in/out pair given.
 */
size_t hla_linear_attn_chunked_workspace(int B, int N, int H, int D, int chunk_tokens);
hla_status hla_linear_attn_chunked(hla_dtype dt, int B, int N, int H, int D, int chunk_tokens,
                                   const void *q, const void *k, const void *v, const void *g,
                                   const hla_rope3d *rope, float eps,
                                   const float *kv_in, const float *ksum_in,
                                   float *kv_out, float *ksum_out,
                                   void *o, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Token-causal linear attention (SANA-Video notes, section 3.4, the causal
 * equation with the own term included): token i gets
 *   o_i = (a_i KV_i) / (relu(q_i) . z_i + eps),  then the optional gate,
 * with KV_i = KV_in + sum_{j <= i} c_j^T v_j and z_i = z_in + sum_{j <= i}
 * relu(k_j) (a, c as in hla_linear_attn). It equals hla_linear_attn_chunked
 * with chunk_tokens = 1, computed in 32-token steps on the matrix cores.
 * kv_in/ksum_in (may both be NULL: zero state) and kv_out/ksum_out (may both
 * be NULL: no commit; receive the state after the last token; may alias the
 * inputs) as in hla_linear_attn_chunked. Other arguments as hla_linear_attn.
 * Errors: as hla_linear_attn_chunked, plus UNSUPPORTED for dt != HLA_BF16 and
 * for a rope whose band widths are not multiples of 8 or whose tables are not
 * 16-byte aligned.
 */
size_t hla_linear_attn_causal_workspace(int B, int N, int H, int D);
hla_status hla_linear_attn_causal(hla_dtype dt, int B, int N, int H, int D,
                                  const void *q, const void *k, const void *v, const void *g,
                                  const hla_rope3d *rope, float eps,
                                  const float *kv_in, const float *ksum_in,
                                  float *kv_out, float *ksum_out,
                                  void *o, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gradients of hla_linear_attn (bf16). Given the forward's inputs and dO, the
 * gradient of a scalar loss with respect to o, it writes dq, dk, dv and dg (the
 * latter when g is given). With s = sigmoid(g) (1 without a gate),
 * y_i = num_i / den_i, den_i = relu(q_i) . z + eps:
 *   dg_i = dO_i y_i s_i (1 - s_i),  dY_i = dO_i s_i
 *   dnum_i = dY_i / den_i,  dden_i = -(dY_i . y_i) / den_i
 *   dq_i = (R_i^T (KV dnum_i) + dden_i z) [q_i > 0]
 *   G = sum_i a_i^T dnum_i,  Gz = sum_i dden_i relu(q_i)
 *   dk_j = (R_j^T (G v_j) + Gz) [k_j > 0],  dv_j = G^T c_j
 * (R_i the rotation of token i, a_i and c_i as in hla_linear_attn; the ReLU's
 * derivative is taken as 0 at 0). The forward is recomputed, nothing of it is
 * kept. q, k, v, g, dO, dq, dk, dv, dg: [B][N][H][D] bf16 (dt must be HLA_BF16);
 * dg must be given exactly when g is. Products run on bf16 matrix cores with
 * float accumulation, the D x D matrices split into bf16 high and low parts;
 * dnum is rounded to bf16 for the sums over queries.
 * ws: at least hla_linear_attn_backward_workspace(B, N, H, D) bytes.
 * Errors: as hla_linear_attn, plus INVALID_ARG for null dO/dq/dk/dv or a gate
 * given without dg (or dg without g), UNSUPPORTED for dt != HLA_BF16.
 */
size_t hla_linear_attn_backward_workspace(int B, int N, int H, int D);
hla_status hla_linear_attn_backward(hla_dtype dt, int B, int N, int H, int D,
                                    const void *q, const void *k, const void *v, const void *g,
                                    const hla_rope3d *rope, float eps, const void *dO,
                                    void *dq, void *dk, void *dv, void *dg,
                                    void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_linear_attn_backward given the forward's state instead of rebuilding it:
 * kv[(b*H + h)][d][e] = sum_j c_j[d] v_j[e] and ksum[(b*H + h)][d] = sum_j relu(k_j)[d]
 * over the whole sequence (c_j the rotated relu(k_j), as in hla_linear_attn), float,
 * [B][H][D][D] and [B][H][D], as hla_linear_attn_chunked writes them to kv_out and
 * ksum_out for chunk_tokens = N and no carried state (that call's o equals
 * hla_linear_attn's bit for bit). The first state build of the backward is then
 * skipped; with that state the results are bitwise those of
 * hla_linear_attn_backward. Arguments and workspace otherwise as
 * hla_linear_attn_backward.
 * Errors: as hla_linear_attn_backward, plus INVALID_ARG for a null kv or ksum.
 */
hla_status hla_linear_attn_backward_saved(hla_dtype dt, int B, int N, int H, int D,
                                          const void *q, const void *k, const void *v, const void *g,
                                          const hla_rope3d *rope, float eps,
                                          const float *kv, const float *ksum, const void *dO,
                                          void *dq, void *dk, void *dv, void *dg,
                                          void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gradients of hla_linear_attn_chunked (bf16), including the carried and the
 * returned cache. The loss is taken as L(o) + sum(dkv_out * kv_out) +
 * sum(dksum_out * ksum_out): dO is dL/do and dkv_out [B][H][D][D], dksum_out
 * [B][H][D] (float; may both be NULL for zero) are the gradients reaching the
 * returned cache. Chunk c's queries use the cache P_c, Z_c of the forward and
 * give dq as in hla_linear_attn_backward; a key of chunk c sees the suffix sums
 *   G_c = dkv_out + sum over chunks c' >= c of sum_{i in c'} a_i^T dnum_i
 *   Gz_c = dksum_out + sum over chunks c' >= c of sum_{i in c'} dden_i relu(q_i)
 * and dkv_in, dksum_in (may both be NULL) receive G_0 and Gz_0, the gradient of
 * the carried state. kv_in, ksum_in are the forward's carried state (may both
 * be NULL for zero). dkv_in may equal dkv_out and dksum_in may equal dksum_out.
 * Other arguments as hla_linear_attn_backward and hla_linear_attn_chunked.
 * ws: at least hla_linear_attn_chunked_backward_workspace(B, N, H, D,
 * chunk_tokens) bytes.
 * Errors: as hla_linear_attn_backward, plus INVALID_ARG for chunk_tokens <= 0
 * or only one of each state pair given.
 */
size_t hla_linear_attn_chunked_backward_workspace(int B, int N, int H, int D, int chunk_tokens);
hla_status hla_linear_attn_chunked_backward(hla_dtype dt, int B, int N, int H, int D, int chunk_tokens,
                                            const void *q, const void *k, const void *v, const void *g,
                                            const hla_rope3d *rope, float eps,
                                            const float *kv_in, const float *ksum_in, const void *dO,
                                            const float *dkv_out, const float *dksum_out,
                                            void *dq, void *dk, void *dv, void *dg,
                                            float *dkv_in, float *dksum_in,
                                            void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gated non-causal softmax attention, the anchor layer of the 3:1 hybrid
 * (SANA-Video 2.0 abstract and summary; textbook scaled dot-product form):
 *   o_i = sigmoid(g_i) * sum_j softmax_j(scale * q_i . k_j) v_j
 * q, k, v, g, o: [B][N][H][D] bf16 (dt must be HLA_BF16); g may be NULL.
 * The P.V product runs on bf16 matrix cores (weights rounded to bf16, float
 * accumulation). The scores take one of two forms, per group of 512 query rows
 * of one head:
 *   - where every row's bound b_i = scale log2(e) |q_i| max_j |k_j| (by
 *     Cauchy-Schwarz no |scale log2(e) q_i . k_j| exceeds it) is at most 48,
 *     scale log2(e) |q_i| <= 2^10, max_j |k_j| <= 2^10 and no finite |v| exceeds
 *     2^40: fp16 matrix-core products of K and of q pre-scaled by
 *     scale log2(e) (rounded to fp16, 11 significant bits), the weights 2 to
 *     the power of those products, with no reference subtracted (they stay
 *     within 2^(+-48));
 *   - otherwise bf16 products and a float online softmax whose running row
 *     maximum is refreshed lazily.
 * Both give the exact result up to rounding of the order of bf16's.
 * ws: device workspace of at least hla_softmax_anchor_workspace(B, N, H, D)
 *     bytes; it receives V transposed per head, K in fp16, and the largest
 *     squared K norm and largest finite |v| of every 64-key block (contents on
 *     entry ignored).
 * Errors: INVALID_ARG for null q/k/v/o, B, N or H <= 0, scale not finite and
 * positive; UNSUPPORTED for D != 64 or dt != HLA_BF16; WORKSPACE if ws is NULL
 * or ws_bytes is too small.
 */
size_t hla_softmax_anchor_workspace(int B, int N, int H, int D);
hla_status hla_softmax_anchor(hla_dtype dt, int B, int N, int H, int D,
                              const void *q, const void *k, const void *v, const void *g,
                              float scale, void *o, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_softmax_anchor that also writes each row's normaliser (the log-sum-exp
 * that FlashAttention-style training keeps for the backward pass):
 *   lse[(b*H + h)*N + n] = log sum_j exp(scale * q_n . k_j)   (natural log)
 * for batch b, head h, query n. lse: device float [B][H][N], caller-owned. It is
 * the log of the forward's own normaliser (the sum of its bf16-rounded weights
 * relative to its running max), so exp(scale q.k - lse) are exactly the weights
 * the forward used, up to float rounding. Same workspace as hla_softmax_anchor.
 * Errors: as hla_softmax_anchor, plus INVALID_ARG for a null lse.
 */
hla_status hla_softmax_anchor_lse(hla_dtype dt, int B, int N, int H, int D,
                                  const void *q, const void *k, const void *v, const void *g,
                                  float scale, void *o, float *lse, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * Gradients of hla_softmax_anchor (bf16). Given the forward's inputs and dO, the
 * gradient of a scalar loss with respect to o, it writes dq, dk, dv and dg (the
 * latter when g is given). With p_ij the softmax weights, y_i = sum_j p_ij v_j
 * the ungated output and s = sigmoid(g) (1 without a gate):
 *   dg_i = dO_i y_i s_i (1 - s_i),  dY_i = dO_i s_i,  dP_ij = dY_i . v_j
 *   Delta_i = dY_i . y_i,  dL_ij = p_ij (dP_ij - Delta_i)
 *   dq_i = scale sum_j dL_ij k_j,  dk_j = scale sum_i dL_ij q_i,  dv_j = sum_i p_ij dY_i
 * The forward is recomputed (a pass that also yields each row's normaliser,
 * with the score forms of hla_softmax_anchor), nothing of it is kept. q, k, v,
 * g, dO, dq, dk, dv, dg: [B][N][H][D] bf16; dg must be given exactly when g
 * is. The gradient products run on bf16 matrix cores with float accumulation;
 * p, dL and dY are rounded to bf16 as product operands.
 * No atomics: repeated calls are bitwise identical.
 * ws: at least hla_softmax_anchor_backward_workspace(B, N, H, D) bytes.
 * Errors: as hla_softmax_anchor, plus INVALID_ARG for null dO/dq/dk/dv or a
 * gate given without dg (or dg without g).
 */
size_t hla_softmax_anchor_backward_workspace(int B, int N, int H, int D);
hla_status hla_softmax_anchor_backward(hla_dtype dt, int B, int N, int H, int D,
                                       const void *q, const void *k, const void *v, const void *g,
                                       float scale, const void *dO,
                                       void *dq, void *dk, void *dv, void *dg,
                                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_softmax_anchor_backward from a saved forward: o and lse as written by
 * hla_softmax_anchor_lse for the same q, k, v, g and scale. The second forward
 * pass is replaced by an elementwise preparation, with s = sigmoid(g):
 *   dY = dO s,  dg = dO o (1 - s),  Delta = dO . o   (= dY . y),
 * and the weights are p_ij = exp(scale q_i . k_j - lse_i). The results match
 * hla_softmax_anchor_backward up to rounding (Delta is formed from o instead of
 * the bf16 dY and the float y, and dg from the bf16 o). o: [B][N][H][D] bf16,
 * lse: float [B][H][N]; the other arguments and the workspace as
 * hla_softmax_anchor_backward. Repeated calls are bitwise identical.
 * Errors: as hla_softmax_anchor_backward, plus INVALID_ARG for a null o or lse.
 */
hla_status hla_softmax_anchor_backward_saved(hla_dtype dt, int B, int N, int H, int D,
                                             const void *q, const void *k, const void *v, const void *g,
                                             float scale, const void *o, const float *lse, const void *dO,
                                             void *dq, void *dk, void *dv, void *dg,
                                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Block-sparse form of hla_softmax_anchor. The pages name a sparse anchor
 * (SANA-Video 2.0 summary, efficiency paragraph) without its pattern, so the
 * pattern is an input. Query rows form blocks of HLA_SPARSE_Q_BLOCK = 128
 * (block r: rows [128 r, min(128 (r+1), N))), keys blocks of
 * HLA_SPARSE_K_BLOCK = 64. For each (b, h, r), with nqb = ceil(N / 128):
 *   counts[(b H + h) nqb + r]                    number of entries used
 *   blocks[((b H + h) nqb + r) max_blocks + m]   key block named by entry m
 * and every row of block r attends to the keys of the named blocks only:
 *   o_i = sigmoid(g_i) * sum_{j in K_r} softmax_{j in K_r}(scale q_i . k_j) v_j,
 * o_i = 0 when K_r is empty. blocks and counts are int32 DEVICE arrays. Counts
 * are clamped to [0, max_blocks]; entries outside [0, ceil(N / 64)) name
 * nothing; the named blocks form a set (order and repeats do not matter; they
 * are visited in ascending order). Other arguments, workspace and numerics as
 * hla_softmax_anchor (same workspace size).
 * Errors: as hla_softmax_anchor, plus INVALID_ARG for null blocks/counts or
 * max_blocks <= 0, UNSUPPORTED for N above 1 677 312 (the key-block bitmaps
 * must fit in 16 KB of LDS).
 */
#define HLA_SPARSE_Q_BLOCK 128
#define HLA_SPARSE_K_BLOCK 64
hla_status hla_softmax_anchor_block_sparse(hla_dtype dt, int B, int N, int H, int D,
                                           const void *q, const void *k, const void *v, const void *g,
                                           float scale, const int *blocks, const int *counts, int max_blocks,
                                           void *o, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Block attention-residual router (SANA-Video 2.0 summary, method section,
 * router equation). For each of the B*T tokens, with u_b = w + phi_t[b]:
 *   l_i = u_b . RMSNorm(v_i),  RMSNorm(v) = v / sqrt(mean_c v_c^2 + eps)
 *   alpha = softmax_i(l),      h = sum_i alpha_i v_i   (raw sources)
 * v: HOST array of S device pointers, each [B][T][C] of dtype dt.
 * w: [C] float; phi_t: [B][C] float or NULL (router without timestep).
 * h: [B][T][C] of dtype dt; alpha: [B][T][S] float or NULL.
 * Errors: INVALID_ARG for null v, v[i], w or h, B, T or C <= 0, C % 8 != 0,
 * S outside [1, 16]; UNSUPPORTED for C > 4096 or an unknown dtype.
 */
hla_status hla_attnres_route(hla_dtype dt, int B, int T, int C, int S,
                             const void *const *v, const float *w, const float *phi_t, float eps,
                             void *h, float *alpha, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char *hla_status_string(hla_status s);

#ifdef __cplusplus
}
#endif

#endif /* HLA_H */
