/*
 * libh3blk -- one MiniMax H3 Omni-Transformer block forward on an AMD
 * Instinct MI355X (gfx950), as six device calls.
 *
 * Sources cited below by short name:
 *   [notes]   "05 · MiniMax-H3: native audio-video joint generation"
 *             (note.shouss.top/research/video_generation/minimax_h3/)
 *   [reading] "MiniMax-H3 paper reading" (gojay.top/paper-reading/minimax-h3.html)
 *
 * A block forward is, per [notes] section 3:
 *   a   = h3_adaln_modulate(x, ATTN)          modulated norm
 *   qkv = h3_gemm_bf16(a, W_qkv)              5376 -> 3 x 7168
 *   h3_qknorm_rope3d(q, k)                    per-head RMSNorm, then 3-D RoPE
 *   o   = h3_attention_fwd(q, k, v)           full bidirectional attention
 *   y   = h3_gemm_bf16(o, W_o)                7168 -> 5376
 *   x1  = h3_gate_residual(x, y, ATTN)        x + gate * y
 *   a2  = h3_adaln_modulate(x1, FFN)
 *   gu  = h3_gemm_bf16(a2, W_gu)              5376 -> 2 x 14336  [gate | up]
 *   h   = h3_swiglu(gu)                       SiLU(gate) * up
 *   f   = h3_gemm_bf16(h, W_d)                14336 -> 5376
 *   out = h3_gate_residual(x1, f, FFN)
 *
 * The fused entry points h3_gemm_qknorm_rope (QKV projection + per-head
 * norm and RoPE of q and k), h3_gemm_gate_residual (output projection +
 * gated residual) and h3_gemm_swiglu (gate/up projection + SwiGLU) run the
 * same block in seven calls, without writing y, gu or f to memory or
 * reading q and k back.
 *
 * Conventions shared by every call:
 *   - Tensors are row-major with tokens as rows.  Every pointer argument is
 *     a device pointer unless marked "host".  The caller owns all memory;
 *     the library allocates nothing and keeps no state, so calls may be
 *     made from several host threads on different streams.
 *   - `dt` selects the storage type of activations and weights: H3_BF16
 *     (bf16 storage, fp32 accumulation and epilogue math, round to nearest
 *     even on every store) or H3_F32 (fp32 everywhere).  The modulation
 *     table, gains and lse are always fp32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work and returns; nothing synchronises.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on any error code nothing runs and no output is touched.  Device
 *     faults surface at the caller's next synchronisation.
 *   - Pointers must be 16-byte aligned; row strides must keep every row
 *     16-byte aligned (a multiple of 8 bf16 or 4 fp32 elements).
 *   - n_tok == 0 (or M == 0) is valid and enqueues nothing.
 */
#ifndef H3BLK_H
#define H3BLK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    H3_OK = 0,
    H3_ERR_ARG = 1,       /* null pointer, negative size, bad enum value      */
    H3_ERR_SEGMENTS = 2,  /* intervals unsorted, overlapping, gapped, not covering
                             [0, n_tok), len != T*H*W, mod_set out of range   */
    H3_ERR_DTYPE = 3,     /* unknown dtype                                    */
    H3_ERR_ALIGN = 4,     /* pointer or row stride breaks 16-byte alignment   */
    H3_ERR_SHAPE = 5,     /* a size the kernels do not support                */
    H3_ERR_HIP = 6        /* the HIP runtime refused a launch                 */
} h3_status;

typedef enum { H3_BF16 = 0, H3_F32 = 1 } h3_dtype;

/* Which half of a modality's six modulation vectors a call uses:
 * ATTN takes chunks (shift1, scale1, gate1) = 0,1,2; FFN takes 3,4,5. */
typedef enum { H3_BRANCH_ATTN = 0, H3_BRANCH_FFN = 1 } h3_branch;

/* One interval of the packed multimodal sequence.  [notes] 2.2: the packed
 * sequence keeps an index range for each interval (text, visual condition,
 * audio, target video).  Tokens of an interval are a (T, H, W) grid
 * flattened with t slowest and w fastest ([reading] 7.3); text and audio are
 * T = len, H = W = 1, so they sit on the time axis with h = w = 0
 * ([reading] 7.4).  Token l of the interval has 3-D position
 *   (t0 + l / (H*W), h0 + (l / W) % H, w0 + l % W).
 * mod_set is the row of the modulation table the interval uses
 * (by convention 0 text, 1 visual, 2 audio). */
typedef struct {
    int64_t start;   /* first token                                   */
    int64_t len;     /* number of tokens, must equal T*H*W            */
    int32_t mod_set; /* modulation row, 0 <= mod_set < n_sets         */
    int32_t T, H, W; /* grid, each >= 1                               */
    int32_t t0, h0, w0; /* position offsets, >= 0                     */
} h3_segment;

#define H3_MAX_SEGMENTS 64

/* Human-readable name of a status code (static string, never NULL). */
const char* h3_status_str(h3_status s);

/* Modulated RMSNorm of [notes] section 3, with the per-interval modality
 * selection of [notes] 3.1:
 *   y[i,:] = x[i,:] / sqrt(mean(x[i,:]^2) + eps) * (1 + scale[s(i)]) + shift[s(i)]
 * where s(i) is the mod_set of the interval holding token i, and shift/scale
 * are chunks (3*br, 3*br+1) of mod.
 *   x, y : [n_tok][dim] in dt, contiguous (may not alias)
 *   mod  : fp32 [n_sets][6][dim], contiguous
 *   segs : host array of n_segs intervals (1..64) covering [0, n_tok)
 * dim must be a multiple of 8 and at most 8192 (bf16) / 4096 (fp32). */
h3_status h3_adaln_modulate(const void* x, void* y, int64_t n_tok, int32_t dim,
                            const float* mod, int32_t n_sets, h3_branch br,
                            const h3_segment* segs, int32_t n_segs, float eps,
                            h3_dtype dt, void* stream);

/* C = A . W^T: the bias-free projections of the block (QKV, output, FFN
 * gate/up and down; [notes] 3.2 table).
 *   A : [M][K] with row stride lda (elements)
 *   W : [N][K] with row stride ldw (weights stored out-features major)
 *   C : [M][N] with row stride ldc; must not overlap A or W
 * bf16: K a multiple of 64; fp32: K a multiple of 32; N a multiple of 8.
 * Accumulation is fp32 in MFMA; C is rounded once. */
h3_status h3_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw,
                       void* C, int64_t ldc, int64_t M, int32_t N, int32_t K,
                       h3_dtype dt, void* stream);

/* The output projection fused with the modality-gated residual ([notes]
 * section 3: the attention and FFN outputs each re-enter the stream through
 * the modality's gate and a residual add):
 *   out[i,:] = x[i,:] + gate[s(i)] * (A . W^T)[i,:],  gate = chunk 3*br+2 of mod,
 * the same value as h3_gemm_bf16 followed by h3_gate_residual, except that
 * the product is not rounded to dt before the gate multiplies it.
 *   A : [M][K] row stride lda;  W : [N][K] row stride ldw
 *   x, out : [M][N] with row stride ldo; out may equal x (in place), must not
 *            partially overlap x, and must not overlap A or W
 *   mod    : fp32 [n_sets][6][N], n_sets >= 1
 *   segs   : host intervals covering [0, M)
 * Shape rules of h3_gemm_bf16 apply. */
h3_status h3_gemm_gate_residual(const void* A, int64_t lda, const void* W, int64_t ldw,
                                const void* x, void* out, int64_t ldo, int64_t M, int32_t N,
                                int32_t K, const float* mod, int32_t n_sets, h3_branch br,
                                const h3_segment* segs, int32_t n_segs, h3_dtype dt,
                                void* stream);

/* The FFN gate/up projection fused with SwiGLU ([notes] 3.2: the FFN is a
 * SiLU-gated linear unit of width F):
 *   H[i,f] = SiLU(a_i . Wg_f) * (a_i . Wu_f),  SiLU(z) = z / (1 + e^-z).
 *   Wgu : [2F][K] row stride ldw, the gate and up weights interleaved in
 *         32-row groups: rows 64u..64u+31 are gate rows 32u..32u+31 and rows
 *         64u+32..64u+63 the up rows 32u..32u+31 (the [gate | up] weight of
 *         h3_gemm_bf16 with its rows permuted once, when weights are loaded)
 *   A   : [M][K] row stride lda;  H : [M][F] row stride ldh, must not overlap
 *         A or Wgu
 * F a multiple of 32; other shape rules of h3_gemm_bf16 apply.  Equals
 * h3_gemm_bf16 followed by h3_swiglu except that gate and up are not rounded
 * to dt before SiLU. */
h3_status h3_gemm_swiglu(const void* A, int64_t lda, const void* Wgu, int64_t ldw,
                         void* H, int64_t ldh, int64_t M, int32_t F, int32_t K,
                         h3_dtype dt, void* stream);

/* The row permutation that turns the [gate | up] FFN weight of width F
 * ([notes] 3.2) into the interleaved Wgu that h3_gemm_swiglu and
 * h3_gemm_fp8_swiglu read; a copy, done once when weights are loaded:
 *   w_il row 64u + j = w_gu row 32u + j          (j < 32, gate)
 *   w_il row 64u + j = w_gu row F + 32u + j - 32 (j >= 32, up)
 *   w_gu : [2F][K] row stride ld_src (gate rows [0, F), up rows [F, 2F))
 *   w_il : [2F][K] row stride ld_dst, must not overlap w_gu
 * F a multiple of 32 (F = 0 is a no-op); K * sizeof(dt) a multiple of 16;
 * ld_src, ld_dst >= K with rows starting on 16-byte boundaries. */
h3_status h3_interleave_gate_up(const void* w_gu, int64_t ld_src, void* w_il, int64_t ld_dst,
                                int32_t F, int32_t K, h3_dtype dt, void* stream);

/* Per-head RMSNorm on Q and K ([notes] 3.2: applied per head, before the
 * positional encoding), then 3-D MM-RoPE ([reading] 5 and 7.4), in place:
 *   u <- gamma * u / sqrt(mean(u^2) + eps)      over each head's head_dim values
 *   then inside each head the dims are cut into [t: d_t | h: d_h | w: d_w];
 *   adjacent pairs (2j, 2j+1) of the chunk of axis a are rotated by the angle
 *   p_a * rope_base^(-2j/d_a), p_a the token's position on axis a:
 *     (u0, u1) <- (u0 cos - u1 sin, u0 sin + u1 cos).
 *   q, k    : [n_tok][heads*head_dim] views with row stride ld (elements),
 *             e.g. the q and k column blocks of the QKV output
 *   gamma_q, gamma_k : fp32 [head_dim], or NULL for a gain of 1
 *   segs    : host intervals giving every token's (t, h, w)
 * head_dim in {64, 128}; d_t, d_h, d_w even, >= 0, summing to head_dim. */
h3_status h3_qknorm_rope3d(void* q, void* k, int64_t ld, int64_t n_tok,
                           int32_t heads, int32_t head_dim,
                           const float* gamma_q, const float* gamma_k, float eps,
                           int32_t d_t, int32_t d_h, int32_t d_w, float rope_base,
                           const h3_segment* segs, int32_t n_segs,
                           h3_dtype dt, void* stream);

/* The QKV projection fused with h3_qknorm_rope3d ([notes] 3.2: q and k
 * are normed per head before the positional encoding; [reading] 5 and 7.4
 * for the 3-D RoPE):
 *   C = A . W^T, then columns [0, heads*head_dim) (q heads) and
 *   [heads*head_dim, 2*heads*head_dim) (k heads) are normed and rotated as
 *   h3_qknorm_rope3d does; later columns (v) are stored as computed.
 * The product is rounded to dt before the norm, so q and k are computed from
 * the values h3_gemm_bf16 would store.  The angles are taken in fp32
 * (revolutions reduced to [-1/2, 1/2], hardware sine and cosine), not in
 * double as h3_qknorm_rope3d does: q and k may differ from that call's by a
 * unit in the last place of dt.
 *   A : [M][K] row stride lda;  W : [N][K] row stride ldw;  C : [M][N] row
 *       stride ldc, must not overlap A or W
 *   gamma_q, gamma_k, eps, d_t, d_h, d_w, rope_base, segs : as for
 *       h3_qknorm_rope3d (segs cover [0, M))
 * heads*head_dim a multiple of 256 and 2*heads*head_dim <= N; other shape
 * rules of h3_gemm_bf16 and h3_qknorm_rope3d apply. */
h3_status h3_gemm_qknorm_rope(const void* A, int64_t lda, const void* W, int64_t ldw,
                              void* C, int64_t ldc, int64_t M, int32_t N, int32_t K,
                              int32_t heads, int32_t head_dim,
                              const float* gamma_q, const float* gamma_k, float eps,
                              int32_t d_t, int32_t d_h, int32_t d_w, float rope_base,
                              const h3_segment* segs, int32_t n_segs,
                              h3_dtype dt, void* stream);

/* Full bidirectional softmax attention per head ([notes] section 5: one
 * non-causal self-attention over all valid tokens, no mask):
 *   o[i, h] = sum_j softmax_j(scale * q[i,h] . k[j,h]) v[j,h]
 *   q, k, v : [n_tok][heads*head_dim] views sharing row stride ld_qkv
 *   o       : [n_tok][heads*head_dim] with row stride ld_o (must not alias q/k/v)
 *   lse     : optional fp32 [heads][n_tok], receives
 *             log(sum_j exp(scale * q[i,h] . k[j,h])) (natural log); NULL to skip
 * head_dim in {64, 128}; n_tok < 2^31; scale finite and > 0. */
h3_status h3_attention_fwd(const void* q, const void* k, const void* v, int64_t ld_qkv,
                           void* o, int64_t ld_o, int64_t n_tok, int32_t heads,
                           int32_t head_dim, float scale, float* lse,
                           h3_dtype dt, void* stream);

/* SwiGLU of the gated FFN ([notes] 3.2): h = SiLU(g) * u, SiLU(z) = z / (1 + e^-z).
 *   gu : [n_tok][2F] holding [gate | up]
 *   h  : [n_tok][F]
 * F a multiple of 8. */
h3_status h3_swiglu(const void* gu, void* h, int64_t n_tok, int32_t F,
                    h3_dtype dt, void* stream);

/* Modality-gated residual ([notes] section 3: "modality gate + residual"):
 *   out[i,:] = x[i,:] + gate[s(i)] * y[i,:],  gate = chunk 3*br+2 of mod.
 *   x, y, out : [n_tok][dim] contiguous; out may equal x (in place), must not
 *               partially overlap x or y.
 * dim a multiple of 8. */
h3_status h3_gate_residual(const void* x, const void* y, void* out, int64_t n_tok,
                           int32_t dim, const float* mod, int32_t n_sets, h3_branch br,
                           const h3_segment* segs, int32_t n_segs,
                           h3_dtype dt, void* stream);

/* Euler step of the flow sampler, in place ([notes] section 6: video and
 * audio follow separately configured shifted schedules and each receives an
 * Euler update from its velocity prediction; [notes] section 5: an update
 * mask keeps fixed reference latents unchanged):
 *   x[i,:] += coef[s(i)] * v[i,:],   coef[s] = sigma_next - sigma of the
 *   schedule interval s follows, 0 for the intervals the step leaves alone
 *   (text, reference images, reference video and audio).
 *   x, v : [n_tok][dim] contiguous, must not overlap
 *   coef : host fp32 array, one finite value per interval of segs
 * Rows whose coefficient is 0 are not touched.  dim a multiple of 8. */
h3_status h3_euler_update(void* x, const void* v, int64_t n_tok, int32_t dim, const float* coef,
                          const h3_segment* segs, int32_t n_segs, h3_dtype dt, void* stream);

/* Patchify of a latent for the backbone's input projection ([notes] 4.1: the
 * 24-channel visual latent is cut into 1x2x2 patches over (t, h, w), 96
 * values each; [reading] 7.3: the patch grid is then flattened with t
 * slowest and w fastest; [notes] 4.3: an audio token carries 32 latent
 * channels, i.e. a 1x1x1 patch):
 *   tokens[i, f] = latent[t*pt + dt, h*ph + dh, w*pw + dw, c],
 *   i = (t * H/ph + h) * W/pw + w,   f = ((dt*ph + dh)*pw + dw)*C + c,
 * and tokens[i, f] = 0 for pt*ph*pw*C <= f < ld, so a token row can feed
 * h3_gemm_bf16 with K = ld (zero features times zero weight columns).
 *   latent : [T][H][W][C] contiguous, channels last
 *   tokens : [(T/pt)(H/ph)(W/pw)][ld] row-major; must not overlap latent
 * T, H, W multiples of pt, ph, pw; C a multiple of 8 (bf16) or 4 (fp32);
 * ld >= pt*ph*pw*C and a multiple of 8 (bf16) or 4 (fp32); T == 0 is a
 * no-op.  Bits are copied, never rounded. */
h3_status h3_patchify(const void* latent, int32_t T, int32_t H, int32_t W, int32_t C,
                      int32_t pt, int32_t ph, int32_t pw, void* tokens, int64_t ld,
                      h3_dtype dt, void* stream);

/* Inverse of h3_patchify for the output projection ([notes] 2.3: the
 * backbone predicts the update of the video and audio latents): columns
 * f < pt*ph*pw*C of every token row go back to their latent positions;
 * columns at or past that are not read.  Same argument rules. */
h3_status h3_unpatchify(const void* tokens, int64_t ld, int32_t T, int32_t H, int32_t W,
                        int32_t C, int32_t pt, int32_t ph, int32_t pw, void* latent,
                        h3_dtype dt, void* stream);

/* FP8 variant of the projections (the pages mention only that the community
 * runs the model in FP8 ([commentary]); gfx950 contracts OCP FP8 at twice the
 * bf16 MFMA rate).  Format: OCP e4m3 -- sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, subnormals below 2^-6, largest finite 448, no
 * infinities, NaN codes 0x7F / 0xFF.
 *
 * Row-wise quantisation: for each row i of x,
 *   scales[i] = max_k |x[i,k]| / 448   (fp32 division; 1 for an all-zero row)
 *   q[i,k]    = e4m3(x[i,k] / scales[i])   (fp32 division, then the nearest
 *               e4m3 value, ties to the even code, saturating at +-448)
 *   x      : [n_rows][K] in dt (bf16 or fp32), row stride ldx
 *   q      : [n_rows][K] bytes, row stride ldq (a multiple of 16)
 *   scales : fp32 [n_rows]
 * K a multiple of 16.  Used for activations (per token) and for weights
 * stored [out][in] (per output channel). */
h3_status h3_quantize_fp8(const void* x, int64_t ldx, int64_t n_rows, int32_t K,
                          void* q, int64_t ldq, float* scales, h3_dtype dt, void* stream);

/* C = diag(a_scale) . (A . W^T) . diag(w_scale) with A [M][K] and W [N][K]
 * in e4m3 (row strides lda, ldw in bytes, multiples of 16), exact products
 * accumulated in fp32 by MFMA, scaled in fp32 and stored once in out_dt.
 *   a_scale : fp32 [M], w_scale : fp32 [N] (as written by h3_quantize_fp8)
 *   C       : [M][N] in out_dt, row stride ldc; must not overlap the inputs
 * K a multiple of 128, N a multiple of 8. */
h3_status h3_gemm_fp8(const void* A, int64_t lda, const float* a_scale, const void* W,
                      int64_t ldw, const float* w_scale, void* C, int64_t ldc, int64_t M,
                      int32_t N, int32_t K, h3_dtype out_dt, void* stream);

/* The fp8 forms of the fused projections (h3_gemm_gate_residual and
 * h3_gemm_swiglu, [notes] section 3 and 3.2) for the FP8 variant of the
 * block ([commentary]): the product of h3_gemm_fp8 (e4m3 codes with their
 * row scales, fp32 sums, scaled in fp32) enters the same epilogue,
 *   out[i,:] = x[i,:] + gate[s(i)] * (diag(a_scale) A W^T diag(w_scale))[i,:]
 *   H[i,f]   = SiLU(g_if) * u_if with g, u the scaled gate and up products,
 * bf16 x, out and H.  Wgu and w_scale of the SwiGLU form are the gate/up
 * codes and their scales with rows in h3_gemm_swiglu's 32-row interleave.
 * Argument rules of h3_gemm_fp8 (K a multiple of 128), h3_gemm_gate_residual
 * and h3_gemm_swiglu apply; x must not overlap A. */
h3_status h3_gemm_fp8_gate_residual(const void* A, int64_t lda, const float* a_scale, const void* W,
                                    int64_t ldw, const float* w_scale, const void* x, void* out,
                                    int64_t ldo, int64_t M, int32_t N, int32_t K, const float* mod,
                                    int32_t n_sets, h3_branch br, const h3_segment* segs,
                                    int32_t n_segs, void* stream);
h3_status h3_gemm_fp8_swiglu(const void* A, int64_t lda, const float* a_scale, const void* Wgu,
                             int64_t ldw, const float* w_scale, void* H, int64_t ldh, int64_t M,
                             int32_t F, int32_t K, void* stream);

/* The FP8 QKV projection fused with the per-head norm and RoPE of q and k
 * (h3_gemm_qknorm_rope on e4m3 operands): C = diag(a_scale) (A . W^T)
 * diag(w_scale) as h3_gemm_fp8 computes it, rounded to bf16, then q and k
 * normed and rotated as h3_gemm_qknorm_rope does.  C is bf16.  Shape and
 * layout rules of h3_gemm_fp8 and the head rules of h3_gemm_qknorm_rope
 * apply. */
h3_status h3_gemm_fp8_qknorm_rope(const void* A, int64_t lda, const float* a_scale, const void* W,
                                  int64_t ldw, const float* w_scale, void* C, int64_t ldc, int64_t M,
                                  int32_t N, int32_t K, int32_t heads, int32_t head_dim,
                                  const float* gamma_q, const float* gamma_k, float eps,
                                  int32_t d_t, int32_t d_h, int32_t d_w, float rope_base,
                                  const h3_segment* segs, int32_t n_segs, void* stream);

/* FP8 attention operands (same e4m3 format and rounding as h3_quantize_fp8;
 * [notes] section 5 defines the attention, [commentary] the FP8 practice):
 *   sq[h, i] = max_d |q[i, h, d]| / 448            (one scale per token and head)
 *   sk[h]    = max_{i,d} |k[i, h, d]| / 448,  sv[h] likewise for v (per head)
 *   q8[i, h*128 + d] = e4m3(q[i,h,d] / sq[h,i]),  k8 likewise with sk[h]
 *   vt[(h*128 + d) * n_pad + 64 t + p] = e4m3(v[64 t + key(p), h, d] / sv[h])
 *     with key(p) = 32 (b / 16) + 8 ((b % 16) / 4) + 4 g + b % 4 for
 *     p = 32 g + b (v transposed, each 64-key group permuted into the order
 *     h3_attention_fp8 packs its weights in); a position whose key is
 *     n_tok or later holds 0.
 * A scale is 1 where the maximum is 0.
 *   q, k, v : bf16 [n_tok][heads*128] views with row stride ld
 *   q8, k8  : [n_tok][heads*128] bytes;  vt : [heads][128][n_pad] bytes
 *   sq      : fp32 [heads][n_tok];  sk, sv : fp32 [heads]
 * head_dim 128 (else H3_ERR_SHAPE); n_pad a multiple of 64 and >= n_tok
 * (else H3_ERR_ARG); heads <= 65535, n_tok * heads < 2^31 and
 * n_pad * 128 < 2^32 (else H3_ERR_SHAPE); outputs must not overlap each
 * other or the inputs (H3_ERR_ARG).  Enqueues nine kernels; sk and sv hold
 * maxima until the last two turn them into scales. */
h3_status h3_quantize_qkv_fp8(const void* q, const void* k, const void* v, int64_t ld,
                              int64_t n_tok, int32_t heads, int32_t head_dim, void* q8,
                              void* k8, void* vt, int64_t n_pad, float* sq, float* sk,
                              float* sv, h3_dtype dt, void* stream);

/* Full bidirectional attention on FP8 operands (the quantised form of
 * h3_attention_fwd, [notes] section 5): with q^, k^, v^ the dequantised
 * values (codes times their scales),
 *   o[i, h] = sum_j softmax_j(scale * q^[i,h] . k^[j,h]) v^[j,h],
 * where q^.k^ and P.v^ are formed on e4m3 MFMA with fp32 sums, and the
 * softmax weights themselves are rounded to e4m3 (scaled so that the largest
 * is near 16, so weights down to about 2^-13 of it are kept); the row sums
 * use exactly those rounded weights.  o : bf16 [n_tok][heads*128], row
 * stride ld_o, must not overlap the operands (H3_ERR_ARG).  Operands and
 * sizes as h3_quantize_qkv_fp8 writes them, with the same limits; scale
 * finite and > 0 (else H3_ERR_ARG). */
h3_status h3_attention_fp8(const void* q8, const void* k8, const void* vt, int64_t n_pad,
                           const float* sq, const float* sk, const float* sv, void* o,
                           int64_t ld_o, int64_t n_tok, int32_t heads, int32_t head_dim,
                           float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* H3BLK_H */
