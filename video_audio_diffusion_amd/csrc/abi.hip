// The C ABI of libh3blk: argument validation, then one launch per call.
// Everything is checked on the host before anything is enqueued, so an
// error code always means that no work ran and no output was touched.
#include <math.h>
#include <string.h>

#include "../../include/h3blk.h"
#include "launch.h"

using namespace h3;

namespace {

constexpr int64_t kMaxTok = (int64_t)1 << 31;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool valid_dt(h3_dtype dt) { return dt == H3_BF16 || dt == H3_F32; }
inline int esize(h3_dtype dt) { return dt == H3_BF16 ? 2 : 4; }
inline bool valid_branch(h3_branch br) { return br == H3_BRANCH_ATTN || br == H3_BRANCH_FFN; }

// Byte range [lo, hi) spanned by a strided [rows][cols] view.
struct Span {
    uintptr_t lo, hi;
};
inline Span span(const void* p, int64_t rows, int64_t cols, int64_t ld, int es) {
    const uintptr_t lo = (uintptr_t)p;
    if (rows <= 0 || cols <= 0) return {lo, lo};
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * es)};
}
inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Intervals must be sorted, contiguous, non-empty, cover [0, n_tok) and
// have len == T*H*W; mod_set must index the modulation table when one is
// used (n_sets > 0).
h3_status build_segs(const h3_segment* segs, int32_t n_segs, int64_t n_tok, int32_t n_sets, SegTable* tab) {
    if (n_segs < 0 || n_segs > H3_MAX_SEGMENTS) return H3_ERR_SEGMENTS;
    if (n_segs > 0 && !segs) return H3_ERR_ARG;
    memset(tab, 0, sizeof(*tab));
    int64_t pos = 0;
    for (int i = 0; i < n_segs; ++i) {
        const h3_segment& s = segs[i];
        if (s.start != pos || s.len < 1) return H3_ERR_SEGMENTS;
        if (s.T < 1 || s.H < 1 || s.W < 1 || s.t0 < 0 || s.h0 < 0 || s.w0 < 0) return H3_ERR_SEGMENTS;
        if ((int64_t)s.T * s.H * s.W != s.len) return H3_ERR_SEGMENTS;
        if ((int64_t)s.H * s.W > INT32_MAX) return H3_ERR_SEGMENTS;
        if ((int64_t)s.t0 + s.T > INT32_MAX || (int64_t)s.h0 + s.H > INT32_MAX ||
            (int64_t)s.w0 + s.W > INT32_MAX)
            return H3_ERR_SEGMENTS;
        if (n_sets > 0 && (s.mod_set < 0 || s.mod_set >= n_sets)) return H3_ERR_SEGMENTS;
        pos += s.len;
        if (pos > n_tok) return H3_ERR_SEGMENTS;
        tab->s[i] = SegDev{(int32_t)s.start, s.mod_set, s.H * s.W, s.W, s.H, s.t0, s.h0, s.w0};
    }
    if (pos != n_tok) return H3_ERR_SEGMENTS;
    tab->n = n_segs;
    return H3_OK;
}

// Shape and layout checks shared by the three GEMM entry points.
h3_status check_gemm(const void* A, int64_t lda, const void* W, int64_t ldw, const void* C, int64_t ldc,
                     int64_t M, int32_t N, int32_t K, int32_t Ncols, h3_dtype dt) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!A || !W || !C || M < 0 || N < 1 || K < 1) return H3_ERR_ARG;
    const int es = esize(dt);
    if (lda < K || ldw < K || ldc < Ncols) return H3_ERR_ARG;
    if (M >= kMaxTok || N % 8 || K % (dt == H3_BF16 ? 64 : 32)) return H3_ERR_SHAPE;
    // a 256-row operand tile is addressed with 32-bit byte offsets
    if (lda * es * 256 >= ((int64_t)1 << 31) || ldw * es * 256 >= ((int64_t)1 << 31)) return H3_ERR_SHAPE;
    if (!aligned16(A) || !aligned16(W) || !aligned16(C) || (lda * es) % 16 || (ldw * es) % 16 ||
        (ldc * es) % 16)
        return H3_ERR_ALIGN;
    const Span c = span(C, M, Ncols, ldc, es);
    if (overlap(c, span(A, M, K, lda, es)) || overlap(c, span(W, N, K, ldw, es))) return H3_ERR_ARG;
    return H3_OK;
}

inline h3_status hip_status(hipError_t e) { return e == hipSuccess ? H3_OK : H3_ERR_HIP; }
// The launchers report hipGetLastError() after their launches; an error left
// by an earlier, unrelated HIP call of the thread is cleared first so that
// it is not taken for this call's.
inline void clear_last_error() { (void)hipGetLastError(); }

// Per-pair rotation table, exact in double: pair p of a head lies in the
// t, h or w chunk (widths d_t, d_h, d_w, already checked to sum to
// head_dim) and turns at base^(-2j/d_axis), j its index inside the chunk.
void fill_rope(int32_t head_dim, int32_t d_t, int32_t d_h, int32_t d_w, float rope_base, RopeTable* rt) {
    memset(rt, 0, sizeof(*rt));
    const int split[3] = {d_t, d_h, d_w};
    int axis = 0, first = 0;
    for (int p = 0; p < head_dim / 2; ++p) {
        while (2 * p >= first + split[axis]) first += split[axis++];
        const int j = p - first / 2;
        rt->axis[p] = (int8_t)axis;
        rt->inv_freq[p] = pow((double)rope_base, -2.0 * j / (double)split[axis]);
    }
}

// Checks of the q/k norm and rotation fused into a QKV projection of N
// columns (after the GEMM's own checks); fills the interval and rotation
// tables.
h3_status check_qkrope(int64_t M, int32_t N, int32_t heads, int32_t head_dim, const float* gamma_q,
                       const float* gamma_k, float eps, int32_t d_t, int32_t d_h, int32_t d_w, float rope_base,
                       const h3_segment* segs, int32_t n_segs, SegTable* tab, RopeTable* rt) {
    if (heads < 1 || !(eps >= 0.f) || !isfinite(eps) || !(rope_base > 0.f) || !isfinite(rope_base))
        return H3_ERR_ARG;
    if (head_dim != 64 && head_dim != 128) return H3_ERR_SHAPE;
    if (d_t < 0 || d_h < 0 || d_w < 0 || d_t % 2 || d_h % 2 || d_w % 2 || d_t + d_h + d_w != head_dim)
        return H3_ERR_SHAPE;
    // q and k heads fill whole 256-column tiles, and both fit in C's columns
    const int64_t q_cols = (int64_t)heads * head_dim;
    if (q_cols % 256 || 2 * q_cols > N) return H3_ERR_SHAPE;
    if (((uintptr_t)gamma_q & 3) || ((uintptr_t)gamma_k & 3)) return H3_ERR_ALIGN;
    const h3_status st = build_segs(segs, n_segs, M, 0, tab);
    if (st != H3_OK) return st;
    fill_rope(head_dim, d_t, d_h, d_w, rope_base, rt);
    return H3_OK;
}

}  // namespace

extern "C" {

const char* h3_status_str(h3_status s) {
    switch (s) {
        case H3_OK: return "ok";
        case H3_ERR_ARG: return "invalid argument";
        case H3_ERR_SEGMENTS: return "invalid interval table";
        case H3_ERR_DTYPE: return "unsupported dtype";
        case H3_ERR_ALIGN: return "misaligned pointer or row stride";
        case H3_ERR_SHAPE: return "unsupported size";
        case H3_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

h3_status h3_adaln_modulate(const void* x, void* y, int64_t n_tok, int32_t dim, const float* mod,
                            int32_t n_sets, h3_branch br, const h3_segment* segs, int32_t n_segs,
                            float eps, h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!x || !y || !mod || n_tok < 0 || n_sets < 1 || !valid_branch(br) || !(eps >= 0.f) || !isfinite(eps))
        return H3_ERR_ARG;
    if (n_tok >= kMaxTok || dim < 8 || dim % 8 || dim > kWave * kRowMaxVecPerLane * (16 / esize(dt)))
        return H3_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(y) || !aligned16(mod)) return H3_ERR_ALIGN;
    if (overlap(span(x, n_tok, dim, dim, esize(dt)), span(y, n_tok, dim, dim, esize(dt)))) return H3_ERR_ARG;
    SegTable tab;
    const h3_status st = build_segs(segs, n_segs, n_tok, n_sets, &tab);
    if (st != H3_OK) return st;
    if (n_tok == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_adaln(dt == H3_BF16, x, y, (int32_t)n_tok, dim, mod, (int32_t)br, tab, eps,
                                   (hipStream_t)stream));
}

h3_status h3_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
                       int64_t M, int32_t N, int32_t K, h3_dtype dt, void* stream) {
    const h3_status st = check_gemm(A, lda, W, ldw, C, ldc, M, N, K, N, dt);
    if (st != H3_OK) return st;
    if (M == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_gemm(dt == H3_BF16, A, lda, W, ldw, C, ldc, M, N, K, (hipStream_t)stream));
}

h3_status h3_gemm_gate_residual(const void* A, int64_t lda, const void* W, int64_t ldw, const void* x, void* out,
                                int64_t ldo, int64_t M, int32_t N, int32_t K, const float* mod, int32_t n_sets,
                                h3_branch br, const h3_segment* segs, int32_t n_segs, h3_dtype dt,
                                void* stream) {
    h3_status st = check_gemm(A, lda, W, ldw, out, ldo, M, N, K, N, dt);
    if (st != H3_OK) return st;
    if (!x || !mod || n_sets < 1 || !valid_branch(br)) return H3_ERR_ARG;
    if (!aligned16(x) || !aligned16(mod)) return H3_ERR_ALIGN;
    const int es = esize(dt);
    if (out != x && overlap(span(out, M, N, ldo, es), span(x, M, N, ldo, es))) return H3_ERR_ARG;
    SegTable tab;
    st = build_segs(segs, n_segs, M, n_sets, &tab);
    if (st != H3_OK) return st;
    if (M == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_gemm_gate(dt == H3_BF16, A, lda, W, ldw, x, out, ldo, M, N, K, mod, n_sets,
                                       (int32_t)br, tab, (hipStream_t)stream));
}

h3_status h3_gemm_swiglu(const void* A, int64_t lda, const void* Wgu, int64_t ldw, void* H, int64_t ldh,
                         int64_t M, int32_t F, int32_t K, h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (F < 1 || F > (1 << 29)) return H3_ERR_ARG;
    if (F % 32) return H3_ERR_SHAPE;
    const h3_status st = check_gemm(A, lda, Wgu, ldw, H, ldh, M, 2 * F, K, F, dt);
    if (st != H3_OK) return st;
    if (M == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_gemm_swiglu(dt == H3_BF16, A, lda, Wgu, ldw, H, ldh, M, F, K, (hipStream_t)stream));
}

h3_status h3_qknorm_rope3d(void* q, void* k, int64_t ld, int64_t n_tok, int32_t heads, int32_t head_dim,
                           const float* gamma_q, const float* gamma_k, float eps, int32_t d_t, int32_t d_h,
                           int32_t d_w, float rope_base, const h3_segment* segs, int32_t n_segs,
                           h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!q || !k || n_tok < 0 || heads < 1 || !(eps >= 0.f) || !isfinite(eps) || !(rope_base > 0.f) ||
        !isfinite(rope_base))
        return H3_ERR_ARG;
    if (head_dim != 64 && head_dim != 128) return H3_ERR_SHAPE;
    if (d_t < 0 || d_h < 0 || d_w < 0 || d_t % 2 || d_h % 2 || d_w % 2 || d_t + d_h + d_w != head_dim)
        return H3_ERR_SHAPE;
    if (n_tok >= kMaxTok) return H3_ERR_SHAPE;
    const int es = esize(dt);
    const int64_t width = (int64_t)heads * head_dim;
    if (ld < width) return H3_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || (ld * es) % 16 || ((uintptr_t)gamma_q & 3) ||
        ((uintptr_t)gamma_k & 3))
        return H3_ERR_ALIGN;
    if (overlap(span(q, n_tok, width, ld, es), span(k, n_tok, width, ld, es))) {
        // q and k may be interleaved column blocks of one buffer, never the same columns
        const intptr_t diff = (intptr_t)((uintptr_t)k - (uintptr_t)q) / es;
        const intptr_t rem = ((diff % ld) + ld) % ld;
        if (rem < width || ld - rem < width) return H3_ERR_ARG;
    }
    SegTable tab;
    const h3_status st = build_segs(segs, n_segs, n_tok, 0, &tab);
    if (st != H3_OK) return st;
    if (n_tok == 0) return H3_OK;
    RopeTable rt;
    fill_rope(head_dim, d_t, d_h, d_w, rope_base, &rt);
    return clear_last_error(), hip_status(launch_qknorm_rope(dt == H3_BF16, q, k, ld, (int32_t)n_tok, heads, head_dim, gamma_q,
                                         gamma_k, eps, rt, tab, (hipStream_t)stream));
}

h3_status h3_gemm_qknorm_rope(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
                              int64_t M, int32_t N, int32_t K, int32_t heads, int32_t head_dim,
                              const float* gamma_q, const float* gamma_k, float eps, int32_t d_t, int32_t d_h,
                              int32_t d_w, float rope_base, const h3_segment* segs, int32_t n_segs, h3_dtype dt,
                              void* stream) {
    h3_status st = check_gemm(A, lda, W, ldw, C, ldc, M, N, K, N, dt);
    if (st != H3_OK) return st;
    SegTable tab;
    RopeTable rt;
    st = check_qkrope(M, N, heads, head_dim, gamma_q, gamma_k, eps, d_t, d_h, d_w, rope_base, segs, n_segs, &tab, &rt);
    if (st != H3_OK || M == 0) return st;
    return clear_last_error(), hip_status(launch_gemm_qknorm_rope(dt == H3_BF16, A, lda, W, ldw, C, ldc, M, N, K, heads, head_dim,
                                              gamma_q, gamma_k, eps, rt, tab, (hipStream_t)stream));
}

h3_status h3_attention_fwd(const void* q, const void* k, const void* v, int64_t ld_qkv, void* o, int64_t ld_o,
                           int64_t n_tok, int32_t heads, int32_t head_dim, float scale, float* lse,
                           h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!q || !k || !v || !o || n_tok < 0 || heads < 1 || !isfinite(scale) || !(scale > 0.f)) return H3_ERR_ARG;
    if (head_dim != 64 && head_dim != 128) return H3_ERR_SHAPE;
    const int es = esize(dt);
    const int64_t width = (int64_t)heads * head_dim;
    if (ld_qkv < width || ld_o < width) return H3_ERR_ARG;
    // the kernel addresses a 64-key tile with 32-bit byte offsets
    if (n_tok >= kMaxTok || ld_qkv * es >= ((int64_t)1 << 25)) return H3_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (ld_qkv * es) % 16 ||
        (ld_o * es) % 16 || ((uintptr_t)lse & 3))
        return H3_ERR_ALIGN;
    const Span so = span(o, n_tok, width, ld_o, es);
    if (overlap(so, span(q, n_tok, width, ld_qkv, es)) || overlap(so, span(k, n_tok, width, ld_qkv, es)) ||
        overlap(so, span(v, n_tok, width, ld_qkv, es)))
        return H3_ERR_ARG;
    if (lse && overlap(span(lse, 1, (int64_t)heads * n_tok, 0, 4), so)) return H3_ERR_ARG;
    if (n_tok == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_attention(dt == H3_BF16, q, k, v, ld_qkv, o, ld_o, (int32_t)n_tok, heads, head_dim,
                                       scale, lse, (hipStream_t)stream));
}

h3_status h3_swiglu(const void* gu, void* h, int64_t n_tok, int32_t F, h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!gu || !h || n_tok < 0 || F < 1) return H3_ERR_ARG;
    if (F % 8 || n_tok >= kMaxTok) return H3_ERR_SHAPE;
    if (!aligned16(gu) || !aligned16(h)) return H3_ERR_ALIGN;
    const int es = esize(dt);
    if (overlap(span(gu, n_tok, 2 * (int64_t)F, 2 * (int64_t)F, es), span(h, n_tok, F, F, es))) return H3_ERR_ARG;
    if (n_tok == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_swiglu(dt == H3_BF16, gu, h, n_tok, F, (hipStream_t)stream));
}

h3_status h3_interleave_gate_up(const void* w_gu, int64_t ld_src, void* w_il, int64_t ld_dst, int32_t F,
                                int32_t K, h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!w_gu || !w_il || F < 0 || K < 1) return H3_ERR_ARG;
    const int es = esize(dt);
    if (F % 32 || (K * es) % 16 || (int64_t)F * 2 >= kMaxTok) return H3_ERR_SHAPE;
    if (ld_src < K || ld_dst < K || (ld_src * es) % 16 || (ld_dst * es) % 16) return H3_ERR_SHAPE;
    if (!aligned16(w_gu) || !aligned16(w_il)) return H3_ERR_ALIGN;
    if (overlap(span(w_gu, 2 * (int64_t)F, K, ld_src, es), span(w_il, 2 * (int64_t)F, K, ld_dst, es)))
        return H3_ERR_ARG;
    if (F == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_interleave_gate_up(w_gu, ld_src * es, w_il, ld_dst * es, F, (int64_t)K * es,
                                                (hipStream_t)stream));
}

h3_status h3_gate_residual(const void* x, const void* y, void* out, int64_t n_tok, int32_t dim,
                           const float* mod, int32_t n_sets, h3_branch br, const h3_segment* segs,
                           int32_t n_segs, h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!x || !y || !out || !mod || n_tok < 0 || n_sets < 1 || !valid_branch(br)) return H3_ERR_ARG;
    if (dim < 8 || dim % 8 || n_tok >= kMaxTok) return H3_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(y) || !aligned16(out) || !aligned16(mod)) return H3_ERR_ALIGN;
    const int es = esize(dt);
    const Span so = span(out, n_tok, dim, dim, es);
    if (overlap(so, span(y, n_tok, dim, dim, es))) return H3_ERR_ARG;
    if (out != x && overlap(so, span(x, n_tok, dim, dim, es))) return H3_ERR_ARG;
    SegTable tab;
    const h3_status st = build_segs(segs, n_segs, n_tok, n_sets, &tab);
    if (st != H3_OK) return st;
    if (n_tok == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_gate_residual(dt == H3_BF16, x, y, out, (int32_t)n_tok, dim, mod, (int32_t)br, tab,
                                           (hipStream_t)stream));
}

h3_status h3_euler_update(void* x, const void* v, int64_t n_tok, int32_t dim, const float* coef,
                          const h3_segment* segs, int32_t n_segs, h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!x || !v || n_tok < 0 || (n_segs > 0 && !coef)) return H3_ERR_ARG;
    if (dim < 8 || dim % 8 || n_tok >= kMaxTok) return H3_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(v)) return H3_ERR_ALIGN;
    const int es = esize(dt);
    if (overlap(span(x, n_tok, dim, dim, es), span(v, n_tok, dim, dim, es))) return H3_ERR_ARG;
    SegTable tab;
    const h3_status st = build_segs(segs, n_segs, n_tok, 0, &tab);
    if (st != H3_OK) return st;
    SegCoef c;
    for (int i = 0; i < kMaxSegs; ++i) c.c[i] = 0.f;
    for (int i = 0; i < n_segs; ++i) {
        if (!isfinite(coef[i])) return H3_ERR_ARG;
        c.c[i] = coef[i];
    }
    if (n_tok == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_euler(dt == H3_BF16, x, v, (int32_t)n_tok, dim, tab, c, (hipStream_t)stream));
}

// Shared checks of the patch calls: grid and patch sizes, the vector width,
// the row stride, alignment and overlap.  Writes the token count to *n_tok.
static h3_status check_patch(const void* lat, const void* tok, int64_t ld, int32_t T, int32_t H, int32_t W,
                             int32_t C, int32_t pt, int32_t ph, int32_t pw, h3_dtype dt, int64_t* n_tok) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!lat || !tok || T < 0 || H < 1 || W < 1 || C < 1 || pt < 1 || ph < 1 || pw < 1) return H3_ERR_ARG;
    if (T % pt || H % ph || W % pw) return H3_ERR_SHAPE;
    const int es = esize(dt), vec = 16 / es;
    if (C % vec) return H3_ERR_SHAPE;
    const int64_t P = (int64_t)pt * ph * pw * C;
    if (P >= (1 << 30) || (int64_t)H * W * C >= ((int64_t)1 << 40)) return H3_ERR_SHAPE;
    if (ld < P) return H3_ERR_ARG;
    if (ld % vec || !aligned16(lat) || !aligned16(tok)) return H3_ERR_ALIGN;
    const int64_t n = (int64_t)(T / pt) * (H / ph) * (W / pw);
    if (n >= kMaxTok) return H3_ERR_SHAPE;
    if (overlap(span(lat, 1, (int64_t)T * H * W * C, 0, es), span(tok, n, ld, ld, es))) return H3_ERR_ARG;
    *n_tok = n;
    return H3_OK;
}

h3_status h3_patchify(const void* latent, int32_t T, int32_t H, int32_t W, int32_t C, int32_t pt, int32_t ph,
                      int32_t pw, void* tokens, int64_t ld, h3_dtype dt, void* stream) {
    int64_t n = 0;
    const h3_status st = check_patch(latent, tokens, ld, T, H, W, C, pt, ph, pw, dt, &n);
    if (st != H3_OK) return st;
    if (n == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_patchify(dt == H3_BF16, latent, tokens, ld, PatchGeom{T, H, W, C, pt, ph, pw}, n,
                                      (hipStream_t)stream));
}

h3_status h3_unpatchify(const void* tokens, int64_t ld, int32_t T, int32_t H, int32_t W, int32_t C, int32_t pt,
                        int32_t ph, int32_t pw, void* latent, h3_dtype dt, void* stream) {
    int64_t n = 0;
    const h3_status st = check_patch(latent, tokens, ld, T, H, W, C, pt, ph, pw, dt, &n);
    if (st != H3_OK) return st;
    if (n == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_unpatchify(dt == H3_BF16, tokens, ld, latent, PatchGeom{T, H, W, C, pt, ph, pw},
                                        (hipStream_t)stream));
}

h3_status h3_quantize_fp8(const void* x, int64_t ldx, int64_t n_rows, int32_t K, void* q, int64_t ldq,
                          float* scales, h3_dtype dt, void* stream) {
    if (!valid_dt(dt)) return H3_ERR_DTYPE;
    if (!x || !q || !scales || n_rows < 0 || K < 1 || ldx < K || ldq < K) return H3_ERR_ARG;
    if (n_rows >= kMaxTok || K % 16) return H3_ERR_SHAPE;
    const int es = esize(dt);
    if (!aligned16(x) || !aligned16(q) || (ldx * es) % 16 || ldq % 16 || ((uintptr_t)scales & 3)) return H3_ERR_ALIGN;
    const Span sq = span(q, n_rows, K, ldq, 1);
    if (overlap(sq, span(x, n_rows, K, ldx, es)) || overlap(span(scales, 1, n_rows, 0, 4), sq) ||
        overlap(span(scales, 1, n_rows, 0, 4), span(x, n_rows, K, ldx, es)))
        return H3_ERR_ARG;
    if (n_rows == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_quantize_fp8(dt == H3_BF16, x, ldx, (int32_t)n_rows, K, q, ldq, scales,
                                          (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Shared checks of the fp8 GEMMs: A [M][K] and W [N][K] e4m3 codes with
// their scales, C [M][Ncols] of element size es.
h3_status check_gemm_fp8(const void* A, int64_t lda, const float* a_scale, const void* W, int64_t ldw,
                         const float* w_scale, const void* C, int64_t ldc, int64_t M, int32_t N, int32_t K,
                         int32_t Ncols, int es) {
    if (!A || !W || !C || !a_scale || !w_scale || M < 0 || N < 1 || K < 1) return H3_ERR_ARG;
    if (lda < K || ldw < K || ldc < Ncols) return H3_ERR_ARG;
    if (M >= kMaxTok || N % 8 || K % 128) return H3_ERR_SHAPE;
    if (lda * 256 >= ((int64_t)1 << 31) || ldw * 256 >= ((int64_t)1 << 31)) return H3_ERR_SHAPE;
    if (!aligned16(A) || !aligned16(W) || !aligned16(C) || lda % 16 || ldw % 16 || (ldc * es) % 16 ||
        ((uintptr_t)a_scale & 3) || ((uintptr_t)w_scale & 3))
        return H3_ERR_ALIGN;
    const Span c = span(C, M, Ncols, ldc, es);
    if (overlap(c, span(A, M, K, lda, 1)) || overlap(c, span(W, N, K, ldw, 1)) ||
        overlap(c, span(a_scale, 1, M, 0, 4)) || overlap(c, span(w_scale, 1, N, 0, 4)))
        return H3_ERR_ARG;
    return H3_OK;
}

}  // namespace

extern "C" {

h3_status h3_gemm_fp8(const void* A, int64_t lda, const float* a_scale, const void* W, int64_t ldw,
                      const float* w_scale, void* C, int64_t ldc, int64_t M, int32_t N, int32_t K, h3_dtype out_dt,
                      void* stream) {
    if (!valid_dt(out_dt)) return H3_ERR_DTYPE;
    const h3_status st = check_gemm_fp8(A, lda, a_scale, W, ldw, w_scale, C, ldc, M, N, K, N, esize(out_dt));
    if (st != H3_OK) return st;
    if (M == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_gemm_fp8(A, lda, a_scale, W, ldw, w_scale, C, ldc, M, N, K, out_dt == H3_BF16,
                                      (hipStream_t)stream));
}

h3_status h3_gemm_fp8_gate_residual(const void* A, int64_t lda, const float* a_scale, const void* W, int64_t ldw,
                                    const float* w_scale, const void* x, void* out, int64_t ldo, int64_t M, int32_t N,
                                    int32_t K, const float* mod, int32_t n_sets, h3_branch br, const h3_segment* segs,
                                    int32_t n_segs, void* stream) {
    h3_status st = check_gemm_fp8(A, lda, a_scale, W, ldw, w_scale, out, ldo, M, N, K, N, 2);
    if (st != H3_OK) return st;
    if (!x || !mod || n_sets < 1 || !valid_branch(br)) return H3_ERR_ARG;
    if (!aligned16(x) || !aligned16(mod)) return H3_ERR_ALIGN;
    const Span so = span(out, M, N, ldo, 2);
    if (out != x && overlap(so, span(x, M, N, ldo, 2))) return H3_ERR_ARG;
    if (overlap(span(x, M, N, ldo, 2), span(A, M, K, lda, 1))) return H3_ERR_ARG;
    SegTable tab;
    st = build_segs(segs, n_segs, M, n_sets, &tab);
    if (st != H3_OK) return st;
    if (M == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_gemm_fp8_gate(A, lda, a_scale, W, ldw, w_scale, x, out, ldo, M, N, K, mod, n_sets,
                                           (int32_t)br, tab, (hipStream_t)stream));
}

h3_status h3_gemm_fp8_swiglu(const void* A, int64_t lda, const float* a_scale, const void* Wgu, int64_t ldw,
                             const float* w_scale, void* H, int64_t ldh, int64_t M, int32_t F, int32_t K, void* stream) {
    if (F < 1 || F > (1 << 29)) return H3_ERR_ARG;
    if (F % 32) return H3_ERR_SHAPE;
    const h3_status st = check_gemm_fp8(A, lda, a_scale, Wgu, ldw, w_scale, H, ldh, M, 2 * F, K, F, 2);
    if (st != H3_OK) return st;
    if (M == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_gemm_fp8_swiglu(A, lda, a_scale, Wgu, ldw, w_scale, H, ldh, M, F, K,
                                             (hipStream_t)stream));
}

h3_status h3_gemm_fp8_qknorm_rope(const void* A, int64_t lda, const float* a_scale, const void* W, int64_t ldw,
                                  const float* w_scale, void* C, int64_t ldc, int64_t M, int32_t N, int32_t K,
                                  int32_t heads, int32_t head_dim, const float* gamma_q, const float* gamma_k,
                                  float eps, int32_t d_t, int32_t d_h, int32_t d_w, float rope_base,
                                  const h3_segment* segs, int32_t n_segs, void* stream) {
    h3_status st = check_gemm_fp8(A, lda, a_scale, W, ldw, w_scale, C, ldc, M, N, K, N, 2);
    if (st != H3_OK) return st;
    SegTable tab;
    RopeTable rt;
    st = check_qkrope(M, N, heads, head_dim, gamma_q, gamma_k, eps, d_t, d_h, d_w, rope_base, segs, n_segs, &tab, &rt);
    if (st != H3_OK || M == 0) return st;
    return clear_last_error(), hip_status(launch_gemm_fp8_qknorm_rope(A, lda, a_scale, W, ldw, w_scale, C, ldc, M, N, K, heads, head_dim,
                                                  gamma_q, gamma_k, eps, rt, tab, (hipStream_t)stream));
}

h3_status h3_quantize_qkv_fp8(const void* q, const void* k, const void* v, int64_t ld, int64_t n_tok, int32_t heads,
                              int32_t head_dim, void* q8, void* k8, void* vt, int64_t n_pad, float* sq, float* sk,
                              float* sv, h3_dtype dt, void* stream) {
    if (dt != H3_BF16) return valid_dt(dt) ? H3_ERR_SHAPE : H3_ERR_DTYPE;
    if (!q || !k || !v || !q8 || !k8 || !vt || !sq || !sk || !sv || n_tok < 0 || heads < 1) return H3_ERR_ARG;
    if (head_dim != 128) return H3_ERR_SHAPE;
    const int64_t width = (int64_t)heads * 128;
    if (ld < width || n_pad < ((n_tok + 63) / 64) * 64 || n_pad % 64) return H3_ERR_ARG;
    if (n_tok >= kMaxTok || n_pad * 128 >= ((int64_t)1 << 32) || width * 64 >= ((int64_t)1 << 31) ||
        heads > 65535 || n_tok * heads >= ((int64_t)1 << 31))
        return H3_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (ld * 2) % 16 || !aligned16(q8) || !aligned16(k8) ||
        !aligned16(vt) || ((uintptr_t)sq & 3) || ((uintptr_t)sk & 3) || ((uintptr_t)sv & 3))
        return H3_ERR_ALIGN;
    const Span outs[6] = {span(q8, n_tok, width, width, 1), span(k8, n_tok, width, width, 1),
                          span(vt, (int64_t)heads * 128, n_pad, n_pad, 1), span(sq, 1, (int64_t)heads * n_tok, 0, 4),
                          span(sk, 1, heads, 0, 4), span(sv, 1, heads, 0, 4)};
    const Span ins[3] = {span(q, n_tok, width, ld, 2), span(k, n_tok, width, ld, 2), span(v, n_tok, width, ld, 2)};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 3; ++j)
            if (overlap(outs[i], ins[j])) return H3_ERR_ARG;
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j])) return H3_ERR_ARG;
    }
    if (n_tok == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_quantize_qkv_fp8(q, k, v, ld, (int32_t)n_tok, heads, q8, k8, vt, n_pad, sq, sk, sv,
                                              (hipStream_t)stream));
}

h3_status h3_attention_fp8(const void* q8, const void* k8, const void* vt, int64_t n_pad, const float* sq,
                           const float* sk, const float* sv, void* o, int64_t ld_o, int64_t n_tok, int32_t heads,
                           int32_t head_dim, float scale, void* stream) {
    if (!q8 || !k8 || !vt || !sq || !sk || !sv || !o || n_tok < 0 || heads < 1 || !isfinite(scale) ||
        !(scale > 0.f))
        return H3_ERR_ARG;
    if (head_dim != 128) return H3_ERR_SHAPE;
    const int64_t width = (int64_t)heads * 128;
    if (ld_o < width || n_pad < ((n_tok + 63) / 64) * 64 || n_pad % 64) return H3_ERR_ARG;
    if (n_tok >= kMaxTok || n_pad * 128 >= ((int64_t)1 << 32) || width * 64 >= ((int64_t)1 << 31) ||
        heads > 65535 || n_tok * heads >= ((int64_t)1 << 31))
        return H3_ERR_SHAPE;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(vt) || !aligned16(o) || (ld_o * 2) % 16 ||
        ((uintptr_t)sq & 3) || ((uintptr_t)sk & 3) || ((uintptr_t)sv & 3))
        return H3_ERR_ALIGN;
    const Span so = span(o, n_tok, width, ld_o, 2);
    if (overlap(so, span(q8, n_tok, width, width, 1)) || overlap(so, span(k8, n_tok, width, width, 1)) ||
        overlap(so, span(vt, (int64_t)heads * 128, n_pad, n_pad, 1)) ||
        overlap(so, span(sq, 1, (int64_t)heads * n_tok, 0, 4)) || overlap(so, span(sk, 1, heads, 0, 4)) ||
        overlap(so, span(sv, 1, heads, 0, 4)))
        return H3_ERR_ARG;
    if (n_tok == 0) return H3_OK;
    return clear_last_error(), hip_status(launch_attention_fp8(q8, k8, vt, n_pad, sq, sk, sv, o, ld_o, (int32_t)n_tok, heads, scale,
                                           (hipStream_t)stream));
}

}  // extern "C"
