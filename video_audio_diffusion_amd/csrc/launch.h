// Internal launchers of libh3blk (host side).  The C ABI in abi.hip checks
// every argument and then calls exactly one of these.
#pragma once

#include "common.h"

namespace h3 {

// Per-pair RoPE table: pair p of a head (elements 2p, 2p+1) turns with
// the position on axis[p] (0 = t, 1 = h, 2 = w) at frequency inv_freq[p].
struct RopeTable {
    double inv_freq[64];
    int8_t axis[64];
};

hipError_t launch_adaln(bool bf, const void* x, void* y, int32_t n, int32_t dim,
                        const float* mod, int32_t br, const SegTable& tab, float eps,
                        hipStream_t st);
hipError_t launch_euler(bool bf, void* x, const void* v, int32_t n, int32_t dim, const SegTable& tab,
                        const SegCoef& coef, hipStream_t st);
hipError_t launch_gate_residual(bool bf, const void* x, const void* y, void* out, int32_t n,
                                int32_t dim, const float* mod, int32_t br, const SegTable& tab,
                                hipStream_t st);
hipError_t launch_swiglu(bool bf, const void* gu, void* h, int64_t n, int32_t F, hipStream_t st);
hipError_t launch_interleave_gate_up(const void* src, int64_t ld_src_bytes, void* dst, int64_t ld_dst_bytes,
                                     int32_t F, int64_t row_bytes, hipStream_t st);
hipError_t launch_qknorm_rope(bool bf, void* q, void* k, int64_t ld, int32_t n, int32_t heads,
                              int32_t hd, const float* gq, const float* gk, float eps,
                              const RopeTable& rt, const SegTable& tab, hipStream_t st);
hipError_t launch_gemm_gate(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, const void* x,
                            void* out, int64_t ldo, int64_t M, int32_t N, int32_t K, const float* mod,
                            int32_t n_sets, int32_t br, const SegTable& tab, hipStream_t st);
hipError_t launch_gemm_swiglu(bool bf, const void* A, int64_t lda, const void* Wgu, int64_t ldw, void* H,
                              int64_t ldh, int64_t M, int32_t F, int32_t K, hipStream_t st);
hipError_t launch_gemm_qknorm_rope(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                                  int64_t ldc, int64_t M, int32_t N, int32_t K, int32_t heads, int32_t hd,
                                  const float* gq, const float* gk, float eps, const RopeTable& rt,
                                  const SegTable& tab, hipStream_t st);
// Latent grid [T][H][W][C] and its (pt, ph, pw) patch.
struct PatchGeom {
    int32_t T, H, W, C, pt, ph, pw;
};
hipError_t launch_patchify(bool bf, const void* lat, void* tok, int64_t ld, const PatchGeom& g, int64_t n_tok,
                           hipStream_t st);
hipError_t launch_unpatchify(bool bf, const void* tok, int64_t ld, void* lat, const PatchGeom& g, hipStream_t st);
hipError_t launch_gemm_fp8(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw, const float* sw,
                           void* C, int64_t ldc, int64_t M, int32_t N, int32_t K, bool out_bf16, hipStream_t st);
hipError_t launch_gemm_fp8_gate(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw,
                                const float* sw, const void* x, void* out, int64_t ldo, int64_t M, int32_t N,
                                int32_t K, const float* mod, int32_t n_sets, int32_t br, const SegTable& tab,
                                hipStream_t st);
hipError_t launch_gemm_fp8_qknorm_rope(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw,
                                      const float* sw, void* C, int64_t ldc, int64_t M, int32_t N, int32_t K,
                                      int32_t heads, int32_t hd, const float* gq, const float* gk, float eps,
                                      const RopeTable& rt, const SegTable& tab, hipStream_t st);
hipError_t launch_gemm_fp8_swiglu(const void* A, int64_t lda, const float* sa, const void* Wgu, int64_t ldw,
                                  const float* sw, void* H, int64_t ldh, int64_t M, int32_t F, int32_t K,
                                  hipStream_t st);
hipError_t launch_quantize_fp8(bool bf, const void* x, int64_t ldx, int32_t n, int32_t K, void* q, int64_t ldq,
                               float* scales, hipStream_t st);
hipError_t launch_quantize_qkv_fp8(const void* q, const void* k, const void* v, int64_t ld, int32_t n, int32_t heads,
                                   void* q8, void* k8, void* vt, int64_t n_pad, float* sq, float* sk, float* sv,
                                   hipStream_t st);
hipError_t launch_attention_fp8(const void* q8, const void* k8, const void* vt, int64_t n_pad, const float* sq,
                                const float* sk, const float* sv, void* o, int64_t ldo, int32_t n, int32_t heads,
                                float scale, hipStream_t st);
hipError_t launch_gemm(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                       int64_t ldc, int64_t M, int32_t N, int32_t K, hipStream_t st);
hipError_t launch_attention(bool bf, const void* q, const void* k, const void* v, int64_t ld_qkv,
                            void* o, int64_t ld_o, int32_t n, int32_t heads, int32_t hd,
                            float scale, float* lse, hipStream_t st);

// Largest row width (elements) the one-wave-per-row kernels hold in registers.
constexpr int kRowMaxVecPerLane = 16;

}  // namespace h3
