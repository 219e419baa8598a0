// Row-wise quantisation to OCP FP8 e4m3 (4 exponent bits, bias 7, 3 mantissa
// bits, largest finite value 448, no infinities, NaN = 0x7F / 0xFF) for the
// fp8 projections: each row gets the scale max|x| / 448 (1 for an all-zero
// row) and q = e4m3(x / scale), rounded to nearest with ties to even.
#include "launch.h"

namespace h3 {

// |a| -> e4m3 code 0..0x7E (finite a >= 0), nearest-even, saturating at 448.
// Below 2^-6 the format is subnormal with step 2^-9, so the code is the
// nearest integer to a * 2^9 (exact scaling); above it, the fp32 mantissa is
// rounded to 3 bits (a carry moves into the exponent) and the exponent rebased
// from bias 127 to bias 7.
__device__ __forceinline__ uint32_t e4m3_magnitude(float a) {
    if (!(a < 448.0f)) return 0x7Eu;
    if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    const uint32_t c = ((((b >> 23) - 120u)) << 3) | ((b >> 20) & 7u);
    return c > 0x7Eu ? 0x7Eu : c;
}

__device__ __forceinline__ uint32_t e4m3_code(float x) {
    if (x != x) return 0x7Fu;
    return e4m3_magnitude(__builtin_fabsf(x)) | ((__float_as_uint(x) >> 24) & 0x80u);
}

// The same codes, fast, for x / s with s finite and > 0, |x| <= the max |x|
// the scale was taken from (so |x / s| <= 448 (1 + 2^-23)) and x not NaN:
//  * the quotient: for fp32 x and s with |x / s| in fp32's normal range,
//    x / s is never an fp32 rounding midpoint and lies at least 2^-49
//    (relative) from every one (x / s = midpoint would need a 25-bit odd
//    significand from 24-bit operands; the distance is a nonzero integer
//    over a 48-bit denominator), so rounding the fp64 product
//    x * RN64(1 / s), within 2^-52 of x / s, to fp32 gives exactly the
//    correctly rounded fp32 quotient.  Below 2^-126 the fp32 grid is fixed
//    and the argument fails (the two can differ by one subnormal step), but
//    every such quotient is far below e4m3's smallest step 2^-9 and both
//    encode to a signed zero;
//  * the encoding: the hardware fp32 -> e4m3 conversion gives e4m3_code's
//    result for every fp32 value of magnitude below 464 (checked on all 2^32
//    bit patterns; above that it returns NaN where e4m3_code saturates).
// r = 1 / (double)s.  Four codes, value e in bits 8e .. 8e+7.
__device__ __forceinline__ uint32_t e4m3_codes4(float a, float b, float c, float d, double r) {
    const float qa = (float)((double)a * r), qb = (float)((double)b * r);
    const float qc = (float)((double)c * r), qd = (float)((double)d * r);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(qa, qb, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qc, qd, lo, true);
}

// Largest |x| of eight bf16 values (as stored) by their bit patterns: below
// 0x7F80 all eight are finite and it is the bf16 pattern of their max |x|
// (non-negative values order like their bit patterns).
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(const u32x4& u) {
    u16x2 m = __builtin_bit_cast(u16x2, u[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, u[i] & 0x7FFF7FFFu));
    return m[0] > m[1] ? m[0] : m[1];
}

// One wavefront per row: max |x| over the row, then the scaled codes, four
// per 32-bit store.
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ x, int64_t ldx, int32_t n, int32_t K,
                                                           uint8_t* __restrict__ q, int64_t ldq,
                                                           float* __restrict__ scales) {
    constexpr int V = Vec<T>::N;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const char* xr = reinterpret_cast<const char*>(x + (int64_t)row * ldx);
    const int nv = K / V;
    float mx = 0.f;
    for (int j = lane; j < nv; j += kWave) {
        float v[V];
        Vec<T>::load(xr + 16 * j, v);
#pragma unroll
        for (int e = 0; e < V; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[e]));
    }
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, kWave));
    const float scale = mx > 0.f ? mx / 448.0f : 1.0f;
    if (lane == 0) scales[row] = scale;
    uint8_t* qr = q + (int64_t)row * ldq;
    for (int j = lane; j < nv; j += kWave) {
        float v[V];
        Vec<T>::load(xr + 16 * j, v);
#pragma unroll
        for (int e = 0; e < V; e += 4) {
            const uint32_t w = e4m3_code(v[e] / scale) | (e4m3_code(v[e + 1] / scale) << 8) |
                               (e4m3_code(v[e + 2] / scale) << 16) | (e4m3_code(v[e + 3] / scale) << 24);
            *reinterpret_cast<uint32_t*>(qr + j * V + e) = w;
        }
    }
}

// bf16 rows of at most 64 VPL vectors: one wavefront per row, the row read
// once and held in registers; its max |x| from the bit patterns; codes by
// e4m3_codes4, eight per 8-byte store.  A row holding an infinity or a NaN
// takes the general kernel's arithmetic (fmaxf max, e4m3_code of x / scale).
template <int VPL>
__global__ __launch_bounds__(256) void quantize_fp8_rows_kernel(const bf16* __restrict__ x, int64_t ldx, int32_t n,
                                                                int32_t K, uint8_t* __restrict__ q, int64_t ldq,
                                                                float* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const char* xr = reinterpret_cast<const char*>(x + (int64_t)row * ldx);
    const int nv = K / 8;
    u32x4 raw[VPL];
    uint32_t mb = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int j = lane + 64 * k;
        raw[k] = j < nv ? *reinterpret_cast<const u32x4*>(xr + 16 * j) : (u32x4){};
    }
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const uint32_t b = bf16x8_absmax_bits(raw[k]);
        mb = b > mb ? b : mb;
    }
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mb, m, kWave);
        mb = o > mb ? o : mb;
    }
    uint8_t* qr = q + (int64_t)row * ldq;
    if (mb < 0x7F80u) {
        const float mx = __uint_as_float(mb << 16);
        const float scale = mx > 0.f ? mx / 448.0f : 1.0f;
        if (lane == 0) scales[row] = scale;
        const double r = 1.0 / (double)scale;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int j = lane + 64 * k;
            if (j < nv) {
                float v[8];
                Vec<bf16>::load(&raw[k], v);
                *reinterpret_cast<u32x2*>(qr + 8 * j) =
                    (u32x2){e4m3_codes4(v[0], v[1], v[2], v[3], r), e4m3_codes4(v[4], v[5], v[6], v[7], r)};
            }
        }
    } else {
        float mx = 0.f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            float v[8];
            Vec<bf16>::load(&raw[k], v);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[e]));
        }
#pragma unroll
        for (int m = kWave / 2; m > 0; m >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, kWave));
        const float scale = mx > 0.f ? mx / 448.0f : 1.0f;
        if (lane == 0) scales[row] = scale;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int j = lane + 64 * k;
            if (j < nv) {
                float v[8];
                Vec<bf16>::load(&raw[k], v);
                uint32_t w[2] = {0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e >> 2] |= e4m3_code(v[e] / scale) << (8 * (e & 3));
                *reinterpret_cast<u32x2*>(qr + 8 * j) = (u32x2){w[0], w[1]};
            }
        }
    }
}

// ---------------------------------------------------------------- attention operands
// Quantisation of q, k and v ([n][heads * 128] views, bf16) for the fp8
// attention: q per (token, head) -- its scale folds into that query's softmax
// multiplier -- and k and v per head, whose scales fold into constants.  v is
// written transposed, [head][d][n_pad], with each group of 64 keys permuted
// into the byte order in which the attention kernel packs P: position
// p = 32 g + b of a group holds key 32 (b / 16) + 8 ((b % 16) / 4) + 4 g + b % 4,
// so that every fragment of V^T is 32 contiguous bytes.  Keys past n are 0.

__device__ __forceinline__ int vt_key(int p) {
    const int g = p >> 5, b = p & 31;
    return 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * g + (b & 3);
}

__global__ void zero_floats(float* a, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = 0.f;
}

// max |x| over every token of each head: one workgroup per (head, 1024-row
// chunk); 16 lanes per row, 16 rows per pass; one atomic max per workgroup on
// the float's bits (non-negative floats order like their bit patterns).
__global__ __launch_bounds__(256) void absmax_heads_kernel(const bf16* __restrict__ x, int64_t ld, int32_t n,
                                                           float* amax) {
    const int head = blockIdx.x, r0 = blockIdx.y * 1024;
    const int sub = threadIdx.x & 15, rr = threadIdx.x >> 4;
    float mx = 0.f;
    for (int r = r0 + rr; r < n && r < r0 + 1024; r += 16) {
        float v[8];
        Vec<bf16>::load(x + (int64_t)r * ld + head * 128 + sub * 8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[e]));
    }
#pragma unroll
    for (int m = kWave / 2; m > 0; m >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, kWave));
    __shared__ float wmax[4];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float m = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
        atomicMax(reinterpret_cast<unsigned int*>(amax + head), __float_as_uint(m));
    }
}

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.f ? amax / 448.0f : 1.0f; }

// q: 16 lanes per (token, head): the group's max, its scale, 8 codes per lane.
__global__ __launch_bounds__(256) void quantize_q_kernel(const bf16* __restrict__ q, int64_t ld, int32_t n,
                                                         int32_t heads, uint8_t* __restrict__ q8,
                                                         float* __restrict__ sq) {
    const int64_t grp = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    const int sub = threadIdx.x & 15;
    if (grp >= (int64_t)n * heads) return;        // uniform across a group's 16 lanes
    const int row = (int)(grp / heads), head = (int)(grp % heads);
    const u32x4 raw = *reinterpret_cast<const u32x4*>(q + (int64_t)row * ld + head * 128 + sub * 8);
    float v[8];
    Vec<bf16>::load(&raw, v);
    // the group's max |x| by bit patterns (a group with an infinity or a NaN
    // takes e4m3_code below, with the fmaxf max)
    uint32_t mb = bf16x8_absmax_bits(raw);
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mb, m, kWave);
        mb = o > mb ? o : mb;
    }
    uint32_t w0 = 0, w1 = 0;
    float sc;
    if (mb < 0x7F80u) {
        sc = scale_of(__uint_as_float(mb << 16));
        const double r = 1.0 / (double)sc;
        w0 = e4m3_codes4(v[0], v[1], v[2], v[3], r);
        w1 = e4m3_codes4(v[4], v[5], v[6], v[7], r);
    } else {
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[e]));
#pragma unroll
        for (int m = 8; m > 0; m >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, kWave));
        sc = scale_of(mx);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0 |= e4m3_code(v[e] / sc) << (8 * e);
            w1 |= e4m3_code(v[e + 4] / sc) << (8 * e);
        }
    }
    if (sub == 0) sq[(int64_t)head * n + row] = sc;
    *reinterpret_cast<u32x2*>(q8 + (int64_t)row * heads * 128 + head * 128 + sub * 8) = (u32x2){w0, w1};
}

// k: one thread per 8 values with its head's scale.
__global__ __launch_bounds__(256) void quantize_k_kernel(const bf16* __restrict__ k, int64_t ld, int32_t n,
                                                         int32_t heads, const float* __restrict__ amax,
                                                         uint8_t* __restrict__ k8) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per_row = heads * 16;
    if (idx >= (int64_t)n * per_row) return;
    const int row = (int)(idx / per_row), c = (int)(idx % per_row);
    const float sc = scale_of(amax[c >> 4]);
    const u32x4 raw = *reinterpret_cast<const u32x4*>(k + (int64_t)row * ld + c * 8);
    float v[8];
    Vec<bf16>::load(&raw, v);
    uint32_t w0 = 0, w1 = 0;
    // the head's max (finite scale) bounds these values; an infinity or a
    // NaN among them takes e4m3_code
    if (sc < __builtin_inff() && bf16x8_absmax_bits(raw) < 0x7F80u) {
        const double r = 1.0 / (double)sc;
        w0 = e4m3_codes4(v[0], v[1], v[2], v[3], r);
        w1 = e4m3_codes4(v[4], v[5], v[6], v[7], r);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0 |= e4m3_code(v[e] / sc) << (8 * e);
            w1 |= e4m3_code(v[e + 4] / sc) << (8 * e);
        }
    }
    *reinterpret_cast<u32x2*>(k8 + (int64_t)row * heads * 128 + c * 8) = (u32x2){w0, w1};
}

// v -> V^T: one workgroup per (64-key group, head); the group's [64][128]
// values go through LDS, then each thread writes 16 permuted bytes of a d row.
__global__ __launch_bounds__(256) void quantize_vt_kernel(const bf16* __restrict__ v, int64_t ld, int32_t n,
                                                          const float* __restrict__ amax, uint8_t* __restrict__ vt,
                                                          int64_t n_pad) {
    const int t = blockIdx.x, head = blockIdx.y;
    __shared__ float tile[64][129];
    __shared__ int nonfinite;
    if (threadIdx.x == 0) nonfinite = 0;
    __syncthreads();
    bool nf = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int item = threadIdx.x + 256 * u;        // 64 keys x 16 vectors
        const int key = item >> 4, c = item & 15;
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (t * 64 + key < n) raw = *reinterpret_cast<const u32x4*>(v + (int64_t)(t * 64 + key) * ld + head * 128 + c * 8);
        nf |= bf16x8_absmax_bits(raw) >= 0x7F80u;
        float val[8];
        Vec<bf16>::load(&raw, val);
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[key][c * 8 + e] = val[e];
    }
    if (nf) nonfinite = 1;
    __syncthreads();
    const float sc = scale_of(amax[head]);
    // the head's max (finite scale) bounds the tile; a tile holding an
    // infinity or a NaN takes e4m3_code (uniform over the workgroup)
    const bool fast = sc < __builtin_inff() && !nonfinite;
    const double r = 1.0 / (double)sc;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int item = threadIdx.x + 256 * u;        // 128 d rows x 4 slots of 16 bytes
        const int d = item >> 2, slot = item & 3;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (fast) {
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                w[i >> 2] = e4m3_codes4(tile[vt_key(slot * 16 + i)][d], tile[vt_key(slot * 16 + i + 1)][d],
                                        tile[vt_key(slot * 16 + i + 2)][d], tile[vt_key(slot * 16 + i + 3)][d], r);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                w[i >> 2] |= e4m3_code(tile[vt_key(slot * 16 + i)][d] / sc) << (8 * (i & 3));
        }
        *reinterpret_cast<u32x4*>(vt + ((int64_t)head * 128 + d) * n_pad + t * 64 + slot * 16) =
            (u32x4){w[0], w[1], w[2], w[3]};
    }
}

__global__ void finalize_scales(float* a, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = scale_of(a[i]);
}

hipError_t launch_quantize_qkv_fp8(const void* q, const void* k, const void* v, int64_t ld, int32_t n, int32_t heads,
                                   void* q8, void* k8, void* vt, int64_t n_pad, float* sq, float* sk, float* sv,
                                   hipStream_t st) {
    const int hb = (heads + 255) / 256;
    zero_floats<<<hb, 256, 0, st>>>(sk, heads);
    zero_floats<<<hb, 256, 0, st>>>(sv, heads);
    const dim3 ag(heads, (n + 1023) / 1024);
    absmax_heads_kernel<<<ag, 256, 0, st>>>((const bf16*)k, ld, n, sk);
    absmax_heads_kernel<<<ag, 256, 0, st>>>((const bf16*)v, ld, n, sv);
    const int64_t groups = (int64_t)n * heads;
    quantize_q_kernel<<<(int)((groups * 16 + 255) / 256), 256, 0, st>>>((const bf16*)q, ld, n, heads, (uint8_t*)q8, sq);
    quantize_k_kernel<<<(int)((groups * 16 + 255) / 256), 256, 0, st>>>((const bf16*)k, ld, n, heads, sk,
                                                                       (uint8_t*)k8);
    quantize_vt_kernel<<<dim3((unsigned)(n_pad / 64), heads), 256, 0, st>>>((const bf16*)v, ld, n, sv, (uint8_t*)vt, n_pad);
    finalize_scales<<<hb, 256, 0, st>>>(sk, heads);
    finalize_scales<<<hb, 256, 0, st>>>(sv, heads);
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(bool bf, const void* x, int64_t ldx, int32_t n, int32_t K, void* q, int64_t ldq,
                               float* scales, hipStream_t st) {
    const int blocks = (n + 3) / 4;
    const int vpl = (K / 8 + 63) / 64;                 // bf16 vectors per lane of a row
#define H3_Q8ROWS(V) \
    quantize_fp8_rows_kernel<V><<<blocks, 256, 0, st>>>((const bf16*)x, ldx, n, K, (uint8_t*)q, ldq, scales)
    if (bf && vpl <= 4) H3_Q8ROWS(4);
    else if (bf && vpl <= 8) H3_Q8ROWS(8);
    else if (bf && vpl <= 11) H3_Q8ROWS(11);
    else if (bf && vpl <= 14) H3_Q8ROWS(14);
    else if (bf && vpl <= 16) H3_Q8ROWS(16);
    else if (bf && vpl <= 22) H3_Q8ROWS(22);
    else if (bf && vpl <= 28) H3_Q8ROWS(28);
    else if (bf)
        quantize_fp8_kernel<bf16><<<blocks, 256, 0, st>>>((const bf16*)x, ldx, n, K, (uint8_t*)q, ldq, scales);
    else
        quantize_fp8_kernel<float><<<blocks, 256, 0, st>>>((const float*)x, ldx, n, K, (uint8_t*)q, ldq, scales);
#undef H3_Q8ROWS
    return hipGetLastError();
}

}  // namespace h3
