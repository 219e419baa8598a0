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

hipError_t launch_quantize_fp8(bool bf, const void* x, int64_t ldx, int32_t n, int32_t K, void* q, int64_t ldq,
                               float* scales, hipStream_t st) {
    const int blocks = (n + 3) / 4;
    if (bf)
        quantize_fp8_kernel<bf16><<<blocks, 256, 0, st>>>((const bf16*)x, ldx, n, K, (uint8_t*)q, ldq, scales);
    else
        quantize_fp8_kernel<float><<<blocks, 256, 0, st>>>((const float*)x, ldx, n, K, (uint8_t*)q, ldq, scales);
    return hipGetLastError();
}

}  // namespace h3
