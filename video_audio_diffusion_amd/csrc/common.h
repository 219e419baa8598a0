// Device-side helpers shared by the libh3blk kernels (gfx950 only).
#pragma once
#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- intervals
// Interval table passed by value in the kernel arguments.  Intervals are
// sorted, contiguous and cover [0, n_tok) (checked on the host), so the
// interval of token i is the last one whose start is <= i.
constexpr int kMaxSegs = 64;
struct SegDev {
    int32_t start, mod_set, HW, W, H, t0, h0, w0;
};
struct SegTable {
    int32_t n;
    int32_t pad;
    SegDev s[kMaxSegs];
};

// One fp32 coefficient per interval, passed by value with the table.
struct SegCoef {
    float c[kMaxSegs];
};

__device__ __forceinline__ int find_seg(const SegTable& tab, int32_t i) {
    int k = 0;
    for (int j = 1; j < tab.n; ++j)
        if (tab.s[j].start <= i) k = j;
    return k;
}

// ---------------------------------------------------------------- 16-byte vectors
// A "vector" is 16 bytes of a row: 8 bf16 or 4 fp32, widened to fp32 in
// registers.  Stores round fp32 -> bf16 to nearest even (v_cvt_pk_bf16_f32).
template <typename T> struct Vec;

template <> struct Vec<bf16> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void load(const void* p, float* f) {
        u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void store(void* p, const float* f) {
        u32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x2 b = __builtin_convertvector((f32x2){f[2 * i], f[2 * i + 1]}, bf16x2);
            u[i] = __builtin_bit_cast(uint32_t, b);
        }
        *reinterpret_cast<u32x4*>(p) = u;
    }
};

template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void load(const void* p, float* f) {
        f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = v[i];
    }
    __device__ __forceinline__ static void store(void* p, const float* f) {
        *reinterpret_cast<f32x4*>(p) = (f32x4){f[0], f[1], f[2], f[3]};
    }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------- reductions
// Sum over aligned groups of WIDTH lanes by the xor butterfly (masks
// WIDTH/2, ..., 1), every lane ending with its group's total.  For WIDTH 16
// the steps are DPP moves inside each 16-lane row instead of LDS permutes:
// row_ror:8 is lane ^ 8; after that step the values are symmetric under
// ^ 8, so row_ror:4 delivers lane ^ 4's value; quad_perm gives ^ 2 and ^ 1.
// The same pairs are added in the same order, so the sums are identical.
template <int WIDTH>
__device__ __forceinline__ float sum_lanes(float v) {
    if constexpr (WIDTH == 16) {
        auto dpp = [](float x, auto ctrl) __attribute__((always_inline)) {
            return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                      decltype(ctrl)::value, 0xF, 0xF, true));
        };
        v += dpp(v, std::integral_constant<int, 0x128>{});   // row_ror:8
        v += dpp(v, std::integral_constant<int, 0x124>{});   // row_ror:4
        v += dpp(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
        v += dpp(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
        return v;
    } else {
#pragma unroll
        for (int m = WIDTH / 2; m > 0; m >>= 1) v += __shfl_xor(v, m, kWave);
        return v;
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- buffer loads
// Raw buffer resource over [base, base + bytes): loads at or past `bytes`
// return zeros, which is how tiles that run past the last row are padded.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt immediate: at most n vector-memory operations of this wavefront
// outstanding and, with lgkm0, no LDS operation outstanding (the expcnt
// field is left unconstrained).
template <int n, bool lgkm0>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((((n >> 4) & 3) << 14) | ((lgkm0 ? 0 : 0xF) << 8) | (0x7 << 4) | (n & 15));
}

// s_waitcnt immediate: at most vm vector-memory and lgkm LDS operations of
// this wavefront outstanding.
template <int vm, int lgkm>
__device__ __forceinline__ void wait_cnt() {
    static_assert(vm >= 0 && vm < 64 && lgkm >= 0 && lgkm < 16, "count range");
    __builtin_amdgcn_s_waitcnt((((vm >> 4) & 3) << 14) | (lgkm << 8) | (0x7 << 4) | (vm & 15));
}

#define H3_LDS(p) ((__attribute__((address_space(3))) void*)(p))

}  // namespace h3
