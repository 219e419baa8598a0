// C = A . W^T on MFMA for the four projections of the H3 block.
//
// A [M][K] and W [N][K] are both K-contiguous, which is exactly the operand
// layout of the 32x32 MFMA: lane l supplies row (l % 32) and a 16-byte run of
// k at offset (l / 32) * 16 bytes inside a 32-byte k-chunk.  So both operands
// are staged through LDS as [rows][128 bytes of k] tiles and read back as
// whole 16-byte vectors.
//
// Tile: 256 x 256 per workgroup, 4 wavefronts in a 2 x 2 layout, 128 x 128
// (4 x 4 MFMA blocks) per wavefront; 128 bytes of K per step (64 bf16 or 32
// fp32).  LDS is double-buffered (2 x 64 KB); the next K step is fetched into
// registers while the current one is multiplied.  LDS rows are XOR-swizzled
// in 16-byte chunks (chunk c of row r lives at c ^ (r & 7)) so that both the
// row-wise stores and the column-wise fragment reads hit distinct banks.
//
// Tiles are numbered so that consecutive workgroups on one XCD (hardware
// deals workgroups to the 8 XCDs round-robin) form GROUP_M x n blocks of the
// output: their A and W panels are then shared in that XCD's L2.
#include "launch.h"

namespace h3 {

template <typename T> struct GemmMfma;

template <> struct GemmMfma<bf16> {
    // one v_mfma_f32_32x32x16_bf16: 16 k per 32-byte chunk
    __device__ __forceinline__ static void mma(f32x16& acc, const u32x4& a, const u32x4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    __device__ __forceinline__ static void store(bf16* p, float v) { *p = (bf16)v; }
};

template <> struct GemmMfma<float> {
    // four v_mfma_f32_32x32x2_f32: lane group g holds k = 4g..4g+3 of the
    // 8-wide chunk, the j-th MFMA contracts k = j and k = 4 + j.
    __device__ __forceinline__ static void mma(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc,
                                                       0, 0, 0);
    }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};

constexpr int kBM = 256, kBN = 256, kRowBytes = 128, kGroupM = 8;
constexpr int kTileBytes = kBM * kRowBytes;   // 32 KB per operand per stage

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, int64_t lda,
                                                   const T* __restrict__ W, int64_t ldw,
                                                   T* __restrict__ C, int64_t ldc, int32_t M, int32_t N,
                                                   int32_t K, int32_t tiles_m, int32_t tiles_n) {
    constexpr int EPB = 16 / sizeof(T);                 // elements per 16-byte chunk
    constexpr int BK = kRowBytes / sizeof(T);           // elements of K per step
    __shared__ __attribute__((aligned(16))) char smem[2][2][kTileBytes];

    // ---- tile order: XCD-contiguous, then GROUP_M-grouped
    const int G = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = G >> 3, extra = G & 7;
    const int L = xcd * base + (xcd < extra ? xcd : extra) + local;
    const int group = kGroupM * tiles_n;
    const int first_m = (L / group) * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (L % group) % gm;
    const int tn = (L % group) / gm;
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global -> register staging: thread loads chunk (tid % 8) of rows tid/8 + 32 i
    const int ld_chunk = tid & 7, ld_row = tid >> 3;
    const char* a_src[8];
    const char* w_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t ra = m0 + ld_row + 32 * i;
        ra = ra < M ? ra : M - 1;                      // clamp: rows past M are never stored
        int rw = n0 + ld_row + 32 * i;
        rw = rw < N ? rw : N - 1;
        a_src[i] = reinterpret_cast<const char*>(A + ra * lda) + ld_chunk * 16;
        w_src[i] = reinterpret_cast<const char*>(W + (int64_t)rw * ldw) + ld_chunk * 16;
    }
    u32x4 sa[8], sw[8];
    auto fetch = [&](int kstep) {
        const int off = kstep * kRowBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sa[i] = *reinterpret_cast<const u32x4*>(a_src[i] + off);
            sw[i] = *reinterpret_cast<const u32x4*>(w_src[i] + off);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = ld_row + 32 * i;
            *reinterpret_cast<u32x4*>(&smem[buf][0][swz(r, ld_chunk)]) = sa[i];
            *reinterpret_cast<u32x4*>(&smem[buf][1][swz(r, ld_chunk)]) = sw[i];
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

    const int nk = K / BK;
    fetch(0);
    stash(0);
    __syncthreads();
    const int frow = lane & 31, fhalf = lane >> 5;
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) fetch(ks + 1);
        const char* As = smem[buf][0];
        const char* Ws = smem[buf][1];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int chunk = kk * 2 + fhalf;
            u32x4 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = *reinterpret_cast<const u32x4*>(As + swz(wm * 128 + i * 32 + frow, chunk));
                bfr[i] = *reinterpret_cast<const u32x4*>(Ws + swz(wn * 128 + i * 32 + frow, chunk));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) GemmMfma<T>::mma(acc[i][j], af[i], bfr[j]);
        }
        if (ks + 1 < nk) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: accumulator (lane, r) -> row 8(r/4) + 4(lane/32) + r%4, col lane%32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 128 + j * 32 + frow;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
                if (row < M) GemmMfma<T>::store(C + row * ldc + col, acc[i][j][r]);
            }
        }
    }
    (void)EPB;
}

hipError_t launch_gemm(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                       int64_t ldc, int64_t M, int32_t N, int32_t K, hipStream_t st) {
    const int tiles_m = (int)((M + kBM - 1) / kBM);
    const int tiles_n = (N + kBN - 1) / kBN;
    const int grid = tiles_m * tiles_n;
    if (bf)
        gemm_kernel<bf16><<<grid, 256, 0, st>>>((const bf16*)A, lda, (const bf16*)W, ldw, (bf16*)C, ldc,
                                                (int32_t)M, N, K, tiles_m, tiles_n);
    else
        gemm_kernel<float><<<grid, 256, 0, st>>>((const float*)A, lda, (const float*)W, ldw, (float*)C,
                                                 ldc, (int32_t)M, N, K, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace h3
