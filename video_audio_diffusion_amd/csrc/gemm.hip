// C = A . W^T on MFMA for the four projections of the H3 block.
//
// A [M][K] and W [N][K] are both K-contiguous, which is exactly the operand
// layout of the 32x32 MFMA: lane l supplies row (l % 32) and a 16-byte run of
// k at offset (l / 32) * 16 bytes inside a 32-byte k-chunk.  So both operands
// are staged in LDS as [rows][128 bytes of k] tiles and read back as whole
// 16-byte vectors.
//
// Tile: 256 x 256 per workgroup, 4 wavefronts in a 2 x 2 layout, 128 x 128
// (4 x 4 MFMA blocks, 256 accumulator registers) per wavefront; 128 bytes of
// K per step (64 bf16 or 32 fp32).  Each step's A and W tiles are copied from
// global memory straight into LDS by buffer->LDS loads into one of two LDS
// buffer pairs, so the copy of step k+1 runs while step k is multiplied; the
// buffer resources stop at row M (N), so tiles that run past the end are
// padded with zeros.  Inside a step all fragments are read from LDS before
// the step's 64 MFMAs are issued.
//
// LDS rows are XOR-swizzled in 16-byte chunks: chunk c of row r lives at
// c ^ ((r >> 1) & 7), so any 16 consecutive rows read at one chunk -- a
// fragment read -- and any two rows written whole land on 16 distinct
// 16-byte slots of the 256-byte bank window.
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

// Copy this wavefront's quarter (64 rows) of one operand's k-step tile into
// LDS: 8 pieces of 1 KB (8 rows each); lane offsets precomputed in voff,
// koff = byte offset of the k-step inside a row.
__device__ __forceinline__ void copy_operand(char* lds, int wave, const void* base, uint32_t bytes,
                                             const uint32_t* voff, uint32_t koff) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base, bytes);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, H3_LDS(lds + (wave * 8 + j) * 1024), 16, voff[j], koff, 0, 0);
}

template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, int64_t lda,
                                                   const T* __restrict__ W, int64_t ldw,
                                                   T* __restrict__ C, int64_t ldc, int32_t M, int32_t N,
                                                   int32_t K, int32_t tiles_m, int32_t tiles_n) {
    constexpr int ES = sizeof(T);
    constexpr int BK = kRowBytes / ES;                  // elements of K per step
    __shared__ __attribute__((aligned(1024))) char sa0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sw0[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sa1[kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sw1[kTileBytes];

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
    const int m0 = tm * kBM;
    const int n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // ---- copy offsets: piece j of this wavefront holds tile rows
    //      64 wave + 8 j + lane / 8; LDS slot lane % 8 of the row gets chunk
    //      (lane % 8) ^ ((row >> 1) & 7)
    const uint32_t ldab = (uint32_t)(lda * ES), ldwb = (uint32_t)(ldw * ES);
    uint32_t va[8], vw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = 64 * wave + 8 * j + (lane >> 3);
        const uint32_t c = (uint32_t)((lane & 7) ^ ((row >> 1) & 7));
        va[j] = (uint32_t)row * ldab + c * 16;
        vw[j] = (uint32_t)row * ldwb + c * 16;
    }
    const uint32_t bytes_a = (uint32_t)(M - m0 < kBM ? M - m0 : kBM) * ldab;
    const uint32_t bytes_w = (uint32_t)(N - n0 < kBN ? N - n0 : kBN) * ldwb;
    const T* a_base = A + (int64_t)m0 * lda;
    const T* w_base = W + (int64_t)n0 * ldw;

    // ---- fragment offsets: row (32 i + frow) of the wave's 128-row panel,
    //      chunk 2 kk + fhalf; (row >> 1) & 7 depends on frow only
    const int frow = lane & 31, fhalf = lane >> 5;
    uint32_t fo[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fo[kk] = (uint32_t)(frow * kRowBytes + (((2 * kk + fhalf) ^ ((frow >> 1) & 7)) << 4));
    const int a_panel = wm * 128 * kRowBytes, w_panel = wn * 128 * kRowBytes;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

    // One k-step from LDS: all 32 fragment reads first (LDS returns them in
    // order, so the MFMAs of chunk kk only wait for chunk kk's reads), then
    // 4 k-chunks x 16 MFMAs.
    auto compute = [&](const char* As, const char* Ws) {
        u32x4 af[4][4], bw[4][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[kk][i] = *reinterpret_cast<const u32x4*>(As + a_panel + i * 32 * kRowBytes + fo[kk]);
                bw[kk][i] = *reinterpret_cast<const u32x4*>(Ws + w_panel + i * 32 * kRowBytes + fo[kk]);
            }
        __builtin_amdgcn_sched_barrier(0);   // keep every read ahead of the MFMAs
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) GemmMfma<T>::mma(acc[i][j], af[kk][i], bw[kk][j]);
    };

    const int nk = K / BK;
    copy_operand(sa0, wave, a_base, bytes_a, va, 0);
    copy_operand(sw0, wave, w_base, bytes_w, vw, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        // buffer pair ks & 1 holds this step; the copy of step ks + 1 goes to the other
        const bool odd = ks & 1;
        if (ks + 1 < nk) {
            copy_operand(odd ? sa0 : sa1, wave, a_base, bytes_a, va, (uint32_t)(ks + 1) * kRowBytes);
            copy_operand(odd ? sw0 : sw1, wave, w_base, bytes_w, vw, (uint32_t)(ks + 1) * kRowBytes);
        }
        compute(odd ? sa1 : sa0, odd ? sw1 : sw0);
        __builtin_amdgcn_sched_barrier(0);   // the wait below must not rise above the MFMAs
        __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of step ks + 1 have landed
        __syncthreads();                 // ... everyone's, and step ks's buffers are free
    }

    // ---- epilogue: accumulator (lane, r) -> row 8(r/4) + 4(lane/32) + r%4, col lane%32
    const bool full = m0 + kBM <= M && n0 + kBN <= N;
    T* cbase = C + (int64_t)(m0 + wm * 128 + 4 * fhalf) * ldc + n0 + wn * 128 + frow;
    if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    GemmMfma<T>::store(cbase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32,
                                       acc[i][j][r]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn * 128 + j * 32 + frow;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
                    if (row < M && col < N)
                        GemmMfma<T>::store(cbase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32,
                                           acc[i][j][r]);
                }
            }
    }
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
