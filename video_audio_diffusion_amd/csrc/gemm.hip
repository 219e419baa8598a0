// C = A . W^T on MFMA for the four projections of the H3 block.
//
// A [M][K] and W [N][K] are both K-contiguous, which is exactly the operand
// layout of the 32x32 MFMA: lane l supplies row (l % 32) and a 16-byte run of
// k at offset (l / 32) * 16 bytes inside a 32-byte k-chunk.  So both operands
// are staged in LDS as [rows][128 bytes of k] tiles and read back as whole
// 16-byte vectors.
//
// Tile: 256 x 256 per workgroup, 4 wavefronts in a 2 x 2 layout, 128 x 128
// (4 x 4 MFMA blocks, 256 accumulator registers) per wavefront; 64 bytes of
// K per step (32 bf16 or 16 fp32).  Each step's A and W tiles are copied from
// global memory straight into LDS by buffer->LDS loads into a 4-stage ring
// (128 KB), so the copies of the next three steps are in flight while a
// step is multiplied; the buffer resources stop at row M (N), so tiles that
// run past the end are padded with zeros.  Fragments are double-buffered in
// registers per 32-byte k-chunk: the reads of the next chunk are issued
// before the current chunk's 16 MFMAs, so LDS latency hides under them.
//
// LDS rows (64 bytes) are XOR-swizzled in 16-byte chunks: chunk c of row r
// lives at c ^ ((r >> 2) & 3), so the 16 rows of a half-wavefront fragment
// read land on 16 distinct 16-byte slots of the 256-byte bank window.
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

constexpr int kBM = 256, kBN = 256, kGroupM = 8;
constexpr int kRowBytes = 64;                  // bytes of K per step and tile row
constexpr int kStages = 4;                     // LDS ring depth: 3 steps of lookahead
constexpr int kTileBytes = kBM * kRowBytes;    // 16 KB per operand per stage
constexpr int kPieces = kTileBytes / 1024 / 4; // 1 KB copies per wavefront per operand

// s_waitcnt immediate: at most n vector-memory operations of this wavefront
// outstanding and, with lgkm0, no LDS operation outstanding (the expcnt
// field is left unconstrained).
template <int n, bool lgkm0>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((((n >> 4) & 3) << 14) | ((lgkm0 ? 0 : 0xF) << 8) | (0x7 << 4) | (n & 15));
}

// Copy this wavefront's quarter (64 rows) of one operand's k-step tile into
// LDS: kPieces pieces of 1 KB (16 rows each); lane offsets precomputed in
// voff, koff = byte offset of the k-step inside a row.
__device__ __forceinline__ void copy_operand(char* lds, int wave, const void* base, uint32_t bytes,
                                             const uint32_t* voff, uint32_t koff) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base, bytes);
#pragma unroll
    for (int j = 0; j < kPieces; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, H3_LDS(lds + (wave * kPieces + j) * 1024), 16, voff[j], koff, 0,
                                                 0);
}

template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, int64_t lda,
                                                   const T* __restrict__ W, int64_t ldw,
                                                   T* __restrict__ C, int64_t ldc, int32_t M, int32_t N,
                                                   int32_t K, int32_t tiles_m, int32_t tiles_n) {
    constexpr int ES = sizeof(T);
    constexpr int BK = kRowBytes / ES;                  // elements of K per step
    constexpr int KCH = kRowBytes / 32;                 // 32-byte MFMA k-chunks per step
    // stage s: A tile at ring + 2 s kTileBytes, W tile right after it
    __shared__ __attribute__((aligned(1024))) char ring[kStages * 2 * kTileBytes];

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
    //      64 wave + 16 j + lane / 4; LDS slot lane % 4 of the row gets chunk
    //      (lane % 4) ^ ((row >> 2) & 3)
    const uint32_t ldab = (uint32_t)(lda * ES), ldwb = (uint32_t)(ldw * ES);
    uint32_t va[kPieces], vw[kPieces];
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
        const int row = 64 * wave + 16 * j + (lane >> 2);
        const uint32_t c = (uint32_t)((lane & 3) ^ ((row >> 2) & 3));
        va[j] = (uint32_t)row * ldab + c * 16;
        vw[j] = (uint32_t)row * ldwb + c * 16;
    }
    const uint32_t bytes_a = (uint32_t)(M - m0 < kBM ? M - m0 : kBM) * ldab;
    const uint32_t bytes_w = (uint32_t)(N - n0 < kBN ? N - n0 : kBN) * ldwb;
    const T* a_base = A + (int64_t)m0 * lda;
    const T* w_base = W + (int64_t)n0 * ldw;
    auto copy_step = [&](int ks) {
        char* st = ring + (ks % kStages) * 2 * kTileBytes;
        copy_operand(st, wave, a_base, bytes_a, va, (uint32_t)ks * kRowBytes);
        copy_operand(st + kTileBytes, wave, w_base, bytes_w, vw, (uint32_t)ks * kRowBytes);
    };

    // ---- fragment offsets: row (32 i + frow) of the wave's 128-row panel,
    //      chunk 2 kk + fhalf; (row >> 2) & 3 depends on frow only
    const int frow = lane & 31, fhalf = lane >> 5;
    uint32_t fo[KCH];
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk)
        fo[kk] = (uint32_t)(frow * kRowBytes + (((2 * kk + fhalf) ^ ((frow >> 2) & 3)) << 4));
    const int a_panel = wm * 128 * kRowBytes, w_panel = kTileBytes + wn * 128 * kRowBytes;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

    // Fragments are double-buffered per 32-byte k-chunk: slot kk holds chunk
    // kk of a step (4 A + 4 W 16-byte reads), and the next chunk's reads are
    // issued before the current chunk's 16 MFMAs.
    static_assert(KCH == 2, "one register slot per k-chunk of a step");
    u32x4 fa[KCH][4], fw[KCH][4];
    auto read_chunk = [&](int ks, int kk, u32x4 (&a)[4], u32x4 (&w)[4]) {
        const char* st = ring + (ks % kStages) * 2 * kTileBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = *reinterpret_cast<const u32x4*>(st + a_panel + i * 32 * kRowBytes + fo[kk]);
            w[i] = *reinterpret_cast<const u32x4*>(st + w_panel + i * 32 * kRowBytes + fo[kk]);
        }
    };
    auto mfma_chunk = [&](const u32x4 (&a)[4], const u32x4 (&w)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) GemmMfma<T>::mma(acc[i][j], a[i], w[j]);
    };
    // Wait until step s has landed in LDS for every wavefront and this
    // wavefront's reads of the step before are done: at most the copies of
    // steps s+1, s+2 (already issued) may still be outstanding.  Then the
    // stage of step s-1 is free for the copy of step s+3.  A plain s_barrier
    // is used: __syncthreads() would also wait for the later copies.
    auto step_ready = [&](int s, int nk) {
        if (s + 2 < nk) wait_vm<4 * kPieces, true>();
        else if (s + 1 < nk) wait_vm<2 * kPieces, true>();
        else wait_vm<0, true>();
        __builtin_amdgcn_s_barrier();
        if (s + kStages - 1 < nk) copy_step(s + kStages - 1);
    };

    const int nk = K / BK;
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < nk) copy_step(s);
    step_ready(0, nk);
    read_chunk(0, 0, fa[0], fw[0]);
    for (int ks = 0; ks < nk; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        // Chunk 0's reads were issued a whole chunk of MFMAs ago; retiring
        // them here keeps at most 8 LDS reads in flight (the counter holds 15).
        wait_vm<63, true>();
        read_chunk(ks, 1, fa[1], fw[1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_chunk(fa[0], fw[0]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < nk) {
            step_ready(ks + 1, nk);
            read_chunk(ks + 1, 0, fa[0], fw[0]);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_chunk(fa[1], fw[1]);
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
