// C = A . W^T on MFMA for the four projections of the H3 block.
//
// A [M][K] and W [N][K] are both K-contiguous, which is exactly the operand
// layout of the MFMAs: for 32x32 lane l supplies row (l % 32) and a 16-byte
// run of k at offset (l / 32) * 16 bytes inside a 32-byte k-chunk; for
// 16x16x32 (the bf16 default) row (l % 16) and the 16 bytes at (l / 16) * 16
// of a 64-byte chunk.  So both operands are staged in LDS as [rows][128 bytes
// of k] tiles and read back as whole 16-byte vectors.
//
// Tile: 256 x 256 per workgroup.  With 8 wavefronts (two per SIMD, so one
// can issue MFMAs while the other waits) each owns a 128 x 64 panel (4 x 2
// blocks of 32x32, or 8 x 4 of 16x16).  Each k-step's A and W tiles (ROWB bytes of K per row) are
// staged in a ring of LDS stages; fragments are double-buffered in
// registers per 32-byte k-chunk: the reads of the next chunk are issued
// before the current chunk's MFMAs.  Ways of filling the ring:
//   * bf16 with K up to 8192 (gemm_mainloop_dma16 on 16x16x32 MFMAs):
//     buffer -> LDS DMA, the copies of step s+2 spread over the regions
//     after step s's barrier;
//   * bf16 with larger K (gemm_mainloop_staged16 on 16x16x32 MFMAs, or
//     gemm_mainloop_staged on 32x32x16) and fp8 (gemm_mainloop_staged_fp8
//     on 32x32x64): global -> registers -> LDS, spread over the step, each
//     load landing a step before its LDS write;
//   * fp32 (and fp8 when H3_GEMM_FP8_STAGED is 0; the ring loop in
//     gemm_kernel): buffer -> LDS DMA, one step's copies issued at the
//     step's barrier.
// The buffer resources stop at row M (N), so tiles that run past the end are
// padded with zeros.
//
// LDS rows are XOR-swizzled in 16-byte chunks so that the 16 rows of a
// half-wavefront fragment read fall on 16 distinct 16-byte slots of the
// 256-byte bank window (see GemmGeom::slot).
//
// Tiles are numbered so that consecutive workgroups on one XCD (hardware
// deals workgroups to the 8 XCDs round-robin) form GROUP_M x n blocks of the
// output: their A and W panels are then shared in that XCD's L2.
#include "launch.h"

#include <cstring>
#include <type_traits>

namespace h3 {

// Launch configuration.  bf16: 128 bytes of K per step, two LDS stages,
// eight wavefronts of 128 x 64 on 16x16x32 MFMAs, one memory instruction
// issued beside each MFMA, XCD groups 4 tiles high (measured best on the
// block's four projection shapes; four wavefronts of 128 x 128, one per
// SIMD, ran about 4 % slower).  The ring is filled by LDS DMA up to
// K = H3_GEMM_BF16_DMA_MAX_K and through registers beyond: at the block's
// shapes the DMA loop was 2.8-4.3 % faster at K 5376 and 7168, and the
// register-staged one 0-2.6 % faster at K 14336.  fp8: the register-staged
// ring on 32x32x64 MFMAs, groups 2 high.  fp32: the LDS-DMA ring with the
// H3_GEMM_* configuration, groups 2 high.  The macros only exist so that other configurations of the
// same templates can be built and timed.
#ifndef H3_GEMM_ROWB
#define H3_GEMM_ROWB 128
#endif
#ifndef H3_GEMM_STAGES
#define H3_GEMM_STAGES 2
#endif
#ifndef H3_GEMM_GROUP_M
#define H3_GEMM_GROUP_M 2
#endif
#ifndef H3_GEMM_WAVES
#define H3_GEMM_WAVES 8
#endif
#ifndef H3_GEMM_BF16_STAGED
#define H3_GEMM_BF16_STAGED 1
#endif
#ifndef H3_GEMM_STAGED_INTERLEAVE
#define H3_GEMM_STAGED_INTERLEAVE 1
#endif
#ifndef H3_GEMM_BF16_WAVES
#define H3_GEMM_BF16_WAVES 8
#endif
#ifndef H3_GEMM_BF16_GROUP_M
#define H3_GEMM_BF16_GROUP_M 4
#endif
#ifndef H3_GEMM_MFMA16
#define H3_GEMM_MFMA16 1
#endif
#ifndef H3_GEMM_BF16_DMA_MAX_K
#define H3_GEMM_BF16_DMA_MAX_K 8192
#endif
#ifndef H3_GEMM_FP8_STAGED
#define H3_GEMM_FP8_STAGED 1
#endif

template <typename T> struct GemmMfma;

template <> struct GemmMfma<bf16> {
    // one v_mfma_f32_32x32x16_bf16: 16 k per 32-byte chunk
    __device__ __forceinline__ static void mma(f32x16& acc, const u32x4& a, const u32x4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    __device__ __forceinline__ static void store(bf16* p, float v) { *p = (bf16)v; }
    __device__ __forceinline__ static float load(const bf16* p) { return (float)*p; }
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
    __device__ __forceinline__ static float load(const float* p) { return *p; }
};

// Operand policies: bytes of K one MFMA contracts per row (one k-chunk), the
// fragment one lane reads for it (16 bytes at offset (lane / 32) * 16 of a
// 32-byte chunk, or 32 bytes at (lane / 32) * 32 of a 64-byte fp8 chunk --
// the same place in A and in W, so the K order inside a chunk cancels) and
// the MFMA.  fp8 is OCP e4m3 (v_mfma_f32_32x32x64_f8f6f4, formats 0/0,
// unit scales).
using fp8 = uint8_t;
template <typename T> struct GemmOp;
template <> struct GemmOp<bf16> {
    static constexpr int CHUNK = 32;
    using Frag = u32x4;
    __device__ __forceinline__ static Frag read(const char* lo, const char* hi) {
        (void)hi;
        return *reinterpret_cast<const u32x4*>(lo);
    }
    __device__ __forceinline__ static void mma(f32x16& acc, const Frag& a, const Frag& b) { GemmMfma<bf16>::mma(acc, a, b); }
};
template <> struct GemmOp<float> {
    static constexpr int CHUNK = 32;
    using Frag = u32x4;
    __device__ __forceinline__ static Frag read(const char* lo, const char* hi) {
        (void)hi;
        return *reinterpret_cast<const u32x4*>(lo);
    }
    __device__ __forceinline__ static void mma(f32x16& acc, const Frag& a, const Frag& b) { GemmMfma<float>::mma(acc, a, b); }
};
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
template <> struct GemmOp<fp8> {
    static constexpr int CHUNK = 64;
    struct Frag { u32x4 lo, hi; };
    __device__ __forceinline__ static Frag read(const char* lo, const char* hi) {
        return Frag{*reinterpret_cast<const u32x4*>(lo), *reinterpret_cast<const u32x4*>(hi)};
    }
    __device__ __forceinline__ static void mma(f32x16& acc, const Frag& a, const Frag& b) {
        const i32x8 av = {(int32_t)a.lo[0], (int32_t)a.lo[1], (int32_t)a.lo[2], (int32_t)a.lo[3],
                          (int32_t)a.hi[0], (int32_t)a.hi[1], (int32_t)a.hi[2], (int32_t)a.hi[3]};
        const i32x8 bv = {(int32_t)b.lo[0], (int32_t)b.lo[1], (int32_t)b.lo[2], (int32_t)b.lo[3],
                          (int32_t)b.hi[0], (int32_t)b.hi[1], (int32_t)b.hi[2], (int32_t)b.hi[3]};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
    }
};

constexpr int kBM = 256, kBN = 256;

// Tile geometry for ROWB bytes of K per step (64 or 128) and a STAGES-deep
// LDS ring.  Rows of ROWB bytes hold CPR 16-byte chunks; 256 / ROWB rows
// share one 256-byte bank window, so chunk c of row r is stored at
// c ^ ((r / (256 / ROWB)) % CPR): the 16 rows of a half-wavefront fragment
// read then fall on 16 distinct 16-byte slots.
template <int ROWB, int STAGES, int NWAVES, int CHUNK = 32>
struct GemmGeom {
    static constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
    static constexpr int RPW = 256 / ROWB;               // rows per bank window
    static constexpr int TILE = kBM * ROWB;              // bytes per operand per stage
    static constexpr int PIECES = TILE / 1024 / NWAVES;  // 1 KB copies per wavefront per operand
    static constexpr int NJ = NWAVES == 4 ? 4 : 2;        // 32-column W blocks per wavefront
    static constexpr int ROWS_PER_WAVE = kBM / NWAVES;   // tile rows each wavefront copies
    static constexpr int ROWS_PER_PIECE = 1024 / ROWB;
    static constexpr int KCH = ROWB / CHUNK;             // MFMA k-chunks per step
    static_assert(STAGES >= 2 && STAGES * 2 * TILE <= 160 * 1024, "LDS ring too large");
    __device__ static int slot(int row, int c) { return c ^ ((row / RPW) % CPR); }
};

// Copy this wavefront's share of one operand's k-step tile into LDS: PIECES
// pieces of 1 KB; lane offsets precomputed in voff, koff = byte offset of the
// k-step inside a row.
template <int PIECES>
__device__ __forceinline__ void copy_operand(char* lds, int wave, const void* base, uint32_t bytes,
                                             const uint32_t* voff, uint32_t koff) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base, bytes);
#pragma unroll
    for (int j = 0; j < PIECES; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, H3_LDS(lds + (wave * PIECES + j) * 1024), 16, voff[j], koff, 0,
                                                 0);
}

// One 1 KB piece by buffer -> LDS DMA: lane l's 16 bytes at voff + soff of
// the buffer land at dst + 16 l.
__device__ __forceinline__ void dma_piece(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, H3_LDS(dst), 16, voff, soff, 0, 0);
}

// Epilogues.  EpiStore writes C.  EpiGate writes out = x + gate * C with
// the modality gate of each row's interval (the block's gated residual, so
// the projection output never goes to memory).  EpiSwiglu takes W with its
// rows interleaved in 64-row units -- rows 64u..64u+31 the gate rows
// 32u..32u+31, rows 64u+32..64u+63 the matching up rows -- so every
// wavefront's two 32-column blocks hold a gate column and its up column in
// the same lanes, and writes h = SiLU(gate) * up at half the width.
struct EpiStore {};
struct EpiGate {
    const void* x;          // [M][N], row stride ldc (may equal C)
    const float* mod;       // [n_sets][6][N]
    int32_t chunk;          // gate chunk index 3 * branch + 2
    SegTable tab;
};
struct EpiSwiglu {};
// EpiQkRope: the QKV projection with the per-head RMSNorm and the 3-D RoPE
// of q and k applied before the store.  Columns [0, q_cols) are q heads and
// [q_cols, 2 q_cols) k heads, HD wide; later columns (v) are stored as
// computed.  q_cols is a multiple of the 256-column tile, so a tile is all
// q, all k or all v.  A q or k tile is first rounded to the output type into
// LDS -- the values a separate norm pass would read back from memory --
// then each (row, head) is scaled by 1 / sqrt(mean square + eps) and the gain,
// and pair p (elements 2p, 2p+1 of a head) turns by fr[p] * pos revolutions,
// pos being the row's position on axis[p].  fr is held as two floats and
// the product reduced to about [-1/2, 1/2] revolutions with an fma, so the
// angle keeps about 2^-40 revolutions of precision at any position (a plain
// fp32 product loses 2^-24 of pos * fr: 1e-4 rad at position 5000); sine and
// cosine are the hardware's for bf16 output and the precise sincospif for
// fp32.
template <int HD>
struct EpiQkRope {
    static constexpr int kHd = HD;
    const float* gq;        // [HD] gain of the q heads (null: 1)
    const float* gk;        // [HD] gain of the k heads
    float eps;
    int32_t q_cols;         // heads * HD
    float fr_hi[HD / 2];    // revolutions per unit of position of pair p,
    float fr_lo[HD / 2];    //   as an fp32 pair: fr_hi + fr_lo
    int8_t axis[HD / 2];    // 0 = t, 1 = h, 2 = w
    SegTable tab;
};
template <typename E> struct IsQkRope : std::false_type {};
template <int HD> struct IsQkRope<EpiQkRope<HD>> : std::true_type {};

// ---------------------------------------------------------------- register-staged ring (bf16)
// Same tile, two 64 KB LDS stages, swizzle and fragment layout as the ring
// loop (256 x 256, 128 bytes of K per step; 8 wavefronts of 128 x 64 or 4 of
// 128 x 128), but the tiles travel global -> registers -> LDS instead of by
// LDS DMA, spread over the step: in chunk kk of step s each wavefront
// writes a quarter of its 1 KB pieces of step s+1 (loaded during step s-1)
// into the stage of step s-1, which every wavefront finished reading before
// the barrier that opened step s, then loads the same pieces of step s+2
// into the same registers.  A load therefore has a whole step to land before
// its data is written, the loads reach the memory system at an even rate
// (issuing a step's loads in one burst at the barrier held every
// wavefront's MFMAs behind them), and the one barrier per step only waits
// for this wavefront's LDS reads and writes.
template <int NWAVES>
__device__ __forceinline__ void gemm_mainloop_staged(f32x16 (&acc)[4][NWAVES == 4 ? 4 : 2], char* ring,
                                                     const bf16* __restrict__ A, int64_t lda,
                                                     const bf16* __restrict__ W, int64_t ldw, int32_t M, int32_t N,
                                                     int32_t K, int m0, int n0, int wave, int lane) {
    constexpr int ROWB = 128, KCH = 4;
    using Geo = GemmGeom<ROWB, 2, NWAVES, 32>;
    constexpr int NJ = Geo::NJ;
    constexpr int TILE = Geo::TILE;                      // 32 KB per operand per stage
    constexpr int PIECES = Geo::PIECES;                  // 1 KB pieces per wavefront per operand (4 or 8)
    constexpr int NP = 2 * PIECES;                       // pieces per wavefront and step: A first, then W
    constexpr int PPC = NP / KCH;                        // pieces per chunk (2 or 4)
    static_assert((NWAVES == 8 && PIECES == 4) || (NWAVES == 4 && PIECES == 8), "staging layout");
    const int wm = NWAVES == 4 ? wave >> 1 : wave >> 2;
    const int wn = NWAVES == 4 ? wave & 1 : wave & 3;

    // piece j of this wavefront: tile rows 32 wave + 8 (j % 4) + lane / 8, its
    // 16-byte chunk (lane % 8) ^ swizzle, into LDS at the piece's 1 KB + 16 lane
    const uint32_t ldab = (uint32_t)(lda * 2), ldwb = (uint32_t)(ldw * 2);
    uint32_t voff[NP];
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
        const int row = Geo::ROWS_PER_WAVE * wave + Geo::ROWS_PER_PIECE * j + lane / Geo::CPR;
        const uint32_t c = (uint32_t)Geo::slot(row, lane % Geo::CPR);
        voff[j] = (uint32_t)row * ldab + c * 16;
        voff[PIECES + j] = (uint32_t)row * ldwb + c * 16;
    }
    const uint32_t bytes_a = (uint32_t)(M - m0 < kBM ? M - m0 : kBM) * ldab;
    const uint32_t bytes_w = (uint32_t)(N - n0 < kBN ? N - n0 : kBN) * ldwb;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A + (int64_t)m0 * lda, bytes_a);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + (int64_t)n0 * ldw, bytes_w);
    const int nk = K / 64;
    u32x4 stg[NP];
    auto load_piece = [&](int j, int ks) __attribute__((always_inline)) {
        stg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(j < PIECES ? ra : rw, voff[j],
                                                                                  (uint32_t)ks * ROWB, 0));
    };
    auto write_piece = [&](int j, int ks) __attribute__((always_inline)) {
        char* st = ring + (ks & 1) * 2 * TILE + (j < PIECES ? 0 : TILE) + (wave * PIECES + j % PIECES) * 1024;
        *reinterpret_cast<u32x4*>(st + lane * 16) = stg[j];
    };

    const int frow = lane & 31, fhalf = lane >> 5;
    uint32_t fo[KCH];
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk) fo[kk] = (uint32_t)(frow * ROWB + (Geo::slot(frow, 2 * kk + fhalf) << 4));
    const int a_panel = wm * 128 * ROWB, w_panel = TILE + wn * NJ * 32 * ROWB;
    u32x4 fa[2][4], fw[2][NJ];
    auto read_chunk = [&](int ks, int kk, u32x4 (&a)[4], u32x4 (&w)[NJ]) __attribute__((always_inline)) {
        const char* st = ring + (ks & 1) * 2 * TILE;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4*>(st + a_panel + i * 32 * ROWB + fo[kk]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) w[j] = *reinterpret_cast<const u32x4*>(st + w_panel + j * 32 * ROWB + fo[kk]);
    };
    // The step barrier as asm with a memory clobber, so that the compiler
    // keeps every LDS access on its side of it.
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: step 0 written to stage 0, step 1 in registers
#pragma unroll
    for (int j = 0; j < NP; ++j) load_piece(j, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) write_piece(j, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) load_piece(j, nk > 1 ? 1 : 0);
    wait_cnt<63, 0>();
    barrier();
    read_chunk(0, 0, fa[0], fw[0]);
#if H3_GEMM_STAGED_INTERLEAVE
    // One memory instruction beside each MFMA.  Chunks 0-2 of a step: the
    // next chunk's fragment reads first, then the piece writes and loads.
    // Chunk 3: the piece writes, the step barrier, the next step's chunk-0
    // reads, then the loads.
    constexpr int NM = 4 * NJ, NR = 4 + NJ;
    auto mfma_i = [&](int kk, int m) __attribute__((always_inline)) {
        GemmMfma<bf16>::mma(acc[m / NJ][m % NJ], fa[kk & 1][m / NJ], fw[kk & 1][m % NJ]);
    };
    // schedule groups: nops memory instructions of one kind (0 LDS read,
    // 1 LDS write, 2 global load), each after one of the MFMAs [mi, NM)
    auto groups = [&](int& mi, int nops, int kind) __attribute__((always_inline)) {
#pragma unroll
        for (int o = 0; o < nops; ++o) {
            if (mi < NM) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                ++mi;
            }
            if (kind == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else if (kind == 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };
    for (int ks = 0; ks < nk; ++ks) {
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk) {
            int mi = 0;
            if (kk + 1 < KCH) {
                read_chunk(ks, kk + 1, fa[(kk + 1) & 1], fw[(kk + 1) & 1]);
#pragma unroll
                for (int q = 0; q < PPC; ++q) write_piece(PPC * kk + q, ks + 1);
#pragma unroll
                for (int q = 0; q < PPC; ++q) load_piece(PPC * kk + q, ks + 2 < nk ? ks + 2 : nk - 1);
#pragma unroll
                for (int m = 0; m < NM; ++m) mfma_i(kk, m);
                groups(mi, NR, 0);
                groups(mi, PPC, 1);
                groups(mi, PPC, 2);
#pragma unroll
                for (int m = mi; m < NM; ++m) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                constexpr int M1 = NM / 4;      // MFMAs before the barrier
#pragma unroll
                for (int q = 0; q < PPC; ++q) write_piece(PPC * kk + q, ks + 1);
#pragma unroll
                for (int m = 0; m < M1; ++m) mfma_i(kk, m);
#pragma unroll
                for (int q = 0; q < PPC; ++q) {
                    if (q < M1) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                }
#pragma unroll
                for (int q = PPC; q < M1; ++q) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                // (after the last step the reads fetch a stage nobody uses:
                // the code stays branch-free, so one schedule covers it)
                wait_cnt<63, 0>();
                barrier();
                read_chunk(ks + 1, 0, fa[0], fw[0]);
#pragma unroll
                for (int q = 0; q < PPC; ++q) load_piece(PPC * kk + q, ks + 2 < nk ? ks + 2 : nk - 1);
#pragma unroll
                for (int m = M1; m < NM; ++m) mfma_i(kk, m);
                mi = M1;
                groups(mi, NR, 0);
                groups(mi, PPC, 2);
#pragma unroll
                for (int m = mi; m < NM; ++m) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
#else
    for (int ks = 0; ks < nk; ++ks) {
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk) {
            __builtin_amdgcn_sched_barrier(0);
            // pieces 2 kk, 2 kk + 1: step ks+1 to LDS, then step ks+2 loads.
            // Past the last step the loads repeat it and the writes go to a
            // stage nobody reads again: the code stays straight, so the
            // compiler waits for exactly the load each write needs.
#pragma unroll
            for (int q = 0; q < PPC; ++q) write_piece(PPC * kk + q, ks + 1);
#pragma unroll
            for (int q = 0; q < PPC; ++q) load_piece(PPC * kk + q, ks + 2 < nk ? ks + 2 : nk - 1);
            if (kk + 1 < KCH) {
                read_chunk(ks, kk + 1, fa[(kk + 1) & 1], fw[(kk + 1) & 1]);
            } else if (ks + 1 < nk) {
                // this wavefront's reads of step ks and writes of step ks+1
                // are complete; the barrier makes it so for all of them
                wait_cnt<63, 0>();
                barrier();
                read_chunk(ks + 1, 0, fa[0], fw[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) GemmMfma<bf16>::mma(acc[i][j], fa[kk & 1][i], fw[kk & 1][j]);
        }
    }
#endif
}

// ---------------------------------------------------------------- staged ring on 16x16x32 MFMAs (bf16)
// The same ring, pieces and barrier as gemm_mainloop_staged, with
// v_mfma_f32_16x16x32_bf16 (the same flops in twice as many MFMAs, which
// draw less power, so the part holds a higher clock).  Lane l supplies row
// (l % 16) of a 16-row block and the 16 bytes at (l / 16) * 16 of a 64-byte
// k-chunk, so a 128-byte step row holds two chunks.  A wavefront's 128-row
// A panel is 8 blocks and its W panel 2 NJ blocks; 16x16 block (ib, jb) is
// sub-block 2 (ib % 2) + (jb % 2) of the 32x32 block (ib / 2, jb / 2) of acc,
// four floats each (column l % 16, rows 4 (l / 16) .. + 3 of the sub-block).
//
// Each chunk is eight regions, one per A block ib: its 2 NJ MFMAs with
// memory instructions slotted between them.  A fragments rotate through one
// set of registers: A block ib of the next chunk is read in region ib + 1,
// after the last MFMA that uses the current one (block 7 in region 0 of the
// chunk that uses it); W fragments are double-buffered.  Chunk 0: W reads
// and piece writes in regions 0-3, loads in regions 4-7.  Chunk 1: the
// writes in regions 0-1, then the step barrier, then the next step's W
// reads and the loads in regions 2-5.
template <int NWAVES>
__device__ __forceinline__ void gemm_mainloop_staged16(f32x16 (&acc)[4][NWAVES == 4 ? 4 : 2], char* ring,
                                                       const bf16* __restrict__ A, int64_t lda,
                                                       const bf16* __restrict__ W, int64_t ldw, int32_t M, int32_t N,
                                                       int32_t K, int m0, int n0, int wave, int lane) {
    constexpr int ROWB = 128, KCH = 2;
    using Geo = GemmGeom<ROWB, 2, NWAVES, 64>;
    constexpr int NJ = Geo::NJ;
    constexpr int NB = 2 * NJ;                           // 16-column W blocks per wavefront
    constexpr int TILE = Geo::TILE;
    constexpr int PIECES = Geo::PIECES;
    constexpr int NP = 2 * PIECES;                       // pieces per wavefront and step: A first, then W
    constexpr int PPC = NP / KCH;                        // pieces per chunk (4 or 8)
    static_assert((NWAVES == 8 && PIECES == 4) || (NWAVES == 4 && PIECES == 8), "staging layout");
    static_assert(NB % 4 == 0 && PPC % 4 == 0, "region split");
    const int wm = NWAVES == 4 ? wave >> 1 : wave >> 2;
    const int wn = NWAVES == 4 ? wave & 1 : wave & 3;

    const uint32_t ldab = (uint32_t)(lda * 2), ldwb = (uint32_t)(ldw * 2);
    uint32_t voff[NP];
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
        const int row = Geo::ROWS_PER_WAVE * wave + Geo::ROWS_PER_PIECE * j + lane / Geo::CPR;
        const uint32_t c = (uint32_t)Geo::slot(row, lane % Geo::CPR);
        voff[j] = (uint32_t)row * ldab + c * 16;
        voff[PIECES + j] = (uint32_t)row * ldwb + c * 16;
    }
    const uint32_t bytes_a = (uint32_t)(M - m0 < kBM ? M - m0 : kBM) * ldab;
    const uint32_t bytes_w = (uint32_t)(N - n0 < kBN ? N - n0 : kBN) * ldwb;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A + (int64_t)m0 * lda, bytes_a);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + (int64_t)n0 * ldw, bytes_w);
    const int nk = K / 64;
    u32x4 stg[NP];
    auto load_piece = [&](int j, int ks) __attribute__((always_inline)) {
        stg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(j < PIECES ? ra : rw, voff[j],
                                                                                  (uint32_t)ks * ROWB, 0));
    };
    auto write_piece = [&](int j, int ks) __attribute__((always_inline)) {
        char* st = ring + (ks & 1) * 2 * TILE + (j < PIECES ? 0 : TILE) + (wave * PIECES + j % PIECES) * 1024;
        *reinterpret_cast<u32x4*>(st + lane * 16) = stg[j];
    };

    // fragment offset of chunk kc inside a 16-row block: the block's first
    // row is even and a multiple of 16, so the swizzle only depends on l % 16
    const int frow = lane & 15, fq = lane >> 4;
    uint32_t fo[KCH];
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) fo[kc] = (uint32_t)(frow * ROWB + (Geo::slot(frow, 4 * kc + fq) << 4));
    const int a_panel = wm * 128 * ROWB, w_panel = TILE + wn * NJ * 32 * ROWB;
    u32x4 fa[8], fw[2][NB];
    auto read_a = [&](int ks, int kc, int ib) __attribute__((always_inline)) {
        fa[ib] = *reinterpret_cast<const u32x4*>(ring + (ks & 1) * 2 * TILE + a_panel + ib * 16 * ROWB + fo[kc]);
    };
    auto read_w = [&](int ks, int kc, int jb) __attribute__((always_inline)) {
        fw[kc][jb] = *reinterpret_cast<const u32x4*>(ring + (ks & 1) * 2 * TILE + w_panel + jb * 16 * ROWB + fo[kc]);
    };
    // the loop accumulates into plain 4-register tuples (slices of acc's
    // 16-register vectors made the compiler copy them between AGPRs and
    // VGPRs around every MFMA once they no longer fit in the VGPRs); they
    // are packed into acc after the loop
    f32x4 c16[8][NB];
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) c16[ib][jb] = (f32x4){};
    auto mfma = [&](int kc, int ib, int jb) __attribute__((always_inline)) {
        c16[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[ib]),
                                                              __builtin_bit_cast(bf16x8, fw[kc][jb]), c16[ib][jb],
                                                              0, 0, 0);
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // the issue order of a region: one memory instruction after each MFMA,
    // LDS reads first, then LDS writes, then global loads
    auto order = [&](int nrd, int nwr, int nld) __attribute__((always_inline)) {
        int m = 0;
#pragma unroll
        for (int o = 0; o < nrd + nwr + nld; ++o) {
            if (m < NB) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                ++m;
            }
            if (o < nrd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else if (o < nrd + nwr) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
#pragma unroll
        for (; m < NB; ++m) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: step 0 written to stage 0, step 1 in registers, the
    //      fragments of step 0's chunk 0 except A block 7
#pragma unroll
    for (int j = 0; j < NP; ++j) load_piece(j, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) write_piece(j, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) load_piece(j, nk > 1 ? 1 : 0);
    wait_cnt<63, 0>();
    barrier();
#pragma unroll
    for (int ib = 0; ib < 7; ++ib) read_a(0, 0, ib);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) read_w(0, 0, jb);
    __builtin_amdgcn_sched_barrier(0);

    constexpr int W4 = NB / 4, P4 = PPC / 4, P2 = PPC / 2;
    for (int ks = 0; ks < nk; ++ks) {
        const int kn = ks + 2 < nk ? ks + 2 : nk - 1;    // loads past the last step repeat it
        // ---- chunk 0
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
            if (ib == 0) read_a(ks, 0, 7);
            else read_a(ks, 1, ib - 1);
            if (ib < 4) {
#pragma unroll
                for (int q = 0; q < W4; ++q) read_w(ks, 1, W4 * ib + q);
#pragma unroll
                for (int q = 0; q < P4; ++q) write_piece(P4 * ib + q, ks + 1);
            } else {
#pragma unroll
                for (int q = 0; q < P4; ++q) load_piece(P4 * (ib - 4) + q, kn);
            }
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) mfma(0, ib, jb);
            if (ib < 4) order(1 + W4, P4, 0);
            else order(1, 0, P4);
        }
        // ---- chunk 1
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
            if (ib < 2) {
                if (ib == 0) read_a(ks, 1, 7);
#pragma unroll
                for (int q = 0; q < P2; ++q) write_piece(PPC + P2 * ib + q, ks + 1);
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) mfma(1, ib, jb);
                order(ib == 0 ? 1 : 0, P2, 0);
                if (ib == 1) {
                    // this wavefront's reads of step ks and writes of step
                    // ks+1 are done; the barrier makes it so for all of them
                    // (after the last step the reads below fetch a stage
                    // nobody uses: the code stays branch-free)
                    wait_cnt<63, 0>();
                    barrier();
                }
            } else {
                if (ib == 2) read_a(ks + 1, 0, 0);
                read_a(ks + 1, 0, ib - 1);
                if (ib < 6) {
#pragma unroll
                    for (int q = 0; q < W4; ++q) read_w(ks + 1, 0, W4 * (ib - 2) + q);
#pragma unroll
                    for (int q = 0; q < P4; ++q) load_piece(PPC + P4 * (ib - 2) + q, kn);
                }
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) mfma(1, ib, jb);
                order((ib == 2 ? 2 : 1) + (ib < 6 ? W4 : 0), 0, ib < 6 ? P4 : 0);
            }
        }
    }
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int jb = 0; jb < NB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[ib >> 1][jb >> 1][4 * (2 * (ib & 1) + (jb & 1)) + e] = c16[ib][jb][e];
}

// ---------------------------------------------------------------- LDS-DMA ring on 16x16x32 MFMAs (bf16)
// gemm_mainloop_staged16's fragment schedule with the tile pieces copied by
// buffer -> LDS DMA instead of through registers: the same 1 KB pieces land
// at the same LDS addresses, so the fragments and sums are the same.  The
// copies of step ks+2 go out in regions 2-7 of chunk 1 of step ks, right
// after the step barrier that frees stage ks % 2, and have until the
// barrier of step ks+1 to land: that barrier waits for every copy the
// wavefront has in flight (vmcnt 0), which are exactly those.
template <int NWAVES>
__device__ __forceinline__ void gemm_mainloop_dma16(f32x16 (&acc)[4][NWAVES == 4 ? 4 : 2], char* ring,
                                                    const bf16* __restrict__ A, int64_t lda,
                                                    const bf16* __restrict__ W, int64_t ldw, int32_t M, int32_t N,
                                                    int32_t K, int m0, int n0, int wave, int lane) {
    constexpr int ROWB = 128, KCH = 2;
    using Geo = GemmGeom<ROWB, 2, NWAVES, 64>;
    constexpr int NJ = Geo::NJ;
    constexpr int NB = 2 * NJ;
    constexpr int TILE = Geo::TILE;
    constexpr int PIECES = Geo::PIECES;
    constexpr int NP = 2 * PIECES;
    static_assert((NWAVES == 8 && PIECES == 4 && NB == 4) || (NWAVES == 4 && PIECES == 8 && NB == 8), "DMA ring layout");
    constexpr int W4 = NB / 4;                           // W blocks read per region
    const int wm = NWAVES == 4 ? wave >> 1 : wave >> 2;
    const int wn = NWAVES == 4 ? wave & 1 : wave & 3;

    const uint32_t ldab = (uint32_t)(lda * 2), ldwb = (uint32_t)(ldw * 2);
    uint32_t voff[NP];
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
        const int row = Geo::ROWS_PER_WAVE * wave + Geo::ROWS_PER_PIECE * j + lane / Geo::CPR;
        const uint32_t c = (uint32_t)Geo::slot(row, lane % Geo::CPR);
        voff[j] = (uint32_t)row * ldab + c * 16;
        voff[PIECES + j] = (uint32_t)row * ldwb + c * 16;
    }
    const uint32_t bytes_a = (uint32_t)(M - m0 < kBM ? M - m0 : kBM) * ldab;
    const uint32_t bytes_w = (uint32_t)(N - n0 < kBN ? N - n0 : kBN) * ldwb;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A + (int64_t)m0 * lda, bytes_a);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + (int64_t)n0 * ldw, bytes_w);
    const int nk = K / 64;
    auto copy_piece = [&](int j, int ks) __attribute__((always_inline)) {
        char* st = ring + (ks & 1) * 2 * TILE + (j < PIECES ? 0 : TILE) + (wave * PIECES + j % PIECES) * 1024;
        dma_piece(j < PIECES ? ra : rw, st, voff[j], (uint32_t)ks * ROWB);
    };

    const int frow = lane & 15, fq = lane >> 4;
    uint32_t fo[KCH];
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc) fo[kc] = (uint32_t)(frow * ROWB + (Geo::slot(frow, 4 * kc + fq) << 4));
    const int a_panel = wm * 128 * ROWB, w_panel = TILE + wn * NJ * 32 * ROWB;
    u32x4 fa[8], fw[2][NB];
    auto read_a = [&](int ks, int kc, int ib) __attribute__((always_inline)) {
        fa[ib] = *reinterpret_cast<const u32x4*>(ring + (ks & 1) * 2 * TILE + a_panel + ib * 16 * ROWB + fo[kc]);
    };
    auto read_w = [&](int ks, int kc, int jb) __attribute__((always_inline)) {
        fw[kc][jb] = *reinterpret_cast<const u32x4*>(ring + (ks & 1) * 2 * TILE + w_panel + jb * 16 * ROWB + fo[kc]);
    };
    f32x4 c16[8][NB];
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) c16[ib][jb] = (f32x4){};
    auto mfma = [&](int kc, int ib, int jb) __attribute__((always_inline)) {
        c16[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[ib]),
                                                              __builtin_bit_cast(bf16x8, fw[kc][jb]), c16[ib][jb],
                                                              0, 0, 0);
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto order = [&](int nrd, int nld) __attribute__((always_inline)) {
        int m = 0;
#pragma unroll
        for (int o = 0; o < nrd + nld; ++o) {
            if (m < NB) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                ++m;
            }
            if (o < nrd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
#pragma unroll
        for (; m < NB; ++m) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: steps 0 and 1 copied, step 0 landed and visible; the
    //      fragments of step 0's chunk 0 except A block 7
#pragma unroll
    for (int j = 0; j < NP; ++j) copy_piece(j, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) copy_piece(j, nk > 1 ? 1 : 0);
    wait_cnt<NP, 0>();
    barrier();
#pragma unroll
    for (int ib = 0; ib < 7; ++ib) read_a(0, 0, ib);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) read_w(0, 0, jb);
    __builtin_amdgcn_sched_barrier(0);

    for (int ks = 0; ks < nk; ++ks) {
        const int kn = ks + 2 < nk ? ks + 2 : nk - 1;    // copies past the last step repeat it
        // ---- chunk 0: fragment reads only
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
            if (ib == 0) read_a(ks, 0, 7);
            else read_a(ks, 1, ib - 1);
            if (ib < 4) {
#pragma unroll
                for (int q = 0; q < W4; ++q) read_w(ks, 1, W4 * ib + q);
            }
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) mfma(0, ib, jb);
            order(ib < 4 ? 1 + W4 : 1, 0);
        }
        // ---- chunk 1
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
            if (ib < 2) {
                if (ib == 0) read_a(ks, 1, 7);
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) mfma(1, ib, jb);
                order(ib == 0 ? 1 : 0, 0);
                if (ib == 1) {
                    // this wavefront's reads of step ks are done and its copies
                    // of step ks+1 have landed; the barrier makes it so for all
                    wait_cnt<0, 0>();
                    barrier();
                }
            } else {
                if (ib == 2) read_a(ks + 1, 0, 0);
                read_a(ks + 1, 0, ib - 1);
                if (ib < 6) {
#pragma unroll
                    for (int q = 0; q < W4; ++q) read_w(ks + 1, 0, W4 * (ib - 2) + q);
                }
                // the NP copies over regions 2-7: 8 waves 2, 2, 1, 1, 1, 1;
                // 4 waves 3, 3, 3, 3, 2, 2
                constexpr int HI = NP == 8 ? 2 : 3, LO = NP == 8 ? 1 : 2;
                const int nc = ib < (NP == 8 ? 4 : 6) ? HI : LO;
                const int c0 = NP == 8 ? (ib < 4 ? 2 * (ib - 2) : ib) : (ib < 6 ? 3 * (ib - 2) : 12 + 2 * (ib - 6));
#pragma unroll
                for (int q = 0; q < nc; ++q) copy_piece(c0 + q, kn);
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) mfma(1, ib, jb);
                order((ib == 2 ? 2 : 1) + (ib < 6 ? W4 : 0), nc);
            }
        }
    }
    wait_cnt<0, 0>();    // no copy may land after the loop (the epilogue may reuse the ring)
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int jb = 0; jb < NB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[ib >> 1][jb >> 1][4 * (2 * (ib & 1) + (jb & 1)) + e] = c16[ib][jb][e];
}

// ---------------------------------------------------------------- staged ring for fp8 operands
// The register-staged ring of gemm_mainloop_staged16 (same pieces, loads a
// step ahead, LDS writes, barrier) for e4m3 operands on the 32x32x64 MFMA of
// the ring loop (lane l supplies row l % 32 and the 32 bytes at (l / 32) * 32
// of a 64-byte k-chunk: two 16-byte slots), so the accumulators keep the
// 32x32 layout and the products equal the ring loop's.  A 128-byte step row
// holds two chunks; a chunk is four regions, one per 32-row A block, each
// its two MFMAs (64 cycles each) with the memory instructions after them.
// A fragments rotate through one set of registers (block i of the next
// chunk is read in region i + 1, block 3 in region 0 of the chunk that uses
// it); W fragments are double-buffered.
__device__ __forceinline__ void gemm_mainloop_staged_fp8(f32x16 (&acc)[4][2], char* ring,
                                                         const uint8_t* __restrict__ A, int64_t lda,
                                                         const uint8_t* __restrict__ W, int64_t ldw, int32_t M,
                                                         int32_t N, int32_t K, int m0, int n0, int wave, int lane) {
    constexpr int NWAVES = 8, ROWB = 128, KCH = 2;
    using Geo = GemmGeom<ROWB, 2, NWAVES, 64>;
    constexpr int TILE = Geo::TILE;
    constexpr int PIECES = Geo::PIECES;                  // 4
    constexpr int NP = 2 * PIECES;
    constexpr int PPC = NP / KCH;                        // 4 pieces per chunk
    static_assert(PIECES == 4 && Geo::NJ == 2, "staging layout");
    using Op = GemmOp<fp8>;
    using Frag = Op::Frag;
    const int wm = wave >> 2, wn = wave & 3;

    const uint32_t ldab = (uint32_t)lda, ldwb = (uint32_t)ldw;
    uint32_t voff[NP];
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
        const int row = Geo::ROWS_PER_WAVE * wave + Geo::ROWS_PER_PIECE * j + lane / Geo::CPR;
        const uint32_t c = (uint32_t)Geo::slot(row, lane % Geo::CPR);
        voff[j] = (uint32_t)row * ldab + c * 16;
        voff[PIECES + j] = (uint32_t)row * ldwb + c * 16;
    }
    const uint32_t bytes_a = (uint32_t)(M - m0 < kBM ? M - m0 : kBM) * ldab;
    const uint32_t bytes_w = (uint32_t)(N - n0 < kBN ? N - n0 : kBN) * ldwb;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A + (int64_t)m0 * lda, bytes_a);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + (int64_t)n0 * ldw, bytes_w);
    const int nk = K / ROWB;
    u32x4 stg[NP];
    auto load_piece = [&](int j, int ks) __attribute__((always_inline)) {
        stg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(j < PIECES ? ra : rw, voff[j],
                                                                                  (uint32_t)ks * ROWB, 0));
    };
    auto write_piece = [&](int j, int ks) __attribute__((always_inline)) {
        char* st = ring + (ks & 1) * 2 * TILE + (j < PIECES ? 0 : TILE) + (wave * PIECES + j % PIECES) * 1024;
        *reinterpret_cast<u32x4*>(st + lane * 16) = stg[j];
    };

    // fragment slots of chunk kc: 4 kc + 2 (l / 32) and the next, in row l % 32
    // of a 32-row block (block starts are multiples of 32: the swizzle only
    // depends on l % 32)
    const int frow = lane & 31, fhalf = lane >> 5;
    uint32_t fo[KCH][2];
#pragma unroll
    for (int kc = 0; kc < KCH; ++kc)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            fo[kc][h] = (uint32_t)(frow * ROWB + (Geo::slot(frow, 4 * kc + 2 * fhalf + h) << 4));
    const int a_panel = wm * 128 * ROWB, w_panel = TILE + wn * 2 * 32 * ROWB;
    Frag fa[4], fw[2][2];
    auto read_a = [&](int ks, int kc, int i) __attribute__((always_inline)) {
        const char* b = ring + (ks & 1) * 2 * TILE + a_panel + i * 32 * ROWB;
        fa[i] = Op::read(b + fo[kc][0], b + fo[kc][1]);
    };
    auto read_w = [&](int ks, int kc, int j) __attribute__((always_inline)) {
        const char* b = ring + (ks & 1) * 2 * TILE + w_panel + j * 32 * ROWB;
        fw[kc][j] = Op::read(b + fo[kc][0], b + fo[kc][1]);
    };
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // a region's issue order: its two MFMAs, each followed by memory
    // instructions (LDS reads, then LDS writes, then global loads), the rest
    // after the second
    auto order = [&](int nrd, int nwr, int nld) __attribute__((always_inline)) {
        const int n = nrd + nwr + nld, first = n < 2 ? n : (n + 1) / 2;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
        for (int o = 0; o < n; ++o) {
            if (o == first) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (o < nrd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else if (o < nrd + nwr) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        if (first >= n) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: step 0 written to stage 0, step 1 in registers, the
    //      fragments of step 0's chunk 0 except A block 3
#pragma unroll
    for (int j = 0; j < NP; ++j) load_piece(j, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) write_piece(j, 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) load_piece(j, nk > 1 ? 1 : 0);
    wait_cnt<63, 0>();
    barrier();
#pragma unroll
    for (int i = 0; i < 3; ++i) read_a(0, 0, i);
#pragma unroll
    for (int j = 0; j < 2; ++j) read_w(0, 0, j);
    __builtin_amdgcn_sched_barrier(0);

    for (int ks = 0; ks < nk; ++ks) {
        const int kn = ks + 2 < nk ? ks + 2 : nk - 1;    // loads past the last step repeat it
        // ---- chunk 0: A reads (block 3 of this chunk, then blocks 0-2 of
        //      chunk 1), chunk 1's W reads in regions 0-1, piece writes, loads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i == 0) read_a(ks, 0, 3);
            else read_a(ks, 1, i - 1);
            if (i < 2) read_w(ks, 1, i);
            write_piece(i, ks + 1);
            if (i >= 2) {
                load_piece(2 * (i - 2), kn);
                load_piece(2 * (i - 2) + 1, kn);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) Op::mma(acc[i][j], fa[i], fw[0][j]);
            order(i < 2 ? 4 : 2, 1, i < 2 ? 0 : 2);
        }
        // ---- chunk 1: block 3's A read and the piece writes in regions
        //      0-1, the step barrier, then the next step's chunk-0 reads and
        //      the loads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < 2) {
                if (i == 0) read_a(ks, 1, 3);
                write_piece(PPC + 2 * i, ks + 1);
                write_piece(PPC + 2 * i + 1, ks + 1);
#pragma unroll
                for (int j = 0; j < 2; ++j) Op::mma(acc[i][j], fa[i], fw[1][j]);
                order(i == 0 ? 2 : 0, 2, 0);
                if (i == 1) {
                    // this wavefront's reads of step ks and writes of step
                    // ks+1 are done; the barrier makes it so for all of them
                    // (after the last step the reads below fetch a stage
                    // nobody uses: the code stays branch-free)
                    wait_cnt<63, 0>();
                    barrier();
                }
            } else {
                if (i == 2) {
                    read_a(ks + 1, 0, 0);
                    read_a(ks + 1, 0, 1);
                    read_w(ks + 1, 0, 0);
                    read_w(ks + 1, 0, 1);
                } else {
                    read_a(ks + 1, 0, 2);
                }
                load_piece(PPC + 2 * (i - 2), kn);
                load_piece(PPC + 2 * (i - 2) + 1, kn);
#pragma unroll
                for (int j = 0; j < 2; ++j) Op::mma(acc[i][j], fa[i], fw[1][j]);
                order(i == 2 ? 8 : 2, 0, 2);
            }
        }
    }
}

// TI: operand type (bf16, float, fp8); T: output type.  With fp8 operands
// the accumulators are scaled by sa[row] * sw[col] (per-row and per-column
// quantisation scales) before the epilogue.  STAGED selects the
// register-staged ring (bf16 and fp8); otherwise the LDS-DMA ring loop
// below runs (fp32 operands, or fp8 with H3_GEMM_FP8_STAGED 0).
// row and column of accumulator element r inside its 32x32 block, less the
// lane's own offsets (lrow, lcol in gemm_kernel)
template <bool M16>
__device__ __forceinline__ constexpr int acc_row(int r) {
    return M16 ? 16 * (r >> 3) + (r & 3) : 8 * (r >> 2) + (r & 3);
}
template <bool M16>
__device__ __forceinline__ constexpr int acc_col(int r) {
    return M16 ? 16 * ((r >> 2) & 1) : 0;
}

template <typename TI, typename T, int ROWB, int STAGES, int NWAVES, bool STAGED, typename EPI, bool DMA16 = false>
__global__ __launch_bounds__(NWAVES * 64) void gemm_kernel(const TI* __restrict__ A, int64_t lda,
                                                   const TI* __restrict__ W, int64_t ldw,
                                                   T* __restrict__ C, int64_t ldc, int32_t M, int32_t N,
                                                   int32_t K, int32_t tiles_m, int32_t tiles_n, int32_t group_m,
                                                   const EPI epi, const float* __restrict__ sa,
                                                   const float* __restrict__ sw) {
    using Op = GemmOp<TI>;
    using Geo = GemmGeom<ROWB, STAGES, NWAVES, Op::CHUNK>;
    constexpr int NJ = Geo::NJ;
    constexpr int ES = sizeof(TI);
    constexpr int BK = ROWB / ES;                       // elements of K per step
    constexpr int TILE = Geo::TILE, PIECES = Geo::PIECES, KCH = Geo::KCH;
    // stage s: A tile at ring + 2 s TILE, W tile right after it
    __shared__ __attribute__((aligned(1024))) char ring[STAGES * 2 * TILE];

    // ---- tile order: XCD-contiguous, then grouped group_m tiles high
    const int G = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = G >> 3, extra = G & 7;
    const int L = xcd * base + (xcd < extra ? xcd : extra) + local;
    const int group = group_m * tiles_n;
    const int first_m = (L / group) * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int tm = first_m + (L % group) % gm;
    const int tn = (L % group) / gm;
    const int m0 = tm * kBM;
    const int n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // 4 wavefronts: 2 x 2 panels of 128 x 128; 8 wavefronts: 2 x 4 of 128 x 64
    const int wm = NWAVES == 4 ? wave >> 1 : wave >> 2;
    const int wn = NWAVES == 4 ? wave & 1 : wave & 3;

    // Accumulator layout.  Element r of 32x32 block (i, j) is output row
    // 32 i + erow(r) + lrow and column 32 j + ecol(r) + lcol of the
    // wavefront's panel: for the 32x32 MFMA rows 8 (r / 4) + r % 4 + 4 (l / 32)
    // of column l % 32; for 16x16x32 sub-block r / 4 holds rows
    // 16 (r / 8) + r % 4 + 4 (l / 16 % 4) of column 16 (r / 4 % 2) + l % 16.
    constexpr bool M16 = STAGED && std::is_same<TI, bf16>::value && H3_GEMM_MFMA16;
    const int lrow = M16 ? 4 * ((lane >> 4) & 3) : 4 * (lane >> 5);
    const int lcol = M16 ? lane & 15 : lane & 31;

    f32x16 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = (f32x16){};
    if constexpr (STAGED && std::is_same<TI, fp8>::value) {
        static_assert(ROWB == 128 && STAGES == 2 && NWAVES == 8, "staged fp8 shape");
        gemm_mainloop_staged_fp8(acc, ring, A, lda, W, ldw, M, N, K, m0, n0, wave, lane);
    } else if constexpr (STAGED) {
        static_assert(std::is_same<TI, bf16>::value && ROWB == 128 && STAGES == 2, "staged shape");
        if constexpr (M16 && DMA16)
            gemm_mainloop_dma16<NWAVES>(acc, ring, A, lda, W, ldw, M, N, K, m0, n0, wave, lane);
        else if constexpr (M16) gemm_mainloop_staged16<NWAVES>(acc, ring, A, lda, W, ldw, M, N, K, m0, n0, wave, lane);
        else gemm_mainloop_staged<NWAVES>(acc, ring, A, lda, W, ldw, M, N, K, m0, n0, wave, lane);
    } else {
        // ---- copy offsets: piece j of this wavefront holds tile rows
        //      64 wave + ROWS_PER_PIECE j + lane / CPR; LDS slot lane % CPR of the
        //      row receives the chunk stored there
        const uint32_t ldab = (uint32_t)(lda * ES), ldwb = (uint32_t)(ldw * ES);
        uint32_t va[PIECES], vw[PIECES];
#pragma unroll
        for (int j = 0; j < PIECES; ++j) {
            const int row = Geo::ROWS_PER_WAVE * wave + Geo::ROWS_PER_PIECE * j + lane / Geo::CPR;
            const uint32_t c = (uint32_t)Geo::slot(row, lane % Geo::CPR);
            va[j] = (uint32_t)row * ldab + c * 16;
            vw[j] = (uint32_t)row * ldwb + c * 16;
        }
        const uint32_t bytes_a = (uint32_t)(M - m0 < kBM ? M - m0 : kBM) * ldab;
        const uint32_t bytes_w = (uint32_t)(N - n0 < kBN ? N - n0 : kBN) * ldwb;
        const TI* a_base = A + (int64_t)m0 * lda;
        const TI* w_base = W + (int64_t)n0 * ldw;
        auto copy_step = [&](int ks) {
            char* st = ring + (ks % STAGES) * 2 * TILE;
            copy_operand<PIECES>(st, wave, a_base, bytes_a, va, (uint32_t)ks * ROWB);
            copy_operand<PIECES>(st + TILE, wave, w_base, bytes_w, vw, (uint32_t)ks * ROWB);
        };
        // ---- fragment offsets: row (32 i + frow) of the wave's 128-row panel,
        //      chunk 2 kk + fhalf; the row's swizzle depends on frow only
        const int frow = lane & 31, fhalf = lane >> 5;
        constexpr int CPC = Op::CHUNK / 16;                 // 16-byte slots per k-chunk
        uint32_t fo[KCH], fo2[KCH];
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk) {
            const int c0 = CPC * kk + fhalf * (CPC / 2);
            fo[kk] = (uint32_t)(frow * ROWB + (Geo::slot(frow, c0) << 4));
            fo2[kk] = (uint32_t)(frow * ROWB + (Geo::slot(frow, c0 + 1) << 4));
        }
        const int a_panel = wm * 128 * ROWB, w_panel = TILE + wn * NJ * 32 * ROWB;


        // Fragments are double-buffered per 32-byte k-chunk: chunk kk of a step
        // lives in register slot kk % 2 (4 A + 4 W 16-byte reads), and the next
        // chunk's reads are issued before the current chunk's 16 MFMAs.
        using Frag = typename Op::Frag;
        Frag fa[2][4], fw[2][NJ];
        auto read_chunk = [&](int ks, int kk, Frag (&a)[4], Frag (&w)[NJ]) {
            const char* st = ring + (ks % STAGES) * 2 * TILE;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = Op::read(st + a_panel + i * 32 * ROWB + fo[kk], st + a_panel + i * 32 * ROWB + fo2[kk]);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                w[j] = Op::read(st + w_panel + j * 32 * ROWB + fo[kk], st + w_panel + j * 32 * ROWB + fo2[kk]);
        };
        auto mfma_chunk = [&](const Frag (&a)[4], const Frag (&w)[NJ]) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Op::mma(acc[i][j], a[i], w[j]);
        };
        // Wait until step s has landed in LDS for every wavefront and this
        // wavefront's reads of the step before are done: at most the copies of
        // the (up to STAGES - 2) later steps already issued may be outstanding.
        // Then the stage of step s-1 is free for the copy of step s+STAGES-1.
        // A plain s_barrier is used: __syncthreads() would also wait for the
        // later copies.
        constexpr int PER_STEP = 2 * PIECES;
        auto step_ready = [&](int s, int nk) {
            const int later = nk - 1 - s;      // copies of min(later, STAGES - 2) later steps may be in flight
            const int ahead = later < STAGES - 2 ? later : STAGES - 2;
            if (ahead >= 3) wait_vm<(3 * PER_STEP < 63 ? 3 * PER_STEP : 63), true>();
            else if (ahead == 2) wait_vm<2 * PER_STEP, true>();
            else if (ahead == 1) wait_vm<PER_STEP, true>();
            else wait_vm<0, true>();
            __builtin_amdgcn_s_barrier();
            if (s + STAGES - 1 < nk) copy_step(s + STAGES - 1);
        };

        const int nk = K / BK;
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nk) copy_step(s);
        step_ready(0, nk);
        read_chunk(0, 0, fa[0], fw[0]);
        for (int ks = 0; ks < nk; ++ks) {
#pragma unroll
            for (int kk = 0; kk < KCH; ++kk) {
                __builtin_amdgcn_sched_barrier(0);
                if (kk + 1 < KCH) {
                    // the previous chunk's reads were issued a chunk of MFMAs ago;
                    // retiring them keeps at most 8 LDS reads in flight (the
                    // counter holds 15)
                    wait_vm<63, true>();
                    read_chunk(ks, kk + 1, fa[(kk + 1) & 1], fw[(kk + 1) & 1]);
                } else {
                    // This chunk's fragments (read a chunk of MFMAs ago) land
                    // here on every path, so the MFMAs below never wait for the
                    // next step's reads issued after the barrier; without it the
                    // compiler merges the last step's counter state into the
                    // common path and stalls every step on those fresh reads.
                    wait_vm<63, true>();
                    if (ks + 1 < nk) {
                        step_ready(ks + 1, nk);
                        read_chunk(ks + 1, 0, fa[0], fw[0]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // the reads above go out before these MFMAs
                mfma_chunk(fa[kk & 1], fw[kk & 1]);
            }
        }
    }

    const bool full = m0 + kBM <= M && n0 + kBN <= N;
    // CB column halves per 32x32 block take their own column-indexed values
    constexpr int CB = M16 ? 2 : 1;
    auto rof = [](int r) __attribute__((always_inline)) { return acc_row<M16>(r); };
    auto cof = [](int r) __attribute__((always_inline)) { return acc_col<M16>(r); };
    if constexpr (std::is_same<TI, fp8>::value) {
        // dequantise: acc * sa[row] * sw[col] (rows and columns past M / N
        // take scale 0 and are never stored)
        float cs[NJ][CB];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int h = 0; h < CB; ++h) {
                const int col = n0 + wn * NJ * 32 + j * 32 + 16 * h + lcol;
                cs[j][h] = col < N ? sw[col] : 0.f;
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + i * 32 + rof(r) + lrow;
                const float rs = row < M ? sa[row] : 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j][r] *= rs * cs[j][cof(r) >> 4];
            }
    }
    // plain store of the accumulators (rows and columns past M, N skipped)
    auto store_c = [&]() __attribute__((always_inline)) {
        T* cbase = C + (int64_t)(m0 + wm * 128 + lrow) * ldc + n0 + wn * NJ * 32 + lcol;
        if (full) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        GemmMfma<T>::store(cbase + (int64_t)(i * 32 + rof(r)) * ldc + j * 32 + cof(r), acc[i][j][r]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = m0 + wm * 128 + i * 32 + rof(r) + lrow;
                        const int col = n0 + wn * NJ * 32 + j * 32 + cof(r) + lcol;
                        if (row < M && col < N)
                            GemmMfma<T>::store(cbase + (int64_t)(i * 32 + rof(r)) * ldc + j * 32 + cof(r),
                                               acc[i][j][r]);
                    }
                }
        }
    };
    if constexpr (std::is_same<EPI, EpiStore>::value) {
        store_c();
    } else if constexpr (std::is_same<EPI, EpiGate>::value) {
        const T* xb = reinterpret_cast<const T*>(epi.x);
        // One interval usually covers the whole tile: then every row takes the
        // same modality set; otherwise each row looks its interval up.
        const int last = (m0 + kBM < M ? m0 + kBM : M) - 1;
        const int seg0 = find_seg(epi.tab, m0);
        const bool one_set = seg0 == find_seg(epi.tab, last);
        const int set0 = epi.tab.s[seg0].mod_set;
        // gates of this lane's columns: loaded once for a one-set tile, per row
        // (from cache) on the few tiles an interval boundary crosses
        const float* gbase = epi.mod + (int64_t)epi.chunk * N + n0 + wn * NJ * 32 + lcol;
        const int64_t set_stride = (int64_t)6 * N;
        float g0[NJ][CB];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int h = 0; h < CB; ++h)
                g0[j][h] = n0 + wn * NJ * 32 + j * 32 + 16 * h + lcol < N
                               ? gbase[set0 * set_stride + j * 32 + 16 * h] : 0.f;
        auto gate = [&](int row, int j, int r) __attribute__((always_inline)) {
            return one_set ? g0[j][cof(r) >> 4]
                           : gbase[epi.tab.s[find_seg(epi.tab, row)].mod_set * set_stride + j * 32 + cof(r)];
        };
        const int64_t obase = (int64_t)(m0 + wm * 128 + lrow) * ldc + n0 + wn * NJ * 32 + lcol;
        // bf16 output of a full tile (staged and DMA loops, whose 128 KB ring
        // is free now): the fp32 products go through LDS, 128 tile rows per
        // pass, so that x is read and out written as 16-byte vectors of eight
        // columns of one row (a wavefront covers two 512-byte row runs)
        // instead of the accumulators' 2-byte scatter.  Same arithmetic as
        // below: out = bf16(x + gate * acc).
        constexpr bool LDS_GATE = std::is_same<T, bf16>::value && STAGED && STAGES * 2 * TILE >= 128 * 1024;
        if (LDS_GATE && full) {
            // 16-byte chunk c (four columns) of tile row rl at slot c ^ (rl % 64)
            auto fchunk = [&](int rl, int c) __attribute__((always_inline)) -> float* {
                return reinterpret_cast<float*>(ring + rl * 1024 + ((c ^ (rl & 63)) << 4));
            };
            const int cg = tid & 31;                          // this thread's eight columns: 8 cg ..
            const float* gcol = epi.mod + (int64_t)epi.chunk * N + n0 + 8 * cg;
            float gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[e] = gcol[set0 * set_stride + e];
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                __syncthreads();          // the ring is free (main loop, or the previous pass, done)
                if (wm == pass) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int rl = i * 32 + rof(r) + lrow;
                                const int col = wn * NJ * 32 + j * 32 + cof(r) + lcol;
                                fchunk(rl, col >> 2)[col & 3] = acc[i][j][r];
                            }
                }
                __syncthreads();
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int rl = (tid >> 5) + 16 * k;
                    const int row = m0 + pass * 128 + rl;
                    const f32x4 a0 = *reinterpret_cast<const f32x4*>(fchunk(rl, 2 * cg));
                    const f32x4 a1 = *reinterpret_cast<const f32x4*>(fchunk(rl, 2 * cg + 1));
                    const int64_t o = (int64_t)row * ldc + n0 + 8 * cg;
                    const u32x4 xw = *reinterpret_cast<const u32x4*>(xb + o);
                    const float* gr = one_set ? nullptr : gcol + epi.tab.s[find_seg(epi.tab, row)].mod_set * set_stride;
                    float xv[8], av[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // a bf16 widens to fp32 by its bits moved to the top half
                        const uint32_t w = xw[e];
                        xv[2 * e] = __builtin_bit_cast(float, w << 16);
                        xv[2 * e + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
                        av[e] = a0[e];
                        av[4 + e] = a1[e];
                    }
                    u32x4 ow;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float g0e = one_set ? gv[2 * e] : gr[2 * e];
                        const float g1e = one_set ? gv[2 * e + 1] : gr[2 * e + 1];
                        ow[e] = pack_bf16x2(xv[2 * e] + g0e * av[2 * e], xv[2 * e + 1] + g1e * av[2 * e + 1]);
                    }
                    *reinterpret_cast<u32x4*>(C + o) = ow;
                }
            }
        } else if (full) {
            // per 32-row block: all 16 x NJ residual loads first, then the stores
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float xv[16][NJ];
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        xv[r][j] = GemmMfma<T>::load(xb + obase + (int64_t)(i * 32 + rof(r)) * ldc + j * 32 + cof(r));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + i * 32 + rof(r) + lrow;
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        GemmMfma<T>::store(C + obase + (int64_t)(i * 32 + rof(r)) * ldc + j * 32 + cof(r),
                                           xv[r][j] + gate(row, j, r) * acc[i][j][r]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + i * 32 + rof(r) + lrow;
                    if (row >= M) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int col = n0 + wn * NJ * 32 + j * 32 + cof(r) + lcol;
                        if (col >= N) continue;
                        const int64_t o = (int64_t)row * ldc + col;
                        GemmMfma<T>::store(C + o, GemmMfma<T>::load(xb + o) + gate(row, j, r) * acc[i][j][r]);
                    }
                }
        }
    } else if constexpr (IsQkRope<EPI>::value) {
        if (n0 >= 2 * epi.q_cols) {
            store_c();    // a v tile
        } else {
            // The ring is reused as RPASS rows of the tile in T (16-byte chunk
            // c of row r at slot c ^ (r % CPR)): all 256 rows for bf16, two
            // passes of 128 for fp32.  The kernel declares no LDS beyond the
            // ring: an allocation above 128 KB per workgroup was measured to
            // slow the main loop by a sixth.  The CPH lanes that hold one row
            // of a head (consecutive lanes, one 16-byte chunk each) sum its
            // squares with a butterfly, so no per-row table is kept.
            constexpr int HD = EPI::kHd;
            constexpr int TB = (int)sizeof(T);
            constexpr int RING = STAGES * 2 * TILE;
            constexpr int RAVAIL = RING / (kBN * TB);   // tile rows the ring holds
            constexpr int RPASS = RAVAIL >= kBM ? kBM : RAVAIL >= 128 ? 128 : RAVAIL >= 64 ? 64 : 32;
            constexpr int CPR = kBN * TB / 16;        // 16-byte chunks per tile row
            constexpr int VN = 16 / TB;               // values per chunk
            constexpr int CPH = HD / VN;              // chunks (lanes) per row of a head
            constexpr int HPT = kBN / HD;             // heads per tile
            constexpr int NT = NWAVES * 64;
            constexpr int RSTEP = NT / CPH;           // rows between a thread's rows
            constexpr int RPT = RPASS / RSTEP;        // rows per thread and pass
            static_assert(CPH <= 64 && NT % CPH == 0 && RPASS % RSTEP == 0 && kBM % RPASS == 0, "epilogue split");
            auto chunk_at = [&](int rl, int ch) __attribute__((always_inline)) -> char* {
                return ring + rl * (CPR * 16) + ((ch ^ (rl % CPR)) << 4);
            };
            const float* gam = n0 < epi.q_cols ? epi.gq : epi.gk;
            // a thread always takes chunk cp of its rows: its pairs' gains,
            // frequencies and axes are loaded once
            const int cp = tid % CPH, d0 = cp * VN, r0 = tid / CPH;
            float g[VN], frh[VN / 2], frl[VN / 2];
            int ax[VN / 2];
#pragma unroll
            for (int e = 0; e < VN; ++e) g[e] = gam ? gam[d0 + e] : 1.0f;
#pragma unroll
            for (int e = 0; e < VN / 2; ++e) {
                const int p = d0 / 2 + e;
                frh[e] = epi.fr_hi[p];
                frl[e] = epi.fr_lo[p];
                ax[e] = epi.axis[p];
            }
#pragma unroll
            for (int pass = 0; pass < kBM / RPASS; ++pass) {
                // positions of this thread's rows (loads in flight during step 1)
                int pt[RPT], ph[RPT], pw[RPT];
#pragma unroll
                for (int k = 0; k < RPT; ++k) {
                    const int row = m0 + pass * RPASS + r0 + k * RSTEP;
                    pt[k] = ph[k] = pw[k] = 0;
                    if (row < M) {
                        const SegDev& sg = epi.tab.s[find_seg(epi.tab, row)];
                        const int l = row - sg.start;
                        pt[k] = sg.t0 + l / sg.HW;
                        ph[k] = sg.h0 + (l / sg.W) % sg.H;
                        pw[k] = sg.w0 + l % sg.W;
                    }
                }
                // 1. this pass's rows, rounded to T (a 32-row block of a
                //    wavefront lies in one pass); pass 0 first waits until
                //    every wavefront's fragment reads are done
                if (pass == 0) __syncthreads();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if ((wm * 128 + i * 32) / RPASS != pass) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int col = wn * NJ * 32 + j * 32 + cof(r) + lcol;
                            const int rl = wm * 128 + i * 32 + rof(r) + lrow - pass * RPASS;
                            reinterpret_cast<T*>(chunk_at(rl, col / VN))[col % VN] = (T)acc[i][j][r];
                        }
                    }
                }
                __syncthreads();
                // 2. per row: the angles of the thread's pairs, then per head
                //    the 1/rms (butterfly over the row's CPH lanes), gain,
                //    rotation and store.  Every lane runs the butterfly;
                //    rows past M only skip the store.
#pragma unroll
                for (int k = 0; k < RPT; ++k) {
                    const int rl = r0 + k * RSTEP;
                    const int row = m0 + pass * RPASS + rl;
                    float cs[VN / 2], sn[VN / 2];
#pragma unroll
                    for (int e = 0; e < VN / 2; ++e) {
                        // pos * fr - (whole turns): the fma subtracts the turns from
                        // the exact product pos * fr_hi, so the reduction is exact
                        // whether or not the compiler contracts the sum after it
                        const float pos = (float)(ax[e] == 0 ? pt[k] : ax[e] == 1 ? ph[k] : pw[k]);
                        const float turns = __builtin_rintf(pos * frh[e]);
                        const float x = __builtin_fmaf(pos, frh[e], -turns) + pos * frl[e];
                        if constexpr (TB == 4) {
                            sincospif(2.0f * x, &sn[e], &cs[e]);
                        } else {
                            sn[e] = __builtin_amdgcn_sinf(x);          // v_sin / v_cos take revolutions
                            cs[e] = __builtin_amdgcn_cosf(x);
                        }
                    }
#pragma unroll
                    for (int hh = 0; hh < HPT; ++hh) {
                        float f[VN];
                        Vec<T>::load(chunk_at(rl, hh * CPH + cp), f);
                        float ss = 0.f;
#pragma unroll
                        for (int e = 0; e < VN; ++e) ss += f[e] * f[e];
                        ss = sum_lanes<CPH>(ss);
                        const float rstd = 1.0f / __builtin_sqrtf(ss / (float)HD + epi.eps);
#pragma unroll
                        for (int e = 0; e < VN; ++e) f[e] *= rstd * g[e];
#pragma unroll
                        for (int e = 0; e < VN; e += 2) {
                            const float u0 = f[e], u1 = f[e + 1];
                            f[e] = u0 * cs[e >> 1] - u1 * sn[e >> 1];
                            f[e + 1] = u0 * sn[e >> 1] + u1 * cs[e >> 1];
                        }
                        if (row < M) Vec<T>::store(C + (int64_t)row * ldc + n0 + hh * HD + d0, f);
                    }
                }
                if (pass + 1 < kBM / RPASS) __syncthreads();   // the next pass rewrites the tile
            }
        }
    } else {
        static_assert(std::is_same<EPI, EpiSwiglu>::value && NJ % 2 == 0, "SwiGLU pairs a wavefront's blocks");
        // blocks 2q and 2q+1 of a wavefront are a 32-column gate block and its
        // up block; their output columns start at half the interleaved index
        const int F = N >> 1;
        auto hval = [&](float gt, float up) __attribute__((always_inline)) {
            return gt / (1.0f + __expf(-gt)) * up;
        };
#pragma unroll
        for (int q = 0; q < NJ / 2; ++q) {
            const int hcol = ((n0 + wn * NJ * 32) >> 1) + q * 32 + lcol;
            T* hbase = C + (int64_t)(m0 + wm * 128 + lrow) * ldc + hcol;
            if (full) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        GemmMfma<T>::store(hbase + (int64_t)(i * 32 + rof(r)) * ldc + cof(r),
                                           hval(acc[i][2 * q][r], acc[i][2 * q + 1][r]));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = m0 + wm * 128 + i * 32 + rof(r) + lrow;
                        if (row < M && hcol + cof(r) < F)
                            GemmMfma<T>::store(hbase + (int64_t)(i * 32 + rof(r)) * ldc + cof(r),
                                               hval(acc[i][2 * q][r], acc[i][2 * q + 1][r]));
                    }
            }
        }
    }
}

template <typename TI, typename TO, typename EPI>
hipError_t launch_gemm_t(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int64_t M,
                         int32_t N, int32_t K, const EPI& epi, const float* sa, const float* sw, hipStream_t st) {
    const int tiles_m = (int)((M + kBM - 1) / kBM);
    const int tiles_n = (N + kBN - 1) / kBN;
    const int grid = tiles_m * tiles_n;
    constexpr bool BF = std::is_same<TI, bf16>::value;
    if constexpr (BF && H3_GEMM_BF16_STAGED) {
        // the LDS-DMA loop for K up to H3_GEMM_BF16_DMA_MAX_K (measured faster at
        // K 5376 and 7168), the register-staged loop beyond (faster at 14336);
        // XCD groups 2 tiles high when the output is at most 32 tiles wide (the
        // 5376-wide projections, 3 % faster), else H3_GEMM_BF16_GROUP_M
        const int gm = tiles_n <= 32 ? 2 : H3_GEMM_BF16_GROUP_M;
        if (K <= H3_GEMM_BF16_DMA_MAX_K)
            gemm_kernel<TI, TO, 128, 2, H3_GEMM_BF16_WAVES, true, EPI, true><<<grid, H3_GEMM_BF16_WAVES * 64, 0, st>>>(
                (const TI*)A, lda, (const TI*)W, ldw, (TO*)C, ldc, (int32_t)M, N, K, tiles_m, tiles_n, gm, epi, sa,
                sw);
        else
            gemm_kernel<TI, TO, 128, 2, H3_GEMM_BF16_WAVES, true, EPI><<<grid, H3_GEMM_BF16_WAVES * 64, 0, st>>>(
                (const TI*)A, lda, (const TI*)W, ldw, (TO*)C, ldc, (int32_t)M, N, K, tiles_m, tiles_n, gm, epi, sa,
                sw);
    } else if constexpr (std::is_same<TI, fp8>::value && H3_GEMM_FP8_STAGED) {
        gemm_kernel<TI, TO, 128, 2, 8, true, EPI><<<grid, 8 * 64, 0, st>>>(
            (const TI*)A, lda, (const TI*)W, ldw, (TO*)C, ldc, (int32_t)M, N, K, tiles_m, tiles_n,
            H3_GEMM_GROUP_M, epi, sa, sw);
    } else {
        gemm_kernel<TI, TO, H3_GEMM_ROWB, H3_GEMM_STAGES, H3_GEMM_WAVES, false, EPI><<<grid, H3_GEMM_WAVES * 64, 0, st>>>(
            (const TI*)A, lda, (const TI*)W, ldw, (TO*)C, ldc, (int32_t)M, N, K, tiles_m, tiles_n, H3_GEMM_GROUP_M,
            epi, sa, sw);
    }
    return hipGetLastError();
}

template <typename EPI>
hipError_t launch_gemm_epi(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
                           int64_t M, int32_t N, int32_t K, const EPI& epi, hipStream_t st) {
    return bf ? launch_gemm_t<bf16, bf16>(A, lda, W, ldw, C, ldc, M, N, K, epi, nullptr, nullptr, st)
              : launch_gemm_t<float, float>(A, lda, W, ldw, C, ldc, M, N, K, epi, nullptr, nullptr, st);
}

hipError_t launch_gemm_fp8(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw, const float* sw,
                           void* C, int64_t ldc, int64_t M, int32_t N, int32_t K, bool out_bf16, hipStream_t st) {
    return out_bf16 ? launch_gemm_t<fp8, bf16>(A, lda, W, ldw, C, ldc, M, N, K, EpiStore{}, sa, sw, st)
                    : launch_gemm_t<fp8, float>(A, lda, W, ldw, C, ldc, M, N, K, EpiStore{}, sa, sw, st);
}

hipError_t launch_gemm(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                       int64_t ldc, int64_t M, int32_t N, int32_t K, hipStream_t st) {
    return launch_gemm_epi(bf, A, lda, W, ldw, C, ldc, M, N, K, EpiStore{}, st);
}

hipError_t launch_gemm_gate(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, const void* x,
                            void* out, int64_t ldo, int64_t M, int32_t N, int32_t K, const float* mod,
                            int32_t n_sets, int32_t br, const SegTable& tab, hipStream_t st) {
    EpiGate e;
    e.x = x;
    e.mod = mod;
    e.chunk = 3 * br + 2;
    e.tab = tab;
    return launch_gemm_epi(bf, A, lda, W, ldw, out, ldo, M, N, K, e, st);
}

hipError_t launch_gemm_swiglu(bool bf, const void* A, int64_t lda, const void* Wgu, int64_t ldw, void* H,
                              int64_t ldh, int64_t M, int32_t F, int32_t K, hipStream_t st) {
    return launch_gemm_epi(bf, A, lda, Wgu, ldw, H, ldh, M, 2 * F, K, EpiSwiglu{}, st);
}

template <int HD>
static EpiQkRope<HD> make_qkrope(int32_t heads, const float* gq, const float* gk, float eps, const RopeTable& rt,
                                 const SegTable& tab) {
    EpiQkRope<HD> e;
    memset(&e, 0, sizeof(e));
    e.gq = gq;
    e.gk = gk;
    e.eps = eps;
    e.q_cols = heads * HD;
    for (int p = 0; p < HD / 2; ++p) {
        const double fr = rt.inv_freq[p] / (2.0 * 3.14159265358979323846);
        e.fr_hi[p] = (float)fr;
        e.fr_lo[p] = (float)(fr - (double)e.fr_hi[p]);
        e.axis[p] = rt.axis[p];
    }
    e.tab = tab;
    return e;
}

hipError_t launch_gemm_qknorm_rope(bool bf, const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                                  int64_t ldc, int64_t M, int32_t N, int32_t K, int32_t heads, int32_t hd,
                                  const float* gq, const float* gk, float eps, const RopeTable& rt,
                                  const SegTable& tab, hipStream_t st) {
    if (hd == 128)
        return launch_gemm_epi(bf, A, lda, W, ldw, C, ldc, M, N, K, make_qkrope<128>(heads, gq, gk, eps, rt, tab), st);
    return launch_gemm_epi(bf, A, lda, W, ldw, C, ldc, M, N, K, make_qkrope<64>(heads, gq, gk, eps, rt, tab), st);
}

hipError_t launch_gemm_fp8_qknorm_rope(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw,
                                      const float* sw, void* C, int64_t ldc, int64_t M, int32_t N, int32_t K,
                                      int32_t heads, int32_t hd, const float* gq, const float* gk, float eps,
                                      const RopeTable& rt, const SegTable& tab, hipStream_t st) {
    if (hd == 128)
        return launch_gemm_t<fp8, bf16>(A, lda, W, ldw, C, ldc, M, N, K,
                                        make_qkrope<128>(heads, gq, gk, eps, rt, tab), sa, sw, st);
    return launch_gemm_t<fp8, bf16>(A, lda, W, ldw, C, ldc, M, N, K, make_qkrope<64>(heads, gq, gk, eps, rt, tab),
                                    sa, sw, st);
}

hipError_t launch_gemm_fp8_gate(const void* A, int64_t lda, const float* sa, const void* W, int64_t ldw,
                                const float* sw, const void* x, void* out, int64_t ldo, int64_t M, int32_t N,
                                int32_t K, const float* mod, int32_t n_sets, int32_t br, const SegTable& tab,
                                hipStream_t st) {
    EpiGate e;
    e.x = x;
    e.mod = mod;
    e.chunk = 3 * br + 2;
    e.tab = tab;
    return launch_gemm_t<fp8, bf16>(A, lda, W, ldw, out, ldo, M, N, K, e, sa, sw, st);
}

hipError_t launch_gemm_fp8_swiglu(const void* A, int64_t lda, const float* sa, const void* Wgu, int64_t ldw,
                                  const float* sw, void* H, int64_t ldh, int64_t M, int32_t F, int32_t K,
                                  hipStream_t st) {
    return launch_gemm_t<fp8, bf16>(A, lda, Wgu, ldw, H, ldh, M, 2 * F, K, EpiSwiglu{}, sa, sw, st);
}

}  // namespace h3
