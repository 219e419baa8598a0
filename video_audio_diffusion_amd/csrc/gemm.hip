// C = A . W^T on MFMA for the four projections of the H3 block.
//
// A [M][K] and W [N][K] are both K-contiguous, which is exactly the operand
// layout of the 32x32 MFMA: lane l supplies row (l % 32) and a 16-byte run of
// k at offset (l / 32) * 16 bytes inside a 32-byte k-chunk.  So both operands
// are staged in LDS as [rows][128 bytes of k] tiles and read back as whole
// 16-byte vectors.
//
// Tile: 256 x 256 per workgroup.  With 8 wavefronts (two per SIMD, so one
// can issue MFMAs while the other waits) each owns a 128 x 64 panel (4 x 2
// MFMA blocks); with 4 wavefronts each owns 128 x 128.  Each k-step's A and W
// tiles (ROWB bytes of K per row) are copied from global memory straight into
// LDS by buffer->LDS loads into a STAGES-deep ring, so the next steps' copies
// are in flight while a step is multiplied; the buffer resources stop at row
// M (N), so tiles that run past the end are padded with zeros.  Fragments
// are double-buffered in registers per 32-byte k-chunk: the reads of the
// next chunk are issued before the current chunk's MFMAs.
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

// TI: operand type (bf16, float, fp8); T: output type.  With fp8 operands
// the accumulators are scaled by sa[row] * sw[col] (per-row and per-column
// quantisation scales) before the epilogue.
template <typename TI, typename T, int ROWB, int STAGES, int NWAVES, typename EPI>
__global__ __launch_bounds__(NWAVES * 64) void gemm_kernel(const TI* __restrict__ A, int64_t lda,
                                                   const TI* __restrict__ W, int64_t ldw,
                                                   T* __restrict__ C, int64_t ldc, int32_t M, int32_t N,
                                                   int32_t K, int32_t tiles_m, int32_t tiles_n, int32_t group_m,
                                                   EPI epi, const float* __restrict__ sa,
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

    f32x16 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = (f32x16){};

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
        const int later = nk - 1 - s;
        if constexpr (STAGES >= 4) {
            if (later >= 2) wait_vm<2 * PER_STEP, true>();
            else if (later == 1) wait_vm<PER_STEP, true>();
            else wait_vm<0, true>();
        } else if constexpr (STAGES == 3) {
            if (later >= 1) wait_vm<PER_STEP, true>();
            else wait_vm<0, true>();
        } else {
            wait_vm<0, true>();
        }
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

    // ---- epilogue: accumulator (lane, r) -> row 8(r/4) + 4(lane/32) + r%4, col lane%32
    const bool full = m0 + kBM <= M && n0 + kBN <= N;
    if constexpr (std::is_same<TI, fp8>::value) {
        // dequantise: acc * sa[row] * sw[col] (rows and columns past M / N
        // take scale 0 and are never stored)
        float cs[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = n0 + wn * NJ * 32 + j * 32 + frow;
            cs[j] = col < N ? sw[col] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
                const float rs = row < M ? sa[row] : 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j][r] *= rs * cs[j];
            }
    }
    // plain store of the accumulators (rows and columns past M, N skipped)
    auto store_c = [&]() __attribute__((always_inline)) {
        T* cbase = C + (int64_t)(m0 + wm * 128 + 4 * fhalf) * ldc + n0 + wn * NJ * 32 + frow;
        if (full) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        GemmMfma<T>::store(cbase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32,
                                           acc[i][j][r]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int col = n0 + wn * NJ * 32 + j * 32 + frow;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
                        if (row < M && col < N)
                            GemmMfma<T>::store(cbase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32,
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
        const float* gbase = epi.mod + (int64_t)epi.chunk * N + n0 + wn * NJ * 32 + frow;
        const int64_t set_stride = (int64_t)6 * N;
        float g0[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            g0[j] = n0 + wn * NJ * 32 + j * 32 + frow < N ? gbase[set0 * set_stride + j * 32] : 0.f;
        auto gate = [&](int row, int j) __attribute__((always_inline)) {
            return one_set ? g0[j] : gbase[epi.tab.s[find_seg(epi.tab, row)].mod_set * set_stride + j * 32];
        };
        const int64_t obase = (int64_t)(m0 + wm * 128 + 4 * fhalf) * ldc + n0 + wn * NJ * 32 + frow;
        if (full) {
            // per 32-row block: all 16 x NJ residual loads first, then the stores
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float xv[16][NJ];
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        xv[r][j] = GemmMfma<T>::load(xb + obase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc +
                                                     j * 32);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        GemmMfma<T>::store(C + obase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32,
                                           xv[r][j] + gate(row, j) * acc[i][j][r]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
                    if (row >= M) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int col = n0 + wn * NJ * 32 + j * 32 + frow;
                        if (col >= N) continue;
                        const int64_t o = (int64_t)row * ldc + col;
                        GemmMfma<T>::store(C + o, GemmMfma<T>::load(xb + o) + gate(row, j) * acc[i][j][r]);
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
            constexpr int RPASS = RING / (kBN * TB) < kBM ? RING / (kBN * TB) : kBM;
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
                        const int col = wn * NJ * 32 + j * 32 + frow;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int rl = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3) - pass * RPASS;
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
        static_assert(std::is_same<EPI, EpiSwiglu>::value && NJ == 2, "SwiGLU pairs a wavefront's two blocks");
        // output column of this lane: half the interleaved column index
        const int hcol = (n0 >> 1) + wn * 32 + frow;
        const int F = N >> 1;
        auto hval = [&](float gt, float up) __attribute__((always_inline)) {
            return gt / (1.0f + __expf(-gt)) * up;
        };
        T* hbase = C + (int64_t)(m0 + wm * 128 + 4 * fhalf) * ldc + hcol;
        if (full) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    GemmMfma<T>::store(hbase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc,
                                       hval(acc[i][0][r], acc[i][1][r]));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
                    if (row < M && hcol < F)
                        GemmMfma<T>::store(hbase + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc,
                                           hval(acc[i][0][r], acc[i][1][r]));
                }
        }
    }
}

// Launch configuration (measured best on the block's four projection
// shapes): 128 bytes of K per step, 2 LDS stages, 8 wavefronts (two per
// SIMD, 128 x 64 each), XCD groups 2 tiles high.  The macros only exist so
// that other configurations of the same template can be built and timed.
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

template <typename TI, typename TO, typename EPI>
hipError_t launch_gemm_t(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int64_t M,
                         int32_t N, int32_t K, const EPI& epi, const float* sa, const float* sw, hipStream_t st) {
    const int tiles_m = (int)((M + kBM - 1) / kBM);
    const int tiles_n = (N + kBN - 1) / kBN;
    const int grid = tiles_m * tiles_n;
    gemm_kernel<TI, TO, H3_GEMM_ROWB, H3_GEMM_STAGES, H3_GEMM_WAVES, EPI><<<grid, H3_GEMM_WAVES * 64, 0, st>>>(
        (const TI*)A, lda, (const TI*)W, ldw, (TO*)C, ldc, (int32_t)M, N, K, tiles_m, tiles_n, H3_GEMM_GROUP_M, epi,
        sa, sw);
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
