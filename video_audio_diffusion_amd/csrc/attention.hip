// Full bidirectional softmax attention, flash style, on MFMA.
//
// Work split: one workgroup = 8 wavefronts = 256 query rows of one head;
// each wavefront owns 32 queries (one 32-query MFMA block) for the whole key
// sweep, so its output accumulators, running max and running sum never leave
// registers.  Two wavefronts share each SIMD, so one's softmax (VALU) can run
// under the other's MFMAs.
//
// Key/value tiles (128 keys for 16-bit data) are copied from global memory
// straight into LDS by buffer->LDS loads, double-buffered in two LDS objects:
// the copy of tile t+1 runs while tile t is multiplied.  The buffer
// resource of each tile stops at the last key, so rows past the end arrive
// as zeros.  Rows are stored in LDS as they are in memory ([key][d]) with
// their 16-byte chunks XOR-permuted per row, which keeps both fragment reads
// below free of bank conflicts.
//
// Orientation: the kernel computes S^T = K . Q^T (keys as MFMA rows, queries
// as MFMA columns).  A 32x32 accumulator then gives each lane one query and
// 16 keys -- register r of lane l holds key 8(r/4) + 4(l/32) + r%4 of its
// 32-key block -- so a query's block max is local max operations plus one
// swap with lane^32, and the probabilities P^T are already in the B-operand
// layout of the second product O^T += V^T . P^T.  The A operand V^T comes
// from row-major V through the LDS transpose read (ds_read_b64_tr_b16): in
// each 16-lane group every lane reads 4 consecutive 16-bit values and lane
// 4a + e receives value e of lanes a, 4 + a, 8 + a and 12 + a.  Lane
// 16q + 4r + a reads key 4(q/2) + r of a 16-key half-block at d offset
// 16(q%2) + 4a, so lane l receives V[key][d = l % 32] for the four keys
// 4(l/32) + 0..3 -- the same keys, in the same order, as its P^T register
// run.  (For fp32 the MFMA takes one key per lane; V^T is read element-wise.)
//
// Softmax: logits are scaled by scale*log2(e) once; exponentials are exp2
// (v_exp_f32).  Each query keeps a reference max m and a running sum l per
// lane; the two lane halves of a query are summed once at the end.  Within a
// tile the QK product of the next 32-key block is issued in the same basic
// block as the softmax of the current one, so the MFMA pipe has independent
// work while the exponentials run.
//
// The layouts above are those of the 32x32x16 kernels (attn_bf16_kernel and
// the fp32 attn_fwd_kernel).  The bf16 default, attn_bf16_m16_kernel, keeps
// the work split, tiles, copies and softmax and changes the MFMA shape to
// 16x16x32; its own layouts are described where it is defined.
#include "launch.h"

#include <type_traits>

// bf16 kernel: 1 = 16x16x32 MFMAs (attn_bf16_m16_kernel, the default:
// 1.5-3.8 % faster on the 92840-token sweep), 0 = 32x32x16
// (attn_bf16_kernel, kept buildable as the reference point).
#ifndef H3_ATTN_MFMA16
#define H3_ATTN_MFMA16 1
#endif

namespace h3 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define H3_LDS_S4(p) ((__attribute__((address_space(3))) s16x4*)(p))

template <typename T> struct AttnMfma;

template <> struct AttnMfma<bf16> {
    // QK: a 32-byte chunk of head_dim is 16 bf16 = one MFMA
    __device__ __forceinline__ static void qk(f32x16& acc, const u32x4& a, const u32x4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

template <> struct AttnMfma<float> {
    // four v_mfma_f32_32x32x2_f32: lane group g holds d = 4g..4g+3 of the
    // 8-wide chunk, the j-th MFMA contracts d = j and d = 4 + j
    __device__ __forceinline__ static void qk(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc,
                                                       0, 0, 0);
    }
};

constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kBQ = kAttnWaves * 32;         // 256 queries per workgroup
// The reference max of a query only moves when a block's max exceeds it by
// more than this (log2 units), so probabilities stay <= 2^8 and the output
// rescale is skipped for most blocks; the result is unchanged because the
// final division uses the same reference.
constexpr float kLazyMax = 8.0f;
// Pipelined kernel: largest row sum of one block's exponentials (per lane, 16
// keys) accepted against the current reference before it is raised.  Bounds
// every exponential by 2^20, far inside fp32 range for the sums and outputs.
constexpr float kRedoSum = 1048576.0f;

// 16-byte chunk c of the row of key `key` sits at chunk c ^ swz(key).
template <int CH> __device__ __forceinline__ int kswz(int key) { return key & (CH >= 16 ? 15 : CH - 1); }
template <int CH> __device__ __forceinline__ int vswz(int key) {
    return CH >= 16 ? (key & 3) << 2 : (key & 2) << 1;
}

// Copy one K tile and one V tile into LDS (K at buf, V at buf + TILE): the
// wavefront's IPW 1 KB pieces of each, lane offsets precomputed in dk / dv.
template <int IPW, int TILE, typename T>
__device__ __forceinline__ void copy_kv_tile(char* buf, int wave, const T* Kp, const T* Vp, int64_t hoff, int kv0,
                                             int n, int bkv, int64_t ld, uint32_t ldb, const uint32_t* dk,
                                             const uint32_t* dv) {
    const int rem = n - kv0;
    // tiles past the end read as zeros; readfirstlane keeps the descriptor in
    // scalar registers (a clamp evaluated on the VALU would make it look divergent)
    const int nvalid = __builtin_amdgcn_readfirstlane(rem < 0 ? 0 : (rem < bkv ? rem : bkv));
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kp + (int64_t)kv0 * ld + hoff, (uint32_t)nvalid * ldb);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vp + (int64_t)kv0 * ld + hoff, (uint32_t)nvalid * ldb);
#pragma unroll
    for (int i = 0; i < IPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, H3_LDS(buf + (wave * IPW + i) * 1024), 16, dk[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < IPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, H3_LDS(buf + TILE + (wave * IPW + i) * 1024), 16, dv[i], 0, 0,
                                                 0);
}

// The same copy with the K and V tiles in separate LDS buffers.
template <int IPW>
__device__ __forceinline__ void copy_kv_tile2(char* kbuf, char* vbuf, int wave, const bf16* Kp, const bf16* Vp,
                                              int64_t hoff, int kv0, int n, int bkv, int64_t ld, uint32_t ldb,
                                              const uint32_t* dk, const uint32_t* dv) {
    const int rem = n - kv0;
    // tiles past the end read as zeros; readfirstlane keeps the descriptor in
    // scalar registers (a clamp evaluated on the VALU would make it look divergent)
    const int nvalid = __builtin_amdgcn_readfirstlane(rem < 0 ? 0 : (rem < bkv ? rem : bkv));
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kp + (int64_t)kv0 * ld + hoff, (uint32_t)nvalid * ldb);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vp + (int64_t)kv0 * ld + hoff, (uint32_t)nvalid * ldb);
#pragma unroll
    for (int i = 0; i < IPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, H3_LDS(kbuf + (wave * IPW + i) * 1024), 16, dk[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < IPW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, H3_LDS(vbuf + (wave * IPW + i) * 1024), 16, dv[i], 0, 0, 0);
}

// Clear `bytes` of LDS at p (a multiple of 16) with the workgroup's
// threads.  The K/V buffers are cleared once, before the first tile copy:
// keys past the end get P = 0, but 0 times bits left in LDS by an earlier
// workgroup (Inf or NaN among them) is not 0, and a buffer may be read
// before any tile has been copied into it (the sweep's padded tail) or
// hold rows a ragged tile did not fill.  Afterwards every buffer holds
// zeros or rows of an earlier tile, which are finite.
__device__ __forceinline__ void zero_lds(char* p, int bytes, int tid) {
    for (int o = tid * 16; o < bytes; o += kAttnThreads * 16) *reinterpret_cast<u32x4*>(p + o) = (u32x4){};
}

template <typename T, int HD>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ Kp, const T* __restrict__ Vp, int64_t ld,
    T* __restrict__ O, int64_t ldo, int32_t n, int32_t heads, float sl2, float* __restrict__ lse,
    int32_t nqt) {
    constexpr int ES = sizeof(T);
    constexpr int RB = HD * ES;                  // bytes of one K or V row
    constexpr int CH = RB / 16;                  // 16-byte chunks per row
    constexpr int BKV = RB <= 256 ? 128 : 64;    // keys per tile
    constexpr int NKB = BKV / 32;                // 32-key blocks per tile
    constexpr int TILE = BKV * RB;               // bytes of one operand tile
    constexpr int IPW = TILE / (1024 * kAttnWaves);   // 1 KB copies per wavefront per operand
    constexpr int NCH = RB / 32;                 // 32-byte MFMA k-chunks over head_dim
    constexpr int DB = HD / 32;                  // 32-wide d blocks of the output
    static_assert(IPW >= 1 && TILE % (1024 * kAttnWaves) == 0, "tile split");

    __shared__ __attribute__((aligned(1024))) char lds0[2 * TILE];   // [K tile | V tile]
    __shared__ __attribute__((aligned(1024))) char lds1[2 * TILE];

    // ---- workgroup -> (head, query tile); consecutive tiles on one XCD share a head
    const int G = heads * nqt;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = G >> 3, extra = G & 7;
    const int L = xcd * base + (xcd < extra ? xcd : extra) + local;
    const int head = L / nqt;
    const int qt = L - head * nqt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int q0 = qt * kBQ + wave * 32;
    const int64_t hoff = (int64_t)head * HD;
    const uint32_t ldb = (uint32_t)(ld * ES);    // bytes between key rows

    // ---- Q^T fragments (B operand): lane holds one query, 16 bytes of d per chunk
    u32x4 qf[NCH];
    {
        const int qi = q0 + col;
        const char* src = reinterpret_cast<const char*>(Q + (int64_t)(qi < n ? qi : n - 1) * ld + hoff);
#pragma unroll
        for (int c = 0; c < NCH; ++c) qf[c] = *reinterpret_cast<const u32x4*>(src + c * 32 + g * 16);
    }

    // ---- tile copies: LDS chunk p = 64 (wave IPW + i) + lane of a tile is
    //      chunk (p % CH) ^ swz(key) of key p / CH
    uint32_t dk[IPW], dv[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int p = 64 * (wave * IPW + i) + lane;
        const int key = p / CH, ph = p % CH;
        dk[i] = (uint32_t)key * ldb + (uint32_t)((ph ^ kswz<CH>(key)) << 4);
        dv[i] = (uint32_t)key * ldb + (uint32_t)((ph ^ vswz<CH>(key)) << 4);
    }
    // ---- fragment read offsets (constant per lane)
    // K chunk (2c + g) of key kb*32 + col
    uint32_t ko[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) ko[c] = (uint32_t)(col * RB + (((2 * c + g) ^ kswz<CH>(col)) << 4));
    // V transpose read: lane 16q + 4r + a reads key 4(q/2) + r of a 16-key
    // half-block and d = 32 db + 16(q%2) + 4a .. +3
    uint32_t vo[DB];
    {
        const int q = lane >> 4, r = (lane >> 2) & 3, a = lane & 3;
        const int kr = 4 * (q >> 1) + r;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int c = 4 * db + 2 * (q & 1) + (a >> 1);
            vo[db] = (uint32_t)(kr * RB + ((c ^ vswz<CH>(kr)) << 4) + (a & 1) * 8);
        }
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
    float m_run = -__builtin_inff(), l_run = 0.f;

    auto qk_block = [&](f32x16& s, const u32x4* kf) {
        s = (f32x16){};
#pragma unroll
        for (int c = 0; c < NCH; ++c) AttnMfma<T>::qk(s, kf[c], qf[c]);
    };

    auto tile = [&](const char* buf, int kv0) {
        const char* KB = buf;
        const char* VB = buf + TILE;
        u32x4 kf[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) kf[c] = *reinterpret_cast<const u32x4*>(KB + ko[c]);
        f32x16 s;
        qk_block(s, kf);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int kbase = kv0 + kb * 32;
            if (kbase >= n) break;                        // block entirely past the last key
            if (kbase + 32 > n) {                         // ragged block: keys past n get -inf
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kbase + 8 * (r >> 2) + 4 * g + (r & 3) >= n) s[r] = -__builtin_inff();
            }
            // K fragments of the next block (its QK runs under this block's softmax)
            if (kb + 1 < NKB) {
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    kf[c] = *reinterpret_cast<const u32x4*>(KB + (kb + 1) * 32 * RB + ko[c]);
            }
            // V^T fragments of this block
            u32x4 vf[DB][2];
            if constexpr (ES == 2) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const char* vp = VB + (kb * 32 + 16 * h) * RB + vo[db];
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(H3_LDS_S4(vp));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(H3_LDS_S4(vp + 8 * RB));
                        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                        vf[db][h] = (u32x4){l2[0], l2[1], h2[0], h2[1]};
                    }
            }

            // ---- softmax of this block: block max, lazily moved reference
            float mx = fmaxf(s[0], s[1]);
#pragma unroll
            for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * sl2;
            const bool grow = mx > m_run + kLazyMax;
            const float m_new = grow ? fmaxf(m_run, mx) : m_run;
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = fast_exp2(__builtin_fmaf(s[r], sl2, -m_new));
                rs += s[r];
            }
            l_run = __builtin_fmaf(l_run, alpha, rs);

            // ---- QK of the next block (independent MFMA work)
            f32x16 s_next;
            if (kb + 1 < NKB) qk_block(s_next, kf);

            if (__builtin_amdgcn_ballot_w64(grow)) {      // rare: some reference moved
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            }

            // ---- O^T += V^T P^T over this block
            if constexpr (ES == 2) {
                u32x4 pf[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int w = 0; w < 4; ++w) pf[h][w] = pack_bf16x2(s[8 * h + 2 * w], s[8 * h + 2 * w + 1]);
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, vf[db][h]), __builtin_bit_cast(bf16x8, pf[h]), oacc[db], 0,
                            0, 0);
            } else {
                // fp32: four 32x32x2 MFMAs per 8 keys; MFMA j of group c takes key 8c + 4g + j
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int d = db * 32 + col;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int key = kb * 32 + 8 * c + 4 * g + j;
                            const float v = *reinterpret_cast<const float*>(
                                VB + key * RB + (((d >> 2) ^ vswz<CH>(key)) << 4) + (d & 3) * 4);
                            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(v, s[4 * c + j], oacc[db], 0, 0, 0);
                        }
                }
            }
            if (kb + 1 < NKB) s = s_next;
        }
    };

    // Retire the Q loads before the key loop: otherwise the wait-count
    // analysis still sees them in flight there and makes the QK products
    // wait for tile copies as well.
    zero_lds(lds0, 2 * TILE, tid);
    zero_lds(lds1, 2 * TILE, tid);
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);
    const int ntiles = (n + BKV - 1) / BKV;
    copy_kv_tile<IPW, TILE>(lds0, wave, Kp, Vp, hoff, 0, n, BKV, ld, ldb, dk, dv);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
        if (t + 1 < ntiles) copy_kv_tile<IPW, TILE>(lds1, wave, Kp, Vp, hoff, (t + 1) * BKV, n, BKV, ld, ldb, dk, dv);
        tile(lds0, t * BKV);
        __builtin_amdgcn_s_waitcnt(0);    // this wave's copies into lds1 have landed
        __syncthreads();                  // ... everyone's, and lds0 is free again
        if (t + 1 >= ntiles) break;
        if (t + 2 < ntiles) copy_kv_tile<IPW, TILE>(lds0, wave, Kp, Vp, hoff, (t + 2) * BKV, n, BKV, ld, ldb, dk, dv);
        tile(lds1, (t + 1) * BKV);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- normalise and store: O^T lane (query, g) holds d = 32db + 8(r/4) + 4g + r%4
    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    const float inv = 1.0f / l_tot;
    const int qi = q0 + col;
    if (qi < n) {
        T* orow = O + (int64_t)qi * ldo + hoff;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * g;
                const f32x16& a = oacc[db];
                if constexpr (ES == 2) {
                    *reinterpret_cast<u32x2*>(orow + d) =
                        (u32x2){pack_bf16x2(a[4 * r4] * inv, a[4 * r4 + 1] * inv),
                                pack_bf16x2(a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv)};
                } else {
                    *reinterpret_cast<f32x4*>(orow + d) =
                        (f32x4){a[4 * r4] * inv, a[4 * r4 + 1] * inv, a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv};
                }
            }
        if (lse && g == 0) lse[(int64_t)head * n + qi] = m_run * 0.69314718055994531f + __logf(l_tot);
    }
}

// ---------------------------------------------------------------- bf16: pipelined key sweep
// Same work split (8 wavefronts x 32 queries) and fragment layouts as above;
// the key sweep of each wavefront is software-pipelined over 32-key blocks.
// Iteration j issues QK of block j+1 (one MFMA per 32-byte chunk of
// head_dim) interleaved with the exponentials of block j, then PV of block
// j (one MFMA per d block and key half) with the V^T reads of block j+1, all
// in one basic block: a wavefront's own independent VALU instructions are
// what issue while its MFMAs execute.
//
// LDS: K and V tiles of 64 keys (2 blocks) in a ring of four buffers per
// operand (128 KB in all; a workgroup above 128 KB of LDS was measured to
// run its loop a sixth slower), each operand's buffers declared together so
// that every fragment address is a per-lane base plus an immediate offset.
// K fragments of block b are read in iteration b-2, V^T fragments in
// iteration b-1, so tile u is read in iterations 2u-2 .. 2u.  One barrier per
// tile, before iteration 2u, makes tile u+1 visible (its copies went out two
// barriers earlier, tile u+2's one barrier earlier) and frees the buffer of
// tile u-1, whose reads ended in iteration 2u-2, for the copy of tile u+3.
// Copies are issued for every tile, past the end too (they read zeros), so
// each wait can leave exactly one tile's copies outstanding.
template <int HD>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Kp, const bf16* __restrict__ Vp, int64_t ld,
    bf16* __restrict__ O, int64_t ldo, int32_t n, int32_t heads, float sl2, float* __restrict__ lse,
    int32_t nqt) {
    constexpr int RB = HD * 2;                   // bytes of one K or V row
    constexpr int CH = RB / 16;                  // 16-byte chunks per row
    constexpr int BKV = 64;                      // keys per tile (2 blocks)
    constexpr int TILE = BKV * RB;               // bytes of one operand tile
    constexpr int IPW = TILE / (1024 * kAttnWaves);
    constexpr int NCH = RB / 32;                 // QK MFMAs per block
    constexpr int DB = HD / 32;                  // 32-wide d blocks of the output
    constexpr int NPV = 2 * DB;                  // PV MFMAs per block
    static_assert(IPW >= 1 && IPW <= 2 && TILE % (1024 * kAttnWaves) == 0, "tile split (two copy slots per step)");
    static_assert(16 % NCH == 0, "exponentials spread evenly over the QK slots");

    // Four K then four V tile buffers: each operand's ring lies in one
    // window of at most 64 KB.  Separate objects let the compiler see that
    // a copy into one buffer leaves reads of the others free to proceed.
    __shared__ __attribute__((aligned(1024))) char k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds2[TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds3[TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds2[TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds3[TILE];
    auto kbuf = [&](int i) __attribute__((always_inline)) -> char* {
        return i == 0 ? k_lds0 : i == 1 ? k_lds1 : i == 2 ? k_lds2 : k_lds3;
    };
    auto vbuf = [&](int i) __attribute__((always_inline)) -> char* {
        return i == 0 ? v_lds0 : i == 1 ? v_lds1 : i == 2 ? v_lds2 : v_lds3;
    };
    constexpr int CPT = 2 * IPW;                 // copies per tile and wavefront

    const int G = heads * nqt;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = G >> 3, extra = G & 7;
    const int L = xcd * base + (xcd < extra ? xcd : extra) + local;
    const int head = L / nqt;
    const int qt = L - head * nqt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int q0 = qt * kBQ + wave * 32;
    const int64_t hoff = (int64_t)head * HD;
    const uint32_t ldb = (uint32_t)(ld * 2);

    u32x4 qf[NCH];
    {
        const int qi = q0 + col;
        const char* src = reinterpret_cast<const char*>(Q + (int64_t)(qi < n ? qi : n - 1) * ld + hoff);
#pragma unroll
        for (int c = 0; c < NCH; ++c) qf[c] = *reinterpret_cast<const u32x4*>(src + c * 32 + g * 16);
    }
    uint32_t ko[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) ko[c] = (uint32_t)(col * RB + (((2 * c + g) ^ kswz<CH>(col)) << 4));
    uint32_t vo[DB];
    {
        const int q = lane >> 4, r = (lane >> 2) & 3, a = lane & 3;
        const int kr = 4 * (q >> 1) + r;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int c = 4 * db + 2 * (q & 1) + (a >> 1);
            vo[db] = (uint32_t)(kr * RB + ((c ^ vswz<CH>(kr)) << 4) + (a & 1) * 8);
        }
    }

    // Hide the offsets' value range from the compiler: otherwise it proves
    // offset and block displacement bit-disjoint and builds each address with
    // a v_or instead of the instruction's immediate offset.
#pragma unroll
    for (int c = 0; c < NCH; ++c) asm volatile("" : "+v"(ko[c]));
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(vo[db]));

    const int NB = (n + 31) >> 5;    // 32-key blocks
    const int NBF = n >> 5;          // blocks with 32 valid keys

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
    float m_ref, l_run = 0.f;
    f32x16 s;              // logits of the block whose softmax is next
    u32x4 kf[NCH];         // K fragments of the next QK
    u32x4 vf[DB][2];       // V^T fragments of the next PV

    // LDS copy of tile t into kb / vb (lane offsets recomputed: they serve once per tile)
    auto copy_tile = [&](char* kb, char* vb, int t) __attribute__((always_inline)) {
        uint32_t dk[IPW], dv[IPW];
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int p = 64 * (wave * IPW + i) + lane;
            const int key = p / CH, ph = p % CH;
            dk[i] = (uint32_t)key * ldb + (uint32_t)((ph ^ kswz<CH>(key)) << 4);
            dv[i] = (uint32_t)key * ldb + (uint32_t)((ph ^ vswz<CH>(key)) << 4);
        }
        copy_kv_tile2<IPW>(kb, vb, wave, Kp, Vp, hoff, t * BKV, n, BKV, ld, ldb, dk, dv);
    };
    // One 1 KB piece of tile t (operand op: 0 K, 1 V; piece i of this
    // wavefront's share) into dst, for copies spread over a step's MFMAs.
    auto copy_piece = [&](char* dst, int t, int op, int i) __attribute__((always_inline)) {
        const int p = 64 * (wave * IPW + i) + lane;
        const int key = p / CH, ph = p % CH;
        const uint32_t off = (uint32_t)key * ldb + (uint32_t)((ph ^ (op ? vswz<CH>(key) : kswz<CH>(key))) << 4);
        const int rem = n - t * BKV;
        const int nvalid = __builtin_amdgcn_readfirstlane(rem < 0 ? 0 : (rem < BKV ? rem : BKV));
        const __amdgpu_buffer_rsrc_t r =
            buffer_rsrc((op ? Vp : Kp) + (int64_t)t * BKV * ld + hoff, (uint32_t)nvalid * ldb);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, H3_LDS(dst + (wave * IPW + i) * 1024), 16, off, 0, 0, 0);
    };
    auto read_k1 = [&](const char* buf, int blk, int c) __attribute__((always_inline)) {
        kf[c] = *reinterpret_cast<const u32x4*>(buf + blk * 32 * RB + ko[c]);
    };
    auto read_v1 = [&](const char* buf, int blk, int db, int h) __attribute__((always_inline)) {
        const char* vp = buf + blk * 32 * RB + 16 * h * RB + vo[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(H3_LDS_S4(vp));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(H3_LDS_S4(vp + 8 * RB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        vf[db][h] = (u32x4){l2[0], l2[1], h2[0], h2[1]};
    };
    auto mask = [&](f32x16& acc, int kbase) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (kbase + 8 * (r >> 2) + 4 * g + (r & 3) >= n) acc[r] = -__builtin_inff();
    };
    // scaled max of a block for this lane's query (both lane halves)
    auto block_max = [&](const f32x16& a) __attribute__((always_inline)) -> float {
        float mx = __builtin_fmaxf(__builtin_fmaxf(a[0], a[1]), a[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, a[r]), a[r + 1]);
        mx = __builtin_fmaxf(mx, a[15]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        return __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
    };
    // Exponentials of block j under the current reference, packed as bf16
    // pairs (the B operand of PV); rs = their row sum over this lane's 16 keys,
    // taken from the packed values with v_dot2 (the weights PV sees).
    auto softmax_exp = [&](u32x4 (&pfr)[2], float& rs) __attribute__((always_inline)) {
        const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
        rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(__builtin_fmaf(s[r], sl2, -m_ref));
            const float p1 = fast_exp2(__builtin_fmaf(s[r + 1], sl2, -m_ref));
            const uint32_t w = pack_bf16x2(p0, p1);
            pfr[r >> 3][(r >> 1) & 3] = w;
            rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one2, rs, false);
        }
    };

    // One iteration.  Blocks past the last key hold zeros or rows of an
    // earlier tile (the buffers are cleared before the first copy) and are
    // masked to -inf here, so the sweep may run a few blocks past the end at
    // no cost to the result.  Only the last trips test
    // for that (CHECK).
    //
    // Reference: the exponentials of block j are taken against the current
    // reference without first computing the block max; only if some query's
    // row sum over the block comes out above kRedoSum (or not finite) is the
    // block max taken, the reference raised, the output and sum rescaled and
    // the exponentials redone.  Every exponential the sums and PV see is
    // therefore at most kRedoSum, and the result is the same softmax: the
    // final division uses the same reference.
    //
    // kp/b2: buffer and block of block j+2's K (prefetched); vb/b1: those of
    // block j+1's V^T.
    // cps(c): this step's share of tile copies, issued after QK MFMA c
    auto step = [&](int j, auto chk, const char* kp, int b2, const char* vb, int b1, auto cps)
                    __attribute__((always_inline)) {
        constexpr bool CHECK = decltype(chk)::value;   // block j+1 may hold keys past the end
        f32x16 sn = (f32x16){};
        u32x4 pfr[2];
        float rs;
        // ---- QK of block j+1 and block j+2's K reads, exponentials of block j
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[c]),
                                                         __builtin_bit_cast(bf16x8, qf[c]), sn, 0, 0, 0);
            read_k1(kp, b2, c);
            cps(c);
        }
        softmax_exp(pfr, rs);
        // Issue order: each QK MFMA with one K read, a tile copy after MFMAs
        // 1 and 5, and its share of the exponentials (fma, exp, fma, exp,
        // pack, dot2).
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (c == 1 || c == 5) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 48 / NCH, 0);
        }
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(rs <= kRedoSum)) != 0, 0)) {   // rare: raise the reference
            const float mx = block_max(s);
            const float m_new = __builtin_fmaxf(m_ref, mx);
            const float alpha = fast_exp2(m_ref - m_new);
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            l_run *= alpha;
            m_ref = m_new;
            softmax_exp(pfr, rs);
        }
        // ---- PV of block j, V^T fragments of block j+1
#pragma unroll
        for (int k = 0; k < NPV; ++k) {
            const int db = k >> 1, h = k & 1;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[db][h]),
                                                               __builtin_bit_cast(bf16x8, pfr[h]), oacc[db], 0, 0, 0);
            read_v1(vb, b1, db, h);
        }
        l_run += rs;
        if (CHECK && __builtin_expect(j + 1 >= NBF, 0)) mask(sn, (j + 1) * 32);
        s = sn;
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // Barrier before iteration 2u: this wavefront's copies of tile u+1 have
    // landed (only tile u+2's may be outstanding), then everyone's have;
    // tile u-1's buffer takes tile u+3.  No LDS read needs draining: the
    // last reads of tile u-1 were in iteration 2u-2.  The copies of tile
    // u+3 go out a piece at a time inside iterations 2u (K) and 2u+1 (V),
    // all before the next barrier, so each wait still leaves exactly one
    // tile's copies in flight (a burst of every wavefront's copies right
    // after the barrier held their MFMAs back).
    auto nocp = [](int) __attribute__((always_inline)) {};
    // Iterations j .. j+7 for j = 8w + 2 (tiles 4w+1 .. 4w+5): ring
    // positions are compile-time constants.
    auto trip = [&](int j, auto chk) __attribute__((always_inline)) {
        const int u = j >> 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = u + i / 2 + 3, op = i & 1;
            char* dst = op ? vbuf((i / 2) % 4) : kbuf((i / 2) % 4);
            if (op == 0) {
                wait_vm<CPT, false>();
                __builtin_amdgcn_s_barrier();
            }
            auto cps = [&](int c) __attribute__((always_inline)) {
                if (c == 1) copy_piece(dst, t, op, 0);
                if (c == 5 && IPW > 1) copy_piece(dst, t, op, 1);
            };
            step(j + i, chk, kbuf(((4 + i) / 2) % 4), i & 1, vbuf(((3 + i) / 2) % 4), (i + 1) & 1, cps);
        }
    };

    // ---- prologue: tiles 0 and 1 visible, tiles 2 and 3 in flight; block
    //      0's logits and V^T, block 1's K
    zero_lds(k_lds0, TILE, tid);
    zero_lds(k_lds1, TILE, tid);
    zero_lds(k_lds2, TILE, tid);
    zero_lds(k_lds3, TILE, tid);
    zero_lds(v_lds0, TILE, tid);
    zero_lds(v_lds1, TILE, tid);
    zero_lds(v_lds2, TILE, tid);
    zero_lds(v_lds3, TILE, tid);
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);
    copy_tile(k_lds0, v_lds0, 0);
    copy_tile(k_lds1, v_lds1, 1);
    copy_tile(k_lds2, v_lds2, 2);
    copy_tile(k_lds3, v_lds3, 3);
    wait_vm<2 * CPT, false>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int c = 0; c < NCH; ++c) read_k1(k_lds0, 0, c);
    s = (f32x16){};
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[c]), __builtin_bit_cast(bf16x8, qf[c]),
                                                   s, 0, 0, 0);
    if (NBF == 0) mask(s, 0);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) read_v1(v_lds0, 0, db, h);
    m_ref = block_max(s);
#pragma unroll
    for (int c = 0; c < NCH; ++c) read_k1(k_lds0, 1, c);
    step(0, T_{}, k_lds1, 0, v_lds0, 1, nocp);
    step(1, T_{}, k_lds1, 1, v_lds1, 0, nocp);
    int j = 2;
    for (; j + 8 < NBF; j += 8) trip(j, F_{});   // blocks up to j + 8 complete
    for (; j < NB; j += 8) trip(j, T_{});
    wait_vm<0, true>();    // no tile copy may land after the workgroup's LDS is released

    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    const float inv = 1.0f / l_tot;
    const int qi = q0 + col;
    if (qi < n) {
        bf16* orow = O + (int64_t)qi * ldo + hoff;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * g;
                const f32x16& a = oacc[db];
                *reinterpret_cast<u32x2*>(orow + d) =
                    (u32x2){pack_bf16x2(a[4 * r4] * inv, a[4 * r4 + 1] * inv),
                            pack_bf16x2(a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv)};
            }
        if (lse && g == 0) lse[(int64_t)head * n + qi] = m_ref * 0.69314718055994531f + __logf(l_tot);
    }
}

// ---------------------------------------------------------------- bf16 on 16x16x32 MFMAs
// The same work split, tile ring, copies and barriers as attn_bf16_kernel,
// on v_mfma_f32_16x16x32_bf16 instead of 32x32x16: the same flops in twice
// as many MFMAs, which on this part draw less power, so the clock settles
// about 10 % higher under the same load.  Twice the MFMA issues leave less
// room beside them for the exponentials, so those are spread evenly: the
// key-tile-1 half of block j's exponentials runs beside QK of block j+1,
// the key-tile-0 half of block j+1's beside PV of block j (1.5 VALU
// instructions per MFMA throughout; with all of a block's exponentials in
// one phase this kernel was no faster than the 32x32x16 one).
//
// Layouts (lane l, c = l % 16, g = l / 16).  A 16x16x32 MFMA takes from
// lane l row c of A and column c of B over k = 8g .. 8g+7, and leaves rows
// 4g .. 4g+3 of column c of D in lane l.
//   QK: S^T = K . Q^T per (16-key tile kt, 16-query tile t, 32-wide d chunk
//       cc): lane l supplies K[key 16kt + c][d 32cc + 8g ..] from LDS and
//       Q[query 16t + c][d 32cc + 8g ..] from registers, and holds the
//       logits of keys 16kt + 4g + i (i < 4) for query 16t + c.
//   PV: O^T += V^T . P^T per 16-wide d tile and query tile, the 32 keys of
//       a block as the MFMA's k.  Lane l's B operand is its own 8 weights
//       of query 16t + c: keys 4g + i (tile 0) then 16 + 4g + i (tile 1),
//       taken as k = 8g .. 8g+7, so P needs no shuffle.  The A operand
//       must put V[same keys][d] in the same k slots: the transposing read
//       (in each 16-lane group lane 4a+e receives value e of lanes a, 4+a,
//       8+a, 12+a) delivers that when source lane 16g + 4j + a reads the four
//       d values 4a .. 4a+3 of the tile from key 4g + j (and 16 + 4g + j for
//       the second half).
// V rows are stored with their 16-byte chunks XOR-ed by 2 (key mod 8), so
// the 16 rows x 32 bytes of one transposing read fall two per bank slot.
template <int CH> __device__ __forceinline__ int vswz16(int key) {
    return CH >= 16 ? (key & 7) << 1 : ((key >> 1) & 3) << 1;
}

template <int HD>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_bf16_m16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Kp, const bf16* __restrict__ Vp, int64_t ld,
    bf16* __restrict__ O, int64_t ldo, int32_t n, int32_t heads, float sl2, float* __restrict__ lse,
    int32_t nqt) {
    constexpr int RB = HD * 2;                   // bytes of one K or V row
    constexpr int CH = RB / 16;                  // 16-byte chunks per row
    constexpr int BKV = 64;                      // keys per tile (2 blocks)
    constexpr int TILE = BKV * RB;               // bytes of one operand tile
    constexpr int IPW = TILE / (1024 * kAttnWaves);
    constexpr int NC = HD / 32;                  // 32-wide d chunks (QK)
    constexpr int DT = HD / 16;                  // 16-wide d tiles (PV, output)
    constexpr int NG = 2 * NC;                   // QK groups of two MFMAs per block
    static_assert(IPW >= 1 && IPW <= 2 && TILE % (1024 * kAttnWaves) == 0, "tile split (two copy slots per step)");
    static_assert(48 % NG == 0, "exponentials spread evenly over the QK groups");

    // V's ring first: its eight per-lane read offsets then reach every V
    // buffer through the read's 16-bit immediate; K's four take one base.
    __shared__ __attribute__((aligned(1024))) char v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds2[TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds3[TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds2[TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds3[TILE];
    auto kbuf = [&](int i) __attribute__((always_inline)) -> char* {
        return i == 0 ? k_lds0 : i == 1 ? k_lds1 : i == 2 ? k_lds2 : k_lds3;
    };
    auto vbuf = [&](int i) __attribute__((always_inline)) -> char* {
        return i == 0 ? v_lds0 : i == 1 ? v_lds1 : i == 2 ? v_lds2 : v_lds3;
    };
    constexpr int CPT = 2 * IPW;                 // copies per tile and wavefront

    const int G = heads * nqt;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = G >> 3, extra = G & 7;
    const int L = xcd * base + (xcd < extra ? xcd : extra) + local;
    const int head = L / nqt;
    const int qt = L - head * nqt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;
    const int q0 = qt * kBQ + wave * 32;
    const int64_t hoff = (int64_t)head * HD;
    const uint32_t ldb = (uint32_t)(ld * 2);

    u32x4 qf[2][NC];                             // Q fragments: [query tile][d chunk]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int qi = q0 + 16 * t + c16;
        const char* src = reinterpret_cast<const char*>(Q + (int64_t)(qi < n ? qi : n - 1) * ld + hoff);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) qf[t][cc] = *reinterpret_cast<const u32x4*>(src + cc * 64 + g * 16);
    }
    uint32_t ko[NC];                             // K read: row c16 of a 16-key tile, chunk 4cc + g
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) ko[cc] = (uint32_t)(c16 * RB + (((4 * cc + g) ^ kswz<CH>(c16)) << 4));
    uint32_t vo[DT];                             // V^T read: key 4g + j, d 16db + 4a
    {
        const int j = (lane >> 2) & 3, a = lane & 3;
        const int kr = 4 * g + j;
#pragma unroll
        for (int db = 0; db < DT; ++db)
            vo[db] = (uint32_t)(kr * RB + (((2 * db + (a >> 1)) ^ vswz16<CH>(kr)) << 4) + (a & 1) * 8);
    }
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) asm volatile("" : "+v"(ko[cc]));
#pragma unroll
    for (int db = 0; db < DT; ++db) asm volatile("" : "+v"(vo[db]));

    const int NB = (n + 31) >> 5;    // 32-key blocks
    const int NBF = n >> 5;          // blocks with 32 valid keys

    f32x4 oacc[DT][2];
#pragma unroll
    for (int db = 0; db < DT; ++db) oacc[db][0] = oacc[db][1] = (f32x4){};
    float m_ref[2], l_run[2] = {0.f, 0.f};
    f32x4 s[2][2];         // [key tile][query tile] logits of the block whose softmax is next
    u32x4 kf[2][NC];       // K fragments of the next QK: [key tile][d chunk]
    u32x4 vf[3];           // V^T fragments of the current PV, three d tiles ahead

    auto mfma16 = [](const u32x4& a, const u32x4& b, f32x4 c) __attribute__((always_inline)) -> f32x4 {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    };
    // one 1 KB piece (operand op: 0 K, 1 V; piece i of this wavefront) of tile t into dst
    auto copy_piece = [&](char* dst, int t, int op, int i) __attribute__((always_inline)) {
        const int p = 64 * (wave * IPW + i) + lane;
        const int key = p / CH, ph = p % CH;
        const uint32_t off = (uint32_t)key * ldb + (uint32_t)((ph ^ (op ? vswz16<CH>(key) : kswz<CH>(key))) << 4);
        const int rem = n - t * BKV;
        const int nvalid = __builtin_amdgcn_readfirstlane(rem < 0 ? 0 : (rem < BKV ? rem : BKV));
        const __amdgpu_buffer_rsrc_t r =
            buffer_rsrc((op ? Vp : Kp) + (int64_t)t * BKV * ld + hoff, (uint32_t)nvalid * ldb);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, H3_LDS(dst + (wave * IPW + i) * 1024), 16, off, 0, 0, 0);
    };
    auto read_k = [&](const char* buf, int blk, int kt, int cc) __attribute__((always_inline)) {
        kf[kt][cc] = *reinterpret_cast<const u32x4*>(buf + blk * 32 * RB + kt * 16 * RB + ko[cc]);
    };
    auto read_v = [&](const char* buf, int blk, int db) __attribute__((always_inline)) {
        const char* vp = buf + blk * 32 * RB + vo[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(H3_LDS_S4(vp));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(H3_LDS_S4(vp + 16 * RB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        vf[db % 3] = (u32x4){l2[0], l2[1], h2[0], h2[1]};
    };
    auto mask = [&](f32x4 (&acc)[2][2], int kbase) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kbase + 16 * kt + 4 * g + i >= n) acc[kt][0][i] = acc[kt][1][i] = -__builtin_inff();
    };
    // scaled max of a block for query tile t (the four lanes of a query)
    auto block_max = [&](int t) __attribute__((always_inline)) -> float {
        float mx = __builtin_fmaxf(__builtin_fmaxf(s[0][t][0], s[0][t][1]), __builtin_fmaxf(s[0][t][2], s[0][t][3]));
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(s[1][t][0], s[1][t][1]),
                                                  __builtin_fmaxf(s[1][t][2], s[1][t][3])));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, kWave));
        return mx * sl2;
    };
    // exponentials of key tile kt of the logits sv under the current
    // references, into pfr[t] words 2kt, 2kt+1; rs[t] = their sum.  Written
    // stage by stage (all eight fmas, then the exponentials, the packs, the
    // sums) so that the VALU groups placed beside each MFMA pair hold
    // independent instructions: half the hazard nops of the per-pair order,
    // same values.
    auto softmax_half = [&](const f32x4 (&sv)[2][2], int kt, u32x4 (&pfr)[2], float (&rs)[2])
                            __attribute__((always_inline)) {
        const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
        float x[2][4];
        uint32_t w[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[t][i] = __builtin_fmaf(sv[kt][t][i], sl2, -m_ref[t]);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[t][i] = fast_exp2(x[t][i]);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                w[t][i] = pack_bf16x2(x[t][2 * i], x[t][2 * i + 1]);
                pfr[t][2 * kt + i] = w[t][i];
            }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            rs[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[t][0]), one2, 0.f, false);
            rs[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[t][1]), one2, rs[t], false);
        }
    };
    // exponentials of a block under the current references, packed as bf16
    // pairs in PV's k order; rs[t] = their sum over this lane's 8 keys
    auto softmax_exp = [&](u32x4 (&pfr)[2], float (&rs)[2]) __attribute__((always_inline)) {
        const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            rs[t] = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float p0 = fast_exp2(__builtin_fmaf(s[kt][t][i], sl2, -m_ref[t]));
                    const float p1 = fast_exp2(__builtin_fmaf(s[kt][t][i + 1], sl2, -m_ref[t]));
                    const uint32_t w = pack_bf16x2(p0, p1);
                    pfr[t][2 * kt + (i >> 1)] = w;
                    rs[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one2, rs[t], false);
                }
        }
    };

    // One iteration: QK of block j+1 (with block j+2's K reads and the first
    // three V^T tiles of block j) beside the key-tile-1 exponentials of
    // block j; the rare reference raise, decided on block j's whole row sum;
    // then PV of block j, reading its V^T three d tiles ahead (holding a
    // whole block of V^T fragments a block ahead, as attn_bf16_kernel does,
    // does not fit in the registers here), beside the key-tile-0
    // exponentials of block j+1 -- taken after the raise, so always against
    // the reference block j+1's other half will use.
    // kp/b2: buffer and block of block j+2's K; vb/b0: those of block j's V.
    // Carried between iterations: block j's key-tile-0 weights (words 0, 1
    // of pfr_a[t]) and their row sums, computed beside the previous PV.
    u32x4 pfr_a[2];
    float rs_a[2];
    auto step = [&](int j, auto chk, const char* kp, int b2, const char* vb, int b0, auto cps)
                    __attribute__((always_inline)) {
        constexpr bool CHECK = decltype(chk)::value;
        f32x4 sn[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sn[kt][0] = sn[kt][1] = (f32x4){};
        u32x4 pfr[2] = {pfr_a[0], pfr_a[1]};
        float rs_b[2];
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sn[kt][0] = mfma16(kf[kt][cc], qf[0][cc], sn[kt][0]);
                sn[kt][1] = mfma16(kf[kt][cc], qf[1][cc], sn[kt][1]);
                read_k(kp, b2, kt, cc);
                cps(2 * cc + kt);
            }
#pragma unroll
        for (int db = 0; db < 3; ++db) read_v(vb, b0, db);
        softmax_half(s, 1, pfr, rs_b);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (gi < NG - 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            if (gi == 1 || gi == (NG > 5 ? 5 : NG - 1)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 24 / NG, 0);
        }
        float rs[2] = {rs_a[0] + rs_b[0], rs_a[1] + rs_b[1]};
        if (CHECK && __builtin_expect(j + 1 >= NBF, 0)) mask(sn, (j + 1) * 32);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(rs[0] <= kRedoSum) || !(rs[1] <= kRedoSum)) != 0, 0)) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float m_new = __builtin_fmaxf(m_ref[t], block_max(t));
                const float alpha = fast_exp2(m_ref[t] - m_new);
#pragma unroll
                for (int db = 0; db < DT; ++db) oacc[db][t] *= alpha;
                l_run[t] *= alpha;
                m_ref[t] = m_new;
            }
            softmax_exp(pfr, rs);
        }
        float rs_n[2];
        softmax_half(sn, 0, pfr_a, rs_n);       // block j+1's key tile 0, beside PV(j)
#pragma unroll
        for (int db = 0; db < DT; ++db) {
            oacc[db][0] = mfma16(vf[db % 3], pfr[0], oacc[db][0]);
            oacc[db][1] = mfma16(vf[db % 3], pfr[1], oacc[db][1]);
            if (db + 3 < DT) read_v(vb, b0, db + 3);
        }
#pragma unroll
        for (int db = 0; db < DT; ++db) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (db + 3 < DT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 24 / DT, 0);
        }
        l_run[0] += rs[0];
        l_run[1] += rs[1];
        rs_a[0] = rs_n[0];
        rs_a[1] = rs_n[1];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[kt][0] = sn[kt][0], s[kt][1] = sn[kt][1];
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    auto nocp = [](int) __attribute__((always_inline)) {};
    // Barrier before iteration 2u; the copies of tile u+3 go out a piece at
    // a time inside iterations 2u (K) and 2u+1 (V).  See attn_bf16_kernel.
    auto trip = [&](int j, auto chk) __attribute__((always_inline)) {
        const int u = j >> 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = u + i / 2 + 3, op = i & 1;
            char* dst = op ? vbuf((i / 2) % 4) : kbuf((i / 2) % 4);
            if (op == 0) {
                wait_vm<CPT, false>();
                __builtin_amdgcn_s_barrier();
            }
            auto cps = [&](int gi) __attribute__((always_inline)) {
                if (gi == 1) copy_piece(dst, t, op, 0);
                if (gi == (NG > 5 ? 5 : NG - 1) && IPW > 1) copy_piece(dst, t, op, 1);
            };
            step(j + i, chk, kbuf(((4 + i) / 2) % 4), i & 1, vbuf(((2 + i) / 2) % 4), i & 1, cps);
        }
    };

    // ---- prologue: tiles 0 and 1 visible, tiles 2 and 3 in flight; block
    //      0's logits and V^T, block 1's K
    zero_lds(k_lds0, TILE, tid);
    zero_lds(k_lds1, TILE, tid);
    zero_lds(k_lds2, TILE, tid);
    zero_lds(k_lds3, TILE, tid);
    zero_lds(v_lds0, TILE, tid);
    zero_lds(v_lds1, TILE, tid);
    zero_lds(v_lds2, TILE, tid);
    zero_lds(v_lds3, TILE, tid);
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            copy_piece(kbuf(t), t, 0, i);
            copy_piece(vbuf(t), t, 1, i);
        }
    wait_vm<2 * CPT, false>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) read_k(k_lds0, 0, kt, cc);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt][0] = s[kt][1] = (f32x4){};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt][0] = mfma16(kf[kt][cc], qf[0][cc], s[kt][0]);
            s[kt][1] = mfma16(kf[kt][cc], qf[1][cc], s[kt][1]);
        }
    if (NBF == 0) mask(s, 0);
    m_ref[0] = block_max(0);
    m_ref[1] = block_max(1);
    softmax_half(s, 0, pfr_a, rs_a);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) read_k(k_lds0, 1, kt, cc);
    step(0, T_{}, k_lds1, 0, v_lds0, 0, nocp);
    step(1, T_{}, k_lds1, 1, v_lds0, 1, nocp);
    int j = 2;
    for (; j + 8 < NBF; j += 8) trip(j, F_{});
    for (; j < NB; j += 8) trip(j, T_{});
    wait_vm<0, true>();    // no tile copy may land after the workgroup's LDS is released

#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float l_tot = l_run[t] + __shfl_xor(l_run[t], 16, kWave);
        l_tot += __shfl_xor(l_tot, 32, kWave);
        const float inv = 1.0f / l_tot;
        const int qi = q0 + 16 * t + c16;
        if (qi < n) {
            bf16* orow = O + (int64_t)qi * ldo + hoff + 4 * g;
#pragma unroll
            for (int db = 0; db < DT; ++db) {
                const f32x4& a = oacc[db][t];
                *reinterpret_cast<u32x2*>(orow + 16 * db) =
                    (u32x2){pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)};
            }
            if (lse && g == 0) lse[(int64_t)head * n + qi] = m_ref[t] * 0.69314718055994531f + __logf(l_tot);
        }
    }
}

// ---------------------------------------------------------------- fp8 attention
// head_dim 128, operands from the fp8 quantisation of q, k and v: Q8 and K8
// [n][heads * 128] e4m3 codes, VT [heads][128][n_pad] (v transposed, each
// 64-key group permuted into the byte order in which P is packed below), q
// scales per (head, token), k and v scales per head.
//
// 8 wavefronts x 32 queries, 64-key tiles on v_mfma_f32_32x32x64_f8f6f4.
// Per tile a wavefront runs two blocks:
//   V(t): the exponentials of tile t's logits, packed to e4m3, while the K
//         fragments of tile t+1 are read;
//   M(t): the V^T fragments of tile t are read while QK of tile t+1 runs
//         (2 key halves x 2 d chunks), then PV of tile t (4 d blocks of 32
//         keys x 64 -- P^T is the B operand, 32 bytes per lane: the 16
//         values a lane holds of each key half) and a fifth PV MFMA whose A
//         operand is all ones, so every row of that accumulator is the row
//         sum of exactly the fp8 weights PV used.
// At 246+ VGPRs two wavefronts share a SIMD.  If both ran the same block at
// the same time, one unit (matrix core or VALU) would idle, so the two
// wavefronts of each SIMD take opposite roles: one runs half a step behind
// the other, and a barrier ends every half step.  Each SIMD then overlaps
// one wavefront's exponentials with the other's MFMAs.  The roles come from
// the SIMD id the hardware reports and an LDS counter per SIMD, so they do
// not depend on how wavefronts are placed.
//
// Softmax: x = s * sl2 * sq[query] * sk[head] - m_ref, p = 2^(x + 4): a key
// at the reference gets weight 16, so keys down to 2^-13 of it still count
// (e4m3's smallest subnormal is 2^-9) and the reference may be overtaken by
// up to 4.8 (base 2) before a weight passes 448, e4m3's largest finite
// value; for logits of unit spread the first tile's maximum is within that
// of the row's, so a tile rarely has to be redone.  A tile whose largest p
// exceeds 448 raises the reference to its max first.  The output is
// O * sv[head] / l.
//
// LDS: a ring of kF8Buf K tiles (64 keys x 128 bytes) and V^T tiles (128 d
// rows x 64 bytes), 16-byte slots XOR-swizzled by row (K: (row / 2) % 8,
// V^T: (row / 4) % 4) so each half-wavefront fragment read hits 16 distinct
// slots.  Half steps are numbered h = 0, 1, ...; the leading wavefronts run
// V(t) in half step 2t and M(t) in 2t+1, the trailing ones V(t) in 2t+1 and
// M(t) in 2t+2.  Tile u is read in half steps 2u-2 .. 2u+2; at the start of
// half step 2j every wavefront issues its share of tile j+kF8Buf-2 into the
// buffer of tile j-2.  Odd half steps end with the wavefront's LDS reads
// complete and all but its last kF8Buf-4 copies landed (tile j+2 at the end
// of half step 2j+1), then the barrier.  That count is exact only because
// every wave issues the copies of every tile, past the last tile too (those
// read zeros): with fewer copies in flight the wait would let the tile read
// next still be on its way.
constexpr int kF8Buf = 8;

// Buffer descriptor words of [base, base + bytes), stride 0, as SGPRs (the
// layout __builtin_amdgcn_make_buffer_rsrc builds; reads past `bytes` give 0).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return (u32x4){(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu),
                   (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// LDS DMA of 16 bytes per lane: [descriptor + voff + soff] -> LDS at lds +
// 16 * lane.  It has no register result.  Written as asm because the
// compiler otherwise makes every later LDS read of the same array wait for
// the copy to land, ring slot or not; the ring's own vmcnt waits and
// barriers order it instead.  s_nop 4 covers a VALU-written descriptor
// SGPR (readfirstlane) read by VMEM, s_nop 0 the M0 write before the DMA.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

__device__ __forceinline__ int simd_of_wave() { return (int)((__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 4) & 3); }

__global__ __launch_bounds__(kAttnThreads, 2) void attn_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ VT, int64_t n_pad,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    bf16* __restrict__ O, int64_t ldo, int32_t n, int32_t heads, float sl2, int32_t nqt) {
    constexpr int KT = 64 * 128;                 // bytes of one K tile and of one V^T tile
    typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
    __shared__ __attribute__((aligned(1024))) char kl[kF8Buf * KT];
    __shared__ __attribute__((aligned(1024))) char vl[kF8Buf * KT];
    // The role counters live in the last V^T buffer: they are used only in
    // the prologue, and that buffer is first written in half step 2, after
    // the prologue's barrier.  The workgroup then takes exactly 128 KB.
    int* simd_count = reinterpret_cast<int*>(vl + (kF8Buf - 1) * KT);

    const int G = heads * nqt;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = G >> 3, extra = G & 7;
    const int L = xcd * base + (xcd < extra ? xcd : extra) + local;
    const int head = L / nqt;
    const int qt = L - head * nqt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int q0 = qt * kBQ + wave * 32;
    const int qi = q0 + col, qc = qi < n ? qi : n - 1;
    const int64_t ldq = (int64_t)heads * 128;
    const int NT = (n + 63) >> 6;

    // Q^T fragments (B operand of QK): 32 bytes of d chunk c at g * 32
    i32x8 qf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint8_t* src = Q8 + (int64_t)qc * ldq + head * 128 + c * 64 + g * 32;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(src), hi = *reinterpret_cast<const u32x4*>(src + 16);
        qf[c] = (i32x8){(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                        (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
    }
    const float sl2q = sl2 * sq[(int64_t)head * n + qc] * sk[head];

    // fragment offsets (the swizzle depends on the lane only)
    uint32_t ko[2][2], vo[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 2; ++e) ko[c][e] = (uint32_t)(col * 128 + (((4 * c + 2 * g + e) ^ ((col >> 1) & 7)) << 4));
#pragma unroll
    for (int e = 0; e < 2; ++e) vo[e] = (uint32_t)(col * 64 + (((2 * g + e) ^ ((col >> 2) & 3)) << 4));
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 2; ++e) asm volatile("" : "+v"(ko[c][e]));
#pragma unroll
    for (int e = 0; e < 2; ++e) asm volatile("" : "+v"(vo[e]));

    // copy offsets: K rows 8 wave + lane / 8 (8 slots each), V^T rows 16 wave + lane / 4 (4 slots)
    const int krow = 8 * wave + (lane >> 3), kslot = lane & 7;
    const uint32_t kdo = (uint32_t)(krow * ldq + head * 128 + ((kslot ^ ((krow >> 1) & 7)) << 4));
    const int vrow = 16 * wave + (lane >> 2), vslot = lane & 3;
    const uint32_t vdo = (uint32_t)(vrow * n_pad + ((vslot ^ ((vrow >> 2) & 3)) << 4));
    const u32x4 vr = rsrc_words(VT + (int64_t)head * 128 * n_pad, (uint32_t)(128 * n_pad));
    const uint32_t kl0 = (uint32_t)(uintptr_t)H3_LDS(kl + wave * 1024);
    const uint32_t vl0 = (uint32_t)(uintptr_t)H3_LDS(vl + wave * 1024);
    // Tiles past the last one are copied too, through descriptors of zero
    // bytes (every lane reads 0 and no memory is touched), so that each
    // wave always has exactly two copies per tile in flight and the fixed
    // vmcnt of the odd half steps always covers the tile read next.
    auto copy_tile = [&](int t) __attribute__((always_inline)) {
        const int rem = n - t * 64;
        const int nvalid = __builtin_amdgcn_readfirstlane(rem < 0 ? 0 : rem < 64 ? rem : 64);
        const u32x4 kr = rsrc_words(K8 + (int64_t)(t < NT ? t : 0) * 64 * ldq, (uint32_t)(nvalid * ldq));
        u32x4 vrt = vr;
        vrt[2] = t < NT ? vr[2] : 0u;
        const uint32_t slot = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(t % kF8Buf) * KT);
        lds_dma16(kr, kl0 + slot, kdo, 0u);
        lds_dma16(vrt, vl0 + slot, vdo, (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(t < NT ? t * 64 : 0)));
    };

    i32x8 kf[2][2];                 // K fragments of the next QK: [key half][d chunk]
    i32x8 vf[4];                    // V^T fragments of the next PV: [d block]
    auto rd8 = [&](const char* p0, const char* p1) __attribute__((always_inline)) -> i32x8 {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p0), hi = *reinterpret_cast<const u32x4*>(p1);
        return (i32x8){(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                       (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
    };
    auto read_k = [&](int t, int h, int c) __attribute__((always_inline)) {
        const char* bp = kl + (t % kF8Buf) * KT + h * 32 * 128;
        kf[h][c] = rd8(bp + ko[c][0], bp + ko[c][1]);
    };
    auto read_v = [&](int t, int db) __attribute__((always_inline)) {
        const char* bp = vl + (t % kF8Buf) * KT + db * 32 * 64;
        vf[db] = rd8(bp + vo[0], bp + vo[1]);
    };
    auto mfma8 = [&](const i32x8& a, const i32x8& bb, f32x16& acc) __attribute__((always_inline)) {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, acc, 0, 0, 0, 0, 0, 0);
    };

    f32x16 s[2];                    // logits of the tile in flight: [key half]
    auto mask = [&](int kbase) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kbase + 32 * h + 8 * (r >> 2) + 4 * g + (r & 3) >= n) s[h][r] = -__builtin_inff();
    };
    auto tile_max = [&]() __attribute__((always_inline)) -> float {
        float mx = __builtin_fmaxf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[0][r], s[1][r]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        return __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2q;
    };

    f32x16 oacc[5];
#pragma unroll
    for (int db = 0; db < 5; ++db) oacc[db] = (f32x16){};
    const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838};
    float m_ref;
    i32x8 pf;                       // the tile's weights as e4m3, 32 bytes per lane (key half 0 then 1)

    // pmax = the largest weight.  The first conversion of each word writes
    // its low half only and the second its high half, so the word may start
    // from any value.
    auto softmax_pack = [&](float& pmax) __attribute__((always_inline)) {
        const float mo = m_ref - 4.0f;
        pmax = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = fast_exp2(__builtin_fmaf(s[h][4 * w + e], sl2q, -mo));
                    pmax = __builtin_fmaxf(pmax, p[e]);
                }
                int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __builtin_nondeterministic_value(0), false);
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
                pf[4 * h + w] = wd;
            }
    };
    // V(t): K fragments for M(t), then tile t's weights
    auto vblock = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 2; ++c) read_k(t + 1, h, c);
        if (__builtin_expect((t + 1) * 64 > n, 0)) mask(t * 64);
        float pmax;
        softmax_pack(pmax);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(pmax <= 448.0f)) != 0, 0)) {   // rare
            const float m_new = __builtin_fmaxf(m_ref, tile_max());
            const float alpha = fast_exp2(m_ref - m_new);
#pragma unroll
            for (int db = 0; db < 5; ++db) oacc[db] *= alpha;
            m_ref = m_new;
            softmax_pack(pmax);
        }
    };
    // M(t): QK of tile t+1 while tile t's V^T fragments arrive, PV of tile t
    // (the scheduling barriers keep all four V^T reads ahead of the QK
    // MFMAs that cover their latency, and each block inside its half step)
    auto mblock = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) read_v(t, db);
        __builtin_amdgcn_sched_barrier(0);
        s[0] = (f32x16){};
        s[1] = (f32x16){};
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h) mfma8(kf[h][c], qf[c], s[h]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) mfma8(vf[db], pf, oacc[db]);
        mfma8(ones, pf, oacc[4]);
    };
    auto end_even = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto end_odd = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<2 * (kF8Buf - 4), true>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: roles, tiles 0 .. kF8Buf-3, QK of tile 0
    if (tid < 4) simd_count[tid] = 0;
    zero_lds(kl, kF8Buf * KT, tid);
    zero_lds(vl, kF8Buf * KT, tid);
    __syncthreads();
    int rank = 0;
    if (lane == 0) rank = atomicAdd(&simd_count[simd_of_wave()], 1);
    const bool trailing = (__builtin_amdgcn_readfirstlane(rank) & 1) != 0;
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int t = 0; t < kF8Buf - 2; ++t) copy_tile(t);
    wait_vm<0, false>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 2; ++c) read_k(0, h, c);
    s[0] = (f32x16){};
    s[1] = (f32x16){};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) mfma8(kf[h][c], qf[c], s[h]);
    if (n < 64) mask(0);
    m_ref = tile_max();

    // ---- 2 NT + 1 half steps, each ending in a barrier, for both roles
    if (!trailing) {
        for (int t = 0; t < NT; ++t) {
            copy_tile(t + kF8Buf - 2);          // half step 2t
            vblock(t);
            end_even();
            mblock(t);                          // half step 2t+1
            end_odd();
        }
        end_even();                             // half step 2 NT
    } else {
        copy_tile(kF8Buf - 2);                  // half step 0
        end_even();
        for (int t = 0; t < NT; ++t) {
            vblock(t);                          // half step 2t+1
            end_odd();
            copy_tile(t + kF8Buf - 1);          // half step 2t+2
            mblock(t);
            end_even();
        }
    }
    wait_vm<0, true>();

    if (qi < n) {
        const float inv = sv[head] / oacc[4][0];
        bf16* orow = O + (int64_t)qi * ldo + head * 128;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * g;
                const f32x16& a = oacc[db];
                *reinterpret_cast<u32x2*>(orow + d) =
                    (u32x2){pack_bf16x2(a[4 * r4] * inv, a[4 * r4 + 1] * inv),
                            pack_bf16x2(a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv)};
            }
    }
}

hipError_t launch_attention_fp8(const void* q8, const void* k8, const void* vt, int64_t n_pad, const float* sq,
                                const float* sk, const float* sv, void* o, int64_t ldo, int32_t n, int32_t heads,
                                float scale, hipStream_t st) {
    const int nqt = (n + kBQ - 1) / kBQ;
    const float sl2 = (float)((double)scale * 1.4426950408889634);
    attn_fp8_kernel<<<nqt * heads, kAttnThreads, 0, st>>>((const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)vt,
                                                          n_pad, sq, sk, sv, (bf16*)o, ldo, n, heads, sl2, nqt);
    return hipGetLastError();
}

hipError_t launch_attention(bool bf, const void* q, const void* k, const void* v, int64_t ld, void* o,
                            int64_t ldo, int32_t n, int32_t heads, int32_t hd, float scale, float* lse,
                            hipStream_t st) {
    const int nqt = (n + kBQ - 1) / kBQ;
    const int grid = nqt * heads;
    const float sl2 = (float)((double)scale * 1.4426950408889634);
#define H3_ATTN(TY, D)                                                                                    \
    attn_fwd_kernel<TY, D><<<grid, kAttnThreads, 0, st>>>((const TY*)q, (const TY*)k, (const TY*)v, ld,  \
                                                          (TY*)o, ldo, n, heads, sl2, lse, nqt)
    if (bf) {
#if H3_ATTN_MFMA16
        if (hd == 128)
            attn_bf16_m16_kernel<128><<<grid, kAttnThreads, 0, st>>>((const bf16*)q, (const bf16*)k, (const bf16*)v,
                                                                      ld, (bf16*)o, ldo, n, heads, sl2, lse, nqt);
        else
            attn_bf16_m16_kernel<64><<<grid, kAttnThreads, 0, st>>>((const bf16*)q, (const bf16*)k, (const bf16*)v,
                                                                     ld, (bf16*)o, ldo, n, heads, sl2, lse, nqt);
#else
        if (hd == 128)
            attn_bf16_kernel<128><<<grid, kAttnThreads, 0, st>>>((const bf16*)q, (const bf16*)k, (const bf16*)v, ld,
                                                                  (bf16*)o, ldo, n, heads, sl2, lse, nqt);
        else
            attn_bf16_kernel<64><<<grid, kAttnThreads, 0, st>>>((const bf16*)q, (const bf16*)k, (const bf16*)v, ld,
                                                                 (bf16*)o, ldo, n, heads, sl2, lse, nqt);
#endif
    } else {
        if (hd == 128) H3_ATTN(float, 128);
        else H3_ATTN(float, 64);
    }
#undef H3_ATTN
    return hipGetLastError();
}

}  // namespace h3
