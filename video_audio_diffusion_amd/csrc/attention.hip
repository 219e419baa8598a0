// Full bidirectional softmax attention, flash style, on MFMA.
//
// Work split: one workgroup = 8 wavefronts = 256 query rows of one head;
// each wavefront owns 32 queries (one 32-query MFMA block) for the whole key
// sweep, so its output accumulators, running max and running sum never leave
// registers.  A wavefront needs ~170 VGPRs, so two of them share each SIMD
// and one's softmax (VALU) runs under the other's MFMAs.  Keys stream
// through LDS in tiles of 64, double-buffered: the next tile is fetched into
// registers (buffer loads against a per-tile resource, which also zero-fills
// rows past the last key) while the current tile is multiplied; wavefronts
// 0-3 stage (and transpose) V, wavefronts 4-7 stage K.
//
// Orientation: the kernel computes S^T = K . Q^T (keys as MFMA rows, queries
// as MFMA columns).  A 32x32 accumulator then gives each lane one query and
// 16 keys, so a query's block max is 15 local max operations plus one swap
// with lane^32, and the probabilities P^T are already in the B-operand
// layout of the second product O^T += V^T . P^T -- no LDS round trip for P.
// Accumulator register r of lane l holds key 8(r/4) + 4(l/32) + r%4 of its
// 32-key block.  The PV product contracts over keys in that same order, so
// V^T is read from LDS as runs of 4 consecutive keys at key offsets
// 8(r/4) + 4(l/32): V is stored transposed ([d][key]) in LDS.
//
// LDS rows are padded (K rows by 16 bytes, V^T rows by one 4-key run) so
// that the 32 rows one fragment read touches fall on distinct banks while
// every address stays base + constant.
//
// Softmax: logits are scaled by scale*log2(e) once; exponentials are exp2
// (v_exp_f32).  Each query keeps a reference max m and a running sum l per
// lane; the two lane halves of a query are summed once at the end.
#include "launch.h"

namespace h3 {

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
constexpr int kQB = 1;                       // 32-query blocks per wavefront
constexpr int kBQ = kAttnWaves * kQB * 32;   // 256 queries per workgroup
constexpr int kBKV = 64;                     // keys per LDS tile
constexpr int kKB = kBKV / 32;               // 32-key score blocks per tile
// The reference max of a query only moves when a block's max exceeds it by
// more than this (log2 units), so probabilities stay <= 2^8 and the output
// rescale is skipped for most blocks; the result is unchanged because the
// final division uses the same reference.
constexpr float kLazyMax = 8.0f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <typename T, int HD>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ Kp,
                                                       const T* __restrict__ Vp, int64_t ld,
                                                       T* __restrict__ O, int64_t ldo, int32_t n,
                                                       int32_t heads, float sl2, float* __restrict__ lse,
                                                       int32_t nqt) {
    constexpr int ES = sizeof(T);
    constexpr int KRB = HD * ES;             // bytes of one K row
    constexpr int KRBP = KRB + 16;           // padded K row in LDS
    constexpr int KCH = KRB / 16;            // 16-byte chunks per K row
    constexpr int NCH = KRB / 32;            // 32-byte MFMA k-chunks over head_dim
    constexpr int RUNB = 4 * ES;             // bytes of a 4-key run of V^T
    constexpr int VRBP = kBKV * ES + RUNB;   // padded V^T row (64 keys + one run)
    constexpr int DV = KRB / 16;             // 16-byte vectors per V row
    constexpr int EPV = 16 / ES;             // d values per 16-byte vector
    constexpr int KSLOTS = kBKV * KCH / 256; // K chunks each staging thread moves
    constexpr int VPAIRS = 16 * DV;          // (4-key run, d vector) pairs per tile
    constexpr int VSLOTS = (VPAIRS + 255) / 256;
    constexpr int DB = HD / 32;              // 32-wide d blocks of the output
    static_assert(KSLOTS >= 1 && (kBKV * KCH) % 256 == 0 && 256 % KCH == 0, "K tile split");
    static_assert(VPAIRS <= 256 || VPAIRS % 256 == 0, "V tile split");

    __shared__ __attribute__((aligned(16))) char ks[2][kBKV * KRBP];
    __shared__ __attribute__((aligned(16))) char vts[2][HD * VRBP];

    // ---- workgroup -> (head, query tile); consecutive tiles on one XCD share a head
    const int G = heads * nqt;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = G >> 3, extra = G & 7;
    const int L = xcd * base + (xcd < extra ? xcd : extra) + local;
    const int head = L / nqt;
    const int qt = L - head * nqt;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, g = lane >> 5;
    const int q0 = qt * kBQ + wave * (kQB * 32);
    const int64_t hoff = (int64_t)head * HD;
    const uint32_t ldb = (uint32_t)(ld * ES);   // bytes between key rows

    // ---- Q^T fragments (B operand): lane holds one query, 16 bytes of d per chunk
    u32x4 qf[kQB][NCH];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = q0 + qb * 32 + col;
        const char* src = reinterpret_cast<const char*>(Q + (int64_t)(qi < n ? qi : n - 1) * ld + hoff);
#pragma unroll
        for (int c = 0; c < NCH; ++c) qf[qb][c] = *reinterpret_cast<const u32x4*>(src + c * 32 + g * 16);
    }
    // Retire the Q loads here: otherwise the wait-count analysis still sees
    // them in flight inside the key loop and makes every QK product wait for
    // the next tile's prefetch as well.
    __builtin_amdgcn_s_waitcnt(0);

    // ---- K / V staging.  Threads 0..255 move V: 4-key run (idx % 16) of d
    //      vector idx / 16, idx = tid + 256 i.  Threads 256..511 move K:
    //      chunk (st % KCH) of key st / KCH + (256 / KCH) i, st = tid - 256.
    const bool stage_v = tid < 256;
    const int st = stage_v ? tid : tid - 256;
    const uint32_t k_voff = (uint32_t)(st / KCH) * ldb + (uint32_t)(st % KCH) * 16;
    constexpr int NREG = KSLOTS > 4 * VSLOTS ? KSLOTS : 4 * VSLOTS;
    u32x4 sreg[NREG];
    auto fetch = [&](int kv0) {
        const int nvalid = n - kv0 < kBKV ? n - kv0 : kBKV;
        if (stage_v) {
            const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vp + (int64_t)kv0 * ld + hoff, (uint32_t)nvalid * ldb);
#pragma unroll
            for (int i = 0; i < VSLOTS; ++i) {
                const int idx = st + 256 * i;
                const uint32_t voff = (uint32_t)(4 * (idx % 16)) * ldb + (uint32_t)(idx / 16 % DV) * 16;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sreg[4 * i + e] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff, e * ldb, 0);
            }
        } else {
            const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kp + (int64_t)kv0 * ld + hoff, (uint32_t)nvalid * ldb);
#pragma unroll
            for (int i = 0; i < KSLOTS; ++i)
                sreg[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, k_voff, i * (256 / KCH) * ldb, 0);
#pragma unroll
            for (int i = KSLOTS; i < NREG; ++i) sreg[i] = (u32x4){0, 0, 0, 0};   // both paths define every slot
        }
    };
    auto stash = [&](int buf) {
        if (!stage_v) {
#pragma unroll
            for (int i = 0; i < KSLOTS; ++i) {
                const int key = st / KCH + (256 / KCH) * i, ch = st % KCH;
                *reinterpret_cast<u32x4*>(&ks[buf][key * KRBP + ch * 16]) = sreg[i];
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < VSLOTS; ++i) {
            const int idx = st + 256 * i;
            if (VPAIRS % 256 == 0 || idx < VPAIRS) {
                const int run = idx % 16, dv = idx / 16;
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    char* dst = &vts[buf][(dv * EPV + e) * VRBP + run * RUNB];
                    if constexpr (ES == 2) {
                        // d = 2w (+1): low (high) bf16 of dword w of each key's vector
                        const int w = e >> 1;
                        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                        *reinterpret_cast<u32x2*>(dst) =
                            (u32x2){__builtin_amdgcn_perm(sreg[4 * i + 1][w], sreg[4 * i][w], sel),
                                    __builtin_amdgcn_perm(sreg[4 * i + 3][w], sreg[4 * i + 2][w], sel)};
                    } else {
                        *reinterpret_cast<u32x4*>(dst) =
                            (u32x4){sreg[4 * i][e], sreg[4 * i + 1][e], sreg[4 * i + 2][e], sreg[4 * i + 3][e]};
                    }
                }
            }
        }
    };

    f32x16 oacc[kQB][DB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] = (f32x16){};
    float m_run[kQB], l_run[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        m_run[qb] = -__builtin_inff();
        l_run[qb] = 0.f;
    }

    const int ntiles = (n + kBKV - 1) / kBKV;
    fetch(0);
    stash(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int kv0 = t * kBKV;
        if (t + 1 < ntiles) fetch(kv0 + kBKV);
        const char* K_l = ks[buf] + col * KRBP + g * 16;
        const char* V_l = vts[buf] + col * VRBP + g * RUNB;

#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            if (kv0 + kb * 32 >= n) break;          // block entirely past the last key
            // ---- S^T = K Q^T for 32 keys x (kQB x 32) queries
            f32x16 s[kQB];
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[qb] = (f32x16){};
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(K_l + kb * 32 * KRBP + c * 32);
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) AttnMfma<T>::qk(s[qb], kf, qf[qb][c]);
            }
            if (kv0 + kb * 32 + 32 > n) {           // ragged block: keys past n get -inf
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= n)
#pragma unroll
                        for (int qb = 0; qb < kQB; ++qb) s[qb][r] = -__builtin_inff();
                }
            }

            // ---- online softmax with a lazily moved reference max
            float mx[kQB];
            bool grow = false;
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                float v = s[qb][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) v = fmaxf(v, s[qb][r]);
                v = fmaxf(v, __shfl_xor(v, 32, kWave)) * sl2;
                mx[qb] = v;
                grow |= v > m_run[qb] + kLazyMax;
            }
            if (__builtin_amdgcn_ballot_w64(grow)) {   // some query's max moved by > 2^kLazyMax
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    const float m_new = fmaxf(m_run[qb], mx[qb]);
                    const float alpha = fast_exp2(m_run[qb] - m_new);
                    m_run[qb] = m_new;
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
                }
            }
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                float rs = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(__builtin_fmaf(s[qb][r], sl2, -m_run[qb]));
                    s[qb][r] = p;
                    rs += p;
                }
                l_run[qb] += rs;
            }

            // ---- O^T += V^T P^T over these 32 keys
            if constexpr (ES == 2) {
                // one MFMA per 16 keys: P regs 8h..8h+7; V^T runs at keys 16h + 4g and 16h + 8 + 4g
                u32x4 pf[kQB][2];
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            pf[qb][h][w] = pack_bf16x2(s[qb][8 * h + 2 * w], s[qb][8 * h + 2 * w + 1]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const char* vp = V_l + db * 32 * VRBP + (kb * 32 + 16 * h) * ES;
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8 * ES);
                        const u32x4 vf = (u32x4){lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                        for (int qb = 0; qb < kQB; ++qb)
                            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pf[qb][h]),
                                oacc[qb][db], 0, 0, 0);
                    }
                }
            } else {
                // fp32: four 32x32x2 MFMAs per 8 keys; lane group g holds keys 8c + 4g .. +3
#pragma unroll
                for (int db = 0; db < DB; ++db) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const f32x4 vf = *reinterpret_cast<const f32x4*>(V_l + db * 32 * VRBP +
                                                                         (kb * 32 + 8 * c) * ES);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int qb = 0; qb < kQB; ++qb)
                                oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[j], s[qb][4 * c + j],
                                                                                   oacc[qb][db], 0, 0, 0);
                    }
                }
            }
        }

        if (t + 1 < ntiles) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- normalise and store: O^T lane (query, g) holds d = 32db + 8(r/4) + 4g + r%4
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, kWave);
        const float inv = 1.0f / l_tot;
        const int qi = q0 + qb * 32 + col;
        if (qi < n) {
            T* orow = O + (int64_t)qi * ldo + hoff;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = db * 32 + 8 * r4 + 4 * g;
                    const f32x16& a = oacc[qb][db];
                    if constexpr (ES == 2) {
                        *reinterpret_cast<u32x2*>(orow + d) =
                            (u32x2){pack_bf16x2(a[4 * r4] * inv, a[4 * r4 + 1] * inv),
                                    pack_bf16x2(a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv)};
                    } else {
                        *reinterpret_cast<f32x4*>(orow + d) =
                            (f32x4){a[4 * r4] * inv, a[4 * r4 + 1] * inv, a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv};
                    }
                }
            if (lse && g == 0)
                lse[(int64_t)head * n + qi] = m_run[qb] * 0.69314718055994531f + __logf(l_tot);
        }
    }
}

hipError_t launch_attention(bool bf, const void* q, const void* k, const void* v, int64_t ld, void* o,
                            int64_t ldo, int32_t n, int32_t heads, int32_t hd, float scale, float* lse,
                            hipStream_t st) {
    const int nqt = (n + kBQ - 1) / kBQ;
    const int grid = nqt * heads;
    const float sl2 = (float)((double)scale * 1.4426950408889634);
#define H3_ATTN(TY, D)                                                                                  \
    attn_fwd_kernel<TY, D><<<grid, kAttnThreads, 0, st>>>((const TY*)q, (const TY*)k, (const TY*)v, ld, (TY*)o, \
                                                 ldo, n, heads, sl2, lse, nqt)
    if (bf) {
        if (hd == 128) H3_ATTN(bf16, 128);
        else H3_ATTN(bf16, 64);
    } else {
        if (hd == 128) H3_ATTN(float, 128);
        else H3_ATTN(float, 64);
    }
#undef H3_ATTN
    return hipGetLastError();
}

}  // namespace h3
