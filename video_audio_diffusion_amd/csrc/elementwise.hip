// Bandwidth-bound passes of the H3 block: modulated RMSNorm, modality-gated
// residual, SwiGLU, and per-head QK RMSNorm fused with 3-D MM-RoPE.
//
// All of them stream 16-byte vectors with consecutive lanes on consecutive
// addresses and keep every value in fp32 between the load and the one
// rounding at the store.  Row kernels give one wavefront to one token row so
// the interval lookup and the row reduction are per-wave scalars.
#include "launch.h"

namespace h3 {

// --------------------------------------------------------------------------
// Modulated RMSNorm (one wavefront per row, the row held in registers).
//   y = x * rsqrt(mean(x^2) + eps) * (1 + scale[set]) + shift[set]
template <typename T, int VPL>
__global__ __launch_bounds__(256) void adaln_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                    int32_t n, int32_t dim,
                                                    const float* __restrict__ mod, int32_t br,
                                                    SegTable tab, float eps) {
    constexpr int N = Vec<T>::N;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const int nv = dim / N;
    const char* xr = reinterpret_cast<const char*>(x + (int64_t)row * dim);
    char* yr = reinterpret_cast<char*>(y + (int64_t)row * dim);
    float v[VPL][N];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int j = lane + kWave * i;
        if (j < nv) {
            Vec<T>::load(xr + 16 * j, v[i]);
#pragma unroll
            for (int e = 0; e < N; ++e) ss += v[i][e] * v[i][e];
        }
    }
    ss = sum_lanes<kWave>(ss);
    const float rstd = 1.0f / __builtin_sqrtf(ss / (float)dim + eps);
    const int s = find_seg(tab, row);
    const float* shift = mod + ((int64_t)tab.s[s].mod_set * 6 + 3 * br) * dim;
    const float* scale = shift + dim;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int j = lane + kWave * i;
        if (j < nv) {
            float o[N];
#pragma unroll
            for (int e = 0; e < N; e += 4) {
                const f32x4 sh = *reinterpret_cast<const f32x4*>(shift + j * N + e);
                const f32x4 sc = *reinterpret_cast<const f32x4*>(scale + j * N + e);
#pragma unroll
                for (int u = 0; u < 4; ++u) o[e + u] = v[i][e + u] * rstd * (1.0f + sc[u]) + sh[u];
            }
            Vec<T>::store(yr + 16 * j, o);
        }
    }
}

// --------------------------------------------------------------------------
// Modulated RMSNorm for wide rows.  A grid of at most kAdalnBlocks
// workgroups of 256 threads sweeps the rows in step: workgroup w takes rows
// w, w + G, w + 2G, ... (G = the grid size), so at any moment the grid
// streams one contiguous window of about G rows, the access order that gets
// the most out of HBM here (a grid-stride copy beats one in which each
// workgroup streams its own contiguous run by about 8 %).  Thread t owns the
// 16-byte column vectors t, t + 256, ... of every row, so its shift and
// scale stay in registers while the rows' modality set stays the same (a
// workgroup's rows only move forward, so it reloads them, uniformly, once per
// interval boundary it crosses): the row-per-wavefront form read the 43 KB
// of fp32 shift and scale of a 5376-wide row once per row, four times the
// row's own bytes.  Two rows are held in registers as stored: the next
// row's loads are issued before the current one is reduced per wavefront,
// its four wavefront sums exchanged through LDS (double-buffered, one
// barrier per row that waits for LDS only, so loads and stores stay in
// flight), normalised, modulated and stored.
// Measured at 92840 x 5376 bf16 on a cold input: 0.370-0.373 ms at 1024
// workgroups (5.35-5.40 TB/s), 0.376-0.44 ms at other grid sizes from 768
// to 3072, 0.41 ms for 768 contiguous runs of rows; a grid-stride device
// copy of the same bytes takes 0.38-0.39 ms.  Inside the block, where part
// of x is still in the caches from the kernel before, it takes 0.354-0.356
// ms.  Loads and stores marked non-temporal were 3 % faster on a cold input
// but 2 % slower inside the block, so they are not used.
constexpr int kAdalnBlocks = 1024;
template <typename T, int VPT>
__global__ __launch_bounds__(256) void adaln_rows_kernel(const T* __restrict__ x, T* __restrict__ y, int32_t n,
                                                         int32_t dim, const float* __restrict__ mod, int32_t br,
                                                         SegTable tab, float eps) {
    constexpr int N = Vec<T>::N;
    __shared__ float part[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nv = dim / N;
    int cur_set = -1;
    float sh[VPT][N], sc[VPT][N];
    // row `row` as stored (zeros past the last row or the row's end)
    auto load_row = [&](u32x4 (&raw)[VPT], int row) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int j = tid + 256 * k;
            raw[k] = (row < n && j < nv)
                         ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(x + (int64_t)row * dim) + 16 * j)
                         : (u32x4){};
        }
    };
    auto process = [&](u32x4 (&raw)[VPT], int row, int buf) __attribute__((always_inline)) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            float f[N];
            Vec<T>::load(&raw[k], f);
#pragma unroll
            for (int e = 0; e < N; ++e) ss += f[e] * f[e];
        }
        ss = sum_lanes<kWave>(ss);
        // keep the vectors packed until the second use (otherwise the
        // compiler keeps both unpacked halves live across the barrier)
#pragma unroll
        for (int k = 0; k < VPT; ++k) asm volatile("" : "+v"(raw[k]));
        if (lane == 0) part[buf][wave] = ss;
        // LDS-only barrier: the partial sums are visible, while this
        // thread's loads of the next row and stores of earlier ones stay
        // in flight
        wait_cnt<63, 0>();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const float tot = part[buf][0] + part[buf][1] + part[buf][2] + part[buf][3];
        const float rstd = 1.0f / __builtin_sqrtf(tot / (float)dim + eps);
        const int set = tab.s[find_seg(tab, row)].mod_set;
        if (set != cur_set) {           // uniform: the row and the table are the workgroup's
            cur_set = set;
            const float* shift = mod + ((int64_t)set * 6 + 3 * br) * dim;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int j = tid + 256 * k;
                if (j < nv) {
#pragma unroll
                    for (int e = 0; e < N; e += 4) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(shift + j * N + e);
                        const f32x4 c = *reinterpret_cast<const f32x4*>(shift + dim + j * N + e);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            sh[k][e + u] = a[u];
                            sc[k][e + u] = 1.0f + c[u];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int j = tid + 256 * k;
            if (j < nv) {
                float f[N], o[N];
                Vec<T>::load(&raw[k], f);
#pragma unroll
                for (int e = 0; e < N; ++e) o[e] = f[e] * rstd * sc[k][e] + sh[k][e];
                Vec<T>::store(reinterpret_cast<char*>(y + (int64_t)row * dim) + 16 * j, o);
            }
        }
    };
    // two rows in registers: the next row's loads go out before this row is
    // reduced, normalised and stored
    u32x4 ra[VPT], rb[VPT];
    const int G = gridDim.x;
    load_row(ra, blockIdx.x);
    for (int row = blockIdx.x; row < n; row += 2 * G) {
        load_row(rb, row + G);
        process(ra, row, 0);
        if (row + G >= n) break;
        load_row(ra, row + 2 * G);
        process(rb, row + G, 1);
    }
}

// --------------------------------------------------------------------------
// Modality-gated residual: out = x + gate[set] * y (one wavefront per row).
template <typename T>
__global__ __launch_bounds__(256) void gate_residual_kernel(const T* x, const T* __restrict__ y, T* out,
                                                            int32_t n, int32_t dim,
                                                            const float* __restrict__ mod, int32_t br,
                                                            SegTable tab) {
    constexpr int N = Vec<T>::N;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const int nv = dim / N;
    const int s = find_seg(tab, row);
    const float* gate = mod + ((int64_t)tab.s[s].mod_set * 6 + 3 * br + 2) * dim;
    const char* xr = reinterpret_cast<const char*>(x + (int64_t)row * dim);
    const char* yr = reinterpret_cast<const char*>(y + (int64_t)row * dim);
    char* orow = reinterpret_cast<char*>(out + (int64_t)row * dim);
    for (int j = lane; j < nv; j += kWave) {
        float a[N], b[N], o[N];
        Vec<T>::load(xr + 16 * j, a);
        Vec<T>::load(yr + 16 * j, b);
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const f32x4 g = *reinterpret_cast<const f32x4*>(gate + j * N + e);
#pragma unroll
            for (int u = 0; u < 4; ++u) o[e + u] = a[e + u] + g[u] * b[e + u];
        }
        Vec<T>::store(orow + 16 * j, o);
    }
}

// --------------------------------------------------------------------------
// Euler flow update x += c[interval] * v, one coefficient per interval (zero
// for the intervals the sampler leaves alone).  Same row mapping as the gate
// residual: a wavefront per row, 16-byte vectors.
template <typename T>
__global__ __launch_bounds__(256) void euler_kernel(T* x, const T* __restrict__ v, int32_t n, int32_t dim,
                                                    SegTable tab, SegCoef coef) {
    constexpr int N = Vec<T>::N;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const float c = coef.c[find_seg(tab, row)];
    if (c == 0.f) return;                       // the row stays exactly as it is
    const int nv = dim / N;
    char* xr = reinterpret_cast<char*>(x + (int64_t)row * dim);
    const char* vr = reinterpret_cast<const char*>(v + (int64_t)row * dim);
    for (int j = lane; j < nv; j += kWave) {
        float a[N], b[N];
        Vec<T>::load(xr + 16 * j, a);
        Vec<T>::load(vr + 16 * j, b);
#pragma unroll
        for (int e = 0; e < N; ++e) a[e] = __builtin_fmaf(c, b[e], a[e]);
        Vec<T>::store(xr + 16 * j, a);
    }
}

// --------------------------------------------------------------------------
// SwiGLU: h = g / (1 + exp(-g)) * u over [gate | up] rows.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const T* __restrict__ gu, T* __restrict__ h,
                                                     int64_t n, int32_t F) {
    constexpr int N = Vec<T>::N;
    const int64_t fv = F / N;
    const int64_t total = n * fv;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = idx / fv;
        const int64_t c = idx - row * fv;
        const T* g = gu + row * 2 * F + c * N;
        float a[N], b[N], o[N];
        Vec<T>::load(g, a);
        Vec<T>::load(g + F, b);
#pragma unroll
        for (int e = 0; e < N; ++e) o[e] = a[e] / (1.0f + __expf(-a[e])) * b[e];
        Vec<T>::store(h + row * F + c * N, o);
    }
}

// Gate/up weight rows into the 32-row interleave of the fused SwiGLU GEMM:
// destination row r of [2F][K] is gate row 32u + j (r = 64u + j, j < 32) or
// up row 32u + j - 32 (F + ...).  16-byte pieces, grid-stride; rows are
// K * es bytes with K * es a multiple of 16.
__global__ __launch_bounds__(256) void interleave_gate_up_kernel(const uint8_t* __restrict__ src, int64_t ld_src,
                                                               uint8_t* __restrict__ dst, int64_t ld_dst,
                                                               int32_t F, int64_t row_pieces) {
    const int64_t total = 2 * (int64_t)F * row_pieces;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / row_pieces;
        const int64_t c = idx - r * row_pieces;
        const int64_t j = r & 63;
        const int64_t s = (r >> 6) * 32 + (j & 31) + (j < 32 ? 0 : F);
        *reinterpret_cast<u32x4*>(dst + r * ld_dst + c * 16) =
            *reinterpret_cast<const u32x4*>(src + s * ld_src + c * 16);
    }
}

// --------------------------------------------------------------------------
// Per-head RMSNorm of Q and K, then 3-D MM-RoPE, in place.  One workgroup
// per token: the token's (cos, sin) per pair are computed once into LDS and
// reused by all 2*heads head vectors; LPH lanes share one head vector.  A
// thread's head vectors are handled QR at a time with every load issued
// before any is used (the pass is bound by how many bytes are in flight),
// and the first batch's loads go out before the (cos, sin) computation.
template <typename T, int HD>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(T* q, T* k, int64_t ld, int32_t n,
                                                          int32_t heads,
                                                          const float* __restrict__ gq,
                                                          const float* __restrict__ gk, float eps,
                                                          RopeTable rt, SegTable tab) {
    constexpr int N = Vec<T>::N;
    constexpr int LPH = HD / N;           // lanes per head vector
    constexpr int GROUPS = 256 / LPH;     // head vectors per round
    constexpr int QR = 4;                 // rounds whose loads are in flight together
    __shared__ f32x2 cs[HD / 2];
    const int row = blockIdx.x;
    if (row >= n) return;                 // uniform for the workgroup
    const int sub = threadIdx.x % LPH;
    const int grp = threadIdx.x / LPH;
    const int nhv = 2 * heads;
    auto vec_ptr = [&](int hv) __attribute__((always_inline)) -> T* {
        const bool isq = hv < heads;
        return (isq ? q : k) + (int64_t)row * ld + (int64_t)(isq ? hv : hv - heads) * HD + sub * N;
    };
    float v[QR][N];
    auto load_batch = [&](int hv0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < QR; ++u) {
            const int hv = hv0 + u * GROUPS;
            if (hv < nhv) Vec<T>::load(vec_ptr(hv), v[u]);
        }
    };
    load_batch(grp);
    // this thread's N gains for q and for k, loaded once (1 when absent)
    float gqv[N], gkv[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
        gqv[e] = gq ? gq[sub * N + e] : 1.0f;
        gkv[e] = gk ? gk[sub * N + e] : 1.0f;
    }
    if (threadIdx.x < HD / 2) {
        const int p = threadIdx.x;
        const int s = find_seg(tab, row);
        const SegDev& sg = tab.s[s];
        const int l = row - sg.start;
        const int axis = rt.axis[p];
        const int pos = axis == 0 ? sg.t0 + l / sg.HW : axis == 1 ? sg.h0 + (l / sg.W) % sg.H
                                                                  : sg.w0 + l % sg.W;
        double sn, c;
        sincos((double)pos * rt.inv_freq[p], &sn, &c);
        cs[p] = (f32x2){(float)c, (float)sn};
    }
    __syncthreads();
    for (int hv0 = grp; hv0 < nhv; hv0 += QR * GROUPS) {
        if (hv0 != grp) load_batch(hv0);
#pragma unroll
        for (int u = 0; u < QR; ++u) {
            const int hv = hv0 + u * GROUPS;
            // hv < nhv is uniform across a head vector's LPH lanes (the
            // lane-sum below stays among them)
            if (hv >= nhv) break;
            const bool isq = hv < heads;
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < N; ++e) ss += v[u][e] * v[u][e];
            ss = sum_lanes<LPH>(ss);
            const float rstd = 1.0f / __builtin_sqrtf(ss / (float)HD + eps);
#pragma unroll
            for (int e = 0; e < N; ++e) v[u][e] *= rstd * (isq ? gqv[e] : gkv[e]);
#pragma unroll
            for (int e = 0; e < N; e += 2) {
                const f32x2 t = cs[(sub * N + e) / 2];
                const float u0 = v[u][e], u1 = v[u][e + 1];
                v[u][e] = u0 * t.x - u1 * t.y;
                v[u][e + 1] = u0 * t.y + u1 * t.x;
            }
            Vec<T>::store(vec_ptr(hv), v[u]);
        }
    }
}

// --------------------------------------------------------------------------
// Patchify / unpatchify of a channels-last latent [T][H][W][C] with a
// (pt, ph, pw) patch.  Token i = (t * Hp + h) * Wp + w (w fastest) holds its
// patch's values in (dt, dh, dw, c) order, then zeros up to the row stride
// ld, so a token row can feed a GEMM whose K is ld.  One thread per 16-byte
// vector: C is a multiple of the vector width, so a vector never leaves one
// latent position.  Pure data movement: bits are copied, never rounded.
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(const T* __restrict__ lat, T* __restrict__ tok, int64_t ld,
                                                       PatchGeom g, int64_t n_tok) {
    constexpr int V = Vec<T>::N;
    const int Hp = g.H / g.ph, Wp = g.W / g.pw;
    const int P = g.pt * g.ph * g.pw * g.C;
    const int64_t vpr = ld / V;
    const int64_t total = n_tok * vpr;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / vpr;
        const int f = (int)(idx - i * vpr) * V;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (f < P) {
            const int c = f % g.C;
            int q = f / g.C;
            const int dw = q % g.pw;
            q /= g.pw;
            const int dh = q % g.ph, dt = q / g.ph;
            const int w = (int)(i % Wp);
            const int64_t r = i / Wp;
            const int h = (int)(r % Hp), t = (int)(r / Hp);
            const int64_t src =
                (((int64_t)(t * g.pt + dt) * g.H + h * g.ph + dh) * g.W + w * g.pw + dw) * g.C + c;
            val = *reinterpret_cast<const u32x4*>(lat + src);
        }
        *reinterpret_cast<u32x4*>(tok + i * ld + f) = val;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void unpatchify_kernel(const T* __restrict__ tok, int64_t ld,
                                                         T* __restrict__ lat, PatchGeom g, int64_t n_vec) {
    constexpr int V = Vec<T>::N;
    const int Hp = g.H / g.ph, Wp = g.W / g.pw;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n_vec;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = idx * V;
        const int c = (int)(e % g.C);
        int64_t pos = e / g.C;
        const int wl = (int)(pos % g.W);
        pos /= g.W;
        const int hl = (int)(pos % g.H), tl = (int)(pos / g.H);
        const int64_t i = ((int64_t)(tl / g.pt) * Hp + hl / g.ph) * Wp + wl / g.pw;
        const int f = (((tl % g.pt) * g.ph + hl % g.ph) * g.pw + wl % g.pw) * g.C + c;
        *reinterpret_cast<u32x4*>(lat + e) = *reinterpret_cast<const u32x4*>(tok + i * ld + f);
    }
}

static int stream_blocks(int64_t work) {
    const int64_t b = (work + 255) / 256;
    return (int)(b < 8192 ? (b < 1 ? 1 : b) : 8192);
}

hipError_t launch_patchify(bool bf, const void* lat, void* tok, int64_t ld, const PatchGeom& g, int64_t n_tok,
                           hipStream_t st) {
    const int64_t work = n_tok * (ld / (bf ? 8 : 4));
    if (bf)
        patchify_kernel<bf16><<<stream_blocks(work), 256, 0, st>>>((const bf16*)lat, (bf16*)tok, ld, g, n_tok);
    else
        patchify_kernel<float><<<stream_blocks(work), 256, 0, st>>>((const float*)lat, (float*)tok, ld, g, n_tok);
    return hipGetLastError();
}

hipError_t launch_unpatchify(bool bf, const void* tok, int64_t ld, void* lat, const PatchGeom& g, hipStream_t st) {
    const int64_t n_vec = (int64_t)g.T * g.H * g.W * g.C / (bf ? 8 : 4);
    if (bf)
        unpatchify_kernel<bf16><<<stream_blocks(n_vec), 256, 0, st>>>((const bf16*)tok, ld, (bf16*)lat, g, n_vec);
    else
        unpatchify_kernel<float><<<stream_blocks(n_vec), 256, 0, st>>>((const float*)tok, ld, (float*)lat, g, n_vec);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// launchers

template <typename T, int VPL>
static hipError_t adaln_t(const void* x, void* y, int32_t n, int32_t dim, const float* mod, int32_t br,
                          const SegTable& tab, float eps, hipStream_t st) {
    adaln_kernel<T, VPL><<<(n + 3) / 4, 256, 0, st>>>((const T*)x, (T*)y, n, dim, mod, br, tab, eps);
    return hipGetLastError();
}

template <typename T, int VPT>
static hipError_t adaln_rows_t(const void* x, void* y, int32_t n, int32_t dim, const float* mod, int32_t br,
                               const SegTable& tab, float eps, hipStream_t st) {
    const int blocks = n < kAdalnBlocks ? n : kAdalnBlocks;
    adaln_rows_kernel<T, VPT><<<blocks, 256, 0, st>>>((const T*)x, (T*)y, n, dim, mod, br, tab, eps);
    return hipGetLastError();
}

// Rows of at most 4 * 64 vectors (2048 bf16 / 1024 fp32 values) keep the
// row-per-wavefront form; wider rows take the grid-sweep form.
template <typename T>
static hipError_t adaln_dispatch(const void* x, void* y, int32_t n, int32_t dim, const float* mod,
                                 int32_t br, const SegTable& tab, float eps, hipStream_t st) {
    const int nv = dim / Vec<T>::N;
    const int per_lane = (nv + kWave - 1) / kWave;
    if (per_lane <= 1) return adaln_t<T, 1>(x, y, n, dim, mod, br, tab, eps, st);
    if (per_lane <= 2) return adaln_t<T, 2>(x, y, n, dim, mod, br, tab, eps, st);
    if (per_lane <= 4) return adaln_t<T, 4>(x, y, n, dim, mod, br, tab, eps, st);
    const int per_thread = (nv + 255) / 256;
    if (per_thread <= 3) return adaln_rows_t<T, 3>(x, y, n, dim, mod, br, tab, eps, st);
    if (per_thread <= 4) return adaln_rows_t<T, 4>(x, y, n, dim, mod, br, tab, eps, st);
    if (per_thread <= 6) return adaln_rows_t<T, 6>(x, y, n, dim, mod, br, tab, eps, st);
    return adaln_t<T, kRowMaxVecPerLane>(x, y, n, dim, mod, br, tab, eps, st);
}

hipError_t launch_adaln(bool bf, const void* x, void* y, int32_t n, int32_t dim, const float* mod,
                        int32_t br, const SegTable& tab, float eps, hipStream_t st) {
    return bf ? adaln_dispatch<bf16>(x, y, n, dim, mod, br, tab, eps, st)
              : adaln_dispatch<float>(x, y, n, dim, mod, br, tab, eps, st);
}

hipError_t launch_gate_residual(bool bf, const void* x, const void* y, void* out, int32_t n,
                                int32_t dim, const float* mod, int32_t br, const SegTable& tab,
                                hipStream_t st) {
    const int blocks = (n + 3) / 4;
    if (bf)
        gate_residual_kernel<bf16><<<blocks, 256, 0, st>>>((const bf16*)x, (const bf16*)y, (bf16*)out,
                                                           n, dim, mod, br, tab);
    else
        gate_residual_kernel<float><<<blocks, 256, 0, st>>>((const float*)x, (const float*)y,
                                                            (float*)out, n, dim, mod, br, tab);
    return hipGetLastError();
}

hipError_t launch_euler(bool bf, void* x, const void* v, int32_t n, int32_t dim, const SegTable& tab,
                        const SegCoef& coef, hipStream_t st) {
    const int blocks = (n + 3) / 4;
    if (bf)
        euler_kernel<bf16><<<blocks, 256, 0, st>>>((bf16*)x, (const bf16*)v, n, dim, tab, coef);
    else
        euler_kernel<float><<<blocks, 256, 0, st>>>((float*)x, (const float*)v, n, dim, tab, coef);
    return hipGetLastError();
}

hipError_t launch_swiglu(bool bf, const void* gu, void* h, int64_t n, int32_t F, hipStream_t st) {
    const int64_t total = n * (F / (bf ? 8 : 4));
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;   // grid-stride beyond 64 workgroups per CU
    if (bf)
        swiglu_kernel<bf16><<<(unsigned)blocks, 256, 0, st>>>((const bf16*)gu, (bf16*)h, n, F);
    else
        swiglu_kernel<float><<<(unsigned)blocks, 256, 0, st>>>((const float*)gu, (float*)h, n, F);
    return hipGetLastError();
}

hipError_t launch_interleave_gate_up(const void* src, int64_t ld_src_bytes, void* dst, int64_t ld_dst_bytes,
                                     int32_t F, int64_t row_bytes, hipStream_t st) {
    const int64_t pieces = row_bytes / 16;
    interleave_gate_up_kernel<<<stream_blocks(2 * (int64_t)F * pieces), 256, 0, st>>>(
        (const uint8_t*)src, ld_src_bytes, (uint8_t*)dst, ld_dst_bytes, F, pieces);
    return hipGetLastError();
}

hipError_t launch_qknorm_rope(bool bf, void* q, void* k, int64_t ld, int32_t n, int32_t heads,
                              int32_t hd, const float* gq, const float* gk, float eps,
                              const RopeTable& rt, const SegTable& tab, hipStream_t st) {
    if (bf) {
        if (hd == 128)
            qknorm_rope_kernel<bf16, 128><<<n, 256, 0, st>>>((bf16*)q, (bf16*)k, ld, n, heads, gq, gk,
                                                             eps, rt, tab);
        else
            qknorm_rope_kernel<bf16, 64><<<n, 256, 0, st>>>((bf16*)q, (bf16*)k, ld, n, heads, gq, gk,
                                                            eps, rt, tab);
    } else {
        if (hd == 128)
            qknorm_rope_kernel<float, 128><<<n, 256, 0, st>>>((float*)q, (float*)k, ld, n, heads, gq,
                                                              gk, eps, rt, tab);
        else
            qknorm_rope_kernel<float, 64><<<n, 256, 0, st>>>((float*)q, (float*)k, ld, n, heads, gq,
                                                             gk, eps, rt, tab);
    }
    return hipGetLastError();
}

}  // namespace h3
