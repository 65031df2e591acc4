// LNQ (layer-wise non-uniform quantization) on gfx950.
//
// GuidedQuant blog page (jinukkim.me/blog/guidedquant), section "LNQ": per output
// row j, a one-hot assignment P^(j) (P 1_m = 1) and a codebook c^(j); the
// algorithm box repeats a closed-form "(codebook)" step
//     c <- (P^T F P)^{-1} P^T F w
// and an "(assignment)" pass over i = 1..d_in that gives each coordinate the
// codebook entry minimising (w_hat - w)^T F (w_hat - w).  Here F is the damped
// GuidedQuant Fisher block of the row's group, F' = F_g + lambda_g I.
//
// Work split on the GPU
//   k_ridge        lambda_g = rho * mean(diag F_g)                       (float64)
//   k_split        F' -> two bfloat16 planes hi + lo (F' ~= hi + lo to ~2^-17),
//                  plus diag(F') in float32
//   k_lnq_init     per row: m linear quantiles of w_j (float32 weights: from a sort in
//                  LDS; bfloat16: order statistics by radix select), nearest codes
//   k_grid_init    per row: the uniform min-max grid of the fixed-grid backend, nearest codes
//   k_err_split    E = C[P] - W in float32, split into bfloat16 hi + lo planes
//   k_mm (gq_lnq_mm.hip)  residual R = E F' and the codebook Gram blocks
//                  P_j^T F' P_j on the matrix cores
//   k_solve        per row: g = P_j^T r_j, the m x m system from the Gram
//                  partials, float64 Cholesky on the non-empty codes and the
//                  closed-form codebook c <- c - A^{-1} g (= A^{-1} P^T F' w);
//                  also the row objective e . r
//   k_sweep        per 16-row group: the ascending coordinate pass (see there)
//   k_reduce_rows  float64 layer sums in a fixed order
//   k_iter_tail    per iteration: the two trace sums, the move count, counter reset
//   k_check_claim  debug check: a pass's claimed row objectives against fresh ones
#include "gq_common.h"
#include "gq_internal.h"

namespace gq {

constexpr int MAX_M = 16;

// ---------------------------------------------------------------------------
// lambda_g = rho * mean(diag F_g) + lam_abs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ridge(const float* __restrict__ F, int64_t d,
                                              double rho, double lam_abs,
                                              double* __restrict__ lam) {
    __shared__ double red[256];
    const int g = blockIdx.x;
    const float* Fg = F + (size_t)g * d * d;
    double s = 0.0;
    for (int64_t a = threadIdx.x; a < d; a += 256) s += (double)Fg[a * d + a];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) lam[g] = (rho * red[0]) / (double)d + lam_abs;
}

// ---------------------------------------------------------------------------
// F' = F + lambda I -> k-blocked bf16 planes (hi, lo) and float32 diagonal.  One
// thread per (group, 16-block of k, row a of the padded plane): 16 elements of
// row a (zeros for padding rows), written as 32 contiguous bytes per plane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_split(const float* __restrict__ F, int64_t d,
                                              int64_t a_pad, const double* __restrict__ lam,
                                              uint16_t* __restrict__ hi_plane,
                                              uint16_t* __restrict__ lo_plane,
                                              float* __restrict__ dF, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int64_t nkb = d / 16;
    const int64_t a = idx % a_pad;
    const int64_t kb = (idx / a_pad) % nkb;
    const int64_t g = idx / (a_pad * nkb);
    float v[16];
    if (a < d) {
        const float4* src = (const float4*)(F + (g * d + a) * d + kb * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 x = src[k];
            v[4 * k] = x.x; v[4 * k + 1] = x.y; v[4 * k + 2] = x.z; v[4 * k + 3] = x.w;
        }
        if (a >= kb * 16 && a < kb * 16 + 16) {
            const int k = (int)(a - kb * 16);
            v[k] = (float)((double)v[k] + lam[g]);
            dF[g * d + a] = v[k];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = 0.f;
    }
    u32x4 h[2], l[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float f0 = v[2 * k], f1 = v[2 * k + 1];
        const uint32_t hb = pack_bf16x2(f0, f1);
        h[k >> 2][k & 3] = hb;
        l[k >> 2][k & 3] = pack_bf16x2(f0 - __uint_as_float(hb << 16),
                                       f1 - __uint_as_float(hb & 0xffff0000u));
    }
    const int64_t off = ((g * nkb + kb) * a_pad + a) * 16;
    *(u32x4*)(hi_plane + off) = h[0];
    *(u32x4*)(hi_plane + off + 8) = h[1];
    *(u32x4*)(lo_plane + off) = l[0];
    *(u32x4*)(lo_plane + off + 8) = l[1];
}

// ---------------------------------------------------------------------------
// Initial codebook: m quantiles of w_j at levels (q+1/2)/m (linear interpolation
// between order statistics), stored float32; codes: nearest entry, lowest index on
// ties, compared in float64.  One block (1024 threads) per row.
// ---------------------------------------------------------------------------
__device__ __noinline__ double quantile_interp(double lo_v, double hi_v, double frac) {
#pragma clang fp contract(off)
    double diff = hi_v - lo_v;
    double prod = frac * diff;
    return lo_v + prod;
}

template <bool BF16>
__global__ __launch_bounds__(1024) void k_lnq_init(const void* __restrict__ W, int64_t d,
                                                  int npow2, int m, float* __restrict__ C,
                                                  uint8_t* __restrict__ P) {
    extern __shared__ float init_keys[];
    __shared__ float cb[MAX_M];
    const int64_t j = blockIdx.x;
    const int tid = threadIdx.x;
    for (int i = tid; i < npow2; i += 1024)
        init_keys[i] = (i < d) ? load_elem<BF16>(W, j * d + i) : __builtin_inff();
    __syncthreads();
    for (int k = 2; k <= npow2; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            for (int i = tid; i < npow2; i += 1024) {
                const int ixj = i ^ jj;
                if (ixj > i) {
                    const float a = init_keys[i], b = init_keys[ixj];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        init_keys[i] = b;
                        init_keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    if (tid < m) {
        const double h = (double)((d - 1) * (int64_t)(2 * tid + 1)) / (double)(2 * m);
        const double fl = floor(h);
        const int64_t lo = (int64_t)fl;
        const int64_t hi = (lo + 1 < d) ? lo + 1 : d - 1;
        const double v = quantile_interp((double)init_keys[lo], (double)init_keys[hi], h - fl);
        const float cf = (float)v;
        cb[tid] = cf;
        C[j * m + tid] = cf;
    }
    __syncthreads();
    for (int64_t i = tid; i < d; i += 1024) {
        const double w = (double)load_elem<BF16>(W, j * d + i);
        double best = fabs(w - (double)cb[0]);
        int bq = 0;
        for (int q = 1; q < m; ++q) {
            const double dist = fabs(w - (double)cb[q]);
            if (dist < best) { best = dist; bq = q; }
        }
        P[j * d + i] = (uint8_t)bq;
    }
}

// Fixed uniform grid of a row, the scalar backend the GuidedQuant objective is
// plugged into when the codebook is not optimised: m equally spaced values from
// lo = min_i w_i to hi = max_i w_i, c_q = lo + q (hi - lo)/(m - 1) formed in float64
// (no fused multiply-add) and stored float32; codes: nearest entry, lowest index
// on ties, compared in float64.  One block (256 threads) per row.
__device__ __noinline__ double grid_point(double lo, double step, int q) {
#pragma clang fp contract(off)
    double prod = (double)q * step;
    return lo + prod;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_grid_init(const void* __restrict__ W, int64_t d, int m,
                                                  float* __restrict__ C,
                                                  uint8_t* __restrict__ P) {
    __shared__ float red[2][4];
    __shared__ float cb[MAX_M];
    const int64_t j = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int64_t i = tid; i < d; i += 256) {
        const float v = load_elem<BF16>(W, j * d + i);
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, 64));
        hi = fmaxf(hi, __shfl_xor(hi, off, 64));
    }
    if (lane == 0) { red[0][wave] = lo; red[1][wave] = hi; }
    __syncthreads();
    if (tid < m) {
        float l = red[0][0], h = red[1][0];
#pragma unroll
        for (int k = 1; k < 4; ++k) { l = fminf(l, red[0][k]); h = fmaxf(h, red[1][k]); }
        const double step = ((double)h - (double)l) / (double)(m - 1);
        const float cf = (float)grid_point((double)l, step, tid);
        cb[tid] = cf;
        C[j * m + tid] = cf;
    }
    __syncthreads();
    for (int64_t i = tid; i < d; i += 256) {
        const double w = (double)load_elem<BF16>(W, j * d + i);
        double best = fabs(w - (double)cb[0]);
        int bq = 0;
        for (int q = 1; q < m; ++q) {
            const double dist = fabs(w - (double)cb[q]);
            if (dist < best) { best = dist; bq = q; }
        }
        P[j * d + i] = (uint8_t)bq;
    }
}

// The same initial codebook and codes for bfloat16 weights, with the order statistics
// found by a two-pass radix select instead of a sort.  A bfloat16 value maps to a
// 16-bit key whose unsigned order is the value order (sign set: all bits flipped;
// else the sign bit set).  Pass 1 counts the keys by high byte; each needed rank
// (positions floor(h_q) and floor(h_q) + 1) is located in its high-byte bin; pass 2
// counts the low bytes of the keys in those bins; a scan of that count gives the key
// at the rank.  The quantiles are then formed exactly as from the sorted row.  One
// block (256 threads) per row.
__device__ __forceinline__ uint32_t bf16_order_key(uint32_t b) {
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}
__device__ __forceinline__ float bf16_from_order_key(uint32_t k) {
    const uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
    return __uint_as_float(b << 16);
}

__global__ __launch_bounds__(256) void k_lnq_init_select(const uint16_t* __restrict__ W,
                                                         int64_t d, int m,
                                                         float* __restrict__ C,
                                                         uint8_t* __restrict__ P) {
    constexpr int NR = 2 * MAX_M;                // ranks: floor(h_q) and the next, per q
    __shared__ int hist1[256];
    __shared__ int pre1[257];
    __shared__ int hist2[NR][256];
    __shared__ int slot_of_bin[256];
    __shared__ int rank_bin[NR], rank_rem[NR];
    __shared__ float ostat[NR];
    __shared__ float cb[MAX_M];
    const int64_t j = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint16_t* Wj = W + j * d;
    const int nr = 2 * m;
    hist1[tid] = 0;
    slot_of_bin[tid] = -1;
    for (int e = tid; e < NR * 256; e += 256) (&hist2[0][0])[e] = 0;
    __syncthreads();
    // pass 1: high bytes (d % 32 == 0: 8 elements per 16-byte load)
    for (int64_t i = 8 * (int64_t)tid; i < d; i += 8 * 256) {
        const u32x4 v = *(const u32x4*)(Wj + i);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            atomicAdd(&hist1[bf16_order_key((v[e >> 1] >> (16 * (e & 1))) & 0xffffu) >> 8], 1);
    }
    __syncthreads();
    if (wave == 0) {              // exclusive scan of the 256 counts, 4 per lane
        int c[4], t = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) { c[u] = hist1[4 * lane + u]; t += c[u]; }
        int incl = t;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        int run = incl - t;
#pragma unroll
        for (int u = 0; u < 4; ++u) { pre1[4 * lane + u] = run; run += c[u]; }
        if (lane == 63) pre1[256] = incl;
    }
    __syncthreads();
    if (tid < nr) {               // the bin of each rank
        const int q = tid >> 1;
        const double h = (double)((d - 1) * (int64_t)(2 * q + 1)) / (double)(2 * m);
        const int64_t lo = (int64_t)floor(h);
        const int64_t r = (tid & 1) ? ((lo + 1 < d) ? lo + 1 : d - 1) : lo;
        int b = 0;
        for (int st = 128; st > 0; st >>= 1)
            if (pre1[b + st] <= r) b += st;
        rank_bin[tid] = b;
        rank_rem[tid] = (int)(r - pre1[b]);
    }
    __syncthreads();
    if (tid == 0)                 // one low-byte count per distinct bin
        for (int t = 0; t < nr; ++t)
            if (slot_of_bin[rank_bin[t]] < 0) slot_of_bin[rank_bin[t]] = t;
    __syncthreads();
    // pass 2: low bytes of the keys in those bins
    for (int64_t i = 8 * (int64_t)tid; i < d; i += 8 * 256) {
        const u32x4 v = *(const u32x4*)(Wj + i);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t key = bf16_order_key((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            const int sl = slot_of_bin[key >> 8];
            if (sl >= 0) atomicAdd(&hist2[sl][key & 0xffu], 1);
        }
    }
    __syncthreads();
    for (int t = wave; t < nr; t += 4) {   // the key at each rank: a scan per rank
        const int* hb = hist2[slot_of_bin[rank_bin[t]]];
        const int want = rank_rem[t];
        int c[4], tot = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) { c[u] = hb[4 * lane + u]; tot += c[u]; }
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        int run = incl - tot, low = -1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (low < 0 && want >= run && want < run + c[u]) low = 4 * lane + u;
            run += c[u];
        }
        const unsigned long long hit = __ballot(low >= 0);
        const int src = __ffsll((long long)hit) - 1;
        const int lb = __shfl(low, src, 64);
        if (lane == 0) ostat[t] = bf16_from_order_key(((uint32_t)rank_bin[t] << 8) | (uint32_t)lb);
    }
    __syncthreads();
    if (tid < m) {
        const double h = (double)((d - 1) * (int64_t)(2 * tid + 1)) / (double)(2 * m);
        const double fl = floor(h);
        const double v = quantile_interp((double)ostat[2 * tid], (double)ostat[2 * tid + 1], h - fl);
        const float cf = (float)v;
        cb[tid] = cf;
        C[j * m + tid] = cf;
    }
    __syncthreads();
    for (int64_t i = tid; i < d; i += 256) {
        const double w = (double)bf16_bits_to_f32(Wj[i]);
        double best = fabs(w - (double)cb[0]);
        int bq = 0;
        for (int q = 1; q < m; ++q) {
            const double dist = fabs(w - (double)cb[q]);
            if (dist < best) { best = dist; bq = q; }
        }
        P[j * d + i] = (uint8_t)bq;
    }
}

// ---------------------------------------------------------------------------
// E = C[j][P[j][i]] - W[j][i] (float32) -> k-blocked bf16 planes hi + lo.  A block
// covers 64 padded rows x 64 k; thread t takes row t / 4 and k-block t % 4 (16
// elements), so a wave reads 16 rows x 64 contiguous bytes of codes (x 128 of
// weights) and writes, per k-block, 16 consecutive rows = 512 contiguous bytes
// per plane.  Padding rows (past a group's rows) are zero.
// ---------------------------------------------------------------------------
template <bool WBF16>
__global__ __launch_bounds__(256) void k_err_split(const float* __restrict__ C, int m,
                                                  const uint8_t* __restrict__ P,
                                                  const void* __restrict__ W, int64_t d,
                                                  int64_t rpg, int64_t rpg_pad, int64_t erows,
                                                  uint16_t* __restrict__ Ehi,
                                                  uint16_t* __restrict__ Elo,
                                                  const unsigned long long* __restrict__ skip) {
    if (skip && *skip != 0ull) return;
    const int64_t rowp = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
    const int64_t kb = (int64_t)blockIdx.y * 4 + (threadIdx.x & 3);
    if (rowp >= erows || kb * 16 >= d) return;
    const int64_t g = rowp / rpg_pad, jl = rowp - g * rpg_pad;
    u32x4 h[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}}, l[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (jl < rpg) {
        const int64_t j = g * rpg + jl;
        const float* cj = C + j * m;
        const int64_t e0 = j * d + kb * 16;
        const u32x4 pc = *(const u32x4*)(P + e0);
        float w[16];
        if constexpr (WBF16) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 wv = *(const u32x4*)((const uint16_t*)W + e0 + 8 * hh);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    w[8 * hh + 2 * k] = __uint_as_float(wv[k] << 16);
                    w[8 * hh + 2 * k + 1] = __uint_as_float(wv[k] & 0xffff0000u);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 x = *(const float4*)((const float*)W + e0 + 4 * k);
                w[4 * k] = x.x; w[4 * k + 1] = x.y; w[4 * k + 2] = x.z; w[4 * k + 3] = x.w;
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t c0 = (pc[k >> 1] >> (16 * (k & 1))) & 0xffu;
            const uint32_t c1 = (pc[k >> 1] >> (16 * (k & 1) + 8)) & 0xffu;
            const float x0 = cj[c0 < (uint32_t)m ? c0 : 0] - w[2 * k];
            const float x1 = cj[c1 < (uint32_t)m ? c1 : 0] - w[2 * k + 1];
            const uint32_t hb = pack_bf16x2(x0, x1);
            h[k >> 2][k & 3] = hb;
            l[k >> 2][k & 3] = pack_bf16x2(x0 - __uint_as_float(hb << 16),
                                           x1 - __uint_as_float(hb & 0xffff0000u));
        }
    }
    const int64_t off = (kb * erows + rowp) * 16;
    *(u32x4*)(Ehi + off) = h[0];
    *(u32x4*)(Ehi + off + 8) = h[1];
    *(u32x4*)(Elo + off) = l[0];
    *(u32x4*)(Elo + off + 8) = l[1];
}

// lane l's value of v, in every lane
__device__ __forceinline__ double readlane_d(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)b, l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __hiloint2double(hi, lo);
}

// s + x(0) + x(1) + ... + x(n-1), added in that order, the loads issued 8 at a time
template <typename Get>
__device__ __forceinline__ double ordered_sum(int n, Get x, double s) {
    int t = 0;
    for (; t + 8 <= n; t += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = x(t + u);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += (double)v[u];
    }
    for (; t < n; ++t) s += (double)x(t);
    return s;
}

// ---------------------------------------------------------------------------
// k_solve: one wave per row (4 rows per block).
//   Always: obj[j] = sum_a e_a r_a (float64), e = C[j][P[j][a]] - W[j][a].
//   SOLVE:  g = P^T r (the objective's gradient in c, halved), counts per code,
//           A = B + B^T from the Gram partials (summed over a-tiles in order),
//           float64 Cholesky of A on the non-empty codes S and
//               c_S <- c_S - A_SS^{-1} g_S,
//           which is the closed form (P^T F' P)^{-1} P^T F' w because
//           g = P^T F'(P c - w) = A c - P^T F' w.  Empty codes keep c.
// ---------------------------------------------------------------------------
template <int M, bool WBF16, bool SOLVE>
__global__ __launch_bounds__(256) void k_solve(const float* __restrict__ part, int ntile_a,
                                              const float* __restrict__ R,
                                              const uint8_t* __restrict__ P,
                                              const void* __restrict__ W, float* __restrict__ C,
                                              int64_t d, int64_t d_out,
                                              double* __restrict__ obj,
                                              unsigned long long* __restrict__ n_not_pd,
                                              const unsigned long long* __restrict__ mode,
                                              double* __restrict__ afull,
                                              const int* __restrict__ ccount,
                                              const float* __restrict__ dA, int nslices) {
    __shared__ double sB[4][M][M];
    __shared__ double sg[4][M];
    __shared__ int scnt[4][M];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t j0 = (int64_t)blockIdx.x * 4 + wave;
    const bool valid = j0 < d_out;
    const int64_t j = valid ? j0 : 0;

    // lane q < M holds c_q; a coordinate's value is read from the lane of its code
    const float cl = C[j * M + (lane < M ? lane : 0)];

    double o = 0.0;
    float gl[M];
    uint32_t used = 0u;                  // bit q: this lane saw code q
#pragma unroll
    for (int k = 0; k < M; ++k) gl[k] = 0.f;
    if (valid) {
        // 4 consecutive coordinates per lane and step (d % 32 == 0: aligned vectors); the
        // trip count is the same in every lane, so the lanes holding the codebook are
        // active at every shuffle
        const uint8_t* Pj = P + j * d;
        const float* Rj = R + j * d;
#pragma unroll 4
        for (int64_t b0 = 0; b0 < d; b0 += 256) {
            const int64_t a0 = b0 + 4 * lane;
            const bool in = a0 < d;
            uint32_t c4 = 0u;
            float rv[4] = {0.f, 0.f, 0.f, 0.f}, wv[4] = {0.f, 0.f, 0.f, 0.f};
            if (in) {
                c4 = *(const uint32_t*)(Pj + a0);
                const float4 r4 = *(const float4*)(Rj + a0);
                rv[0] = r4.x; rv[1] = r4.y; rv[2] = r4.z; rv[3] = r4.w;
                if constexpr (WBF16) {
                    const u32x2 w2 = *(const u32x2*)((const uint16_t*)W + j * d + a0);
                    wv[0] = __uint_as_float(w2[0] << 16); wv[1] = __uint_as_float(w2[0] & 0xffff0000u);
                    wv[2] = __uint_as_float(w2[1] << 16); wv[3] = __uint_as_float(w2[1] & 0xffff0000u);
                } else {
                    const float4 w4 = *(const float4*)((const float*)W + j * d + a0);
                    wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
                }
            }
            float ck[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) ck[u] = __shfl(cl, (int)((c4 >> (8 * u)) & 0xffu), 64);
            if (in) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int code = (int)((c4 >> (8 * u)) & 0xffu);
                    const float r = rv[u];
                    const float e = ck[u] - wv[u];
                    o += (double)e * (double)r;
                    if (SOLVE) {
                        used |= code < M ? 1u << code : 0u;
#pragma unroll
                        for (int k = 0; k < M; ++k) gl[k] += (code == k) ? r : 0.f;
                    }
                }
            }
        }
    }
    o = wave_sum_f64(o);
    if (valid && lane == 0 && obj) obj[j] = o;
    if (!SOLVE) return;

#pragma unroll
    for (int off = 32; off > 0; off >>= 1) used |= (uint32_t)__shfl_xor((int)used, off, 64);
#pragma unroll
    for (int k = 0; k < M; ++k) {
        const double s = wave_sum_f64((double)gl[k]);
        if (lane == 0) { sg[wave][k] = s; scnt[wave][k] = (int)((used >> k) & 1u); }
    }
    // B_j[q'][q] = sum over a-tiles of part[ta][(j M + q) M + q'], stored as sB[q][q'],
    // so that A = B + B^T.  From the changed coordinates instead (mode 1): sB = A / 2
    // with A = the stored matrix plus the slices' updates, in slice order.  A is stored
    // for the next step.
    const bool incr = mode && *mode != 0ull;
    double* Aj = afull ? afull + (size_t)j * M * M : nullptr;
    if (valid) {
        const bool moved = incr && ccount[j] > 0;
        for (int e = lane; e < M * M; e += 64) {
            const int q = e / M, qp = e - q * M;
            double s = 0.0;
            if (incr) {
                s = Aj[e];
                if (moved)
                    s = ordered_sum(nslices, [&](int sl) {
                        return dA[((size_t)j * nslices + sl) * M * M + e]; }, s);
                s *= 0.5;
            } else {
                s = ordered_sum(ntile_a, [&](int ta) {
                    return part[((size_t)ta * d_out * M + (size_t)(j * M + q)) * M + qp]; }, s);
            }
            sB[wave][q][qp] = s;
        }
    }
    __syncthreads();
    if (valid && Aj) {
        for (int e = lane; e < M * M; e += 64) {
            const int q = e / M, qp = e - q * M;
            Aj[e] = sB[wave][q][qp] + sB[wave][qp][q];
        }
    }
    // Cholesky and the two triangular solves, spread over the wave: lane r holds row r
    // of A (then of L) in registers.  An empty code's row and column are replaced by
    // those of the identity (with g = 0), which leaves the factor of the non-empty
    // codes, taken in increasing code order, unchanged and gives that code a zero
    // step.  Every entry sees the same operations in the same order as the textbook
    // left-looking recurrences
    //     L_rc = (A_rc - sum_{k<c} L_rk L_ck) / L_cc,  L_cc = sqrt(A_cc - sum_{k<c} L_ck^2),
    //     y_r = (-g_r - sum_{k<r} L_rk y_k) / L_rr,    x_r = (y_r - sum_{k>r} L_kr x_k) / L_rr.
    if (valid) {
        const int r = lane;
        const bool rin = r < M;
        const int rr = rin ? r : 0;
        const bool ract = rin && scnt[wave][rr] > 0;
        double a[M];
#pragma unroll
        for (int c = 0; c < M; ++c)
            a[c] = (ract && scnt[wave][c] > 0) ? sB[wave][rr][c] + sB[wave][c][rr]
                                               : ((r == c) ? 1.0 : 0.0);
        bool ok = true;
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const double piv = readlane_d(a[k], k);
            if (!(piv > 0.0)) { ok = false; break; }
            const double lkk = sqrt(piv);
            if (r == k) a[k] = lkk;
            else if (r > k) a[k] = a[k] / lkk;
#pragma unroll
            for (int c = k + 1; c < M; ++c) {
                const double lck = readlane_d(a[k], c);
                if (r >= c) a[c] = fma(-a[k], lck, a[c]);
            }
        }
        if (ok) {
            double t = ract ? -sg[wave][rr] : 0.0;
            double x[M];                  // uniform across the wave
#pragma unroll
            for (int k = 0; k < M; ++k) {
                x[k] = readlane_d(t, k) / readlane_d(a[k], k);
                if (r > k) t = fma(-a[k], x[k], t);
            }
#pragma unroll
            for (int q = M - 1; q >= 0; --q) {
                double s2 = x[q];
#pragma unroll
                for (int k = q + 1; k < M; ++k) s2 = fma(-readlane_d(a[q], k), x[k], s2);
                x[q] = s2 / readlane_d(a[q], q);
            }
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < M; ++k)
                    if (scnt[wave][k] > 0) C[j * M + k] = (float)((double)C[j * M + k] + x[k]);
            }
        } else if (lane == 0 && n_not_pd) {
            atomicAdd(n_not_pd, 1ull);
        }
    }
}

// ---------------------------------------------------------------------------
// k_sweep: the assignment pass.  One block = 16 rows of one group, one row per
// wave (16 waves).  Coordinates are visited in ascending order in blocks of 64
// (one coordinate per lane), grouped into super-blocks of sbsz = 64 .. 512 (the
// assignment block B of the options).
//   * Effect of earlier moves on later residuals, in two levels on the matrix
//     cores (v_mfma_f32_16x16x32_bf16, three products of bf16 hi/lo planes,
//     D hi.F hi + D hi.F lo + D lo.F hi, float32 accumulation):
//       - inside a super-block, before each 64-block, left-looking from the
//         super-block's earlier blocks, corr = D_sb[:, 0:o] F'[sb:sb+o, block],
//         with D_sb (the value changes of the super-block) held in LDS; the
//         terms from all but the previous block are summed while the previous
//         block's chain runs, by the waves whose chains are done;
//       - at the end of a super-block, right-looking into the residual array,
//         R[:, later] += D_sb F'[sb, later], streaming long contiguous panels
//         of F' with the next two chunks' loads in flight during the current
//         two chunks' products (each residual element is owned by one wave,
//         which adds a 16 x 16 tile with 16-byte read-modify-writes; no atomics).
//     The products of 32-coordinate chunks in which no row of the block moved
//     are skipped (the right-looking update still loads them, keeping its loads
//     a fixed distance ahead); a super-block without moves skips the update.
//   * Chain (per wave), first-mover form: every lane t of the 64-block not yet
//     visited evaluates, from the current residual, its m candidate changes
//         Delta_q = delta_q (F'_tt delta_q + 2 r_t),  delta_q = c_q - w_hat_t,
//     keeping the lowest q among equal minima.  Coordinates are visited in
//     ascending order and only a strict decrease changes r, so every coordinate
//     before the first lane with a strictly negative best change keeps its code,
//     exactly as a one-at-a-time pass would decide; a ballot + find-first-set
//     gives that lane t, its move applies r += delta F'[t, block] in registers
//     (the F' rows of the block are staged once through LDS for the 16 rows),
//     and the scan resumes after t.  A block costs (its moves + 1) scans instead
//     of 64 dependent steps, with the same decisions and the same arithmetic.
//   * The row objective e.r at the start of the pass is summed (float64) before
//     any update; the objective after it adds the accepted changes.
//   The residual array R is updated in place (it is workspace).  When recording (for a
//   codebook step updated from the moved coordinates) the pass also writes its moves
//   (clist, ccount) and the codes as they were before it (pprev).
// ---------------------------------------------------------------------------
constexpr int SW_ROWS = 16;     // rows (= waves) per block
constexpr int SW_SUB = 64;      // coordinates per chain block (one per lane)
constexpr int SW_SB = 512;      // largest super-block (the LDS arrays are sized for it)
constexpr int SW_DP = SW_SB + 8;  // bf16 pitch of the LDS rows of D_sb

template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Integer key with the order of the float values (finite or infinite; -0.0 maps
// to -1, +0.0 to 0), so a float minimum becomes one v_min_i32 per DPP step.
__device__ __forceinline__ int f32_order_key(float x) {
    const int b = __float_as_int(x);
    return b ^ ((b >> 31) & 0x7fffffff);
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

// minimum over each row of 16 lanes, available in all 16 lanes
__device__ __forceinline__ int row16_min_i(int v) {
    v = imin(v, dpp_mov_i<0xB1>(v));    // quad_perm [1,0,3,2]
    v = imin(v, dpp_mov_i<0x4E>(v));    // quad_perm [2,3,0,1]
    v = imin(v, dpp_mov_i<0x141>(v));   // row_half_mirror
    v = imin(v, dpp_mov_i<0x140>(v));   // row_mirror
    return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <bool WBF16, int M>
__global__ __launch_bounds__(1024, 1) void k_sweep(
    const float* __restrict__ F, const float* __restrict__ dF,
    const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo,
    int64_t d, int64_t rows_per_group, int wgs_per_group, int total_wgs,
    const float* __restrict__ C, int m, uint8_t* __restrict__ P, const void* __restrict__ W,
    float* __restrict__ R, double* __restrict__ obj_start, double* __restrict__ obj_end,
    unsigned long long* __restrict__ n_changed, uint32_t* __restrict__ clist,
    int* __restrict__ ccount, uint8_t* __restrict__ pprev, int sbsz) {
    __shared__ __attribute__((aligned(16))) uint16_t dsb_hi[SW_ROWS][SW_DP];   // 16.3 KB
    __shared__ __attribute__((aligned(16))) uint16_t dsb_lo[SW_ROWS][SW_DP];   // 16.3 KB
    __shared__ __attribute__((aligned(16))) float corr_p[2][4][SW_ROWS][SW_SUB];   // 32 KB
    __shared__ int ll_next;                            // next left-looking item to take
    __shared__ __attribute__((aligned(16))) float fdb[SW_SUB][SW_SUB];         // 16 KB
    __shared__ float fdd[SW_SUB];                      // diag(F') of the block
    __shared__ uint32_t chunk_moved[SW_SB / 32];       // a move in a 32-chunk of the super-block

    // XCD-aware order: hardware block h runs on XCD h % 8; consecutive logical
    // blocks (the rows of one group) go to the same XCD and share F' in its L2.
    const int nb = gridDim.x;
    const int hw = blockIdx.x;
    const int lin = (hw & 7) * (nb >> 3) + (hw >> 3);
    if (lin >= total_wgs) return;        // whole block exits together

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lin / wgs_per_group;
    const int64_t local = (int64_t)(lin % wgs_per_group) * SW_ROWS;
    const int64_t jl = local + wave;
    const bool rvalid = jl < rows_per_group;
    const int64_t j = (int64_t)g * rows_per_group + (rvalid ? jl : 0);
    const int64_t row0 = (int64_t)g * rows_per_group + local;      // first row of the block
    const int nrows = (int)((rows_per_group - local) < SW_ROWS ? (rows_per_group - local) : SW_ROWS);

    const float* Fg = F + (size_t)g * d * d;
    const float* dFg = dF + (size_t)g * d;
    // k-blocked F' planes: element (a, k) at ((k / 16) * a_pad + a) * 16 + k % 16; the
    // 8 elements (a, k .. k + 7) with k % 8 == 0 are contiguous, and k + 32 is
    // 32 * a_pad elements further on
    const int64_t a_pad = lnq_pad256(d);
    const uint16_t* Fh = Fhi + (size_t)g * d * a_pad;
    const uint16_t* Fl = Flo + (size_t)g * d * a_pad;
    const uint32_t kstep32 = (uint32_t)(32 * a_pad);        // < 2^31 for d <= 32768
    auto plane_at = [&](const uint16_t* base, int64_t a, int64_t k) {
        return base + ((k >> 4) * a_pad + a) * 16 + (k & 15);
    };

    const float cl = (lane < M && rvalid) ? C[j * M + lane] : 0.f;   // candidate of this lane
    float cq[M];                                                     // the row's codebook
#pragma unroll
    for (int q = 0; q < M; ++q) cq[q] = rvalid ? C[j * M + q] : 0.f;
    double dsum = 0.0;       // sum of the accepted changes (uniform in the wave)
    unsigned moves = 0;

    // objective at the start of the pass, before R is updated; the loads of 8 columns
    // per lane are issued together (d % 64 == 0), the sum keeps the column order
    double ostart = 0.0;
    if (rvalid) {
        const int64_t nck = d / 64;
        int64_t c = 0;
        for (; c + 8 <= nck; c += 8) {
            float wv[8], rv[8];
            int pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t col = (c + u) * 64 + lane;
                wv[u] = load_elem<WBF16>(W, j * d + col);
                pv[u] = (int)P[j * d + col];
                rv[u] = R[j * d + col];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float cv = __shfl(cl, pv[u], 64);
                ostart += (double)(cv - wv[u]) * (double)rv[u];
            }
        }
        for (; c < nck; ++c) {
            const int64_t col = c * 64 + lane;
            const float wv = load_elem<WBF16>(W, j * d + col);
            const float cv = __shfl(cl, (int)P[j * d + col], 64);
            ostart += (double)(cv - wv) * (double)R[j * d + col];
        }
    }
    ostart = wave_sum_f64(ostart);

    const int ko = 8 * (lane >> 4);      // k offset of this lane in a 32-wide MFMA step
    const int mrow = lane & 15;          // A-operand row / B-operand column of this lane

    // Loads of the next 64-block of the same super-block, issued while the current
    // block's chain runs: the diagonal 64 x 64 block of F (one float4 per thread), diag
    // F' of the block, and this row's code and residual at its coordinate.  The first
    // block of a super-block loads them itself, after the right-looking update that
    // rewrites later residuals (nothing is carried across that update).
    const int frr = tid >> 4, fcc = (tid & 15) * 4;
    float4 pf_f = make_float4(0.f, 0.f, 0.f, 0.f);
    float pf_d = 0.f, pf_r = 0.f;
    int pf_code = 0;
    auto prefetch = [&](int64_t bsn) {
        pf_f = *(const float4*)(Fg + (bsn + frr) * d + bsn + fcc);
        if (tid < SW_SUB) pf_d = dFg[bsn + tid];
        if (rvalid) {
            pf_code = P[j * d + bsn + lane];
            pf_r = R[j * d + bsn + lane];
        }
    };

    // left-looking item it (0 .. 15) for the block at offset on of the super-block:
    // column tile it % 4, k-slice it / 4, over the 32-chunks c < cend of that slice
    // (in ascending order, chunks without moves skipped), into corr_p[buf]
    auto ll_item = [&](int64_t sb0, int on, int it, int cend, int buf) {
        const int ct = it & 3, sl = it >> 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int64_t fcol = sb0 + on + ct * 16 + mrow;
        const uint16_t* Fh_c = plane_at(Fh, fcol, sb0 + ko);
        const uint16_t* Fl_c = plane_at(Fl, fcol, sb0 + ko);
        for (int c = sl; c < cend; c += 4) {
            if (__builtin_amdgcn_readfirstlane((int)chunk_moved[c]) == 0) continue;
            const u32x4 fh = *(const u32x4*)(Fh_c + (uint32_t)c * kstep32);
            const u32x4 fl = *(const u32x4*)(Fl_c + (uint32_t)c * kstep32);
            const u32x4 dh = *(const u32x4*)(&dsb_hi[mrow][c * 32 + ko]);
            const u32x4 dl = *(const u32x4*)(&dsb_lo[mrow][c * 32 + ko]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh), as_bf16x8(fh), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh), as_bf16x8(fl), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dl), as_bf16x8(fh), acc, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) corr_p[buf][sl][4 * (lane >> 4) + t][ct * 16 + mrow] = acc[t];
    };
    // F' fragments of the last two chunks before the block at offset on, for the column
    // tile and chunk of waves 0 .. 7 (wave w: tile w % 4, chunk on / 32 - 2 + w / 4)
    u32x4 lf_h = {0u, 0u, 0u, 0u}, lf_l = {0u, 0u, 0u, 0u};
    auto ll_tail_load = [&](int64_t sb0, int on) {
        if (wave < 8) {
            const int c = on / 32 - 2 + (wave >> 2);
            const int64_t fcol = sb0 + on + (wave & 3) * 16 + mrow;
            lf_h = *(const u32x4*)(plane_at(Fh, fcol, sb0 + ko) + (uint32_t)c * kstep32);
            lf_l = *(const u32x4*)(plane_at(Fl, fcol, sb0 + ko) + (uint32_t)c * kstep32);
        }
    };

    for (int64_t sb0 = 0; sb0 < d; sb0 += sbsz) {
        const int sblen = (int)((d - sb0) < sbsz ? (d - sb0) : sbsz);
        if (tid < SW_SB / 32) chunk_moved[tid] = 0u;
        // the first block of the super-block has no left-looking correction
#pragma unroll
        for (int k = 0; k < 4; ++k) (&corr_p[0][0][0][0])[tid + 1024 * k] = 0.f;
        prefetch(sb0);
        __syncthreads();
        for (int o = 0; o < sblen; o += SW_SUB) {
            const int64_t bs = sb0 + o;
            const int nb = (o / SW_SUB) & 1;      // this block's correction buffer
            // ---- left-looking correction from this super-block's earlier blocks, in
            // 4 column tiles x 4 k-slices of 32-chunks (slice = chunk % 4).  The chunks
            // before the previous block were summed while the previous block's chain ran
            // (items taken by the waves that finished it first); the previous block's two
            // chunks are added here, each as the last term of its slice, so every slice
            // is summed in ascending chunk order.
            if (o >= SW_SUB) {
                if (wave < 8) {
                    const int ct = wave & 3;
                    const int c = o / 32 - 2 + (wave >> 2);
                    const int sl = c & 3;
                    f32x4 acc;
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[t] = corr_p[nb][sl][4 * (lane >> 4) + t][ct * 16 + mrow];
                    if (__builtin_amdgcn_readfirstlane((int)chunk_moved[c]) != 0) {
                        const u32x4 dh = *(const u32x4*)(&dsb_hi[mrow][c * 32 + ko]);
                        const u32x4 dl = *(const u32x4*)(&dsb_lo[mrow][c * 32 + ko]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh), as_bf16x8(lf_h), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh), as_bf16x8(lf_l), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dl), as_bf16x8(lf_h), acc, 0, 0, 0);
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) corr_p[nb][sl][4 * (lane >> 4) + t][ct * 16 + mrow] = acc[t];
                }
            }
            // the diagonal 64 x 64 block of F (rows bs.., columns bs..), loaded ahead
            *(float4*)&fdb[frr][fcc] = pf_f;
            if (tid < SW_SUB) fdd[tid] = pf_d;
            const int code_in = pf_code;
            const float r_in = pf_r;
            if (tid == 0) ll_next = 0;
            __syncthreads();
            if (o + SW_SUB < sblen) prefetch(bs + SW_SUB);

            float dv = 0.f;
            if (rvalid) {
                const int64_t col = bs + lane;
                float r = r_in;
#pragma unroll
                for (int k = 0; k < 4; ++k) r += corr_p[nb][k][wave][lane];
                int code = code_in;
                if (pprev) pprev[j * d + col] = (uint8_t)code;   // the code before the pass
                float wh = __shfl(cl, code, 64);
                const float wh0 = wh;
                const float fdiag = fdd[lane];            // F'[col][col]
                int start = 0;                            // first coordinate not yet visited
                while (true) {
                    float best = 0.f, bdl = 0.f, bc = 0.f;
                    int bq = -1;
#pragma unroll
                    for (int q = 0; q < M; ++q) {
                        const float dl = cq[q] - wh;
                        const float dq = dl * fmaf(fdiag, dl, 2.f * r);
                        if (dq < best) { best = dq; bq = q; bdl = dl; bc = cq[q]; }
                    }
                    const unsigned long long want = __ballot(lane >= start && bq >= 0);
                    if (want == 0ull) break;
                    const int t = __ffsll((long long)want) - 1;
                    const float delta = readlane_f(bdl, t);
                    dsum += (double)readlane_f(best, t);
                    r = fmaf(delta, fdb[t][lane], r);     // F[bs + t][bs + lane]
                    if (lane == t) {
                        if (clist)                        // (coordinate, old code, new code)
                            clist[j * d + moves] = (uint32_t)col | ((uint32_t)code << 16) |
                                                   ((uint32_t)bq << 24);
                        code = bq;
                        wh = bc;
                    }
                    moves += 1;
                    start = t + 1;
                }
                P[j * d + col] = (uint8_t)code;
                dv = wh - wh0;
                const unsigned long long moved = __ballot(dv != 0.f);
                if (lane == 0) {
                    if (moved & 0xffffffffull) chunk_moved[o / 32] = 1u;
                    if (moved >> 32) chunk_moved[o / 32 + 1] = 1u;
                }
            }
            const uint32_t hb = f32_to_bf16_bits(dv);
            dsb_hi[wave][o + lane] = (uint16_t)hb;
            dsb_lo[wave][o + lane] = (uint16_t)f32_to_bf16_bits(dv - __uint_as_float(hb << 16));
            if (o + SW_SUB < sblen) {
                // the next block's correction from the chunks before this block (their
                // value changes are final), items taken in turn by the waves whose chains
                // are done, so the slowest row's wait absorbs them; then the F' fragments
                // of this block's two chunks for the next block's remaining terms
                for (;;) {
                    int it = 0;
                    if (lane == 0) it = atomicAdd(&ll_next, 1);
                    it = __builtin_amdgcn_readfirstlane(it);
                    if (it >= 16) break;
                    ll_item(sb0, o + SW_SUB, it, o / 32, nb ^ 1);
                }
                ll_tail_load(sb0, o + SW_SUB);
            }
            __syncthreads();
        }
        // ---- right-looking update of the later residuals of the block's rows:
        // R[rows, sb_end:] += D_sb F'[sb0:sb_end, sb_end:], one 16-column tile per wave
        const int64_t sb_end = sb0 + sblen;
        const int ntiles = (int)((d - sb_end) / 16);
        const int nch = sblen / 32;
        uint32_t mv = 0u;                                  // moved chunks as a bit mask
        for (int c = 0; c < nch; ++c) mv |= (chunk_moved[c] != 0u ? 1u : 0u) << c;
        mv = __builtin_amdgcn_readfirstlane(mv);
        for (int ctile = wave; mv != 0u && ctile < ntiles; ctile += SW_ROWS) {
            const int64_t fcol = sb_end + (int64_t)ctile * 16 + mrow;
            const uint16_t* Fh_c = plane_at(Fh, fcol, sb0 + ko);
            const uint16_t* Fl_c = plane_at(Fl, fcol, sb0 + ko);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            // two register sets of two 32-coordinate chunks each: the loads of one set
            // are in flight while the other's products run (nch is even: sblen % 64 == 0)
            u32x4 ah[2], al[2], bh[2], bl[2];
            auto load2 = [&](u32x4 (&h)[2], u32x4 (&l)[2], int c0) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    h[u] = *(const u32x4*)(Fh_c + (uint32_t)(c0 + u) * kstep32);
                    l[u] = *(const u32x4*)(Fl_c + (uint32_t)(c0 + u) * kstep32);
                }
            };
            auto mfma2 = [&](const u32x4 (&h)[2], const u32x4 (&l)[2], int c0) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int c = c0 + u;
                    if ((mv >> c) & 1u) {
                        const u32x4 dh = *(const u32x4*)(&dsb_hi[mrow][c * 32 + ko]);
                        const u32x4 dl = *(const u32x4*)(&dsb_lo[mrow][c * 32 + ko]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh), as_bf16x8(h[u]), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh), as_bf16x8(l[u]), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dl), as_bf16x8(h[u]), acc, 0, 0, 0);
                    }
                }
            };
            load2(ah, al, 0);
            for (int c0 = 0; c0 < nch; c0 += 4) {
                if (c0 + 2 < nch) load2(bh, bl, c0 + 2);
                mfma2(ah, al, c0);
                if (c0 + 4 < nch) load2(ah, al, c0 + 4);
                if (c0 + 2 < nch) mfma2(bh, bl, c0 + 2);
            }
            // the 16 x 16 tile (row 4 (lane / 16) + t, column lane % 16 in acc[t]) is
            // transposed through this wave's quarter of corr_p (unused during the
            // update) so that lane l adds columns 4 (l % 4) .. + 3 of row l / 4 with one
            // 16-byte read-modify-write
            {
                float* xp = &corr_p[0][0][0][0] + wave * 256;
#pragma unroll
                for (int t = 0; t < 4; ++t) xp[(4 * (lane >> 4) + t) * 16 + mrow] = acc[t];
                const int rr = lane >> 2;
                if (rr < nrows) {
                    f32x4* dst = (f32x4*)(R + (row0 + rr) * d + sb_end + (int64_t)ctile * 16 +
                                          4 * (lane & 3));
                    const f32x4 rv = *dst;
                    *dst = rv + *(const f32x4*)(xp + 4 * lane);
                }
            }
        }
        __syncthreads();
    }
    if (rvalid && lane == 0) {
        if (obj_start) obj_start[j] = ostart;
        if (obj_end) obj_end[j] = ostart + dsum;
        if (n_changed) atomicAdd(n_changed, (unsigned long long)moves);
        if (ccount) ccount[j] = (int)moves;
    }
}

// ---------------------------------------------------------------------------
// k_delta: the inputs of the codebook step after an assignment pass that changed
// few coordinates, from those coordinates alone instead of from scratch.
//   Gram: with Delta = P_new - P_old (row i equal to e_v - e_u for a coordinate i
//   that moved from code u to code v, zero elsewhere),
//       A_new - A_old = Delta^T F' P_old + P_new^T F' Delta = X + Y^T,
//       X[q][q'] = sum_i (e_v - e_u)[q] (F' P_old)[i][q'],  Y likewise with P_new,
//   so each changed coordinate needs row i of F' summed by its old and by its new
//   codes: 2m sums over d, taken on the matrix cores as row i times an exact
//   one-hot of [old codes | new codes].  F' rows come from the float32 Fisher
//   (contiguous rows; the diagonal from diag F'), split into bf16 hi + lo as the
//   dense planes are.
//   Residual: the pass has already added each move's effect on the coordinates of
//   later super-blocks; the rest, r[k] += delta_i F'[i][k] for k before the end of
//   i's super-block, is summed in float32 from the same rows.
//   Work item = (row, range of DL_SL-coordinate slices, wider for rows with fewer
//   moves); one block (4 waves) each, longest items first.  The pass lists each row's
//   moves (coordinate, old code, new code) in ascending order; an item takes them DL_G
//   at a time (tiles of 16,
//   one MFMA row block each), its waves interleaving the slice's 32-coordinate
//   chunks.  An item updates the residual of its own coordinates and leaves its
//   share of A_new - A_old (summed per entry in float64 over the changes, in order)
//   for the solve, which adds the slices in order.
// ---------------------------------------------------------------------------
constexpr int DL_TILES = 4;               // 16-change tiles per group
constexpr int DL_G = 16 * DL_TILES;       // changes per group
constexpr int DL_SL = 512;                // coordinates per work item

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over each row of 16 lanes, available in all 16 lanes
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);     // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);     // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);    // row_half_mirror
    v += dpp_f<0x140>(v);    // row_mirror
    return v;
}

// One wave's share of a group of NT tiles (16 changes each): the interleaved
// 32-coordinate chunks c_begin + wave, + 4, ... below c_end.  Each batch issues the loads of CB
// chunks x NT tiles (at most 4 row segments of F per lane), the codes and the
// residual of those chunks, before any of them is used.  Leaves the wave's partial
// sums of the F' rows by [old | new] code in hw[change][column].
template <int M, int NT>
__device__ __forceinline__ void delta_pass(int n, const int* s_i, const float* s_dl,
                                           const uint8_t* __restrict__ po,
                                           const uint8_t* __restrict__ pn,
                                           const float* __restrict__ Fg,
                                           const float* __restrict__ dFg, float* __restrict__ Rj,
                                           int64_t d, int c_begin, int c_end, int wave,
                                           int lane, float (*hw)[16 * ((2 * M + 15) / 16)],
                                           int sbshift) {
    constexpr int NB = (2 * M + 15) / 16;
    constexpr int CB = NT == 1 ? 4 : NT == 2 ? 2 : 1;
    const int mr = lane & 15, ko = 8 * (lane >> 4);
    int ci[NT], sbi[NT];
    float dl[NT];
    const float* frow[NT];                       // row ci of F (row 0 for an empty slot)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int idx = 16 * t + mr;
        const bool ok = idx < n;
        ci[t] = ok ? s_i[idx] : -1;
        dl[t] = ok ? s_dl[idx] : 0.f;
        sbi[t] = ok ? ci[t] >> sbshift : -1;
        frow[t] = Fg + (ok ? (int64_t)ci[t] * d : 0);
    }
    f32x4 acc[NT][NB];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[t][nb] = {0.f, 0.f, 0.f, 0.f};

    for (int cb = c_begin + wave; cb < c_end; cb += 4 * CB) {
        u32x2 co[CB], cn[CB];
        float4 rr[CB];
        float f[CB][NT][8];
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            const int c = cb + 4 * b;
            const int k0 = 32 * c + ko;
            const bool live = c < c_end;
            co[b] = live ? *(const u32x2*)(po + k0) : u32x2{0u, 0u};
            cn[b] = live ? *(const u32x2*)(pn + k0) : u32x2{0u, 0u};
            rr[b] = (live && mr < 2) ? *(const float4*)(Rj + k0 + 4 * mr)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (live && ci[t] >= 0) {
                    const float4* src = (const float4*)(frow[t] + k0);
                    const float4 x0 = src[0], x1 = src[1];
                    f[b][t][0] = x0.x; f[b][t][1] = x0.y; f[b][t][2] = x0.z; f[b][t][3] = x0.w;
                    f[b][t][4] = x1.x; f[b][t][5] = x1.y; f[b][t][6] = x1.z; f[b][t][7] = x1.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[b][t][e] = 0.f;
                }
            }
        }
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            const int c = cb + 4 * b;
            if (c >= c_end) continue;                    // uniform in the wave
            const int k0 = 32 * c + ko;                  // this lane's 8 coordinates
            const int sbk = (32 * c) >> sbshift;
            u32x4 oh[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int col = 16 * nb + mr;
                const bool isold = col < M, used = col < 2 * M;
                const uint32_t tgt = (uint32_t)(isold ? col : col - M);
                const u32x2 cc = isold ? co[b] : cn[b];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t b0 = (cc[e >> 1] >> (16 * (e & 1))) & 0xffu;
                    const uint32_t b1 = (cc[e >> 1] >> (16 * (e & 1) + 8)) & 0xffu;
                    oh[nb][e] = ((used && b0 == tgt) ? 0x3F80u : 0u) |
                                ((used && b1 == tgt) ? 0x3F800000u : 0u);
                }
            }
            float pr[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pr[e] = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int off = ci[t] - k0;
                if ((unsigned)off < 8u) {                 // F'[i][i] = diag F'
                    const float di = dFg[ci[t]];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (off == e) f[b][t][e] = di;
                }
                u32x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f0 = f[b][t][2 * e], f1 = f[b][t][2 * e + 1];
                    const uint32_t hb = pack_bf16x2(f0, f1);
                    hi[e] = hb;
                    lo[e] = pack_bf16x2(f0 - __uint_as_float(hb << 16),
                                        f1 - __uint_as_float(hb & 0xffff0000u));
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi), as_bf16x8(oh[nb]), acc[t][nb], 0, 0, 0);
                    acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), as_bf16x8(oh[nb]), acc[t][nb], 0, 0, 0);
                }
                const float dd = (sbi[t] >= sbk) ? dl[t] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = fmaf(dd, f[b][t][e], pr[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) pr[e] = row16_sum(pr[e]);
            if (mr < 2) {
                float4 x = rr[b];
                x.x += mr ? pr[4] : pr[0];
                x.y += mr ? pr[5] : pr[1];
                x.z += mr ? pr[6] : pr[2];
                x.w += mr ? pr[7] : pr[3];
                *(float4*)(Rj + k0 + 4 * mr) = x;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) hw[16 * t + 4 * (lane >> 4) + e][16 * nb + mr] = acc[t][nb][e];
}

// Work items, longest first.  Rows are ordered by decreasing move count (buckets of
// 16 moves; the order within a bucket is arbitrary and affects scheduling only).  A
// row with K moves is split into min(slices, ceil(K / 16)) items over contiguous
// ranges of DL_SL-coordinate slices, so that items carry similar work and none is long.
// Item: row | first slice << 32 | end slice << 48.  One block of 1024 threads.
__global__ __launch_bounds__(1024) void k_order_rows(const unsigned long long* __restrict__ mode,
                                                    const int* __restrict__ ccount, int64_t n,
                                                    int nslices, int* __restrict__ order,
                                                    unsigned long long* __restrict__ items,
                                                    int* __restrict__ nitems) {
    constexpr int NBK = 64;
    __shared__ int hist[NBK];
    __shared__ int base[NBK];
    __shared__ int wsum[16];
    __shared__ int run;
    if (*mode == 0ull) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < NBK) hist[tid] = 0;
    if (tid == 0) run = 0;
    __syncthreads();
    auto bucket = [](int c) {
        int b = (c + 15) >> 4;
        b = b < 0 ? 0 : (b > NBK - 1 ? NBK - 1 : b);
        return NBK - 1 - b;
    };
    for (int64_t j = tid; j < n; j += 1024) atomicAdd(&hist[bucket(ccount[j])], 1);
    __syncthreads();
    if (tid == 0) {
        int a = 0;
        for (int b = 0; b < NBK; ++b) { base[b] = a; a += hist[b]; }
    }
    __syncthreads();
    for (int64_t j = tid; j < n; j += 1024) order[atomicAdd(&base[bucket(ccount[j])], 1)] = (int)j;
    __syncthreads();
    // items in that order: an exclusive scan of the item counts, 1024 rows at a time
    for (int64_t c0 = 0; c0 < n; c0 += 1024) {
        const int64_t p = c0 + tid;
        int row = 0, k = 0, cnt = 0;
        if (p < n) {
            row = order[p];
            k = ccount[row];
            cnt = k <= 0 ? 0 : ((k + 15) / 16 < nslices ? (k + 15) / 16 : nslices);
        }
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int ex = run + incl - cnt;
        for (int w = 0; w < wave; ++w) ex += wsum[w];
        for (int i = 0; i < cnt; ++i) {
            const unsigned long long lo = (unsigned long long)(i * nslices / cnt);
            const unsigned long long hi = (unsigned long long)((i + 1) * nslices / cnt);
            items[ex + i] = (unsigned long long)(unsigned)row | (lo << 32) | (hi << 48);
        }
        __syncthreads();
        if (tid == 0) {
            int tot = 0;
            for (int w = 0; w < 16; ++w) tot += wsum[w];
            run += tot;
        }
        __syncthreads();
    }
    if (tid == 0) *nitems = run;
}

template <int M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(M <= 8 ? 3 : 2, 4))) void k_delta(
    const unsigned long long* __restrict__ mode, const float* __restrict__ F,
    const float* __restrict__ dF, int64_t d, int64_t rows_per_group,
    const uint8_t* __restrict__ Pold, const uint8_t* __restrict__ Pnew,
    const float* __restrict__ C, float* __restrict__ R, const uint32_t* __restrict__ clist,
    const int* __restrict__ ccount, const unsigned long long* __restrict__ items,
    const int* __restrict__ nitems, int nslices, float* __restrict__ dA, int sbshift) {
    constexpr int NB = (2 * M + 15) / 16;     // 16-column blocks of [old | new] one-hots
    __shared__ int s_i[DL_G];                 // coordinate of each change of the group
    __shared__ int s_uv[DL_G];                // old code | new code << 8
    __shared__ float s_dl[DL_G];              // c[new] - c[old]
    __shared__ float s_h[4][DL_G][16 * NB];   // per-wave partial sums of the F' rows
    if (*mode == 0ull) return;

    if ((int)blockIdx.x >= *nitems) return;
    const unsigned long long item = items[blockIdx.x];
    const int64_t j = (int64_t)(item & 0xffffffffull);
    const int s_lo = (int)((item >> 32) & 0xffffu), s_hi = (int)(item >> 48);
    const int K = ccount[j];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t g = j / rows_per_group;
    const uint8_t* po = Pold + j * d;
    const uint8_t* pn = Pnew + j * d;
    const float* Fg = F + (size_t)g * d * d;
    const float* dFg = dF + (size_t)g * d;
    float* Rj = R + j * d;
    const float* cj = C + j * M;
    const uint32_t* lj = clist + j * d;
    const int nch = (int)(d / 32);
    const int c_begin = s_lo * (DL_SL / 32);
    const int c_end = (s_hi * (DL_SL / 32)) < nch ? (s_hi * (DL_SL / 32)) : nch;
    const int aq = tid / M, aqq = tid % M;    // entry of A owned by threads tid < M * M
    double accA = 0.0;

    for (int g0 = 0; g0 < K; g0 += DL_G) {
        const int n = (K - g0) < DL_G ? (K - g0) : DL_G;
        if (tid < n) {
            const uint32_t e = lj[g0 + tid];
            const int u = (int)((e >> 16) & 0xffu), v = (int)(e >> 24);
            s_i[tid] = (int)(e & 0xffffu);
            s_uv[tid] = u | (v << 8);
            s_dl[tid] = cj[v] - cj[u];
        }
        __syncthreads();
        switch ((n + 15) >> 4) {
            case 1: delta_pass<M, 1>(n, s_i, s_dl, po, pn, Fg, dFg, Rj, d, c_begin, c_end, wave, lane, s_h[wave], sbshift); break;
            case 2: delta_pass<M, 2>(n, s_i, s_dl, po, pn, Fg, dFg, Rj, d, c_begin, c_end, wave, lane, s_h[wave], sbshift); break;
            case 3: delta_pass<M, 3>(n, s_i, s_dl, po, pn, Fg, dFg, Rj, d, c_begin, c_end, wave, lane, s_h[wave], sbshift); break;
            default: delta_pass<M, 4>(n, s_i, s_dl, po, pn, Fg, dFg, Rj, d, c_begin, c_end, wave, lane, s_h[wave], sbshift); break;
        }
        __syncthreads();
        // ---- this slice's part of A_new - A_old, entry (aq, aqq): X[aq][aqq] + Y[aqq][aq]
        if (tid < M * M) {
            for (int kk = 0; kk < n; ++kk) {
                const int uv = s_uv[kk], u = uv & 0xff, v = uv >> 8;
                const int sg1 = (v == aq) - (u == aq);
                const int sg2 = (v == aqq) - (u == aqq);
                if (sg1) {
                    const double h = (double)s_h[0][kk][aqq] + s_h[1][kk][aqq] + s_h[2][kk][aqq] +
                                     s_h[3][kk][aqq];
                    accA += sg1 * h;
                }
                if (sg2) {
                    const double h = (double)s_h[0][kk][M + aq] + s_h[1][kk][M + aq] +
                                     s_h[2][kk][M + aq] + s_h[3][kk][M + aq];
                    accA += sg2 * h;
                }
            }
        }
        __syncthreads();
    }
    // the item's share goes to its first slice; the other slices it covers hold zero
    if (tid < M * M) {
        dA[((size_t)j * nslices + s_lo) * M * M + tid] = (float)accA;
        for (int sl = s_lo + 1; sl < s_hi; ++sl) dA[((size_t)j * nslices + sl) * M * M + tid] = 0.f;
    }
}

// float64 sums of consecutive rows in a fixed order: out[0] = sum_j x[j]
__global__ __launch_bounds__(256) void k_reduce_rows(const double* __restrict__ x, int64_t n,
                                                    double* __restrict__ out) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += x[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = red[0];
}

__global__ void k_store_i64(const unsigned long long* __restrict__ src, int64_t* __restrict__ dst) {
    *dst = (int64_t)*src;
}

__global__ void k_add_i64(const unsigned long long* __restrict__ src, int64_t* __restrict__ dst) {
    *dst += (int64_t)*src;
}

// End of one LNQ iteration, in one launch: block 0 sums the objectives before the
// codebook step (trace entry 2t - 2), block 1 those before the assignment pass
// (entry 2t - 1), each in a fixed order; block 2 stores the pass's move count and
// clears the counter for the next pass.
__global__ __launch_bounds__(256) void k_iter_tail(const double* __restrict__ objA,
                                                  const double* __restrict__ objB, int64_t n,
                                                  double* __restrict__ trace,
                                                  unsigned long long* __restrict__ cnt,
                                                  int64_t* __restrict__ n_changed,
                                                  int64_t incr_max) {
    __shared__ double red[256];
    if (blockIdx.x == 2) {
        if (threadIdx.x == 0) {
            const unsigned long long moves = cnt[0];
            if (n_changed) *n_changed = (int64_t)moves;
            cnt[2] = (incr_max >= 0 && moves <= (unsigned long long)incr_max) ? 1ull : 0ull;
            cnt[0] = 0ull;
        }
        return;
    }
    if (!trace) return;
    const double* x = blockIdx.x == 0 ? objA : objB;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += x[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) trace[blockIdx.x] = red[0];
}

// ---------------------------------------------------------------------------
// Debug check of an assignment pass: the objective each row reached through the pass's
// running residual (its start plus the accepted changes, `claimed`) against the same
// row's objective recomputed from scratch (`fresh`).  Rows whose two figures differ by
// more than tol |start| (or are not finite) are counted into *bad.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_check_claim(const double* __restrict__ start,
                                                    const double* __restrict__ claimed,
                                                    const double* __restrict__ fresh, int64_t n,
                                                    double tol,
                                                    unsigned long long* __restrict__ bad) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    const double d = fabs(claimed[j] - fresh[j]);
    if (!(d <= tol * fabs(start[j]))) atomicAdd(bad, 1ull);
}

// ---------------------------------------------------------------------------
// Checked calls: *flag |= 1 if any of the n values (float32 or bfloat16) is NaN or
// +-Inf (all exponent bits set).  16-byte vectors where whole, elements at the tail.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_nonfinite(const void* __restrict__ p, int64_t n,
                                                  int bf16, unsigned long long* __restrict__ flag) {
    const int64_t per_vec = bf16 ? 8 : 4;
    const int64_t nvec = n / per_vec;
    const int64_t stride = (int64_t)gridDim.x * 256;
    bool bad = false;
    for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += stride) {
        const u32x4 x = ((const u32x4*)p)[v];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (bf16) {
                bad |= (x[k] & 0x7f80u) == 0x7f80u;
                bad |= (x[k] & 0x7f800000u) == 0x7f800000u;
            } else {
                bad |= (x[k] & 0x7f800000u) == 0x7f800000u;
            }
        }
    }
    for (int64_t e = nvec * per_vec + (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += stride) {
        if (bf16) bad |= (((const uint16_t*)p)[e] & 0x7f80u) == 0x7f80u;
        else bad |= (((const uint32_t*)p)[e] & 0x7f800000u) == 0x7f800000u;
    }
    if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0) atomicOr(flag, 1ull);
}

__global__ void k_zero_u64(unsigned long long* __restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

}  // namespace gq

// ===========================================================================
// Host launchers
// ===========================================================================
namespace gq {

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

LnqSizes lnq_sizes(int64_t d_out, int64_t d, int groups, int m) {
    LnqSizes z{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const int64_t a_pad = lnq_pad256(d), rpg_pad = lnq_pad256(d_out / groups);
    z.o_fhi = take((size_t)groups * d * a_pad * 2);
    z.o_flo = take((size_t)groups * d * a_pad * 2);
    z.o_dF = take((size_t)groups * d * 4);
    z.o_lam = take((size_t)groups * 8);
    z.o_R = take((size_t)d_out * d * 4);
    z.o_ehi = take((size_t)groups * rpg_pad * d * 2);
    z.o_elo = take((size_t)groups * rpg_pad * d * 2);
    z.o_part = take(lnq_gram_partial_floats(d_out, d, m) * 4);
    z.o_objA = take((size_t)d_out * 8);
    z.o_objB = take((size_t)d_out * 8);
    z.o_objC = take((size_t)d_out * 8);
    z.o_cnt = take(16 * 8);
    z.o_pprev = take((size_t)d_out * d);
    z.o_afull = take((size_t)d_out * m * m * 8);
    z.o_clist = take((size_t)d_out * d * 4);
    z.o_ccount = take((size_t)d_out * 4);
    z.o_order = take((size_t)d_out * 4);
    z.o_items = take((size_t)d_out * ((d + DL_SL - 1) / DL_SL) * 8);
    z.o_nitems = take(8);
    z.o_dA = take((size_t)d_out * ((d + DL_SL - 1) / DL_SL) * m * m * 4);
    z.total = off;
    return z;
}

LnqWs lnq_carve(void* base, const LnqSizes& z) {
    char* b = (char*)base;
    LnqWs w{};
    w.fhi = (uint16_t*)(b + z.o_fhi);
    w.flo = (uint16_t*)(b + z.o_flo);
    w.dF = (float*)(b + z.o_dF);
    w.lam = (double*)(b + z.o_lam);
    w.R = (float*)(b + z.o_R);
    w.ehi = (uint16_t*)(b + z.o_ehi);
    w.elo = (uint16_t*)(b + z.o_elo);
    w.part = (float*)(b + z.o_part);
    w.objA = (double*)(b + z.o_objA);
    w.objB = (double*)(b + z.o_objB);
    w.objC = (double*)(b + z.o_objC);
    w.cnt = (unsigned long long*)(b + z.o_cnt);
    w.pprev = (uint8_t*)(b + z.o_pprev);
    w.afull = (double*)(b + z.o_afull);
    w.clist = (uint32_t*)(b + z.o_clist);
    w.ccount = (int*)(b + z.o_ccount);
    w.order = (int*)(b + z.o_order);
    w.items = (unsigned long long*)(b + z.o_items);
    w.nitems = (int*)(b + z.o_nitems);
    w.dA = (float*)(b + z.o_dA);
    return w;
}

hipError_t lnq_prepare(const float* F, int groups, int64_t d, double rho, double lam_abs,
                       const LnqWs& w, hipStream_t st) {
    StageTimer tm(ST_LNQ_PREPARE, st);
    hipLaunchKernelGGL(k_ridge, dim3(groups), dim3(256), 0, st, F, d, rho, lam_abs, w.lam);
    GQ_LAUNCH_CHECK();
    const int64_t a_pad = lnq_pad256(d);
    const int64_t total = (int64_t)groups * (d / 16) * a_pad;
    hipLaunchKernelGGL(k_split, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, F, d,
                       a_pad, w.lam, w.fhi, w.flo, w.dF, total);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_init_run(const void* W, bool w_bf16, int64_t d_out, int64_t d, int m, float* C,
                        uint8_t* P, hipStream_t st) {
    int npow2 = 1;
    while (npow2 < d) npow2 <<= 1;
    const size_t lds = (size_t)npow2 * sizeof(float);
    StageTimer tm(ST_LNQ_INIT, st);
    if (w_bf16) {
        hipLaunchKernelGGL(k_lnq_init_select, dim3((unsigned)d_out), dim3(256), 0, st,
                           (const uint16_t*)W, d, m, C, P);
    } else {
        hipError_t e = ensure_dynamic_lds((const void*)k_lnq_init<false>, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_lnq_init<false>, dim3((unsigned)d_out), dim3(1024), lds, st, W, d,
                           npow2, m, C, P);
    }
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t grid_init_run(const void* W, bool w_bf16, int64_t d_out, int64_t d, int m, float* C,
                         uint8_t* P, hipStream_t st) {
    StageTimer tm(ST_LNQ_INIT, st);
    if (w_bf16)
        hipLaunchKernelGGL(k_grid_init<true>, dim3((unsigned)d_out), dim3(256), 0, st, W, d, m, C, P);
    else
        hipLaunchKernelGGL(k_grid_init<false>, dim3((unsigned)d_out), dim3(256), 0, st, W, d, m, C, P);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_residual_from(const float* C, int m, const uint8_t* P, const void* W, bool w_bf16,
                             int64_t d_out, int64_t d, int groups, const LnqWs& w,
                             const unsigned long long* skip, hipStream_t st) {
    {
        StageTimer tm(ST_LNQ_RESID, st);
        const int64_t rpg = d_out / groups, rpg_pad = lnq_pad256(rpg);
        const int64_t erows = (int64_t)groups * rpg_pad;
        const dim3 grid((unsigned)(erows / 64), (unsigned)((d / 16 + 3) / 4));   // erows % 256 == 0
        if (w_bf16)
            hipLaunchKernelGGL(k_err_split<true>, grid, dim3(256), 0, st, C, m, P, W, d, rpg,
                               rpg_pad, erows, w.ehi, w.elo, skip);
        else
            hipLaunchKernelGGL(k_err_split<false>, grid, dim3(256), 0, st, C, m, P, W, d, rpg,
                               rpg_pad, erows, w.ehi, w.elo, skip);
        GQ_LAUNCH_CHECK();
    }
    return lnq_residual(w.ehi, w.elo, d_out, d, groups, w.fhi, w.flo, w.R, skip, st);
}

template <int M, bool WB, bool SOLVE>
static hipError_t launch_solve(const float* part, int nta, const float* R, const uint8_t* P,
                               const void* W, float* C, int64_t d, int64_t d_out, double* obj,
                               unsigned long long* n_not_pd, const unsigned long long* mode,
                               const LnqWs* w, hipStream_t st) {
    const int nsl = (int)((d + DL_SL - 1) / DL_SL);
    hipLaunchKernelGGL((k_solve<M, WB, SOLVE>), dim3((unsigned)((d_out + 3) / 4)), dim3(256), 0,
                       st, part, nta, R, P, W, C, d, d_out, obj, n_not_pd, mode,
                       w ? w->afull : nullptr, w ? w->ccount : nullptr, w ? w->dA : nullptr, nsl);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

template <bool WB, bool SOLVE>
static hipError_t solve_m(int m, const float* part, int nta, const float* R, const uint8_t* P,
                          const void* W, float* C, int64_t d, int64_t d_out, double* obj,
                          unsigned long long* n_not_pd, const unsigned long long* mode,
                          const LnqWs* w, hipStream_t st) {
    switch (m) {
        case 2: return launch_solve<2, WB, SOLVE>(part, nta, R, P, W, C, d, d_out, obj, n_not_pd, mode, w, st);
        case 4: return launch_solve<4, WB, SOLVE>(part, nta, R, P, W, C, d, d_out, obj, n_not_pd, mode, w, st);
        case 8: return launch_solve<8, WB, SOLVE>(part, nta, R, P, W, C, d, d_out, obj, n_not_pd, mode, w, st);
        case 16: return launch_solve<16, WB, SOLVE>(part, nta, R, P, W, C, d, d_out, obj, n_not_pd, mode, w, st);
        default: return hipErrorInvalidValue;
    }
}

template <int M>
static hipError_t launch_delta(const unsigned long long* mode, const float* F, int64_t d,
                               int64_t d_out, int groups, const uint8_t* P, const float* C,
                               const LnqWs& w, hipStream_t st) {
    const int nsl = (int)((d + DL_SL - 1) / DL_SL);
    hipLaunchKernelGGL(k_order_rows, dim3(1), dim3(1024), 0, st, mode, w.ccount, d_out, nsl,
                       w.order, w.items, w.nitems);
    GQ_LAUNCH_CHECK();
    hipLaunchKernelGGL((k_delta<M>), dim3((unsigned)(d_out * nsl)), dim3(256), 0, st, mode, F,
                       w.dF, d, d_out / groups, w.pprev, P, C, w.R, w.clist, w.ccount, w.items, w.nitems,
                       nsl, w.dA, w.sb_shift);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

static hipError_t delta_m(int m, const unsigned long long* mode, const float* F, int64_t d,
                          int64_t d_out, int groups, const uint8_t* P, const float* C,
                          const LnqWs& w, hipStream_t st) {
    switch (m) {
        case 2: return launch_delta<2>(mode, F, d, d_out, groups, P, C, w, st);
        case 4: return launch_delta<4>(mode, F, d, d_out, groups, P, C, w, st);
        case 8: return launch_delta<8>(mode, F, d, d_out, groups, P, C, w, st);
        case 16: return launch_delta<16>(mode, F, d, d_out, groups, P, C, w, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t lnq_codebook_step(const float* F, const void* W, bool w_bf16, int64_t d_out, int64_t d,
                             int groups, int m, const uint8_t* P, float* C, const LnqWs& w,
                             double* obj_before, unsigned long long* n_not_pd,
                             const unsigned long long* mode, hipStream_t st) {
    // from scratch (skipped on the device when *mode != 0)
    hipError_t e = lnq_residual_from(C, m, P, W, w_bf16, d_out, d, groups, w, mode, st);
    if (e != hipSuccess) return e;
    if ((e = lnq_gram(P, m, d_out, d, groups, w.fhi, w.flo, w.part, mode, st)) != hipSuccess)
        return e;
    if (mode) {
        // from the changed coordinates (nothing when *mode == 0)
        StageTimer tm(ST_LNQ_DELTA, st);
        if ((e = delta_m(m, mode, F, d, d_out, groups, P, C, w, st)) != hipSuccess) return e;
    }
    const int nta = (int)((d + 255) / 256);
    StageTimer tm(ST_LNQ_SOLVE, st);
    return w_bf16 ? solve_m<true, true>(m, w.part, nta, w.R, P, W, C, d, d_out, obj_before, n_not_pd, mode, &w, st)
                  : solve_m<false, true>(m, w.part, nta, w.R, P, W, C, d, d_out, obj_before, n_not_pd, mode, &w, st);
}

hipError_t lnq_objective_rows(const void* W, bool w_bf16, int64_t d_out, int64_t d, int groups,
                              int m, const uint8_t* P, const float* C, const LnqWs& w,
                              double* obj, hipStream_t st) {
    hipError_t e = lnq_residual_from(C, m, P, W, w_bf16, d_out, d, groups, w, nullptr, st);
    if (e != hipSuccess) return e;
    StageTimer tm(ST_LNQ_SOLVE, st);
    return w_bf16 ? solve_m<true, false>(m, nullptr, 0, w.R, P, W, (float*)C, d, d_out, obj, nullptr, nullptr, nullptr, st)
                  : solve_m<false, false>(m, nullptr, 0, w.R, P, W, (float*)C, d, d_out, obj, nullptr, nullptr, nullptr, st);
}

template <bool WB>
static hipError_t launch_sweep(const float* F, const void* W, int64_t d_out, int64_t d,
                               int groups, const float* C, int m, uint8_t* P, const LnqWs& w,
                               double* obj_start, double* obj_end, unsigned long long* counter,
                               bool record, hipStream_t st) {
    const int64_t rpg = d_out / groups;
    const int wgs = (int)((rpg + SW_ROWS - 1) / SW_ROWS);
    const int total = wgs * groups;
    const int grid = (total + 7) / 8 * 8;          // the XCD remap needs a multiple of 8
    auto kern = (m == 2) ? k_sweep<WB, 2> : (m == 4) ? k_sweep<WB, 4> : (m == 8) ? k_sweep<WB, 8>
                                                                         : k_sweep<WB, 16>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(1024), 0, st, F, w.dF, w.fhi,
                       w.flo, d, rpg, wgs, total, C, m, P, W, w.R, obj_start, obj_end, counter,
                       record ? w.clist : nullptr, record ? w.ccount : nullptr,
                       record ? w.pprev : nullptr, 1 << w.sb_shift);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_sweep_step(const float* F, const void* W, bool w_bf16, int64_t d_out,
                          int64_t d, int groups, const float* C, int m, uint8_t* P,
                          const LnqWs& w, double* obj_start, double* obj_end,
                          unsigned long long* counter, bool record, hipStream_t st) {
    if (w.sb_shift < 6 || w.sb_shift > 9 || d % SW_SUB) return hipErrorInvalidValue;
    hipError_t e = lnq_residual_from(C, m, P, W, w_bf16, d_out, d, groups, w, nullptr, st);
    if (e != hipSuccess) return e;
    StageTimer tm(ST_LNQ_SWEEP, st);
    return w_bf16 ? launch_sweep<true>(F, W, d_out, d, groups, C, m, P, w, obj_start, obj_end, counter, record, st)
                  : launch_sweep<false>(F, W, d_out, d, groups, C, m, P, w, obj_start, obj_end, counter, record, st);
}

hipError_t lnq_reduce(const double* rows, int64_t n, double* out, hipStream_t st) {
    StageTimer tm(ST_LNQ_SMALL, st);
    hipLaunchKernelGGL(k_reduce_rows, dim3(1), dim3(256), 0, st, rows, n, out);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_iter_tail(const double* objA, const double* objB, int64_t n, double* trace,
                         unsigned long long* cnt, int64_t* n_changed, int64_t incr_max,
                         hipStream_t st) {
    StageTimer tm(ST_LNQ_SMALL, st);
    hipLaunchKernelGGL(k_iter_tail, dim3(3), dim3(256), 0, st, objA, objB, n, trace, cnt,
                       n_changed, incr_max);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_check_claim(const double* start, const double* claimed, const double* fresh,
                           int64_t n, double tol, unsigned long long* bad, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    StageTimer tm(ST_LNQ_SMALL, st);
    hipLaunchKernelGGL(k_check_claim, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, start,
                       claimed, fresh, n, tol, bad);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_zero_counter(unsigned long long* c, int n, hipStream_t st) {
    StageTimer tm(ST_LNQ_SMALL, st);
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, st, c, n);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t scan_nonfinite(const void* p, bool bf16, int64_t n, unsigned long long* flag,
                          hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t vecs = n / (bf16 ? 8 : 4) + 1;
    const int64_t blocks = (vecs + 255) / 256;
    hipLaunchKernelGGL(k_nonfinite, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0,
                       st, p, n, bf16 ? 1 : 0, flag);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_store_counter(const unsigned long long* c, int64_t* dst, hipStream_t st) {
    StageTimer tm(ST_LNQ_SMALL, st);
    hipLaunchKernelGGL(k_store_i64, dim3(1), dim3(1), 0, st, c, dst);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

}  // namespace gq
