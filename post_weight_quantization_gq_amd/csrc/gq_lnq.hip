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
//   k_lnq_init     per row: sort w_j in LDS, m linear quantiles, nearest codes
//   k_fgemm        MFMA products with F': V = W F' (iteration invariant) and
//                  U_j = F' P_j for every row (P_j one-hot, built from the codes
//                  while staging; exact in bfloat16)
//   k_solve        per row: A_j = P_j^T U_j, b_j = P_j^T v_j, float64 Cholesky on
//                  the non-empty codes, residual r_j = U_j c_j - v_j and objectives
//   k_sweep        per 16-row group: ascending coordinate descent on the residual;
//                  inside a block of B coordinates every update is applied at once
//                  (registers + LDS), the effect of earlier blocks on the next one
//                  is gathered on MFMA from the recorded value changes (left-looking)
//   k_reduce_rows  float64 layer sums in a fixed order
#include "gq_common.h"

namespace gq {

constexpr int MAX_M = 16;

// ---------------------------------------------------------------------------
// lambda_g = rho * mean(diag F_g)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ridge(const float* __restrict__ F, int64_t d,
                                              double rho, double* __restrict__ lam) {
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
    if (threadIdx.x == 0) lam[g] = (rho * red[0]) / (double)d;
}

// ---------------------------------------------------------------------------
// F' = F + lambda I -> bf16 planes (hi, lo) and float32 diagonal.  8 elems / thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_split(const float* __restrict__ F, int64_t d,
                                              const double* __restrict__ lam,
                                              uint16_t* __restrict__ hi_plane,
                                              uint16_t* __restrict__ lo_plane,
                                              float* __restrict__ dF, int64_t total8) {
    const int64_t idx8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx8 >= total8) return;
    const int64_t e0 = idx8 * 8;
    const int64_t dd = d * d;
    const int64_t g = e0 / dd;
    const int64_t rem = e0 - g * dd;
    const int64_t a = rem / d;
    const int64_t i0 = rem - a * d;       // d % 8 == 0: the 8 elements share a row
    const float4* src = (const float4*)(F + e0);
    float4 x0 = src[0], x1 = src[1];
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (a >= i0 && a < i0 + 8) {
        const int k = (int)(a - i0);
        v[k] = (float)((double)v[k] + lam[g]);
        dF[g * d + a] = v[k];
    }
    u32x4 h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float f0 = v[2 * k], f1 = v[2 * k + 1];
        uint32_t hb = pack_bf16x2(f0, f1);
        float r0 = f0 - __uint_as_float(hb << 16);
        float r1 = f1 - __uint_as_float(hb & 0xffff0000u);
        h[k] = hb;
        l[k] = pack_bf16x2(r0, r1);
    }
    *(u32x4*)(hi_plane + e0) = h;
    *(u32x4*)(lo_plane + e0) = l;
}

// float32 rows -> bf16 planes (hi, lo), 8 elements per thread (d % 8 == 0)
__global__ __launch_bounds__(256) void k_split_rows(const float* __restrict__ W,
                                                   uint16_t* __restrict__ hi_plane,
                                                   uint16_t* __restrict__ lo_plane,
                                                   int64_t total8) {
    const int64_t idx8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx8 >= total8) return;
    const int64_t e0 = idx8 * 8;
    const float4* src = (const float4*)(W + e0);
    float4 x0 = src[0], x1 = src[1];
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    u32x4 h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t hb = pack_bf16x2(v[2 * k], v[2 * k + 1]);
        h[k] = hb;
        l[k] = pack_bf16x2(v[2 * k] - __uint_as_float(hb << 16),
                           v[2 * k + 1] - __uint_as_float(hb & 0xffff0000u));
    }
    *(u32x4*)(hi_plane + e0) = h;
    *(u32x4*)(lo_plane + e0) = l;
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

// ---------------------------------------------------------------------------
// k_fgemm: out[g][n][a] (=|+=) sum_i A[n][i] * F'_g[i][a]   (F' symmetric: F'[i][a]
// is read as row a of the plane).  A is either a bf16 matrix (rows of W or of a
// bf16 plane of W) or the one-hot expansion of the codes: row n = j*m + q is
// [P[j][i] == q].  Block tile 256 (n) x 256 (a), 4 waves of 128 x 128 = 4x4 MFMA
// 32x32x16 tiles, K staged 32 at a time through LDS (pitch 40 = conflict-free).
// ---------------------------------------------------------------------------
constexpr int GT = 256;
constexpr int GKC = 32;
constexpr int GPITCH = 40;
constexpr int G_PLANE = GT * GPITCH;         // bf16 elements per staged 256x32 operand

template <bool ONEHOT, int NPB>
__global__ __launch_bounds__(256, 1) void k_fgemm(
    const uint16_t* __restrict__ Abf,  // bf16 rows [rows_total][d] (ONEHOT=false)
    const uint8_t* __restrict__ codes, // [rows_total][d] (ONEHOT=true)
    int m, int64_t rows_per_group, int g_first,
    const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo, int64_t d,
    int n_tiles_n, int n_tiles_a, int accumulate, float* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) uint16_t fgemm_lds[];
    // per stage: A plane (or codes) + NPB F' planes
    constexpr int STAGE = G_PLANE * (1 + NPB);
    auto stage_base = [&](int b) { return fgemm_lds + b * STAGE; };

    const int bid = blockIdx.x;
    const int tn = bid % n_tiles_n;
    const int ta = (bid / n_tiles_n) % n_tiles_a;
    const int gl = bid / (n_tiles_n * n_tiles_a);     // group within this launch
    const int g = g_first + gl;
    const int64_t N = ONEHOT ? rows_per_group * m : rows_per_group;
    const int64_t n0 = (int64_t)tn * GT, a0 = (int64_t)ta * GT;
    const int64_t row_base = (int64_t)g * rows_per_group;   // first W/code row of group
    const uint16_t* Fh = Fhi + (size_t)g * d * d;
    const uint16_t* Fl = (NPB > 1) ? Flo + (size_t)g * d * d : nullptr;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wa = wave >> 1;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // staging map: 256 rows x 4 quads of 8 elements; thread covers rows r0 + 64*s
    const int sr = tid >> 2, sq = tid & 3;
    u32x4 pa[4], pf[NPB][4];
    u32x4 pc = {0u, 0u, 0u, 0u};  // ONEHOT: 16 codes of one j-row
    const int jrows = ONEHOT ? GT / m : 0;   // distinct j-rows in an n tile

    auto fetch = [&](int64_t k0) {
        const int64_t kk = k0 + 8 * sq;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = sr + 64 * s;
            const int64_t arow = a0 + r;
#pragma unroll
            for (int p = 0; p < NPB; ++p) {
                const uint16_t* base = (p == 0) ? Fh : Fl;
                pf[p][s] = (arow < d && kk < d) ? *(const u32x4*)(base + arow * d + kk)
                                                : u32x4{0u, 0u, 0u, 0u};
            }
            if constexpr (!ONEHOT) {
                const int64_t nrow = n0 + r;
                pa[s] = (nrow < N && kk < d) ? *(const u32x4*)(Abf + (row_base + nrow) * d + kk)
                                             : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if constexpr (ONEHOT) {
            // jrows (<= 128) rows x 32 codes: thread covers row tid/2, bytes 16*(tid%2)
            const int r = tid >> 1;
            const int64_t jl = n0 / m + r;
            const int64_t kc = k0 + 16 * (tid & 1);
            if (r < jrows && jl < rows_per_group && kc < d) {
                pc = *(const u32x4*)(codes + (row_base + jl) * d + kc);
            } else {
                pc = u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};  // matches no code
            }
        }
    };
    auto stage = [&](int buf) {
        uint16_t* S = stage_base(buf);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = sr + 64 * s;
#pragma unroll
            for (int p = 0; p < NPB; ++p)
                *(u32x4*)(S + G_PLANE * (1 + p) + r * GPITCH + 8 * sq) = pf[p][s];
            if constexpr (!ONEHOT) *(u32x4*)(S + r * GPITCH + 8 * sq) = pa[s];
        }
        if constexpr (ONEHOT) {
            uint8_t* cs = (uint8_t*)S;
            *(u32x4*)(cs + (tid >> 1) * 32 + 16 * (tid & 1)) = pc;
        }
    };

    const int nk = (int)((d + GKC - 1) / GKC);
    fetch(0);
    stage(0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        const bool more = kc + 1 < nk;
        if (more) fetch((int64_t)(kc + 1) * GKC);
        const uint16_t* S = stage_base(buf);
#pragma unroll 1
        for (int ks = 0; ks < GKC / 16; ++ks) {
            const int koff = ks * 16 + 8 * (lane >> 5);
            bf16x8 af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int nl = 128 * wn + 32 * i + (lane & 31);
                if constexpr (ONEHOT) {
                    const int jr = nl / m, q = nl - jr * m;
                    const u32x2 cv = *(const u32x2*)((const uint8_t*)S + jr * 32 + koff);
                    u32x4 o;
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t word = cv[h >> 1];
                        const uint32_t b0 = (word >> (16 * (h & 1))) & 0xffu;
                        const uint32_t b1 = (word >> (16 * (h & 1) + 8)) & 0xffu;
                        o[h] = ((b0 == (uint32_t)q) ? 0x3F80u : 0u) |
                               ((b1 == (uint32_t)q) ? 0x3F800000u : 0u);
                    }
                    af[i] = as_bf16x8(o);
                } else {
                    af[i] = as_bf16x8(*(const u32x4*)(S + nl * GPITCH + koff));
                }
            }
#pragma unroll
            for (int p = 0; p < NPB; ++p) {
                bf16x8 bfr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bfr[j] = as_bf16x8(*(const u32x4*)(S + G_PLANE * (1 + p) +
                                                       (128 * wa + 32 * j + (lane & 31)) * GPITCH + koff));
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        }
        if (more) stage(buf ^ 1);
        __syncthreads();
    }

    float* O = out + (size_t)gl * N * d + (size_t)n0 * d + a0;
    const int nrem = (int)((N - n0) < GT ? (N - n0) : GT);
    const int arem = (int)((d - a0) < GT ? (d - a0) : GT);
    const int di = (int)d;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int acol = 128 * wa + 32 * j + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int nrow = 128 * wn + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (nrow < nrem && acol < arem) {
                    float* dst = O + (size_t)(nrow * di) + acol;
                    float x = acc[i][j][v];
                    if (accumulate) x += *dst;
                    *dst = x;
                }
            }
        }
}

// ---------------------------------------------------------------------------
// k_solve: one wave per row (4 rows per block).
//   MODE 0 (SOLVE): codebook step on the non-empty codes, then r = U c_new - v
//   MODE 1 (RESID): keep c, r = U c - v
// Writes R[j] (if R != null), obj_old[j] = e_old . r_old, obj_new[j] = e_new . r_new.
// U holds the rows of the current group chunk: U[(j - j_first) * m + q][a].
// ---------------------------------------------------------------------------
template <bool BF16, int MODE>
__global__ __launch_bounds__(256) void k_solve(
    const float* __restrict__ U, int64_t j_first, int64_t j_count, const float* __restrict__ V,
    const uint8_t* __restrict__ P, const void* __restrict__ W, float* __restrict__ C, int m,
    int64_t d, float* __restrict__ R, double* __restrict__ obj_old, double* __restrict__ obj_new,
    unsigned long long* __restrict__ n_not_pd) {
    __shared__ double sA[4][MAX_M][MAX_M];
    __shared__ double sL[4][MAX_M][MAX_M];
    __shared__ double sb[4][MAX_M];
    __shared__ double sy[4][MAX_M];
    __shared__ int scnt[4][MAX_M];
    __shared__ int sidx[4][MAX_M];
    __shared__ float sc_old[4][MAX_M];
    __shared__ float sc_new[4][MAX_M];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t jl = (int64_t)blockIdx.x * 4 + wave;
    const bool valid = jl < j_count;
    const int64_t j = j_first + (valid ? jl : 0);
    const float* Uj = U + (size_t)(valid ? jl : 0) * m * d;
    const float* vj = V + (size_t)j * d;
    const uint8_t* pj = P + (size_t)j * d;

    if (lane < m) sc_old[wave][lane] = valid ? C[j * m + lane] : 0.f;
    if (MODE == 0 && valid) {
        // b = P^T v and the code counts
        float bacc[MAX_M];
        int cnt[MAX_M];
#pragma unroll
        for (int k = 0; k < MAX_M; ++k) { bacc[k] = 0.f; cnt[k] = 0; }
        for (int64_t a = lane; a < d; a += 64) {
            const int code = pj[a];
            const float v = vj[a];
#pragma unroll
            for (int k = 0; k < MAX_M; ++k) {
                bacc[k] += (code == k) ? v : 0.f;
                cnt[k] += (code == k) ? 1 : 0;
            }
        }
#pragma unroll
        for (int k = 0; k < MAX_M; ++k) {
            if (k < m) {
                const double sum = wave_sum_f64((double)bacc[k]);
                int c = cnt[k];
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
                if (lane == 0) { sb[wave][k] = sum; scnt[wave][k] = c; }
            }
        }
        // A[:, q] = P^T U[:, q]
        for (int q = 0; q < m; ++q) {
            float aacc[MAX_M];
#pragma unroll
            for (int k = 0; k < MAX_M; ++k) aacc[k] = 0.f;
            const float* Uq = Uj + (size_t)q * d;
            for (int64_t a = lane; a < d; a += 64) {
                const int code = pj[a];
                const float u = Uq[a];
#pragma unroll
                for (int k = 0; k < MAX_M; ++k) aacc[k] += (code == k) ? u : 0.f;
            }
#pragma unroll
            for (int k = 0; k < MAX_M; ++k) {
                if (k < m) {
                    const double sum = wave_sum_f64((double)aacc[k]);
                    if (lane == 0) sA[wave][k][q] = sum;
                }
            }
        }
    }
    __syncthreads();
    if (MODE == 0 && valid && lane == 0) {
        // float64 Cholesky of the symmetric part of A on the non-empty codes
        int ns = 0;
        for (int k = 0; k < m; ++k)
            if (scnt[wave][k] > 0) sidx[wave][ns++] = k;
        bool ok = true;
        for (int r = 0; r < ns && ok; ++r) {
            for (int c = 0; c <= r; ++c) {
                const int ir = sidx[wave][r], ic = sidx[wave][c];
                double sum = 0.5 * (sA[wave][ir][ic] + sA[wave][ic][ir]);
                for (int k = 0; k < c; ++k) sum -= sL[wave][r][k] * sL[wave][c][k];
                if (r == c) {
                    if (!(sum > 0.0)) { ok = false; break; }
                    sL[wave][r][r] = sqrt(sum);
                } else {
                    sL[wave][r][c] = sum / sL[wave][c][c];
                }
            }
        }
        for (int k = 0; k < m; ++k) sc_new[wave][k] = sc_old[wave][k];
        if (ok) {
            for (int r = 0; r < ns; ++r) {
                double sum = sb[wave][sidx[wave][r]];
                for (int k = 0; k < r; ++k) sum -= sL[wave][r][k] * sy[wave][k];
                sy[wave][r] = sum / sL[wave][r][r];
            }
            for (int r = ns - 1; r >= 0; --r) {
                double sum = sy[wave][r];
                for (int k = r + 1; k < ns; ++k) sum -= sL[wave][k][r] * sy[wave][k];
                sy[wave][r] = sum / sL[wave][r][r];     // x overwrites y from the back
            }
            for (int r = 0; r < ns; ++r) sc_new[wave][sidx[wave][r]] = (float)sy[wave][r];
        } else if (n_not_pd) {
            atomicAdd(n_not_pd, 1ull);
        }
    }
    if (MODE == 1 && lane < m) sc_new[wave][lane] = sc_old[wave][lane];
    __syncthreads();
    if (!valid) return;
    if (MODE == 0 && lane < m) C[j * m + lane] = sc_new[wave][lane];

    double o_old = 0.0, o_new = 0.0;
    float cn[MAX_M], co[MAX_M];
#pragma unroll
    for (int k = 0; k < MAX_M; ++k) {
        cn[k] = (k < m) ? sc_new[wave][k] : 0.f;
        co[k] = (k < m) ? sc_old[wave][k] : 0.f;
    }
    for (int64_t a = lane; a < d; a += 64) {
        float rn = 0.f, ro = 0.f;
#pragma unroll
        for (int k = 0; k < MAX_M; ++k) {
            if (k < m) {
                const float u = Uj[(size_t)k * d + a];
                rn = fmaf(cn[k], u, rn);
                ro = fmaf(co[k], u, ro);
            }
        }
        const float v = vj[a];
        rn -= v;
        ro -= v;
        const int code = pj[a];
        const double w = (double)load_elem<BF16>(W, j * d + a);
        const double en = (double)sc_new[wave][code] - w;
        const double eo = (double)sc_old[wave][code] - w;
        o_new += en * (double)rn;
        o_old += eo * (double)ro;
        if (R) R[j * d + a] = rn;
    }
    o_new = wave_sum_f64(o_new);
    o_old = wave_sum_f64(o_old);
    if (lane == 0) {
        if (obj_new) obj_new[j] = o_new;
        if (obj_old) obj_old[j] = o_old;
    }
}

// ---------------------------------------------------------------------------
// k_sweep: the assignment pass.  One block = 16 rows of one group, one row per
// wave (16 waves).  Coordinates are visited in ascending order in sub-blocks of
// 64, one coordinate per lane.
//   * Deferred update: once per B-block, the effect of every earlier move of
//     this pass on the block's residuals is gathered left-looking on the matrix
//     cores, corr = D[rows, 0:bB] F'[0:bB, B-block] with v_mfma_f32_16x16x32_bf16
//     and three products of the bf16 hi/lo planes (D hi.F hi + D hi.F lo +
//     D lo.F hi); 16 waves split it into NCT column tiles x NSL k-slices whose
//     partials are summed in a fixed order.  32-coordinate chunks in which no
//     row of the block moved are skipped.  Inside a B-block, each later 64-wide
//     sub-block gets the same correction from the block's earlier sub-blocks.
//   * Chain (per wave, per sub-block): for coordinate t the residual, current
//     value and damped diagonal are read from lane t (v_readlane); lanes
//     0..m-1 each evaluate one candidate change
//         Delta_q = delta_q (F'_tt delta_q + 2 r_t),  delta_q = c_q - w_hat_t,
//     a 16-lane DPP min gives the best change, a ballot + find-first-set gives
//     the lowest index attaining it, and a strict decrease applies
//     r += delta F'[t, sub-block] in registers (F' column of the sub-block held
//     in 64 registers per lane, staged once through LDS for the 16 rows).
//   * The codes and the value changes (bf16 hi + lo) are written back.
// ---------------------------------------------------------------------------
constexpr int SW_ROWS = 16;     // rows (= waves) per block
constexpr int SW_SUB = 64;      // chain sub-block (one coordinate per lane)
constexpr int SW_PF = 2;        // k-chunks in flight per wave in the deferred update
constexpr int SW_SEG = 8;       // chain steps unrolled per F' column preload

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

// acc += D[arow, kk..kk+7] . F'[ncol, kk..kk+7] over the 32-wide k-chunks
// k_first, k_first + kstride, ... < k_end; chunks whose flag is 0 are skipped
// (the flag is block-uniform).  Rows past the group's end read a valid row's D:
// their outputs are never used.
__device__ __forceinline__ void sweep_corr(f32x4& acc, const uint16_t* __restrict__ Dh,
                                           const uint16_t* __restrict__ Dl,
                                           const uint16_t* __restrict__ Fh,
                                           const uint16_t* __restrict__ Fl,
                                           int64_t k_first, int64_t k_end, int64_t kstride,
                                           const uint32_t* flags, int lane) {
    const int ko = 8 * (lane >> 4);
    for (int64_t k0 = k_first; k0 < k_end; k0 += SW_PF * kstride) {
        u32x4 dh[SW_PF], dl[SW_PF], fh[SW_PF], fl[SW_PF];
        bool on[SW_PF];
#pragma unroll
        for (int u = 0; u < SW_PF; ++u) {
            const int64_t kc = k0 + u * kstride;
            on[u] = kc < k_end && __builtin_amdgcn_readfirstlane((int)flags[kc >> 5]) != 0;
            if (on[u]) {
                dh[u] = *(const u32x4*)(Dh + kc + ko);
                dl[u] = *(const u32x4*)(Dl + kc + ko);
                fh[u] = *(const u32x4*)(Fh + kc + ko);
                fl[u] = *(const u32x4*)(Fl + kc + ko);
            }
        }
#pragma unroll
        for (int u = 0; u < SW_PF; ++u) {
            if (on[u]) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh[u]), as_bf16x8(fh[u]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dh[u]), as_bf16x8(fl[u]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(dl[u]), as_bf16x8(fh[u]), acc, 0, 0, 0);
            }
        }
    }
}

template <int B>
__global__ __launch_bounds__(1024, 1) void k_sweep(
    const float* __restrict__ F, const float* __restrict__ dF,
    const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo,
    int64_t d, int64_t rows_per_group, int wgs_per_group, int total_wgs,
    const float* __restrict__ C, int m, uint8_t* __restrict__ P,
    const float* __restrict__ R, uint16_t* __restrict__ Dhi, uint16_t* __restrict__ Dlo,
    const double* __restrict__ obj_in, double* __restrict__ obj_out,
    unsigned long long* __restrict__ n_changed) {
    constexpr int NCT = B / 16;          // 16-column tiles of a B-block
    constexpr int NSL = 256 / B;         // k-slices of the B-block correction
    constexpr int NSUB = B / SW_SUB;     // 64-wide sub-blocks per B-block
    __shared__ float corr_b[NSL][SW_ROWS][B];          // 16 KB
    __shared__ float corr_s[4][SW_ROWS][SW_SUB];       // 16 KB
    __shared__ __attribute__((aligned(16))) float fdb[SW_SUB][SW_SUB];   // 16 KB
    __shared__ float fdd[SW_SUB];                      // diag(F') of the sub-block
    extern __shared__ uint32_t sweep_flags[];          // [d / 32]

    // XCD-aware order: hardware block h runs on XCD h % 8; consecutive logical
    // blocks (the rows of one group) go to the same XCD and share F' in its L2.
    const int nb = gridDim.x;
    const int hw = blockIdx.x;
    const int lin = (hw & 7) * (nb >> 3) + (hw >> 3);
    if (lin >= total_wgs) return;        // whole block exits together

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lin / wgs_per_group;
    const int64_t local = (int64_t)(lin % wgs_per_group) * SW_ROWS;
    const int64_t jl = local + wave;
    const bool rvalid = jl < rows_per_group;
    const int64_t j = (int64_t)g * rows_per_group + (rvalid ? jl : 0);

    const float* Fg = F + (size_t)g * d * d;
    const float* dFg = dF + (size_t)g * d;
    const uint16_t* Fh = Fhi + (size_t)g * d * d;
    const uint16_t* Fl = Flo + (size_t)g * d * d;

    for (int i = tid; i < (int)(d / 32); i += 1024) sweep_flags[i] = 0u;

    const float cl = (lane < m && rvalid) ? C[j * m + lane] : 0.f;   // candidate of this lane
    double dsum = 0.0;
    unsigned moves = 0;

    // operand rows of the correction products: the block's 16 rows
    const int64_t arow_l = local + (lane & 15);
    const bool arow_ok = arow_l < rows_per_group;
    const int64_t arow = (int64_t)g * rows_per_group + (arow_ok ? arow_l : 0);
    const uint16_t* Dh_row = Dhi + arow * d;
    const uint16_t* Dl_row = Dlo + arow * d;
    __syncthreads();

    for (int64_t bB = 0; bB < d; bB += B) {
        // ---- deferred update of the B-block from all earlier B-blocks
        {
            const int ct = wave % NCT, sl = wave / NCT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int64_t ncol = bB + ct * 16 + (lane & 15);
            sweep_corr(acc, Dh_row, Dl_row, Fh + ncol * d, Fl + ncol * d, (int64_t)sl * 32, bB,
                       (int64_t)32 * NSL, sweep_flags, lane);
#pragma unroll
            for (int t = 0; t < 4; ++t) corr_b[sl][4 * (lane >> 4) + t][ct * 16 + (lane & 15)] = acc[t];
        }
        for (int s = 0; s < NSUB; ++s) {
            const int64_t bs = bB + (int64_t)s * SW_SUB;
            // stage the diagonal 64 x 64 block of F (rows bs.., columns bs..)
            {
                const int rr = tid >> 4, cc = (tid & 15) * 4;
                *(float4*)&fdb[rr][cc] = *(const float4*)(Fg + (bs + rr) * d + bs + cc);
                if (tid < SW_SUB) fdd[tid] = dFg[bs + tid];
            }
            // in-block correction from this B-block's earlier sub-blocks
            if (s > 0) {
                const int ct = wave & 3, sl = wave >> 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int64_t ncol = bs + ct * 16 + (lane & 15);
                sweep_corr(acc, Dh_row, Dl_row, Fh + ncol * d, Fl + ncol * d,
                           bB + (int64_t)sl * 32, bs, 128, sweep_flags, lane);
#pragma unroll
                for (int t = 0; t < 4; ++t) corr_s[sl][4 * (lane >> 4) + t][ct * 16 + (lane & 15)] = acc[t];
            }
            __syncthreads();

            if (rvalid) {
                const int64_t col = bs + lane;
                float r = R[j * d + col];
#pragma unroll
                for (int k = 0; k < NSL; ++k) r += corr_b[k][wave][s * SW_SUB + lane];
                if (s > 0) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) r += corr_s[k][wave][lane];
                }
                int code = P[j * d + col];
                float wh = __shfl(cl, code, 64);
                const float wh0 = wh;
                const bool cand = lane < m;
                const float fdiag = fdd[lane];            // F'[col][col]
                for (int t0 = 0; t0 < SW_SUB; t0 += SW_SEG) {
                    float fc[SW_SEG];                     // F[bs + t][bs + lane], t = t0..
#pragma unroll
                    for (int u = 0; u < SW_SEG; ++u) fc[u] = fdb[t0 + u][lane];
#pragma unroll
                    for (int u = 0; u < SW_SEG; ++u) {
                        const int t = t0 + u;
                        const float ft = readlane_f(fdiag, t);
                        const float rt = readlane_f(r, t);
                        const float wt = readlane_f(wh, t);
                        const float dl = cl - wt;
                        const float dq = dl * fmaf(ft, dl, 2.f * rt);
                        const int key = cand ? f32_order_key(dq) : 0x7fffffff;
                        const int bk = __builtin_amdgcn_readlane(row16_min_i(key), 0);
                        if (bk < -1) {                    // a strictly negative change exists
                            const int q = __ffsll((long long)__ballot(key == bk)) - 1;
                            const float cq = readlane_f(cl, q);
                            const float delta = cq - wt;
                            r = fmaf(delta, fc[u], r);
                            if (lane == __builtin_amdgcn_readfirstlane(t)) {
                                code = q;
                                wh = cq;
                            }
                            dsum += (double)readlane_f(dq, q);
                            moves += 1;
                        }
                    }
                }
                P[j * d + col] = (uint8_t)code;
                const float dv = wh - wh0;
                const uint32_t hb = f32_to_bf16_bits(dv);
                Dhi[j * d + col] = (uint16_t)hb;
                Dlo[j * d + col] = (uint16_t)f32_to_bf16_bits(dv - __uint_as_float(hb << 16));
                const unsigned long long moved = __ballot(dv != 0.f);
                if (lane == 0) {
                    if (moved & 0xffffffffull) sweep_flags[bs >> 5] = 1u;
                    if (moved >> 32) sweep_flags[(bs >> 5) + 1] = 1u;
                }
            }
            __syncthreads();
        }
    }
    if (rvalid && lane == 0) {
        obj_out[j] = obj_in[j] + dsum;
        if (n_changed) atomicAdd(n_changed, (unsigned long long)moves);
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

__global__ void k_zero_u64(unsigned long long* __restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

}  // namespace gq

// ===========================================================================
// Host launchers
// ===========================================================================
#include "gq_internal.h"

namespace gq {

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

LnqSizes lnq_sizes(int64_t d_out, int64_t d, int groups, int m, bool w_f32) {
    LnqSizes z{};
    const int64_t rpg = d_out / groups;
    const size_t u_group = (size_t)rpg * m * d * sizeof(float);
    const size_t u_budget = (size_t)4 << 30;
    int gchunk = (int)(u_budget / (u_group ? u_group : 1));
    if (gchunk < 1) gchunk = 1;
    if (gchunk > groups) gchunk = groups;
    z.gchunk = gchunk;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    z.o_fhi = take((size_t)groups * d * d * 2);
    z.o_flo = take((size_t)groups * d * d * 2);
    z.o_dF = take((size_t)groups * d * 4);
    z.o_lam = take((size_t)groups * 8);
    z.o_V = take((size_t)d_out * d * 4);
    z.o_U = take(u_group * gchunk);
    z.o_R = take((size_t)d_out * d * 4);
    z.o_dhi = take((size_t)d_out * d * 2);
    z.o_dlo = take((size_t)d_out * d * 2);
    z.o_whi = w_f32 ? take((size_t)d_out * d * 2) : 0;
    z.o_wlo = w_f32 ? take((size_t)d_out * d * 2) : 0;
    z.o_objA = take((size_t)d_out * 8);
    z.o_objB = take((size_t)d_out * 8);
    z.o_objC = take((size_t)d_out * 8);
    z.o_cnt = take(16 * 8);
    z.total = off;
    return z;
}

LnqWs lnq_carve(void* base, const LnqSizes& z, bool w_f32) {
    char* b = (char*)base;
    LnqWs w{};
    w.fhi = (uint16_t*)(b + z.o_fhi);
    w.flo = (uint16_t*)(b + z.o_flo);
    w.dF = (float*)(b + z.o_dF);
    w.lam = (double*)(b + z.o_lam);
    w.V = (float*)(b + z.o_V);
    w.U = (float*)(b + z.o_U);
    w.R = (float*)(b + z.o_R);
    w.dhi = (uint16_t*)(b + z.o_dhi);
    w.dlo = (uint16_t*)(b + z.o_dlo);
    w.whi = w_f32 ? (uint16_t*)(b + z.o_whi) : nullptr;
    w.wlo = w_f32 ? (uint16_t*)(b + z.o_wlo) : nullptr;
    w.objA = (double*)(b + z.o_objA);
    w.objB = (double*)(b + z.o_objB);
    w.objC = (double*)(b + z.o_objC);
    w.cnt = (unsigned long long*)(b + z.o_cnt);
    w.gchunk = z.gchunk;
    return w;
}

hipError_t lnq_prepare(const float* F, int groups, int64_t d, double rho, const LnqWs& w,
                       hipStream_t st) {
    StageTimer tm(ST_LNQ_PREPARE, st);
    hipLaunchKernelGGL(k_ridge, dim3(groups), dim3(256), 0, st, F, d, rho, w.lam);
    GQ_LAUNCH_CHECK();
    const int64_t total8 = (int64_t)groups * d * d / 8;
    hipLaunchKernelGGL(k_split, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, st, F, d,
                       w.lam, w.fhi, w.flo, w.dF, total8);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

template <bool ONEHOT, int NPB>
static hipError_t launch_fgemm(const uint16_t* A, const uint8_t* codes, int m, int64_t rpg,
                               int g_first, int g_count, const LnqWs& w, int64_t d,
                               int accumulate, float* out, hipStream_t st) {
    const int64_t N = ONEHOT ? rpg * m : rpg;
    const int ntn = (int)((N + GT - 1) / GT);
    const int nta = (int)((d + GT - 1) / GT);
    const size_t lds = (size_t)2 * G_PLANE * (1 + NPB) * sizeof(uint16_t);
    hipError_t e = hipFuncSetAttribute((const void*)k_fgemm<ONEHOT, NPB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const unsigned nblocks = (unsigned)ntn * nta * g_count;
    StageTimer tm(ONEHOT ? ST_LNQ_U : ST_LNQ_WF, st);
    hipLaunchKernelGGL((k_fgemm<ONEHOT, NPB>), dim3(nblocks), dim3(256), lds, st, A, codes, m,
                       rpg, g_first, w.fhi, w.flo, d, ntn, nta, accumulate, out);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_compute_v(const void* W, bool w_bf16, int64_t d_out, int64_t d, int groups,
                         const LnqWs& w, hipStream_t st) {
    const int64_t rpg = d_out / groups;
    if (w_bf16) {
        return launch_fgemm<false, 2>((const uint16_t*)W, nullptr, 1, rpg, 0, groups, w, d, 0,
                                      w.V, st);
    }
    const int64_t total8 = d_out * d / 8;
    StageTimer tm(ST_LNQ_WF, st);
    hipLaunchKernelGGL(k_split_rows, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, st,
                       (const float*)W, w.whi, w.wlo, total8);
    GQ_LAUNCH_CHECK();
    hipError_t e = launch_fgemm<false, 2>(w.whi, nullptr, 1, rpg, 0, groups, w, d, 0, w.V, st);
    if (e != hipSuccess) return e;
    return launch_fgemm<false, 1>(w.wlo, nullptr, 1, rpg, 0, groups, w, d, 1, w.V, st);
}

hipError_t lnq_init_run(const void* W, bool w_bf16, int64_t d_out, int64_t d, int m, float* C,
                        uint8_t* P, hipStream_t st) {
    int npow2 = 1;
    while (npow2 < d) npow2 <<= 1;
    const size_t lds = (size_t)npow2 * sizeof(float);
    StageTimer tm(ST_LNQ_INIT, st);
    if (w_bf16) {
        hipError_t e = hipFuncSetAttribute((const void*)k_lnq_init<true>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_lnq_init<true>, dim3((unsigned)d_out), dim3(1024), lds, st, W, d,
                           npow2, m, C, P);
    } else {
        hipError_t e = hipFuncSetAttribute((const void*)k_lnq_init<false>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_lnq_init<false>, dim3((unsigned)d_out), dim3(1024), lds, st, W, d,
                           npow2, m, C, P);
    }
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_u_solve(int mode, const void* W, bool w_bf16, int64_t d_out, int64_t d,
                       int groups, int m, const uint8_t* P, float* C, const LnqWs& w, float* R,
                       double* obj_old, double* obj_new, unsigned long long* n_not_pd,
                       hipStream_t st) {
    const int64_t rpg = d_out / groups;
    for (int g0 = 0; g0 < groups; g0 += w.gchunk) {
        const int gc = (g0 + w.gchunk <= groups) ? w.gchunk : groups - g0;
        hipError_t e = launch_fgemm<true, 2>(nullptr, P, m, rpg, g0, gc, w, d, 0, w.U, st);
        if (e != hipSuccess) return e;
        const int64_t jf = (int64_t)g0 * rpg, jc = (int64_t)gc * rpg;
        const dim3 grid((unsigned)((jc + 3) / 4));
        StageTimer tm(ST_LNQ_SOLVE, st);
        if (w_bf16) {
            if (mode == 0)
                hipLaunchKernelGGL((k_solve<true, 0>), grid, dim3(256), 0, st, w.U, jf, jc, w.V, P,
                                   W, C, m, d, R, obj_old, obj_new, n_not_pd);
            else
                hipLaunchKernelGGL((k_solve<true, 1>), grid, dim3(256), 0, st, w.U, jf, jc, w.V, P,
                                   W, C, m, d, R, obj_old, obj_new, n_not_pd);
        } else {
            if (mode == 0)
                hipLaunchKernelGGL((k_solve<false, 0>), grid, dim3(256), 0, st, w.U, jf, jc, w.V,
                                   P, W, C, m, d, R, obj_old, obj_new, n_not_pd);
            else
                hipLaunchKernelGGL((k_solve<false, 1>), grid, dim3(256), 0, st, w.U, jf, jc, w.V,
                                   P, W, C, m, d, R, obj_old, obj_new, n_not_pd);
        }
        GQ_LAUNCH_CHECK();
    }
    return hipSuccess;
}

template <int B>
static hipError_t launch_sweep(const float* F, int64_t d_out, int64_t d, int groups,
                               const float* C, int m, uint8_t* P, const LnqWs& w,
                               const double* obj_in, double* obj_out,
                               unsigned long long* counter, hipStream_t st) {
    const int64_t rpg = d_out / groups;
    const int wgs = (int)((rpg + SW_ROWS - 1) / SW_ROWS);
    const int total = wgs * groups;
    const int grid = (total + 7) / 8 * 8;          // the XCD remap needs a multiple of 8
    const size_t lds = (size_t)(d / 32) * sizeof(uint32_t);
    StageTimer tm(ST_LNQ_SWEEP, st);
    hipLaunchKernelGGL(k_sweep<B>, dim3((unsigned)grid), dim3(1024), lds, st, F, w.dF, w.fhi,
                       w.flo, d, rpg, wgs, total, C, m, P, w.R, w.dhi, w.dlo, obj_in, obj_out,
                       counter);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_sweep_run(int block, const float* F, int64_t d_out, int64_t d, int groups,
                         const float* C, int m, uint8_t* P, const LnqWs& w,
                         const double* obj_in, double* obj_out, unsigned long long* counter,
                         hipStream_t st) {
    switch (block) {
        case 64: return launch_sweep<64>(F, d_out, d, groups, C, m, P, w, obj_in, obj_out, counter, st);
        case 128: return launch_sweep<128>(F, d_out, d, groups, C, m, P, w, obj_in, obj_out, counter, st);
        case 256: return launch_sweep<256>(F, d_out, d, groups, C, m, P, w, obj_in, obj_out, counter, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t lnq_reduce(const double* rows, int64_t n, double* out, hipStream_t st) {
    StageTimer tm(ST_LNQ_SMALL, st);
    hipLaunchKernelGGL(k_reduce_rows, dim3(1), dim3(256), 0, st, rows, n, out);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_zero_counter(unsigned long long* c, hipStream_t st) {
    StageTimer tm(ST_LNQ_SMALL, st);
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, st, c, 1);
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
