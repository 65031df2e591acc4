// GANQ-style assignment on gfx950: back-substitution over the Cholesky factor of F'.
//
// GANQ summary page (atlas.scime.ai, "GANQ: GPU-Adaptive Non-Uniform Quantization"),
// "Approach": per row, alternating updates of a closed-form least-squares codebook and
// an assignment of the indices by Cholesky / back-substitution.  With F' = L L^T the
// row objective is ||L^T e||^2 (e = w_hat - w), whose j-th term
// (L^T e)_j = L_jj e_j + s_j,  s_j = sum_{k>j} L_kj e_k,
// involves coordinates j..d-1 only.  The assignment visits j = d-1 down to 0 and gives
// coordinate j the codebook entry nearest to w_j - s_j / L_jj.
//
// Work split on the GPU
//   k_chol_init    A = F + lambda I as float64 (lower triangle), per group
//   k_chol_diag    one 64 x 64 diagonal block: unblocked Cholesky in LDS, its inverse
//   k_chol_panel   the panel below it: L21 = A21 L11^{-T}
//   k_chol_update  trailing lower triangle: A22 -= L21 L21^T (float64 FMAs, 64 x 64 tiles)
//   k_ganq_prep    U = L^T as k-blocked bfloat16 planes (hi + lo) for the matrix cores,
//                  diag(L) in float32
//   k_ganq         the pass: 16 rows per block, coordinates from the last to the first
//                  in 64-blocks grouped into super-blocks of 512:
//                    * s from later super-blocks: a running array S, updated at the end
//                      of each super-block for all earlier coordinates on the matrix
//                      cores, S[:, :sb] += E_sb U[:sb, sb]^T (three bf16 products);
//                    * s from later 64-blocks of the same super-block: the same product
//                      before each block;
//                    * inside a block, 64 dependent steps: lane t takes its entry (a
//                      binary search over the midpoints of the sorted codebook), and
//                      every lane i < t adds L[t][i] e_t (the block of L staged in LDS).
#include "gq_common.h"
#include "gq_internal.h"

#include <utility>

namespace gq {

constexpr int CB = 64;                 // panel width of the factorization

// ---------------------------------------------------------------------------
// Cholesky of F' = F + lambda I (float64), in place in A [groups][d][d] (lower)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_chol_init(const float* __restrict__ F,
                                                  const double* __restrict__ lam, int64_t d,
                                                  double* __restrict__ A,
                                                  int* __restrict__ bad) {
    const int g = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e == 0) bad[g] = 0;
    if (e >= d * d) return;
    const int64_t i = e / d, j = e - i * d;
    const float* Fg = F + (size_t)g * d * d;
    A[(size_t)g * d * d + e] = (j <= i) ? (double)Fg[e] + (i == j ? lam[g] : 0.0) : 0.0;
}

// v from the lane given by a quad permutation (all four lanes of a quad active)
template <int CTRL>
__device__ __forceinline__ double quad_dpp_f64(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// One block per group factors diagonal block p and writes L_pp (lower) back to A and
// its inverse to Linv [groups][64][64].  Thread (ti, tj) of a 16 x 16 grid keeps
// a[ti + 16 u][tj + 16 v] (u, v < 4) in registers; at step c the owner of (c, c) takes
// the pivot, the owners of column c scale it by 1 / L_cc and publish it in LDS, and
// every thread updates its elements with c < j <= i.  A pivot that is not positive (F'
// singular, e.g. a group whose gradients vanish) marks the group in `bad` and is replaced
// by 1 so the rest of the factorization stays finite; a marked group's codes are left as
// they are.
__global__ __launch_bounds__(256) void k_chol_diag(double* __restrict__ A, int64_t d, int p,
                                                  double* __restrict__ Linv,
                                                  int* __restrict__ bad) {
    __shared__ double a[CB][CB + 1];
    __shared__ double x[CB][CB + 1];
    __shared__ double col[CB];            // column c of L below the diagonal, at step c
    __shared__ double rpiv[CB];           // 1 / L_cc
    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    double* Ag = A + (size_t)g * d * d;
    const int64_t o = (int64_t)p * CB;
    const int ti = tid >> 4, tj = tid & 15;
    if (tid < CB) col[tid] = 0.0;         // finite before any step reads it
    double r[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = ti + 16 * u, j = tj + 16 * v;
            r[u][v] = (j <= i) ? Ag[(o + i) * d + o + j] : 0.0;
        }
    for (int c = 0; c < CB; ++c) {
        const int cu = c >> 4, cr = c & 15;
        if (ti == cr && tj == cr) {
            double pv = r[cu][cu];
            if (!(pv > 0.0)) {
                bad[g] = 1;
                pv = 1.0;
            }
            pv = sqrt(pv);
            r[cu][cu] = pv;
            rpiv[c] = 1.0 / pv;
        }
        __syncthreads();
        if (tj == cr) {
            const double rp = rpiv[c];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = ti + 16 * u;
                if (i > c) {
                    r[u][cu] = r[u][cu] * rp;
                    col[i] = r[u][cu];
                }
            }
        }
        __syncthreads();
        // every column j > c takes the update, without branches: the entries above the
        // diagonal that this also changes are never read or stored; finished columns
        // (j <= c) see a zero factor
        double ci[4], cj[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ci[u] = col[ti + 16 * u];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const double cv = col[tj + 16 * v];
            cj[v] = (tj + 16 * v > c) ? cv : 0.0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) r[u][v] = fma(-ci[u], cj[v], r[u][v]);
        // col is rewritten at step c + 1 only after that step's first barrier
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            a[ti + 16 * u][tj + 16 * v] = r[u][v];
            x[ti + 16 * u][tj + 16 * v] = 0.0;
        }
    __syncthreads();
    // inverse of the lower-triangular block, column c by the four adjacent lanes
    // 4c .. 4c + 3 (lane q of the four takes k = c + q, c + q + 4, ...; the four partial
    // sums are combined across the quad with DPP moves):
    // X_cc = 1 / L_cc,  X_ic = -(sum_{k=c}^{i-1} L_ik X_kc) / L_ii, the division as a
    // product with the pivot reciprocal kept from the factorization
    {
        const int c = tid >> 2, q = tid & 3;
        if (q == 0) x[c][c] = rpiv[c];
        for (int i = c + 1; i < CB; ++i) {
            double s = 0.0;
            for (int k = c + q; k < i; k += 4) s += a[i][k] * x[k][c];
            s += quad_dpp_f64<0xB1>(s);       // quad_perm [1,0,3,2]
            s += quad_dpp_f64<0x4E>(s);       // quad_perm [2,3,0,1]
            if (q == 0) x[i][c] = -s * rpiv[i];
            // the four lanes of column c read x[i][c] in the next row: the write above
            // and those reads come from one wave, in order
        }
    }
    __syncthreads();
    double* Lg = Linv + (size_t)g * CB * CB;
    for (int e = tid; e < CB * CB; e += 256) {
        const int i = e / CB, j = e % CB;
        if (j <= i) Ag[(o + i) * d + o + j] = a[i][j];
        Lg[e] = x[i][j];
    }
}

// Rows below diagonal block p, 64 at a time: L[r][c] = sum_k A[r][k] Linv[c][k]
// (Linv lower, so k <= c).  Grid (row tiles, groups), 256 threads, 4 x 4 outputs each.
__global__ __launch_bounds__(256) void k_chol_panel(double* __restrict__ A, int64_t d, int p,
                                                   const double* __restrict__ Linv) {
    __shared__ double li[CB][CB + 1];
    __shared__ double ar[CB][CB + 1];
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    double* Ag = A + (size_t)g * d * d;
    const int64_t o = (int64_t)p * CB;
    const int64_t r0 = o + CB + (int64_t)blockIdx.x * CB;
    const double* Lg = Linv + (size_t)g * CB * CB;
    for (int e = tid; e < CB * CB; e += 256) {
        const int i = e / CB, j = e % CB;
        li[i][j] = Lg[e];
        ar[i][j] = (r0 + i < d) ? Ag[(r0 + i) * d + o + j] : 0.0;
    }
    __syncthreads();
    const int tr = tid / 16, tc = tid % 16;        // rows tr + 16 u, columns tc + 16 v
    double acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
    for (int k = 0; k < CB; ++k) {
        double av[4], lv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) av[u] = ar[tr + 16 * u][k];
#pragma unroll
        for (int v = 0; v < 4; ++v) lv[v] = li[tc + 16 * v][k];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = fma(av[u], lv[v], acc[u][v]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t r = r0 + tr + 16 * u;
        if (r < d) {
#pragma unroll
            for (int v = 0; v < 4; ++v) Ag[r * d + o + tc + 16 * v] = acc[u][v];
        }
    }
}

// Trailing update after panel p: tiles (ti, tj), tj <= ti, of the lower triangle
// (counted from tile p + 1): A[ti][tj] -= L[ti][p] L[tj][p]^T.  `part` 1 takes the
// next panel's column (tj = 0, one tile per block), `part` 2 the rest (tj >= 1, a
// linear index over that triangle).
__global__ __launch_bounds__(256) void k_chol_update(double* __restrict__ A, int64_t d, int p,
                                                    int part) {
    __shared__ double li[CB][CB + 1];
    __shared__ double lj[CB][CB + 1];
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    int ti, tj;
    if (part == 1) {
        ti = blockIdx.x;
        tj = 0;
    } else {
        int t = blockIdx.x, r = 0;
        while (t > r) { t -= r + 1; ++r; }
        ti = r + 1;
        tj = t + 1;
    }
    const int64_t oi = (int64_t)(p + 1 + ti) * CB, oj = (int64_t)(p + 1 + tj) * CB;
    const int64_t o = (int64_t)p * CB;
    double* Ag = A + (size_t)g * d * d;
    for (int e = tid; e < CB * CB; e += 256) {
        const int i = e / CB, k = e % CB;
        li[i][k] = Ag[(oi + i) * d + o + k];
        lj[i][k] = Ag[(oj + i) * d + o + k];
    }
    __syncthreads();
    const int tr = tid / 16, tc = tid % 16;
    double acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
    for (int k = 0; k < CB; ++k) {
        double av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) av[u] = li[tr + 16 * u][k];
#pragma unroll
        for (int v = 0; v < 4; ++v) bv[v] = lj[tc + 16 * v][k];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = fma(av[u], bv[v], acc[u][v]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = tr + 16 * u, j = tc + 16 * v;
            if (ti != tj || j <= i) Ag[(oi + i) * d + oj + j] -= acc[u][v];
        }
}

// ---------------------------------------------------------------------------
// U = L^T as k-blocked bf16 planes: element (a, k) = U[a][k] = L[k][a] for k > a, else
// 0, at ((k / 16) * a_pad + a) * 16 + k % 16 (the layout of the F' planes); dL = diag L.
// One thread per (group, 16-block of k, a).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ganq_prep(const double* __restrict__ A, int64_t d,
                                                  int64_t a_pad, uint16_t* __restrict__ Uhi,
                                                  uint16_t* __restrict__ Ulo,
                                                  float* __restrict__ dL) {
    const int g = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nkb = d / 16;
    if (t >= nkb * a_pad) return;
    const int64_t kb = t / a_pad, a = t - kb * a_pad;
    const double* Ag = A + (size_t)g * d * d;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        float v2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t k = kb * 16 + 2 * q + h;
            v2[h] = (a < d && k > a) ? (float)Ag[k * d + a] : 0.f;
        }
        hi[q] = pack_bf16x2(v2[0], v2[1]);
        const float r0 = v2[0] - bf16_bits_to_f32(hi[q] & 0xffffu);
        const float r1 = v2[1] - bf16_bits_to_f32(hi[q] >> 16);
        lo[q] = pack_bf16x2(r0, r1);
    }
    const size_t off = ((size_t)g * nkb * a_pad + (size_t)t) * 16;
    u32x4* H = (u32x4*)(Uhi + off);
    u32x4* Lo = (u32x4*)(Ulo + off);
    H[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    H[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
    Lo[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    Lo[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
    if (kb == 0 && a < d) dL[(size_t)g * d + a] = (float)Ag[a * d + a];
}

// the factor as float32, zeros above the diagonal
__global__ void k_ganq_export(const double* __restrict__ A, int64_t n, float* __restrict__ L) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) L[i] = (float)A[i];
}

__device__ __forceinline__ float ganq_readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// The row's codebook in ascending order (equal values keep their index order) and the
// midpoints between neighbours.  For ascending a <= b, b is nearer to x than a exactly
// when x > (a + b) / 2.  Entries are placed by rank, so every register index is a
// compile-time constant.
template <int M>
__device__ __forceinline__ void ganq_sorted_codebook(const float (&cq)[M], float (&sv)[M],
                                                     float (&mid)[M - 1]) {
    int rank[M];
#pragma unroll
    for (int q = 0; q < M; ++q) {
        rank[q] = 0;
#pragma unroll
        for (int p = 0; p < M; ++p)
            rank[q] += (cq[p] < cq[q] || (cq[p] == cq[q] && p < q)) ? 1 : 0;
    }
#pragma unroll
    for (int r = 0; r < M; ++r) {
        sv[r] = 0.f;
#pragma unroll
        for (int q = 0; q < M; ++q) sv[r] = (rank[q] == r) ? cq[q] : sv[r];
    }
#pragma unroll
    for (int k = 0; k < M - 1; ++k) mid[k] = 0.5f * sv[k] + 0.5f * sv[k + 1];
}

// The entry nearest to x: a binary search over the midpoints.  Each level compares x
// with the middle midpoint and keeps the upper or lower half of the candidate values and
// midpoints with selects (log2 N compares).  At a midpoint itself the lower entry.  The
// halves are built from index packs so that no register array is indexed by a variable.
template <int N>
struct GanqNearest {
    template <int... K, int... J>
    static __device__ __forceinline__ float level(float x, const float (&v)[N],
                                                  const float (&b)[N - 1],
                                                  std::integer_sequence<int, K...>,
                                                  std::integer_sequence<int, J...>) {
        constexpr int H = N / 2;
        const bool up = x > b[H - 1];
        const float v2[H] = {(up ? v[K + H] : v[K])...};
        const float b2[H - 1] = {(up ? b[J + H] : b[J])...};
        return GanqNearest<H>::run(x, v2, b2);
    }
    static __device__ __forceinline__ float run(float x, const float (&v)[N],
                                                const float (&b)[N - 1]) {
        return level(x, v, b, std::make_integer_sequence<int, N / 2>{},
                     std::make_integer_sequence<int, N / 2 - 1>{});
    }
};
template <>
struct GanqNearest<2> {
    static __device__ __forceinline__ float run(float x, const float (&v)[2], const float (&b)[1]) {
        return x > b[0] ? v[1] : v[0];
    }
};

__global__ void k_zero_f32(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// The assignment pass.  One block = 16 rows of one group (one row per wave).
// ---------------------------------------------------------------------------
constexpr int GQ_ROWS = 16;
constexpr int GQ_SUB = 64;
constexpr int GQ_SB = 512;
constexpr int GQ_DP = GQ_SB + 8;

template <bool WBF16, int M>
__global__ __launch_bounds__(1024, 1) void k_ganq(
    const double* __restrict__ A, const float* __restrict__ dL,
    const uint16_t* __restrict__ Uhi, const uint16_t* __restrict__ Ulo, int64_t d,
    int64_t rows_per_group, int wgs_per_group, int total_wgs, const float* __restrict__ C,
    uint8_t* __restrict__ P, const void* __restrict__ W, float* __restrict__ S,
    const int* __restrict__ bad, unsigned long long* __restrict__ n_changed) {
    __shared__ __attribute__((aligned(16))) uint16_t esb_hi[GQ_ROWS][GQ_DP];
    __shared__ __attribute__((aligned(16))) uint16_t esb_lo[GQ_ROWS][GQ_DP];
    __shared__ __attribute__((aligned(16))) float corr_p[4][GQ_ROWS][GQ_SUB];
    __shared__ float lb[GQ_SUB][GQ_SUB];         // lb[t][i] = L[bs + t][bs + i] for t > i, else 0
    __shared__ float ldiag[GQ_SUB];

    const int nb = gridDim.x;
    const int hw = blockIdx.x;
    const int lin = (hw & 7) * (nb >> 3) + (hw >> 3);
    if (lin >= total_wgs) return;                 // whole block exits together
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lin / wgs_per_group;
    if (bad[g]) return;                           // F' not positive definite: codes kept
    const int64_t local = (int64_t)(lin % wgs_per_group) * GQ_ROWS;
    const int64_t jl = local + wave;
    const bool rvalid = jl < rows_per_group;
    const int64_t j = (int64_t)g * rows_per_group + (rvalid ? jl : 0);
    const int64_t row0 = (int64_t)g * rows_per_group + local;
    const int nrows = (int)((rows_per_group - local) < GQ_ROWS ? (rows_per_group - local) : GQ_ROWS);

    const double* Ag = A + (size_t)g * d * d;
    const float* dLg = dL + (size_t)g * d;
    const int64_t a_pad = lnq_pad256(d);
    const uint16_t* Uh = Uhi + (size_t)g * d * a_pad;
    const uint16_t* Ul = Ulo + (size_t)g * d * a_pad;
    const uint32_t kstep32 = (uint32_t)(32 * a_pad);
    auto plane_at = [&](const uint16_t* base, int64_t a, int64_t k) {
        return base + ((k >> 4) * a_pad + a) * 16 + (k & 15);
    };
    float cq[M];
#pragma unroll
    for (int q = 0; q < M; ++q) {
        cq[q] = rvalid ? C[j * M + q] : 0.f;
        // keep the codebook in vector registers: the nearest-entry scan selects from it
        // with v_cndmask, which takes its second operand from a vector register
        asm volatile("" : "+v"(cq[q]));
    }
    float sv[M], mid[M - 1];
    ganq_sorted_codebook<M>(cq, sv, mid);
    unsigned moves = 0;
    const int ko = 8 * (lane >> 4);
    const int mrow = lane & 15;

    const int64_t last_sb = ((d - 1) / GQ_SB) * GQ_SB;
    for (int64_t sb0 = last_sb; sb0 >= 0; sb0 -= GQ_SB) {
        const int sblen = (int)((d - sb0) < GQ_SB ? (d - sb0) : GQ_SB);
        const int nch = sblen / 32;
        for (int o = sblen - GQ_SUB; o >= 0; o -= GQ_SUB) {
            const int64_t bs = sb0 + o;
            // ---- the super-block's later blocks: corr_i = sum_{k in sb, k >= o + 64}
            // U[bs + i][sb0 + k] e_k, 4 column tiles x 4 k-slices of 32-chunks
            {
                const int ct = wave & 3, sl = wave >> 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int64_t fcol = bs + ct * 16 + mrow;
                const uint16_t* Uh_c = plane_at(Uh, fcol, sb0 + ko);
                const uint16_t* Ul_c = plane_at(Ul, fcol, sb0 + ko);
                for (int c = (o + GQ_SUB) / 32 + sl; c < nch; c += 4) {
                    const u32x4 fh = *(const u32x4*)(Uh_c + (uint32_t)c * kstep32);
                    const u32x4 fl = *(const u32x4*)(Ul_c + (uint32_t)c * kstep32);
                    const u32x4 eh = *(const u32x4*)(&esb_hi[mrow][c * 32 + ko]);
                    const u32x4 el = *(const u32x4*)(&esb_lo[mrow][c * 32 + ko]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(eh), as_bf16x8(fh), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(eh), as_bf16x8(fl), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(el), as_bf16x8(fh), acc, 0, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) corr_p[sl][4 * (lane >> 4) + t][ct * 16 + mrow] = acc[t];
            }
            // ---- stage the block of L (strictly lower part) and its diagonal
            for (int e = tid; e < GQ_SUB * GQ_SUB; e += 1024) {
                const int t = e >> 6, i = e & 63;
                lb[t][i] = (t > i) ? (float)Ag[(bs + t) * d + bs + i] : 0.f;
            }
            if (tid < GQ_SUB) ldiag[tid] = dLg[bs + tid];
            __syncthreads();

            float ev = 0.f;
            if (rvalid) {
                const int64_t col = bs + lane;
                float s = S[j * d + col];
#pragma unroll
                for (int k = 0; k < 4; ++k) s += corr_p[k][wave][lane];
                const float wv = load_elem<WBF16>(W, j * d + col);
                const float inv_u = 1.f / ldiag[lane];
                const int old = P[j * d + col];
                // step t: lane t's entry, nearest to w - s / L_tt, then lanes i < t add
                // L[t][i] e_t (lb[t][i] = 0 for i >= t).  A lane's s is final from its
                // own step on.
#pragma unroll
                for (int t = GQ_SUB - 1; t >= 0; --t) {
                    const float bc = GanqNearest<M>::run(fmaf(-s, inv_u, wv), sv, mid);
                    s = fmaf(lb[t][lane], ganq_readlane_f(bc - wv, t), s);
                }
                // every lane's own entry, from its final s: the same arithmetic as at its step
                const float bsel = GanqNearest<M>::run(fmaf(-s, inv_u, wv), sv, mid);
                ev = bsel - wv;
                // its code: the lowest index holding the chosen value
                int code = 0;
#pragma unroll
                for (int q = M - 1; q >= 0; --q)
                    if (cq[q] == bsel) code = q;
                P[j * d + col] = (uint8_t)code;
                const unsigned long long chg = __ballot(code != old);
                moves += (unsigned)__popcll(chg);
            }
            const uint32_t hb = f32_to_bf16_bits(ev);
            esb_hi[wave][o + lane] = (uint16_t)hb;
            esb_lo[wave][o + lane] = (uint16_t)f32_to_bf16_bits(ev - __uint_as_float(hb << 16));
            __syncthreads();
        }
        // ---- earlier coordinates: S[rows, :sb0] += E_sb U[:sb0, sb]^T, one 16-column
        // tile per wave.  Two register sets of two 32-chunks alternate, one set's loads in
        // flight while the other's products run (nch is even: sblen % 64 == 0); the tile's
        // 16 x 16 sum is transposed through this wave's quarter of corr_p (unused here) so
        // that lane l adds columns 4 (l % 4) .. + 3 of row l / 4 with one 16-byte
        // read-modify-write.
        const int ntiles = (int)(sb0 / 16);
        for (int ctile = wave; ctile < ntiles; ctile += GQ_ROWS) {
            const int64_t fcol = (int64_t)ctile * 16 + mrow;
            const uint16_t* Uh_c = plane_at(Uh, fcol, sb0 + ko);
            const uint16_t* Ul_c = plane_at(Ul, fcol, sb0 + ko);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            u32x4 ah[2], al[2], bh[2], bl[2];
            auto load2 = [&](u32x4 (&h)[2], u32x4 (&l)[2], int c0) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    h[u] = *(const u32x4*)(Uh_c + (uint32_t)(c0 + u) * kstep32);
                    l[u] = *(const u32x4*)(Ul_c + (uint32_t)(c0 + u) * kstep32);
                }
            };
            auto mfma2 = [&](const u32x4 (&h)[2], const u32x4 (&l)[2], int c0) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int c = c0 + u;
                    const u32x4 eh = *(const u32x4*)(&esb_hi[mrow][c * 32 + ko]);
                    const u32x4 el = *(const u32x4*)(&esb_lo[mrow][c * 32 + ko]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(eh), as_bf16x8(h[u]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(eh), as_bf16x8(l[u]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(el), as_bf16x8(h[u]), acc, 0, 0, 0);
                }
            };
            load2(ah, al, 0);
            for (int c0 = 0; c0 < nch; c0 += 4) {
                if (c0 + 2 < nch) load2(bh, bl, c0 + 2);
                mfma2(ah, al, c0);
                if (c0 + 4 < nch) load2(ah, al, c0 + 4);
                if (c0 + 2 < nch) mfma2(bh, bl, c0 + 2);
            }
            float* xp = &corr_p[0][0][0] + wave * 256;
#pragma unroll
            for (int t = 0; t < 4; ++t) xp[(4 * (lane >> 4) + t) * 16 + mrow] = acc[t];
            const int rr = lane >> 2;
            if (rr < nrows) {
                f32x4* dst = (f32x4*)(S + (row0 + rr) * d + (int64_t)ctile * 16 + 4 * (lane & 3));
                const f32x4 sv0 = *dst;
                *dst = sv0 + *(const f32x4*)(xp + 4 * lane);
            }
        }
        __syncthreads();
    }
    if (rvalid && lane == 0 && n_changed) atomicAdd(n_changed, (unsigned long long)moves);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
size_t ganq_extra_bytes(int64_t d, int groups) {
    const int64_t a_pad = lnq_pad256(d);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)groups * d * d * 8) + 2 * al((size_t)groups * d * a_pad * 2) +
           al((size_t)groups * d * 4) + al((size_t)groups * CB * CB * 8) + al((size_t)groups * 4);
}

GanqWs ganq_carve(void* base, int64_t d, int groups) {
    const int64_t a_pad = lnq_pad256(d);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char* b = (char*)base;
    GanqWs w;
    w.A = (double*)b;            b += al((size_t)groups * d * d * 8);
    w.uhi = (uint16_t*)b;        b += al((size_t)groups * d * a_pad * 2);
    w.ulo = (uint16_t*)b;        b += al((size_t)groups * d * a_pad * 2);
    w.dL = (float*)b;            b += al((size_t)groups * d * 4);
    w.Linv = (double*)b;         b += al((size_t)groups * CB * CB * 8);
    w.bad = (int*)b;
    return w;
}

// The factorization with one panel of lookahead.  Per panel p, on the caller's stream:
// the diagonal block and the panel, then the part of the trailing update that the next
// panel needs (its column); on a second stream, once panel p is done, the rest of the
// trailing update.  The next diagonal block and panel thus run beside the bulk of the
// update.  Ordering: the column update of panel p waits for the rest-update of panel
// p - 1 (both write tile column p + 1 and later); the rest-update of panel p writes
// columns p + 2 on, which the next diagonal block and panel do not touch.
hipError_t ganq_factor(const float* F, const double* lam, int64_t d, int groups, const GanqWs& w,
                       hipStream_t st) {
    StageTimer tm(ST_GANQ_CHOL, st);
    {
        const dim3 grid((unsigned)((d * d + 255) / 256), (unsigned)groups);
        hipLaunchKernelGGL(k_chol_init, grid, dim3(256), 0, st, F, lam, d, w.A, w.bad);
        GQ_LAUNCH_CHECK();
    }
    const int nt = (int)(d / CB);               // d % 64 == 0
    hipStream_t side = nullptr;
    hipEvent_t panel_done = nullptr, rest_done = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&panel_done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&rest_done, hipEventDisableTiming);
    bool rest_recorded = false;
    for (int p = 0; p < nt && e == hipSuccess; ++p) {
        hipLaunchKernelGGL(k_chol_diag, dim3((unsigned)groups), dim3(256), 0, st, w.A, d, p, w.Linv,
                           w.bad);
        if ((e = hipGetLastError()) != hipSuccess) break;
        const int rest = nt - p - 1;
        if (rest == 0) break;
        hipLaunchKernelGGL(k_chol_panel, dim3((unsigned)rest, (unsigned)groups), dim3(256), 0, st,
                           w.A, d, p, w.Linv);
        if ((e = hipGetLastError()) != hipSuccess) break;
        if ((e = hipEventRecord(panel_done, st)) != hipSuccess) break;
        if (rest_recorded && (e = hipStreamWaitEvent(st, rest_done, 0)) != hipSuccess) break;
        hipLaunchKernelGGL(k_chol_update, dim3((unsigned)rest, (unsigned)groups), dim3(256), 0, st,
                           w.A, d, p, 1);
        if ((e = hipGetLastError()) != hipSuccess) break;
        if (rest > 1) {
            if ((e = hipStreamWaitEvent(side, panel_done, 0)) != hipSuccess) break;
            const int ntri = (rest - 1) * rest / 2;
            hipLaunchKernelGGL(k_chol_update, dim3((unsigned)ntri, (unsigned)groups), dim3(256), 0,
                               side, w.A, d, p, 2);
            if ((e = hipGetLastError()) != hipSuccess) break;
            if ((e = hipEventRecord(rest_done, side)) != hipSuccess) break;
            rest_recorded = true;
        }
    }
    // the caller's stream resumes after the side stream's last update
    if (e == hipSuccess && rest_recorded) e = hipStreamWaitEvent(st, rest_done, 0);
    if (panel_done) (void)hipEventDestroy(panel_done);
    if (rest_done) (void)hipEventDestroy(rest_done);
    if (side) (void)hipStreamDestroy(side);
    if (e != hipSuccess) return e;
    const int64_t a_pad = lnq_pad256(d);
    const dim3 grid((unsigned)(((d / 16) * a_pad + 255) / 256), (unsigned)groups);
    hipLaunchKernelGGL(k_ganq_prep, grid, dim3(256), 0, st, w.A, d, a_pad, w.uhi, w.ulo, w.dL);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t ganq_factor_out(const GanqWs& w, int64_t d, int groups, float* L, int* bad_out,
                           hipStream_t st) {
    // L [groups][d][d] float32 (lower triangle; zeros above) and the per-group flags
    if (L) {
        const int64_t n = (int64_t)groups * d * d;
        hipLaunchKernelGGL(k_ganq_export, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w.A,
                           n, L);
        GQ_LAUNCH_CHECK();
    }
    if (bad_out) {
        hipError_t e = hipMemcpyAsync(bad_out, w.bad, (size_t)groups * 4, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <bool WB>
static hipError_t launch_ganq(const GanqWs& g, int64_t d, int64_t d_out, int groups,
                              const float* C, int m, uint8_t* P, const void* W, float* S,
                              unsigned long long* counter, hipStream_t st) {
    const int64_t rpg = d_out / groups;
    const int wgs = (int)((rpg + GQ_ROWS - 1) / GQ_ROWS);
    const int total = wgs * groups;
    const int grid = (total + 7) / 8 * 8;
    auto kern = (m == 2) ? k_ganq<WB, 2> : (m == 4) ? k_ganq<WB, 4> : (m == 8) ? k_ganq<WB, 8>
                                                                  : k_ganq<WB, 16>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(1024), 0, st, g.A, g.dL, g.uhi, g.ulo, d,
                       rpg, wgs, total, C, P, W, S, g.bad, counter);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t ganq_assign_run(const GanqWs& g, int64_t d, int64_t d_out, int groups, const float* C,
                           int m, uint8_t* P, const void* W, bool w_bf16, float* S,
                           unsigned long long* counter, hipStream_t st) {
    StageTimer tm(ST_GANQ_PASS, st);
    const int64_t n = d_out * d;
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, S, n);
    GQ_LAUNCH_CHECK();
    return w_bf16 ? launch_ganq<true>(g, d, d_out, groups, C, m, P, W, S, counter, st)
                  : launch_ganq<false>(g, d, d_out, groups, C, m, P, W, S, counter, st);
}

}  // namespace gq
