// Matrix-core products with the damped Fisher F' for LNQ on gfx950.
//
// GuidedQuant blog page (jinukkim.me/blog/guidedquant), section "LNQ": the
// "(codebook)" line needs P_j^T F' P_j and P_j^T F' w_j for every row j, and the
// "(assignment)" objective (w_hat - w)^T F' (w_hat - w) is tracked through the
// residual r_j = F'(w_hat_j - w_j).  Two products over all rows of a group do
// the dense work:
//
//   MM_RESID  R[j][a] = sum_i E[j][i] F'[a][i],  E = C[P] - W split into bf16
//             hi + lo planes, F' as bf16 hi + lo planes; three products
//             (Ehi Fhi + Ehi Flo + Elo Fhi) give float32-level accuracy.
//   MM_GRAM   A_j = P_j^T F' P_j.  With the one-hot P_j built from the codes in
//             registers (exact in bf16) the kernel forms
//                 T[a][(j,q)] = sum_{i >= tile(a)} F'[a][i] [P[j][i] == q]
//             over the upper-triangle tiles of F' only (the diagonal tile at
//             half weight), and the epilogue bins T by the code of coordinate a:
//                 B_j[q'][q] += sum_a [P[j][a] == q'] T[a][(j,q)].
//             Then A_j = B_j + B_j^T (by the symmetry of F').  Per-a-tile
//             partials are written in a fixed layout and summed in a fixed order.
//
// Block tile 256 x 256, 4 waves of 128 x 128 as 4 x 4 v_mfma_f32_32x32x16_bf16
// tiles, k staged 32 at a time through LDS (80-byte rows), register prefetch of
// the next stage while the current one is multiplied.
#include "gq_common.h"
#include "gq_internal.h"

namespace gq {

constexpr int MT = 256;        // block tile edge
constexpr int MKC = 32;        // k per LDS stage
constexpr int MPITCH = 40;     // bf16 per staged row
constexpr int M_PLANE = MT * MPITCH;
constexpr int MM_RESID = 0, MM_GRAM = 1;

template <int MODE>
constexpr int mm_stage_elems() {
    // RESID: Ehi, Elo, Fhi, Flo planes.  GRAM: Fhi, Flo planes + up to 128 rows x 32 code bytes.
    return MODE == MM_RESID ? 4 * M_PLANE : 2 * M_PLANE + (128 * 32) / 2;
}

template <int MODE>
constexpr size_t mm_lds_bytes() {
    return (size_t)2 * mm_stage_elems<MODE>() * sizeof(uint16_t);
}

// Hardware block h -> logical block: within each round of 256 blocks, XCD x
// (= h % 8) receives 32 consecutive logical blocks.
__device__ __forceinline__ int mm_remap(int hw) {
    return (hw & ~255) + (hw & 7) * 32 + ((hw & 255) >> 3);
}

template <int MODE, int M>
__global__ __launch_bounds__(256, 1) void k_mm(
    const uint16_t* __restrict__ Ehi, const uint16_t* __restrict__ Elo,
    const uint8_t* __restrict__ codes, int64_t rpg, int g_first, int g_count,
    const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo, int64_t d,
    int ntile_n, int ntile_a, int total, float* __restrict__ out, int64_t d_out) {
    extern __shared__ __attribute__((aligned(16))) uint16_t mm_lds[];
    constexpr int STAGE = mm_stage_elems<MODE>();
    const int lin = mm_remap(blockIdx.x);
    if (lin >= total) return;

    int tn, ta, gl;
    if (MODE == MM_RESID) {
        ta = lin % ntile_a;
        tn = (lin / ntile_a) % ntile_n;
        gl = lin / (ntile_a * ntile_n);
    } else {
        tn = lin % ntile_n;
        gl = (lin / ntile_n) % g_count;
        ta = lin / (ntile_n * g_count);
    }
    const int g = g_first + gl;
    const int64_t a0 = (int64_t)ta * MT;
    const int64_t n0 = (int64_t)tn * MT;
    // number of valid rows of the "n" operand: RESID rows of E; GRAM (j, q) pairs
    const int64_t N = (MODE == MM_RESID) ? rpg : rpg * M;
    const int64_t row_base = (int64_t)g * rpg;           // first row j of the group
    const uint16_t* Fh = Fhi + (size_t)g * d * d;
    const uint16_t* Fl = Flo + (size_t)g * d * d;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w0 = wave & 1, w1 = wave >> 1;
    const int sr = tid >> 2, sq = tid & 3;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;

    const int64_t k_begin = (MODE == MM_GRAM) ? a0 : 0;
    const int nk = (int)((d - k_begin + MKC - 1) / MKC);
    const int ndiag = (MODE == MM_GRAM) ? (int)((((d - a0) < MT ? (d - a0) : MT) + MKC - 1) / MKC) : 0;

    constexpr int NPL = (MODE == MM_RESID) ? 4 : 2;
    u32x4 pf[NPL][4];
    u32x4 pc = {0u, 0u, 0u, 0u};
    const int jrows = MT / M;                 // GRAM: code rows per n tile

    auto fetch = [&](int64_t k0) {
        const int64_t kk = k0 + 8 * sq;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = sr + 64 * s;
            if (MODE == MM_RESID) {
                const int64_t nrow = n0 + r, arow = a0 + r;
                const bool nok = nrow < N && kk < d, aok = arow < d && kk < d;
                pf[0][s] = nok ? *(const u32x4*)(Ehi + (row_base + nrow) * d + kk) : z;
                pf[1][s] = nok ? *(const u32x4*)(Elo + (row_base + nrow) * d + kk) : z;
                pf[2][s] = aok ? *(const u32x4*)(Fh + arow * d + kk) : z;
                pf[3][s] = aok ? *(const u32x4*)(Fl + arow * d + kk) : z;
            } else {
                const int64_t arow = a0 + r;
                const bool aok = arow < d && kk < d;
                pf[0][s] = aok ? *(const u32x4*)(Fh + arow * d + kk) : z;
                pf[1][s] = aok ? *(const u32x4*)(Fl + arow * d + kk) : z;
            }
        }
        if (MODE == MM_GRAM) {
            // jrows rows x 32 code bytes: thread covers row tid/2, bytes 16*(tid%2)
            const int r = tid >> 1;
            const int64_t jl = n0 / M + r;
            const int64_t kc = k0 + 16 * (tid & 1);
            pc = (r < jrows && jl < rpg && kc < d)
                     ? *(const u32x4*)(codes + (row_base + jl) * d + kc)
                     : u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        }
    };
    auto stage = [&](int buf) {
        uint16_t* S = mm_lds + buf * STAGE;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = sr + 64 * s;
#pragma unroll
            for (int p = 0; p < NPL; ++p) *(u32x4*)(S + p * M_PLANE + r * MPITCH + 8 * sq) = pf[p][s];
        }
        if (MODE == MM_GRAM) {
            uint8_t* cs = (uint8_t*)(S + 2 * M_PLANE);
            *(u32x4*)(cs + (tid >> 1) * 32 + 16 * (tid & 1)) = pc;
        }
    };

    fetch(k_begin);
    stage(0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        const bool more = kc + 1 < nk;
        if (more) fetch(k_begin + (int64_t)(kc + 1) * MKC);
        const uint16_t* S = mm_lds + buf * STAGE;
#pragma unroll
        for (int ks = 0; ks < MKC / 16; ++ks) {
            const int koff = ks * 16 + 8 * (lane >> 5);
            if (MODE == MM_RESID) {
                bf16x8 eh[4], el[4], fh[4], fl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = (128 * w0 + 32 * i + (lane & 31)) * MPITCH + koff;
                    eh[i] = as_bf16x8(*(const u32x4*)(S + rr));
                    el[i] = as_bf16x8(*(const u32x4*)(S + M_PLANE + rr));
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int rr = (128 * w1 + 32 * jj + (lane & 31)) * MPITCH + koff;
                    fh[jj] = as_bf16x8(*(const u32x4*)(S + 2 * M_PLANE + rr));
                    fl[jj] = as_bf16x8(*(const u32x4*)(S + 3 * M_PLANE + rr));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(eh[i], fh[jj], acc[i][jj], 0, 0, 0);
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(eh[i], fl[jj], acc[i][jj], 0, 0, 0);
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(el[i], fh[jj], acc[i][jj], 0, 0, 0);
                    }
            } else {
                bf16x8 fh[4], fl[4], oh[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = (128 * w0 + 32 * i + (lane & 31)) * MPITCH + koff;
                    fh[i] = as_bf16x8(*(const u32x4*)(S + rr));
                    fl[i] = as_bf16x8(*(const u32x4*)(S + M_PLANE + rr));
                }
                const uint8_t* cs = (const uint8_t*)(S + 2 * M_PLANE);
                // the diagonal tile enters B_j at half weight: one-hot value 0.5 (exact)
                const uint32_t one = (kc < ndiag) ? 0x3F00u : 0x3F80u;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int nl = 128 * w1 + 32 * jj + (lane & 31);
                    const int jr = nl / M, q = nl - jr * M;
                    const u32x2 cv = *(const u32x2*)(cs + jr * 32 + koff);
                    u32x4 o;
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t word = cv[h >> 1];
                        const uint32_t b0 = (word >> (16 * (h & 1))) & 0xffu;
                        const uint32_t b1 = (word >> (16 * (h & 1) + 8)) & 0xffu;
                        o[h] = ((b0 == (uint32_t)q) ? one : 0u) | ((b1 == (uint32_t)q) ? (one << 16) : 0u);
                    }
                    oh[jj] = as_bf16x8(o);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh[i], oh[jj], acc[i][jj], 0, 0, 0);
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl[i], oh[jj], acc[i][jj], 0, 0, 0);
                    }
            }
        }
        if (more) stage(buf ^ 1);
        __syncthreads();
    }

    if (MODE == MM_RESID) {
        float* O = out + (size_t)row_base * d;
        const int nrem = (int)((N - n0) < MT ? (N - n0) : MT);
        const int arem = (int)((d - a0) < MT ? (d - a0) : MT);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int acol = 128 * w1 + 32 * jj + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int nrow = 128 * w0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    if (nrow < nrem && acol < arem)
                        O[(size_t)(n0 + nrow) * d + a0 + acol] = acc[i][jj][v];
                }
            }
    } else {
        // ---- epilogue: bin T[a][(j,q)] by the code of coordinate a
        // stage the codes of the block's rows for its 256 coordinates: jrows x 256 bytes
        uint8_t* ctile = (uint8_t*)mm_lds;       // the stages are free after the last sync
        for (int e = tid; e < jrows * (MT / 16); e += 256) {
            const int r = e / (MT / 16), c16 = (e - r * (MT / 16)) * 16;
            const int64_t jl = n0 / M + r;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (jl < rpg && a0 + c16 < d) v = *(const u32x4*)(codes + (row_base + jl) * d + a0 + c16);
            *(u32x4*)(ctile + r * MT + c16) = v;
        }
        __syncthreads();
        float* xch = (float*)(mm_lds + (MT / M) * MT / 2 + 64);   // after the code tile
        const int arem = (int)((d - a0) < MT ? (d - a0) : MT);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int nl = 128 * w1 + 32 * jj + (lane & 31);
            const int jr = nl / M, q = nl - jr * M;
            float bins[M];
#pragma unroll
            for (int k = 0; k < M; ++k) bins[k] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int al = 128 * w0 + 32 * i + 8 * v4 + 4 * (lane >> 5);
                    const uint32_t cw = *(const uint32_t*)(ctile + jr * MT + al);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t code = (cw >> (8 * e)) & 0xffu;
                        const float x = (al + e < arem) ? acc[i][jj][4 * v4 + e] : 0.f;
#pragma unroll
                        for (int k = 0; k < M; ++k) bins[k] += (code == (uint32_t)k) ? x : 0.f;
                    }
                }
            // lanes l and l + 32 hold the same (j, q) for the other half of the a's
#pragma unroll
            for (int k = 0; k < M; ++k) bins[k] += __shfl_xor(bins[k], 32, 64);
            // waves with w0 = 1 hand their sums to the waves with w0 = 0
            if (w0 == 1 && lane < 32) {
#pragma unroll
                for (int k = 0; k < M; ++k) xch[(w1 * 32 + lane) * M + k] = bins[k];
            }
            __syncthreads();
            if (w0 == 0 && lane < 32) {
                const int64_t n = n0 + nl;
                if (n < N) {
                    float* dst = out + ((size_t)ta * d_out * M + (size_t)(row_base * M + n)) * M;
#pragma unroll
                    for (int k = 0; k < M; ++k) dst[k] = bins[k] + xch[(w1 * 32 + lane) * M + k];
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <int MODE, int M>
static hipError_t launch_mm(const uint16_t* Ehi, const uint16_t* Elo, const uint8_t* codes,
                            int64_t rpg, int g_first, int g_count, const uint16_t* Fhi,
                            const uint16_t* Flo, int64_t d, float* out, int64_t d_out,
                            hipStream_t st) {
    const int64_t N = (MODE == MM_RESID) ? rpg : rpg * M;
    const int ntn = (int)((N + MT - 1) / MT);
    const int nta = (int)((d + MT - 1) / MT);
    const int total = ntn * nta * g_count;
    const int grid = (total + 255) / 256 * 256;        // whole rounds for the XCD remap
    const size_t lds = mm_lds_bytes<MODE>();
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)k_mm<MODE, M>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    StageTimer tm(MODE == MM_RESID ? ST_LNQ_RESID : ST_LNQ_GRAM, st);
    hipLaunchKernelGGL((k_mm<MODE, M>), dim3((unsigned)grid), dim3(256), lds, st, Ehi, Elo, codes,
                       rpg, g_first, g_count, Fhi, Flo, d, ntn, nta, total, out, d_out);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

size_t lnq_gram_partial_floats(int64_t d_out, int64_t d, int m) {
    const int64_t nta = (d + MT - 1) / MT;
    return (size_t)nta * d_out * m * m;
}

hipError_t lnq_residual(const uint16_t* Ehi, const uint16_t* Elo, int64_t d_out, int64_t d,
                        int groups, const uint16_t* Fhi, const uint16_t* Flo, float* R,
                        hipStream_t st) {
    return launch_mm<MM_RESID, 1>(Ehi, Elo, nullptr, d_out / groups, 0, groups, Fhi, Flo, d, R,
                                  d_out, st);
}

hipError_t lnq_gram(const uint8_t* P, int m, int64_t d_out, int64_t d, int groups,
                    const uint16_t* Fhi, const uint16_t* Flo, float* part, hipStream_t st) {
    const int64_t rpg = d_out / groups;
    switch (m) {
        case 2: return launch_mm<MM_GRAM, 2>(nullptr, nullptr, P, rpg, 0, groups, Fhi, Flo, d, part, d_out, st);
        case 4: return launch_mm<MM_GRAM, 4>(nullptr, nullptr, P, rpg, 0, groups, Fhi, Flo, d, part, d_out, st);
        case 8: return launch_mm<MM_GRAM, 8>(nullptr, nullptr, P, rpg, 0, groups, Fhi, Flo, d, part, d_out, st);
        case 16: return launch_mm<MM_GRAM, 16>(nullptr, nullptr, P, rpg, 0, groups, Fhi, Flo, d, part, d_out, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gq
