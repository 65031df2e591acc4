// Grouped Fisher blocks for GuidedQuant on gfx950.
//
// GuidedQuant blog page (jinukkim.me/blog/guidedquant), objective equation and
// the sentence after it: per-output-channel Fisher blocks F_j = X^T diag(G_:j^2) X
// are grouped and averaged within each group.  By linearity the group average is
// F_g = X^T diag(s_g) X with s_g[t] = mean_{j in g} G[t, j]^2.
//
// Kernels
//   k_group_scale     s_g[t] for every token (HBM stream over G).
//   k_fisher_mfma     bf16 MFMA (v_mfma_f32_32x32x16_bf16) SYRK-like contraction over
//                     tokens for the upper-triangle 256x256 tiles of every F_g; the
//                     gradient-square scale is fused into the LDS staging of one
//                     operand; tokens may be split across blocks (split-K) to fill the
//                     chip, each split writing its own partial tile.
//   k_fisher_finalize sums the split partials in a fixed order and writes the tile
//                     and its mirror image (exactly symmetric F), optionally adding.
//   k_fisher_plain    float64-accumulating path for float32 inputs (and the fallback
//                     for shapes the MFMA kernel does not take).
#include "gq_common.h"
#include "gq_internal.h"

namespace gq {

// ---------------------------------------------------------------------------
// s_g[t] = (1/|g|) sum_{j in g} G[t, j]^2          one wave per (token, group)
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void k_group_scale(const void* __restrict__ G, int64_t n,
                                                      int64_t d_out, int groups,
                                                      float* __restrict__ S) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int g = blockIdx.y;
    if (t >= n) return;
    const int64_t size = d_out / groups;
    const int64_t base = t * d_out + (int64_t)g * size;
    float acc = 0.f;
    if constexpr (BF16) {
        const uint16_t* p = (const uint16_t*)G + base;
        if ((size & 7) == 0 && (base & 7) == 0) {
            for (int64_t e = (int64_t)lane * 8; e < size; e += 512) {
                u32x4 v = *(const u32x4*)(p + e);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float lo = __uint_as_float(v[k] << 16);
                    float hi = __uint_as_float(v[k] & 0xffff0000u);
                    acc += lo * lo;
                    acc += hi * hi;
                }
            }
        } else {
            for (int64_t e = lane; e < size; e += 64) {
                float x = bf16_bits_to_f32(p[e]);
                acc += x * x;
            }
        }
    } else {
        const float* p = (const float*)G + base;
        for (int64_t e = lane; e < size; e += 64) {
            float x = p[e];
            acc += x * x;
        }
    }
    acc = wave_sum_f32(acc);
    if (lane == 0) S[(int64_t)g * n + t] = acc / (float)size;
}

// ---------------------------------------------------------------------------
// bf16 MFMA Fisher.  Block tile 256 (a) x 256 (b) of one group, 4 waves in a 2x2
// arrangement, each wave owning 128 x 128 outputs as 4x4 MFMA 32x32 tiles.
// Tokens are staged 64 at a time through LDS in [feature][token] layout (token
// contiguous, 72-element pitch), the layout the MFMA operand reads want.  Each
// thread loads an 8-token x 8-feature piece of both operands (16-byte global
// loads along the feature axis), transposes it in registers with v_perm_b32 and
// writes 16-byte rows; the B operand is scaled by s_g[t] and rounded to bf16
// before the transpose.
// ---------------------------------------------------------------------------
constexpr int FT = 256;        // tile edge
constexpr int FKC = 64;        // tokens per LDS stage
constexpr int FPITCH = 72;     // bf16 elements per LDS row (144 B: conflict-free reads and writes)
constexpr int F_STAGE_ELEMS = FT * FPITCH;               // one operand, one stage
constexpr size_t F_LDS_BYTES = (size_t)4 * F_STAGE_ELEMS * 2;  // 2 operands x 2 stages

__device__ __forceinline__ void tri_pair(int p, int T, int& ta, int& tb) {
    // p enumerates (ta <= tb) row by row: row ta holds T - ta pairs.
    int a = 0;
    while (p >= T - a) { p -= T - a; ++a; }
    ta = a;
    tb = a + p;
}

__device__ __forceinline__ void scale_piece(u32x4 (&v)[8], const float (&s)[8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float lo = __uint_as_float(v[r][k] << 16) * s[r];
            const float hi = __uint_as_float(v[r][k] & 0xffff0000u) * s[r];
            v[r][k] = pack_bf16x2(lo, hi);
        }
    }
}

// transpose an 8 (token) x 8 (feature) bf16 piece and store 8 rows of 8 tokens
__device__ __forceinline__ void store_piece_T(uint16_t* lds_rows, const u32x4 (&v)[8]) {
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        const int p = f >> 1;
        const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
        u32x4 o;
        o[0] = __builtin_amdgcn_perm(v[1][p], v[0][p], sel);
        o[1] = __builtin_amdgcn_perm(v[3][p], v[2][p], sel);
        o[2] = __builtin_amdgcn_perm(v[5][p], v[4][p], sel);
        o[3] = __builtin_amdgcn_perm(v[7][p], v[6][p], sel);
        *(u32x4*)(lds_rows + f * FPITCH) = o;
    }
}

__global__ __launch_bounds__(256, 1) void k_fisher_mfma(
    const uint16_t* __restrict__ X, const float* __restrict__ S, int64_t n, int64_t d_in,
    int groups, int T, int npairs, int nsplit, int64_t ksplit, int total_blocks,
    float* __restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) uint16_t fisher_lds[];
    // XCD-aware remap: hardware block h lands on XCD h % 8; give each XCD a
    // contiguous range of logical blocks (same split, neighbouring tiles, all groups).
    const int nb = gridDim.x;
    const int hw = blockIdx.x;
    const int lin = (hw & 7) * (nb >> 3) + (hw >> 3);
    if (lin >= total_blocks) return;
    const int g = lin % groups;
    const int pair = (lin / groups) % npairs;
    const int split = lin / (groups * npairs);
    int ta, tb;
    tri_pair(pair, T, ta, tb);
    const int64_t a0 = (int64_t)ta * FT, b0 = (int64_t)tb * FT;
    const int64_t kb = (int64_t)split * ksplit;
    const int64_t ke = (kb + ksplit < n) ? kb + ksplit : n;
    const float* __restrict__ Sg = S + (int64_t)g * n;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wa = wave & 1, wb = wave >> 1;
    const int fc = tid >> 3;     // feature group: features 8*fc .. 8*fc+7
    const int tg = tid & 7;      // token group: tokens 8*tg .. 8*tg+7

    // stage b: A operand at fisher_lds + 2b*STAGE, B operand right after it
    auto sA = [&](int b) { return fisher_lds + (2 * b) * F_STAGE_ELEMS; };
    auto sB = [&](int b) { return fisher_lds + (2 * b + 1) * F_STAGE_ELEMS; };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nchunks = (int)((ke - kb + FKC - 1) / FKC);

    // Loads use a block-uniform base pointer for the stage and 32-bit per-lane
    // byte offsets (no 64-bit address arithmetic per load, no branches).  Rows
    // past the split's end (only in its last stage) load the stage's first
    // token, a valid address, and get a zero scale; features past d_in load
    // feature 0 and are never written.
    const uint32_t fa = (uint32_t)((a0 + 8 * fc < d_in) ? a0 + 8 * fc : 0);
    const uint32_t fb = (uint32_t)((b0 + 8 * fc < d_in) ? b0 + 8 * fc : 0);
    const uint32_t row0 = (uint32_t)(8 * tg) * (uint32_t)d_in;
    u32x4 pa[8], pb[8];
    float sraw[8];
    auto fetch = [&](int c) {
        const int64_t t0 = kb + (int64_t)c * FKC;          // first token of the stage
        const char* Xs = (const char*)(X + t0 * d_in);
        const bool full = t0 + FKC <= ke;                  // block-uniform
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            uint32_t ro = row0 + (uint32_t)r * (uint32_t)d_in;
            if (!full && t0 + 8 * tg + r >= ke) ro = 0;
            pa[r] = *(const u32x4*)(Xs + 2u * (ro + fa));
            pb[r] = *(const u32x4*)(Xs + 2u * (ro + fb));
            const int64_t tk = t0 + 8 * tg + r;
            sraw[r] = Sg[(tk < ke) ? tk : t0];
        }
    };
    auto stage = [&](int c, int buf) {
        const int64_t tok0 = kb + (int64_t)c * FKC + 8 * tg;
        float sv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) sv[r] = (tok0 + r < ke) ? sraw[r] : 0.f;
        scale_piece(pb, sv);
        store_piece_T(sA(buf) + (8 * fc) * FPITCH + 8 * tg, pa);
        store_piece_T(sB(buf) + (8 * fc) * FPITCH + 8 * tg, pb);
    };

    if (nchunks > 0) {
        fetch(0);
        stage(0, 0);
    }
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        // the next stage's loads (a stage past the last one is staged but never read)
        if (c + 1 < nchunks) fetch(c + 1);
        const uint16_t* A = sA(buf);
        const uint16_t* B = sB(buf);
        // fragments of k-step ks + 1 are read from LDS while the MFMAs of k-step ks run
        bf16x8 af[2][4], bfr[2][4];
        auto read_frags = [&](int ks, int set) {
            const int koff = ks * 16 + 8 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[set][i] = as_bf16x8(*(const u32x4*)(A + (128 * wa + 32 * i + (lane & 31)) * FPITCH + koff));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[set][j] = as_bf16x8(*(const u32x4*)(B + (128 * wb + 32 * j + (lane & 31)) * FPITCH + koff));
        };
        read_frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < FKC / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < FKC / 16) read_frags(ks + 1, cur ^ 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
            if (ks + 1 < FKC / 16) {
                // interleave: 2 MFMAs, 1 LDS read, repeated
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
        }
        if (c + 1 < nchunks) stage(c + 1, buf ^ 1);
        __syncthreads();
    }

    // partial tile [256][256] row-major (a_local, b_local)
    float* P = part + (size_t)lin * (FT * FT);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int al = 128 * wa + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int bl = 128 * wb + 32 * j + (lane & 31);
                P[al * FT + bl] = acc[i][j][v];
            }
}

// Sum split partials (fixed order) and write the tile plus its mirror.
__global__ __launch_bounds__(256) void k_fisher_finalize(const float* __restrict__ part,
                                                        int64_t d_in, int groups, int T,
                                                        int npairs, int nsplit,
                                                        int accumulate, float* __restrict__ F) {
    __shared__ float sub[64][65];
    const int pair = blockIdx.x;
    const int g = blockIdx.y;
    int ta, tb;
    tri_pair(pair, T, ta, tb);
    const int tid = threadIdx.x;
    float* Fg = F + (size_t)g * d_in * d_in;
    for (int sb = 0; sb < 16; ++sb) {
        const int sr = (sb >> 2) * 64, sc = (sb & 3) * 64;
        // direct write F[a][b]
        const int col = tid & 63;
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const int r = (tid >> 6) + 4 * k;
            float v = 0.f;
            for (int s = 0; s < nsplit; ++s) {
                const size_t lin = ((size_t)s * npairs + pair) * groups + g;
                v += part[lin * (FT * FT) + (size_t)(sr + r) * FT + (sc + col)];
            }
            sub[r][col] = v;
            const int64_t a = (int64_t)ta * FT + sr + r, b = (int64_t)tb * FT + sc + col;
            if (a < d_in && b < d_in && (ta < tb || a <= b)) {
                float* dst = Fg + a * d_in + b;
                *dst = accumulate ? *dst + v : v;
            }
        }
        __syncthreads();
        // mirror write F[b][a]
        const int rr = tid & 63;
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const int cc = (tid >> 6) + 4 * k;
            const int64_t a = (int64_t)ta * FT + sr + rr, b = (int64_t)tb * FT + sc + cc;
            if (a < d_in && b < d_in && (ta < tb || a < b)) {
                float v = sub[rr][cc];
                float* dst = Fg + b * d_in + a;
                *dst = accumulate ? *dst + v : v;
            }
        }
        __syncthreads();
    }
}

// float64-accumulating path: one thread per (a, b) with a <= b.
template <bool BF16>
__global__ __launch_bounds__(256) void k_fisher_plain(const void* __restrict__ X,
                                                     const float* __restrict__ S, int64_t n,
                                                     int64_t d_in, int accumulate,
                                                     float* __restrict__ F) {
    const int64_t a = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
    const int64_t b = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    const int g = blockIdx.z;
    if (a >= d_in || b >= d_in || a > b) return;
    const float* Sg = S + (int64_t)g * n;
    double acc = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        double xa = load_elem<BF16>(X, t * d_in + a);
        double xb = load_elem<BF16>(X, t * d_in + b);
        acc += (double)Sg[t] * xa * xb;
    }
    float v = (float)acc;
    float* Fg = F + (size_t)g * d_in * d_in;
    float* d1 = Fg + a * d_in + b;
    *d1 = accumulate ? *d1 + v : v;
    if (a != b) {
        float* d2 = Fg + b * d_in + a;
        *d2 = accumulate ? *d2 + v : v;
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
struct FisherPlan {
    bool mfma;
    int T, npairs, nsplit;
    int64_t ksplit;
    int total, grid;
    size_t part_bytes;
};

FisherPlan fisher_plan(int64_t n, int64_t d_in, int groups, bool bf16) {
    FisherPlan p{};
    p.mfma = bf16 && (d_in % 8 == 0);
    if (!p.mfma) return p;
    p.T = (int)((d_in + FT - 1) / FT);
    p.npairs = p.T * (p.T + 1) / 2;
    const int tiles = p.npairs * groups;
    const int slots = 256;  // one 144 KB block per CU
    // model: time ~ ceil(tiles*s/slots) * (n/s) + s * tiles * finalize_cost
    double best = 1e300;
    int best_s = 1;
    for (int s = 1; s <= 16; ++s) {
        const int64_t chunk = ((n + s - 1) / s + FKC - 1) / FKC * FKC;
        if (s > 1 && chunk < 2048) break;
        const double rounds = (double)((tiles * (int64_t)s + slots - 1) / slots);
        // one token-step of a 256x256 block costs ~ 131072 flop; one partial tile
        // read+write in the finalize ~ 256 KB at ~5 TB/s
        const double t_main = rounds * (double)chunk * 131072.0 / (9.77e12 * 0.6);
        const double t_fin = (double)s * tiles * 262144.0 / 5e12;
        const double t = t_main + t_fin;
        if (t < best * 0.999) { best = t; best_s = s; }
    }
    p.nsplit = best_s;
    p.ksplit = ((n + best_s - 1) / best_s + FKC - 1) / FKC * FKC;
    p.total = tiles * p.nsplit;
    p.grid = (p.total + 7) / 8 * 8;
    p.part_bytes = (size_t)p.total * FT * FT * sizeof(float);
    return p;
}

size_t fisher_workspace(int64_t n, int64_t d_in, int groups, bool bf16) {
    FisherPlan p = fisher_plan(n, d_in, groups, bf16);
    size_t s_bytes = ((size_t)groups * n * sizeof(float) + 255) / 256 * 256;
    return s_bytes + (p.mfma ? p.part_bytes : 0);
}

hipError_t fisher_run(const void* X, const void* G, bool bf16, int64_t n, int64_t d_in,
                      int64_t d_out, int groups, float* F, int accumulate, void* ws,
                      hipStream_t st) {
    FisherPlan p = fisher_plan(n, d_in, groups, bf16);
    float* S = (float*)ws;
    size_t s_bytes = ((size_t)groups * n * sizeof(float) + 255) / 256 * 256;
    float* part = (float*)((char*)ws + s_bytes);
    dim3 gs((unsigned)((n + 3) / 4), (unsigned)groups);
    {
        StageTimer tm(ST_GROUP_SCALE, st);
        if (bf16)
            hipLaunchKernelGGL(k_group_scale<true>, gs, dim3(256), 0, st, G, n, d_out, groups, S);
        else
            hipLaunchKernelGGL(k_group_scale<false>, gs, dim3(256), 0, st, G, n, d_out, groups, S);
        GQ_LAUNCH_CHECK();
    }
    if (p.mfma) {
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute((const void*)k_fisher_mfma,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)F_LDS_BYTES);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        {
            StageTimer tm(ST_FISHER_MFMA, st);
            hipLaunchKernelGGL(k_fisher_mfma, dim3(p.grid), dim3(256), F_LDS_BYTES, st,
                               (const uint16_t*)X, S, n, d_in, groups, p.T, p.npairs, p.nsplit,
                               p.ksplit, p.total, part);
            GQ_LAUNCH_CHECK();
        }
        StageTimer tm(ST_FISHER_FINALIZE, st);
        hipLaunchKernelGGL(k_fisher_finalize, dim3(p.npairs, groups), dim3(256), 0, st, part,
                           d_in, groups, p.T, p.npairs, p.nsplit, accumulate, F);
        GQ_LAUNCH_CHECK();
    } else {
        dim3 gp((unsigned)((d_in + 15) / 16), (unsigned)((d_in + 15) / 16), (unsigned)groups);
        StageTimer tm(ST_FISHER_PLAIN, st);
        if (bf16)
            hipLaunchKernelGGL(k_fisher_plain<true>, gp, dim3(256), 0, st, X, S, n, d_in,
                               accumulate, F);
        else
            hipLaunchKernelGGL(k_fisher_plain<false>, gp, dim3(256), 0, st, X, S, n, d_in,
                               accumulate, F);
        GQ_LAUNCH_CHECK();
    }
    return hipSuccess;
}

}  // namespace gq
