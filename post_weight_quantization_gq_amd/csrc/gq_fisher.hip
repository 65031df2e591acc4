// Grouped Fisher blocks for GuidedQuant on gfx950.
//
// GuidedQuant blog page (jinukkim.me/blog/guidedquant), objective equation and
// the sentence after it: per-output-channel Fisher blocks F_j = X^T diag(G_:j^2) X
// are grouped and averaged within each group.  By linearity the group average is
// F_g = X^T diag(s_g) X with s_g[t] = mean_{j in g} G[t, j]^2.
//
// Kernels
//   k_group_scale     s_g[t] for every token (HBM stream over G).
//   k_fisher_pack     packs X feature-major (XT) and, per group, the scaled copy
//                     YT[g] = (s_g * X)^T in bf16, zero-padded to whole tiles.
//   k_fisher_mfma     bf16 MFMA (v_mfma_f32_32x32x16_bf16) contraction XT YT[g]^T over
//                     tokens for the upper-triangle 256x256 tiles of every F_g;
//                     tokens may be split across blocks (split-K) to fill the chip,
//                     each split writing its own partial tile.
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
// Operand packing.  The contraction reads both operands feature-major with tokens
// contiguous, the layout the MFMA operand fragments want, blocked by 32 tokens:
//     XT[t/32][a][t%32]    = X[t][a]
//     YT[g][t/32][a][t%32] = bf16(s_g[t] * X[t][a])   (float32 product, one rounding)
// so that the 256 feature rows of one 32-token stage of a tile are 16 KB of
// contiguous memory.  Features are padded with zero rows to a multiple of 256 and
// tokens with zeros to a multiple of 64, so every tile and stage is whole.  One
// block per 64-token x 64-feature tile: 16-byte loads along the features into
// LDS, then 16-byte stores of 8 consecutive tokens per feature.
// ---------------------------------------------------------------------------
constexpr int PK = 64;
constexpr int PK_G = 16;       // groups whose scales are staged in LDS at a time

// element offset of (token t, feature a) in a blocked operand (t % 8 == 0 here)
__device__ __forceinline__ int64_t blk_off(int64_t t, int64_t a, int64_t d_pad) {
    return ((t >> 5) * d_pad + a) * 32 + (t & 31);
}

__global__ __launch_bounds__(256) void k_fisher_pack(const uint16_t* __restrict__ X,
                                                    const float* __restrict__ S, int64_t n,
                                                    int64_t n_pad, int64_t d, int64_t d_pad,
                                                    int groups, uint16_t* __restrict__ XT,
                                                    uint16_t* __restrict__ YT) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[PK][PK + 8];   // [token][feature]
    __shared__ __attribute__((aligned(16))) float ss[PK_G][PK];          // s_g[t0 + t]
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * PK;
    const int64_t f0 = (int64_t)blockIdx.y * PK;
    const int fc = tid & 7;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = (tid >> 3) + 32 * h;
        const int64_t t = t0 + r, f = f0 + 8 * fc;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (t < n && f < d) v = *(const u32x4*)(X + t * d + f);     // d % 8 == 0
        *(u32x4*)&tile[r][8 * fc] = v;
    }
    __syncthreads();
    const int c = tid & 7;                 // token chunk: tokens t0 + 8c .. + 7
    const int64_t col = t0 + 8 * c;
    uint32_t xs[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int a = (tid >> 3) + 32 * h;
#pragma unroll
        for (int k = 0; k < 8; ++k) xs[h][k] = tile[8 * c + k][a];
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = xs[h][2 * k] | (xs[h][2 * k + 1] << 16);
        *(u32x4*)(XT + blk_off(col, f0 + a, d_pad)) = o;     // f0 + a < d_pad: whole 64-tiles
    }
    for (int g0 = 0; g0 < groups; g0 += PK_G) {
        const int gn = (groups - g0) < PK_G ? (groups - g0) : PK_G;
        __syncthreads();
        for (int e = tid; e < gn * PK; e += 256) {
            const int gi = e / PK, tt = e - gi * PK;
            ss[gi][tt] = (t0 + tt < n) ? S[(int64_t)(g0 + gi) * n + t0 + tt] : 0.f;
        }
        __syncthreads();
        for (int gi = 0; gi < gn; ++gi) {
            const float4 s_lo = *(const float4*)&ss[gi][8 * c];
            const float4 s_hi = *(const float4*)&ss[gi][8 * c + 4];
            const float sv[8] = {s_lo.x, s_lo.y, s_lo.z, s_lo.w, s_hi.x, s_hi.y, s_hi.z, s_hi.w};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int a = (tid >> 3) + 32 * h;
                u32x4 y;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    y[k] = pack_bf16x2(__uint_as_float(xs[h][2 * k] << 16) * sv[2 * k],
                                       __uint_as_float(xs[h][2 * k + 1] << 16) * sv[2 * k + 1]);
                *(u32x4*)(YT + (int64_t)(g0 + gi) * d_pad * n_pad + blk_off(col, f0 + a, d_pad)) = y;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA Fisher: upper-triangle 256 (a) x 256 (b) tiles of F_g = XT YT[g]^T.
// 8 waves (two per SIMD, so one covers the other's barrier and LDS waits) in a
// 2 (a) x 4 (b) arrangement, each owning 128 x 64 outputs as 4x2
// v_mfma_f32_32x32x16_bf16 tiles (128 accumulator registers of a lane).
// Tokens are staged 32 at a time in a ring of 4 LDS stages (4 x 32 KB), filled by
// direct buffer-to-LDS loads issued three stages ahead, so no staging registers
// and no LDS stores are needed.  An operand row of a stage is 64 bytes of the
// blocked XT or YT, kept as four 16-byte slots; chunk c of row r sits in slot
// r*4 + (c ^ ((r >> 2) & 3)).  Each load instruction fills 16 whole rows (1 KB
// of consecutive LDS), and a fragment read (one chunk of 16 consecutive rows per
// quarter-wave) touches 16 distinct 16-byte bank groups.  One barrier per stage.
// ---------------------------------------------------------------------------
constexpr int FT = 256;        // tile edge
constexpr int FKC = 32;        // tokens per LDS stage
constexpr int FRING = 4;       // LDS stages in flight (4 x 32 KB = 128 KB)
constexpr int F_SLOTS = FT * 4;                                     // 16-byte slots, one operand, one stage
constexpr size_t F_LDS_BYTES = (size_t)FRING * 2 * F_SLOTS * 16;

// Pairs (ta <= tb) are enumerated column by column (column tb holds tb + 1 pairs),
// so consecutive logical blocks share the b band, the per-group operand, and
// differ in the a band, which all groups share.
__device__ __forceinline__ void tri_pair(int p, int T, int& ta, int& tb) {
    int b = 0;
    while (p > b) { p -= b + 1; ++b; }
    (void)T;
    ta = p;
    tb = b;
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_fisher_mfma(
    const uint16_t* __restrict__ XT, const uint16_t* __restrict__ YT, int64_t n_pad,
    int64_t d_pad, int groups, int T, int npairs, int64_t ksplit, int total_blocks,
    float* __restrict__ part) {
    extern __shared__ u32x4 fisher_lds[];
    // XCD-aware remap: hardware block h lands on XCD h % 8.  Within each round of
    // 256 blocks, XCD x takes 32 consecutive logical blocks (neighbouring tile pairs,
    // all groups: their bands meet in its L2), and a round covers consecutive logical
    // blocks, so all XCDs stream the same token split at once (shared in the MALL).
    const int hw = blockIdx.x;
    const int lin = (hw & ~255) + (hw & 7) * 32 + ((hw & 255) >> 3);
    if (lin >= total_blocks) return;
    const int g = lin % groups;
    const int pair = (lin / groups) % npairs;
    const int split = lin / (groups * npairs);
    int ta, tb;
    tri_pair(pair, T, ta, tb);
    const int64_t kb = (int64_t)split * ksplit;
    const int64_t ke = (kb + ksplit < n_pad) ? kb + ksplit : n_pad;
    const int nst = kb < ke ? (int)((ke - kb) / FKC) : 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the LDS targets go to M0
    const int wa = wave & 1, wb = wave >> 1;   // wa 0..1 (128 rows), wb 0..3 (64 columns)

    // A stage of the a band is 256 rows x 64 bytes, contiguous in the blocked XT
    // (likewise the b band in YT[g]).  Load instruction k of a wave fills rows
    // 16q .. 16q + 15 (q = 8k + wave): lane L takes row 16q + L/4 and slot L%4,
    // i.e. chunk (L%4) ^ ((L/16)%4), at byte 1024 q + 64 (L/4) + 16 chunk of the
    // stage: a per-lane vector offset plus a uniform scalar offset, against a
    // buffer descriptor rebuilt per stage (scalar arithmetic only).
    const uint16_t* Abase = XT + ((kb >> 5) * d_pad + (int64_t)ta * FT) * 32;
    const uint16_t* Bbase = YT + (int64_t)g * d_pad * n_pad + ((kb >> 5) * d_pad + (int64_t)tb * FT) * 32;
    const int64_t stage_elems = d_pad * 32;
    const uint32_t voff = (uint32_t)(lane >> 2) * 64u +
                          16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));

    auto sA = [&](int st) { return fisher_lds + st * (2 * F_SLOTS); };
    auto sB = [&](int st) { return fisher_lds + st * (2 * F_SLOTS) + F_SLOTS; };

    auto issue = [&](int s) {
        const int st = s % FRING;
        const __amdgpu_buffer_rsrc_t Ar = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Abase + (int64_t)s * stage_elems), (short)0, F_SLOTS * 16, 0x00020000);
        const __amdgpu_buffer_rsrc_t Br = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Bbase + (int64_t)s * stage_elems), (short)0, F_SLOTS * 16, 0x00020000);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = 8 * k + wave;
            const uint32_t so = (uint32_t)q * 1024u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Ar, (lds_ptr_t)(sA(st) + 64 * q), 16, voff, so, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Br, (lds_ptr_t)(sB(st) + 64 * q), 16, voff, so, 0, 0);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int sw = (lane >> 2) & 3;      // slot swizzle of the fragment rows
    // wait until stage `want` has landed, given stages up to `last` issued
    auto wait_stage = [&](int want, int last) {
        const int newer = last - want;
        if (newer >= 4) wait_vmcnt<16>();
        else if (newer == 3) wait_vmcnt<12>();
        else if (newer == 2) wait_vmcnt<8>();
        else if (newer == 1) wait_vmcnt<4>();
        else wait_vmcnt<0>();
    };
    {
        const int pre = nst < FRING - 1 ? nst : FRING - 1;
        for (int s = 0; s < pre; ++s) issue(s);
    }
    int slot = 0;                        // ring slot of stage s
    for (int s = 0; s < nst; ++s) {
        // this wave's loads of stage s are done (4 per stage and wave; later stages
        // may still be in flight), then every wave's are
        const int last = (s + FRING - 2 < nst) ? s + FRING - 2 : nst - 1;
        wait_stage(s, last);
        __builtin_amdgcn_s_barrier();
        // every wave has finished stage s - 1: its slot of the ring takes stage s + FRING - 1
        if (s + FRING - 1 < nst) issue(s + FRING - 1);
        const u32x4* A = fisher_lds + slot * (2 * F_SLOTS);
        const u32x4* B = A + F_SLOTS;
        bf16x8 af[2][4], bfr[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int cs = (2 * ks + (lane >> 5)) ^ sw;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[ks][i] = as_bf16x8(A[(128 * wa + 32 * i + (lane & 31)) * 4 + cs]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[ks][j] = as_bf16x8(B[(64 * wb + 32 * j + (lane & 31)) * 4 + cs]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        slot = (slot + 1 == FRING) ? 0 : slot + 1;
    }

    // partial tile [256][256] row-major (a_local, b_local)
    float* P = part + (size_t)lin * (FT * FT);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int al = 128 * wa + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int bl = 64 * wb + 32 * j + (lane & 31);
                P[al * FT + bl] = acc[i][j][v];
            }
}

// Sum split partials (fixed order) and write the tile plus its mirror.  One block
// per 64 x 64 sub-tile of a (pair, group): each thread sums 4 rows x 4 columns
// with float4 loads, writes F[a][b] and, through LDS, the mirror F[b][a] with
// float4 stores (d_in % 8 == 0 on this path, F 16-byte aligned).
__global__ __launch_bounds__(256) void k_fisher_finalize(const float* __restrict__ part,
                                                        int64_t d_in, int groups, int T,
                                                        int npairs, int nsplit,
                                                        int accumulate, float* __restrict__ F) {
    __shared__ float sub[64][65];
    const int pair = blockIdx.x >> 4;
    const int sbk = blockIdx.x & 15;
    const int g = blockIdx.y;
    int ta, tb;
    tri_pair(pair, T, ta, tb);
    const int sr = (sbk >> 2) * 64, sc = (sbk & 3) * 64;
    const int64_t a0 = (int64_t)ta * FT + sr, b0 = (int64_t)tb * FT + sc;
    if (a0 >= d_in || b0 >= d_in) return;
    if (ta == tb && sr > sc) return;                 // strictly below the diagonal
    const int tid = threadIdx.x;
    const int c4 = (tid & 15) * 4;
    float* Fg = F + (size_t)g * d_in * d_in;
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < nsplit; ++s) {
        const size_t lin = ((size_t)s * npairs + pair) * groups + g;
        const float* P = part + lin * (FT * FT) + (size_t)sr * FT + sc + c4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 x = *(const float4*)(P + (size_t)((tid >> 4) + 16 * k) * FT);
            v[k].x += x.x; v[k].y += x.y; v[k].z += x.z; v[k].w += x.w;
        }
    }
    const bool diag = (ta == tb) && (sr == sc);      // a <= b needed per element
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = (tid >> 4) + 16 * k;
        sub[r][c4] = v[k].x; sub[r][c4 + 1] = v[k].y; sub[r][c4 + 2] = v[k].z; sub[r][c4 + 3] = v[k].w;
        const int64_t a = a0 + r, b = b0 + c4;
        if (a >= d_in || b >= d_in) continue;        // d_in % 8 == 0: b + 3 < d_in too
        float* dst = Fg + a * d_in + b;
        if (!diag) {
            float4 o = v[k];
            if (accumulate) {
                const float4 y = *(const float4*)dst;
                o.x += y.x; o.y += y.y; o.z += y.z; o.w += y.w;
            }
            *(float4*)dst = o;
        } else {
            const float e[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (a <= b + q) dst[q] = accumulate ? dst[q] + e[q] : e[q];
        }
    }
    __syncthreads();
    // mirror: F[b][a] for a < b
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int rb = (tid >> 4) + 16 * k;         // b offset
        const int64_t b = b0 + rb, a = a0 + c4;
        if (a >= d_in || b >= d_in) continue;
        float* dst = Fg + b * d_in + a;
        const float e[4] = {sub[c4][rb], sub[c4 + 1][rb], sub[c4 + 2][rb], sub[c4 + 3][rb]};
        if (!diag) {
            float4 o = make_float4(e[0], e[1], e[2], e[3]);
            if (accumulate) {
                const float4 y = *(const float4*)dst;
                o.x += y.x; o.y += y.y; o.z += y.z; o.w += y.w;
            }
            *(float4*)dst = o;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (a + q < b) dst[q] = accumulate ? dst[q] + e[q] : e[q];
        }
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
    int64_t n;                 // tokens per pass (the call's n, or the pass limit)
    int64_t n_pad, d_pad;
    int T, npairs, nsplit;
    int64_t ksplit;
    int total, grid;
    size_t s_bytes, xt_bytes, yt_bytes, part_bytes;
};

// The packed operands take (1 + groups) * d_pad * n_pad * 2 bytes.  Token ranges
// whose packed operands would exceed this budget run as several passes, each
// adding into F.
constexpr size_t F_PACK_BUDGET = (size_t)16 << 30;

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

FisherPlan fisher_plan(int64_t n_call, int64_t d_in, int groups, bool bf16,
                       int max_split = 16) {
    FisherPlan p{};
    p.mfma = bf16 && (d_in % 8 == 0);
    {
        const int64_t d_pad = (d_in + FT - 1) / FT * FT;
        int64_t cap = (int64_t)(F_PACK_BUDGET / ((size_t)(1 + groups) * d_pad * 2)) / PK * PK;
        if (cap < PK) cap = PK;
        p.n = (bf16 && d_in % 8 == 0 && n_call > cap) ? cap : n_call;
    }
    p.s_bytes = al256((size_t)groups * p.n * sizeof(float));
    if (!p.mfma) return p;
    p.n_pad = (p.n + PK - 1) / PK * PK;            // the packing tile
    p.T = (int)((d_in + FT - 1) / FT);
    p.d_pad = (int64_t)p.T * FT;
    p.npairs = p.T * (p.T + 1) / 2;
    const int tiles = p.npairs * groups;
    const int slots = 256;  // one 128 KB block per CU
    // model: time ~ ceil(tiles*s/slots) * (n/s) + s * tiles * finalize_cost
    double best = 1e300;
    int best_s = 1;
    for (int s = 1; s <= max_split; ++s) {
        const int64_t chunk = ((p.n_pad + s - 1) / s + FKC - 1) / FKC * FKC;
        if (s > 1 && chunk < 2048) break;
        const double rounds = (double)((tiles * (int64_t)s + slots - 1) / slots);
        // one token-step of a 256x256 block costs 131072 flop at ~60 % of a CU's
        // bf16 peak; one partial tile read + write in the finalize ~256 KB at ~5 TB/s
        const double t_main = rounds * (double)chunk * 131072.0 / (9.77e12 * 0.6);
        const double t_fin = (double)s * tiles * 262144.0 / 5e12;
        const double t = t_main + t_fin;
        if (t < best * 0.999) { best = t; best_s = s; }
    }
    p.nsplit = best_s;
    p.ksplit = ((p.n_pad + best_s - 1) / best_s + FKC - 1) / FKC * FKC;
    p.total = tiles * p.nsplit;
    p.grid = (p.total + 255) / 256 * 256;         // whole rounds for the remap
    p.xt_bytes = al256((size_t)p.d_pad * p.n_pad * 2);
    p.yt_bytes = al256((size_t)groups * p.d_pad * p.n_pad * 2);
    p.part_bytes = (size_t)p.total * FT * FT * sizeof(float);
    return p;
}

size_t fisher_workspace(int64_t n, int64_t d_in, int groups, bool bf16) {
    FisherPlan p = fisher_plan(n, d_in, groups, bf16);
    return p.s_bytes + (p.mfma ? p.xt_bytes + p.yt_bytes + p.part_bytes : 0);
}

static hipError_t fisher_pass(const FisherPlan& p, const void* X, const void* G, bool bf16,
                              int64_t n, int64_t d_in, int64_t d_out, int groups, float* F,
                              int accumulate, void* ws, hipStream_t st) {
    float* S = (float*)ws;
    char* w = (char*)ws + p.s_bytes;
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
        uint16_t* XT = (uint16_t*)w;
        uint16_t* YT = (uint16_t*)(w + p.xt_bytes);
        float* part = (float*)(w + p.xt_bytes + p.yt_bytes);
        const int64_t n_pad = (n + PK - 1) / PK * PK;
        {
            hipError_t e = ensure_dynamic_lds((const void*)k_fisher_mfma, F_LDS_BYTES);
            if (e != hipSuccess) return e;
        }
        {
            StageTimer tm(ST_FISHER_PACK, st);
            dim3 gp((unsigned)(n_pad / PK), (unsigned)(p.d_pad / PK));
            hipLaunchKernelGGL(k_fisher_pack, gp, dim3(256), 0, st, (const uint16_t*)X, S, n,
                               n_pad, d_in, p.d_pad, groups, XT, YT);
            GQ_LAUNCH_CHECK();
        }
        // the split plan of this pass's token count (no more partial tiles than the
        // workspace holds)
        const FisherPlan q = fisher_plan(n, d_in, groups, bf16, p.nsplit);
        {
            StageTimer tm(ST_FISHER_MFMA, st);
            hipLaunchKernelGGL(k_fisher_mfma, dim3(q.grid), dim3(512), F_LDS_BYTES, st, XT, YT,
                               n_pad, q.d_pad, groups, q.T, q.npairs, q.ksplit, q.total, part);
            GQ_LAUNCH_CHECK();
        }
        StageTimer tm(ST_FISHER_FINALIZE, st);
        hipLaunchKernelGGL(k_fisher_finalize, dim3(q.npairs * 16, groups), dim3(256), 0, st, part,
                           d_in, groups, q.T, q.npairs, q.nsplit, accumulate, F);
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

hipError_t fisher_run(const void* X, const void* G, bool bf16, int64_t n, int64_t d_in,
                      int64_t d_out, int groups, float* F, int accumulate, void* ws,
                      hipStream_t st) {
    const FisherPlan p = fisher_plan(n, d_in, groups, bf16);
    const size_t esz = bf16 ? 2 : 4;
    for (int64_t t0 = 0; t0 < n; t0 += p.n) {
        const int64_t nt = (n - t0) < p.n ? (n - t0) : p.n;
        hipError_t e = fisher_pass(p, (const char*)X + (size_t)t0 * d_in * esz,
                                   (const char*)G + (size_t)t0 * d_out * esz, bf16, nt, d_in,
                                   d_out, groups, F, (t0 > 0) ? 1 : accumulate, ws, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gq
