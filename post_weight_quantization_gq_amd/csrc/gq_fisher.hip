// Grouped Fisher blocks for GuidedQuant on gfx950.
//
// GuidedQuant blog page (jinukkim.me/blog/guidedquant), objective equation and
// the sentence after it: per-output-channel Fisher blocks F_j = X^T diag(G_:j^2) X
// are grouped and averaged within each group.  By linearity the group average is
// F_g = X^T diag(s_g) X with s_g[t] = mean_{j in g} G[t, j]^2.
//
// Kernels
//   k_group_scale     s_g[t] for every token (HBM stream over G), zero past the last.
//   k_fisher_pack     packs X feature-major (XT) in bf16, zero-padded to whole tiles.
//   k_fisher_mfma_g4  group counts that are multiples of 4: bf16 MFMA
//                     (v_mfma_f32_32x32x16_bf16) contraction over tokens for the
//                     upper-triangle 128x128 tiles of the four F_g of a quad at once,
//                     from one unscaled XT band pair in LDS; s_g is applied to the b
//                     fragment in registers (bf16(s_g[t] X[t][b]), one rounding of the
//                     float32 product).
//   k_fisher_mfma     other group counts: the upper-triangle 256x256 tiles of one F_g
//                     per block, the b band scaled by s_g on its way into LDS.
//                     Either contraction may split tokens across blocks (split-K) to
//                     fill the chip, each split writing its own partial tiles.
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
// S is [groups][pitch], or with quad set [groups / 4][pitch][4] (the four groups of a
// quad side by side per token); tokens n .. pitch - 1 get 0 (the padding of the packed
// operand).
template <bool BF16>
__global__ __launch_bounds__(256) void k_group_scale(const void* __restrict__ G, int64_t n,
                                                      int64_t d_out, int groups, int64_t pitch,
                                                      int quad, float* __restrict__ S) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int g = blockIdx.y;
    if (t >= pitch) return;
    const int64_t at = quad ? ((int64_t)(g >> 2) * pitch + t) * 4 + (g & 3) : (int64_t)g * pitch + t;
    if (t >= n) {
        if (lane == 0) S[at] = 0.f;
        return;
    }
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
    if (lane == 0) S[at] = acc / (float)size;
}

// ---------------------------------------------------------------------------
// Operand packing.  The contraction reads the activations feature-major with tokens
// contiguous, the layout the MFMA operand fragments want, blocked by 32 tokens:
//     XT[t/32][a][t%32] = X[t][a]
// so that the 256 feature rows of one 32-token stage of a tile are 16 KB of
// contiguous memory.  Features are padded with zero rows to a multiple of 256 and
// tokens with zeros to a multiple of 64, so every tile and stage is whole.  One
// block per 64-token x 64-feature tile: 16-byte loads along the features into
// LDS, then 16-byte stores of 8 consecutive tokens per feature.
// ---------------------------------------------------------------------------
constexpr int PK = 64;

// element offset of (token t, feature a) in a blocked operand (t % 8 == 0 here)
__device__ __forceinline__ int64_t blk_off(int64_t t, int64_t a, int64_t d_pad) {
    return ((t >> 5) * d_pad + a) * 32 + (t & 31);
}

__global__ __launch_bounds__(256) void k_fisher_pack(const uint16_t* __restrict__ X, int64_t n,
                                                    int64_t d, int64_t d_pad,
                                                    uint16_t* __restrict__ XT) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[PK][PK + 8];   // [token][feature]
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
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int a = (tid >> 3) + 32 * h;
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o[k] = (uint32_t)tile[8 * c + 2 * k][a] | ((uint32_t)tile[8 * c + 2 * k + 1][a] << 16);
        *(u32x4*)(XT + blk_off(col, f0 + a, d_pad)) = o;     // f0 + a < d_pad: whole 64-tiles
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA Fisher: upper-triangle 256 (a) x 256 (b) tiles of F_g = XT (s_g XT)^T.
// 8 waves (two per SIMD, so one covers the other's barrier and LDS waits) in a
// 2 (a) x 4 (b) arrangement, each owning 128 x 64 outputs as 4x2
// v_mfma_f32_32x32x16_bf16 tiles (128 accumulator registers of a lane).
// Tokens are staged 32 at a time in a ring of 4 LDS stages (4 x 32 KB), filled three
// stages ahead.  An operand row of a stage is 64 bytes of the blocked XT, kept as four
// 16-byte slots; chunk c of row r sits in slot r*4 + (c ^ ((r >> 2) & 3)), so a
// fragment read (one chunk of 16 consecutive rows per quarter-wave) touches 16
// distinct 16-byte bank groups.  The a band arrives by direct buffer-to-LDS loads
// (each instruction fills 16 whole rows, 1 KB of consecutive LDS).  The b band is
// the gradient-scaled operand, formed on the way in: each thread loads 16 tokens of
// one feature row of XT and the 16 scales s_g[t] into registers five stages ahead,
// and writes bf16(s_g[t] X[t][b]) into the ring three stages ahead, so no scaled copy
// of the activations ever exists in memory.  One barrier per stage.
// ---------------------------------------------------------------------------
constexpr int FT = 256;        // tile edge
constexpr int FKC = 32;        // tokens per LDS stage
constexpr int FRING = 4;       // LDS stages in flight (4 x 32 KB = 128 KB)
constexpr int F_SLOTS = FT * 4;                                     // 16-byte slots, one operand, one stage
constexpr size_t F_LDS_BYTES = (size_t)FRING * 2 * F_SLOTS * 16;
static_assert(PK % (2 * FKC) == 0, "padded token counts must be whole pairs of stages");

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

// wait until at most N vector-memory operations and no LDS operation of this wave
// are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// 16 consecutive tokens of one feature row of XT and their 16 scales s_g[t]
struct FisherBStage {
    u32x4 x[2];      // one feature row, 16 tokens
    float s;         // lane L: the scale of token L % 16 of those (the same for every row)
};

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_fisher_mfma(
    const uint16_t* __restrict__ XT, const float* __restrict__ S, int64_t n_pad,
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

    // A stage of a band is 256 rows x 64 bytes, contiguous in the blocked XT.  a band:
    // load instruction k of a wave fills rows 16q .. 16q + 15 (q = 8k + wave): lane L
    // takes row 16q + L/4 and slot L%4, i.e. chunk (L%4) ^ ((L/16)%4), at byte
    // 1024 q + 64 (L/4) + 16 chunk of the stage: a per-lane vector offset plus a
    // uniform scalar offset, against a buffer descriptor rebuilt per stage.
    const uint16_t* Abase = XT + ((kb >> 5) * d_pad + (int64_t)ta * FT) * 32;
    const uint16_t* Bbase = XT + ((kb >> 5) * d_pad + (int64_t)tb * FT) * 32;
    const float* Sg = S + (int64_t)g * n_pad + kb;      // scales of this split's tokens
    const int64_t stage_elems = d_pad * 32;
    const uint32_t voff = (uint32_t)(lane >> 2) * 64u +
                          16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));

    auto sA = [&](int st) { return fisher_lds + st * (2 * F_SLOTS); };
    auto sB = [&](int st) { return fisher_lds + st * (2 * F_SLOTS) + F_SLOTS; };

    // Every iteration issues the same operations, so the wait counts below hold at
    // every stage: loads of stages past the last read the last stage again (their
    // ring slots are never read), and nst is even (splits are whole 64-token steps).
    auto clamp = [&](int s) { return s < nst ? s : nst - 1; };
    auto issue_a = [&](int s) {
        const int st = s % FRING;
        const __amdgpu_buffer_rsrc_t Ar = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Abase + (int64_t)clamp(s) * stage_elems), (short)0, F_SLOTS * 16, 0x00020000);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = 8 * k + wave;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Ar, (lds_ptr_t)(sA(st) + 64 * q), 16, voff,
                                                     (uint32_t)q * 1024u, 0, 0);
        }
    };
    // b band: wave w takes tokens 16 bh .. 16 bh + 15 (bh = w % 2, chunks 2 bh and
    // 2 bh + 1) of rows 64 (w / 2) .. + 63, one row per lane, so the 16 scales are
    // the same for the whole wave: one load spreads them over lanes 0..15 (and again
    // over 16..63), and each is broadcast from its lane when the band is written
    const int bh = wave & 1;
    const int br = (wave >> 1) * 64 + lane;
    const int bsw = (br >> 2) & 3;
    auto load_b = [&](int s, FisherBStage& b) {
        const int sc = clamp(s);
        const uint16_t* src = Bbase + (int64_t)sc * stage_elems + br * 32 + 16 * bh;
        b.x[0] = *(const u32x4*)src;
        b.x[1] = *(const u32x4*)(src + 8);
        b.s = Sg[32 * (int64_t)sc + 16 * bh + (lane & 15)];
    };
    auto write_b = [&](int s, const FisherBStage& b) {
        u32x4* dst = sB(s % FRING);
        float sv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            sv[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b.s), k));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4 y;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t xw = b.x[c][k];
                y[k] = pack_bf16x2(__uint_as_float(xw << 16) * sv[8 * c + 2 * k],
                                   __uint_as_float(xw & 0xffff0000u) * sv[8 * c + 2 * k + 1]);
            }
            dst[br * 4 + ((2 * bh + c) ^ bsw)] = y;
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
    // Vector-memory operations of iteration s, in issue order: the a band of stage
    // s + 3 (2), then the b band of stage s + 5 (3); the prologue issues the a bands of
    // stages 1 and 2 and the b bands of stages 3 and 4 in the same interleaving.  So
    // when iteration s writes the b band of stage s + 3, at most 5 operations issued
    // after its loads (a band s + 2, b band s + 4) may be outstanding, and waiting for
    // it also completes the a band of stage s + 1 for the next iteration's barrier.
    FisherBStage b_odd, b_even;          // b band of stages x in registers: odd x, even x
    if (nst > 0) {
        issue_a(0);
#pragma unroll
        for (int s = 0; s < FRING - 1; ++s) {
            load_b(s, b_even);
            wait_vmcnt<0>();
            write_b(s, b_even);
        }
        issue_a(1);
        load_b(3, b_odd);
        issue_a(2);
        load_b(4, b_even);
    }
    // Iteration s writes the b band of stage s + 3 and loads that of stage s + 5: the
    // same parity, so one register buffer per iteration (odd s + 3 for even s).
    auto iteration = [&](int s, FisherBStage& bb) {
        const int slot = s % FRING;
        wait_vmcnt_lds<63>();            // this wave's LDS writes of the b band are done
        __builtin_amdgcn_s_barrier();
        // every wave has finished stage s - 1: its slot of the ring takes stage s + 3,
        // and every wave's a and b bands of stage s are in LDS
        wait_vmcnt<5>();
        write_b(s + FRING - 1, bb);
        issue_a(s + FRING - 1);
        load_b(s + FRING + 1, bb);
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
    };
    for (int s = 0; s < nst; s += 2) {
        iteration(s, b_odd);
        iteration(s + 1, b_even);
    }
    wait_vmcnt<0>();     // no load into this block's LDS may land after it ends

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

// ---------------------------------------------------------------------------
// bf16 MFMA Fisher, four groups per block: 128 (a) x 128 (b) tiles of F_g for the four
// groups g of a quad, from one unscaled XT band pair.  The scales are applied to the b
// operand in registers, so the bands are fetched once for four groups: half the LDS
// fill and L2 traffic of one 256 x 256 tile per group, and a third of the LDS
// fragment reads, for the same flops.
//   4 waves (one per SIMD); wave w owns the 128 a rows x b columns 32w .. 32w + 31 of
//   all four groups: 4 (groups) x 4 (a blocks of 32) v_mfma_f32_32x32x16_bf16
//   accumulators, 256 registers.
//   A ring of 8 LDS stages of 32 tokens; a stage holds the a band and the b band
//   (128 rows x 64 bytes each, the slot swizzle of the 256-tile kernel) and the
//   quad's scales of its 32 tokens (512 bytes), all filled by direct buffer-to-LDS
//   loads seven stages ahead.
//   The b fragment of a lane holds 8 consecutive tokens, the same 8 for a half-wave.
//   The scale vector of a lane holds s of token 16 ks + 8 h + e in lane
//   16 (2 h + r) + 8 ks + e (r = 0, 1), so each lane's scale for element e of step ks
//   is that of lane 8 ks + e of its row of 16: a DPP row broadcast folded into the
//   multiply, bf16(s_g[t] X[t][b]) with one float32 product as in the other kernel.
//   Per stage: the first 16-token half's MFMAs, then the barrier that frees the
//   stage's slot and publishes the next stage, the refill of the slot and the next
//   stage's fragment reads, then the second half's MFMAs, so the reads land while the
//   matrix cores work.
// ---------------------------------------------------------------------------
constexpr int G4_TE = 128;                     // tile edge
constexpr int G4_RING = 8;                     // LDS stages
constexpr int G4_BAND = G4_TE * 4;             // 16-byte slots of one band-stage (8 KB)
constexpr int G4_SLOT = 2 * G4_BAND + 32;      // a band, b band, 32 tokens x 4 scales
constexpr size_t G4_LDS_BYTES = (size_t)G4_RING * G4_SLOT * 16;
constexpr int G4_VM_PER_STAGE = 5;             // per wave: 2 (a) + 2 (b) + 1 (scales)

// Pairs (ta <= tb) of 128-tiles in panels of 4 tile columns: within a panel, row by
// row (ta), so the 32 consecutive logical blocks one XCD runs at once span about 8 a
// bands and 4 b bands.
__device__ __forceinline__ void panel_pair(int p, int T, int& ta, int& tb) {
    for (int c0 = 0;; c0 += 4) {
        const int nc = (T - c0) < 4 ? (T - c0) : 4;
        const int full = nc * c0;                      // rows above the panel's diagonal
        const int cnt = full + nc * (nc + 1) / 2;
        if (p < cnt) {
            if (p < full) {
                ta = p / nc;
                tb = c0 + p % nc;
            } else {
                int q = p - full, i = 0;
                while (q >= nc - i) { q -= nc - i; ++i; }
                ta = c0 + i;
                tb = c0 + i + q;
            }
            return;
        }
        p -= cnt;
    }
}

// lane broadcast within each row of 16 lanes (DPP row_newbcast)
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + N, 0xf, 0xf, true));
}

// the b fragment of a 16-token step as 8 floats (tokens 2k, 2k + 1 in word k)
__device__ __forceinline__ void g4_unpack(u32x4 bx, float (&xf)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        xf[2 * k] = __uint_as_float(bx[k] << 16);
        xf[2 * k + 1] = __uint_as_float(bx[k] & 0xffff0000u);
    }
}

// bf16(s_g[t] X[t][b]) for the 8 tokens of step KS, sg the group's scale vector
template <int KS>
__device__ __forceinline__ bf16x8 g4_scale(const float (&xf)[8], float sg) {
    u32x4 y;
    y[0] = pack_bf16x2(xf[0] * row_bcast<8 * KS + 0>(sg), xf[1] * row_bcast<8 * KS + 1>(sg));
    y[1] = pack_bf16x2(xf[2] * row_bcast<8 * KS + 2>(sg), xf[3] * row_bcast<8 * KS + 3>(sg));
    y[2] = pack_bf16x2(xf[4] * row_bcast<8 * KS + 4>(sg), xf[5] * row_bcast<8 * KS + 5>(sg));
    y[3] = pack_bf16x2(xf[6] * row_bcast<8 * KS + 6>(sg), xf[7] * row_bcast<8 * KS + 7>(sg));
    return as_bf16x8(y);
}

__device__ __forceinline__ void g4_mfma(f32x16 (&acc)[4], const u32x4 (&a)[4], bf16x8 b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), b, acc[i], 0, 0, 0);
}

// ask the scheduler to alternate one MFMA with a few VALU operations over a region of
// 16 MFMAs, so the scaling of the next group runs while the matrix core works
__device__ __forceinline__ void g4_interleave() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // up to five VALU
    }
}

struct G4Frag {
    u32x4 a[2][4];     // [16-token step][a block of 32 rows]
    u32x4 b[2];        // [16-token step]
    float4 sv;         // the quad's scales (see above)
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_fisher_mfma_g4(
    const uint16_t* __restrict__ XT, const float* __restrict__ S4, int64_t n_pad, int64_t d_pad,
    int nquad, int T, int npairs, int64_t ksplit, int total_blocks, float* __restrict__ part) {
    extern __shared__ u32x4 fisher_lds[];
    // XCD-aware remap as in the 256-tile kernel: XCD x takes 32 consecutive logical
    // blocks of each round of 256
    const int hw = blockIdx.x;
    const int lin = (hw & ~255) + (hw & 7) * 32 + ((hw & 255) >> 3);
    if (lin >= total_blocks) return;
    const int quad = lin % nquad;
    const int pair = (lin / nquad) % npairs;
    const int split = lin / (nquad * npairs);
    int ta, tb;
    panel_pair(pair, T, ta, tb);
    const int64_t kb = (int64_t)split * ksplit;
    const int64_t ke = (kb + ksplit < n_pad) ? kb + ksplit : n_pad;
    const int nst = kb < ke ? (int)((ke - kb) / FKC) : 0;       // even (64-token splits)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets go to M0

    const uint16_t* Abase = XT + ((kb >> 5) * d_pad + (int64_t)ta * G4_TE) * 32;
    const uint16_t* Bbase = XT + ((kb >> 5) * d_pad + (int64_t)tb * G4_TE) * 32;
    const float* Sq = S4 + ((int64_t)quad * n_pad + kb) * 4;     // [token][4] of this split
    const int64_t stage_elems = d_pad * 32;
    // band loads: instruction k of wave w fills rows 16q .. 16q + 15 (q = 4k + w) with
    // the slot swizzle; scale loads: wave w moves bytes 256 (w % 2) .. + 255 of the
    // stage's 512 (waves w and w + 2 write the same bytes)
    const uint32_t voff = (uint32_t)(lane >> 2) * 64u +
                          16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t shalf = 256u * (uint32_t)(wave & 1);
    auto clamp = [&](int s) { return s < nst ? s : nst - 1; };
    auto issue = [&](int s) {
        u32x4* slot = fisher_lds + (s % G4_RING) * G4_SLOT;
        const int64_t off = (int64_t)clamp(s) * stage_elems;
        const __amdgpu_buffer_rsrc_t Ar = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Abase + off), (short)0, G4_BAND * 16, 0x00020000);
        const __amdgpu_buffer_rsrc_t Br = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Bbase + off), (short)0, G4_BAND * 16, 0x00020000);
        const __amdgpu_buffer_rsrc_t Sr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Sq + (int64_t)clamp(s) * (FKC * 4)), (short)0, FKC * 16, 0x00020000);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = 4 * k + wave;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Ar, (lds_ptr_t)(slot + 64 * q), 16, voff,
                                                     (uint32_t)q * 1024u, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = 4 * k + wave;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Br, (lds_ptr_t)(slot + G4_BAND + 64 * q), 16,
                                                     voff, (uint32_t)q * 1024u, 0, 0);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Sr, (lds_ptr_t)((char*)(slot + 2 * G4_BAND) + shalf), 4, 4u * (uint32_t)lane, shalf,
            0, 0);
    };
    const int sw = (lane >> 2) & 3;          // slot swizzle of the fragment rows
    const int tau = 16 * ((lane >> 3) & 1) + 8 * (lane >> 5) + (lane & 7);
    auto read_frags = [&](int s, G4Frag& f) {
        const u32x4* A = fisher_lds + (s % G4_RING) * G4_SLOT;
        const u32x4* B = A + G4_BAND;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int cs = (2 * ks + (lane >> 5)) ^ sw;
#pragma unroll
            for (int i = 0; i < 4; ++i) f.a[ks][i] = A[(32 * i + (lane & 31)) * 4 + cs];
            f.b[ks] = B[(32 * wave + (lane & 31)) * 4 + cs];
        }
        const u32x4 v = A[2 * G4_BAND + tau];
        f.sv = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                           __uint_as_float(v[3]));
    };

    f32x16 acc[4][4];                    // [group of the quad][a block of 32 rows]
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[g][i][v] = 0.f;

    // Every stage issues the same 5 loads per wave (stages past the last load the last
    // one again into slots that are never read), so when stage s's second half is
    // due, the loads of stage s + 1 are complete once at most 6 x 5 later ones (stages
    // s + 2 .. s + 7) are outstanding.
    //   The scaling is software-pipelined one group ahead of the MFMAs: each half of a
    // stage issues the MFMAs of groups 0..3 while it scales the b operand of the next
    // (group, half), the last of them being group 0 of the next half (of the next
    // stage, from its freshly read fragments).
    G4Frag f0, f1;
    bf16x8 y_first;                      // scaled b operand, step 0 of the stage, group 0
    if (nst > 0) {
#pragma unroll
        for (int s = 0; s < G4_RING; ++s) issue(s);
        wait_vmcnt_lds<(G4_RING - 1) * G4_VM_PER_STAGE>();
        __builtin_amdgcn_s_barrier();
        read_frags(0, f0);
        float xf[8];
        g4_unpack(f0.b[0], xf);
        y_first = g4_scale<0>(xf, f0.sv.x);
    }
    auto stage = [&](int s, G4Frag& cur, G4Frag& nxt) {
        float x0[8], x1[8];
        g4_unpack(cur.b[0], x0);
        g4_unpack(cur.b[1], x1);
        {
            const bf16x8 y1 = g4_scale<0>(x0, cur.sv.y);
            g4_mfma(acc[0], cur.a[0], y_first);
            const bf16x8 y2 = g4_scale<0>(x0, cur.sv.z);
            g4_mfma(acc[1], cur.a[0], y1);
            const bf16x8 y3 = g4_scale<0>(x0, cur.sv.w);
            g4_mfma(acc[2], cur.a[0], y2);
            y_first = g4_scale<1>(x1, cur.sv.x);       // step 1, group 0
            g4_mfma(acc[3], cur.a[0], y3);
            g4_interleave();
        }
        __builtin_amdgcn_sched_barrier(0);
        // this wave's loads of stage s + 1 have landed and its reads of stage s are
        // done; after the barrier, so are everyone's
        wait_vmcnt_lds<(G4_RING - 2) * G4_VM_PER_STAGE>();
        __builtin_amdgcn_s_barrier();
        issue(s + G4_RING);
        read_frags(s + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        {
            const bf16x8 z1 = g4_scale<1>(x1, cur.sv.y);
            g4_mfma(acc[0], cur.a[1], y_first);
            const bf16x8 z2 = g4_scale<1>(x1, cur.sv.z);
            g4_mfma(acc[1], cur.a[1], z1);
            const bf16x8 z3 = g4_scale<1>(x1, cur.sv.w);
            g4_mfma(acc[2], cur.a[1], z2);
            float xn[8];
            g4_unpack(nxt.b[0], xn);
            y_first = g4_scale<0>(xn, nxt.sv.x);       // next stage, step 0, group 0
            g4_mfma(acc[3], cur.a[1], z3);
            g4_interleave();
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int s = 0; s < nst; s += 2) {
        stage(s, f0, f1);
        stage(s + 1, f1, f0);
    }
    wait_vmcnt<0>();     // no load into this block's LDS may land after it ends

    // partial tiles [4][128][128] row-major (group of the quad, a_local, b_local)
    float* P = part + (size_t)lin * (4 * G4_TE * G4_TE);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int al = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int bl = 32 * wave + (lane & 31);
                P[(g * G4_TE + al) * G4_TE + bl] = acc[g][i][v];
            }
}

// Sum split partials (fixed order) and write the tile plus its mirror.  One block
// per 64 x 64 sub-tile of a (pair, group): each thread sums 4 rows x 4 columns
// with float4 loads, writes F[a][b] and, through LDS, the mirror F[b][a] with
// float4 stores (d_in % 8 == 0 on this path, F 16-byte aligned).  TE is the tile
// edge and GB the groups per contraction block: partial tiles are
// [split][pair][groups / GB][GB][TE][TE]; PANEL selects the pair order of the
// four-group kernel.
template <int TE, int GB, bool PANEL>
__global__ __launch_bounds__(256) void k_fisher_finalize(const float* __restrict__ part,
                                                        int64_t d_in, int groups, int T,
                                                        int npairs, int nsplit,
                                                        int accumulate, float* __restrict__ F) {
    constexpr int SUB = TE / 64;                 // 64 x 64 sub-tiles per tile edge
    __shared__ float sub[64][65];
    const int pair = blockIdx.x / (SUB * SUB);
    const int sbk = blockIdx.x % (SUB * SUB);
    const int g = blockIdx.y;
    int ta, tb;
    if (PANEL) panel_pair(pair, T, ta, tb);
    else tri_pair(pair, T, ta, tb);
    const int sr = (sbk / SUB) * 64, sc = (sbk % SUB) * 64;
    const int64_t a0 = (int64_t)ta * TE + sr, b0 = (int64_t)tb * TE + sc;
    if (a0 >= d_in || b0 >= d_in) return;
    if (ta == tb && sr > sc) return;                 // strictly below the diagonal
    const int tid = threadIdx.x;
    const int c4 = (tid & 15) * 4;
    float* Fg = F + (size_t)g * d_in * d_in;
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < nsplit; ++s) {
        const size_t lin = ((size_t)s * npairs + pair) * (groups / GB) + g / GB;
        const float* P = part + (lin * GB + g % GB) * (TE * TE) + (size_t)sr * TE + sc + c4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 x = *(const float4*)(P + (size_t)((tid >> 4) + 16 * k) * TE);
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
    bool quad;                 // groups % 4 == 0: the four-group kernel (128-tiles)
    int64_t n;                 // tokens per pass (the call's n, or the pass limit)
    int64_t n_pad, d_pad;
    int T, npairs, nsplit;
    int64_t ksplit;
    int total, grid;
    size_t s_bytes, xt_bytes, part_bytes;
};

// The packed operand takes d_pad * n_pad * 2 bytes.  Token ranges beyond this budget,
// or beyond F_PASS_TOKENS tokens, run as several passes, each adding into F.
constexpr size_t F_PACK_BUDGET = (size_t)16 << 30;
constexpr int64_t F_PASS_TOKENS = (int64_t)1 << 20;

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

FisherPlan fisher_plan(int64_t n_call, int64_t d_in, int groups, bool bf16,
                       int max_split = 16) {
    FisherPlan p{};
    p.mfma = bf16 && (d_in % 8 == 0);
    p.quad = p.mfma && groups % 4 == 0;
    const int te = p.quad ? G4_TE : FT;
    {
        const int64_t d_pad = (d_in + te - 1) / te * te;
        int64_t cap = (int64_t)(F_PACK_BUDGET / ((size_t)d_pad * 2)) / PK * PK;
        if (cap > F_PASS_TOKENS) cap = F_PASS_TOKENS;
        if (cap < PK) cap = PK;
        p.n = (bf16 && d_in % 8 == 0 && n_call > cap) ? cap : n_call;
    }
    p.n_pad = (p.n + PK - 1) / PK * PK;            // the packing tile
    // S [groups][n_pad]: the scales of the tokens, zero on the padding
    p.s_bytes = al256((size_t)groups * p.n_pad * sizeof(float));
    if (!p.mfma) return p;
    p.T = (int)((d_in + te - 1) / te);
    p.d_pad = (int64_t)p.T * te;
    p.npairs = p.T * (p.T + 1) / 2;
    // contraction blocks per token split; either kernel's block makes 65536 outputs
    const int tiles = p.npairs * (p.quad ? groups / 4 : groups);
    const int slots = 256;  // one block (128 or 132 KB of LDS) per CU
    // model: time ~ ceil(tiles*s/slots) * (n/s) + s * tiles * finalize_cost
    double best = 1e300;
    int best_s = 1;
    for (int s = 1; s <= max_split; ++s) {
        const int64_t chunk = ((p.n_pad + s - 1) / s + 2 * FKC - 1) / (2 * FKC) * (2 * FKC);
        if (s > 1 && chunk < 2048) break;
        const double rounds = (double)((tiles * (int64_t)s + slots - 1) / slots);
        // one token of a block (65536 outputs) costs 131072 flop at ~60 % of a CU's
        // bf16 peak; one block's partial tiles read + written in the finalize ~256 KB
        // at ~5 TB/s
        const double t_main = rounds * (double)chunk * 131072.0 / (9.77e12 * 0.6);
        const double t_fin = (double)s * tiles * 262144.0 / 5e12;
        const double t = t_main + t_fin;
        if (t < best * 0.999) { best = t; best_s = s; }
    }
    p.nsplit = best_s;
    // whole 64-token steps (an even number of stages per split; n_pad is a multiple of 64)
    p.ksplit = ((p.n_pad + best_s - 1) / best_s + 2 * FKC - 1) / (2 * FKC) * (2 * FKC);
    p.total = tiles * p.nsplit;
    p.grid = (p.total + 255) / 256 * 256;         // whole rounds for the remap
    p.xt_bytes = al256((size_t)p.d_pad * p.n_pad * 2);
    p.part_bytes = (size_t)p.total * FT * FT * sizeof(float);   // = 4 x 128 x 128 per block
    return p;
}

size_t fisher_workspace(int64_t n, int64_t d_in, int groups, bool bf16) {
    FisherPlan p = fisher_plan(n, d_in, groups, bf16);
    return p.s_bytes + (p.mfma ? p.xt_bytes + p.part_bytes : 0);
}

static hipError_t fisher_pass(const FisherPlan& p, const void* X, const void* G, bool bf16,
                              int64_t n, int64_t d_in, int64_t d_out, int groups, float* F,
                              int accumulate, void* ws, hipStream_t st) {
    float* S = (float*)ws;
    char* w = (char*)ws + p.s_bytes;
    // the matrix-core path reads S with the pitch of the padded tokens (zeros there)
    const int64_t n_pad = (n + PK - 1) / PK * PK;
    const int64_t pitch = p.mfma ? n_pad : n;
    dim3 gs((unsigned)((pitch + 3) / 4), (unsigned)groups);
    const int quad = p.quad ? 1 : 0;
    {
        StageTimer tm(ST_GROUP_SCALE, st);
        if (bf16)
            hipLaunchKernelGGL(k_group_scale<true>, gs, dim3(256), 0, st, G, n, d_out, groups,
                               pitch, quad, S);
        else
            hipLaunchKernelGGL(k_group_scale<false>, gs, dim3(256), 0, st, G, n, d_out, groups,
                               pitch, quad, S);
        GQ_LAUNCH_CHECK();
    }
    if (p.mfma) {
        uint16_t* XT = (uint16_t*)w;
        float* part = (float*)(w + p.xt_bytes);
        {
            hipError_t e = p.quad ? ensure_dynamic_lds((const void*)k_fisher_mfma_g4, G4_LDS_BYTES)
                                  : ensure_dynamic_lds((const void*)k_fisher_mfma, F_LDS_BYTES);
            if (e != hipSuccess) return e;
        }
        {
            StageTimer tm(ST_FISHER_PACK, st);
            dim3 gp((unsigned)(n_pad / PK), (unsigned)(p.d_pad / PK));
            hipLaunchKernelGGL(k_fisher_pack, gp, dim3(256), 0, st, (const uint16_t*)X, n, d_in,
                               p.d_pad, XT);
            GQ_LAUNCH_CHECK();
        }
        // the split plan of this pass's token count (no more partial tiles than the
        // workspace holds)
        const FisherPlan q = fisher_plan(n, d_in, groups, bf16, p.nsplit);
        {
            StageTimer tm(ST_FISHER_MFMA, st);
            if (q.quad)
                hipLaunchKernelGGL(k_fisher_mfma_g4, dim3(q.grid), dim3(256), G4_LDS_BYTES, st, XT,
                                   S, n_pad, q.d_pad, groups / 4, q.T, q.npairs, q.ksplit, q.total,
                                   part);
            else
                hipLaunchKernelGGL(k_fisher_mfma, dim3(q.grid), dim3(512), F_LDS_BYTES, st, XT, S,
                                   n_pad, q.d_pad, groups, q.T, q.npairs, q.ksplit, q.total, part);
            GQ_LAUNCH_CHECK();
        }
        StageTimer tm(ST_FISHER_FINALIZE, st);
        if (q.quad)
            hipLaunchKernelGGL((k_fisher_finalize<G4_TE, 4, true>), dim3(q.npairs * 4, groups),
                               dim3(256), 0, st, part, d_in, groups, q.T, q.npairs, q.nsplit,
                               accumulate, F);
        else
            hipLaunchKernelGGL((k_fisher_finalize<FT, 1, false>), dim3(q.npairs * 16, groups),
                               dim3(256), 0, st, part, d_in, groups, q.T, q.npairs, q.nsplit,
                               accumulate, F);
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
