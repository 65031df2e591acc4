// Lookup-table dequantisation GEMV for LNQ's output on gfx950.
//
// GuidedQuant blog page (jinukkim.me/blog/guidedquant), section "LNQ": each row j
// of the quantized layer is a codebook c^(j) (m = 2^b entries) and b-bit indices
// P^(j); the page notes that the result runs on the same lookup-table kernel as
// SqueezeLLM.  This file holds that consumer:
//
//   k_lut_pack       P [d_out][d_in] (one byte per code) -> packed words.  Codes are
//                    taken in pairs (i, i + 1); a pair is the 2b-bit index
//                    code_i | code_{i+1} << b, and a 32-bit word holds 16 / b pairs
//                    (integer division), low bits first: 32, 16, 10 or 8 codes per
//                    word for b = 1..4.  A row is padded with zero words to a
//                    multiple of 4 words.
//   k_lut_gemv_bf16  y[b][j] = sum_i c^(j)[p_ji] x[b][i] for bfloat16 activations:
//                    per row a table of the m^2 codebook pairs as packed bfloat16
//                    (the codebook rounded to nearest even), one table read per
//                    code pair, and v_dot2c_f32_bf16 (both products exact, float32
//                    accumulation).  x is staged once per block in LDS as bfloat16
//                    pairs, word w's pairs at w * XST + p with XST = (16 / b) | 1
//                    (odd), so lanes reading consecutive words hit distinct banks.
//   k_lut_gemv_f32   the same product for float32 activations with the float32
//                    codebook and float32 FMAs (a reference-precision path).
//
// Bound: HBM (the packed codes, b/8 bytes per weight); x, the codebook and y are
// small next to them.
#include "gq_common.h"
#include "gq_internal.h"

namespace gq {

constexpr int LUT_WAVES = 8;          // waves per block of the GEMV (16 where that form fits)
constexpr int LUT_UNROLL = 8;         // code words in flight per lane
constexpr int LUT_SPAN = 64 * LUT_UNROLL;   // words per chunk of a row

__host__ __device__ constexpr int lut_ppw(int bits) { return 16 / bits; }      // pairs per word
// LDS words per staged word of x: its 16 / b pairs, as 16-byte vectors when that is a
// whole number of them (b = 1, 2, 4), else padded to an odd count (b = 3: 5) so lanes
// reading consecutive words touch distinct banks
__host__ __device__ constexpr int lut_xst(int bits) {
    return (16 / bits) % 4 == 0 ? 16 / bits : (16 / bits) | 1;
}

int64_t lut_row_words(int64_t d_in, int bits) {
    const int64_t cpw = 2 * lut_ppw(bits);
    return ((d_in + cpw - 1) / cpw + 3) / 4 * 4;
}

// one thread per packed word
__global__ __launch_bounds__(256) void k_lut_pack(const uint8_t* __restrict__ P, int64_t d_out,
                                                 int64_t d_in, int bits, int64_t rw,
                                                 uint32_t* __restrict__ Q) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= d_out * rw) return;
    const int64_t j = t / rw, w = t - j * rw;
    const int cpw = 2 * (16 / bits);
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t i0 = w * cpw;
    uint32_t word = 0u;
    for (int s = 0; s < cpw; ++s) {
        const int64_t i = i0 + s;
        if (i < d_in) word |= ((uint32_t)P[j * d_in + i] & mask) << (bits * s);
    }
    Q[t] = word;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// staged words per activation vector for a segment of sw row words: those words and one
// word of zeros, which every word past the row reads (as code 0)
__host__ __device__ inline int64_t lut_staged_words(int64_t sw) { return sw + 1; }

// LDS: one table of M * M words per wave (wave w's at w * M * M, so a table index is
// or-ed onto its base), then x pairs [B][staged words * XST].  Rows: block r takes rows
// r * rows_per_block .. + rows_per_block - 1, wave w every WAVES-th.  A row's words are
// taken in segments of seg_words (a multiple of LUT_SPAN; at least the row when it fits):
// per segment the block stages that part of x, and each wave runs its rows over it,
// adding the segment's sums into y (the first segment writes them).
template <int BITS, int B, int WAVES, bool SEG>
__global__ __launch_bounds__(64 * WAVES) void k_lut_gemv_bf16(
    const uint32_t* __restrict__ Q, int64_t rw, const float* __restrict__ C, int64_t d_out,
    int64_t d_in, const uint16_t* __restrict__ x, int whole_pairs, int rows_per_block,
    int64_t seg_words, float* __restrict__ y) {
    constexpr int M = 1 << BITS;
    constexpr int PPW = lut_ppw(BITS);
    constexpr int XST = lut_xst(BITS);
    constexpr uint32_t PMASK = (uint32_t)(M * M - 1);
    static_assert(XST == PPW, "staged words hold their pairs contiguously");
    extern __shared__ __attribute__((aligned(16))) uint32_t lut_lds[];
    const int64_t seg_alloc = (SEG && seg_words < rw) ? seg_words : rw;
    const int64_t xwords = lut_staged_words(seg_alloc) * XST;
    uint32_t* const xlds = lut_lds + WAVES * M * M;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* tab = lut_lds + wave * (M * M);
    const uint32_t tab_bytes = (uint32_t)(wave * M * M) * 4u;

    // Work of a wave in a segment: its rows (every WAVES-th of the block's), each in
    // chunks of LUT_SPAN words; item t = (row k, chunk c0 + cl).  The codes (and, at a
    // row's first chunk of the segment, the codebook) of item t + 1 are loaded while item
    // t is computed.
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    int nrows = 0;
    for (int rr = wave; rr < rows_per_block && r0 + rr < d_out; rr += WAVES) ++nrows;
    const int nch = (int)((rw + LUT_SPAN - 1) / LUT_SPAN);
    const int cps = SEG ? (int)(seg_words / LUT_SPAN) : nch;   // chunks per segment
    const int nseg = SEG ? (nch + cps - 1) / cps : 1;
    auto fetch = [&](int k, int c, bool first, uint32_t (&wv)[LUT_UNROLL], float& cv) {
        const int64_t j = r0 + wave + (int64_t)WAVES * k;
        const uint32_t* Qj = Q + j * rw;
        const int w0 = c * LUT_SPAN + lane;
        if ((int64_t)(c + 1) * LUT_SPAN <= rw) {
#pragma unroll
            for (int u = 0; u < LUT_UNROLL; ++u) wv[u] = Qj[w0 + 64 * u];
        } else {
#pragma unroll
            for (int u = 0; u < LUT_UNROLL; ++u) {
                const int wi = w0 + 64 * u;
                wv[u] = wi < rw ? Qj[wi] : 0u;
            }
        }
        if (first) cv = lane < M ? C[j * M + lane] : 0.f;
    };

    // x pair pr = w * PPW + p holds elements 2 pr, 2 pr + 1 (zero past d_in);
    // whole_pairs (even d_in, x 4-byte aligned): each pair is one 4-byte load.  With
    // XST == PPW the staged pairs are x itself, zero-padded, so when the copies' starts
    // are 16-byte aligned, 16-byte loads copy them, all in flight at once.
    const int64_t dpairs = d_in >> 1;
    const bool even = whole_pairs != 0;
    auto stage = [&](int64_t w_lo, int64_t sw) {
        const int64_t spairs = lut_staged_words(sw) * PPW;
        const int64_t gp0 = w_lo * PPW;                         // first pair of the segment
        const bool vec = even && (((uintptr_t)x & 15u) == 0) && (d_in % 8 == 0) &&
                         (xwords % 4 == 0) && (spairs % 4 == 0) && (gp0 % 4 == 0);
        for (int b = 0; b < B; ++b) {
            const uint16_t* xb = x + (int64_t)b * d_in;
            uint32_t* xs = xlds + (int64_t)b * xwords;
            if (vec) {
                const u32x4* src = (const u32x4*)xb + gp0 / 4;
                u32x4* dst = (u32x4*)xs;
                const int64_t nv = spairs / 4;
                const int64_t dv = (dpairs - gp0) / 4;          // whole vectors before d_in
#pragma unroll 4
                for (int64_t i = tid; i < nv; i += 64 * WAVES)
                    dst[i] = i < dv ? src[i] : u32x4{0u, 0u, 0u, 0u};
                continue;
            }
            for (int64_t pr = tid; pr < spairs; pr += 64 * WAVES) {
                const int64_t g = gp0 + pr;
                uint32_t v;
                if (even) {
                    v = g < dpairs ? ((const uint32_t*)xb)[g] : 0u;
                } else {
                    const int64_t i = 2 * g;
                    const uint32_t lo = i < d_in ? xb[i] : 0u;
                    const uint32_t hi = i + 1 < d_in ? xb[i + 1] : 0u;
                    v = lo | (hi << 16);
                }
                const int64_t w = pr / PPW;
                xs[w * XST + (pr - w * PPW)] = v;
            }
        }
    };

    // two accumulator sets (even and odd words of a chunk) for independent chains
    float acc[2][B];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[h][b] = 0.f;
    const char* lds_bytes = (const char*)lut_lds;
    // li: staged word index of the segment (its zero word past the row)
    auto word_step = [&](uint32_t word, int li, int h) {
        const uint32_t* xw = xlds + li * XST;
        uint32_t xv[B][PPW];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if constexpr (PPW % 4 == 0) {          // XST == PPW: whole 16-byte vectors
#pragma unroll
                for (int q = 0; q < PPW / 4; ++q) {
                    const u32x4 v = *(const u32x4*)(xw + b * xwords + 4 * q);
                    xv[b][4 * q] = v[0]; xv[b][4 * q + 1] = v[1];
                    xv[b][4 * q + 2] = v[2]; xv[b][4 * q + 3] = v[3];
                }
            } else {
#pragma unroll
                for (int p = 0; p < PPW; ++p) xv[b][p] = xw[b * xwords + p];
            }
        }
#pragma unroll
        for (int p = 0; p < PPW; ++p) {
            // byte address of table entry ((word >> 2 b p) & PMASK) of this wave's table
            const uint32_t off = (2 * BITS * p >= 2)
                ? ((word >> (2 * BITS * p - 2)) & (PMASK << 2)) | tab_bytes
                : ((word << 2) & (PMASK << 2)) | tab_bytes;
            const uint32_t lv = *(const uint32_t*)(lds_bytes + off);
#pragma unroll
            for (int b = 0; b < B; ++b) acc[h][b] = dot2_bf16(lv, xv[b][p], acc[h][b]);
        }
    };

    for (int sg = 0; sg < nseg; ++sg) {
        const int c0 = sg * cps;
        const int cn = (nch - c0) < cps ? (nch - c0) : cps;
        const int64_t w_lo = (int64_t)c0 * LUT_SPAN;
        const int64_t sw = ((rw - w_lo) < (int64_t)cn * LUT_SPAN) ? (rw - w_lo) : (int64_t)cn * LUT_SPAN;
        const int nitems = nrows * cn;
        uint32_t cur[LUT_UNROLL];
        float ccur = 0.f;
        if (nitems > 0) fetch(0, c0, true, cur, ccur);
        if (SEG && sg > 0) __syncthreads();   // every wave is done with the previous segment's x
        stage(w_lo, sw);
        __syncthreads();
        for (int t = 0; t < nitems; ++t) {
            const int k = t / cn, cl = t - k * cn;
            uint32_t nxt[LUT_UNROLL];
            float cnxt = 0.f;
            if (t + 1 < nitems) {
                const int k1 = (t + 1) / cn, cl1 = (t + 1) - k1 * cn;
                fetch(k1, c0 + cl1, cl1 == 0, nxt, cnxt);
            }
            if (cl == 0) {
                // the row's pair table: entry q0 | q1 << BITS = (bf16 c_q0, bf16 c_q1); the
                // previous row's reads of it came earlier in this wave's LDS order
                for (int e = lane; e < M * M; e += 64)
                    tab[e] = pack_bf16x2(__shfl(ccur, e & (M - 1), 64), __shfl(ccur, e >> BITS, 64));
            }
            // a word past the row is code 0 against the staged zero word
            const int c = c0 + cl;
            const int lw0 = cl * LUT_SPAN + lane;                // staged index of word w0
            if ((int64_t)(c + 1) * LUT_SPAN <= rw) {
#pragma unroll
                for (int u = 0; u < LUT_UNROLL; ++u) word_step(cur[u], lw0 + 64 * u, u & 1);
            } else {
#pragma unroll
                for (int u = 0; u < LUT_UNROLL; ++u) {
                    const int li = lw0 + 64 * u;
                    word_step(cur[u], li < sw ? li : (int)sw, u & 1);
                }
            }
            if (cl == cn - 1) {
                const int64_t j = r0 + wave + (int64_t)WAVES * k;
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float s = wave_sum_f32(acc[0][b] + acc[1][b]);
                    if (lane == 0) {
                        float* yp = y + (int64_t)b * d_out + j;
                        *yp = (!SEG || sg == 0) ? s : *yp + s;
                    }
                    acc[0][b] = 0.f;
                    acc[1][b] = 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < LUT_UNROLL; ++u) cur[u] = nxt[u];
            if (cl == cn - 1) ccur = cnxt;
        }
    }
}

// float32 activations: float32 codebook, float32 FMAs, x read from global memory.
template <int BITS>
__global__ __launch_bounds__(256) void k_lut_gemv_f32(const uint32_t* __restrict__ Q, int64_t rw,
                                                     const float* __restrict__ C, int64_t d_out,
                                                     int64_t d_in, const float* __restrict__ x,
                                                     int batch, float* __restrict__ y) {
    constexpr int M = 1 << BITS;
    constexpr int CPW = 2 * lut_ppw(BITS);
    const int lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= d_out) return;
    const float cl = lane < M ? C[j * M + lane] : 0.f;
    const uint32_t* Qj = Q + j * rw;
    for (int b = 0; b < batch; ++b) {
        const float* xb = x + (int64_t)b * d_in;
        float acc = 0.f;
        // uniform trip count: every lane takes part in the table shuffles
        for (int64_t w0 = 0; w0 < rw; w0 += 64) {
            const int64_t w = w0 + lane;
            const uint32_t word = w < rw ? Qj[w] : 0u;
#pragma unroll
            for (int s = 0; s < CPW; ++s) {
                const int code = (int)((word >> (BITS * s)) & (uint32_t)(M - 1));
                const float v = __shfl(cl, code, 64);
                const int64_t i = w * CPW + s;
                if (w < rw && i < d_in) acc = fmaf(v, xb[i], acc);
            }
        }
        const float s = wave_sum_f32(acc);
        if (lane == 0) y[(int64_t)b * d_out + j] = s;
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
hipError_t lut_pack_run(const uint8_t* P, int64_t d_out, int64_t d_in, int bits, uint32_t* Q,
                        hipStream_t st) {
    const int64_t rw = lut_row_words(d_in, bits);
    const int64_t n = d_out * rw;
    StageTimer tm(ST_LUT_PACK, st);
    hipLaunchKernelGGL(k_lut_pack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, P, d_out,
                       d_in, bits, rw, Q);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

constexpr size_t LUT_LDS_CU = 160 * 1024;     // LDS of a compute unit

// LDS of a block that stages sw row words per vector
static size_t lut_lds_bytes(int64_t sw, int bits, int batch, int waves) {
    const int m = 1 << bits;
    return (size_t)(batch * lut_staged_words(sw) * lut_xst(bits) + waves * m * m) * 4;
}

// Words per segment when a whole row does not fit: the largest multiple of LUT_SPAN
// whose staging fits one block (0 if not even one chunk does).
static int64_t lut_segment_words(int bits, int batch, int waves) {
    const size_t tables = (size_t)waves * (1u << (2 * bits)) * 4;
    if (tables >= LUT_LDS_CU) return 0;
    const int64_t words = (int64_t)((LUT_LDS_CU - tables) / (4 * (size_t)batch * lut_xst(bits))) - 1;
    return words / LUT_SPAN * LUT_SPAN;
}

// whether some form of the product fits the LDS: the whole row, or segments of one chunk
bool lut_gemv_fits(int64_t d_in, int bits, int batch) {
    const int64_t rw = lut_row_words(d_in, bits);
    const int64_t first = rw < LUT_SPAN ? rw : LUT_SPAN;
    return lut_lds_bytes(first, bits, batch, LUT_WAVES) <= LUT_LDS_CU;
}

template <int BITS, int B, int WAVES, bool SEG>
static hipError_t launch_bf16_w(const uint32_t* Q, const float* C, int64_t d_out, int64_t d_in,
                                const uint16_t* x, float* y, int64_t blocks_target,
                                int64_t seg_words, hipStream_t st) {
    const int64_t rw = lut_row_words(d_in, BITS);
    const size_t lds = lut_lds_bytes(seg_words < rw ? seg_words : rw, BITS, B, WAVES);
    {
        hipError_t e = ensure_dynamic_lds((const void*)k_lut_gemv_bf16<BITS, B, WAVES, SEG>, lds);
        if (e != hipSuccess) return e;
    }
    // about blocks_target blocks, at least one row per wave
    int64_t rpb = (d_out + blocks_target - 1) / blocks_target;
    if (rpb < WAVES) rpb = WAVES;
    const int64_t grid = (d_out + rpb - 1) / rpb;
    hipLaunchKernelGGL((k_lut_gemv_bf16<BITS, B, WAVES, SEG>), dim3((unsigned)grid), dim3(64 * WAVES),
                       lds, st, Q, rw, C, d_out, d_in, x,
                       (int)((d_in % 2 == 0) && (((uintptr_t)x & 3u) == 0)), (int)rpb, seg_words,
                       y);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

// One 16-wave block per compute unit where the kernel stays within the 128 registers of
// such a block without spilling (3- and 4-bit codes, and 2-bit codes with up to 4 vectors)
// and its LDS fits: the activations are staged once per 16 waves' rows.  Else two 8-wave
// blocks per unit where their LDS fits, else one.  Where no whole row fits, the row is
// staged in segments, in a 16-wave block where that kernel does not spill.
template <int BITS, int B>
static hipError_t launch_bf16(const uint32_t* Q, const float* C, int64_t d_out, int64_t d_in,
                              const uint16_t* x, float* y, hipStream_t st) {
    constexpr bool WIDE = BITS >= 3 || (BITS == 2 && B <= 4);
    const int64_t rw = lut_row_words(d_in, BITS);
    const int64_t whole = (rw + LUT_SPAN - 1) / LUT_SPAN * LUT_SPAN;      // one segment
    if constexpr (WIDE) {
        if (lut_lds_bytes(rw, BITS, B, 2 * LUT_WAVES) <= LUT_LDS_CU)
            return launch_bf16_w<BITS, B, 2 * LUT_WAVES, false>(Q, C, d_out, d_in, x, y, 256, whole,
                                                                st);
    }
    if (lut_lds_bytes(rw, BITS, B, LUT_WAVES) <= LUT_LDS_CU) {
        const int64_t blocks = 2 * lut_lds_bytes(rw, BITS, B, LUT_WAVES) <= LUT_LDS_CU ? 512 : 256;
        return launch_bf16_w<BITS, B, LUT_WAVES, false>(Q, C, d_out, d_in, x, y, blocks, whole, st);
    }
    // the segmented kernel holds a few more registers: 16 waves where that still fits
    constexpr bool SEG_WIDE = (BITS == 4 && B <= 4) || (BITS == 3 && B <= 3) || (BITS == 2 && B <= 2);
    if constexpr (SEG_WIDE) {
        const int64_t s16 = lut_segment_words(BITS, B, 2 * LUT_WAVES);
        if (s16 >= LUT_SPAN)
            return launch_bf16_w<BITS, B, 2 * LUT_WAVES, true>(Q, C, d_out, d_in, x, y, 256, s16,
                                                               st);
    }
    const int64_t seg = lut_segment_words(BITS, B, LUT_WAVES);
    if (seg < LUT_SPAN) return hipErrorInvalidValue;   // rejected before any launch
    return launch_bf16_w<BITS, B, LUT_WAVES, true>(Q, C, d_out, d_in, x, y, 256, seg, st);
}

template <int BITS>
static hipError_t launch_bf16_b(int batch, const uint32_t* Q, const float* C, int64_t d_out,
                                int64_t d_in, const uint16_t* x, float* y, hipStream_t st) {
    switch (batch) {
        case 1: return launch_bf16<BITS, 1>(Q, C, d_out, d_in, x, y, st);
        case 2: return launch_bf16<BITS, 2>(Q, C, d_out, d_in, x, y, st);
        case 3: return launch_bf16<BITS, 3>(Q, C, d_out, d_in, x, y, st);
        case 4: return launch_bf16<BITS, 4>(Q, C, d_out, d_in, x, y, st);
        case 5: return launch_bf16<BITS, 5>(Q, C, d_out, d_in, x, y, st);
        case 6: return launch_bf16<BITS, 6>(Q, C, d_out, d_in, x, y, st);
        case 7: return launch_bf16<BITS, 7>(Q, C, d_out, d_in, x, y, st);
        default: return launch_bf16<BITS, 8>(Q, C, d_out, d_in, x, y, st);
    }
}

hipError_t lut_gemv_run(const uint32_t* Q, const float* C, int64_t d_out, int64_t d_in, int bits,
                        const void* x, bool x_bf16, int batch, float* y, hipStream_t st) {
    StageTimer tm(ST_LUT_GEMV, st);
    if (x_bf16) {
        const uint16_t* xb = (const uint16_t*)x;
        switch (bits) {
            case 1: return launch_bf16_b<1>(batch, Q, C, d_out, d_in, xb, y, st);
            case 2: return launch_bf16_b<2>(batch, Q, C, d_out, d_in, xb, y, st);
            case 3: return launch_bf16_b<3>(batch, Q, C, d_out, d_in, xb, y, st);
            default: return launch_bf16_b<4>(batch, Q, C, d_out, d_in, xb, y, st);
        }
    }
    const int64_t rw = lut_row_words(d_in, bits);
    const dim3 grid((unsigned)((d_out + 3) / 4));
    const float* xf = (const float*)x;
    switch (bits) {
        case 1: hipLaunchKernelGGL(k_lut_gemv_f32<1>, grid, dim3(256), 0, st, Q, rw, C, d_out, d_in, xf, batch, y); break;
        case 2: hipLaunchKernelGGL(k_lut_gemv_f32<2>, grid, dim3(256), 0, st, Q, rw, C, d_out, d_in, xf, batch, y); break;
        case 3: hipLaunchKernelGGL(k_lut_gemv_f32<3>, grid, dim3(256), 0, st, Q, rw, C, d_out, d_in, xf, batch, y); break;
        default: hipLaunchKernelGGL(k_lut_gemv_f32<4>, grid, dim3(256), 0, st, Q, rw, C, d_out, d_in, xf, batch, y); break;
    }
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

}  // namespace gq
