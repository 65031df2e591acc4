// Matrix-core products with the damped Fisher F' for LNQ on gfx950.
//
// GuidedQuant blog page (jinukkim.me/blog/guidedquant), section "LNQ": the
// "(codebook)" line needs P_j^T F' P_j and P_j^T F' w_j for every row j, and the
// "(assignment)" objective (w_hat - w)^T F' (w_hat - w) is tracked through the
// residual r_j = F'(w_hat_j - w_j).  Two products over all rows of a group do
// the dense work:
//
//   k_resid  R[j][a] = sum_i E[j][i] F'[a][i],  E = C[P] - W split into bf16
//            hi + lo planes, F' as bf16 hi + lo planes; three products
//            (Ehi Fhi + Ehi Flo + Elo Fhi) give float32-level accuracy.
//   k_gram   A_j = P_j^T F' P_j.  With the one-hot P_j (exact in bf16) the kernel
//            forms
//                T[a][(j,q)] = sum_{i >= tile(a)} F'[a][i] [P[j][i] == q]
//            over the upper-triangle tiles of F' only (the diagonal tile at half
//            weight), and the epilogue bins T by the code of coordinate a:
//                B_j[q'][q] += sum_a [P[j][a] == q'] T[a][(j,q)].
//            Then A_j = B_j + B_j^T (by the symmetry of F').  Per-a-tile partials
//            are written in a fixed layout and summed in a fixed order.
//
// Both operands live in k-blocked bf16 planes (element (row, k) at
// ((k / 16) * rows + row) * 16 + k % 16, rows padded to whole 256-row tiles), so
// one 16-deep stage of a 256-row band is 8 KB of contiguous memory.  Block tile
// 256 x 256, 4 waves (one per SIMD) of 128 x 128 as 4 x 4 v_mfma_f32_32x32x16_bf16
// tiles.  The stages go through a ring of 4 LDS stages filled by direct
// buffer-to-LDS loads ahead of use; a 32-byte operand row sits in two 16-byte
// slots, chunk c of row r in slot 2 r + (c ^ ((r >> 3) & 1)), so each quarter-wave
// fragment read (16 consecutive rows) touches 16 distinct bank groups.  k_gram takes
// 32-deep stages (two k-blocks) and builds its one-hot operand in registers from
// the codes, which travel through LDS beside the F' bands.
#include "gq_common.h"
#include "gq_internal.h"

namespace gq {

constexpr int MT = 256;                 // block tile edge
constexpr int MRING = 4;                // LDS stages in the ring
constexpr int M_SLOTS = MT * 2;         // 16-byte slots of one 256-row, 16-deep operand band

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int N>
__device__ __forceinline__ void mm_wait_vmcnt() {
    // vmcnt(N), and lgkmcnt(0): the LDS writes of this wave are done too
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Hardware block h -> logical block: within each round of 256 blocks, XCD x
// (= h % 8) receives 32 consecutive logical blocks.
__device__ __forceinline__ int mm_remap(int hw) {
    return (hw & ~255) + (hw & 7) * 32 + ((hw & 255) >> 3);
}

// Buffer descriptor on one stage of a 256-row band (8 KB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t band_rsrc(const uint16_t* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, M_SLOTS * 16, 0x00020000);
}

// Copy rows 32 q .. 32 q + 31 (q of 8) of one stage of a 256-row band (rows of 32
// bytes) into their LDS slots with one instruction; lane L takes row 32 q + L/2 and slot
// L%2, i.e. chunk (L%2) ^ ((L/16)%2).  The 8 instructions of a stage are spread over
// the block's waves.
__device__ __forceinline__ void band_to_lds(__amdgpu_buffer_rsrc_t r, u32x4* dst, int q,
                                            uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + 64 * q), 16, voff,
                                             (uint32_t)q * 1024u, 0, 0);
}

__device__ __forceinline__ uint32_t band_voff(int lane) {
    return (uint32_t)(lane >> 1) * 32u + 16u * (uint32_t)((lane & 1) ^ ((lane >> 4) & 1));
}

// fragment slot of row `row` (its low 5 bits from the lane) for a 16-deep k-step
__device__ __forceinline__ int frag_slot(int row, int lane) {
    return row * 2 + ((lane >> 5) ^ ((lane >> 3) & 1));
}

// ---------------------------------------------------------------------------
// R = E F'.  Tile (256 rows j of a group) x (256 coordinates a), 4 waves (one per
// SIMD); wave w owns rows 128 (w % 2) .. + 127 and coordinates 128 (w / 2) .. + 127
// as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators (256 registers), so a stage's 16
// fragment reads from LDS feed 48 MFMAs (a hi fragment 8, a lo fragment 4).
//   Each 16-deep stage of the four bands (Ehi, Elo, Fhi, Flo) is refilled into the ring
// four stages ahead with the same 8 loads per wave at every stage (stages past the
// last reload it into a slot that is never read), so fixed vmcnt waits hold.  One
// barrier per stage, between the two halves of its 48 MFMAs: after it the stage's
// slot is refilled and the next stage's fragments are read while the second half runs.
// ---------------------------------------------------------------------------
struct RFrag {
    u32x4 eh[4], el[4];     // rows 128 (w % 2) + 32 i
    u32x4 fh[4], fl[4];     // coordinates 128 (w / 2) + 32 j
};

// MFMA t (0..23) of one half (rows i0, i0 + 1): product t / 8 (Ehi Fhi, Ehi Flo,
// Elo Fhi) of accumulator (i0 + (t % 8) / 4, t % 4), so the same accumulator
// comes back only every 8 MFMAs.
template <int I0>
__device__ __forceinline__ void resid_mfma(f32x16 (&acc)[4][4], const RFrag& f, int t) {
    const int p = t >> 3, i = I0 + ((t & 7) >> 2), j = t & 3;
    const u32x4 a = p == 2 ? f.el[i] : f.eh[i];
    const u32x4 b = p == 1 ? f.fl[j] : f.fh[j];
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc[i][j], 0, 0, 0);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_resid(
    const uint16_t* __restrict__ Ehi, const uint16_t* __restrict__ Elo, int64_t erows,
    int64_t rpg_pad, const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo,
    int64_t a_pad, int64_t d, int64_t rpg, int ntn, int nta, int total, float* __restrict__ R,
    const unsigned long long* __restrict__ skip) {
    extern __shared__ u32x4 mm_lds[];
    if (skip && *skip != 0ull) return;
    // row tiles fastest: the blocks one XCD runs together share their F' bands (the larger
    // operand) in its L2, a band being read by all ntn row tiles of its group
    const int lin = mm_remap(blockIdx.x);
    if (lin >= total) return;
    const int tn = lin % ntn;
    const int ta = (lin / ntn) % nta;
    const int g = lin / (nta * ntn);
    const int64_t a0 = (int64_t)ta * MT, n0 = (int64_t)tn * MT;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w0 = wave & 1, w1 = wave >> 1;
    const uint32_t voff = band_voff(lane);

    // stage s of each band: + s * (rows of the plane) * 16 elements
    const uint16_t* Eh = Ehi + ((int64_t)g * rpg_pad + n0) * 16;
    const uint16_t* El = Elo + ((int64_t)g * rpg_pad + n0) * 16;
    const int64_t fg = (int64_t)g * d * a_pad;
    const uint16_t* Fh = Fhi + fg + a0 * 16;
    const uint16_t* Fl = Flo + fg + a0 * 16;
    const int64_t estep = erows * 16, fstep = a_pad * 16;
    const int nst = (int)(d / 16);                      // even: d % 32 == 0

    // Stages are refilled in order; eo / fo is the element offset of the next one,
    // held at the last stage once it is reached.
    int64_t eo = 0, fo = 0;
    __amdgpu_buffer_rsrc_t rs[4];
    auto next_rsrc = [&]() {
        rs[0] = band_rsrc(Eh + eo);
        rs[1] = band_rsrc(El + eo);
        rs[2] = band_rsrc(Fh + fo);
        rs[3] = band_rsrc(Fl + fo);
    };
    auto advance = [&](int s) {
        if (s + 1 < nst) { eo += estep; fo += fstep; }
    };
    // load k (0..7) of a stage's refill: band k % 4, rows 32 (wave + 4 (k / 4)) .. + 31
    auto issue_one = [&](u32x4* base, int k) {
        band_to_lds(rs[k & 3], base + (k & 3) * M_SLOTS, wave + 4 * (k >> 2), voff);
    };
    auto issue = [&](int s) {
        u32x4* base = mm_lds + (s % MRING) * (4 * M_SLOTS);
        next_rsrc();
#pragma unroll
        for (int k = 0; k < 8; ++k) issue_one(base, k);
        advance(s);
    };
    // fragment read k (0..15) of stage s, in the order the first half uses them
    auto read_one = [&](int s, RFrag& f, int k) {
        const u32x4* S = mm_lds + (s % MRING) * (4 * M_SLOTS);
        const int ei = 128 * w0 + (lane & 31), fj = 128 * w1 + (lane & 31);
        switch (k) {
            case 0: f.eh[0] = S[frag_slot(ei, lane)]; break;
            case 1: f.fh[0] = S[2 * M_SLOTS + frag_slot(fj, lane)]; break;
            case 2: f.fh[1] = S[2 * M_SLOTS + frag_slot(fj + 32, lane)]; break;
            case 3: f.fh[2] = S[2 * M_SLOTS + frag_slot(fj + 64, lane)]; break;
            case 4: f.fh[3] = S[2 * M_SLOTS + frag_slot(fj + 96, lane)]; break;
            case 5: f.eh[1] = S[frag_slot(ei + 32, lane)]; break;
            case 6: f.fl[0] = S[3 * M_SLOTS + frag_slot(fj, lane)]; break;
            case 7: f.fl[1] = S[3 * M_SLOTS + frag_slot(fj + 32, lane)]; break;
            case 8: f.fl[2] = S[3 * M_SLOTS + frag_slot(fj + 64, lane)]; break;
            case 9: f.fl[3] = S[3 * M_SLOTS + frag_slot(fj + 96, lane)]; break;
            case 10: f.el[0] = S[M_SLOTS + frag_slot(ei, lane)]; break;
            case 11: f.el[1] = S[M_SLOTS + frag_slot(ei + 32, lane)]; break;
            case 12: f.eh[2] = S[frag_slot(ei + 64, lane)]; break;
            case 13: f.eh[3] = S[frag_slot(ei + 96, lane)]; break;
            case 14: f.el[2] = S[M_SLOTS + frag_slot(ei + 64, lane)]; break;
            default: f.el[3] = S[M_SLOTS + frag_slot(ei + 96, lane)]; break;
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // 8 loads per wave and stage: when stage s's second half is due, stage s + 1 has
    // landed once at most the 2 x 8 loads of stages s + 2 and s + 3 are outstanding
    RFrag f0, f1;
    if (nst > 0) {
#pragma unroll
        for (int s = 0; s < MRING; ++s) issue(s);
        mm_wait_vmcnt<(MRING - 1) * 8>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int k = 0; k < 16; ++k) read_one(0, f0, k);
    }
    auto stage = [&](int s, RFrag& cur, RFrag& nxt) {
#pragma unroll
        for (int t = 0; t < 24; ++t) resid_mfma<0>(acc, cur, t);
        __builtin_amdgcn_sched_barrier(0);
        mm_wait_vmcnt<(MRING - 2) * 8>();   // also: this wave's reads of stage s are done
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // second half, one MFMA per step: the next stage's 16 fragment reads (two a
        // step), then the 8 loads refilling this stage's slot, read by everyone by now
        u32x4* base = mm_lds + (s % MRING) * (4 * M_SLOTS);
#pragma unroll
        for (int t = 0; t < 24; ++t) {
            resid_mfma<2>(acc, cur, t);
            if (t < 8) {
                read_one(s + 1, nxt, 2 * t);
                read_one(s + 1, nxt, 2 * t + 1);
            } else if (t == 8) {
                next_rsrc();
            } else if (t < 17) {
                issue_one(base, t - 9);
            } else if (t == 17) {
                advance(s + MRING);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int s = 0; s < nst; s += 2) {
        stage(s, f0, f1);
        stage(s + 1, f1, f0);
    }
    mm_wait_vmcnt<0>();      // no load into this block's LDS may land after it ends

    float* O = R + ((int64_t)g * rpg) * d;
    const int nrem = (int)((rpg - n0) < MT ? (rpg - n0) : MT);
    const int arem = (int)((d - a0) < MT ? (d - a0) : MT);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int acol = 128 * w1 + 32 * j + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int nrow = 128 * w0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (nrow < nrem && acol < arem)
                    O[(n0 + nrow) * d + a0 + acol] = acc[i][j][v];
            }
        }
}

// ---------------------------------------------------------------------------
// Gram partials.  Tile (256 coordinates a) x (256 columns (j, q): 256 / M rows j
// of a group, M codes each), k from a0 to d.
// ---------------------------------------------------------------------------
// One-hot of 4 code bytes against q: the bf16 pair `onepair` where the byte
// equals q, else 0; returns the halfwords of bytes 0,1 (lo) and 2,3 (hi).
__device__ __forceinline__ u32x2 onehot4(uint32_t codes, uint32_t qq, uint32_t onepair) {
    const uint32_t y = codes ^ qq;                                   // zero byte <=> equal
    const uint32_t nz = (((y & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | y) & 0x80808080u;
    const uint32_t eq = (nz ^ 0x80808080u) >> 7;                     // 1 per equal byte
    const uint32_t m8 = (eq << 8) - eq;                              // 0xFF per equal byte
    u32x2 r;
    r[0] = __builtin_amdgcn_perm(m8, m8, 0x01010000u) & onepair;
    r[1] = __builtin_amdgcn_perm(m8, m8, 0x03030202u) & onepair;
    return r;
}

// One-hot B fragment (8 k-values of one (j, q) column, two k per dword, bf16) from
// the 8 codes c (one byte each) of row j.  For M <= 8 each code selects a byte of a
// per-lane table through v_perm_b32: tl / th hold, at byte q, the low / high byte
// of the bf16 weight (1.0 = 0x3F80, 0.5 = 0x3F00) and zero elsewhere, so the lookup
// yields the weight's two bytes where the code equals q and zero where it does not;
// two more byte permutes interleave them into bf16 pairs.  M = 16 takes codes up to
// 15, past the 8-byte table, and compares bytes instead.
template <int M>
__device__ __forceinline__ u32x4 gram_onehot(u32x2 c, uint32_t tl0, uint32_t tl1,
                                             uint32_t th0, uint32_t th1, uint32_t qq,
                                             uint32_t onepair) {
    u32x4 r;
    if constexpr (M <= 8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t lo = __builtin_amdgcn_perm(tl1, tl0, c[h]);
            const uint32_t hi = __builtin_amdgcn_perm(th1, th0, c[h]);
            r[2 * h] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            r[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
    } else {
        const u32x2 a = onehot4(c[0], qq, onepair), b = onehot4(c[1], qq, onepair);
        r = u32x4{a[0], a[1], b[0], b[1]};
    }
    return r;
}

// An accumulator value read out of its AGPR where it is used: keeps the 256
// accumulators in AGPRs until the epilogue bins them, one fragment at a time, instead
// of all being copied to (and spilled from) the 256 arch VGPRs at the loop's exit.
// Every use follows the last MFMA by a global-memory wait and two barriers, far past
// the MFMA result latency.
__device__ __forceinline__ float acc_read(float a) {
    float v;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// bins[OFF + k] += x[e] for the 4 values x[0..3] whose codes are the bytes of cw,
// each a bin index k < NB (<= 8) or 0x0C (no bin).  The codes are spread into byte-permute
// selectors (0x0C selects a zero byte), and for each bin a lookup in an 8-byte table
// holding 0x3C at byte k yields, per value, the high byte of the half-precision 1.0
// or 0; each accumulation is then one fused multiply-add of a float32 by a half.
template <int NB, int OFF, int M>
__device__ __forceinline__ void gram_bin4(float (&bins)[M], uint32_t cw, const float (&x)[4]) {
    const uint32_t s0 = __builtin_amdgcn_perm(cw, 0x0C0C0C0Cu, 0x05000400u);   // 0C c0 0C c1
    const uint32_t s1 = __builtin_amdgcn_perm(cw, 0x0C0C0C0Cu, 0x07000600u);   // 0C c2 0C c3
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const uint32_t t0 = k < 4 ? 0x3Cu << (8 * k) : 0u;
        const uint32_t t1 = k < 4 ? 0u : 0x3Cu << (8 * (k - 4));
        const uint32_t h0 = __builtin_amdgcn_perm(t1, t0, s0);
        const uint32_t h1 = __builtin_amdgcn_perm(t1, t0, s1);
        float b = bins[OFF + k];
        b = __builtin_fmaf(x[0], (float)__builtin_bit_cast(_Float16, (uint16_t)(h0 & 0xffffu)), b);
        b = __builtin_fmaf(x[1], (float)__builtin_bit_cast(_Float16, (uint16_t)(h0 >> 16)), b);
        b = __builtin_fmaf(x[2], (float)__builtin_bit_cast(_Float16, (uint16_t)(h1 & 0xffffu)), b);
        b = __builtin_fmaf(x[3], (float)__builtin_bit_cast(_Float16, (uint16_t)(h1 >> 16)), b);
        bins[OFF + k] = b;
    }
}

// The Gram kernel: 32-deep stages (two 16-deep k-blocks) through a ring of GRING
// stages, each stage the four F' bands (hi and lo of both k-blocks, 32 KB) and the
// codes of the block's rows j for those 32 coordinates (32 bytes a row, 4 KB); 4
// waves (one per SIMD), wave w owning coordinates a = 128 (w % 2) .. + 127 and
// columns (j, q) = 128 (w / 2) .. + 127 as 4 x 4 accumulators.  The one-hot operand
// is built in registers from the codes, one k-block ahead of its MFMAs.  One barrier
// per stage, between the k-blocks: after it the stage's slot is refilled and the next
// stage's fragments and codes are read, spread between the second k-block's MFMAs.
constexpr int GRING = 4;
constexpr int G_CSLOTS = 256;           // 16-byte slots of one code stage (128 rows x 32 B)

struct GFrag {
    u32x4 fh[2][4], fl[2][4];           // [k-block][i]: coordinates 128 (w % 2) + 32 i
    u32x2 c[2][4];                      // [k-block][jj]: codes of this lane's column
};

template <int M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gram(
    const uint8_t* __restrict__ P, int64_t rpg, int64_t d_out, int groups,
    const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo, int64_t a_pad,
    int64_t d, int ntn, int nta, int total, float* __restrict__ out,
    const unsigned long long* __restrict__ skip) {
    extern __shared__ u32x4 mm_lds[];
    if (skip && *skip != 0ull) return;
    u32x4* cring = mm_lds + GRING * 4 * M_SLOTS;
    const int lin = mm_remap(blockIdx.x);
    if (lin >= total) return;
    const int tn = lin % ntn;
    const int g = (lin / ntn) % groups;
    const int ta = lin / (ntn * groups);
    const int64_t a0 = (int64_t)ta * MT;
    const int64_t n0 = (int64_t)tn * MT;                 // first (j, q) column
    const int64_t N = rpg * M;
    const int64_t row_base = (int64_t)g * rpg;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w0 = wave & 1, w1 = wave >> 1;
    const uint32_t voff = band_voff(lane);

    const int64_t fg = (int64_t)g * d * a_pad;
    const int nst = (int)((d - a0) / 32);               // d % 32 == 0, a0 % 256 == 0
    const int ndst = (int)((((d - a0) < MT ? (d - a0) : MT)) / 32);   // stages at half weight
    const uint16_t* Fh = Fhi + fg + ((a0 >> 4) * a_pad + a0) * 16;
    const uint16_t* Fl = Flo + fg + ((a0 >> 4) * a_pad + a0) * 16;
    const int64_t fstep = a_pad * 16;                   // one 16-deep k-block

    // codes: wave w copies rows j = n0 / M + 32 w .. + 31 (lane L: row 32 w + L / 2,
    // bytes 16 (L % 2) .. + 15 of the stage's 32), rows past the group's end clamped
    // to its last row; their columns (j, q) are past N and never stored
    const int64_t j0 = n0 / M;
    const int64_t jb = (j0 + 32 * wave < rpg) ? j0 + 32 * wave : rpg - 1;
    const int64_t jr = (j0 + 32 * wave + (lane >> 1) < rpg) ? j0 + 32 * wave + (lane >> 1) : rpg - 1;
    const uint8_t* Pw = P + (row_base + jb) * d + a0;
    const uint32_t coff = (uint32_t)((jr - jb) * d) + 16u * (uint32_t)(lane & 1);

    // this lane's one-hot column: q = (lane % 32) % M in every 32-column fragment
    const int q = (lane & 31) % M;
    const uint64_t tl = (uint64_t)0x80u << (8 * (q & 7)), th = (uint64_t)0x3Fu << (8 * (q & 7));
    const uint32_t tl0 = (uint32_t)tl, tl1 = (uint32_t)(tl >> 32);
    const uint32_t th0 = (uint32_t)th, th1 = (uint32_t)(th >> 32);
    const uint32_t qq = (uint32_t)q * 0x01010101u;
    // code LDS offset (bytes, within a code stage) of fragment jj's row for this lane:
    // row (128 w1 + 32 jj + lane % 32) / M, i.e. cofs + jj (32 / M) rows (M divides 32)
    const int cofs = ((128 * w1 + (lane & 31)) / M) * 32 + 8 * (lane >> 5);

    // Stages are refilled in order; fo / co locate the next one, held at the last
    // stage once it is reached.
    int64_t fo = 0;
    uint32_t co = 0;
    __amdgpu_buffer_rsrc_t rs[5];
    auto next_rsrc = [&]() {
        rs[0] = band_rsrc(Fh + fo);
        rs[1] = band_rsrc(Fh + fo + fstep);
        rs[2] = band_rsrc(Fl + fo);
        rs[3] = band_rsrc(Fl + fo + fstep);
        rs[4] = __builtin_amdgcn_make_buffer_rsrc((void*)(Pw + co), (short)0, (int)0x7fffffff,
                                                  0x00020000);
    };
    auto advance = [&](int x) {
        if (x + 1 < nst) { fo += 2 * fstep; co += 32u; }
    };
    // load k (0..8) of a stage's refill: bands (k % 4) for rows 32 (wave + 4 (k / 4)),
    // then the codes
    auto issue_one = [&](int x, int k) {
        if (k < 8) {
            u32x4* base = mm_lds + (x % GRING) * (4 * M_SLOTS);
            band_to_lds(rs[k & 3], base + (k & 3) * M_SLOTS, wave + 4 * (k >> 2), voff);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs[4], (lds_ptr_t)(cring + (x % GRING) * G_CSLOTS + 64 * wave), 16, coff, 0, 0, 0);
        }
    };
    auto issue = [&](int x) {
        next_rsrc();
#pragma unroll
        for (int k = 0; k < 9; ++k) issue_one(x, k);
        advance(x);
    };
    // read k (0..23) of stage x: the 8 code reads, then the 16 F' fragments
    auto read_one = [&](int x, GFrag& f, int k) {
        if (k < 8) {
            const uint8_t* C = (const uint8_t*)(cring + (x % GRING) * G_CSLOTS);
            const int kb = k >> 2, jj = k & 3;
            f.c[kb][jj] = *(const u32x2*)(C + cofs + jj * (32 / M) * 32 + 16 * kb);
        } else {
            const u32x4* S = mm_lds + (x % GRING) * (4 * M_SLOTS);
            const int kk = k - 8, pl = kk >> 3, kb = (kk >> 2) & 1, i = kk & 3;
            const u32x4 v = S[(2 * pl + kb) * M_SLOTS + frag_slot(128 * w0 + 32 * i + (lane & 31), lane)];
            if (pl == 0) f.fh[kb][i] = v;
            else f.fl[kb][i] = v;
        }
    };
    // weight 0.5 on the diagonal tile, 1 above it, 0 on the padding stage past the end
    auto onehot = [&](const GFrag& f, int x, int kb, int jj) {
        const bool half = x < ndst, none = x >= nst;
        const uint32_t one = none ? 0u : (half ? 0x3F00u : 0x3F80u);
        return gram_onehot<M>(f.c[kb][jj], (half || none) ? 0u : tl0, (half || none) ? 0u : tl1,
                              none ? 0u : th0, none ? 0u : th1, qq, one | (one << 16));
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;

    // MFMA t (0..31) of k-block kb: plane t / 16 (hi, lo) of accumulator
    // ((t % 16) / 4, t % 4), so the same accumulator comes back every 16 MFMAs
    auto mfma = [&](const GFrag& f, const u32x4 (&oh)[4], int kb, int t) {
        const int pl = t >> 4, i = (t & 15) >> 2, jj = t & 3;
        const u32x4 av = pl ? f.fl[kb][i] : f.fh[kb][i];
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(oh[jj]),
                                                             acc[i][jj], 0, 0, 0);
    };

    // 9 loads per wave and stage: when stage x's second k-block is due, stage x + 1 has
    // landed once at most the loads of stages x + 2 .. x + GRING - 1 are outstanding
    GFrag f0, f1;
    u32x4 oh0[4], oh1[4];
    if (nst > 0) {
#pragma unroll
        for (int x = 0; x < GRING; ++x) issue(x);
        mm_wait_vmcnt<(GRING - 1) * 9>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int k = 0; k < 24; ++k) read_one(0, f0, k);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) oh0[jj] = onehot(f0, 0, 0, jj);
    }
    auto stage = [&](int x, GFrag& cur, GFrag& nxt) {
        // first k-block, with the one-hot of the second built between its MFMAs
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            mfma(cur, oh0, 0, t);
            if ((t & 3) == 1 && t < 16) oh1[t >> 2] = onehot(cur, x, 1, t >> 2);
            __builtin_amdgcn_sched_barrier(0);
        }
        mm_wait_vmcnt<(GRING - 2) * 9>();   // also: this wave's reads of stage x are done
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // second k-block: the next stage's codes and fragments (two reads a step), the
        // refill of this stage's slot (one load a step), the next stage's first one-hot
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            mfma(cur, oh1, 1, t);
            if (t < 12) {
                read_one(x + 1, nxt, 2 * t);
                read_one(x + 1, nxt, 2 * t + 1);
            } else if (t == 12) {
                next_rsrc();
            } else if (t < 22) {
                issue_one(x + GRING, t - 13);
            } else if (t == 22) {
                advance(x + GRING);
            } else if (t >= 24 && t < 28) {
                oh0[t - 24] = onehot(nxt, x + 1, 0, t - 24);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // an even number of stages: an odd count gets one more, a reload of the last stage
    // (as every refill past the end is) that adds nothing, its one-hot being zero
    const int nst2 = (nst + 1) & ~1;
    for (int x = 0; x < nst2; x += 2) {
        stage(x, f0, f1);
        stage(x + 1, f1, f0);
    }
    mm_wait_vmcnt<0>();      // no load into this block's LDS may land after it ends
    __syncthreads();

    __syncthreads();

    // ---- epilogue: bin T[a][(j,q)] by the code of coordinate a
    // stage the codes of the block's rows for its 256 coordinates: jrows x 256 bytes
    // (0x0C past d or past the group's rows: T is zero at a >= d, as the padded rows of
    // the F' planes are, and columns past N are not stored)
    constexpr int jrows = MT / M;
    uint8_t* ctile = (uint8_t*)mm_lds;
    for (int e = tid; e < jrows * (MT / 16); e += 256) {
        const int r = e / (MT / 16), c16 = (e - r * (MT / 16)) * 16;
        const int64_t jrow = j0 + r;
        u32x4 v = {0x0C0C0C0Cu, 0x0C0C0C0Cu, 0x0C0C0C0Cu, 0x0C0C0C0Cu};
        if (jrow < rpg && a0 + c16 < d) v = *(const u32x4*)(P + (row_base + jrow) * d + a0 + c16);
        *(u32x4*)(ctile + r * MT + c16) = v;
    }
    __syncthreads();
    float* xch = (float*)(ctile + jrows * MT);
    // one column fragment jj at a time (a compile-time index, so the accumulators stay
    // in registers)
    auto bin_fragment = [&](auto jjc) {
        constexpr int jj = decltype(jjc)::value;
        __builtin_amdgcn_sched_barrier(0);
        const int nl = 128 * w1 + 32 * jj + (lane & 31);
        const int jl = nl / M;
        float bins[M];
#pragma unroll
        for (int k = 0; k < M; ++k) bins[k] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int al = 128 * w0 + 32 * i + 8 * v4 + 4 * (lane >> 5);
                const uint32_t cw = *(const uint32_t*)(ctile + jl * MT + al);
                const float xv[4] = {acc_read(acc[i][jj][4 * v4]), acc_read(acc[i][jj][4 * v4 + 1]),
                                     acc_read(acc[i][jj][4 * v4 + 2]),
                                     acc_read(acc[i][jj][4 * v4 + 3])};
                if constexpr (M <= 8) {
                    gram_bin4<M, 0>(bins, cw, xv);
                } else {
                    // codes 8..15 -> 0..7 for the upper bins, 0..7 -> 0x0C for them, and
                    // the other way round for the lower bins
                    const uint32_t b3 = (cw >> 3) & 0x01010101u;
                    const uint32_t hi = (b3 << 8) - b3;                  // 0xFF per code >= 8
                    const uint32_t clo = (hi & 0x0C0C0C0Cu) | (~hi & cw);
                    const uint32_t chi = (hi & cw & 0x07070707u) | (~hi & 0x0C0C0C0Cu);
                    gram_bin4<8, 0>(bins, clo, xv);
                    gram_bin4<8, 8>(bins, chi, xv);
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
    };
    bin_fragment(std::integral_constant<int, 0>{});
    bin_fragment(std::integral_constant<int, 1>{});
    bin_fragment(std::integral_constant<int, 2>{});
    bin_fragment(std::integral_constant<int, 3>{});
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
constexpr size_t RESID_LDS = (size_t)MRING * 4 * M_SLOTS * 16;          // 128 KB
constexpr size_t GRAM_LDS = (size_t)GRING * (4 * M_SLOTS + G_CSLOTS) * 16;   // 144 KB

size_t lnq_gram_partial_floats(int64_t d_out, int64_t d, int m) {
    const int64_t nta = (d + MT - 1) / MT;
    return (size_t)nta * d_out * m * m;
}

hipError_t lnq_residual(const uint16_t* Ehi, const uint16_t* Elo, int64_t d_out, int64_t d,
                        int groups, const uint16_t* Fhi, const uint16_t* Flo, float* R,
                        const unsigned long long* skip, hipStream_t st) {
    const int64_t rpg = d_out / groups;
    const int64_t rpg_pad = lnq_pad256(rpg), a_pad = lnq_pad256(d);
    const int ntn = (int)(rpg_pad / MT);
    const int nta = (int)(a_pad / MT);
    const int total = ntn * nta * groups;
    const int grid = (total + 255) / 256 * 256;        // whole rounds for the XCD remap
    {
        hipError_t e = ensure_dynamic_lds((const void*)k_resid, RESID_LDS);
        if (e != hipSuccess) return e;
    }
    StageTimer tm(ST_LNQ_RESID, st);
    hipLaunchKernelGGL(k_resid, dim3((unsigned)grid), dim3(256), RESID_LDS, st, Ehi, Elo,
                       (int64_t)groups * rpg_pad, rpg_pad, Fhi, Flo, a_pad, d, rpg, ntn, nta,
                       total, R, skip);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

template <int M>
static hipError_t launch_gram(const uint8_t* P, int64_t d_out, int64_t d, int groups,
                              const uint16_t* Fhi, const uint16_t* Flo, float* part,
                              const unsigned long long* skip, hipStream_t st) {
    static_assert((MT / M) * MT + 64 * M * 4 <= GRAM_LDS, "Gram epilogue exceeds the LDS");
    const int64_t rpg = d_out / groups;
    const int ntn = (int)((rpg * M + MT - 1) / MT);
    const int nta = (int)((d + MT - 1) / MT);
    const int total = ntn * nta * groups;
    const int grid = (total + 255) / 256 * 256;
    {
        hipError_t e = ensure_dynamic_lds((const void*)k_gram<M>, GRAM_LDS);
        if (e != hipSuccess) return e;
    }
    StageTimer tm(ST_LNQ_GRAM, st);
    hipLaunchKernelGGL((k_gram<M>), dim3((unsigned)grid), dim3(256), GRAM_LDS, st, P, rpg, d_out,
                       groups, Fhi, Flo, lnq_pad256(d), d, ntn, nta, total, part, skip);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

hipError_t lnq_gram(const uint8_t* P, int m, int64_t d_out, int64_t d, int groups,
                    const uint16_t* Fhi, const uint16_t* Flo, float* part,
                    const unsigned long long* skip, hipStream_t st) {
    switch (m) {
        case 2: return launch_gram<2>(P, d_out, d, groups, Fhi, Flo, part, skip, st);
        case 4: return launch_gram<4>(P, d_out, d, groups, Fhi, Flo, part, skip, st);
        case 8: return launch_gram<8>(P, d_out, d, groups, Fhi, Flo, part, skip, st);
        case 16: return launch_gram<16>(P, d_out, d, groups, Fhi, Flo, part, skip, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gq
