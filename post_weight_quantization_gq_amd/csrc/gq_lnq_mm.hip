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
// 256 x 256, 8 waves (two per SIMD) of 128 x 64 as 4 x 2 v_mfma_f32_32x32x16_bf16
// tiles.  The
// stages go through a ring of 4 LDS stages filled by direct buffer-to-LDS loads
// three stages ahead; a 32-byte operand row sits in two 16-byte slots, chunk c
// of row r in slot 2 r + (c ^ ((r >> 3) & 1)), so each quarter-wave fragment
// read (16 consecutive rows) touches 16 distinct bank groups.  The one-hot
// operand of k_gram is built once per stage into LDS, one stage ahead; k_gram
// takes 32-deep stages (two k-blocks) through a ring of 3.
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

// Copy one stage of a 256-row band (rows of 32 bytes) into 512 LDS slots: wave w
// (of 8) issues one instruction filling rows 32w .. 32w + 31; lane L takes row
// 32w + L/2 and slot L%2, i.e. chunk (L%2) ^ ((L/16)%2).
__device__ __forceinline__ void band_to_lds(__amdgpu_buffer_rsrc_t r, u32x4* dst, int wave,
                                            uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + 64 * wave), 16, voff,
                                             (uint32_t)wave * 1024u, 0, 0);
}

__device__ __forceinline__ uint32_t band_voff(int lane) {
    return (uint32_t)(lane >> 1) * 32u + 16u * (uint32_t)((lane & 1) ^ ((lane >> 4) & 1));
}

// fragment slot of row `row` (its low 5 bits from the lane) for a 16-deep k-step
__device__ __forceinline__ int frag_slot(int row, int lane) {
    return row * 2 + ((lane >> 5) ^ ((lane >> 3) & 1));
}

// ---------------------------------------------------------------------------
// R = E F'.  Tile (256 rows j of a group) x (256 coordinates a).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_resid(
    const uint16_t* __restrict__ Ehi, const uint16_t* __restrict__ Elo, int64_t erows,
    int64_t rpg_pad, const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo,
    int64_t a_pad, int64_t d, int64_t rpg, int ntn, int nta, int total, float* __restrict__ R,
    const unsigned long long* __restrict__ skip) {
    extern __shared__ u32x4 mm_lds[];
    if (skip && *skip != 0ull) return;
    const int lin = mm_remap(blockIdx.x);
    if (lin >= total) return;
    const int ta = lin % nta;
    const int tn = (lin / nta) % ntn;
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
    const int nst = (int)(d / 16);

    auto issue = [&](int s) {
        u32x4* base = mm_lds + (s % MRING) * (4 * M_SLOTS);
        band_to_lds(band_rsrc(Eh + s * estep), base, wave, voff);
        band_to_lds(band_rsrc(El + s * estep), base + M_SLOTS, wave, voff);
        band_to_lds(band_rsrc(Fh + s * fstep), base + 2 * M_SLOTS, wave, voff);
        band_to_lds(band_rsrc(Fl + s * fstep), base + 3 * M_SLOTS, wave, voff);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;

    {
        const int pre = nst < MRING - 1 ? nst : MRING - 1;
        for (int s = 0; s < pre; ++s) issue(s);
    }
    int slot = 0;
    for (int s = 0; s < nst; ++s) {
        // 4 load instructions per stage and wave: stage s has landed once at most
        // 4 x (later stages issued) are outstanding
        const int newer = ((s + MRING - 2 < nst) ? s + MRING - 2 : nst - 1) - s;
        if (newer >= 2) mm_wait_vmcnt<8>();
        else if (newer == 1) mm_wait_vmcnt<4>();
        else mm_wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (s + MRING - 1 < nst) issue(s + MRING - 1);
        const u32x4* S = mm_lds + slot * (4 * M_SLOTS);
        bf16x8 eh[4], el[4], fh[2], fl[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sl = frag_slot(128 * w0 + 32 * i + (lane & 31), lane);
            eh[i] = as_bf16x8(S[sl]);
            el[i] = as_bf16x8(S[M_SLOTS + sl]);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int sl = frag_slot(64 * w1 + 32 * jj + (lane & 31), lane);
            fh[jj] = as_bf16x8(S[2 * M_SLOTS + sl]);
            fl[jj] = as_bf16x8(S[3 * M_SLOTS + sl]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(eh[i], fh[jj], acc[i][jj], 0, 0, 0);
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(eh[i], fl[jj], acc[i][jj], 0, 0, 0);
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(el[i], fh[jj], acc[i][jj], 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
        slot = (slot + 1 == MRING) ? 0 : slot + 1;
    }

    float* O = R + ((int64_t)g * rpg) * d;
    const int nrem = (int)((rpg - n0) < MT ? (rpg - n0) : MT);
    const int arem = (int)((d - a0) < MT ? (d - a0) : MT);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int acol = 64 * w1 + 32 * jj + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int nrow = 128 * w0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (nrow < nrem && acol < arem)
                    O[(n0 + nrow) * d + a0 + acol] = acc[i][jj][v];
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

// The Gram kernel runs 32-deep stages (two 16-deep k-blocks) through a ring of
// GRING stages, to halve the per-stage barrier and fragment-read overhead against
// its 16 MFMAs per k-block and wave.
constexpr int GRING = 3;

template <int M>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gram(
    const uint8_t* __restrict__ P, int64_t rpg, int64_t d_out, int groups,
    const uint16_t* __restrict__ Fhi, const uint16_t* __restrict__ Flo, int64_t a_pad,
    int64_t d, int ntn, int nta, int total, float* __restrict__ out,
    const unsigned long long* __restrict__ skip) {
    extern __shared__ u32x4 mm_lds[];
    if (skip && *skip != 0ull) return;
    // LDS: ring of GRING stages of four bands (Fhi and Flo of two k-blocks); two
    // one-hot stages of two k-blocks (512 slots each); ring of GRING code stages
    // (slot 64 w + 32 h + c for column 32 w + c, codes 16 h .. 16 h + 15)
    u32x4* ohbuf = mm_lds + GRING * 4 * M_SLOTS;
    u32x4* cring = ohbuf + 4 * M_SLOTS;
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
    const int64_t k_begin = a0;
    const int nst = (int)((d - k_begin) / 32);          // d % 32 == 0, a0 % 256 == 0
    const int ndiag = (int)((((d - a0) < MT ? (d - a0) : MT)) / 16);   // k-blocks at half weight
    const uint16_t* Fh = Fhi + fg + ((k_begin >> 4) * a_pad + a0) * 16;
    const uint16_t* Fl = Flo + fg + ((k_begin >> 4) * a_pad + a0) * 16;
    const int64_t fstep = a_pad * 16;                   // one 16-deep k-block

    // code load: lane L of wave w copies codes 16 (L / 32) .. + 15 of stage x for
    // one-hot column c = 32 w + L % 32 ((j, q) = n0 + c); a row past the group's end
    // reads the group's first row and is masked when the one-hot is built
    const int ccol = 32 * wave + (lane & 31);
    const int64_t jl = n0 / M + ccol / M;
    const bool jvalid = jl < rpg;
    const uint8_t* Pg = P + row_base * d + k_begin;
    const uint32_t coff = (uint32_t)((jvalid ? jl : 0) * d) + 16u * (uint32_t)(lane >> 5);
    auto issue_codes = [&](int x) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Pg + (int64_t)x * 32), (short)0, (int)0x7fffffff, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(cring + (x % GRING) * 512 + 64 * wave),
                                                 16, coff, 0, 0, 0);
    };
    // thread t builds k-block kb = t / 256 of column c = t % 256
    const int bcol = tid & 255, bkb = tid >> 8;
    const int64_t bjl = n0 / M + bcol / M;
    const uint32_t bqq = (uint32_t)(bcol % M) * 0x01010101u;
    const bool bvalid = bjl < rpg;
    const int csl = 64 * (bcol >> 5) + 32 * bkb + (bcol & 31);
    const int osw = (bcol >> 3) & 1;
    auto build = [&](int x) {
        u32x4 cv = cring[(x % GRING) * 512 + csl];
        if (!bvalid) cv = u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        const uint32_t one = (2 * x + bkb < ndiag) ? 0x3F00u : 0x3F80u;   // 0.5 on the diagonal tile
        const uint32_t onepair = one | (one << 16);
        const u32x2 h0 = onehot4(cv[0], bqq, onepair), h1 = onehot4(cv[1], bqq, onepair);
        const u32x2 h2 = onehot4(cv[2], bqq, onepair), h3 = onehot4(cv[3], bqq, onepair);
        u32x4* O = ohbuf + ((x & 1) * 2 + bkb) * M_SLOTS + bcol * 2;
        O[0 ^ osw] = u32x4{h0[0], h0[1], h1[0], h1[1]};          // k 0..7 of the k-block
        O[1 ^ osw] = u32x4{h2[0], h2[1], h3[0], h3[1]};          // k 8..15
    };
    // batch x: the four bands of stage x, then the codes of stage x + 1 (5 loads per wave)
    auto issue = [&](int x) {
        u32x4* base = mm_lds + (x % GRING) * (4 * M_SLOTS);
        band_to_lds(band_rsrc(Fh + (2 * x) * fstep), base, wave, voff);
        band_to_lds(band_rsrc(Fh + (2 * x + 1) * fstep), base + M_SLOTS, wave, voff);
        band_to_lds(band_rsrc(Fl + (2 * x) * fstep), base + 2 * M_SLOTS, wave, voff);
        band_to_lds(band_rsrc(Fl + (2 * x + 1) * fstep), base + 3 * M_SLOTS, wave, voff);
        if (x + 1 < nst) issue_codes(x + 1);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;

    if (nst > 0) {
        issue_codes(0);
        const int pre = nst < GRING - 1 ? nst : GRING - 1;
        for (int x = 0; x < pre; ++x) issue(x);
        // codes of stage 0: the oldest load of this wave
        if (pre >= 2) mm_wait_vmcnt<9>();
        else mm_wait_vmcnt<4>();
        __builtin_amdgcn_s_barrier();
        build(0);
    }
    int slot = 0;
    for (int s = 0; s < nst; ++s) {
        // batch s (bands of s, codes of s + 1) has landed once at most 4 loads of
        // this wave (batch s + 1, if issued) are outstanding
        if (s + 1 < nst) mm_wait_vmcnt<4>();
        else mm_wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (s + GRING - 1 < nst) issue(s + GRING - 1);
        const u32x4* S = mm_lds + slot * (4 * M_SLOTS);
        const u32x4* OH = ohbuf + (s & 1) * 2 * M_SLOTS;
        bf16x8 fh[2][4], fl[2][4], oh[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = frag_slot(128 * w0 + 32 * i + (lane & 31), lane);
                fh[kb][i] = as_bf16x8(S[kb * M_SLOTS + sl]);
                fl[kb][i] = as_bf16x8(S[(2 + kb) * M_SLOTS + sl]);
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                oh[kb][jj] = as_bf16x8(OH[kb * M_SLOTS + frag_slot(64 * w1 + 32 * jj + (lane & 31), lane)]);
        }
        // the one-hot of stage s + 1 (past the last stage it fills a buffer no one
        // reads, from a ring slot in bounds), built while the MFMAs of stage s run
        build(s + 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh[kb][i], oh[kb][jj], acc[i][jj], 0, 0, 0);
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl[kb][i], oh[kb][jj], acc[i][jj], 0, 0, 0);
                }
        // order: the 20 fragment reads and the code read, then one MFMA per two
        // VALU operations of the build, its LDS writes, the remaining MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 21, 0);
#pragma unroll
        for (int k = 0; k < 22; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
        slot = (slot + 1 == GRING) ? 0 : slot + 1;
    }
    __syncthreads();

    // ---- epilogue: bin T[a][(j,q)] by the code of coordinate a
    // stage the codes of the block's rows for its 256 coordinates: jrows x 256 bytes
    constexpr int jrows = MT / M;
    uint8_t* ctile = (uint8_t*)mm_lds;
    for (int e = tid; e < jrows * (MT / 16); e += 512) {
        const int r = e / (MT / 16), c16 = (e - r * (MT / 16)) * 16;
        const int64_t jr = n0 / M + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (jr < rpg && a0 + c16 < d) v = *(const u32x4*)(P + (row_base + jr) * d + a0 + c16);
        *(u32x4*)(ctile + r * MT + c16) = v;
    }
    __syncthreads();
    float* xch = (float*)(ctile + jrows * MT);
    const int arem = (int)((d - a0) < MT ? (d - a0) : MT);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int nl = 64 * w1 + 32 * jj + (lane & 31);
        const int jr = nl / M;
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

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
constexpr size_t RESID_LDS = (size_t)MRING * 4 * M_SLOTS * 16;          // 128 KB
constexpr size_t GRAM_LDS = ((size_t)(GRING * 4 + 4) * M_SLOTS + GRING * 512) * 16;   // 152 KB

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
    hipLaunchKernelGGL(k_resid, dim3((unsigned)grid), dim3(512), RESID_LDS, st, Ehi, Elo,
                       (int64_t)groups * rpg_pad, rpg_pad, Fhi, Flo, a_pad, d, rpg, ntn, nta,
                       total, R, skip);
    GQ_LAUNCH_CHECK();
    return hipSuccess;
}

template <int M>
static hipError_t launch_gram(const uint8_t* P, int64_t d_out, int64_t d, int groups,
                              const uint16_t* Fhi, const uint16_t* Flo, float* part,
                              const unsigned long long* skip, hipStream_t st) {
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
    hipLaunchKernelGGL((k_gram<M>), dim3((unsigned)grid), dim3(512), GRAM_LDS, st, P, rpg, d_out,
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
