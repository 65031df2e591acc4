// Host-side interfaces between the C ABI (gq_api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace gq {

// ---- per-stage HIP-event timing (gq_api.hip); stage ids are gq_stage of gq.h
enum Stage {
    ST_GROUP_SCALE = 0, ST_FISHER_MFMA, ST_FISHER_FINALIZE, ST_FISHER_PLAIN, ST_LNQ_PREPARE,
    ST_LNQ_RESID, ST_LNQ_INIT, ST_LNQ_GRAM, ST_LNQ_SOLVE, ST_LNQ_SWEEP, ST_LNQ_SMALL, ST_FISHER_PACK,
    ST_LNQ_DELTA, ST_LUT_PACK, ST_LUT_GEMV, ST_FISHER_H2D, ST_GANQ_CHOL, ST_GANQ_PASS, ST_COUNT
};
// Raise a kernel's dynamic-LDS limit to at least `bytes` on the current device, once per
// kernel, device and size (the attribute belongs to the device that is current).
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);

bool timing_on(Stage s);
void timing_mark(Stage s, hipStream_t st, bool begin);
// Records a start event on construction and a stop event on destruction when
// timing is on; the launches in between are attributed to the stage.
struct StageTimer {
    Stage s;
    hipStream_t st;
    bool on;
    StageTimer(Stage s_, hipStream_t st_) : s(s_), st(st_), on(timing_on(s_)) {
        if (on) timing_mark(s, st, true);
    }
    ~StageTimer() {
        if (on) timing_mark(s, st, false);
    }
};

// ---- Fisher (gq_fisher.hip)
size_t fisher_workspace(int64_t n, int64_t d_in, int groups, bool bf16);
hipError_t fisher_run(const void* X, const void* G, bool bf16, int64_t n, int64_t d_in,
                      int64_t d_out, int groups, float* F, int accumulate, void* ws,
                      hipStream_t st);

// ---- LNQ (gq_lnq.hip, gq_lnq_mm.hip)
// The bf16 planes of F' ([groups][d / 16][a_pad][16]) and of E = C[P] - W
// ([d / 16][groups * rpg_pad][16]) are blocked by 16 along k: element (row, k) of a
// plane with `rows` rows sits at ((k / 16) * rows + row) * 16 + k % 16.  Rows are
// padded with zeros to whole 256-row tiles.
__host__ __device__ inline int64_t lnq_pad256(int64_t x) { return (x + 255) / 256 * 256; }

struct LnqSizes {
    size_t o_fhi, o_flo, o_dF, o_lam, o_R, o_ehi, o_elo, o_part;
    size_t o_objA, o_objB, o_objC, o_cnt, o_pprev, o_afull, o_clist, o_ccount, o_order, o_dA;
    size_t o_items, o_nitems;
    size_t total;
};
struct LnqWs {
    uint16_t *fhi, *flo;          // F' planes, k-blocked: [groups][d / 16][a_pad][16]
    float* dF;                    // diag F' [groups][d]
    double* lam;                  // [groups]
    float* R;                     // residual F'(C[P] - W) [d_out][d]
    uint16_t *ehi, *elo;          // C[P] - W as k-blocked bf16 planes [d / 16][groups * rpg_pad][16]
    float* part;                  // Gram partials [d / 256][d_out * m][m]
    double *objA, *objB, *objC;   // per-row objectives [d_out]
    unsigned long long* cnt;      // [0] moves of the pass, [1] rows not positive definite,
                                  // [2] update mode of the next codebook step (0 from
                                  // scratch, 1 from the changed coordinates)
    uint8_t* pprev;               // codes before the last assignment pass [d_out][d]
    double* afull;                // A_j = P_j^T F' P_j of the last codebook step [d_out][m][m]
    uint32_t* clist;              // moves of the last pass per row, ascending [d_out][d]:
                                  // coordinate | old code << 16 | new code << 24
    int* ccount;                  // number of moves per row [d_out]
    int* order;                   // rows, most moves first [d_out]
    unsigned long long* items;    // work items of the update, longest first
    int* nitems;                  // their number
    float* dA;                    // per (row, coordinate slice): share of A_new - A_old
    int sb_shift = 9;             // log2 of the assignment pass's super-block (64 .. 512),
                                  // shared by the pass and the update from its moves
};

LnqSizes lnq_sizes(int64_t d_out, int64_t d, int groups, int m);
LnqWs lnq_carve(void* base, const LnqSizes& z);
size_t lnq_gram_partial_floats(int64_t d_out, int64_t d, int m);
// lambda_g = rho * mean(diag F_g) + lam_abs, the F' planes and diag(F')
hipError_t lnq_prepare(const float* F, int groups, int64_t d, double rho, double lam_abs,
                       const LnqWs& w, hipStream_t st);
hipError_t lnq_init_run(const void* W, bool w_bf16, int64_t d_out, int64_t d, int m, float* C,
                        uint8_t* P, hipStream_t st);
// uniform min-max grid per row (float32) and nearest codes
hipError_t grid_init_run(const void* W, bool w_bf16, int64_t d_out, int64_t d, int m, float* C,
                         uint8_t* P, hipStream_t st);
// `skip` (device, may be null): the launch does nothing when *skip != 0
hipError_t lnq_residual(const uint16_t* Ehi, const uint16_t* Elo, int64_t d_out, int64_t d,
                        int groups, const uint16_t* Fhi, const uint16_t* Flo, float* R,
                        const unsigned long long* skip, hipStream_t st);
hipError_t lnq_gram(const uint8_t* P, int m, int64_t d_out, int64_t d, int groups,
                    const uint16_t* Fhi, const uint16_t* Flo, float* part,
                    const unsigned long long* skip, hipStream_t st);
// codebook step on every row; obj_before[j] = objective of (C, P) before it.  With
// `mode` (device, may be null) set to 1, A and the residual are brought up to date
// from the coordinates the last pass changed (w.pprev -> P, F the raw Fisher)
// instead of being recomputed.
hipError_t lnq_codebook_step(const float* F, const void* W, bool w_bf16, int64_t d_out, int64_t d,
                             int groups, int m, const uint8_t* P, float* C, const LnqWs& w,
                             double* obj_before, unsigned long long* n_not_pd,
                             const unsigned long long* mode, hipStream_t st);
hipError_t lnq_objective_rows(const void* W, bool w_bf16, int64_t d_out, int64_t d, int groups,
                              int m, const uint8_t* P, const float* C, const LnqWs& w,
                              double* obj, hipStream_t st);
// assignment pass (super-blocks of 1 << w.sb_shift coordinates); obj_start/obj_end[j] =
// objective before / after it (may be null); record: list the moves of each row (w.clist,
// w.ccount) for an update from them
hipError_t lnq_sweep_step(const float* F, const void* W, bool w_bf16, int64_t d_out,
                          int64_t d, int groups, const float* C, int m, uint8_t* P,
                          const LnqWs& w, double* obj_start, double* obj_end,
                          unsigned long long* counter, bool record, hipStream_t st);
hipError_t lnq_reduce(const double* rows, int64_t n, double* out, hipStream_t st);
hipError_t lnq_zero_counter(unsigned long long* c, int n, hipStream_t st);
// after iteration t: trace[0..1] = sums of objA and objB (if trace), *n_changed = cnt[0]
// (if n_changed), cnt[2] = (0 <= incr_max && cnt[0] <= incr_max), cnt[0] = 0
hipError_t lnq_iter_tail(const double* objA, const double* objB, int64_t n, double* trace,
                         unsigned long long* cnt, int64_t* n_changed, int64_t incr_max,
                         hipStream_t st);
hipError_t lnq_store_counter(const unsigned long long* c, int64_t* dst, hipStream_t st);
// *bad += number of rows j with |claimed[j] - fresh[j]| > tol |start[j]| (or not finite)
hipError_t lnq_check_claim(const double* start, const double* claimed, const double* fresh,
                           int64_t n, double tol, unsigned long long* bad, hipStream_t st);
// *flag |= 1 when any of the n float32 / bfloat16 values at p is NaN or +-Inf
hipError_t scan_nonfinite(const void* p, bool bf16, int64_t n, unsigned long long* flag,
                          hipStream_t st);

// LUT dequantisation GEMV (gq_lut.hip)
int64_t lut_row_words(int64_t d_in, int bits);          // 32-bit words per packed row
bool lut_gemv_fits(int64_t d_in, int bits, int batch);
hipError_t lut_pack_run(const uint8_t* P, int64_t d_out, int64_t d_in, int bits, uint32_t* Q,
                        hipStream_t st);
hipError_t lut_gemv_run(const uint32_t* Q, const float* C, int64_t d_out, int64_t d_in, int bits,
                        const void* x, bool x_bf16, int batch, float* y, hipStream_t st);

// GANQ-style assignment (gq_ganq.hip)
struct GanqWs {
    double* A;                    // F' then its Cholesky factor L (lower) [groups][d][d]
    uint16_t *uhi, *ulo;          // U = L^T as k-blocked bf16 planes [groups][d / 16][a_pad][16]
    float* dL;                    // diag L [groups][d]
    double* Linv;                 // inverse of the current diagonal block [groups][64][64]
    int* bad;                     // F'_g not positive definite [groups]
};
size_t ganq_extra_bytes(int64_t d, int groups);
GanqWs ganq_carve(void* base, int64_t d, int groups);
hipError_t ganq_factor(const float* F, const double* lam, int64_t d, int groups, const GanqWs& w,
                       hipStream_t st);
hipError_t ganq_factor_out(const GanqWs& w, int64_t d, int groups, float* L, int* bad_out,
                           hipStream_t st);
hipError_t ganq_assign_run(const GanqWs& g, int64_t d, int64_t d_out, int groups, const float* C,
                           int m, uint8_t* P, const void* W, bool w_bf16, float* S,
                           unsigned long long* counter, hipStream_t st);

}  // namespace gq
