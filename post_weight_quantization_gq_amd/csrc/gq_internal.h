// Host-side interfaces between the C ABI (gq_api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace gq {

// ---- per-stage HIP-event timing (gq_api.hip); stage ids are gq_stage of gq.h
enum Stage {
    ST_GROUP_SCALE = 0, ST_FISHER_MFMA, ST_FISHER_FINALIZE, ST_FISHER_PLAIN, ST_LNQ_PREPARE,
    ST_LNQ_WF, ST_LNQ_INIT, ST_LNQ_U, ST_LNQ_SOLVE, ST_LNQ_SWEEP, ST_LNQ_SMALL, ST_COUNT
};
bool timing_on();
void timing_mark(Stage s, hipStream_t st, bool begin);
// Records a start event on construction and a stop event on destruction when
// timing is on; the launches in between are attributed to the stage.
struct StageTimer {
    Stage s;
    hipStream_t st;
    bool on;
    StageTimer(Stage s_, hipStream_t st_) : s(s_), st(st_), on(timing_on()) {
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

// ---- LNQ (gq_lnq.hip)
struct LnqSizes {
    size_t o_fhi, o_flo, o_dF, o_lam, o_V, o_U, o_R, o_dhi, o_dlo, o_whi, o_wlo;
    size_t o_objA, o_objB, o_objC, o_cnt, total;
    int gchunk;
};
struct LnqWs {
    uint16_t *fhi, *flo;          // F' planes [groups][d][d]
    float* dF;                    // diag F' [groups][d]
    double* lam;                  // [groups]
    float* V;                     // W F' [d_out][d]
    float* U;                     // F' P_j for gchunk groups [rows*m][d]
    float* R;                     // residual [d_out][d]
    uint16_t *dhi, *dlo;          // value changes of the current pass [d_out][d]
    uint16_t *whi, *wlo;          // float32 W split into bf16 planes (else null)
    double *objA, *objB, *objC;   // per-row objectives [d_out]
    unsigned long long* cnt;      // counters [16]
    int gchunk;                   // groups per U chunk
};

LnqSizes lnq_sizes(int64_t d_out, int64_t d, int groups, int m, bool w_f32);
LnqWs lnq_carve(void* base, const LnqSizes& z, bool w_f32);
hipError_t lnq_prepare(const float* F, int groups, int64_t d, double rho, const LnqWs& w,
                       hipStream_t st);
hipError_t lnq_compute_v(const void* W, bool w_bf16, int64_t d_out, int64_t d, int groups,
                         const LnqWs& w, hipStream_t st);
hipError_t lnq_init_run(const void* W, bool w_bf16, int64_t d_out, int64_t d, int m, float* C,
                        uint8_t* P, hipStream_t st);
hipError_t lnq_u_solve(int mode, const void* W, bool w_bf16, int64_t d_out, int64_t d,
                       int groups, int m, const uint8_t* P, float* C, const LnqWs& w, float* R,
                       double* obj_old, double* obj_new, unsigned long long* n_not_pd,
                       hipStream_t st);
hipError_t lnq_sweep_run(int block, const float* F, int64_t d_out, int64_t d, int groups,
                         const float* C, int m, uint8_t* P, const LnqWs& w,
                         const double* obj_in, double* obj_out, unsigned long long* counter,
                         hipStream_t st);
hipError_t lnq_reduce(const double* rows, int64_t n, double* out, hipStream_t st);
hipError_t lnq_zero_counter(unsigned long long* c, hipStream_t st);
hipError_t lnq_store_counter(const unsigned long long* c, int64_t* dst, hipStream_t st);

}  // namespace gq
