// gla_kernels.hpp -- host-visible launch entry points of the gfx950 kernels
// (internal to the library; the public ABI is include/gla.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

struct PassArgs {
    const void *q, *k, *v, *g, *dO;
    const float *h0, *dhT;
    const int32_t* seg;
    void* o;
    float *hT, *dh0;
    float* ws_S;   // state pass output, [B*H][NC+1][DK][DV] in the input dtype
    int64_t B, T, H, Hqk;
    // exact sequence split: P pieces of PL chunks each (P = 1: no split)
    int64_t P, PL;
    const float* S_in;   // [B*H][P][DK][DV]: state entering each piece (P > 1)
    float *L_out, *D_out;  // piece summaries: local end state [B*H][P][DK][DV], decay [B*H][P][DK]
};


struct RevArgs {
    const void *q, *k, *v, *g, *dO;
    const int32_t* seg;
    const void* ws_S;   // [B*H][NC+1][DK][DV] in the input dtype: state entering each chunk, then hT
    const float* dhT;
    void *dq, *dk, *dv, *dg;
    float* dh0;
    float *ws_dq, *ws_dk;  // per-head fp32 [B][T][H][DK] when heads share q/k
    float *ws_xs, *ws_bnd; // scalar gate: per-slice partial sums [B*H][slices][T], [B*H][slices][NC]
    int64_t B, T, H, Hqk;
    int64_t P, PL;          // exact sequence split (P = 1: none)
    const float* dS_out;    // [B*H][P][DK][DV]: gradient of the state at each piece's end (P > 1)
};

// summary modes of the state pass: per-chunk states, or per-piece summaries
enum { ST_STATES = 0, ST_SUM_FWD = 1, ST_SUM_REV = 2 };

template <typename T, bool VEC, int DK, int DV>
hipError_t launch_states(const PassArgs& a, int mode, hipStream_t st);

// S_in(0) = init, S_in(p+1) = D_p * S_in(p) + L_p (rev: from the last piece down)
hipError_t launch_piece_combine(const float* L, const float* D, const float* init, float* out,
                                int64_t BH, int64_t P, int DK, int DV, bool rev, hipStream_t st);

template <typename T, bool VEC, int DK, int DV>
hipError_t launch_rev(const RevArgs& a, hipStream_t st);

template <typename T, bool VEC, int DK, int DV, int NV>
hipError_t launch_fwd(const PassArgs& a, hipStream_t st);

template <typename T, int DK>
hipError_t launch_group_sum(const float* src, void* dst, int64_t B, int64_t Tn, int64_t H,
                            int64_t Hqk, hipStream_t st);

}  // namespace gla
