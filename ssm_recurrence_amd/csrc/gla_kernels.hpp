// gla_kernels.hpp -- host-visible launch entry points of the gfx950 kernels
// (internal to the library; the public ABI is include/gla.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

enum { MODE_OUT = 0, MODE_STATES = 1, MODE_DSTATE = 2 };

struct PassArgs {
    const void *q, *k, *v, *g, *dO;
    const float *h0, *dhT;
    const int32_t* seg;
    void* o;
    float *hT, *dh0;
    float* ws_S;   // [B*H][NC+1][DK][DV]: state entering each chunk, then the final state
    float* ws_dS;  // [B*H][NC][DK][DV]: gradient of the state at each chunk's end
    int64_t B, T, H, Hqk;
};

struct GradArgs {
    const void *q, *k, *v, *g, *dO;
    const int32_t* seg;
    const float* ws_S;
    const float* ws_dS;
    void *dq, *dk, *dv, *dg;
    float *ws_dq, *ws_dk;  // per-head fp32 [B][T][H][DK] when heads share q/k
    int64_t B, T, H, Hqk;
};

template <typename T, bool VEC, int DK, int DV, int MODE>
hipError_t launch_pass(const PassArgs& a, hipStream_t st);

template <typename T, bool VEC, int DK, int DV, int NV>
hipError_t launch_fwd(const PassArgs& a, hipStream_t st);

template <typename T, bool VEC, int DK, int DV>
hipError_t launch_grad(const GradArgs& a, hipStream_t st);

template <typename T, int DK>
hipError_t launch_group_sum(const float* src, void* dst, int64_t B, int64_t Tn, int64_t H,
                            int64_t Hqk, hipStream_t st);

}  // namespace gla
