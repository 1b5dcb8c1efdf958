// gla_group.hip -- deterministic sum of per-head dq / dk over the heads that
// share one q/k head (FLAT page, "FLAT: Flash Linear Attention on TPUs",
// Pallas Kernels > Gated Linear Attention: each input may be shared by a group
// of heads; its gradient is the sum over the group).  Fixed summation order,
// no atomics.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// dq[b,t,hq,:] = sum over the G heads h of group hq of src[b,t,h,:]
// (dst rows are ld_dst elements apart; src is packed [rows][H][DK])
template <typename T, int DK>
__global__ __launch_bounds__(NT) void k_group_sum(const float* src, T* dst, int64_t ld_dst,
                                                   int64_t rows, int64_t H, int64_t Hqk) {
    const int64_t G = H / Hqk;
    const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;  // over rows * Hqk * DK
    const int64_t total = rows * Hqk * DK;
    if (idx >= total) return;
    const int64_t c = idx % DK;
    const int64_t hq = (idx / DK) % Hqk;
    const int64_t bt = idx / (DK * Hqk);
    float s = 0.f;
    for (int64_t h = hq * G; h < (hq + 1) * G; ++h) s += src[(bt * H + h) * DK + c];
    dst[bt * ld_dst + hq * DK + c] = from_f32<T>(s);
}

template <typename T, int DK>
hipError_t launch_group_sum(const float* src, void* dst, int64_t ld_dst, int64_t B, int64_t Tn,
                            int64_t H, int64_t Hqk, hipStream_t st) {
    const int64_t total = B * Tn * Hqk * DK;
    if (total == 0) return hipSuccess;
    const int64_t grid = (total + NT - 1) / NT;
    hipLaunchKernelGGL((k_group_sum<T, DK>), dim3((unsigned)grid), dim3(NT), 0, st, src, (T*)dst,
                       ld_dst, B * Tn, H, Hqk);
    return hipGetLastError();
}

template hipError_t launch_group_sum<float, 64>(const float*, void*, int64_t, int64_t, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_group_sum<float, 128>(const float*, void*, int64_t, int64_t, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_group_sum<bf16, 64>(const float*, void*, int64_t, int64_t, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_group_sum<bf16, 128>(const float*, void*, int64_t, int64_t, int64_t, int64_t, int64_t, hipStream_t);

}  // namespace gla
