// gla_norm.hip -- output norm and gate: a per-head RMSNorm of the recurrence
// output times a swish gate, forward and backward (gfx950).
//
// FLAT page ("FLAT: Flash Linear Attention on TPUs"), Full Linear Attention
// Layer: the layer's output is the per-head RMSNorm of o multiplied by a swish
// output gate.  Per row (b, t, h) of d channels:
//     r = 1 / sqrt(mean_j o_j^2 + eps),  n = o r,  y = gamma n swish(z),
// swish(z) = z sigmoid(z), one scale vector gamma[d] for every head.  Backward:
//     dz = dy gamma n swish'(z),  dn = dy gamma swish(z),
//     do = r (dn - n mean_j(dn_j n_j)),  dgamma = sum over rows of dy n swish(z).
//
// Work split: a lane loads 16 bytes of a row (8 bf16 or 4 fp32 channels), so a
// row of d channels is d / 8 (or d / 4) consecutive lanes and a wave covers a few
// whole rows with one contiguous request per tensor.  The row's sums of squares
// (and, backward, of dn n) are added across its lanes with xor shuffles.  Each
// wave keeps NU row groups in flight.  The backward's dgamma partials are summed
// over a workgroup in a fixed order and written once per workgroup; a second
// kernel adds the partials in a fixed order (no atomics).
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

namespace {

constexpr int NW = 4;   // waves per workgroup
constexpr int NU = 4;   // row groups in flight per wave

template <typename T, int D> struct NormShape {
    static constexpr int E = 16 / (int)sizeof(T);  // channels per lane
    static constexpr int LPR = D / E;              // lanes per row
    static constexpr int RPW = 64 / LPR;           // rows per wave-wide group
    typedef __attribute__((__vector_size__(16))) T vec;
};

__device__ __forceinline__ float sigm(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// sum over the LPR lanes of one row (xor shuffles stay inside the row's lanes)
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(64 * NW) void k_norm_gate_fwd(const NormArgs a) {
    using S = NormShape<T, D>;
    constexpr int E = S::E, LPR = S::LPR, RPW = S::RPW;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * NW + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * NW;
    const int sub = lane / LPR, c0 = (lane % LPR) * E;
    const int64_t rows = a.rows, ngroups = (rows + RPW - 1) / RPW;
    float gam[E];
    {
        const f32x4* gp = reinterpret_cast<const f32x4*>(a.gamma + c0);
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            const f32x4 v = gp[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) gam[4 * i + e] = v[e];
        }
    }
    for (int64_t g0 = wave; g0 < ngroups; g0 += nwaves * NU) {
        typename S::vec ov[NU], zv[NU];
        int64_t row[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            row[u] = (g0 + u * nwaves) * RPW + sub;
            const int64_t rr = row[u] < rows ? row[u] : rows - 1;  // (an existing row, unused)
            ov[u] = *reinterpret_cast<const typename S::vec*>((const T*)a.o + rr * D + c0);
            zv[u] = *reinterpret_cast<const typename S::vec*>((const T*)a.z + rr * D + c0);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) ss += (float)ov[u][e] * (float)ov[u][e];
            ss = row_sum<LPR>(ss);
            const float r = rsqrtf(ss * (1.f / D) + a.eps);
            typename S::vec yv;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float z = (float)zv[u][e];
                yv[e] = (T)(gam[e] * ((float)ov[u][e] * r) * (z * sigm(z)));
            }
            if (row[u] < rows) *reinterpret_cast<typename S::vec*>((T*)a.y + row[u] * D + c0) = yv;
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(64 * NW) void k_norm_gate_bwd(const NormArgs a) {
    using S = NormShape<T, D>;
    constexpr int E = S::E, LPR = S::LPR, RPW = S::RPW;
    __shared__ float sg[NW - 1][D];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t wave = (int64_t)blockIdx.x * NW + wv;
    const int64_t nwaves = (int64_t)gridDim.x * NW;
    const int sub = lane / LPR, c0 = (lane % LPR) * E;
    const int64_t rows = a.rows, ngroups = (rows + RPW - 1) / RPW;
    float gam[E], acc[E];
    {
        const f32x4* gp = reinterpret_cast<const f32x4*>(a.gamma + c0);
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            const f32x4 v = gp[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) gam[4 * i + e] = v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int64_t g0 = wave; g0 < ngroups; g0 += nwaves * NU) {
        typename S::vec ov[NU], zv[NU], gv[NU];
        int64_t row[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            row[u] = (g0 + u * nwaves) * RPW + sub;
            const int64_t rr = row[u] < rows ? row[u] : rows - 1;  // (an existing row, unused)
            ov[u] = *reinterpret_cast<const typename S::vec*>((const T*)a.o + rr * D + c0);
            zv[u] = *reinterpret_cast<const typename S::vec*>((const T*)a.z + rr * D + c0);
            gv[u] = *reinterpret_cast<const typename S::vec*>((const T*)a.dy + rr * D + c0);
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const bool live = row[u] < rows;
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) ss += (float)ov[u][e] * (float)ov[u][e];
            ss = row_sum<LPR>(ss);
            const float r = rsqrtf(ss * (1.f / D) + a.eps);
            float n[E], dn[E], dot = 0.f;
            typename S::vec dzv;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float z = (float)zv[u][e], dy = (float)gv[u][e];
                const float s = sigm(z), sw = z * s;
                n[e] = (float)ov[u][e] * r;
                const float dyn = dy * n[e];
                dzv[e] = (T)(dyn * gam[e] * s * (1.f + z * (1.f - s)));
                dn[e] = dy * gam[e] * sw;
                dot += dn[e] * n[e];
                if (live) acc[e] += dyn * sw;
            }
            dot = row_sum<LPR>(dot) * (1.f / D);
            typename S::vec dov;
#pragma unroll
            for (int e = 0; e < E; ++e) dov[e] = (T)(r * (dn[e] - n[e] * dot));
            if (live) {
                *reinterpret_cast<typename S::vec*>((T*)a.d_o + row[u] * D + c0) = dov;
                *reinterpret_cast<typename S::vec*>((T*)a.dz + row[u] * D + c0) = dzv;
            }
        }
    }
    // dgamma: the wave's rows (lanes sub = 0 .. RPW-1 of one channel block), then
    // the workgroup's waves in order
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
    if (wv > 0 && sub == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) sg[wv - 1][c0 + e] = acc[e];
    }
    __syncthreads();
    if (wv == 0 && sub == 0) {
        float* part = a.ws + (int64_t)blockIdx.x * D + c0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float s = acc[e];
#pragma unroll
            for (int w = 0; w < NW - 1; ++w) s += sg[w][c0 + e];
            part[e] = s;
        }
    }
}

// dgamma[c] = sum of the nparts partials [nparts][D], in a fixed order: a
// workgroup takes 64 channels; each of its 16 waves adds a sixteenth of the
// partials (all its loads issued at once), and the sixteenths are added in wave
// order.
constexpr int RW = 16;      // waves of the reduction
constexpr int RQ = 64;      // partials per wave at most
__global__ __launch_bounds__(64 * RW) void k_norm_gate_reduce(const float* ws, float* dgamma, int D,
                                                             int64_t nparts) {
    __shared__ float sq[RW - 1][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const bool live = c < D;
    const int cc = live ? c : 0;
    const int64_t q = (nparts + RW - 1) / RW;  // <= RQ (the host caps nparts)
    const int64_t p0 = wv * q, p1 = p0 + q < nparts ? p0 + q : nparts;
    float v[RQ];
#pragma unroll
    for (int j = 0; j < RQ; ++j) v[j] = p0 + j < p1 ? ws[(p0 + j) * D + cc] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < RQ; ++j) s += v[j];
    if (wv > 0) sq[wv - 1][lane] = s;
    __syncthreads();
    if (wv == 0 && live) {
#pragma unroll
        for (int w = 0; w < RW - 1; ++w) s += sq[w][lane];
        dgamma[c] = s;
    }
}

// grids (measured, bf16 d = 128, 524,288 rows): the forward at 2048 workgroups
// ran 83 us against 86 at 1536; the backward at 768 (three resident per compute
// unit at its register count) ran as fast as at 1024 and leaves fewer partials
constexpr int64_t kFwdMaxWG = 2048, kBwdMaxWG = 768;
static_assert(kBwdMaxWG <= RW * RQ, "the reduction takes at most RW * RQ partials");

template <typename T, int D> int64_t groups(int64_t rows) {
    constexpr int RPW = NormShape<T, D>::RPW;
    return (rows + RPW - 1) / RPW;
}

}  // namespace

template <typename T, int D>
int64_t norm_gate_partials(int64_t rows) {
    const int64_t wg = (groups<T, D>(rows) + NW * NU - 1) / (NW * NU);
    return wg < kBwdMaxWG ? wg : kBwdMaxWG;
}

template <typename T, int D>
hipError_t launch_norm_gate_fwd(const NormArgs& a, hipStream_t st) {
    int64_t wg = (groups<T, D>(a.rows) + NW * NU - 1) / (NW * NU);
    if (wg == 0) return hipSuccess;
    wg = wg < kFwdMaxWG ? wg : kFwdMaxWG;
    hipLaunchKernelGGL((k_norm_gate_fwd<T, D>), dim3((unsigned)wg), dim3(64 * NW), 0, st, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_norm_gate_bwd(const NormArgs& a, hipStream_t st) {
    const int64_t np = norm_gate_partials<T, D>(a.rows);
    if (np > 0) {
        hipLaunchKernelGGL((k_norm_gate_bwd<T, D>), dim3((unsigned)np), dim3(64 * NW), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_norm_gate_reduce, dim3((unsigned)((D + 63) / 64)), dim3(64 * RW), 0, st,
                       (const float*)a.ws, a.dgamma, D, np);
    return hipGetLastError();
}

#define GLA_NORM_INST(T, D)                                                       \
    template int64_t norm_gate_partials<T, D>(int64_t);                           \
    template hipError_t launch_norm_gate_fwd<T, D>(const NormArgs&, hipStream_t); \
    template hipError_t launch_norm_gate_bwd<T, D>(const NormArgs&, hipStream_t);
GLA_NORM_INST(float, 64)
GLA_NORM_INST(float, 128)
GLA_NORM_INST(bf16, 64)
GLA_NORM_INST(bf16, 128)
#undef GLA_NORM_INST

}  // namespace gla
