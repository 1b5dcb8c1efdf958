// gla_conv.hip -- short depthwise causal convolution with bias and SiLU, forward
// and backward (gfx950).
//
// FLAT page ("FLAT: Flash Linear Attention on TPUs"), Depthwise Causal Short
// Convolution: z_t = b + sum_k W_k * x_{t-(K-1-k)}, y_t = SiLU(z_t), per channel;
// the backward passes dy through SiLU' to dz, forms dx as the anti-causal
// correlation of dz with the same taps, and reduces x-shifted-times-dz (dW) and
// dz (db) over every position.  As on the page, the convolution is a sum of K
// shifted copies on the vector ALUs: a depthwise 4-tap filter has no
// contraction for the matrix cores to do.
//
// Work split: a lane owns 4 or 8 consecutive channels (8 or 16 bytes of a bf16
// row), so a wave reads 256 or 512 channels of a time step as one contiguous request;
// the wave walks a strip of CL time steps keeping the last K-1 inputs (and, in
// the backward, the next K-1 values of dz) in registers, so every input row is
// requested once plus a K-1 row halo per strip.  A workgroup's four waves take
// four consecutive strips of the same channels; the backward sums their dW and
// db partials in LDS and writes one partial per workgroup, which a second kernel
// reduces in a fixed order (no atomics: results do not depend on scheduling).
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

namespace {

constexpr int CK = 4;         // taps
constexpr int CL = 64;        // time steps per wave
constexpr int CW = 4;         // waves per workgroup (consecutive strips)
constexpr int CTH = 64 * CW;  // threads per workgroup
constexpr int CVMIN = 4;      // channels per lane in the narrowest layout; C is a multiple of 8

// CV consecutive channels (4 or 8) of one time step, as stored
template <typename T, int CV> struct Row {
    typedef __attribute__((__vector_size__(CV * sizeof(T)))) T vec;
    vec v;
    __device__ __forceinline__ void load(const T* p) { v = *reinterpret_cast<const vec*>(p); }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};

template <typename T, int CV>
__device__ __forceinline__ void store_row(T* p, const float (&v)[CV]) {
    typename Row<T, CV>::vec o;
#pragma unroll
    for (int e = 0; e < CV; ++e) o[e] = (T)v[e];
    *reinterpret_cast<typename Row<T, CV>::vec*>(p) = o;
}

__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

template <int CV>
struct Taps {
    float w[CK][CV], b[CV];
    __device__ __forceinline__ void load(const ConvArgs& a, int64_t c0) {
#pragma unroll
        for (int k = 0; k < CK; ++k) {
            Row<float, CV> r;
            r.load(a.w + k * a.C + c0);
#pragma unroll
            for (int e = 0; e < CV; ++e) w[k][e] = r.get(e);
        }
#pragma unroll
        for (int e = 0; e < CV; ++e) b[e] = 0.f;
        if (a.bias) {
            Row<float, CV> r;
            r.load(a.bias + c0);
#pragma unroll
            for (int e = 0; e < CV; ++e) b[e] = r.get(e);
        }
    }
};

// Forward: y_t = SiLU(b + sum_k W_k x_{t-(K-1-k)}) for the lane's 8 channels and
// the wave's strip of time steps.
template <typename T, int CV, int CB>
__global__ __launch_bounds__(CTH) void k_conv_fwd(const ConvArgs a) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * CV;
    const int64_t t0 = ((int64_t)blockIdx.y * CW + wv) * CL;
    const int64_t T_ = a.T, C_ = a.C;
    if (c0 >= C_ || t0 >= T_) return;  // no barriers in this kernel
    const T* x = (const T*)a.x + (int64_t)blockIdx.z * T_ * C_ + c0;
    T* y = (T*)a.y + (int64_t)blockIdx.z * T_ * C_ + c0;
    Taps<CV> tp;
    tp.load(a, c0);

    // the K-1 inputs before the strip (zero before t = 0)
    float win[CK - 1][CV];
#pragma unroll
    for (int j = 0; j < CK - 1; ++j) {
        const int64_t t = t0 - (CK - 1) + j;
        Row<T, CV> r;
        r.load(x + (t >= 0 ? t : 0) * C_);
#pragma unroll
        for (int e = 0; e < CV; ++e) win[j][e] = t >= 0 ? r.get(e) : 0.f;
    }
    const int64_t tend = t0 + CL < T_ ? t0 + CL : T_;
    for (int64_t tb = t0; tb < tend; tb += CB) {
        // CB rows requested together (a row past the end reads the last row, unused)
        Row<T, CV> r[CB];
#pragma unroll
        for (int i = 0; i < CB; ++i) r[i].load(x + (tb + i < T_ ? tb + i : T_ - 1) * C_);
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            float xt[CV], out[CV];
#pragma unroll
            for (int e = 0; e < CV; ++e) {
                xt[e] = r[i].get(e);
                float z = tp.b[e] + tp.w[CK - 1][e] * xt[e];
#pragma unroll
                for (int k = 0; k < CK - 1; ++k) z += tp.w[k][e] * win[k][e];
                out[e] = z * sigmoid(z);
            }
            if (tb + i < tend) store_row<T, CV>(y + (tb + i) * C_, out);
#pragma unroll
            for (int e = 0; e < CV; ++e) {
#pragma unroll
                for (int k = 0; k < CK - 2; ++k) win[k][e] = win[k + 1][e];
                win[CK - 2][e] = xt[e];
            }
        }
    }
}

// Backward: dz_u = dy_u SiLU'(z_u) for u in the strip and the K-1 steps after it,
// dx_t = sum_k W_k dz_{t+(K-1-k)}, and the lane's partial sums of x-shifted times
// dz (dW) and of dz (db) over the strip; the workgroup's four strips are summed in
// LDS and written as one partial [K+1][C] per workgroup.
template <typename T, int CV, int CB>
__global__ __launch_bounds__(CTH) void k_conv_bwd(const ConvArgs a) {
    __shared__ float sred[CW - 1][CK + 1][CV][64];  // (CV = 8: 30 KB)
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * CV;
    const int64_t t0 = ((int64_t)blockIdx.y * CW + wv) * CL;
    const int64_t T_ = a.T, C_ = a.C;
    const bool live = c0 < C_;  // (every wave reaches the barrier below)
    const int64_t cc = live ? c0 : 0;
    const T* x = (const T*)a.x + (int64_t)blockIdx.z * T_ * C_ + cc;
    const T* dy = (const T*)a.dy + (int64_t)blockIdx.z * T_ * C_ + cc;
    T* dx = (T*)a.dx + (int64_t)blockIdx.z * T_ * C_ + cc;
    Taps<CV> tp;
    tp.load(a, cc);

    float acc[CK + 1][CV];  // dW_0 .. dW_{K-1}, db
#pragma unroll
    for (int k = 0; k <= CK; ++k)
#pragma unroll
        for (int e = 0; e < CV; ++e) acc[k][e] = 0.f;

    if (live && t0 < T_) {
        float xw[CK - 1][CV];   // x_{u-3} .. x_{u-1}
        float dzw[CK - 1][CV];  // dz_{u-3} .. dz_{u-1}
#pragma unroll
        for (int j = 0; j < CK - 1; ++j) {
            const int64_t t = t0 - (CK - 1) + j;
            Row<T, CV> r;
            r.load(x + (t >= 0 ? t : 0) * C_);
#pragma unroll
            for (int e = 0; e < CV; ++e) {
                xw[j][e] = t >= 0 ? r.get(e) : 0.f;
                dzw[j][e] = 0.f;
            }
        }
        const int64_t send = t0 + CL < T_ ? t0 + CL : T_;  // end of the strip
        const int64_t uend = send + (CK - 1) < T_ ? send + (CK - 1) : T_;  // dz needed up to here
        for (int64_t ub = t0; ub < send + (CK - 1); ub += CB) {
            Row<T, CV> rx[CB], rg[CB];
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                const int64_t u = ub + i < T_ ? ub + i : T_ - 1;
                rx[i].load(x + u * C_);
                rg[i].load(dy + u * C_);
            }
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                const int64_t u = ub + i;
                if (u >= send + (CK - 1)) break;
                const bool inT = u < uend;       // dz_u exists (u < T)
                const bool inS = u < send;       // u is in the strip: dW, db
                float xu[CV], dzu[CV];
#pragma unroll
                for (int e = 0; e < CV; ++e) {
                    xu[e] = inT ? rx[i].get(e) : 0.f;
                    float z = tp.b[e] + tp.w[CK - 1][e] * xu[e];
#pragma unroll
                    for (int k = 0; k < CK - 1; ++k) z += tp.w[k][e] * xw[k][e];
                    const float s = sigmoid(z);
                    dzu[e] = inT ? rg[i].get(e) * s * (1.f + z * (1.f - s)) : 0.f;
                    if (inS) {
#pragma unroll
                        for (int k = 0; k < CK - 1; ++k) acc[k][e] += xw[k][e] * dzu[e];
                        acc[CK - 1][e] += xu[e] * dzu[e];
                        acc[CK][e] += dzu[e];
                    }
                }
                // dx at t = u - (K-1): sum_k W_k dz_{t+(K-1-k)}
                const int64_t t = u - (CK - 1);
                if (t >= t0 && t < send) {
                    float out[CV];
#pragma unroll
                    for (int e = 0; e < CV; ++e) {
                        float v = tp.w[0][e] * dzu[e];
#pragma unroll
                        for (int k = 1; k < CK; ++k) v += tp.w[k][e] * dzw[CK - 1 - k][e];
                        out[e] = v;
                    }
                    store_row<T, CV>(dx + t * C_, out);
                }
#pragma unroll
                for (int e = 0; e < CV; ++e) {
#pragma unroll
                    for (int k = 0; k < CK - 2; ++k) {
                        xw[k][e] = xw[k + 1][e];
                        dzw[k][e] = dzw[k + 1][e];
                    }
                    xw[CK - 2][e] = xu[e];
                    dzw[CK - 2][e] = dzu[e];
                }
            }
        }
    }

    // the four strips' partial sums, added in wave order
    if (wv > 0) {
#pragma unroll
        for (int k = 0; k <= CK; ++k)
#pragma unroll
            for (int e = 0; e < CV; ++e) sred[wv - 1][k][e][lane] = acc[k][e];
    }
    __syncthreads();
    if (wv == 0 && live) {
        float* part = a.ws + ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * (CK + 1) * C_ + c0;
#pragma unroll
        for (int k = 0; k <= CK; ++k) {
            float v[CV];
#pragma unroll
            for (int e = 0; e < CV; ++e) {
                float s = acc[k][e];
#pragma unroll
                for (int w = 0; w < CW - 1; ++w) s += sred[w][k][e][lane];
                v[e] = s;
            }
            store_row<float, CV>(part + k * C_, v);
        }
    }
}

// dW[k][c] and db[c] from the per-workgroup partials, summed in a fixed order:
// a workgroup takes 64 consecutive (k, c) entries; its four waves each add a
// quarter of the partials (loads issued eight at a time), and the quarters are
// added in wave order through LDS.
constexpr int RW = 4;
__global__ __launch_bounds__(64 * RW) void k_conv_reduce(const ConvArgs a, int64_t nparts) {
    __shared__ float sq[RW - 1][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t C_ = a.C;
    const int64_t i = (int64_t)blockIdx.x * 64 + lane;
    const bool live = i < (CK + 1) * C_;
    const int64_t ii = live ? i : 0;
    const int k = (int)(ii / C_);
    const int64_t c = ii % C_;
    const int64_t q = (nparts + RW - 1) / RW;
    const int64_t p0 = wv * q, p1 = p0 + q < nparts ? p0 + q : nparts;
    float s = 0.f;
    for (int64_t p = p0; p < p1; p += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t pp = p + j < p1 ? p + j : p0;  // (an existing partial, unused)
            v[j] = a.ws[(pp * (CK + 1) + k) * C_ + c];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (p + j < p1) s += v[j];
    }
    if (wv > 0) sq[wv - 1][lane] = s;
    __syncthreads();
    if (wv == 0 && live) {
#pragma unroll
        for (int w = 0; w < RW - 1; ++w) s += sq[w][lane];
        if (k < CK) a.dw[k * C_ + c] = s;
        else if (a.db) a.db[c] = s;
    }
}

}  // namespace

int64_t conv_partials(int64_t B, int64_t T) { return B * ((T + CW * CL - 1) / (CW * CL)); }

// channels per lane and rows requested together (measured at B=8, T=4096, C=2048,
// bf16: forward 8 x 8 at 52 us against 60 with 4 rows; backward 4 x 4 at 104 us,
// within 4 % of the other three shapes, with the fewest registers)
template <typename T> struct ConvShape {
    static constexpr int FWD_CV = 8, FWD_CB = 8, BWD_CV = 4, BWD_CB = 4;
};

template <typename T>
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st) {
    constexpr int CV = ConvShape<T>::FWD_CV, CB = ConvShape<T>::FWD_CB;
    const dim3 grid((unsigned)((a.C + 64 * CV - 1) / (64 * CV)), (unsigned)((a.T + CW * CL - 1) / (CW * CL)),
                    (unsigned)a.B);
    hipLaunchKernelGGL((k_conv_fwd<T, CV, CB>), grid, dim3(CTH), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_bwd(const ConvArgs& a, hipStream_t st) {
    constexpr int CV = ConvShape<T>::BWD_CV, CB = ConvShape<T>::BWD_CB;
    if (a.T > 0) {  // (T = 0: the reduction alone writes dW = db = 0)
        const dim3 grid((unsigned)((a.C + 64 * CV - 1) / (64 * CV)),
                        (unsigned)((a.T + CW * CL - 1) / (CW * CL)), (unsigned)a.B);
        hipLaunchKernelGGL((k_conv_bwd<T, CV, CB>), grid, dim3(CTH), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n = (CK + 1) * a.C;
    hipLaunchKernelGGL(k_conv_reduce, dim3((unsigned)((n + 63) / 64)), dim3(64 * RW), 0, st, a,
                       conv_partials(a.B, a.T));
    return hipGetLastError();
}

template hipError_t launch_conv_fwd<float>(const ConvArgs&, hipStream_t);
template hipError_t launch_conv_fwd<bf16>(const ConvArgs&, hipStream_t);
template hipError_t launch_conv_bwd<float>(const ConvArgs&, hipStream_t);
template hipError_t launch_conv_bwd<bf16>(const ConvArgs&, hipStream_t);

}  // namespace gla
