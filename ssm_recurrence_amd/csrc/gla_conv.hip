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
// Work split: a lane owns 8 consecutive channels (one 16-byte bf16 row piece),
// so a wave reads 512 channels of a time step as one contiguous 1 KB request;
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
constexpr int CV = 8;         // channels per lane
constexpr int CL = 64;        // time steps per wave
constexpr int CW = 4;         // waves per workgroup (consecutive strips)
constexpr int CTH = 64 * CW;  // threads per workgroup
constexpr int CB = 8;         // rows requested together

// eight consecutive channels of one time step, as stored
template <typename T> struct Row8;
template <> struct Row8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};
template <> struct Row8<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void load(const float* p) {
        lo = *reinterpret_cast<const f32x4*>(p);
        hi = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? lo[e] : hi[e - 4]; }
};

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[CV]) {
    if constexpr (sizeof(T) == 2) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < CV; ++e) o[e] = (bf16)v[e];
        *reinterpret_cast<bf16x8*>(p) = o;
    } else {
        *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

struct Taps {
    float w[CK][CV], b[CV];
    __device__ __forceinline__ void load(const ConvArgs& a, int64_t c0) {
#pragma unroll
        for (int k = 0; k < CK; ++k) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(a.w + k * a.C + c0);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(a.w + k * a.C + c0 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w[k][e] = lo[e];
                w[k][e + 4] = hi[e];
            }
        }
#pragma unroll
        for (int e = 0; e < CV; ++e) b[e] = 0.f;
        if (a.bias) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(a.bias + c0);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(a.bias + c0 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                b[e] = lo[e];
                b[e + 4] = hi[e];
            }
        }
    }
};

// Forward: y_t = SiLU(b + sum_k W_k x_{t-(K-1-k)}) for the lane's 8 channels and
// the wave's strip of time steps.
template <typename T>
__global__ __launch_bounds__(CTH) void k_conv_fwd(const ConvArgs a) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * CV;
    const int64_t t0 = ((int64_t)blockIdx.y * CW + wv) * CL;
    const int64_t T_ = a.T, C_ = a.C;
    if (c0 >= C_ || t0 >= T_) return;  // no barriers in this kernel
    const T* x = (const T*)a.x + (int64_t)blockIdx.z * T_ * C_ + c0;
    T* y = (T*)a.y + (int64_t)blockIdx.z * T_ * C_ + c0;
    Taps tp;
    tp.load(a, c0);

    // the K-1 inputs before the strip (zero before t = 0)
    float win[CK - 1][CV];
#pragma unroll
    for (int j = 0; j < CK - 1; ++j) {
        const int64_t t = t0 - (CK - 1) + j;
        Row8<T> r;
        r.load(x + (t >= 0 ? t : 0) * C_);
#pragma unroll
        for (int e = 0; e < CV; ++e) win[j][e] = t >= 0 ? r.get(e) : 0.f;
    }
    const int64_t tend = t0 + CL < T_ ? t0 + CL : T_;
    for (int64_t tb = t0; tb < tend; tb += CB) {
        // CB rows requested together (a row past the end reads the last row, unused)
        Row8<T> r[CB];
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
            if (tb + i < tend) store8<T>(y + (tb + i) * C_, out);
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
template <typename T>
__global__ __launch_bounds__(CTH) void k_conv_bwd(const ConvArgs a) {
    __shared__ float sred[CW - 1][CK + 1][CV][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * CV;
    const int64_t t0 = ((int64_t)blockIdx.y * CW + wv) * CL;
    const int64_t T_ = a.T, C_ = a.C;
    const bool live = c0 < C_;  // (every wave reaches the barrier below)
    const int64_t cc = live ? c0 : 0;
    const T* x = (const T*)a.x + (int64_t)blockIdx.z * T_ * C_ + cc;
    const T* dy = (const T*)a.dy + (int64_t)blockIdx.z * T_ * C_ + cc;
    T* dx = (T*)a.dx + (int64_t)blockIdx.z * T_ * C_ + cc;
    Taps tp;
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
            Row8<T> r;
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
            Row8<T> rx[CB], rg[CB];
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
                    store8<T>(dx + t * C_, out);
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
            *reinterpret_cast<f32x4*>(part + k * C_) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(part + k * C_ + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
    }
}

// dW[k][c] and db[c] from the per-workgroup partials, summed in a fixed order
__global__ __launch_bounds__(256) void k_conv_reduce(const ConvArgs a, int64_t nparts) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t C_ = a.C;
    if (i >= (CK + 1) * C_) return;
    const int k = (int)(i / C_);
    const int64_t c = i % C_;
    float s = 0.f;
    for (int64_t p = 0; p < nparts; ++p) s += a.ws[(p * (CK + 1) + k) * C_ + c];
    if (k < CK) a.dw[k * C_ + c] = s;
    else if (a.db) a.db[c] = s;
}

}  // namespace

int64_t conv_partials(int64_t B, int64_t T) { return B * ((T + CW * CL - 1) / (CW * CL)); }

template <typename T>
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.C + 64 * CV - 1) / (64 * CV)), (unsigned)((a.T + CW * CL - 1) / (CW * CL)),
                    (unsigned)a.B);
    hipLaunchKernelGGL(k_conv_fwd<T>, grid, dim3(CTH), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_bwd(const ConvArgs& a, hipStream_t st) {
    if (a.T > 0) {  // (T = 0: the reduction alone writes dW = db = 0)
        const dim3 grid((unsigned)((a.C + 64 * CV - 1) / (64 * CV)),
                        (unsigned)((a.T + CW * CL - 1) / (CW * CL)), (unsigned)a.B);
        hipLaunchKernelGGL(k_conv_bwd<T>, grid, dim3(CTH), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n = (CK + 1) * a.C;
    hipLaunchKernelGGL(k_conv_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a,
                       conv_partials(a.B, a.T));
    return hipGetLastError();
}

template hipError_t launch_conv_fwd<float>(const ConvArgs&, hipStream_t);
template hipError_t launch_conv_fwd<bf16>(const ConvArgs&, hipStream_t);
template hipError_t launch_conv_bwd<float>(const ConvArgs&, hipStream_t);
template hipError_t launch_conv_bwd<bf16>(const ConvArgs&, hipStream_t);

}  // namespace gla
