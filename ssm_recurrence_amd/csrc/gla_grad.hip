// gla_grad.hip -- per-chunk input gradients of the gated linear-attention
// recurrence (gfx950), and the sum over heads that share a q/k head.
//
// One workgroup (4 waves) owns one chunk of one (b, h).  It reads the state
// entering the chunk S0, the state at its end S1 and the gradient at its end
// dS1 (written by the sequential passes) and computes, with beta the
// chunk-local log-gate prefix, Gamma its total, E = exp(beta - m) around
// m = beta_31 (vector gate), dA = dO V^T masked to s <= r in one document
// (times exp(beta_r - beta_s) for the scalar gate):
//
//   dv[s] = sum_{r>=s} A[r][s] dO[r] + [s in last doc] dS1^T (k[s] exp(Gamma - beta_s))
//   dq[r] = sum_s dA[r][s] k[s] exp(beta_r - beta_s) + [r in first doc] exp(beta_r) (S0 dO[r])
//   dk[s] = sum_r dA[r][s] q[r] exp(beta_r - beta_s) + [s in last doc] exp(Gamma - beta_s) (dS1 v[s])
//   dg[u] = sum_{t>=u, same doc} (q (.) dq - k (.) dk)[t] + [u in last doc] rowsum(S1 (.) dS1)
//           (0 at reset tokens; summed over channels for the scalar gate)
//
// These are the chunkwise input gradients and the log-gate gradient of the
// FLAT page ("FLAT: Flash Linear Attention on TPUs", Linear Attention >
// Backward Recurrence and Pallas Kernels > Backward Kernels: grad K and grad V
// use the state gradient from later chunks; the gate gradient is the adjoint
// of the chunk-local prefix sum, a suffix sum of q*dq - k*dk plus the boundary
// term from the carried state).  The suffix sum and its inputs stay in fp32.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

template <typename T> struct PitchG {
    static constexpr int pad = 16 / (int)sizeof(T);
    static constexpr int of(int d) { return d + pad; }
};

template <typename T, int N>
__device__ __forceinline__ void vcopy(const T* src, T* dst) {
    typedef __attribute__((__vector_size__(16))) int i32x4;
#pragma unroll
    for (int i = 0; i < (int)(N * sizeof(T) / 16); ++i)
        reinterpret_cast<i32x4*>(dst)[i] = reinterpret_cast<const i32x4*>(src)[i];
}

template <typename T, int D, int P>
__device__ __forceinline__ void g_stage_rows(T* dst, const T* src, int64_t rs, int nvalid) {
    constexpr int VE = 16 / sizeof(T);
    constexpr int VPR = D / VE;
    for (int idx = threadIdx.x; idx < C * VPR; idx += NT) {
        const int r = idx / VPR, cv = (idx % VPR) * VE;
        T buf[VE];
        if (r < nvalid) {
            vcopy<T, VE>(src + (int64_t)r * rs + cv, buf);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) buf[e] = from_f32<T>(0.f);
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) dst[r * P + cv + e] = buf[e];
    }
}

// fp32 global rows -> operand fragment: X(i, k) = base[i*ld + k]
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag glb_rows(const float* base, int ld, int i0, int k0) {
    const int l = lane_id();
    const float* p = base + (int64_t)(i0 + (l & 15)) * ld + k0 + (l >> 4) * Mma<T>::KPL;
    typename Mma<T>::frag f;
    if constexpr (Mma<T>::KPL == 1) {
        f = *p;
    } else {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
        for (int e = 0; e < 4; ++e) { f[e] = (bf16)x0[e]; f[4 + e] = (bf16)x1[e]; }
    }
    return f;
}
// fp32 global columns -> operand fragment: X(i, k) = base[k*ld + i]
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag glb_cols(const float* base, int ld, int i0, int k0) {
    const int l = lane_id();
    const float* p = base + (int64_t)(k0 + (l >> 4) * Mma<T>::KPL) * ld + i0 + (l & 15);
    typename Mma<T>::frag f;
    if constexpr (Mma<T>::KPL == 1) {
        f = *p;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)p[(int64_t)e * ld];
    }
    return f;
}
// rows of a T tensor in global memory (row i at base + i*rs), zero past nvalid
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag glb_rows_t(const T* base, int64_t rs, int i0, int k0,
                                                            int nvalid) {
    const int l = lane_id();
    const int i = i0 + (l & 15);
    typename Mma<T>::frag f = Mma<T>::zero();
    if (i < nvalid) {
        const T* p = base + (int64_t)i * rs + k0 + (l >> 4) * Mma<T>::KPL;
        if constexpr (Mma<T>::KPL == 1) f = *p;
        else f = *reinterpret_cast<const bf16x8*>(p);
    }
    return f;
}

template <typename T, bool VEC, int DK, int DV>
struct GradCfg {
    static constexpr int PK = PitchG<T>::of(DK);
    static constexpr int PV = PitchG<T>::of(DV);
    static constexpr int PS = PitchG<T>::of(C);
    static constexpr int QK_BYTES = 2 * C * PK * (int)sizeof(T);
    static constexpr int X_BYTES = C * (DK + 1) * 4;
    static constexpr int QK_REGION = QK_BYTES > X_BYTES ? QK_BYTES : X_BYTES;
    static constexpr int BASE = QK_REGION + C * PV * (int)sizeof(T) + C * PS * (int)sizeof(T) +
                                (VEC ? C * DK * 4 : 0) + 4096;
    static constexpr bool V_LDS = BASE + C * PV * (int)sizeof(T) <= 160 * 1024;
};

template <typename T, bool VEC, int DK, int DV>
__global__ __launch_bounds__(NT) void k_grad(const GradArgs a) {
    using Cfg = GradCfg<T, VEC, DK, DV>;
    constexpr int PK = Cfg::PK, PV = Cfg::PV, PS = Cfg::PS;
    constexpr bool V_LDS = Cfg::V_LDS;
    constexpr int NCT = DK / 16, NNT = DV / 16;
    using M = Mma<T>;

    __shared__ __attribute__((aligned(16))) char sQKraw[Cfg::QK_REGION];
    __shared__ __attribute__((aligned(16))) T sV[V_LDS ? C * PV : 1];
    __shared__ __attribute__((aligned(16))) T sdO[C * PV];
    __shared__ __attribute__((aligned(16))) T sdA[C * PS];
    __shared__ __attribute__((aligned(16))) float sE[VEC ? C * DK : 1];
    __shared__ ChunkDocs cd;
    __shared__ float sBeta[C], sEq[C], sEk[C];
    __shared__ float sEm[VEC ? DK : 1], sEGm[VEC ? DK : 1];
    __shared__ float sPart[(NT / DK) * DK];
    __shared__ float sBnd[DK];
    T* sQ = reinterpret_cast<T*>(sQKraw);
    T* sK = sQ + C * PK;
    float* sX = reinterpret_cast<float*>(sQKraw);  // [C][DK+1], after the products

    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t ci = blockIdx.x % NC;
    const int64_t bh = blockIdx.x / NC;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int64_t t0 = ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;

    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.g;
    const T* dO = (const T*)a.dO;
    const int64_t rs_qk = a.Hqk * DK, rs_v = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qrow = q + (b * T_ + t0) * rs_qk + hq * DK;
    const T* krow = k + (b * T_ + t0) * rs_qk + hq * DK;
    const T* vrow = v + (b * T_ + t0) * rs_v + h * DV;
    const T* dorow = dO + (b * T_ + t0) * rs_v + h * DV;
    const float* S0 = a.ws_S + (bh * (NC + 1) + ci) * DK * DV;
    const float* S1 = S0 + DK * DV;
    const float* dS1 = a.ws_dS + (bh * NC + ci) * DK * DV;

    // ---- stage
    g_stage_rows<T, DK, PK>(sQ, qrow, rs_qk, nvalid);
    g_stage_rows<T, DK, PK>(sK, krow, rs_qk, nvalid);
    if constexpr (V_LDS) g_stage_rows<T, DV, PV>(sV, vrow, rs_v, nvalid);
    g_stage_rows<T, DV, PV>(sdO, dorow, rs_v, nvalid);
    chunk_docs(&cd, a.seg, b, T_, t0);
    if (!VEC && w == 0) {
        const int r = l;
        const float gr = r < nvalid ? to_f32(g[(b * T_ + t0 + r) * rs_g + h]) : 0.f;
        const float beta = wave_incl_scan(gr);
        const float Gam = __shfl(beta, 63, 64);
        sBeta[r] = beta;
        sEq[r] = __expf(beta);
        sEk[r] = __expf(Gam - beta);
    }
    // boundary term rowsum(S1 * dS1) (partial sums over column ranges)
    {
        constexpr int TPR = NT / DK, NPT = DV / TPR;
        const int c = threadIdx.x % DK, pr = threadIdx.x / DK;
        float acc = 0.f;
        for (int n = pr * NPT; n < (pr + 1) * NPT; ++n) acc += S1[c * DV + n] * dS1[c * DV + n];
        sPart[pr * DK + c] = acc;
    }
    __syncthreads();
    const int first_reset = cd.first_reset, last_reset = cd.last_reset;
    if (threadIdx.x < DK) {
        float s = 0.f;
        for (int p = 0; p < NT / DK; ++p) s += sPart[p * DK + threadIdx.x];
        sBnd[threadIdx.x] = s;
    }
    __syncthreads();

    if constexpr (VEC) {
        constexpr int TPC = NT / DK, RPT = C / TPC;
        const int c = threadIdx.x % DK, qd = threadIdx.x / DK;
        const T* gcol = g + (b * T_ + t0) * rs_g + h * DK + c;
        float part = 0.f;
        for (int r = qd * RPT; r < (qd + 1) * RPT; ++r)
            if (r < nvalid) part += to_f32(gcol[r * rs_g]);
        sPart[qd * DK + c] = part;
        __syncthreads();
        float pre = 0.f, m = 0.f, Gam = 0.f;
#pragma unroll
        for (int p = 0; p < TPC; ++p) {
            const float x = sPart[p * DK + c];
            if (p < qd) pre += x;
            if (p < TPC / 2) m += x;
            Gam += x;
        }
        if (qd == 0) {
            sEm[c] = __expf(m);
            sEGm[c] = __expf(Gam - m);
        }
        float run = pre;
        for (int r = qd * RPT; r < (qd + 1) * RPT; ++r) {
            if (r < nvalid) run += to_f32(gcol[r * rs_g]);
            const float E = __expf(run - m);
            sE[r * DK + c] = E;
            sQ[r * PK + c] = from_f32<T>(to_f32(sQ[r * PK + c]) * E);
            sK[r * PK + c] = from_f32<T>(to_f32(sK[r * PK + c]) / E);
        }
    }
    __syncthreads();

    // ---- A and dA on all rows, this wave's 16 columns s in [16w, 16w+16)
    f32x4 A[4], dA[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        A[rt] = zero4();
        dA[rt] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += M::KSTEP)
            A[rt] = M::mma(frag_ld<T, PK, 1>(sQ, 16 * rt, k0), frag_ld<T, PK, 1>(sK, 16 * w, k0), A[rt]);
#pragma unroll
        for (int n0 = 0; n0 < DV; n0 += M::KSTEP) {
            typename M::frag vb;
            if constexpr (V_LDS) vb = frag_ld<T, PV, 1>(sV, 16 * w, n0);
            else vb = glb_rows_t<T>(vrow, rs_v, 16 * w, n0, nvalid);
            dA[rt] = M::mma(frag_ld<T, PV, 1>(sdO, 16 * rt, n0), vb, dA[rt]);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * j4 + e, s = 16 * w + i16;
            const bool keep = s <= r && cd.doc[s] == cd.doc[r];
            const float d = VEC ? 1.f : __expf(sBeta[r] - sBeta[s]);
            A[rt][e] = keep ? A[rt][e] * d : 0.f;
            dA[rt][e] = keep ? dA[rt][e] * d : 0.f;
            sdA[r * PS + s] = from_f32<T>(dA[rt][e]);
        }
    __syncthreads();

    const int s_row0 = 16 * w;  // this wave's rows for dv, dq, dk

    // ---- dv[s][n] for s in this wave's tile
    {
        T* dvo = (T*)a.dv;
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
            f32x4 acc = zero4();
            if constexpr (M::KPL == 1) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub)
                        acc = M::mma(frag_from_acc<T>(A[rt], A[rt], sub),
                                     frag_ld_ctile<T, 1, PV>(sdO, 16 * nt, 16 * rt, sub), acc);
            } else {
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    acc = M::mma(frag_from_acc<T>(A[2 * p], A[2 * p + 1], 0),
                                 frag_ld_ctile<T, 1, PV>(sdO, 16 * nt, 32 * p, 0), acc);
            }
            // + KU dS1, KU[s][c] = k[s][c] exp(Gamma - beta_s[c]) for s in the last document
            const int s = s_row0 + i16;
            const float ms = s >= last_reset ? 1.f : 0.f;
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += M::KSTEP) {
                typename M::frag ku = frag_ld<T, PK, 1>(sK, s_row0, k0);
#pragma unroll
                for (int e = 0; e < M::KPL; ++e) {
                    const int c = k0 + j4 * M::KPL + e;
                    float x;
                    if constexpr (M::KPL == 1) x = to_f32(ku); else x = to_f32(ku[e]);
                    const float f = VEC ? sEGm[c] * ms : sEk[s] * ms;
                    M::set(ku, e, x * f);
                }
                acc = M::mma(ku, glb_cols<T>(dS1, DV, 16 * nt, k0), acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sr = s_row0 + 4 * j4 + e;
                if (sr < nvalid)
                    dvo[((b * T_ + t0 + sr) * a.H + h) * DV + 16 * nt + i16] = from_f32<T>(acc[e]);
            }
        }
    }

    // ---- dq and dk on this wave's rows, all channels
    f32x4 dq[NCT], dk[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += M::KSTEP)
            a1 = M::mma(frag_ld<T, PS, 1>(sdA, s_row0, k0), frag_ld<T, 1, PK>(sK, 16 * ct, k0), a1);
#pragma unroll
        for (int n0 = 0; n0 < DV; n0 += M::KSTEP)
            a2 = M::mma(frag_ld<T, PV, 1>(sdO, s_row0, n0), glb_rows<T>(S0, DV, 16 * ct, n0), a2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = s_row0 + 4 * j4 + e, c = 16 * ct + i16;
            const float first = r < first_reset ? 1.f : 0.f;
            if constexpr (VEC) {
                const float E = sE[r * DK + c];
                dq[ct][e] = E * a1[e] + first * E * sEm[c] * a2[e];
            } else {
                dq[ct][e] = a1[e] + first * sEq[r] * a2[e];
            }
        }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        f32x4 a1 = zero4(), a2 = zero4();
        if constexpr (M::KPL == 1) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
                    a1 = M::mma(frag_from_acc<T>(dA[rt], dA[rt], sub),
                                frag_ld_ctile<T, 1, PK>(sQ, 16 * ct, 16 * rt, sub), a1);
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p)
                a1 = M::mma(frag_from_acc<T>(dA[2 * p], dA[2 * p + 1], 0),
                            frag_ld_ctile<T, 1, PK>(sQ, 16 * ct, 32 * p, 0), a1);
        }
#pragma unroll
        for (int n0 = 0; n0 < DV; n0 += M::KSTEP) {
            typename M::frag va;
            if constexpr (V_LDS) va = frag_ld<T, PV, 1>(sV, s_row0, n0);
            else va = glb_rows_t<T>(vrow, rs_v, s_row0, n0, nvalid);
            a2 = M::mma(va, glb_rows<T>(dS1, DV, 16 * ct, n0), a2);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = s_row0 + 4 * j4 + e, c = 16 * ct + i16;
            const float last = s >= last_reset ? 1.f : 0.f;
            if constexpr (VEC) {
                const float Ei = 1.0f / sE[s * DK + c];
                dk[ct][e] = Ei * a1[e] + last * sEGm[c] * Ei * a2[e];
            } else {
                dk[ct][e] = a1[e] + last * sEk[s] * a2[e];
            }
        }
    }

    // ---- write dq, dk (per head in fp32 when heads share q/k)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = s_row0 + 4 * j4 + e, c = 16 * ct + i16;
            if (r >= nvalid) continue;
            if (G == 1) {
                const int64_t o = ((b * T_ + t0 + r) * a.Hqk + hq) * DK + c;
                ((T*)a.dq)[o] = from_f32<T>(dq[ct][e]);
                ((T*)a.dk)[o] = from_f32<T>(dk[ct][e]);
            } else {
                const int64_t o = ((b * T_ + t0 + r) * a.H + h) * DK + c;
                a.ws_dq[o] = dq[ct][e];
                a.ws_dk[o] = dk[ct][e];
            }
        }

    // ---- gate gradient: x = q*dq - k*dk (per head, fp32), suffix sum within documents
    __syncthreads();  // everyone done with sQ / sK
    constexpr int PX = DK + 1;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = s_row0 + 4 * j4 + e, c = 16 * ct + i16;
            float x = 0.f;
            if (r < nvalid) {
                const float qv = to_f32(qrow[(int64_t)r * rs_qk + c]);
                const float kv = to_f32(krow[(int64_t)r * rs_qk + c]);
                x = qv * dq[ct][e] - kv * dk[ct][e];
            }
            sX[r * PX + c] = x;
        }
    __syncthreads();
    T* dgo = (T*)a.dg;
    if constexpr (VEC) {
        if (threadIdx.x < DK) {
            const int c = threadIdx.x;
            float run = sBnd[c];
            for (int r = nvalid - 1; r >= 0; --r) {
                if (r < nvalid - 1 && cd.doc[r + 1] != cd.doc[r]) run = 0.f;
                run += sX[r * PX + c];
                const bool reset = r > 0 ? cd.doc[r] != cd.doc[r - 1] : cd.doc[0] != 0;
                dgo[((b * T_ + t0 + r) * a.H + h) * DK + c] = from_f32<T>(reset ? 0.f : run);
            }
        }
    } else {
        if (w == 0) {
            const int r = l;
            float xs = 0.f;
            for (int c = 0; c < DK; ++c) xs += sX[r * PX + c];
            float bnd = 0.f;
            for (int c = l; c < DK; c += 64) bnd += sBnd[c];
            for (int d = 32; d >= 1; d >>= 1) bnd += __shfl_xor(bnd, d, 64);
            sPart[r] = xs;
            // one wave: its LDS accesses complete in order; keep the compiler from
            // moving the reads above the writes
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (l == 0) {
                float run = bnd;
                for (int rr = nvalid - 1; rr >= 0; --rr) {
                    if (rr < nvalid - 1 && cd.doc[rr + 1] != cd.doc[rr]) run = 0.f;
                    run += sPart[rr];
                    const bool reset = rr > 0 ? cd.doc[rr] != cd.doc[rr - 1] : cd.doc[0] != 0;
                    dgo[(b * T_ + t0 + rr) * a.H + h] = from_f32<T>(reset ? 0.f : run);
                }
            }
        }
    }
}

template <typename T, bool VEC, int DK, int DV>
hipError_t launch_grad(const GradArgs& a, hipStream_t st) {
    const int64_t NC = (a.T + C - 1) / C;
    const int64_t grid = a.B * a.H * NC;
    hipLaunchKernelGGL((k_grad<T, VEC, DK, DV>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    return hipGetLastError();
}

// dq[b,t,hq,:] = sum over the G heads h of group hq of src[b,t,h,:]
template <typename T, int DK>
__global__ __launch_bounds__(NT) void k_group_sum(const float* src, T* dst, int64_t rows,
                                                   int64_t H, int64_t Hqk) {
    const int64_t G = H / Hqk;
    const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;  // over rows * Hqk * DK
    const int64_t total = rows * Hqk * DK;
    if (idx >= total) return;
    const int64_t c = idx % DK;
    const int64_t hq = (idx / DK) % Hqk;
    const int64_t bt = idx / (DK * Hqk);
    float s = 0.f;
    for (int64_t h = hq * G; h < (hq + 1) * G; ++h) s += src[(bt * H + h) * DK + c];
    dst[idx] = from_f32<T>(s);
}

template <typename T, int DK>
hipError_t launch_group_sum(const float* src, void* dst, int64_t B, int64_t Tn, int64_t H,
                            int64_t Hqk, hipStream_t st) {
    const int64_t total = B * Tn * Hqk * DK;
    if (total == 0) return hipSuccess;
    const int64_t grid = (total + NT - 1) / NT;
    hipLaunchKernelGGL((k_group_sum<T, DK>), dim3((unsigned)grid), dim3(NT), 0, st, src, (T*)dst,
                       B * Tn, H, Hqk);
    return hipGetLastError();
}

#define GLA_INST_GRAD(T, VEC, DK, DV) \
    template hipError_t launch_grad<T, VEC, DK, DV>(const GradArgs&, hipStream_t);
#define GLA_INST_GRAD_D(T, VEC) \
    GLA_INST_GRAD(T, VEC, 64, 64) GLA_INST_GRAD(T, VEC, 64, 128) \
    GLA_INST_GRAD(T, VEC, 128, 64) GLA_INST_GRAD(T, VEC, 128, 128)
GLA_INST_GRAD_D(float, false)
GLA_INST_GRAD_D(float, true)
GLA_INST_GRAD_D(bf16, false)
GLA_INST_GRAD_D(bf16, true)
template hipError_t launch_group_sum<float, 64>(const float*, void*, int64_t, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_group_sum<float, 128>(const float*, void*, int64_t, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_group_sum<bf16, 64>(const float*, void*, int64_t, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_group_sum<bf16, 128>(const float*, void*, int64_t, int64_t, int64_t, int64_t, hipStream_t);

}  // namespace gla
