// gla_pass.hip -- sequential chunk passes that keep the state tile resident
// in matrix-core accumulators for the whole sequence (gfx950).
//
// One workgroup (4 waves) owns one (batch row b, head h, 64-column slice of
// d_v).  Columns of the state evolve independently, so slices need no
// exchange.  Wave w owns state columns [16w, 16w+16) of the slice; the state
// S[c][n] lives in registers as d_k/16 C-layout tiles and never goes to HBM
// between chunks (FLAT page, "FLAT: Flash Linear Attention on TPUs", Pallas
// Kernels > Forward Kernels: the fused block-recurrent kernel keeps the state
// on chip and does state passing and readout in one program).
//
// Per chunk of C = 64 tokens with chunk-local inclusive log-gate prefix
// beta_r and total Gamma = beta_{C-1} (the chunkwise form on the same page,
// Linear Attention > Forward Recurrence, with the gate ratios written as
// exponentiated chunk-local prefix sums of log f, Pallas Kernels > Mamba-2):
//
//   A[r][s]  = sum_c q[r][c] k[s][c] exp(beta_r[c] - beta_s[c])  for s <= r, same document
//   o[r]     = sum_s A[r][s] v[s] + [r in first doc] (q[r] * exp(beta_r))^T S
//   S        = [no reset in chunk] diag(exp Gamma) S + sum_{s in last doc} (k[s] * exp(Gamma - beta_s)) v[s]^T
//
// The vector gate factors the intra term around m = beta_31 (mid chunk):
// QA = q exp(beta - m), KA = k exp(m - beta), A = QA KA^T.  The scalar gate
// multiplies QK^T by exp(beta_r - beta_s) directly.
//
// Modes:
//   MODE_OUT    forward: o, and hT at the end.
//   MODE_STATES state pass for the backward: writes the state entering every
//               chunk, and the final state, to ws (no readout).
//   MODE_DSTATE reverse state-gradient pass: dS (gradient of the state at a
//               chunk's end) walks chunks last to first, dS <- [no reset]
//               diag(exp Gamma) dS + sum_{r in first doc} (q[r] exp(beta_r)) dO[r]^T,
//               writes dS at every chunk end to ws and dh0 at the start
//               (FLAT page, Linear Attention > Backward Recurrence: the state
//               gradient is a linear attention run in reverse with q and dO in
//               the roles of k and v).
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

template <typename T> struct Pitch {
    // row pitch (elements) for [rows][D] tiles in LDS: 16-byte aligned rows,
    // shifted by 16 bytes per row
    static constexpr int pad = 16 / (int)sizeof(T);
    static constexpr int of(int d) { return d + pad; }
};

template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* src, T* dst) {
    // N elements, 16-byte aligned
    static_assert((N * sizeof(T)) % 16 == 0, "");
    typedef __attribute__((__vector_size__(16))) int i32x4;
    const i32x4* s = reinterpret_cast<const i32x4*>(src);
    i32x4* d = reinterpret_cast<i32x4*>(dst);
#pragma unroll
    for (int i = 0; i < (int)(N * sizeof(T) / 16); ++i) d[i] = s[i];
}

// Stage a [C][D] row tile (rows t0.., row stride `rs` elements) into LDS with
// pitch P; rows >= nvalid are zero.
template <typename T, int D, int P>
__device__ __forceinline__ void stage_rows(T* dst, const T* src, int64_t rs, int nvalid) {
    constexpr int VE = 16 / sizeof(T);
    constexpr int VPR = D / VE;  // vectors per row
    for (int idx = threadIdx.x; idx < C * VPR; idx += NT) {
        const int r = idx / VPR, cv = (idx % VPR) * VE;
        T buf[VE];
        if (r < nvalid) {
            load_vec<T, VE>(src + (int64_t)r * rs + cv, buf);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) buf[e] = from_f32<T>(0.f);
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) dst[r * P + cv + e] = buf[e];
    }
}

// Stage the transpose of a [C][W] row tile: dst[n][r] = src[r][n] (pitch P).
template <typename T, int W, int P>
__device__ __forceinline__ void stage_cols(T* dst, const T* src, int64_t rs, int nvalid) {
    constexpr int VE = 16 / sizeof(T);
    constexpr int VPR = W / VE;
    for (int idx = threadIdx.x; idx < C * VPR; idx += NT) {
        const int r = idx % C, cv = (idx / C) * VE;
        T buf[VE];
        if (r < nvalid) {
            load_vec<T, VE>(src + (int64_t)r * rs + cv, buf);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) buf[e] = from_f32<T>(0.f);
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) dst[(cv + e) * P + r] = buf[e];
    }
}

template <typename T, bool VEC, int DK, int DV, int MODE>
__global__ __launch_bounds__(NT) void k_pass(const PassArgs a) {
    constexpr int NV = 64;             // state columns per workgroup
    constexpr int NVS = DV / NV;       // slices per head
    constexpr int PK = Pitch<T>::of(DK);
    constexpr int PS = Pitch<T>::of(C);
    constexpr int NCT = DK / 16;       // state row tiles
    using M = Mma<T>;
    constexpr bool OUT = MODE == MODE_OUT;
    constexpr bool REV = MODE == MODE_DSTATE;

    // LDS: sX = q (OUT) / k (STATES) / q (DSTATE) operands; see per-mode use.
    __shared__ __attribute__((aligned(16))) T sQ[C * PK];    // OUT: QA (or raw q)
    __shared__ __attribute__((aligned(16))) T sK[C * PK];    // OUT: KA (or raw k); later A
    __shared__ __attribute__((aligned(16))) T sU[C * PK];    // update operand: KU (fwd) / QR (rev)
    __shared__ __attribute__((aligned(16))) T sR[OUT && VEC ? C * PK : 1];  // OUT+VEC: QR
    __shared__ __attribute__((aligned(16))) T sVt[NV * PS];  // v^T (fwd) / dO^T (rev) slice
    __shared__ ChunkDocs cd;
    __shared__ float sBeta[C], sEq[C], sEk[C];
    __shared__ float sDecay[VEC ? DK : 1];
    __shared__ float sPart[VEC ? (NT / DK) * DK : 1];

    const int64_t bh = blockIdx.x / NVS;
    const int vs = blockIdx.x % NVS;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int nv0 = vs * NV;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;

    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.g;
    const T* dO = (const T*)a.dO;
    const int64_t rs_qk = a.Hqk * DK, rs_v = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;

    // ---- initial state (C layout: S[ct][e] = state[16ct + 4*j4 + e][nv0 + 16w + i16])
    f32x4 S[NCT];
    {
        const float* init = REV ? a.dhT : a.h0;
        const int n = nv0 + 16 * w + i16;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * ct + 4 * j4 + e;
                S[ct][e] = init ? init[(bh * DK + c) * DV + n] : 0.f;
            }
    }

    for (int64_t it = 0; it < NC; ++it) {
        const int64_t ci = REV ? NC - 1 - it : it;
        const int64_t t0 = ci * C;
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;

        // ---- stage inputs
        const T* qrow = q + (b * T_ + t0) * rs_qk + hq * DK;
        const T* krow = k + (b * T_ + t0) * rs_qk + hq * DK;
        if (OUT || REV) stage_rows<T, DK, PK>(sQ, qrow, rs_qk, nvalid);
        if (!REV) stage_rows<T, DK, PK>(sK, krow, rs_qk, nvalid);
        if (REV) {
            stage_cols<T, NV, PS>(sVt, dO + (b * T_ + t0) * rs_v + h * DV + nv0, rs_v, nvalid);
        } else {
            stage_cols<T, NV, PS>(sVt, v + (b * T_ + t0) * rs_v + h * DV + nv0, rs_v, nvalid);
        }
        chunk_docs(&cd, a.seg, b, T_, t0);
        if (!VEC && w == 0) {
            // scalar gate: wave scan of the chunk's log gates
            const int r = l;
            const float gr = r < nvalid ? to_f32(g[(b * T_ + t0 + r) * rs_g + h]) : 0.f;
            const float beta = wave_incl_scan(gr);
            const float Gam = __shfl(beta, 63, 64);
            sBeta[r] = beta;
            // readout rows: first document only; update rows: last document only
            // (the docs are written by wave 0 above, read back after the barrier)
            sEq[r] = __expf(beta);
            sEk[r] = __expf(Gam - beta);
            if (r == 0) sDecay[0] = __expf(Gam);
        }
        __syncthreads();
        const int first_reset = cd.first_reset, last_reset = cd.last_reset;
        const bool any_reset = last_reset >= 0;

        if constexpr (VEC) {
            // per-column scan: TPC threads per column, RPT rows each
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
            if (qd == 0) sDecay[c] = any_reset ? 0.f : __expf(Gam);
            const float eGm = __expf(Gam - m), em = __expf(m);
            float run = pre;
            for (int r = qd * RPT; r < (qd + 1) * RPT; ++r) {
                if (r < nvalid) run += to_f32(gcol[r * rs_g]);
                const float E = __expf(run - m);  // exp(beta - m)
                const float Ei = 1.0f / E;        // exp(m - beta)
                if constexpr (OUT) {
                    const float qv = to_f32(sQ[r * PK + c]);
                    const float kv = to_f32(sK[r * PK + c]);
                    sQ[r * PK + c] = from_f32<T>(qv * E);
                    sK[r * PK + c] = from_f32<T>(kv * Ei);
                    sR[r * PK + c] = from_f32<T>(r < first_reset ? qv * E * em : 0.f);
                    sU[r * PK + c] = from_f32<T>(r >= last_reset ? kv * Ei * eGm : 0.f);
                } else if constexpr (REV) {
                    const float qv = to_f32(sQ[r * PK + c]);
                    sU[r * PK + c] = from_f32<T>(r < first_reset ? qv * E * em : 0.f);
                } else {
                    const float kv = to_f32(sK[r * PK + c]);
                    sU[r * PK + c] = from_f32<T>(r >= last_reset ? kv * Ei * eGm : 0.f);
                }
            }
        } else {
            // scalar gate: row factors
            for (int idx = threadIdx.x; idx < C * DK; idx += NT) {
                const int r = idx / DK, c = idx % DK;
                if constexpr (REV) {
                    const float f = r < first_reset ? sEq[r] : 0.f;
                    sU[r * PK + c] = from_f32<T>(to_f32(sQ[r * PK + c]) * f);
                } else {
                    const float f = r >= last_reset ? sEk[r] : 0.f;
                    sU[r * PK + c] = from_f32<T>(to_f32(sK[r * PK + c]) * f);
                }
            }
            if (threadIdx.x == 0 && any_reset) sDecay[0] = 0.f;
        }
        __syncthreads();

        if constexpr (OUT) {
            // ---- intra: A = QA KA^T on rows [16w, 16w+16), all 64 columns
            f32x4 A[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                A[st] = zero4();
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += M::KSTEP)
                    A[st] = M::mma(frag_ld<T, PK, 1>(sQ, 16 * w, k0),
                                   frag_ld<T, PK, 1>(sK, 16 * st, k0), A[st]);
            }
            // mask (causal, same document) and the scalar gate's decay
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * w + 4 * j4 + e, s = 16 * st + i16;
                    const bool keep = s <= r && cd.doc[s] == cd.doc[r];
                    float x = A[st][e];
                    if (!VEC) x *= __expf(sBeta[r] - sBeta[s]);
                    A[st][e] = keep ? x : 0.f;
                }
            __syncthreads();  // all waves done reading sK
            T* sA = sK;       // A[r][s], pitch PS
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sA[(16 * w + 4 * j4 + e) * PS + 16 * st + i16] = from_f32<T>(A[st][e]);
            __syncthreads();

            // ---- o = A v + QR S on all 64 rows, this wave's 16 columns
            f32x4 O[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                O[rt] = zero4();
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += M::KSTEP)
                    O[rt] = M::mma(frag_ld<T, PS, 1>(sA, 16 * rt, k0),
                                   frag_ld<T, PS, 1>(sVt, 16 * w, k0), O[rt]);
                f32x4 R = zero4();
                const T* qr = VEC ? sR : sQ;
                if constexpr (M::KPL == 1) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int sub = 0; sub < 4; ++sub)
                            R = M::mma(frag_ld_ctile<T, PK, 1>(qr, 16 * rt, 16 * ct, sub),
                                       frag_from_acc<T>(S[ct], S[ct], sub), R);
                } else {
#pragma unroll
                    for (int p = 0; p < NCT / 2; ++p)
                        R = M::mma(frag_ld_ctile<T, PK, 1>(qr, 16 * rt, 32 * p, 0),
                                   frag_from_acc<T>(S[2 * p], S[2 * p + 1], 0), R);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rt + 4 * j4 + e;
                    float f = 1.f;
                    if (!VEC) f = r < first_reset ? sEq[r] : 0.f;
                    O[rt][e] += f * R[e];
                }
            }
            // write o (rows < nvalid)
            T* o = (T*)a.o;
            const int n = nv0 + 16 * w + i16;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rt + 4 * j4 + e;
                    if (r < nvalid) o[((b * T_ + t0 + r) * a.H + h) * DV + n] = from_f32<T>(O[rt][e]);
                }
        }

        if constexpr (MODE == MODE_STATES || MODE == MODE_DSTATE) {
            // state entering this chunk (forward) / gradient at this chunk's end (reverse)
            float* dst = (REV ? a.ws_dS : a.ws_S) + ((bh * (NC + (REV ? 0 : 1)) + ci) * DK) * DV;
            const int n = nv0 + 16 * w + i16;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(16 * ct + 4 * j4 + e) * DV + n] = S[ct][e];
        }

        // ---- state update: S = decay * S + U^T W  (U = KU or QR, W = v or dO)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * ct + 4 * j4 + e;
                S[ct][e] *= VEC ? sDecay[c] : sDecay[0];
            }
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += M::KSTEP)
                S[ct] = M::mma(frag_ld<T, 1, PK>(sU, 16 * ct, k0),
                               frag_ld<T, PS, 1>(sVt, 16 * w, k0), S[ct]);
        }
        __syncthreads();  // LDS reused by the next chunk
    }

    // ---- final state
    float* fin = nullptr;
    if constexpr (MODE == MODE_OUT) fin = a.hT;
    if constexpr (MODE == MODE_STATES) fin = a.ws_S + (bh * (NC + 1) + NC) * DK * DV;
    if constexpr (MODE == MODE_DSTATE) fin = a.dh0;
    if (fin) {
        if constexpr (MODE != MODE_STATES) fin += bh * DK * DV;
        const int n = nv0 + 16 * w + i16;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) fin[(16 * ct + 4 * j4 + e) * DV + n] = S[ct][e];
    }
}

template <typename T, bool VEC, int DK, int DV, int MODE>
hipError_t launch_pass(const PassArgs& a, hipStream_t st) {
    const int64_t grid = a.B * a.H * (DV / 64);
    hipLaunchKernelGGL((k_pass<T, VEC, DK, DV, MODE>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    return hipGetLastError();
}

#define GLA_INST_PASS(T, VEC, DK, DV)                                                   \
    template hipError_t launch_pass<T, VEC, DK, DV, MODE_OUT>(const PassArgs&, hipStream_t); \
    template hipError_t launch_pass<T, VEC, DK, DV, MODE_STATES>(const PassArgs&, hipStream_t); \
    template hipError_t launch_pass<T, VEC, DK, DV, MODE_DSTATE>(const PassArgs&, hipStream_t);
#define GLA_INST_PASS_D(T, VEC) \
    GLA_INST_PASS(T, VEC, 64, 64) GLA_INST_PASS(T, VEC, 64, 128) \
    GLA_INST_PASS(T, VEC, 128, 64) GLA_INST_PASS(T, VEC, 128, 128)
GLA_INST_PASS_D(float, false)
GLA_INST_PASS_D(float, true)
GLA_INST_PASS_D(bf16, false)
GLA_INST_PASS_D(bf16, true)

}  // namespace gla
