// gla_states.hip -- backward state recompute (gfx950): the forward recurrence
// without readout, writing the state that enters every chunk, and the final
// state, to the workspace in the input dtype as [c][n] tiles.
//
// This is the state-passing half of the two-kernel backward on the FLAT page
// ("FLAT: Flash Linear Attention on TPUs", Linear Attention > Backward
// Recurrence: a state-passing kernel reruns the forward recurrence and stores
// the state at the start of every chunk; Pallas Kernels > Backward Kernels).
// The update S <- diag(decay) S + KU^T v splits into independent 64x64 blocks
// of S (rows by key channel, columns by value column), so one workgroup owns
// one block of one (b, h) and there is no exchange between workgroups.
//
// Each wave owns the 16 key channels [16w, 16w+16) of its block and keeps the
// transposed state S^T (rows n, columns c) for them in accumulators, so its
// C-layout lanes hold four consecutive n of one channel c: the [c][n] stores
// are 8 bytes wide.
#include "gla_common.hpp"
#include "gla_kernels.hpp"
#include "gla_tile.hpp"

namespace gla {

template <typename T, bool VEC, int DK, int DV>
__global__ __launch_bounds__(NT) void k_states(const PassArgs a) {
    constexpr int CB = 64, NB = 64;          // block of the state
    constexpr int NCB = DK / CB, NNB = DV / NB;
    constexpr int PB = Pitch16<T>::of(CB);   // pitch of [row][64] tiles
    constexpr int NNT = NB / 16;
    using M = Mma<T>;

    __shared__ __attribute__((aligned(16))) T sK[C * PB];
    __shared__ __attribute__((aligned(16))) T sV[C * PB];
    __shared__ __attribute__((aligned(16))) T sG[VEC ? C * PB : 1];
    __shared__ float sFu[C];
    __shared__ float sDecay[CB];
    __shared__ int sLastReset;

    const int64_t L = xcd_logical_block(a.B * a.H * NCB * NNB);
    const int64_t bh = L / (NCB * NNB);
    const int blk = (int)(L % (NCB * NNB));
    const int c0 = (blk / NNB) * CB, n0 = (blk % NNB) * NB;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;

    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.g;
    const int64_t rs_qk = a.Hqk * DK, rs_v = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* kbase = k + b * T_ * rs_qk + hq * DK + c0;
    const T* vbase = v + b * T_ * rs_v + h * DV + n0;
    const T* gbase = g + b * T_ * rs_g + (VEC ? h * DK + c0 : h);
    T* ws = (T*)a.ws_S;  // [B*H][NC+1][DK][DV]

    // S^T tiles of this wave: (nt, channel tile w); lane c = c0 + 16w + i16, rows n
    f32x4 St[NNT];
    const int cme = c0 + 16 * w + i16;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            St[nt][e] = a.h0 ? a.h0[(bh * DK + cme) * DV + n0 + 16 * nt + 4 * j4 + e] : 0.f;

    TileRegs<T, CB> pk, pg;
    TileRegs<T, NB> pv;
    RowRegs rr;
    auto prefetch = [&](int64_t t0) {
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;
        pk.load(kbase + t0 * rs_qk, rs_qk, nvalid);
        pv.load(vbase + t0 * rs_v, rs_v, nvalid);
        if constexpr (VEC) pg.load(gbase + t0 * rs_g, rs_g, nvalid);
        if (w == 0) rr.load(gbase + t0 * rs_g, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    };
    auto store_state = [&](int64_t ci) {
        T* dst = ws + ((bh * (NC + 1) + ci) * DK + cme) * DV + n0;
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
            Vec4<T> x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x.set(e, St[nt][e]);
            x.store(dst + 16 * nt + 4 * j4);
        }
    };
    prefetch(0);

    for (int64_t ci = 0; ci < NC; ++ci) {
        const int64_t t0 = ci * C;
        store_state(ci);
        pk.store_rows(sK, PB);
        pv.store_rows(sV, PB);
        if constexpr (VEC) pg.store_rows(sG, PB);
        if (w == 0) {
            const int r = l;
            const uint64_t msk = __ballot(rr.reset);
            const int last_reset = msk ? 63 - __builtin_clzll(msk) : -1;
            if (r == 0) sLastReset = last_reset;
            if constexpr (!VEC) {
                const float beta = wave_incl_scan(rr.g);
                const float Gam = __shfl(beta, 63, 64);
                sFu[r] = r >= last_reset ? __expf(Gam - beta) : 0.f;
                if (r == 0) sDecay[0] = msk ? 0.f : __expf(Gam);
            }
        }
        __syncthreads();
        if (ci + 1 < NC) prefetch(t0 + C);

        if constexpr (VEC) {
            // per-channel prefix on the matrix cores; KU = k exp(Gamma - beta), last document only
            f32x4 beta[1][4];
            gate_prefix_mfma<T, 1, PB>(sG, beta);
            const int last_reset = sLastReset;
            const int cl = 16 * w + 4 * j4;  // this lane's 4 channels (block-local)
            float Gam[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) Gam[e] = __shfl(beta[0][3][e], 16 * j4 + 15, 64);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r = 16 * rt + i16;
                Vec4<T> kv = Vec4<T>::load(sK + r * PB + cl);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    kv.set(e, r >= last_reset ? kv.get(e) * __expf(Gam[e] - beta[0][rt][e]) : 0.f);
                kv.store(sK + r * PB + cl);
            }
            if (i16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sDecay[cl + e] = last_reset >= 0 ? 0.f : __expf(Gam[e]);
            __syncthreads();
        }

        // S^T[n][c] <- decay_c S^T[n][c] + sum_s v[s][n] KU[s][c], in place
        const float dec = VEC ? sDecay[16 * w + i16] : sDecay[0];
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) St[nt][e] *= dec;
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += M::KSTEP) {
            typename M::frag ku = frag_col<T, PB, false>(sK, 16 * w, k0);
            if constexpr (!VEC) {
#pragma unroll
                for (int e = 0; e < M::KPL; ++e) {
                    const int s = k0 + j4 * M::KPL + e;
                    float x;
                    if constexpr (M::KPL == 1) x = to_f32(ku); else x = to_f32(ku[e]);
                    M::set(ku, e, x * sFu[s]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt)
                St[nt] = M::mma(frag_col<T, PB, false>(sV, 16 * nt, k0), ku, St[nt]);
        }
        __syncthreads();
    }
    store_state(NC);
}

template <typename T, bool VEC, int DK, int DV>
hipError_t launch_states(const PassArgs& a, hipStream_t st) {
    const int64_t grid = a.B * a.H * (DK / 64) * (DV / 64);
    hipLaunchKernelGGL((k_states<T, VEC, DK, DV>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    return hipGetLastError();
}

#define GLA_INST_ST(T, VEC, DK, DV) \
    template hipError_t launch_states<T, VEC, DK, DV>(const PassArgs&, hipStream_t);
#define GLA_INST_ST_D(T, VEC)                                     \
    GLA_INST_ST(T, VEC, 64, 64) GLA_INST_ST(T, VEC, 64, 128)      \
    GLA_INST_ST(T, VEC, 128, 64) GLA_INST_ST(T, VEC, 128, 128)
GLA_INST_ST_D(float, false)
GLA_INST_ST_D(float, true)
GLA_INST_ST_D(bf16, false)
GLA_INST_ST_D(bf16, true)

}  // namespace gla
