// gla_fwd.hip -- fused chunk-parallel forward of gated linear attention (gfx950).
//
// One workgroup (4 waves) owns one (batch row b, head h, NV-column slice of
// d_v) and walks the sequence chunk by chunk (C = 64 tokens).  The state
// slice S[d_k][NV] stays on chip for the whole sequence: an fp32 master copy
// in matrix-core accumulators (each wave owns some 16x16 tiles) and a copy in
// the operand dtype in LDS for the readout.  State passing and readout run in
// the same program (FLAT page, "FLAT: Flash Linear Attention on TPUs", Pallas
// Kernels > Forward Kernels: the fused block-recurrent kernel).
//
// Per chunk, with beta the chunk-local inclusive prefix of the log gates and
// Gamma its total (FLAT page, Linear Attention > Forward Recurrence, the
// chunkwise form, and Pallas Kernels > Mamba-2 / Gated Linear Attention: all
// gate ratios are exponentials of chunk-local prefix sums of log f):
//
//   A[r][s] = sum_c q[r][c] k[s][c] exp(beta_r[c] - beta_s[c]),  s <= r in one document
//   o[r]    = sum_s A[r][s] v[s] + [r in the chunk's first document] (q[r] exp(beta_r))^T S
//   S      <- [no reset in chunk] diag(exp Gamma) S
//              + sum_{s in the chunk's last document} (k[s] exp(Gamma - beta_s)) v[s]^T
//
// Vector gate: A = QA KA^T with QA = q exp(beta - m), KA = k exp(m - beta),
// m = beta at row 31 (a reference inside the chunk keeps every exponent within
// half the chunk's total decay); the readout uses QA * exp(m) and the update
// KA * exp(Gamma - m).  A chunk with a gate too strong for that factored form
// (gla_exact.hpp) forms its scores from the prefixes directly, one channel tile
// of prefixes at a time, and reads out with q exp(beta), updates with
// k exp(Gamma - beta).  Scalar gate: A = (q k^T) * exp(beta_r - beta_s); row
// factors exp(beta_r) and exp(Gamma - beta_s) go on the readout and update.
//
// Pipelining: the next chunk's q, k, v, g and reset flags are loaded into
// registers while the current chunk computes.  Wave w owns output rows
// [16w, 16w+16): it forms only the tiles of A^T at or below the diagonal for
// those rows and feeds them to the A v product straight from its accumulators.
#include "gla_common.hpp"
#include "gla_exact.hpp"
#include "gla_kernels.hpp"
#include "gla_tile.hpp"

namespace gla {



template <typename T, bool VEC, int DK, int DV, int NV>
__global__ __launch_bounds__(NT) void k_fwd(const PassArgs a) {
    constexpr int NVS = DV / NV;
    constexpr int PK = Pitch16<T>::of(DK);
    constexpr int PV = Pitch16<T>::of(NV);
    constexpr int PSS = Pitch16<T>::of(DK);
    constexpr int NCT = DK / 16, NNT = NV / 16;
    constexpr int UPW = NCT * NNT / 4;  // state tiles per wave
    static_assert(UPW >= 1, "");
    constexpr int CPW = NCT / 4;        // channel tiles per wave in the gate scan
    static_assert(UPW == CPW * NNT, "state tiles of a wave cover its scan channel tiles");
    using M = Mma<T>;

    __shared__ __attribute__((aligned(16))) T sQ[C * PK];    // raw q, then QA (vector gate)
    __shared__ __attribute__((aligned(16))) T sK[C * PK];    // raw k, then KA (vector gate)
    __shared__ __attribute__((aligned(16))) T sG[VEC ? C * PK : 1];   // gate tile [row][channel]
    __shared__ __attribute__((aligned(16))) T sV[C * PV];    // v slice [row][column]
    __shared__ __attribute__((aligned(16))) T sS[NV * PSS];  // state (x exp(m)) as [n][c]
    __shared__ int sDoc[C];
    __shared__ float sBeta[C], sFq[C], sFu[C];
    __shared__ float sDecay[VEC ? DK : 1];
    __shared__ float sEGm[VEC ? DK : 1];
    __shared__ int sAnyReset;
    // strong-gate chunks: one channel tile of fp32 prefixes [row][16], the per-wave flags
    constexpr int PBB = 20;
    __shared__ __attribute__((aligned(16))) float sBB[VEC ? C * PBB : 4];
    __shared__ int sStrong[4];

    // block -> (b, h, piece, slice); the slices of one piece are adjacent (one XCD)
    const int64_t P = a.P;
    const int64_t L = xcd_logical_block(a.B * a.H * NVS * P);
    const int ns = (int)(L % NVS);
    const int64_t piece = (L / NVS) % P;
    const int64_t bh = L / NVS / P;
    const int n0 = ns * NV;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t cbeg = piece * a.PL;
    const int64_t cend = (cbeg + a.PL < NC) ? cbeg + a.PL : NC;

    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.g;
    const int64_t rs_qk = a.ld_qk, rs_v = a.ld_v;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qbase = q + b * T_ * rs_qk + hq * DK;
    const T* kbase = k + b * T_ * rs_qk + hq * DK;
    const T* vbase = v + b * T_ * rs_v + h * DV + n0;
    const T* gbase = g + b * T_ * rs_g + (VEC ? h * DK : h);

    // ---- state tiles owned by this wave: u -> (ct, nt), fp32 master copy
    f32x4 S[UPW];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int u = w * UPW + i, ct = u / NNT, nt = u % NNT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * ct + 4 * j4 + e, n = n0 + 16 * nt + i16;
            if (P > 1) S[i][e] = a.S_in[((bh * P + piece) * DK + c) * DV + n];
            else S[i][e] = a.h0 ? a.h0[(bh * DK + c) * DV + n] : 0.f;
        }
    }

    TileRegs<T, DK> pq, pk;
    TileRegs<T, NV> pv;
    TileRegs<T, VEC ? DK : 16> pg;
    RowRegs rr;
    auto prefetch = [&](int64_t t0) {
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;
        pq.load(qbase + t0 * rs_qk, rs_qk, nvalid);
        pk.load(kbase + t0 * rs_qk, rs_qk, nvalid);
        pv.load(vbase + t0 * rs_v, rs_v, nvalid);
        if constexpr (VEC) pg.load(gbase + t0 * rs_g, rs_g, nvalid);
        if (w == 0) rr.load(gbase + t0 * rs_g, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    };
    [[maybe_unused]] const TriOnes<T> tri;  // gate prefix operands (vector gate)
    prefetch(cbeg * C);

    for (int64_t it = cbeg; it < cend; ++it) {
        const int64_t t0 = it * C;
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;

        // ---- stage this chunk from registers
        pq.store_rows(sQ, PK);
        pk.store_rows(sK, PK);
        pv.store_rows(sV, PV);
        if constexpr (VEC) {
            pg.store_rows(sG, PK);
            strong_flag_put(sStrong, gate_regs_strong(pg));
        }
        if (w == 0) {
            const int r = l;
            const int doc = wave_incl_scan_i(rr.reset());
            const uint64_t msk = __ballot(rr.reset());
            const int first_reset = msk ? __builtin_ctzll(msk) : C;
            const int last_reset = msk ? 63 - __builtin_clzll(msk) : -1;
            sDoc[r] = doc;
            if (r == 0) sAnyReset = msk != 0;
            if constexpr (!VEC) {
                const float beta = wave_incl_scan(rr.g());
                const float Gam = __shfl(beta, 63, 64);
                sBeta[r] = beta;
                sFq[r] = r < first_reset ? __expf(beta) : 0.f;
                sFu[r] = r >= last_reset ? __expf(Gam - beta) : 0.f;
                if (r == 0) sDecay[0] = msk ? 0.f : __expf(Gam);
            } else {
                sFq[r] = r < first_reset ? 1.f : 0.f;
                sFu[r] = r >= last_reset ? 1.f : 0.f;
            }
        }
        __syncthreads();
        [[maybe_unused]] const bool strong = VEC && strong_flag_get<4>(sStrong);
        if (it + 1 < cend) prefetch(t0 + C);

        // strong-gate chunks: this wave's A^T tiles (rows s = 16st + 4j4 + e, column
        // r = 16w + i16) summed over the channel tiles from the prefixes themselves
        f32x4 Ax[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) Ax[st] = zero4();
        if constexpr (VEC) {
            // ---- gate prefix on the matrix cores; QA, KA in place; per-channel factors
            f32x4 beta[CPW][4];
            gate_prefix_mfma<T, CPW, PK>(sG, tri, beta);
            const bool any_reset = sAnyReset != 0;
            if (strong) {
                // (loops kept rolled: this path is rare and must not add register pressure)
                const int r = 16 * w + i16;
                const int dr = sDoc[r];
#pragma unroll 1
                for (int ct = 0; ct < NCT; ++ct) {
                    if (w == ct / CPW) {
                        const int cc = ct % CPW;
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float b = beta[0][rt][e];
#pragma unroll
                                for (int u = 1; u < CPW; ++u) b = cc == u ? beta[u][rt][e] : b;
                                sBB[(16 * rt + i16) * PBB + 4 * j4 + e] = b;
                            }
                    }
                    __syncthreads();
#pragma unroll 1
                    for (int idx = 0; idx < 16; ++idx) {
                        const int st = idx >> 2, e = idx & 3;
                        const int s = 16 * st + 4 * j4 + e;
                        if (st > w) break;
                        if (s <= r && sDoc[s] == dr) {
                            const float x = exact_dot<T>(sQ + r * PK + 16 * ct, sK + s * PK + 16 * ct,
                                                         sBB + r * PBB, sBB + s * PBB, 16, 0.f);
#pragma unroll
                            for (int u = 0; u < 16; ++u) Ax[u >> 2][u & 3] += idx == u ? x : 0.f;
                        }
                    }
                    __syncthreads();
                }
            }
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) {
                const int c0 = 16 * (CPW * w + cc) + 4 * j4;   // this lane's 4 channels
                float m[4], Gam[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    m[e] = strong ? 0.f : __shfl(beta[cc][1][e], 16 * j4 + 15, 64);  // row 31
                    Gam[e] = __shfl(beta[cc][3][e], 16 * j4 + 15, 64);               // row 63
                }
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int r = 16 * rt + i16;
                    Vec4<T> qv = Vec4<T>::load(sQ + r * PK + c0);
                    Vec4<T> kv = Vec4<T>::load(sK + r * PK + c0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float E = __expf(beta[cc][rt][e] - m[e]);
                        // (strong: the update operand k exp(Gamma - beta) itself)
                        const float Ei = strong ? __expf(Gam[e] - beta[cc][rt][e]) : __builtin_amdgcn_rcpf(E);
                        qv.set(e, qv.get(e) * E);
                        kv.set(e, kv.get(e) * Ei);
                    }
                    qv.store(sQ + r * PK + c0);
                    kv.store(sK + r * PK + c0);
                }
                if (i16 == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sDecay[c0 + e] = any_reset ? 0.f : __expf(Gam[e]);
                        sEGm[c0 + e] = strong ? 1.f : __expf(Gam[e] - m[e]);
                    }
                }
                // readout copy of the state, scaled by exp(m) per channel: this
                // wave's state tiles are exactly its scan channel tiles
#pragma unroll
                for (int nt = 0; nt < NNT; ++nt) {
                    const int i = cc * NNT + nt;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sS[(16 * nt + i16) * PSS + c0 + e] = from_f32<T>(S[i][e] * __expf(m[e]));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < UPW; ++i) {
                const int u = w * UPW + i, ct = u / NNT, nt = u % NNT;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sS[(16 * nt + i16) * PSS + 16 * ct + 4 * j4 + e] = from_f32<T>(S[i][e]);
            }
        }
        __syncthreads();

        // ---- this wave's rows r in [16w, 16w+16): A^T tiles, then A v and the readout
        const int r_me = 16 * w + i16;
        const int doc_r = sDoc[r_me];
        const float beta_r = VEC ? 0.f : sBeta[r_me];
        constexpr int KF = DK / M::KSTEP;
        typename M::frag qf[KF];
#pragma unroll
        for (int kk = 0; kk < KF; ++kk) qf[kk] = frag_ld<T, PK, 1>(sQ, 16 * w, kk * M::KSTEP);
        f32x4 At[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            At[st] = Ax[st];
            if (st <= w && !strong) {
#pragma unroll
                for (int kk = 0; kk < KF; ++kk)
                    At[st] = M::mma(frag_ld<T, PK, 1>(sK, 16 * st, kk * M::KSTEP), qf[kk], At[st]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * st + 4 * j4 + e;
                    const bool keep = s <= r_me && sDoc[s] == doc_r;
                    float x = At[st][e];
                    if constexpr (!VEC) x *= __expf(beta_r - sBeta[s]);
                    At[st][e] = keep ? x : 0.f;
                }
            }
        }
        {
            T* o = (T*)a.o;
            // output tile C layout (M = r, N = n): lane n, rows 4*j4 + e
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
                f32x4 O = zero4(), R = zero4();
                if constexpr (M::KPL == 1) {
#pragma unroll
                    for (int st = 0; st < 4; ++st)
                        if (st <= w)
#pragma unroll
                            for (int sub = 0; sub < 4; ++sub)
                                O = M::mma(frag_col<T, PV, true>(sV, 16 * nt, 16 * st, sub),
                                           frag_from_acc<T>(At[st], At[st], sub), O);
                } else {
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        if (2 * p <= w)
                            O = M::mma(frag_col<T, PV, true>(sV, 16 * nt, 32 * p),
                                       frag_from_acc<T>(At[2 * p], At[2 * p + 1], 0), O);
                }
#pragma unroll
                for (int kk = 0; kk < KF; ++kk)
                    R = M::mma(frag_ld<T, PSS, 1>(sS, 16 * nt, kk * M::KSTEP), qf[kk], R);
                // O, R are o^T tiles: lane r = 16w + i16, rows n = 16nt + 4*j4 + e
                const float fq = sFq[r_me];
                if (r_me < nvalid) {
                    T* orow = o + ((b * T_ + t0 + r_me) * a.H + h) * DV + n0 + 16 * nt + 4 * j4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) orow[e] = from_f32<T>(O[e] + fq * R[e]);
                }
            }
        }

        // ---- state update on this wave's tiles
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            const int u = w * UPW + i, ct = u / NNT, nt = u % NNT;
            f32x4 U = zero4();
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += M::KSTEP) {
                typename M::frag ku = frag_col<T, PK, false>(sK, 16 * ct, k0);
#pragma unroll
                for (int e = 0; e < M::KPL; ++e) {
                    const int s = k0 + j4 * M::KPL + e;
                    float x;
                    if constexpr (M::KPL == 1) x = to_f32(ku); else x = to_f32(ku[e]);
                    M::set(ku, e, x * sFu[s]);
                }
                U = M::mma(ku, frag_col<T, PV, false>(sV, 16 * nt, k0), U);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * ct + 4 * j4 + e;
                if constexpr (VEC) S[i][e] = sDecay[c] * S[i][e] + sEGm[c] * U[e];
                else S[i][e] = sDecay[0] * S[i][e] + U[e];
            }
        }
        __syncthreads();
    }

    if (a.hT && piece == P - 1) {
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            const int u = w * UPW + i, ct = u / NNT, nt = u % NNT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * ct + 4 * j4 + e, n = n0 + 16 * nt + i16;
                a.hT[(bh * DK + c) * DV + n] = S[i][e];
            }
        }
    }
}

template <typename T, bool VEC, int DK, int DV, int NV>
hipError_t launch_fwd(const PassArgs& a, hipStream_t st) {
    const int64_t grid = a.B * a.H * (DV / NV) * a.P;
    hipLaunchKernelGGL((k_fwd<T, VEC, DK, DV, NV>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    return hipGetLastError();
}

#define GLA_INST_FWD(T, VEC, DK, DV, NV) \
    template hipError_t launch_fwd<T, VEC, DK, DV, NV>(const PassArgs&, hipStream_t);
#define GLA_INST_FWD_NV(T, VEC, DK, DV) GLA_INST_FWD(T, VEC, DK, DV, 16) GLA_INST_FWD(T, VEC, DK, DV, 32)
#define GLA_INST_FWD_D(T, VEC)                                            \
    GLA_INST_FWD_NV(T, VEC, 64, 64) GLA_INST_FWD_NV(T, VEC, 64, 128)      \
    GLA_INST_FWD_NV(T, VEC, 128, 64) GLA_INST_FWD_NV(T, VEC, 128, 128)
#define GLA_INST_FWD_D64(T, VEC)                                          \
    GLA_INST_FWD(T, VEC, 64, 64, 64) GLA_INST_FWD(T, VEC, 64, 128, 64)   \
    GLA_INST_FWD(T, VEC, 128, 64, 64) GLA_INST_FWD(T, VEC, 128, 128, 64)
GLA_INST_FWD_D(float, false)
GLA_INST_FWD_D(float, true)
GLA_INST_FWD_D(bf16, false)
GLA_INST_FWD_D(bf16, true)
GLA_INST_FWD_D64(bf16, false)
GLA_INST_FWD_D64(bf16, true)

}  // namespace gla
