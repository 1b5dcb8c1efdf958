// gla_grad.hip -- chunk-parallel gradient kernel of the backward (gfx950).
//
// The FLAT page ("FLAT: Flash Linear Attention on TPUs", Linear Attention >
// Backward Recurrence) notes that the state gradient obeys a recurrence of the
// forward's form with q and dO in the roles of k and v, and (Forward
// Recurrence) that a GPU splits the forward into a state kernel and a
// chunk-parallel output kernel to occupy its many cores.  The backward here
// does the same: the state pass stores the state entering every chunk (S0),
// the state-gradient pass stores the gradient of the state at every chunk's
// end (dS1), both in the input dtype, and then every (b, h, chunk) is an
// independent workgroup of this kernel.  With no carried state, a workgroup
// needs little LDS and several fit on one compute unit, so their load and
// matrix-core phases overlap.
//
// Per chunk (beta the chunk-local log-gate prefix, Gamma its total), with
// dA = dO v^T masked to s <= r in one document:
//   dq[r] = sum_s dA[r][s] k[s] exp(beta_r - beta_s) + [r in first doc] exp(beta_r) (S0 dO[r])
//   dk[s] = sum_r dA[r][s] q[r] exp(beta_r - beta_s) + [s in last doc] exp(Gamma - beta_s) (dS1 v[s])
//   dv[s] = sum_r A[r][s] dO[r]                      + [s in last doc] dS1^T (k[s] exp(Gamma - beta_s))
//   dg[u] = sum_{t >= u, same doc} (q*dq - k*dk)[t] + [u in last doc] rowsum(S1 * dS1)   (0 at resets)
// (FLAT page, Backward Recurrence: the log-gate gradient is a suffix sum of
// q*dq - k*dk inside the chunk plus a boundary term from the carried states.)
// The boundary term needs S1, the state after the chunk; it is not read from
// memory but expanded as S1 = diag(decay) S0 + KU^T v, KU = k exp(Gamma - beta)
// on the last document, so that
//   rowsum(S1 * dS1)_c = decay_c rowsum(S0 * dS1)_c + sum_s KU[s][c] (v dS1^T)[s][c],
// and the second sum reuses the inter-chunk part of dk.
//
// A vector-gate chunk whose gates are too strong for the factored form
// QA = q exp(beta - m), KA = k exp(m - beta) (gla_exact.hpp) forms A and the
// intra-chunk parts of dq and dk from the prefixes directly, and its
// carried-state terms from exp(beta) and exp(Gamma - beta).
//
// Two kinds of workgroups per chunk:
//   QK: 64 key channels, each wave 16 of them: dq, dk and dg (the suffix sums
//       stay inside one wave); the state and its gradient come straight from
//       memory in the register layouts the products want;
//   V:  64 value columns, each wave 16 of them: dv.
#include "gla_bwd.hpp"
#include "gla_common.hpp"
#include "gla_exact.hpp"
#include "gla_kernels.hpp"
#include "gla_tile.hpp"

namespace gla {

template <typename T, bool VEC, int DK, int DV>
struct GradCfg {
    static constexpr int CS = 64, NS = 64;     // key channels per QK, value columns per V workgroup
    static constexpr int NQK = DK / CS, NVR = DV / NS;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int PB = Pitch16<T>::of(64);
    static constexpr int PK = Pitch16<T>::of(DK);
    static constexpr int PV = Pitch16<T>::of(DV);
    // [DK][64] state-gradient slice: 8-byte aligned rows, as short as that allows so
    // that it fits in the place of the gate tile
    static constexpr int PD = sizeof(T) == 2 ? 68 : 66;
    static constexpr int PE = 68;              // fp32 [64][64] scratch
    static constexpr int max_(int a, int b) { return a > b ? a : b; }

    // QK role: q, k (, g) slices, dA [r][s], dO and v.  The dg scratch of chunks
    // with documents inside takes the g / dA region once the products are done.
    static constexpr int TILE64 = C * PB * ES;
    static constexpr int QK_OFF_G = 2 * TILE64;
    static constexpr int QK_OFF_DA = QK_OFF_G + (VEC ? TILE64 : 0);
    static constexpr int QK_OFF_DO = QK_OFF_DA + TILE64;
    static constexpr int QK_BYTES = QK_OFF_DO + 2 * C * PV * ES;
    static_assert(!VEC || 2 * TILE64 >= C * PE * 4, "dg scratch does not fit");

    // V role: q, k (, g) for all channels, the dO slice and A^T; the dS1 slice takes
    // the place of g once g is consumed when it fits there.
    static constexpr int TILEK = C * PK * ES;
    static constexpr bool DS_IN_G = VEC && DK * PD <= C * PK;
    static constexpr int V_OFF_G = 2 * TILEK;
    static constexpr int V_OFF_DO = V_OFF_G + (VEC ? TILEK : 0);
    static constexpr int V_OFF_A = V_OFF_DO + TILE64;
    static constexpr int V_OFF_DS = DS_IN_G ? V_OFF_G : V_OFF_A + TILE64;
    static constexpr int V_BYTES = V_OFF_A + TILE64 + (DS_IN_G ? 0 : DK * PD * ES);

    static constexpr int BYTES = max_(QK_BYTES, V_BYTES);
};

// Small per-workgroup arrays (both roles).
struct GradSmall {
    RevChunk ck;
    float sEGm[128];      // vector gate: exp(Gamma - m) per channel (V role)
    float sBnd[4][16];    // per-wave boundary terms (QK role, chunks with documents inside)
    float sXs[4][C];      // scalar gate: per-wave partial sums
    float sBs[4];
    int sStrong[4];       // vector gate: per-wave flags, a gate too strong for the factored form
};

// ============================================================== QK role
// Outputs are computed transposed (rows = key channels, columns = chunk rows):
// lane (i, j) of the wave holds rows r = 16rt + i and the four channels
// cw + 4j + e, which is also where the gate prefix leaves exp(beta - m), so the
// gate factors never leave registers and dq, dk, dg go out as 4-channel stores.
template <typename T, bool VEC, int DK, int DV>
__device__ void grad_qk(const RevArgs& a, char* lds, GradSmall& sm, int64_t bh, int64_t ci, int slice) {
    using Cfg = GradCfg<T, VEC, DK, DV>;
    using M = Mma<T>;
    constexpr int PB = Cfg::PB, PV = Cfg::PV, PE = Cfg::PE;
    constexpr int KS = M::KSTEP, NKV = DV / KS;

    T* sQ = reinterpret_cast<T*>(lds);
    T* sK = sQ + C * PB;
    T* sG = reinterpret_cast<T*>(lds + Cfg::QK_OFF_G);    // vector gate only
    T* sdA = reinterpret_cast<T*>(lds + Cfg::QK_OFF_DA);  // [r][s]
    T* sdO = reinterpret_cast<T*>(lds + Cfg::QK_OFF_DO);
    T* sV = sdO + C * PV;
    float* sX = reinterpret_cast<float*>(lds + Cfg::QK_OFF_G);  // dg scratch [r][c], after the products
    RevChunk& ck = sm.ck;

    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int cs0 = slice * Cfg::CS;
    const int cw = cs0 + 16 * w;  // first channel of this wave's tile
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t t0 = ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t rs_qk = a.ld_qk, rs_v = a.ld_v, rs_do = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qrow = (const T*)a.q + (b * T_ + t0) * rs_qk + hq * DK + cs0;
    const T* krow = (const T*)a.k + (b * T_ + t0) * rs_qk + hq * DK + cs0;
    const T* vrow = (const T*)a.v + (b * T_ + t0) * rs_v + h * DV;
    const T* dorow = (const T*)a.dO + (b * T_ + t0) * rs_do + h * DV;
    const T* grow = (const T*)a.g + (b * T_ + t0) * rs_g + (VEC ? h * DK + cs0 : h);
    // rows cw + i of S0 and dS1, the A operands of dO S0^T and v dS1^T (k = n)
    const T* S0 = (const T*)a.ws_S + ((bh * (NC + 1) + ci) * DK + cw + i16) * DV;
    const T* dS1 = (const T*)a.ws_dS + ((bh * NC + ci) * DK + cw + i16) * DV;

    // ---- loads
    TileRegs<T, 64> pq, pk, pg;
    TileRegs<T, DV> pv, pdo;
    RowRegs rr;
    pq.load(qrow, rs_qk, nvalid);
    pk.load(krow, rs_qk, nvalid);
    if constexpr (VEC) pg.load(grow, rs_g, nvalid);
    pv.load(vrow, rs_v, nvalid);
    pdo.load(dorow, rs_do, nvalid);
    if (w == 0) rr.load(grow, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    typename M::frag s0f[NKV], dsf[NKV];
#pragma unroll
    for (int kk = 0; kk < NKV; ++kk) {
        if constexpr (M::KPL == 1) {
            s0f[kk] = S0[kk * KS + j4];
            dsf[kk] = dS1[kk * KS + j4];
        } else {
            s0f[kk] = *reinterpret_cast<const bf16x8*>(S0 + kk * KS + 8 * j4);
            dsf[kk] = *reinterpret_cast<const bf16x8*>(dS1 + kk * KS + 8 * j4);
        }
    }
    [[maybe_unused]] const TriOnes<T> tri;

    pq.store_rows(sQ, PB);
    pk.store_rows(sK, PB);
    if constexpr (VEC) {
        pg.store_rows(sG, PB);
        strong_flag_put(sm.sStrong, gate_regs_strong(pg));
    }
    pv.store_rows(sV, PV);
    pdo.store_rows(sdO, PV);
    if (w == 0) rev_chunk_info<T, VEC>(&ck, rr);
    // rowsum(S0 * dS1) of channel cw + i16 over this lane's n
    float sd = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKV; ++kk) sd = frag_dot(s0f[kk], dsf[kk], sd);
    __syncthreads();
    [[maybe_unused]] const bool strong = VEC && strong_flag_get<4>(sm.sStrong);

    // raw q, k at this lane's output positions (rows 16rt + i16, channels cw + 4j4 + e)
    Vec4<T> qraw[4], kraw[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        qraw[rt] = Vec4<T>::load(sQ + (16 * rt + i16) * PB + 16 * w + 4 * j4);
        kraw[rt] = Vec4<T>::load(sK + (16 * rt + i16) * PB + 16 * w + 4 * j4);
    }
    // exp(beta - m) at those positions (vector gate; strong-gate chunks: beta itself)
    float E[4][4];
    // em = exp(m), egm = exp(Gamma - m) (strong-gate chunks: 1 and Gamma itself)
    float em[4], egm[4], dec[4];
    if constexpr (VEC) {
        // gate prefix on the matrix cores; this wave's q, k columns scaled in place to
        // QA = q exp(beta - m), KA = k exp(m - beta), m the prefix at row 31 (factored exponent)
        f32x4 beta[1][4];
        gate_prefix_mfma<T, 1, PB>(sG, tri, beta);
        float m[4], Gam[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[e] = __shfl(beta[0][1][e], 16 * j4 + 15, 64);
            Gam[e] = __shfl(beta[0][3][e], 16 * j4 + 15, 64);
        }
        const bool reset_in_chunk = ck.last_reset >= 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            em[e] = strong ? 1.f : __expf(m[e]);
            egm[e] = strong ? Gam[e] : __expf(Gam[e] - m[e]);
            dec[e] = reset_in_chunk ? 0.f : __expf(Gam[e]);
        }
        if (strong) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) E[rt][e] = beta[0][rt][e];
        } else {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            Vec4<T> qa, ka;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                E[rt][e] = __expf(beta[0][rt][e] - m[e]);
                qa.set(e, qraw[rt].get(e) * E[rt][e]);
                ka.set(e, kraw[rt].get(e) * __builtin_amdgcn_rcpf(E[rt][e]));
            }
            qa.store(sQ + (16 * rt + i16) * PB + 16 * w + 4 * j4);
            ka.store(sK + (16 * rt + i16) * PB + 16 * w + 4 * j4);
        }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            em[e] = egm[e] = 1.f;
            dec[e] = ck.decay;
        }
    }

    // ---- dA^T = v dO^T on the 10 lower tiles (+ the two upper tiles a 32-wide k
    // step reads), masked, stored as dA[r][s]
    for (int ti = w; ti < 12; ti += 4) {
        const int rt = score_tile_rt(ti);
        const int st = score_tile_st(ti);
        f32x4 acc = zero4();
        if (ti < 10) {
#pragma unroll
            for (int n0 = 0; n0 < DV; n0 += KS)
                acc = M::mma(frag_ld<T, PV, 1>(sV, 16 * st, n0), frag_ld<T, PV, 1>(sdO, 16 * rt, n0), acc);
        }
        store_masked_N<T, VEC, PB>(sdA, ck, rt, st, ti < 10, acc);
    }
    __syncthreads();

    const bool gqa = G > 1;
    // q*dq - k*dk; strong-gate chunks: the same without the diagonal pairs of the
    // scores (which cancel) and without k * (the carried part of dk), kept in z
    float x[4][4];
    [[maybe_unused]] float z[4][4];
    // ---- dq^T = KA^T dA^T + [first doc] exp(m) S0 dO^T, times exp(beta - m)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        f32x4 a1 = zero4(), a2 = zero4();
        const int kend = ((16 * (rt + 1) + KS - 1) / KS) * KS;
        if (!strong) {
#pragma unroll
            for (int k0 = 0; k0 < kend; k0 += KS)
                a1 = M::mma(frag_col<T, PB, false>(sK, 16 * w, k0), frag_ld<T, PB, 1>(sdA, 16 * rt, k0), a1);
        }
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk)
            a2 = M::mma(s0f[kk], frag_ld<T, PV, 1>(sdO, 16 * rt, kk * KS), a2);
        const int r = 16 * rt + i16;
        const float fq = ck.fq[r];
        float dq[4];
        if (strong) {
            float dx[4] = {0.f, 0.f, 0.f, 0.f}, dd[4] = {0.f, 0.f, 0.f, 0.f};
            exact_dq<T, PB, PB>(dx, dd, rt, E, sdA, sK + 16 * w + 4 * j4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dqx = dx[e] + fq * __expf(E[rt][e]) * a2[e];
                dq[e] = dqx + dd[e];
                x[rt][e] = qraw[rt].get(e) * dqx;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dqp = a1[e] + fq * em[e] * a2[e];
                dq[e] = VEC ? E[rt][e] * dqp : dqp;
                x[rt][e] = qraw[rt].get(e) * dq[e];
            }
        }
        if (r < nvalid) {
            if (!gqa) store4<T>((T*)a.dq + (b * T_ + t0 + r) * a.ld_dqk + hq * DK + cw + 4 * j4, dq);
            else store4<float>(a.ws_dq + ((b * T_ + t0 + r) * a.H + h) * DK + cw + 4 * j4, dq);
        }
    }
    // ---- dk^T = QA^T dA + [last doc] exp(Gamma - m) dS1 v^T, times exp(m - beta);
    // the boundary sum: sum_s KU[s][c] (v dS1^T)[s][c]
    float bsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        f32x4 a1 = zero4(), a2 = zero4();
        const int kbeg = (16 * st / KS) * KS;
        if (!strong) {
#pragma unroll
            for (int k0 = kbeg; k0 < C; k0 += KS)
                a1 = M::mma(frag_col<T, PB, false>(sQ, 16 * w, k0), frag_col<T, PB, false>(sdA, 16 * st, k0), a1);
        }
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk)
            a2 = M::mma(dsf[kk], frag_ld<T, PV, 1>(sV, 16 * st, kk * KS), a2);
        const int s = 16 * st + i16;
        const float fu = ck.fu[s];
        float dk[4];
        if (strong) {
            float dx[4] = {0.f, 0.f, 0.f, 0.f}, dd[4] = {0.f, 0.f, 0.f, 0.f};
            exact_dk<T, PB, PB>(dx, dd, st, E, sdA, sQ + 16 * w + 4 * j4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float inter = fu * __expf(egm[e] - E[st][e]) * a2[e];
                const float kr = kraw[st].get(e);
                dk[e] = dx[e] + dd[e] + inter;
                x[st][e] -= kr * dx[e];
                z[st][e] = kr * inter;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float inter = fu * egm[e] * a2[e];
                const float rE = VEC ? __builtin_amdgcn_rcpf(E[st][e]) : 1.f;
                const float kr = kraw[st].get(e);
                dk[e] = (a1[e] + inter) * rE;
                x[st][e] -= kr * dk[e];
                bsum[e] += kr * inter * rE;
            }
        }
        if (s < nvalid) {
            if (!gqa) store4<T>((T*)a.dk + (b * T_ + t0 + s) * a.ld_dqk + hq * DK + cw + 4 * j4, dk);
            else store4<float>(a.ws_dk + ((b * T_ + t0 + s) * a.H + h) * DK + cw + 4 * j4, dk);
        }
    }
    // boundary term rowsum(S1 * dS1) per channel cw + 4j4 + e
    sd += __shfl_xor(sd, 16, 64);
    sd += __shfl_xor(sd, 32, 64);
    float bnd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) bnd[e] = dec[e] * __shfl(sd, 4 * j4 + e, 64) + row_sum16(bsum[e]);

    // ---- gate gradient
    if constexpr (VEC) {
        T* dgo = (T*)a.dg + ((b * T_ + t0) * a.H + h) * DK + cw + 4 * j4;
        // strong-gate chunks: dg[r] = (suffix of x from r, within r's document) + (sum of
        // k * (carried part of dk) over the rows before r) + [no reset] decay rowsum(S0 * dS1),
        // the same sum as the suffix form with every cancelling pair left out (the
        // rows before r reach dS1 only through token r's gate; z is 0 outside the
        // chunk's last document); bnd holds the decay term alone then (bsum is 0)
        float zp[4][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float zc[4] = {0.f, 0.f, 0.f, 0.f}, zo[4] = {0.f, 0.f, 0.f, 0.f};
            if (strong) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) zc[rt] = z[rt][e];
                rows_excl_prefix(zc, zo);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) zp[rt][e] = zo[rt];
        }
        if (ck.first_reset == C) {
            // no reset in this chunk: suffix sums over the 16 rows of a tile (lanes),
            // then across tiles, starting from the boundary term
            float carry[4] = {bnd[0], bnd[1], bnd[2], bnd[3]};
#pragma unroll
            for (int rt = 3; rt >= 0; --rt) {
                float dg[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = row_suffix16(x[rt][e]);
                    dg[e] = y + carry[e] + zp[rt][e];
                    carry[e] += __shfl(y, 0, 16);
                }
                const int r = 16 * rt + i16;
                if (r < nvalid) store4<T>(dgo + (int64_t)r * a.H * DK, dg);
            }
        } else {
            // documents inside the chunk: serial segmented suffix sum per channel in LDS
            __syncthreads();  // the scratch takes the place of g and dA
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                *reinterpret_cast<f32x4*>(sX + (16 * rt + i16) * PE + 16 * w + 4 * j4) =
                    f32x4{x[rt][0], x[rt][1], x[rt][2], x[rt][3]};
            if (i16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.sBnd[w][4 * j4 + e] = bnd[e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (j4 == 0) {
                const int cl = 16 * w + i16;
                float run = sm.sBnd[w][i16];
                for (int r = C - 1; r >= 0; --r) {
                    float val = 0.f;
                    if (r < nvalid) {
                        if (r < nvalid - 1 && ck.doc[r + 1] != ck.doc[r]) run = 0.f;
                        run += sX[r * PE + cl];
                        const bool reset = r > 0 ? ck.doc[r] != ck.doc[r - 1] : ck.doc[0] != 0;
                        val = reset ? 0.f : run;
                    }
                    sX[r * PE + cl] = val;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r = 16 * rt + i16;
                const f32x4 v = *reinterpret_cast<const f32x4*>(sX + r * PE + 16 * w + 4 * j4);
                const bool reset = r > 0 ? ck.doc[r] != ck.doc[r - 1] : ck.doc[0] != 0;
                float dg[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) dg[e] = v[e] + (reset ? 0.f : zp[rt][e]);
                if (r < nvalid) store4<T>(dgo + (int64_t)r * a.H * DK, dg);
            }
        }
    } else {
        // scalar gate: partial sums over this workgroup's channels; a finisher adds slices
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            float y = x[rt][0] + x[rt][1] + x[rt][2] + x[rt][3];
            y += __shfl_xor(y, 16, 64);
            y += __shfl_xor(y, 32, 64);
            if (j4 == 0) sm.sXs[w][16 * rt + i16] = y;
        }
        float bb = bnd[0] + bnd[1] + bnd[2] + bnd[3];
        bb += __shfl_xor(bb, 16, 64);
        bb += __shfl_xor(bb, 32, 64);
        if (l == 0) sm.sBs[w] = bb;
        __syncthreads();
        if (w == 0) {
            const int r = l;
            const float tot = sm.sXs[0][r] + sm.sXs[1][r] + sm.sXs[2][r] + sm.sXs[3][r];
            if (r < nvalid) a.ws_xs[(bh * Cfg::NQK + slice) * T_ + t0 + r] = tot;
            if (r == 0) a.ws_bnd[(bh * Cfg::NQK + slice) * NC + ci] = sm.sBs[0] + sm.sBs[1] + sm.sBs[2] + sm.sBs[3];
        }
    }
}

// ============================================================== V role
// dv computed transposed (rows = value columns n, columns = chunk rows s):
// lane (i, j) holds row s = 16st + i and the four columns n0s + 16w + 4j + e.
template <typename T, bool VEC, int DK, int DV>
__device__ void grad_v(const RevArgs& a, char* lds, GradSmall& sm, int64_t bh, int64_t ci, int slice) {
    using Cfg = GradCfg<T, VEC, DK, DV>;
    using M = Mma<T>;
    constexpr int PB = Cfg::PB, PK = Cfg::PK, PD = Cfg::PD;
    constexpr int NCT = DK / 16;
    constexpr int KS = M::KSTEP;
    constexpr int CPW = NCT / 4;

    T* sQ = reinterpret_cast<T*>(lds);
    T* sK = sQ + C * PK;
    T* sG = reinterpret_cast<T*>(lds + Cfg::V_OFF_G);   // vector gate only
    T* sdO = reinterpret_cast<T*>(lds + Cfg::V_OFF_DO); // [r][64 columns of the slice]
    T* sAT = reinterpret_cast<T*>(lds + Cfg::V_OFF_A);  // A transposed, [s][r]
    T* sdS = reinterpret_cast<T*>(lds + Cfg::V_OFF_DS); // [c][64 columns] (vector gate: after g is consumed)
    RevChunk& ck = sm.ck;

    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int n0s = slice * Cfg::NS;
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t t0 = ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t rs_qk = a.ld_qk, rs_do = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qrow = (const T*)a.q + (b * T_ + t0) * rs_qk + hq * DK;
    const T* krow = (const T*)a.k + (b * T_ + t0) * rs_qk + hq * DK;
    const T* dorow = (const T*)a.dO + (b * T_ + t0) * rs_do + h * DV + n0s;
    const T* grow = (const T*)a.g + (b * T_ + t0) * rs_g + (VEC ? h * DK : h);
    const T* dS1 = (const T*)a.ws_dS + (bh * NC + ci) * DK * DV + n0s;  // [c][n0s ..]

    TileRegs<T, DK> pq, pk, pg;
    TileRegs<T, 64> pdo;
    TileRegs<T, 64> pds[DK / 64];  // dS1 rows c = 64u .. 64u + 63, this slice's 64 columns
    RowRegs rr;
    pq.load(qrow, rs_qk, nvalid);
    pk.load(krow, rs_qk, nvalid);
    if constexpr (VEC) pg.load(grow, rs_g, nvalid);
    pdo.load(dorow, rs_do, nvalid);
#pragma unroll
    for (int u = 0; u < DK / 64; ++u) pds[u].load(dS1 + (int64_t)u * 64 * DV, DV, 64);
    if (w == 0) rr.load(grow, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    [[maybe_unused]] const TriOnes<T> tri;

    pq.store_rows(sQ, PK);
    pk.store_rows(sK, PK);
    if constexpr (VEC) {
        pg.store_rows(sG, PK);
        strong_flag_put(sm.sStrong, gate_regs_strong(pg));
    }
    pdo.store_rows(sdO, PB);
    if constexpr (!VEC) {
#pragma unroll
        for (int u = 0; u < DK / 64; ++u) pds[u].store_rows_b64(sdS + u * 64 * PD, PD);
    }
    if (w == 0) rev_chunk_info<T, VEC>(&ck, rr);
    __syncthreads();
    [[maybe_unused]] const bool strong = VEC && strong_flag_get<4>(sm.sStrong);

    // strong-gate chunks: this wave's score tiles (C layout: rows r = 16rt + 4j4 + e,
    // column s = 16st + i16) summed over the channel tiles from the prefixes themselves
    f32x4 Ax[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) Ax[u] = zero4();
    if constexpr (VEC) {
        f32x4 beta[CPW][4];
        gate_prefix_mfma<T, CPW, PK>(sG, tri, beta);
        if (strong) {
            // one channel tile of prefixes at a time, [row][16] in the place of A^T
            constexpr int PBB = 20;
            float* sBB = reinterpret_cast<float*>(sAT);
            static_assert(C * PBB * 4 <= Cfg::TILE64, "prefix block does not fit");
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                if (w == ct / CPW) {
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) sBB[(16 * rt + i16) * PBB + 4 * j4 + e] = beta[ct % CPW][rt][e];
                }
                __syncthreads();
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const int ti = w + 4 * u;
                    if (ti >= 10) continue;
                    const int rt = score_tile_rt(ti), st = score_tile_st(ti);
                    const int s = 16 * st + i16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * rt + 4 * j4 + e;
                        if (s <= r && ck.doc[s] == ck.doc[r])
                            Ax[u][e] = exact_dot<T>(sQ + r * PK + 16 * ct, sK + s * PK + 16 * ct,
                                                    sBB + r * PBB, sBB + s * PBB, 16, Ax[u][e]);
                    }
                }
                __syncthreads();
            }
        }
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int c4 = 16 * (CPW * w + cc) + 4 * j4;
            float m[4], Gam[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m[e] = strong ? 0.f : __shfl(beta[cc][1][e], 16 * j4 + 15, 64);
                Gam[e] = __shfl(beta[cc][3][e], 16 * j4 + 15, 64);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r = 16 * rt + i16;
                Vec4<T> qv = Vec4<T>::load(sQ + r * PK + c4);
                Vec4<T> kv = Vec4<T>::load(sK + r * PK + c4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float E = __expf(beta[cc][rt][e] - m[e]);
                    // (strong: k exp(Gamma - beta) itself, the operand of the dv update term)
                    const float Ei = strong ? __expf(Gam[e] - beta[cc][rt][e]) : __builtin_amdgcn_rcpf(E);
                    qv.set(e, qv.get(e) * E);
                    kv.set(e, kv.get(e) * Ei);
                }
                qv.store(sQ + r * PK + c4);
                kv.store(sK + r * PK + c4);
            }
            if (i16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.sEGm[c4 + e] = strong ? 1.f : __expf(Gam[e] - m[e]);
        }
        __syncthreads();
        // dS1 rows scaled by exp(Gamma - m) of their channel, so that KA dS1' = KU dS1
#pragma unroll
        for (int u = 0; u < DK / 64; ++u) pds[u].scale_rows(&sm.sEGm[64 * u]);
#pragma unroll
        for (int u = 0; u < DK / 64; ++u) pds[u].store_rows_b64(sdS + u * 64 * PD, PD);
    }

    // ---- A = QA KA^T on the lower tiles (+ two zero upper tiles), transposed: sAT[s][r]
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int ti = w + 4 * u;
        const int rt = score_tile_rt(ti);
        const int st = score_tile_st(ti);
        f32x4 acc = Ax[u];
        if (ti < 10 && !strong) {
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KS)
                acc = M::mma(frag_ld<T, PK, 1>(sQ, 16 * rt, k0), frag_ld<T, PK, 1>(sK, 16 * st, k0), acc);
        }
        store_masked_T<T, VEC, PB>(sAT, ck, rt, st, ti < 10, acc);
    }
    __syncthreads();

    // ---- dv^T = dO^T A + [last doc] dS1'^T KA^T (rows n, columns s)
    T* dvo = (T*)a.dv + (b * T_ + t0) * a.ld_dv + h * DV + n0s + 16 * w + 4 * j4;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        f32x4 a1 = zero4(), a2 = zero4();
        const int kbeg = (16 * st / KS) * KS;
#pragma unroll
        for (int k0 = kbeg; k0 < C; k0 += KS)
            a1 = M::mma(frag_col<T, PB, false>(sdO, 16 * w, k0), frag_ld<T, PB, 1>(sAT, 16 * st, k0), a1);
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KS)
            a2 = M::mma(frag_col<T, PD, false>(sdS, 16 * w, k0), frag_ld<T, PK, 1>(sK, 16 * st, k0), a2);
        const int s = 16 * st + i16;
        const float fu = ck.fu[s];
        float dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dv[e] = a1[e] + fu * a2[e];
        if (s < nvalid) store4<T>(dvo + (int64_t)s * a.ld_dv, dv);
    }
}

template <typename T, bool VEC, int DK, int DV>
__global__ __launch_bounds__(NT) void k_grad(const RevArgs a) {
    put_stamp(a.stamp_out, a.stamp_val);  // the states the passes before this one found or stored
    using Cfg = GradCfg<T, VEC, DK, DV>;
    __shared__ __attribute__((aligned(16))) char lds[Cfg::BYTES];
    __shared__ GradSmall sm;
    constexpr int PER = Cfg::NQK + Cfg::NVR;
    const int64_t NC = (a.T + C - 1) / C;
    // block -> (b, h, chunk, role); the roles of one chunk are adjacent (one XCD)
    const int64_t L = xcd_logical_block(a.B * a.H * NC * PER);
    const int role = (int)(L % PER);
    const int64_t ci = (L / PER) % NC;
    const int64_t bh = L / PER / NC;
    if (role < Cfg::NQK) grad_qk<T, VEC, DK, DV>(a, lds, sm, bh, ci, role);
    else grad_v<T, VEC, DK, DV>(a, lds, sm, bh, ci, role - Cfg::NQK);
}

// Scalar gate: dg[u] = sum_{t >= u, same doc} x[t] + [u in last doc] bnd, with x and bnd
// summed over the key-channel slices; 0 at reset tokens.  One wave per (b, h, chunk).
__global__ __launch_bounds__(64) void k_dg_scalar(const RevArgs a, int nslices, float* dgo_f32,
                                                  bf16* dgo_bf16) {
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t ci = blockIdx.x % NC, bh = blockIdx.x / NC;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t t0 = ci * C;
    const int r = threadIdx.x;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t t = t0 + r;
    int reset = 0;
    if (a.seg != nullptr && r < nvalid && t > 0) reset = a.seg[b * T_ + t] != a.seg[b * T_ + t - 1];
    float x = 0.f, bnd = 0.f;
    for (int s = 0; s < nslices; ++s) {
        if (r < nvalid) x += a.ws_xs[(bh * nslices + s) * T_ + t];
        bnd += a.ws_bnd[(bh * nslices + s) * NC + ci];
    }
    // segmented suffix scan over the chunk: documents end where the next row resets
    const int doc = wave_incl_scan_i(reset);
    float run = (r < nvalid ? x : 0.f) + ((r == nvalid - 1) ? bnd : 0.f);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_down(run, d, 64);
        const int dd = __shfl_down(doc, d, 64);
        if (r + d < 64 && dd == doc) run += y;
    }
    if (r < nvalid) {
        const float val = reset ? 0.f : run;
        const int64_t o = (b * T_ + t) * a.H + h;
        if (dgo_f32) dgo_f32[o] = val;
        else dgo_bf16[o] = (bf16)val;
    }
}

hipError_t launch_dg_scalar(const RevArgs& a, int nslices, bool bf16_out, hipStream_t st) {
    const int64_t NC = (a.T + C - 1) / C;
    hipLaunchKernelGGL(k_dg_scalar, dim3((unsigned)(a.B * a.H * NC)), dim3(64), 0, st, a, nslices,
                       bf16_out ? nullptr : (float*)a.dg, bf16_out ? (bf16*)a.dg : nullptr);
    return hipGetLastError();
}

template <typename T, bool VEC, int DK, int DV>
hipError_t launch_grad(const RevArgs& a, hipStream_t st) {
    // bf16 heads of 128 x 128: one eight-wave workgroup per chunk (every input loaded
    // once); the scalar gate's are walked instead (launch_grad8_walk), never sent here
    if constexpr (sizeof(T) == 2 && DK == 128 && DV == 128) {
        if constexpr (VEC) return launch_grad8(a, st);
        else return hipErrorInvalidValue;
    }
    // fp32, scalar gate, 128 x 128: fp32 products as three bf16 matrix-core products
    if constexpr (sizeof(T) == 4 && !VEC && DK == 128 && DV == 128) return launch_grad_f32s(a, st);
    using Cfg = GradCfg<T, VEC, DK, DV>;
    const int64_t NC = (a.T + C - 1) / C;
    const int64_t grid = a.B * a.H * NC * (Cfg::NQK + Cfg::NVR);
    hipLaunchKernelGGL((k_grad<T, VEC, DK, DV>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || VEC) return e;
    return launch_dg_scalar(a, Cfg::NQK, sizeof(T) == 2, st);
}

#define GLA_INST_GRAD(T, VEC, DK, DV) \
    template hipError_t launch_grad<T, VEC, DK, DV>(const RevArgs&, hipStream_t);
#define GLA_INST_GRAD_D(T, VEC)                                       \
    GLA_INST_GRAD(T, VEC, 64, 64) GLA_INST_GRAD(T, VEC, 64, 128)      \
    GLA_INST_GRAD(T, VEC, 128, 64) GLA_INST_GRAD(T, VEC, 128, 128)
GLA_INST_GRAD_D(float, false)
GLA_INST_GRAD_D(float, true)
GLA_INST_GRAD_D(bf16, false)
GLA_INST_GRAD_D(bf16, true)

}  // namespace gla
