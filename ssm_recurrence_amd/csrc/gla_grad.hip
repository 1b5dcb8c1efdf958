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
// Two kinds of workgroups per chunk:
//   QK: 64 key channels, each wave 16 of them: dq, dk and dg (the suffix sums
//       stay inside one wave); the state and its gradient come straight from
//       memory in the register layouts the products want;
//   V:  64 value columns, each wave 16 of them: dv.
#include "gla_bwd.hpp"
#include "gla_common.hpp"
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
    static constexpr bool STAGE = sizeof(T) == 2;  // bf16 outputs go through LDS to row stores
    static constexpr int max_(int a, int b) { return a > b ? a : b; }

    // QK role: q, k (, g) slices and dA; then dO and v.  After the products the
    // dO / v region holds the staged outputs and the g / dA region the fp32 dg scratch.
    static constexpr int TILE64 = C * PB * ES;
    static constexpr int QK_OFF_G = 2 * TILE64;
    static constexpr int QK_OFF_DA = QK_OFF_G + (VEC ? TILE64 : 0);
    static constexpr int QK_OFF_DO = QK_OFF_DA + TILE64;
    static constexpr int QK_REGION = max_(2 * C * PV * ES, STAGE ? (2 + (VEC ? 1 : 0)) * TILE64 : 0);
    static constexpr int QK_BYTES = QK_OFF_DO + QK_REGION;
    static_assert(!VEC || 2 * TILE64 >= C * PE * 4, "dg scratch does not fit");

    // V role: q, k (, g) for all channels, the dO slice and A; the dS1 slice takes the
    // place of g once g is consumed when it fits there.  Staged dv reuses q.
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
    float sM[128], sEm[128], sEGm[128];   // vector gate: per-channel m, exp(m), exp(Gamma - m)
    float sDecay[128];
    float sXs[4][C];                       // scalar gate: per-wave partial sums
    float sBs[4];
};

// out[rt][e] = base[(16rt + 4j + e) * P + col0 + i] for lane (i, j): the values of
// a natural [row][col] tile at the C-layout positions of this wave's column tile.
template <typename T, int P>
__device__ __forceinline__ void col_vals(const T* base, int col0, float (&out)[4][4]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const bf16x8 f = frag_col<T, P, true>(base, col0, 32 * p);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[2 * p][e] = (float)f[e];
                out[2 * p + 1][e] = (float)f[4 + e];
            }
        }
    } else {
        const int l = lane_id();
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[rt][e] = to_f32(base[(16 * rt + 4 * (l >> 4) + e) * P + col0 + (l & 15)]);
    }
}

// ============================================================== QK role
template <typename T, bool VEC, int DK, int DV>
__device__ void grad_qk(const RevArgs& a, char* lds, GradSmall& sm, int64_t bh, int64_t ci, int slice) {
    using Cfg = GradCfg<T, VEC, DK, DV>;
    using M = Mma<T>;
    constexpr int PB = Cfg::PB, PV = Cfg::PV, PE = Cfg::PE;
    constexpr int NNT = DV / 16;
    constexpr int KS = M::KSTEP;

    T* sQ = reinterpret_cast<T*>(lds);
    T* sK = sQ + C * PB;
    T* sG = reinterpret_cast<T*>(lds + Cfg::QK_OFF_G);    // vector gate only
    T* sdA = reinterpret_cast<T*>(lds + Cfg::QK_OFF_DA);  // [r][s]
    T* sdO = reinterpret_cast<T*>(lds + Cfg::QK_OFF_DO);
    T* sV = sdO + C * PV;
    float* sX = reinterpret_cast<float*>(lds + Cfg::QK_OFF_G);  // dg scratch, after the products
    T* sOq = sdO;                                                // staged outputs, after the products
    T* sOk = sOq + C * PB;
    T* sOg = sOk + C * PB;
    RevChunk& ck = sm.ck;

    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int cs0 = slice * Cfg::CS;
    const int cl = 16 * w + i16;  // this lane's channel within the slice
    const int c = cs0 + cl;       // ... within the head
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t t0 = ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t rs_qk = a.Hqk * DK, rs_v = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qrow = (const T*)a.q + (b * T_ + t0) * rs_qk + hq * DK + cs0;
    const T* krow = (const T*)a.k + (b * T_ + t0) * rs_qk + hq * DK + cs0;
    const T* vrow = (const T*)a.v + (b * T_ + t0) * rs_v + h * DV;
    const T* dorow = (const T*)a.dO + (b * T_ + t0) * rs_v + h * DV;
    const T* grow = (const T*)a.g + (b * T_ + t0) * rs_g + (VEC ? h * DK + cs0 : h);
    const T* S0 = (const T*)a.ws_S + ((bh * (NC + 1) + ci) * DK + c) * DV;  // row c of S0
    const T* dS1 = (const T*)a.ws_dS + ((bh * NC + ci) * DK + c) * DV;     // row c of dS1

    // ---- loads: the chunk's tiles, then this lane's rows of S0 and dS1
    TileRegs<T, 64> pq, pk, pg;
    TileRegs<T, DV> pv, pdo;
    RowRegs rr;
    pq.load(qrow, rs_qk, nvalid);
    pk.load(krow, rs_qk, nvalid);
    if constexpr (VEC) pg.load(grow, rs_g, nvalid);
    pv.load(vrow, rs_v, nvalid);
    pdo.load(dorow, rs_v, nvalid);
    if (w == 0) rr.load(grow, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    // S0 as B operands of dO S0^T (k = n): lane (i, j) holds S0[c][k0 + j*KPL + e]
    typename M::frag s0f[DV / KS];
#pragma unroll
    for (int kk = 0; kk < DV / KS; ++kk) {
        if constexpr (M::KPL == 1) s0f[kk] = S0[kk * KS + j4];
        else s0f[kk] = *reinterpret_cast<const bf16x8*>(S0 + kk * KS + 8 * j4);
    }
    // dS1^T in C layout (lane c, rows n = 16nt + 4*j4 + e), and the matching S0 values
    Vec4<T> dsr[NNT], s0r[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
        dsr[nt] = Vec4<T>::load(dS1 + 16 * nt + 4 * j4);
        s0r[nt] = Vec4<T>::load(S0 + 16 * nt + 4 * j4);
    }

    pq.store_rows(sQ, PB);
    pk.store_rows(sK, PB);
    if constexpr (VEC) pg.store_rows(sG, PB);
    pv.store_rows(sV, PV);
    pdo.store_rows(sdO, PV);
    if (w == 0) rev_chunk_info<T, VEC>(&ck, rr);

    f32x4 dSt[NNT];
    float sd = 0.f;  // this lane's part of rowsum(S0 * dS1) for channel c
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dSt[nt][e] = dsr[nt].get(e);
            sd += s0r[nt].get(e) * dSt[nt][e];
        }
    __syncthreads();
    const int first_reset = ck.first_reset, last_reset = ck.last_reset;

    if constexpr (VEC) {
        // gate prefix on the matrix cores; q, k scaled in place to QA = q exp(beta - m),
        // KA = k exp(m - beta) with m the prefix at row 31 (factored exponent)
        f32x4 beta[1][4];
        gate_prefix_mfma<T, 1, PB>(sG, beta);
        const int c4 = 16 * w + 4 * j4;  // this lane's 4 channels (slice-local)
        float m[4], Gam[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[e] = __shfl(beta[0][1][e], 16 * j4 + 15, 64);
            Gam[e] = __shfl(beta[0][3][e], 16 * j4 + 15, 64);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int r = 16 * rt + i16;
            Vec4<T> qv = Vec4<T>::load(sQ + r * PB + c4);
            Vec4<T> kv = Vec4<T>::load(sK + r * PB + c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float E = __expf(beta[0][rt][e] - m[e]);
                qv.set(e, qv.get(e) * E);
                kv.set(e, kv.get(e) * __builtin_amdgcn_rcpf(E));
            }
            qv.store(sQ + r * PB + c4);
            kv.store(sK + r * PB + c4);
        }
        if (i16 == 0)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sm.sM[c4 + e] = m[e];
                sm.sEm[c4 + e] = __expf(m[e]);
                sm.sEGm[c4 + e] = __expf(Gam[e] - m[e]);
                sm.sDecay[c4 + e] = last_reset >= 0 ? 0.f : __expf(Gam[e]);
            }
    }

    // ---- dA = dO v^T on the 10 lower tiles (+ the two upper tiles a 32-wide k step reads)
    for (int ti = w; ti < 12; ti += 4) {
        const int rt = ti < 10 ? (ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3) : (ti == 10 ? 0 : 2);
        const int st = ti < 10 ? ti - rt * (rt + 1) / 2 : (ti == 10 ? 1 : 3);
        f32x4 acc = zero4();
        if (ti < 10) {
#pragma unroll
            for (int n0 = 0; n0 < DV; n0 += KS)
                acc = M::mma(frag_ld<T, PV, 1>(sdO, 16 * rt, n0), frag_ld<T, PV, 1>(sV, 16 * st, n0), acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * j4 + e, s = 16 * st + i16;
            float x = 0.f;
            if (ti < 10 && s <= r && ck.doc[s] == ck.doc[r]) {
                x = acc[e];
                if constexpr (!VEC) x *= __expf(ck.beta[r] - ck.beta[s]);
            }
            sdA[r * PB + s] = from_f32<T>(x);
        }
    }
    __syncthreads();

    // ---- exp(beta - m) at this lane's output positions (rows 16rt + 4*j4 + e,
    // channel cl): the prefix once more, as L G, in the layout of dq and dk
    f32x4 Ex[4];
    if constexpr (VEC) {
        const float mc = sm.sM[cl];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc = zero4();
            const int r = 16 * rt + i16;
#pragma unroll
            for (int k0 = 0; k0 < ((16 * (rt + 1) + KS - 1) / KS) * KS; k0 += KS) {
                typename M::frag lt;
#pragma unroll
                for (int e = 0; e < M::KPL; ++e) M::set(lt, e, k0 + j4 * M::KPL + e <= r ? 1.f : 0.f);
                acc = M::mma(lt, frag_col<T, PB, false>(sG, 16 * w, k0), acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Ex[rt][e] = __expf(acc[e] - mc);
        }
    }

    // ---- dq (before the exp(beta - m) factor: dqp), x = QA*dqp = q*dq
    const float em = VEC ? sm.sEm[cl] : 1.f, egm = VEC ? sm.sEGm[cl] : 1.f;
    float x[4][4], dqv[4][4], dkv[4][4];
    {
        float qa[4][4];
        col_vals<T, PB>(sQ, 16 * w, qa);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 a1 = zero4(), a2 = zero4();
            const int kend = ((16 * (rt + 1) + KS - 1) / KS) * KS;
#pragma unroll
            for (int k0 = 0; k0 < kend; k0 += KS)
                a1 = M::mma(frag_ld<T, PB, 1>(sdA, 16 * rt, k0), frag_col<T, PB, false>(sK, 16 * w, k0), a1);
#pragma unroll
            for (int kk = 0; kk < DV / KS; ++kk)
                a2 = M::mma(frag_ld<T, PV, 1>(sdO, 16 * rt, kk * KS), s0f[kk], a2);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * j4 + e;
                const float dqp = a1[e] + ck.fq[r] * em * a2[e];
                x[rt][e] = qa[rt][e] * dqp;
                dqv[rt][e] = VEC ? Ex[rt][e] * dqp : dqp;
            }
        }
    }
    // ---- dk (dkp before the exp(m - beta) factor), x -= KA*dkp; the boundary sum
    float bs = 0.f;  // this lane's part of sum_s KU[s][c] (v dS1^T)[s][c]
    {
        float ka[4][4];
        col_vals<T, PB>(sK, 16 * w, ka);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 a1 = zero4(), a2 = zero4();
            const int kbeg = (16 * st / KS) * KS;
#pragma unroll
            for (int k0 = kbeg; k0 < C; k0 += KS)
                a1 = M::mma(frag_col<T, PB, false>(sdA, 16 * st, k0), frag_col<T, PB, false>(sQ, 16 * w, k0), a1);
            if constexpr (M::KPL == 1) {
#pragma unroll
                for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub)
                        a2 = M::mma(frag_ld_ctile<T, PV, 1>(sV, 16 * st, 16 * nt, sub),
                                    frag_from_acc<T>(dSt[nt], dSt[nt], sub), a2);
            } else {
#pragma unroll
                for (int p = 0; p < NNT / 2; ++p)
                    a2 = M::mma(frag_ld_ctile<T, PV, 1>(sV, 16 * st, 32 * p, 0),
                                frag_from_acc<T>(dSt[2 * p], dSt[2 * p + 1], 0), a2);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * st + 4 * j4 + e;
                const float inter = ck.fu[s] * egm * a2[e];
                const float dkp = a1[e] + inter;
                x[st][e] -= ka[st][e] * dkp;
                bs += ka[st][e] * inter;
                dkv[st][e] = VEC ? dkp * __builtin_amdgcn_rcpf(Ex[st][e]) : dkp;
            }
        }
    }
    // boundary term rowsum(S1 * dS1) for channel c (sum over the four lane groups)
    sd += __shfl_xor(sd, 16, 64);
    sd += __shfl_xor(sd, 32, 64);
    bs += __shfl_xor(bs, 16, 64);
    bs += __shfl_xor(bs, 32, 64);
    const float bnd = (VEC ? sm.sDecay[cl] : ck.decay) * sd + bs;
    __syncthreads();  // every wave is done with dO, v, g and dA: their LDS is reused below

    // ---- outputs dq, dk: staged for row stores (bf16, unshared q/k) or stored directly
    const bool staged = Cfg::STAGE && G == 1;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * j4 + e;
            if (staged) {
                sOq[r * PB + cl] = from_f32<T>(dqv[rt][e]);
                sOk[r * PB + cl] = from_f32<T>(dkv[rt][e]);
            } else if (r < nvalid) {
                if (G == 1) {
                    const int64_t o = ((b * T_ + t0 + r) * a.Hqk + hq) * DK + c;
                    ((T*)a.dq)[o] = from_f32<T>(dqv[rt][e]);
                    ((T*)a.dk)[o] = from_f32<T>(dkv[rt][e]);
                } else {
                    const int64_t o = ((b * T_ + t0 + r) * a.H + h) * DK + c;
                    a.ws_dq[o] = dqv[rt][e];
                    a.ws_dk[o] = dkv[rt][e];
                }
            }
        }

    // ---- gate gradient
    if constexpr (VEC) {
        T* dgo = (T*)a.dg;
        auto put_dg = [&](int r, float val) {
            if constexpr (Cfg::STAGE) sOg[r * PB + cl] = from_f32<T>(val);
            else if (r < nvalid) dgo[((b * T_ + t0 + r) * a.H + h) * DK + c] = from_f32<T>(val);
        };
        if (first_reset == C) {
            // no reset in this chunk: suffix sums in-lane over e, across the four
            // lane groups of a channel, and across row tiles
            float carry = bnd;
#pragma unroll
            for (int rt = 3; rt >= 0; --rt) {
                float suf[4];
                suf[3] = x[rt][3];
                suf[2] = suf[3] + x[rt][2];
                suf[1] = suf[2] + x[rt][1];
                suf[0] = suf[1] + x[rt][0];
                float tot[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) tot[jj] = __shfl(suf[0], 16 * jj + i16, 64);
                float above = carry;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) above += jj > j4 ? tot[jj] : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) put_dg(16 * rt + 4 * j4 + e, above + suf[e]);
                carry += tot[0] + tot[1] + tot[2] + tot[3];
            }
        } else {
            // documents inside the chunk: serial segmented suffix sum per channel
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) sX[(16 * rt + 4 * j4 + e) * PE + cl] = x[rt][e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (j4 == 0) {
                float run = bnd;
                for (int r = C - 1; r >= 0; --r) {
                    if (r >= nvalid) { put_dg(r, 0.f); continue; }
                    if (r < nvalid - 1 && ck.doc[r + 1] != ck.doc[r]) run = 0.f;
                    run += sX[r * PE + cl];
                    const bool reset = r > 0 ? ck.doc[r] != ck.doc[r - 1] : ck.doc[0] != 0;
                    put_dg(r, reset ? 0.f : run);
                }
            }
        }
    } else {
        // scalar gate: partial sums over this workgroup's channels; a finisher adds slices
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = x[rt][e];
#pragma unroll
                for (int d = 1; d < 16; d <<= 1) y += __shfl_xor(y, d, 64);
                if (i16 == 0) sm.sXs[w][16 * rt + 4 * j4 + e] = y;
            }
        float bb = bnd;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) bb += __shfl_xor(bb, d, 64);
        if (l == 0) sm.sBs[w] = bb;
    }
    __syncthreads();

    // ---- row stores of the staged tiles; scalar-gate partial sums
    if (staged) {
        constexpr int VPR = 64 * (int)sizeof(T) / 16;  // 16-byte vectors per 64-channel row
        for (int idx = threadIdx.x; idx < C * VPR; idx += NT) {
            const int r = idx / VPR, cv = (idx % VPR) * (16 / (int)sizeof(T));
            if (r >= nvalid) continue;
            const int64_t o = ((b * T_ + t0 + r) * a.Hqk + hq) * DK + cs0 + cv;
            *reinterpret_cast<i32x4*>((T*)a.dq + o) = *reinterpret_cast<const i32x4*>(sOq + r * PB + cv);
            *reinterpret_cast<i32x4*>((T*)a.dk + o) = *reinterpret_cast<const i32x4*>(sOk + r * PB + cv);
        }
    }
    if constexpr (VEC && Cfg::STAGE) {
        constexpr int VPR = 64 * (int)sizeof(T) / 16;
        for (int idx = threadIdx.x; idx < C * VPR; idx += NT) {
            const int r = idx / VPR, cv = (idx % VPR) * (16 / (int)sizeof(T));
            if (r >= nvalid) continue;
            const int64_t o = ((b * T_ + t0 + r) * a.H + h) * DK + cs0 + cv;
            *reinterpret_cast<i32x4*>((T*)a.dg + o) = *reinterpret_cast<const i32x4*>(sOg + r * PB + cv);
        }
    }
    if constexpr (!VEC) {
        if (w == 0) {
            const int r = l;
            const float tot = sm.sXs[0][r] + sm.sXs[1][r] + sm.sXs[2][r] + sm.sXs[3][r];
            if (r < nvalid) a.ws_xs[(bh * Cfg::NQK + slice) * T_ + t0 + r] = tot;
            if (r == 0) a.ws_bnd[(bh * Cfg::NQK + slice) * NC + ci] = sm.sBs[0] + sm.sBs[1] + sm.sBs[2] + sm.sBs[3];
        }
    }
}

// ============================================================== V role
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
    T* sA = reinterpret_cast<T*>(lds + Cfg::V_OFF_A);   // [r][s]
    T* sdS = reinterpret_cast<T*>(lds + Cfg::V_OFF_DS); // [c][64 columns], after g is consumed
    T* sOv = sQ;                                         // staged dv [s][column], after A
    RevChunk& ck = sm.ck;

    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int n0s = slice * Cfg::NS;
    const int n = n0s + 16 * w + i16;  // this lane's value column
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t t0 = ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    const int64_t rs_qk = a.Hqk * DK, rs_v = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qrow = (const T*)a.q + (b * T_ + t0) * rs_qk + hq * DK;
    const T* krow = (const T*)a.k + (b * T_ + t0) * rs_qk + hq * DK;
    const T* dorow = (const T*)a.dO + (b * T_ + t0) * rs_v + h * DV + n0s;
    const T* grow = (const T*)a.g + (b * T_ + t0) * rs_g + (VEC ? h * DK : h);
    const T* dS1 = (const T*)a.ws_dS + (bh * NC + ci) * DK * DV + n0s;  // [c][n0s ..]

    TileRegs<T, DK> pq, pk, pg;
    TileRegs<T, 64> pdo;
    TileRegs<T, 64> pds[DK / 64];  // dS1 rows c = 64u .. 64u + 63, this slice's 64 columns
    RowRegs rr;
    pq.load(qrow, rs_qk, nvalid);
    pk.load(krow, rs_qk, nvalid);
    if constexpr (VEC) pg.load(grow, rs_g, nvalid);
    pdo.load(dorow, rs_v, nvalid);
#pragma unroll
    for (int u = 0; u < DK / 64; ++u) pds[u].load(dS1 + (int64_t)u * 64 * DV, DV, 64);
    if (w == 0) rr.load(grow, rs_g, a.seg, b, T_, t0, nvalid, !VEC);

    pq.store_rows(sQ, PK);
    pk.store_rows(sK, PK);
    if constexpr (VEC) pg.store_rows(sG, PK);
    pdo.store_rows(sdO, PB);
    if constexpr (!Cfg::DS_IN_G) {
#pragma unroll
        for (int u = 0; u < DK / 64; ++u) pds[u].store_rows_b64(sdS + u * 64 * PD, PD);
    }
    if (w == 0) rev_chunk_info<T, VEC>(&ck, rr);
    __syncthreads();

    if constexpr (VEC) {
        f32x4 beta[CPW][4];
        gate_prefix_mfma<T, CPW, PK>(sG, beta);
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int c4 = 16 * (CPW * w + cc) + 4 * j4;
            float m[4], Gam[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m[e] = __shfl(beta[cc][1][e], 16 * j4 + 15, 64);
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
                    qv.set(e, qv.get(e) * E);
                    kv.set(e, kv.get(e) * __builtin_amdgcn_rcpf(E));
                }
                qv.store(sQ + r * PK + c4);
                kv.store(sK + r * PK + c4);
            }
            if (i16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.sEGm[c4 + e] = __expf(Gam[e] - m[e]);
        }
        __syncthreads();
        if constexpr (Cfg::DS_IN_G) {
#pragma unroll
            for (int u = 0; u < DK / 64; ++u) pds[u].store_rows_b64(sdS + u * 64 * PD, PD);
        }
    }

    // ---- A = QA KA^T on the lower tiles (+ two zero upper tiles) -> sA[r][s]
    for (int ti = w; ti < 12; ti += 4) {
        const int rt = ti < 10 ? (ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3) : (ti == 10 ? 0 : 2);
        const int st = ti < 10 ? ti - rt * (rt + 1) / 2 : (ti == 10 ? 1 : 3);
        f32x4 acc = zero4();
        if (ti < 10) {
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KS)
                acc = M::mma(frag_ld<T, PK, 1>(sQ, 16 * rt, k0), frag_ld<T, PK, 1>(sK, 16 * st, k0), acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * j4 + e, s = 16 * st + i16;
            float x = 0.f;
            if (ti < 10 && s <= r && ck.doc[s] == ck.doc[r]) {
                x = acc[e];
                if constexpr (!VEC) x *= __expf(ck.beta[r] - ck.beta[s]);
            }
            sA[r * PB + s] = from_f32<T>(x);
        }
    }
    __syncthreads();

    // ---- dv[s][n] for this wave's 16 columns: A^T dO + [s in last doc] KU dS1,
    // KU = KA exp(Gamma - m) (vector gate) or k (scalar gate: fu carries the factor)
    T* dvo = (T*)a.dv;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        f32x4 a1 = zero4(), a2 = zero4();
        const int kbeg = (16 * st / KS) * KS;
#pragma unroll
        for (int k0 = kbeg; k0 < C; k0 += KS)
            a1 = M::mma(frag_col<T, PB, false>(sA, 16 * st, k0), frag_col<T, PB, false>(sdO, 16 * w, k0), a1);
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KS) {
            typename M::frag ku = frag_ld<T, PK, 1>(sK, 16 * st, k0);
            if constexpr (VEC) frag_scale_k<T>(ku, k0, [&](int cc) { return sm.sEGm[cc]; });
            a2 = M::mma(ku, frag_col<T, PD, false>(sdS, 16 * w, k0), a2);
        }
        // dv^T tile: lane n, rows s = 16st + 4*j4 + e
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 16 * st + 4 * j4 + e;
            const float val = a1[e] + ck.fu[s] * a2[e];
            if constexpr (Cfg::STAGE) sOv[s * PB + 16 * w + i16] = from_f32<T>(val);
            else if (s < nvalid) dvo[((b * T_ + t0 + s) * a.H + h) * DV + n] = from_f32<T>(val);
        }
    }
    if constexpr (Cfg::STAGE) {
        __syncthreads();
        constexpr int VPR = 64 * (int)sizeof(T) / 16;
        for (int idx = threadIdx.x; idx < C * VPR; idx += NT) {
            const int r = idx / VPR, cv = (idx % VPR) * (16 / (int)sizeof(T));
            if (r >= nvalid) continue;
            const int64_t o = ((b * T_ + t0 + r) * a.H + h) * DV + n0s + cv;
            *reinterpret_cast<i32x4*>(dvo + o) = *reinterpret_cast<const i32x4*>(sOv + r * PB + cv);
        }
    }
}

template <typename T, bool VEC, int DK, int DV>
__global__ __launch_bounds__(NT) void k_grad(const RevArgs a) {
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
