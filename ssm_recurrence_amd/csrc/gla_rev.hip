// gla_rev.hip -- reverse pass of the backward (gfx950): walks the chunks last
// to first carrying the state gradient dS on chip, and produces dq, dk, dv,
// the log-gate gradient and dh0 (FLAT page, "FLAT: Flash Linear Attention on
// TPUs", Linear Attention > Backward Recurrence and Pallas Kernels > Backward
// Kernels: the gradient kernel visits chunks last to first with the state
// gradient in fast memory; dK and dV use the state gradient from later chunks,
// so the chunk's own contribution is added afterwards; the log-gate gradient
// is a suffix sum of q*dq - k*dk within the chunk plus a boundary term from
// the carried state, kept in fp32).
//
// Per chunk (beta the chunk-local log-gate prefix, Gamma its total, S0 the
// state entering the chunk from the state pass, S1 the state at its end, dS
// the gradient of S1), with dA = dO v^T masked to s <= r in one document:
//   dq[r] = sum_s dA[r][s] k[s] exp(beta_r - beta_s) + [r in first doc] exp(beta_r) (S0 dO[r])
//   dk[s] = sum_r dA[r][s] q[r] exp(beta_r - beta_s) + [s in last doc] exp(Gamma - beta_s) (dS v[s])
//   dv[s] = sum_r A[r][s] dO[r]                      + [s in last doc] dS^T (k[s] exp(Gamma - beta_s))
//   dg[u] = sum_{t >= u, same doc} (q*dq - k*dk)[t] + [u in last doc] rowsum(S1 * dS)   (0 at resets)
//   dS   <- [no reset] diag(exp Gamma) dS + sum_{r in first doc} (q[r] exp(beta_r)) dO[r]^T
//
// dq, dk and dg need sums over value columns; dv needs sums over key
// channels.  So one launch runs two kinds of workgroups per (b, h), each
// carrying its own slice of dS (the slices evolve independently):
//   QK: 64 key channels; each wave owns 16 of them, holding dS^T (rows n,
//       columns c) for all value columns, and computes dq, dk and dg for them
//       (so the suffix sums stay inside one wave);
//   V:  64 value columns; each wave owns 16, holding dS (rows c) for all key
//       channels, and computes dv and dh0 for them.
// Both recompute the shared per-chunk products (dA for QK, A for V).
#include "gla_common.hpp"
#include "gla_kernels.hpp"
#include "gla_tile.hpp"

namespace gla {

template <typename T, bool VEC, int DK, int DV>
struct RevCfg {
    static constexpr int CS = 64;                 // key channels per QK workgroup
    static constexpr int NS = 64;                 // value columns per V workgroup
    static constexpr int NQK = DK / CS, NVR = DV / NS;
    static constexpr int PB = Pitch16<T>::of(64);
    static constexpr int PK = Pitch16<T>::of(DK);
    static constexpr int PV = Pitch16<T>::of(DV);
    static constexpr int PE = 68;                 // fp32 [64][64] tiles
    // QK role
    // bf16: raw q, k copies (vector gate) and dq, dk, dg output tiles staged for row stores
    static constexpr bool STAGE_OUT = sizeof(T) == 2;
    static constexpr int QK_BYTES_NOV = (2 + (VEC ? 1 : 0)) * C * PB * (int)sizeof(T) +  // q k g slices
                                        2 * C * PV * (int)sizeof(T) +                   // dO, S0
                                        C * PB * (int)sizeof(T) +                      // dA
                                        (VEC ? C * PE * 4 : 0) +                       // E / x (vector gate)
                                        (STAGE_OUT ? (VEC ? 5 : 2) : 0) * C * PB * (int)sizeof(T);
    static constexpr bool V_LDS = QK_BYTES_NOV + C * PV * (int)sizeof(T) <= 150 * 1024;
    static constexpr int QK_BYTES = QK_BYTES_NOV + (V_LDS ? C * PV * (int)sizeof(T) : 0);
    // V role
    static constexpr int V_BYTES = (2 + (VEC ? 1 : 0)) * C * PK * (int)sizeof(T) +  // q k g
                                   (STAGE_OUT ? 3 : 2) * C * PB * (int)sizeof(T);   // dO slice, A, dv
    static constexpr int BYTES = QK_BYTES > V_BYTES ? QK_BYTES : V_BYTES;
};

// rows of a global T tensor as an operand fragment in ctile k order
// (lane i, k = k0 + 4j + e, k0 + 16 + 4j + e; f32: k0 + 4j + sub); zero past nvalid
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag glb_rows_ctile(const T* base, int64_t rs, int i0, int k0,
                                                                int sub, int nvalid) {
    const int l = lane_id();
    const int i = i0 + (l & 15), j = l >> 4;
    typename Mma<T>::frag f = Mma<T>::zero();
    if (i < nvalid) {
        const T* p = base + (int64_t)i * rs;
        if constexpr (Mma<T>::KPL == 1) {
            f = p[k0 + 4 * j + sub];
        } else {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + k0 + 4 * j);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + k0 + 16 + 4 * j);
            f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    return f;
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag glb_rows_nat(const T* base, int64_t rs, int i0, int k0,
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

// scale each k element of a fragment: element e has k = k0 + j*KPL + e
template <typename T, typename F>
__device__ __forceinline__ void frag_scale_k(typename Mma<T>::frag& f, int k0, F&& factor) {
    const int j = lane_id() >> 4;
#pragma unroll
    for (int e = 0; e < Mma<T>::KPL; ++e) {
        float x;
        if constexpr (Mma<T>::KPL == 1) x = to_f32(f); else x = to_f32(f[e]);
        Mma<T>::set(f, e, x * factor(k0 + j * Mma<T>::KPL + e));
    }
}
// same, for a fragment in ctile k order
template <typename T, typename F>
__device__ __forceinline__ void frag_scale_k_ctile(typename Mma<T>::frag& f, int k0, int sub, F&& factor) {
    const int j = lane_id() >> 4;
    if constexpr (Mma<T>::KPL == 1) {
        f = f * factor(k0 + 4 * j + sub);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = e < 4 ? k0 + 4 * j + e : k0 + 16 + 4 * j + (e - 4);
            f[e] = (bf16)((float)f[e] * factor(k));
        }
    }
}

// Chunk-level document data shared by both roles (wave 0 fills it).
struct RevChunk {
    int doc[C];
    float beta[C];   // scalar gate: chunk-local prefix
    float fq[C];     // readout rows: [r in first doc] (* exp(beta_r) for the scalar gate)
    float fu[C];     // update rows:  [s in last doc]  (* exp(Gamma - beta_s) for the scalar gate)
    float decay;     // scalar gate: exp(Gamma), 0 if the chunk has a reset
    int first_reset, last_reset;
};

template <typename T, bool VEC>
__device__ __forceinline__ void rev_chunk_info(RevChunk* ci, const RowRegs& rr) {
    const int r = lane_id();
    const int doc = wave_incl_scan_i(rr.reset);
    const uint64_t msk = __ballot(rr.reset);
    const int first_reset = msk ? __builtin_ctzll(msk) : C;
    const int last_reset = msk ? 63 - __builtin_clzll(msk) : -1;
    ci->doc[r] = doc;
    if (r == 0) {
        ci->first_reset = first_reset;
        ci->last_reset = last_reset;
    }
    if constexpr (!VEC) {
        const float beta = wave_incl_scan(rr.g);
        const float Gam = __shfl(beta, 63, 64);
        ci->beta[r] = beta;
        ci->fq[r] = r < first_reset ? __expf(beta) : 0.f;
        ci->fu[r] = r >= last_reset ? __expf(Gam - beta) : 0.f;
        if (r == 0) ci->decay = msk ? 0.f : __expf(Gam);
    } else {
        ci->fq[r] = r < first_reset ? 1.f : 0.f;
        ci->fu[r] = r >= last_reset ? 1.f : 0.f;
    }
}

// ============================================================== QK role
template <typename T, bool VEC, int DK, int DV>
__device__ void rev_qk(const RevArgs& a, char* lds, int64_t bh, int64_t piece, int slice) {
    using Cfg = RevCfg<T, VEC, DK, DV>;
    using M = Mma<T>;
    constexpr int PB = Cfg::PB, PV = Cfg::PV, PE = Cfg::PE;
    constexpr bool V_LDS = Cfg::V_LDS;
    constexpr int NNT = DV / 16;
    constexpr int KS = M::KSTEP;

    T* sQ = reinterpret_cast<T*>(lds);
    T* sK = sQ + C * PB;
    T* sG = sK + C * PB;                          // vector gate only
    T* sdO = sG + (VEC ? C * PB : 0);
    T* sS = sdO + C * PV;                         // state entering the chunk, [c][n]
    T* sdA = sS + C * PV;                         // [r][s]
    float* sE = reinterpret_cast<float*>(sdA + C * PB);  // exp(beta - m) [r][c]; later x
    T* sOq = reinterpret_cast<T*>(sE + (VEC ? C * PE : 0));  // staged dq, dk (, dg) tiles [r][c]
    T* sOk = sOq + (Cfg::STAGE_OUT ? C * PB : 0);
    T* sOg = sOk + (Cfg::STAGE_OUT ? C * PB : 0);
    T* sQr = sOg + (Cfg::STAGE_OUT && VEC ? C * PB : 0);  // raw q, k (vector gate)
    T* sKr = sQr + (Cfg::STAGE_OUT && VEC ? C * PB : 0);
    T* sV = sKr + (Cfg::STAGE_OUT && VEC ? C * PB : 0);   // when it fits
    __shared__ RevChunk ck;
    __shared__ float sEm[64], sEGm[64], sDecay[64];
    __shared__ float sXs[4][C];
    __shared__ float sBs[4];

    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int cs0 = slice * Cfg::CS;
    const int cl = 16 * w + i16;                  // this lane's channel within the slice
    const int c = cs0 + cl;                       // ... within the head
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t P = a.P;
    const int64_t cbeg = piece * a.PL;
    const int64_t cend = (cbeg + a.PL < NC) ? cbeg + a.PL : NC;
    // gradient of the state at the end of this piece: dhT for the last piece
    const float* dSend = P > 1 ? a.dS_out + (bh * P + piece) * DK * DV : (a.dhT ? a.dhT + bh * DK * DV : nullptr);

    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.g;
    const T* dO = (const T*)a.dO;
    const T* Sws = (const T*)a.ws_S;
    const int64_t rs_qk = a.Hqk * DK, rs_v = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qbase = q + b * T_ * rs_qk + hq * DK + cs0;
    const T* kbase = k + b * T_ * rs_qk + hq * DK + cs0;
    const T* vbase = v + b * T_ * rs_v + h * DV;
    const T* dobase = dO + b * T_ * rs_v + h * DV;
    const T* gbase = g + b * T_ * rs_g + (VEC ? h * DK + cs0 : h);

    // dS^T tiles (nt, channel tile w): lane c, rows n = 16nt + 4*j4 + e
    f32x4 dSt[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dSt[nt][e] = dSend ? dSend[c * DV + 16 * nt + 4 * j4 + e] : 0.f;

    // boundary term of the last chunk: rowsum(hT * dhT) for this channel
    auto rowsum_with = [&](auto Sget) {
        float acc = 0.f;
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += Sget(16 * nt + 4 * j4 + e) * dSt[nt][e];
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        return acc;
    };
    float bnd;
    {
        const T* Send = Sws + ((bh * (NC + 1) + cend) * DK + c) * DV;
        bnd = rowsum_with([&](int n) { return to_f32(Send[n]); });
    }

    TileRegs<T, 64> pq, pk, pg;
    TileRegs<T, DV> pv, pdo, ps;
    RowRegs rr;
    auto prefetch = [&](int64_t ci) {
        const int64_t t0 = ci * C;
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;
        pq.load(qbase + t0 * rs_qk, rs_qk, nvalid);
        pk.load(kbase + t0 * rs_qk, rs_qk, nvalid);
        if constexpr (VEC) pg.load(gbase + t0 * rs_g, rs_g, nvalid);
        if constexpr (V_LDS) pv.load(vbase + t0 * rs_v, rs_v, nvalid);
        pdo.load(dobase + t0 * rs_v, rs_v, nvalid);
        ps.load(Sws + ((bh * (NC + 1) + ci) * DK + cs0) * DV, DV, C);
        if (w == 0) rr.load(gbase + t0 * rs_g, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    };
    prefetch(cend - 1);

    for (int64_t ci = cend - 1; ci >= cbeg; --ci) {
        const int64_t t0 = ci * C;
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;

        pq.store_rows(sQ, PB);
        pk.store_rows(sK, PB);
        if constexpr (VEC) pg.store_rows(sG, PB);
        if constexpr (Cfg::STAGE_OUT && VEC) {
            pq.store_rows(sQr, PB);
            pk.store_rows(sKr, PB);
        }
        if constexpr (V_LDS) pv.store_rows(sV, PV);
        pdo.store_rows(sdO, PV);
        ps.store_rows(sS, PV);
        if (w == 0) rev_chunk_info<T, VEC>(&ck, rr);
        __syncthreads();
        if (ci > cbeg) prefetch(ci - 1);
        const int first_reset = ck.first_reset, last_reset = ck.last_reset;

        if constexpr (VEC) {
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
                f32x4 Ev;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float E = __expf(beta[0][rt][e] - m[e]);
                    Ev[e] = E;
                    qv.set(e, qv.get(e) * E);
                    kv.set(e, kv.get(e) * __builtin_amdgcn_rcpf(E));
                }
                qv.store(sQ + r * PB + c4);
                kv.store(sK + r * PB + c4);
                *reinterpret_cast<f32x4*>(sE + r * PE + c4) = Ev;
            }
            if (i16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sEm[c4 + e] = __expf(m[e]);
                    sEGm[c4 + e] = __expf(Gam[e] - m[e]);
                    sDecay[c4 + e] = last_reset >= 0 ? 0.f : __expf(Gam[e]);
                }
        }

        // ---- dA = dO v^T on the 10 lower tiles (+ the two upper tiles a 32-wide k step reads)
        {
            const T* vrow = vbase + t0 * rs_v;
            for (int ti = w; ti < 12; ti += 4) {
                const int rt = ti < 10 ? (ti < 1 ? 0 : ti < 3 ? 1 : ti < 6 ? 2 : 3) : (ti == 10 ? 0 : 2);
                const int st = ti < 10 ? ti - rt * (rt + 1) / 2 : (ti == 10 ? 1 : 3);
                f32x4 acc = zero4();
                if (ti < 10) {
#pragma unroll
                    for (int n0 = 0; n0 < DV; n0 += KS) {
                        typename M::frag vb;
                        if constexpr (V_LDS) vb = frag_ld<T, PV, 1>(sV, 16 * st, n0);
                        else vb = glb_rows_nat<T>(vrow, rs_v, 16 * st, n0, nvalid);
                        acc = M::mma(frag_ld<T, PV, 1>(sdO, 16 * rt, n0), vb, acc);
                    }
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
        }
        __syncthreads();

        // ---- dq, then dk, for this wave's 16 channels and all 64 rows; each is
        // folded into x = q*dq - k*dk (fp32, raw inputs) and written out at once,
        // so the two never occupy registers together
        const float em = VEC ? sEm[cl] : 1.f, egm = VEC ? sEGm[cl] : 1.f;
        const T* sQraw = (Cfg::STAGE_OUT && VEC) ? sQr : sQ;
        const T* sKraw = (Cfg::STAGE_OUT && VEC) ? sKr : sK;
        const bool staged = Cfg::STAGE_OUT && G == 1;
        auto raw_at = [&](const T* sraw, const T* gbase_qk, int r) -> float {
            if (VEC && !Cfg::STAGE_OUT)  // fp32 vector gate: raw values from memory
                return r < nvalid ? to_f32(gbase_qk[(t0 + r) * rs_qk + cl]) : 0.f;
            return to_f32(sraw[r * PB + cl]);
        };
        auto put_grad = [&](T* stile, void* dst, float* wsd, int r, float val) {
            if (staged) {
                stile[r * PB + cl] = from_f32<T>(val);
            } else if (r < nvalid) {
                if (G == 1) ((T*)dst)[((b * T_ + t0 + r) * a.Hqk + hq) * DK + c] = from_f32<T>(val);
                else wsd[((b * T_ + t0 + r) * a.H + h) * DK + c] = val;
            }
        };
        float x[4][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 a1 = zero4(), a2 = zero4();
            const int kend = ((16 * (rt + 1) + KS - 1) / KS) * KS;
            for (int k0 = 0; k0 < kend; k0 += KS)
                a1 = M::mma(frag_ld<T, PB, 1>(sdA, 16 * rt, k0), frag_col<T, PB, false>(sK, 16 * w, k0), a1);
#pragma unroll
            for (int n0 = 0; n0 < DV; n0 += KS)
                a2 = M::mma(frag_ld<T, PV, 1>(sdO, 16 * rt, n0), frag_ld<T, PV, 1>(sS, 16 * w, n0), a2);
            // C layout: lane = channel, rows r = 16rt + 4*j4 + e
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * j4 + e;
                float dq;
                if constexpr (VEC) dq = sE[r * PE + cl] * (a1[e] + ck.fq[r] * em * a2[e]);
                else dq = a1[e] + ck.fq[r] * a2[e];
                x[rt][e] = raw_at(sQraw, qbase, r) * dq;
                put_grad(sOq, a.dq, a.ws_dq, r, dq);
            }
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 a1 = zero4(), a2 = zero4();
            const int kbeg = (16 * st / KS) * KS;
            for (int k0 = kbeg; k0 < C; k0 += KS)
                a1 = M::mma(frag_col<T, PB, false>(sdA, 16 * st, k0), frag_col<T, PB, false>(sQ, 16 * w, k0), a1);
            const T* vrow = vbase + t0 * rs_v;
            if constexpr (M::KPL == 1) {
#pragma unroll
                for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub) {
                        typename M::frag va;
                        if constexpr (V_LDS) va = frag_ld_ctile<T, PV, 1>(sV, 16 * st, 16 * nt, sub);
                        else va = glb_rows_ctile<T>(vrow, rs_v, 16 * st, 16 * nt, sub, nvalid);
                        a2 = M::mma(va, frag_from_acc<T>(dSt[nt], dSt[nt], sub), a2);
                    }
            } else {
#pragma unroll
                for (int p = 0; p < NNT / 2; ++p) {
                    typename M::frag va;
                    if constexpr (V_LDS) va = frag_ld_ctile<T, PV, 1>(sV, 16 * st, 32 * p, 0);
                    else va = glb_rows_ctile<T>(vrow, rs_v, 16 * st, 32 * p, 0, nvalid);
                    a2 = M::mma(va, frag_from_acc<T>(dSt[2 * p], dSt[2 * p + 1], 0), a2);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * st + 4 * j4 + e;
                float dk;
                if constexpr (VEC) dk = __builtin_amdgcn_rcpf(sE[s * PE + cl]) * (a1[e] + ck.fu[s] * egm * a2[e]);
                else dk = a1[e] + ck.fu[s] * a2[e];
                x[st][e] -= raw_at(sKraw, kbase, s) * dk;
                put_grad(sOk, a.dk, a.ws_dk, s, dk);
            }
        }

        // ---- dS^T <- decay dS^T + dO^T QR  (rows n, this wave's channels), in place
        {
            const float dec = VEC ? sDecay[cl] : ck.decay;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) dSt[nt][e] *= dec;
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += KS) {
                typename M::frag qr = frag_col<T, PB, false>(sQ, 16 * w, k0);
                frag_scale_k<T>(qr, k0, [&](int r) { return ck.fq[r] * em; });
#pragma unroll
                for (int nt = 0; nt < NNT; ++nt)
                    dSt[nt] = M::mma(frag_col<T, PV, false>(sdO, 16 * nt, k0), qr, dSt[nt]);
            }
        }
        // boundary term of the previous chunk: rowsum(S0 * dS) with dS the new gradient
        const float bnd_chunk = bnd;
        bnd = rowsum_with([&](int n) { return to_f32(sS[cl * PV + n]); });

        // ---- gate gradient
        if constexpr (VEC) {
            T* dgo = (T*)a.dg;
            auto put_dg = [&](int r, float val) {
                if constexpr (Cfg::STAGE_OUT) sOg[r * PB + cl] = from_f32<T>(val);
                else if (r < nvalid) dgo[((b * T_ + t0 + r) * a.H + h) * DK + c] = from_f32<T>(val);
            };
            if (first_reset == C) {
                // no reset in this chunk: suffix sums in-lane over e, across the four
                // lane groups of a channel, and across row tiles
                float carry = bnd_chunk;
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
                float* sX = sE;  // this wave's columns only
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sX[(16 * rt + 4 * j4 + e) * PE + cl] = x[rt][e];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (j4 == 0) {
                    float run = bnd_chunk;
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
                    if (i16 == 0) sXs[w][16 * rt + 4 * j4 + e] = y;
                }
            float bs = bnd_chunk;
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) bs += __shfl_xor(bs, d, 64);
            if (l == 0) sBs[w] = bs;
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
        if constexpr (VEC && Cfg::STAGE_OUT) {
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
                const float tot = sXs[0][r] + sXs[1][r] + sXs[2][r] + sXs[3][r];
                if (r < nvalid) a.ws_xs[(bh * Cfg::NQK + slice) * T_ + t0 + r] = tot;
                if (r == 0)
                    a.ws_bnd[(bh * Cfg::NQK + slice) * NC + ci] = sBs[0] + sBs[1] + sBs[2] + sBs[3];
            }
        }
    }
}

// ============================================================== V role
template <typename T, bool VEC, int DK, int DV>
__device__ void rev_v(const RevArgs& a, char* lds, int64_t bh, int64_t piece, int slice) {
    using Cfg = RevCfg<T, VEC, DK, DV>;
    using M = Mma<T>;
    constexpr int PB = Cfg::PB, PK = Cfg::PK;
    constexpr int NCT = DK / 16;
    constexpr int KS = M::KSTEP;
    constexpr int CPW = NCT / 4;

    T* sQ = reinterpret_cast<T*>(lds);
    T* sK = sQ + C * PK;
    T* sG = sK + C * PK;
    T* sdO = sG + (VEC ? C * PK : 0);             // [r][64 columns of the slice]
    T* sA = sdO + C * PB;                          // [r][s]
    T* sOv = sA + C * PB;                          // staged dv tile [s][column] (bf16)
    __shared__ RevChunk ck;
    __shared__ float sEm[DK], sEGm[DK], sDecay[DK];

    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int n0s = slice * Cfg::NS;
    const int n = n0s + 16 * w + i16;             // this lane's value column
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t P = a.P;
    const int64_t cbeg = piece * a.PL;
    const int64_t cend = (cbeg + a.PL < NC) ? cbeg + a.PL : NC;
    // gradient of the state at the end of this piece: dhT for the last piece
    const float* dSend = P > 1 ? a.dS_out + (bh * P + piece) * DK * DV : (a.dhT ? a.dhT + bh * DK * DV : nullptr);

    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* g = (const T*)a.g;
    const T* dO = (const T*)a.dO;
    const int64_t rs_qk = a.Hqk * DK, rs_v = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const T* qbase = q + b * T_ * rs_qk + hq * DK;
    const T* kbase = k + b * T_ * rs_qk + hq * DK;
    const T* dobase = dO + b * T_ * rs_v + h * DV + n0s;
    const T* gbase = g + b * T_ * rs_g + (VEC ? h * DK : h);

    // dS tiles (ct, column tile w): lane n, rows c = 16ct + 4*j4 + e
    f32x4 dS[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dS[ct][e] = dSend ? dSend[(16 * ct + 4 * j4 + e) * DV + n] : 0.f;

    TileRegs<T, DK> pq, pk, pg;
    TileRegs<T, 64> pdo;
    RowRegs rr;
    auto prefetch = [&](int64_t ci) {
        const int64_t t0 = ci * C;
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;
        pq.load(qbase + t0 * rs_qk, rs_qk, nvalid);
        pk.load(kbase + t0 * rs_qk, rs_qk, nvalid);
        if constexpr (VEC) pg.load(gbase + t0 * rs_g, rs_g, nvalid);
        pdo.load(dobase + t0 * rs_v, rs_v, nvalid);
        if (w == 0) rr.load(gbase + t0 * rs_g, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    };
    prefetch(cend - 1);

    for (int64_t ci = cend - 1; ci >= cbeg; --ci) {
        const int64_t t0 = ci * C;
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;

        pq.store_rows(sQ, PK);
        pk.store_rows(sK, PK);
        if constexpr (VEC) pg.store_rows(sG, PK);
        pdo.store_rows(sdO, PB);
        if (w == 0) rev_chunk_info<T, VEC>(&ck, rr);
        __syncthreads();
        if (ci > cbeg) prefetch(ci - 1);
        const int last_reset = ck.last_reset;

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
                    for (int e = 0; e < 4; ++e) {
                        sEm[c4 + e] = __expf(m[e]);
                        sEGm[c4 + e] = __expf(Gam[e] - m[e]);
                        sDecay[c4 + e] = last_reset >= 0 ? 0.f : __expf(Gam[e]);
                    }
            }
            __syncthreads();
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

        // ---- dv[s][n] for this wave's 16 columns
        {
            T* dvo = (T*)a.dv;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                f32x4 a1 = zero4(), a2 = zero4();
                const int kbeg = (16 * st / KS) * KS;
                for (int k0 = kbeg; k0 < C; k0 += KS)
                    a1 = M::mma(frag_col<T, PB, false>(sA, 16 * st, k0), frag_col<T, PB, false>(sdO, 16 * w, k0), a1);
                if constexpr (M::KPL == 1) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int sub = 0; sub < 4; ++sub) {
                            typename M::frag ku = frag_ld_ctile<T, PK, 1>(sK, 16 * st, 16 * ct, sub);
                            if constexpr (VEC) frag_scale_k_ctile<T>(ku, 16 * ct, sub, [&](int cc) { return sEGm[cc]; });
                            a2 = M::mma(ku, frag_from_acc<T>(dS[ct], dS[ct], sub), a2);
                        }
                } else {
#pragma unroll
                    for (int p = 0; p < NCT / 2; ++p) {
                        typename M::frag ku = frag_ld_ctile<T, PK, 1>(sK, 16 * st, 32 * p, 0);
                        if constexpr (VEC) frag_scale_k_ctile<T>(ku, 32 * p, 0, [&](int cc) { return sEGm[cc]; });
                        a2 = M::mma(ku, frag_from_acc<T>(dS[2 * p], dS[2 * p + 1], 0), a2);
                    }
                }
                // dv^T tile: lane n, rows s = 16st + 4*j4 + e
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * st + 4 * j4 + e;
                    const float val = a1[e] + ck.fu[s] * a2[e];
                    if constexpr (Cfg::STAGE_OUT) sOv[s * PB + 16 * w + i16] = from_f32<T>(val);
                    else if (s < nvalid) dvo[((b * T_ + t0 + s) * a.H + h) * DV + n] = from_f32<T>(val);
                }
            }
        }

        // ---- dS <- decay dS + QR^T dO  (rows c, this wave's columns), in place
        {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) dS[ct][e] *= VEC ? sDecay[16 * ct + 4 * j4 + e] : ck.decay;
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += KS) {
                const typename M::frag dob = frag_col<T, PB, false>(sdO, 16 * w, k0);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    typename M::frag qr = frag_col<T, PK, false>(sQ, 16 * ct, k0);
                    const float emc = VEC ? sEm[16 * ct + i16] : 1.f;
                    frag_scale_k<T>(qr, k0, [&](int r) { return ck.fq[r] * emc; });
                    dS[ct] = M::mma(qr, dob, dS[ct]);
                }
            }
        }
        __syncthreads();
        if constexpr (Cfg::STAGE_OUT) {
            constexpr int VPR = 64 * (int)sizeof(T) / 16;
            for (int idx = threadIdx.x; idx < C * VPR; idx += NT) {
                const int r = idx / VPR, cv = (idx % VPR) * (16 / (int)sizeof(T));
                if (r >= nvalid) continue;
                const int64_t o = ((b * T_ + t0 + r) * a.H + h) * DV + n0s + cv;
                *reinterpret_cast<i32x4*>((T*)a.dv + o) = *reinterpret_cast<const i32x4*>(sOv + r * PB + cv);
            }
        }
    }
    if (a.dh0 && piece == 0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.dh0[(bh * DK + 16 * ct + 4 * j4 + e) * DV + n] = dS[ct][e];
    }
}

template <typename T, bool VEC, int DK, int DV>
__global__ __launch_bounds__(NT) void k_rev(const RevArgs a) {
    using Cfg = RevCfg<T, VEC, DK, DV>;
    __shared__ __attribute__((aligned(16))) char lds[Cfg::BYTES];
    constexpr int PER = Cfg::NQK + Cfg::NVR;
    // block -> (b, h, piece, role); the roles of one piece are adjacent (one XCD)
    const int64_t L = xcd_logical_block(a.B * a.H * a.P * PER);
    const int role = (int)(L % PER);
    const int64_t piece = (L / PER) % a.P;
    const int64_t bh = L / PER / a.P;
    if (role < Cfg::NQK) rev_qk<T, VEC, DK, DV>(a, lds, bh, piece, role);
    else rev_v<T, VEC, DK, DV>(a, lds, bh, piece, role - Cfg::NQK);
}

// Scalar gate: dg[u] = sum_{t >= u, same doc} x[t] + [u in last doc] bnd, with x and bnd
// summed over the key-channel slices; 0 at reset tokens.  One wave per (b, h, chunk).
__global__ __launch_bounds__(64) void k_dg_scalar_f32(const RevArgs a, int nslices, float* dgo_f32,
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
    // segmented suffix sum over the chunk: documents end where the next row resets
    const int doc = wave_incl_scan_i(reset);
    const int last_doc = __shfl(doc, nvalid - 1, 64);
    float run = (r < nvalid ? x : 0.f) + ((r == nvalid - 1) ? bnd : 0.f);
    // suffix scan within equal doc ids
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_down(run, d, 64);
        const int dd = __shfl_down(doc, d, 64);
        if (r + d < 64 && dd == doc) run += y;
    }
    (void)last_doc;
    if (r < nvalid) {
        const float val = reset ? 0.f : run;
        const int64_t o = (b * T_ + t) * a.H + h;
        if (dgo_f32) dgo_f32[o] = val;
        else dgo_bf16[o] = (bf16)val;
    }
}

template <typename T, bool VEC, int DK, int DV>
hipError_t launch_rev(const RevArgs& a, hipStream_t st) {
    using Cfg = RevCfg<T, VEC, DK, DV>;
    const int64_t grid = a.B * a.H * a.P * (Cfg::NQK + Cfg::NVR);
    hipLaunchKernelGGL((k_rev<T, VEC, DK, DV>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || VEC) return e;
    const int64_t NC = (a.T + C - 1) / C;
    hipLaunchKernelGGL(k_dg_scalar_f32, dim3((unsigned)(a.B * a.H * NC)), dim3(64), 0, st, a,
                       Cfg::NQK, sizeof(T) == 4 ? (float*)a.dg : nullptr,
                       sizeof(T) == 2 ? (bf16*)a.dg : nullptr);
    return hipGetLastError();
}

#define GLA_INST_REV(T, VEC, DK, DV) \
    template hipError_t launch_rev<T, VEC, DK, DV>(const RevArgs&, hipStream_t);
#define GLA_INST_REV_D(T, VEC)                                      \
    GLA_INST_REV(T, VEC, 64, 64) GLA_INST_REV(T, VEC, 64, 128)      \
    GLA_INST_REV(T, VEC, 128, 64) GLA_INST_REV(T, VEC, 128, 128)
GLA_INST_REV_D(float, false)
GLA_INST_REV_D(float, true)
GLA_INST_REV_D(bf16, false)
GLA_INST_REV_D(bf16, true)

}  // namespace gla
