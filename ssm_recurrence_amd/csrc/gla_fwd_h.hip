// gla_fwd_h.hip -- fused chunk-parallel forward for bf16 heads with 128 key
// channels and 128 value columns (gfx950): one 8-wave workgroup per
// (b, h, piece) holding the whole fp32 state.
//
// The recurrence, the per-chunk algebra and the split of the sequence into
// pieces are those of gla_fwd.hip (FLAT page, "FLAT: Flash Linear Attention on
// TPUs", Linear Attention > Forward Recurrence, chunkwise form; Pallas Kernels >
// Forward Kernels, the fused block-recurrent kernel; Pallas Kernels > Mamba-2 /
// Gated Linear Attention for the two gates).  The work split is that of the
// fp32 whole-head kernel (gla_fwd_f32s.hip): wave w owns the state's column
// tile w for all 128 channels, so the readout S^T q takes its S^T operand from
// the wave's accumulators and no workgroup repeats another's q k^T.  Per chunk:
//   stage    q, k, v, v restricted to the chunk's last document (scaled by
//            exp(Gamma - beta_s) for the scalar gate), and the vector gate tile;
//   (vector gate) per-channel prefix on the matrix cores, wave w for channel
//            tile w: QA = q exp(beta - m), KA = k exp(m - beta) in place, with
//            m = beta at row 31, and the channel factors exp(Gamma),
//            exp(Gamma - m), exp(m); a chunk with a gate too strong for that
//            factored form (gla_exact.hpp) gets its scores from the prefixes
//            directly and takes m = 0 for the readout and update operands;
//   scores   masked score tiles spread over the waves (scalar gate: times
//            exp(beta_r - beta_s)), stored to LDS; the readout of each wave's
//            columns; the state update of each wave's columns;
//   output   the intra-chunk product and o = O + [first doc] (exp(beta_r)) R.
// Operand reads are issued one step ahead of the products that consume them.
#include "gla_common.hpp"
#include "gla_exact.hpp"
#include "gla_kernels.hpp"
#include "gla_tile.hpp"

namespace gla {

namespace {

constexpr int DK = 128, DV = 128, KS = 32, NTH = 512;
// row pitches (bf16 elements) for the LDS reads each tile serves on gfx950
// (measured): ctile 8-byte reads want 12 mod 64, transposed reads any pitch but
// 12 mod 128, 16-byte row reads 16 mod 64.  q and k are read in ctile order only
// (any channel order common to both gives the same scores); k also transposed.
constexpr int PQ = DK + 12;   // q (QA)
constexpr int PKH = DK + 20;  // k (KA)
constexpr int PH = DK + 8;    // v, last-document v, gate tile
constexpr int PA = C + 16;    // scores [r][s]
constexpr int PO = DV + 8;    // output rows, written to HBM a whole row at a time
constexpr int PBF = DK + 4;   // fp32 prefixes of a chunk (strong-gate chunks only)

template <bool VEC>
struct FwdHLds {
    bf16 sQ[C * PQ];
    bf16 sK[C * PKH];
    bf16 sV[C * PH];
    bf16 sVu[C * PH];
    bf16 sA[C * PA];
    // the output rows; in a strong-gate chunk first the fp32 gate prefixes, which
    // are dead before the output is assembled
    union {
        bf16 sO[C * PO];
        float sBF[VEC ? C * PBF : 4];
    };
    bf16 sG[VEC ? C * PH : 8];
    bf16 sKU[VEC ? C * PH : 8];    // vector gate: k exp(Gamma - beta), the update's operand
    alignas(16) int sDoc[C];
    alignas(16) float sBeta[C];
    alignas(16) float sDecay[VEC ? DK : 4];
    alignas(16) float sEm[VEC ? DK : 4];
    alignas(16) int sStrong[8];
    int sAnyReset;
};

template <bool VEC>
__global__ __launch_bounds__(NTH) void k_fwd_h(const PassArgs a) {
    using M = Mma<bf16>;
    __shared__ __attribute__((aligned(16))) FwdHLds<VEC> sm;
    put_stamp(a.stamp_out, a.expect);  // the states this kernel stores

    const int64_t P = a.P;
    const int64_t L = xcd_logical_block(a.B * a.H * P);
    const int64_t piece = L % P;
    const int64_t bh = L / P;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t G = a.H / a.Hqk, hq = h / G;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t cbeg = piece * a.PL;
    const int64_t cend = (cbeg + a.PL < NC) ? cbeg + a.PL : NC;

    const int64_t rs_qk = a.ld_qk, rs_v = a.ld_v, rs_o = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const bf16* qbase = (const bf16*)a.q + b * T_ * rs_qk + hq * DK;
    const bf16* kbase = (const bf16*)a.k + b * T_ * rs_qk + hq * DK;
    const bf16* vbase = (const bf16*)a.v + b * T_ * rs_v + h * DV;
    const bf16* gbase = (const bf16*)a.g + b * T_ * rs_g + (VEC ? h * DK : h);
    bf16* obase = (bf16*)a.o + b * T_ * rs_o + h * DV;
    // a chunk's output is assembled in LDS and written out at the next chunk's start
    // with 16-byte stores of whole rows (each wave holds 16 columns of every row)
    auto write_out = [&](int64_t t0, int nvalid) {
        using TR = TileRegs<bf16, DV, NTH>;
#pragma unroll
        for (int i = 0; i < TR::NVEC; ++i) {
            const int idx = threadIdx.x + i * NTH;
            const int row = idx / TR::VPR, cv = (idx % TR::VPR) * TR::VE;
            if (row < nvalid)
                *reinterpret_cast<i32x4*>(obase + (t0 + row) * rs_o + cv) =
                    *reinterpret_cast<const i32x4*>(sm.sO + row * PO + cv);
        }
    };

    // state tiles ct = 0..7 of column tile w: lane holds S[16ct + 4j4 + e][16w + i16]
    f32x4 S[DK / 16];
    load_entry_state_128(a, bh, piece, w, j4, i16, S);

    TileRegs<bf16, DK, NTH> pq, pk, pv;
    TileRegs<bf16, VEC ? DK : 8, NTH> pg;
    RowRegs rr;
    auto prefetch = [&](int64_t t0) {
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;
        pq.load(qbase + t0 * rs_qk, rs_qk, nvalid);
        pk.load(kbase + t0 * rs_qk, rs_qk, nvalid);
        pv.load(vbase + t0 * rs_v, rs_v, nvalid);
        if constexpr (VEC) pg.load(gbase + t0 * rs_g, rs_g, nvalid);
        rr.load(gbase + t0 * rs_g, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    };
    prefetch(cbeg * C);

    for (int64_t it = cbeg; it < cend; ++it) {
        const int64_t t0 = it * C;
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;

        // ---- chunk structure, in every wave (lane = row)
        const int doc = wave_incl_scan_i(rr.reset());
        const uint64_t msk = __ballot(rr.reset());
        const int first_reset = msk ? __builtin_ctzll(msk) : C;
        const int last_reset = msk ? 63 - __builtin_clzll(msk) : -1;
        float fu, fq, decay = 0.f;
        if constexpr (!VEC) {
            const float beta = wave_incl_scan(rr.g());
            const float Gam = __shfl(beta, 63, 64);
            fu = l >= last_reset ? __expf(Gam - beta) : 0.f;
            fq = l < first_reset ? __expf(beta) : 0.f;
            decay = msk ? 0.f : __expf(Gam);
            if (w == 0) sm.sBeta[l] = beta;
        } else {
            fu = l >= last_reset ? 1.f : 0.f;
            fq = l < first_reset ? 1.f : 0.f;
        }
        if (w == 0) {
            sm.sDoc[l] = doc;
            if (l == 0) sm.sAnyReset = msk != 0;
        }

        // ---- staging; the previous chunk's output
        if (it > cbeg) write_out(t0 - C, C);
        pq.store_rows_b64(sm.sQ, PQ);  // rows of q and k are 8-byte aligned only
        pk.store_rows_b64(sm.sK, PKH);
        pv.store_rows(sm.sV, PH);
        if constexpr (VEC) {
            pg.store_rows(sm.sG, PH);
            strong_flag_put(sm.sStrong, gate_regs_strong(pg));
        }
        {
            using TR = TileRegs<bf16, DV, NTH>;
            static_assert(TR::NV_TOT % NTH == 0, "");
#pragma unroll
            for (int i = 0; i < TR::NVEC; ++i) {
                const int idx = threadIdx.x + i * NTH;
                const int row = idx / TR::VPR, cv = (idx % TR::VPR) * TR::VE;
                const float f = __shfl(fu, row, 64);
                bf16x8 x = __builtin_bit_cast(bf16x8, pv.get(i));
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * f);
                *reinterpret_cast<bf16x8*>(sm.sVu + row * PH + cv) = x;
            }
        }
        // (for the backward) the state entering this chunk, stored while the staged
        // tiles' registers are free and before the next chunk's loads are issued
        if (!VEC && a.save_S) store_state_128<bf16>((bf16*)a.save_S + (bh * (NC + 1) + it) * DK * DV, S);
        if (it + 1 < cend) prefetch(t0 + C);
        __syncthreads();
        [[maybe_unused]] const bool strong = VEC && strong_flag_get<8>(sm.sStrong);

        if constexpr (VEC) {
            // ---- per-channel prefix for channel tile w; QA, KA in place; channel factors
            f32x4 beta[1][4];
            {
                const TriOnes<bf16> tri;  // built here: live only for the prefix
                gate_prefix_mfma<bf16, 1, PH>(sm.sG, tri, beta);
            }
            const bool any_reset = sm.sAnyReset != 0;
            const int c0 = 16 * w + 4 * j4;  // this lane's 4 channels
            float m[4], Gam[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m[e] = __shfl(beta[0][1][e], 16 * j4 + 15, 64);    // row 31
                Gam[e] = __shfl(beta[0][3][e], 16 * j4 + 15, 64);  // row 63
            }
            if (strong) {
                // scores from the prefixes themselves (raw q, k still in LDS); then the
                // readout operand q exp(beta) with the unscaled state (m = 0) and the update
                // operand k exp(Gamma - beta)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sm.sBF[(16 * rt + i16) * PBF + c0 + e] = beta[0][rt][e];
                __syncthreads();
                exact_scores<bf16, DK, NTH, PQ, PKH, PBF, PA, false>(sm.sA, sm.sQ, sm.sK, sm.sBF, sm.sDoc);
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = 0.f;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int r = 16 * rt + i16;
                    Vec4<bf16> qv = Vec4<bf16>::load(sm.sQ + r * PQ + c0);
                    const Vec4<bf16> kv = Vec4<bf16>::load(sm.sK + r * PKH + c0);
                    Vec4<bf16> ku;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qv.set(e, qv.get(e) * __expf(beta[0][rt][e]));
                        ku.set(e, kv.get(e) * __expf(Gam[e] - beta[0][rt][e]));
                    }
                    qv.store(sm.sQ + r * PQ + c0);
                    ku.store(sm.sKU + r * PH + c0);
                }
            } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r = 16 * rt + i16;
                Vec4<bf16> qv = Vec4<bf16>::load(sm.sQ + r * PQ + c0);
                Vec4<bf16> kv = Vec4<bf16>::load(sm.sK + r * PKH + c0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float E = __expf(beta[0][rt][e] - m[e]);
                    qv.set(e, qv.get(e) * E);
                    kv.set(e, kv.get(e) * __builtin_amdgcn_rcpf(E));
                }
                qv.store(sm.sQ + r * PQ + c0);
                kv.store(sm.sK + r * PKH + c0);
                Vec4<bf16> ku;
#pragma unroll
                for (int e = 0; e < 4; ++e) ku.set(e, kv.get(e) * __expf(Gam[e] - m[e]));
                ku.store(sm.sKU + r * PH + c0);
            }
            }
            if (i16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.sDecay[c0 + e] = any_reset ? 0.f : __expf(Gam[e]);
                    sm.sEm[c0 + e] = __expf(m[e]);
                }
            }
            __syncthreads();
        }

        // ---- masked score tiles, computed transposed (rows s, column r), stored sA[r][s];
        // tiles 10 and 11 are the zero tiles (0,1) and (2,3) that a 32-wide step reads
        for (int ti = w; ti < (strong ? 0 : 12); ti += 8) {
            const int rt = score_tile_rt(ti);
            const int st = score_tile_st(ti);
            f32x4 acc = zero4();
            if (ti < 10) {
                bf16x8 ka = frag_ld_ctile<bf16, PKH, 1>(sm.sK, 16 * st, 0, 0);
                bf16x8 qa = frag_ld_ctile<bf16, PQ, 1>(sm.sQ, 16 * rt, 0, 0);
#pragma unroll
                for (int kk = 0; kk < DK / KS; ++kk) {
                    bf16x8 kb, qb;
                    if (kk + 1 < DK / KS) {
                        kb = frag_ld_ctile<bf16, PKH, 1>(sm.sK, 16 * st, (kk + 1) * KS, 0);
                        qb = frag_ld_ctile<bf16, PQ, 1>(sm.sQ, 16 * rt, (kk + 1) * KS, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    acc = M::mma(ka, qa, acc);
                    __builtin_amdgcn_sched_barrier(0);
                    ka = kb;
                    qa = qb;
                }
            }
            const int r = 16 * rt + i16, s0 = 16 * st + 4 * j4;
            const int dr = sm.sDoc[r];
            const int4 d4 = *reinterpret_cast<const int4*>(&sm.sDoc[s0]);
            const int ds[4] = {d4.x, d4.y, d4.z, d4.w};
            float br = 0.f, bs[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (!VEC) {
                br = sm.sBeta[r];
                const float4 b4 = *reinterpret_cast<const float4*>(&sm.sBeta[s0]);
                bs[0] = b4.x; bs[1] = b4.y; bs[2] = b4.z; bs[3] = b4.w;
            }
            Vec4<bf16> x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = 0.f;
                if (ti < 10 && s0 + e <= r && ds[e] == dr) {
                    y = acc[e];
                    if constexpr (!VEC) y *= __expf(br - bs[e]);
                }
                x.set(e, y);
            }
            x.store(sm.sA + r * PA + s0);
        }

        // ---- readout R^T[n][r] = sum_c S'[c][n] q'[r][c] for this wave's columns
        // (scalar gate: S' = S, q' = q; vector gate: S' = S exp(m_c), q' = QA); the
        // S'^T operand, k = channel in ctile order, comes from the accumulators
        f32x4 R[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) R[rt] = zero4();
        {
            // (vector gate: the state's channel decays are applied here too, once
            // the readout operand is taken)
            auto sfrag = [&](int p) {
                if constexpr (VEC) {
                    const float4 e0 = *reinterpret_cast<const float4*>(&sm.sEm[32 * p + 4 * j4]);
                    const float4 e1 = *reinterpret_cast<const float4*>(&sm.sEm[32 * p + 16 + 4 * j4]);
                    const float4 d0 = *reinterpret_cast<const float4*>(&sm.sDecay[32 * p + 4 * j4]);
                    const float4 d1 = *reinterpret_cast<const float4*>(&sm.sDecay[32 * p + 16 + 4 * j4]);
                    f32x4 x0 = S[2 * p], x1 = S[2 * p + 1];
                    x0[0] *= e0.x; x0[1] *= e0.y; x0[2] *= e0.z; x0[3] *= e0.w;
                    x1[0] *= e1.x; x1[1] *= e1.y; x1[2] *= e1.z; x1[3] *= e1.w;
                    S[2 * p][0] *= d0.x; S[2 * p][1] *= d0.y; S[2 * p][2] *= d0.z; S[2 * p][3] *= d0.w;
                    S[2 * p + 1][0] *= d1.x; S[2 * p + 1][1] *= d1.y; S[2 * p + 1][2] *= d1.z; S[2 * p + 1][3] *= d1.w;
                    return frag_from_acc<bf16>(x0, x1, 0);
                } else {
                    return frag_from_acc<bf16>(S[2 * p], S[2 * p + 1], 0);
                }
            };
            bf16x8 qa = frag_ld_ctile<bf16, PQ, 1>(sm.sQ, 0, 0, 0);
            bf16x8 sf = sfrag(0);
#pragma unroll
            for (int idx = 0; idx < 16; ++idx) {
                const int p = idx >> 2, rt = idx & 3;
                bf16x8 qb;
                if (idx + 1 < 16) qb = frag_ld_ctile<bf16, PQ, 1>(sm.sQ, 16 * ((idx + 1) & 3), KS * ((idx + 1) >> 2), 0);
                __builtin_amdgcn_sched_barrier(0);
                R[rt] = M::mma(sf, qa, R[rt]);
                __builtin_amdgcn_sched_barrier(0);
                if (rt == 3 && p < 3) sf = sfrag(p + 1);
                qa = qb;
            }
        }

        // ---- state update of this wave's columns: S = decay S + KU^T v_last, KU = k
        // (scalar gate; v_last carries exp(Gamma - beta_s)) or k exp(Gamma - beta) (vector gate)
        {
            bf16x8 vu[C / KS];
#pragma unroll
            for (int k = 0; k < C / KS; ++k) vu[k] = frag_col<bf16, PH, false>(sm.sVu, 16 * w, k * KS);
            // (the vector gate's decays were applied with the readout)
            if constexpr (!VEC) {
#pragma unroll
                for (int ct = 0; ct < DK / 16; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[ct][e] *= decay;
            }
            const bf16* sKu = VEC ? sm.sKU : sm.sK;
            constexpr int PU = VEC ? PH : PKH;
            bf16x8 ka = frag_col<bf16, PU, false>(sKu, 0, 0);
#pragma unroll
            for (int idx = 0; idx < 16; ++idx) {
                const int k = idx >> 3, ct = idx & 7;
                bf16x8 kb;
                if (idx + 1 < 16) kb = frag_col<bf16, PU, false>(sKu, 16 * ((idx + 1) & 7), KS * ((idx + 1) >> 3));
                __builtin_amdgcn_sched_barrier(0);
                S[ct] = M::mma(ka, vu[k], S[ct]);
                __builtin_amdgcn_sched_barrier(0);
                ka = kb;
            }
        }
        __syncthreads();

        // ---- intra-chunk product and output: o^T[n][r] = sum_s v[s][n] A[r][s] + fq_r R^T[n][r]
        {
            bf16x8 vt[C / KS];
#pragma unroll
            for (int p = 0; p < C / KS; ++p) vt[p] = frag_col<bf16, PH, false>(sm.sV, 16 * w, p * KS);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 O = zero4();
#pragma unroll
                for (int p = 0; p <= rt / 2; ++p) O = M::mma(vt[p], frag_ld<bf16, PA, 1>(sm.sA, 16 * rt, p * KS), O);
                const int r = 16 * rt + i16;
                const float fr = __shfl(fq, r, 64);
                Vec4<bf16> out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out.set(e, O[e] + fr * R[rt][e]);
                out.store(sm.sO + r * PO + 16 * w + 4 * j4);
            }
        }
        __syncthreads();
    }
    if (cend > cbeg) {
        const int64_t tl = (cend - 1) * C;
        write_out(tl, T_ - tl < C ? (int)(T_ - tl) : C);
    }

    if (!VEC && a.save_S && piece == P - 1) store_state_128<bf16>((bf16*)a.save_S + (bh * (NC + 1) + NC) * DK * DV, S);
    if (a.hT && piece == P - 1) {
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * ct + 4 * j4 + e, n = 16 * w + i16;
                a.hT[(bh * DK + c) * DV + n] = S[ct][e];
            }
        }
    }
}

}  // namespace

template <bool VEC>
hipError_t launch_fwd_h(const PassArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_fwd_h<VEC>, dim3((unsigned)(a.B * a.H * a.P)), dim3(NTH), 0, st, a);
    return hipGetLastError();
}

template hipError_t launch_fwd_h<false>(const PassArgs&, hipStream_t);
template hipError_t launch_fwd_h<true>(const PassArgs&, hipStream_t);

}  // namespace gla
