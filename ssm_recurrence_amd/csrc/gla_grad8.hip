// gla_grad8.hip -- gradients for bf16 heads with 128 key channels and 128 value
// columns (gfx950), one workgroup of eight waves per chunk at a time: the vector
// gate one workgroup per (b, h, chunk); the scalar gate a reverse walk, one
// workgroup per (b, h, piece) carrying the state gradient from chunk to chunk.
//
// Same per-chunk mathematics as gla_grad.hip (FLAT page, "FLAT: Flash Linear
// Attention on TPUs", Linear Attention > Backward Recurrence): dq, dk and dg
// from the intra-chunk scores, the state entering the chunk and the state
// gradient at its end; dv likewise.  The difference is the work split.  On
// this device a compute unit pulls requested bytes at about the same rate
// whether they hit in L2 or not, so duplicate requests cost as much as HBM
// traffic; the two-role kernel asks for each chunk's q, k, g, v and dO two or
// three times.  Here one workgroup loads every input of its chunk once (about
// 144 KB: five 64 x 128 tiles, the state rows and the state-gradient rows) and
// its eight waves share the products:
//   phase 1  all tiles to LDS, S0 and dS1 rows of the wave's 16 channels to registers;
//   phase 2  gate prefix and the q, k scaling for the wave's 16 channels, the
//            scaled dS1 rows to LDS, dA tiles; then A tiles;
//   phase 3  dq, dk (and the log-gate gradient) for the wave's 16 key channels,
//            dv for its 16 value columns;
//   phase 4  (walk) the state gradient at the previous chunk's end.
// The scalar gate's log-gate gradient sums over all 128 channels, which are
// all in this workgroup, so it is finished here too.  A vector-gate chunk with a
// gate too strong for the factored form (gla_exact.hpp) forms A and the
// intra-chunk parts of dq and dk from the prefixes directly, and its
// carried-state terms from exp(beta) and exp(Gamma - beta).  In the walk the state
// gradient's rows come from LDS instead of HBM and no state gradient is stored.
#include "gla_bwd.hpp"
#include "gla_common.hpp"
#include "gla_exact.hpp"
#include "gla_kernels.hpp"
#include "gla_tile.hpp"

namespace gla {

typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;

template <bool VEC, bool WALK>
struct Grad8Cfg {
    using T = bf16;
    static constexpr int NW = 8, NTH = 64 * NW;
    static constexpr int DK = 128, DV = 128;
    // 16-byte row reads of bf16 tiles are free of bank conflicts at pitches of
    // 16 (mod 64) elements (measured on gfx950; 8 (mod 64) gives two-way conflicts)
    static constexpr int P = 128 + 16;             // [rows][128] tiles
    static constexpr int PB = 64 + 16;             // [64][64] score tiles
    static constexpr int PE = 132;                 // fp32 [64][128] dg scratch
    static constexpr int PF = 132;                 // fp32 [128][128] state gradient (walk)
    static constexpr int PBF = 132;                // fp32 [64][128] prefixes (strong-gate chunks)
    static constexpr int TILE = C * P * 2;
    static constexpr int OFF_Q = 0, OFF_K = TILE, OFF_G = 2 * TILE;
    static constexpr int OFF_V = OFF_G + (VEC ? TILE : 0);
    static constexpr int OFF_DO = OFF_V + TILE;
    static constexpr int OFF_DA = OFF_DO + TILE;   // dA [r][s]
    static constexpr int OFF_AT = OFF_DA + C * PB * 2;  // A^T [s][r]
    static constexpr int OFF_DS = OFF_AT + C * PB * 2;  // dS1' [c][n] (walk: fp32)
    static constexpr int BYTES = OFF_DS + (WALK ? DK * PF * 4 : DK * P * 2);
    static_assert(2 * TILE >= C * PE * 4, "dg scratch does not fit in the v / dO region");
    static_assert(!VEC || DK * P * 2 >= C * PBF * 4, "prefixes do not fit in the state-gradient region");
};

// WALK (scalar gate only): a workgroup walks the chunks of one (b, h, piece) from
// last to first with the state gradient in LDS (fp32), applying the reverse update
// dS <- decay dS + sum over the chunk's first-document rows of exp(beta_r) q_r dO_r^T
// after each chunk (FLAT page, Linear Attention > Backward Recurrence: the state
// gradient runs backwards in time, scaled by the gate at each step), so the state
// gradient is never written per chunk.
template <bool VEC, bool WALK>
__global__ __launch_bounds__(512) void k_grad8(const RevArgs a) {
    static_assert(VEC != WALK, "the walk serves the scalar gate, one item per workgroup the vector gate");
    using T = bf16;
    using Cfg = Grad8Cfg<VEC, WALK>;
    using M = Mma<T>;
    constexpr int P = Cfg::P, PB = Cfg::PB, PE = Cfg::PE, PF = Cfg::PF, DK = 128, DV = 128;
    put_stamp(a.stamp_out, a.stamp_val);  // the states the pass before this one found or stored
    constexpr int NTH = Cfg::NTH, KS = M::KSTEP, NKV = DV / KS;

    __shared__ __attribute__((aligned(16))) char lds[Cfg::BYTES];
    __shared__ RevChunk ck;
    __shared__ float sBs[8];
    __shared__ float sBnd[VEC ? 8 : 1][16];
    __shared__ int sStrong[8];
    T* sQ = reinterpret_cast<T*>(lds + Cfg::OFF_Q);
    T* sK = reinterpret_cast<T*>(lds + Cfg::OFF_K);
    T* sG = reinterpret_cast<T*>(lds + Cfg::OFF_G);  // vector gate only
    T* sV = reinterpret_cast<T*>(lds + Cfg::OFF_V);
    T* sdO = reinterpret_cast<T*>(lds + Cfg::OFF_DO);
    T* sdA = reinterpret_cast<T*>(lds + Cfg::OFF_DA);
    T* sAT = reinterpret_cast<T*>(lds + Cfg::OFF_AT);
    T* sdS = reinterpret_cast<T*>(lds + Cfg::OFF_DS);
    float* sM = reinterpret_cast<float*>(lds + Cfg::OFF_DS);  // walk: state gradient [c][n]
    // strong-gate chunks: the fp32 prefixes [r][c], until the state-gradient rows are staged
    float* sBF = reinterpret_cast<float*>(lds + Cfg::OFF_DS);
    float* sX = reinterpret_cast<float*>(lds + Cfg::OFF_V);  // dg scratch [r][c], after dv
    // scalar gate: per-wave row sums [8][C] for dg, in the dA tile (read only before dv)
    float (*sXs)[C] = reinterpret_cast<float (*)[C]>(lds + Cfg::OFF_DA);

    const int64_t T_ = a.T;
    const int64_t NC = (T_ + C - 1) / C;
    const int64_t nitems = a.B * a.H * NC;
    const int w = wave_id(), l = lane_id(), j4 = l >> 4, i16 = l & 15;
    const int cw = 16 * w;  // the wave's key channels (dq, dk, dg) and value columns (dv)
    const int64_t rs_qk = a.ld_qk, rs_v = a.ld_v, rs_do = a.H * DV;
    const int64_t rs_g = VEC ? a.H * DK : a.H;
    const int64_t G = a.H / a.Hqk;

    // The walk: a persistent loop, the next chunk's tiles loaded into registers while
    // the current one computes.  Vector gate: one item per workgroup (the prefetch
    // registers would not fit next to its gate factors).
    constexpr bool PREFETCH = WALK;
    TileRegs<T, 128, NTH> pq, pk, pg, pv, pdo;
    RowRegs rr;
    // item indices in 32 bits (the launch checks B * H * NC < 2^31)
    const uint32_t NC32 = (uint32_t)NC, H32 = (uint32_t)a.H, G32 = (uint32_t)G;
    auto issue = [&](uint32_t bh, uint32_t ci) {
        const uint32_t b = bh / H32, h = bh - b * H32, hq = h / G32;
        const int64_t t0 = (int64_t)ci * C;
        const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
        pq.load((const T*)a.q + (b * T_ + t0) * rs_qk + hq * DK, rs_qk, nvalid);
        pk.load((const T*)a.k + (b * T_ + t0) * rs_qk + hq * DK, rs_qk, nvalid);
        const T* grow = (const T*)a.g + (b * T_ + t0) * rs_g + (VEC ? h * DK : h);
        if constexpr (VEC) pg.load(grow, rs_g, nvalid);
        pv.load((const T*)a.v + (b * T_ + t0) * rs_v + h * DV, rs_v, nvalid);
        pdo.load((const T*)a.dO + (b * T_ + t0) * rs_do + h * DV, rs_do, nvalid);
        if (w == 0) rr.load(grow, rs_g, a.seg, b, T_, t0, nvalid, !VEC);
    };
    // Work order.  Units are items (b, h, chunk), or for the walk pieces (b, h, piece),
    // strided over the grid; a walk visits its unit's chunks from last to first.
    // A position is (unit, bh, ci, cb): cb is the unit's first chunk (its last in the walk).
    const uint32_t nunits = (uint32_t)(WALK ? a.B * a.H * a.P : nitems);
    const uint32_t P32 = (uint32_t)a.P, PL32 = (uint32_t)a.PL;
    struct Pos { uint32_t unit, bh, ci, cb; };
    auto unit_pos = [&](uint32_t u) -> Pos {
        if constexpr (WALK) {
            const uint32_t bh = u / P32, cb = (u - bh * P32) * PL32;
            const uint32_t ce = cb + PL32 < NC32 ? cb + PL32 : NC32;
            return Pos{u, bh, ce - 1, cb};
        } else {
            const uint32_t bh = u / NC32, ci = u - bh * NC32;
            return Pos{u, bh, ci, ci};
        }
    };
    const uint32_t stride = PREFETCH ? gridDim.x : nunits;
    Pos cur = unit_pos(blockIdx.x < nunits ? blockIdx.x : 0);
    cur.unit = blockIdx.x;
    bool unit_start = true;
    if constexpr (PREFETCH) {
        if (cur.unit < nunits) issue(cur.bh, cur.ci);
    }
    for (; cur.unit < nunits;) {
    if constexpr (!PREFETCH) issue(cur.bh, cur.ci);
    const uint32_t ci = cur.ci, bh = cur.bh;
    const uint32_t b = bh / H32, h = bh - b * H32, hq = h / G32;
    const int64_t t0 = (int64_t)ci * C;
    const int nvalid = (T_ - t0) < C ? (int)(T_ - t0) : C;
    // the item after this one
    const bool unit_end = ci == cur.cb;
    Pos nxt;
    if (!unit_end) nxt = Pos{cur.unit, bh, ci - 1, cur.cb};
    else if (cur.unit + stride < nunits) nxt = unit_pos(cur.unit + stride);
    else nxt = Pos{nunits, 0, 0, 0};
    // rows cw + i of S0 and dS1 (the A operands of dO S0^T and v dS1^T, k = n)
    const T* S0 = (const T*)a.ws_S + (((int64_t)bh * (NC + 1) + ci) * DK + cw + i16) * DV;

    // ---- phase 1: this item's tiles to LDS; its S0 and dS1 rows to registers
    bf16x8 s0f[NKV], dsf[NKV];
#pragma unroll
    for (int kk = 0; kk < NKV; ++kk) s0f[kk] = *reinterpret_cast<const bf16x8*>(S0 + kk * KS + 8 * j4);
    if constexpr (WALK) {
        // the wave's own rows of the state gradient: set at a walk's start (the
        // gradient at the piece's end), else left by the update after the chunk above
        float* mrow = sM + (cw + i16) * PF;
        if (unit_start) {
            const float* src = a.P > 1 ? a.dS_in + ((int64_t)cur.unit * DK + cw + i16) * DV
                                       : (a.dhT ? a.dhT + ((int64_t)bh * DK + cw + i16) * DV : nullptr);
#pragma unroll
            for (int nt = 0; nt < DV / 16; ++nt)
                *reinterpret_cast<f32x4*>(mrow + 16 * nt + 4 * j4) =
                    src ? *reinterpret_cast<const f32x4*>(src + 16 * nt + 4 * j4) : zero4();
        }
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(mrow + kk * KS + 8 * j4);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(mrow + kk * KS + 8 * j4 + 4);
            const f32x8 x = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
            dsf[kk] = __builtin_convertvector(x, bf16x8);
        }
    } else {
        const T* dS1 = (const T*)a.ws_dS + (((int64_t)bh * NC + ci) * DK + cw + i16) * DV;
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) dsf[kk] = *reinterpret_cast<const bf16x8*>(dS1 + kk * KS + 8 * j4);
    }
    pq.store_rows(sQ, P);
    pk.store_rows(sK, P);
    if constexpr (VEC) {
        pg.store_rows(sG, P);
        strong_flag_put(sStrong, gate_regs_strong(pg));
    }
    pv.store_rows(sV, P);
    pdo.store_rows(sdO, P);
    if (w == 0) rev_chunk_info<T, VEC>(&ck, rr);
    __syncthreads();
    [[maybe_unused]] const bool strong = VEC && strong_flag_get<8>(sStrong);
    // The next item's tiles (after the last item: this one's again, unused).  The
    // requests are unconditional so that a wait for this item's S0 rows, requested
    // before them, is counted exactly and does not wait for them as well.
    if constexpr (PREFETCH) {
        const bool more = nxt.unit < nunits;
        issue(more ? nxt.bh : bh, more ? nxt.ci : ci);
    }
    [[maybe_unused]] const TriOnes<T> tri;

    // ---- phase 2: gate prefix, scaling, dS1' rows, dA
    // raw q, k at this lane's output positions (rows 16rt + i16, channels cw + 4j4 + e)
    Vec4<T> qraw[4], kraw[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        qraw[rt] = Vec4<T>::load(sQ + (16 * rt + i16) * P + cw + 4 * j4);
        kraw[rt] = Vec4<T>::load(sK + (16 * rt + i16) * P + cw + 4 * j4);
    }
    // factored form: E = exp(beta - m), em = exp(m), egm = exp(Gamma - m); strong-gate
    // chunks: E = beta, egm = Gamma themselves (the exponentials are formed per use)
    float E[4][4];
    float em[4], egm[4], dec[4];
    if constexpr (VEC) {
        f32x4 beta[1][4];
        gate_prefix_mfma<T, 1, P>(sG, tri, beta);  // channel tile w
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
                for (int e = 0; e < 4; ++e) {
                    E[rt][e] = beta[0][rt][e];
                    sBF[(16 * rt + i16) * Cfg::PBF + cw + 4 * j4 + e] = beta[0][rt][e];
                }
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
            qa.store(sQ + (16 * rt + i16) * P + cw + 4 * j4);
            ka.store(sK + (16 * rt + i16) * P + cw + 4 * j4);
        }
        // dS1 rows of this wave's channels scaled by exp(Gamma - m) of the channel
        // (KA dS1' = KU dS1 for dv); lane i16 holds channel cw + i16, whose prefix
        // values sit in lane (i16 / 4, 15), element i16 % 4
        float mi = 0.f, gi = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float mv = __shfl(beta[0][1][e], 16 * (i16 >> 2) + 15, 64);
            const float gv = __shfl(beta[0][3][e], 16 * (i16 >> 2) + 15, 64);
            if ((i16 & 3) == e) {
                mi = mv;
                gi = gv;
            }
        }
        const float egm_i = __expf(gi - mi);
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) {
            bf16x8 d = dsf[kk];
#pragma unroll
            for (int e = 0; e < 8; ++e) d[e] = (bf16)((float)d[e] * egm_i);
            *reinterpret_cast<bf16x8*>(sdS + (cw + i16) * P + kk * KS + 8 * j4) = d;
        }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            em[e] = egm[e] = 1.f;
            dec[e] = ck.decay;
        }
    }
    // dA^T = v dO^T tiles, masked, stored as dA[r][s] (10 lower + 2 zero upper tiles)
    for (int ti = w; ti < 12; ti += Cfg::NW) {
        const int rt = score_tile_rt(ti);
        const int st = score_tile_st(ti);
        f32x4 acc = zero4();
        if (ti < 10) {
#pragma unroll
            for (int n0 = 0; n0 < DV; n0 += KS)
                acc = M::mma(frag_ld<T, P, 1>(sV, 16 * st, n0), frag_ld<T, P, 1>(sdO, 16 * rt, n0), acc);
        }
        store_masked_N<T, VEC, PB>(sdA, ck, rt, st, ti < 10, acc);
    }
    __syncthreads();
    // A = QA KA^T tiles (all channels, now scaled), masked, stored transposed A^T[s][r]
    if (strong) exact_scores<T, DK, NTH, P, P, Cfg::PBF, PB, true>(sAT, sQ, sK, sBF, ck.doc);
    for (int ti = w; ti < (strong ? 0 : 12); ti += Cfg::NW) {
        const int rt = score_tile_rt(ti);
        const int st = score_tile_st(ti);
        f32x4 acc = zero4();
        if (ti < 10) {
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KS)
                acc = M::mma(frag_ld<T, P, 1>(sQ, 16 * rt, k0), frag_ld<T, P, 1>(sK, 16 * st, k0), acc);
        }
        store_masked_T<T, VEC, PB>(sAT, ck, rt, st, ti < 10, acc);
    }

    // ---- phase 3a: dq, dk for key channels cw .. cw + 15 (computed transposed)
    const bool gqa = G > 1;
    float x[4][4];  // q*dq - k*dk (factored form)
    float bnd[4];   // the boundary term rowsum(S1 * dS1) per channel (factored form)
    if (strong) {
        // A strong-gate chunk (gla_exact.hpp): the intra-chunk parts of dq and dk from
        // the prefixes (E holds beta, egm holds Gamma), the carried parts with exp(beta)
        // and exp(Gamma - beta).  The log-gate gradient goes out here too, as
        //   dg[r] = (suffix of y from r within r's document) + (sum of z over the rows
        //           before r) + [no reset] decay rowsum(S0 * dS1),
        // y = q * dq - k * dk without the diagonal score pairs (they cancel exactly) and
        // without z = k * (carried part of dk): the suffix form with every cancelling
        // pair left out (rows before r reach dS1 only through token r's gate; z is 0
        // outside the chunk's last document).  Scratch: the prefixes' region, free
        // once every wave is past the scores.
        __syncthreads();
        float y[4][4], z[4][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 a2 = zero4();
#pragma unroll
            for (int kk = 0; kk < NKV; ++kk) a2 = M::mma(s0f[kk], frag_ld<T, P, 1>(sdO, 16 * rt, kk * KS), a2);
            const int r = 16 * rt + i16;
            const float fq = ck.fq[r];
            float dx[4] = {0.f, 0.f, 0.f, 0.f}, dd[4] = {0.f, 0.f, 0.f, 0.f}, dq[4];
            exact_dq<T, P, PB>(dx, dd, rt, E, sdA, sK + cw + 4 * j4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dqx = dx[e] + fq * __expf(E[rt][e]) * a2[e];
                dq[e] = dqx + dd[e];
                y[rt][e] = qraw[rt].get(e) * dqx;
            }
            if (r < nvalid) {
                if (!gqa) store4<T>((T*)a.dq + (b * T_ + t0 + r) * a.ld_dqk + hq * DK + cw + 4 * j4, dq);
                else store4<float>(a.ws_dq + ((b * T_ + t0 + r) * a.H + h) * DK + cw + 4 * j4, dq);
            }
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 a2 = zero4();
#pragma unroll
            for (int kk = 0; kk < NKV; ++kk) a2 = M::mma(dsf[kk], frag_ld<T, P, 1>(sV, 16 * st, kk * KS), a2);
            const int s = 16 * st + i16;
            const float fu = ck.fu[s];
            float dx[4] = {0.f, 0.f, 0.f, 0.f}, dd[4] = {0.f, 0.f, 0.f, 0.f}, dk[4];
            exact_dk<T, P, PB>(dx, dd, st, E, sdA, sQ + cw + 4 * j4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float inter = fu * __expf(egm[e] - E[st][e]) * a2[e];
                const float kr = kraw[st].get(e);
                dk[e] = dx[e] + dd[e] + inter;
                y[st][e] -= kr * dx[e];
                z[st][e] = kr * inter;
            }
            if (s < nvalid) {
                if (!gqa) store4<T>((T*)a.dk + (b * T_ + t0 + s) * a.ld_dqk + hq * DK + cw + 4 * j4, dk);
                else store4<float>(a.ws_dk + ((b * T_ + t0 + s) * a.H + h) * DK + cw + 4 * j4, dk);
            }
        }
        float zp[4][4], bnd0[4];
        float sd = 0.f;  // rowsum(S0 * dS1) of channel cw + i16 over this lane's n
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) sd = frag_dot(s0f[kk], dsf[kk], sd);
        sd += __shfl_xor(sd, 16, 64);
        sd += __shfl_xor(sd, 32, 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float zc[4], zo[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) zc[rt] = z[rt][e];
            rows_excl_prefix(zc, zo);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) zp[rt][e] = zo[rt];
            bnd0[e] = dec[e] * __shfl(sd, 4 * j4 + e, 64);
        }
        vec_dg_serial<T, Cfg::PBF>(sBF, sBnd[w], ck, cw, y, bnd0, zp, nvalid,
                                   (T*)a.dg + ((b * T_ + t0) * a.H + h) * DK, a.H * DK);
        // the update operand KU = k exp(Gamma - beta) in place of this wave's k columns
        // (only this wave read them above) for dv; the state-gradient rows, unscaled, in
        // the scratch's place once every wave is done with it
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            Vec4<T> ku;
#pragma unroll
            for (int e = 0; e < 4; ++e) ku.set(e, kraw[st].get(e) * __expf(egm[e] - E[st][e]));
            ku.store(sK + (16 * st + i16) * P + cw + 4 * j4);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk)
            *reinterpret_cast<bf16x8*>(sdS + (cw + i16) * P + kk * KS + 8 * j4) = dsf[kk];
        __syncthreads();  // A^T complete
    } else {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 a1 = zero4(), a2 = zero4();
            const int kend = ((16 * (rt + 1) + KS - 1) / KS) * KS;
#pragma unroll
            for (int k0 = 0; k0 < kend; k0 += KS)
                a1 = M::mma(frag_col<T, P, false>(sK, cw, k0), frag_ld<T, PB, 1>(sdA, 16 * rt, k0), a1);
#pragma unroll
            for (int kk = 0; kk < NKV; ++kk) a2 = M::mma(s0f[kk], frag_ld<T, P, 1>(sdO, 16 * rt, kk * KS), a2);
            const int r = 16 * rt + i16;
            const float fq = ck.fq[r];
            float dq[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dqp = a1[e] + fq * em[e] * a2[e];
                dq[e] = VEC ? E[rt][e] * dqp : dqp;
                x[rt][e] = qraw[rt].get(e) * dq[e];
            }
            if (r < nvalid) {
                if (!gqa) store4<T>((T*)a.dq + (b * T_ + t0 + r) * a.ld_dqk + hq * DK + cw + 4 * j4, dq);
                else store4<float>(a.ws_dq + ((b * T_ + t0 + r) * a.H + h) * DK + cw + 4 * j4, dq);
            }
        }
        float bsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 a1 = zero4(), a2 = zero4();
            const int kbeg = (16 * st / KS) * KS;
#pragma unroll
            for (int k0 = kbeg; k0 < C; k0 += KS)
                a1 = M::mma(frag_col<T, P, false>(sQ, cw, k0), frag_col<T, PB, false>(sdA, 16 * st, k0), a1);
#pragma unroll
            for (int kk = 0; kk < NKV; ++kk) a2 = M::mma(dsf[kk], frag_ld<T, P, 1>(sV, 16 * st, kk * KS), a2);
            const int s = 16 * st + i16;
            const float fu = ck.fu[s];
            float dk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float inter = fu * egm[e] * a2[e];
                const float rE = VEC ? __builtin_amdgcn_rcpf(E[st][e]) : 1.f;
                const float kr = kraw[st].get(e);
                dk[e] = (a1[e] + inter) * rE;
                x[st][e] -= kr * dk[e];
                bsum[e] += kr * inter * rE;
            }
            if (s < nvalid) {
                if (!gqa) store4<T>((T*)a.dk + (b * T_ + t0 + s) * a.ld_dqk + hq * DK + cw + 4 * j4, dk);
                else store4<float>(a.ws_dk + ((b * T_ + t0 + s) * a.H + h) * DK + cw + 4 * j4, dk);
            }
        }
        // boundary term rowsum(S1 * dS1) per channel cw + 4j4 + e
        float sd = 0.f;  // rowsum(S0 * dS1) of channel cw + i16 over this lane's n
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) sd = frag_dot(s0f[kk], dsf[kk], sd);
        sd += __shfl_xor(sd, 16, 64);
        sd += __shfl_xor(sd, 32, 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) bnd[e] = dec[e] * __shfl(sd, 4 * j4 + e, 64) + row_sum16(bsum[e]);
        __syncthreads();  // A^T complete
    }

    // ---- phase 3b: dv^T = dO^T A + [last doc] dS1'^T KA^T for value columns cw .. cw + 15
    {
        T* dvo = (T*)a.dv + (b * T_ + t0) * a.ld_dv + h * DV + cw + 4 * j4;
        // dS1'^T rows (value columns cw + i16), k = key channel
        bf16x8 dsc[DK / KS];
#pragma unroll
        for (int kk = 0; kk < DK / KS; ++kk) {
            if constexpr (WALK) {
                f32x8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = sM[(kk * KS + 8 * j4 + e) * PF + cw + i16];
                dsc[kk] = __builtin_convertvector(x, bf16x8);
            } else {
                dsc[kk] = frag_col<T, P, false>(sdS, cw, kk * KS);
            }
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 a1 = zero4(), a2 = zero4();
            const int kbeg = (16 * st / KS) * KS;
#pragma unroll
            for (int k0 = kbeg; k0 < C; k0 += KS)
                a1 = M::mma(frag_col<T, P, false>(sdO, cw, k0), frag_ld<T, PB, 1>(sAT, 16 * st, k0), a1);
#pragma unroll
            for (int kk = 0; kk < DK / KS; ++kk)
                a2 = M::mma(dsc[kk], frag_ld<T, P, 1>(sK, 16 * st, kk * KS), a2);
            const int s = 16 * st + i16;
            const float fu = ck.fu[s];
            float dv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) dv[e] = a1[e] + fu * a2[e];
            if (s < nvalid) store4<T>(dvo + (int64_t)s * a.ld_dv, dv);
        }
    }

    // ---- phase 3c: log-gate gradient
    if constexpr (VEC) {
        if (strong) {
            // (done with dq and dk above)
        } else {
        T* dgo = (T*)a.dg + ((b * T_ + t0) * a.H + h) * DK + cw + 4 * j4;
        if (ck.first_reset == C) {
            float carry[4] = {bnd[0], bnd[1], bnd[2], bnd[3]};
#pragma unroll
            for (int rt = 3; rt >= 0; --rt) {
                float dg[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = row_suffix16(x[rt][e]);
                    dg[e] = y + carry[e];
                    carry[e] += __shfl(y, 0, 16);
                }
                const int r = 16 * rt + i16;
                if (r < nvalid) store4<T>(dgo + (int64_t)r * a.H * DK, dg);
            }
        } else {
            // documents inside the chunk: serial segmented suffix sum per channel, in the
            // scratch that takes the place of v and dO
            __syncthreads();
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                *reinterpret_cast<f32x4*>(sX + (16 * rt + i16) * PE + cw + 4 * j4) =
                    f32x4{x[rt][0], x[rt][1], x[rt][2], x[rt][3]};
            if (i16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sBnd[w][4 * j4 + e] = bnd[e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (j4 == 0) {
                const int c = cw + i16;
                float run = sBnd[w][i16];
                for (int r = C - 1; r >= 0; --r) {
                    float val = 0.f;
                    if (r < nvalid) {
                        if (r < nvalid - 1 && ck.doc[r + 1] != ck.doc[r]) run = 0.f;
                        run += sX[r * PE + c];
                        const bool reset = r > 0 ? ck.doc[r] != ck.doc[r - 1] : ck.doc[0] != 0;
                        val = reset ? 0.f : run;
                    }
                    sX[r * PE + c] = val;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r = 16 * rt + i16;
                const f32x4 v = *reinterpret_cast<const f32x4*>(sX + r * PE + cw + 4 * j4);
                const float dg[4] = {v[0], v[1], v[2], v[3]};
                if (r < nvalid) store4<T>(dgo + (int64_t)r * a.H * DK, dg);
            }
        }
        }
    } else {
        // scalar gate: sum over all 128 channels of this workgroup, then a segmented
        // suffix sum over the chunk rows (documents end where the next row resets)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            float y = x[rt][0] + x[rt][1] + x[rt][2] + x[rt][3];
            y += __shfl_xor(y, 16, 64);
            y += __shfl_xor(y, 32, 64);
            if (j4 == 0) sXs[w][16 * rt + i16] = y;
        }
        float bb = bnd[0] + bnd[1] + bnd[2] + bnd[3];
        bb += __shfl_xor(bb, 16, 64);
        bb += __shfl_xor(bb, 32, 64);
        if (l == 0) sBs[w] = bb;
        __syncthreads();
        if (w == 0) {
            const int r = l;
            float xt = 0.f, bt = 0.f;
#pragma unroll
            for (int u = 0; u < Cfg::NW; ++u) {
                xt += sXs[u][r];
                bt += sBs[u];
            }
            const int doc = ck.doc[r];
            float run = (r < nvalid ? xt : 0.f) + (r == nvalid - 1 ? bt : 0.f);
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float y = __shfl_down(run, d, 64);
                const int dd = __shfl_down(doc, d, 64);
                if (r + d < 64 && dd == doc) run += y;
            }
            const bool reset = r > 0 ? doc != ck.doc[r - 1] : doc != 0;
            if (r < nvalid) ((T*)a.dg)[(b * T_ + t0 + r) * a.H + h] = from_f32<T>(reset ? 0.f : run);
        }
    }
    if constexpr (WALK) {
        // ---- phase 4: the state gradient at the previous chunk's end, rows cw + i16
        // (every wave has read the columns dv needs: the barrier of phase 3c), as
        // C-layout tiles [n][c]: lane n = 16nt + 4j4 + e, c = cw + i16
        bf16x8 qf[C / KS];
#pragma unroll
        for (int kk = 0; kk < C / KS; ++kk) {
            qf[kk] = frag_col<T, P, false>(sQ, cw, kk * KS);
            const f32x4 f0 = *reinterpret_cast<const f32x4*>(&ck.fq[kk * KS + 8 * j4]);
            const f32x4 f1 = *reinterpret_cast<const f32x4*>(&ck.fq[kk * KS + 8 * j4 + 4]);
            const f32x8 f = __builtin_shufflevector(f0, f1, 0, 1, 2, 3, 4, 5, 6, 7);
            f32x8 x = __builtin_convertvector(qf[kk], f32x8);
            qf[kk] = __builtin_convertvector(x * f, bf16x8);
        }
        const float dec = ck.decay;
        float* mrow = sM + (cw + i16) * PF;
        f32x4 acc[DV / 16];
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt) acc[nt] = *reinterpret_cast<const f32x4*>(mrow + 16 * nt + 4 * j4) * dec;
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt)
#pragma unroll
            for (int kk = 0; kk < C / KS; ++kk)
                acc[nt] = M::mma(frag_col<T, P, false>(sdO, 16 * nt, kk * KS), qf[kk], acc[nt]);
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt) *reinterpret_cast<f32x4*>(mrow + 16 * nt + 4 * j4) = acc[nt];
        if (unit_end && ci == 0 && a.dh0) {
#pragma unroll
            for (int nt = 0; nt < DV / 16; ++nt)
                *reinterpret_cast<f32x4*>(a.dh0 + ((int64_t)bh * DK + cw + i16) * DV + 16 * nt + 4 * j4) = acc[nt];
        }
    }
    __syncthreads();  // LDS and the chunk data are rewritten by the next item
    if constexpr (!PREFETCH) break;  // vector gate: one item per workgroup
    unit_start = unit_end;
    cur = nxt;
    }
}

// the walk: one resident workgroup per compute unit (the LDS holds one), each
// walking pieces in turn; vector gate: one workgroup per item
constexpr int64_t kGrad8Workers = 256;

hipError_t launch_grad8(const RevArgs& a, hipStream_t st) {
    const int64_t NC = (a.T + C - 1) / C;
    const int64_t items = a.B * a.H * NC;
    if (items >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_grad8<true, false>), dim3((unsigned)items), dim3(Grad8Cfg<true, false>::NTH), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_grad8_walk(const RevArgs& a, hipStream_t st) {
    if (a.B * a.H * ((a.T + C - 1) / C) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const int64_t units = a.B * a.H * a.P;
    const int64_t grid = units < kGrad8Workers ? units : kGrad8Workers;
    hipLaunchKernelGGL((k_grad8<false, true>), dim3((unsigned)grid), dim3(Grad8Cfg<false, true>::NTH), 0, st, a);
    return hipGetLastError();
}


}  // namespace gla
