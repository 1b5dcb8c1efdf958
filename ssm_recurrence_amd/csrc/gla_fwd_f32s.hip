// gla_fwd_f32s.hip -- fused chunk-parallel forward for fp32 inputs with the
// scalar gate and 128 x 128 heads (gfx950), on the bf16 matrix cores.
//
// The recurrence, the per-chunk algebra and the split of the sequence into
// pieces are those of gla_fwd.hip (FLAT page, "FLAT: Flash Linear Attention on
// TPUs", Linear Attention > Forward Recurrence, chunkwise form; Pallas Kernels >
// Forward Kernels, the fused block-recurrent kernel): per chunk, with beta the
// chunk-local prefix of the log gates and Gamma its total,
//
//   A[r][s] = (q[r] . k[s]) exp(beta_r - beta_s),   s <= r in one document
//   o[r]    = sum_s A[r][s] v[s] + [r in the first document] exp(beta_r) S^T q[r]
//   S      <- [no reset] exp(Gamma) S + sum_{s in the last document} exp(Gamma - beta_s) k[s] v[s]^T
//
// Every product runs as three bf16 matrix-core products on hi/lo halves of the
// fp32 operands (gla_split.hpp); the state and all accumulation stay fp32.
#include "gla_common.hpp"
#include "gla_kernels.hpp"
#include "gla_split.hpp"
#include "gla_tile.hpp"

namespace gla {

namespace {

constexpr int DK = 128, DV = 128, KS = 32;

// One workgroup of 8 waves per (b, h, piece) holds the whole 128 x 128 state.
// Wave w owns the state's column tile w (all 128 channels): the readout
// S^T q for those columns takes its S^T operand straight from the wave's
// accumulators (a C-layout tile is an operand fragment in ctile order), so the
// state is never copied to LDS, and no workgroup repeats another's q k^T.
// Per chunk: stage the split q, k, v and exp(Gamma - beta_s) v tiles; then
// the masked score tiles (spread over the waves, stored split to LDS), the
// readout and the state update of each wave's columns; then, once every score
// tile is in LDS, the intra-chunk product and the output.  Operand reads are
// issued one step ahead of the matrix-core products that consume them.
//
// Row pitches (bf16 elements) chosen for the LDS reads each tile serves on
// gfx950 (measured): 8-byte reads of four consecutive columns at 16 rows
// (ctile operands) run conflict-free at pitch 12 mod 64, transposed reads at
// any pitch but 12 mod 128 and 16-byte row reads at 16 mod 64.  q and k are read
// in ctile order only (their product is summed over channels, so any channel
// order common to both operands gives the same scores); k also transposed.
constexpr int PQ = DK + 12, PLQ = C * PQ;   // q [64 rows][128]
constexpr int PKH = DK + 20, PLKH = C * PKH; // k [64 rows][128]
constexpr int PH = DK + 8, PLH = C * PH;    // v, scaled v [64 rows][128] (transposed reads)
constexpr int PA = C + 8, PLA = C * PA;     // [64 r][64 s] split score tile

__global__ __launch_bounds__(512) void k_fwd_f32h(const PassArgs a) {
    constexpr int NTH = 512;
    put_stamp(a.stamp_out, a.expect);  // the states this kernel stores
    __shared__ __attribute__((aligned(16))) bf16 sQ[2 * PLQ];
    __shared__ __attribute__((aligned(16))) bf16 sK[2 * PLKH];
    __shared__ __attribute__((aligned(16))) bf16 sV[2 * PLH];
    __shared__ __attribute__((aligned(16))) bf16 sVu[2 * PLH];   // exp(Gamma - beta_s) [last doc] v
    __shared__ __attribute__((aligned(16))) bf16 sA[2 * PLA];    // masked scores [r][s]
    __shared__ __attribute__((aligned(16))) int sDoc[C];
    __shared__ __attribute__((aligned(16))) float sBeta[C];

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
    const float* qbase = (const float*)a.q + b * T_ * rs_qk + hq * DK;
    const float* kbase = (const float*)a.k + b * T_ * rs_qk + hq * DK;
    const float* vbase = (const float*)a.v + b * T_ * rs_v + h * DV;
    const float* gbase = (const float*)a.g + b * T_ * a.H + h;
    float* obase = (float*)a.o + b * T_ * rs_o + h * DV + 16 * w + 4 * j4;

    // state tiles ct = 0..7 of column tile w: lane holds S[16ct + 4j4 + e][16w + i16]
    f32x4 S[DK / 16];
    load_entry_state_128(a, bh, piece, w, j4, i16, S);

    TileRegs<float, DK, NTH> pq, pk, pv;
    RowRegs rr;
    auto prefetch = [&](int64_t t0) {
        const int64_t nv64 = T_ - t0;
        const int nvalid = nv64 < C ? (int)nv64 : C;
        pq.load(qbase + t0 * rs_qk, rs_qk, nvalid);
        pk.load(kbase + t0 * rs_qk, rs_qk, nvalid);
        pv.load(vbase + t0 * rs_v, rs_v, nvalid);
        rr.load(gbase + t0 * a.H, a.H, a.seg, b, T_, t0, nvalid, true);
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
        const float beta = wave_incl_scan(rr.g());
        const float Gam = __shfl(beta, 63, 64);
        const float fu = l >= last_reset ? __expf(Gam - beta) : 0.f;
        const float fq = l < first_reset ? __expf(beta) : 0.f;
        const float decay = msk ? 0.f : __expf(Gam);
        if (w == 0) {
            sDoc[l] = doc;
            sBeta[l] = beta;
        }

        // ---- staging
        store_rows_split<DK, NTH>(pq, sQ, PQ, PLQ);
        store_rows_split<DK, NTH>(pk, sK, PKH, PLKH);
        {
            using TR = TileRegs<float, DK, NTH>;
            static_assert(TR::NV_TOT % NTH == 0, "");
#pragma unroll
            for (int i = 0; i < TR::NVEC; ++i) {
                const int idx = threadIdx.x + i * NTH;
                const int row = idx / TR::VPR, cv = (idx % TR::VPR) * 4;
                const float f = __shfl(fu, row, 64);
                const f32x4 x = __builtin_bit_cast(f32x4, pv.get(i));
                split4_store(x[0], x[1], x[2], x[3], sV + row * PH + cv, sV + PLH + row * PH + cv);
                split4_store(x[0] * f, x[1] * f, x[2] * f, x[3] * f, sVu + row * PH + cv,
                             sVu + PLH + row * PH + cv);
            }
        }
        // (for the backward) the state entering this chunk, stored while the staged
        // tiles' registers are free and before the next chunk's loads are issued
        if (a.save_S) store_state_128<float>((float*)a.save_S + (bh * (NC + 1) + it) * DK * DV, S);
        if (it + 1 < cend) prefetch(t0 + C);
        __syncthreads();

        // ---- masked score tiles, computed transposed (rows s, column r), stored sA[r][s];
        // tiles 10 and 11 are the zero tiles (0,1) and (2,3) that a 32-wide step reads
        for (int ti = w; ti < 12; ti += 8) {
            const int rt = score_tile_rt(ti);
            const int st = score_tile_st(ti);
            f32x4 acc = zero4();
            if (ti < 10) {
#pragma unroll
                for (int kk = 0; kk < DK / KS; ++kk)
                    acc = mma3(sld_ctile<PKH, PLKH>(sK, 16 * st, kk * KS), sld_ctile<PQ, PLQ>(sQ, 16 * rt, kk * KS),
                               acc);
            }
            const int r = 16 * rt + i16, s0 = 16 * st + 4 * j4;
            const int dr = sDoc[r];
            const float br = sBeta[r];
            const int4 d4 = *reinterpret_cast<const int4*>(&sDoc[s0]);
            const float4 b4 = *reinterpret_cast<const float4*>(&sBeta[s0]);
            const int ds[4] = {d4.x, d4.y, d4.z, d4.w};
            const float bs[4] = {b4.x, b4.y, b4.z, b4.w};
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = (ti < 10 && s0 + e <= r && ds[e] == dr) ? acc[e] * __expf(br - bs[e]) : 0.f;
            split4_store(x[0], x[1], x[2], x[3], sA + r * PA + s0, sA + PLA + r * PA + s0);
        }

        // ---- readout R^T[n][r] = sum_c S[c][n] q[r][c] for this wave's columns
        // (the S^T operand, k = channel in ctile order, is split from the
        // accumulators).  Operand reads run one step ahead of the products.
        f32x4 R[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) R[rt] = zero4();
        {
            SFrag qa = sld_ctile<PQ, PLQ>(sQ, 0, 0);
            SFrag sf = split8(S[0], S[1]);
#pragma unroll
            for (int idx = 0; idx < 16; ++idx) {
                const int p = idx >> 2, rt = idx & 3;
                SFrag qb;
                if (idx + 1 < 16) qb = sld_ctile<PQ, PLQ>(sQ, 16 * ((idx + 1) & 3), KS * ((idx + 1) >> 2));
                __builtin_amdgcn_sched_barrier(0);  // keep the next reads ahead of these products
                R[rt] = mma3(sf, qa, R[rt]);
                __builtin_amdgcn_sched_barrier(0);
                if (rt == 3 && p < 3) sf = split8(S[2 * p + 2], S[2 * p + 3]);
                qa = qb;
            }
        }

        // ---- state update of this wave's columns: S = decay S + K^T (fu v),
        // accumulated straight into the state
        {
            SFrag vu[C / KS];
#pragma unroll
            for (int k = 0; k < C / KS; ++k) vu[k] = scol<PH, PLH>(sVu, 16 * w, k * KS);
#pragma unroll
            for (int ct = 0; ct < DK / 16; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[ct][e] *= decay;
            SFrag ka = scol<PKH, PLKH>(sK, 0, 0);
#pragma unroll
            for (int idx = 0; idx < 16; ++idx) {
                const int k = idx >> 3, ct = idx & 7;
                SFrag kb;
                if (idx + 1 < 16) kb = scol<PKH, PLKH>(sK, 16 * ((idx + 1) & 7), KS * ((idx + 1) >> 3));
                __builtin_amdgcn_sched_barrier(0);
                S[ct] = mma3(ka, vu[k], S[ct]);
                __builtin_amdgcn_sched_barrier(0);
                ka = kb;
            }
        }
        __syncthreads();

        // ---- intra-chunk product and output: o^T[n][r] = sum_s v[s][n] A[r][s] + fq_r R^T[n][r]
        {
            SFrag vt[C / KS];
#pragma unroll
            for (int p = 0; p < C / KS; ++p) vt[p] = scol<PH, PLH>(sV, 16 * w, p * KS);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 O = zero4();
#pragma unroll
                for (int p = 0; p <= rt / 2; ++p) O = mma3(vt[p], sld<PA, PLA>(sA, 16 * rt, p * KS), O);
                const int r = 16 * rt + i16;
                const float fr = __shfl(fq, r, 64);
                if (r < nvalid) {
                    f32x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = O[e] + fr * R[rt][e];
                    *reinterpret_cast<f32x4*>(obase + (t0 + r) * rs_o) = out;
                }
            }
        }
        __syncthreads();
    }

    if (a.save_S && piece == P - 1) store_state_128<float>((float*)a.save_S + (bh * (NC + 1) + NC) * DK * DV, S);
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

hipError_t launch_fwd_f32h(const PassArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_fwd_f32h, dim3((unsigned)(a.B * a.H * a.P)), dim3(512), 0, st, a);
    return hipGetLastError();
}

}  // namespace gla
