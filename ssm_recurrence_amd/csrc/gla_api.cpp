// gla_api.cpp -- the C ABI declared in include/gla.h: argument checks (all on
// the host, before anything is enqueued), workspace sizing and dispatch to the
// gfx950 kernels.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "../../include/gla.h"
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace {

using gla::bf16;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Size and kind checks shared by every entry point.
int check_problem(const gla_problem* p) {
    if (!p) return GLA_E_NULL;
    if (p->dtype != GLA_F32 && p->dtype != GLA_BF16) return GLA_E_DTYPE;
    if (p->gate != GLA_GATE_SCALAR && p->gate != GLA_GATE_VECTOR) return GLA_E_DTYPE;
    if (p->split < 0) return GLA_E_SHAPE;
    if (p->B < 1 || p->T < 0 || p->H < 1 || p->H_qk < 1 || p->H_qk > p->H) return GLA_E_SHAPE;
    if (p->H % p->H_qk != 0) return GLA_E_SHAPE;
    if (p->d_k < 1 || p->d_v < 1 || p->chunk < 1) return GLA_E_SHAPE;
    if ((p->flags & ~GLA_SAVE_STATES) || p->reserved != 0) return GLA_E_UNSUPPORTED;
    if ((p->d_k != 64 && p->d_k != 128) || (p->d_v != 64 && p->d_v != 128)) return GLA_E_UNSUPPORTED;
    if (p->chunk != 64) return GLA_E_UNSUPPORTED;
    // every element count and launch grid must fit
    int64_t x, bt, bth;
    if (!mul_ok(p->B, p->T, &bt) || !mul_ok(bt, p->H, &bth) || !mul_ok(bth, 128, &x)) return GLA_E_SHAPE;
    if (x > ((int64_t)1 << 40)) return GLA_E_SHAPE;
    const int64_t nc = (p->T + 63) / 64;
    // launch grids reach B * H * chunks * 8 workgroups (forward, 16-column slices, split)
    if (p->B * p->H * (nc > 0 ? nc : 1) > (((int64_t)1 << 31) - 1) / 8) return GLA_E_SHAPE;
    // row strides: 0 (packed), or at least the packed width, whole 16-byte units,
    // and every element offset within range
    const int64_t per16 = p->dtype == GLA_BF16 ? 8 : 4;
    const int64_t lds[4][2] = {{p->ld_qk, p->H_qk * p->d_k}, {p->ld_v, p->H * p->d_v},
                               {p->ld_dqk, p->H_qk * p->d_k}, {p->ld_dv, p->H * p->d_v}};
    for (const auto& l : lds) {
        if (l[0] == 0) continue;
        if (l[0] < l[1] || l[0] % per16 != 0) return GLA_E_SHAPE;
        if (!mul_ok(bt, l[0], &x) || x > ((int64_t)1 << 40)) return GLA_E_SHAPE;
    }
    return GLA_OK;
}

int64_t ld_or_packed(int64_t ld, int64_t packed) { return ld ? ld : packed; }

// Sequence pieces per (b, h) and chunks per piece.  The sequential passes need
// enough workgroups to occupy the device.  Forward: one per compute unit (256)
// at the widest column slice.  Backward: the paired state and state-gradient
// passes (small workgroups, up to four per unit) are left unsplit from 512
// workgroups up, since a split adds a summary walk of the same length; below
// that they are split towards 1024.  At least 8 chunks stay in a piece so that
// the combine remains small next to the walks.
constexpr int64_t kTargetWG = 256, kNoSplitBwd = 512, kTargetWGBwd = 1024, kMinPieceChunks = 8;

struct Split {
    int64_t P = 1, PL = 0;
};

// bf16, scalar gate, 128 x 128: the backward walks each piece in reverse with the
// state gradient resident (no per-chunk state-gradient pass)
bool walk_bwd(const gla_problem* p) {
    return p->dtype == GLA_BF16 && p->gate == GLA_GATE_SCALAR && p->d_k == 128 && p->d_v == 128;
}

// The forward stores the per-chunk states for the backward (GLA_SAVE_STATES) on
// the walking backward's shape, whose state pass runs alone before the walk, and
// on the fp32 scalar-gate 128 x 128 shape, whose backward then runs its
// state-gradient pass alone, split for that pass.  Elsewhere (vector gate) the
// state pass's share of its paired launch is small next to the forward's store
// of the states: the flag changes nothing there but the workspace size.
bool f32_scalar_128(const gla_problem* p) {
    return p->dtype == GLA_F32 && p->gate == GLA_GATE_SCALAR && p->d_k == 128 && p->d_v == 128;
}
bool saves_states(const gla_problem* p) {
    return (p->flags & GLA_SAVE_STATES) && (walk_bwd(p) || f32_scalar_128(p));
}
bool flag_save(const gla_problem* p) { return (p->flags & GLA_SAVE_STATES) != 0; }

Split plan_split(const gla_problem* p, int for_backward) {
    Split s;
    const int64_t nc = (p->T + 63) / 64;
    s.PL = nc;
    if (nc == 0) return s;
    const int64_t bh = p->B * p->H;
    int64_t P = 1;
    if (p->split > 0) {
        P = p->split;
    } else {
        int64_t per_head, target;  // workgroups per (b, h) without a split
        if (for_backward && (walk_bwd(p) || saves_states(p))) {
            // one walking workgroup per piece; or (fp32 with stored states) one
            // whole-state workgroup per piece of the state-gradient pass alone
            per_head = 1;
            if (bh >= kTargetWG) return s;
            target = kTargetWG;
        } else if (for_backward) {
            // the state and state-gradient passes run side by side
            per_head = 2 * (p->d_k / 64) * (p->d_v / 64);
            if (bh * per_head >= kNoSplitBwd) return s;
            target = kTargetWGBwd;
        } else {
            per_head = p->d_v / (p->dtype == GLA_BF16 ? 64 : 32);
            if (p->d_k == 128 && p->d_v == 128 && (p->dtype == GLA_BF16 || p->gate == GLA_GATE_SCALAR))
                per_head = 1;  // one workgroup holds the whole state
            target = kTargetWG;
        }
        P = (target + bh * per_head - 1) / (bh * per_head);
        const int64_t pmax = nc / kMinPieceChunks;
        if (P > pmax) P = pmax;
        if (P < 1) P = 1;
    }
    if (P > nc) P = nc;
    s.PL = (nc + P - 1) / P;
    s.P = (nc + s.PL - 1) / s.PL;  // no empty piece
    return s;
}

// The fp32 scalar-gate 128 x 128 gradient kernel sums dq, dk over the heads that
// share q/k itself; every other path writes per-head fp32 dq, dk and sums them after.
bool per_head_dqdk(const gla_problem* p) {
    if (p->H_qk == p->H) return false;
    return !(p->dtype == GLA_F32 && p->gate == GLA_GATE_SCALAR && p->d_k == 128 && p->d_v == 128);
}

struct WsLayout {
    size_t S = 0, dS = 0, dq = 0, dk = 0, xs = 0, bnd = 0;
    size_t pL0 = 0, pL1 = 0, pS = 0, pdS = 0, pD = 0, total = 0;
    size_t stamp = 0;  // GLA_SAVE_STATES: the stamp, at the start (S follows it)
    Split sp;
};

// Workspace.  When the sequence is split: per-piece summaries (L0 forward, L1
// reverse, fp32), decay products D, and the piece entry states (backward also
// the state gradients at the piece ends).  Backward only: the state entering
// every chunk (and the final state) and the state gradient at every chunk's
// end, in the input dtype; per-head fp32 dq, dk when heads share q/k;
// per-slice partial gate-gradient sums for the scalar gate.
WsLayout ws_layout_one(const gla_problem* p, int for_backward);

// GLA_SAVE_STATES: one workspace serves both calls; its size is the larger of
// the two.  Where the forward stores states, both lay it out as the stamp, the
// states entering every chunk, then the rest of that call's own layout.
WsLayout ws_layout(const gla_problem* p, int for_backward) {
    WsLayout L = ws_layout_one(p, for_backward);
    if (flag_save(p)) {
        const size_t other = ws_layout_one(p, !for_backward).total;
        if (other > L.total) L.total = other;
    }
    return L;
}

// what a workspace's saved states are computed from (GLA_SAVE_STATES)
gla::Stamp states_stamp(const gla_problem* p, const void* q, const void* k, const void* v, const void* g,
                        const float* h0, const int32_t* seg) {
    const uint64_t words[] = {0x73657461'74732d67ull /* tag */, (uint64_t)p->B, (uint64_t)p->T, (uint64_t)p->H,
                              (uint64_t)p->H_qk, (uint64_t)p->d_k | ((uint64_t)p->d_v << 32),
                              (uint64_t)p->gate | ((uint64_t)p->dtype << 32), (uint64_t)(uintptr_t)q,
                              (uint64_t)(uintptr_t)k, (uint64_t)(uintptr_t)v, (uint64_t)(uintptr_t)g,
                              (uint64_t)(uintptr_t)h0, (uint64_t)(uintptr_t)seg,
                              (uint64_t)ld_or_packed(p->ld_qk, p->H_qk * p->d_k),
                              (uint64_t)ld_or_packed(p->ld_v, p->H * p->d_v), (uint64_t)p->generation};
    static_assert(sizeof words / sizeof words[0] == gla::kStampWords, "stamp words");
    gla::Stamp st;
    for (int i = 0; i < gla::kStampWords; ++i) st.w[i] = words[i];
    return st;
}

WsLayout ws_layout_one(const gla_problem* p, int for_backward) {
    WsLayout L;
    L.sp = plan_split(p, for_backward);
    const int64_t nc = (p->T + 63) / 64;
    const size_t es = p->dtype == GLA_BF16 ? 2 : 4;
    const size_t st = (size_t)p->d_k * (size_t)p->d_v * es;
    const size_t bh = (size_t)(p->B * p->H);
    size_t off = 0;
    if (saves_states(p)) {
        // the stamp and the per-chunk states first, where both calls find them
        L.stamp = 0;
        off = (size_t)gla::kStampBytes;
        L.S = off;
        off += round_up(bh * (size_t)(nc + 1) * st);
    }
    if (L.sp.P > 1) {
        const size_t np = bh * (size_t)L.sp.P;
        const size_t pst = round_up(np * (size_t)(p->d_k * p->d_v) * sizeof(float));
        L.pL0 = off;
        off += pst;
        L.pS = off;
        off += pst;
        if (for_backward) {
            L.pL1 = off;
            off += pst;
            L.pdS = off;
            off += pst;
        }
        L.pD = off;
        off += round_up(np * (size_t)p->d_k * sizeof(float));
    }
    if (!for_backward) {
        L.total = off;
        return L;
    }
    if (!saves_states(p)) {
        L.S = off;
        off += round_up(bh * (size_t)(nc + 1) * st);
    }
    if (!walk_bwd(p)) {
        L.dS = off;
        off += round_up(bh * (size_t)nc * st);
    }
    if (per_head_dqdk(p)) {
        const size_t n = (size_t)(p->B * p->T * p->H * p->d_k) * sizeof(float);
        L.dq = off;
        off += round_up(n);
        L.dk = off;
        off += round_up(n);
    }
    if (p->gate == GLA_GATE_SCALAR) {
        const size_t ns = (size_t)(p->d_k / 64);
        L.xs = off;
        off += round_up(bh * ns * (size_t)p->T * sizeof(float));
        L.bnd = off;
        off += round_up(bh * ns * (size_t)nc * sizeof(float));
    }
    L.total = off;
    return L;
}

bool aligned(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// The current device must be a gfx950.  The answer is cached per device id.
int check_device() {
    static std::mutex mu;
    static signed char known[64];  // 0 unknown, 1 ok, -1 not gfx950
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GLA_E_DEVICE;
    if (dev < 64) {
        std::lock_guard<std::mutex> lock(mu);
        if (known[dev] == 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GLA_E_DEVICE;
            known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        }
        return known[dev] == 1 ? GLA_OK : GLA_E_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GLA_E_DEVICE;
    return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? GLA_OK : GLA_E_DEVICE;
}

__global__ void k_copy_state(float* dst, const float* src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

int copy_state(float* dst, const float* src, int64_t n, hipStream_t st) {
    if (!dst || n == 0) return GLA_OK;
    hipLaunchKernelGGL(k_copy_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, src, n);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

gla::CombineArgs combine_args(const gla::PassArgs& pa, int DK, int DV, int which) {
    gla::CombineArgs c;
    c.L_fwd = pa.L_out[0];
    c.L_rev = pa.L_out[1];
    c.D = pa.D_out;
    c.h0 = pa.h0;
    c.dhT = pa.dhT;
    c.S_in = (float*)pa.S_in;
    c.dS_in = (float*)pa.dS_in;
    c.BH = pa.B * pa.H;
    c.P = pa.P;
    c.DK = DK;
    c.DV = DV;
    c.which = which;
    c.stamp = pa.stamp;
    c.expect = pa.expect;
    c.check_stamp = pa.check_stamp;
    return c;
}

// Piece entry states for a split forward: summaries, then the combine from h0.
// pa.L_out[0], pa.D_out hold the summaries and pa.S_in receives the entry states.
// State-pass block shape: 64 x d_v blocks request each head's v (or dO) once per
// pass instead of once per 64-channel block; they are used when they still give
// `want` workgroups.
bool wide_blocks(const gla::PassArgs& pa, int DK, int64_t passes, int64_t want) {
    return pa.B * pa.H * pa.P * (DK / 64) * passes >= want;
}

template <typename T, bool VEC, int DK, int DV>
hipError_t run_split_fwd_states(const gla::PassArgs& pa, hipStream_t st) {
    hipError_t e = gla::launch_states<T, VEC, DK, DV>(pa, gla::ST_SUM_FWD, wide_blocks(pa, DK, 1, 256), st);
    if (e != hipSuccess || pa.entry_from_summaries) return e;
    return gla::launch_piece_combine(combine_args(pa, DK, DV, 1), st);
}

// Split forwards of the whole-state kernels (128 x 128 heads: bf16, or fp32 with
// the scalar gate) with at most this many pieces skip the combine: the workgroup
// of piece p reads the p summaries before it, P (P - 1) / 2 in all, against 3 P
// for the combine's round trip through S_in, and one launch fewer.
constexpr int64_t kChainPieces = 8;

// Columns of the state per forward workgroup: the widest slice that still
// gives at least 256 workgroups (one per compute unit), else 16.
template <typename T, bool VEC, int DK, int DV>
hipError_t run_fwd(const gla::PassArgs& a0, hipStream_t st) {
    constexpr bool whole = DK == 128 && DV == 128 && (sizeof(T) == 2 || !VEC);
    gla::PassArgs a = a0;
    a.entry_from_summaries = whole && a.P > 1 && a.P <= kChainPieces;
    if (a.P > 1) {
        const hipError_t e = run_split_fwd_states<T, VEC, DK, DV>(a, st);
        if (e != hipSuccess) return e;
    }
    const int64_t wg = a.B * a.H * a.P;
    if constexpr (sizeof(T) == 4 && !VEC && DK == 128 && DV == 128)
        return gla::launch_fwd_f32h(a, st);
    if constexpr (sizeof(T) == 2 && DK == 128 && DV == 128)
        return gla::launch_fwd_h<VEC>(a, st);
    if constexpr (sizeof(T) == 2)  // fp32 tiles with 64 columns exceed the LDS
        if (DV >= 64 && wg * (DV / 64) >= 256) return gla::launch_fwd<T, VEC, DK, DV, 64>(a, st);
    if (wg * (DV / 32) >= 256) return gla::launch_fwd<T, VEC, DK, DV, 32>(a, st);
    return gla::launch_fwd<T, VEC, DK, DV, 16>(a, st);
}

// Backward: (split: both summaries in one launch, or in two where the forward's
// states may be found; both combines in one launch) the state and state-gradient
// passes in one launch (the walk: the state pass, then the walk), the gradients,
// and the sums over heads that share q/k.
template <typename T, bool VEC, int DK, int DV>
hipError_t run_bwd(const gla::PassArgs& pa, const gla::RevArgs& ra, hipStream_t st) {
    hipError_t e;
    // paired passes in 64 x d_v blocks from 256 workgroups on for bf16 (B=4 T=4096
    // H=16, vector gate: 419 against 438 us for the backward with 64 x 64 blocks)
    const bool wide = wide_blocks(pa, DK, 2, sizeof(T) == 2 ? 256 : 512);
    // the states entering the chunks are in ws for these inputs once the state pass
    // has run (or found the forward's): the launch after it writes the stamp that
    // says so (its workgroup 0, at its start)
    uint64_t* const stamp_out = pa.check_stamp ? const_cast<uint64_t*>(pa.stamp) : nullptr;
    // the state and state-gradient passes of a split of up to kChainPieces pieces
    // chain the summaries themselves (no combine launch); the walk reads the
    // combine's state gradients
    constexpr bool walk = sizeof(T) == 2 && !VEC && DK == 128 && DV == 128;
    gla::PassArgs pb = pa;
    pb.entry_from_summaries = !walk && pa.P > 1 && pa.P <= kChainPieces;
    if (pa.P > 1) {
        gla::PassArgs sa = pa;
        sa.d_from_rev = 1;
        if (pa.check_stamp) {
            // the forward's states may be in ws, and then its summaries exit at once:
            // they take the last half of the blocks, after the reverse summaries (bf16,
            // B=1 T=65536 H=16: 141 us for the reverse summaries alone against 202 us
            // interleaved with workgroups that exit)
            e = gla::launch_states_trail<T, VEC, DK, DV>(sa, true, wide_blocks(sa, DK, 1, 256), st);
        } else {
            e = gla::launch_states_pair<T, VEC, DK, DV>(sa, true, wide, st);
        }
        if (e != hipSuccess) return e;
        if (!pb.entry_from_summaries) {
            e = gla::launch_piece_combine(combine_args(pa, DK, DV, 3), st);
            if (e != hipSuccess) return e;
        }
    }
    if constexpr (sizeof(T) == 2 && !VEC && DK == 128 && DV == 128) {
        e = gla::launch_states<T, VEC, DK, DV>(pa, gla::ST_STATES, wide_blocks(pa, DK, 1, 256), st);
        if (e != hipSuccess) return e;
        gla::RevArgs wa = ra;
        wa.stamp_out = stamp_out;
        wa.stamp_val = pa.expect;
        e = gla::launch_grad8_walk(wa, st);
    } else {
        gla::RevArgs ga = ra;
        if (pa.check_stamp) {
            // the forward's states may be in ws: the state pass, which then exits at
            // once, takes the last half of the blocks after the state-gradient pass;
            // the gradient kernel writes the stamp
            e = gla::launch_states_trail<T, VEC, DK, DV>(pb, false, wide_blocks(pa, DK, 1, 256), st);
            ga.stamp_out = stamp_out;
            ga.stamp_val = pa.expect;
        } else {
            e = gla::launch_states_pair<T, VEC, DK, DV>(pb, false, wide, st);
        }
        if (e != hipSuccess) return e;
        e = gla::launch_grad<T, VEC, DK, DV>(ga, st);
    }
    if (e != hipSuccess) return e;
    if (ra.ws_dq) {
        e = gla::launch_group_sum<T, DK>(ra.ws_dq, ra.dq, ra.ld_dqk, ra.B, ra.T, ra.H, ra.Hqk, st);
        if (e != hipSuccess) return e;
        e = gla::launch_group_sum<T, DK>(ra.ws_dk, ra.dk, ra.ld_dqk, ra.B, ra.T, ra.H, ra.Hqk, st);
    }
    return e;
}

// Dispatch over (dtype, gate, d_k, d_v) to a template instance.
template <template <typename, bool, int, int> class F, typename... Args>
hipError_t dispatch(const gla_problem* p, Args&&... args) {
#define GLA_DK_DV(T, VEC)                                                                      \
    if (p->d_k == 64 && p->d_v == 64) return F<T, VEC, 64, 64>::run(args...);                \
    if (p->d_k == 64 && p->d_v == 128) return F<T, VEC, 64, 128>::run(args...);              \
    if (p->d_k == 128 && p->d_v == 64) return F<T, VEC, 128, 64>::run(args...);              \
    return F<T, VEC, 128, 128>::run(args...);
    if (p->dtype == GLA_F32) {
        if (p->gate == GLA_GATE_VECTOR) { GLA_DK_DV(float, true) }
        GLA_DK_DV(float, false)
    }
    if (p->gate == GLA_GATE_VECTOR) { GLA_DK_DV(bf16, true) }
    GLA_DK_DV(bf16, false)
#undef GLA_DK_DV
}

template <typename T, bool VEC, int DK, int DV> struct FwdF {
    static hipError_t run(const gla::PassArgs& a, hipStream_t st) { return run_fwd<T, VEC, DK, DV>(a, st); }
};
template <typename T, bool VEC, int DK, int DV> struct BwdF {
    static hipError_t run(const gla::PassArgs& pa, const gla::RevArgs& ra, hipStream_t st) {
        return run_bwd<T, VEC, DK, DV>(pa, ra, st);
    }
};

// output norm and gate: checks and the dispatch over (dtype, d)
int check_norm(const gla_norm_gate_problem* p) {
    if (!p) return GLA_E_NULL;
    if (p->dtype != GLA_F32 && p->dtype != GLA_BF16) return GLA_E_DTYPE;
    if (p->B < 1 || p->T < 0 || p->H < 1 || p->d < 1) return GLA_E_SHAPE;
    if (!(p->eps >= 0.f) || !(p->eps < 3.0e38f)) return GLA_E_SHAPE;  // (rejects NaN and inf)
    if (p->d != 64 && p->d != 128) return GLA_E_UNSUPPORTED;
    int64_t bt, rows, x;
    if (!mul_ok(p->B, p->T, &bt) || !mul_ok(bt, p->H, &rows) || !mul_ok(rows, p->d, &x) ||
        x > ((int64_t)1 << 40))
        return GLA_E_SHAPE;
    return GLA_OK;
}

int64_t norm_rows(const gla_norm_gate_problem* p) { return p->B * p->T * p->H; }

template <typename F>
hipError_t norm_dispatch(const gla_norm_gate_problem* p, F&& f) {
    if (p->dtype == GLA_BF16)
        return p->d == 64 ? f(gla::bf16(), std::integral_constant<int, 64>())
                          : f(gla::bf16(), std::integral_constant<int, 128>());
    return p->d == 64 ? f(float(), std::integral_constant<int, 64>())
                      : f(float(), std::integral_constant<int, 128>());
}

// gated delta rule: checks and the workspace
int check_delta(const gla_delta_problem* p) {
    if (!p) return GLA_E_NULL;
    if (p->dtype != GLA_F32 && p->dtype != GLA_BF16) return GLA_E_DTYPE;
    if (p->B < 1 || p->T < 0 || p->H < 1 || p->d_k < 1 || p->d_v < 1) return GLA_E_SHAPE;
    if ((p->d_k != 64 && p->d_k != 128) || (p->d_v != 64 && p->d_v != 128)) return GLA_E_UNSUPPORTED;
    if (p->flags & ~GLA_DELTA_WS_FROM_FWD) return GLA_E_UNSUPPORTED;
    int64_t bt, bth, x;
    if (!mul_ok(p->B, p->T, &bt) || !mul_ok(bt, p->H, &bth) || !mul_ok(bth, 128, &x) || x > ((int64_t)1 << 40))
        return GLA_E_SHAPE;
    const int64_t nc = (p->T + 63) / 64;
    if (p->B * p->H * (nc > 0 ? nc : 1) > ((int64_t)1 << 31) - 1) return GLA_E_SHAPE;
    return GLA_OK;
}

// ws: the stamp, then the forward's per-chunk factors; scratch: the backward's
// per-chunk intermediates
// (with GLA_DELTA_WS_FROM_FWD the states entering the chunks and the effective
// writes move from the scratch to ws, where the forward stores them)
bool delta_states_in_ws(const gla_delta_problem* p) { return (p->flags & GLA_DELTA_WS_FROM_FWD) != 0; }
size_t delta_ws_bytes(const gla_delta_problem* p) {
    const int64_t nc = (p->T + 63) / 64;
    return (size_t)gla::kDeltaHeaderBytes +
           (size_t)(p->B * p->H * nc) *
               (size_t)gla::delta_fwd_floats_per_chunk(p->d_k, p->d_v, delta_states_in_ws(p)) * sizeof(float);
}
size_t delta_scratch_bytes(const gla_delta_problem* p) {
    const int64_t nc = (p->T + 63) / 64;
    return (size_t)(p->B * p->H * nc) *
           (size_t)gla::delta_bwd_floats_per_chunk(p->d_k, p->d_v, delta_states_in_ws(p)) * sizeof(float);
}

gla::DeltaArgs delta_args(const gla_delta_problem* p, const void* q, const void* k, const void* v,
                          const void* g, const void* beta, const int32_t* seg, void* ws) {
    gla::DeltaArgs a;
    memset(&a, 0, sizeof a);
    a.B = p->B; a.T = p->T; a.H = p->H; a.dk = p->d_k; a.dv = p->d_v;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.seg = seg;
    a.stamp = (uint64_t*)ws;
    a.ws = (float*)((char*)ws + gla::kDeltaHeaderBytes);
    a.states_in_ws = delta_states_in_ws(p);
    a.ws_chunk = gla::delta_fwd_floats_per_chunk(p->d_k, p->d_v, a.states_in_ws);
    // what the per-chunk factors (and states) in ws are computed from; the flags
    // word keeps a forward that stored no states from vouching for them
    const uint64_t words[] = {0x61746c65642d6177ull /* tag */, (uint64_t)p->B, (uint64_t)p->T,
                              (uint64_t)p->H, (uint64_t)p->d_k, (uint64_t)p->d_v, (uint64_t)p->dtype,
                              (uint64_t)(uintptr_t)q, (uint64_t)(uintptr_t)k, (uint64_t)(uintptr_t)v,
                              (uint64_t)(uintptr_t)g, (uint64_t)(uintptr_t)beta, (uint64_t)(uintptr_t)seg,
                              (uint64_t)p->generation, (uint64_t)(uint32_t)p->flags, 0};
    static_assert(sizeof words / sizeof words[0] == gla::kStampWords, "stamp words");
    for (int i = 0; i < gla::kStampWords; ++i) a.expect.w[i] = words[i];
    return a;
}

// The forward after its argument checks: dispatch with a workspace of at least
// ws_layout(p, 0).total bytes.
int fwd_checked(const gla_problem* p, const WsLayout& L, const void* q, const void* k, const void* v,
                const void* g, const float* h0, const int32_t* segment_ids, void* o, float* hT, void* ws,
                hipStream_t st) {
    if (p->T == 0) return copy_state(hT, h0, p->B * p->H * p->d_k * p->d_v, st);
    gla::PassArgs a;
    memset(&a, 0, sizeof a);
    a.q = q; a.k = k; a.v = v; a.g = g; a.h0 = h0; a.seg = segment_ids; a.o = o; a.hT = hT;
    a.B = p->B; a.T = p->T; a.H = p->H; a.Hqk = p->H_qk;
    a.ld_qk = ld_or_packed(p->ld_qk, p->H_qk * p->d_k);
    a.ld_v = ld_or_packed(p->ld_v, p->H * p->d_v);
    a.P = L.sp.P; a.PL = L.sp.PL;
    if (a.P > 1) {
        char* w = (char*)ws;
        a.L_out[0] = (float*)(w + L.pL0);
        a.S_in = (const float*)(w + L.pS);
        a.D_out = (float*)(w + L.pD);
    }
    if (saves_states(p)) {
        // the forward kernel stores the states and writes the stamp that vouches for them
        a.save_S = (char*)ws + L.S;
        a.stamp_out = (uint64_t*)((char*)ws + L.stamp);
        a.expect = states_stamp(p, q, k, v, g, h0, segment_ids);
    }
    if (dispatch<FwdF>(p, a, st) != hipSuccess) return GLA_E_LAUNCH;
    return GLA_OK;
}

// ---- the forward that allocates nothing (gla_fwd_noalloc)
// Its workspace is this fixed device array: one copy per device, the whole life
// of the process.  Host code never names the array itself (on the host that name
// is only a stand-in for the symbol): it takes each device's address once, with
// that device current, and passes that address on.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_on_current_device(void** out) {
    static std::mutex mu;
    static void* addr[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GLA_E_DEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GLA_E_DEVICE;
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return GLA_OK;
}

}  // namespace

extern "C" {

int gla_workspace_size(const gla_problem* p, int for_backward, size_t* bytes) {
    const int rc = check_problem(p);
    if (rc) return rc;
    if (!bytes) return GLA_E_NULL;
    *bytes = ws_layout(p, for_backward).total;
    return GLA_OK;
}

int gla_fwd(const gla_problem* p, const void* q, const void* k, const void* v, const void* g,
            const float* h0, const int32_t* segment_ids, void* o, float* hT, void* ws,
            size_t ws_bytes, void* stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->T > 0 && (!q || !k || !v || !g || !o)) return GLA_E_NULL;
    const void* ptrs[] = {q, k, v, g, h0, segment_ids, o, hT, ws};
    for (const void* x : ptrs)
        if (x && !aligned(x)) return GLA_E_ALIGN;
    const WsLayout L = ws_layout(p, 0);
    if (ws_bytes < L.total || (L.total > 0 && !ws)) return GLA_E_WORKSPACE;
    rc = check_device();
    if (rc) return rc;
    return fwd_checked(p, L, q, k, v, g, h0, segment_ids, o, hT, ws, (hipStream_t)stream);
}

int gla_fwd_noalloc(const gla_problem* p, const void* q, const void* k, const void* v, const void* g,
                    const float* h0, const int32_t* segment_ids, void* o, float* hT, void* stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->flags & GLA_SAVE_STATES) return GLA_E_UNSUPPORTED;  // (no workspace to hand to a backward)
    if (p->T > 0 && (!q || !k || !v || !g || !o)) return GLA_E_NULL;
    const void* ptrs[] = {q, k, v, g, h0, segment_ids, o, hT};
    for (const void* x : ptrs)
        if (x && !aligned(x)) return GLA_E_ALIGN;
    const WsLayout L = ws_layout(p, 0);
    if (L.total > kScratchBytes) return GLA_E_SCRATCH;
    rc = check_device();
    if (rc) return rc;
    // (every buffer the kernels keep there is written before it is read: nothing
    // in the scratch needs to start at zero)
    void* ws = nullptr;
    if (L.total > 0) {
        rc = scratch_on_current_device(&ws);
        if (rc) return rc;
    }
    return fwd_checked(p, L, q, k, v, g, h0, segment_ids, o, hT, ws, (hipStream_t)stream);
}

size_t gla_fwd_noalloc_max_scratch(void) { return kScratchBytes; }

int gla_bwd(const gla_problem* p, const void* q, const void* k, const void* v, const void* g,
            const float* h0, const int32_t* segment_ids, const void* dO, const float* dhT,
            void* dq, void* dk, void* dv, void* dg, float* dh0, void* ws, size_t ws_bytes,
            void* stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->T > 0 && (!q || !k || !v || !g || !dO || !dq || !dk || !dv || !dg)) return GLA_E_NULL;
    const void* ptrs[] = {q, k, v, g, h0, segment_ids, dO, dhT, dq, dk, dv, dg, dh0, ws};
    for (const void* x : ptrs)
        if (x && !aligned(x)) return GLA_E_ALIGN;
    const WsLayout L = ws_layout(p, 1);
    if (ws_bytes < L.total || (L.total > 0 && !ws)) return GLA_E_WORKSPACE;
    rc = check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (p->T == 0) return copy_state(dh0, dhT, p->B * p->H * p->d_k * p->d_v, st);

    char* w = (char*)ws;
    gla::PassArgs pa;
    memset(&pa, 0, sizeof pa);
    pa.q = q; pa.k = k; pa.v = v; pa.g = g; pa.dO = dO; pa.h0 = h0; pa.dhT = dhT; pa.seg = segment_ids;
    pa.dh0 = dh0;
    pa.ws_S = (float*)(w + L.S);
    pa.ws_dS = walk_bwd(p) ? nullptr : w + L.dS;
    pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.Hqk = p->H_qk;
    pa.ld_qk = ld_or_packed(p->ld_qk, p->H_qk * p->d_k);
    pa.ld_v = ld_or_packed(p->ld_v, p->H * p->d_v);
    pa.P = L.sp.P; pa.PL = L.sp.PL;
    if (pa.P > 1) {
        pa.L_out[0] = (float*)(w + L.pL0);
        pa.L_out[1] = (float*)(w + L.pL1);
        pa.S_in = (const float*)(w + L.pS);
        pa.dS_in = (const float*)(w + L.pdS);
        pa.D_out = (float*)(w + L.pD);
    }
    if (saves_states(p)) {
        pa.stamp = (const uint64_t*)(w + L.stamp);
        pa.expect = states_stamp(p, q, k, v, g, h0, segment_ids);
        pa.check_stamp = 1;
    }
    gla::RevArgs ra;
    memset(&ra, 0, sizeof ra);
    ra.q = q; ra.k = k; ra.v = v; ra.g = g; ra.dO = dO; ra.seg = segment_ids;
    ra.ws_S = w + L.S;
    ra.ws_dS = pa.ws_dS;
    ra.dhT = dhT; ra.dh0 = dh0;
    ra.dq = dq; ra.dk = dk; ra.dv = dv; ra.dg = dg;
    if (per_head_dqdk(p)) {
        ra.ws_dq = (float*)(w + L.dq);
        ra.ws_dk = (float*)(w + L.dk);
    }
    if (p->gate == GLA_GATE_SCALAR) {
        ra.ws_xs = (float*)(w + L.xs);
        ra.ws_bnd = (float*)(w + L.bnd);
    }
    ra.B = p->B; ra.T = p->T; ra.H = p->H; ra.Hqk = p->H_qk;
    ra.ld_qk = pa.ld_qk;
    ra.ld_v = pa.ld_v;
    ra.ld_dqk = ld_or_packed(p->ld_dqk, p->H_qk * p->d_k);
    ra.ld_dv = ld_or_packed(p->ld_dv, p->H * p->d_v);
    ra.P = pa.P; ra.PL = pa.PL; ra.dS_in = pa.dS_in;
    return dispatch<BwdF>(p, pa, ra, st) == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

// ---- short depthwise causal convolution
static int check_conv(const gla_conv_problem* p) {
    if (!p) return GLA_E_NULL;
    if (p->dtype != GLA_F32 && p->dtype != GLA_BF16) return GLA_E_DTYPE;
    if (p->B < 1 || p->T < 0 || p->C < 1) return GLA_E_SHAPE;
    if (p->K != 4) return GLA_E_UNSUPPORTED;
    if (p->C % 8 != 0) return GLA_E_UNSUPPORTED;
    int64_t bt, x;
    if (!mul_ok(p->B, p->T, &bt) || !mul_ok(bt, p->C, &x) || x > ((int64_t)1 << 40)) return GLA_E_SHAPE;
    // grid: C / 512 x T / 256 x B workgroups
    if (p->B > 65535 || (p->T + 255) / 256 > 65535 || (p->C + 511) / 512 > 65535) return GLA_E_SHAPE;
    return GLA_OK;
}

static gla::ConvArgs conv_args(const gla_conv_problem* p) {
    gla::ConvArgs a;
    memset(&a, 0, sizeof a);
    a.B = p->B; a.T = p->T; a.C = p->C;
    return a;
}

int gla_conv_workspace_size(const gla_conv_problem* p, size_t* bytes) {
    const int rc = check_conv(p);
    if (rc) return rc;
    if (!bytes) return GLA_E_NULL;
    *bytes = (size_t)gla::conv_partials(p->B, p->T) * (size_t)(p->K + 1) * (size_t)p->C * sizeof(float);
    return GLA_OK;
}

int gla_conv_fwd(const gla_conv_problem* p, const void* x, const float* w, const float* bias, void* y,
                 void* stream) {
    int rc = check_conv(p);
    if (rc) return rc;
    // (an empty row has no activations: their pointers may then be NULL)
    if (!w || (p->T > 0 && (!x || !y))) return GLA_E_NULL;
    const void* ptrs[] = {x, w, bias, y};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return GLA_E_ALIGN;
    rc = check_device();
    if (rc) return rc;
    if (p->T == 0) return GLA_OK;
    gla::ConvArgs a = conv_args(p);
    a.x = x; a.w = w; a.bias = bias; a.y = y;
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e = p->dtype == GLA_BF16 ? gla::launch_conv_fwd<gla::bf16>(a, st)
                                              : gla::launch_conv_fwd<float>(a, st);
    return e == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

int gla_conv_bwd(const gla_conv_problem* p, const void* x, const float* w, const float* bias,
                 const void* dy, void* dx, float* dw, float* db, void* ws, size_t ws_bytes,
                 void* stream) {
    int rc = check_conv(p);
    if (rc) return rc;
    if (!w || !dw || (p->T > 0 && (!x || !dy || !dx))) return GLA_E_NULL;
    const void* ptrs[] = {x, w, bias, dy, dx, dw, db, ws};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return GLA_E_ALIGN;
    size_t need = 0;
    gla_conv_workspace_size(p, &need);
    if (ws_bytes < need || (need > 0 && !ws)) return GLA_E_WORKSPACE;
    rc = check_device();
    if (rc) return rc;
    gla::ConvArgs a = conv_args(p);
    a.x = x; a.w = w; a.bias = bias; a.dy = dy; a.dx = dx; a.dw = dw; a.db = db; a.ws = (float*)ws;
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e = p->dtype == GLA_BF16 ? gla::launch_conv_bwd<gla::bf16>(a, st)
                                              : gla::launch_conv_bwd<float>(a, st);
    return e == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

// ---- gated delta rule
int gla_delta_workspace_size(const gla_delta_problem* p, int for_backward, size_t* bytes) {
    const int rc = check_delta(p);
    if (rc) return rc;
    if (!bytes) return GLA_E_NULL;
    *bytes = for_backward ? delta_scratch_bytes(p) : delta_ws_bytes(p);
    return GLA_OK;
}

int gla_delta_fwd(const gla_delta_problem* p, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* h0, const int32_t* segment_ids, void* o, float* hT,
                  void* ws, size_t ws_bytes, void* stream) {
    int rc = check_delta(p);
    if (rc) return rc;
    if (p->T > 0 && (!q || !k || !v || !g || !beta || !o)) return GLA_E_NULL;
    const void* ptrs[] = {q, k, v, g, beta, h0, segment_ids, o, hT, ws};
    for (const void* x : ptrs)
        if (x && !aligned(x)) return GLA_E_ALIGN;
    const size_t need = delta_ws_bytes(p);
    if (ws_bytes < need || (need > 0 && !ws)) return GLA_E_WORKSPACE;
    rc = check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (p->T == 0) return copy_state(hT, h0, p->B * p->H * p->d_k * p->d_v, st);
    gla::DeltaArgs a = delta_args(p, q, k, v, g, beta, segment_ids, ws);
    a.h0 = h0; a.o = o; a.hT = hT;
    const hipError_t e = p->dtype == GLA_BF16 ? gla::launch_delta_fwd<gla::bf16>(a, st)
                                              : gla::launch_delta_fwd<float>(a, st);
    return e == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

int gla_delta_bwd(const gla_delta_problem* p, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* h0, const int32_t* segment_ids, const void* dO,
                  const float* dhT, void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dh0,
                  void* ws, size_t ws_bytes, void* scratch, size_t scratch_bytes, void* stream) {
    int rc = check_delta(p);
    if (rc) return rc;
    if (p->T > 0 && (!q || !k || !v || !g || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta))
        return GLA_E_NULL;
    const void* ptrs[] = {q, k, v, g, beta, h0, segment_ids, dO, dhT, dq, dk, dv, dg, dbeta, dh0, ws, scratch};
    for (const void* x : ptrs)
        if (x && !aligned(x)) return GLA_E_ALIGN;
    const size_t need = delta_ws_bytes(p), need2 = delta_scratch_bytes(p);
    if (ws_bytes < need || (need > 0 && !ws)) return GLA_E_WORKSPACE;
    if (scratch_bytes < need2 || (need2 > 0 && !scratch)) return GLA_E_WORKSPACE;
    rc = check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (p->T == 0) return copy_state(dh0, dhT, p->B * p->H * p->d_k * p->d_v, st);
    gla::DeltaArgs a = delta_args(p, q, k, v, g, beta, segment_ids, ws);
    a.h0 = h0; a.dO = dO;
    a.dhT = dhT; a.dq = dq; a.dk_out = dk; a.dv_out = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.ws2 = (float*)scratch;
    a.ws2_chunk = gla::delta_bwd_floats_per_chunk(p->d_k, p->d_v, a.states_in_ws);
    a.check_stamp = (p->flags & GLA_DELTA_WS_FROM_FWD) != 0;
    const hipError_t e = p->dtype == GLA_BF16 ? gla::launch_delta_bwd<gla::bf16>(a, st)
                                              : gla::launch_delta_bwd<float>(a, st);
    return e == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

// ---- output norm and gate
int gla_norm_gate_workspace_size(const gla_norm_gate_problem* p, size_t* bytes) {
    const int rc = check_norm(p);
    if (rc) return rc;
    if (!bytes) return GLA_E_NULL;
    int64_t np = 0;
    (void)norm_dispatch(p, [&](auto t, auto d) {
        np = gla::norm_gate_partials<decltype(t), decltype(d)::value>(norm_rows(p));
        return hipSuccess;
    });
    *bytes = (size_t)np * (size_t)p->d * sizeof(float);
    return GLA_OK;
}

int gla_norm_gate_fwd(const gla_norm_gate_problem* p, const void* o, const void* z, const float* gamma,
                      void* y, void* stream) {
    int rc = check_norm(p);
    if (rc) return rc;
    if (!gamma || (p->T > 0 && (!o || !z || !y))) return GLA_E_NULL;
    const void* ptrs[] = {o, z, gamma, y};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return GLA_E_ALIGN;
    rc = check_device();
    if (rc) return rc;
    gla::NormArgs a;
    memset(&a, 0, sizeof a);
    a.o = o; a.z = z; a.gamma = gamma; a.y = y; a.rows = norm_rows(p); a.eps = p->eps;
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e = norm_dispatch(p, [&](auto t, auto d) {
        return gla::launch_norm_gate_fwd<decltype(t), decltype(d)::value>(a, st);
    });
    return e == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

int gla_norm_gate_bwd(const gla_norm_gate_problem* p, const void* o, const void* z, const float* gamma,
                      const void* dy, void* d_o, void* dz, float* dgamma, void* ws, size_t ws_bytes,
                      void* stream) {
    int rc = check_norm(p);
    if (rc) return rc;
    if (!gamma || !dgamma || (p->T > 0 && (!o || !z || !dy || !d_o || !dz))) return GLA_E_NULL;
    const void* ptrs[] = {o, z, gamma, dy, d_o, dz, dgamma, ws};
    for (const void* q : ptrs)
        if (q && !aligned(q)) return GLA_E_ALIGN;
    size_t need = 0;
    gla_norm_gate_workspace_size(p, &need);
    if (ws_bytes < need || (need > 0 && !ws)) return GLA_E_WORKSPACE;
    rc = check_device();
    if (rc) return rc;
    gla::NormArgs a;
    memset(&a, 0, sizeof a);
    a.o = o; a.z = z; a.gamma = gamma; a.dy = dy; a.d_o = d_o; a.dz = dz; a.dgamma = dgamma;
    a.ws = (float*)ws; a.rows = norm_rows(p); a.eps = p->eps;
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e = norm_dispatch(p, [&](auto t, auto d) {
        return gla::launch_norm_gate_bwd<decltype(t), decltype(d)::value>(a, st);
    });
    return e == hipSuccess ? GLA_OK : GLA_E_LAUNCH;
}

const char* gla_status_str(int s) {
    switch (s) {
        case GLA_OK: return "ok";
        case GLA_E_NULL: return "a required pointer is NULL";
        case GLA_E_SHAPE: return "sizes inconsistent or out of range";
        case GLA_E_DTYPE: return "unknown dtype or gate kind";
        case GLA_E_UNSUPPORTED: return "no kernel for this d_k / d_v / chunk (convolution: K / channel count)";
        case GLA_E_ALIGN: return "a pointer is not 16-byte aligned";
        case GLA_E_WORKSPACE: return "workspace missing or too small";
        case GLA_E_DEVICE: return "no HIP device, or the current device is not gfx950";
        case GLA_E_LAUNCH: return "kernel launch failed";
        case GLA_E_SCRATCH: return "the problem needs more workspace than the fixed scratch of gla_fwd_noalloc holds";
        default: return "unknown status";
    }
}

int gla_version(void) { return 200; }

}  // extern "C"
