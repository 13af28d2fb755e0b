// kda_kernels.hip -- gfx950 kernels of the KDA decode step.
//
// The step per (stream m, head h), "GLM-5.3 deep dive" 8.2.3 Eq. 1 in the
// order of 8.2.6 (fade, predict, correct, read):
//
//   S'  = Diag(alpha) S                         fade rows (key channels)
//   u   = S'^T k^        w = S'^T q^            both reductions in ONE sweep
//   d   = beta (v - u)                          delta correction
//   S'' = S' + k^ d^T                           rank-1 write, stored in place
//   o   = S''^T q^ = w + d (k^ . q^)            read (same value, no 2nd sweep)
//
// where q^, k^ are the L2-normalised (eps 1e-6) conv+SiLU outputs and q^
// carries the q scale (8.2.4 steps 2 and 6, 8.2.6 implementation notes).
//
// Design (MI355X, CDNA4, wave64):
//  * The step is a matrix-vector update at < 2 FLOP/byte: HBM-bound, no MFMA.
//  * One workgroup owns one head (or 1/NSPLIT of its value columns).  Each
//    lane owns VEC consecutive value columns of RPL key rows and holds them in
//    VGPRs for the whole step, so the state is read once and written once and
//    LDS never holds it (LDS holds the q/k/v/alpha vectors and per-wave
//    partial sums, at most ~19 KiB at 16 waves: occupancy is set by VGPRs).
//  * Loads and stores of the state are 16 bytes per lane; a wave covers whole
//    contiguous rows (512 B f32 / 256 B bf16), so every access is coalesced.
//  * All state loads are issued before the conv prologue is computed; the
//    barriers in between only fence LDS, so the loads stay in flight.  On
//    f32 grids of 2048 heads and more the odd workgroups (those of the odd
//    XCDs) issue theirs after the conv instead, so that the two XCDs of each
//    pair request their heads' state out of phase.
//  * Reductions over key rows: in-lane FMAs, then a butterfly across the lanes
//    that share columns, then (NWAVES > 1) one exchange through LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ------------------------------------------------------------ decode step --
//
// TS      state storage: float or uint16_t (bf16 bits)
// D       head width (dk = dv)
// NSPLIT  workgroups per head; each owns D/NSPLIT value columns and every key
//         row of them, so the reductions over key rows stay in one workgroup
// NWAVES  waves per workgroup
// VEC     state elements per lane access (16 bytes for D = 128)
// RMAP    0: a workgroup access covers consecutive rows (waves side by side);
//         1: each wave owns a contiguous band of rows
// FUSED   true: conv prologue from bf16 x + conv state; false: f32 q|k|v input
// XG      XCD-aware workgroup order: keep the NSPLIT workgroups of a head on
//         one XCD (they read the same q/k inputs, which then come from that
//         XCD's L2); with whole heads, alternate consecutive workgroups
//         between the two halves of the heads (block_unit)
// WT      state stores with agent scope as well as non-temporal (store_sc1)
template <typename TS, int D, int NSPLIT, int NWAVES, int VEC, int RMAP>
struct Geo {
    static constexpr int NT = NWAVES * 64;
    static constexpr int COLS = D / NSPLIT;          // value columns of one workgroup
    static constexpr int CG = COLS / VEC;            // lanes across one row segment
    static_assert(COLS % VEC == 0 && CG >= 1 && 64 % CG == 0, "row segment must tile the wave");
    static constexpr int RPW = 64 / CG;              // rows per wave access
    static constexpr int RS = RPW * NWAVES;          // rows per workgroup access
    static_assert(RS <= D && D % RS == 0, "row slices must tile the key axis");
    static constexpr int RPL = D / RS;               // rows per lane
    // the prologue works on groups of 4 channels (8 bytes of bf16)
    static constexpr int GQ = D / 4;                 // q groups (then k, then own v)
    static constexpr int NG = 2 * GQ + COLS / 4;     // prologue groups
    static constexpr int QK_PER_SPLIT = 2 * GQ / NSPLIT;  // q/k groups each split writes back
    static_assert(COLS % 4 == 0 && (2 * GQ) % NSPLIT == 0, "channel groups must tile the split");
    static_assert(NG <= NT - D / 4, "prologue and alpha lanes must not overlap");
    static constexpr int IO_VEC = VEC;               // state elements per lane access
    static constexpr int NSPLIT_ = NSPLIT;
    typedef Chunk<TS, VEC> IO;
    typedef typename IO::raw_t raw_t;
    // key row of access t of (wave wv, row-in-wave rw)
    static __device__ __forceinline__ int row(int wv, int rw, int t) {
        return RMAP == 0 ? wv * RPW + rw + RS * t : (wv * RPL + t) * RPW + rw;
    }
};



// Workgroup b -> (unit = m*H + h, split).  Plain: the splits of a unit are
// consecutive workgroups.  XG: workgroups are handed to the 8 XCDs round
// robin, so within each run of 8*NSPLIT workgroups, those on one XCD are the
// NSPLIT splits of one unit; a ragged tail of units falls back to plain.
// XG with whole heads (NSPLIT 1): consecutive workgroups alternate between
// the two halves of the heads, so the even XCDs stream the first half of the
// states upwards (b -> b/2) and the odd ones the second half downwards
// (b -> units - 1 - b/2).  Measured on MI355X for the 16-wave f32 grid (34
// layers, us per layer, plain / alternating, both halves upwards): M = 32
// 47.8 / 46.4, M = 48 72.1 / 69.9, M = 64 94.5 / 91.1, M = 128 186.0 /
// 176.1; with the states placed 3 GB further into memory M = 32 47.1 /
// 46.8.  The second half downwards, with the staggered state requests (one
// process, alternating builds, M = 32): plain 46.9 -> 46.8, gated 47.6 ->
// 46.9, layer 47.4 -> 47.2.  The 4-wave grids (bf16; one round of f32) and
// XCD-contiguous heads (each XCD an eighth of the states) are slower.
template <int NSPLIT, bool XG>
__device__ __forceinline__ void block_unit(int b, int units, int& unit, int& split) {
    if constexpr (XG && NSPLIT == 1) {
        if ((units & 1) == 0) {
            unit = (b & 1) ? units - 1 - (b >> 1) : (b >> 1);
            split = 0;
            return;
        }
    }
    if constexpr (XG && NSPLIT > 1) {
        constexpr int GB = 8 * NSPLIT;
        const int full = units >> 3;
        if (b < full * GB) {
            const int g = b / GB, r = b - g * GB;
            unit = g * 8 + (r & 7);
            split = r >> 3;
            return;
        }
        b -= full * GB;
        unit = full * 8 + b / NSPLIT;
        split = b - (b / NSPLIT) * NSPLIT;
        return;
    }
    unit = b / NSPLIT;
    split = b - unit * NSPLIT;
}

// First channel (in [0, 3HD)) of prologue group g of head h, split `split`:
// groups [0, GQ) are q, [GQ, 2GQ) k, the rest this split's v columns.
template <class G, int D>
__device__ __forceinline__ size_t group_channel(int g, int h, int split, size_t HD) {
    const int tensor = g < G::GQ ? 0 : (g < 2 * G::GQ ? 1 : 2);
    const int within = tensor < 2 ? 4 * (g - tensor * G::GQ) : split * G::COLS + 4 * (g - 2 * G::GQ);
    return (size_t)tensor * HD + (size_t)h * D + within;
}

__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(uint16_t* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// One unit's small inputs, held in VGPRs from their loads to the conv.
struct Pro {
    u32x2 xv, t0, t1, t2;      // raw bf16 x and taps of 4 channels (FUSED)
    u32x4 w01, w23;            // their 4 conv taps each
    f32x4 q0;                  // f32 q|k|v of 4 channels (!FUSED)
    f32x4 av;                  // 4 alpha values (MODE 0)
    u32x2 fv;                  // 4 raw bf16 gate values (MODE >= 1)
    f32x4 bias;                // their dt_bias
    float alog;                // A_log of the head
    float b;                   // beta of the unit (MODE 0), its logit (MODE >= 1)
    float og, nw;              // output gate and norm weight of column tid (MODE 2)
};

// LDS of one workgroup: conv outputs (q at [0, D), k at [D, 2D), this
// workgroup's v columns at [2D, 2D + COLS)), alpha, per-wave partial sums,
// and the delta vector.
template <class G, int D>
struct Smem {
    __attribute__((aligned(16))) float z[2 * D + G::COLS];
    __attribute__((aligned(16))) float a[D];
    float red[G::NT / 64][2][G::COLS];
    float d[G::COLS];
    float w[G::COLS];
};

// Issue the small loads of unit `unit`: lanes [0, NG) own 4 channels each
// (q, k, this split's v); the last D/4 lanes of the workgroup load alpha.
template <class G, int D, bool FUSED, int MODE>
__device__ __forceinline__ void load_pro(Pro& in, const Ptrs& p, int unit, int split) {
    const int tid = threadIdx.x;
    const int m = unit / p.H, h = unit - m * p.H;
    const size_t HD = (size_t)p.H * D, C3 = 3 * HD;
    if (tid < G::NG) {
        const size_t ch = group_channel<G, D>(tid, h, split, HD);
        if constexpr (FUSED) {
            in.xv = ld8(p.x + (size_t)m * C3 + ch);
            const uint16_t* ci = p.conv_in + (size_t)m * 3 * C3 + ch;
            in.t0 = ld8(ci);
            in.t1 = ld8(ci + C3);
            in.t2 = ld8(ci + 2 * C3);
            const u32x4* wp = reinterpret_cast<const u32x4*>(p.conv_w + 4 * ch);
            in.w01 = wp[0];
            in.w23 = wp[1];
        } else {
            in.q0 = *reinterpret_cast<const f32x4*>(p.qkv + (size_t)m * C3 + ch);
        }
    }
    const int ag = tid - (G::NT - D / 4);
    if constexpr (MODE == 0) {
        if (ag >= 0) in.av = *reinterpret_cast<const f32x4*>(p.alpha + (size_t)unit * D + 4 * ag);
        in.b = p.beta[unit];
    } else {
        if (ag >= 0) {
            in.fv = ld8(p.fgate + (size_t)unit * D + 4 * ag);
            in.bias = *reinterpret_cast<const f32x4*>(p.dt_bias + (size_t)h * D + 4 * ag);
        }
        in.alog = p.A_log[h];
        in.b = bf16_lo(p.blogit[unit]);
        if constexpr (MODE == 2) {
            if (tid < D) {
                in.og = bf16_lo(p.ogate[(size_t)unit * D + tid]);
                in.nw = p.norm_w[tid];
            }
        }
    }
}

// Forget gate of one channel, "GLM-5.3 deep dive" 8.2.3 (the gate as fla
// computes it): g = lb * sigmoid(exp(A) (f + b)) with a lower bound lb < 0,
// or g = -exp(A) softplus(f + b); alpha = exp(g).
__device__ __forceinline__ float gate_alpha(float fb, float eA, int kind, float lb) {
    float g;
    if (kind == 0) {
        g = lb / (1.0f + expf(-eA * fb));
    } else {
        const float sp = fb > 0.0f ? fb + log1pf(expf(-fb)) : log1pf(expf(fb));
        g = -eA * sp;
    }
    return expf(g);
}

// Issue every state load of this lane for unit `unit`.  live == false issues
// the same number of loads, all from the unit's first row segment (a
// placeholder that keeps the instruction stream, and its wait counts, fixed).
template <typename TS, class G, int D, int T0 = 0, int T1 = G::RPL>
__device__ __forceinline__ void load_state(typename G::raw_t (&raw)[G::RPL], const Ptrs& p, int unit,
                                           int split, bool live) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cg = lane % G::CG, rw = lane / G::CG;
    const TS* st = static_cast<const TS*>(p.state) + (size_t)unit * D * D + split * G::COLS + cg * G::IO_VEC;
#pragma unroll
    for (int t = T0; t < T1; ++t) raw[t] = G::IO::load(st + (live ? (size_t)G::row(wv, rw, t) * D : 0));
}

// Conv + SiLU of one unit's channels into LDS and the conv state shift;
// alpha into LDS.  The caller places a barrier after it.
template <class G, int D, bool FUSED, int MODE>
__device__ __forceinline__ void conv_unit(const Pro& in, const Ptrs& p, int unit, int split, Smem<G, D>& sm) {
    constexpr int NT = G::NT;
    const int tid = threadIdx.x;
    const int m = unit / p.H, h = unit - m * p.H;
    const size_t HD = (size_t)p.H * D, C3 = 3 * HD;

    // ---- conv + SiLU into LDS; advance the conv state ----
    if (tid < G::NG) {
        f32x4 z0;
        if constexpr (FUSED) {
            // channel 2c uses the low halves, channel 2c+1 the high halves;
            // weights: 4 taps per channel, two channels per 16-byte word
            z0 = f32x4{conv_silu(u32x2{in.w01.x, in.w01.y}, bf16_lo(in.t0.x), bf16_lo(in.t1.x),
                                 bf16_lo(in.t2.x), bf16_lo(in.xv.x)),
                       conv_silu(u32x2{in.w01.z, in.w01.w}, bf16_hi(in.t0.x), bf16_hi(in.t1.x),
                                 bf16_hi(in.t2.x), bf16_hi(in.xv.x)),
                       conv_silu(u32x2{in.w23.x, in.w23.y}, bf16_lo(in.t0.y), bf16_lo(in.t1.y),
                                 bf16_lo(in.t2.y), bf16_lo(in.xv.y)),
                       conv_silu(u32x2{in.w23.z, in.w23.w}, bf16_hi(in.t0.y), bf16_hi(in.t1.y),
                                 bf16_hi(in.t2.y), bf16_hi(in.xv.y))};
            // every split reads all q/k taps; each writes back its own share
            // of them, and its own v taps (with NSPLIT > 1 the host requires
            // conv_out != conv_in)
            if (tid >= 2 * G::GQ || G::NSPLIT_ == 1 || tid / G::QK_PER_SPLIT == split) {
                uint16_t* co = p.conv_out + (size_t)m * 3 * C3 + group_channel<G, D>(tid, h, split, HD);
                st8(co, in.t1);
                st8(co + C3, in.t2);
                st8(co + 2 * C3, in.xv);
            }
        } else {
            z0 = in.q0;
        }
        reinterpret_cast<f32x4*>(sm.z)[tid] = z0;
    }
    const int ag = tid - (NT - D / 4);
    if (ag >= 0) {
        if constexpr (MODE == 0) {
            reinterpret_cast<f32x4*>(sm.a)[ag] = in.av;
        } else {
            const float eA = expf(in.alog);
            reinterpret_cast<f32x4*>(sm.a)[ag] =
                f32x4{gate_alpha(bf16_lo(in.fv.x) + in.bias.x, eA, p.gate_kind, p.lower_bound),
                      gate_alpha(bf16_hi(in.fv.x) + in.bias.y, eA, p.gate_kind, p.lower_bound),
                      gate_alpha(bf16_lo(in.fv.y) + in.bias.z, eA, p.gate_kind, p.lower_bound),
                      gate_alpha(bf16_hi(in.fv.y) + in.bias.w, eA, p.gate_kind, p.lower_bound)};
        }
    }
}

// The rest of one unit, after conv_unit and a barrier: norms, fade and both
// reductions, one cross-wave exchange, delta correction, readout, rank-1
// write and the stores.  PK (bf16 state): the state stays in its packed
// registers; the reductions and the write each unpack the rows again (the
// same products in the same order, so the same results) instead of
// holding them as f32 -- 64 VGPRs instead of 112, 8 workgroups per CU.
template <typename TS, class G, int D, int MODE, bool WT, bool PK = false>
__device__ __forceinline__ void update_unit(const Pro& in, typename G::raw_t (&raw)[G::RPL], const Ptrs& p,
                                            int unit, int split, Smem<G, D>& sm) {
    constexpr int NT = G::NT, COLS = G::COLS, CG = G::CG, RPL = G::RPL, VEC = G::IO_VEC;
    constexpr int NWAVES = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int cg = lane % CG, rw = lane / CG;
    const int col0 = split * COLS + cg * VEC;
    float* const s_q = sm.z;
    float* const s_k = sm.z + D;
    float* const s_v = sm.z + 2 * D;

    // beta, or (MODE >= 1) the sigmoid of its logit ("GLM-5.3 deep dive"
    // 8.2.4 step 4)
    const float b = MODE == 0 ? in.b : 1.0f / (1.0f + expf(-in.b));

    // ---- L2 norms and k^.q^ (every wave reduces the same D values) ----
    float sqq = 0.0f, skk = 0.0f, sqk = 0.0f;
#pragma unroll
    for (int i = lane; i < D; i += 64) {
        const float qv = s_q[i], kv = s_k[i];
        sqq = fmaf(qv, qv, sqq);
        skk = fmaf(kv, kv, skk);
        sqk = fmaf(qv, kv, sqk);
    }
    sqq = wave_sum(sqq);
    skk = wave_sum(skk);
    sqk = wave_sum(sqk);
    const float rq = p.scale * rsqrtf(sqq + 1e-6f);
    const float rk = rsqrtf(skk + 1e-6f);
    const float kq = sqk * rq * rk;                    // k^ . q^

    // ---- fade, and the two reductions over this lane's rows ----
    static_assert(!PK || sizeof(TS) == 2, "the packed form is for a bf16 state");
    float sreg[PK ? 1 : RPL][VEC], kk[PK ? 1 : RPL];
    float u[VEC], wq[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) { u[e] = 0.0f; wq[e] = 0.0f; }
    if constexpr (PK) {
        // four rows between scheduling fences, so that the rows' LDS
        // scalars are not all fetched (and held) at once
#pragma unroll
        for (int t = 0; t < RPL; ++t) {
            if (t % 4 == 0) __builtin_amdgcn_sched_barrier(0);
            const int i = G::row(wv, rw, t);
            const float a = sm.a[i], qq = s_q[i] * rq, k_ = s_k[i] * rk;
            float s4[VEC];
            G::IO::unpack(raw[t], s4);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float sv = s4[e] * a;
                u[e] = fmaf(sv, k_, u[e]);
                wq[e] = fmaf(sv, qq, wq[e]);
            }
        }
    } else
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
        const int i = G::row(wv, rw, t);
        const float a = sm.a[i], qq = s_q[i] * rq;
        kk[t] = s_k[i] * rk;
        G::IO::unpack(raw[t], sreg[t]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float sv = sreg[t][e] * a;
            sreg[t][e] = sv;
            u[e] = fmaf(sv, kk[t], u[e]);
            wq[e] = fmaf(sv, qq, wq[e]);
        }
    }
    // lanes that share columns differ in the bits above log2(CG).  Column
    // splits (small grids, latency-bound) take the row and half-wave swaps
    // on the VALU; whole heads keep the LDS permutes, which measured faster
    // on the bandwidth-bound grids (M = 32 f32 48.2 against 48.3-48.4 us).
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        if constexpr (G::NSPLIT_ > 1) {
            u[e] = xor_reduce_from<CG>(u[e]);
            wq[e] = xor_reduce_from<CG>(wq[e]);
        } else {
#pragma unroll
            for (int off = CG; off < 64; off <<= 1) {
                u[e] += __shfl_xor(u[e], off, 64);
                wq[e] += __shfl_xor(wq[e], off, 64);
            }
        }
    }

    // ---- delta correction and readout ----
    float d[VEC];
    uint16_t* const ou = p.o + (size_t)unit * D + split * COLS;
    if constexpr (NWAVES > 1) {
        // partial sums of every wave to LDS; one thread per column adds the
        // u partials and forms d, another adds the w partials; d goes back
        // to every lane through LDS, and o = w + d (k^.q^) is written after
        static_assert(2 * COLS <= NT, "u and w sums need 2*COLS threads");
        if (rw == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                sm.red[wv][0][cg * VEC + e] = u[e];
                sm.red[wv][1][cg * VEC + e] = wq[e];
            }
        }
        lds_barrier();
        if (tid < COLS) {
            float U = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) U += sm.red[w][0][tid];
            sm.d[tid] = b * (s_v[tid] - U);
        } else if (tid < 2 * COLS) {
            float W = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) W += sm.red[w][1][tid - COLS];
            sm.w[tid - COLS] = W;
        }
        lds_barrier();
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = sm.d[cg * VEC + e];
        if (MODE != 2 && tid < COLS) ou[tid] = (uint16_t)f32_to_bf16_rne(fmaf(sm.d[tid], kq, sm.w[tid]));
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = b * (s_v[cg * VEC + e] - u[e]);
        if (MODE != 2 && rw == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                ou[cg * VEC + e] = (uint16_t)f32_to_bf16_rne(fmaf(d[e], kq, wq[e]));
        }
    }

    // ---- rank-1 write and store ----
    TS* const st = static_cast<TS*>(p.state) + (size_t)unit * D * D;
    const auto rs = stream_rsrc(st, D * D * (int)sizeof(TS));   // used with WT only
    if constexpr (PK) {
        // the faded row formed again from the packed bf16 (the products
        // the reductions used), then the rank-1 write.  The raw pairs and
        // the store offsets' base pass through empty asm statements, so the
        // compiler neither keeps the reductions' unpacked rows (64 VGPRs)
        // nor the load addresses live until here.
        int lo = G::row(wv, rw, 0) * D + col0;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int t = 0; t < RPL; ++t) asm volatile("" : "+v"(raw[t]));
#pragma unroll
        for (int t = 0; t < RPL; ++t) {
            if (t % 4 == 0) __builtin_amdgcn_sched_barrier(0);
            const int i = G::row(wv, rw, t);
            const float a = sm.a[i], k_ = s_k[i] * rk;
            float s4[VEC];
            G::IO::unpack(raw[t], s4);
#pragma unroll
            for (int e = 0; e < VEC; ++e) s4[e] = fmaf(k_, d[e], s4[e] * a);
            const int off = lo + (G::row(0, 0, t) - G::row(0, 0, 0)) * D;
            if constexpr (WT)
                G::IO::store_sc1(rs, off * (int)sizeof(TS), s4);
            else
                G::IO::store(st + off, s4);
        }
    } else
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) sreg[t][e] = fmaf(kk[t], d[e], sreg[t][e]);
        const int off = G::row(wv, rw, t) * D + col0;
        if constexpr (WT)
            G::IO::store_sc1(rs, off * (int)sizeof(TS), sreg[t]);
        else
            G::IO::store(st + off, sreg[t]);
    }

    // ---- gated RMSNorm of the head's outputs (MODE 2), "GLM-5.3 deep dive"
    // 8.2.4 step 7: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(g), from the
    // unrounded o; the state stores above are already in flight ----
    if constexpr (MODE == 2) {
        constexpr int HW = (D + 63) / 64;              // waves that hold one column each
        static_assert(G::NSPLIT_ == 1 && HW <= NWAVES, "the output norm needs the whole head");
        if constexpr (NWAVES == 1) {
            // d and w are still per lane: put them in LDS like the
            // cross-wave path does
            if (rw == 0) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    sm.d[cg * VEC + e] = d[e];
                    sm.w[cg * VEC + e] = wq[e];
                }
            }
            lds_barrier();
        }
        float oj = 0.0f;
        if (tid < D) oj = fmaf(sm.d[tid], kq, sm.w[tid]);
        const float ss = wave_sum(oj * oj);
        if (wv < HW && lane == 0) sm.red[wv][0][0] = ss;
        lds_barrier();
        if (tid < D) {
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < HW; ++w) tot += sm.red[w][0][0];
            const float r = rsqrtf(tot / (float)D + p.norm_eps);
            const float y = oj * r * in.nw / (1.0f + expf(-in.og));
            ou[tid] = (uint16_t)f32_to_bf16_rne(y);
        }
    }
}

// One workgroup per (unit, split): grid M*H*NSPLIT.  The small prologue
// loads go first, then every state load of the lane (all in flight
// together); the conv + SiLU runs while the state is still arriving.
// Staggered (f32 state, WT grids: 2048 heads and more): the odd workgroups
// -- dealt round robin to the 8 XCDs, those of the odd XCDs -- request their
// state only after the conv, so half the grid's state requests trail the
// other half's.  Measured (34 layers in a hipGraph, one process,
// alternating builds, us per layer at M = 32): plain 47.25 -> 46.74-46.92,
// gated 48.04 -> 47.06, layer 47.48 -> 47.36; odd pairs of workgroups late
// 47.45, the first round's odd workgroups only 47.68-47.99.  bf16 grids
// (M = 32: 26.6 against 25.9 us; M = 128: 96.3 against 95.7) and the
// single-round grids of M = 8 (f32 13.9 against 12.3) lose, so they keep
// the plain requests.
// PK (bf16 state, see update_unit): half of each lane's state loads before
// the conv and half after it, so the conv's inputs and the state's packed
// registers fit 64 VGPRs together (8 workgroups per CU).
template <typename TS, int D, int NSPLIT, int NWAVES, int VEC, int RMAP, bool FUSED, bool XG, int MODE, bool WT,
          bool PK = false>
__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(PK ? 8 : 1)))
void decode_kernel(const Ptrs p, const int units)
{
    typedef Geo<TS, D, NSPLIT, NWAVES, VEC, RMAP> G;
    __shared__ Smem<G, D> sm;
    int unit, split;
    block_unit<NSPLIT, XG>((int)blockIdx.x, units, unit, split);
    Pro in;
    load_pro<G, D, FUSED, MODE>(in, p, unit, split);
    // keep the scheduler from sinking these loads below the state loads:
    // the conv prologue then waits only for them, not for the state
    __builtin_amdgcn_sched_barrier(0);
    typename G::raw_t raw[G::RPL];
    constexpr bool STAG = WT && sizeof(TS) == 4;
    const bool late = STAG && (blockIdx.x & 1) != 0;
    if constexpr (PK) load_state<TS, G, D, 0, G::RPL / 2>(raw, p, unit, split, true);
    else if (!late) load_state<TS, G, D>(raw, p, unit, split, true);
    __builtin_amdgcn_sched_barrier(0);
    conv_unit<G, D, FUSED, MODE>(in, p, unit, split, sm);
    lds_barrier();
    if constexpr (PK) load_state<TS, G, D, G::RPL / 2, G::RPL>(raw, p, unit, split, true);
    else if (late) load_state<TS, G, D>(raw, p, unit, split, true);
    update_unit<TS, G, D, MODE, WT, PK>(in, raw, p, unit, split, sm);
}

// ------------------------------------------------------- T tokens per launch --
//
// fla's decode mode runs inputs of up to 64 tokens through the recurrent form
// ("GLM-5.3 deep dive" 8.2.6): here one workgroup owns one head for all T
// tokens of a stream, so the state is read once and written once per launch
// instead of once per token.
//
// Only the fade, the reductions and the rank-1 write depend on the state.
// Everything else (conv + SiLU, the norms, alpha, beta) is computed for a
// chunk of TC tokens at once: the workgroup's threads take the chunk's
// (token j, channel group g) items in turn, each computing the 4 channels of
// group g for token j from the three previous raw inputs of those channels
// (from x, or from the conv state for the first three tokens); one wave per
// token then forms its norms.  The serial loop over the chunk's tokens then
// touches only LDS and the state registers, with two barriers per token.
// The first chunk is computed before the state is requested: a wave's loads
// complete in order, so inputs requested after the state would wait for it,
// and requested together with it they would hold registers beside it.

template <typename TS, int D, int NWAVES, int VEC, int RMAP, int TCMAX = 16>
struct MultiGeo {
    typedef Geo<TS, D, 1, NWAVES, VEC, RMAP> G;
    static constexpr int NGT = 3 * D / 4;            // channel groups of one token
    static constexpr int TC = TCMAX;                 // tokens per chunk
    static constexpr int ITEMS = (TC * NGT + G::NT - 1) / G::NT;   // (token, group) items per thread
    static constexpr int ZW = 3 * D;                 // conv outputs of one token: q, k, v
};

template <class MG, int D>
struct MultiSmem {
    __attribute__((aligned(16))) float z[MG::TC][MG::ZW];   // conv outputs q|k|v of the chunk's tokens
    __attribute__((aligned(16))) float a[MG::TC][D];        // alpha
    float b[MG::TC];                                         // beta
    float rq[MG::TC], rk[MG::TC];                            // scale / |q|, 1 / |k| (the L2 norms)
    float kq[MG::TC];                                        // k^.q^ / rk
    float red[MG::G::NT / 64][2][D];                         // per-wave partial column sums (k, q)
    float d[D];                                              // rk * delta of the current token
    float w[D];                                              // S^T q^ of the current token
};

// Raw input (4 bf16 channels at channel offset ch) at sequence position pos
// of stream m: pos < 0 is a cached tap (tap 3 + pos of conv_in), pos >= 0 is
// token pos of x.
__device__ __forceinline__ u32x2 seq_input(const Ptrs& p, int T, int m, size_t C3, size_t ch, int pos) {
    if (pos < 0) return ld8(p.conv_in + (size_t)m * 3 * C3 + (size_t)(3 + pos) * C3 + ch);
    return ld8(p.x + ((size_t)m * T + pos) * C3 + ch);
}

// Conv, alpha, beta and norms of tokens [c0, c0 + n) into LDS.
struct NoLoads {
    __device__ __forceinline__ void operator()() const {}
};

// KEEP: the items also leave the raw inputs of the conv state after T tokens
// (positions T-3 .. T-1) in sm.cs, so that it is written at the end without
// loading them again (the chunk form's single chunk).
template <class MG, int D, bool ALL = true, class SM = MultiSmem<MG, D>, class After = NoLoads, bool KEEP = false>
__device__ __forceinline__ void multi_chunk(const Ptrs& p, int T, int m, int h, int c0, int n, SM& sm,
                                            After after = After()) {
    typedef typename MG::G G;
    constexpr int IT = MG::ITEMS;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const size_t HD = (size_t)p.H * D, C3 = 3 * HD;
    // ALL: every item's loads go out before any is used (the chunk waits
    // for memory once); otherwise item by item, which holds a third of the
    // registers (chunks after the first, when the state is in registers).
    // An item's inputs live in a struct of its own, so the item-by-item loop
    // (not unrolled) indexes no register array at a run-time position.
    struct Item {
        u32x2 xv, t0, t1, t2;
        u32x4 w01, w23;
        f32x4 av;
        float bv;
    };
    auto load_item = [&](int k, Item& it) {
        const int idx = tid + k * G::NT, j = idx / MG::NGT, g = idx - j * MG::NGT;
        if (j < n) {
            const int tok = c0 + j;
            const size_t ch = group_channel<G, D>(g, h, 0, HD);
            it.xv = seq_input(p, T, m, C3, ch, tok);
            it.t2 = seq_input(p, T, m, C3, ch, tok - 1);
            it.t1 = seq_input(p, T, m, C3, ch, tok - 2);
            it.t0 = seq_input(p, T, m, C3, ch, tok - 3);
            const u32x4* wp = reinterpret_cast<const u32x4*>(p.conv_w + 4 * ch);
            it.w01 = wp[0];
            it.w23 = wp[1];
            const size_t mt = (size_t)m * T + tok;
            if (g < D / 4) it.av = *reinterpret_cast<const f32x4*>(p.alpha + mt * HD + (size_t)h * D + 4 * g);
            if (g == 0) it.bv = p.beta[mt * p.H + h];
        }
    };
    auto conv_item = [&](int k, const Item& it) {
        const int idx = tid + k * G::NT, j = idx / MG::NGT, g = idx - j * MG::NGT;
        if (j < n) {
            const u32x4 wa = it.w01, wb = it.w23;
            const u32x2 x0 = it.t0, x1 = it.t1, x2 = it.t2, x3 = it.xv;
            reinterpret_cast<f32x4*>(sm.z[j])[g] =
                f32x4{conv_silu(u32x2{wa.x, wa.y}, bf16_lo(x0.x), bf16_lo(x1.x), bf16_lo(x2.x), bf16_lo(x3.x)),
                      conv_silu(u32x2{wa.z, wa.w}, bf16_hi(x0.x), bf16_hi(x1.x), bf16_hi(x2.x), bf16_hi(x3.x)),
                      conv_silu(u32x2{wb.x, wb.y}, bf16_lo(x0.y), bf16_lo(x1.y), bf16_lo(x2.y), bf16_lo(x3.y)),
                      conv_silu(u32x2{wb.z, wb.w}, bf16_hi(x0.y), bf16_hi(x1.y), bf16_hi(x2.y), bf16_hi(x3.y))};
            if (g < D / 4) reinterpret_cast<f32x4*>(sm.a[j])[g] = it.av;
            if (g == 0) sm.b[j] = it.bv;
            if constexpr (KEEP) {
                // this item's token, and for the first token its older taps
                // (positions -2 and -1), where they fall in T-3 .. T-1
                const int tok = c0 + j, sx = tok - (T - 3);
                if (sx >= 0 && sx < 3) sm.cs[sx][g] = it.xv;
                if (tok == 0) {
                    if (T <= 1) sm.cs[1 - T][g] = it.t1;
                    if (T <= 2) sm.cs[2 - T][g] = it.t2;
                }
            }
        }
    };
    if constexpr (ALL) {
        Item its[IT];
#pragma unroll
        for (int k = 0; k < IT; ++k) load_item(k, its[k]);
        after();                         // loads the caller issues behind the items'
#pragma unroll
        for (int k = 0; k < IT; ++k) conv_item(k, its[k]);
    } else {
#pragma unroll 1
        for (int k = 0; k < IT; ++k) {
            Item it;
            load_item(k, it);
            conv_item(k, it);
        }
    }
    lds_barrier();
    // one wave per token: the L2 norms of q and k and k^.q^
    for (int t = wv; t < n; t += G::NT / 64) {
        float sqq = 0.0f, skk = 0.0f, sqk = 0.0f;
#pragma unroll
        for (int i = lane; i < D; i += 64) {
            const float qv = sm.z[t][i], kv = sm.z[t][D + i];
            sqq = fmaf(qv, qv, sqq);
            skk = fmaf(kv, kv, skk);
            sqk = fmaf(qv, kv, sqk);
        }
        sqq = wave_sum(sqq);
        skk = wave_sum(skk);
        sqk = wave_sum(sqk);
        if (lane == 0) {
            const float rq = p.scale * rsqrtf(sqq + 1e-6f), rk = rsqrtf(skk + 1e-6f);
            sm.rq[t] = rq;
            sm.rk[t] = rk;
            sm.kq[t] = sqk * rq;   // k^.q^ / rk: the token loop carries d rk
        }
    }
    lds_barrier();
}

// The state-dependent part of token c0 + t: fade, both reductions, delta
// correction, readout, rank-1 write.  Two barriers.
template <typename TS, class MG, int D>
__device__ __forceinline__ void multi_token(float (&sreg)[MG::G::RPL][MG::G::IO_VEC], const Ptrs& p, int T,
                                            int m, int h, int tok, int t, MultiSmem<MG, D>& sm) {
    typedef typename MG::G G;
    constexpr int NT = G::NT, COLS = G::COLS, CG = G::CG, RPL = G::RPL, VEC = G::IO_VEC;
    constexpr int NWAVES = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int cg = lane % CG, rw = lane / CG;
    const float rq = sm.rq[t], rk = sm.rk[t], kq = sm.kq[t], b = sm.b[t];

    // the sums run over the conv outputs z_q, z_k themselves; the norms
    // scale the column sums (u = rk S^T z_k, w = rq S^T z_q) and the update
    // takes d rk against z_k, so no row is multiplied by rk or rq
    float kk[RPL], u[VEC], wq[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) { u[e] = 0.0f; wq[e] = 0.0f; }
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int i = G::row(wv, rw, r);
        const float a = sm.a[t][i], qq = sm.z[t][i];
        kk[r] = sm.z[t][D + i];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float sv = sreg[r][e] * a;
            sreg[r][e] = sv;
            u[e] = fmaf(sv, kk[r], u[e]);
            wq[e] = fmaf(sv, qq, wq[e]);
        }
    }
    // lanes that share columns differ in the bits above log2(CG); the token
    // loop is latency-bound, so the half-wave and row steps use the VALU swaps
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        u[e] = xor_reduce_from<CG>(u[e]);
        wq[e] = xor_reduce_from<CG>(wq[e]);
    }

    float d[VEC];
    uint16_t* const ou = p.o + ((size_t)m * T + tok) * ((size_t)p.H * D) + (size_t)h * D;
    const float* const sv_ = sm.z[t] + 2 * D;
    if constexpr (NWAVES > 1) {
        static_assert(2 * COLS <= NT, "u and w sums need 2*COLS threads");
        if (rw == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                sm.red[wv][0][cg * VEC + e] = u[e];
                sm.red[wv][1][cg * VEC + e] = wq[e];
            }
        }
        lds_barrier();
        if (tid < COLS) {
            float U = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) U += sm.red[w][0][tid];
            sm.d[tid] = rk * (b * (sv_[tid] - rk * U));
        } else if (tid < 2 * COLS) {
            float W = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) W += sm.red[w][1][tid - COLS];
            sm.w[tid - COLS] = rq * W;
        }
        lds_barrier();
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = sm.d[cg * VEC + e];
        if (tid < COLS) ou[tid] = (uint16_t)f32_to_bf16_rne(fmaf(sm.d[tid], kq, sm.w[tid]));
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = rk * (b * (sv_[cg * VEC + e] - rk * u[e]));
        if (rw == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                ou[cg * VEC + e] = (uint16_t)f32_to_bf16_rne(fmaf(d[e], kq, rq * wq[e]));
        }
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int e = 0; e < VEC; ++e) sreg[r][e] = fmaf(kk[r], d[e], sreg[r][e]);
}

// One workgroup per (stream, head), T >= 1 tokens; x [M][T][3][H*D],
// alpha [M][T][H][D], beta [M][T][H], o [M][T][H][D].
template <typename TS, int D, int NWAVES, int VEC, int RMAP, int TCMAX = 16>
__global__ __launch_bounds__(NWAVES * 64, D == 128 ? 4 : 1)   // D = 128: 4 workgroups per CU
void decode_multi_kernel(const Ptrs p, const int units, const int T)
{
    typedef MultiGeo<TS, D, NWAVES, VEC, RMAP, TCMAX> MG;
    typedef typename MG::G G;
    __shared__ MultiSmem<MG, D> sm;
    const int unit = (int)blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int cg = lane % G::CG, rw = lane / G::CG;
    const int m = unit / p.H, h = unit - m * p.H;
    const size_t HD = (size_t)p.H * D, C3 = 3 * HD;

    // the first chunk's inputs are computed before the state is requested,
    // so its items and the in-flight state never hold registers together
    TS* const st = static_cast<TS*>(p.state) + (size_t)unit * D * D + cg * G::IO_VEC;
    float sreg[G::RPL][G::IO_VEC];
    {
        const int n = min(MG::TC, T);
        multi_chunk<MG, D>(p, T, m, h, 0, n, sm);
        typename G::raw_t raw[G::RPL];
#pragma unroll
        for (int r = 0; r < G::RPL; ++r) raw[r] = G::IO::load(st + (size_t)G::row(wv, rw, r) * D);
#pragma unroll
        for (int r = 0; r < G::RPL; ++r) G::IO::unpack(raw[r], sreg[r]);
        for (int t = 0; t < n; ++t) multi_token<TS, MG, D>(sreg, p, T, m, h, t, t, sm);
        // the next chunk overwrites the vectors the last token read
        lds_barrier();
    }
    for (int c0 = MG::TC; c0 < T; c0 += MG::TC) {
        const int n = min(MG::TC, T - c0);
        multi_chunk<MG, D, false>(p, T, m, h, c0, n, sm);
        for (int t = 0; t < n; ++t) multi_token<TS, MG, D>(sreg, p, T, m, h, c0 + t, t, sm);
        lds_barrier();
    }

    // the lane's state addresses, formed again here from a value the
    // compiler cannot see into, so that they are not kept live (or spilled)
    // across the token loop; both row maps place lane row rw at
    // row(wv, 0, r) + rw
    int lo = rw * D + cg * G::IO_VEC;
    asm volatile("" : "+v"(lo));
    TS* const so = static_cast<TS*>(p.state) + (size_t)unit * D * D + lo;
#pragma unroll
    for (int r = 0; r < G::RPL; ++r) G::IO::store(so + (size_t)G::row(wv, 0, r) * D, sreg[r]);
    // conv state after T tokens: sequence positions T-3, T-2, T-1 (a
    // position < 0 is one of the cached taps, read before it is overwritten)
    if (tid < MG::NGT) {
        const size_t ch = group_channel<G, D>(tid, h, 0, HD);
        const u32x2 n0 = seq_input(p, T, m, C3, ch, T - 3);
        const u32x2 n1 = seq_input(p, T, m, C3, ch, T - 2);
        const u32x2 n2 = seq_input(p, T, m, C3, ch, T - 1);
        uint16_t* co = p.conv_out + (size_t)m * 3 * C3 + ch;
        st8(co, n0);
        st8(co + C3, n1);
        st8(co + 2 * C3, n2);
    }
}

// -------------------------------------- T tokens per launch, chunk form --
//
// D = 128: the tokens of a (stream, head) pass through the state in chunks of
// up to 8, each in the chunkwise form of the recurrence ("GLM-5.3 deep dive"
// 8.2.5, Eq. 3-9, the WY representation; here without the division by the
// cumulative decay, since a caller's alpha may be 0).  With S the state
// before the chunk (rows i = key channels, columns j = value channels), token
// t's decay g_t = a_t, the decay from token s to token t
// g(t,s) = prod_{s<r<=t} a_r (per channel; g(t,t) = 1), and P_t = g(t,-1) the
// decay of S itself up to token t:
//   delta_t = beta_t (v_t - S^T (P_t k^_t) - sum_{s<t} (k^_s . g(t,s) k^_t) delta_s)
//   o_t     = S^T (P_t q^_t) + sum_{s<=t} (k^_s . g(t,s) q^_t) delta_s
//   S'      = Diag(P_{n-1}) S + sum_s (g(n-1,s) k^_s) delta_s^T
// which is the token-by-token step (fade, predict, correct, write, read)
// unrolled over the chunk.  The two state products, X = C^T S for the 16
// vectors C = (P_t z_k,t | P_t z_q,t) and the rank-8 write, run on the f32
// matrix cores (v_mfma_f32_16x16x4f32) straight from the state registers
// (X of a bf16 state's single chunk on the bf16 ones, see PackedRegs);
// the 8 x 8 pair sums are sums over the channels, and the triangular solve
// runs per value column.  z_k, z_q are the conv outputs before the L2 norms
// (k^ = rk z_k, q^ = rq z_q), so the norms scale the small sums instead of
// every row.
//
// State layout in registers (4 waves): wave w owns value columns
// [32 w, 32 w + 32) for all 128 rows; lane (g = lane / 16, n = lane % 16)
// holds rows 16 mb + 4 g + r (mb < 8, r < 4) and columns 32 w + 2 n + c
// (c < 2), which is at once the B operand of X = C^T S (k index g at step
// 4 mb + r) and the C / D operand of the write (row 4 g + r of tile mb).

namespace wy {
constexpr int D = 128, NT = 256, TC = 8;
constexpr int CS = 20;                 // row stride of C (16 vectors + pad)
constexpr int KS = 144;                // row stride of the write's A operand
constexpr int CBS = 136;               // vector stride of the bf16 pieces of C (128 slots + pad)
// Row slot of key row i in the bf16 pieces of C: lane group g of a 32-row
// block j reads slots 32 j + 8 g .. + 7, which are the rows 32 j + 4 g + r
// and 32 j + 16 + 4 g + r (r < 4) that its state registers hold.
__device__ __forceinline__ int cb_slot(int i) {
    return (i & ~31) | (((i >> 2) & 3) << 3) | (((i >> 4) & 1) << 2) | (i & 3);
}
}

struct WySmem {
    // inputs of the chunk, as the serial kernel's chunk step writes them
    __attribute__((aligned(16))) float z[wy::TC][3 * wy::D];   // q | k | v; each wave's X / Y tile later
    __attribute__((aligned(16))) float a[wy::TC][wy::D];       // alpha; each wave's delta rows later
    float b[wy::TC], rq[wy::TC], rk[wy::TC], kq[wy::TC];
    union {
        __attribute__((aligned(16))) float C[wy::D][wy::CS];   // A operand of X: P_t z_k,t | P_t z_q,t
        // the same as three bf16 pieces (bf16 state, one chunk), [piece][vector][row slot]
        __attribute__((aligned(16))) uint16_t Cb[3][16][wy::CBS];
    };
    union {
        __attribute__((aligned(16))) float K[wy::TC][wy::KS];  // A operand of the write: g(n-1,s) z_k,s
        // the same as two bf16 pieces (bf16 state, one chunk), [piece][row]: a row's 8 tokens
        u32x4 Kp[2][wy::D];
    };
    __attribute__((aligned(16))) float G[wy::D];               // P_{n-1}
    float red[4][2][16];                                       // pair sums per wave (64 channels each)
    u32x2 cs[3][3 * wy::D / 4];                                // bf16 state, one chunk: the new conv state
};

// The partner lane's value across lane bit B (B = 0, 1: quad swaps; 3: the
// rotation by 8 within a row, which is l ^ 8).
template <int B>
__device__ __forceinline__ float xlane(float x) {
    if constexpr (B == 0) return dpp_mov<kDppQuadXor1>(x);
    else if constexpr (B == 1) return dpp_mov<kDppQuadXor2>(x);
    else return dpp_mov<0x128>(x);
}

// One step of a transposed sum: the lane keeps half of its N values (the
// low half if lane bit B is 0) and adds its partner's values of that half.
template <int N, int B>
__device__ __forceinline__ void tsum_step(float (&v)[16], int lane) {
    constexpr int H = N / 2;
    if constexpr (B == 4 || B == 5) {
        // row / half-wave swap of (low, high): even rows (halves) end with
        // both lows, odd ones with both highs
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const unsigned lo = __float_as_uint(v[k]), hi = __float_as_uint(v[k + H]);
            const auto r = B == 4 ? __builtin_amdgcn_permlane16_swap(lo, hi, false, false)
                                  : __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
            v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    } else {
        const bool up = (lane >> B) & 1;
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const float keep = up ? v[k + H] : v[k], send = up ? v[k] : v[k + H];
            v[k] = keep + xlane<B>(send);
        }
    }
}

// Sums 16 values over the 64 lanes of a wave: lane l ends with the sum of
// entry e(l) = 8 b4 + 4 b0 + 2 b1 + b3 (b_k = bit k of l).
__device__ __forceinline__ float tsum16(float (&v)[16], int lane) {
    tsum_step<16, 4>(v, lane);
    tsum_step<8, 0>(v, lane);
    tsum_step<4, 1>(v, lane);
    tsum_step<2, 3>(v, lane);
    float x = xor_add<32>(v[0]);
    return x + __shfl_xor(x, 4, 64);
}

__device__ __forceinline__ int tsum16_entry(int lane) {
    return ((lane >> 4) & 1) * 8 + (lane & 1) * 4 + ((lane >> 1) & 1) * 2 + ((lane >> 3) & 1);
}

template <typename TS> struct WyIO;
template <> struct WyIO<float> {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef f2 raw_t;
    static __device__ __forceinline__ raw_t load(const float* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const f2*>(p));
    }
    static __device__ __forceinline__ void unpack(raw_t r, float& x, float& y) { x = r.x; y = r.y; }
    static __device__ __forceinline__ void store(float* p, float x, float y) {
        __builtin_nontemporal_store(f2{x, y}, reinterpret_cast<f2*>(p));
    }
};
template <> struct WyIO<uint16_t> {
    typedef uint32_t raw_t;
    static __device__ __forceinline__ raw_t load(const uint16_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    static __device__ __forceinline__ void unpack(raw_t r, float& x, float& y) { x = bf16_lo(r); y = bf16_hi(r); }
    static __device__ __forceinline__ void store(uint16_t* p, float x, float y) {
        __builtin_nontemporal_store(pack_bf16x2(x, y), reinterpret_cast<uint32_t*>(p));
    }
};

// Pair index of (t, s), s < t < 8: t (t - 1) / 2 + s; pairs with t <= 5 form
// batch 0 (indices 0..14), t = 6, 7 batch 1 (15..27).
__device__ __forceinline__ constexpr int wy_pair(int t, int s) { return t * (t - 1) / 2 + s; }

// Per-channel coefficients of one chunk of n tokens: thread (part, c), c the
// channel.  Part 0 writes C and the k.k pair sums, part 1 K, G and the k.q
// pair sums (both over the 64 channels of the wave, into red).
template <bool XB = false>
__device__ __forceinline__ void wy_coeffs(int n, WySmem& sm) {
    using namespace wy;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c = tid & (D - 1), part = tid >> 7;
    float av[TC], zk[TC], zq[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) {
        const bool in = t < n;
        av[t] = in ? sm.a[t][c] : 1.0f;
        zk[t] = in ? sm.z[t][D + c] : 0.0f;
        zq[t] = in ? sm.z[t][c] : 0.0f;
    }
    // pair sums: (t, s) -> g(t,s) z_k,s w_t, w = z_k (part 0) or z_q (part 1)
    float pv[16];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) {
#pragma unroll
        for (int k = 0; k < 16; ++k) pv[k] = 0.0f;
#pragma unroll
        for (int t = 1; t < TC; ++t) {
            if ((t <= 5) != (bt == 0)) continue;
            const float w = part ? zq[t] : zk[t];
            float g = 1.0f;
#pragma unroll
            for (int s = t - 1; s >= 0; --s) {
                g *= av[s + 1];
                pv[wy_pair(t, s) - 15 * bt] = g * zk[s] * w;
            }
        }
        const float x = tsum16(pv, lane);
        if ((lane & 0x24) == 0) sm.red[wv][bt][tsum16_entry(lane)] = x;
    }
    // prefix decays P_t: C (part 0); G and the write's coefficients (part 1)
    if (part == 0) {
        float P = 1.0f, ck[TC], cq[TC];
#pragma unroll
        for (int t = 0; t < TC; ++t) {
            P *= av[t];
            ck[t] = P * zk[t];
            cq[t] = P * zq[t];
        }
        if constexpr (XB) {
            // three bf16 pieces per value (round to nearest even; each
            // remainder is exact in f32), vector v at slot cb_slot(c)
            const int sl = cb_slot(c);
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const float x0 = v < 8 ? ck[v] : cq[v - 8], x1 = v < 8 ? ck[v + 1] : cq[v - 7];
                const uint32_t p0 = pack_bf16x2(x0, x1);
                const float r0 = x0 - bf16_lo(p0), r1 = x1 - bf16_hi(p0);
                const uint32_t p1 = pack_bf16x2(r0, r1);
                const uint32_t p2 = pack_bf16x2(r0 - bf16_lo(p1), r1 - bf16_hi(p1));
                sm.Cb[0][v][sl] = (uint16_t)p0;
                sm.Cb[0][v + 1][sl] = (uint16_t)(p0 >> 16);
                sm.Cb[1][v][sl] = (uint16_t)p1;
                sm.Cb[1][v + 1][sl] = (uint16_t)(p1 >> 16);
                sm.Cb[2][v][sl] = (uint16_t)p2;
                sm.Cb[2][v + 1][sl] = (uint16_t)(p2 >> 16);
            }
        } else {
            f32x4* row = reinterpret_cast<f32x4*>(sm.C[c]);
            row[0] = f32x4{ck[0], ck[1], ck[2], ck[3]};
            row[1] = f32x4{ck[4], ck[5], ck[6], ck[7]};
            row[2] = f32x4{cq[0], cq[1], cq[2], cq[3]};
            row[3] = f32x4{cq[4], cq[5], cq[6], cq[7]};
        }
    } else {
        float suf = 1.0f, kv[TC];
#pragma unroll
        for (int s = TC - 1; s >= 0; --s) {
            kv[s] = suf * zk[s];                   // 0 past the chunk's last token
            if (s < n) suf *= av[s];
        }
        if constexpr (XB) {
            // two bf16 pieces per value (the second the nearest bf16 of the
            // remainder: the pair carries 16 bits), row c's tokens in order
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                hi[q] = pack_bf16x2(kv[2 * q], kv[2 * q + 1]);
                lo[q] = pack_bf16x2(kv[2 * q] - bf16_lo(hi[q]), kv[2 * q + 1] - bf16_hi(hi[q]));
            }
            sm.Kp[0][c] = u32x4{hi[0], hi[1], hi[2], hi[3]};
            sm.Kp[1][c] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        } else {
#pragma unroll
            for (int s = 0; s < TC; ++s) sm.K[s][c] = kv[s];
        }
        sm.G[c] = suf;                             // prod of a_0 .. a_{n-1}
    }
}

// The state-dependent part of one chunk of n tokens (tokens c0 .. c0 + n - 1),
// after wy_coeffs and a barrier: X = C^T S, the solve and the outputs, the
// write.
// The state's registers in the chunk form: lane (g, n) holds rows
// 16 mb + 4 g + r and columns 32 w + 2 n + c.  F32Regs keeps them as f32.
// PackedRegs keeps each row's column pair as the two bf16 of a bf16 state's
// single chunk: one VGPR instead of two; X = C^T S then runs on the bf16
// matrix cores (the state is exact in bf16, C goes as three bf16 pieces:
// 24 v_mfma_f32_16x16x32_bf16 per wave instead of 64 f32 MFMAs), and the
// write widens each tile, updates it in f32 and rounds it once -- the same
// single rounding the state gets on its way back to memory.
struct F32Regs {
    static constexpr bool XB = false;
    float v[8][4][2];
    __device__ __forceinline__ float get(int mb, int r, int c) const { return v[mb][r][c]; }
    __device__ __forceinline__ void set(int mb, int r, float x0, float x1) { v[mb][r][0] = x0; v[mb][r][1] = x1; }
    template <typename TS>
    __device__ __forceinline__ void store(TS* p, int mb, int r) const { WyIO<TS>::store(p, v[mb][r][0], v[mb][r][1]); }
    // at byte offset off of a stream_rsrc buffer, agent scope + non-temporal
    template <typename TS>
    __device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t rs, int off, int mb, int r) const {
        if constexpr (sizeof(TS) == 4)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[mb][r][0]), __float_as_uint(v[mb][r][1])},
                                                  rs, off, 0, kCpolSc1Nt);
        else
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(v[mb][r][0], v[mb][r][1]), rs, off, 0, kCpolSc1Nt);
    }
};
struct PackedRegs {
    static constexpr bool XB = true;
    uint32_t v[8][4];
    __device__ __forceinline__ float get(int mb, int r, int c) const {
        return c ? bf16_hi(v[mb][r]) : bf16_lo(v[mb][r]);
    }
    __device__ __forceinline__ void set(int mb, int r, float x0, float x1) { v[mb][r] = pack_bf16x2(x0, x1); }
    __device__ __forceinline__ void store(uint16_t* p, int mb, int r) const {
        __builtin_nontemporal_store(v[mb][r], reinterpret_cast<uint32_t*>(p));
    }
    template <typename TS>
    __device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t rs, int off, int mb, int r) const {
        __builtin_amdgcn_raw_buffer_store_b32(v[mb][r], rs, off, 0, kCpolSc1Nt);
    }
    // B fragment of 32-row block j, column c: k slot i of lane group g is row
    // 32 j + 16 (i / 4) + 4 g + i % 4, two bf16 per dword
    __device__ __forceinline__ u32x4 bfrag(int j, int c) const {
        const uint32_t sel = c ? 0x07060302u : 0x05040100u;   // high or low halves of (x, y) -> y:x
        return u32x4{__builtin_amdgcn_perm(v[2 * j][1], v[2 * j][0], sel),
                     __builtin_amdgcn_perm(v[2 * j][3], v[2 * j][2], sel),
                     __builtin_amdgcn_perm(v[2 * j + 1][1], v[2 * j + 1][0], sel),
                     __builtin_amdgcn_perm(v[2 * j + 1][3], v[2 * j + 1][2], sel)};
    }
};

// STORE: the last chunk, which stores the new state: f32 each row tile as
// soon as its products are done, so the stores overlap the remaining ones
// (M = 32, T = 8: 58.1 against 58.6 us); bf16 after the last tile and a
// barrier, so that the two waves whose 64-byte pieces share each 128-byte
// line store together (M = 128, T = 8: 164.2 against 166.6 us without).
// WT: the stores with agent scope as well as non-temporal (as the one-token
// step's WT).
template <typename TS, bool STORE, bool WT, class SR>
__device__ __forceinline__ void wy_chunk(SR& S, const Ptrs& p, int T, int m, int h, int c0, int n, WySmem& sm) {
    using namespace wy;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, nn = lane & 15;
    const size_t HD = (size_t)p.H * D;

    // ---- X = C^T S: vectors 0..7 from z_k, 8..15 from z_q ----
    f32x4 acc[2][2] = {};
    if constexpr (SR::XB) {
        typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 b0 = S.bfrag(j, 0), b1 = S.bfrag(j, 1);
#pragma unroll
            for (int pc = 0; pc < 3; ++pc) {
                const u32x4 af = *reinterpret_cast<const u32x4*>(&sm.Cb[pc][nn][32 * j + 8 * g]);
                acc[0][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, af), __builtin_bit_cast(bf16x8_t, b0), acc[0][j & 1], 0, 0, 0);
                acc[1][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, af), __builtin_bit_cast(bf16x8_t, b1), acc[1][j & 1], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float a = sm.C[16 * mb + 4 * g + r][nn];
                acc[0][mb & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, S.get(mb, r, 0), acc[0][mb & 1], 0, 0, 0);
                acc[1][mb & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, S.get(mb, r, 1), acc[1][mb & 1], 0, 0, 0);
            }
    }
    // the wave's X tile [16][32] goes to the q | k rows of z (dead now), its
    // delta rows [8][32] to alpha's (dead too)
    auto xy = [&](int v, int j) -> float& { return sm.z[2 * wv + (v >> 3)][(v & 7) * 32 + j]; };
    auto drow = [&](int s, int j) -> float& { return sm.a[2 * wv + (s >> 2)][(s & 3) * 32 + j]; };
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const f32x4 x = acc[c][0] + acc[c][1];
#pragma unroll
        for (int r = 0; r < 4; ++r) xy(4 * g + r, 2 * nn + c) = x[r];
    }

    // the solve's coefficients, one per lane, read back by v_readlane:
    // lane l < 8: token l's scalars; lane li = pair (< 15) or pair + 1 of the
    // k.k sums times -rk_s rk_t, lane 32 + li of the k.q sums times rk_s rq_t
    float cpair, ck_rk, ck_rq, ck_b, ck_diag;
    {
        const int pt = lane >> 5, bt = (lane >> 4) & 1, e = lane & 15;
        const int pi = 15 * bt + e;                  // pair index (e == 15: padding)
        int t = 1;
        while (t < 7 && (t + 1) * t / 2 <= pi) ++t;
        const int sidx = min(max(pi - t * (t - 1) / 2, 0), TC - 1);
        const float sum = sm.red[2 * pt][bt][e] + sm.red[2 * pt + 1][bt][e];
        cpair = pt == 0 ? -(sm.rk[sidx] * sm.rk[t]) * sum : (sm.rk[sidx] * sm.rq[t]) * sum;
        const int tt = lane & 7;
        ck_rk = sm.rk[tt];
        ck_rq = sm.rq[tt];
        ck_b = sm.b[tt];
        ck_diag = sm.rk[tt] * sm.kq[tt];             // rk_t rq_t (z_k,t . z_q,t)
    }
    auto rl = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
    __builtin_amdgcn_wave_barrier();

    // ---- the triangular solve and the outputs: lane j (and j + 32) takes column 32 wv + j ----
    {
        const int j = lane & 31;
        float dl[TC];
        uint16_t* const ou = p.o + ((size_t)m * T + c0) * HD + (size_t)h * D + 32 * wv + j;
#pragma unroll
        for (int t = 0; t < TC; ++t) {
            if (t < n) {
                const float rk_t = rl(ck_rk, t);
                float acc_d = fmaf(-rk_t, xy(t, j), sm.z[t][2 * D + 32 * wv + j]);
                float acc_o = rl(ck_rq, t) * xy(8 + t, j);
#pragma unroll
                for (int s2 = 0; s2 < t; ++s2) {
                    const int pi = t * (t - 1) / 2 + s2, li = pi < 15 ? pi : pi + 1;
                    acc_d = fmaf(rl(cpair, li), dl[s2], acc_d);
                    acc_o = fmaf(rl(cpair, 32 + li), dl[s2], acc_o);
                }
                dl[t] = rl(ck_b, t) * acc_d;
                acc_o = fmaf(rl(ck_diag, t), dl[t], acc_o);
                if (lane < 32) {
                    ou[(size_t)t * HD] = (uint16_t)f32_to_bf16_rne(acc_o);
                    drow(t, j) = rk_t * dl[t];
                }
            } else if (lane < 32) {
                drow(t, j) = 0.0f;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- S <- Diag(G) S + K^T E on the matrix cores ----
    // f32 registers: two v_mfma_f32_16x16x4f32 per tile over the 8 tokens.
    // Packed bf16 registers (the state is rounded to bf16 after the write):
    // one v_mfma_f32_16x16x32_bf16 per tile whose k slots hold K_hi E_hi,
    // K_hi E_lo, K_lo E_hi (8 tokens each) and zeros, the two-piece operands
    // carrying 16 bits: the update's error stays about 2^-16 of it, far
    // below the state's final rounding.
    float e[2][2];
    u32x4 eb[2];
    if constexpr (SR::XB) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float e0 = drow(2 * q, 2 * nn + c), e1 = drow(2 * q + 1, 2 * nn + c);
                hi[q] = pack_bf16x2(e0, e1);
                lo[q] = pack_bf16x2(e0 - bf16_lo(hi[q]), e1 - bf16_hi(hi[q]));
            }
            eb[c] = g == 1 ? u32x4{lo[0], lo[1], lo[2], lo[3]}
                           : (g == 3 ? u32x4{0u, 0u, 0u, 0u} : u32x4{hi[0], hi[1], hi[2], hi[3]});
        }
    } else {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int c = 0; c < 2; ++c) e[st][c] = drow(4 * st + g, 2 * nn + c);
    }
    TS* const head = static_cast<TS*>(p.state) + (size_t)(m * p.H + h) * D * D;
    const __amdgpu_buffer_rsrc_t rs = stream_rsrc(head, D * D * (int)sizeof(TS));
    int lo = 0;
    if constexpr (STORE) {
        // the lane's offset in the head, formed here from a value the
        // compiler cannot see into, so its addresses are not kept live
        // across the chunk
        lo = 32 * wv + 2 * nn + 4 * g * D;
        asm volatile("" : "+v"(lo));
    }
    auto store_row = [&](int mb, int r) {
        const int e = lo + (16 * mb + r) * D;
        if constexpr (WT) S.template store_sc1<TS>(rs, e * (int)sizeof(TS), mb, r);
        else S.store(head + e, mb, r);
    };
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const f32x4 gd = *reinterpret_cast<const f32x4*>(&sm.G[16 * mb + 4 * g]);
        f32x4 cv[2];
        if constexpr (SR::XB) {
            typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
            const u32x4 ka = g == 3 ? u32x4{0u, 0u, 0u, 0u} : sm.Kp[g == 2][16 * mb + nn];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                cv[c] = f32x4{S.get(mb, 0, c) * gd[0], S.get(mb, 1, c) * gd[1], S.get(mb, 2, c) * gd[2],
                              S.get(mb, 3, c) * gd[3]};
                cv[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                                __builtin_bit_cast(bf16x8_t, eb[c]), cv[c], 0, 0, 0);
            }
        } else {
            const float k0 = sm.K[g][16 * mb + nn], k1 = sm.K[4 + g][16 * mb + nn];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                cv[c] = f32x4{S.get(mb, 0, c) * gd[0], S.get(mb, 1, c) * gd[1], S.get(mb, 2, c) * gd[2],
                              S.get(mb, 3, c) * gd[3]};
                cv[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(k0, e[0][c], cv[c], 0, 0, 0);
                cv[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(k1, e[1][c], cv[c], 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) S.set(mb, r, cv[0][r], cv[1][r]);
        if constexpr (STORE && sizeof(TS) == 4) {
#pragma unroll
            for (int r = 0; r < 4; ++r) store_row(mb, r);
        }
    }
    if constexpr (STORE && sizeof(TS) == 2) {
        lds_barrier();
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) store_row(mb, r);
    }
    // the next chunk overwrites the inputs, X, delta, C, K and G
    if constexpr (!STORE) lds_barrier();
}

// ONE: T <= 8, a single chunk, its state requested in two halves, the first
// right behind the chunk's input loads and the second once their registers
// are free, so the state streams in while the inputs wait and the
// coefficients are formed.  With STAG (f32 only) the odd workgroups --
// which, dealt round robin to the 8 XCDs, are those of the odd XCDs --
// request their whole state only after forming the coefficients, so the
// first round of workgroups does not ask for every head's state at once.
// f32 single chunks also take the one-token step's XCD-aware order (even
// workgroups the first half of the heads upwards, odd ones the second half
// downwards; one process, alternating builds, us per call: M = 32 T = 8
// 57.3 -> 56.8, T = 6 55.8 -> 55.1, T = 4 unchanged, M = 8 T = 8 16.9 ->
// 16.4).  Otherwise chunk after chunk, the state requested once the first
// chunk's coefficients are formed.  WT: the state stores with agent scope as
// well (grids of several rounds of workgroups).
template <typename TS, bool ONE, bool WT, bool STAG = false>
__global__ __launch_bounds__(wy::NT, 4)
void decode_wy_kernel(const Ptrs p, const int units, const int T)
{
    using namespace wy;
    typedef MultiGeo<TS, D, 4, 4, 1, TC> MG;
    typedef WyIO<TS> IO;
    __shared__ WySmem sm;
    const int b = (int)blockIdx.x;
    const int unit = sizeof(TS) == 4 && ONE && (units & 1) == 0 ? ((b & 1) ? units - 1 - (b >> 1) : (b >> 1)) : b;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, nn = lane & 15;
    const int m = unit / p.H, h = unit - m * p.H;
    const size_t HD = (size_t)p.H * D, C3 = 3 * HD;

    if constexpr (ONE) {
        const TS* st = static_cast<const TS*>(p.state) + (size_t)unit * D * D + 32 * wv + 2 * nn;
        typename IO::raw_t raw[8][4];
        auto half = [&](int h2) {
#pragma unroll
            for (int mb = 4 * h2; mb < 4 * h2 + 4; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) raw[mb][r] = IO::load(st + (size_t)(16 * mb + 4 * g + r) * D);
        };
        // (bf16: the whole state fits beside the chunk's input registers)
        const bool late = sizeof(TS) == 4 && STAG && (blockIdx.x & 1) != 0;
        auto after = [&]() {
            if (!late) half(0);
            if constexpr (sizeof(TS) == 2) half(1);
        };
        // bf16: the new conv state kept in LDS (its reloads at the end would
        // wait behind the state stores: M = 128 T = 8 141.0 -> 139.1 us,
        // M = 32 43.5 -> 41.9; f32 1.2% slower with it, so f32 reloads)
        multi_chunk<MG, D, true, WySmem, decltype(after), sizeof(TS) == 2>(p, T, m, h, 0, T, sm, after);
        if constexpr (sizeof(TS) == 4) {
            if (!late) {
                half(1);
                wy_coeffs(T, sm);
            } else {
                wy_coeffs(T, sm);
                half(0);
                half(1);
            }
            lds_barrier();
            F32Regs S;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) IO::unpack(raw[mb][r], S.v[mb][r][0], S.v[mb][r][1]);
            wy_chunk<TS, true, WT>(S, p, T, m, h, 0, T, sm);
        } else {
            wy_coeffs<true>(T, sm);
            lds_barrier();
            PackedRegs S;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) S.v[mb][r] = raw[mb][r];
            wy_chunk<TS, true, WT>(S, p, T, m, h, 0, T, sm);
        }
    } else {
        F32Regs S;
        // the first chunk's inputs and coefficients before the state is
        // requested: a wave's loads complete in order
        const int n = min(TC, T);
        multi_chunk<MG, D, true, WySmem>(p, T, m, h, 0, n, sm);
        wy_coeffs(n, sm);
        const TS* st = static_cast<const TS*>(p.state) + (size_t)unit * D * D + 32 * wv + 2 * nn;
        typename IO::raw_t raw[8][4];
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) raw[mb][r] = IO::load(st + (size_t)(16 * mb + 4 * g + r) * D);
        lds_barrier();
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) IO::unpack(raw[mb][r], S.v[mb][r][0], S.v[mb][r][1]);
        wy_chunk<TS, false, false>(S, p, T, m, h, 0, n, sm);
        for (int c0 = TC; c0 < T; c0 += TC) {
            const int n2 = min(TC, T - c0);
            multi_chunk<MG, D, false, WySmem>(p, T, m, h, c0, n2, sm);   // item by item beside the state
            wy_coeffs(n2, sm);
            lds_barrier();
            wy_chunk<TS, false, false>(S, p, T, m, h, c0, n2, sm);
        }
        int lo = 32 * wv + 2 * nn + 4 * g * D;
        asm volatile("" : "+v"(lo));
        TS* const head = static_cast<TS*>(p.state) + (size_t)unit * D * D;
        const __amdgpu_buffer_rsrc_t rs = stream_rsrc(head, D * D * (int)sizeof(TS));
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = lo + (16 * mb + r) * D;
                if constexpr (WT) S.template store_sc1<TS>(rs, e * (int)sizeof(TS), mb, r);
                else IO::store(head + e, S.v[mb][r][0], S.v[mb][r][1]);
            }
    }

    if (tid < MG::NGT) {
        const size_t ch = group_channel<typename MG::G, D>(tid, h, 0, HD);
        u32x2 n0, n1, n2;
        if constexpr (ONE && sizeof(TS) == 2) {
            n0 = sm.cs[0][tid];
            n1 = sm.cs[1][tid];
            n2 = sm.cs[2][tid];
        } else {
            n0 = seq_input(p, T, m, C3, ch, T - 3);
            n1 = seq_input(p, T, m, C3, ch, T - 2);
            n2 = seq_input(p, T, m, C3, ch, T - 1);
        }
        uint16_t* co = p.conv_out + (size_t)m * 3 * C3 + ch;
        st8(co, n0);
        st8(co + C3, n1);
        st8(co + 2 * C3, n2);
    }
}

// -------------------------------------------------------------- conv step --
// One thread per 8 consecutive channels of one stream.
__global__ __launch_bounds__(256)
void conv_kernel(const int M, const int C, const uint16_t* __restrict__ x,
                 const uint16_t* __restrict__ conv_w, const uint16_t* conv_in,
                 uint16_t* conv_out, float* __restrict__ y)
{
    const int groups = C / 8;
    const long g = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= (long)M * groups) return;
    const int m = (int)(g / groups);
    const int c0 = (int)(g - (long)m * groups) * 8;
    const uint16_t* ci = conv_in + (size_t)m * 3 * C + c0;
    const u32x4 t0 = *reinterpret_cast<const u32x4*>(ci);
    const u32x4 t1 = *reinterpret_cast<const u32x4*>(ci + C);
    const u32x4 t2 = *reinterpret_cast<const u32x4*>(ci + 2 * (size_t)C);
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (size_t)m * C + c0);
    const u32x4* wp = reinterpret_cast<const u32x4*>(conv_w + 4 * (size_t)c0);
    const u32x4 w01 = wp[0], w23 = wp[1], w45 = wp[2], w67 = wp[3];
    const uint32_t a0[4] = {t0.x, t0.y, t0.z, t0.w};
    const uint32_t a1[4] = {t1.x, t1.y, t1.z, t1.w};
    const uint32_t a2[4] = {t2.x, t2.y, t2.z, t2.w};
    const uint32_t ax[4] = {xv.x, xv.y, xv.z, xv.w};
    const u32x2 wc[8] = {{w01.x, w01.y}, {w01.z, w01.w}, {w23.x, w23.y}, {w23.z, w23.w},
                         {w45.x, w45.y}, {w45.z, w45.w}, {w67.x, w67.y}, {w67.z, w67.w}};
    float out[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        out[2 * p] = conv_silu(wc[2 * p], bf16_lo(a0[p]), bf16_lo(a1[p]), bf16_lo(a2[p]), bf16_lo(ax[p]));
        out[2 * p + 1] = conv_silu(wc[2 * p + 1], bf16_hi(a0[p]), bf16_hi(a1[p]), bf16_hi(a2[p]), bf16_hi(ax[p]));
    }
    uint16_t* co = conv_out + (size_t)m * 3 * C + c0;
    *reinterpret_cast<u32x4*>(co) = t1;
    *reinterpret_cast<u32x4*>(co + C) = t2;
    *reinterpret_cast<u32x4*>(co + 2 * (size_t)C) = xv;
    f32x4* yp = reinterpret_cast<f32x4*>(y + (size_t)m * C + c0);
    yp[0] = f32x4{out[0], out[1], out[2], out[3]};
    yp[1] = f32x4{out[4], out[5], out[6], out[7]};
}

// ---------------------------------------------------------------- launch --


template <typename TS, int D, int NSPLIT, int NWAVES, int VEC, bool FUSED, bool XG, int RMAP = 0, int MODE = 0,
          bool WT = false, bool PK = false>
static hipError_t launch_decode(const StepArgs& a) {
    Ptrs p = make_ptrs(a);
    int units = a.M * a.H;
    void* args[] = {(void*)&p, (void*)&units};
    const dim3 grid((unsigned)((long)units * NSPLIT));
    const dim3 block(NWAVES * 64);
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&decode_kernel<TS, D, NSPLIT, NWAVES, VEC, RMAP, FUSED, XG, MODE, WT, PK>), grid,
        block, args, 0, (hipStream_t)a.stream);
}

// D = 128 launch shapes, from measurement on MI355X (34 layers of distinct
// state, DRAM-resident):
//  f32, whole head per workgroup: 16 waves (4 rows x 4 columns per lane)
//    once there are >= 2048 heads to run; 4 waves, each a band of 32 rows
//    (16 rows per lane, 4 workgroups per CU), for 256 to 768 heads, one
//    round of workgroups (M = 8: 12.35 against 12.6 us with 8 waves of 8
//    rows in bands, itself 4% faster than interleaved rows there); else 8
//    waves with interleaved rows (fewer heads: idle CUs; more: several
//    rounds; both slower with bands).
//  bf16, whole head per workgroup: 4 waves, each owning a band of 32 rows,
//    16 rows x 4 columns per lane (8-byte accesses), 4 workgroups per CU
//    (the plain step in one round of up to 8 heads per CU: the packed form,
//    8 workgroups per CU, dispatch_wide_bf16):
//    against 8 waves of 8 rows, M = 8 7.70 / 7.81 us, M = 32 26.1 / 26.7,
//    M = 128 97.4 / 98.0 (with the hardware bf16 rounding; before it the
//    8-wave form was the faster one).  With 8 columns per lane and 16-byte
//    accesses a row spans 16 lanes and the column sums take two cross-lane
//    steps: slower at every M measured.
//  column splits (small M*H only): 8 waves (f32, 2-way), else 4 waves.
//  state stores with agent scope (WT) once there are >= 2048 heads, i.e.
//    several rounds of workgroups per CU: 1.5% faster at 32 x 64 heads (f32)
//    and 0.8% at 128 x 64 (bf16); 15% slower at 1 x 64, where one round of
//    workgroups waits for its own last stores.
// A split leaves every workgroup a row segment of >= 128 bytes for f32 at
// 2- and 4-way and bf16 at 2-way; bf16 at 4-way (64 bytes) is supported but
// shares cache lines between workgroups and is never chosen by the library.
// The output norm (MODE 2) needs a whole head per workgroup: no splits.
template <bool FUSED, int MODE>
static hipError_t dispatch_wide_f32(const StepArgs& a) {
    if (a.nsplit == 1) {
        const long heads = (long)a.M * a.H;
        if (heads >= 2048) return launch_decode<float, 128, 1, 16, 4, FUSED, true, 0, MODE, true>(a);
        if (heads >= 256 && heads <= 768) return launch_decode<float, 128, 1, 4, 4, FUSED, false, 1, MODE>(a);
        return launch_decode<float, 128, 1, 8, 4, FUSED, false, 0, MODE>(a);
    }
    if constexpr (MODE != 2) {
        if (a.nsplit == 2) return launch_decode<float, 128, 2, 8, 4, FUSED, true, 0, MODE>(a);
        if (a.nsplit == 4) return launch_decode<float, 128, 4, 4, 4, FUSED, true, 0, MODE>(a);
    }
    return hipErrorInvalidValue;
}

template <bool FUSED, int MODE>
static hipError_t dispatch_wide_bf16(const StepArgs& a) {
    if (a.nsplit == 1) {
        const long heads = (long)a.M * a.H;
        // plain step, one round of 8 packed workgroups per CU: M = 32 25.8
        // -> 25.4 us, M = 8 7.73 -> 7.56 (one process, alternating builds);
        // with several rounds (M = 128 95.9 -> 98.0) and for the gated and
        // layer steps (26.1 -> 27.5 at M = 32: their gate inputs spill at
        // 64 VGPRs) the unpacked form at 4 workgroups per CU stays
        if constexpr (MODE == 0) {
            const int cus = stream_cu_count(a.stream);
            if (cus > 0 && heads <= 8L * cus)
                return heads >= 2048 ? launch_decode<uint16_t, 128, 1, 4, 4, FUSED, false, 1, MODE, true, true>(a)
                                     : launch_decode<uint16_t, 128, 1, 4, 4, FUSED, false, 1, MODE, false, true>(a);
        }
        return heads >= 2048 ? launch_decode<uint16_t, 128, 1, 4, 4, FUSED, false, 1, MODE, true>(a)
                             : launch_decode<uint16_t, 128, 1, 4, 4, FUSED, false, 1, MODE>(a);
    }
    if constexpr (MODE != 2) {
        if (a.nsplit == 2) return launch_decode<uint16_t, 128, 2, 4, 8, FUSED, true, 0, MODE>(a);
        if (a.nsplit == 4) return launch_decode<uint16_t, 128, 4, 4, 8, FUSED, true, 0, MODE>(a);
    }
    return hipErrorInvalidValue;
}

template <bool FUSED, int MODE>
static hipError_t dispatch(const StepArgs& a) {
    const bool f32 = a.state_dtype == 0;
    if (a.D != 128 && a.nsplit != 1) return hipErrorInvalidValue;
    switch (a.D) {
    case 16:
        return f32 ? launch_decode<float, 16, 1, 1, 4, FUSED, false, 0, MODE>(a)
                   : launch_decode<uint16_t, 16, 1, 1, 4, FUSED, false, 0, MODE>(a);
    case 32:
        return f32 ? launch_decode<float, 32, 1, 1, 4, FUSED, false, 0, MODE>(a)
                   : launch_decode<uint16_t, 32, 1, 1, 8, FUSED, false, 0, MODE>(a);
    case 64:
        return f32 ? launch_decode<float, 64, 1, 2, 4, FUSED, false, 0, MODE>(a)
                   : launch_decode<uint16_t, 64, 1, 2, 8, FUSED, false, 0, MODE>(a);
    case 128:
        return f32 ? dispatch_wide_f32<FUSED, MODE>(a) : dispatch_wide_bf16<FUSED, MODE>(a);
    default:
        return hipErrorInvalidValue;
    }
}

template <typename TS, int D, int NWAVES, int VEC, int RMAP, int TC>
static hipError_t launch_multi(const StepArgs& a) {
    Ptrs p = make_ptrs(a);
    int units = a.M * a.H;
    int T = a.T;
    void* args[] = {(void*)&p, (void*)&units, (void*)&T};
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_multi_kernel<TS, D, NWAVES, VEC, RMAP, TC>),
                           dim3((unsigned)units), dim3(NWAVES * 64), args, 0, (hipStream_t)a.stream);
}

template <typename TS>
static hipError_t launch_wy(const StepArgs& a) {
    Ptrs p = make_ptrs(a);
    int units = a.M * a.H;
    int T = a.T;
    void* args[] = {(void*)&p, (void*)&units, (void*)&T};
    // agent-scope stores from 2048 heads on, as the one-token step (M = 128
    // bf16, T = 8: 154.6 -> 149.1 us; M = 32 f32 unchanged)
    const bool wt = units >= 2048;
    // f32 single chunks of 5 to 8 tokens: the staggered form, half the
    // workgroups requesting their state after the coefficients (one process,
    // alternating builds, us per call, M = 32: T = 8 58.3 -> 57.6, T = 6
    // 56.4 -> 56.1, T = 5 55.5 -> 55.3, but T = 4 54.3 -> 54.5 and T = 2
    // 51.8 -> 53.0; M = 8: T = 8 18.6 -> 16.7, T = 6 16.9 -> 16.1)
    const bool stag = sizeof(TS) == 4 && T >= 5;
    const void* fn = T <= wy::TC
        ? (stag ? (wt ? reinterpret_cast<const void*>(&decode_wy_kernel<TS, true, true, true>)
                      : reinterpret_cast<const void*>(&decode_wy_kernel<TS, true, false, true>))
                : (wt ? reinterpret_cast<const void*>(&decode_wy_kernel<TS, true, true>)
                      : reinterpret_cast<const void*>(&decode_wy_kernel<TS, true, false>)))
        : (wt ? reinterpret_cast<const void*>(&decode_wy_kernel<TS, false, true>)
              : reinterpret_cast<const void*>(&decode_wy_kernel<TS, false, false>));
    return hipLaunchKernel(fn, dim3((unsigned)units), dim3(wy::NT), args, 0, (hipStream_t)a.stream);
}

// T tokens per launch, one workgroup per head.
hipError_t launch_decode_multi(const StepArgs& a) {
    const bool f32 = a.state_dtype == 0;
    switch (a.D) {
    case 16: return f32 ? launch_multi<float, 16, 1, 4, 0, 5>(a) : launch_multi<uint16_t, 16, 1, 4, 0, 5>(a);
    case 32: return f32 ? launch_multi<float, 32, 1, 4, 0, 2>(a) : launch_multi<uint16_t, 32, 1, 8, 0, 2>(a);
    case 64: return f32 ? launch_multi<float, 64, 2, 4, 0, 2>(a) : launch_multi<uint16_t, 64, 2, 8, 0, 2>(a);
    case 128:
        // 4 waves per head either way.  The chunk form pays its matrix
        // products per chunk, the token loop its sweep per token; measured
        // on MI355X (us per call, token loop / chunk form, 34 layers):
        //   f32, M = 32:   T = 1 50.9 / 51.3, 2 53.8 / 53.2, 4 57.3 / 55.3,
        //                  8 69.0 / 59.3, 9 76.3 / 77.3, 16 104.5 / 89.3,
        //                  17 110.3 / 105.4, 32 176.8 / 151.6
        //   bf16, M = 128: T = 1 97.8 / 125.0, 2 103.2 / 131.7, 4 128.6 / 136.1,
        //                  5 138.2 / 138.1, 6 146.2 / 144.8, 8 190.5 / 154
        //                  (one chunk: X on the bf16 matrix cores), 9 216.1 /
        //                  241.5, 12 263.5 / 261.1, 16 329.4 / 286.1, 17 352.6 /
        //                  356.7, 20 407.0 / 376.0, 32 611.7 / 513.1
        // so f32 takes the chunk form from T = 2 on, and bf16 where
        // 116 ceil(T / 8) < 17.5 T + 30 (the fitted per-chunk and per-token
        // costs at M = 128): T = 5..8, 12..16 and every T >= 19.
        if (f32) return a.T >= 2 ? launch_wy<float>(a) : launch_multi<float, 128, 4, 4, 1, 8>(a);
        {
            const long chunks = ((long)a.T + wy::TC - 1) / wy::TC;
            return 232 * chunks < 35L * a.T + 60 ? launch_wy<uint16_t>(a) : launch_multi<uint16_t, 128, 4, 4, 1, 8>(a);
        }
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_step(const StepArgs& a) { return dispatch<true, 0>(a); }
hipError_t launch_recurrent_step(const StepArgs& a) { return dispatch<false, 0>(a); }
hipError_t launch_decode_step_gated(const StepArgs& a) { return dispatch<true, 1>(a); }
hipError_t launch_layer_step(const StepArgs& a) { return dispatch<true, 2>(a); }

hipError_t launch_conv_step(int M, int C, const void* x, const void* w, const void* cin,
                            void* cout, float* y, void* stream) {
    const long threads = (long)M * (C / 8);
    const int block = 256;
    const dim3 grid((unsigned)((threads + block - 1) / block));
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* wp = (const uint16_t*)w;
    const uint16_t* ci = (const uint16_t*)cin;
    uint16_t* co = (uint16_t*)cout;
    void* args[] = {(void*)&M, (void*)&C, (void*)&xp, (void*)&wp, (void*)&ci, (void*)&co, (void*)&y};
    return hipLaunchKernel(reinterpret_cast<const void*>(&conv_kernel), grid, dim3(block), args, 0,
                           (hipStream_t)stream);
}

int device_cu_count(int dev) {
    static int cached[64] = {0};
    if (dev < 0) return 0;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    if (dev < 64) cached[dev] = n;
    return n;
}

int stream_cu_count(void* stream) {
    int dev = 0;
    if (stream) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice((hipStream_t)stream, &d) != hipSuccess) return 0;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return 0;
    }
    return device_cu_count(dev);
}

}  // namespace kda
