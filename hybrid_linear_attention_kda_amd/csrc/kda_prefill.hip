// kda_prefill.hip -- chunked KDA over a sequence of tokens, on gfx950 MFMA.
//
// "GLM-5.3 deep dive" 8.2.5 (training in chunks: the WY representation and
// the UT transform), for one chunk of C tokens with incoming state S,
// cumulative per-channel decay Gamma (inclusive, from the chunk start),
// normalised keys K, scaled queries Q and values V (C-row matrices):
//
//   A     = StrictTril(Diag(beta) (Gamma . K) (K / Gamma)^T)
//   W     = (I + A)^-1 Diag(beta) (Gamma . K),   U = (I + A)^-1 Diag(beta) V
//   Delta = U - W S
//   O     = (Gamma . Q) S + Tril((Gamma . Q)(K / Gamma)^T) Delta
//   S'    = Diag(gamma_C) S + ((gamma_C / Gamma) . K)^T Delta
//
// This is the same recurrence as the per-token step (8.2.3 Eq. 1), reordered
// so that its work is matrix products.  The chunk is 16 tokens and the
// forget gate is the bounded one with a lower bound in [-5, 0): then the
// cumulative log-decay inside a chunk is >= -80, so Gamma and 1 / Gamma stay
// inside f32's range (the deep dive's reading of the -5 bound: e^(+-80) is
// below f32's e^88.7, which lets 16-token blocks be factored into plain
// matrix products).
//
// Design (MI355X, CDNA4): one workgroup of 4 waves per (stream, head) sweeps
// the head's chunks in order, two workgroups per CU.  The head's 128 x 128
// f32 state stays in the accumulator layout of the 16 x 16 MFMAs for the
// whole sequence: wave w owns value columns [32w, 32w + 32), each lane 64
// state values (row k = 16 mt + 4 (lane / 16) + r, column n = 32 w + 16 nt +
// lane % 16).  Per chunk, five phases:
//
//   1. inputs: waves 0, 1 run the conv + SiLU of q and k (each lane two
//      channels over the chunk's 16 tokens, the three previous raw inputs
//      carried in registers from chunk to chunk) and the L2 norms (one
//      transposing reduction over the wave for all 16 tokens); waves 2, 3
//      each take half of the channels of v and of the forget gate with its
//      running decay product, and wave 3 the write strengths.  The raw
//      inputs of the next chunk are then requested, so their HBM latency
//      hides behind phases 2 to 5.
//   2. A (waves 0, 1) and P (waves 2, 3) as 16 x 16 products, each wave
//      over one half of the 128 channels (f32 MFMA; the halves are added
//      where A and P are read); then all waves split Gamma . Q and
//      (gamma_C / Gamma) . K into bf16 pieces, in MFMA fragment order.
//   3. the triangular solves for W and U, right-looking, one column per
//      thread (256 columns), straight from (I + A) W = Diag(beta)(Gamma . K).
//   4. Delta = U - W S and (Gamma . Q) S (-W split into its bf16 pieces
//      once, a quarter by each wave); each wave needs only its own columns
//      of Delta afterwards, so no workgroup barrier separates it from
//      phase 5.
//   5. O = (Gamma . Q) S + P Delta, stored; S' = Diag(gamma_C) S + ...
//
// Phases 3 to 5 are the chunk's serial path; on sequences of more than four
// chunks they run at a raised wave priority, so that the other workgroup
// on the CU fills their gaps with its vector-bound phases 1 and 2.
//
// The three state products (phases 4 and 5) run on the bf16 matrix cores
// from three-way bf16 splits of both operands, six piece pairs per product,
// f32 accumulation: FP32 accuracy at a fraction of the f32 MFMA time (f32
// MFMA shares its issue budget with vector work on this chip; bf16 MFMA is
// 16 times faster per flop).  The state's own registers of a 32-row block
// (rows 32 kb + 4 (lane / 16) + {0..3, 16..19}) form the B fragment of
// v_mfma_f32_16x16x32_bf16 directly.
//
// LDS: the [token][channel] arrays have rows of 132 floats; the bf16
// fragment arrays are lane-major, so a half-wave reads 512 contiguous bytes
// (row-strided 16-byte reads cost several times a contiguous one).  Where a
// 16 x 16 x 4 contraction runs over tokens, the MFMA's k slot lane / 16
// stands for tokens 4 (lane / 16) + kk.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {


namespace {

constexpr int PD = 128;            // head width (dk = dv)
constexpr int PC = 16;             // chunk length, tokens
constexpr int PNT = 256;           // threads per workgroup (4 waves)
constexpr int LS = PD + 4;         // LDS row stride of the [token][channel] arrays, floats
constexpr int LT = PC + 4;         // LDS row stride of the 16 x 16 arrays, floats

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Three-way bf16 splits: x = x1 + x2 + x3 up to f32 rounding, each piece the
// round-to-nearest-even bf16 of what the previous ones leave (the remainder
// is exact in f32).  A product of two split operands then takes the six
// terms x_a y_b with a + b <= 4 (pieces numbered from 1), which keeps
// products to f32 accuracy while running on the bf16 matrix cores.  The one
// product that feeds only the output, (Gamma . Q) S, takes the three terms
// with a + b <= 3: each dropped term is below 2^-17 of its product (RNE
// pieces: |x - x1| <= 2^-9 |x|, |x - x1 - x2| <= 2^-18 |x|), far inside the
// output's single bf16 rounding, while the state keeps f32 accuracy.
// Fragments hold 8 bf16 (one per k slot of v_mfma_f32_16x16x32_bf16), as
// 4 dwords, slot 2i in the low half of dword i.
struct PrefillSmem {
    float kh[PC][LS];              // k^; after the solve, -W
    float vv[PC][LS];              // v; after the solve, U
    float eg[PC][LS];              // Gamma (decay from the chunk start); after the state products, Delta
    union {
        float qi[2][PC][LS];       // [0] q^ (normalised, scaled), [1] 1 / Gamma; dead after phase 2
        u32x4 dp[3][4][2][2][16];  // Delta pieces [piece][wave][tile][token half][column]: 8 tokens each
    };
    u32x4 gqp[2][4][64];           // (Gamma . q^) pieces 1, 2 [piece][32-row block][lane]: A operand of (Gamma . Q) S
    u32x4 wpk[4][3][64];           // -W pieces [32-row block][piece][lane]: A operand of W S, split once per chunk
    u32x4 ktp[3][8][2][16];        // ((gamma_C / Gamma) . k^) pieces [piece][row tile][token half][row]
    float Z[2][PC][LT];            // Z[j][i] = sum_c (Gamma . k^)[i][c] (k^ / Gamma)[j][c], per channel half
    float P[2][PC][LT];            // Tril((Gamma . q^)(k^ / Gamma)^T), row = query token, per channel half
    float gam[PD];                 // gamma_C, the decay over the whole chunk
    float beta[PC];
};

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Orders this wave's LDS writes before its later LDS reads (data handed
// between lanes of one wave), without waiting for the other waves.
__device__ __forceinline__ void lds_wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// two f32 -> packed bf16, a in the low half
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) { return pack_bf16x2(a, b); }

// e^x from the hardware 2^x (v_exp_f32) of the rounded product x log2(e).
// Rounding the product (and log2(e)) moves the result by at most about
// 8e-8 |x| relative: 4e-7 for a decay exponent in [-5, 0], 1.3e-6 for a
// SiLU argument of 16.  Within a chunk the decays multiply up over at most
// 16 tokens, and a decay's error only matters in proportion to what it
// decays, so the state moves by far less than its f32 tolerance (the
// state and output errors against the oracle are unchanged to four
// digits).  Sigmoid and SiLU take the hardware reciprocal as well.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(1.44269502162933349609375f * x); }
__device__ __forceinline__ float sigmoid_hw(float y) { return __builtin_amdgcn_rcpf(1.0f + exp_hw(-y)); }
__device__ __forceinline__ float silu_hw(float y) { return y * sigmoid_hw(y); }

// the three bf16 pieces of (a, b), one packed dword each
__device__ __forceinline__ void split2(float a, float b, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
    p0 = cvt_pk_bf16(a, b);
    const float a1 = a - bf16_lo(p0), b1 = b - bf16_hi(p0);
    p1 = cvt_pk_bf16(a1, b1);
    p2 = cvt_pk_bf16(a1 - bf16_lo(p1), b1 - bf16_hi(p1));
}

// the pieces of 8 values (slots 0..3 in lo, 4..7 in hi) as three fragments
__device__ __forceinline__ void split8(f32x4 lo, f32x4 hi, u32x4 (&pc)[3]) {
    uint32_t a[3], b[3], c[3], d[3];
    split2(lo.x, lo.y, a[0], a[1], a[2]);
    split2(lo.z, lo.w, b[0], b[1], b[2]);
    split2(hi.x, hi.y, c[0], c[1], c[2]);
    split2(hi.z, hi.w, d[0], d[1], d[2]);
#pragma unroll
    for (int q = 0; q < 3; ++q) pc[q] = u32x4{a[q], b[q], c[q], d[q]};
}

// The six piece pairs (a, b) of a split product, 0-based: (0,0) (0,1) (1,0)
// (0,2) (1,1) (2,0).  In the state update they are laid along k, two per
// 32-slot MFMA: MFMA m takes pair 2m in slots 0..15 and pair 2m+1 in 16..31.
__device__ constexpr int PAIR_A[6] = {0, 0, 1, 0, 1, 2};
__device__ constexpr int PAIR_B[6] = {0, 1, 0, 2, 1, 0};

__device__ __forceinline__ float load_state_elem(const float* s) { return *s; }
__device__ __forceinline__ float load_state_elem(const uint16_t* s) { return bf16_lo(*s); }
__device__ __forceinline__ void store_state_elem(float* s, float v) { *s = v; }
__device__ __forceinline__ void store_state_elem(uint16_t* s, float v) { *s = (uint16_t)f32_to_bf16_rne(v); }

// Cross-lane moves inside 16-lane rows (DPP, no LDS round trip): rotate by 8
// (lane i <-> i ^ 8), mirror inside each 8-lane half, swaps inside quads.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_ROW_ROR8 = 0x128, DPP_HALF_MIRROR = 0x141, DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E;

// Sums over the 64 lanes of a wave for 16 values at once.  Each exchange
// halves the values a lane carries: lane bit 3 picks tokens 8..15 (partner
// across the row rotation by 8), bit 2 the upper four of those (partner in
// the mirrored half-row), bit 5 and bit 4 (partners 32 and 16 lanes away,
// the only exchanges that leave the row); the last four lanes of a quad then
// add up.  Lane l ends with the total of token 8 b3 + 4 b2 + 2 b5 + b4 of l;
// sum16_lane(j) is a lane that holds token j's total.
__device__ __forceinline__ float wave_sum16(const float (&v)[PC], int lane) {
    float a8[8], a4[4], a2[2];
    const bool b3 = lane & 8, b2 = lane & 4, b5 = lane & 32, b4 = lane & 16;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float keep = b3 ? v[k + 8] : v[k], send = b3 ? v[k] : v[k + 8];
        a8[k] = keep + dpp_mov<DPP_ROW_ROR8>(send);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float keep = b2 ? a8[k + 4] : a8[k], send = b2 ? a8[k] : a8[k + 4];
        a4[k] = keep + dpp_mov<DPP_HALF_MIRROR>(send);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float keep = b5 ? a4[k + 2] : a4[k], send = b5 ? a4[k] : a4[k + 2];
        a2[k] = keep + __shfl_xor(send, 32, 64);
    }
    float t = (b4 ? a2[1] : a2[0]) + __shfl_xor(b4 ? a2[0] : a2[1], 16, 64);
    t += dpp_mov<DPP_QUAD_XOR1>(t);
    t += dpp_mov<DPP_QUAD_XOR2>(t);
    return t;
}

constexpr int sum16_lane(int j) { return 8 * (j >> 3) + 4 * ((j >> 2) & 1) + 32 * ((j >> 1) & 1) + 16 * (j & 1); }

__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// One column of (I + A) X = Diag(beta) R, right-looking, in place in cv:
// c_i holds R_i minus the columns already solved, x_j = beta_j c_j once every
// earlier column is in.  Z[0] + Z[1] (the two channel halves) holds
// A'[i][j] at [j][i] (A = StrictTril(Diag(beta) A')).
// The 256 entries of Z sit in the wave's registers (lane j + 16 (i / 4),
// element i % 4) and beta in lanes 0..15; each coefficient comes to the
// whole wave with one v_readlane, so the 16-step chain never waits on LDS.
__device__ __forceinline__ void solve_column(float (&cv)[PC], const float (*Z)[PC][LT], const float* beta, int lane) {
    const f32x4 zv = lds4(&Z[0][lane & 15][4 * (lane >> 4)]) + lds4(&Z[1][lane & 15][4 * (lane >> 4)]);
    const float bv = beta[lane & 15];
#pragma unroll
    for (int j = 0; j < PC; ++j) {
        const float xj = lane_value(bv, j) * cv[j];
        cv[j] = xj;
#pragma unroll
        for (int i = j + 1; i < PC; ++i) cv[i] = fmaf(-lane_value(zv[i & 3], j + 16 * (i >> 2)), xj, cv[i]);
    }
}

}  // namespace

// NS workgroups per (stream, head), each owning 128 / NS value columns of
// the state (the columns evolve independently: only the state products,
// the update and the outputs are split; the inputs, A, P and the solves are
// computed by each).  x [M][L][3][H*D], fgate [M][L][H*D], blogit [M][L][H],
// o [M][L][H][D].
template <typename TS, int NS>
__global__ __launch_bounds__(PNT, 2)
void prefill_kernel(const Ptrs p, const int L)
{
    static_assert(NS == 1 || NS == 2, "one or two workgroups per head");
    constexpr int NTW = 2 / NS;                        // 16-column tiles per wave
    __shared__ PrefillSmem sm;
    const int unit = (int)blockIdx.x / NS, split = (int)blockIdx.x - unit * NS;
    const int m = unit / p.H, h = unit - m * p.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform: roles branch on it
    const int l16 = lane & 15, g4 = lane >> 4;
    const size_t HD = (size_t)p.H * PD, C3 = 3 * HD;
    const int ncol = (PD / NS) * split + 16 * NTW * wv;   // this wave's value columns

    // ---- the state, in the MFMA output layout ----
    TS* const st = static_cast<TS*>(p.state) + (size_t)unit * PD * PD;
    float S[8][NTW][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][nt][r] = load_state_elem(st + (size_t)(16 * mt + 4 * g4 + r) * PD + ncol + 16 * nt + l16);

    // ---- per-lane constants of the input phase ----
    // waves 0, 1: channels 2 lane, 2 lane + 1 of q (wave 0) or k (wave 1);
    // waves 2, 3: channel vc = 64 (wave - 2) + lane of v and of the forget
    // gate, so that the gate's transcendentals (four per element against
    // two for a conv output) are shared by two waves rather than loading the
    // fourth SIMD alone.  Wave 3's lanes 0..15 also take the write strength.
    const bool qk = wv < 2;
    const int vc = 64 * (wv & 1) + lane;
    const size_t ch = qk ? (size_t)wv * HD + (size_t)h * PD + 2 * lane : 2 * HD + (size_t)h * PD + vc;
    const size_t fc = (size_t)h * PD + vc;              // gate channel (waves 2, 3)
    float cw[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float a0 = 0.f, a1 = 0.f, a2 = 0.f;                // raw inputs of the 3 previous tokens, channel 2 lane (or vc)
    float b0 = 0.f, b1 = 0.f, b2 = 0.f;                // the same, channel 2 lane + 1 (waves 0, 1)
    const float eA = expf(p.A_log[h]);
    const float lb = p.lower_bound;
    const uint16_t* ci = p.conv_in + (size_t)m * 3 * C3 + ch;
    float db = 0.f;
    if (qk) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p.conv_w + 4 * ch);
        cw[0] = bf16_lo(w.x); cw[1] = bf16_hi(w.x); cw[2] = bf16_lo(w.y); cw[3] = bf16_hi(w.y);
        cw[4] = bf16_lo(w.z); cw[5] = bf16_hi(w.z); cw[6] = bf16_lo(w.w); cw[7] = bf16_hi(w.w);
        const uint32_t t0v = *reinterpret_cast<const uint32_t*>(ci);
        const uint32_t t1v = *reinterpret_cast<const uint32_t*>(ci + C3);
        const uint32_t t2v = *reinterpret_cast<const uint32_t*>(ci + 2 * C3);
        a0 = bf16_lo(t0v); a1 = bf16_lo(t1v); a2 = bf16_lo(t2v);
        b0 = bf16_hi(t0v); b1 = bf16_hi(t1v); b2 = bf16_hi(t2v);
    } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p.conv_w + 4 * ch);
        cw[0] = bf16_lo(w.x); cw[1] = bf16_hi(w.x); cw[2] = bf16_lo(w.y); cw[3] = bf16_hi(w.y);
        a0 = bf16_lo(ci[0]); a1 = bf16_lo(ci[C3]); a2 = bf16_lo(ci[2 * C3]);
        db = p.dt_bias[fc];
    }

    // raw inputs of one chunk, two 16-bit streams per lane: waves 0, 1 the
    // bf16 of channels 2 lane (raw) and 2 lane + 1 (rawf) of q or k; waves
    // 2, 3 the bf16 of v (raw) and of the forget-gate projection (rawf); and
    // in every wave the write-strength logit of token lane % 16 (used by
    // wave 3).  Every wave issues the same loads from pointers chosen by its
    // role, so the loaded registers are the loop-carried ones: loads written
    // per role make the compiler copy the registers where the role paths
    // join, which waits for the loads right after issuing them.  Past the
    // end of the sequence the last token is read again; its results are
    // masked out.
    const uint16_t* const s1 = p.x + (size_t)m * L * C3 + ch;
    const uint16_t* const s2 = qk ? s1 + 1 : p.fgate + (size_t)m * L * HD + fc;
    const size_t d2 = qk ? C3 : HD;                     // token stride of s2
    const uint16_t* const sb = p.blogit + (size_t)m * L * p.H + h;
    uint32_t raw[PC], rawf[PC], rawb;
    auto fetch = [&](int t0) {
        const int last = min(PC, L - t0) - 1;
#pragma unroll
        for (int j = 0; j < PC; ++j) {
            const size_t t = (size_t)(t0 + min(j, last));
            raw[j] = s1[t * C3];
            rawf[j] = s2[t * d2];
        }
        rawb = sb[(size_t)(t0 + min(lane & (PC - 1), last)) * p.H];
    };
    fetch(0);

    const bool prio = L > 4 * PC;
    for (int t0 = 0; t0 < L; t0 += PC) {
        const int n = min(PC, L - t0);

        // ---- 1. inputs ----
        if (qk) {
            // tokens past the end give 0 (the carried taps are then stale,
            // but only the last chunk has such tokens); SiLU(0) = 0, so the
            // argument is masked rather than the result (no branch)
            float z0[PC], z1[PC];
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const float x0 = bf16_lo(raw[j]), x1 = bf16_lo(rawf[j]);
                float y0 = cw[0] * a0;
                y0 = fmaf(cw[1], a1, y0);
                y0 = fmaf(cw[2], a2, y0);
                y0 = fmaf(cw[3], x0, y0);
                float y1 = cw[4] * b0;
                y1 = fmaf(cw[5], b1, y1);
                y1 = fmaf(cw[6], b2, y1);
                y1 = fmaf(cw[7], x1, y1);
                z0[j] = silu_hw(j < n ? y0 : 0.f);
                z1[j] = silu_hw(j < n ? y1 : 0.f);
                a0 = a1; a1 = a2; a2 = x0;
                b0 = b1; b1 = b2; b2 = x1;
            }
            float (*dst)[LS] = wv == 0 ? sm.qi[0] : sm.kh;
            float ss[PC];
#pragma unroll
            for (int j = 0; j < PC; ++j) ss[j] = fmaf(z0[j], z0[j], z1[j] * z1[j]);
            const float tot = wave_sum16(ss, lane);
            const float rn = (wv == 0 ? p.scale : 1.0f) * rsqrtf(tot + 1e-6f);
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const float rj = lane_value(rn, sum16_lane(j));
                *reinterpret_cast<float2*>(&dst[j][2 * lane]) = make_float2(z0[j] * rj, z1[j] * rj);
            }
        } else {
            // v: conv + SiLU as above.  Gate: g = lb * sigmoid(exp(A) (f + b)),
            // alpha = e^g; Gamma_j is the running product of alpha from the
            // chunk start (the decay the per-token recurrence applies between
            // the chunk start and j)
            float e = 1.f;
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const float x0 = bf16_lo(raw[j]);
                float y0 = cw[0] * a0;
                y0 = fmaf(cw[1], a1, y0);
                y0 = fmaf(cw[2], a2, y0);
                y0 = fmaf(cw[3], x0, y0);
                sm.vv[j][vc] = silu_hw(j < n ? y0 : 0.f);
                a0 = a1; a1 = a2; a2 = x0;
                const float g = lb * sigmoid_hw(eA * (bf16_lo(rawf[j]) + db));
                e *= exp_hw(j < n ? g : 0.f);
                sm.eg[j][vc] = e;
                sm.qi[1][j][vc] = __builtin_amdgcn_rcpf(e);
            }
            sm.gam[vc] = e;
            if (wv == 3 && lane < PC)
                sm.beta[lane] = lane < n ? sigmoid_hw(bf16_lo(rawb)) : 0.0f;
        }
        if (t0 + PC < L) fetch(t0 + PC);
        lds_barrier();

        // ---- 2. A (waves 0, 1) and P (waves 2, 3), each wave one half of the
        // channels; then the bf16 pieces of the A operands of phases 4 and 5 ----
        {
            // lane / 16 takes channels [cb + 16 (lane / 16), cb + 16 (lane / 16) + 16)
            const int cb = 64 * (wv & 1);
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            if (wv < 2) {
                // D[i][j] = sum_c (Gamma k^)[i][c] (k^ / Gamma)[j][c] = Z[j][i]
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = cb + 16 * g4 + 4 * q;
                    const f32x4 k4 = lds4(&sm.kh[l16][c]), e4 = lds4(&sm.eg[l16][c]), i4 = lds4(&sm.qi[1][l16][c]);
                    acc0 = mfma16(k4.x * e4.x, k4.x * i4.x, acc0);
                    acc1 = mfma16(k4.y * e4.y, k4.y * i4.y, acc1);
                    acc0 = mfma16(k4.z * e4.z, k4.z * i4.z, acc0);
                    acc1 = mfma16(k4.w * e4.w, k4.w * i4.w, acc1);
                }
                *reinterpret_cast<f32x4*>(&sm.Z[wv & 1][l16][4 * g4]) = acc0 + acc1;
            } else {
                // D[s][t] = sum_c (k^ / Gamma)[s][c] (Gamma q^)[t][c] = P[t][s]
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = cb + 16 * g4 + 4 * q;
                    const f32x4 k4 = lds4(&sm.kh[l16][c]), i4 = lds4(&sm.qi[1][l16][c]);
                    const f32x4 q4 = lds4(&sm.qi[0][l16][c]), e4 = lds4(&sm.eg[l16][c]);
                    acc0 = mfma16(k4.x * i4.x, q4.x * e4.x, acc0);
                    acc1 = mfma16(k4.y * i4.y, q4.y * e4.y, acc1);
                    acc0 = mfma16(k4.z * i4.z, q4.z * e4.z, acc0);
                    acc1 = mfma16(k4.w * i4.w, q4.w * e4.w, acc1);
                }
                f32x4 d = acc0 + acc1;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g4 + r > l16) d[r] = 0.f;     // keep s <= t
                *reinterpret_cast<f32x4*>(&sm.P[wv & 1][l16][4 * g4]) = d;
            }
            // Gamma . q^: fragment (32-row block kb, lane ln) holds token ln % 16
            // at the 8 state rows the state's own lanes carry
            {
                const int kb = tid >> 6, ln = tid & 63, tk = ln & 15, c0 = 32 * kb + 4 * (ln >> 4);
                u32x4 pc[3];
                split8(lds4(&sm.qi[0][tk][c0]) * lds4(&sm.eg[tk][c0]),
                       lds4(&sm.qi[0][tk][c0 + 16]) * lds4(&sm.eg[tk][c0 + 16]), pc);
#pragma unroll
                for (int q = 0; q < 2; ++q) sm.gqp[q][kb][ln] = pc[q];
            }
            // (gamma_C / Gamma) . k^: fragment (row tile mt, token half hf, row)
            // holds 8 tokens of state row 16 mt + row
            {
                const int mt = tid >> 5, hf = (tid >> 4) & 1, k = 16 * mt + (tid & 15);
                const float gk = sm.gam[k];
                float v[8];
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) v[s2] = sm.kh[8 * hf + s2][k] * (gk * sm.qi[1][8 * hf + s2][k]);
                u32x4 pc[3];
                split8(f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]}, pc);
#pragma unroll
                for (int q = 0; q < 3; ++q) sm.ktp[q][mt][hf][tid & 15] = pc[q];
            }
        }
        lds_barrier();

        // Wave priority: the two workgroups on a CU drift out of step, and the
        // phases on the serial path of a chunk go first -- the solves (a
        // 16-step chain of readlane and FMA per column) highest, the state
        // products and the update next -- so that the other workgroup's
        // vector-bound inputs, A and P fill their gaps rather than delay them
        // (8 x 2048 f32: 1.23 -> 1.10 ms per layer).  Only for sequences of
        // more than 4 chunks: with fewer, the state's load and store, which
        // run at the base priority, are a large part of a workgroup's life,
        // and delaying them costs more (32 x 16 f32: 69 -> 75 us).
        if (prio) __builtin_amdgcn_s_setprio(2);
        // ---- 3. (I + A) W = Diag(beta)(Gamma . K), (I + A) U = Diag(beta) V ----
        // Waves 0, 1 solve for W (stored negated), waves 2, 3 for U.
        {
            const int col = tid & (PD - 1);
            float (*X)[LS] = wv < 2 ? sm.kh : sm.vv;
            float cv[PC];
            if (wv < 2) {
#pragma unroll
                for (int j = 0; j < PC; ++j) cv[j] = sm.kh[j][col] * sm.eg[j][col];
            } else {
#pragma unroll
                for (int j = 0; j < PC; ++j) cv[j] = sm.vv[j][col];
            }
            solve_column(cv, sm.Z, sm.beta, lane);
            // each thread reads and overwrites only its own column of k^ or v
            const float sg = wv < 2 ? -1.0f : 1.0f;
#pragma unroll
            for (int j = 0; j < PC; ++j) X[j][col] = cv[j] * sg;
        }
        lds_barrier();

        // ---- 4. Delta = U - W S and (Gamma . Q) S, this wave's 32 value columns ----
        if (prio) __builtin_amdgcn_s_setprio(1);
        // Per 32-row block of the state: the lane's 8 state values of each
        // column tile (rows 32 kb + 4 (lane / 16) + {0..3, 16..19}: its own
        // registers) are the B fragment; the A fragments (-W and Gamma . q^
        // of token lane % 16 at the same rows) come split from LDS.  Six bf16
        // products per pair of split operands for W S (the state's path),
        // the first three of them for (Gamma . Q) S (the output's).
        // -W is split once: wave w splits 32-row block w for every wave (the
        // barrier below waits for all four blocks behind the split of the
        // state's block 0, which needs no LDS).
        {
            u32x4 wq[3];
            split8(lds4(&sm.kh[l16][32 * wv + 4 * g4]), lds4(&sm.kh[l16][32 * wv + 16 + 4 * g4]), wq);
#pragma unroll
            for (int q = 0; q < 3; ++q) sm.wpk[wv][q][lane] = wq[q];
        }
        f32x4 dacc[NTW], oacc[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) dacc[nt][r] = sm.vv[4 * g4 + r][ncol + 16 * nt + l16];
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            u32x4 sb[NTW][3], wp[3], gp[2];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
                split8(f32x4{S[2 * kb][nt][0], S[2 * kb][nt][1], S[2 * kb][nt][2], S[2 * kb][nt][3]},
                       f32x4{S[2 * kb + 1][nt][0], S[2 * kb + 1][nt][1], S[2 * kb + 1][nt][2], S[2 * kb + 1][nt][3]},
                       sb[nt]);
            if (kb == 0) lds_barrier();
#pragma unroll
            for (int q = 0; q < 3; ++q) wp[q] = sm.wpk[kb][q][lane];                                  // -W
#pragma unroll
            for (int q = 0; q < 2; ++q) gp[q] = sm.gqp[q][kb][lane];
#pragma unroll
            for (int pr = 0; pr < 6; ++pr)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    dacc[nt] = mfma_bf16(wp[PAIR_A[pr]], sb[nt][PAIR_B[pr]], dacc[nt]);
                    if (pr < 3) oacc[nt] = mfma_bf16(gp[PAIR_A[pr]], sb[nt][PAIR_B[pr]], oacc[nt]);
                }
        }
        // Delta replaces Gamma, which nobody reads any more; its pieces go
        // where q^ and 1 / Gamma were: this lane's 4 tokens 4 (lane / 16) + r
        // are half of the fragment of token half (lane / 32)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.eg[4 * g4 + r][ncol + 16 * nt + l16] = dacc[nt][r];
            uint32_t p0a, p1a, p2a, p0b, p1b, p2b;
            split2(dacc[nt][0], dacc[nt][1], p0a, p1a, p2a);
            split2(dacc[nt][2], dacc[nt][3], p0b, p1b, p2b);
            u32x2* const dst = reinterpret_cast<u32x2*>(&sm.dp[0][wv][nt][g4 >> 1][l16]) + (g4 & 1);
            constexpr int PIECE = sizeof(sm.dp[0]) / sizeof(u32x2);
            dst[0] = u32x2{p0a, p0b};
            dst[PIECE] = u32x2{p1a, p1b};
            dst[2 * PIECE] = u32x2{p2a, p2b};
        }
        // phase 5 reads only this wave's columns of Delta and its own pieces
        lds_wave_fence();

        // ---- 5. O = (Gamma . Q) S + P Delta; S' = Diag(gamma_C) S + ((gamma_C / Gamma) . K)^T Delta ----
        // contraction over tokens: the k slot lane / 16 is token 4 (lane / 16) + kk
        float dl[NTW][4];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) dl[nt][kk] = sm.eg[4 * g4 + kk][ncol + 16 * nt + l16];
        {
            const f32x4 p4 = lds4(&sm.P[0][l16][4 * g4]) + lds4(&sm.P[1][l16][4 * g4]);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) oacc[nt] = mfma16(p4[kk], dl[nt][kk], oacc[nt]);
                const int col = ncol + 16 * nt + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * g4 + r;
                    if (t < n)
                        p.o[(((size_t)m * L + t0 + t) * p.H + h) * PD + col] = (uint16_t)f32_to_bf16_rne(oacc[nt][r]);
                }
            }
        }
        // state update: the contraction runs over the 16 tokens of each of
        // the six piece pairs, 96 k slots = three MFMAs; lane / 16 = 2 s + hh
        // takes pair 2 m + s, tokens 8 hh .. 8 hh + 7
        {
            const int hh = g4 & 1, sel = g4 >> 1;
            u32x4 db[3][NTW];
#pragma unroll
            for (int mm = 0; mm < 3; ++mm)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    db[mm][nt] = sm.dp[sel ? PAIR_B[2 * mm + 1] : PAIR_B[2 * mm]][wv][nt][hh][l16];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const f32x4 gm = lds4(&sm.gam[16 * mt + 4 * g4]);
                u32x4 ka[3];
#pragma unroll
                for (int mm = 0; mm < 3; ++mm) ka[mm] = sm.ktp[sel ? PAIR_A[2 * mm + 1] : PAIR_A[2 * mm]][mt][hh][l16];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    f32x4 acc = {S[mt][nt][0] * gm.x, S[mt][nt][1] * gm.y, S[mt][nt][2] * gm.z, S[mt][nt][3] * gm.w};
#pragma unroll
                    for (int mm = 0; mm < 3; ++mm) acc = mfma_bf16(ka[mm], db[mm][nt], acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[mt][nt][r] = acc[r];
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // the next chunk's inputs overwrite every array above
        lds_barrier();
    }

    // the lane's offset into the state, recomputed here so that the compiler
    // does not keep 64 addresses alive across the sweep
    int so = 4 * g4 * PD + ncol + l16;
    asm volatile("" : "+v"(so));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_state_elem(st + so + (16 * mt + r) * PD + 16 * nt, S[mt][nt][r]);
    // conv state after the sequence: the raw inputs of positions L-3, L-2,
    // L-1, where a position < 0 is a cached tap (read before this lane
    // overwrites it: conv_out may be conv_in, and each lane owns its channels;
    // with NS = 2 the first workgroup of the head writes it, and the host
    // requires conv_out != conv_in, since the other one reads conv_in)
    if (split == 0) {
        uint16_t* co = p.conv_out + (size_t)m * 3 * C3 + ch;
        if (qk) {
            uint32_t nt3[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int pos = L - 3 + k;
                nt3[k] = pos < 0 ? *reinterpret_cast<const uint32_t*>(ci + (size_t)(3 + pos) * C3)
                                 : *reinterpret_cast<const uint32_t*>(p.x + ((size_t)m * L + pos) * C3 + ch);
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) *reinterpret_cast<uint32_t*>(co + (size_t)k * C3) = nt3[k];
        } else {
            uint16_t nt3[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int pos = L - 3 + k;
                nt3[k] = pos < 0 ? ci[(size_t)(3 + pos) * C3] : p.x[((size_t)m * L + pos) * C3 + ch];
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) co[(size_t)k * C3] = nt3[k];
        }
    }
}

// ---------------------------------------------------------------------------
// Two-pass form.  "GLM-5.3 deep dive" 8.2.5 computes each chunk's intra-chunk
// matrices without the state (parallel over chunks) and carries only the
// state from chunk to chunk (sequential).  Pass 1 (prep_kernel) does phases 1
// to 3 for every (stream, head, chunk) at once -- conv + SiLU, gate, beta,
// norms, A, P and both solves -- and writes a record per chunk; pass 2
// (scan_kernel) sweeps each head's chunks in order doing only phases 4 and 5.
// A single long prompt then fills the device in pass 1, and pass 2's serial
// chain holds no input or solve work.
//
// Record of one (stream, head, chunk), in 16-byte units, each array in the
// fragment order pass 2 reads (lane-major, so a wave's read is contiguous):
//   Wp [4 kb][3 piece][64 lane]   -W split three ways, A operand of W S
//   Gq [4 kb][2 piece][64 lane]   Gamma . q^ split two ways, A operand of (Gamma . Q) S
//   Kt [3 piece][8 mt][2 hf][16]  (gamma_C / Gamma) . k^ split three ways, A operand of the update
//   P  [64 lane]                  Tril((Gamma . q^)(k^ / Gamma)^T) as the f32 MFMA A operand
//   Gm [32]                       gamma_C, 4 channels per unit
//   U  [8 ct][64 lane]            U of column tile ct, the D layout of a 16 x 16 tile
namespace {
constexpr int R_WP = 0;
constexpr int R_GQ = R_WP + 4 * 3 * 64;
constexpr int R_KT = R_GQ + 4 * 2 * 64;
constexpr int R_P = R_KT + 3 * 8 * 2 * 16;
constexpr int R_GM = R_P + 64;
constexpr int R_SHARED = R_GM + 32;     // the part every column tile reads
constexpr int R_U = R_SHARED;
constexpr int R_SIZE = R_U + 8 * 64;    // 2656 units = 42,496 bytes

}  // namespace

size_t prefill_record_bytes() { return (size_t)R_SIZE * 16; }

namespace {

struct PrepSmem {
    float kh[PC][LS];              // k^; after the solve, -W
    float vv[PC][LS];              // v; after the solve, U
    float eg[PC][LS];              // Gamma
    float qi[2][PC][LS];           // [0] q^ (normalised, scaled), [1] 1 / Gamma
    float Z[2][PC][LT];            // as PrefillSmem
    float P[2][PC][LT];
    float gam[PD];
    float beta[PC];
};

// Pass 1: one workgroup of 4 waves per (group of cpw chunks, stream, head) of
// a segment of nch chunks starting at chunk c0; block b = (group, m, h)
// row-major.  Per chunk, phases 1 to 3 as prefill_kernel; the raw inputs of
// the group's next chunk are requested while the current one runs phases 2
// and 3, and the three raw inputs before each chunk are carried from the
// previous one (read from x, or for the sequence's first chunk from the
// cached taps, at the start of the group).  Chunk cl of the segment writes
// record (cl, m, h).
__global__ __launch_bounds__(PNT, 3)
void prep_kernel(const Ptrs p, const int L, const int M, const int c0, const int nch, const int cpw,
                 u32x4* __restrict__ ws)
{
    __shared__ PrepSmem sm;
    const int b = (int)blockIdx.x;
    const int h = b % p.H, mg = b / p.H, m = mg % M, grp = mg / M;
    const int cl0 = grp * cpw, cl1 = min(nch, cl0 + cpw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const size_t HD = (size_t)p.H * PD, C3 = 3 * HD;

    const bool qk = wv < 2;
    const int vc = 64 * (wv & 1) + lane;
    const size_t ch = qk ? (size_t)wv * HD + (size_t)h * PD + 2 * lane : 2 * HD + (size_t)h * PD + vc;
    const size_t fc = (size_t)h * PD + vc;
    const uint16_t* const s1 = p.x + (size_t)m * L * C3 + ch;
    const uint16_t* const s2 = p.fgate + (size_t)m * L * HD + fc;
    const uint16_t* const ci = p.conv_in + (size_t)m * 3 * C3 + ch;
    const float eA = expf(p.A_log[h]);
    const float lb = p.lower_bound;

    // conv weights and the three raw inputs before the group's first chunk
    float cw[8], a0, a1, a2, b0 = 0.f, b1 = 0.f, b2 = 0.f, db = 0.f;
    {
        const int t0 = (c0 + cl0) * PC;
        uint32_t prev[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int pos = t0 - 3 + k;
            const uint16_t* src = pos < 0 ? ci + (size_t)(3 + pos) * C3 : s1 + (size_t)pos * C3;
            prev[k] = qk ? *reinterpret_cast<const uint32_t*>(src) : (uint32_t)*src;
        }
        a0 = bf16_lo(prev[0]); a1 = bf16_lo(prev[1]); a2 = bf16_lo(prev[2]);
        if (qk) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(p.conv_w + 4 * ch);
            cw[0] = bf16_lo(w.x); cw[1] = bf16_hi(w.x); cw[2] = bf16_lo(w.y); cw[3] = bf16_hi(w.y);
            cw[4] = bf16_lo(w.z); cw[5] = bf16_hi(w.z); cw[6] = bf16_lo(w.w); cw[7] = bf16_hi(w.w);
            b0 = bf16_hi(prev[0]); b1 = bf16_hi(prev[1]); b2 = bf16_hi(prev[2]);
        } else {
            const u32x2 w = *reinterpret_cast<const u32x2*>(p.conv_w + 4 * ch);
            cw[0] = bf16_lo(w.x); cw[1] = bf16_hi(w.x); cw[2] = bf16_lo(w.y); cw[3] = bf16_hi(w.y);
            cw[4] = cw[5] = cw[6] = cw[7] = 0.f;
            db = p.dt_bias[fc];
        }
    }

    // raw inputs of one chunk (the last token again past the end of the
    // sequence; its results are masked out): q/k waves two channels per
    // 32-bit load, v/gate waves the v and forget-gate channel; every lane
    // the write-strength logit of token lane % 16
    uint32_t raw[PC], rawf[PC], rawb;
    auto fetch = [&](int t0) {
        const int last = min(PC, L - t0) - 1;
#pragma unroll
        for (int j = 0; j < PC; ++j) {
            const size_t t = (size_t)(t0 + min(j, last));
            raw[j] = qk ? *reinterpret_cast<const uint32_t*>(s1 + t * C3) : (uint32_t)s1[t * C3];
            rawf[j] = qk ? 0u : (uint32_t)s2[t * HD];
        }
        rawb = p.blogit[((size_t)m * L + t0 + min(lane & (PC - 1), last)) * p.H + h];
    };
    fetch((c0 + cl0) * PC);

    for (int cl = cl0; cl < cl1; ++cl) {
        const int t0 = (c0 + cl) * PC;
        const int n = min(PC, L - t0);
        u32x4* const rec = ws + ((size_t)cl * M + m) * p.H * R_SIZE + (size_t)h * R_SIZE;

        // ---- 1. inputs ----
        if (qk) {
            float z0[PC], z1[PC];
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const float x0 = bf16_lo(raw[j]), x1 = bf16_hi(raw[j]);
                float y0 = cw[0] * a0;
                y0 = fmaf(cw[1], a1, y0);
                y0 = fmaf(cw[2], a2, y0);
                y0 = fmaf(cw[3], x0, y0);
                float y1 = cw[4] * b0;
                y1 = fmaf(cw[5], b1, y1);
                y1 = fmaf(cw[6], b2, y1);
                y1 = fmaf(cw[7], x1, y1);
                z0[j] = silu_hw(j < n ? y0 : 0.f);
                z1[j] = silu_hw(j < n ? y1 : 0.f);
                a0 = a1; a1 = a2; a2 = x0;
                b0 = b1; b1 = b2; b2 = x1;
            }
            float (*dst)[LS] = wv == 0 ? sm.qi[0] : sm.kh;
            float ss[PC];
#pragma unroll
            for (int j = 0; j < PC; ++j) ss[j] = fmaf(z0[j], z0[j], z1[j] * z1[j]);
            const float tot = wave_sum16(ss, lane);
            const float rn = (wv == 0 ? p.scale : 1.0f) * rsqrtf(tot + 1e-6f);
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const float rj = lane_value(rn, sum16_lane(j));
                *reinterpret_cast<float2*>(&dst[j][2 * lane]) = make_float2(z0[j] * rj, z1[j] * rj);
            }
        } else {
            float e = 1.f;
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                const float x0 = bf16_lo(raw[j]);
                float y0 = cw[0] * a0;
                y0 = fmaf(cw[1], a1, y0);
                y0 = fmaf(cw[2], a2, y0);
                y0 = fmaf(cw[3], x0, y0);
                sm.vv[j][vc] = silu_hw(j < n ? y0 : 0.f);
                a0 = a1; a1 = a2; a2 = x0;
                const float g = lb * sigmoid_hw(eA * (bf16_lo(rawf[j]) + db));
                e *= exp_hw(j < n ? g : 0.f);
                sm.eg[j][vc] = e;
                sm.qi[1][j][vc] = __builtin_amdgcn_rcpf(e);
            }
            sm.gam[vc] = e;
            if (wv == 3 && lane < PC)
                sm.beta[lane] = lane < n ? sigmoid_hw(bf16_lo(rawb)) : 0.0f;
        }
        if (cl + 1 < cl1) fetch(t0 + PC);
        lds_barrier();

        // ---- 2. A and P; the record's Gamma . q^ and (gamma_C / Gamma) . k^ pieces ----
        {
            const int cb = 64 * (wv & 1);
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            if (wv < 2) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = cb + 16 * g4 + 4 * q;
                    const f32x4 k4 = lds4(&sm.kh[l16][c]), e4 = lds4(&sm.eg[l16][c]), i4 = lds4(&sm.qi[1][l16][c]);
                    acc0 = mfma16(k4.x * e4.x, k4.x * i4.x, acc0);
                    acc1 = mfma16(k4.y * e4.y, k4.y * i4.y, acc1);
                    acc0 = mfma16(k4.z * e4.z, k4.z * i4.z, acc0);
                    acc1 = mfma16(k4.w * e4.w, k4.w * i4.w, acc1);
                }
                *reinterpret_cast<f32x4*>(&sm.Z[wv & 1][l16][4 * g4]) = acc0 + acc1;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = cb + 16 * g4 + 4 * q;
                    const f32x4 k4 = lds4(&sm.kh[l16][c]), i4 = lds4(&sm.qi[1][l16][c]);
                    const f32x4 q4 = lds4(&sm.qi[0][l16][c]), e4 = lds4(&sm.eg[l16][c]);
                    acc0 = mfma16(k4.x * i4.x, q4.x * e4.x, acc0);
                    acc1 = mfma16(k4.y * i4.y, q4.y * e4.y, acc1);
                    acc0 = mfma16(k4.z * i4.z, q4.z * e4.z, acc0);
                    acc1 = mfma16(k4.w * i4.w, q4.w * e4.w, acc1);
                }
                f32x4 d = acc0 + acc1;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g4 + r > l16) d[r] = 0.f;
                *reinterpret_cast<f32x4*>(&sm.P[wv & 1][l16][4 * g4]) = d;
            }
            {
                const int kb = tid >> 6, ln = tid & 63, tk = ln & 15, cq = 32 * kb + 4 * (ln >> 4);
                u32x4 pc[3];
                split8(lds4(&sm.qi[0][tk][cq]) * lds4(&sm.eg[tk][cq]),
                       lds4(&sm.qi[0][tk][cq + 16]) * lds4(&sm.eg[tk][cq + 16]), pc);
#pragma unroll
                for (int q = 0; q < 2; ++q) rec[R_GQ + (kb * 2 + q) * 64 + ln] = pc[q];
            }
            {
                const int mt = tid >> 5, hf = (tid >> 4) & 1, k = 16 * mt + (tid & 15);
                const float gk = sm.gam[k];
                float v[8];
#pragma unroll
                for (int s2i = 0; s2i < 8; ++s2i) v[s2i] = sm.kh[8 * hf + s2i][k] * (gk * sm.qi[1][8 * hf + s2i][k]);
                u32x4 pc[3];
                split8(f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]}, pc);
#pragma unroll
                for (int q = 0; q < 3; ++q) rec[R_KT + ((q * 8 + mt) * 2 + hf) * 16 + (tid & 15)] = pc[q];
            }
        }
        lds_barrier();

        // ---- 3. (I + A) W = Diag(beta)(Gamma . K), (I + A) U = Diag(beta) V ----
        {
            const int col = tid & (PD - 1);
            float (*X)[LS] = wv < 2 ? sm.kh : sm.vv;
            float cv[PC];
            if (wv < 2) {
#pragma unroll
                for (int j = 0; j < PC; ++j) cv[j] = sm.kh[j][col] * sm.eg[j][col];
            } else {
#pragma unroll
                for (int j = 0; j < PC; ++j) cv[j] = sm.vv[j][col];
            }
            solve_column(cv, sm.Z, sm.beta, lane);
            const float sg = wv < 2 ? -1.0f : 1.0f;
#pragma unroll
            for (int j = 0; j < PC; ++j) X[j][col] = cv[j] * sg;
        }
        lds_barrier();

        // ---- the record's -W pieces, U tiles, P and gamma_C ----
        {
            const int kb = wv;
            u32x4 wp[3];
            split8(lds4(&sm.kh[l16][32 * kb + 4 * g4]), lds4(&sm.kh[l16][32 * kb + 16 + 4 * g4]), wp);
#pragma unroll
            for (int q = 0; q < 3; ++q) rec[R_WP + (kb * 3 + q) * 64 + lane] = wp[q];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ct = 2 * wv + i, col = 16 * ct + l16;
                const f32x4 u = {sm.vv[4 * g4][col], sm.vv[4 * g4 + 1][col], sm.vv[4 * g4 + 2][col],
                                 sm.vv[4 * g4 + 3][col]};
                rec[R_U + ct * 64 + lane] = __builtin_bit_cast(u32x4, u);
            }
            if (wv == 0) {
                const f32x4 p4 = lds4(&sm.P[0][l16][4 * g4]) + lds4(&sm.P[1][l16][4 * g4]);
                rec[R_P + lane] = __builtin_bit_cast(u32x4, p4);
            } else if (wv == 1 && lane < 32) {
                rec[R_GM + lane] = __builtin_bit_cast(u32x4, lds4(&sm.gam[4 * lane]));
            }
        }
        // the next chunk's phase 1 overwrites what the record was read from
        lds_barrier();
    }
}

// Pass 2: per workgroup TPW column tiles of head (m, h), KS waves per tile,
// for chunks [c0, c0 + nch).  Tile ct = TPW * split + i covers value columns
// [16 ct, 16 ct + 16); its KS waves split the key rows: wave ks of the tile
// holds rows [128 ks / KS, 128 (ks + 1) / KS) (state blocks kb of 32 rows,
// KB = 4 / KS of them) in the D layout of the 16 x 16 MFMAs -- lane (l16, g4)
// holds rows 16 mt + 4 g4 + r of column 16 ct + l16.  Per chunk each wave
// forms its rows' share of W S (wave 0 of the tile starting from U) and of
// (Gamma . Q) S; the shares meet in LDS after a barrier and every wave of the
// tile adds them in the same order, so all hold the same Delta; each wave
// writes the outputs of 4 / KS of a lane's four tokens and updates its own
// rows.  The shared part of each chunk's record is staged in LDS,
// double-buffered: a chunk's part is fetched into registers two chunks ahead
// and written to the other buffer at the end of the chunk before it (two
// barriers per chunk).  The state comes from `sin` and goes to `sout`: the
// caller's state (type TS) at the ends of the call, f32 in the workspace
// between segments.
template <int TPW, int KS>
struct ScanSmem {
    // the shared record part, then the U tiles of the workgroup's TPW
    // column tiles, rounded up to whole staging rounds of its threads (the
    // units past them repeat the record's first ones and are not read)
    u32x4 rec[2][(R_SHARED + TPW * 64 + TPW * KS * 64 - 1) / (TPW * KS * 64) * (TPW * KS * 64)];
    f32x4 part[TPW * KS][2][64];       // [wave][W S share, (Gamma . Q) S share][lane]
    u32x4 dp[TPW * KS][3][2][16];      // Delta pieces [wave][piece][token half][column]
};

// the sum of the KS shares of one tile's waves w0 .. w0 + KS - 1, as a
// balanced tree (the same order in every wave)
template <int KS>
__device__ __forceinline__ f32x4 sum_shares(const f32x4 (*part)[2][64], int w0, int which, int lane) {
    if constexpr (KS == 2) {
        return part[w0][which][lane] + part[w0 + 1][which][lane];
    } else {
        return (part[w0][which][lane] + part[w0 + 1][which][lane]) +
               (part[w0 + 2][which][lane] + part[w0 + 3][which][lane]);
    }
}

template <typename TSI, typename TSO, int TPW, int KS>
__global__ __launch_bounds__(TPW * KS * 64)
void scan_kernel(const Ptrs p, const int L, const int M, const int c0, const int nch,
                 const u32x4* __restrict__ ws, const TSI* sin, TSO* sout, const int write_conv)
{
    static_assert(KS == 2 || KS == 4, "two or four waves per tile");
    constexpr int KB = 4 / KS;                         // 32-row state blocks per wave
    constexpr int NS = 8 / TPW;                        // workgroups per head
    constexpr int NT = TPW * KS * 64;
    constexpr int STAGED = R_SHARED + TPW * 64;        // shared part + this workgroup's U tiles
    constexpr int PER = (STAGED + NT - 1) / NT;        // 16-byte units each thread stages
    __shared__ ScanSmem<TPW, KS> sm;
    // XCD-aware: workgroups go to the 8 XCDs round robin; the NS workgroups of
    // a head sit on one XCD, so they read its records through one L2
    const int units = M * p.H;
    int unit, split;
    {
        const int b = (int)blockIdx.x;
        const int full = units >> 3;
        if (NS > 1 && b < full * 8 * NS) {
            const int g = b / (8 * NS), r = b - g * 8 * NS;
            unit = g * 8 + (r & 7);
            split = r >> 3;
        } else {
            const int bb = b - (NS > 1 ? full * 8 * NS : 0);
            unit = (NS > 1 ? full * 8 : 0) + bb / NS;
            split = bb - (bb / NS) * NS;
        }
    }
    const int m = unit / p.H, h = unit - m * p.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ks = wv % KS, ti = wv / KS, w0 = wv - ks;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int ct = TPW * split + ti, col = 16 * ct + l16;
    const size_t rstride = (size_t)M * p.H * R_SIZE;   // from one chunk's records to the next
    const u32x4* const rec0 = ws + (size_t)unit * R_SIZE;

    float S[2 * KB][4];
    {
        const TSI* const st = sin + (size_t)unit * PD * PD;
#pragma unroll
        for (int mi = 0; mi < 2 * KB; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mi][r] = load_state_elem(st + (size_t)(16 * (2 * KB * ks + mi) + 4 * g4 + r) * PD + col);
    }

    // Records are fetched two chunks ahead (their latency from HBM exceeds
    // a chunk's work): register set 0 holds even chunks, set 1 odd ones,
    // and the loop runs two chunks per iteration so that both sets stay
    // compile-time arrays.  Every thread issues the same loads on every
    // chunk (the index clamped to the last chunk, so the last two chunks
    // load a record again, unused), and they are consumed only by the
    // staging stores: with conditional loads, or loads consumed elsewhere,
    // the compiler cannot count the loads issued after a set's and waits for
    // all of them.  Unit e of the staged span is record unit e below
    // R_SHARED, then the U tiles of this workgroup's column tiles, then
    // repeats of the record's first units.
    // The loads are raw buffer loads over one record: a wave-uniform
    // descriptor per chunk and loop-invariant per-thread byte offsets, so no
    // address register is rewritten per chunk (a rewritten address register
    // that once held a load's result makes the compiler wait for loads
    // still in flight).
    int src[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = tid + i * NT;
        src[i] = 16 * (e < R_SHARED ? e : (e < STAGED ? R_U + TPW * split * 64 + (e - R_SHARED) : e - STAGED));
    }
    u32x4 stg0[PER], stg1[PER];
    auto fetch = [&](u32x4 (&stg)[PER], int c) {
        const auto rs = stream_rsrc(rec0 + (size_t)c * rstride, R_SIZE * 16);
#pragma unroll
        for (int i = 0; i < PER; ++i)
            stg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, src[i], 0, 0));
    };
    auto put = [&](const u32x4 (&stg)[PER], int buf) {
#pragma unroll
        for (int i = 0; i < PER; ++i) sm.rec[buf][tid + i * NT] = stg[i];
    };

    // chunk c from LDS buffer c & 1; `nxt` (chunk c + 1's record, fetched a
    // chunk ago) goes to the other buffer at the end, and `cur` (free once
    // chunk c's record is in LDS) takes chunk c + 2's
    auto chunk = [&](int c, u32x4 (&cur)[PER], const u32x4 (&nxt)[PER]) {
        const int buf = c & 1;
        const u32x4* const R = sm.rec[buf];
        const int t0 = (c0 + c) * PC;
        fetch(cur, min(c + 2, nch - 1));

        // ---- 4. this wave's share of Delta = U - W S and of (Gamma . Q) S ----
        u32x4 wp[KB][3], gp[KB][2];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int kb = KB * ks + i;
#pragma unroll
            for (int q = 0; q < 3; ++q) wp[i][q] = R[R_WP + (kb * 3 + q) * 64 + lane];
#pragma unroll
            for (int q = 0; q < 2; ++q) gp[i][q] = R[R_GQ + (kb * 2 + q) * 64 + lane];
        }
        f32x4 dk[KB], ok = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KB; ++i)
            dk[i] = (i == 0 && ks == 0) ? __builtin_bit_cast(f32x4, R[R_SHARED + ti * 64 + lane])
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            u32x4 sb[3];
            split8(f32x4{S[2 * i][0], S[2 * i][1], S[2 * i][2], S[2 * i][3]},
                   f32x4{S[2 * i + 1][0], S[2 * i + 1][1], S[2 * i + 1][2], S[2 * i + 1][3]}, sb);
#pragma unroll
            for (int pr = 0; pr < 6; ++pr) {
                dk[i] = mfma_bf16(wp[i][PAIR_A[pr]], sb[PAIR_B[pr]], dk[i]);
                if (pr < 3) ok = mfma_bf16(gp[i][PAIR_A[pr]], sb[PAIR_B[pr]], ok);
            }
        }
        // the update's operands from the record, read before the barrier
        const int hh = g4 & 1, sel = g4 >> 1;
        u32x4 ka[2 * KB][3];
        f32x4 gm[2 * KB];
#pragma unroll
        for (int mi = 0; mi < 2 * KB; ++mi) {
            const int mt = 2 * KB * ks + mi;
            gm[mi] = __builtin_bit_cast(f32x4, R[R_GM + 4 * mt + g4]);
#pragma unroll
            for (int mm = 0; mm < 3; ++mm) {
                const int q = sel ? PAIR_A[2 * mm + 1] : PAIR_A[2 * mm];
                ka[mi][mm] = R[R_KT + ((q * 8 + mt) * 2 + hh) * 16 + l16];
            }
        }
        if constexpr (KB == 2)
            sm.part[wv][0][lane] = dk[0] + dk[1];
        else
            sm.part[wv][0][lane] = dk[0];
        sm.part[wv][1][lane] = ok;
        lds_barrier();
        const f32x4 dacc = sum_shares<KS>(sm.part, w0, 0, lane);
        {
            uint32_t p0a, p1a, p2a, p0b, p1b, p2b;
            split2(dacc[0], dacc[1], p0a, p1a, p2a);
            split2(dacc[2], dacc[3], p0b, p1b, p2b);
            u32x2* const dst = reinterpret_cast<u32x2*>(&sm.dp[wv][0][g4 >> 1][l16]) + (g4 & 1);
            constexpr int PIECE = sizeof(sm.dp[0][0]) / sizeof(u32x2);
            dst[0] = u32x2{p0a, p0b};
            dst[PIECE] = u32x2{p1a, p1b};
            dst[2 * PIECE] = u32x2{p2a, p2b};
        }
        lds_wave_fence();

        // ---- 5. S' = Diag(gamma_C) S + ((gamma_C / Gamma) . K)^T Delta; O = (Gamma . Q) S + P Delta ----
        {
            u32x4 db[3];
#pragma unroll
            for (int mm = 0; mm < 3; ++mm) db[mm] = sm.dp[wv][sel ? PAIR_B[2 * mm + 1] : PAIR_B[2 * mm]][hh][l16];
#pragma unroll
            for (int mi = 0; mi < 2 * KB; ++mi) {
                f32x4 acc = {S[mi][0] * gm[mi].x, S[mi][1] * gm[mi].y, S[mi][2] * gm[mi].z, S[mi][3] * gm[mi].w};
#pragma unroll
                for (int mm = 0; mm < 3; ++mm) acc = mfma_bf16(ka[mi][mm], db[mm], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) S[mi][r] = acc[r];
            }
        }
        {
            // every wave of the tile forms the tile's outputs; each stores
            // 4 / KS of a lane's four tokens
            f32x4 oacc = sum_shares<KS>(sm.part, w0, 1, lane);
            const f32x4 p4 = __builtin_bit_cast(f32x4, R[R_P + lane]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) oacc = mfma16(p4[kk], dacc[kk], oacc);
            // a buffer store over this chunk's valid tokens: the hardware
            // drops the stores of tokens past the end of the sequence, so the
            // store is unconditional and the compiler counts it exactly when
            // it waits for the staged loads issued before it
            const int nvalid = min(PC, L - t0);
            const auto orsrc = stream_rsrc(p.o + (((size_t)m * L + t0) * p.H + h) * PD,
                                           nvalid * p.H * PD * (int)sizeof(uint16_t));
#pragma unroll
            for (int rr = 0; rr < 4 / KS; ++rr) {
                const int r = (4 / KS) * ks + rr;
                const int t = 4 * g4 + r;
                const float v = r == 0 ? oacc[0] : (r == 1 ? oacc[1] : (r == 2 ? oacc[2] : oacc[3]));
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(cvt_pk_bf16(v, 0.0f) & 0xffffu), orsrc,
                                                      (t * p.H * PD + col) * (int)sizeof(uint16_t), 0, 0);
            }
        }
        // the next chunk's shared record part into the other buffer; the
        // shares and Delta pieces are rewritten only after the barrier
        if (c + 1 < nch) put(nxt, buf ^ 1);
        lds_barrier();
    };

    fetch(stg0, 0);
    fetch(stg1, min(1, nch - 1));
    put(stg0, 0);
    lds_barrier();
    for (int c = 0; c < nch; c += 2) {
        chunk(c, stg0, stg1);
        if (c + 1 < nch) chunk(c + 1, stg1, stg0);
    }

    {
        int so = (128 / KS * ks + 4 * g4) * PD + col;
        asm volatile("" : "+v"(so));
        TSO* const st = sout + (size_t)unit * PD * PD + so;
#pragma unroll
        for (int mi = 0; mi < 2 * KB; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) store_state_elem(st + (16 * mi + r) * PD, S[mi][r]);
    }
    // conv state after the sequence (last segment only): the raw inputs of
    // positions L-3, L-2, L-1 of the workgroup's share of the head's q, k, v
    // channels, one channel per thread; a position < 0 is a cached tap, read
    // by the same thread before it overwrites it
    if (write_conv) {
        constexpr int CPS = PD / NS;                   // channels of each tensor per workgroup
        static_assert(3 * CPS <= NT, "one thread per channel");
        if (tid < 3 * CPS) {
            const size_t HD = (size_t)p.H * PD, C3 = 3 * HD;
            const int tensor = tid / CPS, c = split * CPS + (tid - tensor * CPS);
            const size_t chn = (size_t)tensor * HD + (size_t)h * PD + c;
            uint16_t v3[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int pos = L - 3 + k;
                v3[k] = pos < 0 ? p.conv_in[(size_t)m * 3 * C3 + (size_t)(3 + pos) * C3 + chn]
                                : p.x[((size_t)m * L + pos) * C3 + chn];
            }
            uint16_t* co = p.conv_out + (size_t)m * 3 * C3 + chn;
#pragma unroll
            for (int k = 0; k < 3; ++k) co[(size_t)k * C3] = v3[k];
        }
    }
}

}  // namespace

// Two-pass prefill over a caller workspace: the sequence runs in segments of
// as many chunks as the workspace holds records for (every stream and head
// of a chunk at once), pass 1 then pass 2 per segment.  Between segments the
// state is carried in f32: in the caller's state for f32 storage, in the
// workspace after the records for bf16 storage (so bf16 state is rounded
// once, at the end of the call, however many segments run).
template <typename TSI, typename TSO>
static hipError_t launch_scan(int tpw, int ks, const Ptrs& p, int L, int M, int c0, int nch, const u32x4* ws,
                              const void* sin, void* sout, int write_conv, int units, hipStream_t stream) {
    const TSI* si = static_cast<const TSI*>(sin);
    TSO* so = static_cast<TSO*>(sout);
    void* args[] = {(void*)&p, (void*)&L, (void*)&M, (void*)&c0, (void*)&nch, (void*)&ws, (void*)&si, (void*)&so,
                    (void*)&write_conv};
    const void* fn = tpw == 4 ? reinterpret_cast<const void*>(&scan_kernel<TSI, TSO, 4, 2>)
                              : reinterpret_cast<const void*>(&scan_kernel<TSI, TSO, 2, 4>);
    return hipLaunchKernel(fn, dim3((unsigned)(units * (8 / tpw))), dim3(tpw * ks * 64), args, 0, stream);
}

size_t prefill_state_stage_bytes(int M, int H) { return (size_t)M * H * PD * PD * sizeof(float); }

hipError_t launch_prefill_ws(const StepArgs& a, void* ws, size_t ws_bytes, int ncu) {
    if (a.D != PD) return hipErrorInvalidValue;
    Ptrs p = make_ptrs(a);
    const int L = a.T, M = a.M;
    const int units = M * a.H;
    const int nchunks = (L + PC - 1) / PC;
    const size_t per_chunk = (size_t)units * R_SIZE * 16;
    const bool bf16 = a.state_dtype != 0;
    // records of one segment; bf16 state also needs its f32 stage when the
    // sequence takes more than one segment
    size_t seg = ws_bytes / per_chunk;
    if ((long)seg < nchunks && bf16) {
        const size_t stage = prefill_state_stage_bytes(M, a.H);
        seg = ws_bytes > stage ? (ws_bytes - stage) / per_chunk : 0;
    }
    if (seg < 1) return hipErrorInvalidValue;
    const int seg_chunks = (int)((long)seg < nchunks ? (long)seg : nchunks);
    const int nseg = (nchunks + seg_chunks - 1) / seg_chunks;
    u32x4* const rec = static_cast<u32x4*>(ws);
    float* const stage = bf16 ? reinterpret_cast<float*>(static_cast<char*>(ws) + (size_t)seg_chunks * per_chunk)
                              : static_cast<float*>(a.state);
    // pass-2 workgroups: 2 column tiles of 4 waves each (one 32-row state
    // block per wave; 8 waves) while that gives at most one workgroup per
    // CU, else 4 tiles of 2 waves (8 waves; LDS allows one workgroup per CU)
    const long want = ncu > 0 ? ncu : 256;
    const int tpw = (long)units * 4 <= want ? 2 : 4;
    const int ks = tpw == 4 ? 2 : 4;
    const hipStream_t stream = (hipStream_t)a.stream;
    for (int sgi = 0; sgi < nseg; ++sgi) {
        int c0 = sgi * seg_chunks;
        const int nch = min(seg_chunks, nchunks - c0);
        {
            // chunks per pass-1 workgroup: several (their input latency then
            // hides behind the previous chunk's work) while the grid still
            // gives every CU about four rounds of three workgroups
            const long slots = 12L * want;
            int cpw = (int)((long)nch * units / slots);
            cpw = cpw < 1 ? 1 : (cpw > 8 ? 8 : cpw);
            int Li = L, Mi = M, nchi = nch;
            u32x4* w = rec;
            void* args[] = {(void*)&p, (void*)&Li, (void*)&Mi, (void*)&c0, (void*)&nchi, (void*)&cpw, (void*)&w};
            const long groups = (nch + cpw - 1) / cpw;
            hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&prep_kernel),
                                           dim3((unsigned)(groups * units)), dim3(PNT), args, 0, stream);
            if (e != hipSuccess) return e;
        }
        const bool first = sgi == 0, last = sgi == nseg - 1;
        const void* sin = first ? a.state : static_cast<const void*>(stage);
        void* sout = last ? a.state : static_cast<void*>(stage);
        hipError_t e;
        if (!bf16)
            e = launch_scan<float, float>(tpw, ks, p, L, M, c0, nch, rec, sin, sout, last, units, stream);
        else if (first && last)
            e = launch_scan<uint16_t, uint16_t>(tpw, ks, p, L, M, c0, nch, rec, sin, sout, last, units, stream);
        else if (first)
            e = launch_scan<uint16_t, float>(tpw, ks, p, L, M, c0, nch, rec, sin, sout, last, units, stream);
        else if (last)
            e = launch_scan<float, uint16_t>(tpw, ks, p, L, M, c0, nch, rec, sin, sout, last, units, stream);
        else
            e = launch_scan<float, float>(tpw, ks, p, L, M, c0, nch, rec, sin, sout, last, units, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Scratch memory of the allocation-free entry point: the two-pass form's
// workspace as a file-scope device array, one copy per GPU the library runs
// on, held until the process ends.  Host code never passes `scratch` itself
// (its host-side name is not a device address): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

size_t prefill_scratch_bytes() { return kScratchBytes; }

hipError_t prefill_scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Two workgroups per head when the heads alone would leave more than half
// of the CUs idle (the duplicated input, A, P and solve work then costs
// nothing but otherwise idle CUs) and conv_out is a buffer of its own.
hipError_t launch_prefill(const StepArgs& a) {
    if (a.D != PD) return hipErrorInvalidValue;
    Ptrs p = make_ptrs(a);
    int L = a.T;
    void* args[] = {(void*)&p, (void*)&L};
    int ncu = stream_cu_count(a.stream);
    if (ncu <= 0) ncu = 256;
    const long units = (long)a.M * a.H;
    const bool two = a.nsplit == 0 && a.conv_out != a.conv_in && 2 * units <= ncu;   // nsplit 0: choose
    const bool f32 = a.state_dtype == 0;
    const void* fn = two ? (f32 ? reinterpret_cast<const void*>(&prefill_kernel<float, 2>)
                                : reinterpret_cast<const void*>(&prefill_kernel<uint16_t, 2>))
                         : (f32 ? reinterpret_cast<const void*>(&prefill_kernel<float, 1>)
                                : reinterpret_cast<const void*>(&prefill_kernel<uint16_t, 1>));
    return hipLaunchKernel(fn, dim3((unsigned)(units * (two ? 2 : 1))), dim3(PNT), args, 0, (hipStream_t)a.stream);
}

}  // namespace kda
