// kda_prefill.hip -- chunked KDA over a sequence of tokens, on gfx950 MFMA.
//
// "GLM-5.3 deep dive" 8.2.5 (training in chunks: the WY representation and
// the UT transform), for one chunk of C tokens with incoming state S,
// cumulative per-channel decay Gamma (inclusive, from the chunk start),
// normalised keys K, scaled queries Q and values V (C-row matrices):
//
//   A     = StrictTril(Diag(beta) (Gamma . K) (K / Gamma)^T)
//   M     = (I + A)^-1 Diag(beta)                      forward substitution
//   W     = M (Gamma . K),   U = M V
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
// the head's chunks in order.  The head's 128 x 128 f32 state stays in the
// accumulator registers of v_mfma_f32_16x16x4f32 for the whole sequence:
// wave w owns value columns [32w, 32w + 32), each lane 64 state values in the
// instruction's output layout (row k = 16 mt + 4 (lane / 16) + r, column
// n = 32 w + 16 nt + lane % 16).  That layout is also a valid B operand for
// W S and (Gamma . Q) S when the contraction index is enumerated in the same
// order, so the state is never rearranged.  Per chunk the conv + SiLU, the
// gate, the norms and the decay products are formed elementwise into LDS,
// the small C x C products and the 16 x 16 triangular solve run on one or
// two waves, and the four products with the state run on all four waves.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int PD = 128;            // head width (dk = dv)
constexpr int PC = 16;             // chunk length, tokens
constexpr int PNT = 256;           // threads per workgroup (4 waves)
constexpr int PNG = 3 * PD / 4;    // conv channel groups of 4 per token (q, k, v)

struct PrefillSmem {
    float z[PC][3 * PD];           // conv outputs q | k | v; the q part later holds Delta
    float G[PC][PD];               // log decays, summed in place; later holds W
    float GK[PC][PD];              // Gamma . k^
    float KG[PC][PD];              // k^ / Gamma
    float GQ[PC][PD];              // Gamma . q^
    float KT[PC][PD];              // (gamma_C / Gamma) . k^
    float gam[PD];                 // gamma_C (decay over the whole chunk)
    float A[PC][PC + 1];
    float P[PC][PC + 1];
    float Mx[PC][PC + 1];
    float beta[PC], rq[PC], rk[PC];
};

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Raw input (4 bf16 channels at channel offset ch) at sequence position pos
// of stream m: pos < 0 is a cached tap (tap 3 + pos of conv_in).
__device__ __forceinline__ u32x2 prefill_input(const Ptrs& p, int L, int m, size_t C3, size_t ch, int pos) {
    if (pos < 0) return *reinterpret_cast<const u32x2*>(p.conv_in + (size_t)m * 3 * C3 + (size_t)(3 + pos) * C3 + ch);
    return *reinterpret_cast<const u32x2*>(p.x + ((size_t)m * L + pos) * C3 + ch);
}

__device__ __forceinline__ float load_state_elem(const float* s) { return *s; }
__device__ __forceinline__ float load_state_elem(const uint16_t* s) { return bf16_lo(*s); }
__device__ __forceinline__ void store_state_elem(float* s, float v) { *s = v; }
__device__ __forceinline__ void store_state_elem(uint16_t* s, float v) { *s = (uint16_t)f32_to_bf16_rne(v); }

}  // namespace

// One workgroup per (stream, head); x [M][L][3][H*D], fgate [M][L][H*D],
// blogit [M][L][H], o [M][L][H][D].
template <typename TS>
__global__ __launch_bounds__(PNT)
void prefill_kernel(const Ptrs p, const int L)
{
    __shared__ PrefillSmem sm;
    const int unit = (int)blockIdx.x;
    const int m = unit / p.H, h = unit - m * p.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const size_t HD = (size_t)p.H * PD, C3 = 3 * HD;
    const int ncol = 32 * wv;                          // this wave's value columns

    // ---- the state, in the MFMA output layout ----
    TS* const st = static_cast<TS*>(p.state) + (size_t)unit * PD * PD;
    float S[8][2][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][nt][r] = load_state_elem(st + (size_t)(16 * mt + 4 * g4 + r) * PD + ncol + 16 * nt + l16);

    const float eA = expf(p.A_log[h]);
    const float lb = p.lower_bound;

    for (int t0 = 0; t0 < L; t0 += PC) {
        const int n = min(PC, L - t0);

        // ---- conv + SiLU of the chunk's tokens (q, k, v), 4 channels per item ----
        for (int idx = tid; idx < PC * PNG; idx += PNT) {
            const int j = idx / PNG, g = idx - j * PNG;
            f32x4 zv = {0.0f, 0.0f, 0.0f, 0.0f};
            if (j < n) {
                const int tok = t0 + j;
                const int tensor = g / (PD / 4);
                const size_t ch = (size_t)tensor * HD + (size_t)h * PD + 4 * (g - tensor * (PD / 4));
                const u32x2 xv = prefill_input(p, L, m, C3, ch, tok);
                const u32x2 t2 = prefill_input(p, L, m, C3, ch, tok - 1);
                const u32x2 t1 = prefill_input(p, L, m, C3, ch, tok - 2);
                const u32x2 t0v = prefill_input(p, L, m, C3, ch, tok - 3);
                const u32x4* wp = reinterpret_cast<const u32x4*>(p.conv_w + 4 * ch);
                const u32x4 w01 = wp[0], w23 = wp[1];
                zv = f32x4{conv_silu(u32x2{w01.x, w01.y}, bf16_lo(t0v.x), bf16_lo(t1.x), bf16_lo(t2.x), bf16_lo(xv.x)),
                           conv_silu(u32x2{w01.z, w01.w}, bf16_hi(t0v.x), bf16_hi(t1.x), bf16_hi(t2.x), bf16_hi(xv.x)),
                           conv_silu(u32x2{w23.x, w23.y}, bf16_lo(t0v.y), bf16_lo(t1.y), bf16_lo(t2.y), bf16_lo(xv.y)),
                           conv_silu(u32x2{w23.z, w23.w}, bf16_hi(t0v.y), bf16_hi(t1.y), bf16_hi(t2.y), bf16_hi(xv.y))};
            }
            reinterpret_cast<f32x4*>(sm.z[j])[g] = zv;
        }
        // forget gate in log space, g = lb * sigmoid(exp(A) (f + b)) (0 past the end)
        for (int idx = tid; idx < PC * (PD / 4); idx += PNT) {
            const int j = idx / (PD / 4), q = idx - j * (PD / 4);
            f32x4 gl = {0.0f, 0.0f, 0.0f, 0.0f};
            if (j < n) {
                const u32x2 fv = *reinterpret_cast<const u32x2*>(
                    p.fgate + ((size_t)m * L + t0 + j) * HD + (size_t)h * PD + 4 * q);
                const f32x4 bv = *reinterpret_cast<const f32x4*>(p.dt_bias + (size_t)h * PD + 4 * q);
                gl = f32x4{lb / (1.0f + expf(-eA * (bf16_lo(fv.x) + bv.x))),
                           lb / (1.0f + expf(-eA * (bf16_hi(fv.x) + bv.y))),
                           lb / (1.0f + expf(-eA * (bf16_lo(fv.y) + bv.z))),
                           lb / (1.0f + expf(-eA * (bf16_hi(fv.y) + bv.w)))};
            }
            reinterpret_cast<f32x4*>(sm.G[j])[q] = gl;
        }
        if (tid < PC) {
            sm.beta[tid] = tid < n
                ? 1.0f / (1.0f + expf(-bf16_lo(p.blogit[((size_t)m * L + t0 + tid) * p.H + h])))
                : 0.0f;
        }
        lds_barrier();

        // ---- norms (one wave per token) and cumulative decays (one thread per channel) ----
        for (int j = wv; j < PC; j += PNT / 64) {
            float sqq = 0.0f, skk = 0.0f;
#pragma unroll
            for (int i = lane; i < PD; i += 64) {
                const float qv = sm.z[j][i], kv = sm.z[j][PD + i];
                sqq = fmaf(qv, qv, sqq);
                skk = fmaf(kv, kv, skk);
            }
            sqq = wave_sum(sqq);
            skk = wave_sum(skk);
            if (lane == 0) {
                sm.rq[j] = j < n ? p.scale * rsqrtf(sqq + 1e-6f) : 0.0f;
                sm.rk[j] = j < n ? rsqrtf(skk + 1e-6f) : 0.0f;
            }
        }
        if (tid < PD) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < PC; ++j) {
                acc += sm.G[j][tid];
                sm.G[j][tid] = acc;
            }
            sm.gam[tid] = expf(acc);
        }
        lds_barrier();

        // ---- decay-weighted keys and queries ----
        for (int e = tid; e < PC * PD; e += PNT) {
            const int j = e / PD, c = e - j * PD;
            const float Gj = sm.G[j][c];
            const float kh = sm.z[j][PD + c] * sm.rk[j], qh = sm.z[j][c] * sm.rq[j];
            const float eg = expf(Gj), ig = expf(-Gj);
            sm.GK[j][c] = kh * eg;
            sm.KG[j][c] = kh * ig;
            sm.GQ[j][c] = qh * eg;
            sm.KT[j][c] = kh * expf(sm.G[PC - 1][c] - Gj);
        }
        lds_barrier();

        // ---- A (wave 0) and P (wave 1): 16 x 16 products over the 128 channels ----
        if (wv < 2) {
            const float (*X)[PD] = wv == 0 ? sm.GK : sm.GQ;
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
            for (int kk = 0; kk < PD / 4; ++kk)
                acc = mfma16(X[l16][4 * kk + g4], sm.KG[l16][4 * kk + g4], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r, s = l16;
                if (wv == 0) sm.A[t][s] = s < t ? sm.beta[t] * acc[r] : 0.0f;
                else sm.P[t][s] = s <= t ? acc[r] : 0.0f;
            }
        }
        lds_barrier();

        // ---- M = (I + A)^-1 Diag(beta): forward substitution, one column per lane ----
        if (tid < PC) {
            const int c = tid;
            float x[PC];
#pragma unroll
            for (int i = 0; i < PC; ++i) {
                float v = i == c ? sm.beta[i] : 0.0f;
#pragma unroll
                for (int j = 0; j < i; ++j) v = fmaf(-sm.A[i][j], x[j], v);
                x[i] = v;
                sm.Mx[i][c] = v;
            }
        }
        lds_barrier();

        // ---- W = M (Gamma . K) into LDS (G's storage), U = M V in registers ----
        f32x4 U[2], Wr[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 aw = {0.0f, 0.0f, 0.0f, 0.0f}, au = {0.0f, 0.0f, 0.0f, 0.0f};
            const int col = ncol + 16 * nt + l16;
#pragma unroll
            for (int kk = 0; kk < PC / 4; ++kk) {
                const float a = sm.Mx[l16][4 * kk + g4];
                aw = mfma16(a, sm.GK[4 * kk + g4][col], aw);
                au = mfma16(a, sm.z[4 * kk + g4][2 * PD + col], au);
            }
            Wr[nt] = aw;
            U[nt] = au;
        }
        // W replaces the cumulative decays, which nobody reads any more
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.G[4 * g4 + r][ncol + 16 * nt + l16] = Wr[nt][r];
        lds_barrier();

        // ---- Delta = U - W S and (Gamma . Q) S, this wave's 32 value columns ----
        f32x4 dacc[2] = {U[0], U[1]};
        f32x4 oacc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = 16 * mt + 4 * g4 + r;
                const float aw = -sm.G[l16][k], aq = sm.GQ[l16][k];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    dacc[nt] = mfma16(aw, S[mt][nt][r], dacc[nt]);
                    oacc[nt] = mfma16(aq, S[mt][nt][r], oacc[nt]);
                }
            }
        }
        // Delta replaces the conv q outputs, which nobody reads any more
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.z[4 * g4 + r][ncol + 16 * nt + l16] = dacc[nt][r];
        lds_barrier();

        // ---- O = (Gamma . Q) S + P Delta ----
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int col = ncol + 16 * nt + l16;
#pragma unroll
            for (int kk = 0; kk < PC / 4; ++kk)
                oacc[nt] = mfma16(sm.P[l16][4 * kk + g4], sm.z[4 * kk + g4][col], oacc[nt]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                if (t < n)
                    p.o[(((size_t)m * L + t0 + t) * p.H + h) * PD + col] = (uint16_t)f32_to_bf16_rne(oacc[nt][r]);
            }
        }

        // ---- S' = Diag(gamma_C) S + ((gamma_C / Gamma) . K)^T Delta ----
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gk = sm.gam[16 * mt + 4 * g4 + r];
                S[mt][0][r] *= gk;
                S[mt][1][r] *= gk;
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 acc = {S[mt][nt][0], S[mt][nt][1], S[mt][nt][2], S[mt][nt][3]};
#pragma unroll
                for (int kk = 0; kk < PC / 4; ++kk)
                    acc = mfma16(sm.KT[4 * kk + g4][16 * mt + l16], sm.z[4 * kk + g4][ncol + 16 * nt + l16], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) S[mt][nt][r] = acc[r];
            }
        }
        // the next chunk overwrites every vector above
        lds_barrier();
    }

#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_state_elem(st + (size_t)(16 * mt + 4 * g4 + r) * PD + ncol + 16 * nt + l16, S[mt][nt][r]);
    // conv state after the sequence: positions L-3, L-2, L-1 (a position < 0
    // is a cached tap, read before it is overwritten)
    if (tid < PNG) {
        const int tensor = tid / (PD / 4);
        const size_t ch = (size_t)tensor * HD + (size_t)h * PD + 4 * (tid - tensor * (PD / 4));
        const u32x2 n0 = prefill_input(p, L, m, C3, ch, L - 3);
        const u32x2 n1 = prefill_input(p, L, m, C3, ch, L - 2);
        const u32x2 n2 = prefill_input(p, L, m, C3, ch, L - 1);
        uint16_t* co = p.conv_out + (size_t)m * 3 * C3 + ch;
        *reinterpret_cast<u32x2*>(co) = n0;
        *reinterpret_cast<u32x2*>(co + C3) = n1;
        *reinterpret_cast<u32x2*>(co + 2 * C3) = n2;
    }
}

hipError_t launch_prefill(const StepArgs& a) {
    if (a.D != PD) return hipErrorInvalidValue;
    Ptrs p = make_ptrs(a);
    int L = a.T;
    void* args[] = {(void*)&p, (void*)&L};
    const void* fn = a.state_dtype == 0 ? reinterpret_cast<const void*>(&prefill_kernel<float>)
                                        : reinterpret_cast<const void*>(&prefill_kernel<uint16_t>);
    return hipLaunchKernel(fn, dim3((unsigned)(a.M * a.H)), dim3(PNT), args, 0, (hipStream_t)a.stream);
}

}  // namespace kda
