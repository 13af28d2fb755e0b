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
//    LDS never holds it (LDS per workgroup stays ~3 KiB: occupancy is set by
//    VGPRs only).
//  * Loads and stores of the state are 16 bytes per lane; a wave covers whole
//    contiguous rows (512 B f32 / 256 B bf16), so every access is coalesced.
//  * All state loads are issued before the conv prologue is computed; the
//    barriers in between only fence LDS, so the loads stay in flight.
//  * Reductions over key rows: in-lane FMAs, then a butterfly across the lanes
//    that share columns, then (NWAVES > 1) one exchange through LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_launch.h"

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// f32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x0040u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Workgroup barrier that orders LDS only: global loads issued before it stay
// in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// One lane's share of a state row: VEC consecutive elements, 16 (or 8) bytes.
template <typename TS, int VEC> struct Chunk;

template <> struct Chunk<float, 4> {
    typedef f32x4 raw_t;
    static __device__ __forceinline__ raw_t load(const float* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    }
    static __device__ __forceinline__ void unpack(const raw_t& r, float* f) {
        f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
    }
    static __device__ __forceinline__ void store(float* p, const float* f) {
        f32x4 r = {f[0], f[1], f[2], f[3]};
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(p));
    }
};

template <> struct Chunk<uint16_t, 8> {
    typedef u32x4 raw_t;
    static __device__ __forceinline__ raw_t load(const uint16_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    static __device__ __forceinline__ void unpack(const raw_t& r, float* f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float* f) {
        u32x4 r = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                   pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
        __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));
    }
};

template <> struct Chunk<uint16_t, 4> {
    typedef u32x2 raw_t;
    static __device__ __forceinline__ raw_t load(const uint16_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    }
    static __device__ __forceinline__ void unpack(const raw_t& r, float* f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float* f) {
        u32x2 r = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
        __builtin_nontemporal_store(r, reinterpret_cast<u32x2*>(p));
    }
};

// Short causal conv (kernel 4) + SiLU for one channel, "GLM-5.3 deep dive"
// 8.2.4 step 2.  w4 packs the channel's 4 bf16 taps (tap 3 = current token).
__device__ __forceinline__ float conv_silu(u32x2 w4, float t0, float t1, float t2, float xc) {
    float y = bf16_lo(w4.x) * t0;
    y = fmaf(bf16_hi(w4.x), t1, y);
    y = fmaf(bf16_lo(w4.y), t2, y);
    y = fmaf(bf16_hi(w4.y), xc, y);
    return y / (1.0f + expf(-y));
}

// ------------------------------------------------------------ decode step --
//
// TS      state storage: float or uint16_t (bf16 bits)
// D       head width (dk = dv)
// NSPLIT  workgroups per head (each owns D/NSPLIT value columns)
// NWAVES  waves per workgroup
// VEC     state elements per lane access
// FUSED   true: conv prologue from bf16 x + conv state; false: f32 q|k|v input
template <typename TS, int D, int NSPLIT, int NWAVES, int VEC, bool FUSED>
__global__ __launch_bounds__(NWAVES * 64)
void decode_kernel(const int H, TS* __restrict__ state,
                   const uint16_t* __restrict__ x, const uint16_t* __restrict__ conv_w,
                   const uint16_t* conv_in, uint16_t* conv_out,
                   const float* __restrict__ qkv,
                   const float* __restrict__ alpha, const float* __restrict__ beta,
                   const float scale, uint16_t* __restrict__ o)
{
    constexpr int NT = NWAVES * 64;
    constexpr int COLS = D / NSPLIT;          // value columns of this workgroup
    constexpr int CG = COLS / VEC;            // lanes across one row segment
    static_assert(COLS % VEC == 0 && 64 % CG == 0, "row segment must tile the wave");
    constexpr int RPW = 64 / CG;              // rows per wave access
    constexpr int RS = RPW * NWAVES;          // row slices per workgroup
    static_assert(D % RS == 0, "row slices must tile the key axis");
    constexpr int RPL = D / RS;               // rows per lane
    constexpr int NCH = 2 * D + COLS;         // prologue channels: q, k, own v
    constexpr int PIT = (NCH + NT - 1) / NT;  // prologue iterations per thread
    typedef Chunk<TS, VEC> IO;

    // conv outputs: q at [0, D), k at [D, 2D), this workgroup's v columns at
    // [2D, 2D + COLS); the tail is scratch for threads past the last channel
    __shared__ float s_z[PIT * NT];
    float* const s_q = s_z;
    float* const s_k = s_z + D;
    float* const s_v = s_z + 2 * D;
    __shared__ float s_a[D];
    __shared__ float s_red[NWAVES > 1 ? NWAVES : 1][2][COLS];
    __shared__ float s_d[COLS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int split = (int)(blockIdx.x % NSPLIT);
    const int unit = (int)(blockIdx.x / NSPLIT);        // m * H + h
    const int m = unit / H;
    const int h = unit - m * H;
    const size_t HD = (size_t)H * D;
    const size_t C3 = 3 * HD;

    const int cg = lane % CG;
    const int rw = lane / CG;
    const int rs = wv * RPW + rw;
    const int col0 = split * COLS + cg * VEC;
    TS* st = state + (size_t)unit * D * D;

    // ---- 1. prologue loads (small; issued first so they retire first) ----
    // Loads are unconditional (a thread past the last channel re-reads the
    // last one and discards it) so they issue as straight-line code.
    u32x2 pw[PIT];
    uint32_t bx[PIT], b0[PIT], b1[PIT], b2[PIT];   // raw bf16 bits (FUSED)
    float px[PIT];                                  // f32 input (!FUSED)
    size_t pch[PIT];
#pragma unroll
    for (int it = 0; it < PIT; ++it) {
        const int c = min(tid + it * NT, NCH - 1);
        const int tensor = c < D ? 0 : (c < 2 * D ? 1 : 2);
        const int within = tensor < 2 ? c - tensor * D : split * COLS + (c - 2 * D);
        pch[it] = (size_t)tensor * HD + (size_t)h * D + within;   // channel in [0, 3HD)
        if constexpr (FUSED) {
            bx[it] = x[(size_t)m * C3 + pch[it]];
            const uint16_t* ci = conv_in + (size_t)m * 3 * C3 + pch[it];
            b0[it] = ci[0];
            b1[it] = ci[C3];
            b2[it] = ci[2 * C3];
            pw[it] = *reinterpret_cast<const u32x2*>(conv_w + 4 * pch[it]);
        } else {
            px[it] = qkv[(size_t)m * C3 + pch[it]];
        }
    }
    const float a_pre = alpha[(size_t)unit * D + min(tid, D - 1)];
    const float b = beta[unit];
    // keep the scheduler from sinking these loads below the state loads:
    // the conv prologue then waits only for them, not for the state
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. issue every state load of this lane ----
    typename IO::raw_t raw[RPL];
#pragma unroll
    for (int t = 0; t < RPL; ++t) raw[t] = IO::load(st + (size_t)(rs + RS * t) * D + col0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. conv + SiLU into LDS; advance the conv state ----
    // (computed unconditionally so the compiler keeps the loads above)
#pragma unroll
    for (int it = 0; it < PIT; ++it) {
        const int c = tid + it * NT;
        float z;
        if constexpr (FUSED) {
            z = conv_silu(pw[it], bf16_lo(b0[it]), bf16_lo(b1[it]), bf16_lo(b2[it]),
                          bf16_lo(bx[it]));
        } else {
            z = px[it];
        }
        s_z[c] = z;
        if constexpr (FUSED) {
            // q/k taps are shared by the NSPLIT workgroups of a head: only
            // split 0 writes them (the host keeps NSPLIT = 1 when in place).
            if (c < NCH && (c >= 2 * D || split == 0)) {
                uint16_t* co = conv_out + (size_t)m * 3 * C3 + pch[it];
                co[0] = (uint16_t)b1[it];
                co[C3] = (uint16_t)b2[it];
                co[2 * C3] = (uint16_t)bx[it];
            }
        }
    }
    if (tid < D) s_a[tid] = a_pre;
    lds_barrier();

    // ---- 4. L2 norms and k^.q^ (every wave reduces the same D values) ----
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
    const float rq = scale * rsqrtf(sqq + 1e-6f);
    const float rk = rsqrtf(skk + 1e-6f);
    const float kq = sqk * rq * rk;                    // k^ . q^

    // ---- 5. fade, and the two reductions over this lane's rows ----
    float sreg[RPL][VEC];
    float u[VEC], wq[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) { u[e] = 0.0f; wq[e] = 0.0f; }
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
        const int i = rs + RS * t;
        const float a = s_a[i], kk = s_k[i] * rk, qq = s_q[i] * rq;
        IO::unpack(raw[t], sreg[t]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float sv = sreg[t][e] * a;
            sreg[t][e] = sv;
            u[e] = fmaf(sv, kk, u[e]);
            wq[e] = fmaf(sv, qq, wq[e]);
        }
    }
    // lanes that share columns differ in the bits above log2(CG)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            u[e] += __shfl_xor(u[e], off, 64);
            wq[e] += __shfl_xor(wq[e], off, 64);
        }
    }

    // ---- 6. delta correction and readout ----
    float d[VEC];
    if constexpr (NWAVES > 1) {
        if (rw == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                s_red[wv][0][cg * VEC + e] = u[e];
                s_red[wv][1][cg * VEC + e] = wq[e];
            }
        }
        lds_barrier();
        if (tid < COLS) {
            float U = 0.0f, W = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) { U += s_red[w][0][tid]; W += s_red[w][1][tid]; }
            const float dj = b * (s_v[tid] - U);
            s_d[tid] = dj;
            o[(size_t)unit * D + split * COLS + tid] = (uint16_t)f32_to_bf16_rne(fmaf(dj, kq, W));
        }
        lds_barrier();
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = s_d[cg * VEC + e];
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = b * (s_v[cg * VEC + e] - u[e]);
        if (rw == 0) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                o[(size_t)unit * D + split * COLS + cg * VEC + e] =
                    (uint16_t)f32_to_bf16_rne(fmaf(d[e], kq, wq[e]));
        }
    }

    // ---- 7. rank-1 write and store ----
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
        const int i = rs + RS * t;
        const float kk = s_k[i] * rk;
#pragma unroll
        for (int e = 0; e < VEC; ++e) sreg[t][e] = fmaf(kk, d[e], sreg[t][e]);
        IO::store(st + (size_t)i * D + col0, sreg[t]);
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

template <typename TS, int D, int NSPLIT, int NWAVES, int VEC, bool FUSED>
static hipError_t launch_decode(const StepArgs& a) {
    void* args[] = {(void*)&a.H, (void*)&a.state, (void*)&a.x, (void*)&a.conv_w,
                    (void*)&a.conv_in, (void*)&a.conv_out, (void*)&a.qkv,
                    (void*)&a.alpha, (void*)&a.beta, (void*)&a.scale, (void*)&a.o};
    const dim3 grid((unsigned)((long)a.M * a.H * NSPLIT));
    const dim3 block(NWAVES * 64);
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_kernel<TS, D, NSPLIT, NWAVES, VEC, FUSED>),
                           grid, block, args, 0, (hipStream_t)a.stream);
}

template <typename TS, int D, int VEC, int NWAVES, bool FUSED>
static hipError_t dispatch_split(const StepArgs& a) {
    if constexpr (D == 128) {
        switch (a.nsplit) {
        case 1: return launch_decode<TS, D, 1, NWAVES, VEC, FUSED>(a);
        case 2: return launch_decode<TS, D, 2, NWAVES, VEC, FUSED>(a);
        case 4: return launch_decode<TS, D, 4, NWAVES, VEC, FUSED>(a);
        default: return hipErrorInvalidValue;
        }
    } else {
        if (a.nsplit != 1) return hipErrorInvalidValue;
        return launch_decode<TS, D, 1, NWAVES, VEC, FUSED>(a);
    }
}

template <bool FUSED>
static hipError_t dispatch(const StepArgs& a) {
    const bool f32 = a.state_dtype == 0;
    switch (a.D) {
    case 16:
        return f32 ? dispatch_split<float, 16, 4, 1, FUSED>(a) : dispatch_split<uint16_t, 16, 4, 1, FUSED>(a);
    case 32:
        return f32 ? dispatch_split<float, 32, 4, 1, FUSED>(a) : dispatch_split<uint16_t, 32, 8, 1, FUSED>(a);
    case 64:
        return f32 ? dispatch_split<float, 64, 4, 2, FUSED>(a) : dispatch_split<uint16_t, 64, 8, 2, FUSED>(a);
    case 128:
        return f32 ? dispatch_split<float, 128, 4, 4, FUSED>(a) : dispatch_split<uint16_t, 128, 8, 4, FUSED>(a);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_step(const StepArgs& a) { return dispatch<true>(a); }
hipError_t launch_recurrent_step(const StepArgs& a) { return dispatch<false>(a); }

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

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    if (dev < 64) cached[dev] = n;
    return n;
}

}  // namespace kda
