// kda_device.h -- device helpers shared by the gfx950 kernels of the KDA
// library (decode step and chunked prefill).  Internal, not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_launch.h"

namespace kda {

// Kernel arguments of every decode / prefill launch (pointers already
// validated by the host).
struct Ptrs {
    int H;
    void* state;
    const uint16_t* x;
    const uint16_t* conv_w;
    const uint16_t* conv_in;
    uint16_t* conv_out;
    const float* qkv;
    const float* alpha;
    const float* beta;
    float scale;
    uint16_t* o;
    // gated prologue (MODE >= 1): raw gate inputs instead of alpha / beta
    const uint16_t* fgate;     // bf16 [M][H*D] forget-gate projection
    const float* A_log;        // [H]
    const float* dt_bias;      // [H*D]
    const uint16_t* blogit;    // bf16 [M][H] write-strength logits
    int gate_kind;             // 0: bounded sigmoid, 1: softplus
    float lower_bound;         // gate_kind 0 only
    // gated RMSNorm epilogue (MODE == 2): o is replaced by y
    const uint16_t* ogate;     // bf16 [M][H*D] output-gate projection
    const float* norm_w;       // [D]
    float norm_eps;
};

inline Ptrs make_ptrs(const StepArgs& a) {
    Ptrs p;
    p.H = a.H;
    p.state = a.state;
    p.x = static_cast<const uint16_t*>(a.x);
    p.conv_w = static_cast<const uint16_t*>(a.conv_w);
    p.conv_in = static_cast<const uint16_t*>(a.conv_in);
    p.conv_out = static_cast<uint16_t*>(a.conv_out);
    p.qkv = a.qkv;
    p.alpha = a.alpha;
    p.beta = a.beta;
    p.scale = a.scale;
    p.o = static_cast<uint16_t*>(a.o);
    p.fgate = static_cast<const uint16_t*>(a.fgate);
    p.A_log = a.A_log;
    p.dt_bias = a.dt_bias;
    p.blogit = static_cast<const uint16_t*>(a.beta_logit);
    p.gate_kind = a.gate_kind;
    p.lower_bound = a.lower_bound;
    p.ogate = static_cast<const uint16_t*>(a.out_gate);
    p.norm_w = a.norm_w;
    p.norm_eps = a.norm_eps;
    return p;
}


typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// Two f32 -> packed bf16, lo in the low half: gfx950's v_cvt_pk_bf16_f32,
// round to nearest even (the default rounding mode), subnormals kept, a NaN
// stays a NaN of the same sign.  One VALU instruction per pair; a software
// rounding of the bit pattern costs about six per value, and its NaN test
// compiles to a branch per value.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
}

// f32 -> bf16 (low 16 bits), as above.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// Workgroup barrier that orders LDS only: global loads issued before it stay
// in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// x + (x of lane l ^ OFF).  OFF = 16 and 32 use gfx950's row and half-wave
// swaps on the VALU (v_permlane16_swap / v_permlane32_swap: swapping x with
// itself leaves the values of the two partner lanes in the two results);
// other offsets go through the LDS crossbar.  IEEE addition commutes, so
// each lane gets the bits of x[l] + x[l ^ OFF] either way.
template <int OFF>
__device__ __forceinline__ float xor_add(float x) {
    if constexpr (OFF == 32) {
        const unsigned b = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (OFF == 16) {
        const unsigned b = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        return x + __shfl_xor(x, OFF, 64);
    }
}

// Sum over the lanes that differ from this one in lane-index bits
// log2(FROM) and up (FROM a power of two), lowest bit first.
template <int FROM>
__device__ __forceinline__ float xor_reduce_from(float x) {
    if constexpr (FROM >= 64) {
        return x;
    } else {
        return xor_reduce_from<2 * FROM>(xor_add<FROM>(x));
    }
}

// A DPP lane move within rows of 16 lanes (gfx9 control codes).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]: lane l reads l ^ 1
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]: lane l reads l ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane l reads 7 - l within its 8
constexpr int kDppMirror = 0x140;      // lane l reads 15 - l within its 16
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the wave, the same in every lane, on the VALU: steps 1 and 2 swap
// within quads; once the quads hold their sums, mirroring within 8 and then
// within 16 lanes pairs each lane with the other quad (half) of its group,
// exactly the partner that l ^ 4 (l ^ 8) names, so every step adds the same
// two operands, in the same order, as the butterfly over l ^ 1 .. l ^ 32.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<kDppQuadXor1>(x);
    x += dpp_mov<kDppQuadXor2>(x);
    x += dpp_mov<kDppHalfMirror>(x);
    x += dpp_mov<kDppMirror>(x);
    return xor_add<32>(xor_add<16>(x));
}

// Stores with agent scope (sc1) as well as the non-temporal hint.  On MI355X
// an in-place 16-byte stream over 128 MiB runs at 6.56 TB/s with them
// against 6.41 TB/s with non-temporal stores alone (non-temporal loads
// either way), but a launch of a single round of workgroups per CU takes
// longer to drain its last such stores, so the launch code chooses per grid
// size.  hipcc exposes cache-policy bits beyond the non-temporal one only on
// buffer accesses, hence a raw buffer store over a wave-uniform base; being
// compiler-visible, it also gets the wait states that a store of more than
// 8 bytes needs before its data registers may be rewritten.
constexpr int kCpolSc1Nt = 16 | 2;                   // cache-policy operand: sc1 = 16, nt = 2
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base, int bytes) {
    // base is the same in every lane of the wave; reading it from the first
    // lane lets the compiler keep the descriptor in scalar registers (else it
    // may wrap each store in a loop over distinct descriptors)
    const uint64_t a = reinterpret_cast<uintptr_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    // raw (stride 0) descriptor over [base, base + bytes), 32-bit data format
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(hi << 32 | lo), 0, bytes, 0x00020000);
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
    // at byte offset off of a stream_rsrc buffer, agent scope + non-temporal
    static __device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t rs, int off, const float* f) {
        const u32x4 r = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
        __builtin_amdgcn_raw_buffer_store_b128(r, rs, off, 0, kCpolSc1Nt);
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
    static __device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t rs, int off, const float* f) {
        const u32x4 r = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                         pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
        __builtin_amdgcn_raw_buffer_store_b128(r, rs, off, 0, kCpolSc1Nt);
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
    static __device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t rs, int off, const float* f) {
        const u32x2 r = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
        __builtin_amdgcn_raw_buffer_store_b64(r, rs, off, 0, kCpolSc1Nt);
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

}  // namespace kda
