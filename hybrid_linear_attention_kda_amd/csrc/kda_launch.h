// kda_launch.h -- internal interface between the C ABI (kda_api.cpp) and the
// gfx950 kernels (kda_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

// Arguments of one decode / recurrent launch, already validated by the host.
struct StepArgs {
    int M, H, D;
    int T;                // tokens per stream (multi-token step)
    int state_dtype;      // 0 = f32, 1 = bf16
    int nsplit;           // workgroups per head: 1, 2 or 4 (D == 128 only)
    void* state;
    const void* x;        // bf16 [M][3][H*D]        (fused step)
    const void* conv_w;   // bf16 [3*H*D][4]         (fused step)
    const void* conv_in;  // bf16 [M][3][3*H*D]      (fused step)
    void* conv_out;       // bf16 [M][3][3*H*D]      (fused step)
    const float* qkv;     // f32  [M][3][H*D]        (recurrent step)
    const float* alpha;
    const float* beta;
    float scale;
    void* o;              // bf16 [M][H][D]: o, or y for the layer step
    void* stream;
    // gated step and layer step
    const void* fgate;       // bf16 [M][H*D]
    const float* A_log;      // [H]
    const float* dt_bias;    // [H*D]
    const void* beta_logit;  // bf16 [M][H]
    int gate_kind;
    float lower_bound;
    // layer step
    const void* out_gate;    // bf16 [M][H*D]
    const float* norm_w;     // [D]
    float norm_eps;
};

hipError_t launch_decode_step(const StepArgs& a);
hipError_t launch_recurrent_step(const StepArgs& a);
hipError_t launch_decode_step_gated(const StepArgs& a);
hipError_t launch_layer_step(const StepArgs& a);
hipError_t launch_decode_multi(const StepArgs& a);
hipError_t launch_prefill(const StepArgs& a);
// two-pass prefill over a workspace of ws_bytes (already validated); ncu =
// compute units of the device the stream runs on
hipError_t launch_prefill_ws(const StepArgs& a, void* ws, size_t ws_bytes, int ncu);
// bytes of one (stream, head, chunk) record of the two-pass prefill
size_t prefill_record_bytes();
// f32 copy of the state kept between segments for bf16 storage
size_t prefill_state_stage_bytes(int M, int H);
// size of the allocation-free entry point's per-device scratch array, and
// its device address on device `dev` (looked up on the first call per device)
size_t prefill_scratch_bytes();
hipError_t prefill_scratch_address(int dev, void** out);
hipError_t launch_conv_step(int M, int C, const void* x, const void* w, const void* cin,
                            void* cout, float* y, void* stream);

// Compute units of device `dev` (0 if unknown).
int device_cu_count(int dev);
// Compute units of the device `stream` belongs to (NULL: the current
// device); 0 if unknown.
int stream_cu_count(void* stream);

}  // namespace kda
