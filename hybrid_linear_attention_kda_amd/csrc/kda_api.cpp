// kda_api.cpp -- the C ABI declared in include/kda.h.
//
// Host-side argument validation (before any HIP call), launch-shape choice,
// and error mapping.  The library holds no state besides a per-device cache
// of the compute-unit count.

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"
#include "kda_launch.h"

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

inline Range span(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool supported_d(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }

// Size of M * a * b * c elements of `bytes` each; false on overflow or if the
// element count exceeds what the kernels index with 32-bit unit counts.
bool checked_bytes(long M, long a, long b, long c, long bytes, size_t* out) {
    const long long lim = (1LL << 46);
    long long n = (long long)M;
    const long f[3] = {a, b, c};
    for (long v : f) {
        if (v < 0 || (v > 0 && n > lim / v)) return false;
        n *= v;
    }
    if (n > lim / bytes) return false;
    *out = (size_t)(n * bytes);
    return true;
}

int map_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Workgroups per head.  A head is one workgroup (its whole state) unless M*H
// is below the device's compute-unit count, in which case its value columns
// are split so that more CUs take part.  Splitting needs distinct conv
// buffers: the split workgroups of a head all read the head's q/k taps, so
// none may overwrite them in place.  bf16 state splits at most 2-way (a
// 4-way split would leave 64-byte row segments, half a cache line).
// Compute units of the device the caller's stream runs on (256, MI355X's
// count, if the runtime cannot tell).
int stream_cus(void* stream) {
    const int n = kda::stream_cu_count(stream);
    return n > 0 ? n : 256;
}

int choose_split(int M, int H, int D, int sdt, bool conv_in_place, void* stream) {
    if (D != 128 || conv_in_place) return 1;
    const long units = (long)M * H;
    const int cus = stream_cus(stream);
    if (units >= cus) return 1;
    if (sdt == KDA_STATE_BF16 || 2 * units >= cus) return 2;
    return 4;
}

struct StepSizes {
    size_t state, x, w, conv, alpha, beta, o, qkv;
    size_t fgate, A_log, dt_bias, blogit, norm_w;
};

int step_sizes(int M, int H, int D, int sdt, StepSizes* s) {
    const long HD = (long)H * D;
    const long sb = sdt == KDA_STATE_F32 ? 4 : 2;
    if (!checked_bytes(M, H, D, D, sb, &s->state)) return KDA_ERR_ARG;
    if (!checked_bytes(M, 3, HD, 1, 2, &s->x)) return KDA_ERR_ARG;
    if (!checked_bytes(1, 3, HD, 4, 2, &s->w)) return KDA_ERR_ARG;
    if (!checked_bytes(M, 3, 3, HD, 2, &s->conv)) return KDA_ERR_ARG;
    if (!checked_bytes(M, H, D, 1, 4, &s->alpha)) return KDA_ERR_ARG;
    if (!checked_bytes(M, H, 1, 1, 4, &s->beta)) return KDA_ERR_ARG;
    if (!checked_bytes(M, H, D, 1, 2, &s->o)) return KDA_ERR_ARG;
    if (!checked_bytes(M, 3, HD, 1, 4, &s->qkv)) return KDA_ERR_ARG;
    if (!checked_bytes(M, H, D, 1, 2, &s->fgate)) return KDA_ERR_ARG;
    if (!checked_bytes(1, H, 1, 1, 4, &s->A_log)) return KDA_ERR_ARG;
    if (!checked_bytes(1, H, D, 1, 4, &s->dt_bias)) return KDA_ERR_ARG;
    if (!checked_bytes(M, H, 1, 1, 2, &s->blogit)) return KDA_ERR_ARG;
    if (!checked_bytes(1, D, 1, 1, 4, &s->norm_w)) return KDA_ERR_ARG;
    // the kernels index workgroups as M*H*nsplit in 32 bits
    if ((long long)M * H * 4 > 0x7fffffffLL) return KDA_ERR_ARG;
    return KDA_OK;
}

int check_common(int M, int H, int D, int sdt, float scale) {
    if (M < 0) return KDA_ERR_ARG;
    if (H < 1 || !supported_d(D)) return KDA_ERR_SHAPE;
    if (sdt != KDA_STATE_F32 && sdt != KDA_STATE_BF16) return KDA_ERR_DTYPE;
    if (!isfinite(scale)) return KDA_ERR_ARG;
    return KDA_OK;
}

int validate_decode(int M, int H, int D, int sdt, void* state, const void* x, const void* w,
                    const void* cin, void* cout, const float* alpha, const float* beta,
                    float scale, void* o, StepSizes* sz) {
    int rc = check_common(M, H, D, sdt, scale);
    if (rc != KDA_OK) return rc;
    if (M == 0) return KDA_OK;
    if (!state || !x || !w || !cin || !cout || !alpha || !beta || !o) return KDA_ERR_NULL;
    const void* ptrs[] = {state, x, w, cin, cout, alpha, beta, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    rc = step_sizes(M, H, D, sdt, sz);
    if (rc != KDA_OK) return rc;
    const Range rs = span(state, sz->state), ro = span(o, sz->o), rco = span(cout, sz->conv);
    const Range inputs[] = {span(x, sz->x), span(w, sz->w), span(cin, sz->conv),
                            span(alpha, sz->alpha), span(beta, sz->beta)};
    for (const Range& r : inputs)
        if (overlap(rs, r) || overlap(ro, r)) return KDA_ERR_ALIAS;
    if (overlap(rs, ro) || overlap(rs, rco) || overlap(ro, rco)) return KDA_ERR_ALIAS;
    for (int i = 0; i < 5; ++i) {
        if (i == 2 && cout == cin) continue;  // exact in-place conv state is allowed
        if (overlap(rco, inputs[i])) return KDA_ERR_ALIAS;
    }
    return KDA_OK;
}

int run_decode(int M, int H, int D, int sdt, void* state, const void* x, const void* w,
               const void* cin, void* cout, const float* alpha, const float* beta,
               float scale, void* o, void* stream, int nsplit) {
    StepSizes sz;
    int rc = validate_decode(M, H, D, sdt, state, x, w, cin, cout, alpha, beta, scale, o, &sz);
    if (rc != KDA_OK || M == 0) return rc;
    const bool in_place = cout == cin;
    if (nsplit == 0) {
        nsplit = choose_split(M, H, D, sdt, in_place, stream);
    } else {
        if (nsplit != 1 && nsplit != 2 && nsplit != 4) return KDA_ERR_ARG;
        if (nsplit > 1 && (D != 128 || in_place)) return KDA_ERR_ARG;
    }
    kda::StepArgs a{};
    a.M = M; a.H = H; a.D = D; a.state_dtype = sdt; a.nsplit = nsplit;
    a.state = state; a.x = x; a.conv_w = w; a.conv_in = cin; a.conv_out = cout;
    a.qkv = nullptr; a.alpha = alpha; a.beta = beta; a.scale = scale; a.o = o;
    a.stream = stream;
    return map_hip(kda::launch_decode_step(a));
}

// The gated step and the layer step: the inputs of kda_decode_step without
// alpha and beta, plus the raw gate inputs (and, for the layer step, the
// output gate and norm weight).  `out` is o or y.
struct GatedCall {
    int M, H, D, sdt;
    void* state;
    const void *x, *w, *cin;
    void* cout;
    const void* fgate;
    const float *A_log, *dt_bias;
    const void* blogit;
    int gate_kind;
    float lower_bound, scale;
    const void* ogate;      // layer step only (else NULL)
    const float* norm_w;    // layer step only
    float norm_eps;
    void* out;
    void* stream;
};

int run_gated(const GatedCall& c, bool layer) {
    int rc = check_common(c.M, c.H, c.D, c.sdt, c.scale);
    if (rc != KDA_OK) return rc;
    if (c.gate_kind != KDA_GATE_BOUNDED && c.gate_kind != KDA_GATE_SOFTPLUS) return KDA_ERR_ARG;
    if (c.gate_kind == KDA_GATE_BOUNDED && !(isfinite(c.lower_bound) && c.lower_bound < 0.0f))
        return KDA_ERR_ARG;
    if (layer && !(isfinite(c.norm_eps) && c.norm_eps >= 0.0f)) return KDA_ERR_ARG;
    if (c.M == 0) return KDA_OK;
    const void* need[] = {c.state, c.x, c.w, c.cin, c.cout, c.fgate, c.A_log, c.dt_bias, c.blogit, c.out};
    for (const void* p : need)
        if (!p) return KDA_ERR_NULL;
    if (layer && (!c.ogate || !c.norm_w)) return KDA_ERR_NULL;
    for (const void* p : need)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    if (layer && (!aligned16(c.ogate) || !aligned16(c.norm_w))) return KDA_ERR_ALIGN;
    StepSizes sz;
    rc = step_sizes(c.M, c.H, c.D, c.sdt, &sz);
    if (rc != KDA_OK) return rc;
    const Range rs = span(c.state, sz.state), ro = span(c.out, sz.o), rco = span(c.cout, sz.conv);
    Range inputs[9] = {span(c.x, sz.x), span(c.w, sz.w), span(c.cin, sz.conv),
                       span(c.fgate, sz.fgate), span(c.A_log, sz.A_log), span(c.dt_bias, sz.dt_bias),
                       span(c.blogit, sz.blogit), Range{0, 0}, Range{0, 0}};
    int n_in = 7;
    if (layer) {
        inputs[n_in++] = span(c.ogate, sz.fgate);
        inputs[n_in++] = span(c.norm_w, sz.norm_w);
    }
    for (int i = 0; i < n_in; ++i)
        if (overlap(rs, inputs[i]) || overlap(ro, inputs[i])) return KDA_ERR_ALIAS;
    if (overlap(rs, ro) || overlap(rs, rco) || overlap(ro, rco)) return KDA_ERR_ALIAS;
    for (int i = 0; i < n_in; ++i) {
        if (i == 2 && c.cout == c.cin) continue;  // exact in-place conv state is allowed
        if (overlap(rco, inputs[i])) return KDA_ERR_ALIAS;
    }
    kda::StepArgs a{};
    a.M = c.M; a.H = c.H; a.D = c.D; a.state_dtype = c.sdt;
    a.nsplit = layer ? 1 : choose_split(c.M, c.H, c.D, c.sdt, c.cout == c.cin, c.stream);
    a.state = c.state; a.x = c.x; a.conv_w = c.w; a.conv_in = c.cin; a.conv_out = c.cout;
    a.scale = c.scale; a.o = c.out; a.stream = c.stream;
    a.fgate = c.fgate; a.A_log = c.A_log; a.dt_bias = c.dt_bias; a.beta_logit = c.blogit;
    a.gate_kind = c.gate_kind; a.lower_bound = c.lower_bound;
    a.out_gate = c.ogate; a.norm_w = c.norm_w; a.norm_eps = c.norm_eps;
    return map_hip(layer ? kda::launch_layer_step(a) : kda::launch_decode_step_gated(a));
}

}  // namespace

extern "C" {

int kda_decode_step_gated(int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                          const void* conv_w, const void* conv_in, void* conv_out,
                          const void* f_gate, const float* A_log, const float* dt_bias,
                          const void* beta_logit, int gate_kind, float gate_lower_bound,
                          float scale, void* o, void* stream) {
    GatedCall c{M, H, D, state_dtype, state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log,
                dt_bias, beta_logit, gate_kind, gate_lower_bound, scale, nullptr, nullptr, 0.0f,
                o, stream};
    return run_gated(c, false);
}

int kda_decode_layer_step(int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                          const void* conv_w, const void* conv_in, void* conv_out,
                          const void* f_gate, const float* A_log, const float* dt_bias,
                          const void* beta_logit, int gate_kind, float gate_lower_bound,
                          float scale, const void* out_gate, const float* norm_weight,
                          float norm_eps, void* y, void* stream) {
    GatedCall c{M, H, D, state_dtype, state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log,
                dt_bias, beta_logit, gate_kind, gate_lower_bound, scale, out_gate, norm_weight,
                norm_eps, y, stream};
    return run_gated(c, true);
}


int kda_decode_step(int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                    const void* conv_w, const void* conv_in, void* conv_out, const float* alpha,
                    const float* beta, float scale, void* o, void* stream) {
    return run_decode(M, H, D, state_dtype, state, x_qkv, conv_w, conv_in, conv_out, alpha, beta,
                      scale, o, stream, 0);
}

int kda_decode_step_split(int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                          const void* conv_w, const void* conv_in, void* conv_out,
                          const float* alpha, const float* beta, float scale, void* o,
                          void* stream, int nsplit) {
    if (nsplit < 1) return KDA_ERR_ARG;
    return run_decode(M, H, D, state_dtype, state, x_qkv, conv_w, conv_in, conv_out, alpha, beta,
                      scale, o, stream, nsplit);
}

int kda_decode_multi(int T, int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                     const void* conv_w, const void* conv_in, void* conv_out, const float* alpha,
                     const float* beta, float scale, void* o, void* stream) {
    if (T < 0 || T > KDA_MAX_TOKENS) return KDA_ERR_ARG;
    int rc = check_common(M, H, D, state_dtype, scale);
    if (rc != KDA_OK) return rc;
    if (M == 0 || T == 0) return KDA_OK;
    const void* need[] = {state, x_qkv, conv_w, conv_in, conv_out, alpha, beta, o};
    for (const void* p : need)
        if (!p) return KDA_ERR_NULL;
    for (const void* p : need)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    StepSizes sz;
    rc = step_sizes(M, H, D, state_dtype, &sz);
    if (rc != KDA_OK) return rc;
    // per-token tensors span T times their single-token size
    size_t bx, ba, bb, bo;
    const long HD = (long)H * D;
    if (!checked_bytes((long)M * T, 3, HD, 1, 2, &bx) || !checked_bytes((long)M * T, H, D, 1, 4, &ba) ||
        !checked_bytes((long)M * T, H, 1, 1, 4, &bb) || !checked_bytes((long)M * T, H, D, 1, 2, &bo))
        return KDA_ERR_ARG;
    if ((long long)M * T * 3 * HD > 0x7fffffffLL * 4LL) return KDA_ERR_ARG;
    const Range rs = span(state, sz.state), ro = span(o, bo), rco = span(conv_out, sz.conv);
    const Range inputs[] = {span(x_qkv, bx), span(conv_w, sz.w), span(conv_in, sz.conv),
                            span(alpha, ba), span(beta, bb)};
    for (const Range& r : inputs)
        if (overlap(rs, r) || overlap(ro, r)) return KDA_ERR_ALIAS;
    if (overlap(rs, ro) || overlap(rs, rco) || overlap(ro, rco)) return KDA_ERR_ALIAS;
    for (int i = 0; i < 5; ++i) {
        if (i == 2 && conv_out == conv_in) continue;
        if (overlap(rco, inputs[i])) return KDA_ERR_ALIAS;
    }
    kda::StepArgs a{};
    a.M = M; a.H = H; a.D = D; a.T = T; a.state_dtype = state_dtype; a.nsplit = 1;
    a.state = state; a.x = x_qkv; a.conv_w = conv_w; a.conv_in = conv_in; a.conv_out = conv_out;
    a.alpha = alpha; a.beta = beta; a.scale = scale; a.o = o; a.stream = stream;
    return map_hip(kda::launch_decode_multi(a));
}

// Host validation shared by the prefill entry points; fills `a` and the
// input ranges (for the workspace's alias check).
static int check_prefill(int L, int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                         const void* conv_w, const void* conv_in, void* conv_out, const void* f_gate,
                         const float* A_log, const float* dt_bias, const void* beta_logit, float gate_lower_bound,
                         float scale, void* o, void* stream, kda::StepArgs* a, Range (&all)[10]) {
    if (L < 0 || L > KDA_MAX_TOKENS) return KDA_ERR_ARG;
    int rc = check_common(M, H, D, state_dtype, scale);
    if (rc != KDA_OK) return rc;
    if (D != 128) return KDA_ERR_SHAPE;
    if (!(isfinite(gate_lower_bound) && gate_lower_bound >= -5.0f && gate_lower_bound < 0.0f))
        return KDA_ERR_ARG;
    if (M == 0 || L == 0) return -1;        // nothing to do
    const void* need[] = {state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log, dt_bias, beta_logit, o};
    for (const void* p : need)
        if (!p) return KDA_ERR_NULL;
    for (const void* p : need)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    StepSizes sz;
    rc = step_sizes(M, H, D, state_dtype, &sz);
    if (rc != KDA_OK) return rc;
    size_t bx, bf, bb, bo;
    const long HD = (long)H * D;
    if (!checked_bytes((long)M * L, 3, HD, 1, 2, &bx) || !checked_bytes((long)M * L, HD, 1, 1, 2, &bf) ||
        !checked_bytes((long)M * L, H, 1, 1, 2, &bb) || !checked_bytes((long)M * L, HD, 1, 1, 2, &bo))
        return KDA_ERR_ARG;
    const Range rs = span(state, sz.state), ro = span(o, bo), rco = span(conv_out, sz.conv);
    const Range inputs[] = {span(x_qkv, bx), span(conv_w, sz.w), span(conv_in, sz.conv), span(f_gate, bf),
                            span(A_log, sz.A_log), span(dt_bias, sz.dt_bias), span(beta_logit, bb)};
    for (const Range& r : inputs)
        if (overlap(rs, r) || overlap(ro, r)) return KDA_ERR_ALIAS;
    if (overlap(rs, ro) || overlap(rs, rco) || overlap(ro, rco)) return KDA_ERR_ALIAS;
    for (int i = 0; i < 7; ++i) {
        if (i == 2 && conv_out == conv_in) continue;
        if (overlap(rco, inputs[i])) return KDA_ERR_ALIAS;
    }
    for (int i = 0; i < 7; ++i) all[i] = inputs[i];
    all[7] = rs;
    all[8] = ro;
    all[9] = rco;
    *a = kda::StepArgs{};
    a->M = M; a->H = H; a->D = D; a->T = L; a->state_dtype = state_dtype; a->nsplit = 0;
    a->state = state; a->x = x_qkv; a->conv_w = conv_w; a->conv_in = conv_in; a->conv_out = conv_out;
    a->fgate = f_gate; a->A_log = A_log; a->dt_bias = dt_bias; a->beta_logit = beta_logit;
    a->gate_kind = KDA_GATE_BOUNDED; a->lower_bound = gate_lower_bound; a->scale = scale; a->o = o;
    a->stream = stream;
    return KDA_OK;
}

int kda_prefill_gated(int L, int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                      const void* conv_w, const void* conv_in, void* conv_out, const void* f_gate,
                      const float* A_log, const float* dt_bias, const void* beta_logit,
                      float gate_lower_bound, float scale, void* o, void* stream) {
    kda::StepArgs a;
    Range all[10];
    const int rc = check_prefill(L, M, H, D, state_dtype, state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log,
                                 dt_bias, beta_logit, gate_lower_bound, scale, o, stream, &a, all);
    if (rc == -1) return KDA_OK;
    if (rc != KDA_OK) return rc;
    return map_hip(kda::launch_prefill(a));
}

size_t kda_prefill_workspace_bytes(int L, int M, int H, int D) {
    if (L <= 0 || M <= 0 || H <= 0 || D != 128 || L > KDA_MAX_TOKENS) return 0;
    const long long chunks = (L + 15) / 16;
    const long long n = chunks * (long long)M * H;
    if (n > (1LL << 40) / (long long)kda::prefill_record_bytes()) return 0;
    return (size_t)n * kda::prefill_record_bytes();
}

int kda_prefill_gated_ws(int L, int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                         const void* conv_w, const void* conv_in, void* conv_out, const void* f_gate,
                         const float* A_log, const float* dt_bias, const void* beta_logit,
                         float gate_lower_bound, float scale, void* o, void* workspace, size_t workspace_bytes,
                         int passes, void* stream) {
    if (passes < 0 || passes > 2) return KDA_ERR_ARG;
    kda::StepArgs a;
    Range all[10];
    const int rc = check_prefill(L, M, H, D, state_dtype, state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log,
                                 dt_bias, beta_logit, gate_lower_bound, scale, o, stream, &a, all);
    if (rc == -1) return KDA_OK;
    if (rc != KDA_OK) return rc;
    const long units = (long)M * H;
    if (passes != 1) {
        // checked whatever the choice, so that validity does not depend on the device
        if (!workspace) return KDA_ERR_NULL;
        if (!aligned16(workspace)) return KDA_ERR_ALIGN;
        const size_t full = kda_prefill_workspace_bytes(L, M, H, D);
        if (full == 0) return KDA_ERR_ARG;
        size_t need = (size_t)units * kda::prefill_record_bytes();
        if (state_dtype == KDA_STATE_BF16 && workspace_bytes < full) need += kda::prefill_state_stage_bytes(M, H);
        if (workspace_bytes < need) return KDA_ERR_ARG;
        const Range rw = span(workspace, workspace_bytes);
        for (const Range& r : all)
            if (overlap(rw, r)) return KDA_ERR_ALIAS;
    }
    const int ncu = stream_cus(stream);
    // the two-pass form while the heads alone leave most CUs idle; above
    // that, one workgroup per head already fills the device
    const bool two = passes == 2 || (passes == 0 && units * 2 <= ncu);
    if (!two) return map_hip(kda::launch_prefill(a));
    return map_hip(kda::launch_prefill_ws(a, workspace, workspace_bytes, ncu));
}

int kda_prefill_gated_noalloc(int L, int M, int H, int D, int state_dtype, void* state, const void* x_qkv,
                              const void* conv_w, const void* conv_in, void* conv_out, const void* f_gate,
                              const float* A_log, const float* dt_bias, const void* beta_logit,
                              float gate_lower_bound, float scale, void* o, void* stream) {
    kda::StepArgs a;
    Range all[10];
    const int rc = check_prefill(L, M, H, D, state_dtype, state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log,
                                 dt_bias, beta_logit, gate_lower_bound, scale, o, stream, &a, all);
    if (rc == -1) return KDA_OK;
    if (rc != KDA_OK) return rc;
    const long units = (long)M * H;
    const int ncu = stream_cus(stream);
    if (units * 2 > ncu) return map_hip(kda::launch_prefill(a));     // one pass: no scratch
    // two passes through the device's scratch array: it must hold one
    // chunk's records for every (stream, head), and for bf16 state with more
    // than one segment also the f32 stage
    const size_t cap = kda::prefill_scratch_bytes();
    const size_t full = kda_prefill_workspace_bytes(L, M, H, D);
    size_t need = (size_t)units * kda::prefill_record_bytes();
    if (state_dtype == KDA_STATE_BF16 && full > cap) need += kda::prefill_state_stage_bytes(M, H);
    if (full == 0 || need > cap) return KDA_ERR_ARG;
    int dev = 0;
    if (stream) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice((hipStream_t)stream, &d) != hipSuccess) return KDA_ERR_HIP;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return KDA_ERR_HIP;
    }
    void* ws = nullptr;
    if (kda::prefill_scratch_address(dev, &ws) != hipSuccess) return KDA_ERR_HIP;
    return map_hip(kda::launch_prefill_ws(a, ws, cap, ncu));
}

int kda_conv_step(int M, int C, const void* x, const void* conv_w, const void* conv_in,
                  void* conv_out, float* y, void* stream) {
    if (M < 0 || C < 1 || (C % 8) != 0) return KDA_ERR_ARG;
    if (M == 0) return KDA_OK;
    if (!x || !conv_w || !conv_in || !conv_out || !y) return KDA_ERR_NULL;
    const void* ptrs[] = {x, conv_w, conv_in, conv_out, y};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    size_t bx, bw, bc, by;
    if (!checked_bytes(M, C, 1, 1, 2, &bx) || !checked_bytes(1, C, 4, 1, 2, &bw) ||
        !checked_bytes(M, 3, C, 1, 2, &bc) || !checked_bytes(M, C, 1, 1, 4, &by))
        return KDA_ERR_ARG;
    if ((long long)M * (C / 8) > 0x7fffffffLL * 256LL) return KDA_ERR_ARG;
    const Range ry = span(y, by), rco = span(conv_out, bc);
    const Range rx = span(x, bx), rw = span(conv_w, bw), rci = span(conv_in, bc);
    if (overlap(ry, rx) || overlap(ry, rw) || overlap(ry, rci) || overlap(ry, rco))
        return KDA_ERR_ALIAS;
    if (overlap(rco, rx) || overlap(rco, rw)) return KDA_ERR_ALIAS;
    if (conv_out != conv_in && overlap(rco, rci)) return KDA_ERR_ALIAS;
    return map_hip(kda::launch_conv_step(M, C, x, conv_w, conv_in, conv_out, y, stream));
}

int kda_recurrent_step(int M, int H, int D, int state_dtype, void* state, const float* qkv,
                       const float* alpha, const float* beta, float scale, void* o,
                       void* stream) {
    int rc = check_common(M, H, D, state_dtype, scale);
    if (rc != KDA_OK) return rc;
    if (M == 0) return KDA_OK;
    if (!state || !qkv || !alpha || !beta || !o) return KDA_ERR_NULL;
    const void* ptrs[] = {state, qkv, alpha, beta, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    StepSizes sz;
    rc = step_sizes(M, H, D, state_dtype, &sz);
    if (rc != KDA_OK) return rc;
    const Range rs = span(state, sz.state), ro = span(o, sz.o);
    const Range inputs[] = {span(qkv, sz.qkv), span(alpha, sz.alpha), span(beta, sz.beta)};
    for (const Range& r : inputs)
        if (overlap(rs, r) || overlap(ro, r)) return KDA_ERR_ALIAS;
    if (overlap(rs, ro)) return KDA_ERR_ALIAS;
    kda::StepArgs a{};
    a.M = M; a.H = H; a.D = D; a.state_dtype = state_dtype;
    a.nsplit = choose_split(M, H, D, state_dtype, false, stream);
    a.state = state; a.qkv = qkv; a.alpha = alpha; a.beta = beta; a.scale = scale; a.o = o;
    a.stream = stream;
    return map_hip(kda::launch_recurrent_step(a));
}

const char* kda_status_string(int status) {
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "unsupported shape (H < 1 or D not in {16, 32, 64, 128})";
    case KDA_ERR_DTYPE: return "unknown state dtype";
    case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KDA_ERR_ALIAS: return "an output overlaps an input";
    case KDA_ERR_ARG: return "invalid argument (negative size, non-finite scale, bad gate or norm parameter, overflow, workspace too small)";
    case KDA_ERR_HIP: return "the HIP runtime refused the launch";
    default: return "unknown status";
    }
}

int kda_version(void) { return 10200; }

}  // extern "C"
