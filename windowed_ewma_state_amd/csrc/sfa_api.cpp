// sfa_api.cpp -- the extern "C" entry points declared in include/sfa.h.
//
// Every entry point validates its arguments on the host before enqueuing
// anything, then launches the kernels on the caller's stream.  The library
// allocates nothing and never synchronises.  Its only global state is a
// per-device cache of the decode kernels' resident workgroup counts (atomics,
// written once per device with the value the runtime reports).
#include <atomic>
#include <climits>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/sfa.h"
#include "sfa_internal.h"

// ---- scratch of the no-allocation prefill (sfa_prefill_noalloc) -----------
// One copy of this array per device, loaded with the library's code object
// and held until the process ends.  In host code the name only stands in for
// the symbol: every host use goes through the device's own address, looked up
// once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SFA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];

// device address of `scratch` on the device that owns `stream` (looked up with
// that device current, once per device); NULL with *err set on failure
void *scratch_for(hipStream_t stream, hipError_t *err) {
    int dev = 0;
    *err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxScratchDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    int cur = 0;
    *err = hipGetDevice(&cur);
    if (*err != hipSuccess) return nullptr;
    if (cur != dev && (*err = hipSetDevice(dev)) != hipSuccess) return nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t restore = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (*err != hipSuccess) return nullptr;
    if ((*err = restore) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool dtype_ok(int t) { return t == SFA_F32 || t == SFA_BF16; }
float scale_log2e(float scale, int d) {
    const float s = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
    return s * 1.4426950408889634f;
}
int hip_status(hipError_t e) { return e == hipSuccess ? SFA_OK : SFA_ERR_HIP; }

}  // namespace

extern "C" {

const char *sfa_status_string(int status) {
    switch (status) {
        case SFA_OK: return "SFA_OK";
        case SFA_ERR_INVALID_ARG: return "SFA_ERR_INVALID_ARG: invalid argument";
        case SFA_ERR_UNSUPPORTED: return "SFA_ERR_UNSUPPORTED: unsupported head_dim, hidden size or dtype";
        case SFA_ERR_HIP: return "SFA_ERR_HIP: kernel launch failed";
        case SFA_ERR_TOO_LARGE:
            return "SFA_ERR_TOO_LARGE: the call needs more scratch than the no-allocation entry point's "
                   "static buffer holds";
        default: return "SFA: unknown status";
    }
}

int sfa_abi_version(void) { return 2; }

size_t sfa_prefill_workspace_size(int B, int n, int Hkv, int d) {
    if (B <= 0 || n <= 0 || Hkv <= 0 || d <= 0) return 0;
    return sfa::prefill_workspace_bytes(B, n, Hkv, d);
}

namespace {

constexpr int kNothingToDo = -1;

// argument checks of every prefill entry point except those of the workspace:
// SFA_OK, an error code, or kNothingToDo for zero-sized work
int prefill_check(int parts, int mode, const void *q, const void *k, const void *v,
                  const float *gamma, const float *alpha, void *out, void *ring_k, void *ring_v,
                  float *state, const int32_t *pos0, int B, int n, int Hq, int Hkv, int d, int window,
                  int in_dtype, int out_dtype) {
    if (parts != SFA_PREFILL_SINGLE_PASS && (parts < 1 || parts > (SFA_PREFILL_SCAN | SFA_PREFILL_ATTEND)))
        return SFA_ERR_INVALID_ARG;
    if (B < 0 || n < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return SFA_ERR_INVALID_ARG;
    if (window < 1 || window > SFA_MAX_WINDOW) return SFA_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return SFA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return SFA_ERR_UNSUPPORTED;
    if ((ring_k == nullptr) != (ring_v == nullptr)) return SFA_ERR_INVALID_ARG;
    if (pos0 && (ring_k == nullptr || state == nullptr)) return SFA_ERR_INVALID_ARG;
    if (n > INT_MAX - sfa::kTile) return SFA_ERR_INVALID_ARG;  // token indices of the last tile are 32-bit
    {   // scan waves and attention workgroups are numbered with 32-bit integers
        const long long chains = (long long)B * (mode == sfa::kQueryHead ? Hq : Hkv);
        if (chains * ((n + sfa::kTile - 1) / sfa::kTile) * 4 >= (1LL << 31)) return SFA_ERR_INVALID_ARG;
    }
    if (parts == SFA_PREFILL_SINGLE_PASS &&
        (mode != sfa::kKvHead || in_dtype != SFA_BF16 || (n + sfa::kTile - 1) / sfa::kTile > sfa::kFusedMaxTiles))
        return SFA_ERR_UNSUPPORTED;
    if (B == 0 || n == 0) return kNothingToDo;
    if (!q || !k || !v || !gamma || !alpha || !out) return SFA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        (ring_k && (!aligned(ring_k, 16) || !aligned(ring_v, 16))) || (state && !aligned(state, 16)))
        return SFA_ERR_INVALID_ARG;
    return SFA_OK;
}

// workspace bytes of a prefill call in this mode (sizes already checked)
size_t prefill_need(int mode, int B, int n, int Hq, int Hkv, int d) {
    const int chains = mode == sfa::kQueryHead ? Hq : mode == sfa::kRunningMean ? 3 * Hkv : Hkv;
    return sfa::prefill_workspace_bytes(B, n, chains, d);
}

// one prefill call; mode: sfa::kKvHead, kQueryHead (γ and S per query head,
// Hs = Hq) or kRunningMean (state [B,Hkv,2,d], three times the workspace)
int prefill_impl(int parts, int mode, const void *q, const void *k, const void *v,
                 const float *gamma, const float *alpha, void *out, void *ring_k, void *ring_v,
                 float *state, const int32_t *pos0, int B, int n, int Hq, int Hkv, int d, int window,
                 float scale, int in_dtype, int out_dtype, void *workspace, size_t workspace_bytes,
                 void *stream) {
    const int chk = prefill_check(parts, mode, q, k, v, gamma, alpha, out, ring_k, ring_v, state, pos0, B,
                                  n, Hq, Hkv, d, window, in_dtype, out_dtype);
    if (chk == kNothingToDo) return SFA_OK;
    if (chk != SFA_OK) return chk;
    if (!workspace || !aligned(workspace, 16)) return SFA_ERR_INVALID_ARG;
    if (workspace_bytes < prefill_need(mode, B, n, Hq, Hkv, d)) return SFA_ERR_INVALID_ARG;
    const int s_per_query = mode == sfa::kQueryHead, running_mean = mode == sfa::kRunningMean;
    const int Hs = s_per_query ? Hq : Hkv;

    sfa::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.gamma = gamma; a.alpha = alpha;
    a.out = out; a.ring_k = ring_k; a.ring_v = ring_v; a.state = state; a.pos0 = pos0;
    a.B = B; a.n = n; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.W = window; a.group = Hq / Hkv;
    a.ntiles = (n + sfa::kTile - 1) / sfa::kTile;
    a.scale_log2e = scale_log2e(scale, d);
    a.in_bf16 = in_dtype == SFA_BF16;
    a.out_bf16 = out_dtype == SFA_BF16;
    a.Hs = Hs;
    a.s_per_query = s_per_query;
    a.running_mean = running_mean;
    const size_t per = (size_t)B * Hs * a.ntiles * d;
    float *ws = static_cast<float *>(workspace);
    a.agg16 = ws;
    a.agg64 = ws + 4 * per;
    a.carry = ws + 5 * per;
    a.csum16 = a.csum64 = a.ccarry = a.beta64 = nullptr;
    // the single pass (when it applies) uses the same memory for its
    // published aggregates [B*Hkv][ntiles][d] (8 bytes each) and the carried S
    a.tagged = reinterpret_cast<uint64_t *>(ws);
    a.sinit = ws + 2 * per;
    if (running_mean) {
        a.csum16 = ws + 6 * per;
        a.csum64 = ws + 10 * per;
        a.ccarry = ws + 11 * per;
        a.beta64 = ws + 12 * per;  // B*Hkv*ntiles floats
    }
    return hip_status(sfa::launch_prefill(a, static_cast<hipStream_t>(stream), parts));
}

int decode_impl(int mode, const void *q, const void *k_new, const void *v_new, void *ring_k,
                void *ring_v, float *state, const int32_t *pos, const float *gamma, const float *alpha,
                void *out, int L, int B, int Hq, int Hkv, int d, int window, float scale, int in_dtype,
                int out_dtype, void *stream) {
    if (L < 0 || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return SFA_ERR_INVALID_ARG;
    if (window < 1 || window > SFA_MAX_WINDOW) return SFA_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return SFA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return SFA_ERR_UNSUPPORTED;
    if (L == 0 || B == 0) return SFA_OK;
    if ((long long)L * B * Hkv >= (1LL << 31) / 64) return SFA_ERR_INVALID_ARG;  // unit indices are 32-bit
    if ((long long)L * B * Hq >= (1LL << 31) / 128) return SFA_ERR_INVALID_ARG;  // state/query element offsets
    if (!q || !k_new || !v_new || !ring_k || !ring_v || !state || !pos || !gamma || !alpha || !out)
        return SFA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(ring_k, 16) ||
        !aligned(ring_v, 16) || !aligned(state, 16) || !aligned(out, 16))
        return SFA_ERR_INVALID_ARG;

    sfa::DecodeArgs a;
    a.q = q; a.k_new = k_new; a.v_new = v_new;
    a.ring_k = ring_k; a.ring_v = ring_v; a.state = state;
    a.pos = pos; a.gamma = gamma; a.alpha = alpha; a.out = out;
    a.L = L; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.W = window; a.group = Hq / Hkv;
    a.scale_log2e = scale_log2e(scale, d);
    a.in_bf16 = in_dtype == SFA_BF16;
    a.out_bf16 = out_dtype == SFA_BF16;
    a.s_per_query = mode == sfa::kQueryHead;
    a.running_mean = mode == sfa::kRunningMean;
    return hip_status(sfa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

int sfa_prefill(const void *q, const void *k, const void *v, const float *gamma, const float *alpha,
                void *out, void *ring_k, void *ring_v, float *state, const int32_t *pos0, int B,
                int n, int Hq, int Hkv, int d, int window, float scale, int in_dtype, int out_dtype,
                void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(SFA_PREFILL_SCAN | SFA_PREFILL_ATTEND, sfa::kKvHead, q, k, v, gamma, alpha, out,
                        ring_k, ring_v, state, pos0, B, n, Hq, Hkv, d, window, scale, in_dtype,
                        out_dtype, workspace, workspace_bytes, stream);
}

int sfa_prefill_part(int parts, const void *q, const void *k, const void *v, const float *gamma,
                     const float *alpha, void *out, void *ring_k, void *ring_v, float *state,
                     const int32_t *pos0, int B, int n, int Hq, int Hkv, int d, int window,
                     float scale, int in_dtype, int out_dtype, void *workspace,
                     size_t workspace_bytes, void *stream) {
    return prefill_impl(parts, sfa::kKvHead, q, k, v, gamma, alpha, out, ring_k, ring_v, state, pos0, B,
                        n, Hq, Hkv, d, window, scale, in_dtype, out_dtype, workspace, workspace_bytes,
                        stream);
}

int sfa_prefill_qh(const void *q, const void *k, const void *v, const float *gamma, const float *alpha,
                   void *out, void *ring_k, void *ring_v, float *state, const int32_t *pos0, int B,
                   int n, int Hq, int Hkv, int d, int window, float scale, int in_dtype,
                   int out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(SFA_PREFILL_SCAN | SFA_PREFILL_ATTEND, sfa::kQueryHead, q, k, v, gamma, alpha,
                        out, ring_k, ring_v, state, pos0, B, n, Hq, Hkv, d, window, scale, in_dtype,
                        out_dtype, workspace, workspace_bytes, stream);
}

int sfa_prefill_rm(const void *q, const void *k, const void *v, const float *gamma, const float *alpha,
                   void *out, void *ring_k, void *ring_v, float *state, const int32_t *pos0, int B,
                   int n, int Hq, int Hkv, int d, int window, float scale, int in_dtype,
                   int out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(SFA_PREFILL_SCAN | SFA_PREFILL_ATTEND, sfa::kRunningMean, q, k, v, gamma, alpha,
                        out, ring_k, ring_v, state, pos0, B, n, Hq, Hkv, d, window, scale, in_dtype,
                        out_dtype, workspace, workspace_bytes, stream);
}

int sfa_prefill_noalloc(const void *q, const void *k, const void *v, const float *gamma,
                        const float *alpha, void *out, void *ring_k, void *ring_v, float *state,
                        const int32_t *pos0, int B, int n, int Hq, int Hkv, int d, int window,
                        float scale, int in_dtype, int out_dtype, void *stream) {
    const int parts = SFA_PREFILL_SCAN | SFA_PREFILL_ATTEND;
    const int chk = prefill_check(parts, sfa::kKvHead, q, k, v, gamma, alpha, out, ring_k, ring_v, state,
                                  pos0, B, n, Hq, Hkv, d, window, in_dtype, out_dtype);
    if (chk == kNothingToDo) return SFA_OK;
    if (chk != SFA_OK) return chk;
    if (prefill_need(sfa::kKvHead, B, n, Hq, Hkv, d) > SFA_NOALLOC_SCRATCH_BYTES) return SFA_ERR_TOO_LARGE;
    hipError_t err = hipSuccess;
    void *ws = scratch_for(static_cast<hipStream_t>(stream), &err);
    if (!ws) return SFA_ERR_HIP;
    return prefill_impl(parts, sfa::kKvHead, q, k, v, gamma, alpha, out, ring_k, ring_v, state, pos0, B, n,
                        Hq, Hkv, d, window, scale, in_dtype, out_dtype, ws, SFA_NOALLOC_SCRATCH_BYTES,
                        stream);
}

int sfa_decode_step(const void *q, const void *k_new, const void *v_new, void *ring_k, void *ring_v,
                    float *state, const int32_t *pos, const float *gamma, const float *alpha,
                    void *out, int L, int B, int Hq, int Hkv, int d, int window, float scale,
                    int in_dtype, int out_dtype, void *stream) {
    return decode_impl(sfa::kKvHead, q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha, out, L,
                       B, Hq, Hkv, d, window, scale, in_dtype, out_dtype, stream);
}

int sfa_decode_step_qh(const void *q, const void *k_new, const void *v_new, void *ring_k,
                       void *ring_v, float *state, const int32_t *pos, const float *gamma,
                       const float *alpha, void *out, int L, int B, int Hq, int Hkv, int d,
                       int window, float scale, int in_dtype, int out_dtype, void *stream) {
    return decode_impl(sfa::kQueryHead, q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha, out,
                       L, B, Hq, Hkv, d, window, scale, in_dtype, out_dtype, stream);
}

int sfa_decode_step_rm(const void *q, const void *k_new, const void *v_new, void *ring_k,
                       void *ring_v, float *state, const int32_t *pos, const float *gamma,
                       const float *alpha, void *out, int L, int B, int Hq, int Hkv, int d,
                       int window, float scale, int in_dtype, int out_dtype, void *stream) {
    return decode_impl(sfa::kRunningMean, q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha,
                       out, L, B, Hq, Hkv, d, window, scale, in_dtype, out_dtype, stream);
}

int sfa_decode_step_enhance(const void *q, const void *k_new, const void *v_new, void *ring_k, void *ring_v,
                            float *state, const int32_t *pos, const float *gamma, const float *alpha,
                            void *out, float *e_ring, float *field, const void *prepared, int shared_pool,
                            float *enhancement, int L, int B, int Hq, int Hkv, int d, int window, float scale,
                            int layer0, int n_layers, float alpha_base, float cross_decay, float ema_gamma,
                            float temperature, float clip, int ring_size, int n_slots, int in_dtype,
                            int out_dtype, void *stream) {
    if (L < 0 || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return SFA_ERR_INVALID_ARG;
    if (window < 1 || window > SFA_MAX_WINDOW) return SFA_ERR_INVALID_ARG;
    if (ring_size < 1 || ring_size > SFA_MAX_WINDOW || n_slots < 1 || n_slots > 64) return SFA_ERR_INVALID_ARG;
    if (!(temperature > 0.f) || !(clip >= 0.f) || layer0 < 0 || n_layers < 1 || n_layers < layer0 + L)
        return SFA_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return SFA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return SFA_ERR_UNSUPPORTED;
    // the fused form: bf16 inputs, up to 16 query heads per KV head, a hidden
    // row of at most 4096 (held in LDS)
    if (in_dtype != SFA_BF16 || Hq / Hkv > 16 || (long long)Hq * d > 4096) return SFA_ERR_UNSUPPORTED;
    if (L == 0 || B == 0) return SFA_OK;
    if ((long long)L * B * Hkv >= (1LL << 31) / 64) return SFA_ERR_INVALID_ARG;
    if ((long long)L * B * Hq >= (1LL << 31) / 128) return SFA_ERR_INVALID_ARG;
    if ((long long)L * B * ring_size * Hq * d >= (1LL << 31)) return SFA_ERR_INVALID_ARG;  // ring offsets
    if (!q || !k_new || !v_new || !ring_k || !ring_v || !state || !pos || !gamma || !alpha || !out || !e_ring ||
        !field || !prepared)
        return SFA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(ring_k, 16) ||
        !aligned(ring_v, 16) || !aligned(state, 16) || !aligned(out, 16) || !aligned(e_ring, 16) ||
        !aligned(field, 16) || !aligned(prepared, 256) || (enhancement && !aligned(enhancement, 16)))
        return SFA_ERR_INVALID_ARG;
    sfa::DecodeEnhanceArgs a{};
    sfa::DecodeArgs &da = a.d;
    da.q = q; da.k_new = k_new; da.v_new = v_new;
    da.ring_k = ring_k; da.ring_v = ring_v; da.state = state;
    da.pos = pos; da.gamma = gamma; da.alpha = alpha; da.out = out;
    da.L = L; da.B = B; da.Hq = Hq; da.Hkv = Hkv; da.d = d; da.W = window; da.group = Hq / Hkv;
    da.scale_log2e = scale_log2e(scale, d);
    da.in_bf16 = 1;
    da.out_bf16 = out_dtype == SFA_BF16;
    da.s_per_query = 0;
    da.running_mean = 0;
    a.out = out; a.ring = e_ring; a.field = field; a.enhancement = enhancement;
    a.pool_rec = static_cast<const unsigned char *>(prepared);
    a.pool_rec_bytes = shared_pool ? 0 : sfa::pool_rec_bytes(Hq * d);
    a.H = Hq * d; a.R = ring_size; a.n_slots = n_slots; a.layer0 = layer0; a.n_layers = n_layers;
    a.alpha_base = alpha_base; a.cross_decay = cross_decay; a.ema_gamma = ema_gamma;
    a.inv_temp_log2e = 1.4426950408889634f / temperature;
    a.clip = clip;
    return hip_status(sfa::launch_decode_enhance(a, static_cast<hipStream_t>(stream)));
}

size_t sfa_enhance_workspace_size(int L, int T, int H) {
    if (L <= 0 || T <= 0 || H <= 0) return 0;
    return sfa::enhance_workspace_bytes(L, T, H, L);
}

size_t sfa_enhance_pool_bytes(int n_pool_layers, int H) {
    if (n_pool_layers <= 0 || H <= 0) return 0;
    return (size_t)n_pool_layers * (size_t)sfa::pool_rec_bytes(H);
}

namespace {

// checks shared by the enhancement entry points (pool and workspace aside):
// SFA_OK, an error code, or kNothingToDo for zero-sized work
int enhance_check(const void *attn, void *out, float *ring, float *field, float *enhancement, int L,
                  int layer0, int n_layers, int T, int H, int t0, float temperature, float clip,
                  int ring_size, int n_slots, int in_dtype, int out_dtype) {
    if (L < 0 || T < 0 || H <= 0 || layer0 < 0 || t0 < 0 || n_layers < layer0 + L || n_layers < 1)
        return SFA_ERR_INVALID_ARG;
    if (ring_size < 1 || ring_size > SFA_MAX_WINDOW || n_slots < 1 || n_slots > 64)
        return SFA_ERR_INVALID_ARG;
    if (!(temperature > 0.f) || !(clip >= 0.f)) return SFA_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return SFA_ERR_UNSUPPORTED;
    if (H % 64 != 0) return SFA_ERR_UNSUPPORTED;
    // token indices of the last tile and the workgroup numbers are 32-bit
    if (T > INT_MAX - sfa::kTile) return SFA_ERR_INVALID_ARG;
    if ((long long)L * ((T + sfa::kTile - 1) / sfa::kTile) * ((H + 127) / 128) >= (1LL << 31))
        return SFA_ERR_INVALID_ARG;
    if (L == 0 || T == 0) return kNothingToDo;
    if (!attn || !out || !ring || !field) return SFA_ERR_INVALID_ARG;
    if (!aligned(attn, 16) || !aligned(out, 16) || !aligned(ring, 16) || !aligned(field, 16) ||
        (enhancement && !aligned(enhancement, 16)))
        return SFA_ERR_INVALID_ARG;
    return SFA_OK;
}

sfa::EnhanceArgs enhance_args(const void *attn, void *out, float *ring, float *field, float *enhancement,
                              int L, int layer0, int n_layers, int T, int H, int t0, float alpha_base,
                              float cross_decay, float ema_gamma, float temperature, float clip,
                              int ring_size, int n_slots, int in_dtype, int out_dtype) {
    sfa::EnhanceArgs a{};
    a.attn = attn; a.out = out; a.ring = ring; a.field = field; a.enhancement = enhancement;
    a.L = L; a.layer0 = layer0; a.n_layers = n_layers; a.T = T; a.H = H; a.t0 = t0;
    a.R = ring_size; a.n_slots = n_slots;
    a.ntiles = (T + sfa::kTile - 1) / sfa::kTile;
    a.alpha_base = alpha_base; a.cross_decay = cross_decay; a.ema_gamma = ema_gamma;
    a.inv_temp_log2e = 1.4426950408889634f / temperature;
    a.clip = clip;
    a.in_bf16 = in_dtype == SFA_BF16;
    a.out_bf16 = out_dtype == SFA_BF16;
    return a;
}

// the workspace after the pool records: field aggregates and carries, the
// carried ring, the slot weights, the operand table and α per layer
void carve_enhance_workspace(sfa::EnhanceArgs &a, unsigned char *rest) {
    const size_t per = (size_t)a.L * a.ntiles * a.H;
    float *ws = reinterpret_cast<float *>(rest);
    a.agg64 = ws;
    a.carry = ws + per;
    a.halo = ws + 2 * per;
    a.wsem = reinterpret_cast<uint16_t *>(ws + 2 * per + (size_t)a.L * SFA_MAX_WINDOW * a.H);
    a.coef = a.wsem + (size_t)a.L * a.ntiles * 4 * 4 * 512;
    a.alpha_tab = reinterpret_cast<float *>(a.coef + (size_t)8 * 2 * 64 * 8);
}

}  // namespace

int sfa_enhance(const void *attn, void *out, float *ring, float *field, const float *pool,
                long long pool_layer_stride, float *enhancement, int L, int layer0, int n_layers,
                int T, int H, int t0, float alpha_base, float cross_decay, float ema_gamma,
                float temperature, float clip, int ring_size, int n_slots, int in_dtype,
                int out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (pool_layer_stride < 0) return SFA_ERR_INVALID_ARG;
    const int chk = enhance_check(attn, out, ring, field, enhancement, L, layer0, n_layers, T, H, t0,
                                  temperature, clip, ring_size, n_slots, in_dtype, out_dtype);
    if (chk == kNothingToDo) return SFA_OK;
    if (chk != SFA_OK) return chk;
    if (!pool || !workspace) return SFA_ERR_INVALID_ARG;
    if (pool_layer_stride != 0 && pool_layer_stride < (long long)n_slots * H) return SFA_ERR_INVALID_ARG;
    if (!aligned(pool, 16) || !aligned(workspace, 16) || (pool_layer_stride % 4) != 0)
        return SFA_ERR_INVALID_ARG;
    const int n_pool_layers = pool_layer_stride == 0 ? 1 : L;
    if (workspace_bytes < sfa::enhance_workspace_bytes(L, T, H, n_pool_layers)) return SFA_ERR_INVALID_ARG;

    sfa::EnhanceArgs a = enhance_args(attn, out, ring, field, enhancement, L, layer0, n_layers, T, H, t0,
                                      alpha_base, cross_decay, ema_gamma, temperature, clip, ring_size,
                                      n_slots, in_dtype, out_dtype);
    a.pool = pool; a.pool_stride = pool_layer_stride; a.n_pool_layers = n_pool_layers;
    a.pool_rec = static_cast<unsigned char *>(workspace);
    a.pool_rec_bytes = sfa::pool_rec_bytes(H);
    a.prepare_pool = 1;
    carve_enhance_workspace(a, a.pool_rec + (size_t)n_pool_layers * a.pool_rec_bytes);
    return hip_status(sfa::launch_enhance(a, static_cast<hipStream_t>(stream)));
}

int sfa_enhance_prepare_pool(const float *pool, long long pool_layer_stride, int n_pool_layers,
                             int n_slots, int H, void *prepared, size_t prepared_bytes, void *stream) {
    if (n_pool_layers < 0 || n_slots < 1 || n_slots > 64 || H <= 0 || pool_layer_stride < 0)
        return SFA_ERR_INVALID_ARG;
    if (H % 64 != 0) return SFA_ERR_UNSUPPORTED;
    if ((long long)n_pool_layers * (H / 32 + 64) >= (1LL << 31)) return SFA_ERR_INVALID_ARG;
    if (n_pool_layers == 0) return SFA_OK;
    if (!pool || !prepared) return SFA_ERR_INVALID_ARG;
    if (n_pool_layers > 1 && pool_layer_stride < (long long)n_slots * H) return SFA_ERR_INVALID_ARG;
    if (!aligned(pool, 16) || !aligned(prepared, 256) || (pool_layer_stride % 4) != 0)
        return SFA_ERR_INVALID_ARG;
    if (prepared_bytes < sfa_enhance_pool_bytes(n_pool_layers, H)) return SFA_ERR_INVALID_ARG;
    sfa::EnhanceArgs a{};
    a.pool = pool; a.pool_stride = pool_layer_stride; a.n_pool_layers = n_pool_layers;
    a.n_slots = n_slots; a.H = H;
    a.pool_rec = static_cast<unsigned char *>(prepared);
    a.pool_rec_bytes = sfa::pool_rec_bytes(H);
    return hip_status(sfa::launch_pool_prepare(a, static_cast<hipStream_t>(stream)));
}

int sfa_enhance_prepared(const void *attn, void *out, float *ring, float *field, const void *prepared,
                         int shared_pool, float *enhancement, int L, int layer0, int n_layers, int T,
                         int H, int t0, float alpha_base, float cross_decay, float ema_gamma,
                         float temperature, float clip, int ring_size, int n_slots, int in_dtype,
                         int out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    const int chk = enhance_check(attn, out, ring, field, enhancement, L, layer0, n_layers, T, H, t0,
                                  temperature, clip, ring_size, n_slots, in_dtype, out_dtype);
    if (chk == kNothingToDo) return SFA_OK;
    if (chk != SFA_OK) return chk;
    if (!prepared || !workspace || !aligned(prepared, 256) || !aligned(workspace, 16))
        return SFA_ERR_INVALID_ARG;
    if (workspace_bytes < sfa::enhance_workspace_bytes(L, T, H, 0)) return SFA_ERR_INVALID_ARG;
    sfa::EnhanceArgs a = enhance_args(attn, out, ring, field, enhancement, L, layer0, n_layers, T, H, t0,
                                      alpha_base, cross_decay, ema_gamma, temperature, clip, ring_size,
                                      n_slots, in_dtype, out_dtype);
    a.pool = nullptr; a.pool_stride = 0;
    a.n_pool_layers = shared_pool ? 1 : L;
    a.pool_rec = static_cast<unsigned char *>(const_cast<void *>(prepared));
    a.pool_rec_bytes = sfa::pool_rec_bytes(H);
    a.prepare_pool = 0;
    carve_enhance_workspace(a, static_cast<unsigned char *>(workspace));
    return hip_status(sfa::launch_enhance(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
