// decode.hip -- batched SFA decode step for gfx950.
//
// Page "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩",
// section 2.1 (near field over the last k tokens, far-field EWMA of the keys
// that leave the window, O = O_near + α·S) applied to one new token, with the
// constant-memory k-slot ring of section 2.2 (k = 16).
//
// One wave64 owns one (layer, sequence, KV head) unit and serves all query
// heads of its GQA group.  Every load of the unit (ring K/V rows, the group's
// queries, S, the new key/value) is issued before the first use, so each wave
// keeps ~13 KB in flight; 4 units share a 256-thread workgroup and one launch
// covers all layers.
//   scores   MFMA v_mfma_f32_16x16x32_bf16 (fp32 inputs: 16x16x4 f32):
//            A = ring K rows (row = slot, the new key substituted into slot
//            pos mod W), B = queries (column = head of the group);
//            lane l then holds slots 4*(l/16)+i of head l%16.
//   softmax  over slots: 4 values per lane + two cross-group shuffles.
//   PV       VALU fp32, lane l owns head-dim elements [l*d/64, (l+1)*d/64),
//            probabilities broadcast through LDS.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "decode_unit.h"
#include "sfa_common.h"
#include "sfa_internal.h"

namespace sfa {

namespace {

constexpr int kMaxDevices = 64;

constexpr int kUnitsPerBlock = 4;

template <int D>
__device__ __forceinline__ f32x4 score_tile(const __bf16 *krow, bool krow_ok, const __bf16 *qrow,
                                            bool qrow_ok, int q4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
        bf16x8 a = {}, b = {};
        if (krow_ok) a = *reinterpret_cast<const bf16x8 *>(krow + 32 * st + 8 * q4);
        if (qrow_ok) b = *reinterpret_cast<const bf16x8 *>(qrow + 32 * st + 8 * q4);
        acc = mfma_bf16_16x16x32(a, b, acc);
    }
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 score_tile(const float *krow, bool krow_ok, const float *qrow,
                                            bool qrow_ok, int q4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (krow_ok) a = *reinterpret_cast<const float4 *>(krow + 16 * u + 4 * q4);
        if (qrow_ok) b = *reinterpret_cast<const float4 *>(qrow + 16 * u + 4 * q4);
        acc = mfma_f32_16x16x4(a.x, b.x, acc);
        acc = mfma_f32_16x16x4(a.y, b.y, acc);
        acc = mfma_f32_16x16x4(a.z, b.z, acc);
        acc = mfma_f32_16x16x4(a.w, b.w, acc);
    }
    return acc;
}

// EPL = head-dim elements per lane (d / 64)
template <typename T, int EPL> struct Vec;
template <typename T> struct Vec<T, 1> {
    __device__ __forceinline__ static void load(const T *p, float *x) { x[0] = Elem<T>::load(p); }
    __device__ __forceinline__ static void store(T *p, const float *x) { Elem<T>::store(p, x[0]); }
    __device__ __forceinline__ static void copy(T *dst, const T *src) { *dst = *src; }
};
template <typename T> struct Vec<T, 2> {
    __device__ __forceinline__ static void load(const T *p, float *x) { load2(p, x[0], x[1]); }
    __device__ __forceinline__ static void store(T *p, const float *x) { store2(p, x[0], x[1]); }
    __device__ __forceinline__ static void copy(T *dst, const T *src) {
        if constexpr (sizeof(T) == 2)
            *reinterpret_cast<uint32_t *>(dst) = *reinterpret_cast<const uint32_t *>(src);
        else
            *reinterpret_cast<float2 *>(dst) = *reinterpret_cast<const float2 *>(src);
    }
};

// MODE (far-field variant): kKvHead, kQueryHead (γ and S per query head:
// state [L,B,Hq,d], gamma [L,Hq]) or kRunningMean (state [L,B,Hkv,2,d]: S and
// the mean M of the keys that have left the window, which is the EWMA input)
template <typename TIn, typename TOut, int D, int MODE>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
    constexpr bool QH = MODE == kQueryHead, RM = MODE == kRunningMean;
    constexpr int EPL = D / kWave;
    __shared__ float4 P_lds[kUnitsPerBlock][16][4];  // [unit][head in tile][slots/4]

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int c16 = lane & 15;
    const long unit = (long)blockIdx.x * kUnitsPerBlock + wave;
    const long n_units = (long)a.L * a.B * a.Hkv;
    if (unit >= n_units) return;  // wave-uniform

    const int G = (int)(unit % a.Hkv);
    const long lb = unit / a.Hkv;  // l * B + b
    const int b = (int)(lb % a.B);
    const int l = (int)(lb / a.B);
    const int W = a.W;
    const int group = a.group;
    const int p = a.pos[b];
    if (p < 0) return;  // invalid position: the unit is left untouched
    const int s = p % W;
    const int nvalid = (p >= W - 1) ? W : p + 1;

    TIn *ringK = reinterpret_cast<TIn *>(a.ring_k) + unit * W * D;
    TIn *ringV = reinterpret_cast<TIn *>(a.ring_v) + unit * W * D;
    const TIn *kn = reinterpret_cast<const TIn *>(a.k_new) + unit * D;
    const TIn *vn = reinterpret_cast<const TIn *>(a.v_new) + unit * D;
    const TIn *qg = reinterpret_cast<const TIn *>(a.q) + (lb * a.Hq + (long)G * group) * D;
    float *S_ptr = a.state + unit * (RM ? 2 * D : D);
    const int e0 = lane * EPL;

    // ---- issue the unit's loads -------------------------------------------
    float S[EPL], M[EPL], kev[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) S[e] = M[e] = kev[e] = 0.f;
    if constexpr (!QH) Vec<float, EPL>::load(S_ptr + e0, S);
    if constexpr (RM) Vec<float, EPL>::load(S_ptr + D + e0, M);
    const bool evict = p >= W;
    if (evict) Vec<TIn, EPL>::load(ringK + (long)s * D + e0, kev);

    float vrow[kMaxWindow][EPL];
#pragma unroll
    for (int j = 0; j < kMaxWindow; ++j) {
        if (j < nvalid) {
            const TIn *src = (j == s) ? vn : ringV + (long)j * D;
            Vec<TIn, EPL>::load(src + e0, vrow[j]);
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) vrow[j][e] = 0.f;
        }
    }

    // ---- far field: the key of position p-W leaves the window -------------
    if (!QH && evict) {
        const float gm = a.gamma[(long)l * a.Hkv + G];
        if constexpr (RM) {  // the key joins the mean of the p-W keys that left before it
            const float mf = (float)(p - W + 1);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                M[e] += (kev[e] - M[e]) / mf;
                S[e] = gm * S[e] + (1.f - gm) * M[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) S[e] = gm * S[e] + (1.f - gm) * kev[e];
        }
    }

    // ---- near field, 16 heads of the group per MFMA tile --------------------
    const bool krow_ok = c16 < W;
    const TIn *krow = (c16 == s) ? kn : ringK + (long)c16 * D;
    const float *alpha = a.alpha + (long)l * a.Hq + (long)G * group;
    TOut *outg = reinterpret_cast<TOut *>(a.out) + (lb * a.Hq + (long)G * group) * D;

    for (int ht = 0; ht < group; ht += 16) {
        const int head = ht + c16;
        const bool qrow_ok = head < group;
        const f32x4 sc = score_tile<D>(krow, krow_ok, qg + (long)head * D, qrow_ok, q4);

        float x[4], m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (4 * q4 + i < nvalid) ? sc[i] * a.scale_log2e : -INFINITY;
            m = fmaxf(m, x[i]);
        }
        m = max_over_groups(m);
        float ex[4], sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ex[i] = (4 * q4 + i < nvalid) ? exp2f(x[i] - m) : 0.f;
            sum += ex[i];
        }
        sum = sum_over_groups(sum);
        const float inv = 1.f / sum;
        if (qrow_ok) P_lds[wave][c16][q4] = make_float4(ex[0] * inv, ex[1] * inv, ex[2] * inv, ex[3] * inv);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        const int nh = min(16, group - ht);
        for (int hh = 0; hh < nh; ++hh) {
            const float4 P4[4] = {P_lds[wave][hh][0], P_lds[wave][hh][1], P_lds[wave][hh][2],
                                  P_lds[wave][hh][3]};
            const float *P = reinterpret_cast<const float *>(P4);
            float o[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxWindow; ++j)
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = fmaf(P[j], vrow[j][e], o[e]);
            const float al = alpha[ht + hh];
            float Sh[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) Sh[e] = S[e];
            if constexpr (QH) {  // this query head's own S, evicted key folded in
                const long hs = lb * a.Hq + (long)G * group + ht + hh;
                Vec<float, EPL>::load(a.state + hs * D + e0, Sh);
                if (evict) {
                    const float gh = a.gamma[(long)l * a.Hq + (long)G * group + ht + hh];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) Sh[e] = gh * Sh[e] + (1.f - gh) * kev[e];
                }
                Vec<float, EPL>::store(a.state + hs * D + e0, Sh);
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = fmaf(al, Sh[e], o[e]);
            Vec<TOut, EPL>::store(outg + (long)(ht + hh) * D + e0, o);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- cache update (after every read of the unit's ring) -----------------
    if constexpr (!QH) Vec<float, EPL>::store(S_ptr + e0, S);
    if constexpr (RM) Vec<float, EPL>::store(S_ptr + D + e0, M);
    Vec<TIn, EPL>::copy(ringK + (long)s * D + e0, kn + e0);
    Vec<TIn, EPL>::copy(ringV + (long)s * D + e0, vn + e0);
}

// ---------------------------------------------------------------------------
// k_decode_mfma: bf16 inputs, up to 16 query heads per KV head.
//
// Each wave walks units (layer, sequence, KV head) with a stride of the grid's
// wave count and prefetches the next unit's loads into the second of two
// register buffers while it computes the current one.  Slots past the valid
// ones have masked scores and zeroed V rows; heads past the group repeat the
// last head and their outputs are never stored.  Per unit:
//   scores  one v_mfma_f32_16x16x32_bf16 tile per 32 head-dim elements:
//           A = K rows from the wave's LDS tile (row = slot, the new key in
//           slot pos mod W), B = queries (column = head) from the same tile;
//           lane holds P[head l%16][slots 4(l/16)+i]
//           after the softmax, which is exactly the B operand of
//   PV      v_mfma_f32_16x16x16_bf16 with A = V^T rows (from a per-wave LDS
//           tile) and B = P split into bf16 hi + lo.  V^T row m of tile dt is
//           head-dim element 32(dt/2) + 8(m/4) + 4(dt%2) + m%4, so each lane
//           ends with 8 consecutive outputs of its head (16-byte stores).
//   S       evicted key (read from the K tile before the new key replaces
//           it) folded in (e-pair layout: lane owns d = 2l, 2l+1), broadcast
//           to the epilogue through LDS.
// ---------------------------------------------------------------------------
template <typename TOut, int D, int QN, int MODE>
__global__ __launch_bounds__(256, 2) void k_decode_mfma(DecodeArgs a) {
    constexpr bool QH = MODE == kQueryHead;
    constexpr int VTS = kMaxWindow + 4;  // V^T row stride (bf16): 16 slots + pad
    __shared__ __attribute__((aligned(16))) __bf16 Vt[4][D * VTS];
    __shared__ __attribute__((aligned(16))) float Sl[4][D];
    __shared__ __attribute__((aligned(16))) __bf16 KQ[4][kMaxWindow * (D + 8)];  // K, then Q rows

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int n_units = a.L * a.B * a.Hkv;
    const int stride = gridDim.x * 4;
    int unit = blockIdx.x * 4 + wave;
    __bf16 *vt = Vt[wave];
    float *sl = Sl[wave];
    __bf16 *kqt = KQ[wave];

    // Two register buffers in turn: the next unit's loads are in flight while
    // the current one computes.  The count of outstanding memory operations
    // drains in issue order and the compiler waits on it by position, so every
    // path issues the same loads and stores: the last prefetch is issued too
    // (all lanes at one chunk), the per-query-head S rows of a unit go out
    // before the next unit's prefetch, no store is skipped, and the first step
    // is peeled so that the loop is entered with the same history as its back
    // edge (the previous step's stores after the prefetch).
    if (unit >= n_units) return;
    UnitLoads<D, QN> A, Bf;
    LateLoads<D, QH> late;
    unit_load<D, QN, MODE>(a, unit, A, lane, true);
    int next = unit + stride;
    bool more = next < n_units;
    late_load<D, QH>(a, unit, late, lane);
    unit_load<D, QN, MODE>(a, more ? next : unit, Bf, lane, more);
    unit_compute<TOut, D, QN, MODE>(a, unit, A, late, lane, vt, sl, kqt);
    while (more) {
        unit = next;
        next = unit + stride;
        more = next < n_units;
        late_load<D, QH>(a, unit, late, lane);
        unit_load<D, QN, MODE>(a, more ? next : unit, A, lane, more);
        unit_compute<TOut, D, QN, MODE>(a, unit, Bf, late, lane, vt, sl, kqt);
        if (!more) break;
        unit = next;
        next = unit + stride;
        more = next < n_units;
        late_load<D, QH>(a, unit, late, lane);
        unit_load<D, QN, MODE>(a, more ? next : unit, Bf, lane, more);
        unit_compute<TOut, D, QN, MODE>(a, unit, A, late, lane, vt, sl, kqt);
    }
}

// Grid of one wave per (unit, unit + stride, ...) chain: no more blocks than the
// device holds at once (one round of waves, no partly filled tail round) and no
// more waves than units.  A launch smaller than the resident capacity (one
// layer, say) runs one unit per wave: more units in flight beat the prefetch
// overlap that several units per wave would give.
template <typename K>
hipError_t launch_persistent(K kernel, const DecodeArgs &a, long units, hipStream_t stream) {
    static std::atomic<int> resident[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int cap = resident[dev].load(std::memory_order_relaxed);
    if (cap == 0) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0);
        if (e != hipSuccess) return e;
        cap = std::max(1, cus * std::max(1, per_cu));
        resident[dev].store(cap, std::memory_order_relaxed);
    }
    const long blocks = std::max<long>(1, std::min<long>(cap, (units + 3) / 4));
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut, int MODE>
hipError_t launch_q(const DecodeArgs &a, hipStream_t stream) {
    const long units = (long)a.L * a.B * a.Hkv;
    if constexpr (std::is_same<TIn, __bf16>::value) {
        if (a.group <= 16) {
            // query rows per load instruction: 4 (d 128) or 8 (d 64)
            const bool half = a.group <= 8;
            if (a.d == 128)
                return half ? launch_persistent(k_decode_mfma<TOut, 128, 2, MODE>, a, units, stream)
                            : launch_persistent(k_decode_mfma<TOut, 128, 4, MODE>, a, units, stream);
            return half ? launch_persistent(k_decode_mfma<TOut, 64, 1, MODE>, a, units, stream)
                        : launch_persistent(k_decode_mfma<TOut, 64, 2, MODE>, a, units, stream);
        }
    }
    const dim3 grid((unsigned)((units + kUnitsPerBlock - 1) / kUnitsPerBlock));
    if (a.d == 128)
        hipLaunchKernelGGL((k_decode<TIn, TOut, 128, MODE>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((k_decode<TIn, TOut, 64, MODE>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_t(const DecodeArgs &a, hipStream_t stream) {
    if (a.s_per_query) return launch_q<TIn, TOut, kQueryHead>(a, stream);
    if (a.running_mean) return launch_q<TIn, TOut, kRunningMean>(a, stream);
    return launch_q<TIn, TOut, kKvHead>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_t<__bf16, __bf16>(a, stream) : launch_t<__bf16, float>(a, stream);
    return a.out_bf16 ? launch_t<float, __bf16>(a, stream) : launch_t<float, float>(a, stream);
}

}  // namespace sfa
