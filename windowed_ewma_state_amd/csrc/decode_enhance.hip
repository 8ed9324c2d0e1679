// decode_enhance.hip -- the SFA decode step fused with the triple-channel
// enhancement, for gfx950.
//
// Page "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩",
// sections 2.1-2.2: the decode step (near field over the k-slot ring, the
// key leaving the window folded into S, O = O_near + α·S).  Page "Dalin Soma
// SFA基于信号场注意力机制的神经网络推理加速框架", section 2.1 (ring mean of the
// last attention outputs, EMA field, 64-slot semantic pool), section 2.2
// (enhancement = ring_mean + 0.5·field + 0.5·semantic, clipped, scaled by
// α_layer, added to the attention output) and section 2.4 (the ring mean
// divides by the ring size).  The engine of page "Signal Field Attention
// (SFA)" applies the enhancement per layer to each new token's attention
// output; here that output never leaves the chip.
//
// One workgroup per (layer, sequence) owns the sequence's whole attention row
// (every query head, hidden H = Hq·d):
//   (1) its waves run the decode units of the row's KV heads (the same unit
//       routine as the batched decode step, decode_unit.h), writing the
//       outputs into the row in LDS instead of memory;
//   (2) per column x of the row (a thread per column, 512 apart): a_x is the
//       output as the caller's dtype holds it; the ring sum with a_x in slot
//       pos mod R, the field update, and the cosine numerators
//       Σ_x a_x·s_j[x] of all 64 slots, accumulated in registers (the 64
//       slot values of a column are eight 16-byte hi/lo chunk pairs of the
//       prepared pool's semantic operand table);
//   (3) a reduce-scatter over each wave (lane j ends with slot j's sum), the
//       eight waves' sums, the softmax over the slots;
//   (4) per column again: 0.5·Σ_j w_j·s_j[x], e = ring mean + 0.5·field +
//       0.5·semantic, out = a + α_l·clip(e).
// Each thread keeps all of its columns' ring and field loads in flight
// together, and the next column's 16 pool chunks load while the current
// column accumulates.
// The pool is read once per workgroup, so this form suits few sequences
// (one per layer, the engine's shape); a batch of many sequences reads every
// layer's pool once per sequence.
#include "decode_unit.h"
#include "sfa_common.h"
#include "sfa_internal.h"

namespace sfa {

namespace {

constexpr int kDeMaxH = 4096;   // largest hidden row (fp32 in LDS, twice)
constexpr int kDeSlots = 64;

// one reduce-scatter step over lanes l and l ^ HALF: each keeps the half of
// v it owns (upper if its HALF bit is set) summed with the partner's
template <int HALF>
__device__ __forceinline__ void rs_step(float *v, int lane) {
    const bool up = (lane & HALF) != 0;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const float keep = up ? v[i + HALF] : v[i];
        const float give = up ? v[i] : v[i + HALF];
        v[i] = keep + __shfl_xor(give, HALF);
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// The 64 slot values of column x in the prepared pool's semantic operand
// table: 16-column group xg = 2·(x/32) + ((x%32)/4)%2, row r = 4·((x%32)/8) + x%4;
// chunk (sk, q4) holds slots 32sk + 4q4 + e (e < 4) and 32sk + 16 + 4q4 + e - 4,
// as bf16 hi (first) and lo (512 elements on) halves.
struct PoolCol { u32x4 h[8], l[8]; };

__device__ __forceinline__ void pool_col_load(const uint16_t *poolT, int x, PoolCol &pc) {
    const int r32 = x & 31;
    const int xg = 2 * (x >> 5) + ((r32 >> 2) & 1);
    const int row = 4 * (r32 >> 3) + (r32 & 3);
#pragma unroll
    for (int sk = 0; sk < 2; ++sk) {
        const uint16_t *base = poolT + ((long)(xg * 2 + sk) * 2) * 512;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            pc.h[4 * sk + q4] = *reinterpret_cast<const u32x4 *>(base + (16 * q4 + row) * 8);
            pc.l[4 * sk + q4] = *reinterpret_cast<const u32x4 *>(base + 512 + (16 * q4 + row) * 8);
        }
    }
}

// slot value s_j[x] = hi + lo for the 64 slots, fed to f(slot, value)
template <typename F>
__device__ __forceinline__ void pool_col_each(const PoolCol &pc, F f) {
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        const int sk = ch >> 2, q4 = ch & 3;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float hv = (e & 1) ? bf16_hi(pc.h[ch][e >> 1]) : bf16_lo(pc.h[ch][e >> 1]);
            const float lv = (e & 1) ? bf16_hi(pc.l[ch][e >> 1]) : bf16_lo(pc.l[ch][e >> 1]);
            f(32 * sk + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + e - 4), hv + lv);
        }
    }
}

constexpr int kDeThreads = 512;                  // 8 waves: 4 run the decode units
constexpr int kDeWaves = kDeThreads / kWave;
constexpr int kDeCols = kDeMaxH / kDeThreads;    // columns per thread, at most

template <typename TOut, int D, int QN>
__global__ __launch_bounds__(kDeThreads) void k_decode_enhance(DecodeEnhanceArgs a) {
    constexpr int VTS = kMaxWindow + 4;
    __shared__ __attribute__((aligned(16))) __bf16 Vt[4][D * VTS];
    __shared__ __attribute__((aligned(16))) float Sl[4][D];
    __shared__ __attribute__((aligned(16))) __bf16 KQ[4][kMaxWindow * (D + 8)];
    __shared__ __attribute__((aligned(16))) float arow[kDeMaxH];  // the attention row, then a
    __shared__ __attribute__((aligned(16))) float ebuf[kDeMaxH];  // ring mean + 0.5·field
    __shared__ float part[kDeWaves][kDeSlots + 1];  // per-wave cosine numerators and Σa²
    __shared__ __attribute__((aligned(16))) float wsl[kDeSlots];  // 0.5·softmax weights

    const DecodeArgs &da = a.d;
    // layer · B + sequence, XCD-aware: each XCD takes a contiguous run of
    // (layer, sequence) pairs, so the sequences of one layer share that XCD's
    // L2 copy of the layer's pool records
    const int lb = xcd_remap(blockIdx.x, da.L * da.B);
    const int l = lb / da.B, b = lb % da.B;
    const int p = load_uniform(da.pos + b);
    if (p < 0) return;  // a skipped sequence: nothing of it is written
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // ---- (1) the decode units of this row, outputs into LDS (waves 0..3) ---------
    if (wave < 4) {
        for (int G = wave; G < da.Hkv; G += 4) {
            const int unit = lb * da.Hkv + G;
            UnitLoads<D, QN> u;
            LateLoads<D, false> late;
            unit_load<D, QN, kKvHead>(da, unit, u, lane, true);
            unit_compute<TOut, D, QN, kKvHead, true>(da, unit, u, late, lane, Vt[wave], Sl[wave], KQ[wave],
                                                     arow);
        }
    }
    __syncthreads();

    // ---- (2) ring, field: every column's loads in flight together ----------------
    const int H = a.H, R = a.R;
    const int rs = p % a.R;  // the ring slot of this token
    float *ring = a.ring + (long)lb * R * H;
    float *field = a.field + (long)lb * H;
    const unsigned char *rec = a.pool_rec + (long long)l * a.pool_rec_bytes;
    const float *inv_norm = reinterpret_cast<const float *>(rec);
    const uint16_t *poolT = reinterpret_cast<const uint16_t *>(rec + kPoolRecHeader) + (long)H * 128;
    const float g = a.ema_gamma;
    const float invR = 1.f / (float)R;
    const int ncol = (H - tid + kDeThreads - 1) / kDeThreads;  // this thread's columns tid + 512 i
    float av[kDeCols], sum[kDeCols], fl[kDeCols];
#pragma unroll
    for (int i = 0; i < kDeCols; ++i) {
        const int x = tid + kDeThreads * i;
        av[i] = sum[i] = fl[i] = 0.f;
        if (i < ncol) {
            float v = arow[x];
            if constexpr (std::is_same<TOut, __bf16>::value) v = (float)(__bf16)v;  // as the row is stored
            av[i] = v;
            fl[i] = field[x];
        }
    }
    // ring slots four at a time (their loads in flight together), summed in slot order
#pragma unroll
    for (int j0 = 0; j0 < kMaxWindow; j0 += 4) {
        if (j0 < R) {
            float rv[4][kDeCols];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int i = 0; i < kDeCols; ++i) {
                    const int j = j0 + jj;
                    rv[jj][i] = (j < R && j != rs && i < ncol) ? ring[(long)j * H + tid + kDeThreads * i] : 0.f;
                }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int i = 0; i < kDeCols; ++i)
                    if (j0 + jj < R) sum[i] += j0 + jj == rs ? av[i] : rv[jj][i];
        }
    }
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < kDeCols; ++i) {
        if (i < ncol) {
            const int x = tid + kDeThreads * i;
            arow[x] = av[i];
            ring[(long)rs * H + x] = av[i];
            const float F = g * fl[i] + (1.f - g) * av[i];
            field[x] = F;
            ebuf[x] = sum[i] * invR + 0.5f * F;
            sq = fmaf(av[i], av[i], sq);
        }
    }
    // ---- cosine numerators: the next column's pool chunks load while this one accumulates
    float c[kDeSlots];
#pragma unroll
    for (int j = 0; j < kDeSlots; ++j) c[j] = 0.f;
    {
        PoolCol buf[2];
        if (ncol > 0) pool_col_load(poolT, tid, buf[0]);
#pragma unroll
        for (int i = 0; i < kDeCols; ++i) {
            if (i < ncol) {
                if (i + 1 < ncol) pool_col_load(poolT, tid + kDeThreads * (i + 1), buf[(i + 1) & 1]);
                const float ai = av[i];
                pool_col_each(buf[i & 1], [&](int slot, float v) { c[slot] = fmaf(ai, v, c[slot]); });
            }
        }
    }
    // ---- (3) reduce over the workgroup, softmax over the slots ----------------
    rs_step<32>(c, lane);
    rs_step<16>(c, lane);
    rs_step<8>(c, lane);
    rs_step<4>(c, lane);
    rs_step<2>(c, lane);
    rs_step<1>(c, lane);
    sq = wave_sum(sq);
    part[wave][lane] = c[0];  // slot `lane`, summed over this wave
    if (lane == 0) part[wave][kDeSlots] = sq;
    __syncthreads();
    if (wave == 0) {
        float num = 0.f, sqt = 0.f;
#pragma unroll
        for (int w = 0; w < kDeWaves; ++w) {
            num += part[w][lane];
            sqt += part[w][kDeSlots];
        }
        const float inv_na = 1.f / fmaxf(sqrtf(sqt), 1e-12f);
        const bool live = lane < a.n_slots;
        const float z = live ? num * inv_na * inv_norm[lane] * a.inv_temp_log2e : -INFINITY;
        const float m = wave_max(z);
        const float ez = live ? exp2f(z - m) : 0.f;
        wsl[lane] = 0.5f * ez / wave_sum(ez);
    }
    __syncthreads();
    // ---- (4) semantic sum, fusion, clip, output -------------------------------
    float w[kDeSlots];
#pragma unroll
    for (int j = 0; j < kDeSlots; j += 4) {
        const float4 w4 = *reinterpret_cast<const float4 *>(&wsl[j]);
        w[j] = w4.x; w[j + 1] = w4.y; w[j + 2] = w4.z; w[j + 3] = w4.w;
    }
    const float al = alpha_layer(a.alpha_base, a.cross_decay, a.layer0 + l, a.n_layers);
    TOut *out = reinterpret_cast<TOut *>(a.out) + (long)lb * H;
    float *enh = a.enhancement ? a.enhancement + (long)lb * H : nullptr;
    {
        PoolCol buf[2];
        if (ncol > 0) pool_col_load(poolT, tid, buf[0]);
#pragma unroll
        for (int i = 0; i < kDeCols; ++i) {
            if (i < ncol) {
                if (i + 1 < ncol) pool_col_load(poolT, tid + kDeThreads * (i + 1), buf[(i + 1) & 1]);
                float sem = 0.f;
                pool_col_each(buf[i & 1], [&](int slot, float v) { sem = fmaf(w[slot], v, sem); });
                const int x = tid + kDeThreads * i;
                const float e = __builtin_amdgcn_fmed3f(ebuf[x] + sem, -a.clip, a.clip);
                out[x] = (TOut)fmaf(al, e, av[i]);
                if (enh) enh[x] = al * e;
            }
        }
    }
}

template <typename TOut, int D>
hipError_t launch_d(const DecodeEnhanceArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((long)a.d.L * a.d.B));
    if (a.d.group <= 8) {
        if constexpr (D == 128) hipLaunchKernelGGL((k_decode_enhance<TOut, 128, 2>), grid, dim3(kDeThreads), 0, stream, a);
        else hipLaunchKernelGGL((k_decode_enhance<TOut, 64, 1>), grid, dim3(kDeThreads), 0, stream, a);
    } else {
        if constexpr (D == 128) hipLaunchKernelGGL((k_decode_enhance<TOut, 128, 4>), grid, dim3(kDeThreads), 0, stream, a);
        else hipLaunchKernelGGL((k_decode_enhance<TOut, 64, 2>), grid, dim3(kDeThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_enhance(const DecodeEnhanceArgs &a, hipStream_t stream) {
    if (a.d.out_bf16) return a.d.d == 128 ? launch_d<__bf16, 128>(a, stream) : launch_d<__bf16, 64>(a, stream);
    return a.d.d == 128 ? launch_d<float, 128>(a, stream) : launch_d<float, 64>(a, stream);
}

}  // namespace sfa
