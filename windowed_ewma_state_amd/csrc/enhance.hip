// enhance.hip -- optional triple-channel SFA enhancement for gfx950.
//
// Page "Dalin Soma SFA基于信号场注意力机制的神经网络推理加速框架":
//   section 2.1 -- channel 1, ring buffer of the last 16 attention outputs
//   (mean); channel 2, EMA field f = γ f + (1-γ) a with γ = 0.98; channel 3,
//   64-slot semantic pool aggregated by attention at temperature 0.07;
//   section 2.2 -- enhancement = ring_mean + 0.5·field + 0.5·semantic, clipped
//   to ±ε, scaled by α_layer = α_base·(0.3 + 0.7·layer_ratio)·decay^layer and
//   added to the attention output;
//   section 2.4 -- the ring mean divides by the ring size.
// Defaults (α_base 0.1, cross_decay 0.8, γ 0.98, 16 ring slots, 64 semantic
// slots, clip 0.5) are the SFA_Config of page "Signal Field Attention (SFA)".
//
// Launches:
//   k_pool_prep    pool -> bf16 hi/lo in the two MFMA operand orders.
//   k_slot_norm    |s| of every pool slot.
//   k_field_agg    EMA of each 64-token tile from zero (a thread per 16-byte column chunk).
//   k_field_carry  field before each tile (exclusive scan), final field.
//   k_enhance      one workgroup per (layer, 64-token tile), XCD-aware order;
//                  wave w owns a quarter of the hidden dimension:
//                    cosine scores  C^T = pool · a^T over its quarter (MFMA,
//                                   each pool operand reused by 4 token
//                                   groups of 16), partials summed via LDS,
//                    softmax over the 64 slots (wave w: token group w),
//                    per 64-column chunk of its quarter and 16-token group:
//                    ring-mean + field scan into LDS, semantic sum
//                    sem^T = pool^T · w^T (MFMA), clip, scale, add, store.
//   k_ring_out     last min(R, T) attention rows -> ring (after all reads).
// Precision: the fp32 pool and the softmax weights enter the MFMAs as bf16
// hi + lo pairs (x = hi + lo to ~2^-17 relative); bf16 attention values are
// exact, fp32 attention values are split the same way.
#include <type_traits>

#include "sfa_common.h"
#include "sfa_internal.h"

namespace sfa {

namespace {

constexpr int kSlots = 64;
constexpr int kCols = 64;          // columns per epilogue chunk (one per lane)
constexpr int kOpElems = 64 * 8;   // one MFMA operand (64 lanes x 8 bf16)

__device__ __forceinline__ float alpha_layer(float base, float decay, int layer, int n_layers) {
    const float ratio = n_layers > 1 ? (float)layer / (float)(n_layers - 1) : 0.f;
    return base * (0.3f + 0.7f * ratio) * powf(decay, (float)layer);
}

__device__ __forceinline__ void split8(const float *v, uint16_t *hi, uint16_t *lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)v[e];
        const __bf16 l = (__bf16)(v[e] - (float)h);
        hi[e] = __builtin_bit_cast(uint16_t, h);
        lo[e] = __builtin_bit_cast(uint16_t, l);
    }
}
__device__ __forceinline__ void put8(uint16_t *dst, const uint16_t *v) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)v[2 * i] | ((uint32_t)v[2 * i + 1] << 16);
    *reinterpret_cast<u32x4 *>(dst) = w;
}
__device__ __forceinline__ bf16x8 get8(const uint16_t *src) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(src));
}

// ---------------------------------------------------------------------------
// k_pool_prep.  Per pool layer pl:
//   poolA[pl][ks][j][hl][lane][8]: slot 16j + lane%16, x = 32ks + 8(lane/16) + e
//       (A operand of the cosine scores, k = hidden dim)
//   poolT[pl][xg][ks][hl][lane][8]: x = 16xg + lane%16,
//       slot = 32ks + (e<4 ? 4(lane/16)+e : 16+4(lane/16)+e-4)
//       (A operand of the semantic sum, k = slot)
// One workgroup per (pool layer, 32-column step); 256 threads = 4 j x 64 lanes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pool_prep(EnhanceArgs a) {
    const int ksteps = a.H / 32;
    const int pl = blockIdx.x / ksteps, ks = blockIdx.x % ksteps;
    const float *P = a.pool + (long)pl * a.pool_stride;
    const int j = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int q4 = lane / 16, c16 = lane % 16;
    uint16_t *poolA = a.poolA + (long)pl * ksteps * 4 * 2 * kOpElems;
    uint16_t *poolT = a.poolT + (long)pl * (a.H / 16) * 2 * 2 * kOpElems;
    uint16_t hi[8], lo[8];
    {   // cosine operand
        const int slot = 16 * j + c16;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = slot < a.n_slots ? P[(long)slot * a.H + 32 * ks + 8 * q4 + e] : 0.f;
        split8(v, hi, lo);
        uint16_t *dst = poolA + (((long)ks * 4 + j) * 2) * kOpElems + lane * 8;
        put8(dst, hi);
        put8(dst + kOpElems, lo);
    }
    if (j < 2) {  // semantic operand for the two 16-column tiles of this step
        const int xg = 2 * ks + j;
        const int x = 16 * xg + c16;
#pragma unroll
        for (int sk = 0; sk < 2; ++sk) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int slot = 32 * sk + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + e - 4);
                v[e] = slot < a.n_slots ? P[(long)slot * a.H + x] : 0.f;
            }
            split8(v, hi, lo);
            uint16_t *dst = poolT + (((long)xg * 2 + sk) * 2) * kOpElems + lane * 8;
            put8(dst, hi);
            put8(dst + kOpElems, lo);
        }
    }
}

// ---------------------------------------------------------------------------
// k_field_agg: EMA of each 64-token tile from zero.  A thread owns one 16-byte
// column chunk and scans the tile's tokens in batches of 16 loads in flight.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void k_field_agg(EnhanceArgs a) {
    constexpr int EPC = 16 / sizeof(TIn);
    const int H = a.H, T = a.T;
    const int chunks = H / EPC;
    const int cpb = (chunks + 255) / 256;  // workgroups per (layer, tile)
    const int tl = blockIdx.x / cpb;
    const int ch = (blockIdx.x % cpb) * 256 + threadIdx.x;
    if (ch >= chunks) return;
    const int tile = tl % a.ntiles, l = tl / a.ntiles;
    const float g = a.ema_gamma;
    const int t0 = tile * kTile, len = min(kTile, T - t0);
    const TIn *A = reinterpret_cast<const TIn *>(a.attn) + ((long)l * T + t0) * H + ch * EPC;
    float f[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) f[e] = 0.f;
    for (int j0 = 0; j0 < len; j0 += kBlk) {
        u32x4 raw[kBlk];
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            raw[j] = u32x4{0u, 0u, 0u, 0u};
            if (j0 + j < len) raw[j] = *reinterpret_cast<const u32x4 *>(A + (long)(j0 + j) * H);
        }
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const float keep = (j0 + j < len) ? 1.f : 0.f;  // past the end: f unchanged
            float v[EPC];
            if constexpr (sizeof(TIn) == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = bf16_lo(raw[j][i]);
                    v[2 * i + 1] = bf16_hi(raw[j][i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(raw[j][i]);
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const float nf = g * f[e] + (1.f - g) * v[e];
                f[e] = keep != 0.f ? nf : f[e];
            }
        }
    }
    float *dst = a.agg64 + ((long)l * a.ntiles + tile) * H + ch * EPC;
#pragma unroll
    for (int e = 0; e < EPC; ++e) dst[e] = f[e];
}

// ---------------------------------------------------------------------------
// k_field_carry: field before each tile and the final field (thread per column)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_field_carry(EnhanceArgs a) {
    const int cpb = (a.H + 255) / 256;
    const int l = blockIdx.x / cpb;
    const int x = (blockIdx.x % cpb) * 256 + threadIdx.x;
    if (x >= a.H) return;
    const float g = a.ema_gamma;
    const float gfull = powi(g, kTile);
    float F = a.field[(long)l * a.H + x];
    const float *A = a.agg64 + (long)l * a.ntiles * a.H + x;
    float *C = a.carry + (long)l * a.ntiles * a.H + x;
    for (int i0 = 0; i0 < a.ntiles; i0 += kBlk) {
        float ag[kBlk];
#pragma unroll
        for (int j = 0; j < kBlk; ++j) ag[j] = (i0 + j < a.ntiles) ? A[(long)(i0 + j) * a.H] : 0.f;
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int i = i0 + j;
            if (i < a.ntiles) {
                C[(long)i * a.H] = F;
                const int len = min(kTile, a.T - i * kTile);
                const float gl = len == kTile ? gfull : powi(g, len);
                F = gl * F + ag[j];
            }
        }
    }
    a.field[(long)l * a.H + x] = F;
}

// ---------------------------------------------------------------------------
// k_enhance
// ---------------------------------------------------------------------------
// eight attention values (raw 16-byte words) -> bf16 hi (+ lo for fp32) and Σa²
template <typename TIn>
__device__ __forceinline__ void split_a8(const u32x4 *w, bf16x8 &hi, bf16x8 &lo, float &sq);
template <>
__device__ __forceinline__ void split_a8<__bf16>(const u32x4 *w, bf16x8 &hi, bf16x8 &lo, float &sq) {
    hi = __builtin_bit_cast(bf16x8, w[0]);
    lo = bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = (float)hi[e];
        sq = fmaf(v, v, sq);
    }
}
template <>
__device__ __forceinline__ void split_a8<float>(const u32x4 *w, bf16x8 &hi, bf16x8 &lo, float &sq) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = __uint_as_float(w[e >> 2][e & 3]);
        __bf16 h, l;
        split_bf16(v, h, l);
        hi[e] = h;
        lo[e] = l;
        sq = fmaf(v, v, sq);
    }
}

template <typename T>
__device__ __forceinline__ f32x4 load4f(const T *p);
template <>
__device__ __forceinline__ f32x4 load4f<float>(const float *p) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    return f32x4{v.x, v.y, v.z, v.w};
}
template <>
__device__ __forceinline__ f32x4 load4f<__bf16>(const __bf16 *p) {
    const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
    return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
}

template <typename TOut>
__device__ __forceinline__ void store4o(TOut *p, f32x4 v);
template <>
__device__ __forceinline__ void store4o<float>(float *p, f32x4 v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void store4o<__bf16>(__bf16 *p, f32x4 v) {
    u32x2 w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2 *>(p) = w;
}

template <typename TIn, typename TOut>
__global__ __launch_bounds__(256, 2) void k_enhance(EnhanceArgs a) {
    constexpr bool kPrecise = std::is_same<TIn, float>::value;  // fp32 inputs: split a as well
    constexpr int XS = kCols + 4;                                // LDS row stride (floats)
    // phase 4 stages a quarter of the tile's columns (256) for tokens tb-16 ..
    // tb+63 in LDS, aliasing the phase 1 exchange (cosine partials)
    constexpr int kRowsE = kBlk + kTile;          // staged rows: tokens tb-16 .. tb+63
    constexpr int kQCols = 4 * kCols;             // columns per quarter, one 64-column chunk per wave
    constexpr int EPC = 16 / sizeof(TIn);         // elements per 16-byte piece
    constexpr int QCH = kQCols / EPC;             // 16-byte pieces per staged row
    constexpr int AS = kQCols + EPC;              // staged row stride (elements)
    constexpr int NST = kRowsE * QCH / 256;       // staging loads per thread
    static_assert(kRowsE * QCH % 256 == 0, "staging must split evenly over the workgroup");
    struct Phase1 {
        f32x4 cp[4][2][4][64];  // [wave][slot tile in round][token group][lane]
        float sq[4][4][64];     // [wave][token group][lane]
    };
    constexpr int kStageBytes = kRowsE * AS * (int)sizeof(TIn);
    __shared__ __attribute__((aligned(16))) unsigned char smem[sizeof(Phase1) > kStageBytes
                                                               ? sizeof(Phase1) : kStageBytes];
    __shared__ __attribute__((aligned(16))) float Xs[4][kBlk * XS];  // per wave: ring mean/R + 0.5·field
    __shared__ __attribute__((aligned(16))) u32x4 Wx[4][2][2][64];  // [tg][ks][hi/lo][lane]
    Phase1 &p1 = *reinterpret_cast<Phase1 *>(smem);
    TIn *Ast = reinterpret_cast<TIn *>(smem);

    const int lid = xcd_remap(blockIdx.x, a.L * a.ntiles);
    const int l = lid / a.ntiles, tile = lid % a.ntiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q4 = lane >> 4, c16 = lane & 15;
    const int H = a.H, T = a.T, R = a.R;
    const int tb = tile * kTile;
    const int pl = a.pool_stride == 0 ? 0 : l;
    const int ksteps = H / 32;
    const uint16_t *poolA = a.poolA + (long)pl * ksteps * 4 * 2 * kOpElems + lane * 8;
    const uint16_t *poolT = a.poolT + (long)pl * (H / 16) * 2 * 2 * kOpElems + lane * 8;
    const float *snorm = a.slot_norm + pl * kSlots;
    const TIn *Ag = reinterpret_cast<const TIn *>(a.attn) + (long)l * T * H;
    const float al = alpha_layer(a.alpha_base, a.cross_decay, a.layer0 + l, a.n_layers);
    const int nj = (a.n_slots + 15) / 16;

    // ---- (1) partial cosine scores over this wave's quarter of the hidden dim ----
    // lane holds C^T[slot 16j+4q4+i][token tb+16tg+c16] for its k-steps
    const int ks0 = wave * ksteps / 4, ks1 = (wave + 1) * ksteps / 4;
    f32x4 C[4][4];
    float sq[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
        sq[tg] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) C[j][tg] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const TIn *arow[4];
    bool tok_ok[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
        const int t = tb + 16 * tg + c16;
        tok_ok[tg] = t < T;
        arow[tg] = Ag + (long)(tok_ok[tg] ? t : tb) * H + 8 * q4;
    }
    // k-step operands: attention values of the four token groups and the pool
    // tiles; two buffers in turn, so one k-step's loads fly while the other
    // k-step's MFMAs run
    constexpr int AW = kPrecise ? 2 : 1;  // 16-byte loads per token group
    struct Ops {
        u32x4 a[4][AW];
        bf16x8 ph[4], pl[4];
    };
    auto load_ops = [&](int ks, Ops &o) {
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
#pragma unroll
            for (int h = 0; h < AW; ++h)
                o.a[tg][h] = *reinterpret_cast<const u32x4 *>(arow[tg] + 32 * ks + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < nj) {
                const uint16_t *op = poolA + (((long)ks * 4 + j) * 2) * kOpElems;
                o.ph[j] = get8(op);
                o.pl[j] = get8(op + kOpElems);
            }
        }
    };
    auto compute_ops = [&](const Ops &o) {
        bf16x8 bh[4], bl[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            split_a8<TIn>(o.a[tg], bh[tg], bl[tg], sq[tg]);
            if (!tok_ok[tg]) bh[tg] = bl[tg] = bf16x8{};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < nj) {
#pragma unroll
                for (int tg = 0; tg < 4; ++tg) {
                    C[j][tg] = mfma_bf16_16x16x32(o.ph[j], bh[tg], C[j][tg]);
                    C[j][tg] = mfma_bf16_16x16x32(o.pl[j], bh[tg], C[j][tg]);
                    if constexpr (kPrecise) C[j][tg] = mfma_bf16_16x16x32(o.ph[j], bl[tg], C[j][tg]);
                }
            }
        }
    };
    {
        Ops o0, o1;
        if (ks0 < ks1) load_ops(ks0, o0);
        for (int ks = ks0; ks < ks1; ks += 2) {
            if (ks + 1 < ks1) load_ops(ks + 1, o1);
            compute_ops(o0);
            if (ks + 1 >= ks1) break;
            if (ks + 2 < ks1) load_ops(ks + 2, o0);
            compute_ops(o1);
        }
    }
    // the first column quarter's staging loads fly during phases 2 and 3
    u32x4 stg[NST];
    auto stage_load = [&](int q) {
#pragma unroll
        for (int k = 0; k < NST; ++k) {
            const int idx = threadIdx.x + 256 * k;
            const int r = idx / QCH, c = idx % QCH;
            const int t = tb - kBlk + r;
            const int col = q * kQCols + c * EPC;
            stg[k] = u32x4{0u, 0u, 0u, 0u};
            if (t >= 0 && t < T && col < H) stg[k] = *reinterpret_cast<const u32x4 *>(Ag + (long)t * H + col);
        }
    };
    auto stage_store = [&]() {
#pragma unroll
        for (int k = 0; k < NST; ++k) {
            const int idx = threadIdx.x + 256 * k;
            const int r = idx / QCH, c = idx % QCH;
            *reinterpret_cast<u32x4 *>(&Ast[r * AS + c * EPC]) = stg[k];
        }
    };
    stage_load(0);

    // ---- (2) reduce the four partials: wave w ends with token group tg = w -------
    f32x4 Cw[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) p1.sq[wave][tg][lane] = sq[tg];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) p1.cp[wave][jj][tg][lane] = C[2 * r + jj][tg];
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            f32x4 acc = p1.cp[0][jj][wave][lane];
#pragma unroll
            for (int w2 = 1; w2 < 4; ++w2) {
                const f32x4 o = p1.cp[w2][jj][wave][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += o[i];
            }
            Cw[2 * r + jj] = acc;
        }
        __syncthreads();
    }
    float sqw = p1.sq[0][wave][lane] + p1.sq[1][wave][lane] + p1.sq[2][wave][lane] + p1.sq[3][wave][lane];

    // ---- (3) softmax over slots for token group tg = wave ------------------------
    {
        const float inv_na = 1.f / fmaxf(sqrtf(sum_over_groups(sqw)), 1e-12f);
        float w[16], m = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int slot = 16 * j + 4 * q4 + i;
                w[4 * j + i] = slot < a.n_slots ? Cw[j][i] * inv_na / snorm[slot] * a.inv_temp_log2e
                                                : -INFINITY;
                m = fmaxf(m, w[4 * j + i]);
            }
        m = max_over_groups(m);
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            w[k] = (16 * (k >> 2) + 4 * q4 + (k & 3) < a.n_slots) ? exp2f(w[k] - m) : 0.f;
            sum += w[k];
        }
        const float inv = 1.f / sum_over_groups(sum);
        // B operand of the semantic sum: k-step ks holds slot tiles 2ks (e<4), 2ks+1 (e>=4)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 h8, l8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 h, lo_;
                split_bf16(w[4 * (2 * ks + (e >> 2)) + (e & 3)] * inv, h, lo_);
                h8[e] = h;
                l8[e] = lo_;
            }
            Wx[wave][ks][0][lane] = __builtin_bit_cast(u32x4, h8);
            Wx[wave][ks][1][lane] = __builtin_bit_cast(u32x4, l8);
        }
    }
    __syncthreads();

    // ---- (4) column quarters: stage, then each wave scans its 64-column chunk ----
    // from LDS (ring mean and field along the tokens), and per 16-token group
    // does the semantic sum (MFMA) and the epilogue
    const float g = a.ema_gamma;
    const float invR = 1.f / (float)R;
    const int len = min(kTile, T - tb);
    const float *ringl = a.ring + (long)l * R * H;
    const int ring0 = a.t0 % R;   // slot of relative token 0
    const bool reach_ring = tb < R;  // only the first tile looks back before token 0
    const float *carry = a.carry + ((long)l * a.ntiles + tile) * H;
    float *Xw = Xs[wave];
    TOut *Og = reinterpret_cast<TOut *>(a.out) + (long)l * T * H;
    float *Eg = a.enhancement ? a.enhancement + (long)l * T * H : nullptr;
    const int nch = H / kCols;
    const int nq = (H + kQCols - 1) / kQCols;

    for (int q = 0; q < nq; ++q) {
        __syncthreads();  // the previous quarter (or phase 1) is done with the LDS
        stage_store();
        const int ch = 4 * q + wave;
        const bool has = ch < nch;  // wave-uniform: a partial last quarter leaves waves idle
        const int xc = ch * kCols;
        const int x = xc + lane;
        const int xq = wave * kCols;  // the chunk's first column within the quarter
        // the chunk's own global reads go out before the next quarter's staging
        // loads, so waiting for them never waits for the prefetch: the
        // semantic-sum A operands (4 column tiles x k-steps x hi/lo, shared by
        // the four token groups), the field carried into the tile, and in the
        // first tile the R tokens before it from the carried ring, slot
        // (t0 + t) mod R for t = -R..-1, parked in rows 16-R..15 of the X tile
        bf16x8 pt[kCols / 16][4];
        float F = 0.f;
        if (has) {
#pragma unroll
            for (int xt = 0; xt < kCols / 16; ++xt)
#pragma unroll
                for (int o = 0; o < 4; ++o) pt[xt][o] = get8(poolT + ((long)(xc / 16 + xt) * 4 + o) * kOpElems);
            F = carry[x];
            if (reach_ring) {
#pragma unroll
                for (int k = 0; k < kBlk; ++k) {
                    const int t = k - kBlk;
                    if (t >= -R) {
                        const int slot = ring0 + t < 0 ? ring0 + t + R : ring0 + t;
                        Xw[k * XS + lane] = ringl[(long)slot * H + x];
                    }
                }
            }
        }
        if (q + 1 < nq) stage_load(q + 1);
        __syncthreads();
        if (!has) continue;
        // value of relative token t (-16 <= t < 64) at column x: staged rows, or
        // for t < 0 in the first tile the parked ring values
        const TIn *Acol = Ast + xq + lane;
        auto before = [&](int t) -> float {  // t < 0
            const float xa = Xw[max(0, kBlk + t) * XS + lane];
            const float sa = (float)Acol[(kBlk + t) * AS];
            return reach_ring ? xa : sa;
        };
        // ring mean of tokens -R .. -1 (kept pre-divided by R), then slide:
        // + token t, - token t-R; the field is kept pre-halved (F' = F / 2)
        float rs = 0.f;
#pragma unroll
        for (int k = 0; k < kBlk; ++k) {
            const float v = before(-1 - k);
            rs += k < R ? v : 0.f;
        }
        rs *= invR;
        F *= 0.5f;
        const float hg = 0.5f * (1.f - g);
        for (int tg = 0; tg < 4; ++tg) {
            const int j0 = 16 * tg;
            if (j0 >= len) break;  // wave-uniform
            // the group's 32 reads go out together; the first group takes the
            // tokens before the tile where t - R < 0
            float cur[kBlk], old[kBlk];
#pragma unroll
            for (int j = 0; j < kBlk; ++j) {
                const int t = j0 + j;
                cur[j] = (float)Acol[(kBlk + t) * AS];
                const float os = (float)Acol[(kBlk + t - R) * AS];
                old[j] = (tg == 0 && t - R < 0) ? before(t - R) : os;
            }
            if (j0 + kBlk <= len) {  // wave-uniform: a whole group of tokens
#pragma unroll
                for (int j = 0; j < kBlk; ++j) {
                    rs = fmaf(cur[j] - old[j], invR, rs);
                    F = fmaf(g, F, hg * cur[j]);
                    Xw[j * XS + lane] = rs + F;
                }
            } else {
#pragma unroll
                for (int j = 0; j < kBlk; ++j) {
                    const bool ok = j0 + j < len;
                    rs = ok ? fmaf(cur[j] - old[j], invR, rs) : rs;
                    F = ok ? fmaf(g, F, hg * cur[j]) : F;
                    Xw[j * XS + lane] = rs + F;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const bf16x8 wh0 = __builtin_bit_cast(bf16x8, Wx[tg][0][0][lane]);
            const bf16x8 wl0 = __builtin_bit_cast(bf16x8, Wx[tg][0][1][lane]);
            const bf16x8 wh1 = __builtin_bit_cast(bf16x8, Wx[tg][1][0][lane]);
            const bf16x8 wl1 = __builtin_bit_cast(bf16x8, Wx[tg][1][1][lane]);
            const bool tok_ok_g = tb + j0 + c16 < T;
#pragma unroll
            for (int xt = 0; xt < kCols / 16; ++xt) {
                const bf16x8 th0 = pt[xt][0], tl0 = pt[xt][1], th1 = pt[xt][2], tl1 = pt[xt][3];
                f32x4 sm = {0.f, 0.f, 0.f, 0.f};
                sm = mfma_bf16_16x16x32(th0, wh0, sm);
                sm = mfma_bf16_16x16x32(th0, wl0, sm);
                sm = mfma_bf16_16x16x32(tl0, wh0, sm);
                sm = mfma_bf16_16x16x32(th1, wh1, sm);
                sm = mfma_bf16_16x16x32(th1, wl1, sm);
                sm = mfma_bf16_16x16x32(tl1, wh1, sm);
                // lane: sem[x = xc + 16xt + 4q4 + i][token tb + j0 + c16]
                const int xl = 16 * xt + 4 * q4;
                const f32x4 X4 = *reinterpret_cast<const f32x4 *>(&Xw[c16 * XS + xl]);
                const f32x4 A4 = load4f<TIn>(&Ast[(kBlk + j0 + c16) * AS + xq + xl]);
                f32x4 o, en;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = fminf(fmaxf(X4[i] + 0.5f * sm[i], -a.clip), a.clip);
                    en[i] = al * e;
                    o[i] = A4[i] + en[i];
                }
                // the output goes back into the X tile (row c16, same byte row): a
                // bf16 value lands on fp32 columns [xl/2, xl/2 + 2), which every
                // lane has read by this column tile, an fp32 value on its own spot
                store4o<TOut>(reinterpret_cast<TOut *>(&Xw[c16 * XS]) + xl, o);
                if (Eg && tok_ok_g) store4o<float>(Eg + (long)(tb + j0 + c16) * H + xc + xl, en);
            }
            // whole 128- or 256-byte rows of the 16 x 64 output tile
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            constexpr int OPR = kCols * (int)sizeof(TOut) / 16;  // 16-byte pieces per output row
#pragma unroll
            for (int k = 0; k < kBlk * OPR / 64; ++k) {
                const int idx = lane + 64 * k;
                const int r = idx / OPR, c = idx % OPR;
                const u32x4 w = *reinterpret_cast<const u32x4 *>(
                    reinterpret_cast<const unsigned char *>(&Xw[r * XS]) + 16 * c);
                if (j0 + r < len)
                    st_stream(reinterpret_cast<unsigned char *>(Og + (long)(tb + j0 + r) * H + xc) + 16 * c, w);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// last min(R, T) attention rows -> ring slots (t0 + t) mod R; one workgroup
// per (layer, row)
template <typename TIn>
__global__ __launch_bounds__(256) void k_ring_out(EnhanceArgs a) {
    const int l = blockIdx.x / a.R, r = blockIdx.x % a.R;
    const int first = max(0, a.T - a.R);
    const int t = first + r;
    if (t >= a.T) return;
    const TIn *A = reinterpret_cast<const TIn *>(a.attn) + ((long)l * a.T + t) * a.H;
    float *dst = a.ring + ((long)l * a.R + (a.t0 % a.R + t % a.R) % a.R) * a.H;
    for (int x = threadIdx.x; x < a.H; x += 256) dst[x] = Elem<TIn>::load(A + x);
}

// per-slot norms: one workgroup per (pool layer, slot)
__global__ __launch_bounds__(256) void k_slot_norm(EnhanceArgs a) {
    __shared__ float red[4];
    const int pl = blockIdx.x / kSlots, slot = blockIdx.x % kSlots;
    float ss = 0.f;
    if (slot < a.n_slots) {
        const float *P = a.pool + (long)pl * a.pool_stride + (long)slot * a.H;
        for (int x = threadIdx.x; x < a.H; x += 256) ss = fmaf(P[x], P[x], ss);
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0)
        a.slot_norm[pl * kSlots + slot] = fmaxf(sqrtf(red[0] + red[1] + red[2] + red[3]), 1e-12f);
}

template <typename TIn, typename TOut>
hipError_t launch_t(const EnhanceArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(k_pool_prep, dim3(a.n_pool_layers * (a.H / 32)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(k_slot_norm, dim3(a.n_pool_layers * kSlots), dim3(256), 0, stream, a);
    const int fchunks = a.H / (16 / (int)sizeof(TIn));
    hipLaunchKernelGGL((k_field_agg<TIn>), dim3(a.L * a.ntiles * ((fchunks + 255) / 256)), dim3(256), 0,
                       stream, a);
    hipLaunchKernelGGL(k_field_carry, dim3(a.L * ((a.H + 255) / 256)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((k_enhance<TIn, TOut>), dim3(a.L * a.ntiles), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((k_ring_out<TIn>), dim3(a.L * a.R), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t enhance_workspace_bytes(int L, int T, int H, int n_pool_layers) {
    const size_t nt = (size_t)((T + kTile - 1) / kTile);
    const size_t floats = 2 * (size_t)L * nt * H + (size_t)n_pool_layers * kSlots;
    // poolA and poolT: H/32 steps x 4 tiles (resp. H/16 x 2 steps) x hi/lo x 512 bf16
    const size_t ops = (size_t)n_pool_layers * (size_t)H * 64 * 2 * 2;
    return floats * sizeof(float) + ops * sizeof(uint16_t);
}

hipError_t launch_enhance(const EnhanceArgs &a, hipStream_t stream) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_t<__bf16, __bf16>(a, stream) : launch_t<__bf16, float>(a, stream);
    return a.out_bf16 ? launch_t<float, __bf16>(a, stream) : launch_t<float, float>(a, stream);
}

}  // namespace sfa
