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
//   k_pool_prep    pool -> bf16 hi/lo in the two MFMA operand orders, 1/|s| and
//                  max |s[x]| of every slot: one record per pool layer.  Run per
//                  call by sfa_enhance, once by sfa_enhance_prepare_pool (the
//                  pool is read-only, so its records can be kept).
//   k_field_agg    EMA of each 64-token tile from zero (a thread per 16-byte
//                  column chunk); only for hidden sizes above kAggMaxH.
//   k_sem          one workgroup per (layer, 64-token tile): cosine scores
//                  C^T = pool · a^T (MFMA), softmax over the slots, 0.5·weights
//                  as MFMA operands in the workspace; on the same pass over
//                  the tile, its field aggregate (EMA from zero).  Extra
//                  workgroups copy the carried ring to the workspace.
//   k_field_carry  field before each tile (exclusive scan), final field; extra
//                  workgroups write the band/field operand table, α and the
//                  semantic-operand choice of each layer, and the new ring (the
//                  last min(R, T) attention rows).
//   k_cols         one workgroup per (layer, 64-token tile, 128 columns): the
//                  tile staged column-major in LDS; ring mean, field and the
//                  semantic sum as one MFMA contraction per 16-token group,
//                  clip, scale, add, store.
// Precision: the fp32 pool, the softmax weights and the band/field
// coefficients enter the MFMAs as bf16 hi + lo pairs (x = hi + lo to ~2^-17
// relative); bf16 attention values are exact, fp32 attention values are split
// the same way (and pass through the epilogue from LDS, unsplit).  With bf16
// inputs, a layer whose error bound allows it (kSemSingleBound below) takes the
// pool^T and weight operands of the semantic sum in k_cols as bf16 hi alone.
#include <type_traits>

#include "sfa_common.h"
#include "sfa_internal.h"

namespace sfa {

namespace {

constexpr int kSlots = 64;
constexpr int kOpElems = 64 * 8;   // one MFMA operand (64 lanes x 8 bf16)
constexpr int kAggMaxH = 8192;     // hidden sizes whose field aggregate k_sem computes
constexpr int kCoefEnt = 8;        // (token group, k-step) pairs of the band/field operand
constexpr int kTabEntries = kCoefEnt * 2 * 64;  // band/field operands (u32x4)
// Single-bf16 semantic operands.  With x = hi(x)·(1+ε), |ε| <= 2^-9, the product
// of the rounded weight 0.5·w_s and the rounded slot entry s_sx is off by at
// most (2^-8 + 2^-18)·0.5·w_s·|s_sx|; the weights sum to one, so the semantic
// term 0.5·sem_x moves by at most 0.5·(2^-8 + 2^-18)·max|s|, and clip (1-
// Lipschitz) and α_l carry that to the output.  A layer takes the single
// operands when α_l times that is at most kSemSingleBound.
constexpr float kSemSingleErr = 0.5f * (0x1p-8f + 0x1p-18f);
constexpr float kSemSingleBound = 1e-5f;
// workgroups that write the band/field operand table, and α and the
// semantic-operand choice of each layer
__host__ __device__ inline int kCallTableBlocks(const EnhanceArgs &a) { return kTabEntries / 256 + (a.L + 255) / 256; }

// sum over the 16 lanes of a DPP row (every lane of the row gets it)
__device__ __forceinline__ float row_sum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, true));  // row_ror:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, true));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, true));  // row_ror:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, true));  // row_ror:1
    return v;
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

// the prepared record of pool layer pl: slot norms, then the two operand tables
__device__ __forceinline__ unsigned char *pool_rec(const EnhanceArgs &a, int pl) {
    return a.pool_rec + (long long)pl * a.pool_rec_bytes;
}
__device__ __forceinline__ uint16_t *rec_poolA(const EnhanceArgs &a, int pl) {
    return reinterpret_cast<uint16_t *>(pool_rec(a, pl) + kPoolRecHeader);
}
__device__ __forceinline__ uint16_t *rec_poolT(const EnhanceArgs &a, int pl) {
    return rec_poolA(a, pl) + (long)a.H * 128;
}

// ---------------------------------------------------------------------------
// Pool operands (the first workgroups of k_pool_prep).  Per pool layer pl:
//   poolA[pl][ks][j][hl][lane][8]: slot 16j + lane%16, x = 32ks + 8(lane/16) + e
//       (A operand of the cosine scores, k = hidden dim)
//   poolT[pl][xg][ks][hl][lane][8]: x = 16xg + lane%16,
//       slot = 32ks + (e<4 ? 4(lane/16)+e : 16+4(lane/16)+e-4)
//       (A operand of the semantic sum, k = slot)
// One workgroup per (pool layer, 32-column step); 256 threads = 4 j x 64 lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pool_prep_block(const EnhanceArgs &a, int bid) {
    const int ksteps = a.H / 32;
    const int pl = bid / ksteps, ks = bid % ksteps;
    const float *P = a.pool + (long)pl * a.pool_stride;
    const int j = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int q4 = lane / 16, c16 = lane % 16;
    uint16_t *poolA = rec_poolA(a, pl);
    uint16_t *poolT = rec_poolT(a, pl);
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
        // row m of half h of the 32-column pair p = xg/2 is column
        // 32p + 8(m/4) + 4h + m%4: after both halves a lane of the MFMA output
        // holds 8 consecutive columns
        const int x = 32 * (xg >> 1) + 8 * (c16 >> 2) + 4 * (xg & 1) + (c16 & 3);
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
// k_field_carry: field before each tile and the final field.  One workgroup per
// (layer, 32 columns); the tiles are split into 8 consecutive parts, each
// folded on its own as (X, Γ) = (field from zero, product of decays), then
// every part takes its carry-in from the parts before it (through LDS) and
// writes the field before each of its tiles.
// ---------------------------------------------------------------------------
constexpr int kFcParts = 8, kFcCols = 32;
__device__ void call_tables_block(const EnhanceArgs &a, int bid);
template <typename TIn>
__device__ void ring_write_block(const EnhanceArgs &a, int bid);

template <typename TIn>
__global__ __launch_bounds__(256) void k_field_carry(EnhanceArgs a) {
    __shared__ float pX[kFcParts][kFcCols], pG[kFcParts];
    const int cpb = a.H / kFcCols;
    {   // past the carry workgroups: the call's operand table and α, then the new ring
        const int extra = (int)blockIdx.x - a.L * cpb;
        const int ntab = kCallTableBlocks(a);
        if (extra >= ntab) return ring_write_block<TIn>(a, extra - ntab);
        if (extra >= 0) return call_tables_block(a, extra);
    }
    const int l = blockIdx.x / cpb;
    const int col = threadIdx.x % kFcCols, part = threadIdx.x / kFcCols;
    const int x = (blockIdx.x % cpb) * kFcCols + col;
    const float g = a.ema_gamma;
    const float gfull = powi(g, kTile);
    const int nt = a.ntiles;
    const int per = (nt + kFcParts - 1) / kFcParts;
    const int i0 = min(part * per, nt), i1 = min(i0 + per, nt);
    const float *A = a.agg64 + (long)l * nt * a.H + x;
    float *C = a.carry + (long)l * nt * a.H + x;
    auto decay = [&](int i) {
        const int len = min(kTile, a.T - i * kTile);
        return len == kTile ? gfull : powi(g, len);
    };
    float X = 0.f, Gm = 1.f;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) {
        const float gl = decay(i);
        X = gl * X + A[(long)i * a.H];
        Gm *= gl;
    }
    // the field before the call's first token, read by every part before the
    // barrier that precedes the last part's write of the final field
    float F = a.field[(long)l * a.H + x];
    pX[part][col] = X;
    if (col == 0) pG[part] = Gm;
    __syncthreads();
    for (int p = 0; p < part; ++p) F = pG[p] * F + pX[p][col];
#pragma unroll 8
    for (int i = i0; i < i1; ++i) {
        C[(long)i * a.H] = F;
        F = decay(i) * F + A[(long)i * a.H];
    }
    if (i1 == nt && i0 < i1) a.field[(long)l * a.H + x] = F;  // the part holding the last tile
}

// ---------------------------------------------------------------------------
// k_sem: one workgroup per (layer, 64-token tile), XCD-aware order.  Wave w
// first scores a quarter of the hidden dimension for all 64 tokens (cosine
// numerators C^T = pool · a^T on MFMA, each pool operand reused by the four
// 16-token groups), the partials meet in LDS, then wave w takes token group w
// through the softmax over the slots and writes 0.5·w as the bf16 hi/lo B
// operands of the semantic sum.
// ---------------------------------------------------------------------------
// eight fp32 attention values (two raw 16-byte words) -> bf16 hi + lo and Σa²
__device__ __forceinline__ void split_a8(const u32x4 *w, bf16x8 &hi, bf16x8 &lo, float &sq) {
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

// copy of the carried ring (row bid of [L][R]) into the workspace: k_cols
// reads the band's tokens before the call from there, so the ring itself can
// be rewritten before k_cols runs
__device__ __forceinline__ void halo_copy_block(const EnhanceArgs &a, int bid) {
    const float4 *src = reinterpret_cast<const float4 *>(a.ring + (long)bid * a.H);
    float4 *dst = reinterpret_cast<float4 *>(a.halo + (long)bid * a.H);
    for (int x = threadIdx.x; x < a.H / 4; x += 256) dst[x] = src[x];
}

template <typename TIn>
__global__ __launch_bounds__(256, 2) void k_sem(EnhanceArgs a) {
    if ((int)blockIdx.x >= a.L * a.ntiles) return halo_copy_block(a, blockIdx.x - a.L * a.ntiles);
    constexpr bool kPrecise = std::is_same<TIn, float>::value;  // fp32 inputs: split a as well
    struct Phase1 {
        f32x4 cp[4][2][4][64];  // [wave][slot tile in round][token group][lane]
        float sq[4][4][64];     // [wave][token group][lane]
    };
    __shared__ __attribute__((aligned(16))) Phase1 p1;
    // during the k-steps the same memory collects the tile's field aggregate
    static_assert(kAggMaxH * sizeof(float) <= sizeof(Phase1), "aggregate must fit the exchange buffer");
    float *aggS = reinterpret_cast<float *>(&p1);

    const int lid = xcd_remap(blockIdx.x, a.L * a.ntiles);
    const int l = lid / a.ntiles, tile = lid % a.ntiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q4 = lane >> 4, c16 = lane & 15;
    const int H = a.H, T = a.T;
    const int tb = tile * kTile;
    const int pl = a.n_pool_layers == 1 ? 0 : l;
    const int ksteps = H / 32;
    const uint16_t *poolA = rec_poolA(a, pl) + lane * 8;
    const float *sinv = reinterpret_cast<const float *>(pool_rec(a, pl));  // 1 / |s| per slot
    const TIn *Ag = reinterpret_cast<const TIn *>(a.attn) + (long)l * T * H;
    const int nj = (a.n_slots + 15) / 16;
    // B operands of this wave's token group, [ks][hi/lo][lane][8]
    uint16_t *wsem = a.wsem + (((long)l * a.ntiles + tile) * 4 + wave) * 4 * kOpElems + lane * 8;

    // ---- (1) partial cosine scores over this wave's quarter of the hidden dim ----
    // lane holds C^T[slot 16j+4q4+i][token tb+16tg+c16] for its k-steps
    const int ks0 = wave * ksteps / 4, ks1 = (wave + 1) * ksteps / 4;
    const bool fuse_agg = H <= kAggMaxH;
    float om[4];  // EMA weight of the lane's token in each group: (1-γ)γ^(len-1-t), 0 past the end
    {
        const int len = min(kTile, T - tb);
        const float g = a.ema_gamma;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            const int t = 16 * tg + c16;
            om[tg] = t < len ? (1.f - g) * powi(g, len - 1 - t) : 0.f;
        }
    }
    f32x4 C[4][4];
    float sq[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
        sq[tg] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) C[j][tg] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // rows past the end read the tile's first row: their scores and weights
    // only reach outputs that are never stored, and their field weight is 0
    const TIn *arow[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
        const int t = tb + 16 * tg + c16;
        arow[tg] = Ag + (long)(t < T ? t : tb) * H + 8 * q4;
    }
    // k-step operands: attention values of the four token groups and the pool
    // tiles
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
    auto compute_ops = [&](const Ops &o, int ks) {
        bf16x8 bh[4], bl[4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            if constexpr (kPrecise) {
                split_a8(o.a[tg], bh[tg], bl[tg], sq[tg]);
            } else {
                bh[tg] = __builtin_bit_cast(bf16x8, o.a[tg][0]);
                bl[tg] = bf16x8{};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = (float)bh[tg][e];
                    sq[tg] = fmaf(v, v, sq[tg]);
                }
            }
        }
        if (fuse_agg) {
            // Σ_t (1-γ)γ^(len-1-t)·a[t][x] over the lane's 4 tokens, then over
            // the 16 lanes of its row; lane c16 = 0 parks the 8 sums in LDS
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = 0.f;
#pragma unroll
                for (int tg = 0; tg < 4; ++tg) {
                    float v;
                    if constexpr (kPrecise) v = __uint_as_float(o.a[tg][e >> 2][e & 3]);
                    else v = (e & 1) ? bf16_hi(o.a[tg][0][e >> 1]) : bf16_lo(o.a[tg][0][e >> 1]);
                    p[e] = fmaf(om[tg], v, p[e]);
                }
                p[e] = row_sum16(p[e]);
            }
            if (c16 == 0) {
                float *d = aggS + 32 * ks + 8 * q4;
                *reinterpret_cast<float4 *>(d) = make_float4(p[0], p[1], p[2], p[3]);
                *reinterpret_cast<float4 *>(d + 4) = make_float4(p[4], p[5], p[6], p[7]);
            }
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
    {   // two buffers in turn: one k-step's loads fly while the other's MFMAs run
        Ops o0, o1;
        if (ks0 < ks1) load_ops(ks0, o0);
        for (int ks = ks0; ks < ks1; ks += 2) {
            if (ks + 1 < ks1) load_ops(ks + 1, o1);
            compute_ops(o0, ks);
            if (ks + 1 >= ks1) break;
            if (ks + 2 < ks1) load_ops(ks + 2, o0);
            compute_ops(o1, ks + 1);
        }
    }
    // the reciprocal norms of this lane's 16 slots
    float isn[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) isn[k] = sinv[16 * (k >> 2) + 4 * q4 + (k & 3)];
    if (fuse_agg) {  // the tile's field aggregate, all H columns
        __syncthreads();
        float *dst = a.agg64 + ((long)l * a.ntiles + tile) * H;
        for (int x = 4 * threadIdx.x; x < H; x += 4 * 256)
            *reinterpret_cast<float4 *>(dst + x) = *reinterpret_cast<const float4 *>(aggS + x);
        __syncthreads();  // the exchange below reuses the buffer
    }

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
                w[4 * j + i] = slot < a.n_slots ? Cw[j][i] * inv_na * isn[4 * j + i] * a.inv_temp_log2e
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
                split_bf16(0.5f * w[4 * (2 * ks + (e >> 2)) + (e & 3)] * inv, h, lo_);  // 0.5·semantic
                h8[e] = h;
                l8[e] = lo_;
            }
            u32x4 *dst = reinterpret_cast<u32x4 *>(wsem + (ks * 2) * kOpElems);
            dst[0] = __builtin_bit_cast(u32x4, h8);
            dst[kOpElems / 8] = __builtin_bit_cast(u32x4, l8);
        }
    }
}

// ---------------------------------------------------------------------------
// k_cols: one workgroup per (layer, 64-token tile, 128-column block); wave w
// owns the 32 columns 32w .. 32w+31 of the block.  The block's attention
// values for tokens tb-16 .. tb+63 are staged in LDS column by column (tokens
// contiguous), so one 16-byte read hands a lane its MFMA operand of eight
// consecutive tokens.  Per 16-token group one accumulator takes
//   D[x][t] = Σ_j A[j][x]·Coef[t][j] + Σ_s pool[s][x]·0.5·w[t][s],
//   Coef[t][j] = 1/R on the ring band (tokens t-R+1 .. t)
//              + 0.5(1-γ)γ^(t-j) for the tile's tokens j <= t,
// and a second one passes a itself through (an identity operand, exact for
// bf16 values); then
//   e = D + 0.5·γ^(t+1)·(field before the tile)
//         [+ the carried ring's share of the band in the call's first tile],
//   out = a + α_l·clip(e).
// Every load is issued before the first output store (outputs wait in
// registers until the end), so no wait for a load ever waits for a store;
// the outputs leave through LDS as whole rows (full 128-byte lines).
// ---------------------------------------------------------------------------
constexpr int kCB = 128;       // columns per workgroup
// token group tg uses the k-steps s = 0 .. kSteps[tg]-1 (staged rows 32s .. 32s+31),
// table entries {0, 1, 3, 5}[tg] + s; its own tokens sit in k-step kIdStep[tg]

template <typename TIn>
struct ColLayout;
// kRows: staged tokens per staging item (one 16-byte piece of each), moved into
// LDS as one 16-byte write per column
template <>
struct ColLayout<__bf16> {
    // column c: chunk b (staged tokens 8b .. 8b+7, 16 bytes) at 16·(b ^ ((4c + c/8) mod 16));
    // both the staging writes and the operand reads meet 16 distinct bank quads
    static constexpr int kColBytes = 256, kRows = 8;
    __device__ static int chunk(int c, int b) { return c * kColBytes + 16 * (b ^ ((4 * c + (c >> 3)) & 15)); }
};
template <>
struct ColLayout<float> {
    // column c: chunk b (staged tokens 4b .. 4b+3, 16 bytes) at 16·b
    static constexpr int kColBytes = 336, kRows = 4;
    __device__ static int chunk(int c, int b) { return c * kColBytes + 16 * b; }
};

// value of the band/field operand: token t of the tile, staged row j (token j-16)
__device__ __forceinline__ float band_field_coef(int t, int j, int R, float g) {
    const int tj = j - kBlk;
    float c = (tj >= t - R + 1 && tj <= t && j < kBlk + kTile) ? 1.f / (float)R : 0.f;
    if (tj >= 0 && tj <= t) c += 0.5f * (1.f - g) * powi(g, t - tj);
    return c;
}

// the staged tile, and at the end the output tile (row-major, 16-byte padded rows)
template <typename TIn, typename TOut>
constexpr int cols_lds_bytes() {
    return kCB * ColLayout<TIn>::kColBytes > kTile * (kCB * (int)sizeof(TOut) + 16)
               ? kCB * ColLayout<TIn>::kColBytes : kTile * (kCB * (int)sizeof(TOut) + 16);
}

// one (layer, tile, column block); kSemLo: the semantic operands (pool^T and
// the slot weights) as bf16 hi + lo pairs, else as bf16 hi alone
template <typename TIn, typename TOut, bool kSemLo>
__device__ __forceinline__ void cols_block(const EnhanceArgs &a, int lid, unsigned char *AsT, u32x4 *TabS) {
    constexpr bool kPrecise = std::is_same<TIn, float>::value;  // fp32 inputs: split a
    using LY = ColLayout<TIn>;
    constexpr int kRowsE = kBlk + kTile;     // staged tokens tb-16 .. tb+63
    constexpr int EPC = 16 / sizeof(TIn);    // columns per 16-byte piece
    constexpr int CPR = kCB / EPC;           // pieces per staged row
    constexpr int RPI = LY::kRows;             // staged tokens per item
    constexpr int NITEM = kRowsE / RPI * CPR;  // staging items: RPI tokens x one piece
    constexpr int NIT = (NITEM + 255) / 256;
    constexpr int NTAB = kTabEntries;
    static_assert(NTAB % 256 == 0, "table copy must split evenly");
    constexpr int kSteps[4] = {1, 2, 2, 3}, kIdStep[4] = {0, 1, 1, 2};
    constexpr int OW = 2 * (int)sizeof(TOut);  // output dwords per 8 values

    const int ncb = (a.H + kCB - 1) / kCB;
    const int cb = lid % ncb, lt = lid / ncb;  // lt = layer * ntiles + tile
    const int l = lt / a.ntiles, tile = lt % a.ntiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q4 = lane >> 4, c16 = lane & 15;
    const int H = a.H, T = a.T, R = a.R;
    const int tb = tile * kTile;
    const int len = min(kTile, T - tb);
    const int xb = cb * kCB;        // the workgroup's first column
    const int xw = xb + 32 * wave;  // the wave's first column
    const bool has = xw < H;        // wave-uniform: H is a multiple of 64
    const int x0 = xw + 8 * q4;     // this lane's 8 output columns
    const TIn *Ag = reinterpret_cast<const TIn *>(a.attn) + (long)l * T * H;

    // ---- (1) loads: staging items, the operand table, pool^T, field carry ----
    // (rows past the end and columns past H read a clamped valid piece: they
    // only feed outputs that are never stored; rows before the stream start,
    // in the call's first tile only, must contribute zero to the band)
    u32x4 stg[NIT][RPI];
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int it = threadIdx.x + 256 * k;
        if (it < NITEM) {
            const int rq = it / CPR, cp = it % CPR;
            const int col = min(xb + cp * EPC, H - EPC);
#pragma unroll
            for (int i = 0; i < RPI; ++i) {
                const int t = min(max(tb - kBlk + RPI * rq + i, 0), T - 1);
                stg[k][i] = *reinterpret_cast<const u32x4 *>(Ag + (long)t * H + col);
            }
            if (tb < kBlk) {  // the first tile: zero the rows before the stream start
#pragma unroll
                for (int i = 0; i < RPI; ++i)
                    if (tb - kBlk + RPI * rq + i < 0) stg[k][i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    u32x4 tab[NTAB / 256];
#pragma unroll
    for (int k = 0; k < NTAB / 256; ++k) tab[k] = reinterpret_cast<const u32x4 *>(a.coef)[threadIdx.x + 256 * k];
    const int pl = a.n_pool_layers == 1 ? 0 : l;
    const uint16_t *poolT = rec_poolT(a, pl) + lane * 8;
    constexpr int SL = kSemLo ? 2 : 1;  // the semantic operands as bf16 hi (+ lo)
    bf16x8 pt[2][2][SL];  // [half][slot k-step][hi/lo]
    float Fc[8];
    if (has) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int sk = 0; sk < 2; ++sk)
#pragma unroll
                for (int hl = 0; hl < SL; ++hl)
                    pt[h][sk][hl] = get8(poolT + (((long)(xw / 16 + h) * 2 + sk) * 2 + hl) * kOpElems);
        const float *carry = a.carry + (long)lt * H + x0;
#pragma unroll
        for (int k = 0; k < 8; k += 4) {
            const float4 c4 = *reinterpret_cast<const float4 *>(carry + k);
            Fc[k] = c4.x; Fc[k + 1] = c4.y; Fc[k + 2] = c4.z; Fc[k + 3] = c4.w;
        }
    }
    // semantic weights of the tile, B operands [tg][ks][hi/lo]: two token groups
    // ahead, the next pair as each group finishes with its own
    const uint16_t *wsem = a.wsem + (long)lt * 4 * 4 * kOpElems + lane * 8;
    bf16x8 wb[2][2][SL];  // [buffer][slot k-step][hi/lo]
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int hl = 0; hl < SL; ++hl) wb[b][ks][hl] = get8(wsem + (b * 4 + ks * 2 + hl) * kOpElems);

    // ---- (2) staging -> column-major LDS tile; table -> LDS ------------------
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int it = threadIdx.x + 256 * k;
        if (it < NITEM) {
            const int rq = it / CPR, cp = it % CPR;
            if constexpr (!kPrecise) {
                // 8 tokens x 8 columns, transposed: per column the 8 tokens as one chunk
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int wd = e >> 1;
                    // bytes of the low (e even) or high (e odd) halves of two rows
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    u32x4 v;
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        v[d] = __builtin_amdgcn_perm(stg[k][2 * d + 1][wd], stg[k][2 * d][wd], sel);
                    *reinterpret_cast<u32x4 *>(AsT + LY::chunk(cp * 8 + e, rq)) = v;
                }
            } else {
                // 4 tokens x 4 columns: per column one 16-byte write
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<u32x4 *>(AsT + LY::chunk(cp * 4 + e, rq)) =
                        u32x4{stg[k][0][e], stg[k][1][e], stg[k][2][e], stg[k][3][e]};
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NTAB / 256; ++k) TabS[threadIdx.x + 256 * k] = tab[k];
    __syncthreads();
    uint32_t ob[4][OW];  // outputs of the lane's 8 columns per token group
    if (has) {  // wave-uniform: a partial last block leaves waves without columns
        // ---- (3) A operands: the staged values, row m of half h = column 8(m/4) + 4h + m%4
        bf16x8 Av[3][2], Al[kPrecise ? 3 : 1][2];
#pragma unroll
        for (int st = 0; st < 3; ++st)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 32 * wave + 8 * (c16 >> 2) + 4 * h + (c16 & 3);
                int b = 4 * st + q4;  // 8-token chunk; past the 80 staged tokens read 16 earlier
                if (b >= kRowsE / 8) b -= 2;  // (their coefficients are zero)
                if constexpr (!kPrecise) {
                    Av[st][h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(AsT + LY::chunk(c, b)));
                } else {
                    const u32x4 w0 = *reinterpret_cast<const u32x4 *>(AsT + LY::chunk(c, 2 * b));
                    const u32x4 w1 = *reinterpret_cast<const u32x4 *>(AsT + LY::chunk(c, 2 * b + 1));
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = __uint_as_float(w0[e]);
                        v[4 + e] = __uint_as_float(w1[e]);
                    }
                    uint16_t hi[8], lo[8];
                    split8(v, hi, lo);
                    Av[st][h] = get8(hi);
                    Al[st][h] = get8(lo);
                }
            }

        // ---- (4) per token group: contraction, epilogue; outputs held until the end
        const float g = a.ema_gamma;
        const float invR = 1.f / (float)R;
        const float al = load_uniform(a.alpha_tab + l);  // α of this layer
        const float gc = powi(g, c16 + 1), g16 = powi(g, kBlk);
        const float *ringl = a.halo + (long)l * R * H;  // the ring as it was before the call
        const int ring0 = a.t0 % R;  // slot of relative token 0
        float *Eg = a.enhancement ? a.enhancement + (long)l * T * H : nullptr;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            if (16 * tg >= len) break;  // wave-uniform
            const int t = 16 * tg + c16;  // this lane's token (tile-relative)
            // the accumulator starts from the field carried into the tile, 0.5·γ^(t+1)·F
            const float cF = 0.5f * gc * powi(g16, tg);
            f32x4 D[2], Da[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int i = 0; i < 4; ++i) D[h][i] = cF * Fc[4 * h + i];
                Da[h] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int st = 0; st < kSteps[tg]; ++st) {
                const int ent = (tg == 0 ? 0 : tg == 1 ? 1 : tg == 2 ? 3 : 5) + st;
                const bf16x8 ch_ = __builtin_bit_cast(bf16x8, TabS[(ent * 2) * 64 + lane]);
                const bf16x8 cl_ = __builtin_bit_cast(bf16x8, TabS[(ent * 2 + 1) * 64 + lane]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    D[h] = mfma_bf16_16x16x32(Av[st][h], ch_, D[h]);
                    D[h] = mfma_bf16_16x16x32(Av[st][h], cl_, D[h]);
                    if constexpr (kPrecise) D[h] = mfma_bf16_16x16x32(Al[st][h], ch_, D[h]);
                }
            }
            // 0.5·semantic: pool^T · (0.5 w)^T (hi·hi + hi·lo + lo·hi with the pairs)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 *w = wb[tg & 1][ks];
                    D[h] = mfma_bf16_16x16x32(pt[h][ks][0], w[0], D[h]);
                    if constexpr (kSemLo) {
                        D[h] = mfma_bf16_16x16x32(pt[h][ks][0], w[1], D[h]);
                        D[h] = mfma_bf16_16x16x32(pt[h][ks][1], w[0], D[h]);
                    }
                }
            }
            if (tg + 2 < 4) {  // every tile has all four groups' weights
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int hl = 0; hl < SL; ++hl)
                        wb[tg & 1][ks][hl] = get8(wsem + ((tg + 2) * 4 + ks * 2 + hl) * kOpElems);
            }
            if constexpr (!kPrecise) {
                // a itself through the identity operand: B[k][n] = 1 where staged row
                // 32·kIdStep + k is token n of the group (row 16 + 16tg + n)
                const int eid = kBlk + 16 * tg + c16 - 32 * kIdStep[tg] - 8 * q4;  // this lane's 1, if 0..7
                const uint32_t one = eid & 1 ? 0x3f800000u : 0x3f80u;
                u32x4 idw;
#pragma unroll
                for (int d = 0; d < 4; ++d) idw[d] = (eid >= 0 && eid < 8 && (eid >> 1) == d) ? one : 0u;
                const bf16x8 id = __builtin_bit_cast(bf16x8, idw);
#pragma unroll
                for (int h = 0; h < 2; ++h) Da[h] = mfma_bf16_16x16x32(Av[kIdStep[tg]][h], id, Da[h]);
            }
            // epilogue for the lane's 8 columns of token t
            if (tg == 0 && tile == 0 && t < R - 1) {
                float halo[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) halo[k] = 0.f;
                // the band's tokens before the call: the carried ring, slot (t0 + j) mod R
                for (int j = t - R + 1; j < 0; ++j) {
                    const int slot = ring0 + j < 0 ? ring0 + j + R : ring0 + j;
                    const float *rr = ringl + (long)slot * H + x0;
#pragma unroll
                    for (int k = 0; k < 8; k += 4) {
                        const float4 r4 = *reinterpret_cast<const float4 *>(rr + k);
                        halo[k] += r4.x; halo[k + 1] += r4.y; halo[k + 2] += r4.z; halo[k + 3] += r4.w;
                    }
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) D[k >> 2][k & 3] += halo[k] * invR;
            }
            float o[8], en[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int h = k >> 2, i = k & 3;
                const float e = __builtin_amdgcn_fmed3f(D[h][i], -a.clip, a.clip);  // clip (clip >= 0)
                en[k] = al * e;
                float av;
                if constexpr (kPrecise) {
                    const int c = 32 * wave + 8 * q4 + k, r = kBlk + t;
                    av = *reinterpret_cast<const float *>(AsT + LY::chunk(c, r >> 2) + 4 * (r & 3));
                } else {
                    av = Da[h][i];
                }
                o[k] = fmaf(al, e, av);
            }
            if constexpr (std::is_same<TOut, float>::value) {
#pragma unroll
                for (int k = 0; k < 8; ++k) ob[tg][k] = __float_as_uint(o[k]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) ob[tg][i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
            }
            if (Eg && tb + t < T) {
                float *ed = Eg + (long)(tb + t) * H + x0;
                *reinterpret_cast<float4 *>(ed) = make_float4(en[0], en[1], en[2], en[3]);
                *reinterpret_cast<float4 *>(ed + 4) = make_float4(en[4], en[5], en[6], en[7]);
            }
        }
    }
    // ---- (5) the output tile through LDS, then whole rows per 16 lanes -----------
    constexpr int ORB = kCB * (int)sizeof(TOut) + 16;  // LDS row stride of the output tile (bytes)
    constexpr int PPR = kCB * (int)sizeof(TOut) / 16;  // 16-byte pieces per output row
    TOut *Og = reinterpret_cast<TOut *>(a.out) + (long)l * T * H;
    __syncthreads();  // every wave is done with the staged tile
    if (has) {
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            if (16 * tg >= len) break;
            unsigned char *d = AsT + (16 * tg + c16) * ORB + (32 * wave + 8 * q4) * (int)sizeof(TOut);
#pragma unroll
            for (int k = 0; k < OW / 4; ++k)
                *reinterpret_cast<u32x4 *>(d + 16 * k) =
                    u32x4{ob[tg][4 * k], ob[tg][4 * k + 1], ob[tg][4 * k + 2], ob[tg][4 * k + 3]};
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < len * PPR; idx += 256) {
        const int r = idx / PPR, pc = idx % PPR;
        const int col = xb + pc * (16 / (int)sizeof(TOut));
        if (col < H)
            st_stream(Og + (long)(tb + r) * H + col, *reinterpret_cast<const u32x4 *>(AsT + r * ORB + 16 * pc));
    }
}

template <typename TIn, typename TOut>
__global__ __launch_bounds__(256, 2) void k_cols(EnhanceArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char AsT[cols_lds_bytes<TIn, TOut>()];
    __shared__ __attribute__((aligned(16))) u32x4 TabS[kTabEntries];
    const int ncb = (a.H + kCB - 1) / kCB;
    const int lid = xcd_remap(blockIdx.x, a.L * a.ntiles * ncb);
    if constexpr (std::is_same<TIn, float>::value) {
        cols_block<TIn, TOut, true>(a, lid, AsT, TabS);
    } else {
        const int l = lid / ncb / a.ntiles;
        if (load_uniform(a.alpha_tab + a.L + l) != 0.f) cols_block<TIn, TOut, false>(a, lid, AsT, TabS);
        else cols_block<TIn, TOut, true>(a, lid, AsT, TabS);
    }
}

// last min(R, T) attention rows -> ring slots (t0 + t) mod R; one workgroup
// per (layer, row).  Runs after the carried ring was copied to the workspace.
template <typename TIn>
__device__ void ring_write_block(const EnhanceArgs &a, int bid) {
    const int l = bid / a.R, r = bid % a.R;
    const int first = max(0, a.T - a.R);
    const int t = first + r;
    if (t >= a.T) return;
    const TIn *A = reinterpret_cast<const TIn *>(a.attn) + ((long)l * a.T + t) * a.H;
    float *dst = a.ring + ((long)l * a.R + (a.t0 % a.R + t % a.R) % a.R) * a.H;
    for (int x = threadIdx.x; x < a.H; x += 256) dst[x] = Elem<TIn>::load(A + x);
}

// the band/field operands of k_cols (the same for every layer and tile),
// entry (e, hi/lo) for e = {0, 1, 3, 5}[tg] + s (the first kTabEntries/256
// workgroups), then α of each layer of the call
__device__ void call_tables_block(const EnhanceArgs &a, int bid) {
    if (bid >= kTabEntries / 256) {
        const int l = (bid - kTabEntries / 256) * 256 + threadIdx.x;
        if (l < a.L) {
            const float al = alpha_layer(a.alpha_base, a.cross_decay, a.layer0 + l, a.n_layers);
            a.alpha_tab[l] = al;
            // bf16 inputs: the semantic operands as single bf16 values where that
            // moves the layer's outputs by at most kSemSingleBound (see below)
            // (the 64 per-slot maxima as 16 loads issued together)
            const float4 *smax = reinterpret_cast<const float4 *>(
                reinterpret_cast<const float *>(pool_rec(a, a.n_pool_layers == 1 ? 0 : l)) + kSlots);
            float4 mv[kSlots / 4];
#pragma unroll
            for (int k = 0; k < kSlots / 4; ++k) mv[k] = smax[k];
            float m = 0.f;
#pragma unroll
            for (int k = 0; k < kSlots / 4; ++k) {
                if (4 * k + 0 < a.n_slots) m = fmaxf(m, mv[k].x);
                if (4 * k + 1 < a.n_slots) m = fmaxf(m, mv[k].y);
                if (4 * k + 2 < a.n_slots) m = fmaxf(m, mv[k].z);
                if (4 * k + 3 < a.n_slots) m = fmaxf(m, mv[k].w);
            }
            a.alpha_tab[a.L + l] = a.in_bf16 && fabsf(al) * kSemSingleErr * m <= kSemSingleBound ? 1.f : 0.f;
        }
        return;
    }
    const int idx = bid * 256 + threadIdx.x;
    const int ln = idx % 64;
    const int ent = idx / 128, hl = (idx / 64) & 1;
    const int tg = ent >= 5 ? 3 : ent >= 3 ? 2 : ent >= 1 ? 1 : 0;
    const int st = ent - (tg == 0 ? 0 : tg == 1 ? 1 : tg == 2 ? 3 : 5);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = band_field_coef(16 * tg + (ln & 15), 32 * st + 8 * (ln >> 4) + e, a.R, a.ema_gamma);
    uint16_t hi[8], lo[8], pick[8];
    split8(v, hi, lo);
#pragma unroll
    for (int e = 0; e < 8; ++e) pick[e] = hl ? lo[e] : hi[e];
    put8(a.coef + (long)idx * 8, pick);
}

// 1/|s| and max_x |s[x]| of one slot: one workgroup per (pool layer, slot)
__device__ __forceinline__ void slot_norm_block(const EnhanceArgs &a, int bid) {
    __shared__ float red[4], redm[4];
    const int pl = bid / kSlots, slot = bid % kSlots;
    float ss = 0.f, mx = 0.f;
    if (slot < a.n_slots) {
        const float *P = a.pool + (long)pl * a.pool_stride + (long)slot * a.H;
        for (int x = threadIdx.x; x < a.H; x += 256) {
            ss = fmaf(P[x], P[x], ss);
            mx = fmaxf(mx, fabsf(P[x]));
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        ss += __shfl_xor(ss, o);
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x >> 6] = ss;
        redm[threadIdx.x >> 6] = mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float *hdr = reinterpret_cast<float *>(pool_rec(a, pl));
        hdr[slot] = 1.f / fmaxf(sqrtf(red[0] + red[1] + red[2] + red[3]), 1e-12f);
        hdr[kSlots + slot] = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
    }
}

// k_pool_prep: the operand tables (the first n_pool_layers·H/32 workgroups),
// then the slot norms, of every pool layer
__global__ __launch_bounds__(256) void k_pool_prep(EnhanceArgs a) {
    const int npp = a.n_pool_layers * (a.H / 32);
    if ((int)blockIdx.x < npp) pool_prep_block(a, blockIdx.x);
    else slot_norm_block(a, blockIdx.x - npp);
}

template <typename TIn, typename TOut>
hipError_t launch_t(const EnhanceArgs &a, hipStream_t stream) {
    if (a.prepare_pool)
        hipLaunchKernelGGL(k_pool_prep, dim3(a.n_pool_layers * (a.H / 32 + kSlots)), dim3(256), 0, stream, a);
    if (a.H > kAggMaxH) {  // k_sem computes the tile aggregates itself up to kAggMaxH
        const int fchunks = a.H / (16 / (int)sizeof(TIn));
        hipLaunchKernelGGL((k_field_agg<TIn>), dim3(a.L * a.ntiles * ((fchunks + 255) / 256)), dim3(256), 0,
                           stream, a);
    }
    hipLaunchKernelGGL((k_sem<TIn>), dim3(a.L * a.ntiles + a.L * a.R), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((k_field_carry<TIn>), dim3(a.L * (a.H / kFcCols) + kCallTableBlocks(a) + a.L * a.R),
                       dim3(256), 0, stream, a);
    hipLaunchKernelGGL((k_cols<TIn, TOut>), dim3(a.L * a.ntiles * ((a.H + kCB - 1) / kCB)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

size_t enhance_workspace_bytes(int L, int T, int H, int n_pool_layers) {
    const size_t nt = ((size_t)T + kTile - 1) / kTile;
    // prepared pool records (a multiple of 256 bytes each)
    const size_t recs = (size_t)n_pool_layers * (size_t)pool_rec_bytes(H);
    // field aggregates and carries, and the carried ring [L][R <= 16][H]
    const size_t floats = 2 * (size_t)L * nt * H + (size_t)L * kMaxWindow * H;
    // semantic weights: per tile 4 token groups x 2 k-steps x hi/lo x 512 bf16;
    // the band/field operand table
    const size_t wsem = (size_t)L * nt * 4 * 4 * kOpElems + (size_t)kTabEntries * 8;
    // α per layer and the per-layer semantic-operand choice, rounded up to 64 floats
    const size_t alphas = (2 * (size_t)L + 63) / 64 * 64;
    return recs + (floats + alphas) * sizeof(float) + wsem * sizeof(uint16_t);
}

hipError_t launch_pool_prepare(const EnhanceArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(k_pool_prep, dim3(a.n_pool_layers * (a.H / 32 + kSlots)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_enhance(const EnhanceArgs &a, hipStream_t stream) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_t<__bf16, __bf16>(a, stream) : launch_t<__bf16, float>(a, stream);
    return a.out_bf16 ? launch_t<float, __bf16>(a, stream) : launch_t<float, float>(a, stream);
}

}  // namespace sfa
