// prefill.hip -- SFA prefill for gfx950: causal sliding-window attention over
// the last W <= 16 tokens plus the far-field EWMA of the keys that leave the
// window, fused as O = O_near + α·S_t.
//
// Page "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩",
// section 2.1: near-field equation (softmax(q·K_near^T/sqrt(d))·V_near over
// the most recent k tokens), far-field equation (S_t = γ S_{t-1} + (1-γ)·key
// leaving the window) and the fusion equation; section 2.2 (O(k·n·d) time).
//
// Three launches per call:
//   k_ewma_agg    one wave per (b, KV head, 64-token tile): the tile's local
//                 EWMA aggregate (scan from 0; with the running mean, its map
//                 and key sum) and, where the attention kernel reads them, its
//                 16-token blocks' (fp32 inputs; with γ per query head, as
//                 block-start partials of every query head's chain).
//   k_ewma_carry  one workgroup per (scan chain, 16 head-dim columns):
//                 exclusive scan of the tile aggregates -> S just before every
//                 tile; writes the final S.
//   k_window_attn one workgroup per (b, KV head, tile), XCD-aware order:
//                 stages K rows [t0-16, t0+64) row-major and V transposed in
//                 LDS, shared by all query heads of the GQA group; each wave
//                 owns 16 tokens: EWMA scan from its carry, then per head
//                 8 score MFMAs (two 16-key tiles) + 16 PV MFMAs (P split into
//                 bf16 hi + lo) and the α·S epilogue.
// A fourth, tiny launch copies the last W keys/values into the ring when the
// call continues an existing cache (the first tile reads the old ring).
//
// Folded carries (S per KV head, bf16 inputs, at most 64 tiles per sequence;
// chosen by the library for such calls): k_ewma_agg also writes the first
// tile's carry (S before the call), k_ewma_carry does not run, and every
// k_window_attn<.., FOLD> workgroup folds the aggregates of the tiles before
// it onto that carry; the last tile writes the final S.
//
// Single pass (on request; S per KV head, bf16 inputs, at most 64 tiles per
// sequence):
//   k_fused_init  clears the published-aggregate words, saves the carried S;
//   k_window_attn<.., FUSED> forms each tile's aggregate from its own scan,
//                 publishes it, and folds those of the earlier tiles of its
//                 sequence (no scan launches, K read once).
// Measured slower than the two launches of the scan on every workload tried:
// the workgroups wait for the published aggregates, whose round trips queue
// behind the streaming Q/K/V/O traffic.
#include <type_traits>

#include "sfa_common.h"
#include "sfa_internal.h"

namespace sfa {

namespace {

constexpr int kRows = kTile + kMaxWindow;  // staged rows: tokens t0-16 .. t0+63

// pointer to the key/value row of relative token index t (t < 0 reads the ring
// of a continued sequence; returns nullptr when the position does not exist)
template <typename T>
__device__ __forceinline__ const T *kv_row(const T *x_bg, long row_stride, const T *ring_bg, int t,
                                           int n, int p0, int W, int D) {
    if (t >= 0) return t < n ? x_bg + (long)t * row_stride : nullptr;
    const int pos = p0 + t;
    if (pos < 0 || ring_bg == nullptr) return nullptr;
    return ring_bg + (long)(pos % W) * D;
}

template <typename T, int EPL>
__device__ __forceinline__ void load_epl(const T *p, float *x) {
    if constexpr (EPL == 2) {
        load2(p, x[0], x[1]);
    } else {
        x[0] = Elem<T>::load(p);
    }
}

// ---------------------------------------------------------------------------
// k_ewma_agg: local aggregates A (EWMA from zero) of 16-token blocks and tiles.
// One wave per 64-token tile of one (b, KV head) chain (four chains per
// workgroup).  Lane (w, c) owns the 16-byte chunk c of the head dimension for
// block w of the tile, so every load is a 16-byte vector and a block's 16 rows
// are in flight together.  A block's scan carries A/(1-γ), one FMA per evicted
// key and element, and applies (1-γ) once at its end.
//
// RM (running mean of the keys that have left the window): a segment maps the
// incoming (S, C) to g·S + β·C + s and C + c, with g = γ^(evicting steps), c
// the sum of the keys it evicts, s its S from (0, 0) and β = Σ over its
// evicting steps of (1-γ)·γ^(later evicting steps)/m; m = p-W+1 at position p.
// The kernel writes s and c per tile (fp32 inputs: per block too) and β per
// tile.
// ---------------------------------------------------------------------------
template <typename TIn, int D, bool RM, bool QH>
__global__ __launch_bounds__(256) void k_ewma_agg(PrefillArgs a) {
    constexpr int EPC = 16 / sizeof(TIn);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;           // chunks per row (8 or 16 for bf16, 16 or 32 for fp32)
    constexpr int LPB = 64 / 4;            // lanes per block: 16
    constexpr int CPL = CPR / LPB > 0 ? CPR / LPB : 1;  // chunks per lane
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tiles_per_bg = a.ntiles;
    // chain fastest: the waves of a workgroup take the same tile of consecutive
    // (b, KV head) pairs, i.e. neighbouring 256-byte pieces of the same rows.
    // With γ per query head the wave folds its keys, loaded once, into the
    // scan chain of every query head of the group.
    const int nkv = a.B * a.Hkv;
    const int gt = blockIdx.x * 4 + wave;
    if (gt >= nkv * tiles_per_bg) return;
    const int tile = gt / nkv, kvp = gt - tile * nkv;
    const int b = kvp / a.Hkv, G = kvp % a.Hkv;
    const int nh = QH ? a.group : 1;  // scan chains these keys feed
    const int n = a.n, W = a.W;
    const int p0 = a.pos0 ? max(0, a.pos0[b]) : 0;
    const long row_stride = (long)a.Hkv * D;
    const TIn *Kbg = reinterpret_cast<const TIn *>(a.k) + ((long)b * n * a.Hkv + G) * D;
    const TIn *ringK = a.pos0 ? reinterpret_cast<const TIn *>(a.ring_k) + ((long)b * a.Hkv + G) * W * D : nullptr;
    const int blk = lane / LPB, c0 = lane % LPB;
    const int tb = tile * kTile + kBlk * blk;
    const bool lane_ok = c0 < CPR;  // d = 64 bf16 has 8 chunks per row: half the lanes idle

    // the keys this lane's block of 16 tokens evicts, loaded once
    u32x4 raw[kBlk][CPL];
    bool use[kBlk];
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
        const int t = tb + j;
        use[j] = lane_ok && (t < n) && (p0 + t >= W);
        const TIn *row = use[j] ? kv_row(Kbg, row_stride, ringK, t - W, n, p0, W, D) : nullptr;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            raw[j][cc] = u32x4{0u, 0u, 0u, 0u};
            if (row) raw[j][cc] = *reinterpret_cast<const u32x4 *>(row + (c0 + LPB * cc) * EPC);
        }
    }
    __shared__ float blkv[4][4][D];  // [wave][block][d]
    __shared__ float blkc[RM ? 4 : 1][4][RM ? D : 1];
    __shared__ float decay[4][4], beta[4][4];
    if constexpr (!RM && !QH) {
        if (a.fold && tile == 0) {  // the first tile's carry: S before the call
            const long bgs = (long)b * a.Hkv + G;
            float *c0p = a.carry + bgs * a.ntiles * D;
            for (int e = lane; e < D; e += 64) c0p[e] = (a.pos0 && p0 > 0) ? a.state[bgs * D + e] : 0.f;
        }
    }
    // γ per query head: the keys are converted once per pass and folded into
    // HC chains at a time (heads past the group repeat the last one)
    constexpr int HC = QH ? 2 : 1;
    const int blen = max(0, min(kBlk, n - tb));
    const int steps = max(0, blen - max(0, W - p0 - tb));
    for (int h0 = 0; h0 < nh; h0 += HC) {
    float gmh[HC];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) gmh[hh] = a.gamma[QH ? G * a.group + min(h0 + hh, nh - 1) : G];
    float Ah[HC][CPL][EPC], Cs[RM ? CPL : 1][EPC];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < EPC; ++e) Ah[hh][cc][e] = 0.f;
    // RM: the block folds the running means C_j/m_j of its evicting tokens,
    // Σ_j γ^(evicting tokens after j)·C_j/m_j = Σ_i k_i·w_i with
    // w_i = Σ_{j >= i} γ^(evicting tokens after j)/m_j (a suffix sum, the same
    // for every lane of the block); w at the first evicting token is β/(1-γ).
    // 1/m by v_rcp_f32 (within 1 ulp; m >= 1 is exact in fp32), not the IEEE
    // division sequence.
    float wt[RM ? kBlk : 1];
    float wsum = 0.f;
    if constexpr (RM) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < EPC; ++e) Cs[cc][e] = 0.f;
        float gp = 1.f;
#pragma unroll
        for (int j = kBlk - 1; j >= 0; --j) {
            const int p = p0 + tb + j;
            if (tb + j < n && p >= W) {
                wsum = fmaf(gp, __builtin_amdgcn_rcpf((float)(p - W + 1)), wsum);
                gp *= gmh[0];
            }
            wt[j] = wsum;
        }
    }
    if (lane_ok) {
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            if (!use[j]) continue;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                float v[EPC];
                if constexpr (sizeof(TIn) == 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] = bf16_lo(raw[j][cc][i]);
                        v[2 * i + 1] = bf16_hi(raw[j][cc][i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(raw[j][cc][i]);
                }
                // A/(1-γ), one FMA per step; the factor is applied once below
                if constexpr (RM) {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        Cs[cc][e] += v[e];
                        Ah[0][cc][e] = fmaf(wt[j], v[e], Ah[0][cc][e]);
                    }
                } else {
#pragma unroll
                    for (int hh = 0; hh < HC; ++hh)
#pragma unroll
                        for (int e = 0; e < EPC; ++e) Ah[hh][cc][e] = fmaf(gmh[hh], Ah[hh][cc][e], v[e]);
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < HC; ++hh)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                for (int e = 0; e < EPC; ++e) Ah[hh][cc][e] *= 1.f - gmh[hh];
    }
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
    if (h0 + hh >= nh) break;
    const int hs = QH ? G * a.group + h0 + hh : G;  // the scan chain's S head
    const int bg = b * a.Hs + hs;
    const float gm = gmh[hh];
    float (&A)[CPL][EPC] = Ah[hh];
    // 16-token block aggregates, then the tile aggregate: blocks combined in
    // order through LDS, T = ((A0·g1 + A1)·g2 + A2)·g3 + A3 with g_w the decay
    // over block w's evicting steps (RM: T = g_w·T + β_w·TC + A_w, TC += C_w)
    float *a16 = a.agg16 + (((long)bg * a.ntiles + tile) * 4 + blk) * D;
    const float gl = powi(gm, steps);
    const float bw = RM ? (1.f - gm) * wsum : 0.f;  // RM: β of this lane's block
    // (with bf16 inputs and S per KV head, plain or with the running mean, the
    // attention kernel forms the block maps from its own scan and reads only
    // the tile carries; with γ per query head the tile composition below
    // writes the running partials)
    constexpr bool kWrite16 = !QH && sizeof(TIn) != 2;
    if (lane_ok && kWrite16) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < EPC; ++e) a16[(c0 + LPB * cc) * EPC + e] = A[cc][e];
        if constexpr (RM) {
            float *c16 = a.csum16 + (((long)bg * a.ntiles + tile) * 4 + blk) * D;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                for (int e = 0; e < EPC; ++e) c16[(c0 + LPB * cc) * EPC + e] = Cs[cc][e];
        }
    }
    if (lane_ok) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                blkv[wave][blk][(c0 + LPB * cc) * EPC + e] = A[cc][e];
                if constexpr (RM) blkc[wave][blk][(c0 + LPB * cc) * EPC + e] = Cs[cc][e];
            }
    }
    if (c0 == 0) {
        decay[wave][blk] = gl;
        beta[wave][blk] = bw;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const long trec = (long)bg * a.ntiles + tile;
    float *a64 = a.agg64 + trec * D;
    for (int e = lane; e < D; e += 64) {
        float T = 0.f, TC = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // QH: slot w-1 holds P(w), the EWMA from zero over blocks 0 .. w-1
            // (what block w starts from before the tile's carry is added)
            if constexpr (QH) {
                if (w > 0) a.agg16[(trec * 4 + w - 1) * D + e] = T;
            }
            if constexpr (RM) {
                T = decay[wave][w] * T + beta[wave][w] * TC + blkv[wave][w][e];
                TC += blkc[wave][w][e];
            } else {
                T = decay[wave][w] * T + blkv[wave][w][e];
            }
        }
        a64[e] = T;
        if constexpr (RM) a.csum64[trec * D + e] = TC;
    }
    if constexpr (RM) {
        if (lane == 0) {
            float Bt = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) Bt = decay[wave][w] * Bt + beta[wave][w];
            a.beta64[trec] = Bt;
        }
    }
    // the next chain reuses this wave's LDS rows
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    }
}

// number of evicting steps (positions >= W) among tokens [s0, s0+len)
__device__ __forceinline__ int evict_steps(int p0, int s0, int len, int W) {
    const int first = max(s0, W - p0);  // first relative token with p0 + t >= W
    return max(0, s0 + len - max(first, s0));
}

// ---------------------------------------------------------------------------
// k_ewma_carry: S before each tile (exclusive scan over tiles) and final S.
// One workgroup per (scan chain, 16 head-dim elements); 64 parts of the tile
// range are scanned in parallel (up to kCarryRegs tiles per part: every load
// of the part issued at once and kept in registers for the rescan), the part
// aggregates are combined by one wave per column (a shuffle scan over the 64
// parts, between two barriers), and each part is rescanned from its carry-in.
// ---------------------------------------------------------------------------
constexpr int kCarryParts = 64, kCarryCols = 16, kCarryRegs = 16;

// RM: the same scan over the affine maps (g, β, s, c) of the tiles, carrying
// (S, C); parts compose as (G, B, X, Cx) then (g, β, s, c) ->
// (g·G, g·B + β, g·X + β·Cx + s, Cx + c).  It also writes C before each tile
// and the final mean C/m.
template <bool RM>
__global__ __launch_bounds__(1024) void k_ewma_carry(PrefillArgs a) {
    static_assert(kCarryParts == kWave && kCarryCols * kCarryParts == 1024, "one wave per column, one lane per part");
    __shared__ float partX[kCarryParts][kCarryCols];
    __shared__ float partC[RM ? kCarryParts : 1][kCarryCols];
    __shared__ float partG[kCarryParts], partB[kCarryParts];
    const int D = a.d;
    const int cblocks = D / kCarryCols;
    const int bg = blockIdx.x / cblocks;
    const int e = (blockIdx.x % cblocks) * kCarryCols + threadIdx.x % kCarryCols;
    const int part = threadIdx.x / kCarryCols;
    const int col = threadIdx.x % kCarryCols;
    const int b = bg / a.Hs, hs = bg % a.Hs;
    const int n = a.n, W = a.W, nt = a.ntiles;
    const int p0 = a.pos0 ? max(0, a.pos0[b]) : 0;
    const float gm = a.gamma[hs];
    const long sw = RM ? 2L * D : (long)D;  // state words per chain
    const float S_init = (a.pos0 && p0 > 0) ? a.state[(long)bg * sw + e] : 0.f;
    // RM: the key sum restarts as the carried mean times the keys it averages
    const float C_init = (RM && a.pos0 && p0 > 0) ? a.state[(long)bg * sw + D + e] * (float)max(0, p0 - W) : 0.f;
    const float g64 = powi(gm, kTile);

    const int per = (nt + kCarryParts - 1) / kCarryParts;
    const int i0 = min(part * per, nt), i1 = min(i0 + per, nt);
    const float *A = a.agg64 + (long)bg * nt * D + e;
    const float *Cs = RM ? a.csum64 + (long)bg * nt * D + e : nullptr;
    const float *Bt = RM ? a.beta64 + (long)bg * nt : nullptr;
    // γ^(evicting steps of tile i): every tile but the first (which may start
    // inside the first window, W <= 16 < 64) and the last (which may be
    // short) evicts 64 keys
    const float g_first = powi(gm, evict_steps(p0, 0, min(kTile, n), W));
    const float g_last = powi(gm, evict_steps(p0, (nt - 1) * kTile, n - (nt - 1) * kTile, W));
    auto decay_of = [&](int i) { return i == 0 ? g_first : i == nt - 1 ? g_last : g64; };
    // the part's tiles in registers when it has at most kCarryRegs of them
    // (tiles past the part read its first tile and are never used)
    const bool regs = per <= kCarryRegs;
    float Ar[kCarryRegs], Cr[RM ? kCarryRegs : 1], Br[RM ? kCarryRegs : 1];
    if (regs) {
#pragma unroll
        for (int j = 0; j < kCarryRegs; ++j) {
            const int i = i0 + j < i1 ? i0 + j : min(i0, nt - 1);
            Ar[j] = A[(long)i * D];
            if constexpr (RM) {
                Cr[j] = Cs[(long)i * D];
                Br[j] = Bt[i];
            }
        }
    }
    float X = 0.f, Gam = 1.f, Bc = 0.f, Cx = 0.f;
    if (regs) {
        // tiles past the part fold as the identity (decay 1, zero terms)
#pragma unroll
        for (int j = 0; j < kCarryRegs; ++j) {
            const bool in = i0 + j < i1;
            const float gl = in ? decay_of(i0 + j) : 1.f, av = in ? Ar[j] : 0.f;
            if constexpr (RM) {
                const float be = in ? Br[j] : 0.f;
                X = gl * X + be * Cx + av;
                Cx += in ? Cr[j] : 0.f;
                Bc = gl * Bc + be;
            } else {
                X = gl * X + av;
            }
            Gam *= gl;
        }
    } else {
#pragma unroll 8
        for (int i = i0; i < i1; ++i) {
            const float gl = decay_of(i);
            if constexpr (RM) {
                const float be = Bt[i];
                X = gl * X + be * Cx + A[(long)i * D];
                Cx += Cs[(long)i * D];
                Bc = gl * Bc + be;
            } else {
                X = gl * X + A[(long)i * D];
            }
            Gam *= gl;
        }
    }
    // inclusive scan of the part aggregates over parts: wave w takes column
    // w, lane = part, log2(parts) shuffle steps with the combine
    // (X_a, Γ_a) then (X_b, Γ_b) -> (Γ_b·X_a + X_b, Γ_a·Γ_b)
    // (RM: X = Γ_b·X_a + B_b·Cx_a + X_b, Cx = Cx_a + Cx_b, B = Γ_b·B_a + B_b)
    partX[part][col] = X;
    if constexpr (RM) partC[part][col] = Cx;
    if (col == 0) {
        partG[part] = Gam;
        partB[part] = Bc;
    }
    __syncthreads();
    {
        const int w = threadIdx.x / kWave, ln = threadIdx.x % kWave;
        float x = partX[ln][w], g = partG[ln];
        float c = RM ? partC[ln][w] : 0.f, bb = RM ? partB[ln] : 0.f;
#pragma unroll
        for (int off = 1; off < kCarryParts; off <<= 1) {
            const float px = __shfl_up(x, off), pg = __shfl_up(g, off);
            const float pc = RM ? __shfl_up(c, off) : 0.f, pb = RM ? __shfl_up(bb, off) : 0.f;
            if (ln >= off) {
                if constexpr (RM) {
                    x = g * px + bb * pc + x;
                    c = pc + c;
                    bb = g * pb + bb;
                } else {
                    x = g * px + x;
                }
                g = pg * g;
            }
        }
        __syncthreads();  // every wave has read the part aggregates
        partX[ln][w] = x;
        if constexpr (RM) partC[ln][w] = c;
        if (w == 0) {
            partG[ln] = g;
            partB[ln] = bb;
        }
    }
    __syncthreads();
    // carry into this part: (S_init, C_init) through all earlier parts
    float C = S_init, K = C_init;
    if (part > 0) {
        C = partG[part - 1] * S_init + partX[part - 1][col];
        if constexpr (RM) {
            C += partB[part - 1] * C_init;
            K = C_init + partC[part - 1][col];
        }
    }
    float *Cout = a.carry + (long)bg * nt * D + e;
    float *Kout = RM ? a.ccarry + (long)bg * nt * D + e : nullptr;
    X = C;
    if (regs) {
#pragma unroll
        for (int j = 0; j < kCarryRegs; ++j) {
            if (i0 + j < i1) {
                const int i = i0 + j;
                Cout[(long)i * D] = X;
                if constexpr (RM) {
                    Kout[(long)i * D] = K;
                    X = decay_of(i) * X + Br[j] * K + Ar[j];
                    K += Cr[j];
                } else {
                    X = decay_of(i) * X + Ar[j];
                }
            }
        }
    } else {
#pragma unroll 8
        for (int i = i0; i < i1; ++i) {
            Cout[(long)i * D] = X;
            if constexpr (RM) {
                Kout[(long)i * D] = K;
                X = decay_of(i) * X + Bt[i] * K + A[(long)i * D];
                K += Cs[(long)i * D];
            } else {
                X = decay_of(i) * X + A[(long)i * D];
            }
        }
    }
    if (part == kCarryParts - 1 && a.state) {
        a.state[(long)bg * sw + e] = X;
        if constexpr (RM) {
            const int m_end = max(0, p0 + n - W);
            a.state[(long)bg * sw + D + e] = m_end > 0 ? K / (float)m_end : 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// k_window_attn: windowed softmax attention + α·S epilogue
// ---------------------------------------------------------------------------
// One step of a log-step scan of S = A·S + V over the 16 lanes of a DPP row:
// lane c16 takes the (A, V) of lane c16 - SH (row_shr; lanes below SH keep theirs)
template <int SH>
__device__ __forceinline__ float row_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + SH, 0xf, 0xf, true));
}
// one step of a log-step prefix sum over the 16 lanes of a DPP row
template <int SH, int NK>
__device__ __forceinline__ void row_sum_step(f32x4 (*V)[2]) {
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int i = 0; i < 4; ++i) V[k][half][i] += row_shr<SH>(V[k][half][i]);
}
// the same scan as row_scan_step carrying a second, scalar V (B = A·B + β)
template <int SH, int NK>
__device__ __forceinline__ void row_scan_step2(f32x4 (*V)[2], float &B, float &A, int c16) {
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int i = 0; i < 4; ++i) V[k][half][i] = fmaf(A, row_shr<SH>(V[k][half][i]), V[k][half][i]);
    B = fmaf(A, row_shr<SH>(B), B);
    const float Ap = row_shr<SH>(A);
    A = c16 >= SH ? A * Ap : A;
}
template <int SH, int NK>
__device__ __forceinline__ void row_scan_step(f32x4 (*V)[2], float &A, int c16) {
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int i = 0; i < 4; ++i) V[k][half][i] = fmaf(A, row_shr<SH>(V[k][half][i]), V[k][half][i]);
    const float Ap = row_shr<SH>(A);
    A = c16 >= SH ? A * Ap : A;
}

// ---------------------------------------------------------------------------
// Single pass (S per KV head, bf16 inputs, at most kFusedMaxTiles tiles per
// sequence): no scan launches.  Each attention workgroup publishes its tile's
// aggregate (the EWMA of the tile's evicted keys from zero) and folds the
// aggregates of the earlier tiles of its sequence onto the carried S.
// ---------------------------------------------------------------------------
constexpr uint64_t kAggTag = 1ull << 32;  // high word of a published aggregate element
constexpr int kSpinLimit = 1 << 20;       // polls before a workgroup gives up waiting

// workgroup -> (chain, tile) with the tiles of a chain in dispatch order, so a
// workgroup only ever waits for workgroups dispatched before it.  With a
// multiple of 8 chains, chain c runs on XCD c mod 8 (consecutive tiles share
// that XCD's L2 for the K/V halo); otherwise in workgroup order.
__device__ __forceinline__ int fused_tile_order(int bid, int nchains, int ntiles) {
    if (nchains % 8 == 0) {
        const int xcd = bid % 8, idx = bid / 8;
        return ((idx / ntiles) * 8 + xcd) * ntiles + idx % ntiles;
    }
    return bid;
}

// S before tile `tile` of chain bg: wave 0 first publishes this tile's
// aggregate (its four blocks composed, from the block aggregates in LDS); then
// the earlier tiles are split into four contiguous ranges, wave w folds range
// w as (Γ_w, X_w) = (decay over the range, EWMA of the range from zero), and
// C = the carried S composed with the four ranges in order.
template <int D, int EPL>
__device__ __forceinline__ void fused_carry(const PrefillArgs &a, int bg, int tile, int p0, float gm, int wave,
                                            int lane, int e0, const float (*BlkAgg)[D], float (*FoldX)[D],
                                            float *FoldG, float *C) {
    const int n = a.n, W = a.W;
    uint64_t *rec = a.tagged + (long)bg * a.ntiles * D;
    auto tile_decay = [&](int j) {
        const int s0 = j * kTile;
        return powi(gm, evict_steps(p0, s0, min(kTile, n - s0), W));
    };
    if (wave == 0) {
        float X[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) X[e] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int s0 = tile * kTile + kBlk * w;
            const float gl = s0 < n ? powi(gm, evict_steps(p0, s0, min(kBlk, n - s0), W)) : 1.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) X[e] = gl * X[e] + BlkAgg[w][e0 + e];
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            __hip_atomic_store(rec + (long)tile * D + e0 + e, kAggTag | __float_as_uint(X[e]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    constexpr int kPer = (kFusedMaxTiles + 3) / 4;  // earlier tiles per wave, at most
    const int per = (tile + 3) / 4;
    const int j0 = min(__builtin_amdgcn_readfirstlane(wave) * per, tile), j1 = min(j0 + per, tile);
    uint64_t v[kPer][EPL];
    bool ready = false;
    for (int it = 0; it < kSpinLimit && !ready; ++it) {
        if (it > 0) __builtin_amdgcn_s_sleep(2);
        bool ok = true;
#pragma unroll
        for (int jj = 0; jj < kPer; ++jj) {
            if (j0 + jj < j1) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    v[jj][e] = __hip_atomic_load(rec + (long)(j0 + jj) * D + e0 + e, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                    ok = ok && (v[jj][e] >> 32) == (kAggTag >> 32);
                }
            }
        }
        ready = __builtin_amdgcn_ballot_w64(!ok) == 0;  // every lane's words published
    }
    // (an earlier tile is whole; only the first can evict fewer than 64 keys,
    // since W <= 16: the others all decay by γ^64)
    const float g64 = powi(gm, kTile), gfirst = tile_decay(0);
    float X[EPL], G = 1.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) X[e] = 0.f;
#pragma unroll
    for (int jj = 0; jj < kPer; ++jj) {
        if (j0 + jj < j1) {
            const float g = j0 + jj == 0 ? gfirst : g64;
#pragma unroll
            for (int e = 0; e < EPL; ++e) X[e] = g * X[e] + __uint_as_float((uint32_t)v[jj][e]);
            G *= g;
        }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) FoldX[wave][e0 + e] = X[e];
    if (lane == 0) FoldG[wave] = G;
    __syncthreads();
    const float *si = a.sinit + (long)bg * D + e0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) C[e] = si[e];
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < EPL; ++e) C[e] = FoldG[w] * C[e] + FoldX[w][e0 + e];
}

// before the single pass: clear the published-aggregate words (tag 0: not yet
// published) and take the carried S (or 0) out of `state`, which the pass
// itself overwrites with the final S
__global__ __launch_bounds__(256) void k_fused_init(PrefillArgs a) {
    const long words = (long)a.B * a.Hkv * a.ntiles * a.d;
    const long zero_blocks = (words / 2 + 255) / 256;
    if ((long)blockIdx.x < zero_blocks) {
        const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 2;
        if (i < words) *reinterpret_cast<u32x4 *>(a.tagged + i) = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const long idx = ((long)blockIdx.x - zero_blocks) * 256 + threadIdx.x;
    if (idx >= (long)a.B * a.Hkv * a.d) return;
    const int b = (int)(idx / ((long)a.Hkv * a.d));
    const bool carried = a.pos0 != nullptr && a.pos0[b] > 0;
    a.sinit[idx] = carried ? a.state[idx] : 0.f;
}

template <typename TIn> struct Lds;
template <> struct Lds<__bf16> { static constexpr int kpad = 8, vpad = 0; };
template <> struct Lds<float> { static constexpr int kpad = 4, vpad = 4; };

// bf16 V^T tile: rows of 80 keys (40 dwords) with the dword column XORed by
// 2·((row / 8) mod 4).  The PV operand reads of 16 lanes hit rows r + 8a + b
// (a, b < 4): the row stride alone maps a to the same banks, the XOR moves the
// four a to distinct dword pairs, so a read is free of bank conflicts.
__device__ __forceinline__ int vt_dword(int row, int col) { return row * (kRows / 2) + (col ^ (2 * ((row >> 3) & 3))); }

template <typename TOut>
__device__ __forceinline__ void store4(TOut *p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float *p, f32x4 v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16 *p, f32x4 v) {
    u32x2 w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2 *>(p) = w;
}

// query heads whose Q operands are in flight together: 4 at d = 128; at d = 64
// the registers hold 8, so groups of up to 8 heads need no refills
template <int D> constexpr int q_slots() { return D == 64 ? 8 : 4; }

template <typename TOut>
__device__ __forceinline__ void store8(TOut *p, const float *v);
template <>
__device__ __forceinline__ void store8<float>(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store8<__bf16>(__bf16 *p, const float *v) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4 *>(p) = w;
}

// QH: γ and S per query head (scan chains (b, query head)); each head's S tile
// is rebuilt in the head loop from its carry and the wave's evicted keys.
// RM: the running mean of the keys that have left the window is the EWMA
// input; the wave starts from the tile's carried (S, C) and the maps of its
// earlier blocks (bf16: formed by the waves' own row scans, shared through
// LDS; fp32: written by k_ewma_agg), then scans C += k, S = γS + (1-γ)·C/m.
// Two workgroups per CU, except fp32 inputs at d = 128: their fp32 K rows and
// split V^T staging take 119 KB of LDS, so one workgroup per CU is all the
// LDS allows and the register budget follows that.
template <typename TIn, int D>
constexpr int attn_wg_per_cu() { return std::is_same<TIn, float>::value && D == 128 ? 1 : 2; }
template <typename TIn, typename TOut, int D, int MODE, bool FUSED = false, bool FOLD = false>
__global__ __launch_bounds__(256, (attn_wg_per_cu<TIn, D>())) void k_window_attn(PrefillArgs a) {
    constexpr bool QH = MODE == kQueryHead, RM = MODE == kRunningMean;
    constexpr bool kBf16 = std::is_same<TIn, __bf16>::value;
    constexpr int EPL = D / kWave;
    constexpr int KS = D + Lds<TIn>::kpad;      // Klds row stride (elements)
    constexpr int VS = kRows + Lds<TIn>::vpad;  // Vt row stride (elements)
    constexpr int SS = D + 4;                   // Sb row stride (floats)
    constexpr int EPC = 16 / sizeof(TIn);       // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                // chunks per row

    __shared__ __attribute__((aligned(16))) TIn Klds[kRows * KS];
    __shared__ __attribute__((aligned(16))) TIn Vt[D * VS];
    // S per KV head with bf16 inputs stays in registers (epilogue layout, a row
    // scan over the wave's 16 tokens); the LDS slot then only carries S at the
    // block start.  The other modes keep each token's S row in LDS.
    constexpr bool kRegS = !QH && kBf16;
    static_assert(!(FUSED || FOLD) || (kRegS && !RM), "the single-pass and folded forms exist for S per KV head with bf16 inputs");
    static_assert(!(FUSED && FOLD), "one carry form at a time");
    __shared__ __attribute__((aligned(16))) float Sb[4][kRegS ? D : kBlk * SS];
    // kRegS: each wave's block aggregate (the EWMA of its 16 tokens from zero);
    // single pass: the waves' partial folds of the earlier tiles' aggregates
    __shared__ __attribute__((aligned(16))) float BlkAgg[kRegS ? 4 : 1][kRegS ? D : 1];
    // kRegS with the running mean: each wave's block key sum, its map's decay
    // and β, and the key sum C at its block start
    constexpr bool kRegC = kRegS && RM;
    __shared__ __attribute__((aligned(16))) float BlkC[kRegC ? 4 : 1][kRegC ? D : 1];
    __shared__ __attribute__((aligned(16))) float Kb[kRegC ? 4 : 1][kRegC ? D : 1];
    __shared__ float BlkG[4], BlkB[4];
    __shared__ __attribute__((aligned(16))) float FoldX[FUSED || FOLD ? 4 : 1][FUSED || FOLD ? D : 1];
    __shared__ float FoldG[4];

    const int nblk = a.B * a.Hkv * a.ntiles;
    const int lid = FUSED ? fused_tile_order(blockIdx.x, a.B * a.Hkv, a.ntiles) : xcd_remap(blockIdx.x, nblk);
    const int tile = lid % a.ntiles;
    const int bg = lid / a.ntiles;
    const int b = bg / a.Hkv, G = bg % a.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q4 = lane >> 4, c16 = lane & 15;
    const int n = a.n, W = a.W, group = a.group;
    const int t0 = tile * kTile;
    const int p0 = a.pos0 ? max(0, a.pos0[b]) : 0;
    const float gm = QH ? 0.f : a.gamma[G];  // KV-head decay (QH reads its heads' own)
    const int tb = t0 + kBlk * wave;  // this wave's 16 tokens
    const int tok = tb + c16;         // this lane's token in the MFMA layouts
    const bool tok_ok = tok < n;

    const long row_stride = (long)a.Hkv * D;
    const TIn *Kbg = reinterpret_cast<const TIn *>(a.k) + ((long)b * n * a.Hkv + G) * D;
    const TIn *Vbg = reinterpret_cast<const TIn *>(a.v) + ((long)b * n * a.Hkv + G) * D;
    const bool cont = a.pos0 != nullptr;
    const TIn *ringKr = cont ? reinterpret_cast<const TIn *>(a.ring_k) + (long)bg * a.W * D : nullptr;
    const TIn *ringVr = cont ? reinterpret_cast<const TIn *>(a.ring_v) + (long)bg * a.W * D : nullptr;
    // a fresh prompt hands its last W keys/values to the ring here
    const bool write_ring = !cont && a.ring_k != nullptr;
    TIn *ringKw = write_ring ? reinterpret_cast<TIn *>(a.ring_k) + (long)bg * a.W * D : nullptr;
    TIn *ringVw = write_ring ? reinterpret_cast<TIn *>(a.ring_v) + (long)bg * a.W * D : nullptr;
    const TIn *Qtok = reinterpret_cast<const TIn *>(a.q) + (((long)b * n + tok) * a.Hq + (long)G * group) * D;
    TOut *Otok = reinterpret_cast<TOut *>(a.out) + (((long)b * n + tok) * a.Hq + (long)G * group) * D;

    // The wave issues its query and K/V loads at a raised priority, so that they go
    // out ahead of the other resident workgroup's arithmetic (0.3% per step).
    __builtin_amdgcn_s_setprio(1);
    // ---- (0) the first heads' queries go out before the K/V staging ----------
    // (B operands of the score MFMA: lane = token c16, 8 head-dim elements)
    // Qc[i] holds the head h with h % kQSlots == i; it is refilled with head
    // h + kQSlots as soon as head h is done, so kQSlots heads are always in flight.
    // The loads are row-shaped: lane L reads the 16-byte chunk L % (D/8) of token
    // L / (D/8) (+ 64/(D/8) per load) of the block, whole rows per instruction;
    // an LDS tile turns them into MFMA operands.
    constexpr int kQSlots = q_slots<D>();
    constexpr int CPT = D / 8, TPI = 64 / CPT, QLD = kBlk / TPI;
    const int rt = lane / CPT, rc = lane % CPT;
    const TIn *Qrow = reinterpret_cast<const TIn *>(a.q) + (((long)b * n + tb + rt) * a.Hq + (long)G * group) * D + 8 * rc;
    const long qtok_stride = (long)TPI * a.Hq * D;  // next token of this lane
    u32x4 Qc[kQSlots][QLD];
    if constexpr (kBf16) {
#pragma unroll
        for (int hh = 0; hh < kQSlots; ++hh)
#pragma unroll
            for (int j = 0; j < QLD; ++j) {
                Qc[hh][j] = u32x4{0u, 0u, 0u, 0u};
                if (hh < group && tb + rt + TPI * j < n)
                    Qc[hh][j] = ld_stream(Qrow + j * qtok_stride + (long)hh * D);
            }
    }

    // the S carried into the tile and the aggregates of this wave's earlier
    // blocks (read in step 2) go out with the queries, ahead of the staging
    const int e0 = lane * EPL;
    // carry of scan chain `chain` at this tile and the aggregates of the
    // wave's earlier blocks
    auto carry_loads = [&](long chain, float *Cx, float (*Ax)[EPL]) {
        const long tbase = chain * a.ntiles + tile;
        const float *C = a.carry + tbase * D + e0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) Cx[e] = C[e];
        if constexpr (QH) {
            // the partial P(wave) of this wave's block start (wave 0 loads P(1)
            // and ignores it: one unconditional load keeps the waits exact)
            const float *A = a.agg16 + (tbase * 4 + max(wave - 1, 0)) * D + e0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) Ax[0][e] = A[e];
        } else {
            // (all three blocks are loaded unconditionally, in bounds for every
            // wave; only w < wave are used)
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                const float *A = a.agg16 + (tbase * 4 + w) * D + e0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) Ax[w][e] = A[e];
            }
        }
    };
    // QH: chain of query head h of this group
    const long chain0 = QH ? (long)b * a.Hq + (long)G * group : (long)bg;
    float Cin[EPL], Ain[kRegS ? 1 : 3][EPL];
    // FOLD: wave w folds the earlier tiles [fj0, fj1) (a quarter of them); their
    // aggregates are loaded here, unconditionally (a clamped index past the
    // range), so the waits for these loads are counted exactly
    constexpr int kFoldPer = FOLD ? (kFusedMaxTiles + 3) / 4 : 1;
    float foldv[kFoldPer][FOLD ? EPL : 1];
    const int fper = (tile + 3) / 4;
    const int fj0 = min(__builtin_amdgcn_readfirstlane(wave) * fper, tile), fj1 = min(fj0 + fper, tile);
    if constexpr (kRegS) {
        // the block aggregates come from this tile's own scan (step 3); the
        // single pass folds the earlier tiles' aggregates instead of a carry,
        // and the folded form folds them onto the first tile's carry
        if constexpr (!FUSED) {
            const float *C = a.carry + (chain0 * a.ntiles + (FOLD ? 0 : tile)) * D + e0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) Cin[e] = C[e];
        }
        if constexpr (FOLD) {
            const float *A64 = a.agg64 + chain0 * a.ntiles * D + e0;
#pragma unroll
            for (int jj = 0; jj < kFoldPer; ++jj) {
                const int j = min(fj0 + jj, a.ntiles - 1);
#pragma unroll
                for (int e = 0; e < EPL; ++e) foldv[jj][e] = A64[(long)j * D + e];
            }
        }
    } else {
        carry_loads(chain0, Cin, Ain);
    }
    // RM: the key sum carried into the tile and (S rows in LDS) the earlier
    // blocks' key sums
    float Kin[RM ? EPL : 1], Kblk[RM && !kRegS ? 3 : 1][RM && !kRegS ? EPL : 1];
    if constexpr (RM) {
        const long tbase = chain0 * a.ntiles + tile;
#pragma unroll
        for (int e = 0; e < EPL; ++e) Kin[e] = a.ccarry[tbase * D + e0 + e];
        if constexpr (!kRegS) {
#pragma unroll
            for (int w = 0; w < 3; ++w)
#pragma unroll
                for (int e = 0; e < EPL; ++e) Kblk[w][e] = a.csum16[(tbase * 4 + w) * D + e0 + e];
        }
    }

    // ---- (1) stage K rows (row-major) and V (transposed) ---------------------
    // Every load of the staging is issued before the first LDS write, so the
    // tile waits for one memory latency, not one per chunk.
    constexpr int KCH = kRows * CPR;  // 16-byte chunks of the staged K rows
    constexpr int KIT = (KCH + 255) / 256;
    u32x4 kst[KIT];
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
        const int idx = tid + 256 * it;
        kst[it] = u32x4{0u, 0u, 0u, 0u};
        if (idx < KCH) {
            const TIn *src = kv_row(Kbg, row_stride, ringKr, t0 - kMaxWindow + idx / CPR, n, p0, W, D);
            if (src) kst[it] = *reinterpret_cast<const u32x4 *>(src + (idx % CPR) * EPC);
        }
    }
    if constexpr (kBf16) {
        // two keys per thread so each LDS write is one aligned dword; key pairs
        // vary fastest across lanes so a write instruction hits consecutive banks
        constexpr int kPairs = kRows / 2;
        constexpr int VCH = kPairs * CPR;
        constexpr int VIT = (VCH + 255) / 256;
        u32x4 vsa[VIT], vsb[VIT];
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = tid + 256 * it;
            vsa[it] = vsb[it] = u32x4{0u, 0u, 0u, 0u};
            if (idx < VCH) {
                const int m = idx % kPairs, c = idx / kPairs;
                const int ta = t0 - kMaxWindow + 2 * m;
                const TIn *sa = kv_row(Vbg, row_stride, ringVr, ta, n, p0, W, D);
                const TIn *sb = kv_row(Vbg, row_stride, ringVr, ta + 1, n, p0, W, D);
                if (sa) vsa[it] = *reinterpret_cast<const u32x4 *>(sa + c * EPC);
                if (sb) vsb[it] = *reinterpret_cast<const u32x4 *>(sb + c * EPC);
            }
        }
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int idx = tid + 256 * it;
            if (idx < KCH) {
                const int r = idx / CPR, c = idx % CPR;
                const int t = t0 - kMaxWindow + r;
                *reinterpret_cast<u32x4 *>(&Klds[r * KS + c * EPC]) = kst[it];
                if (write_ring && t >= t0 && t < n && t >= n - W)
                    *reinterpret_cast<u32x4 *>(ringKw + (long)(t % W) * D + c * EPC) = kst[it];
            }
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = tid + 256 * it;
            if (idx < VCH) {
                const int m = idx % kPairs, c = idx / kPairs;
                const int ta = t0 - kMaxWindow + 2 * m;
                const u32x4 va = vsa[it], vb = vsb[it];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t lo = (va[i] & 0xffffu) | (vb[i] << 16);
                    const uint32_t hi = (va[i] >> 16) | (vb[i] & 0xffff0000u);
                    reinterpret_cast<uint32_t *>(Vt)[vt_dword(c * EPC + 2 * i, m)] = lo;
                    reinterpret_cast<uint32_t *>(Vt)[vt_dword(c * EPC + 2 * i + 1, m)] = hi;
                }
                if (write_ring) {
                    if (ta >= t0 && ta < n && ta >= n - W)
                        *reinterpret_cast<u32x4 *>(ringVw + (long)(ta % W) * D + c * EPC) = va;
                    if (ta + 1 >= t0 && ta + 1 < n && ta + 1 >= n - W)
                        *reinterpret_cast<u32x4 *>(ringVw + (long)((ta + 1) % W) * D + c * EPC) = vb;
                }
            }
        }
    } else {
        constexpr int VCH = kRows * CPR;
        constexpr int VIT = (VCH + 255) / 256;
        float4 vs[VIT];
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = tid + 256 * it;
            vs[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (idx < VCH) {
                const int r = idx % kRows, c = idx / kRows;
                const TIn *src = kv_row(Vbg, row_stride, ringVr, t0 - kMaxWindow + r, n, p0, W, D);
                if (src) vs[it] = *reinterpret_cast<const float4 *>(src + c * EPC);
            }
        }
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int idx = tid + 256 * it;
            if (idx < KCH) {
                const int r = idx / CPR, c = idx % CPR;
                const int t = t0 - kMaxWindow + r;
                *reinterpret_cast<u32x4 *>(&Klds[r * KS + c * EPC]) = kst[it];
                if (write_ring && t >= t0 && t < n && t >= n - W)
                    *reinterpret_cast<u32x4 *>(ringKw + (long)(t % W) * D + c * EPC) = kst[it];
            }
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int idx = tid + 256 * it;
            if (idx < VCH) {
                const int r = idx % kRows, c = idx / kRows;
                const int t = t0 - kMaxWindow + r;
                const float4 val = vs[it];
                Vt[(c * EPC + 0) * VS + r] = val.x;
                Vt[(c * EPC + 1) * VS + r] = val.y;
                Vt[(c * EPC + 2) * VS + r] = val.z;
                Vt[(c * EPC + 3) * VS + r] = val.w;
                if (write_ring && t >= t0 && t < n && t >= n - W)
                    *reinterpret_cast<float4 *>(ringVw + (long)(t % W) * D + c * EPC) = val;
            }
        }
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- (2) S just before this wave's 16-token block (KV heads) ------------
    // S_{block start} = carry through the wave's earlier blocks of the tile
    auto block_start = [&](float g, const float *Cx, float (*Ax)[EPL], float *Sx) {
        if constexpr (QH) {
            // S = (decay over blocks 0 .. wave-1)·C + P(wave)
            const int s0 = t0, len = min(kBlk * wave, n - s0);
            const float gw = powi(g, evict_steps(p0, s0, max(len, 0), W));
#pragma unroll
            for (int e = 0; e < EPL; ++e) Sx[e] = wave > 0 ? gw * Cx[e] + Ax[0][e] : Cx[e];
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) Sx[e] = Cx[e];
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                if (w < wave) {
                    const int s0 = t0 + kBlk * w;
                    const float gl = powi(g, evict_steps(p0, s0, min(kBlk, n - s0), W));
#pragma unroll
                    for (int e = 0; e < EPL; ++e) Sx[e] = gl * Sx[e] + Ax[w][e];
                }
            }
        }
    };
    float *Sw = Sb[wave];
    f32x4 Sreg[kRegS ? D / 32 : 1][2];  // kRegS: S of the lane's token at d = 32k + 8q4 + 4half + i
    // QH: the keys evicted by this wave's 16 tokens, kept in registers (the K
    // staging area is reused in the head loop)
    float kev[QH ? kBlk : 1][EPL];
    float Ac = 1.f;  // kRegS: decay from the block start to the lane's token
    float Bq = 0.f;  // kRegC: weight of the block-start key sum in the lane's S
    if constexpr (kRegS) {
        __syncthreads();
        // ---- (3) EWMA through the block from zero, then the block aggregate ----
        // lane (q4, c16) needs S_t for its token t = tb + c16 at
        // d = 32k + 8q4 + 4half + i.  Per token the step is S = A·S + V with
        // (A, V) = (γ, (1-γ)·k_{t-W}) if t evicts, else (1, 0); a log-step
        // scan over the 16 lanes of the row composes them.  Lane c16 = 15 then
        // holds the whole block's map: its V is the block's aggregate.
        const int t = tb + c16;
        const bool ev = t < n && p0 + t >= W;
        Ac = ev ? gm : 1.f;
        const float w1 = ev ? 1.f - gm : 0.f;
        // token t - W sits in staged row (t - W) - (t0 - 16)
        const TIn *kr = &Klds[(kBlk * wave + c16 + kMaxWindow - W) * KS + 8 * q4];
        f32x4 Kreg[kRegC ? D / 32 : 1][2];
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
            const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(kr + 32 * k);
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (kRegC)
                        Kreg[k][half][i] = ev ? (float)kk[4 * half + i] : 0.f;
                    else
                        Sreg[k][half][i] = w1 * (float)kk[4 * half + i];
                }
        }
        if constexpr (kRegC) {
            // running mean: per evicting token C += k and S = γ·S + β_t·C with
            // β_t = (1-γ)/m_t.  From the block start (S0, C0), C_t = C0 + K_t
            // (K_t the block's prefix sum of evicted keys) and
            // S_t = Γ_t·S0 + B_t·C0 + V_t, where V_t = γ_t·V_{t-1} + β_t·K_t
            // and B_t = γ_t·B_{t-1} + β_t: a prefix sum, then the scan of
            // (γ_t, β_t·K_t) carrying B beside V.
            const float bt = ev ? (1.f - gm) * __builtin_amdgcn_rcpf((float)(p0 + t - W + 1)) : 0.f;
            row_sum_step<1, D / 32>(Kreg);
            row_sum_step<2, D / 32>(Kreg);
            row_sum_step<4, D / 32>(Kreg);
            row_sum_step<8, D / 32>(Kreg);
#pragma unroll
            for (int k = 0; k < D / 32; ++k)
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Sreg[k][half][i] = bt * Kreg[k][half][i];
            Bq = bt;
            row_scan_step2<1, D / 32>(Sreg, Bq, Ac, c16);
            row_scan_step2<2, D / 32>(Sreg, Bq, Ac, c16);
            row_scan_step2<4, D / 32>(Sreg, Bq, Ac, c16);
            row_scan_step2<8, D / 32>(Sreg, Bq, Ac, c16);
        } else {
            row_scan_step<1, D / 32>(Sreg, Ac, c16);
            row_scan_step<2, D / 32>(Sreg, Ac, c16);
            row_scan_step<4, D / 32>(Sreg, Ac, c16);
            row_scan_step<8, D / 32>(Sreg, Ac, c16);
        }
        if (c16 == kBlk - 1) {
#pragma unroll
            for (int k = 0; k < D / 32; ++k)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    *reinterpret_cast<f32x4 *>(&BlkAgg[wave][32 * k + 8 * q4 + 4 * half]) = Sreg[k][half];
                    if constexpr (kRegC)
                        *reinterpret_cast<f32x4 *>(&BlkC[wave][32 * k + 8 * q4 + 4 * half]) = Kreg[k][half];
                }
            if (kRegC && q4 == 0) {
                BlkG[wave] = Ac;
                BlkB[wave] = Bq;
            }
        }
    } else if constexpr (!QH) {
        float S[EPL], Ck[RM ? EPL : 1];
        if constexpr (RM) {
            // (S, C) at the block start: each earlier block w maps them to
            // g_w·S + β_w·C + A_w and C + K_w
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                S[e] = Cin[e];
                Ck[e] = Kin[e];
            }
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                if (w < wave) {
                    const int s0 = t0 + kBlk * w;
                    const int len = min(kBlk, n - s0);
                    const float gl = powi(gm, evict_steps(p0, s0, len, W));
                    float bw = 0.f;
                    for (int j = 0; j < len; ++j) {
                        const int p = p0 + s0 + j;
                        if (p >= W) bw = gm * bw + (1.f - gm) / (float)(p - W + 1);
                    }
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        S[e] = gl * S[e] + bw * Ck[e] + Ain[w][e];
                        Ck[e] += Kblk[w][e];
                    }
                }
            }
        } else {
            block_start(gm, Cin, Ain, S);
        }
        __syncthreads();

        // ---- (3) EWMA through the block: S_t after token t's own eviction -----
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int t = tb + j;
            if (t < n && p0 + t >= W) {
                // token t - W sits in staged row (t - W) - (t0 - 16)
                const TIn *kr = &Klds[(kBlk * wave + j + kMaxWindow - W) * KS + e0];
                float kv[EPL];
                load_epl<TIn, EPL>(kr, kv);
                if constexpr (RM) {
                    const float inv_m = 1.f / (float)(p0 + t - W + 1);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        Ck[e] += kv[e];
                        S[e] = gm * S[e] + (1.f - gm) * (Ck[e] * inv_m);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) S[e] = gm * S[e] + (1.f - gm) * kv[e];
                }
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) Sw[j * SS + e0 + e] = S[e];
        }
    } else {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kBlk; ++j)
            load_epl<TIn, EPL>(&Klds[(kBlk * wave + j + kMaxWindow - W) * KS + e0], kev[j]);
    }
    __syncthreads();
    if constexpr (kRegS) {
        // ---- S before the tile, and at this wave's block start ----------------
        float C[EPL];
        if constexpr (FUSED) {
            fused_carry<D, EPL>(a, bg, tile, p0, gm, wave, lane, e0, BlkAgg, FoldX, FoldG, C);
        } else if constexpr (FOLD) {
            // (Γ_w, X_w) of this wave's range, then C = the first tile's carry
            // composed with the four ranges in order
            // (an earlier tile is whole; only the first can evict fewer than
            // 64 keys, since W <= 16: the others all decay by γ^64)
            const float g64 = powi(gm, kTile);
            const float gfirst = powi(gm, evict_steps(p0, 0, kTile, W));
            float X[EPL], Gr = 1.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) X[e] = 0.f;
#pragma unroll
            for (int jj = 0; jj < kFoldPer; ++jj) {
                if (fj0 + jj < fj1) {
                    const float g = fj0 + jj == 0 ? gfirst : g64;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) X[e] = g * X[e] + foldv[jj][e];
                    Gr *= g;
                }
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) FoldX[wave][e0 + e] = X[e];
            if (lane == 0) FoldG[wave] = Gr;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < EPL; ++e) C[e] = Cin[e];
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int e = 0; e < EPL; ++e) C[e] = FoldG[w] * C[e] + FoldX[w][e0 + e];
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) C[e] = Cin[e];
        }
        if constexpr (kRegC) {
            // (S, C) through the earlier blocks: S = g_w·S + β_w·C + s_w, C += c_w
            float K[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) K[e] = Kin[e];
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                if (w < wave) {
                    const float gw = BlkG[w], bw = BlkB[w];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        C[e] = gw * C[e] + bw * K[e] + BlkAgg[w][e0 + e];
                        K[e] += BlkC[w][e0 + e];
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) Kb[wave][e0 + e] = K[e];
        } else {
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                if (w < wave) {
                    const int s0 = t0 + kBlk * w;
                    const float gl = powi(gm, evict_steps(p0, s0, min(kBlk, n - s0), W));
#pragma unroll
                    for (int e = 0; e < EPL; ++e) C[e] = gl * C[e] + BlkAgg[w][e0 + e];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) Sw[e0 + e] = C[e];
        wave_lds_sync();
        // S_t = A_{..t}·S_start + V_{..t} (running mean: + B_t·C_start)
#pragma unroll
        for (int k = 0; k < D / 32; ++k)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&Sw[32 * k + 8 * q4 + 4 * half]);
                if constexpr (kRegC) {
                    const f32x4 k0 = *reinterpret_cast<const f32x4 *>(&Kb[wave][32 * k + 8 * q4 + 4 * half]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Sreg[k][half][i] = fmaf(Ac, s0[i], fmaf(Bq, k0[i], Sreg[k][half][i]));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) Sreg[k][half][i] = fmaf(Ac, s0[i], Sreg[k][half][i]);
                }
            }
        if constexpr (FUSED || FOLD) {
            // the single pass and the folded form write S after the last token:
            // lanes c16 = 15 of the last wave (tokens past the end leave S unchanged)
            if (tile == a.ntiles - 1 && wave == 3 && c16 == kBlk - 1 && a.state) {
                float *st = a.state + (long)bg * D;
#pragma unroll
                for (int k = 0; k < D / 32; ++k)
#pragma unroll
                    for (int half = 0; half < 2; ++half)
                        *reinterpret_cast<f32x4 *>(st + 32 * k + 8 * q4 + 4 * half) = Sreg[k][half];
            }
        }
    }
    // QH: S tile of query head h (its carry in Cin/Ain) into Sw; the next
    // head's carry loads go out here
    auto head_S = [&](int h) {
        if constexpr (QH) {
            const float gh = load_uniform(a.gamma + (chain0 - (long)b * a.Hq + h));
            float Cx[EPL], Ax[3][EPL], S[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) Cx[e] = Cin[e];
#pragma unroll
            for (int w = 0; w < 3; ++w)
#pragma unroll
                for (int e = 0; e < EPL; ++e) Ax[w][e] = Ain[w][e];
            // unconditional (the last head reloads its own carry), so that the
            // waits for these loads are counted exactly
            carry_loads(chain0 + min(h + 1, group - 1), Cin, Ain);
            block_start(gh, Cx, Ax, S);
#pragma unroll
            for (int j = 0; j < kBlk; ++j) {
                const int t = tb + j;
                if (t < n && p0 + t >= W) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) S[e] = gh * S[e] + (1.f - gh) * kev[j][e];
                }
#pragma unroll
                for (int e = 0; e < EPL; ++e) Sw[j * SS + e0 + e] = S[e];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    };

    // ---- (4) score-validity mask -------------------------------------------------
    // element T*4+i is key (tb-16) + 16T + 4*q4 + i for token tb + c16; key tiles
    // T0 = staged rows 16*wave + [0,16), T1 = 16*wave + 16 + [0,16)
    unsigned mask = 0;
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kr = tb - kMaxWindow + 16 * T + 4 * q4 + i;
            if (kr <= tok && kr > tok - W && p0 + kr >= 0) mask |= 1u << (4 * T + i);
        }
    const float *alpha = a.alpha + (long)G * group;

    if constexpr (kBf16) {
        bf16x8 Kc[2][D / 32];
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int st = 0; st < D / 32; ++st)
                Kc[T][st] = *reinterpret_cast<const bf16x8 *>(
                    &Klds[(kBlk * wave + 16 * T + c16) * KS + 32 * st + 8 * q4]);
        const uint32_t *vt32 = reinterpret_cast<const uint32_t *>(Vt);
        const int vcol = (kBlk * wave + 4 * q4) / 2;   // dword column of keys 4q4.. of T0 (+8: of T1)
        const float *Srow = &Sw[c16 * SS + 8 * q4];     // S of token c16 at d = 32k + 8q4 + e
        // bf16 outputs go through a per-wave [16 tokens][D] tile in the K staging
        // area (free once every wave holds its K operands) so that each store
        // instruction writes 4 whole rows of D bf16
        constexpr bool kTileOut = std::is_same<TOut, __bf16>::value;
        constexpr int OS = D + 8;  // Q / output tile row stride (bf16)
        static_assert(4 * kBlk * OS * 2 <= (int)sizeof(Klds), "output tiles must fit the K area");
        uint16_t *Ot = reinterpret_cast<uint16_t *>(Klds) + wave * kBlk * OS;
        __syncthreads();

        for (int h0 = 0; h0 < group; h0 += kQSlots) {
#pragma unroll
            for (int hh = 0; hh < kQSlots; ++hh) {
                const int h = h0 + hh;
                if (h >= group) continue;  // unrolled: keeps Qc indices static
                head_S(h);
                // row layout -> LDS tile -> B operands (lane: token c16, 8 elements)
#pragma unroll
                for (int j = 0; j < QLD; ++j)
                    *reinterpret_cast<u32x4 *>(&Ot[(rt + TPI * j) * OS + 8 * rc]) = Qc[hh][j];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                bf16x8 Qh[D / 32];
#pragma unroll
                for (int st = 0; st < D / 32; ++st)
                    Qh[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&Ot[c16 * OS + 32 * st + 8 * q4]));
                if (h + kQSlots < group) {  // refill the slot with head h + kQSlots
#pragma unroll
                    for (int j = 0; j < QLD; ++j)
                        if (tb + rt + TPI * j < n)
                            Qc[hh][j] = ld_stream(Qrow + j * qtok_stride + (long)(h + kQSlots) * D);
                }
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
                for (int st = 0; st < D / 32; ++st) {
                    s0 = mfma_bf16_16x16x32(Kc[0][st], Qh[st], s0);
                    s1 = mfma_bf16_16x16x32(Kc[1][st], Qh[st], s1);
                }
                float x[8], m = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = (mask >> i & 1) ? s0[i] * a.scale_log2e : -INFINITY;
                    x[4 + i] = (mask >> (4 + i) & 1) ? s1[i] * a.scale_log2e : -INFINITY;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, x[i]);
                m = max_over_groups(m);
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[i] = (mask >> i & 1) ? __builtin_amdgcn_exp2f(x[i] - m) : 0.f;
                    sum += x[i];
                }
                sum = sum_over_groups(sum);
                const float inv = 1.f / sum;
                bf16x8 Ph, Pl;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __bf16 hi_, lo_;
                    split_bf16(x[i] * inv, hi_, lo_);
                    Ph[i] = hi_;
                    Pl[i] = lo_;
                }
                // (a scalar load: a vector load here would make the wait for it
                // also wait for the query prefetch issued just before)
                const float al = load_uniform(alpha + h);
                // PV in 16-row V^T tiles; row m of tile dt is head-dim element
                // 32(dt/2) + 8(m/4) + 4(dt%2) + m%4, so after tiles 2k and 2k+1
                // lane group q4 holds elements [32k + 8q4, +8) of its token and
                // the four lanes of a token store 64 contiguous bytes
#pragma unroll
                for (int k = 0; k < D / 32; ++k) {
                    float ov[8];
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int drow = 32 * k + 8 * (c16 >> 2) + 4 * half + (c16 & 3);
                        const uint32_t *vr = vt32 + vt_dword(drow, vcol);
                        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr);
                        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 8);
                        const bf16x8 vop = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                        f32x4 o = {0.f, 0.f, 0.f, 0.f};
                        o = mfma_bf16_16x16x32(vop, Ph, o);
                        o = mfma_bf16_16x16x32(vop, Pl, o);
                        f32x4 s4;
                        if constexpr (kRegS) s4 = Sreg[k][half];
                        else s4 = *reinterpret_cast<const f32x4 *>(Srow + 32 * k + 4 * half);
#pragma unroll
                        for (int i = 0; i < 4; ++i) ov[4 * half + i] = fmaf(al, s4[i], o[i]);
                    }
                    if constexpr (kTileOut) {
                        u32x4 w;
#pragma unroll
                        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(ov[2 * i], ov[2 * i + 1]);
                        *reinterpret_cast<u32x4 *>(&Ot[c16 * OS + 32 * k + 8 * q4]) = w;
                    } else {
                        if (tok_ok) store8<TOut>(Otok + (long)h * D + 32 * k + 8 * q4, ov);
                    }
                }
                if constexpr (kTileOut) {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    // lane L: token rt + TPI*j of the block, 16-byte chunk rc
#pragma unroll
                    for (int j = 0; j < kBlk / TPI; ++j) {
                        const int tt = rt + TPI * j;
                        const u32x4 w = *reinterpret_cast<const u32x4 *>(&Ot[tt * OS + 8 * rc]);
                        if (tb + tt < n)
                            st_stream(reinterpret_cast<TOut *>(a.out) +
                                          (((long)b * n + tb + tt) * a.Hq + (long)G * group + h) * D + 8 * rc, w);
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }
    } else {
        float4 Kc[2][D / 16];
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int u = 0; u < D / 16; ++u)
                Kc[T][u] = *reinterpret_cast<const float4 *>(
                    &Klds[(kBlk * wave + 16 * T + c16) * KS + 16 * u + 4 * q4]);
        for (int hh = 0; hh < group; ++hh) {
            head_S(hh);
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
            for (int u = 0; u < D / 16; ++u) {
                float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (tok_ok) qv = *reinterpret_cast<const float4 *>(Qtok + (long)hh * D + 16 * u + 4 * q4);
                s0 = mfma_f32_16x16x4(Kc[0][u].x, qv.x, s0);
                s0 = mfma_f32_16x16x4(Kc[0][u].y, qv.y, s0);
                s0 = mfma_f32_16x16x4(Kc[0][u].z, qv.z, s0);
                s0 = mfma_f32_16x16x4(Kc[0][u].w, qv.w, s0);
                s1 = mfma_f32_16x16x4(Kc[1][u].x, qv.x, s1);
                s1 = mfma_f32_16x16x4(Kc[1][u].y, qv.y, s1);
                s1 = mfma_f32_16x16x4(Kc[1][u].z, qv.z, s1);
                s1 = mfma_f32_16x16x4(Kc[1][u].w, qv.w, s1);
            }
            float x[8], m = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (mask >> i & 1) ? s0[i] * a.scale_log2e : -INFINITY;
                x[4 + i] = (mask >> (4 + i) & 1) ? s1[i] * a.scale_log2e : -INFINITY;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, x[i]);
            m = max_over_groups(m);
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = (mask >> i & 1) ? __builtin_amdgcn_exp2f(x[i] - m) : 0.f;
                sum += x[i];
            }
            sum = sum_over_groups(sum);
            const float inv = 1.f / sum;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] *= inv;
            const float al = load_uniform(alpha + hh);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                // k-step s: lane group q4 supplies key 4*q4 + s of tile s/4
                const float *vr = &Vt[(16 * dt + c16) * VS + kBlk * wave + 4 * q4];
                const float4 v0 = *reinterpret_cast<const float4 *>(vr);
                const float4 v1 = *reinterpret_cast<const float4 *>(vr + 16);
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
                o = mfma_f32_16x16x4(v0.x, x[0], o);
                o = mfma_f32_16x16x4(v0.y, x[1], o);
                o = mfma_f32_16x16x4(v0.z, x[2], o);
                o = mfma_f32_16x16x4(v0.w, x[3], o);
                o = mfma_f32_16x16x4(v1.x, x[4], o);
                o = mfma_f32_16x16x4(v1.y, x[5], o);
                o = mfma_f32_16x16x4(v1.z, x[6], o);
                o = mfma_f32_16x16x4(v1.w, x[7], o);
                const f32x4 s4 = *reinterpret_cast<const f32x4 *>(&Sw[c16 * SS + 16 * dt + 4 * q4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = fmaf(al, s4[i], o[i]);
                if (tok_ok) store4<TOut>(Otok + (long)hh * D + 16 * dt + 4 * q4, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_ring_handoff: last min(W, n) keys/values of a continued call -> ring slots
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void k_ring_handoff(PrefillArgs a) {
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv, G = bg % a.Hkv;
    const int n = a.n, W = a.W, D = a.d;
    const int p0 = max(0, a.pos0[b]);
    const int first = max(0, n - W);
    const long row_stride = (long)a.Hkv * D;
    const TIn *Kbg = reinterpret_cast<const TIn *>(a.k) + ((long)b * n * a.Hkv + G) * D;
    const TIn *Vbg = reinterpret_cast<const TIn *>(a.v) + ((long)b * n * a.Hkv + G) * D;
    TIn *rk = reinterpret_cast<TIn *>(a.ring_k) + (long)bg * W * D;
    TIn *rv = reinterpret_cast<TIn *>(a.ring_v) + (long)bg * W * D;
    const int cnt = (n - first) * D;
    for (int idx = threadIdx.x; idx < cnt; idx += 256) {
        const int t = first + idx / D, e = idx % D;
        const int slot = (p0 + t) % W;
        rk[(long)slot * D + e] = Kbg[(long)t * row_stride + e];
        rv[(long)slot * D + e] = Vbg[(long)t * row_stride + e];
    }
}

template <typename TIn, typename TOut, int D>
hipError_t launch_t(const PrefillArgs &a, hipStream_t stream, int parts) {
    const unsigned tiles = (unsigned)(a.B * a.Hkv * a.ntiles);
    if constexpr (std::is_same<TIn, __bf16>::value) {
        // single pass (requested explicitly; the caller checked the limits)
        if (parts == kPrefillSinglePass) {
            const long words = (long)tiles * D;
            const long init_blocks = (words / 2 + 255) / 256 + ((long)a.B * a.Hkv * D + 255) / 256;
            hipLaunchKernelGGL(k_fused_init, dim3((unsigned)init_blocks), dim3(256), 0, stream, a);
            hipLaunchKernelGGL((k_window_attn<TIn, TOut, D, kKvHead, true>), dim3(tiles), dim3(256), 0, stream, a);
            if (a.pos0 && a.ring_k)
                hipLaunchKernelGGL((k_ring_handoff<TIn>), dim3(a.B * a.Hkv), dim3(256), 0, stream, a);
            return hipGetLastError();
        }
    }
    // folded carries: S per KV head, bf16 inputs, at most kFusedMaxTiles tiles
    PrefillArgs af = a;
    af.fold = std::is_same<TIn, __bf16>::value && !a.s_per_query && !a.running_mean && a.ntiles <= kFusedMaxTiles;
    if (af.fold) {
        if constexpr (std::is_same<TIn, __bf16>::value) {
            if (parts & kPrefillScan)
                hipLaunchKernelGGL((k_ewma_agg<TIn, D, false, false>), dim3((tiles + 3) / 4), dim3(256), 0, stream,
                                   af);
            if (parts & kPrefillAttend) {
                hipLaunchKernelGGL((k_window_attn<TIn, TOut, D, kKvHead, false, true>), dim3(tiles), dim3(256), 0,
                                   stream, af);
                if (a.pos0 && a.ring_k)
                    hipLaunchKernelGGL((k_ring_handoff<TIn>), dim3(a.B * a.Hkv), dim3(256), 0, stream, af);
            }
        }
        return hipGetLastError();
    }
    if (parts & kPrefillScan) {
        // one wave per (tile, b, KV head); per query head it feeds the group's chains
        const unsigned scan_tiles = (unsigned)(a.B * a.Hkv * a.ntiles);
        const dim3 agg_grid((scan_tiles + 3) / 4), carry_grid(a.B * a.Hs * (D / kCarryCols));
        if (a.running_mean) {
            hipLaunchKernelGGL((k_ewma_agg<TIn, D, true, false>), agg_grid, dim3(256), 0, stream, af);
            hipLaunchKernelGGL(k_ewma_carry<true>, carry_grid, dim3(1024), 0, stream, af);
        } else {
            if (a.s_per_query)
                hipLaunchKernelGGL((k_ewma_agg<TIn, D, false, true>), agg_grid, dim3(256), 0, stream, af);
            else
                hipLaunchKernelGGL((k_ewma_agg<TIn, D, false, false>), agg_grid, dim3(256), 0, stream, af);
            hipLaunchKernelGGL(k_ewma_carry<false>, carry_grid, dim3(1024), 0, stream, af);
        }
    }
    if (parts & kPrefillAttend) {
        if (a.s_per_query)
            hipLaunchKernelGGL((k_window_attn<TIn, TOut, D, kQueryHead>), dim3(tiles), dim3(256), 0, stream, af);
        else if (a.running_mean)
            hipLaunchKernelGGL((k_window_attn<TIn, TOut, D, kRunningMean>), dim3(tiles), dim3(256), 0, stream, af);
        else
            hipLaunchKernelGGL((k_window_attn<TIn, TOut, D, kKvHead>), dim3(tiles), dim3(256), 0, stream, af);
        if (a.pos0 && a.ring_k)
            hipLaunchKernelGGL((k_ring_handoff<TIn>), dim3(a.B * a.Hkv), dim3(256), 0, stream, af);
    }
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_d(const PrefillArgs &a, hipStream_t stream, int parts) {
    return a.d == 128 ? launch_t<TIn, TOut, 128>(a, stream, parts)
                      : launch_t<TIn, TOut, 64>(a, stream, parts);
}

}  // namespace

size_t prefill_workspace_bytes(int B, int n, int Hkv, int d) {
    const size_t nt = ((size_t)n + kTile - 1) / kTile;
    return (size_t)B * Hkv * nt * d * sizeof(float) * 6;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream, int parts) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_d<__bf16, __bf16>(a, stream, parts)
                          : launch_d<__bf16, float>(a, stream, parts);
    return a.out_bf16 ? launch_d<float, __bf16>(a, stream, parts) : launch_d<float, float>(a, stream, parts);
}

}  // namespace sfa
