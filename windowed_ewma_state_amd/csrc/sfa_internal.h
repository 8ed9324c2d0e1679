// sfa_internal.h -- launch interfaces between the C ABI (sfa_api.cpp) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sfa {

// far-field variants of the prefill and decode kernels
constexpr int kKvHead = 0;       // S and γ per KV head, one evicted key per step (the main reading)
constexpr int kQueryHead = 1;    // S and γ per query head
constexpr int kRunningMean = 2;  // per KV head; EWMA input = mean of every key that has left the window

struct DecodeArgs {
    const void *q, *k_new, *v_new;
    void *ring_k, *ring_v;
    float *state;
    const int32_t *pos;
    const float *gamma, *alpha;
    void *out;
    int L, B, Hq, Hkv, d, W, group;
    float scale_log2e;
    int in_bf16, out_bf16;
    int s_per_query;   // S and γ per query head ([L,B,Hq,d], [L,Hq]) instead of per KV head
    int running_mean;  // state [L,B,Hkv,2,d]: S, then the mean of the keys that have left the window
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// prefill tiling: 64-token tiles, four 16-token wave blocks per tile
constexpr int kTile = 64;
constexpr int kBlk = 16;

struct PrefillArgs {
    const void *q, *k, *v;
    const float *gamma, *alpha;
    void *out;
    void *ring_k, *ring_v;
    float *state;
    const int32_t *pos0;
    int B, n, Hq, Hkv, d, W, group, ntiles;
    float scale_log2e;
    int in_bf16, out_bf16;
    // far-field heads: Hs = Hkv (S and γ per KV head) or Hq (per query head,
    // s_per_query = 1); the scan runs over B*Hs chains
    int Hs, s_per_query;
    // running mean (state [B,Hkv,2,d]): the EWMA input at p >= W is C/m, C the
    // sum of the m = p-W+1 keys that have left the window
    int running_mean;
    // workspace carve-up (fp32)
    float *agg16;  // [B*Hs][ntiles][4][d]  local EWMA aggregate of each 16-token block
    float *agg64;  // [B*Hs][ntiles][d]     local EWMA aggregate of each 64-token tile
    float *carry;  // [B*Hs][ntiles][d]     S just before each tile
    // running mean only: the same for the key sum C, and per tile the
    // coefficient of the incoming C in the tile's outgoing S
    float *csum16, *csum64, *ccarry;  // as agg16, agg64, carry
    float *beta64;                    // [B*Hs][ntiles]
    // single-pass form (S per KV head, bf16 inputs, at most kFusedMaxTiles tiles
    // per sequence): every attention workgroup publishes its tile's EWMA
    // aggregate as tagged words and folds those of the tiles before it
    uint64_t *tagged;  // [B*Hkv][ntiles][d]  (fp32 bits, tag in the high word)
    float *sinit;      // [B*Hkv][d]          S carried into the call (0 for a fresh sequence)
    // folded carries (S per KV head, bf16 inputs, at most kFusedMaxTiles tiles):
    // the scan writes the tile aggregates and, as the first tile's carry, S
    // before the call; each attention workgroup folds the earlier tiles'
    // aggregates onto it (no carry launch) and the last tile writes the final S
    int fold;
};
constexpr int kFusedMaxTiles = 64;
size_t prefill_workspace_bytes(int B, int n, int Hkv, int d);
constexpr int kPrefillScan = 1, kPrefillAttend = 2, kPrefillSinglePass = 4;
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream, int parts);

struct EnhanceArgs {
    const void *attn;
    void *out;
    float *ring, *field;
    const float *pool;
    long long pool_stride;
    float *enhancement;
    int L, layer0, n_layers, T, H, t0, R, n_slots, ntiles, n_pool_layers;
    float alpha_base, cross_decay, ema_gamma, inv_temp_log2e, clip;
    int in_bf16, out_bf16;
    // prepared pool: one record of pool_rec_bytes per pool layer (in the
    // workspace when the call prepares it, else the caller's buffer):
    //   floats [0, 64)     1 / |slot|
    //   floats [64, 128)   max_x |slot[x]| of each slot
    //   bytes  [1024, ..)  poolA [H/32][4][2][64][8] bf16 hi/lo, cosine operand,
    //                      then poolT [H/16][2][2][64][8] bf16 hi/lo, semantic operand
    unsigned char *pool_rec;
    long long pool_rec_bytes;
    int prepare_pool;       // the call prepares the records (sfa_enhance) or finds them ready
    // workspace carve-up
    float *agg64;           // [L][ntiles][H]   EMA of each 64-token tile from zero
    float *carry;           // [L][ntiles][H]   field just before each tile
    float *halo;            // [L][R][H]        the carried ring, read before the ring is rewritten
    uint16_t *wsem;         // [L][ntiles][4][2][2][64][8] bf16 hi/lo of 0.5·(slot weights)
    uint16_t *coef;         // [8 x 2][64][8] band/field operands
    float *alpha_tab;       // [L] α of each layer of the call
};
constexpr int kPoolRecHeader = 1024;  // bytes before the operands in a pool record
__host__ __device__ constexpr long long pool_rec_bytes(int H) { return kPoolRecHeader + 512LL * H; }
// workspace bytes of a call: with n_pool_layers > 0 the call also prepares that
// many pool records in the workspace
size_t enhance_workspace_bytes(int L, int T, int H, int n_pool_layers);
hipError_t launch_enhance(const EnhanceArgs &a, hipStream_t stream);
hipError_t launch_pool_prepare(const EnhanceArgs &a, hipStream_t stream);

// the decode step fused with the triple-channel enhancement of each
// (layer, sequence)'s attention row (hidden H = Hq·d)
struct DecodeEnhanceArgs {
    DecodeArgs d;            // the decode step (its out is not used)
    void *out;               // [L,B,H] out_dtype: a + α_l·clip(e)
    float *ring;             // [L,B,R,H] the last R attention rows of the sequence (slot pos mod R)
    float *field;            // [L,B,H]
    float *enhancement;      // [L,B,H] α_l·clip(e), or null
    const unsigned char *pool_rec;  // prepared pool records (1/|s| and the bf16 hi/lo operand tables)
    long long pool_rec_bytes;       // stride between layers' records (0: one shared record)
    int H, R, n_slots, layer0, n_layers;
    float alpha_base, cross_decay, ema_gamma, inv_temp_log2e, clip;
};
hipError_t launch_decode_enhance(const DecodeEnhanceArgs &a, hipStream_t stream);

// XCD-aware block remap: consecutive logical indices land on the same XCD
// (hardware dispatches workgroups round-robin over the 8 XCDs of an MI355X).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    constexpr int kXcd = 8;
    const int xcd = bid % kXcd;
    const int idx = bid / kXcd;
    const int per = nblk / kXcd;
    const int rem = nblk % kXcd;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// γ^k for small non-negative integer k (exponentiation by squaring, fp32)
__device__ __forceinline__ float powi(float g, int k) {
    float r = 1.0f;
    while (k > 0) {
        if (k & 1) r *= g;
        g *= g;
        k >>= 1;
    }
    return r;
}

}  // namespace sfa
