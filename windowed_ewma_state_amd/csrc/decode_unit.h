// decode_unit.h -- one (layer, sequence, KV head) unit of the SFA decode step
// on gfx950: its loads (row-shaped, issued ahead of use) and its compute
// (ring update, eviction into S, scores and PV on MFMA, α·S epilogue).  Used
// by the batched decode kernel and by the decode step fused with the
// triple-channel enhancement.
//
// Page "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩",
// section 2.1 (near field over the last k tokens, far-field EWMA of the keys
// that leave the window, O = O_near + α·S) and section 2.2 (the k-slot ring).
#pragma once

#include <type_traits>

#include "sfa_common.h"
#include "sfa_internal.h"

namespace sfa {

namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Every global load of a unit is row-shaped: CPR consecutive lanes read one
// whole row (16 bytes each), so an instruction moves RPI complete rows.  On
// this memory system whole-row requests stream markedly faster than the
// MFMA operand shape (16 rows x 64 bytes per instruction); the operands are
// formed from a per-wave LDS tile instead.  The ring rows are read as they
// are (the new key/value is put into slot pos mod W in LDS), so every
// lane's load offsets are the same for all units and only the scalar bases
// change.
template <int D, int QN>
struct UnitLoads {
    static constexpr int EPL = D / kWave;
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int RPI = kWave / CPR;          // whole rows per load instruction (4 or 8)
    static constexpr int NI = kMaxWindow / RPI;      // instructions per 16 rows (4 or 2)
    // QN query instructions cover QN * RPI heads: half the register space
    // when the group has at most 8 heads
    u32x4 k[NI], q[QN], v[NI];
    float S[EPL], M[EPL];  // S (and with the running mean, M) of the unit
    uint32_t kn, vn;  // this lane's head-dim elements of k_new / v_new (raw bits)
    float gm;         // γ of the unit's S (per query head: of head c16)
    float al;         // α of head c16 (0 past the group)
    int p;            // the sequence's position
};

// `live` false: the loop's last prefetch, issued anyway (see k_decode_mfma)
// with every lane of an instruction at one 16-byte chunk of the unit.
template <int D, int QN, int MODE>
__device__ __forceinline__ void unit_load(const DecodeArgs &a, int unit, UnitLoads<D, QN> &u, int lane, bool live) {
    constexpr bool QH = MODE == kQueryHead, RM = MODE == kRunningMean;
    using U = UnitLoads<D, QN>;
    constexpr int EPL = D / kWave;
    const int G = unit % a.Hkv;
    const int lb = unit / a.Hkv;
    const int b = lb % a.B;
    const int W = a.W, group = a.group;
    // No load here depends on the position, and every small value the step
    // needs (position, γ, α) is loaded with the unit: the counter of
    // outstanding loads drains in issue order, so a load issued during the
    // previous unit's compute would make that compute wait for this whole
    // prefetch.
    u.p = load_uniform(a.pos + b);
    const int l = lb / a.B;
    const int c16 = lane & 15;
    const int hc = live && c16 < group ? c16 : group - 1;
    u.gm = QH ? a.gamma[(long)l * a.Hq + (long)G * group + hc] : load_uniform(a.gamma + (long)l * a.Hkv + G);
    u.al = a.alpha[(long)l * a.Hq + (long)G * group + hc];
    const __bf16 *ringK = reinterpret_cast<const __bf16 *>(a.ring_k) + (long)unit * W * D;
    const __bf16 *ringV = reinterpret_cast<const __bf16 *>(a.ring_v) + (long)unit * W * D;
    const __bf16 *kn = reinterpret_cast<const __bf16 *>(a.k_new) + (long)unit * D;
    const __bf16 *vn = reinterpret_cast<const __bf16 *>(a.v_new) + (long)unit * D;
    const __bf16 *qg = reinterpret_cast<const __bf16 *>(a.q) + ((long)lb * a.Hq + G * group) * D;
    const int rj = lane / U::CPR, rc = lane % U::CPR;
    // K rows RPI*i + rj and V rows NI*rj + i (each lane then holds NI
    // consecutive slots of V, which pair up into the dwords of the V^T tile);
    // rows past a ring shorter than 16 repeat its last row.  Q rows = heads
    // RPI*i + rj, as many instructions as the group needs, heads past the
    // group repeating the last one (the step computes and stores that head's
    // output for them once more, bit for bit the same).  Every load is
    // issued, whatever the group size, so the number of loads in flight is a
    // compile-time constant.  (32-bit byte offsets from the unit's scalar bases)
    constexpr uint32_t RB = D * sizeof(__bf16);
    const uint32_t lm = live ? ~0u : 0u;
#pragma unroll
    for (int i = 0; i < U::NI; ++i) {
        const uint32_t ok = ((uint32_t)min(U::RPI * i + rj, W - 1) * RB + 16u * rc) & lm;
        const uint32_t ov = ((uint32_t)min(U::NI * rj + i, W - 1) * RB + 16u * rc) & lm;
        const uint32_t oq = ((uint32_t)min(U::RPI * i + rj, group - 1) * RB + 16u * rc) & lm;
        u.k[i] = ld_stream(reinterpret_cast<const char *>(ringK) + ok);
        u.v[i] = ld_stream(reinterpret_cast<const char *>(ringV) + ov);
        if (i < QN) u.q[i] = ld_stream(reinterpret_cast<const char *>(qg) + oq);
    }
    // far-field state, new key/value (e-pair layout: lane owns d = EPL*lane ..)
    const int e0 = live ? lane * EPL : 0;
    if constexpr (!QH) {  // (per query head, the compute step reads its heads' S)
        const float *S_ptr = a.state + (long)unit * (RM ? 2 * D : D) + e0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) u.S[e] = S_ptr[e];
        if constexpr (RM) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) u.M[e] = S_ptr[D + e];
        }
    }
    if (EPL == 2) {
        u.kn = *reinterpret_cast<const uint32_t *>(kn + e0);
        u.vn = *reinterpret_cast<const uint32_t *>(vn + e0);
    } else {
        u.kn = *reinterpret_cast<const uint16_t *>(kn + e0);
        u.vn = *reinterpret_cast<const uint16_t *>(vn + e0);
    }
}

// Per query head, the S rows of the unit's heads in the epilogue layout (lane
// (q4, c16): head c16 at d = 32k + 8q4 + 4half + i), loaded just before the
// next unit's prefetch.
template <int D, bool QH> struct LateLoads { f32x4 Sq[QH ? D / 32 : 1][2]; };

template <int D, bool QH>
__device__ __forceinline__ void late_load(const DecodeArgs &a, int unit, LateLoads<D, QH> &L, int lane) {
    if constexpr (QH) {
        const int q4 = lane >> 4, c16 = lane & 15;
        const int G = unit % a.Hkv, lb = unit / a.Hkv;
        const int hc = c16 < a.group ? c16 : a.group - 1;
        const float *Sg = a.state + ((long)lb * a.Hq + (long)G * a.group + hc) * D + 8 * q4;
#pragma unroll
        for (int k = 0; k < D / 32; ++k)
#pragma unroll
            for (int half = 0; half < 2; ++half)
                L.Sq[k][half] = *reinterpret_cast<const f32x4 *>(Sg + 32 * k + 4 * half);
    }
}

// Target of the stores of a unit whose position is negative (it must be left
// untouched): the store is issued all the same, 16 bytes per lane.
__device__ __attribute__((aligned(256))) uint32_t g_decode_sink[kWave * 4];

// each lane takes the four dwords of the lane 8 away within its 16-lane row
__device__ __forceinline__ u32x4 row_ror8(u32x4 v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[i], 0x128, 0xf, 0xf, true);
    return r;
}

template <typename T>
__device__ __forceinline__ T *sink_or(T *p, bool skip, int lane) {
    return skip ? reinterpret_cast<T *>(g_decode_sink + 4 * lane) : p;
}

// ToLds: instead of storing the outputs, write them as fp32 into `arow`, the
// unit's sequence's hidden row in LDS (head h of the unit's group at
// columns [(G·group + h)·D, +D)); for the fused enhancement.
template <typename TOut, int D, int QN, int MODE, bool ToLds = false>
__device__ __forceinline__ void unit_compute(const DecodeArgs &a, int unit, const UnitLoads<D, QN> &u,
                                             const LateLoads<D, MODE == kQueryHead> &late, int lane,
                                             __bf16 *vt, float *sl, __bf16 *kqt, float *arow = nullptr) {
    constexpr bool QH = MODE == kQueryHead, RM = MODE == kRunningMean;
    constexpr int EPL = D / kWave;
    constexpr int VTS = kMaxWindow + 4;
    const int q4 = lane >> 4, c16 = lane & 15;
    const int W = a.W, group = a.group;
    const int e0 = lane * EPL;
    // A negative position leaves the unit untouched: the step runs as for
    // position 0 and every store of it goes to the sink.
    const bool skip = u.p < 0;
    const int p = skip ? 0 : u.p;
    {
        const int G = unit % a.Hkv;
        const int lb = unit / a.Hkv;
        const int s = p % W;
        const int nvalid = (p >= W - 1) ? W : p + 1;
        using U = UnitLoads<D, QN>;
        constexpr int KS = D + 8;  // K/Q tile row stride (bf16): an operand read's 16 rows hit distinct banks
        const int rj = lane / U::CPR, rc = lane % U::CPR;
        // (a) ring K rows into the wave's tile and V into the V^T tile (row =
        // head-dim element, 16 slots = 8 dwords per row; the lane's NI
        // consecutive slots pair up into dword columns).  Slots past the valid
        // ones hold whatever the ring holds: their K scores are masked, their
        // V rows are zeroed (a probability of exactly 0 must meet finite data).
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
            *reinterpret_cast<u32x4 *>(&kqt[(U::RPI * i + rj) * KS + 8 * rc]) = u.k[i];
        u32x4 vr[U::NI];
#pragma unroll
        for (int i = 0; i < U::NI; ++i) vr[i] = u.v[i];
        if (nvalid < kMaxWindow) {
#pragma unroll
            for (int i = 0; i < U::NI; ++i)
                if (U::NI * rj + i >= nvalid) vr[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int pp = 0; pp < U::NI / 2; ++pp) {
            const int col = U::NI / 2 * rj + pp;
            const u32x4 va = vr[2 * pp], vb = vr[2 * pp + 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = (va[i] & 0xffffu) | (vb[i] << 16);
                const uint32_t hi = (va[i] >> 16) | (vb[i] & 0xffff0000u);
                *reinterpret_cast<uint32_t *>(&vt[(8 * rc + 2 * i) * VTS + 2 * col]) = lo;
                *reinterpret_cast<uint32_t *>(&vt[(8 * rc + 2 * i + 1) * VTS + 2 * col]) = hi;
            }
        }
        wave_lds_sync();
        // (b) the key of position p-W (ring slot s) leaves the window: read it
        // from the tile before the new key takes its slot
        const uint16_t *krow_s = reinterpret_cast<const uint16_t *>(kqt) + s * KS;
        float kev[EPL];
        if constexpr (EPL == 2) {
            const uint32_t kw = *reinterpret_cast<const uint32_t *>(krow_s + e0);
            kev[0] = bf16_lo(kw);
            kev[EPL - 1] = bf16_hi(kw);
        } else {
            kev[0] = bf16_bits_to_f32(krow_s[e0]);
        }
        float S[EPL], M[EPL];
        if constexpr (!QH) {
            const float gm = u.gm;
            if constexpr (RM) {  // the key joins the mean of the p-W keys that left before it
                const float mf = (float)(p - W + 1);
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    M[e] = (p >= W) ? u.M[e] + (kev[e] - u.M[e]) / mf : u.M[e];
                    S[e] = (p >= W) ? gm * u.S[e] + (1.f - gm) * M[e] : u.S[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) S[e] = (p >= W) ? gm * u.S[e] + (1.f - gm) * kev[e] : u.S[e];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) sl[e0 + e] = S[e];
        }
        // per query head: lane (q4, c16) reads the S of head c16 and the evicted
        // key at its own epilogue positions d = 32k + 8q4 + 4half + i
        const int hc = c16 < group ? c16 : group - 1;
        f32x4 Sq[QH ? D / 32 : 1][2];
        u32x2 kq[QH ? D / 32 : 1][2];
        float gq = 0.f;
        if constexpr (QH) {
#pragma unroll
            for (int k = 0; k < D / 32; ++k)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    Sq[k][half] = late.Sq[k][half];
                    kq[k][half] = *reinterpret_cast<const u32x2 *>(krow_s + 32 * k + 8 * q4 + 4 * half);
                }
            gq = u.gm;
        }
        wave_lds_sync();
        // (c) the new key and value into slot s
        if constexpr (EPL == 2) {
            *reinterpret_cast<uint32_t *>(&kqt[s * KS + e0]) = u.kn;
            reinterpret_cast<uint16_t *>(vt)[e0 * VTS + s] = (uint16_t)(u.vn & 0xffffu);
            reinterpret_cast<uint16_t *>(vt)[(e0 + 1) * VTS + s] = (uint16_t)(u.vn >> 16);
        } else {
            reinterpret_cast<uint16_t *>(kqt)[s * KS + e0] = (uint16_t)u.kn;
            reinterpret_cast<uint16_t *>(vt)[e0 * VTS + s] = (uint16_t)u.vn;
        }
        wave_lds_sync();
        // (d) A operands (row = slot c16, 8 head-dim elements at 32 st + 8 q4),
        // then the same tile takes the queries (row = head = B operand column)
        bf16x8 kop[D / 32], qop[D / 32];
#pragma unroll
        for (int st = 0; st < D / 32; ++st)
            kop[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&kqt[c16 * KS + 32 * st + 8 * q4]));
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < QN; ++i)
            if (U::RPI * i < group)
                *reinterpret_cast<u32x4 *>(&kqt[(U::RPI * i + rj) * KS + 8 * rc]) = u.q[i];
        wave_lds_sync();
        const int hr = c16 < group ? c16 : group - 1;
#pragma unroll
        for (int st = 0; st < D / 32; ++st)
            qop[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&kqt[hr * KS + 32 * st + 8 * q4]));
        // scores and softmax over the valid slots
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < D / 32; ++st) sc = mfma_bf16_16x16x32(kop[st], qop[st], sc);
        float x[4], mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (4 * q4 + i < nvalid) ? sc[i] * a.scale_log2e : -INFINITY;
            mx = fmaxf(mx, x[i]);
        }
        mx = max_over_groups(mx);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (4 * q4 + i < nvalid) ? __builtin_amdgcn_exp2f(x[i] - mx) : 0.f;
            sum += x[i];
        }
        const float inv = 1.f / sum_over_groups(sum);
        bf16x4_t Ph, Pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __bf16 h, lo_;
            split_bf16(x[i] * inv, h, lo_);
            Ph[i] = h;
            Pl[i] = lo_;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        const float al = u.al;
        TOut *orow = reinterpret_cast<TOut *>(a.out) + ((long)lb * a.Hq + G * group + hc) * D;
        // up to 8 heads: lanes c16 >= 8 (duplicates otherwise) take over the next
        // k-step (bf16) or the upper half (fp32) of head c16 - 8, rotated over by
        // 8 lanes, so every store covers whole 128-byte lines of the output rows
        constexpr bool kPairStore = QN * UnitLoads<D, QN>::RPI <= 8;
        const bool upper = c16 >= 8;
        TOut *orow2 = reinterpret_cast<TOut *>(a.out) +
                      ((long)lb * a.Hq + G * group + min(c16 & 7, group - 1)) * D;
        [[maybe_unused]] u32x4 wprev;  // bf16: the packed outputs of the even k-step
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
            float ov[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int drow = 32 * k + 8 * (c16 >> 2) + 4 * half + (c16 & 3);
                const bf16x4_t vop = __builtin_bit_cast(bf16x4_t, *reinterpret_cast<const u32x2 *>(&vt[drow * VTS + 4 * q4]));
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
                o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, Ph, o, 0, 0, 0);
                o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, Pl, o, 0, 0, 0);
                f32x4 s4;
                if constexpr (QH) {
                    s4 = Sq[k][half];
                    if (p >= W) {
                        const u32x2 kw = kq[k][half];
                        const float kv[4] = {bf16_lo(kw[0]), bf16_hi(kw[0]), bf16_lo(kw[1]), bf16_hi(kw[1])};
#pragma unroll
                        for (int i = 0; i < 4; ++i) s4[i] = gq * s4[i] + (1.f - gq) * kv[i];
                    }
                    Sq[k][half] = s4;
                } else {
                    s4 = *reinterpret_cast<const f32x4 *>(&sl[32 * k + 8 * q4 + 4 * half]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[4 * half + i] = fmaf(al, s4[i], o[i]);
            }
            if constexpr (ToLds) {
                if (c16 < group) {
                    float *dst = arow + (G * group + c16) * D + 32 * k + 8 * q4;
                    *reinterpret_cast<f32x4 *>(dst) = f32x4{ov[0], ov[1], ov[2], ov[3]};
                    *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{ov[4], ov[5], ov[6], ov[7]};
                }
            } else if constexpr (kPairStore && std::is_same<TOut, float>::value) {
                u32x4 lo4, hi4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo4[i] = __float_as_uint(ov[i]);
                    hi4[i] = __float_as_uint(ov[4 + i]);
                }
                const u32x4 r = row_ror8(hi4);
                *sink_or(reinterpret_cast<u32x4 *>(orow2 + 32 * k + 8 * q4 + (upper ? 4 : 0)), skip, lane) =
                    upper ? r : lo4;
            } else if constexpr (kPairStore) {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(ov[2 * i], ov[2 * i + 1]);
                if (k & 1) {
                    const u32x4 r = row_ror8(w);
                    st_stream(sink_or(reinterpret_cast<u32x4 *>(orow2 + 32 * (upper ? k : k - 1) + 8 * q4), skip, lane),
                              upper ? r : wprev);
                } else {
                    wprev = w;
                }
            } else if constexpr (std::is_same<TOut, float>::value) {
                *sink_or(reinterpret_cast<float4 *>(orow + 32 * k + 8 * q4), skip, lane) = make_float4(ov[0], ov[1], ov[2], ov[3]);
                *sink_or(reinterpret_cast<float4 *>(orow + 32 * k + 8 * q4 + 4), skip, lane) = make_float4(ov[4], ov[5], ov[6], ov[7]);
            } else {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(ov[2 * i], ov[2 * i + 1]);
                st_stream(sink_or(reinterpret_cast<u32x4 *>(orow + 32 * k + 8 * q4), skip, lane), w);
            }
        }
        // cache update (every read of this unit's ring is done)
        if constexpr (QH) {
            float *Sg = a.state + ((long)lb * a.Hq + (long)G * group + hc) * D + 8 * q4;
#pragma unroll
            for (int k = 0; k < D / 32; ++k)
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    *sink_or(reinterpret_cast<f32x4 *>(Sg + 32 * k + 4 * half), skip, lane) = Sq[k][half];
        } else {
            float *S_ptr = a.state + (long)unit * (RM ? 2 * D : D) + e0;
            if constexpr (EPL == 2) {
                *sink_or(reinterpret_cast<float2 *>(S_ptr), skip, lane) = make_float2(S[0], S[EPL - 1]);
                if constexpr (RM)
                    *sink_or(reinterpret_cast<float2 *>(S_ptr + D), skip, lane) = make_float2(M[0], M[EPL - 1]);
            } else {
                *sink_or(S_ptr, skip, lane) = S[0];
                if constexpr (RM) *sink_or(S_ptr + D, skip, lane) = M[0];
            }
        }
        __bf16 *ringK = sink_or(reinterpret_cast<__bf16 *>(a.ring_k) + ((long)unit * W + s) * D + e0, skip, lane);
        __bf16 *ringV = sink_or(reinterpret_cast<__bf16 *>(a.ring_v) + ((long)unit * W + s) * D + e0, skip, lane);
        if constexpr (EPL == 2) {
            *reinterpret_cast<uint32_t *>(ringK) = u.kn;
            *reinterpret_cast<uint32_t *>(ringV) = u.vn;
        } else {
            *reinterpret_cast<uint16_t *>(ringK) = (uint16_t)u.kn;
            *reinterpret_cast<uint16_t *>(ringV) = (uint16_t)u.vn;
        }
        __builtin_amdgcn_wave_barrier();
    }
}


}  // namespace

}  // namespace sfa
