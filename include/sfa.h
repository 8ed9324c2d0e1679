/*
 * sfa.h -- C ABI of the MI355X (gfx950) Signal Field Attention library, libsfa.so.
 *
 * Signal Field Attention (SFA) is a dual-channel attention:
 *   near field  O_near = softmax(q_t · K_near^T / sqrt(d)) · V_near over the most
 *               recent W (= k = 16) tokens, the current one included;
 *   far field   S_t = γ·S_{t-1} + (1-γ)·k_evicted, where k_evicted is the key that
 *               leaves the window at step t (the key of position t-W);
 *   fusion      O = O_near + α·S_t.
 * Source (the "first page" of the comments below): page
 * "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩",
 * section 2.1 (near-field, far-field and fusion equations) and section 2.2
 * (k = 16, constant O(k·d) memory).  The optional triple-channel enhancement
 * follows page "Dalin Soma SFA基于信号场注意力机制的神经网络推理加速框架"
 * sections 2.1-2.2 and the SFA_Config defaults of page "Signal Field Attention
 * (SFA)" (project README).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees, copies to the host or synchronises.  Work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream) and is
 *    asynchronous: results are valid once the stream reaches that point.
 *  - Layouts are dense and row-major.  "BNHD" = [batch, tokens, heads, head_dim]
 *    (the layout a fused QKV projection emits).
 *  - Every tensor pointer and the workspace must be 16-byte aligned (the
 *    kernels move 16-byte pieces); a misaligned one returns
 *    SFA_ERR_INVALID_ARG.
 *  - Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 *  - S (the far-field state) is one fp32 d-vector per KV head; γ is per KV head,
 *    α per query head.
 *  - Ring cache: W slots per (layer, sequence, KV head); the key/value of
 *    position p lives in slot p mod W.
 *  - dtype codes: SFA_F32 (IEEE fp32) or SFA_BF16 (bfloat16).  in_dtype applies
 *    to q/k/v, the ring and the attention input; out_dtype to the outputs.
 *    Arithmetic is fp32 (bf16 MFMA products with fp32 accumulation, exact for
 *    bf16 operands; fp32 inputs use fp32 MFMA).
 *  - Errors: arguments are validated before anything is enqueued.  A NULL
 *    required pointer, a negative or inconsistent size, Hq % Hkv != 0,
 *    window outside [1,16] or a too-small workspace returns
 *    SFA_ERR_INVALID_ARG; head_dim other than 64/128 or an unknown dtype
 *    returns SFA_ERR_UNSUPPORTED; a failed kernel launch returns SFA_ERR_HIP.
 *    Sizes past the kernels' 32-bit tile and workgroup numbering also return
 *    SFA_ERR_INVALID_ARG: prefill needs n <= 2^31 - 64 and
 *    4 * B * Hs * ceil(n/64) < 2^31 (Hs: KV heads, query heads for the
 *    per-query-head variant); decode needs 64 * L * B * Hkv < 2^31 and
 *    128 * L * B * Hq < 2^31; the enhancement needs T <= 2^31 - 64 and
 *    L * ceil(T/64) * ceil(H/128) < 2^31.
 *    On any error nothing has been written.  Zero-sized work (n == 0, B == 0,
 *    T == 0, L == 0) returns SFA_OK and enqueues nothing.
 *  - Thread safety: the library's global state is a per-device cache of how
 *    many decode workgroups the device holds at once (an atomic, written once
 *    per device with the value the runtime reports), a 1 KB device array that
 *    the stores of skipped decode sequences go to (never read back) and, for
 *    sfa_prefill_noalloc only, a static scratch array per device with a cache
 *    of its address.  Concurrent calls are safe as long as they do not share
 *    output, state or workspace buffers, and no two sfa_prefill_noalloc calls
 *    overlap on one GPU.
 */
#ifndef SFA_H
#define SFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SFA_OK = 0,
    SFA_ERR_INVALID_ARG = 1,
    SFA_ERR_UNSUPPORTED = 2,
    SFA_ERR_HIP = 3,
    SFA_ERR_TOO_LARGE = 4 /* sfa_prefill_noalloc: the call needs more than its static scratch */
};

enum { SFA_F32 = 0, SFA_BF16 = 1 };

/* Largest window (ring slots) supported: the k = 16 of the near field. */
#define SFA_MAX_WINDOW 16

/* Human-readable name of a status code (static storage, never NULL). */
const char *sfa_status_string(int status);

/* Library ABI version (incremented on any signature change). */
int sfa_abi_version(void);

/*
 * Workspace bytes sfa_prefill needs for (B, n, Hkv, d): the chunked EWMA scan
 * keeps fp32 per-chunk aggregates and carries, proportional to B·Hkv·ceil(n/64)·d.
 * Returns 0 for zero-sized work.  The workspace must be 16-byte aligned.
 */
size_t sfa_prefill_workspace_size(int B, int n, int Hkv, int d);

/*
 * sfa_prefill -- near-field windowed attention + far-field EWMA over a prompt.
 * (Near-field, far-field and fusion equations of the first page, section 2.1.)
 *
 * For every batch b, query head h (KV head G = h / (Hq/Hkv)) and token t with
 * position p = p0[b] + t (p0 = pos0[b], or 0 when pos0 is NULL):
 *   if p >= W:  S <- γ[G]·S + (1-γ[G])·key(p-W)         (the key leaving the window)
 *   O[b,t,h] = Σ_{j=max(0,p-W+1)}^{p} softmax_j(scale·<q, key(j)>)·value(j) + α[h]·S
 * S starts at 0 for a fresh sequence (pos0 NULL or pos0[b] == 0) and at
 * state[b,G] otherwise.  key/value(j) for j < p0 come from the ring.
 *
 *  q        [B,n,Hq,d]  in_dtype, BNHD.
 *  k, v     [B,n,Hkv,d] in_dtype, BNHD.
 *  gamma    [Hkv] fp32, decay of each KV head's far field, in [0,1].
 *  alpha    [Hq]  fp32, far-field mixing coefficient of each query head.
 *  out      [B,n,Hq,d]  out_dtype (written).
 *  ring_k, ring_v [B,Hkv,W,d] in_dtype.  On return slot p mod W holds the
 *           key/value of position p for the last min(W, p0+n) positions;
 *           slots of older positions are left untouched.  With pos0 != NULL
 *           they are also read (positions p0-W..p0-1).  May both be NULL only
 *           when pos0 is NULL (then the ring is not produced).
 *  state    [B,Hkv,d] fp32: S after the last token (written).  With
 *           pos0 != NULL it is read first as the carried S.  May be NULL
 *           only when pos0 is NULL.
 *  pos0     [B] int32 device array or NULL: position of each sequence's first
 *           token in this call (chunked prefill / continuation).  Read-only;
 *           negative entries are treated as 0.
 *  window   W in [1,16]; scale <= 0 selects 1/sqrt(d).
 *  workspace, workspace_bytes: device scratch of at least
 *           sfa_prefill_workspace_size(B, n, Hkv, d) bytes, 16-byte aligned.
 */
int sfa_prefill(const void *q, const void *k, const void *v,
                const float *gamma, const float *alpha,
                void *out, void *ring_k, void *ring_v, float *state,
                const int32_t *pos0,
                int B, int n, int Hq, int Hkv, int d, int window, float scale,
                int in_dtype, int out_dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * sfa_prefill_part -- the two phases of sfa_prefill, for callers that schedule
 * or time them separately (same arguments as sfa_prefill, plus `parts`).
 *   SFA_PREFILL_SCAN    far-field EWMA scan: per-chunk aggregates and the S
 *                       carried into every 64-token chunk (into the
 *                       workspace), and the final S into `state`.
 *   SFA_PREFILL_ATTEND  windowed attention + α·S epilogue for every token
 *                       (reads the carries from the workspace), and the ring
 *                       hand-off.  Must run after SCAN with the same arguments
 *                       and workspace, on the same stream (or ordered after it).
 *   With bf16 inputs, S per KV head and at most 64 chunks per sequence the
 *   carries are folded instead: SCAN writes the chunk aggregates and the S
 *   before the call, and ATTEND composes each chunk's carry from them and
 *   writes the final S into `state` (one launch fewer, same results).
 * parts = SCAN | ATTEND is exactly sfa_prefill.
 *   SFA_PREFILL_SINGLE_PASS  the whole call in one pass over the inputs (no
 *                       scan launches, K read once): every attention
 *                       workgroup forms its 64-token chunk's EWMA aggregate
 *                       from its own keys, publishes it in the workspace, and
 *                       folds those of the chunks before it onto the carried S
 *                       (first page, section 2.1 far-field equation, as a
 *                       chunked scan).  Same results and arguments as
 *                       sfa_prefill, for bf16 inputs and at most 64 chunks
 *                       (4096 tokens) per sequence; other calls return
 *                       SFA_ERR_UNSUPPORTED.  It is measured slower than
 *                       sfa_prefill (the waits for the published aggregates
 *                       cost more than the separate scan) and offered for
 *                       callers that must not read K twice.
 * Other values of `parts` return SFA_ERR_INVALID_ARG.
 */
enum { SFA_PREFILL_SCAN = 1, SFA_PREFILL_ATTEND = 2, SFA_PREFILL_SINGLE_PASS = 4 };
int sfa_prefill_part(int parts, const void *q, const void *k, const void *v,
                     const float *gamma, const float *alpha,
                     void *out, void *ring_k, void *ring_v, float *state,
                     const int32_t *pos0,
                     int B, int n, int Hq, int Hkv, int d, int window, float scale,
                     int in_dtype, int out_dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * sfa_prefill_qh -- sfa_prefill under the other reading of "per-head γ" with
 * grouped-query attention: γ and the far-field state S belong to each QUERY
 * head.  Every query head of a group folds the same evicted keys (those of its
 * KV head) into its own S with its own decay; the near field and the ring are
 * those of sfa_prefill.  (First page, section 2.1 far-field and fusion
 * equations; under grouped-query attention a per-head γ can mean either kind
 * of head.)
 *  gamma    [Hq] fp32.
 *  state    [B,Hq,d] fp32 (written; read first when pos0 != NULL).
 *  workspace at least sfa_prefill_workspace_size(B, n, Hq, d) bytes (the scan
 *           keeps one chain per query head).
 * Every other argument, layout and error code is that of sfa_prefill.
 */
int sfa_prefill_qh(const void *q, const void *k, const void *v,
                   const float *gamma, const float *alpha,
                   void *out, void *ring_k, void *ring_v, float *state,
                   const int32_t *pos0,
                   int B, int n, int Hq, int Hkv, int d, int window, float scale,
                   int in_dtype, int out_dtype,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * sfa_prefill_rm -- sfa_prefill under the other reading of "mean(K_hist)" in
 * the first page's section 2.1 far-field equation: at a position p >= W the
 * EWMA input is the mean M_p of every key that has left the window so far
 * (positions 0..p-W, m = p-W+1 keys), not only the key leaving at p:
 *   S_p = γ·S_{p-1} + (1-γ)·M_p,   O = O_near + α·S_p.
 * S and γ are per KV head; the near field and the ring are those of
 * sfa_prefill.
 *  state    [B,Hkv,2,d] fp32: S, then M (written; read first when pos0 != NULL,
 *           M then standing for the max(0, pos0-W) keys that left before).
 *  workspace at least sfa_prefill_workspace_size(B, n, 3*Hkv, d) bytes.
 * Every other argument, layout and error code is that of sfa_prefill.
 */
int sfa_prefill_rm(const void *q, const void *k, const void *v,
                   const float *gamma, const float *alpha,
                   void *out, void *ring_k, void *ring_v, float *state,
                   const int32_t *pos0,
                   int B, int n, int Hq, int Hkv, int d, int window, float scale,
                   int in_dtype, int out_dtype,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * sfa_prefill_noalloc -- sfa_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace: the scan's per-chunk aggregates and
 * carries go to a static device array of SFA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The call
 * allocates and frees nothing (no hipMalloc, no allocating library routine);
 * the caller still passes every input and output.
 *
 * Every argument, layout, result and error code is that of sfa_prefill, plus:
 *  - SFA_ERR_TOO_LARGE (nothing enqueued or written) when
 *    sfa_prefill_workspace_size(B, n, Hkv, d) > SFA_NOALLOC_SCRATCH_BYTES
 *    (16 MiB: e.g. B·Hkv·ceil(n/64)·d up to 699,050 words of 24 bytes, which
 *    holds one 65,536-token layer with 4 KV heads at head_dim 128);
 *  - the scratch is shared by every call on the same GPU and keeps the last
 *    call's contents (nothing in it needs to start at zero): calls that
 *    overlap on one GPU (different streams, or threads without ordering) race
 *    and must not be issued;
 *  - the scratch address is looked up once per device, with the device that
 *    owns `stream` current, on that device's first call.
 */
#define SFA_NOALLOC_SCRATCH_BYTES (16u << 20)
int sfa_prefill_noalloc(const void *q, const void *k, const void *v,
                        const float *gamma, const float *alpha,
                        void *out, void *ring_k, void *ring_v, float *state,
                        const int32_t *pos0,
                        int B, int n, int Hq, int Hkv, int d, int window, float scale,
                        int in_dtype, int out_dtype, void *stream);

/*
 * sfa_decode_step -- one generated token for L layers at once.
 * (First page, section 2.1 equations with the constant-memory k-slot ring of
 * section 2.2.)
 *
 * For each layer l, sequence b and KV head G, with p = pos[b] and s = p mod W:
 *   if p >= W:  S <- γ[l,G]·S + (1-γ[l,G])·ring_k[s]   (old contents: position p-W)
 *   ring_k[s] <- k_new;  ring_v[s] <- v_new
 *   for each query head h of the group: softmax over the valid slots (all W
 *   when p >= W-1, else slots 0..p), O = Σ p_j·ring_v[j] + α[l,h]·S.
 * The result equals token p of a prefill of the whole sequence.
 *
 *  q            [L,B,Hq,d]  in_dtype.
 *  k_new, v_new [L,B,Hkv,d] in_dtype.
 *  ring_k, ring_v [L,B,Hkv,W,d] in_dtype, updated in place (only slot s).
 *  state        [L,B,Hkv,d] fp32, updated in place.
 *  pos          [B] int32, >= 0, read-only; the caller advances it once per
 *               step (so one launch can cover all L layers without a race).
 *               A sequence with a negative entry is skipped (nothing written).
 *  gamma        [L,Hkv] fp32;  alpha [L,Hq] fp32.
 *  out          [L,B,Hq,d] out_dtype (written).
 */
int sfa_decode_step(const void *q, const void *k_new, const void *v_new,
                    void *ring_k, void *ring_v, float *state,
                    const int32_t *pos, const float *gamma, const float *alpha,
                    void *out, int L, int B, int Hq, int Hkv, int d, int window,
                    float scale, int in_dtype, int out_dtype, void *stream);

/*
 * sfa_decode_step_qh -- sfa_decode_step with γ and S per query head (see
 * sfa_prefill_qh): when the key of position pos-W leaves the window it enters
 * the S of every query head of its group, each with that head's decay.
 *  gamma  [L,Hq] fp32;  state [L,B,Hq,d] fp32 (in/out).
 * Every other argument, layout and error code is that of sfa_decode_step.
 */
int sfa_decode_step_qh(const void *q, const void *k_new, const void *v_new,
                       void *ring_k, void *ring_v, float *state,
                       const int32_t *pos, const float *gamma, const float *alpha,
                       void *out, int L, int B, int Hq, int Hkv, int d, int window, float scale,
                       int in_dtype, int out_dtype, void *stream);

/*
 * sfa_decode_step_rm -- sfa_decode_step with the running mean of the keys
 * that have left the window as the EWMA input (see sfa_prefill_rm): when the
 * key of position pos-W leaves, M <- (M·(m-1) + k)/m with m = pos-W+1, then
 * S <- γ·S + (1-γ)·M.
 *  state  [L,B,Hkv,2,d] fp32 (in/out): S, then M.
 * Every other argument, layout and error code is that of sfa_decode_step.
 */
int sfa_decode_step_rm(const void *q, const void *k_new, const void *v_new,
                       void *ring_k, void *ring_v, float *state,
                       const int32_t *pos, const float *gamma, const float *alpha,
                       void *out, int L, int B, int Hq, int Hkv, int d, int window, float scale,
                       int in_dtype, int out_dtype, void *stream);

/*
 * Workspace bytes sfa_enhance (and sfa_enhance_prepared) needs for (L, T, H):
 * per-chunk fp32 aggregates of the EMA field, proportional to L·ceil(T/64)·H,
 * the carried ring, the slot weights of every 64-token chunk and, for
 * sfa_enhance, the pool's MFMA operands.  16-byte aligned.
 */
size_t sfa_enhance_workspace_size(int L, int T, int H);

/*
 * sfa_enhance -- optional triple-channel enhancement applied to an attention
 * output.  (Page "Dalin Soma SFA..." section 2.1: ring-buffer channel, EMA
 * field channel, 64-slot semantic pool; section 2.2: fusion, clip and the
 * per-layer factor; section 2.4: the ring mean always divides by the ring
 * size.  Defaults from the SFA_Config of page "Signal Field Attention (SFA)".)
 *
 * For layer i (global index lg = layer0 + i) and token t (global index t0 + t),
 * with a = attn[i,t,:] (H = hidden size, the whole row; no per-head split):
 *   ring[(t0+t) mod R] <- a;  rm = Σ ring / R
 *   field <- γ_e·field + (1-γ_e)·a
 *   c_j = <a, s_j> / (max(|a|,1e-12)·max(|s_j|,1e-12)),  w = softmax(c / T),
 *   sem = Σ_j w_j·s_j
 *   e = rm + 0.5·field + 0.5·sem
 *   enh = α_lg·clip(e, -clip, +clip),  out = a + enh
 *   α_lg = α_base·(0.3 + 0.7·lg/(n_layers-1))·cross_decay^lg  (ratio 0 if n_layers == 1)
 *
 *  attn         [L,T,H] in_dtype.
 *  out          [L,T,H] out_dtype (written; may not alias attn).
 *  ring         [L,R,H] fp32, carried ring (zeros for a fresh stream), updated.
 *  field        [L,H] fp32, carried field (zeros for a fresh stream), updated.
 *  pool         fp32 slots of layer i at pool + i·pool_layer_stride, each
 *               [n_slots,H]; pool_layer_stride = 0 shares one pool.  Read-only.
 *  enhancement  [L,T,H] fp32 or NULL: enh values (written when non-NULL).
 *  R = ring_size in [1,16]; n_slots in [1,64]; temperature > 0; clip >= 0.
 *  workspace:   at least sfa_enhance_workspace_size(L, T, H) bytes.
 *
 * Precision: the contractions run on bf16 MFMAs with fp32 accumulation; bf16
 * attention values enter exactly, fp32 ones and every other operand as bf16
 * hi + lo pairs (about 2^-17 relative).  Exception, bf16 inputs only: a layer
 * whose α_lg·0.5·(2^-8 + 2^-18)·max|s| (max over that layer's pool entries)
 * is at most 1e-5 takes the pool and the slot weights of its semantic sum as
 * single bf16 values, which moves its outputs by at most that bound.
 */
int sfa_enhance(const void *attn, void *out, float *ring, float *field,
                const float *pool, long long pool_layer_stride, float *enhancement,
                int L, int layer0, int n_layers, int T, int H, int t0,
                float alpha_base, float cross_decay, float ema_gamma, float temperature,
                float clip, int ring_size, int n_slots,
                int in_dtype, int out_dtype,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * The semantic pool is read-only ("Dalin Soma SFA..." section 2.1: a fixed set
 * of 64 slots), so the MFMA operands sfa_enhance derives from it on every call
 * (the slots split into bf16 hi + lo in the two operand orders, 1/|slot| and
 * the largest |element| of every slot) can be derived once and kept:
 *
 * sfa_enhance_pool_bytes -- bytes of the prepared form of n_pool_layers pool
 *   layers at hidden size H: one record of sfa_enhance_pool_bytes(1, H) bytes
 *   (a multiple of 256) per layer, in layer order.
 *
 * sfa_enhance_prepare_pool -- writes the prepared form of pool layers
 *   0..n_pool_layers-1 (layer j at pool + j·pool_layer_stride floats, each
 *   [n_slots, H] fp32, as in sfa_enhance) into `prepared` (device memory of at
 *   least sfa_enhance_pool_bytes(n_pool_layers, H) bytes, 256-byte aligned,
 *   owned by the caller).  Asynchronous on `stream`; the pool is only read.
 *   n_slots in [1,64], H a multiple of 64 (else SFA_ERR_UNSUPPORTED),
 *   pool_layer_stride >= n_slots·H when n_pool_layers > 1.
 *
 * sfa_enhance_prepared -- sfa_enhance with the pool given in prepared form:
 *   with shared_pool != 0 every layer of the call uses record 0 of
 *   `prepared`; otherwise layer i of the call uses record i (for a call that
 *   starts at global layer layer0, pass prepared + layer0·sfa_enhance_pool_bytes(1, H)
 *   when the records are kept for every layer of the model).  n_slots must be
 *   the value the records were prepared with.  Every other argument, result
 *   and error code is that of sfa_enhance; the workspace is the same size.
 */
size_t sfa_enhance_pool_bytes(int n_pool_layers, int H);
int sfa_enhance_prepare_pool(const float *pool, long long pool_layer_stride, int n_pool_layers,
                             int n_slots, int H, void *prepared, size_t prepared_bytes, void *stream);
int sfa_enhance_prepared(const void *attn, void *out, float *ring, float *field,
                         const void *prepared, int shared_pool, float *enhancement,
                         int L, int layer0, int n_layers, int T, int H, int t0,
                         float alpha_base, float cross_decay, float ema_gamma, float temperature,
                         float clip, int ring_size, int n_slots,
                         int in_dtype, int out_dtype,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * sfa_decode_step_enhance -- sfa_decode_step fused with the triple-channel
 * enhancement of every (layer, sequence)'s attention output, which never
 * leaves the chip (first page, sections 2.1-2.2, for the step; page "Dalin
 * Soma SFA..." sections 2.1, 2.2 and 2.4 for the enhancement, applied per
 * layer to each new token's attention output as the engine of page "Signal
 * Field Attention (SFA)" does).
 *
 * For layer l (global index lg = layer0 + l) and sequence b with p = pos[b]:
 * the decode step of sfa_decode_step (S per KV head) gives the attention row
 * o (all Hq heads, H = Hq·d values); a = o as out_dtype holds it (rounded to
 * bf16 for SFA_BF16); then, on that sequence's enhancement state,
 *   e_ring[l,b][p mod R] <- a;  rm = Σ e_ring[l,b] / R
 *   field[l,b] <- γ_e·field[l,b] + (1-γ_e)·a
 *   c_j = <a, s_j> / (max(|a|,1e-12)·|s_j|),  w = softmax(c / T),  sem = Σ_j w_j·s_j
 *   out[l,b] = a + α_lg·clip(rm + 0.5·field + 0.5·sem, -clip, +clip)
 * with α_lg as in sfa_enhance.  This equals sfa_decode_step (out_dtype) then
 * sfa_enhance of the one token at stream position p, per sequence (here the
 * semantic operands are always bf16 hi + lo pairs).
 *
 *  q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha: as
 *               sfa_decode_step (S per KV head).  A negative pos[b] skips
 *               the sequence: nothing of it is written.
 *  out          [L,B,H] out_dtype (written): the enhanced attention rows.
 *  e_ring       [L,B,R,H] fp32, each sequence's last R attention rows
 *               (slot p mod R), updated; zeros for a fresh stream.
 *  field        [L,B,H] fp32, updated; zeros for a fresh stream.
 *  prepared     pool records of sfa_enhance_prepare_pool for hidden size H:
 *               shared_pool != 0: record 0 for every layer; otherwise layer
 *               l of the call uses record l.  n_slots as prepared.
 *  enhancement  [L,B,H] fp32 or NULL: α_lg·clip(...) (written when non-NULL).
 *  Limits (else SFA_ERR_UNSUPPORTED): bf16 inputs, Hq/Hkv <= 16, H <= 4096.
 *  One workgroup per (layer, sequence) reads its layer's pool: the form
 *  suits the engine's shape (one sequence, every layer); a large batch
 *  re-reads every pool once per sequence.
 */
int sfa_decode_step_enhance(const void *q, const void *k_new, const void *v_new,
                            void *ring_k, void *ring_v, float *state,
                            const int32_t *pos, const float *gamma, const float *alpha,
                            void *out, float *e_ring, float *field,
                            const void *prepared, int shared_pool, float *enhancement,
                            int L, int B, int Hq, int Hkv, int d, int window, float scale,
                            int layer0, int n_layers, float alpha_base, float cross_decay,
                            float ema_gamma, float temperature, float clip, int ring_size,
                            int n_slots, int in_dtype, int out_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SFA_H */
