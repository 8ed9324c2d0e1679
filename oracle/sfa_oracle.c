/*
 * sfa_oracle.c -- plain CPU fp64 oracle for Signal Field Attention (SFA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load this library.  The GPU library never links,
 * includes or calls it, and it shares no code with the GPU kernels.
 *
 * Every output is computed from its definition, token by token, in double
 * precision, with no tiling, no chunked scan and no reordering beyond what the
 * definition states.  Large inputs arrive as float (bf16 and fp32 values are
 * exact in float) and are widened to double before any arithmetic.
 *
 * Pages cited (titles as published):
 *   [P1] "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩"
 *        (adg.csdn.net) -- section 2.1 architecture: near-field equation,
 *        far-field EWMA equation, fusion equation; section 2.2 complexity
 *        table (window k = 16).
 *   [P2] "Signal Field Attention (SFA)" project page (mhpn.cn) -- triple-channel
 *        engine diagram, SFA_Config defaults, cross-layer decay formula.
 *   [P3] "Dalin Soma SFA基于信号场注意力机制的神经网络推理加速框架"
 *        (171host.com) -- section 2.1 three channels, section 2.2 fusion,
 *        section 2.4 Metal ring-mean kernel.
 *
 * Readings of points the pages leave open (window includes the current token,
 * one evicted key enters S per step, S_0 = 0, S per KV head, ring slot
 * p mod W, clip-then-scale, ring mean always divides by the ring size, ...)
 * are stated where they are used below.
 *
 * Parity pins: every function here is pinned by the CPU tests in
 * tests/test_oracle_pins.py (closed forms, library special cases, brute force,
 * hand-computed fixtures); none is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* A size the definitions do not cover stops the process with a message: the
 * oracle never returns a result it did not compute. */
static void require(int ok, const char *what) {
    if (!ok) {
        fprintf(stderr, "sfa oracle: invalid argument: %s\n", what);
        fflush(stderr);
        abort();
    }
}

/* threads the OpenMP loops below use (reported with CPU timings) */
int oracle_num_threads(void) { return omp_get_max_threads(); }

#define IDX4(a, b, c, e, B_, C_, E_) ((((size_t)(a) * (B_) + (b)) * (C_) + (c)) * (E_) + (e))

/* --------------------------------------------------------------------------
 * Windowed attention + EWMA far field, prefill form.
 *
 * [P1] §2.1: near field O_near = softmax(Q_t K_near^T / sqrt(d)) V_near over
 * the most recent k tokens; far field S_t = γ S_{t-1} + (1-γ)·(keys that left
 * the window); output O = O_near + α S.
 *
 * Readings used:
 *  - the window of the token at position p is positions max(0,p-W+1) .. p
 *    (the current token included, so it is never empty);
 *  - S starts at 0; at position p >= W exactly one key, the one at p-W,
 *    leaves the window and enters S; the token at p uses S after its own
 *    eviction, so window and S together account for keys 0..p exactly once;
 *  - S is per KV head (γ indexed by KV head), α per query head; with
 *    s_per_query set, the other reading of "per-head γ": γ and S per query
 *    head (every query head of a group folds the same evicted keys with its
 *    own decay);
 *  - query head h reads KV head h / (Hq/Hkv);
 *  - scale <= 0 means 1/sqrt(d);
 *  - with running_mean set, the other reading of "mean(K_hist)": the EWMA
 *    input at position p >= W is the mean M_p of all keys that have left the
 *    window so far, positions 0..p-W (m_p = p-W+1 keys), instead of the one
 *    key leaving at p.  The mean is kept as a running fp64 sum divided by
 *    the count.
 *
 * Continuation: pos0[b] (NULL = all zero) is the position of the first token
 * of this call.  When pos0[b] > 0, keys and values at positions < pos0[b] are
 * read from the ring (position q in slot q mod W) and S starts from state[b]
 * (with running_mean, M as well: the sum restarts as M times the
 * max(0, pos0-W) keys it averages).
 *
 * Layouts: q [B,n,Hq,d]; k, v [B,n,Hkv,d]; out [B,n,Hq,d];
 * ring_k, ring_v [B,Hkv,W,d] (in/out); state [B,Hkv,d] (in/out);
 * gamma [Hkv]; alpha [Hq].  With s_per_query: state [B,Hq,d], gamma [Hq].
 * With running_mean: state [B,Hs,2,d], S then M.
 * ------------------------------------------------------------------------ */

/* key/value of position qpos for batch b, KV head G */
static const double *kv_row(const float *x, const double *ring, int b, int G, int qpos,
                            int p0, int n, int Hkv, int d, int W, double *tmp) {
    if (qpos >= p0) {
        const float *src = x + IDX4(b, qpos - p0, G, 0, n, Hkv, d);
        for (int e = 0; e < d; ++e) tmp[e] = (double)src[e];
        return tmp;
    }
    return ring + IDX4(b, G, qpos % W, 0, Hkv, W, d);
}

void oracle_prefill(const float *q, const float *k, const float *v,
                    const double *gamma, const double *alpha,
                    double *out, double *ring_k, double *ring_v, double *state,
                    const int32_t *pos0,
                    int B, int n, int Hq, int Hkv, int d, int W, double scale, int s_per_query,
                    int running_mean) {
    const int group = Hq / Hkv;
    const int Hs = s_per_query ? Hq : Hkv; /* heads that own an S */
    const int sw = running_mean ? 2 * d : d; /* state words per S head */
    require(B >= 0 && n >= 0 && d >= 1 && W >= 1 && Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0,
            "prefill sizes (W >= 1, Hq a multiple of Hkv)");
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    /* final state of each (b, S head), written to state after the loop so that
     * every head reads the caller's ring/state as they were on entry */
    double *final_S = (double *)calloc((size_t)B * Hs * sw, sizeof(double));

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int G = h / group;
            const int hs = s_per_query ? h : G; /* the head that owns this S */
            const int p0 = pos0 ? pos0[b] : 0;
            const double g = gamma[hs];
            double *S = (double *)malloc(sizeof(double) * d);
            double *C = (double *)malloc(sizeof(double) * d); /* running_mean: sum of the left keys */
            double *o = (double *)malloc(sizeof(double) * d);
            double *tk = (double *)malloc(sizeof(double) * d);
            double *tv = (double *)malloc(sizeof(double) * d);
            double *sc = (double *)malloc(sizeof(double) * W);
            const double *st_in = state + ((size_t)b * Hs + hs) * sw;
            const int m_in = (p0 - W > 0) ? p0 - W : 0; /* keys left before this call */
            for (int e = 0; e < d; ++e) {
                S[e] = (p0 > 0) ? st_in[e] : 0.0;
                C[e] = (running_mean && p0 > 0) ? st_in[d + e] * m_in : 0.0;
            }

            for (int t = 0; t < n; ++t) {
                const int p = p0 + t;
                /* far field: the key at p-W leaves the window now */
                if (p >= W) {
                    const double *ke = kv_row(k, ring_k, b, G, p - W, p0, n, Hkv, d, W, tk);
                    if (running_mean) {
                        const double m = (double)(p - W + 1); /* keys left so far */
                        for (int e = 0; e < d; ++e) {
                            C[e] += ke[e];
                            S[e] = g * S[e] + (1.0 - g) * (C[e] / m);
                        }
                    } else {
                        for (int e = 0; e < d; ++e) S[e] = g * S[e] + (1.0 - g) * ke[e];
                    }
                }
                /* near field: softmax over positions lo..p */
                const int lo = (p - W + 1 > 0) ? p - W + 1 : 0;
                const float *qr = q + IDX4(b, t, h, 0, n, Hq, d);
                double m = -INFINITY;
                for (int j = lo; j <= p; ++j) {
                    const double *kr = kv_row(k, ring_k, b, G, j, p0, n, Hkv, d, W, tk);
                    double s = 0.0;
                    for (int e = 0; e < d; ++e) s += (double)qr[e] * kr[e];
                    s *= scale;
                    sc[j - lo] = s;
                    if (s > m) m = s;
                }
                double den = 0.0;
                for (int j = lo; j <= p; ++j) {
                    sc[j - lo] = exp(sc[j - lo] - m);
                    den += sc[j - lo];
                }
                for (int e = 0; e < d; ++e) o[e] = 0.0;
                for (int j = lo; j <= p; ++j) {
                    const double *vr = kv_row(v, ring_v, b, G, j, p0, n, Hkv, d, W, tv);
                    const double pj = sc[j - lo] / den;
                    for (int e = 0; e < d; ++e) o[e] += pj * vr[e];
                }
                /* fusion: O = O_near + α S */
                double *dst = out + IDX4(b, t, h, 0, n, Hq, d);
                for (int e = 0; e < d; ++e) dst[e] = o[e] + alpha[h] * S[e];
            }
            if (s_per_query || h % group == 0) {
                double *fs = final_S + ((size_t)b * Hs + hs) * sw;
                const int m_end = (p0 + n - W > 0) ? p0 + n - W : 0;
                for (int e = 0; e < d; ++e) {
                    fs[e] = S[e];
                    if (running_mean) fs[d + e] = m_end > 0 ? C[e] / m_end : 0.0;
                }
            }
            free(S); free(C); free(o); free(tk); free(tv); free(sc);
        }
    }

    /* ring hand-off: the last min(W, p0+n) positions sit in slot p mod W;
     * slots whose position is older than pos0 and still in the window keep
     * their contents */
    for (int b = 0; b < B; ++b) {
        const int p0 = pos0 ? pos0[b] : 0;
        const int first = (p0 + n - W > p0) ? p0 + n - W : p0;
        for (int G = 0; G < Hkv; ++G) {
            for (int p = first; p < p0 + n; ++p) {
                double *rk = ring_k + IDX4(b, G, p % W, 0, Hkv, W, d);
                double *rv = ring_v + IDX4(b, G, p % W, 0, Hkv, W, d);
                const float *sk = k + IDX4(b, p - p0, G, 0, n, Hkv, d);
                const float *sv = v + IDX4(b, p - p0, G, 0, n, Hkv, d);
                for (int e = 0; e < d; ++e) { rk[e] = sk[e]; rv[e] = sv[e]; }
            }
        }
        for (int i = 0; i < Hs * sw; ++i) state[(size_t)b * Hs * sw + i] = final_S[(size_t)b * Hs * sw + i];
    }
    free(final_S);
}

/* --------------------------------------------------------------------------
 * One decode step over L layers.  [P1] §2.1 equations applied to a single
 * new token, with the k-slot ring of [P1] §2.2 (O(k·d) memory, k = 16) and the
 * O(1) ring-buffer KV cache named in [P1]'s module list.
 *
 * For each (l, b, KV head G): p = pos[b] is the position of the new token,
 * s = p mod W its slot.  If p >= W the slot still holds the key of position
 * p-W, which leaves the window: S <- γ S + (1-γ) ring_k[s].  Then the new key
 * and value overwrite slot s.  Attention runs over the valid slots: all W once
 * p >= W-1, else slots 0..p (position j < W lives in slot j).
 *
 * Layouts: q [L,B,Hq,d]; k_new, v_new [L,B,Hkv,d]; ring_k, ring_v
 * [L,B,Hkv,W,d] (in/out); state [L,B,Hkv,d] (in/out); pos [B];
 * gamma [L,Hkv]; alpha [L,Hq]; out [L,B,Hq,d].  With s_per_query (γ and S per
 * query head, see oracle_prefill): state [L,B,Hq,d], gamma [L,Hq]; every query
 * head folds the same evicted key into its own S.  With running_mean (see
 * oracle_prefill): state [L,B,Hs,2,d], S then M; the evicted key joins the
 * mean of the m = p-W keys that left before it, and S takes the new mean.
 * A sequence with a negative position is skipped: nothing of it is written.
 * ------------------------------------------------------------------------ */
void oracle_decode_step(const float *q, const float *k_new, const float *v_new,
                        double *ring_k, double *ring_v, double *state,
                        const int32_t *pos, const double *gamma, const double *alpha,
                        double *out, int L, int B, int Hq, int Hkv, int d, int W,
                        double scale, int s_per_query, int running_mean) {
    const int group = Hq / Hkv;
    const int sw = running_mean ? 2 * d : d; /* state words per S head */
    require(L >= 0 && B >= 0 && d >= 1 && W >= 1 && Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0,
            "decode sizes (W >= 1, Hq a multiple of Hkv)");
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);

#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int l = 0; l < L; ++l) {
        for (int b = 0; b < B; ++b) {
            for (int G = 0; G < Hkv; ++G) {
                const int p = pos[b];
                if (p < 0) continue;
                const int s = p % W;
                const size_t unit = ((size_t)l * B + b) * Hkv + G;
                double *rk = ring_k + unit * W * d;
                double *rv = ring_v + unit * W * d;
                const float *kn = k_new + unit * d;
                const float *vn = v_new + unit * d;

                /* the evicted key (old contents of slot s) enters every S of the unit */
                const int n_s = s_per_query ? group : 1;
                for (int i = 0; i < n_s; ++i) {
                    const size_t hs = s_per_query ? ((size_t)l * B + b) * Hq + (size_t)G * group + i : unit;
                    const double g = s_per_query ? gamma[(size_t)l * Hq + (size_t)G * group + i]
                                                 : gamma[(size_t)l * Hkv + G];
                    double *S = state + hs * sw;
                    if (p >= W && running_mean) {
                        double *M = S + d;
                        const double m = (double)(p - W + 1); /* keys left, this one included */
                        for (int e = 0; e < d; ++e) {
                            M[e] = (M[e] * (m - 1.0) + rk[(size_t)s * d + e]) / m;
                            S[e] = g * S[e] + (1.0 - g) * M[e];
                        }
                    } else if (p >= W) {
                        for (int e = 0; e < d; ++e) S[e] = g * S[e] + (1.0 - g) * rk[(size_t)s * d + e];
                    }
                }
                for (int e = 0; e < d; ++e) {
                    rk[(size_t)s * d + e] = kn[e];
                    rv[(size_t)s * d + e] = vn[e];
                }
                const int nvalid = (p >= W - 1) ? W : p + 1;

                double *sc = (double *)malloc(sizeof(double) * W);
                for (int hh = 0; hh < group; ++hh) {
                    const int h = G * group + hh;
                    const float *qr = q + (((size_t)l * B + b) * Hq + h) * d;
                    double m = -INFINITY;
                    for (int j = 0; j < nvalid; ++j) {
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e) acc += (double)qr[e] * rk[(size_t)j * d + e];
                        sc[j] = acc * scale;
                        if (sc[j] > m) m = sc[j];
                    }
                    double den = 0.0;
                    for (int j = 0; j < nvalid; ++j) { sc[j] = exp(sc[j] - m); den += sc[j]; }
                    double *dst = out + (((size_t)l * B + b) * Hq + h) * d;
                    const double a = alpha[(size_t)l * Hq + h];
                    const double *S = state + (s_per_query ? ((size_t)l * B + b) * Hq + h : unit) * sw;
                    for (int e = 0; e < d; ++e) {
                        double o = 0.0;
                        for (int j = 0; j < nvalid; ++j) o += (sc[j] / den) * rv[(size_t)j * d + e];
                        dst[e] = o + a * S[e];
                    }
                }
                free(sc);
            }
        }
    }
}

/* --------------------------------------------------------------------------
 * Triple-channel enhancement.  [P3] §2.1 (three channels), §2.2 (fusion and
 * the per-layer factor), [P2] engine diagram and SFA_Config defaults.
 *
 * For layer l (global index lg = layer0 + l of n_layers) and token t (global
 * index t0 + t), with a = attn[l, t, :]:
 *   ring channel  : R[(t0+t) mod R_size] <- a;  rm = sum(R) / R_size
 *                   (ring zero-initialised, always divided by the ring size,
 *                   as the ring-mean kernel of [P3] §2.4 does)
 *   field channel : F <- γ_e F + (1-γ_e) a   (update with the current token,
 *                   then use it)
 *   semantic pool : c_i = <a, s_i> / (max(|a|,1e-12) max(|s_i|,1e-12));
 *                   w = softmax(c / T);  sem = sum_i w_i s_i  (pool read-only)
 *   fusion        : e = rm + 0.5 F + 0.5 sem;
 *                   enh = α_l clip(e, -clip, +clip);  out = a + enh
 *   α_l = α_base (0.3 + 0.7 lg/(n_layers-1)) cross_decay^lg
 *         (the ratio is 0 when n_layers == 1)
 *
 * Layouts: attn, out, enhancement [L,T,H]; ring [L,R_size,H] and field [L,H]
 * (in/out); pool layer l at pool + l*pool_layer_stride, [n_slots,H].
 * enhancement may be NULL.
 * ------------------------------------------------------------------------ */
double oracle_alpha_layer(double alpha_base, double cross_decay, int layer, int n_layers) {
    const double ratio = (n_layers > 1) ? (double)layer / (double)(n_layers - 1) : 0.0;
    return alpha_base * (0.3 + 0.7 * ratio) * pow(cross_decay, (double)layer);
}

void oracle_enhance(const float *attn, double *out, double *ring, double *field,
                    const float *pool, long pool_layer_stride, double *enhancement,
                    int L, int layer0, int n_layers, int T, int H, int t0,
                    double alpha_base, double cross_decay, double ema_gamma,
                    double temperature, double clip, int ring_size, int n_slots) {
    require(L >= 0 && T >= 0 && H >= 1 && ring_size >= 1 && n_slots >= 1 && temperature > 0.0,
            "enhance sizes (ring_size, n_slots >= 1, temperature > 0)");
#pragma omp parallel for schedule(dynamic)
    for (int l = 0; l < L; ++l) {
        const double al = oracle_alpha_layer(alpha_base, cross_decay, layer0 + l, n_layers);
        double *R = ring + (size_t)l * ring_size * H;
        double *F = field + (size_t)l * H;
        const float *P = pool + (size_t)l * pool_layer_stride;
        double *a = (double *)malloc(sizeof(double) * H);
        double *c = (double *)malloc(sizeof(double) * n_slots);
        double *pn = (double *)malloc(sizeof(double) * n_slots);

        for (int i = 0; i < n_slots; ++i) {
            double ss = 0.0;
            for (int x = 0; x < H; ++x) ss += (double)P[(size_t)i * H + x] * (double)P[(size_t)i * H + x];
            pn[i] = sqrt(ss);
            if (pn[i] < 1e-12) pn[i] = 1e-12;
        }

        for (int t = 0; t < T; ++t) {
            const float *src = attn + ((size_t)l * T + t) * H;
            for (int x = 0; x < H; ++x) a[x] = (double)src[x];

            /* ring channel */
            const int slot = (int)(((long)t0 + t) % ring_size);
            for (int x = 0; x < H; ++x) R[(size_t)slot * H + x] = a[x];
            /* field channel */
            for (int x = 0; x < H; ++x) F[x] = ema_gamma * F[x] + (1.0 - ema_gamma) * a[x];
            /* semantic channel: cosine scores, temperature softmax */
            double na = 0.0;
            for (int x = 0; x < H; ++x) na += a[x] * a[x];
            na = sqrt(na);
            if (na < 1e-12) na = 1e-12;
            double m = -INFINITY;
            for (int i = 0; i < n_slots; ++i) {
                double dot = 0.0;
                for (int x = 0; x < H; ++x) dot += a[x] * (double)P[(size_t)i * H + x];
                c[i] = dot / (na * pn[i]) / temperature;
                if (c[i] > m) m = c[i];
            }
            double den = 0.0;
            for (int i = 0; i < n_slots; ++i) { c[i] = exp(c[i] - m); den += c[i]; }

            for (int x = 0; x < H; ++x) {
                double rs = 0.0;
                for (int r = 0; r < ring_size; ++r) rs += R[(size_t)r * H + x];
                const double rm = rs / ring_size;
                double sem = 0.0;
                for (int i = 0; i < n_slots; ++i) sem += (c[i] / den) * (double)P[(size_t)i * H + x];
                double e = rm + 0.5 * F[x] + 0.5 * sem;
                if (e > clip) e = clip;
                if (e < -clip) e = -clip;
                const double enh = al * e;
                out[((size_t)l * T + t) * H + x] = a[x] + enh;
                if (enhancement) enhancement[((size_t)l * T + t) * H + x] = enh;
            }
        }
        free(a); free(c); free(pn);
    }
}
