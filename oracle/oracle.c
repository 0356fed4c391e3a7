/*
 * CPU oracle for one transformer-decoder decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes. The pages name the operators of the step but print no
 * formulas: the MPK article (devpress.csdn.net, §1 "GPU计算中的任务调度挑战")
 * gives the layer as Attention followed by MLP, and the Ada-MK summary
 * (gist.science, "Methodik") speaks of the Transformer decoder plus the
 * LM head. The oracle therefore writes out the plain definition of a
 * pre-norm decoder decode step (Qwen3-style: RMSNorm, QKV projection,
 * per-head QK RMSNorm, rotate-half RoPE, grouped-query attention over the
 * KV cache, O projection, SwiGLU MLP, final RMSNorm, LM head). Readings for
 * every point the pages leave open are listed with the design notes; in
 * short: eps inside the square root; RoPE pairs (i, i + D/2) with
 * theta_i = pos * base^(-2i/D); query head h reads KV head
 * floor(h * Hkv / Hq); the new K/V are rounded to the cache type and
 * appended at position pos before attention, which then covers pos + 1
 * keys; silu(z) = z / (1 + exp(-z)).
 *
 * Precision: every intermediate vector is stored as float32; every sum
 * (dot products, norms, softmax) accumulates in double; bf16 inputs are
 * widened exactly. Dot products run in index order. The only
 * parallelism (optional OpenMP) is across independent output rows, which
 * changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_W4 = 2 };

/*
 * W4 matrices (weight-only 4-bit quantisation, the Ada-MK summary's W4A16,
 * gist.science "Hauptbeiträge" 4; the pages fix no format, so: symmetric
 * 4-bit codes with offset 8 and one bf16 scale per group of 128 inputs of a
 * row). One buffer per [rows, cols] matrix: the codes, rows * cols / 2
 * bytes, element (r, c) in byte (r * cols + c) / 2, low nibble for even c,
 * high nibble for odd c; then, from byte rows * cols / 2 rounded up to 256,
 * the scales, bf16 [rows][cols / 128]. The weight is (code - 8) * scale.
 */


static inline float bf16_to_f32(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

static inline size_t w4_scale_offset(int rows, int cols) { return (((size_t)rows * cols / 2) + 255) / 256 * 256; }

/* weight (r, c) of a W4 matrix, dequantised exactly */
static inline double w4_elem(const void* W, int rows, int cols, int r, int c) {
    const uint8_t* q = (const uint8_t*)W;
    const size_t i = (size_t)r * cols + c;
    const int code = (c & 1) ? (q[i / 2] >> 4) : (q[i / 2] & 15);
    const uint16_t* sc = (const uint16_t*)((const char*)W + w4_scale_offset(rows, cols));
    return (double)(code - 8) * (double)bf16_to_f32(sc[(size_t)r * (cols / 128) + c / 128]);
}

/* element i of a weight/cache array of either type, widened exactly */
static inline double elem(const void* p, int type, int64_t i) {
    if (type == ORC_BF16) return (double)bf16_to_f32(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* RMSNorm: y_i = g_i * x_i / sqrt(mean(x^2) + eps). */
void orc_rmsnorm(const float* x, int n, const void* gain, int gtype, double eps, float* y) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i) y[i] = (float)(elem(gain, gtype, i) * ((double)x[i] * inv));
}

/* y = W x with W row-major [rows, cols]: y_r = sum_c W[r, c] x[c]. */
void orc_matvec(const void* W, int wtype, int rows, int cols, const float* x, float* y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        const int64_t base = (int64_t)r * cols;
        if (wtype == ORC_W4) {
            for (int c = 0; c < cols; ++c) acc += w4_elem(W, rows, cols, r, c) * (double)x[c];
        } else if (wtype == ORC_BF16) {
            const uint16_t* w = (const uint16_t*)W + base;
            for (int c = 0; c < cols; ++c) acc += (double)bf16_to_f32(w[c]) * (double)x[c];
        } else {
            const float* w = (const float*)W + base;
            for (int c = 0; c < cols; ++c) acc += (double)w[c] * (double)x[c];
        }
        y[r] = (float)acc;
    }
}

/* Rotate-half RoPE in place on one head vector of length D at position pos. */
void orc_rope(float* v, int D, int pos, double base) {
    const int half = D / 2;
    for (int i = 0; i < half; ++i) {
        double theta = (double)pos * pow(base, -2.0 * (double)i / (double)D);
        double c = cos(theta), s = sin(theta);
        double a = v[i], b = v[i + half];
        v[i] = (float)(a * c - b * s);
        v[i + half] = (float)(b * c + a * s);
    }
}

static inline double silu(double z) { return z / (1.0 + exp(-z)); }

/* out_i = silu(g_i) * u_i */
void orc_swiglu(const float* g, const float* u, int n, float* out) {
    for (int i = 0; i < n; ++i) out[i] = (float)(silu((double)g[i]) * (double)u[i]);
}

/*
 * Single-head softmax attention over n keys:
 *   s_j = (q . K_j) / sqrt(D);  a = softmax(s);  out = sum_j a_j V_j.
 * K, V are [n, D] rows of the given type. probs (optional) receives a.
 */
void orc_attention_head(const float* q, const void* K, const void* V, int kvtype, int n, int D, float* out,
                        double* probs) {
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    const double scale = 1.0 / sqrt((double)D);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += (double)q[d] * elem(K, kvtype, (int64_t)j * D + d);
        s[j] = acc * scale;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j) acc += s[j] * elem(V, kvtype, (int64_t)j * D + d);
        out[d] = (float)(acc / l);
    }
    if (probs)
        for (int j = 0; j < n; ++j) probs[j] = s[j] / l;
    free(s);
}

typedef struct {
    int n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
    int qk_norm;  /* per-head RMSNorm of q and k before RoPE */
    int wtype;    /* ORC_F32 / ORC_BF16 for every weight and gain */
    int mtype;    /* type of the layer matrices: wtype, or ORC_W4 (gains, embedding and LM head stay wtype) */
    int kvtype;   /* cache element type */
    double eps, rope_base;
} orc_cfg;

typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} orc_layer;

/* store one new cache row (rounded to the cache type) */
static void cache_store(void* C, int kvtype, int64_t off, const float* src, int D) {
    if (kvtype == ORC_BF16) {
        uint16_t* c = (uint16_t*)C + off;
        for (int d = 0; d < D; ++d) c[d] = f32_to_bf16_rne(src[d]);
    } else {
        float* c = (float*)C + off;
        for (int d = 0; d < D; ++d) c[d] = src[d];
    }
}

static inline size_t kv_es(int kvtype) { return kvtype == ORC_BF16 ? 2 : 4; }

/*
 * One decoder layer for one sequence, x [H] in/out.
 * kc, vc: this layer's cache of the sequence, [Hkv][cap][D]. The new K/V
 * are written at position pos; attention covers positions 0..pos.
 */
void orc_layer_forward(const orc_cfg* c, const orc_layer* w, void* kc, void* vc, int cap, int pos, float* x) {
    const int H = c->hidden, D = c->head_dim, Hq = c->n_heads, Hkv = c->n_kv_heads, F = c->ffn;
    const int QD = Hq * D, KD = Hkv * D;
    float* xn = (float*)malloc(sizeof(float) * (size_t)(H > F ? H : F));
    float* q = (float*)malloc(sizeof(float) * (size_t)QD);
    float* k = (float*)malloc(sizeof(float) * (size_t)KD);
    float* v = (float*)malloc(sizeof(float) * (size_t)KD);
    float* att = (float*)malloc(sizeof(float) * (size_t)QD);
    float* y = (float*)malloc(sizeof(float) * (size_t)(H > F ? H : F));
    float* g = (float*)malloc(sizeof(float) * (size_t)F);
    float* u = (float*)malloc(sizeof(float) * (size_t)F);
    float* tmp = (float*)malloc(sizeof(float) * (size_t)D);

    /* attention block */
    orc_rmsnorm(x, H, w->attn_norm, c->wtype, c->eps, xn);
    orc_matvec(w->wq, c->mtype, QD, H, xn, q);
    orc_matvec(w->wk, c->mtype, KD, H, xn, k);
    orc_matvec(w->wv, c->mtype, KD, H, xn, v);
    for (int h = 0; h < Hq; ++h) {
        if (c->qk_norm) {
            orc_rmsnorm(q + h * D, D, w->q_norm, c->wtype, c->eps, tmp);
            memcpy(q + h * D, tmp, sizeof(float) * (size_t)D);
        }
        orc_rope(q + h * D, D, pos, c->rope_base);
    }
    for (int h = 0; h < Hkv; ++h) {
        if (c->qk_norm) {
            orc_rmsnorm(k + h * D, D, w->k_norm, c->wtype, c->eps, tmp);
            memcpy(k + h * D, tmp, sizeof(float) * (size_t)D);
        }
        orc_rope(k + h * D, D, pos, c->rope_base);
        int64_t off = ((int64_t)h * cap + pos) * D;
        cache_store(kc, c->kvtype, off, k + h * D, D);
        cache_store(vc, c->kvtype, off, v + h * D, D);
    }
    const size_t es = kv_es(c->kvtype);
#pragma omp parallel for schedule(static)
    for (int h = 0; h < Hq; ++h) {
        int hk = (int)(((int64_t)h * Hkv) / Hq);
        const char* Kh = (const char*)kc + (size_t)hk * cap * D * es;
        const char* Vh = (const char*)vc + (size_t)hk * cap * D * es;
        orc_attention_head(q + h * D, Kh, Vh, c->kvtype, pos + 1, D, att + h * D, NULL);
    }
    orc_matvec(w->wo, c->mtype, H, QD, att, y);
    for (int i = 0; i < H; ++i) x[i] = (float)((double)x[i] + (double)y[i]);

    /* MLP block */
    orc_rmsnorm(x, H, w->mlp_norm, c->wtype, c->eps, xn);
    orc_matvec(w->w_gate, c->mtype, F, H, xn, g);
    orc_matvec(w->w_up, c->mtype, F, H, xn, u);
    orc_swiglu(g, u, F, xn);
    orc_matvec(w->w_down, c->mtype, H, F, xn, y);
    for (int i = 0; i < H; ++i) x[i] = (float)((double)x[i] + (double)y[i]);

    free(xn); free(q); free(k); free(v); free(att); free(y); free(g); free(u); free(tmp);
}

/*
 * Whole decode step for one sequence: x = E[token]; every layer; logits =
 * W_lm . RMSNorm(x; final gain). kc, vc: the sequence's cache
 * [n_layers][Hkv][cap][D]. Returns 0, or -1 if token is out of range.
 */
int orc_model_forward(const orc_cfg* c, const void* embed, const orc_layer* layers, const void* final_norm,
                      const void* lm_head, void* kc, void* vc, int cap, int token, int pos, float* logits) {
    const int H = c->hidden;
    if (token < 0 || token >= c->vocab) return -1;
    float* x = (float*)malloc(sizeof(float) * (size_t)H);
    float* xn = (float*)malloc(sizeof(float) * (size_t)H);
    for (int i = 0; i < H; ++i) x[i] = (float)elem(embed, c->wtype, (int64_t)token * H + i);
    const size_t layer_elems = (size_t)c->n_kv_heads * cap * c->head_dim;
    const size_t es = kv_es(c->kvtype);
    for (int l = 0; l < c->n_layers; ++l)
        orc_layer_forward(c, &layers[l], (char*)kc + l * layer_elems * es, (char*)vc + l * layer_elems * es, cap,
                          pos, x);
    orc_rmsnorm(x, H, final_norm, c->wtype, c->eps, xn);
    orc_matvec(lm_head, c->wtype, c->vocab, H, xn, logits);
    free(x);
    free(xn);
    return 0;
}
