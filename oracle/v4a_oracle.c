/*
 * v4a_oracle.c -- plain, slow CPU oracle for the DeepSeek-V4 CSA/HCA attention
 * hot path, in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Every function writes out a definition from the page "CSA And HCA:
 * Definition, State, And Cost Model" (cited below as [Def]) directly: no
 * blocking, no fusion, no online softmax.  Inputs arrive as float64 arrays
 * decoded exactly from the stored formats (decoders at the end of this file,
 * written from the OCP FP8 and MX v1.0 specifications).
 *
 * Readings taken where the pages leave a step open (each is listed in the
 * design notes):
 *   - RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma.
 *   - RoPE on the last rope_dims channels, adjacent pairs (2i, 2i+1) of that
 *     slice, angle = pos * base^(-2i/rope_dims), (x,y) -> (x cos - y sin,
 *     x sin + y cos); the inverse uses -pos.
 *   - Compressed entries are stored already normalised and rotated at their
 *     anchor (m*s for CSA, m'*s for HCA); queries are rotated at t and local
 *     rows at j when attention reads them.
 *   - Top-k ties go to the lower entry index; the selected indices are
 *     returned in ascending order, padded with -1.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* [Def] section 1 (visibility of completed entries) and section 5.1 (window) */
/* ------------------------------------------------------------------------- */

/* Number of completed compressed entries visible to query t for ratio r:
 * the set {s : 0 <= s < floor((t+1)/r)}. */
int64_t v4o_visible_count(int64_t t, int64_t r) { return (t + 1) / r; }

/* Local window L_t = {j : max(0, t-w+1) <= j <= t}. */
void v4o_window(int64_t t, int64_t w, int64_t* lo, int64_t* len) {
    int64_t a = t - w + 1;
    if (a < 0) a = 0;
    *lo = a;
    *len = t - a + 1;
}

/* Per-query sets for queries t0 .. t0+T-1: completed count E_t (ratio m),
 * selected count cnt_t = min(k, E_t) (k <= 0: dense, cnt = E_t), window. */
void v4o_sets(int64_t t0, int64_t T, int64_t m, int64_t k, int64_t w,
              int32_t* E, int32_t* cnt, int32_t* win_lo, int32_t* win_len) {
    for (int64_t j = 0; j < T; ++j) {
        int64_t t = t0 + j, e = v4o_visible_count(t, m), lo, len;
        v4o_window(t, w, &lo, &len);
        E[j] = (int32_t)e;
        cnt[j] = (int32_t)((k > 0 && k < e) ? k : e);
        win_lo[j] = (int32_t)lo;
        win_len[j] = (int32_t)len;
    }
}

/* ------------------------------------------------------------------------- */
/* [Def] section 5.2: RMSNorm and partial RoPE                                */
/* ------------------------------------------------------------------------- */

void v4o_rmsnorm(const double* x, int64_t c, const double* gamma, double eps, double* y) {
    double ss = 0.0;
    for (int64_t i = 0; i < c; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)c + eps);
    for (int64_t i = 0; i < c; ++i) y[i] = x[i] * inv * (gamma ? gamma[i] : 1.0);
}

/* Rotate the last rope_dims channels of x (length c) in place by position pos. */
void v4o_rope(double* x, int64_t c, int64_t rope_dims, double base, double pos) {
    double* r = x + (c - rope_dims);
    for (int64_t i = 0; i < rope_dims / 2; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)rope_dims);
        double ang = pos * theta;
        double cs = cos(ang), sn = sin(ang);
        double a = r[2 * i], b = r[2 * i + 1];
        r[2 * i] = a * cs - b * sn;
        r[2 * i + 1] = a * sn + b * cs;
    }
}

/* ------------------------------------------------------------------------- */
/* [Def] sections 2.1 (CSA, overlapping two streams) and 2.2 (HCA, one stream) */
/* ------------------------------------------------------------------------- */

/*
 * Emit compressed entries i = i_begin .. i_end-1.
 *   C, Z   : [n_buf][width] rows; row r holds absolute token position tok_base + r.
 *            overlap = 1: width = 2c, stream a in columns [0,c), stream b in [c,2c).
 *            overlap = 0: width = c.
 *   B      : [(1+overlap)*m][c] positional bias; rows 0..m-1 are B^a (or B), rows
 *            m..2m-1 are B^b.
 *   For entry i and channel ch, one softmax over positions runs jointly over the
 *   a-stream rows of block i (logit Z^a + B^a) and, when overlap = 1 and i > 0,
 *   the b-stream rows of block i-1 (logit Z^b + B^b).  For i = 0 the b-stream is
 *   absent (weight zero).  The entry is the softmax-weighted sum of the matching
 *   C rows.  Then optional RMSNorm (gamma != NULL) and RoPE at anchor m*i.
 *   out    : [i_end - i_begin][c]
 * Returns 0, or -1 if a needed row is outside the buffer.
 */
int v4o_compress(const double* C, const double* Z, int64_t n_buf, int64_t tok_base,
                 int64_t i_begin, int64_t i_end, int64_t c, int64_t m, int overlap,
                 const double* B, const double* gamma, double eps,
                 int64_t rope_dims, double rope_base, double* out) {
    int64_t width = overlap ? 2 * c : c;
    for (int64_t i = i_begin; i < i_end; ++i) {
        int64_t first = (overlap && i > 0) ? m * (i - 1) : m * i;
        if (first - tok_base < 0 || m * (i + 1) - tok_base > n_buf) return -1;
    }
    int64_t ne = i_end - i_begin;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < ne; ++e) {
        int64_t i = i_begin + e;
        double* row = out + e * c;
        double* logit = (double*)malloc(sizeof(double) * 2 * m);
        double* val = (double*)malloc(sizeof(double) * 2 * m);
        if (!logit || !val) { bad = 1; free(logit); free(val); continue; }
        for (int64_t ch = 0; ch < c; ++ch) {
            int64_t np_ = 0;
            for (int64_t j = 0; j < m; ++j) {              /* stream a: block i */
                int64_t r = m * i + j - tok_base;
                logit[np_] = Z[r * width + ch] + B[j * c + ch];
                val[np_] = C[r * width + ch];
                ++np_;
            }
            if (overlap && i > 0) {
                for (int64_t j = 0; j < m; ++j) {          /* stream b: block i-1 */
                    int64_t r = m * (i - 1) + j - tok_base;
                    logit[np_] = Z[r * width + c + ch] + B[(m + j) * c + ch];
                    val[np_] = C[r * width + c + ch];
                    ++np_;
                }
            }
            double mx = -INFINITY;
            for (int64_t p = 0; p < np_; ++p) if (logit[p] > mx) mx = logit[p];
            double den = 0.0, num = 0.0;
            for (int64_t p = 0; p < np_; ++p) {
                double ex = exp(logit[p] - mx);
                den += ex;
                num += ex * val[p];
            }
            row[ch] = num / den;
        }
        free(logit);
        free(val);
        if (gamma) v4o_rmsnorm(row, c, gamma, eps, row);
        if (rope_dims > 0) v4o_rope(row, c, rope_dims, rope_base, (double)(m * i));
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------- */
/* [Def] section 3.1: lightning-indexer score and top-k                        */
/* ------------------------------------------------------------------------- */

/*
 * I[t][s] = sum_h wI[t][h] * max(0, qI[t][h] . KI[s])  for s < floor((t+1)/m).
 *   qI : [T][n_hI][cI], wI : [T][n_hI], KI : [>=E][cI]; query row j is position t0+j.
 *   scores : [T][ld]; entries s >= E_t are set to NAN.
 */
void v4o_index_scores(const double* qI, const double* KI, const double* wI,
                      int64_t T, int64_t t0, int64_t n_hI, int64_t cI, int64_t m,
                      int64_t ld, double* scores) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < T; ++j) {
        int64_t E = v4o_visible_count(t0 + j, m);
        double* srow = scores + j * ld;
        for (int64_t s = 0; s < ld; ++s) srow[s] = NAN;
        for (int64_t s = 0; s < E && s < ld; ++s) {
            double acc = 0.0;
            for (int64_t h = 0; h < n_hI; ++h) {
                const double* qv = qI + (j * n_hI + h) * cI;
                const double* kv = KI + s * cI;
                double dot = 0.0;
                for (int64_t d = 0; d < cI; ++d) dot += qv[d] * kv[d];
                acc += wI[j * n_hI + h] * (dot > 0.0 ? dot : 0.0);
            }
            srow[s] = acc;
        }
    }
}

typedef struct { double v; int64_t s; } v4o_kv;

/* order: larger score first, then lower index */
static int cmp_desc(const void* a, const void* b) {
    const v4o_kv* x = (const v4o_kv*)a;
    const v4o_kv* y = (const v4o_kv*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/*
 * Top-k over the visible entries of each query: sort s < E_t by (score desc,
 * s asc), keep the first min(k, E_t), return them in ascending s, pad with -1.
 *   scores : [T][ld], idx : [T][k], cnt : [T]
 */
void v4o_topk(const double* scores, int64_t T, int64_t t0, int64_t m, int64_t k,
              int64_t ld, int32_t* idx, int32_t* cnt) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < T; ++j) {
        int64_t E = v4o_visible_count(t0 + j, m);
        if (E > ld) E = ld;
        v4o_kv* buf = (v4o_kv*)malloc(sizeof(v4o_kv) * (E > 0 ? E : 1));
        for (int64_t s = 0; s < E; ++s) { buf[s].v = scores[j * ld + s]; buf[s].s = s; }
        qsort(buf, (size_t)E, sizeof(v4o_kv), cmp_desc);
        int64_t n = E < k ? E : k;
        int32_t* out = idx + j * k;
        for (int64_t r = 0; r < n; ++r) out[r] = (int32_t)buf[r].s;
        qsort(out, (size_t)n, sizeof(int32_t), cmp_i32);
        for (int64_t r = n; r < k; ++r) out[r] = -1;
        cnt[j] = (int32_t)n;
        free(buf);
    }
}

/* ------------------------------------------------------------------------- */
/* [Def] sections 3.2, 4, 5.1-5.3: shared-KV MQA over one candidate list      */
/* ------------------------------------------------------------------------- */

/*
 * One query position t, all heads.  Candidates: ncomp compressed rows (pointers,
 * used as stored) followed by the local rows of the window (raw, normalised with
 * kv_gamma when given and rotated at their own position j).  One softmax per head
 * over the whole list, plus the optional sink logit in the denominator only.
 * Output = sum a * v, then inverse RoPE at t on the last rope_dims channels.
 */
static void attend_one(const double* q_t /*[n_h][c]*/, int64_t t,
                       const double* const* comp, int64_t ncomp,
                       const double* local, int64_t loc_base, int64_t w,
                       const double* sink, const double* q_gamma, const double* kv_gamma,
                       int kv_norm, int q_norm, double eps, int64_t rope_dims, double rope_base,
                       double scale, int64_t n_h, int64_t c, double* out /*[n_h][c]*/) {
    int64_t lo, nl;
    v4o_window(t, w, &lo, &nl);
    int64_t N = ncomp + nl;
    double* cand = (double*)malloc(sizeof(double) * N * c);
    for (int64_t u = 0; u < ncomp; ++u) memcpy(cand + u * c, comp[u], sizeof(double) * c);
    for (int64_t u = 0; u < nl; ++u) {
        int64_t j = lo + u;
        double* dst = cand + (ncomp + u) * c;
        const double* src = local + (j - loc_base) * c;
        if (kv_norm) v4o_rmsnorm(src, c, kv_gamma, eps, dst);
        else memcpy(dst, src, sizeof(double) * c);
        if (rope_dims > 0) v4o_rope(dst, c, rope_dims, rope_base, (double)j);
    }
    double* qp = (double*)malloc(sizeof(double) * c);
    double* z = (double*)malloc(sizeof(double) * N);
    for (int64_t h = 0; h < n_h; ++h) {
        if (q_norm) v4o_rmsnorm(q_t + h * c, c, q_gamma, eps, qp);
        else memcpy(qp, q_t + h * c, sizeof(double) * c);
        if (rope_dims > 0) v4o_rope(qp, c, rope_dims, rope_base, (double)t);
        double mx = sink ? sink[h] : -INFINITY;
        for (int64_t u = 0; u < N; ++u) {
            double d = 0.0;
            for (int64_t i = 0; i < c; ++i) d += qp[i] * cand[u * c + i];
            z[u] = d * scale;
            if (z[u] > mx) mx = z[u];
        }
        double den = sink ? exp(sink[h] - mx) : 0.0;
        for (int64_t u = 0; u < N; ++u) den += exp(z[u] - mx);
        double* o = out + h * c;
        for (int64_t i = 0; i < c; ++i) o[i] = 0.0;
        for (int64_t u = 0; u < N; ++u) {
            double a = exp(z[u] - mx) / den;
            for (int64_t i = 0; i < c; ++i) o[i] += a * cand[u * c + i];
        }
        if (rope_dims > 0) v4o_rope(o, c, rope_dims, rope_base, -(double)t);
    }
    free(cand);
    free(qp);
    free(z);
}

/*
 * CSA attention for query rows of a chunk [t0, t0+T).
 *   q        : [T][n_h][c] raw queries
 *   kv_comp  : [>=E][c] compressed entries as stored (normalised + rotated)
 *   kv_local : [n_loc][c] raw local rows, row r = position loc_base + r
 *   idx, cnt : [T][k], [T] selected entries (from top-k)
 *   rows     : which query rows (0-based within the chunk) to compute; NULL = all
 *   out      : [nrows][n_h][c]
 */
void v4o_attend_csa(const double* q, const double* kv_comp, const double* kv_local,
                    int64_t loc_base, const int32_t* idx, const int32_t* cnt, int64_t k,
                    const double* sink, const double* q_gamma, const double* kv_gamma,
                    int q_norm, int kv_norm, double eps, int64_t rope_dims, double rope_base,
                    double scale, int64_t t0, int64_t n_h, int64_t c, int64_t w,
                    const int64_t* rows, int64_t nrows, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t j = rows ? rows[r] : r;
        int64_t nc = cnt[j];
        const double** comp = (const double**)malloc(sizeof(double*) * (nc > 0 ? nc : 1));
        for (int64_t u = 0; u < nc; ++u) comp[u] = kv_comp + (int64_t)idx[j * k + u] * c;
        attend_one(q + j * n_h * c, t0 + j, comp, nc, kv_local, loc_base, w, sink, q_gamma,
                   kv_gamma, kv_norm, q_norm, eps, rope_dims, rope_base, scale, n_h, c,
                   out + r * n_h * c);
        free(comp);
    }
}

/* HCA attention: compressed candidates are every completed entry s < floor((t+1)/m'). */
void v4o_attend_hca(const double* q, const double* kv_comp, const double* kv_local,
                    int64_t loc_base, const double* sink, const double* q_gamma,
                    const double* kv_gamma, int q_norm, int kv_norm, double eps,
                    int64_t rope_dims, double rope_base, double scale, int64_t t0,
                    int64_t n_h, int64_t c, int64_t m_prime, int64_t w,
                    const int64_t* rows, int64_t nrows, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t j = rows ? rows[r] : r;
        int64_t t = t0 + j;
        int64_t nc = v4o_visible_count(t, m_prime);
        const double** comp = (const double**)malloc(sizeof(double*) * (nc > 0 ? nc : 1));
        for (int64_t u = 0; u < nc; ++u) comp[u] = kv_comp + u * c;
        attend_one(q + j * n_h * c, t, comp, nc, kv_local, loc_base, w, sink, q_gamma,
                   kv_gamma, kv_norm, q_norm, eps, rope_dims, rope_base, scale, n_h, c,
                   out + r * n_h * c);
        free(comp);
    }
}

/*
 * Decode attention at position t for one sequence with a ring of w slots
 * (token j in slot j mod w; the slot of t must already hold token t).
 */
void v4o_attend_decode(const double* q /*[n_h][c]*/, const double* kv_comp,
                       const double* ring /*[w][c]*/, int64_t t, const int32_t* idx,
                       int64_t cnt, const double* sink, const double* q_gamma,
                       const double* kv_gamma, int q_norm, int kv_norm, double eps,
                       int64_t rope_dims, double rope_base, double scale, int64_t n_h,
                       int64_t c, int64_t w, double* out) {
    int64_t lo, nl;
    v4o_window(t, w, &lo, &nl);
    /* unroll the ring into positions lo .. t so attend_one can index by position */
    double* lin = (double*)malloc(sizeof(double) * nl * c);
    for (int64_t u = 0; u < nl; ++u)
        memcpy(lin + u * c, ring + ((lo + u) % w) * c, sizeof(double) * c);
    const double** comp = (const double**)malloc(sizeof(double*) * (cnt > 0 ? cnt : 1));
    for (int64_t u = 0; u < cnt; ++u) comp[u] = kv_comp + (int64_t)idx[u] * c;
    attend_one(q, t, comp, cnt, lin, lo, w, sink, q_gamma, kv_gamma, kv_norm, q_norm, eps,
               rope_dims, rope_base, scale, n_h, c, out);
    free(comp);
    free(lin);
}

/* ------------------------------------------------------------------------- */
/* Exact decoders of the stored formats (OCP OFP8 v1.0, OCP MX v1.0)         */
/* ------------------------------------------------------------------------- */

void v4o_decode_bf16(const uint16_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)in[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        out[i] = (double)f;
    }
}

/* E4M3: sign | 4-bit exponent (bias 7) | 3-bit mantissa; exponent 0 is subnormal
 * (mantissa * 2^-9); S.1111.111 is NaN; no infinities. */
static double e4m3_value(uint8_t b) {
    int sgn = b >> 7, e = (b >> 3) & 15, mnt = b & 7;
    double v;
    if (e == 15 && mnt == 7) return NAN;
    if (e == 0) v = ldexp((double)mnt, -9);
    else v = ldexp(1.0 + mnt / 8.0, e - 7);
    return sgn ? -v : v;
}

/* codes [rows][cols] with one float32 scale per row (scale may be NULL: 1.0). */
void v4o_decode_fp8_rows(const uint8_t* codes, const float* scale, int64_t rows,
                         int64_t cols, double* out) {
    for (int64_t r = 0; r < rows; ++r) {
        double s = scale ? (double)scale[r] : 1.0;
        for (int64_t i = 0; i < cols; ++i) out[r * cols + i] = e4m3_value(codes[r * cols + i]) * s;
    }
}

/* E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent 0 is 0 or 0.5. */
static double e2m1_value(uint8_t nib) {
    int sgn = (nib >> 3) & 1, e = (nib >> 1) & 3, mnt = nib & 1;
    double v = (e == 0) ? 0.5 * mnt : ldexp(1.0 + 0.5 * mnt, e - 1);
    return sgn ? -v : v;
}

/* packed [rows][cols/2] (element 2j low nibble, 2j+1 high nibble),
 * e8m0 [rows][cols/32] (value 2^(code-127), code 255 = NaN). */
void v4o_decode_mxfp4_rows(const uint8_t* packed, const uint8_t* e8m0, int64_t rows,
                           int64_t cols, double* out) {
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < cols; ++i) {
            uint8_t byte = packed[r * (cols / 2) + i / 2];
            uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 15);
            uint8_t sc = e8m0[r * (cols / 32) + i / 32];
            double s = (sc == 255) ? NAN : ldexp(1.0, (int)sc - 127);
            out[r * cols + i] = e2m1_value(nib) * s;
        }
    }
}

int v4o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
