/*
 * zha_oracle.c -- plain fp64 CPU reference ("oracle") of the ZHA decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP implementation, and the HIP
 * implementation never calls it.
 *
 * Page references used below (each is one of the web pages describing
 * Zyphra Hierarchical Attention, cited by site and section heading):
 *   [wqu]   wqu.guru, "Zyphra发布层级注意力ZHA：稀疏搜索实现亚二次复杂度"
 *   [flux]  fluxbbs.com, "Zyphra ZHA 稀疏注意力：8.2 万参数与 373 倍加速推算"
 *   [aitop] aitop.news, "Zyphra 提出树结构索引器 ZHA，实现亚二次复杂度长上下文注意力"
 *           (carries the paper's abstract)
 *   [icwork] ic.work article on ZHA
 *
 * Conventions (readings of the pages, all fixed here once):
 *   - Everything is one (sequence, KV head) unit: keys K[N][d], values V[N][d],
 *     reference queries refs[R][d] shared by every level, and the G query
 *     heads q[G][d] of that KV head, already multiplied by the logit scale.
 *   - Level 1 nodes are leaf chunks of C consecutive raw tokens; a level-l node
 *     covers C^l tokens; only complete leaf chunks enter the tree, so the tree
 *     spans Nc = C*floor(N/C) tokens and the last node of a level may be
 *     partial.  Node j of level l covers [j*C^l, min((j+1)*C^l, Nc)).
 *   - A node's summary is one tangent plane per reference query r:
 *     LSE_r = log sum_t exp(r.k_t), m_r = sum_t softmax_t(r.k) k_t,
 *     b_r = LSE_r - r.m_r; the node's score for a query q is
 *     max_r (b_r + q.m_r)  ([wqu] "Building the tree": each reference query
 *     gives a tangent-plane estimate of the chunk's log attention mass and the
 *     maximum over the planes is the estimate).
 *   - Routing is top-down with a per-level top-p over the estimated mass
 *     ([wqu] "How does top-p routing pick tokens?"; [flux] tree section).
 *     The G heads of one KV head share one kept set: the mass of a node is the
 *     mean over heads of each head's frontier-normalised mass.
 *   - The attention set is token 0 (the sink), the tokens of the kept leaf
 *     chunks and the trailing partial chunk [Nc, N); a query of a block of
 *     queries after the N cached tokens also reads the block's rows up to its
 *     own position.
 *
 * Every floating-point quantity is double.  OpenMP only splits independent
 * outputs across threads; each output is computed by one thread in a fixed
 * order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ZO_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------ helpers */

static double zo_dot(const double* a, const double* b, int d)
{
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += a[i] * b[i];
    return s;
}

static int64_t zo_ipow(int64_t base, int e)
{
    int64_t r = 1;
    for (int i = 0; i < e; ++i) r *= base;
    return r;
}

ZO_EXPORT int zo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

ZO_EXPORT void zo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Tokens covered by the tree: complete leaf chunks only. */
ZO_EXPORT int64_t zo_tree_tokens(int64_t N, int C)
{
    return (N / C) * C;
}

/* Number of nodes at level l (1-based): ceil(Nc / C^l). */
ZO_EXPORT int64_t zo_level_nodes(int64_t N, int C, int l)
{
    int64_t Nc = zo_tree_tokens(N, C);
    int64_t span = zo_ipow(C, l);
    return (Nc + span - 1) / span;
}

/* -------------------------------------------------------- tree, by definition */

/*
 * Planes of the node covering tokens [t0, t1) (t1 > t0), straight from the
 * definition: for each reference query r,
 *   LSE_r = log sum_t exp(r.k_t)        (computed with the maximum subtracted)
 *   m_r   = sum_t exp(r.k_t - LSE_r) k_t
 *   b_r   = LSE_r - r.m_r
 * ([wqu] "Building the tree"; [flux] tree section: summaries come from the
 * reference queries' tangent-plane estimates of the chunk's log mass.)
 */
ZO_EXPORT void zo_node_planes(const double* K, int d, int64_t t0, int64_t t1,
                              const double* refs, int R,
                              double* m /*[R][d]*/, double* b /*[R]*/, double* lse /*[R]*/)
{
    for (int r = 0; r < R; ++r) {
        const double* rv = refs + (int64_t)r * d;
        double mx = -INFINITY;
        for (int64_t t = t0; t < t1; ++t) {
            double x = zo_dot(rv, K + t * d, d);
            if (x > mx) mx = x;
        }
        double s = 0.0;
        for (int64_t t = t0; t < t1; ++t) s += exp(zo_dot(rv, K + t * d, d) - mx);
        double L = mx + log(s);
        double* mr = m + (int64_t)r * d;
        for (int i = 0; i < d; ++i) mr[i] = 0.0;
        for (int64_t t = t0; t < t1; ++t) {
            double w = exp(zo_dot(rv, K + t * d, d) - L);
            for (int i = 0; i < d; ++i) mr[i] += w * K[t * d + i];
        }
        lse[r] = L;
        b[r] = L - zo_dot(rv, mr, d);
    }
}

/*
 * Whole tree by definition.  Levels are stored one after the other: level l
 * starts at node offset sum_{l' < l} n_{l'}; m_out is [nodes][R][d], b_out and
 * lse_out are [nodes][R].
 */
ZO_EXPORT void zo_tree_definition(const double* K, int64_t N, int d, const double* refs, int R,
                                  int C, int L, double* m_out, double* b_out, double* lse_out)
{
    int64_t Nc = zo_tree_tokens(N, C);
    int64_t off = 0;
    for (int l = 1; l <= L; ++l) {
        int64_t n = zo_level_nodes(N, C, l);
        int64_t span = zo_ipow(C, l);
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t j = 0; j < n; ++j) {
            int64_t t0 = j * span;
            int64_t t1 = (j + 1) * span < Nc ? (j + 1) * span : Nc;
            int64_t o = off + j;
            zo_node_planes(K, d, t0, t1, refs, R, m_out + o * R * d, b_out + o * R, lse_out + o * R);
        }
        off += n;
    }
}

/*
 * Whole tree by recursion: leaf chunks by definition, every parent by the
 * exact log-sum-exp combination of its children at the same reference query
 * ([aitop] abstract: the tree is built from recursively compressed key
 * summaries).  With LSE_c the children's log masses and m_c their mean keys:
 *   LSE_P = log sum_c exp(LSE_c),  m_P = sum_c exp(LSE_c - LSE_P) m_c,
 *   b_P = LSE_P - r.m_P.
 * Equal to zo_tree_definition in exact arithmetic; kept separate so the two
 * constructions check each other.
 */
ZO_EXPORT void zo_tree_merge(const double* K, int64_t N, int d, const double* refs, int R,
                             int C, int L, double* m_out, double* b_out, double* lse_out)
{
    int64_t Nc = zo_tree_tokens(N, C);
    int64_t n1 = zo_level_nodes(N, C, 1);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < n1; ++j) {
        int64_t t1 = (j + 1) * C < Nc ? (j + 1) * C : Nc;
        zo_node_planes(K, d, j * C, t1, refs, R, m_out + j * R * d, b_out + j * R, lse_out + j * R);
    }
    int64_t child_off = 0, off = n1;
    for (int l = 2; l <= L; ++l) {
        int64_t n = zo_level_nodes(N, C, l);
        int64_t nchild = zo_level_nodes(N, C, l - 1);
        #pragma omp parallel for schedule(dynamic, 4)
        for (int64_t j = 0; j < n; ++j) {
            int64_t c0 = j * C, c1 = (j + 1) * C < nchild ? (j + 1) * C : nchild;
            for (int r = 0; r < R; ++r) {
                const double* rv = refs + (int64_t)r * d;
                double mx = -INFINITY;
                for (int64_t c = c0; c < c1; ++c) {
                    double x = lse_out[(child_off + c) * R + r];
                    if (x > mx) mx = x;
                }
                double s = 0.0;
                for (int64_t c = c0; c < c1; ++c) s += exp(lse_out[(child_off + c) * R + r] - mx);
                double LP = mx + log(s);
                double* mp = m_out + ((off + j) * R + r) * d;
                for (int i = 0; i < d; ++i) mp[i] = 0.0;
                for (int64_t c = c0; c < c1; ++c) {
                    double w = exp(lse_out[(child_off + c) * R + r] - LP);
                    const double* mc = m_out + ((child_off + c) * R + r) * d;
                    for (int i = 0; i < d; ++i) mp[i] += w * mc[i];
                }
                lse_out[(off + j) * R + r] = LP;
                b_out[(off + j) * R + r] = LP - zo_dot(rv, mp, d);
            }
        }
        child_off = off;
        off += n;
    }
}

/* ------------------------------------------------------------------ routing */

/* ------------------------------------------------------- fp8 router summaries
 *
 * Optional low-precision storage of the planes' m ([wqu] opening bullets: a
 * router variant in a 4-bit format was also tested; the pages name no format;
 * this is the 8-bit reading).  The grid is OCP fp8 e4m3: sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; normal values (1 + f/8) 2^(e-7) for biased e in
 * 1..15 up to 448 = 1.75 * 2^8 (code 0x7F is not a number), subnormals f * 2^-9.
 * A row of m (one node, one reference query) is stored as grid values times a
 * power of two 2^s, s the smallest integer with max|m| 2^-s <= 448, each value
 * rounded to the nearest grid value, ties to the value whose last mantissa bit
 * is 0.  b = LSE - r.m~ is formed from the stored m~, as for any storage.
 */

/* Nearest e4m3 grid value to x (|x| <= 448), ties to even mantissa. */
ZO_EXPORT double zo_e4m3_round(double x)
{
    const double a = fabs(x);
    double step;
    if (a < ldexp(1.0, -6)) {
        step = ldexp(1.0, -9);                 /* subnormal spacing */
    } else {
        int e;
        frexp(a, &e);                          /* a = f 2^e, f in [0.5, 1): binade 2^(e-1) */
        step = ldexp(1.0, (e - 1) - 3);        /* three mantissa bits */
    }
    const double n = a / step;                 /* exact: step is a power of two */
    double r = floor(n);
    const double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    const double v = r * step;
    return x < 0 ? -v : v;
}

/* Scale exponent s of a row with largest magnitude amax: the smallest integer
 * with amax 2^-s <= 448 (0 for an all-zero row). */
ZO_EXPORT int zo_e4m3_row_exp(double amax)
{
    if (!(amax > 0.0)) return 0;
    int e;
    frexp(amax, &e);
    int s = e - 12;                            /* amax 2^-s >= 2^11 > 448 */
    while (ldexp(amax, -s) > 448.0) ++s;
    return s;
}

/* Stores n rows of d values as fp8 summaries: out = grid value * 2^s per row,
 * scale[i] = 2^s_i. */
ZO_EXPORT void zo_fp8_rows(const double* m, int64_t n, int d, double* out, double* scale)
{
    for (int64_t i = 0; i < n; ++i) {
        double amax = 0.0;
        for (int k = 0; k < d; ++k) amax = fmax(amax, fabs(m[i * d + k]));
        const int sx = zo_e4m3_row_exp(amax);
        for (int k = 0; k < d; ++k) out[i * d + k] = ldexp(zo_e4m3_round(ldexp(m[i * d + k], -sx)), sx);
        scale[i] = ldexp(1.0, sx);
    }
}

/* Planes of n nodes with fp8-stored means.  m [n][R][d] and lse [n][R] are a
 * node's exact means and log-sum-exps; mq receives the stored means (one scale
 * per (node, reference) row, scale [n][R]) and b = LSE - r.m~ is formed from the
 * stored mq, so every plane still equals LSE exactly at q = r. */
ZO_EXPORT void zo_fp8_planes(const double* m, const double* lse, const double* refs, int64_t n, int R, int d,
                             double* mq, double* b, double* scale)
{
    zo_fp8_rows(m, n * R, d, mq, scale);
    for (int64_t i = 0; i < n; ++i)
        for (int r = 0; r < R; ++r)
            b[i * R + r] = lse[i * R + r] - zo_dot(refs + (int64_t)r * d, mq + (i * R + r) * d, d);
}

/* ------------------------------------------------------- fp4 router summaries
 *
 * The 4-bit reading of the same passage ([wqu] opening bullets).  The grid is
 * OCP fp4 e2m1: sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes
 * 0 and 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6.  Four bits cannot hold a whole row
 * under one scale, so a row of m is cut into blocks of 32 consecutive values,
 * each stored as grid values times a power of two 2^s, s the smallest integer
 * with max|m_block| 2^-s <= 6; each value rounded to the nearest grid value,
 * ties to the value whose mantissa bit is 0.  b = LSE - r.m~ from the stored m~.
 */

/* Nearest e2m1 grid value to x (|x| <= 6), ties to even mantissa. */
ZO_EXPORT double zo_e2m1_round(double x)
{
    const double a = fabs(x);
    const double step = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);   /* spacing of the binade */
    const double n = a / step;
    double r = floor(n);
    const double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    const double v = r * step;
    return x < 0 ? -v : v;
}

/* Scale exponent s of a block with largest magnitude amax: the smallest integer
 * with amax 2^-s <= 6 (0 for an all-zero block). */
ZO_EXPORT int zo_e2m1_block_exp(double amax)
{
    if (!(amax > 0.0)) return 0;
    int e;
    frexp(amax, &e);
    int s = e - 4;                             /* amax 2^-s >= 2^3 > 6 */
    while (ldexp(amax, -s) > 6.0) ++s;
    return s;
}

/* Stores n rows of d values (d a multiple of 32) as fp4 summaries: out = grid
 * value * 2^s per block of 32, scale[i][k / 32] = 2^s. */
ZO_EXPORT void zo_fp4_rows(const double* m, int64_t n, int d, double* out, double* scale)
{
    const int nb = d / 32;
    for (int64_t i = 0; i < n; ++i)
        for (int blk = 0; blk < nb; ++blk) {
            const double* mb = m + i * d + blk * 32;
            double amax = 0.0;
            for (int k = 0; k < 32; ++k) amax = fmax(amax, fabs(mb[k]));
            const int sx = zo_e2m1_block_exp(amax);
            for (int k = 0; k < 32; ++k) out[i * d + blk * 32 + k] = ldexp(zo_e2m1_round(ldexp(mb[k], -sx)), sx);
            scale[i * nb + blk] = ldexp(1.0, sx);
        }
}

/* Planes of n nodes with fp4-stored means (scale [n][R][d/32], one per block of
 * 32 values); b = LSE - r.m~ from the stored means, as for fp8. */
ZO_EXPORT void zo_fp4_planes(const double* m, const double* lse, const double* refs, int64_t n, int R, int d,
                             double* mq, double* b, double* scale)
{
    zo_fp4_rows(m, n * R, d, mq, scale);
    for (int64_t i = 0; i < n; ++i)
        for (int r = 0; r < R; ++r) {
            const double* stored = mq + (i * R + r) * d;
            b[i * R + r] = lse[i * R + r] - zo_dot(refs + (int64_t)r * d, stored, d);
        }
}

/* Node score for head h: the maximum over the R tangent planes (query pre-scaled). */
static double zo_score(const double* m_node, const double* b_node, int R, int d, const double* qh)
{
    double best = -INFINITY;
    for (int r = 0; r < R; ++r) {
        double v = b_node[r] + zo_dot(qh, m_node + (int64_t)r * d, d);
        if (v > best) best = v;
    }
    return best;
}

typedef struct { double w; int32_t id; int64_t pos; } zo_rank_t;

/* Order: estimated mass descending, node id ascending on equal mass. */
static int zo_rank_cmp(const void* pa, const void* pb)
{
    const zo_rank_t* a = (const zo_rank_t*)pa;
    const zo_rank_t* b = (const zo_rank_t*)pb;
    if (a->w > b->w) return -1;
    if (a->w < b->w) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

static int zo_i32_cmp(const void* pa, const void* pb)
{
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/*
 * One routing level ([wqu] "How does top-p routing pick tokens?": keep the
 * smallest node set holding a fraction p of the estimated attention mass).
 *
 * m_l/b_l: the level's planes indexed by node id ([n][R][d], [n][R]).
 * F[nF]: frontier node ids.  q[G][d]: the KV head's query heads, pre-scaled.
 *   s_{h,i} = max_r (b_{i,r} + q_h . m_{i,r})
 *   pi_{h,i} = exp(s_{h,i} - logsumexp_{j in F} s_{h,j})
 *   w_i = (1/G) sum_h pi_{h,i}
 * Sort F by (w desc, id asc); c_k = running sum in that order; W = c_nF;
 * k* = min{k : c_k >= p W} (k* = nF when p >= 1).  The kept set is the first
 * k* nodes of that order, returned sorted by id.
 *
 * Optional outputs: w_out[nF] (frontier order), order_out[nF] (frontier
 * positions in sorted order), csum_out[nF] (c_1..c_nF).  Returns k*.
 */
ZO_EXPORT int64_t zo_select(const double* m_l, const double* b_l, int R, int d,
                            const double* q, int G, const int32_t* F, int64_t nF, double p,
                            int32_t* kept_out, double* w_out, int64_t* order_out, double* csum_out)
{
    if (nF <= 0) return 0;
    double* s = (double*)malloc(sizeof(double) * (size_t)G * (size_t)nF);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nF; ++i) {
        const double* mn = m_l + (int64_t)F[i] * R * d;
        const double* bn = b_l + (int64_t)F[i] * R;
        for (int h = 0; h < G; ++h) s[(int64_t)h * nF + i] = zo_score(mn, bn, R, d, q + (int64_t)h * d);
    }
    double* lse = (double*)malloc(sizeof(double) * (size_t)G);
    for (int h = 0; h < G; ++h) {
        double mx = -INFINITY;
        for (int64_t i = 0; i < nF; ++i) if (s[(int64_t)h * nF + i] > mx) mx = s[(int64_t)h * nF + i];
        double acc = 0.0;
        for (int64_t i = 0; i < nF; ++i) acc += exp(s[(int64_t)h * nF + i] - mx);
        lse[h] = mx + log(acc);
    }
    zo_rank_t* rk = (zo_rank_t*)malloc(sizeof(zo_rank_t) * (size_t)nF);
    for (int64_t i = 0; i < nF; ++i) {
        double w = 0.0;
        for (int h = 0; h < G; ++h) w += exp(s[(int64_t)h * nF + i] - lse[h]);
        w /= (double)G;
        rk[i].w = w;
        rk[i].id = F[i];
        rk[i].pos = i;
        if (w_out) w_out[i] = w;
    }
    qsort(rk, (size_t)nF, sizeof(zo_rank_t), zo_rank_cmp);
    double* c = (double*)malloc(sizeof(double) * (size_t)nF);
    double run = 0.0;
    for (int64_t k = 0; k < nF; ++k) { run += rk[k].w; c[k] = run; }
    double W = c[nF - 1];
    int64_t kstar = nF;
    if (p < 1.0) {
        for (int64_t k = 0; k < nF; ++k) {
            if (c[k] >= p * W) { kstar = k + 1; break; }
        }
    }
    for (int64_t k = 0; k < kstar; ++k) kept_out[k] = rk[k].id;
    qsort(kept_out, (size_t)kstar, sizeof(int32_t), zo_i32_cmp);
    if (order_out) for (int64_t k = 0; k < nF; ++k) order_out[k] = rk[k].pos;
    if (csum_out) for (int64_t k = 0; k < nF; ++k) csum_out[k] = c[k];
    free(c); free(rk); free(lse); free(s);
    return kstar;
}

/*
 * Children of a sorted kept list at level l, as the level-(l-1) frontier
 * (ascending ids).  Only existing children (id < n_child) are listed.
 */
ZO_EXPORT int64_t zo_expand(const int32_t* kept, int64_t nK, int C, int64_t n_child, int32_t* F_out)
{
    int64_t n = 0;
    for (int64_t k = 0; k < nK; ++k)
        for (int c = 0; c < C; ++c) {
            int64_t id = (int64_t)kept[k] * C + c;
            if (id < n_child) F_out[n++] = (int32_t)id;
        }
    return n;
}

/*
 * Full top-down route of one unit ([wqu] "How does top-p routing pick
 * tokens?": score the top nodes, keep the smallest set holding mass p, expand
 * only those nodes' children and repeat down to the raw entries).
 *
 * m_all/b_all: the tree in the level-after-level layout of zo_tree_definition.
 * F_out/K_out: per level, concatenated in the same node-offset layout
 * (level l's slots start at the level's node offset); nF_out[l-1]/nK_out[l-1]
 * hold the counts.  Level L's frontier is every level-L node.
 */
ZO_EXPORT void zo_route(const double* m_all, const double* b_all, int64_t N, int d, int R, int C, int L,
                        const double* q, int G, double p,
                        int32_t* F_out, int64_t* nF_out, int32_t* K_out, int64_t* nK_out)
{
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L + 2));
    off[1] = 0;
    for (int l = 1; l <= L; ++l) off[l + 1] = off[l] + zo_level_nodes(N, C, l);
    int64_t nL = zo_level_nodes(N, C, L);
    for (int64_t j = 0; j < nL; ++j) F_out[off[L] + j] = (int32_t)j;
    int64_t nF = nL;
    for (int l = L; l >= 1; --l) {
        nF_out[l - 1] = nF;
        int64_t nK = zo_select(m_all + off[l] * R * d, b_all + off[l] * R, R, d, q, G,
                               F_out + off[l], nF, p, K_out + off[l], NULL, NULL, NULL);
        nK_out[l - 1] = nK;
        if (l > 1) nF = zo_expand(K_out + off[l], nK, C, zo_level_nodes(N, C, l - 1), F_out + off[l - 1]);
    }
    free(off);
}

/* ---------------------------------------------------------------- attention */

/*
 * Attention set of one unit: {0} (the sink, [wqu] "How does top-p routing pick
 * tokens?": the first token is always kept), the tokens of the kept leaf
 * chunks, and the trailing partial chunk [Nc, N).  Sorted, no duplicates.
 * tokens_out must hold N entries.  Returns |S|.
 */
ZO_EXPORT int64_t zo_attend_set(int64_t N, int C, const int32_t* kept, int64_t nK, int64_t* tokens_out)
{
    if (N <= 0) return 0;
    unsigned char* in = (unsigned char*)calloc((size_t)N, 1);
    int64_t Nc = zo_tree_tokens(N, C);
    in[0] = 1;
    for (int64_t k = 0; k < nK; ++k)
        for (int c = 0; c < C; ++c) {
            int64_t t = (int64_t)kept[k] * C + c;
            if (t < Nc) in[t] = 1;
        }
    for (int64_t t = Nc; t < N; ++t) in[t] = 1;
    int64_t n = 0;
    for (int64_t t = 0; t < N; ++t) if (in[t]) tokens_out[n++] = t;
    free(in);
    return n;
}

/*
 * Attention set of query t of a block of queries standing at positions N, N+1, ...
 * right after a cache of N tokens (a prefill chunk, or the drafts of a speculative
 * verification step): the decode set over the N cached tokens (token 0, the kept
 * chunks, the partial chunk [Nc, N)) and the block's own rows N .. N+t, no later one.
 * Reading: every query of the block descends the tree as it stood before the block
 * ([aitop] abstract: later queries traverse the tree from the top; [flux]
 * "树形索引是怎么搭的": routing plus attention per query is sublinear, so a whole
 * sequence is subquadratic), and attention is causal.  tokens_out holds N + t + 1
 * entries at most.
 */
ZO_EXPORT int64_t zo_block_attend_set(int64_t N, int C, const int32_t* kept, int64_t nK, int64_t t,
                                      int64_t* tokens_out)
{
    int64_t E = N + t + 1;          /* positions 0 .. N+t may be read */
    if (N < 0 || t < 0) return 0;
    unsigned char* in = (unsigned char*)calloc((size_t)E, 1);
    int64_t Nc = zo_tree_tokens(N, C);
    in[0] = 1;
    for (int64_t k = 0; k < nK; ++k)
        for (int c = 0; c < C; ++c) {
            int64_t x = (int64_t)kept[k] * C + c;
            if (x < Nc) in[x] = 1;
        }
    for (int64_t x = Nc; x < E; ++x) in[x] = 1;
    int64_t n = 0;
    for (int64_t x = 0; x < E; ++x) if (in[x]) tokens_out[n++] = x;
    free(in);
    return n;
}

/*
 * Exact softmax attention of the G heads over the token set S:
 *   lse_h = log sum_{t in S} exp(q_h . k_t),  out_h = sum_{t in S} exp(q_h . k_t - lse_h) v_t.
 * ([wqu] "What is Zyphra Hierarchical Attention (ZHA)?": the full KV cache is
 * kept and exact attention reads only the selected raw entries.)
 */
ZO_EXPORT void zo_attend(const double* q, int G, int d, const double* K, const double* V,
                         const int64_t* S, int64_t nS, double* out /*[G][d]*/, double* lse /*[G]*/)
{
    #pragma omp parallel for schedule(static)
    for (int h = 0; h < G; ++h) {
        const double* qh = q + (int64_t)h * d;
        double mx = -INFINITY;
        for (int64_t i = 0; i < nS; ++i) {
            double x = zo_dot(qh, K + S[i] * d, d);
            if (x > mx) mx = x;
        }
        double s = 0.0;
        for (int64_t i = 0; i < nS; ++i) s += exp(zo_dot(qh, K + S[i] * d, d) - mx);
        double L = mx + log(s);
        double* o = out + (int64_t)h * d;
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        for (int64_t i = 0; i < nS; ++i) {
            double w = exp(zo_dot(qh, K + S[i] * d, d) - L);
            for (int j = 0; j < d; ++j) o[j] += w * V[S[i] * d + j];
        }
        lse[h] = L;
    }
}

/*
 * The same attention computed block by block with the running-maximum
 * (online softmax) merge of partial results; a second construction of
 * zo_attend used to cross-check it.
 */
ZO_EXPORT void zo_attend_blockwise(const double* q, int G, int d, const double* K, const double* V,
                                   const int64_t* S, int64_t nS, int64_t block,
                                   double* out, double* lse)
{
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    for (int h = 0; h < G; ++h) {
        const double* qh = q + (int64_t)h * d;
        double M = -INFINITY, Z = 0.0;
        for (int j = 0; j < d; ++j) acc[j] = 0.0;
        for (int64_t b0 = 0; b0 < nS; b0 += block) {
            int64_t b1 = b0 + block < nS ? b0 + block : nS;
            double bm = -INFINITY;
            for (int64_t i = b0; i < b1; ++i) {
                double x = zo_dot(qh, K + S[i] * d, d);
                if (x > bm) bm = x;
            }
            double newM = M > bm ? M : bm;
            double f = exp(M - newM);
            Z *= f;
            for (int j = 0; j < d; ++j) acc[j] *= f;
            for (int64_t i = b0; i < b1; ++i) {
                double e = exp(zo_dot(qh, K + S[i] * d, d) - newM);
                Z += e;
                for (int j = 0; j < d; ++j) acc[j] += e * V[S[i] * d + j];
            }
            M = newM;
        }
        for (int j = 0; j < d; ++j) out[(int64_t)h * d + j] = acc[j] / Z;
        lse[h] = M + log(Z);
    }
    free(acc);
}
