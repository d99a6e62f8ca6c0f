/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the hierarchical
 * locality-preserving attention path (cube reorder, 3D RoPE with temporal
 * scale r_t, asymmetric global-local attention, cube unorder).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or constant with the HIP library; every constant here
 * is re-derived from the definitions below.
 *
 * Sources (web pages; cited by title and section):
 *   [TS]  "Technische Samenvatting: AtlasVid" (gist.science, Dutch).
 *         Sections used: Probleemstelling; Methodologie 1 "Ontkoppeld
 *         Tweestapsproces" (Fase 1, Fase 2); Methodologie 2 "Efficiente
 *         Gezamenlijke Denoising" (Asymmetrische Hierarchische Attention,
 *         Positie-uitlijning).  The French and Portuguese pages of the same
 *         site carry translations of the same summary.
 *   [AB]  "AtlasVid: Efficient Ultra-High-Resolution Long Video Generation
 *         via Decoupled Global-Local Modeling" (arxivdaily), English abstract.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - cubes are enumerated in raster order (t, then h, then w) over the cube
 *     grid, and tokens inside a cube in raster order too;
 *   - head_dim is split into D/2 - 2*floor(D/6) temporal pairs followed by
 *     floor(D/6) height pairs and floor(D/6) width pairs; pair i holds the
 *     adjacent elements (2i, 2i+1); axis a with n_a pairs uses the frequency
 *     ladder theta^(-j/n_a), j = 0..n_a-1;
 *   - a global token at raster position (tg, hg, wg) of the proxy grid sits at
 *     RoPE coordinates (r_t*tg, (H/Hg)*hg, (W/Wg)*wg); detail tokens sit at
 *     their integer (t, h, w);
 *   - a detail query sees every key of its own cube plus ALL global keys, a
 *     global query sees all global keys and nothing else, both through one
 *     softmax with scale 1/sqrt(D) unless another scale is given.
 *
 * Tensor layout everywhere: [tokens][heads][D], row-major, contiguous.
 * Boundary dtypes: 0 = bf16 (raw 16-bit patterns), 1 = fp32, 2 = fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F64 = 2 };

/* ---- element access ---------------------------------------------------- */

static double orc_ld(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    if (dtype == ORC_F32)
        return (double)((const float *)base)[i];
    return ((const double *)base)[i];
}

/* Round an fp64 value to the nearest bf16, ties to even, straight from the
 * exact value (no detour through fp32, which could round twice).  bf16 keeps
 * 8 significant bits and fp32's exponent range (normal min 2^-126, subnormal
 * quantum 2^-133, largest finite (2 - 2^-7) * 2^127). */
uint16_t orc_round_bf16(double x)
{
    uint32_t bits;
    float f;
    if (isnan(x)) {
        return 0x7FC0;
    }
    if (x == 0.0) {
        return signbit(x) ? 0x8000 : 0x0000;
    }
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                 /* ax = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                 /* quantum of an 8-bit significand */
    if (q < -133)
        q = -133;                  /* subnormal range */
    double scaled = ldexp(ax, -q); /* exact: power-of-two scaling */
    double r = nearbyint(scaled);  /* default rounding mode: ties to even */
    double y = ldexp(r, q);
    if (y >= ldexp(1.0, 128))
        y = INFINITY;
    f = (float)y;                  /* exact: y is representable in bf16 */
    memcpy(&bits, &f, 4);
    uint16_t h = (uint16_t)(bits >> 16);
    if (signbit(x))
        h |= 0x8000;
    return h;
}

/* Element-wise orc_round_bf16 over an array. */
void orc_round_bf16_array(uint16_t *out, const double *x, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_round_bf16(x[i]);
}

/* ---- O1: cube permutation ----------------------------------------------
 * [TS] Methodologie 1, Fase 2: the latent volume T x H x W is cut into
 * spatiotemporal cubes and the tokens are reordered so that the tokens of one
 * cube are contiguous.  Cube-order position p maps to raster index pi(p). */

int64_t orc_cube_src(int64_t p, int64_t T, int64_t H, int64_t W,
                     int64_t ct, int64_t ch, int64_t cw)
{
    (void)T;
    int64_t nH = H / ch, nW = W / cw;
    int64_t V = ct * ch * cw;
    int64_t c = p / V, o = p % V;
    int64_t a = c / (nH * nW), b = (c / nW) % nH, e = c % nW;
    int64_t dt = o / (ch * cw), dh = (o / cw) % ch, dw = o % cw;
    int64_t t = a * ct + dt, h = b * ch + dh, w = e * cw + dw;
    return (t * H + h) * W + w;
}

/* Inverse of orc_cube_src: raster index r -> cube-order position p. */
int64_t orc_cube_dst(int64_t r, int64_t T, int64_t H, int64_t W,
                     int64_t ct, int64_t ch, int64_t cw)
{
    (void)T;
    int64_t nH = H / ch, nW = W / cw;
    int64_t V = ct * ch * cw;
    int64_t t = r / (H * W), h = (r / W) % H, w = r % W;
    int64_t a = t / ct, dt = t % ct;
    int64_t b = h / ch, dh = h % ch;
    int64_t e = w / cw, dw = w % cw;
    int64_t c = (a * nH + b) * nW + e;
    int64_t o = (dt * ch + dh) * cw + dw;
    return c * V + o;
}

void orc_cube_perm(int64_t *pi, int64_t T, int64_t H, int64_t W,
                   int64_t ct, int64_t ch, int64_t cw)
{
    int64_t N = T * H * W;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < N; ++p)
        pi[p] = orc_cube_src(p, T, H, W, ct, ch, cw);
}

/* reorder: dst[p] = src[pi(p)], one token row (row_bytes bytes) per token */
void orc_cube_reorder(void *dst, const void *src, int64_t row_bytes,
                      int64_t T, int64_t H, int64_t W,
                      int64_t ct, int64_t ch, int64_t cw)
{
    int64_t N = T * H * W;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < N; ++p) {
        int64_t r = orc_cube_src(p, T, H, W, ct, ch, cw);
        memcpy((char *)dst + p * row_bytes, (const char *)src + r * row_bytes,
               (size_t)row_bytes);
    }
}

/* unorder: dst[pi(p)] = src[p] */
void orc_cube_unorder(void *dst, const void *src, int64_t row_bytes,
                      int64_t T, int64_t H, int64_t W,
                      int64_t ct, int64_t ch, int64_t cw)
{
    int64_t N = T * H * W;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < N; ++p) {
        int64_t r = orc_cube_src(p, T, H, W, ct, ch, cw);
        memcpy((char *)dst + r * row_bytes, (const char *)src + p * row_bytes,
               (size_t)row_bytes);
    }
}

/* ---- O2: 3D RoPE --------------------------------------------------------
 * [TS] Methodologie 1, Fase 1: temporal RoPE indices of the proxy are
 * multiplied by r_t.  [TS] Methodologie 2, Positie-uitlijning: global-token
 * RoPE coordinates are scaled by the resolution ratios onto the detail grid.
 * The rotation itself is the standard rotary embedding applied per axis. */

/* RoPE coordinates of a detail token at cube-order position p */
void orc_pos_detail(double *pos3, int64_t p, int64_t T, int64_t H, int64_t W,
                    int64_t ct, int64_t ch, int64_t cw)
{
    int64_t r = orc_cube_src(p, T, H, W, ct, ch, cw);
    pos3[0] = (double)(r / (H * W));
    pos3[1] = (double)((r / W) % H);
    pos3[2] = (double)(r % W);
}

/* RoPE coordinates of a global token at raster position r of (Tg, Hg, Wg) */
void orc_pos_global(double *pos3, int64_t r, int64_t H, int64_t W,
                    int64_t Tg, int64_t Hg, int64_t Wg, double r_t)
{
    (void)Tg;
    int64_t tg = r / (Hg * Wg), hg = (r / Wg) % Hg, wg = r % Wg;
    pos3[0] = r_t * (double)tg;
    pos3[1] = ((double)H / (double)Hg) * (double)hg;
    pos3[2] = ((double)W / (double)Wg) * (double)wg;
}

/* Axis and frequency of rotation pair i for head_dim D. */
static void orc_pair(int i, int D, double theta, int *axis, double *omega)
{
    int nhw = D / 6;
    int nt = D / 2 - 2 * nhw;
    int a, j, na;
    if (i < nt) {
        a = 0; j = i; na = nt;
    } else if (i < nt + nhw) {
        a = 1; j = i - nt; na = nhw;
    } else {
        a = 2; j = i - nt - nhw; na = nhw;
    }
    *axis = a;
    *omega = pow(theta, -(double)j / (double)na);
}

/* Rotate one head vector x[D] (fp64, in place) to the coordinates pos3. */
void orc_rope_vec(double *x, int D, const double *pos3, double theta)
{
    for (int i = 0; i < D / 2; ++i) {
        int a;
        double om;
        orc_pair(i, D, theta, &a, &om);
        double phi = pos3[a] * om;
        double c = cos(phi), s = sin(phi);
        double x0 = x[2 * i], x1 = x[2 * i + 1];
        x[2 * i] = x0 * c - x1 * s;
        x[2 * i + 1] = x0 * s + x1 * c;
    }
}

/* Rotate n token rows [n][heads][D] (fp64, in place); pos is [n][3]. */
void orc_rope_rows(double *x, const double *pos, int64_t n, int heads, int D,
                   double theta)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t)
        for (int h = 0; h < heads; ++h)
            orc_rope_vec(x + (t * heads + h) * D, D, pos + 3 * t, theta);
}

/* ---- O3: asymmetric hierarchical attention ------------------------------
 * [TS] Methodologie 2, Asymmetrische Hierarchische Attention: global and
 * detail tokens are concatenated; global tokens attend only to themselves;
 * detail tokens attend to their own neighbourhood (the cube, after the
 * reorder of Fase 2) and to the global tokens; global -> detail is masked
 * with -inf.  A masked softmax over the concatenation is one softmax over
 * each query's allowed key set, which is what is computed here. */

/* One query row: softmax over nw window keys (rows kw0.. of kd/vd) and ng
 * global keys (rows 0.. of kg/vg), all of head `head`.  out[D] in fp64. */
static double orc_attn_row(double *out, const double *q, int dtype,
                           const void *kd, const void *vd, int64_t kw0, int64_t nw,
                           const void *kg, const void *vg, int64_t ng, const int32_t *gidx,
                           int heads, int head, int D, double scale, double *s)
{
    /* global key j of the list is row gidx[j] of kg/vg, or row j without a list */
#define ORC_GROW(j) (gidx ? (int64_t)gidx[(j)] : (int64_t)(j))
    int64_t nk = nw + ng;
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
        const void *kb = j < nw ? kd : kg;
        int64_t row = j < nw ? kw0 + j : ORC_GROW(j - nw);
        int64_t base = (row * heads + head) * (int64_t)D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += q[d] * orc_ld(kb, dtype, base + d);
        s[j] = acc * scale;
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        const void *vb = j < nw ? vd : vg;
        int64_t row = j < nw ? kw0 + j : ORC_GROW(j - nw);
        int64_t base = (row * heads + head) * (int64_t)D;
        double w = s[j] / l;
        for (int d = 0; d < D; ++d)
            out[d] += w * orc_ld(vb, dtype, base + d);
    }
#undef ORC_GROW
    return m + log(l);   /* log of the softmax denominator of the scaled logits */
}

/*
 * Selected outputs of the attention.  Detail tensors hold N rows in cube
 * order, window c being rows c*V .. c*V+V-1; global tensors hold G rows.
 * Selection k: (row[k], head[k], is_global[k]); out is [nsel][D] fp64.
 * lse (may be NULL) receives log sum_j exp(scale <q, k_j>) over the row's key
 * set, natural log.  All inputs share one boundary dtype.
 * goff/gidx (both NULL for the plain mask) restrict the global keys of a
 * detail query in window c to rows gidx[goff[c] .. goff[c+1]) of kg/vg (the
 * window keys and the global queries' keys are unchanged).
 */
void orc_hier_attn(double *out, double *lse,
                   const void *qd, const void *kd, const void *vd,
                   const void *qg, const void *kg, const void *vg,
                   int dtype, int64_t N, int64_t V, int64_t G,
                   int heads, int D, double scale,
                   const int64_t *row, const int32_t *head,
                   const int8_t *is_global, int64_t nsel,
                   const int64_t *goff, const int32_t *gidx)
{
    /* the longest key list: a window's list may repeat keys and exceed G */
    int64_t maxng = G;
    for (int64_t c = 0; goff && c < N / V; ++c)
        if (goff[c + 1] - goff[c] > maxng)
            maxng = goff[c + 1] - goff[c];
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(V + maxng + 1));
        double *q = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 4)
        for (int64_t k = 0; k < nsel; ++k) {
            int hd = head[k];
            const void *qb = is_global[k] ? qg : qd;
            int64_t base = (row[k] * heads + hd) * (int64_t)D;
            for (int d = 0; d < D; ++d)
                q[d] = orc_ld(qb, dtype, base + d);
            double z;
            if (is_global[k]) {
                z = orc_attn_row(out + k * D, q, dtype, kd, vd, 0, 0, kg, vg, G, NULL,
                                 heads, hd, D, scale, s);
            } else {
                int64_t c = row[k] / V;
                if (goff)
                    z = orc_attn_row(out + k * D, q, dtype, kd, vd, c * V, V, kg, vg,
                                     goff[c + 1] - goff[c], gidx + goff[c], heads, hd, D, scale, s);
                else
                    z = orc_attn_row(out + k * D, q, dtype, kd, vd, c * V, V, kg, vg, G, NULL,
                                     heads, hd, D, scale, s);
            }
            if (lse)
                lse[k] = z;
        }
        free(s);
        free(q);
    }
}

/* ---- co-located ("aligned") global subset -------------------------------
 * The summary's mask lets a detail query attend to the "aligned" global tokens
 * (Methodologie 2, Asymmetrische Hierarchische Attention); the Positie-uitlijning
 * step maps proxy token (tg, hg, wg) to the detail coordinates
 * (r_t*tg, (H/Hg)*hg, (W/Wg)*wg).  The subset reading: cube c sees the proxy
 * tokens whose mapped position lies in its box
 *   [a*ct, (a+1)*ct) x [b*ch, (b+1)*ch) x [e*cw, (e+1)*cw),
 * the comparisons done exactly (H*hg against b*ch*Hg in integers; r_t*tg in
 * fp64).  Lists per cube in increasing proxy raster order; cubes in raster
 * order over the cube grid.  goff has C+1 entries; gidx holds goff[C] <= G
 * indices (every proxy token lies in at most one box).  Returns goff[C].
 * This is a brute-force scan over (cube, proxy token) pairs.
 */
int64_t orc_aligned_subset(int64_t *goff, int32_t *gidx,
                           int64_t T, int64_t H, int64_t W,
                           int64_t ct, int64_t ch, int64_t cw,
                           int64_t Tg, int64_t Hg, int64_t Wg, double r_t)
{
    int64_t nT = T / ct, nH = H / ch, nW = W / cw;
    int64_t G = Tg * Hg * Wg, n = 0;
    goff[0] = 0;
    for (int64_t c = 0; c < nT * nH * nW; ++c) {
        int64_t a = c / (nH * nW), b = (c / nW) % nH, e = c % nW;
        for (int64_t g = 0; g < G; ++g) {
            int64_t tg = g / (Hg * Wg), hg = (g / Wg) % Hg, wg = g % Wg;
            double pt = r_t * (double)tg;
            int in_t = pt >= (double)(a * ct) && pt < (double)((a + 1) * ct);
            int in_h = H * hg >= b * ch * Hg && H * hg < (b + 1) * ch * Hg;
            int in_w = W * wg >= e * cw * Wg && W * wg < (e + 1) * cw * Wg;
            if (in_t && in_h && in_w) {
                if (gidx)
                    gidx[n] = (int32_t)g;
                ++n;
            }
        }
        goff[c + 1] = n;
    }
    return n;
}

/* ---- backward of O3 -----------------------------------------------------
 * Gradient of the attention of one head with respect to q, k and v, given the
 * upstream gradient dO of its output.  For a query i with key set K(i) (the
 * keys the masked softmax of the attention section lets it see):
 *   P_ij  = exp(scale <q_i, k_j> - lse_i),  lse_i = log sum_{j in K(i)} exp(scale <q_i, k_j>)
 *   dP_ij = <dO_i, v_j>
 *   D_i   = sum_j P_ij dP_ij            (equal to <dO_i, o_i>)
 *   dS_ij = P_ij (dP_ij - D_i)          (derivative of the softmax)
 *   dq_i  = scale sum_{j in K(i)} dS_ij k_j
 *   dk_j  = scale sum_{i : j in K(i)} dS_ij q_i
 *   dv_j  = sum_{i : j in K(i)} P_ij dO_i
 * The pages train LoRA adapters of the attention projections at 720P, which
 * needs exactly these gradients (Methodologie 2); the chain rule through the
 * softmax is textbook calculus and nothing on the pages changes it.
 *
 * Error scales (the *_rss entry points; tolerance bookkeeping of the tests,
 * not part of what the method computes): each gradient element above is a
 * sum of terms (scale dS_ij k_j, scale dS_ij q_i or P_ij dO_i over the same
 * pairs).  With sq = 1 the same loops add the squares of those terms instead,
 * and the result is returned as sqrt(sum of squares), the root-sum-square
 * that sizes independent rounding errors of the terms.
 */

/* One query row.  p and ds (length nw + ng) receive P_ij and dS_ij for the
 * window keys (rows kw0.. of kd/vd) followed by the global keys (rows 0.. of
 * kg/vg, or rows gidx[0 .. ng) of them when a list is given); dq[D] receives
 * dq_i.  Returns lse_i; *delta receives D_i. */
#define ORC_TERM(acc, t) ((acc) += sq ? (t) * (t) : (t))

static double orc_bwd_row(double *dq, double *p, double *ds, double *delta,
                          const double *q, const double *dO, int dtype,
                          const void *kd, const void *vd, int64_t kw0, int64_t nw,
                          const void *kg, const void *vg, int64_t ng, const int32_t *gidx,
                          int heads, int head, int D, double scale, int sq)
{
#define ORC_BROW(j) (j < nw ? kw0 + j : (gidx ? (int64_t)gidx[j - nw] : j - nw))
    int64_t nk = nw + ng;
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
        const void *kb = j < nw ? kd : kg;
        int64_t row = ORC_BROW(j);
        int64_t base = (row * heads + head) * (int64_t)D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += q[d] * orc_ld(kb, dtype, base + d);
        p[j] = acc * scale;
        if (p[j] > m)
            m = p[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j)
        l += exp(p[j] - m);
    double lse = m + log(l);
    double dlt = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        const void *vb = j < nw ? vd : vg;
        int64_t row = ORC_BROW(j);
        int64_t base = (row * heads + head) * (int64_t)D;
        p[j] = exp(p[j] - lse);
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += dO[d] * orc_ld(vb, dtype, base + d);
        ds[j] = acc;                       /* dP_ij for now */
        dlt += p[j] * acc;
    }
    for (int d = 0; d < D; ++d)
        dq[d] = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        const void *kb = j < nw ? kd : kg;
        int64_t row = ORC_BROW(j);
        int64_t base = (row * heads + head) * (int64_t)D;
        ds[j] = p[j] * (ds[j] - dlt);
        for (int d = 0; d < D; ++d)
            ORC_TERM(dq[d], scale * ds[j] * orc_ld(kb, dtype, base + d));
    }
    *delta = dlt;
#undef ORC_BROW
    return lse;
}

static void orc_sqrt_all(double *x, int64_t n)
{
    for (int64_t e = 0; x && e < n; ++e)
        x[e] = sqrt(x[e]);
}

static void orc_load_row(double *x, const void *b, int dtype, int64_t row, int heads, int head, int D)
{
    int64_t base = (row * heads + head) * (int64_t)D;
    for (int d = 0; d < D; ++d)
        x[d] = orc_ld(b, dtype, base + d);
}

/*
 * Full backward.  Inputs: detail q/k/v/dO [N][heads][D] in cube order (window
 * c = rows c*V .. c*V+V-1), global q/k/v/dO [G][heads][D], one boundary dtype.
 * Outputs (fp64): dq/dk/dv of both sets in the same layouts, lse and D of every
 * query as [heads][N] and [heads][G].  First every query's own row (dq, lse, D
 * and its window keys' share of dk/dv, owned by its window); then, per global
 * key, the sum over every query that sees it.
 * goff/gidx (both NULL for the plain mask): the per-window global subset, as in
 * orc_hier_attn (indices in [0, G); a key listed twice for a window is two
 * terms of that window's softmax).  Then each detail query's share of the
 * listed keys' dk/dv is added while its row is computed (one thread per head,
 * so no two threads touch one key row), and the per-key pass adds the global
 * queries only.
 */
static void orc_bwd_full(double *dqd, double *dkd, double *dvd,
                         double *dqg, double *dkg, double *dvg,
                         double *lse_d, double *lse_g, double *dl_d, double *dl_g,
                         const void *qd, const void *kd, const void *vd, const void *dod,
                         const void *qg, const void *kg, const void *vg, const void *dog,
                         int dtype, int64_t N, int64_t V, int64_t G,
                         int heads, int D, double scale,
                         const int64_t *goff, const int32_t *gidx, int sq)
{
    int64_t C = N / V;
    int64_t maxng = G;   /* the longest key list (a subset list may exceed G) */
    for (int64_t c = 0; goff && c < C; ++c)
        if (goff[c + 1] - goff[c] > maxng)
            maxng = goff[c + 1] - goff[c];
    memset(dkd, 0, sizeof(double) * (size_t)(N * heads * D));
    memset(dvd, 0, sizeof(double) * (size_t)(N * heads * D));
    if (G > 0) {
        memset(dkg, 0, sizeof(double) * (size_t)(G * heads * D));
        memset(dvg, 0, sizeof(double) * (size_t)(G * heads * D));
    }
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(V + maxng + 1));
        double *ds = (double *)malloc(sizeof(double) * (size_t)(V + maxng + 1));
        double *q = (double *)malloc(sizeof(double) * (size_t)D);
        double *g = (double *)malloc(sizeof(double) * (size_t)D);
        /* detail queries, one (head, window) per task (one head per task with
         * a subset): the window's keys get contributions from this window's
         * queries only */
        const int64_t per = goff ? 1 : C;
#pragma omp for schedule(dynamic, 1)
        for (int64_t task = 0; task < (int64_t)heads * per; ++task) {
            int h = (int)(task / per);
            int64_t c0 = goff ? 0 : task % C, c1 = goff ? C : c0 + 1;
            for (int64_t c = c0; c < c1; ++c) {
                const int64_t ng = goff ? goff[c + 1] - goff[c] : G;
                const int32_t *gl = goff ? gidx + goff[c] : NULL;
                for (int64_t i = c * V; i < (c + 1) * V; ++i) {
                    orc_load_row(q, qd, dtype, i, heads, h, D);
                    orc_load_row(g, dod, dtype, i, heads, h, D);
                    lse_d[(int64_t)h * N + i] =
                        orc_bwd_row(dqd + (i * heads + h) * D, p, ds, &dl_d[(int64_t)h * N + i], q,
                                    g, dtype, kd, vd, c * V, V, kg, vg, ng, gl, heads, h, D, scale, sq);
                    for (int64_t j = 0; j < V; ++j) {
                        double *dk = dkd + ((c * V + j) * heads + h) * D;
                        double *dv = dvd + ((c * V + j) * heads + h) * D;
                        for (int d = 0; d < D; ++d) {
                            ORC_TERM(dk[d], scale * ds[j] * q[d]);
                            ORC_TERM(dv[d], p[j] * g[d]);
                        }
                    }
                    for (int64_t m = 0; gl && m < ng; ++m) {
                        double *dk = dkg + ((int64_t)gl[m] * heads + h) * D;
                        double *dv = dvg + ((int64_t)gl[m] * heads + h) * D;
                        for (int d = 0; d < D; ++d) {
                            ORC_TERM(dk[d], scale * ds[V + m] * q[d]);
                            ORC_TERM(dv[d], p[V + m] * g[d]);
                        }
                    }
                }
            }
        }
        /* global queries: global keys only */
#pragma omp for schedule(dynamic, 8)
        for (int64_t task = 0; task < (int64_t)heads * G; ++task) {
            int h = (int)(task / G);
            int64_t i = task % G;
            orc_load_row(q, qg, dtype, i, heads, h, D);
            orc_load_row(g, dog, dtype, i, heads, h, D);
            lse_g[(int64_t)h * G + i] =
                orc_bwd_row(dqg + (i * heads + h) * D, p, ds, &dl_g[(int64_t)h * G + i], q, g,
                            dtype, kd, vd, 0, 0, kg, vg, G, NULL, heads, h, D, scale, sq);
        }
        /* global keys: every global query sees them, and every detail query
         * too without a subset */
#pragma omp for schedule(dynamic, 4)
        for (int64_t task = 0; task < (int64_t)heads * G; ++task) {
            int h = (int)(task / G);
            int64_t j = task % G;
            double *kk = (double *)malloc(sizeof(double) * (size_t)D);
            double *vv = (double *)malloc(sizeof(double) * (size_t)D);
            orc_load_row(kk, kg, dtype, j, heads, h, D);
            orc_load_row(vv, vg, dtype, j, heads, h, D);
            double *dk = dkg + (j * heads + h) * D;
            double *dv = dvg + (j * heads + h) * D;
            for (int64_t i = goff ? N : 0; i < N + G; ++i) {
                int is_g = i >= N;
                int64_t r = is_g ? i - N : i;
                orc_load_row(q, is_g ? qg : qd, dtype, r, heads, h, D);
                orc_load_row(g, is_g ? dog : dod, dtype, r, heads, h, D);
                double s = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) {
                    s += q[d] * kk[d];
                    dp += g[d] * vv[d];
                }
                double lse = is_g ? lse_g[(int64_t)h * G + r] : lse_d[(int64_t)h * N + r];
                double dlt = is_g ? dl_g[(int64_t)h * G + r] : dl_d[(int64_t)h * N + r];
                double pij = exp(s * scale - lse);
                double dsij = pij * (dp - dlt);
                for (int d = 0; d < D; ++d) {
                    ORC_TERM(dk[d], scale * dsij * q[d]);
                    ORC_TERM(dv[d], pij * g[d]);
                }
            }
            free(kk);
            free(vv);
        }
        free(p);
        free(ds);
        free(q);
        free(g);
    }
    if (sq) {
        orc_sqrt_all(dqd, N * heads * D);
        orc_sqrt_all(dkd, N * heads * D);
        orc_sqrt_all(dvd, N * heads * D);
        if (G > 0) {
            orc_sqrt_all(dqg, G * heads * D);
            orc_sqrt_all(dkg, G * heads * D);
            orc_sqrt_all(dvg, G * heads * D);
        }
    }
}

void orc_hier_attn_bwd(double *dqd, double *dkd, double *dvd,
                       double *dqg, double *dkg, double *dvg,
                       double *lse_d, double *lse_g, double *dl_d, double *dl_g,
                       const void *qd, const void *kd, const void *vd, const void *dod,
                       const void *qg, const void *kg, const void *vg, const void *dog,
                       int dtype, int64_t N, int64_t V, int64_t G,
                       int heads, int D, double scale,
                       const int64_t *goff, const int32_t *gidx)
{
    orc_bwd_full(dqd, dkd, dvd, dqg, dkg, dvg, lse_d, lse_g, dl_d, dl_g, qd, kd, vd, dod, qg, kg,
                 vg, dog, dtype, N, V, G, heads, D, scale, goff, gidx, 0);
}

/* root-sum-square error scales of every gradient element (see above) */
void orc_hier_attn_bwd_rss(double *dqd, double *dkd, double *dvd,
                           double *dqg, double *dkg, double *dvg,
                           double *lse_d, double *lse_g, double *dl_d, double *dl_g,
                           const void *qd, const void *kd, const void *vd, const void *dod,
                           const void *qg, const void *kg, const void *vg, const void *dog,
                           int dtype, int64_t N, int64_t V, int64_t G,
                           int heads, int D, double scale,
                           const int64_t *goff, const int32_t *gidx)
{
    orc_bwd_full(dqd, dkd, dvd, dqg, dkg, dvg, lse_d, lse_g, dl_d, dl_g, qd, kd, vd, dod, qg, kg,
                 vg, dog, dtype, N, V, G, heads, D, scale, goff, gidx, 1);
}

/* Backward of selected query rows: dq[nsel][D], lse[nsel], delta[nsel] for
 * selection k = (row[k], head[k], is_global[k]); each row needs only its own
 * key set. */
static void orc_bwd_rows(double *dq, double *lse, double *delta,
                         const void *qd, const void *kd, const void *vd, const void *dod,
                         const void *qg, const void *kg, const void *vg, const void *dog,
                         int dtype, int64_t N, int64_t V, int64_t G, int heads, int D,
                         double scale, const int64_t *row, const int32_t *head,
                         const int8_t *is_global, int64_t nsel, int sq)
{
    (void)N;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(V + G + 1));
        double *ds = (double *)malloc(sizeof(double) * (size_t)(V + G + 1));
        double *q = (double *)malloc(sizeof(double) * (size_t)D);
        double *g = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t k = 0; k < nsel; ++k) {
            int h = head[k];
            if (is_global[k]) {
                orc_load_row(q, qg, dtype, row[k], heads, h, D);
                orc_load_row(g, dog, dtype, row[k], heads, h, D);
                lse[k] = orc_bwd_row(dq + k * D, p, ds, &delta[k], q, g, dtype, kd, vd, 0, 0,
                                     kg, vg, G, NULL, heads, h, D, scale, sq);
            } else {
                int64_t c = row[k] / V;
                orc_load_row(q, qd, dtype, row[k], heads, h, D);
                orc_load_row(g, dod, dtype, row[k], heads, h, D);
                lse[k] = orc_bwd_row(dq + k * D, p, ds, &delta[k], q, g, dtype, kd, vd, c * V, V,
                                     kg, vg, G, NULL, heads, h, D, scale, sq);
            }
        }
        free(p);
        free(ds);
        free(q);
        free(g);
    }
    if (sq)
        orc_sqrt_all(dq, nsel * D);
}

void orc_hier_attn_bwd_rows(double *dq, double *lse, double *delta,
                            const void *qd, const void *kd, const void *vd, const void *dod,
                            const void *qg, const void *kg, const void *vg, const void *dog,
                            int dtype, int64_t N, int64_t V, int64_t G, int heads, int D,
                            double scale, const int64_t *row, const int32_t *head,
                            const int8_t *is_global, int64_t nsel)
{
    orc_bwd_rows(dq, lse, delta, qd, kd, vd, dod, qg, kg, vg, dog, dtype, N, V, G, heads, D, scale,
                 row, head, is_global, nsel, 0);
}

void orc_hier_attn_bwd_rows_rss(double *dq, double *lse, double *delta,
                                const void *qd, const void *kd, const void *vd, const void *dod,
                                const void *qg, const void *kg, const void *vg, const void *dog,
                                int dtype, int64_t N, int64_t V, int64_t G, int heads, int D,
                                double scale, const int64_t *row, const int32_t *head,
                                const int8_t *is_global, int64_t nsel)
{
    orc_bwd_rows(dq, lse, delta, qd, kd, vd, dod, qg, kg, vg, dog, dtype, N, V, G, heads, D, scale,
                 row, head, is_global, nsel, 1);
}

/* dk, dv [V][D] of the detail keys of window c, head h: the sum over the
 * window's V queries (the only queries that see these keys). */
static void orc_bwd_window(double *dk, double *dv,
                           const void *qd, const void *kd, const void *vd, const void *dod,
                           const void *kg, const void *vg,
                           int dtype, int64_t V, int64_t G, int heads, int D, double scale,
                           int head, int64_t c, int sq)
{
    memset(dk, 0, sizeof(double) * (size_t)(V * D));
    memset(dv, 0, sizeof(double) * (size_t)(V * D));
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(V + G + 1));
        double *ds = (double *)malloc(sizeof(double) * (size_t)(V + G + 1));
        double *q = (double *)malloc(sizeof(double) * (size_t)D);
        double *g = (double *)malloc(sizeof(double) * (size_t)D);
        double *dq = (double *)malloc(sizeof(double) * (size_t)D);
        double *mk = (double *)calloc((size_t)(V * D), sizeof(double));
        double *mv = (double *)calloc((size_t)(V * D), sizeof(double));
        double dlt;
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = c * V; i < (c + 1) * V; ++i) {
            orc_load_row(q, qd, dtype, i, heads, head, D);
            orc_load_row(g, dod, dtype, i, heads, head, D);
            orc_bwd_row(dq, p, ds, &dlt, q, g, dtype, kd, vd, c * V, V, kg, vg, G, NULL, heads, head,
                        D, scale, sq);
            for (int64_t j = 0; j < V; ++j)
                for (int d = 0; d < D; ++d) {
                    ORC_TERM(mk[j * D + d], scale * ds[j] * q[d]);
                    ORC_TERM(mv[j * D + d], p[j] * g[d]);
                }
        }
#pragma omp critical
        {
            for (int64_t e = 0; e < V * D; ++e) {
                dk[e] += mk[e];
                dv[e] += mv[e];
            }
        }
        free(p);
        free(ds);
        free(q);
        free(g);
        free(dq);
        free(mk);
        free(mv);
    }
    if (sq) {
        orc_sqrt_all(dk, V * D);
        orc_sqrt_all(dv, V * D);
    }
}

void orc_hier_attn_bwd_window(double *dk, double *dv,
                              const void *qd, const void *kd, const void *vd, const void *dod,
                              const void *kg, const void *vg,
                              int dtype, int64_t V, int64_t G, int heads, int D, double scale,
                              int head, int64_t c)
{
    orc_bwd_window(dk, dv, qd, kd, vd, dod, kg, vg, dtype, V, G, heads, D, scale, head, c, 0);
}

void orc_hier_attn_bwd_window_rss(double *dk, double *dv,
                                  const void *qd, const void *kd, const void *vd, const void *dod,
                                  const void *kg, const void *vg,
                                  int dtype, int64_t V, int64_t G, int heads, int D, double scale,
                                  int head, int64_t c)
{
    orc_bwd_window(dk, dv, qd, kd, vd, dod, kg, vg, dtype, V, G, heads, D, scale, head, c, 1);
}

/* dk, dv [nsel][D] of selected global keys key[0..nsel) of head h.  Every
 * detail query and every global query sees a global key, so first each
 * query's lse_i and D_i (its own row of the attention), then per key the sum
 * over all N + G queries of scale * dS_ij * q_i and P_ij * dO_i. */
static void orc_bwd_gkeys(double *dk, double *dv,
                          const void *qd, const void *kd, const void *vd, const void *dod,
                          const void *qg, const void *kg, const void *vg, const void *dog,
                          int dtype, int64_t N, int64_t V, int64_t G, int heads, int D,
                          double scale, int head, const int64_t *key, int64_t nsel, int sq)
{
    double *lse = (double *)malloc(sizeof(double) * (size_t)(N + G));
    double *dl = (double *)malloc(sizeof(double) * (size_t)(N + G));
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(V + G + 1));
        double *ds = (double *)malloc(sizeof(double) * (size_t)(V + G + 1));
        double *q = (double *)malloc(sizeof(double) * (size_t)D);
        double *g = (double *)malloc(sizeof(double) * (size_t)D);
        double *dq = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < N + G; ++i) {
            if (i < N) {
                int64_t c = i / V;
                orc_load_row(q, qd, dtype, i, heads, head, D);
                orc_load_row(g, dod, dtype, i, heads, head, D);
                lse[i] = orc_bwd_row(dq, p, ds, &dl[i], q, g, dtype, kd, vd, c * V, V, kg, vg, G,
                                     NULL, heads, head, D, scale, 0);
            } else {
                orc_load_row(q, qg, dtype, i - N, heads, head, D);
                orc_load_row(g, dog, dtype, i - N, heads, head, D);
                lse[i] = orc_bwd_row(dq, p, ds, &dl[i], q, g, dtype, kd, vd, 0, 0, kg, vg, G,
                                     NULL, heads, head, D, scale, 0);
            }
        }
        /* the implicit barrier of the loop above: every lse_i and D_i is set */
#pragma omp for schedule(dynamic, 1)
        for (int64_t k = 0; k < nsel; ++k) {
            double *kk = (double *)malloc(sizeof(double) * (size_t)D);
            double *vv = (double *)malloc(sizeof(double) * (size_t)D);
            orc_load_row(kk, kg, dtype, key[k], heads, head, D);
            orc_load_row(vv, vg, dtype, key[k], heads, head, D);
            double *a = dk + k * D, *b = dv + k * D;
            for (int d = 0; d < D; ++d)
                a[d] = b[d] = 0.0;
            for (int64_t i = 0; i < N + G; ++i) {
                int is_g = i >= N;
                int64_t r = is_g ? i - N : i;
                orc_load_row(q, is_g ? qg : qd, dtype, r, heads, head, D);
                orc_load_row(g, is_g ? dog : dod, dtype, r, heads, head, D);
                double sv = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) {
                    sv += q[d] * kk[d];
                    dp += g[d] * vv[d];
                }
                double pij = exp(sv * scale - lse[i]);
                double dsij = pij * (dp - dl[i]);
                for (int d = 0; d < D; ++d) {
                    ORC_TERM(a[d], scale * dsij * q[d]);
                    ORC_TERM(b[d], pij * g[d]);
                }
            }
            free(kk);
            free(vv);
        }
        free(p);
        free(ds);
        free(q);
        free(g);
        free(dq);
    }
    free(lse);
    free(dl);
    if (sq) {
        orc_sqrt_all(dk, nsel * D);
        orc_sqrt_all(dv, nsel * D);
    }
}

void orc_hier_attn_bwd_gkeys(double *dk, double *dv,
                             const void *qd, const void *kd, const void *vd, const void *dod,
                             const void *qg, const void *kg, const void *vg, const void *dog,
                             int dtype, int64_t N, int64_t V, int64_t G, int heads, int D,
                             double scale, int head, const int64_t *key, int64_t nsel)
{
    orc_bwd_gkeys(dk, dv, qd, kd, vd, dod, qg, kg, vg, dog, dtype, N, V, G, heads, D, scale, head,
                  key, nsel, 0);
}

void orc_hier_attn_bwd_gkeys_rss(double *dk, double *dv,
                                 const void *qd, const void *kd, const void *vd, const void *dod,
                                 const void *qg, const void *kg, const void *vg, const void *dog,
                                 int dtype, int64_t N, int64_t V, int64_t G, int heads, int D,
                                 double scale, int head, const int64_t *key, int64_t nsel)
{
    orc_bwd_gkeys(dk, dv, qd, kd, vd, dod, qg, kg, vg, dog, dtype, N, V, G, heads, D, scale, head,
                  key, nsel, 1);
}

/* ---- O1..O4 end to end, for selected output rows -------------------------
 * Inputs are raw (pre-RoPE) q/k/v in RASTER order for detail tokens and
 * raster order over the proxy grid for global tokens, all in one boundary
 * dtype.  Mirrors the storage between the four calls: the rotated q and k are
 * rounded to the boundary dtype (round to nearest even) before attention.
 * Selection k: (row[k] = raster row for detail / proxy row for global,
 * head[k], is_global[k]); out[k][D] is the output at that raster row, i.e.
 * after the unorder.  Global keys are rotated once per head used.
 */
static double orc_round_to(double x, int dtype)
{
    if (dtype == ORC_BF16) {
        uint32_t u = (uint32_t)orc_round_bf16(x) << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    if (dtype == ORC_F32)
        return (double)(float)x;
    return x;
}

void orc_pipeline_rows(double *out,
                       const void *qd, const void *kd, const void *vd,
                       const void *qg, const void *kg, const void *vg,
                       int dtype,
                       int64_t T, int64_t H, int64_t W,
                       int64_t ct, int64_t ch, int64_t cw,
                       int64_t Tg, int64_t Hg, int64_t Wg,
                       double r_t, double theta, int heads, int D, double scale,
                       const int64_t *row, const int32_t *head,
                       const int8_t *is_global, int64_t nsel)
{
    int64_t V = ct * ch * cw;
    int64_t G = Tg * Hg * Wg;
    /* rotated + rounded global keys for every head that is used */
    double *kg_rot = NULL;
    int8_t *used = (int8_t *)calloc((size_t)heads, 1);
    for (int64_t k = 0; k < nsel; ++k)
        used[head[k]] = 1;
    if (G > 0) {
        kg_rot = (double *)malloc(sizeof(double) * (size_t)(G * heads * D));
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < G; ++j) {
            double pos[3];
            orc_pos_global(pos, j, H, W, Tg, Hg, Wg, r_t);
            for (int h = 0; h < heads; ++h) {
                if (!used[h])
                    continue;
                double *x = kg_rot + (j * heads + h) * D;
                for (int d = 0; d < D; ++d)
                    x[d] = orc_ld(kg, dtype, (j * heads + h) * (int64_t)D + d);
                orc_rope_vec(x, D, pos, theta);
                for (int d = 0; d < D; ++d)
                    x[d] = orc_round_to(x[d], dtype);
            }
        }
    }
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(V + G + 1));
        double *q = (double *)malloc(sizeof(double) * (size_t)D);
        double *kw = (double *)malloc(sizeof(double) * (size_t)(V * D));
        double *vw = (double *)malloc(sizeof(double) * (size_t)(V * D));
#pragma omp for schedule(dynamic, 1)
        for (int64_t k = 0; k < nsel; ++k) {
            int hd = head[k];
            double pos[3];
            int64_t nw = 0;
            if (is_global[k]) {
                orc_pos_global(pos, row[k], H, W, Tg, Hg, Wg, r_t);
                for (int d = 0; d < D; ++d)
                    q[d] = orc_ld(qg, dtype, (row[k] * heads + hd) * (int64_t)D + d);
            } else {
                int64_t p = orc_cube_dst(row[k], T, H, W, ct, ch, cw);
                orc_pos_detail(pos, p, T, H, W, ct, ch, cw);
                for (int d = 0; d < D; ++d)
                    q[d] = orc_ld(qd, dtype, (row[k] * heads + hd) * (int64_t)D + d);
                /* keys/values of the query's own cube, rotated and rounded */
                int64_t c = p / V;
                nw = V;
                for (int64_t j = 0; j < V; ++j) {
                    int64_t pk = c * V + j;
                    int64_t rk = orc_cube_src(pk, T, H, W, ct, ch, cw);
                    double pk3[3];
                    orc_pos_detail(pk3, pk, T, H, W, ct, ch, cw);
                    for (int d = 0; d < D; ++d) {
                        kw[j * D + d] = orc_ld(kd, dtype, (rk * heads + hd) * (int64_t)D + d);
                        vw[j * D + d] = orc_ld(vd, dtype, (rk * heads + hd) * (int64_t)D + d);
                    }
                    orc_rope_vec(kw + j * D, D, pk3, theta);
                    for (int d = 0; d < D; ++d)
                        kw[j * D + d] = orc_round_to(kw[j * D + d], dtype);
                }
            }
            orc_rope_vec(q, D, pos, theta);
            for (int d = 0; d < D; ++d)
                q[d] = orc_round_to(q[d], dtype);
            /* one softmax over window keys then global keys */
            int64_t nk = nw + G;
            double m = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                const double *kr = j < nw ? kw + j * D : kg_rot + ((j - nw) * heads + hd) * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d)
                    acc += q[d] * kr[d];
                s[j] = acc * scale;
                if (s[j] > m)
                    m = s[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            double *o = out + k * D;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                double w = s[j] / l;
                if (j < nw) {
                    for (int d = 0; d < D; ++d)
                        o[d] += w * vw[j * D + d];
                } else {
                    int64_t base = ((j - nw) * heads + hd) * (int64_t)D;
                    for (int d = 0; d < D; ++d)
                        o[d] += w * orc_ld(vg, dtype, base + d);
                }
            }
        }
        free(s);
        free(q);
        free(kw);
        free(vw);
    }
    free(kg_rot);
    free(used);
}
