/*
 * Grouped Query Experts (GQE) attention, forward (prefill) pass: the plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct definition that the
 * GPU library is checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header or constant with the HIP
 * library under sparse_moe_query_amd/, and nothing in the product path calls it.
 *
 * Sources (the web pages on GQE; cited by page title and section):
 *  [R]  "GQE: Grouped Query Experts" repository README, sections "Algorithm Overview",
 *       "Usage" and "Parameters" (the authors' own description).
 *  [T]  "Grouped Query Experts: Mixture-of-Experts on GQA Self-Attention", gist.science
 *       explainer, "Technical Summary" -> "Architecture and Routing", "Training and Loss".
 *  [M]  "Grouped-query attention and mixture of experts" tutorial (cseroadmap), sections
 *       "Multi-head, multi-query and grouped-query attention" and "Mixture of experts (MoE)"
 *       (the moe_layer sketch and its tested properties).
 *
 * Arithmetic: every input arrives as double (the caller widens the fp32 or bf16-rounded
 * values exactly); every dot product, softmax sum and output accumulation is done in
 * double, in plain sequential loop order.  There is no blocking, no fusion and no
 * reordering beyond the definition.  OpenMP only splits independent tokens.
 *
 * Notation (README "Parameters"): d = dim, N = num_query_experts, G = num_kv_heads,
 * k = top_k, dh = head_dim; n = N/G experts per group; expert e belongs to group
 * g = e / n with local index j = e % n (contiguous grouping, as in GQA where each
 * group of query heads shares one KV head [M]).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - top-k is taken on the logits (softmax is strictly monotone, so the selected set
 *    is the one "softmax then top-k" gives); equal logits -> lower local index first;
 *    rank order within the selection is descending logit, then ascending index.
 *  - renormalised weights w = p_sel / sum(p_sel) over the k selected experts [T], [M].
 *  - "hard concat": each selected expert's head output goes through its own d_h x d
 *    slice of the output projection (MHA concat with unselected slots zero).
 *  - "renormalised weighted-sum slot": one extra d_h slot per group with its own
 *    projection W_oR[g], fed with sum_r w_r * o_r.
 *  - weighted_concat: the selected expert's slot is scaled by its in-group softmax
 *    probability p (not renormalised).
 *  - the shared head (a flag, default on) attends to KV group shared_kv_group.
 *  - attention scale 1/sqrt(dh); causal mask keeps keys s' <= s; no projection biases.
 *    Positional encoding: none on the pages; optionally (rope_base > 0) the rotary position
 *    embedding of RoFormer (Su et al., "RoFormer: Enhanced Transformer with Rotary Position
 *    Embedding"), read with interleaved pairs: the pair (v[2i], v[2i+1]) of every query and
 *    key head vector at position m is rotated by the angle m * rope_base^(-2i/dh).
 *  - aux loss (Switch style, [R] "Algorithm Overview", [T] "Training and Loss"):
 *    f_e = count_e/(T k), P_e = mean_t p[t,e], L_g = n * sum_{e in g} f_e P_e,
 *    aux = mean_g L_g; unscaled (the caller multiplies by 0.01, [R] "Usage").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t dim;             /* d   */
    int32_t num_query_experts; /* N */
    int32_t num_kv_heads;    /* G   */
    int32_t top_k;           /* k   */
    int32_t head_dim;        /* dh  */
    int32_t variant;         /* 0 gqe, 1 weighted_concat, 2 hard_concat */
    int32_t shared_head;     /* 1 = one always-on shared query head */
    int32_t shared_kv_group; /* KV group the shared head reads */
    int32_t pos0;            /* position of the first token of every sequence (normally 0) */
    int32_t pad_;
    double rope_base;        /* rotary position embedding base; 0 = no positional encoding */
} oracle_cfg;

/* Rotary position embedding of one head vector at position m (see the readings above):
 * (v[2i], v[2i+1]) -> (v[2i] cos a - v[2i+1] sin a, v[2i] sin a + v[2i+1] cos a),
 * a = m * base^(-2i/dh).  No-op when base == 0. */
static void rope(double* v, int dh, int64_t m, double base)
{
    if (base <= 0.0) return;
    for (int i = 0; i < dh / 2; ++i) {
        const double a = (double)m * pow(base, -2.0 * i / dh);
        const double c = cos(a), s = sin(a);
        const double x0 = v[2 * i], x1 = v[2 * i + 1];
        v[2 * i] = x0 * c - x1 * s;
        v[2 * i + 1] = x0 * s + x1 * c;
    }
}

/* ---------------------------------------------------------------------------------
 * Router, for one token: logits, in-group softmax, top-k, renormalised weights.
 * [R] "Algorithm Overview": softmax over experts inside each GQA group, then top-k.
 * [M] moe_layer: probs = softmax(x @ router_w); keep the best top_k; mix by
 * renormalised router weights.
 *   logits[e] = sum_i x[i] * Wr[i][e] + br[e]
 *   p[e]      = exp(logits[e] - m_g) / sum_{j in g} exp(logits[j] - m_g)
 *   idx[g][r] = r-th best expert of group g (global id), w[g][r] = p / sum_sel p
 *   gap[g]    = logit of the k-th choice minus logit of the (k+1)-th (+inf if k = n)
 * --------------------------------------------------------------------------------- */
static void router_token(const oracle_cfg* c, const double* x, const double* Wr,
                         const double* br, double* logits, double* p, int32_t* idx,
                         double* w, double* gap)
{
    const int d = c->dim, N = c->num_query_experts, G = c->num_kv_heads, k = c->top_k;
    const int n = N / G;
    for (int e = 0; e < N; ++e) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += x[i] * Wr[(size_t)i * N + e];
        logits[e] = acc + (br ? br[e] : 0.0);
    }
    for (int g = 0; g < G; ++g) {
        const double* lg = logits + g * n;
        double m = lg[0];
        for (int j = 1; j < n; ++j) if (lg[j] > m) m = lg[j];
        double den = 0.0;
        for (int j = 0; j < n; ++j) den += exp(lg[j] - m);
        for (int j = 0; j < n; ++j) p[g * n + j] = exp(lg[j] - m) / den;

        /* top-k by repeated selection of the best remaining local index */
        int taken[64];
        for (int j = 0; j < n; ++j) taken[j] = 0;
        int sel[64];
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int j = 0; j < n; ++j) {
                if (taken[j]) continue;
                if (best < 0 || lg[j] > lg[best]) best = j; /* strict: lower j wins ties */
            }
            taken[best] = 1;
            sel[r] = best;
        }
        if (k < n) {
            int next = -1;
            for (int j = 0; j < n; ++j) {
                if (taken[j]) continue;
                if (next < 0 || lg[j] > lg[next]) next = j;
            }
            gap[g] = lg[sel[k - 1]] - lg[next];
        } else {
            gap[g] = INFINITY;
        }
        double psum = 0.0;
        for (int r = 0; r < k; ++r) psum += p[g * n + sel[r]];
        for (int r = 0; r < k; ++r) {
            idx[g * k + r] = g * n + sel[r];
            w[g * k + r] = p[g * n + sel[r]] / psum;
        }
    }
}

/* x: [T, d]; outputs per token: logits/p [T, N], idx/w [T, G, k], gap [T, G]. */
int gqe_oracle_router(const oracle_cfg* c, int64_t T, const double* x, const double* Wr,
                      const double* br, double* logits, double* p, int32_t* idx, double* w,
                      double* gap)
{
    const int d = c->dim, N = c->num_query_experts, G = c->num_kv_heads, k = c->top_k;
    if (N <= 0 || G <= 0 || N % G != 0 || k < 1 || k > N / G || N / G > 64) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        router_token(c, x + t * d, Wr, br, logits + t * N, p + t * N, idx + t * G * k,
                     w + t * G * k, gap + t * G);
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Load-balancing statistics ([R] "Algorithm Overview": Switch-style auxiliary loss;
 * [T] "Training and Loss": encourage even use of the experts within each group).
 *   count_e = #tokens that selected e;  P_e = (1/T) sum_t p[t,e]
 *   f_e = count_e / (T k);  L_g = n sum_{e in g} f_e P_e;  aux = (1/G) sum_g L_g
 *   active_heads = G k + (shared head ? 1 : 0)   ([R] "Algorithm Overview": 9 of 16)
 * --------------------------------------------------------------------------------- */
int gqe_oracle_aux(const oracle_cfg* c, int64_t T, const double* p, const int32_t* idx,
                   int64_t* counts, double* mean_prob, double* aux, int32_t* active_heads)
{
    const int N = c->num_query_experts, G = c->num_kv_heads, k = c->top_k;
    const int n = N / G;
    for (int e = 0; e < N; ++e) { counts[e] = 0; mean_prob[e] = 0.0; }
    for (int64_t t = 0; t < T; ++t) {
        for (int a = 0; a < G * k; ++a) counts[idx[t * G * k + a]] += 1;
        for (int e = 0; e < N; ++e) mean_prob[e] += p[t * N + e];
    }
    for (int e = 0; e < N; ++e) mean_prob[e] /= (double)T;
    double total = 0.0;
    for (int g = 0; g < G; ++g) {
        double Lg = 0.0;
        for (int j = 0; j < n; ++j) {
            const int e = g * n + j;
            const double f = (double)counts[e] / ((double)T * (double)k);
            Lg += f * mean_prob[e];
        }
        total += (double)n * Lg;
    }
    *aux = total / (double)G;
    *active_heads = G * k + (c->shared_head ? 1 : 0);
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Token-to-expert bucketing: the global gather that lets each routed expert read a
 * contiguous list of its tokens ([R] "Algorithm Overview": a router selects k experts
 * per token in every group, and only those experts' query heads are computed).
 * Definition: the T*G*k assignments (t, g, r) with expert e = idx[t][g][r], sorted
 * stably by e (tokens ascending inside each expert):
 *   offs[e]           = number of assignments to experts below e   (offs[N] = T*G*k)
 *   perm[offs[e] + i] = token of the i-th assignment to expert e
 *   inv[t][g][r]      = position of assignment (t, g, r) in perm
 * Written as a counting sort: count per expert, exclusive prefix, then one pass over
 * the assignments in (t, g, r) order.
 * --------------------------------------------------------------------------------- */
int gqe_oracle_bucket(const oracle_cfg* c, int64_t T, const int32_t* idx, int64_t* offs,
                      int64_t* perm, int64_t* inv)
{
    const int N = c->num_query_experts, G = c->num_kv_heads, k = c->top_k;
    const int64_t A = T * G * k;
    int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (!next) return -1;
    for (int e = 0; e <= N; ++e) offs[e] = 0;
    for (int64_t a = 0; a < A; ++a) offs[idx[a] + 1] += 1;
    for (int e = 0; e < N; ++e) offs[e + 1] += offs[e];
    for (int e = 0; e < N; ++e) next[e] = offs[e];
    for (int64_t a = 0; a < A; ++a) {
        const int e = idx[a];
        const int64_t pos = next[e]++;
        perm[pos] = a / ((int64_t)G * k);
        inv[a] = pos;
    }
    free(next);
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Dense KV path ([R] "Algorithm Overview": all KV heads remain dense and unchanged;
 * [T] "Dense KV Path").  For every token and every group g:
 *   K[t][g][:] = x[t] @ Wk[:, g dh:(g+1) dh],  V likewise.   Wk, Wv: [d, G dh]
 * then, with the rotary embedding, K[t][g] rotated at position pos0 + t % S (S = tokens per
 * sequence).  Output layout K, V: [T, G, dh].
 * --------------------------------------------------------------------------------- */
int gqe_oracle_kv(const oracle_cfg* c, int64_t T, int64_t S, const double* x, const double* Wk,
                  const double* Wv, double* K, double* V)
{
    const int d = c->dim, G = c->num_kv_heads, dh = c->head_dim;
    const int W = G * dh;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int col = 0; col < W; ++col) {
            double ak = 0.0, av = 0.0;
            for (int i = 0; i < d; ++i) {
                ak += x[t * d + i] * Wk[(size_t)i * W + col];
                av += x[t * d + i] * Wv[(size_t)i * W + col];
            }
            K[t * W + col] = ak;
            V[t * W + col] = av;
        }
        for (int g = 0; g < G; ++g) rope(K + t * W + (size_t)g * dh, dh, c->pos0 + t % S, c->rope_base);
    }
    return 0;
}

/* Causal softmax attention of one query row over keys 0..s of one sequence and one
 * KV group (two passes: the maximum, then the exponential sums).
 * Kseq/Vseq point at position 0 of the sequence; row stride between positions is
 * G*dh, and the group's dh values start at offset g*dh. */
static void attend(int s, int dh, int G, int g, const double* q, const double* Kseq,
                   const double* Vseq, double* o)
{
    const double scale = 1.0 / sqrt((double)dh);
    double m = -INFINITY;
    for (int j = 0; j <= s; ++j) {
        const double* kj = Kseq + (size_t)j * G * dh + (size_t)g * dh;
        double sc = 0.0;
        for (int i = 0; i < dh; ++i) sc += q[i] * kj[i];
        sc *= scale;
        if (sc > m) m = sc;
    }
    double den = 0.0;
    for (int i = 0; i < dh; ++i) o[i] = 0.0;
    for (int j = 0; j <= s; ++j) {
        const double* kj = Kseq + (size_t)j * G * dh + (size_t)g * dh;
        const double* vj = Vseq + (size_t)j * G * dh + (size_t)g * dh;
        double sc = 0.0;
        for (int i = 0; i < dh; ++i) sc += q[i] * kj[i];
        sc *= scale;
        const double a = exp(sc - m);
        den += a;
        for (int i = 0; i < dh; ++i) o[i] += a * vj[i];
    }
    for (int i = 0; i < dh; ++i) o[i] /= den;
}

/* ---------------------------------------------------------------------------------
 * One output token of the layer, given the routing of that token.
 *  - routed queries: q_{g,r} = x[t] @ Wq[idx[g][r]]  (only the selected experts are
 *    computed: [R] "Algorithm Overview", only the active query-head computation);
 *  - shared query:   q_s = x[t] @ Wqs, always on ([R], [T] "Always-On Shared Head");
 *  - with the rotary embedding, every query rotated at position pos0 + s;
 *  - each query attends causally to its group's dense K/V ([T] "Dense KV Path");
 *  - output construction by variant ([R] "Parameters"/"Ablations", [T] "Output
 *    Construction"):
 *      hard_concat:     y = sum_g sum_r o_{g,r} Wo[e] + o_s Wos
 *      weighted_concat: y = sum_g sum_r p_e o_{g,r} Wo[e] + o_s Wos
 *      gqe:             y = sum_g sum_r o_{g,r} Wo[e] + sum_g (sum_r w_r o_{g,r}) WoR[g]
 *                           + o_s Wos
 *    (o_s terms only when the shared head is on.)
 * w is recomputed from p and the given selection (renormalisation over the selected).
 * Shapes: Wq [N, d, dh], Wqs [d, dh], Wo [N, dh, d], WoR [G, dh, d], Wos [dh, d];
 * Kseq/Vseq: [S, G, dh] of the token's sequence; s = position of the token.
 * q_out/o_out (optional) receive [H_act, dh] in virtual-head order v = g k + r, then
 * the shared head.
 * --------------------------------------------------------------------------------- */
static void token_output(const oracle_cfg* c, int s, const double* xt, const double* pt,
                         const int32_t* idxt, const double* Wq, const double* Wqs,
                         const double* Kseq, const double* Vseq, const double* Wo,
                         const double* WoR, const double* Wos, double* yt, double* q_out,
                         double* o_out)
{
    const int d = c->dim, N = c->num_query_experts, G = c->num_kv_heads, k = c->top_k;
    const int dh = c->head_dim;
    (void)N;
    double* q = (double*)malloc(sizeof(double) * dh);
    double* o = (double*)malloc(sizeof(double) * dh);
    double* slot = (double*)malloc(sizeof(double) * dh);
    for (int i = 0; i < d; ++i) yt[i] = 0.0;

    for (int g = 0; g < G; ++g) {
        double psel = 0.0;
        for (int r = 0; r < k; ++r) psel += pt[idxt[g * k + r]];
        for (int i = 0; i < dh; ++i) slot[i] = 0.0;
        for (int r = 0; r < k; ++r) {
            const int e = idxt[g * k + r];
            for (int j = 0; j < dh; ++j) {
                double a = 0.0;
                for (int i = 0; i < d; ++i) a += xt[i] * Wq[((size_t)e * d + i) * dh + j];
                q[j] = a;
            }
            rope(q, dh, c->pos0 + s, c->rope_base);
            attend(s, dh, G, g, q, Kseq, Vseq, o);
            if (q_out) memcpy(q_out + (size_t)(g * k + r) * dh, q, sizeof(double) * dh);
            if (o_out) memcpy(o_out + (size_t)(g * k + r) * dh, o, sizeof(double) * dh);
            double coef = 1.0;
            if (c->variant == 1) coef = pt[e];
            for (int col = 0; col < d; ++col) {
                double a = 0.0;
                for (int j = 0; j < dh; ++j) a += o[j] * Wo[((size_t)e * dh + j) * d + col];
                yt[col] += coef * a;
            }
            const double wr = pt[e] / psel;
            for (int j = 0; j < dh; ++j) slot[j] += wr * o[j];
        }
        if (c->variant == 0) {
            for (int col = 0; col < d; ++col) {
                double a = 0.0;
                for (int j = 0; j < dh; ++j) a += slot[j] * WoR[((size_t)g * dh + j) * d + col];
                yt[col] += a;
            }
        }
    }
    if (c->shared_head) {
        for (int j = 0; j < dh; ++j) {
            double a = 0.0;
            for (int i = 0; i < d; ++i) a += xt[i] * Wqs[(size_t)i * dh + j];
            q[j] = a;
        }
        rope(q, dh, c->pos0 + s, c->rope_base);
        attend(s, dh, G, c->shared_kv_group, q, Kseq, Vseq, o);
        if (q_out) memcpy(q_out + (size_t)(G * k) * dh, q, sizeof(double) * dh);
        if (o_out) memcpy(o_out + (size_t)(G * k) * dh, o, sizeof(double) * dh);
        for (int col = 0; col < d; ++col) {
            double a = 0.0;
            for (int j = 0; j < dh; ++j) a += o[j] * Wos[(size_t)j * d + col];
            yt[col] += a;
        }
    }
    free(q);
    free(o);
    free(slot);
}

/* Layer output for a list of tokens (global ids t = b*S + s in [0, B*S)).
 * x [B*S, d]; p [B*S, N]; idx [B*S, G, k]; K, V [B*S, G, dh] from gqe_oracle_kv.
 * y [nrows, d]; q_out, o_out optional [nrows, H_act, dh]. */
int gqe_oracle_rows(const oracle_cfg* c, int64_t B, int64_t S, const double* x,
                    const double* p, const int32_t* idx, const double* Wq, const double* Wqs,
                    const double* K, const double* V, const double* Wo, const double* WoR,
                    const double* Wos, const int64_t* rows, int64_t nrows, double* y,
                    double* q_out, double* o_out)
{
    const int d = c->dim, N = c->num_query_experts, G = c->num_kv_heads, k = c->top_k;
    const int dh = c->head_dim;
    const int Hact = G * k + (c->shared_head ? 1 : 0);
    if (c->shared_head && (c->shared_kv_group < 0 || c->shared_kv_group >= G)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t t = rows[r];
        if (t < 0 || t >= B * S) continue;
        const int64_t b = t / S, s = t % S;
        const double* Kseq = K + (size_t)b * S * G * dh;
        const double* Vseq = V + (size_t)b * S * G * dh;
        token_output(c, (int)s, x + t * d, p + t * N, idx + t * G * k, Wq, Wqs, Kseq, Vseq,
                     Wo, WoR, Wos, y + r * d, q_out ? q_out + r * Hact * dh : NULL,
                     o_out ? o_out + r * Hact * dh : NULL);
    }
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Backward pass: gradients of  L = sum_t dy[t] . y[t] + aux_coef * aux  with respect to x and
 * every weight, the routing decisions idx held fixed (top-k is piecewise constant; the loss
 * of the README's "Usage" adds 0.01 * aux).  Each step is the chain rule applied to the
 * forward definition above, in reverse order:
 *  output construction   y += c o W_o[e]:  dW_o[e] += c o^T dy,  do += c dy W_o[e]^T;
 *                        weighted_concat (c = p_e): dp_e += o . (dy W_o[e]^T)
 *                        gqe slot y += (sum_r w_r o_r) W_oR[g]:  dW_oR[g] += slot^T dy,
 *                        do_r += w_r dy W_oR[g]^T,  dw_r = o_r . (dy W_oR[g]^T)
 *                        shared head y += o_s W_os:  dW_os += o_s^T dy,  do_s = dy W_os^T
 *  renormalisation       w_r = p_r / P, P = sum_sel p:  dp_r += (dw_r - sum_r' w_r' dw_r') / P
 *  aux loss              aux = (1/G) sum_g n sum_e f_e P_e, P_e = (1/T) sum_t p[t,e], f_e a
 *                        count (constant):  dp[t,e] += aux_coef n f_e / (G T)
 *  in-group softmax      dl_e = p_e (dp_e - sum_{e' in g} p_e' dp_e')
 *  router logits         dW_r += x^T dl,  db_r += dl,  dx += dl W_r^T
 *  attention             a_j = softmax_j(q . k_j / sqrt(dh)), j <= s:  dv_j += a_j do,
 *                        dz_j = a_j (do . v_j - do . o),  dq = sum_j dz_j k_j / sqrt(dh),
 *                        dk_j += dz_j q / sqrt(dh)
 *  rotary embedding      orthogonal rotation: the gradient is rotated back (angle -m theta)
 *  projections           dW_q[e] += x^T dq,  dx += dq W_q[e]^T;  likewise W_qs, W_k, W_v.
 * Every gradient output is overwritten (dWqs / dWos may be NULL without the shared head,
 * dWoR without the gqe slot).  Single-threaded: the key and value gradients of a token
 * collect contributions from all later tokens.  Small shapes only.
 * --------------------------------------------------------------------------------- */
int gqe_oracle_backward(const oracle_cfg* c, int64_t B, int64_t S, const double* x,
                        const double* Wr, const double* br, const double* Wq, const double* Wqs,
                        const double* Wk, const double* Wv, const double* Wo, const double* WoR,
                        const double* Wos, const int32_t* idx, const double* dy, double aux_coef,
                        double* dx, double* dWr, double* dbr, double* dWq, double* dWqs,
                        double* dWk, double* dWv, double* dWo, double* dWoR, double* dWos)
{
    const int d = c->dim, N = c->num_query_experts, G = c->num_kv_heads, k = c->top_k;
    const int n = N / G, dh = c->head_dim, W = G * dh;
    const int sh = c->shared_head ? 1 : 0, H = G * k + sh;
    const int64_t T = B * S;
    const double scale = 1.0 / sqrt((double)dh);
    if (N <= 0 || G <= 0 || N % G != 0 || k < 1 || k > n || n > 64) return -1;

    memset(dx, 0, sizeof(double) * T * d);
    memset(dWr, 0, sizeof(double) * d * N);
    memset(dbr, 0, sizeof(double) * N);
    memset(dWq, 0, sizeof(double) * N * d * dh);
    memset(dWk, 0, sizeof(double) * d * W);
    memset(dWv, 0, sizeof(double) * d * W);
    memset(dWo, 0, sizeof(double) * N * dh * d);
    if (dWqs) memset(dWqs, 0, sizeof(double) * d * dh);
    if (dWos) memset(dWos, 0, sizeof(double) * dh * d);
    if (dWoR) memset(dWoR, 0, sizeof(double) * G * dh * d);

    /* ---- forward quantities: router probabilities, K/V, per-head queries, attention weights, outputs */
    double* logits = (double*)malloc(sizeof(double) * N);
    double* p = (double*)malloc(sizeof(double) * T * N);
    int32_t* tidx = (int32_t*)malloc(sizeof(int32_t) * G * k);
    double* tw = (double*)malloc(sizeof(double) * G * k);
    double* tgap = (double*)malloc(sizeof(double) * G);
    for (int64_t t = 0; t < T; ++t) router_token(c, x + t * d, Wr, br, logits, p + t * N, tidx, tw, tgap);
    double* K = (double*)malloc(sizeof(double) * T * W);
    double* V = (double*)malloc(sizeof(double) * T * W);
    gqe_oracle_kv(c, T, S, x, Wk, Wv, K, V);
    double* q = (double*)calloc((size_t)T * H * dh, sizeof(double));
    double* o = (double*)calloc((size_t)T * H * dh, sizeof(double));
    double* a = (double*)calloc((size_t)T * H * S, sizeof(double));   /* a[t][h][j], j <= s */
    for (int64_t t = 0; t < T; ++t) {
        const int64_t b = t / S, s = t % S;
        for (int h = 0; h < H; ++h) {
            const int routed = h < G * k;
            const int g = routed ? h / k : c->shared_kv_group;
            const int e = routed ? idx[t * G * k + h] : -1;
            double* qh = q + ((size_t)t * H + h) * dh;
            for (int j = 0; j < dh; ++j) {
                double acc = 0.0;
                for (int i = 0; i < d; ++i)
                    acc += x[t * d + i] * (routed ? Wq[((size_t)e * d + i) * dh + j] : Wqs[(size_t)i * dh + j]);
                qh[j] = acc;
            }
            rope(qh, dh, c->pos0 + s, c->rope_base);
            double* ah = a + ((size_t)t * H + h) * S;
            double m = -INFINITY;
            for (int64_t js = 0; js <= s; ++js) {
                const double* kj = K + (size_t)(b * S + js) * W + (size_t)g * dh;
                double sc = 0.0;
                for (int i = 0; i < dh; ++i) sc += qh[i] * kj[i];
                ah[js] = sc * scale;
                if (ah[js] > m) m = ah[js];
            }
            double den = 0.0;
            for (int64_t js = 0; js <= s; ++js) { ah[js] = exp(ah[js] - m); den += ah[js]; }
            for (int64_t js = 0; js <= s; ++js) ah[js] /= den;
            double* oh = o + ((size_t)t * H + h) * dh;
            for (int64_t js = 0; js <= s; ++js) {
                const double* vj = V + (size_t)(b * S + js) * W + (size_t)g * dh;
                for (int i = 0; i < dh; ++i) oh[i] += ah[js] * vj[i];
            }
        }
    }
    int64_t* counts = (int64_t*)calloc(N, sizeof(int64_t));
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < G * k; ++i) counts[idx[t * G * k + i]] += 1;

    /* ---- output construction, renormalisation, aux, softmax and router */
    double* dob = (double*)calloc((size_t)T * H * dh, sizeof(double));
    double* u = (double*)malloc(sizeof(double) * dh);
    double* vg = (double*)malloc(sizeof(double) * dh);
    double* slot = (double*)malloc(sizeof(double) * dh);
    double* dp = (double*)malloc(sizeof(double) * N);
    double* dw = (double*)malloc(sizeof(double) * k);
    for (int64_t t = 0; t < T; ++t) {
        const double* dyt = dy + t * d;
        const double* pt = p + t * N;
        for (int e = 0; e < N; ++e) dp[e] = 0.0;
        for (int g = 0; g < G; ++g) {
            double psel = 0.0;
            for (int r = 0; r < k; ++r) psel += pt[idx[t * G * k + g * k + r]];
            if (c->variant == 0) {
                for (int j = 0; j < dh; ++j) {
                    double acc = 0.0;
                    for (int col = 0; col < d; ++col) acc += dyt[col] * WoR[((size_t)g * dh + j) * d + col];
                    vg[j] = acc;
                    slot[j] = 0.0;
                }
                for (int r = 0; r < k; ++r) {
                    const double wr = pt[idx[t * G * k + g * k + r]] / psel;
                    const double* orr = o + ((size_t)t * H + g * k + r) * dh;
                    for (int j = 0; j < dh; ++j) slot[j] += wr * orr[j];
                }
                for (int j = 0; j < dh; ++j)
                    for (int col = 0; col < d; ++col) dWoR[((size_t)g * dh + j) * d + col] += slot[j] * dyt[col];
            }
            for (int r = 0; r < k; ++r) {
                const int e = idx[t * G * k + g * k + r];
                const double* orr = o + ((size_t)t * H + g * k + r) * dh;
                double* dorr = dob + ((size_t)t * H + g * k + r) * dh;
                const double coef = c->variant == 1 ? pt[e] : 1.0;
                double ou = 0.0, ov = 0.0;
                for (int j = 0; j < dh; ++j) {
                    double acc = 0.0;
                    for (int col = 0; col < d; ++col) acc += dyt[col] * Wo[((size_t)e * dh + j) * d + col];
                    u[j] = acc;
                    ou += orr[j] * acc;
                    for (int col = 0; col < d; ++col) dWo[((size_t)e * dh + j) * d + col] += coef * orr[j] * dyt[col];
                    dorr[j] = coef * acc;
                }
                if (c->variant == 1) dp[e] += ou;
                if (c->variant == 0) {
                    const double wr = pt[e] / psel;
                    for (int j = 0; j < dh; ++j) {
                        dorr[j] += wr * vg[j];
                        ov += orr[j] * vg[j];
                    }
                    dw[r] = ov;
                }
            }
            if (c->variant == 0) {
                double sw = 0.0;
                for (int r = 0; r < k; ++r) sw += (pt[idx[t * G * k + g * k + r]] / psel) * dw[r];
                for (int r = 0; r < k; ++r) dp[idx[t * G * k + g * k + r]] += (dw[r] - sw) / psel;
            }
        }
        if (sh) {
            const double* os = o + ((size_t)t * H + G * k) * dh;
            double* dos = dob + ((size_t)t * H + G * k) * dh;
            for (int j = 0; j < dh; ++j) {
                double acc = 0.0;
                for (int col = 0; col < d; ++col) {
                    acc += dyt[col] * Wos[(size_t)j * d + col];
                    dWos[(size_t)j * d + col] += os[j] * dyt[col];
                }
                dos[j] = acc;
            }
        }
        for (int e = 0; e < N; ++e)
            dp[e] += aux_coef * (double)n * ((double)counts[e] / ((double)T * (double)k)) / ((double)G * (double)T);
        for (int g = 0; g < G; ++g) {
            double sdp = 0.0;
            for (int j = 0; j < n; ++j) sdp += pt[g * n + j] * dp[g * n + j];
            for (int j = 0; j < n; ++j) {
                const int e = g * n + j;
                const double dl = pt[e] * (dp[e] - sdp);
                dbr[e] += dl;
                for (int i = 0; i < d; ++i) {
                    dWr[(size_t)i * N + e] += x[t * d + i] * dl;
                    dx[t * d + i] += Wr[(size_t)i * N + e] * dl;
                }
            }
        }
    }

    /* ---- attention */
    double* dq = (double*)calloc((size_t)T * H * dh, sizeof(double));
    double* dK = (double*)calloc((size_t)T * W, sizeof(double));
    double* dV = (double*)calloc((size_t)T * W, sizeof(double));
    for (int64_t t = 0; t < T; ++t) {
        const int64_t b = t / S, s = t % S;
        for (int h = 0; h < H; ++h) {
            const int g = h < G * k ? h / k : c->shared_kv_group;
            const double* doh = dob + ((size_t)t * H + h) * dh;
            const double* oh = o + ((size_t)t * H + h) * dh;
            const double* qh = q + ((size_t)t * H + h) * dh;
            const double* ah = a + ((size_t)t * H + h) * S;
            double* dqh = dq + ((size_t)t * H + h) * dh;
            double D = 0.0;
            for (int i = 0; i < dh; ++i) D += doh[i] * oh[i];
            for (int64_t js = 0; js <= s; ++js) {
                const int64_t tj = b * S + js;
                const double* kj = K + (size_t)tj * W + (size_t)g * dh;
                const double* vj = V + (size_t)tj * W + (size_t)g * dh;
                double dA = 0.0;
                for (int i = 0; i < dh; ++i) dA += doh[i] * vj[i];
                const double dz = ah[js] * (dA - D);
                for (int i = 0; i < dh; ++i) {
                    dqh[i] += dz * kj[i] * scale;
                    dK[(size_t)tj * W + (size_t)g * dh + i] += dz * qh[i] * scale;
                    dV[(size_t)tj * W + (size_t)g * dh + i] += ah[js] * doh[i];
                }
            }
        }
    }

    /* ---- rotary embedding (rotate back), then the projections */
    for (int64_t t = 0; t < T; ++t) {
        const int64_t s = t % S;
        for (int h = 0; h < H; ++h) rope(dq + ((size_t)t * H + h) * dh, dh, -(c->pos0 + s), c->rope_base);
        for (int g = 0; g < G; ++g) rope(dK + (size_t)t * W + (size_t)g * dh, dh, -(c->pos0 + s), c->rope_base);
    }
    for (int64_t t = 0; t < T; ++t) {
        const double* xt = x + t * d;
        for (int h = 0; h < H; ++h) {
            const int routed = h < G * k;
            const int e = routed ? idx[t * G * k + h] : -1;
            const double* dqh = dq + ((size_t)t * H + h) * dh;
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dh; ++j) {
                    if (routed) {
                        dWq[((size_t)e * d + i) * dh + j] += xt[i] * dqh[j];
                        acc += Wq[((size_t)e * d + i) * dh + j] * dqh[j];
                    } else {
                        dWqs[(size_t)i * dh + j] += xt[i] * dqh[j];
                        acc += Wqs[(size_t)i * dh + j] * dqh[j];
                    }
                }
                dx[t * d + i] += acc;
            }
        }
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int col = 0; col < W; ++col) {
                dWk[(size_t)i * W + col] += xt[i] * dK[(size_t)t * W + col];
                dWv[(size_t)i * W + col] += xt[i] * dV[(size_t)t * W + col];
                acc += Wk[(size_t)i * W + col] * dK[(size_t)t * W + col] + Wv[(size_t)i * W + col] * dV[(size_t)t * W + col];
            }
            dx[t * d + i] += acc;
        }
    }
    free(logits); free(p); free(tidx); free(tw); free(tgap); free(K); free(V); free(q); free(o);
    free(a); free(counts); free(dob); free(u); free(vg); free(slot); free(dp); free(dw); free(dq);
    free(dK); free(dV);
    return 0;
}
