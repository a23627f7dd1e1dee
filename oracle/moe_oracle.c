/*
 * CPU oracle for one MoE layer's forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C.  Every floating-point reduction is carried
 * in double and rounded only at the points named below.  Nothing here is
 * shared with the HIP library (no headers, helpers or tables); only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.
 *
 * What each function follows is cited by page title and section:
 *   [PF]  "PopFetcher: Towards Accelerated Mixture-of-Experts Training Via
 *          Popularity Based Expert-Wise Prefetch (ATC 2025)" (wiki summary)
 *   [GPS] "MoE-GPS框架：动态专家复制的负载均衡优化策略" (blog)
 *   [EPS] "EPS-MoE: Expert Pipeline Scheduler for Cost-Efficient MoE Inference"
 *   [MPMC]"Fast MoE Inference via Predictive Prefetching and Expert Replication"
 * Where the pages leave a step open, the reading taken is stated in place.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

/* Round a double to the nearest bf16 value (ties to even), returned as bits.
 * bf16 keeps 8 significant bits; the value is scaled so that its significand
 * is an integer in [128, 256) and rounded with rint() (default mode: nearest,
 * ties to even).  Subnormal bf16 values share fp32's spacing 2^-133. */
static uint16_t bf16_from_double(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    double q;
    if (e - 1 < -126) {                 /* bf16 subnormal range */
        q = ldexp(rint(ldexp(a, 133)), -133);
    } else {
        q = ldexp(rint(ldexp(a, 8 - e)), e - 8);
    }
    float f = (float)q;                 /* exact: q has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t b = (uint16_t)(u >> 16);
    return v < 0 ? (uint16_t)(b | 0x8000u) : b;
}

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* dtype codes: 0 = fp32, 1 = bf16 (bit patterns in uint16) */
static double load_elem(const void* p, int dt, int64_t i) {
    return dt == 1 ? bf16_to_double(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

static void store_elem(void* p, int dt, int64_t i, double v) {
    if (dt == 1) ((uint16_t*)p)[i] = bf16_from_double(v);
    else ((float*)p)[i] = (float)v;
}

/* Round a double to the activation dtype and return the rounded value. */
static double round_to_dtype(double v, int dt) {
    return dt == 1 ? bf16_to_double(bf16_from_double(v)) : (double)(float)v;
}

int oracle_bf16_round_bits(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_from_double(v[i]);
    return 0;
}

/* ------------------------------------------------------------------ route */
/*
 * Top-k softmax gate ([PF] observations/trade-offs: the naive top-k gate;
 * [MPMC] problem statement: softmax-based routing).  The pages do not print
 * the gate's equations; the reading taken:
 *   - experts are ordered by logit descending, equal logits by expert index
 *     ascending; slots 0..k-1 take the first k in that order (slot 0 = top-1);
 *   - p_e = softmax over all E logits (computed in double with the max
 *     subtracted);
 *   - the kept probabilities are renormalised to sum to one:
 *     w_i = p_{idx_i} / sum_j p_{idx_j}, rounded to fp32.
 * Selection compares the fp32 logits themselves, so no rounding decides it.
 */
int oracle_route(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w) {
    if (E < 1 || E > 4096 || k < 1 || k > E) return -1;
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int i = 0; i < k; ++i) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: lower index wins ties */
            }
            taken[best] = 1;
            idx[t * k + i] = best;
        }
        double m = (double)l[idx[t * k]];
        double z = 0.0;
        for (int e = 0; e < E; ++e) { p[e] = exp((double)l[e] - m); z += p[e]; }
        for (int e = 0; e < E; ++e) p[e] /= z;
        double kept = 0.0;
        for (int i = 0; i < k; ++i) kept += p[idx[t * k + i]];
        for (int i = 0; i < k; ++i) w[t * k + i] = (float)(p[idx[t * k + i]] / kept);
    }
    free(taken);
    free(p);
    return 0;
}

/* -------------------------------------------------------------- statistics */
/*
 * Per-expert load n[e] = number of (token, slot) pairs routed to e
 * ([PF] Routing Information Collector / observation 1; [GPS] 2.1: n_i, the
 * tokens handled by expert i).
 */
int oracle_histogram(const int32_t* idx, int64_t T, int k, int E, int32_t* counts) {
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t j = 0; j < T * k; ++j) {
        int e = idx[j];
        if (e < 0 || e >= E) return -1;
        counts[e] += 1;
    }
    return 0;
}

/*
 * Layer-to-layer co-occurrence behind [PF] Eq.(2) (observation 2: given that
 * layer j selects expert x, how often layer j+1 selects x').  With top-k at
 * both layers every one of a token's k x k (previous, next) pairs is counted:
 * C[a*E + b] = #{(t,i,j) : prev[t,i] = a and next[t,j] = b}.
 */
int oracle_cooccurrence(const int32_t* prev, const int32_t* next, int64_t T, int k, int E, int32_t* C) {
    for (int64_t q = 0; q < (int64_t)E * E; ++q) C[q] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < k; ++i)
            for (int j = 0; j < k; ++j) {
                int a = prev[t * k + i], b = next[t * k + j];
                if (a < 0 || a >= E || b < 0 || b >= E) return -1;
                C[(int64_t)a * E + b] += 1;
            }
    return 0;
}

/*
 * Sequence popularity, [PF] Eq.(1) (not printed; [GPS] 2.1 gives p_i = n_i/N
 * with a sliding-window average): the share of the window's assignments that
 * went to each expert, p[e] = Nw[e] / sum_e Nw[e], where Nw sums the last s
 * iterations' counts.  Both operands are exact integers in fp32, and the fp32
 * division is correctly rounded.  An empty window gives zeros.
 */
int oracle_popularity(const int64_t* Nw, int E, float* p_seq) {
    int64_t tot = 0;
    for (int e = 0; e < E; ++e) tot += Nw[e];
    for (int e = 0; e < E; ++e) p_seq[e] = tot > 0 ? (float)Nw[e] / (float)tot : 0.0f;
    return 0;
}

/*
 * Conditional probability Pr(E^{b,l+1} | E^{a,l}), [PF] Eq.(2): the windowed
 * co-occurrence normalised per previous-layer expert a (each row sums to one;
 * a row with no mass stays zero).
 */
int oracle_conditional(const int64_t* Cw, int E, float* P) {
    for (int a = 0; a < E; ++a) {
        int64_t row = 0;
        for (int b = 0; b < E; ++b) row += Cw[(int64_t)a * E + b];
        for (int b = 0; b < E; ++b)
            P[(int64_t)a * E + b] = row > 0 ? (float)Cw[(int64_t)a * E + b] / (float)row : 0.0f;
    }
    return 0;
}

/*
 * Next-layer popularity, [PF] Eq.(3): propagate this layer's sequence
 * popularity through the conditional matrix,
 *   p_hat[b] = sum_a p_seq[a] * P[a,b]   (a ascending, double, then fp32).
 */
int oracle_predict_next(const float* p_seq, const float* P, int E, float* p_hat) {
    for (int b = 0; b < E; ++b) {
        double s = 0.0;
        for (int a = 0; a < E; ++a) s += (double)p_seq[a] * (double)P[(int64_t)a * E + b];
        p_hat[b] = (float)s;
    }
    return 0;
}

/*
 * Decayed window popularity ([GPS] 2.1: the sliding-window average is given a
 * decay factor against distribution drift).  Reading taken: the m recorded
 * iterations of the window, youngest first (hist[age*E + e], age 0 = the
 * current iteration), weigh lambda^age; the weights are formed by repeated
 * multiplication w_0 = 1, w_{j+1} = w_j * lambda and D[e] = sum_age w_age *
 * n_e(age) is taken in age order, all in double; p[e] = D[e] / sum_e D[e]
 * (expert order; 0 when the sum is 0), rounded to fp32.  lambda = 1 is the
 * plain window of Eq.(1); lambda = 0 keeps the current iteration only.
 */
int oracle_decayed_popularity(const int32_t* hist, int m, int E, double lambda, float* p) {
    double* D = (double*)calloc((size_t)E, sizeof(double));
    double w = 1.0;
    for (int age = 0; age < m; ++age) {
        for (int e = 0; e < E; ++e) D[e] = D[e] + w * (double)hist[(int64_t)age * E + e];
        w = w * lambda;
    }
    double tot = 0.0;
    for (int e = 0; e < E; ++e) tot = tot + D[e];
    for (int e = 0; e < E; ++e) p[e] = tot > 0.0 ? (float)(D[e] / tot) : 0.0f;
    free(D);
    return 0;
}

/*
 * Load-state check ([GPS] 6.1: a load departing from its expectation by more
 * than twice the history's standard deviation triggers re-evaluation; the
 * load-prediction study's transient state of obvious load fluctuation versus
 * the stable state of temporal locality).  Reading taken: the history is the
 * m - 1 window iterations before the current one (ages 1 .. m-1); with h = m-1
 * >= 2, expert e is anomalous when (n_e - mu_e)^2 > 4 var_e, mu_e and var_e
 * being the history's mean and population variance (double, age order; the
 * square form avoids a square root); with h < 2 every expert is flagged, there
 * being no history to trust.  The layer is transient when more than a fifth of
 * its experts are flagged (5 * n_flagged > E; the fraction is a chosen
 * constant, the pages print none).
 */
int oracle_load_anomalies(const int32_t* hist, int m, int E, int32_t* flags, int32_t* summary) {
    const int h = m - 1;
    int32_t n = 0;
    for (int e = 0; e < E; ++e) {
        int f = 1;
        if (h >= 2) {
            double s = 0.0;
            for (int age = 1; age < m; ++age) s = s + (double)hist[(int64_t)age * E + e];
            const double mu = s / (double)h;
            double v = 0.0;
            for (int age = 1; age < m; ++age) {
                const double d = (double)hist[(int64_t)age * E + e] - mu;
                v = v + d * d;
            }
            v = v / (double)h;
            const double d0 = (double)hist[e] - mu;
            f = d0 * d0 > 4.0 * v;
        }
        flags[e] = f;
        n += f;
    }
    summary[0] = n;
    summary[1] = 5 * n > E;
    return 0;
}

/*
 * Replica counts for hot experts.  [GPS] 2.1's duplicate_experts rule gives an
 * expert whose load exceeds the target ceil(load/target) - 1 extra copies;
 * [MPMC] contribution 3 bounds the replica count by a memory budget, and [PF]
 * fills its budget greedily by popularity.  Reading taken: target mu = T*k/E
 * with threshold 1.0 (not 1.2), and a budget of R extra slots filled one at a
 * time, each going to the expert with the largest per-copy load n_e/(r_e+1)
 * among those still above target (n_e > mu*(r_e+1)); equal per-copy loads go
 * to the lower expert index; stop when none qualifies.  All comparisons are
 * exact integer cross-multiplications.
 */
int oracle_replicas(const int32_t* counts, int E, int64_t T, int k, int R, int32_t* r) {
    for (int e = 0; e < E; ++e) r[e] = 0;
    const int64_t tk = T * (int64_t)k;
    for (int step = 0; step < R; ++step) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            int64_t n = counts[e];
            if (!(n * E > tk * (int64_t)(r[e] + 1))) continue;     /* still above target? */
            if (best < 0 || n * (int64_t)(r[best] + 1) > (int64_t)counts[best] * (int64_t)(r[e] + 1))
                best = e;
        }
        if (best < 0) break;
        r[best] += 1;
    }
    return 0;
}

/*
 * Replicas planned ahead of routing.  [MPMC] contribution 2-3 and [PF] plan the
 * replica placement from predicted expert activity before the layer runs; the
 * prediction here is [PF] Eq.(3)'s next-layer popularity p_hat.  Reading
 * taken: predicted rows c_hat[e] = p_hat[e] * total (total = T*k of the layer
 * to come), the product taken in double and rounded to the nearest integer
 * with halves to even; NaN, zero or negative shares give 0 and values at or
 * past 2^31 - 1 clamp there.  The plan is then the greedy rule of
 * oracle_replicas applied to c_hat with sum(c_hat) standing for T*k.
 */
int oracle_predicted_counts(const float* p_hat, int E, int64_t total, int32_t* c_hat) {
    for (int e = 0; e < E; ++e) {
        double v = (double)p_hat[e] * (double)total;
        if (!(v > 0.0)) c_hat[e] = 0;
        else if (v >= 2147483647.0) c_hat[e] = 2147483647;
        else c_hat[e] = (int32_t)nearbyint(v);
    }
    return 0;
}

int oracle_plan_replicas(const float* p_hat, int E, int64_t total, int R, int32_t* c_hat, int32_t* r) {
    oracle_predicted_counts(p_hat, E, total, c_hat);
    int64_t sum = 0;
    for (int e = 0; e < E; ++e) sum += c_hat[e];
    return oracle_replicas(c_hat, E, sum, 1, R, r);
}

/* rank order of the top-n: value descending, then expert index ascending; NaN counts as -inf */
static double rank_value(double v) { return v != v ? -INFINITY : v; }

static void top_n_set(const double* v, int E, int n, unsigned char* in) {
    for (int e = 0; e < E; ++e) in[e] = 0;
    for (int j = 0; j < n; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!in[e] && (best < 0 || rank_value(v[e]) > rank_value(v[best]))) best = e;
        in[best] = 1;
    }
}

/*
 * How well a prediction matched the routing that followed, and how evenly a
 * replica plan spread the rows ([MPMC] reports prediction accuracy and load
 * balance; the load-prediction study measures prediction error of expert
 * load; [GPS] 2.1 targets per-copy load near the mean).  Definitions taken:
 *   out[0] total-variation distance 0.5 * sum_e |q_e - a_e| between the
 *          prediction normalised to sum one (q = p_hat / sum p_hat) and the
 *          actual shares a = counts / sum counts; 1 if either sum is not > 0;
 *   out[1] top-n hit rate: |top_n(p_hat) & top_n(counts)| / n, n = min(top_n, E);
 *   out[2] population standard deviation of the per-slot row loads, expert e
 *          with r_e replicas being cut into r_e + 1 chunks as dispatch cuts it
 *          (chunk rho holds floor((rho+1) n_e/(r_e+1)) - floor(rho n_e/(r_e+1)));
 *   out[3] largest slot load over the mean slot load sum(counts)/slots (0 if
 *          there are no rows).
 * Sums run in expert (slot) order in double; each output is rounded to fp32 once.
 * replicas == NULL means one slot per expert; replica counts are clamped to
 * [0, 4096] (the largest budget a plan hands out).
 */
static int64_t copies_of(const int32_t* replicas, int e) {
    if (!replicas) return 1;
    int32_t r = replicas[e] < 0 ? 0 : replicas[e];
    return 1 + (r > 4096 ? 4096 : r);
}

int oracle_prediction_quality(const float* p_hat, const int32_t* counts, int E, const int32_t* replicas,
                              int top_n, float* out) {
    if (E < 1 || top_n < 1) return -1;
    double S = 0.0;
    int64_t A = 0;
    for (int e = 0; e < E; ++e) {
        S += (double)p_hat[e];
        A += counts[e];
    }
    double tv = 1.0;
    if (S > 0.0 && A > 0) {
        double acc = 0.0;
        for (int e = 0; e < E; ++e) acc += fabs((double)p_hat[e] / S - (double)counts[e] / (double)A);
        tv = 0.5 * acc;
    }
    const int n = top_n < E ? top_n : E;
    double* vp = (double*)malloc(sizeof(double) * (size_t)E);
    double* vc = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* ip = (unsigned char*)malloc((size_t)E);
    unsigned char* ic = (unsigned char*)malloc((size_t)E);
    for (int e = 0; e < E; ++e) {
        vp[e] = (double)p_hat[e];
        vc[e] = (double)counts[e];
    }
    top_n_set(vp, E, n, ip);
    top_n_set(vc, E, n, ic);
    int hit = 0;
    for (int e = 0; e < E; ++e) hit += ip[e] && ic[e];
    free(vp); free(vc); free(ip); free(ic);

    int64_t slots = 0, mx = 0;
    for (int e = 0; e < E; ++e) slots += copies_of(replicas, e);
    const double mean = (double)A / (double)slots;
    double var = 0.0;
    for (int e = 0; e < E; ++e) {
        const int64_t copies = copies_of(replicas, e);
        const int64_t ne = counts[e];
        for (int64_t rho = 0; rho < copies; ++rho) {
            const int64_t load = ((rho + 1) * ne) / copies - (rho * ne) / copies;
            const double d = (double)load - mean;
            var += d * d;
            if (load > mx) mx = load;
        }
    }
    out[0] = (float)tv;
    out[1] = (float)((double)hit / (double)n);
    out[2] = (float)sqrt(var / (double)slots);
    out[3] = A > 0 ? (float)((double)mx / mean) : 0.0f;
    return 0;
}

/*
 * Dispatch: group the (token, slot) pairs by expert into contiguous rows.
 * Experts occupy consecutive row ranges (exclusive prefix sum of the counts);
 * inside an expert the rows follow ascending token index.  perm_src[row] is
 * the source token, inv_pos[t*k+i] the row holding (t, idx[t,i]).  With
 * replicas, expert e's rows are cut into r_e+1 contiguous chunks in token
 * order, chunk rho being [off_e + floor(rho*n_e/(r_e+1)), off_e +
 * floor((rho+1)*n_e/(r_e+1))) -- one slot each, slots expert-major
 * ([MPMC] method: replicas of one expert serve disjoint token subsets).
 * replicas == NULL means no replication (one slot per expert).
 */
int oracle_dispatch(const int32_t* idx, int64_t T, int k, int E, const int32_t* replicas,
                    int32_t* expert_off, int32_t* perm_src, int32_t* inv_pos,
                    int32_t* slot_off, int32_t* slot_expert, int32_t* n_slots) {
    int32_t* n = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int64_t j = 0; j < T * k; ++j) {
        if (idx[j] < 0 || idx[j] >= E) { free(n); free(fill); return -1; }
        n[idx[j]] += 1;
    }
    expert_off[0] = 0;
    for (int e = 0; e < E; ++e) expert_off[e + 1] = expert_off[e] + n[e];
    for (int e = 0; e < E; ++e) fill[e] = expert_off[e];
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < k; ++i) {
            int e = idx[t * k + i];
            int32_t row = fill[e]++;
            perm_src[row] = (int32_t)t;
            inv_pos[t * k + i] = row;
        }
    int s = 0;
    for (int e = 0; e < E; ++e) {
        int copies = 1 + (replicas ? replicas[e] : 0);
        for (int rho = 0; rho < copies; ++rho) {
            slot_expert[s] = e;
            slot_off[s] = expert_off[e] + (int32_t)(((int64_t)rho * n[e]) / copies);
            ++s;
        }
    }
    slot_off[s] = expert_off[E];
    *n_slots = s;
    free(n);
    free(fill);
    return 0;
}

/* Row permutation X_perm[row] = X[perm_src[row]], a byte copy. */
int oracle_permute(const void* x, int64_t T, int64_t row_bytes, const int32_t* perm_src, int64_t M,
                   void* x_perm) {
    for (int64_t r = 0; r < M; ++r) {
        int32_t t = perm_src[r];
        if (t < 0 || t >= T) return -1;
        memcpy((char*)x_perm + r * row_bytes, (const char*)x + (int64_t)t * row_bytes, (size_t)row_bytes);
    }
    return 0;
}

/* ------------------------------------------------------------- expert FFN */
/*
 * One expert's FFN applied to independent rows.  [EPS] section 3 names the
 * gate, up and down matrices of the expert FFN; the activations are the ones
 * the workloads name (pages silent on their form).  Weights use the
 * [out, in] layout: w_gate, w_up are [I, H], w_down is [H, I] for this expert.
 *   SwiGLU: g = Wg x, u = Wu x, a = silu(g) * u with silu(z) = z / (1 + e^-z),
 *           a rounded to the activation dtype, y = Wd a.
 *   GELU:   z = W1 x, a = z/2 * (1 + erf(z / sqrt 2)) rounded to the dtype,
 *           y = W2 a.
 * Dot products are double sums of exact products; y is rounded to the dtype.
 * act: 0 = SwiGLU, 1 = GELU (w_up unused).  dt: 0 = fp32, 1 = bf16 bits.
 * x: n_rows x H, expert[j] picks the expert of row j, y: n_rows x H.
 */
int oracle_ffn_rows(const void* x, int dt, int64_t n_rows, int H, int I, const int32_t* expert, int E,
                    const void* w_gate, const void* w_up, const void* w_down, int act, void* y) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    for (int64_t j = 0; j < n_rows; ++j) {
        int e = expert[j];
        if (e < 0 || e >= E) { free(xr); free(a); return -1; }
        for (int h = 0; h < H; ++h) xr[h] = load_elem(x, dt, j * H + h);
        const int64_t wbase = (int64_t)e * I * H;     /* same for [I,H] and [H,I] */
        for (int i = 0; i < I; ++i) {
            double g = 0.0;
            for (int h = 0; h < H; ++h) g += load_elem(w_gate, dt, wbase + (int64_t)i * H + h) * xr[h];
            double v;
            if (act == 0) {
                double u = 0.0;
                for (int h = 0; h < H; ++h) u += load_elem(w_up, dt, wbase + (int64_t)i * H + h) * xr[h];
                v = g / (1.0 + exp(-g)) * u;
            } else {
                v = 0.5 * g * (1.0 + erf(g / sqrt(2.0)));
            }
            a[i] = round_to_dtype(v, dt);
        }
        for (int h = 0; h < H; ++h) {
            double s = 0.0;
            for (int i = 0; i < I; ++i) s += load_elem(w_down, dt, wbase + (int64_t)h * I + i) * a[i];
            store_elem(y, dt, j * H + h, s);
        }
    }
    free(xr);
    free(a);
    return 0;
}

/* ---------------------------------------------------------------- combine */
/*
 * Weighted combine back to token order ([EPS] section 3: the LocalReduce after
 * the expert computation): out[t] = sum_i w[t,i] * Y[inv_pos[t*k+i]], in
 * double, rounded to the dtype.
 */
int oracle_combine(const void* y_perm, int dt, int64_t M, const int32_t* inv_pos, const float* w,
                   int64_t T, int k, int H, void* out) {
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            double s = 0.0;
            for (int i = 0; i < k; ++i) {
                int32_t r = inv_pos[t * k + i];
                if (r < 0 || r >= M) return -1;
                s += (double)w[t * k + i] * load_elem(y_perm, dt, (int64_t)r * H + h);
            }
            store_elem(out, dt, t * H + h, s);
        }
    return 0;
}
