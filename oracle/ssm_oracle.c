/*
 * Selective-scan ORACLE -- test infrastructure, not product code.
 *
 * A plain, slow, sequential float64 evaluation of what the HIP library
 * computes.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it.  It shares no code, header or table with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *  - "mambazip mamba1/model.rs" (docs.infotheory.dev), forward_impl's
 *    per-channel step and selective_scan_state16: per state j,
 *    decay = exp(dt * A[ch][j]), h_j = h_j * decay + (u * dt) * B_j,
 *    y = D[ch] * u + sum_j C_j * h_j; softplus with a threshold of 20.
 *  - "ggmlR tests/testthat/test-ssm-rwkv.R" (rdrr.io): the ssm_conv and
 *    ssm_scan operand shapes (make_scan), the packed output (sequence output
 *    then final state), ids selecting one state row per sequence, and the
 *    depthwise convolution written out in R (the last tap multiplies the
 *    newest input).
 *  - "kizzasi-model backprop_ssm.rs" (docs.rs), ssm_backward: the adjoint
 *    dL/dh_t = C^T dL/dy_t + A_bar dL/dh_{t+1}, with dL/dh_0 = A_bar dL/dh_1.
 *  - "mambazip mamba1/model.rs", accumulate_token_step_gradients: the
 *    per-element gradients of the selective step (dC, dB, d(u), d(dt), dA, dD).
 *  - "ggmlR tests/testthat/test-ssm-rwkv.R", the ssm_conv backward block:
 *    ggml_ssm_conv_back packs the gradient of sx then that of the conv
 *    weights; its tests compare both with a central difference and give the
 *    weight gradient of loss = sum(output) in closed form.
 *  - The backward of the fused conv + SiLU is the chain rule through the
 *    forward above (the d_conv-1 conv-state inputs, then the tokens; SiLU's
 *    derivative sigma(c)(1 + c(1 - sigma(c))); each tap's adjoint), in the
 *    order the ggmlR page's ssm_conv backward block fixes for the
 *    standalone op: the gradient of the inputs, then of the conv weights.
 *  - "mambazip mamba1/model.rs", forward_impl's single-token step: the conv
 *    window of the last d_conv-1 inputs plus the new one (depthwise_conv_step),
 *    SiLU, dt = softplus(dt_raw + dt_bias), the in-place state update of
 *    selective_scan_state16, and the output times SiLU(z).
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes): dt is used as given unless the softplus flag is set; the initial
 * state of sequence i is row ids[i] of s and its final state is written to
 * row i of the state block; head h uses B/C group h / (n_head / n_group);
 * D multiplies the scan input u (the conv+SiLU output when the conv is fused).
 *
 * Layouts are row-major, slowest axis first (see the ssm_inputs module).
 * Every function returns 0 on success and a negative code on bad arguments.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n_seqs, n_tokens, n_head, head_dim, d_state, n_group, n_state_rows;
    int32_t a_per_state; /* 1: A[n_head][d_state]; 0: A[n_head] */
    int32_t d_conv;      /* 0: x is the scan input; K > 0: u = SiLU(conv_K(x)) */
    int32_t has_D;
    int32_t dt_softplus; /* 1: dt := softplus(dt) before use */
} oracle_dims;

typedef struct {
    const oracle_dims *d;
    const int64_t *grp_of_head;
    const double *s, *x, *dt, *A, *B, *C, *D, *conv_w, *conv_state;
    const int32_t *ids;
    /* forward outputs */
    double *y, *state_out, *conv_state_out;
    /* backward inputs / outputs */
    const double *dy, *dstate;
    double *d_s, *d_x, *d_dt, *d_A, *d_D, *d_conv_w, *d_conv_state;
    double *dB_part, *dC_part; /* [n_threads][n_seqs][L][G][N] */
    int n_threads;
    int tid;
    int backward;
} job_t;

static double softplus(double v) { return v > 20.0 ? v : log1p(exp(v)); }
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }
static double silu(double c) { return c / (1.0 + exp(-c)); }

/* Scan input u of sequence i, head h, channel p at token t.  With the fused
 * conv (Mamba-1 form only, head_dim 1): the causal depthwise conv over the
 * sequence x[i][.][h] preceded by the d_conv-1 conv-state values (zeros when
 * no conv state is given), then SiLU.  win holds those d_conv-1 values. */
/* Input tau of the conv of sequence i, head h: tau < 0 reads the conv state. */
static double conv_in(const job_t *J, int64_t i, int64_t tau, int64_t h, const double *win) {
    const oracle_dims *d = J->d;
    return tau < 0 ? win[tau + d->d_conv - 1] : J->x[(i * d->n_tokens + tau) * d->n_head + h];
}

/* The conv's output (SiLU's argument) at token t. */
static double conv_pre(const job_t *J, int64_t i, int64_t t, int64_t h, const double *win) {
    const int64_t K = J->d->d_conv;
    double c = 0.0;
    for (int64_t j = 0; j < K; j++) {
        int64_t tau = t - (K - 1) + j; /* tap j reads input tau; tap K-1 the newest */
        c += J->conv_w[h * K + j] * conv_in(J, i, tau, h, win);
    }
    return c;
}

static double scan_input(const job_t *J, int64_t i, int64_t t, int64_t h, int64_t p,
                         const double *win) {
    const oracle_dims *d = J->d;
    const int64_t L = d->n_tokens, H = d->n_head, P = d->head_dim;
    if (!d->d_conv) return J->x[((i * L + t) * H + h) * P + p];
    return silu(conv_pre(J, i, t, h, win));
}

static double dt_at(const job_t *J, int64_t i, int64_t t, int64_t h) {
    const oracle_dims *d = J->d;
    double v = J->dt[(i * d->n_tokens + t) * d->n_head + h];
    return d->dt_softplus ? softplus(v) : v;
}

static double A_at(const job_t *J, int64_t h, int64_t n) {
    return J->d->a_per_state ? J->A[h * J->d->d_state + n] : J->A[h];
}

static void load_window(const job_t *J, int64_t r, int64_t h, double *win) {
    const int64_t K = J->d->d_conv;
    for (int64_t j = 0; j + 1 < K; j++)
        win[j] = J->conv_state ? J->conv_state[(r * J->d->n_head + h) * (K - 1) + j] : 0.0;
}

/* Forward of one head for every sequence and channel of that head. */
static void forward_head(const job_t *J, int64_t h, double *st, double *win) {
    const oracle_dims *d = J->d;
    const int64_t L = d->n_tokens, H = d->n_head, P = d->head_dim, N = d->d_state,
                  G = d->n_group, K = d->d_conv;
    const int64_t g = J->grp_of_head[h];
    for (int64_t i = 0; i < d->n_seqs; i++) {
        const int64_t r = J->ids[i];
        for (int64_t p = 0; p < P; p++) {
            for (int64_t n = 0; n < N; n++) st[n] = J->s[((r * H + h) * P + p) * N + n];
            if (K) load_window(J, r, h, win);
            for (int64_t t = 0; t < L; t++) {
                const double u = scan_input(J, i, t, h, p, win);
                const double dtv = dt_at(J, i, t, h);
                const double *Bt = J->B + ((i * L + t) * G + g) * N;
                const double *Ct = J->C + ((i * L + t) * G + g) * N;
                double yv = 0.0;
                for (int64_t n = 0; n < N; n++) {
                    const double decay = exp(dtv * A_at(J, h, n));
                    st[n] = decay * st[n] + dtv * Bt[n] * u;
                    yv += Ct[n] * st[n];
                }
                if (d->has_D) yv += J->D[h] * u;
                J->y[((i * L + t) * H + h) * P + p] = yv;
            }
            for (int64_t n = 0; n < N; n++) J->state_out[((i * H + h) * P + p) * N + n] = st[n];
            if (K && J->conv_state_out) {
                /* the last K-1 inputs of the sequence, oldest first */
                for (int64_t j = 0; j + 1 < K; j++) {
                    int64_t tau = L - (K - 1) + j;
                    J->conv_state_out[(i * H + h) * (K - 1) + j] =
                        tau < 0 ? win[tau + K - 1] : J->x[(i * L + tau) * H + h];
                }
            }
        }
    }
}

/* Backward of one head: recompute the states h_{-1..L-1} of each row, then
 * run the adjoint recurrence from the last token to the first. */
static void backward_head(const job_t *J, int64_t h, double *hs, double *g, double *du_t,
                          double *win) {
    const oracle_dims *d = J->d;
    const int64_t L = d->n_tokens, H = d->n_head, P = d->head_dim, N = d->d_state,
                  G = d->n_group, K = d->d_conv;
    const int64_t grp = J->grp_of_head[h];
    double *dB = J->dB_part + (int64_t)J->tid * d->n_seqs * L * G * N;
    double *dC = J->dC_part + (int64_t)J->tid * d->n_seqs * L * G * N;
    double dD_h = 0.0;
    for (int64_t i = 0; i < d->n_seqs; i++) {
        const int64_t r = J->ids[i];
        for (int64_t p = 0; p < P; p++) {
            /* hs[(t+1)*N + n] = h_t[n]; hs[0..N) = initial state */
            for (int64_t n = 0; n < N; n++) hs[n] = J->s[((r * H + h) * P + p) * N + n];
            if (K) load_window(J, r, h, win);
            for (int64_t t = 0; t < L; t++) {
                const double u = scan_input(J, i, t, h, p, win);
                const double dtv = dt_at(J, i, t, h);
                const double *Bt = J->B + ((i * L + t) * G + grp) * N;
                for (int64_t n = 0; n < N; n++)
                    hs[(t + 1) * N + n] =
                        exp(dtv * A_at(J, h, n)) * hs[t * N + n] + dtv * Bt[n] * u;
            }
            /* g = dL/dh_t, seeded with the upstream gradient of the final state */
            for (int64_t n = 0; n < N; n++) g[n] = J->dstate[((i * H + h) * P + p) * N + n];
            for (int64_t t = L - 1; t >= 0; t--) {
                const double u = scan_input(J, i, t, h, p, win);
                const double dtv = dt_at(J, i, t, h);
                const double dyt = J->dy[((i * L + t) * H + h) * P + p];
                const double *Bt = J->B + ((i * L + t) * G + grp) * N;
                const double *Ct = J->C + ((i * L + t) * G + grp) * N;
                double *dBt = dB + ((i * L + t) * G + grp) * N;
                double *dCt = dC + ((i * L + t) * G + grp) * N;
                double du = d->has_D ? J->D[h] * dyt : 0.0;
                double ddt = 0.0;
                if (d->has_D) dD_h += dyt * u;
                for (int64_t n = 0; n < N; n++) {
                    const double An = A_at(J, h, n);
                    const double decay = exp(dtv * An);
                    const double h_prev = hs[t * N + n];
                    const double h_cur = hs[(t + 1) * N + n];
                    g[n] += Ct[n] * dyt;          /* y_t = C_t . h_t + ... */
                    dCt[n] += dyt * h_cur;
                    du += g[n] * dtv * Bt[n];     /* h_t = decay h_{t-1} + dt B_t u_t */
                    dBt[n] += g[n] * dtv * u;
                    ddt += g[n] * (h_prev * decay * An + Bt[n] * u);
                    const double dAn = g[n] * h_prev * decay * dtv;
                    if (d->a_per_state) J->d_A[h * N + n] += dAn; else J->d_A[h] += dAn;
                    g[n] *= decay;                /* now dL/dh_{t-1} */
                }
                if (d->dt_softplus) ddt *= sigmoid(J->dt[(i * L + t) * H + h]);
                J->d_dt[(i * L + t) * H + h] += ddt;
                if (K) du_t[t] = du;  /* dL/du_t; the conv adjoint follows */
                else J->d_x[((i * L + t) * H + h) * P + p] = du;
            }
            for (int64_t n = 0; n < N; n++) J->d_s[((r * H + h) * P + p) * N + n] += g[n];
            if (K) {
                /* u_t = SiLU(c_t): dL/dc_t = dL/du_t sigma(c_t) (1 + c_t (1 - sigma(c_t))) */
                for (int64_t t = 0; t < L; t++) {
                    const double c = conv_pre(J, i, t, h, win);
                    const double sg = sigmoid(c);
                    du_t[t] *= sg * (1.0 + c * (1.0 - sg));
                }
                /* c_t = sum_j w[j] in(t - (K-1) + j): input tau feeds tokens tau + K-1 - j */
                for (int64_t tau = -(K - 1); tau < L; tau++) {
                    double gin = 0.0;
                    for (int64_t j = 0; j < K; j++) {
                        const int64_t t = tau + (K - 1) - j;
                        if (t >= 0 && t < L) gin += J->conv_w[h * K + j] * du_t[t];
                    }
                    if (tau >= 0) J->d_x[(i * L + tau) * H + h] = gin;
                    else J->d_conv_state[(r * H + h) * (K - 1) + tau + K - 1] += gin;
                }
                for (int64_t j = 0; j < K; j++) {
                    double gw = 0.0;
                    for (int64_t t = 0; t < L; t++)
                        gw += du_t[t] * conv_in(J, i, t - (K - 1) + j, h, win);
                    J->d_conv_w[h * K + j] += gw;
                }
            }
        }
    }
    if (d->has_D) J->d_D[h] += dD_h;
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    const oracle_dims *d = J->d;
    const int64_t N = d->d_state, L = d->n_tokens;
    double *buf = NULL, *buf2 = NULL, *buf3 = NULL;
    double *win = (double *)malloc(sizeof(double) * (size_t)(d->d_conv > 1 ? d->d_conv : 1));
    if (J->backward) {
        buf = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
        buf2 = (double *)malloc(sizeof(double) * (size_t)N);
        buf3 = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    } else {
        buf = (double *)malloc(sizeof(double) * (size_t)N);
        buf2 = buf3 = (double *)malloc(sizeof(double));
    }
    if (!buf || !buf2 || !buf3 || !win) {
        free(buf); free(buf2); if (J->backward) free(buf3); free(win);
        return (void *)1;
    }
    /* static partition of heads: thread tid takes heads tid, tid+T, ... */
    for (int64_t h = J->tid; h < d->n_head; h += J->n_threads) {
        if (J->backward) backward_head(J, h, buf, buf2, buf3, win);
        else forward_head(J, h, buf, win);
    }
    free(buf);
    free(buf2);
    if (J->backward) free(buf3);
    free(win);
    return NULL;
}

static int check_dims(const oracle_dims *d, const int64_t *grp, const int32_t *ids) {
    if (!d || !grp || !ids) return -1;
    if (d->n_seqs < 0 || d->n_tokens < 0 || d->n_head < 1 || d->head_dim < 1 ||
        d->d_state < 1 || d->n_group < 1 || d->n_state_rows < 1 || d->d_conv < 0)
        return -2;
    if (d->d_conv && d->head_dim != 1) return -3;
    for (int64_t h = 0; h < d->n_head; h++)
        if (grp[h] < 0 || grp[h] >= d->n_group) return -4;
    for (int64_t i = 0; i < d->n_seqs; i++)
        if (ids[i] < 0 || ids[i] >= d->n_state_rows) return -5;
    return 0;
}

static int run_jobs(job_t *proto, int n_threads) {
    if (n_threads < 1) n_threads = 1;
    if (n_threads > proto->d->n_head) n_threads = (int)proto->d->n_head;
    job_t *jobs = (job_t *)calloc((size_t)n_threads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -10; }
    int rc = 0;
    for (int k = 0; k < n_threads; k++) {
        jobs[k] = *proto;
        jobs[k].tid = k;
        jobs[k].n_threads = n_threads;
    }
    for (int k = 1; k < n_threads; k++)
        if (pthread_create(&th[k], NULL, worker, &jobs[k])) { rc = -11; n_threads = k; break; }
    if (worker(&jobs[0])) rc = -12;
    for (int k = 1; k < n_threads; k++) {
        void *ret = NULL;
        pthread_join(th[k], &ret);
        if (ret) rc = -12;
    }
    free(jobs);
    free(th);
    return rc;
}

int oracle_threads_used(const oracle_dims *d, int n_threads) {
    if (n_threads < 1) n_threads = 1;
    return n_threads > d->n_head ? (int)d->n_head : n_threads;
}

/* Forward: y [n_seqs][L][H][P], state_out [n_seqs][H][P][N],
 * conv_state_out [n_seqs][H][d_conv-1] (may be NULL). */
int oracle_scan_fwd(const oracle_dims *d, const int64_t *grp_of_head, const double *s,
                    const double *x, const double *dt, const double *A, const double *B,
                    const double *C, const double *D, const int32_t *ids,
                    const double *conv_w, const double *conv_state, double *y,
                    double *state_out, double *conv_state_out, int n_threads) {
    int rc = check_dims(d, grp_of_head, ids);
    if (rc) return rc;
    if (!s || !x || !dt || !A || !B || !C || !y || !state_out) return -1;
    if (d->has_D && !D) return -1;
    if (d->d_conv && !conv_w) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.d = d; J.grp_of_head = grp_of_head; J.s = s; J.x = x; J.dt = dt; J.A = A;
    J.B = B; J.C = C; J.D = D; J.ids = ids; J.conv_w = conv_w; J.conv_state = conv_state;
    J.y = y; J.state_out = state_out; J.conv_state_out = conv_state_out;
    return run_jobs(&J, n_threads);
}

/* Backward.  Outputs are overwritten: d_s [n_state_rows][H][P][N] (rows not
 * referenced by ids are zero, repeated ids accumulate), d_x like x (with the
 * fused conv: the gradient of the pre-conv input x), d_dt like dt, d_A like
 * A, d_B/d_C like B/C, d_D [H] (only when has_D); with the fused conv also
 * d_conv_w [H][K] and d_conv_state [n_state_rows][H][K-1] (the gradient of
 * the gathered conv-state inputs, scattered to rows ids[i]; conv_state may
 * be NULL for zeros). */
int oracle_scan_bwd(const oracle_dims *d, const int64_t *grp_of_head, const double *s,
                    const double *x, const double *dt, const double *A, const double *B,
                    const double *C, const double *D, const int32_t *ids,
                    const double *conv_w, const double *conv_state,
                    const double *dy, const double *dstate, double *d_s, double *d_x,
                    double *d_dt, double *d_A, double *d_B, double *d_C, double *d_D,
                    double *d_conv_w, double *d_conv_state, int n_threads) {
    int rc = check_dims(d, grp_of_head, ids);
    if (rc) return rc;
    if (!s || !x || !dt || !A || !B || !C || !dy || !dstate || !d_s || !d_x || !d_dt ||
        !d_A || !d_B || !d_C)
        return -1;
    if (d->has_D && (!D || !d_D)) return -1;
    if (d->d_conv && (!conv_w || !d_conv_w || !d_conv_state)) return -1;
    const int64_t H = d->n_head, P = d->head_dim, N = d->d_state, L = d->n_tokens,
                  G = d->n_group, S = d->n_seqs;
    memset(d_s, 0, sizeof(double) * (size_t)(d->n_state_rows * H * P * N));
    memset(d_x, 0, sizeof(double) * (size_t)(S * L * H * P));
    memset(d_dt, 0, sizeof(double) * (size_t)(S * L * H));
    memset(d_A, 0, sizeof(double) * (size_t)(d->a_per_state ? H * N : H));
    if (d->has_D) memset(d_D, 0, sizeof(double) * (size_t)H);
    if (d->d_conv) {
        memset(d_conv_w, 0, sizeof(double) * (size_t)(H * d->d_conv));
        memset(d_conv_state, 0, sizeof(double) * (size_t)(d->n_state_rows * H * (d->d_conv - 1)));
    }
    int T = oracle_threads_used(d, n_threads);
    const size_t part = (size_t)(S * L * G * N);
    double *dBp = (double *)calloc(part * (size_t)T, sizeof(double));
    double *dCp = (double *)calloc(part * (size_t)T, sizeof(double));
    if (!dBp || !dCp) { free(dBp); free(dCp); return -10; }
    job_t J;
    memset(&J, 0, sizeof J);
    J.d = d; J.grp_of_head = grp_of_head; J.s = s; J.x = x; J.dt = dt; J.A = A;
    J.B = B; J.C = C; J.D = D; J.ids = ids; J.dy = dy; J.dstate = dstate;
    J.conv_w = conv_w; J.conv_state = conv_state;
    J.d_s = d_s; J.d_x = d_x; J.d_dt = d_dt; J.d_A = d_A; J.d_D = d_D;
    J.d_conv_w = d_conv_w; J.d_conv_state = d_conv_state;
    J.dB_part = dBp; J.dC_part = dCp; J.backward = 1;
    rc = run_jobs(&J, T);
    /* fixed-order reduction of the per-thread partial sums */
    for (size_t e = 0; e < part; e++) {
        double b = 0.0, c = 0.0;
        for (int k = 0; k < T; k++) { b += dBp[(size_t)k * part + e]; c += dCp[(size_t)k * part + e]; }
        d_B[e] = b;
        d_C[e] = c;
    }
    free(dBp);
    free(dCp);
    return rc;
}

/* ggml-style standalone depthwise conv: sx [n_s][d_inner][d_conv-1+n_t]
 * (time fastest, carrying d_conv-1 earlier inputs), w [d_inner][d_conv],
 * out [n_s][n_t][d_inner]; out = sum_j sx[t+j] * w[j], then SiLU if asked. */
int oracle_conv_fwd(const double *sx, const double *w, double *out, int64_t n_s,
                    int64_t n_t, int64_t d_inner, int32_t d_conv, int32_t apply_silu) {
    if (!sx || !w || !out || n_s < 0 || n_t < 0 || d_inner < 1 || d_conv < 1) return -1;
    const int64_t len = d_conv - 1 + n_t;
    for (int64_t s = 0; s < n_s; s++)
        for (int64_t t = 0; t < n_t; t++)
            for (int64_t ch = 0; ch < d_inner; ch++) {
                double acc = 0.0;
                for (int64_t j = 0; j < d_conv; j++)
                    acc += sx[(s * d_inner + ch) * len + t + j] * w[ch * d_conv + j];
                out[(s * n_t + t) * d_inner + ch] = apply_silu ? silu(acc) : acc;
            }
    return 0;
}

/* Backward of oracle_conv_fwd, the ggmlR extension's ssm_conv backward
 * ("ggmlR tests/testthat/test-ssm-rwkv.R", the ssm_conv backward block:
 * ggml_ssm_conv_back packs the gradient of sx followed by that of the
 * weights).  With z_t = sum_j sx[t+j] w[j], out_t = z_t (or SiLU(z_t)) and
 * the upstream gradient dout [n_s][n_t][d_inner]:
 *   g_t   = dout_t, or dout_t * s(z_t) (1 + z_t (1 - s(z_t))) with the SiLU
 *           (the derivative of z s(z), s the logistic function);
 *   d_sx[tau] = sum over the (t, j) with t + j = tau of g_t w[j];
 *   d_w[j]    = sum over sequences and t of g_t sx[t+j].
 * d_sx has the layout of sx, d_w that of w. */
int oracle_conv_bwd(const double *sx, const double *w, const double *dout, double *d_sx,
                    double *d_w, int64_t n_s, int64_t n_t, int64_t d_inner, int32_t d_conv,
                    int32_t apply_silu) {
    if (!sx || !w || !dout || !d_sx || !d_w || n_s < 0 || n_t < 0 || d_inner < 1 || d_conv < 1)
        return -1;
    const int64_t len = d_conv - 1 + n_t;
    memset(d_sx, 0, (size_t)(n_s * d_inner * len) * sizeof(double));
    memset(d_w, 0, (size_t)(d_inner * d_conv) * sizeof(double));
    for (int64_t s = 0; s < n_s; s++)
        for (int64_t t = 0; t < n_t; t++)
            for (int64_t ch = 0; ch < d_inner; ch++) {
                const double *row = sx + (s * d_inner + ch) * len;
                double g = dout[(s * n_t + t) * d_inner + ch];
                if (apply_silu) {
                    double z = 0.0;
                    for (int64_t j = 0; j < d_conv; j++) z += row[t + j] * w[ch * d_conv + j];
                    const double sg = sigmoid(z);
                    g *= sg * (1.0 + z * (1.0 - sg));
                }
                for (int64_t j = 0; j < d_conv; j++) {
                    d_sx[(s * d_inner + ch) * len + t + j] += g * w[ch * d_conv + j];
                    d_w[ch * d_conv + j] += g * row[t + j];
                }
            }
    return 0;
}

/* sum_j w[j] win[j] over the window of the K-1 previous inputs (oldest first)
 * followed by the new one. */
static double w_tap_sum(const double *w, const double *prev, double xin, int64_t K) {
    double c = 0.0;
    for (int64_t j = 0; j < K - 1; j++) c += w[j] * prev[j];
    return c + w[K - 1] * xin;
}

/* One token of every sequence of a batch, updating states in place
 * ("mambazip mamba1/model.rs", forward_impl's single-token step; the conv
 * taps in ggml's order, the last weight on the newest input).  For sequence
 * i, row r = ids[i], head h, channel p:
 *   with d_conv = K > 0 (head_dim 1): win = conv_state[r][h][0..K-2] then
 *     x[i][h]; c = sum_j w[h][j] win[j]; u = SiLU(c); conv_state[r][h] keeps
 *     the last K-1 entries of win;  otherwise u = x[i][h][p];
 *   d = dt[i][h] (+ dt_bias[h] when given), then softplus when asked;
 *   s[r][h][p][n] = exp(d A) s[r][h][p][n] + d B[i][g][n] u   for every n;
 *   y[i][h][p] = sum_n C[i][g][n] s[r][h][p][n] + D[h] u, times SiLU(z[i][h][p])
 *     when z is given.
 * Rows are updated in sequence order, so ids should be distinct (a repeated
 * row would be stepped twice).  n_tokens in d is ignored (one token). */
int oracle_state_update(const oracle_dims *d, const int64_t *grp_of_head, double *s,
                        const double *x, const double *dt, const double *dt_bias,
                        const double *A, const double *B, const double *C, const double *D,
                        const double *z, const int32_t *ids, const double *conv_w,
                        double *conv_state, double *y) {
    int rc = check_dims(d, grp_of_head, ids);
    if (rc) return rc;
    if (!s || !x || !dt || !A || !B || !C || !y) return -1;
    if (d->has_D && !D) return -1;
    if (d->d_conv && (!conv_w || !conv_state)) return -1;
    const int64_t H = d->n_head, P = d->head_dim, N = d->d_state, G = d->n_group, K = d->d_conv;
    for (int64_t i = 0; i < d->n_seqs; i++) {
        const int64_t r = ids[i];
        for (int64_t h = 0; h < H; h++) {
            const int64_t g = grp_of_head[h];
            double dd = dt[i * H + h] + (dt_bias ? dt_bias[h] : 0.0);
            if (d->dt_softplus) dd = softplus(dd);
            for (int64_t p = 0; p < P; p++) {
                double u;
                if (K) {
                    double *cs = conv_state + (r * H + h) * (K - 1);
                    const double xin = x[i * H + h];
                    double c = w_tap_sum(conv_w + h * K, cs, xin, K);
                    for (int64_t j = 0; j + 1 < K - 1; j++) cs[j] = cs[j + 1];
                    if (K > 1) cs[K - 2] = xin;
                    u = silu(c);
                } else {
                    u = x[(i * H + h) * P + p];
                }
                double *st = s + ((r * H + h) * P + p) * N;
                double acc = 0.0;
                for (int64_t n = 0; n < N; n++) {
                    const double a = exp(dd * (d->a_per_state ? A[h * N + n] : A[h]));
                    st[n] = a * st[n] + dd * B[(i * G + g) * N + n] * u;
                    acc += C[(i * G + g) * N + n] * st[n];
                }
                if (d->has_D) acc += D[h] * u;
                if (z) acc *= silu(z[(i * H + h) * P + p]);
                y[(i * H + h) * P + p] = acc;
            }
        }
    }
    return 0;
}
