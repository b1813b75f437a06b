/*
 * kda_oracle.c -- fp64 reference for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE. This file is the correctness oracle for the HIP path.
 * It is compiled with the host C compiler only, shares no code, header,
 * table or helper with the HIP library, and is called only from tests/,
 * the smoke check and the CPU-baseline leg of bench.py. The product path
 * never links or calls it.
 *
 * What it computes (the method's plain definition, one token at a time):
 *
 *   The Kimi K3 explainer (SemiAnalysis, Chinese translation), DeltaNet
 *   section: the delta rule S_t = S_{t-1} - beta_t (S_{t-1} k_t - v_t) k_t^T,
 *   obtained as one SGD step on 0.5 ||S k_t - v_t||^2.
 *   Same page, GDN/KDA paragraph: GDN multiplies S by a forget gate alpha
 *   before the delta step; KDA turns alpha into a diagonal matrix, i.e. one
 *   decay per key channel.
 *   Same page, FlashKDA paragraph ("another form of the recurrence"): D_t is
 *   the diagonal of alpha_t, u_t is the delta; decode follows this form.
 *
 * Storage convention: the state of one (sequence, head) chain is held as
 * M = S^T with shape [Dk][Dv] (row = key channel, Dv contiguous). Then, per
 * token t, with alpha_t = exp(g_t) (g is the natural-log decay, one value per
 * key channel):
 *
 *     M'  = Diag(alpha_t) M_{t-1}          decay every key row
 *     p   = M'^T k_t                       what the decayed memory returns
 *     u_t = beta_t (v_t - p)               the delta
 *     M_t = M' + k_t u_t^T                 rank-1 write
 *     o_t = M_t^T q_t                      read-out (sees token t's write)
 *
 * In S orientation this is S_t = S_{t-1}D_t - beta_t (S_{t-1}D_t k_t - v_t)k_t^T
 * and o_t = S_t q_t. No 1/sqrt(d) scaling, no normalisation of q or k.
 *
 * Parity status: pinned (see tests/test_oracle_pins.py): DeltaNet and GDN
 * special cases, zero-beta, zero-alpha, exact retrieval, linear-attention
 * closed form, a hand-worked fixture, and agreement with the separately
 * written chunked form in chunked_naive.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *S0;
    double *out, *S_out;
    const int64_t *cu;       /* [N+1] token offsets of each sequence */
    int N, H, Dk, Dv;
    int next;                /* next chain index to hand out */
    pthread_mutex_t lock;
} oracle_job;

/* One (sequence n, head h) chain, token by token. */
static void run_chain(const oracle_job *J, int n, int h, double *M, double *u)
{
    const int H = J->H, Dk = J->Dk, Dv = J->Dv;
    const size_t state_off = ((size_t)n * H + h) * (size_t)Dk * Dv;

    if (J->S0)
        memcpy(M, J->S0 + state_off, sizeof(double) * (size_t)Dk * Dv);
    else
        memset(M, 0, sizeof(double) * (size_t)Dk * Dv);

    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const size_t row = (size_t)t * H + h;
        const double *qt = J->q + row * Dk;
        const double *kt = J->k + row * Dk;
        const double *vt = J->v + row * Dv;
        const double *gt = J->g + row * Dk;
        const double bt = J->beta[row];

        /* M' = Diag(exp(g_t)) M */
        for (int c = 0; c < Dk; ++c) {
            const double a = exp(gt[c]);
            double *Mr = M + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) Mr[j] *= a;
        }
        /* u = beta (v - M'^T k) */
        for (int j = 0; j < Dv; ++j) u[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double kc = kt[c];
            const double *Mr = M + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) u[j] += Mr[j] * kc;
        }
        for (int j = 0; j < Dv; ++j) u[j] = bt * (vt[j] - u[j]);
        /* M = M' + k u^T */
        for (int c = 0; c < Dk; ++c) {
            const double kc = kt[c];
            double *Mr = M + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) Mr[j] += kc * u[j];
        }
        /* o = M^T q */
        double *ot = J->out + row * Dv;
        for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double qc = qt[c];
            const double *Mr = M + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) ot[j] += Mr[j] * qc;
        }
    }
    if (J->S_out)
        memcpy(J->S_out + state_off, M, sizeof(double) * (size_t)Dk * Dv);
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    double *M = (double *)malloc(sizeof(double) * (size_t)J->Dk * J->Dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)J->Dv);
    if (!M || !u) { free(M); free(u); return (void *)1; }
    const int chains = J->N * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int idx = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (idx >= chains) break;
        run_chain(J, idx / J->H, idx % J->H, M, u);
    }
    free(M);
    free(u);
    return NULL;
}

/*
 * kda_oracle_run: the whole recurrence for N packed sequences.
 *
 *   q, k, g : [T_total][H][Dk]   (T_total = cu_seqlens[N])
 *   v, out  : [T_total][H][Dv]
 *   beta    : [T_total][H]
 *   S0      : [N][H][Dk][Dv] or NULL (zero initial state)
 *   S_out   : [N][H][Dk][Dv] or NULL (final state not returned)
 *   cu_seqlens : int64 [N+1], non-decreasing, cu_seqlens[0] == 0
 *   nthreads: worker threads over the N*H independent chains (>= 1)
 *
 * Returns 0 on success, -1 on bad arguments, -2 if a thread failed.
 */
int kda_oracle_run(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *S0,
                   double *out, double *S_out, const int64_t *cu_seqlens,
                   int N, int H, int Dk, int Dv, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !out || !cu_seqlens) return -1;
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    if (cu_seqlens[0] != 0) return -1;
    for (int n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > N * H) nthreads = N * H > 0 ? N * H : 1;

    oracle_job J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0;
    J.out = out; J.S_out = S_out; J.cu = cu_seqlens;
    J.N = N; J.H = H; J.Dk = Dk; J.Dv = Dv; J.next = 0;
    pthread_mutex_init(&J.lock, NULL);

    int rc = 0;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) { pthread_mutex_destroy(&J.lock); return -2; }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) { rc = -2; break; }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret) rc = -2;
    }
    if (started == 0) {           /* no thread could start: run inline */
        rc = worker(&J) ? -2 : 0;
    }
    free(th);
    pthread_mutex_destroy(&J.lock);
    return rc;
}
