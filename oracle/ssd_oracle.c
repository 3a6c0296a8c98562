/*
 * ssd_oracle.c -- plain fp64 CPU oracle of the selective state space layer core.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg
 * do. It shares no code, header or table with the GPU library.
 *
 * What it computes is the *definition* of the layer, token by token, with no
 * chunking, blocking or re-association:
 *
 *   for every batch row b and head h (group g = h / (H/G)):
 *     S <- init_state[b,h]            (N x P, zeros when absent)
 *     for t = 0 .. T-1:
 *       abar    = exp(dt[b,t,h] * A[h])                      (1)
 *       S[n,p]  = abar * S[n,p] + (dt[b,t,h] * B[b,t,g,n]) * x[b,t,h,p]   (2)
 *       y[b,t,h,p] = sum_n C[b,t,g,n] * S[n,p] + D[h] * x[b,t,h,p]        (3)
 *     final_state[b,h] <- S
 *
 * (1),(2),(3): discretisation abar_t = exp(dt_t A), bbar_t = dt_t B_t, state
 * update h_t = abar_t h_{t-1} + bbar_t x_t and read-out y_t = C_t h_t, on the
 * youngju.dev "Mamba / selective SSM" page, section "LTIからSelectionへの切り替え"
 * (the selective SSM equations); A is one negative scalar per head and heads
 * share B, C inside a group (Qiita "Mamba-2" article, sections 4.1-4.2); the D
 * skip term is the "skip connection" of the selective-scan code on the same
 * youngju.dev page (applied per head here, as the head-scalar layer defines
 * it). The recurrent form is the inference mode of the waylandz LLM book,
 * chapter 32, section 32.2.4.
 *
 * Inputs arrive as float32 arrays that hold the exact stored values (bf16
 * values are exactly representable in float32); every operation is done in
 * double. init/state inputs are double so that a final state can be fed back
 * without rounding. Decode (the recurrent single-token mode) is the same loop
 * body applied to a given state; a run of decode steps is the same loop with
 * the step axis outermost in memory.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Token-major strided view of one problem. All strides are in elements. */
typedef struct {
    const float *x, *dt, *A, *B, *C, *D; /* D may be NULL (= 0) */
    const double *init;                  /* [b,H,N,P] or NULL (= 0) */
    long T;
    int H, P, N, G;
    /* element offset of (b, t) for each tensor: off = b*s_b + t*s_t */
    long x_sb, x_st, dt_sb, dt_st, bc_sb, bc_st;
} problem;

/* One unit of work: columns [p0, p1) of head h of batch row b. */
typedef struct {
    int b, h, p0, p1;
    double *y;       /* y of column p0 at token 0, or NULL */
    long y_st;       /* element stride of y between consecutive tokens */
    long y_sp;       /* element stride of y between consecutive columns */
    double *fin;     /* final S[0][p0], or NULL */
    long fin_sn;     /* element stride of fin between consecutive n */
    long fin_sp;     /* element stride of fin between consecutive columns */
} task;

typedef struct {
    const problem *pb;
    const task *tasks;
    long ntasks;
    long next; /* atomically incremented */
    int pmax;
} pool;

static void run_task(const problem *pb, const task *tk, double *S /* N * (p1-p0) */)
{
    const int N = pb->N, H = pb->H, P = pb->P;
    const int w = tk->p1 - tk->p0;
    const int g = tk->h / (H / pb->G);
    const double Ah = (double)pb->A[tk->h];
    const double Dh = pb->D ? (double)pb->D[tk->h] : 0.0;

    for (int n = 0; n < N; ++n)
        for (int j = 0; j < w; ++j)
            S[n * w + j] = pb->init
                ? pb->init[(((long)tk->b * H + tk->h) * N + n) * P + tk->p0 + j]
                : 0.0;

    for (long t = 0; t < pb->T; ++t) {
        const float *xr = pb->x + tk->b * pb->x_sb + t * pb->x_st + (long)tk->h * P + tk->p0;
        const double dtv = (double)pb->dt[tk->b * pb->dt_sb + t * pb->dt_st + tk->h];
        const float *Br = pb->B + tk->b * pb->bc_sb + t * pb->bc_st + (long)g * N;
        const float *Cr = pb->C + tk->b * pb->bc_sb + t * pb->bc_st + (long)g * N;
        const double abar = exp(dtv * Ah);                          /* (1) */
        for (int n = 0; n < N; ++n) {
            const double bbar = dtv * (double)Br[n];                /* (2) */
            double *Sn = S + n * w;
            for (int j = 0; j < w; ++j)
                Sn[j] = abar * Sn[j] + bbar * (double)xr[j];
        }
        if (tk->y) {
            double *yt = tk->y + t * tk->y_st;
            for (int j = 0; j < w; ++j) {                           /* (3) */
                double acc = 0.0;
                for (int n = 0; n < N; ++n)
                    acc += (double)Cr[n] * S[n * w + j];
                yt[j * tk->y_sp] = acc + Dh * (double)xr[j];
            }
        }
    }
    if (tk->fin)
        for (int n = 0; n < N; ++n)
            for (int j = 0; j < w; ++j)
                tk->fin[n * tk->fin_sn + j * tk->fin_sp] = S[n * w + j];
}

static void *worker(void *arg)
{
    pool *pl = (pool *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)pl->pb->N * (size_t)pl->pmax);
    if (!S)
        return (void *)1;
    for (;;) {
        long i = __atomic_fetch_add(&pl->next, 1, __ATOMIC_RELAXED);
        if (i >= pl->ntasks)
            break;
        run_task(pl->pb, &pl->tasks[i], S);
    }
    free(S);
    return NULL;
}

static int run_pool(const problem *pb, const task *tasks, long ntasks, int pmax, int nthreads)
{
    pool pl = {pb, tasks, ntasks, 0, pmax};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > ntasks)
        nthreads = (int)(ntasks > 0 ? ntasks : 1);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th)
        return 1;
    int err = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &pl) != 0) {
            err = 1;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            err = 1;
    }
    free(th);
    return err;
}

static int check_dims(long batch, long T, int H, int P, int N, int G)
{
    if (batch < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G)
        return 2;
    return 0;
}

#define PBLK 8

/*
 * Full forward: y [b,T,H,P] and final [b,H,N,P] (either may be NULL).
 * Returns 0 on success.
 */
int oracle_ssd_fwd(const float *x, const float *dt, const float *A, const float *B,
                   const float *C, const float *D, const double *init,
                   double *y, double *final_state,
                   int batch, long T, int H, int P, int N, int G, int nthreads)
{
    if (check_dims(batch, T, H, P, N, G))
        return 2;
    problem pb = {x, dt, A, B, C, D, init, T, H, P, N, G,
                  T * H * P, (long)H * P, T * H, H, T * G * N, (long)G * N};
    long nblk = (P + PBLK - 1) / PBLK;
    long nt = (long)batch * H * nblk;
    task *tasks = (task *)calloc((size_t)nt, sizeof(task));
    if (!tasks)
        return 1;
    long i = 0;
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < H; ++h)
            for (int p0 = 0; p0 < P; p0 += PBLK, ++i) {
                task *tk = &tasks[i];
                tk->b = b; tk->h = h; tk->p0 = p0;
                tk->p1 = p0 + PBLK < P ? p0 + PBLK : P;
                tk->y = y ? y + (((long)b * T) * H + h) * P + p0 : NULL;
                tk->y_st = (long)H * P; tk->y_sp = 1;
                tk->fin = final_state ? final_state + (((long)b * H + h) * N) * P + p0 : NULL;
                tk->fin_sn = P; tk->fin_sp = 1;
            }
    int r = run_pool(&pb, tasks, nt, PBLK, nthreads);
    free(tasks);
    return r;
}

/*
 * Forward restricted to selected columns (b_i, h_i, p_i): y_cols [ncols][T],
 * final_cols [ncols][N] (either may be NULL). Each column evolves on its own
 * (the state's column p only ever meets x[...,p]), so this is exact.
 */
int oracle_ssd_fwd_columns(const float *x, const float *dt, const float *A, const float *B,
                           const float *C, const float *D, const double *init,
                           int ncols, const int *col_b, const int *col_h, const int *col_p,
                           double *y_cols, double *final_cols,
                           int batch, long T, int H, int P, int N, int G, int nthreads)
{
    if (check_dims(batch, T, H, P, N, G) || ncols < 1)
        return 2;
    problem pb = {x, dt, A, B, C, D, init, T, H, P, N, G,
                  T * H * P, (long)H * P, T * H, H, T * G * N, (long)G * N};
    task *tasks = (task *)calloc((size_t)ncols, sizeof(task));
    if (!tasks)
        return 1;
    for (int i = 0; i < ncols; ++i) {
        if (col_b[i] < 0 || col_b[i] >= batch || col_h[i] < 0 || col_h[i] >= H ||
            col_p[i] < 0 || col_p[i] >= P) {
            free(tasks);
            return 2;
        }
        task *tk = &tasks[i];
        tk->b = col_b[i]; tk->h = col_h[i]; tk->p0 = col_p[i]; tk->p1 = col_p[i] + 1;
        tk->y = y_cols ? y_cols + (long)i * T : NULL;
        tk->y_st = 1; tk->y_sp = 0;
        tk->fin = final_cols ? final_cols + (long)i * N : NULL;
        tk->fin_sn = 1; tk->fin_sp = 0;
    }
    int r = run_pool(&pb, tasks, ncols, 1, nthreads);
    free(tasks);
    return r;
}

/*
 * `steps` chained decode updates (the recurrent mode, one token per step):
 * state0 [b,H,N,P]; per-step inputs stacked on a leading axis:
 * xs [S,b,H,P], dts [S,b,H], Bs/Cs [S,b,G,N]. Outputs ys [S,b,H,P] and the
 * state after the last step, state_out [b,H,N,P] (either may be NULL).
 * Heads may be restricted to the pairs (sel_b[i], sel_h[i]) when nsel > 0;
 * then ys is [nsel][S][P] and state_out [nsel][N][P].
 */
int oracle_ssd_decode(const double *state0, const float *xs, const float *dts,
                      const float *A, const float *Bs, const float *Cs, const float *D,
                      double *ys, double *state_out,
                      int batch, int steps, int H, int P, int N, int G,
                      int nsel, const int *sel_b, const int *sel_h, int nthreads)
{
    if (check_dims(batch, steps, H, P, N, G))
        return 2;
    problem pb = {xs, dts, A, Bs, Cs, D, state0, steps, H, P, N, G,
                  (long)H * P, (long)batch * H * P, H, (long)batch * H,
                  (long)G * N, (long)batch * G * N};
    long nblk = (P + PBLK - 1) / PBLK;
    long nheads = nsel > 0 ? nsel : (long)batch * H;
    long nt = nheads * nblk;
    task *tasks = (task *)calloc((size_t)nt, sizeof(task));
    if (!tasks)
        return 1;
    long i = 0;
    for (long k = 0; k < nheads; ++k) {
        int b = nsel > 0 ? sel_b[k] : (int)(k / H);
        int h = nsel > 0 ? sel_h[k] : (int)(k % H);
        if (b < 0 || b >= batch || h < 0 || h >= H) {
            free(tasks);
            return 2;
        }
        for (int p0 = 0; p0 < P; p0 += PBLK, ++i) {
            task *tk = &tasks[i];
            tk->b = b; tk->h = h; tk->p0 = p0;
            tk->p1 = p0 + PBLK < P ? p0 + PBLK : P;
            if (nsel > 0) {
                tk->y = ys ? ys + (k * steps) * P + p0 : NULL;
                tk->y_st = P;
                tk->fin = state_out ? state_out + k * N * P + p0 : NULL;
            } else {
                tk->y = ys ? ys + ((long)b * H + h) * P + p0 : NULL;
                tk->y_st = (long)batch * H * P;
                tk->fin = state_out ? state_out + (((long)b * H + h) * N) * P + p0 : NULL;
            }
            tk->y_sp = 1;
            tk->fin_sn = P; tk->fin_sp = 1;
        }
    }
    int r = run_pool(&pb, tasks, nt, PBLK, nthreads);
    free(tasks);
    return r;
}


/*
 * Packed variable-length sequences: sequence i is tokens cu[i] .. cu[i+1]-1
 * of one token axis (x [T,H,P], dt [T,H], B/C [T,G,N]). Each sequence starts
 * from its own state, init[i] (zeros when init is NULL), so nothing of one
 * sequence reaches the next (youngju.dev "Mamba / selective SSM" page,
 * section "状態初期化とシーケンス境界": the state is set explicitly at the start
 * of every sequence so that sequences in one batch do not mix). The
 * recurrence is the same as above; y [T,H,P], final [nseq,H,N,P] (either may
 * be NULL). A sequence with no tokens leaves its initial state as its final
 * state.
 */
typedef struct {
    const float *x, *dt, *A, *B, *C, *D;
    const double *init;
    const int *cu;
    int nseq;
    long T;
    int H, P, N, G;
    double *y, *fin;
    long ntasks, next;   /* tasks: (h, column block), handed out atomically */
} vproblem;

static void run_vtask(vproblem *pb, long task_id, double *S)
{
    const int H = pb->H, P = pb->P, N = pb->N;
    const long nblk = (P + PBLK - 1) / PBLK;
    const int h = (int)(task_id / nblk);
    const int p0 = (int)(task_id % nblk) * PBLK;
    const int p1 = p0 + PBLK < P ? p0 + PBLK : P;
    const int w = p1 - p0;
    const int g = h / (H / pb->G);
    const double Ah = (double)pb->A[h];
    const double Dh = pb->D ? (double)pb->D[h] : 0.0;
    for (int i = 0; i < pb->nseq; ++i) {
        for (int n = 0; n < N; ++n)
            for (int j = 0; j < w; ++j)
                S[n * w + j] = pb->init ? pb->init[(((long)i * H + h) * N + n) * P + p0 + j] : 0.0;
        for (long t = pb->cu[i]; t < pb->cu[i + 1]; ++t) {
            const float *xr = pb->x + (t * H + h) * P + p0;
            const double dtv = (double)pb->dt[t * H + h];
            const float *Br = pb->B + (t * pb->G + g) * N;
            const float *Cr = pb->C + (t * pb->G + g) * N;
            const double abar = exp(dtv * Ah);
            for (int n = 0; n < N; ++n) {
                const double bbar = dtv * (double)Br[n];
                double *Sn = S + n * w;
                for (int j = 0; j < w; ++j)
                    Sn[j] = abar * Sn[j] + bbar * (double)xr[j];
            }
            if (pb->y)
                for (int j = 0; j < w; ++j) {
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n)
                        acc += (double)Cr[n] * S[n * w + j];
                    pb->y[(t * H + h) * P + p0 + j] = acc + Dh * (double)xr[j];
                }
        }
        if (pb->fin)
            for (int n = 0; n < N; ++n)
                for (int j = 0; j < w; ++j)
                    pb->fin[(((long)i * H + h) * N + n) * P + p0 + j] = S[n * w + j];
    }
}

static void *vworker(void *arg)
{
    vproblem *pb = (vproblem *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)pb->N * PBLK);
    if (!S)
        return (void *)1;
    for (;;) {
        long i = __atomic_fetch_add(&pb->next, 1, __ATOMIC_RELAXED);
        if (i >= pb->ntasks)
            break;
        run_vtask(pb, i, S);
    }
    free(S);
    return NULL;
}

int oracle_ssd_fwd_varlen(const float *x, const float *dt, const float *A, const float *B,
                          const float *C, const float *D, const int *cu, int nseq,
                          const double *init, double *y, double *final_state,
                          long T, int H, int P, int N, int G, int nthreads)
{
    if (check_dims(1, T, H, P, N, G) || nseq < 1 || cu[0] != 0 || cu[nseq] != T)
        return 2;
    for (int i = 0; i < nseq; ++i)
        if (cu[i + 1] < cu[i])
            return 2;
    vproblem pb = {x, dt, A, B, C, D, init, cu, nseq, T, H, P, N, G, y, final_state,
                   (long)H * ((P + PBLK - 1) / PBLK), 0};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > pb.ntasks)
        nthreads = (int)pb.ntasks;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th)
        return 1;
    int err = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, vworker, &pb) != 0) {
            err = 1;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            err = 1;
    }
    free(th);
    return err;
}
