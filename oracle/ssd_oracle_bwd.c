/*
 * ssd_oracle_bwd.c -- plain fp64 CPU oracle of the gradients of the selective
 * state space layer core.
 *
 * TEST INFRASTRUCTURE ONLY, like ssd_oracle.c: nothing in the product path
 * links, loads or calls it, and it shares no code with the GPU library.
 *
 * The layer (youngju.dev "Mamba / selective SSM" page, section
 * "LTIからSelectionへの切り替え": abar_t = exp(dt_t A), bbar_t = dt_t B_t,
 * h_t = abar_t h_{t-1} + bbar_t x_t, y_t = C_t h_t; scalar A per head and B/C
 * shared by the heads of a group, Qiita "Mamba-2" article, sections 4.1-4.2;
 * D x skip term per head), for one batch row b, head h (group g) and one
 * column p of the N x P state, which only ever meets x[.., p] and y[.., p]:
 *
 *   s_{-1} = init[b,h,:,p]
 *   s_t    = exp(dt_t A) s_{t-1} + dt_t B_t x_t[p]          (N-vector)   (1)
 *   y_t[p] = C_t . s_t + D x_t[p]                                        (2)
 *   final[b,h,:,p] = s_{T-1}
 *
 * Given dL/dy and dL/dfinal, the gradients are reverse-mode differentiation
 * of (1) and (2), token by token, with no chunking or re-association. With
 * g_t = dL/ds_t (total), walking t = T-1 .. 0:
 *
 *   g_t      = [t == T-1] dfinal + C_t dy_t[p] + exp(dt_{t+1} A) g_{t+1}
 *   dx_t[p] += dt_t (B_t . g_t) + D dy_t[p]
 *   dB_t    += dt_t x_t[p] g_t                 (summed over p and the heads of g)
 *   dC_t    += dy_t[p] s_t                     (summed over p and the heads of g)
 *   ddt_t   += A exp(dt_t A) (g_t . s_{t-1}) + x_t[p] (B_t . g_t)   (summed over p)
 *   dA      += dt_t exp(dt_t A) (g_t . s_{t-1})                     (summed over b, t, p)
 *   dD      += dy_t[p] x_t[p]                                       (summed over b, t, p)
 *   dinit[b,h,:,p] = exp(dt_0 A) g_0
 *
 * (d s_t / d dt_t = A exp(dt_t A) s_{t-1} + B_t x_t[p]; d s_t / d A = dt_t
 * exp(dt_t A) s_{t-1}; d s_t / d s_{t-1} = exp(dt_t A).) The states s_t of a
 * column are kept from a forward pass over the column (T x N doubles).
 *
 * Work is split over (batch row, group) pairs; inside one, the heads of the
 * group and then the columns run in order, so every sum above is formed in
 * a fixed order. dA and dD are summed over batch rows at the end, in order.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *x, *dt, *A, *B, *C, *D, *dy;   /* D may be NULL (= 0) */
    const double *init, *dfinal;                 /* [b,H,N,P] or NULL (= 0) */
    double *dx, *ddt, *dB, *dC, *dinit;          /* dinit may be NULL */
    double *dA_part, *dD_part;                   /* [b, H] */
    long T;
    int batch, H, P, N, G;
    long next;                                   /* next task, atomically incremented */
} bproblem;

static void run_btask(bproblem *pb, long task, double *S /* T * N */, double *gv /* N */)
{
    const long T = pb->T;
    const int H = pb->H, P = pb->P, N = pb->N, G = pb->G;
    const int b = (int)(task / G), g = (int)(task % G);
    const int hpg = H / G;
    for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
        const double Ah = (double)pb->A[h];
        const double Dh = pb->D ? (double)pb->D[h] : 0.0;
        const long bh = (long)b * H + h;
        double dA_acc = 0.0, dD_acc = 0.0;
        for (int p = 0; p < P; ++p) {
            /* forward over the column, keeping every state: (1) */
            for (long t = 0; t < T; ++t) {
                const long tok = (long)b * T + t;
                const double dtv = (double)pb->dt[tok * H + h];
                const double abar = exp(dtv * Ah);
                const double xv = (double)pb->x[(tok * H + h) * P + p];
                const float *Br = pb->B + (tok * G + g) * N;
                double *s = S + t * N;
                for (int n = 0; n < N; ++n) {
                    const double prev = t > 0 ? S[(t - 1) * N + n]
                                              : (pb->init ? pb->init[(bh * N + n) * P + p] : 0.0);
                    s[n] = abar * prev + dtv * (double)Br[n] * xv;
                }
            }
            /* reverse sweep */
            for (int n = 0; n < N; ++n)
                gv[n] = pb->dfinal ? pb->dfinal[(bh * N + n) * P + p] : 0.0;
            for (long t = T - 1; t >= 0; --t) {
                const long tok = (long)b * T + t;
                const double dtv = (double)pb->dt[tok * H + h];
                const double abar = exp(dtv * Ah);
                const double xv = (double)pb->x[(tok * H + h) * P + p];
                const double dyv = (double)pb->dy[(tok * H + h) * P + p];
                const float *Br = pb->B + (tok * G + g) * N;
                const float *Cr = pb->C + (tok * G + g) * N;
                double *dBr = pb->dB + (tok * G + g) * N;
                double *dCr = pb->dC + (tok * G + g) * N;
                const double *s = S + t * N;
                double gB = 0.0, gs = 0.0;
                for (int n = 0; n < N; ++n) {
                    gv[n] += (double)Cr[n] * dyv;                    /* through (2) */
                    dCr[n] += dyv * s[n];
                    const double prev = t > 0 ? S[(t - 1) * N + n]
                                              : (pb->init ? pb->init[(bh * N + n) * P + p] : 0.0);
                    gB += (double)Br[n] * gv[n];
                    gs += gv[n] * prev;
                }
                pb->dx[(tok * H + h) * P + p] = dtv * gB + Dh * dyv;
                for (int n = 0; n < N; ++n)
                    dBr[n] += dtv * xv * gv[n];
                pb->ddt[tok * H + h] += Ah * abar * gs + xv * gB;
                dA_acc += dtv * abar * gs;
                dD_acc += dyv * xv;
                for (int n = 0; n < N; ++n)                          /* through (1) */
                    gv[n] *= abar;
            }
            if (pb->dinit)
                for (int n = 0; n < N; ++n)
                    pb->dinit[(bh * N + n) * P + p] = gv[n];
        }
        pb->dA_part[bh] = dA_acc;
        pb->dD_part[bh] = dD_acc;
    }
}

static void *bworker(void *arg)
{
    bproblem *pb = (bproblem *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)pb->T * (size_t)pb->N);
    double *gv = (double *)malloc(sizeof(double) * (size_t)pb->N);
    void *ret = NULL;
    if (!S || !gv) {
        ret = (void *)1;
    } else {
        const long ntasks = (long)pb->batch * pb->G;
        for (;;) {
            const long i = __atomic_fetch_add(&pb->next, 1, __ATOMIC_RELAXED);
            if (i >= ntasks)
                break;
            run_btask(pb, i, S, gv);
        }
    }
    free(S);
    free(gv);
    return ret;
}

/*
 * Gradients of the forward for upstream dy [b,T,H,P] and dfinal [b,H,N,P]
 * (NULL = 0). Outputs (double): dx [b,T,H,P], ddt [b,T,H], dA [H],
 * dB [b,T,G,N], dC [b,T,G,N], dD [H], dinit [b,H,N,P] (NULL: not written).
 * Inputs as for oracle_ssd_fwd. Returns 0 on success, 2 for bad dimensions,
 * 1 for a resource failure.
 */
int oracle_ssd_bwd(const float *x, const float *dt, const float *A, const float *B, const float *C,
                   const float *D, const double *init, const float *dy, const double *dfinal, double *dx,
                   double *ddt, double *dA, double *dB, double *dC, double *dD, double *dinit, long batch,
                   long T, int H, int P, int N, int G, int nthreads)
{
    if (batch < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G)
        return 2;
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC || !dD)
        return 2;
    bproblem pb;
    memset(&pb, 0, sizeof(pb));
    pb.x = x; pb.dt = dt; pb.A = A; pb.B = B; pb.C = C; pb.D = D; pb.dy = dy;
    pb.init = init; pb.dfinal = dfinal;
    pb.dx = dx; pb.ddt = ddt; pb.dB = dB; pb.dC = dC; pb.dinit = dinit;
    pb.T = T; pb.batch = (int)batch; pb.H = H; pb.P = P; pb.N = N; pb.G = G;
    pb.dA_part = (double *)calloc((size_t)batch * H, sizeof(double));
    pb.dD_part = (double *)calloc((size_t)batch * H, sizeof(double));
    if (!pb.dA_part || !pb.dD_part) {
        free(pb.dA_part);
        free(pb.dD_part);
        return 1;
    }
    memset(ddt, 0, sizeof(double) * (size_t)batch * T * H);
    memset(dB, 0, sizeof(double) * (size_t)batch * T * G * N);
    memset(dC, 0, sizeof(double) * (size_t)batch * T * G * N);

    const long ntasks = batch * G;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > ntasks)
        nthreads = (int)ntasks;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int err = th ? 0 : 1, started = 0;
    for (int i = 0; !err && i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, bworker, &pb) != 0)
            err = 1;
        else
            ++started;
    }
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            err = 1;
    }
    free(th);
    if (!err)
        for (int h = 0; h < H; ++h) {
            double a = 0.0, d = 0.0;
            for (long b = 0; b < batch; ++b) {
                a += pb.dA_part[b * H + h];
                d += pb.dD_part[b * H + h];
            }
            dA[h] = a;
            dD[h] = d;
        }
    free(pb.dA_part);
    free(pb.dD_part);
    return err;
}
