/*
 * Gradient oracle for the Mamba-2 SSD recurrence -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow fp64 reverse-mode differentiation of the token recurrence that
 * ssd_oracle.c evaluates (page "Accelerating Mamba-2 with High-Performance Forward Pass
 * Kernels in NVIDIA CUDA Tile", section "Mamba-2 architecture"):
 *
 *   H_{-1} = h0 (zeros when absent);  for t = 0 .. L-1:
 *     H_t = exp(A dt_t) H_{t-1} + dt_t x_t (outer) B_t      (H is [headdim][dstate])
 *     y_t = H_t C_t + D x_t
 *   final = H_{L-1}
 *
 * Given dL/dy_t and dL/dfinal it returns dL/d(x, dt, A, B, C, D, h0). With
 * Lam_t = dL/dH_t (all later uses of H_t included) the chain rule gives, walking t down:
 *
 *   Lam_t  = dy_t (outer) C_t + exp(A dt_{t+1}) Lam_{t+1}     (Lam_{L-1} gets dfinal too)
 *   dx_t   = D dy_t + dt_t Lam_t B_t
 *   dB_t  += dt_t Lam_t^T x_t                 (summed over the heads of B's group)
 *   dC_t  += H_t^T dy_t                       (summed over the heads of C's group)
 *   da_t   = exp(A dt_t) <Lam_t, H_{t-1}>     (d/d of the exponent a_t = A dt_t)
 *   ddt_t  = x_t . (Lam_t B_t) + A da_t
 *   dA    += dt_t da_t,   dD += dy_t . x_t,   dh0 = exp(A dt_0) Lam_0
 *
 * Inputs are double here (so that finite differences can perturb them); values that
 * come from bf16 or fp32 tensors are passed exactly. H_t is recomputed from checkpoints
 * taken every 64 tokens; nothing else is blocked or reordered. Threads run over
 * (batch, group) pairs so that each thread owns its group's dB and dC rows; dA and dD are
 * returned per (batch, head) and summed by the caller. Build plainly (no -ffast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CKPT 64

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
    const double *x, *dt, *A, *Bm, *Cm, *D, *h0, *dy, *dfinal;
    double *y, *hfinal;                                  /* forward */
    double *dx, *ddt, *dA_bh, *dB, *dC, *dD_bh, *dh0;    /* backward */
    int64_t next; /* guarded by lock */
    pthread_mutex_t lock;
    int failed;
} gjob_t;

/* state after token t of head (b, h): H <- exp(A dt) H + dt x B^T */
static void step(const gjob_t* J, int64_t b, int64_t h, int64_t t, double* H) {
    const int64_t L = J->seqlen, Hn = J->nheads, P = J->headdim, S = J->dstate;
    const int64_t G = J->ngroups, g = h / (Hn / G);
    const double dtv = J->dt[(b * L + t) * Hn + h];
    const double alpha = exp(J->A[h] * dtv);
    const double* xt = J->x + ((b * L + t) * Hn + h) * P;
    const double* Bt = J->Bm + ((b * L + t) * G + g) * S;
    for (int64_t p = 0; p < P; ++p)
        for (int64_t s = 0; s < S; ++s) H[p * S + s] = alpha * H[p * S + s] + dtv * Bt[s] * xt[p];
}

static void init_state(const gjob_t* J, int64_t b, int64_t h, double* H) {
    const int64_t PS = J->headdim * J->dstate;
    if (J->h0) memcpy(H, J->h0 + (b * J->nheads + h) * PS, sizeof(double) * (size_t)PS);
    else memset(H, 0, sizeof(double) * (size_t)PS);
}

static void forward_head(const gjob_t* J, int64_t b, int64_t h, double* H) {
    const int64_t L = J->seqlen, Hn = J->nheads, P = J->headdim, S = J->dstate;
    const int64_t G = J->ngroups, g = h / (Hn / G);
    const double Dh = J->D ? J->D[h] : 0.0;
    init_state(J, b, h, H);
    for (int64_t t = 0; t < L; ++t) {
        step(J, b, h, t, H);
        if (J->y) {
            const double* xt = J->x + ((b * L + t) * Hn + h) * P;
            const double* Ct = J->Cm + ((b * L + t) * G + g) * S;
            double* yt = J->y + ((b * L + t) * Hn + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t s = 0; s < S; ++s) acc += H[p * S + s] * Ct[s];
                yt[p] = acc + Dh * xt[p];
            }
        }
    }
    if (J->hfinal) memcpy(J->hfinal + (b * Hn + h) * P * S, H, sizeof(double) * (size_t)(P * S));
}

/* Backward through one head; seg holds CKPT+1 states, ckpt the checkpoints. */
static void backward_head(gjob_t* J, int64_t b, int64_t h, double* ckpt, double* seg,
                          double* Lam, double* u) {
    const int64_t L = J->seqlen, Hn = J->nheads, P = J->headdim, S = J->dstate, PS = P * S;
    const int64_t G = J->ngroups, g = h / (Hn / G);
    const double Ah = J->A[h];
    const double Dh = J->D ? J->D[h] : 0.0;
    const int64_t nseg = (L + CKPT - 1) / CKPT;

    /* checkpoints: ckpt[k] = H_{k*CKPT - 1}, the state before token k*CKPT */
    init_state(J, b, h, seg);
    for (int64_t t = 0; t < L; ++t) {
        if (t % CKPT == 0) memcpy(ckpt + (t / CKPT) * PS, seg, sizeof(double) * (size_t)PS);
        step(J, b, h, t, seg);
    }

    if (J->dfinal) memcpy(Lam, J->dfinal + (b * Hn + h) * PS, sizeof(double) * (size_t)PS);
    else memset(Lam, 0, sizeof(double) * (size_t)PS);
    double dA = 0.0, dD = 0.0;

    for (int64_t k = nseg - 1; k >= 0; --k) {
        const int64_t t0 = k * CKPT, t1 = (t0 + CKPT < L) ? t0 + CKPT : L;
        /* seg[i] = H_{t0 - 1 + i}, i = 0 .. t1 - t0 */
        memcpy(seg, ckpt + k * PS, sizeof(double) * (size_t)PS);
        for (int64_t t = t0; t < t1; ++t) {
            double* next = seg + (t - t0 + 1) * PS;
            memcpy(next, seg + (t - t0) * PS, sizeof(double) * (size_t)PS);
            step(J, b, h, t, next);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double* Ht = seg + (t - t0 + 1) * PS;
            const double* Hprev = seg + (t - t0) * PS;
            const double dtv = J->dt[(b * L + t) * Hn + h];
            const double alpha = exp(Ah * dtv);
            const double* xt = J->x + ((b * L + t) * Hn + h) * P;
            const double* Bt = J->Bm + ((b * L + t) * G + g) * S;
            const double* Ct = J->Cm + ((b * L + t) * G + g) * S;
            const double* dyt = J->dy + ((b * L + t) * Hn + h) * P;
            double* dxt = J->dx + ((b * L + t) * Hn + h) * P;
            double* dBt = J->dB + ((b * L + t) * G + g) * S;
            double* dCt = J->dC + ((b * L + t) * G + g) * S;

            /* Lam_t = dy_t C_t^T + (already carried) exp(a_{t+1}) Lam_{t+1} */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t s = 0; s < S; ++s) Lam[p * S + s] += dyt[p] * Ct[s];

            double v = 0.0, inner = 0.0, dyx = 0.0;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t s = 0; s < S; ++s) acc += Lam[p * S + s] * Bt[s];
                u[p] = acc;
                dxt[p] = Dh * dyt[p] + dtv * acc;
                v += xt[p] * acc;
                dyx += dyt[p] * xt[p];
            }
            for (int64_t s = 0; s < S; ++s) {
                double db = 0.0, dc = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    db += Lam[p * S + s] * xt[p];
                    dc += Ht[p * S + s] * dyt[p];
                }
                dBt[s] += dtv * db;
                dCt[s] += dc;
            }
            for (int64_t i = 0; i < PS; ++i) inner += Lam[i] * Hprev[i];
            const double da = alpha * inner;
            J->ddt[(b * L + t) * Hn + h] = v + Ah * da;
            dA += dtv * da;
            dD += dyx;

            /* carry to token t-1 */
            for (int64_t i = 0; i < PS; ++i) Lam[i] *= alpha;
        }
    }
    memcpy(J->dh0 + (b * Hn + h) * PS, Lam, sizeof(double) * (size_t)PS);
    J->dA_bh[b * Hn + h] = dA;
    J->dD_bh[b * Hn + h] = dD;
}

static void* fwd_worker(void* arg) {
    gjob_t* J = (gjob_t*)arg;
    double* H = (double*)malloc(sizeof(double) * (size_t)(J->headdim * J->dstate));
    if (!H) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t k = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (k >= J->batch * J->nheads) break;
        forward_head(J, k / J->nheads, k % J->nheads, H);
    }
    free(H);
    return NULL;
}

static void* bwd_worker(void* arg) {
    gjob_t* J = (gjob_t*)arg;
    const int64_t PS = J->headdim * J->dstate;
    const int64_t nseg = (J->seqlen + CKPT - 1) / CKPT;
    double* ckpt = (double*)malloc(sizeof(double) * (size_t)((nseg + 1) * PS));
    double* seg = (double*)malloc(sizeof(double) * (size_t)((CKPT + 1) * PS));
    double* Lam = (double*)malloc(sizeof(double) * (size_t)PS);
    double* u = (double*)malloc(sizeof(double) * (size_t)J->headdim);
    if (!ckpt || !seg || !Lam || !u) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
    } else {
        const int64_t hpg = J->nheads / J->ngroups;
        for (;;) {
            pthread_mutex_lock(&J->lock);
            const int64_t k = J->next++;
            pthread_mutex_unlock(&J->lock);
            if (k >= J->batch * J->ngroups) break;
            const int64_t b = k / J->ngroups, g = k % J->ngroups;
            for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) backward_head(J, b, h, ckpt, seg, Lam, u);
        }
    }
    free(ckpt);
    free(seg);
    free(Lam);
    free(u);
    return NULL;
}

static int run(gjob_t* J, void* (*fn)(void*), int nthreads) {
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return 2;
    pthread_mutex_init(&J->lock, NULL);
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, fn, J) != 0) break;
        ++started;
    }
    if (started == 0) fn(J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J->lock);
    free(th);
    return J->failed ? 2 : 0;
}

static int check(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                 int64_t ngroups) {
    return batch < 1 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 ||
           nheads % ngroups != 0;
}

/*
 * fp64-input forward (y and final may be NULL). Layouts as in ssd_oracle.c:
 *   x [batch, seqlen, nheads, headdim], dt [batch, seqlen, nheads], A, D [nheads],
 *   B, C [batch, seqlen, ngroups, dstate], h0, final [batch, nheads, headdim, dstate],
 *   y [batch, seqlen, nheads, headdim]. Returns 0, 1 (bad sizes) or 2 (no memory).
 */
int ssd_oracle_forward_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                           int64_t dstate, int64_t ngroups, const double* x, const double* dt,
                           const double* A, const double* Bm, const double* Cm, const double* D,
                           const double* h0, double* y, double* hfinal, int nthreads) {
    if (check(batch, seqlen, nheads, headdim, dstate, ngroups) || !x || !dt || !A || !Bm || !Cm)
        return 1;
    gjob_t J;
    memset(&J, 0, sizeof(J));
    J.batch = batch; J.seqlen = seqlen; J.nheads = nheads; J.headdim = headdim;
    J.dstate = dstate; J.ngroups = ngroups;
    J.x = x; J.dt = dt; J.A = A; J.Bm = Bm; J.Cm = Cm; J.D = D; J.h0 = h0;
    J.y = y; J.hfinal = hfinal;
    return run(&J, fwd_worker, nthreads);
}

/*
 * Gradients of sum(dy * y) + sum(dfinal * final) (dfinal may be NULL = 0). Outputs,
 * written in full: dx, dy-shaped; ddt [batch, seqlen, nheads]; dB, dC [batch, seqlen,
 * ngroups, dstate]; dh0 [batch, nheads, headdim, dstate]; dA_bh, dD_bh [batch, nheads]
 * (per-batch terms of dA and dD). Returns 0, 1 or 2 as above.
 */
int ssd_oracle_backward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t ngroups, const double* x, const double* dt,
                        const double* A, const double* Bm, const double* Cm, const double* D,
                        const double* h0, const double* dy, const double* dfinal, double* dx,
                        double* ddt, double* dA_bh, double* dB, double* dC, double* dD_bh,
                        double* dh0, int nthreads) {
    if (check(batch, seqlen, nheads, headdim, dstate, ngroups) || !x || !dt || !A || !Bm ||
        !Cm || !dy || !dx || !ddt || !dA_bh || !dB || !dC || !dD_bh || !dh0)
        return 1;
    gjob_t J;
    memset(&J, 0, sizeof(J));
    J.batch = batch; J.seqlen = seqlen; J.nheads = nheads; J.headdim = headdim;
    J.dstate = dstate; J.ngroups = ngroups;
    J.x = x; J.dt = dt; J.A = A; J.Bm = Bm; J.Cm = Cm; J.D = D; J.h0 = h0;
    J.dy = dy; J.dfinal = dfinal;
    J.dx = dx; J.ddt = ddt; J.dA_bh = dA_bh; J.dB = dB; J.dC = dC; J.dD_bh = dD_bh; J.dh0 = dh0;
    memset(dB, 0, sizeof(double) * (size_t)(batch * seqlen * ngroups * dstate));
    memset(dC, 0, sizeof(double) * (size_t)(batch * seqlen * ngroups * dstate));
    return run(&J, bwd_worker, nthreads);
}
