/*
 * Reference oracle for the Mamba-2 SSD forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is a plain, slow, obviously-correct CPU evaluation of the state-space
 * recurrence, used only by the test suite, by the package's smoke check and by the
 * benchmark's CPU-baseline leg. The GPU product path never links, loads or calls it,
 * and it shares no code, header, constant or helper with the GPU kernels.
 *
 * What it computes (page "Accelerating Mamba-2 with High-Performance Forward Pass
 * Kernels in NVIDIA CUDA Tile", section "Mamba-2 architecture": the core recurrence
 * and its renamed form with a_t = A*dt_t and b_t = dt_t*B_t):
 *
 *   for every batch b and head h, with group g = h / (nheads / ngroups):
 *     state <- h0[b,h]                      (zeros when h0 is NULL)
 *     for t = 0 .. L-1:
 *       state <- exp(A[h]*dt[b,t,h]) * state + dt[b,t,h] * x[b,t,h,:] (outer) B[b,t,g,:]
 *       y[b,t,h,:] = state . C[b,t,g,:] + D[h] * x[b,t,h,:]
 *     final[b,h] = state
 *
 * Readings taken where the page is loose (each is listed with its reason in the
 * project's design notes):
 *   - the output reads the state AFTER the token's own update (inclusive), as in the
 *     page's chunk-output derivation and its causal mask that keeps the diagonal;
 *   - the state is stored [headdim][dstate] with dstate fastest (the page's kernels
 *     tile it as [head-dim tile, state tile]); mathematically it is the transpose of
 *     the S-by-P matrix of the page's prose;
 *   - D is one scalar per head; exp is the natural exponential, in double.
 *
 * Inputs arrive as float32 (every bf16 or fp32 input value is exactly representable)
 * and all arithmetic is IEEE double. Build plainly (no -ffast-math).
 *
 * Optionally the state is emitted every `emit_every` tokens, BEFORE the token at
 * t = k*emit_every is applied: that is the initial state of chunk k when the chunk
 * size is emit_every (the quantity the page's state-passing kernel stores per chunk).
 *
 * Parallel only over (batch, head) pairs, with POSIX threads; the per-pair loop is
 * sequential over tokens exactly as written above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
    const float *x, *dt, *A, *Bm, *Cm, *D, *h0;
    double *y, *hfinal, *hemit;
    int64_t emit_every, n_emit;
    int64_t next_pair; /* guarded by lock */
    pthread_mutex_t lock;
    int failed;
} job_t;

static void run_pair(job_t* J, int64_t b, int64_t h, double* state) {
    const int64_t L = J->seqlen, H = J->nheads, P = J->headdim, S = J->dstate;
    const int64_t G = J->ngroups, hpg = H / G, g = h / hpg;
    const double Ah = (double)J->A[h];
    const double Dh = J->D ? (double)J->D[h] : 0.0;

    if (J->h0) {
        const float* src = J->h0 + (b * H + h) * P * S;
        for (int64_t i = 0; i < P * S; ++i) state[i] = (double)src[i];
    } else {
        memset(state, 0, sizeof(double) * (size_t)(P * S));
    }

    for (int64_t t = 0; t < L; ++t) {
        if (J->hemit && J->emit_every > 0 && t % J->emit_every == 0) {
            double* dst = J->hemit + ((b * H + h) * J->n_emit + t / J->emit_every) * P * S;
            memcpy(dst, state, sizeof(double) * (size_t)(P * S));
        }
        const double dtv = (double)J->dt[(b * L + t) * H + h];
        const double alpha = exp(Ah * dtv);
        const float* xt = J->x + ((b * L + t) * H + h) * P;
        const float* Bt = J->Bm + ((b * L + t) * G + g) * S;
        const float* Ct = J->Cm + ((b * L + t) * G + g) * S;
        double* yt = J->y ? J->y + ((b * L + t) * H + h) * P : NULL;
        for (int64_t p = 0; p < P; ++p) {
            double* row = state + p * S;
            const double xp = (double)xt[p];
            double acc = 0.0;
            for (int64_t s = 0; s < S; ++s) {
                const double bs = dtv * (double)Bt[s]; /* b_t = dt_t * B_t */
                row[s] = alpha * row[s] + bs * xp;     /* state <- e^{a_t} state + b_t x_t^T */
                acc += row[s] * (double)Ct[s];         /* c_t^T state (after the update) */
            }
            if (yt) yt[p] = acc + Dh * xp;
        }
    }
    if (J->hfinal) {
        memcpy(J->hfinal + (b * H + h) * P * S, state, sizeof(double) * (size_t)(P * S));
    }
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    double* state = (double*)malloc(sizeof(double) * (size_t)(J->headdim * J->dstate));
    if (!state) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
        return NULL;
    }
    const int64_t npairs = J->batch * J->nheads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t k = J->next_pair++;
        pthread_mutex_unlock(&J->lock);
        if (k >= npairs) break;
        run_pair(J, k / J->nheads, k % J->nheads, state);
    }
    free(state);
    return NULL;
}

/*
 * Returns 0 on success, 1 on an invalid argument, 2 on an allocation or thread failure.
 * Layouts (row-major, last index fastest):
 *   x [batch, seqlen, nheads, headdim]    dt [batch, seqlen, nheads]    A, D [nheads]
 *   Bm, Cm [batch, seqlen, ngroups, dstate]
 *   h0, hfinal [batch, nheads, headdim, dstate]
 *   y [batch, seqlen, nheads, headdim]
 *   hemit [batch, nheads, ceil(seqlen / emit_every), headdim, dstate]
 * D, h0, y, hfinal and hemit may be NULL.
 */
int ssd_oracle_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, const float* x, const float* dt,
                       const float* A, const float* Bm, const float* Cm, const float* D,
                       const float* h0, double* y, double* hfinal, int64_t emit_every,
                       double* hemit, int nthreads) {
    if (batch < 1 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1)
        return 1;
    if (nheads % ngroups != 0) return 1;
    if (!x || !dt || !A || !Bm || !Cm) return 1;
    if (hemit && emit_every < 1) return 1;

    job_t J;
    memset(&J, 0, sizeof(J));
    J.batch = batch; J.seqlen = seqlen; J.nheads = nheads; J.headdim = headdim;
    J.dstate = dstate; J.ngroups = ngroups;
    J.x = x; J.dt = dt; J.A = A; J.Bm = Bm; J.Cm = Cm; J.D = D; J.h0 = h0;
    J.y = y; J.hfinal = hfinal; J.hemit = hemit;
    J.emit_every = emit_every;
    J.n_emit = emit_every > 0 ? (seqlen + emit_every - 1) / emit_every : 0;
    pthread_mutex_init(&J.lock, NULL);

    const int64_t npairs = batch * nheads;
    int nt = nthreads < 1 ? 1 : nthreads;
    if (nt > npairs) nt = (int)npairs;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) return 2;
    int started = 0;
    for (int i = 0; i < nt; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? 2 : 0;
}
