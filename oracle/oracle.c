/*
 * oracle.c -- plain fp64 CPU oracle for causal linear attention run as the
 * unified recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg load it; the product library never
 * does, and this file shares no code, header or table with it.
 *
 * What it computes, per (batch b, head h) pair, written out from its
 * definition (the token-by-token recurrence):
 *
 *   S <- S0 (or 0) [dk x dv],  z <- z0 (or 0) [dk]
 *   for t = 0 .. L-1:
 *       a_t  = 1 | gamma[h] | exp(log_alpha[b,h,t,:])       (the gate A_t)
 *       qf   = phi(q_t),  kf = phi(k_t)        (phi = identity or elu+1)
 *       S    = diag(a_t) S + kf v_t^T          (decay old state, add token)
 *       z    = a_t * z + kf                    (only when normalising)
 *       o_t  = qf^T S   [/ (qf . z) when normalising]      (read after update)
 *
 * Sources (cited by page title and section):
 *  - "Module 22: Linear & Recurrent Attention", section "The Math: Linear
 *    Attention": phi = elu+1, the running S and Z sums and the normalised
 *    read-out; section "Retention: Add a Decay to the State": S_n = gamma
 *    S_{n-1} + k_n^T v_n with no normaliser; section "Interactive
 *    Exploration: The One Recurrence Behind Them All": S_t = A_t S_{t-1} +
 *    k_t^T v_t with the gate table A_t in {1, gamma, f(x_t)}.
 *  - "linear_sparse_attention.py", function linear_attn_recurrent: the state
 *    is d_k x d_v and it is updated before o_t is read (self-inclusive).
 *  - "causal linear attention as an RNN": S_0 = 0, Z_0 = 0 and the output
 *    phi(Q_t) S_t / phi(Q_t) Z_t.
 *
 * Two further fp64 forms of the same function are coded independently of the
 * token loop; they exist to cross-check it:
 *  - oracle_parallel: the masked all-pairs form (the "parallel face" in the
 *    Module 22 sections "Code: The Two Faces of Linear Attention" and "The
 *    Three Faces of Retention", decay matrix D), O(L^2) per pair, with the
 *    decay between s and t taken as the direct product of the gates in
 *    between (so gamma = 0 works: an empty product is 1).
 *  - oracle_chunkwise: the chunkwise form of "The Three Faces of Retention"
 *    (intra-chunk term, cross-chunk term scaled by the decay up to and
 *    including t, carried-state update), generalised to per-channel gates and
 *    to a ragged last chunk as in linear_attn_chunkwise of
 *    "linear_sparse_attention.py".  All decays are direct products.
 *
 * Readings taken where the pages are silent:
 *  - under a gate, z follows the same gate as S (z is S for an all-ones
 *    value column);
 *  - no epsilon in the divide;
 *  - elu uses alpha = 1;
 *  - S0 is decayed by the first token's gate like any older state.
 *
 * oracle_backward is the reverse-mode derivative of the token loop above,
 * written out step by step in reverse (no chunking, no cumulative-sum
 * identities): with G the gradient of the loss with respect to the state
 * after token t,
 *
 *   G     += qf_t do_t^T              (o_t = qf_t^T S_t reads S_t)
 *   dqf_t  = S_t do_t
 *   dkf_t  = G v_t,   dv_t = G^T kf_t  (S_t = diag(a_t) S_{t-1} + kf_t v_t^T)
 *   d log a_t,i = a_t,i sum_j G[i,j] S_{t-1}[i,j]   (diagonal gate only)
 *   G      = diag(a_t) G               (the gradient of S_{t-1})
 *
 * starting from G = dS_final and ending with dS0 = G; the chain rule through
 * phi gives dq = dqf phi'(q), dk = dkf phi'(k).  The states S_t are
 * recomputed block by block from checkpoints every `ck` tokens.  The
 * normalised read-out has no backward here.  None of this comes from the
 * pages (they give no gradients); it is the plain derivative of the loop.
 *
 * oracle_delta_run is the delta rule's token loop (see form 4 below).
 *
 * The global `oracle_mutation` plants a known mistake for the mutation tests
 * that prove the pins can catch it; it is 0 (no mutation) everywhere else.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

enum { GATE_NONE = 0, GATE_GAMMA = 1, GATE_DIAG = 2 };
enum { PHI_IDENTITY = 0, PHI_ELU1 = 1 };

/* Planted mistakes, test-only.  0 = the correct oracle. */
enum {
    MUT_NONE = 0,
    MUT_Z_FROZEN = 1,      /* z never updated after z0              */
    MUT_NO_DIVIDE = 2,     /* normaliser computed but not applied    */
    MUT_READ_BEFORE = 3,   /* o_t read from S_{t-1}                  */
    MUT_TRANSPOSED = 4,    /* S += v k^T (rows indexed by d_v)        */
    MUT_DECAY_AFTER = 5,   /* S = A (S + k v^T): decays the new token */
    MUT_PHI_ON_V = 6,      /* phi also applied to v                   */
    MUT_GATE_DROPPED = 7,  /* A_t treated as 1                        */
    MUT_CROSS_OFF_BY_1 = 8,/* chunkwise: cross term decayed to t-1     */
    MUT_STATE_OFF_BY_1 = 9,/* chunkwise: carried state decayed c-1     */
    MUT_GAMMA_SQUARED = 10,/* retention gate applied twice per token  */
    MUT_BWD_NO_DECAY = 11, /* backward: G not decayed by a_t           */
    MUT_BWD_DQ_PREV = 12,  /* backward: dq read from S_{t-1}           */
    MUT_DELTA_NO_ERASE = 13,   /* delta rule: erase term dropped       */
    MUT_DELTA_ERASE_AFTER = 14 /* delta rule: erase applied after write */
};

int oracle_mutation = 0;

void oracle_set_mutation(int m) { oracle_mutation = m; }
int oracle_get_mutation(void) { return oracle_mutation; }

/* phi(x) = elu(x) + 1 = x + 1 for x > 0, exp(x) for x <= 0 (alpha = 1). */
double oracle_phi(int phi, double x) {
    if (phi == PHI_ELU1) return x > 0.0 ? x + 1.0 : exp(x);
    return x;
}

/* Multi-scale retention decays gamma_h = 1 - 2^(-5-h), h = 0..n-1
 * ("Module 22", section on multi-scale retention after the three faces). */
void oracle_multiscale_decays(int n, double* out) {
    for (int h = 0; h < n; ++h) out[h] = 1.0 - pow(2.0, -5.0 - (double)h);
}

typedef struct {
    int B, H, L, dk, dv;
    int gate_mode;
    const double* gamma;     /* [H]            (GAMMA)  */
    const double* log_alpha; /* [B,H,L,dk]     (DIAG)   */
    int phi, normalize;
    const double *q, *k, *v; /* [B,H,L,dk|dv]           */
    const double *S0, *z0;   /* [B,H,dk,dv], [B,H,dk]; may be NULL */
    double* out;             /* [B,H,L,dv]              */
    double *S_final, *z_final; /* may be NULL           */
    int chunk;               /* chunkwise form only     */
    /* backward (form 3) */
    const double *dout, *dS_final;          /* [B,H,L,dv], [B,H,dk,dv] (may be NULL) */
    double *dq, *dk_out, *dv_out;           /* [B,H,L,dk|dv]          */
    double *dlog_alpha, *dS0;               /* [B,H,L,dk], [B,H,dk,dv] (may be NULL) */
    int ck;                                 /* checkpoint spacing      */
    /* delta rule (form 4) */
    const double* beta;                     /* [B,H,L] write strengths */
    int use_delta;                          /* 0: additive S += k v^T  */
    int form;                /* 0 loop, 1 parallel, 2 chunkwise, 3 backward, 4 delta */
    int nthreads;
    int next_pair;           /* work counter (guarded by mu) */
    pthread_mutex_t mu;
} job_t;

/* Gate of token t (pair bh) on channel i. */
static double gate_at(const job_t* J, int bh, int t, int i) {
    if (oracle_mutation == MUT_GATE_DROPPED) return 1.0;
    if (J->gate_mode == GATE_GAMMA) {
        double g = J->gamma[bh % J->H];
        if (oracle_mutation == MUT_GAMMA_SQUARED) return g * g;
        return g;
    }
    if (J->gate_mode == GATE_DIAG)
        return exp(J->log_alpha[((size_t)bh * J->L + t) * J->dk + i]);
    return 1.0;
}

/* ---------------------------------------------------------------------- */
/* Form 0: the token loop (the definition).                                */
/* ---------------------------------------------------------------------- */
static void run_loop_pair(const job_t* J, int bh) {
    const int L = J->L, dk = J->dk, dv = J->dv;
    double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* z = (double*)calloc((size_t)dk, sizeof(double));
    double* qf = (double*)malloc(sizeof(double) * dk);
    double* kf = (double*)malloc(sizeof(double) * dk);
    double* vv = (double*)malloc(sizeof(double) * dv);
    double* a = (double*)malloc(sizeof(double) * dk);
    if (J->S0) memcpy(S, J->S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
    if (J->z0) memcpy(z, J->z0 + (size_t)bh * dk, sizeof(double) * dk);

    for (int t = 0; t < L; ++t) {
        const double* qt = J->q + ((size_t)bh * L + t) * dk;
        const double* kt = J->k + ((size_t)bh * L + t) * dk;
        const double* vt = J->v + ((size_t)bh * L + t) * dv;
        double* ot = J->out + ((size_t)bh * L + t) * dv;
        for (int i = 0; i < dk; ++i) {
            qf[i] = oracle_phi(J->phi, qt[i]);
            kf[i] = oracle_phi(J->phi, kt[i]);
            a[i] = gate_at(J, bh, t, i);
        }
        for (int j = 0; j < dv; ++j)
            vv[j] = oracle_mutation == MUT_PHI_ON_V ? oracle_phi(J->phi, vt[j]) : vt[j];

        /* o_t read from the previous state (planted mistake only). */
        if (oracle_mutation == MUT_READ_BEFORE) {
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += qf[i] * S[(size_t)i * dv + j];
                ot[j] = acc;
            }
        }

        /* S <- diag(a) S + kf v^T */
        for (int i = 0; i < dk; ++i) {
            double* Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) {
                double add;
                if (oracle_mutation == MUT_TRANSPOSED)
                    add = kf[j < dk ? j : 0] * vv[i < dv ? i : 0]; /* S[i][j] += v_i k_j */
                else
                    add = kf[i] * vv[j];
                if (oracle_mutation == MUT_DECAY_AFTER)
                    Si[j] = a[i] * (Si[j] + add);
                else
                    Si[j] = a[i] * Si[j] + add;
            }
        }
        /* z <- a z + kf */
        if (J->normalize && oracle_mutation != MUT_Z_FROZEN)
            for (int i = 0; i < dk; ++i) z[i] = a[i] * z[i] + kf[i];

        if (oracle_mutation != MUT_READ_BEFORE) {
            /* o_t = qf^T S_t */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += qf[i] * S[(size_t)i * dv + j];
                ot[j] = acc;
            }
        }
        if (J->normalize && oracle_mutation != MUT_NO_DIVIDE) {
            double den = 0.0;
            for (int i = 0; i < dk; ++i) den += qf[i] * z[i];
            for (int j = 0; j < dv; ++j) ot[j] /= den;
        }
    }
    if (J->S_final) memcpy(J->S_final + (size_t)bh * dk * dv, S, sizeof(double) * dk * dv);
    if (J->z_final) memcpy(J->z_final + (size_t)bh * dk, z, sizeof(double) * dk);
    free(S); free(z); free(qf); free(kf); free(vv); free(a);
}

/* ---------------------------------------------------------------------- */
/* Form 1: all pairs (s <= t) at once, decay as a direct product.          */
/*   out_t = sum_{s<=t} [sum_i qf_ti kf_si prod_{r=s+1..t} a_ri] v_s        */
/*         + sum_i qf_ti [prod_{r=0..t} a_ri] S0[i,:]                       */
/*   den_t = same with v_s -> 1 and S0 -> z0.                              */
/* ---------------------------------------------------------------------- */
static void run_parallel_pair(const job_t* J, int bh) {
    const int L = J->L, dk = J->dk, dv = J->dv;
    double* A = (double*)malloc(sizeof(double) * (size_t)L * dk); /* gates */
    double* QF = (double*)malloc(sizeof(double) * (size_t)L * dk);
    double* KF = (double*)malloc(sizeof(double) * (size_t)L * dk);
    double* prod = (double*)malloc(sizeof(double) * dk);
    for (int t = 0; t < L; ++t)
        for (int i = 0; i < dk; ++i) {
            A[(size_t)t * dk + i] = gate_at(J, bh, t, i);
            QF[(size_t)t * dk + i] = oracle_phi(J->phi, J->q[((size_t)bh * L + t) * dk + i]);
            KF[(size_t)t * dk + i] = oracle_phi(J->phi, J->k[((size_t)bh * L + t) * dk + i]);
        }
    for (int t = 0; t < L; ++t) {
        double* ot = J->out + ((size_t)bh * L + t) * dv;
        double den = 0.0;
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int s = 0; s <= t; ++s) {
            /* score with decay D_ts,i = prod_{r=s+1..t} a_ri */
            double score = 0.0;
            for (int i = 0; i < dk; ++i) {
                double d = 1.0;
                for (int r = s + 1; r <= t; ++r) d *= A[(size_t)r * dk + i];
                score += QF[(size_t)t * dk + i] * KF[(size_t)s * dk + i] * d;
            }
            const double* vs = J->v + ((size_t)bh * L + s) * dv;
            for (int j = 0; j < dv; ++j) ot[j] += score * vs[j];
            den += score;
        }
        if (J->S0 || J->z0) {
            for (int i = 0; i < dk; ++i) {
                double d = 1.0;
                for (int r = 0; r <= t; ++r) d *= A[(size_t)r * dk + i];
                double w = QF[(size_t)t * dk + i] * d;
                if (J->S0)
                    for (int j = 0; j < dv; ++j)
                        ot[j] += w * J->S0[((size_t)bh * dk + i) * dv + j];
                if (J->z0) den += w * J->z0[(size_t)bh * dk + i];
            }
        }
        if (J->normalize)
            for (int j = 0; j < dv; ++j) ot[j] /= den;
    }
    /* Final state: S_L = sum_s [prod_{r=s+1..L-1} a_r] kf_s v_s^T + [prod_r a_r] S0 */
    if (J->S_final || J->z_final) {
        for (int i = 0; i < dk; ++i) {
            double dall = 1.0;
            for (int r = 0; r < L; ++r) dall *= A[(size_t)r * dk + i];
            if (J->S_final) {
                double* Si = J->S_final + ((size_t)bh * dk + i) * dv;
                for (int j = 0; j < dv; ++j)
                    Si[j] = J->S0 ? dall * J->S0[((size_t)bh * dk + i) * dv + j] : 0.0;
            }
            if (J->z_final) {
                const double z0i = J->z0 ? J->z0[(size_t)bh * dk + i] : 0.0;
                J->z_final[(size_t)bh * dk + i] = J->normalize ? dall * z0i : z0i;
            }
            for (int s = 0; s < L; ++s) {
                double d = 1.0;
                for (int r = s + 1; r < L; ++r) d *= A[(size_t)r * dk + i];
                double w = KF[(size_t)s * dk + i] * d;
                if (J->S_final) {
                    double* Si = J->S_final + ((size_t)bh * dk + i) * dv;
                    const double* vs = J->v + ((size_t)bh * L + s) * dv;
                    for (int j = 0; j < dv; ++j) Si[j] += w * vs[j];
                }
                if (J->z_final && J->normalize) J->z_final[(size_t)bh * dk + i] += w;
            }
        }
    }
    (void)prod;
    free(A); free(QF); free(KF); free(prod);
}

/* ---------------------------------------------------------------------- */
/* Form 2: chunkwise.  Chunk [c0, c0+c) with chunk-local t, s:             */
/*   G_t,i   = prod_{r=0..t} a_ri                 (decay up to and incl. t) */
/*   o_t     = sum_i qf_ti G_ti R[i,:]                       (cross-chunk)  */
/*           + sum_{s<=t} [sum_i qf_ti kf_si prod_{r=s+1..t} a_ri] v_s     */
/*   R       <- diag(G_{c-1}) R + sum_s (kf_s * prod_{r=s+1..c-1} a_r) v_s^T */
/* With a = gamma: G_t = gamma^(t+1), the intra decay gamma^(t-s), the      */
/* carried decay gamma^c and gamma^(c-1-s), as in "The Three Faces of       */
/* Retention"; c is the actual length of a ragged last chunk.               */
/* ---------------------------------------------------------------------- */
static void run_chunk_pair(const job_t* J, int bh) {
    const int L = J->L, dk = J->dk, dv = J->dv, C = J->chunk;
    double* R = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* zr = (double*)calloc((size_t)dk, sizeof(double));
    double* A = (double*)malloc(sizeof(double) * (size_t)C * dk);
    double* G = (double*)malloc(sizeof(double) * (size_t)C * dk);
    double* QF = (double*)malloc(sizeof(double) * (size_t)C * dk);
    double* KF = (double*)malloc(sizeof(double) * (size_t)C * dk);
    double* Rn = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* zn = (double*)malloc(sizeof(double) * (size_t)dk);
    if (J->S0) memcpy(R, J->S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
    if (J->z0) memcpy(zr, J->z0 + (size_t)bh * dk, sizeof(double) * dk);

    for (int c0 = 0; c0 < L; c0 += C) {
        const int c = (L - c0) < C ? (L - c0) : C;
        for (int t = 0; t < c; ++t)
            for (int i = 0; i < dk; ++i) {
                A[(size_t)t * dk + i] = gate_at(J, bh, c0 + t, i);
                QF[(size_t)t * dk + i] = oracle_phi(J->phi, J->q[((size_t)bh * L + c0 + t) * dk + i]);
                KF[(size_t)t * dk + i] = oracle_phi(J->phi, J->k[((size_t)bh * L + c0 + t) * dk + i]);
            }
        for (int i = 0; i < dk; ++i) {
            double g = 1.0;
            for (int t = 0; t < c; ++t) {
                g *= A[(size_t)t * dk + i];
                G[(size_t)t * dk + i] = g;
            }
        }
        for (int t = 0; t < c; ++t) {
            double* ot = J->out + ((size_t)bh * L + c0 + t) * dv;
            double den = 0.0;
            /* cross-chunk term: (qf_t * G_t)^T R */
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                double gt = G[(size_t)t * dk + i];
                if (oracle_mutation == MUT_CROSS_OFF_BY_1)
                    gt = t > 0 ? G[(size_t)(t - 1) * dk + i] : 1.0;
                double w = QF[(size_t)t * dk + i] * gt;
                for (int j = 0; j < dv; ++j) ot[j] += w * R[(size_t)i * dv + j];
                den += w * zr[i];
            }
            /* intra-chunk term */
            for (int s = 0; s <= t; ++s) {
                double score = 0.0;
                for (int i = 0; i < dk; ++i) {
                    double d = 1.0;
                    for (int r = s + 1; r <= t; ++r) d *= A[(size_t)r * dk + i];
                    score += QF[(size_t)t * dk + i] * KF[(size_t)s * dk + i] * d;
                }
                const double* vs = J->v + ((size_t)bh * L + c0 + s) * dv;
                for (int j = 0; j < dv; ++j) ot[j] += score * vs[j];
                den += score;
            }
            if (J->normalize)
                for (int j = 0; j < dv; ++j) ot[j] /= den;
        }
        /* carried state update */
        for (int i = 0; i < dk; ++i) {
            double gc = G[(size_t)(c - 1) * dk + i];
            if (oracle_mutation == MUT_STATE_OFF_BY_1)
                gc = c > 1 ? G[(size_t)(c - 2) * dk + i] : 1.0;
            for (int j = 0; j < dv; ++j) Rn[(size_t)i * dv + j] = gc * R[(size_t)i * dv + j];
            zn[i] = J->normalize ? gc * zr[i] : zr[i];
            for (int s = 0; s < c; ++s) {
                double d = 1.0;
                for (int r = s + 1; r < c; ++r) d *= A[(size_t)r * dk + i];
                double w = KF[(size_t)s * dk + i] * d;
                const double* vs = J->v + ((size_t)bh * L + c0 + s) * dv;
                for (int j = 0; j < dv; ++j) Rn[(size_t)i * dv + j] += w * vs[j];
                if (J->normalize) zn[i] += w;
            }
        }
        memcpy(R, Rn, sizeof(double) * dk * dv);
        memcpy(zr, zn, sizeof(double) * dk);
    }
    if (J->S_final) memcpy(J->S_final + (size_t)bh * dk * dv, R, sizeof(double) * dk * dv);
    if (J->z_final) memcpy(J->z_final + (size_t)bh * dk, zr, sizeof(double) * dk);
    free(R); free(zr); free(A); free(G); free(QF); free(KF); free(Rn); free(zn);
}

/* ---------------------------------------------------------------------- */
/* Backward of the token loop (no normaliser).                             */
/* ---------------------------------------------------------------------- */
static double phi_prime(int phi, double x) {
    if (phi == PHI_ELU1) return x > 0.0 ? 1.0 : exp(x);
    return 1.0;
}

/* One forward step S <- diag(a_t) S + kf_t v_t^T for token t of pair bh. */
static void fwd_step(const job_t* J, int bh, int t, double* S) {
    const int L = J->L, dk = J->dk, dv = J->dv;
    const double* kt = J->k + ((size_t)bh * L + t) * dk;
    const double* vt = J->v + ((size_t)bh * L + t) * dv;
    for (int i = 0; i < dk; ++i) {
        const double a = gate_at(J, bh, t, i), kf = oracle_phi(J->phi, kt[i]);
        double* Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) Si[j] = a * Si[j] + kf * vt[j];
    }
}

static void run_backward_pair(const job_t* J, int bh) {
    const int L = J->L, dk = J->dk, dv = J->dv, ck = J->ck;
    const size_t SS = (size_t)dk * dv;
    const int nblk = (L + ck - 1) / ck;
    /* checkpoints: the state before token b*ck */
    double* cp = (double*)calloc((size_t)(nblk > 0 ? nblk : 1) * SS, sizeof(double));
    double* S = (double*)calloc(SS, sizeof(double));
    if (J->S0) memcpy(S, J->S0 + (size_t)bh * SS, sizeof(double) * SS);
    for (int t = 0; t < L; ++t) {
        if (t % ck == 0) memcpy(cp + (size_t)(t / ck) * SS, S, sizeof(double) * SS);
        fwd_step(J, bh, t, S);
    }
    /* states inside one block: blk[m] = state after token b*ck + m - 1 */
    double* blk = (double*)malloc((size_t)(ck + 1) * SS * sizeof(double));
    double* G = (double*)calloc(SS, sizeof(double));
    if (J->dS_final) memcpy(G, J->dS_final + (size_t)bh * SS, sizeof(double) * SS);
    for (int b = nblk - 1; b >= 0; --b) {
        const int t0 = b * ck, t1 = (t0 + ck < L) ? t0 + ck : L;
        memcpy(blk, cp + (size_t)b * SS, sizeof(double) * SS);
        for (int t = t0; t < t1; ++t) {
            memcpy(blk + (size_t)(t - t0 + 1) * SS, blk + (size_t)(t - t0) * SS, sizeof(double) * SS);
            fwd_step(J, bh, t, blk + (size_t)(t - t0 + 1) * SS);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const double* St = blk + (size_t)(t - t0 + 1) * SS;   /* after token t  */
            const double* Sp = blk + (size_t)(t - t0) * SS;       /* before token t */
            const double* qt = J->q + ((size_t)bh * L + t) * dk;
            const double* kt = J->k + ((size_t)bh * L + t) * dk;
            const double* vt = J->v + ((size_t)bh * L + t) * dv;
            const double* dot = J->dout + ((size_t)bh * L + t) * dv;
            double* dqt = J->dq + ((size_t)bh * L + t) * dk;
            double* dkt = J->dk_out + ((size_t)bh * L + t) * dk;
            double* dvt = J->dv_out + ((size_t)bh * L + t) * dv;
            const double* Sq = oracle_mutation == MUT_BWD_DQ_PREV ? Sp : St;
            for (int i = 0; i < dk; ++i) {
                const double qf = oracle_phi(J->phi, qt[i]);
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    G[(size_t)i * dv + j] += qf * dot[j];
                    acc += Sq[(size_t)i * dv + j] * dot[j];
                }
                dqt[i] = acc * phi_prime(J->phi, qt[i]);
            }
            for (int j = 0; j < dv; ++j) dvt[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                const double kf = oracle_phi(J->phi, kt[i]);
                const double* Gi = G + (size_t)i * dv;
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    acc += Gi[j] * vt[j];
                    dvt[j] += Gi[j] * kf;
                }
                dkt[i] = acc * phi_prime(J->phi, kt[i]);
            }
            for (int i = 0; i < dk; ++i) {
                const double a = gate_at(J, bh, t, i);
                double* Gi = G + (size_t)i * dv;
                if (J->gate_mode == GATE_DIAG && J->dlog_alpha) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += Gi[j] * Sp[(size_t)i * dv + j];
                    J->dlog_alpha[((size_t)bh * L + t) * dk + i] = a * acc;
                }
                if (oracle_mutation != MUT_BWD_NO_DECAY)
                    for (int j = 0; j < dv; ++j) Gi[j] *= a;
            }
        }
    }
    if (J->dS0) memcpy(J->dS0 + (size_t)bh * SS, G, sizeof(double) * SS);
    free(cp); free(S); free(blk); free(G);
}

/* ---------------------------------------------------------------------- */
/* Form 4: the delta rule ("linear_sparse_attention.py", function          */
/* delta_rule_recurrent).  The page writes S_t = S_{t-1}(I - beta_t k_t     */
/* k_t^T) + beta_t v_t k_t^T with S indexed [d_v][d_k]; in the [d_k][d_v]  */
/* orientation used everywhere here that is                                 */
/*     S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,              */
/* first erasing what the state returns for k_t, then writing v_t there.    */
/* The erase is applied as S - beta k (k^T S), the same product.  Keys are  */
/* used as given (the page's function assumes the caller normalised them). */
/* The read-out o_t = q_t^T S_t after the update follows the rest of the   */
/* pages (the page's function returns the states only).  use_delta = 0     */
/* drops the erase (additive linear attention, the page's fallback).       */
/* ---------------------------------------------------------------------- */
static void run_delta_pair(const job_t* J, int bh) {
    const int L = J->L, dk = J->dk, dv = J->dv;
    double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* u = (double*)malloc(sizeof(double) * dv);
    if (J->S0) memcpy(S, J->S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
    for (int t = 0; t < L; ++t) {
        const double* qt = J->q + ((size_t)bh * L + t) * dk;
        const double* kt = J->k + ((size_t)bh * L + t) * dk;
        const double* vt = J->v + ((size_t)bh * L + t) * dv;
        const double b = J->beta[(size_t)bh * L + t];
        const int erase = J->use_delta && oracle_mutation != MUT_DELTA_NO_ERASE;
        const int after = oracle_mutation == MUT_DELTA_ERASE_AFTER;
        if (erase && !after) {
            /* u = S^T k: what the state returns for k_t */
            for (int j = 0; j < dv; ++j) u[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) u[j] += kt[i] * S[(size_t)i * dv + j];
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] -= b * kt[i] * u[j];
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += b * kt[i] * vt[j];
        if (erase && after) {
            for (int j = 0; j < dv; ++j) u[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) u[j] += kt[i] * S[(size_t)i * dv + j];
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] -= b * kt[i] * u[j];
        }
        double* ot = J->out + ((size_t)bh * L + t) * dv;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += qt[i] * S[(size_t)i * dv + j];
            ot[j] = acc;
        }
    }
    if (J->S_final) memcpy(J->S_final + (size_t)bh * dk * dv, S, sizeof(double) * dk * dv);
    free(u);
    free(S);
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int npairs = J->B * J->H;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int bh = J->next_pair++;
        pthread_mutex_unlock(&J->mu);
        if (bh >= npairs) break;
        if (J->form == 0) run_loop_pair(J, bh);
        else if (J->form == 1) run_parallel_pair(J, bh);
        else if (J->form == 2) run_chunk_pair(J, bh);
        else if (J->form == 3) run_backward_pair(J, bh);
        else run_delta_pair(J, bh);
    }
    return NULL;
}

static int run_job(job_t* J) {
    if (J->B < 0 || J->H < 1 || J->L < 0 || J->dk < 1 || J->dv < 1) return 1;
    if (J->gate_mode == GATE_GAMMA && !J->gamma) return 1;
    if (J->gate_mode == GATE_DIAG && !J->log_alpha) return 1;
    if (J->form == 2 && J->chunk < 1) return 1;
    if (J->form == 3 && (J->normalize || J->ck < 1 || !J->dout || !J->dq || !J->dk_out || !J->dv_out))
        return 1;
    if (J->form == 4 && (!J->beta || !J->out)) return 1;
    const int npairs = J->B * J->H;
    int nt = J->nthreads < 1 ? 1 : J->nthreads;
    if (nt > npairs) nt = npairs;
    J->next_pair = 0;
    pthread_mutex_init(&J->mu, NULL);
    if (nt <= 1) {
        worker(J);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nt);
        for (int i = 0; i < nt; ++i) pthread_create(&th[i], NULL, worker, J);
        for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J->mu);
    return 0;
}

#define FILL_JOB(FORM, CHUNK, NT)                                              \
    job_t J;                                                                   \
    memset(&J, 0, sizeof J);                                                   \
    J.B = B; J.H = H; J.L = L; J.dk = dk; J.dv = dv;                           \
    J.gate_mode = gate_mode; J.gamma = gamma; J.log_alpha = log_alpha;         \
    J.phi = phi; J.normalize = normalize;                                      \
    J.q = q; J.k = k; J.v = v; J.S0 = S0; J.z0 = z0;                           \
    J.out = out; J.S_final = S_final; J.z_final = z_final;                     \
    J.form = FORM; J.chunk = CHUNK; J.nthreads = NT;

/* Token loop over every (b,h) pair; `nthreads` workers split the pairs. */
int oracle_run(int B, int H, int L, int dk, int dv, int gate_mode,
               const double* gamma, const double* log_alpha, int phi,
               int normalize, const double* q, const double* k,
               const double* v, const double* S0, const double* z0,
               double* out, double* S_final, double* z_final, int nthreads) {
    FILL_JOB(0, 0, nthreads)
    return run_job(&J);
}

/* All-pairs form; O(L^3 dk) per pair with the direct decay products, so
 * intended for tiny L only. */
int oracle_parallel(int B, int H, int L, int dk, int dv, int gate_mode,
                    const double* gamma, const double* log_alpha, int phi,
                    int normalize, const double* q, const double* k,
                    const double* v, const double* S0, const double* z0,
                    double* out, double* S_final, double* z_final) {
    FILL_JOB(1, 0, 1)
    return run_job(&J);
}

/* Chunkwise form with chunk length `chunk` (the last chunk may be shorter). */
int oracle_chunkwise(int B, int H, int L, int dk, int dv, int gate_mode,
                     const double* gamma, const double* log_alpha, int phi,
                     int normalize, const double* q, const double* k,
                     const double* v, const double* S0, const double* z0,
                     int chunk, double* out, double* S_final, double* z_final,
                     int nthreads) {
    FILL_JOB(2, chunk, nthreads)
    return run_job(&J);
}

/* Backward of the token loop: given dout (and optionally dS_final), the
 * gradients dq, dk, dv, d log_alpha (diagonal gate, may be NULL) and dS0
 * (may be NULL).  `ck` is the checkpoint spacing (any value >= 1 gives the
 * same result).  The normalised read-out is not supported (returns 1). */
int oracle_backward(int B, int H, int L, int dk, int dv, int gate_mode,
                    const double* gamma, const double* log_alpha, int phi,
                    const double* q, const double* k, const double* v,
                    const double* S0, const double* dout, const double* dS_final,
                    double* dq, double* dk_out, double* dv_out,
                    double* dlog_alpha, double* dS0, int ck, int nthreads) {
    const int normalize = 0;
    const double* z0 = NULL;
    double *out = NULL, *S_final = NULL, *z_final = NULL;
    FILL_JOB(3, 0, nthreads)
    J.dout = dout; J.dS_final = dS_final;
    J.dq = dq; J.dk_out = dk_out; J.dv_out = dv_out;
    J.dlog_alpha = dlog_alpha; J.dS0 = dS0; J.ck = ck;
    return run_job(&J);
}

/* The delta rule's token loop (form 4): out [B,H,L,dv] and S_final
 * [B,H,dk,dv] (may be NULL) from q, k [B,H,L,dk], v [B,H,L,dv], the write
 * strengths beta [B,H,L] and S0 (may be NULL).  use_delta = 0 gives the
 * additive fallback. */
int oracle_delta_run(int B, int H, int L, int dk, int dv, const double* beta,
                     const double* q, const double* k, const double* v,
                     const double* S0, double* out, double* S_final,
                     int use_delta, int nthreads) {
    const int gate_mode = GATE_NONE, phi = PHI_IDENTITY, normalize = 0;
    const double *gamma = NULL, *log_alpha = NULL, *z0 = NULL;
    double* z_final = NULL;
    FILL_JOB(4, 0, nthreads)
    J.beta = beta;
    J.use_delta = use_delta;
    return run_job(&J);
}
