/*
 * CPU oracle for the selective state-space scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, sequential, float64.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this; the GPU library neither links
 * nor calls it and shares no code, header or table with it.
 *
 * Sources (pages, by title and section):
 *  [TP]  "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습"
 *        §2.1  selective-scan recurrence h_t = Ā_t h_{t-1} + B̄_t x_t, with
 *              input-dependent B, C and Δ, strictly sequential in t;
 *        §3.1  Mamba-2 restricts the state matrix to a scalar times identity,
 *              A_t = a_t I, so all N state rows of a head share one decay;
 *        §4.3  a zero transition (A_t = 0) forgets the previous state.
 *  [INF] "Scaling State-Space Models on Multiple GPUs with Tensor Parallelism",
 *        Abstract: an SSM state cache carried from prefill into decode.
 *
 * The pages leave Ā and B̄ undefined.  Reading used here: Ā = exp(Δ·A),
 * B̄ = Δ·B, the output y_t = C_tᵀ h_t + D·x_t reads the state after token t's
 * own update, and Δ = softplus(raw) when the caller asks for it.
 *
 * Every function here is the definition written out: one time step after
 * another, no chunking, no reordering.  OpenMP only splits independent
 * sequences (batch row x head, or batch row x channel block).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(r) = log(1 + e^r), written so that neither branch overflows. */
static double softplus(double r)
{
    return r > 0.0 ? r + log1p(exp(-r)) : log1p(exp(r));
}

int oracle_version(void) { return 1; }

/* Number of threads a parallel region here uses (1 without OpenMP). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Mamba-2 SSD scan over a whole sequence ([TP] §2.1 with the scalar-identity
 * state matrix of §3.1).  For every batch row b and head h, with group
 * g = h / (nheads/ngroups) and the N x P state S (S = h0 or 0 before t = 0):
 *     Δ_t      = softplus(dt[b,t,h])  (or dt itself)
 *     S       <- exp(Δ_t·A[h]) · S + Δ_t · B[b,t,g,:] x[b,t,h,:]ᵀ
 *     y[b,t,h] = Sᵀ C[b,t,g,:] + D[h] · x[b,t,h,:]
 * Layouts (row-major): x, y [b][L][H][P]; dt [b][L][H]; B, C [b][L][G][N];
 * A, D [H]; h0, hfinal [b][H][N][P].  D, h0 and hfinal may be NULL.
 */
void oracle_ssd_scan(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                     int dt_softplus, const double *x, const double *dt, const double *A,
                     const double *B, const double *C, const double *D, const double *h0,
                     double *y, double *hfinal)
{
    const int P = headdim, N = dstate, H = nheads, G = ngroups, L = seqlen;
    const int R = H / G;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < H; ++h) {
            const int g = h / R;
            double *S = (double *)malloc(sizeof(double) * (size_t)N * P);
            double *acc = (double *)malloc(sizeof(double) * (size_t)P);
            const size_t soff = ((size_t)b * H + h) * (size_t)N * P;
            if (h0)
                memcpy(S, h0 + soff, sizeof(double) * (size_t)N * P);
            else
                memset(S, 0, sizeof(double) * (size_t)N * P);
            for (int t = 0; t < L; ++t) {
                const size_t row = (size_t)b * L + t;
                const double *xt = x + (row * H + h) * P;
                const double *Bt = B + (row * G + g) * N;
                const double *Ct = C + (row * G + g) * N;
                const double raw = dt[row * H + h];
                const double delta = dt_softplus ? softplus(raw) : raw;
                const double a = exp(delta * A[h]);
                for (int n = 0; n < N; ++n) {
                    const double coef = delta * Bt[n];
                    double *Sn = S + (size_t)n * P;
                    for (int p = 0; p < P; ++p)
                        Sn[p] = a * Sn[p] + coef * xt[p];
                }
                const double d = D ? D[h] : 0.0;
                for (int p = 0; p < P; ++p)
                    acc[p] = d * xt[p];
                for (int n = 0; n < N; ++n) {
                    const double cn = Ct[n];
                    const double *Sn = S + (size_t)n * P;
                    for (int p = 0; p < P; ++p)
                        acc[p] += cn * Sn[p];
                }
                memcpy(y + (row * H + h) * P, acc, sizeof(double) * P);
            }
            if (hfinal)
                memcpy(hfinal + soff, S, sizeof(double) * (size_t)N * P);
            free(acc);
            free(S);
        }
    }
}

/*
 * Gradient of the SSD scan above (reverse-mode, the chain rule taken one time
 * step at a time).  The forward states h_t of one (b, h) are kept, then the
 * adjoint g = dL/dh_t runs backwards from g = dL/dh_final (or 0):
 *     g      += C_t dy_tᵀ                      (y_t reads h_t)
 *     dC_t   += h_tᵀ-contract dy_t = Σ_p h_t[n,p] dy_t[p]
 *     dD     += x_t · dy_t;       dx_t = D·dy_t + Δ_t Σ_n B_t[n] g[n,:]
 *     dB_t   += Δ_t Σ_p g[n,p] x_t[p]
 *     dΔ_t    = Σ g[n,p] B_t[n] x_t[p]  +  A·a_t·Σ g[n,p] h_{t-1}[n,p]
 *     dA     += Δ_t·a_t·Σ g h_{t-1};     ddt_t = dΔ_t·σ(raw) when Δ = softplus(raw)
 *     g       = a_t·g                          (h_t = a_t h_{t-1} + Δ_t B_t x_tᵀ)
 * and dh0 = g after t = 0.  dB and dC are returned per head, [b][L][H][N]
 * (the caller sums the heads of a group); dA, dD are [b][H] per batch row.
 * dy [b][L][H][P]; dhfinal [b][H][N][P] or NULL; every output is written.
 */
void oracle_ssd_scan_bwd(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                         int dt_softplus, const double *x, const double *dt, const double *A,
                         const double *B, const double *C, const double *D, const double *h0,
                         const double *dy, const double *dhfinal, double *dx, double *ddt,
                         double *dA, double *dB_head, double *dC_head, double *dD, double *dh0)
{
    const int P = headdim, N = dstate, H = nheads, G = ngroups, L = seqlen;
    const int R = H / G;
    const size_t NP = (size_t)N * P;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < H; ++h) {
            const int g = h / R;
            const size_t soff = ((size_t)b * H + h) * NP;
            /* hs[t+1] = state after token t; hs[0] = state before the sequence */
            double *hs = (double *)malloc(sizeof(double) * NP * (size_t)(L + 1));
            double *adj = (double *)malloc(sizeof(double) * NP);
            if (h0)
                memcpy(hs, h0 + soff, sizeof(double) * NP);
            else
                memset(hs, 0, sizeof(double) * NP);
            for (int t = 0; t < L; ++t) {
                const size_t row = (size_t)b * L + t;
                const double *xt = x + (row * H + h) * P;
                const double *Bt = B + (row * G + g) * N;
                const double raw = dt[row * H + h];
                const double delta = dt_softplus ? softplus(raw) : raw;
                const double a = exp(delta * A[h]);
                const double *prev = hs + (size_t)t * NP;
                double *cur = hs + (size_t)(t + 1) * NP;
                for (int n = 0; n < N; ++n)
                    for (int p = 0; p < P; ++p)
                        cur[(size_t)n * P + p] = a * prev[(size_t)n * P + p] + delta * Bt[n] * xt[p];
            }
            if (dhfinal)
                memcpy(adj, dhfinal + soff, sizeof(double) * NP);
            else
                memset(adj, 0, sizeof(double) * NP);
            double dA_acc = 0.0, dD_acc = 0.0;
            const double Dh = D ? D[h] : 0.0;
            for (int t = L - 1; t >= 0; --t) {
                const size_t row = (size_t)b * L + t;
                const double *xt = x + (row * H + h) * P;
                const double *dyt = dy + (row * H + h) * P;
                const double *Bt = B + (row * G + g) * N;
                const double *Ct = C + (row * G + g) * N;
                const double raw = dt[row * H + h];
                const double delta = dt_softplus ? softplus(raw) : raw;
                const double a = exp(delta * A[h]);
                const double *ht = hs + (size_t)(t + 1) * NP;
                const double *hprev = hs + (size_t)t * NP;
                double *dxt = dx + (row * H + h) * P;
                double *dBt = dB_head + (row * H + h) * N;
                double *dCt = dC_head + (row * H + h) * N;
                /* output read: y_t = h_tᵀ C_t + D x_t */
                for (int n = 0; n < N; ++n) {
                    double s = 0.0;
                    for (int p = 0; p < P; ++p) {
                        adj[(size_t)n * P + p] += Ct[n] * dyt[p];
                        s += ht[(size_t)n * P + p] * dyt[p];
                    }
                    dCt[n] = s;
                }
                for (int p = 0; p < P; ++p) {
                    dD_acc += xt[p] * dyt[p];
                    dxt[p] = Dh * dyt[p];
                }
                /* state update: h_t = a h_{t-1} + Δ B_t x_tᵀ */
                double gin = 0.0, gprev = 0.0;
                for (int n = 0; n < N; ++n) {
                    double sb = 0.0;
                    for (int p = 0; p < P; ++p) {
                        const double gv = adj[(size_t)n * P + p];
                        dxt[p] += delta * Bt[n] * gv;
                        sb += gv * xt[p];
                        gprev += gv * hprev[(size_t)n * P + p];
                    }
                    dBt[n] = delta * sb;
                    gin += Bt[n] * sb;
                }
                const double ddelta = gin + A[h] * a * gprev;
                dA_acc += delta * a * gprev;
                ddt[row * H + h] = dt_softplus ? ddelta / (1.0 + exp(-raw)) : ddelta;
                for (size_t i = 0; i < NP; ++i)
                    adj[i] *= a;
            }
            dA[(size_t)b * H + h] = dA_acc;
            dD[(size_t)b * H + h] = dD_acc;
            if (dh0)
                memcpy(dh0 + soff, adj, sizeof(double) * NP);
            free(adj);
            free(hs);
        }
    }
}

/*
 * One decode step against a cached state ([INF] Abstract: the state cache
 * carried from prefill into decode; the update is the same single step of
 * [TP] §2.1 as above).  state [b][H][N][P] is read and overwritten;
 * x, y [b][H][P]; dt [b][H]; B, C [b][G][N].
 */
void oracle_ssd_decode(int batch, int nheads, int headdim, int dstate, int ngroups,
                       int dt_softplus, const double *x, const double *dt, const double *A,
                       const double *B, const double *C, const double *D, double *state,
                       double *y)
{
    const int P = headdim, N = dstate, H = nheads, G = ngroups;
    const int R = H / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < H; ++h) {
            const int g = h / R;
            const double *xt = x + ((size_t)b * H + h) * P;
            const double *Bt = B + ((size_t)b * G + g) * N;
            const double *Ct = C + ((size_t)b * G + g) * N;
            double *S = state + ((size_t)b * H + h) * (size_t)N * P;
            double *yt = y + ((size_t)b * H + h) * P;
            const double raw = dt[(size_t)b * H + h];
            const double delta = dt_softplus ? softplus(raw) : raw;
            const double a = exp(delta * A[h]);
            for (int n = 0; n < N; ++n) {
                const double coef = delta * Bt[n];
                for (int p = 0; p < P; ++p)
                    S[(size_t)n * P + p] = a * S[(size_t)n * P + p] + coef * xt[p];
            }
            const double d = D ? D[h] : 0.0;
            for (int p = 0; p < P; ++p)
                yt[p] = d * xt[p];
            for (int n = 0; n < N; ++n)
                for (int p = 0; p < P; ++p)
                    yt[p] += Ct[n] * S[(size_t)n * P + p];
        }
    }
}

/*
 * Mamba-1 selective scan with a diagonal state matrix per channel ([TP] §2.1:
 * input-dependent B, C, Δ; one recurrence per channel).  For batch row b and
 * channel d, with an N-vector state s (zero before t = 0):
 *     Δ      = softplus(delta[b,t,d])  (or delta itself)
 *     s[n]  <- exp(Δ·A[d,n]) · s[n] + Δ · B[b,t,n] · u[b,t,d]
 *     y      = Σ_n C[b,t,n] s[n] + Dk[d] · u[b,t,d]
 *     out    = y · z · sigmoid(z)     with z = z[b,t,d]   (no gate if z == NULL)
 * Layouts: u, delta, z, out [b][L][dim]; A [dim][N]; B, C [b][L][N]; Dk [dim];
 * hfinal [b][dim][N].  Dk, z and hfinal may be NULL.
 * Channels are processed in blocks of 64 with t as the outer loop, which is
 * the same arithmetic per channel in a cache-friendly order.
 */
void oracle_selective_scan(int batch, int seqlen, int dim, int dstate, int delta_softplus,
                           const double *u, const double *delta, const double *A,
                           const double *B, const double *C, const double *Dk, const double *z,
                           double *out, double *hfinal)
{
    const int L = seqlen, N = dstate;
    const int DB = 64;
    const int nblk = (dim + DB - 1) / DB;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        for (int blk = 0; blk < nblk; ++blk) {
            const int d0 = blk * DB;
            const int d1 = d0 + DB < dim ? d0 + DB : dim;
            double *s = (double *)calloc((size_t)DB * N, sizeof(double));
            for (int t = 0; t < L; ++t) {
                const size_t row = (size_t)b * L + t;
                const double *Bt = B + row * N;
                const double *Ct = C + row * N;
                for (int d = d0; d < d1; ++d) {
                    double *sd = s + (size_t)(d - d0) * N;
                    const double ut = u[row * dim + d];
                    const double raw = delta[row * dim + d];
                    const double dl = delta_softplus ? softplus(raw) : raw;
                    double yv = Dk ? Dk[d] * ut : 0.0;
                    for (int n = 0; n < N; ++n) {
                        sd[n] = exp(dl * A[(size_t)d * N + n]) * sd[n] + dl * Bt[n] * ut;
                        yv += Ct[n] * sd[n];
                    }
                    if (z) {
                        const double zt = z[row * dim + d];
                        yv *= zt / (1.0 + exp(-zt));
                    }
                    out[row * dim + d] = yv;
                }
            }
            if (hfinal)
                for (int d = d0; d < d1; ++d)
                    memcpy(hfinal + ((size_t)b * dim + d) * N, s + (size_t)(d - d0) * N,
                           sizeof(double) * N);
            free(s);
        }
    }
}

/*
 * Causal depthwise 1-D convolution of the inner activations ([TP] §2.2: the
 * SSM inputs come out of a 1-D convolution and an activation).  For batch row
 * b, channel c and time t, with window width W:
 *     v = bias[c] + Σ_{k=0}^{W-1} w[c][k]·u(t - (W-1) + k),   y = silu(v) or v
 * where u(s) = x[b][s][c] for s >= 0 and, for s < 0, the carried state
 * state0[b][W-1+s][c] (zero without one).  The final state holds the last
 * W-1 inputs, u(L-W+1) .. u(L-1), oldest first.
 */
void oracle_causal_conv1d(int batch, int seqlen, int channels, int width, int apply_silu,
                          const double *x, const double *w, const double *bias,
                          const double *state0, double *y, double *state_out)
{
    const int W1 = width - 1;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) collapse(2)
#endif
    for (int b = 0; b < batch; ++b)
        for (int c = 0; c < channels; ++c) {
            for (int t = 0; t < seqlen; ++t) {
                double v = bias ? bias[c] : 0.0;
                for (int k = 0; k < width; ++k) {
                    const int s = t - W1 + k;
                    double u = 0.0;
                    if (s >= 0)
                        u = x[((size_t)b * seqlen + s) * channels + c];
                    else if (state0)
                        u = state0[((size_t)b * W1 + (W1 + s)) * channels + c];
                    v += w[(size_t)c * width + k] * u;
                }
                y[((size_t)b * seqlen + t) * channels + c] = apply_silu ? v / (1.0 + exp(-v)) : v;
            }
            if (state_out)
                for (int r = 0; r < W1; ++r) {
                    const int s = seqlen - W1 + r;
                    double u = 0.0;
                    if (s >= 0)
                        u = x[((size_t)b * seqlen + s) * channels + c];
                    else if (state0)
                        u = state0[((size_t)b * W1 + (W1 + s)) * channels + c];
                    state_out[((size_t)b * W1 + r) * channels + c] = u;
                }
        }
}

/*
 * Gated grouped RMS normalisation of the scan output ([TP] §4.1: the norm
 * runs over groups of channels, so each group's statistics stay local).  For
 * row r, the channels split into G contiguous groups of channels/G; with
 * g = y·silu(z) (g = y without z):
 *     out[c] = g[c] / sqrt(mean over c's group of g² + eps) · weight[c]
 */
void oracle_gated_rmsnorm(int rows, int channels, int ngroups, double eps, const double *y,
                          const double *z, const double *weight, double *out)
{
    const int cg = channels / ngroups;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) collapse(2)
#endif
    for (int r = 0; r < rows; ++r)
        for (int gi = 0; gi < ngroups; ++gi) {
            const size_t base = (size_t)r * channels + (size_t)gi * cg;
            double ss = 0.0;
            for (int c = 0; c < cg; ++c) {
                double g = y[base + c];
                if (z) g *= z[base + c] / (1.0 + exp(-z[base + c]));
                ss += g * g;
            }
            const double inv = 1.0 / sqrt(ss / cg + eps);
            for (int c = 0; c < cg; ++c) {
                double g = y[base + c];
                if (z) g *= z[base + c] / (1.0 + exp(-z[base + c]));
                out[base + c] = g * inv * weight[(size_t)gi * cg + c];
            }
        }
}
