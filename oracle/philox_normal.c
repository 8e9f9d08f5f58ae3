/*
 * Oracle (test infrastructure only): counter-based random streams.
 *
 * Only tests/, the smoke check and the bench's CPU-baseline leg may load this
 * file's library. It is the CPU side of the random-number specification that
 * the GPU path implements independently; the two share no code.
 *
 * Philox4x32-10 follows its published definition (Salmon, Moraes, Dror and
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds of
 * two 32x32->64-bit products, with the key bumped by the Weyl constants
 * between rounds.  The pages ("Zeroth-Order Fine-Tuning Was an Inference
 * Workload All Along", section "The System Reorganization") only require that
 * the random-direction stream is a fixed function of its seed; the generator
 * choice is ours.
 *
 * Gaussian transform: Box-Muller (1958) written with IEEE-754 binary64 +, -,
 * *, / and sqrt only, each correctly rounded, in a fixed order, with no fused
 * multiply-add.  ln uses an exact frexp split and the atanh series, sin and
 * cos use nested Taylor forms.  Any other implementation that performs the
 * same operations in the same order gets the same bits.
 *
 * Build with: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 */
#include <stdint.h>
#include <math.h>

/* ---- Philox4x32-10 ---------------------------------------------------- */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ---- exact-operation elementary functions ------------------------------ */
/* ln 2 split so that e*LN2_HI is exact for |e| < 2^20 (low 21 bits zero). */
static const double LN2_HI = 0x1.62e42fee00000p-1;
static const double LN2_LO = 0x1.a39ef35793c76p-33;
static const double SQRT_HALF = 0x1.6a09e667f3bcdp-1;
static const double PI_OVER_4 = 0x1.921fb54442d18p-1;

/* natural log of u in (0, 1]: u = m * 2^e with m in [sqrt(1/2), sqrt(2)),
   ln m = 2 atanh(s), s = (m-1)/(m+1), atanh(s) = s * sum_k s^(2k) / (2k+1). */
double oracle_ln(double u)
{
    int e;
    double m = frexp(u, &e);          /* exact: m in [0.5, 1) */
    if (m < SQRT_HALF) { m = m * 2.0; e = e - 1; }
    double s = (m - 1.0) / (m + 1.0);
    double s2 = s * s;
    double p = 1.0 / 23.0;
    for (int k = 10; k >= 0; --k) {
        double t = p * s2;
        p = t + 1.0 / (double)(2 * k + 1);
    }
    double sp = s * p;
    double lnm = sp + sp;
    double ed = (double)e;
    double lo = ed * LN2_LO;
    double hi = ed * LN2_HI;
    return hi + (lo + lnm);
}

/* sin and cos of phi in [0, pi/4] by nested Taylor forms:
   sin x = x (1 - x^2/(2*3) (1 - x^2/(4*5) (1 - ...)))  through x^21
   cos x = 1 - x^2/(1*2) (1 - x^2/(3*4) (1 - ...))      through x^22 */
double oracle_sin_q(double x)
{
    double x2 = x * x;
    double p = 1.0;
    for (int k = 10; k >= 1; --k) {
        double r = 1.0 / (double)((2 * k) * (2 * k + 1));
        double t = x2 * r;
        double tp = t * p;
        p = 1.0 - tp;
    }
    return x * p;
}

double oracle_cos_q(double x)
{
    double x2 = x * x;
    double p = 1.0;
    for (int k = 11; k >= 1; --k) {
        double r = 1.0 / (double)((2 * k - 1) * (2 * k));
        double t = x2 * r;
        double tp = t * p;
        p = 1.0 - tp;
    }
    return p;
}

/* One Box-Muller pair from a radius word wa and an angle word wb.
   u = (wa + 1/2) 2^-32 in (0,1); R = sqrt(-2 ln u).
   Angle: quadrant = top 2 bits of wb, half-quadrant bit h = bit 29,
   f = (low 29 bits + 1/2) 2^-29, phi = f * pi/4.
   h = 0: psi = phi;  h = 1: psi = pi/2 - phi  (cos and sin swap).
   theta = quadrant * pi/2 + psi, applied as exact sign flips and swaps. */
void oracle_box_muller(uint32_t wa, uint32_t wb, double* za, double* zb)
{
    double u = ((double)wa + 0.5) * 0x1p-32;
    double l = oracle_ln(u);
    double m2 = -2.0 * l;
    double R = sqrt(m2);
    uint32_t quad = wb >> 30;
    uint32_t h = (wb >> 29) & 1u;
    double f = ((double)(wb & 0x1FFFFFFFu) + 0.5) * 0x1p-29;
    double phi = f * PI_OVER_4;
    double c = oracle_cos_q(phi), s = oracle_sin_q(phi);
    double cp = h ? s : c;   /* cos psi */
    double sp = h ? c : s;   /* sin psi */
    double ct, st;
    switch (quad) {
        case 0: ct = cp;  st = sp;  break;
        case 1: ct = -sp; st = cp;  break;
        case 2: ct = -cp; st = -sp; break;
        default: ct = sp; st = -cp; break;
    }
    *za = R * ct;
    *zb = R * st;
}

/* Element e of a stream keyed by (seed, tag, tau) is lane e%4 of the Philox
   block with counter (e/4, tag, lo32(tau), hi32(tau)) and key (lo32(seed),
   hi32(seed)); lanes (0,1) and (2,3) form the two Box-Muller pairs. */
void oracle_normal_fill(uint64_t seed, uint32_t tag, uint64_t tau,
                        int64_t first, int64_t n, double* out)
{
    const uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int64_t e = first + i;
        uint32_t ctr[4] = { (uint32_t)(e >> 2), tag, (uint32_t)tau, (uint32_t)(tau >> 32) };
        uint32_t w[4];
        oracle_philox4x32_10(ctr, key, w);
        double z[4];
        oracle_box_muller(w[0], w[1], &z[0], &z[1]);
        oracle_box_muller(w[2], w[3], &z[2], &z[3]);
        out[i] = z[e & 3];
    }
}

/* Raw words of the same stream, for the bit-exact checks. */
void oracle_words_fill(uint64_t seed, uint32_t tag, uint64_t tau,
                       int64_t first_block, int64_t n_blocks, uint32_t* out)
{
    const uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < n_blocks; ++b) {
        int64_t j = first_block + b;
        uint32_t ctr[4] = { (uint32_t)j, tag, (uint32_t)tau, (uint32_t)(tau >> 32) };
        oracle_philox4x32_10(ctr, key, out + 4 * b);
    }
}

/* Elementwise wrappers used by the pins. */
void oracle_ln_array(const double* u, double* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_ln(u[i]); }
void oracle_sincos_array(const double* x, double* s, double* c, int64_t n)
{ for (int64_t i = 0; i < n; ++i) { s[i] = oracle_sin_q(x[i]); c[i] = oracle_cos_q(x[i]); } }
void oracle_box_muller_array(const uint32_t* wa, const uint32_t* wb, double* za, double* zb, int64_t n)
{ for (int64_t i = 0; i < n; ++i) oracle_box_muller(wa[i], wb[i], &za[i], &zb[i]); }
void oracle_philox_array(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) oracle_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i); }
