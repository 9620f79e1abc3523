/*
 * oracle.c -- plain CPU oracle for the decode-step linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the GPU library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load it; the product path never does.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * Every routine is a direct, slow, sequential transcription of a definition:
 * no blocking, no vectorisation, no reordering of sums.  Accumulation is fp64 in
 * increasing k order.
 *
 * Sources (the pages are cited by title and section):
 *  - "Fast LLM inference from scratch (using CUDA)" (yalm), CPU matmul section:
 *    the matrix-vector product W (d,n) @ x (n,), row-major, out[i] = sum_j w[i*n+j]*x[j].
 *  - "How I Built an LLM Inference Engine From Scratch in CUDA" (tinyinfer), TL;DR:
 *    4-bit weights plus one fp16 scale per 64 weights.  The rounding, clamp and
 *    packing rules follow the int4-g64 workload definition used by this library:
 *    s = fp16(absmax/7) per 64 consecutive k, q = round(w/s) clamped to [-8, 7],
 *    two codes per byte along k.
 *  - "llm-rs" (roofline essay), section 5 "Batching moves decode from memory toward
 *    math": a batch of M tokens multiplies the same weights, i.e. Y = X . W^T.
 *  - yalm post, GPU matmul section (fusing): the product with the residual add
 *    accumulated into its destination, and Mistral's gated product
 *    silu(w1(x)) * w3(x) computed by the kernel that forms both products; silu
 *    is the sigmoid-weighted linear unit, silu(g) = g / (1 + exp(-g)).
 *  - "How I Built an LLM Inference Engine From Scratch in CUDA" (tinyinfer),
 *    decode section (norms folded into the projections) and the TileInfer.jl
 *    post, "Incremental acceleration" (norms fused): RMSNorm, the input of a
 *    projection divided by the root mean square of its entries and multiplied
 *    by a per-channel gain, computed by the projection kernel itself.
 *  - TileInfer.jl post, "Pushing further with cheating: INT8 quantization":
 *    symmetric INT8 in -127..127 with one Float32 scale per output channel,
 *    scale = max|w| / 127, every weight rounded to the nearest multiple of the
 *    scale; the product multiplies the INT8 values in and applies the channel's
 *    scale once at the end.
 *
 * Readings where the definition leaves a step open (each is also pinned by a test):
 *  - bf16 and fp16 are decoded from their bit definitions (IEEE-754 binary16;
 *    bfloat16 = the upper 16 bits of binary32).
 *  - Within a byte the even k sits in the low nibble, the odd k in the high nibble.
 *  - A nibble stores q as 4-bit two's complement: q = ((n ^ 8) - 8).
 *  - round(w/s) rounds half to even; w/s is formed in fp64.
 *  - The scale used to quantize is the stored fp16 value.  A group whose absmax
 *    is 0 gets s = 0 and q = 0.  A scale beyond the fp16 range saturates to the
 *    largest finite fp16 (65504); weights are assumed finite.
 *  - INT8: the stored scale is the fp32 nearest to max|w| / 127 (formed as an
 *    fp64 quotient rounded to fp32); q = round_half_even(w / s) with w / s in
 *    fp64, clamped to [-127, 127]; a row whose absmax is 0 gets s = 0, q = 0.
 *  - RMSNorm: h[k] = x[k] g[k] / sqrt(mean_k x[k]^2 + eps), evaluated in fp64
 *    and rounded once to the nearest bfloat16 (ties to even): the bf16
 *    activation that a separate normalisation would hand to the projection.
 *
 * Parity status: every function below is pinned by tests/test_oracle.py against
 * brute force, closed forms, library conversions or figures printed on the pages.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* ---- number formats ---------------------------------------------------- */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double orc_bf16_value(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double mag;
    if (e == 0xFF) {
        mag = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        mag = ldexp((double)f, -126 - 7);          /* subnormal: f * 2^-133 */
    } else {
        mag = ldexp((double)(128 + f), e - 127 - 7); /* (1 + f/128) * 2^(e-127) */
    }
    return sign ? -mag : mag;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_value(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1F;
    int f = bits & 0x3FF;
    double mag;
    if (e == 0x1F) {
        mag = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        mag = ldexp((double)f, -24);                /* subnormal: f * 2^-24 */
    } else {
        mag = ldexp((double)(1024 + f), e - 15 - 10);
    }
    return sign ? -mag : mag;
}

/* Round a non-negative value that is exact in fp64 to the nearest integer,
 * ties to even. */
static double round_half_even(double t) {
    double fl = floor(t);
    double diff = t - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Nearest binary16 to v, ties to even; overflow gives infinity. */
uint16_t orc_f16_from_f64(double v) {
    if (isnan(v)) return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a >= 65520.0) return sign | 0x7C00;        /* halfway to 2^16 and above */
    if (a < ldexp(1.0, -14)) {                     /* subnormal range, step 2^-24 */
        double q = round_half_even(ldexp(a, 24));  /* 0..1024; 1024 = min normal */
        return sign | (uint16_t)q;
    }
    int ex;
    frexp(a, &ex);                                 /* a = m * 2^ex, m in [0.5, 1) */
    int E = ex - 1;                                /* a in [2^E, 2^(E+1)) */
    double sig = round_half_even(ldexp(a, 10 - E));/* in [1024, 2048] */
    if (sig == 2048.0) { sig = 1024.0; E += 1; }
    if (E + 15 >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)sig - 1024));
}

/* Nearest bfloat16 to v, ties to even; overflow gives infinity. */
uint16_t orc_bf16_from_f64(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    /* the largest finite bf16 is (2 - 2^-7) 2^127; from halfway to 2^128 up: inf */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7F80;
    if (a < ldexp(1.0, -126)) {                    /* subnormal range, step 2^-133 */
        double q = round_half_even(ldexp(a, 133)); /* 0..128; 128 = min normal */
        return sign | (uint16_t)q;
    }
    int ex;
    frexp(a, &ex);                                 /* a = m * 2^ex, m in [0.5, 1) */
    int E = ex - 1;                                /* a in [2^E, 2^(E+1)) */
    double sig = round_half_even(ldexp(a, 7 - E)); /* in [128, 256] */
    if (sig == 256.0) { sig = 128.0; E += 1; }
    return sign | (uint16_t)(((E + 127) << 7) | ((int)sig - 128));
}

/* ---- dense product ------------------------------------------------------ */

/* Y[m][n] = sum_k W[n][k] * X[m][k] in fp64, k ascending, and the error-bound
 * term B[m][n] = sum_k |W[n][k] * X[m][k]|.
 * W: bf16 bits, row-major [N][K].  X: bf16 bits, row-major [M][K].
 * Y, B: row-major [M][N].  B may be NULL. */
void orc_gemm_dense(const uint16_t* W, const uint16_t* X, int64_t M, int64_t N,
                    int64_t K, double* Y, double* B) {
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = orc_bf16_value(W[n * K + k]) * orc_bf16_value(X[m * K + k]);
                acc += p;
                mag += fabs(p);
            }
            Y[m * N + n] = acc;
            if (B) B[m * N + n] = mag;
        }
    }
}

/* Same product with fp64 weights (used for dequantised int4 weights). */
void orc_gemm_f64w(const double* Wd, const uint16_t* X, int64_t M, int64_t N,
                   int64_t K, double* Y, double* B) {
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = Wd[n * K + k] * orc_bf16_value(X[m * K + k]);
                acc += p;
                mag += fabs(p);
            }
            Y[m * N + n] = acc;
            if (B) B[m * N + n] = mag;
        }
    }
}

/* ---- int4, one fp16 scale per 64 weights along k ------------------------ */

/* The signed code stored at position k of row n. */
static int q4_code(const uint8_t* Wq, int64_t K, int64_t n, int64_t k) {
    uint8_t byte = Wq[n * (K / 2) + k / 2];
    int nib = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    return (nib ^ 8) - 8;                          /* 4-bit two's complement */
}

/* w[n][k] = q[n][k] * s[n][k/64], exact in fp64.
 * Wq: [N][K/2] bytes, S: fp16 bits [N][K/64], Wd: [N][K]. */
void orc_dequant_q4g64(const uint8_t* Wq, const uint16_t* S, int64_t N, int64_t K,
                       double* Wd) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Wd[n * K + k] = (double)q4_code(Wq, K, n, k) * orc_f16_value(S[n * (K / 64) + k / 64]);
}

/* Y = X . deq(Wq, S)^T with the same k-ascending fp64 sum and bound term. */
void orc_gemm_q4g64(const uint8_t* Wq, const uint16_t* S, const uint16_t* X,
                    int64_t M, int64_t N, int64_t K, double* Y, double* B) {
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = (double)q4_code(Wq, K, n, k) * orc_f16_value(S[n * (K / 64) + k / 64]);
                double p = w * orc_bf16_value(X[m * K + k]);
                acc += p;
                mag += fabs(p);
            }
            Y[m * N + n] = acc;
            if (B) B[m * N + n] = mag;
        }
    }
}

/* Quantise bf16 weights W[N][K] (K a multiple of 64) to int4-g64.
 * Per row n and group g of 64 consecutive k:
 *   a = max |w|;  s = fp16 nearest to a/7 (saturated to 65504);
 *   q = s > 0 ? clamp(round_half_even(w/s), -8, 7) : 0;
 *   byte j of the row = (q[2j] & 0xF) | ((q[2j+1] & 0xF) << 4).
 * Wq: [N][K/2] bytes, S: fp16 bits [N][K/64]. */
void orc_quantize_q4g64(const uint16_t* W, int64_t N, int64_t K, uint8_t* Wq,
                        uint16_t* S) {
    int64_t G = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            double a = 0.0;
            for (int64_t k = g * 64; k < g * 64 + 64; ++k) {
                double w = fabs(orc_bf16_value(W[n * K + k]));
                if (w > a) a = w;
            }
            uint16_t sbits = orc_f16_from_f64(a / 7.0);
            if ((sbits & 0x7FFF) == 0x7C00) sbits = 0x7BFF;   /* saturate */
            S[n * G + g] = sbits;
            double s = orc_f16_value(sbits);
            for (int64_t k = g * 64; k < g * 64 + 64; k += 2) {
                int q[2];
                for (int t = 0; t < 2; ++t) {
                    double w = orc_bf16_value(W[n * K + k + t]);
                    double r = 0.0;
                    if (s > 0.0) {
                        double v = w / s;
                        r = (v < 0.0) ? -round_half_even(-v) : round_half_even(v);
                        if (r < -8.0) r = -8.0;
                        if (r > 7.0) r = 7.0;
                    }
                    q[t] = (int)r;
                }
                Wq[n * (K / 2) + k / 2] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
            }
        }
    }
}

/* ---- int8, one fp32 scale per output channel ---------------------------- */

/* Quantise bf16 weights W[N][K] to int8 with one fp32 scale per row n:
 *   a = max_k |w|;  s = fp32 nearest to a/127;
 *   q = s > 0 ? clamp(round_half_even(w/s), -127, 127) : 0.
 * Wq: int8 [N][K], S: fp32 [N]. */
void orc_quantize_i8(const uint16_t* W, int64_t N, int64_t K, int8_t* Wq, float* S) {
    for (int64_t n = 0; n < N; ++n) {
        double a = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double w = fabs(orc_bf16_value(W[n * K + k]));
            if (w > a) a = w;
        }
        float s = (float)(a / 127.0);
        S[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            double r = 0.0;
            if (s > 0.0f) {
                double v = orc_bf16_value(W[n * K + k]) / (double)s;
                r = (v < 0.0) ? -round_half_even(-v) : round_half_even(v);
                if (r < -127.0) r = -127.0;
                if (r > 127.0) r = 127.0;
            }
            Wq[n * K + k] = (int8_t)r;
        }
    }
}

/* w[n][k] = q[n][k] * s[n], exact in fp64.  Wd: [N][K]. */
void orc_dequant_i8(const int8_t* Wq, const float* S, int64_t N, int64_t K, double* Wd) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) Wd[n * K + k] = (double)Wq[n * K + k] * (double)S[n];
}

/* Y[m][n] = s[n] * sum_k q[n][k] * X[m][k]: the integer weights multiply in
 * (fp64, k ascending) and the channel scale is applied once at the end.
 * B[m][n] = sum_k |q[n][k] * s[n] * X[m][k]|.  B may be NULL. */
void orc_gemm_i8(const int8_t* Wq, const float* S, const uint16_t* X, int64_t M, int64_t N,
                 int64_t K, double* Y, double* B) {
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)Wq[n * K + k] * orc_bf16_value(X[m * K + k]);
                acc += p;
                mag += fabs(p);
            }
            Y[m * N + n] = (double)S[n] * acc;
            if (B) B[m * N + n] = fabs((double)S[n]) * mag;
        }
    }
}

/* ---- fused epilogues ------------------------------------------------------ */

/* H[i] = silu(G[i]) * U[i] with silu(g) = g / (1 + exp(-g)), in fp64. */
void orc_swiglu(const double* G, const double* U, int64_t n, double* H) {
    for (int64_t i = 0; i < n; ++i) H[i] = G[i] / (1.0 + exp(-G[i])) * U[i];
}

/* Y[i] = P[i] + R[i]: a product plus the residual it is accumulated into. */
void orc_residual_add(const double* P, const float* R, int64_t n, double* Y) {
    for (int64_t i = 0; i < n; ++i) Y[i] = P[i] + (double)R[i];
}

/* ---- RMSNorm prologue ----------------------------------------------------- */

/* H[m][k] = bf16(X[m][k] * G[k] / sqrt(sum_k X[m][k]^2 / K + eps)) for each
 * token row m: the sum of squares in fp64, k ascending, one rounding to
 * bfloat16 at the end.  X, H: bf16 [M][K]; G: bf16 [K]; K >= 1. */
void orc_rmsnorm(const uint16_t* X, const uint16_t* G, int64_t M, int64_t K, double eps,
                 uint16_t* H) {
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double x = orc_bf16_value(X[m * K + k]);
            ss += x * x;
        }
        double inv = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            H[m * K + k] = orc_bf16_from_f64(orc_bf16_value(X[m * K + k]) *
                                             orc_bf16_value(G[k]) * inv);
    }
}
