/*
 * Plain fp64 CPU oracle for one tensor-parallel rank's share of a
 * Megatron-style transformer layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The product path never
 * calls it, and it shares no code, header or table with the HIP library.
 *
 * What it computes (every function is the plain definition, no blocking,
 * no reordering of sums):
 *   - "Tensor vs Pipeline Parallelism" (xingyuzhitong.com), section "Tensor
 *     parallelism: split inside each layer": the MLP's leading matrix is cut
 *     along output columns and its trailing matrix along input rows; the
 *     ranks' partial products are then added.
 *   - "AI Infrastructure series, Part 5" (drpranayjha.com), section "How does
 *     tensor parallelism split a layer?": the same column-then-row cut in
 *     every block, so a rank stores and streams 1/N of each matrix.
 *   - "Tensor Parallelism" glossary (aidolsgroup.com), "Full definition":
 *     every rank sees the same input; the partial products are added.
 *   - Same page series, "Short answers": splitting computes the same maths;
 *     only the order of additions changes the last digits. The oracle
 *     therefore sums every dot product in ascending k, in fp64.
 *
 * Numbers are bf16 bit patterns (uint16_t) on input. Arithmetic is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* bf16 -> fp64. A bf16 value is the upper 16 bits of a binary32 value. */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * fp64 -> bf16, round to nearest, ties to even, straight from fp64 (one
 * rounding). bf16 has 8 significant bits and the exponent range of binary32:
 * normal values down to 2^-126, subnormals in steps of 2^-133, largest finite
 * value (2 - 2^-7) * 2^127. Values that round above it become infinity.
 */
uint16_t orc_f64_to_bf16(double x) {
  if (isnan(x)) return (uint16_t)0x7FC0;
  uint16_t sign = signbit(x) ? (uint16_t)0x8000 : (uint16_t)0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  int e;
  (void)frexp(a, &e);           /* a = f * 2^e, 0.5 <= f < 1: top bit is 2^(e-1) */
  int q = e - 8;                /* quantum (ulp) exponent for 8 significant bits */
  if (q < -133) q = -133;       /* subnormal range: fixed quantum 2^-133 */
  double r = nearbyint(ldexp(a, -q)); /* exact scaling; default mode = ties to even */
  double v = ldexp(r, q);
  const double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  if (v > max_finite) return (uint16_t)(sign | 0x7F80);
  float f = (float)v;           /* exact: v is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

void orc_round_bf16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(x[i]);
}

void orc_bf16_to_f64_array(const uint16_t* b, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(b[i]);
}

/*
 * The local product of one shard, with the shard given by index lists into
 * the full weight:
 *   Y[m][j] = sum_{kk = 0 .. Kr-1} X[m][kk] * W[rows[kk]][cols[j]]
 * X is [M x Kr] row-major with leading dimension ldx (bf16 bits), W is the
 * full logical weight, [K_full x N_full] row-major with leading dimension ldw
 * (bf16 bits), Y is [M x Nc] fp64 row-major. Each output has one fp64
 * accumulator and kk runs in ascending order.
 *
 * A column shard is rows = 0..K-1, cols = the rank's columns; a row shard is
 * rows = the rank's rows, cols = 0..N-1, with X the rank's input slice.
 */
void orc_shard_matmul(const uint16_t* X, int64_t M, int64_t ldx, int64_t Kr,
                      const uint16_t* W, int64_t ldw, const int64_t* rows,
                      const int64_t* cols, int64_t Nc, double* Y) {
  /* Work split over threads only (each output is still one in-order sum):
   * tasks of CH columns of one row, all rows of a column stripe before the
   * next stripe, so threads working at the same time read the same stripe
   * of W from the host's caches. */
  const int64_t CH = 256;
  int64_t nch = (Nc + CH - 1) / CH;
  int64_t ntask = M * nch;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < ntask; ++task) {
    int64_t m = task % M;
    int64_t j0 = (task / M) * CH;
    int64_t j1 = j0 + CH < Nc ? j0 + CH : Nc;
    double* y = Y + m * Nc;
    for (int64_t j = j0; j < j1; ++j) y[j] = 0.0;
    for (int64_t kk = 0; kk < Kr; ++kk) {
      double x = orc_bf16_to_f64(X[m * ldx + kk]);
      const uint16_t* w = W + rows[kk] * ldw;
      for (int64_t j = j0; j < j1; ++j) y[j] += x * orc_bf16_to_f64(w[cols[j]]);
    }
  }
}

/*
 * SwiGLU of one rank's gate and up outputs: H = bf16_RNE(SiLU(G) * U),
 * SiLU(g) = g / (1 + e^-g), applied to the gate. For g -> -inf this gives
 * -0 (e^-g = inf), for g -> +inf it gives g.
 */
void orc_swiglu(const double* G, const double* U, int64_t n, uint16_t* H) {
  for (int64_t i = 0; i < n; ++i) {
    double g = G[i];
    double s = g / (1.0 + exp(-g));
    H[i] = orc_f64_to_bf16(s * U[i]);
  }
}

/*
 * Sum of t partial outputs, in rank order 0, 1, ..., t-1:
 *   Y[i] = (((0 + P_0[i]) + P_1[i]) + ...) + P_{t-1}[i]
 * P_r starts at P + r * stride.
 */
void orc_sum_partials(const double* P, int64_t stride, int32_t t, int64_t n, double* Y) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int32_t r = 0; r < t; ++r) s += P[(int64_t)r * stride + i];
    Y[i] = s;
  }
}

/*
 * The same product on fp64 operands (dequantised 8-bit weights, gradients,
 * attention scores and probabilities):
 *   C[m][n] = sum_{k = 0 .. K-1} A(m, k) * B(k, n)
 * with A(m, k) = A[m * sam + k * sak] and B(k, n) = B[k * sbk + n * sbn]
 * (element strides, so a transposed operand is read in place). C is [M x N]
 * row-major. One fp64 accumulator per output, k ascending, no blocking: the
 * plain definition, exactly as orc_shard_matmul sums.
 */
void orc_matmul_f64(const double* A, int64_t M, int64_t K, int64_t sam, int64_t sak,
                    const double* B, int64_t N, int64_t sbk, int64_t sbn, double* C) {
  const int64_t CH = 256; /* work split only, as in orc_shard_matmul */
  int64_t nch = (N + CH - 1) / CH;
  int64_t ntask = M * nch;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < ntask; ++task) {
    int64_t m = task % M;
    int64_t j0 = (task / M) * CH;
    int64_t j1 = j0 + CH < N ? j0 + CH : N;
    double* y = C + m * N;
    for (int64_t j = j0; j < j1; ++j) y[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double a = A[m * sam + k * sak];
      const double* b = B + k * sbk;
      for (int64_t j = j0; j < j1; ++j) y[j] += a * b[j * sbn];
    }
  }
}
