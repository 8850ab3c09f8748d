// Oracle in plain C++17 + OpenMP -- TEST INFRASTRUCTURE ONLY.
//
// A second, independently written CPU implementation of what the GPU library
// computes, from "Full-Stack FP4: Stable LLM Pretraining with Quantized
// Projections, Optimizers, and Attention" (arXiv 2607.04422):
//   * the NVFP4 format of §2 ("Preliminaries", paragraph "NVFP4 format"):
//     E2M1 element codes, one FP8 E4M3 scale per 16-element block, one FP32
//     scale per tensor, value = x_E2M1 * s * s_g;
//   * the NVFP4 Newton-Schulz iteration of §3.4 ("NVFP4 Root Optimizer"):
//     per step qX = Q_1x16(X), qX16 = Q_16x1(X), A = qX qX^T, qA = Q_1x16(A),
//     B = b A + c qA qA16, qB = Q_1x16(B), X' = a X + qB qX16, every
//     quantization round-to-nearest.
// Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
// load it; the GPU library neither calls it nor shares code with it.
//
// Readings of the pages (the same ones the numpy oracle and the GPU take):
//   s_g = RN_f32(amax / 2688); s = RNE_E4M3FN(amax_b / (6 s_g)) of the exact
//   quotient, saturating at 448, 0 at or below 2^-10; the element magnitude
//   is RNE_E2M1(|x| / (s s_g)) of the exact quotient (ties to the even code,
//   saturating at 6, 0 when s or s_g is 0), the sign bit is that of x; any
//   NaN or infinity makes amax NaN, then s_g is NaN, every scale byte 0x7F
//   and every magnitude 0.  Element 2i goes to the low nibble of byte i;
//   scales are one byte per block, row-major.  Q_16x1(T) is Q_1x16(T^T) in
//   the layout of T^T.  X_0 = clamp(G, +-clip) / (||clamp(G)||_F + 1e-7),
//   on G^T when m > n.  b A and a X use the unquantized A and X.
//
// Exactness.  No division decides a code: the E4M3 midpoints times 6 s_g
// and the E2M1 midpoints times s s_g are exact in double (at most 31
// significant bits), so each code is a count of exact comparisons.  s_g is
// one double division rounded to float: double carries 53 >= 2 * 24 + 2
// bits, so rounding the double quotient to float equals rounding the exact
// quotient.  Products of dequantized values are exact in double; their
// sums (the GEMMs) accumulate in double.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <vector>

#include <omp.h>

namespace {

// ---- E4M3FN (OCP FP8, bias 7, no infinity, 0x7F = NaN, max 448) ----------
double e4m3_value(int code) {                 // code 0 .. 0x7E, non-negative
  const int e = code >> 3, m = code & 7;
  return e == 0 ? std::ldexp((double)m, -9) : std::ldexp(8.0 + m, e - 10);
}

struct E4M3Table {
  double mid[126];                            // midpoint between codes j and j + 1
  E4M3Table() {
    for (int j = 0; j < 126; ++j) mid[j] = 0.5 * (e4m3_value(j) + e4m3_value(j + 1));
  }
};
const E4M3Table kE4M3;

// Byte of RNE_E4M3FN(num / den), num >= 0 finite, den > 0: the number of
// midpoints below num (each midpoint times den exact), a tie resolved to
// the even code.
int e4m3_encode(double num, double den) {
  int lo = 0, hi = 126;                       // first midpoint index with mid * den >= num
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (kE4M3.mid[mid] * den < num) lo = mid + 1; else hi = mid;
  }
  int code = lo;                              // midpoints strictly below num
  if (lo < 126 && kE4M3.mid[lo] * den == num && (lo & 1)) code = lo + 1;   // tie: even code
  return code;
}

// ---- E2M1 (1 sign, 2 exponent, 1 mantissa bit) ---------------------------
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
const double kE2M1Mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};

// Magnitude code of RNE_E2M1(a / unit), a >= 0, unit > 0: a count of the
// midpoints below a; midpoint k lies between codes k and k + 1, a tie stays
// on an even k and moves up from an odd one (to the even k + 1).
int e2m1_encode(double a, double unit) {
  int code = 0;
  for (int k = 0; k < 7; ++k) {
    const double t = kE2M1Mid[k] * unit;      // exact
    code += (k & 1) ? (a >= t) : (a > t);
  }
  return code;
}

double e2m1_value(int nib) {
  const double v = kE2M1[nib & 7];
  return (nib & 8) ? -v : v;
}

// s_g from the tensor maximum (NaN for a non-finite tensor).
float global_scale(double amax) {
  if (std::isnan(amax)) return NAN;
  return (float)(amax / 2688.0);
}

// Q_1x16 of a rows x cols matrix whose tensor maximum is amax.
template <class T>
void quantize_rows(const T* x, int64_t rows, int64_t cols, double amax, uint8_t* codes,
                   uint8_t* scales, float* sg_out) {
  const float sg = global_scale(amax);
  *sg_out = sg;
  const double sgd = (double)sg;
  const int64_t nblk = cols / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nblk; ++b) {
      const T* v = x + r * cols + 16 * b;
      int scode;
      if (std::isnan(sgd)) {
        scode = 0x7F;
      } else if (sgd == 0.0) {
        scode = 0;
      } else {
        double amax_b = 0.0;
        for (int i = 0; i < 16; ++i) amax_b = std::max(amax_b, std::fabs((double)v[i]));
        scode = e4m3_encode(amax_b, 6.0 * sgd);            // 6 s_g exact
      }
      scales[r * nblk + b] = (uint8_t)scode;
      const double unit = (scode == 0x7F || scode == 0) ? 0.0 : e4m3_value(scode) * sgd;
      for (int i = 0; i < 16; i += 2) {
        int nib[2];
        for (int t = 0; t < 2; ++t) {
          const double d = (double)v[i + t];
          const int sign = std::signbit(d) ? 8 : 0;
          nib[t] = sign | (unit > 0.0 ? e2m1_encode(std::fabs(d), unit) : 0);
        }
        codes[(r * cols + 16 * b + i) / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
      }
    }
  }
}

template <class T>
double tensor_amax(const T* x, int64_t n) {
  double m = 0.0;
  int bad = 0;
#pragma omp parallel for reduction(max : m) reduction(| : bad) schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double a = std::fabs((double)x[i]);
    if (!std::isfinite(a)) bad = 1; else m = std::max(m, a);
  }
  return bad ? NAN : m;
}

// Exact values q * s * s_g of a Q_1x16 tensor, rows x cols.
void dequantize_rows(const uint8_t* codes, const uint8_t* scales, float sg, int64_t rows,
                     int64_t cols, double* out) {
  const int64_t nblk = cols / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const int sc = scales[r * nblk + c / 16];
      const double s = sc == 0x7F ? NAN : e4m3_value(sc);
      const uint8_t byte = codes[(r * cols + c) / 2];
      const int nib = (c & 1) ? (byte >> 4) : (byte & 15);
      out[r * cols + c] = e2m1_value(nib) * s * (double)sg;
    }
}

// C = P Q^T in double, P: M x K, Q: N x K (both K-contiguous).  Blocks of 32
// rows of each operand and 512 of K; each entry sums its K-blocks in order,
// each block by eight interleaved partial sums.  sym (P == Q): only j >= i is
// computed and mirrored, so C is exactly symmetric.
void gemm_nt(const double* P, const double* Q, int64_t M, int64_t N, int64_t K, bool sym,
             double* C) {
  constexpr int64_t BI = 32, BJ = 32, BK = 512;
  const int64_t ti = (M + BI - 1) / BI, tj = (N + BJ - 1) / BJ;
  std::fill(C, C + M * N, 0.0);
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int64_t bi = 0; bi < ti; ++bi)
    for (int64_t bj = 0; bj < tj; ++bj) {
      if (sym && bj < bi) continue;
      for (int64_t k0 = 0; k0 < K; k0 += BK) {
        const int64_t k1 = std::min(K, k0 + BK);
        for (int64_t i = bi * BI; i < std::min(M, (bi + 1) * BI); ++i)
          for (int64_t j = bj * BJ; j < std::min(N, (bj + 1) * BJ); ++j) {
            if (sym && j < i) continue;
            const double* p = P + i * K;
            const double* q = Q + j * K;
            double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            int64_t k = k0;
            for (; k + 8 <= k1; k += 8)
              for (int t = 0; t < 8; ++t) acc[t] += p[k + t] * q[k + t];
            double s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
            for (; k < k1; ++k) s += p[k] * q[k];
            C[i * N + j] += s;
          }
      }
    }
  if (sym)
    for (int64_t i = 0; i < M; ++i)
      for (int64_t j = 0; j < i; ++j) C[i * N + j] = C[j * N + i];
}

void transpose(const double* a, int64_t r, int64_t c, double* t) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < c; ++j)
    for (int64_t i = 0; i < r; ++i) t[j * r + i] = a[i * c + j];
}

// Q_1x16 of T (rows x cols, double) and its exact dequantization; amax
// given (NaN: any non-finite element) or computed.
struct Quantized {
  std::vector<uint8_t> codes, scales;
  float sg = 0.0f;
  std::vector<double> values;                 // dequantized, rows x cols
};

void quantize_dequantize(const double* t, int64_t rows, int64_t cols, double amax, Quantized& q) {
  q.codes.resize((size_t)(rows * cols / 2));
  q.scales.resize((size_t)(rows * cols / 16));
  q.values.resize((size_t)(rows * cols));
  quantize_rows(t, rows, cols, amax, q.codes.data(), q.scales.data(), &q.sg);
  dequantize_rows(q.codes.data(), q.scales.data(), q.sg, rows, cols, q.values.data());
}

// One NVFP4 NS step on the xm x xn iterate X (xm <= xn), in place.
void ns_step(std::vector<double>& X, int64_t xm, int64_t xn, double a, double b, double c) {
  const double amax_x = tensor_amax(X.data(), xm * xn);
  Quantized qx, qt, qa, qb;
  quantize_dequantize(X.data(), xm, xn, amax_x, qx);                    // Q_1x16(X)
  std::vector<double> Xt((size_t)(xm * xn));
  transpose(X.data(), xm, xn, Xt.data());
  quantize_dequantize(Xt.data(), xn, xm, amax_x, qt);                   // Q_16x1(X) as rows of X^T
  std::vector<double> A((size_t)(xm * xm)), B((size_t)(xm * xm)), P((size_t)(xm * xm));
  gemm_nt(qx.values.data(), qx.values.data(), xm, xm, xn, true, A.data());   // A = qX qX^T
  quantize_dequantize(A.data(), xm, xm, tensor_amax(A.data(), xm * xm), qa); // Q_1x16(A)
  // Q_16x1(A) is Q_1x16(A^T) stored as rows of A^T; A is exactly symmetric,
  // so its rows are those of qA and the product is qA qA^T
  gemm_nt(qa.values.data(), qa.values.data(), xm, xm, xm, true, P.data());
  for (int64_t i = 0; i < xm * xm; ++i) B[i] = b * A[i] + c * P[i];
  quantize_dequantize(B.data(), xm, xm, tensor_amax(B.data(), xm * xm), qb); // Q_1x16(B)
  std::vector<double> U((size_t)(xm * xn));
  gemm_nt(qb.values.data(), qt.values.data(), xm, xn, xm, false, U.data()); // qB qX16
  for (int64_t i = 0; i < xm * xn; ++i) X[i] = a * X[i] + U[i];
}

}  // namespace

extern "C" {

int orc_threads(void) { return omp_get_max_threads(); }

// Q_1x16 of a rows x cols float (f32 != 0) or double matrix; amax NaN means
// "compute the tensor maximum" (any other value is used as given).
void orc_quantize_rows(const void* x, int f32, int64_t rows, int64_t cols, double amax,
                       uint8_t* codes, uint8_t* scales, float* sg) {
  if (f32) {
    const float* p = static_cast<const float*>(x);
    if (std::isnan(amax)) amax = tensor_amax(p, rows * cols);
    quantize_rows(p, rows, cols, amax, codes, scales, sg);
  } else {
    const double* p = static_cast<const double*>(x);
    if (std::isnan(amax)) amax = tensor_amax(p, rows * cols);
    quantize_rows(p, rows, cols, amax, codes, scales, sg);
  }
}

void orc_dequantize_rows(const uint8_t* codes, const uint8_t* scales, float sg, int64_t rows,
                         int64_t cols, double* out) {
  dequantize_rows(codes, scales, sg, rows, cols, out);
}

void orc_gemm_nt(const double* P, const double* Q, int64_t M, int64_t N, int64_t K, int sym,
                 double* C) {
  gemm_nt(P, Q, M, N, K, sym != 0, C);
}

// k NVFP4 NS steps (coeffs: k triples) on an m x n double matrix, with the
// clip and normalisation; out is m x n.
void orc_ns_nvfp4(const double* G, int64_t m, int64_t n, const double* coeffs, int k, double clip,
                  double* out) {
  const bool tr = m > n;
  const int64_t xm = tr ? n : m, xn = tr ? m : n;
  std::vector<double> X((size_t)(m * n));
  if (tr) transpose(G, m, n, X.data()); else std::memcpy(X.data(), G, sizeof(double) * m * n);
  double ss = 0.0;
  for (int64_t i = 0; i < m * n; ++i) {
    double v = X[i];
    if (v > clip) v = clip; else if (v < -clip) v = -clip;   // NaN passes through
    X[i] = v;
    ss += v * v;
  }
  const double den = std::sqrt(ss) + 1e-7;
  for (int64_t i = 0; i < m * n; ++i) X[i] /= den;
  for (int s = 0; s < k; ++s) ns_step(X, xm, xn, coeffs[3 * s], coeffs[3 * s + 1], coeffs[3 * s + 2]);
  if (tr) transpose(X.data(), xm, xn, out); else std::memcpy(out, X.data(), sizeof(double) * m * n);
}

// One step from a given iterate (m <= n), out = X'.
void orc_ns_nvfp4_step(const double* X, int64_t m, int64_t n, double a, double b, double c,
                       double* out) {
  std::vector<double> V(X, X + m * n);
  ns_step(V, m, n, a, b, c);
  std::memcpy(out, V.data(), sizeof(double) * m * n);
}

}  // extern "C"
