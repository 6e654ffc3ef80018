/*
 * Seeded synthetic workload generator.
 *
 * This file produces input tensors only: it holds none of the quantizer's or
 * the attention's arithmetic.  Both the CPU oracle and the GPU library
 * consume the buffers it writes, so the two sides always see the same bits.
 *
 * Randomness is counter based: value i of stream s under seed S is a pure
 * function of (S, s, i), so any slice of a tensor can be regenerated on its
 * own and threads can split the index space freely.
 *   key(S, s)      = mix64(S ^ (s * 0xD1B54A32D192ED03))
 *   u64(S, s, i)   = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 *   uniform(i)     = (u64 >> 11) * 2^-53                        in [0, 1)
 *   normal(i)      = sqrt(-2 ln(1 - uniform(2i))) * cos(2 pi uniform(2i+1))
 * mix64 is the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014): two
 * xor-shift-multiply rounds and a final xor-shift.
 *
 * Float results are rounded fp64 -> fp32 -> bf16, each step round to nearest
 * even, and stored as raw uint16 bf16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline double uni_k(uint64_t key, uint64_t i) {
  uint64_t u = mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
  return (double)(u >> 11) * (1.0 / 9007199254740992.0);
}

static inline double gauss_k(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = uni_k(key, 2 * i), u2 = uni_k(key, 2 * i + 1);
  return sqrt(-2.0 * log(1.0 - u1)) * cos(two_pi * u2);
}

static inline uint16_t to_bf16(double x) {
  float f = (float)x; /* fp64 -> fp32, round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf */
  u += 0x7FFFu + ((u >> 16) & 1u); /* fp32 -> bf16, ties to even */
  return (uint16_t)(u >> 16);
}

/* ---- raw streams ---------------------------------------------------- */

void synth_uniform(uint64_t seed, uint64_t stream, uint64_t i0, int64_t n,
                   double* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = uni_k(key, i0 + (uint64_t)i);
}

void synth_gauss(uint64_t seed, uint64_t stream, uint64_t i0, int64_t n,
                 double* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = gauss_k(key, i0 + (uint64_t)i);
}

void synth_round_bf16(const double* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = to_bf16(x[i]);
}

/* ---- LLM-style tensors ---------------------------------------------- *
 * out[b][t][h][c] (bf16) for absolute positions pos = pos0 + t.
 * z ~ N(0,1) at counter index ((b * 2^32 + pos) * H + h) * D + c, so a
 * slice of positions generated alone equals the same slice of a longer run.
 * If sigma != NULL the raw draw is scaled by sigma[h*D + c].
 * If rope != 0 the rotary embedding is applied at position pos with the
 * half-split pairing (c, c + D/2), angle pos * theta^(-2c/D):
 *   y_c = x_c cos - x_{c+D/2} sin,  y_{c+D/2} = x_c sin + x_{c+D/2} cos.
 * Per-sequence position offsets are not needed by any workload here.     */
void synth_llm(uint64_t seed, uint64_t stream, int32_t B, int32_t T,
               int32_t H, int32_t D, int64_t pos0, const double* sigma,
               int32_t rope, double theta, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
  int half = D / 2;
#pragma omp parallel for collapse(2) schedule(static)
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t t = 0; t < T; ++t) {
      double x[256];
      uint64_t pos = (uint64_t)(pos0 + t);
      for (int32_t h = 0; h < H; ++h) {
        uint64_t base = (((uint64_t)b << 32) + pos) * (uint64_t)H + (uint64_t)h;
        for (int32_t c = 0; c < D; ++c) {
          double z = gauss_k(key, base * (uint64_t)D + (uint64_t)c);
          x[c] = sigma ? z * sigma[h * D + c] : z;
        }
        uint16_t* o = out + (((int64_t)b * T + t) * H + h) * D;
        if (rope) {
          for (int32_t c = 0; c < half; ++c) {
            double ang = (double)pos * pow(theta, -2.0 * c / (double)D);
            double cs = cos(ang), sn = sin(ang);
            double a = x[c], bb = x[c + half];
            o[c] = to_bf16(a * cs - bb * sn);
            o[c + half] = to_bf16(a * sn + bb * cs);
          }
        } else {
          for (int32_t c = 0; c < D; ++c) o[c] = to_bf16(x[c]);
        }
      }
    }
  }
}

/* ---- video-latent tensors ------------------------------------------- *
 * Frames are rows x cols grids (row-major pixel index).  For each
 * (head, channel) an i.i.d. N(0,1) field eps_f is drawn per frame at
 * counter index ((f * H + h) * D + c) * (rows*cols) + pixel, smoothed by the
 * separable binomial kernel [1 4 6 4 1]/16 with circular boundaries along
 * columns and then rows, and scaled by 256/70 to unit variance: S(eps_f).
 * The process is X_0 = S(eps_0), X_f = rho X_{f-1} + sqrt(1-rho^2) S(eps_f).
 * out[t][h][c] (bf16) holds the first T tokens, t = f * rows*cols + pixel. */
void synth_video(uint64_t seed, uint64_t stream, int32_t H, int32_t D,
                 int32_t rows, int32_t cols, int64_t T, double rho,
                 uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
  const int64_t P = (int64_t)rows * cols;
  const int64_t n_frames = (T + P - 1) / P;
  const double w5[5] = {1.0 / 16, 4.0 / 16, 6.0 / 16, 4.0 / 16, 1.0 / 16};
  const double gain = 256.0 / 70.0, innov = sqrt(1.0 - rho * rho);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t h = 0; h < H; ++h) {
    for (int32_t c = 0; c < D; ++c) {
      double eps[4096], tmp[4096], cur[4096];
      for (int64_t f = 0; f < n_frames; ++f) {
        uint64_t base = ((uint64_t)f * H + h) * (uint64_t)D + c;
        for (int64_t p = 0; p < P; ++p) eps[p] = gauss_k(key, base * P + p);
        for (int32_t r = 0; r < rows; ++r)
          for (int32_t q = 0; q < cols; ++q) {
            double s = 0.0;
            for (int k = -2; k <= 2; ++k)
              s += w5[k + 2] * eps[r * cols + ((q + k + cols) % cols)];
            tmp[r * cols + q] = s;
          }
        for (int32_t r = 0; r < rows; ++r)
          for (int32_t q = 0; q < cols; ++q) {
            double s = 0.0;
            for (int k = -2; k <= 2; ++k)
              s += w5[k + 2] * tmp[((r + k + rows) % rows) * cols + q];
            s *= gain;
            int64_t p = (int64_t)r * cols + q;
            cur[p] = (f == 0) ? s : rho * cur[p] + innov * s;
          }
        for (int64_t p = 0; p < P; ++p) {
          int64_t t = f * P + p;
          if (t < T) out[(t * H + h) * D + c] = to_bf16(cur[p]);
        }
      }
    }
  }
}
