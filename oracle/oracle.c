/*
 * CPU oracle for the INT2 KV-cache path.  TEST INFRASTRUCTURE ONLY: the
 * tests, the smoke check and the bench's CPU-baseline leg may call it; the
 * GPU library never does, and this file shares no code with it.
 *
 * Plain and slow on purpose: every loop runs in the order the method
 * states, fp32 where the method takes a discrete decision (the fp32
 * arithmetic *is* the specification there) and fp64 for continuous
 * results (dequantised values, attention).
 *
 * Sources (web pages, cited by title and section):
 *  [QWM]  "QuantWM: Training-Free 2-bit KV Cache Quantization for Stable
 *         Video World Models", section "QuantWM Framework": 1. QSAC, 2. PSAC.
 *  [OKV]  "OmniKVQuant: KV Cache Quantization for Omni-LLMs", English
 *         abstract: per-window key ranges, rotated values (separately per
 *         modality), fused decode.
 *  [WUSH] "WUSH-KV Applies Data-Adaptive Transforms to KV Cache
 *         Quantization": affine (min/max) low-bit quantizer.
 * The pages give no formulas; where they are silent the reading used is
 * stated next to the code.
 *
 * Arithmetic contract: IEEE binary32 round-to-nearest-even, no contraction
 * (build with -ffp-contract=off), fmaf only where written, subnormals kept.
 * fp16 and bf16 conversions below are written from the IEEE 754 definition.
 */
#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 32  /* channels per value / residual group */
#define WINDOW 64 /* tokens per key-range window          */

enum { KEY_WINDOW = 0, KEY_CENTROID = 1, KEY_CENTROID_QSAC = 2 };
enum { VAL_GROUP = 0, VAL_HADAMARD = 1, VAL_HADAMARD_MODAL = 2 };

/* OpenMP threads the oracle's parallel loops may use. */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

float orc_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary16 -> value (exact). */
double orc_f16_to_f64(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

static float f16_to_f32(uint16_t h) { return (float)orc_f16_to_f64(h); }

/* value -> binary16, round to nearest, ties to even; overflow -> inf.
 * Works on the exact value of a float (or double) argument. */
uint16_t orc_f64_to_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (isnan(x)) return sign | 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00; /* halfway to 2^16 rounds up */
  if (a < ldexp(1.0, -14)) {              /* subnormal range: units of 2^-24 */
    double m = nearbyint(ldexp(a, 24));  /* default rounding mode: RNE */
    return sign | (uint16_t)m;           /* m == 1024 is the smallest normal */
  }
  int ex;
  frexp(a, &ex); /* a in [2^(ex-1), 2^ex) */
  int E = ex - 1;
  double m = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (m == 2048.0) {
    m = 1024.0;
    E += 1;
  }
  if (E > 15) return sign | 0x7C00;
  return sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024));
}

static uint16_t f32_to_f16(float f) { return orc_f64_to_f16((double)f); }

/* ------------------------------------------------------------------ */
/* INT2 group quantizer.  [WUSH] names an affine low-bit quantizer; the  */
/* INT2 form (asymmetric min/max, fp16 scale and zero) is the reading   */
/* used throughout.                                                     */
/*   mn, mx = min, max of the group (inputs canonicalised x + 0.0f)     */
/*   s_h = f16((mx - mn) / 3), z_h = f16(mn)                            */
/*   s, z = the stored fp16 values widened to fp32                      */
/*   s == 0: every code is 0                                            */
/*   else code = [x >= t0] + [x >= t1] + [x >= t2], tj = fma(j+.5, s, z)*/
/* i.e. round half up to the nearest level of the stored grid.          */
/* ------------------------------------------------------------------ */
void orc_q2(const float* x, int n, int stride, uint8_t* code,
            uint16_t* s_bits, uint16_t* z_bits) {
  float mn = x[0] + 0.0f, mx = mn;
  for (int i = 1; i < n; ++i) {
    float v = x[(size_t)i * stride] + 0.0f;
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  float s32 = (mx - mn) / 3.0f;
  uint16_t sh = f32_to_f16(s32), zh = f32_to_f16(mn);
  float s = f16_to_f32(sh), z = f16_to_f32(zh);
  for (int i = 0; i < n; ++i) {
    float v = x[(size_t)i * stride] + 0.0f;
    int c = 0;
    if (s != 0.0f) {
      c += v >= fmaf(0.5f, s, z);
      c += v >= fmaf(1.5f, s, z);
      c += v >= fmaf(2.5f, s, z);
    }
    code[i] = (uint8_t)c;
  }
  *s_bits = sh;
  *z_bits = zh;
}

/* Parameters are stored as one 32-bit word: scale bits low, zero bits high. */
static uint32_t pack_params(uint16_t s, uint16_t z) {
  return (uint32_t)s | ((uint32_t)z << 16);
}

/* Packing: byte j of a token row holds channels 4j..4j+3, channel 4j+t in
 * bits [2t, 2t+1]; codes (0,1,2,3) therefore pack to 0xE4. */
void orc_pack_row(const uint8_t* codes, int D, uint8_t* row) {
  for (int j = 0; j < D / 4; ++j) {
    row[j] = (uint8_t)(codes[4 * j] | (codes[4 * j + 1] << 2) |
                       (codes[4 * j + 2] << 4) | (codes[4 * j + 3] << 6));
  }
}

static int unpack_code(const uint8_t* row, int c) {
  return (row[c >> 2] >> (2 * (c & 3))) & 3;
}

/* Walsh-Hadamard rotation of values ([OKV] rotates values before
 * quantization; the size-D Sylvester transform, orthonormal scaling and no
 * random signs are the reading used).  fp32, stages h = 1, 2, 4, ...,
 * D/2, pairs (i, i+h) for (i & h) == 0 become (a+b, a-b); then every
 * element is multiplied by f32(1/sqrt(D)). */
void orc_wht_f32(float* x, int D) {
  for (int h = 1; h < D; h <<= 1)
    for (int i = 0; i < D; ++i)
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  float c = (float)(1.0 / sqrt((double)D));
  for (int i = 0; i < D; ++i) x[i] = x[i] * c;
}

/* The same orthonormal transform in fp64 with exact 1/sqrt(D); it is its
 * own inverse, so it also rotates attention outputs back. */
void orc_wht_f64(double* x, int D) {
  for (int h = 1; h < D; h <<= 1)
    for (int i = 0; i < D; ++i)
      if ((i & h) == 0) {
        double a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  double c = 1.0 / sqrt((double)D);
  for (int i = 0; i < D; ++i) x[i] *= c;
}

/* Per-modality rotation ([OKV] rotates values separately per modality;
 * the page does not say how the rotations differ).  Reading: modality m
 * of a head has its own sign vector sigma_m in {+1,-1}^D and the rotation
 * R_m = diag(sigma_m) H, H the orthonormal Walsh-Hadamard transform above:
 * the rotated row is orc_wht_f32(x) with channel c negated where
 * sigma_m[c] = -1 (a negation is exact).  R_m is orthogonal and
 * R_m^T = H diag(sigma_m), so attention rotates back with one H after
 * summing p_t sigma_m(t) . vhat_t over the tokens of every modality.
 * Signs: bit c % 32 of word c / 32 of the modality's row set means -1. */
static int modal_sign(const uint32_t* signs_row, int c) {
  return (signs_row[c / 32] >> (c % 32)) & 1u;
}

void orc_rotate_modal_f32(float* x, int D, const uint32_t* signs_row) {
  orc_wht_f32(x, D);
  for (int c = 0; c < D; ++c)
    if (modal_sign(signs_row, c)) x[c] = -x[c];
}

/* ------------------------------------------------------------------ */
/* Centroid assignment.  [QWM] 1: each key is assigned to a cluster     */
/* center kept at higher precision, the residual goes to 2 bits.  The   */
/* distance is fp32 in channel order: t = k_d - C_jd, acc = fma(t,t,acc);*/
/* the first minimum wins (ties -> lowest index).                        */
/* ------------------------------------------------------------------ */
static float sq_dist(const float* k, const float* c, int D) {
  float acc = 0.0f;
  for (int d = 0; d < D; ++d) {
    float t = k[d] - c[d];
    acc = fmaf(t, t, acc);
  }
  return acc;
}

static float w_dist(const float* k, const float* c, const float* w, int D) {
  float acc = 0.0f;
  for (int d = 0; d < D; ++d) {
    float t = k[d] - c[d];
    float wt = w[d] * t;
    acc = fmaf(wt, t, acc);
  }
  return acc;
}

int orc_assign_plain(const float* k, const float* cent, int C, int D) {
  int best = 0;
  float bd = sq_dist(k, cent, D);
  for (int j = 1; j < C; ++j) {
    float dj = sq_dist(k, cent + (size_t)j * D, D);
    if (dj < bd) {
      bd = dj;
      best = j;
    }
  }
  return best;
}

/* Residual r = k - C_j quantised per group of 32; rhat = fma(code, s, z)
 * in fp32; e = r - rhat.  Writes codes (one per channel), params and e. */
static void residual_q2(const float* k, const float* c, int D, uint8_t* codes,
                        uint32_t* params, float* e) {
  float r[256];
  for (int d = 0; d < D; ++d) r[d] = k[d] - c[d];
  for (int g = 0; g < D / GROUP; ++g) {
    uint16_t sh, zh;
    orc_q2(r + g * GROUP, GROUP, 1, codes + g * GROUP, &sh, &zh);
    params[g] = pack_params(sh, zh);
    float s = f16_to_f32(sh), z = f16_to_f32(zh);
    for (int i = 0; i < GROUP; ++i) {
      int d = g * GROUP + i;
      float rh = fmaf((float)codes[d], s, z);
      e[d] = (r[d] + 0.0f) - rh;
    }
  }
}

/* Range-based perturbation estimate of one candidate ([QWM] 1: from the
 * residual groups' dynamic range and the query sensitivity): INT2 rounding
 * noise has variance s^2/12 per element of a group with step s, weighted by
 * the group's summed sensitivity W_g.  The common factor 1/12 is left out
 * (it does not change which candidate is smallest):
 *   W_g = fold acc = acc + w_d over the group's channels in order (fp32),
 *   s_g = f32(f16((max r - min r) / 3)), the step the quantizer stores,
 *   E = fold over groups in order of acc = fma(s_g * s_g, W_g, acc). */
static float range_estimate(const float* k, const float* c, const float* w, int D) {
  float E = 0.0f;
  for (int g = 0; g < D / GROUP; ++g) {
    float W = 0.0f, mn = INFINITY, mx = -INFINITY;
    for (int i = 0; i < GROUP; ++i) {
      int d = g * GROUP + i;
      float r = k[d] - c[d];
      W = W + w[d];
      if (r < mn) mn = r;
      if (r > mx) mx = r;
    }
    float s = f16_to_f32(f32_to_f16((mx - mn) / 3.0f));
    E = fmaf(s * s, W, E);
  }
  return E;
}

/* QSAC ([QWM] 1).  Candidates: the topk smallest (weighted distance,
 * index) pairs, weighted distance acc = fma(w_d t, t, acc) with w_d t
 * rounded first.  The attention-perturbation estimate E of each candidate
 * is, with score 0, the sensitivity-weighted squared error of its actual
 * INT2 residual, E = fold acc = fma(w_d e_d, e_d, acc) in channel order;
 * with score 1, the range-based estimate above.  The lexicographic minimum
 * (E, index) is chosen. */
int orc_assign_qsac(const float* k, const float* cent, int C, int D,
                    const float* w, int topk, int score) {
  if (topk > C) topk = C;
  if (topk > 16) topk = 16;
  int cand[16];
  float cd[16];
  int n = 0;
  for (int j = 0; j < C; ++j) {
    float dj = w_dist(k, cent + (size_t)j * D, w, D);
    /* insert into the sorted candidate list (ascending (dist, index)) */
    if (n < topk || dj < cd[n - 1]) {
      int p = (n < topk) ? n++ : n - 1;
      while (p > 0 && dj < cd[p - 1]) {
        cd[p] = cd[p - 1];
        cand[p] = cand[p - 1];
        --p;
      }
      cd[p] = dj;
      cand[p] = j;
    }
  }
  int best = -1;
  float bestE = 0.0f;
  for (int i = 0; i < n; ++i) {
    int j = cand[i];
    float E = 0.0f;
    if (score == 1) {
      E = range_estimate(k, cent + (size_t)j * D, w, D);
    } else {
      uint8_t codes[256];
      uint32_t prm[8];
      float e[256];
      residual_q2(k, cent + (size_t)j * D, D, codes, prm, e);
      for (int d = 0; d < D; ++d) {
        float we = w[d] * e[d];
        E = fmaf(we, e[d], E);
      }
    }
    if (best < 0 || E < bestE || (E == bestE && j < best)) {
      best = j;
      bestE = E;
    }
  }
  return best;
}

/* ------------------------------------------------------------------ */
/* Cache update (the kv_quantize_append contract).                      */
/* Buffers, per (b, h) with capacity Tcap tokens, D channels:           */
/*   k_codes           u8  [B][H][Tcap][D/4]   token rows (packing above)  */
/*   v_codes           u8  [B][H][Tcap/64][D][16]  per 64-token tile,      */
/*                     channel-major: the code of tile token t (0..63)     */
/*                     for channel c sits in byte 16c + t/4, bits 2(t%4)   */
/*   v_params          u32 [B][H][Tcap][D/32]                           */
/*   k_params  window: u32 [B][H][Tcap/64][D]; centroid: u32 [..][Tcap][D/32] */
/*   k_tail            u16 [B][H][64][D]    (bf16, window mode)          */
/*   k_idx             u8  [B][H][Tcap]     (centroid modes)            */
/*   centroids         f32 [B][H][C][D];  sens_w f32 [B][H][D]          */
/*   psac_basis        f32 [B][H][D][R];  k_psac u16 [B][H][Tcap][R]     */
/*   (INT8 coefficients: k_psac8 i8 [B][H][Tcap][R] + k_psac_sc u16       */
/*   [B][H][Tcap], the per-token fp16 scale)                              */
/* New tokens: k_in, v_in bf16 [B][n_new][H][D] at positions              */
/* cur_len .. cur_len+n_new-1 of every sequence.                         */
/* ------------------------------------------------------------------ */
typedef struct {
  int B, H, D, Tcap, key_mode, value_mode, C, topk, R, qsac_score, psac_fmt;
  int M;                    /* modalities (VAL_HADAMARD_MODAL)             */
  const uint32_t* v_signs;  /* u32 [H][M][D/32] sign bits                  */
  const uint8_t* v_modal;   /* u8 [B][Tcap] modality of each token         */
} layout_t;

static size_t bh(const layout_t* L, int b, int h) {
  return (size_t)b * L->H + h;
}

/* Byte holding the value code of token p, channel c of sequence-head s. */
static uint8_t* value_code_byte(uint8_t* v_codes, size_t s, int Tcap, int D, int p, int c) {
  return v_codes + ((s * (size_t)(Tcap / WINDOW) + (size_t)(p / WINDOW)) * D + c) * 16 +
         (p % WINDOW) / 4;
}

static void quantize_value_row(const layout_t* L, const uint16_t* v, int b, int h,
                               uint8_t* v_codes, size_t s, int p, uint32_t* prm) {
  int D = L->D;
  float x[256];
  uint8_t codes[256];
  for (int d = 0; d < D; ++d) x[d] = orc_bf16_to_f32(v[d]);
  if (L->value_mode == VAL_HADAMARD) orc_wht_f32(x, D);
  if (L->value_mode == VAL_HADAMARD_MODAL) {
    const int m = L->v_modal[(size_t)b * L->Tcap + p];
    orc_rotate_modal_f32(x, D, L->v_signs + ((size_t)h * L->M + m) * (D / 32));
  }
  for (int g = 0; g < D / GROUP; ++g) {
    uint16_t sh, zh;
    orc_q2(x + g * GROUP, GROUP, 1, codes + g * GROUP, &sh, &zh);
    prm[g] = pack_params(sh, zh);
  }
  const int sh = 2 * (p % 4);
  for (int c = 0; c < D; ++c) {
    uint8_t* byte = value_code_byte(v_codes, s, L->Tcap, D, p, c);
    *byte = (uint8_t)((*byte & ~(3u << sh)) | ((unsigned)codes[c] << sh));
  }
}

/* INT8 PSAC coefficients ([QWM] 2 quantizes them to INT8): symmetric, one
 * fp16 scale per token: sc = f16(max_m |a_m| / 127); q_m = a_m / sc
 * rounded to the nearest integer (ties to even), clamped to [-127, 127];
 * all zero when sc is 0.  The coefficient used is q_m * sc. */
static void psac_int8(const float* a, int R, int8_t* q, uint16_t* sc_out) {
  float amax = 0.0f;
  for (int m = 0; m < R; ++m)
    if (fabsf(a[m]) > amax) amax = fabsf(a[m]);
  uint16_t sh = f32_to_f16(amax / 127.0f);
  float sc = f16_to_f32(sh);
  for (int m = 0; m < R; ++m) {
    float v = (sc == 0.0f) ? 0.0f : rintf(a[m] / sc);
    if (v > 127.0f) v = 127.0f;
    if (v < -127.0f) v = -127.0f;
    q[m] = (int8_t)v;
  }
  *sc_out = sh;
}

static void quantize_centroid_key(const layout_t* L, const uint16_t* kin,
                                  const float* cent, const float* w,
                                  const float* U, uint8_t* idx_out,
                                  uint8_t* code_row, uint32_t* prm,
                                  uint16_t* psac, int8_t* psac8, uint16_t* psac_sc) {
  int D = L->D;
  float k[256], e[256];
  uint8_t codes[256];
  for (int d = 0; d < D; ++d) k[d] = orc_bf16_to_f32(kin[d]);
  int j = (L->key_mode == KEY_CENTROID_QSAC)
              ? orc_assign_qsac(k, cent, L->C, D, w, L->topk, L->qsac_score)
              : orc_assign_plain(k, cent, L->C, D);
  residual_q2(k, cent + (size_t)j * D, D, codes, prm, e);
  orc_pack_row(codes, D, code_row);
  *idx_out = (uint8_t)j;
  /* PSAC ([QWM] 2): coefficients of the key error along the principal
   * query directions, a_m = fold acc = fma(U_dm, e_d, acc), stored as fp16
   * (psac_fmt 0) or INT8 with a per-token scale (psac_fmt 1). */
  float a[16];
  for (int m = 0; m < L->R; ++m) {
    float acc = 0.0f;
    for (int d = 0; d < D; ++d) acc = fmaf(U[(size_t)d * L->R + m], e[d], acc);
    a[m] = acc;
  }
  if (L->R > 0 && L->psac_fmt == 1)
    psac_int8(a, L->R, psac8, psac_sc);
  else
    for (int m = 0; m < L->R; ++m) psac[m] = f32_to_f16(a[m]);
}

/* Key-range windows ([OKV]: the key quantization range is set over each
 * short window of the input stream).  Windows are 64 tokens aligned to
 * absolute stream position; a window is quantised per channel once all 64
 * of its tokens are present; tokens of the unfinished last window wait
 * verbatim (bf16) in the tail at slot position % 64.  The packed cache
 * therefore depends on the token sequence only, not on how it was split
 * into appends. */
int orc_quantize_append(int B, int H, int D, int Tcap, int key_mode,
                        int value_mode, int C, int topk, int R, int qsac_score,
                        int psac_fmt, int M, const uint32_t* v_signs,
                        const uint8_t* v_modal, uint8_t* k_codes, uint32_t* k_params,
                        uint16_t* k_tail, uint8_t* k_idx, const float* centroids,
                        const float* sens_w, const float* psac_basis,
                        uint16_t* k_psac, int8_t* k_psac8, uint16_t* k_psac_sc,
                        uint8_t* v_codes, uint32_t* v_params,
                        const uint16_t* k_in, const uint16_t* v_in, int cur_len,
                        int n_new) {
  layout_t L = {B, H, D, Tcap, key_mode, value_mode, C, topk, R, qsac_score, psac_fmt,
                M, v_signs, v_modal};
  if (cur_len < 0 || n_new < 0 || cur_len + n_new > Tcap) return -3;
  if (value_mode == VAL_HADAMARD_MODAL) {
    if (M < 1 || !v_signs || !v_modal) return -1;
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < n_new; ++i)
        if (v_modal[(size_t)b * Tcap + cur_len + i] >= M) return -1;
  }
  const int rb = D / 4, ng = D / GROUP;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      size_t s = bh(&L, b, h);
      for (int i = 0; i < n_new; ++i) {
        int p = cur_len + i;
        const uint16_t* v = v_in + (((size_t)b * n_new + i) * H + h) * D;
        quantize_value_row(&L, v, b, h, v_codes, s, p, v_params + (s * Tcap + p) * ng);
      }
      if (key_mode == KEY_WINDOW) {
        uint16_t* tail = k_tail + s * WINDOW * D;
        int end = cur_len + n_new;
        for (int w = cur_len / WINDOW; (w + 1) * WINDOW <= end; ++w) {
          float blk[WINDOW * 256];
          uint8_t col[WINDOW];
          uint8_t codes[WINDOW][256];
          for (int t = 0; t < WINDOW; ++t) {
            int p = w * WINDOW + t;
            const uint16_t* src =
                (p < cur_len)
                    ? tail + (size_t)(p % WINDOW) * D
                    : k_in + (((size_t)b * n_new + (p - cur_len)) * H + h) * D;
            for (int d = 0; d < D; ++d) blk[t * D + d] = orc_bf16_to_f32(src[d]);
          }
          for (int d = 0; d < D; ++d) {
            uint16_t sh, zh;
            orc_q2(blk + d, WINDOW, D, col, &sh, &zh);
            k_params[(s * (Tcap / WINDOW) + w) * D + d] = pack_params(sh, zh);
            for (int t = 0; t < WINDOW; ++t) codes[t][d] = col[t];
          }
          for (int t = 0; t < WINDOW; ++t)
            orc_pack_row(codes[t], D, k_codes + (s * Tcap + w * WINDOW + t) * rb);
        }
        int tail_start = (end / WINDOW) * WINDOW;
        if (tail_start < cur_len) tail_start = cur_len;
        for (int p = tail_start; p < end; ++p) {
          const uint16_t* src = k_in + (((size_t)b * n_new + (p - cur_len)) * H + h) * D;
          memcpy(tail + (size_t)(p % WINDOW) * D, src, (size_t)D * 2);
        }
      } else {
        const float* cent = centroids + s * (size_t)C * D;
        const float* w = sens_w ? sens_w + s * D : NULL;
        const float* U = (R > 0) ? psac_basis + s * (size_t)D * R : NULL;
        for (int i = 0; i < n_new; ++i) {
          int p = cur_len + i;
          const uint16_t* kin = k_in + (((size_t)b * n_new + i) * H + h) * D;
          uint16_t* ps = (R > 0) ? k_psac + (s * Tcap + p) * R : NULL;
          int8_t* ps8 = (R > 0) ? k_psac8 + (s * Tcap + p) * R : NULL;
          uint16_t* psc = (R > 0) ? k_psac_sc + s * Tcap + p : NULL;
          quantize_centroid_key(&L, kin, cent, w, U, k_idx + s * Tcap + p,
                                k_codes + (s * Tcap + p) * rb,
                                k_params + (s * Tcap + p) * ng, ps, ps8, psc);
        }
      }
    }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Exact dequantisation (fp64): code * s + z with the stored fp16 s, z.  */
/* ------------------------------------------------------------------ */
static double deq(int code, uint32_t prm) {
  return (double)code * orc_f16_to_f64((uint16_t)(prm & 0xFFFF)) +
         orc_f16_to_f64((uint16_t)(prm >> 16));
}

/* keys of (b, h), tokens [0, n): out f64 [n][D] (without PSAC) */
void orc_dequant_keys(int B, int H, int D, int Tcap, int key_mode, int C,
                      const uint8_t* k_codes, const uint32_t* k_params,
                      const uint16_t* k_tail, const uint8_t* k_idx,
                      const float* centroids, int b, int h, int n,
                      double* out) {
  (void)B;
  size_t s = (size_t)b * H + h;
  const int rb = D / 4;
  int full = (n / WINDOW) * WINDOW;
  for (int p = 0; p < n; ++p) {
    const uint8_t* row = k_codes + (s * Tcap + p) * rb;
    for (int d = 0; d < D; ++d) {
      double v;
      if (key_mode == KEY_WINDOW) {
        if (p < full)
          v = deq(unpack_code(row, d),
                  k_params[(s * (Tcap / WINDOW) + p / WINDOW) * D + d]);
        else
          v = (double)orc_bf16_to_f32(k_tail[(s * WINDOW + p % WINDOW) * D + d]);
      } else {
        int j = k_idx[s * Tcap + p];
        v = (double)centroids[(s * C + j) * D + d] +
            deq(unpack_code(row, d), k_params[(s * Tcap + p) * (D / GROUP) + d / GROUP]);
      }
      out[(size_t)p * D + d] = v;
    }
  }
}

/* values of (b, h), tokens [0, n): out f64 [n][D], in the rotated basis when
 * values were rotated. */
void orc_dequant_values(int H, int D, int Tcap, const uint8_t* v_codes,
                        const uint32_t* v_params, int b, int h, int n,
                        double* out) {
  size_t s = (size_t)b * H + h;
  for (int p = 0; p < n; ++p) {
    for (int d = 0; d < D; ++d) {
      const int code = (*value_code_byte((uint8_t*)v_codes, s, Tcap, D, p, d) >> (2 * (p % 4))) & 3;
      out[(size_t)p * D + d] = deq(code, v_params[(s * Tcap + p) * (D / GROUP) + d / GROUP]);
    }
  }
}

/* ------------------------------------------------------------------ */
/* Attention over the dequantised cache (fp64): for query head hq the    */
/* kv head is hq / (Hq/H); logits scale * (q.khat + [PSAC] (U^T q).a);   */
/* softmax over all n cached tokens (no mask); o = sum p vhat, rotated   */
/* back with the orthonormal WHT when values were rotated;               */
/* lse = max + log(sum exp(logit - max)).                                 */
/* q f64 [B][Lq][Hq][D]; out f64 [B][Lq][Hq][D]; lse f64 [B][Hq][Lq].     */
/* ------------------------------------------------------------------ */
int orc_attention(int B, int H, int D, int Tcap, int key_mode, int value_mode,
                  int C, int R, int psac_fmt, int M, const uint32_t* v_signs,
                  const uint8_t* v_modal, const uint8_t* k_codes,
                  const uint32_t* k_params, const uint16_t* k_tail,
                  const uint8_t* k_idx, const float* centroids,
                  const float* psac_basis, const uint16_t* k_psac,
                  const int8_t* k_psac8, const uint16_t* k_psac_sc,
                  const uint8_t* v_codes,
                  const uint32_t* v_params, int n, const double* q, int Lq,
                  int Hq, double scale, double* out, double* lse) {
  if (Hq % H != 0 || n < 1) return -1;
  if (value_mode == VAL_HADAMARD_MODAL && (M < 1 || !v_signs || !v_modal)) return -1;
  const int grp = Hq / H;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      double* kh = (double*)malloc(sizeof(double) * (size_t)n * D);
      double* vh = (double*)malloc(sizeof(double) * (size_t)n * D);
      if (!kh || !vh) {
        free(kh);
        free(vh);
        return -2;
      }
      orc_dequant_keys(B, H, D, Tcap, key_mode, C, k_codes, k_params, k_tail,
                       k_idx, centroids, b, h, n, kh);
      orc_dequant_values(H, D, Tcap, v_codes, v_params, b, h, n, vh);
      /* per-modality rotation: R_m^T = H diag(sigma_m), so each rotated
       * value takes its modality's signs before the one final H */
      if (value_mode == VAL_HADAMARD_MODAL)
        for (int t = 0; t < n; ++t) {
          const int m = v_modal[(size_t)b * Tcap + t];
          if (m >= M) {
            free(kh);
            free(vh);
            return -1;
          }
          const uint32_t* row = v_signs + ((size_t)h * M + m) * (D / 32);
          for (int d = 0; d < D; ++d)
            if (modal_sign(row, d)) vh[(size_t)t * D + d] = -vh[(size_t)t * D + d];
        }
      size_t s = (size_t)b * H + h;
#pragma omp parallel for collapse(2) schedule(dynamic)
      for (int g = 0; g < grp; ++g)
        for (int i = 0; i < Lq; ++i) {
          int hq = h * grp + g;
          const double* qi = q + (((size_t)b * Lq + i) * Hq + hq) * D;
          double qp[16] = {0};
          for (int m = 0; m < R; ++m)
            for (int d = 0; d < D; ++d)
              qp[m] += psac_basis[(s * D + d) * R + m] * qi[d];
          double* lg = (double*)malloc(sizeof(double) * (size_t)n);
          double mx = -INFINITY;
          for (int t = 0; t < n; ++t) {
            double a = 0.0;
            for (int d = 0; d < D; ++d) a += qi[d] * kh[(size_t)t * D + d];
            for (int m = 0; m < R; ++m)
              a += qp[m] * (psac_fmt == 1
                                ? (double)k_psac8[(s * Tcap + t) * R + m] *
                                      orc_f16_to_f64(k_psac_sc[s * Tcap + t])
                                : orc_f16_to_f64(k_psac[(s * Tcap + t) * R + m]));
            lg[t] = scale * a;
            if (lg[t] > mx) mx = lg[t];
          }
          double sum = 0.0;
          for (int t = 0; t < n; ++t) {
            lg[t] = exp(lg[t] - mx);
            sum += lg[t];
          }
          double o[256];
          for (int d = 0; d < D; ++d) o[d] = 0.0;
          for (int t = 0; t < n; ++t) {
            double p = lg[t] / sum;
            for (int d = 0; d < D; ++d) o[d] += p * vh[(size_t)t * D + d];
          }
          if (value_mode == VAL_HADAMARD || value_mode == VAL_HADAMARD_MODAL) orc_wht_f64(o, D);
          double* oo = out + (((size_t)b * Lq + i) * Hq + hq) * D;
          for (int d = 0; d < D; ++d) oo[d] = o[d];
          lse[((size_t)b * Hq + hq) * Lq + i] = mx + log(sum);
          free(lg);
        }
      free(kh);
      free(vh);
    }
  return 0;
}

/* Top-1 cached token of each query row (the attention-shift diagnostic of
 * "QuantWM: Training-Free 2-bit KV Cache Quantization for Stable Video World
 * Models": Figure 2 and "Experimental Validation", Table 1 count how often
 * key quantization moves a query's highest-scoring history token): the
 * token t < n with the largest logit
 * q.khat_t (+ (U^T q).a_t with PSAC), the same logit orc_attention uses
 * before its scale, in fp64 over the exactly dequantised cache; the first
 * index on ties.  idx i32 [B][Hq][Lq]; logit f64 [B][Hq][Lq]. */
int orc_top1(int B, int H, int D, int Tcap, int key_mode, int C, int R, int psac_fmt,
             const uint8_t* k_codes, const uint32_t* k_params, const uint16_t* k_tail,
             const uint8_t* k_idx, const float* centroids, const float* psac_basis,
             const uint16_t* k_psac, const int8_t* k_psac8, const uint16_t* k_psac_sc,
             int n, const double* q, int Lq, int Hq, int32_t* idx, double* logit) {
  if (Hq % H != 0 || n < 1) return -1;
  const int grp = Hq / H;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      double* kh = (double*)malloc(sizeof(double) * (size_t)n * D);
      if (!kh) return -2;
      orc_dequant_keys(B, H, D, Tcap, key_mode, C, k_codes, k_params, k_tail, k_idx,
                       centroids, b, h, n, kh);
      size_t s = (size_t)b * H + h;
#pragma omp parallel for collapse(2) schedule(dynamic)
      for (int g = 0; g < grp; ++g)
        for (int i = 0; i < Lq; ++i) {
          int hq = h * grp + g;
          const double* qi = q + (((size_t)b * Lq + i) * Hq + hq) * D;
          double qp[16] = {0};
          for (int m = 0; m < R; ++m)
            for (int d = 0; d < D; ++d) qp[m] += psac_basis[(s * D + d) * R + m] * qi[d];
          int best = 0;
          double bl = -INFINITY;
          for (int t = 0; t < n; ++t) {
            double a = 0.0;
            for (int d = 0; d < D; ++d) a += qi[d] * kh[(size_t)t * D + d];
            for (int m = 0; m < R; ++m)
              a += qp[m] * (psac_fmt == 1
                                ? (double)k_psac8[(s * Tcap + t) * R + m] *
                                      orc_f16_to_f64(k_psac_sc[s * Tcap + t])
                                : orc_f16_to_f64(k_psac[(s * Tcap + t) * R + m]));
            if (t == 0 || a > bl) {
              bl = a;
              best = t;
            }
          }
          idx[((size_t)b * Hq + hq) * Lq + i] = best;
          logit[((size_t)b * Hq + hq) * Lq + i] = bl;
        }
      free(kh);
    }
  return 0;
}

/* Merge of attention partials over disjoint token sets: with partial
 * (m_s, l_s, o_s) (running max, sum of exp(logit - m_s), unnormalised
 * output) M = max m_s, l = sum exp(m_s - M) l_s,
 * o = sum exp(m_s - M) o_s / l, lse = M + log l. */
void orc_merge(int S, int D, const double* m, const double* l,
               const double* o, double* out, double* lse) {
  double M = -INFINITY;
  for (int s = 0; s < S; ++s)
    if (m[s] > M) M = m[s];
  double L = 0.0;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int s = 0; s < S; ++s) {
    double f = exp(m[s] - M);
    L += f * l[s];
    for (int d = 0; d < D; ++d) out[d] += f * o[(size_t)s * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] /= L;
  *lse = M + log(L);
}

/* ------------------------------------------------------------------ */
/* Calibration (host side; its outputs are inputs to both sides).        */
/* ------------------------------------------------------------------ */

/* Lloyd k-means on the f32 keys x [n][D] of one head: centroids start at
 * the given token picks; each iteration assigns every key with the fp32
 * channel-order distance above and then sets each centroid to
 * f32(fp64 mean of its members, summed in token order); an empty cluster
 * keeps its centroid.  cent f32 [C][D] out; assign i32 [n] out (last
 * iteration's assignment, or the initial one when iters == 0). */
void orc_kmeans(const float* x, int n, int D, int C, const int64_t* init,
                int iters, float* cent, int32_t* assign) {
  for (int j = 0; j < C; ++j)
    memcpy(cent + (size_t)j * D, x + (size_t)init[j] * D, sizeof(float) * D);
  for (int it = 0; it < iters; ++it) {
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i)
      assign[i] = orc_assign_plain(x + (size_t)i * D, cent, C, D);
    double* sum = (double*)calloc((size_t)C * D, sizeof(double));
    int64_t* cnt = (int64_t*)calloc((size_t)C, sizeof(int64_t));
    for (int i = 0; i < n; ++i) {
      int j = assign[i];
      cnt[j]++;
      for (int d = 0; d < D; ++d) sum[(size_t)j * D + d] += (double)x[(size_t)i * D + d];
    }
    for (int j = 0; j < C; ++j)
      if (cnt[j] > 0)
        for (int d = 0; d < D; ++d)
          cent[(size_t)j * D + d] = (float)(sum[(size_t)j * D + d] / (double)cnt[j]);
    free(sum);
    free(cnt);
  }
  if (iters == 0)
    for (int i = 0; i < n; ++i)
      assign[i] = orc_assign_plain(x + (size_t)i * D, cent, C, D);
}

/* Query sensitivity ([QWM] 1 and 2 use statistics of historical
 * queries): w_d = f32(mean over the N queries of q_d^2), fp64 sums. */
void orc_sens_weights(const double* q, int N, int D, float* w) {
  for (int d = 0; d < D; ++d) {
    double a = 0.0;
    for (int i = 0; i < N; ++i) a += q[(size_t)i * D + d] * q[(size_t)i * D + d];
    w[d] = (float)(a / N);
  }
}

/* Principal query directions ([QWM] 2): eigenvectors of the uncentred
 * second moment M = (1/N) sum q q^T (the queries' energy), by cyclic Jacobi
 * rotations in fp64, ordered by descending eigenvalue (ties: lower original
 * index first).  Each vector's largest-magnitude component (first on ties)
 * is made positive.  U f32 [D][R] out; evals f64 [D] out (descending);
 * returns the number of sweeps. */
int orc_pca(const double* q, int N, int D, int R, float* U, double* evals) {
  double* A = (double*)calloc((size_t)D * D, sizeof(double));
  double* V = (double*)calloc((size_t)D * D, sizeof(double));
  for (int i = 0; i < N; ++i)
    for (int a = 0; a < D; ++a)
      for (int c = 0; c < D; ++c)
        A[(size_t)a * D + c] += q[(size_t)i * D + a] * q[(size_t)i * D + c];
  for (int a = 0; a < D * D; ++a) A[a] /= N;
  for (int a = 0; a < D; ++a) V[(size_t)a * D + a] = 1.0;
  int sweep = 0;
  for (; sweep < 100; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int a = 0; a < D; ++a)
      for (int c = 0; c < D; ++c) {
        if (a != c) off += A[(size_t)a * D + c] * A[(size_t)a * D + c];
        else diag += A[(size_t)a * D + c] * A[(size_t)a * D + c];
      }
    if (off <= 1e-24 * diag) break;
    for (int p = 0; p < D - 1; ++p)
      for (int r = p + 1; r < D; ++r) {
        double apr = A[(size_t)p * D + r];
        if (apr == 0.0) continue;
        double app = A[(size_t)p * D + p], arr = A[(size_t)r * D + r];
        double theta = (arr - app) / (2.0 * apr);
        double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < D; ++k) { /* A <- A J (columns p, r) */
          double akp = A[(size_t)k * D + p], akr = A[(size_t)k * D + r];
          A[(size_t)k * D + p] = c * akp - s * akr;
          A[(size_t)k * D + r] = s * akp + c * akr;
        }
        for (int k = 0; k < D; ++k) { /* A <- J^T A (rows p, r) */
          double apk = A[(size_t)p * D + k], ark = A[(size_t)r * D + k];
          A[(size_t)p * D + k] = c * apk - s * ark;
          A[(size_t)r * D + k] = s * apk + c * ark;
        }
        for (int k = 0; k < D; ++k) { /* V <- V J */
          double vkp = V[(size_t)k * D + p], vkr = V[(size_t)k * D + r];
          V[(size_t)k * D + p] = c * vkp - s * vkr;
          V[(size_t)k * D + r] = s * vkp + c * vkr;
        }
      }
  }
  int* ord = (int*)malloc(sizeof(int) * D);
  for (int a = 0; a < D; ++a) ord[a] = a;
  for (int a = 1; a < D; ++a) { /* stable insertion sort, descending */
    int x = ord[a], p = a;
    while (p > 0 && A[(size_t)ord[p - 1] * D + ord[p - 1]] < A[(size_t)x * D + x]) {
      ord[p] = ord[p - 1];
      --p;
    }
    ord[p] = x;
  }
  for (int a = 0; a < D; ++a) evals[a] = A[(size_t)ord[a] * D + ord[a]];
  for (int m = 0; m < R; ++m) {
    int col = ord[m], arg = 0;
    for (int d = 1; d < D; ++d)
      if (fabs(V[(size_t)d * D + col]) > fabs(V[(size_t)arg * D + col])) arg = d;
    double sg = V[(size_t)arg * D + col] < 0 ? -1.0 : 1.0;
    for (int d = 0; d < D; ++d) U[(size_t)d * R + m] = (float)(sg * V[(size_t)d * D + col]);
  }
  free(ord);
  free(A);
  free(V);
  return sweep;
}
