/*
 * oracle.c - plain, slow, float64 CPU oracle for the FP8 e4m3 paged KV cache
 * (and E5M2) and GQA paged decode attention.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The product (the HIP library and its
 * Python binding) never calls it, and it shares no code, header or table with
 * the product: everything here is written from the definitions below.
 *
 * Sources of each definition (page title, then section):
 *  - E4M3 format (1 sign, 4 exponent, 3 mantissa bits, max 448): "FP8量化与长
 *    上下文推理" section 1 (format table); "cooking-agi: FP8 and the KV cache",
 *    section "dynamic vs static scale" (max 448) and section "how to enable
 *    it in the engine" (smallest subnormal 2^-9). Exponent bias 7, no
 *    infinities and the single NaN mantissa pattern are the OCP definition
 *    the latter page refers to.
 *  - E5M2 format (1 sign, 5 exponent, 2 mantissa bits, range about +-57344):
 *    "FP8量化与长上下文推理" section 1 (format table); offered as a KV-cache
 *    dtype (fp8_e5m2) in "cooking-agi", section "how to enable it in the
 *    engine". Exponent bias 15, infinities (S.11111.00) and NaNs
 *    (S.11111.xx, xx != 0) are the OCP definition.
 *  - Saturating conversion (overflow clamps to the largest finite value):
 *    "cooking-agi", section "dynamic vs static scale"; applied to both
 *    formats (E5M2 infinities saturate too, like E4M3's).
 *  - Symmetric scaled quantisation q = round(x / s), dequantisation q * s,
 *    s = max_abs / 448: "FP8量化与长上下文推理" section 1.1.
 *  - Cache write into pages with a scalar or per-KV-head scale: "State of FP8
 *    KV cache and attention quantization in vLLM", section "Kernel and vLLM
 *    improvements", paragraph "Per-head scales".
 *  - Attention softmax(q k^T) v with online rescaling and split partials:
 *    same post, section "Single-request benchmark" (online softmax
 *    rescaling) and paragraph "Two-level accumulation".
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): round-to-nearest-even; IEEE fp32 division x / s; Inf
 * saturates; NaN keeps its sign (0x7F / 0xFF); the sign of zero is kept;
 * softmax scale 1/sqrt(D); query head i uses KV head i / G; the attended
 * window is the last W positions including the newest; amax == 0 gives s = 1.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -shared -fPIC -pthread.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* E4M3 decode: the OCP definition written out.                              */
/* ------------------------------------------------------------------------ */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;               /* S.1111.111 */
  if (e == 0)
    mag = ldexp((double)m, -9);                    /* m/8 * 2^(1-7) */
  else
    mag = ldexp((double)(8 + m), e - 10);          /* (1+m/8) * 2^(e-7) */
  return s ? -mag : mag;
}

void orc_e4m3_decode_all(double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = orc_e4m3_decode((uint8_t)c);
}

/* ------------------------------------------------------------------------ */
/* E4M3 encode, saturating, round-to-nearest-even: the plain definition.     */
/* The 127 non-negative finite values (codes 0x00..0x7E) increase with the   */
/* code, so the nearest value is found between two neighbours of the sorted  */
/* table; an exact midpoint goes to the neighbour whose code is even.        */
/* ------------------------------------------------------------------------ */
static double g_table[127];
static pthread_once_t g_table_once = PTHREAD_ONCE_INIT;

static void build_table(void) {
  for (int c = 0; c < 127; ++c) g_table[c] = orc_e4m3_decode((uint8_t)c);
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

uint8_t orc_e4m3_encode(float y) {
  pthread_once(&g_table_once, build_table);
  uint32_t sign = f32_bits(y) >> 31;
  if (isnan(y)) return (uint8_t)(0x7F | (sign << 7));
  double a = fabs((double)y);
  int code;
  if (a >= g_table[126]) {
    code = 126;                                    /* saturate, Inf too */
  } else {
    int lo = 0, hi = 126;                          /* g_table[lo] <= a < g_table[hi] */
    while (hi - lo > 1) {
      int mid = (lo + hi) / 2;
      if (g_table[mid] <= a) lo = mid; else hi = mid;
    }
    double below = g_table[lo], above = g_table[hi];
    double mid = 0.5 * (below + above);            /* exact in double */
    if (a < mid) code = lo;
    else if (a > mid) code = hi;
    else code = (lo % 2 == 0) ? lo : hi;
  }
  return (uint8_t)(code | (sign << 7));
}

/* The same definition by a linear scan over all 127 values: nearest value,
 * ties to the even code. Used on samples to pin the binary search. */
uint8_t orc_e4m3_encode_scan(float y) {
  pthread_once(&g_table_once, build_table);
  uint32_t sign = f32_bits(y) >> 31;
  if (isnan(y)) return (uint8_t)(0x7F | (sign << 7));
  double a = fabs((double)y);
  if (a > g_table[126]) a = g_table[126];
  int best = 0;
  double best_d = fabs(a - g_table[0]);
  for (int c = 1; c < 127; ++c) {
    double d = fabs(a - g_table[c]);
    if (d < best_d || (d == best_d && (c % 2 == 0))) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(best | (sign << 7));
}

/* ------------------------------------------------------------------------ */
/* A second, independent encoder working on the fp32 bit fields, used only  */
/* to pin orc_e4m3_encode over all 2^32 inputs.                              */
/* ------------------------------------------------------------------------ */
uint8_t orc_e4m3_encode_bits(uint32_t u) {
  uint32_t sign = (u >> 31) << 7;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7F);         /* NaN */
  if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7E);        /* >= 448 */
  uint32_t E = a >> 23;
  if (E >= 121) {                                              /* >= 2^-6 */
    /* Keep 3 of the 23 mantissa bits with RNE on the integer E:M, then move
     * the exponent bias from 127 to 7. A carry out of the mantissa bumps the
     * exponent, as it should. */
    uint32_t keep = a >> 20;
    uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep += 1;
    return (uint8_t)(sign | (keep - (120u << 3)));
  }
  if (E == 0) return (uint8_t)sign;                            /* fp32 subnormal */
  /* Below 2^-6: multiples of 2^-9. k = RNE(value * 2^9), value * 2^9 =
   * (2^23 + M) * 2^(E - 141). k = 8 is the smallest normal, code 0x08. */
  uint32_t mant = (1u << 23) | (a & 0x7FFFFFu);
  uint32_t shift = 141u - E;                                   /* >= 21 */
  if (shift >= 32) return (uint8_t)sign;
  uint32_t k = mant >> shift;
  uint32_t r = mant & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (r > half || (r == half && (k & 1u))) k += 1;
  return (uint8_t)(sign | k);
}

/* Exhaustive comparison of the two encoders over [lo, hi) of the 32-bit
 * patterns, threaded. Returns the number of disagreements; the first one is
 * written to *first_bad (if any). */
typedef struct {
  uint64_t lo, hi, bad, first;
} sweep_job;

static void* sweep_worker(void* p) {
  sweep_job* j = (sweep_job*)p;
  j->bad = 0;
  j->first = UINT64_MAX;
  for (uint64_t u = j->lo; u < j->hi; ++u) {
    float f;
    uint32_t b = (uint32_t)u;
    memcpy(&f, &b, 4);
    if (orc_e4m3_encode(f) != orc_e4m3_encode_bits(b)) {
      if (j->bad == 0) j->first = u;
      j->bad++;
    }
  }
  return NULL;
}

uint64_t orc_sweep_encoders(uint64_t lo, uint64_t hi, int nthreads,
                            uint64_t* first_bad) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  sweep_job jobs[256];
  uint64_t n = hi - lo;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].lo = lo + n * (uint64_t)i / (uint64_t)nthreads;
    jobs[i].hi = lo + n * (uint64_t)(i + 1) / (uint64_t)nthreads;
    pthread_create(&th[i], NULL, sweep_worker, &jobs[i]);
  }
  uint64_t bad = 0, first = UINT64_MAX;
  for (int i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    bad += jobs[i].bad;
    if (jobs[i].first < first) first = jobs[i].first;
  }
  if (first_bad) *first_bad = first;
  return bad;
}

/* ------------------------------------------------------------------------ */
/* E5M2 decode: the OCP definition written out.                              */
/* ------------------------------------------------------------------------ */
double orc_e5m2_decode(uint8_t c) {
  int s = c >> 7;
  int e = (c >> 2) & 31;
  int m = c & 3;
  double mag;
  if (e == 31) {
    if (m != 0) return NAN;                        /* S.11111.xx */
    mag = INFINITY;                                /* S.11111.00 */
  } else if (e == 0) {
    mag = ldexp((double)m, -16);                   /* m/4 * 2^(1-15) */
  } else {
    mag = ldexp((double)(4 + m), e - 17);          /* (1+m/4) * 2^(e-15) */
  }
  return s ? -mag : mag;
}

void orc_e5m2_decode_all(double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = orc_e5m2_decode((uint8_t)c);
}

/* E5M2 encode, saturating, round-to-nearest-even: nearest of the 124
 * non-negative finite values (codes 0x00..0x7B, increasing with the code),
 * an exact midpoint to the even code; |y| >= 57344 and Inf give 0x7B, NaN
 * gives 0x7F with the sign of y. */
static double g_table5[124];
static pthread_once_t g_table5_once = PTHREAD_ONCE_INIT;

static void build_table5(void) {
  for (int c = 0; c < 124; ++c) g_table5[c] = orc_e5m2_decode((uint8_t)c);
}

uint8_t orc_e5m2_encode(float y) {
  pthread_once(&g_table5_once, build_table5);
  uint32_t sign = f32_bits(y) >> 31;
  if (isnan(y)) return (uint8_t)(0x7F | (sign << 7));
  double a = fabs((double)y);
  int code;
  if (a >= g_table5[123]) {
    code = 123;                                    /* saturate, Inf too */
  } else {
    int lo = 0, hi = 123;                          /* g_table5[lo] <= a < g_table5[hi] */
    while (hi - lo > 1) {
      int mid = (lo + hi) / 2;
      if (g_table5[mid] <= a) lo = mid; else hi = mid;
    }
    double below = g_table5[lo], above = g_table5[hi];
    double mid = 0.5 * (below + above);            /* exact in double */
    if (a < mid) code = lo;
    else if (a > mid) code = hi;
    else code = (lo % 2 == 0) ? lo : hi;
  }
  return (uint8_t)(code | (sign << 7));
}

/* The same definition by a linear scan (samples only). */
uint8_t orc_e5m2_encode_scan(float y) {
  pthread_once(&g_table5_once, build_table5);
  uint32_t sign = f32_bits(y) >> 31;
  if (isnan(y)) return (uint8_t)(0x7F | (sign << 7));
  double a = fabs((double)y);
  if (a > g_table5[123]) a = g_table5[123];
  int best = 0;
  double best_d = fabs(a - g_table5[0]);
  for (int c = 1; c < 124; ++c) {
    double d = fabs(a - g_table5[c]);
    if (d < best_d || (d == best_d && (c % 2 == 0))) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(best | (sign << 7));
}

/* A second, independent E5M2 encoder on the fp32 bit fields (pins the
 * table encoder over all 2^32 inputs). */
uint8_t orc_e5m2_encode_bits(uint32_t u) {
  uint32_t sign = (u >> 31) << 7;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7F);         /* NaN */
  if (a >= 0x47600000u) return (uint8_t)(sign | 0x7B);        /* >= 57344, Inf */
  uint32_t E = a >> 23;
  if (E >= 113) {                                              /* >= 2^-14 */
    /* Keep 2 of the 23 mantissa bits with RNE on the integer E:M, then move
     * the exponent bias from 127 to 15. */
    uint32_t keep = a >> 21;
    uint32_t rem = a & 0x1FFFFFu;
    if (rem > 0x100000u || (rem == 0x100000u && (keep & 1u))) keep += 1;
    return (uint8_t)(sign | (keep - (112u << 2)));
  }
  if (E == 0) return (uint8_t)sign;                            /* fp32 subnormal */
  /* Below 2^-14: multiples of 2^-16. k = RNE(value * 2^16), value * 2^16 =
   * (2^23 + M) * 2^(E - 134). k = 4 is the smallest normal, code 0x04. */
  uint32_t mant = (1u << 23) | (a & 0x7FFFFFu);
  uint32_t shift = 134u - E;                                   /* >= 22 */
  if (shift >= 32) return (uint8_t)sign;
  uint32_t k = mant >> shift;
  uint32_t r = mant & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (r > half || (r == half && (k & 1u))) k += 1;
  return (uint8_t)(sign | k);
}

typedef struct {
  uint64_t lo, hi, bad, first;
} sweep5_job;

static void* sweep5_worker(void* p) {
  sweep5_job* j = (sweep5_job*)p;
  j->bad = 0;
  j->first = UINT64_MAX;
  for (uint64_t u = j->lo; u < j->hi; ++u) {
    float f;
    uint32_t b = (uint32_t)u;
    memcpy(&f, &b, 4);
    if (orc_e5m2_encode(f) != orc_e5m2_encode_bits(b)) {
      if (j->bad == 0) j->first = u;
      j->bad++;
    }
  }
  return NULL;
}

uint64_t orc_sweep_encoders_e5m2(uint64_t lo, uint64_t hi, int nthreads,
                                 uint64_t* first_bad) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  sweep5_job jobs[256];
  uint64_t n = hi - lo;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].lo = lo + n * (uint64_t)i / (uint64_t)nthreads;
    jobs[i].hi = lo + n * (uint64_t)(i + 1) / (uint64_t)nthreads;
    pthread_create(&th[i], NULL, sweep5_worker, &jobs[i]);
  }
  uint64_t bad = 0, first = UINT64_MAX;
  for (int i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    bad += jobs[i].bad;
    if (jobs[i].first < first) first = jobs[i].first;
  }
  if (first_bad) *first_bad = first;
  return bad;
}

/* ------------------------------------------------------------------------ */
/* Quantisation: code = E4M3_sat_RNE( fp32(x) / s ), fp32 IEEE division.     */
/* ------------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint8_t orc_quantize_f32(float x, float s) {
  volatile float y = x / s;                        /* one correctly rounded divide */
  return orc_e4m3_encode(y);
}

/* The same quantisation into either format: fmt 1 = E4M3, 2 = E5M2. */
uint8_t orc_quantize_fmt(int fmt, float x, float s) {
  volatile float y = x / s;
  return fmt == 2 ? orc_e5m2_encode(y) : orc_e4m3_encode(y);
}

void orc_quantize_f32_array(const float* x, int64_t n, float s, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_quantize_f32(x[i], s);
}

/* Threaded variant for large arrays (same per-element definition). */
typedef struct {
  const float* x;
  int64_t lo, hi;
  float s;
  int fmt;
  uint8_t* out;
} qjob;

static void* quant_worker(void* p) {
  qjob* j = (qjob*)p;
  for (int64_t i = j->lo; i < j->hi; ++i) j->out[i] = orc_quantize_fmt(j->fmt, j->x[i], j->s);
  return NULL;
}

void orc_quantize_fmt_array_mt(int fmt, const float* x, int64_t n, float s, uint8_t* out,
                               int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  qjob jobs[256];
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].x = x;
    jobs[i].lo = n * (int64_t)i / nthreads;
    jobs[i].hi = n * (int64_t)(i + 1) / nthreads;
    jobs[i].s = s;
    jobs[i].fmt = fmt;
    jobs[i].out = out;
    pthread_create(&th[i], NULL, quant_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

void orc_quantize_f32_array_mt(const float* x, int64_t n, float s, uint8_t* out,
                               int nthreads) {
  orc_quantize_fmt_array_mt(1, x, n, s, out, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Scale calibration: s = fp32(amax) / 448 over one KV head (or the tensor). */
/* ------------------------------------------------------------------------ */
/* s = fp32(amax) / fmax, fmax = 448 (E4M3, fmt 1) or 57344 (E5M2, fmt 2):
 * the largest value lands on the format's largest finite value. */
void orc_scale_from_amax_fmt(const uint16_t* x, int64_t T, int H, int D,
                             int per_head, int fmt, float* out) {
  const float fmax = fmt == 2 ? 57344.0f : 448.0f;
  int nout = per_head ? H : 1;
  for (int o = 0; o < nout; ++o) {
    double amax = 0.0;
    int saw_nan = 0;
    for (int64_t t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h) {
        if (per_head && h != o) continue;
        for (int d = 0; d < D; ++d) {
          double v = (double)bf16_to_f32(x[(t * H + h) * D + d]);
          if (isnan(v)) saw_nan = 1;
          else if (fabs(v) > amax) amax = fabs(v);
        }
      }
    if (saw_nan) out[o] = NAN;
    else if (amax == 0.0) out[o] = 1.0f;
    else {
      volatile float a = (float)amax;              /* exact: a bf16 value or Inf */
      out[o] = a / fmax;
    }
  }
}

void orc_scale_from_amax(const uint16_t* x, int64_t T, int H, int D,
                         int per_head, float* out) {
  orc_scale_from_amax_fmt(x, T, H, D, per_head, 1, out);
}

/* ------------------------------------------------------------------------ */
/* Cache layout (as documented in the library header, written out here on   */
/* its own): byte offset of element (row r, dim d) inside the block of one   */
/* (page, kv head); e = bytes per element.                                   */
/* ------------------------------------------------------------------------ */
int64_t orc_k_offset(int r, int d, int e) {
  int ce = 16 / e;
  return ((int64_t)(d / ce) * 16 + r) * 16 + (int64_t)(d % ce) * e;
}

int64_t orc_v_offset(int r, int d, int e) {
  int db = 64 / e;
  return (int64_t)(d / db) * 1024 + (int64_t)(r / 4) * 256 +
         (int64_t)(d % db) * 4 * e + (int64_t)(r % 4) * e;
}

/* Cache write. k, v: bf16 bits [T][H][D]. dtype 1 = fp8 e4m3, 2 = fp8 e5m2,
 * 0 = bf16. Scales are read at index h when per_head, else index 0. */
void orc_kv_cache_write(int H, int D, int dtype, int per_head,
                        const uint16_t* k, const uint16_t* v,
                        const int64_t* slots, int64_t T, uint8_t* kc,
                        uint8_t* vc, int64_t num_pages, const float* ks,
                        const float* vs) {
  int e = dtype == 0 ? 2 : 1;
  int64_t pb = 16LL * D * e;
  for (int64_t t = 0; t < T; ++t) {
    int64_t slot = slots[t];
    if (slot < 0) continue;
    int64_t page = slot / 16;
    int r = (int)(slot % 16);
    if (page >= num_pages) continue;
    for (int h = 0; h < H; ++h) {
      uint8_t* kb = kc + (page * H + h) * pb;
      uint8_t* vb = vc + (page * H + h) * pb;
      for (int d = 0; d < D; ++d) {
        uint16_t kx = k[(t * H + h) * D + d];
        uint16_t vx = v[(t * H + h) * D + d];
        if (dtype != 0) {
          float sk = ks[per_head ? h : 0], sv = vs[per_head ? h : 0];
          kb[orc_k_offset(r, d, 1)] = orc_quantize_fmt(dtype, bf16_to_f32(kx), sk);
          vb[orc_v_offset(r, d, 1)] = orc_quantize_fmt(dtype, bf16_to_f32(vx), sv);
        } else {
          int64_t ko = orc_k_offset(r, d, 2), vo = orc_v_offset(r, d, 2);
          kb[ko] = (uint8_t)(kx & 0xFF);
          kb[ko + 1] = (uint8_t)(kx >> 8);
          vb[vo] = (uint8_t)(vx & 0xFF);
          vb[vo + 1] = (uint8_t)(vx >> 8);
        }
      }
    }
  }
}

/* Threaded cache write: tokens are split across threads; each token is
 * written exactly as orc_kv_cache_write writes it. Tokens sharing a slot
 * must not be split across threads (callers pass distinct slots). */
typedef struct {
  int H, D, dtype, per_head;
  const uint16_t *k, *v;
  const int64_t* slots;
  int64_t lo, hi;
  uint8_t *kc, *vc;
  int64_t num_pages;
  const float *ks, *vs;
} wjob;

static void* write_worker(void* p) {
  wjob* j = (wjob*)p;
  int64_t off = j->lo * j->H * j->D;
  orc_kv_cache_write(j->H, j->D, j->dtype, j->per_head, j->k + off, j->v + off,
                     j->slots + j->lo, j->hi - j->lo, j->kc, j->vc, j->num_pages,
                     j->ks, j->vs);
  return NULL;
}

void orc_kv_cache_write_mt(int H, int D, int dtype, int per_head,
                           const uint16_t* k, const uint16_t* v,
                           const int64_t* slots, int64_t T, uint8_t* kc,
                           uint8_t* vc, int64_t num_pages, const float* ks,
                           const float* vs, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (T < 4096) nthreads = 1;
  pthread_t th[256];
  wjob jobs[256];
  for (int i = 0; i < nthreads; ++i) {
    wjob w = {H, D, dtype, per_head, k, v, slots, T * i / nthreads,
              T * (i + 1) / nthreads, kc, vc, num_pages, ks, vs};
    jobs[i] = w;
    pthread_create(&th[i], NULL, write_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* Cache write with dynamic per-token scales ("FP8量化与长上下文推理" section
 * 2.2: every new token gets its own scale; "cooking-agi", section "dynamic
 * vs static scale": each token's largest magnitude lands on the format's
 * largest value). mode 2: one scale per token over all H*D of its values;
 * mode 3: one per (token, KV head) over D values; K and V separately. The
 * scale follows the static calibration rule (orc_scale_from_amax_fmt: amax
 * / fmax, 1 for an all-zero set, NaN if a NaN is present) and is stored for
 * slot (page, r) of head h at pool[(page * H + h) * 16 + r]; the codes are
 * then those of the static write with that scale. bf16 layers copy and
 * leave the pools alone. */
void orc_kv_cache_write_dyn(int H, int D, int dtype, int mode, const uint16_t* k,
                            const uint16_t* v, const int64_t* slots, int64_t T,
                            uint8_t* kc, uint8_t* vc, int64_t num_pages, float* ks_pool,
                            float* vs_pool) {
  float sk[256], sv[256];   /* H <= 256, the library's limit for these modes */
  for (int64_t t = 0; t < T; ++t) {
    int64_t slot = slots[t];
    if (slot < 0 || slot / 16 >= num_pages) continue;
    const uint16_t* kt = k + t * H * D;
    const uint16_t* vt = v + t * H * D;
    if (dtype != 0) {
      orc_scale_from_amax_fmt(kt, 1, H, D, mode == 3, dtype, sk);
      orc_scale_from_amax_fmt(vt, 1, H, D, mode == 3, dtype, sv);
      if (mode != 3)
        for (int h = 1; h < H; ++h) {
          sk[h] = sk[0];
          sv[h] = sv[0];
        }
      int64_t page = slot / 16;
      int r = (int)(slot % 16);
      for (int h = 0; h < H; ++h) {
        ks_pool[(page * H + h) * 16 + r] = sk[h];
        vs_pool[(page * H + h) * 16 + r] = sv[h];
      }
    }
    orc_kv_cache_write(H, D, dtype, 1, kt, vt, &slots[t], 1, kc, vc, num_pages, sk, sv);
  }
}

typedef struct {
  int H, D, dtype, mode;
  const uint16_t *k, *v;
  const int64_t* slots;
  int64_t lo, hi;
  uint8_t *kc, *vc;
  int64_t num_pages;
  float *ks, *vs;
} dwjob;

static void* dyn_write_worker(void* p) {
  dwjob* j = (dwjob*)p;
  int64_t off = j->lo * j->H * j->D;
  orc_kv_cache_write_dyn(j->H, j->D, j->dtype, j->mode, j->k + off, j->v + off,
                         j->slots + j->lo, j->hi - j->lo, j->kc, j->vc, j->num_pages,
                         j->ks, j->vs);
  return NULL;
}

/* Threaded: tokens split across threads (callers pass distinct slots). */
void orc_kv_cache_write_dyn_mt(int H, int D, int dtype, int mode, const uint16_t* k,
                               const uint16_t* v, const int64_t* slots, int64_t T,
                               uint8_t* kc, uint8_t* vc, int64_t num_pages, float* ks_pool,
                               float* vs_pool, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (T < 4096) nthreads = 1;
  pthread_t th[256];
  dwjob jobs[256];
  for (int i = 0; i < nthreads; ++i) {
    dwjob w = {H, D, dtype, mode, k, v, slots, T * i / nthreads, T * (i + 1) / nthreads,
               kc, vc, num_pages, ks_pool, vs_pool};
    jobs[i] = w;
    pthread_create(&th[i], NULL, dyn_write_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* Dequantised element (float64) of the K or V cache. */
static double cache_value(const uint8_t* cache, int is_v, int64_t page, int H,
                          int h, int r, int d, int D, int dtype, double scale) {
  int e = dtype == 0 ? 2 : 1;
  int64_t pb = 16LL * D * e;
  const uint8_t* blk = cache + (page * H + h) * pb;
  int64_t off = is_v ? orc_v_offset(r, d, e) : orc_k_offset(r, d, e);
  if (dtype == 1) return orc_e4m3_decode(blk[off]) * scale;
  if (dtype == 2) return orc_e5m2_decode(blk[off]) * scale;
  uint16_t bits = (uint16_t)(blk[off] | (blk[off + 1] << 8));
  return (double)bf16_to_f32(bits);
}

/* ------------------------------------------------------------------------ */
/* Attention.                                                                */
/* ------------------------------------------------------------------------ */
typedef struct {
  int B, Hq, Hkv, D, dtype, per_head, window;
  double sm_scale;
  const uint16_t* q;
  const uint8_t *kc, *vc;
  const int32_t* bt;
  int max_pages;
  const int32_t* lens;
  const float *ks, *vs;
  double* out;
  /* split variant */
  int part_tokens;
  /* reduced-precision accumulation variant */
  int acc_bits, acc_tile;
  /* all-FP8 attention variant: q quantised to e4m3 in gather */
  int q8;
} att_args;

/* Softmax-weighted sum over n positions: out[d] = sum_t p_t v[t][d] / sum p,
 * p_t = exp(z_t - max z). The max skips NaN logits; a NaN logit makes its
 * p_t NaN, and so the whole output. */
void orc_softmax_weighted_sum(const double* z, const double* v, int64_t n,
                              int D, double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n <= 0) return;
  double m = -INFINITY;
  for (int64_t t = 0; t < n; ++t)
    if (z[t] > m) m = z[t];
  double l = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    double p = exp(z[t] - m);
    l += p;
    for (int d = 0; d < D; ++d) out[d] += p * v[t * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] /= l;
}

/* Gather the attended window of one (sequence, query head): logits z and
 * dequantised values v (float64). Returns the window length n. */
static int64_t gather_at(const att_args* a, int b, int i, int64_t L, const uint16_t* qi,
                         double* z, double* v) {
  int G = a->Hq / a->Hkv;
  int h = i / G;
  if (L <= 0) return 0;
  int64_t lo = (a->window > 0 && L > a->window) ? L - a->window : 0;
  /* per_head: 0 per tensor, 1 per KV head, 2 / 3 dynamic (per-slot pools) */
  double ks = a->dtype != 0 && a->per_head < 2 ? (double)a->ks[a->per_head ? h : 0] : 1.0;
  double vs = a->dtype != 0 && a->per_head < 2 ? (double)a->vs[a->per_head ? h : 0] : 1.0;
  /* the query as the attention reads it: its bf16 values, or (all-FP8
   * variant) their e4m3 codes times the row's scale */
  double qv[512];
  if (a->q8) {
    float sq = 0.0f;
    uint16_t qrow[1][1][512];
    for (int d = 0; d < a->D; ++d) qrow[0][0][d] = qi[d];
    orc_scale_from_amax_fmt(&qrow[0][0][0], 1, 1, a->D, 1, 1, &sq);
    for (int d = 0; d < a->D; ++d)
      qv[d] = orc_e4m3_decode(orc_quantize_f32(bf16_to_f32(qi[d]), sq)) * (double)sq;
  } else {
    for (int d = 0; d < a->D; ++d) qv[d] = (double)bf16_to_f32(qi[d]);
  }
  for (int64_t t = lo; t < L; ++t) {
    int64_t page = a->bt[(int64_t)b * a->max_pages + t / 16];
    int r = (int)(t % 16);
    if (a->dtype != 0 && a->per_head >= 2) {     /* dynamic: the slot's own scales */
      ks = (double)a->ks[(page * a->Hkv + h) * 16 + r];
      vs = (double)a->vs[(page * a->Hkv + h) * 16 + r];
    }
    double dot = 0.0;
    for (int d = 0; d < a->D; ++d) {
      double kh = cache_value(a->kc, 0, page, a->Hkv, h, r, d, a->D, a->dtype, ks);
      dot += qv[d] * kh;
      v[(t - lo) * a->D + d] =
          cache_value(a->vc, 1, page, a->Hkv, h, r, d, a->D, a->dtype, vs);
    }
    z[t - lo] = a->sm_scale * dot;
  }
  return L - lo;
}

static int64_t gather(const att_args* a, int b, int i, double* z, double* v) {
  return gather_at(a, b, i, a->lens[b], a->q + ((int64_t)b * a->Hq + i) * a->D, z, v);
}

typedef struct {
  const att_args* a;
  int lo, hi; /* range of (b, i) pairs */
  int mode;   /* 0 plain, 1 split-merge, 2 reduced-precision accumulation */
} att_job;

/* Split the window into partitions of part_tokens positions, compute
 * (m_p, l_p, o_p) per partition and merge them:
 *   M = max m_p, w_p = exp(m_p - M), out = sum w_p o_p / sum w_p l_p. */
static void split_merge(const double* z, const double* v, int64_t n, int D,
                        int part, double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n <= 0) return;
  int64_t np = (n + part - 1) / part;
  double* m = (double*)malloc(sizeof(double) * np);
  double* l = (double*)malloc(sizeof(double) * np);
  double* o = (double*)calloc((size_t)np * D, sizeof(double));
  for (int64_t p = 0; p < np; ++p) {
    int64_t t0 = p * part, t1 = t0 + part < n ? t0 + part : n;
    m[p] = -INFINITY;
    for (int64_t t = t0; t < t1; ++t)
      if (z[t] > m[p]) m[p] = z[t];
    l[p] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      double w = exp(z[t] - m[p]);
      l[p] += w;
      for (int d = 0; d < D; ++d) o[p * D + d] += w * v[t * D + d];
    }
  }
  double M = -INFINITY;
  for (int64_t p = 0; p < np; ++p)
    if (m[p] > M) M = m[p];
  double Lam = 0.0;
  for (int64_t p = 0; p < np; ++p) {
    double w = exp(m[p] - M);
    Lam += w * l[p];
    for (int d = 0; d < D; ++d) out[d] += w * o[p * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] /= Lam;
  free(m);
  free(l);
  free(o);
}

/* Round x to `bits` significand bits by truncation toward zero: a model of an
 * accumulator that keeps fewer bits than FP32 ("cooking-agi", section on
 * training recipes: FP8 GEMM accumulation on H800 keeps about 14 bits). */
static double trunc_bits(double x, int bits) {
  if (x == 0.0 || !isfinite(x)) return x;
  int ex;
  double f = frexp(x, &ex);                          /* x = f * 2^ex, |f| in [0.5,1) */
  double scale = ldexp(1.0, bits);
  f = trunc(f * scale) / scale;
  return ldexp(f, ex);
}

/* Negative control: the P*V sum and the normaliser accumulated in one level
 * with `bits` significand bits (tile <= 0), or in tiles of `tile` positions
 * with `bits` bits inside a tile and each tile promoted into a float64 sum
 * (tile > 0): a model of two-level accumulation. */
static void lowprec_sum(const double* z, const double* v, int64_t n, int D,
                        int bits, int tile, double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n <= 0) return;
  double m = -INFINITY;
  for (int64_t t = 0; t < n; ++t)
    if (z[t] > m) m = z[t];
  double* acc = (double*)calloc((size_t)D, sizeof(double));
  double* tacc = (double*)calloc((size_t)D, sizeof(double));
  double l = 0.0, tl = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    double p = exp(z[t] - m);
    if (tile > 0) {
      tl = trunc_bits(tl + p, bits);
      for (int d = 0; d < D; ++d) tacc[d] = trunc_bits(tacc[d] + p * v[t * D + d], bits);
      if ((t + 1) % tile == 0 || t + 1 == n) {
        l += tl;
        tl = 0.0;
        for (int d = 0; d < D; ++d) {
          acc[d] += tacc[d];
          tacc[d] = 0.0;
        }
      }
    } else {
      l = trunc_bits(l + p, bits);
      for (int d = 0; d < D; ++d) acc[d] = trunc_bits(acc[d] + p * v[t * D + d], bits);
    }
  }
  for (int d = 0; d < D; ++d) out[d] = acc[d] / l;
  free(acc);
  free(tacc);
}

/* All-FP8 attention (the FP8 ScoreV product): the attended positions fall
 * into aligned blocks of 32 (block j holds positions 32j .. 32j+31). In
 * block j, with M_j the largest logit of its attended positions,
 *   p~_t = E4M3_sat_RNE( fp32(exp(z_t - M_j)) )        (the quantised P)
 *   S_j  = sum_t p~_t v_t,   L_j = sum_t exp(z_t - M_j)   (P unquantised)
 * and with M = max_j M_j:  out = sum_j e^(M_j-M) S_j / sum_j e^(M_j-M) L_j.
 * lo is the first attended position (the window start), z and v are indexed
 * from it. */
static void fp8attn_sum(const double* z, const double* v, int64_t n, int64_t lo,
                        int D, double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n <= 0) return;
  int64_t j0 = lo / 32, j1 = (lo + n - 1) / 32;
  int64_t nb = j1 - j0 + 1;
  double* mb = (double*)malloc(sizeof(double) * nb);
  double* lb = (double*)malloc(sizeof(double) * nb);
  double* sb = (double*)calloc((size_t)nb * D, sizeof(double));
  for (int64_t j = 0; j < nb; ++j) {
    int64_t t0 = (j0 + j) * 32 - lo, t1 = t0 + 32;
    if (t0 < 0) t0 = 0;
    if (t1 > n) t1 = n;
    mb[j] = -INFINITY;
    for (int64_t t = t0; t < t1; ++t)
      if (z[t] > mb[j]) mb[j] = z[t];
    lb[j] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      double e = exp(z[t] - mb[j]);
      lb[j] += e;
      double pq = orc_e4m3_decode(orc_e4m3_encode((float)e));
      for (int d = 0; d < D; ++d) sb[j * D + d] += pq * v[t * D + d];
    }
  }
  double M = -INFINITY;
  for (int64_t j = 0; j < nb; ++j)
    if (mb[j] > M) M = mb[j];
  double Lam = 0.0;
  for (int64_t j = 0; j < nb; ++j) {
    double w = exp(mb[j] - M);
    Lam += w * lb[j];
    for (int d = 0; d < D; ++d) out[d] += w * sb[j * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] /= Lam;
  free(mb);
  free(lb);
  free(sb);
}

static void* att_worker(void* p) {
  att_job* j = (att_job*)p;
  const att_args* a = j->a;
  int64_t maxn = 0;
  for (int b = 0; b < a->B; ++b)
    if (a->lens[b] > maxn) maxn = a->lens[b];
  double* z = (double*)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1));
  double* v = (double*)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1) * a->D);
  for (int idx = j->lo; idx < j->hi; ++idx) {
    int b = idx / a->Hq, i = idx % a->Hq;
    double* out = a->out + (int64_t)idx * a->D;
    int64_t n = gather(a, b, i, z, v);
    int64_t L = a->lens[b];
    int64_t lo = (a->window > 0 && L > a->window) ? L - a->window : 0;
    if (j->mode == 3)
      fp8attn_sum(z, v, n, lo, a->D, out);
    else if (j->mode == 0)
      orc_softmax_weighted_sum(z, v, n, a->D, out);
    else if (j->mode == 1)
      split_merge(z, v, n, a->D, a->part_tokens, out);
    else
      lowprec_sum(z, v, n, a->D, a->acc_bits, a->acc_tile, out);
  }
  free(z);
  free(v);
  return NULL;
}

static void run_attention(att_args* a, int mode, int nthreads) {
  int total = a->B * a->Hq;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > total) nthreads = total > 0 ? total : 1;
  pthread_t th[256];
  att_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].a = a;
    jobs[t].lo = total * t / nthreads;
    jobs[t].hi = total * (t + 1) / nthreads;
    jobs[t].mode = mode;
    pthread_create(&th[t], NULL, att_worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

static void fill_args(att_args* a, int B, int Hq, int Hkv, int D, int dtype,
                      int per_head, int window, double sm_scale,
                      const uint16_t* q, const uint8_t* kc, const uint8_t* vc,
                      const int32_t* bt, int max_pages, const int32_t* lens,
                      const float* ks, const float* vs, double* out) {
  a->B = B; a->Hq = Hq; a->Hkv = Hkv; a->D = D; a->dtype = dtype;
  a->per_head = per_head; a->window = window;
  a->sm_scale = sm_scale > 0.0 ? sm_scale : 1.0 / sqrt((double)D);
  a->q = q; a->kc = kc; a->vc = vc; a->bt = bt; a->max_pages = max_pages;
  a->lens = lens; a->ks = ks; a->vs = vs; a->out = out;
  a->part_tokens = 0; a->acc_bits = 0; a->acc_tile = 0; a->q8 = 0;
}

/* out: float64 [B][Hq][D]. sm_scale <= 0 means 1/sqrt(D). */
void orc_attention(int B, int Hq, int Hkv, int D, int dtype, int per_head,
                   int window, double sm_scale, const uint16_t* q,
                   const uint8_t* kc, const uint8_t* vc, const int32_t* bt,
                   int max_pages, const int32_t* lens, const float* ks,
                   const float* vs, double* out, int nthreads) {
  att_args a;
  fill_args(&a, B, Hq, Hkv, D, dtype, per_head, window, sm_scale, q, kc, vc, bt,
            max_pages, lens, ks, vs, out);
  run_attention(&a, 0, nthreads);
}

void orc_attention_split(int B, int Hq, int Hkv, int D, int dtype, int per_head,
                         int window, double sm_scale, const uint16_t* q,
                         const uint8_t* kc, const uint8_t* vc, const int32_t* bt,
                         int max_pages, const int32_t* lens, const float* ks,
                         const float* vs, double* out, int part_tokens,
                         int nthreads) {
  att_args a;
  fill_args(&a, B, Hq, Hkv, D, dtype, per_head, window, sm_scale, q, kc, vc, bt,
            max_pages, lens, ks, vs, out);
  a.part_tokens = part_tokens > 0 ? part_tokens : 1;
  run_attention(&a, 1, nthreads);
}

void orc_attention_lowprec(int B, int Hq, int Hkv, int D, int dtype,
                           int per_head, int window, double sm_scale,
                           const uint16_t* q, const uint8_t* kc,
                           const uint8_t* vc, const int32_t* bt, int max_pages,
                           const int32_t* lens, const float* ks,
                           const float* vs, double* out, int acc_bits,
                           int acc_tile, int nthreads) {
  att_args a;
  fill_args(&a, B, Hq, Hkv, D, dtype, per_head, window, sm_scale, q, kc, vc, bt,
            max_pages, lens, ks, vs, out);
  a.acc_bits = acc_bits;
  a.acc_tile = acc_tile;
  run_attention(&a, 2, nthreads);
}

/* Prefill (chunked prefill) attention: the causal self-attention of a chunk
 * of new tokens over the paged cache ("State of FP8 KV cache and attention
 * quantization in vLLM", section "Single-request benchmark": prefill is the
 * compute-bound phase, self-attention over the input, quadratic in its
 * length). Sequence b's n_b = qs[b+1] - qs[b] query rows are its last n_b
 * written positions: row j sits at position pos = lens[b] - n_b + j and
 * attends to [lo, pos] (lo = max(0, pos + 1 - W) with a window W), i.e. it
 * is the decode attention of a context of pos + 1 positions. Rows are taken
 * one (row, head) at a time; `rows` (n_rows entries, or NULL for all T) picks
 * which rows to compute, and out is [n_rows][Hq][D]. A row whose position
 * falls before 0 gives zeros. */
typedef struct {
  const att_args* a;
  const int32_t* qs;
  const int32_t* rows;
  int64_t lo, hi;        /* range of (row index, head) pairs */
  int fp8attn;           /* the all-FP8 arithmetic (fp8attn_sum, q quantised) */
} pf_job;

static void fp8attn_sum(const double* z, const double* v, int64_t n, int64_t lo, int D,
                        double* out);

static void* prefill_worker(void* p) {
  pf_job* j = (pf_job*)p;
  const att_args* a = j->a;
  int64_t maxn = 0;
  for (int b = 0; b < a->B; ++b)
    if (a->lens[b] > maxn) maxn = a->lens[b];
  double* z = (double*)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1));
  double* v = (double*)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1) * a->D);
  for (int64_t idx = j->lo; idx < j->hi; ++idx) {
    int64_t ri = idx / a->Hq;
    int i = (int)(idx % a->Hq);
    int64_t row = j->rows ? j->rows[ri] : ri;
    int b = 0;
    while (b + 1 < a->B && j->qs[b + 1] <= row) ++b;
    int64_t n = j->qs[b + 1] - j->qs[b];
    int64_t pos = a->lens[b] - n + (row - j->qs[b]);
    double* out = a->out + idx * a->D;
    int64_t cnt = gather_at(a, b, i, pos + 1, a->q + (row * a->Hq + i) * a->D, z, v);
    if (j->fp8attn) {
      int64_t lo = (a->window > 0 && pos + 1 > a->window) ? pos + 1 - a->window : 0;
      fp8attn_sum(z, v, cnt, lo, a->D, out);
    } else {
      orc_softmax_weighted_sum(z, v, cnt, a->D, out);
    }
  }
  free(z);
  free(v);
  return NULL;
}

void orc_prefill_attention(int B, int Hq, int Hkv, int D, int dtype, int per_head, int window,
                           double sm_scale, const uint16_t* q, const uint8_t* kc,
                           const uint8_t* vc, const int32_t* bt, int max_pages,
                           const int32_t* query_start, const int32_t* lens, const float* ks,
                           const float* vs, const int32_t* rows, int64_t n_rows, double* out,
                           int fp8attn, int nthreads) {
  att_args a;
  fill_args(&a, B, Hq, Hkv, D, dtype, per_head, window, sm_scale, q, kc, vc, bt, max_pages,
            lens, ks, vs, out);
  a.q8 = fp8attn ? 1 : 0;
  int64_t total = n_rows * Hq;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > total) nthreads = total > 0 ? (int)total : 1;
  pthread_t th[256];
  pf_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].a = &a;
    jobs[t].qs = query_start;
    jobs[t].rows = rows;
    jobs[t].lo = total * t / nthreads;
    jobs[t].hi = total * (t + 1) / nthreads;
    jobs[t].fp8attn = fp8attn;
    pthread_create(&th[t], NULL, prefill_worker, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* All-FP8 attention: q quantised to e4m3 per (sequence, query head) with
 * s_q = fp32(amax |q row|) / 448, the QK^T product on those codes and the
 * cache codes, and P quantised per aligned 32-position block (fp8attn_sum).
 * Sources: "State of FP8 KV cache and attention quantization in vLLM"
 * (introduction: the whole attention, QK and ScoreV, in FP8 e4m3; section
 * on fixes: query quantisation fused ahead of the kernel); the scale rule
 * and the block reference are this library's reading. */
void orc_attention_fp8attn(int B, int Hq, int Hkv, int D, int dtype, int per_head,
                           int window, double sm_scale, const uint16_t* q,
                           const uint8_t* kc, const uint8_t* vc, const int32_t* bt,
                           int max_pages, const int32_t* lens, const float* ks,
                           const float* vs, double* out, int nthreads) {
  att_args a;
  fill_args(&a, B, Hq, Hkv, D, dtype, per_head, window, sm_scale, q, kc, vc, bt,
            max_pages, lens, ks, vs, out);
  a.q8 = 1;
  run_attention(&a, 3, nthreads);
}
