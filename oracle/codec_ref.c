/*
 * codec_ref.c — a second, value-based FP8 encoder in plain C (test
 * infrastructure; CPU oracle).  It exists so that the oracle's bit-level
 * encoder (oracle/codec.py, `encode`) can be checked against an independent
 * implementation over every one of the 2^32 fp32 bit patterns in reasonable
 * time.  Nothing in the GPU library loads this file.
 *
 * Formats: the OCP 8-bit floating-point formats ("4.2 Hopper I — Transformer
 * Engine·FP8", §4.2.3 and §4.2.8; "FP8 and low-precision formats", "Deep
 * dive"): E4M3 (bias 7, no infinity, S.1111.111 = NaN, max 448) and E5M2
 * (bias 15, IEEE-like infinities and NaNs, max 57344).
 *
 * Encoding rule (the reading of round_to_fp8 in §4.2.4 used throughout):
 *   NaN          -> sign | 0x7F
 *   |x| > max    -> sign | max code (saturation; infinities included)
 *   otherwise    -> the finite code whose value is nearest to |x|; at an
 *                   exact midpoint, the code with an even last bit; the sign
 *                   bit of x is kept (so -0 and values that round to zero
 *                   keep their sign).
 *
 * Method (unlike the oracle's integer shift-and-round): a table of the values
 * of the non-negative finite codes, decoded from their bit fields; a binary
 * search for the largest value <= |x|; a comparison of |x| with the exact
 * midpoint to the next value.  Every FP8 value has at most 4 significant bits,
 * so each midpoint is exact in double, as is every fp32 value.
 *
 * Build: gcc -O2 -shared -fPIC codec_ref.c -o libcodecref.so
 */
#include <stdint.h>
#include <string.h>

typedef struct {
  int ebits, mbits, bias, max_code, has_inf;
} fmt_t;

static const fmt_t kFormats[2] = {
    {4, 3, 7, 0x7E, 0}, /* E4M3 */
    {5, 2, 15, 0x7B, 1} /* E5M2 */
};

/* Value of a non-negative finite code from its exponent and mantissa fields. */
static double code_value(const fmt_t* f, int code) {
  const int e = code >> f->mbits;
  const int m = code & ((1 << f->mbits) - 1);
  const double frac = (double)m / (double)(1 << f->mbits);
  double v;
  int i;
  if (e == 0) {
    v = frac; /* subnormal: 0.m * 2^(1 - bias) */
    for (i = 0; i < f->bias - 1; ++i) v *= 0.5;
  } else {
    v = 1.0 + frac; /* normal: 1.m * 2^(e - bias) */
    for (i = 0; i < e - f->bias; ++i) v *= 2.0;
    for (i = 0; i < f->bias - e; ++i) v *= 0.5;
  }
  return v;
}

static double g_table[2][128];
static int g_ready[2];

static void make_table(int which) {
  if (g_ready[which]) return;
  for (int c = 0; c <= kFormats[which].max_code; ++c) g_table[which][c] = code_value(&kFormats[which], c);
  g_ready[which] = 1;
}

static uint8_t encode_one(int which, uint32_t bits) {
  const fmt_t* f = &kFormats[which];
  const double* t = g_table[which];
  const uint8_t sign = (uint8_t)((bits >> 31) << 7);
  const uint32_t mag_bits = bits & 0x7FFFFFFFu;
  float xf;
  double v;
  int lo, hi;
  if (mag_bits > 0x7F800000u) return sign | 0x7F; /* NaN */
  memcpy(&xf, &mag_bits, sizeof xf);
  v = (double)xf; /* exact; +Inf stays +Inf */
  if (v > t[f->max_code]) return sign | (uint8_t)f->max_code;
  /* largest code with t[lo] <= v (t[0] = 0 <= v) */
  lo = 0;
  hi = f->max_code;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (t[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  if (t[lo] == v || lo == f->max_code) return sign | (uint8_t)lo;
  {
    const double midpoint = (t[lo] + t[lo + 1]) * 0.5; /* exact */
    int code;
    if (v < midpoint) code = lo;
    else if (v > midpoint) code = lo + 1;
    else code = (lo & 1) ? lo + 1 : lo; /* tie: the even code */
    return sign | (uint8_t)code;
  }
}

/* Encode the bit patterns start, start+1, ..., start+count-1 (wrapping modulo
 * 2^32) as format `which` (0 = E4M3, 1 = E5M2) into out[0 .. count-1].
 * Returns 0, or -1 for an unknown format. */
int fp8ref_encode_range(int which, uint32_t start, uint64_t count, uint8_t* out) {
  uint64_t i;
  if (which != 0 && which != 1) return -1;
  make_table(which);
  for (i = 0; i < count; ++i) out[i] = encode_one(which, (uint32_t)(start + i));
  return 0;
}

/* Encode `count` arbitrary bit patterns. */
int fp8ref_encode_bits(int which, const uint32_t* bits, uint64_t count, uint8_t* out) {
  uint64_t i;
  if (which != 0 && which != 1) return -1;
  make_table(which);
  for (i = 0; i < count; ++i) out[i] = encode_one(which, bits[i]);
  return 0;
}
