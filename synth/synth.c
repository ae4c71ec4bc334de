/*
 * Seeded synthetic inputs for the Stable-LatentMoE layer with MXFP4 experts.
 *
 * This file holds only random-number generation and the byte layout of the
 * inputs; it contains none of the layer's arithmetic.  Both the CPU oracle and
 * the GPU path consume arrays produced here, so they always see identical
 * bytes.
 *
 * Generator: a counter-based splitmix64.  The splitmix64 output function
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014; the 64-bit finaliser constants of Stafford's "variant 13") is
 * applied to   base(seed, stream) + (i + 1) * 0x9E3779B97F4A7C15,
 * where base = mix(seed ^ (stream * 0xD1B54A32D192ED03)).  Draw i of a stream
 * therefore depends only on (seed, stream, i), so any slice of a tensor can be
 * generated independently and in parallel without changing a value.
 *
 * Normals use the Box-Muller transform in double precision on draws 2i and
 * 2i+1; the result is scaled by the standard deviation, rounded to float and
 * then to bfloat16 with round-to-nearest-even.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -fopenmp synth.c -o libsynth.so -lm
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define STREAM_MUL 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
  return mix64(seed ^ (stream * STREAM_MUL));
}

static inline uint64_t draw(uint64_t base, uint64_t i) {
  return mix64(base + (i + 1) * GOLDEN);
}

/* uniform in (0, 1]: never 0, so log() is finite */
static inline double unif_open0(uint64_t bits) {
  return ((double)(bits >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}
/* uniform in [0, 1) */
static inline double unif(uint64_t bits) {
  return (double)(bits >> 11) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

uint64_t synth_draw(uint64_t seed, uint64_t stream, uint64_t i) {
  return draw(stream_base(seed, stream), i);
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t i) {
  uint64_t b = stream_base(seed, stream);
  double u1 = unif_open0(draw(b, 2 * i));
  double u2 = unif(draw(b, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* out[j] = bf16(std * N(0,1) draw number (first + j)) for j < n */
void synth_normal_bf16(uint64_t seed, uint64_t stream, double std_dev, uint64_t first, int64_t n,
                       uint16_t* out) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = first + (uint64_t)j;
    double u1 = unif_open0(draw(b, 2 * i));
    double u2 = unif(draw(b, 2 * i + 1));
    double v = std_dev * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
    out[j] = f32_to_bf16_rne((float)v);
  }
}

/* out[j] = byte (first + j) of the stream: byte b of a draw is (draw >> 8b) & 0xFF */
void synth_bytes(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, uint8_t* out) {
  uint64_t b = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = first + (uint64_t)j;
    out[j] = (uint8_t)(draw(b, i >> 3) >> (8 * (i & 7)));
  }
}

/* out[j] = lo + (draw(first + j) mod (hi - lo + 1)), an integer in [lo, hi] stored as a byte */
void synth_int_bytes(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, int lo, int hi,
                     uint8_t* out) {
  uint64_t b = stream_base(seed, stream);
  uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = (uint8_t)(lo + (int)(draw(b, first + (uint64_t)j) % span));
}

/* out[j] = draw(first + j) mod m, for small categorical draws */
void synth_categorical(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, uint32_t m,
                       int32_t* out) {
  uint64_t b = stream_base(seed, stream);
  for (int64_t j = 0; j < n; ++j) out[j] = (int32_t)(draw(b, first + (uint64_t)j) % m);
}

/* a seeded permutation of 0..n-1 by Fisher-Yates, swap partner of i drawn from draw(i) */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t* out) {
  uint64_t b = stream_base(seed, stream);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)(draw(b, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/*
 * Expert blob: num_experts records of rec_bytes each.  Inside a record the
 * gate, up and down matrices follow each other; each matrix stores its code
 * bytes (rows x cols/2) and then its scale bytes (rows x cols/32).  Gate and up
 * are d_ffn x d_latent, down is d_latent x d_ffn.  Code bytes are uniform over
 * 0..255 (both nibbles uniform over the 16 codes), scale bytes uniform over
 * [scale_lo, scale_hi].  Code byte j of matrix m of record e is byte
 * (e*3 + m) * (d_ffn*d_latent/2) + j of the code stream; scale bytes likewise
 * with d_ffn*d_latent/32 per matrix.  Fills records [e0, e0 + ne) into out.
 */
void synth_expert_blob(uint64_t seed, uint64_t code_stream, uint64_t scale_stream, int32_t d_latent,
                       int32_t d_ffn, int32_t e0, int32_t ne, int scale_lo, int scale_hi,
                       uint8_t* out) {
  const int64_t ncode = (int64_t)d_ffn * d_latent / 2;
  const int64_t nscale = (int64_t)d_ffn * d_latent / 32;
  const int64_t mat = ncode + nscale;
  const int64_t rec = 3 * mat;
  for (int32_t e = 0; e < ne; ++e) {
    for (int m = 0; m < 3; ++m) {
      uint8_t* base = out + (int64_t)e * rec + m * mat;
      uint64_t ge = (uint64_t)(e0 + e) * 3 + (uint64_t)m;
      synth_bytes(seed, code_stream, ge * (uint64_t)ncode, ncode, base);
      synth_int_bytes(seed, scale_stream, ge * (uint64_t)nscale, nscale, scale_lo, scale_hi,
                      base + ncode);
    }
  }
}
