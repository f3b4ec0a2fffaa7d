/* Seeded synthetic inputs, host implementation (gcc, OpenMP).
 *
 * Implements the recipe in synth_recipe.md; synth_dev.hip implements the same
 * recipe on the GPU and a GPU test compares their bytes.  Build with
 * -ffp-contract=off so that every fp32 operation rounds once, as on the device.
 * This file encodes random weights only; it decodes nothing and holds none of
 * the MoE layer's arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "blob_pos.h"

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t rng(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

uint64_t synth_key(uint64_t seed, uint64_t kind, uint64_t cfg, uint64_t a, uint64_t b, uint64_t c) {
  return mix64(mix64(seed) ^ (kind << 60) ^ (cfg << 52) ^ (a << 32) ^ (b << 8) ^ c);
}

static inline uint32_t sum16(uint64_t r) {
  return (uint32_t)(r & 0xFFFF) + (uint32_t)((r >> 16) & 0xFFFF) + (uint32_t)((r >> 32) & 0xFFFF) +
         (uint32_t)(r >> 48);
}

/* Irwin-Hall(12) deviate number i of stream key. */
static inline float normal_dev(uint64_t key, uint64_t i) {
  uint32_t s = sum16(rng(key, 3 * i)) + sum16(rng(key, 3 * i + 1)) + sum16(rng(key, 3 * i + 2));
  return (float)((int32_t)s - 393210) * (1.0f / 65536.0f);
}

static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static inline uint16_t bf16_rne_bits(float f) {
  uint32_t u = f2u(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* positive finite v -> E4M3FN byte, round to nearest even, saturating at 448 */
static inline uint8_t e4m3_encode(float v) {
  if (!(v > 0.0f)) return 0;
  if (v < 0.015625f) { /* below 2^-6: subnormal m * 2^-9 */
    float m = rintf(v * 512.0f);
    return (uint8_t)m; /* m == 8 is the smallest normal, byte 0x08 */
  }
  uint32_t u = f2u(v);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20; /* exp8:mant3 */
  int32_t b = (int32_t)r - 960;                          /* rebias 127 -> 7 */
  if (b > 0x7E) b = 0x7E;
  return (uint8_t)b;
}

static inline float e4m3_value(uint8_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return (float)m * (1.0f / 512.0f);
  return u2f(((e + 120u) << 23) | (m << 20));
}

static inline uint8_t e2m1_encode(float q) {
  float a = fabsf(q);
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  if (c != 0 && q < 0.0f) c |= 8;
  return c;
}

float synth_global_scale(uint64_t seed, int cfg, int layer, int expert, int matrix) {
  uint64_t r = rng(synth_key(seed, 2, cfg, layer, expert, matrix), 0);
  float f = 1.0f + (float)(r >> 56) * (1.0f / 256.0f);
  float base = 0.12f / 2688.0f;
  return base * f;
}

/* One matrix (rows x K) of expert (layer, expert), codes and scales placed as
 * blob_pos.h states. */
static void gen_matrix(uint64_t seed, int cfg, int layer, int expert, int m, int rows, int K,
                       uint8_t* codes, uint8_t* scales) {
  uint64_t key = synth_key(seed, 1, cfg, layer, expert, m);
  float G = synth_global_scale(seed, cfg, layer, expert, m);
  float t6 = 6.0f * G;
  int nb = K / 16;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < rows; n++) {
    for (int b = 0; b < nb; b++) {
      float w[16];
      float amax = 0.0f;
      for (int j = 0; j < 16; j++) {
        uint64_t i = (uint64_t)n * (uint64_t)K + (uint64_t)(16 * b + j);
        float z = normal_dev(key, i);
        w[j] = 0.02f * z;
        float a = fabsf(w[j]);
        if (a > amax) amax = a;
      }
      float sv = amax / t6;
      uint8_t sb = e4m3_encode(sv);
      scales[synth_scale_pos((uint64_t)n, b, K)] = sb;
      uint8_t* cp = codes + synth_code_pos((uint64_t)n, b, K);
      if (sb == 0) { memset(cp, 0, 8); continue; }
      float d = e4m3_value(sb) * G;
      for (int j = 0; j < 8; j++) {
        uint8_t lo = e2m1_encode(w[2 * j] / d);
        uint8_t hi = e2m1_encode(w[2 * j + 1] / d);
        cp[j] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* Fill one blob (caller zeroes `out`, which must hold off_globals + 12 bytes). */
void synth_expert_blob(uint64_t seed, int cfg, int layer, int expert, int H, int I,
                       const uint64_t* off_codes, const uint64_t* off_scales, uint64_t off_globals,
                       uint8_t* out) {
  for (int m = 0; m < 3; m++) {
    int rows = m < 2 ? I : H, K = m < 2 ? H : I;
    gen_matrix(seed, cfg, layer, expert, m, rows, K, out + off_codes[m], out + off_scales[m]);
    float G = synth_global_scale(seed, cfg, layer, expert, m);
    memcpy(out + off_globals + 4 * m, &G, 4);
  }
}

/* MX recipe: the same weights w as gen_matrix (stream kind 1); per 32-value
 * block, E8M0 byte sb = (fp32 exponent field of amax) - 2 (0 if that is
 * negative), codes e2m1_encode(w * 2^(127 - sb)), the factor an exact power of
 * two. */
static void gen_matrix_mx(uint64_t seed, int cfg, int layer, int expert, int m, int rows, int K,
                          uint8_t* codes, uint8_t* scales) {
  uint64_t key = synth_key(seed, 1, cfg, layer, expert, m);
  int nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < rows; n++) {
    for (int b = 0; b < nb; b++) {
      float w[32];
      float amax = 0.0f;
      for (int j = 0; j < 32; j++) {
        uint64_t i = (uint64_t)n * (uint64_t)K + (uint64_t)(32 * b + j);
        w[j] = 0.02f * normal_dev(key, i);
        float a = fabsf(w[j]);
        if (a > amax) amax = a;
      }
      uint32_t ef = (f2u(amax) >> 23) & 0xFFu;
      uint8_t sb = ef >= 2 ? (uint8_t)(ef - 2) : 0;
      scales[synth_mx_scale_pos((uint64_t)n, b, K)] = sb;
      float inv = u2f((uint32_t)(254 - sb) << 23);
      for (int h = 0; h < 2; h++) {
        uint8_t* cp = codes + synth_code_pos((uint64_t)n, 2 * b + h, K);
        for (int j = 0; j < 8; j++) {
          uint8_t lo = e2m1_encode(w[16 * h + 2 * j] * inv);
          uint8_t hi = e2m1_encode(w[16 * h + 2 * j + 1] * inv);
          cp[j] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
  }
}

/* Fill one MX blob (caller zeroes `out`). */
void synth_expert_blob_mx(uint64_t seed, int cfg, int layer, int expert, int H, int I,
                          const uint64_t* off_codes, const uint64_t* off_scales, uint8_t* out) {
  for (int m = 0; m < 3; m++) {
    int rows = m < 2 ? I : H, K = m < 2 ? H : I;
    gen_matrix_mx(seed, cfg, layer, expert, m, rows, K, out + off_codes[m], out + off_scales[m]);
  }
}

void synth_x(uint64_t seed, int cfg, int layer, int step, int T, int H, uint16_t* out) {
  uint64_t key = synth_key(seed, 3, cfg, layer, step, 0);
  int64_t n = (int64_t)T * H;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = bf16_rne_bits(normal_dev(key, (uint64_t)i));
}

void synth_w_router(uint64_t seed, int cfg, int layer, int H, int E, float* out) {
  uint64_t key = synth_key(seed, 4, cfg, layer, 0, 0);
  int64_t n = (int64_t)H * E;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = 0.02f * normal_dev(key, (uint64_t)i);
}

void synth_w_shared_gate(uint64_t seed, int cfg, int layer, int H, float* out) {
  uint64_t key = synth_key(seed, 5, cfg, layer, 0, 0);
  for (int i = 0; i < H; i++) out[i] = 0.02f * normal_dev(key, (uint64_t)i);
}
