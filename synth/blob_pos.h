/* Byte placement of block-FP4 codes and scales inside a blob matrix, shared by
 * the host and device synthetic generators (the format is the expert blob
 * format of include/moe.h).  A matrix of R rows and K columns is stored in
 * blocks of 16 rows; row n, 16-value block b (columns 16 b .. 16 b + 15):
 *   codes: block n / 16 starts at 8 K (n / 16); 32-column chunk j = b / 2 of
 *          its row r = n % 16 is 16 bytes at 256 j + 16 r, block b the
 *          half 8 (b % 2) of them;
 *   scale: block n / 16 starts at K (n / 16); chunks form groups of 16, group
 *          g = j / 16 starts at 512 g and holds L = 2 min(16, K/32 - 16 g)
 *          bytes per row, row r's at L r, scale b at byte b - 32 g of them. */
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define SYNTH_HD __host__ __device__
#else
#define SYNTH_HD
#endif

static inline SYNTH_HD uint64_t synth_code_pos(uint64_t n, int b, int K) {
  return (n >> 4) * 8ull * (uint64_t)K + 256ull * (uint64_t)(b >> 1) + 16ull * (n & 15) + 8ull * (uint64_t)(b & 1);
}

/* MX blobs: the E8M0 scale of row n, 32-value block B sits at
 * (n / 16)(K / 2) + 64 (B / 4) + 4 (n % 16) + B % 4; codes as above. */
static inline SYNTH_HD uint64_t synth_mx_scale_pos(uint64_t n, int B, int K) {
  return (n >> 4) * (uint64_t)(K / 2) + 64ull * (uint64_t)(B >> 2) + 4ull * (n & 15) + (uint64_t)(B & 3);
}

static inline SYNTH_HD uint64_t synth_scale_pos(uint64_t n, int b, int K) {
  const int g = b >> 5, nc = K / 32;
  const int len = 2 * ((nc - 16 * g) < 16 ? nc - 16 * g : 16);
  return (n >> 4) * (uint64_t)K + 512ull * (uint64_t)g + (uint64_t)len * (n & 15) + (uint64_t)(b - 32 * g);
}
