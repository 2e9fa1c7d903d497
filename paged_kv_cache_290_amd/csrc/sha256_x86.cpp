// SHA-256 compression (FIPS 180-4) with the x86 SHA extensions, for the prefix-cache
// block keys on the host.  Host-only source (compiled by the host C++ compiler); the
// caller checks sha256_x86_available() and otherwise uses the portable rounds.
//
// The instructions carry the state as two quads, {A, B, E, F} and {C, D, G, H}
// (element 3 first); sha256rnds2 performs two rounds from the low two words of W+K
// and returns the new {A, B, E, F}, the old one becoming {C, D, G, H}.  The message
// schedule quad j >= 4 is sha256msg2(sha256msg1(W[j-4], W[j-3]) + (W[j-2], W[j-1])
// shifted by one word, W[j-1]): W[t-16] + s0(W[t-15]) + W[t-7] + s1(W[t-2]).
#include <immintrin.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

bool sha256_x86_available() {
  static const int ok = __builtin_cpu_supports("sha") && __builtin_cpu_supports("sse4.1");
  return ok != 0;
}

namespace {
alignas(16) const uint32_t kK[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4,
    0xab1c5ed5, 0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe,
    0x9bdc06a7, 0xc19bf174, 0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f,
    0x4a7484aa, 0x5cb0a9dc, 0x76f988da, 0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7,
    0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967, 0x27b70a85, 0x2e1b2138, 0x4d2c6dfc,
    0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85, 0xa2bfe8a1, 0xa81a664b,
    0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070, 0x19a4c116,
    0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7,
    0xc67178f2};
}  // namespace

__attribute__((target("sha,sse4.1"))) void sha256_x86_chunks(uint32_t h[8],
                                                               const uint8_t *data,
                                                               size_t nchunks) {
  // Big-endian words: reverse the bytes of each 32-bit lane.
  const __m128i bswap = _mm_set_epi8(12, 13, 14, 15, 8, 9, 10, 11, 4, 5, 6, 7, 0, 1, 2, 3);
  __m128i abef = _mm_set_epi32((int)h[0], (int)h[1], (int)h[4], (int)h[5]);
  __m128i cdgh = _mm_set_epi32((int)h[2], (int)h[3], (int)h[6], (int)h[7]);
  for (size_t c = 0; c < nchunks; ++c, data += 64) {
    const __m128i abef0 = abef, cdgh0 = cdgh;
    __m128i w[4];
#pragma GCC unroll 4
    for (int j = 0; j < 4; ++j)
      w[j] = _mm_shuffle_epi8(_mm_loadu_si128(reinterpret_cast<const __m128i *>(data + 16 * j)),
                              bswap);
#pragma GCC unroll 16
    for (int j = 0; j < 16; ++j) {
      __m128i wj;
      if (j < 4) {
        wj = w[j];
      } else {
        __m128i x = _mm_sha256msg1_epu32(w[j % 4], w[(j + 1) % 4]);   // W[j-4], W[j-3]
        x = _mm_add_epi32(x, _mm_alignr_epi8(w[(j + 3) % 4], w[(j + 2) % 4], 4));
        wj = _mm_sha256msg2_epu32(x, w[(j + 3) % 4]);                   // W[j-1]
        w[j % 4] = wj;
      }
      const __m128i wk = _mm_add_epi32(wj, _mm_load_si128(reinterpret_cast<const __m128i *>(kK + 4 * j)));
      cdgh = _mm_sha256rnds2_epu32(cdgh, abef, wk);                      // rounds 4j, 4j+1
      abef = _mm_sha256rnds2_epu32(abef, cdgh, _mm_shuffle_epi32(wk, 0x0E));  // 4j+2, 4j+3
    }
    abef = _mm_add_epi32(abef, abef0);
    cdgh = _mm_add_epi32(cdgh, cdgh0);
  }
  h[0] = (uint32_t)_mm_extract_epi32(abef, 3);
  h[1] = (uint32_t)_mm_extract_epi32(abef, 2);
  h[4] = (uint32_t)_mm_extract_epi32(abef, 1);
  h[5] = (uint32_t)_mm_extract_epi32(abef, 0);
  h[2] = (uint32_t)_mm_extract_epi32(cdgh, 3);
  h[3] = (uint32_t)_mm_extract_epi32(cdgh, 2);
  h[6] = (uint32_t)_mm_extract_epi32(cdgh, 1);
  h[7] = (uint32_t)_mm_extract_epi32(cdgh, 0);
}

}  // namespace pkv
