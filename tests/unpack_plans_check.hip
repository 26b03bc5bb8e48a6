// Host check of the slot plans: for every width, the fp16 bits that unpack_step puts in
// slot k of step s equal code[chan(s,k)] << exp(s,k), stay inside the 10-bit subnormal
// mantissa, and chan(., .) is a permutation of the group. The value plans (unpack_step_v,
// VSlots) must also give the chunks of one K-step the same exponents: exp(s, k) depends on
// (s % 4, k) only. No code sits more than 4 bits below the top of the 10-bit mantissa (2 bits:
// from bit 4; 3, 4 bits: from bit 2; 5, 7 bits: from bit 1), where the MFMA sums them precisely.
#include "code_plans.h"
#include <cstdio>
#include <random>
using namespace kvq;
template <int B>
constexpr int min_exp() { return B == 2 ? 4 : B <= 4 ? 2 : B == 6 ? 0 : B == 8 ? 2 : 1; }
template <int B>
int check(std::mt19937& g) {
  int bad = 0;
  for (int s = 0; s < 8; ++s)
    for (int k = 0; k < 4; ++k)
      if (Slots<B>::exp(s, k) < min_exp<B>()) ++bad;
  for (int trial = 0; trial < 2000; ++trial) {
    uint32_t codes[32], w[B] = {};
    for (int i = 0; i < 32; ++i) codes[i] = g() & ((1u << B) - 1);
    if (trial == 0) for (int i = 0; i < 32; ++i) codes[i] = (1u << B) - 1;
    for (int i = 0; i < 32; ++i)
      for (int j = 0; j < B; ++j) {
        const int k = i * B + j;
        w[k / 32] |= ((codes[i] >> j) & 1u) << (k % 32);
      }
    int seen[32] = {};
    for (int s = 0; s < 8; ++s) {
      const u32x2 r = unpack_step<B>(w, 0, s);
      const uint32_t halves[4] = {r[0] & 0xFFFF, r[0] >> 16, r[1] & 0xFFFF, r[1] >> 16};
      for (int k = 0; k < 4; ++k) {
        const int ch = Slots<B>::chan(s, k), e = Slots<B>::exp(s, k);
        seen[ch]++;
        const uint32_t want = codes[ch] << e;
        if (halves[k] != want || want >= 1024u) ++bad;
      }
    }
    for (int i = 0; i < 32; ++i) if (seen[i] != 1) ++bad;
  }
  printf("B=%d: %d mismatches\n", B, bad);
  return bad;
}
template <int B>
int check_v(std::mt19937& g) {
  int bad = 0;
  for (int s = 2; s < 8; ++s)
    for (int k = 0; k < 4; ++k)
      if (VSlots<B>::exp(s, k) != VSlots<B>::exp(s & 3, k)) ++bad;
  for (int s = 0; s < 8; ++s)
    for (int k = 0; k < 4; ++k)
      if (VSlots<B>::exp(s, k) < min_exp<B>()) ++bad;
  for (int trial = 0; trial < 2000; ++trial) {
    uint32_t codes[32], w[B] = {};
    for (int i = 0; i < 32; ++i) codes[i] = g() & ((1u << B) - 1);
    if (trial == 0) for (int i = 0; i < 32; ++i) codes[i] = (1u << B) - 1;
    for (int i = 0; i < 32; ++i)
      for (int j = 0; j < B; ++j) {
        const int k = i * B + j;
        w[k / 32] |= ((codes[i] >> j) & 1u) << (k % 32);
      }
    int seen[32] = {};
    for (int s = 0; s < 8; ++s) {
      const u32x2 r = unpack_step_v<B>(w, 0, s);
      const uint32_t halves[4] = {r[0] & 0xFFFF, r[0] >> 16, r[1] & 0xFFFF, r[1] >> 16};
      for (int k = 0; k < 4; ++k) {
        const int ch = VSlots<B>::chan(s, k), e = VSlots<B>::exp(s, k);
        seen[ch]++;
        const uint32_t want = codes[ch] << e;
        if (halves[k] != want || want >= 1024u) ++bad;
      }
    }
    for (int i = 0; i < 32; ++i) if (seen[i] != 1) ++bad;
  }
  printf("value plan B=%d: %d mismatches\n", B, bad);
  return bad;
}
// The value stream order the plans imply: element e = 8 c + u of a stream (chunk c, token u)
// is read by step 2 c + u / 4, slot u % 4, which takes stream position VSlots::chan of it.
template <int B>
void print_stream_order() {
  printf("value stream order B=%d:", B);
  for (int e = 0; e < 32; ++e) printf(" %d", VSlots<B>::chan(2 * (e / 8) + (e % 8) / 4, e % 4));
  printf("\n");
}
int main() {
  std::mt19937 g(7);
  print_stream_order<2>(); print_stream_order<3>(); print_stream_order<4>(); print_stream_order<5>();
  print_stream_order<6>(); print_stream_order<7>(); print_stream_order<8>();
  int bad = check<2>(g) + check<3>(g) + check<4>(g) + check<5>(g) + check<6>(g) + check<7>(g) + check<8>(g);
  bad += check_v<2>(g) + check_v<3>(g) + check_v<4>(g) + check_v<5>(g) + check_v<6>(g) + check_v<7>(g) +
         check_v<8>(g);
  return bad ? 1 : 0;
}
