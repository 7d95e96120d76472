// Packs pairs of floats into one byte with ROCm's fp4x2 storage conversion
// (hip/hip_fp4.h, __hip_cvt_float2_to_fp4x2), compiled for the host only, so
// its software E2M1 encoder runs: an implementation of the packed E2M1 pair
// layout independent of the oracle.  Reads lines "a b" and prints the byte.
#include <hip/hip_fp4.h>

#include <cstdio>

int main() {
  float a, b;
  while (std::scanf("%f %f", &a, &b) == 2) {
    float2 v;
    v.x = a;
    v.y = b;
    const __hip_fp4x2_storage_t p = __hip_cvt_float2_to_fp4x2(v, __HIP_E2M1, hipRoundNearest);
    std::printf("%u\n", (unsigned)p);
  }
  return 0;
}
