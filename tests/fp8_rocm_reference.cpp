// Independent reference for the oracle's fp8 encoder: ROCm's own software conversion of
// fp32 to OCP e4m3fn (hip/hip_fp8.h, host path), round to nearest even, in its
// saturate-to-finite mode.  Reads fp32 bit patterns (hex, one per line) from stdin and
// prints the e4m3fn code of each (hex).  Built and run on the host by the oracle's pin
// tests; it touches no GPU.
#include <hip/hip_fp8.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

int main() {
  unsigned bits;
  while (std::scanf("%x", &bits) == 1) {
    float x;
    std::memcpy(&x, &bits, sizeof x);
    std::printf("%02x\n", (unsigned)__hip_cvt_float_to_fp8(x, __HIP_SATFINITE, __HIP_E4M3));
  }
  return 0;
}
