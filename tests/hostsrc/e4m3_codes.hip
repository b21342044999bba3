// Host build of the query kernels' FP8 encoder: writes the e4m3 code of
// v * q for every finite bf16 value v and every scale q read from stdin (one
// per line), as raw bytes, in that order.  Compiled and run by the CPU test
// suite; it runs no GPU code.
#include "../../mqa_latent_kv_amd/csrc/query.hip"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

int main() {
  std::vector<float> qs;
  float q;
  while (std::scanf("%a", &q) == 1) qs.push_back(q);
  std::vector<uint8_t> out;
  out.reserve(qs.size() * 65536);
  for (const float s : qs) {
    for (uint32_t b = 0; b < 65536; ++b) {
      const uint32_t bits = b << 16;
      float v;
      std::memcpy(&v, &bits, 4);
      if (!std::isfinite(v)) continue;
      out.push_back(mla::e4m3_of_product(v, s));
    }
  }
  return std::fwrite(out.data(), 1, out.size(), stdout) == out.size() ? 0 : 1;
}
