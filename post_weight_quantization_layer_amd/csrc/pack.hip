// b-bit codes -> least-significant-bit-first bit stream per row ("GPTQ",
// sections Jak dziala and Zlozonosc obliczeniowa: 4- or 3-bit weights,
// about 4.x bits per weight as stored).
//
// One thread per output word: word w of a row holds stream bits
// [32w, 32w + 32), i.e. the codes k with k*b in (32w - b, 32w + 32).
#include "common.h"

namespace gptq {
namespace {

__global__ void __launch_bounds__(256)
    pack_kernel(const uint8_t *__restrict__ codes, int64_t rows, int64_t cols, int bits,
                uint32_t *__restrict__ out) {
  const int64_t wpr = cols * bits / 32;  // words per row
  const int64_t total = rows * wpr;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * 256) {
    const int64_t r = t / wpr, w = t % wpr;
    const uint8_t *c = codes + r * cols;
    const int64_t b0 = w * 32;
    int64_t k = b0 / bits;  // first code with bits in this word
    uint64_t acc = 0;
    for (; k * bits < b0 + 32; ++k) {
      const int64_t off = k * bits - b0;  // may be negative for a straddling code
      const uint64_t v = c[k] & mask;
      acc |= off >= 0 ? (v << off) : (v >> (-off));
    }
    out[t] = (uint32_t)acc;
  }
}

}  // namespace

gptq_status pack_impl(const uint8_t *codes, int64_t rows, int64_t cols, int bits,
                      uint32_t *packed, hipStream_t stream) {
  const int64_t total = rows * (cols * bits / 32);
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total, 256), 65536);
  return launch("pack", pack_kernel, dim3(blocks), dim3(256), 0, stream, codes, rows, cols, bits,
                packed);
}

}  // namespace gptq
