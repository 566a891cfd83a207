// Weight preparation: fp16 scale/bias arrays from row-major [rows][G] (G groups of 64 per
// row) into 16-row tiles, element (n, g) at ((n/16) G + g) 16 + n%16.
//
// "Optimizing on-device inference for Apple Silicon", section "Prefill > Dequantize
// weights during matmul": each group of 64 weights carries one scale and one bias.  The
// tiled order serves both forms: a 128-k step of the grouped GEMM reads, for 16 rows, the
// two groups of the step as one run of 64 bytes (row-major order would touch 16 separate
// lines for 4 bytes each), and a decode task of 16 rows reads all groups of its rows as
// one contiguous block.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// One thread per destination element (writes coalesced); a wave reads 16 rows x 4 groups.
__global__ __launch_bounds__(256) void k_pack_qparams(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                                      int64_t total, int G) {
  const int64_t tile_elems = kQpRows * (int64_t)G;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t tile = i / tile_elems;
    const int rem = (int)(i - tile * tile_elems);
    const int g = rem / kQpRows, r = rem % kQpRows;
    dst[i] = src[(tile * kQpRows + r) * G + g];
  }
}

}  // namespace

hipError_t launch_pack_qparams(const uint16_t *src, uint16_t *dst, int64_t rows, int G, hipStream_t s) {
  const int64_t total = rows * (int64_t)G;
  const int64_t want = (total + 255) / 256;
  const int blocks = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_pack_qparams, dim3(blocks), dim3(256), 0, s, src, dst, total, G);
  return hipGetLastError();
}

}  // namespace moe
