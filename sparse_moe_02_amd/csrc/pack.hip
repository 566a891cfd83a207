// Weight preparation: code words and fp16 scale/bias arrays from row-major order into the
// tiles the kernels read.  Codes: 16 rows x 128 k per tile, a row's 16 words of the tile
// contiguous.  Scale/bias (G groups of 64 per row): 16 rows per tile, element (n, g) at
// ((n/16) G + g) 16 + n%16.
//
// "Optimizing on-device inference for Apple Silicon", section "Prefill > Dequantize
// weights during matmul": each group of 64 weights carries one scale and one bias.  The
// tiled order serves both forms: a 128-k step of the grouped GEMM reads, for 16 rows, the
// two groups of the step as one run of 64 bytes (row-major order would touch 16 separate
// lines for 4 bytes each) and the codes of the step as one run of 1 KB (row-major: 16
// half lines), and a decode task of 16 rows reads all groups of its rows as one
// contiguous block.
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

// One thread per destination 16-byte piece (four words of one row in one tile).
__global__ __launch_bounds__(256) void k_pack_codes(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                    int64_t total, int KW) {
  const int steps = KW / 16;  // 128-k tiles per row
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t tile = i / 64;  // 64 pieces (16 rows x 4) per tile
    const int rem = (int)(i & 63);
    const int64_t n16 = tile / steps;
    const int kt = (int)(tile - n16 * steps);
    const int r = rem >> 2, pc = rem & 3;
    dst[i] = src[((n16 * 16 + r) * KW + kt * 16) / 4 + pc];
  }
}

}  // namespace

hipError_t launch_pack_codes(const uint32_t *src, uint32_t *dst, int64_t rows, int K, hipStream_t s) {
  const int64_t total = rows * (int64_t)(K / 32);  // 16-byte pieces
  const int64_t want = (total + 255) / 256;
  const int blocks = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_pack_codes, dim3(blocks), dim3(256), 0, s, (const uint4 *)src, (uint4 *)dst, total, K / 8);
  return hipGetLastError();
}

hipError_t launch_pack_qparams(const uint16_t *src, uint16_t *dst, int64_t rows, int G, hipStream_t s) {
  const int64_t total = rows * (int64_t)G;
  const int64_t want = (total + 255) / 256;
  const int blocks = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_pack_qparams, dim3(blocks), dim3(256), 0, s, src, dst, total, G);
  return hipGetLastError();
}

}  // namespace moe
