// pack.hip -- moe_pack_bank's kernels: the one-time reorder of a bank's codes and per-row scales
// into 16-row tiles stored piece-major, the order in which the expert kernels load them
// (one wave instruction = one contiguous 1 KB run = 16 rows x 64 bytes of matrix-core
// operand).  A pure byte permutation, except for Q4_0 codes, whose nibbles are also regrouped.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace qmoe {

// Matrix of `rows` rows x `pitch` bytes (rows % 16 == 0, pitch % U == 0): unit j (U bytes)
// of row r moves from r*pitch + j*U to (r/16)*16*pitch + j*16*U + (r%16)*U.  Threads walk
// the destination in order, so the stores are contiguous.
template <int U>
__global__ __launch_bounds__(256) void k_pack_tile16(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                     size_t rows, uint32_t pitch) {
  const size_t units = pitch / U, per_tile = 16 * units, n = rows * units;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t tile = i / per_tile, rem = i - tile * per_tile;
    const size_t j = rem / 16, r = tile * 16 + rem % 16;
    const uint8_t *s = src + r * pitch + j * U;
    uint8_t *d = dst + i * U;
    if constexpr (U == 16) {
      *reinterpret_cast<uint4 *>(d) = *reinterpret_cast<const uint4 *>(s);
    } else {
#pragma unroll
      for (int b = 0; b < U; b++) d[b] = s[b];
    }
  }
}

// Transposed source: E matrices of `pitch` rows x N columns (bytes); destination row r =
// e*N + n holds the bytes of source column n of matrix e.  Destination order as above; each
// unit gathers U bytes down a source column.
template <int U>
__global__ __launch_bounds__(256) void k_pack_tile16_t(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                       size_t E, size_t N, uint32_t pitch) {
  const size_t units = pitch / U, per_tile = 16 * units, n_units = E * N * units;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_units; i += (size_t)gridDim.x * 256) {
    const size_t tile = i / per_tile, rem = i - tile * per_tile;
    const size_t j = rem / 16, r = tile * 16 + rem % 16;
    const size_t e = r / N, n = r - e * N;
    const uint8_t *col = src + e * pitch * N + j * U * N + n;
    uint8_t *d = dst + i * U;
#pragma unroll
    for (int b = 0; b < U; b++) d[b] = col[(size_t)b * N];
  }
}

// Q4_0 codes: rows of `pitch` bytes = pitch/16 blocks of 32 elements, block byte j holding
// element j (low nibble) and element j + 16 (high nibble).  Destination piece (s, g) of a
// row (16 bytes, same tile-16 placement as the FP4 codes: (r/16)*16*pitch + (4s+g)*256 +
// (r%16)*16) holds one dword per block 4s+q (q = 0..3): that block's elements 8g..8g+7, with
// element 8g+2i in bits [4i, 4i+4) and element 8g+2i+1 in bits [16+4i, 20+4i).  A kernel
// then turns each dword into 4 bf16 pairs with one shift and one mask-or per pair.
__global__ __launch_bounds__(256) void k_pack_q4_0(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                   size_t rows, uint32_t pitch) {
  const size_t pieces = pitch / 16, per_tile = 16 * pieces, n = rows * pieces;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t tile = i / per_tile, rem = i - tile * per_tile;
    const size_t pc = rem / 16, r = tile * 16 + rem % 16;
    const size_t st = pc / 4;
    const int g = (int)(pc % 4);
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      // elements 8g..8g+7 of block 4st+q: bytes 8(g&1)..+7, low nibbles for g < 2
      const uint8_t *b = src + r * pitch + (4 * st + q) * 16 + 8 * (g & 1);
      const int sh = 4 * (g >> 1);
      uint32_t d = 0;
#pragma unroll
      for (int i2 = 0; i2 < 4; i2++) {
        d |= ((uint32_t)(b[2 * i2] >> sh) & 0xFu) << (4 * i2);
        d |= ((uint32_t)(b[2 * i2 + 1] >> sh) & 0xFu) << (16 + 4 * i2);
      }
      out[q] = d;
    }
    *reinterpret_cast<uint4 *>(dst + i * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

hipError_t launch_pack_q4_0(const void *src, void *dst, size_t rows, uint32_t pitch, hipStream_t s) {
  const size_t n = rows * (pitch / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<size_t>((n + 255) / 256, (size_t)1 << 20)), block(256);
  hipLaunchKernelGGL(k_pack_q4_0, grid, block, 0, s, static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst),
                     rows, pitch);
  return hipGetLastError();
}

hipError_t launch_pack_tile16_t(const void *src, void *dst, size_t E, size_t N, uint32_t pitch, int unit,
                                hipStream_t s) {
  const size_t n = E * N * (pitch / unit);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<size_t>((n + 255) / 256, (size_t)1 << 20)), block(256);
  const auto *in = static_cast<const uint8_t *>(src);
  auto *out = static_cast<uint8_t *>(dst);
  if (unit == 16)
    hipLaunchKernelGGL(k_pack_tile16_t<16>, grid, block, 0, s, in, out, E, N, pitch);
  else
    hipLaunchKernelGGL(k_pack_tile16_t<1>, grid, block, 0, s, in, out, E, N, pitch);
  return hipGetLastError();
}

hipError_t launch_pack_tile16(const void *src, void *dst, size_t rows, uint32_t pitch, int unit, hipStream_t s) {
  const size_t n = rows * (pitch / unit);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<size_t>((n + 255) / 256, (size_t)1 << 20)), block(256);
  const auto *in = static_cast<const uint8_t *>(src);
  auto *out = static_cast<uint8_t *>(dst);
  if (unit == 16)
    hipLaunchKernelGGL(k_pack_tile16<16>, grid, block, 0, s, in, out, rows, pitch);
  else if (unit == 8)
    hipLaunchKernelGGL(k_pack_tile16<8>, grid, block, 0, s, in, out, rows, pitch);
  else if (unit == 2)
    hipLaunchKernelGGL(k_pack_tile16<2>, grid, block, 0, s, in, out, rows, pitch);
  else
    hipLaunchKernelGGL(k_pack_tile16<1>, grid, block, 0, s, in, out, rows, pitch);
  return hipGetLastError();
}

}  // namespace qmoe
