// pack.hip -- moe_pack_bank's kernel: the one-time reorder of a bank's codes and FP4 scales
// into 16-row tiles stored piece-major, the order in which the expert kernels load them
// (one wave instruction = one contiguous 1 KB run = 16 rows x 64 bytes of matrix-core
// operand).  A pure byte permutation.
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
  else if (unit == 2)
    hipLaunchKernelGGL(k_pack_tile16<2>, grid, block, 0, s, in, out, rows, pitch);
  else
    hipLaunchKernelGGL(k_pack_tile16<1>, grid, block, 0, s, in, out, rows, pitch);
  return hipGetLastError();
}

}  // namespace qmoe
