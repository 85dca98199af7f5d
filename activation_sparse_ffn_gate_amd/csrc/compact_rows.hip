// Row gather for dropping dead gate units from a layer, for gfx950.
//
// A unit that no token activates adds exact zeros to every output row
// (pulsen.vercel.app article, dead-neuron paragraph: over 30% of units end up
// never active at the recommended L1 coefficient), so a compacted layer keeps
// only the live rows of Wg, WuT and Wd, padded with zero rows to whole TwELL
// tiles (a zero gate row gives z = 0, which is never active). This kernel
// builds one compacted matrix: out[i] = W[src[i]], or a zero row where src[i]
// is negative or past the matrix.
//
// One wave per output row, 16-byte loads and stores (a row is 2d bytes, d a
// multiple of 256): HBM-bound, 4d bytes moved per row.
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kRowsPerWG = 4;

__global__ __launch_bounds__(64 * kRowsPerWG) void gather_rows_kernel(const uint16_t* W, int F, int d,
                                                                      const int32_t* src, int n,
                                                                      uint16_t* out) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kRowsPerWG + (threadIdx.x >> 6);
  if (i >= n) return;
  const int s = src[i];
  const int pieces = d / 8;  // 16-byte pieces per row
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(i) * d);
  if (s < 0 || s >= F) {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int p = lane; p < pieces; p += 64) dst[p] = zero;
    return;
  }
  const u32x4_t* row = reinterpret_cast<const u32x4_t*>(W + static_cast<size_t>(s) * d);
  for (int p = lane; p < pieces; p += 64) dst[p] = row[p];
}

}  // namespace

hipError_t launch_gather_rows(const uint16_t* W, int F, int d, const int32_t* src, int n, uint16_t* out,
                              hipStream_t s) {
  const dim3 grid((n + kRowsPerWG - 1) / kRowsPerWG), block(64 * kRowsPerWG);
  gather_rows_kernel<<<grid, block, 0, s>>>(W, F, d, src, n, out);
  return hipGetLastError();
}

}  // namespace twell
