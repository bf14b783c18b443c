// tg_gather: copy the kept rows X[idx[r]] -> dst[r] (TokenGate §4.1: the
// residual stream of a pruned token stops at the gate layer).
//
// Pure data movement, bound by HBM bandwidth: 2 * row_bytes per kept row.
// Each block copies kRows rows with 16-byte vector loads/stores; all loads of
// a thread are issued before its stores so several rows are in flight.  Both
// directions are non-temporal: the rows stream through once, and stores that
// do not allocate in the L2 took back-to-back copies of the 128k layer's
// 8704 rows from 15.1 to 12.8 us.
#include "common.h"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;

__global__ __launch_bounds__(kThreads) void gather_vec16(
    const char* __restrict__ src, int64_t src_stride, int64_t n_src, int64_t n_vec,
    const int32_t* __restrict__ idx, int64_t n_rows, char* __restrict__ dst, int64_t dst_stride) {
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  int64_t srow[kRows];
  bool valid[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t r = r0 + i;
    const int64_t s = r < n_rows ? (int64_t)idx[r] : -1;
    valid[i] = s >= 0 && s < n_src;
    srow[i] = valid[i] ? s : 0;
  }
  for (int64_t vbase = 0; vbase < n_vec; vbase += kThreads * 2) {
    u32x4 buf[kRows][2];
#pragma unroll
    for (int i = 0; i < kRows; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t v = vbase + threadIdx.x + j * kThreads;
        u32x4 z = {0u, 0u, 0u, 0u};
        if (valid[i] && v < n_vec)
          z = ld_nt16(reinterpret_cast<const u32x4*>(src + srow[i] * src_stride) + v);
        buf[i][j] = z;
      }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int64_t r = r0 + i;
      if (r >= n_rows) break;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t v = vbase + threadIdx.x + j * kThreads;
        if (v < n_vec)
          __builtin_nontemporal_store(buf[i][j], reinterpret_cast<u32x4*>(dst + r * dst_stride) + v);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void gather_word(
    const char* __restrict__ src, int64_t src_stride, int64_t n_src, int64_t n_word,
    const int32_t* __restrict__ idx, int64_t n_rows, char* __restrict__ dst, int64_t dst_stride) {
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  for (int i = 0; i < kRows; ++i) {
    const int64_t r = r0 + i;
    if (r >= n_rows) break;
    const int64_t s = idx[r];
    const bool ok = s >= 0 && s < n_src;
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(src + (ok ? s : 0) * src_stride);
    uint32_t* dp = reinterpret_cast<uint32_t*>(dst + r * dst_stride);
    for (int64_t w = threadIdx.x; w < n_word; w += kThreads) dp[w] = ok ? sp[w] : 0u;
  }
}

}  // namespace

hipError_t launch_gather(const void* src, int64_t src_stride, int64_t n_src, int64_t row_bytes,
                         const int32_t* idx, int64_t n_rows, void* dst, int64_t dst_stride,
                         hipStream_t st) {
  const dim3 grid((unsigned)((n_rows + kRows - 1) / kRows));
  const bool vec = row_bytes % 16 == 0 && src_stride % 16 == 0 && dst_stride % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(gather_vec16, grid, dim3(kThreads), 0, st, (const char*)src, src_stride,
                       n_src, row_bytes / 16, idx, n_rows, (char*)dst, dst_stride);
  else
    hipLaunchKernelGGL(gather_word, grid, dim3(kThreads), 0, st, (const char*)src, src_stride,
                       n_src, row_bytes / 4, idx, n_rows, (char*)dst, dst_stride);
  return hipGetLastError();
}

}  // namespace tg
