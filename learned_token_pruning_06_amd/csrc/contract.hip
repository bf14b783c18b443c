// Device-side contract checks (off by default, tg_set_contract_checks).
//
// Some preconditions of the calls depend on device data the host does not
// read: the packing offsets, the budgets, the kept indices and positions.
// The kernels never access memory outside their buffers when these are
// broken (offsets are clamped, out-of-range indices give zero rows, outputs
// past the capacity are dropped), but the results are then meaningless.
// With the checks on, each call also launches a small kernel before (or,
// for the selection's output count, after) its own work that tests those
// preconditions and ORs a bit per broken rule into a per-device flag word;
// tg_contract_status reads the word back and clears it.
#include <atomic>
#include <mutex>

#include "common.h"
#include "tokengate.h"

// The flag word, one per GPU.  Host code uses the address returned by
// hipGetSymbolAddress, never this name.
static __device__ __align__(256) unsigned int contract_flags[1];

namespace tg {
namespace {

std::atomic<int> g_checks{0};

TG_DEVINL void raise(unsigned int* flags, unsigned int bit) {
  // every lane that finds a breach ORs its bit (a vector atomic)
  atomicOr(flags, bit);
}

// cu[0] >= 0, non-decreasing, cu[n] <= limit
__global__ __launch_bounds__(256) void check_offsets(const int32_t* __restrict__ cu, int n,
                                                     int64_t limit, unsigned int bit,
                                                     unsigned int* flags) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i <= n;
       i += (int64_t)gridDim.x * 256) {
    const int32_t c = cu[i];
    bool bad = c < 0 || (int64_t)c > limit;
    if (i < n) bad = bad || cu[i + 1] < c;
    if (bad) raise(flags, bit);
  }
}

// budgets >= 0
__global__ __launch_bounds__(256) void check_budgets(const int32_t* __restrict__ k, int n,
                                                     unsigned int* flags) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
    if (k[i] < 0) raise(flags, TG_CONTRACT_NEGATIVE_BUDGET);
}

// kept count (kept_cu[n]) within the capacity
__global__ __launch_bounds__(64) void check_capacity(const int32_t* __restrict__ kept_cu, int n,
                                                     int64_t cap, unsigned int* flags) {
  if (threadIdx.x == 0 && (int64_t)kept_cu[n] > cap) raise(flags, TG_CONTRACT_CAPACITY);
}

// gather indices within [0, n_src)
__global__ __launch_bounds__(256) void check_indices(const int32_t* __restrict__ idx, int64_t n,
                                                     int64_t n_src, unsigned int* flags) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    if (idx[i] < 0 || (int64_t)idx[i] >= n_src) raise(flags, TG_CONTRACT_INDEX);
}

// kept positions >= 0 and strictly increasing within each sequence of cu
// (row r belongs to the sequence s with cu[s] <= r < cu[s+1]; a row is
// compared with the next one when both are in the same sequence)
__global__ __launch_bounds__(256) void check_positions(const int32_t* __restrict__ pos,
                                                       const int32_t* __restrict__ cu, int n_seq,
                                                       int64_t t, unsigned int* flags) {
  for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < t;
       r += (int64_t)gridDim.x * 256) {
    if (pos[r] < 0) {
      raise(flags, TG_CONTRACT_POSITIONS);
      continue;
    }
    if (r + 1 >= t) continue;
    // is r + 1 the first row of some sequence?  (binary search over cu)
    int lo = 0, hi = n_seq, starts = 0;
    while (lo <= hi) {
      const int mid = (lo + hi) >> 1;
      const int64_t c = cu[mid];
      if (c == r + 1) {
        starts = 1;
        break;
      }
      if (c < r + 1) lo = mid + 1;
      else hi = mid - 1;
    }
    if (!starts && pos[r + 1] <= pos[r]) raise(flags, TG_CONTRACT_POSITIONS);
  }
}

__global__ __launch_bounds__(64) void clear_flags(unsigned int* flags) {
  if (threadIdx.x == 0) flags[0] = 0u;
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

}  // namespace

bool contract_checks_on() { return g_checks.load(std::memory_order_relaxed) != 0; }
void set_contract_checks(bool on) { g_checks.store(on ? 1 : 0, std::memory_order_relaxed); }

hipError_t contract_flags_ptr(unsigned int** ptr) {
  static std::mutex mu;
  static unsigned int* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(contract_flags));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<unsigned int*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t contract_offsets(const int32_t* cu, int n, int64_t limit, unsigned int bit,
                            hipStream_t st) {
  unsigned int* f = nullptr;
  hipError_t e = contract_flags_ptr(&f);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_offsets, dim3(grid_for(n + 1)), dim3(256), 0, st, cu, n, limit, bit, f);
  return hipGetLastError();
}

hipError_t contract_budgets(const int32_t* k, int n, hipStream_t st) {
  unsigned int* f = nullptr;
  hipError_t e = contract_flags_ptr(&f);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_budgets, dim3(grid_for(n)), dim3(256), 0, st, k, n, f);
  return hipGetLastError();
}

hipError_t contract_capacity(const int32_t* kept_cu, int n, int64_t cap, hipStream_t st) {
  unsigned int* f = nullptr;
  hipError_t e = contract_flags_ptr(&f);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_capacity, dim3(1), dim3(64), 0, st, kept_cu, n, cap, f);
  return hipGetLastError();
}

hipError_t contract_indices(const int32_t* idx, int64_t n, int64_t n_src, hipStream_t st) {
  unsigned int* f = nullptr;
  hipError_t e = contract_flags_ptr(&f);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_indices, dim3(grid_for(n)), dim3(256), 0, st, idx, n, n_src, f);
  return hipGetLastError();
}

hipError_t contract_positions(const int32_t* pos, const int32_t* cu, int n_seq, int64_t t,
                              hipStream_t st) {
  unsigned int* f = nullptr;
  hipError_t e = contract_flags_ptr(&f);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_positions, dim3(grid_for(t)), dim3(256), 0, st, pos, cu, n_seq, t, f);
  return hipGetLastError();
}

// the word of this device after the work queued on `st`, then cleared (a
// one-thread kernel writes the zero, so nothing else on the stream races it)
hipError_t contract_read_and_clear(unsigned int* out, hipStream_t st) {
  unsigned int* f = nullptr;
  hipError_t e = contract_flags_ptr(&f);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(out, f, sizeof(unsigned int), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clear_flags, dim3(1), dim3(64), 0, st, f);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace tg
