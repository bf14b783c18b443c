// Shared device helpers and internal launch entry points of libtokengate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define TG_DEVINL __device__ __forceinline__

namespace tg {

// ---------------------------------------------------------------------------
// sequence chunking without a lookup table
//
// Sequence s owns grid slots [slot0(s), slot0(s+1)) with
//   slot0(s) = s + floor(cu[s] / CH).
// slot0(s+1) - slot0(s) = 1 + floor(cu[s+1]/CH) - floor(cu[s]/CH)
//                      >= 1 + floor(len_s/CH) >= ceil(len_s/CH),
// so every chunk of every sequence has a slot; surplus slots exit at once.
// A grid of n_seq + ceil(t_in / CH) slots covers every sequence.
// ---------------------------------------------------------------------------
TG_DEVINL int64_t slot0_of(const int32_t* cu, int s, int ch) {
  return (int64_t)s + (int64_t)(cu[s] / ch);
}

// Largest s in [0, n_seq) with slot0(s) <= slot; -1 if none.
TG_DEVINL int seq_of_slot(const int32_t* cu, int n_seq, int64_t slot, int ch) {
  int lo = 0, hi = n_seq - 1, ans = -1;
  while (lo <= hi) {
    int mid = (lo + hi) >> 1;
    if (slot0_of(cu, mid, ch) <= slot) {
      ans = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  return ans;
}

// ---------------------------------------------------------------------------
// order-preserving 32-bit key of a score: a larger float gives a larger key,
// -0.0 and +0.0 share a key, every NaN maps to 0 (below -inf, whose key is
// 0x007FFFFF).
// ---------------------------------------------------------------------------
TG_DEVINL uint32_t score_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// wave / block reductions (wave64)
// ---------------------------------------------------------------------------
template <typename T>
TG_DEVINL T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

TG_DEVINL float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// inclusive prefix sum over the 64 lanes of a wave
TG_DEVINL int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT % 64 == 0) in thread
// order; returns the exclusive prefix and writes the block total.
// `scratch` must hold NT/64 ints; contains a barrier.
template <int NT>
TG_DEVINL int block_excl_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int s = scratch[i];
    base += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads/stores on a native vector type (HIP's uint4 is a struct with
// a union inside, and copies of it can keep values in scratch memory)
TG_DEVINL u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
TG_DEVINL void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// 16-byte load that does not keep the line in cache (streamed operands)
TG_DEVINL u32x4 ld_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

TG_DEVINL uint32_t ld_acquire_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tg

// ---------------------------------------------------------------------------
// internal launchers (arguments already validated by api.hip)
// ---------------------------------------------------------------------------
namespace tg {

// compute units of the current device, cached per device (host side; sizes
// the persistent attention grid and the scorer's row tiles)
inline hipError_t device_cu_count(int* n_cu) {
  static int cache[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *n_cu = cache[dev];
    return hipSuccess;
  }
  e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*n_cu < 1) *n_cu = 1;
  if (dev >= 0 && dev < 64) cache[dev] = *n_cu;
  return hipSuccess;
}

constexpr int kScoreChunk = 2048;    // tokens per normalisation block
constexpr int kSelChunk = 2048;      // tokens per selection block

size_t score_ws_bytes(int64_t t_in, int n_seq);
hipError_t launch_score(const void* x, int dt, int64_t x_row_stride, int64_t t_in, int d, int h,
                        const void* w1, const float* b1, const float* w2, float b2,
                        const uint8_t* prunable, const int32_t* cu, int n_seq, float eps,
                        float norm_eps, float* b_raw, float* b, void* ws, hipStream_t st);

size_t select_ws_bytes(int64_t t_in, int n_seq);
hipError_t launch_select(const float* b, const uint8_t* prunable, const int32_t* cu,
                         const int32_t* k, int n_seq, int64_t t_in, int64_t cap,
                         int32_t* kept_idx, int32_t* kept_pos, float* kept_b,
                         int32_t* kept_cu, void* ws, hipStream_t st);

hipError_t launch_gather(const void* src, int64_t src_stride, int64_t n_src, int64_t row_bytes,
                         const int32_t* idx, int64_t n_rows, void* dst, int64_t dst_stride,
                         hipStream_t st);

hipError_t launch_qkv_proj(const void* x, int64_t x_row_stride, int64_t t, int d, const void* w,
                           int nq, int nkv, void* q, void* k, void* v, hipStream_t st);
// The same with the per-head RMSNorm of q and k (weights qn, kn over dh, null
// to skip) and the rotate-half rotary embedding at pos[row] (rope_theta > 1,
// or <= 0 to skip); dh is 64 or 128, nq and nkv multiples of 128.
hipError_t launch_qkv_proj_rope(const void* x, int64_t x_row_stride, int64_t t, int d,
                                const void* w, int nq, int nkv, int dh, const int32_t* pos,
                                const float* qn, const float* kn, float eps, float rope_theta,
                                void* q, void* k, void* v, hipStream_t st);

size_t decode_ws_bytes(int n_seq, int hq, int hkv, int dh, int64_t max_len);
hipError_t launch_decode(const void* q, const void* k, const void* v, void* out,
                         const float* cache_b, const int32_t* cache_cu, const int32_t* q_pos,
                         int n_seq, int64_t t_cache, int64_t max_len, int hq, int hkv, int dh,
                         const float* gain, const float* temp, float sm_scale, void* ws,
                         hipStream_t st);

size_t score_bwd_ws_bytes(int64_t t, int n_seq, int d, int h);
hipError_t launch_score_dz(const void* x, int64_t xs, int64_t t_in, int d, const void* w1,
                           const float* b1, const float* w2, const float* dbt, void* dz, void* dzt,
                           int64_t ldt, float* dw2p, float* db1p, float* db2p, int64_t* blocks,
                           hipStream_t st);
int64_t score_dz_blocks(int64_t t_in, int n_cu);
hipError_t launch_gemm_abt_f32(const void* x, int64_t xs, int64_t m, const void* w, int64_t ldw,
                               int n, int64_t kdim, int splits, float* y, int64_t ldy,
                               hipStream_t st);
// The same with W stored K-major, W[k][n] (rows ldw elements apart, w_rows
// valid rows): Y[m, n] = sum_k X[m, k] W[k, n] over each split's K range.
hipError_t launch_gemm_ab_kmajor_f32(const void* x, int64_t xs, int64_t m, const void* w,
                                     int64_t ldw, int64_t w_rows, int n, int64_t kdim, int splits,
                                     float* y, int64_t ldy, hipStream_t st);
hipError_t launch_score_bwd(const void* x, int dt, int64_t xs, int64_t t, int d, int h,
                            const void* w1, const float* b1, const float* w2, const uint8_t* pr,
                            const int32_t* cu, int n_seq, float eps, const float* b_raw,
                            const int32_t* kept_idx, const int32_t* kept_cu, int64_t t_kept,
                            const float* db_kept, float* dx, float* dw1, float* db1, float* dw2,
                            float* db2, void* ws, hipStream_t st);

size_t attn_bwd_ws_bytes(int64_t t, int n_seq, int hq, int hkv);
// fwd_out and fwd_lse2 (both or neither; bf16 only): the forward's output
// and row statistics.  With them D = rowsum(dO . O) replaces the statistics
// pass and fwd_lse2 is used as the rows' log2-sum-exp.
hipError_t launch_attn_bwd_mfma(const void* q, const void* k, const void* v, const void* dout,
                                int64_t t, const float* kept_b, const int32_t* kept_pos,
                                const int32_t* cu, int n_seq, int hq, int hkv, int dh,
                                const float* gain, const float* temp, float sm, float* lse2,
                                float* dsum, float* dq, float* dk, float* dv, float* dbpart,
                                double* gpart, const void* fwd_out, const float* fwd_lse2,
                                hipStream_t st);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dt,
                           int64_t t, const float* kept_b, const int32_t* kept_pos,
                           const int32_t* cu, int n_seq, int hq, int hkv, int dh,
                           const float* gain, const float* temp, float sm_scale, float* dq,
                           float* dk, float* dv, float* db, float* dgain, float* dtemp,
                           const void* fwd_out, const float* fwd_lse2, void* ws, hipStream_t st);

// lse2 (optional, [hq][t_kept]): each row's log2-sum-exp of its scaled
// logits, the statistic the backward recomputes otherwise
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out,
                            int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                            const int32_t* kept_cu, int n_seq, int max_len, int hq, int hkv,
                            int dh, const float* gain, const float* temp, float sm_scale,
                            float* lse2, hipStream_t st);

hipError_t launch_attn_f32(const void* q, const void* k, const void* v, void* out,
                           int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                           const int32_t* kept_cu, int n_seq, int max_len, int hq, int hkv,
                           int dh, const float* gain, const float* temp, float sm_scale,
                           hipStream_t st);

}  // namespace tg
