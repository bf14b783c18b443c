// Shared device helpers and internal launch entry points of libtokengate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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
// DPP move of a value of any size (a multiple of 4 bytes), word by word:
// CTRL is a full permutation of the lanes of each row of 16
template <int CTRL, typename T>
TG_DEVINL T dpp_move(T v) {
  static_assert(sizeof(T) % 4 == 0, "whole 32-bit words");
  struct Words {
    int w[sizeof(T) / 4];
  };
  Words a = __builtin_bit_cast(Words, v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i)
    a.w[i] = __builtin_amdgcn_update_dpp(0, a.w[i], CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(T, a);
}
template <typename T>
TG_DEVINL T read_lane(T v, int l) {
  struct Words {
    int w[sizeof(T) / 4];
  };
  Words a = __builtin_bit_cast(Words, v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) a.w[i] = __builtin_amdgcn_readlane(a.w[i], l);
  return __builtin_bit_cast(T, a);
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]: lane i <-> i ^ 1
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]: lane i <-> i ^ 2
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7 - i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15 - i within each 16

// Sum over the 64 lanes of a wave (all lanes active), the same value in every
// lane: DPP butterflies inside each row of 16 lanes (partners i ^ 1, i ^ 2,
// then the mirrored half row and the mirrored row; both partners add the
// same two values, so every lane of a row holds the same sum), then the four
// row sums in a fixed order.  No LDS round trips.
template <typename T>
TG_DEVINL T wave_sum(T v) {
  v += dpp_move<kDppQuadXor1>(v);
  v += dpp_move<kDppQuadXor2>(v);
  v += dpp_move<kDppRowHalfMirror>(v);
  v += dpp_move<kDppRowMirror>(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

TG_DEVINL float wave_max(float v) {
  v = fmaxf(v, dpp_move<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_move<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_move<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_move<kDppRowMirror>(v));
  return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}

// inclusive prefix sum over the 64 lanes of a wave (all lanes active): DPP
// shifts right by 1, 2, 4 and 8 inside each row of 16 lanes (lanes with no
// source in the row add 0), then each row adds the totals of the rows below
// it, read from lanes 15, 31 and 47.  No LDS round trips, unlike a shuffle
// per step.
TG_DEVINL int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
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

constexpr int kMaxDevices = 64;      // devices the per-device host caches cover

// compute units of the current device (host side; sizes the persistent
// attention grid and the scorer's row tiles), cached per device; the cache
// entries are atomics, so concurrent first calls race benignly (both store
// the same value)
hipError_t device_cu_count(int* n_cu);

// Device-side contract checks (contract.hip): on/off switch, and launchers
// of the check kernels, each ORing its TG_CONTRACT_* bit into this device's
// flag word.
bool contract_checks_on();
void set_contract_checks(bool on);
hipError_t contract_offsets(const int32_t* cu, int n, int64_t limit, unsigned int bit,
                            hipStream_t st);
hipError_t contract_budgets(const int32_t* k, int n, hipStream_t st);
hipError_t contract_capacity(const int32_t* kept_cu, int n, int64_t cap, hipStream_t st);
hipError_t contract_indices(const int32_t* idx, int64_t n, int64_t n_src, hipStream_t st);
hipError_t contract_positions(const int32_t* pos, const int32_t* cu, int n_seq, int64_t t,
                              hipStream_t st);
hipError_t contract_read_and_clear(unsigned int* out, hipStream_t st);

// Bytes of the selector's static scratch array (tg_select_topk_noalloc).
constexpr size_t kSelScratchBytes = (size_t)8 << 20;
// Device address of this GPU's copy of that array (looked up once per device).
hipError_t select_scratch(void** ptr);

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
                           const float* b1, const float* w2, const float* dbt, void* dz,
                           float* dw2p, float* db1p, float* db2p, float norm_eps, float* rowc,
                           int64_t* blocks, hipStream_t st);
int64_t score_dz_blocks(int64_t t_in, int n_cu);
// rowc (optional, splits == 1 only): Y[m, n] -= rowc[m] * A[m, n] after the
// product, A bf16 with rows lda elements apart (the LN2 term of the scorer's
// input gradient)
hipError_t launch_gemm_abt_f32(const void* x, int64_t xs, int64_t m, const void* w, int64_t ldw,
                               int n, int64_t kdim, int splits, float* y, int64_t ldy,
                               hipStream_t st, const float* rowc = nullptr,
                               const void* a = nullptr, int64_t lda = 0);
// Both operands stored K-major, A[k][m] (rows lda elements apart) and W[k][n]
// (rows ldw apart), k_rows valid rows in each (later ones read as zeros):
// Y[m, n] = sum_k A[k, m] W[k, n] over each split's K range; m <= 256.
hipError_t launch_gemm_atb_kmajor_f32(const void* a, int64_t lda, int64_t m, const void* w,
                                      int64_t ldw, int64_t k_rows, int n, int64_t kdim,
                                      int splits, float* y, int64_t ldy, hipStream_t st);
hipError_t launch_score_bwd(const void* x, int dt, int64_t xs, int64_t t, int d, int h,
                            const void* w1, const float* b1, const float* w2, const uint8_t* pr,
                            const int32_t* cu, int n_seq, float eps, float norm_eps,
                            const float* b_raw,
                            const int32_t* kept_idx, const int32_t* kept_cu, int64_t t_kept,
                            const float* db_kept, float* dx, float* dw1, float* db1, float* dw2,
                            float* db2, void* ws, hipStream_t st);

size_t attn_bwd_ws_bytes(int64_t t, int n_seq, int hq, int hkv);
// slots of the gain / temperature partials the matrix-core dQ pass writes
// (one per block of its queries; no more than the vector-ALU passes' slots)
int64_t attn_bwd_mfma_gslots(int64_t t, int n_seq);
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
// ws (optional, attn_split_ws_bytes): with it the workgroups draw their
// query blocks from a work counter, and blocks with more key tiles than a
// workgroup's share are split into key chunks whose partial results a second
// launch merges
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out,
                            int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                            const int32_t* kept_cu, int n_seq, int max_len, int hq, int hkv,
                            int dh, const float* gain, const float* temp, float sm_scale,
                            float* lse2, hipStream_t st, void* ws = nullptr);
size_t attn_split_ws_bytes(int64_t t_kept, int n_seq, int max_len, int hq, int hkv, int dh);

hipError_t launch_attn_f32(const void* q, const void* k, const void* v, void* out,
                           int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                           const int32_t* kept_cu, int n_seq, int max_len, int hq, int hkv,
                           int dh, const float* gain, const float* temp, float sm_scale,
                           hipStream_t st);

}  // namespace tg
