// tg_gated_attn_bwd: gradients of token-gated attention (TokenGate §4.2
// Eq. 8 with the gain of Eq. 6 and the temperature of Eq. 7), the path by
// which the loss reaches the gate's scores b_j (§4.3).  With
//   z_ij = s q_i.k_j + g_h b_j,  l_ij = tau_i z_ij (j <= i),  P = softmax_j(l),
//   dP_ij = dO_i.v_j,  D_i = sum_j P_ij dP_ij,  dl_ij = P_ij (dP_ij - D_i):
//   dv_j = sum_i P_ij dO_i            dq_i = s tau_i sum_j dl_ij k_j
//   dk_j = s sum_i tau_i dl_ij q_i    db_j = sum_{h,i} tau_i g_h dl_ij
//   dg_h = sum_ij tau_i b_j dl_ij     dtemp_h = sum_ij lambda_i z_ij dl_ij
//
// fp32 inputs: fp32 arithmetic on the vector ALU, in four launches, all with
// a fixed reduction order (bitwise reproducible); bf16 inputs run the
// matrix-core passes of attn_bwd_mfma.hip and share the last launch:
//   1. bwd_stats  per (64-query tile, head): log2-sum-exp of each row and
//                 D_i, by an online merge over 32-key tiles (no O needed);
//   2. bwd_dkdv   per (32-key tile, KV head): loops over the G heads and the
//                 query tiles at or after it; dK, dV in registers, b's
//                 gradient per KV head to the workspace;
//   3. bwd_dq     per (64-query tile, head): loops over the key tiles; dQ in
//                 registers, the tile's gain / temperature partial sums to
//                 the workspace;
//   4. bwd_finish sums the per-KV-head b gradients and the per-tile gain /
//                 temperature partials.
// Tiles live in LDS as fp32 rows padded by 4 floats; each thread owns a
// 4 x 2 block of the 64 x 32 score tile (rows 4ty + r, columns tx + 16c)
// and 2 x 8 or 4 x 8 blocks of the gradient tiles.  Attention scores are
// recomputed in passes 2 and 3 (P is never stored in HBM).
#include <type_traits>

#include "common.h"

namespace tg {
namespace {

constexpr int kBQ = 64;             // queries per tile
constexpr int kBK = 32;             // keys per tile
constexpr int kThr = 256;
constexpr int kLDP = kBK + 4;       // stride of the P / dS tiles (queries x keys)
constexpr int kLDT = kBQ + 4;       // stride of the transposed dS tile (keys x queries)
constexpr float kLog2e = 1.4426950408889634f;

TG_DEVINL void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
TG_DEVINL void load8(const uint16_t* p, float* o) {
  const u32x4 w = ld16(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(w[k] << 16);
    o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}

// Rows [r0, r0 + R) of head `hd` of a [*, H, DH] tensor whose sequence starts
// at row `lo` and has `len` rows, into LDS as fp32 (zeros past the sequence).
template <int DH, int R, typename T>
TG_DEVINL void load_tile(float* dst, const T* __restrict__ src, int64_t lo, int len, int r0, int H,
                         int hd) {
  constexpr int LD = DH + 4, CPR = DH / 8;
  for (int u = threadIdx.x; u < R * CPR; u += kThr) {
    const int r = u / CPR, c = u % CPR;
    float v[8];
    if (r0 + r < len) {
      load8(src + ((lo + r0 + r) * H + hd) * (int64_t)DH + 8 * c, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    *reinterpret_cast<float4*>(dst + r * LD + 8 * c) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + r * LD + 8 * c + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// acc[r][c] += A[ra + r] . B[rb + 16 c] over DH (rows of padded LDS tiles)
template <int DH, int NR, int NC>
TG_DEVINL void mm_abt(float (&acc)[NR][NC], const float* A, int ra, const float* B, int rb) {
  constexpr int LD = DH + 4;
#pragma unroll 4
  for (int d = 0; d < DH; d += 4) {
    float4 a[NR], b[NC];
#pragma unroll
    for (int r = 0; r < NR; ++r) a[r] = *reinterpret_cast<const float4*>(A + (ra + r) * LD + d);
#pragma unroll
    for (int c = 0; c < NC; ++c) b[c] = *reinterpret_cast<const float4*>(B + (rb + 16 * c) * LD + d);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float t = acc[r][c];
        t = fmaf(a[r].x, b[c].x, t);
        t = fmaf(a[r].y, b[c].y, t);
        t = fmaf(a[r].z, b[c].z, t);
        acc[r][c] = fmaf(a[r].w, b[c].w, t);
      }
  }
}

TG_DEVINL float length_lambda(const int32_t* kept_pos, int64_t row, int local) {
  if (!kept_pos) return 1.0f;
  return logf((float)(local + 1)) / logf(fmaxf(2.0f, (float)kept_pos[row] + 1.0f));
}

// Shared preamble of the query-tile kernels: sequence and first query of a slot.
TG_DEVINL bool query_tile(const int32_t* cu, int n_seq, int64_t t, int64_t slot, int& s,
                          int64_t& lo, int& len, int& q0) {
  s = seq_of_slot(cu, n_seq, slot, kBQ);
  if (s < 0) return false;
  lo = cu[s] < t ? cu[s] : t;
  const int64_t hi = cu[s + 1] < t ? cu[s + 1] : t;
  len = hi > lo ? (int)(hi - lo) : 0;
  q0 = (int)(slot - slot0_of(cu, s, kBQ)) * kBQ;
  return q0 < len;
}

// ---- 1. row statistics: lse2_i = log2 sum_j 2^(l_ij log2e), D_i = sum_j P_ij dP_ij
template <int DH, typename T>
__global__ __launch_bounds__(kThr) void bwd_stats(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ cu, int n_seq, int64_t t,
    int hq, int hkv, const float* __restrict__ gain, const float* __restrict__ temp, float sm,
    float* __restrict__ lse2, float* __restrict__ dsum) {
  constexpr int LD = DH + 4;
  __shared__ __attribute__((aligned(16))) float sQ[kBQ * LD], sO[kBQ * LD];
  __shared__ __attribute__((aligned(16))) float sK[kBK * LD], sV[kBK * LD];
  __shared__ float stau[kBQ], sb[kBK];
  int s, len, q0;
  int64_t lo;
  if (!query_tile(cu, n_seq, t, blockIdx.x, s, lo, len, q0)) return;
  const int h = blockIdx.y, kvh = h / (hq / hkv);
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float g = gain[h];
  if (tid < kBQ)
    stau[tid] = q0 + tid < len ? temp[h] * length_lambda(kept_pos, lo + q0 + tid, q0 + tid) : 0.0f;
  load_tile<DH, kBQ>(sQ, q, lo, len, q0, hq, h);
  load_tile<DH, kBQ>(sO, dout, lo, len, q0, hq, h);
  float m[4], L[4], U[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    L[r] = 0.0f;
    U[r] = 0.0f;
  }
  const int q_end = q0 + kBQ < len ? q0 + kBQ : len;
  for (int k0 = 0; k0 < q_end; k0 += kBK) {
    __syncthreads();
    load_tile<DH, kBK>(sK, k, lo, len, k0, hkv, kvh);
    load_tile<DH, kBK>(sV, v, lo, len, k0, hkv, kvh);
    if (tid < kBK) sb[tid] = k0 + tid < len ? kept_b[lo + k0 + tid] : 0.0f;
    __syncthreads();
    float S[4][2] = {}, dP[4][2] = {};
    mm_abt<DH, 4, 2>(S, sQ, 4 * ty, sK, tx);
    mm_abt<DH, 4, 2>(dP, sO, 4 * ty, sV, tx);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int i = q0 + 4 * ty + r, j = k0 + tx + 16 * c;
        if (i < len && j <= i) {
          const float l2 = stau[4 * ty + r] * fmaf(sm, S[r][c], g * sb[tx + 16 * c]) * kLog2e;
          const float mn = fmaxf(m[r], l2);
          const float f = __builtin_amdgcn_exp2f(m[r] - mn), e = __builtin_amdgcn_exp2f(l2 - mn);
          L[r] = fmaf(L[r], f, e);
          U[r] = fmaf(U[r], f, e * dP[r][c]);
          m[r] = mn;
        }
      }
  }
  // merge the 16 threads of a row group (lanes differing in bits 0-3)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float m2 = __shfl_xor(m[r], o, 64), L2 = __shfl_xor(L[r], o, 64),
                  U2 = __shfl_xor(U[r], o, 64);
      const float mn = fmaxf(m[r], m2);
      if (mn != -INFINITY) {
        const float f1 = __builtin_amdgcn_exp2f(m[r] - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);
        L[r] = L[r] * f1 + L2 * f2;
        U[r] = U[r] * f1 + U2 * f2;
        m[r] = mn;
      }
    }
    const int i = q0 + 4 * ty + r;
    if (tx == 0 && i < len) {
      lse2[(lo + i) * hq + h] = m[r] + __log2f(L[r]);
      dsum[(lo + i) * hq + h] = U[r] / L[r];
    }
  }
}

// scores of one 64 x 32 tile: P (masked) and dS' = dl * tau * s, for thread
// (ty, tx): rows 4ty + r, columns tx + 16c
TG_DEVINL void tile_p_ds(float (&S)[4][2], float (&dP)[4][2], int ty, int tx, int q0, int k0,
                         int len, float sm, float g, const float* stau, const float* slse,
                         const float* sD, const float* sb, float (&P)[4][2], float (&dl)[4][2]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = q0 + 4 * ty + r, j = k0 + tx + 16 * c;
      float p = 0.0f;
      if (i < len && j <= i) {
        const float l2 = stau[4 * ty + r] * fmaf(sm, S[r][c], g * sb[tx + 16 * c]) * kLog2e;
        p = __builtin_amdgcn_exp2f(l2 - slse[4 * ty + r]);
      }
      P[r][c] = p;
      dl[r][c] = p * (dP[r][c] - sD[4 * ty + r]);
    }
}

// ---- 2. dK, dV and the per-KV-head part of db, per (32-key tile, KV head)
template <int DH, typename T>
__global__ __launch_bounds__(kThr) void bwd_dkdv(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ cu, int n_seq, int64_t t,
    int hq, int hkv, const float* __restrict__ gain, const float* __restrict__ temp, float sm,
    const float* __restrict__ lse2, const float* __restrict__ dsum, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dbpart) {
  constexpr int LD = DH + 4, NE = DH / 16;     // d values per thread in the gradient tiles
  __shared__ __attribute__((aligned(16))) float sK[kBK * LD], sV[kBK * LD];
  __shared__ __attribute__((aligned(16))) float sQ[kBQ * LD], sO[kBQ * LD];
  __shared__ __attribute__((aligned(16))) float sP[kBQ * kLDP], sDS[kBQ * kLDP];
  __shared__ float stau[kBQ], slse[kBQ], sD[kBQ], sb[kBK];
  const int s = seq_of_slot(cu, n_seq, blockIdx.x, kBK);
  if (s < 0) return;
  const int64_t lo = cu[s] < t ? cu[s] : t;
  const int64_t hi = cu[s + 1] < t ? cu[s + 1] : t;
  const int len = hi > lo ? (int)(hi - lo) : 0;
  const int k0 = (int)(blockIdx.x - slot0_of(cu, s, kBK)) * kBK;
  if (k0 >= len) return;
  const int kvh = blockIdx.y, G = hq / hkv;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  load_tile<DH, kBK>(sK, k, lo, len, k0, hkv, kvh);
  load_tile<DH, kBK>(sV, v, lo, len, k0, hkv, kvh);
  if (tid < kBK) sb[tid] = k0 + tid < len ? kept_b[lo + k0 + tid] : 0.0f;
  // gradient tiles: thread owns keys 2ty + kk and dims 4tx + e + 64 u
  float aV[2][NE], aK[2][NE];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      aV[kk][e] = 0.0f;
      aK[kk][e] = 0.0f;
    }
  float dbacc = 0.0f;
  for (int hh = 0; hh < G; ++hh) {
    const int h = kvh * G + hh;
    const float g = gain[h];
    for (int q0 = (k0 / kBQ) * kBQ; q0 < len; q0 += kBQ) {
      __syncthreads();
      load_tile<DH, kBQ>(sQ, q, lo, len, q0, hq, h);
      load_tile<DH, kBQ>(sO, dout, lo, len, q0, hq, h);
      if (tid < kBQ) {
        const int i = q0 + tid;
        const bool ok = i < len;
        stau[tid] = ok ? temp[h] * length_lambda(kept_pos, lo + i, i) : 0.0f;
        slse[tid] = ok ? lse2[(lo + i) * hq + h] : 0.0f;
        sD[tid] = ok ? dsum[(lo + i) * hq + h] : 0.0f;
      }
      __syncthreads();
      float S[4][2] = {}, dP[4][2] = {}, P[4][2], dl[4][2];
      mm_abt<DH, 4, 2>(S, sQ, 4 * ty, sK, tx);
      mm_abt<DH, 4, 2>(dP, sO, 4 * ty, sV, tx);
      tile_p_ds(S, dP, ty, tx, q0, k0, len, sm, g, stau, slse, sD, sb, P, dl);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          sP[(4 * ty + r) * kLDP + tx + 16 * c] = P[r][c];
          sDS[(4 * ty + r) * kLDP + tx + 16 * c] = dl[r][c] * stau[4 * ty + r];
        }
      __syncthreads();
      // dV[j] += sum_i P_ij dO_i ;  dK[j] += s * sum_i (tau_i dl_ij) q_i
#pragma unroll 4
      for (int i = 0; i < kBQ; ++i) {
        const float2 p = *reinterpret_cast<const float2*>(sP + i * kLDP + 2 * ty);
        const float2 w = *reinterpret_cast<const float2*>(sDS + i * kLDP + 2 * ty);
#pragma unroll
        for (int u = 0; u < NE / 4; ++u) {
          const float4 o = *reinterpret_cast<const float4*>(sO + i * LD + 64 * u + 4 * tx);
          const float4 x = *reinterpret_cast<const float4*>(sQ + i * LD + 64 * u + 4 * tx);
          const float ov[4] = {o.x, o.y, o.z, o.w}, xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            aV[0][4 * u + e] = fmaf(p.x, ov[e], aV[0][4 * u + e]);
            aV[1][4 * u + e] = fmaf(p.y, ov[e], aV[1][4 * u + e]);
            aK[0][4 * u + e] = fmaf(w.x, xv[e], aK[0][4 * u + e]);
            aK[1][4 * u + e] = fmaf(w.y, xv[e], aK[1][4 * u + e]);
          }
        }
      }
      if (tid < kBK) {                  // db_j += g_h * sum_i tau_i dl_ij
        float cs = 0.0f;
        for (int i = 0; i < kBQ; ++i) cs += sDS[i * kLDP + tid];
        dbacc = fmaf(g, cs, dbacc);
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int j = k0 + 2 * ty + kk;
    if (j < len) {
#pragma unroll
      for (int u = 0; u < NE / 4; ++u) {
        const int64_t off = ((lo + j) * hkv + kvh) * (int64_t)DH + 64 * u + 4 * tx;
        *reinterpret_cast<float4*>(dv + off) =
            make_float4(aV[kk][4 * u], aV[kk][4 * u + 1], aV[kk][4 * u + 2], aV[kk][4 * u + 3]);
        *reinterpret_cast<float4*>(dk + off) =
            make_float4(sm * aK[kk][4 * u], sm * aK[kk][4 * u + 1], sm * aK[kk][4 * u + 2],
                        sm * aK[kk][4 * u + 3]);
      }
    }
  }
  if (tid < kBK && k0 + tid < len) dbpart[(int64_t)kvh * t + lo + k0 + tid] = dbacc;
}

// ---- 3. dQ and the gain / temperature partial sums, per (64-query tile, head)
template <int DH, typename T>
__global__ __launch_bounds__(kThr) void bwd_dq(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ cu, int n_seq, int64_t t,
    int hq, int hkv, const float* __restrict__ gain, const float* __restrict__ temp, float sm,
    const float* __restrict__ lse2, const float* __restrict__ dsum, float* __restrict__ dq,
    double* __restrict__ gpart) {
  constexpr int LD = DH + 4, NE = DH / 16;
  __shared__ __attribute__((aligned(16))) float sQ[kBQ * LD], sO[kBQ * LD];
  __shared__ __attribute__((aligned(16))) float sK[kBK * LD], sV[kBK * LD];
  __shared__ __attribute__((aligned(16))) float sDT[kBK * kLDT];
  __shared__ float stau[kBQ], slam[kBQ], slse[kBQ], sD[kBQ], sb[kBK];
  __shared__ double sred[2][kThr / 64];
  const int h = blockIdx.y, kvh = h / (hq / hkv);
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  double* gp = gpart + ((int64_t)blockIdx.x * hq + h) * 2;
  int s, len, q0;
  int64_t lo;
  if (!query_tile(cu, n_seq, t, blockIdx.x, s, lo, len, q0)) {
    if (tid == 0) {                      // every slot leaves a partial, zero here
      gp[0] = 0.0;
      gp[1] = 0.0;
    }
    return;
  }
  const float g = gain[h];
  if (tid < kBQ) {
    const int i = q0 + tid;
    const bool ok = i < len;
    const float lam = ok ? length_lambda(kept_pos, lo + i, i) : 0.0f;
    slam[tid] = lam;
    stau[tid] = temp[h] * lam;
    slse[tid] = ok ? lse2[(lo + i) * hq + h] : 0.0f;
    sD[tid] = ok ? dsum[(lo + i) * hq + h] : 0.0f;
  }
  load_tile<DH, kBQ>(sQ, q, lo, len, q0, hq, h);
  load_tile<DH, kBQ>(sO, dout, lo, len, q0, hq, h);
  float aQ[4][NE];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < NE; ++e) aQ[r][e] = 0.0f;
  double accg = 0.0, acct = 0.0;        // sums of both signs over every pair: fp64
  const int q_end = q0 + kBQ < len ? q0 + kBQ : len;
  for (int k0 = 0; k0 < q_end; k0 += kBK) {
    __syncthreads();
    load_tile<DH, kBK>(sK, k, lo, len, k0, hkv, kvh);
    load_tile<DH, kBK>(sV, v, lo, len, k0, hkv, kvh);
    if (tid < kBK) sb[tid] = k0 + tid < len ? kept_b[lo + k0 + tid] : 0.0f;
    __syncthreads();
    float S[4][2] = {}, dP[4][2] = {}, P[4][2], dl[4][2];
    mm_abt<DH, 4, 2>(S, sQ, 4 * ty, sK, tx);
    mm_abt<DH, 4, 2>(dP, sO, 4 * ty, sV, tx);
    tile_p_ds(S, dP, ty, tx, q0, k0, len, sm, g, stau, slse, sD, sb, P, dl);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float tdl = dl[r][c] * stau[4 * ty + r];
        const float bj = sb[tx + 16 * c];
        sDT[(tx + 16 * c) * kLDT + 4 * ty + r] = tdl;
        accg = fma((double)tdl, (double)bj, accg);
        acct = fma((double)(dl[r][c] * slam[4 * ty + r]), (double)fmaf(sm, S[r][c], g * bj), acct);
      }
    __syncthreads();
    // dQ_i += sum_j (tau_i dl_ij) k_j   (times s at the end)
#pragma unroll 4
    for (int j = 0; j < kBK; ++j) {
      const float4 w = *reinterpret_cast<const float4*>(sDT + j * kLDT + 4 * ty);
      const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int u = 0; u < NE / 4; ++u) {
        const float4 kk = *reinterpret_cast<const float4*>(sK + j * LD + 64 * u + 4 * tx);
        const float kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) aQ[r][4 * u + e] = fmaf(wv[r], kv[e], aQ[r][4 * u + e]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = q0 + 4 * ty + r;
    if (i < len) {
#pragma unroll
      for (int u = 0; u < NE / 4; ++u) {
        const int64_t off = ((lo + i) * hq + h) * (int64_t)DH + 64 * u + 4 * tx;
        *reinterpret_cast<float4*>(dq + off) =
            make_float4(sm * aQ[r][4 * u], sm * aQ[r][4 * u + 1], sm * aQ[r][4 * u + 2],
                        sm * aQ[r][4 * u + 3]);
      }
    }
  }
  accg = wave_sum(accg);
  acct = wave_sum(acct);
  if ((tid & 63) == 0) {
    sred[0][tid >> 6] = accg;
    sred[1][tid >> 6] = acct;
  }
  __syncthreads();
  if (tid == 0) {
    gp[0] = (sred[0][0] + sred[0][1]) + (sred[0][2] + sred[0][3]);
    gp[1] = (sred[1][0] + sred[1][1]) + (sred[1][2] + sred[1][3]);
  }
}

// ---- 4. db over the KV heads; dgain, dtemp over the query tiles
__global__ __launch_bounds__(kThr) void bwd_finish(const float* __restrict__ dbpart,
                                                   const double* __restrict__ gpart,
                                                   const int32_t* __restrict__ cu, int n_seq,
                                                   int64_t t, int hq, int hkv, int64_t n_qslots,
                                                   float* __restrict__ db,
                                                   float* __restrict__ dgain,
                                                   float* __restrict__ dtemp) {
  const int64_t n_rows = cu[n_seq] < t ? cu[n_seq] : t;
  const int64_t nb = (t + kThr - 1) / kThr;
  if (blockIdx.x < nb) {
    const int64_t j = (int64_t)blockIdx.x * kThr + threadIdx.x;
    if (j < t) {
      float acc = 0.0f;
      if (j < n_rows)
        for (int kv = 0; kv < hkv; ++kv) acc += dbpart[(int64_t)kv * t + j];
      db[j] = acc;
    }
    return;
  }
  for (int h = threadIdx.x; h < hq; h += kThr) {
    double ag = 0.0, at = 0.0;
    for (int64_t sl = 0; sl < n_qslots; ++sl) {
      ag += gpart[(sl * hq + h) * 2];
      at += gpart[(sl * hq + h) * 2 + 1];
    }
    dgain[h] = (float)ag;
    dtemp[h] = (float)at;
  }
}

int64_t qslots(int64_t t, int n_seq) { return (int64_t)n_seq + (t + kBQ - 1) / kBQ; }
int64_t kslots(int64_t t, int n_seq) { return (int64_t)n_seq + (t + kBK - 1) / kBK; }

template <int DH, typename T>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* dout, int64_t t,
                    const float* kept_b, const int32_t* kept_pos, const int32_t* cu, int n_seq,
                    int hq, int hkv, const float* gain, const float* temp, float sm, float* dq,
                    float* dk, float* dv, float* db, float* dgain, float* dtemp,
                    const void* fwd_out, const float* fwd_lse2, void* ws, hipStream_t st) {
  float* lse2 = static_cast<float*>(ws);
  float* dsum = lse2 + t * hq;
  float* dbpart = dsum + t * hq;
  // fp64 partials, 8-byte aligned after the fp32 arrays
  double* gpart = reinterpret_cast<double*>(
      reinterpret_cast<uintptr_t>(dbpart + t * hkv + 1) & ~(uintptr_t)7);
  const T* qp = static_cast<const T*>(q);
  const T* kp = static_cast<const T*>(k);
  const T* vp = static_cast<const T*>(v);
  const T* op = static_cast<const T*>(dout);
  const int64_t nq = qslots(t, n_seq), nk = kslots(t, n_seq);
  if constexpr (std::is_same<T, uint16_t>::value) {
    // bf16: the matrix-core passes, then the shared final sums
    const hipError_t e = launch_attn_bwd_mfma(q, k, v, dout, t, kept_b, kept_pos, cu, n_seq, hq,
                                              hkv, DH, gain, temp, sm, lse2, dsum, dq, dk, dv,
                                              dbpart, gpart, fwd_out, fwd_lse2, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_finish, dim3((unsigned)((t + kThr - 1) / kThr + 1)), dim3(kThr), 0, st,
                       dbpart, gpart, cu, n_seq, t, hq, hkv, attn_bwd_mfma_gslots(t, n_seq), db,
                       dgain, dtemp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bwd_stats<DH, T>), dim3((unsigned)nq, hq), dim3(kThr), 0, st, qp, kp, vp,
                     op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse2, dsum);
  hipLaunchKernelGGL((bwd_dkdv<DH, T>), dim3((unsigned)nk, hkv), dim3(kThr), 0, st, qp, kp, vp,
                     op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse2, dsum, dk,
                     dv, dbpart);
  hipLaunchKernelGGL((bwd_dq<DH, T>), dim3((unsigned)nq, hq), dim3(kThr), 0, st, qp, kp, vp, op,
                     kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse2, dsum, dq,
                     gpart);
  hipLaunchKernelGGL(bwd_finish, dim3((unsigned)((t + kThr - 1) / kThr + 1)), dim3(kThr), 0, st,
                     dbpart, gpart, cu, n_seq, t, hq, hkv, nq, db, dgain, dtemp);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_ws_bytes(int64_t t, int n_seq, int hq, int hkv) {
  return sizeof(float) * (size_t)(2 * t * hq + t * hkv + 2) +
         sizeof(double) * (size_t)(qslots(t, n_seq) * hq * 2);
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dt,
                           int64_t t, const float* kept_b, const int32_t* kept_pos,
                           const int32_t* cu, int n_seq, int hq, int hkv, int dh,
                           const float* gain, const float* temp, float sm_scale, float* dq,
                           float* dk, float* dv, float* db, float* dgain, float* dtemp,
                           const void* fwd_out, const float* fwd_lse2, void* ws, hipStream_t st) {
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / sqrtf((float)dh);
#define TG_BWD(DHv, Tv)                                                                         \
  return launch_t<DHv, Tv>(q, k, v, dout, t, kept_b, kept_pos, cu, n_seq, hq, hkv, gain, temp, \
                           sm_scale, dq, dk, dv, db, dgain, dtemp, fwd_out, fwd_lse2, ws, st);
  if (dt == 1) {
    if (dh == 128) { TG_BWD(128, uint16_t) }
    if (dh == 64) { TG_BWD(64, uint16_t) }
  } else {
    if (dh == 128) { TG_BWD(128, float) }
    if (dh == 64) { TG_BWD(64, float) }
  }
#undef TG_BWD
  return hipErrorInvalidValue;
}

}  // namespace tg
