// tg_score_bwd: gradients of the gate's scorer (TokenGate §4.1 Eq. 3) from
// the gradient that reaches the kept scores b through the attention (§4.3).
// Per sequence, with prunable set P, r = sqrt(mean_P b~^2 + eps) and
// C = sum_{kept j in P} db_j b~_j:
//   db~_k = [k kept] db_k / r - b~_k C / (|P| r^3)   (k in P; 0 on prompt tokens)
// then through z = W1 x + b1, u = SiLU(z), b~ = w2 . u + b2:
//   dz = db~ w2 SiLU'(z),  dW1 = sum_j dz_j x_j^T,  dx_j = W1^T dz_j,
//   db1 = sum_j dz_j,      dw2 = sum_j db~_j u_j,    db2 = sum_j db~_j.
//
// bf16 inputs with h = 256 and d % 256 == 0 run the products on the matrix
// cores: z is recomputed by the scorer's own MFMA tiling with a backward
// epilogue (dz in bf16 in both layouts, per-workgroup dw2 / db1 / db2 sums),
// W1 is transposed once (x is read as stored: the GEMM core's K-major form
// stages its token-major tiles and transposes them on the LDS reads), and
// dW1 = dz^T x (split over token ranges) and dx = dz W1 run on the
// projection's GEMM core with fp32 output.  dz
// enters both products rounded to bf16.  Otherwise (fp32 inputs, other
// shapes) everything is fp32 on the vector ALU, seven launches, fixed
// reduction orders:
//   sbwd_part, sbwd_cpart, sbwd_seq   per 2048-token / kept-row chunk, then
//               per sequence: r, |P| and C (fp64 sums) -> 1/r, C/(|P| r^3)
//   sbwd_dbt    per token: the normaliser term (every prunable token)
//   sbwd_kept   per kept row: db / r plus the normaliser term at its token, in
//               fp64 (the two nearly cancel in sequences of few prunable tokens)
//   sbwd_dz     per 64 tokens x 64 hidden units: recomputes z (K = d), writes
//               dz and the block's dw2, db1, db2 partial sums
//   sbwd_dw1    per 64 hidden x 64 input columns and token split: dz^T x
//   sbwd_dx     per 64 tokens x 64 input columns: dz W1 (K = h)
//   sbwd_finish sums the partials.
// The products are register-blocked micro-GEMMs over padded fp32 LDS tiles,
// each thread owning 4 x 4 outputs (rows 4ty + r, columns tx + 16c).
//
// LN2 in front of the scorer (norm_eps >= 0; x rows are the residual a, W1
// carries the norm's weight, §3 Eq. 1): with inv = 1 / sqrt(mean_c a_c^2 +
// norm_eps) per row and z = inv W1 a + b1, the stored dz is dz inv, so the
// same products give dW1 = sum_j (dz inv)_j a_j^T and the first part of
//   da_j = W1^T (dz inv)_j - c_j a_j,   c_j = inv^3 / d * sum_h dz_jh (W1 a_j)_h,
// the second being the derivative of the norm itself.  The matrix-core path
// takes inv and c from the scorer's epilogue and subtracts c a in the dx
// product's epilogue; the vector path has a row pass for inv (sbwd_rowinv),
// per-64-hidden-unit partials of c from sbwd_dz, and the subtraction in
// sbwd_dx.
#include <type_traits>

#include "common.h"

namespace tg {
namespace {

constexpr int kThr = 256;
constexpr int kT = 64;              // output tile edge
constexpr int kKC = 32;             // reduction chunk
constexpr int kSplitMax = 8;        // token splits of dW1

TG_DEVINL float ldf(const float* p) { return *p; }
TG_DEVINL float ldf(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

TG_DEVINL int seq_of_row(const int32_t* cu, int n_seq, int64_t row) {
  int lo = 0, hi = n_seq - 1, ans = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) {
      ans = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  return ans;
}

// ---- per sequence: 1/r and C / (|P| r^3), from chunk partials (fp64)
constexpr int kCh = 2048;            // tokens (or kept rows) per partial

struct SqPart {
  double sq;
  int64_t n;
};

// sum of b~^2 and count over the prunable tokens of one 2048-token chunk
__global__ __launch_bounds__(kThr) void sbwd_part(const float* __restrict__ b_raw,
                                                  const uint8_t* __restrict__ pr,
                                                  const int32_t* __restrict__ cu, int n_seq,
                                                  int64_t t, SqPart* __restrict__ part) {
  __shared__ double s1[kThr / 64];
  __shared__ int64_t sn[kThr / 64];
  const int64_t slot = blockIdx.x;
  const int s = seq_of_slot(cu, n_seq, slot, kCh);
  double sq = 0.0;
  int64_t n = 0;
  if (s >= 0) {
    const int64_t lo = cu[s] < t ? cu[s] : t, hi = cu[s + 1] < t ? cu[s + 1] : t;
    const int64_t b0 = lo + (slot - slot0_of(cu, s, kCh)) * kCh;
    const int64_t e0 = b0 + kCh < hi ? b0 + kCh : hi;
    for (int64_t j = b0 + threadIdx.x; j < e0; j += kThr)
      if (pr[j]) {
        const double v = b_raw[j];
        sq = fma(v, v, sq);
        ++n;
      }
  }
  sq = wave_sum(sq);
  n = wave_sum(n);
  if ((threadIdx.x & 63) == 0) {
    s1[threadIdx.x >> 6] = sq;
    sn[threadIdx.x >> 6] = n;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    part[slot].sq = (s1[0] + s1[1]) + (s1[2] + s1[3]);
    part[slot].n = sn[0] + sn[1] + sn[2] + sn[3];
  }
}

// sum of db * b~ over the kept prunable rows of one 2048-row chunk
__global__ __launch_bounds__(kThr) void sbwd_cpart(const float* __restrict__ b_raw,
                                                   const uint8_t* __restrict__ pr,
                                                   const int32_t* __restrict__ kept_idx,
                                                   const int32_t* __restrict__ kept_cu, int n_seq,
                                                   int64_t t, int64_t t_kept,
                                                   const float* __restrict__ db_kept,
                                                   double* __restrict__ cpart) {
  __shared__ double s1[kThr / 64];
  const int64_t slot = blockIdx.x;
  const int s = seq_of_slot(kept_cu, n_seq, slot, kCh);
  double c = 0.0;
  if (s >= 0) {
    const int64_t lo = kept_cu[s] < t_kept ? kept_cu[s] : t_kept;
    const int64_t hi = kept_cu[s + 1] < t_kept ? kept_cu[s + 1] : t_kept;
    const int64_t b0 = lo + (slot - slot0_of(kept_cu, s, kCh)) * kCh;
    const int64_t e0 = b0 + kCh < hi ? b0 + kCh : hi;
    for (int64_t r = b0 + threadIdx.x; r < e0; r += kThr) {
      const int64_t j = kept_idx[r];
      if (j >= 0 && j < t && pr[j]) c = fma((double)db_kept[r], (double)b_raw[j], c);
    }
  }
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) s1[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) cpart[slot] = (s1[0] + s1[1]) + (s1[2] + s1[3]);
}

// per sequence: its chunk partials in order -> (1/r, C / (|P| r^3)), in fp64
__global__ __launch_bounds__(64) void sbwd_seq(const int32_t* __restrict__ cu,
                                               const int32_t* __restrict__ kept_cu,
                                               const SqPart* __restrict__ part,
                                               const double* __restrict__ cpart, float eps,
                                               double2* __restrict__ seqc) {
  const int s = blockIdx.x;
  if (threadIdx.x != 0) return;
  const int64_t p0 = slot0_of(cu, s, kCh), p1 = slot0_of(cu, s + 1, kCh);
  const int64_t c0 = slot0_of(kept_cu, s, kCh), c1 = slot0_of(kept_cu, s + 1, kCh);
  double SQ = 0.0, CC = 0.0;
  int64_t N = 0;
  for (int64_t i = p0; i < p1; ++i) {
    SQ += part[i].sq;
    N += part[i].n;
  }
  for (int64_t i = c0; i < c1; ++i) CC += cpart[i];
  double2 out = make_double2(0.0, 0.0);
  if (N > 0) {
    const double r = sqrt(SQ / (double)N + (double)eps);
    out = make_double2(1.0 / r, CC / ((double)N * r * r * r));
  }
  seqc[s] = out;
}

// ---- per token: db~ = -b~ C / (|P| r^3) on prunable tokens, 0 elsewhere
__global__ __launch_bounds__(kThr) void sbwd_dbt(const float* __restrict__ b_raw,
                                                 const uint8_t* __restrict__ pr,
                                                 const int32_t* __restrict__ cu, int n_seq,
                                                 int64_t t, const double2* __restrict__ seqc,
                                                 float* __restrict__ dbt) {
  const int64_t j = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (j >= t) return;
  const int s = seq_of_row(cu, n_seq, j);
  const bool in = s >= 0 && j < cu[s + 1];
  dbt[j] = (in && pr[j]) ? (float)(-(double)b_raw[j] * seqc[s].y) : 0.0f;
}

// ---- per kept row: db~ = db / r - b~ C / (|P| r^3) at the kept token (prunable
// only: b := 0 on prompts)
__global__ __launch_bounds__(kThr) void sbwd_kept(const float* __restrict__ b_raw,
                                                  const uint8_t* __restrict__ pr,
                                                  const int32_t* __restrict__ kept_idx,
                                                  const int32_t* __restrict__ kept_cu, int n_seq,
                                                  int64_t t, int64_t t_kept,
                                                  const float* __restrict__ db_kept,
                                                  const double2* __restrict__ seqc,
                                                  float* __restrict__ dbt) {
  const int64_t r = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (r >= t_kept) return;
  const int s = seq_of_row(kept_cu, n_seq, r);
  if (s < 0 || r >= kept_cu[s + 1]) return;
  const int64_t j = kept_idx[r];
  // the whole value in fp64, rounded once: the two terms nearly cancel when
  // the sequence has few prunable tokens (one token: db eps / r^3)
  if (j >= 0 && j < t && pr[j])
    dbt[j] = (float)fma((double)db_kept[r], seqc[s].x, -(double)b_raw[j] * seqc[s].y);
}

// ---- LN2: 1 / RMS of each row, one wave per row (4 rows per block)
template <typename T>
__global__ __launch_bounds__(kThr) void sbwd_rowinv(const T* __restrict__ x, int64_t xs, int64_t t,
                                                    int d, float norm_eps,
                                                    float* __restrict__ inv) {
  const int64_t j = (int64_t)blockIdx.x * (kThr / 64) + (threadIdx.x >> 6);
  if (j >= t) return;
  float ss = 0.0f;
  for (int c = threadIdx.x & 63; c < d; c += 64) {
    const float v = ldf(x + j * xs + c);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) inv[j] = 1.0f / sqrtf(ss / (float)d + norm_eps);
}

// ---- dz for 64 tokens x 64 hidden units; z recomputed over d.  With inv
// (LN2): z = inv acc + b1, the stored dz is dz inv, and rowp[blockIdx.y][j]
// gets this block's sum over its hidden units of dz acc (for c_j).
template <typename T>
__global__ __launch_bounds__(kThr) void sbwd_dz(const T* __restrict__ x, int64_t xs, int64_t t,
                                                int d, int h, const T* __restrict__ w1,
                                                const float* __restrict__ b1,
                                                const float* __restrict__ w2,
                                                const float* __restrict__ dbt,
                                                float* __restrict__ dz, float* __restrict__ dw2p,
                                                float* __restrict__ db1p,
                                                float* __restrict__ db2p,
                                                const float* __restrict__ inv,
                                                float* __restrict__ rowp) {
  constexpr int LD = kKC + 4;
  __shared__ __attribute__((aligned(16))) float sx[kT * LD], sw[kT * LD];
  __shared__ float sred[2][16][kT];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t j0 = (int64_t)blockIdx.x * kT;
  const int h0 = blockIdx.y * kT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += kKC) {
    __syncthreads();
    for (int u = tid; u < kT * kKC; u += kThr) {
      const int r = u / kKC, c = u % kKC;
      sx[r * LD + c] = j0 + r < t ? ldf(x + (j0 + r) * xs + k0 + c) : 0.0f;
      sw[r * LD + c] = ldf(w1 + (int64_t)(h0 + r) * d + k0 + c);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKC; k += 4) {
      float4 a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = *reinterpret_cast<const float4*>(sx + (4 * ty + r) * LD + k);
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = *reinterpret_cast<const float4*>(sw + (tx + 16 * c) * LD + k);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float v = acc[r][c];
          v = fmaf(a[r].x, b[c].x, v);
          v = fmaf(a[r].y, b[c].y, v);
          v = fmaf(a[r].z, b[c].z, v);
          acc[r][c] = fmaf(a[r].w, b[c].w, v);
        }
    }
  }
  float pu[4] = {0.f, 0.f, 0.f, 0.f}, pz[4] = {0.f, 0.f, 0.f, 0.f};   // per hidden column c
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t j = j0 + 4 * ty + r;
    const float g = j < t ? dbt[j] : 0.0f;
    const float iv = inv && j < t ? inv[j] : 1.0f;
    float pc = 0.0f;                                  // LN2: sum over the row's columns of dz acc
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int hid = h0 + tx + 16 * c;
      const float z = fmaf(acc[r][c], iv, b1 ? b1[hid] : 0.0f);
      const float sg = 1.0f / (1.0f + expf(-z));
      const float dzv = g * w2[hid] * sg * fmaf(z, 1.0f - sg, 1.0f);
      if (j < t) dz[j * h + hid] = dzv * iv;
      pu[c] = fmaf(g, z * sg, pu[c]);
      pz[c] += dzv;
      pc = fmaf(dzv, acc[r][c], pc);
    }
    if (inv) {
      // the 16 threads of a row are 16 consecutive lanes (tx)
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) pc += __shfl_xor(pc, o, 64);
      if (tx == 0 && j < t) rowp[(int64_t)blockIdx.y * t + j] = pc;
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    sred[0][ty][tx + 16 * c] = pu[c];
    sred[1][ty][tx + 16 * c] = pz[c];
  }
  __syncthreads();
  if (tid < kT) {
    float a = 0.0f, b = 0.0f;
    for (int y = 0; y < 16; ++y) {
      a += sred[0][y][tid];
      b += sred[1][y][tid];
    }
    dw2p[(int64_t)blockIdx.x * h + h0 + tid] = a;
    db1p[(int64_t)blockIdx.x * h + h0 + tid] = b;
  }
  if (blockIdx.y == 0 && tid == 64) {
    float a = 0.0f;
    for (int r = 0; r < kT; ++r) a += j0 + r < t ? dbt[j0 + r] : 0.0f;
    db2p[blockIdx.x] = a;
  }
}

// ---- dW1 partial of one token split: [64 hidden x 64 columns] += dz^T x
template <typename T>
__global__ __launch_bounds__(kThr) void sbwd_dw1(const T* __restrict__ x, int64_t xs, int64_t t,
                                                 int d, int h, const float* __restrict__ dz,
                                                 int64_t per_split, float* __restrict__ dw1p) {
  constexpr int LD = kT + 4;
  __shared__ __attribute__((aligned(16))) float sz[kKC * LD], sx[kKC * LD];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int h0 = blockIdx.x * kT, c0 = blockIdx.y * kT;
  const int64_t jb = (int64_t)blockIdx.z * per_split;
  const int64_t je = jb + per_split < t ? jb + per_split : t;
  float acc[4][4] = {};
  for (int64_t j0 = jb; j0 < je; j0 += kKC) {
    __syncthreads();
    for (int u = tid; u < kKC * kT; u += kThr) {
      const int r = u / kT, c = u % kT;
      const bool ok = j0 + r < je;
      sz[r * LD + c] = ok ? dz[(j0 + r) * h + h0 + c] : 0.0f;
      sx[r * LD + c] = ok ? ldf(x + (j0 + r) * xs + c0 + c) : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kKC; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(sz + k * LD + 4 * ty);
      const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float b = sx[k * LD + tx + 16 * c];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][c] = fmaf(av[r], b, acc[r][c]);
      }
    }
  }
  float* out = dw1p + (int64_t)blockIdx.z * h * d;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) out[(int64_t)(h0 + 4 * ty + r) * d + c0 + tx + 16 * c] = acc[r][c];
}

// ---- dx for 64 tokens x 64 columns: dz W1 over the hidden units; with inv
// (LN2) minus c_j x_j, c_j = inv^3 / d * (sum of the nhb partials in rowp)
template <typename T>
__global__ __launch_bounds__(kThr) void sbwd_dx(int64_t t, int d, int h, const T* __restrict__ w1,
                                                const float* __restrict__ dz,
                                                float* __restrict__ dx,
                                                const T* __restrict__ x, int64_t xs,
                                                const float* __restrict__ inv,
                                                const float* __restrict__ rowp, int nhb) {
  constexpr int LDZ = kT + 4, LDW = kT + 4;
  __shared__ __attribute__((aligned(16))) float szt[kKC * LDZ], sw[kKC * LDW];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t j0 = (int64_t)blockIdx.x * kT;
  const int c0 = blockIdx.y * kT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < h; k0 += kKC) {
    __syncthreads();
    for (int u = tid; u < kKC * kT; u += kThr) {
      const int r = u / kKC, k = u % kKC;          // token r, hidden k0 + k (transposed store)
      szt[k * LDZ + r] = j0 + r < t ? dz[(j0 + r) * h + k0 + k] : 0.0f;
      const int kk = u / kT, c = u % kT;
      sw[kk * LDW + c] = ldf(w1 + (int64_t)(k0 + kk) * d + c0 + c);
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kKC; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(szt + k * LDZ + 4 * ty);
      const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float b = sw[k * LDW + tx + 16 * c];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][c] = fmaf(av[r], b, acc[r][c]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t j = j0 + 4 * ty + r;
    if (j < t) {
      float cj = 0.0f;
      if (inv) {
        for (int k = 0; k < nhb; ++k) cj += rowp[(int64_t)k * t + j];
        const float iv = inv[j];
        cj *= iv * iv * iv / (float)d;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = c0 + tx + 16 * c;
        dx[j * d + col] = inv ? fmaf(-cj, ldf(x + j * xs + col), acc[r][c]) : acc[r][c];
      }
    }
  }
}

// ---- sums of the partials
__global__ __launch_bounds__(kThr) void sbwd_finish(int64_t hd, int h, int n_split, int64_t n_tb,
                                                    const float* __restrict__ dw1p,
                                                    const float* __restrict__ dw2p,
                                                    const float* __restrict__ db1p,
                                                    const float* __restrict__ db2p,
                                                    float* __restrict__ dw1,
                                                    float* __restrict__ dw2,
                                                    float* __restrict__ db1,
                                                    float* __restrict__ db2) {
  __shared__ float sa[kThr / 64], sb[kThr / 64];
  const int64_t nb = (hd + kThr - 1) / kThr;
  if (blockIdx.x < nb) {
    const int64_t e = (int64_t)blockIdx.x * kThr + threadIdx.x;
    if (e < hd) {
      float a = 0.0f;
      for (int sp = 0; sp < n_split; ++sp) a += dw1p[sp * hd + e];
      dw1[e] = a;
    }
    return;
  }
  // block nb + hid sums hidden unit hid over the token blocks; the last block does db2
  const int64_t hid = blockIdx.x - nb;
  float a = 0.0f, b = 0.0f;
  for (int64_t blk = threadIdx.x; blk < n_tb; blk += kThr) {
    if (hid < h) {
      a += dw2p[blk * h + hid];
      b += db1p[blk * h + hid];
    } else {
      a += db2p[blk];
    }
  }
  a = wave_sum(a);
  b = wave_sum(b);
  if ((threadIdx.x & 63) == 0) {
    sa[threadIdx.x >> 6] = a;
    sb[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float ta = (sa[0] + sa[1]) + (sa[2] + sa[3]);
    const float tb = (sb[0] + sb[1]) + (sb[2] + sb[3]);
    if (hid < h) {
      dw2[hid] = ta;
      db1[hid] = tb;
    } else {
      *db2 = ta;
    }
  }
}

// bf16 [R rows][C cols] (row stride ld_in) -> [C][ldo], zeros where r >= R;
// 64 x 64 tiles through LDS with 16-byte global loads and stores (C, ldo
// and ld_in multiples of 8, as the callers guarantee)
__global__ __launch_bounds__(256) void transpose_bf16(const uint16_t* __restrict__ in,
                                                      int64_t ld_in, int64_t R, int64_t C,
                                                      uint16_t* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  for (int u = threadIdx.x; u < 64 * 8; u += 256) {
    const int rr = u / 8, ch = u % 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + rr < R && c0 + 8 * ch < C) v = ld16(in + (r0 + rr) * ld_in + c0 + 8 * ch);
    st16(&tile[rr][8 * ch], v);
  }
  __syncthreads();
  for (int u = threadIdx.x; u < 64 * 8; u += 256) {
    const int cc = u / 8, ch = u % 8;                  // output row c0 + cc, rows 8ch .. +8
    if (c0 + cc < C && r0 + 8 * ch < ldo) {
      u32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[k] = (uint32_t)tile[8 * ch + 2 * k][cc] | ((uint32_t)tile[8 * ch + 2 * k + 1][cc] << 16);
      st16(out + (c0 + cc) * ldo + r0 + 8 * ch, v);
    }
  }
}

bool mfma_path(int dt, int d, int h) { return dt == 1 && h == 256 && d % 256 == 0; }

struct Layout {
  int64_t n_tb, per_split, tp;
  int n_split;
  bool mfma;
  size_t seqc, part, cpart, dbt, dz, dw2p, db1p, db2p, dw1p, inv, rowc, w1t, total;
};

Layout layout(int64_t t, int64_t t_kept, int n_seq, int d, int h, int dt, int n_cu) {
  Layout L;
  L.mfma = mfma_path(dt, d, h);
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  if (L.mfma) {
    // dz in bf16 [t][h] and transposed [h][tp] (tp = t rounded up to 64),
    // W1^T [d][h]; dW1 split over token ranges of whole 64-steps
    L.tp = (t + 63) / 64 * 64;
    L.n_tb = score_dz_blocks(t, n_cu);
    const int64_t steps = L.tp / 64 > 0 ? L.tp / 64 : 1;
    const int64_t ns = 32 < steps ? 32 : steps;
    const int64_t per_steps = (steps + ns - 1) / ns;
    L.per_split = per_steps * 64;
    L.n_split = (int)((steps + per_steps - 1) / per_steps);
  } else {
    L.tp = t;
    L.n_tb = (t + kT - 1) / kT;
    const int64_t tiles = (int64_t)(h / kT) * (d / kT);
    int ns = (int)((1024 + tiles - 1) / tiles);
    if (ns > kSplitMax) ns = kSplitMax;
    if (ns < 1) ns = 1;
    int64_t per = (t + ns - 1) / ns;
    per = ((per + kKC - 1) / kKC) * kKC;
    if (per < kKC) per = kKC;
    L.per_split = per;
    L.n_split = ns;
  }
  size_t off = 0;
  L.seqc = off; off += al(sizeof(double2) * (size_t)n_seq);
  L.part = off; off += al(sizeof(SqPart) * (size_t)(n_seq + (t + kCh - 1) / kCh));
  L.cpart = off; off += al(sizeof(double) * (size_t)(n_seq + (t_kept + kCh - 1) / kCh));
  L.dbt = off; off += al(sizeof(float) * (size_t)t);
  L.dz = off; off += al((L.mfma ? sizeof(uint16_t) : sizeof(float)) * (size_t)t * h);
  L.dw2p = off; off += al(sizeof(float) * (size_t)L.n_tb * h);
  L.db1p = off; off += al(sizeof(float) * (size_t)L.n_tb * h);
  L.db2p = off; off += al(sizeof(float) * (size_t)L.n_tb);
  L.dw1p = off; off += al(sizeof(float) * (size_t)L.n_split * h * d);
  // LN2: each row's 1 / RMS (vector path) and c (matrix-core path: [t];
  // vector path: partials per 64 hidden units, [h / 64][t])
  L.inv = off; off += al(sizeof(float) * (size_t)t);
  L.rowc = off; off += al(sizeof(float) * (size_t)t * (L.mfma ? 1 : h / kT));
  L.w1t = off;
  if (L.mfma) {
    L.w1t = off; off += al(sizeof(uint16_t) * (size_t)d * h);
  }
  L.total = off;
  return L;
}

template <typename T>
hipError_t launch_t(const void* xv, int64_t xs, int64_t t, int d, int h, const void* w1v,
                    const float* b1, const float* w2, const uint8_t* pr, const int32_t* cu,
                    int n_seq, float eps, float norm_eps, const float* b_raw,
                    const int32_t* kept_idx,
                    const int32_t* kept_cu, int64_t t_kept, const float* db_kept, float* dx,
                    float* dw1, float* db1, float* dw2, float* db2, void* ws, hipStream_t st) {
  int n_cu = 0;
  const hipError_t ce = device_cu_count(&n_cu);
  if (ce != hipSuccess) return ce;
  const Layout L = layout(t, t_kept, n_seq, d, h, std::is_same<T, uint16_t>::value ? 1 : 0, n_cu);
  char* w = static_cast<char*>(ws);
  double2* seqc = reinterpret_cast<double2*>(w + L.seqc);
  float* dbt = reinterpret_cast<float*>(w + L.dbt);
  float* dz = reinterpret_cast<float*>(w + L.dz);
  float* dw2p = reinterpret_cast<float*>(w + L.dw2p);
  float* db1p = reinterpret_cast<float*>(w + L.db1p);
  float* db2p = reinterpret_cast<float*>(w + L.db2p);
  float* dw1p = reinterpret_cast<float*>(w + L.dw1p);
  const T* x = static_cast<const T*>(xv);
  const T* w1 = static_cast<const T*>(w1v);
  SqPart* part = reinterpret_cast<SqPart*>(w + L.part);
  double* cpart = reinterpret_cast<double*>(w + L.cpart);
  const bool ln2 = norm_eps >= 0.0f;
  float* inv = ln2 ? reinterpret_cast<float*>(w + L.inv) : nullptr;
  float* rowc = ln2 ? reinterpret_cast<float*>(w + L.rowc) : nullptr;
  hipLaunchKernelGGL(sbwd_part, dim3((unsigned)(n_seq + (t + kCh - 1) / kCh)), dim3(kThr), 0, st,
                     b_raw, pr, cu, n_seq, t, part);
  hipLaunchKernelGGL(sbwd_cpart, dim3((unsigned)(n_seq + (t_kept + kCh - 1) / kCh)), dim3(kThr), 0,
                     st, b_raw, pr, kept_idx, kept_cu, n_seq, t, t_kept, db_kept, cpart);
  hipLaunchKernelGGL(sbwd_seq, dim3(n_seq), dim3(64), 0, st, cu, kept_cu, part, cpart, eps, seqc);
  if (t > 0)
    hipLaunchKernelGGL(sbwd_dbt, dim3((unsigned)((t + kThr - 1) / kThr)), dim3(kThr), 0, st, b_raw,
                       pr, cu, n_seq, t, seqc, dbt);
  if (t_kept > 0)
    hipLaunchKernelGGL(sbwd_kept, dim3((unsigned)((t_kept + kThr - 1) / kThr)), dim3(kThr), 0, st,
                       b_raw, pr, kept_idx, kept_cu, n_seq, t, t_kept, db_kept, seqc, dbt);
  if (L.mfma && t > 0) {
    if constexpr (std::is_same<T, uint16_t>::value) {
      uint16_t* dzb = reinterpret_cast<uint16_t*>(w + L.dz);
      uint16_t* w1t = reinterpret_cast<uint16_t*>(w + L.w1t);
      int64_t nb = 0;
      hipError_t e = launch_score_dz(x, xs, t, d, w1, b1, w2, dbt, dzb, dw2p, db1p, db2p,
                                     norm_eps, rowc, &nb, st);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)(d / 64), (unsigned)((h + 63) / 64)),
                         dim3(256), 0, st, w1, (int64_t)d, (int64_t)h, (int64_t)d, w1t, (int64_t)h);
      // dW1[h][c] = sum_j dz[j][h] x[j][c]  (dz and x both read as stored,
      // token-major; token splits, fp32 partials; tokens past t read as zeros)
      e = launch_gemm_atb_kmajor_f32(dzb, h, h, x, xs, t, d, L.tp, L.n_split, dw1p, d, st);
      if (e != hipSuccess) return e;
      // dx[j][c] = sum_h dz[j][h] W1^T[c][h]  (LN2: - c_j x[j][c])
      if (dx) {
        e = launch_gemm_abt_f32(dzb, h, t, w1t, h, d, h, 1, dx, d, st, rowc, x, xs);
        if (e != hipSuccess) return e;
      }
    }
  } else if (t > 0) {
    if (ln2)
      hipLaunchKernelGGL((sbwd_rowinv<T>), dim3((unsigned)((t + kThr / 64 - 1) / (kThr / 64))),
                         dim3(kThr), 0, st, x, xs, t, d, norm_eps, inv);
    hipLaunchKernelGGL((sbwd_dz<T>), dim3((unsigned)L.n_tb, h / kT), dim3(kThr), 0, st, x, xs, t,
                       d, h, w1, b1, w2, dbt, dz, dw2p, db1p, db2p, inv, rowc);
    hipLaunchKernelGGL((sbwd_dw1<T>), dim3(h / kT, d / kT, L.n_split), dim3(kThr), 0, st, x, xs, t,
                       d, h, dz, L.per_split, dw1p);
    if (dx)
      hipLaunchKernelGGL((sbwd_dx<T>), dim3((unsigned)L.n_tb, d / kT), dim3(kThr), 0, st, t, d, h,
                         w1, dz, dx, x, xs, inv, rowc, h / kT);
  }
  const int64_t hd = (int64_t)h * d;
  hipLaunchKernelGGL(sbwd_finish, dim3((unsigned)((hd + kThr - 1) / kThr + h + 1)), dim3(kThr), 0, st,
                     hd, h, t > 0 ? L.n_split : 0, L.n_tb, dw1p, dw2p, db1p, db2p, dw1, dw2, db1,
                     db2);
  return hipGetLastError();
}

}  // namespace

size_t score_bwd_ws_bytes(int64_t t, int n_seq, int d, int h) {
  // enough for either arithmetic path (the dtype is not an argument here)
  int n_cu = 0;
  if (device_cu_count(&n_cu) != hipSuccess || n_cu < 1) n_cu = 1;
  // kept rows never exceed t (checked by the entry point)
  const size_t a = layout(t, t, n_seq, d, h, 0, n_cu).total;
  const size_t b = layout(t, t, n_seq, d, h, 1, n_cu).total;
  return a > b ? a : b;
}

hipError_t launch_score_bwd(const void* x, int dt, int64_t xs, int64_t t, int d, int h,
                            const void* w1, const float* b1, const float* w2, const uint8_t* pr,
                            const int32_t* cu, int n_seq, float eps, float norm_eps,
                            const float* b_raw, const int32_t* kept_idx, const int32_t* kept_cu,
                            int64_t t_kept, const float* db_kept, float* dx, float* dw1,
                            float* db1, float* dw2, float* db2, void* ws, hipStream_t st) {
  if (dt == 1)
    return launch_t<uint16_t>(x, xs, t, d, h, w1, b1, w2, pr, cu, n_seq, eps, norm_eps, b_raw,
                              kept_idx, kept_cu, t_kept, db_kept, dx, dw1, db1, dw2, db2, ws, st);
  return launch_t<float>(x, xs, t, d, h, w1, b1, w2, pr, cu, n_seq, eps, norm_eps, b_raw, kept_idx,
                         kept_cu, t_kept, db_kept, dx, dw1, db1, dw2, db2, ws, st);
}

}  // namespace tg
