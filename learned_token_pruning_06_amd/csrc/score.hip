// tg_score: the gate's scoring network and its normalisation
// (TokenGate §4.1 Eq. 3):
//   b~_j = w2 . SiLU(W1 x_j + b1) + b2
//   b_j  = b~_j / sqrt(mean_{P_s} b~^2 + eps) on prunable tokens, 0 on prompt tokens.
//
// bf16 path: a skinny GEMM C^T[h, row] = W1[h, d] . x[row, d]^T on MFMA
// (v_mfma_f32_32x32x16_bf16), with the SiLU / w2 epilogue fused so only one
// float per row leaves the kernel.  Each workgroup owns 256 rows and all h
// columns (so the epilogue reduction over h stays in the workgroup); every
// 64-wide K-step of x and W1 goes global -> registers (one step ahead) ->
// padded, double-buffered LDS shared by the 8 waves.  The transposed
// orientation puts one row per lane, so the reduction over h is in-lane plus
// one cross-half exchange.  Bound: HBM (2*d bytes per row) near the MFMA
// ridge.
//
// Optional LN2 (§3 Eq. 1: the scorer reads a~ = LN2(a), an RMSNorm): with
// the norm weight folded into W1 by the caller, W1 (g * a / r) = (W1 g) a / r,
// so the kernel multiplies the raw rows a and divides each row's
// accumulators by r = sqrt(mean(a^2) + eps) in the epilogue.  The sums of
// squares are taken from the x registers as they are staged, so the norm
// costs no extra pass over the rows.
//
// Normalisation: the scoring kernel's epilogue writes, for every sequence
// that meets its rows, an fp64 partial sum of the squared raw scores of the
// sequence's prunable rows (and their count).  Rows of a workgroup and of a
// sequence are contiguous ranges, so (sequence s, workgroup g) pairs that
// meet are told apart by s + g: that is the partial's slot.  A second kernel,
// one block per 2048-token chunk, adds the partials of its sequence in a
// fixed order and divides.  No float atomics, so the result is bitwise
// reproducible.
#include "common.h"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;              // d per K-step
constexpr int kRow = kBK + 8;        // bf16 per LDS row (144 B: rows start 4 banks apart)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

TG_DEVINL bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// acc += lo^2 + hi^2 of a bf16 pair.  Written as one v_dot2_f32_bf16 with the
// same register for both sources: the builtin, given one value twice, was
// compiled to four dot products of the first word of a 16-byte vector.
TG_DEVINL void sq_acc(float& acc, uint32_t w) {
  asm("v_dot2_f32_bf16 %0, %1, %1, %0" : "+v"(acc) : "v"(w));
}

TG_DEVINL float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// One workgroup = 256 rows x all h columns, 8 waves: wave w owns rows
// [64(w%4), +64) and the h tiles [MTA(w/4), +MTA) (two waves per SIMD, 128
// accumulators each).  Each 64-wide K-step of x and W1 is read with
// coalesced 16-byte buffer loads (8 rows x 128 B per wave instruction) one
// step ahead into registers, then staged into double-buffered, padded LDS
// tiles shared by all waves; one barrier per K-step.  Rows past the end of x
// (and hidden units past h) read zeros through the buffer ranges.
struct DzOut {                  // outputs of the backward epilogue (BWD)
  const float* dbt;             // [t_in] gradient at the raw scores
  uint16_t* dz;                 // [t_in][H] bf16
  float* dw2p;                  // [blocks][H] per-workgroup sums of dbt * SiLU(z)
  float* db1p;                  // [blocks][H] per-workgroup sums of dz
  float* db2p;                  // [blocks]    per-workgroup sums of dbt
  float* rowc;                  // [t_in] (LN2 only) each row's c = inv^3 / d * sum_h dz_h acc_h
};

// Backward epilogue shared by the scorer kernels: z = acc + b1,
// dz = dbt w2 SiLU'(z) (bf16, [t_in][H]) and the workgroup's sums over its
// rows of dbt SiLU(z) and dz for each hidden unit: in-lane over the two row
// tiles, a reduce-scatter over the 32 row lanes (lane n ends with value pair
// 2n, 2n + 1), then the RG row groups in order through LDS (red: [2][RG][H]
// floats).  Every thread of the workgroup calls it.
// NORM (LN2 in front of the scorer, acc = W1' a of the raw row a, inv the
// row's 1 / RMS): z = acc inv + b1, and the stored dz is the gradient at the
// unnormalised product, dz inv, which is what dW1' = dz^T a and the first
// part of da = (dz inv) W1' - c a take; the row's c = inv^3 / d * sum_h
// dz_h acc_h (the norm's own derivative) is summed per lane, over the lane
// halves, then over the HS waves of the row group through srow ([HS][RG][64]
// floats) and written to bo.rowc.
template <int H, int MTA, int RG, bool NORM = false, int HS = 1>
TG_DEVINL void dz_epilogue(floatx16 (&acc)[MTA][2], int nmt, int mt0, int rg, int64_t row0,
                           int64_t wg_row0, int64_t t_in, const float* __restrict__ b1,
                           const float* __restrict__ w2, const DzOut& bo, float* red, int tid,
                           int nthreads, float inv0 = 1.0f, float inv1 = 1.0f, int hh = 0,
                           float* srow = nullptr, const float* sinv = nullptr, int d = 1) {
  const int lane = tid & 63, n = lane & 31, g = lane >> 5;
  const int64_t ra = row0 + n, rb = row0 + 32 + n;
  const float ga = ra < t_in ? bo.dbt[ra] : 0.0f, gb = rb < t_in ? bo.dbt[rb] : 0.0f;
  float ca = 0.0f, cb = 0.0f;                       // NORM: sum_h dz_h acc_h of rows ra, rb
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt) {
    if (mt >= nmt) continue;
    float vw[16], vb[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int h0 = 32 * (mt0 + mt) + 8 * r4 + 4 * g;
      uint32_t pa[2] = {0u, 0u}, pb[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * r4 + e;
        const float bb = b1 ? b1[h0 + e] : 0.0f, ww = w2[h0 + e];
        const float za = NORM ? fmaf(acc[mt][0][r], inv0, bb) : acc[mt][0][r] + bb;
        const float zb = NORM ? fmaf(acc[mt][1][r], inv1, bb) : acc[mt][1][r] + bb;
        const float sa = 1.0f / (1.0f + __expf(-za)), sb2 = 1.0f / (1.0f + __expf(-zb));
        const float da = ga * ww * sa * fmaf(za, 1.0f - sa, 1.0f);
        const float db = gb * ww * sb2 * fmaf(zb, 1.0f - sb2, 1.0f);
        vw[r] = fmaf(ga, za * sa, gb * zb * sb2);
        vb[r] = da + db;
        if constexpr (NORM) {
          ca = fmaf(da, acc[mt][0][r], ca);
          cb = fmaf(db, acc[mt][1][r], cb);
        }
        const uint16_t ua = __builtin_bit_cast(uint16_t, (__bf16)(NORM ? da * inv0 : da));
        const uint16_t ub = __builtin_bit_cast(uint16_t, (__bf16)(NORM ? db * inv1 : db));
        pa[e >> 1] |= (uint32_t)ua << (16 * (e & 1));
        pb[e >> 1] |= (uint32_t)ub << (16 * (e & 1));
      }
      if (ra < t_in) *reinterpret_cast<uint2*>(bo.dz + ra * H + h0) = make_uint2(pa[0], pa[1]);
      if (rb < t_in) *reinterpret_cast<uint2*>(bo.dz + rb * H + h0) = make_uint2(pb[0], pb[1]);
    }
    // sum over the 32 row lanes: reduce-scatter over lane bits 4..1 (lane n
    // ends with register n / 2), then add the bit-0 partner
#pragma unroll
    for (int o = 16, c = 16; o >= 2; o >>= 1, c >>= 1) {
      const bool up = (lane & o) != 0;
#pragma unroll
      for (int kk = 0; kk < c / 2; ++kk) {
        const float kw = up ? vw[kk + c / 2] : vw[kk], xw = up ? vw[kk] : vw[kk + c / 2];
        const float kb = up ? vb[kk + c / 2] : vb[kk], xb = up ? vb[kk] : vb[kk + c / 2];
        vw[kk] = kw + __shfl_xor(xw, o, 64);
        vb[kk] = kb + __shfl_xor(xb, o, 64);
      }
    }
    const float tw = vw[0] + __shfl_xor(vw[0], 1, 64);
    const float tb = vb[0] + __shfl_xor(vb[0], 1, 64);
    if ((n & 1) == 0) {
      const int r = n >> 1;
      const int hid = 32 * (mt0 + mt) + 8 * (r / 4) + 4 * g + (r % 4);
      red[(0 * RG + rg) * H + hid] = tw;
      red[(1 * RG + rg) * H + hid] = tb;
    }
  }
  if constexpr (NORM) {
    ca += __shfl_xor(ca, 32, 64);
    cb += __shfl_xor(cb, 32, 64);
    if (g == 0) {
      srow[(hh * RG + rg) * 64 + n] = ca;
      srow[(hh * RG + rg) * 64 + 32 + n] = cb;
    }
  }
  __syncthreads();
  if constexpr (NORM) {
    if (tid < 64 * RG && wg_row0 + tid < t_in) {
      float c = 0.0f;
#pragma unroll
      for (int k = 0; k < HS; ++k) c += srow[(k * RG + tid / 64) * 64 + tid % 64];
      const float iv = sinv[tid];
      bo.rowc[wg_row0 + tid] = c * (iv * iv * iv) / (float)d;
    }
  }
  for (int hid = tid; hid < H; hid += nthreads) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      a += red[(0 * RG + k) * H + hid];
      b += red[(1 * RG + k) * H + hid];
    }
    bo.dw2p[(int64_t)blockIdx.x * H + hid] = a;
    bo.db1p[(int64_t)blockIdx.x * H + hid] = b;
  }
  if (tid == nthreads - 1) {
    float a = 0.0f;
    for (int r = 0; r < 64 * RG; ++r) a += wg_row0 + r < t_in ? bo.dbt[wg_row0 + r] : 0.0f;
    bo.db2p[blockIdx.x] = a;
  }
}

struct Partial {
  double sumsq;
  int64_t count;
};

constexpr int kPartRows = 64;        // rows per workgroup of every scoring kernel: at least 64

// Largest s in [0, n_seq) with cu[s] <= row (0 if none): the first sequence
// that can meet rows from `row` on.
TG_DEVINL int seq_at_row(const int32_t* cu, int n_seq, int64_t row) {
  int lo = 0, hi = n_seq - 1, ans = 0;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid] <= row) {
      ans = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  return ans;
}

// Per-sequence partial sums of the workgroup's rows [r0, r0 + rows) (rows
// past t_in excluded): sq[i] is row r0 + i's squared raw score if it is
// prunable, else 0, and pf[i] its prunable flag.  Wave w takes sequences
// s_a + w, s_a + w + NW, ...; each sum runs over the rows in index order per
// lane and then a fixed butterfly, so the result is reproducible.  Every
// thread calls it after sq and pf are written (and a barrier).
template <int NW>
TG_DEVINL void seq_partials(const double* sq, const int* pf, int64_t r0, int rows, int64_t t_in,
                            const int32_t* cu, int n_seq, int s_a, Partial* part) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r1 = r0 + rows < t_in ? r0 + rows : t_in;
  for (int s = s_a + wv; s < n_seq; s += NW) {
    int64_t lo = cu[s], hi = cu[s + 1];
    lo = lo < 0 ? 0 : (lo > t_in ? t_in : lo);
    hi = hi < lo ? lo : (hi > t_in ? t_in : hi);
    if (lo >= r1) break;
    const int64_t a = lo > r0 ? lo : r0, e = hi < r1 ? hi : r1;
    if (a >= e) continue;
    double acc = 0.0;
    int cnt = 0;
    for (int64_t r = a + lane; r < e; r += 64) {
      acc += sq[r - r0];
      cnt += pf[r - r0];
    }
    acc = wave_sum(acc);
    cnt = wave_sum(cnt);
    if (lane == 0) {
      part[(int64_t)s + blockIdx.x].sumsq = acc;
      part[(int64_t)s + blockIdx.x].count = cnt;
    }
  }
}

template <int MT, bool NORM, int RG, bool BWD = false>
__global__ __launch_bounds__(kThreads) void score_mlp_bf16(
    const uint16_t* __restrict__ x, int64_t xs, int64_t t_in, int d,
    const uint16_t* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    float b2, float norm_eps, float* __restrict__ b_raw, const uint8_t* __restrict__ pr,
    const int32_t* __restrict__ cu, int n_seq, Partial* __restrict__ part, DzOut bo = DzOut{}) {
  constexpr int H = 32 * MT;
  constexpr int ROWS = 64 * RG;              // rows per workgroup (RG groups of 64)
  constexpr int HS = kWaves / RG;            // waves sharing a row group, splitting h
  constexpr int MTA = (MT + HS - 1) / HS;    // h tiles per wave (the last may have fewer)
  constexpr int XV = RG;                     // x vectors per thread per K-step
  constexpr int WV = (H + 63) / 64;          // W1 vectors per thread per K-step
  // pinned operand prefetch: every wave holds MTA full h tiles (no ragged
  // last wave) and the registers allow it (not with the backward epilogue).
  // Not with LN2 either: the pinned order keeps its square-sums out of the
  // MFMA shadow (+3-5% measured, against -5.5% for the plain form at 128k).
  constexpr bool PIPE = !BWD && !NORM && MT % HS == 0 && MTA >= 2;
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][H * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t sx[2][ROWS * kRow];
  __shared__ float sred[HS][RG][64];
  __shared__ float sinv[NORM ? ROWS : 1];    // 1 / RMS of each row (LN2)
  __shared__ double ssq[BWD ? 1 : ROWS];     // squared raw scores of prunable rows
  __shared__ int spf[BWD ? 1 : ROWS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int rg = wv % RG, hh = wv / RG;
  const int mt0 = hh * MTA;
  // h tiles of this wave (may be <= 0 when HS does not divide MT)
  const int nmt = MT % HS == 0 ? MTA : (MT - mt0 < MTA ? MT - mt0 : MTA);
  const int64_t wg_row0 = (int64_t)blockIdx.x * ROWS;
  const int64_t row0 = wg_row0 + rg * 64;
  // for the normalisation partials: the first sequence that can meet this
  // workgroup's rows, and the prunable flags of the rows this lane will hold
  int s_a = 0;
  uint8_t pfa = 0, pfb = 0;
  if constexpr (!BWD) {
    s_a = seq_at_row(cu, n_seq, wg_row0);
    if (row0 + n < t_in) pfa = pr[row0 + n];
    if (row0 + 32 + n < t_in) pfb = pr[row0 + 32 + n];
  }

  // loaders: thread vector i covers row (tid / 8) + 64 i, 16-byte chunk tid % 8
  const int lrow = tid >> 3, lch = tid & 7;
  const int64_t xbytes = (t_in - wg_row0) * xs * 2;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + wg_row0 * xs), (short)0,
      (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w1), (short)0, (int)((int64_t)H * d * 2), 0x00020000);
  int xoff[XV], woff[WV];
#pragma unroll
  for (int i = 0; i < XV; ++i) xoff[i] = (int)(((int64_t)(lrow + 64 * i) * xs + 8 * lch) * 2);
#pragma unroll
  for (int i = 0; i < WV; ++i) woff[i] = ((lrow + 64 * i) * d + 8 * lch) * 2;
  const int ldst = lrow * kRow + 8 * lch;
  u32x4 xr[XV], wr[WV];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XV; ++i)
      xr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i] + 2 * k0, 0, 0));
#pragma unroll
    for (int i = 0; i < WV; ++i)
      wr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i] + 2 * k0, 0, 0));
  };
  float ss[XV];                                   // sums of squares of rows lrow + 64 i
#pragma unroll
  for (int i = 0; i < XV; ++i) ss[i] = 0.f;
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XV; ++i) st16(&sx[buf][ldst + 64 * i * kRow], xr[i]);
    if constexpr (NORM) {
#pragma unroll
      for (int i = 0; i < XV; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) sq_acc(ss[i], xr[i][w]);
    }
#pragma unroll
    for (int i = 0; i < WV; ++i)
      if (lrow + 64 * i < H) st16(&sw[buf][ldst + 64 * i * kRow], wr[i]);
  };

  floatx16 acc[MTA][2];
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[mt][0][r] = 0.f;
      acc[mt][1][r] = 0.f;
    }

  const int nk = d / kBK;
  fetch(0);
  stage(0);
  if (nk > 1) fetch(kBK);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    const uint16_t* xb = sx[buf] + (64 * rg + n) * kRow + 32 * g;
    const uint16_t* wb = sw[buf] + (32 * mt0 + n) * kRow + 32 * g;
    if constexpr (PIPE) {
      // operands of 16-wide substep s + 1 are read from LDS while the MFMAs
      // of substep s run (one read after each MFMA, order pinned)
      bf16x8 bo[2][2], ao[2][MTA];
      auto ld_op = [&](int s, int c, int i) {
        if (i < 2) bo[c][i] = as_bf16x8(ld16(xb + 32 * i * kRow + 8 * s));
        else ao[c][i - 2] = as_bf16x8(ld16(wb + 32 * (i - 2) * kRow + 8 * s));
      };
#pragma unroll
      for (int i = 0; i < 2 + MTA; ++i) ld_op(0, 0, i);
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        const int c = s & 1;
#pragma unroll
        for (int j = 0; j < 2 * MTA; ++j) {
          acc[j >> 1][j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              ao[c][j >> 1], bo[c][j & 1], acc[j >> 1][j & 1], 0, 0, 0);
          if (s + 1 < kBK / 16 && j < 2 + MTA) ld_op(s + 1, c ^ 1, j);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const bf16x8 bop0 = as_bf16x8(ld16(xb + 8 * s));
      const bf16x8 bop1 = as_bf16x8(ld16(xb + 32 * kRow + 8 * s));
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) {
        if (mt < nmt) {
          const bf16x8 aop = as_bf16x8(ld16(wb + 32 * mt * kRow + 8 * s));
          acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop0, acc[mt][0], 0, 0, 0);
          acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop1, acc[mt][1], 0, 0, 0);
        }
      }
    }
    }
    if (it + 1 < nk) {
      stage(buf ^ 1);
      if (it + 2 < nk) fetch((it + 2) * kBK);
    }
    __syncthreads();
  }

  // LN2: the 8 threads of a loader row hold its partial sums of squares
  float inv0 = 1.0f, inv1 = 1.0f;
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      float v = ss[i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      if (lch == 0) sinv[lrow + 64 * i] = 1.0f / sqrtf(v / (float)d + norm_eps);
    }
    __syncthreads();
    inv0 = sinv[64 * rg + n];
    inv1 = sinv[64 * rg + 32 + n];
  }

  if constexpr (BWD) {
    float* red = reinterpret_cast<float*>(&sx[0][0]);          // [2][RG][H], K-loop buffers are free
    dz_epilogue<H, MTA, RG, NORM, HS>(acc, nmt, mt0, rg, row0, wg_row0, t_in, b1, w2, bo, red,
                                      tid, kThreads, inv0, inv1, hh, &sred[0][0][0], sinv, d);
    return;
  }

  // epilogue: lane (n, g) holds h = 32(mt0+mt) + 8(r/4) + 4g + (r%4) of rows 32nt + n;
  // the two h halves of a row group are added through LDS
  float part0 = 0.f, part1 = 0.f;
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int h0 = 32 * (mt0 + mt) + 8 * r4 + 4 * g;
        const float4 bb = b1 ? *reinterpret_cast<const float4*>(b1 + h0) : make_float4(0, 0, 0, 0);
        const float4 ww = *reinterpret_cast<const float4*>(w2 + h0);
        part0 = fmaf(silu_f(fmaf(acc[mt][0][4 * r4 + 0], inv0, bb.x)), ww.x, part0);
        part0 = fmaf(silu_f(fmaf(acc[mt][0][4 * r4 + 1], inv0, bb.y)), ww.y, part0);
        part0 = fmaf(silu_f(fmaf(acc[mt][0][4 * r4 + 2], inv0, bb.z)), ww.z, part0);
        part0 = fmaf(silu_f(fmaf(acc[mt][0][4 * r4 + 3], inv0, bb.w)), ww.w, part0);
        part1 = fmaf(silu_f(fmaf(acc[mt][1][4 * r4 + 0], inv1, bb.x)), ww.x, part1);
        part1 = fmaf(silu_f(fmaf(acc[mt][1][4 * r4 + 1], inv1, bb.y)), ww.y, part1);
        part1 = fmaf(silu_f(fmaf(acc[mt][1][4 * r4 + 2], inv1, bb.z)), ww.z, part1);
        part1 = fmaf(silu_f(fmaf(acc[mt][1][4 * r4 + 3], inv1, bb.w)), ww.w, part1);
      }
    }
  }
  const float tot0 = part0 + __shfl_xor(part0, 32, 64);
  const float tot1 = part1 + __shfl_xor(part1, 32, 64);
  if (hh > 0 && g == 0) {
    sred[hh][rg][n] = tot0;
    sred[hh][rg][32 + n] = tot1;
  }
  __syncthreads();
  if (hh == 0 && g == 0) {
    float a0 = tot0, a1 = tot1;
#pragma unroll
    for (int k = 1; k < HS; ++k) {
      a0 += sred[k][rg][n];
      a1 += sred[k][rg][32 + n];
    }
    const float v0 = a0 + b2, v1 = a1 + b2;
    const bool in0 = row0 + n < t_in, in1 = row0 + 32 + n < t_in;
    if (in0) b_raw[row0 + n] = v0;
    if (in1) b_raw[row0 + 32 + n] = v1;
    const bool p0 = in0 && pfa, p1 = in1 && pfb;
    ssq[64 * rg + n] = p0 ? (double)v0 * (double)v0 : 0.0;
    ssq[64 * rg + 32 + n] = p1 ? (double)v1 * (double)v1 : 0.0;
    spf[64 * rg + n] = p0;
    spf[64 * rg + 32 + n] = p1;
  }
  __syncthreads();
  seq_partials<kWaves>(ssq, spf, wg_row0, ROWS, t_in, cu, n_seq, s_a, part);
}

// fp32 scorer on the vector ALU: 64 rows per block, one wave per row at a
// time (wave w takes rows w, w + 4, ...), lanes over hidden units (with LN2,
// the row's RMS first: lanes over the row, then a wave sum); then the
// normalisation partials of the block's rows.
__global__ __launch_bounds__(256) void score_mlp_f32(const float* __restrict__ x, int64_t xs,
                                                     int64_t t_in, int d, int h,
                                                     const float* __restrict__ w1,
                                                     const float* __restrict__ b1,
                                                     const float* __restrict__ w2, float b2,
                                                     float norm_eps, float* __restrict__ b_raw,
                                                     const uint8_t* __restrict__ pr,
                                                     const int32_t* __restrict__ cu, int n_seq,
                                                     Partial* __restrict__ part) {
  __shared__ double ssq[kPartRows];
  __shared__ int spf[kPartRows];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * kPartRows;
  for (int i = wv; i < kPartRows; i += 4) {
    const int64_t row = r0 + i;
    double sq = 0.0;
    int pf = 0;
    if (row < t_in) {
      const float* xp = x + row * xs;
      float inv = 1.0f;
      if (norm_eps >= 0.0f) {
        float ss = 0.f;
        for (int e = lane; e < d; e += 64) ss = fmaf(xp[e], xp[e], ss);
        ss = wave_sum(ss);
        inv = 1.0f / sqrtf(ss / (float)d + norm_eps);
      }
      float acc_h = 0.f;
      for (int j = lane; j < h; j += 64) {
        const float* wp = w1 + (int64_t)j * d;
        float acc = 0.f;
        for (int e = 0; e < d; ++e) acc = fmaf(xp[e], wp[e], acc);
        const float v = fmaf(acc, inv, b1 ? b1[j] : 0.f);
        acc_h = fmaf(v / (1.0f + expf(-v)), w2[j], acc_h);
      }
      const float val = wave_sum(acc_h) + b2;
      if (lane == 0) b_raw[row] = val;
      pf = pr[row] != 0;
      sq = pf ? (double)val * (double)val : 0.0;
    }
    if (lane == 0) {
      ssq[i] = sq;
      spf[i] = pf;
    }
  }
  __syncthreads();
  seq_partials<4>(ssq, spf, r0, kPartRows, t_in, cu, n_seq, seq_at_row(cu, n_seq, r0), part);
}

constexpr int CH = kScoreChunk;

TG_DEVINL bool locate(const int32_t* cu, int n_seq, int64_t t_in, int64_t slot, int& s,
                      int64_t& begin, int64_t& end, int& nch) {
  s = seq_of_slot(cu, n_seq, slot, CH);
  if (s < 0) return false;
  // token ranges are clamped to [0, t_in): inconsistent offsets cannot read out of bounds
  const int64_t lo = cu[s] < t_in ? cu[s] : t_in;
  const int64_t hi = cu[s + 1] < t_in ? cu[s + 1] : t_in;
  if (hi <= lo) return false;
  begin = lo + (slot - slot0_of(cu, s, CH)) * CH;
  if (begin >= hi) return false;
  end = begin + CH < hi ? begin + CH : hi;
  nch = (int)((hi - lo + CH - 1) / CH);
  return true;
}

// b = b~ / r on the prunable tokens of one 2048-token chunk, 0 on the others,
// with r = sqrt(sum / count + eps) from the sequence's partials (slots s + g
// for the scoring workgroups g that meet it, `rows` rows each), added in a
// fixed order by every chunk of the sequence.
__global__ __launch_bounds__(256) void score_norm(const float* __restrict__ b_raw,
                                                  const uint8_t* __restrict__ pr,
                                                  const int32_t* __restrict__ cu, int n_seq,
                                                  int64_t t_in, const Partial* __restrict__ part,
                                                  int rows, float eps, float* __restrict__ b) {
  __shared__ double sd[4];
  __shared__ int64_t sc[4];
  int s, nch;
  int64_t begin, end;
  if (!locate(cu, n_seq, t_in, blockIdx.x, s, begin, end, nch)) return;
  constexpr int PER = CH / 256;
  uint8_t pv[PER];
  float bv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = begin + threadIdx.x + (int64_t)i * 256;
    pv[i] = j < end ? pr[j] : (uint8_t)0;
    bv[i] = j < end ? b_raw[j] : 0.0f;
  }
  const int64_t lo = cu[s] < t_in ? cu[s] : t_in;
  const int64_t hi = cu[s + 1] < t_in ? cu[s + 1] : t_in;
  const int64_t g0 = lo / rows, ng = (hi - 1) / rows - g0 + 1;
  const Partial* ps = part + s + g0;
  // thread t adds partials t, t + 256, ... in order, eight loads in flight
  double acc = 0.0;
  int64_t cnt = 0;
  for (int64_t base = threadIdx.x; base < ng; base += 8 * 256) {
    Partial v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = base + 256 * k < ng ? ps[base + 256 * k] : Partial{0.0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc += v[k].sumsq;
      cnt += v[k].count;
    }
  }
  acc = wave_sum(acc);
  cnt = wave_sum(cnt);
  if ((threadIdx.x & 63) == 0) {
    sd[threadIdx.x >> 6] = acc;
    sc[threadIdx.x >> 6] = cnt;
  }
  __syncthreads();
  const double tot = ((sd[0] + sd[1]) + sd[2]) + sd[3];
  const int64_t n = sc[0] + sc[1] + sc[2] + sc[3];
  const float r = n > 0 ? (float)sqrt(tot / (double)n + (double)eps) : 1.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = begin + threadIdx.x + (int64_t)i * 256;
    if (j < end) b[j] = pv[i] ? bv[i] / r : 0.0f;
  }
}

int64_t n_slots(int64_t t_in, int n_seq) { return (int64_t)n_seq + (t_in + CH - 1) / CH; }

}  // namespace

// Backward helper: z recomputed with the forward tiling (MT = 8; with LN2
// when norm_eps >= 0, then also each row's c in rowc), with the backward
// epilogue.  Returns the number of workgroups (the partial-sum rows)
// through *blocks.
hipError_t launch_score_dz(const void* x, int64_t xs, int64_t t_in, int d, const void* w1,
                           const float* b1, const float* w2, const float* dbt, void* dz,
                           float* dw2p, float* db1p, float* db2p, float norm_eps, float* rowc,
                           int64_t* blocks, hipStream_t st) {
  int n_cu = 0;
  const hipError_t ce = device_cu_count(&n_cu);
  if (ce != hipSuccess) return ce;
  // at most 128 rows per workgroup: the backward epilogue does not fit the
  // 256-row tile's registers (44 spills there; 900 against 920 us for the
  // whole scorer backward at 131072 rows)
  const int rg = (t_in + 127) / 128 >= n_cu ? 2 : 1;
  const int64_t nb = (t_in + 64 * rg - 1) / (64 * rg);
  *blocks = nb;
  if (t_in == 0) return hipSuccess;
  DzOut bo{dbt, static_cast<uint16_t*>(dz), dw2p, db1p, db2p, rowc};
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* wp = static_cast<const uint16_t*>(w1);
#define TG_DZ(N, R)                                                                            \
  hipLaunchKernelGGL((score_mlp_bf16<8, N, R, true>), dim3((unsigned)nb), dim3(kThreads), 0,  \
                     st, xp, xs, t_in, d, wp, b1, w2, 0.0f, norm_eps, nullptr, nullptr,       \
                     nullptr, 0, nullptr, bo)
  if (norm_eps >= 0.0f) {
    if (rg == 2) TG_DZ(true, 2);
    else TG_DZ(true, 1);
  } else {
    if (rg == 2) TG_DZ(false, 2);
    else TG_DZ(false, 1);
  }
#undef TG_DZ
  return hipGetLastError();
}

int64_t score_dz_blocks(int64_t t_in, int n_cu) {
  const int rg = (t_in + 127) / 128 >= n_cu ? 2 : 1;
  return (t_in + 64 * rg - 1) / (64 * rg);
}

// partial slots: n_seq + (scoring workgroups), every workgroup >= kPartRows rows
int64_t n_parts(int64_t t_in, int n_seq) {
  return (int64_t)n_seq + (t_in + kPartRows - 1) / kPartRows;
}

size_t score_ws_bytes(int64_t t_in, int n_seq) {
  size_t bytes = sizeof(Partial) * (size_t)n_parts(t_in, n_seq);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += sizeof(float) * (size_t)t_in;   // b~ when the caller passes no b_raw
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_score(const void* x, int dt, int64_t x_row_stride, int64_t t_in, int d, int h,
                        const void* w1, const float* b1, const float* w2, float b2,
                        const uint8_t* prunable, const int32_t* cu, int n_seq, float eps,
                        float norm_eps, float* b_raw, float* b, void* ws, hipStream_t st) {
  Partial* part = static_cast<Partial*>(ws);
  size_t off = (sizeof(Partial) * (size_t)n_parts(t_in, n_seq) + 255) & ~(size_t)255;
  float* braw = b_raw ? b_raw : reinterpret_cast<float*>(static_cast<char*>(ws) + off);
  if (t_in == 0) return hipSuccess;
  int part_rows = kPartRows;
  if (dt == 1) {
    // rows per workgroup: 256 when that still gives a workgroup per CU,
    // else 128 or 64 (short inputs), so that small batches fill the chip
    int n_cu = 0;
    const hipError_t ce = device_cu_count(&n_cu);
    if (ce != hipSuccess) return ce;
    const int rg = (t_in + 255) / 256 >= n_cu ? 4 : (t_in + 127) / 128 >= n_cu ? 2 : 1;
    const dim3 grid((unsigned)((t_in + 64 * rg - 1) / (64 * rg)));
    part_rows = 64 * rg;
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(w1);
#define TG_SCORE_LAUNCH(M, N, R)                                                              \
  hipLaunchKernelGGL((score_mlp_bf16<M, N, R>), grid, dim3(kThreads), 0, st, xp, x_row_stride, \
                     t_in, d, wp, b1, w2, b2, norm_eps, braw, prunable, cu, n_seq, part)
#define TG_SCORE_CASE(M)                                                                      \
  case M:                                                                                     \
    if (norm_eps >= 0.0f) {                                                                   \
      if (rg == 4) TG_SCORE_LAUNCH(M, true, 4);                                               \
      else if (rg == 2) TG_SCORE_LAUNCH(M, true, 2);                                          \
      else TG_SCORE_LAUNCH(M, true, 1);                                                       \
    } else {                                                                                  \
      if (rg == 4) TG_SCORE_LAUNCH(M, false, 4);                                              \
      else if (rg == 2) TG_SCORE_LAUNCH(M, false, 2);                                         \
      else TG_SCORE_LAUNCH(M, false, 1);                                                      \
    }                                                                                         \
    break;
    switch (h / 32) {
      TG_SCORE_CASE(1) TG_SCORE_CASE(2) TG_SCORE_CASE(3) TG_SCORE_CASE(4)
      TG_SCORE_CASE(5) TG_SCORE_CASE(6) TG_SCORE_CASE(7) TG_SCORE_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef TG_SCORE_CASE
#undef TG_SCORE_LAUNCH
  } else {
    const dim3 grid((unsigned)((t_in + kPartRows - 1) / kPartRows));
    hipLaunchKernelGGL(score_mlp_f32, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       x_row_stride, t_in, d, h, static_cast<const float*>(w1), b1, w2, b2,
                       norm_eps, braw, prunable, cu, n_seq, part);
  }
  const dim3 g2((unsigned)n_slots(t_in, n_seq));
  hipLaunchKernelGGL(score_norm, g2, dim3(256), 0, st, braw, prunable, cu, n_seq, t_in, part,
                     part_rows, eps, b);
  return hipGetLastError();
}

}  // namespace tg
