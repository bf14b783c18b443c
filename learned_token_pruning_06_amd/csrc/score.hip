// tg_score: the gate's scoring network and its normalisation
// (TokenGate §4.1 Eq. 3):
//   b~_j = w2 . SiLU(W1 x_j + b1) + b2
//   b_j  = b~_j / sqrt(mean_{P_s} b~^2 + eps) on prunable tokens, 0 on prompt tokens.
//
// bf16 path: a skinny GEMM C^T[h, row] = W1[h, d] . x[row, d]^T on MFMA
// (v_mfma_f32_32x32x16_bf16), with the SiLU / w2 epilogue fused so only one
// float per row leaves the kernel.  Each workgroup owns 256 rows and all h
// columns (so the epilogue reduction over h stays in the workgroup): every
// wave holds 64 rows x h in accumulators, streams its own x rows straight
// from HBM into B-operand registers (one K-step of prefetch), and shares the
// W1 K-slice through padded LDS.  The transposed orientation puts one row per
// lane, so the reduction over h is in-lane plus one cross-half exchange.
// Bound: HBM (2*d bytes per row) near the MFMA ridge; see the roofline notes.
//
// Normalisation: per-sequence sums of squares in 2048-token chunks (fp64
// partials, fixed reduction order), then every chunk reduces its sequence's
// partials in the same fixed order and divides.  No float atomics, so the
// result is bitwise reproducible.
#include "common.h"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kRowsPerWG = 256;
constexpr int kBK = 64;              // d per K-step
constexpr int kRow = kBK + 8;        // bf16 per LDS row (144 B: rows start 4 banks apart)

TG_DEVINL bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

TG_DEVINL float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// One K-step of one wave: MFMAs on the W1 slice in LDS (A operand) and the
// wave's 64 x rows staged in its private LDS tile (B operand, two row tiles).
template <int MT>
TG_DEVINL void score_kstep(floatx16 (&acc)[MT][2], const uint16_t* swb, const uint16_t* sxw,
                           int n, int g) {
#pragma unroll
  for (int s = 0; s < kBK / 16; ++s) {
    const bf16x8 bop0 = as_bf16x8(ld16(&sxw[n * kRow + 32 * g + 8 * s]));
    const bf16x8 bop1 = as_bf16x8(ld16(&sxw[(32 + n) * kRow + 32 * g + 8 * s]));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 aop = as_bf16x8(ld16(&swb[(32 * mt + n) * kRow + 32 * g + 8 * s]));
      acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop0, acc[mt][0], 0, 0, 0);
      acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop1, acc[mt][1], 0, 0, 0);
    }
  }
}

// One workgroup = 256 rows x all h columns; wave w owns rows [64w, 64w + 64).
// x is read with coalesced 16-byte loads (8 rows x 128 B per instruction),
// two K-steps ahead, and written to a wave-private LDS tile from which the
// MFMA B operands are read (a wave's LDS operations complete in order, so
// the tile needs no barrier).  The W1 slice of each K-step is shared by the
// four waves through a double-buffered LDS tile (one barrier per K-step),
// staged through registers in two halves.
template <int MT>
__global__ __launch_bounds__(256) void score_mlp_bf16(
    const uint16_t* __restrict__ x, int64_t xs, int64_t t_in, int d,
    const uint16_t* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    float b2, float* __restrict__ b_raw) {
  constexpr int H = 32 * MT;
  constexpr int CPR = kBK / 8;               // 16-byte chunks per row slice (8)
  constexpr int VPT = H * CPR / 256;         // W1 vectors per thread per K-step (= MT)
  constexpr int NSPLIT = VPT % 2 == 0 ? 2 : 1;
  constexpr int VPP = VPT / NSPLIT;
  constexpr int RSTEP = 256 / CPR;           // W1 rows between a thread's vectors (32)
  static_assert(H * CPR % 256 == 0, "loader shape");
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][H * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t sx[4][64 * kRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerWG + wv * 64;
  uint16_t* sxw = sx[wv];

  // x loader: load j covers wave rows 8j + lane/8, 16-byte chunk lane%8
  const uint16_t* xsrc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int64_t r = row0 + 8 * j + (lane >> 3);
    r = r < t_in ? r : t_in - 1;
    xsrc[j] = x + r * xs + 8 * (lane & 7);
  }
  const int xdst = (lane >> 3) * kRow + 8 * (lane & 7);
  // W1 loader: thread vector i -> row tid / CPR + i * RSTEP, chunk tid % CPR
  const uint16_t* wsrc = w1 + (int64_t)(tid / CPR) * d + 8 * (tid % CPR);
  const int wdst = (tid / CPR) * kRow + 8 * (tid % CPR);

  floatx16 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[mt][0][r] = 0.f;
      acc[mt][1][r] = 0.f;
    }

  const int nk = d / kBK;
  u32x4 xa[8], xb[8];          // x of K-steps it+1 (xa) and it+2 (xb), or clamped repeats
  u32x4 wreg[VPP];
  // prologue: W1 slice 0 and x step 0 to LDS, x steps 1 and 2 to registers
#pragma unroll
  for (int p = 0; p < NSPLIT; ++p) {
#pragma unroll
    for (int i = 0; i < VPP; ++i) wreg[i] = ld16(wsrc + (int64_t)(p * VPP + i) * RSTEP * d);
#pragma unroll
    for (int i = 0; i < VPP; ++i) st16(&sw[0][wdst + (p * VPP + i) * RSTEP * kRow], wreg[i]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) st16(&sxw[xdst + 8 * j * kRow], ld_nt16(xsrc[j]));
  {
    const int k1 = (nk > 1 ? 1 : 0) * kBK, k2 = (nk > 2 ? 2 : nk - 1) * kBK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xa[j] = ld_nt16(xsrc[j] + k1);
      xb[j] = ld_nt16(xsrc[j] + k2);
    }
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    // next W1 slice (the last step re-reads its own: no branch, buffer unused)
    const int kw = (it + 1 < nk ? it + 1 : it) * kBK;
#pragma unroll
    for (int i = 0; i < VPP; ++i) wreg[i] = ld16(wsrc + (int64_t)i * RSTEP * d + kw);
    score_kstep<MT>(acc, sw[buf], sxw, n, g);
#pragma unroll
    for (int i = 0; i < VPP; ++i) st16(&sw[buf ^ 1][wdst + i * RSTEP * kRow], wreg[i]);
    if (NSPLIT == 2) {
#pragma unroll
      for (int i = 0; i < VPP; ++i) wreg[i] = ld16(wsrc + (int64_t)(VPP + i) * RSTEP * d + kw);
#pragma unroll
      for (int i = 0; i < VPP; ++i) st16(&sw[buf ^ 1][wdst + (VPP + i) * RSTEP * kRow], wreg[i]);
    }
    // x of step it+1 to the wave's tile (after this step's reads, in order),
    // then rotate the register ring and fetch step it+3
    const int k3 = (it + 3 < nk ? it + 3 : nk - 1) * kBK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      st16(&sxw[xdst + 8 * j * kRow], xa[j]);
      xa[j] = xb[j];
      xb[j] = ld_nt16(xsrc[j] + k3);
    }
    __syncthreads();
  }

  // epilogue: lane (n, g) holds h = 32mt + 8(r/4) + 4g + (r%4) of rows 32nt + n
  float part0 = 0.f, part1 = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int h0 = 32 * mt + 8 * r4 + 4 * g;
      const float4 bb = b1 ? *reinterpret_cast<const float4*>(b1 + h0) : make_float4(0, 0, 0, 0);
      const float4 ww = *reinterpret_cast<const float4*>(w2 + h0);
      part0 = fmaf(silu_f(acc[mt][0][4 * r4 + 0] + bb.x), ww.x, part0);
      part0 = fmaf(silu_f(acc[mt][0][4 * r4 + 1] + bb.y), ww.y, part0);
      part0 = fmaf(silu_f(acc[mt][0][4 * r4 + 2] + bb.z), ww.z, part0);
      part0 = fmaf(silu_f(acc[mt][0][4 * r4 + 3] + bb.w), ww.w, part0);
      part1 = fmaf(silu_f(acc[mt][1][4 * r4 + 0] + bb.x), ww.x, part1);
      part1 = fmaf(silu_f(acc[mt][1][4 * r4 + 1] + bb.y), ww.y, part1);
      part1 = fmaf(silu_f(acc[mt][1][4 * r4 + 2] + bb.z), ww.z, part1);
      part1 = fmaf(silu_f(acc[mt][1][4 * r4 + 3] + bb.w), ww.w, part1);
    }
  }
  const float tot0 = part0 + __shfl_xor(part0, 32, 64);
  const float tot1 = part1 + __shfl_xor(part1, 32, 64);
  if (g == 0) {
    if (row0 + n < t_in) b_raw[row0 + n] = tot0 + b2;
    if (row0 + 32 + n < t_in) b_raw[row0 + 32 + n] = tot1 + b2;
  }
}

// fp32 scorer on the vector ALU: one wave per row, lanes over hidden units.
__global__ __launch_bounds__(256) void score_mlp_f32(const float* __restrict__ x, int64_t xs,
                                                     int64_t t_in, int d, int h,
                                                     const float* __restrict__ w1,
                                                     const float* __restrict__ b1,
                                                     const float* __restrict__ w2, float b2,
                                                     float* __restrict__ b_raw) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= t_in) return;
  const float* xp = x + row * xs;
  float part = 0.f;
  for (int j = lane; j < h; j += 64) {
    const float* wp = w1 + (int64_t)j * d;
    float acc = 0.f;
    for (int e = 0; e < d; ++e) acc = fmaf(xp[e], wp[e], acc);
    const float v = acc + (b1 ? b1[j] : 0.f);
    part = fmaf(v / (1.0f + expf(-v)), w2[j], part);
  }
  part = wave_sum(part);
  if (lane == 0) b_raw[row] = part + b2;
}

struct Partial {
  double sumsq;
  int64_t count;
};

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

__global__ __launch_bounds__(256) void score_partial(const float* __restrict__ b_raw,
                                                     const uint8_t* __restrict__ pr,
                                                     const int32_t* __restrict__ cu, int n_seq,
                                                     int64_t t_in, Partial* __restrict__ part) {
  __shared__ double sd[4];
  __shared__ int64_t sc[4];
  int s, nch;
  int64_t begin, end;
  if (!locate(cu, n_seq, t_in, blockIdx.x, s, begin, end, nch)) return;
  double acc = 0.0;
  int64_t cnt = 0;
  for (int64_t j = begin + threadIdx.x; j < end; j += 256) {
    if (pr[j]) {
      const double v = b_raw[j];
      acc = fma(v, v, acc);
      ++cnt;
    }
  }
  acc = wave_sum(acc);
  cnt = wave_sum(cnt);
  if ((threadIdx.x & 63) == 0) {
    sd[threadIdx.x >> 6] = acc;
    sc[threadIdx.x >> 6] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    part[blockIdx.x].sumsq = ((sd[0] + sd[1]) + sd[2]) + sd[3];
    part[blockIdx.x].count = sc[0] + sc[1] + sc[2] + sc[3];
  }
}

__global__ __launch_bounds__(256) void score_norm(const float* __restrict__ b_raw,
                                                  const uint8_t* __restrict__ pr,
                                                  const int32_t* __restrict__ cu, int n_seq,
                                                  int64_t t_in, const Partial* __restrict__ part,
                                                  float eps,
                                                  float* __restrict__ b) {
  __shared__ double sd[4];
  __shared__ int64_t sc[4];
  int s, nch;
  int64_t begin, end;
  if (!locate(cu, n_seq, t_in, blockIdx.x, s, begin, end, nch)) return;
  // every chunk of the sequence reduces the same partials in the same order
  const int64_t p0 = slot0_of(cu, s, CH);
  double acc = 0.0;
  int64_t cnt = 0;
  for (int i = threadIdx.x; i < nch; i += 256) {
    acc += part[p0 + i].sumsq;
    cnt += part[p0 + i].count;
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
  for (int64_t j = begin + threadIdx.x; j < end; j += 256) b[j] = pr[j] ? b_raw[j] / r : 0.0f;
}

int64_t n_slots(int64_t t_in, int n_seq) { return (int64_t)n_seq + (t_in + CH - 1) / CH; }

}  // namespace

size_t score_ws_bytes(int64_t t_in, int n_seq) {
  size_t bytes = sizeof(Partial) * (size_t)n_slots(t_in, n_seq);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += sizeof(float) * (size_t)t_in;   // b~ when the caller passes no b_raw
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_score(const void* x, int dt, int64_t x_row_stride, int64_t t_in, int d, int h,
                        const void* w1, const float* b1, const float* w2, float b2,
                        const uint8_t* prunable, const int32_t* cu, int n_seq, float eps,
                        float* b_raw, float* b, void* ws, hipStream_t st) {
  Partial* part = static_cast<Partial*>(ws);
  size_t off = (sizeof(Partial) * (size_t)n_slots(t_in, n_seq) + 255) & ~(size_t)255;
  float* braw = b_raw ? b_raw : reinterpret_cast<float*>(static_cast<char*>(ws) + off);
  if (t_in == 0) return hipSuccess;
  if (dt == 1) {
    const dim3 grid((unsigned)((t_in + kRowsPerWG - 1) / kRowsPerWG));
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(w1);
    switch (h / 32) {
#define TG_SCORE_CASE(M)                                                                    \
  case M:                                                                                   \
    hipLaunchKernelGGL(score_mlp_bf16<M>, grid, dim3(256), 0, st, xp, x_row_stride, t_in, d, \
                       wp, b1, w2, b2, braw);                                               \
    break;
      TG_SCORE_CASE(1) TG_SCORE_CASE(2) TG_SCORE_CASE(3) TG_SCORE_CASE(4)
      TG_SCORE_CASE(5) TG_SCORE_CASE(6) TG_SCORE_CASE(7) TG_SCORE_CASE(8)
#undef TG_SCORE_CASE
      default: return hipErrorInvalidValue;
    }
  } else {
    const dim3 grid((unsigned)((t_in + 3) / 4));
    hipLaunchKernelGGL(score_mlp_f32, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       x_row_stride, t_in, d, h, static_cast<const float*>(w1), b1, w2, b2, braw);
  }
  const dim3 g2((unsigned)n_slots(t_in, n_seq));
  hipLaunchKernelGGL(score_partial, g2, dim3(256), 0, st, braw, prunable, cu, n_seq, t_in, part);
  hipLaunchKernelGGL(score_norm, g2, dim3(256), 0, st, braw, prunable, cu, n_seq, t_in, part, eps,
                     b);
  return hipGetLastError();
}

}  // namespace tg
