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
constexpr int kLdsRow = kBK + 8;     // bf16 per LDS row: 144 B, shifts banks by 4 per row

TG_DEVINL bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

TG_DEVINL float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

template <int MT>
__global__ __launch_bounds__(256) void score_mlp_bf16(
    const uint16_t* __restrict__ x, int64_t xs, int64_t t_in, int d,
    const uint16_t* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    float b2, float* __restrict__ b_raw) {
  constexpr int H = 32 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][H * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerWG + wv * 64;

  const uint16_t* xr[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    int64_t r = row0 + 32 * nt + n;
    r = r < t_in ? r : t_in - 1;
    xr[nt] = x + r * xs + 32 * g;
  }

  // W1 K-slice loader: H rows x 64 columns = 8H vectors of 16 bytes
  constexpr int NV = H * kBK / 8;
  constexpr int VPT = (NV + 255) / 256;
  auto load_w = [&](int k0, uint4* reg) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + 256 * i;
      if (v < NV) {
        const int row = v >> 3, ch = v & 7;
        reg[i] = *reinterpret_cast<const uint4*>(w1 + (int64_t)row * d + k0 + 8 * ch);
      }
    }
  };
  auto store_w = [&](int buf, const uint4* reg) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + 256 * i;
      if (v < NV) {
        const int row = v >> 3, ch = v & 7;
        *reinterpret_cast<uint4*>(&sw[buf][row * kLdsRow + 8 * ch]) = reg[i];
      }
    }
  };
  auto load_x = [&](int k0, uint4 (*reg)[4]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        reg[nt][s] = ld_nt16(reinterpret_cast<const uint4*>(xr[nt] + k0) + s);
  };

  floatx16 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  uint4 wreg[VPT];
  uint4 xcur[2][4], xnext[2][4];
  load_w(0, wreg);
  store_w(0, wreg);
  load_x(0, xcur);
  __syncthreads();

  const int nk = d / kBK;
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      load_w((it + 1) * kBK, wreg);
      load_x((it + 1) * kBK, xnext);
    }
    const uint16_t* swb = sw[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 bop0 = as_bf16x8(xcur[0][s]);
      const bf16x8 bop1 = as_bf16x8(xcur[1][s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 aop = as_bf16x8(
            *reinterpret_cast<const uint4*>(&swb[(32 * mt + n) * kLdsRow + 32 * g + 8 * s]));
        acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop0, acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop1, acc[mt][1], 0, 0, 0);
      }
    }
    if (more) store_w(buf ^ 1, wreg);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int s = 0; s < 4; ++s) xcur[nt][s] = xnext[nt][s];
    }
  }

  // epilogue: lane (n, g) holds h = 32mt + 8(r/4) + 4g + (r%4) of rows 32nt + n
  float part[2] = {0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int h0 = 32 * mt + 8 * r4 + 4 * g;
      const float4 bb = b1 ? *reinterpret_cast<const float4*>(b1 + h0) : make_float4(0, 0, 0, 0);
      const float4 ww = *reinterpret_cast<const float4*>(w2 + h0);
      const float bbv[4] = {bb.x, bb.y, bb.z, bb.w};
      const float wwv[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          part[nt] = fmaf(silu_f(acc[mt][nt][4 * r4 + i] + bbv[i]), wwv[i], part[nt]);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float tot = part[nt] + __shfl_xor(part[nt], 32, 64);
    const int64_t r = row0 + 32 * nt + n;
    if (g == 0 && r < t_in) b_raw[r] = tot + b2;
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
