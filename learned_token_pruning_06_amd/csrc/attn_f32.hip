// tg_gated_attn, fp32 on the vector ALU (TokenGate §4.2 Eq. 8).
//
// One wave per (query row, query head): lanes take 64 keys at a time for
// the logits  tau * (s * q.k_j + gain_h * b_j)  and the output dimensions
// for the value sum, with an online softmax over the key blocks.  Meant for
// small fp32 problems and as a full-precision path; the bf16 path on matrix
// cores is the fast one.
#include "common.h"

namespace tg {
namespace {

template <int DH>
__global__ __launch_bounds__(64) void gated_attn_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, const float* __restrict__ kept_b, const int32_t* __restrict__ kept_pos,
    const int32_t* __restrict__ kept_cu, int n_seq, int hq, int hkv,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm_scale) {
  // a row outside every sequence range attends to nothing past itself; keys
  // are read only at indices in [lo, row], all below t_kept
  constexpr int NO = DH / 64;
  __shared__ float sq[DH];
  __shared__ float sp[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int head = blockIdx.y;
  const int kvh = head / (hq / hkv);
  // sequence of this row: largest s with kept_cu[s] <= row
  int lo_s = 0, hi_s = n_seq - 1, s = 0;
  while (lo_s <= hi_s) {
    const int mid = (lo_s + hi_s) >> 1;
    if (kept_cu[mid] <= row) {
      s = mid;
      lo_s = mid + 1;
    } else {
      hi_s = mid - 1;
    }
  }
  const int lo = kept_cu[s] <= row ? kept_cu[s] : row;
  const int a = row - lo;
  float lam = 1.0f;
  if (kept_pos) lam = logf((float)(a + 1)) / logf(fmaxf(2.0f, (float)(kept_pos[row] + 1)));
  const float tau = temp[head] * lam;
  const float gh = gain[head];
  const int64_t ks = (int64_t)hkv * DH;
#pragma unroll
  for (int i = 0; i < NO; ++i) sq[lane + 64 * i] = q[((int64_t)row * hq + head) * DH + lane + 64 * i];
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  float o[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) o[i] = 0.f;
  for (int j0 = 0; j0 <= a; j0 += 64) {
    const int j = j0 + lane;
    float logit = -INFINITY;
    if (j <= a) {
      const float* kp = k + (int64_t)(lo + j) * ks + (int64_t)kvh * DH;
      float dot = 0.f;
      for (int d = 0; d < DH; ++d) dot = fmaf(sq[d], kp[d], dot);
      logit = tau * (sm_scale * dot + gh * kept_b[lo + j]);
    }
    const float cmax = wave_max(logit);
    const float mnew = fmaxf(m, cmax);
    const float alpha = expf(m - mnew);
    const float p = j <= a ? expf(logit - mnew) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] *= alpha;
    m = mnew;
    sp[lane] = p;
    __syncthreads();
    const int nj = a + 1 - j0 < 64 ? a + 1 - j0 : 64;
    for (int jj = 0; jj < nj; ++jj) {
      const float* vp = v + (int64_t)(lo + j0 + jj) * ks + (int64_t)kvh * DH;
#pragma unroll
      for (int i = 0; i < NO; ++i) o[i] = fmaf(sp[jj], vp[lane + 64 * i], o[i]);
    }
    __syncthreads();
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < NO; ++i) out[((int64_t)row * hq + head) * DH + lane + 64 * i] = o[i] * inv;
}

}  // namespace

hipError_t launch_attn_f32(const void* q, const void* k, const void* v, void* out, int64_t t_kept,
                           const float* kept_b, const int32_t* kept_pos, const int32_t* kept_cu,
                           int n_seq, int max_len, int hq, int hkv, int dh, const float* gain,
                           const float* temp, float sm_scale, hipStream_t st) {
  (void)max_len;
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / sqrtf((float)dh);
  const dim3 grid((unsigned)t_kept, (unsigned)hq);
  if (dh == 128)
    hipLaunchKernelGGL(gated_attn_f32<128>, grid, dim3(64), 0, st, (const float*)q,
                       (const float*)k, (const float*)v, (float*)out, kept_b, kept_pos, kept_cu,
                       n_seq, hq, hkv, gain, temp, sm_scale);
  else
    hipLaunchKernelGGL(gated_attn_f32<64>, grid, dim3(64), 0, st, (const float*)q,
                       (const float*)k, (const float*)v, (float*)out, kept_b, kept_pos, kept_cu,
                       n_seq, hq, hkv, gain, temp, sm_scale);
  return hipGetLastError();
}

}  // namespace tg
