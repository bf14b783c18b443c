// tg_gated_decode: one decode step of token-gated attention over the pruned
// KV cache of each sequence (TokenGate §3 "Prefill, decode, and the KV cache":
// a decode step attends to the cache and appends to it; above the gate the
// cache holds the kept tokens only, and generated tokens are never pruned).
// For sequence s with cache rows [c_s, c_{s+1}), the new token's own key and
// value already appended as the last row, and query head h on KV head kv(h):
//
//   logit_j = tau * (sm_scale * q . k_j + gain_h * b_j)        (§4.2 Eq. 8)
//   tau     = temp_h * log(m) / log(max(2, p))                  (Eq. 7)
//   out     = sum_j softmax_j(logit) v_j
//
// with m = the cache length and p = q_pos + 1, i.e. exactly the last query
// row of the prefill attention over the same rows.
//
// Split over the keys (flash decoding).  A workgroup of four waves takes one
// (sequence, KV head) pair for all G query heads of its group and walks the
// sequence's 256-key chunks c, c + n_chunks, ...; each wave owns 64 keys of
// a chunk.  Lanes cover a cache row in 16-byte pieces (DH/8 lanes per row),
// so every wave-wide load reads whole rows; K and V of a step are requested
// together.  The dot products run on v_dot2_f32_bf16 and are summed over the
// lanes of a row by a DPP reduce-scatter that leaves one key per lane; the
// softmax maxima and sums are DPP row reductions plus four lane reads; the
// probabilities reach the lanes that own output dimensions through LDS.  The
// workgroup leaves, per query head, its running maximum (log2 domain),
// normaliser and unnormalised output in the workspace; a second kernel
// merges the chunks.  Decode is bound by reading the cache: 4 * dh bytes per
// key and KV head.
#include "common.h"

namespace tg {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 256;           // keys per workgroup step (64 per wave)
constexpr int kThreads = 256;
constexpr int kTargetBlocks = 512;    // two resident workgroups per CU
constexpr float kLog2e = 1.4426950408889634f;

TG_DEVINL float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}
TG_DEVINL float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
TG_DEVINL float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP lane permutations inside a row of 16 lanes (gfx9 DPP control codes)
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]: lane i <-> i ^ 1
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]: lane i <-> i ^ 2
constexpr int kDppHalfMirror = 0x141;   // lane i <-> i ^ 7
constexpr int kDppMirror = 0x140;       // lane i <-> i ^ 15

template <int CTRL>
TG_DEVINL float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// One reduce-scatter step: the lane and its DPP partner (which differs in
// the lane bit `up` tests) keep complementary halves of their N values and
// add the partner's copy of the kept half.
template <int CTRL, int N>
TG_DEVINL void rs_step(float* v, bool up) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float keep = up ? v[k + N / 2] : v[k];
    const float send = up ? v[k] : v[k + N / 2];
    v[k] = keep + dpp<CTRL>(send);
  }
}

// Reduce-scatter of LPR values over the LPR lanes of a row (LPR = 16 or 8):
// the partner masks 15, 7, 2, 1 are independent, so value 0 of every lane
// ends up as the sum over the row of the value with index (lane mod LPR).
template <int LPR>
TG_DEVINL void reduce_scatter(float* v, int lane) {
  if constexpr (LPR == 16) rs_step<kDppMirror, 16>(v, lane & 8);
  rs_step<kDppHalfMirror, 8>(v, lane & 4);
  rs_step<kDppXor2, 4>(v, lane & 2);
  rs_step<kDppXor1, 2>(v, lane & 1);
}

TG_DEVINL float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// maximum / sum over the 64 lanes: DPP within the rows, then the four rows
TG_DEVINL float wave_max64(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}
TG_DEVINL float wave_sum64(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}

TG_DEVINL __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7fffffff ? (bytes > 0 ? bytes : 0)
                                                                    : 0x7fffffff),
                                           0x00020000);
}

int chunks_for(int n_seq, int hkv, int64_t max_len) {
  const int64_t need = max_len > 0 ? (max_len + kChunk - 1) / kChunk : 1;
  const int64_t pairs = (int64_t)n_seq * hkv;
  int64_t fill = (kTargetBlocks + pairs - 1) / pairs;
  if (fill < 1) fill = 1;
  return (int)(need < fill ? need : fill);
}

template <int DH, int G>
__global__ __launch_bounds__(kThreads) void decode_partial(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const float* __restrict__ cache_b,
    const int32_t* __restrict__ cache_cu, const int32_t* __restrict__ q_pos, int64_t t_cache,
    int hq, int hkv, const float* __restrict__ gain, const float* __restrict__ temp,
    float sm_scale, int n_chunks, float* __restrict__ ws) {
  constexpr int LPR = DH / 8;      // lanes per cache row
  constexpr int RPI = 64 / LPR;    // rows per wave-wide load
  constexpr int NI = LPR;          // loads per wave and step (64 keys)
  __shared__ float sm[4][G], sl[4][G];
  __shared__ __attribute__((aligned(16))) float so[4][G][DH];
  __shared__ __attribute__((aligned(16))) float sp[4][G][64];   // probabilities, per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % LPR, rg = lane / LPR;
  const int kvh = blockIdx.x, chunk = blockIdx.y, s = blockIdx.z;
  // rows are clamped to [0, t_cache): inconsistent offsets cannot read out of bounds
  const int64_t lo = cache_cu[s] < t_cache ? cache_cu[s] : t_cache;
  const int64_t hi = cache_cu[s + 1] < t_cache ? cache_cu[s + 1] : t_cache;
  const int64_t len = hi > lo ? hi - lo : 0;
  const int h0 = kvh * G;
  const int64_t kvs = (int64_t)hkv * DH;

  // per head: logit = a_g * dot + c_g * b_j  (log2 domain)
  float a[G], c[G];
  u32x4 qr[G];
  {
    float lam = 1.0f;
    if (q_pos && len > 0) lam = logf((float)len) / logf(fmaxf(2.0f, (float)q_pos[s] + 1.0f));
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float tau = temp[h0 + g] * lam * kLog2e;
      a[g] = tau * sm_scale;
      c[g] = tau * gain[h0 + g];
      qr[g] = ld16(q + ((int64_t)s * hq + h0 + g) * DH + 8 * sub);
    }
  }

  float mrun[G], lrun[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    lrun[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
  }

  const uint16_t* kbase = kc + lo * kvs + (int64_t)kvh * DH;
  const uint16_t* vbase = vc + lo * kvs + (int64_t)kvh * DH;
  for (int64_t c0 = (int64_t)chunk * kChunk; c0 < len; c0 += (int64_t)n_chunks * kChunk) {
    const int64_t kb = c0 + 64 * wv;                 // this wave's first key
    if (kb >= len) break;                            // later chunks lie further out
    // rows from kb on; rows past the sequence read zeros through the range
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + kb * kvs, (len - kb) * kvs * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + kb * kvs, (len - kb) * kvs * 2);
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int off = (int)(((RPI * i + rg) * kvs + 8 * sub) * 2);
      kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int off = (int)(((RPI * i + rg) * kvs + 8 * sub) * 2);
      vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
    // after the reduce-scatter below, lane (rg, sub) holds key kb + RPI*sub + rg
    const int64_t j = kb + RPI * sub + rg;
    const bool valid = j < len;
    const float bj = (valid && cache_b) ? cache_b[lo + j] : 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float v[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float d = dot2(kr[i][0], qr[g][0], 0.0f);
        d = dot2(kr[i][1], qr[g][1], d);
        d = dot2(kr[i][2], qr[g][2], d);
        v[i] = dot2(kr[i][3], qr[g][3], d);
      }
      reduce_scatter<LPR>(v, lane);
      const float logit = valid ? fmaf(a[g], v[0], c[g] * bj) : -INFINITY;
      const float mnew = fmaxf(mrun[g], wave_max64(logit));   // finite: key kb is valid
      const float scale = __builtin_amdgcn_exp2f(mrun[g] - mnew);
      const float p = valid ? __builtin_amdgcn_exp2f(logit - mnew) : 0.0f;
      lrun[g] = fmaf(lrun[g], scale, wave_sum64(p));
      mrun[g] = mnew;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= scale;
      // row rg needs the probabilities of keys kb + RPI*i + rg, i < NI, which
      // sit in the lanes of that row in order of sub
      sp[wv][g][rg * LPR + sub] = p;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i4 = 0; i4 < NI / 4; ++i4) {
        const float4 pv = *reinterpret_cast<const float4*>(&sp[wv][g][rg * LPR + 4 * i4]);
        const float pk[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const u32x4 w4 = vr[4 * i4 + u];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[g][2 * w] = fmaf(pk[u], bf16_lo(w4[w]), acc[g][2 * w]);
            acc[g][2 * w + 1] = fmaf(pk[u], bf16_hi(w4[w]), acc[g][2 * w + 1]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // sum the RPI row groups of the wave, then merge the four waves
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], o, 64);
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) so[wv][g][8 * sub + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm[wv][g] = mrun[g];
      sl[wv][g] = lrun[g];
    }
  }
  __syncthreads();
  // workspace record per (sequence, query head, chunk): m, l, o[DH]
  for (int i = tid; i < G * DH; i += kThreads) {
    const int g = i / DH, d = i % DH;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, sm[w][g]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = sm[w][g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sm[w][g] - m);
      o = fmaf(f, so[w][g][d], o);
      l = fmaf(f, sl[w][g], l);
    }
    float* rec = ws + (((int64_t)s * hq + h0 + g) * n_chunks + chunk) * (DH + 2);
    rec[2 + d] = o;
    if (d == 0) {
      rec[0] = m;
      rec[1] = l;
    }
  }
}

// One workgroup per (sequence, query head) merges the chunks.  Thread
// (cl, d) folds dimension d of the chunks cl, cl + 256/DH, ... into its own
// running (maximum, normaliser, output), requesting kBatch records at a
// time; the 256/DH partial states then meet in LDS.
template <int DH>
__global__ __launch_bounds__(kThreads) void decode_combine(const float* __restrict__ ws, int hq,
                                                          int n_chunks,
                                                          uint16_t* __restrict__ out) {
  constexpr int NC = kThreads / DH;
  constexpr int kBatch = 16;
  __shared__ float red_m[kThreads], red_l[kThreads], red_o[kThreads];
  const int s = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int d = tid % DH, cl = tid / DH;
  const float* rec = ws + ((int64_t)s * hq + h) * n_chunks * (DH + 2);
  float m = -INFINITY, l = 0.0f, o = 0.0f;
  for (int c0 = cl; c0 < n_chunks; c0 += NC * kBatch) {
    float mc[kBatch], lc[kBatch], oc[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + NC * b;
      const float* r = rec + (int64_t)(c < n_chunks ? c : 0) * (DH + 2);
      mc[b] = c < n_chunks ? r[0] : -INFINITY;
      lc[b] = r[1];
      oc[b] = r[2 + d];
    }
    float mb = m;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) mb = fmaxf(mb, mc[b]);
    if (mb != -INFINITY) {
      const float f0 = __builtin_amdgcn_exp2f(m - mb);      // 0 while m = -inf
      l *= f0;
      o *= f0;
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const float f = mc[b] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc[b] - mb);
        l = fmaf(f, lc[b], l);
        o = fmaf(f, oc[b], o);
      }
      m = mb;
    }
  }
  red_m[tid] = m;
  red_l[tid] = l;
  red_o[tid] = o;
  __syncthreads();
  if (cl == 0) {
    float mt = -INFINITY;
#pragma unroll
    for (int k = 0; k < NC; ++k) mt = fmaxf(mt, red_m[k * DH + d]);
    float ot = 0.0f, lt = 0.0f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const float mk = red_m[k * DH + d];
      const float f = mk == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mk - mt);
      ot = fmaf(f, red_o[k * DH + d], ot);
      lt = fmaf(f, red_l[k * DH + d], lt);
    }
    const __bf16 y = (__bf16)(lt > 0.0f ? ot / lt : 0.0f);
    out[((int64_t)s * hq + h) * DH + d] = __builtin_bit_cast(uint16_t, y);
  }
}

template <int DH, int G>
hipError_t launch_g(const void* q, const void* k, const void* v, void* out, const float* cache_b,
                    const int32_t* cache_cu, const int32_t* q_pos, int n_seq, int64_t t_cache,
                    int n_chunks, int hq, int hkv, const float* gain, const float* temp,
                    float sm_scale, float* ws, hipStream_t st) {
  hipLaunchKernelGGL((decode_partial<DH, G>), dim3(hkv, n_chunks, n_seq), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), cache_b, cache_cu, q_pos, t_cache, hq, hkv,
                     gain, temp, sm_scale, n_chunks, ws);
  hipLaunchKernelGGL((decode_combine<DH>), dim3(n_seq, hq), dim3(kThreads), 0, st, ws, hq, n_chunks,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace

size_t decode_ws_bytes(int n_seq, int hq, int hkv, int dh, int64_t max_len) {
  return (size_t)n_seq * hq * chunks_for(n_seq, hkv, max_len) * (dh + 2) * sizeof(float);
}

hipError_t launch_decode(const void* q, const void* k, const void* v, void* out,
                         const float* cache_b, const int32_t* cache_cu, const int32_t* q_pos,
                         int n_seq, int64_t t_cache, int64_t max_len, int hq, int hkv, int dh,
                         const float* gain, const float* temp, float sm_scale, void* ws,
                         hipStream_t st) {
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / sqrtf((float)dh);
  const int G = hq / hkv;
  const int n_chunks = chunks_for(n_seq, hkv, max_len);
  float* w = static_cast<float*>(ws);
#define TG_DEC(DHv, Gv)                                                                         \
  if (dh == DHv && G == Gv)                                                                     \
    return launch_g<DHv, Gv>(q, k, v, out, cache_b, cache_cu, q_pos, n_seq, t_cache, n_chunks, \
                             hq, hkv, gain, temp, sm_scale, w, st);
  TG_DEC(128, 1) TG_DEC(128, 2) TG_DEC(128, 4) TG_DEC(128, 8)
  TG_DEC(64, 1) TG_DEC(64, 2) TG_DEC(64, 4) TG_DEC(64, 8)
#undef TG_DEC
  return hipErrorInvalidValue;
}

}  // namespace tg
