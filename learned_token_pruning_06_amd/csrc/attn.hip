// tg_gated_attn, bf16 on matrix cores (TokenGate §4.2, Eq. 8 with the
// head-wise gain of Eq. 6 and the temperature of Eq. 7):
//
//   logit_ij = tau_i * (s * q_i.k_j + gain_h * b_j),  tau_i = temp_h * log m_i / log max(2, p_i)
//
// Flash-style causal attention over the kept tokens of each sequence.
// In the log2 domain the logit is c_i * (q_i.k_j + beta_j) with
//   c_i = tau_i * s * log2(e)   (one scalar per query row, > 0)
//   beta_j = gain_h * b_j / s   (one scalar per key and head),
// so the per-key bias is loaded into the accumulator before the Q.K^T MFMAs
// and costs no vector work, and the temperature is folded into the single
// FMA that forms the exponent: p = exp2(c_i * acc - m_i).  Because c_i > 0
// the running maximum is taken on the unscaled accumulator.
//
// Work decomposition (wave64, gfx950 v_mfma_f32_32x32x16_bf16):
//  - a workgroup of 8 waves owns one block of query rows of one sequence and
//    HPW query heads that share one KV head (GQA): every K/V tile staged in
//    LDS feeds all HPW heads; two waves per SIMD let the hardware overlap one
//    wave's softmax (vector ALU) with the other's MFMAs;
//  - a wave owns 32 query rows of one head.  It computes S^T = K.Q^T (keys
//    on the MFMA M axis, queries on N), so each lane holds one query's
//    logits: the softmax statistics are per-lane scalars plus one exchange
//    between the two lane halves;
//  - P^T from the accumulators is directly the B operand of O^T = V^T.P^T
//    (keys permuted consistently between the two operands), so the output
//    accumulator also holds one query per lane;
//  - V is transposed while it is staged to LDS ([d][key]) so its MFMA operand
//    reads are contiguous;
//  - K/V tiles of 64 keys are double-buffered in LDS with one barrier per
//    tile; causal masking runs only on diagonal tiles, tiles past a wave's
//    rows are skipped, and query blocks are issued longest first;
//  - the running maximum is only moved when it grows by more than 2^8 in
//    the exponent (exact: the normaliser absorbs the stale maximum).
#include "common.h"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BKV = 64;                 // keys per tile
constexpr int NWAVE = 8;                // waves per workgroup
constexpr int NTHR = 64 * NWAVE;
constexpr int QW = 32;                  // query rows per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr float kMinScale = 1e-30f;     // keeps c_i > 0 so masked keys stay -inf

TG_DEVINL bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

TG_DEVINL uint32_t word(const uint4& u, int i) {
  return i == 0 ? u.x : (i == 1 ? u.y : (i == 2 ? u.z : u.w));
}

TG_DEVINL uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int DH, int HPW>
struct AttnCfg {
  static constexpr int QB = NWAVE * QW / HPW;    // query rows per workgroup
  static constexpr int KROW = DH + 8;            // bf16 per K row in LDS (16 B pad)
  static constexpr int VROW = BKV + 4;           // bf16 per V^T row in LDS (8 B pad)
  static constexpr int KT = DH / 16;             // MFMA K-steps over the head dim
  static constexpr int DT = DH / 32;             // output tiles over the head dim
  static constexpr int KVEC = BKV * DH / 8;      // 16-byte vectors per K tile
  static constexpr int KVPT = (KVEC + NTHR - 1) / NTHR;
  static constexpr int VUNITS = (BKV / 2) * (DH / 8);   // (2-key pair, 8-dim chunk) units
  static constexpr int VUPT = (VUNITS + NTHR - 1) / NTHR;
};

template <int DH, int HPW>
__global__ __launch_bounds__(NTHR) void gated_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ kept_cu, int n_seq,
    int t_kept, int hq, int hkv, int groups_y, const float* __restrict__ gain,
    const float* __restrict__ temp, float sm_scale) {
  using C = AttnCfg<DH, HPW>;
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][BKV * C::KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][DH * C::VROW];
  __shared__ __attribute__((aligned(16))) float sbias[2][HPW][BKV];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;

  // ---- which (sequence, query block): last slots first (longest first)
  const int64_t slot = (int64_t)gridDim.x - 1 - blockIdx.x;
  const int s = seq_of_slot(kept_cu, n_seq, slot, C::QB);
  if (s < 0) return;
  // rows are clamped to [0, t_kept): inconsistent offsets cannot read out of bounds
  const int lo = kept_cu[s] < t_kept ? kept_cu[s] : t_kept;
  const int len = (kept_cu[s + 1] < t_kept ? kept_cu[s + 1] : t_kept) - lo;
  const int q0 = (int)(slot - slot0_of(kept_cu, s, C::QB)) * C::QB;
  if (q0 >= len) return;

  const int G = hq / hkv;
  const int kvh = blockIdx.y / groups_y;
  const int hbase = kvh * G + (blockIdx.y % groups_y) * HPW;
  const int hl = wv % HPW;
  const int head = hbase + hl;
  const int wq0 = q0 + QW * (wv / HPW);          // first query row of this wave (in sequence)

  // ---- per-lane query constant c = tau * s * log2(e), one query per lane
  const int qa = wq0 + n;
  const bool qvalid = qa < len;
  float cq = kMinScale;
  if (qvalid) {
    float lam = 1.0f;
    if (kept_pos) {
      const float m = (float)(qa + 1);
      const float p = (float)(kept_pos[lo + qa] + 1);
      lam = logf(m) / logf(fmaxf(2.0f, p));
    }
    cq = fmaxf(temp[head] * lam * sm_scale * kLog2e, kMinScale);
  }

  // ---- Q fragments (B operand of S^T = K.Q^T): lane holds q[row][16kk + 8g .. +8]
  bf16x8 qf[C::KT];
  {
    const int a = qvalid ? qa : len - 1;
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)(lo + a) * hq + head) * DH);
#pragma unroll
    for (int kk = 0; kk < C::KT; ++kk) qf[kk] = as_bf16x8(qp[2 * kk + g]);
  }

  // ---- loaders (global -> registers -> LDS) for one tile of 64 keys
  const int q_end = q0 + C::QB < len ? q0 + C::QB : len;
  const int n_tiles = (q_end + BKV - 1) / BKV;
  const int64_t kvstride = (int64_t)hkv * DH;     // elements between token rows of k, v
  const uint16_t* kb_ = k + (int64_t)lo * kvstride + (int64_t)kvh * DH;
  const uint16_t* vb_ = v + (int64_t)lo * kvstride + (int64_t)kvh * DH;
  // loader thread tid < 64*HPW stages key (tid % 64) for head (tid / 64)
  const float my_bscale = tid < BKV * HPW ? gain[hbase + tid / BKV] / sm_scale : 0.0f;

  // prefetch registers for one tile: K as up to two 16-byte vectors per
  // thread, V as one (2-key, 8-dim) unit per thread, one bias value
  static_assert(C::KVPT <= 2 && C::VUPT == 1, "loader shape");
  uint4 kreg0 = make_uint4(0, 0, 0, 0), kreg1 = make_uint4(0, 0, 0, 0);
  uint4 vreg0 = make_uint4(0, 0, 0, 0), vreg1 = make_uint4(0, 0, 0, 0);
  float breg = 0.f;
  // every thread loads; units past the tile wrap around (their stores are skipped)
  const int kvi0 = tid % C::KVEC, kvi1 = (tid + NTHR) % C::KVEC;
  const int vu = tid % C::VUNITS;
  const int vkp = vu % (BKV / 2), vdc = vu / (BKV / 2);

  auto load_tile = [&](int t) {
    const int kv0 = t * BKV;
    {
      int kr = kv0 + kvi0 / (DH / 8);
      kr = kr < len ? kr : len - 1;
      kreg0 = *reinterpret_cast<const uint4*>(kb_ + (int64_t)kr * kvstride + 8 * (kvi0 % (DH / 8)));
    }
    if (C::KVPT == 2) {
      int kr = kv0 + kvi1 / (DH / 8);
      kr = kr < len ? kr : len - 1;
      kreg1 = *reinterpret_cast<const uint4*>(kb_ + (int64_t)kr * kvstride + 8 * (kvi1 % (DH / 8)));
    }
    int k0 = kv0 + 2 * vkp, k1 = k0 + 1;
    k0 = k0 < len ? k0 : len - 1;
    k1 = k1 < len ? k1 : len - 1;
    vreg0 = *reinterpret_cast<const uint4*>(vb_ + (int64_t)k0 * kvstride + 8 * vdc);
    vreg1 = *reinterpret_cast<const uint4*>(vb_ + (int64_t)k1 * kvstride + 8 * vdc);
    if (tid < BKV * HPW) {
      int kr = kv0 + (tid % BKV);
      kr = kr < len ? kr : len - 1;
      breg = kept_b[lo + kr];
    }
  };
  auto store_tile = [&](int buf) {
    if (tid < C::KVEC)
      *reinterpret_cast<uint4*>(&sk[buf][(kvi0 / (DH / 8)) * C::KROW + 8 * (kvi0 % (DH / 8))]) = kreg0;
    if (C::KVPT == 2 && tid + NTHR < C::KVEC)
      *reinterpret_cast<uint4*>(&sk[buf][(kvi1 / (DH / 8)) * C::KROW + 8 * (kvi1 % (DH / 8))]) = kreg1;
    if (tid < C::VUNITS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a0 = word(vreg0, e >> 1), a1 = word(vreg1, e >> 1);
        const uint32_t pk = (e & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u))
                                    : ((a0 & 0xffffu) | (a1 << 16));
        *reinterpret_cast<uint32_t*>(&sv[buf][(8 * vdc + e) * C::VROW + 2 * vkp]) = pk;
      }
    }
    if (tid < BKV * HPW) sbias[buf][tid / BKV][tid % BKV] = breg * my_bscale;
  };

  // ---- running state (one query per lane)
  floatx16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float mrun = -INFINITY;
  float lsum = 0.f;
  const int wq_last = wq0 + QW - 1 < len - 1 ? wq0 + QW - 1 : len - 1;
  const bool wave_has_rows = wq0 < len;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int kv0 = t * BKV;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile(t + 1);

    if (wave_has_rows && kv0 <= wq_last) {
      // S^T = beta + K.Q^T  (keys: 32mt + 8(r/4) + 4g + r%4, query: n)
      floatx16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 bb =
              *reinterpret_cast<const float4*>(&sbias[buf][hl][32 * mt + 8 * r4 + 4 * g]);
          sacc[mt][4 * r4 + 0] = bb.x;
          sacc[mt][4 * r4 + 1] = bb.y;
          sacc[mt][4 * r4 + 2] = bb.z;
          sacc[mt][4 * r4 + 3] = bb.w;
        }
#pragma unroll
      for (int kk = 0; kk < C::KT; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(
              &sk[buf][(32 * mt + n) * C::KROW + 16 * kk + 8 * g]));
          sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[mt], 0, 0, 0);
        }
      }
      // causal mask, only where the tile reaches past the wave's first row
      if (kv0 + BKV - 1 > wq0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = kv0 + 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
            sacc[mt][r] = kj > qa ? -INFINITY : sacc[mt][r];
          }
      }
      // online softmax on the unscaled accumulator (c_i > 0)
      float mx = sacc[0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * cq;
      if (__any(mx > mrun + kRescaleSlack)) {
        const float mnew = fmaxf(mrun, mx);
        const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        mrun = mnew;
      }
      const float negm = mrun == -INFINITY ? 0.0f : -mrun;
      float ls = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r], cq, negm));
          sacc[mt][r] = p;
          ls += p;
        }
      lsum += ls;
      // P^T as the B operand of O^T = V^T.P^T: K-step kk holds keys
      // 16kk + 8(e/4) + 4g + e%4, i.e. registers 8(kk%2) .. +8 of tile kk/2
      bf16x8 pf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const floatx16& sa = sacc[kk >> 1];
        const int o = 8 * (kk & 1);
        uint4 u;
        u.x = pack_bf16x2(sa[o + 0], sa[o + 1]);
        u.y = pack_bf16x2(sa[o + 2], sa[o + 3]);
        u.z = pack_bf16x2(sa[o + 4], sa[o + 5]);
        u.w = pack_bf16x2(sa[o + 6], sa[o + 7]);
        pf[kk] = as_bf16x8(u);
      }
      // O^T += V^T . P^T  (A operand: V^T rows d = 32dt + n, keys as above)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint16_t* vp = &sv[buf][(32 * dt + n) * C::VROW + 16 * kk + 4 * g];
          const uint2 lo2 = *reinterpret_cast<const uint2*>(vp);
          const uint2 hi2 = *reinterpret_cast<const uint2*>(vp + 8);
          const bf16x8 a = as_bf16x8(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], oacc[dt], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, one query per lane; d = 32dt + 8(r/4) + 4g + r%4
  const float lt = lsum + __shfl_xor(lsum, 32, 64);
  if (!qvalid) return;
  const float inv = 1.0f / lt;
  uint16_t* op = out + ((int64_t)(lo + qa) * hq + head) * DH;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      uint2 pk;
      pk.x = pack_bf16x2(oacc[dt][4 * r4 + 0] * inv, oacc[dt][4 * r4 + 1] * inv);
      pk.y = pack_bf16x2(oacc[dt][4 * r4 + 2] * inv, oacc[dt][4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + 32 * dt + 8 * r4 + 4 * g) = pk;
    }
}

template <int DH, int HPW>
hipError_t launch_cfg(const void* q, const void* k, const void* v, void* out, int64_t t_kept,
                      const float* kept_b, const int32_t* kept_pos, const int32_t* kept_cu,
                      int n_seq, int hq, int hkv, const float* gain, const float* temp,
                      float sm_scale, hipStream_t st) {
  constexpr int QB = AttnCfg<DH, HPW>::QB;
  const int G = hq / hkv;
  const int groups_y = G / HPW;
  const dim3 grid((unsigned)(n_seq + (t_kept + QB - 1) / QB), (unsigned)(hkv * groups_y));
  hipLaunchKernelGGL((gated_attn_bf16<DH, HPW>), grid, dim3(NTHR), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), kept_b, kept_pos,
                     kept_cu, n_seq, (int)t_kept, hq, hkv, groups_y, gain, temp, sm_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out, int64_t t_kept,
                            const float* kept_b, const int32_t* kept_pos, const int32_t* kept_cu,
                            int n_seq, int max_len, int hq, int hkv, int dh, const float* gain,
                            const float* temp, float sm_scale, hipStream_t st) {
  (void)max_len;
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / sqrtf((float)dh);
  const int G = hq / hkv;
  const int hpw = G >= 4 ? 4 : G;
#define TG_ATTN(DHv, HPWv)                                                                     \
  if (dh == DHv && hpw == HPWv)                                                                \
    return launch_cfg<DHv, HPWv>(q, k, v, out, t_kept, kept_b, kept_pos, kept_cu, n_seq, hq, \
                                 hkv, gain, temp, sm_scale, st);
  TG_ATTN(128, 1) TG_ATTN(128, 2) TG_ATTN(128, 4)
  TG_ATTN(64, 1) TG_ATTN(64, 2) TG_ATTN(64, 4)
#undef TG_ATTN
  return hipErrorInvalidValue;
}

}  // namespace tg
