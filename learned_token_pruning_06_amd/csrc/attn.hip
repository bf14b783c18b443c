// tg_gated_attn, bf16 on matrix cores (TokenGate §4.2, Eq. 8 with the
// head-wise gain of Eq. 6 and the temperature of Eq. 7):
//
//   logit_ij = tau_i * (s * q_i.k_j + gain_h * b_j),  tau_i = temp_h * log m_i / log max(2, p_i)
//
// Flash-style causal attention over the kept tokens of each sequence.
// In the log2 domain the logit is c_i * (q_i.k_j + beta_j) with
//   c_i = tau_i * s * log2(e)   (one scalar per query row, > 0)
//   beta_j = gain_h * b_j / s   (one scalar per key and head).
// beta rides in the matrix product itself: each staged K row carries 16
// extra bf16 columns holding beta_j split into a high and a low bf16 part
// for each head, and the query side multiplies them by a constant selector
// vector, so one extra MFMA K-step adds beta_j to q.k exactly (to ~2^-17
// relative).  The temperature folds into the single FMA that forms the
// exponent, p = exp2(c_i * acc - m_i); because c_i > 0 the running maximum
// is taken on the unscaled accumulator.
//
// Work decomposition (wave64, gfx950 v_mfma_f32_32x32x16_bf16):
//  - a workgroup of 8 waves owns one block of query rows of one sequence and
//    HPW query heads that share one KV head (GQA): every K/V tile staged in
//    LDS feeds all HPW heads; two waves per SIMD;
//  - a wave owns 32 query rows of one head.  It computes S^T = K.Q^T (keys
//    on the MFMA M axis, queries on N), so each lane holds one query's
//    logits: the softmax statistics are per-lane scalars plus one swap
//    between the two lane halves (v_permlane32_swap);
//  - P^T from the accumulators is directly the B operand of O^T = V^T.P^T
//    with keys permuted consistently between the two operands; V is
//    transposed into LDS ([d][key]) in that permuted key order, so each lane
//    reads its 8 keys with one 16-byte load;
//  - the softmax normaliser sums the bf16-rounded probabilities that enter
//    the P.V product (v_dot2 against (1, 1)), so numerator and denominator
//    carry the same weights;
//  - K/V/bias tiles are double-buffered in LDS: tile t+1 is fetched from HBM
//    into registers (buffer loads whose range ends at the sequence's last
//    row, so a partial last tile reads zeros) while tile t is computed;
//  - causal masking runs only on diagonal tiles, tiles past a wave's rows
//    are skipped, query blocks are issued longest first, and the blocks of
//    one KV head share an XCD (blocks are dealt round-robin over the 8 XCDs,
//    so the head index is taken from the low bits of the block index);
//  - the running maximum is only moved when it grows by more than 2^8 in
//    the exponent (exact: the normaliser absorbs the stale maximum).
#include <type_traits>

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
constexpr int NBUF = 2;                 // LDS tile buffers
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr float kMinScale = 1e-30f;     // keeps c_i > 0 so masked keys stay -inf

TG_DEVINL bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

TG_DEVINL uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// IEEE maximum (NaN-propagating): needs no input canonicalisation and maps
// onto v_maximum3_f32
TG_DEVINL float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// v_permlane32_swap on two copies of x leaves {x[l], x[l ^ 32]} in every
// lane l, one in each register.  Written in asm because the compiler's
// builtin for it hands back the first result for both.
TG_DEVINL void half_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
TG_DEVINL float half_swap_max(float x) {
  float a = x, b = x;
  half_swap(a, b);
  return __builtin_elementwise_maximum(a, b);
}
TG_DEVINL float half_swap_sum(float x) {
  float a = x, b = x;
  half_swap(a, b);
  return a + b;
}

// sum of the two bf16 halves of w, accumulated in fp32
TG_DEVINL float dot2_ones(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// raw buffer resource over [base, base + bytes): loads past the end return 0
TG_DEVINL __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
TG_DEVINL u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
TG_DEVINL float buf_ldf(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// position of key k of a tile in a V^T row: inside each group of 16 keys the
// blocks [4..7] and [8..11] are swapped, so that the 8 keys one lane needs
// for an MFMA K-step (16kk + 8(e/4) + 4g + e%4, e < 8) are contiguous
TG_DEVINL int vpos(int k) {
  const int r = k & 15;
  return (k & ~15) | (r < 4 || r >= 12 ? r : (r < 8 ? r + 4 : r - 4));
}

template <int DH, int HPW>
struct AttnCfg {
  static constexpr int QB = NWAVE * QW / HPW;    // query rows per workgroup
  static constexpr int KROW = DH + 24;           // K row: DH values, 16 bias columns, 8 pad
  static constexpr int VROW = BKV + 8;           // V^T row: 64 keys, 8 pad
  static constexpr int KT = DH / 16;             // MFMA K-steps over the head dim
  static constexpr int DT = DH / 32;             // output tiles over the head dim
  static constexpr int KVEC = BKV * DH / 8;      // 16-byte vectors per K tile
  static constexpr int KVPT = (KVEC + NTHR - 1) / NTHR;
  static constexpr int VUNITS = (BKV / 2) * (DH / 8);   // (2-key pair, 8-dim chunk) units
  static constexpr int KTILE = BKV * KROW;       // bf16 per K buffer
  static constexpr int VTILE = DH * VROW;        // bf16 per V^T buffer
};

template <int DH, int HPW>
__global__ __launch_bounds__(NTHR) void gated_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ kept_cu, int n_seq,
    int t_kept, int hq, int hkv, int groups_y, int n_slots, const float* __restrict__ gain,
    const float* __restrict__ temp, float sm_scale) {
  using C = AttnCfg<DH, HPW>;
  static_assert(C::KVPT <= 2 && C::VUNITS <= NTHR, "loader shape");
  __shared__ __attribute__((aligned(16))) uint16_t sk[NBUF * C::KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv[NBUF * C::VTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;

  // ---- block -> (head group, sequence, query block); head group from the
  // low bits (one XCD per KV head), query slots last-first (longest first)
  const int n_hg = hkv * groups_y;
  const int hg = (int)(blockIdx.x % (unsigned)n_hg);
  const int64_t slot = (int64_t)n_slots - 1 - (int64_t)(blockIdx.x / (unsigned)n_hg);
  const int s = seq_of_slot(kept_cu, n_seq, slot, C::QB);
  if (s < 0) return;
  // rows are clamped to [0, t_kept): inconsistent offsets cannot read out of bounds
  const int lo = kept_cu[s] < t_kept ? kept_cu[s] : t_kept;
  const int len = (kept_cu[s + 1] < t_kept ? kept_cu[s + 1] : t_kept) - lo;
  const int q0 = (int)(slot - slot0_of(kept_cu, s, C::QB)) * C::QB;
  if (q0 >= len) return;

  const int G = hq / hkv;
  const int kvh = hg / groups_y;
  const int hbase = kvh * G + (hg % groups_y) * HPW;
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

  // ---- Q fragments (B operand of S^T = K.Q^T): lane holds q[row][16kk + 8g .. +8],
  // plus the selector of this head's two bias columns (16 extra columns, lane half 0)
  bf16x8 qf[C::KT];
  {
    const int a = qvalid ? qa : len - 1;
    const uint16_t* qp = q + ((int64_t)(lo + a) * hq + head) * DH;
#pragma unroll
    for (int kk = 0; kk < C::KT; ++kk) qf[kk] = as_bf16x8(ld16(qp + 16 * kk + 8 * g));
  }
  bf16x8 qsel;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    qsel[e] = (__bf16)((g == 0 && (e >> 1) == hl) ? 1.0f : 0.0f);

  // ---- tile loaders (global -> registers -> LDS), per-thread state fixed up front
  const int q_end = q0 + C::QB < len ? q0 + C::QB : len;
  const int n_tiles = (q_end + BKV - 1) / BKV;
  const int64_t kvstride = (int64_t)hkv * DH;     // elements between token rows of k, v
  const uint16_t* kb_ = k + (int64_t)lo * kvstride + (int64_t)kvh * DH;
  const uint16_t* vb_ = v + (int64_t)lo * kvstride + (int64_t)kvh * DH;
  // K: vectors tid and tid + NTHR of the tile (row key, 16-byte chunk ch)
  const int kvi0 = tid % C::KVEC, kvi1 = (tid + NTHR) % C::KVEC;
  const int krow0 = kvi0 / (DH / 8), krow1 = kvi1 / (DH / 8);
  const int kcol0 = 8 * (kvi0 % (DH / 8)), kcol1 = 8 * (kvi1 % (DH / 8));
  const int kdst0 = krow0 * C::KROW + kcol0, kdst1 = krow1 * C::KROW + kcol1;
  // V: unit (key pair vkp, 8-dim chunk vdc), transposed into V^T rows 8vdc..+8
  const int vu = tid % C::VUNITS;
  const int vkp = vu % (BKV / 2), vdc = vu / (BKV / 2);
  const int vdst = (8 * vdc) * C::VROW + vpos(2 * vkp);
  float bsc[4];                                   // gain_h / s of the HPW heads
#pragma unroll
  for (int i = 0; i < 4; ++i) bsc[i] = i < HPW ? gain[hbase + i] / sm_scale : 0.0f;

  // per-thread byte offsets inside a tile (rows of k and v are kvstride apart)
  const int koff0 = (krow0 * (int)kvstride + kcol0) * 2;
  const int koff1 = (krow1 * (int)kvstride + kcol1) * 2;
  const int voff0 = ((2 * vkp) * (int)kvstride + 8 * vdc) * 2;
  const int voff1 = voff0 + (int)kvstride * 2;
  const int boff = (tid % BKV) * 4;

  u32x4 kreg0 = {0u, 0u, 0u, 0u}, kreg1 = {0u, 0u, 0u, 0u};
  u32x4 vreg0 = {0u, 0u, 0u, 0u}, vreg1 = {0u, 0u, 0u, 0u};
  float breg = 0.f;

  auto load_tile = [&](int t) {
    const int kv0 = t * BKV;
    const int rows = len - kv0 < BKV ? len - kv0 : BKV;      // rows of this tile in the sequence
    const int64_t off = (int64_t)kv0 * kvstride;
    const int bytes = rows * (int)kvstride * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb_ + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb_ + off, bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(kept_b + lo + kv0, rows * 4);
    kreg0 = buf_ld16(rk, koff0);
    if (C::KVPT == 2) kreg1 = buf_ld16(rk, koff1);
    vreg0 = buf_ld16(rv, voff0);
    vreg1 = buf_ld16(rv, voff1);
    breg = buf_ldf(rb, boff);
  };
  auto store_tile = [&](auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    uint16_t* skb = sk + BUF * C::KTILE;
    uint16_t* svb = sv + BUF * C::VTILE;
    if (tid < C::KVEC) st16(&skb[kdst0], kreg0);
    if (C::KVPT == 2 && tid + NTHR < C::KVEC) st16(&skb[kdst1], kreg1);
    if (tid < C::VUNITS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a0 = vreg0[e >> 1], a1 = vreg1[e >> 1];
        const uint32_t pk = (e & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u))
                                    : ((a0 & 0xffffu) | (a1 << 16));
        *reinterpret_cast<uint32_t*>(&svb[vdst + e * C::VROW]) = pk;
      }
    }
    if (tid < BKV) {
      // bias columns of key tid: (hi, lo) bf16 parts of gain_h * b / s per head
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float beta = breg * bsc[i];
        const float hi = (float)(__bf16)beta;
        w[i] = i < HPW ? pack_bf16x2(hi, beta - hi) : 0u;
      }
      st16(&skb[tid * C::KROW + DH], (u32x4){w[0], w[1], w[2], w[3]});
      st16(&skb[tid * C::KROW + DH + 8], (u32x4){0u, 0u, 0u, 0u});
    }
  };

  // per-lane LDS operand bases: every fragment read is base + constant offset
  const uint16_t* klane = sk + n * C::KROW + 8 * g;
  const uint16_t* vlane = sv + n * C::VROW + 8 * g;

  // ---- running state (one query per lane)
  floatx16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float mrun = -INFINITY;
  float negm = 0.f;                              // -mrun, 0 while mrun is -inf
  float lsum = 0.f;
  const int wq_last = wq0 + QW - 1 < len - 1 ? wq0 + QW - 1 : len - 1;
  const int w_tiles = wq0 < len ? wq_last / BKV + 1 : 0;   // tiles this wave needs

  // one tile of one wave: S^T = K'.Q'^T (bias step first), softmax, O^T += V^T.P^T
  auto compute = [&](auto BUFC, int t) {
    constexpr int BUF = decltype(BUFC)::value;
    const int kv0 = t * BKV;
    const uint16_t* kl = klane + BUF * C::KTILE;
    const uint16_t* vl = vlane + BUF * C::VTILE;
    const floatx16 zero = {};
    floatx16 sc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(kl + DH)), qsel, zero,
                                                           0, 0, 0);
    floatx16 sc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        as_bf16x8(ld16(kl + 32 * C::KROW + DH)), qsel, zero, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < C::KT; ++kk) {
      sc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(kl + 16 * kk)), qf[kk], sc0,
                                                    0, 0, 0);
      sc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          as_bf16x8(ld16(kl + 32 * C::KROW + 16 * kk)), qf[kk], sc1, 0, 0, 0);
    }
    // causal mask, only where the tile reaches past the wave's first row:
    // key 8(r/4) + 4g + r%4 (+32 for sc1) of the tile is masked when it lies
    // past this lane's query
    if (kv0 + BKV - 1 > wq0) {
      const int dq = qa - kv0 - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + (r & 3);
        sc0[r] = kr > dq ? -INFINITY : sc0[r];
        sc1[r] = kr + 32 > dq ? -INFINITY : sc1[r];
      }
    }
    // online softmax on the unscaled accumulator (c_i > 0)
    float ma = fmax3(sc0[0], sc0[1], sc0[2]);
    float mb = fmax3(sc1[0], sc1[1], sc1[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = fmax3(ma, sc0[r], sc0[r + 1]);
      mb = fmax3(mb, sc1[r], sc1[r + 1]);
    }
    const float mx = half_swap_max(fmax3(ma, mb, __builtin_elementwise_maximum(sc0[15], sc1[15])))
                     * cq;
    if (__any(mx > mrun + kRescaleSlack)) {
      const float mnew = __builtin_elementwise_maximum(mrun, mx);
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      mrun = mnew;
      negm = mnew == -INFINITY ? 0.0f : -mnew;
    }
    // p = exp2(c * acc - m), rounded to bf16 as P^T, the B operand of
    // O^T = V^T.P^T: K-step kk holds keys 16kk + 8(e/4) + 4g + e%4, i.e.
    // registers 8(kk%2) .. +8 of tile kk/2
    uint32_t pw[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pw[i] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc0[2 * i], cq, negm)),
                          __builtin_amdgcn_exp2f(fmaf(sc0[2 * i + 1], cq, negm)));
      pw[8 + i] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc1[2 * i], cq, negm)),
                              __builtin_amdgcn_exp2f(fmaf(sc1[2 * i + 1], cq, negm)));
    }
    float la = dot2_ones(pw[0], lsum), lb = dot2_ones(pw[1], 0.0f);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      la = dot2_ones(pw[i], la);
      lb = dot2_ones(pw[i + 1], lb);
    }
    lsum = la + lb;
    bf16x8 pf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      pf[kk] = as_bf16x8((u32x4){pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]});
    // O^T += V^T . P^T  (A operand: V^T row d = 32dt + n, 8 permuted keys)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = as_bf16x8(ld16(vl + 32 * dt * C::VROW + 16 * kk));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], oacc[dt], 0, 0, 0);
      }
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  load_tile(0);
  store_tile(B0{});
  __syncthreads();
  // double-buffered tiles, unrolled by two so every LDS offset is a constant
  for (int t = 0; t < n_tiles; t += 2) {
    if (t + 1 < n_tiles) load_tile(t + 1);
    if (t < w_tiles) compute(B0{}, t);
    if (t + 1 < n_tiles) store_tile(B1{});
    __syncthreads();
    if (t + 1 >= n_tiles) break;
    if (t + 2 < n_tiles) load_tile(t + 2);
    if (t + 1 < w_tiles) compute(B1{}, t + 1);
    if (t + 2 < n_tiles) store_tile(B0{});
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, one query per lane; d = 32dt + 8(r/4) + 4g + r%4
  const float lt = half_swap_sum(lsum);
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
  const int64_t n_slots = n_seq + (t_kept + QB - 1) / QB;
  const int64_t blocks = n_slots * hkv * groups_y;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gated_attn_bf16<DH, HPW>), dim3((unsigned)blocks), dim3(NTHR), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), kept_b, kept_pos,
                     kept_cu, n_seq, (int)t_kept, hq, hkv, groups_y, (int)n_slots, gain, temp,
                     sm_scale);
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
