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
//  - P^T from the accumulators is directly the B operand of O^T = V^T.P^T;
//    the keys of P^T's K-steps come in runs of four, and V stays row-major
//    in LDS: two transposing reads (ds_read_b64_tr_b16) hand each lane the
//    two runs of four keys of its head dimension;
//  - the softmax normaliser sums the bf16-rounded probabilities that enter
//    the P.V product (v_dot2 against (1, 1)), so numerator and denominator
//    carry the same weights;
//  - K/V/bias tiles rotate through three LDS buffers: tile t+1 is fetched
//    from HBM into registers (buffer loads whose range ends at the
//    sequence's last row, so a partial last tile reads zeros) while tile t
//    is computed;
//  - the two waves that share a SIMD run half a tile apart (one does
//    S then P.V of tile t, the other P.V of tile t-1 then S of tile t), so
//    the matrix products of one overlap the softmax of the other;
//  - inside a phase the instruction order is pinned with scheduling
//    barriers so that LDS operand reads run four MFMAs ahead of their use;
//  - workgroups are persistent (one per CU): the workgroups of one head
//    group take its query blocks longest first in snake order, which
//    balances the causal triangle; the blocks of one KV head share an XCD
//    (workgroups are dealt round-robin over the 8 XCDs, so the head group is
//    taken from the low bits of the workgroup index);
//  - causal masking runs only on diagonal tiles and tiles past a wave's rows
//    are skipped;
//  - the running maximum is only moved when it grows by more than 2^8 in
//    the exponent (exact: the normaliser absorbs the stale maximum).
#include <type_traits>

#include "common.h"


namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int BKV = 64;                 // keys per tile
constexpr int kAttnWaves = 8;           // waves per workgroup (two per SIMD)
constexpr int QW = 32;                  // query rows per wave
constexpr int NBUF = 3;                 // LDS tile buffers
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

template <int DH, int HPW, int NWAVE>
struct AttnCfg {
  static constexpr int NTHR = 64 * NWAVE;        // threads per workgroup
  static constexpr int QB = NWAVE * QW / HPW;    // query rows per workgroup
  static constexpr int KROW = DH + 24;           // K row: DH values, 16 bias columns, 8 pad
  static constexpr int VROW = DH + 16;           // V row: DH values, 16 pad (rows 32 B apart mod 256 B)
  static constexpr int KT = DH / 16;             // MFMA K-steps over the head dim
  static constexpr int DT = DH / 32;             // output tiles over the head dim
  static constexpr int KVEC = BKV * DH / 8;      // 16-byte vectors per K tile
  static constexpr int KVPT = (KVEC + NTHR - 1) / NTHR;
  static constexpr int VVPT = (KVEC + NTHR - 1) / NTHR;  // V: same 16-byte vectors as K
  static constexpr int KTILE = BKV * KROW;       // bf16 per K buffer
  static constexpr int VTILE = BKV * VROW;       // bf16 per V buffer (row-major)
};

template <int DH, int HPW, int NWAVE>
__device__ __forceinline__ void gated_attn_item(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ kept_cu, int n_seq,
    int t_kept, int hq, int hkv, int groups_y, int hg, int64_t slot,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm_scale,
    float* __restrict__ lse2, uint16_t* sk, uint16_t* sv) {
  using C = AttnCfg<DH, HPW, NWAVE>;
  constexpr int NTHR = C::NTHR;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
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
  float bsc[4];                                   // gain_h / s of the HPW heads
#pragma unroll
  for (int i = 0; i < 4; ++i) bsc[i] = i < HPW ? gain[hbase + i] / sm_scale : 0.0f;

  // K and V: 16-byte vectors tid + i*NTHR of the tile (row, 8-element
  // chunk), to LDS row-major with their padded row strides.  Offsets in
  // global memory are bytes from the tile's first row (rows of k and v are
  // kvstride elements apart).
  int koff[C::KVPT], kdst[C::KVPT], vdst[C::KVPT];
#pragma unroll
  for (int i = 0; i < C::KVPT; ++i) {
    const int kvi = (tid + i * NTHR) % C::KVEC;
    const int row = kvi / (DH / 8), col = 8 * (kvi % (DH / 8));
    koff[i] = (row * (int)kvstride + col) * 2;
    kdst[i] = row * C::KROW + col;
    vdst[i] = row * C::VROW + col;
  }
  const int boff = (tid % BKV) * 4;

  u32x4 kreg[C::KVPT], vreg[C::KVPT];
  float breg = 0.f;

  auto load_tile = [&](int t) {
    const int kv0 = t * BKV;
    const int rows = len - kv0 < BKV ? len - kv0 : BKV;      // rows of this tile in the sequence
    const int64_t off = (int64_t)kv0 * kvstride;
    const int bytes = rows * (int)kvstride * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb_ + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb_ + off, bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(kept_b + lo + kv0, rows * 4);
#pragma unroll
    for (int i = 0; i < C::KVPT; ++i)
      if (C::KVEC % NTHR == 0 || tid + i * NTHR < C::KVEC) kreg[i] = buf_ld16(rk, koff[i]);
#pragma unroll
    for (int i = 0; i < C::KVPT; ++i)
      if (C::KVEC % NTHR == 0 || tid + i * NTHR < C::KVEC) vreg[i] = buf_ld16(rv, koff[i]);
    breg = buf_ldf(rb, boff);
  };
  auto store_tile = [&](auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    uint16_t* skb = sk + BUF * C::KTILE;
    uint16_t* svb = sv + BUF * C::VTILE;
#pragma unroll
    for (int i = 0; i < C::KVPT; ++i)
      if (C::KVEC % NTHR == 0 || tid + i * NTHR < C::KVEC) st16(&skb[kdst[i]], kreg[i]);
#pragma unroll
    for (int i = 0; i < C::KVPT; ++i)
      if (C::KVEC % NTHR == 0 || tid + i * NTHR < C::KVEC) st16(&svb[vdst[i]], vreg[i]);
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
  // V fragments by transposing reads: within each 16-lane group, lane s
  // points at row 4kg + s/4 (kg = lane/32), columns 16((lane/16)%2) + 4(s%4)
  // .. +4; the read hands lane i of the group the 4 keys of that row block
  // at column 16((lane/16)%2) + i, i.e. the A operand of dim lane%32
  const uint16_t* vlane =
      sv + (4 * (lane >> 5) + ((lane & 15) >> 2)) * C::VROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

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

  // Phase S of one tile of one wave: S^T = K'.Q'^T (bias step first), mask,
  // running maximum and the probabilities P^T as bf16 words in pw.  The
  // instruction order is fixed by scheduling barriers: K fragment reads run
  // four MFMAs ahead of their use.
  uint32_t pw[16];
  auto phase_s = [&](auto BUFC, int t) {
    constexpr int BUF = decltype(BUFC)::value;
    const int kv0 = t * BKV;
    const uint16_t* kl = klane + BUF * C::KTILE;
    // K fragment j of the tile: key half j & 1, K-step (j >> 1) - 1 (-1: bias columns)
    auto kfrag = [&](int j) {
      const int st = (j >> 1) - 1;
      return ld16(kl + 32 * (j & 1) * C::KROW + (st < 0 ? DH : 16 * st));
    };
    constexpr int NK = 2 * (C::KT + 1);          // MFMAs of S^T
    u32x4 kr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kr[j] = kfrag(j);
    __builtin_amdgcn_sched_barrier(0);
    floatx16 sc[2];
    const floatx16 zero = {};
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const bf16x8 bop = j < 2 ? qsel : qf[(j >> 1) - 1];
      sc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[j % 4]), bop,
                                                          j < 2 ? zero : sc[j & 1], 0, 0, 0);
      if (j + 4 < NK) kr[j % 4] = kfrag(j + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    // causal mask, only where the tile reaches past the wave's first row:
    // key 8(r/4) + 4g + r%4 (+32 for sc[1]) of the tile is masked when it
    // lies past this lane's query
    if (kv0 + BKV - 1 > wq0) {
      const int dq = qa - kv0 - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr_ = 8 * (r >> 2) + (r & 3);
        sc[0][r] = kr_ > dq ? -INFINITY : sc[0][r];
        sc[1][r] = kr_ + 32 > dq ? -INFINITY : sc[1][r];
      }
    }
    // online softmax on the unscaled accumulator (c_i > 0)
    float ma = fmax3(sc[0][0], sc[0][1], sc[0][2]);
    float mb = fmax3(sc[1][0], sc[1][1], sc[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = fmax3(ma, sc[0][r], sc[0][r + 1]);
      mb = fmax3(mb, sc[1][r], sc[1][r + 1]);
    }
    const float mx =
        half_swap_max(fmax3(ma, mb, __builtin_elementwise_maximum(sc[0][15], sc[1][15]))) * cq;
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
    // registers 8(kk%2) .. +8 of sc[kk/2]; word w of group kk packs the
    // pair 2w, 2w+1 of those eight
    float la = lsum, lb = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const floatx16& sa = sc[kk >> 1];
        const int o = 8 * (kk & 1) + 2 * w;
        pw[4 * kk + w] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sa[o], cq, negm)),
                                     __builtin_amdgcn_exp2f(fmaf(sa[o + 1], cq, negm)));
        if (w & 1)
          lb = dot2_ones(pw[4 * kk + w], lb);
        else
          la = dot2_ones(pw[4 * kk + w], la);
      }
    lsum = la + lb;
  };

  // O^T += V^T . P^T for the tile in buffer BUF and the P^T words in pw
  // (A operand: dim 32dt + n, the 8 keys of K-step kk in P^T's order); the
  // V reads run four MFMAs ahead of their use
  auto phase_pv = [&](auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    const uint16_t* vl = vlane + BUF * C::VTILE;
    // keys 16kk + 4kg + 0..3 and 16kk + 8 + 4kg + 0..3 of dims 32dt + lane%32
    auto vfrag = [&](int i) {
      const uint16_t* p = vl + 16 * (i / C::DT) * C::VROW + 32 * (i % C::DT);
      const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(p));
      const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(p + 8 * C::VROW));
      const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
      return (u32x4){ua.x, ua.y, ub.x, ub.y};
    };
    constexpr int NV = 4 * C::DT;
    u32x4 vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = vfrag(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int kk = i / C::DT, dt = i % C::DT;
      const bf16x8 pf = as_bf16x8((u32x4){pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2],
                                          pw[4 * kk + 3]});
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vr[i % 4]), pf, oacc[dt], 0, 0,
                                                         0);
      if (i + 4 < NV) vr[i % 4] = vfrag(i + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tiles rotate through three LDS buffers; iteration t computes tile t while
  // tile t+1 is fetched and stored.  The two waves that share a SIMD work
  // half a tile apart: waves 0..3 run S(t) then P.V(t), waves 4..7 run
  // P.V(t-1) then S(t), so one wave's matrix products overlap the other's
  // softmax instead of both contending for the matrix core at once.
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  const bool lag = wv >= NWAVE / 2;
  load_tile(0);
  store_tile(B0{});
  __syncthreads();
  auto step = [&](auto BC, auto BP, auto BN, int t) {
    if (t + 1 < n_tiles) load_tile(t + 1);
    if (!lag) {
      if (t < w_tiles) {
        phase_s(BC, t);
        phase_pv(BC);
      }
    } else {
      if (t >= 1 && t - 1 < w_tiles) phase_pv(BP);
      if (t < w_tiles) phase_s(BC, t);
    }
    if (t + 1 < n_tiles) store_tile(BN);
    __syncthreads();
  };
  int t = 0;
  for (; t < n_tiles; t += 3) {
    step(B0{}, B2{}, B1{}, t);
    if (t + 1 >= n_tiles) {
      t += 1;
      break;
    }
    step(B1{}, B0{}, B2{}, t + 1);
    if (t + 2 >= n_tiles) {
      t += 2;
      break;
    }
    step(B2{}, B1{}, B0{}, t + 2);
  }
  // t == n_tiles here; the lagging waves still owe P.V of the last tile
  if (lag && n_tiles - 1 < w_tiles) {
    const int bl = (n_tiles - 1) % 3;
    if (bl == 0)
      phase_pv(B0{});
    else if (bl == 1)
      phase_pv(B1{});
    else
      phase_pv(B2{});
  }

  // ---- epilogue: O = O^T / l, one query per lane; d = 32dt + 8(r/4) + 4g + r%4
  const float lt = half_swap_sum(lsum);
  if (!qvalid) return;
  const float inv = 1.0f / lt;
  // optional row statistic for the backward: log2 sum_j exp2(c_i acc_ij), in
  // the units of the exponent, head-major [hq][t_kept] so the 32 queries of
  // a wave store 128 contiguous bytes (both lane halves hold it; the first
  // stores)
  if (lse2 && g == 0) lse2[(int64_t)head * t_kept + lo + qa] = mrun + __log2f(lt);
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

// two waves per SIMD: at most 256 registers per lane
template <int DH, int HPW, int NWAVE>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(2)))
void gated_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ kept_cu, int n_seq,
    int t_kept, int hq, int hkv, int groups_y, int n_slots, const float* __restrict__ gain,
    const float* __restrict__ temp, float sm_scale, float* __restrict__ lse2) {
  using C = AttnCfg<DH, HPW, NWAVE>;
  static_assert(NWAVE % HPW == 0 && C::NTHR >= BKV, "workgroup shape");
  __shared__ __attribute__((aligned(16))) uint16_t sk[NBUF * C::KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sv[NBUF * C::VTILE];

  // ---- persistent workgroups: the head group comes from the low bits of the
  // block index (blocks are dealt round-robin over the 8 XCDs, so the blocks
  // of one KV head share an XCD and its L2); the pj blocks of a head group
  // take its query slots last-first (longest first under the causal mask)
  // in snake order, so every block gets a long and a short slot per pair of
  // rounds
  const int n_hg = hkv * groups_y;
  const int hg = (int)(blockIdx.x % (unsigned)n_hg);
  const int jb = (int)(blockIdx.x / (unsigned)n_hg);
  const int pj = (int)(gridDim.x / (unsigned)n_hg);
  // slots past the last query block of the last sequence hold no work: rank
  // from the last real one
  int64_t n_real = n_slots;
  if (n_seq > 0) {
    const int last_lo = kept_cu[n_seq - 1] < t_kept ? kept_cu[n_seq - 1] : t_kept;
    const int last_hi = kept_cu[n_seq] < t_kept ? kept_cu[n_seq] : t_kept;
    const int last_len = last_hi > last_lo ? last_hi - last_lo : 0;
    const int64_t end = slot0_of(kept_cu, n_seq - 1, C::QB) + (last_len + C::QB - 1) / C::QB;
    if (end >= 0 && end < n_real) n_real = end;
  }
  for (int64_t round = 0;; ++round) {
    const int64_t rank = round * pj + ((round & 1) ? pj - 1 - jb : jb);
    if (rank >= n_real) break;
    gated_attn_item<DH, HPW, NWAVE>(q, k, v, out, kept_b, kept_pos, kept_cu, n_seq, t_kept, hq,
                                    hkv, groups_y, hg, n_real - 1 - rank, gain, temp, sm_scale,
                                    lse2, sk, sv);
    __syncthreads();                               // LDS buffers are reused by the next slot
  }
}

template <int DH, int HPW, int NWAVE>
hipError_t launch_cfg(const void* q, const void* k, const void* v, void* out, int64_t t_kept,
                      const float* kept_b, const int32_t* kept_pos, const int32_t* kept_cu,
                      int n_seq, int hq, int hkv, const float* gain, const float* temp,
                      float sm_scale, float* lse2, hipStream_t st) {
  constexpr int QB = AttnCfg<DH, HPW, NWAVE>::QB;
  const int G = hq / hkv;
  const int groups_y = G / HPW;
  const int64_t n_slots = n_seq + (t_kept + QB - 1) / QB;
  const int n_hg = hkv * groups_y;
  // persistent grid: one workgroup per CU (the register budget allows one),
  // the same number for every head group
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  int64_t pj = n_cu / n_hg;
  if (pj < 1) pj = 1;
  if (pj > n_slots) pj = n_slots;
  const int64_t blocks = (int64_t)n_hg * pj;
  if (n_slots > 0x7fffffff || blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gated_attn_bf16<DH, HPW, NWAVE>), dim3((unsigned)blocks), dim3(64 * NWAVE), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), kept_b, kept_pos,
                     kept_cu, n_seq, (int)t_kept, hq, hkv, groups_y, (int)n_slots, gain, temp,
                     sm_scale, lse2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out, int64_t t_kept,
                            const float* kept_b, const int32_t* kept_pos, const int32_t* kept_cu,
                            int n_seq, int max_len, int hq, int hkv, int dh, const float* gain,
                            const float* temp, float sm_scale, float* lse2, hipStream_t st) {
  (void)max_len;
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / sqrtf((float)dh);
  const int G = hq / hkv;
  const int hpw = G >= 4 ? 4 : G;
#define TG_ATTN(DHv, HPWv)                                                                     \
  if (dh == DHv && hpw == HPWv)                                                                \
    return launch_cfg<DHv, HPWv, kAttnWaves>(q, k, v, out, t_kept, kept_b, kept_pos, kept_cu, n_seq, hq, \
                                 hkv, gain, temp, sm_scale, lse2, st);
  TG_ATTN(128, 1) TG_ATTN(128, 2) TG_ATTN(128, 4)
  TG_ATTN(64, 1) TG_ATTN(64, 2) TG_ATTN(64, 4)
#undef TG_ATTN
  return hipErrorInvalidValue;
}

}  // namespace tg
