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
//  - K/V tiles rotate through three LDS buffers (one LDS array each): tile
//    t+1 goes from HBM straight into the LDS (buffer loads that write the
//    LDS, whose range ends at the sequence's last row, so a partial last
//    tile reads zeros) while tile t is computed; rows are 2*DH bytes with
//    their 16-byte chunks permuted per row (XOR swizzle), so the operand
//    reads hit distinct banks without padding.  The keys' bias columns sit
//    in a small array of their own, written from registers;
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
//
// tg_gated_attn_split (the SPLIT instance of the same kernel, for short or
// ragged inputs): a one-workgroup launch (attn_plan) lists the query
// blocks, cuts the ones with more key tiles than a workgroup's share of
// the causal work into key chunks, and sorts all items by size, largest
// first; the attention deals that list to the workgroups in the same snake
// order; each chunk leaves a bf16 partial output with its f32 maximum and
// sum, and attn_merge combines the chunks of each split block.
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
TG_DEVINL float buf_ldf(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <int DH, int HPW, int NWAVE>
struct AttnCfg {
  static constexpr int NTHR = 64 * NWAVE;        // threads per workgroup
  static constexpr int QB = NWAVE * QW / HPW;    // query rows per workgroup
  static constexpr int KROW = DH;                // K row: DH values (bias columns apart)
  static constexpr int VROW = DH;                // V row: DH values
  static constexpr int KT = DH / 16;             // MFMA K-steps over the head dim
  static constexpr int DT = DH / 32;             // output tiles over the head dim
  static constexpr int KTILE = BKV * KROW;       // bf16 per K buffer
  static constexpr int VTILE = BKV * VROW;       // bf16 per V buffer
  static constexpr int BTILE = BKV * 16;         // bf16 per bias buffer (16 per key)
  static constexpr int CPR = DH / 8;             // 16-byte chunks per row
  static constexpr int RPB = 1024 / (2 * DH);    // rows per 1 KB DMA block
  static constexpr int RW = 256 / (2 * DH);      // rows per 256 B of LDS
  static constexpr int NBLK = BKV / RPB;         // DMA blocks per tile
  static constexpr int KDMA = NBLK / NWAVE;      // DMA instructions per wave and tile, each of K and V
  // Logical 16-byte chunk c of row r is stored at chunk c ^ fk(r) (K) or
  // c ^ fv(r) (V).  The LDS serves 256 B per cycle.  A K read (16 bytes per
  // lane) has 16 lanes on 16 rows at one chunk: fk spreads them over the 16
  // chunk slots of 256 B.  A V read (transposing, 8 bytes per lane) has 32
  // lanes on 4 rows at chunks 4dt + 0..3: fv moves each of the 4 rows to
  // its own group of 4 chunks.
  static __device__ __forceinline__ int fk(int r) { return (r / RW) & (CPR - 1); }
  static __device__ __forceinline__ int fv(int r) { return 4 * ((r / RW) & (CPR / 4 - 1)); }
};

template <int DH, int HPW, int NWAVE, bool SPLIT>
__device__ __forceinline__ void gated_attn_item(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ kept_cu, int n_seq,
    int t_kept, int hq, int hkv, int groups_y, int hg, int64_t slot,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm_scale,
    float* __restrict__ lse2, uint16_t* sk0, uint16_t* sk1, uint16_t* sk2, uint16_t* sv0,
    uint16_t* sv1, uint16_t* sv2, uint16_t* sb, int chunk_tiles, int c_max, int chunk,
    uint16_t* __restrict__ ws_o, float2* __restrict__ ws_ml) {
  using C = AttnCfg<DH, HPW, NWAVE>;
  // one LDS array per buffer, so that reads of one buffer need not wait for
  // the DMA into another
  auto kbuf = [&](auto BUFC) {
    constexpr int B = decltype(BUFC)::value;
    return B == 0 ? sk0 : (B == 1 ? sk1 : sk2);
  };
  auto vbuf = [&](auto BUFC) {
    constexpr int B = decltype(BUFC)::value;
    return B == 0 ? sv0 : (B == 1 ? sv1 : sv2);
  };
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
  // key tiles [t_lo, t_hi) of this item: chunk `chunk` of chunk_tiles tiles
  // (the last of the c_max chunks runs to the block's end).  A block of at
  // most chunk_tiles tiles is one item and writes its output; a longer one
  // leaves partial results for attn_merge.
  const int q_end = q0 + C::QB < len ? q0 + C::QB : len;
  const int n_all = (q_end + BKV - 1) / BKV;
  int t_lo = 0, t_hi = n_all;
  bool part = false;
  if constexpr (SPLIT) {
    const int64_t t_lo64 = (int64_t)chunk * chunk_tiles;
    if (t_lo64 >= n_all) return;                 // no keys in this chunk
    t_lo = (int)t_lo64;
    t_hi = chunk == c_max - 1 || n_all - t_lo <= chunk_tiles ? n_all : t_lo + chunk_tiles;
    part = n_all > chunk_tiles;
  }
  const int n_tiles = t_hi - t_lo;

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
  const int64_t kvstride = (int64_t)hkv * DH;     // elements between token rows of k, v
  const uint16_t* kb_ = k + (int64_t)lo * kvstride + (int64_t)kvh * DH;
  const uint16_t* vb_ = v + (int64_t)lo * kvstride + (int64_t)kvh * DH;
  float bsc[4];                                   // gain_h / s of the HPW heads
#pragma unroll
  for (int i = 0; i < 4; ++i) bsc[i] = i < HPW ? gain[hbase + i] / sm_scale : 0.0f;

  // K and V tiles by DMA (buffer loads that write the LDS): instruction i of
  // a wave fills the 1 KB block b = wave + NWAVE * i of the tile, rows
  // RPB * b .. +RPB; lane l brings row RPB * b + l / CPR into physical chunk
  // l % CPR, i.e. the logical chunk that the row's swizzle puts there.
  // Offsets are bytes from the tile's first row in global memory.
  static_assert(C::NBLK % NWAVE == 0, "DMA blocks per wave");
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  int kvo[C::KDMA], vvo[C::KDMA];
#pragma unroll
  for (int i = 0; i < C::KDMA; ++i) {
    const int row = C::RPB * (wvu + NWAVE * i) + lane / C::CPR, p = lane % C::CPR;
    kvo[i] = (row * (int)kvstride + 8 * (p ^ C::fk(row))) * 2;
    vvo[i] = (row * (int)kvstride + 8 * (p ^ C::fv(row))) * 2;
  }
  const int boff = (tid % BKV) * 4;
  float breg = 0.f;

  auto load_tile = [&](int t, auto BUFC) {
    const int kv0 = t * BKV;
    const int rows = len - kv0 < BKV ? len - kv0 : BKV;      // rows of this tile in the sequence
    const int64_t off = (int64_t)kv0 * kvstride;
    const int bytes = rows * (int)kvstride * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb_ + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb_ + off, bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(kept_b + lo + kv0, rows * 4);
    uint16_t* skb = kbuf(BUFC);
    uint16_t* svb = vbuf(BUFC);
#pragma unroll
    for (int i = 0; i < C::KDMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(skb + (wvu + NWAVE * i) * 512), 16, kvo[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < C::KDMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)(svb + (wvu + NWAVE * i) * 512), 16, vvo[i], 0, 0, 0);
    breg = buf_ldf(rb, boff);
  };
  auto store_tile = [&](auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    uint16_t* sbb = sb + BUF * C::BTILE;
    if (tid < BKV) {
      // bias columns of key tid: (hi, lo) bf16 parts of gain_h * b / s per head
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float beta = breg * bsc[i];
        const float hi = (float)(__bf16)beta;
        w[i] = i < HPW ? pack_bf16x2(hi, beta - hi) : 0u;
      }
      st16(&sbb[tid * 16], (u32x4){w[0], w[1], w[2], w[3]});
      st16(&sbb[tid * 16 + 8], (u32x4){0u, 0u, 0u, 0u});
    }
  };

  // per-lane LDS operand offsets: a K read is its row's base plus the
  // swizzled chunk of its K-step, a V read the lane's column plus the
  // swizzled output tile
  const int klane = n * C::KROW;
  const uint16_t* blane = sb + n * 16 + 8 * g;
  // physical offset of the lane's K chunk 2 st + g (the row's swizzle; rows
  // n and n + 32 share it)
  int kcol[C::KT];
#pragma unroll
  for (int st = 0; st < C::KT; ++st) kcol[st] = 8 * ((2 * st + g) ^ C::fk(n));
  // V fragments by transposing reads: within each 16-lane group, lane s
  // points at row 4kg + s/4 (kg = lane/32), columns 16((lane/16)%2) + 4(s%4)
  // .. +4; the read hands lane i of the group the 4 keys of that row block
  // at column 16((lane/16)%2) + i, i.e. the A operand of dim lane%32
  const int vrow = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int vlane = vrow * C::VROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // column of output tile dt in the lane's rows (16kk and 8 keep the swizzle)
  int vcol[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) vcol[dt] = 32 * (dt ^ (C::fv(vrow) >> 2));

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
    const uint16_t* kl = kbuf(BUFC) + klane;
    const uint16_t* bl = blane + BUF * C::BTILE;
    // K fragment j of the tile: key half j & 1, K-step (j >> 1) - 1 (-1: bias columns)
    auto kfrag = [&](int j) {
      const int st = (j >> 1) - 1;
      return st < 0 ? ld16(bl + 32 * (j & 1) * 16) : ld16(kl + 32 * (j & 1) * C::KROW + kcol[st < 0 ? 0 : st]);
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
    const uint16_t* vl = vbuf(BUFC) + vlane;
    // keys 16kk + 4kg + 0..3 and 16kk + 8 + 4kg + 0..3 of dims 32dt + lane%32
    auto vfrag = [&](int i) {
      const uint16_t* p = vl + 16 * (i / C::DT) * C::VROW + vcol[i % C::DT];
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
  // t counts the chunk's tiles from 0; its key tile is t_lo + t, and the
  // wave needs the first wt of them
  // (n_tiles >= 1: an item has at least one key tile.  The first tile is
  // loaded and stored unconditionally, so the Q fragment loads above are
  // complete on every path into the loop and the loop waits for none of them.)
  const int wt = w_tiles - t_lo;
  load_tile(t_lo, B0{});
  store_tile(B0{});
  __syncthreads();
  auto step = [&](auto BC, auto BP, auto BN, int t) {
    if (t + 1 < n_tiles) load_tile(t_lo + t + 1, BN);
    if (!lag) {
      if (t < wt) {
        phase_s(BC, t_lo + t);
        phase_pv(BC);
      }
    } else {
      if (t >= 1 && t - 1 < wt) phase_pv(BP);
      if (t < wt) phase_s(BC, t_lo + t);
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
  if (lag && n_tiles - 1 < wt) {
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
  if (SPLIT && part) {
    // a part of the keys: this part's output O_c / l_c (bf16, normalised by
    // its own sum), the running maximum m_c and the sum l_c, for the merge
    // (attn_merge).  A wave's rows start at a multiple of 32 and a tile's
    // keys at a multiple of 64, so every tile the wave computes begins at or
    // before its first row: each row has a finite maximum from the chunk's
    // first tile on.  A wave that needs none of the chunk's tiles leaves
    // (-inf, 0) and O = 0, which the merge weighs 0.
    const int64_t pr = ((int64_t)chunk * t_kept + lo + qa) * hq + head;
    if (g == 0) ws_ml[pr] = make_float2(mrun, lt);
    const float pinv = lt > 0.0f ? 1.0f / lt : 0.0f;
    uint16_t* po = ws_o + pr * DH;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 pk;
        pk.x = pack_bf16x2(oacc[dt][4 * r4 + 0] * pinv, oacc[dt][4 * r4 + 1] * pinv);
        pk.y = pack_bf16x2(oacc[dt][4 * r4 + 2] * pinv, oacc[dt][4 * r4 + 3] * pinv);
        *reinterpret_cast<uint2*>(po + 32 * dt + 8 * r4 + 4 * g) = pk;
      }
    return;
  }
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
template <int DH, int HPW, int NWAVE, bool SPLIT>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(2)))
void gated_attn_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, const float* __restrict__ kept_b,
    const int32_t* __restrict__ kept_pos, const int32_t* __restrict__ kept_cu, int n_seq,
    int t_kept, int hq, int hkv, int groups_y, int n_slots, const float* __restrict__ gain,
    const float* __restrict__ temp, float sm_scale, float* __restrict__ lse2, int chunk_tiles,
    int c_max, const int* __restrict__ plan, uint16_t* __restrict__ ws_o,
    float2* __restrict__ ws_ml) {
  using C = AttnCfg<DH, HPW, NWAVE>;
  static_assert(NWAVE % HPW == 0 && C::NTHR >= BKV, "workgroup shape");
  __shared__ __attribute__((aligned(1024))) uint16_t sk0[C::KTILE], sk1[C::KTILE], sk2[C::KTILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sv0[C::VTILE], sv1[C::VTILE], sv2[C::VTILE];
  __shared__ __attribute__((aligned(16))) uint16_t sb[NBUF * C::BTILE];

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
  if constexpr (!SPLIT) {
    for (int64_t round = 0;; ++round) {
      const int64_t rank = round * pj + ((round & 1) ? pj - 1 - jb : jb);
      if (rank >= n_real) break;
      gated_attn_item<DH, HPW, NWAVE, false>(q, k, v, out, kept_b, kept_pos, kept_cu, n_seq,
                                             t_kept, hq, hkv, groups_y, hg, n_real - 1 - rank,
                                             gain, temp, sm_scale, lse2, sk0, sk1, sk2, sv0, sv1, sv2, sb, 0, 1, 0, nullptr,
                                             nullptr);
      __syncthreads();                             // LDS buffers are reused by the next slot
    }
  } else {
    // ---- the split form: the items attn_plan listed (a query block, or one
    // key chunk of a long one, coded slot * 8 + chunk), largest first, dealt
    // to the head group's workgroups in snake order
    const int64_t n_it = plan[0];
    const int* __restrict__ list = plan + 64;
    for (int64_t round = 0;; ++round) {
      const int64_t r = round * pj + ((round & 1) ? pj - 1 - jb : jb);
      if (r >= n_it) break;
      const int code = list[r];
      gated_attn_item<DH, HPW, NWAVE, true>(q, k, v, out, kept_b, kept_pos, kept_cu, n_seq, t_kept,
                                            hq, hkv, groups_y, hg, code >> 3, gain, temp, sm_scale,
                                            lse2, sk0, sk1, sk2, sv0, sv1, sv2, sb, chunk_tiles, c_max, code & 7, ws_o,
                                            ws_ml);
      __syncthreads();                               // LDS buffers are reused by the next item
    }
  }
}

// ---------------------------------------------------------------------------
// The plan of a split launch, one workgroup: every query block's items (the
// block, or its key chunks as gated_attn_item cuts them), sorted by their
// key tiles, largest first (a counting sort; items of one size in no fixed
// order, which changes only which workgroup runs them), and the list of
// split blocks for the merge.  plan[0] = items, plan[1] = split blocks;
// plan + 64 the items; splits[i] = (first row, rows, chunks) of split block i.
// ---------------------------------------------------------------------------
constexpr int kPlanBuckets = 4096;               // item sizes sorted exactly up to 4095 tiles
constexpr int kPlanCache = 4096;                 // slots whose block shape is kept between the passes

__global__ __launch_bounds__(1024) void attn_plan(const int32_t* __restrict__ kept_cu, int n_seq,
                                                  int t_kept, int n_slots, int qb,
                                                  int chunk_tiles, int c_max,
                                                  int* __restrict__ plan,
                                                  int4* __restrict__ splits) {
  __shared__ int cnt[kPlanBuckets];
  __shared__ int3 shape[kPlanCache];               // (key tiles, first row, rows) per slot
  __shared__ int sh[1024 / 64];
  __shared__ int n_split;
  const int tid = threadIdx.x;
  for (int i = tid; i < kPlanBuckets; i += 1024) cnt[i] = 0;
  if (tid == 0) n_split = 0;
  __syncthreads();
  // key tiles of slot's query block (0: no work), its first row and rows
  auto block_of = [&](int slot, int& row0, int& rows) -> int {
    const int s = seq_of_slot(kept_cu, n_seq, slot, qb);
    if (s < 0) return 0;
    const int lo = kept_cu[s] < t_kept ? kept_cu[s] : t_kept;
    const int len = (kept_cu[s + 1] < t_kept ? kept_cu[s + 1] : t_kept) - lo;
    const int q0 = (int)(slot - slot0_of(kept_cu, s, qb)) * qb;
    if (q0 >= len) return 0;
    const int q_end = q0 + qb < len ? q0 + qb : len;
    row0 = lo + q0;
    rows = q_end - q0;
    return (q_end + BKV - 1) / BKV;
  };
  auto chunks_of = [&](int n_all) {
    if (n_all <= chunk_tiles) return 1;
    const int c = (n_all + chunk_tiles - 1) / chunk_tiles;
    return c < c_max ? c : c_max;
  };
  auto tiles_of = [&](int n_all, int j) {
    const int t_lo = j * chunk_tiles;
    return (j == c_max - 1 || n_all - t_lo <= chunk_tiles ? n_all : t_lo + chunk_tiles) - t_lo;
  };
  // bucket 0 holds the largest items
  auto bucket = [&](int tiles) {
    return kPlanBuckets - 1 - (tiles < kPlanBuckets - 1 ? tiles : kPlanBuckets - 1);
  };
  for (int slot = tid; slot < n_slots; slot += 1024) {
    int row0 = 0, rows = 0;
    const int n_all = block_of(slot, row0, rows);
    if (slot < kPlanCache) shape[slot] = make_int3(n_all, row0, rows);
    if (n_all == 0) continue;
    const int nc = chunks_of(n_all);
    for (int j = 0; j < nc; ++j) atomicAdd(&cnt[bucket(tiles_of(n_all, j))], 1);
  }
  __syncthreads();
  // exclusive prefix sums of the bucket counts: four buckets per thread,
  // then a scan over the threads
  static_assert(kPlanBuckets == 4 * 1024, "four buckets per thread");
  int a[4], tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = cnt[4 * tid + i];
    tot += a[i];
  }
  int total;
  int run = block_excl_scan<1024>(tot, sh, &total);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cnt[4 * tid + i] = run;
    run += a[i];
  }
  __syncthreads();
  int* __restrict__ list = plan + 64;
  for (int slot = tid; slot < n_slots; slot += 1024) {
    int row0 = 0, rows = 0, n_all;
    if (slot < kPlanCache) {
      const int3 sv = shape[slot];
      n_all = sv.x;
      row0 = sv.y;
      rows = sv.z;
    } else {
      n_all = block_of(slot, row0, rows);
    }
    if (n_all == 0) continue;
    const int nc = chunks_of(n_all);
    for (int j = 0; j < nc; ++j) list[atomicAdd(&cnt[bucket(tiles_of(n_all, j))], 1)] = slot * 8 + j;
    if (nc > 1) splits[atomicAdd(&n_split, 1)] = make_int4(row0, rows, nc, 0);
  }
  __syncthreads();
  if (tid == 0) {
    plan[0] = total;
    plan[1] = n_split;
  }
}

// The key chunks of the split query blocks merged, one wave per (row, head):
// with each chunk's (m_c, l_c, o_c = O_c / l_c) (O_c and l_c relative to
// m_c), M = max m_c, w_c = 2^(m_c - M) l_c, O = sum w_c o_c / sum w_c, and
// the row's lse2 = M + log2(sum w_c).  blockIdx.x: the split block (of
// attn_plan's list), blockIdx.y: 256 / (DH / 8) of its (row, head) pairs,
// DH / 8 threads per pair, each merging 8 dims with one 16-byte load per
// chunk, all issued before the first is used.
constexpr int kMaxChunks = 8;

template <int DH>
__global__ __launch_bounds__(256) void attn_merge(const uint16_t* __restrict__ ws_o,
                                                  const float2* __restrict__ ws_ml,
                                                  const int* __restrict__ plan,
                                                  const int4* __restrict__ splits, int t_kept,
                                                  int hq, uint16_t* __restrict__ out,
                                                  float* __restrict__ lse2) {
  constexpr int TPP = DH / 8;                      // threads per (row, head) pair, 8 dims each
  constexpr int PPB = 256 / TPP;                   // pairs per workgroup
  if ((int)blockIdx.x >= plan[1]) return;
  const int4 sp = splits[blockIdx.x];              // first row, rows, chunks
  const int pair = blockIdx.y * PPB + threadIdx.x / TPP;
  const int part = threadIdx.x % TPP;              // dims 8 part .. +8
  const int r = pair / hq;
  if (r >= sp.y) return;
  const int head = pair % hq;
  const int64_t row = (int64_t)sp.x + r;
  const int nc = sp.z;
  float2 ml[kMaxChunks];
  u32x4 ov[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nc) {
      const int64_t pr = ((int64_t)c * t_kept + row) * hq + head;
      ml[c] = ws_ml[pr];
      ov[c] = ld16(ws_o + pr * DH + 8 * part);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
    if (c < nc) M = fmaxf(M, ml[c].x);
  float L = 0.0f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nc) {
      const float w =
          ml[c].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[c].x - M) * ml[c].y;
      L += w;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t wd = ov[c][i >> 1];
        acc[i] = fmaf(w, __uint_as_float((i & 1) ? (wd & 0xffff0000u) : (wd << 16)), acc[i]);
      }
    }
  }
  const float inv = 1.0f / L;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  st16(out + (row * hq + head) * DH + 8 * part, o);
  if (lse2 && part == 0) lse2[(int64_t)head * t_kept + row] = M + __log2f(L);
}

// How tg_gated_attn_split divides the keys: query blocks of more than
// chunk_tiles key tiles are split into chunks of chunk_tiles tiles (at most
// c_max of them, the last running to the block's end).  chunk_tiles is a
// workgroup's share of the causal work (key tiles per workgroup of a head
// group when the sequences are as long as max_len allows, where the work is
// largest), so that, sorted largest first, the items fill the workgroups
// evenly.  Nothing is split when the longest block exceeds that share by
// less than a quarter: the plan and the merge then cost more than the
// shorter critical path saves (measured at 7000 kept rows: 110 tiles against
// a share of 96).  Workgroups are counted for a full 256-CU gfx950 whatever
// the device reports: the plan's shape, the workspace size and the results
// depend on the sizes alone.
// Chunks are at least kMinChunkTiles tiles, and only inputs whose longest
// block has kMinSplitTiles tiles or more are split: below, the plan and the
// merge cost more than the shorter critical path saves (measured at 522,
// 826 and 1100 kept rows).
struct SplitPlan {
  int chunk_tiles;     // key tiles per chunk (kNoSplit: no block is split)
  int c_max;           // chunks of the longest block (1: no partial results)
};
constexpr int kNoSplit = 1 << 30;
constexpr int kMinChunkTiles = 8;
constexpr int kMinSplitTiles = 20;

// workspace layout of the split form (byte offsets, each 256-aligned)
struct SplitLayout {
  size_t list, splits, o, ml, total;
};

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

SplitLayout split_layout(int64_t t_kept, int64_t n_slots, int c_max, int hq, int dh) {
  SplitLayout l{};
  l.list = 0;                                              // 64 header ints + the items
  l.splits = round256((64 + (size_t)n_slots * c_max) * 4);
  l.o = l.splits + round256((size_t)n_slots * 16);
  l.ml = l.o + (c_max > 1 ? round256((size_t)c_max * t_kept * hq * dh * 2) : 0);
  l.total = l.ml + (c_max > 1 ? (size_t)c_max * t_kept * hq * 8 : 0);
  return l;
}

template <int DH, int HPW, int NWAVE>
hipError_t launch_cfg(const void* q, const void* k, const void* v, void* out, int64_t t_kept,
                      const float* kept_b, const int32_t* kept_pos, const int32_t* kept_cu,
                      int n_seq, int hq, int hkv, const float* gain, const float* temp,
                      float sm_scale, float* lse2, const SplitPlan* sp, void* ws,
                      hipStream_t st) {
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
  const int c_max = sp ? sp->c_max : 1;
  const int chunk_tiles = sp && sp->c_max > 1 ? sp->chunk_tiles : kNoSplit;
  const int64_t n_items = n_slots * c_max;
  int64_t pj = n_cu / n_hg;
  if (pj < 1) pj = 1;
  if (pj > n_items) pj = n_items;
  const int64_t blocks = (int64_t)n_hg * pj;
  if (n_items > 0x7fffffff / 8 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  int* plan = nullptr;
  int4* splits = nullptr;
  uint16_t* ws_o = nullptr;
  float2* ws_ml = nullptr;
  if (sp) {
    const SplitLayout l = split_layout(t_kept, n_slots, c_max, hq, DH);
    char* base = static_cast<char*>(ws);
    plan = reinterpret_cast<int*>(base + l.list);
    splits = reinterpret_cast<int4*>(base + l.splits);
    if (c_max > 1) {
      ws_o = reinterpret_cast<uint16_t*>(base + l.o);
      ws_ml = reinterpret_cast<float2*>(base + l.ml);
    }
    hipLaunchKernelGGL(attn_plan, dim3(1), dim3(1024), 0, st, kept_cu, n_seq, (int)t_kept,
                       (int)n_slots, QB, chunk_tiles, c_max, plan, splits);
  }
  auto kern = sp ? gated_attn_bf16<DH, HPW, NWAVE, true> : gated_attn_bf16<DH, HPW, NWAVE, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * NWAVE), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), kept_b, kept_pos,
                     kept_cu, n_seq, (int)t_kept, hq, hkv, groups_y, (int)n_slots, gain, temp,
                     sm_scale, lse2, chunk_tiles, c_max, plan, ws_o, ws_ml);
  if (ws_o) {
    constexpr int PPB = 256 / (DH / 8);            // pairs per merge workgroup
    const int64_t gy = ((int64_t)QB * hq + PPB - 1) / PPB;
    if (gy > 65535 || n_slots > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_merge<DH>), dim3((unsigned)n_slots, (unsigned)gy), dim3(256), 0, st,
                       ws_o, ws_ml, plan, splits, (int)t_kept, hq, static_cast<uint16_t*>(out),
                       lse2);
  }
  return hipGetLastError();
}

// query rows per workgroup of the configuration launch_attn_bf16 picks
int attn_qb(int hq, int hkv) {
  const int G = hq / hkv;
  const int hpw = G >= 4 ? 4 : G;
  return kAttnWaves * QW / hpw;
}

// key tiles of one sequence of n rows over its query blocks of qb rows
int64_t causal_tiles(int64_t n, int64_t qb) {
  if (n <= 0) return 0;
  const int64_t nb = (n + qb - 1) / qb;
  // blocks 0 .. nb-2 are full: block i reaches (i + 1) qb / BKV tiles
  return qb / BKV * (nb - 1) * nb / 2 + (n + BKV - 1) / BKV;
}

SplitPlan split_plan(int64_t t_kept, int n_seq, int max_len, int hq, int hkv) {
  constexpr int n_cu = 256;
  const int G = hq / hkv;
  const int hpw = G >= 4 ? 4 : G;
  const int n_hg = hkv * (G / hpw);
  SplitPlan p{kNoSplit, 1};
  const int64_t qb = attn_qb(hq, hkv);
  const int64_t ml = max_len < 1 ? 1 : (max_len < t_kept ? max_len : (t_kept > 0 ? t_kept : 1));
  // the most causal work t_kept rows in n_seq sequences of at most ml rows
  // can hold: as many full-length sequences as fit, then the rest
  int64_t n_full = t_kept / ml;
  if (n_full > n_seq) n_full = n_seq;
  const int64_t rest = t_kept - n_full * ml;
  const int64_t work = n_full * causal_tiles(ml, qb) + (n_full < n_seq ? causal_tiles(rest, qb) : 0);
  int64_t pj = n_cu / n_hg;
  if (pj < 1) pj = 1;
  const int64_t share = (work + pj - 1) / pj;
  const int64_t max_tiles = (ml + BKV - 1) / BKV;
  if (max_tiles < kMinSplitTiles || 4 * max_tiles <= 5 * share) return p;
  int64_t per = share;
  if (per < (max_tiles + kMaxChunks - 1) / kMaxChunks) per = (max_tiles + kMaxChunks - 1) / kMaxChunks;
  if (per < kMinChunkTiles) per = kMinChunkTiles;
  if (per >= max_tiles) return p;
  p.chunk_tiles = (int)per;
  p.c_max = (int)((max_tiles + per - 1) / per);
  return p;
}

}  // namespace

size_t attn_split_ws_bytes(int64_t t_kept, int n_seq, int max_len, int hq, int hkv, int dh) {
  const SplitPlan p = split_plan(t_kept, n_seq, max_len, hq, hkv);
  const int64_t n_slots = n_seq + (t_kept + attn_qb(hq, hkv) - 1) / attn_qb(hq, hkv);
  return split_layout(t_kept, n_slots, p.c_max, hq, dh).total;
}

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* out, int64_t t_kept,
                            const float* kept_b, const int32_t* kept_pos, const int32_t* kept_cu,
                            int n_seq, int max_len, int hq, int hkv, int dh, const float* gain,
                            const float* temp, float sm_scale, float* lse2, hipStream_t st,
                            void* ws) {
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / sqrtf((float)dh);
  SplitPlan plan{};
  if (ws) plan = split_plan(t_kept, n_seq, max_len, hq, hkv);
  // one sequence with no block split: its blocks already run largest first
  // (the plain launch's order), so the plan is skipped
  const SplitPlan* pp = ws && (plan.c_max > 1 || n_seq > 1) ? &plan : nullptr;
  const int G = hq / hkv;
  const int hpw = G >= 4 ? 4 : G;
#define TG_ATTN(DHv, HPWv)                                                                     \
  if (dh == DHv && hpw == HPWv)                                                                \
    return launch_cfg<DHv, HPWv, kAttnWaves>(q, k, v, out, t_kept, kept_b, kept_pos, kept_cu, n_seq, hq, \
                                 hkv, gain, temp, sm_scale, lse2, pp, ws, st);
  TG_ATTN(128, 1) TG_ATTN(128, 2) TG_ATTN(128, 4)
  TG_ATTN(64, 1) TG_ATTN(64, 2) TG_ATTN(64, 4)
#undef TG_ATTN
  return hipErrorInvalidValue;
}

}  // namespace tg
