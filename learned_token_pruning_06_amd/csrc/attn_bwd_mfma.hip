// tg_gated_attn_bwd for bf16 inputs on the matrix cores (the same gradients
// as the vector-ALU passes: TokenGate §4.2 Eq. 8, with the gain of Eq. 6 and
// the temperature of Eq. 7; §4.3 names the path into the gate's scores).
//
// Passes, all products on v_mfma_f32_32x32x16_bf16 with fp32 accumulation,
// four waves per workgroup (one per SIMD) holding their own rows' operands
// in registers:
//   bwdm_dsum   (with the forward's output and lse2) D_i = dO_i . O_i;
//   bwdm_q<STATS> (without them) the row log2-sum-exp and D_i by an online
//               merge, per (128-query block, head);
//   bwdm_kv     per (128-key block, KV head), waves holding the K and V rows
//               of 32 keys, looping over the group's heads and the 64-query
//               tiles at or after the block: S and dP from the staged Q and
//               dO, P and dS = tau dl in registers (bf16) as the A operands
//               of dV += P^T.dO and dK += dS^T.Q; the b gradient per KV head
//               from the fp32 dS values;
//   bwdm_q      per (128-query block, head), waves holding the Q and dO rows
//               of 32 queries, looping over the 64-key tiles up to the
//               diagonal: S^T, dP^T, dS in bf16 as the A operand of
//               dQ += dS.K; the gain / temperature partial sums from the
//               fp32 values.
// The workspace and the final sums (bwd_finish) are shared with the
// vector-ALU passes.  P and dS enter the dV, dK and dQ products rounded to
// bf16, as in flash-attention backward passes; the statistics, D, and the
// score, gain and temperature gradients use the fp32 values.
//
// Operand staging: the Q/dO (or K/V) tiles sit in LDS in a swizzled
// row-major layout read both ways: 16-byte row reads for the operands whose
// contraction runs along the row, two transposing 8-byte reads
// (ds_read_b64_tr_b16) for those whose contraction runs down the rows.
#include "common.h"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kB = 64;               // queries and keys per tile
constexpr float kLog2e = 1.4426950408889634f;

TG_DEVINL bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// 4 consecutive rows of one column per lane by a transposing LDS read
// (ds_read_b64_tr_b16): within each 16-lane group, output element e of lane
// i is element i % 4 of the 8 bytes that lane 4e + i / 4 addresses, so lane
// s pointing at row s / 4, columns 4(s % 4) .. +4 hands lane i the rows
// 0 .. 3 of column i
TG_DEVINL uint2 ld_tr4(const uint16_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p)));
}

// C layout of a 32 x 32 tile: register j of lane (n, g) is row 8(j/4) + 4g + j%4, column n
TG_DEVINL int crow(int j, int g) { return 8 * (j >> 2) + 4 * g + (j & 3); }

// Swizzled tile layout for tiles read both row-wise (16-byte reads) and by
// transposing 8-byte reads: rows of DH + 32 elements (320 B for DH 128,
// 192 B for DH 64: four consecutive rows start in the four 64-byte quarters
// of the 256 bytes the LDS serves per cycle, which the transposing reads
// need), and the 16-byte chunk c of row r stored at chunk c ^ ((r / 4) % 4),
// which spreads the 16 rows of a 16-byte read over distinct banks too.
template <int DH>
TG_DEVINL constexpr int swz_ld() { return DH + 32; }
template <int DH>
TG_DEVINL int swz_off(int row, int chunk) {
  return row * swz_ld<DH>() + 8 * (chunk ^ ((row >> 2) & 3));
}

// 64 rows of head hd of a [*, H, DH] bf16 tensor fetched into registers one
// tile ahead, then stored into the swizzled layout.
// Buffer loads: the resource starts at the tile's first row of head hd and
// ends after the sequence's last row of that head, so rows past `len` read
// zeros with no per-row test, and each thread's byte offsets within a tile
// are fixed for the kernel (set once by init).
template <int DH, int NT>
struct Pf {
  static constexpr int N = kB * (DH / 8) / NT;
  u32x4 r[N];
  int off[N];
  TG_DEVINL void init(int H) {
    constexpr int CPR = DH / 8;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = threadIdx.x + i * NT, row = u / CPR, c = u % CPR;
      off[i] = (row * H * DH + 8 * c) * 2;
    }
  }
  TG_DEVINL void load(const uint16_t* __restrict__ src, int64_t lo, int len, int r0, int H,
                      int hd) {
    const int64_t rowel = (int64_t)H * DH;           // elements between token rows
    const int64_t rows = (int64_t)len - r0;
    int64_t bytes = rows > 0 ? ((rows - 1) * rowel + DH) * 2 : 0;
    if (bytes > 0x7fffffff) bytes = 0x7fffffff;     // beyond every offset of a tile
    const uint16_t* base = src + ((lo + r0) * rowel + (int64_t)hd * DH);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base), (short)0, (int)bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, 0));
  }
  // into the swizzled layout of swz_off
  TG_DEVINL void store_swz(uint16_t* dst) const {
    constexpr int CPR = DH / 8;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = threadIdx.x + i * NT, row = u / CPR, c = u % CPR;
      st16(dst + swz_off<DH>(row, c), r[i]);
    }
  }
};

TG_DEVINL float length_lambda(const int32_t* kept_pos, int64_t row, int local) {
  if (!kept_pos) return 1.0f;
  return logf((float)(local + 1)) / logf(fmaxf(2.0f, (float)kept_pos[row] + 1.0f));
}

struct Seq {
  int64_t lo;
  int len;
};

// Work item of block b in the one-dimensional grids of the three passes.
// Blocks are dealt round-robin over the 8 XCDs, each with its own L2, so the
// KV head is taken from the low bits of the block index: with 8 KV heads
// every XCD works on one head group, and its workgroups share the K/V (or
// Q/dO) tiles of that group in its L2.  Per-head passes (hq heads) put the
// G query heads of a group on consecutive blocks of one XCD; `reverse`
// deals the slots last-first (the longest causal work first when each slot
// is a query tile).
TG_DEVINL void work_item(int64_t b, int hkv, int g_heads, int64_t n_slots, bool reverse,
                         int64_t& slot, int& kvh, int& hh) {
  kvh = (int)(b % hkv);
  const int64_t r = b / hkv;
  hh = (int)(r % g_heads);
  slot = r / g_heads;
  if (reverse) slot = n_slots - 1 - slot;
}

// ---- pass 1 from saved forward state: D per (query, head) as dO_i . O_i,
// which equals sum_j P_ij dP_ij because O_i = sum_j P_ij V_j and
// dP_ij = dO_i . V_j.  DH / 8 lanes per (row, head), 16 bytes each.
template <int DH>
__global__ __launch_bounds__(256) void bwdm_dsum(const uint16_t* __restrict__ o,
                                                 const uint16_t* __restrict__ dout, int64_t pairs,
                                                 float* __restrict__ dsum) {
  constexpr int L = DH / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t p = gid / L;
  float acc = 0.0f;
  if (p < pairs) {
    const u32x4 a = ld16(o + gid * 8), b = ld16(dout + gid * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), acc);
      acc = fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (p < pairs && (threadIdx.x % L) == 0) dsum[p] = acc;
}

// ---- pass 2: dK, dV and the
// per-KV-head b gradient, per (block of 128 keys, KV head).  Four waves, one
// per SIMD; wave w owns keys k0 + 32w .. +32 and holds their K and V rows in
// registers for the whole pass (the B operands of S = Q.K^T and dP = dO.V^T,
// keys on the MFMA N axis).  The Q and dO tiles of 64 queries are staged in
// LDS (two buffers, one barrier per tile) and read twice: row-wise as the A
// operands of S and dP, and by transposing reads as the B operands of
// dV += P^T.dO and dK += dS^T.Q.  In the S accumulator lane (n, g) holds key
// n and queries 8(j/4) + 4g + j%4, so its P and dS values are directly the A
// operand of those products: K-step kk takes queries 16kk + 8(e/4) + 4g +
// e%4, and the transposing reads fetch dO and Q rows in that same order.
// The bias enters S as one more K-step (a selector on the query side, the
// head's gain * b / s split into two bf16 parts on the key side).
constexpr int kKB = 128;             // keys per workgroup of this pass
constexpr int kKvThr = 256;          // 4 waves

TG_DEVINL bool block_of_slot(const int32_t* cu, int n_seq, int64_t t, int64_t slot, int ch,
                             Seq& sq, int& t0) {
  const int s = seq_of_slot(cu, n_seq, slot, ch);
  if (s < 0) return false;
  sq.lo = cu[s] < t ? cu[s] : t;
  const int64_t hi = cu[s + 1] < t ? cu[s + 1] : t;
  sq.len = hi > sq.lo ? (int)(hi - sq.lo) : 0;
  t0 = (int)(slot - slot0_of(cu, s, ch)) * ch;
  return t0 < sq.len;
}

TG_DEVINL uint32_t pack2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int DH>
__global__ __launch_bounds__(kKvThr) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwdm_kv(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
             const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
             const float* __restrict__ kept_b, const int32_t* __restrict__ kept_pos,
             const int32_t* __restrict__ cu, int n_seq, int64_t t, int hq, int hkv,
             const float* __restrict__ gain, const float* __restrict__ temp, float sm,
             const float* __restrict__ lse2, const float* __restrict__ dsum,
             float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dbpart,
             int64_t n_slots) {
  constexpr int LD = swz_ld<DH>(), KS = DH / 16, NDT = DH / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][kB * LD], sO[2][kB * LD];
  // per query of a staged tile: c = tau s log2(e), lse2 (+inf past the
  // sequence), D and tau
  __shared__ __attribute__((aligned(16))) float sC[2][kB], sL[2][kB], sD[2][kB], sT[2][kB];
  Seq sq;
  int k0;
  int64_t slot;
  int kvh, hh0;
  work_item(blockIdx.x, hkv, 1, n_slots, false, slot, kvh, hh0);
  if (!block_of_slot(cu, n_seq, t, slot, kKB, sq, k0)) return;
  const int G = hq / hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, g = lane >> 5;
  const int kw0 = k0 + 32 * wv;                       // the wave's first key
  const int len = sq.len;

  // K and V rows of key kw0 + n (B operands: dims 16s + 8g .. +8), zeros past the end
  u32x4 kf[KS], vf[KS];
  float bk = 0.0f;
  {
    const bool ok = kw0 + n < len;
    const int64_t row = ((sq.lo + (ok ? kw0 + n : 0)) * hkv + kvh) * (int64_t)DH + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = ok ? ld16(k + row + 16 * s) : (u32x4){0u, 0u, 0u, 0u};
      vf[s] = ok ? ld16(v + row + 16 * s) : (u32x4){0u, 0u, 0u, 0u};
    }
    if (ok) bk = kept_b[sq.lo + kw0 + n];
  }
  // selector of the bias K-step: query-side columns 0 and 1 (lane half 0)
  const u32x4 sel = g == 0 ? (u32x4){pack2(1.0f, 1.0f), 0u, 0u, 0u} : (u32x4){0u, 0u, 0u, 0u};

  floatx16 aV[NDT], aK[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      aV[d][j] = 0.0f;
      aK[d][j] = 0.0f;
    }
  float dbacc = 0.0f;

  // tiles (head hh, query tile q0): per head, from the last query tile down
  // to the one holding the block's first key; the next tile's rows and
  // per-query values are fetched while the current one is computed
  const int qfirst = (k0 / kB) * kB;
  const int qlast = ((len - 1) / kB) * kB;
  const int nq = (qlast - qfirst) / kB + 1;
  const int total = G * nq;
  Pf<DH, kKvThr> pq, po;
  pq.init(hq);
  po.init(hq);
  float pc = 0.0f, pl = 0.0f, pd = 0.0f, pt = 0.0f;
  auto fetch = [&](int it) {
    const int hh = it / nq, q0 = qlast - (it % nq) * kB;
    const int h = kvh * G + hh;
    pq.load(q, sq.lo, len, q0, hq, h);
    po.load(dout, sq.lo, len, q0, hq, h);
    if (tid < kB) {
      const int i = q0 + tid;
      const bool ok = i < len;
      const float tau = ok ? temp[h] * length_lambda(kept_pos, sq.lo + i, i) : 0.0f;
      pc = tau * sm * kLog2e;
      pt = tau;
      pl = ok ? lse2[(int64_t)h * t + sq.lo + i] : INFINITY;
      pd = ok ? dsum[(sq.lo + i) * hq + h] : 0.0f;
    }
  };
  auto stash = [&](int buf) {
    pq.store_swz(sQ[buf]);
    po.store_swz(sO[buf]);
    if (tid < kB) {
      sC[buf][tid] = pc;
      sL[buf][tid] = pl;
      sD[buf][tid] = pd;
      sT[buf][tid] = pt;
    }
  };
  fetch(0);
  stash(0);
  __syncthreads();
  const floatx16 zero = {};
  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    if (it + 1 < total) fetch(it + 1);
    const int hh = it / nq, q0 = qlast - (it % nq) * kB;
    const int h = kvh * G + hh;
    const float gh = gain[h];
    // bias operand of this head: gain * b / s as a high and a low bf16 part
    const float beta = gh * bk / sm;
    const float bhi = (float)(__bf16)beta;
    const u32x4 bop = g == 0 ? (u32x4){pack2(bhi, beta - bhi), 0u, 0u, 0u} : (u32x4){0u, 0u, 0u, 0u};
    const uint16_t* qt = sQ[buf];
    const uint16_t* ot = sO[buf];
    float dsl = 0.0f;                                 // sum of this lane's dS values
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int qb = q0 + 32 * qh;                    // first query of the half
      if (kw0 > qb + 31) continue;                    // every key after every query
      // S' = Q.K^T + bias and dP = dO.V^T for 32 queries x the wave's 32 keys;
      // A operands: row 32qh + n, chunk 2s + g, stored at chunk (2s + g) ^ fr
      // with fr = (n / 4) % 4, i.e. 4(s/2) + ((2(s%2)) ^ g ^ fr)
      floatx16 sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sel), as_bf16x8(bop),
                                                              zero, 0, 0, 0);
      floatx16 pacc = zero;
      {
        const int v = g ^ ((n >> 2) & 3);
        const int row = (32 * qh + n) * LD;
        const int e0 = row + 8 * v, e1 = row + 8 * (v ^ 2);
        // product m: S' (even m, Q row) or dP (odd m, dO row) of K-step m / 2;
        // its A operand is read four products ahead, the order pinned by
        // scheduling barriers (one wave per SIMD: nothing else hides the
        // LDS latency)
        auto opnd = [&](int m) {
          const int st = m >> 1;
          return ld16(((m & 1) ? ot : qt) + ((st & 1) ? e1 : e0) + 32 * (st >> 1));
        };
        constexpr int NM = 2 * KS;
        u32x4 ra[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ra[m] = opnd(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (m & 1)
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ra[m % 4]),
                                                           as_bf16x8(vf[m >> 1]), pacc, 0, 0, 0);
          else
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ra[m % 4]),
                                                           as_bf16x8(kf[m >> 1]), sacc, 0, 0, 0);
          if (m + 4 < NM) ra[m % 4] = opnd(m + 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // element j: query qb + 8(j/4) + 4g + j%4, key kw0 + n; keys after the
      // query are masked (only halves that reach past the diagonal test)
      uint32_t pw[8], dw[8];
      auto elementwise = [&](auto MASKC) {
        constexpr bool MASK = decltype(MASKC)::value;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int qi = 32 * qh + 8 * r4 + 4 * g;    // query of j = 4 r4, in the tile
          const float4 c4 = *reinterpret_cast<const float4*>(&sC[buf][qi]);
          const float4 l4 = *reinterpret_cast<const float4*>(&sL[buf][qi]);
          const float4 d4 = *reinterpret_cast<const float4*>(&sD[buf][qi]);
          const float4 t4 = *reinterpret_cast<const float4*>(&sT[buf][qi]);
          const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, ll[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dd[4] = {d4.x, d4.y, d4.z, d4.w}, tt[4] = {t4.x, t4.y, t4.z, t4.w};
          float P[4], S[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * r4 + e;
            float l2 = fmaf(cc[e], sacc[j], -ll[e]);
            if (MASK && kw0 + n > q0 + qi + e) l2 = -INFINITY;
            P[e] = __builtin_amdgcn_exp2f(l2);
            S[e] = P[e] * (pacc[j] - dd[e]) * tt[e];
            dsl += S[e];
          }
          pw[2 * r4] = pack2(P[0], P[1]);
          pw[2 * r4 + 1] = pack2(P[2], P[3]);
          dw[2 * r4] = pack2(S[0], S[1]);
          dw[2 * r4 + 1] = pack2(S[2], S[3]);
        }
      };
      if (kw0 + 31 > qb) elementwise(std::true_type{});
      else elementwise(std::false_type{});
      // dV += P^T.dO and dK += dS^T.Q over the half's queries: K-step kk is
      // registers j = 8kk .. +8 (words 4kk .. +4); B rows 16kk + 4g + 0..3 and
      // 16kk + 8 + 4g + 0..3 of dim 32d + n, by two transposing reads each.
      // Lane (16-lane group h, i = lane % 16) points at row R + i/4 (R =
      // 32qh + 16kk + 4g, so (row / 4) % 4 = g, and g ^ 2 eight rows on),
      // logical chunk 4d + 2h + (i%4)/2, element 4((i%4)%2) within it.
      {
        const int h2 = (lane >> 4) & 1, c = lane & 3;
        const int lrow = 4 * g + ((lane & 15) >> 2);
        const int t0 = lrow * LD + 8 * ((2 * h2 + (c >> 1)) ^ g) + 4 * (c & 1);
        const int t1 = (lrow + 8) * LD + 8 * ((2 * h2 + (c >> 1)) ^ g ^ 2) + 4 * (c & 1);
        // product i: dV (even i, dO rows) or dK (odd i, Q rows) of K-step
        // kk = (i / 2) / NDT, dims 32 d .. +32 with d = (i / 2) % NDT; its B
        // operand is read four products ahead, as above
        auto topnd = [&](int i) {
          const int pd = i >> 1, kk = pd / NDT, d = pd % NDT;
          const uint16_t* base = ((i & 1) ? qt : ot) + (32 * qh + 16 * kk) * LD + 32 * d;
          const uint2 a = ld_tr4(base + t0), b = ld_tr4(base + t1);
          return (u32x4){a.x, a.y, b.x, b.y};
        };
        const bf16x8 pa[2] = {as_bf16x8((u32x4){pw[0], pw[1], pw[2], pw[3]}),
                              as_bf16x8((u32x4){pw[4], pw[5], pw[6], pw[7]})};
        const bf16x8 da[2] = {as_bf16x8((u32x4){dw[0], dw[1], dw[2], dw[3]}),
                              as_bf16x8((u32x4){dw[4], dw[5], dw[6], dw[7]})};
        constexpr int NP = 4 * NDT;
        u32x4 rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = topnd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int pd = i >> 1, kk = pd / NDT, d = pd % NDT;
          if (i & 1)
            aK[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[kk], as_bf16x8(rb[i % 4]), aK[d], 0,
                                                            0, 0);
          else
            aV[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], as_bf16x8(rb[i % 4]), aV[d], 0,
                                                            0, 0);
          if (i + 4 < NP) rb[i % 4] = topnd(i + 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    dbacc = fmaf(gh, dsl, dbacc);
    if (it + 1 < total) stash(buf ^ 1);
    __syncthreads();
  }
  // dV, dK rows: register j of lane (n, g) is key kw0 + 8(j/4) + 4g + j%4, dim 32d + n
#pragma unroll
  for (int d = 0; d < NDT; ++d)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = kw0 + crow(j, g);
      if (key < len) {
        const int64_t off = ((sq.lo + key) * hkv + kvh) * (int64_t)DH + 32 * d + n;
        dv[off] = aV[d][j];
        dk[off] = sm * aK[d][j];
      }
    }
  // the b gradient of key kw0 + n: the two lane halves hold its two query halves
  dbacc += __shfl_xor(dbacc, 32, 64);
  if (g == 0 && kw0 + n < len) dbpart[(int64_t)kvh * t + sq.lo + kw0 + n] = dbacc;
}

// ---- pass 3: dQ and the gain / temperature partials, per (block of 128
// queries, head).  Four waves, one per SIMD; wave w owns queries q0 + 32w ..
// +32 and holds their Q and dO rows in registers (the B operands of
// S^T = K.Q^T and dP^T = V.dO^T, queries on the MFMA N axis), looping over
// the 64-key tiles up to the block's diagonal.  K and V tiles are staged in
// LDS (two buffers, one barrier per tile; K in the swizzled layout, as it is
// also read by transposing reads), with each key's bias A operand (the
// head's gain * b / s as two bf16 parts) beside them.  In the S^T
// accumulator lane (n, g) holds query n and keys 8(j/4) + 4g + j%4, so its
// dS values are directly the A operand of dQ += dS.K (keys in runs of four,
// matched by transposing reads of K); the query's lse2, D, tau and lambda
// are per-lane scalars.
// STATS: pass 1 in the same form (without the forward's saved state): the
// row statistics lse2 and D = sum_j P_ij dP_ij by an online merge per lane
// (each lane half holds half of the keys), then across the two halves.
constexpr int kQB = 128;             // queries per workgroup of this pass

template <int DH, bool STATS = false>
__global__ __launch_bounds__(kKvThr) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwdm_q(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
            const float* __restrict__ kept_b, const int32_t* __restrict__ kept_pos,
            const int32_t* __restrict__ cu, int n_seq, int64_t t, int hq, int hkv,
            const float* __restrict__ gain, const float* __restrict__ temp, float sm,
            const float* __restrict__ lse2, const float* __restrict__ dsum,
            float* __restrict__ dq, double* __restrict__ gpart, int64_t n_slots,
            float* __restrict__ lse2_out = nullptr, float* __restrict__ dsum_out = nullptr) {
  constexpr int LD = swz_ld<DH>(), KS = DH / 16, NDT = DH / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kB * LD], sV[2][kB * LD];
  __shared__ __attribute__((aligned(16))) uint32_t sBias[2][kB];   // (hi, lo) bf16 pair per key
  __shared__ __attribute__((aligned(16))) float sb[2][kB];         // b per key
  __shared__ double sred[2][kKvThr / 64];
  int64_t slot;
  int kvh, hh;
  work_item(blockIdx.x, hkv, hq / hkv, n_slots, true, slot, kvh, hh);
  const int h = kvh * (hq / hkv) + hh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, g = lane >> 5;
  double* gp = gpart + (slot * hq + h) * 2;
  Seq sq;
  int q0;
  if (!block_of_slot(cu, n_seq, t, slot, kQB, sq, q0)) {
    if (!STATS && tid == 0) {                          // every slot leaves a partial
      gp[0] = 0.0;
      gp[1] = 0.0;
    }
    return;
  }
  const int len = sq.len;
  const int qw0 = q0 + 32 * wv;                       // the wave's first query
  const int qi = qw0 + n;                             // this lane's query
  const bool qok = qi < len;
  const float gh = gain[h];
  // per-lane query values; past the sequence: nothing (lse2 +inf, c 0)
  float c = 0.0f, lse = INFINITY, D = 0.0f, tau = 0.0f, lam = 0.0f;
  if (qok) {
    lam = length_lambda(kept_pos, sq.lo + qi, qi);
    tau = temp[h] * lam;
    c = tau * sm * kLog2e;
    if constexpr (!STATS) {
      lse = lse2[(int64_t)h * t + sq.lo + qi];
      D = dsum[(sq.lo + qi) * hq + h];
    }
  }
  float sm_m = -INFINITY, sm_l = 0.0f, sm_u = 0.0f;   // STATS: running max, sum, sum of p dP
  // Q and dO rows of query qi (B operands: dims 16s + 8g .. +8)
  u32x4 qf[KS], of[KS];
  {
    const int64_t row = ((sq.lo + (qok ? qi : 0)) * hq + h) * (int64_t)DH + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = qok ? ld16(q + row + 16 * s) : (u32x4){0u, 0u, 0u, 0u};
      of[s] = qok ? ld16(dout + row + 16 * s) : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  const u32x4 sel = g == 0 ? (u32x4){pack2(1.0f, 1.0f), 0u, 0u, 0u} : (u32x4){0u, 0u, 0u, 0u};

  floatx16 aQ[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d)
#pragma unroll
    for (int j = 0; j < 16; ++j) aQ[d][j] = 0.0f;
  double dg = 0.0, dt = 0.0;                          // fp64 sums of the per-tile fp32 sums

  const int q_end = q0 + kQB < len ? q0 + kQB : len;
  const int n_tiles = (q_end + kB - 1) / kB;          // key tiles up to the block's diagonal
  Pf<DH, kKvThr> pk, pv;
  pk.init(hkv);
  pv.init(hkv);
  float pb = 0.0f;
  auto fetch = [&](int kt) {
    pk.load(k, sq.lo, len, kt * kB, hkv, kvh);
    pv.load(v, sq.lo, len, kt * kB, hkv, kvh);
    if (tid < kB) pb = kt * kB + tid < len ? kept_b[sq.lo + kt * kB + tid] : 0.0f;
  };
  auto stash = [&](int buf) {
    pk.store_swz(sK[buf]);
    pv.store_swz(sV[buf]);
    if (tid < kB) {
      const float beta = gh * pb / sm;
      const float bhi = (float)(__bf16)beta;
      sBias[buf][tid] = pack2(bhi, beta - bhi);
      sb[buf][tid] = pb;
    }
  };
  fetch(0);
  stash(0);
  __syncthreads();
  const floatx16 zero = {};
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) fetch(kt + 1);
    const int k0 = kt * kB;
    const uint16_t* kt_ = sK[buf];
    const uint16_t* vt_ = sV[buf];
    float pg = 0.0f, pt = 0.0f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int kb0 = k0 + 32 * kh;                   // first key of the half
      if (kb0 > qw0 + 31) continue;                   // every key after every query
      // S^T' = K.Q^T + bias and dP^T = V.dO^T for 32 keys x the wave's 32
      // queries; A operands: key row 32kh + n, chunk 2s + g (swizzled)
      const u32x4 bia = g == 0 ? (u32x4){sBias[buf][32 * kh + n], 0u, 0u, 0u}
                               : (u32x4){0u, 0u, 0u, 0u};
      floatx16 sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bia), as_bf16x8(sel),
                                                              zero, 0, 0, 0);
      floatx16 pacc = zero;
      {
        const int vv = g ^ ((n >> 2) & 3);
        const int row = (32 * kh + n) * LD;
        const int e0 = row + 8 * vv, e1 = row + 8 * (vv ^ 2);
        // product m: S^T' (even m, K row) or dP^T (odd m, V row) of K-step
        // m / 2, its A operand read four products ahead (as in bwdm_kv)
        auto opnd = [&](int m) {
          const int st = m >> 1;
          return ld16(((m & 1) ? vt_ : kt_) + ((st & 1) ? e1 : e0) + 32 * (st >> 1));
        };
        constexpr int NM = 2 * KS;
        u32x4 ra[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ra[m] = opnd(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (m & 1)
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ra[m % 4]),
                                                           as_bf16x8(of[m >> 1]), pacc, 0, 0, 0);
          else
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ra[m % 4]),
                                                           as_bf16x8(qf[m >> 1]), sacc, 0, 0, 0);
          if (m + 4 < NM) ra[m % 4] = opnd(m + 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // element j: key kb0 + 8(j/4) + 4g + j%4, query qi
      if constexpr (STATS) {
        const bool mask = kb0 + 31 > qw0;
        float l2[16];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          l2[j] = c * sacc[j];
          if (mask && kb0 + crow(j, g) > qi) l2[j] = -INFINITY;
          mt = fmaxf(mt, l2[j]);
        }
        if (qok && mt != -INFINITY) {
          const float mn = fmaxf(sm_m, mt);
          const float f = __builtin_amdgcn_exp2f(sm_m - mn);
          sm_l *= f;
          sm_u *= f;
          sm_m = mn;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float p = __builtin_amdgcn_exp2f(l2[j] - mn);
            sm_l += p;
            sm_u = fmaf(p, pacc[j], sm_u);
          }
        }
        continue;
      }
      uint32_t dw[8];
      auto elementwise = [&](auto MASKC) {
        constexpr bool MASK = decltype(MASKC)::value;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int kl = 32 * kh + 8 * r4 + 4 * g;    // key of j = 4 r4, in the tile
          const float4 b4 = *reinterpret_cast<const float4*>(&sb[buf][kl]);
          const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
          float S[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * r4 + e;
            float l2 = fmaf(c, sacc[j], -lse);
            if (MASK && k0 + kl + e > qi) l2 = -INFINITY;
            const float P = __builtin_amdgcn_exp2f(l2);
            const float dl = P * (pacc[j] - D);
            S[e] = dl * tau;
            pg = fmaf(S[e], bb[e], pg);
            pt = fmaf(dl, sacc[j], pt);
          }
          dw[2 * r4] = pack2(S[0], S[1]);
          dw[2 * r4 + 1] = pack2(S[2], S[3]);
        }
      };
      if (kb0 + 31 > qw0) elementwise(std::true_type{});
      else elementwise(std::false_type{});
      // dQ += dS.K over the half's keys: K-step kk is registers j = 8kk .. +8;
      // B rows 16kk + 4g + 0..3 and 16kk + 8 + 4g + 0..3 of dim 32d + n of
      // the K tile, by two transposing reads each (swizzled as in bwdm_kv)
      {
        const int h2 = (lane >> 4) & 1, cc = lane & 3;
        const int lrow = 4 * g + ((lane & 15) >> 2);
        const int t0 = lrow * LD + 8 * ((2 * h2 + (cc >> 1)) ^ g) + 4 * (cc & 1);
        const int t1 = (lrow + 8) * LD + 8 * ((2 * h2 + (cc >> 1)) ^ g ^ 2) + 4 * (cc & 1);
        // product i: K-step kk = i / NDT, dims 32 d .. +32 with d = i % NDT;
        // its B operand read four products ahead
        auto topnd = [&](int i) {
          const int kk = i / NDT, d = i % NDT;
          const uint16_t* base = kt_ + (32 * kh + 16 * kk) * LD + 32 * d;
          const uint2 a = ld_tr4(base + t0), b = ld_tr4(base + t1);
          return (u32x4){a.x, a.y, b.x, b.y};
        };
        const bf16x8 da[2] = {as_bf16x8((u32x4){dw[0], dw[1], dw[2], dw[3]}),
                              as_bf16x8((u32x4){dw[4], dw[5], dw[6], dw[7]})};
        constexpr int NP = 2 * NDT;
        u32x4 rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = topnd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          aQ[i % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[i / NDT], as_bf16x8(rb[i % 4]),
                                                                aQ[i % NDT], 0, 0, 0);
          if (i + 4 < NP) rb[i % 4] = topnd(i + 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    dg += (double)pg;
    dt += (double)pt;
    if (kt + 1 < n_tiles) stash(buf ^ 1);
    __syncthreads();
  }
  if constexpr (STATS) {
    // merge the two lane halves (disjoint keys of the same query)
    const float m2 = __shfl_xor(sm_m, 32, 64), l2s = __shfl_xor(sm_l, 32, 64);
    const float u2 = __shfl_xor(sm_u, 32, 64);
    const float mn = fmaxf(sm_m, m2);
    const float f1 = sm_m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sm_m - mn);
    const float f2 = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m2 - mn);
    const float L = fmaf(sm_l, f1, l2s * f2), U = fmaf(sm_u, f1, u2 * f2);
    if (g == 0 && qok) {
      const int64_t row = sq.lo + qi;
      lse2_out[(int64_t)h * t + row] = mn + __log2f(L);
      dsum_out[row * hq + h] = U / L;
    }
    return;
  }
  // dQ rows: register j of lane (n, g) is query qw0 + 8(j/4) + 4g + j%4, dim 32d + n
#pragma unroll
  for (int d = 0; d < NDT; ++d)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = qw0 + crow(j, g);
      if (i < len) dq[((sq.lo + i) * hq + h) * (int64_t)DH + 32 * d + n] = sm * aQ[d][j];
    }
  // dgain = sum tau b dl; dtemp = sum lambda z dl with z = s S' (S' = q.k + gain b / s)
  dg = wave_sum(dg);
  dt = wave_sum(dt * (double)(lam * sm));
  if (lane == 0) {
    sred[0][wv] = dg;
    sred[1][wv] = dt;
  }
  __syncthreads();
  if (tid == 0) {
    gp[0] = (sred[0][0] + sred[0][1]) + (sred[0][2] + sred[0][3]);
    gp[1] = (sred[1][0] + sred[1][1]) + (sred[1][2] + sred[1][3]);
  }
}

}  // namespace

int64_t attn_bwd_mfma_gslots(int64_t t, int n_seq) { return n_seq + (t + kQB - 1) / kQB; }

hipError_t launch_attn_bwd_mfma(const void* q, const void* k, const void* v, const void* dout,
                                int64_t t, const float* kept_b, const int32_t* kept_pos,
                                const int32_t* cu, int n_seq, int hq, int hkv, int dh,
                                const float* gain, const float* temp, float sm, float* lse2,
                                float* dsum, float* dq, float* dk, float* dv, float* dbpart,
                                double* gpart, const void* fwd_out, const float* fwd_lse2,
                                hipStream_t st) {
  const int64_t nkb = n_seq + (t + kKB - 1) / kKB;     // key blocks of the dK/dV pass
  const int64_t nqb = attn_bwd_mfma_gslots(t, n_seq);   // query blocks of the dQ pass
  const bool saved = fwd_out != nullptr && fwd_lse2 != nullptr;
  const float* lse = saved ? fwd_lse2 : lse2;
  const int64_t dsum_blocks = (t * hq * (dh / 8) + 255) / 256;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  const uint16_t* op = static_cast<const uint16_t*>(dout);
#define TG_BWDM(DHv)                                                                             \
  if (saved)                                                                                     \
    hipLaunchKernelGGL((bwdm_dsum<DHv>), dim3((unsigned)dsum_blocks), dim3(256), 0, st,          \
                       static_cast<const uint16_t*>(fwd_out), op, t * hq, dsum);                 \
  else                                                                                           \
    hipLaunchKernelGGL((bwdm_q<DHv, true>), dim3((unsigned)(nqb * hq)), dim3(kKvThr), 0, st, qp, \
                       kp, vp, op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm,      \
                       nullptr, nullptr, nullptr, nullptr, nqb, lse2, dsum);                     \
  hipLaunchKernelGGL((bwdm_kv<DHv>), dim3((unsigned)(nkb * hkv)), dim3(kKvThr), 0, st, qp, kp,   \
                     vp, op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse, dsum, \
                     dk, dv, dbpart, nkb);                                                       \
  hipLaunchKernelGGL((bwdm_q<DHv>), dim3((unsigned)(nqb * hq)), dim3(kKvThr), 0, st, qp, kp,    \
                     vp, op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse, dsum, \
                     dq, gpart, nqb);
  if (dh == 128) {
    TG_BWDM(128)
  } else if (dh == 64) {
    TG_BWDM(64)
  } else {
    return hipErrorInvalidValue;
  }
#undef TG_BWDM
  return hipGetLastError();
}

}  // namespace tg
