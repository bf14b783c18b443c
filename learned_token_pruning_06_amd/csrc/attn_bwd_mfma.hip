// tg_gated_attn_bwd for bf16 inputs on the matrix cores (the same gradients
// as the vector-ALU passes: TokenGate §4.2 Eq. 8, with the gain of Eq. 6 and
// the temperature of Eq. 7; §4.3 names the path into the gate's scores).
//
// Three passes over 64 x 64 (query x key) tiles, 8 waves per workgroup, all
// products on v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//   bwdm_stats  per (query tile, head): S^T = K.Q^T and dP^T = V.dO^T
//               (waves 0-3 and 4-7, one 32 x 32 tile each), then the row
//               log2-sum-exp and D_i = sum_j P_ij dP_ij by an online merge;
//   bwdm_dkdv   per (key tile, KV head), looping over the group's heads and
//               the query tiles at or after it: S^T, dP^T as above, then
//               P^T and dS^T = (tau dl)^T in bf16 in LDS, then
//               dV += P^T.dO and dK += dS^T.Q (one 32 x 32 tile of each per
//               wave); the b gradient per KV head from the fp32 dS values;
//   bwdm_dq     per (query tile, head), looping over key tiles: S^T, dP^T,
//               dS in bf16, dQ += dS.K; the gain / temperature partial sums
//               from the fp32 values.
// The workspace and the final sums (bwd_finish) are shared with the
// vector-ALU passes.  P and dS enter the dV, dK and dQ products rounded to
// bf16, as in flash-attention backward passes; the statistics, D, and the
// score, gain and temperature gradients use the fp32 values.
//
// Operand staging: every tile sits in LDS row-major with its contraction
// index contiguous where it is an A operand or the B' operand of C = A.B'^T
// (one 16-byte read per lane and K-step); where the contraction runs down
// the rows of a row-major tile (dO and Q in the dV/dK products, K in dQ)
// the B operand is two transposing 8-byte reads (ds_read_b64_tr_b16).
#include "common.h"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int kB = 64;               // queries and keys per tile
constexpr int kThr = 512;            // 8 waves
constexpr int kLX = kB + 1;          // fp32 exchange tile stride
constexpr int kLP = kB + 8;          // bf16 P^T / dS tile stride
constexpr float kLog2e = 1.4426950408889634f;

TG_DEVINL bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
TG_DEVINL uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// acc[32 x 32] += A[32 rows][K] . B'[32 rows][K]^T, k contiguous in both
// (ZERO: acc = the product, the first step adding to a zero constant)
template <int KSTEPS, bool ZERO = false>
TG_DEVINL void mma_abt(floatx16& acc, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                       int lane) {
  const int r = lane & 31, kg = lane >> 5;
  const floatx16 zero = {};
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const bf16x8 a = as_bf16x8(ld16(A + r * lda + 16 * s + 8 * kg));
    const bf16x8 b = as_bf16x8(ld16(B + r * ldb + 16 * s + 8 * kg));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, (ZERO && s == 0) ? zero : acc, 0, 0, 0);
  }
}

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

// acc[32 x 32] += A[32 rows][K] . B[K][32 cols]; A k-contiguous, B row-major
// (its 32 columns contiguous) in LDS, 8-byte aligned rows: the B operand of
// lane (n, kg), rows 16s + 8kg .. +8 of column n, is two transposing reads
template <int KSTEPS>
TG_DEVINL void mma_ab_rows(floatx16& acc, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                           int lane) {
  const int r = lane & 31, kg = lane >> 5;
  const uint16_t* bp = B + (8 * kg + ((lane & 15) >> 2)) * ldb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const bf16x8 a = as_bf16x8(ld16(A + r * lda + 16 * s + 8 * kg));
    const uint2 lo = ld_tr4(bp + 16 * s * ldb), hi = ld_tr4(bp + (16 * s + 4) * ldb);
    const bf16x8 b = as_bf16x8((u32x4){lo.x, lo.y, hi.x, hi.y});
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
}

// C layout of a 32 x 32 tile: register j of lane (n, g) is row 8(j/4) + 4g + j%4, column n
TG_DEVINL int crow(int j, int g) { return 8 * (j >> 2) + 4 * g + (j & 3); }

// 64 rows of head `hd` of a [*, H, DH] bf16 tensor, rows past `len` zero,
// into LDS rows of stride DH + 8
template <int DH>
TG_DEVINL void load_rows(uint16_t* dst, const uint16_t* __restrict__ src, int64_t lo, int len,
                         int r0, int H, int hd) {
  constexpr int LD = DH + 8, CPR = DH / 8;
  for (int u = threadIdx.x; u < kB * CPR; u += kThr) {
    const int r = u / CPR, c = u % CPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + r < len) v = ld16(src + ((lo + r0 + r) * H + hd) * (int64_t)DH + 8 * c);
    st16(dst + r * LD + 8 * c, v);
  }
}

// The same rows fetched into registers one iteration ahead, then stored.
// Buffer loads: the resource starts at the tile's first row of head hd and
// ends after the sequence's last row of that head, so rows past `len` read
// zeros with no per-row test, and each thread's byte offsets within a tile
// are fixed for the kernel (set once by init).
template <int DH>
struct Pf {
  static constexpr int N = kB * (DH / 8) / kThr;
  u32x4 r[N];
  int off[N];
  TG_DEVINL void init(int H) {
    constexpr int CPR = DH / 8;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = threadIdx.x + i * kThr, row = u / CPR, c = u % CPR;
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
  TG_DEVINL void store(uint16_t* dst) const {
    constexpr int CPR = DH / 8, LD = DH + 8;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = threadIdx.x + i * kThr, row = u / CPR, c = u % CPR;
      st16(dst + row * LD + 8 * c, r[i]);
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

TG_DEVINL bool tile_of_slot(const int32_t* cu, int n_seq, int64_t t, int64_t slot, Seq& sq,
                            int& t0) {
  const int s = seq_of_slot(cu, n_seq, slot, kB);
  if (s < 0) return false;
  sq.lo = cu[s] < t ? cu[s] : t;
  const int64_t hi = cu[s + 1] < t ? cu[s + 1] : t;
  sq.len = hi > sq.lo ? (int)(hi - sq.lo) : 0;
  t0 = (int)(slot - slot0_of(cu, s, kB)) * kB;
  return t0 < sq.len;
}

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

// Phase A of every pass: waves 0-3 compute S^T = K.Q^T for tile (kt, qt) =
// (w & 1, w >> 1), waves 4-7 compute dP^T = V.dO^T for the same tile.  The
// elementwise work is then split evenly: registers 0-7 of a lane (key rows
// 32kt + 0..15) go to the S wave, registers 8-15 (rows 32kt + 16..31) to the
// dP wave, so each wave parks the other half of its tile in the fp32
// exchange tile sX[key][query] (the two halves never overlap).
template <int DH>
TG_DEVINL void phase_a(floatx16& acc, int wv, int lane, const uint16_t* sK, const uint16_t* sV,
                       const uint16_t* sQ, const uint16_t* sO, float* sX) {
  constexpr int LD = DH + 8;
  const int w4 = wv & 3, kt = w4 & 1, qt = w4 >> 1;
  const int n = lane & 31, g = lane >> 5;
  if (wv < 4) mma_abt<DH / 16, true>(acc, sK + 32 * kt * LD, LD, sQ + 32 * qt * LD, LD, lane);
  else mma_abt<DH / 16, true>(acc, sV + 32 * kt * LD, LD, sO + 32 * qt * LD, LD, lane);
  // the parked half as a vector select of the two halves (a run-time
  // register index would cost a mode switch and a move per element); key
  // row crow(8 + j) is crow(j) + 16
  const floatx8 lo = __builtin_shufflevector(acc, acc, 0, 1, 2, 3, 4, 5, 6, 7);
  const floatx8 hi = __builtin_shufflevector(acc, acc, 8, 9, 10, 11, 12, 13, 14, 15);
  const floatx8 park = wv < 4 ? hi : lo;
  float* xrow = sX + (32 * kt + (wv < 4 ? 16 : 0)) * kLX + 32 * qt + n;
#pragma unroll
  for (int j = 0; j < 8; ++j) xrow[crow(j, g) * kLX] = park[j];
}

// After phase A and a barrier: this wave's 8 elements (S, dP).  Element jj
// sits at key row kbase + kofs(jj) of the tile (kbase = 32kt + 4g, plus 16
// on the dP wave, whose elements are registers 8..15); the lane's query row
// is 32qt + n.
TG_DEVINL constexpr int kofs(int jj) { return 8 * (jj >> 2) + (jj & 3); }

struct Elems {
  float S[8], dP[8];
  int kbase;
  TG_DEVINL int kr(int jj) const { return kbase + kofs(jj); }
};

// (Vector selects of the two halves of acc: a register index chosen at run
// time would cost a mode switch and a move per element.)
TG_DEVINL void gather(const floatx16& acc, int wv, int lane, const float* sX, Elems& e) {
  const int w4 = wv & 3, kt = w4 & 1, qt = w4 >> 1;
  const int n = lane & 31, g = lane >> 5, qr = 32 * qt + n;
  const bool sw = wv < 4;
  e.kbase = 32 * kt + 4 * g + (sw ? 0 : 16);
  const floatx8 lo = __builtin_shufflevector(acc, acc, 0, 1, 2, 3, 4, 5, 6, 7);
  const floatx8 hi = __builtin_shufflevector(acc, acc, 8, 9, 10, 11, 12, 13, 14, 15);
  const floatx8 mine = sw ? lo : hi;
  const float* xr = sX + e.kbase * kLX + qr;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const float x = xr[kofs(jj) * kLX];
    e.S[jj] = sw ? mine[jj] : x;
    e.dP[jj] = sw ? x : mine[jj];
  }
}

// log2-domain logits of the 8 elements minus `off` (the row's lse2 where the
// probabilities follow at once, else 0); -inf where masked.  Tiles wholly
// below the diagonal and inside the sequence skip the per-element test
// (lanes where `full` holds for all take no masking branch).
TG_DEVINL void logits(const Elems& e, float (&l2)[8], int qi, int k0, bool full, float c1, float c2,
                      const float* sb, float off = 0.0f) {
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) l2[jj] = fmaf(c1, e.S[jj], fmaf(c2, sb[e.kr(jj)], -off));
  if (!full) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (k0 + e.kr(jj) > qi) l2[jj] = -INFINITY;
  }
}

// ---- pass 1: lse2 and D per (query, head)
template <int DH>
__global__ __launch_bounds__(kThr) void bwdm_stats(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ kept_b, const int32_t* __restrict__ kept_pos,
    const int32_t* __restrict__ cu, int n_seq, int64_t t, int hq, int hkv,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm,
    float* __restrict__ lse2, float* __restrict__ dsum, int64_t n_slots) {
  constexpr int LD = DH + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kB * LD], sO[kB * LD], sK[kB * LD],
      sV[kB * LD];
  __shared__ float sX[kB * kLX];
  __shared__ float stau[kB], sb[kB], sm_[4][kB], sl_[4][kB], su_[4][kB];
  Seq sq;
  int q0;
  int64_t slot;
  int kvh, hh;
  work_item(blockIdx.x, hkv, hq / hkv, n_slots, true, slot, kvh, hh);
  if (!tile_of_slot(cu, n_seq, t, slot, sq, q0)) return;
  const int h = kvh * (hq / hkv) + hh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, g = lane >> 5, w4 = wv & 3, kt = w4 & 1, qt = w4 >> 1;
  const float gh = gain[h];
  if (tid < kB)
    stau[tid] = q0 + tid < sq.len ? temp[h] * length_lambda(kept_pos, sq.lo + q0 + tid, q0 + tid)
                                  : 0.0f;
  load_rows<DH>(sQ, q, sq.lo, sq.len, q0, hq, h);
  load_rows<DH>(sO, dout, sq.lo, sq.len, q0, hq, h);
  float m = -INFINITY, L = 0.0f, U = 0.0f;            // this lane's query, its keys so far
  const int qr = 32 * qt + n, qi = q0 + qr;
  const int q_end = q0 + kB < sq.len ? q0 + kB : sq.len;
  Pf<DH> pk, pv;                                      // key tile k0 + 64, in flight
  pk.init(hkv);
  pv.init(hkv);
  float pb = 0.0f;
  pk.load(k, sq.lo, sq.len, 0, hkv, kvh);
  pv.load(v, sq.lo, sq.len, 0, hkv, kvh);
  if (tid < kB) pb = tid < sq.len ? kept_b[sq.lo + tid] : 0.0f;
  __syncthreads();
  const float tau = stau[qr];
  const float c1 = tau * sm * kLog2e, c2 = tau * gh * kLog2e;
  for (int k0 = 0; k0 < q_end; k0 += kB) {
    __syncthreads();
    pk.store(sK);
    pv.store(sV);
    if (tid < kB) sb[tid] = pb;
    if (k0 + kB < q_end) {
      pk.load(k, sq.lo, sq.len, k0 + kB, hkv, kvh);
      pv.load(v, sq.lo, sq.len, k0 + kB, hkv, kvh);
      if (tid < kB) pb = k0 + kB + tid < sq.len ? kept_b[sq.lo + k0 + kB + tid] : 0.0f;
    }
    __syncthreads();
    floatx16 acc;
    phase_a<DH>(acc, wv, lane, sK, sV, sQ, sO, sX);
    __syncthreads();
    if (qi < sq.len) {
      Elems e;
      gather(acc, wv, lane, sX, e);
      float l2[8];
      logits(e, l2, qi, k0, k0 + kB <= q0, c1, c2, sb);
      float mt = l2[0];
#pragma unroll
      for (int jj = 1; jj < 8; ++jj) mt = fmaxf(mt, l2[jj]);
      if (mt != -INFINITY) {
        const float mn = fmaxf(m, mt);
        const float f = __builtin_amdgcn_exp2f(m - mn);
        L *= f;
        U *= f;
        m = mn;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(l2[jj] - mn);
          L += p;
          U = fmaf(p, e.dP[jj], U);
        }
      }
    }
  }
  // merge the two lane halves, then the four partial states of each query
  // (two waves per tile x two key halves)
  const float m2 = __shfl_xor(m, 32, 64), L2 = __shfl_xor(L, 32, 64), U2 = __shfl_xor(U, 32, 64);
  const float mn = fmaxf(m, m2);
  if (mn != -INFINITY) {
    const float f1 = __builtin_amdgcn_exp2f(m - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);
    L = L * f1 + L2 * f2;
    U = U * f1 + U2 * f2;
    m = mn;
  }
  const int part = 2 * kt + (wv >> 2);
  if (g == 0) {
    sm_[part][qr] = m;
    sl_[part][qr] = L;
    su_[part][qr] = U;
  }
  __syncthreads();
  if (tid < kB && q0 + tid < sq.len) {
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < 4; ++p) mx = fmaxf(mx, sm_[p][tid]);
    float Lt = 0.0f, Ut = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float f = sm_[p][tid] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sm_[p][tid] - mx);
      Lt = fmaf(sl_[p][tid], f, Lt);
      Ut = fmaf(su_[p][tid], f, Ut);
    }
    const int64_t row = sq.lo + q0 + tid;
    lse2[(int64_t)h * t + row] = mx + __log2f(Lt);
    dsum[row * hq + h] = Ut / Lt;
  }
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

// P and dl = P (dP - D) of this wave's 8 elements
// l2 already has the row's lse2 taken off (logits with off = lse2)
TG_DEVINL void probs(const Elems& e, const float (&l2)[8], float D, float (&P)[8],
                     float (&dl)[8]) {
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    P[jj] = __builtin_amdgcn_exp2f(l2[jj]);           // 0 where masked
    dl[jj] = P[jj] * (e.dP[jj] - D);
  }
}

// ---- pass 2: dK, dV and the per-KV-head b gradient, per (key tile, KV head)
template <int DH>
__global__ __launch_bounds__(kThr) void bwdm_dkdv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ kept_b, const int32_t* __restrict__ kept_pos,
    const int32_t* __restrict__ cu, int n_seq, int64_t t, int hq, int hkv,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm,
    const float* __restrict__ lse2, const float* __restrict__ dsum, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dbpart, int64_t n_slots) {
  constexpr int LD = DH + 8, NDT = DH / 32;            // 32-wide d tiles
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kB * LD], sO[kB * LD], sK[kB * LD],
      sV[kB * LD];
  __shared__ __attribute__((aligned(16))) uint16_t sPT[kB * kLP], sDT[kB * kLP];
  __shared__ float sX[kB * kLX];
  __shared__ float stau[kB], slse[kB], sD[kB], sb[kB];
  Seq sq;
  int k0;
  int64_t slot;
  int kvh, hh0;
  work_item(blockIdx.x, hkv, 1, n_slots, false, slot, kvh, hh0);
  if (!tile_of_slot(cu, n_seq, t, slot, sq, k0)) return;
  const int G = hq / hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, w4 = wv & 3, qt = w4 >> 1;
  const int ct = wv & 1, dt = wv >> 1;                  // phase C tile: keys 32ct, d 32dt
  load_rows<DH>(sK, k, sq.lo, sq.len, k0, hkv, kvh);
  load_rows<DH>(sV, v, sq.lo, sq.len, k0, hkv, kvh);
  if (tid < kB) sb[tid] = k0 + tid < sq.len ? kept_b[sq.lo + k0 + tid] : 0.0f;
  floatx16 aV, aK;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    aV[j] = 0.0f;
    aK[j] = 0.0f;
  }
  float dbacc = 0.0f;
  // iterations (head hh, query tile q0), query tiles from the last one down
  // to the diagonal, so that the workgroups of one head group that run
  // together read the same Q and dO tiles at about the same time; the next
  // iteration's Q, dO and row scalars are fetched while the current one is
  // computed
  const int qfirst = (k0 / kB) * kB;
  const int qlast = ((sq.len - 1) / kB) * kB;
  Pf<DH> pq, po;
  pq.init(hq);
  po.init(hq);
  float ptau = 0.0f, plse = 0.0f, pD = 0.0f;
  auto fetch = [&](int hh, int q0) {
    const int h = kvh * G + hh;
    pq.load(q, sq.lo, sq.len, q0, hq, h);
    po.load(dout, sq.lo, sq.len, q0, hq, h);
    if (tid < kB) {
      const int i = q0 + tid;
      const bool ok = i < sq.len;
      ptau = ok ? temp[h] * length_lambda(kept_pos, sq.lo + i, i) : 0.0f;
      plse = ok ? lse2[(int64_t)h * t + sq.lo + i] : 0.0f;
      pD = ok ? dsum[(sq.lo + i) * hq + h] : 0.0f;
    }
  };
  fetch(0, qlast);
  for (int hh = 0; hh < G; ++hh) {
    const int h = kvh * G + hh;
    const float gh = gain[h];
    for (int q0 = qlast; q0 >= qfirst; q0 -= kB) {
      __syncthreads();
      pq.store(sQ);
      po.store(sO);
      if (tid < kB) {
        stau[tid] = ptau;
        slse[tid] = plse;
        sD[tid] = pD;
      }
      if (q0 - kB >= qfirst) fetch(hh, q0 - kB);
      else if (hh + 1 < G) fetch(hh + 1, qlast);
      __syncthreads();
      floatx16 acc;
      phase_a<DH>(acc, wv, lane, sK, sV, sQ, sO, sX);
      __syncthreads();
      {
        const int qr = 32 * qt + n, qi = q0 + qr;
        Elems e;
        gather(acc, wv, lane, sX, e);
        const float tau = stau[qr];
        float l2[8], P[8], dl[8];
        logits(e, l2, qi < sq.len ? qi : -1, k0, q0 > k0 && qi < sq.len, tau * sm * kLog2e,
               tau * gh * kLog2e, sb, slse[qr]);
        probs(e, l2, sD[qr], P, dl);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int kr = e.kr(jj);
          const float ds = dl[jj] * tau;
          sPT[kr * kLP + qr] = f2bf(P[jj]);
          sDT[kr * kLP + qr] = f2bf(ds);
          sX[kr * kLX + qr] = ds;                      // fp32, for the b gradient
        }
      }
      __syncthreads();
      if (dt < NDT) {
        // dV[key][d] += sum_q P^T[key][q] dO[q][d];  dK[key][d] += sum_q dS^T[key][q] Q[q][d]
        mma_ab_rows<kB / 16>(aV, sPT + 32 * ct * kLP, kLP, sO + 32 * dt, LD, lane);
        mma_ab_rows<kB / 16>(aK, sDT + 32 * ct * kLP, kLP, sQ + 32 * dt, LD, lane);
      }
      {                                                 // db_j += g_h sum_q tau_q dl_qj
        const int key = tid >> 3, part = tid & 7;       // 8 threads per key, 8 queries each
        float cs = 0.0f;
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) cs += sX[key * kLX + 8 * part + qq];
        cs += __shfl_xor(cs, 1, 64);
        cs += __shfl_xor(cs, 2, 64);
        cs += __shfl_xor(cs, 4, 64);
        dbacc = fmaf(gh, cs, dbacc);                    // every thread of the key holds it
      }
    }
  }
  if (dt < NDT) {
    const int g = lane >> 5;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = k0 + 32 * ct + crow(j, g);
      if (key < sq.len) {
        const int64_t off = ((sq.lo + key) * hkv + kvh) * (int64_t)DH + 32 * dt + n;
        dv[off] = aV[j];
        dk[off] = sm * aK[j];
      }
    }
  }
  if ((tid & 7) == 0 && k0 + (tid >> 3) < sq.len)
    dbpart[(int64_t)kvh * t + sq.lo + k0 + (tid >> 3)] = dbacc;
}

// ---- pass 3: dQ and the gain / temperature partials, per (query tile, head)
template <int DH>
__global__ __launch_bounds__(kThr) void bwdm_dq(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ kept_b, const int32_t* __restrict__ kept_pos,
    const int32_t* __restrict__ cu, int n_seq, int64_t t, int hq, int hkv,
    const float* __restrict__ gain, const float* __restrict__ temp, float sm,
    const float* __restrict__ lse2, const float* __restrict__ dsum, float* __restrict__ dq,
    double* __restrict__ gpart, int64_t n_slots) {
  constexpr int LD = DH + 8, NDT = DH / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kB * LD], sO[kB * LD], sK[kB * LD],
      sV[kB * LD];
  __shared__ __attribute__((aligned(16))) uint16_t sDS[kB * kLP];
  __shared__ float sX[kB * kLX];
  __shared__ float stau[kB], slam[kB], slse[kB], sD[kB], sb[kB];
  __shared__ double sred[2][kThr / 64];
  int64_t slot;
  int kvh, hh;
  work_item(blockIdx.x, hkv, hq / hkv, n_slots, true, slot, kvh, hh);
  const int h = kvh * (hq / hkv) + hh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, w4 = wv & 3, qt = w4 >> 1;
  const int ct = wv & 1, dt = wv >> 1;                  // phase C: queries 32ct, d 32dt
  double* gp = gpart + (slot * hq + h) * 2;
  Seq sq;
  int q0;
  if (!tile_of_slot(cu, n_seq, t, slot, sq, q0)) {
    if (tid == 0) {                                    // every slot leaves a partial
      gp[0] = 0.0;
      gp[1] = 0.0;
    }
    return;
  }
  const float gh = gain[h];
  if (tid < kB) {
    const int i = q0 + tid;
    const bool ok = i < sq.len;
    const float lam = ok ? length_lambda(kept_pos, sq.lo + i, i) : 0.0f;
    slam[tid] = lam;
    stau[tid] = temp[h] * lam;
    slse[tid] = ok ? lse2[(int64_t)h * t + sq.lo + i] : 0.0f;
    sD[tid] = ok ? dsum[(sq.lo + i) * hq + h] : 0.0f;
  }
  load_rows<DH>(sQ, q, sq.lo, sq.len, q0, hq, h);
  load_rows<DH>(sO, dout, sq.lo, sq.len, q0, hq, h);
  floatx16 aQ;
#pragma unroll
  for (int j = 0; j < 16; ++j) aQ[j] = 0.0f;
  double accg = 0.0, acct = 0.0;
  const int q_end = q0 + kB < sq.len ? q0 + kB : sq.len;
  Pf<DH> pk, pv;                                      // key tile k0 + 64, in flight
  pk.init(hkv);
  pv.init(hkv);
  float pb = 0.0f;
  pk.load(k, sq.lo, sq.len, 0, hkv, kvh);
  pv.load(v, sq.lo, sq.len, 0, hkv, kvh);
  if (tid < kB) pb = tid < sq.len ? kept_b[sq.lo + tid] : 0.0f;
  __syncthreads();
  const int qr = 32 * qt + n, qi = q0 + qr;
  const float tau = stau[qr], lam = slam[qr], lse = slse[qr], D = sD[qr];
  const float c1 = tau * sm * kLog2e, c2 = tau * gh * kLog2e;
  for (int k0 = 0; k0 < q_end; k0 += kB) {
    __syncthreads();
    pk.store(sK);
    pv.store(sV);
    if (tid < kB) sb[tid] = pb;
    if (k0 + kB < q_end) {
      pk.load(k, sq.lo, sq.len, k0 + kB, hkv, kvh);
      pv.load(v, sq.lo, sq.len, k0 + kB, hkv, kvh);
      if (tid < kB) pb = k0 + kB + tid < sq.len ? kept_b[sq.lo + k0 + kB + tid] : 0.0f;
    }
    __syncthreads();
    floatx16 acc;
    phase_a<DH>(acc, wv, lane, sK, sV, sQ, sO, sX);
    __syncthreads();
    {
      Elems e;
      gather(acc, wv, lane, sX, e);
      float l2[8], P[8], dl[8];
      logits(e, l2, qi < sq.len ? qi : -1, k0, k0 + kB <= q0 && qi < sq.len, c1, c2, sb, lse);
      probs(e, l2, D, P, dl);
      // the tile's 8 terms in fp32, then into the fp64 sums
      float pg = 0.0f, pt = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int kr = e.kr(jj);
        const float tdl = dl[jj] * tau;
        sDS[qr * kLP + kr] = f2bf(tdl);
        pg = fmaf(tdl, sb[kr], pg);
        pt = fmaf(dl[jj] * lam, fmaf(sm, e.S[jj], gh * sb[kr]), pt);
      }
      accg += (double)pg;
      acct += (double)pt;
    }
    __syncthreads();
    // dQ[q][d] += sum_key dS[q][key] K[key][d]
    if (dt < NDT) mma_ab_rows<kB / 16>(aQ, sDS + 32 * ct * kLP, kLP, sK + 32 * dt, LD, lane);
  }
  if (dt < NDT) {
    const int g = lane >> 5;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = q0 + 32 * ct + crow(j, g);
      if (i < sq.len) dq[((sq.lo + i) * hq + h) * (int64_t)DH + 32 * dt + n] = sm * aQ[j];
    }
  }
  accg = wave_sum(accg);
  acct = wave_sum(acct);
  if (lane == 0) {
    sred[0][wv] = accg;
    sred[1][wv] = acct;
  }
  __syncthreads();
  if (tid == 0) {
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int w = 0; w < kThr / 64; ++w) {
      a += sred[0][w];
      b += sred[1][w];
    }
    gp[0] = a;
    gp[1] = b;
  }
}

}  // namespace

hipError_t launch_attn_bwd_mfma(const void* q, const void* k, const void* v, const void* dout,
                                int64_t t, const float* kept_b, const int32_t* kept_pos,
                                const int32_t* cu, int n_seq, int hq, int hkv, int dh,
                                const float* gain, const float* temp, float sm, float* lse2,
                                float* dsum, float* dq, float* dk, float* dv, float* dbpart,
                                double* gpart, const void* fwd_out, const float* fwd_lse2,
                                hipStream_t st) {
  const int64_t nq = n_seq + (t + kB - 1) / kB;
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
    hipLaunchKernelGGL((bwdm_stats<DHv>), dim3((unsigned)(nq * hq)), dim3(kThr), 0, st, qp, kp, \
                       vp, op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse2,    \
                       dsum, nq);                                                                \
  hipLaunchKernelGGL((bwdm_dkdv<DHv>), dim3((unsigned)(nq * hkv)), dim3(kThr), 0, st, qp, kp, vp, \
                     op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse, dsum,     \
                     dk, dv, dbpart, nq);                                                        \
  hipLaunchKernelGGL((bwdm_dq<DHv>), dim3((unsigned)(nq * hq)), dim3(kThr), 0, st, qp, kp, vp,  \
                     op, kept_b, kept_pos, cu, n_seq, t, hq, hkv, gain, temp, sm, lse, dsum, dq, \
                     gpart, nq);
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
