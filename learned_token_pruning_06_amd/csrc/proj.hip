// tg_qkv_proj: the query, key and value projections of the kept rows,
//   Q = X_S Wq^T,  K = X_S Wk^T,  V = X_S Wv^T,
// i.e. the step between the gather and the token-gated attention (TokenGate
// §4.1: the kept tokens continue through the layers above the gate, whose
// attention §4.2 Eq. 8 reads q, k and v of the kept tokens only).
//
// One bf16 GEMM  Y[t, n] = sum_d X[t, d] W[n, d]  over the concatenated
// weight W = [Wq; Wk; Wv] ([n_tot, d], one row per output feature, the
// nn.Linear layout), on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// The output columns are routed to q, k or v in the epilogue.
//
// A workgroup owns a 256-row x 256-column output tile; 8 waves (two per
// SIMD), wave w owns rows [64(w%4), +64) and columns [128(w/4), +128), i.e.
// 2 x 4 accumulator tiles of 32 x 32 in C^T orientation (columns on the MFMA
// M axis, rows on N), so each lane ends up holding four consecutive output
// columns of one row.  Each 64-wide K-step stages the X and W slices in
// double-buffered, padded LDS tiles (global -> registers one step ahead ->
// LDS; one barrier per step).  Rows past t read zeros through the buffer
// range and are not stored.
#include "common.h"

namespace tg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;           // rows and columns per workgroup
constexpr int kBK = 64;              // d per K-step
constexpr int kRow = kBK + 8;        // bf16 per LDS row (144 B: rows start 4 banks apart)
constexpr int kThreads = 512;

TG_DEVINL bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

TG_DEVINL uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

TG_DEVINL __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7fffffff ? (bytes > 0 ? bytes : 0)
                                                                    : 0x7fffffff),
                                           0x00020000);
}

// F32OUT: the same GEMM for other callers, Y[t, n] (fp32, row stride ldy)
// over the K range [k_per * z, +k_per) of workgroup z (split-K partials at
// Y + z * ys), with W's rows ldw elements apart.
// WROWS (with F32OUT): W is stored K-major instead, W[k][n] with rows ldw
// elements apart and w_rows valid rows (later ones read as zeros).  Its
// K-step tile is staged as [64 k][256 n] (rows padded to 272 elements) and
// the A operand, 8 consecutive k of one column, is two transposing reads
// (ds_read_b64_tr_b16): within each 16-lane group, output element e of lane
// i is element i % 4 of the 8 bytes that lane 4e + i / 4 addresses.
// XROWS (with WROWS): X is stored K-major too, X[k][m] with rows xs elements
// apart and the same w_rows valid rows, staged and read like W (the B
// operand, 8 consecutive k of one row m of the product, by two transposing
// reads).  Both operands of Y = X^T-as-stored . W then come straight from
// token-major arrays, e.g. dW1 = dz^T x with dz [T][h] and x [T][d].
// bf16 per K-major W row: the tile is read only by transposing 8-byte reads,
// served 32 lanes (256 B) at a time over rows r = 0..3 at byte 32h + 8c, so
// rows start 64 B apart mod 256 B (576 B) to keep the 32 addresses on
// distinct banks (544 B rows gave 28% of the LDS-active cycles in conflicts)
constexpr int kRowW = kTile + 32;

TG_DEVINL uint2 ld_tr4(const uint16_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p)));
}

// QKE (bf16 form): the q and k columns get the per-head RMSNorm over dh
// (weight qn / kn, skipped when null) and then the rotate-half rotary
// embedding at position pos[row] (skipped when log2_theta is 0) before they
// are rounded; dh is 64 or 128 and q, k, v start on 128-column boundaries,
// so the 128 columns of a wave are one or two whole heads of one tensor.
struct QkEpi {
  const int32_t* pos;
  const float* qn;
  const float* kn;
  float eps;
  int dh;
  double log2_theta;            // log2 of the rotary base; 0 turns the rotation off
};

// Row correction of the fp32 form (CORR, one K split): Y[row, c] -= c[row] *
// A[row, c] before the store, A bf16 with rows lda elements apart.
struct RowCorr {
  const float* c;               // null: no correction
  const uint16_t* a;
  int64_t lda;
};

template <bool F32OUT, bool WROWS = false, bool QKE = false, bool CORR = false,
          bool XROWS = false>
__global__ __launch_bounds__(kThreads) void gemm_abt_bf16(
    const uint16_t* __restrict__ x, int64_t xs, int64_t t, int d,
    const uint16_t* __restrict__ w, int nq, int nkv, uint16_t* __restrict__ q,
    uint16_t* __restrict__ k, uint16_t* __restrict__ v, int64_t ldw, int k_per,
    float* __restrict__ y, int64_t ldy, int64_t ys, int64_t w_rows = 0, QkEpi ep = QkEpi{},
    RowCorr rc = RowCorr{}) {
  static_assert(F32OUT || !WROWS, "K-major W is for the fp32-output form");
  static_assert(!(F32OUT && QKE), "the q/k epilogue is for the bf16 form");
  static_assert(F32OUT || !CORR, "the row correction is for the fp32 form");
  static_assert(WROWS || !XROWS, "K-major X goes with K-major W");
  __shared__ double s_turns[64];                  // QKE: rotation per position, in turns
  __shared__ float s_norm[2][128];                 // QKE: the q and k norm weights
  __shared__ __attribute__((aligned(16))) uint16_t sx[2][XROWS ? kBK * kRowW : kTile * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][WROWS ? kBK * kRowW : kTile * kRow];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int rg = wv & 3, ch = wv >> 2;
  // (column tile, K split) of this workgroup.  K-major W (one row tile): the
  // column tiles of a split share its X slice, so they are placed on one XCD
  // (workgroups are dealt round-robin over the 8 XCDs, each with its own L2)
  int by = blockIdx.y, bz = blockIdx.z;
  if constexpr (WROWS) {
    const int tiles = gridDim.y * gridDim.z;
    if (gridDim.x == 1 && tiles % 8 == 0) {
      const int lin = blockIdx.y + gridDim.y * blockIdx.z;
      const int l = (lin % 8) * (tiles / 8) + lin / 8;
      by = l % gridDim.y;
      bz = l / gridDim.y;
    }
  }
  const int col0 = by * kTile;
  if constexpr (QKE) {                            // published by the K loop's first barrier
    if (tid < ep.dh / 2)
      s_turns[tid] = exp2(-2.0 * tid / ep.dh * ep.log2_theta) * 0.15915494309189535;
    if (tid < ep.dh) {
      s_norm[0][tid] = ep.qn ? ep.qn[tid] : 1.0f;
      s_norm[1][tid] = ep.kn ? ep.kn[tid] : 1.0f;
    }
  }
  int64_t w_bytes = (int64_t)kTile * ldw * 2;   // W rows of this tile (row-major W)
  if constexpr (F32OUT) {                        // this workgroup's K range
    const int64_t kb = (int64_t)bz * k_per;
    x += XROWS ? kb * xs : kb;
    if constexpr (WROWS) {
      w += kb * ldw;
      w_bytes = ((w_rows - kb) < 0 ? 0 : (w_rows - kb)) * ldw * 2 - (int64_t)col0 * 2;
    } else {
      w += kb;
    }
    d = (int)((d - kb) < k_per ? (d - kb) : k_per);
    y += (int64_t)bz * ys;
  } else {
    ldw = d;
    w_bytes = (int64_t)kTile * ldw * 2;
  }

  // row tiles blockIdx.x, + gridDim.x, ...: the fp32 form runs fewer
  // workgroups than row tiles, so a tile's stores drain while the next
  // tile's loads and products run
  const int64_t m_tiles = (t + kTile - 1) / kTile;
  for (int64_t rt = blockIdx.x; rt < m_tiles; rt += gridDim.x) {
  const int64_t row0 = rt * kTile;
  // loaders: thread vector i covers row (tid / 8) + 64 i, 16-byte chunk tid % 8
  // of the K-step, for both X (rows of this tile) and W (its output features)
  const int lrow = tid >> 3, lch = tid & 7;
  // K-major X: the tile's columns row0 .. of the w_rows - kb valid k rows
  const int64_t x_krows = XROWS ? (w_rows - (int64_t)bz * k_per) : 0;
  const __amdgpu_buffer_rsrc_t rx =
      XROWS ? make_rsrc(x + row0, (x_krows < 0 ? 0 : x_krows) * xs * 2 - row0 * 2)
            : make_rsrc(x + row0 * xs, (t - row0) * xs * 2);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(WROWS ? w + col0 : w + (int64_t)col0 * ldw, w_bytes);
  // K-major W: thread vector i covers k-row (tid / 32) + 16 i, 16-byte chunk tid % 32
  const int wrow = tid >> 5, wch = tid & 31;
  int xoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xoff[i] = XROWS ? (int)(((int64_t)(wrow + 16 * i) * xs + 8 * wch) * 2)
                    : (int)(((int64_t)(lrow + 64 * i) * xs + 8 * lch) * 2);
    woff[i] = WROWS ? (int)(((int64_t)(wrow + 16 * i) * ldw + 8 * wch) * 2)
                    : (int)(((int64_t)(lrow + 64 * i) * ldw + 8 * lch) * 2);
  }
  const int ldst = lrow * kRow + 8 * lch;
  const int wdst = WROWS ? wrow * kRowW + 8 * wch : ldst;
  const int xdst = XROWS ? wdst : ldst;
  u32x4 xr[4], wr[4];
  auto fetch = [&](int k0) {
    const int wk = WROWS ? (int)(2 * (int64_t)k0 * ldw) : 2 * k0;
    const int xk = XROWS ? (int)(2 * (int64_t)k0 * xs) : 2 * k0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i] + xk, 0, 0));
      wr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i] + wk, 0, 0));
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(&sx[buf][xdst + (XROWS ? 16 * i * kRowW : 64 * i * kRow)], xr[i]);
      st16(&sw[buf][wdst + (WROWS ? 16 * i * kRowW : 64 * i * kRow)], wr[i]);
    }
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[mt][0][r] = 0.f;
      acc[mt][1][r] = 0.f;
    }

  const int nsteps = d / kBK;
  fetch(0);
  stage(0);
  if (nsteps > 1) fetch(kBK);
  __syncthreads();
  for (int it = 0; it < nsteps; ++it) {
    const int buf = it & 1;
    const uint16_t* xb = sx[buf] + (64 * rg + n) * kRow + 32 * g;
    const uint16_t* wb = sw[buf] + (128 * ch + n) * kRow + 32 * g;
    // K-major W: lane (m, g) needs k = 32g + 8s .. +8 of column 128ch + 32mt + m
    const uint16_t* wt = sw[buf] + (32 * g + ((lane & 15) >> 2)) * kRowW + 128 * ch +
                         16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // K-major X: lane (n, g) needs k = 32g + 8s .. +8 of row 64rg + 32i + n
    const uint16_t* xt = sx[buf] + (32 * g + ((lane & 15) >> 2)) * kRowW + 64 * rg +
                         16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // operands of 16-wide substep s + 1 are read from LDS while the MFMAs of
    // substep s run: one read after each MFMA, the order pinned
    bf16x8 bo[2][2], ao[2][4];
    auto ld_op = [&](int s, int c, int i) {
      if (i < 2) {
        if constexpr (XROWS) {
          const uint2 lo = ld_tr4(xt + 8 * s * kRowW + 32 * i);
          const uint2 hi = ld_tr4(xt + (8 * s + 4) * kRowW + 32 * i);
          bo[c][i] = as_bf16x8((u32x4){lo.x, lo.y, hi.x, hi.y});
        } else {
          bo[c][i] = as_bf16x8(ld16(xb + 32 * i * kRow + 8 * s));
        }
      } else if constexpr (WROWS) {
        const uint2 lo = ld_tr4(wt + 8 * s * kRowW + 32 * (i - 2));
        const uint2 hi = ld_tr4(wt + (8 * s + 4) * kRowW + 32 * (i - 2));
        ao[c][i - 2] = as_bf16x8((u32x4){lo.x, lo.y, hi.x, hi.y});
      } else {
        ao[c][i - 2] = as_bf16x8(ld16(wb + 32 * (i - 2) * kRow + 8 * s));
      }
    };
#pragma unroll
    for (int i = 0; i < 6; ++i) ld_op(0, 0, i);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int c = s & 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j >> 1][j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao[c][j >> 1], bo[c][j & 1],
                                                                     acc[j >> 1][j & 1], 0, 0, 0);
        if (s + 1 < kBK / 16 && j < 6) ld_op(s + 1, c ^ 1, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (it + 1 < nsteps) {
      stage(buf ^ 1);
      if (it + 2 < nsteps) fetch((it + 2) * kBK);
    }
    __syncthreads();
  }

  // epilogue: lane (n, g) holds columns 32mt + 8(r/4) + 4g + r%4 of this
  // wave's column range, row 32 nt + n of its row range
  if constexpr (F32OUT) {
    // fp32 rows leave through LDS (the K loop's tiles are free after its last
    // barrier): per half of the wave's columns, the wave's 64 x 64 block goes
    // to its own 16 KB region, then 16 lanes write 256 contiguous bytes of a
    // row, 4 rows per store.  The stores are non-temporal: the outputs (dx is
    // 1 GiB at 131072 rows) stream out once and would otherwise leave dirty
    // lines in the L2 for the next kernel to write back.
    constexpr int kLd = 68;                      // floats per staged row (rows 4 banks apart)
    float* stage = reinterpret_cast<float*>(wv < 4 ? &sx[0][0] : &sw[0][0]) + (wv & 3) * 64 * kLd;
    // row correction (CORR): once a half is staged, the lane's A values
    // and row factors are loaded 8 rows at a time ahead of their stores, so
    // the stores wait for 4 round trips per tile instead of one per row
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int mt = 2 * hf + m2;
            *reinterpret_cast<float4*>(stage + (32 * nt + n) * kLd + 32 * m2 + 8 * r4 + 4 * g) =
                make_float4(acc[mt][nt][4 * r4], acc[mt][nt][4 * r4 + 1], acc[mt][nt][4 * r4 + 2],
                            acc[mt][nt][4 * r4 + 3]);
          }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        uint2 av[8];
        float cv[8];
        if constexpr (CORR) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int64_t row = row0 + 64 * rg + 4 * (8 * ib + j) + (lane >> 4);
            const int col = col0 + 128 * ch + 64 * hf + 4 * (lane & 15);
            cv[j] = row < t ? rc.c[row] : 0.0f;
            av[j] = row < t ? *reinterpret_cast<const uint2*>(rc.a + row * rc.lda + col)
                            : make_uint2(0u, 0u);
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * ib + j;
          const int rr = 4 * i + (lane >> 4), c4 = lane & 15;
          const int64_t row = row0 + 64 * rg + rr;
          float4 v4 = *reinterpret_cast<const float4*>(stage + rr * kLd + 4 * c4);
          const int col = col0 + 128 * ch + 64 * hf + 4 * c4;
          if constexpr (CORR) {
            v4.x = fmaf(-cv[j], __uint_as_float(av[j].x << 16), v4.x);
            v4.y = fmaf(-cv[j], __uint_as_float(av[j].x & 0xffff0000u), v4.y);
            v4.z = fmaf(-cv[j], __uint_as_float(av[j].y << 16), v4.z);
            v4.w = fmaf(-cv[j], __uint_as_float(av[j].y & 0xffff0000u), v4.w);
          }
          if (row < t) {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            const f32x4 o = {v4.x, v4.y, v4.z, v4.w};
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(y + row * ldy + col));
          }
        }
      }
    }
  } else {
  if constexpr (QKE) {
    const int wbase = col0 + 128 * ch;               // the wave's 128 columns: q, k or v
    if (wbase < nq + nkv) {
      const bool norm = wbase < nq ? ep.qn != nullptr : ep.kn != nullptr;
      const float* nw = s_norm[wbase < nq ? 0 : 1];
      const int dh = ep.dh;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if (norm) {
          // per head: sum of squares over the lane's 64 values of the row and
          // its partner lane (n, 1 - g), then scale by weight / RMS
          float ss0 = 0.f, ss1 = 0.f;                  // heads of mt 0-1 and 2-3 (dh 64)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float a = acc[mt][nt][r];
              if (mt < 2) ss0 = fmaf(a, a, ss0);
              else ss1 = fmaf(a, a, ss1);
            }
          ss0 += __shfl_xor(ss0, 32, 64);
          ss1 += __shfl_xor(ss1, 32, 64);
          const float inv0 = dh == 128 ? 1.0f / sqrtf((ss0 + ss1) / 128.0f + ep.eps)
                                       : 1.0f / sqrtf(ss0 / 64.0f + ep.eps);
          const float inv1 = dh == 128 ? inv0 : 1.0f / sqrtf(ss1 / 64.0f + ep.eps);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);   // column in the wave
              acc[mt][nt][r] *= (mt < 2 ? inv0 : inv1) * nw[c % dh];
            }
        }
        if (ep.log2_theta > 0.0) {
          // rotate pair (e, e + dh/2): e in columns of mt (dh 128: mt 0, 1 with
          // partners mt + 2; dh 64: mt 0, 2 with partners mt + 1)
          const int64_t row = row0 + 64 * rg + 32 * nt + n;
          const double p = row < t ? (double)ep.pos[row] : 0.0;
#pragma unroll
          for (int pi = 0; pi < 2; ++pi) {
            const int mlo = dh == 128 ? pi : 2 * pi, mhi = dh == 128 ? pi + 2 : 2 * pi + 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int e = (dh == 128 ? 32 * pi : 0) + 8 * (r >> 2) + 4 * g + (r & 3);
              // the angle in turns, reduced to [-1/2, 1/2] in fp64; the
              // hardware sine and cosine take turns
              const double turns = p * s_turns[e];
              const float fr = (float)(turns - rint(turns));
              const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
              const float x1 = acc[mlo][nt][r], x2 = acc[mhi][nt][r];
              acc[mlo][nt][r] = x1 * cs - x2 * sn;
              acc[mhi][nt][r] = x2 * cs + x1 * sn;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int cbase = col0 + 128 * ch + 32 * mt;      // 32 columns, one destination (dh % 32 == 0)
    uint16_t* dst;
    int ld, c0;
    if (cbase < nq) {
      dst = q; ld = nq; c0 = cbase;
    } else if (cbase < nq + nkv) {
      dst = k; ld = nkv; c0 = cbase - nq;
    } else {
      dst = v; ld = nkv; c0 = cbase - nq - nkv;
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t row = row0 + 64 * rg + 32 * nt + n;
      if (row < t) {
        uint16_t* p = dst + row * ld + c0 + 4 * g;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[mt][nt][4 * r4 + 0], acc[mt][nt][4 * r4 + 1]);
          pk.y = pack_bf16x2(acc[mt][nt][4 * r4 + 2], acc[mt][nt][4 * r4 + 3]);
          *reinterpret_cast<uint2*>(p + 8 * r4) = pk;
        }
      }
    }
  }
  }
  __syncthreads();                               // LDS is restaged by the next row tile
  }
}

}  // namespace

hipError_t launch_qkv_proj(const void* x, int64_t x_row_stride, int64_t t, int d, const void* w,
                           int nq, int nkv, void* q, void* k, void* v, hipStream_t st) {
  if (t == 0) return hipSuccess;
  const int n_tot = nq + 2 * nkv;
  const dim3 grid((unsigned)((t + kTile - 1) / kTile), (unsigned)(n_tot / kTile));
  hipLaunchKernelGGL(gemm_abt_bf16<false>, grid, dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(x), x_row_stride, t, d,
                     static_cast<const uint16_t*>(w), nq, nkv, static_cast<uint16_t*>(q),
                     static_cast<uint16_t*>(k), static_cast<uint16_t*>(v), (int64_t)d, d,
                     nullptr, (int64_t)0, (int64_t)0, (int64_t)0, QkEpi{});
  return hipGetLastError();
}

hipError_t launch_qkv_proj_rope(const void* x, int64_t x_row_stride, int64_t t, int d,
                                const void* w, int nq, int nkv, int dh, const int32_t* pos,
                                const float* qn, const float* kn, float eps, float rope_theta,
                                void* q, void* k, void* v, hipStream_t st) {
  if (t == 0) return hipSuccess;
  const int n_tot = nq + 2 * nkv;
  const dim3 grid((unsigned)((t + kTile - 1) / kTile), (unsigned)(n_tot / kTile));
  // rope_theta > 1 (checked by the caller) gives log2_theta > 0; <= 0 turns RoPE off
  QkEpi ep{pos, qn, kn, eps, dh, rope_theta > 1.0f ? log2((double)rope_theta) : 0.0};
  hipLaunchKernelGGL((gemm_abt_bf16<false, false, true>), grid, dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(x), x_row_stride, t, d,
                     static_cast<const uint16_t*>(w), nq, nkv, static_cast<uint16_t*>(q),
                     static_cast<uint16_t*>(k), static_cast<uint16_t*>(v), (int64_t)d, d,
                     nullptr, (int64_t)0, (int64_t)0, (int64_t)0, ep);
  return hipGetLastError();
}

// fp32 forms: one workgroup per CU in all (the kernel holds 147 KB of LDS),
// each looping over row tiles; 0 in x when the CU count is unavailable
dim3 f32_grid(int64_t m, int n, int splits) {
  int n_cu = 0;
  if (device_cu_count(&n_cu) != hipSuccess) return dim3(0, 1, 1);
  const int64_t m_tiles = (m + kTile - 1) / kTile;
  const int64_t others = (int64_t)(n / kTile) * splits;
  int64_t gx = others > 0 ? n_cu / others : 1;
  if (gx < 1) gx = 1;
  if (gx > m_tiles) gx = m_tiles;
  return dim3((unsigned)gx, (unsigned)(n / kTile), (unsigned)splits);
}

hipError_t launch_gemm_atb_kmajor_f32(const void* a, int64_t lda, int64_t m, const void* w,
                                      int64_t ldw, int64_t k_rows, int n, int64_t kdim,
                                      int splits, float* y, int64_t ldy, hipStream_t st) {
  if (m == 0) return hipSuccess;
  if (m > kTile) return hipErrorInvalidValue;     // one row tile: X's columns are the rows of Y
  int64_t k_per = (kdim + splits - 1) / splits;
  k_per = (k_per + kBK - 1) / kBK * kBK;
  const dim3 grid = f32_grid(m, n, splits);
  if (grid.x == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_abt_bf16<true, true, false, false, true>), grid, dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(a), lda, m, (int)kdim,
                     static_cast<const uint16_t*>(w), 0, 0, nullptr, nullptr, nullptr, ldw,
                     (int)k_per, y, ldy, m * ldy, k_rows, QkEpi{}, RowCorr{});
  return hipGetLastError();
}

hipError_t launch_gemm_abt_f32(const void* x, int64_t xs, int64_t m, const void* w, int64_t ldw,
                               int n, int64_t kdim, int splits, float* y, int64_t ldy,
                               hipStream_t st, const float* rowc, const void* a, int64_t lda) {
  if (m == 0) return hipSuccess;
  if (rowc && (splits != 1 || !a || lda % 4 != 0)) return hipErrorInvalidValue;
  int64_t k_per = (kdim + splits - 1) / splits;
  k_per = (k_per + kBK - 1) / kBK * kBK;
  const dim3 grid = f32_grid(m, n, splits);
  if (grid.x == 0) return hipErrorInvalidValue;
  if (rowc)
    hipLaunchKernelGGL((gemm_abt_bf16<true, false, false, true>), grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(x), xs, m, (int)kdim,
                       static_cast<const uint16_t*>(w), 0, 0, nullptr, nullptr, nullptr, ldw,
                       (int)k_per, y, ldy, m * ldy, (int64_t)0, QkEpi{},
                       RowCorr{rowc, static_cast<const uint16_t*>(a), lda});
  else
    hipLaunchKernelGGL(gemm_abt_bf16<true>, grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(x), xs, m, (int)kdim,
                       static_cast<const uint16_t*>(w), 0, 0, nullptr, nullptr, nullptr, ldw,
                       (int)k_per, y, ldy, m * ldy, (int64_t)0, QkEpi{}, RowCorr{});
  return hipGetLastError();
}

}  // namespace tg
