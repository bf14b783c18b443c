// tg_select_topk: S_s = top-K_{j in P_s}(b_j)  U  N_s   (TokenGate §4.1 Eq. 4)
//
// Integer work on order-preserving 32-bit keys of the scores (common.h).
// Per sequence, the K'-th largest key tau (K' = min(K, |P|)) is found by a
// three-digit radix select over the key bits 31..24, 23..12 and 11..0.
// The sequence's tokens are cut into 2048-token chunks, one block each, and
// the selection runs in four launches with no cross-block handshake inside a
// launch: every block re-derives what it needs from what earlier launches
// wrote.
//
//   pass0  each chunk writes the histogram of its prunable tokens' top digit
//          (256 bins) to a record of its own, so nothing has to be zeroed
//          first; the blocks also zero the per-sequence histograms of the
//          two later digits.
//   pass1  each block adds up its sequence's chunk histograms (the sum of the
//          bins is |P|), picks the top digit of tau and how many keys are
//          still needed among those that share it, and adds the middle digit
//          of those keys into the sequence's histogram (integer atomics).
//   pass2  each block picks the middle digit from that histogram and adds
//          the low digit of the keys sharing the top 20 bits into the last
//          histogram.  It also records, per chunk, how many tokens are kept
//          whatever the low digit (prompt tokens, keys above the 20-bit
//          prefix, or every token when K' = |P|) and the low digits of the
//          tokens that share the prefix (the candidates).  One extra block
//          writes kept_cu_seqlens: a sequence keeps min(K, |P|) + |N| tokens.
//   write  each block picks the low digit, hence tau and the number `need`
//          of tokens equal to tau that are kept (lower index first).  The
//          chunk's output offset is the earlier chunks' definite keeps plus
//          their candidates above tau plus min(need, their candidates equal
//          to tau), since ties are taken in index order; then its own kept
//          tokens are written in ascending index.
#include <cstddef>
#include <mutex>

#include "common.h"

// Scratch memory of the allocation-free selector (tg_select_topk_noalloc):
// one copy per GPU, held until the process ends.  Host code never passes
// this name to a kernel: the device address comes from hipGetSymbolAddress
// (select_scratch below), once per device.
static __device__ __align__(256) unsigned char scratch[tg::kSelScratchBytes];

namespace tg {
namespace {

constexpr int CH = kSelChunk;          // tokens per block
constexpr int NT = 256;                // threads per block
constexpr int PER = CH / NT;           // tokens per thread
constexpr int NB0 = 256;               // bins of the top digit (key bits 31..24)
constexpr int NB1 = 4096;              // bins of the middle and low digits (23..12, 11..0)

enum : int { MODE_NONE = 0, MODE_ALL = 1, MODE_RADIX = 2 };

// Selection state of a sequence: digits fixed so far and how many keys are
// still to be taken among those that match them.
struct Sel {
  int mode;
  uint32_t prefix;
  uint32_t need;
  uint32_t npr;      // |P| of the sequence
};

// Per-chunk record.
constexpr int NSMALL = 28;             // candidate digits kept in the record itself
struct Slot {
  uint32_t h0[NB0];  // pass0: top-digit histogram of the chunk's prunable tokens
  uint32_t def;      // pass2: tokens kept whatever the low digit
  uint32_t ncand;    // pass2: prunable tokens whose key shares the 20-bit prefix
  uint16_t small[NSMALL];  // pass2: their low digits when ncand <= NSMALL
};
static_assert(sizeof(Slot) % 16 == 0 && offsetof(Slot, def) % 16 == 0 &&
                  sizeof(Slot) - offsetof(Slot, def) == 64,
              "slot records are read with 16-byte loads");

struct SelWs {
  Sel* stage;            // [2][n_seq]: state after the top and the middle digit
  uint32_t* n_prunable;  // [n_seq]
  uint32_t* hist1;       // [n_seq][NB1] middle digit
  uint32_t* hist2;       // [n_seq][NB1] low digit
  Slot* slot;            // [n_slots]
  uint16_t* cand;        // [n_slots][CH] low digits of the candidates
};

int64_t n_slots_of(int64_t t_in, int n_seq) { return (int64_t)n_seq + (t_in + CH - 1) / CH; }

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t ws_layout(int64_t t_in, int n_seq, size_t off[6]) {
  const size_t ns = (size_t)n_slots_of(t_in, n_seq);
  size_t p = 0;
  off[0] = p; p = align256(p + sizeof(Sel) * 2 * (size_t)n_seq);
  off[1] = p; p = align256(p + sizeof(uint32_t) * (size_t)n_seq);
  off[2] = p; p = align256(p + sizeof(uint32_t) * NB1 * (size_t)n_seq);
  off[3] = p; p = align256(p + sizeof(uint32_t) * NB1 * (size_t)n_seq);
  off[4] = p; p = align256(p + sizeof(Slot) * ns);
  off[5] = p; p = align256(p + sizeof(uint16_t) * CH * ns);
  return p;
}

SelWs carve(void* ws, int64_t t_in, int n_seq) {
  size_t off[6];
  ws_layout(t_in, n_seq, off);
  char* p = static_cast<char*>(ws);
  SelWs w;
  w.stage = reinterpret_cast<Sel*>(p + off[0]);
  w.n_prunable = reinterpret_cast<uint32_t*>(p + off[1]);
  w.hist1 = reinterpret_cast<uint32_t*>(p + off[2]);
  w.hist2 = reinterpret_cast<uint32_t*>(p + off[3]);
  w.slot = reinterpret_cast<Slot*>(p + off[4]);
  w.cand = reinterpret_cast<uint16_t*>(p + off[5]);
  return w;
}

// Token range [lo, hi) of sequence s, clamped to [0, t_in): inconsistent
// offsets cannot read out of bounds.
TG_DEVINL void seq_range(const int32_t* cu, int s, int64_t t_in, int64_t& lo, int64_t& hi) {
  lo = cu[s] < t_in ? cu[s] : t_in;
  hi = cu[s + 1] < t_in ? cu[s + 1] : t_in;
  if (lo < 0) lo = 0;
  if (hi < lo) hi = lo;
}

// Which chunk of which sequence this block handles; false if none.
struct Chunk {
  int s;
  int ci;             // chunk index within the sequence
  int64_t slot, s0;   // this block's slot and the sequence's first slot
  int64_t lo, begin, end;
};

TG_DEVINL bool locate(const int32_t* cu, int n_seq, int64_t t_in, Chunk& c) {
  c.slot = blockIdx.x;
  c.s = seq_of_slot(cu, n_seq, c.slot, CH);
  if (c.s < 0) return false;
  int64_t hi;
  seq_range(cu, c.s, t_in, c.lo, hi);
  if (hi <= c.lo) return false;
  c.s0 = slot0_of(cu, c.s, CH);
  c.ci = (int)(c.slot - c.s0);
  c.begin = c.lo + (int64_t)c.ci * CH;
  if (c.begin >= hi) return false;
  c.end = c.begin + CH < hi ? c.begin + CH : hi;
  return true;
}

TG_DEVINL int n_chunks(int64_t lo, int64_t hi) { return (int)((hi - lo + CH - 1) / CH); }

// The chunk's tokens, CH / NT per thread: thread t holds tokens
// begin + t * PER + i (contiguous, so thread order is index order).  Tokens
// past the chunk read as prompt tokens with score 0 and are flagged !in.
struct Tokens {
  float b[PER];
  uint8_t pr[PER];
  bool in[PER];
};

TG_DEVINL void load_tokens(const float* b, const uint8_t* pr, const Chunk& c, Tokens& tk) {
  const int64_t j0 = c.begin + (int64_t)threadIdx.x * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = j0 + i;
    tk.in[i] = j < c.end;
    tk.pr[i] = tk.in[i] ? pr[j] : (uint8_t)0;
    tk.b[i] = tk.in[i] ? b[j] : 0.0f;
  }
}

TG_DEVINL Sel sel_start(uint32_t npr, int kb) {
  const uint32_t k = kb > 0 ? (uint32_t)kb : 0u;
  const uint32_t kp = k < npr ? k : npr;
  Sel st;
  st.mode = kp == 0 ? MODE_NONE : (kp == npr ? MODE_ALL : MODE_RADIX);
  st.prefix = 0u;
  st.need = kp;
  st.npr = npr;
  return st;
}

// Narrow (prefix, need) with a histogram of NBINS bins given per thread (c,
// NBINS / NT bins of thread t, counted from the top: bins
// NBINS-1 - (t * per + i)).  Block-wide; every thread returns the same
// result.  Contains barriers.
template <int NBINS, int SHIFT>
TG_DEVINL void sel_narrow_vals(Sel& st, const uint32_t (&c)[NBINS / NT], int* sh) {
  constexpr int per = NBINS / NT;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) mine += (int)c[i];
  int tot;
  const int above = block_excl_scan<NT>(mine, sh, &tot);
  if ((uint32_t)above < st.need && (uint32_t)(above + mine) >= st.need) {
    uint32_t acc = (uint32_t)above;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (acc + c[i] >= st.need) {
        sh[NT / 64] = NBINS - 1 - (threadIdx.x * per + i);
        sh[NT / 64 + 1] = (int)(st.need - acc);
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  st.prefix = (st.prefix << SHIFT) | (uint32_t)sh[NT / 64];
  st.need = (uint32_t)sh[NT / 64 + 1];
  __syncthreads();
}

// A histogram in global memory, read with coalesced 16-byte loads.  The
// loads are issued as soon as the sequence is known, next to the block's
// other independent loads, so they do not add a round trip after the
// selection state arrives.
template <int NBINS>
struct HistRegs {
  u32x4 v[NBINS / 4 / NT];                     // 16-byte vectors of this thread
};
template <int NBINS>
TG_DEVINL void hist_load(const uint32_t* h, HistRegs<NBINS>& r) {
#pragma unroll
  for (int k = 0; k < NBINS / 4 / NT; ++k) r.v[k] = ld16(h + 4 * (threadIdx.x + k * NT));
}

// Narrow with such a histogram: its vectors go to LDS (stage, NBINS words,
// 16-byte aligned), then each thread takes its NBINS / NT bins from there.
template <int NBINS, int SHIFT>
TG_DEVINL void sel_narrow(Sel& st, const HistRegs<NBINS>& r, uint32_t* stage, int* sh) {
  constexpr int per = NBINS / NT;
#pragma unroll
  for (int k = 0; k < NBINS / 4 / NT; ++k) st16(stage + 4 * (threadIdx.x + k * NT), r.v[k]);
  __syncthreads();
  uint32_t c[per];
#pragma unroll
  for (int i = 0; i < per; ++i) c[i] = stage[NBINS - 1 - (threadIdx.x * per + i)];
  sel_narrow_vals<NBINS, SHIFT>(st, c, sh);     // starts with a barrier-protected scan
}

// Block-wide sums of three per-thread counts, every thread gets all three:
// one exchange of the wave totals (sh3: 3 * NT / 64 ints, not reused by the
// caller afterwards, so a single barrier suffices).
TG_DEVINL void block_sum3(int& a, int& b, int& c, int* sh3) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b), ic = wave_incl_scan(c);
  if (lane == 63) {
    sh3[w] = ia;
    sh3[NW + w] = ib;
    sh3[2 * NW + w] = ic;
  }
  __syncthreads();
  a = b = c = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    a += sh3[i];
    b += sh3[NW + i];
    c += sh3[2 * NW + i];
  }
}

// ---------------------------------------------------------------- pass 0
__global__ __launch_bounds__(NT) void sel_pass0(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu, int n_seq,
                                               int64_t t_in, SelWs w) {
  __shared__ uint32_t lh[NB0];
  // zero the later digits' histograms of every sequence (read-modify-written
  // by pass1 and pass2, which start after this launch ends)
  {
    const int64_t n = (int64_t)n_seq * NB1;
    const int64_t gsz = (int64_t)gridDim.x * NT;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += gsz) {
      w.hist1[i] = 0u;
      w.hist2[i] = 0u;
    }
  }
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  Tokens tk;
  load_tokens(b, pr, c, tk);
  lh[threadIdx.x] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (tk.pr[i]) atomicAdd(&lh[score_key(tk.b[i]) >> 24], 1u);
  __syncthreads();
  w.slot[c.slot].h0[threadIdx.x] = lh[threadIdx.x];
}

// State after the top digit: the chunk histograms of the sequence added up
// (integer sums, so every block of the sequence gets the same result).
// Thread t adds bins 4 (t % 64) .. +4 of every fourth chunk starting at
// t / 64, eight 16-byte loads in flight at a time; the four partial sums of
// a bin meet in LDS (red4: [4][NB0]).
TG_DEVINL Sel stage0(const SelWs& w, int kb, const Chunk& c, int nch, int64_t ns,
                     uint32_t* red4, int* sh) {
  const int vi = threadIdx.x & 63, cp = threadIdx.x >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int base = cp; base < nch; base += 64) {
    u32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int64_t sl = c.s0 + base + 4 * k;
      v[k] = (base + 4 * k < nch && sl >= 0 && sl < ns) ? ld16(&w.slot[sl].h0[4 * vi])
                                                       : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) acc += v[k];
  }
  *reinterpret_cast<u32x4*>(&red4[cp * NB0 + 4 * vi]) = acc;
  __syncthreads();
  const uint32_t v = red4[threadIdx.x] + red4[NB0 + threadIdx.x] + red4[2 * NB0 + threadIdx.x] +
                     red4[3 * NB0 + threadIdx.x];
  __syncthreads();
  red4[threadIdx.x] = v;
  int tot;
  block_excl_scan<NT>((int)v, sh, &tot);
  uint32_t* red = red4;
  Sel st = sel_start((uint32_t)tot, kb);
  if (st.mode == MODE_RADIX) {
    uint32_t cv[NB0 / NT];
#pragma unroll
    for (int i = 0; i < NB0 / NT; ++i) cv[i] = red[NB0 - 1 - (threadIdx.x * (NB0 / NT) + i)];
    sel_narrow_vals<NB0, 8>(st, cv, sh);
  }
  return st;
}

// ---------------------------------------------------------------- pass 1
__global__ __launch_bounds__(NT) void sel_pass1(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu,
                                               const int32_t* __restrict__ kbud, int n_seq,
                                               int64_t t_in, SelWs w) {
  __shared__ uint32_t lh[NB1];
  __shared__ __attribute__((aligned(16))) uint32_t red4[4 * NB0];
  __shared__ int sh[NT / 64 + 2];
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  const int kb = kbud[c.s];
  Tokens tk;
  load_tokens(b, pr, c, tk);              // issued before the histogram sums
  // the middle-digit histogram starts at zero; stage0's barriers order these
  // stores before the atomics below
  for (int i = threadIdx.x; i < NB1; i += NT) lh[i] = 0u;
  int64_t lo, hi;
  seq_range(cu, c.s, t_in, lo, hi);
  const Sel st = stage0(w, kb, c, n_chunks(lo, hi), (int64_t)gridDim.x, red4, sh);
  if (c.ci == 0 && threadIdx.x == 0) {
    w.stage[c.s] = st;
    w.n_prunable[c.s] = st.npr;
  }
  if (st.mode != MODE_RADIX) return;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (tk.pr[i]) {
      const uint32_t key = score_key(tk.b[i]);
      if ((key >> 24) == st.prefix) atomicAdd(&lh[(key >> 12) & 0xfffu], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = w.hist1 + (size_t)c.s * NB1;
  for (int i = threadIdx.x; i < NB1; i += NT) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(gh + i, v);
  }
}

// ---------------------------------------------------------------- pass 2
__global__ __launch_bounds__(NT) void sel_pass2(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu,
                                               const int32_t* __restrict__ kbud, int n_seq,
                                               int64_t t_in, SelWs w,
                                               int32_t* __restrict__ kept_cu) {
  __shared__ __attribute__((aligned(16))) uint32_t lh[NB1];   // staging of the middle digit
  __shared__ uint32_t lc[NB1];                                 // low digits of the candidates
  __shared__ int sh[NT / 64 + 2];
  __shared__ uint32_t ncand;
  if (blockIdx.x == gridDim.x - 1) {
    // the launch's extra last block, which meets no chunk: kept_cu[s] = sum
    // over earlier sequences of min(K, |P|) + |N|; an empty sequence was
    // seen by no pass1 block and has |P| = 0
    int acc = 0;
    for (int base = 0; base < n_seq; base += NT) {
      const int i = base + threadIdx.x;
      int v = 0;
      if (i < n_seq) {
        int64_t lo, hi;
        seq_range(cu, i, t_in, lo, hi);
        const int npr = hi > lo ? (int)w.n_prunable[i] : 0;
        const int kb = kbud[i] > 0 ? kbud[i] : 0;
        v = (kb < npr ? kb : npr) + (int)(hi - lo) - npr;
      }
      int tot;
      const int ex = block_excl_scan<NT>(v, sh, &tot);
      if (i < n_seq) kept_cu[i] = acc + ex;
      acc += tot;
    }
    if (threadIdx.x == 0) kept_cu[n_seq] = acc;
    return;
  }
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  Tokens tk;
  load_tokens(b, pr, c, tk);
  HistRegs<NB1> hr;
  hist_load<NB1>(w.hist1 + (size_t)c.s * NB1, hr);    // zeros unless the mode is RADIX
  // the candidates' histogram and count start at zero; the narrowing's
  // barriers order these stores before the atomics below (which only the
  // RADIX mode, where it runs, makes), and thread 0 reads ncand itself
  for (int i = threadIdx.x; i < NB1; i += NT) lc[i] = 0u;
  if (threadIdx.x == 0) ncand = 0u;
  Sel st = w.stage[c.s];
  if (st.mode == MODE_RADIX) sel_narrow<NB1, 12>(st, hr, lh, sh);
  if (c.ci == 0 && threadIdx.x == 0) w.stage[n_seq + c.s] = st;
  uint16_t* cl = w.cand + (size_t)c.slot * CH;
  int def = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (!tk.in[i]) continue;
    if (!tk.pr[i] || st.mode == MODE_ALL) {
      ++def;
    } else if (st.mode == MODE_RADIX) {
      const uint32_t key = score_key(tk.b[i]);
      const uint32_t hi20 = key >> 12;
      if (hi20 > st.prefix) {
        ++def;
      } else if (hi20 == st.prefix) {
        const uint32_t d = key & 0xfffu;
        atomicAdd(&lc[d], 1u);
        const uint32_t at = atomicAdd(&ncand, 1u);   // at most CH candidates per chunk
        cl[at] = (uint16_t)d;
        if (at < (uint32_t)NSMALL) w.slot[c.slot].small[at] = (uint16_t)d;
      }
    }
  }
  int td;
  block_excl_scan<NT>(def, sh, &td);                  // contains barriers
  if (threadIdx.x == 0) {
    w.slot[c.slot].def = (uint32_t)td;
    w.slot[c.slot].ncand = ncand;
  }
  if (st.mode == MODE_RADIX) {
    uint32_t* gh = w.hist2 + (size_t)c.s * NB1;
    for (int i = threadIdx.x; i < NB1; i += NT) {
      const uint32_t v = lc[i];
      if (v) atomicAdd(gh + i, v);
    }
  }
}

// ----------------------------------------------------------------- write
__global__ __launch_bounds__(NT) void sel_write(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu, int n_seq,
                                               int64_t t_in, SelWs w,
                                               const int32_t* __restrict__ kept_cu, int64_t cap,
                                               int32_t* __restrict__ kept_idx,
                                               int32_t* __restrict__ kept_pos,
                                               float* __restrict__ kept_b) {
  __shared__ __attribute__((aligned(16))) uint32_t hs[NB1];
  __shared__ int sh[NT / 64 + 2];
  __shared__ int sh3[3 * (NT / 64)];
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  Tokens tk;
  load_tokens(b, pr, c, tk);
  HistRegs<NB1> hr;
  hist_load<NB1>(w.hist2 + (size_t)c.s * NB1, hr);    // zeros unless the mode is RADIX
  // The earlier chunks of the sequence, one thread each: def, ncand and the
  // short candidate list, the record's last 64 bytes.  The first NT records
  // are loaded here, beside the histogram, before the state is known.
  auto rec_ok = [&](int i) {
    const int64_t sl = c.s0 + i;
    return i < c.ci && sl >= 0 && sl < (int64_t)gridDim.x;
  };
  auto rec_load = [&](int i, u32x4 (&t4)[4]) {
    const u32x4* tail = reinterpret_cast<const u32x4*>(&w.slot[c.s0 + i].def);
#pragma unroll
    for (int k = 0; k < 4; ++k) t4[k] = ld16(tail + k);
  };
  u32x4 r0[4];
  const bool has0 = rec_ok(threadIdx.x);
  if (has0) rec_load(threadIdx.x, r0);
  const int64_t kept0 = kept_cu[c.s];
  Sel st = w.stage[n_seq + c.s];
  if (st.mode == MODE_RADIX) sel_narrow<NB1, 12>(st, hr, hs, sh);
  const uint32_t tau = st.prefix;                  // the K'-th largest key (RADIX)
  const uint32_t d2 = tau & 0xfffu;
  const int need = st.mode == MODE_RADIX ? (int)st.need : 0;
  // definite keeps, candidates above tau and candidates equal to tau of the
  // earlier chunks (a long candidate list is read 32 digits at a time, four
  // 16-byte loads in flight)
  int dsum = 0, gsum = 0, tsum = 0;
  auto rec_count = [&](int i, const u32x4 (&t4)[4]) {
    dsum += (int)t4[0][0];
    if (st.mode != MODE_RADIX) return;
    const int n = (int)(t4[0][1] < (uint32_t)CH ? t4[0][1] : (uint32_t)CH);
    if (n <= NSMALL) {
#pragma unroll
      for (int m = 0; m < NSMALL; ++m) {
        const uint32_t wd = t4[(2 + m / 2) / 4][(2 + m / 2) % 4];
        const uint32_t d = (wd >> (16 * (m & 1))) & 0xffffu;
        gsum += m < n && d > d2;
        tsum += m < n && d == d2;
      }
      return;
    }
    const uint16_t* cl = w.cand + (size_t)(c.s0 + i) * CH;
    for (int e0 = 0; e0 < n; e0 += 32) {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[k] = e0 + 8 * k < n ? ld16(cl + e0 + 8 * k) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t d = (v[k][m >> 1] >> (16 * (m & 1))) & 0xffffu;
          const bool ok = e0 + 8 * k + m < n;
          gsum += ok && d > d2;
          tsum += ok && d == d2;
        }
    }
  };
  if (has0) rec_count(threadIdx.x, r0);
  for (int i = threadIdx.x + NT; i < c.ci; i += NT) {
    if (!rec_ok(i)) continue;
    u32x4 t4[4];
    rec_load(i, t4);
    rec_count(i, t4);
  }
  block_sum3(dsum, gsum, tsum, sh3);
  const int tot_d = dsum, tot_g = gsum, tot_t = tsum;
  const int tie_base = tot_t;
  const int64_t out_base = kept0 + tot_d + tot_g + (tot_t < need ? tot_t : need);
  uint8_t fl[PER];     // 1: kept for sure, 2: tie at tau
  int nt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    uint8_t f = 0;
    if (tk.in[i]) {
      if (!tk.pr[i] || st.mode == MODE_ALL) {
        f = 1;
      } else if (st.mode == MODE_RADIX) {
        const uint32_t key = score_key(tk.b[i]);
        f = key > tau ? 1 : (key == tau ? 2 : 0);
      }
    }
    fl[i] = f;
    nt += f >> 1;
  }
  int tt;
  int trank = tie_base + block_excl_scan<NT>(nt, sh, &tt);
  int nk = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (fl[i] == 2) {
      fl[i] = trank < need ? 1 : 0;
      ++trank;
    }
    nk += fl[i];
  }
  int tk_tot;
  int64_t o = out_base + block_excl_scan<NT>(nk, sh, &tk_tot);
  const int64_t j0 = c.begin + (int64_t)threadIdx.x * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (fl[i]) {
      if (o >= 0 && o < cap) {
        kept_idx[o] = (int32_t)(j0 + i);
        if (kept_pos) kept_pos[o] = (int32_t)(j0 + i - c.lo);
        if (kept_b) kept_b[o] = tk.b[i];
      }
      ++o;
    }
  }
}

}  // namespace

hipError_t select_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t select_ws_bytes(int64_t t_in, int n_seq) {
  size_t off[6];
  return ws_layout(t_in, n_seq, off);
}

hipError_t launch_select(const float* b, const uint8_t* prunable, const int32_t* cu,
                         const int32_t* k, int n_seq, int64_t t_in, int64_t cap,
                         int32_t* kept_idx, int32_t* kept_pos, float* kept_b, int32_t* kept_cu,
                         void* ws, hipStream_t st) {
  SelWs w = carve(ws, t_in, n_seq);
  const int64_t ns = n_slots_of(t_in, n_seq);
  const dim3 grid((unsigned)ns);
  if (t_in > 0) {
    hipLaunchKernelGGL(sel_pass0, grid, dim3(NT), 0, st, b, prunable, cu, n_seq, t_in, w);
    hipLaunchKernelGGL(sel_pass1, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w);
  }
  // every sequence's kept_cu entry is written by the extra last block, also
  // when t_in == 0 (the pass1 state it reads is then never used: every
  // sequence is empty); slot ns lies past every chunk
  hipLaunchKernelGGL(sel_pass2, dim3((unsigned)(ns + 1)), dim3(NT), 0, st, b, prunable, cu, k,
                     n_seq, t_in, w, kept_cu);
  if (t_in > 0)
    hipLaunchKernelGGL(sel_write, grid, dim3(NT), 0, st, b, prunable, cu, n_seq, t_in, w, kept_cu,
                       cap, kept_idx, kept_pos, kept_b);
  return hipGetLastError();
}

}  // namespace tg
