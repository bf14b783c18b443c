// tg_select_topk: S_s = top-K_{j in P_s}(b_j)  U  N_s   (TokenGate §4.1 Eq. 4)
//
// Integer work on order-preserving 32-bit keys of the scores (common.h).
// Per sequence, the K'-th largest key tau is found by a three-pass radix
// select over 11/11/10-bit digits.  Each pass is one launch over all
// 2048-token chunks of all sequences: a chunk's histogram is built in LDS and
// added into the sequence's histogram for that pass with integer atomics.
// There is no cross-block handshake inside a launch: every block of the next
// launch re-derives the digits fixed so far from the (small) histograms of
// the earlier passes, so all blocks reach the same tau and quota without
// fences.  Then every token is kept if it is a prompt token, if key > tau, or
// if key == tau and fewer than `need` earlier tokens of the sequence tie at
// tau (lower index wins).  The kept count of a sequence, min(K, |P|) + |N|,
// is known from the prunable count alone, so sequence offsets need no scan
// of the selection itself; a chunk's offset is the sum of the definite keeps
// of the earlier chunks of its sequence plus min(need, their ties).  Tokens
// are written in ascending original index.
//
// Launches: init, pass0, pass1, pass2, count (+ kept_cu), write (each block
// derives its chunk's offsets from the counts of the earlier chunks).
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
constexpr int NB = 2048;               // histogram bins (11-bit digit)
constexpr int HIST_WORDS = 2048 + 2048 + 1024;   // the three passes' histograms

enum : int { MODE_NONE = 0, MODE_ALL = 1, MODE_RADIX = 2 };

// Selection state of a sequence as derived by one block.
struct Sel {
  int mode;
  uint32_t prefix;   // digits fixed so far (tau after three passes)
  uint32_t need;     // keys still to take among those matching the prefix
  uint32_t pad;
};

struct SelWs {
  Sel* stage;            // [3][n_seq]: state after 1, 2 and 3 digits
  uint32_t* hist;        // [n_seq][HIST_WORDS]
  uint32_t* n_prunable;  // [n_seq]
  int32_t* blk_def;      // [n_slots] kept for sure (prompt, key > tau, or all)
  int32_t* blk_tie;      // [n_slots] prunable tokens with key == tau
};

int64_t n_slots_of(int64_t t_in, int n_seq) { return (int64_t)n_seq + (t_in + CH - 1) / CH; }

SelWs carve(void* ws, int64_t t_in, int n_seq) {
  const int64_t ns = n_slots_of(t_in, n_seq);
  char* p = static_cast<char*>(ws);
  SelWs w;
  w.stage = reinterpret_cast<Sel*>(p);
  p += sizeof(Sel) * 3 * (size_t)n_seq;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * (size_t)n_seq * HIST_WORDS;
  w.n_prunable = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * (size_t)n_seq;
  w.blk_def = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * ns;
  w.blk_tie = reinterpret_cast<int32_t*>(p);
  return w;
}

// Token range [lo, hi) of sequence s, clamped to [0, t_in): inconsistent
// offsets cannot read out of bounds.
TG_DEVINL void seq_range(const int32_t* cu, int s, int64_t t_in, int64_t& lo, int64_t& hi) {
  lo = cu[s] < t_in ? cu[s] : t_in;
  hi = cu[s + 1] < t_in ? cu[s + 1] : t_in;
  if (hi < lo) hi = lo;
}

// Which chunk of which sequence this block handles; false if none.
struct Chunk {
  int s;
  int64_t slot, lo, begin, end;
};

TG_DEVINL bool locate(const int32_t* cu, int n_seq, int64_t t_in, Chunk& c) {
  c.slot = blockIdx.x;
  c.s = seq_of_slot(cu, n_seq, c.slot, CH);
  if (c.s < 0) return false;
  int64_t hi;
  seq_range(cu, c.s, t_in, c.lo, hi);
  if (hi <= c.lo) return false;
  c.begin = c.lo + (c.slot - slot0_of(cu, c.s, CH)) * CH;
  if (c.begin >= hi) return false;
  c.end = c.begin + CH < hi ? c.begin + CH : hi;
  return true;
}

TG_DEVINL Sel sel_start(const SelWs& w, const int32_t* kbud, int s) {
  const uint32_t npr = w.n_prunable[s];
  const int kb = kbud[s];
  const uint32_t k = kb > 0 ? (uint32_t)kb : 0u;
  const uint32_t kp = k < npr ? k : npr;
  Sel st;
  st.mode = kp == 0 ? MODE_NONE : (kp == npr ? MODE_ALL : MODE_RADIX);
  st.prefix = 0u;
  st.need = kp;
  st.pad = 0u;
  return st;
}

// Narrow (prefix, need) with the histogram `h` of NBINS bins (block-wide;
// every thread returns the same result).  Contains barriers.
template <int NBINS, int SHIFT>
TG_DEVINL void sel_narrow(Sel& st, const uint32_t* h, int* sh) {
  constexpr int per = NBINS / NT;
  uint32_t c[per];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    c[i] = h[NBINS - 1 - (threadIdx.x * per + i)];    // bins in descending order
    mine += (int)c[i];
  }
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

// State after `digits` digits (1..3): the state stored by the previous
// launch after digits-1 digits, narrowed once more with histogram digits-1.
// The block of chunk 0 stores the result for the next launch (each launch
// writes a different stage, so no block reads a slot being written).
TG_DEVINL Sel sel_stage(const SelWs& w, const int32_t* kbud, int s, int n_seq, int digits,
                        bool store, int* sh) {
  Sel st = digits == 1 ? sel_start(w, kbud, s) : w.stage[(size_t)(digits - 2) * n_seq + s];
  if (st.mode == MODE_RADIX) {
    const uint32_t* hs = w.hist + (size_t)s * HIST_WORDS;
    if (digits == 1) sel_narrow<2048, 11>(st, hs, sh);
    else if (digits == 2) sel_narrow<2048, 11>(st, hs + 2048, sh);
    else sel_narrow<1024, 10>(st, hs + 4096, sh);
  }
  if (store && threadIdx.x == 0) w.stage[(size_t)(digits - 1) * n_seq + s] = st;
  return st;
}

__global__ __launch_bounds__(NT) void sel_init(int n_seq, SelWs w) {
  const int64_t gtid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t gsz = (int64_t)gridDim.x * NT;
  for (int64_t i = gtid; i < (int64_t)n_seq * HIST_WORDS; i += gsz) w.hist[i] = 0u;
  for (int64_t i = gtid; i < n_seq; i += gsz) w.n_prunable[i] = 0u;
}

template <int P>
__global__ __launch_bounds__(NT) void sel_pass(const float* __restrict__ b,
                                              const uint8_t* __restrict__ pr,
                                              const int32_t* __restrict__ cu,
                                              const int32_t* __restrict__ kbud, int n_seq,
                                              int64_t t_in, SelWs w) {
  __shared__ uint32_t lh[NB];
  __shared__ int sh[NT / 64 + 2];
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  uint32_t* hs = w.hist + (size_t)c.s * HIST_WORDS;
  Sel st = {MODE_RADIX, 0u, 0u, 0u};
  if (P > 0) {
    st = sel_stage(w, kbud, c.s, n_seq, P, c.begin == c.lo, sh);
    if (st.mode != MODE_RADIX) return;
  }
  for (int i = threadIdx.x; i < NB; i += NT) lh[i] = 0u;
  __syncthreads();
  // all loads first (one memory latency per thread, not one per token)
  uint8_t pv[PER];
  float bv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = c.begin + threadIdx.x + (int64_t)i * NT;
    pv[i] = j < c.end ? pr[j] : (uint8_t)0;
    bv[i] = j < c.end ? b[j] : 0.0f;
  }
  int np = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (pv[i]) {
      const uint32_t key = score_key(bv[i]);
      ++np;
      if (P == 0) {
        atomicAdd(&lh[key >> 21], 1u);
      } else if (P == 1) {
        if ((key >> 21) == st.prefix) atomicAdd(&lh[(key >> 10) & 0x7ffu], 1u);
      } else {
        if ((key >> 10) == st.prefix) atomicAdd(&lh[key & 0x3ffu], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = hs + (P == 0 ? 0 : (P == 1 ? 2048 : 4096));
  for (int i = threadIdx.x; i < (P == 2 ? 1024 : 2048); i += NT) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(gh + i, v);
  }
  if (P == 0) {
    np = wave_sum(np);
    if ((threadIdx.x & 63) == 0 && np) atomicAdd(&w.n_prunable[c.s], (uint32_t)np);
  }
}

__global__ __launch_bounds__(NT) void sel_count(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu,
                                               const int32_t* __restrict__ kbud, int n_seq,
                                               int64_t t_in, SelWs w,
                                               int32_t* __restrict__ kept_cu) {
  __shared__ int sh[NT / 64 + 2];
  if (blockIdx.x == 0) {
    // kept_cu[s] = sum over earlier sequences of min(K, |P|) + |N|
    int acc = 0;
    for (int base = 0; base < n_seq; base += NT) {
      const int i = base + threadIdx.x;
      int v = 0;
      if (i < n_seq) {
        int64_t lo, hi;
        seq_range(cu, i, t_in, lo, hi);
        const int npr = (int)w.n_prunable[i];
        const int kb = kbud[i] > 0 ? kbud[i] : 0;
        v = (kb < npr ? kb : npr) + (int)(hi - lo) - npr;
      }
      int tot;
      const int ex = block_excl_scan<NT>(v, sh, &tot);
      if (i < n_seq) kept_cu[i] = acc + ex;
      acc += tot;
    }
    if (threadIdx.x == 0) kept_cu[n_seq] = acc;
  }
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  const Sel st = sel_stage(w, kbud, c.s, n_seq, 3, c.begin == c.lo, sh);
  uint8_t pv[PER], in[PER];
  float bv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = c.begin + threadIdx.x + (int64_t)i * NT;
    in[i] = j < c.end;
    pv[i] = j < c.end ? pr[j] : (uint8_t)0;
    bv[i] = j < c.end ? b[j] : 0.0f;
  }
  int def = 0, tie = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (in[i]) {
      if (!pv[i] || st.mode == MODE_ALL) {
        ++def;
      } else if (st.mode == MODE_RADIX) {
        const uint32_t key = score_key(bv[i]);
        def += key > st.prefix;
        tie += key == st.prefix;
      }
    }
  }
  int td, tt;
  block_excl_scan<NT>(def, sh, &td);
  block_excl_scan<NT>(tie, sh, &tt);
  if (threadIdx.x == 0) {
    w.blk_def[c.slot] = td;
    w.blk_tie[c.slot] = tt;
  }
}

__global__ __launch_bounds__(NT) void sel_write(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu,
                                               const int32_t* __restrict__ kbud, int n_seq,
                                               int64_t t_in, SelWs w,
                                               const int32_t* __restrict__ kept_cu, int64_t cap,
                                               int32_t* __restrict__ kept_idx,
                                               int32_t* __restrict__ kept_pos,
                                               float* __restrict__ kept_b) {
  __shared__ int sh[NT / 64 + 2];
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  const Sel st = w.stage[2 * (size_t)n_seq + c.s];
  const int need = st.mode == MODE_RADIX ? (int)st.need : 0;
  // offsets of this chunk inside its sequence from the counts of the earlier
  // chunks: ties are taken greedily in chunk order, so the earlier chunks
  // took min(need, their ties) tied tokens in total
  const int64_t s0 = slot0_of(cu, c.s, CH);
  const int ci = (int)(c.slot - s0);
  int dsum = 0, tsum = 0;
  for (int i = threadIdx.x; i < ci; i += NT) {
    dsum += w.blk_def[s0 + i];
    tsum += w.blk_tie[s0 + i];
  }
  int tot_d, tot_t;
  block_excl_scan<NT>(dsum, sh, &tot_d);
  block_excl_scan<NT>(tsum, sh, &tot_t);
  const int tie_base = tot_t;
  const int64_t out_base = (int64_t)kept_cu[c.s] + tot_d + (tot_t < need ? tot_t : need);
  // contiguous tokens per thread, so thread order is index order
  const int64_t j0 = c.begin + (int64_t)threadIdx.x * PER;
  float bv[PER];
  uint8_t fl[PER];     // 1: kept for sure, 2: tie at tau
  int nt = 0;
  uint8_t pv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = j0 + i;
    pv[i] = j < c.end ? pr[j] : (uint8_t)0;
    bv[i] = j < c.end ? b[j] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = j0 + i;
    uint8_t f = 0;
    const float v = bv[i];
    if (j < c.end) {
      if (!pv[i] || st.mode == MODE_ALL) {
        f = 1;
      } else if (st.mode == MODE_RADIX) {
        const uint32_t key = score_key(v);
        f = key > st.prefix ? 1 : (key == st.prefix ? 2 : 0);
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
  int tk;
  int64_t o = out_base + block_excl_scan<NT>(nk, sh, &tk);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (fl[i]) {
      if (o < cap) {
        kept_idx[o] = (int32_t)(j0 + i);
        if (kept_pos) kept_pos[o] = (int32_t)(j0 + i - c.lo);
        if (kept_b) kept_b[o] = bv[i];
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
  const int64_t ns = n_slots_of(t_in, n_seq);
  size_t bytes = sizeof(Sel) * 3 * (size_t)n_seq + sizeof(uint32_t) * (size_t)n_seq * HIST_WORDS +
                 sizeof(uint32_t) * (size_t)n_seq + 2 * sizeof(int32_t) * (size_t)ns;
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_select(const float* b, const uint8_t* prunable, const int32_t* cu,
                         const int32_t* k, int n_seq, int64_t t_in, int64_t cap,
                         int32_t* kept_idx, int32_t* kept_pos, float* kept_b, int32_t* kept_cu,
                         void* ws, hipStream_t st) {
  SelWs w = carve(ws, t_in, n_seq);
  const int64_t ns = n_slots_of(t_in, n_seq);
  int64_t init_blocks = ((int64_t)n_seq * HIST_WORDS + NT - 1) / NT;
  if (init_blocks > 1024) init_blocks = 1024;
  hipLaunchKernelGGL(sel_init, dim3((unsigned)init_blocks), dim3(NT), 0, st, n_seq, w);
  const dim3 grid((unsigned)ns);
  if (t_in > 0) {
    hipLaunchKernelGGL(sel_pass<0>, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w);
    hipLaunchKernelGGL(sel_pass<1>, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w);
    hipLaunchKernelGGL(sel_pass<2>, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w);
  }
  // every sequence's kept_cu entry is written by block 0 even when t_in == 0
  hipLaunchKernelGGL(sel_count, dim3((unsigned)(ns > 0 ? ns : 1)), dim3(NT), 0, st, b, prunable, cu,
                     k, n_seq, t_in, w, kept_cu);
  if (t_in > 0)
    hipLaunchKernelGGL(sel_write, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w,
                       kept_cu, cap, kept_idx, kept_pos, kept_b);
  return hipGetLastError();
}

}  // namespace tg
