// tg_select_topk: S_s = top-K_{j in P_s}(b_j)  U  N_s   (TokenGate §4.1 Eq. 4)
//
// Integer work on order-preserving 32-bit keys of the scores (common.h).
// Per sequence, the K'-th largest key tau is found by a three-pass radix
// select over 11/11/10-bit digits; each pass is one launch over all 2048-token
// chunks of all sequences, histograms go from LDS to global with integer
// atomics, and the block that arrives last for a sequence narrows the digit
// (no spinning, no float atomics, so the result is exact and reproducible).
// Then every token is kept if it is a prompt token, if key > tau, or if
// key == tau and fewer than `need` earlier tokens of the sequence tie at tau
// (lower index wins).  Two more launches count and write the kept tokens in
// ascending original index.
//
// Launch sequence: init, pass0, pass1, pass2, count, write.
#include "common.h"

namespace tg {
namespace {

constexpr int CH = kSelChunk;          // tokens per block
constexpr int NT = 256;                // threads per block
constexpr int PER = CH / NT;           // tokens per thread
constexpr int NB = 2048;               // histogram bins (11-bit digit)

enum : int { MODE_NONE = 0, MODE_ALL = 1, MODE_RADIX = 2 };

struct SeqState {
  uint32_t n_prunable;   // |P_s| (pass 0 atomics)
  uint32_t arrive;       // blocks of this sequence done with the current launch
  uint32_t prefix;       // digits fixed so far; tau after pass 2
  uint32_t need;         // keys still to take at the current prefix
  int32_t mode;
  int32_t kept_total;    // |S_s|
  int32_t pad[2];
};

struct SelWs {
  SeqState* st;          // [n_seq]
  uint32_t* hist;        // [n_seq][NB]
  int32_t* blk_def;      // [n_slots] kept for sure (prompt, key > tau, or all)
  int32_t* blk_tie;      // [n_slots] prunable tokens with key == tau
  int32_t* blk_tie_off;  // [n_slots] ties in earlier chunks of the sequence
  int32_t* blk_off;      // [n_slots] kept tokens in earlier chunks
  uint32_t* globals;     // [0] sequences counted, [1] non-empty sequences
};

int64_t n_slots_of(int64_t t_in, int n_seq) { return (int64_t)n_seq + (t_in + CH - 1) / CH; }

SelWs carve(void* ws, int64_t t_in, int n_seq) {
  const int64_t ns = n_slots_of(t_in, n_seq);
  char* p = static_cast<char*>(ws);
  SelWs w;
  w.st = reinterpret_cast<SeqState*>(p);
  p += sizeof(SeqState) * (size_t)n_seq;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * (size_t)n_seq * NB;
  w.blk_def = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * ns;
  w.blk_tie = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * ns;
  w.blk_tie_off = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * ns;
  w.blk_off = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * ns;
  w.globals = reinterpret_cast<uint32_t*>(p);
  return w;
}

// Which chunk of which sequence this block handles; false if none.
struct Chunk {
  int s;
  int64_t slot, begin, end;
  int nchunks;
};

TG_DEVINL bool locate(const int32_t* cu, int n_seq, int64_t t_in, Chunk& c) {
  c.slot = blockIdx.x;
  c.s = seq_of_slot(cu, n_seq, c.slot, CH);
  if (c.s < 0) return false;
  // token ranges are clamped to [0, t_in): inconsistent offsets cannot read out of bounds
  const int64_t lo = cu[c.s] < t_in ? cu[c.s] : t_in;
  const int64_t hi = cu[c.s + 1] < t_in ? cu[c.s + 1] : t_in;
  if (hi <= lo) return false;
  const int64_t ci = c.slot - slot0_of(cu, c.s, CH);
  c.begin = lo + ci * CH;
  if (c.begin >= hi) return false;
  c.end = c.begin + CH < hi ? c.begin + CH : hi;
  c.nchunks = (int)((hi - lo + CH - 1) / CH);
  return true;
}

// Block-uniform "am I the last block of sequence s for this launch?".
TG_DEVINL bool arrive_last(SeqState* st, int nchunks, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t old = __hip_atomic_fetch_add(&st->arrive, 1u, __ATOMIC_ACQ_REL,
                                          __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == (uint32_t)nchunks - 1);
  }
  __syncthreads();
  const bool last = *flag;
  if (last) __threadfence();
  return last;
}

__global__ __launch_bounds__(NT) void sel_init(const int32_t* __restrict__ cu, int n_seq,
                                              int64_t t_in, SelWs w,
                                              int32_t* __restrict__ kept_cu) {
  const int64_t gtid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t gsz = (int64_t)gridDim.x * NT;
  for (int64_t i = gtid; i < (int64_t)n_seq * NB; i += gsz) w.hist[i] = 0u;
  for (int64_t i = gtid; i < n_seq; i += gsz) {
    SeqState z = {};
    w.st[i] = z;
  }
  for (int64_t i = gtid; i <= n_seq; i += gsz) kept_cu[i] = 0;
  if (blockIdx.x == 0) {
    __shared__ int red[NT / 64];
    int cnt = 0;
    for (int s = threadIdx.x; s < n_seq; s += NT) {
      const int64_t lo = cu[s] < t_in ? cu[s] : t_in;
      const int64_t hi = cu[s + 1] < t_in ? cu[s + 1] : t_in;
      cnt += hi > lo ? 1 : 0;
    }
    cnt = wave_sum(cnt);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int i = 0; i < NT / 64; ++i) tot += red[i];
      w.globals[0] = 0u;
      w.globals[1] = (uint32_t)tot;
    }
  }
}

// After pass `P`, narrow (prefix, need) from the histogram of sequence s.
template <int P>
TG_DEVINL void narrow(SeqState* st, uint32_t* ghist, int* sh) {
  constexpr int nb = (P == 2) ? 1024 : 2048;
  constexpr int per = nb / NT;
  const uint32_t need = st->need;
  uint32_t c[per];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int bin = nb - 1 - (threadIdx.x * per + i);
    c[i] = ld_acquire_u32(ghist + bin);
    mine += (int)c[i];
  }
  int tot;
  int above = block_excl_scan<NT>(mine, sh, &tot);
  if ((uint32_t)above < need && (uint32_t)(above + mine) >= need) {
    uint32_t acc = (uint32_t)above;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (acc + c[i] >= need) {
        const uint32_t bin = nb - 1 - (threadIdx.x * per + i);
        const uint32_t prev = st->prefix;
        st->prefix = (P == 0) ? bin : ((P == 1) ? ((prev << 11) | bin) : ((prev << 10) | bin));
        st->need = need - acc;
        break;
      }
      acc += c[i];
    }
  }
  // every thread clears the bins it read, ready for the next pass
#pragma unroll
  for (int i = 0; i < per; ++i) ghist[nb - 1 - (threadIdx.x * per + i)] = 0u;
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
  SeqState* st = w.st + c.s;
  uint32_t prefix = 0;
  if (P > 0) {
    if (st->mode != MODE_RADIX) return;
    prefix = st->prefix;
  }
  for (int i = threadIdx.x; i < NB; i += NT) lh[i] = 0u;
  __syncthreads();
  int np = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = c.begin + threadIdx.x + (int64_t)i * NT;
    if (j < c.end && pr[j]) {
      const uint32_t key = score_key(b[j]);
      ++np;
      if (P == 0) {
        atomicAdd(&lh[key >> 21], 1u);
      } else if (P == 1) {
        if ((key >> 21) == prefix) atomicAdd(&lh[(key >> 10) & 0x7ffu], 1u);
      } else {
        if ((key >> 10) == prefix) atomicAdd(&lh[key & 0x3ffu], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = w.hist + (size_t)c.s * NB;
  for (int i = threadIdx.x; i < NB; i += NT) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(gh + i, v);
  }
  if (P == 0) {
    np = wave_sum(np);
    if ((threadIdx.x & 63) == 0 && np) atomicAdd(&st->n_prunable, (uint32_t)np);
  }
  if (!arrive_last(st, c.nchunks, &sh[NT / 64])) return;
  // ---- last block of sequence s: narrow the digit
  if (P == 0) {
    const uint32_t npr = ld_acquire_u32(&st->n_prunable);
    const int kb = kbud[c.s];
    const uint32_t k = kb > 0 ? (uint32_t)kb : 0u;
    const uint32_t kp = k < npr ? k : npr;
    const int mode = kp == 0 ? MODE_NONE : (kp == npr ? MODE_ALL : MODE_RADIX);
    if (mode != MODE_RADIX) {
      // histogram left as is: later passes skip this sequence
      if (threadIdx.x == 0) {
        st->mode = mode;
        st->arrive = 0u;
      }
      return;
    }
    if (threadIdx.x == 0) {
      st->mode = mode;
      st->need = kp;
    }
    __syncthreads();
  }
  narrow<P>(st, gh, sh);
  if (threadIdx.x == 0) st->arrive = 0u;
}

__global__ __launch_bounds__(NT) void sel_count(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu, int n_seq,
                                               int64_t t_in, SelWs w,
                                               int32_t* __restrict__ kept_cu) {
  __shared__ int sh[NT / 64 + 2];
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  SeqState* st = w.st + c.s;
  const int mode = st->mode;
  const uint32_t tau = st->prefix;
  int def = 0, tie = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = c.begin + threadIdx.x + (int64_t)i * NT;
    if (j < c.end) {
      if (!pr[j] || mode == MODE_ALL) {
        ++def;
      } else if (mode == MODE_RADIX) {
        const uint32_t key = score_key(b[j]);
        def += key > tau;
        tie += key == tau;
      }
    }
  }
  def = wave_sum(def);
  tie = wave_sum(tie);
  if ((threadIdx.x & 63) == 0) {
    sh[threadIdx.x >> 6] = def;
  }
  __syncthreads();
  int tdef = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) tdef += sh[i];
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = tie;
  __syncthreads();
  if (threadIdx.x == 0) {
    int ttie = 0;
    for (int i = 0; i < NT / 64; ++i) ttie += sh[i];
    w.blk_def[c.slot] = tdef;
    w.blk_tie[c.slot] = ttie;
  }
  if (!arrive_last(st, c.nchunks, &sh[NT / 64])) return;
  // ---- last block of sequence s: offsets of its chunks, in chunk order
  if (threadIdx.x == 0) {
    const uint32_t need = mode == MODE_RADIX ? st->need : 0u;
    const int64_t s0 = slot0_of(cu, c.s, CH);
    int tie_off = 0, off = 0;
    for (int i = 0; i < c.nchunks; ++i) {
      const int64_t sl = s0 + i;
      const int d = __hip_atomic_load(w.blk_def + sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int t = __hip_atomic_load(w.blk_tie + sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int take = (int)need - tie_off;
      take = take < 0 ? 0 : (take > t ? t : take);
      w.blk_tie_off[sl] = tie_off;
      w.blk_off[sl] = off;
      tie_off += t;
      off += d + take;
    }
    st->kept_total = off;
    st->arrive = 0u;
    __threadfence();
    const uint32_t old = __hip_atomic_fetch_add(&w.globals[0], 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    sh[NT / 64 + 1] = (old == w.globals[1] - 1u);
  }
  __syncthreads();
  if (!sh[NT / 64 + 1]) return;
  __threadfence();
  // ---- last sequence overall: kept_cu_seqlens = exclusive scan of |S_s|
  int run = 0;
  for (int base = 0; base < n_seq; base += NT) {
    const int s = base + threadIdx.x;
    const int v = s < n_seq ? __hip_atomic_load(&w.st[s].kept_total, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : 0;
    int tot;
    const int ex = block_excl_scan<NT>(v, sh, &tot);
    if (s < n_seq) kept_cu[s] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0) kept_cu[n_seq] = run;
}

__global__ __launch_bounds__(NT) void sel_write(const float* __restrict__ b,
                                               const uint8_t* __restrict__ pr,
                                               const int32_t* __restrict__ cu, int n_seq,
                                               int64_t t_in, SelWs w,
                                               const int32_t* __restrict__ kept_cu,
                                               int64_t cap, int32_t* __restrict__ kept_idx,
                                               int32_t* __restrict__ kept_pos,
                                               float* __restrict__ kept_b) {
  __shared__ int sh[NT / 64 + 2];
  Chunk c;
  if (!locate(cu, n_seq, t_in, c)) return;
  const SeqState* st = w.st + c.s;
  const int mode = st->mode;
  const uint32_t tau = st->prefix;
  const int need = mode == MODE_RADIX ? (int)st->need : 0;
  const int tie_base = w.blk_tie_off[c.slot];
  const int64_t out_base = (int64_t)kept_cu[c.s] + w.blk_off[c.slot];
  const int64_t seq_lo = cu[c.s] < t_in ? cu[c.s] : t_in;
  // contiguous tokens per thread, so thread order is index order
  const int64_t j0 = c.begin + (int64_t)threadIdx.x * PER;
  float bv[PER];
  uint8_t fl[PER];     // bit0: kept for sure, bit1: tie at tau
  int nt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t j = j0 + i;
    uint8_t f = 0;
    float v = 0.f;
    if (j < c.end) {
      v = b[j];
      if (!pr[j] || mode == MODE_ALL) {
        f = 1;
      } else if (mode == MODE_RADIX) {
        const uint32_t key = score_key(v);
        f = key > tau ? 1 : (key == tau ? 2 : 0);
      }
    }
    bv[i] = v;
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
        if (kept_pos) kept_pos[o] = (int32_t)(j0 + i - seq_lo);
        if (kept_b) kept_b[o] = bv[i];
      }
      ++o;
    }
  }
}

}  // namespace

size_t select_ws_bytes(int64_t t_in, int n_seq) {
  const int64_t ns = n_slots_of(t_in, n_seq);
  size_t bytes = sizeof(SeqState) * (size_t)n_seq + sizeof(uint32_t) * (size_t)n_seq * NB +
                 4 * sizeof(int32_t) * (size_t)ns + 2 * sizeof(uint32_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_select(const float* b, const uint8_t* prunable, const int32_t* cu,
                         const int32_t* k, int n_seq, int64_t t_in, int64_t cap,
                         int32_t* kept_idx, int32_t* kept_pos, float* kept_b, int32_t* kept_cu,
                         void* ws, hipStream_t st) {
  SelWs w = carve(ws, t_in, n_seq);
  const int64_t ns = n_slots_of(t_in, n_seq);
  int64_t init_blocks = ((int64_t)n_seq * NB + NT - 1) / NT;
  if (init_blocks > 1024) init_blocks = 1024;
  if (init_blocks < 1) init_blocks = 1;
  hipLaunchKernelGGL(sel_init, dim3((unsigned)init_blocks), dim3(NT), 0, st, cu, n_seq, t_in, w,
                     kept_cu);
  if (t_in == 0) return hipGetLastError();
  const dim3 grid((unsigned)ns);
  hipLaunchKernelGGL(sel_pass<0>, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w);
  hipLaunchKernelGGL(sel_pass<1>, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w);
  hipLaunchKernelGGL(sel_pass<2>, grid, dim3(NT), 0, st, b, prunable, cu, k, n_seq, t_in, w);
  hipLaunchKernelGGL(sel_count, grid, dim3(NT), 0, st, b, prunable, cu, n_seq, t_in, w, kept_cu);
  hipLaunchKernelGGL(sel_write, grid, dim3(NT), 0, st, b, prunable, cu, n_seq, t_in, w, kept_cu,
                     cap, kept_idx, kept_pos, kept_b);
  return hipGetLastError();
}

}  // namespace tg
