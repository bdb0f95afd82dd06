// Jagged tile scheduler and offsets.
//
// Source: "Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a Different Stack",
// section "Bottleneck move 1": once padding is removed, short and long samples finish at
// different times, which exposes tile scheduling and backward accumulation; FAQ "What is a
// jagged tensor?": values plus offsets.  The pages give no schedule; this one is:
//  - forward: one record per (sample, query tile) covering the kv steps that tile can see
//    (causal bottom-right alignment); a tile with more than C kv steps, where
//    C = max(8, ceil(H * total_cost / slots)), splits into ceil(steps / C) near-equal chunks
//    whose partial results a combine pass merges in chunk order;
//  - backward: a query-stationary list (dQ) and a key-stationary list (dK, dV); a sample with
//    one query tile (or else one key tile) takes a single pass that owns all its gradients;
//  - every list is ordered longest first, ties by (sample, tile, first step): a total order,
//    so the lists are unique and bit-reproducible.
// One workgroup of 1024 threads does all of it with block scans and a sort on the inverted cost
// (bitonic or radix in LDS, radix in global memory for long lists); no host round trip.
#include "jfa_internal.h"

namespace jfa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int ST = 1024;
constexpr int SW = ST / 64;
constexpr int LDS_SORT_MAX = 8192;
constexpr int BITONIC_MAX = 1024;

__device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One DPP move of a 64-bit value (both halves with the same control; lanes without a source
// read 0).
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ int64_t dpp64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROW_MASK,
                                                            0xf, BOUND_ZERO);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(
      0, (int)(uint32_t)((uint64_t)x >> 32), CTRL, ROW_MASK, 0xf, BOUND_ZERO);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive scan over the 64 lanes of a wave with DPP: shifts by 1, 2, 4 and 8 lanes within each
// row of 16 (a row's first lanes read 0), then lane 15's sum broadcast into rows 1 and 3 and
// lane 31's into rows 2 and 3.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t x) {
  x += dpp64<0x111, 0xf, true>(x);     // row_shr:1
  x += dpp64<0x112, 0xf, true>(x);     // row_shr:2
  x += dpp64<0x114, 0xf, true>(x);     // row_shr:4
  x += dpp64<0x118, 0xf, true>(x);     // row_shr:8
  x += dpp64<0x142, 0xa, false>(x);    // row_bcast:15 into rows 1, 3
  x += dpp64<0x143, 0xc, false>(x);    // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scan of one value per thread over the workgroup; *total receives the sum.
__device__ __forceinline__ int64_t block_scan(int64_t v, int64_t* total, int64_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t x = wave_incl_scan(v);
  if (lane == 63) red[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int64_t w = wave_incl_scan(lane < SW ? red[lane] : 0);
    if (lane < SW) red[lane] = w;
  }
  __syncthreads();
  const int64_t pre = wave > 0 ? red[wave - 1] : 0;
  *total = red[SW - 1];
  __syncthreads();
  return pre + x - v;
}

// out[i] = sum_{k<i} f(k) for i in [0, L]; returns the total.
template <typename OutT, class F>
__device__ __forceinline__ int64_t scan_to(OutT* out, int64_t L, F f, int64_t* red) {
  int64_t carry = 0;
  for (int64_t base = 0; base < L; base += ST) {
    const int64_t i = base + threadIdx.x;
    const int64_t v = i < L ? f(i) : 0;
    int64_t tot;
    const int64_t ex = block_scan(v, &tot, red);
    if (i < L) out[i] = (OutT)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) out[L] = (OutT)carry;
  __syncthreads();
  return carry;
}

// Largest b with base[b] <= x, for base[0] = 0 <= x < base[B].
__device__ __forceinline__ int owner_of(const int32_t* base, int B, int64_t x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (base[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Ascending bitonic sort of N (a power of two, at most LDS_SORT_MAX) unique keys in LDS.
__device__ __forceinline__ void bitonic_sort(uint32_t* s, int N) {
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < N / 2; i += ST) {
        const int lo = 2 * j * (i / j) + (i % j), hi = lo + j;
        const bool up = (lo & k) == 0;
        const uint32_t x = s[lo], y = s[hi];
        if ((x > y) == up) {
          s[lo] = y;
          s[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Stable ascending sort of words by bits [20, 32), three 4-bit passes; result ends in b.
__device__ __forceinline__ void radix_sort(uint32_t* a, uint32_t* b, int n, int32_t* T,
                                           int64_t* red) {
  const int tid = threadIdx.x;
  const int ipt = (n + ST - 1) / ST;
  const int lo = min(n, tid * ipt), hi = min(n, lo + ipt);
  uint32_t* src = a;
  uint32_t* dst = b;
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = 20 + 4 * pass;
    for (int d = 0; d < 16; ++d) T[d * ST + tid] = 0;
    for (int i = lo; i < hi; ++i) T[((src[i] >> sh) & 15) * ST + tid] += 1;
    __syncthreads();
    int64_t s = 0;
    for (int k = 0; k < 16; ++k) s += T[tid * 16 + k];
    int64_t tot;
    int64_t run = block_scan(s, &tot, red);
    for (int k = 0; k < 16; ++k) {
      const int32_t c = T[tid * 16 + k];
      T[tid * 16 + k] = (int32_t)run;
      run += c;
    }
    __syncthreads();
    for (int i = lo; i < hi; ++i) {
      const uint32_t w = src[i];
      const int d = (w >> sh) & 15;
      const int32_t p = T[d * ST + tid];
      T[d * ST + tid] = p + 1;
      dst[p] = w;
    }
    __syncthreads();
    uint32_t* t = src; src = dst; dst = t;
  }
  // three passes: a -> b -> a -> b
}

// Stable counting sort of n <= CS_MAX records by cost descending (ties in index order), for
// costs in [1, kmax] with kmax * ceil(n / 64) <= 16 * ST.  Records are taken in chunks of 64
// (record i is lane i % 64 of chunk i / 64; a wave handles chunks wave, wave + SW, ...).  The
// rank of record i is the number of records of higher cost, plus those of equal cost in
// earlier chunks, plus those of equal cost on lower lanes of its own chunk (found by matching
// the key bits with ballots).  A handful of barriers, where a bitonic sort of the same list
// needs one per merge phase.  out[rank] = i.
constexpr int CS_MAX = 4096;
__device__ __forceinline__ void count_sort(const int32_t* t_cost, int n, int kmax, uint32_t* out,
                                           int32_t* T,
                           int64_t* red) {
  constexpr int R = CS_MAX / ST;              // records per thread
  const int tid = threadIdx.x, lane = tid & 63;
  const int nchunk = (n + 63) / 64;
  const int nent = kmax * nchunk;             // counters [key][chunk], key = kmax - cost
  for (int i = tid; i < nent; i += ST) T[i] = 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int key[R], r[R], cnt[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = k * ST + tid;
    const bool act = i < n;
    key[k] = act ? kmax - t_cost[i] : 0;
    uint64_t same = __ballot(act);
    for (int bit = 0; (1 << bit) < kmax; ++bit) {
      const uint64_t bal = __ballot(act && ((key[k] >> bit) & 1));
      same &= ((key[k] >> bit) & 1) ? bal : ~bal;
    }
    r[k] = __popcll(same & below);
    cnt[k] = act ? __popcll(same) : 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = k * ST + tid;
    if (i < n && r[k] == cnt[k] - 1) T[key[k] * nchunk + (i >> 6)] = cnt[k];
  }
  __syncthreads();
  // exclusive scan of the counters in (key, chunk) order: EPT contiguous entries per thread
  const int ept = (nent + ST - 1) / ST;
  const int lo = min(nent, tid * ept), hi = min(nent, lo + ept);
  int64_t part = 0;
  for (int i = lo; i < hi; ++i) part += T[i];
  int64_t tot;
  int64_t run = block_scan(part, &tot, red);
  for (int i = lo; i < hi; ++i) {
    const int32_t c = T[i];
    T[i] = (int32_t)run;
    run += c;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = k * ST + tid;
    if (i < n) out[T[key[k] * nchunk + (i >> 6)] + r[k]] = (uint32_t)i;
  }
  __syncthreads();
}

// Sample offsets are copied to LDS when B is at most this (every tile looks its sample up).
constexpr int LDS_OFF_MAX = 4095;

struct Shared {
  uint32_t sa[LDS_SORT_MAX];
  int32_t T[16 * ST];
  int32_t qo[LDS_OFF_MAX + 1];
  int32_t ko[LDS_OFF_MAX + 1];
  int64_t red[SW];
  int32_t flag;
  int64_t sumcost;
};

// The list's work record for list record r of sample b (kernels start an item from it).
__device__ __forceinline__ ItemRec item_of(const SchedArgs& a, int4 r, int slot,
                                           const int32_t* qo,
                                           const int32_t* ko) {
  ItemRec it{};
  it.b = r.x; it.x = r.y; it.y = r.z; it.z = r.w;
  it.slot = slot;
  it.qo = qo[r.x];
  it.n = qo[r.x + 1] - it.qo;
  it.ko = ko[r.x];
  it.m = ko[r.x + 1] - it.ko;
  it.boff = (a.want_bias_off && a.dense_bias) ? a.bias_off[r.x] : 0;
  return it;
}

// Sorts gen_recs[0..n) by cost (desc, ties by generation index) into out / out_slot and the work
// records `items` (each output may be null); the keys (inverted cost << 20 | index) are unique,
// so the order is total.  Short lists use a bitonic sort in LDS; longer ones, whose keys arrive
// in generation order, a stable 3-pass radix sort on the cost bits alone (in LDS up to 4096
// entries, else in global memory).
__device__ __forceinline__ void sort_and_emit(const SchedArgs& a, Shared& sh, int n,
                                              const int32_t* t_cost,
                              int4* out, int32_t* out_slot, ItemRec* items, const int32_t* qo,
                              const int32_t* ko) {
  const uint32_t* sorted;
  int kmax = 0;
  if (n <= CS_MAX) {
    int c = 0;
    for (int i = threadIdx.x; i < n; i += ST) c = max(c, t_cost[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c = max(c, __shfl_xor(c, o, 64));
    if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = c;
    __syncthreads();
    for (int w = 0; w < SW; ++w) kmax = max(kmax, (int)sh.red[w]);
    __syncthreads();
  }
  if (n <= CS_MAX && (int64_t)max(kmax, 1) * ((n + 63) / 64) <= 16 * ST) {
    count_sort(t_cost, n, max(kmax, 1), sh.sa, sh.T, sh.red);
    sorted = sh.sa;
  } else if (n <= BITONIC_MAX) {
    int N = 1;
    while (N < n) N <<= 1;
    for (int i = threadIdx.x; i < N; i += ST)
      sh.sa[i] = i < n ? ((uint32_t)(MAX_COST - t_cost[i]) << 20) | (uint32_t)i : 0xFFFFFFFFu;
    __syncthreads();
    bitonic_sort(sh.sa, N);
    sorted = sh.sa;
  } else if (n <= LDS_SORT_MAX / 2) {
    for (int i = threadIdx.x; i < n; i += ST)
      sh.sa[i] = ((uint32_t)(MAX_COST - t_cost[i]) << 20) | (uint32_t)i;
    __syncthreads();
    radix_sort(sh.sa, sh.sa + LDS_SORT_MAX / 2, n, sh.T, sh.red);
    sorted = sh.sa + LDS_SORT_MAX / 2;
  } else {
    for (int i = threadIdx.x; i < n; i += ST)
      a.words_a[i] = ((uint32_t)(MAX_COST - t_cost[i]) << 20) | (uint32_t)i;
    __syncthreads();
    radix_sort(a.words_a, a.words_b, n, sh.T, sh.red);
    sorted = a.words_b;
  }
  // U records per thread at a time, all their loads issued before any use: the records are
  // gathered from global memory, and one at a time each would wait a full memory round trip
  constexpr int U = 4;
  for (int base = 0; base < n; base += ST * U) {
    int4 r[U];
    int slot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * ST + threadIdx.x;
      if (i < n) {
        const uint32_t idx = sorted[i] & 0xFFFFFu;
        r[u] = a.gen_recs[idx];
        slot[u] = out_slot || items ? a.gen_slot[idx] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * ST + threadIdx.x;
      if (i >= n) continue;
      if (out) out[i] = r[u];
      if (out_slot) out_slot[i] = slot[u];
      if (items) items[i] = item_of(a, r[u], slot[u], qo, ko);
    }
  }
  __syncthreads();
}

// Fast path of a list of n <= CS_MAX records: record i is generated by rec_of(i, rec, slot,
// cost) on thread i % ST, ranked there (cost descending, ties in index order: the same stable
// counting rank as count_sort) and written straight to its rank, so the list makes no round
// trip through global memory.  Returns false, having written nothing but what rec_of writes
// itself, when the list is too long or its costs too spread for the counters; the caller then
// takes the general path.
template <int R, class RecOf>
__device__ __forceinline__ bool rank_emit_r(const SchedArgs& a, Shared& sh, int n, RecOf rec_of,
                                            int4* out,
                            int32_t* out_slot, ItemRec* items, const int32_t* qo,
                            const int32_t* ko) {
  const int tid = threadIdx.x, lane = tid & 63;
  int4 rec[R];
  int slot[R], key[R];
  int c = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = k * ST + tid;
    key[k] = 0;
    slot[k] = -1;
    if (i < n) {
      rec_of(i, rec[k], slot[k], key[k]);
      c = max(c, key[k]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c = max(c, __shfl_xor(c, o, 64));
  if (lane == 0) sh.red[tid >> 6] = c;
  __syncthreads();
  int kmax = 1;
  for (int w = 0; w < SW; ++w) kmax = max(kmax, (int)sh.red[w]);
  __syncthreads();
  const int nchunk = (n + 63) / 64;
  if ((int64_t)kmax * nchunk > 16 * ST) return false;
  // rank = records of higher cost + equal cost in earlier chunks + equal cost on lower lanes
  int32_t* T = sh.T;
  const int nent = kmax * nchunk;             // counters [key][chunk], key = kmax - cost
  for (int i = tid; i < nent; i += ST) T[i] = 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int r[R], cnt[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = k * ST + tid;
    const bool act = i < n;
    key[k] = act ? kmax - key[k] : 0;
    uint64_t same = __ballot(act);
    for (int bit = 0; (1 << bit) < kmax; ++bit) {
      const uint64_t bal = __ballot(act && ((key[k] >> bit) & 1));
      same &= ((key[k] >> bit) & 1) ? bal : ~bal;
    }
    r[k] = __popcll(same & below);
    cnt[k] = act ? __popcll(same) : 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = k * ST + tid;
    if (i < n && r[k] == cnt[k] - 1) T[key[k] * nchunk + (i >> 6)] = cnt[k];
  }
  __syncthreads();
  const int ept = (nent + ST - 1) / ST;
  const int lo = min(nent, tid * ept), hi = min(nent, lo + ept);
  int64_t part = 0;
  for (int i = lo; i < hi; ++i) part += T[i];
  int64_t tot;
  int64_t run = block_scan(part, &tot, sh.red);
  for (int i = lo; i < hi; ++i) {
    const int32_t cc = T[i];
    T[i] = (int32_t)run;
    run += cc;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = k * ST + tid;
    if (i >= n) continue;
    const int pos = T[key[k] * nchunk + (i >> 6)] + r[k];
    if (out) out[pos] = rec[k];
    if (out_slot) out_slot[pos] = slot[k];
    if (items) items[pos] = item_of(a, rec[k], slot[k], qo, ko);
  }
  __syncthreads();
  return true;
}

// R records per thread (registers only: small fully unrolled arrays)
template <class RecOf>
__device__ __forceinline__ bool rank_emit(const SchedArgs& a, Shared& sh, int n, RecOf rec_of,
                                          int4* out,
                          int32_t* out_slot, ItemRec* items, const int32_t* qo,
                          const int32_t* ko) {
  static_assert(CS_MAX == 4 * ST, "record count classes");
  if (n <= ST) return rank_emit_r<1>(a, sh, n, rec_of, out, out_slot, items, qo, ko);
  if (n <= 2 * ST) return rank_emit_r<2>(a, sh, n, rec_of, out, out_slot, items, qo, ko);
  if (n <= CS_MAX) return rank_emit_r<4>(a, sh, n, rec_of, out, out_slot, items, qo, ko);
  return false;
}

// D[h][i] = sum_c dO[i,h,c] * O[i,h,c] for every (query row, head): the softmax backward's
// preprocess, run by the workgroups of the scheduler launch that build no list, so that it
// overlaps the single-workgroup list building.  Each (row, head) vector is LPR consecutive
// lanes with one 16-byte load each of O and dO; lanes combine with xor shuffles.
template <int ES, int D>
__device__ __forceinline__ void delta_rows(const SchedArgs& a, int block, int nblocks) {
  constexpr int EPL = 16 / ES;                    // elements per 16-byte load
  constexpr int LPR = D / EPL;                    // lanes per (row, head) vector
  constexpr int U = 4;                            // vectors in flight per thread
  const int64_t nchunks = a.total_q * a.H * LPR;
  const int64_t stride = (int64_t)nblocks * ST;
  const uint8_t* o = (const uint8_t*)a.d_o;
  const uint8_t* g = (const uint8_t*)a.d_dout;
  for (int64_t base = (int64_t)block * ST + threadIdx.x; base < nchunks; base += U * stride) {
    u32x4 x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * stride;
      if (c < nchunks) {
        x[u] = *(const u32x4*)(o + c * 16);
        y[u] = *(const u32x4*)(g + c * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * stride;
      float acc = 0.f;
      if (c < nchunks) {
        if constexpr (ES == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = fmaf(__uint_as_float(x[u][e] << 16), __uint_as_float(y[u][e] << 16), acc);
            acc = fmaf(__uint_as_float(x[u][e] & 0xffff0000u),
                       __uint_as_float(y[u][e] & 0xffff0000u), acc);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = fmaf(__uint_as_float(x[u][e]), __uint_as_float(y[u][e]), acc);
        }
      }
      // the LPR lanes of a vector are aligned and share c / LPR, so the whole group is either
      // in range or out of it
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (c < nchunks && (threadIdx.x % LPR) == 0) {   // c and the lane agree mod LPR
        const int64_t rh = c / LPR;
        a.d_delta[(rh % a.H) * a.total_q + rh / a.H] = acc;
      }
    }
  }
}

// The same D with MXFP8 dO (O stays bf16): each lane takes 8 elements of a (row, head) vector,
// 16 bytes of O and 8 codes of dO with their E8M0 block scale, dequantised exactly in fp32.
template <int D>
__device__ __forceinline__ void delta_rows_fp8(const SchedArgs& a, int block, int nblocks) {
  constexpr int LPR = D / 8;                      // lanes per (row, head) vector
  constexpr int U = 4;
  const int64_t nchunks = a.total_q * a.H * LPR;
  const int64_t stride = (int64_t)nblocks * ST;
  const uint8_t* o = (const uint8_t*)a.d_o;
  const uint8_t* g = (const uint8_t*)a.d_dout;
  for (int64_t base = (int64_t)block * ST + threadIdx.x; base < nchunks; base += U * stride) {
    u32x4 x[U];
    uint2 y[U];
    uint32_t sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * stride;
      if (c < nchunks) {
        x[u] = *(const u32x4*)(o + c * 16);
        y[u] = *(const uint2*)(g + c * 8);
        sc[u] = a.d_dout_sc[c / 4];               // 32 elements (4 chunks) per scale
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + u * stride;
      float acc = 0.f;
      if (c < nchunks) {
        // 2^(s - 127) as a float (s = 0: 2^-127, a subnormal)
        const float f = sc[u] == 0 ? 5.877471754111438e-39f : __uint_as_float(sc[u] << 23);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t code = ((e < 4 ? y[u].x : y[u].y) >> (8 * (e & 3))) & 255u;
          // E4M3: sign, 4-bit exponent (bias 7), 3-bit mantissa, subnormals at exponent 0
          const uint32_t ex = (code >> 3) & 15u, mt = code & 7u;
          float v = ex ? __uint_as_float(((ex + 120u) << 23) | (mt << 20))
                       : (float)mt * 0.001953125f;
          v = (code & 128u) ? -v : v;
          const uint32_t ow = x[u][e >> 1];
          const float ov = __uint_as_float((e & 1) ? (ow & 0xffff0000u) : (ow << 16));
          acc = fmaf(ov, v * f, acc);
        }
      }
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (c < nchunks && (threadIdx.x % LPR) == 0) {
        const int64_t rh = c / LPR;
        a.d_delta[(rh % a.H) * a.total_q + rh / a.H] = acc;
      }
    }
  }
}

__global__ __launch_bounds__(ST) void schedule_kernel(SchedArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Shared& sh = *reinterpret_cast<Shared*>(smem_raw);
  const int tid = threadIdx.x;
  const int B = a.B;
  const TileCfg tc = a.tc;

  // roles: with a.parallel, workgroup r builds the r-th requested list; otherwise workgroup 0
  // builds them all.  Workgroups past the list builders compute D.
  const int nroles = a.parallel ? __popc(a.lists & 7) : 1;
  if ((int)blockIdx.x >= nroles) {
    const int blk = blockIdx.x - nroles, nblk = gridDim.x - nroles;
    if (a.d_dout_sc) {
      if (a.d_head_dim == 128) delta_rows_fp8<128>(a, blk, nblk);
      else delta_rows_fp8<64>(a, blk, nblk);
    } else if (a.d_esize == 2) {
      if (a.d_head_dim == 128) delta_rows<2, 128>(a, blk, nblk);
      else delta_rows<2, 64>(a, blk, nblk);
    } else {
      if (a.d_head_dim == 128) delta_rows<4, 128>(a, blk, nblk);
      else delta_rows<4, 64>(a, blk, nblk);
    }
    return;
  }
  const int role = blockIdx.x;
  int my_lists = a.lists & 7;
  if (a.parallel) {
    int k = role;
    for (int bit = 0; bit < 3; ++bit)
      if ((a.lists >> bit) & 1) {
        if (k == 0) { my_lists = 1 << bit; break; }
        --k;
      }
  }

  // ---- validation of the offsets (and the sort's cost limit)
  if (tid == 0) sh.flag = 0;
  __syncthreads();
  int bad = 0;
  for (int b = tid; b < B; b += ST) {
    const int64_t n = (int64_t)a.q_off[b + 1] - a.q_off[b];
    const int64_t m = (int64_t)a.kv_off[b + 1] - a.kv_off[b];
    if (n < 0 || m < 0) bad = 1;
    else if (cdiv(m, min(tc.bn, tc.bq_bn)) > MAX_COST || cdiv(n, tc.bk_bm) > MAX_COST) bad = 1;
    // kernels address one sample's rows (plus one tile of overhang) with 32-bit byte offsets
    else if ((n + 256) * a.hd_bytes > INT32_MAX || (m + 256) * a.hd_bytes > INT32_MAX) bad = 1;
    else if (a.dense_bias && (n + 256) * (m + 256) * 4 > INT32_MAX) bad = 1;
  }
  if (tid == 0 && (a.q_off[0] != 0 || a.kv_off[0] != 0 || a.q_off[B] != a.total_q ||
                   a.kv_off[B] != a.total_kv))
    bad = 1;
  if (bad) atomicOr(&sh.flag, 1);
  __syncthreads();
  if (sh.flag) {
    // every role finds the same failure and writes the same values
    if (tid == 0) {
      a.hdr->status = JFA_ERR_DEVICE_DATA;
      for (int i = 0; i < 8; ++i) a.hdr->counts[i] = 0;
      for (int i = 0; i < 8; ++i) a.hdr->tickets[i] = 0;
      for (int i = 0; i < 4; ++i) a.hdr->list_status[i] = JFA_OK;
      if (a.counts_copy) {
        for (int i = 0; i < 8; ++i) a.counts_copy[i] = 0;
        a.counts_copy[6] = JFA_ERR_DEVICE_DATA;
      }
    }
    return;
  }

  // sample offsets: from LDS when they fit (every tile and record looks its sample up)
  const int32_t* qo = a.q_off;
  const int32_t* ko = a.kv_off;
  if (B <= LDS_OFF_MAX) {
    for (int b = tid; b <= B; b += ST) {
      sh.qo[b] = a.q_off[b];
      sh.ko[b] = a.kv_off[b];
    }
    __syncthreads();
    qo = sh.qo;
    ko = sh.ko;
  }
  auto qlen = [&](int b) -> int64_t { return (int64_t)qo[b + 1] - qo[b]; };
  auto klen = [&](int b) -> int64_t { return (int64_t)ko[b + 1] - ko[b]; };

  // ---- dense-bias offsets: running sum of q_len * kv_len
  if (a.want_bias_off)
    scan_to(a.bias_off, B, [&](int64_t b) { return qlen((int)b) * klen((int)b); }, sh.red);

  // per-sample tile base [B+1]: in LDS (the sort-key space, idle during generation) whenever
  // it fits, since every tile looks its sample up there by binary search
  int32_t* lds_ints = reinterpret_cast<int32_t*>(sh.sa);
  int32_t* s_base = (B + 1 <= LDS_SORT_MAX / 2) ? lds_ints : a.s_tmp;
  int32_t* t_cost = a.t_tmp;                 // per record cost (generation order)
  int32_t* t_rb = a.t_tmp + (a.cap_t + 1);   // per tile record base
  int32_t* t_sb = a.t_tmp + 2 * (a.cap_t + 1); // per tile slot base
  int32_t* t_cb = a.t_tmp + 3 * (a.cap_t + 1); // per tile combine index
  int overflow = 0;

  // ================= forward list =================
  const bool want_f = my_lists & 1, want_q = my_lists & 2, want_k = my_lists & 4;
  const int64_t ntiles =
      want_f ? scan_to(s_base, B, [&](int64_t b) { return cdiv(qlen((int)b), tc.bm); }, sh.red) : 0;
  if (ntiles > a.cap_t) overflow = 1;
  // kv steps of forward tile tau, and its sample (32-bit arithmetic: the offsets check bounds
  // every length far below 2^31)
  // first kv step of forward tile t of sample b (0 without a sliding window)
  auto fwd_first = [&](int b, int64_t t) -> int64_t {
    if (a.window <= 0) return 0;
    int64_t s0, s1;
    visible_key_steps(a.causal, a.window, t * tc.bm, min((t + 1) * tc.bm, qlen(b)), qlen(b),
                      klen(b), tc.bn, 0, s0, s1);
    return s0;
  };
  auto fwd_steps = [&](int64_t tau, int& b, int64_t& t) -> int64_t {
    b = owner_of(s_base, B, tau);
    t = tau - s_base[b];
    const int n = (int)qlen(b), m = (int)klen(b);
    const int r1 = min(((int)t + 1) * tc.bm, n);
    if (a.window > 0) {
      int64_t s0, s1;
      visible_key_steps(a.causal, a.window, t * tc.bm, r1, n, m, tc.bn, 0, s0, s1);
      return s1 - s0;
    }
    int e = m;
    if (a.causal) e = max(0, min(m, r1 + (m - n)));
    return (e + tc.bn - 1) / tc.bn;
  };
  // every tile's sample and steps once, into the sort's counter space (idle until the list is
  // ranked): the cost pass, the scans and the record generator read them from there
  const bool tile_cache = want_f && !overflow && ntiles <= 8 * ST;
  int32_t* t_b = sh.T;
  int32_t* t_st = sh.T + 8 * ST;
  if (tile_cache) {
    for (int64_t tau = tid; tau < ntiles; tau += ST) {
      int b;
      int64_t t;
      t_st[tau] = (int32_t)fwd_steps(tau, b, t);
      t_b[tau] = b;
    }
    __syncthreads();
  }
  auto steps_of = [&](int64_t tau, int& b, int64_t& t) -> int64_t {
    if (tile_cache) {
      b = t_b[tau];
      t = tau - s_base[b];
      return t_st[tau];
    }
    return fwd_steps(tau, b, t);
  };
  int64_t C = 0;
  int64_t nrec = 0, nslot = 0, ncomb = 0;
  if (want_f && !overflow && s_base == lds_ints &&
      (int64_t)(B + 1) + 3 * (ntiles + 1) <= LDS_SORT_MAX) {
    t_rb = lds_ints + (B + 1);
    t_sb = t_rb + (ntiles + 1);
    t_cb = t_sb + (ntiles + 1);
  }
  if (want_f && !overflow) {
    // total cost -> split threshold
    int64_t part = 0;
    for (int64_t tau = tid; tau < ntiles; tau += ST) {
      int b; int64_t t;
      part += max((int64_t)1, steps_of(tau, b, t));
    }
    int64_t tot;
    block_scan(part, &tot, sh.red);
    if (tc.slots > 0) C = max((int64_t)8, cdiv((int64_t)a.H * tot, tc.slots));
    auto nch_of = [&](int64_t tau) -> int64_t {
      int b; int64_t t;
      const int st = (int)steps_of(tau, b, t);
      return (C > 0 && st > C) ? (st + (int)C - 1) / (int)C : 1;   // C < st <= MAX_COST
    };
    // record base, slot base and combine index of every tile in one scan: the three counts
    // share a 64-bit word in 21-bit fields (each total stays below 2^21 when the tiles are
    // cached: at most 8192 tiles, and the split chunks are bounded by the slots)
    if (tile_cache && 2 * (int64_t)tc.slots + ntiles < (1 << 20)) {
      int64_t carry = 0;
      for (int64_t base = 0; base < ntiles; base += ST) {
        const int64_t tau = base + tid;
        int64_t v = 0;
        if (tau < ntiles) {
          const int64_t c = nch_of(tau);
          v = c | ((c > 1 ? c : 0) << 21) | ((int64_t)(c > 1) << 42);
        }
        int64_t tot;
        const int64_t ex = carry + block_scan(v, &tot, sh.red);
        if (tau < ntiles) {
          t_rb[tau] = (int32_t)(ex & 0x1FFFFF);
          t_sb[tau] = (int32_t)((ex >> 21) & 0x1FFFFF);
          t_cb[tau] = (int32_t)(ex >> 42);
        }
        carry += tot;
      }
      if (tid == 0) {
        t_rb[ntiles] = (int32_t)(carry & 0x1FFFFF);
        t_sb[ntiles] = (int32_t)((carry >> 21) & 0x1FFFFF);
        t_cb[ntiles] = (int32_t)(carry >> 42);
      }
      __syncthreads();
      nrec = carry & 0x1FFFFF;
      nslot = (carry >> 21) & 0x1FFFFF;
      ncomb = carry >> 42;
    } else {
      nrec = scan_to(t_rb, ntiles, nch_of, sh.red);
      nslot = scan_to(t_sb, ntiles,
                      [&](int64_t tau) { int64_t c = nch_of(tau); return c > 1 ? c : 0; },
                      sh.red);
      ncomb = scan_to(t_cb, ntiles, [&](int64_t tau) { return nch_of(tau) > 1 ? 1 : 0; },
                      sh.red);
    }
    if (nrec > a.cap_f || nrec > a.cap_t || ncomb > a.cap_c || nslot > a.cap_slots) overflow = 1;
  }
  bool done_f = false;
  if (want_f && !overflow) {
    // record i: tile tau (record base t_rb), chunk c of its nch chunks
    const bool split = ncomb > 0;
    auto rec_f = [&](int i, int4& r, int& sl, int& cost) {
      int tau = i;
      int64_t c = 0;
      if (split) {
        tau = owner_of(t_rb, (int)ntiles, i);
        c = i - t_rb[tau];
      }
      int b;
      int64_t t;
      const int st = (int)steps_of(tau, b, t);
      const int nch = (C > 0 && st > C) ? (st + (int)C - 1) / (int)C : 1;
      const int ci = (int)c;
      const int k0 = (int)fwd_first(b, t);
      const int kb = k0 + ci * st / nch, ke = k0 + (ci + 1) * st / nch;
      r = make_int4(b, (int)t, kb, ke);
      sl = nch > 1 ? t_sb[tau] + ci : -1;
      cost = max(1, ke - kb);
      if (nch > 1 && ci == 0) a.comb[t_cb[tau]] = make_int4(b, (int)t, t_sb[tau], nch);
    };
    done_f = rank_emit(a, sh, (int)nrec, rec_f, a.fwd, a.fwd_slot, a.fwd_items, qo, ko);
  }
  if (want_f && !overflow && !done_f) {
    for (int64_t tau = tid; tau < ntiles; tau += ST) {
      int b; int64_t t;
      const int64_t s = steps_of(tau, b, t);
      const int64_t nch = (C > 0 && s > C) ? cdiv(s, C) : 1;
      const int64_t rb = t_rb[tau];
      const int64_t k0 = fwd_first(b, t);
      for (int64_t c = 0; c < nch; ++c) {
        const int64_t kb = k0 + c * s / nch, ke = k0 + (c + 1) * s / nch;
        a.gen_recs[rb + c] = make_int4(b, (int)t, (int)kb, (int)ke);
        a.gen_slot[rb + c] = nch > 1 ? (int32_t)(t_sb[tau] + c) : -1;
        t_cost[rb + c] = (int32_t)max((int64_t)1, ke - kb);
      }
      if (nch > 1) a.comb[t_cb[tau]] = make_int4(b, (int)t, t_sb[tau], (int)nch);
    }
    __syncthreads();
    sort_and_emit(a, sh, (int)nrec, t_cost, a.fwd, a.fwd_slot, a.fwd_items, qo, ko);
  }

  // ================= q-stationary backward list =================
  auto one_q = [&](int b) { return (tc.fuse & 1) && qlen(b) > 0 && qlen(b) <= tc.bq_bm; };
  auto one_k = [&](int b) {
    return (tc.fuse & 2) && !one_q(b) && klen(b) > 0 && klen(b) <= tc.bk_bn;
  };
  int64_t nq = 0, nk = 0;
  if (want_q && !overflow) {
    nq = scan_to(s_base, B,
                 [&](int64_t b) { return one_k((int)b) ? 0 : cdiv(qlen((int)b), tc.bq_bm); },
                 sh.red);
    if (nq > a.cap_q || nq > a.cap_t) overflow = 1;
  }
  bool done_q = false;
  if (want_q && !overflow) {
    auto rec_q = [&](int tau, int4& r, int& sl, int& cost) {
      const int b = owner_of(s_base, B, tau);
      const int t = tau - s_base[b];
      const int n = (int)qlen(b), m = (int)klen(b);
      int64_t s0 = 0, s1 = (m + tc.bq_bn - 1) / tc.bq_bn;
      // a single pass also owns dK/dV, so it visits every key tile (unseen keys get zeros)
      if (!one_q(b))
        visible_key_steps(a.causal, a.window, (int64_t)t * tc.bq_bm,
                          min((int64_t)(t + 1) * tc.bq_bm, (int64_t)n), n, m, tc.bq_bn, 0, s0,
                          s1);
      r = make_int4(b, t, (int)s0, (int)s1);
      sl = -1;
      cost = max(1, (int)(s1 - s0));
    };
    done_q = rank_emit(a, sh, (int)nq, rec_q, a.bq, nullptr, a.bq_items, qo, ko);
  }
  if (want_q && !overflow && !done_q) {
    for (int64_t tau = tid; tau < nq; tau += ST) {
      const int b = owner_of(s_base, B, tau);
      const int64_t t = tau - s_base[b];
      const int64_t n = qlen(b), m = klen(b);
      int64_t s0 = 0, s1 = cdiv(m, tc.bq_bn);
      if (!one_q(b))
        visible_key_steps(a.causal, a.window, t * tc.bq_bm, min((t + 1) * tc.bq_bm, n), n, m,
                          tc.bq_bn, 0, s0, s1);
      a.gen_recs[tau] = make_int4(b, (int)t, (int)s0, (int)s1);
      a.gen_slot[tau] = -1;
      t_cost[tau] = (int32_t)max((int64_t)1, s1 - s0);
    }
    __syncthreads();
    sort_and_emit(a, sh, (int)nq, t_cost, a.bq, nullptr, a.bq_items, qo, ko);
  }

  // ================= kv-stationary backward list =================
  if (want_k && !overflow) {
    nk = scan_to(s_base, B,
                 [&](int64_t b) { return one_q((int)b) ? 0 : cdiv(klen((int)b), tc.bk_bn); },
                 sh.red);
    if (nk > a.cap_k || nk > a.cap_t) overflow = 1;
  }
  bool done_k = false;
  if (want_k && !overflow) {
    auto rec_k = [&](int tau, int4& r, int& sl, int& cost) {
      const int b = owner_of(s_base, B, tau);
      const int u = tau - s_base[b];
      const int n = (int)qlen(b), m = (int)klen(b);
      const int nqs = (n + tc.bk_bm - 1) / tc.bk_bm;
      int64_t s0 = 0, s1 = nqs;
      // a single pass also owns dQ, so it visits every query tile (unseeing queries get zeros)
      if (!one_k(b))
        visible_query_steps(a.causal, a.window, (int64_t)u * tc.bk_bn,
                            min((int64_t)(u + 1) * tc.bk_bn, (int64_t)m), n, m, tc.bk_bm, nqs,
                            s0, s1);
      r = make_int4(b, u, (int)s0, (int)s1);
      sl = -1;
      cost = max(1, (int)(s1 - s0));
    };
    done_k = rank_emit(a, sh, (int)nk, rec_k, a.bk, nullptr, a.bk_items, qo, ko);
  }
  if (want_k && !overflow && !done_k) {
    for (int64_t tau = tid; tau < nk; tau += ST) {
      const int b = owner_of(s_base, B, tau);
      const int64_t u = tau - s_base[b];
      const int64_t n = qlen(b), m = klen(b);
      const int64_t nqs = cdiv(n, tc.bk_bm);
      int64_t s0 = 0, s1 = nqs;
      if (!one_k(b))
        visible_query_steps(a.causal, a.window, u * tc.bk_bn, min((u + 1) * tc.bk_bn, m), n, m,
                            tc.bk_bm, nqs, s0, s1);
      a.gen_recs[tau] = make_int4(b, (int)u, (int)s0, (int)s1);
      a.gen_slot[tau] = -1;
      t_cost[tau] = (int32_t)max((int64_t)1, s1 - s0);
    }
    __syncthreads();
    sort_and_emit(a, sh, (int)nk, t_cost, a.bk, nullptr, a.bk_items, qo, ko);
  }

  if (tid == 0) {
    const int st = overflow ? JFA_ERR_DEVICE_DATA : JFA_OK;
    const int32_t cnt[8] = {overflow ? 0 : (int32_t)nrec, overflow ? 0 : (int32_t)ncomb,
                            overflow ? 0 : (int32_t)nq, overflow ? 0 : (int32_t)nk, (int32_t)C,
                            overflow ? 0 : (int32_t)nslot, st, 0};
    if (!a.parallel) {
      a.hdr->status = st;
      for (int i = 0; i < 8; ++i) a.hdr->counts[i] = cnt[i];
      for (int i = 0; i < 4; ++i) a.hdr->list_status[i] = JFA_OK;
      if (a.counts_copy)
        for (int i = 0; i < 8; ++i) a.counts_copy[i] = cnt[i];
    } else {
      // the offsets are valid (every role checked them alike); a list that overflowed its
      // capacity is left empty and flagged in its own status word
      a.hdr->status = JFA_OK;
      const int li = want_f ? 0 : (want_q ? 1 : 2);
      a.hdr->list_status[li] = st;
      if (want_f) {
        a.hdr->counts[0] = cnt[0];
        a.hdr->counts[1] = cnt[1];
        a.hdr->counts[4] = cnt[4];
        a.hdr->counts[5] = cnt[5];
      }
      if (want_q) a.hdr->counts[2] = cnt[2];
      if (want_k) a.hdr->counts[3] = cnt[3];
      if (role == 0) {
        // words of the lists nobody builds in this call
        if (!(a.lists & 1)) {
          a.hdr->counts[0] = a.hdr->counts[1] = a.hdr->counts[4] = a.hdr->counts[5] = 0;
          a.hdr->list_status[0] = JFA_OK;
        }
        if (!(a.lists & 2)) { a.hdr->counts[2] = 0; a.hdr->list_status[1] = JFA_OK; }
        if (!(a.lists & 4)) { a.hdr->counts[3] = 0; a.hdr->list_status[2] = JFA_OK; }
        a.hdr->list_status[3] = JFA_OK;
        a.hdr->counts[6] = a.hdr->counts[7] = 0;
      }
    }
    if (role == 0)
      for (int i = 0; i < 8; ++i) a.hdr->tickets[i] = 0;
  }
  if (role == 0 && a.xtk && tid < XTK_KINDS * XTK_XCDS) a.xtk[tid * XTK_STRIDE] = 0;
}

// offsets[b+1] = offsets[b] + lengths[b], in int64 with an int32 range check; with bias_off,
// also the dense-bias block offsets bias_off[b+1] = bias_off[b] + lengths[b] * kv_lengths[b]
// (kv_lengths = lengths when null), in int64.  Nothing is written when a length is negative or
// the row total leaves int32.
__global__ __launch_bounds__(ST) void lengths_to_offsets_kernel(const int32_t* len,
                                                                const int32_t* kv_len, int32_t B,
                                                                int32_t* off, int64_t* bias_off,
                                                                int32_t* status) {
  __shared__ int64_t red[SW];
  __shared__ int32_t flag;
  if (threadIdx.x == 0) flag = 0;
  __syncthreads();
  // pass 1: validate (negative lengths, row total past int32)
  int64_t total = 0;
  int bad = 0;
  for (int64_t base = 0; base < B; base += ST) {
    const int64_t i = base + threadIdx.x;
    const int64_t v = i < B ? (int64_t)len[i] : 0;
    const int64_t kv = (i < B && kv_len) ? (int64_t)kv_len[i] : 0;
    if (v < 0 || kv < 0) bad = 1;
    int64_t tot;
    block_scan(v, &tot, red);
    total += tot;
  }
  if (total > INT32_MAX) bad = 1;
  if (bad) atomicOr(&flag, 1);
  __syncthreads();
  const bool ok = flag == 0;
  if (ok) {
    int64_t carry = 0, bcarry = 0;
    for (int64_t base = 0; base < B; base += ST) {
      const int64_t i = base + threadIdx.x;
      const int64_t v = i < B ? (int64_t)len[i] : 0;
      int64_t tot;
      const int64_t ex = block_scan(v, &tot, red);
      if (i < B) off[i] = (int32_t)(carry + ex);
      carry += tot;
      if (bias_off) {
        const int64_t kv = i < B ? (kv_len ? (int64_t)kv_len[i] : v) : 0;
        int64_t btot;
        const int64_t bex = block_scan(v * kv, &btot, red);
        if (i < B) bias_off[i] = bcarry + bex;
        bcarry += btot;
      }
    }
    if (threadIdx.x == 0) {
      off[B] = (int32_t)carry;
      if (bias_off) bias_off[B] = bcarry;
    }
  }
  if (threadIdx.x == 0 && status) *status = ok ? JFA_OK : JFA_ERR_DEVICE_DATA;
}

// BlockAttention's refined offsets: sample b (rows [off[b], off[b+1])) becomes ceil(n_b / W)
// samples, its consecutive blocks of W rows (the last one shorter), in sample order; entries
// past the last block up to out[out_batch] hold the total row count (empty samples).  The
// block count is found first, so nothing is written when it exceeds out_batch.
__global__ __launch_bounds__(ST) void block_offsets_kernel(const int32_t* off, int32_t B,
                                                           int32_t W, int32_t* out,
                                                           int32_t out_batch, int32_t* status) {
  __shared__ int64_t red[SW];
  __shared__ int32_t flag;
  if (threadIdx.x == 0) flag = 0;
  __syncthreads();
  int bad = 0;
  auto nblk = [&](int64_t b) -> int64_t {
    const int64_t n = (int64_t)off[b + 1] - off[b];
    if (n < 0) bad = 1;
    return n > 0 ? (n + W - 1) / W : 0;
  };
  // pass 1: the total number of blocks
  int64_t total = 0;
  for (int64_t base = 0; base < B; base += ST) {
    const int64_t b = base + threadIdx.x;
    int64_t tot;
    block_scan(b < B ? nblk(b) : 0, &tot, red);
    total += tot;
  }
  if (threadIdx.x == 0 && off[0] != 0) bad = 1;
  if (bad) atomicOr(&flag, 1);
  __syncthreads();
  const bool ok = flag == 0 && total <= out_batch;
  if (ok) {
    // pass 2: every sample writes its block starts at its exclusive block count
    int64_t carry = 0;
    for (int64_t base = 0; base < B; base += ST) {
      const int64_t b = base + threadIdx.x;
      const int64_t c = b < B ? nblk(b) : 0;
      int64_t tot;
      const int64_t e0 = carry + block_scan(c, &tot, red);
      for (int64_t k = 0; k < c; ++k) out[e0 + k] = (int32_t)(off[b] + k * W);
      carry += tot;
    }
    const int32_t end = off[B];
    for (int64_t e = total + threadIdx.x; e <= out_batch; e += ST) out[e] = end;
  }
  if (threadIdx.x == 0 && status) *status = ok ? JFA_OK : JFA_ERR_DEVICE_DATA;
}

}  // namespace

hipError_t launch_block_offsets(const int32_t* off, int32_t B, int32_t W, int32_t* out,
                                int32_t out_batch, int32_t* status, hipStream_t s) {
  timing_begin("jfa_block_offsets", s);
  hipLaunchKernelGGL(block_offsets_kernel, dim3(1), dim3(ST), 0, s, off, B, W, out, out_batch,
                     status);
  timing_end(s);
  return hipGetLastError();
}

hipError_t launch_schedule(const SchedArgs& a, hipStream_t s) {
  const size_t lds = sizeof(Shared);
  {
    hipError_t e = ensure_dyn_lds((const void*)schedule_kernel, lds);
    if (e != hipSuccess) return e;
  }
  const int roles = a.parallel ? __builtin_popcount(a.lists & 7) : 1;
  timing_begin("jfa_schedule", s);
  hipLaunchKernelGGL(schedule_kernel, dim3(roles + max(0, (int)a.delta_blocks)), dim3(ST), lds, s,
                     a);
  timing_end(s);
  return hipGetLastError();
}

hipError_t launch_lengths_to_offsets(const int32_t* len, const int32_t* kv_len, int32_t B,
                                     int32_t* off, int64_t* bias_off, int32_t* status,
                                     hipStream_t s) {
  timing_begin("jfa_offsets", s);
  hipLaunchKernelGGL(lengths_to_offsets_kernel, dim3(1), dim3(ST), 0, s, len, kv_len, B, off,
                     bias_off, status);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace jfa
