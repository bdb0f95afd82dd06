// Internal declarations shared by the libjfa HIP sources (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/jfa.h"

namespace jfa {

// ------------------------------------------------------------------ tiles
// Forward (bf16 / MXFP8): one workgroup owns FWD_BM query rows (32 per wave) of one head and
// walks the sample's keys FWD_BN at a time.
constexpr int FWD_BN = 64;
// fp32 path (SIMT): one thread per query (or key) row, 64 rows per workgroup.
constexpr int F32_BM = 64;
constexpr int F32_BN = 64;
// Backward q-stationary pass: 32 query rows per wave, keys in steps of BQ_BN.
constexpr int BQ_BN = 64;
// Backward kv-stationary pass: 32 key rows per wave, queries in steps of BK_BM.
constexpr int BK_BM = 64;

// Upper bound of a record's cost (kv or q steps) that the list sort accepts.
constexpr int MAX_COST = 4095;

// Step range [s0, s1) of `step`-row key steps that query rows [r0, r1) of a sample with n
// queries and m keys can see: key j is visible to query i iff j <= i + (m - n) (causal) and,
// with a window W > 0, i + (m - n) - W < j < i + (m - n) + W.  Empty: s0 = s1 = `empty`.
__host__ __device__ inline void visible_key_steps(int causal, int window, int64_t r0, int64_t r1,
                                                  int64_t n, int64_t m, int step, int64_t empty,
                                                  int64_t& s0, int64_t& s1) {
  const int64_t dl = m - n;
  int64_t a = 0, e = m;
  if (window > 0) {
    a = r0 + dl - window + 1;
    e = r1 - 1 + dl + window;
  }
  if (causal && r1 + dl < e) e = r1 + dl;
  if (a < 0) a = 0;
  if (e > m) e = m;
  if (e > a) {
    s0 = a / step;
    s1 = (e + step - 1) / step;
  } else {
    s0 = s1 = empty;
  }
}
// Step range of `step`-row query steps that keys [c0, c1) can be seen from (same rule).
__host__ __device__ inline void visible_query_steps(int causal, int window, int64_t c0,
                                                    int64_t c1, int64_t n, int64_t m, int step,
                                                    int64_t empty, int64_t& s0, int64_t& s1) {
  const int64_t dl = m - n;
  int64_t a = 0, e = n;
  if (window > 0) {
    a = c0 - dl - window + 1;
    e = c1 - 1 - dl + window;
  }
  if (causal && c0 - dl > a) a = c0 - dl;
  if (a < 0) a = 0;
  if (e > n) e = n;
  if (e > a) {
    s0 = a / step;
    s1 = (e + step - 1) / step;
  } else {
    s0 = s1 = empty;
  }
}

// ------------------------------------------------------------ workspace
// Header at the start of every workspace (device memory, 256 bytes).
struct WsHeader {
  int32_t status;      // JFA_OK or JFA_ERR_DEVICE_DATA
  int32_t counts[8];   // forward, combine, q-stationary, kv-stationary records, threshold, slots
  uint32_t tickets[8]; // work counters for persistent kernels, zeroed by the scheduler
  int32_t list_status[4]; // per list (forward, q-stationary, kv-stationary): JFA_OK, or
                          // JFA_ERR_DEVICE_DATA when the list did not fit its capacity
  int32_t pad[64 - 21];
};
static_assert(sizeof(WsHeader) == 256, "header size");

enum Ticket { TK_FWD = 0, TK_COMB = 1, TK_BQ = 2, TK_BK = 3, TK_DELTA = 4 };
// Per-XCD work counters: kind k, XCD x at dword (8 k + x) * 32 of the workspace's counter area.
constexpr int XTK_KINDS = 8, XTK_XCDS = 8, XTK_STRIDE = 32;
constexpr size_t XTK_BYTES = (size_t)XTK_KINDS * XTK_XCDS * XTK_STRIDE * 4;

struct TileCfg {
  int bm, bn;          // forward tile rows (query), kv step rows
  int slots;           // split slots (<=0: no split)
  int bq_bm, bq_bn;    // q-stationary backward
  int bk_bn, bk_bm;    // kv-stationary backward
  int fuse;            // single-pass backward classes: bit 0 one query tile, bit 1 one key tile
  int fwd_nw, bq_nw, bk_nw;   // waves per workgroup of the three MFMA kernels
};

// Byte layout of the workspace for one problem.
struct Layout {
  size_t header, bias_off, s_tmp, t_tmp, gen_recs, gen_slot, words_a, words_b;
  size_t fwd, comb, bq, bk, xtk;
  size_t part_acc, part_ml, delta;
  size_t dbias_part, dbias_chunk;   // backward with the relative-position table's gradient
  size_t total;
  int64_t cap_f, cap_c, cap_q, cap_k, cap_t, cap_slots;
};

// Work record of the persistent kernels (64 bytes): a list record together with everything a
// kernel needs to start the item, so that one load describes it.
struct ItemRec {
  int32_t b, x, y, z;      // the list record: sample, tile, range (see jfa_build_schedule)
  int32_t slot;            // forward split slot (-1: not split)
  int32_t qo, n, ko, m;    // the sample's first q / kv row and its lengths
  int32_t pad0;
  int64_t boff;            // element offset of the sample's dense-bias block over all heads
  int32_t pad1[4];
};
static_assert(sizeof(ItemRec) == 64, "item record size");

// ------------------------------------------------------- scheduler args
struct SchedArgs {
  const int32_t* q_off;
  const int32_t* kv_off;
  int32_t B, H, causal;
  int32_t window;      // sliding window (0 = none)
  int64_t total_q, total_kv;
  TileCfg tc;
  int want_bias_off;
  int lists;           // bit 0: forward + combine, bit 1: q-stationary, bit 2: kv-stationary
  int64_t hd_bytes;    // bytes of one (row, all heads) vector: H * d * element size
  int32_t dense_bias;  // dense bias present (its per-sample block must fit 32-bit offsets)
  WsHeader* hdr;
  int64_t* bias_off;
  int32_t* s_tmp;      // per-sample scratch [4][B+1]
  int32_t* t_tmp;      // per-tile scratch [4][cap_t+1]
  int4* gen_recs;      // records in generation order
  int32_t* gen_slot;
  uint32_t* words_a;   // sort buffers (global fallback)
  uint32_t* words_b;
  int4* fwd;            // list records (test hook; may be null)
  int32_t* fwd_slot;
  int4* comb;
  int4* bq;
  int4* bk;
  ItemRec* fwd_items;   // the same lists as kernel work records (may be null)
  ItemRec* bq_items;
  ItemRec* bk_items;
  int64_t cap_f, cap_c, cap_q, cap_k, cap_t, cap_slots;
  int32_t* counts_copy; // optional: counts also written here (test hook)
  uint32_t* xtk;        // per-XCD work counters of the persistent kernels (zeroed here)
  int32_t parallel;     // 1: one workgroup per requested list; 0: one workgroup builds them all
  // softmax backward preprocess D = rowsum(dO * O), run by the workgroups after the list
  // builders (delta_blocks of them; 0 = none)
  const void* d_o;
  const void* d_dout;
  float* d_delta;       // [H][total_q]
  int32_t delta_blocks;
  int32_t d_head_dim;
  int32_t d_esize;      // bytes per element of O / dO (2 bf16, 4 fp32)
  const uint8_t* d_dout_sc;   // MXFP8 dO: E4M3 codes in d_dout, E8M0 scales here (O is bf16)
};

// ----------------------------------------------------- kernel parameters
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* q_sc;
  const uint8_t* k_sc;
  const uint8_t* v_sc;
  const int32_t* q_off;
  const int32_t* kv_off;
  const void* bias;
  const int64_t* bias_off;
  void* o;
  float* lse;
  const WsHeader* hdr_ro;
  WsHeader* hdr;
  const ItemRec* items;
  uint32_t* xtk;       // per-XCD work counters of this kernel
  const int4* comb;
  float* part_acc;
  float* part_ml;
  int32_t H;
  int32_t causal;
  int32_t window;     // sliding window (0 = none)
  int32_t bias_kind;
  int32_t num_buckets;
  int32_t normalize;
  float scale;        // qk scale
  int64_t total_q;
};

struct BwdParams {
  const void* q;          // bf16 / fp32 values, or MXFP8 codes (then the scales below)
  const void* k;
  const void* v;
  const uint8_t* q_sc;    // MXFP8 E8M0 scales [rows][H][d/32] of q, k, v and dout (else null)
  const uint8_t* k_sc;
  const uint8_t* v_sc;
  const uint8_t* do_sc;
  const void* o;
  const float* lse;
  const void* dout;
  const int32_t* q_off;
  const int32_t* kv_off;
  const void* bias;
  const int64_t* bias_off;
  void* dq;
  void* dk;
  void* dv;
  float* delta;        // [H][total_q] (softmax)
  void* dbias;         // bias gradient (dense bias: bias layout, bf16) or null
  float* dbias_part;   // relative-position table: per-row sums [total_q][H][halves][buckets]
                       // (halves = dbias_halves(buckets)), or null
  float* dbias_chunk;  // and their per-chunk sums [dbias_chunks(...)][H][halves][buckets]
  WsHeader* hdr;
  const ItemRec* bq;
  const ItemRec* bk;
  uint32_t* xtk_q;     // per-XCD work counters of the query-stationary kernel
  uint32_t* xtk_k;     // and of the key-stationary kernel
  int32_t batch;
  int32_t H;
  int32_t causal;
  int32_t window;      // sliding window (0 = none)
  int32_t bias_kind;
  int32_t num_buckets;
  int32_t normalize;
  int32_t mode;
  int32_t fuse;
  int32_t bq_bm;       // q-stationary tile rows (for the single-pass class test)
  int32_t bk_bn;       // kv-stationary tile rows
  float scale;
  int64_t total_q;
  int64_t total_kv;
};

// Bias gradient of a relative-position table: tables of at most DB_NB buckets are summed per
// lane in LDS and leave one partial row per query row and head (halves 1); wider tables leave
// one per lane half (halves 2).  The rows are reduced in `dbias_chunks` chunks (at most 512,
// and at most 4M floats of chunk sums).
constexpr int DB_NB = 64;
inline int dbias_halves(int nb) { return nb <= DB_NB ? 1 : 2; }
inline int dbias_chunks(int H, int nb, int64_t rows) {
  const int64_t cols = (int64_t)H * dbias_halves(nb) * nb;
  int64_t c = (int64_t)(4 << 20) / cols;
  if (c > 512) c = 512;
  if (c > rows) c = rows;
  return c < 1 ? 1 : (int)c;
}

// ---------------------------------------------------------- launchers
// Each returns hipSuccess or the first launch error.  `grid_slots` sizes persistent grids.
hipError_t launch_schedule(const SchedArgs& a, hipStream_t s);
hipError_t launch_lengths_to_offsets(const int32_t* len, const int32_t* kv_len, int32_t B,
                                     int32_t* off, int64_t* bias_off, int32_t* status,
                                     hipStream_t s);
hipError_t launch_forward(const FwdParams& p, const TileCfg& tc, int head_dim, int mode, int dtype,
                          int64_t max_items, int64_t max_comb_items, int cu_count, hipStream_t s);
hipError_t launch_backward(const BwdParams& p, const TileCfg& tc, int head_dim, int dtype,
                           int64_t max_q_items, int64_t max_k_items, int cu_count, hipStream_t s);
// The backward with the bias gradient (bf16, bias present, tc.fuse == 0): dbias as for p.dbias;
// the relative-position table's partials in p.dbias_part.
hipError_t launch_backward_dbias(const BwdParams& p, const TileCfg& tc, int head_dim,
                                 int64_t max_q_items, int64_t max_k_items, int cu_count,
                                 hipStream_t s);
// The MFMA backward of one (head dim, mode, input format) triple (bwd_inst.hip, one translation
// unit per triple; FP8: MXFP8 inputs); dbias: the variant with the bias gradient (bf16 inputs,
// bias present, tc.fuse == 0).
template <int D, int MODE, bool FP8>
hipError_t launch_bwd_dm(const BwdParams& p, const TileCfg& tc, int64_t max_q_items,
                         int64_t max_k_items, int cu_count, hipStream_t s, bool dbias);
#define JFA_DECLARE_BWD_DM(D_, M_, F_)                                                      \
  template <>                                                                               \
  hipError_t launch_bwd_dm<D_, M_, F_>(const BwdParams&, const TileCfg&, int64_t, int64_t, \
                                       int, hipStream_t, bool);
JFA_DECLARE_BWD_DM(128, 0, false)
JFA_DECLARE_BWD_DM(128, 1, false)
JFA_DECLARE_BWD_DM(128, 2, false)
JFA_DECLARE_BWD_DM(64, 0, false)
JFA_DECLARE_BWD_DM(64, 1, false)
JFA_DECLARE_BWD_DM(64, 2, false)
JFA_DECLARE_BWD_DM(128, 0, true)
JFA_DECLARE_BWD_DM(128, 1, true)
JFA_DECLARE_BWD_DM(128, 2, true)
JFA_DECLARE_BWD_DM(64, 0, true)
JFA_DECLARE_BWD_DM(64, 1, true)
JFA_DECLARE_BWD_DM(64, 2, true)
#undef JFA_DECLARE_BWD_DM

// Sets a kernel's dynamic-LDS limit once per device (thread-safe).
hipError_t ensure_dyn_lds(const void* kernel, size_t bytes);

hipError_t launch_block_offsets(const int32_t* off, int32_t B, int32_t W, int32_t* out,
                                int32_t out_batch, int32_t* status, hipStream_t s);
hipError_t launch_quantize_mxfp8_batch(int32_t count, const void* const* xs,
                                       const int64_t* rows, int32_t d, uint8_t* const* codes,
                                       uint8_t* const* scales, int cu_count, hipStream_t s);
hipError_t launch_quantize_mxfp8(const void* x, int64_t rows, int32_t d, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s);
hipError_t launch_rmsnorm_quantize_mxfp8(const void* x, const float* w, int64_t groups, int32_t n,
                                         float eps, uint8_t* codes, uint8_t* scales,
                                         hipStream_t s);

// Kernel timing hooks (api.cpp): bracket a launch with events when timing is enabled.
void timing_begin(const char* name, hipStream_t s);
void timing_end(hipStream_t s);

// Persistent-grid size: concurrent workgroups of `kernel` on the device (at least 1 per CU).
int resident_grid(const void* kernel, int threads, size_t dyn_lds, int cu_count);

}  // namespace jfa
