// Host side of libjfa: argument checks, tile configuration, workspace layout, launches.
// Entry points and their contracts are declared (with sources) in include/jfa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "jfa_internal.h"

namespace jfa {
namespace {

// ------------------------------------------------------------ device facts
int cu_count_of_current_device() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cache[dev] = cu;
  return cu;
}

// ------------------------------------------------------------- validation
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

jfa_status check_problem(const jfa_problem* p) {
  if (!p) return JFA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads < 1 || p->total_q < 0 || p->total_kv < 0) return JFA_ERR_INVALID_ARG;
  if (p->total_q > INT32_MAX || p->total_kv > INT32_MAX) return JFA_ERR_INVALID_ARG;
  if (p->mode < JFA_MODE_SOFTMAX || p->mode > JFA_MODE_GELU) return JFA_ERR_INVALID_ARG;
  if (p->dtype < JFA_F32 || p->dtype > JFA_MXFP8_E4M3) return JFA_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return JFA_ERR_INVALID_ARG;
  if (p->bias_kind < JFA_BIAS_NONE || p->bias_kind > JFA_BIAS_DENSE) return JFA_ERR_INVALID_ARG;
  if (p->bias_kind == JFA_BIAS_RELPOS && (p->num_buckets < 1 || p->num_buckets > 4096))
    return JFA_ERR_INVALID_ARG;
  if (p->kv_len_normalize < -1 || p->kv_len_normalize > 1) return JFA_ERR_INVALID_ARG;
  if (p->mode == JFA_MODE_SOFTMAX && p->kv_len_normalize == 1) return JFA_ERR_INVALID_ARG;
  if (!std::isfinite(p->qk_scale) || p->qk_scale < 0.f) return JFA_ERR_INVALID_ARG;
  if (p->bwd_fuse < -1 || p->bwd_fuse > 1) return JFA_ERR_INVALID_ARG;
  if (p->window < 0) return JFA_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return JFA_ERR_UNSUPPORTED;
  if ((int64_t)p->heads * p->head_dim > (1 << 20)) return JFA_ERR_UNSUPPORTED;
  return JFA_OK;
}

float qk_scale_of(const jfa_problem& p) {
  return p.qk_scale != 0.f ? p.qk_scale : 1.0f / std::sqrt((float)p.head_dim);
}
int normalize_of(const jfa_problem& p) {
  if (p.mode == JFA_MODE_SOFTMAX) return 0;
  return p.kv_len_normalize == 0 ? 0 : 1;
}

// Tile sizes: query tiles of 64 rows when samples are short on average, else 128.
jfa_status tile_cfg(const jfa_problem& p, TileCfg* t) {
  if (p.dtype == JFA_F32) {
    *t = TileCfg{F32_BM, F32_BN, -1, F32_BM, F32_BN, F32_BN, F32_BM, 0, 1, 1, 1};
    return JFA_OK;
  }
  const bool short_q = p.total_q <= 64 * (int64_t)p.batch;
  const bool short_kv = p.total_kv <= 64 * (int64_t)p.batch;
  // 64-row query tiles for short queries, and for a dense bias at d = 128 (the 128-row kernel
  // would spill registers holding the prefetched bias block)
  t->fwd_nw = (short_q || (p.bias_kind == JFA_BIAS_DENSE && p.head_dim == 128)) ? 2 : 4;
  t->bm = 32 * t->fwd_nw;
  t->bn = FWD_BN;
  if (p.split_slots > 0) {
    t->slots = p.split_slots;
  } else if (p.split_slots < 0) {
    t->slots = -1;
  } else {
    const int cu = cu_count_of_current_device();
    if (cu <= 0) return JFA_ERR_LAUNCH;
    // one slot per CU: a tile splits only when it is longer than twice the average work of a
    // resident workgroup.  (Two or four slots per CU, the resident workgroups, split tiles whose
    // chunks then re-load Q and write fp32 partials for little tail gain: the forward calls of
    // the causal, SiLU and MXFP8 workloads were 8-13% slower.)
    t->slots = cu;
  }
  t->bq_nw = short_q ? 2 : 4;
  t->bq_bm = 32 * t->bq_nw;
  t->bq_bn = BQ_BN;
  // key-stationary tiles: 128 keys, or 64 for short keys and for a dense bias at d = 128
  // (its key-major bias tile would not fit two LDS stages next to the Q / dO tiles)
  t->bk_nw = (short_kv || (p.bias_kind == JFA_BIAS_DENSE && p.head_dim == 128)) ? 2 : 4;
  t->bk_bn = 32 * t->bk_nw;
  t->bk_bm = BK_BM;
  // single-pass backward classes: bit 0, a sample with one query tile runs only the
  // query-stationary pass, which then also writes dK and dV (built for 64-row query tiles);
  // bit 1, a sample with one key tile runs only the key-stationary pass, which then also writes
  // dQ (built at d = 64)
  t->fuse = p.bwd_fuse == 0 ? 0 : ((t->bq_nw == 2 ? 1 : 0) | (p.head_dim == 64 ? 2 : 0));
  return JFA_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout layout_of(const jfa_problem& p, const TileCfg& tc, int backward) {
  Layout L{};
  const int64_t B = p.batch, H = p.heads, d = p.head_dim;
  const int64_t tiles_f = p.total_q / tc.bm + B + 1;
  L.cap_slots = tc.slots > 0 ? 2 * (int64_t)tc.slots / H + 2 : 0;
  L.cap_f = tiles_f + L.cap_slots;
  L.cap_c = tc.slots > 0 ? (int64_t)tc.slots / H + 2 : 1;
  L.cap_q = p.total_q / tc.bq_bm + B + 1;
  L.cap_k = p.total_kv / tc.bk_bn + B + 1;
  L.cap_t = std::max({L.cap_f, L.cap_q, L.cap_k, tiles_f});
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.header = take(sizeof(WsHeader));
  L.bias_off = take(8 * (B + 1));
  L.s_tmp = take(4 * (B + 1));
  L.t_tmp = take(4 * 4 * (L.cap_t + 1));
  L.gen_recs = take(16 * L.cap_t);
  L.gen_slot = take(4 * L.cap_t);
  L.words_a = take(4 * L.cap_t);
  L.words_b = take(4 * L.cap_t);
  L.fwd = take(sizeof(ItemRec) * L.cap_f);
  L.comb = take(16 * L.cap_c);
  L.bq = take(sizeof(ItemRec) * L.cap_q);
  L.bk = take(sizeof(ItemRec) * L.cap_k);
  L.xtk = take(XTK_BYTES);
  if (!backward && L.cap_slots > 0) {
    L.part_acc = take(4 * (size_t)L.cap_slots * H * tc.bm * d);
    L.part_ml = take(4 * 2 * (size_t)L.cap_slots * H * tc.bm);
  }
  if (backward && p.mode == JFA_MODE_SOFTMAX) L.delta = take(4 * (size_t)H * std::max<int64_t>(p.total_q, 1));
  if (backward == 2 && p.bias_kind == JFA_BIAS_RELPOS) {
    const size_t cols = (size_t)H * dbias_halves(p.num_buckets) * p.num_buckets;
    L.dbias_part = take(4 * cols * std::max<int64_t>(p.total_q, 1));
    L.dbias_chunk = take(4 * cols * dbias_chunks(p.heads, p.num_buckets, p.total_q));
  }
  L.total = off;
  return L;
}

SchedArgs sched_args(const jfa_problem& p, const TileCfg& tc, const Layout& L, char* ws,
                     const int32_t* q_off, const int32_t* kv_off) {
  SchedArgs a{};
  a.q_off = q_off;
  a.kv_off = kv_off;
  a.B = p.batch;
  a.H = p.heads;
  a.causal = p.causal;
  a.window = p.window;
  a.total_q = p.total_q;
  a.total_kv = p.total_kv;
  a.tc = tc;
  a.want_bias_off = p.bias_kind == JFA_BIAS_DENSE;   // only a dense bias is addressed by them
  a.lists = 7;
  a.hd_bytes = (int64_t)p.heads * p.head_dim * (p.dtype == JFA_F32 ? 4 : (p.dtype == JFA_BF16 ? 2 : 1));
  if (p.dtype == JFA_MXFP8_E4M3) a.hd_bytes = (int64_t)p.heads * p.head_dim * 2;   // bf16 output rows
  a.dense_bias = p.bias_kind == JFA_BIAS_DENSE;
  a.hdr = (WsHeader*)(ws + L.header);
  a.bias_off = (int64_t*)(ws + L.bias_off);
  a.s_tmp = (int32_t*)(ws + L.s_tmp);
  a.t_tmp = (int32_t*)(ws + L.t_tmp);
  a.gen_recs = (int4*)(ws + L.gen_recs);
  a.gen_slot = (int32_t*)(ws + L.gen_slot);
  a.words_a = (uint32_t*)(ws + L.words_a);
  a.words_b = (uint32_t*)(ws + L.words_b);
  a.fwd = nullptr;
  a.fwd_slot = nullptr;
  a.comb = (int4*)(ws + L.comb);
  a.bq = nullptr;
  a.bk = nullptr;
  a.xtk = (uint32_t*)(ws + L.xtk);
  a.fwd_items = (ItemRec*)(ws + L.fwd);
  a.bq_items = (ItemRec*)(ws + L.bq);
  a.bk_items = (ItemRec*)(ws + L.bk);
  a.cap_f = L.cap_f;
  a.cap_c = L.cap_c;
  a.cap_q = L.cap_q;
  a.cap_k = L.cap_k;
  a.cap_t = L.cap_t;
  a.cap_slots = L.cap_slots;
  a.counts_copy = nullptr;
  return a;
}

jfa_status from_hip(hipError_t e) { return e == hipSuccess ? JFA_OK : JFA_ERR_LAUNCH; }

// ------------------------------------------------------------------ timing
struct TimingRec {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRec> g_timing;
long g_timing_open = -1;   // index of the record waiting for its stop event

}  // namespace

void timing_begin(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing_on) return;
  TimingRec r;
  r.name = name;
  if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) return;
  if (hipEventRecord(r.start, s) != hipSuccess) return;
  g_timing.push_back(r);
  g_timing_open = (long)g_timing.size() - 1;
}

void timing_end(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing_on || g_timing_open < 0) return;
  (void)hipEventRecord(g_timing[g_timing_open].stop, s);
  g_timing_open = -1;
}

hipError_t ensure_dyn_lds(const void* kernel, size_t bytes) {
  static std::mutex mu;
  static std::unordered_map<std::string, int> done;   // (device, kernel, bytes) already set
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const std::string key = std::to_string(dev) + ":" + std::to_string((uintptr_t)kernel) + ":" +
                          std::to_string(bytes);
  std::lock_guard<std::mutex> lk(mu);
  if (done.count(key)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done[key] = 1;
  return e;
}

int resident_grid(const void* kernel, int threads, size_t dyn_lds, int cu_count) {
  static std::mutex mu;
  static std::unordered_map<std::string, int> cache;
  const std::string key = std::to_string((uintptr_t)kernel) + ":" + std::to_string(threads) + ":" +
                          std::to_string(dyn_lds);
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second * cu_count;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn_lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = per_cu;
  return per_cu * cu_count;
}

}  // namespace jfa

using namespace jfa;

extern "C" {

const char* jfa_status_string(jfa_status s) {
  switch (s) {
    case JFA_OK: return "JFA_OK";
    case JFA_ERR_INVALID_ARG: return "JFA_ERR_INVALID_ARG";
    case JFA_ERR_UNSUPPORTED: return "JFA_ERR_UNSUPPORTED";
    case JFA_ERR_WORKSPACE: return "JFA_ERR_WORKSPACE";
    case JFA_ERR_LAUNCH: return "JFA_ERR_LAUNCH";
    case JFA_ERR_DEVICE_DATA: return "JFA_ERR_DEVICE_DATA";
  }
  return "JFA_UNKNOWN_STATUS";
}

jfa_status jfa_tile_config(const jfa_problem* p, int32_t cfg_out[8]) {
  jfa_status st = check_problem(p);
  if (st != JFA_OK) return st;
  if (!cfg_out) return JFA_ERR_INVALID_ARG;
  TileCfg tc;
  st = tile_cfg(*p, &tc);
  if (st != JFA_OK) return st;
  const int32_t v[8] = {tc.bm, tc.bn, tc.slots, tc.bq_bm, tc.bq_bn, tc.bk_bn, tc.bk_bm, tc.fuse};
  std::memcpy(cfg_out, v, sizeof(v));
  return JFA_OK;
}

size_t jfa_workspace_bytes(const jfa_problem* p, int backward) {
  if (check_problem(p) != JFA_OK) return 0;
  TileCfg tc;
  if (tile_cfg(*p, &tc) != JFA_OK) return 0;
  return layout_of(*p, tc, backward < 0 ? 0 : std::min(backward, 2)).total;
}

jfa_status jfa_forward(const jfa_problem* p, const void* q, const void* k, const void* v,
                       const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                       const int32_t* q_offsets, const int32_t* kv_offsets, const void* bias,
                       void* o, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
  jfa_status st = check_problem(p);
  if (st != JFA_OK) return st;
  const bool fp8 = p->dtype == JFA_MXFP8_E4M3;
  if (!q || !k || !v || !o || !q_offsets || !kv_offsets || !workspace) return JFA_ERR_INVALID_ARG;
  if (fp8 && (!q_scale || !k_scale || !v_scale)) return JFA_ERR_INVALID_ARG;
  // a key's scale bytes are read as one word
  if (fp8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return JFA_ERR_INVALID_ARG;
  if ((p->bias_kind != JFA_BIAS_NONE) != (bias != nullptr)) return JFA_ERR_INVALID_ARG;
  if (p->mode == JFA_MODE_SOFTMAX && !lse) return JFA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(workspace, 256) || !aligned(q_offsets, 4) || !aligned(kv_offsets, 4) ||
      (lse && !aligned(lse, 4)) || (bias && !aligned(bias, 4)))
    return JFA_ERR_INVALID_ARG;
  TileCfg tc;
  st = tile_cfg(*p, &tc);
  if (st != JFA_OK) return st;
  const Layout L = layout_of(*p, tc, 0);
  if (workspace_bytes < L.total) return JFA_ERR_WORKSPACE;
  const int cu = cu_count_of_current_device();
  if (cu <= 0) return JFA_ERR_LAUNCH;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  SchedArgs a = sched_args(*p, tc, L, ws, q_offsets, kv_offsets);
  a.lists = 1;
  a.parallel = 1;
  hipError_t e = launch_schedule(a, s);
  if (e != hipSuccess) return JFA_ERR_LAUNCH;

  FwdParams fp{};
  fp.q = q; fp.k = k; fp.v = v;
  fp.q_sc = q_scale; fp.k_sc = k_scale; fp.v_sc = v_scale;
  fp.q_off = q_offsets; fp.kv_off = kv_offsets;
  fp.bias = bias;
  fp.bias_off = (const int64_t*)(ws + L.bias_off);
  fp.o = o; fp.lse = lse;
  fp.hdr_ro = (const WsHeader*)(ws + L.header);
  fp.hdr = (WsHeader*)(ws + L.header);
  fp.items = (const ItemRec*)(ws + L.fwd);
  fp.xtk = (uint32_t*)(ws + L.xtk) + TK_FWD * XTK_XCDS * XTK_STRIDE;
  fp.comb = (const int4*)(ws + L.comb);
  fp.part_acc = L.cap_slots > 0 ? (float*)(ws + L.part_acc) : nullptr;
  fp.part_ml = L.cap_slots > 0 ? (float*)(ws + L.part_ml) : nullptr;
  fp.H = p->heads;
  fp.causal = p->causal;
  fp.window = p->window;
  fp.bias_kind = p->bias_kind;
  fp.num_buckets = p->num_buckets;
  fp.normalize = normalize_of(*p);
  fp.scale = qk_scale_of(*p);
  fp.total_q = p->total_q;
  e = launch_forward(fp, tc, p->head_dim, p->mode, p->dtype, L.cap_f * p->heads,
                     L.cap_c * p->heads, cu, s);
  return from_hip(e);
}

namespace {

// MXFP8 scales of the backward's inputs (null for bf16 / fp32).
struct Fp8Scales {
  const uint8_t* q = nullptr;
  const uint8_t* k = nullptr;
  const uint8_t* v = nullptr;
  const uint8_t* dout = nullptr;
};

// The backward; with dbias (bias gradient wanted) the single-pass classes are off, so that every
// pair's dS is formed in the query-stationary pass.  sc: MXFP8 inputs (dtype JFA_MXFP8_E4M3).
jfa_status backward_impl(const jfa_problem* p, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout,
                         const int32_t* q_offsets, const int32_t* kv_offsets, const void* bias,
                         void* dq, void* dk, void* dv, void* dbias, void* workspace,
                         size_t workspace_bytes, void* stream, const Fp8Scales* sc) {
  jfa_status st = check_problem(p);
  if (st != JFA_OK) return st;
  const bool fp8 = p->dtype == JFA_MXFP8_E4M3;
  if (fp8 && !sc) return JFA_ERR_UNSUPPORTED;       // MXFP8 inputs come with their scales
  if (!fp8 && sc) return JFA_ERR_INVALID_ARG;
  if (fp8 && (!sc->q || !sc->k || !sc->v || !sc->dout)) return JFA_ERR_INVALID_ARG;
  if (dbias && (p->dtype != JFA_BF16 || p->bias_kind == JFA_BIAS_NONE))
    return JFA_ERR_UNSUPPORTED;
  if (dbias && !aligned(dbias, 4)) return JFA_ERR_INVALID_ARG;
  if (!q || !k || !v || !dout || !dq || !dk || !dv || !q_offsets || !kv_offsets || !workspace)
    return JFA_ERR_INVALID_ARG;
  if ((p->bias_kind != JFA_BIAS_NONE) != (bias != nullptr)) return JFA_ERR_INVALID_ARG;
  if (p->mode == JFA_MODE_SOFTMAX && (!o || !lse)) return JFA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || (o && !aligned(o, 16)) ||
      !aligned(workspace, 256) || !aligned(q_offsets, 4) || !aligned(kv_offsets, 4) ||
      (lse && !aligned(lse, 4)) || (bias && !aligned(bias, 4)))
    return JFA_ERR_INVALID_ARG;
  TileCfg tc;
  st = tile_cfg(*p, &tc);
  if (st != JFA_OK) return st;
  if (dbias) tc.fuse = 0;
  const Layout L = layout_of(*p, tc, dbias ? 2 : 1);
  if (workspace_bytes < L.total) return JFA_ERR_WORKSPACE;
  const int cu = cu_count_of_current_device();
  if (cu <= 0) return JFA_ERR_LAUNCH;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  SchedArgs a = sched_args(*p, tc, L, ws, q_offsets, kv_offsets);
  a.lists = 6;
  a.parallel = 1;
  if (p->mode == JFA_MODE_SOFTMAX && p->total_q > 0) {
    // D = rowsum(dO * O) runs on the workgroups the two list builders leave idle
    a.d_o = o;
    a.d_dout = dout;
    a.d_delta = (float*)(ws + L.delta);
    a.d_head_dim = p->head_dim;
    a.d_esize = p->dtype == JFA_F32 ? 4 : 2;
    a.d_dout_sc = fp8 ? sc->dout : nullptr;
    a.delta_blocks = std::max(1, cu - 2);
  }
  hipError_t e = launch_schedule(a, s);
  if (e != hipSuccess) return JFA_ERR_LAUNCH;

  BwdParams bp{};
  bp.q = q; bp.k = k; bp.v = v; bp.o = o; bp.lse = lse; bp.dout = dout;
  if (fp8) {
    bp.q_sc = sc->q; bp.k_sc = sc->k; bp.v_sc = sc->v; bp.do_sc = sc->dout;
  }
  bp.q_off = q_offsets; bp.kv_off = kv_offsets;
  bp.bias = bias;
  bp.bias_off = (const int64_t*)(ws + L.bias_off);
  bp.dq = dq; bp.dk = dk; bp.dv = dv;
  bp.delta = p->mode == JFA_MODE_SOFTMAX ? (float*)(ws + L.delta) : nullptr;
  bp.hdr = (WsHeader*)(ws + L.header);
  bp.bq = (const ItemRec*)(ws + L.bq);
  bp.bk = (const ItemRec*)(ws + L.bk);
  bp.xtk_q = (uint32_t*)(ws + L.xtk) + TK_BQ * XTK_XCDS * XTK_STRIDE;
  bp.xtk_k = (uint32_t*)(ws + L.xtk) + TK_BK * XTK_XCDS * XTK_STRIDE;
  bp.batch = p->batch;
  bp.H = p->heads;
  bp.causal = p->causal;
  bp.window = p->window;
  bp.bias_kind = p->bias_kind;
  bp.num_buckets = p->num_buckets;
  bp.normalize = normalize_of(*p);
  bp.mode = p->mode;
  bp.fuse = tc.fuse;
  bp.bq_bm = tc.bq_bm;
  bp.bk_bn = tc.bk_bn;
  bp.scale = qk_scale_of(*p);
  bp.total_q = p->total_q;
  bp.total_kv = p->total_kv;
  if (dbias) {
    bp.dbias = dbias;
    bp.dbias_part = p->bias_kind == JFA_BIAS_RELPOS ? (float*)(ws + L.dbias_part) : nullptr;
    bp.dbias_chunk = p->bias_kind == JFA_BIAS_RELPOS ? (float*)(ws + L.dbias_chunk) : nullptr;
    e = launch_backward_dbias(bp, tc, p->head_dim, L.cap_q * p->heads, L.cap_k * p->heads, cu, s);
  } else {
    e = launch_backward(bp, tc, p->head_dim, p->dtype, L.cap_q * p->heads, L.cap_k * p->heads,
                        cu, s);
  }
  return from_hip(e);
}

}  // namespace

jfa_status jfa_backward(const jfa_problem* p, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        const int32_t* q_offsets, const int32_t* kv_offsets, const void* bias,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return backward_impl(p, q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, dq, dk, dv,
                       nullptr, workspace, workspace_bytes, stream, nullptr);
}

jfa_status jfa_backward_mxfp8(const jfa_problem* p, const uint8_t* q, const uint8_t* k,
                              const uint8_t* v, const uint8_t* q_scale, const uint8_t* k_scale,
                              const uint8_t* v_scale, const void* o, const float* lse,
                              const uint8_t* dout, const uint8_t* dout_scale,
                              const int32_t* q_offsets, const int32_t* kv_offsets,
                              const void* bias, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!p) return JFA_ERR_INVALID_ARG;
  if (p->dtype != JFA_MXFP8_E4M3) return JFA_ERR_INVALID_ARG;
  if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(dout_scale, 4))
    return JFA_ERR_INVALID_ARG;
  Fp8Scales sc;
  sc.q = q_scale;
  sc.k = k_scale;
  sc.v = v_scale;
  sc.dout = dout_scale;
  return backward_impl(p, q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, dq, dk, dv,
                       nullptr, workspace, workspace_bytes, stream, &sc);
}

jfa_status jfa_backward_dbias(const jfa_problem* p, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dout,
                              const int32_t* q_offsets, const int32_t* kv_offsets,
                              const void* bias, void* dq, void* dk, void* dv, void* dbias,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!dbias) return JFA_ERR_INVALID_ARG;
  return backward_impl(p, q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, dq, dk, dv, dbias,
                       workspace, workspace_bytes, stream, nullptr);
}

jfa_status jfa_build_schedule(const jfa_problem* p, const int32_t* q_offsets,
                              const int32_t* kv_offsets, int32_t* fwd, int32_t* fwd_slot,
                              int32_t* comb, int32_t* bwd_q, int32_t* bwd_kv, int32_t* counts,
                              int64_t capacity, void* workspace, size_t workspace_bytes,
                              void* stream) {
  jfa_status st = check_problem(p);
  if (st != JFA_OK) return st;
  if (!q_offsets || !kv_offsets || !fwd || !fwd_slot || !comb || !bwd_q || !bwd_kv || !counts ||
      !workspace || capacity < 0)
    return JFA_ERR_INVALID_ARG;
  TileCfg tc;
  st = tile_cfg(*p, &tc);
  if (st != JFA_OK) return st;
  const Layout L = layout_of(*p, tc, 0);
  if (workspace_bytes < L.total) return JFA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  SchedArgs a = sched_args(*p, tc, L, ws, q_offsets, kv_offsets);
  a.fwd = (int4*)fwd;
  a.fwd_slot = fwd_slot;
  a.comb = (int4*)comb;
  a.bq = (int4*)bwd_q;
  a.bk = (int4*)bwd_kv;
  a.fwd_items = a.bq_items = a.bk_items = nullptr;
  a.cap_f = std::min<int64_t>(capacity, L.cap_f);
  a.cap_c = std::min<int64_t>(capacity, L.cap_c);
  a.cap_q = std::min<int64_t>(capacity, L.cap_q);
  a.cap_k = std::min<int64_t>(capacity, L.cap_k);
  a.counts_copy = counts;
  return from_hip(launch_schedule(a, (hipStream_t)stream));
}

jfa_status jfa_lengths_to_offsets(const int32_t* lengths, int32_t batch, int32_t* offsets,
                                  int64_t* bias_offsets_or_null,
                                  const int32_t* kv_lengths_or_null, int32_t* status,
                                  void* stream) {
  if (!lengths || !offsets || batch < 0) return JFA_ERR_INVALID_ARG;
  if (!aligned(lengths, 4) || !aligned(offsets, 4) || (status && !aligned(status, 4)) ||
      (bias_offsets_or_null && !aligned(bias_offsets_or_null, 8)) ||
      (kv_lengths_or_null && !aligned(kv_lengths_or_null, 4)))
    return JFA_ERR_INVALID_ARG;
  return from_hip(launch_lengths_to_offsets(lengths, kv_lengths_or_null, batch, offsets,
                                            bias_offsets_or_null, status, (hipStream_t)stream));
}

jfa_status jfa_block_offsets(const int32_t* offsets, int32_t batch, int32_t block,
                             int32_t* block_offsets, int32_t out_batch, int32_t* status,
                             void* stream) {
  if (!offsets || !block_offsets || batch < 0 || block < 1 || out_batch < 0)
    return JFA_ERR_INVALID_ARG;
  if (!aligned(offsets, 4) || !aligned(block_offsets, 4) || (status && !aligned(status, 4)))
    return JFA_ERR_INVALID_ARG;
  return from_hip(launch_block_offsets(offsets, batch, block, block_offsets, out_batch, status,
                                       (hipStream_t)stream));
}

jfa_status jfa_quantize_mxfp8(const void* x_bf16, int64_t rows, int32_t d, uint8_t* codes,
                              uint8_t* scales, void* stream) {
  if (rows < 0 || d <= 0 || d % 32 != 0) return JFA_ERR_INVALID_ARG;
  if (rows == 0) return JFA_OK;            // an empty tensor may have null pointers
  if (!x_bf16 || !codes || !scales) return JFA_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(codes, 8)) return JFA_ERR_INVALID_ARG;
  return from_hip(launch_quantize_mxfp8(x_bf16, rows, d, codes, scales, (hipStream_t)stream));
}

jfa_status jfa_quantize_mxfp8_batch(int32_t count, const void* const* xs_bf16,
                                    const int64_t* rows, int32_t d, uint8_t* const* codes,
                                    uint8_t* const* scales, void* stream) {
  if (count < 1 || count > 4 || !xs_bf16 || !rows || !codes || !scales || d <= 0 || d % 32 != 0)
    return JFA_ERR_INVALID_ARG;
  for (int t = 0; t < count; ++t) {
    if (rows[t] < 0) return JFA_ERR_INVALID_ARG;
    if (rows[t] == 0) continue;           // an empty tensor may have null pointers
    if (!xs_bf16[t] || !codes[t] || !scales[t]) return JFA_ERR_INVALID_ARG;
    if (!aligned(xs_bf16[t], 16) || !aligned(codes[t], 8)) return JFA_ERR_INVALID_ARG;
  }
  const int cu = cu_count_of_current_device();
  if (cu <= 0) return JFA_ERR_LAUNCH;
  return from_hip(launch_quantize_mxfp8_batch(count, xs_bf16, rows, d, codes, scales, cu,
                                              (hipStream_t)stream));
}

jfa_status jfa_rmsnorm_quantize_mxfp8(const void* x_bf16, const float* weight, int64_t groups,
                                      int32_t n, float eps, uint8_t* codes, uint8_t* scales,
                                      void* stream) {
  if (!x_bf16 || !codes || !scales || groups < 0) return JFA_ERR_INVALID_ARG;
  if (n != 32 && n != 64 && n != 128 && n != 256 && n != 512) return JFA_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return JFA_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(codes, 8) || (weight && !aligned(weight, 16)))
    return JFA_ERR_INVALID_ARG;
  return from_hip(launch_rmsnorm_quantize_mxfp8(x_bf16, weight, groups, n, eps, codes, scales,
                                                (hipStream_t)stream));
}

jfa_status jfa_read_device_status(const void* workspace, void* stream, int32_t* status_out) {
  if (!workspace || !status_out) return JFA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return JFA_ERR_LAUNCH;
  WsHeader h;
  if (hipMemcpy(&h, workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return JFA_ERR_LAUNCH;
  // the offsets check, then the per-list capacity checks
  int32_t v = h.status;
  for (int i = 0; i < 3 && v == JFA_OK; ++i) v = h.list_status[i];
  *status_out = v;
  return JFA_OK;
}

void jfa_set_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = enable != 0;
}

jfa_status jfa_kernel_timing(const char* name_prefix, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return JFA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  const std::string pre = name_prefix ? name_prefix : "";
  double tot = 0.0;
  int64_t cnt = 0;
  for (auto& r : g_timing) {
    if (r.name.compare(0, pre.size(), pre) != 0) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return JFA_ERR_LAUNCH;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return JFA_ERR_LAUNCH;
    tot += ms;
    ++cnt;
  }
  *total_ms = tot;
  *launches = cnt;
  return JFA_OK;
}

void jfa_kernel_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (auto& r : g_timing) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_timing.clear();
  g_timing_open = -1;
}

}  // extern "C"
