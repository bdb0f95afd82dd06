// Jagged flash attention forward on MFMA (bf16 or MXFP8 inputs) and the split-KV combine.
//
// Source: "Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a Different Stack",
// section "Bottleneck move 1" (attention directly on jagged tensors, custom biases,
// asymmetric q/kv lengths, GDPA with GELU/SiLU in place of softmax) and "Meta Enhances GEM
// Training Efficiency ...", section "Leveraging Compute Efficiency through Customized
// Kernels" (MXFP8 attention).
//
// Design (gfx950):
//  - A workgroup of NW waves owns BM = 32*NW query rows of one head of one sample and walks
//    the keys 64 at a time.  Each step's K and V tiles (row-major; the V^T operand of PV is
//    read with transposing LDS reads) sit in one of two LDS stages: the next step's global
//    loads are issued before this step's MFMAs and land in the other stage after them, so one
//    barrier per step suffices.
//  - Global loads go through per-(sample, head) buffer resources whose size ends at the
//    sample's last row: rows past the end read as zeros with no branches.
//  - Each wave computes S^T = K Q^T (32x32x16 bf16 MFMA, or the scaled 32x32x64 E4M3 MFMA
//    with the MX block scales applied in hardware).  In the transposed accumulator a lane
//    holds one query column, so the softmax row max/sum are in-lane reductions plus one
//    exchange with the lane 32 away, and the probabilities P^T are already laid out as the B
//    operand of O^T += V^T P^T: no LDS round trip for P.
//  - The additive bias enters as the initial value of the S^T accumulator (bias / qk_scale),
//    so it costs no VALU add: a relative-position bias from a per-step diagonal table in
//    LDS, a dense bias from an LDS tile staged with coalesced loads.
//  - Softmax keeps (max, sum) online in the log2 domain and rescales the accumulator only when
//    the running max grows by more than 8 (2^8 headroom in fp32); the row sum is kept in
//    fp32 from the unrounded probabilities.  GDPA applies the activation
//    elementwise and scales by 1/kv_len at the end.
//  - Work items (tile record, head) come from the longest-first list; persistent workgroups
//    take them with an atomic ticket.  Records that are chunks of a split tile write fp32
//    partials (unnormalised accumulator, max, sum) that the combine kernel merges in chunk
//    order.
#include <algorithm>

#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

constexpr int BN = FWD_BN;
enum BiasT { B_NONE = 0, B_RELPOS = 1, B_DENSE = 2 };

constexpr int align16(int x) { return (x + 15) / 16 * 16; }

// Dynamic LDS layout of one pipeline stage of the forward kernel (two stages are used).
template <int D, int NW, int BIAS, bool FP8>
struct FwdLds {
  static constexpr int BM = 32 * NW;
  static constexpr int KRB = FP8 ? (D + 16) : 2 * (D + 8);   // K row stride in bytes
  static constexpr int K_BYTES = BN * KRB;
  static constexpr int KSC_BYTES = FP8 ? BN * 4 : 0;          // K scales: one dword per key
  static constexpr int VS = tile_row_stride<D>();              // V row stride (bf16)
  static constexpr int V_OFF = align16(K_BYTES + KSC_BYTES);
  static constexpr int V_BYTES = BN * VS * 2;
  static constexpr int RP = diag_stride(BM + BN + 4);          // relpos copy length (floats)
  static constexpr int BS = BN + 8;                            // dense bias row stride (bf16)
  static constexpr int BIAS_BYTES =
      BIAS == B_RELPOS ? 4 * RP * 4 : (BIAS == B_DENSE ? BM * BS * 2 : 0);
  static constexpr int B_OFF = V_OFF + V_BYTES;
  // a stage also holds the epilogue's output rows (one staging area per wave)
  static constexpr int STAGE = align16(B_OFF + BIAS_BYTES) > NW * out_stage_bytes<D>()
                                   ? align16(B_OFF + BIAS_BYTES) : NW * out_stage_bytes<D>();
  static constexpr int TOTAL = 2 * STAGE;
};

// Occupancy: two workgroups per CU.  With 4 waves per workgroup that is 2 waves per SIMD
// (256 registers each); with 2 waves it is one wave per SIMD, which may use all 512.
// WIN: a sliding window is set (its bounds only cost registers and VALU where it is).
template <int D, int NW, int MODE, int BIAS, bool FP8, bool WIN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 2, NW / 2)))
void fwd_kernel(FwdParams p) {
  using L = FwdLds<D, NW, BIAS, FP8>;
  constexpr int BM = L::BM, NT = NW * 64, VS = L::VS;
  constexpr int ES = FP8 ? 1 : 2;                  // bytes per Q/K/V element
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_desc[2][IF_WORDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int H = p.H;
  if (p.hdr_ro->status != JFA_OK) return;
  const int64_t n_items = (int64_t)p.hdr_ro->counts[0] * H;
  // scores are handled as raw = q.k + bias/scale; x = raw * c_log is the (log2) logit
  const float c_log = MODE == MODE_SOFTMAX ? p.scale * LOG2E : p.scale;
  const float inv_scale = 1.0f / p.scale;
  const uint32_t row_bytes = (uint32_t)H * D * ES;           // stride between tokens
  const uint32_t sc_row_bytes = (uint32_t)H * (D / 32);      // MXFP8 scales stride

  // staging assignments
  constexpr int KCH = D * ES / 16;                          // 16-byte chunks per K row
  constexpr int K_LOADS = BN * KCH / NT;                    // per thread
  static_assert(BN * KCH % NT == 0, "K staging");
  constexpr int VBLK = (BN / 4) * (D / 8);                  // 4 keys x 8 dims blocks of V
  // this lane's element of a transposing read: row 4(G/2) + (j/4), column 16(G%2) + 4(j%4) for
  // 16-lane group G and lane j within it (plus the operand's base row and column)
  const int tr_lane = (4 * (lane >> 5) + ((lane & 15) >> 2)) * VS + 16 * ((lane >> 4) & 1) +
                      4 * (lane & 3);
  constexpr int V_LOADS = (VBLK + NT - 1) / NT;

  u32x4 kreg[K_LOADS];
  uint32_t kscreg = 0;
  u32x4 v16[FP8 ? 1 : V_LOADS][4];
  u32x2 v8[FP8 ? V_LOADS : 1][4];
  uint32_t vsc[FP8 ? V_LOADS : 1][4];
  float rp_val = 0.f;                                        // relpos table entry of this thread
  // Dense bias: NDB 16-byte chunks (8 keys of one query row) per thread and step, prefetched
  // into registers with the K/V tiles.
  constexpr int NDB = BIAS == B_DENSE ? BM * (BN / 8) / NT : 1;
  static_assert(!(BIAS == B_DENSE && D == 128 && NW == 4), "dense bias takes 64-row tiles");
  BiasRaw dbr[NDB];

  // Cross-item prefetch: the query fragment and first tiles of the next item are loaded before
  // the last key step of the current one, so that a run of short items keeps loads in flight
  // behind their compute and epilogues.  It needs registers for a second query fragment, which
  // the 4-wave kernel at d = 128 does not have.
  constexpr bool XPF = !(D == 128 && NW == 4);

  // what one item's loads read, from its descriptor (wave-uniform)
  struct Src {
    rsrc_t rk, rv, rq, rks, rvs, rqs, rb;
    int h, q0, n, m, kb, ke;
  };
  auto make_src = [&](const int* d) -> Src {
    Src s;
    s.h = item_field(d, IF_W) % H;
    s.q0 = item_field(d, IF_X) * BM;
    s.kb = item_field(d, IF_Y);
    s.ke = item_field(d, IF_Z);
    s.n = item_field(d, IF_N);
    s.m = item_field(d, IF_M);
    const int qo = item_field(d, IF_QO), ko = item_field(d, IF_KO);
    // per-(sample, head) buffer resources: rows past the sample's end read as zero
    const uint32_t kv_bytes = s.m > 0 ? ((uint32_t)(s.m - 1) * H + 1) * D * ES : 0;
    const uint32_t q_bytes = s.n > 0 ? ((uint32_t)(s.n - 1) * H + 1) * D * ES : 0;
    s.rk = make_rsrc((const uint8_t*)p.k + ((int64_t)ko * H + s.h) * D * ES, kv_bytes);
    s.rv = make_rsrc((const uint8_t*)p.v + ((int64_t)ko * H + s.h) * D * ES, kv_bytes);
    s.rq = make_rsrc((const uint8_t*)p.q + ((int64_t)qo * H + s.h) * D * ES, q_bytes);
    s.rks = s.rk;
    s.rvs = s.rv;
    s.rqs = s.rq;
    if constexpr (FP8) {
      const uint32_t kvs = s.m > 0 ? ((uint32_t)(s.m - 1) * H + 1) * (D / 32) : 0;
      const uint32_t qs = s.n > 0 ? ((uint32_t)(s.n - 1) * H + 1) * (D / 32) : 0;
      s.rks = make_rsrc(p.k_sc + ((int64_t)ko * H + s.h) * (D / 32), kvs);
      s.rvs = make_rsrc(p.v_sc + ((int64_t)ko * H + s.h) * (D / 32), kvs);
      s.rqs = make_rsrc(p.q_sc + ((int64_t)qo * H + s.h) * (D / 32), qs);
    }
    s.rb = s.rk;
    if constexpr (BIAS == B_DENSE)
      s.rb = make_rsrc((const __bf16*)p.bias + (int64_t)H * item_boff(d) +
                           (int64_t)s.h * s.n * s.m,
                       (uint32_t)s.n * (uint32_t)s.m * 2u);
    return s;
  };

  // ---- query fragment (B operand: column = query row, k = head dim), loaded into the *_in
  //      registers and copied to the working set once complete
  constexpr int QK = FP8 ? D / 64 : D / 16;
  i32x8 qf8_in[FP8 ? QK : 1];
  int qsc_in[FP8 ? QK : 1];
  bf16x8 qf_in[FP8 ? 1 : QK];
  auto load_q = [&](const Src& s) {
    const uint32_t qrow = (uint32_t)(s.q0 + wave * 32 + l32);
    const uint32_t qoff = qrow * row_bytes;
    if constexpr (FP8) {
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) {
        const u32x4 lo = ld16(s.rq, qoff + 64 * ks + 16 * g);
        const u32x4 hi = ld16(s.rq, qoff + 64 * ks + 32 + 16 * g);
        i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        qf8_in[ks] = v;
        qsc_in[ks] = (int)ld1(s.rqs, qrow * sc_row_bytes + 2 * ks + g);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) qf_in[ks] = as_bf16x8(ld16(s.rq, qoff + 32 * ks + 16 * g));
    }
  };

  // ---- staging: global -> registers for key step kt of an item
  // [BM][BN] block of the dense bias as chunks of 8 keys, consecutive lanes along a row
  // chunk i of this thread: byte offset and valid element count in the item's bias matrix
  auto dense_at = [&](const Src& s, int i, int j0, uint32_t& off, int& valid) {
    const int id = tid + i * NT;
    const int qq = s.q0 + id / (BN / 8), k0 = j0 + 8 * (id % (BN / 8));
    valid = qq < s.n ? min(8, s.m - k0) : 0;
    off = ((uint32_t)qq * (uint32_t)s.m + (uint32_t)k0) * 2u;
  };
  auto load_step = [&](const Src& s, int kt) {
    const int j0 = kt * BN;
    if constexpr (BIAS == B_DENSE) {
#pragma unroll
      for (int i = 0; i < NDB; ++i) {
        uint32_t off;
        int valid;
        dense_at(s, i, j0, off, valid);
        dbr[i] = bias_chunk_load(s.rb, off, valid, (uint32_t)s.n * (uint32_t)s.m * 2u);
      }
    }
    if constexpr (BIAS == B_RELPOS) {
      // diagonal table: T[x] = bias(dist = q0 + delta - j0 + BM - 1 - x), issued first so
      // that waiting for it never waits for the tile loads behind it
      if (tid < BM + BN - 1) {
        const int dist = s.q0 + (s.m - s.n) - j0 + BM - 1 - tid;
        const float* tab = (const float*)p.bias + (int64_t)s.h * p.num_buckets;
        rp_val = tab[relpos_bucket(dist, p.num_buckets)];
      }
    }
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int id = tid + i * NT;
      const int r = id / KCH, c = id % KCH;
      kreg[i] = ld16(s.rk, (uint32_t)(j0 + r) * row_bytes + 16 * c);
    }
    if constexpr (FP8) {
      if (tid < BN) {
        // the key's D/32 scale bytes are contiguous and aligned: one load, block e in byte e
        // (assembling them from byte loads would wait for the loads here)
        const uint32_t base = (uint32_t)(j0 + tid) * sc_row_bytes;
        static_assert(D == 128 || D == 64, "scale word");
        kscreg = D == 128 ? ld4(s.rks, base) : ld2(s.rks, base);
      }
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int id = tid + i * NT;
      if (VBLK % NT != 0 && id >= VBLK) break;
      const int cb = id % (D / 8), rbk = id / (D / 8);   // lanes along a row
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint32_t row = (uint32_t)(j0 + 4 * rbk + rr);
        if constexpr (FP8) {
          v8[i][rr] = ld8(s.rv, row * row_bytes + 8 * cb);
          vsc[i][rr] = ld1(s.rvs, row * sc_row_bytes + (8 * cb) / 32);
        } else {
          v16[i][rr] = ld16(s.rv, row * row_bytes + 16 * cb);
        }
      }
    }
  };

  ItemPipe pipe{p.xtk, p.items, (int)n_items, H};
  if (wave == 0) pipe.start(s_desc[0], lane);
  __syncthreads();
  bool pref = false;       // this item's query fragment and first tiles are already loading
  for (int buf = 0;; buf ^= 1) {
    const int* dsc = s_desc[buf];
    const int w = item_field(dsc, IF_W);
    if (w >= n_items) break;
    const Src cur = make_src(dsc);
    const int h = cur.h;
    const int kb = cur.kb, ke = cur.ke;
    const int slot = item_field(dsc, IF_SLOT);
    const int qo = item_field(dsc, IF_QO), n = cur.n, m = cur.m;
    const int delta = m - n;
    // the next item: a short item takes its ticket now and reads its record right after this
    // item's first loads, so that both round trips overlap those loads; a longer one claims it
    // CLAIM_AHEAD steps before its end
    const int nsteps = ke - kb;
    const bool short_item = nsteps <= CLAIM_AHEAD;
    if (short_item && wave == 0) pipe.claim(lane);
    const int q0 = cur.q0;
    const int qw0 = q0 + wave * 32;
    const int qil = wave * 32 + l32;        // tile-local query row of this lane
    const int qi = q0 + qil;                // sample-local query row
    // keys [wave_kbeg, wave_kend) hold every pair this wave's rows can see
    const int W = WIN ? p.window : 0;
    int wave_kend = m, wave_kbeg = 0;
    if (p.causal) wave_kend = max(0, min(m, min(n, qw0 + 32) + delta));
    else if (WIN) wave_kend = max(0, min(m, min(n, qw0 + 32) - 1 + delta + W));
    if (WIN) wave_kbeg = max(0, qw0 + delta - W + 1);
    const bool wave_rows = qw0 < n;

    if (!pref) {
      load_q(cur);
      if (nsteps > 0) load_step(cur, kb);
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    float m_run = NEG_INF, l_run = 0.f;

    // ---- staging: registers -> LDS stage `st`
    auto store_step = [&](int st, int kt) {
      unsigned char* base = lds + st * L::STAGE;
#pragma unroll
      for (int i = 0; i < K_LOADS; ++i) {
        const int id = tid + i * NT;
        const int r = id / KCH, c = id % KCH;
        *(u32x4*)(base + r * L::KRB + 16 * c) = kreg[i];
      }
      if constexpr (FP8) {
        if (tid < BN) *(uint32_t*)(base + L::K_BYTES + 4 * tid) = kscreg;
      }
      // V rows [BN][VS]; the PV operand V^T is read from them with transposing reads
      __bf16* vr = reinterpret_cast<__bf16*>(base + L::V_OFF);
#pragma unroll
      for (int i = 0; i < V_LOADS; ++i) {
        const int id = tid + i * NT;
        if (VBLK % NT != 0 && id >= VBLK) break;
        const int cb = id % (D / 8), rbk = id / (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          __bf16* dst = vr + (4 * rbk + rr) * VS + 8 * cb;
          if constexpr (FP8) {
            // dequantise 8 dims (E4M3 x 2^(s-127)) of one key to bf16
            const float sc = e8m0_to_f(vsc[i][rr]);
            u32x4 w;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              const uint32_t src = v8[i][rr][e2 >> 1];
              typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
              const bf2 cv = (e2 & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, sc, true)
                                      : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, sc, false);
              w[e2] = __builtin_bit_cast(uint32_t, cv);
            }
            *(u32x4*)dst = w;
          } else {
            *(u32x4*)dst = v16[i][rr];
          }
        }
      }
      if constexpr (BIAS == B_RELPOS) {
        float* rp = reinterpret_cast<float*>(base + L::B_OFF);
        if (tid < BM + BN - 1) {
          const float v = rp_val * inv_scale;
#pragma unroll
          for (int k = 0; k < 4; ++k) rp[k * L::RP + tid + k] = v;
        }
      } else if constexpr (BIAS == B_DENSE) {
        __bf16* bt = reinterpret_cast<__bf16*>(base + L::B_OFF);
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
          const int id = tid + i * NT;
          uint32_t off;
          int valid;
          dense_at(cur, i, kt * BN, off, valid);
          *(u32x4*)(bt + (id / (BN / 8)) * L::BS + 8 * (id % (BN / 8))) =
              bias_chunk_finish(dbr[i], off, valid, (uint32_t)n * (uint32_t)m * 2u);
        }
      }
    };

    if (short_item && wave == 0) pipe.resolve(lane);
    if (nsteps > 0) store_step(0, kb);
    if (short_item && wave == 0) pipe.publish(s_desc[buf ^ 1], lane);
    // the query fragment (loaded with the first tiles) is complete before the key loop
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // the working copy (with prefetch, the *_in registers take the next item's fragment
    // during the last key step)
    constexpr int QW8 = XPF && FP8 ? QK : 1, QW = XPF && !FP8 ? QK : 1;
    i32x8 qf8_w[QW8];
    int qsc_w[QW8];
    bf16x8 qf_w[QW];
    if constexpr (XPF) {
#pragma unroll
      for (int ks = 0; ks < QW8; ++ks) {
        qf8_w[ks] = qf8_in[ks];
        qsc_w[ks] = qsc_in[ks];
      }
#pragma unroll
      for (int ks = 0; ks < QW; ++ks) qf_w[ks] = qf_in[ks];
    }
    auto& qf8 = [&]() -> auto& { if constexpr (XPF) return qf8_w; else return qf8_in; }();
    auto& qsc = [&]() -> auto& { if constexpr (XPF) return qsc_w; else return qsc_in; }();
    auto& qf = [&]() -> auto& { if constexpr (XPF) return qf_w; else return qf_in; }();
    __syncthreads();
    // one key step on LDS stage it&1 (the loop is peeled so that its loads and stores are
    // unconditional: no load can be pending across the back edge)
    auto compute_step = [&](int it) {
      const int kt = kb + it;
      const int j0 = kt * BN;
      const unsigned char* sb = lds + (it & 1) * L::STAGE;
      if (wave_rows && j0 < wave_kend && (!WIN || j0 + BN > wave_kbeg)) {
        // ---- accumulator init = bias / scale (element (blk, i): key blk*32 + 8(i/4) + 4g + i%4)
        f32x16 sacc[2];
        if constexpr (BIAS == B_RELPOS) {
          const float* rp = reinterpret_cast<const float*>(sb + L::B_OFF);
          const int k = (1 + qil) & 3;                  // copy whose 4-runs are 16-byte aligned
          const float* src = rp + k * L::RP + k + BM - 1 - qil + 4 * g;
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              const f32x4 bv = *(const f32x4*)(src + blk * 32 + 8 * qd);
#pragma unroll
              for (int e = 0; e < 4; ++e) sacc[blk][4 * qd + e] = bv[e];
            }
        } else if constexpr (BIAS == B_DENSE) {
          const __bf16* bt = reinterpret_cast<const __bf16*>(sb + L::B_OFF) + qil * L::BS + 4 * g;
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              const u32x2 bv = *(const u32x2*)(bt + blk * 32 + 8 * qd);
              sacc[blk][4 * qd + 0] = __uint_as_float(bv[0] << 16) * inv_scale;
              sacc[blk][4 * qd + 1] = __uint_as_float(bv[0] & 0xffff0000u) * inv_scale;
              sacc[blk][4 * qd + 2] = __uint_as_float(bv[1] << 16) * inv_scale;
              sacc[blk][4 * qd + 3] = __uint_as_float(bv[1] & 0xffff0000u) * inv_scale;
            }
        } else {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[blk][i] = 0.f;
        }

        // ---- S^T += K Q^T for the 64 keys of this step (two 32-key blocks)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int krow = blk * 32 + l32;
          if constexpr (FP8) {
#pragma unroll
            for (int ks = 0; ks < QK; ++ks) {
              const unsigned char* kr = sb + krow * L::KRB + 64 * ks + 16 * g;
              const u32x4 lo = *(const u32x4*)kr;
              const u32x4 hi = *(const u32x4*)(kr + 32);
              i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
              const uint32_t sw = *(const uint32_t*)(sb + L::K_BYTES + 4 * krow);
              const int sa = (int)((sw >> (8 * (2 * ks + g))) & 255u);
              sacc[blk] = mfma_fp8(a, qf8[ks], sacc[blk], sa, qsc[ks]);
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < QK; ++ks) {
              const bf16x8 a = as_bf16x8(*(const u32x4*)(sb + krow * L::KRB + 32 * ks + 16 * g));
              sacc[blk] = mfma_bf16(a, qf[ks], sacc[blk]);
            }
          }
        }

        // ---- mask (only tiles that cross the sample end, the causal diagonal or a window
        //      edge): element (blk, i) is visible iff its key offset blk*32 + 8(i/4) + i%4
        //      lies in [lo, lim)
        // (GDPA needs no mask at the sample's end: a key past it has K and V rows that read as
        // zero and dense-bias entries that load as zero, so its activation times V is exactly
        // zero; softmax needs it for the row sum)
        const bool need_mask = (MODE == MODE_SOFTMAX && j0 + BN > m) ||
                               (p.causal && j0 + BN - 1 > qw0 + delta) ||
                               (WIN && (j0 <= qw0 + 31 + delta - W ||
                                        (!p.causal && j0 + BN - 1 >= qw0 + delta + W)));
        if (need_mask) {
          if constexpr (WIN) {
            int kend = p.causal ? min(m, qi + delta + 1) : min(m, qi + delta + W);
            const int lim = kend - j0 - 4 * g, lo = qi + delta - W + 1 - j0 - 4 * g;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int o = blk * 32 + 8 * (i >> 2) + (i & 3);
                if (o >= lim || o < lo) sacc[blk][i] = NEG_INF;
              }
          } else {
            const int kend = p.causal ? min(m, qi + delta + 1) : m;
            const int lim = kend - j0 - 4 * g;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
              for (int i = 0; i < 16; ++i)
                if (blk * 32 + 8 * (i >> 2) + (i & 3) >= lim) sacc[blk][i] = NEG_INF;
          }
        }

        // ---- probabilities P^T (bf16 pairs, in MFMA B-operand order)
        uint32_t pk[2][8];
        if constexpr (MODE == MODE_SOFTMAX) {
          float mt = NEG_INF;
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 16; i += 2) mt = vmax(mt, vmax(sacc[blk][i], sacc[blk][i + 1]));
          mt = vmax(mt, __shfl_xor(mt, 32));
          const float mx = mt * c_log;
          if (__any(mx > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = m_new == NEG_INF ? 1.0f : fast_exp2(m_run - m_new);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
            l_run *= alpha;
            m_run = m_new;
          }
          const float mu = m_run == NEG_INF ? 0.f : m_run;
          float ls[4];
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
              const float p0 = fast_exp2(fmaf(sacc[blk][i], c_log, -mu));
              const float p1 = fast_exp2(fmaf(sacc[blk][i + 1], c_log, -mu));
              pk[blk][i >> 1] = pack2bf(p0, p1);
              const int q = (i >> 1) & 3;
              if (blk == 0 && i < 8) ls[q] = p0 + p1;
              else ls[q] += p0 + p1;
            }
          l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        } else {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
              // masked scores are -inf, where SiLU and GELU would give NaN: clamped to -1e30,
              // both are exactly zero (a NaN score still propagates)
              const float a0 = act_fast<MODE>(act_clamp(sacc[blk][i] * c_log));
              const float a1 = act_fast<MODE>(act_clamp(sacc[blk][i + 1] * c_log));
              pk[blk][i >> 1] = pack2bf(a0, a1);
            }
        }

        // ---- O^T += V^T P^T: chunk c covers keys 16c + 8(e/4) + 4g + e%4
        const __bf16* vr = reinterpret_cast<const __bf16*>(sb + L::V_OFF);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 pw = {pk[c >> 1][4 * (c & 1)], pk[c >> 1][4 * (c & 1) + 1],
                            pk[c >> 1][4 * (c & 1) + 2], pk[c >> 1][4 * (c & 1) + 3]};
          const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            // V^T rows = head dims, k = 8g + j <-> key 16c + 8(j/4) + 4g + j%4: two column
            // strips of 4 keys of the V rows
            const __bf16* pv = vr + tr_lane + 16 * c * VS + db * 32;
            const u32x2 lo = lds_read_tr16(pv), hi = lds_read_tr16(pv + 8 * VS);
            const bf16x8 a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            acc[db] = mfma_bf16(a, pb, acc[db]);
          }
        }
      }
    };
    // a longer item claims the next one CLAIM_AHEAD steps before its end and publishes its
    // descriptor before the barrier ahead of its last step, where the prefetch reads it
    const int claim_it = short_item ? -1 : nsteps - CLAIM_AHEAD;
    const int resolve_it = short_item ? -1 : nsteps - 3;
    const int publish_it = short_item ? -1 : nsteps - 2;
    for (int it = 0; it + 1 < nsteps; ++it) {
      if (it == claim_it && wave == 0) pipe.claim(lane);
      if (it == resolve_it && wave == 0) pipe.resolve(lane);
      load_step(cur, kb + it + 1);
      compute_step(it);
      if (it == publish_it && wave == 0) pipe.publish(s_desc[buf ^ 1], lane);
      store_step((it + 1) & 1, kb + it + 1);
      __syncthreads();
    }
    pref = false;
    if constexpr (XPF) {
      const int* nd = s_desc[buf ^ 1];
      if (item_field(nd, IF_W) < n_items) {
        const Src nx = make_src(nd);
        load_q(nx);
        if (nx.ke > nx.kb) load_step(nx, nx.kb);
        pref = true;
      }
    }
    if (nsteps > 0) compute_step(nsteps - 1);

    // ---- epilogue
    float l_tot = l_run;
    if constexpr (MODE == MODE_SOFTMAX) l_tot = l_run + __shfl_xor(l_run, 32);
    if (slot < 0) {
      float mul;
      if constexpr (MODE == MODE_SOFTMAX) mul = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      else mul = (p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
      const uint32_t o_bytes = n > 0 ? ((uint32_t)(n - 1) * H + 1) * D * 2 : 0;
      const rsrc_t ro = make_rsrc((__bf16*)p.o + ((int64_t)qo * H + h) * D, o_bytes);
      // through the stage that the last key step left free (rows of this wave only)
      __bf16* ost = reinterpret_cast<__bf16*>(lds + (nsteps & 1) * L::STAGE +
                                              wave * out_stage_bytes<D>());
      store_rows_via_lds<D>(acc, mul, ost, ro, (uint32_t)qw0 * H * D * 2, (uint32_t)H * D * 2,
                            lane);
      if (MODE == MODE_SOFTMAX && g == 0 && p.lse && qi < n)
        p.lse[(int64_t)h * p.total_q + qo + qi] =
            l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : NEG_INF;
    } else {
      const int64_t pbase = ((int64_t)slot * H + h) * BM + qil;
      float* prow = p.part_acc + pbase * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          f32x4 v = {acc[db][4 * jq], acc[db][4 * jq + 1], acc[db][4 * jq + 2], acc[db][4 * jq + 3]};
          *(f32x4*)(prow + db * 32 + 8 * jq + 4 * g) = v;
        }
      if (g == 0) {
        p.part_ml[2 * pbase] = m_run;
        p.part_ml[2 * pbase + 1] = l_tot;
      }
    }
    __syncthreads();
  }
}

// Merges the chunks of every split tile in chunk order (deterministic).  A work unit is RPU
// rows of one (split tile, head); each thread owns 4 dims of one row, finds the row's running
// max over the chunks and sums the chunks' accumulators with weights e^(m_c - M) / sum_c
// e^(m_c - M) l_c (softmax) or 1/kv_len (GDPA); all of a thread's loads are independent.
template <int D, int BM, int MODE>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
  constexpr int RPU = 1024 / D;            // rows per unit: 256 threads x 4 dims
  constexpr int UPT = BM / RPU;            // units per (tile, head)
  const int H = p.H;
  if (p.hdr_ro->status != JFA_OK) return;
  const int64_t n_units = (int64_t)p.hdr_ro->counts[1] * H * UPT;
  const int r_in = threadIdx.x / (D / 4), c4 = threadIdx.x % (D / 4);
  for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int64_t w = u / UPT;
    const int r = (int)(u % UPT) * RPU + r_in;
    const int4 rec = p.comb[w / H];
    const int h = (int)(w % H);
    const int b = rec.x, t = rec.y, slot0 = rec.z, nch = rec.w;
    const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
    const int m = p.kv_off[b + 1] - p.kv_off[b];
    const int q0 = t * BM;
    if (q0 + r >= n) continue;
    auto pb = [&](int c) { return ((int64_t)(slot0 + c) * H + h) * BM + r; };
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE == MODE_SOFTMAX) {
      float M = NEG_INF;
#pragma unroll 4
      for (int c = 0; c < nch; ++c) M = fmaxf(M, p.part_ml[2 * pb(c)]);
      float Lsum = 0.f;
#pragma unroll 4
      for (int c = 0; c < nch; ++c) {
        const float2 ml = *(const float2*)(p.part_ml + 2 * pb(c));
        const f32x4 a = *(const f32x4*)(p.part_acc + pb(c) * D + 4 * c4);
        const float wgt = M == NEG_INF ? 0.f : fast_exp2(ml.x - M);
        Lsum += wgt * ml.y;
        o += wgt * a;
      }
      o *= Lsum > 0.f ? 1.0f / Lsum : 0.f;
      if (c4 == 0 && p.lse)
        p.lse[(int64_t)h * p.total_q + qo + q0 + r] =
            (M != NEG_INF && Lsum > 0.f) ? (M + __log2f(Lsum)) * LN2 : NEG_INF;
    } else {
#pragma unroll 4
      for (int c = 0; c < nch; ++c) o += *(const f32x4*)(p.part_acc + pb(c) * D + 4 * c4);
      o *= (p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    }
    __bf16* orow = (__bf16*)p.o + ((int64_t)(qo + q0 + r) * H + h) * D;
    const u32x2 pk = {pack2bf(o[0], o[1]), pack2bf(o[2], o[3])};
    *(u32x2*)(orow + 4 * c4) = pk;
  }
}

template <int D, int NW, int MODE, int BIAS, bool FP8, bool WIN>
hipError_t run_fwd(const FwdParams& p, int64_t max_items, int64_t max_comb, int cu_count,
                   hipStream_t s) {
  using L = FwdLds<D, NW, BIAS, FP8>;
  const size_t lds = L::TOTAL;
  auto kern = fwd_kernel<D, NW, MODE, BIAS, FP8, WIN>;
  {
    hipError_t e = ensure_dyn_lds((const void*)kern, lds);
    if (e != hipSuccess) return e;
  }
  int grid = resident_grid((const void*)kern, NW * 64, lds, cu_count);
  if ((int64_t)grid > max_items) grid = (int)max(max_items, (int64_t)1);
  timing_begin(FP8 ? "jfa_fwd_mxfp8" : "jfa_fwd_bf16", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, s, p);
  timing_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_comb <= 0) return e;
  // combine units: (split tile, head, group of 1024/D rows); the count is on the device
  const int64_t units = max_comb * (32 * NW) / (1024 / D);
  const unsigned cgrid = (unsigned)std::min<int64_t>(std::max<int64_t>(units, 1), 2048);
  timing_begin("jfa_fwd_combine", s);
  hipLaunchKernelGGL((combine_kernel<D, 32 * NW, MODE>), dim3(cgrid), dim3(256), 0, s, p);
  timing_end(s);
  return hipGetLastError();
}

template <int D, int NW, int MODE, bool FP8, bool WIN>
hipError_t run_fwd_win(const FwdParams& p, int64_t mi, int64_t mc, int cu, hipStream_t s) {
  switch (p.bias_kind) {
    case JFA_BIAS_RELPOS: return run_fwd<D, NW, MODE, B_RELPOS, FP8, WIN>(p, mi, mc, cu, s);
    case JFA_BIAS_DENSE:
      // the tile configuration takes 64-row tiles for a dense bias at d = 128
      if constexpr (D == 128 && NW == 4) return hipErrorInvalidValue;
      else return run_fwd<D, NW, MODE, B_DENSE, FP8, WIN>(p, mi, mc, cu, s);
    default: return run_fwd<D, NW, MODE, B_NONE, FP8, WIN>(p, mi, mc, cu, s);
  }
}

template <int D, int NW, int MODE, bool FP8>
hipError_t run_fwd_bias(const FwdParams& p, int64_t mi, int64_t mc, int cu, hipStream_t s) {
  return p.window > 0 ? run_fwd_win<D, NW, MODE, FP8, true>(p, mi, mc, cu, s)
                      : run_fwd_win<D, NW, MODE, FP8, false>(p, mi, mc, cu, s);
}

template <int D, int NW, bool FP8>
hipError_t run_fwd_mode(const FwdParams& p, int mode, int64_t mi, int64_t mc, int cu,
                        hipStream_t s) {
  switch (mode) {
    case MODE_SOFTMAX: return run_fwd_bias<D, NW, MODE_SOFTMAX, FP8>(p, mi, mc, cu, s);
    case MODE_SILU: return run_fwd_bias<D, NW, MODE_SILU, FP8>(p, mi, mc, cu, s);
    default: return run_fwd_bias<D, NW, MODE_GELU, FP8>(p, mi, mc, cu, s);
  }
}

}  // namespace

hipError_t launch_forward_f32(const FwdParams& p, const TileCfg& tc, int head_dim, int mode,
                              int64_t max_items, int cu_count, hipStream_t s);

hipError_t launch_forward(const FwdParams& p, const TileCfg& tc, int head_dim, int mode, int dtype,
                          int64_t max_items, int64_t max_comb_items, int cu_count, hipStream_t s) {
  if (dtype == JFA_F32) return launch_forward_f32(p, tc, head_dim, mode, max_items, cu_count, s);
  const bool fp8 = dtype == JFA_MXFP8_E4M3;
  const int nw = tc.fwd_nw;
  const int64_t mc = tc.slots > 0 ? max_comb_items : 0;
#define JFA_FWD_CASE(D_, NW_)                                                          \
  if (head_dim == D_ && nw == NW_)                                                      \
    return fp8 ? run_fwd_mode<D_, NW_, true>(p, mode, max_items, mc, cu_count, s)       \
               : run_fwd_mode<D_, NW_, false>(p, mode, max_items, mc, cu_count, s);
  JFA_FWD_CASE(128, 4)
  JFA_FWD_CASE(128, 2)
  JFA_FWD_CASE(64, 4)
  JFA_FWD_CASE(64, 2)
#undef JFA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace jfa
