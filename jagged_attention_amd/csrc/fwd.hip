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
//    the keys in steps of 64.  K (row-major) and V (transposed) of a step are staged in LDS;
//    the next step's global loads are issued before the current step's MFMAs.
//  - Each wave computes S^T = K Q^T (32x32x16 bf16 MFMA, or the scaled 32x32x64 E4M3 MFMA with
//    the MX block scales applied in hardware).  In the transposed accumulator a lane holds one
//    query column, so the softmax row max/sum are in-lane reductions plus one exchange with
//    the lane 32 away, and the probabilities P^T are already laid out as the B operand of
//    O^T += V^T P^T: no LDS round trip for P.
//  - Softmax keeps (max, sum) online in the log2 domain and rescales the accumulator only when
//    the running max grows by more than 8 (2^8 headroom in fp32/bf16).  GDPA applies the
//    activation elementwise and scales by 1/kv_len at the end.
//  - Work items (tile record, head) come from the longest-first list; persistent workgroups
//    take them with an atomic ticket.  Records that are chunks of a split tile write fp32
//    partials (unnormalised accumulator, max, sum) that the combine kernel merges in chunk
//    order.
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

constexpr int BN = FWD_BN;

// Dynamic LDS layout of the forward kernel.
template <int D, int NW, bool FP8>
struct FwdLds {
  static constexpr int BM = 32 * NW;
  static constexpr int KS = FP8 ? (D + 16) : (D + 8);   // K row stride: bytes (fp8) or bf16
  static constexpr int VS = BN + 4;                      // V^T row stride (bf16)
  static constexpr int BS = BN + 4;                      // dense bias row stride (floats)
  static constexpr int K_BYTES = BN * KS * (FP8 ? 1 : 2);
  static constexpr int KSC_BYTES = FP8 ? BN * (D / 32) : 0;
  static constexpr int V_OFF = (K_BYTES + KSC_BYTES + 15) / 16 * 16;
  static constexpr int V_BYTES = D * VS * 2;
  static constexpr int BIAS_OFF = V_OFF + V_BYTES;
  static constexpr int bias_bytes(int kind) {
    return kind == JFA_BIAS_DENSE ? BM * BS * 4 : (kind == JFA_BIAS_RELPOS ? (BM + BN) * 4 : 0);
  }
  static constexpr int total(int kind) { return BIAS_OFF + bias_bytes(kind) + 16; }
};

template <int D, int NW, int MODE, bool FP8>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(FwdParams p) {
  using L = FwdLds<D, NW, FP8>;
  constexpr int BM = L::BM, NT = NW * 64, KS = L::KS, VS = L::VS, BS = L::BS;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char* k_lds = lds;
  uint8_t* ksc_lds = lds + L::K_BYTES;
  __bf16* vt_lds = reinterpret_cast<__bf16*>(lds + L::V_OFF);
  float* bias_lds = reinterpret_cast<float*>(lds + L::BIAS_OFF);
  __shared__ int s_ticket;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr_ro->counts[0] * H;
  if (p.hdr_ro->status != JFA_OK) return;
  const float c_log = MODE == MODE_SOFTMAX ? p.scale * LOG2E : p.scale;
  const float b_mul = MODE == MODE_SOFTMAX ? LOG2E : 1.0f;

  // per-thread staging registers for one key step
  constexpr int KROW_CH = FP8 ? D / 16 : D / 8;          // 16-byte chunks per K row
  constexpr int KCH = (BN * KROW_CH + NT - 1) / NT;
  constexpr int VBLK = (BN / 4) * (D / 8);               // 4 rows x 8 columns blocks of V
  constexpr int VPT = (VBLK + NT - 1) / NT;
  u32x4 kreg[KCH];
  uint32_t kscreg = 0;
  u32x2 v8reg[FP8 ? VPT : 1][4];
  u32x4 v16reg[FP8 ? 1 : VPT][4];
  uint32_t vscreg[VPT][4];

  for (;;) {
    const int64_t w = next_ticket(&p.hdr->tickets[TK_FWD], &s_ticket);
    if (w >= n_items) break;
    const int ri = (int)(w / H);
    const int h = (int)(w % H);
    const int4 rec = p.recs[ri];
    const int slot = p.rec_slot[ri];
    const int b = rec.x, t = rec.y, kb = rec.z, ke = rec.w;
    const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
    const int ko = p.kv_off[b], m = p.kv_off[b + 1] - ko;
    const int delta = m - n;
    const int q0 = t * BM;
    const int qw0 = q0 + wave * 32;
    const int qil = wave * 32 + l32;        // tile-local query row of this lane
    const int qi = q0 + qil;                // sample-local query row
    const bool wave_rows = qw0 < n;
    int wave_kend = m;
    if (p.causal) wave_kend = max(0, min(m, min(n, qw0 + 32) + delta));

    // ---- query fragment: B operand (column = query row, k = head dim)
    constexpr int QK = FP8 ? D / 64 : D / 16;
    i32x8 qf8[FP8 ? QK : 1];
    int qsc[FP8 ? QK : 1];
    bf16x8 qf[FP8 ? 1 : QK];
    if constexpr (FP8) {
      const uint8_t* qrow = (const uint8_t*)p.q + ((int64_t)(qo + qi) * H + h) * D;
      const uint8_t* srow = p.q_sc + ((int64_t)(qo + qi) * H + h) * (D / 32);
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) {
        u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
        int sc = 127;
        if (qi < n) {
          lo = *(const u32x4*)(qrow + 64 * ks + 16 * g);
          hi = *(const u32x4*)(qrow + 64 * ks + 32 + 16 * g);
          sc = srow[2 * ks + g];
        }
        i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        qf8[ks] = v;
        qsc[ks] = sc;
      }
    } else {
      const __bf16* qrow = (const __bf16*)p.q + ((int64_t)(qo + qi) * H + h) * D;
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) {
        u32x4 v = {0, 0, 0, 0};
        if (qi < n) v = *(const u32x4*)(qrow + 16 * ks + 8 * g);
        qf[ks] = as_bf16x8(v);
      }
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    float m_run = NEG_INF, l_run = 0.f;

    const int64_t bias_base = p.bias_kind == JFA_BIAS_DENSE
                                  ? (int64_t)H * p.bias_off[b] + (int64_t)h * n * m
                                  : 0;

    // ---- staging: global -> registers for key step kt
    auto load_step = [&](int kt) {
      const int j0 = kt * BN;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int id = tid + i * NT;
        const int r = id / KROW_CH, c = id % KROW_CH;
        u32x4 v = {0, 0, 0, 0};
        if (id < BN * KROW_CH && j0 + r < m) {
          if constexpr (FP8)
            v = *(const u32x4*)((const uint8_t*)p.k + ((int64_t)(ko + j0 + r) * H + h) * D + 16 * c);
          else
            v = *(const u32x4*)((const __bf16*)p.k + ((int64_t)(ko + j0 + r) * H + h) * D + 8 * c);
        }
        kreg[i] = v;
      }
      if constexpr (FP8) {
        // K scales: one row (D/32 bytes, at most 4) per thread
        kscreg = 0;
        if (tid < BN) {
          const int r = tid;
          if (j0 + r < m) {
            const uint8_t* sp = p.k_sc + ((int64_t)(ko + j0 + r) * H + h) * (D / 32);
            uint32_t wv = 0;
#pragma unroll
            for (int e = 0; e < D / 32; ++e) wv |= (uint32_t)sp[e] << (8 * e);
            kscreg = wv;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int id = tid + i * NT;
        const int rb = id % (BN / 4), cb = id / (BN / 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = j0 + 4 * rb + rr;
          const bool ok = id < VBLK && row < m;
          if constexpr (FP8) {
            u32x2 v = {0, 0};
            uint32_t sc = 127;
            if (ok) {
              v = *(const u32x2*)((const uint8_t*)p.v + ((int64_t)(ko + row) * H + h) * D + 8 * cb);
              sc = p.v_sc[((int64_t)(ko + row) * H + h) * (D / 32) + (8 * cb) / 32];
            }
            v8reg[i][rr] = v;
            vscreg[i][rr] = sc;
          } else {
            u32x4 v = {0, 0, 0, 0};
            if (ok) v = *(const u32x4*)((const __bf16*)p.v + ((int64_t)(ko + row) * H + h) * D + 8 * cb);
            v16reg[i][rr] = v;
          }
        }
      }
    };

    // ---- staging: registers -> LDS (and the bias tile straight from global)
    auto store_step = [&](int kt) {
      const int j0 = kt * BN;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int id = tid + i * NT;
        const int r = id / KROW_CH, c = id % KROW_CH;
        if (id < BN * KROW_CH) {
          if constexpr (FP8) *(u32x4*)(k_lds + r * KS + 16 * c) = kreg[i];
          else *(u32x4*)(k_lds + (r * KS + 8 * c) * 2) = kreg[i];
        }
      }
      if constexpr (FP8) {
        if (tid < BN) {
#pragma unroll
          for (int e = 0; e < D / 32; ++e) ksc_lds[tid * (D / 32) + e] = (kscreg >> (8 * e)) & 255u;
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int id = tid + i * NT;
        if (id >= VBLK) continue;
        const int rb = id % (BN / 4), cb = id / (BN / 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float f[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            if constexpr (FP8) {
              const uint32_t code = (v8reg[i][rr][e >> 2] >> (8 * (e & 3))) & 255u;
              f[rr] = e4m3_to_f(code) * e8m0_to_f(vscreg[i][rr]);
            } else {
              const uint32_t word = v16reg[i][rr][e >> 1];
              f[rr] = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
            }
          }
          u32x2 pk = {pack2bf(f[0], f[1]), pack2bf(f[2], f[3])};
          *(u32x2*)(vt_lds + (8 * cb + e) * VS + 4 * rb) = pk;
        }
      }
      if (p.bias_kind == JFA_BIAS_RELPOS) {
        // bias by diagonal: entry x holds the bias of (query - key) = x - (BN - 1) in the tile
        if (tid < BM + BN - 1) {
          const int dist = tid - (BN - 1) + q0 + delta - j0;
          const float* tab = (const float*)p.bias + (int64_t)h * p.num_buckets;
          bias_lds[tid] = tab[relpos_bucket(dist, p.num_buckets)] * b_mul;
        }
      } else if (p.bias_kind == JFA_BIAS_DENSE) {
        const __bf16* bp = (const __bf16*)p.bias + bias_base;
        for (int e = tid; e < BM * BN; e += NT) {
          const int r = e / BN, c = e % BN;
          float v = 0.f;
          if (q0 + r < n && j0 + c < m) v = (float)bp[(int64_t)(q0 + r) * m + j0 + c];
          bias_lds[r * BS + c] = v * b_mul;
        }
      }
    };

    if (kb < ke) load_step(kb);
    for (int kt = kb; kt < ke; ++kt) {
      __syncthreads();
      store_step(kt);
      __syncthreads();
      if (kt + 1 < ke) load_step(kt + 1);
      const int j0 = kt * BN;
      if (!wave_rows || j0 >= wave_kend) continue;

      // ---- S^T = K Q^T for the 64 keys of this step (two 32-key blocks)
      f32x16 sacc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[blk][i] = 0.f;
        const int krow = blk * 32 + l32;
        if constexpr (FP8) {
#pragma unroll
          for (int ks = 0; ks < QK; ++ks) {
            const u32x4 lo = *(const u32x4*)(k_lds + krow * KS + 64 * ks + 16 * g);
            const u32x4 hi = *(const u32x4*)(k_lds + krow * KS + 64 * ks + 32 + 16 * g);
            i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int sa = ksc_lds[krow * (D / 32) + 2 * ks + g];
            sacc[blk] = mfma_fp8(a, qf8[ks], sacc[blk], sa, qsc[ks]);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < QK; ++ks) {
            const bf16x8 a = as_bf16x8(*(const u32x4*)(k_lds + (krow * KS + 16 * ks + 8 * g) * 2));
            sacc[blk] = mfma_bf16(a, qf[ks], sacc[blk]);
          }
        }
      }

      // ---- scores: scale, bias, mask (element (blk, i) is key blk*32 + 8(i/4) + 4g + i%4)
      const bool need_mask = (j0 + BN > m) || (p.causal && j0 + BN - 1 > qw0 + delta);
      float x[2][16];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[blk][i] = sacc[blk][i] * c_log;
        if (p.bias_kind == JFA_BIAS_RELPOS) {
          const float* br = bias_lds + (qil + BN - 1 - 4 * g) - blk * 32;
#pragma unroll
          for (int i = 0; i < 16; ++i) x[blk][i] += br[-(8 * (i >> 2) + (i & 3))];
        } else if (p.bias_kind == JFA_BIAS_DENSE) {
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const f32x4 bv = *(const f32x4*)(bias_lds + qil * BS + blk * 32 + 8 * jq + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[blk][4 * jq + e] += bv[e];
          }
        }
      }
      bool valid[2][16];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = j0 + blk * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          valid[blk][i] = !need_mask || (j < m && (!p.causal || j <= qi + delta));
        }

      float pr[2][16];
      if constexpr (MODE == MODE_SOFTMAX) {
        float mt = NEG_INF;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (!valid[blk][i]) x[blk][i] = NEG_INF;
            mt = fmaxf(mt, x[blk][i]);
          }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m_run, mt);
        const bool need = mn > m_run + 8.0f;
        if (__any(need)) {
          const float m_new = need ? mn : m_run;
          const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
          l_run *= alpha;
          m_run = m_new;
        }
        const float mu = m_run == NEG_INF ? 0.f : m_run;
        float ls = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            pr[blk][i] = fast_exp2(x[blk][i] - mu);
            ls += pr[blk][i];
          }
        l_run += ls;
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) pr[blk][i] = valid[blk][i] ? act_f<MODE>(x[blk][i]) : 0.f;
      }

      // ---- O^T += V^T P^T: P^T chunk c covers keys 16c + 8(e/4) + 4g + e%4
      bf16x8 pb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          pk[e2] = pack2bf(pr[c >> 1][8 * (c & 1) + 2 * e2], pr[c >> 1][8 * (c & 1) + 2 * e2 + 1]);
        pb[c] = as_bf16x8(pk);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const __bf16* vrow = vt_lds + (db * 32 + l32) * VS + 4 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x2 lo = *(const u32x2*)(vrow + 16 * c);
          const u32x2 hi = *(const u32x2*)(vrow + 16 * c + 8);
          acc[db] = mfma_bf16(cat_bf16x8(lo, hi), pb[c], acc[db]);
        }
      }
    }

    // ---- epilogue
    float l_tot = l_run;
    if constexpr (MODE == MODE_SOFTMAX) l_tot = l_run + __shfl_xor(l_run, 32);
    if (slot < 0) {
      if (qi < n) {
        float mul;
        if constexpr (MODE == MODE_SOFTMAX) mul = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        else mul = (p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
        __bf16* orow = (__bf16*)p.o + ((int64_t)(qo + qi) * H + h) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            u32x2 pk = {pack2bf(acc[db][4 * jq] * mul, acc[db][4 * jq + 1] * mul),
                        pack2bf(acc[db][4 * jq + 2] * mul, acc[db][4 * jq + 3] * mul)};
            *(u32x2*)(orow + db * 32 + 8 * jq + 4 * g) = pk;
          }
        if (MODE == MODE_SOFTMAX && g == 0 && p.lse)
          p.lse[(int64_t)h * p.total_q + qo + qi] =
              l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : NEG_INF;
      }
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
  }
}

// Merges the chunks of every split tile in chunk order (deterministic).
template <int D, int BM, int MODE>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p) {
  const int H = p.H;
  if (p.hdr_ro->status != JFA_OK) return;
  const int64_t n_items = (int64_t)p.hdr_ro->counts[1] * H;
  const int64_t w = blockIdx.x;
  if (w >= n_items) return;
  const int4 rec = p.comb[w / H];
  const int h = (int)(w % H);
  const int b = rec.x, t = rec.y, slot0 = rec.z, nch = rec.w;
  const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
  const int m = p.kv_off[b + 1] - p.kv_off[b];
  const int q0 = t * BM;
  for (int e = threadIdx.x; e < BM * (D / 4); e += 256) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    if (q0 + r >= n) continue;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse = NEG_INF;
    if constexpr (MODE == MODE_SOFTMAX) {
      float M = NEG_INF;
      for (int c = 0; c < nch; ++c)
        M = fmaxf(M, p.part_ml[2 * (((int64_t)(slot0 + c) * H + h) * BM + r)]);
      if (M != NEG_INF) {
        float Lsum = 0.f;
        for (int c = 0; c < nch; ++c) {
          const int64_t pb = ((int64_t)(slot0 + c) * H + h) * BM + r;
          const float wgt = fast_exp2(p.part_ml[2 * pb] - M);
          Lsum += wgt * p.part_ml[2 * pb + 1];
          const f32x4 a = *(const f32x4*)(p.part_acc + pb * D + 4 * c4);
          o += wgt * a;
        }
        o *= 1.0f / Lsum;
        lse = (M + __log2f(Lsum)) * LN2;
      }
    } else {
      for (int c = 0; c < nch; ++c) {
        const int64_t pb = ((int64_t)(slot0 + c) * H + h) * BM + r;
        o += *(const f32x4*)(p.part_acc + pb * D + 4 * c4);
      }
      o *= (p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    }
    __bf16* orow = (__bf16*)p.o + ((int64_t)(qo + q0 + r) * H + h) * D;
    u32x2 pk = {pack2bf(o[0], o[1]), pack2bf(o[2], o[3])};
    *(u32x2*)(orow + 4 * c4) = pk;
    if (MODE == MODE_SOFTMAX && c4 == 0 && p.lse) p.lse[(int64_t)h * p.total_q + qo + q0 + r] = lse;
  }
}

template <int D, int NW, int MODE, bool FP8>
hipError_t run_fwd(const FwdParams& p, int bias_kind, int64_t max_items, int64_t max_comb,
                   int cu_count, hipStream_t s) {
  using L = FwdLds<D, NW, FP8>;
  const size_t lds = L::total(bias_kind);
  auto kern = fwd_kernel<D, NW, MODE, FP8>;
  static int attr_done = 0;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       L::total(JFA_BIAS_DENSE));
    if (e != hipSuccess) return e;
    attr_done = 1;
  }
  int grid = resident_grid((const void*)kern, NW * 64, lds, cu_count);
  if ((int64_t)grid > max_items) grid = (int)max(max_items, (int64_t)1);
  timing_begin(FP8 ? "jfa_fwd_mxfp8" : "jfa_fwd_bf16", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, s, p);
  timing_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_comb <= 0) return e;
  timing_begin("jfa_fwd_combine", s);
  hipLaunchKernelGGL((combine_kernel<D, 32 * NW, MODE>), dim3((unsigned)max_comb), dim3(256), 0,
                     s, p);
  timing_end(s);
  return hipGetLastError();
}

template <int D, int NW, bool FP8>
hipError_t run_fwd_mode(const FwdParams& p, int mode, int bias_kind, int64_t mi, int64_t mc,
                        int cu, hipStream_t s) {
  switch (mode) {
    case MODE_SOFTMAX: return run_fwd<D, NW, MODE_SOFTMAX, FP8>(p, bias_kind, mi, mc, cu, s);
    case MODE_SILU: return run_fwd<D, NW, MODE_SILU, FP8>(p, bias_kind, mi, mc, cu, s);
    default: return run_fwd<D, NW, MODE_GELU, FP8>(p, bias_kind, mi, mc, cu, s);
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
#define JFA_FWD_CASE(D_, NW_)                                                              \
  if (head_dim == D_ && nw == NW_)                                                          \
    return fp8 ? run_fwd_mode<D_, NW_, true>(p, mode, p.bias_kind, max_items, mc, cu_count, s) \
               : run_fwd_mode<D_, NW_, false>(p, mode, p.bias_kind, max_items, mc, cu_count, s);
  JFA_FWD_CASE(128, 4)
  JFA_FWD_CASE(128, 2)
  JFA_FWD_CASE(64, 4)
  JFA_FWD_CASE(64, 2)
#undef JFA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace jfa
