// Jagged attention backward on MFMA (bf16): softmax preprocess, query-stationary dQ pass and
// key-stationary dK/dV pass.
//
// Source: "Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a Different Stack",
// section "Bottleneck move 1": GDPA (SiLU/GELU in place of softmax) forward and backward;
// removing padding exposes backward accumulation.  The gradients are those of <O, dO>:
//   softmax: dP = dO V^T, dS = P (dP - D), D_i = dO_i . O_i
//   GDPA:    dP = w dO V^T, dS = act'(S) dP, dV = w act(S)^T dO    (w = 1/kv_len or 1)
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO (softmax).
//
// Determinism without float atomics: the query-stationary kernel owns dQ rows and sums over
// key steps in order in registers; the key-stationary kernel owns dK/dV rows and sums over
// query steps in order.  Each recomputes S (and P) from the forward's log-sum-exp.
//
// Layout trick shared with the forward: the query-stationary kernel works on S^T (lane = one
// query), the key-stationary kernel on S (lane = one key); in both the lane's accumulator row
// is exactly the B operand of the next MFMA, so P and dS never go through LDS.
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

// ------------------------------------------------------------------ preprocess
// delta[h][i] = sum_c dO[i,h,c] * O[i,h,c]; LPR lanes read one (row, head) 16 bytes at a time.
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o,
                                                    const T* __restrict__ dout, float* delta,
                                                    int64_t total_q, int H) {
  constexpr int EPL = 16 / sizeof(T);            // elements per 16-byte load
  constexpr int LPR = D / EPL;                   // lanes per (row, head)
  constexpr int RPB = 256 / LPR;                 // (row, head) pairs per block
  const int sub = threadIdx.x % LPR;
  const int64_t rh = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const bool ok = rh < total_q * H;
  float s = 0.f;
  if (ok) {
    const u32x4 a = *(const u32x4*)(o + rh * D + sub * EPL);
    const u32x4 c = *(const u32x4*)(dout + rh * D + sub * EPL);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s += __uint_as_float(a[e] << 16) * __uint_as_float(c[e] << 16);
        s += __uint_as_float(a[e] & 0xffff0000u) * __uint_as_float(c[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) s += __uint_as_float(a[e]) * __uint_as_float(c[e]);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (ok && sub == 0) {
    const int64_t i = rh / H;
    const int h = (int)(rh % H);
    delta[(int64_t)h * total_q + i] = s;
  }
}

// Copies a [rows x D] bf16 block of one head into LDS, row-major (stride RS) and transposed
// (stride TS): each thread moves 4 rows x 8 columns.
template <int D, int ROWS, int NT, int RS, int TS>
__device__ __forceinline__ void stage_rows_and_transpose(const __bf16* base, int64_t row_stride,
                                                         int r0, int rmax, __bf16* row_lds,
                                                         __bf16* t_lds) {
  constexpr int BLK = (ROWS / 4) * (D / 8);
  for (int id = threadIdx.x; id < BLK; id += NT) {
    const int rb = id % (ROWS / 4), cb = id / (ROWS / 4);
    u32x4 v[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * rb + rr;
      v[rr] = u32x4{0, 0, 0, 0};
      if (r0 + r < rmax) v[rr] = *(const u32x4*)(base + (int64_t)(r0 + r) * row_stride + 8 * cb);
      if (row_lds) *(u32x4*)(row_lds + r * RS + 8 * cb) = v[rr];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint32_t word = v[rr][e >> 1];
        h[rr] = (e & 1) ? (word >> 16) : (word & 0xffffu);
      }
      u32x2 pk = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *(u32x2*)(t_lds + (8 * cb + e) * TS + 4 * rb) = pk;
    }
  }
}

// Row-major copy of a [rows x D] bf16 block into LDS with row stride RS.
template <int D, int ROWS, int NT, int RS>
__device__ __forceinline__ void stage_rows(const __bf16* base, int64_t row_stride, int r0, int rmax,
                                           __bf16* row_lds) {
  constexpr int CH = ROWS * (D / 8);
  for (int id = threadIdx.x; id < CH; id += NT) {
    const int r = id / (D / 8), c = id % (D / 8);
    u32x4 v = {0, 0, 0, 0};
    if (r0 + r < rmax) v = *(const u32x4*)(base + (int64_t)(r0 + r) * row_stride + 8 * c);
    *(u32x4*)(row_lds + r * RS + 8 * c) = v;
  }
}

// B-operand fragment of one row (column of the transposed operand): k = 16 ks + 8 g + 0..7.
template <int D>
__device__ __forceinline__ void load_frag(const __bf16* row, bool ok, int g, bf16x8* f) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 v = {0, 0, 0, 0};
    if (ok) v = *(const u32x4*)(row + 16 * ks + 8 * g);
    f[ks] = as_bf16x8(v);
  }
}

__device__ __forceinline__ bf16x8 pack_chunk(const float (&v)[2][16], int c) {
  u32x4 pk;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2)
    pk[e2] = pack2bf(v[c >> 1][8 * (c & 1) + 2 * e2], v[c >> 1][8 * (c & 1) + 2 * e2 + 1]);
  return as_bf16x8(pk);
}

// --------------------------------------------------------- query-stationary dQ
template <int D, int NW>
struct BqLds {
  static constexpr int BM = 32 * NW, BN = BQ_BN;
  static constexpr int KS = D + 8, TS = BN + 4, BS = BN + 4;
  static constexpr int K_OFF = 0;
  static constexpr int KT_OFF = K_OFF + BN * KS * 2;
  static constexpr int V_OFF = KT_OFF + D * TS * 2;
  static constexpr int BIAS_OFF = V_OFF + BN * KS * 2;
  static constexpr int bias_bytes(int kind) {
    return kind == JFA_BIAS_DENSE ? BM * BS * 4 : (kind == JFA_BIAS_RELPOS ? (BM + BN) * 4 : 0);
  }
  static constexpr int total(int kind) { return BIAS_OFF + bias_bytes(kind) + 16; }
};

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64, 2) void bwd_q_kernel(BwdParams p) {
  using L = BqLds<D, NW>;
  constexpr int BM = L::BM, BN = L::BN, NT = NW * 64, KS = L::KS, TS = L::TS, BS = L::BS;
  extern __shared__ __align__(16) unsigned char lds[];
  __bf16* k_lds = reinterpret_cast<__bf16*>(lds + L::K_OFF);
  __bf16* kt_lds = reinterpret_cast<__bf16*>(lds + L::KT_OFF);
  __bf16* v_lds = reinterpret_cast<__bf16*>(lds + L::V_OFF);
  float* bias_lds = reinterpret_cast<float*>(lds + L::BIAS_OFF);
  __shared__ int s_ticket;

  if (p.hdr->status != JFA_OK) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr->counts[2] * H;
  const float c_log = MODE == MODE_SOFTMAX ? p.scale * LOG2E : p.scale;
  const float b_mul = MODE == MODE_SOFTMAX ? LOG2E : 1.0f;

  for (;;) {
    const int64_t w = next_ticket(&p.hdr->tickets[TK_BQ], &s_ticket);
    if (w >= n_items) break;
    const int4 rec = p.bq[w / H];
    const int h = (int)(w % H);
    const int b = rec.x, t = rec.y, steps = rec.w;
    const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
    const int ko = p.kv_off[b], m = p.kv_off[b + 1] - ko;
    const int delta = m - n;
    const float wn = (MODE != MODE_SOFTMAX && p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    const int q0 = t * BM, qw0 = q0 + wave * 32;
    const int qil = wave * 32 + l32, qi = q0 + qil;
    const bool wave_rows = qw0 < n;
    int wave_kend = m;
    if (p.causal) wave_kend = max(0, min(m, min(n, qw0 + 32) + delta));
    const int64_t rowq = (int64_t)(qo + qi) * H + h;

    bf16x8 qf[D / 16], dof[D / 16];
    load_frag<D>((const __bf16*)p.q + rowq * D, qi < n, g, qf);
    load_frag<D>((const __bf16*)p.dout + rowq * D, qi < n, g, dof);
    float lse2 = 0.f, dlt = 0.f;
    if (MODE == MODE_SOFTMAX && qi < n) {
      lse2 = p.lse[(int64_t)h * p.total_q + qo + qi] * LOG2E;
      dlt = p.delta[(int64_t)h * p.total_q + qo + qi];
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    const int64_t bias_base =
        p.bias_kind == JFA_BIAS_DENSE ? (int64_t)H * p.bias_off[b] + (int64_t)h * n * m : 0;
    const __bf16* kbase = (const __bf16*)p.k + ((int64_t)ko * H + h) * D;
    const __bf16* vbase = (const __bf16*)p.v + ((int64_t)ko * H + h) * D;

    for (int kt = 0; kt < steps; ++kt) {
      const int j0 = kt * BN;
      __syncthreads();
      stage_rows_and_transpose<D, BN, NT, KS, TS>(kbase, (int64_t)H * D, j0, m, k_lds, kt_lds);
      stage_rows<D, BN, NT, KS>(vbase, (int64_t)H * D, j0, m, v_lds);
      if (p.bias_kind == JFA_BIAS_RELPOS) {
        if (tid < BM + BN - 1) {
          const int dist = tid - (BN - 1) + q0 + delta - j0;
          bias_lds[tid] = ((const float*)p.bias)[(int64_t)h * p.num_buckets +
                                                relpos_bucket(dist, p.num_buckets)] * b_mul;
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
      __syncthreads();
      if (!wave_rows || j0 >= wave_kend) continue;

      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[blk][i] = 0.f; pacc[blk][i] = 0.f; }
        const int krow = blk * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 ka = as_bf16x8(*(const u32x4*)(k_lds + krow * KS + 16 * ks + 8 * g));
          sacc[blk] = mfma_bf16(ka, qf[ks], sacc[blk]);
          const bf16x8 va = as_bf16x8(*(const u32x4*)(v_lds + krow * KS + 16 * ks + 8 * g));
          pacc[blk] = mfma_bf16(va, dof[ks], pacc[blk]);
        }
      }
      const bool need_mask = (j0 + BN > m) || (p.causal && j0 + BN - 1 > qw0 + delta);
      float ds[2][16];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = sacc[blk][i] * c_log;
        if (p.bias_kind == JFA_BIAS_RELPOS) {
          const float* br = bias_lds + (qil + BN - 1 - 4 * g) - blk * 32;
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] += br[-(8 * (i >> 2) + (i & 3))];
        } else if (p.bias_kind == JFA_BIAS_DENSE) {
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const f32x4 bv = *(const f32x4*)(bias_lds + qil * BS + blk * 32 + 8 * jq + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * jq + e] += bv[e];
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = j0 + blk * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          const bool valid = !need_mask || (j < m && (!p.causal || j <= qi + delta));
          float d;
          if constexpr (MODE == MODE_SOFTMAX) {
            const float pr = valid ? fast_exp2(x[i] - lse2) : 0.f;
            d = pr * (pacc[blk][i] - dlt);
          } else {
            d = valid ? act_grad_f<MODE>(x[i]) * pacc[blk][i] * wn : 0.f;
          }
          ds[blk][i] = d;
        }
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 db_op = pack_chunk(ds, c);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const __bf16* krow = kt_lds + (db * 32 + l32) * TS + 16 * c + 4 * g;
          const u32x2 lo = *(const u32x2*)krow;
          const u32x2 hi = *(const u32x2*)(krow + 8);
          acc[db] = mfma_bf16(cat_bf16x8(lo, hi), db_op, acc[db]);
        }
      }
    }
    if (qi < n) {
      __bf16* out = (__bf16*)p.dq + rowq * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          u32x2 pk = {pack2bf(acc[db][4 * jq] * p.scale, acc[db][4 * jq + 1] * p.scale),
                      pack2bf(acc[db][4 * jq + 2] * p.scale, acc[db][4 * jq + 3] * p.scale)};
          *(u32x2*)(out + db * 32 + 8 * jq + 4 * g) = pk;
        }
    }
  }
}

// ------------------------------------------------------- key-stationary dK, dV
template <int D, int NW>
struct BkLds {
  static constexpr int BNK = 32 * NW, BM = BK_BM;
  static constexpr int QS = D + 8, TS = BM + 4, BS = BM + 4;
  static constexpr int Q_OFF = 0;
  static constexpr int DO_OFF = Q_OFF + BM * QS * 2;
  static constexpr int QT_OFF = DO_OFF + BM * QS * 2;
  static constexpr int DOT_OFF = QT_OFF + D * TS * 2;
  static constexpr int LSE_OFF = DOT_OFF + D * TS * 2;
  static constexpr int DLT_OFF = LSE_OFF + BM * 4;
  static constexpr int BIAS_OFF = DLT_OFF + BM * 4;
  static constexpr int bias_bytes(int kind) {
    return kind == JFA_BIAS_DENSE ? BNK * BS * 4 : (kind == JFA_BIAS_RELPOS ? (BM + BNK) * 4 : 0);
  }
  static constexpr int total(int kind) { return BIAS_OFF + bias_bytes(kind) + 16; }
};

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64, 1) void bwd_kv_kernel(BwdParams p) {
  using L = BkLds<D, NW>;
  constexpr int BNK = L::BNK, BM = L::BM, NT = NW * 64, QS = L::QS, TS = L::TS, BS = L::BS;
  extern __shared__ __align__(16) unsigned char lds[];
  __bf16* q_lds = reinterpret_cast<__bf16*>(lds + L::Q_OFF);
  __bf16* do_lds = reinterpret_cast<__bf16*>(lds + L::DO_OFF);
  __bf16* qt_lds = reinterpret_cast<__bf16*>(lds + L::QT_OFF);
  __bf16* dot_lds = reinterpret_cast<__bf16*>(lds + L::DOT_OFF);
  float* lse_lds = reinterpret_cast<float*>(lds + L::LSE_OFF);
  float* dlt_lds = reinterpret_cast<float*>(lds + L::DLT_OFF);
  float* bias_lds = reinterpret_cast<float*>(lds + L::BIAS_OFF);
  __shared__ int s_ticket;

  if (p.hdr->status != JFA_OK) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr->counts[3] * H;
  const float c_log = MODE == MODE_SOFTMAX ? p.scale * LOG2E : p.scale;
  const float b_mul = MODE == MODE_SOFTMAX ? LOG2E : 1.0f;

  for (;;) {
    const int64_t w = next_ticket(&p.hdr->tickets[TK_BK], &s_ticket);
    if (w >= n_items) break;
    const int4 rec = p.bk[w / H];
    const int h = (int)(w % H);
    const int b = rec.x, u = rec.y, qs_first = rec.z, qs_end = rec.w;
    const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
    const int ko = p.kv_off[b], m = p.kv_off[b + 1] - ko;
    const int delta = m - n;
    const float wn = (MODE != MODE_SOFTMAX && p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    const int j0 = u * BNK, jw0 = j0 + wave * 32;
    const int kvl = wave * 32 + l32, j = j0 + kvl;
    const int64_t rowk = (int64_t)(ko + j) * H + h;

    bf16x8 kf[D / 16], vf[D / 16];
    load_frag<D>((const __bf16*)p.k + rowk * D, j < m, g, kf);
    load_frag<D>((const __bf16*)p.v + rowk * D, j < m, g, vf);
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) { dk[db][i] = 0.f; dv[db][i] = 0.f; }
    const int64_t bias_base =
        p.bias_kind == JFA_BIAS_DENSE ? (int64_t)H * p.bias_off[b] + (int64_t)h * n * m : 0;
    const __bf16* qbase = (const __bf16*)p.q + ((int64_t)qo * H + h) * D;
    const __bf16* dobase = (const __bf16*)p.dout + ((int64_t)qo * H + h) * D;

    for (int qs = qs_first; qs < qs_end; ++qs) {
      const int q0 = qs * BM;
      __syncthreads();
      stage_rows_and_transpose<D, BM, NT, QS, TS>(qbase, (int64_t)H * D, q0, n, q_lds, qt_lds);
      stage_rows_and_transpose<D, BM, NT, QS, TS>(dobase, (int64_t)H * D, q0, n, do_lds, dot_lds);
      if (tid < BM) {
        float l2 = 0.f, dl = 0.f;
        if (MODE == MODE_SOFTMAX && q0 + tid < n) {
          l2 = p.lse[(int64_t)h * p.total_q + qo + q0 + tid] * LOG2E;
          dl = p.delta[(int64_t)h * p.total_q + qo + q0 + tid];
        }
        lse_lds[tid] = l2;
        dlt_lds[tid] = dl;
      }
      if (p.bias_kind == JFA_BIAS_RELPOS) {
        // entry x: bias of (query - key) = x - (BNK - 1) within the tile
        if (tid < BM + BNK - 1) {
          const int dist = tid - (BNK - 1) + q0 + delta - j0;
          bias_lds[tid] = ((const float*)p.bias)[(int64_t)h * p.num_buckets +
                                                relpos_bucket(dist, p.num_buckets)] * b_mul;
        }
      } else if (p.bias_kind == JFA_BIAS_DENSE) {
        // stored transposed: [key][query]
        const __bf16* bp = (const __bf16*)p.bias + bias_base;
        for (int e = tid; e < BM * BNK; e += NT) {
          const int r = e / BNK, c = e % BNK;
          float v = 0.f;
          if (q0 + r < n && j0 + c < m) v = (float)bp[(int64_t)(q0 + r) * m + j0 + c];
          bias_lds[c * BS + r] = v * b_mul;
        }
      }
      __syncthreads();
      if (jw0 >= m || (p.causal && q0 + BM - 1 + delta < jw0)) continue;

      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[blk][i] = 0.f; pacc[blk][i] = 0.f; }
        const int qrow = blk * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 qa = as_bf16x8(*(const u32x4*)(q_lds + qrow * QS + 16 * ks + 8 * g));
          sacc[blk] = mfma_bf16(qa, kf[ks], sacc[blk]);
          const bf16x8 da = as_bf16x8(*(const u32x4*)(do_lds + qrow * QS + 16 * ks + 8 * g));
          pacc[blk] = mfma_bf16(da, vf[ks], pacc[blk]);
        }
      }
      // element (blk, i): query q0 + blk*32 + 8(i/4) + 4g + i%4, key j
      const bool need_mask = (q0 + BM > n) || (jw0 + 32 > m) ||
                             (p.causal && q0 + delta < jw0 + 31);
      float pv[2][16], ds[2][16];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = sacc[blk][i] * c_log;
        if (p.bias_kind == JFA_BIAS_RELPOS) {
          const float* br = bias_lds + (blk * 32 + 4 * g + BNK - 1) - kvl;
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] += br[8 * (i >> 2) + (i & 3)];
        } else if (p.bias_kind == JFA_BIAS_DENSE) {
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const f32x4 bv = *(const f32x4*)(bias_lds + kvl * BS + blk * 32 + 8 * jq + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * jq + e] += bv[e];
          }
        }
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const int ql = blk * 32 + 8 * jq + 4 * g;
          f32x4 l2 = {0.f, 0.f, 0.f, 0.f}, dl = {0.f, 0.f, 0.f, 0.f};
          if constexpr (MODE == MODE_SOFTMAX) {
            l2 = *(const f32x4*)(lse_lds + ql);
            dl = *(const f32x4*)(dlt_lds + ql);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * jq + e;
            const int qi = q0 + ql + e;
            const bool valid = !need_mask || (qi < n && j < m && (!p.causal || j <= qi + delta));
            if constexpr (MODE == MODE_SOFTMAX) {
              const float pr = valid ? fast_exp2(x[i] - l2[e]) : 0.f;
              pv[blk][i] = pr;
              ds[blk][i] = pr * (pacc[blk][i] - dl[e]);
            } else {
              pv[blk][i] = valid ? act_f<MODE>(x[i]) * wn : 0.f;
              ds[blk][i] = valid ? act_grad_f<MODE>(x[i]) * pacc[blk][i] * wn : 0.f;
            }
          }
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS (chunk c covers queries 16c + 8(e/4) + 4g + e%4)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 pop = pack_chunk(pv, c);
        const bf16x8 dsop = pack_chunk(ds, c);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const __bf16* drow = dot_lds + (db * 32 + l32) * TS + 16 * c + 4 * g;
          dv[db] = mfma_bf16(cat_bf16x8(*(const u32x2*)drow, *(const u32x2*)(drow + 8)), pop, dv[db]);
          const __bf16* qrow = qt_lds + (db * 32 + l32) * TS + 16 * c + 4 * g;
          dk[db] = mfma_bf16(cat_bf16x8(*(const u32x2*)qrow, *(const u32x2*)(qrow + 8)), dsop, dk[db]);
        }
      }
    }
    if (j < m) {
      __bf16* okr = (__bf16*)p.dk + rowk * D;
      __bf16* ovr = (__bf16*)p.dv + rowk * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          u32x2 pk = {pack2bf(dk[db][4 * jq] * p.scale, dk[db][4 * jq + 1] * p.scale),
                      pack2bf(dk[db][4 * jq + 2] * p.scale, dk[db][4 * jq + 3] * p.scale)};
          *(u32x2*)(okr + db * 32 + 8 * jq + 4 * g) = pk;
          u32x2 pv2 = {pack2bf(dv[db][4 * jq], dv[db][4 * jq + 1]),
                       pack2bf(dv[db][4 * jq + 2], dv[db][4 * jq + 3])};
          *(u32x2*)(ovr + db * 32 + 8 * jq + 4 * g) = pv2;
        }
    }
  }
}

template <int D, int NW, int MODE>
hipError_t run_bq(const BwdParams& p, int64_t max_items, int cu, hipStream_t s) {
  using L = BqLds<D, NW>;
  auto kern = bwd_q_kernel<D, NW, MODE>;
  static int attr = 0;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       L::total(JFA_BIAS_DENSE));
    if (e != hipSuccess) return e;
    attr = 1;
  }
  const size_t lds = L::total(p.bias_kind);
  int grid = resident_grid((const void*)kern, NW * 64, lds, cu);
  if ((int64_t)grid > max_items) grid = (int)max(max_items, (int64_t)1);
  timing_begin("jfa_bwd_dq", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, s, p);
  timing_end(s);
  return hipGetLastError();
}

template <int D, int NW, int MODE>
hipError_t run_bk(const BwdParams& p, int64_t max_items, int cu, hipStream_t s) {
  using L = BkLds<D, NW>;
  auto kern = bwd_kv_kernel<D, NW, MODE>;
  static int attr = 0;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       L::total(JFA_BIAS_DENSE));
    if (e != hipSuccess) return e;
    attr = 1;
  }
  const size_t lds = L::total(p.bias_kind);
  int grid = resident_grid((const void*)kern, NW * 64, lds, cu);
  if ((int64_t)grid > max_items) grid = (int)max(max_items, (int64_t)1);
  timing_begin("jfa_bwd_dkdv", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, s, p);
  timing_end(s);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t run_bwd(const BwdParams& p, const TileCfg& tc, int64_t mq, int64_t mk, int cu,
                   hipStream_t s) {
  hipError_t e = hipSuccess;
  if (MODE == MODE_SOFTMAX) {
    constexpr int RPB = 256 / (D / 8);
    const int64_t pairs = p.total_q * p.H;
    if (pairs > 0) {
      timing_begin("jfa_bwd_delta", s);
      hipLaunchKernelGGL((delta_kernel<__bf16, D>), dim3((unsigned)((pairs + RPB - 1) / RPB)),
                         dim3(256), 0, s, (const __bf16*)p.o, (const __bf16*)p.dout, p.delta,
                         p.total_q, p.H);
      timing_end(s);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  e = tc.bk_nw == 4 ? run_bk<D, 4, MODE>(p, mk, cu, s) : run_bk<D, 2, MODE>(p, mk, cu, s);
  if (e != hipSuccess) return e;
  return tc.bq_nw == 4 ? run_bq<D, 4, MODE>(p, mq, cu, s) : run_bq<D, 2, MODE>(p, mq, cu, s);
}

}  // namespace

hipError_t launch_backward_f32(const BwdParams& p, const TileCfg& tc, int head_dim,
                               int64_t max_q_items, int64_t max_k_items, int cu_count,
                               hipStream_t s);

hipError_t launch_backward(const BwdParams& p, const TileCfg& tc, int head_dim, int dtype,
                           int64_t max_q_items, int64_t max_k_items, int cu_count, hipStream_t s) {
  if (dtype == JFA_F32)
    return launch_backward_f32(p, tc, head_dim, max_q_items, max_k_items, cu_count, s);
  if (dtype != JFA_BF16) return hipErrorInvalidValue;
#define JFA_BWD_CASE(D_)                                                                       \
  if (head_dim == D_) {                                                                        \
    switch (p.mode) {                                                                          \
      case MODE_SOFTMAX: return run_bwd<D_, MODE_SOFTMAX>(p, tc, max_q_items, max_k_items, cu_count, s); \
      case MODE_SILU: return run_bwd<D_, MODE_SILU>(p, tc, max_q_items, max_k_items, cu_count, s);       \
      default: return run_bwd<D_, MODE_GELU>(p, tc, max_q_items, max_k_items, cu_count, s);              \
    }                                                                                          \
  }
  JFA_BWD_CASE(128)
  JFA_BWD_CASE(64)
#undef JFA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace jfa
