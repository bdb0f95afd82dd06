// Jagged attention backward on MFMA (bf16): softmax preprocess, key-stationary dK/dV pass and
// query-stationary dQ pass.
//
// Source: "Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a Different Stack",
// section "Bottleneck move 1": GDPA (SiLU/GELU in place of softmax) forward and backward;
// removing padding exposes backward accumulation.  The gradients are those of <O, dO>:
//   softmax: dP = dO V^T, dS = P (dP - D), D_i = dO_i . O_i, dV = P^T dO
//   GDPA:    dP = w dO V^T, dS = act'(S) dP, dV = w act(S)^T dO    (w = 1/kv_len or 1)
//   dQ = scale dS K, dK = scale dS^T Q.
//
// Determinism without float atomics: the key-stationary kernel owns dK/dV rows and sums over
// query steps in order in registers; the query-stationary kernel owns dQ rows and sums over
// key steps in order.  Each recomputes S (and P) from the forward's log-sum-exp.
//
// Layout (gfx950), shared with the forward:
//  - the key-stationary kernel works on S = Q K^T with a lane owning one key column; the
//    query-stationary kernel on S^T = K Q^T with a lane owning one query column.  In both the
//    lane's accumulator column is exactly the B operand of the gradient MFMAs, so P and dS
//    never go through LDS;
//  - every tile is staged global -> registers -> LDS one step ahead (two LDS stages, one
//    barrier per step), row-major; operands contracted over the step's rows (Q^T, dO^T, K^T)
//    are read from the row tiles with transposing LDS reads (ds_read_b64_tr_b16);
//  - loads and stores go through per-(sample, head) buffer resources: rows past a sample's
//    end read as zero and are never written, with no branches;
//  - the additive bias initialises the S accumulator (bias / scale).
//
// This file is compiled once per (head dim, mode) pair, with JFA_BWD_D and JFA_BWD_MODE set by
// the build (the instances build in parallel).
#include "jfa_device.h"
#include "jfa_internal.h"

#if !defined(JFA_BWD_D) || !defined(JFA_BWD_MODE) || !defined(JFA_BWD_FP8)
#error "compile with -DJFA_BWD_D=<64|128> -DJFA_BWD_MODE=<0|1|2> -DJFA_BWD_FP8=<0|1>"
#endif
#include <type_traits>

namespace jfa {
namespace {

enum BiasT { B_NONE = 0, B_RELPOS = 1, B_DENSE = 2 };
constexpr int STEP = 64;   // rows per step of either kernel's inner loop

constexpr int align16(int x) { return (x + 15) / 16 * 16; }

// --------------------------------------------------------------- tile staging
// The NT threads that stage a tile are the first NT of the workgroup or, in a workgroup of more
// threads, any NT consecutive ones (thread index taken modulo NT).
// An MXFP8 STEP x D tile is moved as blocks of 4 rows x 8 dims (one load per row).
// Block id -> (row block rb, dim block cb): within each 16 ids, 4 row blocks x 4 dim blocks,
// so that a quarter wave's row-major writes cover all banks.
__device__ __forceinline__ void blk_of(int id, int& rb, int& cb) {
  rb = ((id >> 2) & 3) | (((id >> 4) & 3) << 2);
  cb = (id & 3) | ((id >> 6) << 2);
}

// Row-major-only staging of a STEP x D tile: 16-byte chunks, consecutive lanes along a row.
template <int D, int NT>
struct RowTile {
  static constexpr int KCH = D / 8;
  static constexpr int NL = STEP * KCH / NT;
  static_assert(STEP * KCH % NT == 0, "row tile staging");
  u32x4 v[NL];
  __device__ __forceinline__ void load(rsrc_t r, uint32_t row_bytes, int r0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int id = (int)(threadIdx.x % NT) + i * NT;
      v[i] = ld16(r, (uint32_t)(r0 + id / KCH) * row_bytes + 16 * (id % KCH));
    }
  }
  __device__ __forceinline__ void store(__bf16* rows) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int id = (int)(threadIdx.x % NT) + i * NT;
      *(u32x4*)(rows + (id / KCH) * tile_row_stride<D>() + 8 * (id % KCH)) = v[i];
    }
  }
};

// MXFP8 inputs: the same STEP x D tile staging as Tile (4 rows x 8 dims per block, row-major
// stores only), loading 8 E4M3 codes and the row's E8M0 scale per row and block and storing
// them dequantised to bf16 (exact), so the MFMAs and every LDS layout stay those of bf16.
template <int D, int NT>
struct Fp8Tile {
  static constexpr int NBLK = (STEP / 4) * (D / 8);
  static constexpr int NB = (NBLK + NT - 1) / NT;
  static constexpr int PARTS = 6 * NB;
  u32x2 c[NB][4];
  uint32_t sc[NB][4];

  // rc: codes (row stride crow bytes), rs: scales (row stride srow bytes)
  __device__ __forceinline__ void load(rsrc_t rc, rsrc_t rs, uint32_t crow, uint32_t srow,
                                       int r0) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int id = (int)(threadIdx.x % NT) + i * NT;
      if (NBLK % NT != 0 && id >= NBLK) break;
      int rb, cb;
      blk_of(id, rb, cb);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint32_t row = (uint32_t)(r0 + 4 * rb + rr);
        c[i][rr] = ld8(rc, row * crow + 8 * cb);
        sc[i][rr] = ld1(rs, row * srow + (8 * cb) / 32);
      }
    }
  }
  // parts 0, 1 of block I write its rows 2 PART, 2 PART + 1; parts 2..5 (the transposed copies
  // of Tile) are not used with MXFP8 inputs
  template <int P>
  __device__ __forceinline__ void store_part(__bf16* rows, __bf16* tr) const {
    constexpr int i = P / 6, part = P % 6;
    static_assert(part < 2, "row stores only");
    const int id = (int)(threadIdx.x % NT) + i * NT;
    if (NBLK % NT != 0 && id >= NBLK) return;
    int rb, cb;
    blk_of(id, rb, cb);
#pragma unroll
    for (int rr = 2 * part; rr < 2 * part + 2; ++rr)
      *(bf16x8*)(rows + (4 * rb + rr) * tile_row_stride<D>() + 8 * cb) =
          dequant8_bf16(c[i][rr], sc[i][rr]);
  }
  __device__ __forceinline__ void store(__bf16* rows) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int id = (int)(threadIdx.x % NT) + i * NT;
      if (NBLK % NT != 0 && id >= NBLK) break;
      int rb, cb;
      blk_of(id, rb, cb);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *(bf16x8*)(rows + (4 * rb + rr) * tile_row_stride<D>() + 8 * cb) =
            dequant8_bf16(c[i][rr], sc[i][rr]);
    }
  }
};

// RowTile's staging for MXFP8 inputs: 8 codes per thread and chunk, dequantised on the store.
template <int D, int NT>
struct Fp8RowTile {
  static constexpr int KCH = D / 8;
  static constexpr int NL = STEP * KCH / NT;
  static_assert(STEP * KCH % NT == 0, "row tile staging");
  u32x2 c[NL];
  uint32_t sc[NL];
  __device__ __forceinline__ void load(rsrc_t rc, rsrc_t rs, uint32_t crow, uint32_t srow,
                                       int r0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int id = (int)(threadIdx.x % NT) + i * NT;
      const uint32_t row = (uint32_t)(r0 + id / KCH);
      c[i] = ld8(rc, row * crow + 8 * (id % KCH));
      sc[i] = ld1(rs, row * srow + (8 * (id % KCH)) / 32);
    }
  }
  __device__ __forceinline__ void store(__bf16* rows) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int id = (int)(threadIdx.x % NT) + i * NT;
      *(bf16x8*)(rows + (id / KCH) * tile_row_stride<D>() + 8 * (id % KCH)) =
          dequant8_bf16(c[i], sc[i]);
    }
  }
};

// A lane's 8 consecutive elements of one (row, head) vector as an MFMA operand: bf16 loaded
// directly, or MXFP8 codes and their block scale dequantised (byte offsets of element e0).
template <int D, bool FP8>
__device__ __forceinline__ bf16x8 load_frag8(rsrc_t r, rsrc_t rs, uint32_t row, uint32_t row_b,
                                             uint32_t srow, int e0) {
  if constexpr (FP8)
    return dequant8_bf16(ld8(r, row * row_b + e0), ld1(rs, row * srow + e0 / 32));
  else
    return as_bf16x8(ld16(r, row * row_b + 2 * e0));
}

// Four copies of a diagonal bias table, copy k shifted by k floats, so that any run of 4
// consecutive entries is one aligned 16-byte read from the copy k = (4 - start % 4) % 4.
template <int RP>
__device__ __forceinline__ void store_diag(float* rp, int idx, float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) rp[k * RP + idx + k] = v;
}

// ================================================= key-stationary dK, dV
template <int D, int NW, int BIAS>
struct KvLds {
  static constexpr int BNK = 32 * NW;
  static constexpr int RS = tile_row_stride<D>();
  static constexpr int QR = 0;                            // Q rows [STEP][RS]
  static constexpr int DR = QR + STEP * RS * 2;           // dO rows
  // Q^T and dO^T operands are read from the row tiles with transposing LDS reads
  static constexpr int LS = DR + STEP * RS * 2;           // lse / scale [STEP]
  static constexpr int DL = LS + STEP * 4;                // -delta [STEP]
  static constexpr int BO = DL + STEP * 4;
  static constexpr int RP = diag_stride(STEP + BNK + 4);
  static constexpr int BS = STEP + 8;                     // dense tile [BNK][BS] bf16 (key-major)
  static constexpr int BIAS_BYTES =
      BIAS == B_RELPOS ? 4 * RP * 4 : (BIAS == B_DENSE ? BNK * BS * 2 : 0);
  // a stage also holds the epilogue's dK and dV rows (two staging areas per wave)
  static constexpr int STAGE = align16(BO + BIAS_BYTES) > 2 * NW * out_stage_bytes<D>()
                                   ? align16(BO + BIAS_BYTES) : 2 * NW * out_stage_bytes<D>();
  // single pass for a sample with one key tile (built at d = 64): the item's K rows and each
  // step's dS, from which the workgroup also computes the step's dQ
  static constexpr bool K1 = D == 64;
  static constexpr int QS = STEP + 8;                     // dS tile [BNK keys][QS] (bf16)
  static constexpr int K1_KR = 2 * STAGE;
  static constexpr int K1_DS = K1_KR + BNK * RS * 2;
  static constexpr int TOTAL = 2 * STAGE + (K1 ? BNK * RS * 2 + BNK * QS * 2 : 0);
};

// The key-stationary pass over the kv-stationary list, on the workgroup's dynamic LDS.  (The
// dynamic LDS is named here, not passed in: a pointer argument costs the constant LDS offsets
// and, in the one-query-tile kernels, registers enough to spill.)
// HOME: the first item of workgroup g is item g (the pass starts the launch); otherwise every
// item comes from a ticket.
template <int D, int NW, int MODE, int BIAS, bool HOME, bool WIN, bool FP8>
__device__ __forceinline__ void kv_pass(const BwdParams& p) {
  extern __shared__ __align__(16) unsigned char lds[];
  using L = KvLds<D, NW, BIAS>;
  constexpr int BNK = L::BNK, NT = NW * 64, RS = L::RS;
  __shared__ int s_desc[2][IF_WORDS];

  if (p.hdr->status != JFA_OK) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr->counts[3] * H;
  // this lane's element of a transposing read: row 4(G/2) + (j/4), column 16(G%2) + 4(j%4) for
  // 16-lane group G and lane j within it (plus the operand's base row and column)
  const int tr_lane = (4 * (lane >> 5) + ((lane & 15) >> 2)) * L::RS + 16 * ((lane >> 4) & 1) +
                      4 * (lane & 3);
  const float c_log = MODE == MODE_SOFTMAX ? p.scale * LOG2E : p.scale;
  const float inv_scale = 1.0f / p.scale;
  const uint32_t row_bytes = (uint32_t)H * D * 2;          // bf16 rows (outputs, bf16 inputs)
  constexpr int ES = FP8 ? 1 : 2;                           // bytes per input element
  const uint32_t in_row = (uint32_t)H * D * ES;             // input row stride
  const uint32_t sc_row = (uint32_t)H * (D / 32);           // MXFP8 scale row stride

  // bf16 tiles are staged row-major, consecutive lanes along a row (full cache lines per load)
  std::conditional_t<FP8, Fp8Tile<D, NT>, RowTile<D, NT>> tq, tdo;
  float lsv = 0.f, dlv = 0.f;       // lse / delta entry staged by threads < STEP
  float rpv = 0.f;                  // relpos table entry
  // Dense bias: NDB units per thread and step, each two 16-byte chunks (8 keys of queries q and
  // q + 1) that are stored transposed as (q, q + 1) pairs per key; prefetched into registers
  // with the Q / dO tiles unless registers run short (then loaded while staging).
  constexpr int KCHK = BNK / 8;
  constexpr int NDB = BIAS == B_DENSE ? (STEP / 2) * KCHK / NT : 1;
  constexpr int NPRE = D == 128 ? 0 : NDB;
  BiasRaw dbr[NPRE > 0 ? NPRE : 1][2];

  ItemPipeT<HOME> pipe{p.xtk_k, p.bk, (int)n_items, H};
  if (wave == 0) pipe.start(s_desc[0], lane);
  __syncthreads();
  for (int buf = 0;; buf ^= 1) {
    const int* dsc = s_desc[buf];
    const int w = item_field(dsc, IF_W);
    if (w >= n_items) break;
    const int h = w % H;
    const int u = item_field(dsc, IF_X), qs_first = item_field(dsc, IF_Y);
    const int qs_end = item_field(dsc, IF_Z);
    // the next item: a short item takes its ticket now and reads its record right after this
    // item's first loads (both round trips overlap those loads); a longer one claims it
    // CLAIM_AHEAD steps before its end
    const int nsteps = qs_end - qs_first;
    const bool short_item = nsteps <= CLAIM_AHEAD;
    if (short_item && wave == 0) pipe.claim(lane);
    const int qo = item_field(dsc, IF_QO), n = item_field(dsc, IF_N);
    const int ko = item_field(dsc, IF_KO), m = item_field(dsc, IF_M);
    const int64_t boff = item_boff(dsc);
    const int delta = m - n;
    const float wn = (MODE != MODE_SOFTMAX && p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    const int j0 = u * BNK, jw0 = j0 + wave * 32;
    // single-pass class (the scheduler's test): one key tile and not one query tile
    const bool one_k = L::K1 && (p.fuse & 2) && !((p.fuse & 1) && n > 0 && n <= p.bq_bm) &&
                       m > 0 && m <= BNK;
    const int kvl = wave * 32 + l32, j = j0 + kvl;

    const uint32_t kv_bytes = m > 0 ? ((uint32_t)(m - 1) * H + 1) * D * 2 : 0;
    const uint32_t q_bytes = n > 0 ? ((uint32_t)(n - 1) * H + 1) * D * 2 : 0;
    const uint32_t kv_in = m > 0 ? ((uint32_t)(m - 1) * H + 1) * D * ES : 0;
    const uint32_t q_in = n > 0 ? ((uint32_t)(n - 1) * H + 1) * D * ES : 0;
    const rsrc_t rk = make_rsrc((const uint8_t*)p.k + ((int64_t)ko * H + h) * D * ES, kv_in);
    const rsrc_t rv = make_rsrc((const uint8_t*)p.v + ((int64_t)ko * H + h) * D * ES, kv_in);
    const rsrc_t rq = make_rsrc((const uint8_t*)p.q + ((int64_t)qo * H + h) * D * ES, q_in);
    const rsrc_t rdo = make_rsrc((const uint8_t*)p.dout + ((int64_t)qo * H + h) * D * ES, q_in);
    rsrc_t rks = rk, rvs = rv, rqs = rq, rdos = rdo;
    if constexpr (FP8) {
      const uint32_t kv_s = m > 0 ? ((uint32_t)(m - 1) * H + 1) * (D / 32) : 0;
      const uint32_t q_s = n > 0 ? ((uint32_t)(n - 1) * H + 1) * (D / 32) : 0;
      rks = make_rsrc(p.k_sc + ((int64_t)ko * H + h) * (D / 32), kv_s);
      rvs = make_rsrc(p.v_sc + ((int64_t)ko * H + h) * (D / 32), kv_s);
      rqs = make_rsrc(p.q_sc + ((int64_t)qo * H + h) * (D / 32), q_s);
      rdos = make_rsrc(p.do_sc + ((int64_t)qo * H + h) * (D / 32), q_s);
    }
    rsrc_t rls = rq, rdl = rq, rb = rq;
    if constexpr (MODE == MODE_SOFTMAX) {
      rls = make_rsrc(p.lse + (int64_t)h * p.total_q + qo, (uint32_t)n * 4u);
      rdl = make_rsrc(p.delta + (int64_t)h * p.total_q + qo, (uint32_t)n * 4u);
    }
    if constexpr (BIAS == B_DENSE)
      rb = make_rsrc((const __bf16*)p.bias + (int64_t)H * boff + (int64_t)h * n * m,
                     (uint32_t)n * (uint32_t)m * 2u);

    // this lane's key as the B operand (column = key, k = head dim)
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = load_frag8<D, FP8>(rk, rks, (uint32_t)j, in_row, sc_row, 16 * ks + 8 * g);
      vf[ks] = load_frag8<D, FP8>(rv, rvs, (uint32_t)j, in_row, sc_row, 16 * ks + 8 * g);
    }

    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) { dk[db][i] = 0.f; dv[db][i] = 0.f; }

    // chunk (i, half) of this thread for query step q0: byte offset and valid element count
    auto dense_at = [&](int i, int q0, int half, uint32_t& off, int& valid) {
      const int id = tid + i * NT;
      const int qa = q0 + 2 * (id / KCHK) + half, k0 = j0 + 8 * (id % KCHK);
      valid = qa < n ? min(8, m - k0) : 0;
      off = ((uint32_t)qa * (uint32_t)m + (uint32_t)k0) * 2u;
    };
    const uint32_t bias_bytes = (uint32_t)n * (uint32_t)m * 2u;
    auto dense_chunk = [&](int i, int q0, int half) -> u32x4 {
      uint32_t off;
      int valid;
      dense_at(i, q0, half, off, valid);
      return bias_chunk(rb, off, valid, bias_bytes);
    };
    auto load_step = [&](int qs) {
      const int q0 = qs * STEP;
      if constexpr (BIAS == B_RELPOS) {
        // T[x] = bias(dist = q0 + delta - j0 + x - (BNK - 1)), x = query - key + BNK - 1
        if (tid < STEP + BNK - 1) {
          const int dist = q0 + delta - j0 + tid - (BNK - 1);
          rpv = ((const float*)p.bias)[(int64_t)h * p.num_buckets +
                                       relpos_bucket(dist, p.num_buckets)];
        }
      }
      if constexpr (MODE == MODE_SOFTMAX) {
        if (tid < STEP) {
          lsv = __uint_as_float(ld4(rls, (uint32_t)(q0 + tid) * 4u));
          dlv = __uint_as_float(ld4(rdl, (uint32_t)(q0 + tid) * 4u));
        }
      }
      if constexpr (FP8) {
        tq.load(rq, rqs, in_row, sc_row, q0);
        tdo.load(rdo, rdos, in_row, sc_row, q0);
      } else {
        tq.load(rq, row_bytes, q0);
        tdo.load(rdo, row_bytes, q0);
      }
      if constexpr (BIAS == B_DENSE) {
#pragma unroll
        for (int i = 0; i < NPRE; ++i)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t off;
            int valid;
            dense_at(i, q0, half, off, valid);
            dbr[i][half] = bias_chunk_load(rb, off, valid, bias_bytes);
          }
      }
    };
    // the Q and dO rows of a step into LDS stage st
    auto store_tiles = [&](int st) {
      unsigned char* base = lds + st * L::STAGE;
      if constexpr (FP8) {
        // row stores only (pieces 0, 1 of every 6): no transposed copies
        constexpr int TP = decltype(tq)::PARTS;
        static_for<0, 2 * TP>([&](auto pc) {
          constexpr int P = decltype(pc)::value;
          if constexpr (P % 6 < 2) {
            if constexpr (P < TP)
              tq.template store_part<P>(reinterpret_cast<__bf16*>(base + L::QR), nullptr);
            else
              tdo.template store_part<P - TP>(reinterpret_cast<__bf16*>(base + L::DR), nullptr);
          }
        });
      } else {
        tq.store(reinterpret_cast<__bf16*>(base + L::QR));
        tdo.store(reinterpret_cast<__bf16*>(base + L::DR));
      }
    };
    auto store_step = [&](int st, int qs, bool tiles) {
      unsigned char* base = lds + st * L::STAGE;
      const int q0 = qs * STEP;
      if (tiles) store_tiles(st);
      if constexpr (MODE == MODE_SOFTMAX) {
        if (tid < STEP) {
          // rows without a visible key have lse = -inf; all their pairs are masked to -inf,
          // so any finite value keeps exp2(-inf - lse) = 0
          reinterpret_cast<float*>(base + L::LS)[tid] = lsv == NEG_INF ? 0.f : lsv * LOG2E;
          reinterpret_cast<float*>(base + L::DL)[tid] = -dlv;   // stored negated: dP starts at -D
        }
      }
      if constexpr (BIAS == B_RELPOS) {
        if (tid < STEP + BNK - 1)
          store_diag<L::RP>(reinterpret_cast<float*>(base + L::BO), tid, rpv * inv_scale);
      } else if constexpr (BIAS == B_DENSE) {
        // key-major tile [BNK][BS]: two query rows per thread and key, coalesced along keys
        __bf16* bt = reinterpret_cast<__bf16*>(base + L::BO);
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
          const int id = tid + i * NT;
          u32x4 a, c;
          if (i < NPRE) {
            uint32_t off;
            int valid;
            dense_at(i, q0, 0, off, valid);
            a = bias_chunk_finish(dbr[i][0], off, valid, bias_bytes);
            dense_at(i, q0, 1, off, valid);
            c = bias_chunk_finish(dbr[i][1], off, valid, bias_bytes);
          } else {
            a = dense_chunk(i, q0, 0);
            c = dense_chunk(i, q0, 1);
          }
          __bf16* dst = bt + 8 * (id % KCHK) * L::BS + 2 * (id / KCHK);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            *(uint32_t*)(dst + (2 * w) * L::BS) = lo_halves(a[w], c[w]);
            *(uint32_t*)(dst + (2 * w + 1) * L::BS) = hi_halves(a[w], c[w]);
          }
        }
      }
    };

    // One query step, software-pipelined by hand.  The step is a stream of 64 MFMAs:
    //   A(h), h = 0, 1: S_h = Q_h K^T and dP_h = dO_h V^T    (queries 32h .. 32h+31)
    //   C(h):           dV^T += dO_h^T P_h, dK^T += Q_h^T dS_h
    // in the order A(0) A(1) C(0) C(1).  Every MFMA's LDS operand is read PF MFMAs ahead, and the
    // VALU work B(h) that turns S_h, dP_h into P_h, dS_h is spread one element per MFMA over the
    // next phase (B(0) under A(1), B(1) under C(0)), so the matrix cores stay busy in this
    // one-wave-per-SIMD kernel.  sched_barrier pins that order against the compiler's scheduler.
    auto compute_step = [&](int it, int qs) {
      const int q0 = qs * STEP;
      const unsigned char* sb = lds + (it & 1) * L::STAGE;
      // nothing visible between this step's queries and the wave's keys (past the sample,
      // before the causal diagonal, or outside the window band)
      const int W = WIN ? p.window : 0;
      if (jw0 >= m || (p.causal && q0 + STEP - 1 + delta < jw0) ||
          (WIN && (q0 > jw0 + 31 - delta + W - 1 ||
                   (!p.causal && q0 + STEP - 1 < jw0 - delta - W + 1)))) {
        if (L::K1 && one_k) {     // these keys contribute nothing to this step's dQ
          uint32_t* ds = reinterpret_cast<uint32_t*>(
              reinterpret_cast<__bf16*>(lds + L::K1_DS) + kvl * L::QS);
#pragma unroll
          for (int i = 0; i < STEP / 2 / 2; ++i) ds[2 * i + g] = 0u;
        }
        return;
      }
      const __bf16* qr = reinterpret_cast<const __bf16*>(sb + L::QR);
      const __bf16* dr = reinterpret_cast<const __bf16*>(sb + L::DR);
      const float* lsl = reinterpret_cast<const float*>(sb + L::LS);
      const float* dll = reinterpret_cast<const float*>(sb + L::DL);
      // element (blk, i): query q0 + blk*32 + 8(i/4) + 4g + i%4 of this step, key j
      f32x16 sacc[2], pacc[2];
      if constexpr (BIAS == B_RELPOS) {
        const float* rp = reinterpret_cast<const float*>(sb + L::BO);
        const int k = (1 + kvl) & 3;
        const float* src = rp + k * L::RP + k + 4 * g - kvl + BNK - 1;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x4 bv = *(const f32x4*)(src + blk * 32 + 8 * qd);
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[blk][4 * qd + e] = bv[e];
          }
      } else if constexpr (BIAS == B_DENSE) {
        const __bf16* bt = reinterpret_cast<const __bf16*>(sb + L::BO) + kvl * L::BS + 4 * g;
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
      // pairs that are not visible start at -inf, so P = 0 and dS = 0 with no per-element test
      // later: query offset o = blk*32 + 8(i/4) + i%4 (+4g) is visible iff qlo <= o < qhi
      // (GDPA needs no mask at the sample's ends: a query row past them has Q and dO rows that
      // read as zero, a key past them K and V rows that do, and dense-bias entries there load
      // as zero, so such a pair's terms in dK, dV and dQ vanish; softmax keeps the mask, since
      // its P there would not be zero)
      const bool need_mask = (MODE == MODE_SOFTMAX && (q0 + STEP > n || jw0 + 32 > m)) ||
                             (p.causal && q0 + delta < jw0 + 31) ||
                             (WIN && (q0 + STEP - 1 >= jw0 - delta + W ||
                                      (!p.causal && q0 <= jw0 + 31 - delta - W)));
      if (need_mask) {
        // queries [qlo, qhi) (offsets in the step, less 4g) see key j
        int qhi = j < m ? n - q0 - 4 * g : -1;
        int qlo = p.causal ? j - delta - q0 - 4 * g : -1;
        if constexpr (WIN) {
          if (j < m) qhi = min(n, j - delta + W) - q0 - 4 * g;
          if (!p.causal) qlo = j - delta - W + 1 - q0 - 4 * g;
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int o = blk * 32 + 8 * (i >> 2) + (i & 3);
            if (o < qlo || o >= qhi) sacc[blk][i] = NEG_INF;
          }
      }
      // softmax: dP starts at -delta (loaded straight into the accumulator), so that the VALU
      // work per pair is P = exp2(S c - lse log2 e) (one fma and the exp), dS = P dP (masked
      // pairs stay at -inf); the lse of the lane's queries is read from LDS beside the MFMAs
      if constexpr (MODE == MODE_SOFTMAX) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x4 dl = *(const f32x4*)(dll + blk * 32 + 8 * qd + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) pacc[blk][4 * qd + e] = dl[e];
          }
      } else {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) pacc[blk][i] = 0.f;
      }

      constexpr int NA = D / 8;          // MFMAs per phase: 16 at d = 128, 8 at d = 64
      constexpr int NS = 4 * NA;         // MFMAs per step
      constexpr int PF = 6;              // operand read distance (MFMAs)
      constexpr int RING = 8;
      // operand of stream MFMA s
      auto opnd = [&](int s) -> u32x4 {
        if (s < 2 * NA) {
          const int h = s / NA, jj = s % NA, ks = jj >> 1;
          const __bf16* base = (jj & 1) ? dr : qr;
          return *(const u32x4*)(base + (h * 32 + l32) * RS + 16 * ks + 8 * g);
        }
        // dV^T += dO^T P_h, dK^T += Q^T dS_h: A operand rows = head dims db*32 + (lane % 32),
        // k = 8g + j <-> query 32h + 16cc + 8(j/4) + 4g + j%4 of the step (the order in which
        // P and dS leave the S accumulator), read as two column strips of 4 queries
        const int h = (s - 2 * NA) / NA, jj = (s - 2 * NA) % NA;
        const int cc = jj / (NA / 2), db = (jj % (NA / 2)) >> 1;
        const __bf16* p = ((jj & 1) ? qr : dr) + tr_lane + (32 * h + 16 * cc) * RS + db * 32;
        const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * RS);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      uint32_t pp[2][8], dd[2][8];
      // lse log2 e of this lane's queries of half h, quad qd (softmax)
      f32x4 lq[2][4];
      auto load_lse = [&](int h) {
        if constexpr (MODE == MODE_SOFTMAX) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            lq[h][qd] = *(const f32x4*)(lsl + h * 32 + 8 * qd + 4 * g);
        }
      };
      // B(h) element i (query offset blk*32 + 8(i/4) + i%4 with blk = h), in two stages one MFMA
      // apart, so that no dependent chain of an element waits inside one MFMA slot: b_front
      // forms P (and the activation's derivative) from S, b_back forms dS and packs the pair.
      float pv_t = 0.f, ds_t = 0.f;
      float fr_p[2] = {0.f, 0.f}, fr_d[2] = {0.f, 0.f};   // front results by element parity
      auto b_front = [&](int h, int i) {
        if constexpr (MODE == MODE_SOFTMAX) {
          fr_p[i & 1] = fast_exp2(fmaf(sacc[h][i], c_log, -lq[h][i >> 2][i & 3]));
        } else {
          // masked pairs hold -inf: clamped to -1e30, the activation and its derivative are
          // exactly zero (the exponential and the reciprocal saturate) and a NaN logit still
          // propagates; the weight 1 / kv_len is applied to dK and dV as a whole
          float x = sacc[h][i] * c_log;
          x = act_clamp(x);
          act_pair<MODE>(x, fr_p[i & 1], fr_d[i & 1]);
        }
      };
      auto b_back = [&](int h, int i) {
        const float pv = fr_p[i & 1];
        const float dsv = (MODE == MODE_SOFTMAX ? pv : fr_d[i & 1]) * pacc[h][i];
        if (i & 1) {
          pp[h][i >> 1] = pack2bf(pv_t, pv);
          dd[h][i >> 1] = pack2bf(ds_t, dsv);
        } else {
          pv_t = pv;
          ds_t = dsv;
        }
      };
      auto mfma_s = [&](int s, u32x4 o) {
        const bf16x8 a = as_bf16x8(o);
        if (s < 2 * NA) {
          const int h = s / NA, jj = s % NA, ks = jj >> 1;
          if (jj & 1) pacc[h] = mfma_bf16(a, vf[ks], pacc[h]);
          else sacc[h] = mfma_bf16(a, kf[ks], sacc[h]);
          return;
        }
        const int h = (s - 2 * NA) / NA, jj = (s - 2 * NA) % NA;
        const int cc = jj / (NA / 2), db = (jj % (NA / 2)) >> 1;
        if (jj & 1) {
          const u32x4 w = {dd[h][4 * cc], dd[h][4 * cc + 1], dd[h][4 * cc + 2], dd[h][4 * cc + 3]};
          dk[db] = mfma_bf16(a, as_bf16x8(w), dk[db]);
        } else {
          const u32x4 w = {pp[h][4 * cc], pp[h][4 * cc + 1], pp[h][4 * cc + 2], pp[h][4 * cc + 3]};
          dv[db] = mfma_bf16(a, as_bf16x8(w), dv[db]);
        }
      };
      u32x4 ring[RING];
      static_for<0, PF>([&](auto s) { ring[s] = opnd(s); });
      static_for<0, NS>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        if constexpr (s + PF < NS) ring[(s + PF) % RING] = opnd(s + PF);
        // each half's lse a phase before its exps
        if constexpr (s == NA / 2) load_lse(0);
        if constexpr (s == NA + NA / 2) load_lse(1);
        mfma_s(s, ring[s % RING]);
        // B(0) under A(1), B(1) under C(0): one element per MFMA (16 elements per half), each
        // element's back stage under the MFMA after its front stage (B(0)'s last back stages
        // under the first MFMA of C(0), B(1)'s under the first of C(1): the chunks they feed
        // start later)
        constexpr int EPM = 16 / NA;     // elements per MFMA (1 at d = 128, 2 at d = 64)
        if constexpr (s >= NA + 1 && s <= 2 * NA) {
          static_for<0, EPM>([&](auto e) { b_back(0, (s - NA - 1) * EPM + e); });
        }
        if constexpr (s >= 2 * NA + 1 && s <= 3 * NA) {
          static_for<0, EPM>([&](auto e) { b_back(1, (s - 2 * NA - 1) * EPM + e); });
        }
        if constexpr (s >= NA && s < 2 * NA) {
          static_for<0, EPM>([&](auto e) { b_front(0, (s - NA) * EPM + e); });
        }
        if constexpr (s >= 2 * NA && s < 3 * NA) {
          static_for<0, EPM>([&](auto e) { b_front(1, (s - 2 * NA) * EPM + e); });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (L::K1 && one_k) {
        // dS [key][query] of this step: element pair p of half h holds queries q, q + 1 with
        // q = 32h + 8(p/2) + 4g + 2(p%2)
        __bf16* ds = reinterpret_cast<__bf16*>(lds + L::K1_DS) + kvl * L::QS;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int pi = 0; pi < 8; ++pi)
            *(uint32_t*)(ds + 32 * h + 8 * (pi >> 1) + 4 * g + 2 * (pi & 1)) = dd[h][pi];
      }
    };

    // dQ of a query step of a one-key-tile sample: dQ^T = scale K^T dS^T over the item's keys,
    // both operands read with transposing LDS reads in natural key order (k = 8g + j <-> key
    // 16 kc + 8g + j).  Wave w computes output blocks b = w, w + NW, ... of (query half b % 2,
    // head-dim block b / 2) and stores its rows directly.
    auto dq_step = [&](int qs) {
      if constexpr (L::K1) {
        constexpr int NBLK = 2 * (D / 32), BPW = NBLK / NW;
        static_assert(NBLK % NW == 0, "dQ blocks per wave");
        const __bf16* kr1 = reinterpret_cast<const __bf16*>(lds + L::K1_KR);
        const __bf16* ds1 = reinterpret_cast<const __bf16*>(lds + L::K1_DS);
        const int tr_k = (8 * (lane >> 5) + ((lane & 15) >> 2)) * RS + 16 * ((lane >> 4) & 1) +
                         4 * (lane & 3);
        const int tr_d = (8 * (lane >> 5) + ((lane & 15) >> 2)) * L::QS +
                         16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const rsrc_t rdq = make_rsrc((__bf16*)p.dq + ((int64_t)qo * H + h) * D, q_bytes);
#pragma unroll
        for (int bi = 0; bi < BPW; ++bi) {
          const int b = wave + bi * NW, half = b & 1, db = b >> 1;
          f32x16 qa;
#pragma unroll
          for (int i = 0; i < 16; ++i) qa[i] = 0.f;
#pragma unroll
          for (int kc = 0; kc < BNK / 16; ++kc) {
            const __bf16* pa = kr1 + tr_k + 16 * kc * RS + db * 32;
            const __bf16* pb = ds1 + tr_d + 16 * kc * L::QS + 32 * half;
            const u32x2 a0 = lds_read_tr16(pa), a1 = lds_read_tr16(pa + 4 * RS);
            const u32x2 b0 = lds_read_tr16(pb), b1 = lds_read_tr16(pb + 4 * L::QS);
            qa = mfma_bf16(as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]}),
                           as_bf16x8(u32x4{b0[0], b0[1], b1[0], b1[1]}), qa);
          }
          // lane (query 32 half + l32, g) holds head dims db*32 + 8 jq + 4g + 0..3
          const uint32_t row = (uint32_t)(qs * STEP + 32 * half + l32) * row_bytes;
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const float sw = p.scale * wn;
            const u32x2 v = {pack2bf(qa[4 * jq] * sw, qa[4 * jq + 1] * sw),
                             pack2bf(qa[4 * jq + 2] * sw, qa[4 * jq + 3] * sw)};
            st8(v, rdq, row + 2u * (uint32_t)(db * 32 + 8 * jq + 4 * g));
          }
        }
      }
    };

    if (nsteps > 0) load_step(qs_first);
    if (short_item && wave == 0) pipe.resolve(lane);
    if (nsteps > 0) store_step(0, qs_first, true);
    // the key fragments (loaded with the first tiles) are complete before the query loop
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (L::K1 && one_k) {
      // the item's K rows for the dQ steps: lane (key, g) holds head dims 16 ks + 8g + 0..7
      __bf16* kr1 = reinterpret_cast<__bf16*>(lds + L::K1_KR) + kvl * RS;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) *(bf16x8*)(kr1 + 16 * ks + 8 * g) = kf[ks];
    }
    __syncthreads();
    const int claim_it = short_item ? -1 : nsteps - CLAIM_AHEAD;
    const int resolve_it = short_item ? -1 : nsteps - 2;
    for (int it = 0; it + 1 < nsteps; ++it) {
      if (it == claim_it && wave == 0) pipe.claim(lane);
      if (it == resolve_it && wave == 0) pipe.resolve(lane);
      load_step(qs_first + it + 1);
      compute_step(it, qs_first + it);
      if (one_k) {
        __syncthreads();
        dq_step(qs_first + it);
      }
      store_step((it + 1) & 1, qs_first + it + 1, true);
      __syncthreads();
    }
    if (nsteps > 0) compute_step(nsteps - 1, qs_end - 1);
    if (one_k && nsteps > 0) {
      __syncthreads();
      dq_step(qs_end - 1);
    }
    // publish the next descriptor before the epilogue's stores (see the forward kernel)
    if (wave == 0) pipe.publish(s_desc[buf ^ 1], lane);

    // epilogue: this lane's key row of dK (x scale) and dV; keys past the sample are dropped
    const rsrc_t rdk = make_rsrc((__bf16*)p.dk + ((int64_t)ko * H + h) * D, kv_bytes);
    const rsrc_t rdv = make_rsrc((__bf16*)p.dv + ((int64_t)ko * H + h) * D, kv_bytes);
    // through the stage that the last query step left free (rows of this wave only)
    unsigned char* ost = lds + (nsteps & 1) * L::STAGE + wave * 2 * out_stage_bytes<D>();
    store_rows_via_lds<D>(dk, p.scale * wn, reinterpret_cast<__bf16*>(ost), rdk,
                          (uint32_t)jw0 * row_bytes, row_bytes, lane);
    store_rows_via_lds<D>(dv, wn, reinterpret_cast<__bf16*>(ost + out_stage_bytes<D>()), rdv,
                          (uint32_t)jw0 * row_bytes, row_bytes, lane);
    __syncthreads();
  }
}

// ================================================= query-stationary dQ
template <int D, int NW, int BIAS, bool SPLIT = false>
struct QLds {
  static constexpr int BM = 32 * NW;
  static constexpr int RS = tile_row_stride<D>();
  static constexpr int KR = 0;                            // K rows [STEP][RS]
  static constexpr int VR = KR + STEP * RS * 2;           // V rows
  // the K^T operand is read from the K rows with transposing LDS reads
  static constexpr int BO = VR + STEP * RS * 2;
  static constexpr int RP = diag_stride(BM + STEP + 4);
  static constexpr int BS = STEP + 8;                     // dense tile [BM][BS] bf16 (query-major)
  static constexpr int BIAS_BYTES =
      BIAS == B_RELPOS ? 4 * RP * 4 : (BIAS == B_DENSE ? BM * BS * 2 : 0);
  // a stage also holds the epilogue's dQ rows (one staging area per wave)
  static constexpr int STAGE = align16(BO + BIAS_BYTES) > NW * out_stage_bytes<D>()
                                   ? align16(BO + BIAS_BYTES) : NW * out_stage_bytes<D>();
  // single pass for a sample with one query tile (built for 64-row tiles): the item's Q and dO
  // rows and each step's P and dS [query][key], from which wave w computes the step's dV, dK
  // rows of keys 32w .. 32w + 31
  static constexpr bool Q1 = NW == 2;
  static constexpr int PS = STEP + 8;                     // P / dS tile row stride (bf16)
  static constexpr int Q1_QR = 2 * STAGE;
  static constexpr int Q1_DR = Q1_QR + BM * RS * 2;
  static constexpr int Q1_P = Q1_DR + BM * RS * 2;
  static constexpr int Q1_DS = Q1_P + BM * PS * 2;
  // SPLIT (two more waves compute the dK / dV of the previous step while the query waves work
  // on the current one): P / dS double-buffered, PDS bytes apart
  static constexpr int PDS = SPLIT ? 2 * BM * PS * 2 : 0;
  static constexpr int TOTAL = 2 * STAGE + (Q1 ? 2 * BM * RS * 2 + 2 * BM * PS * 2 + PDS : 0);
  static_assert(!SPLIT || (Q1 && TOTAL <= 160 * 1024 - 512), "LDS of the split pass");
  // bias gradient of a relative-position table of at most DB_NB buckets: per-lane bucket sums,
  // [DB_NB][64] floats per wave (bucket-major, so the 64 lanes hit 64 banks), in place of the
  // single-pass class's area, which that pass does not use
  static constexpr int DBA = 2 * STAGE;
  // and, after them, each step's bucket of every diagonal as a byte table (four copies shifted
  // by one byte, like the bias values: a run of 4 keys is one aligned 4-byte read), one table
  // per stage parity
  static constexpr int RPB = (BM + STEP + 4 + 3) / 4 * 4;
  static constexpr int BKT = DBA + NW * DB_NB * 64 * 4;
  static constexpr int TOTAL_DB = BIAS == B_RELPOS ? (TOTAL > BKT + 2 * 4 * RPB
                                                          ? TOTAL : BKT + 2 * 4 * RPB)
                                                   : TOTAL;
  static_assert(TOTAL_DB <= 160 * 1024, "LDS of the bias-gradient pass");
};

// The query-stationary pass over the q-stationary list (HOME as for kv_pass).  DB: also the
// bias gradient, from each pair's dS as it is formed (dense: dS stored in the bias layout;
// relative-position table: per-lane running sums by bucket, flushed on a change of bucket into
// the lane's own slots, in LDS for at most DB_NB buckets and else (DBG) in its partial row in
// memory; later kernels reduce the rows in a fixed order).  DB runs without the single-pass
// classes.
//
// SPLIT: a workgroup of 4 waves for 64-row tiles.  Waves 0, 1 own the query rows (S, dP, dS, dQ
// as above); waves 2, 3 stage the K / V tiles and, for a one-query-tile sample, compute the dK,
// dV rows of the previous key step from its P / dS while the query waves work on the current
// one, so every SIMD has a wave.
template <int D, int NW, int MODE, int BIAS, bool HOME, bool DB, bool WIN, bool FP8,
          bool SPLIT = false, bool DBG = false>
__device__ __forceinline__ void q_pass(const BwdParams& p) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int QW = SPLIT ? 2 : NW;                 // waves that own query rows
  static_assert(!SPLIT || (NW == 4 && !DB && !FP8 && BIAS != B_DENSE), "split pass");
  using L = QLds<D, QW, BIAS, SPLIT>;
  constexpr int BM = L::BM, RS = L::RS;
  constexpr int NT = SPLIT ? 128 : NW * 64;          // threads that stage K / V (and the bias)
  __shared__ int s_desc[2][IF_WORDS];

  if (p.hdr->status != JFA_OK) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool qrole = !SPLIT || wave < QW;             // owns query rows
  const bool srole = !SPLIT || wave >= QW;            // stages the tiles
  const int tid = SPLIT ? (int)threadIdx.x - 128 : (int)threadIdx.x;   // staging thread index
  const int kvw = SPLIT ? wave - QW : wave;           // key block of the dK / dV step
  const int g = lane >> 5, l32 = lane & 31;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr->counts[2] * H;
  // this lane's element of a transposing read (see the key-stationary kernel)
  const int tr_lane = (4 * (lane >> 5) + ((lane & 15) >> 2)) * L::RS + 16 * ((lane >> 4) & 1) +
                      4 * (lane & 3);
  const float c_log = MODE == MODE_SOFTMAX ? p.scale * LOG2E : p.scale;
  const float inv_scale = 1.0f / p.scale;
  const uint32_t row_bytes = (uint32_t)H * D * 2;          // bf16 rows (outputs, bf16 inputs)
  constexpr int ES = FP8 ? 1 : 2;                           // bytes per input element
  const uint32_t in_row = (uint32_t)H * D * ES;             // input row stride
  const uint32_t sc_row = (uint32_t)H * (D / 32);           // MXFP8 scale row stride

  // bf16 tiles are staged row-major, consecutive lanes along a row (full cache lines per load)
  std::conditional_t<FP8, Fp8Tile<D, NT>, RowTile<D, NT>> tk;
  std::conditional_t<FP8, Fp8RowTile<D, NT>, RowTile<D, NT>> tv;
  float rpv = 0.f;
  int rpk = 0;                      // its bucket (the bias gradient's byte table)
  constexpr int NDB = BIAS == B_DENSE ? BM * (STEP / 8) / NT : 1;
  BiasRaw dbr[NDB];                 // dense bias chunks (8 keys of one query) of the next step
  constexpr bool BIAS_RAW = !(D == 128 && (DB || WIN));

  ItemPipeT<HOME> pipe{p.xtk_q, p.bq, (int)n_items, H};
  if (wave == 0) pipe.start(s_desc[0], lane);
  // relative-position gradient in LDS: this lane's slot of bucket k is dbl[64 k]
  constexpr bool DBL = DB && BIAS == B_RELPOS && !DBG;
  float* dbl = reinterpret_cast<float*>(lds + L::DBA) + wave * DB_NB * 64 + lane;
  if constexpr (DBL)
    for (int k = 0; k < p.num_buckets; ++k) dbl[64 * k] = 0.f;
  __syncthreads();
  for (int buf = 0;; buf ^= 1) {
    const int* dsc = s_desc[buf];
    const int w = item_field(dsc, IF_W);
    if (w >= n_items) break;
    const int h = w % H;
    // key steps [kb0, kb0 + steps) of query tile t
    const int t = item_field(dsc, IF_X), kb0 = WIN ? item_field(dsc, IF_Y) : 0;
    const int steps = item_field(dsc, IF_Z) - kb0;
    // the next item: a short item takes its ticket now and reads its record right after this
    // item's first loads; a longer one claims it CLAIM_AHEAD steps before its end
    const bool short_item = steps <= CLAIM_AHEAD;
    if (short_item && wave == 0) pipe.claim(lane);
    const int qo = item_field(dsc, IF_QO), n = item_field(dsc, IF_N);
    const int ko = item_field(dsc, IF_KO), m = item_field(dsc, IF_M);
    const int64_t boff = item_boff(dsc);
    // single-pass class (the scheduler's test): the sample's queries fit one tile
    const bool one_q = L::Q1 && (p.fuse & 1) && n > 0 && n <= BM;
    const int delta = m - n;
    const float wn = (MODE != MODE_SOFTMAX && p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    // the weight 1 / kv_len per pair (the bias gradient) or on the item's outputs as a whole
    const float wpair = DB ? wn : 1.0f, wout = DB ? 1.0f : wn;
    const int q0 = t * BM, qw0 = q0 + wave * 32;
    const int qil = wave * 32 + l32, qi = q0 + qil;
    // keys [wave_kbeg, wave_kend) hold every pair this wave's rows can see
    const int W = WIN ? p.window : 0;
    int wave_kend = m, wave_kbeg = 0;
    if (p.causal) wave_kend = max(0, min(m, min(n, qw0 + 32) + delta));
    else if (WIN) wave_kend = max(0, min(m, min(n, qw0 + 32) - 1 + delta + W));
    if (WIN) wave_kbeg = max(0, qw0 + delta - W + 1);
    const bool wave_rows = qw0 < n;

    const uint32_t kv_bytes = m > 0 ? ((uint32_t)(m - 1) * H + 1) * D * 2 : 0;
    const uint32_t q_bytes = n > 0 ? ((uint32_t)(n - 1) * H + 1) * D * 2 : 0;
    const uint32_t kv_in = m > 0 ? ((uint32_t)(m - 1) * H + 1) * D * ES : 0;
    const uint32_t q_in = n > 0 ? ((uint32_t)(n - 1) * H + 1) * D * ES : 0;
    const rsrc_t rk = make_rsrc((const uint8_t*)p.k + ((int64_t)ko * H + h) * D * ES, kv_in);
    const rsrc_t rv = make_rsrc((const uint8_t*)p.v + ((int64_t)ko * H + h) * D * ES, kv_in);
    const rsrc_t rq = make_rsrc((const uint8_t*)p.q + ((int64_t)qo * H + h) * D * ES, q_in);
    const rsrc_t rdo = make_rsrc((const uint8_t*)p.dout + ((int64_t)qo * H + h) * D * ES, q_in);
    rsrc_t rks = rk, rvs = rv, rqs = rq, rdos = rdo;
    if constexpr (FP8) {
      const uint32_t kv_s = m > 0 ? ((uint32_t)(m - 1) * H + 1) * (D / 32) : 0;
      const uint32_t q_s = n > 0 ? ((uint32_t)(n - 1) * H + 1) * (D / 32) : 0;
      rks = make_rsrc(p.k_sc + ((int64_t)ko * H + h) * (D / 32), kv_s);
      rvs = make_rsrc(p.v_sc + ((int64_t)ko * H + h) * (D / 32), kv_s);
      rqs = make_rsrc(p.q_sc + ((int64_t)qo * H + h) * (D / 32), q_s);
      rdos = make_rsrc(p.do_sc + ((int64_t)qo * H + h) * (D / 32), q_s);
    }
    rsrc_t rb = rq;
    if constexpr (BIAS == B_DENSE)
      rb = make_rsrc((const __bf16*)p.bias + (int64_t)H * boff + (int64_t)h * n * m,
                     (uint32_t)n * (uint32_t)m * 2u);
    // dense bias gradient: the item's [n][m] block, and this lane's row in it (a row past the
    // sample's end lies past the block, where stores are dropped)
    const uint32_t db_size = (uint32_t)n * (uint32_t)m * 2u;
    const uint32_t db_row = (uint32_t)qi * (uint32_t)m * 2u;
    rsrc_t rdb = rq;
    if constexpr (DB && BIAS == B_DENSE)
      rdb = make_rsrc((const __bf16*)p.dbias + (int64_t)H * boff + (int64_t)h * n * m, db_size);

    bf16x8 qf[D / 16], dof[D / 16];
    if (qrole) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        qf[ks] = load_frag8<D, FP8>(rq, rqs, (uint32_t)qi, in_row, sc_row, 16 * ks + 8 * g);
        dof[ks] = load_frag8<D, FP8>(rdo, rdos, (uint32_t)qi, in_row, sc_row, 16 * ks + 8 * g);
      }
    }
    float lse2 = 0.f, dlt = 0.f;
    // bias gradient, relative-position table: the bucket being summed and its running sum
    // (bucket 0 with a zero sum to begin with: flushing it adds nothing)
    int db_k = 0;
    float db_sum = 0.f;
    auto db_flush = [&]() {
      if constexpr (DB && BIAS == B_RELPOS) {
        if constexpr (DBL) {
          // an LDS add with no result (ds_add_f32): no wait inside the loop; the slot is this
          // lane's own and a wave's LDS operations apply in program order, so the sum's order
          // is fixed
          __hip_atomic_fetch_add(dbl + 64 * db_k, db_sum, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        } else if (qi < n) {
          // the row's own partial row in memory (a row past the sample's end belongs to the
          // next one, and has nothing to add)
          float* pr = p.dbias_part + (((int64_t)(qo + qi) * H + h) * 2 + g) * p.num_buckets;
          pr[db_k] += db_sum;
        }
      }
    };
    if constexpr (MODE == MODE_SOFTMAX) {
      if (qrole && qi < n) {
        // a row without a visible key has lse = -inf and all its pairs at the -inf sentinel:
        // any finite value keeps exp2(-inf - lse2) = 0
        const float l = p.lse[(int64_t)h * p.total_q + qo + qi];
        lse2 = l == NEG_INF ? 0.f : l * LOG2E;
        dlt = p.delta[(int64_t)h * p.total_q + qo + qi];
      }
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    // chunk i of this thread for key step j0: byte offset and valid element count
    const uint32_t bias_bytes = (uint32_t)n * (uint32_t)m * 2u;
    auto dense_at = [&](int i, int j0, uint32_t& off, int& valid) {
      const int id = tid + i * NT;
      const int qq = q0 + id / (STEP / 8), k0 = j0 + 8 * (id % (STEP / 8));
      valid = qq < n ? min(8, m - k0) : 0;
      off = ((uint32_t)qq * (uint32_t)m + (uint32_t)k0) * 2u;
    };
    auto load_step = [&](int kt) {
      const int j0 = kt * STEP;
      if constexpr (BIAS == B_RELPOS) {
        if (tid < BM + STEP - 1) {
          const int dist = q0 + delta - j0 + BM - 1 - tid;
          rpk = relpos_bucket(dist, p.num_buckets);
          rpv = ((const float*)p.bias)[(int64_t)h * p.num_buckets + rpk];
        }
      }
      if constexpr (FP8) {
        tk.load(rk, rks, in_row, sc_row, j0);
        tv.load(rv, rvs, in_row, sc_row, j0);
      } else {
        tk.load(rk, row_bytes, j0);
        tv.load(rv, row_bytes, j0);
      }
      if constexpr (BIAS == B_DENSE) {
        // [BM][STEP] block as chunks of 8 keys, consecutive lanes along a row
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
          uint32_t off;
          int valid;
          dense_at(i, j0, off, valid);
          // (the bias-gradient and window kernels at d = 128 have no registers for the raw
          // loads: they assemble the chunk at once)
          if constexpr (!BIAS_RAW) dbr[i].x = bias_chunk(rb, off, valid, bias_bytes);
          else dbr[i] = bias_chunk_load(rb, off, valid, bias_bytes);
        }
      }
    };
    auto store_step = [&](int st, int kt) {
      unsigned char* base = lds + st * L::STAGE;
      const int j0 = kt * STEP;
      tk.store(reinterpret_cast<__bf16*>(base + L::KR));
      tv.store(reinterpret_cast<__bf16*>(base + L::VR));
      if constexpr (BIAS == B_RELPOS) {
        if (tid < BM + STEP - 1) {
          store_diag<L::RP>(reinterpret_cast<float*>(base + L::BO), tid, rpv * inv_scale);
          if constexpr (DBL) {
            unsigned char* bt = lds + L::BKT + st * 4 * L::RPB;
#pragma unroll
            for (int k = 0; k < 4; ++k) bt[k * L::RPB + tid + k] = (unsigned char)rpk;
          }
        }
      } else if constexpr (BIAS == B_DENSE) {
        __bf16* bt = reinterpret_cast<__bf16*>(base + L::BO);
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
          const int id = tid + i * NT;
          uint32_t off;
          int valid;
          dense_at(i, j0, off, valid);
          *(u32x4*)(bt + (id / (STEP / 8)) * L::BS + 8 * (id % (STEP / 8))) =
              BIAS_RAW ? bias_chunk_finish(dbr[i], off, valid, bias_bytes) : dbr[i].x;
        }
      }
    };

    auto compute_step = [&](int it) {
      const int j0 = (kb0 + it) * STEP;
      const unsigned char* sb = lds + (it & 1) * L::STAGE;
      if (!wave_rows || j0 >= wave_kend || (WIN && j0 + STEP <= wave_kbeg)) {
        if (L::Q1 && one_q) {     // this wave's queries contribute nothing to this step's dK, dV
          uint32_t* pq = reinterpret_cast<uint32_t*>(
              reinterpret_cast<__bf16*>(lds + L::Q1_P + (it & 1) * L::PDS) + qil * L::PS);
          uint32_t* dq = reinterpret_cast<uint32_t*>(
              reinterpret_cast<__bf16*>(lds + L::Q1_DS + (it & 1) * L::PDS) + qil * L::PS);
#pragma unroll
          for (int i = 0; i < STEP / 2 / 2; ++i) {
            pq[2 * i + g] = 0u;
            dq[2 * i + g] = 0u;
          }
        }
        return;
      }
      const __bf16* kr = reinterpret_cast<const __bf16*>(sb + L::KR);
      const __bf16* vr = reinterpret_cast<const __bf16*>(sb + L::VR);
      // element (blk, i): key j0 + blk*32 + 8(i/4) + 4g + i%4, query qi
      // the bias gradient's buckets of this lane's pairs: byte e of bkw[blk][qd] is the bucket
      // of element (blk, 4 qd + e)
      uint32_t bkw[DBL ? 2 : 1][4];
      if constexpr (DBL) {
        const unsigned char* bt = lds + L::BKT + (it & 1) * 4 * L::RPB;
        const int k = (1 + qil) & 3;
        const unsigned char* src = bt + k * L::RPB + k + BM - 1 - qil + 4 * g;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            bkw[blk][qd] = *(const uint32_t*)(src + blk * 32 + 8 * qd);
      }
      f32x16 sacc[2], pacc[2];
      if constexpr (BIAS == B_RELPOS) {
        const float* rp = reinterpret_cast<const float*>(sb + L::BO);
        const int k = (1 + qil) & 3;
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
        const __bf16* bt = reinterpret_cast<const __bf16*>(sb + L::BO) + qil * L::BS + 4 * g;
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
      // softmax: dP starts at -delta, so that dS = P dP with no subtraction per pair
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) pacc[blk][i] = MODE == MODE_SOFTMAX ? -dlt : 0.f;
      // (GDPA without the bias gradient needs no mask at the sample's ends, as in the dK/dV
      // pass; the bias gradient keeps it, since its relative-position sums test each pair's
      // visibility)
      const bool need_mask = ((MODE == MODE_SOFTMAX || DB) && (j0 + STEP > m || qw0 + 32 > n)) ||
                             (p.causal && j0 + STEP - 1 > qw0 + delta) ||
                             (WIN && (j0 <= qw0 + 31 + delta - W ||
                                      (!p.causal && j0 + STEP - 1 >= qw0 + delta + W)));
      if (need_mask) {
        // keys [kbeg, kend) are visible to query qi: offsets [lo, lim) of this lane's elements;
        // the others start at -inf, so that P = 0 and dS = 0 with no per-element test later
        int kend = qi < n ? (p.causal ? min(m, qi + delta + 1) : m) : 0;
        int lo = 0;
        if constexpr (WIN) {
          if (qi < n && !p.causal) kend = min(m, qi + delta + W);
          lo = qi + delta - W + 1 - j0 - 4 * g;
        }
        const int lim = kend - j0 - 4 * g;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = blk * 32 + 8 * (i >> 2) + (i & 3);
            if (off >= lim || (WIN && off < lo)) sacc[blk][i] = NEG_INF;
          }
      }
      uint32_t dd[2][8], pq2[2][8];
      // B(blk) pair pi: dS and P of elements 2 pi, 2 pi + 1 of block blk
      // The VALU work of one pair runs in two stages one MFMA apart: the front (exp or the
      // activation) and the back (times dP, the packing, the bias gradient), so that no
      // dependent chain waits inside one MFMA slot.  Front results are kept by pair parity.
      float fr_p[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, fr_d[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
      auto b_front = [&](int blk, int pi) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ii = 2 * pi + e;
          if constexpr (MODE == MODE_SOFTMAX) {
            fr_p[pi & 1][e] = fast_exp2(fmaf(sacc[blk][ii], c_log, -lse2));
          } else {
            // masked pairs hold -inf: clamped to -1e30, the activation and its derivative are
            // exactly zero and a NaN logit still propagates
            float x = sacc[blk][ii] * c_log;
            x = act_clamp(x);
            act_pair<MODE>(x, fr_p[pi & 1][e], fr_d[pi & 1][e]);
          }
        }
      };
      auto b_back = [&](int blk, int pi) {
        float d2[2], p2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ii = 2 * pi + e;
          if constexpr (MODE == MODE_SOFTMAX) {
            const float pr = fr_p[pi & 1][e];
            d2[e] = pr * pacc[blk][ii];
            p2[e] = pr;
          } else {
            d2[e] = fr_d[pi & 1][e] * pacc[blk][ii] * wpair;
            p2[e] = fr_p[pi & 1][e] * wpair;
          }
          if constexpr (DB) {
            const int j = j0 + blk * 32 + 8 * (ii >> 2) + 4 * g + (ii & 3);
            if constexpr (BIAS == B_DENSE) {
              // masked pairs store their zero; a key past the sample's end would wrap into the
              // next row and is sent past the block instead (a dropped store, no branch)
              st2(__builtin_bit_cast(uint16_t, (__bf16)d2[e]), rdb,
                  j < m ? db_row + 2u * (uint32_t)j : db_size);
            } else if constexpr (BIAS == B_RELPOS) {
              // a pair is visible iff its logit is not the -inf sentinel (the bias is finite),
              // which is exactly qi < n, j < m and (causal) j <= qi + delta.  A pair that is not
              // adds zero to the current bucket (selects, not a branch), so the only branch is
              // the flush on a change of bucket.
              const bool vis = sacc[blk][ii] != NEG_INF;
              int kb;
              if constexpr (DBL)
                kb = (int)((bkw[blk][ii >> 2] >> (8 * (ii & 3))) & 255u);
              else
                kb = relpos_bucket(qi + delta - j, p.num_buckets);
              const int k = vis ? kb : db_k;
              const float dv = vis ? d2[e] : 0.f;
              const bool chg = k != db_k;
              // the new sum as a select ahead of the flush (the empty asm keeps the compiler from
              // moving the add into an else branch around it)
              float nsum = chg ? dv : db_sum + dv;
              asm volatile("" : "+v"(nsum));
              if (chg) db_flush();
              db_sum = nsum;
              db_k = k;
            }
          }
        }
        dd[blk][pi] = pack2bf(d2[0], d2[1]);
        pq2[blk][pi] = pack2bf(p2[0], p2[1]);
      };

      // One key step, software-pipelined by hand, as a stream of MFMAs:
      //   A(blk), blk = 0, 1: S^T and dP^T of keys 32 blk .. 32 blk + 31   (NA MFMAs each)
      //   C: dQ^T += K^T dS^T, key chunk c = 0..3 (chunks 0, 1 use block 0, chunks 2, 3 block 1)
      // in the order A(0) A(1) C.  Each MFMA's LDS operand is read PF MFMAs ahead; the VALU work
      // B(0) (dS, P of block 0) runs under A(1) and B(1) under the first half of C, so the matrix
      // cores keep busy in this one-wave-per-SIMD kernel.
      constexpr int NA = D / 8;          // 16 at d = 128, 8 at d = 64
      constexpr int NCB = D / 32;        // dQ MFMAs per key chunk
      constexpr int NS = 2 * NA + 4 * NCB;
      constexpr int PF = 6;
      constexpr int RING = 8;
      auto opnd = [&](int st) -> u32x4 {
        if (st < 2 * NA) {
          const int blk = st / NA, jj = st % NA, ks = jj >> 1;
          const __bf16* base = (jj & 1) ? vr : kr;
          return *(const u32x4*)(base + (blk * 32 + l32) * RS + 16 * ks + 8 * g);
        }
        // K^T rows = head dims, k = 8g + j <-> key 16c + 8(j/4) + 4g + j%4: two column strips
        // of 4 keys of the K rows
        const int c = (st - 2 * NA) / NCB, db = (st - 2 * NA) % NCB;
        const __bf16* pk = kr + tr_lane + 16 * c * RS + db * 32;
        const u32x2 lo = lds_read_tr16(pk), hi = lds_read_tr16(pk + 8 * RS);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      auto mfma_s = [&](int st, u32x4 o) {
        const bf16x8 a = as_bf16x8(o);
        if (st < 2 * NA) {
          const int blk = st / NA, jj = st % NA, ks = jj >> 1;
          if (jj & 1) pacc[blk] = mfma_bf16(a, dof[ks], pacc[blk]);
          else sacc[blk] = mfma_bf16(a, qf[ks], sacc[blk]);
          return;
        }
        // chunk c covers keys 16c + 8(e/4) + 4g + e%4: elements 8(c%2) .. 8(c%2) + 7 of block c/2
        const int c = (st - 2 * NA) / NCB, db = (st - 2 * NA) % NCB;
        const u32x4 dw = {dd[c >> 1][4 * (c & 1)], dd[c >> 1][4 * (c & 1) + 1],
                          dd[c >> 1][4 * (c & 1) + 2], dd[c >> 1][4 * (c & 1) + 3]};
        acc[db] = mfma_bf16(a, as_bf16x8(dw), acc[db]);
      };
      u32x4 ring[RING];
      static_for<0, PF>([&](auto sc) { ring[decltype(sc)::value] = opnd(decltype(sc)::value); });
      static_for<0, NS>([&](auto sc) {
        constexpr int st = decltype(sc)::value;
        if constexpr (st + PF < NS) ring[(st + PF) % RING] = opnd(st + PF);
        mfma_s(st, ring[st % RING]);
        // B(0) under A(1): the front of pair k in slot NA + ceil(k NA / 8), its back one slot
        // later.  B(1) under C: the front of pair k in slot 2 NA + floor(k NA / 16), its back
        // one slot later, so pairs 0..3 (dS of key chunk 2) are done before chunk 2 and
        // pairs 4..7 before chunk 3.  In each slot the backs come before the fronts.
        if constexpr (st >= NA + 1 && st <= 2 * NA) {
          static_for<((st - 1 - NA) * 8 + NA - 1) / NA, ((st - NA) * 8 + NA - 1) / NA>(
              [&](auto pc) { b_back(0, decltype(pc)::value); });
        }
        if constexpr (st >= 2 * NA + 1 && st <= 2 * NA + NA / 2) {
          static_for<(st - 1 - 2 * NA) * 16 / NA, (st - 2 * NA) * 16 / NA>(
              [&](auto pc) { b_back(1, decltype(pc)::value); });
        }
        if constexpr (st >= NA && st < 2 * NA) {
          static_for<((st - NA) * 8 + NA - 1) / NA, ((st - NA + 1) * 8 + NA - 1) / NA>(
              [&](auto pc) { b_front(0, decltype(pc)::value); });
        }
        if constexpr (st >= 2 * NA && st < 2 * NA + NA / 2) {
          static_for<(st - 2 * NA) * 16 / NA, (st - 2 * NA + 1) * 16 / NA>(
              [&](auto pc) { b_front(1, decltype(pc)::value); });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (L::Q1 && one_q) {
        // P and dS [query][key] of this step: pair p of block blk holds keys k, k + 1 with
        // k = 32 blk + 8(p/2) + 4g + 2(p%2)
        __bf16* pr = reinterpret_cast<__bf16*>(lds + L::Q1_P + (it & 1) * L::PDS) + qil * L::PS;
        __bf16* dr = reinterpret_cast<__bf16*>(lds + L::Q1_DS + (it & 1) * L::PDS) + qil * L::PS;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int pi = 0; pi < 8; ++pi) {
            const int k = 32 * blk + 8 * (pi >> 1) + 4 * g + 2 * (pi & 1);
            *(uint32_t*)(pr + k) = pq2[blk][pi];
            *(uint32_t*)(dr + k) = dd[blk][pi];
          }
      }
    };

    // dK, dV of a key step of a one-query-tile sample: dV^T = dO^T P and dK^T = scale Q^T dS
    // over the tile's queries, operands read with transposing LDS reads in natural query order
    // (k = 8g + j <-> query 16 kc + 8g + j).  Key wave w owns keys 32w .. 32w + 31 of the step
    // and writes their rows through its staging area in the step's (now idle) LDS stage or
    // (SPLIT, where no stage is idle) straight from the accumulators, 4 dims per lane and store.
    auto dkdv_step = [&](int kt) {
      if constexpr (L::Q1) {
        const __bf16* qr1 = reinterpret_cast<const __bf16*>(lds + L::Q1_QR);
        const __bf16* dr1 = reinterpret_cast<const __bf16*>(lds + L::Q1_DR);
        const __bf16* pt = reinterpret_cast<const __bf16*>(lds + L::Q1_P + (kt & 1) * L::PDS);
        const __bf16* st = reinterpret_cast<const __bf16*>(lds + L::Q1_DS + (kt & 1) * L::PDS);
        const int trq = (8 * (lane >> 5) + ((lane & 15) >> 2)) * RS + 16 * ((lane >> 4) & 1) +
                        4 * (lane & 3);
        const int trp = (8 * (lane >> 5) + ((lane & 15) >> 2)) * L::PS +
                        16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        __bf16* ost = reinterpret_cast<__bf16*>(lds + (kt & 1) * L::STAGE +
                                                kvw * out_stage_bytes<D>());
        const uint32_t kv_bytes = m > 0 ? ((uint32_t)(m - 1) * H + 1) * D * 2 : 0;
        const uint32_t row0 = (uint32_t)((kb0 + kt) * STEP + 32 * kvw) * row_bytes;
#pragma unroll
        for (int which = 0; which < 2; ++which) {       // 0: dV = P^T dO, 1: dK = s dS^T Q
          const __bf16* xa = which ? qr1 : dr1;
          const __bf16* xb = which ? st : pt;
          f32x16 o[D / 32];
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
#pragma unroll
            for (int kc = 0; kc < BM / 16; ++kc) {
              const __bf16* pa = xa + trq + 16 * kc * RS + db * 32;
              const __bf16* pb = xb + trp + 16 * kc * L::PS + 32 * kvw;
              const u32x2 a0 = lds_read_tr16(pa), a1 = lds_read_tr16(pa + 4 * RS);
              const u32x2 b0 = lds_read_tr16(pb), b1 = lds_read_tr16(pb + 4 * L::PS);
              o[db] = mfma_bf16(as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]}),
                                as_bf16x8(u32x4{b0[0], b0[1], b1[0], b1[1]}), o[db]);
            }
          }
          const rsrc_t r = make_rsrc((__bf16*)(which ? p.dk : p.dv) + ((int64_t)ko * H + h) * D,
                                     kv_bytes);
          const float mul = which ? p.scale * wout : wout;
          if constexpr (SPLIT) {
            // lane (key l32, g) holds dims 32 db + 8 jq + 4 g + 0..3 of its key row; lanes l and
            // l + 32 (same key) trade halves so that each stores 8 consecutive dims (16 bytes):
            // g = 0 the group 32 db + 16 jp, g = 1 the group 32 db + 16 jp + 8.  Half as many
            // stores, so that waiting for the next tiles' loads never waits for these stores.
            const uint32_t row = row0 + (uint32_t)l32 * row_bytes;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
              for (int jp = 0; jp < 2; ++jp) {
                const int j0 = 8 * jp, j1 = 8 * jp + 4;       // o[] elements of jq = 2 jp, 2 jp + 1
                const u32x2 e = {pack2bf(o[db][j0] * mul, o[db][j0 + 1] * mul),
                                 pack2bf(o[db][j0 + 2] * mul, o[db][j0 + 3] * mul)};
                const u32x2 f = {pack2bf(o[db][j1] * mul, o[db][j1 + 1] * mul),
                                 pack2bf(o[db][j1 + 2] * mul, o[db][j1 + 3] * mul)};
                const u32x2 send = g ? e : f;                 // what the partner lane needs
                const u32x2 got = {(uint32_t)__shfl_xor((int)send[0], 32),
                                   (uint32_t)__shfl_xor((int)send[1], 32)};
                const u32x4 v = g ? u32x4{got[0], got[1], f[0], f[1]}
                                  : u32x4{e[0], e[1], got[0], got[1]};
                st16(v, r, row + 2u * (uint32_t)(db * 32 + 16 * jp + 8 * g));
              }
          } else {
            store_rows_via_lds<D>(o, mul, ost, r, row0, row_bytes, lane);
          }
        }
      }
    };

    if (steps > 0 && srole) load_step(kb0);
    if (short_item && wave == 0) pipe.resolve(lane);
    if (steps > 0 && srole) store_step(0, kb0);
    // the query fragments (loaded with the first tiles) are complete before the key loop
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (L::Q1 && one_q && qrole) {
      // the tile's Q and dO rows for the dK / dV steps: lane (query, g) holds head dims
      // 16 ks + 8g + 0..7
      __bf16* q1 = reinterpret_cast<__bf16*>(lds + L::Q1_QR) + qil * RS;
      __bf16* d1 = reinterpret_cast<__bf16*>(lds + L::Q1_DR) + qil * RS;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        *(bf16x8*)(q1 + 16 * ks + 8 * g) = qf[ks];
        *(bf16x8*)(d1 + 16 * ks + 8 * g) = dof[ks];
      }
    }
    __syncthreads();
    const int claim_it = short_item ? -1 : steps - CLAIM_AHEAD;
    const int resolve_it = short_item ? -1 : steps - 2;
    if constexpr (SPLIT) {
      // step it: the query waves compute it from LDS stage it&1 and write its P / dS; the key
      // waves stage step it + 1 into the other stage and turn the P / dS of step it - 1 into
      // dK, dV rows
      for (int it = 0; it < steps; ++it) {
        if (it == claim_it && wave == 0) pipe.claim(lane);
        if (it == resolve_it && wave == 0) pipe.resolve(lane);
        if (qrole) {
          compute_step(it);
        } else {
          if (it + 1 < steps) load_step(kb0 + it + 1);
          if (one_q && it > 0) dkdv_step(it - 1);
          if (it + 1 < steps) store_step((it + 1) & 1, kb0 + it + 1);
        }
        __syncthreads();
      }
      if (!qrole && one_q && steps > 0) dkdv_step(steps - 1);
    } else {
      for (int it = 0; it + 1 < steps; ++it) {
        if (it == claim_it && wave == 0) pipe.claim(lane);
        if (it == resolve_it && wave == 0) pipe.resolve(lane);
        load_step(kb0 + it + 1);
        compute_step(it);
        if (one_q) {
          __syncthreads();
          dkdv_step(it);
        }
        store_step((it + 1) & 1, kb0 + it + 1);
        __syncthreads();
      }
      if (steps > 0) compute_step(steps - 1);
      if (one_q && steps > 0) {
        __syncthreads();
        dkdv_step(steps - 1);
      }
    }
    // publish the next descriptor before the epilogue's stores (see the forward kernel)
    if (wave == 0) pipe.publish(s_desc[buf ^ 1], lane);

    db_flush();
    if constexpr (DBL) {
      // the row's two lane halves, summed in that order, into its partial row [H][buckets];
      // then the slots start again from zero
      __syncthreads();
      if (g == 0 && qi < n) {
        float* pr = p.dbias_part + ((int64_t)(qo + qi) * H + h) * p.num_buckets;
        for (int k = 0; k < p.num_buckets; ++k) pr[k] = dbl[64 * k] + dbl[64 * k + 32];
      }
      __syncthreads();
      for (int k = 0; k < p.num_buckets; ++k) dbl[64 * k] = 0.f;
    }
    if (qrole) {
      const rsrc_t rdq = make_rsrc((__bf16*)p.dq + ((int64_t)qo * H + h) * D, q_bytes);
      // through the stage that the last key step left free (rows of this wave only)
      __bf16* ost = reinterpret_cast<__bf16*>(lds + (steps & 1) * L::STAGE +
                                              wave * out_stage_bytes<D>());
      store_rows_via_lds<D>(acc, p.scale * wout, ost, rdq, (uint32_t)qw0 * row_bytes, row_bytes,
                            lane);
    }
    __syncthreads();
  }
}

template <int D, int NW, int MODE, int BIAS, bool WIN, bool FP8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_kv_kernel(BwdParams p) {
  kv_pass<D, NW, MODE, BIAS, true, WIN, FP8>(p);
}

template <int D, int NW, int MODE, int BIAS, bool WIN, bool FP8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_q_kernel(BwdParams p) {
  q_pass<D, NW, MODE, BIAS, true, false, WIN, FP8>(p);
}

// The query-stationary pass for 64-row tiles on 4 waves (see q_pass, SPLIT).
template <int D, int MODE, int BIAS, bool WIN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_q1_kernel(BwdParams p) {
  q_pass<D, 4, MODE, BIAS, true, false, WIN, false, true>(p);
}

// Both passes in one persistent launch (they are independent): every workgroup first works
// through the kv-stationary list, then takes q-stationary items by ticket, so the second list
// fills the first one's tail and the two passes share one kernel boundary.
template <int D, int NW, int MODE, int BIAS, bool WIN, bool FP8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_kvq_kernel(BwdParams p) {
  kv_pass<D, NW, MODE, BIAS, true, WIN, FP8>(p);
  __syncthreads();
  q_pass<D, NW, MODE, BIAS, false, false, WIN, FP8>(p);
}

// The query-stationary pass with the bias gradient (DB); the single-pass classes are off.
// DBG: a relative-position table wider than DB_NB buckets.
template <int D, int NW, int MODE, int BIAS, bool WIN, bool DBG>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_q_db_kernel(BwdParams p) {
  q_pass<D, NW, MODE, BIAS, true, true, WIN, false, false, DBG>(p);
}

// Zeroes `count` 16-bit elements of x; with count_from (a dense bias's block offsets), the
// count is H * count_from[B], known only on the device.  A bias gradient has to be zero on every
// pair the passes never visit.  Like every kernel of a call, it writes nothing when the
// scheduler found the offsets malformed (then count_from was never written).
__global__ __launch_bounds__(256) void zero_u16_kernel(const WsHeader* hdr, uint16_t* x,
                                                      int64_t count, const int64_t* count_from,
                                                      int B, int H) {
  if (hdr->status != JFA_OK) return;
  if (count_from) count = (int64_t)H * count_from[B];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256)
    x[i] = 0;
}

// Reduction of the partial rows part[rows][cols] (cols = H * halves * buckets) in a fixed order.
// Stage 1: chunk c (rows_per_chunk consecutive rows) into out1[c][cols]; thread x owns columns
// x, x + 256, ... and keeps 8 running sums (rows r with r % 8 = j), added in j order at the end.
__global__ __launch_bounds__(256) void dbias_rows_kernel(const WsHeader* hdr, const float* part,
                                                        float* out1, int64_t rows, int cols,
                                                        int64_t rows_per_chunk) {
  if (hdr->status != JFA_OK) return;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
  for (int c = threadIdx.x; c < cols; c += 256) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int64_t r = r0;
    for (; r + 8 <= r1; r += 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] += part[(r + j) * cols + c];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (r + j < r1) a[j] += part[(r + j) * cols + c];
    float acc = a[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) acc += a[j];
    out1[(int64_t)blockIdx.x * cols + c] = acc;
  }
}

// Stage 2: dbias[h][k] = sum over chunks and lane halves of out1; one workgroup per (h, k):
// thread x sums chunks x, x + 256, ... (halves in order within a chunk), then a fixed tree.
__global__ __launch_bounds__(256) void dbias_chunks_kernel(const WsHeader* hdr,
                                                          const float* out1, float* out,
                                                          int chunks, int H, int halves, int nb) {
  if (hdr->status != JFA_OK) return;
  __shared__ float red[256];
  const int h = blockIdx.x / nb, k = blockIdx.x % nb;
  const int cols = H * halves * nb;
  float acc = 0.f;
  for (int c = threadIdx.x; c < chunks; c += 256)
    for (int s = 0; s < halves; ++s) acc += out1[(int64_t)c * cols + (h * halves + s) * nb + k];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[(int64_t)h * nb + k] = red[0];
}

template <class K>
hipError_t launch_persistent(K kern, size_t lds, int threads, int64_t max_items, int cu,
                             const BwdParams& p, const char* tname, hipStream_t s) {
  hipError_t e = ensure_dyn_lds((const void*)kern, lds);
  if (e != hipSuccess) return e;
  int grid = resident_grid((const void*)kern, threads, lds, cu);
  if ((int64_t)grid > max_items) grid = (int)max(max_items, (int64_t)1);
  timing_begin(tname, s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, p);
  timing_end(s);
  return hipGetLastError();
}

template <int D, int NW, int MODE, int BIAS, bool WIN, bool FP8 = false>
hipError_t run_bk(const BwdParams& p, int64_t max_items, int cu, hipStream_t s) {
  return launch_persistent(bwd_kv_kernel<D, NW, MODE, BIAS, WIN, FP8>, KvLds<D, NW, BIAS>::TOTAL,
                           NW * 64, max_items, cu, p,
                           FP8 ? "jfa_bwd_dkdv_mxfp8" : "jfa_bwd_dkdv", s);
}
template <int D, int NW, int MODE, int BIAS, bool WIN, bool FP8 = false>
hipError_t run_bq(const BwdParams& p, int64_t max_items, int cu, hipStream_t s) {
  // 64-row tiles of bf16 inputs without a dense bias: the 4-wave variant
  if constexpr (NW == 2 && !FP8 && BIAS != B_DENSE)
    return launch_persistent(bwd_q1_kernel<D, MODE, BIAS, WIN>, QLds<D, 2, BIAS, true>::TOTAL,
                             256, max_items, cu, p, "jfa_bwd_dq", s);
  else
    return launch_persistent(bwd_q_kernel<D, NW, MODE, BIAS, WIN, FP8>, QLds<D, NW, BIAS>::TOTAL,
                             NW * 64, max_items, cu, p, FP8 ? "jfa_bwd_dq_mxfp8" : "jfa_bwd_dq",
                             s);
}

template <int D, int NW, int MODE, int BIAS, bool WIN, bool FP8 = false>
hipError_t run_bkq(const BwdParams& p, int64_t max_items, int cu, hipStream_t s) {
  constexpr size_t lds = KvLds<D, NW, BIAS>::TOTAL > QLds<D, NW, BIAS>::TOTAL
                             ? KvLds<D, NW, BIAS>::TOTAL : QLds<D, NW, BIAS>::TOTAL;
  return launch_persistent(bwd_kvq_kernel<D, NW, MODE, BIAS, WIN, FP8>, lds, NW * 64, max_items,
                           cu, p, FP8 ? "jfa_bwd_kvq_mxfp8" : "jfa_bwd_kvq", s);
}

template <int D, int NW, int MODE, int BIAS, bool WIN>
hipError_t run_bq_db(const BwdParams& p, int64_t max_items, int cu, hipStream_t s) {
  if constexpr (BIAS == B_RELPOS) {
    if (p.num_buckets > DB_NB)
      return launch_persistent(bwd_q_db_kernel<D, NW, MODE, BIAS, WIN, true>,
                               QLds<D, NW, BIAS>::TOTAL_DB, NW * 64, max_items, cu, p,
                               "jfa_dbias_dq", s);
  }
  return launch_persistent(bwd_q_db_kernel<D, NW, MODE, BIAS, WIN, false>,
                           QLds<D, NW, BIAS>::TOTAL_DB, NW * 64, max_items, cu, p, "jfa_dbias_dq",
                           s);
}

// Backward with the bias gradient: zero dbias (dense) or the partials (relative positions),
// the key-stationary pass, the query-stationary pass with DB, then (relative positions) the
// fixed-order reduction into dbias [H][num_buckets] (fp32).
template <int D, int MODE, int BIAS, bool WIN>
hipError_t run_bwd_db(const BwdParams& p, const TileCfg& tc, int64_t mq, int64_t mk, int cu,
                      hipStream_t s) {
  const unsigned zgrid = (unsigned)std::max(1, cu * 4);
  timing_begin("jfa_dbias_zero", s);
  if constexpr (BIAS == B_DENSE)
    hipLaunchKernelGGL(zero_u16_kernel, dim3(zgrid), dim3(256), 0, s, (const WsHeader*)p.hdr,
                       (uint16_t*)p.dbias,
                       (int64_t)0, p.bias_off, p.batch, p.H);
  else
    hipLaunchKernelGGL(zero_u16_kernel, dim3(zgrid), dim3(256), 0, s, (const WsHeader*)p.hdr,
                       (uint16_t*)p.dbias_part,
                       p.total_q * p.H * dbias_halves(p.num_buckets) * p.num_buckets * 2,
                       (const int64_t*)nullptr, 0, 0);
  timing_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = tc.bk_nw == 4 ? run_bk<D, 4, MODE, BIAS, WIN>(p, mk, cu, s) : run_bk<D, 2, MODE, BIAS, WIN>(p, mk, cu, s);
  if (e != hipSuccess) return e;
  e = tc.bq_nw == 4 ? run_bq_db<D, 4, MODE, BIAS, WIN>(p, mq, cu, s)
                    : run_bq_db<D, 2, MODE, BIAS, WIN>(p, mq, cu, s);
  if (e != hipSuccess) return e;
  if constexpr (BIAS == B_RELPOS) {
    const int halves = dbias_halves(p.num_buckets);
    const int cols = p.H * halves * p.num_buckets;
    const int chunks = dbias_chunks(p.H, p.num_buckets, p.total_q);
    const int64_t per = (p.total_q + chunks - 1) / chunks;
    timing_begin("jfa_dbias_reduce", s);
    hipLaunchKernelGGL(dbias_rows_kernel, dim3((unsigned)chunks), dim3(256), 0, s,
                       (const WsHeader*)p.hdr, (const float*)p.dbias_part, p.dbias_chunk, p.total_q, cols, per);
    hipLaunchKernelGGL(dbias_chunks_kernel, dim3((unsigned)(p.H * p.num_buckets)), dim3(256), 0,
                       s, (const WsHeader*)p.hdr, (const float*)p.dbias_chunk, (float*)p.dbias,
                       chunks, p.H, halves,
                       p.num_buckets);
    timing_end(s);
    e = hipGetLastError();
  }
  return e;
}

template <int D, int MODE, int BIAS, bool WIN, bool FP8>
hipError_t run_bwd_bias(const BwdParams& p, const TileCfg& tc, int64_t mq, int64_t mk, int cu,
                        hipStream_t s) {
  // one launch for both passes when their workgroups have the same shape
  if (tc.bk_nw == 4 && tc.bq_nw == 4)
    return run_bkq<D, 4, MODE, BIAS, WIN, FP8>(p, max(mq, mk), cu, s);
  hipError_t e = tc.bk_nw == 4 ? run_bk<D, 4, MODE, BIAS, WIN, FP8>(p, mk, cu, s)
                               : run_bk<D, 2, MODE, BIAS, WIN, FP8>(p, mk, cu, s);
  if (e != hipSuccess) return e;
  return tc.bq_nw == 4 ? run_bq<D, 4, MODE, BIAS, WIN, FP8>(p, mq, cu, s)
                       : run_bq<D, 2, MODE, BIAS, WIN, FP8>(p, mq, cu, s);
}

template <int D, int MODE, bool WIN, bool FP8>
hipError_t run_bwd(const BwdParams& p, const TileCfg& tc, int64_t mq, int64_t mk, int cu,
                   hipStream_t s) {
  // D (softmax) was computed by the scheduler launch
  switch (p.bias_kind) {
    case JFA_BIAS_RELPOS: return run_bwd_bias<D, MODE, B_RELPOS, WIN, FP8>(p, tc, mq, mk, cu, s);
    case JFA_BIAS_DENSE: return run_bwd_bias<D, MODE, B_DENSE, WIN, FP8>(p, tc, mq, mk, cu, s);
    default: return run_bwd_bias<D, MODE, B_NONE, WIN, FP8>(p, tc, mq, mk, cu, s);
  }
}

}  // namespace

// The launcher of one (head dim, mode, input format) triple, defined by the translation unit
// compiled for it.
template <>
hipError_t launch_bwd_dm<JFA_BWD_D, JFA_BWD_MODE, (JFA_BWD_FP8 != 0)>(
    const BwdParams& p, const TileCfg& tc, int64_t mq, int64_t mk, int cu, hipStream_t s,
    bool dbias) {
  constexpr int D = JFA_BWD_D, M = JFA_BWD_MODE;
  constexpr bool FP8 = JFA_BWD_FP8 != 0;
  const bool win = p.window > 0;
  if constexpr (FP8) {
    if (dbias) return hipErrorInvalidValue;        // the bias gradient is built for bf16 inputs
  } else if (dbias) {
    if (p.bias_kind == JFA_BIAS_DENSE)
      return win ? run_bwd_db<D, M, B_DENSE, true>(p, tc, mq, mk, cu, s)
                 : run_bwd_db<D, M, B_DENSE, false>(p, tc, mq, mk, cu, s);
    return win ? run_bwd_db<D, M, B_RELPOS, true>(p, tc, mq, mk, cu, s)
               : run_bwd_db<D, M, B_RELPOS, false>(p, tc, mq, mk, cu, s);
  }
  return win ? run_bwd<D, M, true, FP8>(p, tc, mq, mk, cu, s)
             : run_bwd<D, M, false, FP8>(p, tc, mq, mk, cu, s);
}

}  // namespace jfa
