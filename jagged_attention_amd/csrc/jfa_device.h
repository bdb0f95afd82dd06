// Device helpers shared by the libjfa kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jfa_internal.h"

namespace jfa {

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E), every index a constant
// expression (fully unrolled however large the body).
template <int I> struct ic { static constexpr int value = I; constexpr operator int() const { return I; } };
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG_INF = -__builtin_huge_valf();

enum Mode { MODE_SOFTMAX = 0, MODE_SILU = 1, MODE_GELU = 2 };

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);   // round to nearest even
}
// Two floats to a bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// max without the NaN-quieting canonicalisation of fmaxf (operands here are never NaN)
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 32x32x16 bf16 MFMA: C[m][n] += sum_k A[m][k] B[k][n].  Lane l supplies A row (l % 32) and
// B column (l % 32), eight k values chosen by l / 32; C element i of lane l is
// (row 8*(i/4) + 4*(l/32) + i%4, column l % 32).
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x64 E4M3 MFMA with E8M0 block scales.  Lane (r, g) = (l % 32, l / 32) supplies 32 codes
// of row r: bytes 0..15 belong to k block 0 and bytes 16..31 to k block 1 of the instruction;
// its scale byte is the scale of row r's k block g.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 cat_bf16x8(u32x2 lo, u32x2 hi) {
  u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// Relative-position bucket: exact below 16, four buckets per doubling, clamped to nb - 1.
__device__ __forceinline__ int relpos_bucket(int x, int nb) {
  x = x < 0 ? -x : x;
  int bkt = x;
  if (x >= 16) {
    const int k = 31 - __clz(x);
    bkt = 16 + 4 * (k - 4) + ((x >> (k - 2)) & 3);
  }
  return bkt < nb - 1 ? bkt : nb - 1;
}

// GDPA activations (fp32).  SiLU x*sigmoid(x); GELU 0.5 x (1 + erf(x / sqrt 2)).
template <int MODE>
__device__ __forceinline__ float act_f(float x) {
  if (MODE == MODE_SILU) return x * fast_rcp(1.0f + __expf(-x));
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}
template <int MODE>
__device__ __forceinline__ float act_grad_f(float x) {
  if (MODE == MODE_SILU) {
    const float sg = fast_rcp(1.0f + __expf(-x));
    return sg * (1.0f + x * (1.0f - sg));
  }
  const float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
  const float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
  return cdf + x * pdf;
}

// Branch-free activations for the bf16 / MXFP8 kernels (errors far below bf16 rounding).
// GELU: Phi(x) from the erfc approximation of Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.25 (|error of erf| <= 2.5e-5, far below bf16's rounding of the
// activation): with z = |x|/sqrt 2, t = 1/(1 + p z), erfc(z) ~ t (a1 + t (a2 + t a3)) exp(-z^2).
// exp(-z^2) = exp(-x^2/2) is also the Gaussian density's factor, so the density
// phi(x) = exp(-x^2/2) / sqrt(2 pi) is computed once, and the coefficients here are
// b_i = a_i sqrt(2 pi) / 2, so that t (b1 + t (b2 + t b3)) phi(x) = (1 - erf(z)) / 2.  Value and
// derivative share one exp and one reciprocal.  Returns Phi(x) and writes phi(x) to pdf.
__device__ __forceinline__ float gelu_cdf(float x, float& pdf) {
  const float t = fast_rcp(fmaf(0.47047f * 0.70710678118654752f, fabsf(x), 1.0f));
  // phi(x) = 2^(x^2 (-log2(e) / 2) - log2(sqrt(2 pi)))
  pdf = fast_exp2(fmaf(x * x, -0.72134752044448170f, -1.3257480647361593f));
  float poly = fmaf(t, 0.7478556f * 1.2533141373155001f, -0.0958798f * 1.2533141373155001f);
  poly = fmaf(t, poly, 0.3480242f * 1.2533141373155001f);
  // (1 - erf(z)) / 2 = t poly pdf lies in [0, 1/2]; Phi(x) = 1/2 + sign(x) (1/2 - that)
  return __builtin_copysignf(fmaf(-t * poly, pdf, 0.5f), x) + 0.5f;
}
// x, or -1e30 where x is below it (a masked pair's -inf): every activation and derivative here
// is then exactly zero, while a NaN stays NaN (IEEE maximum: one instruction on gfx950).
__device__ __forceinline__ float act_clamp(float x) {
  return __builtin_elementwise_maximum(x, -1e30f);
}
template <int MODE>
__device__ __forceinline__ float act_fast(float x) {
  if (MODE == MODE_SILU) return x * fast_rcp(1.0f + fast_exp2(-x * 1.4426950408889634f));
  float pdf;
  return x * gelu_cdf(x, pdf);
}
// Activation and its derivative at x.
template <int MODE>
__device__ __forceinline__ void act_pair(float x, float& a, float& da) {
  if (MODE == MODE_SILU) {
    const float sg = fast_rcp(1.0f + fast_exp2(-x * 1.4426950408889634f));
    a = x * sg;
    da = sg * (1.0f + x * (1.0f - sg));
  } else {
    float pdf;
    const float cdf = gelu_cdf(x, pdf);
    a = x * cdf;
    da = fmaf(x, pdf, cdf);
  }
}

// E4M3 code (sign, 4-bit exponent bias 7, 3-bit mantissa, subnormals) to float.
__device__ __forceinline__ float e4m3_to_f(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, f = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (f << 20))
                : (float)f * 0.001953125f;   // f * 2^-9
  return (c & 128u) ? -mag : mag;
}
// 2^(s - 127) for an E8M0 scale code s (0..254).
__device__ __forceinline__ float e8m0_to_f(uint32_t s) {
  return s == 0 ? 5.877471754111438e-39f : __uint_as_float(s << 23);
}

// Eight E4M3 codes (the bytes of c, lowest first) times 2^(s - 127), as eight bf16: the
// hardware's scaled conversion, exact for the scale codes of normal data (an E4M3 value has 4
// significant bits and bf16 8).
__device__ __forceinline__ bf16x8 dequant8_bf16(u32x2 c, uint32_t s) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const float sc = e8m0_to_f(s);
  const bf2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, false);
  const bf2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, true);
  const bf2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, false);
  const bf2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, true);
  const u32x4 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, d), __builtin_bit_cast(uint32_t, e)};
  return __builtin_bit_cast(bf16x8, w);
}

// Length (floats) of one copy of a four-copy diagonal bias table: at least `len`, and 16 mod 64,
// so that the 16 lanes reading 16 consecutive diagonals from rotating copies hit 16 distinct
// 16-byte bank groups.
constexpr int diag_stride(int len) { return (len - 16 + 63) / 64 * 64 + 16; }

// ------------------------------------------------------------------ buffer access
// A buffer resource covers [base, base + bytes): loads at or past `bytes` return zeros and
// stores there are dropped, so ragged rows need no branches.  Offsets are 32-bit bytes.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Every resource here describes one (sample, head) slice, so base and size are uniform over the
// workgroup; readfirstlane states that to the compiler, which otherwise may keep a resource
// it cannot prove uniform in vector registers and wrap each load in a waterfall loop.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 ld8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld2(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld1(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ void st8(u32x2 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void st16(u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void st2(uint16_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ void st4(uint32_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// names 4 consecutive 16-bit elements A[j][0..3]; lane c receives A[4e + c/4][c % 4], e = 0..3.
// With lane j = 4e + q pointing at row r0 + e, columns c0 + 4q .. c0 + 4q + 3 of a row-major
// tile, lane c receives column c0 + c of rows r0 .. r0 + 3: a column strip, as an MFMA operand
// whose contraction runs along the tile's rows needs.
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4* lp;
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Row stride (bf16) of a wave's output staging area: 32 rows of D, padded against bank conflicts.
template <int D>
constexpr int out_stage_stride() { return D + 8; }

// Row stride (bf16 elements) of a 64-row LDS tile that is read both along rows (16-byte reads,
// 16 lanes per LDS cycle) and with transposing 8-byte reads (32 lanes per cycle, 8 rows x 32
// columns).  Over 64 four-byte banks, D + 8 serves the row reads without conflicts but puts the
// transposing reads four-way on the same banks at d = 128; D + 24 keeps the row reads and the
// staging writes conflict-free and halves that to two-way.  At d = 64, D + 8 is already the
// best of both.
template <int D>
constexpr int tile_row_stride() { return D == 128 ? D + 24 : D + 8; }

template <int D>
constexpr int out_stage_bytes() { return 32 * out_stage_stride<D>() * 2; }

// Writes one wave's 32 output rows of D bf16 through LDS, so that the global stores are whole
// 16-byte chunks with consecutive lanes along a row.  acc holds the transposed MFMA layout: lane
// (r, g) = (lane % 32, lane / 32) has row r's elements 32 db + 8 jq + 4 g + 0..3, multiplied by
// `mul` on the way.  `stage` is the wave's own LDS area (out_stage_bytes), read back only by this
// wave; row i goes to byte offset row0 + i * row_bytes of `r` (rows past its range are dropped).
template <int D>
__device__ __forceinline__ void store_rows_via_lds(const f32x16* acc, float mul, __bf16* stage,
                                                   rsrc_t r, uint32_t row0, uint32_t row_bytes,
                                                   int lane) {
  constexpr int OS = out_stage_stride<D>();
  const int rr = lane & 31, g = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const u32x2 v = {pack2bf(acc[db][4 * jq] * mul, acc[db][4 * jq + 1] * mul),
                       pack2bf(acc[db][4 * jq + 2] * mul, acc[db][4 * jq + 3] * mul)};
      *(u32x2*)(stage + rr * OS + db * 32 + 8 * jq + 4 * g) = v;
    }
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
#pragma unroll
  for (int k = 0; k < 32 * CPR / 64; ++k) {
    const int c = k * 64 + lane;
    const int row = c / CPR, col = c % CPR;
    const u32x4 v = *(const u32x4*)(stage + row * OS + 8 * col);
    st16(v, r, row0 + (uint32_t)row * row_bytes + 16u * (uint32_t)col);
  }
}

// Byte permute: result byte k is byte sel_k of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low halves of two words (lo16(a) | lo16(b) << 16) and high halves (hi16(a) | hi16(b) << 16).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return perm(b, a, 0x07060302u); }

// Eight consecutive bf16 of a dense-bias row from byte offset `off` (2-byte aligned) of a buffer
// of `size` bytes, elements at or past `valid` (0..8) set to zero.  Dword-aligned loads of the
// five dwords that cover the chunk, shifted by one element when `off` is not dword-aligned:
// sub-dword loads of the same bytes cost several times more.  The range check drops a dword
// that only partly lies in the buffer, so a final element in such a dword is loaded alone.
// The work is split in two: bias_chunk_load only issues the loads (into raw registers, so that
// a prefetch does not wait for them), bias_chunk_finish assembles the chunk once they are
// needed; both take the same (off, valid, size).
struct BiasRaw {
  u32x4 x;          // the four dwords from off rounded down to a dword
  uint32_t y;       // the dword after them
  uint32_t z;       // the final element of the buffer, when it sits in a partial dword
};
__device__ __forceinline__ bool bias_chunk_tail(uint32_t off, int valid, uint32_t size) {
  return valid > 0 && (size & 2u) && off + 2u * (uint32_t)(valid - 1) + 2u == size;
}
__device__ __forceinline__ BiasRaw bias_chunk_load(rsrc_t r, uint32_t off, int valid,
                                                   uint32_t size) {
  BiasRaw b{{0u, 0u, 0u, 0u}, 0u, 0u};
  if (valid > 0) {
    const uint32_t base = off & ~3u;
    b.x = ld16(r, base);
    b.y = ld4(r, base + 16);
    if (bias_chunk_tail(off, valid, size)) b.z = ld2(r, off + 2u * (uint32_t)(valid - 1));
  }
  return b;
}
__device__ __forceinline__ u32x4 bias_chunk_finish(const BiasRaw& b, uint32_t off, int valid,
                                                   uint32_t size) {
  u32x4 v = b.x;
  if (off & 2u) {
    v[0] = __builtin_amdgcn_alignbyte(b.x[1], b.x[0], 2);
    v[1] = __builtin_amdgcn_alignbyte(b.x[2], b.x[1], 2);
    v[2] = __builtin_amdgcn_alignbyte(b.x[3], b.x[2], 2);
    v[3] = __builtin_amdgcn_alignbyte(b.y, b.x[3], 2);
  }
  if (bias_chunk_tail(off, valid, size)) {
    const int e = valid - 1;
    const uint32_t sh = 16u * (uint32_t)(e & 1);
    v[e >> 1] = (v[e >> 1] & ~(0xFFFFu << sh)) | (b.z << sh);
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t keep = 2 * w + 1 < valid ? 0xFFFFFFFFu : (2 * w < valid ? 0xFFFFu : 0u);
    v[w] &= keep;
  }
  return v;
}
__device__ __forceinline__ u32x4 bias_chunk(rsrc_t r, uint32_t off, int valid, uint32_t size) {
  return bias_chunk_finish(bias_chunk_load(r, off, valid, size), off, valid, size);
}

// Sum of the two bf16 halves of `w` added to `acc` (fp32).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// Workgroup-wide work ticket: thread 0 takes the next item, everyone gets it.
// Work-item pipeline of a persistent workgroup.  Wave 0 claims the next item while the workgroup
// works on the current one, in three steps spread over the item so that none of them waits:
// claim (an atomic ticket, which takes microseconds to return), resolve (turn the ticket into an
// item and load its 64-byte work record, one dword per lane) and publish (write the record and
// the item index to an LDS buffer before the barrier that ends the item).  A workgroup only ever
// holds its current item and the next one.
//
// Items w = record * H + head are striped over the eight XCDs: XCD x owns w = 8k + x, k = 0, 1, ...
// in list order.  Workgroup g runs on XCD g % 8 and starts on item g; later items of its XCD come
// from that XCD's ticket counter.  When H divides 8 (or 8 divides H) an XCD sees only one head of
// a sample, on at most 8 / H XCDs, so the sample's K/V tiles are reused from that XCD's L2.  A
// workgroup whose XCD has run out takes tickets from the XCD with the most items left.
enum ItemField {
  IF_B = 0, IF_X = 1, IF_Y = 2, IF_Z = 3, IF_SLOT = 4, IF_QO = 5, IF_N = 6, IF_KO = 7, IF_M = 8,
  IF_BOFF = 10, IF_W = 16, IF_WORDS = 17
};
// An item of more steps claims the next one this many steps before its end; shorter items claim
// it before their first tile loads.
constexpr int CLAIM_AHEAD = 4;
constexpr int XCDS = 8;
constexpr int XCD_TICKET_STRIDE = 32;   // dwords between per-XCD counters (own cache lines)
static_assert(XCDS == XTK_XCDS && XCD_TICKET_STRIDE == XTK_STRIDE, "workspace counter layout");

// HOME: workgroup g starts on item g (no ticket); otherwise every item, the first included,
// comes from a ticket.
template <bool HOME>
struct ItemPipeT {
  uint32_t* ctr;             // XCDS counters, XCD_TICKET_STRIDE dwords apart, zeroed per call
  const ItemRec* items;
  int n_items;
  int H;
  int cx = 0;                // XCD list being drawn from (wave 0, uniform)
  int v = 0;                 // lane L < IF_W: dword L of the next item's record
  int wn = 0;                // the next item's index (uniform), published as dword IF_W
  int grid = 0;              // workgroups of the launch (read once: the dispatch packet is memory)
  uint32_t t = 0;            // lane 0: the claimed ticket of list cx

  __device__ __forceinline__ int len(int x) const {
    return n_items > x ? (n_items - x + XCDS - 1) / XCDS : 0;
  }
  // workgroups that start on XCD x's list (they take its first entries without a ticket)
  __device__ __forceinline__ int homed(int x) const {
    return HOME ? (grid - x + XCDS - 1) / XCDS : 0;
  }
  // The record load is left in flight (nothing else is written to v before publish, which would
  // otherwise wait for it).
  __device__ __forceinline__ void load_record(int w, int lane) {
    wn = w;
    if (lane < IF_W && w < n_items) v = reinterpret_cast<const int*>(items + w / H)[lane];
  }
  __device__ __forceinline__ void claim(int lane) {
    if (lane == 0) t = atomicAdd(ctr + XCD_TICKET_STRIDE * cx, 1u);
  }
  __device__ __forceinline__ void resolve(int lane) {
    int k = (int)__builtin_amdgcn_readfirstlane(t) + homed(cx);
    if (k >= len(cx)) {
      // this list is exhausted: take from the list with the most entries left.  A failed claim
      // exhausts one more list for good, so at most XCDS attempts precede success or the end.
      k = -1;
      for (int attempt = 0; attempt <= XCDS && k < 0; ++attempt) {
        int rem = 0;
        if (lane < XCDS) {
          const uint32_t c = __hip_atomic_load(ctr + XCD_TICKET_STRIDE * lane, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          rem = len(lane) - ((int)c + homed(lane));
        }
        int best = -1, best_rem = 0;
#pragma unroll
        for (int x = 0; x < XCDS; ++x) {
          const int r = __builtin_amdgcn_readlane(rem, x);
          if (r > best_rem) { best_rem = r; best = x; }
        }
        if (best < 0) break;
        cx = best;
        uint32_t tt = 0;
        if (lane == 0) tt = atomicAdd(ctr + XCD_TICKET_STRIDE * cx, 1u);
        const int kk = (int)__builtin_amdgcn_readfirstlane(tt) + homed(cx);
        if (kk < len(cx)) k = kk;
      }
    }
    load_record(k >= 0 ? XCDS * k + cx : n_items, lane);
  }
  __device__ __forceinline__ void publish(int* dst, int lane) {
    if (lane < IF_WORDS) dst[lane] = lane == IF_W ? wn : v;
  }
  // first descriptor into dst (wave 0; the caller then synchronises the workgroup)
  __device__ __forceinline__ void start(int* dst, int lane) {
    grid = (int)__builtin_amdgcn_readfirstlane(gridDim.x);
    cx = blockIdx.x % XCDS;
    if constexpr (HOME) {
      load_record(blockIdx.x, lane);
    } else {
      // a list that starts while other workgroups are still busy elsewhere: claim the first
      // item like every later one, so that no item waits for a particular workgroup
      claim(lane);
      resolve(lane);
    }
    publish(dst, lane);
  }
};

using ItemPipe = ItemPipeT<true>;

// Item fields read back from LDS, made wave-uniform.
__device__ __forceinline__ int item_field(const int* d, int f) {
  return __builtin_amdgcn_readfirstlane(d[f]);
}
__device__ __forceinline__ int64_t item_boff(const int* d) {
  return ((int64_t)item_field(d, IF_BOFF + 1) << 32) | (uint32_t)item_field(d, IF_BOFF);
}

__device__ __forceinline__ int64_t next_ticket(uint32_t* counter, int* slot) {
  if (threadIdx.x == 0) *slot = (int)atomicAdd(counter, 1u);
  __syncthreads();
  const int64_t w = *slot;
  __syncthreads();
  return w;
}

}  // namespace jfa
