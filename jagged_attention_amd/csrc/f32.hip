// fp32 jagged attention, forward and backward, one thread per query (or key) row.
//
// Same definition as the MFMA kernels (see fwd.hip / bwd.hip; source: "Meta GEM Training
// Efficiency: Why LLM-Scale Recommenders Need a Different Stack", section "Bottleneck move 1"),
// in plain fp32 FMA arithmetic for inputs stored as fp32.  It serves small fp32 problems, where
// exactness matters more than MFMA throughput.  Keys (or queries) are staged in LDS 64 rows
// at a time; the tile lists are the scheduler's with 64-row tiles and no splitting; dQ and
// dK/dV are each owned by one thread and summed in order (deterministic).
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

constexpr int NT = 64;

__device__ __forceinline__ float bias_at(const FwdParams& p, int64_t bias_base, int h, int i,
                                         int j, int n, int m) {
  if (p.bias_kind == JFA_BIAS_RELPOS)
    return ((const float*)p.bias)[(int64_t)h * p.num_buckets +
                                  relpos_bucket(i + (m - n) - j, p.num_buckets)];
  if (p.bias_kind == JFA_BIAS_DENSE)
    return ((const float*)p.bias)[bias_base + (int64_t)i * m + j];
  return 0.f;
}

// Sliding window: key j is out of query i's window (aligned position i + delta) when
// |i + delta - j| >= window (window 0: no window).
__device__ __forceinline__ bool out_of_window(int window, int i, int j, int delta) {
  const int d = i + delta - j;
  return window > 0 && (d >= window || -d >= window);
}

template <int D, int MODE>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdParams p) {
  __shared__ float ks[F32_BN][D + 1];
  __shared__ float vs[F32_BN][D + 1];
  __shared__ int s_ticket;
  if (p.hdr_ro->status != JFA_OK) return;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr_ro->counts[0] * H;
  for (;;) {
    const int64_t w = next_ticket(&p.hdr->tickets[TK_FWD], &s_ticket);
    if (w >= n_items) break;
    const ItemRec& it = p.items[w / H];
    const int4 rec = make_int4(it.b, it.x, it.y, it.z);
    const int h = (int)(w % H);
    const int b = rec.x, t = rec.y, kb = rec.z, ke = rec.w;
    const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
    const int ko = p.kv_off[b], m = p.kv_off[b + 1] - ko;
    const int qi = t * F32_BM + threadIdx.x;
    const int64_t bias_base =
        p.bias_kind == JFA_BIAS_DENSE ? (int64_t)H * p.bias_off[b] + (int64_t)h * n * m : 0;
    float qv[D], acc[D];
    const float* qrow = (const float*)p.q + ((int64_t)(qo + qi) * H + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) { qv[c] = qi < n ? qrow[c] : 0.f; acc[c] = 0.f; }
    float mx = NEG_INF, l = 0.f;
    for (int kt = kb; kt < ke; ++kt) {
      const int j0 = kt * F32_BN;
      __syncthreads();
      for (int e = threadIdx.x; e < F32_BN * D; e += NT) {
        const int r = e / D, c = e % D;
        const bool ok = j0 + r < m;
        const int64_t off = ((int64_t)(ko + j0 + r) * H + h) * D + c;
        ks[r][c] = ok ? ((const float*)p.k)[off] : 0.f;
        vs[r][c] = ok ? ((const float*)p.v)[off] : 0.f;
      }
      __syncthreads();
      if (qi >= n) continue;
      const int jend = min(F32_BN, m - j0);
      for (int jj = 0; jj < jend; ++jj) {
        const int j = j0 + jj;
        if (p.causal && j > qi + (m - n)) break;
        if (out_of_window(p.window, qi, j, m - n)) continue;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) s = fmaf(qv[c], ks[jj][c], s);
        s = s * p.scale + bias_at(p, bias_base, h, qi, j, n, m);
        if constexpr (MODE == MODE_SOFTMAX) {
          if (s > mx) {
            const float corr = expf(mx - s);   // mx = -inf gives 0
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] *= corr;
            l *= corr;
            mx = s;
          }
          const float pr = expf(s - mx);
          l += pr;
#pragma unroll
          for (int c = 0; c < D; ++c) acc[c] = fmaf(pr, vs[jj][c], acc[c]);
        } else {
          const float a = act_f<MODE>(s);
#pragma unroll
          for (int c = 0; c < D; ++c) acc[c] = fmaf(a, vs[jj][c], acc[c]);
        }
      }
    }
    if (qi < n) {
      float mul;
      if constexpr (MODE == MODE_SOFTMAX) mul = l > 0.f ? 1.0f / l : 0.f;
      else mul = (p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
      float* orow = (float*)p.o + ((int64_t)(qo + qi) * H + h) * D;
#pragma unroll
      for (int c = 0; c < D; ++c) orow[c] = acc[c] * mul;
      if (MODE == MODE_SOFTMAX && p.lse)
        p.lse[(int64_t)h * p.total_q + qo + qi] = l > 0.f ? mx + logf(l) : NEG_INF;
    }
  }
}

__device__ __forceinline__ float bias_at_b(const BwdParams& p, int64_t bias_base, int h, int i,
                                           int j, int n, int m) {
  if (p.bias_kind == JFA_BIAS_RELPOS)
    return ((const float*)p.bias)[(int64_t)h * p.num_buckets +
                                  relpos_bucket(i + (m - n) - j, p.num_buckets)];
  if (p.bias_kind == JFA_BIAS_DENSE)
    return ((const float*)p.bias)[bias_base + (int64_t)i * m + j];
  return 0.f;
}

// dQ: one thread per query row, keys in steps of 64.
template <int D, int MODE>
__global__ __launch_bounds__(NT) void bwd_q_f32_kernel(BwdParams p) {
  __shared__ float ks[F32_BN][D + 1];
  __shared__ float vs[F32_BN][D + 1];
  __shared__ int s_ticket;
  if (p.hdr->status != JFA_OK) return;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr->counts[2] * H;
  for (;;) {
    const int64_t w = next_ticket(&p.hdr->tickets[TK_BQ], &s_ticket);
    if (w >= n_items) break;
    const ItemRec& it = p.bq[w / H];
    const int4 rec = make_int4(it.b, it.x, it.y, it.z);
    const int h = (int)(w % H);
    const int b = rec.x, t = rec.y, kb = rec.z, ke = rec.w;
    const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
    const int ko = p.kv_off[b], m = p.kv_off[b + 1] - ko;
    const float wn = (MODE != MODE_SOFTMAX && p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    const int qi = t * F32_BM + threadIdx.x;
    const int64_t rowq = (int64_t)(qo + qi) * H + h;
    const int64_t bias_base =
        p.bias_kind == JFA_BIAS_DENSE ? (int64_t)H * p.bias_off[b] + (int64_t)h * n * m : 0;
    float qv[D], dov[D], dq[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
      qv[c] = qi < n ? ((const float*)p.q)[rowq * D + c] : 0.f;
      dov[c] = qi < n ? ((const float*)p.dout)[rowq * D + c] : 0.f;
      dq[c] = 0.f;
    }
    float lse = 0.f, dl = 0.f;
    if (MODE == MODE_SOFTMAX && qi < n) {
      lse = p.lse[(int64_t)h * p.total_q + qo + qi];
      dl = p.delta[(int64_t)h * p.total_q + qo + qi];
    }
    for (int kt = kb; kt < ke; ++kt) {
      const int j0 = kt * F32_BN;
      __syncthreads();
      for (int e = threadIdx.x; e < F32_BN * D; e += NT) {
        const int r = e / D, c = e % D;
        const bool ok = j0 + r < m;
        const int64_t off = ((int64_t)(ko + j0 + r) * H + h) * D + c;
        ks[r][c] = ok ? ((const float*)p.k)[off] : 0.f;
        vs[r][c] = ok ? ((const float*)p.v)[off] : 0.f;
      }
      __syncthreads();
      if (qi >= n) continue;
      const int jend = min(F32_BN, m - j0);
      for (int jj = 0; jj < jend; ++jj) {
        const int j = j0 + jj;
        if (p.causal && j > qi + (m - n)) break;
        if (out_of_window(p.window, qi, j, m - n)) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          s = fmaf(qv[c], ks[jj][c], s);
          dp = fmaf(dov[c], vs[jj][c], dp);
        }
        s = s * p.scale + bias_at_b(p, bias_base, h, qi, j, n, m);
        float ds;
        if constexpr (MODE == MODE_SOFTMAX) ds = expf(s - lse) * (dp - dl);
        else ds = act_grad_f<MODE>(s) * dp * wn;
#pragma unroll
        for (int c = 0; c < D; ++c) dq[c] = fmaf(ds, ks[jj][c], dq[c]);
      }
    }
    if (qi < n) {
#pragma unroll
      for (int c = 0; c < D; ++c) ((float*)p.dq)[rowq * D + c] = dq[c] * p.scale;
    }
  }
}

// dK, dV: one thread per key row, queries in steps of 64.
template <int D, int MODE>
__global__ __launch_bounds__(NT) void bwd_kv_f32_kernel(BwdParams p) {
  __shared__ float qs_[F32_BM][D + 1];
  __shared__ float ds_[F32_BM][D + 1];
  __shared__ float lse_s[F32_BM], dl_s[F32_BM];
  __shared__ int s_ticket;
  if (p.hdr->status != JFA_OK) return;
  const int H = p.H;
  const int64_t n_items = (int64_t)p.hdr->counts[3] * H;
  for (;;) {
    const int64_t w = next_ticket(&p.hdr->tickets[TK_BK], &s_ticket);
    if (w >= n_items) break;
    const ItemRec& it = p.bk[w / H];
    const int4 rec = make_int4(it.b, it.x, it.y, it.z);
    const int h = (int)(w % H);
    const int b = rec.x, u = rec.y, qs0 = rec.z, qs1 = rec.w;
    const int qo = p.q_off[b], n = p.q_off[b + 1] - qo;
    const int ko = p.kv_off[b], m = p.kv_off[b + 1] - ko;
    const float wn = (MODE != MODE_SOFTMAX && p.normalize && m > 0) ? 1.0f / (float)m : 1.0f;
    const int j = u * F32_BN + threadIdx.x;
    const int64_t rowk = (int64_t)(ko + j) * H + h;
    const int64_t bias_base =
        p.bias_kind == JFA_BIAS_DENSE ? (int64_t)H * p.bias_off[b] + (int64_t)h * n * m : 0;
    float kv[D], vv[D], dk[D], dv[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
      kv[c] = j < m ? ((const float*)p.k)[rowk * D + c] : 0.f;
      vv[c] = j < m ? ((const float*)p.v)[rowk * D + c] : 0.f;
      dk[c] = 0.f;
      dv[c] = 0.f;
    }
    for (int qs = qs0; qs < qs1; ++qs) {
      const int i0 = qs * F32_BM;
      __syncthreads();
      for (int e = threadIdx.x; e < F32_BM * D; e += NT) {
        const int r = e / D, c = e % D;
        const bool ok = i0 + r < n;
        const int64_t off = ((int64_t)(qo + i0 + r) * H + h) * D + c;
        qs_[r][c] = ok ? ((const float*)p.q)[off] : 0.f;
        ds_[r][c] = ok ? ((const float*)p.dout)[off] : 0.f;
      }
      if (MODE == MODE_SOFTMAX) {
        const int r = threadIdx.x;
        const bool ok = i0 + r < n;
        lse_s[r] = ok ? p.lse[(int64_t)h * p.total_q + qo + i0 + r] : 0.f;
        dl_s[r] = ok ? p.delta[(int64_t)h * p.total_q + qo + i0 + r] : 0.f;
      }
      __syncthreads();
      if (j >= m) continue;
      const int iend = min(F32_BM, n - i0);
      for (int ii = 0; ii < iend; ++ii) {
        const int i = i0 + ii;
        if (p.causal && j > i + (m - n)) continue;
        if (out_of_window(p.window, i, j, m - n)) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          s = fmaf(qs_[ii][c], kv[c], s);
          dp = fmaf(ds_[ii][c], vv[c], dp);
        }
        s = s * p.scale + bias_at_b(p, bias_base, h, i, j, n, m);
        float pr, dsv;
        if constexpr (MODE == MODE_SOFTMAX) {
          pr = expf(s - lse_s[ii]);
          dsv = pr * (dp - dl_s[ii]);
        } else {
          pr = act_f<MODE>(s) * wn;
          dsv = act_grad_f<MODE>(s) * dp * wn;
        }
#pragma unroll
        for (int c = 0; c < D; ++c) {
          dv[c] = fmaf(pr, ds_[ii][c], dv[c]);
          dk[c] = fmaf(dsv, qs_[ii][c], dk[c]);
        }
      }
    }
    if (j < m) {
#pragma unroll
      for (int c = 0; c < D; ++c) {
        ((float*)p.dk)[rowk * D + c] = dk[c] * p.scale;
        ((float*)p.dv)[rowk * D + c] = dv[c];
      }
    }
  }
}

template <int D, int MODE>
hipError_t run_fwd32(const FwdParams& p, int64_t max_items, int cu, hipStream_t s) {
  auto kern = fwd_f32_kernel<D, MODE>;
  int grid = resident_grid((const void*)kern, NT, 0, cu);
  if ((int64_t)grid > max_items) grid = (int)max(max_items, (int64_t)1);
  timing_begin("jfa_fwd_f32", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, s, p);
  timing_end(s);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t run_bwd32(const BwdParams& p, int64_t mq, int64_t mk, int cu, hipStream_t s) {
  // D (softmax) was computed by the scheduler launch
  {
    auto kern = bwd_kv_f32_kernel<D, MODE>;
    int grid = resident_grid((const void*)kern, NT, 0, cu);
    if ((int64_t)grid > mk) grid = (int)max(mk, (int64_t)1);
    timing_begin("jfa_bwd_dkdv_f32", s);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, s, p);
    timing_end(s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto kern = bwd_q_f32_kernel<D, MODE>;
  int grid = resident_grid((const void*)kern, NT, 0, cu);
  if ((int64_t)grid > mq) grid = (int)max(mq, (int64_t)1);
  timing_begin("jfa_bwd_dq_f32", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, s, p);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_f32(const FwdParams& p, const TileCfg& tc, int head_dim, int mode,
                              int64_t max_items, int cu_count, hipStream_t s) {
  (void)tc;
#define JFA_F32F(D_)                                                                     \
  if (head_dim == D_) {                                                                  \
    if (mode == MODE_SOFTMAX) return run_fwd32<D_, MODE_SOFTMAX>(p, max_items, cu_count, s); \
    if (mode == MODE_SILU) return run_fwd32<D_, MODE_SILU>(p, max_items, cu_count, s);       \
    return run_fwd32<D_, MODE_GELU>(p, max_items, cu_count, s);                              \
  }
  JFA_F32F(64)
  JFA_F32F(128)
#undef JFA_F32F
  return hipErrorInvalidValue;
}

hipError_t launch_backward_f32(const BwdParams& p, const TileCfg& tc, int head_dim,
                               int64_t max_q_items, int64_t max_k_items, int cu_count,
                               hipStream_t s) {
  (void)tc;
#define JFA_F32B(D_)                                                                           \
  if (head_dim == D_) {                                                                        \
    if (p.mode == MODE_SOFTMAX) return run_bwd32<D_, MODE_SOFTMAX>(p, max_q_items, max_k_items, cu_count, s); \
    if (p.mode == MODE_SILU) return run_bwd32<D_, MODE_SILU>(p, max_q_items, max_k_items, cu_count, s);       \
    return run_bwd32<D_, MODE_GELU>(p, max_q_items, max_k_items, cu_count, s);                              \
  }
  JFA_F32B(64)
  JFA_F32B(128)
#undef JFA_F32B
  return hipErrorInvalidValue;
}

}  // namespace jfa
