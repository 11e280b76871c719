// Phase 2 of v2: log-sum-exp merge of the partitions of one (sequence, query
// head) (page "BI-V100 PagedAttention V2 implementation", "Phase 2: Reduce
// across partitions"):
//   M = max_p m_p,  r_p = exp(m_p - M) * S_p,  out = sum_p r_p O_p / sum_p r_p.
// One 256-thread workgroup per (query head, sequence); sequences with a single
// partition in the window (out already written by Phase 1), on the v1 path,
// or with an invalid length are skipped.  Under a sliding window the merge
// starts at the first partition holding a key of the window; a partition
// with max_logit = -inf adds nothing, and its tmp_out row (never written) is
// not used.
#include "pa_device.h"
#include "pa_launch_kernel.h"

namespace pa {

constexpr int kReduceBatch = 4;  // partitions whose loads one thread issues together

// The 16-byte chunk of a partial row (element type TT) as fp32 values.
template <typename TT>
__device__ __forceinline__ void chunk_to_f32(const u32x4 &v, float (&f)[16 / sizeof(TT)]) {
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (sizeof(TT) == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = bits_f(w[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned short h = (unsigned short)(w[e / 2] >> (16 * (e % 2)));
      f[e] = to_f32(__builtin_bit_cast(TT, h));
    }
  }
}

// Thread (pg, c) reads the 16-byte chunk c of the partial rows of partitions
// pg, pg + PG, ... (TPR threads cover a row, PG = 256 / TPR partitions are
// read per instruction), kReduceBatch partitions at a time so that their
// max_logits, exp_sums and tmp_out loads are in flight together, and folds
// them into a running (max m, sum s = sum exp(m_p - m) S_p, acc = sum
// exp(m_p - m) S_p O_p).  The PG running states of each dim are then merged
// with the same rescale: the result is the merge above with M the global max.
// QT: the output type; TT: the partial type (fp32, or QT).
template <typename QT, typename TT, int D>
__global__ void __launch_bounds__(kThreads) pa_reduce_kernel(const Params p) {
  constexpr int EPT = 16 / sizeof(TT);  // elements per 16-byte chunk
  constexpr int TPR = D / EPT;          // threads per partial row
  constexpr int PG = kThreads / TPR;    // partition groups
  static_assert(kThreads % TPR == 0 && D % EPT == 0, "reduce geometry");
  const int head = blockIdx.x, seq = blockIdx.y;
  const int L = p.seq_lens[seq];
  if (L < 0 || L > p.max_seq_len) return;
  const int t_lo = window_first_token(p.window_left, L);
  if (!seq_uses_v2(p, L - t_lo)) return;
  const int n_part = (L + kPartitionSize - 1) / kPartitionSize;
  const int part_lo = t_lo / kPartitionSize;
  if (n_part - part_lo <= 1) return;

  __shared__ float sm_m[PG], sm_s[PG];
  __shared__ float sm_a[PG][D];

  const size_t row = ((size_t)seq * p.num_heads + head) * p.max_num_partitions;
  const float *ml = p.max_logits + row;
  const float *es = p.exp_sums + row;
  const char *to = reinterpret_cast<const char *>(p.tmp_out) + row * D * sizeof(TT);
  const int c = threadIdx.x % TPR, pg = threadIdx.x / TPR;
  const float ninf = -__builtin_inff();

  float m_run = ninf, s_run = 0.0f, a_run[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) a_run[e] = 0.0f;
  for (int base = part_lo + pg; base < n_part; base += kReduceBatch * PG) {
    float mv[kReduceBatch], ev[kReduceBatch];
    u32x4 ov[kReduceBatch];
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) {
      const int q = base + j * PG;
      const bool ok = q < n_part;
      mv[j] = ok ? ml[q] : ninf;
      ev[j] = ok ? es[q] : 0.0f;
      ov[j] = ok ? load16(to + ((size_t)q * D + c * EPT) * sizeof(TT)) : u32x4{0u, 0u, 0u, 0u};
    }
    float bm = m_run;
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) bm = fmaxf(bm, mv[j]);
    const float keep = (m_run == ninf) ? 0.0f : fast_exp2((m_run - bm) * kLog2e);
    s_run *= keep;
#pragma unroll
    for (int e = 0; e < EPT; ++e) a_run[e] *= keep;
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) {
      const float r = (mv[j] == ninf) ? 0.0f : fast_exp2((mv[j] - bm) * kLog2e) * ev[j];
      float f[EPT];
      chunk_to_f32<TT>(ov[j], f);
      s_run += r;
      const bool live = mv[j] != ninf;
#pragma unroll
      for (int e = 0; e < EPT; ++e) a_run[e] = live ? fmaf(r, f[e], a_run[e]) : a_run[e];
    }
    m_run = bm;
  }
  // Every thread of a partition group holds the same m and s.
  if (c == 0) {
    sm_m[pg] = m_run;
    sm_s[pg] = s_run;
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) sm_a[pg][c * EPT + e] = a_run[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float big_m = ninf;
#pragma unroll
    for (int k = 0; k < PG; ++k) big_m = fmaxf(big_m, sm_m[k]);
    float s = 0.0f, a = 0.0f;
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      const float cf = (sm_m[k] == ninf) ? 0.0f : fast_exp2((sm_m[k] - big_m) * kLog2e);
      s += cf * sm_s[k];
      a += cf * sm_a[k][d];
    }
    QT *out = reinterpret_cast<QT *>(p.out);
    out[((size_t)seq * p.num_heads + head) * D + d] = from_f32<QT>(a / s);
  }
}

template <typename QT, typename TT>
static hipError_t launch_reduce_t(const Params &p, int head_size, const Launch &l) {
  if (head_size == 64) return launch_kernel(pa_reduce_kernel<QT, TT, 64>, l, p);
  if (head_size == 128) return launch_kernel(pa_reduce_kernel<QT, TT, 128>, l, p);
  return hipErrorInvalidValue;
}

// Grid: one workgroup per (query head, sequence).  The partial type is fp32
// when p.tmp_f32 is set, else the output type.
hipError_t launch_reduce(const Params &p, int dtype, int head_size, const Launch &l) {
  switch (dtype) {
    case kDtF32: return launch_reduce_t<float, float>(p, head_size, l);
    case kDtF16:
      return p.tmp_f32 ? launch_reduce_t<_Float16, float>(p, head_size, l)
                       : launch_reduce_t<_Float16, _Float16>(p, head_size, l);
    case kDtBF16:
      return p.tmp_f32 ? launch_reduce_t<__bf16, float>(p, head_size, l)
                       : launch_reduce_t<__bf16, __bf16>(p, head_size, l);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
