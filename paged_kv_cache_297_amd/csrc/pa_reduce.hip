// Phase 2 of v2: log-sum-exp merge of the partitions of one (sequence, query
// head) (page "BI-V100 PagedAttention V2 implementation", "Phase 2: Reduce
// across partitions"):
//   M = max_p m_p,  r_p = exp(m_p - M) * S_p,  out = sum_p r_p O_p / sum_p r_p.
// One 256-thread workgroup per (query head, sequence); sequences with a single
// partition (out already written by Phase 1), on the v1 path, or with an
// invalid length are skipped.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kReduceBatch = 8;  // partitions whose loads one thread issues together

// Thread (pg, d) folds partitions pg, pg + DG, ... of the row into a running
// (max m, sum s = sum exp(m_p - m) S_p, acc = sum exp(m_p - m) S_p O_p[d]),
// loading kReduceBatch partitions at a time so that the loads of max_logits,
// exp_sums and tmp_out are in flight together; the DG partial states of a
// dim are then combined with the same rescale.  The result is the merge above
// with M the global max.
template <typename QT, int D>
__global__ void __launch_bounds__(kThreads) pa_reduce_kernel(const Params p) {
  constexpr int DG = kThreads / D;  // partition groups per dim
  const int head = blockIdx.x, seq = blockIdx.y;
  const int L = p.seq_lens[seq];
  if (L < 0 || L > p.max_seq_len || !seq_uses_v2(p, L)) return;
  const int n_part = (L + kPartitionSize - 1) / kPartitionSize;
  if (n_part <= 1) return;

  __shared__ float sm_m[DG][D], sm_s[DG][D], sm_a[DG][D];

  const size_t row = ((size_t)seq * p.num_heads + head) * p.max_num_partitions;
  const float *ml = p.max_logits + row;
  const float *es = p.exp_sums + row;
  const float *to = p.tmp_out + row * D;
  const int d = threadIdx.x % D, pg = threadIdx.x / D;
  const float ninf = -__builtin_inff();

  float m_run = ninf, s_run = 0.0f, a_run = 0.0f;
  for (int base = pg; base < n_part; base += kReduceBatch * DG) {
    float mv[kReduceBatch], ev[kReduceBatch], ov[kReduceBatch];
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) {
      const int q = base + j * DG;
      const bool ok = q < n_part;
      mv[j] = ok ? ml[q] : ninf;
      ev[j] = ok ? es[q] : 0.0f;
      ov[j] = ok ? to[(size_t)q * D + d] : 0.0f;
    }
    float bm = m_run;
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) bm = fmaxf(bm, mv[j]);
    const float keep = (m_run == ninf) ? 0.0f : fast_exp2((m_run - bm) * kLog2e);
    s_run *= keep;
    a_run *= keep;
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) {
      const float r = (mv[j] == ninf) ? 0.0f : fast_exp2((mv[j] - bm) * kLog2e) * ev[j];
      s_run += r;
      a_run = fmaf(r, ov[j], a_run);
    }
    m_run = bm;
  }
  sm_m[pg][d] = m_run;
  sm_s[pg][d] = s_run;
  sm_a[pg][d] = a_run;
  __syncthreads();
  if (pg == 0) {
    float big_m = ninf;
#pragma unroll
    for (int k = 0; k < DG; ++k) big_m = fmaxf(big_m, sm_m[k][d]);
    float s = 0.0f, a = 0.0f;
#pragma unroll
    for (int k = 0; k < DG; ++k) {
      const float c = (sm_m[k][d] == ninf) ? 0.0f : fast_exp2((sm_m[k][d] - big_m) * kLog2e);
      s += c * sm_s[k][d];
      a += c * sm_a[k][d];
    }
    QT *out = reinterpret_cast<QT *>(p.out);
    out[((size_t)seq * p.num_heads + head) * D + d] = from_f32<QT>(a / s);
  }
}

template <typename QT>
static hipError_t launch_reduce_t(const Params &p, int head_size, const Launch &l) {
  if (head_size == 64) return launch_kernel(pa_reduce_kernel<QT, 64>, l, p);
  if (head_size == 128) return launch_kernel(pa_reduce_kernel<QT, 128>, l, p);
  return hipErrorInvalidValue;
}

// Grid: one workgroup per (query head, sequence).
hipError_t launch_reduce(const Params &p, int dtype, int head_size, const Launch &l) {
  switch (dtype) {
    case kDtF32: return launch_reduce_t<float>(p, head_size, l);
    case kDtF16: return launch_reduce_t<_Float16>(p, head_size, l);
    case kDtBF16: return launch_reduce_t<__bf16>(p, head_size, l);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
