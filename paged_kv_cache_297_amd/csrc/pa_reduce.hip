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

constexpr int kReduceChunk = 1024;  // partitions whose weights sit in LDS at once

__device__ __forceinline__ float block_max(float v, float *sm) {
  v = xor_max<32>(xor_max<16>(row16_max(v)));
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sm[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sm[i]);
  __syncthreads();
  return r;
}

template <typename QT, int D>
__global__ void __launch_bounds__(kThreads) pa_reduce_kernel(const Params p) {
  constexpr int DG = kThreads / D;  // partition lanes per dim
  const int head = blockIdx.x, seq = blockIdx.y;
  const int L = p.seq_lens[seq];
  if (L < 0 || L > p.max_seq_len || !seq_uses_v2(p, L)) return;
  const int n_part = (L + kPartitionSize - 1) / kPartitionSize;
  if (n_part <= 1) return;

  __shared__ float sm_red[kWaves];
  __shared__ float sm_w[kReduceChunk];
  __shared__ float sm_acc[DG][D];

  const size_t row = ((size_t)seq * p.num_heads + head) * p.max_num_partitions;
  const float *ml = p.max_logits + row;
  const float *es = p.exp_sums + row;
  const float *to = p.tmp_out + row * D;
  const int tid = threadIdx.x;

  float m = -__builtin_inff();
  for (int i = tid; i < n_part; i += kThreads) m = fmaxf(m, ml[i]);
  const float big_m = block_max(m, sm_red);

  const int d = tid % D, pg = tid / D;
  float acc = 0.0f, wsum = 0.0f;
  for (int c0 = 0; c0 < n_part; c0 += kReduceChunk) {
    const int cnt = min(kReduceChunk, n_part - c0);
    for (int i = tid; i < cnt; i += kThreads) {
      const float r = fast_exp2((ml[c0 + i] - big_m) * kLog2e) * es[c0 + i];
      sm_w[i] = r;
    }
    __syncthreads();
    const float *src = to + (size_t)c0 * D + d;
    int i = pg;
    for (; i + 3 * DG < cnt; i += 4 * DG) {
      const float v0 = src[(size_t)i * D], v1 = src[(size_t)(i + DG) * D];
      const float v2 = src[(size_t)(i + 2 * DG) * D], v3 = src[(size_t)(i + 3 * DG) * D];
      acc = fmaf(sm_w[i], v0, acc);
      acc = fmaf(sm_w[i + DG], v1, acc);
      acc = fmaf(sm_w[i + 2 * DG], v2, acc);
      acc = fmaf(sm_w[i + 3 * DG], v3, acc);
    }
    for (; i < cnt; i += DG) acc = fmaf(sm_w[i], src[(size_t)i * D], acc);
    for (int j = 0; j < cnt; ++j) wsum += sm_w[j];
    __syncthreads();
  }
  sm_acc[pg][d] = acc;
  __syncthreads();
  if (tid < D) {
    float o = 0.0f;
#pragma unroll
    for (int k = 0; k < DG; ++k) o += sm_acc[k][tid];
    QT *out = reinterpret_cast<QT *>(p.out);
    out[((size_t)seq * p.num_heads + head) * D + tid] = from_f32<QT>(o / wsum);
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
